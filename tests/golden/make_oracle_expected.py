"""Write the stored oracle values of the full-size parity tests.

Calls only the CPU oracle (oracle/julia_oracle.py) on seeded weights and the
seeded batches of each workload configuration; nothing here comes from the GPU
library.  Sequences are independent, so a sequence's values do not depend on
the rest of its batch and large configurations can be sampled by sequence.

    python tests/golden/make_oracle_expected.py logits [--configs 0,1,2,3,4]
        -> oracle_logits.json: the published init (std 0.02, seed 0); all
           sequences of configurations 0-2, sequences 0 and 7 of 3, eight
           sampled sequences of 4.
    python tests/golden/make_oracle_expected.py wide [--configs ...] [--jobs 8]
        -> oracle_logits_wide.json: the wide weight set (std 0.05, seed 0),
           whose option logits spread to order one; every sequence of
           configurations 0-2 and 4 (256 questions), sequences 0 and 7 of 3.
    python tests/golden/make_oracle_expected.py rows [--jobs 4]
        -> oracle_rows_long.npz: hidden rows of sequences 0 and 7 of the
           16 x 8,192 configuration at sampled positions up to 8,191, after
           the first two encoder layers (stages 1 and 2, a global and a
           window layer), after the encoder (stage 22), after the first head layer (stage 24) and
           after the second at the markers (stage 25), plus their logits, for
           both weight sets (float32).

Run from the repository root.
"""
import argparse
import hashlib
import json
import os
import sys
import time
from concurrent.futures import ProcessPoolExecutor

if "--jobs" in sys.argv:  # worker processes: one BLAS thread each (set before NumPy loads BLAS)
    for _v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[_v] = "1"

import numpy as np  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from encoder_transformer_amd import synth  # noqa: E402
from oracle import julia_oracle as jo  # noqa: E402

GOLDEN = os.path.join(ROOT, "tests", "golden")
OUT_LOGITS = os.path.join(GOLDEN, "oracle_logits.json")
OUT_WIDE = os.path.join(GOLDEN, "oracle_logits_wide.json")
OUT_ROWS = os.path.join(GOLDEN, "oracle_rows_long.npz")

# positions of the stored long-sequence rows: both ends, the window and
# 64-/128-query tile edges, the middle and the RoPE table's last rows
LONG_POSITIONS = [0, 1, 63, 64, 65, 127, 128, 129, 1000, 2047, 2048, 4095, 4096, 4097, 6000, 8063, 8064, 8127,
                  8128, 8190, 8191]
LONG_SEQS = [0, 7]
WEIGHT_SETS = {"standard": synth.INIT_STD, "wide": synth.WIDE_STD}


def batch_digest(b) -> str:
    h = hashlib.sha256()
    for a in (b.ids, b.seq_offsets, b.mask_positions, b.qtype):
        h.update(np.ascontiguousarray(a, np.int32).tobytes())
    return h.hexdigest()


def weights_digest(w) -> str:
    h = hashlib.sha256()
    for name, _, _ in synth.weight_spec():
        h.update(name.encode())
        h.update(str(synth.tensor_checksum(w[name])).encode())
    return h.hexdigest()


def sample(config: int, b, wide: bool) -> list:
    if config in (0, 1, 2) or (config == 4 and wide):
        return list(range(b.n_seqs))
    if config == 3:
        return list(LONG_SEQS)
    lens = np.diff(b.seq_offsets)
    r = np.random.default_rng(4242)
    pick = {int(np.argmax(lens)), int(np.argmin(lens))}
    pick.update(int(i) for i in r.choice(b.n_seqs, size=6, replace=False))
    return sorted(pick)


_W = {}


def _weights(std):
    if std not in _W:
        _W[std] = jo.OracleWeights(synth.make_weights(std=std))
    return _W[std]


def _logits_job(args):
    std, config, s = args
    b = synth.make_batch(config)
    ids, marks, qt = b.sequence(s)
    return [float(v) for v in jo.forward_sequence(_weights(std), ids, marks, qt)]


def _rows_job(args):
    std, s = args
    W = _weights(std)
    b = synth.make_batch(3)
    ids, marks, qt = b.sequence(s)
    x = jo.embed(W, ids)
    early = []
    for l in range(jo.N_LAYERS):
        x = jo.encoder_layer(W, l, x)
        if l + 1 in (1, 2):
            early.append(x[LONG_POSITIONS].astype(np.float32))
    h = jo.head_layer(W, 0, jo.head_input(W, x, qt))
    z = jo.head_layer(W, 1, h)[marks]
    return (early[0], early[1], x[LONG_POSITIONS].astype(np.float32), h[LONG_POSITIONS].astype(np.float32),
            z.astype(np.float32), jo.score(W, z))


def _pool(jobs):
    return ProcessPoolExecutor(max_workers=jobs) if jobs > 1 else None


def write_logits(path, std, configs, wide, jobs):
    data = {}
    if os.path.exists(path):
        with open(path) as f:
            data = json.load(f)
    w = synth.make_weights(std=std)
    data["weights_seed"] = synth.WEIGHT_SEED
    data["weights_std"] = std
    data["weights_digest"] = weights_digest(w)
    data.setdefault("configs", {})
    pool = _pool(jobs)
    for c in configs:
        b = synth.make_batch(c)
        seqs = sample(c, b, wide)
        t0 = time.time()
        args = [(std, c, s) for s in seqs]
        res = list(pool.map(_logits_job, args) if pool else map(_logits_job, args))
        data["configs"][str(c)] = {"batch_digest": batch_digest(b), "seqs": seqs, "logits": res}
        print(f"config {c}: {len(seqs)} sequences ({time.time() - t0:.1f}s)", flush=True)
        with open(path, "w") as f:
            json.dump(data, f, indent=0)
    print("wrote", path)


def write_rows(jobs):
    pool = _pool(jobs)
    args = [(std, s) for std in WEIGHT_SETS.values() for s in LONG_SEQS]
    t0 = time.time()
    res = list(pool.map(_rows_job, args) if pool else map(_rows_job, args))
    out = {"positions": np.asarray(LONG_POSITIONS, np.int32), "seqs": np.asarray(LONG_SEQS, np.int32),
           "batch_digest": np.frombuffer(batch_digest(synth.make_batch(3)).encode(), np.uint8)}
    for (std, s), (x1, x2, x22, h24, z25, lg) in zip(args, res):
        name = [k for k, v in WEIGHT_SETS.items() if v == std][0]
        out[f"{name}_s{s}_stage1"] = x1
        out[f"{name}_s{s}_stage2"] = x2
        out[f"{name}_s{s}_stage22"] = x22
        out[f"{name}_s{s}_stage24"] = h24
        out[f"{name}_s{s}_stage25"] = z25
        out[f"{name}_s{s}_logits"] = lg
    np.savez(OUT_ROWS, **out)
    print(f"wrote {OUT_ROWS} ({time.time() - t0:.1f}s)")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("what", choices=["logits", "wide", "rows"])
    ap.add_argument("--configs", default="0,1,2,3,4")
    ap.add_argument("--jobs", type=int, default=1)
    args = ap.parse_args()
    configs = [int(x) for x in args.configs.split(",")]
    if args.what == "logits":
        write_logits(OUT_LOGITS, synth.INIT_STD, configs, False, args.jobs)
    elif args.what == "wide":
        write_logits(OUT_WIDE, synth.WIDE_STD, configs, True, args.jobs)
    else:
        write_rows(args.jobs)


if __name__ == "__main__":
    main()
