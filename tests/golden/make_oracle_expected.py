"""Write tests/golden/oracle_logits.json: oracle logits of the workload configurations.

Calls only the CPU oracle (oracle/julia_oracle.py) on the seeded weights
(seed 0) and the seeded batches of each configuration. The large
configurations are sampled by sequence (sequences are independent, so a
sequence's logits do not depend on the rest of the batch). Run from the
repository root:

    python tests/golden/make_oracle_expected.py [--configs 0,1,2,3,4]
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from encoder_transformer_amd import synth  # noqa: E402
from oracle import julia_oracle as jo  # noqa: E402

OUT = os.path.join(ROOT, "tests", "golden", "oracle_logits.json")


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


def sample(config: int, b) -> list:
    if config in (0, 1, 2):
        return list(range(b.n_seqs))
    if config == 3:
        return [0, 7]
    lens = np.diff(b.seq_offsets)
    r = np.random.default_rng(4242)
    pick = {int(np.argmax(lens)), int(np.argmin(lens))}
    pick.update(int(i) for i in r.choice(b.n_seqs, size=6, replace=False))
    return sorted(pick)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--configs", default="0,1,2,3,4")
    args = ap.parse_args()
    data = {}
    if os.path.exists(OUT):
        with open(OUT) as f:
            data = json.load(f)
    w = synth.make_weights()
    W = jo.OracleWeights(w)
    data["weights_seed"] = synth.WEIGHT_SEED
    data["weights_digest"] = weights_digest(w)
    data.setdefault("configs", {})
    for c in [int(x) for x in args.configs.split(",")]:
        b = synth.make_batch(c)
        seqs = sample(c, b)
        t0 = time.time()
        entry = {"batch_digest": batch_digest(b), "seqs": seqs, "logits": []}
        for s in seqs:
            ids, marks, qt = b.sequence(s)
            entry["logits"].append([float(v) for v in jo.forward_sequence(W, ids, marks, qt)])
            print(f"config {c} seq {s} len {len(ids)} done ({time.time() - t0:.1f}s)", flush=True)
        data["configs"][str(c)] = entry
        with open(OUT, "w") as f:
            json.dump(data, f, indent=1)
    print("wrote", OUT)


if __name__ == "__main__":
    main()
