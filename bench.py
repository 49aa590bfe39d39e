"""Benchmark of the Julia-1 forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step = jl_forward + jl_probs over one packed batch already resident in
HBM (weights loaded, token ids on the device). The headline workload is the
throughput case: 16 sequences of 1,024 tokens, question types cycling
choice/score/noul, 2-20 options of 1-48 tokens, bf16. Extra fields report
the batch-1 latency case (1 x 1,024: mean, per-call percentiles, and host ids
to host logits), the long-context case (16 x 8,192), the ragged serving mix
(256 sequences of 64-2,048 tokens), FP32 mode and FP8 mode.

`roofline` covers the kernel class with the most device time in the timed
region, measured with HIP events bracketing each of its launches on the
launch stream; `cpu_baseline` times the CPU oracle on six of the 1,024-token
sequences. Prints one JSON line.
"""
import argparse
import gc
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix-core peak
PEAK_FP32_TFLOPS = 157.3
HBM_GBPS = 8000.0
D, FFN_HEAD = 384, 1536
ROW_BLOCK_MIN_TOKENS = 8192  # bf16 batches this large use the row-block layer kernel
PROFILE_EVERY = 10  # timed-region steps between the steps whose dominant-class launches carry events


def call_alg_bytes(batch):
    """Algorithmic HBM bytes of one forward + read-off: every bf16 GEMM weight
    once (encoder 22 x 3,833,856 B; head layers 2 x 3,538,944 B), the FP32
    norms, biases, type table and scorer (709,636 B), each token's FP32
    embedding row and id, each marker's logit and probability."""
    return 22 * 3_833_856 + 2 * 3_538_944 + 709_636 + batch.n_tokens * (1536 + 4) + batch.n_markers * 8


def band_pairs(L, w=64):
    p = np.arange(L)
    return int(np.sum(np.minimum(L - 1, p + w) - np.maximum(0, p - w) + 1))


def class_flops(batch, row_block):
    """Algorithmic FLOPs per step of each kernel class (masked work not counted).

    `row_block`: the bf16 path for large batches, where one layer kernel per
    layer runs the out-projection, the MLP and the next layer's QKV (the last
    one the head's first in-projection), and one head-layer kernel the rest of
    the first head layer and the second's keys and values.
    """
    lens = np.diff(batch.seq_offsets).astype(np.int64)
    T, M = int(lens.sum()), batch.n_markers
    glob = int(np.sum(lens * lens))
    band = sum(band_pairs(int(L)) for L in lens)
    qkv, outp, mlp_in, mlp_out = 2 * T * D * 3 * D, 2 * T * D * D, 2 * T * D * 2304, 2 * T * 1152 * D
    f = {k: 0 for k in ("embed", "qkv", "outproj", "mlp_in", "mlp_out", "layer", "head_layer", "ln")}
    # head layer 1 on every token (in-projection, out-projection, feed-forward),
    # layer 2 keys/values on every token and the rest on marker rows
    head_in, head_rest, head_kv = 2 * T * D * 3 * D, 2 * T * D * (D + 2 * FFN_HEAD), 2 * T * D * 2 * D
    head_markers = 2 * M * D * (D + D + 2 * FFN_HEAD)
    if row_block:
        f["embed"] = qkv  # the embedding kernel computes the first layer's QKV
        f["layer"] = 22 * (outp + mlp_in + mlp_out) + 21 * qkv + head_in
        f["head_layer"] = head_rest + head_kv
        f["head_gemm"] = head_markers
    else:
        f.update(qkv=22 * qkv, outproj=22 * outp, mlp_in=22 * mlp_in, mlp_out=22 * mlp_out)
        f["head_gemm"] = head_in + head_rest + head_kv + head_markers
    f["attn_global"] = 8 * 1536 * glob
    f["attn_local"] = 14 * 1536 * band
    # attention of marker queries over their sequence
    f["head_attn"] = 1536 * glob + 1536 * int(sum(len(batch.sequence(b)[1]) * lens[b] for b in range(batch.n_seqs)))
    f["misc"] = 2 * M * D * D + 2 * M * D
    return f


def time_workload(model, batch, steps, warmup, profile_class=None, sample=True):
    import torch
    from encoder_transformer_amd import lib
    ids = torch.from_numpy(np.ascontiguousarray(batch.ids)).to("cuda:0")
    so, mp, qt = batch.seq_offsets, batch.mask_positions, batch.qtype
    logits = torch.empty(batch.n_markers, dtype=torch.float32, device="cuda:0")

    stream = torch.cuda.Stream()  # a capturable stream (torch's default one is the NULL stream)
    torch.cuda.synchronize()

    def step():
        with torch.cuda.stream(stream):
            model.forward(ids, so, mp, qt, out=logits)
            model.probs(logits, so, mp, qt)

    step()  # first call: code objects load, workspace pages in
    torch.cuda.synchronize()
    # warm-up with every class timed, to find where the device time goes
    model.profile(1, (1 << lib.N_KERNEL_CLASSES) - 1)
    for _ in range(max(1, warmup)):
        step()
    torch.cuda.synchronize()
    per_class = {lib.KERNEL_CLASS_NAMES[c]: model.profile_read(c) for c in range(lib.N_KERNEL_CLASSES)}
    dominant = max(per_class, key=lambda k: per_class[k][0]) if profile_class is None else profile_class
    cls_id = lib.KERNEL_CLASS_NAMES.index(dominant)
    # timed region: the dominant class's launches are bracketed by events in
    # every PROFILE_EVERY-th step (a sample of the region; those steps run
    # eagerly, and their event records cost the stream time: measured 3% of
    # the region's time with every 4th step sampled, so about 1% at every
    # 10th).
    # sample=False times plain graph replays only (the latency figures).
    model.profile(1, 0)  # clears the warm-up records
    model.profile(0, 0)
    step()  # one more warm-up step with the timer off: captures this shape's graph
    if sample:
        model.profile(1, 0)
    torch.cuda.synchronize()
    # Python's cyclic garbage collector is paused in the timed region (as
    # timeit does): a full collection of this interpreter's heap stalls the
    # host for ~40 ms, which starves the GPU and belongs to the calling
    # program, not to the library
    gc.collect()
    gc.disable()
    try:
        t0 = time.perf_counter()
        for i in range(steps):
            if sample:
                model.profile(2 if i % PROFILE_EVERY == 0 else 0, 1 << cls_id)
            step()
        torch.cuda.synchronize()
        t = time.perf_counter() - t0
    finally:
        gc.enable()
    dom_ms, dom_n = model.profile_read(cls_id)
    model.profile(0, 0)
    sampled = (steps + PROFILE_EVERY - 1) // PROFILE_EVERY if sample else 0
    return t, dominant, dom_ms, dom_n, per_class, sampled


def serve_timing(model, batch, handles=2, budget=32768, reps=5):
    """The ragged mix as independent host-side requests through jl_serve:
    length-sorted micro-batches of at most `budget` tokens on `handles`
    weight-sharing handles, one stream each, each micro-batch padded to a
    shape bucket and replayed from that bucket's captured graph; host in,
    host out (ids uploaded and results downloaded inside the timed region)."""
    from encoder_transformer_amd import lib
    req = lib.Requests([batch.sequence(b) for b in range(batch.n_seqs)])
    hs = [model.share(budget, 4096) for _ in range(handles)]
    for h in hs:  # micro-batches padded to shape buckets replay one graph per bucket
        h.set_graph_cache(16)
    try:
        lib.serve(hs, req, budget)  # first use: streams, buffers, code paths
        gc.collect()
        gc.disable()
        try:
            t0 = time.perf_counter()
            for _ in range(reps):
                res = lib.serve(hs, req, budget)
            t = (time.perf_counter() - t0) / reps
        finally:
            gc.enable()
        infos = [h.info() for h in hs]
    finally:
        for h in hs:
            h.close()
    return {"ms_per_queue": round(1e3 * t, 3), "requests_per_s": round(req.n / t, 1),
            "tokens_per_s": round(int(req.id_offsets[-1]) / t, 1), "micro_batches": res.n_batches,
            "handles": handles, "max_batch_tokens": budget, "host_to_host": True,
            "graph_captures": sum(i["graph_captures"] for i in infos),
            "graph_replays": sum(i["graph_replays"] for i in infos)}


def call_distribution(model, batch, calls=200):
    """Per-call figures at batch 1. Each call (graph replay) is bracketed by
    HIP events on its stream, which cost the stream a few microseconds; the
    end-to-end figure runs host ids to host logits (pinned copies on the same
    stream, then a synchronize), host-side validation included."""
    import torch
    so, mp, qt = batch.seq_offsets, batch.mask_positions, batch.qtype
    ids_h = torch.from_numpy(np.ascontiguousarray(batch.ids)).pin_memory()
    ids = ids_h.to("cuda:0")
    logits = torch.empty(batch.n_markers, dtype=torch.float32, device="cuda:0")
    logits_h = torch.empty(batch.n_markers, dtype=torch.float32).pin_memory()
    stream = torch.cuda.Stream()

    def call():
        with torch.cuda.stream(stream):
            model.forward(ids, so, mp, qt, out=logits)
            model.probs(logits, so, mp, qt)

    for _ in range(5):
        call()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
    gc.collect()
    gc.disable()
    try:
        for e0, e1 in ev:
            e0.record(stream)
            call()
            e1.record(stream)
        torch.cuda.synchronize()
        per = np.array([e0.elapsed_time(e1) for e0, e1 in ev])
        t0 = time.perf_counter()
        for _ in range(calls):
            with torch.cuda.stream(stream):
                ids.copy_(ids_h, non_blocking=True)
                model.forward(ids, so, mp, qt, out=logits)
                model.probs(logits, so, mp, qt)
                logits_h.copy_(logits, non_blocking=True)
            stream.synchronize()
        e2e = (time.perf_counter() - t0) / calls
    finally:
        gc.enable()
    p10, p50, p90 = np.percentile(per, [10, 50, 90])
    return {"calls": calls, "event_ms_p10": round(float(p10), 4), "event_ms_p50": round(float(p50), 4),
            "event_ms_p90": round(float(p90), 4), "host_to_host_ms_per_call": round(1e3 * e2e, 4)}


def cpu_baseline():
    """The oracle on six 1,024-token sequences of the throughput batch, with
    BLAS on every core this process may run on (its CPU affinity)."""
    from threadpoolctl import threadpool_limits
    from encoder_transformer_amd import synth
    from oracle import julia_oracle as jo
    cores = len(os.sched_getaffinity(0))
    W = jo.OracleWeights(synth.make_weights())
    batch = synth.make_batch(2)
    seqs = [0, 1, 2, 3, 4, 5]
    with threadpool_limits(limits=cores):
        t0 = time.perf_counter()
        jo.forward(W, batch, seqs)
        t = time.perf_counter() - t0
    return {"value": round(len(seqs) / t, 4), "unit": "decisions/s", "cores": cores, "kind": "oracle",
            "sample": f"6 of the 16 x 1,024-token sequences (6,144 tokens), float64 NumPy with {cores} BLAS "
                      f"threads, {t:.1f} s"}


def calibration_copy(mib):
    """A plain device copy of `mib` MiB (3 times), whose FETCH_SIZE / WRITE_SIZE
    counters calibrate the kernels' counter bytes in the same run."""
    if mib <= 0:
        return
    import torch
    src = torch.empty(mib << 18, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--latency-only", action="store_true",
                    help="time only the 1 x 1,024 call (graph replays; for a kernel trace of that workload)")
    ap.add_argument("--only", choices=["16x8192", "ragged256"],
                    help="time only this workload (graph replays; for profiles of that workload)")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="after timing, run a plain device copy of this size (for HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}): the forward pass shards by "
              "sequence with no cross-GPU traffic, and this build measures one GPU's share.", file=sys.stderr)
        sys.exit(2)

    import torch
    from encoder_transformer_amd import lib, synth
    assert torch.cuda.is_available(), "no GPU visible"
    path = synth.cached_weight_file()
    model = lib.Model(path, lib.BF16, max_tokens=300_000, max_markers=4096, device=0)
    model.set_graph_cache(8)  # steps replay captured graphs (profiled steps run eagerly)
    if args.latency_only:
        b1 = synth.make_batch(1)
        t1, *_ = time_workload(model, b1, args.steps, args.warmup, sample=False)
        model.close()
        calibration_copy(args.calibration_copy_mib)
        print(json.dumps({"metric": "ms per call at 1x1024", "value": round(1e3 * t1 / args.steps, 4), "unit": "ms",
                          "steps": args.steps, "warmup": args.warmup, "dtype": "bf16", "data": "synthetic",
                          "calls": 2 + max(1, args.warmup) + args.steps}))
        return

    if args.only:
        b = synth.make_batch({"16x8192": 3, "ragged256": 4}[args.only])
        tt, d, _, _, per_class, _ = time_workload(model, b, args.steps, args.warmup, sample=False)
        fl = sum(class_flops(b, row_block=b.n_tokens >= ROW_BLOCK_MIN_TOKENS).values())
        model.close()
        print(json.dumps({"metric": f"decisions/s at {args.only}", "value": round(b.n_seqs * args.steps / tt, 2),
                          "unit": "decisions/s", "ms_per_step": round(1e3 * tt / args.steps, 3),
                          "step_mfma_frac": round(fl / (tt / args.steps) / 1e12 / PEAK_BF16_TFLOPS, 4),
                          "device_ms_per_step_by_class": {k: round(v[0] / max(1, args.warmup), 4)
                                                          for k, v in per_class.items()},
                          "steps": args.steps, "warmup": args.warmup, "dtype": "bf16", "data": "synthetic"}))
        return

    b2 = synth.make_batch(2)
    t, dom, dom_ms, dom_n, per_class, sampled = time_workload(model, b2, args.steps, args.warmup)
    ms_step = 1e3 * t / args.steps
    flops = class_flops(b2, row_block=b2.n_tokens >= ROW_BLOCK_MIN_TOKENS)
    total_flops = sum(flops.values())
    dom_flops_step = flops[dom]
    achieved = dom_flops_step * sampled / (dom_ms * 1e-3) / 1e12 if dom_ms > 0 else 0.0
    from encoder_transformer_amd import profiling
    traffic = profiling.read_traffic(os.path.join(ROOT, "profiles"), dom)
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": None if traffic is None else round(traffic),
                "traffic_unit": "HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                "kernel": dom, "launches": dom_n, "avg_launch_us": round(1e3 * dom_ms / max(1, dom_n), 2)}

    result = {
        "metric": "decisions/s + tokens/s at 16×1024 bf16 (MFMA % peak); ms/call at 1×1024",
        "value": round(b2.n_seqs * args.steps / t, 2),
        "unit": "decisions/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "16 x 1,024-token questions (choice/score/noul cycling, 2-20 options of "
                               "1-48 tokens), packed unpadded; random-init Julia-1 weights (std 0.02)",
                   "global_batch": b2.n_seqs, "seq_len": 1024, "parallelism": "single GPU"},
        "tokens_per_s": round(b2.n_tokens * args.steps / t, 1),
        "step_tflops": round(total_flops / (ms_step * 1e-3) / 1e12, 2),
        "step_mfma_frac": round(total_flops / (ms_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "device_ms_per_step_by_class": {k: round(v[0] / max(1, args.warmup), 4) for k, v in per_class.items()},
        "roofline": roofline,
    }
    if not args.no_extra:
        extra = {}
        b1 = synth.make_batch(1)
        t1, *_ = time_workload(model, b1, max(args.steps, 20), args.warmup, sample=False)
        extra["1x1024_ms_per_call"] = round(1e3 * t1 / max(args.steps, 20), 4)
        extra["1x1024_calls"] = call_distribution(model, b1)
        # HBM rate of the call: algorithmic bytes, and the counter bytes
        # (FETCH_SIZE + WRITE_SIZE, copy-calibrated) of its committed summary
        call_s = t1 / max(args.steps, 20)
        alg = call_alg_bytes(b1)
        ctr = profiling.read_call_traffic(os.path.join(ROOT, "profiles"))
        extra["1x1024_hbm"] = {
            "alg_bytes": alg, "alg_GBps": round(alg / call_s / 1e9, 1),
            "alg_frac": round(alg / call_s / 1e9 / HBM_GBPS, 4),
            "counter_bytes": None if ctr is None else round(ctr),
            "counter_GBps": None if ctr is None else round(ctr / call_s / 1e9, 1),
            "counter_frac": None if ctr is None else round(ctr / call_s / 1e9 / HBM_GBPS, 4),
            "peak_GBps": HBM_GBPS}
        for name, cfg, st in [("16x8192", 3, 5), ("ragged256", 4, 5)]:
            b = synth.make_batch(cfg)
            tt, d, dms, dn, _, _ = time_workload(model, b, st, 2, sample=False)
            fl = sum(class_flops(b, row_block=b.n_tokens >= ROW_BLOCK_MIN_TOKENS).values())
            extra[name] = {"ms_per_step": round(1e3 * tt / st, 3), "decisions_per_s": round(b.n_seqs * st / tt, 2),
                           "tokens_per_s": round(b.n_tokens * st / tt, 1),
                           "step_mfma_frac": round(fl / (tt / st) / 1e12 / PEAK_BF16_TFLOPS, 4),
                           "dominant_kernel": d}
        extra["ragged256_serve"] = serve_timing(model, synth.make_batch(4))
        # FP32 mode (FP32 products and attention), for context against the
        # FP32 matrix-core peak; the headline is bf16
        m32 = lib.Model(path, lib.FP32, max_tokens=20_000, max_markers=1024, device=0)
        m32.set_graph_cache(2)
        for name, b, st in [("16x1024_fp32", b2, 5), ("1x1024_fp32", b1, 10)]:
            tt, *_ = time_workload(m32, b, st, 2, sample=False)
            fl = sum(class_flops(b, row_block=False).values())
            extra[name] = {"ms_per_step": round(1e3 * tt / st, 3), "decisions_per_s": round(b.n_seqs * st / tt, 2),
                           "fp32_peak_frac": round(fl / (tt / st) / 1e12 / PEAK_FP32_TFLOPS, 4)}
        m32.close()
        # FP8 mode (e4m3 QKV and W_i products: the row-block schedule at
        # 16 x 1,024, the per-GEMM one at 1 x 1,024), for context
        m8 = lib.Model(path, lib.FP8, max_tokens=20_000, max_markers=1024, device=0)
        m8.set_graph_cache(2)
        for name, b, st in [("16x1024_fp8", b2, 10), ("1x1024_fp8", b1, 20)]:
            tt, _, _, _, pc, _ = time_workload(m8, b, st, 2, sample=False)
            extra[name] = {"ms_per_step": round(1e3 * tt / st, 3), "decisions_per_s": round(b.n_seqs * st / tt, 2),
                           "device_ms_per_step_by_class": {k: round(v[0] / 2, 4) for k, v in pc.items() if v[1]}}
        m8.close()
        result["extra"] = extra
    result["ms_per_call_1x1024"] = result.get("extra", {}).get("1x1024_ms_per_call")
    model.close()
    calibration_copy(args.calibration_copy_mib)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
