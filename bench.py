#!/usr/bin/env python3
"""Benchmark of the paged-decode hot path on one MI355X.

One step = the whole hot path over one batch: the slot-mapped cache write of
one new token per sequence, then paged decode attention over the updated cache
(``seq_len + 1`` tokens per sequence). Inputs are seeded synthetic tensors of
the named workload, resident in HBM before timing starts.

Honest bandwidth: MI355X has a 256 MB memory-side cache, so consecutive steps
rotate over ``R`` device copies of the KV pools whose combined footprint is at
least 3x that cache; each step reads a pool that was last touched two steps
earlier (over 700 MB of other traffic in between for the GQA batch).

Prints one JSON line. ``value`` = compulsory HBM bytes of the step (K/V of
every cached token + Q + O + the written rows) / wall time per step.
``roofline`` covers the decode call, timed with HIP events on the stream it
runs on. ``cpu_baseline`` runs the fp64 oracle on the same batch on the host.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from paged_kv_cache_260_amd import _lib, accounting, profiling, workloads  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
FUSED_MERGE_PARTS = 8          # partition counts merged inside the decode kernel
MALL_BYTES = 256 * 2 ** 20     # memory-side (Infinity) cache
HOLD_CYCLES = 250_000          # GPU spin before the timed region (~0.1 ms)
METRIC = "paged decode effective HBM GB/s (% of MI355X peak) + us/batch, GQA bs=128"
DTYPE_NAMES = {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16"}
# profile summaries under profiles/, by workload
PROFILE_NAMES = {1: "paged_decode_tiny_f32_b4", 2: "paged_decode_mha_bf16_b64",
                 3: "paged_decode_gqa_bf16_b128", 4: "paged_decode_long_bf16_b4",
                 5: "paged_decode_prefix_f16_b64"}


def measured_traffic(cfg, fused=True, fp8=False):
    """(HBM bytes per timed call, where they come from): read back from the
    committed FETCH_SIZE/WRITE_SIZE summary of that step under profiles/, not
    measured in this run; (None, reason) when there is none or the decode
    source changed since the counters were taken."""
    return committed_traffic(PROFILE_NAMES[cfg] + ("_fp8" if fp8 else "") + ("" if fused else "_two_call"))


def committed_traffic(name):
    """(HBM bytes per call, source) from profiles/<name>_traffic.json, or
    (None, reason) when there is none or the decode source changed since."""
    rel = os.path.join("profiles", name + "_traffic.json")
    try:
        with open(os.path.join(ROOT, rel)) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None, f"no counter summary ({rel})"
    src = profiling.source_hash()
    if rec.get("decode_source_hash") != src or "traffic_bytes_per_call" not in rec:
        return None, f"{rel} was taken on decode source {rec.get('decode_source_hash')}, not {src}"
    return int(rec["traffic_bytes_per_call"]), f"from {rel} @ decode source {src} (rocprofv3 counters, earlier run)"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def stream_ceiling(device, nbytes=2 * 2 ** 30, iters=10):
    """Measured read ceilings (the library's probe kernels, pkv_probe.h) over
    a 2 GiB buffer, 8x the memory-side cache: a grid-stride non-temporal read,
    4 KiB tiles read in address order, and 4 KiB tiles in shuffled order (the
    decode kernel's pattern: one tile = one 16-token block of one KV head),
    the tile reads at 1, 2 and 4 tiles in flight per wave and two grid sizes
    (the best is reported with its configuration); and torch's device copy of
    the buffer (read + write bytes). HIP events on the stream they run on."""
    stream = torch.cuda.current_stream(device)
    buf = torch.empty(nbytes // 4, dtype=torch.int32, device=device).random_()
    cus = torch.cuda.get_device_properties(device).multi_processor_count
    sink = torch.zeros(64 * cus, dtype=torch.int32, device=device)
    tiles = torch.randperm(nbytes // 4096, device=device).to(torch.int32)

    def timed(run):
        run()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(iters):
            run()
        e1.record(stream)
        torch.cuda.synchronize()
        return nbytes * iters / (e0.elapsed_time(e1) * 1e-3) / 1e9

    res = {"stream_read": round(timed(lambda: _lib.probe_stream_read(buf, 8 * cus, sink, stream=stream)), 1)}
    seq = torch.arange(nbytes // 4096, device=device, dtype=torch.int32)
    for name, order in (("sequential_4k_tiles", seq), ("gather_4k_tiles", tiles)):
        best = (0.0, None)
        for depth in (1, 2, 4):
            for per_cu in (8, 16):
                g = timed(lambda: _lib.probe_gather_tiles(buf, order, depth, per_cu * cus, sink, stream=stream))
                if g > best[0]:
                    best = (g, f"{depth} tiles in flight per wave, {per_cu} workgroups of 4 waves per CU")
        res[name] = round(best[0], 1)
        res[name + "_config"] = best[1]
    # a plain device copy of the same buffer (read + write): the counter
    # summaries under profiles/ scale FETCH_SIZE and WRITE_SIZE by what this
    # copy of known size reads on them
    dst = torch.empty_like(buf)
    res["device_copy_rw"] = round(2 * timed(lambda: dst.copy_(buf)), 1)
    res["buffer_bytes"] = nbytes
    del seq, dst
    del buf, tiles, sink
    torch.cuda.empty_cache()
    return res


def cpu_baseline(w, lens_after, kp_after, vp_after, budget_s, fp8_scales=None):
    """The fp64 oracle on the same batch on host cores, repeated for ~budget_s.
    With ``fp8_scales`` = (k_scale, v_scale) the pools are e4m3 codes and the
    oracle's FP8 decode (dequantize, then attend) runs instead."""
    import oracle  # test infrastructure: only this leg of the benchmark runs it
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    qn = w.q.float().numpy()
    if fp8_scales is None:
        kp = kp_after.float().numpy()
        vp = vp_after.float().numpy()
    else:
        kp, vp = kp_after.numpy(), vp_after.numpy()
        ks, vs = (t.cpu().numpy() for t in fp8_scales)
    reps, t0 = 0, time.perf_counter()
    while True:
        if fp8_scales is None:
            oracle.paged_attn_decode(qn, kp, vp, w.block_tables, lens_after, w.scale, w.n_heads,
                                     w.n_kv_heads, w.head_dim, w.block_size)
        else:
            oracle.fp8.paged_attn_decode_fp8(qn, kp, vp, ks, vs, w.block_tables, lens_after, w.scale,
                                             w.n_heads, w.n_kv_heads, w.head_dim, w.block_size)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    per = el / reps
    nbytes = (accounting.decode_kv_bytes(lens_after, w.n_kv_heads, w.head_dim,
                                         1 if fp8_scales is not None else w.elem_bytes)
              + accounting.decode_qo_bytes(w.num_seqs, w.n_heads, w.head_dim, w.elem_bytes))
    return {"value": round(nbytes / per / 1e9, 4), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"whole batch ({w.num_seqs} seqs, {int(np.sum(lens_after))} tokens), "
                      f"{reps} passes in {el:.1f} s, {per * 1e3:.0f} ms/pass; "
                      f"numpy fp64, one Python thread driving BLAS with {threads} threads"}


def bench_copy_blocks(args, dev):
    """Copy-on-write block copy: pairs of 32 KiB bf16 blocks (8 KV heads x 16
    tokens x 128 dims) in both pools, timed with HIP events on the stream.
    Two workloads: one copy per sequence of a 128-sequence batch (what a
    parallel-sampling step asks for) and 8192 pairs (bandwidth)."""
    Hkv, BS, D, dt = 8, 16, 128, torch.bfloat16
    block_bytes = Hkv * BS * D * 2
    results = {}
    for name, npairs in (("cow_step_b128", 128), ("bulk_8192", 8192)):
        nb = 4 * npairs + 64
        reps = max(3, math.ceil(3 * MALL_BYTES / (2 * nb * block_bytes)))
        pools = [(torch.randn(nb, Hkv, BS, D, device=dev).to(dt), torch.randn(nb, Hkv, BS, D, device=dev).to(dt))
                 for _ in range(reps)]
        rng = np.random.default_rng(npairs)
        perm = rng.permutation(nb)
        pairs = torch.from_numpy(np.stack([perm[npairs:2 * npairs], perm[:npairs]], 1).astype(np.int32)).to(dev)
        for i in range(args.warmup):
            _lib.copy_blocks(*pools[i % reps], pairs)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(args.steps):
            _lib.copy_blocks(*pools[i % reps], pairs)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / args.steps
        moved = 2 * 2 * npairs * block_bytes  # K and V, read + write
        results[name] = {"pairs": npairs, "us": round(us, 3), "bytes": moved,
                         "GBps": round(moved / (us * 1e-6) / 1e9, 1)}
        del pools
        torch.cuda.empty_cache()
    bulk = results["bulk_8192"]
    print(json.dumps({
        "metric": "copy_blocks HBM GB/s (read + write, both pools)", "value": bulk["GBps"], "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "copy-on-write block copy, 32 KiB blocks (Hkv 8, BS 16, D 128, bf16)",
                   **{k: v for k, v in results.items()}},
        "roofline": {"bound": "hbm", "achieved": bulk["GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(bulk["GBps"] / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "copy_blocks_kernel", "algorithmic_bytes": bulk["bytes"]},
    }), flush=True)


def bench_chunk(args, dev):
    """Multi-token chunk attention on two workloads:
    - speculative verification: the GQA batch-128 shapes, each sequence
      scoring its last 4 tokens (HBM-bound, like decode);
    - chunked prefill: 4 sequences of 4 096 cached tokens, each scoring a
      512-token chunk (the last 512 tokens): a dense causal contraction
      (MFMA-bound in principle)."""
    results = {}
    cases = [("spec_verify_qlen4", workloads.make(3), 4),
             ("prefill_chunk512", workloads.build(name="prefill", rng=np.random.default_rng(2607),
                                                  seq_lens=np.full(4, 4096), n_heads=32, n_kv_heads=8,
                                                  head_dim=128, block_size=16, dtype=torch.bfloat16), 512)]
    for name, w, qlen in cases:
        qlens = np.minimum(qlen, w.seq_lens).astype(np.int64)
        qsl = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
        T = int(qsl[-1])
        q = torch.randn(T, w.n_heads, w.head_dim, device=dev).to(w.dtype)
        out = torch.empty_like(q)
        bt = torch.from_numpy(w.block_tables).to(dev)
        sl = torch.from_numpy(w.seq_lens).to(dev)
        qs = torch.from_numpy(qsl).to(dev)
        R = max(3, math.ceil(3 * MALL_BYTES / (2 * w.k_pool.numel() * w.elem_bytes)))
        kps = [w.k_pool.to(dev) for _ in range(R)]
        vps = [w.v_pool.to(dev) for _ in range(R)]
        call = lambda r: _lib.paged_attn_chunk(out, q, kps[r], vps[r], bt, sl, qs, w.scale, w.n_heads,
                                               w.n_kv_heads, w.head_dim, w.block_size, int(qlens.max()))
        for i in range(args.warmup):
            call(i % R)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(args.steps):
            call(i % R)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / args.steps
        kv = accounting.decode_kv_bytes(w.seq_lens, w.n_kv_heads, w.head_dim, w.elem_bytes)
        qo = 2 * T * w.n_heads * w.head_dim * w.elem_bytes
        # visible (query row, token) pairs: token i of a chunk of n sees L - n + i + 1 tokens
        pairs = int(sum(int(n) * (int(L) - int(n)) + int(n) * (int(n) + 1) // 2 for n, L in zip(qlens, w.seq_lens)))
        flops = 4 * pairs * w.n_heads * w.head_dim
        results[name] = {"qlen": qlen, "batch": w.num_seqs, "query_tokens": T, "us": round(us, 3),
                         "GBps": round((kv + qo) / (us * 1e-6) / 1e9, 1),
                         "TFLOPs": round(flops / (us * 1e-6) / 1e12, 2), "bytes": kv + qo, "flops": flops}
        del kps, vps
        torch.cuda.empty_cache()
    sv, pf = results["spec_verify_qlen4"], results["prefill_chunk512"]
    traffic, traffic_src = committed_traffic("paged_decode_chunk_rows_spec_verify_b128")
    extra = {} if args.no_ceiling else {"stream_ceiling_gbs": stream_ceiling(dev)}
    print(json.dumps({
        "metric": "chunk attention: effective HBM GB/s (speculative verify) and TFLOP/s (prefill chunk)",
        "value": sv["GBps"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "paged chunk attention, causal inside the chunk", **results},
        "roofline": {"bound": "hbm", "achieved": sv["GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(sv["GBps"] / HBM_PEAK_GBS, 4), "traffic": traffic, "traffic_source": traffic_src,
                     "kernel": "paged_decode_kernel, chunk rows (speculative verify)", "algorithmic_bytes": sv["bytes"]},
        "roofline_prefill": {"bound": "mfma", "achieved": pf["TFLOPs"], "peak": 2500.0, "unit": "TFLOP/s",
                             "frac": round(pf["TFLOPs"] / 2500.0, 4), "kernel": "paged_chunk_kernel (prefill chunk)",
                             "algorithmic_flops": pf["flops"]},
        **extra,
    }), flush=True)


def bench_shared_prefix(args, dev):
    """Decode of the 16-prompt x 4-sample fp16 workload (1024 shared prompt
    tokens per prompt) two ways: plain decode, which reads the shared blocks
    once per sample, and the shared-prefix call, which reads them once per
    prompt. Bandwidth is counted on the compulsory bytes (each physical block
    once, plus Q and O)."""
    w = workloads.make(5)
    gs, pl, mg = _lib.shared_prefix_groups(w.block_tables, w.seq_lens, w.block_size)
    uniq = accounting.unique_kv_tokens(w.seq_lens, w.block_tables, w.block_size)
    comp = uniq * w.n_kv_heads * w.head_dim * 2 * w.elem_bytes + accounting.decode_qo_bytes(
        w.num_seqs, w.n_heads, w.head_dim, w.elem_bytes)
    logical = accounting.decode_compulsory_bytes(w.seq_lens, w.n_heads, w.n_kv_heads, w.head_dim, w.elem_bytes)
    q = w.q.to(dev)
    out = torch.empty_like(q)
    bt = torch.from_numpy(w.block_tables).to(dev)
    sl = torch.from_numpy(w.seq_lens).to(dev)
    gsd = torch.from_numpy(gs).to(dev)
    pld = torch.from_numpy(pl).to(dev)
    R = max(3, math.ceil(3 * MALL_BYTES / (2 * w.k_pool.numel() * w.elem_bytes)))
    kps = [w.k_pool.to(dev) for _ in range(R)]
    vps = [w.v_pool.to(dev) for _ in range(R)]
    calls = {
        "shared_prefix": lambda r: _lib.paged_attn_decode_shared_prefix(
            out, q, kps[r], vps[r], bt, sl, pld, gsd, w.scale, w.n_heads, w.n_kv_heads, w.head_dim, w.block_size, mg),
        "plain_decode": lambda r: _lib.paged_attn_decode(out, q, kps[r], vps[r], bt, sl, w.scale, w.n_heads,
                                                         w.n_kv_heads, w.head_dim, w.block_size),
    }
    res = {}
    for name, call in calls.items():
        for i in range(args.warmup):
            call(i % R)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(args.steps):
            call(i % R)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / args.steps
        res[name] = {"us": round(us, 3), "GBps_compulsory": round(comp / (us * 1e-6) / 1e9, 1)}
    sp = res["shared_prefix"]
    traffic, traffic_src = committed_traffic("paged_shared_prefix_prompt_samples_f16")
    extra = {}
    if not args.no_ceiling:
        # also the 2 GiB device copy that scales FETCH_SIZE / WRITE_SIZE in
        # the counter summaries of this op
        extra["stream_ceiling_gbs"] = stream_ceiling(dev)
    print(json.dumps({
        "metric": "shared-prefix decode: compulsory-byte HBM GB/s", "value": sp["GBps_compulsory"], "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": workloads.CONFIG_NAMES[5], "groups": int(len(gs) - 1), "max_group_size": int(mg),
                   "compulsory_bytes": comp, "logical_bytes": logical, **res},
        "roofline": {"bound": "hbm", "achieved": sp["GBps_compulsory"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(sp["GBps_compulsory"] / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "traffic_source": traffic_src,
                     "kernel": "paged_attn_decode_shared_prefix call (decode kernel, shared mode, one launch)",
                     "algorithmic_bytes": comp},
        **extra,
    }), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=300,
                    help="untimed steps first (a few hundred let the GPU clocks settle)")
    ap.add_argument("--config", type=int, default=3, choices=[1, 2, 3, 4, 5],
                    help="workload (3 = GQA bf16 batch 128, the headline)")
    ap.add_argument("--replicas", type=int, default=0, help="pool copies to rotate (0 = auto)")
    ap.add_argument("--partition", type=int, default=0, help="partition tokens (0 = automatic)")
    ap.add_argument("--settle-ms", type=float, default=100.0,
                    help="after the warm-up steps, keep stepping (untimed) until this much wall time has passed")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true")
    ap.add_argument("--op", default="decode", choices=["decode", "copy_blocks", "chunk", "shared_prefix"],
                    help="decode = the hot-path step (default); copy_blocks = copy-on-write block copy")
    ap.add_argument("--step", default="append", choices=["append", "two-call"],
                    help="decode step: one call that appends the new token and decodes (default), or the "
                         "cache write followed by the decode call")
    ap.add_argument("--device-plan", action="store_true",
                    help="one-call step: pkv_paged_attn_decode_append[_fp8] (the kernel builds the work order "
                         "from the device lengths) instead of the planned call, which also takes the lengths in "
                         "host memory and builds the order on the host every call")
    ap.add_argument("--kv", default="native", choices=["native", "fp8"],
                    help="KV pool storage: the query dtype (default) or FP8 e4m3 codes with per-head scales")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(this build has no multi-GPU path).", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    _lib.lib()
    _lib.set_partition_tokens(args.partition)   # every op that runs the decode kernel
    if args.op == "copy_blocks":
        bench_copy_blocks(args, dev)
        return
    if args.op == "chunk":
        bench_chunk(args, dev)
        return
    if args.op == "shared_prefix":
        bench_shared_prefix(args, dev)
        return

    log(f"[bench] building workload config {args.config}")
    w = workloads.make(args.config)
    lens0 = w.seq_lens
    lens1 = w.seq_lens_after_write()
    e = w.elem_bytes
    fp8 = args.kv == "fp8"
    if fp8:
        if w.dtype == torch.float32:
            print("FP8 pools need a 16-bit workload", file=sys.stderr)
            sys.exit(2)
        # FP8 pools of the same workload: per-head scale amax / 448, codes by
        # torch's e4m3 conversion (input generation only)
        def to_codes(pool):
            sc = pool.float().abs().amax(dim=(0, 2, 3)).clamp_min(1e-6) / 448.0
            return (pool.float() / sc[None, :, None, None]).to(torch.float8_e4m3fn).view(torch.uint8), sc
        k_codes, k_sc = to_codes(w.k_pool)
        v_codes, v_sc = to_codes(w.v_pool)
    e_kv = 1 if fp8 else e
    pool_bytes = 2 * w.k_pool.numel() * e_kv
    R = args.replicas or max(3, math.ceil(3 * MALL_BYTES / pool_bytes))
    log(f"[bench] pools {pool_bytes / 2**20:.0f} MiB x {R} replicas")
    q = w.q.to(dev)
    out = torch.empty_like(q)
    bt = torch.from_numpy(w.block_tables).to(dev)
    sl = torch.from_numpy(lens1).to(dev)
    slots = torch.from_numpy(w.slot_mapping).to(dev)
    kn = w.k_new.to(dev)
    vn = w.v_new.to(dev)
    kps = [(k_codes if fp8 else w.k_pool).to(dev)]
    vps = [(v_codes if fp8 else w.v_pool).to(dev)]
    if fp8:
        ksd, vsd = k_sc.to(dev), v_sc.to(dev)
    for _ in range(R - 1):
        kps.append(kps[0].clone())
        vps.append(vps[0].clone())
    stream = torch.cuda.current_stream(dev)

    # 16-bit pools: one call appends the new token and decodes (the fused
    # step); --step two-call (and FP8 pools) time the write kernel, then decode
    # (the one-call step is built for 16-bit queries; fp32 always takes two calls)
    fused = args.step == "append" and w.dtype != torch.float32
    # the planned call (one-call step): the lengths also go in host
    # memory, as a serving loop's scheduler holds them, and the library builds
    # the work order from them on the host at every call (inside the timed steps)
    planned = fused and not args.device_plan
    lens_host = np.ascontiguousarray(lens1, dtype=np.int32) if planned else None

    def step(r, ev=None):
        if fused:
            if ev is not None:
                ev[0].record(stream)
            if fp8:
                _lib.paged_attn_decode_append_fp8(out, q, kps[r], vps[r], kn, vn, ksd, vsd, bt, sl, w.scale,
                                                  w.n_heads, w.n_kv_heads, w.head_dim, w.block_size, stream=stream,
                                                  seq_lens_host=lens_host)
            else:
                _lib.paged_attn_decode_append(out, q, kps[r], vps[r], kn, vn, bt, sl, w.scale, w.n_heads,
                                              w.n_kv_heads, w.head_dim, w.block_size, stream=stream,
                                              seq_lens_host=lens_host)
            if ev is not None:
                ev[1].record(stream)
            return
        if fp8:
            _lib.kv_cache_write_fp8(kps[r], vps[r], kn, vn, ksd, vsd, slots, stream=stream)
        else:
            _lib.kv_cache_write(kps[r], vps[r], kn, vn, slots, stream=stream)
        if ev is not None:
            ev[0].record(stream)
        if fp8:
            _lib.paged_attn_decode_fp8(out, q, kps[r], vps[r], ksd, vsd, bt, sl, w.scale, w.n_heads,
                                       w.n_kv_heads, w.head_dim, w.block_size, stream=stream)
        else:
            _lib.paged_attn_decode(out, q, kps[r], vps[r], bt, sl, w.scale, w.n_heads, w.n_kv_heads,
                                   w.head_dim, w.block_size, stream=stream)
        if ev is not None:
            ev[1].record(stream)

    log(f"[bench] warmup {args.warmup}")
    for i in range(args.warmup):
        step(i % R)
    torch.cuda.synchronize()
    # The GPU clocks take tens of milliseconds of steady work to settle (a run
    # timed after a few warm-up steps reads about 1.5 us per call slow): keep
    # stepping, untimed, until --settle-ms of back-to-back steps have run,
    # whatever --warmup asked for.
    settle_steps, t_settle = 0, time.perf_counter()
    while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms:
        for i in range(64):
            step(i % R)
        settle_steps += 64
        torch.cuda.synchronize()
    log(f"[bench] settle {settle_steps} steps")

    K = args.steps
    # pass 1 (the figure): K back-to-back steps bracketed by two events only;
    # an event recorded between kernels makes the next dispatch wait for it
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    log(f"[bench] timing {K} steps")
    torch.cuda.synchronize()
    # An untimed hold on the GPU (a spin of about 0.1 ms) before the start
    # event: the host then has the first timed steps queued by the time the
    # event runs, so the figure covers the K steps and not the host's latency
    # to submit the first one (about 10 us through the binding, 0.5 us per
    # step when K is 20).
    torch.cuda._sleep(HOLD_CYCLES)
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(K):
        step(i % R)
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = start.elapsed_time(stop) / K
    log(f"[bench] wall {wall * 1e3 / K:.4f} ms/step, events {ms_step:.4f} ms/step")
    # pass 2: the same K steps with events around each timed call, for the
    # spread of single calls (each includes one event's dispatch overhead)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(K)]
    torch.cuda.synchronize()
    for i in range(K):
        step(i % R, evs[i])
    torch.cuda.synchronize()
    dec_ms = np.array([a.elapsed_time(b) for a, b in evs])
    # The cache-write kernel alone (one new token per sequence), back to back.
    # It runs for a few microseconds, less than the host takes to submit a
    # call, so the calls are queued behind ~6 ms of probe reads (16 passes
    # over 2 GiB): the GPU then runs them without waiting for the host, and
    # the figure is the kernels' own (the host's submit time is printed
    # beside it as a check).
    n_w = 200
    blk = torch.empty(2 ** 29, dtype=torch.int32, device=dev)
    sink = torch.zeros(8 * torch.cuda.get_device_properties(dev).multi_processor_count, dtype=torch.int32,
                       device=dev)
    w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(16):
        _lib.probe_stream_read(blk, sink.numel(), sink, stream=stream)
    h0 = time.perf_counter()
    w0.record(stream)
    for i in range(n_w):
        if fp8:
            _lib.kv_cache_write_fp8(kps[i % R], vps[i % R], kn, vn, ksd, vsd, slots, stream=stream)
        else:
            _lib.kv_cache_write(kps[i % R], vps[i % R], kn, vn, slots, stream=stream)
    w1.record(stream)
    submit_us = (time.perf_counter() - h0) * 1e6 / n_w
    torch.cuda.synchronize()
    write_us = w0.elapsed_time(w1) * 1e3 / n_w
    del blk, sink

    # compulsory bytes: K/V of each distinct cached token slot once (blocks that
    # several tables share, as in the shared-prompt workload, count once), Q, O
    uniq = accounting.unique_kv_tokens(lens1, w.block_tables, w.block_size)
    logical_kv = accounting.decode_kv_bytes(lens1, w.n_kv_heads, w.head_dim, e_kv)
    dec_bytes = (uniq * w.n_kv_heads * w.head_dim * 2 * e_kv
                 + accounting.decode_qo_bytes(w.num_seqs, w.n_heads, w.head_dim, e))
    n_written = int((w.slot_mapping >= 0).sum())
    # the step's compulsory bytes: decode at the new lengths (which reads each
    # new K/V row once) plus the new rows stored into the pools
    store_bytes = 2 * n_written * w.n_kv_heads * w.head_dim * e_kv
    step_bytes = dec_bytes + store_bytes
    value = step_bytes / (ms_step * 1e-3) / 1e9
    dec_mean = float(dec_ms.mean())
    # the timed call: the whole step when fused (one launch per step, so its
    # average duration is the back-to-back figure of pass 1), else the decode
    # call alone (its mean over the individually bracketed calls of pass 2)
    call_bytes = step_bytes if fused else dec_bytes
    call_ms = ms_step if fused else dec_mean
    achieved = call_bytes / (call_ms * 1e-3) / 1e9
    ptok, nparts = _lib.decode_plan(w.n_heads, w.n_kv_heads, w.block_size, w.num_seqs,
                                    w.max_blocks_per_seq)
    traffic, traffic_source = measured_traffic(args.config, fused, fp8)

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE_NAMES[w.dtype] + ("/fp8-e4m3 KV" if fp8 else ""),
        "data": "synthetic",
        "config": {
            "workload": w.name + (" with FP8 e4m3 KV pools (per-head scales)" if fp8 else ""),
            "batch": w.num_seqs, "n_heads": w.n_heads, "n_kv_heads": w.n_kv_heads,
            "head_dim": w.head_dim, "block_size": w.block_size,
            "cached_tokens": int(lens1.sum()), "mean_seq_len": round(float(lens1.mean()), 1),
            "max_seq_len": int(lens1.max()), "num_blocks": w.num_blocks,
            "partition_tokens": ptok, "max_partitions": nparts, "pool_replicas": R,
            "step": (f"paged_attn_decode_append{'_fp8' if fp8 else ''}{'_planned' if planned else ''}: one call "
                     f"writes the new token (1 per seq) and decodes seq_len+1"
                     + (" (work order built on the host from the host copy of the lengths, every call)"
                        if planned else "") if fused else
                     f"kv_cache_write{'_fp8' if fp8 else ''} (1 token/seq) + paged_attn_decode{'_fp8' if fp8 else ''} "
                     f"(seq_len+1)"),
        },
        "pct_of_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "us_per_batch": round(ms_step * 1e3, 3),
        ("call_us" if fused else "decode_us"): {"mean": round(dec_mean * 1e3, 3),
                      "p10": round(float(np.percentile(dec_ms, 10)) * 1e3, 3),
                      "p50": round(float(np.percentile(dec_ms, 50)) * 1e3, 3),
                      "p90": round(float(np.percentile(dec_ms, 90)) * 1e3, 3)},
        "step_bytes": int(step_bytes),
        "logical_kv_bytes": int(logical_kv),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "traffic_source": traffic_source,
                     "kernel": ("paged_attn_decode_append" if fused else "paged_attn_decode")
                               + ("_fp8" if fp8 else "") + ("_planned" if planned else "")
                               + " call (decode kernel"
                               + (")" if nparts == 1 else
                                  ", partitions merged in-kernel)" if nparts <= FUSED_MERGE_PARTS else
                                  " + partition merge kernel)"),
                     "algorithmic_bytes": int(call_bytes), "call_us": round(call_ms * 1e3, 3)},
        "wall_ms_per_step": round(wall * 1e3 / K, 5),
        "settle_steps": settle_steps,
        "write_kernel_us": {"us": round(write_us, 3), "tokens": n_written, "host_submit_us": round(submit_us, 2),
                            "note": f"kv_cache_write{'_fp8' if fp8 else ''} alone, {n_w} calls queued behind "
                                    f"probe reads and run back to back"},
    }
    if not args.no_ceiling:
        log("[bench] read ceilings (probe kernels)")
        result["stream_ceiling_gbs"] = stream_ceiling(dev)
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        torch.cuda.synchronize()
        kp_after = kps[0].cpu()
        vp_after = vps[0].cpu()
        result["cpu_baseline"] = cpu_baseline(w, lens1, kp_after, vp_after, args.cpu_seconds,
                                              (ksd, vsd) if fp8 else None)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
