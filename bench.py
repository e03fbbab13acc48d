"""Benchmark: latent-space MLA decode on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload dsv3|jagged|spec|fp8|tiny]

One step = the whole hot path over one batch: the split plan (mla_get_split_plan) and the
decode with its split combine (mla_decode_fwd), with inputs already resident in HBM. The
default workload is the DeepSeek-V3-shaped decode b=64, s=1, h=128, t=4096, k=512, p=64,
bf16 paged cache (64-token pages in shuffled physical order), fp32 out + lse.

To keep the 256 MB Infinity Cache from serving the KV cache, the step cycles through
`--rotate` full copies of the cache (>= 1 GiB in total by default).

Prints ONE JSON line (metric, value = us per step, roofline of the decode call, cpu_baseline
= the fp64 oracle timed on a bounded sample of the same workload on the host cores).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MLA decode µs/call, TFLOPS + HBM GB/s (% roofline), b=64 h=128 t=4096 bf16"
PEAK_HBM_GBPS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP8_TFLOPS = 5000.0
K_LAT, P_ROPE = 512, 64


def workload_bytes(w) -> float:
    """Algorithmic HBM bytes of one decode call at the real dtypes: the live tokens of the
    cache, the queries, out (fp32) and lse (fp32), block table and lengths."""
    import numpy as np
    per_tok = 576 * 2 if w.kv_dtype == "bf16" else 640 + 16
    kv = float(np.sum(w.seqlens.astype(np.int64))) * per_tok
    return kv + w.q.size * 2 + w.batch * w.s_q * w.heads * (K_LAT * 4 + 4) + w.block_table.size * 4 + w.batch * 4


def workload_flops(w) -> float:
    """2*b*h*s*t*(2k+p) (the page's FlashMLA cost model), summed over sequences."""
    return float(sum(2.0 * w.heads * w.s_q * int(t) * (2 * K_LAT + P_ROPE) for t in w.seqlens))


def describe(w) -> str:
    import numpy as np
    lens = w.seqlens
    t = f"t={int(lens[0])}" if np.all(lens == lens[0]) else f"t={int(lens.min())}..{int(lens.max())} (sum {int(lens.sum())})"
    return (f"{w.name}: b={w.batch} s={w.s_q} h={w.heads} k=512 p=64 {t} {w.kv_dtype} cache, 64-token pages "
            f"in shuffled order{', causal' if w.causal else ''}, fp32 out+lse")


# kernel sources whose sha256 keys the committed HBM-traffic record
TRAFFIC_SOURCES = ("mla_device.h", "mla_decode_rows32.hip", "mla_plan.hip")


def traffic_from_profile(kernel_srcs, key):
    """HBM traffic of the decode call from a committed rocprofv3 PMC summary, only if it was
    taken on the current kernel sources (sha256 of the .hip files)."""
    path = os.path.join(ROOT, "profiles", "decode_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except Exception:
        return None
    h = hashlib.sha256()
    for p in kernel_srcs:
        h.update(open(p, "rb").read())
    if rec.get("sources_sha256") != h.hexdigest():
        return None
    return rec.get(key, {}).get("bytes_per_call")


def _events_us(stream, fn, n: int) -> float:
    """Mean µs per call of fn(i), i < n, from one pair of HIP events on `stream` around n
    back-to-back calls (a pair per call would add its own gaps between the calls)."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(n):
        fn(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / n


def projections(w, steps: int, warmup: int, copies: int = 16):
    """The two projections around the attention at this workload's shape (tokens = b*s, h
    heads), each timed with one pair of HIP events on the launch stream around `steps`
    back-to-back calls, cycling through `copies` sets of weights (more than the 256 MB
    Infinity Cache holds) with seeded random values: query absorption (mla_absorb_query) and
    output decompression (mla_decompress_output). Bytes are the algorithmic reads and writes
    of one call."""
    import torch
    import mla_latent_space_amd as mla
    dev = "cuda"
    T, H = w.batch * w.s_q, w.heads
    gen = torch.Generator(device=dev).manual_seed(5)
    bf = lambda *shape: torch.randn(shape, generator=gen, device=dev).to(torch.bfloat16)
    q_nope, q_rope = bf(T, H, 128), bf(T, H, 64)
    w_k = [bf(H, 512, 128) for _ in range(copies)]
    w_v = [bf(H, 128, 512) for _ in range(copies)]
    o_lat = torch.randn((T, H, 512), generator=gen, device=dev)
    qz = torch.empty((T, H, 576), dtype=torch.bfloat16, device=dev)
    out = torch.empty((T, H, 128), dtype=torch.float32, device=dev)
    calls = {
        "absorb_query": (lambda i: mla.absorb_query(q_nope, q_rope, w_k[i % copies], out=qz),
                         T * H * (128 + 64 + 576) * 2 + H * 512 * 128 * 2),
        "decompress_output": (lambda i: mla.decompress_output(o_lat, w_v[i % copies], out=out),
                              T * H * (512 + 128) * 4 + H * 128 * 512 * 2),
    }
    stream = torch.cuda.current_stream()
    res = {}
    for name, (fn, byts) in calls.items():
        for i in range(warmup):
            fn(i)
        us = _events_us(stream, fn, steps)
        gbps = byts / (us * 1e-6) / 1e9
        res[name] = {"us": round(us, 2), "bytes": byts, "flops": 2 * T * H * 512 * 128,
                     "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                                  "frac": round(gbps / PEAK_HBM_GBPS, 4)}}
    return res


def hybrid(steps: int, warmup: int, b: int = 32, s_q: int = 16, heads: int = 128, t: int = 4096, n: int = 640):
    """The split latent + decompressed variant at the pages' s=16 configuration (b=32, h=128,
    t=4096): o = t - n old tokens as a paged latent cache, the n newest decompressed (K, V of
    128 channels per head, the shared rope key). One hybrid step = query absorption, plan and
    latent decode over the old tokens, output decompression, then mla_hybrid_merge over the
    new tokens (causal). Beside it the all-latent step at the same shape (absorption, plan,
    causal decode over t tokens, decompression). n = 640 is where the cost model balances the
    MFMA time of the latent tokens against the HBM time of the decompressed ones on MI355X.
    Seeded random inputs generated on the device; two copies of every cache are cycled."""
    import torch
    import mla_latent_space_amd as mla
    dev = "cuda"
    o = t - n
    gen = torch.Generator(device=dev).manual_seed(11)
    bf = lambda *shape: torch.randn(shape, generator=gen, device=dev).to(torch.bfloat16)
    scale = (128 + 64) ** -0.5

    def paged(tokens, copies=2):
        per = (tokens + 63) // 64
        caches = [bf(b * per, 64, 576) for _ in range(copies)]
        bt = torch.randperm(b * per, generator=gen, device=dev).to(torch.int32).view(b, per).contiguous()
        return caches, bt, torch.full((b,), tokens, dtype=torch.int32, device=dev)

    kv_old, bt_old, sl_old = paged(o)
    kv_all, bt_all, sl_all = paged(t)
    q_nope, q_rope = bf(b, s_q, heads, 128), bf(b, s_q, heads, 64)
    w_k = bf(heads, 512, 128) * (128 ** -0.5)
    w_v = bf(heads, 128, 512) * (512 ** -0.5)
    news = [(bf(b, n, heads, 128), bf(b, n, 64), bf(b, n, heads, 128)) for _ in range(2)]
    W = mla.default_num_workers(0)
    qz = torch.empty((b, s_q, heads, 576), dtype=torch.bfloat16, device=dev)
    o_lat = torch.empty((b, s_q, heads, 512), dtype=torch.float32, device=dev)
    lse_a = torch.empty((b, s_q, heads), dtype=torch.float32, device=dev)
    out_old = torch.empty((b, s_q, heads, 128), dtype=torch.float32, device=dev)
    out = torch.empty_like(out_old)
    lse = torch.empty_like(lse_a)
    ws = torch.empty(max(mla.workspace_bytes(b, s_q, heads, W), 16), dtype=torch.uint8, device=dev)
    plan_buf = torch.empty(mla.plan_bytes(b, s_q, heads, W), dtype=torch.uint8, device=dev)

    def latent_part(i, kv, bt, sl, causal):
        mla.absorb_query(q_nope, q_rope, w_k, out=qz)
        plan = mla.get_split_plan(sl, s_q, heads, causal, W, out=plan_buf)
        mla.decode_fwd(qz, kv[i % 2], bt, sl, scale, causal=causal, plan=plan, workspace=ws, out=o_lat, lse=lse_a)
        mla.decompress_output(o_lat, w_v, out=out_old)

    def merge(i):
        k_new, kr_new, v_new = news[i % 2]
        mla.hybrid_merge(q_nope, q_rope, k_new, kr_new, v_new, out_old, lse_a, scale, causal=True, out=out, lse=lse)

    def hybrid_step(i):
        latent_part(i, kv_old, bt_old, sl_old, False)
        merge(i)

    def latent_step(i):
        latent_part(i, kv_all, bt_all, sl_all, True)

    def wall_us(fn):
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            fn(i)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps * 1e6

    hyb_us, lat_us = wall_us(hybrid_step), wall_us(latent_step)
    # the merge alone: back-to-back calls on the latent part of the last step
    latent_part(0, kv_old, bt_old, sl_old, False)
    merge_us = _events_us(torch.cuda.current_stream(), merge, steps)
    rows = b * s_q * heads
    merge_bytes = b * n * heads * 128 * 2 * 2 + b * n * 64 * 2 + rows * ((128 + 64) * 2 + 2 * 128 * 4 + 2 * 4)
    merge_flops = 4.0 * b * heads * s_q * n * 128 + 2.0 * b * heads * s_q * n * 64
    gbps = merge_bytes / (merge_us * 1e-6) / 1e9
    # the pages' cost models (FLOPs, bytes at w = 2)
    lat_flops = 2.0 * b * heads * s_q * t * (2 * K_LAT + P_ROPE)
    lat_bytes = 2.0 * (b * heads * s_q * (2 * K_LAT + P_ROPE) + b * t * (K_LAT + P_ROPE))
    hyb_flops = 2.0 * b * heads * s_q * t * P_ROPE + 4.0 * b * heads * s_q * n * 128 + 4.0 * b * heads * s_q * o * K_LAT
    hyb_bytes = 2.0 * (b * heads * s_q * (P_ROPE + 128 + K_LAT) + b * o * K_LAT + b * t * P_ROPE
                       + 2 * b * heads * n * 128 + b * heads * s_q * (128 + K_LAT))
    bound = lambda f, by: max(f / (PEAK_BF16_TFLOPS * 1e12), by / (PEAK_HBM_GBPS * 1e9)) * 1e6
    return {"workload": f"b={b} s={s_q} h={heads} t={t}: o={o} latent (bf16 paged) + n={n} decompressed, causal",
            "hybrid_step_us": round(hyb_us, 2), "latent_step_us": round(lat_us, 2),
            "merge_us": round(merge_us, 2),
            "merge_roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                               "frac": round(gbps / PEAK_HBM_GBPS, 4), "bytes": merge_bytes, "flops": merge_flops},
            "cost_model_bound_us": {"latent": round(bound(lat_flops, lat_bytes), 1),
                                    "hybrid": round(bound(hyb_flops, hyb_bytes), 1)}}


def sparse(steps: int, warmup: int, b: int = 64, t: int = 32768, topk: int = 2048, heads: int = 128):
    """Token-level sparse decode over an fp8 cache at a DeepSeek-V3.2-like shape: b=64 sequences
    of t=32,768 cached tokens (s=1, h=128), each query token attending to its own 2,048 selected
    tokens (a seeded uniform choice without replacement, in random order). One step = the row
    lists and split plan (mla_get_sparse_plan) and the decode (mla_sparse_decode_fwd). Seeded
    random codes (NaN codes excluded), scales and rope values generated on the device."""
    import torch
    import mla_latent_space_amd as mla
    dev = "cuda"
    gen = torch.Generator(device=dev).manual_seed(21)
    per = t // 64
    pages = b * per
    codes = torch.randint(0, 256, (pages, 64, 512), generator=gen, device=dev, dtype=torch.int32)
    codes = torch.where((codes & 0x7F) == 0x7F, torch.zeros_like(codes), codes).to(torch.uint8)
    rope = torch.randn((pages, 64, 64), generator=gen, device=dev).to(torch.bfloat16).view(torch.uint8)
    kv = torch.cat([codes, rope], dim=2).contiguous()
    del codes, rope
    scales = (torch.rand((pages, 64, 4), generator=gen, device=dev) * 0.01 + 1e-3).contiguous()
    bt = torch.randperm(pages, generator=gen, device=dev).to(torch.int32).view(b, per).contiguous()
    sl = torch.full((b,), t, dtype=torch.int32, device=dev)
    idx = torch.stack([torch.randperm(t, generator=gen, device=dev)[:topk] for _ in range(b)]).to(torch.int32)
    idx = idx.view(b, 1, topk).contiguous()
    q = torch.randn((b, 1, heads, 576), generator=gen, device=dev).to(torch.bfloat16)
    scale = (128 + 64) ** -0.5
    W = mla.default_num_workers(0)
    ws = torch.empty(max(mla.workspace_bytes(b, 1, heads, W), 16), dtype=torch.uint8, device=dev)
    out = torch.empty((b, 1, heads, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((b, 1, heads), dtype=torch.float32, device=dev)
    plan = mla.get_sparse_plan(idx, bt, sl, pages, heads, W)

    def step(i):
        mla.get_sparse_plan(idx, bt, sl, pages, heads, W)
        mla.sparse_decode_fwd(q, kv, scales, scale, plan, workspace=ws, out=out, lse=lse)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    step_us = (time.perf_counter() - t0) / steps * 1e6
    dec_us = _events_us(torch.cuda.current_stream(),
                        lambda i: mla.sparse_decode_fwd(q, kv, scales, scale, plan, workspace=ws, out=out, lse=lse),
                        max(steps, 200))
    rows = b * heads
    byts = float(b * topk * (512 + 128 + 16) + b * topk * 4 + rows * 576 * 2 + rows * (512 + 1) * 4)
    flops = 2.0 * rows * topk * (2 * K_LAT + P_ROPE)
    tf = flops / (dec_us * 1e-6) / 1e12
    bound_us = max(flops / (PEAK_BF16_TFLOPS * 1e12), byts / (PEAK_HBM_GBPS * 1e9)) * 1e6
    return {"workload": f"b={b} s=1 h={heads} t={t} fp8 cache, top-{topk} tokens per query token",
            "step_us": round(step_us, 2), "decode_us": round(dec_us, 2),
            "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / PEAK_BF16_TFLOPS, 4), "bytes": byts, "flops": flops,
                         "bound_us": round(bound_us, 2)}}


_POOL_ARRAYS = None


def _oracle_attach(names, shapes, dtypes):
    """Pool initializer of the cpu_baseline workers: map the workload arrays from shared memory
    (read only; the parent owns and unlinks the segments)."""
    global _POOL_ARRAYS
    from multiprocessing import shared_memory
    import numpy as np
    arrs, keep = [], []
    for n, sh, dt in zip(names, shapes, dtypes):
        if n is None:
            arrs.append(None)
            continue
        m = shared_memory.SharedMemory(name=n)   # (spawned workers share the parent's resource tracker)
        keep.append(m)
        arrs.append(np.ndarray(sh, dtype=dt, buffer=m.buf))
    _POOL_ARRAYS = (arrs, keep)


def _oracle_worker(args):
    """One task of the cpu_baseline pool: the oracle over the given sequences."""
    scale, kv_dtype, causal, seqs = args
    from oracle import mla as om
    q, kv, sc, bt, sl = _POOL_ARRAYS[0]
    om.decode_latent(q, kv, sc, kv_dtype, bt, sl, scale, causal, seqs)
    return len(seqs)


def cpu_baseline(w, budget_s: float):
    """The oracle (as is) on the host cores: a pool of N = len(sched_getaffinity) worker processes,
    each with one BLAS thread, over the workload's sequences in shared memory. Whole passes over
    the batch are repeated until about budget_s of wall time; the result is wall time per pass."""
    import multiprocessing as mp
    from multiprocessing import shared_memory
    import numpy as np
    ncpu = len(os.sched_getaffinity(0))
    model = "unknown CPU"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    arrays = [w.q, w.kv, w.kv_scales, w.block_table, w.seqlens]
    shms, names, shapes, dtypes = [], [], [], []
    try:
        for x in arrays:
            if x is None:
                shms.append(None); names.append(None); shapes.append(None); dtypes.append(None)
                continue
            m = shared_memory.SharedMemory(create=True, size=max(1, x.nbytes))
            np.ndarray(x.shape, dtype=x.dtype, buffer=m.buf)[...] = x
            shms.append(m); names.append(m.name); shapes.append(x.shape); dtypes.append(x.dtype)
        # work items: sequences, longest first, dealt to the pool one by one
        order = [int(i) for i in np.argsort(-w.seqlens.astype(np.int64), kind="stable")]
        env_keys = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")
        saved = {k: os.environ.get(k) for k in env_keys}
        for k in env_keys:
            os.environ[k] = "1"   # one BLAS thread per worker process (inherited at spawn)
        try:
            ctx = mp.get_context("spawn")
            with ctx.Pool(ncpu, initializer=_oracle_attach, initargs=(names, shapes, dtypes)) as pool:
                pool.map(_oracle_worker, [(w.scale, w.kv_dtype, w.causal, order[:1])] * ncpu, chunksize=1)
                passes = 0
                t0 = time.perf_counter()
                while True:
                    pool.map(_oracle_worker, [(w.scale, w.kv_dtype, w.causal, [i]) for i in order], chunksize=1)
                    passes += 1
                    el = time.perf_counter() - t0
                    if el >= budget_s or (passes >= 1 and el * (passes + 1) / passes > 3 * budget_s):
                        break
        finally:
            for k, v in saved.items():
                if v is None:
                    os.environ.pop(k, None)
                else:
                    os.environ[k] = v
    finally:
        for m in shms:
            if m is not None:
                m.close()
                m.unlink()
    return {"value": round(el / passes * 1e6, 1), "unit": "µs/call", "cores": ncpu, "kind": "oracle",
            "sample": f"fp64 oracle over the whole {w.name} batch ({w.batch} sequences), {passes} pass(es) in "
                      f"{el:.1f} s of wall time on a pool of {ncpu} processes with one BLAS thread each "
                      f"({model})"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=500,
                    help="untimed steps first (the clocks settle over the first few hundred steps)")
    ap.add_argument("--workload", default="dsv3")
    ap.add_argument("--rotate", type=int, default=0, help="KV copies to cycle through (0: enough for >= 1 GiB)")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-projections", action="store_true",
                    help="skip timing the query-absorption and output-decompression kernels")
    ap.add_argument("--hybrid", action="store_true",
                    help="also time the split latent + decompressed variant (its latent part runs the same decode "
                         "kernel, so it stays out of the default run's kernel trace)")
    ap.add_argument("--sparse", action="store_true", help="also time the token-sparse fp8 decode")
    ap.add_argument("--no-measured", action="store_true",
                    help="skip the microbenchmarks that measure this device's stream-read rate and MFMA peak")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB --steps times (the reference "
                         "kernel for scaling HBM byte counters), print its size and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: it measures the single-GPU decode path, "
              "so --gpus must be 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import mla_latent_space_amd as mla
    from mla_latent_space_amd import workloads as wl

    torch.cuda.set_device(0)
    if args.copy_calibration:
        nbytes = args.copy_calibration << 20
        src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": nbytes, "calls": args.steps}), flush=True)
        return
    w = wl.make_config(args.workload)
    print(f"[bench] {args.workload} inputs drawn", file=sys.stderr, flush=True)
    dev = torch.device("cuda", 0)
    q = torch.from_numpy(w.q.view(np.int16)).to(dev).view(torch.bfloat16)
    if w.kv_dtype == "bf16":
        kv0 = torch.from_numpy(w.kv.view(np.int16)).to(dev).view(torch.bfloat16)
        sc0 = None
    else:
        kv0 = torch.from_numpy(w.kv).to(dev)
        sc0 = torch.from_numpy(w.kv_scales).to(dev)
    kv_bytes = kv0.numel() * kv0.element_size() + (0 if sc0 is None else sc0.numel() * 4)
    rot = args.rotate or max(1, math.ceil((1 << 30) / kv_bytes))
    kvs = [kv0] + [kv0.clone() for _ in range(rot - 1)]
    scs = [sc0] + [None if sc0 is None else sc0.clone() for _ in range(rot - 1)]
    bt = torch.from_numpy(w.block_table).to(dev)
    sl = torch.from_numpy(w.seqlens).to(dev)
    W = mla.default_num_workers(0)
    out = torch.empty(w.batch, w.s_q, w.heads, 512, dtype=torch.float32, device=dev)
    lse = torch.empty(w.batch, w.s_q, w.heads, dtype=torch.float32, device=dev)
    ws_bytes = mla.workspace_bytes(w.batch, w.s_q, w.heads, W)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    plan_buf = torch.empty(mla.plan_bytes(w.batch, w.s_q, w.heads, W), dtype=torch.uint8, device=dev)

    def step(i):
        plan = mla.get_split_plan(sl, w.s_q, w.heads, w.causal, W, out=plan_buf)
        mla.decode_fwd(q, kvs[i % rot], bt, sl, w.scale, kv_scales=scs[i % rot], causal=w.causal, plan=plan,
                       workspace=ws, out=out, lse=lse)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # timed region: K whole steps, nothing else on the stream
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_us = wall / args.steps * 1e6
    # then the two calls on their own, each timed with one pair of HIP events on the launch
    # stream around K back-to-back calls (the plan once per decode step, the decode once per
    # layer of that step, so the decode calls reuse one plan)
    stream = torch.cuda.current_stream()
    # (at least 200 calls each, so that a short run still averages over a steady state)
    plan = mla.get_split_plan(sl, w.s_q, w.heads, w.causal, W, out=plan_buf)
    # events after every chunk of 10 calls as well (a marker on the stream, no gap between
    # calls): the chunk means give the spread
    chunk = 10
    n_calls = max(args.steps, 200) // chunk * chunk
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n_calls // chunk + 1)]
    e2 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i in range(n_calls):
        mla.decode_fwd(q, kvs[i % rot], bt, sl, w.scale, kv_scales=scs[i % rot], causal=w.causal, plan=plan,
                       workspace=ws, out=out, lse=lse)
        if (i + 1) % chunk == 0:
            ev[(i + 1) // chunk].record(stream)
    for i in range(n_calls):
        mla.get_split_plan(sl, w.s_q, w.heads, w.causal, W, out=plan_buf)
    e2.record(stream)
    torch.cuda.synchronize()
    dec_mean = ev[0].elapsed_time(ev[-1]) * 1e3 / n_calls
    plan_mean = ev[-1].elapsed_time(e2) * 1e3 / n_calls
    chunk_us = np.array([ev[c].elapsed_time(ev[c + 1]) * 1e3 / chunk for c in range(len(ev) - 1)])
    dec_pct = [round(float(np.percentile(chunk_us, p)), 2) for p in (10, 50, 90)]

    flops = workload_flops(w)
    byts = workload_bytes(w)
    achieved_gbps = byts / (dec_mean * 1e-6) / 1e9
    tflops = flops / (dec_mean * 1e-6) / 1e12
    ai = flops / byts
    bound_us = max(byts / (PEAK_HBM_GBPS * 1e9), flops / (PEAK_BF16_TFLOPS * 1e12)) * 1e6
    bound = "hbm" if byts / (PEAK_HBM_GBPS * 1e9) >= flops / (PEAK_BF16_TFLOPS * 1e12) else "mfma"
    srcs = [os.path.join(ROOT, "mla_latent_space_amd", "csrc", f) for f in TRAFFIC_SOURCES]
    traffic = traffic_from_profile(srcs, args.workload)
    if bound == "hbm":
        roof = {"bound": "hbm", "achieved": round(achieved_gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": round(achieved_gbps / PEAK_HBM_GBPS, 4), "traffic": traffic}
    else:
        roof = {"bound": "mfma", "achieved": round(tflops, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tflops / PEAK_BF16_TFLOPS, 4), "traffic": traffic}
    rec = {
        "metric": METRIC,
        "value": round(step_us, 2),
        "unit": "µs/call",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_us / 1e3, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": describe(w), "kv_copies_rotated": rot, "num_workers": W},
        "decode_us": round(dec_mean, 2),
        "decode_us_p10_p50_p90": dec_pct,
        "plan_us": round(plan_mean, 2),
        "tflops": round(tflops, 1),
        "hbm_gbps": round(achieved_gbps, 1),
        "arith_intensity": round(ai, 1),
        "roofline_bound_us": round(bound_us, 2),
        "roofline_frac_of_bound": round(bound_us / dec_mean, 4),
        "roofline": dict(roof, kernel="mla_decode_fwd: decode_rows32_kernel, then combine_rows32_kernel (the "
                                      "merge of split items)", bytes_per_call=byts, flops_per_call=flops),
    }
    if w.kv_dtype == "fp8":
        # the same call priced as if its products ran in fp8 (the kernel dequantises to bf16 and
        # runs bf16 MFMAs): then the HBM time of its 656-B rows bounds it
        hbm_us, f8_us = byts / (PEAK_HBM_GBPS * 1e9) * 1e6, flops / (PEAK_FP8_TFLOPS * 1e12) * 1e6
        rec["bound_with_fp8_math"] = {"bound": "hbm" if hbm_us >= f8_us else "mfma",
                                      "bound_us": round(max(hbm_us, f8_us), 2),
                                      "frac": round(max(hbm_us, f8_us) / dec_mean, 4)}
    if not args.no_measured:
        # after the timed steps: the same fractions against what this device reaches with a plain
        # read stream and with MFMA chains alone (the headline keeps the published peaks)
        from mla_latent_space_amd import roofbench
        m = roofbench.measure(0)
        m["decode_frac_of_stream_read"] = round(achieved_gbps / m["stream_read_gbps"], 4)
        m["decode_frac_of_mfma_loop"] = round(tflops / m["mfma_bf16_tflops"]["1_wave_per_simd"], 4)
        rec["measured_denominators"] = m
    if w.kv_dtype == "bf16" and not args.no_projections:
        rec["projections"] = projections(w, args.steps, min(args.warmup, 50))
    if args.hybrid:
        rec["hybrid"] = hybrid(min(args.steps, 50), min(args.warmup, 20))
    if args.sparse:
        rec["sparse"] = sparse(min(args.steps, 100), min(args.warmup, 50))
    if not args.no_cpu:
        print("[bench] GPU legs done; timing the CPU oracle", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
