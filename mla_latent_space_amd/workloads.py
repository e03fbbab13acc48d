"""Seeded synthetic workloads for latent-space MLA decode.

This module only *makes inputs*: query rows, a paged latent KV cache, a block
table and sequence lengths, with the shapes of the DeepSeek-V3 defaults that the
"Mla Analysis" page lists in its "Tensor Shapes" table (h=128, k=512, p=64,
t=4096, b=64). It holds none of the attention arithmetic, and it is shared by the
GPU tests, the benchmark and the CPU oracle tests so that both sides read the
very same bytes.

Recipe (the same for every workload):

* A CPU ``torch.Generator`` seeded with ``seed``. Draw order: sequence lengths,
  queries, the latent pool (an fp8 pool is encoded page by page as it is drawn),
  then the physical page permutation.
* Query rows ``q[b, s, h, 576]`` and latent rows ``Z[token, 576]`` are N(0, 1)
  float32 draws rounded to bf16 (round-to-nearest-even by torch's cast).
* The pool holds ``sum(ceil(t_i / 64))`` live pages plus ``max(1, live // 16)``
  spare pages. Pages are placed at a random permutation of physical slots;
  ``block_table[i, j]`` names the slot of page ``j`` of sequence ``i`` and is -1
  past the sequence's last page.
* Poison: the unused token slots of each sequence's last page and every spare page
  hold NaN (bf16 0x7FC0, fp8 code 0x7F, scale NaN). A correct decode never lets
  them reach an output.
* fp8 cache (OCP e4m3fn): for each token and each 128-channel tile of the 512
  latent channels, ``scale = max(amax, 2**-126) / 448`` and
  ``code = e4m3fn(x / scale)`` (torch's cast, round to nearest even). The 64 rope
  channels stay bf16. A token row is 640 bytes: 512 codes then 64 bf16 values;
  scales are a separate float32 array ``[pages, 64, 4]``.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np
import torch

PAGE = 64           # tokens per page
KV_LORA = 512       # latent width k
ROPE = 64           # rope width p
DQK = KV_LORA + ROPE  # 576, width of an absorbed query / latent row
FP8_ROW_BYTES = KV_LORA + 2 * ROPE  # 640
FP8_TILE = 128      # channels per fp8 scale
BF16_NAN = 0x7FC0
FP8_NAN = 0x7F


def default_scale() -> float:
    """1/sqrt(d + p) with d=128, p=64 (the explicit form's query/key width)."""
    return 1.0 / math.sqrt(128 + ROPE)


@dataclasses.dataclass
class Workload:
    name: str
    batch: int
    s_q: int
    heads: int
    causal: bool
    kv_dtype: str                 # "bf16" or "fp8"
    seqlens: np.ndarray           # int32 [b]
    q: np.ndarray                 # uint16 bf16 bits [b, s, h, 576]
    kv: np.ndarray                # uint16 [P, 64, 576] (bf16) or uint8 [P, 64, 640] (fp8)
    kv_scales: Optional[np.ndarray]  # float32 [P, 64, 4] or None
    block_table: np.ndarray       # int32 [b, max_pages]
    scale: float
    seed: int

    @property
    def num_pages(self) -> int:
        return int(self.kv.shape[0])

    @property
    def max_pages(self) -> int:
        return int(self.block_table.shape[1])


# The five workloads, sizes as listed for this path.
CONFIGS: Dict[str, dict] = {
    "tiny": dict(batch=2, s_q=1, heads=16, lengths=("uniform", 256), kv_dtype="bf16", causal=False, seed=1000),
    "dsv3": dict(batch=64, s_q=1, heads=128, lengths=("uniform", 4096), kv_dtype="bf16", causal=False, seed=1001),
    "jagged": dict(batch=128, s_q=1, heads=128, lengths=("mix", (96, 64, 2048), (32, 32768, 131072)),
                   kv_dtype="bf16", causal=False, seed=1002),
    "spec": dict(batch=32, s_q=16, heads=128, lengths=("uniform", 4096), kv_dtype="bf16", causal=True, seed=1003),
    "fp8": dict(batch=64, s_q=1, heads=128, lengths=("uniform", 32768), kv_dtype="fp8", causal=False, seed=1004),
}


def _draw_lengths(spec, batch: int, gen: torch.Generator) -> np.ndarray:
    kind = spec[0]
    if kind == "uniform":
        return np.full(batch, int(spec[1]), dtype=np.int32)
    if kind == "list":
        out = np.asarray(spec[1], dtype=np.int32)
        assert out.shape == (batch,)
        return out
    if kind == "mix":
        groups = spec[1:]
        assert sum(g[0] for g in groups) == batch
        vals = []
        for count, lo, hi in groups:
            vals.append(torch.randint(lo, hi + 1, (count,), generator=gen, dtype=torch.int64))
        vals = torch.cat(vals)
        order = torch.randperm(batch, generator=gen)
        return vals[order].numpy().astype(np.int32)
    raise ValueError(kind)


def _randn_bf16_bits(n: int, gen: torch.Generator, chunk: int = 1 << 24) -> np.ndarray:
    out = np.empty(n, dtype=np.uint16)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        x = torch.randn(e - s, generator=gen, dtype=torch.float32)
        out[s:e] = x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return out


def _fp8_encode_pages(gen: torch.Generator, npages: int, chunk_pages: int = 512):
    """Draw N(0,1) latent rows page by page and encode them as fp8 pages."""
    kv = np.empty((npages, PAGE, FP8_ROW_BYTES), dtype=np.uint8)
    scales = np.empty((npages, PAGE, KV_LORA // FP8_TILE), dtype=np.float32)
    for p0 in range(0, npages, chunk_pages):
        p1 = min(npages, p0 + chunk_pages)
        n = (p1 - p0) * PAGE
        x = torch.randn(n, DQK, generator=gen, dtype=torch.float32)
        lat = x[:, :KV_LORA].reshape(n, KV_LORA // FP8_TILE, FP8_TILE)
        amax = lat.abs().amax(dim=2, keepdim=True)
        sc = torch.clamp(amax, min=2.0 ** -126) / 448.0
        codes = (lat / sc).to(torch.float8_e4m3fn).view(torch.uint8).reshape(n, KV_LORA)
        rope = x[:, KV_LORA:].to(torch.bfloat16).view(torch.uint8).reshape(n, 2 * ROPE)
        kv[p0:p1] = torch.cat([codes, rope], dim=1).numpy().reshape(p1 - p0, PAGE, FP8_ROW_BYTES)
        scales[p0:p1] = sc.reshape(p1 - p0, PAGE, KV_LORA // FP8_TILE).numpy()
    return kv, scales


def make_workload(name: str = "custom", *, batch: int, s_q: int, heads: int, seqlens=None,
                  lengths=None, kv_dtype: str = "bf16", causal: bool = False, seed: int = 0,
                  spare_pages: Optional[int] = None, poison: bool = True, max_pages: Optional[int] = None,
                  scale: Optional[float] = None) -> Workload:
    gen = torch.Generator().manual_seed(int(seed))
    if seqlens is not None:
        lens = np.asarray(seqlens, dtype=np.int32).reshape(batch)
    else:
        lens = _draw_lengths(lengths, batch, gen)
    q = _randn_bf16_bits(batch * s_q * heads * DQK, gen).reshape(batch, s_q, heads, DQK)
    pages_per_seq = [(int(t) + PAGE - 1) // PAGE for t in lens]
    live = int(sum(pages_per_seq))
    spare = max(1, live // 16) if spare_pages is None else int(spare_pages)
    total = live + spare
    if kv_dtype == "bf16":
        pool = _randn_bf16_bits(total * PAGE * DQK, gen).reshape(total, PAGE, DQK)
        pool_scales = None
    elif kv_dtype == "fp8":
        pool, pool_scales = _fp8_encode_pages(gen, total)
    else:
        raise ValueError(kv_dtype)
    # logical page order: sequence 0's pages, then sequence 1's, ... then spares
    perm = torch.randperm(total, generator=gen).numpy().astype(np.int64)
    kv = np.empty_like(pool)
    kv[perm] = pool
    kv_scales = None
    if pool_scales is not None:
        kv_scales = np.empty_like(pool_scales)
        kv_scales[perm] = pool_scales
    width = max(1, max(pages_per_seq) if pages_per_seq else 1)
    if max_pages is not None:
        assert max_pages >= width
        width = int(max_pages)
    bt = np.full((batch, width), -1, dtype=np.int32)
    off = 0
    for i, np_i in enumerate(pages_per_seq):
        bt[i, :np_i] = perm[off:off + np_i]
        off += np_i
    if poison:
        spare_slots = perm[live:]
        _poison_pages(kv, kv_scales, spare_slots, 0, kv_dtype)
        for i, t in enumerate(lens):
            t = int(t)
            if t % PAGE:
                last = bt[i, (t - 1) // PAGE]
                _poison_pages(kv, kv_scales, [last], t % PAGE, kv_dtype)
    return Workload(name=name, batch=batch, s_q=s_q, heads=heads, causal=bool(causal), kv_dtype=kv_dtype,
                    seqlens=lens, q=q, kv=kv, kv_scales=kv_scales, block_table=bt,
                    scale=default_scale() if scale is None else float(scale), seed=int(seed))


def _poison_pages(kv, kv_scales, slots, first_token: int, kv_dtype: str):
    for sl in slots:
        if kv_dtype == "bf16":
            kv[sl, first_token:, :] = BF16_NAN
        else:
            kv[sl, first_token:, :KV_LORA] = FP8_NAN
            kv[sl, first_token:, KV_LORA:] = np.frombuffer(np.array([BF16_NAN], dtype=np.uint16).tobytes() * ROPE,
                                                           dtype=np.uint8)
            kv_scales[sl, first_token:, :] = np.nan


def make_config(name: str, seed: Optional[int] = None) -> Workload:
    c = dict(CONFIGS[name])
    s = c.pop("seed") if seed is None else seed
    c.pop("seed", None)
    return make_workload(name, seed=s, **c)



def make_sparse_indices(seqlens, s_q: int, topk: int, seed: int, fill: float = 1.0, pad_frac: float = 0.0,
                        dup_frac: float = 0.0) -> np.ndarray:
    """Seeded top-k token lists for a token-sparse decode: int32 [b, s_q, topk]. For query token
    (i, j) the list holds round(fill * min(topk, t_i)) distinct positions of sequence i drawn
    uniformly without replacement, in random order; a fraction ``dup_frac`` of them is then
    overwritten with copies of other kept positions, and a fraction ``pad_frac`` of all entries
    with padding (-1 or a position >= t_i); the rest of the list is -1. (A CPU
    torch.Generator seeded with ``seed``; draws in (i, j) order.)"""
    gen = torch.Generator().manual_seed(seed)
    lens = np.asarray(seqlens, dtype=np.int64)
    b = lens.shape[0]
    out = np.full((b, s_q, topk), -1, dtype=np.int32)
    for i in range(b):
        t = int(lens[i])
        for j in range(s_q):
            k = int(round(fill * min(topk, t)))
            if k > 0:
                pos = torch.randperm(t, generator=gen)[:k].numpy().astype(np.int32)
                nd = int(dup_frac * k)
                if nd > 0 and k > 1:
                    src = torch.randint(0, k, (nd,), generator=gen).numpy()
                    dst = torch.randint(0, k, (nd,), generator=gen).numpy()
                    pos[dst] = pos[src]
                out[i, j, :k] = pos
            npad = int(pad_frac * topk)
            if npad > 0:
                where = torch.randperm(topk, generator=gen)[:npad].numpy()
                bad = np.where(torch.rand(npad, generator=gen).numpy() < 0.5, -1,
                               t + torch.randint(0, 1000, (npad,), generator=gen).numpy()).astype(np.int32)
                out[i, j, where] = bad
    return out
