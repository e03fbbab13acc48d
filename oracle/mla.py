"""fp64 CPU oracle for latent-space MLA decode (test infrastructure only).

Definitions followed (page "Mla Analysis", skillmd.com):

* Section "Absorption Trick (FlashMLA)": the score against a decompressed key
  K = Z W_k equals the absorbed query Qz = Q W_k^T against the latent row Z, and
  softmax(A) V with V = Z W_v equals (softmax(A) Z) W_v. The path therefore works
  on latent rows only and returns O_latent = softmax(scale * Qz Z^T) Z[:, :k]; the
  decompression by W_v is a separate step.
* Section "Tensor Shapes": k = 512 latent channels, p = 64 rope channels, d = 128,
  Z is [B, T, K] and the shared rope key KPE is [B, T, P]; a cached row here is the
  576-wide concatenation [Z | KPE] and an absorbed query is [q_nope W_k^T | q_rope].
* Section "Cost Models": FLOP and byte models of FlashAttention, FlashMLA and
  MLAvar6+.
* Section "MLAvar6+ Design": o old tokens as latent rows, n new tokens decompressed,
  t = o + n; the attention over their union is exact.

Library card page "FlashMLA: Efficient Multi-head Latent Attention Kernels", its
description and use cases: token-level sparse attention for decoding, with an FP8 cache
(decode_sparse).

FlashMLA-2 newsletter page, section "Architectural Analysis": the latent cache may be
stored in FP8 and is scaled from FP8 to BF16 in registers before the matrix products; OCP
e4m3fn is the format read here, one float32 scale per token per 128-channel tile, and the
value the products read is that BF16 number (fp8_dequant).

Readings where the pages are silent (each listed in the design notes):
* the log-sum-exp is the natural log of the sum of exp(scaled logits);
* ``out`` is normalised (softmax(A) Z);
* with s > 1 query tokens and ``causal``, query j of a sequence with t cached
  tokens (which include the s new ones) sees keys 0 .. t - s + j;
* an empty visible set gives out = 0 and lse = -inf;
* the value is Z[:, :512] (rope excluded);
* the FP8-to-BF16 scaling forms code * scale in float32 (the scale's precision) and rounds
  that product to the nearest BF16, ties to even.

Everything is float64; no blocking, fusion or reordering beyond the definition.
"""
from __future__ import annotations

import math
from typing import Iterable, Optional, Sequence, Tuple

import numpy as np

PAGE = 64
K_LAT = 512
P_ROPE = 64
D_QK = K_LAT + P_ROPE
FP8_TILE = 128


# ----------------------------------------------------------------------------- number formats

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly (bf16 is the top half of a float32)."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u32.view(np.float32).astype(np.float64)


def e4m3fn_to_f64(codes: np.ndarray) -> np.ndarray:
    """OCP e4m3fn code (uint8) -> float64, from the bit layout.

    1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 is
    subnormal (m/8 * 2^-6); S.1111.111 is NaN; there is no infinity; the largest
    finite magnitude is 1.75 * 2^8 = 448.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    subnormal = (m / 8.0) * 2.0 ** -6
    v = sign * np.where(e == 0, subnormal, normal)
    v = np.where((c & 0x7F) == 0x7F, np.nan, v)
    return v


# The decoder above applied once to each of the 256 codes: a code's value is a pure function of
# its 8 bits, so gathering from this table is the same definition, evaluated once per code.
_E4M3FN_VALUES = e4m3fn_to_f64(np.arange(256, dtype=np.uint8))


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> the nearest bf16 (ties to even), returned as float64. bf16 keeps the top 16
    bits of a float32, so rounding adds half of the dropped range (0x7FFF, plus one when the
    kept part is odd) to the bit pattern and truncates; the carry runs into the exponent, which
    is the correct rounding at a binade edge. (Finite inputs; NaN is kept as NaN.)"""
    x = np.asarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    out = r.astype(np.uint32).view(np.float32).astype(np.float64)
    return np.where(np.isnan(x), np.nan, out)


def fp8_dequant(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """The FP8-to-BF16 scaling of the FlashMLA-2 page ("Architectural Analysis"): each e4m3fn
    code's value times its float32 scale, the product formed in float32 and rounded to bf16.
    codes uint8 [..., n], scales float32 broadcastable to it; returns float64."""
    v = _E4M3FN_VALUES[np.asarray(codes, dtype=np.uint8)].astype(np.float32)   # exact in float32
    prod = v * np.asarray(scales, dtype=np.float32)                            # one float32 rounding
    return f32_to_bf16(prod)


# ----------------------------------------------------------------------------- cache gather

def latent_rows(kv: np.ndarray, kv_scales: Optional[np.ndarray], kv_dtype: str,
                block_table_row: np.ndarray, t: int) -> np.ndarray:
    """The first ``t`` cached rows of one sequence, gathered through its block table, as
    float64 [t, 576]. fp8: row[c] = bf16(e4m3fn(code[c]) * scale[token, c // 128]) for
    c < 512 (fp8_dequant), rope channels are bf16."""
    if t == 0:
        return np.zeros((0, D_QK))
    npages = (t + PAGE - 1) // PAGE
    ids = np.asarray(block_table_row[:npages], dtype=np.int64)
    if kv_dtype == "bf16":
        rows = kv[ids].reshape(npages * PAGE, D_QK)[:t]
        return bf16_bits_to_f64(rows)
    if kv_dtype == "fp8":
        raw = kv[ids].reshape(npages * PAGE, -1)[:t]
        sc = kv_scales[ids].reshape(npages * PAGE, K_LAT // FP8_TILE)[:t]
        # channel c of a token times its tile's scale, tile = c // 128
        lat = fp8_dequant(raw[:, :K_LAT].reshape(t, K_LAT // FP8_TILE, FP8_TILE),
                          sc[:, :, None]).reshape(t, K_LAT)
        rope = bf16_bits_to_f64(np.ascontiguousarray(raw[:, K_LAT:]).view(np.uint16))
        return np.concatenate([lat, rope], axis=1)
    raise ValueError(kv_dtype)


def visible_keys(t: int, s_q: int, j: int, causal: bool) -> int:
    """Number of keys query token j sees: all t, or 0 .. t - s_q + j under the causal reading."""
    if not causal:
        return int(t)
    return int(min(max(t - s_q + 1 + j, 0), t))


# ----------------------------------------------------------------------------- attention

def softmax_attention(qrows: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float):
    """out = softmax(scale * qrows keys^T) values and lse = log sum exp(scale * qrows keys^T),
    one row per query. Empty key set -> out 0, lse -inf."""
    nq = qrows.shape[0]
    if keys.shape[0] == 0:
        return np.zeros((nq, values.shape[1])), np.full(nq, -np.inf)
    a = scale * (qrows @ keys.T)
    m = a.max(axis=1, keepdims=True)
    e = np.exp(a - m)
    ell = e.sum(axis=1, keepdims=True)
    p = e / ell
    return p @ values, (m + np.log(ell))[:, 0]


def decode_latent(q_bits: np.ndarray, kv: np.ndarray, kv_scales: Optional[np.ndarray], kv_dtype: str,
                  block_table: np.ndarray, seqlens: np.ndarray, scale: float, causal: bool,
                  seqs: Optional[Iterable[int]] = None):
    """Latent-space MLA decode (absorbed form), per sequence.

    q_bits [b, s, h, 576] bf16 bits; returns out [b, s, h, 512] and lse [b, s, h] in float64
    (rows of sequences not in ``seqs`` are left NaN)."""
    b, s_q, h, _ = q_bits.shape
    out = np.full((b, s_q, h, K_LAT), np.nan)
    lse = np.full((b, s_q, h), np.nan)
    for i in (range(b) if seqs is None else seqs):
        t = int(seqlens[i])
        z = latent_rows(kv, kv_scales, kv_dtype, block_table[i], t)
        for j in range(s_q):
            vis = visible_keys(t, s_q, j, causal)
            qz = bf16_bits_to_f64(q_bits[i, j])
            o, l = softmax_attention(qz, z[:vis], z[:vis, :K_LAT], scale)
            out[i, j] = o
            lse[i, j] = l
    return out, lse


def sparse_keys(indices_row: np.ndarray, t: int) -> np.ndarray:
    """Library card page "FlashMLA: Efficient Multi-head Latent Attention Kernels" (token-level
    sparse attention in decoding): a query token attends to its own list of selected tokens
    instead of the whole cache. Reading: the list holds logical positions of the query's sequence; an entry outside
    [0, t) is padding and dropped; the others are keys in list order (a repeated position is a
    repeated key). Returns the kept positions."""
    idx = np.asarray(indices_row, dtype=np.int64)
    return idx[(idx >= 0) & (idx < t)]


def decode_sparse(q_bits: np.ndarray, kv: np.ndarray, kv_scales: Optional[np.ndarray], kv_dtype: str,
                  block_table: np.ndarray, seqlens: np.ndarray, indices: np.ndarray, scale: float,
                  seqs: Optional[Iterable[int]] = None):
    """Token-level sparse latent decode: query (i, j) attends over the latent rows at
    sparse_keys(indices[i, j], t_i), with the same scores, softmax and value as the dense decode.
    q_bits [b, s, h, 576] bf16 bits, indices int [b, s, topk]; returns out [b, s, h, 512] and
    lse [b, s, h] (rows of sequences not in ``seqs`` are left NaN)."""
    b, s_q, h, _ = q_bits.shape
    out = np.full((b, s_q, h, K_LAT), np.nan)
    lse = np.full((b, s_q, h), np.nan)
    for i in (range(b) if seqs is None else seqs):
        t = int(seqlens[i])
        z = latent_rows(kv, kv_scales, kv_dtype, block_table[i], t)
        for j in range(s_q):
            keys = z[sparse_keys(indices[i, j], t)]
            qz = bf16_bits_to_f64(q_bits[i, j])
            out[i, j], lse[i, j] = softmax_attention(qz, keys, keys[:, :K_LAT], scale)
    return out, lse


# ----------------------------------------------------------------------------- explicit form

def absorbed_query(q_nope: np.ndarray, q_rope: np.ndarray, w_k: np.ndarray) -> np.ndarray:
    """Qz = [q_nope W_k^T | q_rope] per head: q_nope [h, d], q_rope [h, p], W_k [h, k, d]
    (K = Z W_k maps a latent row to a key) -> [h, k + p]."""
    qz_nope = np.einsum("hkd,hd->hk", w_k, q_nope)
    return np.concatenate([qz_nope, q_rope], axis=1)


def decode_explicit(q_nope: np.ndarray, q_rope: np.ndarray, w_k: np.ndarray, w_v: np.ndarray,
                    z: np.ndarray, scale: float):
    """Decompressed (FlashAttention-form) attention for one query token of one sequence:
    K_h = [Z[:, :k] W_k,h | Z[:, k:]], V_h = Z[:, :k] W_v,h, Q_h = [q_nope,h | q_rope,h];
    returns O [h, d] and lse [h]."""
    h = q_nope.shape[0]
    d = w_v.shape[2]
    out = np.empty((h, d))
    lse = np.empty(h)
    for eta in range(h):
        k_eta = np.concatenate([z[:, :K_LAT] @ w_k[eta], z[:, K_LAT:]], axis=1)
        v_eta = z[:, :K_LAT] @ w_v[eta]
        q_eta = np.concatenate([q_nope[eta], q_rope[eta]])[None, :]
        o, l = softmax_attention(q_eta, k_eta, v_eta, scale)
        out[eta] = o[0]
        lse[eta] = l[0]
    return out, lse


def hybrid_visible_new(n: int, s_q: int, j: int, causal: bool) -> int:
    """Split latent + decompressed variant (section "MLAvar6+ Design"): the n newest of a
    sequence's t tokens are the decompressed ones. Under the causal reading query j sees keys
    0 .. t - s + j, i.e. every old token and the first n - s + 1 + j new ones (n >= s)."""
    if not causal:
        return int(n)
    if n < s_q:
        raise ValueError("the causal split needs n >= s_q (the old tokens must all be visible)")
    return int(n - s_q + 1 + j)


def decode_hybrid(q_nope: np.ndarray, q_rope: np.ndarray, w_k: np.ndarray, w_v: np.ndarray,
                  z_old: np.ndarray, k_new: np.ndarray, kr_new: np.ndarray, v_new: np.ndarray,
                  scale: float, vis_new: int):
    """Page "Mla Analysis", section "MLAvar6+ Design": the cache of one sequence is split into
    o old tokens kept as latent rows Z [o, k + p] and n new tokens kept decompressed (K [n, h, d]
    and V [n, h, d], with the shared rope key KPE [n, p]). The attention is the same softmax over
    all of them: for head h the keys are [Z[:, :k] W_k,h | Z[:, k:]] (old) and [K_h | KPE] (new),
    the values Z[:, :k] W_v,h (old) and V_h (new). One query token; the new tokens visible are
    the first ``vis_new``. Returns O [h, d] and lse [h]."""
    h = q_nope.shape[0]
    d = w_v.shape[2]
    out = np.empty((h, d))
    lse = np.empty(h)
    for eta in range(h):
        k_old = np.concatenate([z_old[:, :K_LAT] @ w_k[eta], z_old[:, K_LAT:]], axis=1)
        v_old = z_old[:, :K_LAT] @ w_v[eta]
        k_n = np.concatenate([k_new[:vis_new, eta], kr_new[:vis_new]], axis=1)
        v_n = v_new[:vis_new, eta]
        q_eta = np.concatenate([q_nope[eta], q_rope[eta]])[None, :]
        o, l = softmax_attention(q_eta, np.concatenate([k_old, k_n], axis=0),
                                 np.concatenate([v_old, v_n], axis=0), scale)
        out[eta] = o[0]
        lse[eta] = l[0]
    return out, lse


def decompress_output(out_latent: np.ndarray, w_v: np.ndarray) -> np.ndarray:
    """O = O_latent W_v per head: [h, k] x [h, k, d] -> [h, d]."""
    return np.einsum("hk,hkd->hd", out_latent, w_v)


# ----------------------------------------------------------------------------- split combine

def combine(parts: Sequence[Tuple[np.ndarray, np.ndarray]]):
    """Merge partial results over disjoint key sets by their log-sum-exps:
    lse = log sum_k exp(lse_k); out = sum_k exp(lse_k - lse) out_k. Parts with lse = -inf
    carry no weight; if every part is empty the result is out 0, lse -inf."""
    lses = np.stack([p[1] for p in parts], axis=0)
    outs = np.stack([p[0] for p in parts], axis=0)
    m = lses.max(axis=0)
    safe_m = np.where(np.isfinite(m), m, 0.0)
    w = np.where(np.isfinite(lses), np.exp(lses - safe_m), 0.0)
    tot = w.sum(axis=0)
    lse = np.where(tot > 0, safe_m + np.log(np.where(tot > 0, tot, 1.0)), -np.inf)
    norm = np.where(tot > 0, tot, 1.0)
    out = np.einsum("k...,k...c->...c", w / norm, np.where(np.isfinite(lses)[..., None], outs, 0.0))
    return out, lse


# ----------------------------------------------------------------------------- cost models

def flashattention_cost(b, h, s, t, d=128, p=64, w=2):
    """(FLOPs, bytes) of decompressed attention: 2bhst(2d+p) and w*bh(s+t)(2d+p)."""
    return 2.0 * b * h * s * t * (2 * d + p), float(w) * b * h * (s + t) * (2 * d + p)


def flashmla_cost(b, h, s, t, k=512, p=64, w=2):
    """(FLOPs, bytes) of latent-space attention: 2bhst(2k+p) and w*(bhs(2k+p) + bt(k+p))."""
    return 2.0 * b * h * s * t * (2 * k + p), float(w) * (b * h * s * (2 * k + p) + b * t * (k + p))


def mlavar6_cost(b, h, s, o, n, d=128, p=64, k=512, w=2):
    """(FLOPs, bytes) of the split latent + decompressed variant with o old latent tokens and
    n new decompressed tokens (t = o + n): 2bhstp + 4bhsnd + 4bhsok and
    w(bhsp + bhsd + bhsk + bok + btp + bhnd + bhnd + bhsd + bhsk)."""
    t = o + n
    flops = 2.0 * b * h * s * t * p + 4.0 * b * h * s * n * d + 4.0 * b * h * s * o * k
    byts = float(w) * (b * h * s * p + b * h * s * d + b * h * s * k + b * o * k + b * t * p
                       + b * h * n * d + b * h * n * d + b * h * s * d + b * h * s * k)
    return flops, byts
