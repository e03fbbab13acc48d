"""Pins for the fp64 oracle (CPU only).

Each test checks the oracle against something other than itself: a library routine
computing the same definition, a closed form, brute force on tiny inputs, an identity
the pages state, or a value the pages print. The last group plants mistakes in a copy
of the oracle and checks that the pins catch them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import mla as om
from mla_latent_space_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _sdpa_reference(qz, z, scale, s_q=1, causal=False, t=None):
    """torch's float64 scaled_dot_product_attention with K = Z, V = Z[:, :512] and a
    bottom-right causal mask; lse from torch.logsumexp of the scaled logits."""
    q = torch.from_numpy(qz)            # [s, h, 576]
    k = torch.from_numpy(z)             # [t, 576]
    s, h, _ = q.shape
    tt = k.shape[0]
    mask = None
    if causal:
        jj = torch.arange(s)[:, None]
        uu = torch.arange(tt)[None, :]
        mask = uu <= (tt - s + jj)                      # [s, t]
        mask = mask[:, None, :].expand(s, h, tt).reshape(1, s * h, tt)
    qq = q.reshape(1, s * h, -1)
    out = torch.nn.functional.scaled_dot_product_attention(qq, k[None], k[None, :, :512],
                                                           attn_mask=mask, scale=scale)
    logits = scale * (qq @ k[None].transpose(1, 2))
    if mask is not None:
        logits = logits.masked_fill(~mask, float("-inf"))
    lse = torch.logsumexp(logits, dim=-1)
    return out.reshape(s, h, 512).numpy(), lse.reshape(s, h).numpy()


def _small(seed=0, b=3, s_q=1, h=8, lens=(64, 130, 7), kv="bf16", causal=False):
    return wl.make_workload(batch=b, s_q=s_q, heads=h, seqlens=list(lens), kv_dtype=kv, causal=causal, seed=seed)


def _run(w, seqs=None):
    return om.decode_latent(w.q, w.kv, w.kv_scales, w.kv_dtype, w.block_table, w.seqlens, w.scale, w.causal, seqs)


# ----------------------------------------------------------------------------- number formats

def test_e4m3_all_codes_match_torch_cast():
    codes = np.arange(256, dtype=np.uint8)
    mine = om.e4m3fn_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    both_nan = np.isnan(mine) & np.isnan(ref)
    assert np.all(both_nan | (mine == ref))
    assert np.isnan(mine).sum() == 2  # 0x7F and 0xFF


def test_e4m3_textbook_values():
    # OCP 8-bit float spec: max normal 448, min normal 2^-6, min subnormal 2^-9, 1.0 = 0x38
    v = om.e4m3fn_to_f64(np.array([0x7E, 0x08, 0x01, 0x38, 0xB8, 0x00, 0x80], dtype=np.uint8))
    assert v[0] == 448.0 and v[1] == 2.0 ** -6 and v[2] == 2.0 ** -9
    assert v[3] == 1.0 and v[4] == -1.0 and v[5] == 0.0 and v[6] == 0.0


def _torch_bf16(x_f32):
    return torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def test_f32_to_bf16_matches_torch_rounding():
    """Round to nearest, ties to even, against torch's float32 -> bfloat16 cast: random bit
    patterns of every magnitude, exact ties with an even and an odd kept part, values that
    round up across a binade edge or overflow to infinity, subnormals and zeros."""
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 0x7F800000, 200000, dtype=np.int64).astype(np.uint32)
    bits[::2] |= np.uint32(0x80000000)
    ties = (rng.integers(0, 0x7F80, 2000, dtype=np.int64).astype(np.uint32) << 16) | np.uint32(0x8000)
    edges = np.array([0x3F7FFFFF, 0x3F7F8000, 0x3F7F7FFF, 0x7F7FFFFF, 0x7F7F8000, 0x7F7F7FFF, 0x00000001,
                      0x00008000, 0x00018000, 0x007FFFFF, 0x00000000, 0x80000000, 0xBF808000, 0xBF818000],
                     dtype=np.uint32)
    x = np.concatenate([bits, ties, edges]).view(np.float32)
    mine, ref = om.f32_to_bf16(x), _torch_bf16(x)
    assert np.array_equal(mine, ref)
    assert om.f32_to_bf16(np.array([0x3F808000], dtype=np.uint32).view(np.float32))[0] == 1.0   # tie, even kept part
    assert om.f32_to_bf16(np.array([0x3F818000], dtype=np.uint32).view(np.float32))[0] == 1.0 + 2 ** -6   # tie, odd
    assert om.f32_to_bf16(np.array([0x7F7FFFFF], dtype=np.uint32).view(np.float32))[0] == np.inf


def test_fp8_dequant_definition():
    """bf16(fl32(e4m3fn(code) * scale)): equal to torch's float32 product cast to bf16 for all
    256 codes at many scales; exact when the scale is a power of two; within one bf16 rounding
    (2^-8 relative) of the exact product otherwise."""
    rng = np.random.default_rng(8)
    codes = np.arange(256, dtype=np.uint8)
    codes = codes[(codes & 0x7F) != 0x7F]
    scales = np.concatenate([rng.uniform(1e-4, 1.0, 200), rng.uniform(1.0, 50.0, 56)]).astype(np.float32)
    got = om.fp8_dequant(codes[None, :], scales[:, None])
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32)
    ref = (vals[None, :] * torch.from_numpy(scales)[:, None]).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(got, ref)
    exact = om.e4m3fn_to_f64(codes)[None, :] * scales.astype(np.float64)[:, None]
    assert np.all(np.abs(got - exact) <= 2.0 ** -8 * np.abs(exact) * (1 + 2.0 ** -20))
    assert (got != exact).mean() > 0.5          # the rounding is real at these scales
    p2 = np.array([2.0 ** -9, 2.0 ** -3, 1.0, 8.0], dtype=np.float32)
    assert np.array_equal(om.fp8_dequant(codes[None, :], p2[:, None]),
                          om.e4m3fn_to_f64(codes)[None, :] * p2.astype(np.float64)[:, None])


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 0x7F80, 10000).astype(np.uint16)
    bits[::2] |= 0x8000
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(om.bf16_bits_to_f64(bits), ref)


# ----------------------------------------------------------------------------- attention vs library

@pytest.mark.parametrize("lens", [(64, 130, 7), (1, 64, 65)])
def test_latent_decode_matches_torch_sdpa(lens):
    w = _small(lens=lens, seed=3)
    out, lse = _run(w)
    for i, t in enumerate(w.seqlens):
        z = om.latent_rows(w.kv, None, "bf16", w.block_table[i], int(t))
        ro, rl = _sdpa_reference(om.bf16_bits_to_f64(w.q[i]), z, w.scale)
        np.testing.assert_allclose(out[i], ro, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse[i], rl, rtol=1e-13, atol=1e-13)


def test_causal_decode_matches_torch_sdpa_bottom_right():
    w = _small(s_q=5, h=4, lens=(70, 5, 9), causal=True, seed=4)
    out, lse = _run(w)
    for i, t in enumerate(w.seqlens):
        z = om.latent_rows(w.kv, None, "bf16", w.block_table[i], int(t))
        ro, rl = _sdpa_reference(om.bf16_bits_to_f64(w.q[i]), z, w.scale, s_q=5, causal=True)
        np.testing.assert_allclose(out[i], ro, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse[i], rl, rtol=1e-13, atol=1e-13)


def test_softmax_rows_sum_to_one_and_lse_consistent():
    w = _small(seed=5)
    i, t = 1, int(w.seqlens[1])
    z = om.latent_rows(w.kv, None, "bf16", w.block_table[i], t)
    qz = om.bf16_bits_to_f64(w.q[i, 0])
    _, lse = om.softmax_attention(qz, z, z[:, :512], w.scale)
    a = w.scale * qz @ z.T
    np.testing.assert_allclose(np.exp(a - lse[:, None]).sum(axis=1), 1.0, rtol=0, atol=1e-13)


# ----------------------------------------------------------------------------- closed forms

def test_zero_query_gives_mean_and_log_t():
    z = np.random.default_rng(2).standard_normal((37, 576))
    out, lse = om.softmax_attention(np.zeros((3, 576)), z, z[:, :512], 0.07)
    np.testing.assert_allclose(out, np.broadcast_to(z[:, :512].mean(axis=0), (3, 512)), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, math.log(37), rtol=1e-15)


def test_single_key_and_two_keys_closed_form():
    rng = np.random.default_rng(3)
    z = rng.standard_normal((2, 576))
    q = rng.standard_normal((1, 576))
    out1, lse1 = om.softmax_attention(q, z[:1], z[:1, :512], 0.1)
    np.testing.assert_array_equal(out1[0], z[0, :512])
    assert lse1[0] == pytest.approx(0.1 * float(q[0] @ z[0]), rel=1e-15)
    out2, lse2 = om.softmax_attention(q, z, z[:, :512], 0.1)
    a0, a1 = 0.1 * float(q[0] @ z[0]), 0.1 * float(q[0] @ z[1])
    sig = lambda x: 1.0 / (1.0 + math.exp(-x))
    np.testing.assert_allclose(out2[0], sig(a1 - a0) * z[1, :512] + sig(a0 - a1) * z[0, :512], rtol=1e-13, atol=1e-14)
    assert lse2[0] == pytest.approx(math.log(math.exp(a0) + math.exp(a1)), rel=1e-14)


def test_identical_rows_return_that_row():
    row = np.random.default_rng(4).standard_normal(576)
    z = np.tile(row, (9, 1))
    q = np.random.default_rng(5).standard_normal((4, 576))
    out, _ = om.softmax_attention(q, z, z[:, :512], 0.2)
    np.testing.assert_allclose(out, np.broadcast_to(row[:512], (4, 512)), rtol=1e-14, atol=1e-14)


def test_empty_visible_set():
    out, lse = om.softmax_attention(np.ones((2, 576)), np.zeros((0, 576)), np.zeros((0, 512)), 0.1)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


# ----------------------------------------------------------------------------- absorption identity

def test_absorption_identity_latent_equals_explicit():
    """'Absorption Trick': Q (Z W_k)^T = (Q W_k^T) Z^T and softmax(A)(Z W_v) = (softmax(A) Z) W_v."""
    rng = np.random.default_rng(6)
    h, d, t = 4, 128, 50
    z = rng.standard_normal((t, 576))
    w_k = rng.standard_normal((h, 512, d)) / math.sqrt(512)
    w_v = rng.standard_normal((h, 512, d)) / math.sqrt(512)
    q_nope = rng.standard_normal((h, d))
    q_rope = rng.standard_normal((h, 64))
    scale = 1.0 / math.sqrt(d + 64)
    o_exp, l_exp = om.decode_explicit(q_nope, q_rope, w_k, w_v, z, scale)
    qz = om.absorbed_query(q_nope, q_rope, w_k)
    o_lat, l_lat = om.softmax_attention(qz, z, z[:, :512], scale)
    np.testing.assert_allclose(om.decompress_output(o_lat, w_v), o_exp, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(l_lat, l_exp, rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------- paging, poison

def test_paging_permutation_is_bitwise_invariant():
    w = _small(seed=7, lens=(200, 64, 3))
    out, lse = _run(w)
    rng = np.random.default_rng(8)
    perm = rng.permutation(w.num_pages)
    kv2 = np.empty_like(w.kv)
    kv2[perm] = w.kv
    bt2 = np.where(w.block_table >= 0, perm[np.maximum(w.block_table, 0)], -1).astype(np.int32)
    out2, lse2 = om.decode_latent(w.q, kv2, None, "bf16", bt2, w.seqlens, w.scale, False)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_poison_never_reaches_outputs():
    w = wl.make_workload(batch=2, s_q=1, heads=4, seqlens=[70, 3], seed=9, poison=True)
    clean = wl.make_workload(batch=2, s_q=1, heads=4, seqlens=[70, 3], seed=9, poison=False)
    assert np.isnan(om.bf16_bits_to_f64(w.kv)).any()
    out, lse = _run(w)
    out_c, lse_c = _run(clean)
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    assert np.array_equal(out, out_c) and np.array_equal(lse, lse_c)


# ----------------------------------------------------------------------------- split / combine

def test_combine_of_any_partition_equals_unsplit():
    rng = np.random.default_rng(10)
    z = rng.standard_normal((300, 576))
    q = rng.standard_normal((6, 576))
    full_o, full_l = om.softmax_attention(q, z, z[:, :512], 0.08)
    for trial in range(5):
        cuts = np.sort(rng.choice(np.arange(1, 300), size=trial + 1, replace=False))
        bounds = [0, *cuts.tolist(), 300]
        parts = [om.softmax_attention(q, z[a:b], z[a:b, :512], 0.08) for a, b in zip(bounds[:-1], bounds[1:])]
        parts.append(om.softmax_attention(q, z[:0], z[:0, :512], 0.08))   # an empty part
        o, l = om.combine(parts)
        np.testing.assert_allclose(o, full_o, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(l, full_l, rtol=1e-13, atol=1e-13)


def test_causal_equals_independent_single_token_calls():
    w = _small(s_q=16, h=2, lens=(100, 40, 16), causal=True, seed=11)
    out, lse = _run(w)
    for i, t in enumerate(w.seqlens):
        z = om.latent_rows(w.kv, None, "bf16", w.block_table[i], int(t))
        for j in range(16):
            tj = int(t) - 16 + 1 + j
            o, l = om.softmax_attention(om.bf16_bits_to_f64(w.q[i, j]), z[:tj], z[:tj, :512], w.scale)
            np.testing.assert_array_equal(out[i, j], o)
            np.testing.assert_array_equal(lse[i, j], l)


# ----------------------------------------------------------------------------- fp8 cache

def test_fp8_rows_match_torch_dequant():
    w = _small(kv="fp8", seed=12, lens=(64, 130, 7))
    for i, t in enumerate(w.seqlens):
        t = int(t)
        z = om.latent_rows(w.kv, w.kv_scales, "fp8", w.block_table[i], t)
        ids = w.block_table[i, :(t + 63) // 64]
        raw = torch.from_numpy(w.kv[ids].reshape(-1, 640)[:t].copy())
        # the FP8-to-BF16 scaling: float32 product, rounded to bf16
        lat = raw[:, :512].contiguous().view(torch.float8_e4m3fn).to(torch.float32)
        sc = torch.from_numpy(w.kv_scales[ids].reshape(-1, 4)[:t].copy())
        lat = (lat.reshape(t, 4, 128) * sc[:, :, None]).reshape(t, 512).to(torch.bfloat16).to(torch.float64)
        rope = raw[:, 512:].contiguous().view(torch.bfloat16).to(torch.float64)
        ref = torch.cat([lat, rope], dim=1).numpy()
        assert np.array_equal(z, ref)


def test_fp8_encoding_error_bound():
    """The generator's e4m3 encoding has relative step 2^-3 at most (3 mantissa bits), so each
    decoded value is within half an ulp: |x - x_hat| <= 2^-4 |x| for normals; the bf16 rounding
    of the scaled value adds at most 2^-8 of its magnitude."""
    w = _small(kv="fp8", seed=13, lens=(64,), b=1)
    z = om.latent_rows(w.kv, w.kv_scales, "fp8", w.block_table[0], 64)
    # regenerate the fp32 draws of the pool in the same order to compare
    gen = torch.Generator().manual_seed(13)
    _ = torch.randn(1 * 1 * 8 * 576, generator=gen)           # q
    x = torch.randn(2 * 64, 576, generator=gen).numpy().astype(np.float64)   # live + 1 spare page
    page0 = x[:64, :512]
    sc = w.kv_scales[w.block_table[0, 0]].astype(np.float64)
    tol = np.maximum(np.abs(page0) * 2.0 ** -4, np.repeat(sc, 128, axis=1) * 2.0 ** -10)
    tol = tol + 2.0 ** -8 * (np.abs(page0) + tol)
    assert np.all(np.abs(z[:, :512] - page0) <= tol)


# ----------------------------------------------------------------------------- cost model (printed values)

def test_cost_models_reproduce_printed_intensities():
    g = json.load(open(os.path.join(GOLDEN, "cost_model.json")))
    b, h, t = 64, 128, 4096
    for case in g["cases"]:
        fn = om.flashattention_cost if case["model"] == "flashattention" else om.flashmla_cost
        f, by = fn(b, h, case["s"], t)
        assert abs(f / by - case["printed_ai"]) <= case["tolerance"], case
    fr = g["flop_ratio"]
    ratio = om.flashmla_cost(1, 1, 1, 1)[0] / om.flashattention_cost(1, 1, 1, 1)[0]
    assert abs(ratio - fr["printed"]) <= fr["tolerance"]


def test_mlavar6_interpolates_between_endpoints():
    """'MLAvar6+ Design': n=0 is FlashMLA-like, o=0 is FlashAttention-like."""
    b, h, s, t = 2, 8, 4, 96
    f_lat, _ = om.flashmla_cost(b, h, s, t)
    f_fa, _ = om.flashattention_cost(b, h, s, t)
    f0, _ = om.mlavar6_cost(b, h, s, o=t, n=0)
    f1, _ = om.mlavar6_cost(b, h, s, o=0, n=t)
    assert f0 == pytest.approx(f_lat) and f1 == pytest.approx(f_fa)


def _inventory_bytes(tensors, w=2):
    """Bytes of a list of tensor shapes at w bytes per element, counted by allocating them."""
    dt = {1: np.uint8, 2: np.float16, 4: np.float32}[w]
    return float(sum(np.empty(shape, dtype=dt).nbytes for shape in tensors))


# Tiny shapes with distinct primes, so that a swapped, dropped or repeated factor in a byte
# term changes the total.
_B, _H, _S, _O, _N, _D, _P, _K = 2, 3, 5, 7, 11, 13, 17, 19


def _mlavar6_inventory(b, h, s, o, n, d, p, k):
    """The tensors one MLAvar6+ call moves, from page "Mla Analysis": section "MLAvar6+ Design"
    (o old tokens as latent Z, n new tokens decompressed as K, V; t = o + n) and the layouts of
    section "Tensor Shapes": the query parts Q [B,H,S,D], its absorbed form Qc [B,H,S,K] and its
    rope part QPE [B,H,S,P]; the old latent rows Z [B,o,K]; the rope keys KPE [B,T,P] of all t
    tokens; the new K and V [B,n,H,D]; the decompressed output [B,H,S,D] and the latent output
    [B,H,S,K] that the old part produces before its decompression."""
    t = o + n
    return [(b, h, s, d), (b, h, s, k), (b, h, s, p),     # Q, Qc, QPE
            (b, o, k), (b, t, p),                        # Z (old), KPE (all)
            (b, n, h, d), (b, n, h, d),                  # K, V (new)
            (b, h, s, d), (b, h, s, k)]                  # output, latent output


def test_mlavar6_bytes_match_tensor_inventory():
    """Section "Cost Models", MLAvar6+: the byte model equals the bytes of the tensors the split
    variant reads and writes, counted from arrays of those shapes."""
    for (o, n) in [(_O, _N), (0, _N), (_O, 0), (1, 1)]:
        _, byts = om.mlavar6_cost(_B, _H, _S, o, n, d=_D, p=_P, k=_K)
        assert byts == _inventory_bytes(_mlavar6_inventory(_B, _H, _S, o, n, _D, _P, _K)), (o, n)
    # w scales every term
    _, b4 = om.mlavar6_cost(_B, _H, _S, _O, _N, d=_D, p=_P, k=_K, w=4)
    assert b4 == _inventory_bytes(_mlavar6_inventory(_B, _H, _S, _O, _N, _D, _P, _K), w=4)


def test_flashmla_and_flashattention_bytes_match_tensor_inventory():
    """Section "Cost Models": FlashMLA moves Qc with its rope part and the latent output
    ([B,H,S,K+P] in, [B,H,S,K] out) and the latent cache Z, KPE ([B,T,K+P]); FlashAttention
    moves Q, K, V and O with rope parts, [B,H,S+T,2D+P] in total."""
    t = _O + _N
    mla_inv = [(_B, _H, _S, _K + _P), (_B, _H, _S, _K), (_B, t, _K + _P)]
    assert om.flashmla_cost(_B, _H, _S, t, k=_K, p=_P)[1] == _inventory_bytes(mla_inv)
    fa_inv = [(_B, _H, _S + t, 2 * _D + _P)]
    assert om.flashattention_cost(_B, _H, _S, t, d=_D, p=_P)[1] == _inventory_bytes(fa_inv)


def test_inventory_pin_catches_a_dropped_byte_term(monkeypatch):
    """A planted mistake in the MLAvar6+ byte model (the second new-token term dropped) fails
    the inventory pin."""
    real = om.mlavar6_cost

    def dropped(b, h, s, o, n, d=128, p=64, k=512, w=2):
        f, by = real(b, h, s, o, n, d=d, p=p, k=k, w=w)
        return f, by - w * b * h * n * d

    _mutant(monkeypatch, "mlavar6_cost", dropped)
    with pytest.raises(AssertionError):
        test_mlavar6_bytes_match_tensor_inventory()


def test_inventory_pin_catches_a_transposed_byte_term(monkeypatch):
    """bok written as bhk (the latent rows counted per head) fails the inventory pin."""
    real = om.mlavar6_cost

    def transposed(b, h, s, o, n, d=128, p=64, k=512, w=2):
        f, by = real(b, h, s, o, n, d=d, p=p, k=k, w=w)
        return f, by - w * b * o * k + w * b * h * k

    _mutant(monkeypatch, "mlavar6_cost", transposed)
    with pytest.raises(AssertionError):
        test_mlavar6_bytes_match_tensor_inventory()


# ----------------------------------------------------------------------------- planted mistakes

def _mutant(monkeypatch, name, fn):
    monkeypatch.setattr(om, name, fn)


def _sdpa_pin_fails(w):
    out, lse = _run(w)
    try:
        for i, t in enumerate(w.seqlens):
            z = om.latent_rows(w.kv, None, "bf16", w.block_table[i], int(t))
            ro, rl = _sdpa_reference(om.bf16_bits_to_f64(w.q[i]), z, w.scale, s_q=w.s_q, causal=w.causal)
            np.testing.assert_allclose(out[i], ro, rtol=1e-9, atol=1e-10)
            np.testing.assert_allclose(lse[i], rl, rtol=1e-9, atol=1e-10)
    except AssertionError:
        return True
    return False


def test_pins_catch_truncating_bf16_rounding(monkeypatch):
    """A planted mistake in the bf16 rounding (truncation instead of nearest-even) fails the
    torch rounding pin and the dequant pin."""
    def truncating(x):
        x = np.asarray(x, dtype=np.float32)
        return ((x.view(np.uint32) >> 16) << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    _mutant(monkeypatch, "f32_to_bf16", truncating)
    with pytest.raises(AssertionError):
        test_f32_to_bf16_matches_torch_rounding()
    with pytest.raises(AssertionError):
        test_fp8_dequant_definition()


def test_pins_catch_unrounded_dequant(monkeypatch):
    """A planted mistake that skips the bf16 rounding of the scaled value (the exact product)
    fails the dequant pin and the cache-gather pin."""
    _mutant(monkeypatch, "f32_to_bf16", lambda x: np.asarray(x, dtype=np.float32).astype(np.float64))
    with pytest.raises(AssertionError):
        test_fp8_dequant_definition()
    with pytest.raises(AssertionError):
        test_fp8_rows_match_torch_dequant()


def test_pins_catch_dropped_rope_term(monkeypatch):
    real = om.softmax_attention
    _mutant(monkeypatch, "softmax_attention", lambda q, k, v, s: real(q[:, :512], k[:, :512], v, s))
    assert _sdpa_pin_fails(_small(seed=14))


def test_pins_catch_wrong_causal_offset(monkeypatch):
    _mutant(monkeypatch, "visible_keys", lambda t, s, j, c: min(max(t - s + j, 0), t) if c else t)
    assert _sdpa_pin_fails(_small(s_q=4, h=2, lens=(40, 9, 20), causal=True, seed=15))


def test_pins_catch_missing_scale(monkeypatch):
    real = om.softmax_attention
    _mutant(monkeypatch, "softmax_attention", lambda q, k, v, s: real(q, k, v, 1.0))
    assert _sdpa_pin_fails(_small(seed=16))


def test_pins_catch_reversed_page_gather(monkeypatch):
    """Key order does not change softmax attention, so a wrong page order only shows when it
    moves the partly filled last page: its poisoned tail then enters the visible keys."""
    real = om.latent_rows

    def reversed_gather(kv, sc, dt, row, t):
        n = (t + 63) // 64
        r = np.array(row, copy=True)
        r[:n] = r[:n][::-1]
        return real(kv, sc, dt, r, t)

    w = _small(seed=17, lens=(130, 70, 100))
    out, _ = _run(w)
    assert np.isfinite(out).all()
    _mutant(monkeypatch, "latent_rows", reversed_gather)
    out_bad, _ = _run(w)
    assert not np.isfinite(out_bad).all()
