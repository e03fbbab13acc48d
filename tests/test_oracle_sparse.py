"""Pins of the oracle's token-level sparse decode (library card page "FlashMLA: Efficient
Multi-head Latent Attention Kernels": sparse attention over selected tokens in decoding) to
results fixed independently of it:

* the full list 0 .. t-1 gives the dense decode (decode_latent, pinned in test_oracle_mla.py),
  for bf16 and fp8 caches;
* the result does not depend on the order of the list, nor on padding entries (negative or
  >= t) mixed into it (properties of a softmax over a set of keys);
* a list that repeats one position k times has out = that row and lse = score + log k (a
  closed form);
* an empty (all-padding) list gives out 0 and lse -inf.
"""
import numpy as np
import pytest

from mla_latent_space_amd import workloads as wl
from oracle import mla as om


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_full_list_equals_dense_decode(kv_dtype):
    w = wl.make_workload("sparse-dense", batch=2, s_q=2, heads=16, seqlens=[70, 33], kv_dtype=kv_dtype, seed=61)
    topk = int(w.seqlens.max())
    idx = np.full((w.batch, w.s_q, topk), -1, dtype=np.int32)
    for i in range(w.batch):
        idx[i, :, :int(w.seqlens[i])] = np.arange(int(w.seqlens[i]))
    got, got_lse = om.decode_sparse(w.q, w.kv, w.kv_scales, kv_dtype, w.block_table, w.seqlens, idx, w.scale)
    ref, ref_lse = om.decode_latent(w.q, w.kv, w.kv_scales, kv_dtype, w.block_table, w.seqlens, w.scale, False)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(got_lse, ref_lse, rtol=1e-12, atol=1e-12)


def test_order_and_padding_do_not_matter():
    w = wl.make_workload("sparse-perm", batch=1, s_q=1, heads=16, seqlens=[200], kv_dtype="fp8", seed=62)
    rng = np.random.default_rng(3)
    sel = rng.choice(200, size=50, replace=False).astype(np.int32)
    a = sel[None, None, :]
    padded = np.concatenate([rng.permutation(sel), np.array([-1, 200, 7000, -5], dtype=np.int32)])
    b = rng.permutation(padded)[None, None, :]
    o1, l1 = om.decode_sparse(w.q, w.kv, w.kv_scales, "fp8", w.block_table, w.seqlens, a, w.scale)
    o2, l2 = om.decode_sparse(w.q, w.kv, w.kv_scales, "fp8", w.block_table, w.seqlens, b, w.scale)
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l2, l1, rtol=1e-12, atol=1e-13)


def test_repeated_position_closed_form():
    w = wl.make_workload("sparse-rep", batch=1, s_q=1, heads=16, seqlens=[100], seed=63)
    k, u = 5, 42
    idx = np.full((1, 1, k), u, dtype=np.int32)
    got, got_lse = om.decode_sparse(w.q, w.kv, None, "bf16", w.block_table, w.seqlens, idx, w.scale)
    z = om.latent_rows(w.kv, None, "bf16", w.block_table[0], 100)[u]
    q = om.bf16_bits_to_f64(w.q[0, 0])
    np.testing.assert_allclose(got[0, 0], np.broadcast_to(z[:om.K_LAT], (16, om.K_LAT)), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(got_lse[0, 0], w.scale * (q @ z) + np.log(k), rtol=1e-13, atol=1e-12)


def test_all_padding_is_empty():
    w = wl.make_workload("sparse-empty", batch=1, s_q=1, heads=16, seqlens=[10], seed=64)
    idx = np.array([[[-1, 10, 11]]], dtype=np.int32)
    got, got_lse = om.decode_sparse(w.q, w.kv, None, "bf16", w.block_table, w.seqlens, idx, w.scale)
    assert np.all(got == 0) and np.all(np.isneginf(got_lse))
