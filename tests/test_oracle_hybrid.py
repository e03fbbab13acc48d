"""Pins of the oracle's split latent + decompressed attention (page "Mla Analysis", section
"MLAvar6+ Design") to results fixed independently of it:

* when the new tokens' K, V and rope keys are exactly the decompression of latent rows, the
  split attention equals the explicit attention over all t latent rows (decode_explicit,
  pinned in test_oracle_mla.py) for every split point o, and under the causal reading for
  every query token;
* with a zero query every visible key scores the same, so out is the plain mean of the visible
  values and lse = log(number of visible keys) (a closed form);
* an empty key set gives out 0 and lse -inf.
"""
import numpy as np
import pytest

from oracle import mla as om


def _latent_case(rng, h=3, t=29):
    z = rng.standard_normal((t, om.D_QK))
    w_k = rng.standard_normal((h, om.K_LAT, 128)) * om.K_LAT ** -0.5
    w_v = rng.standard_normal((h, om.K_LAT, 128)) * om.K_LAT ** -0.5
    q_nope = rng.standard_normal((h, 128))
    q_rope = rng.standard_normal((h, om.P_ROPE))
    return z, w_k, w_v, q_nope, q_rope


def _decompressed(z_new, w_k, w_v):
    """The new tokens as the method stores them: K [n, h, d], KPE [n, p], V [n, h, d]."""
    k_new = np.einsum("nk,hkd->nhd", z_new[:, :om.K_LAT], w_k)
    v_new = np.einsum("nk,hkd->nhd", z_new[:, :om.K_LAT], w_v)
    return k_new, z_new[:, om.K_LAT:], v_new


@pytest.mark.parametrize("o", [0, 1, 14, 28, 29])
def test_split_equals_explicit_attention_over_all_rows(o):
    rng = np.random.default_rng(100 + o)
    z, w_k, w_v, qn, qr = _latent_case(rng)
    t = z.shape[0]
    scale = 192 ** -0.5
    k_new, kr_new, v_new = _decompressed(z[o:], w_k, w_v)
    got, got_lse = om.decode_hybrid(qn, qr, w_k, w_v, z[:o], k_new, kr_new, v_new, scale, t - o)
    ref, ref_lse = om.decode_explicit(qn, qr, w_k, w_v, z, scale)
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(got_lse, ref_lse, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("s_q", [1, 3, 8])
def test_causal_split_matches_the_causal_reading(s_q):
    """Query j of s_q sees t - s_q + 1 + j of the t keys: the old ones and the first
    n - s_q + 1 + j new ones."""
    rng = np.random.default_rng(200 + s_q)
    z, w_k, w_v, qn, qr = _latent_case(rng, h=2, t=23)
    t, n = z.shape[0], 9
    o = t - n
    scale = 0.11
    k_new, kr_new, v_new = _decompressed(z[o:], w_k, w_v)
    for j in range(s_q):
        vis_new = om.hybrid_visible_new(n, s_q, j, True)
        assert o + vis_new == om.visible_keys(t, s_q, j, True)
        got, got_lse = om.decode_hybrid(qn, qr, w_k, w_v, z[:o], k_new, kr_new, v_new, scale, vis_new)
        ref, ref_lse = om.decode_explicit(qn, qr, w_k, w_v, z[:o + vis_new], scale)
        np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(got_lse, ref_lse, rtol=1e-12, atol=1e-12)
    with pytest.raises(ValueError):
        om.hybrid_visible_new(2, 3, 0, True)
    assert om.hybrid_visible_new(5, 3, 0, False) == 5


def test_zero_query_gives_the_mean_of_visible_values():
    rng = np.random.default_rng(7)
    h, o, n, vis = 2, 6, 5, 3
    z_old = rng.standard_normal((o, om.D_QK))
    w_k = rng.standard_normal((h, om.K_LAT, 128))
    w_v = rng.standard_normal((h, om.K_LAT, 128))
    k_new = rng.standard_normal((n, h, 128))
    kr_new = rng.standard_normal((n, om.P_ROPE))
    v_new = rng.standard_normal((n, h, 128))
    zero_n, zero_r = np.zeros((h, 128)), np.zeros((h, om.P_ROPE))
    got, got_lse = om.decode_hybrid(zero_n, zero_r, w_k, w_v, z_old, k_new, kr_new, v_new, 0.3, vis)
    for eta in range(h):
        values = np.concatenate([z_old[:, :om.K_LAT] @ w_v[eta], v_new[:vis, eta]], axis=0)
        np.testing.assert_allclose(got[eta], values.mean(axis=0), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(got_lse, np.log(o + vis), rtol=0, atol=1e-14)


def test_empty_key_set():
    h = 2
    got, got_lse = om.decode_hybrid(np.ones((h, 128)), np.ones((h, om.P_ROPE)), np.ones((h, om.K_LAT, 128)),
                                    np.ones((h, om.K_LAT, 128)), np.zeros((0, om.D_QK)), np.zeros((4, h, 128)),
                                    np.zeros((4, om.P_ROPE)), np.zeros((4, h, 128)), 1.0, 0)
    assert np.all(got == 0) and np.all(np.isneginf(got_lse))
