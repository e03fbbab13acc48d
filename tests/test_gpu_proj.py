"""GPU parity of the two projections around the attention (query absorption, output
decompression) against the fp64 oracle, through the C ABI, and the whole chain absorb ->
decode -> decompress against the oracle's explicit (decompressed) attention."""
import numpy as np
import pytest
import torch

import mla_latent_space_amd as mla
from mla_latent_space_amd import workloads as wl
from oracle import mla as om

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _bf16(shape, gen, scale=1.0):
    """Seeded N(0, scale^2) values rounded to bf16: (bf16 tensor, exact float64 values)."""
    t = (torch.randn(shape, generator=gen) * scale).to(torch.bfloat16)
    return t, t.double().numpy()


@pytest.mark.parametrize("tokens,heads", [(1, 16), (3, 16), (37, 32), (64, 128), (65, 16), (100, 64), (300, 16),
                                           (517, 8), (100, 12)])
def test_absorb_query_matches_oracle(tokens, heads):
    """Qz nope part within the bf16 rounding of the exact value (unit roundoff 2^-8) plus the
    fp32 accumulation error (<= 2^-20 sum |q w| for 128 terms); the rope part copied bit for
    bit."""
    gen = torch.Generator().manual_seed(700 + tokens + heads)
    q_nope, qn = _bf16((tokens, heads, 128), gen)
    q_rope, qr = _bf16((tokens, heads, 64), gen)
    w_k, wk = _bf16((heads, 512, 128), gen, 128 ** -0.5)
    _say("absorb", tokens, heads)
    qz = mla.absorb_query(q_nope.cuda(), q_rope.cuda(), w_k.cuda())
    torch.cuda.synchronize()
    got = qz.cpu().double().numpy()
    for t in range(tokens):
        ref = om.absorbed_query(qn[t], qr[t], wk)                     # [h, 576]
        mag = np.einsum("hkd,hd->hk", np.abs(wk), np.abs(qn[t]))       # sum |q w| per output
        err = np.abs(got[t, :, :512] - ref[:, :512])
        bound = 2.0 ** -8 * np.abs(ref[:, :512]) + 2.0 ** -20 * mag + 1e-30
        assert np.all(err <= bound), f"token {t}: worst {np.max(err / bound):.3f} of the bound"
        assert np.array_equal(got[t, :, 512:], ref[:, 512:]), f"token {t}: rope part not copied exactly"


@pytest.mark.parametrize("tokens,heads", [(1, 16), (5, 32), (64, 128), (65, 16), (70, 16), (200, 16), (517, 8),
                                           (300, 128), (2050, 16), (2760, 12)])
def test_decompress_output_matches_oracle(tokens, heads):
    """out within (2^-8 + 2^-14) sum |a w| of the exact product: O_latent is rounded to bf16 on
    load (unit roundoff 2^-8 per term) and 512 terms are accumulated in fp32 (below 2^-14)."""
    gen = torch.Generator().manual_seed(800 + tokens + heads)
    o_lat = torch.randn((tokens, heads, 512), generator=gen, dtype=torch.float32)
    ol = o_lat.double().numpy()
    w_v, wv = _bf16((heads, 512, 128), gen, 512 ** -0.5)              # the oracle's [h, k, d]
    w_v_t = w_v.transpose(1, 2).contiguous()                          # [h, d, k]: contraction innermost
    _say("decompress", tokens, heads)
    out = mla.decompress_output(o_lat.cuda(), w_v_t.cuda())
    torch.cuda.synchronize()
    got = out.cpu().double().numpy()
    for t in range(tokens):
        ref = om.decompress_output(ol[t], wv)                          # [h, 128]
        mag = np.einsum("hk,hkd->hd", np.abs(ol[t]), np.abs(wv))
        err = np.abs(got[t] - ref)
        bound = (2.0 ** -8 + 2.0 ** -14) * mag + 1e-30
        assert np.all(err <= bound), f"token {t}: worst {np.max(err / bound):.3f} of the bound"
    rel = np.linalg.norm(got - np.stack([om.decompress_output(ol[t], wv) for t in range(tokens)])) / np.linalg.norm(got)
    assert rel <= 5e-3, rel


def test_absorb_decode_decompress_chain_matches_explicit_attention():
    """q_nope, q_rope, W_k, W_v and a paged latent cache -> absorb -> decode -> decompress,
    against the oracle's decompressed attention softmax(Q K^T) V with K = [Z W_k | Z_rope] and
    V = Z W_v. The chain rounds Qz to bf16 (a relative 2^-8 per element) and O_latent to
    bf16 for the last product, so it is held to rel L2 <= 1e-2 and |d lse| <= 1e-2; the tight
    bounds are on each kernel above and on the decode's own tests."""
    w = wl.make_workload("chain", batch=3, s_q=1, heads=16, seqlens=[200, 64, 513], seed=41, poison=False)
    gen = torch.Generator().manual_seed(900)
    h = w.heads
    q_nope, qn = _bf16((w.batch, 1, h, 128), gen)
    q_rope, qr = _bf16((w.batch, 1, h, 64), gen)
    w_k, wk = _bf16((h, 512, 128), gen, 128 ** -0.5)
    w_v, wv = _bf16((h, 512, 128), gen, 512 ** -0.5)
    dev = "cuda"
    _say("chain")
    qz = mla.absorb_query(q_nope.to(dev), q_rope.to(dev), w_k.to(dev))
    kv = torch.from_numpy(w.kv.view(np.int16)).to(dev).view(torch.bfloat16)
    bt = torch.from_numpy(w.block_table).to(dev)
    sl = torch.from_numpy(w.seqlens).to(dev)
    o_lat, lse = mla.decode_fwd(qz, kv, bt, sl, w.scale)
    out = mla.decompress_output(o_lat, w_v.transpose(1, 2).contiguous().to(dev))
    torch.cuda.synchronize()
    got, got_lse = out.cpu().double().numpy(), lse.cpu().double().numpy()
    ref = np.empty_like(got)
    ref_lse = np.empty_like(got_lse)
    for b in range(w.batch):
        z = om.latent_rows(w.kv, None, "bf16", w.block_table[b], int(w.seqlens[b]))
        o, l = om.decode_explicit(qn[b, 0], qr[b, 0], wk, wv, z, w.scale)
        ref[b, 0], ref_lse[b, 0] = o, l
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    dl = np.max(np.abs(got_lse - ref_lse))
    assert rel <= 1e-2 and dl <= 1e-2, (rel, dl)
