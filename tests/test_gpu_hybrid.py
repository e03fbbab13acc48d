"""GPU parity of the split latent + decompressed attention (page "Mla Analysis", section
"MLAvar6+ Design") against the fp64 oracle, through the C ABI:

* mla_hybrid_merge alone, with the old part's (out, lse) taken from the oracle: query rows
  s_q 1..32, head counts, new-token counts around the 32-token chunk (0, 1, 31, 33, 200), both
  masks and an empty old part. The kernel rounds P to bf16 and accumulates in fp32, as the
  latent decode does, so it is held to the bf16 decode bounds (rel L2 <= 5e-3, max abs <= 2e-2,
  |d lse| <= 1e-3).
* The whole chain: absorb the queries, latent decode over the old tokens, decompress, merge.
  The chain also rounds Qz and O_latent to bf16 (a relative 2^-8 each), so it is held to rel
  L2 <= 1e-2 and |d lse| <= 1e-2 (the absorb/decode/decompress chain's bound).
"""
import numpy as np
import pytest
import torch

import mla_latent_space_amd as mla
from mla_latent_space_amd import workloads as wl
from oracle import mla as om
from tests.gpu_common import BF16_TOL, compare

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _bf16(shape, gen, scale=1.0):
    t = (torch.randn(shape, generator=gen) * scale).to(torch.bfloat16)
    return t, t.double().numpy()


def _new_tokens(b, n, h, gen):
    k_new, kn = _bf16((b, n, h, 128), gen)
    kr_new, kr = _bf16((b, n, 64), gen)
    v_new, vn = _bf16((b, n, h, 128), gen)
    return (k_new, kr_new, v_new), (kn, kr, vn)


@pytest.mark.parametrize("s_q,heads,n,causal,o_lens", [
    (1, 16, 0, False, [5, 64, 300]),
    (1, 128, 1, False, [0, 1, 200]),
    (4, 32, 31, True, [7, 0, 129]),
    (16, 16, 33, True, [64, 100, 1]),
    (32, 16, 200, False, [0, 0, 0]),
    (2, 64, 200, True, [300, 33, 0]),
    (32, 16, 64, True, [10, 0, 500]),        # the largest query tile, causal
    (16, 128, 640, True, [300]),             # the benchmark's s_q, heads and new tokens (one sequence)
])
def test_merge_matches_oracle(s_q, heads, n, causal, o_lens):
    b = len(o_lens)
    gen = torch.Generator().manual_seed(1000 + 7 * s_q + heads + n)
    q_nope, qn = _bf16((b, s_q, heads, 128), gen)
    q_rope, qr = _bf16((b, s_q, heads, 64), gen)
    w_k = np.asarray(torch.randn((heads, 512, 128), generator=gen).double().numpy()) * 512 ** -0.5 * 4
    w_v = np.asarray(torch.randn((heads, 512, 128), generator=gen).double().numpy()) * 512 ** -0.5
    (k_new, kr_new, v_new), (kn, kr, vn) = _new_tokens(b, n, heads, gen)
    scale = 192 ** -0.5
    # old part from the oracle (latent rows drawn in fp64), then the full reference
    z_old = [torch.randn((o, om.D_QK), generator=gen).double().numpy() for o in o_lens]
    out_old = np.zeros((b, s_q, heads, 128))
    lse_old = np.full((b, s_q, heads), -np.inf)
    ref = np.zeros((b, s_q, heads, 128))
    ref_lse = np.zeros((b, s_q, heads))
    empty_k = np.zeros((0, heads, 128))
    for i in range(b):
        for j in range(s_q):
            out_old[i, j], lse_old[i, j] = om.decode_hybrid(qn[i, j], qr[i, j], w_k, w_v, z_old[i], empty_k,
                                                            np.zeros((0, 64)), empty_k, scale, 0)
            vis = om.hybrid_visible_new(n, s_q, j, causal)
            ref[i, j], ref_lse[i, j] = om.decode_hybrid(qn[i, j], qr[i, j], w_k, w_v, z_old[i], kn[i], kr[i], vn[i],
                                                        scale, vis)
    dev = "cuda"
    _say("hybrid merge", s_q, heads, n, causal, o_lens)
    out, lse = mla.hybrid_merge(q_nope.to(dev), q_rope.to(dev), k_new.to(dev) if n else None,
                                kr_new.to(dev) if n else None, v_new.to(dev) if n else None,
                                torch.from_numpy(out_old).float().to(dev), torch.from_numpy(lse_old).float().to(dev),
                                scale, causal)
    torch.cuda.synchronize()
    compare(out.cpu().numpy(), lse.cpu().numpy(), ref, ref_lse, BF16_TOL, f"hybrid s={s_q} h={heads} n={n}")


def test_merge_with_no_new_token_returns_the_old_part():
    """n = 0: out is the old part as given, lse its lse (to fp32 rounding)."""
    gen = torch.Generator().manual_seed(5)
    b, s_q, h = 2, 3, 16
    q_nope, _ = _bf16((b, s_q, h, 128), gen)
    q_rope, _ = _bf16((b, s_q, h, 64), gen)
    out_old = torch.randn((b, s_q, h, 128), generator=gen)
    lse_old = torch.randn((b, s_q, h), generator=gen)
    lse_old[0, 1, 3] = float("-inf")
    out_old[0, 1, 3] = 0.0
    _say("hybrid n=0")
    out, lse = mla.hybrid_merge(q_nope.cuda(), q_rope.cuda(), None, None, None, out_old.cuda(), lse_old.cuda(), 0.1)
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), out_old)
    got = lse.cpu()
    assert torch.isneginf(got[0, 1, 3])
    fin = torch.isfinite(lse_old)
    assert torch.allclose(got[fin], lse_old[fin], rtol=0, atol=1e-6)


def test_chain_latent_old_part_and_decompressed_new_tokens():
    """q_nope, q_rope, W_k, W_v, a paged latent cache of the old tokens and the new tokens
    decompressed -> absorb -> decode (old) -> decompress -> merge, against the oracle."""
    s_q, n = 4, 40
    w = wl.make_workload("hybrid-chain", batch=3, s_q=1, heads=32, seqlens=[300, 64, 1], seed=43, poison=False)
    b, h = w.batch, w.heads
    gen = torch.Generator().manual_seed(950)
    q_nope, qn = _bf16((b, s_q, h, 128), gen)
    q_rope, qr = _bf16((b, s_q, h, 64), gen)
    w_k, wk = _bf16((h, 512, 128), gen, 128 ** -0.5)
    w_v, wv = _bf16((h, 512, 128), gen, 512 ** -0.5)
    (k_new, kr_new, v_new), (kn, kr, vn) = _new_tokens(b, n, h, gen)
    scale = 192 ** -0.5
    dev = "cuda"
    _say("hybrid chain")
    qz = mla.absorb_query(q_nope.to(dev), q_rope.to(dev), w_k.to(dev))
    kv = torch.from_numpy(w.kv.view(np.int16)).to(dev).view(torch.bfloat16)
    bt = torch.from_numpy(w.block_table).to(dev)
    sl = torch.from_numpy(w.seqlens).to(dev)
    o_lat, lse_old = mla.decode_fwd(qz, kv, bt, sl, scale, causal=False)
    out_old = mla.decompress_output(o_lat, w_v.transpose(1, 2).contiguous().to(dev))
    out, lse = mla.hybrid_merge(q_nope.to(dev), q_rope.to(dev), k_new.to(dev), kr_new.to(dev), v_new.to(dev),
                                out_old, lse_old, scale, causal=True)
    torch.cuda.synchronize()
    got, got_lse = out.cpu().double().numpy(), lse.cpu().double().numpy()
    ref = np.empty_like(got)
    ref_lse = np.empty_like(got_lse)
    for i in range(b):
        z = om.latent_rows(w.kv, None, "bf16", w.block_table[i], int(w.seqlens[i]))
        for j in range(s_q):
            ref[i, j], ref_lse[i, j] = om.decode_hybrid(qn[i, j], qr[i, j], wk, wv, z, kn[i], kr[i], vn[i], scale,
                                                        om.hybrid_visible_new(n, s_q, j, True))
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    dl = np.max(np.abs(got_lse - ref_lse))
    assert rel <= 1e-2 and dl <= 1e-2, (rel, dl)
