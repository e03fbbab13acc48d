"""GPU parity of the token-level sparse decode over an fp8 cache (library card page "FlashMLA:
Efficient Multi-head Latent Attention Kernels": sparse attention over selected tokens in
decoding) against the fp64 oracle, through the C ABI: lists shorter and longer than a
32-token step, random order, duplicates, padding entries, empty lists, query tokens of one
sequence with different lists, several worker counts (split lists), a bitwise repeat, every
row at the full V3.2-like size, and a listed key whose page id is outside the cache (reported
in the status word). Held to the fp8 bounds of the dense decode."""
import numpy as np
import pytest
import torch

import mla_latent_space_amd as mla
from mla_latent_space_amd import workloads as wl
from oracle import mla as om
from tests.gpu_common import FP8_TOL, Dev, compare, fp8_rope_ramp

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _run(w, idx, num_workers=None, expect_status=0):
    """Row lists, plan and decode; out and lse start as NaN and the status word must read
    expect_status afterwards."""
    d = Dev(w)
    ind = torch.from_numpy(idx).cuda()
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    plan = mla.get_sparse_plan(ind, d.bt, d.sl, int(w.kv.shape[0]), w.heads, num_workers, status=status)
    out = torch.full((w.batch, w.s_q, w.heads, 512), float("nan"), device="cuda")
    lse = torch.full((w.batch, w.s_q, w.heads), float("nan"), device="cuda")
    mla.sparse_decode_fwd(d.q, d.kv, d.scales, w.scale, plan, out=out, lse=lse, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == expect_status, int(status.item())
    return out.cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("topk,s_q,fill,pad,dup,W", [
    (1, 1, 1.0, 0.0, 0.0, 256),
    (31, 2, 1.0, 0.0, 0.0, 7),
    (33, 1, 0.7, 0.2, 0.0, 256),
    (100, 4, 1.0, 0.1, 0.1, 1),
    (300, 2, 0.5, 0.05, 0.05, 5),
    (2048, 1, 1.0, 0.0, 0.0, 256),
])
def test_sparse_matches_oracle(topk, s_q, fill, pad, dup, W):
    w = wl.make_workload("sparse", batch=4, s_q=s_q, heads=128, seqlens=[5, 64, 700, 2100], kv_dtype="fp8",
                         seed=70 + topk + s_q)
    idx = wl.make_sparse_indices(w.seqlens, s_q, topk, seed=80 + topk, fill=fill, pad_frac=pad, dup_frac=dup)
    _say("sparse topk", topk, "s_q", s_q, "W", W)
    out, lse = _run(w, idx, W)
    ro, rl = om.decode_sparse(w.q, w.kv, w.kv_scales, "fp8", w.block_table, w.seqlens, idx, w.scale)
    compare(out, lse, ro, rl, FP8_TOL, f"sparse topk={topk} s_q={s_q} W={W}")


def test_sparse_empty_lists_and_bitwise_repeat():
    w = wl.make_workload("sparse-empty", batch=3, s_q=2, heads=128, seqlens=[0, 10, 300], kv_dtype="fp8", seed=91)
    idx = wl.make_sparse_indices(w.seqlens, 2, 64, seed=92)
    idx[1, 0, :] = -1                       # an all-padding list
    idx[2, 1, :] = 5000                     # positions past the sequence
    _say("sparse empty + repeat")
    o1, l1 = _run(w, idx, 13)
    o2, l2 = _run(w, idx, 13)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    for (i, j) in ((0, 0), (0, 1), (1, 0), (2, 1)):
        assert np.all(o1[i, j] == 0) and np.all(np.isneginf(l1[i, j]))
    ro, rl = om.decode_sparse(w.q, w.kv, w.kv_scales, "fp8", w.block_table, w.seqlens, idx, w.scale)
    compare(o1, l1, ro, rl, FP8_TOL, "sparse empty")


def test_sparse_full_size():
    """64 sequences of 32,768 fp8 tokens, 2,048 selected tokens per query token; every output
    element against the oracle."""
    w = wl.make_config("fp8")
    idx = wl.make_sparse_indices(w.seqlens, w.s_q, 2048, seed=93)
    _say("sparse full size")
    out, lse = _run(w, idx)
    ro, rl = om.decode_sparse(w.q, w.kv, w.kv_scales, "fp8", w.block_table, w.seqlens, idx, w.scale)
    compare(out, lse, ro, rl, FP8_TOL, "sparse full size")


def test_sparse_page_out_of_range_reads_as_zeros_and_is_reported():
    """A listed key on a page whose block-table entry is outside [0, num_pages): that key reads
    as a zero row, and the row lists set MLA_DEVICE_PAGE_OUT_OF_RANGE."""
    w = wl.make_workload("sparse-oob", batch=2, s_q=1, heads=128, seqlens=[200, 100], kv_dtype="fp8", seed=96,
                         poison=False)
    bad = w.block_table.copy()
    bad[0, 1] = w.num_pages + 7
    w2 = wl.Workload(**{**w.__dict__, "block_table": bad})
    idx = wl.make_sparse_indices(w.seqlens, 1, 150, seed=97)
    _say("sparse oob page")
    out, lse = _run(w2, idx, 8, expect_status=2)
    kv0 = np.concatenate([w.kv, np.zeros((1,) + w.kv.shape[1:], dtype=w.kv.dtype)])
    sc0 = np.concatenate([w.kv_scales, np.zeros((1,) + w.kv_scales.shape[1:], dtype=w.kv_scales.dtype)])
    bt0 = bad.copy()
    bt0[0, 1] = w.num_pages
    ro, rl = om.decode_sparse(w.q, kv0, sc0, "fp8", bt0, w.seqlens, idx, w.scale)
    compare(out, lse, ro, rl, FP8_TOL, "sparse oob")


@pytest.mark.parametrize("W", [1, 256])
def test_sparse_scores_growing_past_the_reference_window(W):
    """The redo passes on the token-sparse kernel (its own pipeline fill with the row ring):
    scores that grow along the selected tokens by hundreds of log2 units, through the cache's
    bf16 rope channels; full lists in random order."""
    w = wl.make_workload("ramp-sparse", batch=2, s_q=1, heads=128, seqlens=[600, 3000], kv_dtype="fp8", seed=34,
                         poison=False)
    fp8_rope_ramp(w)
    idx = wl.make_sparse_indices(w.seqlens, 1, 3000, seed=95)
    _say("sparse ramp W", W)
    out, lse = _run(w, idx, W)
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    ro, rl = om.decode_sparse(w.q, w.kv, w.kv_scales, "fp8", w.block_table, w.seqlens, idx, w.scale)
    compare(out, lse, ro, rl, FP8_TOL, f"sparse ramp W={W}")
