"""GPU parity: the HIP library (through the C ABI) against the fp64 oracle on the same seeded
inputs. Every case compares every output element, the full-size workloads included (two seeds
each). The split plan must match the oracle's plan definition bit for bit."""
import numpy as np
import pytest
import torch

import mla_latent_space_amd as mla
from mla_latent_space_amd import workloads as wl
from oracle import mla as om
from oracle import plan as op

from gpu_common import BF16_TOL, FP8_TOL, Dev, compare, fp8_rope_ramp

pytestmark = pytest.mark.gpu

PLAN_OVERHEAD = 6   # the library's per-item cost in page units (header word 9 of the plan)


def _say(*a):
    print(*a, flush=True)


def _oracle_all(w, seqs=None):
    return om.decode_latent(w.q, w.kv, w.kv_scales, w.kv_dtype, w.block_table, w.seqlens, w.scale, w.causal, seqs)


def _tol(w):
    return BF16_TOL if w.kv_dtype == "bf16" else FP8_TOL


def _check_full(w, num_workers=None, what=""):
    d = Dev(w)
    out, lse = d.run(num_workers)
    ro, rl = _oracle_all(w)
    return compare(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, _tol(w), what or w.name)


# ----------------------------------------------------------------------------- plan

def _plan_words(p: op.Plan, batch, s_q, heads, causal):
    n = len(p.pages)
    W = p.num_workers
    hdr = [0x4D4C4150, 2, batch, s_q, heads, int(causal), W, p.n_tiles, n, p.overhead, p.total_cost,
           p.active_workers, len(p.split_items), p.n_slots, 0, 0]
    items = np.stack([p.seq, p.tile, p.vis, p.pages, p.cost_begin, p.owner, p.nsplits, p.slot_base], axis=1)
    workers = np.concatenate([p.worker_begin, p.worker_end], axis=1)
    k = p.split_items
    split = np.stack([p.seq[k], p.tile[k], p.nsplits[k], p.slot_base[k]], axis=1).reshape(-1)
    return np.array(hdr, dtype=np.int64), items.astype(np.int64), workers.astype(np.int64), split.astype(np.int64)


PLAN_CASES = [
    dict(seqlens=[4096] * 64, s_q=1, h=128, causal=False, W=256),
    dict(seqlens=[300, 64, 1, 0, 9000, 130], s_q=1, h=128, causal=False, W=7),
    dict(seqlens=[4096] * 32, s_q=16, h=128, causal=True, W=256),
    dict(seqlens=[20, 5, 70, 3], s_q=16, h=16, causal=True, W=5),
    dict(seqlens=[256, 256], s_q=1, h=16, causal=False, W=256),
    dict(seqlens="jagged", s_q=1, h=128, causal=False, W=256),
    dict(seqlens="random3000", s_q=2, h=64, causal=True, W=1000),
    dict(seqlens=[1000] * 2000, s_q=1, h=128, causal=False, W=256),    # one length, radix-size batch
    dict(seqlens=[500] * 300, s_q=1, h=64, causal=False, W=97),        # one length, 257..1024 items
    dict(seqlens=[700, 700, 64, 700] * 70, s_q=1, h=128, causal=False, W=256),   # 257..1024, mixed
    dict(seqlens="random16000", s_q=1, h=128, causal=False, W=1024),  # n + W + 1 > 16384: starts not kept in LDS
    dict(seqlens="random200long", s_q=1, h=128, causal=False, W=4096),  # the most workers, rank sort
]


@pytest.mark.parametrize("case", range(len(PLAN_CASES)))
def test_device_plan_matches_oracle_definition(case):
    c = dict(PLAN_CASES[case])
    if c["seqlens"] == "jagged":
        c["seqlens"] = wl._draw_lengths(wl.CONFIGS["jagged"]["lengths"], 128, torch.Generator().manual_seed(1002)).tolist()
    elif c["seqlens"] == "random3000":
        c["seqlens"] = np.random.default_rng(5).integers(0, 20000, 3000).tolist()
    elif c["seqlens"] == "random16000":
        c["seqlens"] = np.random.default_rng(9).integers(0, 3000, 16000).tolist()
    elif c["seqlens"] == "random200long":
        c["seqlens"] = np.random.default_rng(10).integers(0, 200000, 200).tolist()
    _say("plan case", case, "batch", len(c["seqlens"]))
    sl = torch.tensor(c["seqlens"], dtype=torch.int32, device="cuda")
    plan = mla.get_split_plan(sl, c["s_q"], c["h"], c["causal"], c["W"])
    words = plan.buffer.view(torch.int32).cpu().numpy().astype(np.int64)
    ref = op.split_plan(c["seqlens"], c["s_q"], c["h"], c["causal"], c["W"], PLAN_OVERHEAD)
    hdr, items, workers, split = _plan_words(ref, len(c["seqlens"]), c["s_q"], c["h"], c["causal"])
    n, W = items.shape[0], c["W"]
    assert np.array_equal(words[:16], hdr)
    assert np.array_equal(words[16:16 + 8 * n].reshape(n, 8), items)
    wo = 16 + 8 * n
    assert np.array_equal(words[wo:wo + 4 * W].reshape(W, 4), workers)
    so = wo + 4 * W
    assert np.array_equal(words[so:so + len(split)], split)


# ----------------------------------------------------------------------------- decode, small and exact

def test_tiny_config_all_outputs():
    _say("tiny config")
    _check_full(wl.make_config("tiny"))


@pytest.mark.parametrize("W", [1, 3, 7, 64, 256])
def test_ragged_multi_tile_any_worker_count(W):
    """Lengths that end mid-page and mid-step, a one-token sequence, several pages; any
    number of workers (forcing 1..many splits per sequence)."""
    w = wl.make_workload("ragged", batch=6, s_q=1, heads=128, seqlens=[1, 31, 63, 64, 65, 1000], seed=21)
    _say("ragged W", W)
    _check_full(w, num_workers=W, what=f"ragged W={W}")


@pytest.mark.parametrize("heads,s_q,causal", [(16, 1, False), (32, 1, False), (64, 1, False), (16, 16, True),
                                              (64, 4, True), (128, 3, False), (32, 5, True)])
def test_head_counts_and_query_tokens(heads, s_q, causal):
    lens = [s_q, s_q + 1, 100, 257]
    w = wl.make_workload("heads", batch=4, s_q=s_q, heads=heads, seqlens=lens, causal=causal, seed=22 + heads + s_q)
    _say("heads", heads, "s_q", s_q, "causal", causal)
    _check_full(w, num_workers=13, what=f"h={heads} s={s_q} causal={causal}")


def test_speculative_small():
    w = wl.make_workload("spec-small", batch=3, s_q=16, heads=128, seqlens=[16, 17, 300], causal=True, seed=23)
    _say("spec small")
    _check_full(w, num_workers=17)


def test_empty_visible_sets():
    """t = 0, and causal rows that see nothing (t < s): out 0, lse -inf."""
    w = wl.make_workload("empty", batch=3, s_q=4, heads=32, seqlens=[0, 2, 70], causal=True, seed=24)
    _say("empty visible sets")
    d = Dev(w)
    out, lse = d.run(5)
    ro, rl = _oracle_all(w)
    assert np.isneginf(rl[0]).all() and np.isneginf(rl[1, :2]).all()
    compare(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, BF16_TOL, "empty")
    assert (out[0] == 0).all()


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _bits_to_f32(b: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).float().numpy()


@pytest.mark.parametrize("W", [1, 5, 256])
def test_scores_growing_past_the_reference_window(W):
    """Scores that grow along the sequence by hundreds of log2 units: the first pass's row
    sum overflows, so the kernel redoes the segment taking the row maximum on every step,
    then (a row still leaving the window) with the segment's maximum as the reference."""
    w = wl.make_workload("ramp", batch=2, s_q=1, heads=32, seqlens=[600, 3000], seed=31, poison=False)
    q = _bits_to_f32(w.q)
    q[:, :, :16, :64] = 64.0            # heads 0..15 align with the ramp direction
    w.q = _bf16_bits(q)
    kv = _bits_to_f32(w.kv)
    for b, t in enumerate(w.seqlens):
        for j in range(t):
            page, slot = w.block_table[b, j // 64], j % 64
            kv[page, slot, :64] += 1.0 * j / max(1, t - 1)   # score ramp of 4096 (~426 log2 units)
    w.kv = _bf16_bits(kv)
    _say("ramp W", W)
    ro, rl = _oracle_all(w)
    d = Dev(w)
    out, lse = d.run(W)
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()
    compare(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, BF16_TOL, f"ramp W={W}")


@pytest.mark.parametrize("W", [1, 256])
def test_fp8_scores_growing_past_the_reference_window(W):
    """The redo passes on the fp8 kernel, whose pipeline fill (staging, dequantisation) is its
    own: the same growing scores through the cache's bf16 rope channels."""
    w = wl.make_workload("ramp-fp8", batch=2, s_q=1, heads=32, seqlens=[600, 3000], kv_dtype="fp8", seed=33,
                         poison=False)
    fp8_rope_ramp(w)
    _say("fp8 ramp W", W)
    ro, rl = _oracle_all(w)
    out, lse = Dev(w).run(W)
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()
    compare(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, FP8_TOL, f"fp8 ramp W={W}")


def test_scores_growing_moderately_past_the_reference_window():
    """Heads 0..15 score exactly 90 j / (t - 1) log2 units at token j (one query channel of
    864 against a cached channel that ramps from 0 to 1): the row maximum ends about 87 log2
    units above the first-step reference, so the first pass's row sum is finite but above
    2^60, and the segment is redone with the reference ceil(m + log2 l)."""
    w = wl.make_workload("ramp90", batch=2, s_q=1, heads=32, seqlens=[600, 3000], seed=32, poison=False)
    q = _bits_to_f32(w.q)
    q[:, :, :16, :] = 0.0
    q[:, :, :16, 0] = 864.0
    w.q = _bf16_bits(q)
    kv = _bits_to_f32(w.kv)
    for b, t in enumerate(w.seqlens):
        for j in range(t):
            kv[w.block_table[b, j // 64], j % 64, 0] = j / (t - 1)
    w.kv = _bf16_bits(kv)
    _say("ramp 90")
    ro, rl = _oracle_all(w)
    d = Dev(w)
    out, lse = d.run(1)
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()
    compare(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, BF16_TOL, "ramp 90")


def test_plan_independence_and_bitwise_repeat():
    w = wl.make_workload("indep", batch=5, s_q=1, heads=128, seqlens=[5000, 64, 700, 1, 2049], seed=25)
    d = Dev(w)
    ro, rl = _oracle_all(w)
    outs = []
    for W in (1, 8, 256):
        _say("independence W", W)
        plan = d.plan(W)
        o1, l1 = d.run(plan=plan)
        o2, l2 = d.run(plan=plan)
        assert torch.equal(o1, o2) and torch.equal(l1, l2), "not bitwise reproducible for a fixed plan"
        compare(o1.cpu().numpy(), l1.cpu().numpy(), ro, rl, BF16_TOL, f"W={W}")
        outs.append(o1.cpu().numpy())
    # different split points round P to bf16 against different running maxima, so plans agree
    # to the stated tolerance, not bit for bit
    for o in outs[1:]:
        assert np.linalg.norm(o - outs[0]) / np.linalg.norm(outs[0]) <= BF16_TOL["rel_l2"]
        assert np.max(np.abs(o - outs[0])) <= BF16_TOL["max_abs"]


def test_poison_does_not_propagate():
    """NaN in unused tail slots and spare pages; every output finite and equal to the run
    on the same data without poison (bit for bit, same plan)."""
    kw = dict(batch=3, s_q=1, heads=128, seqlens=[70, 129, 5], seed=26)
    wp = wl.make_workload("poison", poison=True, **kw)
    wc = wl.make_workload("clean", poison=False, **kw)
    _say("poison")
    op_, lp = Dev(wp).run(4)
    oc, lc = Dev(wc).run(4)
    assert torch.isfinite(op_).all() and torch.isfinite(lp).all()
    assert torch.equal(op_, oc) and torch.equal(lp, lc)


def test_page_ids_out_of_range_read_as_zeros_and_are_reported():
    """A block-table entry outside [0, num_pages) must not fault: those rows read as zeros, and
    the call sets MLA_DEVICE_PAGE_OUT_OF_RANGE in its status word."""
    w = wl.make_workload("oob", batch=2, s_q=1, heads=128, seqlens=[192, 64], seed=27, poison=False)
    bad = w.block_table.copy()
    bad[0, 1] = w.num_pages + 1000
    w2 = wl.Workload(**{**w.__dict__, "block_table": bad})
    _say("oob page id")
    out, lse = Dev(w2).run(4, expect_status=2)
    kv0 = np.concatenate([w.kv, np.zeros((1,) + w.kv.shape[1:], dtype=w.kv.dtype)])
    bt0 = bad.copy()
    bt0[0, 1] = w.num_pages
    ro, rl = om.decode_latent(w.q, kv0, None, "bf16", bt0, w.seqlens, w.scale, False)
    compare(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, BF16_TOL, "oob")


@pytest.mark.parametrize("s_q,causal", [(1, False), (4, True)])
def test_lengths_beyond_block_table_capacity(s_q, causal):
    """A length above max_pages * 64 reads as max_pages * 64 (the documented cap): same result
    as the oracle run at the capped length, and MLA_DEVICE_LENGTH_OVER_CAPACITY is reported."""
    w = wl.make_workload("cap", batch=2, s_q=s_q, heads=32, seqlens=[150, 70], causal=causal, seed=28,
                         poison=False)
    cap = w.block_table.shape[1] * 64
    capped = wl.Workload(**{**w.__dict__, "seqlens": np.array([cap, 70], dtype=w.seqlens.dtype)})
    beyond = wl.Workload(**{**w.__dict__, "seqlens": np.array([cap + 40, 70], dtype=w.seqlens.dtype)})
    _say("lengths beyond capacity", s_q, causal)
    out, lse = Dev(beyond).run(5, expect_status=4)
    ro, rl = _oracle_all(capped)
    compare(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, BF16_TOL, f"beyond capacity s_q={s_q}")


def test_graph_capture_replays_match_eager():
    """The plan and decode calls allocate nothing (given their buffers) and never wait on the
    host, so a whole step can be captured in a HIP graph. Every replay, with eager work on the
    same buffers between replays, must equal the eager step bit for bit."""
    w = wl.make_workload("graph", batch=6, s_q=1, heads=128, seqlens=[5000, 64, 700, 1, 2049, 3000], seed=33)
    d = Dev(w)
    W = 64
    plan_buf = torch.empty(mla.plan_bytes(w.batch, w.s_q, w.heads, W), dtype=torch.uint8, device="cuda")
    ws = torch.empty(max(16, mla.workspace_bytes(w.batch, w.s_q, w.heads, W)), dtype=torch.uint8, device="cuda")
    out = torch.empty(w.batch, w.s_q, w.heads, 512, dtype=torch.float32, device="cuda")
    lse = torch.empty(w.batch, w.s_q, w.heads, dtype=torch.float32, device="cuda")

    def step():
        plan = mla.get_split_plan(d.sl, w.s_q, w.heads, w.causal, W, out=plan_buf)
        mla.decode_fwd(d.q, d.kv, d.bt, d.sl, w.scale, kv_scales=d.scales, causal=w.causal, plan=plan,
                       workspace=ws, out=out, lse=lse)

    _say("graph capture")
    step()
    torch.cuda.synchronize()
    ref_out, ref_lse = out.clone(), lse.clone()
    ro, rl = _oracle_all(w)
    compare(ref_out.cpu().numpy(), ref_lse.cpu().numpy(), ro, rl, BF16_TOL, "graph eager step")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(4):
        out.zero_()
        lse.zero_()
        plan_buf.zero_()
        ws.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), f"replay {r} differs from the eager step"


# ----------------------------------------------------------------------------- full-size workloads

def _check_all_sequences(w):
    """Every output element of a full-size workload against the oracle (the oracle takes a few
    seconds per workload on the host cores)."""
    d = Dev(w)
    out, lse = d.run()
    ro, rl = _oracle_all(w)
    return compare(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, _tol(w), f"{w.name} seed {w.seed} all sequences")


@pytest.mark.parametrize("seed", [None, 2001])
def test_dsv3_full_size(seed):
    w = wl.make_config("dsv3", seed=seed)
    _say("dsv3 full size, seed", w.seed)
    _check_all_sequences(w)


@pytest.mark.parametrize("seed", [None, 2003])
def test_speculative_full_size(seed):
    w = wl.make_config("spec", seed=seed)
    _say("spec full size, seed", w.seed)
    _check_all_sequences(w)


@pytest.mark.parametrize("seed", [None, 2002])
def test_jagged_full_size(seed):
    w = wl.make_config("jagged", seed=seed)
    _say("jagged full size, seed", w.seed, "total tokens", int(w.seqlens.sum()))
    _check_all_sequences(w)


@pytest.mark.parametrize("heads,s_q", [(128, 32), (128, 64), (16, 32), (16, 64)])
def test_many_query_tokens_causal(heads, s_q):
    """s_q up to the ABI's 64 under the causal reading: with h = 128 a sequence has s_q tiles
    of one query token each, with h = 16 one tile holds 8 query tokens. Lengths below, at and
    above s_q, several pages, and enough workers to split the long items."""
    lens = [s_q - 5, s_q, s_q + 1, 300, 2100]
    w = wl.make_workload("many-q", batch=5, s_q=s_q, heads=heads, seqlens=lens, causal=True, seed=40 + heads + s_q)
    _say("many query tokens", heads, s_q)
    _check_full(w, num_workers=64, what=f"h={heads} s={s_q} causal")


# ----------------------------------------------------------------------------- split merge, plan reuse, device checks

@pytest.mark.parametrize("W", [8, 24, 96, 256])
def test_split_items_at_several_worker_counts(W):
    """One batch with a long sequence split over many workers beside short ones split a few
    ways or not at all, at worker counts that put the parts of an item on one XCD or on
    several (blocks are dealt to the XCDs round-robin); every output against the oracle."""
    w = wl.make_workload("splits", batch=6, s_q=1, heads=128, seqlens=[20000, 3000, 2500, 700, 64, 1], seed=41)
    d = Dev(w)
    ro, rl = _oracle_all(w)
    plan = d.plan(W)
    nsplits = plan.buffer.view(torch.int32).cpu().numpy()[16:16 + 8 * 6].reshape(6, 8)[:, 6]
    assert (nsplits > 1).any(), nsplits
    _say("split items, W", W, "parts", nsplits.tolist())
    o, l = d.run(plan=plan)
    compare(o.cpu().numpy(), l.cpu().numpy(), ro, rl, BF16_TOL, f"splits W={W}")


@pytest.mark.parametrize("W", [600, 4096])
def test_more_workers_than_compute_units(W):
    """A grid larger than the chip (several work-groups per CU over time, the planner's maximum of
    4,096 workers): long and short sequences cut into many small runs; every output."""
    w = wl.make_workload("wide-grid", batch=5, s_q=2, heads=64, seqlens=[30000, 9000, 700, 65, 2], causal=True,
                         seed=46)
    _say("workers", W)
    _check_full(w, num_workers=W, what=f"workers={W}")


def test_most_items():
    """The largest plan: 16,384 items (16,384 sequences of one 16-row tile), lengths 0..150 drawn
    per sequence, 256 workers; every output."""
    lens = np.random.default_rng(47).integers(0, 151, 16384)
    w = wl.make_workload("most-items", batch=16384, s_q=1, heads=16, seqlens=lens, seed=47)
    _say("most items")
    _check_full(w, num_workers=256, what="16384 items")


def test_widest_block_table():
    """max_pages = 65,535 (the largest block-table row): the table's row stride is taken from
    max_pages, not from the lengths."""
    w = wl.make_workload("wide-table", batch=3, s_q=1, heads=32, seqlens=[5000, 64, 700], seed=48,
                         max_pages=65535)
    assert w.block_table.shape == (3, 65535)
    _say("widest block table")
    _check_full(w, num_workers=32, what="max_pages=65535")


def test_plan_reused_across_calls():
    """One plan serves many calls (as one plan serves every layer of a decode step): five calls,
    outputs NaN before each, all bitwise equal and matching the oracle."""
    w = wl.make_workload("reuse", batch=8, s_q=1, heads=128, seqlens=[4096] * 6 + [900, 33], seed=42)
    d = Dev(w)
    plan = d.plan(256)
    ro, rl = _oracle_all(w)
    first = None
    for r in range(5):
        _say("plan reuse call", r)
        o, l = d.run(plan=plan)
        if first is None:
            first = (o, l)
            compare(o.cpu().numpy(), l.cpu().numpy(), ro, rl, BF16_TOL, "plan reuse")
        else:
            assert torch.equal(o, first[0]) and torch.equal(l, first[1]), f"call {r} differs"


def test_mismatched_plan_is_reported_and_writes_nothing(monkeypatch):
    """A plan built for 8 workers, in a buffer sized for 16, passed with num_workers = 16 (the
    binding checks the buffer size only): the decode and combine kernels check the plan header,
    write nothing (out and
    lse, carved from a guarded buffer, keep their NaN; the guard bytes around them keep their
    values), and set MLA_DEVICE_PLAN_MISMATCH. With MLA_VALIDATE=1 the call returns
    MLA_ERR_INVALID_ARG instead of MLA_OK."""
    w = wl.make_workload("mismatch", batch=3, s_q=1, heads=128, seqlens=[700, 64, 3000], seed=43)
    d = Dev(w)
    big = torch.zeros(mla.plan_bytes(w.batch, 1, 128, 16), dtype=torch.uint8, device="cuda")
    built = mla.get_split_plan(d.sl, 1, 128, False, 8, out=big)
    bad = mla.SplitPlan(built.buffer, built.batch, built.s_q, built.heads, built.causal, 16)
    good = d.plan(8)
    n_out, n_lse = w.batch * 128 * 512, w.batch * 128
    guard = 4096
    buf = torch.full((guard + n_out + guard + n_lse + guard,), 7.0, dtype=torch.float32, device="cuda")
    out = buf[guard:guard + n_out].view(w.batch, 1, 128, 512)
    lse = buf[2 * guard + n_out:2 * guard + n_out + n_lse].view(w.batch, 1, 128)
    out.fill_(float("nan"))
    lse.fill_(float("nan"))
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    _say("mismatched plan")
    mla.decode_fwd(d.q, d.kv, d.bt, d.sl, w.scale, plan=bad, out=out, lse=lse, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 1
    assert torch.isnan(out).all() and torch.isnan(lse).all()
    g = torch.cat([buf[:guard], buf[guard + n_out:2 * guard + n_out], buf[2 * guard + n_out + n_lse:]])
    assert (g == 7.0).all()
    monkeypatch.setenv("MLA_VALIDATE", "1")
    with pytest.raises(mla.MlaError) as ei:
        mla.decode_fwd(d.q, d.kv, d.bt, d.sl, w.scale, plan=bad, out=out, lse=lse)
    assert ei.value.status == 1 and "plan" in str(ei.value)
    # and a correct call passes validation
    o, l = mla.decode_fwd(d.q, d.kv, d.bt, d.sl, w.scale, plan=good)
    ro, rl = _oracle_all(w)
    compare(o.cpu().numpy(), l.cpu().numpy(), ro, rl, BF16_TOL, "validated call")


def test_validate_reports_out_of_range_pages(monkeypatch):
    """MLA_VALIDATE=1 turns a block-table entry outside the cache into MLA_ERR_INVALID_ARG."""
    w = wl.make_workload("oob-validate", batch=2, s_q=1, heads=32, seqlens=[192, 64], seed=44, poison=False)
    bad = w.block_table.copy()
    bad[1, 0] = -5
    d = Dev(wl.Workload(**{**w.__dict__, "block_table": bad}))
    monkeypatch.setenv("MLA_VALIDATE", "1")
    _say("validate oob")
    with pytest.raises(mla.MlaError) as ei:
        mla.decode_fwd(d.q, d.kv, d.bt, d.sl, w.scale, plan=d.plan(4))
    assert "outside [0, num_pages)" in str(ei.value)


def test_binding_rejects_wrong_shapes():
    """Every tensor of decode_fwd is checked before the C call (wrong shape, dtype or size ->
    ValueError; nothing is launched)."""
    w = wl.make_workload("shapes", batch=2, s_q=1, heads=16, seqlens=[100, 64], seed=45)
    d = Dev(w)
    plan = d.plan(4)
    ok = dict(q=d.q, kv_cache=d.kv, block_table=d.bt, seqlens=d.sl, softmax_scale=w.scale, plan=plan)
    cases = {
        "q last dim": dict(q=d.q[..., :512].contiguous()),
        "flattened cache": dict(kv_cache=d.kv.view(-1, 576)),
        "cache row width": dict(kv_cache=d.kv.view(-1, 32, 1152)),
        "bf16 with scales": dict(kv_scales=torch.ones(d.kv.shape[0], 64, 4, device="cuda")),
        "table rows": dict(block_table=d.bt[:1].contiguous()),
        "seqlens length": dict(seqlens=torch.cat([d.sl, d.sl])),
        "out shape": dict(out=torch.empty(2, 1, 16, 128, device="cuda")),
        "lse dtype": dict(lse=torch.empty(2, 1, 16, dtype=torch.float64, device="cuda")),
        "workspace size": dict(workspace=torch.empty(16, dtype=torch.uint8, device="cuda")),
        "status dtype": dict(status=torch.zeros(1, dtype=torch.int64, device="cuda")),
    }
    for name, kw in cases.items():
        with pytest.raises(ValueError):
            mla.decode_fwd(**{**ok, **kw})
        assert name
    mla.decode_fwd(**ok)
    torch.cuda.synchronize()


# ----------------------------------------------------------------------------- fp8 cache

@pytest.mark.parametrize("W", [1, 5, 256])
def test_fp8_ragged_any_worker_count(W):
    """fp8 cache (codes + per-128-channel scales + bf16 rope): lengths that end mid-page and
    mid-step, a one-token sequence, many pages; poisoned tails and spare pages."""
    w = wl.make_workload("fp8-ragged", batch=6, s_q=1, heads=128, seqlens=[1, 31, 63, 64, 65, 1000],
                         kv_dtype="fp8", seed=31)
    _say("fp8 ragged W", W)
    _check_full(w, num_workers=W, what=f"fp8 ragged W={W}")


@pytest.mark.parametrize("heads,s_q,causal", [(16, 1, False), (64, 4, True), (128, 16, True)])
def test_fp8_heads_and_query_tokens(heads, s_q, causal):
    w = wl.make_workload("fp8-heads", batch=3, s_q=s_q, heads=heads, seqlens=[s_q, 130, 517], kv_dtype="fp8",
                         causal=causal, seed=32 + heads + s_q)
    _say("fp8 heads", heads, "s_q", s_q, "causal", causal)
    _check_full(w, num_workers=11, what=f"fp8 h={heads} s={s_q} causal={causal}")


def test_fp8_empty_and_bitwise_repeat():
    w = wl.make_workload("fp8-empty", batch=3, s_q=2, heads=32, seqlens=[0, 1, 300], kv_dtype="fp8", causal=True,
                         seed=33)
    _say("fp8 empty + repeat")
    d = Dev(w)
    plan = d.plan(4)
    o1, l1 = d.run(plan=plan)
    o2, l2 = d.run(plan=plan)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    ro, rl = _oracle_all(w)
    compare(o1.cpu().numpy(), l1.cpu().numpy(), ro, rl, FP8_TOL, "fp8 empty")
    assert (o1[0] == 0).all()


@pytest.mark.parametrize("seed", [None, 2004])
def test_fp8_full_size(seed):
    """64 sequences of 32,768 tokens, fp8 cache; every output element."""
    w = wl.make_config("fp8", seed=seed)
    _say("fp8 full size, seed", w.seed)
    _check_all_sequences(w)
