"""mla_decode_fwd_noalloc (the split partials in the library's own device scratch) against
mla_decode_fwd with a caller workspace, through the C ABI: two calls in a row on one GPU, the
second with a smaller input (fewer sequences, shorter lengths, other split shapes), each
bitwise equal to the workspace call with the same plan, and within the bf16 bounds of the
fp64 oracle."""
import ctypes

import numpy as np
import pytest
import torch

import mla_latent_space_amd as mla
from mla_latent_space_amd import workloads as wl
from oracle import mla as om

from gpu_common import BF16_TOL, Dev, compare

pytestmark = pytest.mark.gpu


def _noalloc(d, plan, out, lse, status):
    w = d.w
    return mla.lib().mla_decode_fwd_noalloc(
        d.q.data_ptr(), d.kv.data_ptr(), None, mla.KV_BF16, int(d.kv.shape[0]), d.bt.data_ptr(), int(d.bt.shape[1]),
        d.sl.data_ptr(), w.batch, w.s_q, w.heads, ctypes.c_float(w.scale), int(w.causal), plan.buffer.data_ptr(),
        plan.num_workers, out.data_ptr(), lse.data_ptr(), status.data_ptr(),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


@pytest.mark.parametrize("first,second", [
    (dict(batch=12, s_q=1, heads=128, seqlens=[4096] * 8 + [3000, 700, 64, 1], W=256),
     dict(batch=3, s_q=2, heads=64, seqlens=[900, 40, 2], causal=True, W=40)),
])
def test_noalloc_matches_workspace_call(first, second):
    for n, cfg in enumerate((first, second)):
        cfg = dict(cfg)
        W = cfg.pop("W")
        w = wl.make_workload(f"noalloc{n}", seed=60 + n, **cfg)
        print("noalloc call", n, "batch", w.batch, "W", W, flush=True)
        d = Dev(w)
        plan = d.plan(W)
        ref_out, ref_lse = d.run(plan=plan)
        out = torch.full_like(ref_out, float("nan"))
        lse = torch.full_like(ref_lse, float("nan"))
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        rc = _noalloc(d, plan, out, lse, status)
        assert rc == 0, mla.lib().mla_last_error_message()
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), f"call {n} differs from the workspace call"
        ro, rl = om.decode_latent(w.q, w.kv, None, "bf16", w.block_table, w.seqlens, w.scale, w.causal)
        compare(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, BF16_TOL, f"noalloc call {n}")


def test_noalloc_rejects_a_shape_beyond_its_scratch():
    """More than 286 workers needs more split scratch than the library holds: refused before
    anything is enqueued, with the reason."""
    f = ctypes.c_void_p(1 << 20)
    rc = mla.lib().mla_decode_fwd_noalloc(f, f, None, 0, 10, f, 4, f, 64, 1, 128, ctypes.c_float(0.07), 0, f, 400,
                                          f, f, None, None)
    assert rc == 3 and b"scratch" in mla.lib().mla_last_error_message()
