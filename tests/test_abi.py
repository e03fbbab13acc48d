"""The C ABI library loads, exports every declared entry point, and rejects bad arguments on
the host before any HIP call (CPU only: no compute is launched). The library must have been
built (``__graft_entry__.build()``): a missing libmla.so fails these tests."""
import ctypes
import os
import re

import pytest
import torch

import mla_latent_space_amd as mla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "libmla.h")


def test_library_is_built():
    assert os.path.exists(mla.LIB_PATH), f"{mla.LIB_PATH} is missing: run __graft_entry__.build() first"


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert {"mla_get_split_plan", "mla_decode_fwd", "mla_plan_bytes", "mla_workspace_bytes", "mla_absorb_query",
            "mla_decompress_output", "mla_hybrid_merge", "mla_get_sparse_plan", "mla_sparse_decode_fwd",
            "mla_sparse_rows_bytes"} <= set(names)
    L = ctypes.CDLL(mla.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n


def test_version_and_status_strings():
    L = mla.lib()
    assert mla.abi_version() == 2
    assert L.mla_status_string(0) == b"MLA_OK"
    assert L.mla_status_string(3) == b"MLA_ERR_WORKSPACE_TOO_SMALL"
    assert L.mla_status_string(99) == b"unknown status"


def test_sizes():
    # 64 items (one 128-row tile each), 256 workers: header, items (8 words), workers (4),
    # split records (4 per item)
    n, W = 64, 256
    assert mla.plan_bytes(64, 1, 128, W) == 4 * (16 + 8 * n + 4 * W + 4 * n)
    assert mla.plan_bytes(32, 16, 128, W) == 4 * (16 + 12 * 32 * 16 + 4 * W)
    # per split part: 128 x 512 bf16 partial out + 128 fp32 lse
    assert mla.workspace_bytes(64, 1, 128, W) == 2 * (W - 1) * (128 * 512 * 2 + 128 * 8)
    assert mla.workspace_bytes(64, 1, 128, 1) == 0
    for bad in [(0, 1, 128, W), (4, 0, 128, W), (4, 1, 96, W), (4, 65, 128, W), (4, 1, 128, 0), (4, 1, 128, 5000),
                (20000, 1, 128, W), (2000, 16, 128, W)]:
        assert mla.plan_bytes(*bad) == 0, bad
        assert mla.workspace_bytes(*bad) == 0, bad


def _plan(L, seqlens, batch, s_q, h, causal, W, plan, nbytes):
    return L.mla_get_split_plan(seqlens, batch, s_q, h, causal, W, plan, nbytes, None)


def test_plan_rejects_bad_arguments_before_launch():
    L = mla.lib()
    fake = ctypes.c_void_p(0x100000)  # never dereferenced: every case fails validation first
    need = mla.plan_bytes(4, 1, 128, 8)
    assert _plan(L, None, 4, 1, 128, 0, 8, fake, need) == 1
    assert _plan(L, fake, 4, 1, 128, 0, 8, None, need) == 1
    assert _plan(L, fake, 4, 1, 128, 2, 8, fake, need) == 1
    assert _plan(L, fake, 4, 1, 100, 0, 8, fake, need) == 2
    assert _plan(L, fake, 4, 1, 128, 0, 8, fake, need - 4) == 3
    assert b"plan_bytes" in L.mla_last_error_message()
    assert _plan(L, fake, 4, 1, 128, 0, 8, ctypes.c_void_p(0x100004), need) == 1   # misaligned


def _decode(L, **kw):
    fake = ctypes.c_void_p(0x100000)
    a = dict(q=fake, kv=fake, scales=None, dtype=0, num_pages=10, bt=fake, max_pages=4, sl=fake, batch=2, s_q=1,
             h=128, scale=0.07, causal=0, plan=fake, W=8, ws=fake, ws_bytes=1 << 30, out=fake, lse=fake)
    a.update(kw)
    return L.mla_decode_fwd(a["q"], a["kv"], a["scales"], a["dtype"], a["num_pages"], a["bt"], a["max_pages"], a["sl"],
                            a["batch"], a["s_q"], a["h"], a["scale"], a["causal"], a["plan"], a["W"], a["ws"],
                            a["ws_bytes"], a["out"], a["lse"], a.get("status"), None)


def test_decode_rejects_bad_arguments_before_launch():
    L = mla.lib()
    fake = ctypes.c_void_p(0x100000)
    assert _decode(L, q=None) == 1
    assert _decode(L, lse=None) == 1
    assert _decode(L, dtype=7) == 1
    assert _decode(L, dtype=1) == 1                      # fp8 without scales
    assert _decode(L, scales=fake) == 1                  # bf16 with scales
    assert _decode(L, num_pages=0) == 1
    assert _decode(L, max_pages=0) == 1
    assert _decode(L, max_pages=70000) == 2
    assert _decode(L, scale=0.0) == 1
    assert _decode(L, scale=float("nan")) == 1
    assert _decode(L, h=48) == 2
    assert _decode(L, s_q=65) == 2
    assert _decode(L, causal=3) == 1
    assert _decode(L, ws_bytes=16) == 3
    assert _decode(L, ws=None) == 3
    assert _decode(L, out=ctypes.c_void_p(0x100008)) == 1  # misaligned
    assert b"16-byte aligned" in L.mla_last_error_message()
    assert _decode(L, status=ctypes.c_void_p(0x100002)) == 1   # a status word must be 4-byte aligned
    assert b"status" in L.mla_last_error_message()


def test_projections_reject_bad_arguments_before_launch():
    """Null pointers, empty shapes and misaligned buffers return a status before anything is
    enqueued (fake, never dereferenced device addresses; no GPU needed)."""
    L = mla.lib()
    fake = 1 << 20
    assert L.mla_absorb_query(None, fake, fake, 4, 16, fake, None) == 1
    assert L.mla_absorb_query(fake, fake, fake, 0, 16, fake, None) == 1
    assert L.mla_absorb_query(fake, fake, fake, 4, 0, fake, None) == 1
    assert L.mla_absorb_query(fake + 8, fake, fake, 4, 16, fake, None) == 1
    assert L.mla_decompress_output(fake, None, 4, 16, fake, None) == 1
    assert L.mla_decompress_output(fake, fake, -1, 16, fake, None) == 1
    assert L.mla_decompress_output(fake, fake, 4, 16, fake + 4, None) == 1
    assert b"16-byte aligned" in L.mla_last_error_message()


def test_hybrid_merge_rejects_bad_arguments_before_launch():
    """Status codes for the split latent + decompressed merge, returned before anything is
    enqueued (fake, never dereferenced device addresses; no GPU needed)."""
    L = mla.lib()
    f = 1 << 20

    def call(q_nope=f, k_new=f, n=64, out_old=f, batch=2, s_q=4, heads=16, scale=0.1, causal=0, out=f):
        return L.mla_hybrid_merge(q_nope, f, k_new, f, f, n, out_old, f, batch, s_q, heads, scale, causal, out, f,
                                  None)

    assert call(q_nope=None) == 1                       # null pointer
    assert call(k_new=None) == 1                        # new tokens required when n > 0
    assert call(n=-1) == 1
    assert call(batch=0) == 1 and call(heads=0) == 1 and call(s_q=0) == 1
    assert call(scale=0.0) == 1 and call(scale=float("inf")) == 1
    assert call(causal=2) == 1
    assert call(s_q=33) == 2                            # one 32-row tile of query rows
    assert call(batch=65536) == 2
    assert call(n=3, s_q=4, causal=1) == 2              # causal needs n >= s_q
    assert b"n_new >= s_q" in L.mla_last_error_message()
    assert call(n=70000, heads=128) == 2                # 31-bit offsets into the new tokens
    assert b"2^31" in L.mla_last_error_message()
    assert call(out=f + 4) == 1
    assert b"16-byte aligned" in L.mla_last_error_message()


def test_sparse_calls_reject_bad_arguments_before_launch():
    """Status codes and sizes of the token-sparse calls, returned before anything is enqueued
    (fake, never dereferenced device addresses; no GPU needed)."""
    L = mla.lib()
    f = 1 << 20
    assert L.mla_sparse_rows_bytes(2, 3, 40) == ((2 * 3 * 64 + 2 * 3) * 4 + 15) // 16 * 16
    assert L.mla_sparse_rows_bytes(0, 3, 40) == 0 and L.mla_sparse_rows_bytes(2, 3, 0) == 0

    def plan(indices=f, topk=64, max_pages=8, batch=2, s_q=1, heads=128, pages=100, W=8, rows_bytes=1 << 20,
             plan_bytes=1 << 20, rows=f):
        return L.mla_get_sparse_plan(indices, topk, f, max_pages, f, batch, s_q, heads, pages, W, rows, rows_bytes, f,
                                     plan_bytes, None, None)

    assert plan(indices=None) == 1
    assert plan(topk=0) == 1 and plan(batch=0) == 1 and plan(pages=0) == 1 and plan(max_pages=0) == 1
    assert plan(heads=64) == 2                          # one 128-row tile per query token
    assert plan(pages=60000) == 2                       # 31-bit row offsets
    assert b"num_pages" in L.mla_last_error_message()
    assert plan(rows_bytes=16) == 3 and plan(plan_bytes=16) == 3
    assert plan(rows=f + 4) == 1

    def dec(kv_dtype=1, q=f, scales=f, heads=128, scale=0.1, ws_bytes=1 << 30, out=f):
        return L.mla_sparse_decode_fwd(q, f, scales, kv_dtype, 100, 2, 1, heads, 64, scale, f, f, 8, f, ws_bytes, out,
                                       f, None, None)

    assert dec(kv_dtype=0) == 2                         # bf16 cache: not on this path
    assert dec(kv_dtype=7) == 1
    assert dec(q=None) == 1 and dec(scales=None) == 1
    assert dec(heads=16) == 2
    assert dec(scale=-1.0) == 1
    assert dec(ws_bytes=16) == 3
    assert dec(out=f + 8) == 1


# ----------------------------------------------------------------------------- Python binding
# The binding checks every tensor's shape, dtype and layout before it looks at devices, so these
# run on CPU tensors: each wrong argument raises ValueError naming the tensor and the fault, and a
# call whose shapes are all right stops at the device check (nothing is enqueued on CPU).


def _decode_inputs(batch=2, s_q=1, heads=16, pages=6, max_pages=4, W=4, fp8=False, causal=False):
    width = 640 if fp8 else 576
    kv = torch.zeros(pages, 64, width, dtype=torch.uint8 if fp8 else torch.bfloat16)
    ok = dict(q=torch.zeros(batch, s_q, heads, 576, dtype=torch.bfloat16), kv_cache=kv,
              block_table=torch.zeros(batch, max_pages, dtype=torch.int32),
              seqlens=torch.zeros(batch, dtype=torch.int32), softmax_scale=0.07, causal=causal,
              plan=mla.SplitPlan(torch.zeros(mla.plan_bytes(batch, s_q, heads, W), dtype=torch.uint8), batch, s_q,
                                 heads, causal, W))
    if fp8:
        ok["kv_scales"] = torch.ones(pages, 64, 4)
    return ok


def test_binding_rejects_wrong_decode_arguments():
    batch, s_q, heads, W = 2, 1, 16, 4
    ok = _decode_inputs(batch, s_q, heads, W=W)
    wide_q = torch.zeros(batch, s_q, heads, 1152, dtype=torch.bfloat16)
    cases = [
        (dict(q=ok["q"][..., :512]), r"q must be \[batch, s_q, heads, 576\]"),
        (dict(q=ok["q"][0]), r"q must be \[batch"),
        (dict(q=ok["q"].float()), "q must have dtype"),
        (dict(q=wide_q[..., :576]), "q must be contiguous"),
        (dict(kv_cache=ok["kv_cache"].view(-1, 576)), r"kv_cache must be \[pages, 64, 576\]"),
        (dict(kv_cache=ok["kv_cache"].view(-1, 32, 1152)), "kv_cache must have shape"),
        (dict(kv_cache=ok["kv_cache"].float()), "kv_cache must be bfloat16"),
        (dict(kv_scales=torch.ones(6, 64, 4)), "kv_scales must be None"),
        (dict(block_table=ok["block_table"][:1]), "block_table must have shape"),
        (dict(block_table=ok["block_table"].flatten()), r"block_table must be \[batch, max_pages\]"),
        (dict(block_table=ok["block_table"].long()), "block_table must have dtype"),
        (dict(seqlens=torch.zeros(batch + 1, dtype=torch.int32)), "seqlens must have shape"),
        (dict(seqlens=ok["seqlens"].long()), "seqlens must have dtype"),
        (dict(plan=mla.SplitPlan(ok["plan"].buffer, batch, s_q, 32, False, W)), "plan was built for different"),
        (dict(causal=True), "plan was built for different"),
        (dict(plan=mla.SplitPlan(ok["plan"].buffer[:64], batch, s_q, heads, False, W)), "plan buffer must be"),
        (dict(out=torch.zeros(batch, s_q, heads, 128)), "out must have shape"),
        (dict(out=torch.zeros(batch, s_q, heads, 512, dtype=torch.float64)), "out must have dtype"),
        (dict(lse=torch.zeros(batch, s_q, heads, 1)), "lse must have shape"),
        (dict(lse=torch.zeros(batch, s_q, heads, dtype=torch.float64)), "lse must have dtype"),
        (dict(workspace=torch.zeros(16, dtype=torch.uint8)), "workspace must be"),
        (dict(status=torch.zeros(1, dtype=torch.int64)), "status must be"),
        (dict(status=torch.zeros(0, dtype=torch.int32)), "status must be"),
    ]
    for kw, msg in cases:
        with pytest.raises(ValueError, match=msg):
            mla.decode_fwd(**{**ok, **kw})
    # the no-allocation entry point goes through the same checks (no workspace argument)
    for kw, msg in cases:
        if "workspace" not in kw:
            with pytest.raises(ValueError, match=msg):
                mla.decode_fwd_noalloc(**{**ok, **kw})
    # right shapes everywhere: the only fault left is that the tensors are not on a GPU
    with pytest.raises(ValueError, match="CUDA"):
        mla.decode_fwd(**ok)
    with pytest.raises(ValueError, match="CUDA"):
        mla.decode_fwd_noalloc(**ok)


def test_binding_rejects_wrong_fp8_decode_arguments():
    ok = _decode_inputs(fp8=True)
    cases = [
        (dict(kv_scales=None), "kv_scales float32 .* is required"),
        (dict(kv_scales=torch.ones(6, 64, 2)), "kv_scales must have shape"),
        (dict(kv_scales=torch.ones(5, 64, 4)), "kv_scales must have shape"),
        (dict(kv_scales=torch.ones(6, 64, 4, dtype=torch.float64)), "kv_scales must have dtype"),
        (dict(kv_cache=torch.zeros(6, 64, 576, dtype=torch.uint8)), "kv_cache must have shape"),
    ]
    for kw, msg in cases:
        with pytest.raises(ValueError, match=msg):
            mla.decode_fwd(**{**ok, **kw})
    with pytest.raises(ValueError, match="CUDA"):
        mla.decode_fwd(**ok)
    with pytest.raises(ValueError, match="CUDA"):
        mla.decode_fwd(**{**ok, "kv_cache": ok["kv_cache"].view(torch.float8_e4m3fn)})


def test_binding_rejects_wrong_plan_and_projection_arguments():
    with pytest.raises(ValueError, match=r"seqlens must be \[batch\]"):
        mla.get_split_plan(torch.zeros(2, 1, dtype=torch.int32), 1, 128)
    with pytest.raises(ValueError, match="seqlens must have dtype"):
        mla.get_split_plan(torch.zeros(2, dtype=torch.int64), 1, 128)
    with pytest.raises(ValueError, match="CUDA"):
        mla.get_split_plan(torch.zeros(2, dtype=torch.int32), 1, 128, num_workers=8)

    b, s, h = 2, 3, 16
    qn = torch.zeros(b, s, h, 128, dtype=torch.bfloat16)
    qr = torch.zeros(b, s, h, 64, dtype=torch.bfloat16)
    wk = torch.zeros(h, 512, 128, dtype=torch.bfloat16)
    for args, msg in [((qn, qr[..., :32], wk), "q_rope must have shape"),
                      ((qn, qr, wk.transpose(1, 2)), "w_k must have shape"),
                      ((qn, qr, torch.zeros(h, 512, 128)), "w_k must have dtype"),
                      ((qn[0, 0, 0], qr, wk), r"q_nope must be \[\.\.\., heads, 128\]"),
                      ((qn, qr, wk, torch.zeros(b, s, h, 576)), "out must have dtype"),
                      ((qn, qr, wk), "CUDA")]:
        with pytest.raises(ValueError, match=msg):
            mla.absorb_query(*args)
    ol = torch.zeros(b, s, h, 512)
    wv = torch.zeros(h, 128, 512, dtype=torch.bfloat16)
    for args, msg in [((ol.bfloat16(), wv), "out_latent must have dtype"),
                      ((ol, wv[:, :64]), "w_v must have shape"),
                      ((ol, wv, torch.zeros(b, s, h, 512)), "out must have shape"),
                      ((ol, wv), "CUDA")]:
        with pytest.raises(ValueError, match=msg):
            mla.decompress_output(*args)


def test_binding_rejects_wrong_hybrid_and_sparse_arguments():
    b, s, h, n = 2, 3, 16, 40
    qn = torch.zeros(b, s, h, 128, dtype=torch.bfloat16)
    qr = torch.zeros(b, s, h, 64, dtype=torch.bfloat16)
    kn = torch.zeros(b, n, h, 128, dtype=torch.bfloat16)
    krn = torch.zeros(b, n, 64, dtype=torch.bfloat16)
    oo = torch.zeros(b, s, h, 128)
    lo = torch.zeros(b, s, h)
    ok = dict(q_nope=qn, q_rope=qr, k_new=kn, kr_new=krn, v_new=kn.clone(), out_old=oo, lse_old=lo,
              softmax_scale=0.1)
    for kw, msg in [(dict(kr_new=torch.zeros(b, n, h, 64, dtype=torch.bfloat16)), "kr_new must have shape"),
                    (dict(v_new=kn[:, :-1]), "v_new must have shape"),
                    (dict(k_new=kn[0]), r"k_new must be \[batch, n_new, heads, 128\]"),
                    (dict(lse_old=lo.double()), "lse_old must have dtype"),
                    (dict(out_old=oo[:1]), "out_old must have shape"),
                    (dict(out=torch.zeros(b, s, h, 512)), "out must have shape"),
                    (dict(q_nope=qn[0]), r"q_nope must be \[batch"),
                    (dict(), "CUDA"),
                    (dict(k_new=None, kr_new=None, v_new=None), "CUDA")]:
        with pytest.raises(ValueError, match=msg):
            mla.hybrid_merge(**{**ok, **kw})

    idx = torch.zeros(b, 1, 64, dtype=torch.int32)
    bt = torch.zeros(b, 4, dtype=torch.int32)
    sl = torch.zeros(b, dtype=torch.int32)
    for args, msg in [((idx[0], bt, sl, 10), r"indices must be \[batch, s_q, topk\]"),
                      ((idx.long(), bt, sl, 10), "indices must have dtype"),
                      ((idx, bt[:1], sl, 10), "block_table must have shape"),
                      ((idx, bt, sl[:1], 10), "seqlens must have shape"),
                      ((idx, bt, sl, 10), "CUDA")]:
        with pytest.raises(ValueError, match=msg):
            mla.get_sparse_plan(*args, num_workers=8)

    pages, W = 10, 8
    plan = mla.SparsePlan(torch.zeros(64, dtype=torch.uint8), torch.zeros(64, dtype=torch.uint8), b, 1, 128, 64,
                          pages, W)
    q = torch.zeros(b, 1, 128, 576, dtype=torch.bfloat16)
    kv = torch.zeros(pages, 64, 640, dtype=torch.uint8)
    sc = torch.ones(pages, 64, 4)
    for kw, msg in [(dict(kv_scales=sc[:, :, :2]), "kv_scales must have shape"),
                    (dict(kv_scales=sc[:5]), "kv_scales must have shape"),
                    (dict(kv_cache=kv[:5]), "kv_cache .* must have shape"),
                    (dict(kv_cache=torch.zeros(pages, 64, 576, dtype=torch.bfloat16)), "kv_cache .* must have shape"),
                    (dict(q=q[:, :, :64]), "q must have shape"),
                    (dict(workspace=torch.zeros(16, dtype=torch.uint8)), "workspace must be"),
                    (dict(lse=torch.zeros(b, 1, 128, dtype=torch.float16)), "lse must have dtype"),
                    (dict(), "CUDA")]:
        with pytest.raises(ValueError, match=msg):
            mla.sparse_decode_fwd(**{**dict(q=q, kv_cache=kv, kv_scales=sc, softmax_scale=0.1, plan=plan), **kw})
