"""The C ABI library loads, exports every declared entry point, and rejects bad arguments on
the host before any HIP call (CPU only: no compute is launched). The library must have been
built (``__graft_entry__.build()``): a missing libmla.so fails these tests."""
import ctypes
import os
import re

import pytest

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
