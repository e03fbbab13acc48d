"""mla_latent_space_amd: latent-space MLA decode on MI355X (gfx950).

Thin ctypes binding over the C ABI in ``include/libmla.h`` (``libmla.so`` in this
package directory). The binding only marshals arguments: every step of the decode
runs in the HIP kernels of the library; PyTorch provides device memory and streams.
If ``libmla.so`` is missing, every call raises -- there is no fallback path.

    plan = get_split_plan(seqlens, s_q, heads, causal=False)
    out, lse = decode_fwd(q, kv_cache, block_table, seqlens, softmax_scale, plan=plan)
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional, Tuple

import torch

__all__ = ["MlaError", "SplitPlan", "lib", "abi_version", "default_num_workers", "plan_bytes", "workspace_bytes",
           "absorb_query", "decompress_output",
           "get_split_plan", "decode_fwd", "decode_fwd_noalloc", "NOALLOC_SCRATCH_BYTES", "LIB_PATH", "KV_BF16", "KV_FP8_E4M3", "hybrid_merge", "SparsePlan", "get_sparse_plan", "sparse_decode_fwd"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmla.so")
KV_BF16 = 0
KV_FP8_E4M3 = 1
NOALLOC_SCRATCH_BYTES = 72 << 20   # MLA_NOALLOC_SCRATCH_BYTES in include/libmla.h
_STATUS = {0: "MLA_OK", 1: "MLA_ERR_INVALID_ARG", 2: "MLA_ERR_UNSUPPORTED", 3: "MLA_ERR_WORKSPACE_TOO_SMALL",
           4: "MLA_ERR_HIP", 5: "MLA_ERR_INTERNAL"}

_lib = None


class MlaError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        super().__init__(f"{_STATUS.get(status, status)}: {message}")


def lib() -> ctypes.CDLL:
    """The loaded libmla.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m mla_latent_space_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    c_i32, c_i64, c_sz, c_p, c_f = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float
    L.mla_abi_version.restype = c_i32
    L.mla_abi_version.argtypes = []
    L.mla_status_string.restype = ctypes.c_char_p
    L.mla_status_string.argtypes = [c_i32]
    L.mla_last_error_message.restype = ctypes.c_char_p
    L.mla_last_error_message.argtypes = []
    L.mla_default_num_workers.restype = c_i32
    L.mla_default_num_workers.argtypes = [c_i32]
    L.mla_plan_bytes.restype = c_sz
    L.mla_plan_bytes.argtypes = [c_i32, c_i32, c_i32, c_i32]
    L.mla_workspace_bytes.restype = c_sz
    L.mla_workspace_bytes.argtypes = [c_i32, c_i32, c_i32, c_i32]
    L.mla_get_split_plan.restype = c_i32
    L.mla_get_split_plan.argtypes = [c_p, c_i32, c_i32, c_i32, c_i32, c_i32, c_p, c_sz, c_p]
    L.mla_decode_fwd.restype = c_i32
    L.mla_decode_fwd.argtypes = [c_p, c_p, c_p, c_i32, c_i64, c_p, c_i32, c_p, c_i32, c_i32, c_i32, c_f, c_i32,
                                 c_p, c_i32, c_p, c_sz, c_p, c_p, c_p, c_p]
    L.mla_decode_fwd_noalloc.restype = c_i32
    L.mla_decode_fwd_noalloc.argtypes = [c_p, c_p, c_p, c_i32, c_i64, c_p, c_i32, c_p, c_i32, c_i32, c_i32, c_f,
                                         c_i32, c_p, c_i32, c_p, c_p, c_p, c_p]
    L.mla_absorb_query.restype = c_i32
    L.mla_absorb_query.argtypes = [c_p, c_p, c_p, c_i32, c_i32, c_p, c_p]
    L.mla_decompress_output.restype = c_i32
    L.mla_decompress_output.argtypes = [c_p, c_p, c_i32, c_i32, c_p, c_p]
    L.mla_sparse_rows_bytes.restype = c_sz
    L.mla_sparse_rows_bytes.argtypes = [c_i32, c_i32, c_i32]
    L.mla_get_sparse_plan.restype = c_i32
    L.mla_get_sparse_plan.argtypes = [c_p, c_i32, c_p, c_i32, c_p, c_i32, c_i32, c_i32, c_i64, c_i32, c_p, c_sz,
                                      c_p, c_sz, c_p, c_p]
    L.mla_sparse_decode_fwd.restype = c_i32
    L.mla_sparse_decode_fwd.argtypes = [c_p, c_p, c_p, c_i32, c_i64, c_i32, c_i32, c_i32, c_i32, c_f, c_p, c_p,
                                        c_i32, c_p, c_sz, c_p, c_p, c_p, c_p]
    L.mla_hybrid_merge.restype = c_i32
    L.mla_hybrid_merge.argtypes = [c_p, c_p, c_p, c_p, c_p, c_i32, c_p, c_p, c_i32, c_i32, c_i32, c_f, c_i32, c_p,
                                   c_p, c_p]
    _lib = L
    return L


def _check(status: int):
    if status != 0:
        raise MlaError(status, lib().mla_last_error_message().decode())


def abi_version() -> int:
    return int(lib().mla_abi_version())


def default_num_workers(device: Optional[int] = None) -> int:
    dev = torch.cuda.current_device() if device is None else int(device)
    n = int(lib().mla_default_num_workers(dev))
    if n < 0:
        raise MlaError(4, lib().mla_last_error_message().decode())
    return n


def plan_bytes(batch: int, s_q: int, heads: int, num_workers: int) -> int:
    return int(lib().mla_plan_bytes(batch, s_q, heads, num_workers))


def workspace_bytes(batch: int, s_q: int, heads: int, num_workers: int) -> int:
    return int(lib().mla_workspace_bytes(batch, s_q, heads, num_workers))


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


@dataclasses.dataclass
class SplitPlan:
    """Device plan buffer plus the arguments it was built for."""
    buffer: torch.Tensor
    batch: int
    s_q: int
    heads: int
    causal: bool
    num_workers: int


def get_split_plan(seqlens: torch.Tensor, s_q: int, heads: int, causal: bool = False,
                   num_workers: Optional[int] = None, out: Optional[torch.Tensor] = None) -> SplitPlan:
    """Enqueue the split-KV planner on the current stream (see mla_get_split_plan). `out`, a
    contiguous uint8 CUDA tensor of at least plan_bytes(...) bytes, is written in place of a
    new buffer (no allocation: usable under graph capture)."""
    if not isinstance(seqlens, torch.Tensor) or seqlens.dim() != 1:
        raise ValueError("seqlens must be [batch]")
    batch = seqlens.numel()
    _need(seqlens, "seqlens", torch.int32, (batch,))
    _same_device(seqlens.device, out=out)
    W = default_num_workers(seqlens.device.index) if num_workers is None else int(num_workers)
    nbytes = plan_bytes(batch, s_q, heads, W)
    if nbytes == 0:
        _check(int(lib().mla_get_split_plan(None, batch, s_q, heads, int(causal), W, None, 0, None)))
    if out is not None:
        _need_bytes(out, "out", nbytes)
        buf = out
    else:
        buf = torch.empty(nbytes, dtype=torch.uint8, device=seqlens.device)
    _check(int(lib().mla_get_split_plan(seqlens.data_ptr(), batch, s_q, heads, int(causal), W, buf.data_ptr(),
                                        nbytes, _stream(seqlens))))
    return SplitPlan(buf, batch, s_q, heads, bool(causal), W)


# Argument checks run in two passes: first the shape, dtype and layout of every tensor (_need,
# _need_bytes), then that every tensor sits on the one CUDA device the call is enqueued on
# (_same_device). A wrong shape is therefore reported as such on any device.

def _need(t, name: str, dtype, shape):
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    dtypes = dtype if isinstance(dtype, tuple) else (dtype,)
    if t.dtype not in dtypes:
        raise ValueError(f"{name} must have dtype {' or '.join(str(d) for d in dtypes)}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _need_bytes(t, name: str, nbytes: int):
    if not isinstance(t, torch.Tensor) or not t.is_contiguous() or t.numel() * t.element_size() < nbytes:
        raise ValueError(f"{name} must be a contiguous tensor of at least {nbytes} bytes")


def _need_status(status):
    if status is not None and (not isinstance(status, torch.Tensor) or status.dtype != torch.int32
                               or status.numel() < 1):
        raise ValueError("status must be an int32 tensor (its first element is the status word)")


def _same_device(device, **tensors):
    if device.type != "cuda":
        raise ValueError(f"the call's tensors must be CUDA tensors, got {device}")
    for name, t in tensors.items():
        if t is not None and t.device != device:
            raise ValueError(f"{name} must be a CUDA tensor on {device}, got {t.device}")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _decode_args(q, kv_cache, block_table, seqlens, kv_scales, causal, plan, out, lse, status, workspace,
                 with_workspace):
    """Checks every tensor of a decode call; allocates the plan, out and lse not given and, if
    `with_workspace`, the workspace. Returns (kv_dtype, plan, out, lse, workspace)."""
    if not isinstance(q, torch.Tensor) or q.dim() != 4 or q.shape[-1] != 576:
        raise ValueError("q must be [batch, s_q, heads, 576]")
    batch, s_q, heads, _ = (int(x) for x in q.shape)
    dev = q.device
    _need(q, "q", torch.bfloat16, (batch, s_q, heads, 576))
    if not isinstance(kv_cache, torch.Tensor) or kv_cache.dim() != 3:
        raise ValueError("kv_cache must be [pages, 64, 576] (bf16) or [pages, 64, 640] (fp8 layout)")
    pages = int(kv_cache.shape[0])
    if kv_cache.dtype == torch.bfloat16:
        kv_dtype = KV_BF16
        _need(kv_cache, "kv_cache", torch.bfloat16, (pages, 64, 576))
        if kv_scales is not None:
            raise ValueError("kv_scales must be None for a bf16 cache")
    elif kv_cache.dtype in (torch.uint8, torch.float8_e4m3fn):
        kv_dtype = KV_FP8_E4M3
        _need(kv_cache, "kv_cache", (torch.uint8, torch.float8_e4m3fn), (pages, 64, 640))
        if kv_scales is None:
            raise ValueError("kv_scales float32 [pages, 64, 4] is required for the fp8 layout")
        _need(kv_scales, "kv_scales", torch.float32, (pages, 64, 4))
    else:
        raise ValueError("kv_cache must be bfloat16, or uint8/float8_e4m3fn for the fp8 layout")
    if not isinstance(block_table, torch.Tensor) or block_table.dim() != 2:
        raise ValueError("block_table must be [batch, max_pages]")
    _need(block_table, "block_table", torch.int32, (batch, int(block_table.shape[1])))
    _need(seqlens, "seqlens", torch.int32, (batch,))
    if plan is not None:
        if (plan.batch, plan.s_q, plan.heads, plan.causal) != (batch, s_q, heads, bool(causal)):
            raise ValueError("plan was built for different arguments")
        _need_bytes(plan.buffer, "plan buffer", plan_bytes(batch, s_q, heads, plan.num_workers))
    if out is not None:
        _need(out, "out", torch.float32, (batch, s_q, heads, 512))
    if lse is not None:
        _need(lse, "lse", torch.float32, (batch, s_q, heads))
    _need_status(status)
    if workspace is not None and plan is not None:
        _need_bytes(workspace, "workspace", workspace_bytes(batch, s_q, heads, plan.num_workers))
    _same_device(dev, kv_cache=kv_cache, kv_scales=kv_scales, block_table=block_table, seqlens=seqlens,
                 plan_buffer=None if plan is None else plan.buffer, out=out, lse=lse, status=status,
                 workspace=workspace)
    if plan is None:
        plan = get_split_plan(seqlens, s_q, heads, causal)
    if with_workspace:
        need = workspace_bytes(batch, s_q, heads, plan.num_workers)
        if workspace is None and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        if workspace is not None:
            _need_bytes(workspace, "workspace", need)
    if out is None:
        out = torch.empty(batch, s_q, heads, 512, dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty(batch, s_q, heads, dtype=torch.float32, device=dev)
    return kv_dtype, plan, out, lse, workspace


def decode_fwd(q: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor, seqlens: torch.Tensor,
               softmax_scale: float, kv_scales: Optional[torch.Tensor] = None, causal: bool = False,
               plan: Optional[SplitPlan] = None, workspace: Optional[torch.Tensor] = None,
               out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
               status: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Latent-space MLA decode (see mla_decode_fwd). q: bf16 [b, s, h, 576]; kv_cache: bf16
    [pages, 64, 576] or uint8 [pages, 64, 640] with kv_scales float32 [pages, 64, 4];
    block_table int32 [b, max_pages]; seqlens int32 [b]. Returns out float32 [b, s, h, 512]
    and lse float32 [b, s, h]. `status`, an int32 CUDA tensor, receives the device-side
    MLA_DEVICE_* bits in its first element (OR-ed, never cleared)."""
    kv_dtype, plan, out, lse, workspace = _decode_args(q, kv_cache, block_table, seqlens, kv_scales, causal, plan,
                                                       out, lse, status, workspace, True)
    batch, s_q, heads = plan.batch, plan.s_q, plan.heads
    W = plan.num_workers
    rc = lib().mla_decode_fwd(
        q.data_ptr(), kv_cache.data_ptr(), None if kv_scales is None else kv_scales.data_ptr(), kv_dtype,
        int(kv_cache.shape[0]), block_table.data_ptr(), int(block_table.shape[1]), seqlens.data_ptr(), batch, s_q,
        heads, float(softmax_scale), int(causal), plan.buffer.data_ptr(), W,
        None if workspace is None else workspace.data_ptr(),
        0 if workspace is None else workspace.numel() * workspace.element_size(),
        out.data_ptr(), lse.data_ptr(), _ptr(status), _stream(q))
    _check(int(rc))
    return out, lse


def decode_fwd_noalloc(q: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor, seqlens: torch.Tensor,
                       softmax_scale: float, kv_scales: Optional[torch.Tensor] = None, causal: bool = False,
                       plan: Optional[SplitPlan] = None, out: Optional[torch.Tensor] = None,
                       lse: Optional[torch.Tensor] = None,
                       status: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """decode_fwd with the split partials in the library's own scratch (see
    mla_decode_fwd_noalloc): no workspace argument, nothing allocated by the library. Pass
    `plan`, `out` and `lse` to allocate nothing here either."""
    kv_dtype, plan, out, lse, _ = _decode_args(q, kv_cache, block_table, seqlens, kv_scales, causal, plan, out, lse,
                                               status, None, False)
    rc = lib().mla_decode_fwd_noalloc(
        q.data_ptr(), kv_cache.data_ptr(), None if kv_scales is None else kv_scales.data_ptr(), kv_dtype,
        int(kv_cache.shape[0]), block_table.data_ptr(), int(block_table.shape[1]), seqlens.data_ptr(), plan.batch,
        plan.s_q, plan.heads, float(softmax_scale), int(causal), plan.buffer.data_ptr(), plan.num_workers,
        out.data_ptr(), lse.data_ptr(), _ptr(status), _stream(q))
    _check(int(rc))
    return out, lse


def absorb_query(q_nope: torch.Tensor, q_rope: torch.Tensor, w_k: torch.Tensor,
                 out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Qz = [q_nope W_k^T | q_rope] per head (see mla_absorb_query). q_nope bf16 [..., h, 128],
    q_rope bf16 [..., h, 64], w_k bf16 [h, 512, 128]; returns bf16 [..., h, 576]."""
    if not isinstance(q_nope, torch.Tensor) or q_nope.dim() < 2:
        raise ValueError("q_nope must be [..., heads, 128]")
    lead = tuple(q_nope.shape[:-2])
    heads = q_nope.shape[-2]
    tokens = 1
    for x in lead:
        tokens *= int(x)
    _need(q_nope, "q_nope", torch.bfloat16, lead + (heads, 128))
    _need(q_rope, "q_rope", torch.bfloat16, lead + (heads, 64))
    _need(w_k, "w_k", torch.bfloat16, (heads, 512, 128))
    if out is not None:
        _need(out, "out", torch.bfloat16, lead + (heads, 576))
    _same_device(q_nope.device, q_rope=q_rope, w_k=w_k, out=out)
    if out is None:
        out = torch.empty(lead + (heads, 576), dtype=torch.bfloat16, device=q_nope.device)
    _check(int(lib().mla_absorb_query(q_nope.data_ptr(), q_rope.data_ptr(), w_k.data_ptr(), tokens, heads,
                                      out.data_ptr(), _stream(q_nope))))
    return out


def decompress_output(out_latent: torch.Tensor, w_v: torch.Tensor,
                      out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out = O_latent W_v^T per head (see mla_decompress_output). out_latent float32
    [..., h, 512], w_v bf16 [h, 128, 512]; returns float32 [..., h, 128]."""
    if not isinstance(out_latent, torch.Tensor) or out_latent.dim() < 2:
        raise ValueError("out_latent must be [..., heads, 512]")
    lead = tuple(out_latent.shape[:-2])
    heads = out_latent.shape[-2]
    tokens = 1
    for x in lead:
        tokens *= int(x)
    _need(out_latent, "out_latent", torch.float32, lead + (heads, 512))
    _need(w_v, "w_v", torch.bfloat16, (heads, 128, 512))
    if out is not None:
        _need(out, "out", torch.float32, lead + (heads, 128))
    _same_device(out_latent.device, w_v=w_v, out=out)
    if out is None:
        out = torch.empty(lead + (heads, 128), dtype=torch.float32, device=out_latent.device)
    _check(int(lib().mla_decompress_output(out_latent.data_ptr(), w_v.data_ptr(), tokens, heads, out.data_ptr(),
                                           _stream(out_latent))))
    return out


def hybrid_merge(q_nope: torch.Tensor, q_rope: torch.Tensor, k_new: Optional[torch.Tensor],
                 kr_new: Optional[torch.Tensor], v_new: Optional[torch.Tensor], out_old: torch.Tensor,
                 lse_old: torch.Tensor, softmax_scale: float, causal: bool = False,
                 out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None):
    """The new tokens' attention merged with the old part (see mla_hybrid_merge). q_nope bf16
    [b, s, h, 128], q_rope bf16 [b, s, h, 64]; k_new, v_new bf16 [b, n, h, 128] and kr_new bf16
    [b, n, 64] (None with n = 0); out_old float32 [b, s, h, 128], lse_old float32 [b, s, h].
    Returns (out float32 [b, s, h, 128], lse float32 [b, s, h])."""
    if not isinstance(q_nope, torch.Tensor) or q_nope.dim() != 4:
        raise ValueError("q_nope must be [batch, s_q, heads, 128]")
    b, s_q, heads = int(q_nope.shape[0]), int(q_nope.shape[1]), int(q_nope.shape[2])
    _need(q_nope, "q_nope", torch.bfloat16, (b, s_q, heads, 128))
    _need(q_rope, "q_rope", torch.bfloat16, (b, s_q, heads, 64))
    if k_new is not None and (not isinstance(k_new, torch.Tensor) or k_new.dim() != 4):
        raise ValueError("k_new must be [batch, n_new, heads, 128]")
    n = 0 if k_new is None else int(k_new.shape[1])
    if n > 0:
        _need(k_new, "k_new", torch.bfloat16, (b, n, heads, 128))
        _need(kr_new, "kr_new", torch.bfloat16, (b, n, 64))
        _need(v_new, "v_new", torch.bfloat16, (b, n, heads, 128))
    _need(out_old, "out_old", torch.float32, (b, s_q, heads, 128))
    _need(lse_old, "lse_old", torch.float32, (b, s_q, heads))
    if out is not None:
        _need(out, "out", torch.float32, (b, s_q, heads, 128))
    if lse is not None:
        _need(lse, "lse", torch.float32, (b, s_q, heads))
    new = (lambda t: t if n > 0 else None)
    _same_device(q_nope.device, q_rope=q_rope, k_new=new(k_new), kr_new=new(kr_new), v_new=new(v_new),
                 out_old=out_old, lse_old=lse_old, out=out, lse=lse)
    if out is None:
        out = torch.empty((b, s_q, heads, 128), dtype=torch.float32, device=q_nope.device)
    if lse is None:
        lse = torch.empty((b, s_q, heads), dtype=torch.float32, device=q_nope.device)
    ptr = (lambda t: t.data_ptr() if t is not None and n > 0 else None)
    _check(int(lib().mla_hybrid_merge(q_nope.data_ptr(), q_rope.data_ptr(), ptr(k_new), ptr(kr_new), ptr(v_new), n,
                                      out_old.data_ptr(), lse_old.data_ptr(), b, s_q, heads, float(softmax_scale),
                                      1 if causal else 0, out.data_ptr(), lse.data_ptr(), _stream(q_nope))))
    return out, lse


class SparsePlan:
    """Cache-row lists and split plan of a token-sparse decode (see mla_get_sparse_plan)."""

    def __init__(self, rows, plan, batch, s_q, heads, topk, num_pages, num_workers):
        self.rows, self.plan = rows, plan
        self.batch, self.s_q, self.heads, self.topk = batch, s_q, heads, topk
        self.num_pages, self.num_workers = num_pages, num_workers


def get_sparse_plan(indices: torch.Tensor, block_table: torch.Tensor, seqlens: torch.Tensor, num_pages: int,
                    heads: int = 128, num_workers: Optional[int] = None,
                    status: Optional[torch.Tensor] = None) -> SparsePlan:
    """indices int32 [b, s, topk] (logical token positions; entries outside [0, t) are padding),
    block_table int32 [b, max_pages], seqlens int32 [b]."""
    if not isinstance(indices, torch.Tensor) or indices.dim() != 3:
        raise ValueError("indices must be [batch, s_q, topk]")
    b, s_q, topk = (int(x) for x in indices.shape)
    dev = indices.device
    _need(indices, "indices", torch.int32, (b, s_q, topk))
    if not isinstance(block_table, torch.Tensor) or block_table.dim() != 2:
        raise ValueError("block_table must be [batch, max_pages]")
    _need(block_table, "block_table", torch.int32, (b, int(block_table.shape[1])))
    _need(seqlens, "seqlens", torch.int32, (b,))
    _need_status(status)
    _same_device(dev, block_table=block_table, seqlens=seqlens, status=status)
    W = default_num_workers(indices.device.index or 0) if num_workers is None else int(num_workers)
    rb = int(lib().mla_sparse_rows_bytes(b, s_q, topk))
    pb = plan_bytes(b * s_q, 1, heads, W)
    if rb == 0 or pb == 0:
        raise MlaError(2, f"unsupported sparse shape b={b} s_q={s_q} topk={topk} heads={heads}")
    rows = torch.empty(rb, dtype=torch.uint8, device=indices.device)
    plan = torch.empty(pb, dtype=torch.uint8, device=indices.device)
    _check(int(lib().mla_get_sparse_plan(indices.data_ptr(), topk, block_table.data_ptr(), int(block_table.shape[1]),
                                         seqlens.data_ptr(), b, s_q, heads, int(num_pages), W, rows.data_ptr(), rb,
                                         plan.data_ptr(), pb, _ptr(status), _stream(indices))))
    return SparsePlan(rows, plan, b, s_q, heads, topk, int(num_pages), W)


def sparse_decode_fwd(q: torch.Tensor, kv_cache: torch.Tensor, kv_scales: torch.Tensor, softmax_scale: float,
                      plan: SparsePlan, workspace: Optional[torch.Tensor] = None,
                      out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                      status: Optional[torch.Tensor] = None):
    """Token-sparse decode over an fp8 cache (see mla_sparse_decode_fwd). q bf16 [b, s, 128, 576];
    kv_cache uint8 [pages, 64, 640]; kv_scales float32 [pages, 64, 4]. Returns out float32
    [b, s, 128, 512] and lse float32 [b, s, 128]."""
    b, s_q, heads = plan.batch, plan.s_q, plan.heads
    dev = q.device
    _need(q, "q", torch.bfloat16, (b, s_q, heads, 576))
    _need(kv_cache, "kv_cache (the fp8 layout the plan was built for)", (torch.uint8, torch.float8_e4m3fn),
          (plan.num_pages, 64, 640))
    _need(kv_scales, "kv_scales", torch.float32, (plan.num_pages, 64, 4))
    W = plan.num_workers
    need = workspace_bytes(b * s_q, 1, heads, W)
    if workspace is not None:
        _need_bytes(workspace, "workspace", need)
    if out is not None:
        _need(out, "out", torch.float32, (b, s_q, heads, 512))
    if lse is not None:
        _need(lse, "lse", torch.float32, (b, s_q, heads))
    _need_status(status)
    _same_device(dev, kv_cache=kv_cache, kv_scales=kv_scales, rows=plan.rows, plan=plan.plan, workspace=workspace,
                 out=out, lse=lse, status=status)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if out is None:
        out = torch.empty(b, s_q, heads, 512, dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty(b, s_q, heads, dtype=torch.float32, device=dev)
    _check(int(lib().mla_sparse_decode_fwd(
        q.data_ptr(), kv_cache.data_ptr(), kv_scales.data_ptr(), KV_FP8_E4M3, plan.num_pages, b, s_q, heads, plan.topk,
        float(softmax_scale), plan.rows.data_ptr(), plan.plan.data_ptr(), W,
        None if workspace is None else workspace.data_ptr(),
        0 if workspace is None else workspace.numel() * workspace.element_size(), out.data_ptr(), lse.data_ptr(),
        _ptr(status), _stream(q))))
    return out, lse
