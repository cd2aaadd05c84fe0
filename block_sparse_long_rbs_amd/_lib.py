"""ctypes binding of librbs.so (include/rbs.h).

Argument marshalling only: each wrapper checks tensor placement and shapes,
allocates outputs with torch on the inputs' device, and passes raw device
pointers plus torch's current HIP stream to the C ABI. Every step of the
computation runs in the library's HIP kernels. There is no fallback: if the
shared library is missing, loading fails with an error.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librbs.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "rbs.h")

RBS_OK, RBS_E_ARG, RBS_E_UNSUPPORTED, RBS_E_CAPACITY, RBS_E_HIP = range(5)
RBS_DT_BF16, RBS_DT_F32 = 0, 1
RBS_SEL_FORCE_SINK = 0x1
RBS_SELECT_STATIC_SCRATCH_BYTES = 16 << 20   # the header's static scratch size

_c_i32, _c_u32, _c_i64, _c_f32, _c_f64 = (ctypes.c_int32, ctypes.c_uint32, ctypes.c_int64,
                                          ctypes.c_float, ctypes.c_double)
_vp = ctypes.c_void_p

_SIGS = {
    "rbs_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "rbs_block_stats": (ctypes.c_int, [ctypes.c_int, _vp, _vp, _c_i32, _c_i32, _c_i32, _c_i32,
                                       _c_i32, _vp, _vp, _vp, _vp, _vp]),
    "rbs_select": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _c_i32, _c_i32, _c_i32, _c_f64, _c_f64,
                                  _c_u32, _vp, _vp, _vp, _c_i64, _vp,
                                  ctypes.POINTER(ctypes.c_size_t), _vp]),
    "rbs_select_capacity": (_c_i64, [_c_i32, _c_i32, _c_f64, _c_f64, _c_u32]),
    "rbs_select_static": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _c_i32, _c_i32, _c_i32, _c_f64,
                                         _c_f64, _c_u32, _vp, _vp, _vp, _c_i64, _vp]),
    "rbs_block_stats_per_head": (ctypes.c_int, [ctypes.c_int, _vp, _vp, _c_i32, _c_i32, _c_i32,
                                                _c_i32, _c_i32, _vp, _vp, _vp, _vp, _vp]),
    "rbs_select_per_head": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _c_i32, _c_i32, _c_i32, _c_i32,
                                           _c_f64, _c_f64, _c_u32, _vp, _vp, _vp, _c_i64, _vp,
                                           ctypes.POINTER(ctypes.c_size_t), _vp]),
    "blocksparse_attn_fwd_per_head": (ctypes.c_int, [ctypes.c_int, _vp, _vp, _vp, _c_i32, _c_i32,
                                                     _c_i32, _c_i32, _c_i32, _vp, _vp, _c_f32,
                                                     _vp, _vp, _vp]),
    "blocksparse_attn_fwd": (ctypes.c_int, [ctypes.c_int, _vp, _vp, _vp, _c_i32, _c_i32, _c_i32,
                                            _c_i32, _c_i32, _vp, _vp, _c_f32, _vp, _vp, _vp]),
    "blocksparse_attn_fwd_shared_query": (ctypes.c_int, [ctypes.c_int, _vp, _vp, _vp, _c_i32,
                                                         _c_i32, _c_i32, _c_i32, _c_i32, _vp, _vp,
                                                         _c_f32, _vp, _vp, _vp]),
    "blocksparse_attn_fwd_fp8": (ctypes.c_int, [_vp, _vp, _vp, _c_i32, _c_i32, _c_i32, _c_i32,
                                                _c_i32, _vp, _vp, _c_f32, _c_f32, _c_f32, _c_f32,
                                                _vp, _vp, _vp]),
    "block_mask_attn_fwd": (ctypes.c_int, [ctypes.c_int, _vp, _vp, _vp, _c_i32, _c_i32, _c_i32,
                                           _c_i32, _c_i32, ctypes.POINTER(_c_i32),
                                           ctypes.POINTER(_c_i32), _c_f32, _c_i32, _c_f32, _vp,
                                           _vp, _vp, ctypes.POINTER(ctypes.c_size_t), _vp]),
}

_lib = None


class RbsError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: status {status} ({status_string(status)})")


def lib() -> ctypes.CDLL:
    """Load librbs.so (once) and declare the C signatures."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run `python -m block_sparse_long_rbs_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


def declared_symbols() -> list:
    """Function names declared in include/rbs.h."""
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([A-Za-z_][A-Za-z0-9_]*)\s*\(",
                      text, flags=re.M)


def status_string(status: int) -> str:
    return lib().rbs_status_string(status).decode()


def _check(fn: str, status: int):
    if status != RBS_OK:
        raise RbsError(fn, status)


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return RBS_DT_BF16
    if t.dtype == torch.float32:
        return RBS_DT_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _need_cuda(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous and on the GPU")


# Host-side shape checks: the kernels trust the sizes passed with the
# pointers, so every tensor is checked against them before a call.

def _check_qkv(fn: str, q, k, v=None):
    if q.dim() != 3 or k.dim() != 3 or k.shape[0] != q.shape[0] or k.shape[2] != q.shape[2]:
        raise ValueError(f"{fn}: q must be [S, Hq, D] and k [S, Hkv, D], got {tuple(q.shape)} "
                         f"and {tuple(k.shape)}")
    if v is not None and v.shape != k.shape:
        raise ValueError(f"{fn}: v must have k's shape {tuple(k.shape)}, got {tuple(v.shape)}")
    for t in (k, v):
        if t is not None and (t.dtype != q.dtype or t.device != q.device):
            raise TypeError(f"{fn}: q, k and v must share dtype and device")


def _check_tensor(fn: str, name: str, t, shape, dtype, device):
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or t.device != device:
        raise ValueError(f"{fn}: {name} must be {dtype} {tuple(shape)} on {device}, got "
                         f"{t.dtype} {tuple(t.shape)} on {t.device}")


def _check_csr(fn: str, row_ptr, col_idx, n_rows: int, device):
    _check_tensor(fn, "row_ptr", row_ptr, (n_rows + 1,), torch.int32, device)
    if col_idx.dim() != 1 or col_idx.dtype != torch.int32 or col_idx.device != device:
        raise ValueError(f"{fn}: col_idx must be a 1-D int32 tensor on {device} (holding at "
                         "least row_ptr[-1] entries)")


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


# ---------------------------------------------------------------------------

def rbs_block_stats(q: torch.Tensor, k: torch.Tensor, block: int):
    """Per-block centroid, radius, representative query and its norm.
    q [S, Hq, D], k [S, Hkv, D] (bf16 or f32) -> fp32 (cen [Hkv,nb,D],
    rad [Hkv,nb], q_rep [Hkv,nb,D], q_rep_norm [Hkv,nb])."""
    _check_qkv("rbs_block_stats", q, k)
    _need_cuda(q, k)
    S, Hq, D = q.shape
    Hkv = k.shape[1]
    nb = -(-S // block)
    f = dict(device=q.device, dtype=torch.float32)
    cen, qrep = torch.empty((Hkv, nb, D), **f), torch.empty((Hkv, nb, D), **f)
    rad, qn = torch.empty((Hkv, nb), **f), torch.empty((Hkv, nb), **f)
    _check("rbs_block_stats", lib().rbs_block_stats(
        _dtype_code(q), q.data_ptr(), k.data_ptr(), S, Hq, Hkv, D, block, cen.data_ptr(),
        rad.data_ptr(), qrep.data_ptr(), qn.data_ptr(), _stream(q)))
    return cen, rad, qrep, qn


def rbs_block_stats_per_head(q: torch.Tensor, k: torch.Tensor, block: int):
    """Centroid and radius per KV head, representative query per query head:
    -> fp32 (cen [Hkv,nb,D], rad [Hkv,nb], q_rep_head [Hq,nb,D],
    q_rep_head_norm [Hq,nb])."""
    _check_qkv("rbs_block_stats_per_head", q, k)
    _need_cuda(q, k)
    S, Hq, D = q.shape
    Hkv = k.shape[1]
    nb = -(-S // block)
    f = dict(device=q.device, dtype=torch.float32)
    cen, qrep = torch.empty((Hkv, nb, D), **f), torch.empty((Hq, nb, D), **f)
    rad, qn = torch.empty((Hkv, nb), **f), torch.empty((Hq, nb), **f)
    _check("rbs_block_stats_per_head", lib().rbs_block_stats_per_head(
        _dtype_code(q), q.data_ptr(), k.data_ptr(), S, Hq, Hkv, D, block, cen.data_ptr(),
        rad.data_ptr(), qrep.data_ptr(), qn.data_ptr(), _stream(q)))
    return cen, rad, qrep, qn


def rbs_select_capacity(n_kv_heads: int, n_blocks: int, keep_ratio_centroid: float,
                        keep_ratio_rescue: float, sink: bool = False) -> int:
    return int(lib().rbs_select_capacity(n_kv_heads, n_blocks, keep_ratio_centroid,
                                         keep_ratio_rescue, RBS_SEL_FORCE_SINK if sink else 0))


def rbs_select(cen, rad, qrep, qnorm, keep_ratio_centroid: float, keep_ratio_rescue: float,
               sink: bool = False, beta: Optional[torch.Tensor] = None, want_beta: bool = False,
               workspace: Optional[torch.Tensor] = None):
    """Dual-branch selection -> (row_ptr [Hkv*nb+1] int32, col_idx [capacity]
    int32, beta_used [Hkv,nb] fp32 or None). Only col_idx[:row_ptr[-1]] is
    meaningful."""
    Hkv, nb, D = cen.shape
    dev = cen.device
    for name, t, shape in (("cen", cen, (Hkv, nb, D)), ("rad", rad, (Hkv, nb)),
                           ("qrep", qrep, (Hkv, nb, D)), ("qnorm", qnorm, (Hkv, nb)),
                           ("beta", beta, (Hkv, nb))):
        if t is not None:
            _check_tensor("rbs_select", name, t, shape, torch.float32, dev)
    _need_cuda(cen, rad, qrep, qnorm, beta)
    flags = RBS_SEL_FORCE_SINK if sink else 0
    L = lib()
    ws = ctypes.c_size_t(0)
    _check("rbs_select", L.rbs_select(None, None, None, None, None, Hkv, nb, D,
                                      keep_ratio_centroid, keep_ratio_rescue, flags, None, None,
                                      None, 0, None, ctypes.byref(ws), None))
    if workspace is None or _nbytes(workspace) < ws.value:
        workspace = torch.empty(ws.value, dtype=torch.uint8, device=cen.device)
    cap = rbs_select_capacity(Hkv, nb, keep_ratio_centroid, keep_ratio_rescue, sink)
    row_ptr = torch.empty(Hkv * nb + 1, dtype=torch.int32, device=cen.device)
    col_idx = torch.empty(max(cap, 1), dtype=torch.int32, device=cen.device)
    beta_out = torch.empty((Hkv, nb), dtype=torch.float32, device=cen.device) if want_beta else None
    wsz = ctypes.c_size_t(_nbytes(workspace))
    _check("rbs_select", L.rbs_select(
        cen.data_ptr(), rad.data_ptr(), qrep.data_ptr(), qnorm.data_ptr(), _ptr(beta), Hkv, nb, D,
        keep_ratio_centroid, keep_ratio_rescue, flags, _ptr(beta_out), row_ptr.data_ptr(),
        col_idx.data_ptr(), cap, workspace.data_ptr(), ctypes.byref(wsz), _stream(cen)))
    return row_ptr, col_idx, beta_out


def rbs_select_static(cen, rad, qrep, qnorm, keep_ratio_centroid: float,
                      keep_ratio_rescue: float, sink: bool = False,
                      beta: Optional[torch.Tensor] = None, want_beta: bool = False,
                      row_ptr: Optional[torch.Tensor] = None,
                      col_idx: Optional[torch.Tensor] = None,
                      beta_out: Optional[torch.Tensor] = None):
    """rbs_select with the library's static scratch instead of a workspace
    (the call itself allocates no device memory). Outputs may be passed in
    (row_ptr [Hkv*nb+1], col_idx [capacity] int32, beta_out [Hkv,nb] fp32), so
    that nothing is allocated here either; otherwise they are allocated."""
    fn = "rbs_select_static"
    Hkv, nb, D = cen.shape
    dev = cen.device
    for name, t, shape in (("cen", cen, (Hkv, nb, D)), ("rad", rad, (Hkv, nb)),
                           ("qrep", qrep, (Hkv, nb, D)), ("qnorm", qnorm, (Hkv, nb)),
                           ("beta", beta, (Hkv, nb)), ("beta_out", beta_out, (Hkv, nb))):
        if t is not None:
            _check_tensor(fn, name, t, shape, torch.float32, dev)
    cap = rbs_select_capacity(Hkv, nb, keep_ratio_centroid, keep_ratio_rescue, sink)
    if row_ptr is None:
        row_ptr = torch.empty(Hkv * nb + 1, dtype=torch.int32, device=dev)
    if col_idx is None:
        col_idx = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
    _check_csr(fn, row_ptr, col_idx, Hkv * nb, dev)
    if want_beta and beta_out is None:
        beta_out = torch.empty((Hkv, nb), dtype=torch.float32, device=dev)
    _need_cuda(cen, rad, qrep, qnorm, beta, row_ptr, col_idx, beta_out)
    flags = RBS_SEL_FORCE_SINK if sink else 0
    _check(fn, lib().rbs_select_static(
        cen.data_ptr(), rad.data_ptr(), qrep.data_ptr(), qnorm.data_ptr(), _ptr(beta), Hkv, nb, D,
        keep_ratio_centroid, keep_ratio_rescue, flags, _ptr(beta_out), row_ptr.data_ptr(),
        col_idx.data_ptr(), col_idx.numel(), _stream(cen)))
    return row_ptr, col_idx, beta_out


def rbs_select_per_head(cen, rad, qrep_head, qnorm_head, keep_ratio_centroid: float,
                        keep_ratio_rescue: float, sink: bool = False,
                        beta: Optional[torch.Tensor] = None, want_beta: bool = False,
                        workspace: Optional[torch.Tensor] = None):
    """Per-query-head selection -> (row_ptr [Hq*nb+1] int32, col_idx int32,
    beta_used [Hkv,nb] fp32 or None); rows h * nb + i."""
    Hkv, nb, D = cen.shape
    Hq = qrep_head.shape[0]
    dev = cen.device
    for name, t, shape in (("cen", cen, (Hkv, nb, D)), ("rad", rad, (Hkv, nb)),
                           ("qrep_head", qrep_head, (Hq, nb, D)), ("qnorm_head", qnorm_head, (Hq, nb)),
                           ("beta", beta, (Hkv, nb))):
        if t is not None:
            _check_tensor("rbs_select_per_head", name, t, shape, torch.float32, dev)
    _need_cuda(cen, rad, qrep_head, qnorm_head, beta)
    flags = RBS_SEL_FORCE_SINK if sink else 0
    L = lib()
    ws = ctypes.c_size_t(0)
    _check("rbs_select_per_head", L.rbs_select_per_head(
        None, None, None, None, None, Hq, Hkv, nb, D, keep_ratio_centroid, keep_ratio_rescue,
        flags, None, None, None, 0, None, ctypes.byref(ws), None))
    if workspace is None or _nbytes(workspace) < ws.value:
        workspace = torch.empty(ws.value, dtype=torch.uint8, device=cen.device)
    cap = rbs_select_capacity(Hq, nb, keep_ratio_centroid, keep_ratio_rescue, sink)
    row_ptr = torch.empty(Hq * nb + 1, dtype=torch.int32, device=cen.device)
    col_idx = torch.empty(max(cap, 1), dtype=torch.int32, device=cen.device)
    beta_out = torch.empty((Hkv, nb), dtype=torch.float32, device=cen.device) if want_beta else None
    wsz = ctypes.c_size_t(_nbytes(workspace))
    _check("rbs_select_per_head", L.rbs_select_per_head(
        cen.data_ptr(), rad.data_ptr(), qrep_head.data_ptr(), qnorm_head.data_ptr(), _ptr(beta),
        Hq, Hkv, nb, D, keep_ratio_centroid, keep_ratio_rescue, flags, _ptr(beta_out),
        row_ptr.data_ptr(), col_idx.data_ptr(), cap, workspace.data_ptr(), ctypes.byref(wsz),
        _stream(cen)))
    return row_ptr, col_idx, beta_out


def blocksparse_attn_fwd_per_head(q, k, v, block: int, row_ptr, col_idx,
                                  softmax_scale: float = 0.0, want_lse: bool = False,
                                  out: Optional[torch.Tensor] = None):
    """Causal GQA attention over per-query-head CSR block lists (row h * nb + i)."""
    fn = "blocksparse_attn_fwd_per_head"
    _check_qkv(fn, q, k, v)
    S, Hq, D = q.shape
    Hkv = k.shape[1]
    _check_csr(fn, row_ptr, col_idx, Hq * -(-S // block), q.device)
    if out is not None:
        _check_tensor(fn, "out", out, q.shape, q.dtype, q.device)
    _need_cuda(q, k, v, row_ptr, col_idx, out)
    if out is None:
        out = torch.empty_like(q)
    lse = torch.empty((Hq, S), dtype=torch.float32, device=q.device) if want_lse else None
    _check("blocksparse_attn_fwd_per_head", lib().blocksparse_attn_fwd_per_head(
        _dtype_code(q), q.data_ptr(), k.data_ptr(), v.data_ptr(), S, Hq, Hkv, D, block,
        row_ptr.data_ptr(), col_idx.data_ptr(), softmax_scale, out.data_ptr(), _ptr(lse),
        _stream(q)))
    return out, lse


def blocksparse_attn_fwd(q, k, v, block: int, row_ptr, col_idx, softmax_scale: float = 0.0,
                         want_lse: bool = False, out: Optional[torch.Tensor] = None):
    """Causal GQA attention over the CSR-selected key blocks -> (out, lse or None)."""
    fn = "blocksparse_attn_fwd"
    _check_qkv(fn, q, k, v)
    S, Hq, D = q.shape
    Hkv = k.shape[1]
    _check_csr(fn, row_ptr, col_idx, Hkv * -(-S // block), q.device)
    if out is not None:
        _check_tensor(fn, "out", out, q.shape, q.dtype, q.device)
    _need_cuda(q, k, v, row_ptr, col_idx, out)
    if out is None:
        out = torch.empty_like(q)
    lse = torch.empty((Hq, S), dtype=torch.float32, device=q.device) if want_lse else None
    _check("blocksparse_attn_fwd", lib().blocksparse_attn_fwd(
        _dtype_code(q), q.data_ptr(), k.data_ptr(), v.data_ptr(), S, Hq, Hkv, D, block,
        row_ptr.data_ptr(), col_idx.data_ptr(), softmax_scale, out.data_ptr(), _ptr(lse),
        _stream(q)))
    return out, lse


def blocksparse_attn_fwd_shared_query(q, k, v, block: int, row_ptr, col_idx,
                                      softmax_scale: float = 0.0, want_lse: bool = False,
                                      out: Optional[torch.Tensor] = None):
    """blocksparse_attn_fwd with neighbouring query blocks processed together
    over the union of their block lists (same result) -> (out, lse or None)."""
    fn = "blocksparse_attn_fwd_shared_query"
    _check_qkv(fn, q, k, v)
    S, Hq, D = q.shape
    Hkv = k.shape[1]
    _check_csr(fn, row_ptr, col_idx, Hkv * -(-S // block), q.device)
    if out is not None:
        _check_tensor(fn, "out", out, q.shape, q.dtype, q.device)
    _need_cuda(q, k, v, row_ptr, col_idx, out)
    if out is None:
        out = torch.empty_like(q)
    lse = torch.empty((Hq, S), dtype=torch.float32, device=q.device) if want_lse else None
    _check(fn, lib().blocksparse_attn_fwd_shared_query(
        _dtype_code(q), q.data_ptr(), k.data_ptr(), v.data_ptr(), S, Hq, Hkv, D, block,
        row_ptr.data_ptr(), col_idx.data_ptr(), softmax_scale, out.data_ptr(), _ptr(lse),
        _stream(q)))
    return out, lse


def blocksparse_attn_fwd_fp8(q, k, v, block: int, row_ptr, col_idx, q_descale: float = 1.0,
                             k_descale: float = 1.0, v_descale: float = 1.0,
                             softmax_scale: float = 0.0, want_lse: bool = False,
                             out: Optional[torch.Tensor] = None):
    """blocksparse_attn_fwd on fp8 (torch.float8_e4m3fn) Q, K, V with per-tensor
    dequantisation factors -> (bf16 out, lse or None)."""
    fn = "blocksparse_attn_fwd_fp8"
    if q.dtype != torch.float8_e4m3fn:
        raise TypeError(f"{fn} takes float8_e4m3fn tensors, got {q.dtype}")
    _check_qkv(fn, q, k, v)
    S, Hq, D = q.shape
    Hkv = k.shape[1]
    _check_csr(fn, row_ptr, col_idx, Hkv * -(-S // block), q.device)
    if out is not None:
        _check_tensor(fn, "out", out, q.shape, torch.bfloat16, q.device)
    _need_cuda(q, k, v, row_ptr, col_idx, out)
    if out is None:
        out = torch.empty((S, Hq, D), dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((Hq, S), dtype=torch.float32, device=q.device) if want_lse else None
    _check("blocksparse_attn_fwd_fp8", lib().blocksparse_attn_fwd_fp8(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), S, Hq, Hkv, D, block, row_ptr.data_ptr(),
        col_idx.data_ptr(), softmax_scale, q_descale, k_descale, v_descale, out.data_ptr(),
        _ptr(lse), _stream(q)))
    return out, lse


def _bmask_args(q, k_cached, v, seg_start, k_rerotate, rope_theta, q_row_begin, softmax_scale,
                out, lse):
    S, Hq, D = q.shape
    Hkv = k_cached.shape[1]
    n_seg = len(seg_start) - 1
    ss = (_c_i32 * (n_seg + 1))(*[int(x) for x in seg_start])
    rr = (_c_i32 * max(n_seg, 1))(*[int(x) for x in k_rerotate])
    return (_dtype_code(q), q.data_ptr(), k_cached.data_ptr(), v.data_ptr(), S, Hq, Hkv, D, n_seg,
            ss, rr, rope_theta, q_row_begin, softmax_scale, _ptr(out), _ptr(lse))


def block_mask_workspace_bytes(q, k_cached, v, seg_start: Sequence[int],
                               k_rerotate: Sequence[int], rope_theta: float,
                               q_row_begin: int = 0) -> int:
    """Workspace bytes block_mask_attn_fwd needs for this layout (size query)."""
    # a size query enqueues nothing; q stands in for the output pointer, which
    # is only checked for alignment
    args = _bmask_args(q, k_cached, v, seg_start, k_rerotate, rope_theta, q_row_begin, 0.0, q,
                       None)
    need = ctypes.c_size_t(0)
    _check("block_mask_attn_fwd", lib().block_mask_attn_fwd(*args, None, ctypes.byref(need), None))
    return need.value


def block_mask_attn_fwd(q, k_cached, v, seg_start: Sequence[int], k_rerotate: Sequence[int],
                        rope_theta: float, q_row_begin: int = 0, softmax_scale: float = 0.0,
                        want_lse: bool = False, out: Optional[torch.Tensor] = None,
                        workspace: Optional[torch.Tensor] = None):
    """Block-attention prefill with RoPE re-encoding of cached keys -> (out, lse or None).
    The workspace (re-encoded keys; partial results of the final block's split
    rows) is allocated when not given or too small."""
    fn = "block_mask_attn_fwd"
    _check_qkv(fn, q, k_cached, v)
    S, Hq, D = q.shape
    if out is not None:
        _check_tensor(fn, "out", out, q.shape, q.dtype, q.device)
    _need_cuda(q, k_cached, v, out)
    if out is None:
        out = torch.empty_like(q)
    lse = torch.empty((Hq, S), dtype=torch.float32, device=q.device) if want_lse else None
    args = _bmask_args(q, k_cached, v, seg_start, k_rerotate, rope_theta, q_row_begin,
                       softmax_scale, out, lse)
    need = ctypes.c_size_t(0)
    _check("block_mask_attn_fwd", lib().block_mask_attn_fwd(*args, None, ctypes.byref(need), None))
    if workspace is None or _nbytes(workspace) < max(need.value, 1):
        workspace = torch.empty(max(need.value, 1), dtype=torch.uint8, device=q.device)
    wsz = ctypes.c_size_t(_nbytes(workspace))
    _check("block_mask_attn_fwd", lib().block_mask_attn_fwd(
        *args, workspace.data_ptr(), ctypes.byref(wsz), _stream(q)))
    return out, lse
