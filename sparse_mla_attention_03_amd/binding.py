"""ctypes binding over libsparsemla (include/sparse_mla.h).

Argument marshalling only: the functions below take torch tensors, check that
their dtypes / devices / layouts are what the C ABI expects, allocate missing
outputs and the workspace with torch, and call the library on torch's current
HIP stream.  Every step of the computation runs in the library's kernels; if
the library is not built this module raises instead of computing anything.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "csrc", "libsparsemla.so")

KV_BF16 = 0
KV_FP8_E4M3 = 1
DV = 512
MAX_SPLITS = 64
DOTS_DEFAULT = 0
DOTS_BF16 = 1
ABI_VERSION = 3
NOALLOC_SCRATCH_BYTES = 32 << 20   # SMLA_NOALLOC_SCRATCH_BYTES

STATUS_NAMES = {0: "SMLA_OK", 1: "SMLA_ERR_NULL", 2: "SMLA_ERR_SHAPE", 3: "SMLA_ERR_DTYPE",
                4: "SMLA_ERR_ALIGN", 5: "SMLA_ERR_INVALID_ARG", 6: "SMLA_ERR_UNSUPPORTED",
                7: "SMLA_ERR_WORKSPACE", 8: "SMLA_ERR_HIP"}


class SparseMLAError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        self.detail = detail
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {detail}")


class Options(ctypes.Structure):
    _fields_ = [("num_splits", ctypes.c_int32), ("dot_precision", ctypes.c_int32),
                ("kernel_events", ctypes.c_void_p * 2), ("sinks", ctypes.c_void_p),
                ("q_scale", ctypes.c_float), ("reserved", ctypes.c_int32 * 3)]


_lib = None


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load libsparsemla.so (built in-tree by __graft_entry__.build())."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise SparseMLAError(8, f"{p} is not built; run `python -c 'import __graft_entry__ as g; "
                                f"g.build()'` (hipcc, gfx950) first")
    lib = ctypes.CDLL(p)
    i64, i32, vp, f32, sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_float, ctypes.c_size_t
    fwd_args = [vp, i64, i64, i64, i64, i64, vp, i32, i64, i64, vp, i64, i64, f32, f32, vp, vp,
                vp, sz, vp]
    lib.sparse_mla_fwd.argtypes = fwd_args
    lib.sparse_mla_fwd.restype = ctypes.c_int
    lib.sparse_mla_fwd_ex.argtypes = fwd_args + [ctypes.POINTER(Options)]
    lib.sparse_mla_fwd_ex.restype = ctypes.c_int
    lib.sparse_mla_fwd_noalloc.argtypes = fwd_args[:17] + [vp, ctypes.POINTER(Options)]
    lib.sparse_mla_fwd_noalloc.restype = ctypes.c_int
    lib.sparse_mla_num_splits.argtypes = [i64, i64, i64, i64, i32, i32]
    lib.sparse_mla_num_splits.restype = i32
    lib.sparse_mla_workspace_bytes.argtypes = [i64, i64, i64, i64, i32, i32]
    lib.sparse_mla_workspace_bytes.restype = sz
    lib.sparse_mla_quantize_q_fp8.argtypes = [vp, i64, i64, i64, i64, i64, vp, vp, vp]
    lib.sparse_mla_quantize_q_fp8.restype = ctypes.c_int
    lib.sparse_mla_status_string.argtypes = [ctypes.c_int]
    lib.sparse_mla_status_string.restype = ctypes.c_char_p
    lib.sparse_mla_last_error.argtypes = []
    lib.sparse_mla_last_error.restype = ctypes.c_char_p
    if path is None or hasattr(lib, "sparse_mla_fwd_varlen"):   # (a library built here always has them)
        lib.sparse_mla_fwd_varlen.argtypes = fwd_args[:13] + [vp] + fwd_args[13:] + [ctypes.POINTER(Options)]
        lib.sparse_mla_fwd_varlen.restype = ctypes.c_int
        lib.sparse_mla_workspace_bytes_varlen.argtypes = [i64, i64, i64, i64, i32]
        lib.sparse_mla_workspace_bytes_varlen.restype = sz
    if path is None or hasattr(lib, "sparse_mla_rope_concat_cache"):
        lib.sparse_mla_rope_concat_cache.argtypes = [vp, i64, i64, vp, i64, i64, vp, i64, vp, i64, vp, vp, i64,
                                                      i32, i64, i64, vp, i32, f32, vp, vp, i32, i64, i64, f32, vp]
        lib.sparse_mla_rope_concat_cache.restype = ctypes.c_int
    lib.sparse_mla_abi_version.argtypes = []
    lib.sparse_mla_abi_version.restype = i32
    if path is None:
        v = lib.sparse_mla_abi_version()
        if v != ABI_VERSION:
            raise SparseMLAError(8, f"{p} has ABI version {v}, this binding needs {ABI_VERSION}; rebuild it")
        _lib = lib
    return lib


def sparse_mla_status_string(status: int) -> str:
    return load_library().sparse_mla_status_string(int(status)).decode()


def sparse_mla_last_error() -> str:
    return load_library().sparse_mla_last_error().decode()


def _check(status: int) -> None:
    if status != 0:
        raise SparseMLAError(status, sparse_mla_last_error())


def _kv_dtype(kv: torch.Tensor) -> int:
    if kv.dtype == torch.bfloat16:
        return KV_BF16
    if kv.dtype in (torch.uint8, torch.float8_e4m3fn):
        return KV_FP8_E4M3
    raise TypeError(f"kv_pool must be bfloat16 or e4m3 (uint8 / float8_e4m3fn), got {kv.dtype}")


def _stream_handle(dev: torch.device, stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def sparse_mla_num_splits(T: int, H: int, K: int, Dqk: int, kv_dtype: int, num_splits: int = 0) -> int:
    s = int(load_library().sparse_mla_num_splits(T, H, K, Dqk, kv_dtype, num_splits))
    if s <= 0:
        raise SparseMLAError(5, sparse_mla_last_error())
    return s


def sparse_mla_workspace_bytes(T: int, H: int, K: int, Dqk: int, kv_dtype: int,
                               num_splits: int = 0) -> int:
    n = load_library().sparse_mla_workspace_bytes(T, H, K, Dqk, kv_dtype, num_splits)
    if n == ctypes.c_size_t(-1).value:
        raise SparseMLAError(5, sparse_mla_last_error())
    return int(n)


def _pool_shape(kv_pool: torch.Tensor):
    if kv_pool.dim() == 3:
        nb, bs, D = kv_pool.shape
    elif kv_pool.dim() == 2:
        (nb, D), bs = kv_pool.shape, 1
    else:
        raise ValueError("kv_pool must be [num_blocks, block_size, Dqk] or [N, Dqk]")
    return nb, bs, D


def _fwd_operands(q, kv_pool, topk_idx, out, lse, q_scale):
    """Checks shared by the forward entry points; returns the sizes and out / lse."""
    if q_scale > 0:
        if q.dim() != 3 or q.dtype not in (torch.uint8, torch.float8_e4m3fn):
            raise TypeError("pre-quantised q must be uint8 / float8_e4m3fn [T, H, Dqk]")
    elif q.dim() != 3 or q.dtype != torch.bfloat16:
        raise TypeError("q must be bfloat16 [T, H, Dqk]")
    if not q.is_cuda:
        raise ValueError("q must live on a GPU")
    T, H, D = q.shape
    if T > 0 and q.stride(2) != 1:
        raise ValueError("q's last dimension must be contiguous")
    nb, bs, Dkv = _pool_shape(kv_pool)
    if Dkv != D:
        raise ValueError(f"kv_pool rows are {Dkv} wide, q rows {D}")
    if not kv_pool.is_contiguous():
        raise ValueError("kv_pool must be contiguous")
    kvd = _kv_dtype(kv_pool)
    if topk_idx.dim() != 2 or topk_idx.dtype != torch.int32 or topk_idx.shape[0] != T:
        raise TypeError("topk_idx must be int32 [T, K]")
    K = topk_idx.shape[1]
    if T > 0 and K > 1 and topk_idx.stride(1) != 1:
        raise ValueError("topk_idx rows must be contiguous")
    for t_, name in ((kv_pool, "kv_pool"), (topk_idx, "topk_idx")):
        if t_.device != q.device:
            raise ValueError(f"{name} is on {t_.device}, q on {q.device}")
    if out is None:
        out = torch.empty((T, H, DV), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((T, H), dtype=torch.float32, device=q.device)
    if out.shape != (T, H, DV) or out.dtype != torch.bfloat16 or not out.is_contiguous():
        raise ValueError("out must be a contiguous bfloat16 [T, H, 512] tensor")
    if lse.shape != (T, H) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [T, H] tensor")
    return T, H, D, nb, bs, kvd, K, out, lse


def _fwd_options(H, q, num_splits, dot_precision, q_scale, sinks, kernel_events=None):
    opts = Options()
    opts.num_splits = num_splits
    opts.dot_precision = dot_precision
    opts.q_scale = float(q_scale)
    if sinks is not None:
        if sinks.shape != (H,) or sinks.dtype != torch.float32 or not sinks.is_contiguous():
            raise ValueError("sinks must be a contiguous float32 [H] tensor")
        if sinks.device != q.device:
            raise ValueError(f"sinks is on {sinks.device}, q on {q.device}")
        opts.sinks = sinks.data_ptr()
    if kernel_events is not None:
        opts.kernel_events[0], opts.kernel_events[1] = kernel_events
    return opts


def sparse_mla_fwd_ex(q: torch.Tensor, kv_pool: torch.Tensor, topk_idx: torch.Tensor,
                      sm_scale: float, kv_scale: float = 1.0, out: torch.Tensor | None = None,
                      lse: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                      num_splits: int = 0, stream=None, kernel_events=None,
                      sinks: torch.Tensor | None = None, dot_precision: int = 0,
                      q_scale: float = 0.0):
    """Sparse MLA forward; returns (out bf16 [T,H,512], lse fp32 [T,H]).

    kernel_events: optional pair of raw hipEvent_t handles (ints) the library
    records around its main kernel (instrumentation for benchmarks).
    sinks: optional float32 [H] per-head sink logits on q's device.
    dot_precision: DOTS_DEFAULT or DOTS_BF16 (e4m3 KV only).
    q_scale: > 0 when q is already quantised: q then holds OCP e4m3 codes (uint8 or
    float8_e4m3fn) and qhat = q_scale * code (e4m3 KV with e4m3 dots only)."""
    lib = load_library()
    T, H, D, nb, bs, kvd, K, out, lse = _fwd_operands(q, kv_pool, topk_idx, out, lse, q_scale)
    ws_ptr, ws_bytes = None, 0
    if T > 0:
        need = sparse_mla_workspace_bytes(T, H, K, D, kvd, num_splits)
        if need > 0:
            if workspace is None or workspace.numel() * workspace.element_size() < need:
                workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
            ws_ptr = workspace.data_ptr()
            ws_bytes = workspace.numel() * workspace.element_size()
    opts = _fwd_options(H, q, num_splits, dot_precision, q_scale, sinks, kernel_events)
    st = lib.sparse_mla_fwd_ex(
        q.data_ptr(), T, H, D, q.stride(0) if T else 0, q.stride(1) if T else 0,
        kv_pool.data_ptr(), kvd, nb, bs,
        topk_idx.data_ptr() if topk_idx.numel() else None, K, topk_idx.stride(0) if T else 0,
        float(sm_scale), float(kv_scale), out.data_ptr(), lse.data_ptr(),
        ws_ptr, ws_bytes, _stream_handle(q.device, stream), ctypes.byref(opts))
    _check(st)
    return out, lse


def sparse_mla_fwd_noalloc(q: torch.Tensor, kv_pool: torch.Tensor, topk_idx: torch.Tensor,
                           sm_scale: float, kv_scale: float = 1.0, out: torch.Tensor | None = None,
                           lse: torch.Tensor | None = None, num_splits: int = 0, stream=None,
                           sinks: torch.Tensor | None = None, dot_precision: int = 0,
                           q_scale: float = 0.0):
    """sparse_mla_fwd_ex without a workspace: the library keeps the split partials in
    its own per-device scratch array and allocates nothing during the call (pass
    out / lse to keep this wrapper from allocating them)."""
    lib = load_library()
    T, H, D, nb, bs, kvd, K, out, lse = _fwd_operands(q, kv_pool, topk_idx, out, lse, q_scale)
    opts = _fwd_options(H, q, num_splits, dot_precision, q_scale, sinks)
    st = lib.sparse_mla_fwd_noalloc(
        q.data_ptr(), T, H, D, q.stride(0) if T else 0, q.stride(1) if T else 0,
        kv_pool.data_ptr(), kvd, nb, bs,
        topk_idx.data_ptr() if topk_idx.numel() else None, K, topk_idx.stride(0) if T else 0,
        float(sm_scale), float(kv_scale), out.data_ptr(), lse.data_ptr(),
        _stream_handle(q.device, stream), ctypes.byref(opts))
    _check(st)
    return out, lse


def sparse_mla_fwd(q, kv_pool, topk_idx, sm_scale, kv_scale=1.0, out=None, lse=None,
                   workspace=None, stream=None):
    """Sparse MLA forward with the library's automatic split-K choice."""
    return sparse_mla_fwd_ex(q, kv_pool, topk_idx, sm_scale, kv_scale, out=out, lse=lse,
                             workspace=workspace, num_splits=0, stream=stream)


def sparse_mla_quantize_q_fp8(q: torch.Tensor, codes: torch.Tensor | None = None,
                              scales: torch.Tensor | None = None, stream=None):
    """Per-tile e4m3 quantisation of q on the GPU -> (codes uint8 [T,H,Dqk], scales fp32 [T,G])."""
    lib = load_library()
    if q.dim() != 3 or q.dtype != torch.bfloat16 or not q.is_cuda:
        raise TypeError("q must be a GPU bfloat16 [T, H, Dqk] tensor")
    T, H, D = q.shape
    if T > 0 and q.stride(2) != 1:
        raise ValueError("q's last dimension must be contiguous")
    G = (H + 63) // 64
    if codes is None:
        codes = torch.empty((T, H, D), dtype=torch.uint8, device=q.device)
    if scales is None:
        scales = torch.empty((T, G), dtype=torch.float32, device=q.device)
    st = lib.sparse_mla_quantize_q_fp8(q.data_ptr(), T, H, D, q.stride(0) if T else 0,
                                       q.stride(1) if T else 0, codes.data_ptr(),
                                       scales.data_ptr(), _stream_handle(q.device, stream))
    _check(st)
    return codes, scales


def sparse_mla_rope_concat_cache(ql_nope: torch.Tensor, q_pe: torch.Tensor, kv_c: torch.Tensor,
                                 k_pe: torch.Tensor, positions: torch.Tensor,
                                 cos_sin_cache: torch.Tensor, is_neox: bool,
                                 slot_mapping: torch.Tensor, kv_cache: torch.Tensor,
                                 q_out: torch.Tensor | None = None, q_fp8: bool = False,
                                 q_scale: float = 1.0, kv_scale: float = 1.0, stream=None):
    """Fused q-RoPE + q-concat + KV-concat + cache write; returns q_out [T, H, 576]
    (bf16, or e4m3 codes as uint8 when q_fp8).  kv_cache [num_blocks, block_size, 576]
    (bf16, or uint8 / float8_e4m3fn codes) is written in place."""
    lib = load_library()
    if ql_nope.dim() != 3 or ql_nope.dtype != torch.bfloat16 or ql_nope.shape[2] != DV:
        raise TypeError("ql_nope must be bfloat16 [T, H, 512]")
    T, H, _ = ql_nope.shape
    if q_pe.shape != (T, H, 64) or q_pe.dtype != torch.bfloat16:
        raise TypeError("q_pe must be bfloat16 [T, H, 64]")
    if kv_c.shape != (T, DV) or kv_c.dtype != torch.bfloat16 or k_pe.shape != (T, 64) or k_pe.dtype != torch.bfloat16:
        raise TypeError("kv_c / k_pe must be bfloat16 [T, 512] / [T, 64]")
    for x, name in ((ql_nope, "ql_nope"), (q_pe, "q_pe")):
        if T > 0 and x.stride(2) != 1:
            raise ValueError(f"{name}'s last dimension must be contiguous")
    for x, name in ((kv_c, "kv_c"), (k_pe, "k_pe")):
        if T > 0 and x.stride(1) != 1:
            raise ValueError(f"{name}'s last dimension must be contiguous")
    if positions.shape != (T,) or positions.dtype != torch.int64 or slot_mapping.shape != (T,) \
            or slot_mapping.dtype != torch.int64:
        raise TypeError("positions and slot_mapping must be int64 [T]")
    if cos_sin_cache.dim() != 2 or cos_sin_cache.shape[1] != 64 or cos_sin_cache.dtype != torch.float32 \
            or not cos_sin_cache.is_contiguous():
        raise TypeError("cos_sin_cache must be a contiguous float32 [max_pos, 64] tensor")
    if kv_cache.dim() != 3 or kv_cache.shape[2] != 576 or not kv_cache.is_contiguous():
        raise TypeError("kv_cache must be a contiguous [num_blocks, block_size, 576] tensor")
    kvd = _kv_dtype(kv_cache)
    qdt = torch.uint8 if q_fp8 else torch.bfloat16
    if q_out is None:
        q_out = torch.empty((T, H, 576), dtype=qdt, device=ql_nope.device)
    if q_out.shape != (T, H, 576) or q_out.dtype != qdt or not q_out.is_contiguous():
        raise ValueError("q_out must be a contiguous [T, H, 576] tensor of the output dtype")
    for x in (q_pe, kv_c, k_pe, positions, cos_sin_cache, slot_mapping, kv_cache, q_out):
        if x.device != ql_nope.device:
            raise ValueError("all tensors must be on one device")
    st = lib.sparse_mla_rope_concat_cache(
        ql_nope.data_ptr(), ql_nope.stride(0), ql_nope.stride(1),
        q_pe.data_ptr(), q_pe.stride(0), q_pe.stride(1),
        kv_c.data_ptr(), kv_c.stride(0), k_pe.data_ptr(), k_pe.stride(0),
        positions.data_ptr(), cos_sin_cache.data_ptr(), cos_sin_cache.shape[0], int(bool(is_neox)),
        T, H, q_out.data_ptr(), 1 if q_fp8 else 0, float(q_scale),
        slot_mapping.data_ptr(), kv_cache.data_ptr(), kvd, kv_cache.shape[0], kv_cache.shape[1],
        float(kv_scale), _stream_handle(ql_nope.device, stream))
    _check(st)
    return q_out


def sparse_mla_workspace_bytes_varlen(T: int, H: int, K: int, Dqk: int, kv_dtype: int) -> int:
    n = load_library().sparse_mla_workspace_bytes_varlen(T, H, K, Dqk, kv_dtype)
    if n == ctypes.c_size_t(-1).value:
        raise SparseMLAError(2, load_library().sparse_mla_last_error().decode())
    return n


def sparse_mla_fwd_varlen(q: torch.Tensor, kv_pool: torch.Tensor, topk_idx: torch.Tensor,
                          topk_len: torch.Tensor, sm_scale: float, kv_scale: float = 1.0,
                          out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                          workspace: torch.Tensor | None = None, stream=None, sinks=None,
                          dot_precision: int = 0, q_scale: float = 0.0):
    """Forward pass with per-token list lengths: token t uses topk_idx[t, :topk_len[t]]
    (int32 [T] on the device); the split over each list is chosen per token."""
    lib = load_library()
    if q_scale > 0:
        if q.dim() != 3 or q.dtype not in (torch.uint8, torch.float8_e4m3fn):
            raise TypeError("pre-quantised q must be uint8 / float8_e4m3fn [T, H, Dqk]")
    elif q.dim() != 3 or q.dtype != torch.bfloat16:
        raise TypeError("q must be bfloat16 [T, H, Dqk]")
    T, H, D = q.shape
    if T > 0 and q.stride(2) != 1:
        raise ValueError("q's last dimension must be contiguous")
    nb, bs, Dkv = _pool_shape(kv_pool)
    if Dkv != D or not kv_pool.is_contiguous():
        raise ValueError("kv_pool must be contiguous with rows as wide as q's")
    kvd = _kv_dtype(kv_pool)
    if topk_idx.dim() != 2 or topk_idx.dtype != torch.int32 or topk_idx.shape[0] != T:
        raise TypeError("topk_idx must be int32 [T, K]")
    K = topk_idx.shape[1]
    if T > 0 and K > 1 and topk_idx.stride(1) != 1:
        raise ValueError("topk_idx rows must be contiguous")
    if topk_len.shape != (T,) or topk_len.dtype != torch.int32 or not topk_len.is_contiguous():
        raise TypeError("topk_len must be a contiguous int32 [T] tensor")
    for t_, name in ((kv_pool, "kv_pool"), (topk_idx, "topk_idx"), (topk_len, "topk_len")):
        if t_.device != q.device:
            raise ValueError(f"{name} is on {t_.device}, q on {q.device}")
    if out is None:
        out = torch.empty((T, H, DV), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((T, H), dtype=torch.float32, device=q.device)
    ws_ptr, ws_bytes = None, 0
    if T > 0:
        need = sparse_mla_workspace_bytes_varlen(T, H, K, D, kvd)
        if workspace is None or workspace.numel() * workspace.element_size() < need:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        ws_ptr = workspace.data_ptr()
        ws_bytes = workspace.numel() * workspace.element_size()
    opts = Options()
    opts.dot_precision = dot_precision
    opts.q_scale = float(q_scale)
    if sinks is not None:
        if sinks.shape != (H,) or sinks.dtype != torch.float32 or not sinks.is_contiguous():
            raise ValueError("sinks must be a contiguous float32 [H] tensor")
        opts.sinks = sinks.data_ptr()
    st = lib.sparse_mla_fwd_varlen(
        q.data_ptr(), T, H, D, q.stride(0) if T else 0, q.stride(1) if T else 0,
        kv_pool.data_ptr(), kvd, nb, bs,
        topk_idx.data_ptr() if topk_idx.numel() else None, K, topk_idx.stride(0) if T else 0,
        topk_len.data_ptr() if T else None,
        float(sm_scale), float(kv_scale), out.data_ptr(), lse.data_ptr(),
        ws_ptr, ws_bytes, _stream_handle(q.device, stream), ctypes.byref(opts))
    _check(st)
    return out, lse
