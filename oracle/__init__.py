"""fp64 CPU oracle for the sparse MLA forward pass (ctypes wrapper).

TEST INFRASTRUCTURE ONLY.  The test suite, the smoke check and the CPU-baseline
leg of the benchmark may import this package; the product path (the HIP library
and its Python binding) never does.  It shares no code with the HIP path: the
arithmetic lives in ``sparse_mla_oracle.c`` (plain C, fp64, OpenMP over
independent (token, head) pairs), built into ``liboracle.so`` next to it.

Inputs are numpy arrays holding the exact bits the GPU sees:
  q    uint16 [T, H, Dqk]  bf16 bit patterns (any strides in the last two axes
                           are honoured; the last axis must be contiguous)
  kv   uint16 [N, Dqk] bf16 bits, or uint8 [N, Dqk] OCP e4m3 codes
  idx  int32  [T, K]       flat slot ids; anything outside [0, N) is padding
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sparse_mla_oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")

KV_BF16 = 0
KV_FP8_E4M3 = 1
Q_EXACT = 0
Q_TILE_FP8 = 1
Q_GIVEN_FP8 = 2

_lib = None


def build(force: bool = False) -> str:
    """Compile liboracle.so with gcc (fp64, -O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
               "-fno-fast-math", "-ffp-contract=off", "-Wall", "-Wextra",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True, cwd=_HERE)
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        build()
    lib = ctypes.CDLL(LIB_PATH)
    c_i64, c_p = ctypes.c_int64, ctypes.c_void_p
    lib.oracle_bf16_value.restype = ctypes.c_double
    lib.oracle_bf16_value.argtypes = [ctypes.c_uint16]
    lib.oracle_e4m3_value.restype = ctypes.c_double
    lib.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_encode_rne_sat.restype = ctypes.c_uint8
    lib.oracle_e4m3_encode_rne_sat.argtypes = [ctypes.c_float]
    lib.oracle_quantize_q_tiles.restype = None
    lib.oracle_quantize_q_tiles.argtypes = [c_p, c_i64, c_i64, c_i64, c_i64, c_i64, c_p, c_p]
    lib.oracle_sparse_mla_fwd.restype = ctypes.c_int
    lib.oracle_sparse_mla_fwd.argtypes = [
        c_p, c_i64, c_i64, c_i64, c_i64, c_i64,
        c_p, ctypes.c_int, c_i64,
        c_p, c_i64, c_i64,
        ctypes.c_double, ctypes.c_double, ctypes.c_int, ctypes.c_double,
        c_p, c_p, c_p]
    lib.oracle_bf16_round.restype = ctypes.c_uint16
    lib.oracle_bf16_round.argtypes = [ctypes.c_double]
    lib.oracle_rope_concat_cache.restype = ctypes.c_int
    lib.oracle_rope_concat_cache.argtypes = [
        c_p, c_i64, c_i64, c_p, c_i64, c_i64, c_p, c_i64, c_p, c_i64,
        c_p, c_p, c_i64, ctypes.c_int, c_i64, c_i64,
        c_p, ctypes.c_int, ctypes.c_double, c_p, c_p, ctypes.c_int, c_i64, ctypes.c_double]
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    lib.oracle_set_num_threads.restype = None
    lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
    _lib = lib
    return lib


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads the oracle's following calls use."""
    _load().oracle_set_num_threads(int(n))


def bf16_value(bits) -> np.ndarray:
    lib = _load()
    b = np.asarray(bits, dtype=np.uint16)
    return np.array([lib.oracle_bf16_value(int(x)) for x in b.ravel()]).reshape(b.shape)


def e4m3_value(codes) -> np.ndarray:
    lib = _load()
    c = np.asarray(codes, dtype=np.uint8)
    return np.array([lib.oracle_e4m3_value(int(x)) for x in c.ravel()]).reshape(c.shape)


def e4m3_encode(x) -> np.ndarray:
    lib = _load()
    a = np.asarray(x, dtype=np.float32)
    return np.array([lib.oracle_e4m3_encode_rne_sat(float(v)) for v in a.ravel()],
                    dtype=np.uint8).reshape(a.shape)


def _strides_elems(a: np.ndarray):
    return tuple(s // a.itemsize for s in a.strides)


def quantize_q(q: np.ndarray):
    """Per-tile e4m3 quantisation of q -> (codes uint8 [T,H,Dqk], scales fp32 [T,ceil(H/64)])."""
    lib = _load()
    assert q.dtype == np.uint16 and q.ndim == 3
    T, H, D = q.shape
    st, sh, sd = _strides_elems(q)
    assert sd == 1
    codes = np.empty((T, H, D), dtype=np.uint8)
    scales = np.empty((T, (H + 63) // 64), dtype=np.float32)
    lib.oracle_quantize_q_tiles(q.ctypes.data, T, H, D, st, sh,
                                codes.ctypes.data, scales.ctypes.data)
    return codes, scales


def sparse_mla_fwd(q: np.ndarray, kv: np.ndarray, idx: np.ndarray,
                   sm_scale: float, kv_scale: float, q_mode: int = Q_TILE_FP8,
                   sinks: np.ndarray | None = None, q_scale: float = 0.0):
    """Return (out fp64 [T,H,512], lse fp64 [T,H]).

    ``q_mode`` matters only for e4m3 KV: Q_TILE_FP8 reproduces the per-tile q
    quantisation of the FP8-dots path, Q_EXACT keeps q exact.
    sm_scale / kv_scale are rounded to fp32 first, as the library receives them.
    ``sinks``: optional [H] per-head sink logits, rounded to fp32 likewise.
    ``q_mode = Q_GIVEN_FP8``: q holds e4m3 codes (uint8), qhat = q_scale * code.
    """
    lib = _load()
    assert q.dtype == (np.uint8 if q_mode == Q_GIVEN_FP8 else np.uint16) and q.ndim == 3
    T, H, D = q.shape
    if T == 0:
        return np.empty((0, H, 512)), np.empty((0, H))
    st, sh, sd = _strides_elems(q)
    assert sd == 1, "last axis of q must be contiguous"
    kv2 = kv.reshape(-1, kv.shape[-1])
    assert kv2.shape[1] == D and kv2.flags["C_CONTIGUOUS"]
    if kv2.dtype == np.uint16:
        kv_dtype = KV_BF16
    elif kv2.dtype == np.uint8:
        kv_dtype = KV_FP8_E4M3
    else:
        raise TypeError(f"kv must hold bf16 bits (uint16) or e4m3 codes (uint8), got {kv2.dtype}")
    assert idx.dtype == np.int32 and idx.ndim == 2 and idx.shape[0] == T
    K = idx.shape[1]
    ist, isk = _strides_elems(idx) if idx.size else (K, 1)
    if K > 0:
        assert isk == 1
    N = kv2.shape[0]
    sk = None
    if sinks is not None:
        sk = np.ascontiguousarray(np.asarray(sinks, dtype=np.float32).astype(np.float64))
        assert sk.shape == (H,)
    out = np.empty((T, H, 512), dtype=np.float64)
    lse = np.empty((T, H), dtype=np.float64)
    rc = lib.oracle_sparse_mla_fwd(
        q.ctypes.data, T, H, D, st, sh,
        kv2.ctypes.data, kv_dtype, N,
        idx.ctypes.data if idx.size else None, K, ist,
        float(np.float32(sm_scale)), float(np.float32(kv_scale)), int(q_mode),
        float(np.float32(q_scale)), sk.ctypes.data if sk is not None else None,
        out.ctypes.data, lse.ctypes.data)
    if rc != 0:
        raise RuntimeError(f"oracle_sparse_mla_fwd failed with code {rc}")
    return out, lse


def bf16_round(v: float) -> int:
    """Nearest bf16 (bits) to the real number v, ties to even."""
    return int(_load().oracle_bf16_round(float(v)))


def rope_concat_cache(ql_nope: np.ndarray, q_pe: np.ndarray, kv_c: np.ndarray, k_pe: np.ndarray,
                      positions: np.ndarray, cos_sin: np.ndarray, is_neox: bool,
                      slot_mapping: np.ndarray, kv_cache: np.ndarray, q_fp8: bool = False,
                      q_scale: float = 1.0, kv_scale: float = 1.0):
    """The fused q-RoPE / concat / cache write.  bf16 inputs as uint16 bits (any
    strides, last axis contiguous); kv_cache [N, 576] of uint16 (bf16) or uint8
    (e4m3) is copied and the copy written.  Returns (q_out [T, H, 576] uint16 or
    uint8, kv_cache_out).  Scales are rounded to fp32 as the library receives them."""
    lib = _load()
    T, H, D = ql_nope.shape
    assert D == 512 and q_pe.shape == (T, H, 64) and kv_c.shape == (T, 512) and k_pe.shape == (T, 64)
    for a in (ql_nope, q_pe, kv_c, k_pe):
        assert a.dtype == np.uint16 and a.strides[-1] == 2
    pos = np.ascontiguousarray(positions, dtype=np.int64)
    slots = np.ascontiguousarray(slot_mapping, dtype=np.int64)
    cs = np.ascontiguousarray(cos_sin, dtype=np.float32)
    assert cs.ndim == 2 and cs.shape[1] == 64
    cache = np.array(kv_cache.reshape(-1, 576), copy=True, order="C")
    kv_fp8 = cache.dtype == np.uint8
    q_out = np.zeros((T, H, 576), dtype=np.uint8 if q_fp8 else np.uint16)
    rc = lib.oracle_rope_concat_cache(
        ql_nope.ctypes.data, *_strides_elems(ql_nope)[:2], q_pe.ctypes.data, *_strides_elems(q_pe)[:2],
        kv_c.ctypes.data, _strides_elems(kv_c)[0], k_pe.ctypes.data, _strides_elems(k_pe)[0],
        pos.ctypes.data, cs.ctypes.data, cs.shape[0], int(bool(is_neox)), T, H,
        q_out.ctypes.data, int(bool(q_fp8)), float(np.float32(q_scale)),
        slots.ctypes.data, cache.ctypes.data, int(kv_fp8), cache.shape[0], float(np.float32(kv_scale)))
    if rc != 0:
        raise RuntimeError(f"oracle_rope_concat_cache failed with code {rc}")
    return q_out, cache.reshape(kv_cache.shape)
