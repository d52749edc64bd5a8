"""Small helpers shared by the test modules (no attention arithmetic here)."""
from __future__ import annotations

import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def bits16(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor (any strides) -> numpy uint16 view of its bits, same strides."""
    assert t.dtype == torch.bfloat16
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def codes8(t: torch.Tensor) -> np.ndarray:
    """uint8 / float8 tensor -> numpy uint8 codes."""
    if t.dtype != torch.uint8:
        t = t.view(torch.uint8)
    return t.detach().cpu().numpy()


def kv_bits(pool: torch.Tensor) -> np.ndarray:
    """KV pool [blocks, block_size, D] -> flat [N, D] numpy bits (uint16 or uint8)."""
    flat = pool.reshape(-1, pool.shape[-1]).cpu()
    return bits16(flat) if flat.dtype == torch.bfloat16 else codes8(flat)


def kv_values_f64(pool: torch.Tensor, kv_scale: float) -> np.ndarray:
    """Dequantised pool values in fp64 via torch's own dtype conversions."""
    flat = pool.reshape(-1, pool.shape[-1]).cpu()
    if flat.dtype == torch.uint8:
        flat = flat.view(torch.float8_e4m3fn)
    return flat.to(torch.float64).numpy() * float(np.float32(kv_scale))


def read_golden(name: str) -> list[list[str]]:
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def rel_l2(a: np.ndarray, b: np.ndarray) -> float:
    return float(np.linalg.norm((a - b).ravel()) / np.linalg.norm(b.ravel()))


# ---------------------------------------------------------------- GPU vs oracle

TOL_OUT = {"bf16": 1e-2, "fp8": 6e-2}     # max |out - oracle|
TOL_LSE = 1e-3                             # max |lse - oracle| on rows with a valid entry
TOL_REL_L2 = {"bf16": 5e-3, "fp8": 1e-2}   # secondary: relative L2 of out


def oracle_for_tokens(case, tokens=None, q_mode=None, idx=None, sinks=None):
    """Oracle result for a subset of tokens, gathering only the rows they use.

    The rows named by the selected tokens' lists are copied to the host, the
    lists are remapped to a compact pool (entries outside [0, N) stay padding),
    and the fp64 oracle runs on that.  Returns (out [n,H,512], lse [n,H])."""
    import oracle
    idx_all = (case.topk_idx if idx is None else idx).cpu().numpy()
    T = idx_all.shape[0]
    tok = np.arange(T) if tokens is None else np.asarray(tokens)
    sel = idx_all[tok]
    N = case.kv_pool.shape[0] * case.kv_pool.shape[1]
    valid = (sel >= 0) & (sel < N)
    rows = np.unique(sel[valid]).astype(np.int64)
    remap = np.full(sel.shape, -1, dtype=np.int32)
    remap[valid] = np.searchsorted(rows, sel[valid]).astype(np.int32)
    flat = case.kv_pool.reshape(-1, case.kv_pool.shape[-1])
    if rows.size:
        sub = flat[torch.from_numpy(rows).to(flat.device)].cpu()
    else:
        sub = flat[:1].cpu()
    kv = bits16(sub) if sub.dtype == torch.bfloat16 else codes8(sub)
    q = bits16(case.q.cpu()[torch.from_numpy(tok)])
    if q_mode is None:
        q_mode = oracle.Q_TILE_FP8
    return oracle.sparse_mla_fwd(np.ascontiguousarray(q), np.ascontiguousarray(kv),
                                 np.ascontiguousarray(remap), case.sm_scale, case.kv_scale,
                                 q_mode=q_mode, sinks=sinks)


def compare(out, lse, ref_out, ref_lse, kv_dtype, what=""):
    """Assert the GPU result meets the parity bar against the oracle."""
    o = out.float().cpu().numpy().astype(np.float64)
    l = lse.float().cpu().numpy().astype(np.float64)
    assert o.shape == ref_out.shape and l.shape == ref_lse.shape
    empty = np.isneginf(ref_lse)
    # rows with no valid entry: exactly +0 output, -inf lse
    assert np.all(np.isneginf(l[empty])), f"{what}: lse of empty rows"
    assert np.all(o[empty] == 0) and not np.any(np.signbit(o[empty])), f"{what}: out of empty rows"
    assert np.all(np.isfinite(l[~empty])) and np.all(np.isfinite(o)), f"{what}: non-finite"
    err_out = float(np.max(np.abs(o - ref_out))) if o.size else 0.0
    err_lse = float(np.max(np.abs(l[~empty] - ref_lse[~empty]))) if (~empty).any() else 0.0
    rel = rel_l2(o[~empty], ref_out[~empty]) if (~empty).any() else 0.0
    assert err_out <= TOL_OUT[kv_dtype], f"{what}: max |out err| {err_out}"
    assert err_lse <= TOL_LSE, f"{what}: max |lse err| {err_lse}"
    assert rel <= TOL_REL_L2[kv_dtype], f"{what}: rel L2 {rel}"
    return err_out, err_lse, rel
