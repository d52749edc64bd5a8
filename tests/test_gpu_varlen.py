"""GPU parity of the per-token-length forward pass (sparse_mla_fwd_varlen) against
the fp64 oracle on the same lists cut at each token's length.

Entries past a token's length are filled with the slot of a poisoned pool row
(NaN everywhere): reading any of them would turn that token's output into NaN,
so the tests also show they are never read.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from sparse_mla_attention_03_amd import binding, synth
from tests.helpers import compare, oracle_for_tokens

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _mixed_case(T, H, D, K, ctx, kv, seed):
    spec = synth.small_spec(T=T, H=H, Dqk=D, K=K, ctx=ctx, kv_dtype=kv, block_size=64, seed=seed)
    case = synth.make_case(spec, device=DEV)
    N = spec.N
    rng = np.random.default_rng(seed)
    # lengths: empty, tiny, tile boundaries, long, full
    base = [0, 1, 63, 64, 65, 300, K, K - 1]
    lens = np.array([base[i] if i < len(base) else int(rng.integers(0, K + 1)) for i in range(T)], np.int32)
    lens = np.minimum(lens, K)
    idx = case.topk_idx.cpu().numpy().copy()
    poison = int(idx.max()) + 1 if int(idx.max()) + 1 < N else 0
    # the poisoned row must not be one any token uses
    used = set(idx[idx >= 0].tolist())
    while poison in used:
        poison = (poison + 1) % N
    for t in range(T):
        idx[t, lens[t]:] = poison
    flat = case.kv_pool.view(N, D)
    if kv == "bf16":
        flat[poison].view(torch.int16).fill_(0x7FC0)      # bf16 NaN
    else:
        flat[poison].fill_(0x7F)                          # e4m3 NaN
    cut = idx.copy()
    for t in range(T):
        cut[t, lens[t]:] = -1
    return case, torch.from_numpy(idx).to(DEV), torch.from_numpy(lens).to(DEV), torch.from_numpy(cut).to(DEV)


VARLEN_CASES = [
    # T, H, Dqk, K, ctx, kv
    (12, 16, 512, 700, 4096, "bf16"),    # 16-head kernel
    (10, 16, 576, 2048, 8192, "fp8"),
    (9, 32, 512, 300, 2048, "fp8"),      # 32-head kernel
    (9, 64, 576, 520, 2048, "bf16"),     # 64 heads, as two 32-head groups
    (8, 128, 512, 1100, 4096, "fp8"),
    (24, 128, 576, 400, 4096, "bf16"),   # 192 (token, 16-head) rows: the merge's 2-chunk slices
    (40, 128, 512, 300, 2048, "fp8"),    # 320 rows: 4-chunk slices
]


@pytest.mark.parametrize("T,H,D,K,ctx,kv", VARLEN_CASES)
def test_varlen_parity_and_no_reads_past_the_length(T, H, D, K, ctx, kv):
    case, idx, lens, cut = _mixed_case(T, H, D, K, ctx, kv, seed=T + H + K)
    out, lse = binding.sparse_mla_fwd_varlen(case.q, case.kv_pool, idx, lens, case.sm_scale, case.kv_scale)
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle_for_tokens(case, idx=cut)
    compare(out, lse, ref_out, ref_lse, kv, f"varlen T{T} H{H} D{D} K{K} {kv}")


def test_varlen_with_sinks_prequantised_q_and_bf16_dots():
    T, H, D, K = 10, 16, 512, 900
    case, idx, lens, cut = _mixed_case(T, H, D, K, 4096, "fp8", seed=77)
    sinks = np.random.default_rng(3).normal(0, 2, H).astype(np.float32)
    sinks[0] = -np.inf
    out, lse = binding.sparse_mla_fwd_varlen(case.q, case.kv_pool, idx, lens, case.sm_scale, case.kv_scale,
                                             sinks=torch.from_numpy(sinks).to(DEV))
    torch.cuda.synchronize()
    ref = oracle_for_tokens(case, idx=cut, sinks=sinks)
    compare(out, lse, ref[0], ref[1], "fp8", "varlen + sinks")
    out, lse = binding.sparse_mla_fwd_varlen(case.q, case.kv_pool, idx, lens, case.sm_scale, case.kv_scale,
                                             dot_precision=binding.DOTS_BF16)
    torch.cuda.synchronize()
    ref = oracle_for_tokens(case, idx=cut, q_mode=oracle.Q_EXACT)
    compare(out, lse, ref[0], ref[1], "bf16", "varlen + bf16 dots")
    codes, scales = binding.sparse_mla_quantize_q_fp8(case.q[:1])
    torch.cuda.synchronize()
    # one token's codes as pre-quantised q: equals the default path on that token
    a = binding.sparse_mla_fwd_varlen(case.q[:1], case.kv_pool, idx[:1], lens[:1], case.sm_scale, case.kv_scale)
    b = binding.sparse_mla_fwd_varlen(codes, case.kv_pool, idx[:1], lens[:1], case.sm_scale, case.kv_scale,
                                      q_scale=float(scales[0, 0].item()))
    torch.cuda.synchronize()
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16)) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("H,D", [(32, 512), (64, 576), (128, 512)])
def test_varlen_bf16_dots_in_the_wide_kernels(H, D):
    T, K = 9, 600
    case, idx, lens, cut = _mixed_case(T, H, D, K, 4096, "fp8", seed=H + D)
    out, lse = binding.sparse_mla_fwd_varlen(case.q, case.kv_pool, idx, lens, case.sm_scale, case.kv_scale,
                                             dot_precision=binding.DOTS_BF16)
    torch.cuda.synchronize()
    ref = oracle_for_tokens(case, idx=cut, q_mode=oracle.Q_EXACT)
    compare(out, lse, ref[0], ref[1], "bf16", f"varlen bf16 dots H{H} D{D}")


@pytest.mark.parametrize("H", [16, 64])
def test_varlen_full_lengths_match_the_padded_call(H):
    # every length = K: the same result as the ordinary call up to summation order
    case = synth.make_case(synth.small_spec(T=6, H=H, Dqk=512, K=1500, ctx=8192, seed=H), device=DEV)
    lens = torch.full((6,), 1500, dtype=torch.int32, device=DEV)
    a = binding.sparse_mla_fwd(case.q, case.kv_pool, case.topk_idx, case.sm_scale)
    b = binding.sparse_mla_fwd_varlen(case.q, case.kv_pool, case.topk_idx, lens, case.sm_scale)
    torch.cuda.synchronize()
    assert (a[0].float() - b[0].float()).abs().max().item() <= 1e-2
    assert (a[1] - b[1]).abs().max().item() <= 1e-4
    ref_out, ref_lse = oracle_for_tokens(case)
    compare(b[0], b[1], ref_out, ref_lse, "bf16", f"varlen full H{H}")


def test_varlen_all_empty():
    case = synth.make_case(synth.small_spec(T=3, H=16, Dqk=512, K=64, ctx=1024, seed=2), device=DEV)
    lens = torch.zeros(3, dtype=torch.int32, device=DEV)
    out, lse = binding.sparse_mla_fwd_varlen(case.q, case.kv_pool, case.topk_idx, lens, case.sm_scale)
    torch.cuda.synchronize()
    o = out.view(torch.int16)
    assert torch.equal(o, torch.zeros_like(o)) and bool(torch.isneginf(lse).all())


def test_dropped_plan_units_turn_every_output_nan(monkeypatch):
    """The plan's unit table is sized past what its unit length can produce, so
    no unit is ever dropped.  Forced smaller from the host, the dropped units
    must show: every output and lse of the call is NaN, not stale memory."""
    T, H, D, K = 12, 16, 512, 700
    case, idx, lens, _ = _mixed_case(T, H, D, K, 4096, "bf16", seed=5)
    out = torch.zeros(T, H, 512, dtype=torch.bfloat16, device=DEV)
    lse = torch.zeros(T, H, dtype=torch.float32, device=DEV)
    monkeypatch.setenv("SPARSEMLA_TEST_UNIT_TABLE", "3")
    binding.sparse_mla_fwd_varlen(case.q, case.kv_pool, idx, lens, case.sm_scale, case.kv_scale, out=out, lse=lse)
    torch.cuda.synchronize()
    assert bool(torch.isnan(out.float()).all()) and bool(torch.isnan(lse).all())
    # the same call with the table at its size: finite again
    monkeypatch.delenv("SPARSEMLA_TEST_UNIT_TABLE")
    binding.sparse_mla_fwd_varlen(case.q, case.kv_pool, idx, lens, case.sm_scale, case.kv_scale, out=out, lse=lse)
    torch.cuda.synchronize()
    assert not bool(torch.isnan(out.float()).any())
