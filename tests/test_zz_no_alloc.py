"""GPU: the allocation-free entry point against the entry point with a workspace.

sparse_mla_fwd_noalloc runs the same kernels as sparse_mla_fwd_ex with the
split partials in the library's per-device scratch array, so with the same
split count its results must be bit-identical.  Two calls in a row (the second
smaller) check that the scratch keeps no state that matters between calls.
"""
from __future__ import annotations

import pytest
import torch

from sparse_mla_attention_03_amd import binding, synth
from sparse_mla_attention_03_amd.binding import sparse_mla_fwd_ex, sparse_mla_fwd_noalloc
from tests.helpers import compare, oracle_for_tokens

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _same(a, b):
    return torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b)


# (T, H, Dqk, K, ctx, kv): a split decode shape first, then a smaller one
PAIRS = [
    ((32, 16, 512, 2048, 16384, "bf16"), (5, 16, 512, 300, 4096, "bf16")),
    ((64, 128, 576, 2048, 8192, "fp8"), (3, 64, 576, 700, 2048, "fp8")),
    ((16, 128, 576, 2048, 8192, "bf16"), (2, 32, 512, 500, 2048, "bf16")),
]


@pytest.mark.parametrize("first,second", PAIRS)
def test_noalloc_matches_the_workspace_entry_point(first, second):
    for n, (T, H, D, K, ctx, kv) in enumerate((first, second)):
        print(f"noalloc call {n}: T{T} H{H} D{D} K{K} {kv}", flush=True)
        spec = synth.small_spec(T=T, H=H, Dqk=D, K=K, ctx=ctx, kv_dtype=kv, mode="decode",
                                seed=T + H + n, sm_scale=1.0 / D ** 0.5)
        case = synth.make_case(spec, device=DEV)
        kvd = 0 if kv == "bf16" else 1
        S = binding.sparse_mla_num_splits(T, H, K, D, kvd, 0)
        if S * T * H * 1044 > binding.NOALLOC_SCRATCH_BYTES:
            # the automatic choice does not fit the scratch: the entry point runs the count that does
            S = max(binding.NOALLOC_SCRATCH_BYTES // (T * H * 1044), 1)
        out = torch.full((T, H, 512), float("nan"), dtype=torch.bfloat16, device=DEV)
        lse = torch.full((T, H), float("nan"), dtype=torch.float32, device=DEV)
        sparse_mla_fwd_noalloc(case.q, case.kv_pool, case.topk_idx, case.sm_scale, case.kv_scale,
                               out=out, lse=lse)
        torch.cuda.synchronize()
        ref_o, ref_l = sparse_mla_fwd_ex(case.q, case.kv_pool, case.topk_idx, case.sm_scale,
                                         case.kv_scale, num_splits=S)
        torch.cuda.synchronize()
        assert _same(out, ref_o) and _same(lse, ref_l), (n, S)
        # and the oracle's bar, as for every entry point
        o_ref, l_ref = oracle_for_tokens(case)
        compare(out, lse, o_ref, l_ref, kv, f"noalloc call {n}")
        if n == 0:
            assert S > 1, "the first call must use the scratch"


def test_noalloc_caps_its_split_choice_to_the_scratch():
    """85 tokens x 192 heads: the automatic choice (2 splits) needs 34 MB of
    partials, more than the scratch holds, so the entry point runs the split
    count that fits (1), with the same result as the workspace entry point at it."""
    T, H, D, K = 85, 192, 512, 2048
    kvd = 0
    S_auto = binding.sparse_mla_num_splits(T, H, K, D, kvd, 0)
    cap = binding.NOALLOC_SCRATCH_BYTES // (T * H * 1044)
    if S_auto * T * H * 1044 <= binding.NOALLOC_SCRATCH_BYTES:
        pytest.skip(f"the automatic choice ({S_auto} splits) fits this device's scratch")
    print(f"noalloc capped: T{T} H{H} auto {S_auto} -> {max(cap, 1)}", flush=True)
    spec = synth.small_spec(T=T, H=H, Dqk=D, K=K, ctx=4096, mode="decode", seed=11)
    case = synth.make_case(spec, device=DEV)
    out, lse = sparse_mla_fwd_noalloc(case.q, case.kv_pool, case.topk_idx, case.sm_scale, case.kv_scale)
    ref_o, ref_l = sparse_mla_fwd_ex(case.q, case.kv_pool, case.topk_idx, case.sm_scale,
                                     case.kv_scale, num_splits=max(cap, 1))
    torch.cuda.synchronize()
    assert _same(out, ref_o) and _same(lse, ref_l)
