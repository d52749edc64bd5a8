"""GPU parity: the HIP path through the C ABI against the fp64 CPU oracle.

Bar: max |out - oracle| <= 1e-2 (bf16 KV) / 6e-2 (e4m3 KV, against the oracle
that repeats the per-tile q quantisation), max |lse - oracle| <= 1e-3 on rows
with a valid entry, all-padding rows bit-exact (+0, -inf), relative L2 as a
secondary bar.  Gather/masking semantics are checked bit for bit: single
entries return that row's V exactly, invalid index spellings equal -1, and the
q quantiser reproduces the oracle's e4m3 codes exactly.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
from sparse_mla_attention_03_amd import binding, synth
from sparse_mla_attention_03_amd.binding import sparse_mla_fwd, sparse_mla_fwd_ex
from tests.helpers import (bits16, codes8, compare, kv_values_f64, oracle_for_tokens,
                           read_golden, rel_l2)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def gpu_case(**kw):
    spec = synth.small_spec(**kw)
    return synth.make_case(spec, device=DEV)


def run(case, num_splits=0, idx=None, q=None, kv_scale=None):
    out, lse = sparse_mla_fwd_ex(case.q if q is None else q, case.kv_pool,
                                 case.topk_idx if idx is None else idx, case.sm_scale,
                                 case.kv_scale if kv_scale is None else kv_scale,
                                 num_splits=num_splits)
    torch.cuda.synchronize()
    return out, lse


# ---------------------------------------------------------------- tiny config

def test_tiny_config_full_parity():
    case = synth.make_case(synth.CONFIGS["tiny_bf16"], device=DEV)
    out, lse = run(case)
    ref_out, ref_lse = oracle_for_tokens(case)
    compare(out, lse, ref_out, ref_lse, "bf16", "tiny_bf16")


# ---------------------------------------------------------------- mini sweep

MINIS = [
    # T, H, Dqk, K, ctx, kv, block_size, pad_frac
    (3, 16, 512, 100, 1024, "bf16", 64, 0.0),     # ragged tail tile
    (5, 16, 512, 300, 4096, "bf16", 64, 0.2),     # padding anywhere
    (2, 16, 576, 257, 2048, "bf16", 64, 0.1),
    (4, 32, 512, 200, 2048, "bf16", 1, 0.0),      # block size 1, 32 heads
    (2, 48, 576, 130, 1024, "bf16", 64, 0.0),     # 3 groups of 16 heads
    (2, 64, 512, 190, 1024, "bf16", 64, 0.05),
    (2, 128, 576, 321, 4096, "bf16", 64, 0.1),
    (3, 16, 512, 100, 1024, "fp8", 64, 0.0),
    (5, 16, 512, 300, 4096, "fp8", 64, 0.2),
    (2, 16, 576, 257, 2048, "fp8", 64, 0.1),
    (4, 32, 512, 200, 2048, "fp8", 1, 0.0),
    (2, 80, 576, 130, 1024, "fp8", 64, 0.0),      # q tiles of 64 + 16 heads
    (2, 128, 576, 321, 4096, "fp8", 64, 0.1),
    (1, 16, 512, 1, 64, "bf16", 64, 0.0),         # K = 1
    (7, 16, 512, 64, 256, "bf16", 64, 0.0),       # exactly one tile
    (2, 64, 512, 190, 1024, "fp8", 64, 0.05),     # 64-head groups, e4m3
    (3, 192, 512, 100, 2048, "bf16", 64, 0.0),    # three 64-head groups
    (2, 64, 576, 40, 512, "bf16", 64, 0.3),       # shorter than one tile
    (2, 128, 512, 700, 8192, "fp8", 1, 0.1),      # many tiles, block size 1
    (3, 48, 512, 333, 2048, "bf16", 64, 0.1),     # three 16-head groups, long lists
    (2, 16, 512, 2047, 4096, "bf16", 1, 0.5),     # long list, half padding, ragged tail
]


@pytest.mark.parametrize("T,H,D,K,ctx,kv,bs,pad", MINIS)
@pytest.mark.parametrize("splits", [0, 1, 3])
def test_mini_parity(T, H, D, K, ctx, kv, bs, pad, splits):
    case = gpu_case(T=T, H=H, Dqk=D, K=K, ctx=ctx, kv_dtype=kv, block_size=bs, seed=T * 7 + H + K)
    idx = case.topk_idx
    if pad > 0:
        rng = np.random.default_rng(K)
        idx = torch.from_numpy(synth.with_padding(idx.cpu().numpy(), rng, pad)).to(DEV)
    out, lse = run(case, num_splits=splits, idx=idx)
    ref_out, ref_lse = oracle_for_tokens(case, idx=idx)
    compare(out, lse, ref_out, ref_lse, kv, f"mini T{T} H{H} D{D} K{K} {kv} bs{bs} S{splits}")


# ---------------------------------------------------------------- gather / masking, bit-exact

@pytest.mark.parametrize("H", [16, 64])
@pytest.mark.parametrize("kv,D", [("bf16", 512), ("bf16", 576), ("fp8", 512), ("fp8", 576)])
def test_single_index_returns_row_exactly(kv, D, H):
    case = gpu_case(T=1, H=H, Dqk=D, K=64, ctx=512, kv_dtype=kv, block_size=64, seed=3)
    N = case.spec.N
    flat = case.kv_pool.reshape(N, D)
    for r in (0, 1, 63, 64, 65, 127, 128, 200, N - 65, N - 64, N - 1):
        for pos in (0, 37, 63):
            idx = torch.full((1, 64), -1, dtype=torch.int32, device=DEV)
            idx[0, pos] = r
            for splits in (1, 0):
                out, lse = run(case, idx=idx, num_splits=splits)
                row = flat[r, :512]
                if kv == "bf16":
                    want = row.float()
                else:
                    want = row.view(torch.float8_e4m3fn).float() * np.float32(case.kv_scale)
                want = want.to(torch.bfloat16)
                want = torch.where(want == 0, torch.zeros_like(want), want).expand(H, 512)
                assert torch.equal(out[0].view(torch.int16), want.contiguous().view(torch.int16)), (r, pos)
    # lse of the last one against the oracle
    ref_out, ref_lse = oracle_for_tokens(case, idx=idx)
    assert np.max(np.abs(lse.cpu().numpy() - ref_lse)) <= 1e-3


@pytest.mark.parametrize("H", [16, 128])
def test_all_padding_and_zero_k(H):
    case = gpu_case(T=3, H=H, K=70, ctx=512, seed=4)
    idx = torch.full((3, 70), -1, dtype=torch.int32, device=DEV)
    for splits in (0, 1, 2):
        out, lse = run(case, idx=idx, num_splits=splits)
        assert torch.all(out.view(torch.int16) == 0) and torch.all(torch.isneginf(lse))
    out, lse = run(case, idx=torch.zeros((3, 0), dtype=torch.int32, device=DEV))
    assert torch.all(out.view(torch.int16) == 0) and torch.all(torch.isneginf(lse))


def test_mixed_empty_and_full_rows():
    case = gpu_case(T=4, H=16, K=130, ctx=1024, seed=5)
    idx = case.topk_idx.clone()
    idx[1] = -1
    idx[3, 64:] = -1
    out, lse = run(case, idx=idx)
    ref_out, ref_lse = oracle_for_tokens(case, idx=idx)
    compare(out, lse, ref_out, ref_lse, "bf16", "mixed")


def test_empty_batch():
    case = gpu_case(T=2, H=16, K=8, ctx=256, seed=6)
    q = case.q[:0]
    out, lse = sparse_mla_fwd(q, case.kv_pool, case.topk_idx[:0], 0.1)
    assert out.shape == (0, 16, 512) and lse.shape == (0, 16)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_invalid_index_spellings_equal_padding(kv):
    case = gpu_case(T=4, H=16, K=200, ctx=2048, kv_dtype=kv, seed=7)
    N = case.spec.N
    idx = case.topk_idx.cpu().numpy()
    rng = np.random.default_rng(3)
    mask = rng.random(idx.shape) < 0.3
    bad = np.array([-2, np.iinfo(np.int32).min, N, N + 1, np.iinfo(np.int32).max, -1], np.int32)
    a = idx.copy()
    a[mask] = rng.choice(bad, size=int(mask.sum()))
    b = idx.copy()
    b[mask] = -1
    oa, la = run(case, idx=torch.from_numpy(a).to(DEV))
    ob, lb = run(case, idx=torch.from_numpy(b).to(DEV))
    assert torch.equal(oa.view(torch.int16), ob.view(torch.int16))
    assert torch.equal(la.view(torch.int32), lb.view(torch.int32))


def test_duplicates_count_with_multiplicity():
    case = gpu_case(T=2, H=16, K=96, ctx=1024, seed=8)
    idx = case.topk_idx.clone()
    idx[0, :] = -1
    idx[0, [3, 40, 70, 95]] = 123          # four copies, spread over two tiles
    idx[1, 10:50] = idx[1, 50:90]          # a run of duplicates among others
    out, lse = run(case, idx=idx)
    ref_out, ref_lse = oracle_for_tokens(case, idx=idx)
    compare(out, lse, ref_out, ref_lse, "bf16", "duplicates")
    flat = case.kv_pool.reshape(-1, 512)
    assert torch.equal(out[0].view(torch.int16),
                       flat[123].expand(16, 512).contiguous().view(torch.int16))


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_order_invariance(kv):
    case = gpu_case(T=4, H=16, K=256, ctx=2048, kv_dtype=kv, seed=9)
    perm = torch.stack([torch.randperm(256, generator=torch.Generator().manual_seed(t))
                        for t in range(4)]).to(DEV)
    o1, l1 = run(case)
    o2, l2 = run(case, idx=torch.gather(case.topk_idx, 1, perm))
    tol = 1e-2 if kv == "bf16" else 6e-2
    assert (o1.float() - o2.float()).abs().max().item() <= tol
    assert (l1 - l2).abs().max().item() <= 1e-4    # fp32 summation order only


def test_strided_q_equals_packed_q():
    case = gpu_case(T=5, H=16, K=200, ctx=2048, seed=10)
    big = torch.zeros((5, 40, 640), dtype=torch.bfloat16, device=DEV)
    big[:, 3:35:2, 64:576] = case.q
    qs = big[:, 3:35:2, 64:576]
    assert not qs.is_contiguous()
    o1, l1 = run(case)
    o2, l2 = run(case, q=qs)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_split_invariance_and_determinism(kv):
    case = gpu_case(T=3, H=16, K=1000, ctx=8192, kv_dtype=kv, seed=11)
    base_o, base_l = run(case, num_splits=1)
    for s in (2, 5, 16, 0):
        o, l = run(case, num_splits=s)
        assert (o.float() - base_o.float()).abs().max().item() <= 2e-3
        assert (l - base_l).abs().max().item() <= 1e-4   # fp32 summation order only
        o2, l2 = run(case, num_splits=s)
        assert torch.equal(o.view(torch.int16), o2.view(torch.int16)) and torch.equal(l, l2)


# The split merge widens its slices with the number of (token, 16-head group)
# rows: 80 rows -> 1 chunk per thread, 192 -> 2, 320 -> 4, 528 -> 8.
@pytest.mark.parametrize("T,H,kv", [(10, 128, "bf16"), (24, 128, "fp8"), (40, 128, "bf16"), (33, 256, "fp8")])
def test_merge_widths_parity(T, H, kv):
    case = gpu_case(T=T, H=H, Dqk=576, K=200, ctx=4096, kv_dtype=kv, seed=T + H)
    ref_out, ref_lse = oracle_for_tokens(case)
    for s in (2, 5):
        out, lse = run(case, num_splits=s)
        compare(out, lse, ref_out, ref_lse, kv, f"merge T{T} H{H} {kv} S{s}")


# Split partials are fp16 against a power-of-two scale per quarter row, so the
# merge must pass outputs of any magnitude through.  V is scaled by 2^e (bf16:
# the pool itself, fp8: kv_scale) and sm_scale by 2^-e: the logits are
# bit-identical, the output is the oracle's times 2^e.
@pytest.mark.parametrize("H,kv,e", [(16, "bf16", 90), (16, "bf16", -60), (128, "bf16", 100),
                                    (16, "fp8", 80), (128, "fp8", -70)])
def test_split_partials_keep_the_range(H, kv, e):
    case = gpu_case(T=5, H=H, Dqk=576 if H == 128 else 512, K=700, ctx=4096, kv_dtype=kv, seed=H + abs(e))
    f = 2.0 ** e
    if kv == "bf16":
        pool, kv_scale = (case.kv_pool.float() * f).to(torch.bfloat16), case.kv_scale
    else:
        pool, kv_scale = case.kv_pool, case.kv_scale * f
    out, lse = sparse_mla_fwd_ex(case.q, pool, case.topk_idx, case.sm_scale / f, kv_scale, num_splits=4)
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle_for_tokens(case)
    back = torch.from_numpy(out.float().cpu().numpy().astype(np.float64) / f)
    compare(back, lse, ref_out, ref_lse, kv, f"range 2^{e} H{H} {kv}")


@pytest.mark.parametrize("H,D", [(16, 512), (64, 576), (128, 512)])
@pytest.mark.parametrize("growing", [True, False])
def test_scores_that_keep_growing(H, D, growing):
    # Every head of a token gets the same q, the scale is large (scores spread
    # over ~+-35 nats) and each list is sorted by score: ascending, the running
    # max rises by far more than the online softmax's rescale threshold over
    # and over; descending, only the first tile sets it.
    case = gpu_case(T=2, H=H, Dqk=D, K=300, ctx=4096, seed=14)
    case.q = case.q[:, :1].expand(-1, H, -1).contiguous()
    case.sm_scale = 8.0 / math.sqrt(D)
    N = case.spec.N
    flat = case.kv_pool.reshape(N, D).float().cpu()
    idx = case.topk_idx.cpu().long()
    q0 = case.q[:, 0].float().cpu()
    sc = torch.einsum("tkd,td->tk", flat[idx], q0)
    order = torch.argsort(sc, dim=1, descending=not growing)
    idx = torch.gather(idx, 1, order).to(torch.int32).to(DEV)
    ref_out, ref_lse = oracle_for_tokens(case, idx=idx)
    for splits in (1, 0):
        out, lse = run(case, num_splits=splits, idx=idx)
        compare(out, lse, ref_out, ref_lse, "bf16", f"growing={growing} H{H} D{D} S{splits}")


def test_kv_scale_multiplies_non_power_of_two():
    case = gpu_case(T=3, H=16, K=150, ctx=1024, seed=12)
    case.kv_scale = 0.37
    out, lse = run(case)
    ref_out, ref_lse = oracle_for_tokens(case)
    compare(out, lse, ref_out, ref_lse, "bf16", "kv_scale 0.37")


def test_poisoned_workspace_is_not_read():
    case = gpu_case(T=2, H=16, K=1000, ctx=8192, seed=13)
    need = binding.sparse_mla_workspace_bytes(2, 16, 1000, 512, 0, 8)
    ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device=DEV)
    idx = case.topk_idx.clone()
    idx[1, 300:] = -1                     # later splits of token 1 are empty
    out, lse = sparse_mla_fwd_ex(case.q, case.kv_pool, idx, case.sm_scale, 1.0,
                                 workspace=ws, num_splits=8)
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle_for_tokens(case, idx=idx)
    compare(out, lse, ref_out, ref_lse, "bf16", "poisoned workspace")


# ---------------------------------------------------------------- e4m3 codecs on the GPU

@pytest.mark.parametrize("kv_scale", [1.0, 0.37])
def test_every_e4m3_code_decodes_exactly(kv_scale):
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    N = 256
    pool = torch.zeros((N, 512), dtype=torch.uint8)
    pool[:codes.size] = torch.from_numpy(codes)[:, None].expand(-1, 512)
    pool = pool.view(4, 64, 512).to(DEV)
    q = torch.randn((1, 16, 512), generator=torch.Generator().manual_seed(0)).to(torch.bfloat16).to(DEV)
    want = (torch.from_numpy(codes).view(torch.float8_e4m3fn).float() * np.float32(kv_scale)).to(torch.bfloat16)
    # out is a weighted sum accumulated from +0, so the code for -0 yields +0 (as in the oracle)
    want = torch.where(want == 0, torch.zeros_like(want), want)
    for i, c in enumerate(codes):
        idx = torch.full((1, 8), -1, dtype=torch.int32, device=DEV)
        idx[0, 2] = i
        out, _ = sparse_mla_fwd_ex(q, pool, idx, 0.05, kv_scale, num_splits=1)
        got = out[0].cpu()
        assert torch.all(got.view(torch.int16) == want[i].view(torch.int16)), hex(c)


def test_q_quantiser_bit_exact():
    rng = np.random.default_rng(21)
    qs = []
    x = rng.standard_normal((6, 128, 576)).astype(np.float32)
    x[1, :64] *= 1e-3
    x[2, 64:] = 0.0                                   # all-zero tile: scale 1
    x[3, :, :100] = 0.0
    x[4] *= 37.0
    x[5, 5, 5] = 1e4                                  # one dominant element
    qs.append(torch.from_numpy(x).to(torch.bfloat16))
    y = rng.standard_normal((3, 80, 512)).astype(np.float32)   # tiles of 64 and 16 heads
    qs.append(torch.from_numpy(y).to(torch.bfloat16))
    # every bf16 magnitude below the amax within one tile (exercises ties / subnormal codes)
    z = torch.arange(0, 0x4000, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
    z = z[torch.isfinite(z.float())][:16 * 512].reshape(1, 16, 512)
    z[0, 0, 0] = 448.0
    qs.append(z.contiguous())
    for q in qs:
        codes, scales = binding.sparse_mla_quantize_q_fp8(q.to(DEV))
        torch.cuda.synchronize()
        ref_codes, ref_scales = oracle.quantize_q(bits16(q))
        assert np.array_equal(scales.cpu().numpy(), ref_scales)
        assert np.array_equal(codes.cpu().numpy(), ref_codes)


# ---------------------------------------------------------------- the five workloads, full size

FULL = ["tiny_bf16", "decode_bf16", "decode_fp8", "rope_decode_bf16", "rope_decode_fp8"] + \
       [f"prefill_bf16_T{T}_K{K}" for T in (256, 512, 1024, 2048) for K in (128, 512, 2048)]


@pytest.mark.parametrize("name", FULL)
def test_full_size_parity(name):
    """Every token (decode) and every query row (prefill) of the workload at its
    full size, in the launch configuration the benchmark times (automatic
    split), against the oracle."""
    spec = synth.CONFIGS[name]
    print(f"full-size parity {name}", flush=True)
    case = synth.make_case(spec, device=DEV)
    out, lse = run(case)
    ref_out, ref_lse = oracle_for_tokens(case)
    compare(out, lse, ref_out, ref_lse, spec.kv_dtype, name)
    del case
    torch.cuda.empty_cache()


# ---------------------------------------------------------------- whole long lists, two workgroups per CU

# (head groups, K, ctx, pad_frac, sinks, strided q): enough (token, head group)
# units for two workgroups per compute unit, so whole lists of 512-wide bf16
# rows run on the kernel that holds two per unit
PREFILL16 = [
    (1, 300, 4096, 0.2, False, False),    # ragged last tile, padding anywhere
    (1, 1100, 8192, 0.0, True, True),     # sinks, strided q
    (3, 257, 2048, 0.1, True, False),     # three 16-head groups per token
    (1, 4100, 16384, 0.3, False, False),  # three rounds of entries per wave, padding dropped
    (1, 2048, 2048, 0.0, False, False),   # every slot of the pool in every list
]


@pytest.mark.parametrize("HG,K,ctx,pad,with_sinks,strided", PREFILL16)
def test_whole_lists_two_workgroups_per_cu(HG, K, ctx, pad, with_sinks, strided):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    H = 16 * HG
    T = (2 * cus + HG - 1) // HG + 5
    case = gpu_case(T=T, H=H, Dqk=512, K=K, ctx=ctx, kv_dtype="bf16", block_size=64, seed=T + K)
    assert binding.sparse_mla_num_splits(T, H, K, 512, 0, 0) == 1
    idx = case.topk_idx.cpu().numpy().copy()
    if pad > 0:
        idx = synth.with_padding(idx, np.random.default_rng(K), pad)
    N = case.spec.N
    idx[0, 0], idx[1, 1], idx[2, 5], idx[3, :] = N, -2, 2**31 - 1, -1   # invalid spellings, an empty list
    idx = torch.from_numpy(idx).to(DEV)
    q = case.q
    if strided:
        big = torch.zeros((T, H, 512 + 64), dtype=torch.bfloat16, device=DEV)
        big[:, :, :512] = case.q
        q = big[:, :, :512]
        assert q.stride(1) == 576
    sinks = _gpu_sinks(H, K) if with_sinks else None
    out, lse = sparse_mla_fwd_ex(q, case.kv_pool, idx, case.sm_scale, case.kv_scale,
                                 sinks=None if sinks is None else torch.from_numpy(sinks).to(DEV))
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle_for_tokens(case, idx=idx, sinks=sinks)
    compare(out, lse, ref_out, ref_lse, "bf16", f"whole lists T{T} H{H} K{K}")
    # the entry order the kernel works in is a function of the list: repeatable
    out2, lse2 = sparse_mla_fwd_ex(q, case.kv_pool, idx, case.sm_scale, case.kv_scale,
                                   sinks=None if sinks is None else torch.from_numpy(sinks).to(DEV))
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16)) and torch.equal(lse, lse2)


# ---------------------------------------------------------------- pools past 4 GiB

# (H, Dqk, kv, tokens, context per token): every pool is larger than 2^32 bytes,
# and its rows past byte 2^32 are named by the lists
BIG_POOLS = [
    (16, 576, "bf16", 8, 1 << 19),     # 4,194,304 rows of 1152 B: 4.83 GB
    (128, 576, "bf16", 8, 1 << 19),
    (16, 512, "fp8", 8, 9 << 17),      # 9,437,184 rows of 512 B: 4.83 GB
    (128, 576, "fp8", 8, 1 << 20),     # 8,388,608 rows of 576 B: 4.83 GB
    (32, 512, "bf16", 8, 5 << 17),     # 5,242,880 rows of 1 KiB: 5.37 GB (32-head kernel)
]


@pytest.mark.parametrize("H,D,kv,T,ctx", BIG_POOLS)
def test_pool_larger_than_4gib(H, D, kv, T, ctx):
    """Slot ids whose rows start past byte 2^32 of the pool gather those rows
    (row r sits at byte r * row_bytes, formed without 32-bit wrap-around)."""
    spec = synth.small_spec(T=T, H=H, Dqk=D, K=2048, ctx=ctx, kv_dtype=kv, mode="decode",
                            seed=H + D, sm_scale=1.0 / math.sqrt(D))
    row_bytes = D * (2 if kv == "bf16" else 1)
    N = spec.N
    assert N * row_bytes > 1 << 32
    print(f"pool past 4 GiB: H{H} D{D} {kv} N={N} ({N * row_bytes / 2**30:.2f} GiB)", flush=True)
    case = synth.make_case(spec, device=DEV)
    idx = case.topk_idx.cpu().numpy().copy()
    first_high = -(-(1 << 32) // row_bytes)            # first row that starts at or past 2^32
    rng = np.random.default_rng(H + D)
    # token 0: only rows past 2^32, including the very last one; token 1: the
    # rows just below and just above the boundary
    idx[0] = rng.choice(np.arange(first_high, N), size=idx.shape[1], replace=False)
    idx[0, 5] = N - 1
    idx[1, :8] = np.arange(first_high - 4, first_high + 4)
    high = (idx >= first_high).sum()
    assert high >= idx.shape[1], high
    idx_d = torch.from_numpy(idx).to(DEV)
    for splits in (0, 1):
        out, lse = run(case, num_splits=splits, idx=idx_d)
        ref_out, ref_lse = oracle_for_tokens(case, idx=idx_d)
        compare(out, lse, ref_out, ref_lse, kv, f"pool {N * row_bytes / 2**30:.2f} GiB H{H} D{D} {kv} S{splits}")
    # a single entry past 2^32 returns that row exactly
    flat = case.kv_pool.reshape(N, D)
    one = torch.full((1, 64), -1, dtype=torch.int32, device=DEV)
    for r in (first_high, N - 1):
        one[0, 3] = r
        o1, _ = sparse_mla_fwd_ex(case.q[:1], case.kv_pool, one, case.sm_scale, case.kv_scale,
                                  num_splits=1)
        torch.cuda.synchronize()
        row = flat[r, :512]
        want = row.float() if kv == "bf16" else row.view(torch.float8_e4m3fn).float() * np.float32(case.kv_scale)
        want = want.to(torch.bfloat16)
        want = torch.where(want == 0, torch.zeros_like(want), want).expand(H, 512)
        assert torch.equal(o1[0].view(torch.int16), want.contiguous().view(torch.int16)), r
    del case, flat
    torch.cuda.empty_cache()



def test_pool_larger_than_4gib_whole_lists():
    """The same on the kernel for whole lists of 512-wide bf16 rows with two
    workgroups per compute unit (each wave's entries ordered by slot range,
    copies from 64-bit lane addresses)."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    T, K = 2 * cus + 5, 256
    ctx = 17 << 18                                      # 4,456,448 rows of 1 KiB: 4.56 GB
    spec = synth.small_spec(T=T, H=16, Dqk=512, K=K, ctx=ctx, seed=29)
    N, row_bytes = spec.N, 1024
    assert N * row_bytes > 1 << 32
    assert binding.sparse_mla_num_splits(T, 16, K, 512, 0, 0) == 1
    print(f"pool past 4 GiB, whole lists: T{T} K{K} N={N}", flush=True)
    case = synth.make_case(spec, device=DEV)
    idx = case.topk_idx.cpu().numpy().copy()
    first_high = (1 << 32) // row_bytes
    rng = np.random.default_rng(29)
    idx[0] = rng.choice(np.arange(first_high, N), size=K, replace=False)
    idx[0, 7] = N - 1
    idx[1, :8] = np.arange(first_high - 4, first_high + 4)
    idx[2, :] = -1
    idx[2, 100] = N - 1                                 # a list whose only row is the last one
    idx_d = torch.from_numpy(idx).to(DEV)
    out, lse = run(case, idx=idx_d)
    ref_out, ref_lse = oracle_for_tokens(case, idx=idx_d)
    compare(out, lse, ref_out, ref_lse, "bf16", f"pool {N * row_bytes / 2**30:.2f} GiB, whole lists")
    row = case.kv_pool.reshape(N, 512)[N - 1].to(torch.bfloat16)
    want = torch.where(row == 0, torch.zeros_like(row), row).expand(16, 512)
    assert torch.equal(out[2].view(torch.int16), want.contiguous().view(torch.int16))
    del case
    torch.cuda.empty_cache()


# ---------------------------------------------------------------- attention sinks

def _gpu_sinks(H, seed):
    """Per-head sinks: normal logits, two heads without a sink, one dominant sink."""
    s = np.random.default_rng(seed).normal(0.0, 3.0, H).astype(np.float32)
    s[0] = -np.inf
    s[H - 1] = -np.inf
    s[H // 2] = 40.0
    return s


SINK_CASES = [
    # T, H, Dqk, K, ctx, kv, pad_frac
    (3, 16, 512, 300, 4096, "bf16", 0.2),     # 16-head kernel
    (2, 32, 512, 200, 2048, "fp8", 0.0),      # 32-head kernel
    (2, 64, 576, 190, 1024, "bf16", 0.1),     # 64-head kernel
    (2, 128, 512, 321, 4096, "fp8", 0.1),
    (2, 16, 576, 257, 2048, "fp8", 0.5),
]


@pytest.mark.parametrize("T,H,D,K,ctx,kv,pad", SINK_CASES)
@pytest.mark.parametrize("splits", [1, 0, 3])
def test_sinks_parity(T, H, D, K, ctx, kv, pad, splits):
    case = gpu_case(T=T, H=H, Dqk=D, K=K, ctx=ctx, kv_dtype=kv, block_size=64, seed=5 * T + H)
    idx = case.topk_idx
    if pad > 0:
        rng = np.random.default_rng(K + 1)
        idx = synth.with_padding(idx.cpu().numpy(), rng, pad)
        idx[0, :] = -1                       # one token with no valid entry
        idx = torch.from_numpy(idx).to(DEV)
    sinks = _gpu_sinks(H, T + K)
    out, lse = sparse_mla_fwd_ex(case.q, case.kv_pool, idx, case.sm_scale, case.kv_scale,
                                 num_splits=splits, sinks=torch.from_numpy(sinks).to(DEV))
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle_for_tokens(case, idx=idx, sinks=sinks)
    compare(out, lse, ref_out, ref_lse, kv, f"sinks T{T} H{H} D{D} {kv} S{splits}")


@pytest.mark.parametrize("H", [16, 32, 64])
@pytest.mark.parametrize("splits", [1, 2])
def test_sinks_without_entries_give_zero_and_the_sink(H, splits):
    case = gpu_case(T=2, H=H, Dqk=512, K=128, ctx=1024, seed=H)
    idx = torch.full((2, 128), -1, dtype=torch.int32, device=DEV)
    sinks = _gpu_sinks(H, 7)
    out, lse = sparse_mla_fwd_ex(case.q, case.kv_pool, idx, case.sm_scale, 1.0,
                                 num_splits=splits, sinks=torch.from_numpy(sinks).to(DEV))
    torch.cuda.synchronize()
    o = out.view(torch.int16)
    assert torch.equal(o, torch.zeros_like(o))
    l = lse.cpu().numpy()
    want = np.broadcast_to(sinks, (2, H))
    fin = np.isfinite(want)
    assert np.array_equal(np.isneginf(l), ~fin)
    assert np.max(np.abs(l[fin] - want[fin])) <= 1e-6 * 40


@pytest.mark.parametrize("H,kv", [(16, "bf16"), (32, "fp8"), (128, "bf16")])
@pytest.mark.parametrize("splits", [1, 0])
def test_sinks_of_minus_infinity_are_bitwise_no_sinks(H, kv, splits):
    case = gpu_case(T=3, H=H, Dqk=512, K=200, ctx=2048, kv_dtype=kv, seed=11)
    a = run(case, num_splits=splits)
    b = sparse_mla_fwd_ex(case.q, case.kv_pool, case.topk_idx, case.sm_scale, case.kv_scale,
                          num_splits=splits,
                          sinks=torch.full((H,), -math.inf, dtype=torch.float32, device=DEV))
    torch.cuda.synchronize()
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16))
    assert torch.equal(a[1], b[1])


# ---------------------------------------------------------------- bf16 dots on e4m3 KV

BF16_DOT_CASES = [
    # T, H, Dqk, K, ctx, pad_frac
    (3, 16, 512, 300, 4096, 0.2),     # 16-head kernel
    (2, 16, 576, 257, 2048, 0.1),
    (2, 32, 512, 200, 2048, 0.0),     # 32-head kernel
    (2, 64, 576, 190, 1024, 0.1),     # 64-head kernel
    (2, 128, 512, 321, 4096, 0.1),
    (3, 128, 576, 700, 4096, 0.1),    # 64-head kernel, several 64-row tiles per split
]


@pytest.mark.parametrize("T,H,D,K,ctx,pad", BF16_DOT_CASES)
@pytest.mark.parametrize("splits", [0, 1, 3])
def test_bf16_dots_parity(T, H, D, K, ctx, pad, splits):
    """e4m3 KV with bf16 dots against the oracle with q exact, at the bf16 bar."""
    case = gpu_case(T=T, H=H, Dqk=D, K=K, ctx=ctx, kv_dtype="fp8", block_size=64, seed=3 * T + H + D)
    idx = case.topk_idx
    if pad > 0:
        rng = np.random.default_rng(K + 2)
        idx = torch.from_numpy(synth.with_padding(idx.cpu().numpy(), rng, pad)).to(DEV)
    out, lse = sparse_mla_fwd_ex(case.q, case.kv_pool, idx, case.sm_scale, case.kv_scale,
                                 num_splits=splits, dot_precision=binding.DOTS_BF16)
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle_for_tokens(case, idx=idx, q_mode=oracle.Q_EXACT)
    compare(out, lse, ref_out, ref_lse, "bf16", f"bf16 dots T{T} H{H} D{D} S{splits}")


def test_dot_precision_errors_match_the_pages():
    """Relative L2 against exact-q attention: e4m3 dots inside the band the pages
    print for FP8 dots, bf16 dots no worse than the pages' bf16-dots figure."""
    band = {r[0]: tuple(map(float, r[1:])) for r in read_golden("pages_numerics.txt")}
    case = gpu_case(T=4, H=16, Dqk=512, K=2048, ctx=8192, kv_dtype="fp8", seed=16)
    exact, _ = oracle_for_tokens(case, q_mode=oracle.Q_EXACT)
    f8, _ = run(case)
    b16, _ = sparse_mla_fwd_ex(case.q, case.kv_pool, case.topk_idx, case.sm_scale, case.kv_scale,
                               dot_precision=binding.DOTS_BF16)
    torch.cuda.synchronize()
    lo, hi = band["fp8_dots_rel_l2"]
    e8 = rel_l2(f8.float().cpu().numpy().astype(np.float64), exact)
    eb = rel_l2(b16.float().cpu().numpy().astype(np.float64), exact)
    assert 0.5 * lo < e8 < 1.5 * hi, e8
    assert eb < 1.5 * band["bf16_dots_rel_l2"][1], eb


# ---------------------------------------------------------------- pre-quantised fp8 q

def _prequantised_q(case):
    """q quantised with one per-tensor scale: OCP e4m3 codes (uint8) and the scale."""
    q = case.q.float()
    q_scale = float(np.float32(q.abs().max().item() / 448.0))
    codes = (q / q_scale).to(torch.float8_e4m3fn).view(torch.uint8).contiguous()
    return codes, q_scale


PREQ_CASES = [
    # T, H, Dqk, K, ctx, pad_frac
    (3, 16, 512, 300, 4096, 0.2),     # 16-head kernel
    (2, 16, 576, 257, 2048, 0.1),
    (2, 32, 512, 200, 2048, 0.0),     # 32-head kernel
    (2, 64, 576, 190, 1024, 0.1),     # 64-head kernel
    (2, 128, 512, 321, 4096, 0.1),
]


@pytest.mark.parametrize("T,H,D,K,ctx,pad", PREQ_CASES)
@pytest.mark.parametrize("splits", [0, 1, 3])
def test_prequantised_q_parity(T, H, D, K, ctx, pad, splits):
    case = gpu_case(T=T, H=H, Dqk=D, K=K, ctx=ctx, kv_dtype="fp8", block_size=64, seed=7 * T + H + D)
    idx = case.topk_idx
    if pad > 0:
        rng = np.random.default_rng(K + 3)
        idx = torch.from_numpy(synth.with_padding(idx.cpu().numpy(), rng, pad)).to(DEV)
    codes, q_scale = _prequantised_q(case)
    out, lse = sparse_mla_fwd_ex(codes, case.kv_pool, idx, case.sm_scale, case.kv_scale,
                                 num_splits=splits, q_scale=q_scale)
    torch.cuda.synchronize()
    # the oracle on the rows these tokens use, with q given as codes
    idx_np = idx.cpu().numpy()
    N = case.kv_pool.shape[0] * case.kv_pool.shape[1]
    valid = (idx_np >= 0) & (idx_np < N)
    rows = np.unique(idx_np[valid]).astype(np.int64)
    remap = np.full(idx_np.shape, -1, dtype=np.int32)
    remap[valid] = np.searchsorted(rows, idx_np[valid]).astype(np.int32)
    sub = case.kv_pool.reshape(N, D)[torch.from_numpy(rows).to(DEV)].cpu()
    ref_out, ref_lse = oracle.sparse_mla_fwd(codes.cpu().numpy(), codes8(sub), remap, case.sm_scale,
                                             case.kv_scale, q_mode=oracle.Q_GIVEN_FP8, q_scale=q_scale)
    compare(out, lse, ref_out, ref_lse, "fp8", f"pre-quantised q T{T} H{H} D{D} S{splits}")


@pytest.mark.parametrize("H", [16, 32, 64])
@pytest.mark.parametrize("D", [512, 576])
def test_prequantised_q_from_the_quantiser_is_bitwise_the_default_path(H, D):
    # one token, H <= 64: one quantisation tile, so its codes and scale as
    # pre-quantised q must reproduce the default (in-kernel quantisation) path
    case = gpu_case(T=1, H=H, Dqk=D, K=300, ctx=2048, kv_dtype="fp8", seed=H + D)
    codes, scales = binding.sparse_mla_quantize_q_fp8(case.q)
    torch.cuda.synchronize()
    for splits in (1, 0):
        a = run(case, num_splits=splits)
        b = sparse_mla_fwd_ex(codes, case.kv_pool, case.topk_idx, case.sm_scale, case.kv_scale,
                              num_splits=splits, q_scale=float(scales[0, 0].item()))
        torch.cuda.synchronize()
        assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16)), splits
        assert torch.equal(a[1], b[1]), splits
