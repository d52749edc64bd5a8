"""GPU parity of the fused q-RoPE / q-concat / KV-concat / cache write against the
fp64 oracle: bit for bit (every output is a bf16 pattern or an e4m3 code that
both sides decide from the same exactly-rounded value), for both pair layouts,
16 and 128 heads, block sizes 1 and 64, bf16 and e4m3 outputs with non-unit
scales, skipped slots and a strided (heads-outermost) ql_nope.
"""
from __future__ import annotations

from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
from sparse_mla_attention_03_amd import binding, synth
from tests.helpers import bits16

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _gpu(case):
    return synth.RopeCase(case.ql_nope.to(DEV), case.q_pe.to(DEV), case.kv_c.to(DEV), case.k_pe.to(DEV),
                          case.positions.to(DEV), case.cos_sin.to(DEV), case.slot_mapping.to(DEV),
                          case.num_blocks, case.block_size)


def _cache(case, kv_fp8):
    # a recognisable fill, so rows that must stay untouched are checked too
    N = case.num_blocks * case.block_size
    fill = np.full((N, 576), 0x3C, dtype=np.uint8) if kv_fp8 else np.full((N, 576), 0x3F80, dtype=np.uint16)
    return fill.reshape(case.num_blocks, case.block_size, 576)


def _check(case, is_neox, q_fp8, kv_fp8, q_scale, kv_scale, ql_gpu=None):
    g = _gpu(case)
    fill = _cache(case, kv_fp8)
    if kv_fp8:
        cache = torch.from_numpy(fill.copy()).to(DEV)
    else:
        cache = torch.from_numpy(fill.view(np.int16).copy()).to(DEV).view(torch.bfloat16)
    q_out = binding.sparse_mla_rope_concat_cache(
        g.ql_nope if ql_gpu is None else ql_gpu, g.q_pe, g.kv_c, g.k_pe, g.positions, g.cos_sin,
        is_neox, g.slot_mapping, cache, q_fp8=q_fp8, q_scale=q_scale, kv_scale=kv_scale)
    torch.cuda.synchronize()
    want_q, want_c = oracle.rope_concat_cache(
        bits16(case.ql_nope), bits16(case.q_pe), bits16(case.kv_c), bits16(case.k_pe),
        case.positions.numpy(), case.cos_sin.numpy(), is_neox, case.slot_mapping.numpy(), fill,
        q_fp8=q_fp8, q_scale=q_scale, kv_scale=kv_scale)
    got_q = q_out.cpu().view(torch.uint8 if q_fp8 else torch.int16).numpy().view(want_q.dtype)
    got_c = cache.cpu().view(torch.uint8 if kv_fp8 else torch.int16).numpy().view(want_c.dtype)
    assert np.array_equal(got_q, want_q), int((got_q != want_q).sum())
    assert np.array_equal(got_c, want_c), int((got_c != want_c).sum())


@pytest.mark.parametrize("is_neox", [True, False])
@pytest.mark.parametrize("H", [16, 128])
@pytest.mark.parametrize("bs", [1, 64])
@pytest.mark.parametrize("q_fp8,kv_fp8", [(False, False), (True, True), (False, True)])
def test_fused_rope_cache_bitwise(is_neox, H, bs, q_fp8, kv_fp8):
    nb = 512 // bs
    case = synth.make_rope_case(T=37, H=H, num_blocks=nb, block_size=bs, max_pos=4096,
                                seed=H + bs + int(is_neox), skip_frac=0.15)
    _check(case, is_neox, q_fp8, kv_fp8, q_scale=0.37, kv_scale=0.59)


@pytest.mark.parametrize("is_neox", [True, False])
def test_fused_rope_cache_strided_ql_nope(is_neox):
    # the production layout: ql_nope is the output of a per-head bmm, stored
    # heads-outermost and seen as [T, H, 512] through a transpose
    case = synth.make_rope_case(T=29, H=16, num_blocks=8, block_size=64, seed=9)
    heads_major = case.ql_nope.transpose(0, 1).contiguous().to(DEV)     # [H, T, 512]
    ql = heads_major.transpose(0, 1)                                    # strided view
    assert not ql.is_contiguous()
    _check(case, is_neox, True, True, q_scale=0.37, kv_scale=0.59, ql_gpu=ql)


def test_fused_outputs_feed_the_forward_pass():
    """The fused op's e4m3 q and cache, fed to sparse_mla_fwd as pre-quantised q
    over that pool, against the oracle run on the oracle's own fused outputs."""
    T, H, nb, bs = 8, 16, 64, 64
    case = synth.make_rope_case(T=T, H=H, num_blocks=nb, block_size=bs, max_pos=4096, seed=21)
    # every slot written once: the first T slots come from the op, the rest from a second batch
    N = nb * bs
    extra = synth.make_rope_case(T=N, H=1, num_blocks=nb, block_size=bs, max_pos=4096, seed=22)
    g, ge = _gpu(case), _gpu(extra)
    q_scale, kv_scale = 0.02, 0.011
    cache = torch.zeros((nb, bs, 576), dtype=torch.uint8, device=DEV)
    binding.sparse_mla_rope_concat_cache(ge.ql_nope, ge.q_pe, ge.kv_c, ge.k_pe, ge.positions, ge.cos_sin,
                                         True, ge.slot_mapping, cache, q_fp8=True, q_scale=q_scale,
                                         kv_scale=kv_scale)
    q8 = binding.sparse_mla_rope_concat_cache(g.ql_nope, g.q_pe, g.kv_c, g.k_pe, g.positions, g.cos_sin,
                                              True, g.slot_mapping, cache, q_fp8=True, q_scale=q_scale,
                                              kv_scale=kv_scale)
    torch.cuda.synchronize()
    # the oracle's own fused outputs, in the same order
    c0 = np.zeros((nb, bs, 576), np.uint8)
    _, c1 = oracle.rope_concat_cache(bits16(extra.ql_nope), bits16(extra.q_pe), bits16(extra.kv_c),
                                     bits16(extra.k_pe), extra.positions.numpy(), extra.cos_sin.numpy(),
                                     True, extra.slot_mapping.numpy(), c0, q_fp8=True, q_scale=q_scale,
                                     kv_scale=kv_scale)
    oq, c2 = oracle.rope_concat_cache(bits16(case.ql_nope), bits16(case.q_pe), bits16(case.kv_c),
                                      bits16(case.k_pe), case.positions.numpy(), case.cos_sin.numpy(),
                                      True, case.slot_mapping.numpy(), c1, q_fp8=True, q_scale=q_scale,
                                      kv_scale=kv_scale)
    assert np.array_equal(cache.cpu().numpy(), c2) and np.array_equal(q8.cpu().numpy(), oq)
    rng = np.random.default_rng(5)
    idx = np.stack([rng.choice(N, 600, replace=False) for _ in range(T)]).astype(np.int32)
    out, lse = binding.sparse_mla_fwd_ex(q8, cache, torch.from_numpy(idx).to(DEV), 1.0 / 24.0, kv_scale,
                                         q_scale=q_scale)
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle.sparse_mla_fwd(oq, c2.reshape(N, 576), idx, 1.0 / 24.0, kv_scale,
                                             q_mode=oracle.Q_GIVEN_FP8, q_scale=q_scale)
    assert np.max(np.abs(out.float().cpu().numpy() - ref_out)) <= 6e-2
    assert np.max(np.abs(lse.cpu().numpy() - ref_lse)) <= 1e-3


# bf16 bit patterns of the edge-value test: zeros, small integers, the largest
# finite bf16, the smallest normal one and 2^-100 (so that products reach the
# subnormal range), and a value one step above 1
_EDGE_BF16 = np.array([0x0000, 0x8000, 0x3F80, 0xBF80, 0x4000, 0xC000, 0x4040, 0x3F81, 0x0D80, 0x0080,
                       0x7F7F, 0xFF7F, 0x3F00, 0x2180, 0xA180], dtype=np.uint16)


def _edge_table():
    """A rotary table whose rows are chosen so that outputs land on the cases the
    bf16 rounding has to get right: exact bf16 midpoints with a tiny second
    product pushing them either way (or not at all), subnormal and underflowing
    outputs, overflow to infinity, exact zeros, and plain angles."""
    cs = np.empty((9, 64), np.float32)
    rows = [(1.0, 0.0), (0.5 + 2.0 ** -9, 2.0 ** -40), (2.0 ** -30, 2.0 ** -31), (0.75, 0.75),
            None, (1.0 - 2.0 ** -24, 2.0 ** -12), (0.0, 1.0), (0.999, -0.0447), (511.0 / 512.0, 0.5)]
    real = synth.rope_cos_sin(4096)[1234]
    for p, r in enumerate(rows):
        if r is None:
            cs[p] = real
        else:
            cs[p, :32], cs[p, 32:] = r
    return cs


@pytest.mark.parametrize("is_neox", [True, False])
@pytest.mark.parametrize("q_fp8,kv_fp8", [(False, False), (True, True)])
def test_fused_rope_cache_rounding_edge_values(is_neox, q_fp8, kv_fp8):
    T, H = 64, 16
    case = synth.make_rope_case(T=T, H=H, num_blocks=2, block_size=64, seed=31)
    rng = np.random.default_rng(32)

    def edge(shape):
        bits = _EDGE_BF16[rng.integers(0, len(_EDGE_BF16), size=shape)]
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)

    case = replace(case, q_pe=edge((T, H, 64)), k_pe=edge((T, 64)),
                   positions=torch.arange(T, dtype=torch.int64) % 9,
                   cos_sin=torch.from_numpy(_edge_table()))
    _check(case, is_neox, q_fp8, kv_fp8, q_scale=1.0, kv_scale=1.0)


@pytest.mark.parametrize("is_neox", [True, False])
def test_fused_rope_cache_midpoint_pushed_by_a_tiny_product(is_neox):
    """x cos on a bf16 midpoint (x = 1, cos = 511/512) with y sin = +-2^-61 or 0
    beside it: the exact value rounds to 0x3F7F, 0x3F80 and (the tie) 0x3F80,
    which the oracle returns; rounding to fp64 first gives 0x3F80 every time."""
    T, H = 4, 16
    case = synth.make_rope_case(T=T, H=H, num_blocks=1, block_size=64, seed=33)
    ys = (0x2180, 0xA180, 0x0000)
    qp = np.zeros((T, H, 64), np.uint16)
    kp = np.zeros((T, 64), np.uint16)
    for i in range(32):
        ix, iy = (i, i + 32) if is_neox else (2 * i, 2 * i + 1)
        qp[..., ix], kp[:, ix] = 0x3F80, 0x3F80
        qp[..., iy], kp[:, iy] = ys[i % 3], ys[(i + 1) % 3]
    cs = np.zeros((1, 64), np.float32)
    cs[:, :32], cs[:, 32:] = 511.0 / 512.0, 0.5
    bf = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    case = replace(case, q_pe=bf(qp), k_pe=bf(kp), positions=torch.zeros(T, dtype=torch.int64),
                   cos_sin=torch.from_numpy(cs))
    _check(case, is_neox, False, False, q_scale=1.0, kv_scale=1.0)


@pytest.mark.parametrize("q_fp8,kv_fp8", [(False, False), (True, True)])
def test_fused_rope_cache_large_call(q_fp8, kv_fp8):
    # 2900 tokens x 17 rows = 49300 rows: past the size from which the kernel
    # interleaves its two kinds of wave, with a ragged last group
    case = synth.make_rope_case(T=2900, H=16, num_blocks=64, block_size=64, max_pos=8192, seed=41,
                                skip_frac=0.05)
    _check(case, True, q_fp8, kv_fp8, q_scale=0.37, kv_scale=0.59)


@pytest.mark.parametrize("scale", [0.37, 1.0, 3.0, 1.0000001, 2.0 ** -64, 2.0 ** 64, 2.0 ** -65, 2.0 ** 65])
def test_fused_rope_cache_e4m3_every_bf16_input(scale):
    """Every finite and infinite bf16 pattern as a latent input of a q row and of a
    cache row, quantised to e4m3 against scales inside, at the ends of and
    outside the range where the kernel forms value / scale without a division.
    (NaN patterns are replaced by zero: NaN inputs are outside what the op
    defines.)"""
    T, H = 128, 1
    case = synth.make_rope_case(T=T, H=H, num_blocks=4, block_size=64, seed=51)
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    nan = ((bits & 0x7F80) == 0x7F80) & ((bits & 0x7F) != 0)
    bits[nan] = 0
    rng = np.random.default_rng(52)
    q_bits, kv_bits = rng.permutation(bits), rng.permutation(bits)

    def bf(b, shape):
        return torch.from_numpy(b.view(np.int16).reshape(shape).copy()).view(torch.bfloat16)

    case = replace(case, ql_nope=bf(q_bits, (T, H, 512)), kv_c=bf(kv_bits, (T, 512)))
    _check(case, True, True, True, q_scale=scale, kv_scale=scale)
