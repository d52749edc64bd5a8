"""Seeded synthetic inputs for the sparse MLA forward pass.

This module only draws random numbers and lays them out; it holds none of the
attention arithmetic, so both the HIP path and the CPU oracle can consume what
it produces.

Layout of a case (all shapes as the library sees them):
  q         bf16  [T, H, Dqk]                ~ N(0, 1)
  kv_pool   bf16  [num_blocks, block_size, Dqk]   ~ N(0, 1)
            or uint8 OCP e4m3 codes of kv / kv_scale, kv_scale = amax / 448
  topk_idx  int32 [T, K]   flat slot ids into kv_pool viewed as [N, Dqk]
                           (N = num_blocks * block_size); -1 = padding

Paging: a sequence owns a list of physical blocks (a block table drawn as one
random permutation of all blocks); logical position p of that sequence lives in
slot  table[p // block_size] * block_size + p % block_size.  The kernel never
sees the table: the top-k list already holds slot ids (one shared KV pool).

Modes for picking each token's top-k positions:
  shared   every token draws K unique positions from one context of `ctx` slots
  decode   token t is the single query of sequence t; K unique positions from
           its own context of `ctx` positions
  prefill  one sequence; the T query rows are its last T positions p, each
           draws K unique positions uniformly from [0, p] (causal), padding
           with -1 where fewer than K exist
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np
import torch

E4M3_MAX = 448.0


@dataclass(frozen=True)
class Spec:
    name: str
    T: int
    H: int
    Dqk: int
    K: int
    ctx: int                 # context length per sequence (slots it owns)
    mode: str                # "shared" | "decode" | "prefill"
    kv_dtype: str = "bf16"   # "bf16" | "fp8"
    block_size: int = 64
    permute_blocks: bool = True
    sm_scale: float | None = None   # default 1/sqrt(Dqk)
    seed: int = 0

    @property
    def n_seq(self) -> int:
        return self.T if self.mode == "decode" else 1

    @property
    def num_blocks(self) -> int:
        return self.n_seq * (self.ctx // self.block_size)

    @property
    def N(self) -> int:
        return self.num_blocks * self.block_size

    @property
    def scale(self) -> float:
        return self.sm_scale if self.sm_scale is not None else 1.0 / math.sqrt(self.Dqk)


def _c4(T: int, K: int) -> Spec:
    return Spec(f"prefill_bf16_T{T}_K{K}", T=T, H=16, Dqk=512, K=K, ctx=8192,
                mode="prefill", seed=4)


#: The five workloads: tiny parity case, two GLM-5.3-Flash-like decode shapes
#: (bf16 and e4m3 KV), rope-free prefill (12 shapes) and DeepSeek-V3.2-like
#: 576-wide rows with 128 heads in both KV precisions.
CONFIGS: dict[str, Spec] = {
    "tiny_bf16": Spec("tiny_bf16", T=4, H=16, Dqk=512, K=128, ctx=1024, mode="shared",
                      permute_blocks=False, seed=0),
    "decode_bf16": Spec("decode_bf16", T=32, H=16, Dqk=512, K=2048, ctx=131072,
                        mode="decode", seed=2),
    "decode_fp8": Spec("decode_fp8", T=64, H=16, Dqk=512, K=2048, ctx=65536,
                       mode="decode", kv_dtype="fp8", seed=3),
    **{f"prefill_bf16_T{T}_K{K}": _c4(T, K) for T in (256, 512, 1024, 2048)
       for K in (128, 512, 2048)},
    "rope_decode_bf16": Spec("rope_decode_bf16", T=64, H=128, Dqk=576, K=2048, ctx=32768,
                             mode="decode", sm_scale=1.0 / 24.0, seed=5),
    "rope_decode_fp8": Spec("rope_decode_fp8", T=64, H=128, Dqk=576, K=2048, ctx=32768,
                            mode="decode", kv_dtype="fp8", sm_scale=1.0 / 24.0, seed=5),
}


@dataclass
class Case:
    spec: Spec
    q: torch.Tensor
    kv_pool: torch.Tensor
    topk_idx: torch.Tensor
    sm_scale: float
    kv_scale: float
    block_table: np.ndarray = field(repr=False, default=None)

    @property
    def kv_dtype(self) -> str:
        return self.spec.kv_dtype


def block_table(spec: Spec, rng: np.random.Generator) -> np.ndarray:
    """[n_seq, ctx // block_size] physical block ids."""
    nb = spec.num_blocks
    perm = rng.permutation(nb) if spec.permute_blocks else np.arange(nb)
    return perm.reshape(spec.n_seq, spec.ctx // spec.block_size).astype(np.int64)


def positions_to_slots(pos: np.ndarray, table_row: np.ndarray, block_size: int) -> np.ndarray:
    valid = pos >= 0
    p = np.where(valid, pos, 0)
    slots = table_row[p // block_size] * block_size + p % block_size
    return np.where(valid, slots, -1)


def topk_positions(spec: Spec, rng: np.random.Generator) -> np.ndarray:
    """Logical positions [T, K] (-1 where a causal row has fewer than K)."""
    T, K, ctx = spec.T, spec.K, spec.ctx
    pos = np.full((T, K), -1, dtype=np.int64)
    for t in range(T):
        if spec.mode in ("shared", "decode"):
            avail = ctx
        elif spec.mode == "prefill":
            avail = ctx - T + t + 1          # positions 0..p, p = ctx - T + t
        else:
            raise ValueError(spec.mode)
        n = min(K, avail)
        pos[t, :n] = rng.choice(avail, size=n, replace=False)
    return pos


def topk_slots(spec: Spec, rng: np.random.Generator, table: np.ndarray) -> np.ndarray:
    pos = topk_positions(spec, rng)
    out = np.empty_like(pos)
    for t in range(spec.T):
        seq = t if spec.mode == "decode" else 0
        out[t] = positions_to_slots(pos[t], table[seq], spec.block_size)
    return out.astype(np.int32)


def _normal_pool_chunks(N: int, D: int, seed: int, device: str, chunk_rows: int):
    """Yield (row0, fp32 chunk) of an N(0,1) [N, D] draw, reproducible per seed."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    for r0 in range(0, N, chunk_rows):
        rows = min(chunk_rows, N - r0)
        yield r0, torch.randn((rows, D), generator=g, device=device, dtype=torch.float32)


def quantize_e4m3(x: torch.Tensor, kv_scale: float) -> torch.Tensor:
    """e4m3 codes (uint8) of x / kv_scale, clamped to +-448 before the cast."""
    y = (x / kv_scale).clamp_(-E4M3_MAX, E4M3_MAX)
    return y.to(torch.float8_e4m3fn).view(torch.uint8)


def make_pool(spec: Spec, device: str, seed: int, chunk_rows: int = 1 << 17):
    """Return (kv_pool [num_blocks, block_size, Dqk], kv_scale)."""
    N, D = spec.N, spec.Dqk
    if spec.kv_dtype == "bf16":
        pool = torch.empty((N, D), dtype=torch.bfloat16, device=device)
        for r0, ch in _normal_pool_chunks(N, D, seed, device, chunk_rows):
            pool[r0:r0 + ch.shape[0]] = ch.to(torch.bfloat16)
        kv_scale = 1.0
    elif spec.kv_dtype == "fp8":
        amax = 0.0
        for _, ch in _normal_pool_chunks(N, D, seed, device, chunk_rows):
            amax = max(amax, float(ch.abs().max()))
        kv_scale = float(np.float32(amax) / np.float32(E4M3_MAX))
        pool = torch.empty((N, D), dtype=torch.uint8, device=device)
        for r0, ch in _normal_pool_chunks(N, D, seed, device, chunk_rows):
            pool[r0:r0 + ch.shape[0]] = quantize_e4m3(ch, kv_scale)
    else:
        raise ValueError(spec.kv_dtype)
    return pool.view(spec.num_blocks, spec.block_size, D), kv_scale


def make_case(spec: Spec, device: str = "cpu", index_sets: int = 1) -> Case | list[Case]:
    """Build one case (or `index_sets` cases sharing one pool, each with its own
    q and top-k lists -- used to rotate working sets past the on-die caches)."""
    rng = np.random.Generator(np.random.PCG64(spec.seed))
    table = block_table(spec, rng)
    pool, kv_scale = make_pool(spec, device, seed=spec.seed + 1000)
    cases = []
    for _ in range(index_sets):
        idx = topk_slots(spec, rng, table)
        qf = rng.standard_normal((spec.T, spec.H, spec.Dqk), dtype=np.float32)
        q = torch.from_numpy(qf).to(torch.bfloat16).to(device)
        cases.append(Case(spec, q, pool, torch.from_numpy(idx).to(device),
                          spec.scale, kv_scale, table))
    return cases[0] if index_sets == 1 else cases


def small_spec(T=4, H=16, Dqk=512, K=128, ctx=1024, kv_dtype="bf16", block_size=64,
               mode="shared", seed=0, sm_scale=None, permute_blocks=True) -> Spec:
    return Spec(f"mini_T{T}_H{H}_D{Dqk}_K{K}_{kv_dtype}", T=T, H=H, Dqk=Dqk, K=K, ctx=ctx,
                mode=mode, kv_dtype=kv_dtype, block_size=block_size,
                permute_blocks=permute_blocks, sm_scale=sm_scale, seed=seed)


def with_padding(idx: np.ndarray, rng: np.random.Generator, frac: float) -> np.ndarray:
    """Replace a random `frac` of the entries of each row with -1 (anywhere in the row)."""
    out = idx.copy()
    mask = rng.random(out.shape) < frac
    out[mask] = -1
    return out


def rope_cos_sin(max_pos: int, base: float = 10000.0) -> np.ndarray:
    """A rotary table in the usual layout: [max_pos, 64] fp32, cosines of the 32
    pair angles pos * base^(-2i/64) in columns 0..31, sines in 32..63."""
    inv = base ** (-np.arange(0, 64, 2, dtype=np.float64) / 64.0)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * inv[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)


@dataclass
class RopeCase:
    ql_nope: torch.Tensor     # bf16 [T, H, 512]
    q_pe: torch.Tensor        # bf16 [T, H, 64]
    kv_c: torch.Tensor        # bf16 [T, 512]
    k_pe: torch.Tensor        # bf16 [T, 64]
    positions: torch.Tensor   # int64 [T]
    cos_sin: torch.Tensor     # fp32 [max_pos, 64]
    slot_mapping: torch.Tensor  # int64 [T], -1 = no cache write
    num_blocks: int
    block_size: int


def make_rope_case(T: int, H: int, num_blocks: int, block_size: int, max_pos: int = 8192,
                   seed: int = 0, skip_frac: float = 0.0, device: str = "cpu") -> RopeCase:
    """Seeded inputs of the fused q-RoPE / cache write: N(0,1) activations,
    random positions, distinct random cache slots (a fraction set to -1)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    def bf(shape):
        return torch.from_numpy(rng.standard_normal(shape, dtype=np.float32)).to(torch.bfloat16)
    ql, qp, kc, kp = bf((T, H, 512)), bf((T, H, 64)), bf((T, 512)), bf((T, 64))
    pos = rng.integers(0, max_pos, size=T).astype(np.int64)
    N = num_blocks * block_size
    slots = rng.choice(N, size=T, replace=False).astype(np.int64)
    if skip_frac > 0:
        slots[rng.random(T) < skip_frac] = -1
    dev = torch.device(device)
    return RopeCase(ql.to(dev), qp.to(dev), kc.to(dev), kp.to(dev), torch.from_numpy(pos).to(dev),
                    torch.from_numpy(rope_cos_sin(max_pos)).to(dev), torch.from_numpy(slots).to(dev),
                    num_blocks, block_size)


__all__ = ["RopeCase", "make_rope_case", "rope_cos_sin", "Spec", "Case", "CONFIGS", "make_case", "make_pool", "small_spec", "topk_slots",
           "topk_positions", "block_table", "positions_to_slots", "quantize_e4m3",
           "with_padding", "E4M3_MAX", "replace"]
