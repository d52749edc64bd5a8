"""The C ABI without a GPU: exports, status strings, host-side validation.

Every error path here is decided on the host before any HIP call, so these
run on a machine with no GPU; nothing is launched.
"""
from __future__ import annotations

import ctypes
import math
import os
import re

import pytest

from sparse_mla_attention_03_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparse_mla.h")

OK, NULL, SHAPE, DTYPE, ALIGN, INVALID, UNSUP, WS, HIP = range(9)


@pytest.fixture(scope="module")
def lib():
    return binding.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sparse_mla_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("sparse_mla_fwd", "sparse_mla_fwd_ex", "sparse_mla_workspace_bytes",
              "sparse_mla_num_splits", "sparse_mla_quantize_q_fp8", "sparse_mla_status_string",
              "sparse_mla_last_error", "sparse_mla_abi_version"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_abi_version_and_status_strings(lib):
    assert lib.sparse_mla_abi_version() == binding.ABI_VERSION == 3
    seen = set()
    for st in range(9):
        s = binding.sparse_mla_status_string(st)
        assert s and s not in seen
        seen.add(s)
    assert binding.sparse_mla_status_string(99) == "unknown status"


# a fake, 256-byte aligned device address: never dereferenced (validation fails
# or T == 0 returns before any launch)
P = 0x7F0000000000


def call(lib, q=P, T=4, H=16, D=512, qst=16 * 512, qsh=512, kv=P, dt=0, nb=16, bs=64,
         idx=P, K=128, ist=128, sm=0.04, kvs=1.0, out=P, lse=P, ws=None, wsb=0, splits=1,
         reserved=0, events=None, dots=0, sinks=None, qsc=0.0):
    opts = binding.Options()
    opts.num_splits = splits
    opts.reserved[0] = reserved
    opts.dot_precision = dots
    opts.sinks = sinks
    opts.q_scale = qsc
    if events:
        opts.kernel_events[0], opts.kernel_events[1] = events
    st = lib.sparse_mla_fwd_ex(q, T, H, D, qst, qsh, kv, dt, nb, bs, idx, K, ist, sm, kvs, out,
                               lse, ws, wsb, None, ctypes.byref(opts))
    return st, binding.sparse_mla_last_error()


def test_empty_batch_is_a_noop(lib):
    assert call(lib, T=0, q=None, kv=None, idx=None, out=None, lse=None)[0] == OK


def test_options_layout():
    # the C struct: int32, int32, two pointers, a pointer, float, int32[3]
    assert ctypes.sizeof(binding.Options) == 48
    assert binding.Options.sinks.offset == 24 and binding.Options.q_scale.offset == 32
    assert binding.Options.reserved.offset == 36


@pytest.mark.parametrize("kw,status,needle", [
    (dict(q=None), NULL, "null"),
    (dict(out=None), NULL, "null"),
    (dict(lse=None), NULL, "null"),
    (dict(idx=None), NULL, "null"),
    (dict(H=24), UNSUP, "H=24"),
    (dict(H=0), SHAPE, "bad sizes"),
    (dict(D=320), UNSUP, "Dqk=320"),
    (dict(dt=2), DTYPE, "dtype"),
    (dict(T=-1), SHAPE, "bad sizes"),
    (dict(K=-5), SHAPE, "bad sizes"),
    (dict(bs=0), SHAPE, "pool"),
    (dict(nb=-1), SHAPE, "pool"),
    (dict(qsh=-512), SHAPE, "stride"),
    (dict(q=P + 2), ALIGN, "q must"),
    (dict(qsh=516), ALIGN, "q must"),
    (dict(kv=P + 8), ALIGN, "kv_pool"),
    (dict(out=P + 4), ALIGN, "out"),
    (dict(lse=P + 2), ALIGN, "lse"),
    (dict(sm=math.inf), INVALID, "finite"),
    (dict(kvs=math.nan), INVALID, "finite"),
    (dict(splits=65), INVALID, "num_splits"),
    (dict(splits=-1), INVALID, "num_splits"),
    (dict(reserved=3), INVALID, "reserved"),
    (dict(dots=2), INVALID, "dot_precision"),
    (dict(dots=-1), INVALID, "dot_precision"),
    (dict(dots=1), INVALID, "e4m3 KV only"),
    (dict(sinks=P + 2), ALIGN, "sinks"),
    (dict(qsc=-1.0), INVALID, "q_scale"),
    (dict(qsc=math.inf), INVALID, "q_scale"),
    (dict(qsc=math.nan), INVALID, "q_scale"),
    (dict(qsc=0.5), INVALID, "e4m3 KV with e4m3 dots"),
    (dict(qsc=0.5, dt=1, dots=1), INVALID, "e4m3 KV with e4m3 dots"),
    (dict(qsc=0.5, dt=1, qsh=520, qst=16 * 520), ALIGN, "multiples of 16 bytes"),
    (dict(events=(P, None)), INVALID, "kernel_events"),
    (dict(splits=2), WS, "workspace"),
    (dict(splits=2, ws=P, wsb=100), WS, "workspace"),
    (dict(splits=2, ws=P + 4, wsb=1 << 30), ALIGN, "workspace"),
])
def test_validation_errors(lib, kw, status, needle):
    st, msg = call(lib, **kw)
    assert st == status, (st, msg)
    assert needle in msg


def test_workspace_and_split_planning_explicit(lib):
    # explicit split counts need no device query
    assert binding.sparse_mla_workspace_bytes(32, 16, 2048, 512, 0, 1) == 0
    # per (split, token, head): 512 fp16 partials, four fp32 quarter scales, one fp32 lse
    assert binding.sparse_mla_workspace_bytes(32, 16, 2048, 512, 0, 8) == 8 * 32 * 16 * (1024 + 16 + 4)
    # never more splits than 64-entry tiles; empty splits are dropped
    assert binding.sparse_mla_num_splits(4, 16, 128, 512, 0, 8) == 2
    assert binding.sparse_mla_num_splits(4, 16, 200, 512, 0, 3) == 2   # 4 tiles -> 2+2
    assert binding.sparse_mla_num_splits(4, 16, 0, 512, 0, 5) == 1
    with pytest.raises(binding.SparseMLAError):
        binding.sparse_mla_num_splits(4, 24, 128, 512, 0, 1)
    with pytest.raises(binding.SparseMLAError):
        binding.sparse_mla_workspace_bytes(4, 16, 128, 600, 0, 1)


def test_quantize_entry_validation(lib):
    st = lib.sparse_mla_quantize_q_fp8(None, 2, 16, 512, 8192, 512, P, P, None)
    assert st == NULL
    st = lib.sparse_mla_quantize_q_fp8(P, 2, 20, 512, 8192, 512, P, P, None)
    assert st == UNSUP
    assert lib.sparse_mla_quantize_q_fp8(None, 0, 16, 512, 0, 0, None, None, None) == OK


def test_varlen_validation(lib):
    opts = binding.Options()
    lens = P
    def v(**kw):
        a = dict(q=P, T=4, H=16, D=512, qst=16 * 512, qsh=512, kv=P, dt=0, nb=16, bs=64, idx=P, K=128,
                 ist=128, lens=lens, sm=0.04, kvs=1.0, out=P, lse=P, ws=P, wsb=1 << 30, splits=0)
        a.update(kw)
        opts.num_splits = a["splits"]
        st = lib.sparse_mla_fwd_varlen(a["q"], a["T"], a["H"], a["D"], a["qst"], a["qsh"], a["kv"], a["dt"],
                                       a["nb"], a["bs"], a["idx"], a["K"], a["ist"], a["lens"], a["sm"],
                                       a["kvs"], a["out"], a["lse"], a["ws"], a["wsb"], None,
                                       ctypes.byref(opts))
        return st, binding.sparse_mla_last_error()
    assert v(lens=None)[0] == NULL
    st, msg = v(splits=2)
    assert st == INVALID and "per token" in msg
    st, msg = v(lens=P + 2)
    assert st == ALIGN and "topk_len" in msg
    assert v(T=0, q=None, kv=None, idx=None, out=None, lse=None, lens=None)[0] == OK


def test_noalloc_rejects_explicit_splits_beyond_its_scratch(lib):
    """An explicit split count whose partials exceed the per-device scratch is
    refused on the host (SMLA_ERR_WORKSPACE) before any HIP call; a bad option
    is refused as in sparse_mla_fwd_ex."""
    opts = binding.Options()
    T, H = 64, 128
    splits = 8                                   # 8 * 64 * 128 * 1044 B > 32 MiB
    assert splits * T * H * 1044 > 32 << 20
    opts.num_splits = splits
    st = lib.sparse_mla_fwd_noalloc(P, T, H, 576, H * 576, 576, P, 0, 512, 64, P, 2048, 2048,
                                    0.04, 1.0, P, P, None, ctypes.byref(opts))
    assert st == WS
    assert "scratch" in binding.sparse_mla_last_error()
    opts.num_splits = 99
    st = lib.sparse_mla_fwd_noalloc(P, T, H, 576, H * 576, 576, P, 0, 512, 64, P, 2048, 2048,
                                    0.04, 1.0, P, P, None, ctypes.byref(opts))
    assert st == INVALID
    # T == 0 is a no-op with null pointers, as for the other entry points
    assert lib.sparse_mla_fwd_noalloc(None, 0, 16, 512, 0, 0, None, 0, 1, 64, None, 8, 8,
                                      0.04, 1.0, None, None, None, None) == OK


def test_ceiling_library_exports_its_header():
    """The device-ceiling probes the benchmark loads (a library of their own)."""
    text = open(os.path.join(ROOT, "include", "smla_ceiling.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = sorted(set(re.findall(r"\b(smla_ceiling_\w+)\s*\(", text)))
    assert names == ["smla_ceiling_gather", "smla_ceiling_lds_read", "smla_ceiling_mfma", "smla_ceiling_stream_read"]
    lib = ctypes.CDLL(os.path.join(ROOT, "sparse_mla_attention_03_amd", "csrc", "libsmla_ceiling.so"))
    for n in names:
        assert ctypes.cast(getattr(lib, n), ctypes.c_void_p).value
    # argument checks return before any launch
    lib.smla_ceiling_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                             ctypes.c_int64, ctypes.c_void_p]
    assert lib.smla_ceiling_stream_read(None, 1 << 20, None, 0, None) == 1
    assert lib.smla_ceiling_stream_read(P, 1 << 20, P, 16, None) == 2


def test_rope_entry_size_guard_does_not_overflow(lib):
    """T (H + 1) 72 bytes must stay below 2^32 for one launch; T and H up to
    2^31 - 1 would overflow that product in 64 bits if it were formed."""
    def call(T, H, ql=P):
        return lib.sparse_mla_rope_concat_cache(ql, 576, 576, P, 64, 64, P, 512, P, 64, P, P, 4096, 1, T, H,
                                                P, 0, 1.0, P, P, 0, 1, 64, 1.0, None)
    big = 0x7FFFFFFF
    assert call(big, big) == UNSUP
    assert call(1000, 10_000_000) == UNSUP
    assert call(big, 1) == UNSUP
    assert call(0, big) == OK                     # nothing to do: a no-op
    assert call(2, 16, ql=None) == NULL           # within the guard: the next check decides
    assert call(big // 100, 16, ql=None) == UNSUP
