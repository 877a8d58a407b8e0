"""Host-only checks of the C ABI: the library loads, exports what the header
declares, and rejects bad arguments before anything reaches a GPU."""

import ctypes
import os
import re
import subprocess

import pytest

import attention_learnable_sinks_amd as als

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn_sink.h")
FAKE = 0x100000  # never dereferenced: every case below fails validation first


@pytest.fixture(scope="module")
def lib():
    return als.load()


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_sink_\w+)\s*\(", src)))


def test_head_dim_128_is_accepted(lib):
    """head_dim 64 and 128 are built: a d=128 shape passes every check (and stops at
    the workspace check here), with workspaces sized for 128 columns."""
    s = _shape(head_dim=128, num_heads_q=64, num_heads_kv=8, total_q=4096, total_k=4096, max_seqlen_q=4096,
               max_seqlen_k=4096)
    n128 = lib.attn_sink_bwd_workspace_bytes(ctypes.byref(s))
    s64 = _shape(num_heads_q=64, num_heads_kv=8, total_q=4096, total_k=4096, max_seqlen_q=4096, max_seqlen_k=4096)
    n64 = lib.attn_sink_bwd_workspace_bytes(ctypes.byref(s64))
    # d=64: 4 head splits (512 workgroups, two per compute unit); d=128: one
    # workgroup per compute unit fits, so 2 splits (256 workgroups)
    fixed = 64 * 2 * 4096 * 4 + 64 * (4096 // 128) * 4
    assert fixed + 2 * 4 * 4096 * 8 * 64 * 4 <= n64 <= fixed + 2 * 4 * 4096 * 8 * 64 * 4 + 4 * 256
    assert fixed + 2 * 2 * 4096 * 8 * 128 * 4 <= n128 <= fixed + 2 * 2 * 4096 * 8 * 128 * 4 + 4 * 256
    assert lib.attn_sink_bwd(ctypes.byref(s), *[FAKE] * 11, FAKE, n128 - 1, None) == als.ERR_WORKSPACE
    d = _decode_shape(head_dim=128)
    assert lib.attn_sink_fwd_decode_workspace_bytes(ctypes.byref(d)) > 0
    assert lib.attn_sink_merge(als.BF16, 128, 8, 0, 2, None, None, FAKE, None, None, None) == als.OK


def test_header_declares_the_entry_points():
    assert _declared() == sorted(["attn_sink_fwd", "attn_sink_bwd", "attn_sink_bwd_workspace_bytes",
                                  "attn_sink_fwd_decode", "attn_sink_fwd_decode_workspace_bytes",
                                  "attn_sink_fwd_decode_noalloc", "attn_sink_merge",
                                  "attn_sink_status_string", "attn_sink_timing_enable", "attn_sink_timing_read"])


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", als.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (attn_sink_\w+)", out))
    for name in _declared():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_status_strings(lib):
    for st in range(5):
        assert lib.attn_sink_status_string(st)
    assert lib.attn_sink_status_string(0) == b"ok"
    assert lib.attn_sink_status_string(99) == b"unknown status"


def _shape(**kw):
    base = dict(dtype=als.BF16, head_dim=64, num_heads_q=8, num_heads_kv=2, num_seqs=1, total_q=128,
                total_k=128, max_seqlen_q=128, max_seqlen_k=128, cu_seqlens_q=FAKE, cu_seqlens_k=FAKE,
                softmax_scale=0.125, causal=1, window=0)
    base.update(kw)
    return als.Shape(**base)


BAD_SHAPES = [
    (dict(head_dim=96), als.ERR_UNSUPPORTED),
    (dict(head_dim=256), als.ERR_UNSUPPORTED),
    (dict(head_dim=0), als.ERR_INVALID_ARG),
    (dict(dtype=7), als.ERR_UNSUPPORTED),
    (dict(num_heads_q=6, num_heads_kv=4), als.ERR_INVALID_ARG),
    (dict(num_heads_kv=0), als.ERR_INVALID_ARG),
    (dict(num_seqs=0), als.ERR_INVALID_ARG),
    (dict(num_seqs=-3), als.ERR_INVALID_ARG),
    (dict(total_q=-1), als.ERR_INVALID_ARG),
    (dict(max_seqlen_k=-1), als.ERR_INVALID_ARG),
    (dict(cu_seqlens_q=None), als.ERR_INVALID_ARG),
    (dict(cu_seqlens_k=None), als.ERR_INVALID_ARG),
    (dict(softmax_scale=0.0), als.ERR_INVALID_ARG),
    (dict(softmax_scale=float("nan")), als.ERR_INVALID_ARG),
    (dict(softmax_scale=float("inf")), als.ERR_INVALID_ARG),
    (dict(causal=2), als.ERR_INVALID_ARG),
    (dict(max_seqlen_q=65535 * 128 + 1), als.ERR_UNSUPPORTED),
]


@pytest.mark.parametrize("kw,status", BAD_SHAPES, ids=[str(k) for k, _ in BAD_SHAPES])
def test_fwd_rejects_bad_shape(lib, kw, status):
    s = _shape(**kw)
    assert lib.attn_sink_fwd(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == status


@pytest.mark.parametrize("kw,status", BAD_SHAPES, ids=[str(k) for k, _ in BAD_SHAPES])
def test_bwd_rejects_bad_shape(lib, kw, status):
    s = _shape(**kw)
    args = [FAKE] * 11 + [FAKE, 1 << 40, None]
    assert lib.attn_sink_bwd(ctypes.byref(s), *args) == status
    assert lib.attn_sink_bwd_workspace_bytes(ctypes.byref(s)) == 0


def _decode_shape(**kw):
    base = dict(num_heads_q=64, num_heads_kv=8, num_seqs=4, total_q=4, total_k=4 * 8192, max_seqlen_q=1,
                max_seqlen_k=8192)
    base.update(kw)
    return _shape(**base)


@pytest.mark.parametrize("kw,status", BAD_SHAPES, ids=[str(k) for k, _ in BAD_SHAPES])
def test_fwd_decode_rejects_bad_shape(lib, kw, status):
    s = _shape(**kw)
    assert lib.attn_sink_fwd_decode(ctypes.byref(s), *[FAKE] * 7, 1 << 40, None) == status
    assert lib.attn_sink_fwd_decode_workspace_bytes(ctypes.byref(s)) == 0


@pytest.mark.parametrize("hq,hkv,max_q,ok", [(64, 8, 4, True), (64, 8, 5, False), (8, 8, 32, True),
                                              (8, 8, 33, False), (64, 1, 1, False), (32, 1, 1, True),
                                              (24, 8, 10, True), (24, 8, 11, False)])
def test_fwd_decode_width_limit(lib, hq, hkv, max_q, ok):
    """(Hq / Hkv) * max_seqlen_q <= 32: the query heads of a kv head times the new
    rows share one 32-column block."""
    s = _decode_shape(num_heads_q=hq, num_heads_kv=hkv, max_seqlen_q=max_q, total_q=4 * max_q)
    n = lib.attn_sink_fwd_decode_workspace_bytes(ctypes.byref(s))
    st = lib.attn_sink_fwd_decode(ctypes.byref(s), *[FAKE] * 7, 0, None)
    if ok:
        assert n > 0 and st == als.ERR_WORKSPACE  # passes the width check, stops at the workspace
    else:
        assert n == 0 and st == als.ERR_UNSUPPORTED


@pytest.mark.parametrize("slot", range(6))
def test_fwd_decode_rejects_null_tensor(lib, slot):
    ptrs = [FAKE] * 6
    ptrs[slot] = None
    s = _decode_shape()
    assert lib.attn_sink_fwd_decode(ctypes.byref(s), *ptrs, FAKE, 1 << 40, None) == als.ERR_INVALID_ARG


def test_fwd_decode_workspace(lib):
    """Partials: per (sequence, kv head, key chunk) one 64-value row plus a (max,
    sum) pair per (query head, new row) column, in float32.  Chunks are a fixed 1024
    keys (batch invariance); with a single chunk nothing is kept (256 bytes are still
    reported)."""
    def parts(seqs, hkv, chunks, cols):
        n = seqs * hkv * chunks * cols
        return -(-n * 64 * 4 // 256) * 256 + -(-n * 2 * 4 // 256) * 256

    s = _decode_shape()  # 4 sequences, 8192 keys = 8 chunks
    assert lib.attn_sink_fwd_decode_workspace_bytes(ctypes.byref(s)) == parts(4, 8, 8, 8)
    s = _decode_shape(max_seqlen_q=4, total_q=16)  # 8 heads x 4 rows = 32 columns
    assert lib.attn_sink_fwd_decode_workspace_bytes(ctypes.byref(s)) == parts(4, 8, 8, 32)
    s = _decode_shape(num_seqs=64, total_q=64, total_k=64 * 16384, max_seqlen_k=16384)
    assert lib.attn_sink_fwd_decode_workspace_bytes(ctypes.byref(s)) == parts(64, 8, 16, 8)
    s = _decode_shape(max_seqlen_k=1025, total_k=4 * 1025)  # 1025 keys straddle two chunks
    assert lib.attn_sink_fwd_decode_workspace_bytes(ctypes.byref(s)) == parts(4, 8, 2, 8)
    s = _decode_shape(max_seqlen_k=1024, total_k=4 * 1024)  # exactly one chunk: no partials
    assert lib.attn_sink_fwd_decode_workspace_bytes(ctypes.byref(s)) == 256
    s = _decode_shape(window=128)  # 128 keys straddle at most 5 tiles: one chunk, no partials
    assert lib.attn_sink_fwd_decode_workspace_bytes(ctypes.byref(s)) == 256
    s = _decode_shape(num_seqs=1, total_q=1, total_k=131072, max_seqlen_k=131072)
    assert lib.attn_sink_fwd_decode_workspace_bytes(ctypes.byref(s)) == parts(1, 8, 128, 8)
    args = [FAKE] * 7
    need = lib.attn_sink_fwd_decode_workspace_bytes(ctypes.byref(_decode_shape()))
    s = _decode_shape()
    assert lib.attn_sink_fwd_decode(ctypes.byref(s), *args[:6], FAKE, need - 1, None) == als.ERR_WORKSPACE
    assert lib.attn_sink_fwd_decode(ctypes.byref(s), *args[:6], None, need, None) == als.ERR_WORKSPACE
    assert lib.attn_sink_fwd_decode(ctypes.byref(s), *args[:6], FAKE + 8, need, None) == als.ERR_WORKSPACE


@pytest.mark.parametrize("args,status", [
    ((als.BF16, 96, 8, 10, 2), als.ERR_UNSUPPORTED),
    ((7, 64, 8, 10, 2), als.ERR_UNSUPPORTED),
    ((als.BF16, 0, 8, 10, 2), als.ERR_INVALID_ARG),
    ((als.BF16, 64, 0, 10, 2), als.ERR_INVALID_ARG),
    ((als.BF16, 64, 8, -1, 2), als.ERR_INVALID_ARG),
    ((als.BF16, 64, 8, 10, 0), als.ERR_INVALID_ARG),
])
def test_merge_rejects_bad_sizes(lib, args, status):
    assert lib.attn_sink_merge(*args, FAKE, FAKE, FAKE, FAKE, FAKE, None) == status


@pytest.mark.parametrize("slot", range(5))
def test_merge_rejects_null_tensor(lib, slot):
    ptrs = [FAKE] * 5
    ptrs[slot] = None
    assert lib.attn_sink_merge(als.FP32, 64, 8, 10, 3, *ptrs, None) == als.ERR_INVALID_ARG


def test_merge_empty_is_a_no_op(lib):
    assert lib.attn_sink_merge(als.FP32, 64, 8, 0, 3, None, None, FAKE, None, None, None) == als.OK


def test_null_shape(lib):
    assert lib.attn_sink_fwd(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == als.ERR_INVALID_ARG
    assert lib.attn_sink_bwd_workspace_bytes(None) == 0
    assert lib.attn_sink_fwd_decode_workspace_bytes(None) == 0


@pytest.mark.parametrize("slot", range(6))
def test_fwd_rejects_null_tensor(lib, slot):
    ptrs = [FAKE] * 6
    ptrs[slot] = None
    s = _shape()
    assert lib.attn_sink_fwd(ctypes.byref(s), *ptrs, None) == als.ERR_INVALID_ARG


@pytest.mark.parametrize("slot", range(11))
def test_bwd_rejects_null_tensor(lib, slot):
    ptrs = [FAKE] * 11
    ptrs[slot] = None
    s = _shape()
    assert lib.attn_sink_bwd(ctypes.byref(s), *ptrs, FAKE, 1 << 40, None) == als.ERR_INVALID_ARG


def test_workspace_size_formula(lib):
    s = _shape(num_heads_q=64, num_heads_kv=8, total_q=4096, total_k=4096, max_seqlen_q=4096, max_seqlen_k=4096)
    n = lib.attn_sink_bwd_workspace_bytes(ctypes.byref(s))
    t, hq, hkv, d = 4096, 64, 8, 64
    splits = 4  # 16 folded key-tile pairs x 8 kv heads x 4 = 512 dK/dV workgroups
    # row statistics, one dS_h partial per (head, sequence, 128-row dQ tile), dK/dV partials
    expect = hq * 2 * t * 4 + hq * (t // 128) * 4 + 2 * splits * t * hkv * d * 4
    assert expect <= n <= expect + 4 * 256
    s = _shape(num_heads_q=64, num_heads_kv=8, total_q=16384, total_k=16384, max_seqlen_q=16384,
               max_seqlen_k=16384)
    n = lib.attn_sink_bwd_workspace_bytes(ctypes.byref(s))
    expect = hq * 2 * 16384 * 4 + hq * (16384 // 128) * 4  # 64 pairs x 8 = 512: no split, no partials
    assert expect <= n <= expect + 4 * 256
    # window layer: dQ tiles pack the 8 query heads of a kv head (16 positions x 8 heads),
    # so dS_h has one partial per head and 16-position tile; no dK/dV split at 16k
    s = _shape(num_heads_q=64, num_heads_kv=8, total_q=16384, total_k=16384, max_seqlen_q=16384,
               max_seqlen_k=16384, window=128)
    n = lib.attn_sink_bwd_workspace_bytes(ctypes.byref(s))
    expect = hq * 2 * 16384 * 4 + hq * (16384 // 16) * 4
    assert expect <= n <= expect + 4 * 256
    # two sequences: one partial per head, sequence and packed tile (still no dK/dV split)
    s = _shape(num_heads_q=64, num_heads_kv=8, num_seqs=2, total_q=32768, total_k=32768, max_seqlen_q=16384,
               max_seqlen_k=16384, window=128)
    n = lib.attn_sink_bwd_workspace_bytes(ctypes.byref(s))
    expect = hq * 2 * 32768 * 4 + hq * 2 * (16384 // 16) * 4
    assert expect <= n <= expect + 4 * 256


def test_bwd_rejects_small_or_misaligned_workspace(lib):
    s = _shape()
    need = lib.attn_sink_bwd_workspace_bytes(ctypes.byref(s))
    assert need > 0
    args = [FAKE] * 11
    assert lib.attn_sink_bwd(ctypes.byref(s), *args, FAKE, need - 1, None) == als.ERR_WORKSPACE
    assert lib.attn_sink_bwd(ctypes.byref(s), *args, None, need, None) == als.ERR_WORKSPACE
    assert lib.attn_sink_bwd(ctypes.byref(s), *args, FAKE + 4, need, None) == als.ERR_WORKSPACE


def test_timing_read_without_records(lib):
    assert lib.attn_sink_timing_enable(1) == 0
    assert lib.attn_sink_timing_read(None, None, None, 0) == 0
    assert lib.attn_sink_timing_enable(0) == 0


def test_load_fails_loudly_without_library(tmp_path):
    with pytest.raises(RuntimeError, match="not found"):
        als.load(str(tmp_path / "missing.so"))


# Pointer alignment: 16 bytes for the tensors the kernels move in 16-byte pieces,
# 4 bytes for the float32 / int32 arrays.  Argument order of each entry point:
#   fwd, fwd_decode: q k v sinks o lse        bwd: q k v sinks o lse dout dq dk dv dsinks
WIDE_FWD, NARROW_FWD = (0, 1, 2, 4), (3, 5)
WIDE_BWD, NARROW_BWD = (0, 1, 2, 4, 6, 7, 8, 9), (3, 5, 10)


def _offset(n, slot, by):
    ptrs = [FAKE] * n
    ptrs[slot] = FAKE + by
    return ptrs


@pytest.mark.parametrize("slot,by", [(s, 8) for s in WIDE_FWD] + [(s, 2) for s in NARROW_FWD])
def test_fwd_rejects_misaligned_tensor(lib, slot, by):
    s = _shape()
    assert lib.attn_sink_fwd(ctypes.byref(s), *_offset(6, slot, by), None) == als.ERR_INVALID_ARG


@pytest.mark.parametrize("slot,by", [(s, 8) for s in WIDE_BWD] + [(s, 2) for s in NARROW_BWD])
def test_bwd_rejects_misaligned_tensor(lib, slot, by):
    s = _shape()
    assert lib.attn_sink_bwd(ctypes.byref(s), *_offset(11, slot, by), FAKE, 1 << 40, None) == als.ERR_INVALID_ARG


@pytest.mark.parametrize("slot,by", [(s, 8) for s in WIDE_FWD] + [(s, 2) for s in NARROW_FWD])
def test_fwd_decode_rejects_misaligned_tensor(lib, slot, by):
    s = _decode_shape()
    ptrs = _offset(6, slot, by)
    assert lib.attn_sink_fwd_decode(ctypes.byref(s), *ptrs, FAKE, 1 << 40, None) == als.ERR_INVALID_ARG


@pytest.mark.parametrize("slot", range(6))
def test_fwd_decode_accepts_minimal_alignment(lib, slot):
    """16 bytes (tensors) and 4 bytes (float32 arrays) pass the pointer check: the call
    goes on to the workspace check, which a zero-byte workspace fails."""
    s = _decode_shape()
    ptrs = _offset(6, slot, 16 if slot in WIDE_FWD else 4)
    assert lib.attn_sink_fwd_decode(ctypes.byref(s), *ptrs, FAKE, 0, None) == als.ERR_WORKSPACE


@pytest.mark.parametrize("slot,by", [(0, 8), (3, 8), (1, 2), (2, 2), (4, 2)])
def test_merge_rejects_misaligned_tensor(lib, slot, by):
    # o_parts lse_parts sinks o lse
    assert lib.attn_sink_merge(als.FP32, 64, 8, 10, 3, *_offset(5, slot, by), None) == als.ERR_INVALID_ARG


@pytest.mark.parametrize("field", ["cu_seqlens_q", "cu_seqlens_k"])
def test_rejects_misaligned_cu_seqlens(lib, field):
    s = _shape(**{field: FAKE + 2})
    assert lib.attn_sink_fwd(ctypes.byref(s), *[FAKE] * 6, None) == als.ERR_INVALID_ARG


def test_noalloc_decode_refuses_shapes_beyond_its_scratch(lib):
    """The allocation-free decoding call rejects, before any device work, a shape
    whose workspace exceeds the fixed scratch (64 sequences x 65,535-key caches)."""
    lib.attn_sink_fwd_decode_noalloc.argtypes = [ctypes.POINTER(als.Shape)] + [ctypes.c_void_p] * 7
    big = _decode_shape(num_seqs=64, total_q=64 * 4, max_seqlen_q=4, total_k=64 * 65535, max_seqlen_k=65535)
    need = lib.attn_sink_fwd_decode_workspace_bytes(ctypes.byref(big))
    assert need > als.DECODE_SCRATCH_BYTES
    assert lib.attn_sink_fwd_decode_noalloc(ctypes.byref(big), *[FAKE] * 6, None) == als.ERR_WORKSPACE
    for kw, status in BAD_SHAPES:  # the shape checks come first, as in attn_sink_fwd_decode
        s = _decode_shape(**kw)
        assert lib.attn_sink_fwd_decode_noalloc(ctypes.byref(s), *[FAKE] * 6, None) == status, kw


def test_thirty_two_bit_offset_bound(lib):
    """A kernel reads one head of one sequence through a buffer descriptor with 32-bit
    byte offsets, and a tile may start on the last row, so (max_seqlen + 128) x row
    pitch must stay below 2^32: Hq = 64, d = 64, bf16 (pitch 8192 B) allows 524159
    query rows, Hkv = 8 (pitch 1024 B) 4194175 key rows; one more is refused."""
    def ws(max_q, max_k):
        s = _shape(num_heads_q=64, num_heads_kv=8, total_q=max_q, total_k=max_k, max_seqlen_q=max_q,
                   max_seqlen_k=max_k)
        return lib.attn_sink_bwd_workspace_bytes(ctypes.byref(s))
    assert ((524159 + 128) * 8192) < 2 ** 32 <= ((524160 + 128) * 8192)
    assert ((4194175 + 128) * 1024) < 2 ** 32 <= ((4194176 + 128) * 1024)
    assert ws(524159, 128) > 0 and ws(524160, 128) == 0
    assert ws(128, 4194175) > 0 and ws(128, 4194176) == 0
    s = _shape(num_heads_q=64, num_heads_kv=8, total_q=524160, max_seqlen_q=524160)
    assert lib.attn_sink_fwd(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == als.ERR_UNSUPPORTED
