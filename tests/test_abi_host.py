"""CPU tests of the C ABI: the built library loads without a GPU, exports every
symbol include/monarch_attn.h declares, and rejects bad arguments on the host
before any HIP call (no compute call is made here)."""

import ctypes
import os
import re

import pytest

import structured_sub_quadratic_amd as ma
from structured_sub_quadratic_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "monarch_attn.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("library not built (run __graft_entry__.build())")
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(monarch_attn_\w+)\s*\(", text)))


def test_header_declares_expected_api():
    names = declared_functions()
    for must in ("monarch_attn_forward", "monarch_attn_workspace_size",
                 "monarch_attn_backward", "monarch_attn_backward_workspace_size",
                 "monarch_attn_status_string"):
        assert must in names


def test_library_exports_every_declared_symbol(lib):
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_problem_struct_layout_matches_header():
    # int64 x4, int32 x5, float, int32 x5, uint32, int32 x2 -> 32 + 20 + 4 + 20 + 4 + 8
    # = 88 (a multiple of the 8-byte alignment of the int64 fields)
    assert ctypes.sizeof(_lib.MAProblem) == 88
    assert _lib.MAProblem.causal.offset == 84
    assert ctypes.sizeof(_lib.MAExports) == 32


def status(p, n_ws=1 << 30, q=256, k=512, v=768, y=1024 * 1024 * 1024, ws=1 << 40):
    lib = _lib.load()
    return lib.monarch_attn_forward(ctypes.byref(p), q, k, v, y, None, ws, n_ws, None)


def good(**kw):
    args = dict(batch=1, heads=2, seq_len=256, head_dim=64, b1=16, b2=16, steps=1)
    args.update(kw)
    return ma.make_problem(**args)


@pytest.mark.parametrize("kw,code", [
    (dict(b1=16, b2=8), 1),                   # N != b1*b2
    (dict(c1=3), 1),                          # c1 does not divide b1
    (dict(c2=5), 1),
    (dict(steps=0), 1),
    (dict(head_dim=96), 2),                   # unsupported d
    (dict(seq_len=512, b1=2, b2=256), 2),     # segment wider than supported
    (dict(layout="fh_w", fhw=(2, 4, 32)), 0),  # fh=8 != b1: checked below separately
    (dict(scale=-1.0), 1),
    (dict(kv_heads=3), 1),                    # does not divide heads = 2
    (dict(kv_heads=4), 1),                    # more K/V heads than query heads
    (dict(kv_heads=1), 0),                    # grouped-query attention, valid
    (dict(causal=1), 0),                      # block-causal use
    (dict(causal=3, c1=2, c2=2, steps=2), 0),
    (dict(causal=-2), 1),
    (dict(seq_len=250), 0),                   # flat sequence padded to the 16 x 16 grid
    (dict(seq_len=241), 0),                   # 15 padding positions < b2
    (dict(seq_len=240), 1),                   # a whole block of padding
    (dict(seq_len=247, c2=2), 1),             # 9 padding positions fill a segment of 8
    (dict(seq_len=249, c2=2), 0),
    (dict(batch=1 << 14, heads=16, seq_len=1 << 14, b1=128, b2=128), 2),   # 2^32 exchange rows
    (dict(batch=1 << 12, heads=16, seq_len=1 << 14, b1=128, b2=128), 0),   # 2^30
])
def test_validation_codes(lib, kw, code):
    p = good(**kw)
    if kw.get("layout") == "fh_w":
        assert status(p) == 1             # (f*h, w) = (8, 32) does not match (16, 16)
        p = good(layout="fh_w", fhw=(4, 4, 16))
        assert ma.workspace_size(p) > 0   # (16, 16): valid
        return
    if code == 0:
        assert ma.workspace_size(p) > 0
        return
    assert status(p) == code
    n = ctypes.c_size_t()
    assert lib.monarch_attn_workspace_size(ctypes.byref(p), ctypes.byref(n)) == code


def test_pointer_checks(lib):
    p = good()
    assert status(p, q=0) == 1                       # null
    assert status(p, q=258) == 1                     # misaligned
    assert status(p, y=600) == 1                     # y overlaps k
    assert status(p, n_ws=10) == 3                   # workspace too small
    assert status(p, ws=(1 << 40) + 8) == 1          # misaligned workspace
    assert status(p, ws=512) == 1                    # workspace overlaps inputs
    assert lib.monarch_attn_forward(None, 0, 0, 0, 0, None, 0, 0, None) == 1


def test_workspace_size_and_launch_plan(lib):
    p = ma.make_problem(1, 12, 16384, 64, 128, 128)
    ws = ma.workspace_size(p)
    # c, u (bf16) + entropy + two normaliser buffers
    assert ws >= 12 * 16384 * (2 * 64 * 2 + 3 * 4)
    assert ma.launch_names(p) == ["stage1_last", "stage2_last"]
    p = ma.make_problem(1, 12, 16384, 64, 128, 128, flags=ma.MA_FLAG_FORCE_FUSED)
    assert ma.launch_names(p) == ["fused_t1"]
    p = ma.make_problem(1, 12, 16384, 64, 128, 128,
                        flags=ma.MA_FLAG_FORCE_FUSED | ma.MA_FLAG_FORCE_STAGED)
    assert ma.launch_names(p) == ["stage1_last", "stage2_last"]
    # columns of at most 64 rows and keys: the L-update and the next queries
    # of the steps before the last in one launch (which also takes the
    # zero-weight fallback, so no tile-means launch)
    p = ma.make_problem(8, 12, 4096, 64, 64, 64, steps=3)
    assert ma.launch_names(p) == ["stage1", "stage2_alpha", "stage1", "stage2_alpha",
                                  "stage1_last", "stage2_last"]
    p = ma.make_problem(8, 12, 4096, 64, 64, 64, steps=3, dtype="f32")
    assert ma.launch_names(p) == ["qbar", "stage1", "stage2_stats", "alpha", "stage1",
                                  "stage2_stats", "alpha", "stage1_last", "stage2_last"]
    p = ma.make_problem(2, 12, 96 * 64, 64, 96, 64, steps=2)      # columns of 96 keys
    assert ma.launch_names(p) == ["qbar", "stage1", "stage2_stats", "alpha", "stage1_last",
                                  "stage2_last"]
    p = ma.make_problem(1, 12, 32760, 128, 630, 52, c1=2, c2=2, layout="fh_w", fhw=(21, 30, 52))
    assert ma.launch_names(p) == ["qbar", "stage1_last", "stage2_last"]
    p = ma.make_problem(1, 12, 32760, 128, 630, 52, c1=2, c2=2, layout="fh_w", fhw=(21, 30, 52),
                        flags=ma.MA_FLAG_FORCE_FUSED)
    assert ma.launch_names(p) == ["fused_t1"]
    assert lib.monarch_attn_num_launches(ctypes.byref(good(b2=8))) == -1
    # a padded flat sequence (ViT: 197 tokens as 15 blocks of 14) needs the
    # tile means for its padding positions; the workspace covers the grid
    p = ma.make_problem(1, 12, 197, 64, 15, 14)
    assert ma.launch_names(p) == ["qbar", "stage1_last", "stage2_last"]
    full = ma.make_problem(1, 12, 210, 64, 15, 14)
    assert ma.launch_names(full) == ["stage1_last", "stage2_last"]
    assert ma.workspace_size(p) >= ma.workspace_size(full)


def test_status_strings(lib):
    for s in range(5):
        assert lib.monarch_attn_status_string(s)
    assert ma.version()


@pytest.mark.parametrize("kw,code", [
    (dict(), 0),
    (dict(steps=2), 0),                       # T > 1: unrolled steps
    (dict(steps=3, dtype="f32", head_dim=128, seq_len=64 * 64, b1=64, b2=64), 0),
    (dict(steps=2, seq_len=250), 0),          # T > 1 padded
    (dict(steps=2, seq_len=200 * 8, b1=200, b2=8), 0),   # T > 1: columns over one key chunk
    (dict(steps=2, head_dim=128), 0),         # T > 1 bf16 at head_dim 128: 64-key blocks
    (dict(steps=2, head_dim=128, seq_len=96 * 16, b1=96, b2=16), 0),   # ... columns over 64 keys
    (dict(steps=2, head_dim=128, seq_len=16 * 96, b1=16, b2=96), 2),   # ... blocks over 64 keys
    (dict(steps=2, kv_heads=1), 0),           # T > 1 grouped K/V
    (dict(c1=2), 0),                          # row tiles
    (dict(c1=2, c2=4), 0),                    # row tiles and key segments
    (dict(c1=2, steps=2), 0),                 # tiled T > 1
    (dict(c1=2, c2=2, steps=2, seq_len=250), 0),   # tiled T > 1 padded
    (dict(c2=2, seq_len=250), 0),             # tiled and padded
    (dict(c1=4, c2=2, seq_len=250, flags=ma.MA_FLAG_PAD_FRONT), 0),   # tiled, padded in front
    (dict(kv_heads=1), 0),                    # grouped K/V
    (dict(seq_len=250), 0),                   # padded
    (dict(seq_len=256 * 200, b1=200, b2=256), 2),   # blocks wider than 128 keys
    (dict(seq_len=630 * 52, b1=630, b2=52), 0),     # columns of 630 keys (walked in chunks)
    (dict(seq_len=4096 * 8, b1=4096, b2=8), 0),     # columns of 4096 keys
    (dict(seq_len=96 * 96, b1=96, b2=96, head_dim=128, dtype="f32"), 2),   # fp32 d128: 64 max
    (dict(seq_len=64 * 64, b1=64, b2=64, head_dim=128, dtype="f32"), 0),
    (dict(steps=0), 1),
    (dict(causal=1), 0),                      # block-causal
    (dict(causal=16), 0),                     # a unit of all 16 blocks masks nothing
    (dict(causal=-1), 1),
])
def test_backward_validation(lib, kw, code):
    p = good(**kw)
    n = ctypes.c_size_t()
    assert lib.monarch_attn_backward_workspace_size(ctypes.byref(p), ctypes.byref(n)) == code
    if code == 0:
        assert n.value >= ma.workspace_size(p)
        # null pointers and a short workspace are rejected before any HIP call
        assert lib.monarch_attn_backward(ctypes.byref(p), 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, None) == 1
        q, k, v, dy, dq, dk, dv, y = (256 * 1024 * 1024 * (j + 1) for j in range(8))
        assert lib.monarch_attn_backward(ctypes.byref(p), q, k, v, None, dy, dq, dk, dv, 1 << 40, 10,
                                         None) == 3
        assert lib.monarch_attn_backward(ctypes.byref(p), q, k, v, y, dy, dq, dk, dv, 1 << 40, 10,
                                         None) == 3
        assert lib.monarch_attn_backward(ctypes.byref(p), q, k, v, None, dy, dq, dq, dv, 1 << 40,
                                         n.value, None) == 1      # dK overlaps dQ
        assert lib.monarch_attn_backward(ctypes.byref(p), q, k, v, dq, dy, dq, dk, dv, 1 << 40,
                                         n.value, None) == 1      # y overlaps dQ
        assert lib.monarch_attn_backward(ctypes.byref(p), q, k, v, y + 4, dy, dq, dk, dv, 1 << 40,
                                         n.value, None) == 1      # y misaligned


@pytest.mark.parametrize("kw,code", [
    (dict(), 1),                                   # layouts agree: the pointer checks run (null -> 1)
    (dict(dtype="f32"), 1),
    (dict(c1=2, c2=2), 1),
    (dict(seq_len=250), 1),
    (dict(steps=2), 2),                            # per-step state: nothing to reuse
    (dict(flags=8), 2),                            # bf16 split aggregate: not the backward's c path
])
def test_backward_reuse_forward_state_layouts(lib, kw, code):
    """MA_FLAG_REUSE_FORWARD_STATE is accepted only where the forward's state
    regions are the backward's; the check runs before any HIP call."""
    flags = kw.pop("flags", 0) | ma.MA_FLAG_REUSE_FORWARD_STATE
    p = good(flags=flags, **kw)
    assert lib.monarch_attn_backward(ctypes.byref(p), 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, None) == code


def test_noalloc_scratch_size_and_host_refusals(lib):
    """The no-alloc entry point's scratch size in the header matches the
    binding, and problems it cannot take are refused on the host, before any
    HIP call: a workspace larger than the scratch array, the fused launch,
    and invalid problems."""
    text = open(HEADER).read()
    m = re.search(r"#define\s+MONARCH_ATTN_SCRATCH_BYTES\s+\((\d+)u\s*<<\s*(\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == _lib.MONARCH_ATTN_SCRATCH_BYTES
    q, k, v, y = (256 * 1024 * 1024 * (j + 1) for j in range(4))
    video = ma.make_problem(1, 12, 32760, 128, 630, 52, dtype="bf16", layout="fh_w", fhw=(21, 30, 52))
    assert ma.workspace_size(video) > _lib.MONARCH_ATTN_SCRATCH_BYTES
    assert lib.monarch_attn_forward_noalloc(ctypes.byref(video), q, k, v, y, None, None) == 3
    fused = good(flags=ma.MA_FLAG_FORCE_FUSED)
    assert lib.monarch_attn_forward_noalloc(ctypes.byref(fused), q, k, v, y, None, None) == 2
    assert lib.monarch_attn_forward_noalloc(ctypes.byref(good(steps=0)), q, k, v, y, None, None) == 1
    assert lib.monarch_attn_forward_noalloc(ctypes.byref(good()), 0, k, v, y, None, None) == 1
    n16k = ma.make_problem(1, 12, 16384, 64, 128, 128, dtype="bf16")
    assert ma.workspace_size(n16k) <= _lib.MONARCH_ATTN_SCRATCH_BYTES
