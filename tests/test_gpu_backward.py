"""Parity of the HIP backward pass (through the C ABI) with the gradient
oracle (oracle.backward: float64 autograd of the forward's steps).

Every case compares dQ, dK and dV of whole slices with the per-slice relative
error max|X - X_ref| / max|X_ref| (1e-4 for fp32 inputs, 2e-2 for bf16), on
seeded synthetic inputs and a seeded upstream gradient dY."""

import numpy as np
import pytest

from oracle import backward as obw
from workloads import WORKLOADS, WorkloadConfig, make_inputs
from workloads.generators import round_to_bf16
from parity_utils import TOL, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import structured_sub_quadratic_amd as ma
    ma._lib.load()          # raise loudly if the library is missing


def run_backward(cfg, Q, K, V, dY, with_y=False, causal=0):
    import torch
    import structured_sub_quadratic_amd as ma
    dt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
    dev = torch.device("cuda:0")
    tq, tk, tv, tdy = (torch.from_numpy(np.ascontiguousarray(x)).to(dev).to(dt) for x in (Q, K, V, dY))
    y = None
    if with_y:        # the forward's output: row sums of the softmax gradient from dY . y
        y = ma.forward(tq, tk, tv, cfg.b1, cfg.b2, cfg.steps, cfg.c1, cfg.c2, layout=cfg.layout,
                       fhw=cfg.fhw, pad=cfg.pad, causal=causal)
    dq, dk, dv = ma.backward(tq, tk, tv, tdy, cfg.b1, cfg.b2, cfg.steps, cfg.c1, cfg.c2,
                             layout=cfg.layout, fhw=cfg.fhw, pad=cfg.pad, y=y, causal=causal)
    torch.cuda.synchronize()
    return tuple(x.float().cpu().numpy() for x in (dq, dk, dv))


def upstream(cfg, seed=77):
    dY = np.random.default_rng(seed).standard_normal(
        (cfg.batch, cfg.heads, cfg.seq_len, cfg.head_dim)).astype(np.float32)
    return round_to_bf16(dY) if cfg.dtype == "bf16" else dY


def check_backward(cfg, slices=None, tol=None, kv_heads=None, with_y=False, causal=0):
    Q, K, V = make_inputs(cfg)
    if kv_heads is not None:        # grouped-query attention: keep the first kv_heads
        K, V = (np.ascontiguousarray(X[:, :kv_heads]) for X in (K, V))
    dY = upstream(cfg)
    got = run_backward(cfg, Q, K, V, dY, with_y, causal)
    all_slices = [(b, h) for b in range(cfg.batch) for h in range(cfg.heads)]
    slices = all_slices if slices is None else slices
    ref = obw.backward(Q, K, V, dY, cfg.b1, cfg.b2, cfg.steps, cfg.c1, cfg.c2,
                       layout=cfg.layout, fhw=cfg.fhw, slices=slices, pad=cfg.pad, causal=causal)
    tol = TOL[cfg.dtype] if tol is None else tol
    group = cfg.heads // K.shape[1]
    kv_slices = sorted({(b, h // group) for (b, h) in slices})
    errs = {n: rel_err(g, r, slices if n == "dQ" else kv_slices)
            for n, g, r in zip(("dQ", "dK", "dV"), got, ref)}
    print(cfg.name, {k: f"{v:.2e}" for k, v in errs.items()})
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"{cfg.name}: {errs} (tol {tol})"
    return got


def case(name, dtype, d, b1, b2, batch=1, heads=2, data="normed", layout="flat", fhw=None, seed=61,
         steps=1, c1=1, c2=1):
    return WorkloadConfig("case", name, batch=batch, heads=heads, seq_len=b1 * b2, head_dim=d,
                          b1=b1, b2=b2, steps=steps, dtype=dtype, data=data, seed=seed,
                          layout=layout, fhw=fhw, c1=c1, c2=c2)


def test_n256_backward():
    check_backward(WORKLOADS["n256"])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
def test_ragged_blocks(dtype, d):
    """b1 = 52, b2 = 40 (neither a multiple of 32) for fp32 head_dim 128's
    64-key limit; 70 x 52 otherwise."""
    b1, b2 = (52, 40) if (dtype == "f32" and d == 128) else (70, 52)
    check_backward(case(f"bwd ragged {dtype} d{d}", dtype, d, b1, b2, data="iid"))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_full_blocks(dtype):
    """128 x 128 keys per block and per column (64 x 64 for fp32 head_dim 128)."""
    check_backward(case(f"bwd 128x96 {dtype}", dtype, 64, 128, 96, heads=2))
    b = 64 if dtype == "f32" else 128
    check_backward(case(f"bwd {b}x{b} {dtype} d128", dtype, 128, b, b, heads=1, seed=62))


@pytest.mark.parametrize("dtype,d,b1", [("bf16", 64, 300), ("f32", 64, 200), ("bf16", 128, 150),
                                         ("f32", 128, 130)])
def test_columns_over_one_key_chunk(dtype, d, b1):
    """Stage-2 columns of more than 128 (fp32 head_dim 128: 64) keys: the
    keys are walked in chunks, D = rowsum(P dP) takes a first sweep, and dQ
    accumulates over the chunks."""
    b2 = 40 if (dtype == "f32" and d == 128) else 52
    check_backward(case(f"bwd b1={b1} {dtype} d{d}", dtype, d, b1, b2, heads=1, data="normed"))


def test_video_layout():
    cfg = case("bwd video w_fh", "bf16", 128, 8, 15, data="video", layout="w_fh", fhw=(3, 5, 8))
    check_backward(cfg)


def test_linear_in_upstream_and_zero():
    """dQ, dK, dV are linear in dY: zero for dY = 0, doubled for 2 dY."""
    cfg = case("bwd linear", "f32", 64, 16, 16)
    Q, K, V = make_inputs(cfg)
    dY = upstream(cfg)
    g1 = run_backward(cfg, Q, K, V, dY)
    g2 = run_backward(cfg, Q, K, V, 2 * dY)
    g0 = run_backward(cfg, Q, K, V, 0 * dY)
    for a, b, z in zip(g1, g2, g0):
        assert np.abs(z).max() == 0
        np.testing.assert_allclose(b, 2 * a, rtol=1e-5, atol=1e-6 * np.abs(a).max())


@pytest.mark.parametrize("dtype,kvh", [("f32", 1), ("bf16", 2)])
def test_grouped_query_attention(dtype, kvh):
    """Four query heads over kv_heads K/V heads: dK, dV sum the group's shares."""
    cfg = case(f"bwd gqa {dtype} kv{kvh}", dtype, 64, 40, 52, batch=2, heads=4)
    check_backward(cfg, kv_heads=kvh)


def test_n16k_backward_sampled():
    """The 16k-token headline shape (12 heads); the oracle differentiates two
    slices, compared whole."""
    check_backward(WORKLOADS["n16k"], slices=[(0, 0), (0, 11)])


def test_video_backward_sampled():
    """The video latent (630, 52), d = 128, 12 heads: two slices compared whole."""
    check_backward(WORKLOADS["video"], slices=[(0, 0), (0, 7)])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("b1,b2", [(1, 40), (40, 1), (1, 1), (3, 5)])
def test_degenerate_grids(dtype, b1, b2):
    """One block (exact attention), one key per block, a single token, and a
    grid smaller than one MFMA tile."""
    check_backward(case(f"bwd {b1}x{b2} {dtype}", dtype, 64, b1, b2, heads=2, data="iid"))


@pytest.mark.parametrize("pad", ["pre", "post"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_padded_vit_shape(pad, dtype):
    """197 tokens as 15 blocks of 14 (13 padding positions): padding keys get
    no gradient, and the query gradient of a padding position goes through
    the tile mean of its column."""
    cfg = WorkloadConfig("case", f"bwd vit pad={pad} {dtype}", batch=2, heads=3, seq_len=197,
                         head_dim=64, b1=15, b2=14, steps=1, dtype=dtype, data="iid", seed=53,
                         pad=pad)
    check_backward(cfg)


@pytest.mark.parametrize("pad", ["pre", "post"])
def test_padded_long_columns(pad):
    """Padding with columns of more than one key chunk (b1 = 200), head_dim 128."""
    cfg = WorkloadConfig("case", f"bwd b1=200 pad={pad}", batch=1, heads=2, seq_len=200 * 40 - 30,
                         head_dim=128, b1=200, b2=40, steps=1, dtype="bf16", data="normed", seed=59,
                         pad=pad)
    check_backward(cfg)


# ---------------------------------------------------------------------------
# T > 1: the gradient through the unrolled steps (each step's L feeds the next
# step's queries q~ = sum_l L q / sum_l L).
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,d,steps", [("f32", 64, 2), ("f32", 64, 3), ("f32", 128, 2),
                                           ("bf16", 64, 2), ("bf16", 64, 3), ("bf16", 128, 2),
                                           ("bf16", 128, 3)])
def test_unrolled_steps_ragged(dtype, d, steps):
    """Ragged blocks (neither b1 nor b2 a multiple of 32); head_dim 128 within
    its 64-key limit."""
    b1, b2 = (52, 40) if d == 128 else (70, 52)
    check_backward(case(f"bwd T={steps} {dtype} d{d}", dtype, d, b1, b2, data="iid", steps=steps))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_unrolled_steps_full_blocks(dtype):
    """128 x 128 at head_dim 64, 64 x 64 (the 64-key builds) at both."""
    check_backward(case(f"bwd T=2 128x128 {dtype}", dtype, 64, 128, 128, heads=2, steps=2))
    check_backward(case(f"bwd T=2 64x64 {dtype} d128", dtype, 128, 64, 64, heads=1, steps=2, seed=63))
    check_backward(case(f"bwd T=2 64x64 {dtype} d64", dtype, 64, 64, 64, heads=2, steps=2, seed=64))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("b1,b2", [(1, 40), (40, 1), (3, 5)])
def test_unrolled_steps_degenerate(dtype, b1, b2):
    """One block (every step is exact attention), one key per block, a grid
    smaller than one MFMA tile; T = 2."""
    check_backward(case(f"bwd T=2 {b1}x{b2} {dtype}", dtype, 64, b1, b2, heads=2, data="iid", steps=2))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_unrolled_steps_grouped_kv(dtype):
    """Four query heads over two K/V heads, T = 2."""
    cfg = case(f"bwd T=2 gqa {dtype}", dtype, 64, 40, 52, batch=2, heads=4, steps=2)
    check_backward(cfg, kv_heads=2)


def test_n4k_t3_backward_sampled():
    """The T = 3 workload (batch 8 x 12 heads, 64 x 64 blocks, low-rank data):
    two slices compared whole."""
    check_backward(WORKLOADS["n4k_t3"], slices=[(0, 0), (7, 11)])


# ---------------------------------------------------------------------------
# Row tiles and key segments (T = 1): each block's R rows run per (row tile,
# key segment), with the tile mean as the query of the other tiles.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("c1,c2", [(2, 2), (2, 1), (1, 2), (4, 4)])
def test_tiled_small(dtype, c1, c2):
    check_backward(case(f"bwd tiled {c1}x{c2} {dtype}", dtype, 64, 16, 16, data="iid", c1=c1, c2=c2))


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 64), ("f32", 128), ("bf16", 128)])
def test_tiled_ragged(dtype, d):
    """Three row tiles of 16 rows, two segments of 26 keys (neither a
    multiple of 32)."""
    check_backward(case(f"bwd tiled ragged {dtype} d{d}", dtype, d, 48, 52, data="normed", c1=3, c2=2))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_tiled_columns_over_one_key_chunk(dtype):
    """b1 * c2 = 200 stage-2 keys per (row tile, column): the key-chunk path."""
    check_backward(case(f"bwd tiled b1=100 {dtype}", dtype, 64, 100, 24, heads=1, c1=2, c2=2))


def test_tiled_grouped_kv():
    cfg = case("bwd tiled gqa", "bf16", 64, 32, 24, batch=2, heads=4, c1=2, c2=3)
    check_backward(cfg, kv_heads=1)


def test_video_tiled_backward_sampled():
    """The tiled video latent (630 x 52, c1 = c2 = 2, d = 128, 12 heads): two
    slices compared whole."""
    check_backward(WORKLOADS["video_tiled"], slices=[(0, 0), (0, 5)])


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 64), ("f32", 128), ("bf16", 128)])
@pytest.mark.parametrize("c1,c2", [(2, 2), (2, 1), (1, 2), (4, 2)])
def test_tiled_unrolled_steps(dtype, d, c1, c2):
    """Row tiles and key segments at T = 2: each step's tiled L gives the
    next queries q~[k, i, t, s] = alpha / beta over the rows of tile t."""
    check_backward(case(f"bwd tiled {c1}x{c2} T=2 {dtype} d{d}", dtype, d, 16, 16, data="iid", c1=c1, c2=c2,
                        steps=2))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_tiled_unrolled_steps_ragged(dtype):
    """T = 3 with ragged tiles: 48 blocks of 52 as 3 x 2 tiles."""
    check_backward(case(f"bwd tiled 3x2 T=3 ragged {dtype}", dtype, 64, 48, 52, data="normed", c1=3, c2=2,
                        steps=3))


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("f32", 128), ("bf16", 128)])
def test_tiled_unrolled_steps_long_columns(dtype, d):
    """T = 2, 2 x 2 tiles with columns of 200 stage-2 keys (several chunks)."""
    b2 = 24 if d == 64 else 16
    check_backward(case(f"bwd tiled 2x2 T=2 b1=100 {dtype} d{d}", dtype, d, 100, b2, heads=1, c1=2, c2=2,
                        steps=2))


@pytest.mark.parametrize("pad", ["pre", "post"])
@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 64), ("bf16", 128)])
def test_tiled_unrolled_steps_padded(pad, dtype, d):
    """T = 2 with 3 x 2 tiles on 205 tokens in 15 blocks of 14: padding
    positions start from the tile means and carry no L row at any step."""
    cfg = WorkloadConfig("case", f"bwd tiled T=2 pad={pad} {dtype} d{d}", batch=1, heads=2,
                         seq_len=15 * 14 - 5, head_dim=d, b1=15, b2=14, steps=2, dtype=dtype, data="iid",
                         seed=73, c1=3, c2=2, pad=pad)
    check_backward(cfg)


def test_tiled_unrolled_steps_grouped_kv():
    cfg = case("bwd tiled T=2 gqa", "bf16", 64, 32, 24, batch=2, heads=4, c1=2, c2=3, steps=2)
    check_backward(cfg, kv_heads=1)


@pytest.mark.parametrize("pad", ["pre", "post"])
@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 64), ("f32", 128), ("bf16", 128)])
def test_tiled_padded(pad, dtype, d):
    """Row tiles and key segments on a padded sequence: 205 tokens as 15
    blocks of 14 (c1 = 3 tiles of 5 rows, c2 = 2 segments of 7 keys), so the
    padded block keeps 2 real keys in one segment.  The tile means average
    the real rows only, a padding position's query gradient goes to them,
    and padding keys get none."""
    cfg = WorkloadConfig("case", f"bwd tiled pad={pad} {dtype} d{d}", batch=2, heads=2,
                         seq_len=15 * 14 - 5, head_dim=d, b1=15, b2=14, steps=1, dtype=dtype,
                         data="iid", seed=67, c1=3, c2=2, pad=pad)
    check_backward(cfg)


@pytest.mark.parametrize("pad", ["pre", "post"])
def test_tiled_padded_long_columns(pad):
    """Tiled and padded with columns of more than one key chunk (b1 = 200,
    c1 = 4, c2 = 2), the upstream row sums taken from the forward's output."""
    cfg = WorkloadConfig("case", f"bwd tiled b1=200 pad={pad}", batch=1, heads=1,
                         seq_len=200 * 24 - 9, head_dim=64, b1=200, b2=24, steps=1, dtype="bf16",
                         data="normed", seed=68, c1=4, c2=2, pad=pad)
    check_backward(cfg, with_y=True)


@pytest.mark.parametrize("pad", ["pre", "post"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_unrolled_steps_padded_vit(pad, dtype):
    """197 tokens as 15 blocks of 14 at T = 2 (the ViT case): padding rows
    hold no L row at either step, padding keys no R mass, and a padding
    position's first query is the tile mean of its column."""
    cfg = WorkloadConfig("case", f"bwd T=2 vit pad={pad} {dtype}", batch=2, heads=3, seq_len=197,
                         head_dim=64, b1=15, b2=14, steps=2, dtype=dtype, data="iid", seed=57,
                         pad=pad)
    check_backward(cfg)


@pytest.mark.parametrize("dtype,d", [("f32", 128), ("bf16", 128), ("bf16", 64)])
def test_unrolled_steps_padded(dtype, d):
    """Ragged padded grids at T = 3: 52 x 40 less 20 positions in front."""
    cfg = WorkloadConfig("case", f"bwd T=3 pad {dtype} d{d}", batch=1, heads=2, seq_len=52 * 40 - 20,
                         head_dim=d, b1=52, b2=40, steps=3, dtype=dtype, data="normed", seed=58,
                         pad="pre")
    check_backward(cfg)


@pytest.mark.parametrize("dtype,d,b1,b2", [("f32", 64, 200, 8), ("bf16", 64, 300, 6), ("f32", 128, 100, 12),
                                           ("bf16", 128, 96, 16), ("bf16", 128, 150, 8)])
def test_unrolled_steps_long_columns(dtype, d, b1, b2):
    """T = 2 with stage-2 columns of several key chunks (128 keys a chunk,
    64 for fp32 and for bf16 at head_dim 128): each step takes a D pass and
    one workgroup per key chunk, the earlier step through alpha and beta."""
    check_backward(case(f"bwd T=2 long columns {dtype} d{d} b1={b1}", dtype, d, b1, b2, heads=2, steps=2))


@pytest.mark.parametrize("with_y", [False, True])
def test_unrolled_steps_long_columns_padded(with_y):
    """T = 3, 200 blocks of 10 less 7 padding positions in front, grouped K/V;
    with_y: the last step's row sums come from the forward's output."""
    cfg = WorkloadConfig("case", f"bwd T=3 long padded y={with_y}", batch=1, heads=4, seq_len=200 * 10 - 7,
                         head_dim=64, b1=200, b2=10, steps=3, dtype="bf16", data="normed", seed=71,
                         pad="pre")
    check_backward(cfg, kv_heads=2, with_y=with_y)


def test_n16k_pad_t2_backward_sampled():
    """The padded headline shape (16284 tokens, 100 padding positions in
    front) at T = 2: two slices compared whole."""
    cfg = WorkloadConfig("case", "bwd T=2 n16k pad", batch=1, heads=12, seq_len=16284, head_dim=64,
                         b1=128, b2=128, steps=2, dtype="bf16", data="normed", seed=1006, pad="pre")
    check_backward(cfg, slices=[(0, 0), (0, 11)])


@pytest.mark.parametrize("name,kw", [
    ("bf16", dict(dtype="bf16", d=64, b1=70, b2=52)),
    ("f32 d128", dict(dtype="f32", d=128, b1=52, b2=40)),
    ("tiled", dict(dtype="bf16", d=64, b1=48, b2=52, c1=3, c2=2)),
    # the forward as one cooperative launch leaves the same state, the bf16
    # tile means of tiled and padded problems included
    ("fused bf16", dict(dtype="bf16", d=128, b1=40, b2=100, fused=True)),
    ("fused tiled", dict(dtype="bf16", d=64, b1=48, b2=52, c1=3, c2=2, fused=True)),
    ("fused padded", dict(dtype="bf16", d=64, b1=70, b2=52, pad=20, fused=True)),
    ("fused padded front", dict(dtype="bf16", d=128, b1=30, b2=40, pad=7, front=True, fused=True)),
])
def test_reuse_forward_state(name, kw):
    """A forward call given the backward's workspace leaves its state there;
    the backward with reuse_forward_state skips rebuilding it and gives the
    gradients of the rebuilding call (fp32 to 1e-6; bf16 outputs may differ
    by one bf16 step (2^-8 of the largest), since the forward's output launch and the rebuild's
    statistics launch reach the same normalisers by different code)."""
    import torch
    import structured_sub_quadratic_amd as ma
    padn = kw.get("pad", 0)
    pad = "pre" if kw.get("front") else "post"
    cfg = WorkloadConfig("case", f"bwd reuse {name}", batch=1, heads=2,
                         seq_len=kw["b1"] * kw["b2"] - padn, head_dim=kw["d"], b1=kw["b1"],
                         b2=kw["b2"], steps=1, dtype=kw["dtype"], data="normed", seed=61,
                         c1=kw.get("c1", 1), c2=kw.get("c2", 1), pad=pad)
    Q, K, V = make_inputs(cfg)
    dY = upstream(cfg)
    dt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
    dev = torch.device("cuda:0")
    tq, tk, tv, tdy = (torch.from_numpy(np.ascontiguousarray(x)).to(dev).to(dt) for x in (Q, K, V, dY))
    prob = ma.make_problem(cfg.batch, cfg.heads, cfg.seq_len, cfg.head_dim, cfg.b1, cfg.b2, 1,
                           cfg.c1, cfg.c2, None, cfg.dtype,
                           flags=ma.MA_FLAG_PAD_FRONT if pad == "pre" else 0)
    ws = torch.empty(ma.backward_workspace_size(prob), dtype=torch.uint8, device=dev)
    ws.fill_(0xFF)          # what the forward leaves must be all the backward reads
    args = (cfg.b1, cfg.b2, 1, cfg.c1, cfg.c2)
    ref = ma.backward(tq, tk, tv, tdy, *args, pad=pad)
    ma.forward(tq, tk, tv, *args, workspace=ws, pad=pad, force_fused=kw.get("fused", False))
    got = ma.backward(tq, tk, tv, tdy, *args, workspace=ws, reuse_forward_state=True, pad=pad)
    torch.cuda.synchronize()
    for g, r in zip(got, ref):
        g, r = g.float().cpu().numpy(), r.float().cpu().numpy()
        assert np.isfinite(g).all(), name
        assert np.abs(g - r).max() <= (1e-6 if cfg.dtype == "f32" else 2.0 ** -7) * np.abs(r).max(), name


@pytest.mark.parametrize("dtype,d,b1", [("bf16", 64, 300), ("f32", 128, 130), ("bf16", 128, 150)])
def test_long_columns_with_output(dtype, d, b1):
    """Columns over one key chunk given the forward's output: the row sums
    D come from dY . y instead of the D pass."""
    b2 = 40 if (dtype == "f32" and d == 128) else 52
    check_backward(case(f"bwd y b1={b1} {dtype} d{d}", dtype, d, b1, b2, heads=1), with_y=True)


@pytest.mark.parametrize("variant", ["pad", "tiled", "video"])
def test_long_columns_with_output_variants(variant):
    if variant == "pad":
        cfg = WorkloadConfig("case", "bwd y b1=200 pad=pre", batch=1, heads=2, seq_len=200 * 40 - 30,
                             head_dim=128, b1=200, b2=40, steps=1, dtype="bf16", data="normed",
                             seed=59, pad="pre")
        check_backward(cfg, with_y=True)
    elif variant == "tiled":
        check_backward(case("bwd y tiled b1=100", "bf16", 64, 100, 24, heads=1, c1=2, c2=2), with_y=True)
    else:
        check_backward(WORKLOADS["video"], slices=[(0, 0), (0, 7)], with_y=True)


VIDEO_LAYOUTS = {"fh_w": (15, 8), "w_fh": (8, 15), "f_hw": (3, 40), "hw_f": (40, 3),
                 "fw_h": (24, 5), "h_fw": (5, 24)}


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("layout", sorted(VIDEO_LAYOUTS))
def test_video_layouts(layout, dtype):
    """Every aligned video layout of a 3 x 5 x 8 latent (rows and columns of
    the grid gather strided tokens)."""
    b1, b2 = VIDEO_LAYOUTS[layout]
    check_backward(case(f"bwd {layout} {dtype}", dtype, 64, b1, b2, data="video", layout=layout,
                        fhw=(3, 5, 8)))


@pytest.mark.parametrize("variant", ["steps", "tiled"])
def test_video_layout_variants(variant):
    """A video layout at T = 2, and with row tiles and key segments."""
    if variant == "steps":
        cfg = case("bwd fh_w T=2", "bf16", 64, 15, 8, data="video", layout="fh_w", fhw=(3, 5, 8),
                   steps=2)
    else:
        cfg = case("bwd fh_w tiled", "bf16", 128, 15, 8, data="video", layout="fh_w", fhw=(3, 5, 8),
                   c1=3, c2=2)
    check_backward(cfg)


@pytest.mark.parametrize("case", ["video", "tiled", "tiled_t2_causal"])
def test_backward_is_deterministic(case):
    """Two backward calls on the same inputs give bitwise equal dQ, dK, dV:
    columns of several key chunks write one dQ part per chunk, summed in
    chunk order (at earlier steps onto the later steps' sum), and the row
    sums of the softmax gradients are added in strip order, so nothing
    depends on the timing of workgroups or waves.  The video latent's
    630-key columns run five key chunks; the last case runs T = 2 with tiles
    and a block-causal mask over 600-key columns."""
    import torch
    import structured_sub_quadratic_amd as ma
    causal = 0
    if case == "video":
        cfg = WORKLOADS["video"]
    elif case == "tiled":
        cfg = WorkloadConfig("case", "bwd det tiled", batch=1, heads=3, seq_len=300 * 24,
                                        head_dim=64, b1=300, b2=24, steps=1, dtype="bf16",
                                        data="normed", seed=63, c1=2, c2=2)
    else:
        cfg = WorkloadConfig("case", "bwd det tiled T=2 causal", batch=1, heads=2, seq_len=300 * 24,
                             head_dim=64, b1=300, b2=24, steps=2, dtype="bf16", data="normed", seed=64,
                             c1=2, c2=2)
        causal = 50
    Q, K, V = make_inputs(cfg)
    dY = upstream(cfg)
    dev = torch.device("cuda:0")
    tq, tk, tv, tdy = (torch.from_numpy(np.ascontiguousarray(x)).to(dev).to(torch.bfloat16)
                       for x in (Q, K, V, dY))
    args = dict(b1=cfg.b1, b2=cfg.b2, steps=cfg.steps, c1=cfg.c1, c2=cfg.c2, layout=cfg.layout, fhw=cfg.fhw,
                causal=causal)
    first = [g.clone() for g in ma.backward(tq, tk, tv, tdy, **args)]
    for _ in range(2):
        again = ma.backward(tq, tk, tv, tdy, **args)
        torch.cuda.synchronize()
        for name, a, b in zip(("dQ", "dK", "dV"), first, again):
            assert torch.equal(a, b), (case, name)


# ---------------------------------------------------------------------------
# Block-causal use: query block l takes key block k only when
# floor(k / g) <= floor(l / g); the masked L entries carry no gradient.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("g,steps,c1,c2", [(1, 1, 1, 1), (4, 1, 1, 1), (2, 1, 2, 2), (1, 2, 1, 1), (2, 3, 1, 1),
                                           (2, 2, 2, 2)])
def test_block_causal(dtype, g, steps, c1, c2):
    cfg = case(f"bwd causal g={g} T={steps} {c1}x{c2} {dtype}", dtype, 64, 16, 16, data="iid", steps=steps,
               c1=c1, c2=c2)
    check_backward(cfg, causal=g)


@pytest.mark.parametrize("with_y", [False, True])
@pytest.mark.parametrize("steps", [1, 2])
def test_block_causal_long_columns(with_y, steps):
    """200 blocks of 8 in causal units of 16 blocks, head_dim 128: the key
    chunks past a row's bound hold only masked entries."""
    cfg = case(f"bwd causal long T={steps} y={with_y}", "bf16", 128, 200, 8, heads=2, steps=steps)
    check_backward(cfg, causal=16, with_y=with_y)


@pytest.mark.parametrize("pad", ["pre", "post"])
def test_block_causal_padded(pad):
    cfg = WorkloadConfig("case", f"bwd causal vit pad={pad}", batch=1, heads=2, seq_len=197, head_dim=64,
                         b1=15, b2=14, steps=2, dtype="bf16", data="iid", seed=79, pad=pad)
    check_backward(cfg, causal=3)


def test_block_causal_video_frames():
    """A 4 x 6 x 8 latent in the (fh, w) layout with units of h = 6 blocks:
    causal over frames."""
    cfg = WorkloadConfig("case", "bwd causal frames", batch=1, heads=2, seq_len=4 * 6 * 8, head_dim=64,
                         b1=24, b2=8, steps=1, dtype="bf16", data="normed", seed=81, layout="fh_w",
                         fhw=(4, 6, 8))
    check_backward(cfg, causal=6)
