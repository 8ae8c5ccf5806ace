"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Small cases are compared element by element on Y, L, R, the row
log-normalisers and the objective; the five benchmark workloads run at their
full sizes in the launch configuration the benchmark times, and are compared
on every output of sampled slices and columns (each column i of a slice is an
independent sub-problem the oracle can compute on its own: R rows [., i, .],
L[i] and y[., i] depend only on column i of the queries and on all keys)."""

import math

import numpy as np
import pytest

import oracle
from workloads import WORKLOADS, WorkloadConfig, make_inputs
from parity_utils import TOL, rel_err, oracle_L_as_gpu, oracle_R_as_gpu, run_hip

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import structured_sub_quadratic_amd as ma
    ma._lib.load()          # raise loudly if the library is missing


def check_case(cfg, slices=None, cols=None, exports=("L", "R", "lse", "objective"),
               noise=None, tol=None, kv_heads=None, **kw):
    """Run the HIP path once on the whole problem, then compare every
    requested slice with the oracle run on that slice alone (so that the
    oracle's memory stays that of one slice at the full sizes)."""
    all_slices = [(b, h) for b in range(cfg.batch) for h in range(cfg.heads)]
    slices = all_slices if slices is None else slices
    Q, K, V = make_inputs(cfg, noise_scale=noise)
    if kv_heads is not None:        # grouped-query attention: keep the first kv_heads
        K, V = (np.ascontiguousarray(X[:, :kv_heads]) for X in (K, V))
    group = cfg.heads // K.shape[1]
    causal = kw.get("causal", 0)
    y, ex = run_hip(cfg, Q, K, V, exports=exports, **kw)
    tiled = cfg.c1 * cfg.c2 > 1
    tol = TOL[cfg.dtype] if tol is None else tol
    errs = {}
    for (b, h) in slices:
        hk = h // group
        ref = oracle.forward(Q[b:b + 1, h:h + 1], K[b:b + 1, hk:hk + 1], V[b:b + 1, hk:hk + 1],
                             cfg.b1, cfg.b2, cfg.steps, cfg.c1, cfg.c2, layout=cfg.layout,
                             fhw=cfg.fhw, cols=cols, pad=cfg.pad, causal=causal)
        one = [(0, 0)]
        tok = ref["grid"][:, ref["cols"]].reshape(-1)
        tok = tok[tok >= 0]                 # padding positions have no token
        e = {"Y": rel_err(y[b:b + 1, h:h + 1, tok], ref["y"][:, :, tok], one)}
        if "L" in ex:
            e["L"] = rel_err(ex["L"][b:b + 1, h:h + 1, ref["cols"]],
                             oracle_L_as_gpu(ref["L"], tiled), one)
        if "R" in ex:
            e["R"] = rel_err(ex["R"][b:b + 1, h:h + 1, :, ref["cols"]],
                             oracle_R_as_gpu(ref["R"], tiled), one)
        if "lse" in ex:
            e["lse"] = rel_err(ex["lse"][b:b + 1, h:h + 1, tok], ref["lse"][:, :, tok], one)
        if "objective" in ex and cols is None:
            obj = ex["objective"].reshape(cfg.batch, cfg.heads)[b, h]
            ft = ref["f_trace"][0, 0, -1]
            e["objective"] = abs(obj - ft) / abs(ft)
        for k_, v_ in e.items():
            errs[k_] = max(errs.get(k_, 0.0), v_)
    print(cfg.name, f"{len(slices)} slices x {cfg.b2 if cols is None else len(cols)} columns",
          {k: f"{v:.2e}" for k, v in errs.items()})
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"{cfg.name}: {errs} (tol {tol})"
    return y, ex, None


# ----------------------------------------------------------------- small

def test_n256_full():
    check_case(WORKLOADS["n256"])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("steps", [1, 2])
def test_ragged_tiles_untiled(dtype, d, steps):
    """b1 = 70 (stage 2 streams 64 + 6 keys), b2 = 52 (stage 1 ragged)."""
    cfg = WorkloadConfig("case", f"ragged {dtype} d{d} T{steps}", batch=1, heads=2, seq_len=70 * 52,
                         head_dim=d, b1=70, b2=52, steps=steps, dtype=dtype, data="iid", seed=11)
    check_case(cfg)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("tiles,steps", [((1, 1), 1), ((2, 2), 2)])
def test_blocks_over_64_keys(dtype, d, tiles, steps):
    """b2 = 100: one 128-key LDS tile in stage 1, walked as a full and a
    partial 64-key chunk; b1 = 24 keeps stage 2 inside one chunk."""
    if dtype == "f32" and d == 128 and tiles == (1, 1):
        pytest.skip("fp32 head_dim 128 supports segments of at most 64 keys")
    cfg = WorkloadConfig("case", f"b2=100 {dtype} d{d} {tiles} T{steps}", batch=1, heads=2,
                         seq_len=24 * 100, head_dim=d, b1=24, b2=100, steps=steps, dtype=dtype,
                         data="normed", seed=29, c1=tiles[0], c2=tiles[1])
    check_case(cfg)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("tiles", [(2, 2), (2, 1), (1, 4), (5, 2)])
@pytest.mark.parametrize("steps", [1, 3])
def test_tiled(dtype, tiles, steps):
    cfg = WorkloadConfig("case", f"tiled {tiles} {dtype} T{steps}", batch=2, heads=1, seq_len=70 * 52,
                         head_dim=64, b1=70, b2=52, steps=steps, dtype=dtype, data="normed",
                         seed=12, c1=tiles[0], c2=tiles[1])
    check_case(cfg)


def test_multi_step_bf16_lowrank():
    cfg = WorkloadConfig("case", "lowrank T3", batch=2, heads=2, seq_len=96 * 40, head_dim=64,
                         b1=96, b2=40, steps=3, dtype="bf16", data="lowrank", seed=13)
    check_case(cfg)


@pytest.mark.parametrize("layout", ["fh_w", "w_fh", "f_hw", "hw_f", "fw_h", "h_fw"])
@pytest.mark.parametrize("steps", [1, 2])
def test_video_layouts(layout, steps):
    fhw = (3, 5, 8)
    sz = dict(f=3, h=5, w=8)
    a, b = layout.split("_")
    b1 = int(np.prod([sz[c] for c in a]))
    b2 = int(np.prod([sz[c] for c in b]))
    c1 = 3 if b1 % 3 == 0 else 1
    c2 = 2 if b2 % 2 == 0 else 1
    for tiles in ((1, 1), (c1, c2)):
        cfg = WorkloadConfig("case", f"video {layout} T{steps} tiles {tiles}", batch=1, heads=2,
                             seq_len=120, head_dim=128, b1=b1, b2=b2, steps=steps, dtype="bf16",
                             data="video", seed=14, layout=layout, fhw=fhw,
                             c1=tiles[0], c2=tiles[1])
        check_case(cfg)


def test_video_layouts_exact_without_noise_fp32():
    """Zero-noise per-axis codes: one step reproduces exact softmax attention
    in every aligned layout, on the GPU as in the oracle."""
    fhw = (3, 4, 10)
    sz = dict(f=3, h=4, w=10)
    base = WorkloadConfig("case", "video exact", batch=1, heads=1, seq_len=120, head_dim=64,
                          b1=12, b2=10, steps=1, dtype="f32", data="video", seed=15,
                          layout="fh_w", fhw=fhw)
    Q, K, V = make_inputs(base, noise_scale=0.0)
    exact = oracle.exact_attention(Q[0, 0].astype(np.float64), K[0, 0].astype(np.float64),
                                   V[0, 0].astype(np.float64), 1 / 8)
    for layout in ("fh_w", "w_fh", "f_hw", "hw_f", "fw_h", "h_fw"):
        a, b = layout.split("_")
        b1 = int(np.prod([sz[c] for c in a]))
        cfg = WorkloadConfig("case", layout, batch=1, heads=1, seq_len=120, head_dim=64, b1=b1,
                             b2=120 // b1, steps=1, dtype="f32", data="video", seed=15,
                             layout=layout, fhw=fhw)
        y, _ = run_hip(cfg, Q, K, V, exports=())
        err = np.abs(y[0, 0] - exact).max() / np.abs(exact).max()
        assert err < 1e-4, (layout, err)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_dense_limits(dtype):
    """b1 = 1 (one block of N keys) and b2 = 1 (N blocks of one key) are
    exact softmax attention."""
    for b1, b2 in ((1, 128), (300, 1)):
        cfg = WorkloadConfig("case", f"dense {b1}x{b2}", batch=1, heads=2, seq_len=b1 * b2,
                             head_dim=64, b1=b1, b2=b2, steps=2, dtype=dtype, data="iid", seed=16)
        Q, K, V = make_inputs(cfg)
        y, _ = run_hip(cfg, Q, K, V, exports=())
        for h in range(2):
            ex = oracle.exact_attention(*(X[0, h].astype(np.float64) for X in (Q, K, V)), 1 / 8)
            err = np.abs(y[0, h] - ex).max() / np.abs(ex).max()
            assert err < TOL[dtype], (b1, b2, h, err)


def test_single_token_and_tiny_grids():
    for (b1, b2) in ((1, 1), (2, 1), (1, 2), (3, 3)):
        cfg = WorkloadConfig("case", f"tiny {b1}x{b2}", batch=2, heads=3, seq_len=b1 * b2,
                             head_dim=64, b1=b1, b2=b2, steps=2, dtype="f32", data="iid", seed=17)
        check_case(cfg)


@pytest.mark.parametrize("fused", [False, True])
def test_timed_entry_point_times_every_launch(fused):
    """monarch_attn_forward_timed: the same output as the plain call, and a
    start and end time stamp for every launch, in launch order."""
    import torch
    import structured_sub_quadratic_amd as ma
    cfg = WorkloadConfig("case", "timed", batch=1, heads=2, seq_len=24 * 100, head_dim=64, b1=24,
                         b2=100, steps=1 if fused else 3, dtype="bf16", data="normed", seed=29)
    Q, K, V = make_inputs(cfg)
    dev = torch.device("cuda:0")
    tq, tk, tv = (torch.from_numpy(x).to(dev).to(torch.bfloat16) for x in (Q, K, V))
    prob = ma.make_problem(1, 2, cfg.seq_len, 64, 24, 100, cfg.steps, dtype="bf16",
                           flags=ma.MA_FLAG_FORCE_FUSED if fused else 0)
    names = ma.launch_names(prob)
    assert len(names) == (1 if fused else 2 * cfg.steps)
    events = [ma.Event() for _ in range(2 * len(names))]
    y_t = ma.forward_timed(tq, tk, tv, 24, 100, events, cfg.steps, force_fused=fused)
    y = ma.forward(tq, tk, tv, 24, 100, cfg.steps, force_fused=fused)
    torch.cuda.synchronize()
    assert torch.equal(y, y_t)
    for j in range(len(names)):
        assert events[2 * j].elapsed_ms(events[2 * j + 1]) > 0
        if j:
            assert events[2 * j - 1].elapsed_ms(events[2 * j]) >= 0


def test_determinism_and_reuse_of_workspace():
    import torch
    import structured_sub_quadratic_amd as ma
    cfg = WorkloadConfig("case", "det", batch=1, heads=3, seq_len=70 * 52, head_dim=128, b1=70,
                         b2=52, steps=2, dtype="bf16", data="normed", seed=18, c1=2, c2=2)
    Q, K, V = make_inputs(cfg)
    dev = torch.device("cuda:0")
    tq, tk, tv = (torch.from_numpy(x).to(dev).to(torch.bfloat16) for x in (Q, K, V))
    prob = ma.make_problem(1, 3, cfg.seq_len, 128, 70, 52, 2, 2, 2, dtype="bf16")
    ws = torch.empty(ma.workspace_size(prob), dtype=torch.uint8, device=dev)
    y1 = ma.forward(tq, tk, tv, 70, 52, 2, 2, 2, workspace=ws).clone()
    ws.fill_(0xFF)          # garbage (NaN patterns) left in the workspace must not matter
    y2 = ma.forward(tq, tk, tv, 70, 52, 2, 2, 2, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


@pytest.mark.parametrize("case", [
    dict(name="c1", dtype="f32", d=64, b1=16, b2=16, c=(1, 1), layout="flat", fhw=None, data="iid"),
    dict(name="ragged", dtype="bf16", d=128, b1=70, b2=52, c=(1, 1), layout="flat", fhw=None, data="iid"),
    dict(name="tiled", dtype="bf16", d=64, b1=70, b2=52, c=(2, 2), layout="flat", fhw=None, data="normed"),
    dict(name="video", dtype="bf16", d=128, b1=8, b2=15, c=(1, 3), layout="w_fh", fhw=(3, 5, 8), data="video"),
    dict(name="f32d128", dtype="f32", d=128, b1=40, b2=48, c=(2, 1), layout="flat", fhw=None, data="iid"),
    dict(name="wide", dtype="bf16", d=64, b1=12, b2=200, c=(3, 2), layout="flat", fhw=None, data="normed"),
    # blocks of 65..128 keys reach the copied-tile fused builds with 128-key
    # tiles: 8 waves at head_dim 64, 4 waves at head_dim 128 (ragged and full)
    dict(name="blk100 d64", dtype="bf16", d=64, b1=24, b2=100, c=(1, 1), layout="flat", fhw=None, data="normed"),
    dict(name="blk100 d128", dtype="bf16", d=128, b1=24, b2=100, c=(1, 1), layout="flat", fhw=None, data="normed"),
    dict(name="blk128 d128", dtype="bf16", d=128, b1=40, b2=128, c=(1, 1), layout="flat", fhw=None, data="iid"),
    dict(name="blk64 d64", dtype="bf16", d=64, b1=72, b2=64, c=(1, 1), layout="flat", fhw=None, data="iid"),
])
def test_t1_fused_and_staged_paths(case):
    """T = 1 as one cooperative launch and as the staged launch sequence: the
    same result, and both match the oracle."""
    cfg = WorkloadConfig("case", f"T1 {case['name']}", batch=2, heads=2, seq_len=case["b1"] * case["b2"],
                         head_dim=case["d"], b1=case["b1"], b2=case["b2"], steps=1, dtype=case["dtype"],
                         data=case["data"], seed=19, c1=case["c"][0], c2=case["c"][1],
                         layout=case["layout"], fhw=case["fhw"])
    y_f, _, _ = check_case(cfg, force_fused=True)
    y_s, _, _ = check_case(cfg, force_staged=True)
    scale = np.abs(y_s).max()
    assert np.abs(y_f - y_s).max() <= 1e-6 * scale


@pytest.mark.parametrize("steps", [1, 2])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_wide_blocks(dtype, steps):
    """b2 = 300 > one key tile: stage 1 streams its segments (c2 = 3, 100
    keys each) in several tiles."""
    cfg = WorkloadConfig("case", f"wide {dtype} T{steps}", batch=1, heads=2, seq_len=10 * 300,
                         head_dim=64, b1=10, b2=300, steps=steps, dtype=dtype, data="normed",
                         seed=23, c1=2, c2=3)
    check_case(cfg)


def test_launch_plan_fused_vs_staged():
    import structured_sub_quadratic_amd as ma
    p = ma.make_problem(1, 12, 16384, 64, 128, 128, flags=ma.MA_FLAG_FORCE_FUSED)
    assert ma.launch_names(p) == ["fused_t1"]
    p = ma.make_problem(1, 12, 16384, 64, 128, 128)
    assert ma.launch_names(p) == ["stage1_last", "stage2_last"]


# ------------------------------------------------ grouped-query attention

@pytest.mark.parametrize("case", [
    dict(dtype="f32", d=64, c=(1, 1), steps=1, kvh=1),
    dict(dtype="f32", d=128, c=(2, 1), steps=2, kvh=2),
    dict(dtype="bf16", d=64, c=(1, 1), steps=1, kvh=2),
    dict(dtype="bf16", d=128, c=(1, 1), steps=2, kvh=1),
    dict(dtype="bf16", d=64, c=(2, 2), steps=1, kvh=2),
    dict(dtype="bf16", d=128, c=(2, 2), steps=2, kvh=4),
])
def test_grouped_query_attention(case):
    """K, V with fewer heads than Q: query head h reads K/V head
    h // (heads / kv_heads), on the staged path and, for T = 1, the fused one."""
    cfg = WorkloadConfig("case", f"gqa {case}", batch=2, heads=4, seq_len=70 * 52,
                         head_dim=case["d"], b1=70, b2=52, steps=case["steps"], dtype=case["dtype"],
                         data="normed", seed=31, c1=case["c"][0], c2=case["c"][1])
    y, _, _ = check_case(cfg, kv_heads=case["kvh"])
    if case["steps"] == 1:
        y_f, _, _ = check_case(cfg, kv_heads=case["kvh"], force_fused=True)
        assert np.abs(y_f - y).max() <= 1e-6 * np.abs(y).max()


def test_grouped_query_attention_n16k_sampled():
    """The n16k shape with 12 query heads over 4 K/V heads, in the default
    launch configuration: three slices, every column."""
    cfg = WORKLOADS["n16k"]
    check_case(cfg, slices=[(0, 0), (0, 5), (0, 11)], exports=("L", "R", "lse", "objective"),
               kv_heads=4)


# ------------------------------------------------ padded flat sequences

@pytest.mark.parametrize("pad", ["pre", "post"])
@pytest.mark.parametrize("dtype,steps", [("f32", 1), ("f32", 2), ("bf16", 1), ("bf16", 2)])
def test_padded_vit_shape(pad, dtype, steps):
    """197 tokens (a ViT class token plus 14 x 14 patches) as 15 blocks of
    14: 13 padding positions, before or after the tokens."""
    cfg = WorkloadConfig("case", f"vit pad={pad} {dtype} T{steps}", batch=2, heads=3, seq_len=197,
                         head_dim=64, b1=15, b2=14, steps=steps, dtype=dtype, data="iid", seed=37,
                         pad=pad)
    check_case(cfg)


@pytest.mark.parametrize("pad", ["pre", "post"])
@pytest.mark.parametrize("case", [
    dict(dtype="bf16", d=128, c=(1, 1), steps=1),
    dict(dtype="bf16", d=64, c=(2, 2), steps=1),
    dict(dtype="bf16", d=64, c=(2, 2), steps=3),
    dict(dtype="f32", d=64, c=(5, 2), steps=2),
    dict(dtype="bf16", d=128, c=(1, 1), steps=2),
])
def test_padded_tiles(pad, case):
    """b1 x b2 = 70 x 52 with 20 padding positions (fewer than a segment of
    26 keys), tiled and untiled, one and several steps."""
    cfg = WorkloadConfig("case", f"pad={pad} {case}", batch=1, heads=2, seq_len=70 * 52 - 20,
                         head_dim=case["d"], b1=70, b2=52, steps=case["steps"], dtype=case["dtype"],
                         data="normed", seed=43, c1=case["c"][0], c2=case["c"][1], pad=pad)
    y, _, _ = check_case(cfg)
    if case["steps"] == 1:
        y_f, _, _ = check_case(cfg, force_fused=True)
        assert np.abs(y_f - y).max() <= 1e-6 * np.abs(y).max()
    if case["dtype"] == "bf16" and case["steps"] == 1:
        check_case(cfg, precise_aggregate=True)


@pytest.mark.parametrize("pad", ["pre", "post"])
@pytest.mark.parametrize("b1,b2,npad", [(100, 100, 60), (72, 128, 127), (128, 65, 1)])
def test_padded_blocks_over_64_keys(pad, b1, b2, npad):
    """T = 1 at head_dim 64 with blocks of 65-128 keys and padding (the
    whole-block stage 1 and the one-chunk stage 2 with padding): every slice,
    every column, every export, including a block whose real keys all but
    one are padding and a grid with a single padding position."""
    cfg = WorkloadConfig("case", f"pad={pad} {b1}x{b2}-{npad}", batch=2, heads=2,
                         seq_len=b1 * b2 - npad, head_dim=64, b1=b1, b2=b2, steps=1, dtype="bf16",
                         data="normed", seed=53, pad=pad)
    check_case(cfg)


@pytest.mark.parametrize("pad", ["pre", "post"])
def test_padded_long_sequence_sampled(pad):
    """16384 - 100 tokens on the 128 x 128 grid, 12 query heads over 4 K/V
    heads, in the default launch configuration: two slices, every column."""
    cfg = WorkloadConfig("case", f"n16k-100 pad={pad}", batch=1, heads=12, seq_len=16384 - 100,
                         head_dim=64, b1=128, b2=128, steps=1, dtype="bf16", data="normed",
                         seed=47, pad=pad)
    check_case(cfg, slices=[(0, 0), (0, 7)], exports=("L", "R", "lse", "objective"), kv_heads=4)


# ------------------------------------------------ benchmark workloads at full size

N4K_T3_SLICES = [(0, 0), (0, 11), (1, 5), (2, 3), (3, 7), (3, 10), (4, 1), (5, 6), (5, 9),
                 (6, 2), (7, 4), (7, 11)]


def test_n4k_t3_sampled():
    """The T = 3 workload: 12 of its 96 slices (spread over batch and head),
    every column, every export."""
    check_case(WORKLOADS["n4k_t3"], slices=N4K_T3_SLICES)


def test_n16k_full():
    """The headline workload in the launch configuration the benchmark times:
    every slice, every column, every export."""
    check_case(WORKLOADS["n16k"])


def test_n16k_fused_full():
    """The headline workload as one cooperative launch (the 8-wave, 128-key
    copied-tile fused build): every slice, every column, every export, and the
    same output as the staged launches."""
    cfg = WORKLOADS["n16k"]
    y_f, _, _ = check_case(cfg, force_fused=True)
    y_s, _, _ = check_case(cfg, exports=(), force_staged=True)
    assert np.abs(y_f - y_s).max() <= 1e-6 * np.abs(y_s).max()


@pytest.mark.parametrize("key", ["n16k", "video", "video_tiled"])
def test_precise_aggregate_t1_workloads(key):
    """The split aggregate path (MA_FLAG_PRECISE_AGGREGATE) on the T = 1
    workloads, whose default is the plain bf16 path: two slices, every
    column."""
    cfg = WORKLOADS[key]
    check_case(cfg, slices=[(0, 0), (0, 5)], exports=("L", "R", "lse"), precise_aggregate=True)


def test_video_sampled():
    """The video latent: two slices, all 52 columns, every export."""
    check_case(WORKLOADS["video"], slices=[(0, 0), (0, 7)])


def test_video_tiled_sampled_and_c1_equality():
    cfg = WORKLOADS["video_tiled"]
    check_case(cfg, slices=[(0, 0), (0, 7)])
    # c1 = c2 = 1 on the same data: equal to the untiled oracle and to the
    # tiled oracle with c = 1
    c4 = WORKLOADS["video"]
    Q, K, V = make_inputs(c4)
    y, _ = run_hip(c4, Q, K, V, exports=())
    cols = [3, 30]
    for tiled in (False, True):
        ref = oracle.forward(Q[:, 2:3], K[:, 2:3], V[:, 2:3], 630, 52, 1, 1, 1, layout="fh_w",
                             fhw=(21, 30, 52), cols=cols, tiled=tiled)
        tok = ref["grid"][:, cols].reshape(-1)
        err = rel_err(y[:, 2:3, tok], ref["y"][:, :, tok], [(0, 0)])
        assert err < TOL["bf16"], (tiled, err)


# ------------------------------------------------ error against exact attention

@pytest.mark.parametrize("key", ["n256", "n4k_t3", "n16k", "video", "video_tiled"])
def test_error_vs_exact_attention_reported(key):
    """The error of Y against exact softmax attention softmax(QK^T/sqrt(d))V,
    ||Y - Y_exact||_F / ||Y_exact||_F, in the launch configuration the
    benchmark times: every row of the language shapes, 4096 seeded query rows
    per head of the video latents.  The method approximates attention and
    the pages give no bound, so the value is reported (printed), and only
    checked to be finite and well below the scale of Y."""
    cfg = WORKLOADS[key]
    Q, K, V = make_inputs(cfg)
    y, _ = run_hip(cfg, Q, K, V, exports=())
    rows = np.arange(cfg.seq_len) if cfg.seq_len <= 16384 else \
        np.sort(np.random.default_rng(4242).choice(cfg.seq_len, 4096, replace=False))
    num = den = 0.0
    for b in range(cfg.batch):
        for h in range(cfg.heads):
            k, v = (X[b, h].astype(np.float64) for X in (K, V))
            for c0 in range(0, rows.size, 2048):
                r = rows[c0:c0 + 2048]
                ex = oracle.exact_attention(Q[b, h, r].astype(np.float64), k, v,
                                            1 / math.sqrt(cfg.head_dim))
                num += float(np.sum((y[b, h, r] - ex) ** 2))
                den += float(np.sum(ex ** 2))
    err = math.sqrt(num / den)
    print(f"{cfg.name}: ||Y - Y_exact|| / ||Y_exact|| = {err:.4f} over "
          f"{'all' if rows.size == cfg.seq_len else rows.size} rows per head")
    assert np.isfinite(err) and err < 1.0


# ------------------------------------------------ block-causal use

@pytest.mark.parametrize("case", [
    dict(dtype="f32", d=64, b1=16, b2=16, g=1, c=(1, 1), steps=1),
    dict(dtype="f32", d=128, b1=40, b2=48, g=3, c=(2, 1), steps=2),
    dict(dtype="bf16", d=64, b1=70, b2=52, g=1, c=(1, 1), steps=1),
    dict(dtype="bf16", d=64, b1=130, b2=40, g=1, c=(1, 1), steps=1),      # stage-2 columns of 3 chunks
    dict(dtype="bf16", d=128, b1=70, b2=52, g=5, c=(1, 1), steps=2),
    dict(dtype="bf16", d=64, b1=70, b2=52, g=2, c=(2, 2), steps=1),
    dict(dtype="bf16", d=64, b1=70, b2=52, g=1, c=(5, 2), steps=3),
    dict(dtype="bf16", d=128, b1=24, b2=100, g=4, c=(1, 1), steps=1),
    dict(dtype="bf16", d=64, b1=96, b2=40, g=7, c=(1, 1), steps=3),
    # columns of 65-128 keys at head_dim 64 with blocks of more than 64 keys:
    # one 128-key chunk an item (staged: the one-chunk kernel, fused: the
    # general stage 2 with 128-key chunks), per-row bounds and whole chunks
    dict(dtype="bf16", d=64, b1=100, b2=100, g=1, c=(1, 1), steps=1),
    dict(dtype="bf16", d=64, b1=120, b2=72, g=20, c=(1, 1), steps=1),
    dict(dtype="bf16", d=64, b1=100, b2=100, g=3, c=(1, 1), steps=2),
])
def test_block_causal(case):
    """Block-causal use: query block l attends to key block k iff
    floor(k/g) <= floor(l/g); every output against the oracle, staged and,
    for T = 1, fused."""
    cfg = WorkloadConfig("case", f"causal {case}", batch=2, heads=2, seq_len=case["b1"] * case["b2"],
                         head_dim=case["d"], b1=case["b1"], b2=case["b2"], steps=case["steps"],
                         dtype=case["dtype"], data="normed", seed=71, c1=case["c"][0], c2=case["c"][1])
    y, _, _ = check_case(cfg, causal=case["g"])
    if case["steps"] == 1:
        y_f, _, _ = check_case(cfg, causal=case["g"], force_fused=True)
        assert np.abs(y_f - y).max() <= 1e-6 * np.abs(y).max()


@pytest.mark.parametrize("pad", ["pre", "post"])
def test_block_causal_padded(pad):
    cfg = WorkloadConfig("case", f"causal pad={pad}", batch=1, heads=3, seq_len=197, head_dim=64,
                         b1=15, b2=14, steps=2, dtype="bf16", data="iid", seed=73, pad=pad)
    check_case(cfg, causal=1)


def test_block_causal_one_token_blocks_is_causal_attention():
    """b2 = 1 with g = 1 is token-causal softmax attention, on the GPU as in
    the oracle (compared with the masked exact product here)."""
    cfg = WorkloadConfig("case", "causal b2=1", batch=1, heads=2, seq_len=300, head_dim=64, b1=300,
                         b2=1, steps=2, dtype="f32", data="iid", seed=74)
    Q, K, V = make_inputs(cfg)
    y, _ = run_hip(cfg, Q, K, V, exports=(), causal=1)
    for h in range(2):
        q, k, v = (X[0, h].astype(np.float64) for X in (Q, K, V))
        s_ = q @ k.T / 8.0
        s_ = np.where(np.tril(np.ones((300, 300), bool)), s_, -np.inf)
        p_ = np.exp(s_ - s_.max(axis=1, keepdims=True))
        ex = (p_ @ v) / p_.sum(axis=1, keepdims=True)
        assert np.abs(y[0, h] - ex).max() / np.abs(ex).max() < 1e-4


def test_block_causal_n16k_full():
    """The headline shape with the block-causal mask over its 128 blocks:
    every slice, every column, every export."""
    check_case(WORKLOADS["n16k"], causal=1)


def test_block_causal_video_frame_causal_sampled():
    """The video latent, frame-causal (g = h = 30 grid blocks per frame):
    two slices, all 52 columns."""
    check_case(WORKLOADS["video"], slices=[(0, 0), (0, 7)], causal=30)


def test_block_causal_video_codes_exact_without_noise():
    """Zero-noise per-axis codes: one step reproduces frame-causal softmax
    attention exactly on the (fh, w) layout with g = h."""
    cfg = WorkloadConfig("case", "video frame-causal exact", batch=1, heads=1, seq_len=3 * 4 * 10,
                         head_dim=64, b1=12, b2=10, steps=1, dtype="f32", data="video", seed=15,
                         layout="fh_w", fhw=(3, 4, 10))
    Q, K, V = make_inputs(cfg, noise_scale=0.0)
    y, _ = run_hip(cfg, Q, K, V, exports=(), causal=4)
    q, k, v = (X[0, 0].astype(np.float64) for X in (Q, K, V))
    frame = np.arange(120) // 40
    s_ = np.where(frame[None, :] <= frame[:, None], q @ k.T / 8.0, -np.inf)
    p_ = np.exp(s_ - s_.max(axis=1, keepdims=True))
    ex = (p_ @ v) / p_.sum(axis=1, keepdims=True)
    assert np.abs(y[0, 0] - ex).max() / np.abs(ex).max() < 1e-4
