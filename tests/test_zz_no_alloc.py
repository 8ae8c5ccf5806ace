"""The allocation-free entry point monarch_attn_forward_noalloc (through the
C ABI): the same outputs as monarch_attn_forward on the same inputs, for two
calls in a row, the second on a smaller problem (its scratch array keeps what
the first call left), and the host-side refusal of a problem whose workspace
exceeds the array."""

import numpy as np
import pytest

from workloads import WORKLOADS, WorkloadConfig, make_inputs
from parity_utils import TOL

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import structured_sub_quadratic_amd as ma
    ma._lib.load()


def _tensors(cfg):
    import torch
    dt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
    Q, K, V = make_inputs(cfg)
    return tuple(torch.from_numpy(x).to("cuda:0").to(dt) for x in (Q, K, V))


def _exports(cfg, dev):
    import torch
    B, H, b1, b2, c1, c2 = cfg.batch, cfg.heads, cfg.b1, cfg.b2, cfg.c1, cfg.c2
    return {"L": torch.empty((B, H, b2, b1, b1 * c2), dtype=torch.float32, device=dev),
            "R": torch.empty((B, H, b1, b2, c1, b2), dtype=torch.float32, device=dev),
            "lse": torch.empty((B, H, cfg.seq_len), dtype=torch.float32, device=dev),
            "objective": torch.empty((B * H,), dtype=torch.float64, device=dev)}


def _rel(a, b):
    a, b = a.double().cpu().numpy(), b.double().cpu().numpy()
    return float(np.abs(a - b).max() / max(np.abs(b).max(), 1e-300))


def test_noalloc_matches_forward_on_two_calls():
    import torch
    import structured_sub_quadratic_amd as ma
    # first call: the 16384-token, 12-head workload (53 MB of workspace)
    big = WORKLOADS["n16k"]
    q, k, v = _tensors(big)
    y_ref = ma.forward(q, k, v, big.b1, big.b2, big.steps)
    y = torch.empty_like(q)
    ma.forward_noalloc(q, k, v, big.b1, big.b2, y, big.steps)
    torch.cuda.synchronize()
    err = _rel(y, y_ref)
    print("n16k noalloc vs forward:", err)
    assert err <= TOL[big.dtype]
    assert torch.equal(y, y_ref)          # the same kernels on the same inputs
    # second call, smaller: tiled, two steps, every export
    small = WorkloadConfig("case", "noalloc small", batch=1, heads=3, seq_len=70 * 52, head_dim=128,
                           b1=70, b2=52, steps=2, dtype="bf16", data="normed", seed=81, c1=2, c2=2)
    q, k, v = _tensors(small)
    y_ref, ex_ref = ma.forward(q, k, v, small.b1, small.b2, small.steps, small.c1, small.c2,
                               exports=("L", "R", "lse", "objective"))
    y = torch.empty_like(q)
    ex = _exports(small, q.device)
    ma.forward_noalloc(q, k, v, small.b1, small.b2, y, small.steps, small.c1, small.c2, exports=ex)
    torch.cuda.synchronize()
    errs = {"Y": _rel(y, y_ref), **{n: _rel(ex[n], ex_ref[n]) for n in ex}}
    print("small noalloc vs forward:", errs)
    assert all(e <= TOL[small.dtype] for e in errs.values()), errs
    assert torch.equal(y, y_ref)


def test_noalloc_refuses_oversized_and_fused_problems():
    import torch
    import structured_sub_quadratic_amd as ma
    from structured_sub_quadratic_amd import _lib
    cfg = WORKLOADS["video"]             # about 0.2 GB of workspace
    prob = ma.make_problem(cfg.batch, cfg.heads, cfg.seq_len, cfg.head_dim, cfg.b1, cfg.b2,
                           cfg.steps, dtype="bf16", layout=cfg.layout, fhw=cfg.fhw)
    assert ma.workspace_size(prob) > _lib.MONARCH_ATTN_SCRATCH_BYTES
    dev = torch.device("cuda:0")
    q = torch.zeros((1, 12, cfg.seq_len, 128), dtype=torch.bfloat16, device=dev)
    k, v, y = torch.zeros_like(q), torch.zeros_like(q), torch.empty_like(q)
    with pytest.raises(ma.MonarchAttnError, match="WORKSPACE_TOO_SMALL"):
        ma.forward_noalloc(q, k, v, cfg.b1, cfg.b2, y, layout=cfg.layout, fhw=cfg.fhw)
    small = torch.zeros((1, 1, 256, 64), dtype=torch.bfloat16, device=dev)
    prob = ma.make_problem(1, 1, 256, 64, 16, 16, dtype="bf16", flags=ma.MA_FLAG_FORCE_FUSED)
    cex = _lib.MAExports(None, None, None, None)
    import ctypes
    st = _lib.load().monarch_attn_forward_noalloc(ctypes.byref(prob), small.data_ptr(),
                                                  small.data_ptr(), small.data_ptr(),
                                                  torch.empty_like(small).data_ptr(),
                                                  ctypes.byref(cex), None)
    assert st == 2                        # MA_ERR_UNSUPPORTED
