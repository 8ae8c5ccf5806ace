"""Shared helpers for the parity tests: run the HIP path and the oracle on the
same seeded inputs and compare them with the relative error

    err(X) = max over slices of  max|X - X_ref| / max|X_ref|   (per slice)

which is the tolerance measure for Y, L and R (1e-4 for fp32 inputs, 2e-2 for
bf16 inputs).  An elementwise ratio would be meaningless for probabilities
near zero, hence the per-slice maximum as the denominator."""

import numpy as np

TOL = {"f32": 1e-4, "bf16": 2e-2}


def rel_err(x, ref, slices):
    """x, ref: arrays indexed [b, h, ...]; slices: list of (b, h)."""
    worst = 0.0
    for (b, h) in slices:
        a, r = np.asarray(x[b, h], np.float64), np.asarray(ref[b, h], np.float64)
        m = np.nanmax(np.abs(r))
        d = float(np.nanmax(np.abs(a - r)))
        # an all-zero reference (e.g. dQ of a single token) is compared absolutely
        worst = max(worst, d / m if m > 0 else d)
    return worst


def oracle_L_as_gpu(L, tiled):
    """oracle L [B,H,nc,b1,b1(,c2)] -> GPU export layout [B,H,nc,b1,b1*c2]."""
    if not tiled:
        return L
    B, H, nc, b1, _, c2 = L.shape
    return L.reshape(B, H, nc, b1, b1 * c2)


def oracle_R_as_gpu(R, tiled):
    """oracle R [B,H,b1,nc,(c1,)b2] -> GPU export layout [B,H,b1,nc,c1,b2]."""
    return R if tiled else R[:, :, :, :, None, :]


def run_hip(cfg_like, Q, K, V, exports=("L", "R", "lse", "objective"), **kw):
    """Run the HIP path on numpy inputs; returns numpy outputs (float32/64)."""
    import torch
    import structured_sub_quadratic_amd as ma
    dt = torch.float32 if cfg_like.dtype == "f32" else torch.bfloat16
    dev = torch.device("cuda:0")
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x)).to(dev).to(dt) for x in (Q, K, V))
    res = ma.forward(tq, tk, tv, cfg_like.b1, cfg_like.b2, cfg_like.steps, cfg_like.c1,
                     cfg_like.c2, layout=cfg_like.layout, fhw=cfg_like.fhw, exports=exports,
                     pad=getattr(cfg_like, "pad", "post"), **kw)
    torch.cuda.synchronize()
    if exports:
        y, ex = res
        return y.float().cpu().numpy(), {k: v.cpu().numpy() for k, v in ex.items()}
    return res.float().cpu().numpy(), {}
