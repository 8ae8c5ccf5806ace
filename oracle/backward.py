"""Gradients of the MonarchAttention forward pass, in float64 PyTorch (CPU).

Test infrastructure only (see the package docstring).

The pages train through the method (MonarchRT "Method" part (3): one-step
fine-tuning; MonarchAttention review discussion of fine-tuning), but give no
backward formulas.  The gradient of Y with respect to Q, K and V is whatever
reverse-mode differentiation of the forward steps gives, through all T
unrolled steps.  So this module transcribes the forward of oracle.monarch
step for step into torch (float64, CPU), and lets torch.autograd produce
dQ, dK, dV for an upstream dY.  Nothing here is tuned or fused.

Pins (tests/test_oracle_pins.py): the transcription equals oracle.forward
(an independent NumPy implementation) to rounding; its gradients equal
central finite differences of oracle.forward; with one block (b1 = 1) they
equal the gradients of exact softmax attention (torch's scaled dot-product
attention, differentiated by torch).
"""

import numpy as np
import torch

from .layouts import grid_index
from .monarch import causal_allowed


def _softmax_masked(z, mask):
    """softmax over the last axis with mask False entries excluded."""
    z = z.masked_fill(~mask, float("-inf"))
    return torch.softmax(z, dim=-1)


def _entropy(p):
    """-sum p log p over the last axis, 0 log 0 = 0 (and a zero gradient there)."""
    safe = torch.where(p > 0, p, torch.ones_like(p))
    return -(torch.where(p > 0, p * torch.log(safe), torch.zeros_like(p))).sum(-1)


def _real_mean(q, rows):
    """Mean of q[l, i] over the real rows l of each column i (zero if none)."""
    n = rows.sum(0).clamp(min=1).to(q.dtype)
    return (q * rows[..., None]).sum(0) / n[:, None]


def forward_slice(qg, kg, vg, steps, scale, c1=1, c2=1, real=None, causal=0):
    """One slice in grid order: qg, kg, vg [b1, b2, d] float64 tensors
    (requires_grad allowed).  Same steps as oracle.monarch.forward_tiled
    (which with c1 = c2 = 1 is the untiled method); causal > 0 masks the
    L-update as there (query block l takes key block k only when
    floor(k / causal) <= floor(l / causal)).  Returns y [b1, b2, dv]."""
    b1, b2, d = qg.shape
    allow = torch.as_tensor(causal_allowed(b1, causal))               # [l, k]
    sw = b2 // c2
    real = torch.ones((b1, b2), dtype=torch.bool) if real is None else torch.as_tensor(real)
    rq = real                                       # real query rows (l, i)
    q = scale * qg * rq[..., None]
    tile = torch.as_tensor((np.arange(b1) * c1) // b1)
    Kseg = kg.reshape(b1, c2, sw, d)
    Vseg = vg.reshape(b1, c2, sw, vg.shape[-1])
    kreal = real.reshape(b1, c2, sw)
    qbar = torch.stack([_real_mean(q[tile == t], rq[tile == t]) for t in range(c1)])   # [c1, b2, d]

    # first R-update's queries: own row tile and real -> q[k, i], else the tile mean
    own = (tile[:, None] == torch.arange(c1)[None, :])                    # [k, t]
    use_q = own[:, None, :] & rq[:, :, None]                             # [k, i, t]
    qt = torch.where(use_q[..., None], q[:, :, None, :], qbar.permute(1, 0, 2)[None])   # [k, i, t, d]
    qt = qt[:, :, :, None, :].expand(b1, b2, c1, c2, d)

    for step in range(steps):
        z = torch.einsum("kitsd,ksjd->kitsj", qt, Kseg)
        R = _softmax_masked(z, kreal[:, None, None].expand_as(z))
        HR = _entropy(R)                                                  # [k, i, t, s]
        C = torch.einsum("kitsj,ksjd->kitsd", R, Kseg)
        # L-update per row tile
        Ls = []
        for t in range(c1):
            rows = torch.nonzero(tile == t).flatten()
            w = torch.einsum("lid,kisd->ilks", q[rows], C[:, :, t]) + HR[:, :, t].permute(1, 0, 2)[:, None]
            w = w.masked_fill(~allow[rows][None, :, :, None], float("-inf"))
            Lt = torch.softmax(w.reshape(b2, rows.numel(), b1 * c2), dim=-1).reshape(w.shape)
            Ls.append(Lt * rq[rows].T[:, :, None, None])
        L = torch.cat(Ls, dim=1)                                         # [i, l, k, s]
        if step < steps - 1:
            nq = []
            for t in range(c1):
                rows = torch.nonzero(tile == t).flatten()
                Lt = L[:, rows]
                alpha = torch.einsum("ilks,lid->kisd", Lt, q[rows])
                beta = Lt.sum(1).permute(1, 0, 2)                        # [k, i, s]
                safe = torch.where(beta > 0, beta, torch.ones_like(beta))
                nq.append(torch.where((beta > 0)[..., None], alpha / safe[..., None],
                                      qbar[t][None, :, None, :]))
            qt = torch.stack(nq, dim=2)                                   # [k, i, t, s, d]
    U = torch.einsum("kitsj,ksjd->kitsd", R, Vseg)
    ys = []
    for t in range(c1):
        rows = torch.nonzero(tile == t).flatten()
        ys.append((rows, torch.einsum("ilks,kisd->lid", L[:, rows], U[:, :, t])))
    y = torch.empty((b1, b2, vg.shape[-1]), dtype=qg.dtype)
    for rows, yt in ys:
        y = y.index_put((rows,), yt)
    return y


def backward(Q, K, V, dY, b1, b2, steps, c1=1, c2=1, scale=None, layout="flat", fhw=None,
             pad="post", slices=None, causal=0):
    """dQ, dK, dV (float64 NumPy) of <dY, Y(Q, K, V)> for [B, H, N, d] inputs
    (K, V may have fewer heads: grouped-query attention, their gradients sum
    over the query heads of a group).  slices: optional list of (b, h) query
    slices to differentiate (dQ of the others is NaN; dK, dV then hold only
    the contributions of the listed slices)."""
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    dY = np.asarray(dY, np.float64)
    B, H, N, d = Q.shape
    Hkv = K.shape[1]
    group = H // Hkv
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    grid = grid_index(N, b1, b2, layout, fhw, pad)
    real = torch.as_tensor(grid >= 0)
    g = torch.as_tensor(np.maximum(grid, 0))
    sel = [(b, h) for b in range(B) for h in range(H)] if slices is None else list(slices)
    dQ = np.full(Q.shape, np.nan)
    dK = np.zeros(K.shape)
    dV = np.zeros(V.shape)
    for (b, h) in sel:
        q = torch.tensor(Q[b, h], requires_grad=True)
        k = torch.tensor(K[b, h // group], requires_grad=True)
        v = torch.tensor(V[b, h // group], requires_grad=True)
        zero = torch.zeros((), dtype=torch.float64)
        grid_of = lambda x: torch.where(real[..., None], x[g], zero)     # token order -> grid
        y = forward_slice(grid_of(q), grid_of(k), grid_of(v), steps, scale, c1, c2, real, causal)
        dyg = torch.where(real[..., None], torch.as_tensor(dY[b, h])[g], zero)
        (y * dyg).sum().backward()
        dQ[b, h] = q.grad.numpy()
        dK[b, h // group] += k.grad.numpy()
        dV[b, h // group] += v.grad.numpy()
    return dQ, dK, dV
