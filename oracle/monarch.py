"""MonarchAttention forward pass, step by step, in float64 NumPy.

Test infrastructure only (see the package docstring).

What the pages fix
------------------
* Attention is replaced by a Monarch matrix M = P L P^T R with L and R block
  diagonal, so that after a fixed permutation M is a grid of rank-one blocks
  ([MRT] "Method" part (1); [MA] scime summary "Approach": block rank-one
  factors).
* L and R are fitted by alternating maximisation of the softmax variational
  objective (linear score term plus entropy, entropy maximised) for T steps,
  never forming the N x N matrix ([MA] scime summary "Proposal"/"Approach";
  OpenReview first review and the author response on concavity).
* L and R are constrained to be positive ([MA] OpenReview first review,
  question on "Alternating Maximization with Constraints", and the response).
* With L fixed the objective is concave in R (author response), so each
  half-step is an exact block-wise maximisation.
* T is small: the objective is stationary after about two steps (author
  response table of f(M) against T).
* Cost Theta(N sqrt(N) d) compute, Theta(N d) IO ([MA] abstract).
* Tiled Monarch: each Monarch block is cut into c1 x c2 sub-tiles that are
  rank one each ([MRT] "Key claims", Theorem 4.1 / section 4.2, and "Method"
  part (2)).

Notation (ours)
---------------
Grid position of a query: (l, i), l in [b1], i in [b2]; of a key: (k, j).
Queries already carry the score scale sigma (sigma = 1/sqrt(d) by default).

    M[(l,i),(k,j)] = L[i,l,k] * R[k,i,j]                       (untiled)
    M[(l,i),(k,j)] = L[i,l,k,s(j)] * R[k,i,t(l),j]             (tiled)

with t(l) = floor(l*c1/b1) the row tile and s(j) = floor(j*c2/b2) the column
segment.  Rows of R sum to one (per segment when tiled) and rows of L sum to
one (over (k, s) when tiled); this fixes the scale freedom of a rank-one block
and loses nothing, since M itself has simplex rows.

The update equations are not printed on the pages.  They follow exactly from
the objective by maximising it over one factor with the other fixed:

  row entropy splits:  H(M_(l,i)) = H(L[i,l,:]) + sum_k L[i,l,k] H(R[k,i,:])

  R-update (L fixed): for every (k, i), the terms holding R[k,i,:] are
      beta * ( <R[k,i,:], qt[k,i] . K_k> + H(R[k,i,:]) )
  with alpha[k,i] = sum_l L[i,l,k] q[l,i], beta[k,i] = sum_l L[i,l,k] and
  qt = alpha / beta, so R[k,i,:] = softmax_j(qt[k,i] . k[k,j]).

  L-update (R fixed): for every (i, l),
      L[i,l,:] = softmax_k( q[l,i] . c[k,i] + H_R[k,i] ),
  c[k,i] = sum_j R[k,i,j] k[k,j] and H_R[k,i] = H(R[k,i,:]).  The entropy
  enters with a plus sign (a reviewer noted that the paper's printed
  expansion had two sign errors that turned entropy into negative entropy).

  Output: y[l,i] = sum_k L[i,l,k] u[k,i], u[k,i] = sum_j R[k,i,j] v[k,j].

Readings where the pages are silent:
  * initialisation L0 = block identity, so qt[k,i] = q[k,i] for the first
    R-update; a step is one R-update then one L-update; the first point of
    the objective trace is f(L0, R1);
  * tiled initialisation: the tiled block identity gives a zero weight
    (beta = 0) to every sub-row with t != t(k); there qt is the mean of
    q[l,i] over the rows l of tile t (the eps -> 0 limit of
    (1-eps) I + eps * uniform).  The same fallback is used whenever beta is
    exactly zero.
  * padding ([MA] author response on block sizes: m = ceil(N/b), pre- or
    post-padding): the objective is the one of the real N x N attention, so
    it sums over real query rows only and M puts no mass on padding keys.
    Hence R rows are softmaxes over the real keys of a segment, padding
    rows carry no L row (exported as zeros), and alpha, beta and the tile
    means run over real rows.  L0 is the block identity on real rows, so a
    padding position (k, i) has beta = 0 at the first R-update and takes the
    fallback: the mean of q over the real rows of its tile and column (zero
    if there are none; its R row then weighs nothing).  Every segment must
    hold a real key.
  * block-causal use ([MA] scime summary "Limitations": causal masking does
    not fit the method; MonarchRT, summary page: few-step autoregressive
    video DiTs, which attend causally across chunks of frames and
    bidirectionally inside a chunk).  Token-level causality cuts through the
    rank-one blocks, but a mask over whole blocks does not: with causal = g,
    query block l may attend to key block k iff floor(k/g) <= floor(l/g)
    (units of g consecutive blocks; g = 1 on a flat sequence is the usual
    block-causal mask with blocks of b2 tokens, g = h on the (fh, w) video
    layout is frame-causal).  M is zero on masked entries, i.e. L[i,l,k] = 0
    there, and the objective runs over the allowed entries only.  Then the
    R-update keeps its form (L is simply zero on masked (l, k), and the
    diagonal k = l is always allowed, so L0 = block identity is admissible),
    and the L-update is the softmax over the allowed k only.

Parity pins (tests/test_oracle_pins.py): dense product P^T L P R on tiny
grids, simplex rows, non-decreasing objective bounded by sum logsumexp, dense
limits b1 = 1 and b2 = 1, exactness on separable scores (all six aligned video
layouts, and failure on a misaligned one), half-steps equal to a generic
numerical maximiser of the dense objective, tiled c1 = c2 = 1 equal to
untiled, tiled c2 = b2 equal to exact attention, and invariance under
relabelling of keys and blocks.
"""

import numpy as np

from .layouts import grid_index, to_grid, from_grid
from .reference_attention import logsumexp, softmax, row_entropy


def tile_of_rows(b1, c1):
    """t(l) = floor(l * c1 / b1) for l in [b1]."""
    return (np.arange(b1) * c1) // b1


def segment_of_cols(b2, c2):
    """s(j) = floor(j * c2 / b2) for j in [b2]."""
    return (np.arange(b2) * c2) // b2


# ---------------------------------------------------------------------------
# untiled Monarch
# ---------------------------------------------------------------------------

def _objective_untiled(q, C, HR, L):
    """f(L, R) from the factored form: sum over rows (l, i) of
    sum_k L[i,l,k] (q[l,i].c[k,i] + H_R[k,i]) + H(L[i,l,:])."""
    w = np.matmul(q.transpose(1, 0, 2), C.transpose(1, 2, 0)) + HR.T[:, None, :]
    return float(np.sum(L * w) + np.sum(row_entropy(L, axis=-1)))


def _real_mean(q, rows):
    """Mean of q[l, i] over the real rows l (rows[l, i] True) of each column
    i; zero for a column without real rows.  q [nr, nc, d], rows [nr, nc]."""
    n = rows.sum(axis=0)
    tot = np.sum(np.where(rows[..., None], q, 0.0), axis=0)
    return tot / np.maximum(n, 1)[:, None]


def _check_real(real, b1, b2, c2=1):
    real = np.ones((b1, b2), bool) if real is None else np.asarray(real, bool)
    if real.shape != (b1, b2):
        raise ValueError("real must be [b1, b2]")
    if not real.reshape(b1, c2, b2 // c2).any(axis=-1).all():
        raise ValueError("every key segment needs a real key")
    return real


def causal_allowed(b1, causal):
    """allowed[l, k]: query block l may attend to key block k, i.e.
    floor(k / causal) <= floor(l / causal); everything when causal == 0."""
    if not causal:
        return np.ones((b1, b1), bool)
    unit = np.arange(b1) // causal
    return unit[None, :] <= unit[:, None]


def forward_untiled(qg, kg, vg, steps, scale, cols=None, history=False, real=None, causal=0):
    """One (batch, head) slice of untiled MonarchAttention.

    qg, kg, vg: [b1, b2, d] in grid order (float64).  cols: optional list of
    columns i to compute (the method is independent across i: R rows [., i, .]
    and L[i] touch only column i of the queries, and all keys).  real:
    optional [b1, b2] bool, False at padding positions (their rows of qg, kg,
    vg are ignored).  causal: 0 (bidirectional) or the number g of blocks per
    causal unit (see causal_allowed).

    Returns dict:
      y       [b1, nc, d]   output rows (l, i) for the selected columns
      L       [nc, b1, b1]  L[i, l, k]
      R       [b1, nc, b2]  R[k, i, j]
      lse     [b1, nc]      logsumexp_k of the last L-update's scores
      f_trace [2*steps]     f(L0,R1), f(L1,R1), f(L1,R2), ..., f(LT,RT)
      history list of (L, R) after every half-step (if history=True)
    """
    b1, b2, d = qg.shape
    if steps < 1:
        raise ValueError("steps must be >= 1")
    cols = np.arange(b2) if cols is None else np.asarray(cols)
    real = _check_real(real, b1, b2)
    allow = causal_allowed(b1, causal)       # allow[l, k]
    rq = real[:, cols]                       # real query rows (l, i)
    q = scale * np.where(rq[..., None], qg[:, cols, :], 0.0)   # q[l, i], sigma folded in
    nc = q.shape[1]
    qmean = _real_mean(q, rq)                # [i, d], the zero-weight fallback

    # L0 = block identity on real rows: L0[i, l, k] = [l == k], hence
    # qt[k, i] = q[k, i]; a padding row (k, i) has beta = 0 -> fallback.
    L = np.broadcast_to(np.eye(b1), (nc, b1, b1)) * rq.T[:, :, None]
    qt = np.where(rq[..., None], q, qmean[None])
    f_trace, hist = [], []

    for step in range(steps):
        # R-update: R[k,i,:] = softmax over the real keys j of qt[k,i] . k[k,j]
        z = np.matmul(qt, kg.transpose(0, 2, 1))          # z[k, i, j]
        z = np.where(real[:, None, :], z, -np.inf)
        R = softmax(z, axis=-1)
        HR = row_entropy(R, axis=-1)                       # H_R[k, i]
        C = np.matmul(R, kg)                               # c[k, i]
        f_trace.append(_objective_untiled(q, C, HR, L))
        if history:
            hist.append((L.copy(), R.copy()))

        # L-update: L[i,l,:] = softmax over the allowed k of
        # q[l,i] . c[k,i] + H_R[k,i]
        w = np.matmul(q.transpose(1, 0, 2), C.transpose(1, 2, 0)) + HR.T[:, None, :]
        wm = np.where(allow[None], w, -np.inf)
        L = softmax(wm, axis=-1) * rq.T[:, :, None]        # L[i, l, k]; padding rows 0
        lse = logsumexp(wm, axis=-1)                       # [i, l]
        f_trace.append(_objective_untiled(q, C, HR, L))
        if history:
            hist.append((L.copy(), R.copy()))

        if step < steps - 1:
            # next R-update's query: qt = alpha / beta
            alpha = np.matmul(L.transpose(0, 2, 1), q.transpose(1, 0, 2))  # [i, k, d]
            beta = np.sum(L, axis=1)                                       # [i, k]
            safe = np.where(beta > 0, beta, 1.0)
            qt_i = np.where((beta > 0)[..., None], alpha / safe[..., None],
                            qmean[:, None, :])
            qt = qt_i.transpose(1, 0, 2)                   # [k, i, d]

    U = np.matmul(R, vg)                                   # u[k, i]
    y = np.matmul(L, U.transpose(1, 0, 2)).transpose(1, 0, 2)   # y[l, i]
    out = dict(y=y, L=L, R=R, lse=lse.T, f_trace=np.array(f_trace))
    if history:
        out["history"] = hist
    return out


# ---------------------------------------------------------------------------
# tiled Monarch
# ---------------------------------------------------------------------------

def _objective_tiled(q, C, HR, L, tile):
    """f(L, R) for the tiled class: sum over rows (l, i) of
    sum_{k,s} L[i,l,k,s] (q[l,i].c[k,i,t(l),s] + H_R[k,i,t(l),s]) + H(L row)."""
    total = 0.0
    for t in np.unique(tile):
        rows = np.nonzero(tile == t)[0]
        w = _tiled_scores(q[rows], C[:, :, t], HR[:, :, t])      # [i, rows, k, s]
        Lt = L[:, rows]
        nc, nr = Lt.shape[:2]
        total += np.sum(Lt * w) + np.sum(row_entropy(Lt.reshape(nc, nr, -1), axis=-1))
    return float(total)


def _tiled_scores(q_rows, C_t, HR_t):
    """w[i, l, k, s] = q[l,i] . c[k,i,t,s] + H_R[k,i,t,s] for rows l of one tile t.

    q_rows [nr, nc, d]; C_t [b1, nc, c2, d]; HR_t [b1, nc, c2]."""
    b1, nc, c2, d = C_t.shape
    Ci = C_t.transpose(1, 0, 2, 3).reshape(nc, b1 * c2, d)          # [i, (k,s), d]
    w = np.matmul(q_rows.transpose(1, 0, 2), Ci.transpose(0, 2, 1))  # [i, l, (k,s)]
    w = w + HR_t.transpose(1, 0, 2).reshape(nc, 1, b1 * c2)
    return w.reshape(nc, q_rows.shape[0], b1, c2)


def forward_tiled(qg, kg, vg, steps, scale, c1, c2, cols=None, history=False, real=None,
                  causal=0):
    """One slice of tiled MonarchAttention with c1 x c2 sub-tiles per block.

    Requires c1 | b1 and c2 | b2 (tiles and segments are then contiguous and
    of equal size).  real, causal: as for forward_untiled (the mask is over
    blocks l, k, so every segment s of an allowed block is allowed).  Returns
    dict:
      y       [b1, nc, d]
      L       [nc, b1, b1, c2]   L[i, l, k, s]
      R       [b1, nc, c1, b2]   R[k, i, t, j]  (each segment of j sums to 1)
      lse     [b1, nc]
      f_trace [2*steps]
    """
    b1, b2, d = qg.shape
    if steps < 1:
        raise ValueError("steps must be >= 1")
    if b1 % c1 or b2 % c2:
        raise ValueError("c1 must divide b1 and c2 must divide b2")
    cols = np.arange(b2) if cols is None else np.asarray(cols)
    real = _check_real(real, b1, b2, c2)
    allow = causal_allowed(b1, causal)             # allow[l, k]
    rq = real[:, cols]                             # real query rows (l, i)
    q = scale * np.where(rq[..., None], qg[:, cols, :], 0.0)   # q[l, i]
    nc = q.shape[1]
    sw = b2 // c2                                  # keys per segment
    tile = tile_of_rows(b1, c1)
    Kseg = kg.reshape(b1, c2, sw, d)               # K[k, s, j'], j = s*sw + j'
    kreal = real.reshape(b1, c2, sw)               # real keys
    dv = vg.shape[-1]
    Vseg = vg.reshape(b1, c2, sw, dv)

    # tile means of the queries over real rows, qbar[t, i]
    qbar = np.stack([_real_mean(q[tile == t], rq[tile == t]) for t in range(c1)])   # [c1, nc, d]

    # initial qt[k, i, t, s]: own tile -> q[k, i]; other tiles (and padding
    # rows) have beta = 0 -> qbar[t, i]
    qt = np.empty((b1, nc, c1, c2, d))
    for k in range(b1):
        for t in range(c1):
            own = np.where(rq[k][:, None], q[k], qbar[t]) if t == tile[k] else qbar[t]
            qt[k, :, t, :, :] = own[:, None, :]

    # L0: tiled block identity on real rows, mass 1/c2 on every segment of
    # the own block
    L = np.zeros((nc, b1, b1, c2))
    L[:, np.arange(b1), np.arange(b1), :] = rq.T[:, :, None] / c2

    f_trace, hist = [], []
    for step in range(steps):
        # R-update, per (k, i, t, s): R = softmax over j in segment s of
        # qt[k,i,t,s] . k[k,j]
        z = np.einsum("kitsd,ksjd->kitsj", qt, Kseg)       # [k, i, t, s, j']
        z = np.where(kreal[:, None, None], z, -np.inf)     # padding keys take no weight
        Rs = softmax(z, axis=-1)
        HR = row_entropy(Rs, axis=-1)                      # [k, i, t, s]
        C = np.einsum("kitsj,ksjd->kitsd", Rs, Kseg)       # [k, i, t, s, d]
        R = Rs.reshape(b1, nc, c1, b2)
        f_trace.append(_objective_tiled(q, C, HR, L, tile))
        if history:
            hist.append((L.copy(), R.copy()))

        # L-update, per (i, l): L[i,l,:,:] = softmax over (k, s) of
        # q[l,i] . c[k,i,t(l),s] + H_R[k,i,t(l),s]
        L = np.empty((nc, b1, b1, c2))
        lse = np.empty((nc, b1))
        for t in range(c1):
            rows = np.nonzero(tile == t)[0]
            w = _tiled_scores(q[rows], C[:, :, t], HR[:, :, t])   # [i, rows, k, s]
            w = np.where(allow[rows][None, :, :, None], w, -np.inf)
            wf = w.reshape(nc, rows.size, b1 * c2)
            L[:, rows] = (softmax(wf, axis=-1) * rq[rows].T[:, :, None]).reshape(nc, rows.size, b1, c2)
            lse[:, rows] = logsumexp(wf, axis=-1)
        f_trace.append(_objective_tiled(q, C, HR, L, tile))
        if history:
            hist.append((L.copy(), R.copy()))

        if step < steps - 1:
            # qt[k,i,t,s] = sum_{l in t} L[i,l,k,s] q[l,i] / sum_{l in t} L[i,l,k,s]
            qt = np.empty((b1, nc, c1, c2, d))
            for t in range(c1):
                rows = np.nonzero(tile == t)[0]
                Lt = L[:, rows]                                   # [i, rows, k, s]
                alpha = np.einsum("ilks,lid->kisd", Lt, q[rows])  # [k, i, s, d]
                beta = np.einsum("ilks->kis", Lt)
                safe = np.where(beta > 0, beta, 1.0)
                qt[:, :, t] = np.where((beta > 0)[..., None], alpha / safe[..., None],
                                       qbar[t][None, :, None, :])

    U = np.einsum("kitsj,ksjd->kitsd", Rs, Vseg)           # u[k, i, t, s]
    y = np.empty((b1, nc, dv))
    for t in range(c1):
        rows = np.nonzero(tile == t)[0]
        # y[l,i] = sum_{k,s} L[i,l,k,s] u[k,i,t(l),s]
        y[rows] = np.einsum("ilks,kisd->lid", L[:, rows], U[:, :, t])
    out = dict(y=y, L=L, R=R, lse=lse.T, f_trace=np.array(f_trace))
    if history:
        out["history"] = hist
    return out


# ---------------------------------------------------------------------------
# dense reconstruction (tiny grids only)
# ---------------------------------------------------------------------------

def dense_from_factors(L, R, b1, b2, c1=1, c2=1):
    """Materialise M in grid order ([N, N], rows (l,i) -> l*b2+i, columns
    (k,j) -> k*b2+j) from the entry formula.  L, R in the untiled shapes
    [b2,b1,b1] / [b1,b2,b2] or the tiled shapes [b2,b1,b1,c2] / [b1,b2,c1,b2]."""
    if L.ndim == 3:
        L = L[..., None]
    if R.ndim == 3:
        R = R[:, :, None, :]
    tile = tile_of_rows(b1, c1)
    seg = segment_of_cols(b2, c2)
    N = b1 * b2
    M = np.empty((N, N))
    for l in range(b1):
        for i in range(b2):
            for k in range(b1):
                for j in range(b2):
                    M[l * b2 + i, k * b2 + j] = L[i, l, k, seg[j]] * R[k, i, tile[l], j]
    return M


# ---------------------------------------------------------------------------
# [B, H, N, d] driver
# ---------------------------------------------------------------------------

def forward(Q, K, V, b1, b2, steps, c1=1, c2=1, scale=None, layout="flat",
            fhw=None, cols=None, tiled=None, slices=None, pad="post", causal=0):
    """MonarchAttention on [B, H, N, d] queries and [B, Hkv, N, d] keys and
    values (any float dtype, upcast to float64).  Hkv < H is grouped-query
    attention: query head h uses key/value head h // (H // Hkv), and the
    method runs per query head unchanged (MonarchAttention, OpenReview author
    response on GQA/MLA: a direct transfer).  The layout permutation maps
    token order to the b1 x b2 grid (oracle.layouts); Y is mapped back.  A
    flat sequence with N < b1*b2 is padded ("pre" or "post", see
    oracle.layouts.grid_index); L rows of padding positions are zero.

    cols: optional columns i to compute (Y is then NaN outside them).
    slices: optional list of (b, h) pairs to compute (others left NaN).
    tiled: force the tiled algorithm (default: tiled iff c1*c2 > 1).
    causal: 0 (bidirectional) or g, the grid blocks per causal unit: query
    block l attends to key block k iff floor(k/g) <= floor(l/g).

    Returns dict with y [B,H,N,d] (token order), L, R (per slice, grid
    order, as returned by forward_untiled / forward_tiled, stacked), lse
    [B,H,N] (token order) and f_trace [B,H,2T].
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    B, H, N, d = Q.shape
    dv = V.shape[-1]
    Hkv = K.shape[1]
    if K.shape[:3] != (B, Hkv, N) or V.shape[:3] != (B, Hkv, N) or H % Hkv:
        raise ValueError("K, V must be [B, Hkv, N, .] with Hkv dividing H")
    group = H // Hkv
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    grid = grid_index(N, b1, b2, layout, fhw, pad)
    real = grid >= 0
    if tiled is None:
        tiled = c1 * c2 > 1
    sel = [(b, h) for b in range(B) for h in range(H)] if slices is None else list(slices)
    colsel = np.arange(b2) if cols is None else np.asarray(cols)
    nc = colsel.size

    y = np.full((B, H, N, dv), np.nan)
    lse = np.full((B, H, N), np.nan)
    if tiled:
        Ls = np.full((B, H, nc, b1, b1, c2), np.nan)
        Rs = np.full((B, H, b1, nc, c1, b2), np.nan)
    else:
        Ls = np.full((B, H, nc, b1, b1), np.nan)
        Rs = np.full((B, H, b1, nc, b2), np.nan)
    ft = np.full((B, H, 2 * steps), np.nan)
    for (b, h) in sel:
        qg = to_grid(Q[b, h], grid)
        kg, vg = (to_grid(X[b, h // group], grid) for X in (K, V))
        if tiled:
            r = forward_tiled(qg, kg, vg, steps, scale, c1, c2, cols=colsel, real=real,
                              causal=causal)
        else:
            r = forward_untiled(qg, kg, vg, steps, scale, cols=colsel, real=real, causal=causal)
        tok = grid[:, colsel].reshape(-1)          # tokens of the computed grid cells
        ok = tok >= 0
        y[b, h][tok[ok]] = r["y"].reshape(-1, dv)[ok]
        lse[b, h][tok[ok]] = r["lse"].reshape(-1)[ok]
        Ls[b, h] = r["L"]
        Rs[b, h] = r["R"]
        ft[b, h] = r["f_trace"]
    return dict(y=y, L=Ls, R=Rs, lse=lse, f_trace=ft, grid=grid, cols=colsel)
