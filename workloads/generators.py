"""Seeded input generators (NumPy PCG64), one independent stream per slice.

Recipes (the readings of the one-line workload descriptions):

  iid      Q, K, V i.i.d. N(0, 1).
  lowrank  per slice Z = A B / sqrt(8) with A ~ N(0,1)^{N x 8}, B ~ N(0,1)^{8 x d},
           shared by Q, K and V of that slice; Q = G_Q + Z, K = G_K + Z,
           V = G_V + Z with G i.i.d. N(0, 1).  The shared rank-8 part gives
           peaked attention rows.
  normed   each token row is r * g / |g| with g ~ 0.5 * N(0, I_d) and
           r ~ U[0.5, 2], drawn independently for Q, K and V.
  video    f x h x w latent, row-major tokens.  d is split into three chunks
           (d_f, d_h, d_w) = (d/3 rounded down to even, the same, the rest);
           the chunk for an axis holds [sin(p w_m), cos(p w_m)] for the
           token's coordinate p on that axis, with w_m = 10000^(-2m/D) and D
           the chunk width.  Q and K are these codes plus independent
           N(0, 0.3^2) noise (the same codes for every head); V ~ N(0, 1).
           With zero noise the scores are a sum of one term per axis.

Seeding: seed = configuration seed; slice (b, h) uses
SeedSequence(seed).spawn(B*H)[b*H + h]; within a slice the draws are made in
the order listed above (Q, K, V, then the extra draws).

bf16 configurations round every value to bfloat16 with round-to-nearest-even
and return it as float32, so that the GPU (bf16 tensors) and the oracle
(float64 upcast) see exactly the same numbers.
"""

import numpy as np


def round_to_bf16(x):
    """Round float32 values to the nearest bfloat16 (ties to even); returns
    float32 holding bf16-representable values.  NaN/Inf are not expected."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    bias = ((u >> 16) & 1) + 0x7FFF
    r = ((u + bias) & 0xFFFF0000).astype(np.uint32)
    return r.view(np.float32).reshape(x.shape)


def slice_rngs(seed, batch, heads):
    ss = np.random.SeedSequence(seed).spawn(batch * heads)
    return [np.random.Generator(np.random.PCG64(s)) for s in ss]


def _sincos_codes(pos, width):
    """[len(pos), width] codes: width/2 sines then width/2 cosines."""
    half = width // 2
    m = np.arange(half, dtype=np.float64)
    omega = 10000.0 ** (-2.0 * m / width)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * omega[None, :]
    return np.concatenate([np.sin(ang), np.cos(ang)], axis=1)


def video_codes(fhw, d):
    """Separable positional codes [f*h*w, d] for a row-major (f, h, w) latent."""
    f, h, w = fhw
    df = (d // 3) // 2 * 2
    dh = df
    dw = d - df - dh
    fi, hi, wi = np.meshgrid(np.arange(f), np.arange(h), np.arange(w), indexing="ij")
    codes = np.concatenate([_sincos_codes(fi.reshape(-1), df),
                            _sincos_codes(hi.reshape(-1), dh),
                            _sincos_codes(wi.reshape(-1), dw)], axis=1)
    return codes


def _draw_slice(rng, cfg, noise_scale=None):
    N, d = cfg.seq_len, cfg.head_dim
    if cfg.data == "iid":
        q = rng.standard_normal((N, d))
        k = rng.standard_normal((N, d))
        v = rng.standard_normal((N, d))
    elif cfg.data == "lowrank":
        q = rng.standard_normal((N, d))
        k = rng.standard_normal((N, d))
        v = rng.standard_normal((N, d))
        a = rng.standard_normal((N, 8))
        bm = rng.standard_normal((8, d))
        z = a @ bm / np.sqrt(8.0)
        q, k, v = q + z, k + z, v + z
    elif cfg.data == "normed":
        out = []
        for _ in range(3):
            g = 0.5 * rng.standard_normal((N, d))
            r = rng.uniform(0.5, 2.0, size=N)
            out.append(r[:, None] * g / np.linalg.norm(g, axis=1, keepdims=True))
        q, k, v = out
    elif cfg.data == "video":
        sd = 0.3 if noise_scale is None else noise_scale
        codes = video_codes(cfg.fhw, d)
        q = codes + sd * rng.standard_normal((N, d))
        k = codes + sd * rng.standard_normal((N, d))
        v = rng.standard_normal((N, d))
    else:
        raise ValueError(f"unknown data recipe {cfg.data!r}")
    return q, k, v


def make_inputs(cfg, slices=None, noise_scale=None):
    """Q, K, V as float32 arrays [B, H, N, d] (values representable in the
    configuration's dtype).  slices: optional list of (b, h) to generate;
    other slices are left zero (their streams are not drawn).  With
    cfg.kv_heads < heads, K and V keep their first kv_heads heads."""
    B, H, N, d = cfg.batch, cfg.heads, cfg.seq_len, cfg.head_dim
    rngs = slice_rngs(cfg.seed, B, H)
    Q = np.zeros((B, H, N, d), np.float32)
    K = np.zeros_like(Q)
    V = np.zeros_like(Q)
    sel = [(b, h) for b in range(B) for h in range(H)] if slices is None else slices
    for (b, h) in sel:
        q, k, v = _draw_slice(rngs[b * H + h], cfg, noise_scale)
        for X, x in ((Q, q), (K, k), (V, v)):
            x = x.astype(np.float32)
            X[b, h] = round_to_bf16(x) if cfg.dtype == "bf16" else x
    kvh = getattr(cfg, "kv_heads", 0) or H
    if kvh < H:
        K, V = np.ascontiguousarray(K[:, :kvh]), np.ascontiguousarray(V[:, :kvh])
    return Q, K, V
