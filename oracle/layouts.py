"""Token order -> Monarch block grid, for flat sequences and video latents.

Test infrastructure only (see the package docstring).

A Monarch factorisation views the N tokens as a b1 x b2 grid: grid position
(l, i) with l in [b1] (block index) and i in [b2] (position inside the block).
For a flat sequence the grid is the plain row-major reshape, token n = l*b2 + i
([MA] OpenReview author response on block sizes: b is the block length and
m = ceil(N/b) the number of blocks).

For a video latent of f x h x w tokens stored row-major in (f, h, w), [MRT]
"Key claims" (section 4.1) and "Method" part (2) say the positional part of
attention is exactly representable only when each of the three axes lies
wholly inside one of the two factors, which leaves six aligned choices,
written (b1 axes, b2 axes):

    (fh, w)  (w, fh)  (f, hw)  (hw, f)  (fw, h)  (h, fw)

Within a factor the axes keep their major-to-minor order (f before h before
w).  The pages do not fix that inner order; any fixed order gives the same
set of Monarch matrices, and this one is the natural row-major choice.
"""

import numpy as np

# name -> (axes of b1, axes of b2); axes are 0=f, 1=h, 2=w.
LAYOUTS = {
    "fh_w": ((0, 1), (2,)),
    "w_fh": ((2,), (0, 1)),
    "f_hw": ((0,), (1, 2)),
    "hw_f": ((1, 2), (0,)),
    "fw_h": ((0, 2), (1,)),
    "h_fw": ((1,), (0, 2)),
}


def grid_index(seq_len, b1, b2, layout="flat", fhw=None, pad="post"):
    """Return an int array G of shape [b1, b2]: G[l, i] is the token at grid
    position (l, i), or -1 for a padding position.

    layout "flat": G[l, i] = l*b2 + i.  A flat sequence with b1*b2 > seq_len
    is padded to the grid ([MA] OpenReview author response on block sizes: b
    is chosen, m = ceil(N/b), and padding goes before the sequence -- "pre",
    as for ViT's leading class token -- or after it -- "post"): with P =
    b1*b2 - seq_len padding positions, G[l, i] = l*b2 + i - P for "pre" and
    l*b2 + i for "post", and positions outside [0, seq_len) are padding.
    Otherwise fhw = (f, h, w) with f*h*w == seq_len, and the token grid
    arange(N).reshape(f, h, w) is transposed so that the b1 axes come first,
    then reshaped to [b1, b2].
    """
    if layout == "flat":
        if b1 * b2 < seq_len:
            raise ValueError("b1*b2 must be at least seq_len")
        if pad not in ("pre", "post"):
            raise ValueError("pad must be 'pre' or 'post'")
        g = np.arange(b1 * b2) - (b1 * b2 - seq_len if pad == "pre" else 0)
        g[(g < 0) | (g >= seq_len)] = -1
        return g.reshape(b1, b2)
    if b1 * b2 != seq_len:
        raise ValueError("b1*b2 must equal seq_len")
    if layout not in LAYOUTS:
        raise ValueError(f"unknown layout {layout!r}")
    f, h, w = fhw
    if f * h * w != seq_len:
        raise ValueError("f*h*w must equal seq_len")
    sizes = (f, h, w)
    a1, a2 = LAYOUTS[layout]
    n1 = int(np.prod([sizes[a] for a in a1]))
    n2 = int(np.prod([sizes[a] for a in a2]))
    if (n1, n2) != (b1, b2):
        raise ValueError(f"layout {layout} on {fhw} gives ({n1},{n2}), not ({b1},{b2})")
    tokens = np.arange(seq_len).reshape(f, h, w)
    return tokens.transpose(a1 + a2).reshape(b1, b2)


def to_grid(x, grid):
    """[N, ...] in token order -> [b1, b2, ...] in grid order (zeros at
    padding positions)."""
    out = x[np.maximum(grid, 0)]
    out[grid < 0] = 0
    return out


def from_grid(xg, grid):
    """[b1, b2, ...] in grid order -> [N, ...] in token order (padding
    positions dropped)."""
    real = grid.reshape(-1) >= 0
    n = int(real.sum())
    out = np.empty((n,) + xg.shape[2:], dtype=xg.dtype)
    out[grid.reshape(-1)[real]] = xg.reshape((grid.size,) + xg.shape[2:])[real]
    return out
