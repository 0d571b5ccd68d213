"""Plain float64 CPU oracle of the Pixtral-class vision tower.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and ``bench.py``'s ``cpu_baseline`` leg, never by the product path.  It shares
no code, header, table or constant generator with the HIP library.

Sources (cited by page title and section):

* "Mistral 3" (KerasFormers model page).  The ``Mistral3VisionModel`` entry
  describes the tower: a convolutional patch embedding, an RMS pre-norm, then
  blocks with a two-dimensional rotary embedding, run over all images packed
  into one variable-resolution patch sequence.  The ``Mistral3Model`` argument
  table gives the vision width 1024, MLP width 4096, depth 24, 16 heads,
  patch 14, rotary base 1e4, ``spatial_merge_size`` 2, a projector without
  bias, and text width 5120; its description names the 2x2 patch-merging
  projector.  The ``Mistral3ImageProcessor`` table gives the normalisation
  mean/std.  "Several images in one conversation" says every image expands to
  its own patch count.
* "Pixtral-12B-2409" (inference-research model record), part (1) Vision and
  the VISION TOKENS paragraph: patch 16, no spatial merge (one token per
  patch), 1024x1024 tiles of 4,096 tokens, a 4096x4096 image as 16 tiles.
* "nemo_automodel.components.models.mistral3_vlm" (NeMo Automodel API page),
  ``forward``: the tower input is float ``pixel_values`` plus ``image_sizes``.

Readings taken where the pages are silent (each is also listed in the design
notes of the repository):

1. MLP: gated SiLU with three bias-free matrices, down(silu(gate y) * up y).
2. Pre-norm residual blocks; ``ln_pre`` after the patch embedding; no final
   norm after the last block.
3. 2-D RoPE on head_dim dh: dh/2 rotation pairs on adjacent dims (2j, 2j+1);
   pairs j < dh/4 turn by the patch row r, pairs j >= dh/4 by the patch
   column c, each axis with the ordinary 1-D ladder
   omega_m = theta^(-2m/(dh/2)), m = 0..dh/4-1.  Positions are 0-based within
   the image (tile).
4. Attention scale 1/sqrt(dh), non-causal, block-diagonal per image.
5. No biases anywhere.
6. 2x2 merge concatenates window offsets (dy,dx) in order 00,01,10,11, channel
   fastest; merged tokens row-major per image, images in input order.
7. The projector is a single bias-free linear map 4*D -> out_dim.
8. RMSNorm: x / sqrt(mean(x^2) + eps) * g with eps = 1e-5.
9. Resize target (the processor's description on the "Mistral 3" page): an
   image whose longest side exceeds ``longest_edge`` is first shrunk by the
   factor longest_edge / max(H, W), each side rounded down to whole pixels;
   smaller images are not enlarged.  Each side is then rounded up to the
   grid the projector consumes (patch * merge pixels), and never past the
   largest multiple of that grid within ``longest_edge``.
10. Resampling: bilinear with pixel centres at half-integers (source
    coordinate (t + 0.5) * in / out - 0.5, clamped at the first pixel, the
    upper neighbour clamped at the last), no antialiasing, on the uint8
    values taken as reals (no re-quantisation after the resize).
11. Normalisation: x / 255 then (x - mean_c) / std_c with the processor
    table's constants; uint8 pixels come in as H x W x 3 (RGB).
12. Tiles ("Pixtral-12B-2409", VISION TOKENS: large images are split into
    1024x1024 tiles, the tile count capped by ``max_num_tiles``): the image
    is scaled by the largest s <= 1 whose tile grid ceil(sH/T) x ceil(sW/T)
    has at most max_num_tiles tiles; each side becomes floor(s * side)
    (at least 1), rounded up to the patch grid; tiles are cut row-major,
    full T x T except the last row/column, which keep the remainder.
13. fp8 variant (the NeMo Automodel page's FP8-native Mistral 3 VLM
    registration): OCP e4m3 with one power-of-two scale per 32 values along
    the contraction axis, X = floor(log2(block max)) - 7, ties to even; the
    four linear maps of every block quantise both operands.
14. Deeper projector (off by default; the "Mistral 3" page names only a
    bias-free 2x2 patch-merging projector): RMSNorm of each patch (own
    gain), the 2x2 gather with a bias-free 4D -> D linear, then D -> out_dim,
    GELU (x Phi(x), the erf form), out_dim -> out_dim, without biases.

Pinning: every function here is pinned in ``tests/test_oracle_pins.py`` by a
check that does not reuse this code path (closed-form counts printed on the
pages, direct convolution loops, textbook dense masked softmax, rotation
identities, identity/zero weights; for the preprocessing, torch's bilinear
interpolate in float64, 2x2 block means, ramps, and a search-based statement
of the target-size rule).  The full tower against a trained model is
parity unpinned: neither weights nor another implementation exist here.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Tuple, Dict, List, Optional, Sequence

import numpy as np


@dataclass(frozen=True)
class TowerConfig:
    """Tower hyper-parameters ("Mistral 3", Mistral3Model argument table;
    "Pixtral-12B-2409", part (1) Vision)."""

    patch: int = 14
    hidden: int = 1024
    heads: int = 16
    mlp: int = 4096
    layers: int = 24
    merge: int = 2  # 1 = no spatial merge (Pixtral-12B)
    out_dim: int = 5120
    rope_theta: float = 1.0e4
    rms_eps: float = 1.0e-5
    deep_projector: bool = False  # reading 14: the deeper projector variant
    rope_interleaved: bool = False  # reading 3: columns on the odd ladder steps

    @property
    def head_dim(self) -> int:
        return self.hidden // self.heads

    @property
    def out_cols(self) -> int:
        return self.out_dim if self.merge == 2 else self.hidden


# --------------------------------------------------------------------------
# a0: per-image counts and index maps
# --------------------------------------------------------------------------
def plan_maps(image_hw: Sequence[Sequence[int]], patch: int, merge: int) -> Dict[str, np.ndarray]:
    """Patch counts, ``cu_seqlens``, (row, col) map and 2x2 merge source map.

    "Mistral 3", Mistral3VisionModel (packed variable-resolution sequence) and
    "Several images in one conversation" (each image keeps its own count);
    "Pixtral-12B-2409", VISION TOKENS (one token per patch without merge).

    Written as explicit loops over images, patches and merged tokens.
    """
    if merge not in (1, 2):
        raise ValueError("merge must be 1 or 2")
    cu = [0]
    rc: List[List[int]] = []
    src: List[List[int]] = []
    for (h, w) in image_hw:
        h, w = int(h), int(w)
        if h <= 0 or w <= 0 or h % (patch * merge) or w % (patch * merge):
            raise ValueError(f"image {h}x{w} is not on the {patch * merge}-pixel grid")
        hp, wp = h // patch, w // patch
        base = cu[-1]
        for j in range(hp * wp):
            rc.append([j // wp, j % wp])
        if merge == 2:
            for big_r in range(hp // 2):
                for big_c in range(wp // 2):
                    row = []
                    for dy in (0, 1):
                        for dx in (0, 1):
                            row.append(base + (2 * big_r + dy) * wp + (2 * big_c + dx))
                    src.append(row)
        cu.append(base + hp * wp)
    out = {
        "cu_seqlens": np.asarray(cu, dtype=np.int64),
        "patch_rc": np.asarray(rc, dtype=np.int64).reshape(-1, 2),
        "n_patches": cu[-1],
    }
    if merge == 2:
        out["merge_src"] = np.asarray(src, dtype=np.int64).reshape(-1, 4)
        out["out_rows"] = len(src)
    else:
        out["out_rows"] = cu[-1]
    return out


# --------------------------------------------------------------------------
# a1: convolutional patch embedding (stride = kernel = patch, no bias)
# --------------------------------------------------------------------------
def patch_embed(pixels: np.ndarray, image_hw, w_patch: np.ndarray, patch: int) -> np.ndarray:
    """X[g, o] = sum_{c,u,v} W[o,c,u,v] * px_i[c, r*p+u, col*p+v].

    "Mistral 3", Mistral3VisionModel (convolutional patch embedding).
    ``pixels`` is the flat concatenation of each image's C x H x W plane set,
    images in input order.  Each image's patches are cut out with a reshape
    (the im2col rows, K order (c,u,v)) and multiplied by the flattened kernel.
    """
    w = np.asarray(w_patch, dtype=np.float64)
    d = w.shape[0]
    wmat = w.reshape(d, -1)
    pix = np.asarray(pixels, dtype=np.float64).reshape(-1)
    rows = []
    off = 0
    for (h, wd) in image_hw:
        h, wd = int(h), int(wd)
        img = pix[off: off + 3 * h * wd].reshape(3, h, wd)
        off += 3 * h * wd
        hp, wp = h // patch, wd // patch
        cols = (img.reshape(3, hp, patch, wp, patch)
                .transpose(1, 3, 0, 2, 4)
                .reshape(hp * wp, 3 * patch * patch))
        rows.append(cols @ wmat.T)
    return np.concatenate(rows, axis=0)


# --------------------------------------------------------------------------
# a2/a3: RMSNorm
# --------------------------------------------------------------------------
def rms_norm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * g, per row ("Mistral 3", Mistral3VisionModel:
    RMS pre-norm)."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(g, dtype=np.float64)


# --------------------------------------------------------------------------
# a5 (part): 2-D rotary position embedding
# --------------------------------------------------------------------------
def rope_omega(head_dim: int, theta: float) -> np.ndarray:
    """Per-axis frequency ladder omega_m = theta^(-2m/(head_dim/2)),
    m = 0..head_dim/4-1 (rotary base from "Mistral 3", Mistral3Model table,
    vision_rope_theta; split between axes per reading 3)."""
    per_axis = head_dim // 4
    m = np.arange(per_axis, dtype=np.float64)
    return np.power(float(theta), -2.0 * m / (head_dim / 2.0))


def rope_axis_omegas(head_dim: int, theta: float, interleaved: bool = False):
    """(row, column) frequency ladders.  Default (reading 3): both axes
    omega_m = theta^(-2m/(head_dim/2)).  interleaved: the axes share one
    ladder theta^(-j/(head_dim/2)), j = 0..head_dim/2-1, rows on the even
    steps j = 2m and columns on the odd steps j = 2m + 1."""
    rows = rope_omega(head_dim, theta)
    if not interleaved:
        return rows, rows.copy()
    m = np.arange(head_dim // 4, dtype=np.float64)
    return rows, np.power(float(theta), -(2.0 * m + 1.0) / (head_dim / 2.0))


def rope_2d(x: np.ndarray, patch_rc: np.ndarray, heads: int, theta: float, interleaved: bool = False) -> np.ndarray:
    """Rotate every head's adjacent pairs (2j, 2j+1) by the patch's row (first
    half of the pairs) or column (second half) times that axis's omega.

    "Mistral 3", Mistral3VisionModel (2-D rotary blocks).
    (x0, x1) -> (x0 cos a - x1 sin a, x0 sin a + x1 cos a).
    """
    x = np.asarray(x, dtype=np.float64)
    n, width = x.shape
    dh = width // heads
    om_r, om_c = rope_axis_omegas(dh, theta, interleaved)
    rc = np.asarray(patch_rc, dtype=np.float64)
    ang = np.concatenate([rc[:, 0:1] * om_r[None, :], rc[:, 1:2] * om_c[None, :]], axis=1)  # [n, dh/2]
    cos = np.cos(ang)[:, None, :]
    sin = np.sin(ang)[:, None, :]
    xp = x.reshape(n, heads, dh // 2, 2)
    x0 = xp[..., 0]
    x1 = xp[..., 1]
    out = np.empty_like(xp)
    out[..., 0] = x0 * cos - x1 * sin
    out[..., 1] = x0 * sin + x1 * cos
    return out.reshape(n, width)


# --------------------------------------------------------------------------
# a5: block-diagonal multi-head attention over the packed sequence
# --------------------------------------------------------------------------
def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, cu_seqlens, heads: int) -> np.ndarray:
    """For each image i and head h: softmax(q k^T / sqrt(dh)) v over the
    image's own patches only ("Mistral 3", Mistral3VisionModel: attention over
    a packed variable-resolution sequence, each image its own block).

    q and k are already rotated.  The row maximum is subtracted before the
    exponential (the softmax is unchanged by it).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, width = q.shape
    dh = width // heads
    scale = 1.0 / np.sqrt(dh)
    out = np.zeros_like(q)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    for i in range(len(cu) - 1):
        a, b = int(cu[i]), int(cu[i + 1])
        if b == a:
            continue
        for h in range(heads):
            cs = slice(h * dh, (h + 1) * dh)
            s = (q[a:b, cs] @ k[a:b, cs].T) * scale
            s -= s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p /= p.sum(axis=1, keepdims=True)
            out[a:b, cs] = p @ v[a:b, cs]
    return out


# --------------------------------------------------------------------------
# a7/a8: vision MLP (reading 1: gated SiLU)
# --------------------------------------------------------------------------
def swiglu_mlp(y: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray, w_down: np.ndarray,
               hidden_map=None) -> np.ndarray:
    """down(silu(y gate^T) * (y up^T)), silu(x) = x / (1 + exp(-x))
    ("Mistral 3", Mistral3Model table, vision_mlp_dim 4096).  ``hidden_map``
    (optional) is applied to silu * up before the down projection."""
    y = np.asarray(y, dtype=np.float64)
    g = y @ np.asarray(w_gate, dtype=np.float64).T
    u = y @ np.asarray(w_up, dtype=np.float64).T
    hmid = g / (1.0 + np.exp(-g)) * u
    if hidden_map is not None:
        hmid = hidden_map(hmid)
    return hmid @ np.asarray(w_down, dtype=np.float64).T


# --------------------------------------------------------------------------
# a11/a12: 2x2 patch merge + projection to the text width
# --------------------------------------------------------------------------
def merge_project(h: np.ndarray, merge_src: np.ndarray, w_merge: np.ndarray) -> np.ndarray:
    """out[t] = concat(h[src[t,0]], h[src[t,1]], h[src[t,2]], h[src[t,3]]) W^T.

    "Mistral 3", Mistral3Model description (2x2 patch-merging projector) and
    argument table (spatial_merge_size 2, projector_bias False, embed_dim 5120).
    """
    h = np.asarray(h, dtype=np.float64)
    src = np.asarray(merge_src, dtype=np.int64)
    z = np.concatenate([h[src[:, 0]], h[src[:, 1]], h[src[:, 2]], h[src[:, 3]]], axis=1)
    return z @ np.asarray(w_merge, dtype=np.float64).T


def gelu(x: np.ndarray) -> np.ndarray:
    """GELU(x) = x Phi(x), Phi the standard normal distribution function,
    Phi(x) = (1 + erf(x / sqrt 2)) / 2."""
    from scipy.special import erf
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + erf(x / math.sqrt(2.0)))


def deep_project(h: np.ndarray, merge_src: np.ndarray, w_merge: np.ndarray, proj: dict, eps: float) -> np.ndarray:
    """The deeper projector variant (reading 14; the pages name only a 2x2
    patch-merging projector without bias): RMSNorm of every patch with its own
    gain, the 2x2 gather and a bias-free 4D -> D linear, then D -> out_dim,
    GELU, out_dim -> out_dim, all bias-free."""
    y = rms_norm(h, proj["norm"], eps)
    m = merge_project(y, merge_src, w_merge)
    a = gelu(m @ np.asarray(proj["w1"], dtype=np.float64).T)
    return a @ np.asarray(proj["w2"], dtype=np.float64).T


# --------------------------------------------------------------------------
# after the tower: masked scatter into the text-embedding sequence
# --------------------------------------------------------------------------
def masked_scatter(token_ids: np.ndarray, image_emb: np.ndarray, text_emb: np.ndarray,
                   image_token_id: int) -> Tuple[np.ndarray, bool]:
    """The k-th placeholder position of the sequence takes image row k.

    "Mistral 3", Mistral3Model argument table: image_token_id is the
    placeholder the processor expands per image; "Several images in one
    conversation": each image's marker expands to that image's own count, so
    the placeholders of all images, in sequence order, line up with the
    merged rows of all images in input order.  Returns (new text embeddings,
    whether the placeholder count equals the number of image rows); on a
    mismatch the first min(count, rows) placeholders are filled.
    """
    ids = np.asarray(token_ids)
    out = np.array(text_emb, copy=True)
    positions = [p for p in range(ids.shape[0]) if int(ids[p]) == int(image_token_id)]
    rows = np.asarray(image_emb)
    for k, p in enumerate(positions):
        if k < rows.shape[0]:
            out[p] = rows[k]
    return out, len(positions) == rows.shape[0]


# --------------------------------------------------------------------------
# before the tower: resize onto the patch grid and normalise (uint8 input)
# --------------------------------------------------------------------------
# "Mistral 3", Mistral3ImageProcessor table: per-channel mean and std
PROCESSOR_MEAN = (0.48145466, 0.4578275, 0.40821073)
PROCESSOR_STD = (0.26862954, 0.26130258, 0.27577711)


def resize_target(h: int, w: int, longest_edge: int, grid: int) -> Tuple[int, int]:
    """(H, W) of the resized image, in exact integer arithmetic.

    "Mistral 3" page, model description: images are resized so that the
    longest edge fits ``longest_edge`` and the sides stay on the patch grid.
    Step 1 (fit): if max(H, W) > longest_edge, each side becomes
    floor(side * longest_edge / max(H, W)) (at least 1).  Step 2 (grid): each
    side is rounded up to a multiple of ``grid``, capped at the largest
    multiple of ``grid`` that is <= longest_edge.
    """
    h, w, L, g = int(h), int(w), int(longest_edge), int(grid)
    if h <= 0 or w <= 0 or g <= 0 or L < g:
        raise ValueError("sides and grid must be positive and longest_edge >= grid")
    m = max(h, w)
    if m > L:
        h = max(1, (h * L) // m)
        w = max(1, (w * L) // m)
    cap = (L // g) * g
    return min(-(-h // g) * g, cap), min(-(-w // g) * g, cap)


def bilinear_taps(n_in: int, n_out: int, t: int) -> Tuple[int, int, float]:
    """Source taps (i0, i1) and weight f of i1 for output index t.

    Pixel centres at half-integers: s = (t + 0.5) * n_in / n_out - 0.5,
    clamped below at 0; i0 = floor(s), i1 = min(i0 + 1, n_in - 1), f = s - i0.
    """
    s = (t + 0.5) * n_in / n_out - 0.5
    if s < 0.0:
        s = 0.0
    i0 = int(math.floor(s))
    i1 = min(i0 + 1, n_in - 1)
    return i0, i1, s - i0


def interp_matrix(n_in: int, n_out: int) -> np.ndarray:
    """[n_out][n_in] matrix of the 1-D bilinear resampling (rows of taps)."""
    m = np.zeros((n_out, n_in), dtype=np.float64)
    for t in range(n_out):
        i0, i1, f = bilinear_taps(n_in, n_out, t)
        m[t, i0] += 1.0 - f
        m[t, i1] += f
    return m


def preprocess_image(img_u8: np.ndarray, th: int, tw: int,
                     mean: Sequence[float] = PROCESSOR_MEAN,
                     std: Sequence[float] = PROCESSOR_STD) -> np.ndarray:
    """uint8 H x W x 3 image -> float64 3 x th x tw planes, resized and
    normalised.

    The bilinear resize is separable: out_c = R_h img_c R_w^T with the two
    1-D interpolation matrices; then x / 255 and (x - mean_c) / std_c
    ("Mistral 3", Mistral3ImageProcessor table).
    """
    img = np.asarray(img_u8)
    if img.ndim != 3 or img.shape[2] != 3:
        raise ValueError("image must be H x W x 3")
    h, w = img.shape[:2]
    rh, rw = interp_matrix(h, th), interp_matrix(w, tw)
    out = np.empty((3, th, tw), dtype=np.float64)
    for c in range(3):
        plane = rh @ img[:, :, c].astype(np.float64) @ rw.T
        out[c] = (plane / 255.0 - mean[c]) / std[c]
    return out


def preprocess_pixel(img_u8: np.ndarray, th: int, tw: int, c: int, y: int, x: int,
                     mean: Sequence[float] = PROCESSOR_MEAN,
                     std: Sequence[float] = PROCESSOR_STD) -> float:
    """One value of ``preprocess_image`` (channel c, row y, column x) from its
    four taps, for spot checks of large images."""
    img = np.asarray(img_u8)
    h, w = img.shape[:2]
    y0, y1, fy = bilinear_taps(h, th, y)
    x0, x1, fx = bilinear_taps(w, tw, x)
    v = ((1 - fy) * ((1 - fx) * float(img[y0, x0, c]) + fx * float(img[y0, x1, c]))
         + fy * ((1 - fx) * float(img[y1, x0, c]) + fx * float(img[y1, x1, c])))
    return (v / 255.0 - mean[c]) / std[c]


def preprocess_batch(images: Sequence[np.ndarray], longest_edge: int, grid: int,
                     mean: Sequence[float] = PROCESSOR_MEAN,
                     std: Sequence[float] = PROCESSOR_STD):
    """uint8 images -> (flat float64 pixels, target sizes) in the tower's input
    layout: each image's 3 x H x W planes after the previous image's."""
    hw = [resize_target(im.shape[0], im.shape[1], longest_edge, grid) for im in images]
    parts = [preprocess_image(im, th, tw, mean, std).reshape(-1) for im, (th, tw) in zip(images, hw)]
    return np.concatenate(parts), hw


def tile_layout(h: int, w: int, tile: int, grid: int, max_num_tiles: int) -> Tuple[int, int, int, int]:
    """(resized H, resized W, tile rows, tile columns) of one image.

    "Pixtral-12B-2409", VISION TOKENS: tiles of ``tile`` x ``tile`` pixels
    (a 4096x4096 image is a 4x4 grid); the processor caps the tile count with
    ``max_num_tiles``.  Scale s = min(1, max over grids r x c with r*c <=
    max_num_tiles of min(r*tile/H, c*tile/W)), exact fractions; each side
    becomes max(1, floor(s * side)) rounded up to a multiple of ``grid``.
    """
    from fractions import Fraction
    h, w, T, g, M = int(h), int(w), int(tile), int(grid), int(max_num_tiles)
    if h <= 0 or w <= 0 or g <= 0 or T < g or T % g or M < 1:
        raise ValueError("bad tile layout arguments")
    best = Fraction(0)
    for r in range(1, M + 1):
        for c in range(1, M // r + 1):
            best = max(best, min(Fraction(r * T, h), Fraction(c * T, w)))
    s = min(Fraction(1), best)
    rh = max(1, math.floor(s * h))
    rw = max(1, math.floor(s * w))
    rh = -(-rh // g) * g
    rw = -(-rw // g) * g
    return rh, rw, -(-rh // T), -(-rw // T)


def tile_image(img_u8: np.ndarray, tile: int, grid: int, max_num_tiles: int,
               mean: Sequence[float] = PROCESSOR_MEAN, std: Sequence[float] = PROCESSOR_STD):
    """uint8 H x W x 3 image -> (list of float64 3 x th x tw tiles, their
    sizes), row-major over the tile grid: the image resized to the
    ``tile_layout`` size and normalised, then cut."""
    img = np.asarray(img_u8)
    rh, rw, rows, cols = tile_layout(img.shape[0], img.shape[1], tile, grid, max_num_tiles)
    full = preprocess_image(img, rh, rw, mean, std)
    tiles, hw = [], []
    for a in range(rows):
        for b in range(cols):
            t = full[:, a * tile: min((a + 1) * tile, rh), b * tile: min((b + 1) * tile, rw)]
            tiles.append(t)
            hw.append((t.shape[1], t.shape[2]))
    return tiles, hw


def tile_batch(images: Sequence[np.ndarray], tile: int, grid: int, max_num_tiles: int,
               mean: Sequence[float] = PROCESSOR_MEAN, std: Sequence[float] = PROCESSOR_STD):
    """Tiles of every image, images in order, in the tower's input layout:
    (flat float64 pixels, tile sizes, tiles per image)."""
    parts, hw, counts = [], [], []
    for im in images:
        tiles, thw = tile_image(im, tile, grid, max_num_tiles, mean, std)
        parts += [t.reshape(-1) for t in tiles]
        hw += thw
        counts.append(len(tiles))
    return np.concatenate(parts), hw, counts


# --------------------------------------------------------------------------
# content key of a uint8 image (embeddings cache)
# --------------------------------------------------------------------------
_M64 = (1 << 64) - 1
KEY_G = (0x9E3779B97F4A7C15, 0xD1B54A32D192ED03)


def splitmix64_mix(z: int) -> int:
    """Output function of the SplitMix64 generator (Steele, Lea and Flood,
    2014; Vigna's constants), on Python integers mod 2^64."""
    z &= _M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
    return z ^ (z >> 31)


def image_key(img_u8: np.ndarray) -> Tuple[int, int]:
    """Two 64-bit lanes over an H x W x 3 uint8 image, for the multimodal
    embeddings cache (the inference-research record's per-model cache):
    words w_i = the bytes as little-endian 64-bit integers, zero-padded;
    acc_s = sum_i mix(w_i + (i + 1) G_s) mod 2^64;
    key_s = mix(acc_s + mix(((H << 32) | W) ^ G_s)).  Written as a loop over
    Python integers (small images only)."""
    img = np.asarray(img_u8, dtype=np.uint8)
    h, w = img.shape[:2]
    data = img.tobytes()
    keys = []
    for g in KEY_G:
        acc = 0
        for i in range(0, len(data), 8):
            word = int.from_bytes(data[i:i + 8].ljust(8, b"\0"), "little")
            acc = (acc + splitmix64_mix(word + (i // 8 + 1) * g)) & _M64
        keys.append(splitmix64_mix(acc + splitmix64_mix(((h << 32) | w) ^ g)))
    return keys[0], keys[1]


# --------------------------------------------------------------------------
# fp8 (e4m3) GEMM variant: block-scaled quantisation of GEMM operands
# --------------------------------------------------------------------------
def e4m3_round(v: np.ndarray) -> np.ndarray:
    """Nearest OCP e4m3 value (1 sign, 4 exponent bits with bias 7, 3
    mantissa bits; normal range 2^-6 .. 448, subnormal step 2^-9), ties to
    the even mantissa, as float64.  Inputs must lie within +-464 (no
    saturation is needed by the block scaling below)."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    if np.any(a >= 464.0):
        raise ValueError("value outside the e4m3 range")
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -6.0)          # below 2^-6 the step stays 2^-9
    step = np.exp2(e - 3.0)
    q = np.round(a / step) * step    # numpy rounds halves to even
    return np.sign(v) * q


def mx_e4m3(x: np.ndarray) -> np.ndarray:
    """Block-scaled e4m3 copy of x along its last axis (blocks of 32
    consecutive elements), dequantised to float64: per block
    X = floor(log2(max |x|)) - 7 clamped to [-120, 120], values
    e4m3(x * 2^-X) * 2^X -- the block maximum lands in [128, 256).
    The scale is a power of two, as in the MX formats' shared exponent
    (E8M0), one per 32 values."""
    x = np.asarray(x, dtype=np.float64)
    k = x.shape[-1]
    if k % 32:
        raise ValueError("the quantised axis must be a multiple of 32")
    blocks = x.reshape(x.shape[:-1] + (k // 32, 32))
    amax = np.max(np.abs(blocks), axis=-1, keepdims=True)
    _, ex = np.frexp(np.where(amax > 0, amax, 1.0))
    X = np.where(amax > 0, ex - 1 - 7, -120).clip(-120, 120).astype(np.float64)
    q = e4m3_round(blocks * np.exp2(-X)) * np.exp2(X)
    return q.reshape(x.shape)


# --------------------------------------------------------------------------
# whole tower
# --------------------------------------------------------------------------
def tower_forward(
    pixels: np.ndarray,
    image_hw,
    weights: dict,
    cfg: TowerConfig,
    layers: Optional[int] = None,
    collect: bool = False,
    fp8: bool = False,
) -> Dict[str, np.ndarray]:
    """Pixels + image sizes -> merged embeddings (or per-patch states when
    merge == 1).

    "Mistral 3", Mistral3VisionModel: patch embedding -> RMS pre-norm -> blocks;
    each block: h += attn(rope(norm(h))), h += mlp(norm(h)).  Then the 2x2
    merging projector ("Mistral 3", Mistral3Model), or no merge
    ("Pixtral-12B-2409", part (1) Vision).

    ``weights``: ``patch_w`` [D,3,p,p], ``ln_pre`` [D], ``layers`` (list of dicts
    with ``attn_norm``, ``wq``, ``wk``, ``wv``, ``wo``, ``ffn_norm``,
    ``w_gate``, ``w_up``, ``w_down``), ``merge_w`` [out_dim, 4D].
    ``layers`` limits the depth (default cfg.layers).  With ``collect`` the
    per-stage tensors are returned too.  With ``fp8`` the four linear maps of
    every block (q/k/v, out-projection, gate/up, down) take both operands
    through ``mx_e4m3`` along their contraction axis first (the fp8 GEMM
    variant); the patch embedding, attention and the merger stay exact.
    """
    qz = mx_e4m3 if fp8 else (lambda a: a)
    n_layers = cfg.layers if layers is None else layers
    maps = plan_maps(image_hw, cfg.patch, cfg.merge)
    res: Dict[str, np.ndarray] = {"maps": maps}
    x = patch_embed(pixels, image_hw, weights["patch_w"], cfg.patch)
    if collect:
        res["patch_embed"] = x.copy()
    h = rms_norm(x, weights["ln_pre"], cfg.rms_eps)
    if collect:
        res["ln_pre"] = h.copy()
        res["attn_out"] = []
        res["block_out"] = []
    cu = maps["cu_seqlens"]
    rc = maps["patch_rc"]
    for li in range(n_layers):
        lw = weights["layers"][li]
        W = {k_: qz(np.asarray(lw[k_], np.float64)) for k_ in ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")}
        y = qz(rms_norm(h, lw["attn_norm"], cfg.rms_eps))
        q = rope_2d(y @ W["wq"].T, rc, cfg.heads, cfg.rope_theta, cfg.rope_interleaved)
        k = rope_2d(y @ W["wk"].T, rc, cfg.heads, cfg.rope_theta, cfg.rope_interleaved)
        v = y @ W["wv"].T
        a = attention(q, k, v, cu, cfg.heads)
        h = h + qz(a) @ W["wo"].T
        if collect:
            res["attn_out"].append(h.copy())
        y = qz(rms_norm(h, lw["ffn_norm"], cfg.rms_eps))
        h = h + swiglu_mlp(y, W["w_gate"], W["w_up"], W["w_down"], hidden_map=qz if fp8 else None)
        if collect:
            res["block_out"].append(h.copy())
    res["tower_out"] = h
    if cfg.merge == 2 and cfg.deep_projector:
        res["out"] = deep_project(h, maps["merge_src"], weights["merge_w"], weights["proj"], cfg.rms_eps)
    elif cfg.merge == 2:
        res["out"] = merge_project(h, maps["merge_src"], weights["merge_w"])
    else:
        res["out"] = h
    return res
