"""Pins of the CPU oracle to things other than itself.

Each test checks an oracle function against what the pages or mathematics
fix: counts the pages print, a direct convolution written as loops, a
textbook dense softmax with an explicit block mask, rotation identities,
identity and zero weights.  None of them re-calls the oracle routine it checks
to produce the expected value.  CPU only.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import pv_oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))


# ---------------------------------------------------------------- counts / maps
def test_token_counts_from_pages():
    with open(os.path.join(HERE, "golden", "token_counts.json")) as fh:
        cases = json.load(fh)["cases"]
    for c in cases:
        m = O.plan_maps(c["image_hw"], c["patch"], c["merge"])
        assert m["n_patches"] == c["n_patches"], c["source"]
        assert m["out_rows"] == c["out_rows"], c["source"]
        assert m["cu_seqlens"][-1] == c["n_patches"]


@pytest.mark.parametrize("hw,patch,merge", [
    ([(28, 28)], 14, 2), ([(28, 56)], 14, 2), ([(56, 28)], 14, 2), ([(42, 70)], 14, 1),
    ([(56, 84), (28, 28), (112, 56)], 14, 2), ([(64, 32), (32, 96)], 16, 2), ([(48, 16)], 16, 1),
])
def test_maps_brute_force(hw, patch, merge):
    m = O.plan_maps(hw, patch, merge)
    # enumerate every pixel-grid position independently: patch index of pixel
    # (y, x) of image i is base_i + (y // p) * Wp + (x // p)
    base = 0
    all_src = []
    for i, (h, w) in enumerate(hw):
        hp, wp = h // patch, w // patch
        assert m["cu_seqlens"][i] == base
        for y in range(0, h, patch):
            for x in range(0, w, patch):
                g = base + (y // patch) * wp + (x // patch)
                assert tuple(m["patch_rc"][g]) == (y // patch, x // patch)
        if merge == 2:
            # merged token (R, C) covers the 2p x 2p pixel window at (2pR, 2pC)
            for big_y in range(0, h, 2 * patch):
                for big_x in range(0, w, 2 * patch):
                    srcs = []
                    for yy in (big_y, big_y + patch):
                        for xx in (big_x, big_x + patch):
                            srcs.append(base + (yy // patch) * wp + xx // patch)
                    all_src.append(srcs)
        base += hp * wp
    assert m["cu_seqlens"][-1] == base
    if merge == 2:
        assert np.array_equal(m["merge_src"], np.array(all_src))
        # every patch is used exactly once
        assert sorted(m["merge_src"].reshape(-1).tolist()) == list(range(base))


@pytest.mark.parametrize("hw,patch,merge", [([(30, 28)], 14, 2), ([(28, 14)], 14, 2), ([(0, 28)], 14, 1), ([(20, 16)], 16, 1)])
def test_maps_reject_off_grid(hw, patch, merge):
    with pytest.raises(ValueError):
        O.plan_maps(hw, patch, merge)


# ---------------------------------------------------------------- patch embed
def _direct_conv(img, w, p):
    """Stride-p, kernel-p convolution as six nested loops."""
    c_in, h, wd = img.shape
    d = w.shape[0]
    hp, wp = h // p, wd // p
    out = np.zeros((hp * wp, d))
    for r in range(hp):
        for c in range(wp):
            for o in range(d):
                s = 0.0
                for ch in range(c_in):
                    for u in range(p):
                        for v in range(p):
                            s += w[o, ch, u, v] * img[ch, r * p + u, c * p + v]
                out[r * wp + c, o] = s
    return out


def test_patch_embed_direct_convolution():
    rng = np.random.default_rng(11)
    p = 4
    hw = [(8, 12), (4, 8)]
    imgs = [rng.standard_normal((3, h, w)) for h, w in hw]
    wts = rng.standard_normal((5, 3, p, p))
    flat = np.concatenate([im.reshape(-1) for im in imgs])
    got = O.patch_embed(flat, hw, wts, p)
    want = np.concatenate([_direct_conv(im, wts, p) for im in imgs])
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_patch_embed_one_hot_selects_pixel():
    rng = np.random.default_rng(3)
    p = 14
    hw = [(28, 42)]
    img = rng.random((3, 28, 42))
    w = np.zeros((3, 3, p, p))
    w[0, 2, 5, 7] = 1.0   # output 0 <- channel 2, (5, 7) inside each patch
    w[1, 0, 13, 0] = 1.0
    w[2, 1, 0, 13] = 1.0
    x = O.patch_embed(img.reshape(-1), hw, w, p)
    for r in range(2):
        for c in range(3):
            g = r * 3 + c
            assert x[g, 0] == img[2, r * p + 5, c * p + 7]
            assert x[g, 1] == img[0, r * p + 13, c * p + 0]
            assert x[g, 2] == img[1, r * p + 0, c * p + 13]


# ---------------------------------------------------------------- RMSNorm
def test_rms_norm_closed_form():
    x = np.array([[3.0, 4.0]])
    g = np.array([2.0, 0.5])
    # mean(x^2) = 12.5 ; with eps = 1e-5
    want = np.array([[3.0 / math.sqrt(12.5 + 1e-5) * 2.0, 4.0 / math.sqrt(12.5 + 1e-5) * 0.5]])
    np.testing.assert_allclose(O.rms_norm(x, g, 1e-5), want, rtol=1e-15)
    # eps matters for tiny rows: x = 1e-3 everywhere -> 1e-3 / sqrt(1e-6 + 1e-5)
    t = np.full((1, 4), 1e-3)
    np.testing.assert_allclose(O.rms_norm(t, np.ones(4), 1e-5), 1e-3 / math.sqrt(1.1e-5), rtol=1e-12)


def test_rms_norm_unit_rms_and_scale_invariance():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((7, 64)) * 5.0
    y = O.rms_norm(x, np.ones(64), 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=1)), 1.0, rtol=1e-12)
    np.testing.assert_allclose(O.rms_norm(3.7 * x, np.ones(64), 0.0), y, rtol=1e-12)


# ---------------------------------------------------------------- RoPE
def _rope_complex(x, r, c, heads, theta):
    """Same rotation written with complex numbers: pair j of a head is the
    complex number x[2j] + i x[2j+1], multiplied by exp(i * pos * omega)."""
    dh = x.shape[0] // heads
    per_axis = dh // 4
    out = np.empty_like(x)
    for h in range(heads):
        for j in range(dh // 2):
            m = j % per_axis
            omega = theta ** (-(2.0 * m) / (dh / 2))
            pos = r if j < per_axis else c
            z = complex(x[h * dh + 2 * j], x[h * dh + 2 * j + 1]) * complex(math.cos(pos * omega), math.sin(pos * omega))
            out[h * dh + 2 * j] = z.real
            out[h * dh + 2 * j + 1] = z.imag
    return out


def test_rope_matches_complex_form():
    rng = np.random.default_rng(5)
    heads, dh = 2, 64
    x = rng.standard_normal((4, heads * dh))
    rc = np.array([[0, 0], [3, 7], [109, 1], [12, 109]])
    got = O.rope_2d(x, rc, heads, 1e4)
    for i in range(4):
        np.testing.assert_allclose(got[i], _rope_complex(x[i], rc[i, 0], rc[i, 1], heads, 1e4), rtol=1e-12, atol=1e-12)


def test_rope_ladder_values():
    om = O.rope_omega(64, 1e4)
    assert om.shape == (16,)
    assert om[0] == 1.0
    np.testing.assert_allclose(om[1], 1e4 ** (-1.0 / 16.0), rtol=1e-15)
    np.testing.assert_allclose(om[15], 1e4 ** (-15.0 / 16.0), rtol=1e-15)


def test_rope_identity_norm_and_axis_split():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((5, 128))
    zero = np.zeros((5, 2), dtype=np.int64)
    np.testing.assert_array_equal(O.rope_2d(x, zero, 2, 1e4), x)
    rc = rng.integers(0, 110, size=(5, 2))
    y = O.rope_2d(x, rc, 2, 1e4)
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-12)
    # rows turn the first 16 pairs of each head, columns the last 16
    row_only = O.rope_2d(x, np.stack([rc[:, 0], np.zeros(5, np.int64)], 1), 2, 1e4)
    col_only = O.rope_2d(x, np.stack([np.zeros(5, np.int64), rc[:, 1]], 1), 2, 1e4)
    for h in range(2):
        first = slice(h * 64, h * 64 + 32)
        second = slice(h * 64 + 32, h * 64 + 64)
        np.testing.assert_array_equal(row_only[:, second], x[:, second])
        np.testing.assert_array_equal(col_only[:, first], x[:, first])


def test_rope_relative_offset_invariance_and_composition():
    rng = np.random.default_rng(7)
    q = rng.standard_normal((1, 64))
    k = rng.standard_normal((1, 64))
    for (p1, p2, d) in [((3, 5), (10, 2), (4, 9)), ((0, 0), (7, 7), (50, 1))]:
        a = np.dot(O.rope_2d(q, np.array([p1]), 1, 1e4)[0], O.rope_2d(k, np.array([p2]), 1, 1e4)[0])
        s1 = (p1[0] + d[0], p1[1] + d[1])
        s2 = (p2[0] + d[0], p2[1] + d[1])
        b = np.dot(O.rope_2d(q, np.array([s1]), 1, 1e4)[0], O.rope_2d(k, np.array([s2]), 1, 1e4)[0])
        np.testing.assert_allclose(a, b, rtol=1e-10)
    # R(p) R(p') = R(p + p')
    two = O.rope_2d(O.rope_2d(q, np.array([[2, 3]]), 1, 1e4), np.array([[5, 11]]), 1, 1e4)
    one = O.rope_2d(q, np.array([[7, 14]]), 1, 1e4)
    np.testing.assert_allclose(two, one, rtol=1e-12, atol=1e-12)


# The interleaved split (PV_FLAG_ROPE_INTERLEAVED): one ladder shared by the
# two axes, rows on its even steps and columns on its odd steps.
def _rope_complex_one_ladder(x, r, c, heads, theta):
    """Complex form of the interleaved split.  The ladder of dh/2 steps
    theta^(-j/(dh/2)) is built by repeated multiplication; row pair m of a
    head takes step 2m, column pair m step 2m + 1."""
    dh = x.shape[0] // heads
    per_axis = dh // 4
    step = theta ** (-1.0 / (dh / 2))
    ladder = [1.0]
    for _ in range(dh // 2 - 1):
        ladder.append(ladder[-1] * step)
    out = np.empty_like(x)
    for h in range(heads):
        for j in range(dh // 2):
            if j < per_axis:
                omega, pos = ladder[2 * j], r
            else:
                omega, pos = ladder[2 * (j - per_axis) + 1], c
            z = complex(x[h * dh + 2 * j], x[h * dh + 2 * j + 1]) * complex(math.cos(pos * omega), math.sin(pos * omega))
            out[h * dh + 2 * j] = z.real
            out[h * dh + 2 * j + 1] = z.imag
    return out


def test_rope_interleaved_matches_one_ladder_complex_form():
    rng = np.random.default_rng(15)
    heads = 2
    x = rng.standard_normal((4, heads * 64))
    rc = np.array([[0, 0], [3, 7], [109, 1], [12, 109]])
    got = O.rope_2d(x, rc, heads, 1e4, interleaved=True)
    for i in range(4):
        np.testing.assert_allclose(got[i], _rope_complex_one_ladder(x[i], rc[i, 0], rc[i, 1], heads, 1e4),
                                   rtol=1e-11, atol=1e-11)
    # and it is not the default split (the columns differ)
    assert np.max(np.abs(got - O.rope_2d(x, rc, heads, 1e4))) > 0.1


def test_rope_interleaved_rows_as_default_columns_at_scaled_positions():
    """Rows turn exactly as in the default split; a column position c turns
    like the default split's column position c * theta^(-1/32) (each column
    frequency is one ladder step below the default's); together the two axes
    cover the whole ladder once."""
    rng = np.random.default_rng(16)
    x = rng.standard_normal((3, 128))
    rows = np.array([[5, 0], [77, 0], [1, 0]])
    np.testing.assert_array_equal(O.rope_2d(x, rows, 2, 1e4, interleaved=True), O.rope_2d(x, rows, 2, 1e4))
    cols = np.array([[0, 5], [0, 77], [0, 1]], dtype=np.float64)
    scaled = cols * np.array([1.0, 1e4 ** (-1.0 / 32.0)])
    np.testing.assert_allclose(O.rope_2d(x, cols, 2, 1e4, interleaved=True), O.rope_2d(x, scaled, 2, 1e4),
                               rtol=1e-12, atol=1e-12)
    om_r, om_c = O.rope_axis_omegas(64, 1e4, interleaved=True)
    both = np.sort(np.concatenate([om_r, om_c]))[::-1]
    np.testing.assert_allclose(both[1:] / both[:-1], 1e4 ** (-1.0 / 32.0), rtol=1e-12)
    assert both[0] == 1.0


def test_rope_interleaved_relative_offset_invariance_per_axis():
    rng = np.random.default_rng(17)
    q = rng.standard_normal((1, 64))
    k = rng.standard_normal((1, 64))

    def dot(p1, p2):
        return np.dot(O.rope_2d(q, np.array([p1]), 1, 1e4, interleaved=True)[0],
                      O.rope_2d(k, np.array([p2]), 1, 1e4, interleaved=True)[0])

    for axis in (0, 1):
        for (p1, p2, d) in [((3, 5), (10, 2), 4), ((0, 0), (7, 7), 50)]:
            s1, s2 = list(p1), list(p2)
            s1[axis] += d
            s2[axis] += d
            np.testing.assert_allclose(dot(p1, p2), dot(tuple(s1), tuple(s2)), rtol=1e-10)
    two = O.rope_2d(O.rope_2d(q, np.array([[2, 3]]), 1, 1e4, True), np.array([[5, 11]]), 1, 1e4, True)
    np.testing.assert_allclose(two, O.rope_2d(q, np.array([[7, 14]]), 1, 1e4, True), rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- attention
def _dense_masked_attention(q, k, v, cu, heads):
    """Textbook softmax over the whole packed sequence with -inf outside each
    image's block, element by element."""
    n, width = q.shape
    dh = width // heads
    img = np.zeros(n, dtype=np.int64)
    for i in range(len(cu) - 1):
        img[cu[i]:cu[i + 1]] = i
    out = np.zeros((n, width))
    for h in range(heads):
        for t in range(n):
            logits = []
            for u in range(n):
                if img[u] == img[t]:
                    logits.append(sum(q[t, h * dh + e] * k[u, h * dh + e] for e in range(dh)) / math.sqrt(dh))
                else:
                    logits.append(-math.inf)
            mx = max(logits)
            w = [math.exp(s - mx) if s != -math.inf else 0.0 for s in logits]
            z = sum(w)
            for e in range(dh):
                out[t, h * dh + e] = sum(w[u] * v[u, h * dh + e] for u in range(n)) / z
    return out


def test_attention_dense_masked_brute_force():
    rng = np.random.default_rng(8)
    cu = np.array([0, 5, 6, 13])
    n, heads, dh = 13, 2, 4
    q, k, v = (rng.standard_normal((n, heads * dh)) * 2 for _ in range(3))
    np.testing.assert_allclose(O.attention(q, k, v, cu, heads), _dense_masked_attention(q, k, v, cu, heads),
                               rtol=1e-12, atol=1e-12)


def test_attention_packed_equals_each_image_alone():
    rng = np.random.default_rng(9)
    lens = [7, 1, 12, 4]
    cu = np.concatenate([[0], np.cumsum(lens)])
    n = cu[-1]
    q, k, v = (rng.standard_normal((n, 64)) for _ in range(3))
    packed = O.attention(q, k, v, cu, 2)
    for i in range(len(lens)):
        a, b = cu[i], cu[i + 1]
        alone = O.attention(q[a:b], k[a:b], v[a:b], np.array([0, b - a]), 2)
        np.testing.assert_allclose(packed[a:b], alone, rtol=1e-13, atol=1e-13)


def test_attention_special_cases():
    rng = np.random.default_rng(10)
    # single-patch image: output = v
    q, k, v = (rng.standard_normal((1, 64)) for _ in range(3))
    np.testing.assert_allclose(O.attention(q, k, v, np.array([0, 1]), 1), v, rtol=1e-14)
    # equal keys: uniform weights -> mean of v
    q = rng.standard_normal((6, 64))
    k = np.tile(rng.standard_normal((1, 64)), (6, 1))
    v = rng.standard_normal((6, 64))
    np.testing.assert_allclose(O.attention(q, k, v, np.array([0, 6]), 1), np.tile(v.mean(0), (6, 1)), rtol=1e-12)
    # permuting the patches permutes the outputs
    q, k, v = (rng.standard_normal((9, 64)) for _ in range(3))
    perm = rng.permutation(9)
    a = O.attention(q, k, v, np.array([0, 9]), 2)
    b = O.attention(q[perm], k[perm], v[perm], np.array([0, 9]), 2)
    np.testing.assert_allclose(b, a[perm], rtol=1e-12, atol=1e-12)


def test_attention_scale_is_inverse_sqrt_head_dim():
    # two keys with logits differing by exactly sqrt(dh) * ln(3) give weights 3:1
    dh = 64
    q = np.zeros((1, dh)); q[0, 0] = 1.0
    k = np.zeros((2, dh)); k[0, 0] = math.sqrt(dh) * math.log(3.0)
    v = np.zeros((2, dh)); v[0, 1] = 1.0; v[1, 2] = 1.0
    # query 0 attends over both keys (one image of 2 patches, query row duplicated)
    qq = np.vstack([q, q])
    out = O.attention(qq, k, v, np.array([0, 2]), 1)
    np.testing.assert_allclose(out[0, 1], 0.75, rtol=1e-12)
    np.testing.assert_allclose(out[0, 2], 0.25, rtol=1e-12)


# ---------------------------------------------------------------- MLP
def test_swiglu_scalar_example():
    y = np.array([[1.0, -2.0]])
    wg = np.array([[0.5, 0.25]])      # gate = 0.0
    wu = np.array([[1.0, 1.0]])       # up = -1
    wd = np.array([[2.0], [3.0]])
    np.testing.assert_allclose(O.swiglu_mlp(y, wg, wu, wd), [[0.0, 0.0]], atol=1e-15)
    wg = np.array([[1.0, 0.0]])       # gate = 1 -> silu = 1/(1+e^-1)
    s = 1.0 / (1.0 + math.exp(-1.0))
    np.testing.assert_allclose(O.swiglu_mlp(y, wg, wu, wd), [[2.0 * s * -1.0, 3.0 * s * -1.0]], rtol=1e-14)


def test_swiglu_zero_down_is_zero():
    rng = np.random.default_rng(1)
    y = rng.standard_normal((4, 8))
    assert np.all(O.swiglu_mlp(y, rng.standard_normal((16, 8)), rng.standard_normal((16, 8)), np.zeros((8, 16))) == 0)


# ---------------------------------------------------------------- merge
@pytest.mark.parametrize("hw", [[(28, 56)], [(56, 28)], [(56, 84), (28, 28)]])
def test_identity_merger_gathers_windows(hw):
    p, d = 14, 3
    m = O.plan_maps(hw, p, 2)
    n = m["n_patches"]
    h = np.arange(n * d, dtype=np.float64).reshape(n, d)
    out = O.merge_project(h, m["merge_src"], np.eye(4 * d))
    t = 0
    base = 0
    for (hh, ww) in hw:
        hp, wp = hh // p, ww // p
        for big_r in range(hp // 2):
            for big_c in range(wp // 2):
                want = np.concatenate([
                    h[base + (2 * big_r) * wp + 2 * big_c], h[base + (2 * big_r) * wp + 2 * big_c + 1],
                    h[base + (2 * big_r + 1) * wp + 2 * big_c], h[base + (2 * big_r + 1) * wp + 2 * big_c + 1]])
                np.testing.assert_array_equal(out[t], want)
                t += 1
        base += hp * wp
    assert t == m["out_rows"]


# ---------------------------------------------------------------- whole tower
def _tiny_weights(rng, d, f, p, layers, out_dim, zero_blocks=False):
    w = {"patch_w": rng.standard_normal((d, 3, p, p)) * 0.1, "ln_pre": 1 + 0.1 * rng.standard_normal(d), "layers": []}
    for _ in range(layers):
        w["layers"].append({
            "attn_norm": 1 + 0.1 * rng.standard_normal(d),
            "wq": rng.standard_normal((d, d)) * 0.2, "wk": rng.standard_normal((d, d)) * 0.2,
            "wv": rng.standard_normal((d, d)) * 0.2,
            "wo": np.zeros((d, d)) if zero_blocks else rng.standard_normal((d, d)) * 0.2,
            "ffn_norm": 1 + 0.1 * rng.standard_normal(d),
            "w_gate": rng.standard_normal((f, d)) * 0.2, "w_up": rng.standard_normal((f, d)) * 0.2,
            "w_down": np.zeros((d, f)) if zero_blocks else rng.standard_normal((d, f)) * 0.2,
        })
    w["merge_w"] = rng.standard_normal((out_dim, 4 * d)) * 0.1
    return w


def test_tower_zero_blocks_reduce_to_embed_norm_merge():
    rng = np.random.default_rng(12)
    cfg = O.TowerConfig(patch=4, hidden=16, heads=2, mlp=24, layers=2, merge=2, out_dim=20)
    hw = [(16, 8), (8, 8)]
    w = _tiny_weights(rng, 16, 24, 4, 2, 20, zero_blocks=True)
    pix = rng.standard_normal(sum(3 * h * ww for h, ww in hw))
    out = O.tower_forward(pix, hw, w, cfg)["out"]
    # independent composition: direct conv -> explicit RMSNorm -> explicit window gather -> matmul
    x = np.concatenate([_direct_conv(pix[:3 * 128].reshape(3, 16, 8), w["patch_w"], 4),
                        _direct_conv(pix[3 * 128:].reshape(3, 8, 8), w["patch_w"], 4)])
    hn = x / np.sqrt((x ** 2).mean(1, keepdims=True) + 1e-5) * w["ln_pre"]
    rows = []
    for base, (hp, wp) in [(0, (4, 2)), (8, (2, 2))]:
        for r in range(hp // 2):
            for c in range(wp // 2):
                g = [base + (2 * r + a) * wp + 2 * c + b for a in (0, 1) for b in (0, 1)]
                rows.append(np.concatenate([hn[i] for i in g]))
    np.testing.assert_allclose(out, np.array(rows) @ w["merge_w"].T, rtol=1e-11, atol=1e-11)


def test_tower_brute_force_tiny():
    """One block computed step by step with the loop-based helpers above."""
    rng = np.random.default_rng(13)
    d, f, p, heads = 8, 12, 2, 2
    cfg = O.TowerConfig(patch=p, hidden=d, heads=heads, mlp=f, layers=1, merge=2, out_dim=6, rope_theta=100.0)
    hw = [(4, 8), (4, 4)]
    w = _tiny_weights(rng, d, f, p, 1, 6)
    pix = rng.standard_normal(3 * 32 + 3 * 16)
    got = O.tower_forward(pix, hw, w, cfg)["out"]
    x = np.concatenate([_direct_conv(pix[:96].reshape(3, 4, 8), w["patch_w"], p),
                        _direct_conv(pix[96:].reshape(3, 4, 4), w["patch_w"], p)])
    rc = [(r, c) for r in range(2) for c in range(4)] + [(r, c) for r in range(2) for c in range(2)]

    def norm(a, g):
        return a / np.sqrt((a ** 2).mean(1, keepdims=True) + 1e-5) * g

    h = norm(x, w["ln_pre"])
    lw = w["layers"][0]
    y = norm(h, lw["attn_norm"])
    q = y @ lw["wq"].T
    k = y @ lw["wk"].T
    v = y @ lw["wv"].T
    q = np.array([_rope_complex(q[i], rc[i][0], rc[i][1], heads, 100.0) for i in range(12)])
    k = np.array([_rope_complex(k[i], rc[i][0], rc[i][1], heads, 100.0) for i in range(12)])
    a = _dense_masked_attention(q, k, v, [0, 8, 12], heads)
    h = h + a @ lw["wo"].T
    y = norm(h, lw["ffn_norm"])
    gt = y @ lw["w_gate"].T
    h = h + ((gt / (1 + np.exp(-gt))) * (y @ lw["w_up"].T)) @ lw["w_down"].T
    rows = []
    for base, (hp, wp) in [(0, (2, 4)), (8, (2, 2))]:
        for r in range(hp // 2):
            for c in range(wp // 2):
                g = [base + (2 * r + a_) * wp + 2 * c + b_ for a_ in (0, 1) for b_ in (0, 1)]
                rows.append(np.concatenate([h[i] for i in g]))
    np.testing.assert_allclose(got, np.array(rows) @ w["merge_w"].T, rtol=1e-10, atol=1e-10)


def test_tower_packing_order_invariance():
    rng = np.random.default_rng(14)
    cfg = O.TowerConfig(patch=4, hidden=16, heads=2, mlp=24, layers=2, merge=2, out_dim=10)
    hw = [(16, 8), (8, 24), (8, 8)]
    w = _tiny_weights(rng, 16, 24, 4, 2, 10)
    imgs = [rng.standard_normal(3 * h * ww) for h, ww in hw]
    a = O.tower_forward(np.concatenate(imgs), hw, w, cfg)["out"]
    order = [2, 0, 1]
    b = O.tower_forward(np.concatenate([imgs[i] for i in order]), [hw[i] for i in order], w, cfg)["out"]
    counts = [(h // 8) * (ww // 8) for h, ww in hw]
    starts = np.concatenate([[0], np.cumsum(counts)])
    pieces_b = np.split(b, np.cumsum([counts[i] for i in order])[:-1])
    for j, i in enumerate(order):
        np.testing.assert_allclose(pieces_b[j], a[starts[i]:starts[i + 1]], rtol=1e-12, atol=1e-12)


def test_tower_no_merge_returns_patch_states():
    rng = np.random.default_rng(15)
    cfg = O.TowerConfig(patch=4, hidden=16, heads=2, mlp=24, layers=1, merge=1)
    hw = [(8, 12)]
    w = _tiny_weights(rng, 16, 24, 4, 1, 10)
    res = O.tower_forward(rng.standard_normal(3 * 96), hw, w, cfg)
    assert res["out"].shape == (6, 16)
    np.testing.assert_array_equal(res["out"], res["tower_out"])


def test_masked_scatter_hand_example():
    """Placeholder id 10 ("Mistral 3", Mistral3Model table): the k-th
    placeholder in sequence order takes image row k; other rows unchanged."""
    ids = np.array([1, 10, 5, 10, 10, 2])
    img = np.array([[1.0, 1.5], [2.0, 2.5], [3.0, 3.5]])
    txt = np.arange(12, dtype=np.float64).reshape(6, 2) + 100
    out, ok = O.masked_scatter(ids, img, txt, 10)
    want = txt.copy()
    want[1], want[3], want[4] = img[0], img[1], img[2]
    assert ok and np.array_equal(out, want)
    assert np.array_equal(txt, np.arange(12, dtype=np.float64).reshape(6, 2) + 100)  # input untouched


def test_masked_scatter_count_mismatch_fills_what_fits():
    ids = np.array([10, 3, 10])
    img = np.array([[7.0], [8.0], [9.0]])
    txt = np.zeros((3, 1))
    out, ok = O.masked_scatter(ids, img, txt, 10)
    assert not ok and out[:, 0].tolist() == [7.0, 0.0, 8.0]
    out, ok = O.masked_scatter(np.array([10, 10, 10, 10]), img, np.zeros((4, 1)), 10)
    assert not ok and out[:, 0].tolist() == [7.0, 8.0, 9.0, 0.0]


# ------------------------------------------------------- preprocessing (uint8)
def test_resize_target_page_sizes():
    """"Mistral 3" processor table: longest_edge 1540, patch 14 (merge 2 ->
    28-pixel grid); a 4096x4096 photo becomes 1540x1540 = 110x110 patches.
    "Pixtral-12B-2409": a 1024x1024 tile with patch 16 stays 1024x1024."""
    assert O.resize_target(4096, 4096, 1540, 28) == (1540, 1540)
    assert O.resize_target(1024, 1024, 1024, 16) == (1024, 1024)
    # already on the grid and within the edge: unchanged, never enlarged
    for h, w in [(28, 28), (224, 1540), (1540, 56), (812, 644)]:
        assert O.resize_target(h, w, 1540, 28) == (h, w)
    # a small off-grid image is only rounded up to the grid
    assert O.resize_target(300, 200, 1540, 28) == (308, 224)
    # wide photo: 1000 x 4000 -> fit 385 x 1540 -> grid 392 x 1540
    assert O.resize_target(1000, 4000, 1540, 28) == (392, 1540)


def test_resize_target_brute_force():
    """Search-based restatement: the fitted side is the largest integer s >= 1
    with s * max(H, W) <= side * L (if max(H, W) > L, else the side itself),
    then the smallest grid multiple >= s, capped at the largest grid multiple
    <= L."""
    rng = np.random.default_rng(21)
    for _ in range(400):
        grid = int(rng.integers(1, 40))
        L = int(rng.integers(grid, 300))
        h, w = (int(v) for v in rng.integers(1, 700, size=2))
        m = max(h, w)
        want = []
        for side in (h, w):
            s = side
            if m > L:
                s = 1
                while (s + 1) * m <= side * L:
                    s += 1
            t = grid
            while t < s:
                t += grid
            cap = grid
            while cap + grid <= L:
                cap += grid
            want.append(min(t, cap))
        got = O.resize_target(h, w, L, grid)
        assert got == tuple(want), (h, w, L, grid)
        assert max(got) <= L and got[0] % grid == 0 and got[1] % grid == 0


@pytest.mark.parametrize("src,dst", [
    ((7, 5), (7, 5)), ((8, 12), (4, 6)), ((9, 13), (28, 28)), ((40, 31), (14, 28)),
    ((1, 6), (5, 3)), ((6, 1), (2, 9)), ((33, 47), (1, 1)), ((4096 // 64, 4096 // 64), (1540 // 64, 1540 // 64)),
])
def test_bilinear_matches_library_interpolate(src, dst):
    """Half-pixel-centre bilinear without antialiasing is torch's
    interpolate(mode='bilinear', align_corners=False) in float64."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(22)
    img = rng.integers(0, 256, size=src + (3,), dtype=np.uint8)
    got = O.preprocess_image(img, dst[0], dst[1], mean=(0, 0, 0), std=(1 / 255, 1 / 255, 1 / 255))
    t = torch.from_numpy(img.astype(np.float64)).permute(2, 0, 1)[None]
    want = torch.nn.functional.interpolate(t, size=dst, mode="bilinear", align_corners=False,
                                           antialias=False)[0].numpy()
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-9)


def test_bilinear_closed_forms():
    rng = np.random.default_rng(23)
    unit = dict(mean=(0, 0, 0), std=(1 / 255, 1 / 255, 1 / 255))  # raw values out
    img = rng.integers(0, 256, size=(10, 14, 3), dtype=np.uint8)
    # same size: an exact copy
    np.testing.assert_array_equal(O.preprocess_image(img, 10, 14, **unit),
                                  img.transpose(2, 0, 1).astype(np.float64))
    # halving each side: every output is the mean of its 2x2 source block
    half = O.preprocess_image(img, 5, 7, **unit)
    blocks = img.astype(np.float64).reshape(5, 2, 7, 2, 3).mean(axis=(1, 3)).transpose(2, 0, 1)
    np.testing.assert_allclose(half, blocks, rtol=0, atol=1e-12)
    # a constant image stays constant at any size
    flat = np.full((9, 6, 3), 77, dtype=np.uint8)
    np.testing.assert_allclose(O.preprocess_image(flat, 13, 4, **unit), 77.0, rtol=0, atol=1e-12)
    # doubling a linear ramp v = 3y + 2x: output t sits at source t/2 - 1/4,
    # so interior outputs are 3(ty/2 - 1/4) + 2(tx/2 - 1/4); the clamped
    # border rows/columns take the edge pixel's coordinate
    ramp = np.zeros((6, 8, 3), dtype=np.uint8)
    yy, xx = np.mgrid[0:6, 0:8]
    ramp[..., 0] = 3 * yy + 2 * xx
    up = O.preprocess_image(ramp, 12, 16, **unit)[0]
    for ty in range(12):
        for tx in range(16):
            sy = min(max(ty / 2 - 0.25, 0.0), 5.0)
            sx = min(max(tx / 2 - 0.25, 0.0), 7.0)
            assert abs(up[ty, tx] - (3 * sy + 2 * sx)) < 1e-12


def test_normalisation_constants_and_channel_order():
    """x/255 then (x - mean_c)/std_c with the processor table's values;
    channel 0 of the output is the image's first (R) component."""
    mean = (0.48145466, 0.4578275, 0.40821073)
    std = (0.26862954, 0.26130258, 0.27577711)
    img = np.zeros((4, 4, 3), dtype=np.uint8)
    img[..., 0] = 255
    img[..., 2] = 51
    out = O.preprocess_image(img, 4, 4)
    np.testing.assert_allclose(out[0], (1.0 - mean[0]) / std[0], rtol=1e-15)
    np.testing.assert_allclose(out[1], -mean[1] / std[1], rtol=1e-15)
    np.testing.assert_allclose(out[2], (0.2 - mean[2]) / std[2], rtol=1e-14)


def test_preprocess_pixel_spot_values_agree_with_planes():
    rng = np.random.default_rng(24)
    img = rng.integers(0, 256, size=(37, 23, 3), dtype=np.uint8)
    full = O.preprocess_image(img, 56, 28)
    for c, y, x in [(0, 0, 0), (1, 55, 27), (2, 17, 9), (0, 31, 20), (1, 1, 26)]:
        assert abs(O.preprocess_pixel(img, 56, 28, c, y, x) - full[c, y, x]) < 1e-12


def test_preprocess_batch_layout():
    rng = np.random.default_rng(25)
    ims = [rng.integers(0, 256, size=(50, 90, 3), dtype=np.uint8),
           rng.integers(0, 256, size=(30, 20, 3), dtype=np.uint8)]
    flat, hw = O.preprocess_batch(ims, 56, 28)
    # 50x90 fits as 31x56, then both sides round up to 56; 30x20 is within
    # the edge and rounds up to 56x28
    assert hw == [(56, 56), (56, 28)]
    assert flat.shape == (3 * 56 * 56 + 3 * 56 * 28,)
    np.testing.assert_array_equal(flat[3 * 56 * 56:].reshape(3, 56, 28), O.preprocess_image(ims[1], 56, 28))


# ------------------------------------------------------------- Pixtral tiles
def test_tile_layout_page_example():
    """"Pixtral-12B-2409", VISION TOKENS: a 4096x4096 image is a 4x4 grid of
    1024x1024 tiles = 16 tiles = 65,536 patches of 16x16."""
    rh, rw, rows, cols = O.tile_layout(4096, 4096, 1024, 16, 16)
    assert (rh, rw, rows, cols) == (4096, 4096, 4, 4)
    assert rows * cols * (1024 // 16) ** 2 == 65536
    # a lower cap scales the image down: 4 tiles -> 2048^2, 1 tile -> 1024^2
    assert O.tile_layout(4096, 4096, 1024, 16, 4) == (2048, 2048, 2, 2)
    assert O.tile_layout(4096, 4096, 1024, 16, 1) == (1024, 1024, 1, 1)
    # no scaling when the grid fits; the sides round up to the patch grid
    assert O.tile_layout(1000, 3000, 1024, 16, 16) == (1008, 3008, 1, 3)
    assert O.tile_layout(300, 200, 1024, 16, 16) == (304, 208, 1, 1)
    # 3 tiles allowed for a 4096^2 image: the best grid is 1x3 / 3x1 / 1x1...
    # -> min(1024/4096, 3072/4096) = 1/4 for 1x3, so 1024^2, one tile
    assert O.tile_layout(4096, 4096, 1024, 16, 3) == (1024, 1024, 1, 1)
    # a wide image with 3 tiles: 1x3 grid, s = 3072/6000
    rh, rw, rows, cols = O.tile_layout(1500, 6000, 1024, 16, 3)
    assert (rows, cols) == (1, 3) and rw == 3072 and rh == 768


def test_tile_layout_brute_force():
    """s* = the largest s in {1} u {k T / H} u {k T / W} (the points where a
    grid side changes) with ceil(sH/T) * ceil(sW/T) <= M and s <= 1."""
    from fractions import Fraction
    rng = np.random.default_rng(26)
    for _ in range(300):
        g = int(rng.choice([1, 2, 4, 8]))
        T = g * int(rng.integers(1, 6))
        M = int(rng.integers(1, 10))
        h, w = (int(v) for v in rng.integers(1, 120, size=2))
        cands = {Fraction(1)} | {Fraction(k * T, h) for k in range(1, 40)} | {Fraction(k * T, w) for k in range(1, 40)}
        ok = [s for s in cands if s <= 1 and math.ceil(s * h / T) * math.ceil(s * w / T) <= M]
        s = max(ok)
        rh = -(-max(1, math.floor(s * h)) // g) * g
        rw = -(-max(1, math.floor(s * w)) // g) * g
        got = O.tile_layout(h, w, T, g, M)
        assert got == (rh, rw, -(-rh // T), -(-rw // T)), (h, w, T, g, M)
        assert got[2] * got[3] <= M


def test_tiles_reassemble_the_resized_image():
    rng = np.random.default_rng(27)
    img = rng.integers(0, 256, size=(70, 45, 3), dtype=np.uint8)
    tiles, hw = O.tile_image(img, 32, 8, 6)
    rh, rw, rows, cols = O.tile_layout(70, 45, 32, 8, 6)
    assert len(tiles) == rows * cols and all(0 < a <= 32 and 0 < b <= 32 and a % 8 == 0 and b % 8 == 0
                                             for a, b in hw)
    full = O.preprocess_image(img, rh, rw)
    rebuilt = np.concatenate([np.concatenate(tiles[r * cols:(r + 1) * cols], axis=2) for r in range(rows)], axis=1)
    np.testing.assert_array_equal(rebuilt, full)


def test_tiles_without_scaling_are_normalised_source_crops():
    """When the source already sits on the tile grid no resampling happens:
    each tile is the normalised crop of the source."""
    rng = np.random.default_rng(28)
    img = rng.integers(0, 256, size=(64, 96, 3), dtype=np.uint8)
    tiles, hw = O.tile_image(img, 32, 16, 6)
    assert hw == [(32, 32)] * 6
    mean = np.asarray(O.PROCESSOR_MEAN)[:, None, None]
    std = np.asarray(O.PROCESSOR_STD)[:, None, None]
    crop = img[32:64, 64:96].transpose(2, 0, 1).astype(np.float64)
    np.testing.assert_allclose(tiles[5], (crop / 255.0 - mean) / std, rtol=0, atol=1e-12)


# ------------------------------------------------------- embeddings cache key
def test_splitmix64_published_outputs():
    """SplitMix64 from state 0: state advances by 0x9E3779B97F4A7C15 and each
    output is mix(state); the generator's first three outputs are the
    published 0xe220a8397b1dcdaf, 0x6e789e6aa1b965f4, 0x06c45d188009454f."""
    g = 0x9E3779B97F4A7C15
    want = [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]
    got = [O.splitmix64_mix((k + 1) * g & ((1 << 64) - 1)) for k in range(3)]
    assert got == want


def test_image_key_properties():
    rng = np.random.default_rng(29)
    img = rng.integers(0, 256, size=(5, 7, 3), dtype=np.uint8)
    k = O.image_key(img)
    assert k == O.image_key(img.copy()) and k[0] != k[1]
    # one changed byte, two swapped words, or the same bytes as another shape
    # give other keys
    b = img.copy()
    b[4, 6, 2] ^= 1
    assert O.image_key(b) != k
    flat = img.reshape(-1).copy()
    flat[0:8], flat[8:16] = img.reshape(-1)[8:16], img.reshape(-1)[0:8]
    if not np.array_equal(flat, img.reshape(-1)):
        assert O.image_key(flat.reshape(5, 7, 3)) != k
    assert O.image_key(img.reshape(7, 5, 3)) != k
    # the zero padding of the last word: 1 x 1 image = one word of 3 bytes
    one = np.array([[[1, 2, 3]]], dtype=np.uint8)
    word = 1 | (2 << 8) | (3 << 16)
    want0 = O.splitmix64_mix((O.splitmix64_mix(word + O.KEY_G[0]) + O.splitmix64_mix((1 << 32 | 1) ^ O.KEY_G[0]))
                             & ((1 << 64) - 1))
    assert O.image_key(one)[0] == want0


# -------------------------------------------------------------- fp8 variant
def test_e4m3_round_table_and_ties():
    """OCP e4m3: 448 is the largest normal, 2^-6 the smallest normal, 2^-9
    the subnormal step; halfway cases go to the even mantissa."""
    cases = {1.0: 1.0, 1.0625: 1.0, 1.1875: 1.25, 448.0: 448.0, 300.0: 288.0, 2.0 ** -6: 2.0 ** -6,
             2.0 ** -10: 0.0, 1.5 * 2.0 ** -10: 2.0 ** -9, 3 * 2.0 ** -10: 2.0 ** -8, -17.0: -16.0,
             240.0: 240.0, 250.0: 256.0, 0.0: 0.0}
    for v, want in cases.items():
        assert float(O.e4m3_round(np.array([v]))[0]) == want, v


def test_e4m3_round_matches_library_cast():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(30)
    v = np.concatenate([rng.standard_normal(20000) * s for s in (1e-3, 0.1, 1.0, 30.0, 120.0)])
    v = v[np.abs(v) < 448].astype(np.float32).astype(np.float64)
    want = torch.from_numpy(v).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.e4m3_round(v), want)


def test_mx_e4m3_block_scale_rule():
    rng = np.random.default_rng(31)
    x = rng.standard_normal((5, 96)) * np.exp2(rng.integers(-20, 20, size=(5, 1)))
    q = O.mx_e4m3(x)
    for r in range(5):
        for b in range(3):
            blk, qb = x[r, 32 * b:32 * b + 32], q[r, 32 * b:32 * b + 32]
            X = math.floor(math.log2(np.max(np.abs(blk)))) - 7
            scaled = np.max(np.abs(blk)) * 2.0 ** -X
            assert 128 <= scaled < 256
            # every value is an e4m3 value times 2^X, within half a step
            np.testing.assert_array_equal(qb, O.e4m3_round(blk * 2.0 ** -X) * 2.0 ** X)
            assert np.all(np.abs(qb - blk) <= np.maximum(2.0 ** (np.floor(np.log2(np.abs(blk) + 1e-300)) - 4),
                                                          2.0 ** (X - 10)) + 1e-300)
    # an all-zero block stays zero; a block of powers of two is exact
    z = np.zeros((1, 32))
    assert np.array_equal(O.mx_e4m3(z), z)
    p2 = np.exp2(np.arange(-8, 24, dtype=np.float64))[None, :] * -1.0
    np.testing.assert_array_equal(O.mx_e4m3(p2)[0, 23:], p2[0, 23:])


def test_fp8_tower_reduces_to_exact_tower_on_e4m3_values():
    """When every operand of the four linear maps is already an e4m3 value
    times its block scale, the fp8 variant changes nothing: weights and
    activations that quantise to themselves (zero blocks make every block
    trivially exact)."""
    rng = np.random.default_rng(32)
    cfg = O.TowerConfig(patch=4, hidden=32, heads=2, mlp=64, layers=1, merge=1)
    hw = [(8, 8)]
    w = _tiny_weights(rng, 32, 64, 4, 1, 10)
    for k in ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down"):
        w["layers"][0][k] = np.zeros_like(w["layers"][0][k])
    px = rng.standard_normal(3 * 64)
    a = O.tower_forward(px, hw, w, cfg)["out"]
    b = O.tower_forward(px, hw, w, cfg, fp8=True)["out"]
    np.testing.assert_array_equal(a, b)
    # with real weights the variant differs (a few e4m3 steps at the worst
    # element of this small tower)
    w2 = _tiny_weights(rng, 32, 64, 4, 1, 10)
    a = O.tower_forward(px, hw, w2, cfg)["out"]
    b = O.tower_forward(px, hw, w2, cfg, fp8=True)["out"]
    rel = np.max(np.abs(a - b)) / np.sqrt(np.mean(a * a))
    assert 1e-4 < rel < 0.5


# ---- the fp8 variant's quantisation points, step by step, against an
# independent quantiser: the nearest of the 254 finite OCP E4M3FN code values
# (decoded from the bit layout: sign, 4 exponent bits with bias 7, 3 mantissa
# bits, subnormals at exponent 0, S.1111.111 = NaN), ties to the even code,
# with the block exponent X found by search (the unique X with
# 128 <= max|block| * 2^-X < 256).
def _e4m3_code_values():
    vals, even = [], []
    for b in range(256):
        s, e, m = b >> 7, (b >> 3) & 15, b & 7
        if e == 15 and m == 7:
            continue                                   # NaN codes
        mag = m * 2.0 ** -9 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
        vals.append(-mag if s else mag)
        even.append(m % 2 == 0)
    return np.array(vals), np.array(even)


_E4M3_VALS, _E4M3_EVEN = _e4m3_code_values()


def _brute_e4m3_block(blk):
    amax = float(np.max(np.abs(blk)))
    if amax == 0.0:
        return np.zeros_like(blk)
    X = next(x for x in range(-150, 151) if 128.0 <= amax * 2.0 ** -x < 256.0)
    X = min(max(X, -120), 120)
    out = np.empty_like(blk)
    for i, v in enumerate(blk * 2.0 ** -X):
        d = np.abs(_E4M3_VALS - v)
        cand = np.flatnonzero(d == d.min())
        pick = [c for c in cand if _E4M3_EVEN[c]] or list(cand)
        out[i] = _E4M3_VALS[pick[0]] * 2.0 ** X
    return out


def _brute_mx(x, axis=-1):
    """Block-scaled e4m3 copy of x, blocks of 32 along `axis`."""
    x = np.moveaxis(np.asarray(x, np.float64), axis, -1)
    out = np.empty_like(x)
    flat, fo = x.reshape(-1, x.shape[-1]), out.reshape(-1, x.shape[-1])
    for r in range(flat.shape[0]):
        for b in range(0, flat.shape[1], 32):
            fo[r, b:b + 32] = _brute_e4m3_block(flat[r, b:b + 32])
    return np.moveaxis(out, -1, axis)


def test_brute_e4m3_quantiser_agrees_with_library_cast():
    """The brute-force quantiser itself, on values in one binade of scale:
    with X = 0 forced (block max in [128, 256)) its values equal torch's
    float8_e4m3fn cast (round to nearest even)."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(33)
    blk = rng.uniform(-255, 255, size=32)
    blk[0] = 200.0
    want = torch.from_numpy(blk).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(_brute_e4m3_block(blk), want)


def _fp8_tower_by_steps(px, hw, w, cfg, mistake=None):
    """The fp8 variant written out step by step: the four linear maps of
    every block take both operands through the block quantiser along their
    contraction axis -- (norm output, wq, wk, wv), (attention output, wo),
    (ffn norm output, w_gate, w_up), (silu(gate) * up, w_down) -- and nothing
    else is quantised.  Returns the residual after each attention and each
    block, and the output.  `mistake` plants one error (to show the pin
    fails)."""
    def qa(a):                     # an activation [rows][K]
        return _brute_mx(a, axis=1)

    def qw(m):                     # a weight [out][K]
        return _brute_mx(m, axis=0 if mistake == "weight_axis" else 1)

    def norm(x, g):
        return x / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + cfg.rms_eps) * g

    maps = O.plan_maps(hw, cfg.patch, cfg.merge)
    h = norm(O.patch_embed(px, hw, w["patch_w"], cfg.patch), w["ln_pre"])
    attn_out, block_out = [], []
    for lw in w["layers"]:
        y = norm(h, lw["attn_norm"])
        y = y if mistake == "skip_norm_out" else qa(y)
        q = O.rope_2d(y @ qw(lw["wq"]).T, maps["patch_rc"], cfg.heads, cfg.rope_theta)
        k = O.rope_2d(y @ qw(lw["wk"]).T, maps["patch_rc"], cfg.heads, cfg.rope_theta)
        v = y @ qw(lw["wv"]).T
        a = O.attention(q, k, v, maps["cu_seqlens"], cfg.heads)
        a = a if mistake == "skip_attn_out" else qa(a)
        h = h + a @ qw(lw["wo"]).T
        attn_out.append(h)
        y2 = qa(norm(h, lw["ffn_norm"]))
        g, u = y2 @ qw(lw["w_gate"]).T, y2 @ qw(lw["w_up"]).T
        hm = g / (1.0 + np.exp(-g)) * u
        hm = hm if mistake == "skip_hidden" else qa(hm)
        h = h + hm @ qw(lw["w_down"]).T
        if mistake == "quantise_residual":
            h = qa(h)
        block_out.append(h)
    out = O.merge_project(h, maps["merge_src"], w["merge_w"]) if cfg.merge == 2 else h
    return attn_out, block_out, out


def _col_err(got, want):
    """max over columns of max|got - want| / RMS of that column of want."""
    rms = np.sqrt(np.mean(want * want, axis=0))
    return float(np.max(np.max(np.abs(got - want), axis=0) / rms))


def test_fp8_tower_quantisation_points_step_by_step():
    """tower_forward(fp8=True) equals the step-by-step fp8 tower with the
    brute-force quantiser (two blocks, two images, merge 2): the residual
    after every attention and every block, column by column, and the output.
    Each planted placement mistake moves some column far beyond that
    agreement.  The odd features are 2^-16 of the even ones (ln_pre gain and
    the rows of wo and w_down that write them): a weight block taken along
    the output axis then spans both magnitudes and flushes the small rows
    into e4m3's subnormals, which the per-column comparison sees."""
    rng = np.random.default_rng(34)
    d, f = 64, 96
    cfg = O.TowerConfig(patch=4, hidden=d, heads=2, mlp=f, layers=2, merge=2, out_dim=24)
    hw = [(8, 8), (16, 8)]
    w = _tiny_weights(rng, d, f, 4, 2, 24)
    small = np.where(np.arange(d) % 2 == 1, 2.0 ** -16, 1.0)
    w["ln_pre"] = w["ln_pre"] * small
    for lw in w["layers"]:
        lw["wo"] = lw["wo"] * small[:, None]
        lw["w_down"] = lw["w_down"] * small[:, None]
    px = rng.standard_normal(sum(3 * a * b for a, b in hw))
    res = O.tower_forward(px, hw, w, cfg, collect=True, fp8=True)
    got = res["attn_out"] + res["block_out"] + [res["out"]]
    a_, b_, o_ = _fp8_tower_by_steps(px, hw, w, cfg)
    want = a_ + b_ + [o_]
    for g_, w_ in zip(got, want):
        assert _col_err(g_, w_) <= 1e-12
    exact = O.tower_forward(px, hw, w, cfg)["out"]
    assert _col_err(exact, o_) > 1e-3                    # the quantisation is really there
    for mistake in ("weight_axis", "skip_norm_out", "skip_attn_out", "skip_hidden", "quantise_residual"):
        a_, b_, o_ = _fp8_tower_by_steps(px, hw, w, cfg, mistake)
        worst = max(_col_err(g_, w_) for g_, w_ in zip(got, a_ + b_ + [o_]))
        assert worst > 1e-3, mistake


# ------------------------------------------------------ deeper projector
def test_gelu_values():
    """GELU(x) = x Phi(x): Phi(1) = 0.8413447460685429 and Phi(-1) =
    0.15865525393145705 (standard normal table values), GELU(0) = 0, and
    GELU(x) -> x, -> 0 far out on either side."""
    x = np.array([0.0, 1.0, -1.0, 40.0, -40.0])
    want = np.array([0.0, 0.8413447460685429, -0.15865525393145705, 40.0, 0.0])
    np.testing.assert_allclose(O.gelu(x), want, rtol=0, atol=1e-15)


def _deep_case(rng, d=16, sel=0, scale=1e6):
    """A tiny merged tower output h over two images, and projector weights
    that make the projector the ReLU of the normed patch at window offset
    `sel` (merge_w picks it, w1 = scale I, w2 = I / scale): GELU(scale m) /
    scale -> relu(m) as scale grows."""
    hw = [(16, 8), (8, 8)]
    maps = O.plan_maps(hw, 4, 2)
    h = rng.standard_normal((maps["n_patches"], d)) * 3.0
    merge_w = np.zeros((d, 4 * d))
    merge_w[:, sel * d:(sel + 1) * d] = np.eye(d)
    proj = {"norm": 1.0 + 0.1 * rng.standard_normal(d), "w1": scale * np.eye(d), "w2": np.eye(d) / scale}
    return h, maps, merge_w, proj


def test_deep_projector_reduces_to_relu_of_one_window_patch():
    rng = np.random.default_rng(40)
    for sel in range(4):
        h, maps, merge_w, proj = _deep_case(rng, sel=sel)
        out = O.deep_project(h, maps["merge_src"], merge_w, proj, 1e-5)
        # independent statement: the normed patch at window offset sel of
        # every merged token, then max(., 0)
        src = maps["merge_src"][:, sel]
        xs = h[src]
        y = xs / np.sqrt(np.mean(xs * xs, axis=1, keepdims=True) + 1e-5) * proj["norm"]
        np.testing.assert_allclose(out, np.maximum(y, 0.0), rtol=0, atol=1e-6)


def test_deep_projector_zero_weights_and_order():
    """w2 = 0 or w1 = 0 gives a zero output; GELU applied after w2 instead of
    between w1 and w2, or the norm left out, both move the output."""
    rng = np.random.default_rng(41)
    h, maps, merge_w, proj = _deep_case(rng, scale=1.0)
    proj["w1"] = rng.standard_normal(proj["w1"].shape)
    proj["w2"] = rng.standard_normal(proj["w2"].shape)
    for k in ("w1", "w2"):
        p0 = dict(proj)
        p0[k] = np.zeros_like(proj[k])
        assert np.array_equal(O.deep_project(h, maps["merge_src"], merge_w, p0, 1e-5), np.zeros((len(maps["merge_src"]), 16)))
    good = O.deep_project(h, maps["merge_src"], merge_w, proj, 1e-5)
    m = O.merge_project(O.rms_norm(h, proj["norm"], 1e-5), maps["merge_src"], merge_w)
    act_after = O.gelu(m @ proj["w1"].T @ proj["w2"].T)
    no_norm = O.gelu(O.merge_project(h, maps["merge_src"], merge_w) @ proj["w1"].T) @ proj["w2"].T
    for bad in (act_after, no_norm):
        assert np.max(np.abs(bad - good)) > 1e-2 * np.max(np.abs(good))


def test_tower_with_deep_projector_zero_blocks():
    """Zero Wo and Wd: the tower output is the deeper projector of
    ln_pre(patch embedding), with the weights as drawn."""
    from vlm_vision_encoder_amd import synth
    wl = synth.Workload("deep", patch=4, layers=1, merge=2, image_hw=((16, 8), (8, 8)), dtype="f32", hidden=16,
                        heads=1, mlp=32, out_dim=24, deep_projector=True)
    w = synth.oracle_weights(synth.make_weights(wl))
    w["layers"][0]["wo"] = np.zeros_like(w["layers"][0]["wo"])
    w["layers"][0]["w_down"] = np.zeros_like(w["layers"][0]["w_down"])
    px = np.random.default_rng(42).standard_normal(sum(3 * a * b for a, b in wl.image_hw))
    cfg = O.TowerConfig(patch=4, hidden=16, heads=1, mlp=32, layers=1, merge=2, out_dim=24, deep_projector=True)
    got = O.tower_forward(px, wl.image_hw, w, cfg)["out"]
    maps = O.plan_maps(wl.image_hw, 4, 2)
    x = np.concatenate([_direct_conv(px[:3 * 128].reshape(3, 16, 8), w["patch_w"], 4),
                        _direct_conv(px[3 * 128:].reshape(3, 8, 8), w["patch_w"], 4)])
    h0 = x / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + 1e-5) * w["ln_pre"]
    want = O.deep_project(h0, maps["merge_src"], w["merge_w"], w["proj"], 1e-5)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)
    assert got.shape == (maps["out_rows"], 24)
