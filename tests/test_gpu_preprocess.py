"""GPU parity of the uint8 input path (resize onto the patch grid + per-channel
normalisation) against the float64 oracle, through the C ABI.

Bar: the target sizes are integer work and bit-exact; the fp32 preprocessed
planes within 1e-4 * RMS of the oracle's; the tower output from uint8 images
within the tower's own bars (2e-2 * RMS bf16, 1e-4 * RMS fp32) of the oracle
run on the oracle's preprocessed pixels.  At the 1540x1540 size (a 4096x4096
photo) the planes are checked on sampled pixels the oracle computes one by
one, and the fused path must equal the two-pass path (preprocess, then the
float forward) bit for bit: both take the same fp32 samples.  The Pixtral
tile path (tiles of max_side, capped by max_num_tiles) is held to the same
bars: tile layouts bit-exact, the tower over the tiles vs the oracle on its
own tiles, and at 4096x4096 (16 tiles; 4 tiles under a cap of 4) sampled
pixels plus bit-equality with preprocess + cut + float forward.
Inputs: seeded uniform uint8 images (vlm_vision_encoder_amd.synth).
"""
import numpy as np
import pytest

from oracle import pv_oracle as O
from vlm_vision_encoder_amd import synth
from vlm_vision_encoder_amd import tower as T

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f32": 1e-4}
TOL_PLANES = 1e-4


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)


def err_over_rms(got, want):
    want = np.asarray(want, np.float64)
    got = np.asarray(got, np.float64)
    rms = float(np.sqrt(np.mean(want * want)))
    return float(np.max(np.abs(got - want)) / rms)


def upload_u8(images):
    torch = _torch()
    flat = np.concatenate([im.reshape(-1) for im in images])
    return torch.from_numpy(flat).cuda()


CASES = [
    # (source sizes, target sizes)
    ([(64, 64)], [(64, 64)]),                       # same size
    ([(128, 96)], [(64, 48)]),                      # exact halving
    ([(37, 53)], [(112, 56)]),                      # enlarging, off-grid source
    ([(301, 199)], [(84, 140)]),                    # shrinking by non-integer ratios
    ([(1, 7)], [(28, 28)]),                         # one source row
    ([(45, 1)], [(3, 5)]),                          # one source column
    ([(90, 70)], [(1, 1)]),                         # to a single pixel
    ([(50, 90), (30, 20), (7, 7)], [(56, 56), (56, 28), (28, 84)]),  # several images
]


@pytest.mark.parametrize("src,dst", CASES)
def test_preprocess_planes_match_oracle(src, dst):
    torch = _torch()
    say(f"preprocess {src} -> {dst}")
    images = synth.make_u8_images(src, seed=41)
    got = T.preprocess_u8(upload_u8(images), src, dst).cpu().numpy()
    torch.cuda.synchronize()
    want = np.concatenate([O.preprocess_image(im, h, w).reshape(-1) for im, (h, w) in zip(images, dst)])
    assert got.shape == want.shape
    e = err_over_rms(got, want)
    say(f"  planes: max-abs-err/RMS = {e:.3e} (max abs {np.max(np.abs(got - want)):.2e})")
    assert e <= TOL_PLANES


def test_preprocess_custom_mean_std():
    torch = _torch()
    say("preprocess with caller mean/std")
    src, dst = [(40, 60)], [(56, 84)]
    ms = (0.5, 0.25, 0.75, 0.125, 0.5, 2.0)
    images = synth.make_u8_images(src, seed=42)
    got = T.preprocess_u8(upload_u8(images), src, dst, mean_std=ms).cpu().numpy()
    torch.cuda.synchronize()
    want = O.preprocess_image(images[0], 56, 84, mean=ms[:3], std=ms[3:]).reshape(-1)
    assert err_over_rms(got, want) <= TOL_PLANES


def small_workload(dtype, merge=2, patch=14):
    return synth.Workload("u8-small", patch=patch, layers=2, merge=merge, image_hw=((28, 28),), dtype=dtype,
                          hidden=256, heads=4, mlp=512, out_dim=384)


@pytest.mark.parametrize("dtype,merge,patch", [("bf16", 2, 14), ("f32", 2, 14), ("bf16", 1, 16), ("f32", 1, 16)])
def test_forward_u8_matches_oracle(dtype, merge, patch):
    torch = _torch()
    max_side = 112
    src = [(100, 150), (61, 33), (300, 90), (20, 20)]
    say(f"forward_u8 {dtype} merge={merge} patch={patch} src={src} max_side={max_side}")
    wl = small_workload(dtype, merge, patch)
    w = synth.make_weights(wl)
    tower = T.Tower(T.config_for(wl, max_side=max_side), T.weights_to_device(w, dtype))
    images = synth.make_u8_images(src, seed=43)
    grid = patch * merge
    info, tgt = tower.plan_u8(src)
    assert tgt == [O.resize_target(h, w_, max_side, grid) for h, w_ in src]
    out = to_np(tower.forward_u8(upload_u8(images), src))
    torch.cuda.synchronize()
    px, hw = O.preprocess_batch(images, max_side, grid)
    assert [tuple(x) for x in hw] == tgt
    cfg = O.TowerConfig(patch=patch, hidden=wl.hidden, heads=wl.heads, mlp=wl.mlp, layers=wl.layers, merge=merge,
                        out_dim=wl.out_dim, rope_theta=wl.rope_theta, rms_eps=wl.rms_eps)
    want = O.tower_forward(px, hw, synth.oracle_weights(w), cfg)["out"]
    assert out.shape == want.shape == (info.out_rows, info.out_cols)
    e = err_over_rms(out, want)
    say(f"  out: max-abs-err/RMS = {e:.3e} (tol {TOL[dtype]})")
    assert e <= TOL[dtype]
    tower.close()


def to_np(t):
    return t.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_forward_u8_equals_two_pass(dtype):
    """Fused resize in the patch-embedding load == preprocess + float
    forward, bit for bit (small tower, several images)."""
    torch = _torch()
    say(f"forward_u8 vs two-pass {dtype}")
    wl = small_workload(dtype)
    tower = T.Tower(T.config_for(wl, max_side=224), T.weights_to_device(synth.make_weights(wl), dtype))
    src = [(500, 333), (100, 224), (17, 260)]
    images = upload_u8(synth.make_u8_images(src, seed=44))
    info, tgt = tower.plan_u8(src)
    a = tower.forward_u8(images, src).clone()
    px = T.preprocess_u8(images, src, tgt)
    b = tower.forward(px, tgt)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    tower.close()


def test_fullsize_4096_photo_to_1540():
    """The Mistral 3 processor size: a 4096x4096 photo -> 1540x1540, 24-layer
    bf16 tower.  Sampled planes against the oracle's per-pixel values; the
    fused forward equals the two-pass forward bit for bit."""
    torch = _torch()
    say("full size: 4096x4096 uint8 -> 1540x1540, 24 layers bf16")
    wl = synth.workload("ms31_1540")
    tower = T.Tower(T.config_for(wl, max_side=1540), T.weights_to_device(synth.make_weights(wl), "bf16"))
    src = [(4096, 4096)]
    host = synth.make_u8_images(src, seed=45)
    images = upload_u8(host)
    info, tgt = tower.plan_u8(src)
    assert tgt == [(1540, 1540)] and info.n_patches == 12100 and info.out_rows == 3025
    planes = T.preprocess_u8(images, src, tgt).cpu().numpy().reshape(3, 1540, 1540)
    rng = np.random.default_rng(46)
    picks = [(int(c), int(y), int(x)) for c, y, x in zip(rng.integers(0, 3, 400), rng.integers(0, 1540, 400),
                                                          rng.integers(0, 1540, 400))]
    picks += [(0, 0, 0), (1, 1539, 1539), (2, 0, 1539), (0, 1539, 0)]
    got = np.array([planes[c, y, x] for c, y, x in picks], np.float64)
    want = np.array([O.preprocess_pixel(host[0], 1540, 1540, c, y, x) for c, y, x in picks])
    e = err_over_rms(got, want)
    say(f"  sampled planes: max-abs-err/RMS = {e:.3e}")
    assert e <= TOL_PLANES
    a = tower.forward_u8(images, src).clone()
    b = tower.forward(torch.from_numpy(planes.reshape(-1)).cuda(), tgt)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    tower.close()


# ------------------------------------------------------------------- tiles
def tiles_from_planes(planes, layout, tile):
    """Cut the resized planes of each image into its tiles (row-major), as a
    flat fp32 tensor in the tower's input layout, plus the tile sizes."""
    torch = _torch()
    parts, hw, off = [], [], 0
    for rh, rw, rows, cols in layout:
        img = planes[off: off + 3 * rh * rw].view(3, rh, rw)
        off += 3 * rh * rw
        for a in range(rows):
            for b in range(cols):
                t = img[:, a * tile: min((a + 1) * tile, rh), b * tile: min((b + 1) * tile, rw)]
                parts.append(t.contiguous().view(-1))
                hw.append((t.shape[1], t.shape[2]))
    return torch.cat(parts), hw


TILE_CASES = [
    # dtype, patch, merge, tile, max_num_tiles, sources
    ("bf16", 16, 1, 64, 4, [(150, 100), (64, 64), (40, 200), (300, 300)]),
    ("f32", 16, 1, 64, 4, [(150, 100), (64, 64), (40, 200), (300, 300)]),
    ("bf16", 14, 2, 56, 3, [(200, 90), (56, 112), (13, 29)]),
    ("f32", 14, 2, 56, 3, [(200, 90), (56, 112), (13, 29)]),
]


@pytest.mark.parametrize("dtype,patch,merge,tile,cap,src", TILE_CASES)
def test_forward_tiles_u8_matches_oracle(dtype, patch, merge, tile, cap, src):
    torch = _torch()
    say(f"forward_tiles_u8 {dtype} patch={patch} merge={merge} tile={tile} max_num_tiles={cap} src={src}")
    wl = small_workload(dtype, merge, patch)
    w = synth.make_weights(wl)
    tower = T.Tower(T.config_for(wl, max_side=tile), T.weights_to_device(w, dtype))
    images = synth.make_u8_images(src, seed=47)
    info, layout = tower.plan_tiles_u8(src, cap)
    grid = patch * merge
    assert layout == [O.tile_layout(h, w_, tile, grid, cap) for h, w_ in src]
    out = to_np(tower.forward_tiles_u8(upload_u8(images), src, cap))
    torch.cuda.synchronize()
    px, hw, counts = O.tile_batch(images, tile, grid, cap)
    assert sum(counts) == info.n_images
    cfg = O.TowerConfig(patch=patch, hidden=wl.hidden, heads=wl.heads, mlp=wl.mlp, layers=wl.layers, merge=merge,
                        out_dim=wl.out_dim, rope_theta=wl.rope_theta, rms_eps=wl.rms_eps)
    want = O.tower_forward(px, hw, synth.oracle_weights(w), cfg)["out"]
    assert out.shape == want.shape
    e = err_over_rms(out, want)
    say(f"  out: max-abs-err/RMS = {e:.3e} (tol {TOL[dtype]}), {info.n_images} tiles")
    assert e <= TOL[dtype]
    tower.close()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_forward_tiles_u8_equals_two_pass(dtype):
    torch = _torch()
    say(f"forward_tiles_u8 vs two-pass {dtype}")
    wl = small_workload(dtype, merge=1, patch=16)
    tower = T.Tower(T.config_for(wl, max_side=64), T.weights_to_device(synth.make_weights(wl), dtype))
    src = [(500, 333), (100, 224), (17, 260)]
    images = upload_u8(synth.make_u8_images(src, seed=48))
    info, layout = tower.plan_tiles_u8(src, 6)
    a = tower.forward_tiles_u8(images, src, 6).clone()
    planes = T.preprocess_u8(images, src, [(l[0], l[1]) for l in layout])
    px, hw = tiles_from_planes(planes, layout, 64)
    b = tower.forward(px, hw)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    tower.close()


@pytest.mark.parametrize("cap,n_tiles", [(16, 16), (4, 4)])
def test_fullsize_pixtral_4096_photo_tiles(cap, n_tiles):
    """Pixtral-12B preset: a 4096x4096 photo as 1024^2 tiles (16 tiles =
    65,536 rows with max_num_tiles 16; 4 tiles of the 2048^2 resize with 4):
    sampled tile pixels vs the oracle's per-pixel values, and the fused path
    bit-equal to preprocess + cut + float forward."""
    torch = _torch()
    say(f"full size: Pixtral 4096x4096 uint8, max_num_tiles={cap}")
    wl = synth.workload("pixtral_tiles16")
    tower = T.Tower(T.preset("pixtral12b"), T.weights_to_device(synth.make_weights(wl), "bf16"))
    src = [(4096, 4096)]
    host = synth.make_u8_images(src, seed=49)
    images = upload_u8(host)
    info, layout = tower.plan_tiles_u8(src, cap)
    rh, rw, rows, cols = layout[0]
    assert rows * cols == n_tiles == info.n_images and info.out_rows == n_tiles * 4096
    planes = T.preprocess_u8(images, src, [(rh, rw)])
    px, hw = tiles_from_planes(planes, layout, 1024)
    cpu = planes.cpu().numpy().reshape(3, rh, rw)
    rng = np.random.default_rng(50)
    picks = [(int(c), int(y), int(x)) for c, y, x in zip(rng.integers(0, 3, 300), rng.integers(0, rh, 300),
                                                          rng.integers(0, rw, 300))]
    got = np.array([cpu[c, y, x] for c, y, x in picks])
    want = np.array([O.preprocess_pixel(host[0], rh, rw, c, y, x) for c, y, x in picks])
    assert err_over_rms(got, want) <= TOL_PLANES
    a = tower.forward_tiles_u8(images, src, cap).clone()
    b = tower.forward(px, hw)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    tower.close()
