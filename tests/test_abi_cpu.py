"""C ABI checks that need no GPU: the library loads, exports every function
include/pv_tower.h declares, validates arguments on the host before any HIP
call, and its host planner's index maps equal the oracle's exactly."""
import ctypes as C
import os
import re

import numpy as np
import pytest

from oracle import pv_oracle as O
from vlm_vision_encoder_amd import synth
from vlm_vision_encoder_amd import tower as T

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pv_tower.h")

pytestmark = pytest.mark.skipif(not os.path.exists(T.LIB_PATH), reason="libpv_tower.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pv_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_expected_entry_points():
    assert declared_functions() == sorted(T.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = T.load_library()
    for name in declared_functions():
        assert hasattr(lib, name), name


FAKE = 1 << 20  # an aligned, never-dereferenced stand-in for device pointers


def fake_weights(layers=2, merge=True):
    lw = [T.PvLayerWeights(*([FAKE] * 9)) for _ in range(layers)]
    arr = (T.PvLayerWeights * max(1, layers))(*lw)
    w = T.PvWeights(FAKE, FAKE, C.cast(arr, C.POINTER(T.PvLayerWeights)) if layers else None,
                    FAKE if merge else None)
    return w, arr


def create(cfg, layers_present=True):
    lib = T.load_library()
    w, arr = fake_weights(cfg.layers if layers_present else 0, cfg.merge == 2)
    h = C.c_void_p()
    st = lib.pv_tower_create(C.byref(cfg), C.byref(w), C.byref(h))
    return st, h, arr


@pytest.mark.parametrize("kw,status", [
    (dict(heads=8), -5),            # head_dim 128
    (dict(hidden=1000, heads=10), -5),
    (dict(mlp=1000), -5),
    (dict(mlp=(1 << 20) + 256), -5),
    (dict(out_dim=5000), -5),
    (dict(merge=3), -1),
    (dict(patch=0), -1),
    (dict(layers=-1), -1),
    (dict(dtype=7), -1),
    (dict(dtype=1), 0),
    (dict(max_side=10), -1),
    (dict(flags=4), -1),
    (dict(flags=2), 0),
    (dict(flags=1), 0),
    (dict(flags=8), 0),               # PV_FLAG_ROPE_INTERLEAVED
    (dict(flags=8, dtype=1), 0),
    (dict(flags=16), -1),             # unknown bit
    (dict(rope_theta=0.0), -1),
])
def test_create_validation(kw, status):
    dt = kw.pop("dtype", None)
    cfg = T.make_config(**{"layers": 2, **kw})
    if dt is not None:
        cfg.dtype = dt
    st, h, _ = create(cfg)
    assert st == status, T.load_library().pv_last_error()
    if st == 0:
        T.load_library().pv_tower_destroy(h)
    else:
        assert T.load_library().pv_last_error()


def test_create_null_pointers():
    lib = T.load_library()
    cfg = T.make_config(layers=1)
    h = C.c_void_p()
    assert lib.pv_tower_create(None, None, C.byref(h)) == -1
    w, arr = fake_weights(1)
    arr[0].wq = None
    assert lib.pv_tower_create(C.byref(cfg), C.byref(w), C.byref(h)) == -1
    assert b"null" in lib.pv_last_error()
    w, arr = fake_weights(1)
    arr[0].wo = FAKE + 2  # misaligned
    assert lib.pv_tower_create(C.byref(cfg), C.byref(w), C.byref(h)) == -1


def test_status_strings():
    lib = T.load_library()
    for code, name in T.STATUS.items():
        assert lib.pv_status_str(code).decode() == name


@pytest.fixture
def tower_handle():
    cfg = T.make_config(layers=2, max_side=1540)
    st, h, arr = create(cfg)
    assert st == 0
    yield T.load_library(), h, cfg
    T.load_library().pv_tower_destroy(h)


def _plan(lib, h, hw):
    arr, n = T._hw_array(hw)
    info = T.PvPlanInfo()
    st = lib.pv_tower_plan(h, arr, n, C.byref(info))
    return st, info


def test_plan_attention_item_size(tower_handle):
    """bf16: 384-query items (12 waves) only where they fill the chip's
    rounds of workgroups at least 0.1 better by count (512 slots of
    256-query items, 256 of 384-query items) at no more query padding."""
    lib, h, cfg = tower_handle

    def q_tile(hw):
        st, info = _plan(lib, h, hw)
        assert st == 0
        return info.attn_q_tile

    # 1540^2: 768 items fill 0.75 of two rounds of 512; 512 fill two of 256
    assert q_tile([(1540, 1540)]) == 384
    # 8,448 patches: 528 items (0.52 of two rounds) against 352 (0.69), same padding
    assert q_tile([(1344, 1232)]) == 384
    # two 1540^2 images: both fill their rounds completely
    assert q_tile([(1540, 1540)] * 2) == 256
    # few items: neither fills a round
    assert q_tile([(224, 224)]) == 256
    # 1,944 patches: fill 0.375 against 0.25, but 2,304 padded queries against 2,048
    assert q_tile([(252, 1512)]) == 256
    # 17 images of 448^2 (the GPU test of the head-by-head order over two
    # chunks): 1,088 items fill 0.71 of three rounds of 512, 816 fill 0.80
    # of four rounds of 256, but 19,584 padded queries against 17,408
    assert q_tile([(448, 448)] * 17) == 256
    # a subset of the images may choose the other size; the workspace of the
    # subset never exceeds that of the whole set (the embeddings cache
    # forwards the missed subset inside the whole set's workspace)
    st, whole = _plan(lib, h, [(28, 28), (1372, 1148)])
    st2, part = _plan(lib, h, [(1372, 1148)])
    assert st == 0 and st2 == 0
    assert (whole.attn_q_tile, part.attn_q_tile) == (384, 256)
    assert part.workspace_bytes <= whole.workspace_bytes
    st, hf, _ = create(T.make_config(layers=1, max_side=1540, dtype="f32"))
    assert st == 0
    arr, n = T._hw_array([(1540, 1540)])
    info = T.PvPlanInfo()
    assert lib.pv_tower_plan(hf, arr, n, C.byref(info)) == 0 and info.attn_q_tile == 64
    lib.pv_tower_destroy(hf)


def test_plan_counts_and_shape_errors(tower_handle):
    lib, h, cfg = tower_handle
    st, info = _plan(lib, h, [(1540, 1540)])
    assert st == 0 and info.n_patches == 12100 and info.out_rows == 3025 and info.out_cols == 5120
    assert info.workspace_bytes > 12100 * 1024 * (4 + 2 + 8)
    for bad in ([(1540, 1554)], [(30, 28)], [(0, 28)], [(28, -28)], [(28, 14)]):
        st, _ = _plan(lib, h, bad)
        assert st == -2, bad
        assert lib.pv_last_error()
    arr, _ = T._hw_array([(28, 28)])
    assert lib.pv_tower_plan(h, arr, 0, C.byref(T.PvPlanInfo())) == -1
    assert lib.pv_tower_plan(h, None, 1, C.byref(T.PvPlanInfo())) == -1


def test_forward_validation_before_any_device_work(tower_handle):
    """Every ARG/SHAPE/CAPACITY error returns before the first HIP call, so
    these run without a GPU (fake device pointers are never touched)."""
    lib, h, cfg = tower_handle
    hw = [(56, 84)]
    st, info = _plan(lib, h, hw)
    arr, n = T._hw_array(hw)
    big = 1 << 40
    ws = FAKE * 256
    assert lib.pv_tower_forward(None, FAKE, arr, n, FAKE, 99, ws, big, None) == -1
    assert lib.pv_tower_forward(h, None, arr, n, FAKE, 99, ws, big, None) == -1
    assert lib.pv_tower_forward(h, FAKE, arr, 0, FAKE, 99, ws, big, None) == -1
    assert lib.pv_tower_forward(h, FAKE, arr, n, FAKE, 99, ws + 8, big, None) == -1       # misaligned ws
    assert lib.pv_tower_forward(h, FAKE, arr, n, FAKE, info.out_rows - 1, ws, big, None) == -3
    assert lib.pv_tower_forward(h, FAKE, arr, n, FAKE, info.out_rows, ws, info.workspace_bytes - 1, None) == -3
    bad, nb = T._hw_array([(56, 70)])
    assert lib.pv_tower_forward(h, FAKE, bad, nb, FAKE, 99, ws, big, None) == -2
    assert lib.pv_tower_forward_stage(h, FAKE, arr, n, 9, 0, FAKE, big, ws, big, None) == -1
    assert lib.pv_tower_forward_stage(h, FAKE, arr, n, 2, 5, FAKE, big, ws, big, None) == -1
    assert lib.pv_tower_forward_stage(h, FAKE, arr, n, 2, 0, FAKE, 16, ws, big, None) == -3
    assert lib.pv_tower_index_maps(h, arr, n, FAKE, FAKE, FAKE, 1, None, 0, None) == -1
    assert lib.pv_tower_index_maps(h, arr, n, FAKE, FAKE, FAKE, 1, ws, 16, None) == -3


@pytest.mark.parametrize("name", ["tiny", "ms31_1540", "packed8", "pixtral_tiles16", "sweep64"])
def test_host_index_maps_equal_oracle(name):
    wl = synth.workload(name)
    cfg = T.config_for(wl)
    st, h, _ = create(cfg)
    assert st == 0
    lib = T.load_library()
    try:
        n = len(wl.image_hw)
        N, Tn = wl.n_patches, (wl.out_rows if wl.merge == 2 else 0)
        cu = np.zeros(n + 1, np.int32)
        rc = np.zeros((N, 2), np.int32)
        ms = np.zeros((max(Tn, 1), 4), np.int32)
        arr, _ = T._hw_array(wl.image_hw)
        assert lib.pv_tower_index_maps(h, arr, n, cu.ctypes.data, rc.ctypes.data,
                                       ms.ctypes.data if Tn else None, 0, None, 0, None) == 0
        m = O.plan_maps(wl.image_hw, wl.patch, wl.merge)
        np.testing.assert_array_equal(cu, m["cu_seqlens"])
        np.testing.assert_array_equal(rc, m["patch_rc"])
        if Tn:
            np.testing.assert_array_equal(ms[:Tn], m["merge_src"])
    finally:
        lib.pv_tower_destroy(h)


@pytest.mark.parametrize("args,status", [
    # (ids, S, image rows, text, dim, elem_bytes, status ptr, ws, ws bytes)
    ((FAKE, 10, FAKE, 4, FAKE, 5120, 2, FAKE, FAKE, 1 << 20), 0),
    ((FAKE, 10, FAKE, 4, FAKE, 5120, 3, FAKE, FAKE, 1 << 20), -1),      # element size
    ((FAKE, 10, FAKE, 4, FAKE, 4, 2, FAKE, FAKE, 1 << 20), -1),         # 8-byte rows
    ((FAKE, 10, FAKE, 4, FAKE, 0, 2, FAKE, FAKE, 1 << 20), -1),         # dim
    ((FAKE, -1, FAKE, 4, FAKE, 5120, 2, FAKE, FAKE, 1 << 20), -1),      # seq_len
    ((FAKE, 10, FAKE, -2, FAKE, 5120, 2, FAKE, FAKE, 1 << 20), -1),     # rows
    ((None, 10, FAKE, 4, FAKE, 5120, 2, FAKE, FAKE, 1 << 20), -1),      # token ids
    ((FAKE, 10, None, 4, FAKE, 5120, 2, FAKE, FAKE, 1 << 20), -1),      # image rows
    ((FAKE, 10, FAKE, 4, FAKE, 5120, 2, None, FAKE, 1 << 20), -1),      # status
    ((FAKE, 10, FAKE + 8, 4, FAKE, 5120, 2, FAKE, FAKE, 1 << 20), -1),  # alignment
    ((FAKE, 10, FAKE, 4, FAKE, 5120, 2, FAKE, FAKE + 16, 1 << 20), -1), # workspace alignment
    ((FAKE, 1000, FAKE, 4, FAKE, 5120, 2, FAKE, FAKE, 64), -3),         # workspace size
])
def test_scatter_validation_before_any_device_work(args, status):
    """Argument checks of the masked scatter; the one valid call is not made
    (it would touch device memory)."""
    lib = T.load_library()
    if status == 0:
        assert lib.pv_scatter_workspace_bytes(args[1]) <= args[9]
        return
    ids, S, img, rows, txt, dim, eb, st, ws, wsb = args
    got = lib.pv_scatter_image_embeddings(ids, S, 10, img, rows, txt, dim, eb, st, ws, wsb, None)
    assert got == status, lib.pv_last_error().decode()
    assert lib.pv_last_error().decode()


def test_scatter_workspace_grows_with_the_sequence():
    lib = T.load_library()
    a, b = lib.pv_scatter_workspace_bytes(0), lib.pv_scatter_workspace_bytes(100_000)
    assert a >= 256 and b >= 400_000 + 256 and b % 256 == 0


# ------------------------------------------------------------ uint8 input
def test_resize_target_equals_oracle():
    """The library's target-size rule is integer work: bit-exact against the
    oracle over random sizes, edges and grids."""
    rng = np.random.default_rng(31)
    hw = [(int(a), int(b)) for a, b in rng.integers(1, 9000, size=(300, 2))]
    hw += [(4096, 4096), (1540, 1540), (1, 1), (1, 32768), (32768, 17), (300, 200), (1000, 4000)]
    for L, g in [(1540, 28), (1024, 16), (1540, 14), (97, 5), (28, 28)]:
        got = T.resize_target(hw, L, g)
        want = [O.resize_target(h, w, L, g) for h, w in hw]
        assert got == want, (L, g)


def test_resize_target_errors():
    lib = T.load_library()
    dst = (C.c_int32 * 4)()
    for hw, L, g, status in [([(0, 5)], 1540, 28, -2), ([(5, 32769)], 1540, 28, -2), ([(5, 5)], 20, 28, -1),
                             ([(5, 5)], 1540, 0, -1)]:
        arr, n = T._hw_array(hw)
        assert lib.pv_resize_target(arr, n, L, g, dst) == status
        assert lib.pv_last_error()
    arr, n = T._hw_array([(5, 5)])
    assert lib.pv_resize_target(arr, 0, 1540, 28, dst) == -1
    assert lib.pv_resize_target(None, 1, 1540, 28, dst) == -1
    assert lib.pv_resize_target(arr, 1, 1540, 28, None) == -1


def test_plan_u8_targets_and_workspace(tower_handle):
    lib, h, cfg = tower_handle
    src = [(4096, 4096), (300, 200), (1000, 4000), (1, 1)]
    arr, n = T._hw_array(src)
    dst = (C.c_int32 * (2 * n))()
    info = T.PvPlanInfo()
    assert lib.pv_tower_plan_u8(h, arr, n, dst, C.byref(info)) == 0
    tgt = [(dst[2 * i], dst[2 * i + 1]) for i in range(n)]
    assert tgt == [O.resize_target(a, b, 1540, 28) for a, b in src]
    st, ref = _plan(lib, h, tgt)
    assert st == 0
    for f in ("n_patches", "out_rows", "out_cols", "workspace_bytes", "max_patches"):
        assert getattr(info, f) == getattr(ref, f), f
    assert lib.pv_tower_plan_u8(h, arr, n, None, C.byref(info)) == 0
    bad, nb = T._hw_array([(40000, 10)])
    assert lib.pv_tower_plan_u8(h, bad, nb, None, C.byref(info)) == -2


def test_forward_u8_and_preprocess_validation_before_device_work(tower_handle):
    lib, h, cfg = tower_handle
    src = [(100, 150)]
    arr, n = T._hw_array(src)
    info = T.PvPlanInfo()
    assert lib.pv_tower_plan_u8(h, arr, n, None, C.byref(info)) == 0
    big = 1 << 40
    ws = FAKE * 256
    ok_ms = (C.c_float * 6)(0.5, 0.5, 0.5, 0.25, 0.25, 0.25)
    bad_ms = (C.c_float * 6)(0.5, 0.5, 0.5, 0.25, 0.0, 0.25)
    f = lib.pv_tower_forward_u8
    assert f(None, FAKE, arr, n, None, FAKE, 99, ws, big, None) == -1
    assert f(h, None, arr, n, None, FAKE, 99, ws, big, None) == -1
    assert f(h, FAKE, None, n, None, FAKE, 99, ws, big, None) == -1
    assert f(h, FAKE, arr, 0, None, FAKE, 99, ws, big, None) == -1
    assert f(h, FAKE, arr, n, bad_ms, FAKE, 99, ws, big, None) == -1
    assert f(h, FAKE, arr, n, ok_ms, FAKE + 8, 99, ws, big, None) == -1       # output alignment
    assert f(h, FAKE, arr, n, None, FAKE, 99, ws + 16, big, None) == -1        # workspace alignment
    assert f(h, FAKE, arr, n, None, FAKE, info.out_rows - 1, ws, big, None) == -3
    assert f(h, FAKE, arr, n, None, FAKE, info.out_rows, ws, info.workspace_bytes - 1, None) == -3
    zero, nz = T._hw_array([(0, 10)])
    assert f(h, FAKE, zero, nz, None, FAKE, 99, ws, big, None) == -2
    p = lib.pv_preprocess_u8
    d, _ = T._hw_array([(28, 28)])
    assert p(None, arr, d, 1, None, FAKE, None) == -1
    assert p(FAKE, arr, None, 1, None, FAKE, None) == -1
    assert p(FAKE, arr, d, 0, None, FAKE, None) == -1
    assert p(FAKE, arr, d, 1, bad_ms, FAKE, None) == -1
    assert p(FAKE, arr, d, 1, None, FAKE + 2, None) == -1
    d0, _ = T._hw_array([(28, 0)])
    assert p(FAKE, arr, d0, 1, None, FAKE, None) == -2
    assert p(FAKE, zero, d, 1, None, FAKE, None) == -2


# ------------------------------------------------------------- tiles, presets
def test_tile_layout_equals_oracle():
    rng = np.random.default_rng(32)
    hw = [(int(a), int(b)) for a, b in rng.integers(1, 9000, size=(150, 2))]
    hw += [(4096, 4096), (1024, 1024), (1000, 3000), (1500, 6000), (1, 1), (32768, 32768)]
    for T_, g, M in [(1024, 16, 16), (1024, 16, 4), (1024, 16, 1), (1024, 16, 3), (1540, 28, 7), (64, 8, 100)]:
        got = T.tile_layout(hw, T_, g, M)
        want = [O.tile_layout(h, w, T_, g, M) for h, w in hw]
        assert got == want, (T_, g, M)


def test_tile_layout_errors():
    lib = T.load_library()
    lay = (C.c_int32 * 4)()
    arr, n = T._hw_array([(100, 100)])
    for tile, grid, M, status in [(1024, 0, 4, -1), (1000, 16, 4, -1), (1024, 16, 0, -1), (1024, 16, 65537, -1),
                                  (65536, 16, 4, -1)]:
        assert lib.pv_tile_layout(arr, n, tile, grid, M, lay) == status
    bad, nb = T._hw_array([(0, 100)])
    assert lib.pv_tile_layout(bad, nb, 1024, 16, 4, lay) == -2
    assert lib.pv_tile_layout(None, 1, 1024, 16, 4, lay) == -1
    assert lib.pv_tile_layout(arr, 0, 1024, 16, 4, lay) == -1


def test_presets_match_the_pages():
    m = T.preset("mistral3")
    assert (m.patch, m.hidden, m.heads, m.mlp, m.layers, m.merge, m.out_dim, m.max_side) == \
        (14, 1024, 16, 4096, 24, 2, 5120, 1540)
    p = T.preset("pixtral12b", "f32")
    assert (p.patch, p.hidden, p.heads, p.mlp, p.layers, p.merge, p.max_side) == (16, 1024, 16, 4096, 24, 1, 1024)
    assert p.dtype == T.PV_F32 and p.out_dtype == T.PV_F32 and m.dtype == T.PV_BF16
    assert m.rope_theta == p.rope_theta == 1.0e4
    lib = T.load_library()
    assert lib.pv_config_preset(7, 0, C.byref(T.PvConfig())) == -1
    assert lib.pv_config_preset(0, 5, C.byref(T.PvConfig())) == -1
    assert lib.pv_config_preset(0, 0, None) == -1
    # both presets create towers (weights are only borrowed, never touched here)
    for cfg in (m, p):
        st, h, _ = create(cfg)
        assert st == 0
        lib.pv_tower_destroy(h)


def test_plan_tiles_u8_counts():
    """Pixtral preset: a 4096x4096 photo with max_num_tiles 16 is 16 tiles of
    1024^2 = 65,536 output rows; the cap 4 gives 4 tiles (16,384 rows)."""
    cfg = T.preset("pixtral12b")
    st, h, _ = create(cfg)
    assert st == 0
    lib = T.load_library()
    try:
        arr, n = T._hw_array([(4096, 4096), (1000, 3000)])
        lay = (C.c_int32 * 8)()
        info = T.PvPlanInfo()
        assert lib.pv_tower_plan_tiles_u8(h, arr, n, 16, lay, C.byref(info)) == 0
        assert list(lay) == [4096, 4096, 4, 4, 1008, 3008, 1, 3]
        assert info.n_images == 19 and info.out_cols == 1024
        assert info.n_patches == 16 * 4096 + 63 * (64 + 64 + 60)
        tiles = [(1024, 1024)] * 16 + [(1008, 1024), (1008, 1024), (1008, 960)]
        st, ref = _plan(lib, h, tiles)
        assert st == 0 and ref.workspace_bytes == info.workspace_bytes and ref.out_rows == info.out_rows
        assert lib.pv_tower_plan_tiles_u8(h, arr, 1, 4, None, C.byref(info)) == 0
        assert info.n_patches == 4 * 4096 and info.n_images == 4
        assert lib.pv_tower_plan_tiles_u8(h, arr, 1, 0, None, C.byref(info)) == -1
        f = lib.pv_tower_forward_tiles_u8
        ws = FAKE * 256
        assert f(h, FAKE, arr, 1, 0, None, FAKE, 1 << 30, ws, 1 << 40, None) == -1
        assert f(h, FAKE, arr, 1, 4, None, FAKE, 4 * 4096 - 1, ws, 1 << 40, None) == -3
        assert f(h, None, arr, 1, 4, None, FAKE, 1 << 30, ws, 1 << 40, None) == -1
    finally:
        lib.pv_tower_destroy(h)


# ------------------------------------------------------------ embeddings cache
def test_embcache_host_side_without_device_work():
    cfg = T.make_config(layers=2, max_side=1540)
    st, h, _ = create(cfg)
    assert st == 0
    lib = T.load_library()
    c = C.c_void_p()
    try:
        row = 5120 * 2
        assert lib.pv_embcache_create(None, None, FAKE, 10 * row, C.byref(c)) == -1
        assert lib.pv_embcache_create(h, None, FAKE + 8, 10 * row, C.byref(c)) == -1
        assert lib.pv_embcache_create(h, None, FAKE, row - 1, C.byref(c)) == -3
        bad = (C.c_float * 6)(0.5, 0.5, 0.5, 0.2, -1.0, 0.2)
        assert lib.pv_embcache_create(h, bad, FAKE, 10 * row, C.byref(c)) == -1
        assert lib.pv_embcache_create(h, None, FAKE, 3025 * row + 7, C.byref(c)) == 0
        st5 = (C.c_int64 * 5)()
        assert lib.pv_embcache_stats(c, st5) == 0 and list(st5) == [0, 0, 3025, 0, 0]
        arr, n = T._hw_array([(4096, 4096), (100, 150)])
        b = C.c_int64()
        assert lib.pv_embcache_workspace_bytes(c, arr, n, C.byref(b)) == 0
        info = T.PvPlanInfo()
        assert lib.pv_tower_plan_u8(h, arr, n, None, C.byref(info)) == 0
        assert b.value >= info.workspace_bytes + 2 * 16
        f = lib.pv_tower_forward_cached_u8
        ws = FAKE * 256
        assert f(None, FAKE, arr, n, None, FAKE, 1 << 20, ws, 1 << 40, None, None) == -1
        assert f(c, FAKE, arr, 0, None, FAKE, 1 << 20, ws, 1 << 40, None, None) == -1
        assert f(c, FAKE + 1, arr, n, None, FAKE, 1 << 20, ws, 1 << 40, None, None) == -1   # hashing needs 4-byte alignment
        assert f(c, FAKE, arr, n, None, FAKE, 1 << 20, ws, b.value - 1, None, None) == -3
        assert f(c, FAKE, arr, n, None, FAKE, info.out_rows - 1, ws, 1 << 40, None, None) == -3
        big, nb = T._hw_array([(0, 5)])
        assert f(c, FAKE, big, nb, None, FAKE, 1 << 20, ws, 1 << 40, None, None) == -2
        assert lib.pv_embcache_clear(c) == 0
        kw = lib.pv_image_keys_workspace_bytes(3)
        assert kw >= 48 and kw % 256 == 0 and lib.pv_image_keys_workspace_bytes(0) == 0
        assert lib.pv_image_keys_u8(FAKE, arr, n, FAKE, ws, 16, None) == -3
        assert lib.pv_image_keys_u8(FAKE + 2, arr, n, FAKE, ws, 1 << 20, None) == -1
        assert lib.pv_image_keys_u8(FAKE, big, nb, FAKE, ws, 1 << 20, None) == -2
    finally:
        lib.pv_embcache_destroy(c)
        lib.pv_tower_destroy(h)


# ------------------------------------------------------------ fp8 variant
def test_fp8_flag_validation_and_workspace():
    lib = T.load_library()
    st, h, _ = create(T.make_config(layers=2, dtype="f32", flags=T.PV_FLAG_FP8))
    assert st == -5
    st, h, _ = create(T.make_config(layers=2, flags=16))
    assert st == -1
    st, h8, _ = create(T.make_config(layers=2, flags=T.PV_FLAG_FP8))
    st2, hb, _ = create(T.make_config(layers=2))
    assert st == 0 and st2 == 0
    try:
        s8, i8 = _plan(lib, h8, [(1540, 1540)])
        sb, ib = _plan(lib, hb, [(1540, 1540)])
        assert s8 == 0 and sb == 0
        # The fp8 variant adds its A operand at its widest ([N][F] fp8 and
        # 32-k scale bytes, in place of the merger's [T][2D] fp4 low part) and
        # the fp8 q|k|v, out-projection and down weights; its gate/up and down
        # copies are fp8 + scales where the bf16 tower holds fp16 ones.
        rnd = lambda x: (x + 255) // 256 * 256  # noqa: E731
        N, Tk, D, F = 12100, 3025, 1024, 4096
        s8, sT = N + 256, Tk + 256
        a8 = rnd(N * F) + rnd(max(F // 128 * s8 * 4, D // 64 * sT * 8)) - rnd(Tk * 2 * D) - rnd(D // 64 * sT * 8)
        gateup = rnd(2 * F * D) + rnd(D // 128 * 2 * F * 4) - rnd(2 * F * D * 2)
        w8 = (rnd(3 * D * D) + rnd(D // 128 * 3 * D * 4) + rnd(D * D) + rnd(D // 128 * D * 4) + rnd(D * F)
              + rnd(F // 128 * D * 4) - rnd(D * F * 2))
        assert i8.workspace_bytes - ib.workspace_bytes == a8 + gateup + w8
        assert lib.pv_quantize_fp8(None, 4, 128, FAKE, FAKE, None) == -1
        assert lib.pv_quantize_fp8(FAKE, 4, 96, FAKE, FAKE, None) == -1
        assert lib.pv_quantize_fp8(FAKE, 0, 128, FAKE, FAKE, None) == -1
        assert lib.pv_quantize_fp8(FAKE + 8, 4, 128, FAKE, FAKE, None) == -1
    finally:
        lib.pv_tower_destroy(h8)
        lib.pv_tower_destroy(hb)


def test_prepared_bytes_and_prepare_validation():
    """pv_tower_prepared_bytes: the padded patch weights plus, per block, the
    fp16 gate, up and down copies (bf16 tower) or the seven fp8 matrices (fp8 variant),
    plus the fp4 copy of the merge weights [O][4D] and its scale bytes (merge
    2); nothing for the fp32 tower.  pv_tower_prepare's argument checks
    return before any device work."""
    lib = T.load_library()
    D, F, L, Kp, O = 1024, 4096, 24, 640, 5120   # patch 14: 3 * 14^2 = 588 -> 640

    def rnd(x):
        return (x + 255) // 256 * 256

    def prepared(cfg):
        st, h, _ = create(cfg)
        assert st == 0
        b = C.c_int64(-1)
        assert lib.pv_tower_prepared_bytes(h, C.byref(b)) == 0
        return h, b.value

    h, b = prepared(T.make_config(layers=L))
    per_layer = rnd(2 * F * D * 2) + rnd(D * F * 2)  # fp16: gate rows then up rows; the down weights
    merge = rnd(O * 4 * D // 2) + rnd(4 * D // 256 * O * 8)
    assert b == rnd(D * Kp * 2) + L * per_layer + merge
    assert lib.pv_tower_prepare(None, FAKE * 256, b, None) == -1
    assert lib.pv_tower_prepare(h, FAKE * 256 + 16, b, None) == -1    # misaligned
    assert lib.pv_tower_prepare(h, FAKE * 256, b - 1, None) == -3     # too small
    assert lib.pv_tower_prepare(h, None, 0, None) == 0                # detach: nothing to do
    assert lib.pv_tower_prepared_bytes(h, None) == -1
    lib.pv_tower_destroy(h)
    h, b8 = prepared(T.make_config(layers=L, flags=T.PV_FLAG_FP8))
    per8 = (rnd(3 * D * D) + rnd(D // 128 * 3 * D * 4) + rnd(D * D) + rnd(D // 128 * D * 4) + rnd(2 * F * D)
            + rnd(D // 128 * 2 * F * 4) + rnd(D * F) + rnd(F // 128 * D * 4))
    assert b8 == rnd(D * Kp * 2) + L * per8 + merge
    lib.pv_tower_destroy(h)
    h, bn = prepared(T.make_config(layers=L, merge=1))   # no merger: no merge copy
    assert bn == rnd(D * Kp * 2) + L * per_layer
    lib.pv_tower_destroy(h)
    h, bf = prepared(T.make_config(layers=L, dtype="f32"))
    assert bf == 0
    lib.pv_tower_destroy(h)


def test_deep_projector_flag_validation():
    """PV_FLAG_DEEP_PROJECTOR: bf16 tower with merge only, projector weights
    required; the planner sizes the big region for the out_dim-wide GELU
    output."""
    lib = T.load_library()
    flag = T.PV_FLAG_DEEP_PROJECTOR
    st, h, _ = create(T.make_config(layers=2, flags=flag))
    assert st == -1 and b"proj" in lib.pv_last_error()
    st, h, _ = create(T.make_config(layers=2, dtype="f32", flags=flag))
    assert st == -5
    st, h, _ = create(T.make_config(layers=2, merge=1, flags=flag))
    assert st == -5
    w, arr = fake_weights(2, True)
    pj = T.PvProjectorWeights(FAKE, FAKE, FAKE)
    w.proj = C.pointer(pj)
    handles = []
    for out_dim, flags in ((5120, flag), (5120, 0), (32768, flag)):
        cfg = T.make_config(layers=2, out_dim=out_dim, flags=flags)
        hd = C.c_void_p()
        assert lib.pv_tower_create(C.byref(cfg), C.byref(w), C.byref(hd)) == 0
        handles.append(hd)
    st_d, deep = _plan(lib, handles[0], [(448, 448)])
    st_p, plain = _plan(lib, handles[1], [(448, 448)])
    st_w, wide = _plan(lib, handles[2], [(448, 448)])
    assert st_d == st_p == st_w == 0
    # 448^2: 1,024 patches, 256 merged tokens; the big region holds 1,024 rows
    # of 4,096 bf16 (8 MiB): 256 x 5,120 bf16 fit, 256 x 32,768 (16 MiB) grow
    # it.  Unprepared, the workspace also holds the fp4 copy of merge_w (its
    # rows x 2D bytes + 4D/256 x rows x 8 scale bytes): 5,120 rows for the
    # plain merge, D = 1,024 rows for the deeper projector's first matrix.
    D = 1024

    def merge_copy(rows):
        return rows * 2 * D + (4 * D // 256) * rows * 8

    assert plain.workspace_bytes - deep.workspace_bytes == merge_copy(5120) - merge_copy(1024)
    assert wide.workspace_bytes - deep.workspace_bytes == 256 * 32768 * 2 - 1024 * 4096 * 2
    for hd in handles:
        lib.pv_tower_destroy(hd)
