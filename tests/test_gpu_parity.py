"""GPU parity of the HIP tower against the float64 oracle, through the C ABI.

Bar: index maps and cu_seqlens bit-exact; floats
max|gpu - oracle| <= tol * RMS(oracle) per tensor, tol = 2e-2 (bf16 path) and
1e-4 (fp32 path).  Inputs are the seeded synthetic ones of
vlm_vision_encoder_amd.synth; every case prints its name before the GPU work.
"""
import os

import numpy as np
import pytest

from oracle import pv_oracle as O
from vlm_vision_encoder_amd import synth
from vlm_vision_encoder_amd import tower as T

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f32": 1e-4}


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)


def oracle_cfg(wl, layers=None):
    return O.TowerConfig(patch=wl.patch, hidden=wl.hidden, heads=wl.heads, mlp=wl.mlp,
                         layers=wl.layers if layers is None else layers, merge=wl.merge, out_dim=wl.out_dim,
                         rope_theta=wl.rope_theta, rms_eps=wl.rms_eps, rope_interleaved=wl.rope_interleaved)


def rel_err(got, want):
    want = np.asarray(want, np.float64)
    got = np.asarray(got, np.float64)
    rms = np.sqrt(np.mean(want * want))
    return float(np.max(np.abs(got - want)) / rms), rms


def to_np(t):
    return t.float().cpu().numpy().astype(np.float64)


class Case:
    """Builds weights/pixels once; runs the GPU tower and the oracle."""

    def __init__(self, wl, weights=None, pixels=None):
        torch = _torch()
        self.wl = wl
        self.w = synth.make_weights(wl) if weights is None else weights
        self.px = synth.make_pixels(wl) if pixels is None else pixels
        self.dev_w = T.weights_to_device(self.w, wl.dtype)
        self.tower = T.Tower(T.config_for(wl), self.dev_w)
        self.pix = torch.from_numpy(self.px).cuda()
        self._ref = None

    def ref(self):
        if self._ref is None:
            self._ref = O.tower_forward(self.px.astype(np.float64), self.wl.image_hw, synth.oracle_weights(self.w),
                                        oracle_cfg(self.wl), collect=True)
        return self._ref

    def run(self):
        torch = _torch()
        out = self.tower.forward(self.pix, self.wl.image_hw)
        torch.cuda.synchronize()
        return out

    def stage(self, name, layer=0):
        torch = _torch()
        out = self.tower.forward_stage(self.pix, self.wl.image_hw, name, layer)
        torch.cuda.synchronize()
        return out


# bf16 keeps 8 significant bits, so rounding a value x to bf16 moves it by
# at most half an ulp <= 2^-8 |x|; fp16 keeps 11: at most 2^-11 |x|
BF16_ULP = 2.0 ** -8
F16_ULP = 2.0 ** -11


def storage_ulp(t):
    """Largest relative storage rounding of a 16-bit stage tensor."""
    torch = _torch()
    return F16_ULP if t.dtype == torch.float16 else BF16_ULP


def check(name, got, want, tol, stored_bf16=False, ulp=BF16_ULP):
    """max|got - want| <= tol * RMS(want).  A tensor that the bf16 path stores
    in 16 bits is also allowed its own storage rounding (at most ulp |want|:
    2^-8 for bf16, 2^-11 for fp16)."""
    want = np.asarray(want, np.float64)
    got = np.asarray(got, np.float64)
    rms = float(np.sqrt(np.mean(want * want)))
    diff = np.abs(got - want)
    if stored_bf16:
        diff = np.maximum(diff - ulp * np.abs(want), 0.0)
    kind = ", bf16-stored" if ulp == BF16_ULP else ", fp16-stored"
    e = float(np.max(diff) / rms)
    say(f"  {name}: max-abs-err/RMS = {e:.3e} (RMS {rms:.3e}, tol {tol}{kind if stored_bf16 else ''})")
    assert np.isfinite(e) and e <= tol, f"{name}: {e} > {tol}"


BF16_STORED = ("qkv", "attn", "mlp_hidden")


def check_per_image(name, got, want, cu_seqlens, tol, stored_bf16=False):
    """check() on every image's rows separately.  Attention is block
    diagonal ("Mistral 3" (KerasFormers), Mistral3VisionModel: every image
    attends only within itself), so each image is its own attention problem
    and is held to the bar relative to its own RMS: a 4-patch image's
    outputs average 4 value rows and sit several times above the RMS of a
    large image's, which dominates the RMS of the whole pack."""
    for i in range(len(cu_seqlens) - 1):
        a, b = int(cu_seqlens[i]), int(cu_seqlens[i + 1])
        check(f"{name} image {i}", got[a:b], want[a:b], tol, stored_bf16)


def oracle_stage(ref, wl, name, layer, w):
    """Oracle value of a debug stage (recomputed from the oracle's own
    per-layer states, never from GPU values)."""
    if name == "patch_embed":
        return ref["patch_embed"]
    if name == "ln_pre":
        return ref["ln_pre"]
    if name == "attn_resid":
        return ref["attn_out"][layer]
    if name == "block_out":
        return ref["block_out"][layer]
    h = ref["ln_pre"] if layer == 0 else ref["block_out"][layer - 1]
    lw = synth.oracle_weights(w)["layers"][layer]
    maps = ref["maps"]
    if name in ("qkv", "attn"):
        y = O.rms_norm(h, lw["attn_norm"], wl.rms_eps)
        q = O.rope_2d(y @ lw["wq"].T, maps["patch_rc"], wl.heads, wl.rope_theta, wl.rope_interleaved)
        k = O.rope_2d(y @ lw["wk"].T, maps["patch_rc"], wl.heads, wl.rope_theta, wl.rope_interleaved)
        v = y @ lw["wv"].T
        if name == "qkv":
            # the bf16 tower stores q in its softmax's exp2 units
            qs = q * (np.log2(np.e) / 8.0) if wl.dtype == "bf16" else q
            return np.concatenate([qs, k, v], axis=1)
        return O.attention(q, k, v, maps["cu_seqlens"], wl.heads)
    if name == "mlp_hidden":
        y = O.rms_norm(ref["attn_out"][layer], lw["ffn_norm"], wl.rms_eps)
        g = y @ lw["w_gate"].T
        return g / (1.0 + np.exp(-g)) * (y @ lw["w_up"].T)
    raise KeyError(name)


ALL_STAGES = ("patch_embed", "ln_pre", "qkv", "attn", "attn_resid", "mlp_hidden", "block_out")


# ------------------------------------------------------------------ index maps
@pytest.mark.parametrize("name", synth.WORKLOADS)
def test_device_index_maps_exact(name):
    _torch()
    wl = synth.workload(name)
    say(f"device index maps {name}")
    dev_w = {"patch_w": None}
    import torch
    # weights are not read by the map kernel; any aligned buffers do, as long
    # as the tower makes no weight copies (prepare=False: preparing would read
    # every matrix at its full size)
    z = torch.zeros(16, dtype=torch.float32, device="cuda")
    lw = {k: z for k in ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate", "w_up", "w_down")}
    tw = T.Tower(T.config_for(wl), {"patch_w": z, "ln_pre": z, "layers": [lw] * wl.layers, "merge_w": z},
                 prepare=False)
    cu, rc, ms = tw.index_maps(wl.image_hw, on_device=True)
    m = O.plan_maps(wl.image_hw, wl.patch, wl.merge)
    np.testing.assert_array_equal(cu, m["cu_seqlens"])
    np.testing.assert_array_equal(rc, m["patch_rc"])
    if wl.merge == 2:
        np.testing.assert_array_equal(ms, m["merge_src"])
    tw.close()


# ------------------------------------------------------------------ fp32 tower
def test_tiny_fp32_full_and_stages():
    wl = synth.workload("tiny")
    say("tiny fp32 224x224, 1 layer")
    c = Case(wl)
    ref = c.ref()
    check("out", to_np(c.run()), ref["out"], TOL["f32"])
    for st in ALL_STAGES:
        check(st, to_np(c.stage(st, 0)), oracle_stage(ref, wl, st, 0, c.w), TOL["f32"])


# ------------------------------------------------------------------ bf16 tower
def _bf16_small(image_hw, layers, patch=14, merge=2, **kw):
    base = synth.workload("ms31_1540")
    return base.with_(name="small", image_hw=tuple(image_hw), layers=layers, patch=patch, merge=merge, **kw)


def test_bf16_stages_single_image():
    wl = _bf16_small([(224, 224)], 2)
    say("bf16 stages 224x224, 2 layers")
    c = Case(wl)
    ref = c.ref()
    for layer in range(2):
        for st in ALL_STAGES[2:]:
            t = c.stage(st, layer)
            check(f"{st}[{layer}]", to_np(t), oracle_stage(ref, wl, st, layer, c.w),
                  TOL["bf16"], stored_bf16=st in BF16_STORED, ulp=storage_ulp(t))
    check("patch_embed", to_np(c.stage("patch_embed")), ref["patch_embed"], TOL["bf16"])
    check("ln_pre", to_np(c.stage("ln_pre")), ref["ln_pre"], TOL["bf16"])
    check("out", to_np(c.run()), ref["out"], TOL["bf16"])


def test_bf16_packed_ragged_batch():
    # 468 + 4 + 248 + 300 patches: none a multiple of 64, one image of 4 patches
    wl = _bf16_small([(252, 364), (28, 28), (56, 868), (420, 140)], 3)
    say(f"bf16 packed ragged {wl.image_hw}, 3 layers")
    c = Case(wl)
    ref = c.ref()
    check("out", to_np(c.run()), ref["out"], TOL["bf16"])
    check("block_out[2]", to_np(c.stage("block_out", 2)), ref["block_out"][2], TOL["bf16"])
    # q,k,v of blocks 1 and 2 (inputs from the down products and norms
    # before them), every image of the ragged pack, with rows of the last
    # tile past the end
    for layer in (1, 2):
        t = c.stage("qkv", layer)
        check_per_image(f"qkv[{layer}]", to_np(t), oracle_stage(ref, wl, "qkv", layer, c.w),
                        ref["maps"]["cu_seqlens"], TOL["bf16"], stored_bf16=True)
    # the same tower writing an fp32 output buffer: no storage rounding
    import torch
    tw = T.Tower(T.config_for(wl, out_dtype="f32"), c.dev_w)
    out = tw.forward(c.pix, wl.image_hw)
    torch.cuda.synchronize()
    assert out.dtype == torch.float32
    check("out (fp32 buffer)", to_np(out), ref["out"], TOL["bf16"])


def test_bf16_no_merge_patch16_single_patch_image():
    # Pixtral-12B style: patch 16, no merge; includes a one-patch image
    wl = _bf16_small([(256, 384), (16, 16), (128, 112)], 2, patch=16, merge=1)
    say(f"bf16 patch16 no-merge {wl.image_hw}")
    c = Case(wl)
    ref = c.ref()
    out = c.run()
    assert tuple(out.shape) == (wl.n_patches, 1024)
    check("out", to_np(out), ref["out"], TOL["bf16"])


def test_bf16_mlp_fp16_range_saturates():
    """The MLP's fp16 operands saturate at +-65504 instead of overflowing: a
    norm weight of 4096 puts the MLP input of layer 0 at up to about
    sqrt(1024) * 4096 = 131072 (past fp16's range), and the silu * up values
    past it too.  The stage and the tower output stay finite (the oracle,
    which does not saturate, is not the bar here)."""
    torch = _torch()
    wl = _bf16_small([(112, 84)], 1)
    w = synth.make_weights(wl)
    w["layers"][0]["ffn_norm"] = np.full_like(w["layers"][0]["ffn_norm"], 4096.0)
    say("bf16 MLP input past fp16 range (ffn_norm = 4096)")
    c = Case(wl, weights=w)
    hid = c.stage("mlp_hidden", 0)
    assert hid.dtype == torch.float16
    hv = hid.float()
    say(f"  mlp_hidden max |value| {hv.abs().max().item():.1f}")
    assert torch.isfinite(hv).all().item()
    assert hv.abs().max().item() == 65504.0  # some values really saturated
    out = c.run()
    assert torch.isfinite(out.float()).all().item()


def test_bf16_merger_width_not_multiple_of_256():
    """Merger output width 384 (a multiple of 128 only): the merger GEMM takes
    its 256 x 128 tiles instead of 256 x 256."""
    wl = _bf16_small([(224, 224), (56, 112)], 1, out_dim=384)
    say(f"bf16 merger width 384 {wl.image_hw}")
    c = Case(wl)
    ref = c.ref()
    out = c.run()
    assert tuple(out.shape) == (wl.out_rows, 384)
    check("out", to_np(out), ref["out"], TOL["bf16"])


def test_bf16_many_tiny_images():
    """150 images of 1 to 9 merged tokens each (28..84 pixels a side): every
    attention work item is a whole small image and row tiles cross many
    image boundaries."""
    rng = np.random.default_rng(81)
    hw = [(28 * int(a), 28 * int(b)) for a, b in rng.integers(1, 4, size=(150, 2))]
    wl = _bf16_small(hw, 2, hidden=256, heads=4, mlp=512, out_dim=384)
    say(f"bf16 {len(hw)} tiny images, {wl.n_patches} patches")
    c = Case(wl)
    ref = c.ref()
    check("out", to_np(c.run()), ref["out"], TOL["bf16"])


def test_bf16_wide_tiles_for_the_hidden_width_products():
    """9 images of 448^2 (9,216 patches, D 1024): the out-projection, down
    and patch-embedding products take their 192 x 256 tiles (one round of
    the chip instead of two partly filled ones) -- checked stage by stage."""
    wl = _bf16_small([(448, 448)] * 9, 1)
    say(f"bf16 wide hidden-width tiles: {wl.n_patches} patches")
    c = Case(wl)
    ref = c.ref()
    check("patch_embed", to_np(c.stage("patch_embed")), ref["patch_embed"], TOL["bf16"])
    check("attn_resid[0]", to_np(c.stage("attn_resid", 0)), ref["attn_out"][0], TOL["bf16"])
    check("block_out[0]", to_np(c.stage("block_out", 0)), ref["block_out"][0], TOL["bf16"])
    check("out", to_np(c.run()), ref["out"], TOL["bf16"])


@pytest.mark.parametrize("n_images,tiles", [(16, "256x256"), (11, "384x192")])
def test_bf16_qkv_and_down_tile_shapes(n_images, tiles):
    """Images of 448^2 (D 1024, MLP 4096), q,k,v and the MLP block checked in
    full.  16 images (16,384 patches): q,k,v and down take 256 x 256 tiles
    (q,k,v 768 tiles in three rounds against 688 tiles of 384 x 192, also
    three rounds; down 256 tiles, one round against two of 128 x 128 or
    192 x 256).  11 images (11,264 patches): q,k,v keeps 384 x 192 tiles
    (480 tiles in two rounds against 528 of 256 x 256 in three)."""
    wl = _bf16_small([(448, 448)] * n_images, 1)
    say(f"bf16 q,k,v in {tiles} tiles: {wl.n_patches} patches")
    c = Case(wl)
    ref = c.ref()
    t = c.stage("qkv", 0)
    check("qkv[0]", to_np(t), oracle_stage(ref, wl, "qkv", 0, c.w), TOL["bf16"],
          stored_bf16=True, ulp=storage_ulp(t))
    check("block_out[0]", to_np(c.stage("block_out", 0)), ref["block_out"][0], TOL["bf16"])
    check("out", to_np(c.run()), ref["out"], TOL["bf16"])


def test_bf16_attention_head_by_head_order_across_chunks():
    """17 images of 448^2, all one length: 68 attention items of 256 queries
    per head, so each XCD walks a full chunk of 64 items head by head and
    then a last chunk of 4 -- the attention stage checked in full, per
    image."""
    wl = _bf16_small([(448, 448)] * 17, 1)
    say(f"bf16 attention head by head over chunks: {wl.n_patches} patches")
    c = Case(wl)
    ref = c.ref()
    got = to_np(c.stage("attn", 0))
    want = oracle_stage(ref, wl, "attn", 0, c.w)
    check_per_image("attn[0]", got, want, ref["maps"]["cu_seqlens"], TOL["bf16"], stored_bf16=True)


@pytest.mark.parametrize("hidden,heads,mlp", [(512, 8, 1024), (768, 12, 2048), (1536, 24, 3072), (2048, 32, 2048)])
def test_bf16_other_widths(hidden, heads, mlp):
    """The other supported widths (norm kernels of 2, 3, 6, 8 row chunks; q,k,v
    with 3D columns in 192-wide tiles; merger K = 4D)."""
    wl = _bf16_small([(224, 168), (56, 84)], 2, hidden=hidden, heads=heads, mlp=mlp, out_dim=640)
    say(f"bf16 width D={hidden} heads={heads} F={mlp}")
    c = Case(wl)
    ref = c.ref()
    check("out", to_np(c.run()), ref["out"], TOL["bf16"])


def test_bf16_sharp_logits():
    """Logit std ~4 instead of ~0.4.  bf16 storage of q and k moves every
    logit s by up to about 2^-8 |s| (two half-ulp roundings), which moves the
    softmax weights by that relative amount, so the bound of the attention
    stage is 2e-2 + 2^-8 * max|s| (max|s| from the oracle's own q, k); the
    tower output is held to the plain 2e-2."""
    wl = _bf16_small([(308, 196), (84, 56)], 1)
    w = synth.make_weights(wl)
    rng = np.random.default_rng(77)
    for lw in w["layers"]:  # logit std ~ 4 instead of ~0.4
        lw["wq"] = synth.round_to_bf16(rng.standard_normal(lw["wq"].shape, dtype=np.float32) * np.float32(0.0625))
        lw["wk"] = synth.round_to_bf16(rng.standard_normal(lw["wk"].shape, dtype=np.float32) * np.float32(0.0625))
    say("bf16 sharp logits")
    c = Case(wl, weights=w)
    ref = c.ref()
    qkv = oracle_stage(ref, wl.with_(dtype="f32"), "qkv", 0, w)  # unscaled q
    cu = ref["maps"]["cu_seqlens"]
    smax = 0.0
    for i in range(len(cu) - 1):
        a, b = cu[i], cu[i + 1]
        for h in range(wl.heads):
            q = qkv[a:b, h * 64:(h + 1) * 64]
            k = qkv[a:b, 1024 + h * 64:1024 + (h + 1) * 64]
            smax = max(smax, float(np.max(np.abs(q @ k.T))) / 8.0)
    tol = TOL["bf16"] + BF16_ULP * smax
    say(f"  max |logit| {smax:.2f} -> tol {tol:.3f}")
    assert smax > 10.0  # the case is really sharp
    check("attn[0]", to_np(c.stage("attn", 0)), oracle_stage(ref, wl, "attn", 0, w), tol, stored_bf16=True)
    # the one-block tower's output (after the out-projection, the MLP and the
    # merger) stays within the plain bar
    check("out", to_np(c.run()), ref["out"], TOL["bf16"])


def test_bf16_online_max_softmax_path():
    """The running-max softmax (the fallback of the fixed-offset one), forced
    on, on a ragged packed batch and on sharp logits."""
    import torch
    wl = _bf16_small([(252, 364), (28, 28), (420, 140)], 2)
    say("bf16 online-max softmax, ragged batch")
    c = Case(wl)
    ref = c.ref()
    tw = T.Tower(T.config_for(wl, flags=T.PV_FLAG_ATTN_ONLINE_MAX), c.dev_w)
    out = tw.forward(c.pix, wl.image_hw)
    torch.cuda.synchronize()
    check("out", to_np(out), ref["out"], TOL["bf16"])
    att = to_np(tw.forward_stage(c.pix, wl.image_hw, "attn", 0))
    torch.cuda.synchronize()
    want = oracle_stage(ref, wl, "attn", 0, c.w)
    # per image, against that image's own RMS: a 4-patch image's attention
    # outputs are barely averaged, so they are large next to the batch RMS
    cu = ref["maps"]["cu_seqlens"]
    for i in range(len(cu) - 1):
        check(f"attn[0] image {i}", att[cu[i]:cu[i + 1]], want[cu[i]:cu[i + 1]], TOL["bf16"], stored_bf16=True)


@pytest.mark.parametrize("image_hw", [
    [(1344, 1232)],
    [(28, 28), (1372, 1148)],
], ids=["one-image", "tiny-image-and-ragged-tail"])
def test_bf16_wide_attention_items(image_hw):
    """At 16 heads the planner takes the 12-wave work items of 384 queries
    for both packs (352 items fill two rounds of 256 workgroups better than
    528 items of 256 queries fill two rounds of 512, at the same padding).
    One 1344x1232 image is 8,448 patches, 22 full items per head.  The second
    pack puts a 4-patch image first (an item with one active wave, 4 live
    queries and 4 keys, waves 1-11 without queries) and then 8,036 patches
    (20 full items and one of 356 queries, whose last wave has 4 live
    queries and clamped rows, and whose last key tile is partly masked).
    Attention of layer 0 against the oracle, per image, with the fixed
    offset and with the running max forced (the fallback pass)."""
    import torch
    wl = _bf16_small(image_hw, 1, mlp=1024)
    say(f"bf16 12-wave attention items: {wl.image_hw}, {wl.n_patches} patches")
    c = Case(wl)
    assert c.tower.plan(wl.image_hw).attn_q_tile == 384
    ref = c.ref()
    want = oracle_stage(ref, wl, "attn", 0, c.w)
    cu = ref["maps"]["cu_seqlens"]
    check_per_image("attn[0]", to_np(c.stage("attn", 0)), want, cu, TOL["bf16"], stored_bf16=True)
    tw = T.Tower(T.config_for(wl, flags=T.PV_FLAG_ATTN_ONLINE_MAX), c.dev_w)
    att = to_np(tw.forward_stage(c.pix, wl.image_hw, "attn", 0))
    torch.cuda.synchronize()
    check_per_image("attn[0] online max", att, want, cu, TOL["bf16"], stored_bf16=True)
    check("out", to_np(c.run()), ref["out"], TOL["bf16"])
    tw.close()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rope_interleaved_flag(dtype):
    """PV_FLAG_ROPE_INTERLEAVED: the column rotary pairs on the odd steps of
    one ladder shared with the rows.  q,k,v of layer 0 and the output of a
    one-block tower against the oracle with the same split, on a non-square
    image beside a small one; the default tower's q,k,v differ from it."""
    import torch
    base = synth.workload("tiny") if dtype == "f32" else synth.workload("ms31_1540")
    wl = base.with_(name="rope-interleaved", image_hw=((224, 336), (112, 56)), layers=1, mlp=1024,
                    rope_interleaved=True)
    say(f"{dtype} interleaved rotary ladder {wl.image_hw}")
    c = Case(wl)  # its own tower keeps the default split
    tw = T.Tower(T.config_for(wl, flags=T.PV_FLAG_ROPE_INTERLEAVED), c.dev_w)
    ref = c.ref()
    stored = dtype == "bf16"
    want = oracle_stage(ref, wl, "qkv", 0, c.w)
    got = to_np(tw.forward_stage(c.pix, wl.image_hw, "qkv", 0))
    torch.cuda.synchronize()
    check("qkv[0]", got, want, TOL[dtype], stored_bf16=stored)
    out = to_np(tw.forward(c.pix, wl.image_hw))
    torch.cuda.synchronize()
    check("out", out, ref["out"], TOL[dtype])
    dflt = to_np(c.stage("qkv", 0))
    moved = float(np.max(np.abs(dflt - got)) / np.sqrt(np.mean(want * want)))
    say(f"  default split moves qkv by {moved:.3e} of RMS")
    assert moved > 0.1
    tw.close()


def test_bf16_fixed_offset_overflow_falls_back():
    """First key tile of the image all zero (zero pixels -> zero keys, offset
    m0 = 0) and large q/k weights: later scores exceed m0 by far more than
    2^127 can hold, so the fixed-offset pass overflows and the work item must
    rerun with the running max -- giving exactly the forced-online result."""
    import torch
    wl = _bf16_small([(224, 224)], 1)
    w = synth.make_weights(wl)
    rng = np.random.default_rng(99)
    lw = w["layers"][0]
    lw["wq"] = synth.round_to_bf16(rng.standard_normal(lw["wq"].shape, dtype=np.float32) * np.float32(0.25))
    lw["wk"] = synth.round_to_bf16(rng.standard_normal(lw["wk"].shape, dtype=np.float32) * np.float32(0.25))
    px = synth.make_pixels(wl).reshape(3, 224, 224).copy()
    px[:, :56, :] = 0.0  # patch rows 0..3 = the first 64 patches
    px = px.reshape(-1)
    say("bf16 fixed-offset overflow -> online-max fallback")
    c = Case(wl, weights=w, pixels=px)
    a0 = c.stage("attn", 0)
    tw = T.Tower(T.config_for(wl, flags=T.PV_FLAG_ATTN_ONLINE_MAX), c.dev_w)
    a1 = tw.forward_stage(c.pix, wl.image_hw, "attn", 0)
    torch.cuda.synchronize()
    assert torch.isfinite(a0.float()).all().item(), "fixed-offset pass left non-finite output"
    assert torch.equal(a0, a1), "fallback result differs from the online-max pass"
    # the scores really are far beyond the fixed offset's range
    ref = c.ref()
    qkv = oracle_stage(ref, wl.with_(dtype="f32"), "qkv", 0, w)  # unscaled q
    s = qkv[64:, :64] @ qkv[64:, 1024:1088].T / 8.0 * np.log2(np.e)
    say(f"  max score {s.max():.1f} (log2 units) vs first-tile offset 0")
    assert s.max() > 130


def test_bf16_packing_invariance_and_determinism_bitexact():
    torch = _torch()
    hw = [(140, 168), (56, 84), (196, 28)]
    wl = _bf16_small(hw, 2)
    say("bf16 packing invariance / determinism")
    c = Case(wl)
    packed = c.run()
    again = c.run()
    assert torch.equal(packed, again), "two runs differ"
    starts = np.cumsum([0] + [(h // 28) * (w // 28) for h, w in hw])
    off = 0
    for i, (h, w) in enumerate(hw):
        n = 3 * h * w
        alone = c.tower.forward(c.pix[off:off + n], [(h, w)])
        torch.cuda.synchronize()
        off += n
        assert torch.equal(alone, packed[starts[i]:starts[i + 1]]), f"image {i} differs when packed"


def test_zero_layer_tower_and_capacity_errors():
    wl = _bf16_small([(56, 56)], 0)
    say("bf16 zero-layer tower")
    c = Case(wl)
    ref = c.ref()
    check("out", to_np(c.run()), ref["out"], TOL["bf16"])


@pytest.mark.parametrize("case", ["narrow-3-images", "full-width"])
def test_bf16_deep_projector(case):
    """The deeper projector variant (PV_FLAG_DEEP_PROJECTOR: RMSNorm -> 2x2
    merge 4D -> D -> D -> out_dim -> GELU -> out_dim -> out_dim) against the
    oracle's deep_project: output at the bf16 bar with an fp32 and with a
    bf16 output buffer."""
    torch = _torch()
    if case == "full-width":
        wl = synth.Workload("deep", patch=14, layers=1, merge=2, image_hw=((448, 448),), deep_projector=True)
    else:
        wl = synth.Workload("deep", patch=14, layers=2, merge=2, image_hw=((448, 392), (224, 280), (84, 140)),
                            hidden=256, heads=4, mlp=512, out_dim=384, deep_projector=True)
    say(f"bf16 deeper projector {case}: {wl.n_patches} patches, out_dim {wl.out_dim}")
    w = synth.make_weights(wl)
    px = synth.make_pixels(wl)
    dev_w = T.weights_to_device(w, "bf16")
    cfg = O.TowerConfig(patch=wl.patch, hidden=wl.hidden, heads=wl.heads, mlp=wl.mlp, layers=wl.layers, merge=2,
                        out_dim=wl.out_dim, rope_theta=wl.rope_theta, rms_eps=wl.rms_eps, deep_projector=True)
    ref = O.tower_forward(px.astype(np.float64), wl.image_hw, synth.oracle_weights(w), cfg)["out"]
    pix = torch.from_numpy(px).cuda()
    for out_dtype in ("f32", "bf16"):
        tw = T.Tower(T.config_for(wl, out_dtype=out_dtype, flags=T.PV_FLAG_DEEP_PROJECTOR), dev_w)
        out = tw.forward(pix, wl.image_hw)
        torch.cuda.synchronize()
        assert tuple(out.shape) == ref.shape
        check(f"deep projector out ({out_dtype} buffer)", to_np(out), ref, TOL["bf16"], stored_bf16=out_dtype == "bf16")
        tw.close()
