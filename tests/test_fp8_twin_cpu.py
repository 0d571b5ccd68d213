"""CPU checks of the fp8 stage chain used by the fp8 GPU tests: without the
twin's roundings it is the oracle's fp8 emulation itself; the twin's bf16
roundings move it by a bounded amount."""
import numpy as np

from fp8_twin import fp8_chain
from oracle import pv_oracle as O
from vlm_vision_encoder_amd import synth


def _case():
    wl = synth.Workload("fp8-chain", patch=14, layers=2, merge=2, image_hw=((112, 84), (56, 56)), dtype="bf16",
                        hidden=256, heads=4, mlp=512, out_dim=384)
    return wl, synth.make_weights(wl), synth.make_pixels(wl)


def test_fp8_chain_equals_oracle_emulation():
    wl, w, px = _case()
    cfg = O.TowerConfig(patch=wl.patch, hidden=wl.hidden, heads=wl.heads, mlp=wl.mlp, layers=wl.layers,
                        merge=wl.merge, out_dim=wl.out_dim, rope_theta=wl.rope_theta, rms_eps=wl.rms_eps)
    ref = O.tower_forward(px.astype(np.float64), wl.image_hw, synth.oracle_weights(w), cfg, collect=True, fp8=True)
    st = fp8_chain(px, wl, w)
    np.testing.assert_array_equal(st["out"], ref["out"])
    for l in range(wl.layers):
        np.testing.assert_array_equal(st["attn_resid"][l], ref["attn_out"][l])
        np.testing.assert_array_equal(st["block_out"][l], ref["block_out"][l])


def test_fp8_twin_moves_the_emulation_a_little():
    wl, w, px = _case()
    emu, twin = fp8_chain(px, wl, w)["out"], fp8_chain(px, wl, w, twin=True)["out"]
    d = np.max(np.abs(twin - emu)) / np.sqrt(np.mean(emu * emu))
    assert 0.0 < d < 0.5
