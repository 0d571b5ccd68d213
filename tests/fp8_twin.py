"""The fp8 variant of the tower written stage by stage from the oracle's
functions, with an optional bf16 twin (test helper, CPU only; imported by
the fp8 GPU tests and pinned to the oracle by test_fp8_twin_cpu.py)."""
import numpy as np

from oracle import pv_oracle as O
from vlm_vision_encoder_amd import synth


def _rms(a):
    return float(np.sqrt(np.mean(np.asarray(a, np.float64) ** 2)))


def fp8_chain(px, wl, w, twin=False):
    """The fp8 variant stage by stage, from the oracle's functions: returns
    per layer the attention output, the residual after attention, silu(gate)
    * up and the residual after the block, and the output.  twin=False is the
    oracle's fp8 emulation (equal to tower_forward(..., fp8=True), checked on
    the CPU in test_fp8_chain_equals_oracle_emulation).  twin=True adds the
    bf16 rounding of the values the bf16 tower stores before they are
    quantised or consumed -- q, k, v, the attention output, silu(gate) * up --
    and nothing else: its distance from the emulation is the size of the
    rounding-boundary flips those roundings cause, the level a correct GPU
    tower sits at."""
    rb = (lambda a: synth.round_to_bf16(np.asarray(a, np.float32)).astype(np.float64)) if twin else (lambda a: a)
    ow = synth.oracle_weights(w)
    maps = O.plan_maps(wl.image_hw, wl.patch, wl.merge)
    h = O.rms_norm(O.patch_embed(px.astype(np.float64), wl.image_hw, ow["patch_w"], wl.patch), ow["ln_pre"],
                   wl.rms_eps)
    st = {"attn": [], "attn_resid": [], "mlp_hidden": [], "block_out": []}
    qz = O.mx_e4m3
    for lw in ow["layers"][:wl.layers]:
        y = qz(O.rms_norm(h, lw["attn_norm"], wl.rms_eps))
        q = rb(O.rope_2d(y @ qz(lw["wq"]).T, maps["patch_rc"], wl.heads, wl.rope_theta))
        k = rb(O.rope_2d(y @ qz(lw["wk"]).T, maps["patch_rc"], wl.heads, wl.rope_theta))
        v = rb(y @ qz(lw["wv"]).T)
        a = rb(O.attention(q, k, v, maps["cu_seqlens"], wl.heads))
        h = h + qz(a) @ qz(lw["wo"]).T
        y2 = qz(O.rms_norm(h, lw["ffn_norm"], wl.rms_eps))
        g, u = y2 @ qz(lw["w_gate"]).T, y2 @ qz(lw["w_up"]).T
        hm = rb(g / (1.0 + np.exp(-g)) * u)
        st["attn"].append(a)
        st["attn_resid"].append(h)
        st["mlp_hidden"].append(hm)
        h = h + qz(hm) @ qz(lw["w_down"]).T
        st["block_out"].append(h)
    st["out"] = O.merge_project(h, maps["merge_src"], ow["merge_w"]) if wl.merge == 2 else h
    return st
