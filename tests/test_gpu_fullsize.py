"""Full-size GPU parity: the 24-layer tower on the benchmark workloads, in the
launch configuration bench.py times, against sampled rows of the float64
oracle's output stored by tests/golden/make_golden.py (which calls only the
oracle).

Bar (bf16 tower): max|gpu - oracle| <= 2e-2 * RMS(oracle output), RMS over
the whole oracle output, for an fp32 and for a bf16 output buffer alike.
For the bf16 buffer the error left after each element's own storage
rounding (at most 2^-8 |value|) is printed beside it: the share of the
tower's arithmetic.
"""
import os

import numpy as np
import pytest

from vlm_vision_encoder_amd import synth
from vlm_vision_encoder_amd import tower as T

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
TOL = 2e-2
BF16_STORE = 2.0 ** -8


def _golden(name):
    path = os.path.join(HERE, "golden", f"{name}.npz")
    if not os.path.exists(path):
        pytest.skip(f"golden values for {name} not generated")
    return np.load(path)


@pytest.mark.parametrize("name", ["ms31_1540", "packed8", "sweep64", "pixtral_tiles16"])
def test_fullsize_against_oracle_samples(name):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gd = _golden(name)
    wl = synth.workload(name)
    assert [tuple(x) for x in gd["image_hw"]] == list(wl.image_hw)
    print(f"[gpu-case] full-size {name}: {wl.n_patches} patches, {wl.layers} layers", flush=True)
    w = synth.make_weights(wl)
    dev_w = T.weights_to_device(w, wl.dtype)
    pix = torch.from_numpy(synth.make_pixels(wl)).cuda()
    rows = torch.from_numpy(gd["rows"]).cuda()
    want = gd["values"].astype(np.float64)
    rms = float(gd["rms"])
    for out_dtype in ("f32", "bf16"):
        tw = T.Tower(T.config_for(wl, out_dtype=out_dtype), dev_w)
        out = tw.forward(pix, wl.image_hw)
        torch.cuda.synchronize()
        assert tuple(out.shape) == tuple(gd["shape"])
        assert torch.isfinite(out.float()).all().item()
        got = out[rows].float().cpu().numpy().astype(np.float64)
        diff = np.abs(got - want)
        plain = float(diff.max() / rms)
        if out_dtype == "bf16":
            diff = np.maximum(diff - BF16_STORE * np.abs(want), 0.0)
        err = float(diff.max() / rms)
        print(f"[gpu-case]   {name} out={out_dtype}: max-abs-err/RMS = {err:.4e}"
              + (f" after the bf16 storage allowance, {plain:.4e} without it" if out_dtype == "bf16" else "")
              + f" over {len(gd['rows'])} rows (RMS {rms:.4f}, tol {TOL})", flush=True)
        tw.close()
        assert plain <= TOL, f"{name} ({out_dtype} output): {plain} > {TOL}"
