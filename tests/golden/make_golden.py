"""Writes full-size expected values for the GPU parity tests.

Runs the float64 oracle (and nothing else) over the full workloads of
vlm_vision_encoder_amd.synth and stores, per workload, a seeded sample of
output rows (float32), their row indices, and the RMS of the whole oracle
output.  Usage:

    python tests/golden/make_golden.py [workload ...]

Output: tests/golden/<workload>.npz.  Several minutes per workload.
With ``--fp8`` the oracle runs its fp8 emulation of the four per-block
linear maps (``tower_forward(..., fp8=True)``) and writes
tests/golden/<workload>_fp8.npz (same sampled rows).
"""
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

from oracle import pv_oracle as O  # noqa: E402
from vlm_vision_encoder_amd import synth  # noqa: E402

N_SAMPLE_ROWS = 32
SAMPLE_SEED = 1234
# at least one sampled row in every band of this many consecutive output rows
# of an image: 128 patch rows, or 64 merged rows (a merged row gathers four
# patches, so 64 of them span about 256 patch rows)
BAND_PATCH_ROWS = 128
BAND_MERGED_ROWS = 64


def sample_rows(out_rows: int, image_starts, band: int = BAND_PATCH_ROWS) -> np.ndarray:
    """Per image: its first and last output row and one seeded row in every
    band of `band` consecutive rows; then seeded rows over the whole batch.
    Sorted and unique."""
    rng = np.random.default_rng(SAMPLE_SEED)
    bounds = list(image_starts) + [out_rows]
    fixed = []
    for s, e in zip(bounds[:-1], bounds[1:]):
        if e <= s:
            continue
        fixed += [s, e - 1]
        for b0 in range(s, e, band):
            b1 = min(b0 + band, e)
            fixed.append(int(rng.integers(b0, b1)))
    rest = rng.choice(out_rows, size=min(N_SAMPLE_ROWS, out_rows), replace=False)
    return np.unique(np.array(fixed + list(rest), dtype=np.int64))


def make(name: str, fp8: bool = False) -> str:
    wl = synth.workload(name)
    t0 = time.time()
    w = synth.oracle_weights(synth.make_weights(wl))
    px = synth.make_pixels(wl).astype(np.float64)
    cfg = O.TowerConfig(patch=wl.patch, hidden=wl.hidden, heads=wl.heads, mlp=wl.mlp, layers=wl.layers,
                        merge=wl.merge, out_dim=wl.out_dim, rope_theta=wl.rope_theta, rms_eps=wl.rms_eps)
    res = O.tower_forward(px, wl.image_hw, w, cfg, fp8=fp8)
    out = res["out"]
    maps = res["maps"]
    if wl.merge == 2:
        starts = np.cumsum([0] + [(h // wl.patch // 2) * (ww // wl.patch // 2) for h, ww in wl.image_hw])[:-1]
    else:
        starts = maps["cu_seqlens"][:-1]
    rows = sample_rows(out.shape[0], [int(x) for x in starts],
                       BAND_MERGED_ROWS if wl.merge == 2 else BAND_PATCH_ROWS)
    path = os.path.join(HERE, f"{name}_fp8.npz" if fp8 else f"{name}.npz")
    np.savez_compressed(path, rows=rows, values=out[rows].astype(np.float32),
                        rms=np.float64(np.sqrt(np.mean(out * out))), shape=np.array(out.shape, np.int64),
                        image_hw=np.array(wl.image_hw, np.int64))
    print(f"{name}: out {out.shape}, rms {np.sqrt(np.mean(out * out)):.6f}, {len(rows)} rows sampled, "
          f"{time.time() - t0:.0f} s -> {path}", flush=True)
    return path


if __name__ == "__main__":
    args = [a for a in sys.argv[1:] if a != "--fp8"]
    names = args or ["ms31_1540", "packed8", "sweep64", "pixtral_tiles16"]
    for n in names:
        make(n, fp8="--fp8" in sys.argv[1:])
