"""Seeded synthetic inputs for the tower: image sizes, pixels and weights.

This module is shared by the tests, the benchmark and the oracle's callers.
It holds no tower arithmetic: it draws random numbers, rounds weights to the
nearest bfloat16 (ties to even) when the workload is bf16, applies the image
processor's per-channel normalisation ("Mistral 3", Mistral3ImageProcessor
table), and cuts a large image into 1024x1024 tiles ("Pixtral-12B-2409",
VISION TOKENS paragraph).

Seeds: weights 0, pixels 1, image sizes 2 (packed-8 batch) and 5 (sweep-64).
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Dict, List, Optional, Tuple

import numpy as np

IMAGE_MEAN = (0.48145466, 0.4578275, 0.40821073)
IMAGE_STD = (0.26862954, 0.26130258, 0.27577711)

SEED_WEIGHTS = 0
SEED_PIXELS = 1


@dataclass(frozen=True)
class Workload:
    name: str
    patch: int
    layers: int
    merge: int
    image_hw: Tuple[Tuple[int, int], ...]
    dtype: str = "bf16"  # "bf16" or "f32"
    hidden: int = 1024
    heads: int = 16
    mlp: int = 4096
    out_dim: int = 5120
    rope_theta: float = 1.0e4
    rms_eps: float = 1.0e-5
    tiles_from: Optional[Tuple[int, int]] = None  # (H, W) of the image the tiles are cut from
    note: str = ""
    deep_projector: bool = False  # the deeper projector variant (merge 2)
    rope_interleaved: bool = False  # rotary columns on the odd steps of one ladder

    @property
    def n_patches(self) -> int:
        return sum((h // self.patch) * (w // self.patch) for h, w in self.image_hw)

    @property
    def out_rows(self) -> int:
        if self.merge == 2:
            return sum((h // self.patch // 2) * (w // self.patch // 2) for h, w in self.image_hw)
        return self.n_patches

    @property
    def out_cols(self) -> int:
        return self.out_dim if self.merge == 2 else self.hidden

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


def _sizes(seed: int, n: int, lo_mult: int, hi_mult: int, step: int = 28) -> Tuple[Tuple[int, int], ...]:
    rng = np.random.default_rng(seed)
    ab = rng.integers(lo_mult, hi_mult + 1, size=(n, 2))
    return tuple((int(a) * step, int(b) * step) for a, b in ab)


def workload(name: str) -> Workload:
    """The five named workloads of the tower."""
    if name == "tiny":
        return Workload("tiny", patch=14, layers=1, merge=2, image_hw=((224, 224),), dtype="f32",
                        note="one 224x224 image, 1 layer, fp32")
    if name == "ms31_1540":
        return Workload("ms31_1540", patch=14, layers=24, merge=2, image_hw=((1540, 1540),),
                        note="one 1540x1540 image, 24 layers, bf16")
    if name == "packed8":
        return Workload("packed8", patch=14, layers=24, merge=2, image_hw=_sizes(2, 8, 8, 55),
                        note="8 images, H,W multiples of 28 in [224,1540], bf16")
    if name == "pixtral_tiles16":
        return Workload("pixtral_tiles16", patch=16, layers=24, merge=1,
                        image_hw=tuple([(1024, 1024)] * 16), tiles_from=(4096, 4096),
                        note="4096x4096 image as 16 tiles of 1024x1024, patch 16, no merge, bf16")
    if name == "sweep64":
        return Workload("sweep64", patch=14, layers=24, merge=2, image_hw=_sizes(5, 64, 4, 28),
                        note="64 images, H,W multiples of 28 in [112,784], bf16")
    raise KeyError(name)


WORKLOADS = ("tiny", "ms31_1540", "packed8", "pixtral_tiles16", "sweep64")


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """float32 array -> float32 array holding the nearest bfloat16 values
    (round to nearest, ties to even).  Inputs here are finite."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 values that are exact bfloat16 -> their uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    return (u >> np.uint32(16)).astype(np.uint16)


def make_weights(wl: Workload, seed: int = SEED_WEIGHTS, layers: Optional[int] = None,
                 std: float = 0.02) -> Dict:
    """Matrices N(0, std^2); norm gains 1 + N(0, std^2).  bf16 workloads get
    their matrices rounded to bf16 (gains stay float32).

    Draw order: patch_w, ln_pre, per layer (attn_norm, wq, wk, wv, wo,
    ffn_norm, w_gate, w_up, w_down), merge_w; with the deeper projector
    merge_w is [D][4D] and proj (norm gain, w1 [out_dim][D], w2
    [out_dim][out_dim]) follows.
    """
    n_layers = wl.layers if layers is None else layers
    rng = np.random.default_rng(seed)
    d, f, p = wl.hidden, wl.mlp, wl.patch

    def mat(*shape):
        m = rng.standard_normal(shape, dtype=np.float32) * np.float32(std)
        return round_to_bf16(m) if wl.dtype == "bf16" else m

    def gain():
        return (np.float32(1.0) + rng.standard_normal((d,), dtype=np.float32) * np.float32(std)).astype(np.float32)

    w: Dict = {"patch_w": mat(d, 3, p, p), "ln_pre": gain(), "layers": []}
    for _ in range(n_layers):
        w["layers"].append({
            "attn_norm": gain(),
            "wq": mat(d, d), "wk": mat(d, d), "wv": mat(d, d), "wo": mat(d, d),
            "ffn_norm": gain(),
            "w_gate": mat(f, d), "w_up": mat(f, d), "w_down": mat(d, f),
        })
    if wl.merge == 2 and wl.deep_projector:
        w["merge_w"] = mat(d, 4 * d)
        w["proj"] = {"norm": gain(), "w1": mat(wl.out_dim, d), "w2": mat(wl.out_dim, wl.out_dim)}
    elif wl.merge == 2:
        w["merge_w"] = mat(wl.out_dim, 4 * d)
    return w


def normalise(img: np.ndarray) -> np.ndarray:
    """(x - mean_c) / std_c per channel, float32 ("Mistral 3",
    Mistral3ImageProcessor table)."""
    mean = np.asarray(IMAGE_MEAN, dtype=np.float32)[:, None, None]
    std = np.asarray(IMAGE_STD, dtype=np.float32)[:, None, None]
    return ((img - mean) / std).astype(np.float32)


def split_tiles(img: np.ndarray, tile: int) -> List[np.ndarray]:
    """Cut a C x H x W image into tile x tile pieces, row-major over the tile
    grid ("Pixtral-12B-2409": large images are split into 1024x1024 tiles)."""
    c, h, w = img.shape
    assert h % tile == 0 and w % tile == 0
    return [img[:, r * tile:(r + 1) * tile, q * tile:(q + 1) * tile]
            for r in range(h // tile) for q in range(w // tile)]


def make_pixels(wl: Workload, seed: int = SEED_PIXELS) -> np.ndarray:
    """U[0,1) pixels, normalised, as one flat float32 array holding each
    image's 3 x H x W planes in input order."""
    rng = np.random.default_rng(seed)
    if wl.tiles_from is not None:
        big = normalise(rng.random((3,) + tuple(wl.tiles_from), dtype=np.float32))
        tile = wl.image_hw[0][0]
        parts = split_tiles(big, tile)
        assert len(parts) == len(wl.image_hw)
        return np.concatenate([np.ascontiguousarray(t).reshape(-1) for t in parts])
    parts = [normalise(rng.random((3, h, w), dtype=np.float32)).reshape(-1) for h, w in wl.image_hw]
    return np.concatenate(parts)


def make_u8_images(hw, seed: int = SEED_PIXELS) -> List[np.ndarray]:
    """Uniform uint8 H x W x 3 (RGB, channel fastest) images of the given
    source sizes, drawn in input order."""
    rng = np.random.default_rng(seed)
    return [rng.integers(0, 256, size=(int(h), int(w), 3), dtype=np.uint8) for h, w in hw]


def oracle_weights(w: Dict) -> Dict:
    """The same weights as float64 arrays (what the oracle consumes)."""
    out = {"patch_w": w["patch_w"].astype(np.float64), "ln_pre": w["ln_pre"].astype(np.float64),
           "layers": [{k: v.astype(np.float64) for k, v in lw.items()} for lw in w["layers"]]}
    if "merge_w" in w:
        out["merge_w"] = w["merge_w"].astype(np.float64)
    if "proj" in w:
        out["proj"] = {k: v.astype(np.float64) for k, v in w["proj"].items()}
    return out
