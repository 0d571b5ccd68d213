"""GPU parity of the masked scatter of merged image embeddings into a
text-embedding sequence, against oracle.masked_scatter (a plain loop).  A
copy: bit-exact."""
import numpy as np
import pytest

from oracle import pv_oracle as O
from vlm_vision_encoder_amd import synth
from vlm_vision_encoder_amd import tower as T

pytestmark = pytest.mark.gpu

IMAGE_TOKEN = 10


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)


def _ids(rng, seq_len, n_placeholders):
    ids = rng.integers(11, 131072, size=seq_len).astype(np.int32)
    pos = rng.choice(seq_len, size=n_placeholders, replace=False)
    ids[pos] = IMAGE_TOKEN
    return ids


def _run(ids, img, txt):
    torch = _torch()
    d_ids = torch.from_numpy(ids).cuda()
    d_img = torch.from_numpy(img).cuda()
    d_txt = torch.from_numpy(txt).cuda()
    st = T.scatter_image_embeddings(d_ids, d_img, d_txt, IMAGE_TOKEN)
    torch.cuda.synchronize()
    return d_txt.cpu().numpy(), int(st.item())


@pytest.mark.parametrize("seq_len,rows,dim,dtype", [
    (5000, 3025, 5120, np.uint16),     # one 1540^2 image's merged tokens, bf16 bits
    (200_003, 7136, 256, np.uint16),   # long sequence: many positions per scan thread
    (777, 100, 64, np.float32),        # fp32 rows of 256 bytes
    (64, 0, 5120, np.uint16),          # no image rows, no placeholders
])
def test_scatter_matches_oracle_bitwise(seq_len, rows, dim, dtype):
    rng = np.random.default_rng(seq_len + rows)
    ids = _ids(rng, seq_len, rows)
    img = rng.integers(0, 65535, size=(rows, dim)).astype(dtype) if dtype == np.uint16 else \
        rng.standard_normal((rows, dim)).astype(dtype)
    txt = rng.integers(0, 65535, size=(seq_len, dim)).astype(dtype) if dtype == np.uint16 else \
        rng.standard_normal((seq_len, dim)).astype(dtype)
    say(f"scatter S={seq_len} rows={rows} dim={dim} {np.dtype(dtype).name}")
    got, status = _run(ids, img, txt)
    want, ok = O.masked_scatter(ids, img, txt, IMAGE_TOKEN)
    assert ok and status == 0
    assert np.array_equal(got, want)


@pytest.mark.parametrize("extra", [+5, -5])
def test_scatter_count_mismatch_sets_status(extra):
    rng = np.random.default_rng(3)
    rows, dim = 50, 128
    ids = _ids(rng, 400, rows + extra)
    img = rng.standard_normal((rows, dim)).astype(np.float32)
    txt = rng.standard_normal((400, dim)).astype(np.float32)
    say(f"scatter count mismatch {extra:+d}")
    got, status = _run(ids, img, txt)
    want, ok = O.masked_scatter(ids, img, txt, IMAGE_TOKEN)
    assert not ok and status == 1
    assert np.array_equal(got, want)


def test_tower_output_into_text_sequence():
    """Two images through the bf16 tower, their merged rows scattered into a
    sequence whose placeholder runs follow the per-image token counts."""
    torch = _torch()
    base = synth.workload("ms31_1540")
    wl = base.with_(name="scatter", image_hw=((224, 224), (112, 280)), layers=1)
    w = synth.make_weights(wl)
    tw = T.Tower(T.config_for(wl), T.weights_to_device(w, wl.dtype))
    pix = torch.from_numpy(synth.make_pixels(wl)).cuda()
    out = tw.forward(pix, wl.image_hw)
    torch.cuda.synchronize()
    counts = [(h // 28) * (ww // 28) for h, ww in wl.image_hw]
    ids = np.concatenate([np.full(3, 1, np.int32), np.full(counts[0], IMAGE_TOKEN, np.int32),
                          np.full(4, 2, np.int32), np.full(counts[1], IMAGE_TOKEN, np.int32),
                          np.full(2, 3, np.int32)])
    txt = torch.zeros((ids.size, out.shape[1]), dtype=out.dtype, device="cuda")
    say(f"tower output into a {ids.size}-token sequence")
    st = T.scatter_image_embeddings(torch.from_numpy(ids).cuda(), out, txt, IMAGE_TOKEN)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    got = txt.float().cpu().numpy()
    want, ok = O.masked_scatter(ids, out.float().cpu().numpy(), np.zeros(got.shape), IMAGE_TOKEN)
    assert ok and np.array_equal(got, want)
    tw.close()
