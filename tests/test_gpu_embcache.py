"""GPU tests of the multimodal embeddings cache and the content keys, through
the C ABI.

Bar: keys are integer work, bit-exact against the oracle's loop over Python
integers; a cached forward's output is bit-equal to the plain uint8 forward
of the same images in the same order, whatever came from the cache (hits,
repeats inside a call, recomputation after eviction); hit flags and counters
are exact.  The side-stream case runs the tower on its own stream and must
equal the default-stream result bit for bit.
Inputs: seeded uniform uint8 images (vlm_vision_encoder_amd.synth).
"""
import numpy as np
import pytest

from oracle import pv_oracle as O
from vlm_vision_encoder_amd import synth
from vlm_vision_encoder_amd import tower as T

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)


def upload(images):
    torch = _torch()
    return torch.from_numpy(np.concatenate([im.reshape(-1) for im in images])).cuda()


def as_u64(t):
    return [(int(a) & 0xFFFFFFFFFFFFFFFF, int(b) & 0xFFFFFFFFFFFFFFFF) for a, b in t.cpu().tolist()]


def test_keys_match_oracle():
    """Odd sizes put most images at offsets that are not multiples of 4 or 8
    in the packed buffer (the unaligned word assembly)."""
    _torch()
    hw = [(1, 1), (5, 7), (3, 3), (17, 29), (64, 64), (2, 1), (1, 2), (41, 37), (120, 90)]
    say(f"image keys {hw}")
    images = synth.make_u8_images(hw, seed=61)
    images[6] = images[5].reshape(1, 2, 3)  # same bytes as image 5, other shape
    got = as_u64(T.image_keys_u8(upload(images), hw))
    want = [O.image_key(im) for im in images]
    assert got == want
    assert len(set(got)) == len(got)


def small_tower(dtype="bf16", max_side=112):
    wl = synth.Workload("cache-small", patch=14, layers=2, merge=2, image_hw=((28, 28),), dtype=dtype,
                        hidden=256, heads=4, mlp=512, out_dim=384)
    return T.Tower(T.config_for(wl, max_side=max_side), T.weights_to_device(synth.make_weights(wl), dtype))


def plain(tower, images, hw):
    torch = _torch()
    out = tower.forward_u8(upload(images), hw).clone()
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_cached_forward_equals_plain_forward(dtype):
    torch = _torch()
    say(f"embeddings cache {dtype}: miss, hit, mixed, repeats")
    tower = small_tower(dtype)
    imgs = synth.make_u8_images([(100, 150), (61, 33), (300, 90), (20, 20)], seed=62)
    A, B, Cc, D = imgs
    hw = {id(A): (100, 150), id(B): (61, 33), id(Cc): (300, 90), id(D): (20, 20)}
    cache = T.EmbCache(tower, capacity_rows=4096)

    def run(batch, want_hits):
        sizes = [hw[id(im)] for im in batch]
        out, hits = cache.forward(upload(batch), sizes)
        torch.cuda.synchronize()
        assert hits == want_hits
        assert torch.equal(out, plain(tower, batch, sizes))

    run([A, B], [0, 0])
    run([B, Cc, A], [1, 0, 1])
    run([D, D, A], [0, 1, 1])
    st = cache.stats()
    assert st["entries"] == 4 and st["hits"] == 4 and st["misses"] == 4
    cache.close()
    tower.close()


def test_cache_eviction_and_caller_keys():
    torch = _torch()
    say("embeddings cache: eviction in a small ring, caller keys")
    tower = small_tower()
    hw = [(112, 112), (112, 56), (56, 112)]
    imgs = synth.make_u8_images(hw, seed=63)
    rows = [(h // 28) * (w // 28) for h, w in hw]  # 16, 8, 8 merged tokens
    cache = T.EmbCache(tower, capacity_rows=rows[0] + rows[1] + 4)
    out, hits = cache.forward(upload(imgs[:2]), hw[:2])
    assert hits == [0, 0]
    # the third image does not fit after the first two (rows [0, 24) of 28):
    # its run wraps to row 0 and evicts the first image
    out, hits = cache.forward(upload(imgs[2:]), hw[2:])
    assert hits == [0] and cache.stats()["entries"] == 2
    # caller keys (the oracle's, equal to the device's): image 0 is a miss,
    # 1 and 2 are hits; the 16-row run for image 0 at rows [8, 24) evicts
    # image 1, whose copy was enqueued before the forward that overwrites it
    keys = [O.image_key(im) for im in imgs]
    out, hits = cache.forward(upload(imgs), hw, keys=keys)
    torch.cuda.synchronize()
    assert hits == [0, 1, 1]
    assert torch.equal(out, plain(tower, imgs, hw))
    st = cache.stats()
    assert st["entries"] == 2 and st["rows_used"] == rows[2] + rows[0] and st["capacity_rows"] == 28
    # misses that need more rows than the cache holds are refused
    big = synth.make_u8_images([(112, 112)] * 2, seed=64)
    with pytest.raises(T.PvError) as e:
        cache.forward(upload(big), [(112, 112)] * 2)
    assert e.value.status == -3
    cache.close()
    tower.close()


def test_side_stream_forward_equals_default_stream():
    """The tower enqueued on its own stream while other work runs on the
    default stream; the consumer waits on an event."""
    torch = _torch()
    say("encoder on a side stream")
    tower = small_tower()
    hw = [(300, 200), (90, 90)]
    images = upload(synth.make_u8_images(hw, seed=65))
    want = plain(tower, synth.make_u8_images(hw, seed=65), hw)
    side = torch.cuda.Stream()
    x = torch.randn(2048, 2048, device="cuda")
    done = torch.cuda.Event()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        out = tower.forward_u8(images, hw, stream=side.cuda_stream)
        done.record(side)
    y = x @ x  # default-stream work meanwhile
    torch.cuda.current_stream().wait_event(done)
    got = out.clone()
    torch.cuda.synchronize()
    assert torch.isfinite(y).all()
    assert torch.equal(got, want)
    tower.close()


def test_fullsize_photo_hit_equals_miss():
    torch = _torch()
    say("full size: 4096x4096 photo through the cache (miss, then hit)")
    wl = synth.workload("ms31_1540")
    tower = T.Tower(T.preset("mistral3"), T.weights_to_device(synth.make_weights(wl), "bf16"))
    src = [(4096, 4096)]
    img = upload(synth.make_u8_images(src, seed=66))
    cache = T.EmbCache(tower, capacity_rows=3025)
    a, h1 = cache.forward(img, src)
    a = a.clone()
    b, h2 = cache.forward(img, src)
    torch.cuda.synchronize()
    assert h1 == [0] and h2 == [1]
    assert torch.equal(a, b)
    assert torch.equal(a, tower.forward_u8(img, src))
    cache.close()
    tower.close()
