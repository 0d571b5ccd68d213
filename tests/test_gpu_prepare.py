"""GPU checks of the prepared weight copies (pv_tower_prepare) and of the
forward's upload ring, through the C ABI.

Bars: a prepared tower's output is bit-equal to the same tower deriving its
weight copies per call (the same kernels compute the same copies); with the
copies prepared a forward launches no weight-copy kernel (per-class launch
counts); forwards of different batches enqueued back to back without any
synchronisation each equal the same forward run alone; the host enqueues
forwards ahead of the GPU (the upload ring never waits for a kernel).
Inputs: the seeded synthetic ones of vlm_vision_encoder_amd.synth.
"""
import time

import numpy as np
import pytest

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


@pytest.mark.parametrize("flags", [0, T.PV_FLAG_FP8])
def test_prepared_equals_per_call_copies(flags):
    torch = _torch()
    wl = synth.Workload("prep", patch=14, layers=3, merge=2, image_hw=((448, 392), (224, 280), (84, 140)),
                        dtype="bf16")
    say(f"prepared vs per-call weight copies, flags {flags}, {wl.n_patches} patches")
    w = T.weights_to_device(synth.make_weights(wl), "bf16")
    pix = torch.from_numpy(synth.make_pixels(wl)).cuda()
    cfg = T.config_for(wl, flags=flags)
    a = T.Tower(cfg, w, prepare=True)
    b = T.Tower(cfg, w, prepare=False)
    assert a.plan(wl.image_hw).workspace_bytes < b.plan(wl.image_hw).workspace_bytes
    oa = a.forward(pix, wl.image_hw)
    ob = b.forward(pix, wl.image_hw)
    torch.cuda.synchronize()
    assert torch.equal(oa, ob)
    # launches per class: the prepared tower skips the patch-weight padding
    # and, per block, the fp16 gate, up and down copies (fp8: the seven fp8
    # copies)
    counts = []
    for tw in (a, b):
        tw.set_profiling(True)
        tw.forward(pix, wl.image_hw)
        torch.cuda.synchronize()
        counts.append({k: v[1] for k, v in tw.read_profile(reset=True).items()})
        tw.set_profiling(False)
    say(f"  launches prepared {counts[0]}, per call {counts[1]}")
    assert counts[0]["patch"] == counts[1]["patch"] - 1
    if flags:
        assert counts[0]["qkv"] == counts[1]["qkv"] - wl.layers
    else:
        assert counts[0]["gateup"] == counts[1]["gateup"] - 2 * wl.layers
        assert counts[0]["down"] == counts[1]["down"] - wl.layers
    # detaching returns to the per-call copies, with the same result
    a.unprepare()
    oc = a.forward(pix, wl.image_hw)
    torch.cuda.synchronize()
    assert torch.equal(oc, ob)
    a.close()
    b.close()


def test_back_to_back_forwards_through_the_upload_ring():
    """Twenty forwards of ten different batches (more distinct uploads than
    the ring's 8 slots), enqueued without any synchronisation into separate
    outputs and workspaces, each bit-equal to the same forward run alone."""
    torch = _torch()
    wl = synth.Workload("ring", patch=14, layers=2, merge=2, image_hw=((224, 224),), dtype="bf16")
    say("upload ring: 20 back-to-back forwards of 10 batches")
    w = T.weights_to_device(synth.make_weights(wl), "bf16")
    tw = T.Tower(T.config_for(wl, max_side=308), w)
    batches = [tuple((28 * (2 + i), 28 * (9 - i // 2)) for _ in range(1 + i % 3)) for i in range(10)]
    pix = [torch.from_numpy(synth.make_pixels(wl.with_(image_hw=b))).cuda() for b in batches]
    alone = []
    for b, p in zip(batches, pix):
        alone.append(tw.forward(p, b).clone())
        torch.cuda.synchronize()
    outs, keep = [], []
    s = torch.cuda.current_stream().cuda_stream
    for i in range(20):
        j = (3 * i) % 10
        info = tw.plan(batches[j])
        out = torch.empty((info.out_rows, info.out_cols), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(info.workspace_bytes, dtype=torch.uint8, device="cuda")
        keep.append(ws)
        tw.forward_raw(pix[j].data_ptr(), batches[j], out.data_ptr(), out.shape[0], ws.data_ptr(), ws.numel(), s)
        outs.append((j, out))
    torch.cuda.synchronize()
    for j, out in outs:
        assert torch.equal(out, alone[j])
    tw.close()


def test_host_runs_ahead_of_the_gpu():
    """Ten 1540x1540 forwards (24 blocks): the host finishes enqueueing them
    in well under half the GPU time (the forward never waits on the GPU)."""
    torch = _torch()
    wl = synth.workload("ms31_1540")
    say("host enqueue vs GPU time, 10 forwards at 1540x1540")
    tw = T.Tower(T.config_for(wl), T.weights_to_device(synth.make_weights(wl), "bf16"))
    pix = torch.from_numpy(synth.make_pixels(wl)).cuda()
    info = tw.plan(wl.image_hw)
    out = torch.empty((info.out_rows, info.out_cols), dtype=torch.bfloat16, device="cuda")
    ws = tw.workspace(info.workspace_bytes)
    s = torch.cuda.current_stream().cuda_stream

    def fwd():
        tw.forward_raw(pix.data_ptr(), wl.image_hw, out.data_ptr(), out.shape[0], ws.data_ptr(), ws.numel(), s)

    fwd()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(10):
        fwd()
    t_host = time.perf_counter() - t0
    torch.cuda.synchronize()
    t_all = time.perf_counter() - t0
    say(f"  enqueue {t_host * 1e3:.2f} ms, enqueue + GPU {t_all * 1e3:.2f} ms")
    assert t_host < 0.5 * t_all
    tw.close()


def test_side_stream_argument_without_stream_context():
    """forward(stream=...) with a torch side stream and with its raw handle,
    without entering the stream's context: the output and a workspace grown
    by the call are allocated for that stream, and the results equal the
    same forwards on the current stream."""
    torch = _torch()
    wl = synth.Workload("side", patch=14, layers=2, merge=2, image_hw=((224, 224),), dtype="bf16")
    say("stream= argument on a side stream")
    w = T.weights_to_device(synth.make_weights(wl), "bf16")
    small, big = ((224, 224),), ((448, 392), (84, 140))
    px_s = torch.from_numpy(synth.make_pixels(wl.with_(image_hw=small))).cuda()
    px_b = torch.from_numpy(synth.make_pixels(wl.with_(image_hw=big))).cuda()
    ref = T.Tower(T.config_for(wl, max_side=448), w)
    want_s, want_b = ref.forward(px_s, small), ref.forward(px_b, big)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    for arg in (side, side.cuda_stream):
        tw = T.Tower(T.config_for(wl, max_side=448), w)
        a = tw.forward(px_s, small, stream=arg)
        b = tw.forward(px_b, big, stream=arg)       # grows the workspace on the side stream
        side.synchronize()
        assert torch.equal(a, want_s) and torch.equal(b, want_b)
        tw.close()
    ref.close()
