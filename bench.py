"""Throughput benchmark of the vision tower on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload ms31_1540]

One step = one full tower forward (patch embedding, 24 blocks, 2x2 merge +
projection) over one batch of seeded synthetic images already resident in HBM.
Prints one JSON line with patches/s (value), merged tokens/s, the fraction of
bf16 MFMA peak of the whole forward, the roofline of the dominant kernel
(timed live with HIP events on the launch stream) and the float64 CPU oracle
timed on a bounded sample of the same workload on this host's cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
FP32_PEAK_TFLOPS = 157.3
HBM_PEAK_GBS = 8000.0

CLASS_FOR_ROOFLINE = ("attn", "gateup", "down", "qkv", "oproj", "merge", "patch")


def flops_by_class(wl):
    """Algorithmic (unpadded) flops of one forward, by kernel class."""
    D, F, L = wl.hidden, wl.mlp, wl.layers
    N = wl.n_patches
    p = wl.patch
    lens = [(h // p) * (w // p) for h, w in wl.image_hw]
    out = {
        "patch": 2.0 * N * D * 3 * p * p,
        "qkv": L * 2.0 * N * D * 3 * D,
        "attn": L * sum(4.0 * n * n * D for n in lens),
        "oproj": L * 2.0 * N * D * D,
        "gateup": L * 2.0 * N * D * 2 * F,
        "down": L * 2.0 * N * F * D,
        "merge": 2.0 * wl.out_rows * 4 * D * wl.out_dim if wl.merge == 2 else 0.0,
    }
    return out


def memory_bound_bytes(wl):
    """Algorithmic HBM bytes of one forward's memory-bound passes, by kernel
    class (bf16 tower).
      norm:     the first pass reads X (4 B) and writes h (4 B) and y (2 B);
                each later attention norm reads h (4 B), writes y (2 B)
      norm_mlp: each MLP norm reads h (4 B), writes y in fp16 (2 B)
      operand:  im2col split: the pixels read once (3 p^2 fp32 per patch),
                2 Kp bf16 written per patch; the merger's input split: 4 B
                read, 2 B (bf16) + 1/2 B (fp4 low part) + one scale byte per
                32 values written (merge), or the fp32 -> bf16 output copy:
                4 + 2 B (no merge)."""
    import math
    N, D, L, p = wl.n_patches, wl.hidden, wl.layers, wl.patch
    if wl.dtype != "bf16" or L == 0:
        return {}
    kp = math.ceil(3 * p * p / 64) * 64
    return {
        "norm": N * D * (10 + (L - 1) * 6),
        "norm_mlp": N * D * L * 6,
        "operand": N * (3 * p * p * 4 + 2 * kp * 2) + N * D * ((6 + 0.5 + 1 / 32) if wl.merge == 2 else 6),
    }


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(wl, weights, pixels, full=False, log=None):
    """The float64 oracle on the GPU host's cores.  full=True: the whole
    forward, every block (a progress line per block); else a bounded sample:
    patch embedding + ln_pre + ONE block + the merge projection of the full
    batch, the forward time extrapolated as embed + L x block + merge."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import pv_oracle as O
    from vlm_vision_encoder_amd import synth

    n_blocks = wl.layers if full else min(1, wl.layers)
    ow = synth.oracle_weights({"patch_w": weights["patch_w"], "ln_pre": weights["ln_pre"],
                               "layers": weights["layers"][:n_blocks], **({"merge_w": weights["merge_w"]}
                                                                          if "merge_w" in weights else {})})
    px = pixels.astype(np.float64)
    t0 = time.perf_counter()
    x = O.patch_embed(px, wl.image_hw, ow["patch_w"], wl.patch)
    h = O.rms_norm(x, ow["ln_pre"], wl.rms_eps)
    t1 = time.perf_counter()
    maps = O.plan_maps(wl.image_hw, wl.patch, wl.merge)
    for i, lw in enumerate(ow["layers"]):
        y = O.rms_norm(h, lw["attn_norm"], wl.rms_eps)
        q = O.rope_2d(y @ lw["wq"].T, maps["patch_rc"], wl.heads, wl.rope_theta)
        k = O.rope_2d(y @ lw["wk"].T, maps["patch_rc"], wl.heads, wl.rope_theta)
        v = y @ lw["wv"].T
        h = h + O.attention(q, k, v, maps["cu_seqlens"], wl.heads) @ lw["wo"].T
        y = O.rms_norm(h, lw["ffn_norm"], wl.rms_eps)
        h = h + O.swiglu_mlp(y, lw["w_gate"], lw["w_up"], lw["w_down"])
        if log:
            log(f"oracle {wl.name}: block {i + 1}/{len(ow['layers'])} done, {time.perf_counter() - t0:.1f} s")
    t2 = time.perf_counter()
    if wl.merge == 2:
        O.merge_project(h, maps["merge_src"], ow["merge_w"])
    t3 = time.perf_counter()
    if full:
        fwd_s = t3 - t0
        sample = (f"float64 numpy oracle: the whole forward of the {wl.name} batch ({wl.n_patches} patches, "
                  f"{wl.layers} blocks), {fwd_s:.1f} s measured")
    else:
        fwd_s = (t1 - t0) + wl.layers * (t2 - t1) / max(1, n_blocks) + (t3 - t2)
        sample = (f"float64 numpy oracle: patch embedding + ln_pre + 1 of {wl.layers} blocks + merge projection "
                  f"of the full {wl.name} batch ({wl.n_patches} patches), timed {t3 - t0:.1f} s; forward time "
                  f"extrapolated as embed + {wl.layers} x block + merge = {fwd_s:.1f} s")
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {
        "value": wl.n_patches / fwd_s,
        "unit": "patches/s",
        "cores": threads,
        "kind": "oracle",
        "sample": sample,
        "extrapolated": not full,
        "merged_tokens_per_s": wl.out_rows / fwd_s,
        "host_cpus": os.cpu_count(),
        "cpu_model": cpu_model(),
    }


def copy_probe(mib):
    import torch
    n = mib * (1 << 20) // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(5):
        torch.mul(x, 1.0, out=y)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n * 4, "copy_probe_bytes_written": n * 4, "launches": 5}), flush=True)


def mfma_ceiling(sizes=(8192, 16384)):
    """The vendor library's bf16 GEMM (torch.matmul -> hipBLASLt) on square
    products, operands drawn from N(0, 1) and, with the same instructions,
    all zeros and all ones: what fraction of the 2.5 PF figure the chip
    sustains on bf16 MFMA work with and without data switching in its
    operands (HIP events around the timed calls)."""
    import torch
    out = []
    for n in sizes:
        g = torch.Generator(device="cuda").manual_seed(0)
        a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16, generator=g)
        b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16, generator=g)
        for name, (x, y) in (("randn", (a, b)), ("zeros", (torch.zeros_like(a), torch.zeros_like(b))),
                             ("ones", (torch.ones_like(a), torch.ones_like(b)))):
            reps = 20 if n > 8192 else 50
            for _ in range(5):
                torch.matmul(x, y)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                torch.matmul(x, y)
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            tf = 2.0 * n ** 3 / ms / 1e9
            rec = {"n": n, "operands": name, "ms": round(ms, 4), "tflops": round(tf, 1),
                   "frac_of_bf16_peak": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)}
            out.append(rec)
            print(json.dumps(rec), flush=True)
        del a, b
    return out


KERNEL_MATCH = {"attn": ("attn_bf16_kernel", "attn_bf16.hip")}


def pmc_summary(args):
    """Writes profiles/traffic_<class>_<workload>.json from rocprofv3 --pmc CSV
    outputs (FETCH_SIZE and WRITE_SIZE, KiB per dispatch) of the tower kernel
    and of the copy probe: bytes = counter KiB * 1024 * (known copy bytes /
    the copy probe's counter bytes)."""
    import csv
    import statistics

    def per_dispatch(path, needle):
        with open(path) as f:
            vals = [float(r["Counter_Value"]) for r in csv.DictReader(f) if needle in r["Kernel_Name"]]
        if not vals:
            raise SystemExit(f"no dispatch of {needle} in {path}")
        return statistics.mean(vals), len(vals)

    kcls, wname = args.pmc_summary
    needle, src = KERNEL_MATCH[kcls]
    copy_bytes = args.copy_probe_mib * (1 << 20)
    f_kib, nf = per_dispatch(args.pmc_fetch, needle)
    w_kib, nw = per_dispatch(args.pmc_write, needle)
    cf_kib, _ = per_dispatch(args.pmc_copy_fetch, "MulFunctor")
    cw_kib, _ = per_dispatch(args.pmc_copy_write, "MulFunctor")
    f_scale, w_scale = copy_bytes / (cf_kib * 1024), copy_bytes / (cw_kib * 1024)
    fetch_b, write_b = f_kib * 1024 * f_scale, w_kib * 1024 * w_scale
    if args.attn_q_tile is None:
        raise SystemExit("--attn-q-tile (the work-item size of the measured run) is required")
    out = {"kernel": needle, "workload": wname, "source": src, "sources_sha256": traffic_sources_sha256(),
           "attn_q_tile": args.attn_q_tile,
           "fetch_scale_note": "the copy probe's FETCH_SIZE per byte; assumes the kernel's request-size mix "
                               "reads like the copy kernel's",
           "fetch_kib_per_dispatch": f_kib, "write_kib_per_dispatch": w_kib, "dispatches": [nf, nw],
           "copy_probe_bytes": copy_bytes, "copy_fetch_kib": cf_kib, "copy_write_kib": cw_kib,
           "fetch_scale": f_scale, "write_scale": w_scale,
           "hbm_fetch_bytes_per_dispatch": fetch_b, "hbm_write_bytes_per_dispatch": write_b,
           "hbm_bytes_per_dispatch": fetch_b + write_b}
    path = os.path.join(ROOT, "profiles", f"traffic_{kcls}_{wname}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))


def time_scatter(out, wl, stream, reps=20):
    """The masked scatter of the merged rows into a text sequence of the
    same tokens plus 1,024 text tokens (HIP events around `reps` calls on the
    launch stream).  Algorithmic bytes: each image row read and written once,
    each token id read once."""
    import numpy as np
    import torch

    from vlm_vision_encoder_amd import tower as T
    rng = np.random.default_rng(9)
    S = out.shape[0] + 1024
    ids = rng.integers(11, 131072, size=S).astype(np.int32)
    ids[rng.choice(S, size=out.shape[0], replace=False)] = 10
    d_ids = torch.from_numpy(ids).cuda()
    txt = torch.zeros((S, out.shape[1]), dtype=out.dtype, device="cuda")
    T.scatter_image_embeddings(d_ids, out, txt, 10)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        st = T.scatter_image_embeddings(d_ids, out, txt, 10)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    nbytes = 2 * out.numel() * out.element_size() + S * 4
    return {"seq_len": S, "image_rows": int(out.shape[0]), "ms": round(ms, 5), "status": int(st.item()),
            "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1), "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def time_u8_input(tw, wl, out, ws, stream, f32_patch_ms, reps=5):
    """The uint8 input path on a 4096x4096 photo (resized to the workload's
    1540x1540, or cut into the Pixtral workload's 16 tiles of 1024x1024):
    the whole forward from uint8 (HIP events around `reps`
    calls), its patch-embedding and operand kernel classes (fused resize +
    normalise + hi|lo im2col, GEMM, the final residual's split) beside the
    float path's, and the
    standalone preprocessing into fp32 planes.  Algorithmic bytes of the
    standalone pass: the source image read once plus the planes written."""
    import torch

    from vlm_vision_encoder_amd import synth
    from vlm_vision_encoder_amd import tower as T
    src = [(4096, 4096)]
    if wl.tiles_from is not None:  # Pixtral: the photo cut into tiles, capped at the workload's tile count
        cap = len(wl.image_hw)
        info, layout = tw.plan_tiles_u8(src, cap)
        tiles = [(min(1024, layout[0][0] - a * 1024), min(1024, layout[0][1] - b * 1024))
                 for a in range(layout[0][2]) for b in range(layout[0][3])]
        if tiles != list(wl.image_hw):
            return None
        tgt = [(layout[0][0], layout[0][1])]
        fwd = lambda: tw.forward_tiles_u8(img, src, cap, out=out, stream=sptr)  # noqa: E731
    else:
        info, tgt = tw.plan_u8(src)
        if tgt != list(wl.image_hw):
            return None
        fwd = lambda: tw.forward_u8(img, src, out=out, stream=sptr)  # noqa: E731
    img = torch.from_numpy(synth.make_u8_images(src, seed=3)[0].reshape(-1)).cuda()
    sptr = stream.cuda_stream
    fwd()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        fwd()
    e1.record(stream)
    torch.cuda.synchronize()
    fwd_ms = e0.elapsed_time(e1) / reps
    tw.set_profiling(True)
    fwd()
    torch.cuda.synchronize()
    prof = tw.read_profile(reset=True)
    tw.set_profiling(False)
    planes = torch.empty(3 * tgt[0][0] * tgt[0][1], dtype=torch.float32, device="cuda")
    T.preprocess_u8(img, src, tgt, out=planes)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        T.preprocess_u8(img, src, tgt, out=planes)
    e1.record(stream)
    torch.cuda.synchronize()
    pre_ms = e0.elapsed_time(e1) / reps
    nbytes = img.numel() + planes.numel() * 4
    return {"source": "4096x4096 uint8 RGB", "target": list(tgt[0]),
            "tiles": len(wl.image_hw) if wl.tiles_from is not None else None, "forward_ms": round(fwd_ms, 4),
            "patches_per_s": round(info.n_patches / (fwd_ms * 1e-3), 1),
            "patch_and_operand_ms": round(prof["patch"][0] + prof["operand"][0], 5),
            "patch_and_operand_ms_float_input": round(f32_patch_ms, 5),
            "preprocess_planes_ms": round(pre_ms, 5),
            "preprocess_planes_gbs": round(nbytes / (pre_ms * 1e-3) / 1e9, 1),
            "preprocess_planes_hbm_frac": round(nbytes / (pre_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def time_embcache(tw, wl, stream, reps=5):
    """The embeddings cache on the 4096x4096 photo: a miss (keys hashed on
    the GPU and read back, tower forward into the cache, copy out) and a hit
    (keys, copy out), each timed on the host around the synchronising call;
    and the key kernel alone (HIP events), whose algorithmic bytes are the
    photo's bytes read once."""
    import torch

    from vlm_vision_encoder_amd import synth
    from vlm_vision_encoder_amd import tower as T
    if wl.tiles_from is not None or len(wl.image_hw) != 1:
        return None
    src = [(4096, 4096)]
    info, tgt = tw.plan_u8(src)
    if tgt != list(wl.image_hw):
        return None
    img = torch.from_numpy(synth.make_u8_images(src, seed=3)[0].reshape(-1)).cuda()
    cache = T.EmbCache(tw, capacity_rows=info.out_rows)
    sptr = stream.cuda_stream
    out, _ = cache.forward(img, src, stream=sptr)
    miss_ms, hit_ms = [], []
    for _ in range(reps):
        cache.clear()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        _, h = cache.forward(img, src, out=out, stream=sptr)
        torch.cuda.synchronize()
        miss_ms.append((time.perf_counter() - t0) * 1e3)
        assert h == [0]
        t0 = time.perf_counter()
        _, h = cache.forward(img, src, out=out, stream=sptr)
        torch.cuda.synchronize()
        hit_ms.append((time.perf_counter() - t0) * 1e3)
        assert h == [1]
    T.image_keys_u8(img, src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        T.image_keys_u8(img, src)
    e1.record(stream)
    torch.cuda.synchronize()
    keys_ms = e0.elapsed_time(e1) / reps
    cache.close()
    return {"source": "4096x4096 uint8 RGB", "rows": int(info.out_rows), "miss_ms": round(min(miss_ms), 4),
            "hit_ms": round(min(hit_ms), 4), "keys_ms": round(keys_ms, 5),
            "keys_gbs": round(img.numel() / (keys_ms * 1e-3) / 1e9, 1),
            "keys_hbm_frac": round(img.numel() / (keys_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def time_fp8_variant(wl, dev_w, pix, stream, reps=5):
    """The fp8 variant (PV_FLAG_FP8) of the same tower on the same input:
    forward time (HIP events around `reps` calls) and per-class times.  A
    different precision: reported beside the bf16 figure, never as it."""
    import torch

    from vlm_vision_encoder_amd import tower as T
    if wl.dtype != "bf16":
        return None
    tw8 = T.Tower(T.config_for(wl, flags=T.PV_FLAG_FP8), dev_w)
    info = tw8.plan(wl.image_hw)
    out = torch.empty((info.out_rows, info.out_cols), dtype=torch.bfloat16, device="cuda")
    sptr = stream.cuda_stream
    tw8.forward(pix, wl.image_hw, out=out, stream=sptr)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        tw8.forward(pix, wl.image_hw, out=out, stream=sptr)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    tw8.set_profiling(True)
    tw8.forward(pix, wl.image_hw, out=out, stream=sptr)
    torch.cuda.synchronize()
    prof = tw8.read_profile(reset=True)
    tw8.set_profiling(False)
    tw8.close()
    return {"dtype": "fp8 e4m3 (per-block linear maps), bf16 elsewhere", "ms_per_step": round(ms, 4),
            "patches_per_s": round(wl.n_patches / (ms * 1e-3), 1),
            "class_ms": {k: round(v[0], 4) for k, v in prof.items() if v[1]}}


def source_sha256(path):
    import hashlib
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


# sources whose change makes a stored traffic measurement stale: the kernel,
# and the planner that chooses its work-item size
TRAFFIC_SOURCES = ("attn_bf16.hip", "kernels.h", "plan.cpp")


def traffic_sources_sha256():
    return {f: source_sha256(os.path.join(ROOT, "vlm_vision_encoder_amd", "csrc", f)) for f in TRAFFIC_SOURCES}


def measured_traffic(kernel_class, wl, attn_q_tile):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3
    counter summary (FETCH_SIZE + WRITE_SIZE per dispatch, each scaled by what
    the same counter reads for a copy kernel of known size), or None when no
    summary exists for this kernel and workload, when the kernel, its launch
    header or the planner has changed since the counters were taken, or when
    this run's attention work-item size differs from the measured one."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel_class}_{wl.name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("sources_sha256") != traffic_sources_sha256() or t.get("attn_q_tile") != attn_q_tile:
        return None
    return float(t["hbm_bytes_per_dispatch"])


def run_workload(wl, dev_w, weights, pixels, args, log, headline):
    """Times one workload: `args.steps` forwards after `args.warmup` (HIP
    events on the launch stream), per-class kernel times over
    `args.profile_steps` more, the dominant kernel's roofline, the memory-bound
    passes' HBM fractions; the headline also times the extra legs."""
    import torch

    from vlm_vision_encoder_amd import tower as T

    tw = T.Tower(T.config_for(wl), dev_w)
    pix = torch.from_numpy(pixels).cuda()
    info = tw.plan(wl.image_hw)
    out = torch.empty((info.out_rows, info.out_cols), dtype=torch.bfloat16 if wl.dtype == "bf16" else torch.float32,
                      device="cuda")
    ws = tw.workspace(info.workspace_bytes)
    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream

    def step():
        tw.forward_raw(pix.data_ptr(), wl.image_hw, out.data_ptr(), out.shape[0], ws.data_ptr(), ws.numel(), sptr)

    steps = args.steps if headline else args.sub_steps
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # an event after every step as well (per-step median and spread)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    ev0.record(stream)
    for i in range(steps):
        step()
        marks[i].record(stream)
    ev1.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall0
    ms_step = ev0.elapsed_time(ev1) / steps
    per_step = sorted([ev0.elapsed_time(marks[0])] + [marks[i - 1].elapsed_time(marks[i])
                                                      for i in range(1, steps)])
    step_stats = {"median_ms": round(per_step[len(per_step) // 2], 4), "min_ms": round(per_step[0], 4),
                  "max_ms": round(per_step[-1], 4)}
    log(f"{wl.name}: timed {steps} steps: {ms_step:.3f} ms/step (wall {t_wall * 1e3 / steps:.3f} ms/step)")
    assert torch.isfinite(out.float()).all().item(), "non-finite output"

    # per-kernel-class times, HIP events around each launch on the same stream
    fl = flops_by_class(wl)
    mb = memory_bound_bytes(wl)
    total_flops = sum(fl.values())
    bf = wl.dtype == "bf16"
    peak = MFMA_BF16_PEAK_TFLOPS if bf else FP32_PEAK_TFLOPS
    kernels, roofline, memory_bound = {}, None, {}
    if args.profile_steps > 0:
        tw.set_profiling(True)
        for _ in range(args.profile_steps):
            step()
        torch.cuda.synchronize()
        prof = tw.read_profile(reset=True)
        tw.set_profiling(False)
        for k, (ms, cnt) in prof.items():
            if cnt == 0:
                continue
            per_launch_ms = ms / cnt
            launches_per_fwd = cnt / args.profile_steps
            d = {"avg_ms": round(per_launch_ms, 5), "launches_per_step": launches_per_fwd,
                 "ms_per_step": round(ms / args.profile_steps, 4)}
            if fl.get(k):
                d["tflops"] = round(fl[k] / (ms / args.profile_steps) / 1e9, 1)
            if mb.get(k):
                d["gbs"] = round(mb[k] / (ms / args.profile_steps) / 1e6, 1)
                d["hbm_frac"] = round(d["gbs"] / HBM_PEAK_GBS, 4)
                memory_bound[k] = {"bytes_per_step": mb[k], "ms_per_step": d["ms_per_step"], "gbs": d["gbs"],
                                   "hbm_frac": d["hbm_frac"]}
            kernels[k] = d
            rate = (f"{d['tflops']} TFLOP/s" if "tflops" in d else "") + (f"{d['gbs']} GB/s" if "gbs" in d else "")
            log(f"  {k:8s} {per_launch_ms:9.4f} ms x {launches_per_fwd:5.1f}/step  {rate}")
        dom = max((k for k in fl if fl[k] > 0 and k in kernels), key=lambda k: kernels[k]["ms_per_step"])
        dom_ms = kernels[dom]["avg_ms"]
        dom_flops_launch = fl[dom] / kernels[dom]["launches_per_step"]
        achieved = dom_flops_launch / (dom_ms * 1e-3) / 1e12
        roofline = {"bound": "mfma" if bf else "alu", "kernel": dom, "achieved": round(achieved, 1), "peak": peak,
                    "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                    "traffic": measured_traffic(dom, wl, info.attn_q_tile) if dom == "attn" else None,
                    "flops_per_launch": dom_flops_launch, "avg_launch_ms": dom_ms}

    res = {
        "workload": wl.name, "ms_per_step": round(ms_step, 4), "step_ms": step_stats,
        "patches_per_s": round(wl.n_patches / (ms_step * 1e-3), 1),
        "merged_tokens_per_s": round(wl.out_rows / (ms_step * 1e-3), 1),
        "forward_tflops": round(total_flops / (ms_step * 1e-3) / 1e12, 1),
        "forward_mfma_frac": round(total_flops / (ms_step * 1e-3) / 1e12 / peak, 4),
        "dtype": wl.dtype, "attn_q_tile": info.attn_q_tile,
        "config": {"workload": wl.name, "images": [list(hw) for hw in wl.image_hw][:8],
                   "n_images": len(wl.image_hw), "patch": wl.patch, "layers": wl.layers, "merge": wl.merge,
                   "n_patches": wl.n_patches, "out_rows": wl.out_rows, "out_cols": wl.out_cols},
        "roofline": roofline, "memory_bound": memory_bound, "kernels": kernels,
    }
    if headline:
        res["scatter"] = time_scatter(out, wl, stream) if wl.merge == 2 else None
        res["u8_input"] = None
        if (len(wl.image_hw) == 1 or wl.tiles_from is not None) and "operand" in kernels:
            res["u8_input"] = time_u8_input(tw, wl, out, ws, stream,
                                            kernels["patch"]["ms_per_step"] + kernels["operand"]["ms_per_step"])
        res["embcache"] = time_embcache(tw, wl, stream)
        res["fp8_variant"] = time_fp8_variant(wl, dev_w, pix, stream)
    tw.close()
    del ws, out, pix
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="ms31_1540", help="the headline workload")
    ap.add_argument("--profile-steps", type=int, default=3)
    ap.add_argument("--sub-steps", type=int, default=10, help="timed steps of each other workload")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="time only the headline workload (no per-workload records)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-quick", action="store_true",
                    help="headline oracle timing from one block, extrapolated (default: the whole forward)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain fp32 copy kernel (y = x * 1) over MIB MiB, 5 times, and exit: the "
                         "reference for scaling rocprofv3's FETCH_SIZE / WRITE_SIZE counters to bytes")
    ap.add_argument("--mfma-ceiling", action="store_true",
                    help="only time the vendor bf16 GEMM (hipBLASLt) at 8192^3 and 16384^3 on random, zero and "
                         "one operands, and exit: the bf16 MFMA rate this chip sustains with real data")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("CLASS", "WORKLOAD"),
                    help="write profiles/traffic_CLASS_WORKLOAD.json from the four CSVs below and exit")
    ap.add_argument("--pmc-fetch")
    ap.add_argument("--pmc-write")
    ap.add_argument("--pmc-copy-fetch")
    ap.add_argument("--pmc-copy-write")
    ap.add_argument("--copy-probe-mib", type=int, default=512)
    ap.add_argument("--attn-q-tile", type=int, default=None,
                    help="with --pmc-summary: the attention work-item size of the measured run")
    args = ap.parse_args()
    if args.pmc_summary:
        pmc_summary(args)
        return
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.mfma_ceiling:
        mfma_ceiling()
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the tower runs on a single MI355X here "
              f"(--gpus {args.gpus} is not supported)", file=sys.stderr)
        sys.exit(2)

    import torch

    from vlm_vision_encoder_amd import synth
    from vlm_vision_encoder_amd import tower as T

    log = lambda m: print(f"[bench] {m}", file=sys.stderr, flush=True)  # noqa: E731
    names = [args.workload] + ([] if args.no_other_workloads else
                               [n for n in synth.WORKLOADS if n != args.workload])
    cache = {}  # weights shared by workloads of the same architecture (same seed, same draws)
    results = {}
    for name in names:
        wl = synth.workload(name)
        key = (wl.patch, wl.merge, wl.layers, wl.dtype)
        log(f"workload {wl.name}: {len(wl.image_hw)} images, {wl.n_patches} patches, {wl.out_rows} out rows, "
            f"{wl.layers} layers, {wl.dtype}")
        if key not in cache:
            cache.clear()
            torch.cuda.empty_cache()
            weights = synth.make_weights(wl)
            cache[key] = (weights, T.weights_to_device(weights, wl.dtype))
        weights, dev_w = cache[key]
        pixels = synth.make_pixels(wl)
        res = run_workload(wl, dev_w, weights, pixels, args, log, headline=(name == args.workload))
        if not args.no_cpu_baseline:
            full = name == args.workload and not args.cpu_quick
            log(f"timing the CPU oracle on {name} ({'the whole forward' if full else 'one block'})")
            res["cpu_baseline"] = cpu_baseline(wl, weights, pixels, full=full, log=log if full else None)
        else:
            res["cpu_baseline"] = None
        results[name] = res
        torch.cuda.empty_cache()

    h = results[args.workload]
    line = {
        "metric": "vision patches/s + merged tokens/s at 1540x1540; % bf16 MFMA peak",
        "value": h["patches_per_s"],
        "unit": "patches/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": h["ms_per_step"],
        "step_ms": h["step_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": h["dtype"],
        "data": "synthetic",
        "config": h["config"],
        "merged_tokens_per_s": h["merged_tokens_per_s"],
        "forward_tflops": h["forward_tflops"],
        "forward_mfma_frac": h["forward_mfma_frac"],
        "attn_q_tile": h["attn_q_tile"],
        "roofline": h["roofline"],
        "memory_bound": h["memory_bound"],
        "kernels": h["kernels"],
        "scatter": h.get("scatter"),
        "u8_input": h.get("u8_input"),
        "embcache": h.get("embcache"),
        "fp8_variant": h.get("fp8_variant"),
        "cpu_baseline": h["cpu_baseline"],
        "workloads": {n: {k: v for k, v in r.items() if k not in ("config",)} | {"config": r["config"]}
                      for n, r in results.items() if n != args.workload},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
