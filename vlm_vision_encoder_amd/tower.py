"""ctypes binding of libpv_tower.so (C ABI in include/pv_tower.h).

Argument marshalling only: every step of the tower runs in the HIP library.
PyTorch provides device memory and the current HIP stream.  If the library has
not been built, loading it raises; there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Dict, List, Optional, Sequence, Tuple

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("PV_TOWER_LIB") or os.path.join(PKG, "libpv_tower.so")

PV_BF16, PV_F32 = 0, 1
PV_FLAG_ATTN_ONLINE_MAX = 1
PV_FLAG_FP8 = 2
PV_FLAG_DEEP_PROJECTOR = 4
PV_FLAG_ROPE_INTERLEAVED = 8
STAGES = {"patch_embed": 0, "ln_pre": 1, "qkv": 2, "attn": 3, "attn_resid": 4, "mlp_hidden": 5, "block_out": 6}
STATUS = {0: "PV_OK", -1: "PV_ERR_ARG", -2: "PV_ERR_SHAPE", -3: "PV_ERR_CAPACITY", -4: "PV_ERR_HIP",
          -5: "PV_ERR_UNSUPPORTED"}

EXPORTED = ("pv_tower_create", "pv_tower_destroy", "pv_tower_plan", "pv_tower_forward",
            "pv_tower_forward_stage", "pv_tower_index_maps", "pv_tower_set_profiling", "pv_tower_read_profile",
            "pv_scatter_workspace_bytes", "pv_scatter_image_embeddings", "pv_resize_target", "pv_tower_plan_u8",
            "pv_tower_forward_u8", "pv_preprocess_u8", "pv_tile_layout", "pv_tower_plan_tiles_u8",
            "pv_tower_forward_tiles_u8", "pv_config_preset", "pv_image_keys_workspace_bytes", "pv_image_keys_u8",
            "pv_embcache_create", "pv_embcache_destroy", "pv_embcache_clear", "pv_embcache_stats",
            "pv_embcache_workspace_bytes", "pv_tower_forward_cached_u8", "pv_quantize_fp8", "pv_last_error", "pv_status_str",
            "pv_tower_prepared_bytes", "pv_tower_prepare", "pv_scatter_image_embeddings_noalloc")
PRESETS = {"mistral3": 0, "pixtral12b": 1}
KERNEL_CLASSES = ("maps", "patch", "norm", "qkv", "attn", "oproj", "gateup", "down", "merge", "norm_mlp", "operand")


class PvConfig(C.Structure):
    _fields_ = [("patch", C.c_int32), ("hidden", C.c_int32), ("heads", C.c_int32), ("mlp", C.c_int32),
                ("layers", C.c_int32), ("merge", C.c_int32), ("out_dim", C.c_int32), ("max_side", C.c_int32),
                ("rope_theta", C.c_double), ("rms_eps", C.c_double), ("dtype", C.c_int32),
                ("out_dtype", C.c_int32), ("flags", C.c_int32)]


class PvLayerWeights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate", "w_up",
                                          "w_down")]


class PvProjectorWeights(C.Structure):
    _fields_ = [("norm", C.c_void_p), ("w1", C.c_void_p), ("w2", C.c_void_p)]


class PvWeights(C.Structure):
    _fields_ = [("patch_w", C.c_void_p), ("ln_pre", C.c_void_p), ("layers", C.POINTER(PvLayerWeights)),
                ("merge_w", C.c_void_p), ("proj", C.POINTER(PvProjectorWeights))]


class PvPlanInfo(C.Structure):
    _fields_ = [("n_patches", C.c_int64), ("out_rows", C.c_int64), ("out_cols", C.c_int64),
                ("workspace_bytes", C.c_int64), ("n_images", C.c_int32), ("max_patches", C.c_int32),
                ("attn_q_tile", C.c_int32)]


class PvError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH):
    """Loads the HIP library (raises if it is missing)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run __graft_entry__.build() "
                           "(python -m vlm_vision_encoder_amd.build_lib)")
    # torch first: its HIP runtime (a copy under torch/lib with the same
    # soname) is then the one the library binds to.  Loaded the other way
    # round, the process would hold two HIP runtimes, one for torch's memory
    # and streams and one for the library's kernels.
    import torch  # noqa: F401
    lib = C.CDLL(path)
    vp, i32, i64, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
    lib.pv_tower_create.argtypes = [C.POINTER(PvConfig), C.POINTER(PvWeights), C.POINTER(vp)]
    lib.pv_tower_create.restype = i32
    lib.pv_tower_destroy.argtypes = [vp]
    lib.pv_tower_destroy.restype = None
    lib.pv_tower_plan.argtypes = [vp, vp, i32, C.POINTER(PvPlanInfo)]
    lib.pv_tower_plan.restype = i32
    lib.pv_tower_forward.argtypes = [vp, vp, vp, i32, vp, i64, vp, sz, vp]
    lib.pv_tower_forward.restype = i32
    lib.pv_tower_forward_stage.argtypes = [vp, vp, vp, i32, i32, i32, vp, i64, vp, sz, vp]
    lib.pv_tower_forward_stage.restype = i32
    lib.pv_tower_index_maps.argtypes = [vp, vp, i32, vp, vp, vp, i32, vp, sz, vp]
    lib.pv_tower_index_maps.restype = i32
    lib.pv_tower_set_profiling.argtypes = [vp, i32]
    lib.pv_tower_set_profiling.restype = i32
    lib.pv_tower_read_profile.argtypes = [vp, C.POINTER(C.c_double), C.POINTER(C.c_int64), i32]
    lib.pv_tower_read_profile.restype = i32
    lib.pv_scatter_workspace_bytes.argtypes = [i64]
    lib.pv_scatter_workspace_bytes.restype = sz
    lib.pv_scatter_image_embeddings.argtypes = [vp, i64, i32, vp, i64, vp, i32, i32, vp, vp, sz, vp]
    lib.pv_scatter_image_embeddings.restype = i32
    lib.pv_resize_target.argtypes = [vp, i32, i32, i32, vp]
    lib.pv_resize_target.restype = i32
    lib.pv_tower_plan_u8.argtypes = [vp, vp, i32, vp, C.POINTER(PvPlanInfo)]
    lib.pv_tower_plan_u8.restype = i32
    lib.pv_tower_forward_u8.argtypes = [vp, vp, vp, i32, vp, vp, i64, vp, sz, vp]
    lib.pv_tower_forward_u8.restype = i32
    lib.pv_preprocess_u8.argtypes = [vp, vp, vp, i32, vp, vp, vp]
    lib.pv_preprocess_u8.restype = i32
    lib.pv_tile_layout.argtypes = [vp, i32, i32, i32, i32, vp]
    lib.pv_tile_layout.restype = i32
    lib.pv_tower_plan_tiles_u8.argtypes = [vp, vp, i32, i32, vp, C.POINTER(PvPlanInfo)]
    lib.pv_tower_plan_tiles_u8.restype = i32
    lib.pv_tower_forward_tiles_u8.argtypes = [vp, vp, vp, i32, i32, vp, vp, i64, vp, sz, vp]
    lib.pv_tower_forward_tiles_u8.restype = i32
    lib.pv_config_preset.argtypes = [i32, i32, C.POINTER(PvConfig)]
    lib.pv_config_preset.restype = i32
    lib.pv_image_keys_workspace_bytes.argtypes = [i32]
    lib.pv_image_keys_workspace_bytes.restype = sz
    lib.pv_image_keys_u8.argtypes = [vp, vp, i32, vp, vp, sz, vp]
    lib.pv_image_keys_u8.restype = i32
    lib.pv_embcache_create.argtypes = [vp, vp, vp, i64, C.POINTER(vp)]
    lib.pv_embcache_create.restype = i32
    lib.pv_embcache_destroy.argtypes = [vp]
    lib.pv_embcache_destroy.restype = None
    lib.pv_embcache_clear.argtypes = [vp]
    lib.pv_embcache_clear.restype = i32
    lib.pv_embcache_stats.argtypes = [vp, vp]
    lib.pv_embcache_stats.restype = i32
    lib.pv_embcache_workspace_bytes.argtypes = [vp, vp, i32, C.POINTER(C.c_int64)]
    lib.pv_embcache_workspace_bytes.restype = i32
    lib.pv_tower_forward_cached_u8.argtypes = [vp, vp, vp, i32, vp, vp, i64, vp, sz, vp, vp]
    lib.pv_tower_forward_cached_u8.restype = i32
    lib.pv_quantize_fp8.argtypes = [vp, i64, i32, vp, vp, vp]
    lib.pv_quantize_fp8.restype = i32
    lib.pv_scatter_image_embeddings_noalloc.argtypes = [vp, i64, i32, vp, i64, vp, i32, i32, vp, vp]
    lib.pv_scatter_image_embeddings_noalloc.restype = i32
    lib.pv_tower_prepared_bytes.argtypes = [vp, C.POINTER(C.c_int64)]
    lib.pv_tower_prepared_bytes.restype = i32
    lib.pv_tower_prepare.argtypes = [vp, vp, i64, vp]
    lib.pv_tower_prepare.restype = i32
    lib.pv_last_error.argtypes = []
    lib.pv_last_error.restype = C.c_char_p
    lib.pv_status_str.argtypes = [i32]
    lib.pv_status_str.restype = C.c_char_p
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        raise PvError(status, _lib.pv_last_error().decode())


def make_config(patch=14, hidden=1024, heads=16, mlp=4096, layers=24, merge=2, out_dim=5120, max_side=1540,
                rope_theta=1.0e4, rms_eps=1.0e-5, dtype="bf16", out_dtype=None, flags=0) -> PvConfig:
    if dtype not in ("bf16", "f32"):
        raise ValueError("dtype must be 'bf16' or 'f32'")
    out_dtype = dtype if out_dtype is None else out_dtype
    if out_dtype not in ("bf16", "f32"):
        raise ValueError("out_dtype must be 'bf16' or 'f32'")
    return PvConfig(patch, hidden, heads, mlp, layers, merge, out_dim, max_side, float(rope_theta),
                    float(rms_eps), PV_BF16 if dtype == "bf16" else PV_F32, PV_BF16 if out_dtype == "bf16" else PV_F32,
                    int(flags))


def _stream_pair(stream):
    """(torch stream object, raw hipStream_t) of a stream argument: None (the
    current stream), a torch.cuda.Stream, or a raw hipStream_t given as an
    int.  The raw handle goes to the library exactly as given; the torch
    object only places and records allocations (the current stream itself
    whenever the handle is the current stream's)."""
    import torch
    cur = torch.cuda.current_stream()
    if stream is None:
        return cur, cur.cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream, stream.cuda_stream
    ptr = int(stream)
    if ptr == cur.cuda_stream:
        return cur, ptr
    return torch.cuda.ExternalStream(ptr), ptr


def _torch_stream(stream):
    return _stream_pair(stream)[0]


def _hw_array(image_hw: Sequence[Sequence[int]]):
    flat = [int(v) for hw in image_hw for v in hw]
    return (C.c_int32 * max(1, len(flat)))(*flat), len(image_hw)


class Tower:
    """One tower object over borrowed device weights.

    ``weights``: dict with torch tensors on the GPU: ``patch_w`` [D,3,p,p],
    ``ln_pre`` [D] fp32, ``layers`` = list of dicts (``attn_norm``, ``wq``,
    ``wk``, ``wv``, ``wo``, ``ffn_norm``, ``w_gate``, ``w_up``, ``w_down``),
    ``merge_w`` [out_dim, 4D] (merge 2).  Matrices in the tower dtype; the
    tensors are kept referenced for the tower's lifetime.

    With ``prepare`` (the default) the tower's derived weight copies (padded
    patch weights, fp4 / fp8 copies of the block matrices) are written once
    into device memory the object owns (``pv_tower_prepare``); without it
    every forward derives them in its workspace.

    ``stream`` arguments take a ``torch.cuda.Stream`` or a raw ``hipStream_t``
    (int); outputs and the workspace are allocated for, and recorded on, the
    stream the call runs on.
    """

    def __init__(self, cfg: PvConfig, weights: Dict, prepare: bool = True):
        self.lib = load_library()
        self.cfg = cfg
        self._keep = weights
        lw = [PvLayerWeights(*[weights["layers"][i][k].data_ptr() for k, _ in PvLayerWeights._fields_])
              for i in range(cfg.layers)]
        self._layers = (PvLayerWeights * max(1, len(lw)))(*lw)
        mw = weights.get("merge_w")
        pj = weights.get("proj")
        self._proj = PvProjectorWeights(pj["norm"].data_ptr(), pj["w1"].data_ptr(), pj["w2"].data_ptr()) if pj else None
        self._w = PvWeights(weights["patch_w"].data_ptr(), weights["ln_pre"].data_ptr(),
                            C.cast(self._layers, C.POINTER(PvLayerWeights)) if lw else None,
                            mw.data_ptr() if mw is not None else None,
                            C.pointer(self._proj) if pj else None)
        h = C.c_void_p()
        _check(self.lib.pv_tower_create(C.byref(cfg), C.byref(self._w), C.byref(h)))
        self.handle = h
        self._ws = None
        self._prep = None
        if prepare:
            self.prepare()

    def prepare(self):
        """Writes the derived weight copies once (pv_tower_prepare) on the
        current stream and waits for them."""
        import torch
        nb = C.c_int64()
        _check(self.lib.pv_tower_prepared_bytes(self.handle, C.byref(nb)))
        if nb.value == 0:
            return
        mem = torch.empty(nb.value, dtype=torch.uint8, device="cuda")
        st = torch.cuda.current_stream()
        _check(self.lib.pv_tower_prepare(self.handle, mem.data_ptr(), nb.value, st.cuda_stream))
        st.synchronize()
        self._prep = mem

    def unprepare(self):
        """Forward calls derive the weight copies per call again."""
        _check(self.lib.pv_tower_prepare(self.handle, None, 0, None))
        self._prep = None

    def close(self):
        if getattr(self, "handle", None):
            self.lib.pv_tower_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ------------------------------------------------------------ host-only
    def plan(self, image_hw) -> PvPlanInfo:
        arr, n = _hw_array(image_hw)
        info = PvPlanInfo()
        _check(self.lib.pv_tower_plan(self.handle, arr, n, C.byref(info)))
        return info

    # ------------------------------------------------------------ device
    def workspace(self, nbytes: int, stream=None):
        """The cached workspace, grown to nbytes on `stream` and recorded on
        it (so the caching allocator never hands its memory to another stream
        while this stream's work is pending)."""
        import torch
        st = _torch_stream(stream)
        if self._ws is None or self._ws.numel() < nbytes:
            if self._ws is not None:
                self._ws.record_stream(st)
            with torch.cuda.stream(st):
                self._ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device="cuda")
        elif st != torch.cuda.current_stream():
            self._ws.record_stream(st)
        return self._ws

    def _new_out(self, info, stream):
        import torch
        with torch.cuda.stream(_torch_stream(stream)):
            return torch.empty((info.out_rows, info.out_cols), dtype=self._out_dtype(), device="cuda")

    def _act_dtype(self):
        import torch
        return torch.bfloat16 if self.cfg.dtype == PV_BF16 else torch.float32

    def _out_dtype(self):
        import torch
        bf_out = self.cfg.dtype == PV_BF16 and self.cfg.out_dtype == PV_BF16
        return torch.bfloat16 if bf_out else torch.float32

    def forward(self, pixels, image_hw, out=None, stream=None):
        """pixels: flat fp32 CUDA tensor of the normalised C x H x W planes."""
        import torch
        arr, n = _hw_array(image_hw)
        info = self.plan(image_hw)
        if out is None:
            out = self._new_out(info, stream)
        ws = self.workspace(info.workspace_bytes, stream)
        s = _stream_pair(stream)[1]
        _check(self.lib.pv_tower_forward(self.handle, pixels.data_ptr(), arr, n, out.data_ptr(), out.shape[0],
                                         ws.data_ptr(), ws.numel(), s))
        return out

    def forward_raw(self, pixels_ptr: int, image_hw, out_ptr: int, out_rows_cap: int, ws_ptr: int,
                    ws_bytes: int, stream: int):
        arr, n = _hw_array(image_hw)
        _check(self.lib.pv_tower_forward(self.handle, pixels_ptr, arr, n, out_ptr, out_rows_cap, ws_ptr,
                                         ws_bytes, stream))

    # ------------------------------------------------------------ uint8 input
    def plan_u8(self, src_hw) -> Tuple[PvPlanInfo, List[Tuple[int, int]]]:
        """Plan of uint8 sources: (info, target sizes)."""
        arr, n = _hw_array(src_hw)
        dst = (C.c_int32 * (2 * n))()
        info = PvPlanInfo()
        _check(self.lib.pv_tower_plan_u8(self.handle, arr, n, dst, C.byref(info)))
        return info, [(dst[2 * i], dst[2 * i + 1]) for i in range(n)]

    def forward_u8(self, images, src_hw, mean_std=None, out=None, stream=None):
        """images: flat uint8 CUDA tensor of the H x W x 3 images in order."""
        import torch
        arr, n = _hw_array(src_hw)
        info, _ = self.plan_u8(src_hw)
        if out is None:
            out = self._new_out(info, stream)
        ws = self.workspace(info.workspace_bytes, stream)
        s = _stream_pair(stream)[1]
        ms = (C.c_float * 6)(*mean_std) if mean_std is not None else None
        _check(self.lib.pv_tower_forward_u8(self.handle, images.data_ptr(), arr, n, ms, out.data_ptr(),
                                            out.shape[0], ws.data_ptr(), ws.numel(), s))
        return out

    def plan_tiles_u8(self, src_hw, max_num_tiles: int):
        """Plan of the tiles of uint8 sources: (info, per-image (resized H,
        resized W, tile rows, tile columns))."""
        arr, n = _hw_array(src_hw)
        lay = (C.c_int32 * (4 * n))()
        info = PvPlanInfo()
        _check(self.lib.pv_tower_plan_tiles_u8(self.handle, arr, n, int(max_num_tiles), lay, C.byref(info)))
        return info, [tuple(lay[4 * i: 4 * i + 4]) for i in range(n)]

    def forward_tiles_u8(self, images, src_hw, max_num_tiles: int, mean_std=None, out=None, stream=None):
        """The tower over the tiles of uint8 images (flat CUDA tensor)."""
        import torch
        arr, n = _hw_array(src_hw)
        info, _ = self.plan_tiles_u8(src_hw, max_num_tiles)
        if out is None:
            out = self._new_out(info, stream)
        ws = self.workspace(info.workspace_bytes, stream)
        s = _stream_pair(stream)[1]
        ms = (C.c_float * 6)(*mean_std) if mean_std is not None else None
        _check(self.lib.pv_tower_forward_tiles_u8(self.handle, images.data_ptr(), arr, n, int(max_num_tiles), ms,
                                                  out.data_ptr(), out.shape[0], ws.data_ptr(), ws.numel(), s))
        return out

    def set_profiling(self, enable: bool):
        _check(self.lib.pv_tower_set_profiling(self.handle, 1 if enable else 0))

    def read_profile(self, reset: bool = True) -> Dict[str, Tuple[float, int]]:
        """{class: (summed ms, launches)} of the recorded forward calls."""
        n = len(KERNEL_CLASSES)
        ms = (C.c_double * n)()
        cnt = (C.c_int64 * n)()
        _check(self.lib.pv_tower_read_profile(self.handle, ms, cnt, 1 if reset else 0))
        return {k: (ms[i], cnt[i]) for i, k in enumerate(KERNEL_CLASSES)}

    def forward_stage(self, pixels, image_hw, stage: str, layer: int = 0):
        import torch
        arr, n = _hw_array(image_hw)
        info = self.plan(image_hw)
        N, D, F = info.n_patches, self.cfg.hidden, self.cfg.mlp
        act = self._act_dtype()
        # the bf16 tower's MLP hidden activation is fp16 (the down product's operand)
        mlp = torch.float16 if act == torch.bfloat16 and not (self.cfg.flags & PV_FLAG_FP8) else act
        shapes = {"patch_embed": ((N, D), torch.float32), "ln_pre": ((N, D), torch.float32),
                  "qkv": ((N, 3 * D), act), "attn": ((N, D), act), "attn_resid": ((N, D), torch.float32),
                  "mlp_hidden": ((N, F), mlp), "block_out": ((N, D), torch.float32)}
        shape, dt = shapes[stage]
        dst = torch.empty(shape, dtype=dt, device="cuda")
        ws = self.workspace(info.workspace_bytes)
        s = torch.cuda.current_stream().cuda_stream
        _check(self.lib.pv_tower_forward_stage(self.handle, pixels.data_ptr(), arr, n, STAGES[stage], layer,
                                               dst.data_ptr(), dst.numel() * dst.element_size(), ws.data_ptr(),
                                               ws.numel(), s))
        return dst

    def index_maps(self, image_hw, on_device: bool):
        import numpy as np
        info = self.plan(image_hw)
        n = len(image_hw)
        T = info.out_rows if self.cfg.merge == 2 else 0
        if not on_device:
            cu = np.zeros(n + 1, np.int32)
            rc = np.zeros((max(1, info.n_patches), 2), np.int32)
            ms = np.zeros((max(1, T), 4), np.int32)
            arr, _ = _hw_array(image_hw)
            _check(self.lib.pv_tower_index_maps(self.handle, arr, n, cu.ctypes.data, rc.ctypes.data,
                                                ms.ctypes.data if T else None, 0, None, 0, None))
            return cu, rc[:info.n_patches], ms[:T]
        import torch
        cu = torch.zeros(n + 1, dtype=torch.int32, device="cuda")
        rc = torch.zeros((max(1, info.n_patches), 2), dtype=torch.int32, device="cuda")
        ms = torch.zeros((max(1, T), 4), dtype=torch.int32, device="cuda")
        ws = self.workspace(info.workspace_bytes)
        arr, _ = _hw_array(image_hw)
        _check(self.lib.pv_tower_index_maps(self.handle, arr, n, cu.data_ptr(), rc.data_ptr(),
                                            ms.data_ptr() if T else None, 1, ws.data_ptr(), ws.numel(),
                                            torch.cuda.current_stream().cuda_stream))
        torch.cuda.synchronize()
        return cu.cpu().numpy(), rc[:info.n_patches].cpu().numpy(), ms[:T].cpu().numpy()


def scatter_image_embeddings(token_ids, image_emb, text_emb, image_token_id: int = 10):
    """In place: the k-th position of token_ids (int32, [S], CUDA) equal to
    image_token_id takes row k of image_emb ([T][dim], CUDA) in text_emb
    ([S][dim], CUDA, same dtype).  Returns the device int32 status (0: the
    placeholder count equals T).  Enqueued on the current stream."""
    import torch
    lib = load_library()
    assert token_ids.dtype == torch.int32 and token_ids.is_contiguous()
    assert image_emb.dtype == text_emb.dtype and image_emb.is_contiguous() and text_emb.is_contiguous()
    S, T = token_ids.numel(), image_emb.shape[0]
    dim = text_emb.shape[1] if text_emb.dim() == 2 else image_emb.shape[1]
    status = torch.empty(1, dtype=torch.int32, device=text_emb.device)
    wsb = lib.pv_scatter_workspace_bytes(S)
    ws = torch.empty(wsb, dtype=torch.uint8, device=text_emb.device)
    _check(lib.pv_scatter_image_embeddings(token_ids.data_ptr() if S else None, S, int(image_token_id),
                                           image_emb.data_ptr() if T else None, T,
                                           text_emb.data_ptr() if S else None, dim, image_emb.element_size(),
                                           status.data_ptr(), ws.data_ptr(), wsb,
                                           torch.cuda.current_stream().cuda_stream))
    return status


def scatter_image_embeddings_noalloc(token_ids, image_emb, text_emb, image_token_id: int = 10):
    """As scatter_image_embeddings, through the allocation-free entry point
    (the library's fixed device scratch; at most 2^20 tokens).  Allocates
    only the returned status word."""
    import torch
    lib = load_library()
    assert token_ids.dtype == torch.int32 and token_ids.is_contiguous()
    assert image_emb.dtype == text_emb.dtype and image_emb.is_contiguous() and text_emb.is_contiguous()
    S, T = token_ids.numel(), image_emb.shape[0]
    dim = text_emb.shape[1] if text_emb.dim() == 2 else image_emb.shape[1]
    status = torch.empty(1, dtype=torch.int32, device=text_emb.device)
    _check(lib.pv_scatter_image_embeddings_noalloc(token_ids.data_ptr() if S else None, S, int(image_token_id),
                                                   image_emb.data_ptr() if T else None, T,
                                                   text_emb.data_ptr() if S else None, dim, image_emb.element_size(),
                                                   status.data_ptr(), torch.cuda.current_stream().cuda_stream))
    return status


def resize_target(src_hw, longest_edge: int, grid: int) -> List[Tuple[int, int]]:
    """Target sizes of the resize onto the patch grid (host only)."""
    lib = load_library()
    arr, n = _hw_array(src_hw)
    dst = (C.c_int32 * (2 * n))()
    _check(lib.pv_resize_target(arr, n, int(longest_edge), int(grid), dst))
    return [(dst[2 * i], dst[2 * i + 1]) for i in range(n)]


def tile_layout(src_hw, tile: int, grid: int, max_num_tiles: int) -> List[Tuple[int, int, int, int]]:
    """Per image (resized H, resized W, tile rows, tile columns) (host only)."""
    lib = load_library()
    arr, n = _hw_array(src_hw)
    lay = (C.c_int32 * (4 * n))()
    _check(lib.pv_tile_layout(arr, n, int(tile), int(grid), int(max_num_tiles), lay))
    return [tuple(lay[4 * i: 4 * i + 4]) for i in range(n)]


def image_keys_u8(images, src_hw):
    """Content keys of uint8 images (flat CUDA tensor): int64 CUDA tensor
    [n][2] holding the two uint64 lanes' bits."""
    import torch
    lib = load_library()
    arr, n = _hw_array(src_hw)
    keys = torch.empty((n, 2), dtype=torch.int64, device=images.device)
    wsb = lib.pv_image_keys_workspace_bytes(n)
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=images.device)
    _check(lib.pv_image_keys_u8(images.data_ptr(), arr, n, keys.data_ptr(), ws.data_ptr(), ws.numel(),
                                torch.cuda.current_stream().cuda_stream))
    return keys


class EmbCache:
    """Embeddings cache over a device buffer of `capacity_rows` output rows of
    `tower`; forward() runs pv_tower_forward_cached_u8."""

    def __init__(self, tower: "Tower", capacity_rows: int, mean_std=None):
        import torch
        self.lib = load_library()
        self.tower = tower
        cols_dtype = tower._out_dtype()
        cols = tower.cfg.out_dim if tower.cfg.merge == 2 else tower.cfg.hidden
        self.mem = torch.empty((capacity_rows, cols), dtype=cols_dtype, device="cuda")
        self._ms = (C.c_float * 6)(*mean_std) if mean_std is not None else None
        h = C.c_void_p()
        _check(self.lib.pv_embcache_create(tower.handle, self._ms, self.mem.data_ptr(),
                                           self.mem.numel() * self.mem.element_size(), C.byref(h)))
        self.handle = h
        self._ws = None

    def workspace_bytes(self, src_hw) -> int:
        arr, n = _hw_array(src_hw)
        b = C.c_int64()
        _check(self.lib.pv_embcache_workspace_bytes(self.handle, arr, n, C.byref(b)))
        return b.value

    def forward(self, images, src_hw, keys=None, out=None, stream=None):
        """Returns (out, hits): hits[i] = 1 where image i came from the cache.
        keys: None (hashed on the device; synchronises) or a host sequence of
        n pairs of uint64."""
        import torch
        arr, n = _hw_array(src_hw)
        info, _ = self.tower.plan_u8(src_hw)
        st, sptr = _stream_pair(stream)
        if out is None:
            out = self.tower._new_out(info, st)
        need = self.workspace_bytes(src_hw)
        if self._ws is None or self._ws.numel() < need:
            if self._ws is not None:
                self._ws.record_stream(st)
            with torch.cuda.stream(st):
                self._ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
        elif st != torch.cuda.current_stream():
            self._ws.record_stream(st)
        k = None
        if keys is not None:
            flat = [int(v) & 0xFFFFFFFFFFFFFFFF for pair in keys for v in pair]
            k = (C.c_uint64 * (2 * n))(*flat)
        hits = (C.c_int32 * n)()
        s = sptr
        _check(self.lib.pv_tower_forward_cached_u8(self.handle, images.data_ptr(), arr, n, k, out.data_ptr(),
                                                   out.shape[0], self._ws.data_ptr(), self._ws.numel(), s, hits))
        return out, list(hits)

    def stats(self) -> Dict[str, int]:
        st = (C.c_int64 * 5)()
        _check(self.lib.pv_embcache_stats(self.handle, st))
        return dict(zip(("entries", "rows_used", "capacity_rows", "hits", "misses"), list(st)))

    def clear(self):
        _check(self.lib.pv_embcache_clear(self.handle))

    def close(self):
        if getattr(self, "handle", None):
            self.lib.pv_embcache_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def quantize_fp8(x):
    """bf16 CUDA matrix [rows][K] -> (uint8 e4m3 codes [rows][K], uint8 scale
    bytes in the GEMM layout [K/128][rows][4])."""
    import torch
    lib = load_library()
    rows, K = x.shape
    codes = torch.empty((rows, K), dtype=torch.uint8, device=x.device)
    scales = torch.empty((K // 128, rows, 4), dtype=torch.uint8, device=x.device)
    _check(lib.pv_quantize_fp8(x.data_ptr(), rows, K, codes.data_ptr(), scales.data_ptr(),
                               torch.cuda.current_stream().cuda_stream))
    return codes, scales


def preset(name: str, dtype: str = "bf16") -> PvConfig:
    """PvConfig of a named tower ("mistral3" or "pixtral12b")."""
    lib = load_library()
    cfg = PvConfig()
    _check(lib.pv_config_preset(PRESETS[name], PV_BF16 if dtype == "bf16" else PV_F32, C.byref(cfg)))
    return cfg


def preprocess_u8(images, src_hw, dst_hw, mean_std=None, out=None):
    """Resize + normalise uint8 images (flat CUDA tensor, H x W x 3 each) to
    dst_hw; returns the flat fp32 CUDA tensor of the 3 x tH x tW planes."""
    import torch
    lib = load_library()
    sa, n = _hw_array(src_hw)
    da, _ = _hw_array(dst_hw)
    total = sum(3 * int(h) * int(w) for h, w in dst_hw)
    if out is None:
        out = torch.empty(max(1, total), dtype=torch.float32, device=images.device)
    ms = (C.c_float * 6)(*mean_std) if mean_std is not None else None
    _check(lib.pv_preprocess_u8(images.data_ptr(), sa, da, n, ms, out.data_ptr(),
                                torch.cuda.current_stream().cuda_stream))
    return out[:total]


# ---------------------------------------------------------------- helpers
def config_for(wl, max_side: Optional[int] = None, out_dtype: Optional[str] = None, flags: int = 0) -> PvConfig:
    """PvConfig of a synth.Workload."""
    ms = max_side if max_side is not None else max(max(h, w) for h, w in wl.image_hw)
    return make_config(patch=wl.patch, hidden=wl.hidden, heads=wl.heads, mlp=wl.mlp, layers=wl.layers,
                       merge=wl.merge, out_dim=wl.out_dim, max_side=ms, rope_theta=wl.rope_theta,
                       rms_eps=wl.rms_eps, dtype=wl.dtype, out_dtype=out_dtype, flags=flags)


def weights_to_device(w: Dict, dtype: str) -> Dict:
    """numpy weights (float32 arrays) -> CUDA tensors in the tower's layout."""
    import torch
    mdt = torch.bfloat16 if dtype == "bf16" else torch.float32

    def mat(a):
        return torch.from_numpy(a.reshape(a.shape[0], -1)).to(device="cuda").to(mdt).contiguous()

    def vec(a):
        return torch.from_numpy(a).to(device="cuda", dtype=torch.float32).contiguous()

    out = {"patch_w": mat(w["patch_w"]), "ln_pre": vec(w["ln_pre"]), "layers": []}
    for lw in w["layers"]:
        out["layers"].append({k: (vec(v) if k.endswith("norm") else mat(v)) for k, v in lw.items()})
    if "merge_w" in w:
        out["merge_w"] = mat(w["merge_w"])
    if "proj" in w:
        out["proj"] = {"norm": vec(w["proj"]["norm"]), "w1": mat(w["proj"]["w1"]), "w2": mat(w["proj"]["w2"])}
    return out
