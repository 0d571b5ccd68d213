"""The allocation-free masked scatter (pv_scatter_image_embeddings_noalloc)
against the workspace entry point (pv_scatter_image_embeddings), both through
the C ABI: bit-equal outputs and status on two calls in a row, the second
with a smaller sequence and fewer rows (the shared device scratch keeps the
first call's list and count, which the second must not see); host-side
validation without a GPU.  Byte work: bit-exact.
Inputs: seeded token sequences with placeholder id 10 at random positions."""
import ctypes as C

import numpy as np
import pytest

from vlm_vision_encoder_amd import tower as T

FAKE = 1 << 20  # an aligned, never-dereferenced stand-in for device pointers
MAX_SEQ = 1 << 20


def test_noalloc_scatter_validation_before_any_device_work():
    lib = T.load_library()
    st = C.c_void_p(FAKE)
    assert lib.pv_scatter_image_embeddings_noalloc(FAKE, 8, 10, FAKE, 2, FAKE, 64, 2, None, None) == -1
    assert lib.pv_scatter_image_embeddings_noalloc(FAKE, -1, 10, FAKE, 2, FAKE, 64, 2, st, None) == -1
    assert lib.pv_scatter_image_embeddings_noalloc(FAKE, 8, 10, FAKE, 2, FAKE, 64, 3, st, None) == -1
    assert lib.pv_scatter_image_embeddings_noalloc(FAKE, 8, 10, FAKE + 8, 2, FAKE, 64, 2, st, None) == -1
    assert lib.pv_scatter_image_embeddings_noalloc(FAKE, MAX_SEQ + 1, 10, FAKE, 2, FAKE, 64, 2, st, None) == -3
    assert b"maximum" in lib.pv_last_error()


def _case(rng, S, T_rows, dim, dtype):
    import torch
    ids = rng.integers(11, 131072, size=S).astype(np.int32)
    ids[rng.choice(S, size=T_rows, replace=False)] = 10
    img = rng.standard_normal((T_rows, dim)).astype(np.float32)
    txt = rng.standard_normal((S, dim)).astype(np.float32)
    t = lambda a: torch.from_numpy(a).cuda().to(dtype).contiguous()  # noqa: E731
    return torch.from_numpy(ids).cuda(), t(img), t(txt)


def _call(lib, fn, ids, img, txt, status, ws=None):
    import torch
    S, T_rows, dim = ids.numel(), img.shape[0], txt.shape[1]
    s = torch.cuda.current_stream().cuda_stream
    args = [ids.data_ptr(), S, 10, img.data_ptr(), T_rows, txt.data_ptr(), dim, img.element_size(), status.data_ptr()]
    if ws is not None:
        args += [ws.data_ptr(), ws.numel()]
    assert fn(*args, s) == 0, lib.pv_last_error()


@pytest.mark.gpu
@pytest.mark.parametrize("dtype_name", ["bf16", "f32"])
def test_noalloc_scatter_equals_workspace_scatter(dtype_name):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print(f"[gpu-case] allocation-free scatter vs workspace scatter, {dtype_name}", flush=True)
    lib = T.load_library()
    dtype = torch.bfloat16 if dtype_name == "bf16" else torch.float32
    rng = np.random.default_rng(77)
    # the first call fills more of the scratch list than the second uses
    for S, T_rows, dim in ((200_000, 3025, 5120 if dtype_name == "bf16" else 1024), (4049, 1089, 1024)):
        ids, img, txt = _case(rng, S, T_rows, dim, dtype)
        want, got = txt.clone(), txt.clone()
        st_w = torch.full((1,), 7, dtype=torch.int32, device="cuda")
        st_g = torch.full((1,), 7, dtype=torch.int32, device="cuda")
        wsb = lib.pv_scatter_workspace_bytes(S)
        ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
        _call(lib, lib.pv_scatter_image_embeddings, ids, img, want, st_w, ws)
        _call(lib, lib.pv_scatter_image_embeddings_noalloc, ids, img, got, st_g)
        torch.cuda.synchronize()
        assert torch.equal(got, want)
        assert int(st_g.item()) == int(st_w.item()) == 0
        # a count mismatch reports the same status on both paths
        short = img[: T_rows - 5].contiguous()
        _call(lib, lib.pv_scatter_image_embeddings, ids, short, want, st_w, ws)
        _call(lib, lib.pv_scatter_image_embeddings_noalloc, ids, short, got, st_g)
        torch.cuda.synchronize()
        assert torch.equal(got, want)
        assert int(st_g.item()) == int(st_w.item()) == 1
