"""rra_batched_gemv_noalloc (the GEMV for callers that cannot allocate device
memory) against rra_batched_gemv, through the C ABI: bitwise the same y on
two calls in a row, the second with a smaller input, and the size limit of
its static scratch."""
import ctypes

import pytest
import torch

import quantized_gemv_flash_amd as rra
import synth

DEV = "cuda"


def _pair(w, x, m):
    y_ref = torch.full((m, w.n), float("nan"), device=DEV)
    y_new = torch.full((m, w.n), float("nan"), device=DEV)
    ws = torch.empty(max(4, rra.rra_batched_gemv_workspace_bytes(w, m)), dtype=torch.uint8,
                     device=DEV)
    rra.rra_batched_gemv(w, x, y_ref, m, ws)
    rra.rra_batched_gemv_noalloc(w, x, y_new, m)
    torch.cuda.synchronize()
    return y_ref, y_new


@pytest.mark.gpu
@pytest.mark.parametrize("fmt,n,k", [("q4", 6144, 4096), ("q8", 1152, 896), ("f32", 300, 256)])
def test_noalloc_gemv_equals_workspace_gemv_twice(fmt, n, k):
    data, scale = synth.weight(n, k, fmt, 0.02, 0, f"noalloc_{fmt}", DEV)
    w = rra.device_weight(data, scale, fmt)
    for m, seed in ((32, 1), (3, 2)):  # the second call smaller than the first
        x = synth.normal((m, k), 1.0, seed, f"noalloc_x{m}", DEV)
        if fmt != "f32":
            need = rra.rra_batched_gemv_workspace_bytes(w, m)
            assert 0 < need <= 16 << 20
        y_ref, y_new = _pair(w, x, m)
        assert not torch.isnan(y_ref).any()
        assert torch.equal(y_ref, y_new), (fmt, m)


@pytest.mark.gpu
def test_noalloc_gemv_rejects_a_call_past_its_scratch():
    # a Q4 weight with K = 2^20 needs a 128 MiB activation image at M = 32:
    # rejected before anything is launched (the fake data is never read)
    t = torch.zeros(16, dtype=torch.uint8, device=DEV)
    w = rra.Weight("q4", 16, 1 << 20, t, None, rra.RRA_TILED)
    assert rra.rra_batched_gemv_workspace_bytes(w, 32) > (16 << 20)
    x = torch.zeros(4, device=DEV)
    with pytest.raises(rra.RraError) as e:
        rra.rra_batched_gemv_noalloc(w, x, x, 32)
    assert e.value.status == rra.RRA_EINVAL and "static scratch" in str(e.value)
    torch.cuda.synchronize()
