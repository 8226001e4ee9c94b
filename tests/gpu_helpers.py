"""Helpers shared by the GPU parity tests (device transfer, tolerance check)."""
import numpy as np

TOL = 4e-3   # |y - y_ref| <= TOL * max|y_ref| for bf16 outputs and FP8 paths


def torch_mod():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch


def dev(a: np.ndarray):
    """numpy array -> contiguous device tensor with the same bytes."""
    torch = torch_mod()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16))
    else:
        t = torch.from_numpy(a)
    return t.cuda()


def host(t, dtype=None) -> np.ndarray:
    a = t.cpu().numpy()
    if dtype is not None:
        a = a.view(dtype)
    return a


def empty(torch, shape, dtype, fill=None):
    t = torch.empty(shape, dtype=dtype, device="cuda")
    if fill is not None:
        t.view(torch.uint8).fill_(fill)
    return t


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits).view(np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def assert_within_tol(y_bits_or_f, y_ref, what="", f32=False):
    y = np.asarray(y_bits_or_f, dtype=np.float64) if f32 else bf16_to_f64(y_bits_or_f)
    ref = np.asarray(y_ref, dtype=np.float64)
    assert y.shape == ref.shape, (y.shape, ref.shape)
    assert np.isfinite(y).all(), f"{what}: non-finite output"
    scale = np.max(np.abs(ref)) if ref.size else 0.0
    err = np.max(np.abs(y - ref)) if ref.size else 0.0
    assert err <= TOL * scale, f"{what}: max|dy| = {err:.6g} > {TOL} * {scale:.6g}"
    return err / scale if scale else 0.0


def e4m3_equal_mod_zero(a: np.ndarray, b: np.ndarray) -> bool:
    a = np.asarray(a, np.uint8)
    b = np.asarray(b, np.uint8)
    return bool(np.all((a == b) | (((a & 0x7F) == 0) & ((b & 0x7F) == 0))))
