"""Helpers shared by the GPU parity tests: device upload, oracle comparison, tolerance checks."""
import numpy as np

Y_RTOL = 1e-5   # rescaled fp32 outputs: relative tolerance against the oracle's fp64 rescale


def dev(a, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def bf16_dev(bits_u16):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits_u16).view(np.int16)).cuda()
    return t.view(torch.bfloat16)


def host(t):
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


def as_u32(t):
    return host(t).view(np.uint32)


def f32_bits(x):
    return np.asarray(x, np.float32).view(np.uint32)


def assert_y_close(y_gpu, y_ref, rtol=Y_RTOL, what="y"):
    y_gpu = np.asarray(y_gpu, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    assert y_gpu.shape == y_ref.shape, (y_gpu.shape, y_ref.shape)
    err = np.abs(y_gpu - y_ref)
    bad = err > rtol * np.abs(y_ref)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} elements outside rtol {rtol}; first at {tuple(i)}: "
                             f"gpu {y_gpu[tuple(i)]!r} ref {y_ref[tuple(i)]!r}")
