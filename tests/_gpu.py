"""Helpers for the GPU parity tests: move generator arrays to the device and back."""
import sys

import numpy as np
import torch

DEV = "cuda"


def banner(msg):
    """Name the case before a GPU step (so a failing run says which case it was)."""
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def dev(x, dtype=None):
    """numpy -> device tensor.  bf16 arrays from the generators hold bf16-exact fp32."""
    if isinstance(x, torch.Tensor):
        return x.to(DEV)
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(DEV)


def bf16(x):
    return dev(np.asarray(x, np.float32), torch.bfloat16)


def f32(x):
    return dev(np.asarray(x, np.float32), torch.float32)


def i32(x):
    return dev(np.asarray(x, np.int32))


def u8(x):
    return dev(np.asarray(x, np.uint8))


def host(t):
    """device tensor -> float64 / int64 numpy (exact for bf16 and fp32)."""
    t = t.detach().cpu()
    if t.dtype in (torch.bfloat16, torch.float16, torch.float32):
        return t.to(torch.float64).numpy()
    return t.numpy()


def assert_close(got, want, atol, rtol, what=""):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = np.abs(got - want) > atol + rtol * np.abs(want)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside atol={atol} rtol={rtol}; "
                             f"first at {tuple(i)}: got {got[tuple(i)]} want {want[tuple(i)]}; "
                             f"max abs err {np.abs(got - want).max():.3g}")
