"""Helpers shared by the GPU parity tests (device transfer, tolerance)."""
import numpy as np
import torch

# fp outputs: |gpu - oracle| <= ATOL + RTOL * |oracle|, elementwise
ATOL = 1e-3
RTOL = 2e-3


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def dev_u8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def dev_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def assert_close(gpu: np.ndarray, ref: np.ndarray, what: str = ""):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    err = np.abs(gpu - ref)
    lim = ATOL + RTOL * np.abs(ref)
    bad = ~(err <= lim)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside tolerance; first at {tuple(i)}: "
                             f"gpu={gpu[tuple(i)]!r} ref={ref[tuple(i)]!r}")


def bf16_round_f64(a: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).double().numpy()
