"""Shared helpers of the GPU parity tests (host-side comparison only)."""
import numpy as np
import pytest
import torch

gpu = pytest.mark.gpu
needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")

# Output tolerance of the pages' target: max-abs error <= 1e-2 x rms(reference)
# for bf16 weights with fp32 accumulation.
TOL = 1e-2


def rel_maxabs(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt(np.mean(ref ** 2))
    if rms == 0.0:
        return float(np.max(np.abs(got))) if got.size else 0.0
    return float(np.max(np.abs(got - ref)) / rms) if got.size else 0.0


def assert_close(got, ref, tol=TOL, what=""):
    e = rel_maxabs(got, ref)
    assert e <= tol, f"{what}: max|err| / rms(ref) = {e:.3e} > {tol}"
    return e


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def host_u32(t: torch.Tensor) -> np.ndarray:
    return host(t).view(np.uint32)


def dev(a: np.ndarray, device="cuda") -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    if a.dtype == np.uint32:
        a = a.view(np.int32)
    return torch.from_numpy(a).to(device)


def banner(msg: str) -> None:
    print(f"[gpu-case] {msg}", flush=True)
