"""Helpers for the GPU parity tests (device transfer of seeded inputs, error metrics)."""
import numpy as np
import torch

ATOL_MAX = 1e-2    # attention: max-abs error vs the fp64 oracle (bf16 inputs)
ATOL_MEAN = 1e-3   # attention: mean-abs error
LSE_ATOL = 1e-3


def dev():
    return torch.device("cuda:0")


def to_dev_bf16(t) -> torch.Tensor:
    """A workloads.Bf16Tensor's bit pattern as a device bfloat16 tensor."""
    return torch.from_numpy(np.ascontiguousarray(t.bits).view(np.int16)).to(dev()).view(torch.bfloat16)


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def assert_attn_close(got: torch.Tensor, ref: np.ndarray, what: str = ""):
    g = got.float().cpu().numpy().astype(np.float64)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    err = np.abs(g - ref)
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    mx, mean = float(err.max()) if err.size else 0.0, float(err.mean()) if err.size else 0.0
    assert mx <= ATOL_MAX and mean <= ATOL_MEAN, f"{what}: max-abs {mx:.3e} mean-abs {mean:.3e}"
    return mx, mean


def assert_lse_close(got: torch.Tensor, ref: np.ndarray, what: str = ""):
    g = got.cpu().numpy().astype(np.float64)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(g), fin), f"{what}: -inf pattern differs"
    if fin.any():
        err = float(np.abs(g[fin] - ref[fin]).max())
        assert err <= LSE_ATOL, f"{what}: LSE max-abs {err:.3e}"
