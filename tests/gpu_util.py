"""Helpers for the GPU parity tests (device transfer of seeded inputs, error metrics)."""
import numpy as np
import torch

ATOL_MAX = 1e-2    # attention: max-abs error vs the fp64 oracle (bf16 inputs)
ATOL_MEAN = 1e-3   # attention: mean-abs error
# attention: relative L2 error ||O - O_ref|| / ||O_ref|| over the compared rows.  |O| shrinks
# like sqrt(e / N) with the key count (about 0.01 at N = 25600), which makes the absolute
# bounds loose at large N; the kernel rounds P and O to bf16 (relative error <= 2^-9 each),
# so its relative L2 error is a few 1e-3 at most, far below this bound.
REL_L2 = 1e-2
LSE_ATOL = 1e-3


def dev():
    return torch.device("cuda:0")


def to_dev_bf16(t) -> torch.Tensor:
    """A workloads.Bf16Tensor's bit pattern as a device bfloat16 tensor."""
    return torch.from_numpy(np.ascontiguousarray(t.bits).view(np.int16)).to(dev()).view(torch.bfloat16)


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def attn_errors(got, ref: np.ndarray) -> dict:
    """max-abs, mean-abs and relative L2 error of an attention output against the oracle."""
    g = got.float().cpu().numpy().astype(np.float64) if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    err = np.abs(g - ref)
    nref = float(np.sqrt(np.sum(ref * ref)))
    return {"max_abs": float(err.max()) if err.size else 0.0,
            "mean_abs": float(err.mean()) if err.size else 0.0,
            "rel_l2": float(np.sqrt(np.sum(err * err))) / nref if nref > 0 else float(np.sqrt(np.sum(err * err))),
            "finite": bool(np.isfinite(g).all())}


def assert_attn_close(got: torch.Tensor, ref: np.ndarray, what: str = ""):
    e = attn_errors(got, ref)
    assert e["finite"], f"{what}: non-finite output"
    assert e["max_abs"] <= ATOL_MAX and e["mean_abs"] <= ATOL_MEAN and e["rel_l2"] <= REL_L2, \
        f"{what}: max-abs {e['max_abs']:.3e} mean-abs {e['mean_abs']:.3e} rel-L2 {e['rel_l2']:.3e}"
    return e["max_abs"], e["mean_abs"]


def assert_lse_close(got: torch.Tensor, ref: np.ndarray, what: str = ""):
    g = got.cpu().numpy().astype(np.float64)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(g), fin), f"{what}: -inf pattern differs"
    if fin.any():
        err = float(np.abs(g[fin] - ref[fin]).max())
        assert err <= LSE_ATOL, f"{what}: LSE max-abs {err:.3e}"
