"""Helpers shared by the GPU tests: bit transfers and the parity bar."""
import numpy as np
import torch

from oracle import attention as OA

# Parity bar: cosine >= 0.99998 (the equivalence threshold of the dense-mask
# check in the SegPagedAttention runtime explainer, section 4) and
# max |O_gpu - O_ref| <= 1e-2 over the compared outputs.
COS_MIN = 0.99998
MAX_ERR = 1e-2
# LSE is fp32 on the GPU; scores are fp32 sums of bf16 products.
LSE_ERR = 2e-3


def to_dev(bits: np.ndarray, dev="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


def to_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def to_f64(t: torch.Tensor) -> np.ndarray:
    return OA.bf16_bits_to_f64(to_bits(t))


def bf16_half_ulp(x: np.ndarray) -> np.ndarray:
    """Half the spacing of the bf16 grid at |x| (8 significant bits)."""
    a = np.maximum(np.abs(x), np.finfo(np.float32).tiny)
    return np.exp2(np.floor(np.log2(a)) - 8)


def parity(got: np.ndarray, ref: np.ndarray, what: str = ""):
    """cos >= 0.99998 and max|err| <= 1e-2 on the value the kernel computes.
    The kernel stores O as bf16, which rounds that value by up to half a bf16
    ulp (0.0078 at |O| in [2, 4)), so each stored element may differ from the
    fp64 oracle by 1e-2 plus half a bf16 ulp of the oracle value."""
    got = np.asarray(got, np.float64).ravel()
    ref = np.asarray(ref, np.float64).ravel()
    diff = np.abs(got - ref)
    err = float(np.max(diff)) if got.size else 0.0
    bound = MAX_ERR + bf16_half_ulp(ref)
    worst = float(np.max(diff / bound)) if got.size else 0.0
    nrm = np.linalg.norm(got) * np.linalg.norm(ref)
    cos = float(np.dot(got, ref) / nrm) if nrm > 0 else (1.0 if np.array_equal(got, ref) else 0.0)
    print(f"[parity] {what}: max|err| {err:.3e} (worst/bound {worst:.3f}) cos {cos:.8f} "
          f"n={got.size}", flush=True)
    assert worst <= 1.0, (what, err, worst)
    assert cos >= COS_MIN, (what, cos)
    return err, cos


def lse_parity(got: np.ndarray, ref: np.ndarray, what: str = ""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin), what
    assert np.all(got[~fin] == ref[~fin]), what
    err = float(np.max(np.abs(got[fin] - ref[fin]))) if fin.any() else 0.0
    assert err <= LSE_ERR, (what, err)
    return err
