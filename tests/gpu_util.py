"""Helpers shared by the GPU tests: bit transfers, the parity bar, and a record
of every comparison (printed per test family at the end of the run)."""
import os

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

# (family, what, max|err|, worst err/bound, cos, min per-(layer, Q head) cos)
RECORDS = []


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


def parity_bound(ref: np.ndarray) -> np.ndarray:
    """Per-element bound: 1e-2, except where bf16 cannot hold a value within 1e-2
    of the oracle (|O| >= 4, half a bf16 step above 1e-2): there, rounding the
    exact value plus 1e-3 of computation."""
    return np.maximum(MAX_ERR, bf16_half_ulp(ref) + 1e-3)


def _cos(a: np.ndarray, b: np.ndarray) -> float:
    nrm = np.linalg.norm(a) * np.linalg.norm(b)
    return float(np.dot(a, b) / nrm) if nrm > 0 else (1.0 if np.array_equal(a, b) else 0.0)


def _family() -> str:
    cur = os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0]
    return cur.split("[")[0]


def parity(got: np.ndarray, ref: np.ndarray, what: str = "", head_axis: int = -2):
    """cos >= 0.99998 and max|err| <= 1e-2 (parity_bound per element). With 3 or
    more dimensions, axis `head_axis` holds the query heads, and the smallest
    cosine over single heads is recorded too."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    head_cos = None
    if got.ndim >= 3 and got.size:
        g2 = np.moveaxis(got, head_axis, 0).reshape(got.shape[head_axis], -1)
        r2 = np.moveaxis(ref, head_axis, 0).reshape(ref.shape[head_axis], -1)
        head_cos = min(_cos(g2[h], r2[h]) for h in range(g2.shape[0]))
    got = got.ravel()
    ref = ref.ravel()
    diff = np.abs(got - ref)
    err = float(np.max(diff)) if got.size else 0.0
    worst = float(np.max(diff / parity_bound(ref))) if got.size else 0.0
    cos = _cos(got, ref)
    RECORDS.append((_family(), what, err, worst, cos, head_cos))
    hc = f" min head cos {head_cos:.8f}" if head_cos is not None else ""
    print(f"[parity] {what}: max|err| {err:.3e} (worst/bound {worst:.3f}) cos {cos:.8f}{hc} "
          f"n={got.size}", flush=True)
    assert worst <= 1.0, (what, err, worst)
    assert cos >= COS_MIN, (what, cos)
    return err, cos


def counter_lines(plan):
    """[begin, end) of the prefill work-counter lines in a plan's device image: L + 1
    lines of 16 ints, followed only by the append list of a growth plan."""
    tail = 2 * plan.num_seqs + 1 if plan.append_capacity > 0 else 0
    end = plan.sizes.table_int32s - tail
    return end - 16 * (plan.num_layers + 1), end


def assert_image_equal(dev_table, plan):
    """The device image equals the plan's host image, except that a prefill call
    leaves its generation in the high word of its counter (the next-item word is
    back at zero)."""
    host = plan.table_host()
    dev = np.asarray(dev_table)[:len(host)].copy()
    c0, c1 = counter_lines(plan)
    lines = dev[c0:c1].reshape(-1, 16)
    assert np.all(lines[:, 0] == 0) and np.all(lines[:, 2:] == 0), lines
    lines[:, 1] = 0
    dev[c0:c1] = lines.ravel()
    assert np.array_equal(dev, host)


def lse_parity(got: np.ndarray, ref: np.ndarray, what: str = ""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin), what
    assert np.all(got[~fin] == ref[~fin]), what
    err = float(np.max(np.abs(got[fin] - ref[fin]))) if fin.any() else 0.0
    assert err <= LSE_ERR, (what, err)
    return err


def summary_lines():
    """Per test family: comparisons, worst max|err|, worst err/bound, smallest
    cosine of a call and of a single (layer, Q head)."""
    fam = {}
    for f, what, err, worst, cos, hcos in RECORDS:
        d = fam.setdefault(f, {"n": 0, "err": 0.0, "worst": 0.0, "what": "", "cos": 1.0,
                               "hcos": None})
        d["n"] += 1
        d["err"] = max(d["err"], err)
        if worst >= d["worst"]:
            d["worst"], d["what"] = worst, what
        d["cos"] = min(d["cos"], cos)
        if hcos is not None:
            d["hcos"] = hcos if d["hcos"] is None else min(d["hcos"], hcos)
    lines = []
    for f in sorted(fam):
        d = fam[f]
        hc = f"{d['hcos']:.8f}" if d["hcos"] is not None else "-"
        lines.append(f"{f}: n={d['n']} max|err| {d['err']:.3e} worst/bound {d['worst']:.3f} "
                     f"({d['what']}) min cos {d['cos']:.8f} min head cos {hc}")
    if RECORDS:
        w = max(RECORDS, key=lambda r: r[3])
        hc = [r[5] for r in RECORDS if r[5] is not None]
        lines.append(f"ALL: n={len(RECORDS)} max|err| {max(r[2] for r in RECORDS):.3e} "
                     f"worst/bound {w[3]:.3f} ({w[1]}) min cos {min(r[4] for r in RECORDS):.8f} "
                     f"min head cos {min(hc) if hc else float('nan'):.8f}")
    return lines
