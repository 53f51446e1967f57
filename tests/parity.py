"""Shared helpers of the GPU parity tests: run the HIP path through the
binding, compare with the fp64 oracle at the stated tolerances."""
from __future__ import annotations

import os

import numpy as np

import fa_inputs as gen

# Parity bar for f16/bf16 inputs: max |dO| <= 1e-2, mean |dO| <= 1e-3 over
# every compared element; LSE within 1e-3 relative, read as
# |dLSE| <= 1e-3 * max(1, |LSE|) (plain relative error is ill-conditioned
# where LSE crosses zero, e.g. causal row 0 whose LSE is one score).
TOL_MAX = 1e-2
TOL_MEAN = 1e-3
TOL_LSE = 1e-3


# O stored in 16 bits: the kernel forms O in fp32 (held to the bar above) and
# rounds it to nearest even, which adds at most half an ulp of the stored
# value: <= 2^-8 |O| (bf16) or 2^-11 |O| (f16, plus 2^-25 below its normal
# range).  That bound is added to the O bars element by element.
HALF_ULP_REL = {"f32": 0.0, "bf16": 2.0 ** -8, "f16": 2.0 ** -11}
HALF_ULP_ABS = {"f32": 0.0, "bf16": 0.0, "f16": 2.0 ** -25}


def compare(o, lse, o_ref, lse_ref, what="", out_dtype="f32"):
    o = np.asarray(o, np.float64)
    lse = np.asarray(lse, np.float64)
    ref_inf = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse), ref_inf), f"{what}: -inf LSE rows differ"
    assert np.all(np.isfinite(o)), f"{what}: non-finite O"
    rounding = HALF_ULP_REL[out_dtype] * np.abs(o_ref) + HALF_ULP_ABS[out_dtype]
    err = np.maximum(np.abs(o - o_ref) - rounding, 0.0)
    max_abs = float(err.max(initial=0.0))
    mean_abs = float(err.mean()) if err.size else 0.0
    fin = ~ref_inf
    lse_err = np.abs(lse[fin] - lse_ref[fin]) / np.maximum(1.0, np.abs(lse_ref[fin]))
    lse_rel = float(lse_err.max(initial=0.0))
    stats = dict(max_abs=max_abs, mean_abs=mean_abs, lse_rel=lse_rel)
    assert max_abs <= TOL_MAX, f"{what}: max abs {max_abs:.3e} {stats}"
    assert mean_abs <= TOL_MEAN, f"{what}: mean abs {mean_abs:.3e} {stats}"
    assert lse_rel <= TOL_LSE, f"{what}: lse {lse_rel:.3e} {stats}"
    return stats


def host_cores(cap=16):
    """Threads for the oracle at full size: the cores this process may run on,
    at most `cap` (a GPU machine shares its host between its GPUs)."""
    return max(1, min(cap, len(os.sched_getaffinity(0))))


def device_tensors(w: gen.FwdInputs, device="cuda"):
    import torch

    q = gen.to_torch(w.q, w.dtype).to(device)
    k = gen.to_torch(w.k, w.dtype).to(device)
    v = gen.to_torch(w.v, w.dtype).to(device)
    kl = None if w.kv_lens is None else torch.from_numpy(w.kv_lens).to(device)
    return q, k, v, kl


def gpu_forward(w: gen.FwdInputs, device="cuda"):
    import torch

    import flashattention_forward_03_amd as fa

    q, k, v, kl = device_tensors(w, device)
    o, lse = fa.forward(q, k, v, scale=w.scale, causal=w.causal, kv_lens=kl)
    torch.cuda.synchronize()
    return o.cpu().numpy(), lse.cpu().numpy()


def sample_rows(B, H, Nq, n_random, seed, full_heads=((0, 0),), edge=128):
    """Flat row ids: every edge row (first and last `edge`) of a few heads, and
    n_random rows spread over all heads."""
    rng = np.random.default_rng(seed)
    rows = []
    for b, h in full_heads:
        base = (b * H + h) * Nq
        rows.extend(range(base, base + min(edge, Nq)))
        rows.extend(range(base + max(0, Nq - edge), base + Nq))
    rows.extend(rng.integers(0, B * H * Nq, size=n_random).tolist())
    return np.unique(np.array(rows, np.int64))


# Gradients (dQ, dK, dV, and the row term D): the bar of the gpu-inference
# page's backward checks (section 02: every gradient held to the reference
# with allclose at atol = rtol = 1e-2), elementwise: |x - ref| <= 1e-2 +
# 1e-2 |ref|.  No separate mean bar: each gradient element is a sum of
# products with 16-bit-rounded factors (P and dS enter the MFMAs rounded),
# so its error scales with the sum of |terms|, which cancellation can make
# much larger than |ref|; the mean error is reported.
GRAD_ATOL = 1e-2
GRAD_RTOL = 1e-2


def compare_grad(x, ref, what=""):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    assert x.shape == ref.shape, f"{what}: shape {x.shape} vs {ref.shape}"
    assert np.all(np.isfinite(x)), f"{what}: non-finite values"
    err = np.abs(x - ref)
    excess = err - (GRAD_ATOL + GRAD_RTOL * np.abs(ref))
    worst = float(excess.max(initial=-np.inf))
    stats = dict(max_abs=float(err.max(initial=0.0)),
                 mean_abs=float(err.mean()) if err.size else 0.0, worst_excess=worst)
    assert worst <= 0.0, f"{what}: outside atol/rtol {stats}"
    return stats
