"""fp64 definition of the pre-LayerNorm attention block (TEST INFRASTRUCTURE
ONLY: called from the tests, the smoke check and the benchmark's CPU leg,
never from the library).

Kernel-Inference-Engine page, encoder-layer chart: the block input x goes
through LayerNorm, the dense Q/K/V projections, softmax(Q K^T / sqrt(d)) V,
the dense output projection W_O, and the residual add of x.  The page's
fused kernel folds the LayerNorm into the attention's prologue; this module
computes the unfused definition:

    xhat = (x - mean(x)) / sqrt(var(x) + eps) * gamma + beta      (per row)
    qkv  = xhat @ W_qkv^T + b_qkv         columns [Q heads | K heads | V heads]
    o    = softmax(q k^T * scale) v        per (batch, head), the attention oracle
    y    = x + o @ W_o^T + b_o

mean and var are the plain population moments of the row (two passes in
IEEE double; the page's kernel uses Welford's one-pass update for the same
quantities).  The block's interface stores qkv and o in the 16-bit input
dtype between the stages (the page's kernels take FP16 Q, K, V); the oracle
rounds its double values to that dtype at exactly those two points
(round-to-nearest-even, through float32 as a float32 result is rounded)
and nowhere else.  The attention stage is ``oracle.attention_fwd``.

The library runs the block on the folded layer W' = W diag(gamma), b' = b +
W beta (``fold_weights``), whose W' is stored in the 16-bit dtype; the
``folded`` form of the block is that computation done exactly, the plain
form is the definition above.

Besides the values, the projections return the sums of absolute products
that a rounding-error bound for a 16-bit-operand, float32-accumulated
product needs (see ``ln_linear``, ``linear``).
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from . import attention_fwd, widen


def _f64(bits, dtype):
    return widen(np.ascontiguousarray(bits, np.uint16), dtype)


def round16(x: np.ndarray, dtype: str) -> np.ndarray:
    """Bits of the 16-bit dtype nearest to float32(x) (round to nearest even)."""
    x32 = np.ascontiguousarray(x, np.float64).astype(np.float32)
    if dtype == "f16":
        return x32.astype(np.float16).view(np.uint16)
    u = x32.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x32)
    r[nan] = 0x7FC0
    return r


def layernorm_stats(x_bits: np.ndarray, dtype: str, eps: float):
    """Per-row mean and 1/sqrt(var + eps) of x [T, C] (population variance)."""
    x = _f64(x_bits, dtype)
    mean = x.mean(axis=1)
    var = ((x - mean[:, None]) ** 2).mean(axis=1)
    return mean, 1.0 / np.sqrt(var + eps)


def layernorm(x_bits, dtype, gamma, beta, eps):
    """xhat [T, C] in double: the normalised rows scaled by gamma, shifted by beta."""
    x = _f64(x_bits, dtype)
    mean, rstd = layernorm_stats(x_bits, dtype, eps)
    g = np.asarray(gamma, np.float64)
    b = np.asarray(beta, np.float64)
    return (x - mean[:, None]) * rstd[:, None] * g[None, :] + b[None, :]


def ln_linear(x_bits, dtype, gamma, beta, w_bits, bias, eps):
    """The LayerNorm-ed rows through a dense layer: LN(x) @ W^T + bias.

    x: [T, C] bits; gamma, beta: [C]; w: [N, C] bits (output-major); bias: [N]
    or None.  Returns (y [T, N], absprod [T, N], rawprod [T, N]) where
    absprod = |(x - mean) * rstd| @ |gamma * W|^T bounds what a relative
    perturbation of the normalised operand or of the weights can move y, and
    rawprod = rstd * (|x| + |mean|) @ |gamma * W|^T bounds what float32
    accumulation of the un-centred products x @ (gamma * W)^T can move it.
    """
    x = _f64(x_bits, dtype)
    mean, rstd = layernorm_stats(x_bits, dtype, eps)
    g = np.asarray(gamma, np.float64)
    w = _f64(w_bits, dtype)
    y = layernorm(x_bits, dtype, gamma, beta, eps) @ w.T
    if bias is not None:
        y = y + np.asarray(bias, np.float64)[None, :]
    gw = np.abs(w * g[None, :])
    absprod = np.abs((x - mean[:, None]) * rstd[:, None]) @ gw.T
    rawprod = ((np.abs(x) + np.abs(mean)[:, None]) * rstd[:, None]) @ gw.T
    return y, absprod, rawprod


def linear(a_bits, dtype, w_bits, bias=None, residual_bits=None):
    """A dense layer with an optional residual: a @ W^T + bias + residual.

    a: [M, K] bits, w: [N, K] bits, bias: [N] or None, residual: [M, N] bits
    or None.  Returns (y [M, N], absprod = |a| @ |W|^T)."""
    a = _f64(a_bits, dtype)
    w = _f64(w_bits, dtype)
    y = a @ w.T
    if bias is not None:
        y = y + np.asarray(bias, np.float64)[None, :]
    if residual_bits is not None:
        y = y + _f64(residual_bits, dtype)
    return y, np.abs(a) @ np.abs(w).T


def fold_weights(gamma, beta, w_bits, bias, dtype):
    """A dense layer after LayerNorm, rewritten on the un-scaled normalised rows:
    LN(x) W^T + b = ((x - mean) rstd) W'^T + b' with W' = W diag(gamma) and
    b' = b + W beta.  W' is returned as the dtype's bits (gamma * w as a
    float32 product, rounded to nearest even): the stored form a 16-bit
    layer holds; b' in double (bias None = 0)."""
    w = _f64(w_bits, dtype)
    g = np.asarray(gamma, np.float64)
    wf_bits = round16(w * g[None, :], dtype)
    bf = w @ np.asarray(beta, np.float64)
    if bias is not None:
        bf = bf + np.asarray(bias, np.float64)
    return wf_bits, bf


def ln_linear_folded(x_bits, dtype, wf_bits, bias_folded, eps):
    """((x - mean) rstd) W'^T + b' in double, for folded weights (see
    ``fold_weights``).  Returns (y, rawprod) with rawprod = rstd (|x| +
    |mean|) @ |W'|^T, the float32-accumulation bound's sum."""
    x = _f64(x_bits, dtype)
    mean, rstd = layernorm_stats(x_bits, dtype, eps)
    wf = _f64(wf_bits, dtype)
    xn = (x - mean[:, None]) * rstd[:, None]
    y = xn @ wf.T + np.asarray(bias_folded, np.float64)[None, :]
    rawprod = ((np.abs(x) + np.abs(mean)[:, None]) * rstd[:, None]) @ np.abs(wf).T
    return y, rawprod


def prenorm_attention(x_bits, dtype, gamma, beta, w_qkv_bits, b_qkv, w_o_bits, b_o,
                      B: int, N: int, H: int, Hkv: int, d: int, eps: float, scale: float,
                      causal: bool, kv_lens: Optional[np.ndarray] = None, nthreads: int = 0,
                      tokens: Optional[np.ndarray] = None, folded: bool = False):
    """The whole block on x [B*N, C] (token t = b*N + n), C = H*d.

    w_qkv: [(H + 2*Hkv)*d, C] bits, b_qkv: [(H + 2*Hkv)*d]; w_o: [C, H*d] bits,
    b_o: [C].  Returns a dict with every stage: ``qkv`` (double), ``qkv_bits``,
    ``o`` (double attention output [B*N, H*d], from the rounded qkv),
    ``o_bits``, ``lse`` [B, H, N], ``y`` (double, from the rounded o) and
    ``oprod`` = |o| @ |W_o|^T.  ``tokens``: optional token ids; then qkv is
    still formed for every token (keys and values need it) but ``o``,
    ``o_bits``, ``y`` and ``oprod`` hold only those tokens' rows, in the given
    order, and ``lse`` is [len(tokens), H].  ``folded``: form qkv from the
    folded layer (``fold_weights``: gamma W stored in the dtype) instead of
    from gamma, beta and W directly.
    """
    T = B * N
    C = H * d
    R = (H + 2 * Hkv) * d
    assert x_bits.shape == (T, C) and w_qkv_bits.shape == (R, C) and w_o_bits.shape == (C, H * d)
    if folded:
        wf_bits, bf = fold_weights(gamma, beta, w_qkv_bits, b_qkv, dtype)
        qkv, _ = ln_linear_folded(x_bits, dtype, wf_bits, bf, eps)
    else:
        qkv, _, _ = ln_linear(x_bits, dtype, gamma, beta, w_qkv_bits, b_qkv, eps)
    qkv_bits = round16(qkv, dtype)
    heads = qkv_bits.reshape(B, N, H + 2 * Hkv, d)
    q = np.ascontiguousarray(heads[:, :, :H].transpose(0, 2, 1, 3))
    k = np.ascontiguousarray(heads[:, :, H:H + Hkv].transpose(0, 2, 1, 3))
    v = np.ascontiguousarray(heads[:, :, H + Hkv:].transpose(0, 2, 1, 3))
    if tokens is None:
        o4, lse = attention_fwd(q, k, v, dtype, scale, causal, kv_lens, nthreads=nthreads)
        o = np.ascontiguousarray(o4.transpose(0, 2, 1, 3)).reshape(T, H * d)
        res_bits = x_bits
    else:
        tok = np.asarray(tokens, np.int64).reshape(-1)
        b, n = tok // N, tok % N
        # attention rows (b*H + h)*N + n of every head of each token
        rows = ((b[:, None] * H + np.arange(H)[None, :]) * N + n[:, None]).reshape(-1)
        o_r, lse_r = attention_fwd(q, k, v, dtype, scale, causal, kv_lens, rows=rows,
                                   nthreads=nthreads)
        o = o_r.reshape(tok.size, H * d)
        lse = lse_r.reshape(tok.size, H)
        res_bits = np.ascontiguousarray(x_bits[tok])
    o_bits = round16(o, dtype)
    y, oprod = linear(o_bits, dtype, w_o_bits, b_o, res_bits)
    return dict(qkv=qkv, qkv_bits=qkv_bits, o=o, o_bits=o_bits, lse=lse, y=y, oprod=oprod)
