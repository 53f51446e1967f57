"""Pins for the fp64 pre-LayerNorm block oracle (``oracle.block``): closed forms,
invariants of the normalisation, an independent pure-Python brute force of the
whole block on tiny shapes, and special weights whose result is known.

Definitions: LayerNorm as on the Kernel-Inference-Engine page (the LayerNorm
kernel's per-row mean and variance, applied before the dense Q/K/V layers in
the encoder-layer chart), population variance with eps under the root; the
block as that chart draws it (LN, dense QKV, softmax(QK^T/sqrt(d)) V, dense
W_O, residual)."""
import math
import struct

import numpy as np
import pytest

import fa_inputs as gen
from oracle import block as ob
from oracle import brute



def _bits(vals, dtype):
    return gen.float_to_bits_exact(np.asarray(vals, np.float32), dtype)


# ----------------------------------------------------------- layernorm ---

@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_layernorm_closed_form_row(dtype):
    x = _bits([[1, 2, 3, 4]], dtype)               # mean 2.5, variance 1.25
    mean, rstd = ob.layernorm_stats(x, dtype, 0.0)
    assert mean[0] == 2.5 and abs(rstd[0] - 1 / math.sqrt(1.25)) < 1e-15
    y = ob.layernorm(x, dtype, np.ones(4), np.zeros(4), 0.0)
    want = (np.array([1, 2, 3, 4]) - 2.5) / math.sqrt(1.25)
    assert np.allclose(y[0], want, rtol=0, atol=1e-15)


@pytest.mark.parametrize("dtype,row", [
    ("f16", [999.5, 1000.0, 1000.5]),     # offset 2000x the spread
    ("bf16", [254.0, 256.0, 258.0]),
])
def test_layernorm_large_offset_row(dtype, row):
    """Three equally spaced values normalise to -sqrt(3/2), 0, sqrt(3/2)
    whatever their offset (population variance of (-a, 0, a) is 2a^2/3)."""
    y = ob.layernorm(_bits([row], dtype), dtype, np.ones(3), np.zeros(3), 0.0)
    s = math.sqrt(1.5)
    assert np.allclose(y[0], [-s, 0.0, s], rtol=0, atol=1e-12)


@pytest.mark.parametrize("eps", [0.0, 1e-5, 0.5])
def test_layernorm_moments(eps):
    w = gen.block_inputs(3, 17, 2, 32, "bf16", 11, row_offset=5.0)
    x = gen.bits_to_float(w.x, "bf16").astype(np.float64)
    var = x.var(axis=1)
    y = ob.layernorm(w.x, "bf16", np.ones(w.C), np.zeros(w.C), eps)
    assert np.allclose(y.mean(axis=1), 0.0, atol=1e-12)
    assert np.allclose((y ** 2).mean(axis=1), var / (var + eps), rtol=1e-12, atol=0)
    # gamma and beta act per column: undoing them restores the moments
    g = w.gamma.astype(np.float64)
    b = w.beta.astype(np.float64)
    z = (ob.layernorm(w.x, "bf16", w.gamma, w.beta, eps) - b) / g
    assert np.allclose(z, y, rtol=0, atol=1e-12)


def test_layernorm_shift_invariance():
    x = _bits(np.arange(-8, 8, dtype=np.float32).reshape(2, 8) * 0.25, "f16")
    x2 = _bits(np.arange(-8, 8, dtype=np.float32).reshape(2, 8) * 0.25 + 64, "f16")
    g = np.linspace(0.5, 1.5, 8)
    b = np.linspace(-1, 1, 8)
    assert np.allclose(ob.layernorm(x, "f16", g, b, 1e-5), ob.layernorm(x2, "f16", g, b, 1e-5),
                       rtol=0, atol=1e-13)


# ----------------------------------------------------- brute force ---

def _py_round16(v, dtype):
    """Pure-Python round to nearest even of float32(v) to the 16-bit dtype."""
    if dtype == "f16":
        return struct.unpack("<e", struct.pack("<e", struct.unpack("<f", struct.pack("<f", v))[0]))[0]
    u = struct.unpack("<I", struct.pack("<f", v))[0]
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return struct.unpack("<f", struct.pack("<I", (u << 16) & 0xFFFFFFFF))[0]


def _py_ln(row, g, b, eps):
    n = len(row)
    m = math.fsum(row) / n
    var = math.fsum((a - m) ** 2 for a in row) / n
    r = 1.0 / math.sqrt(var + eps)
    return [(a - m) * r * gg + bb for a, gg, bb in zip(row, g, b)], m, r


def _py_dense(rows, w, bias):
    return [[math.fsum(a * b for a, b in zip(row, wr)) + (bias[j] if bias is not None else 0.0)
             for j, wr in enumerate(w)] for row in rows]


def _lists(bits, dtype):
    return gen.bits_to_float(bits, dtype).astype(np.float64).tolist()


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_ln_linear_brute_force(dtype):
    w = gen.block_inputs(1, 3, 1, 8, dtype, 21, row_offset=3.0)   # T 3, C 8, R 24
    eps = 1e-5
    x = _lists(w.x, dtype)
    W = _lists(w.w_qkv, dtype)
    g = w.gamma.astype(np.float64).tolist()
    b = w.beta.astype(np.float64).tolist()
    lns = [_py_ln(r, g, b, eps) for r in x]
    want = _py_dense([t[0] for t in lns], W, w.b_qkv.astype(np.float64).tolist())
    y, absprod, rawprod = ob.ln_linear(w.x, dtype, w.gamma, w.beta, w.w_qkv, w.b_qkv, eps)
    assert np.allclose(y, want, rtol=1e-12, atol=1e-12)
    for i, (_, m, r) in enumerate(lns):
        for j in range(len(W)):
            ap = math.fsum(abs((x[i][k] - m) * r) * abs(g[k] * W[j][k]) for k in range(8))
            rp = math.fsum((abs(x[i][k]) + abs(m)) * r * abs(g[k] * W[j][k]) for k in range(8))
            assert abs(absprod[i, j] - ap) <= 1e-12 * ap and abs(rawprod[i, j] - rp) <= 1e-12 * rp


def test_ln_linear_identity_weights():
    """W = I: the projection returns the normalised rows plus the bias."""
    w = gen.block_inputs(2, 4, 2, 8, "bf16", 22)
    C = w.C
    eye = gen.float_to_bits_exact(np.eye(C, dtype=np.float32), "bf16")
    bias = np.linspace(-1, 1, C)
    y, _, _ = ob.ln_linear(w.x, "bf16", w.gamma, w.beta, eye, bias, 1e-5)
    assert np.allclose(y, ob.layernorm(w.x, "bf16", w.gamma, w.beta, 1e-5) + bias, rtol=0, atol=1e-14)


def test_linear_brute_force_and_residual():
    rng = np.random.default_rng(5)
    a = gen.round_bits(rng.standard_normal((3, 16), dtype=np.float32), "f16")
    W = gen.round_bits(rng.standard_normal((5, 16), dtype=np.float32), "f16")
    res = gen.round_bits(rng.standard_normal((3, 5), dtype=np.float32), "f16")
    bias = rng.standard_normal(5)
    y, absprod = ob.linear(a, "f16", W, bias, res)
    want = _py_dense(_lists(a, "f16"), _lists(W, "f16"), bias.tolist())
    want = np.array(want) + gen.bits_to_float(res, "f16")
    assert np.allclose(y, want, rtol=1e-13, atol=1e-13)
    ab = np.abs(gen.bits_to_float(a, "f16").astype(np.float64))
    aw = np.abs(gen.bits_to_float(W, "f16").astype(np.float64))
    assert np.allclose(absprod, [[math.fsum(ab[i] * aw[j]) for j in range(5)] for i in range(3)],
                       rtol=1e-13)


def test_round16_matches_torch_bf16_and_numpy_f16():
    """The oracle's own rounding agrees with torch's float32 -> bfloat16 and
    numpy's float32 -> float16 (both round to nearest even), ties included."""
    rng = np.random.default_rng(9)
    x = rng.standard_normal(20000).astype(np.float32) * 100
    u = x.view(np.uint32)
    ties = ((u & 0xFFFF0000) | 0x8000).view(np.float32)[:500]   # exact bf16 ties
    x = np.concatenate([x, ties, [0.0, -0.0, 65504.0, 1e-8]]).astype(np.float32)
    assert np.array_equal(ob.round16(x.astype(np.float64), "bf16"), gen.round_bits(x, "bf16"))
    assert np.array_equal(ob.round16(x.astype(np.float64), "f16"), gen.round_bits(x, "f16"))


@pytest.mark.parametrize("dtype,causal,Hkv,lens", [
    ("bf16", False, 2, None),
    ("f16", True, 1, None),          # multi-query heads, causal
    ("bf16", False, 2, (1, 3)),      # key padding
])
def test_block_brute_force(dtype, causal, Hkv, lens):
    """Every stage of the block against pure-Python loops (LayerNorm, both dense
    layers, 16-bit storage of qkv and o, the attention brute force)."""
    B, N, H, d = 2, 3, 2, 4
    w = gen.block_inputs(B, N, H, d, dtype, 31 + Hkv, Hkv=Hkv, causal=causal,
                         kv_len_range=lens, row_offset=2.0)
    C, R = H * d, (H + 2 * Hkv) * d
    res = ob.prenorm_attention(w.x, dtype, w.gamma, w.beta, w.w_qkv, w.b_qkv, w.w_o, w.b_o,
                               B, N, H, Hkv, d, w.eps, w.scale, causal, w.kv_lens)
    x = _lists(w.x, dtype)
    g, b = w.gamma.astype(np.float64).tolist(), w.beta.astype(np.float64).tolist()
    xhat = [_py_ln(r, g, b, w.eps)[0] for r in x]
    qkv = _py_dense(xhat, _lists(w.w_qkv, dtype), w.b_qkv.astype(np.float64).tolist())
    assert np.allclose(res["qkv"], qkv, rtol=1e-12, atol=1e-12)
    qkv16 = [[_py_round16(v, dtype) for v in row] for row in qkv]
    assert np.array_equal(gen.bits_to_float(res["qkv_bits"], dtype), np.array(qkv16, np.float32))
    o = [[0.0] * C for _ in range(B * N)]
    lse = np.zeros((B, H, N))
    for bb in range(B):
        for h in range(H):
            kh = h // (H // Hkv)
            rows = range(bb * N, bb * N + N)
            q = [qkv16[t][h * d:(h + 1) * d] for t in rows]
            k = [qkv16[t][(H + kh) * d:(H + kh + 1) * d] for t in rows]
            v = [qkv16[t][(H + Hkv + kh) * d:(H + Hkv + kh + 1) * d] for t in rows]
            kl = None if w.kv_lens is None else int(w.kv_lens[bb])
            oo, ll = brute.attention(q, k, v, w.scale, causal, kl)
            for i, t in enumerate(rows):
                o[t][h * d:(h + 1) * d] = oo[i]
            lse[bb, h] = ll
    assert np.allclose(res["o"], o, rtol=1e-12, atol=1e-12)
    assert np.allclose(res["lse"], lse, rtol=1e-12, atol=1e-12)
    o16 = [[_py_round16(v, dtype) for v in row] for row in o]
    y = _py_dense(o16, _lists(w.w_o, dtype), w.b_o.astype(np.float64).tolist())
    y = [[a + r for a, r in zip(yr, xr)] for yr, xr in zip(y, x)]
    assert np.allclose(res["y"], y, rtol=1e-12, atol=1e-12)
    assert R == res["qkv"].shape[1]


def test_block_zero_qkv_weights_closed_form():
    """W_qkv = 0: every token's q, k, v are the biases, all scores are equal
    and each head's output is its V bias, so y = x + round(b_v) W_o^T + b_o.
    Distinct Q, K and V biases catch a misplaced column split."""
    B, N, H, Hkv, d = 2, 5, 4, 2, 8
    w = gen.block_inputs(B, N, H, d, "bf16", 41, Hkv=Hkv, causal=True)
    R = (H + 2 * Hkv) * d
    zero = np.zeros((R, H * d), np.uint16)
    bq = np.linspace(-3, 3, H * d)
    bk = np.linspace(2, -2, Hkv * d)
    bv = np.linspace(-1, 1, Hkv * d) + 0.37
    res = ob.prenorm_attention(w.x, "bf16", w.gamma, w.beta, zero, np.concatenate([bq, bk, bv]),
                               w.w_o, w.b_o, B, N, H, Hkv, d, w.eps, w.scale, True)
    v16 = gen.bits_to_float(ob.round16(bv, "bf16"), "bf16").astype(np.float64)
    o_head = np.concatenate([v16[(h // (H // Hkv)) * d:(h // (H // Hkv) + 1) * d] for h in range(H)])
    assert np.allclose(res["o"], np.broadcast_to(o_head, (B * N, H * d)), rtol=0, atol=1e-14)
    wo = gen.bits_to_float(w.w_o, "bf16").astype(np.float64)
    x = gen.bits_to_float(w.x, "bf16").astype(np.float64)
    o16 = gen.bits_to_float(ob.round16(o_head, "bf16"), "bf16").astype(np.float64)
    assert np.allclose(res["y"], x + o16 @ wo.T + w.b_o, rtol=0, atol=1e-12)


def test_block_zero_output_weights_is_identity():
    w = gen.block_inputs(1, 7, 2, 16, "f16", 42)
    zero = np.zeros_like(w.w_o)
    res = ob.prenorm_attention(w.x, "f16", w.gamma, w.beta, w.w_qkv, w.b_qkv, zero,
                               np.zeros(w.C), 1, 7, 2, 2, 16, w.eps, w.scale, False)
    assert np.array_equal(res["y"], gen.bits_to_float(w.x, "f16").astype(np.float64))


def test_block_sampled_tokens_match_the_full_block():
    """The sampled-token form returns the full block's rows for those tokens."""
    B, N, H, Hkv, d = 2, 9, 4, 2, 16
    w = gen.block_inputs(B, N, H, d, "bf16", 43, Hkv=Hkv, causal=True, kv_len_range=(3, 9))
    args = (w.x, "bf16", w.gamma, w.beta, w.w_qkv, w.b_qkv, w.w_o, w.b_o, B, N, H, Hkv, d, w.eps,
            w.scale, True, w.kv_lens)
    full = ob.prenorm_attention(*args)
    tok = np.array([17, 0, 9, 5])
    part = ob.prenorm_attention(*args, tokens=tok)
    assert np.array_equal(part["qkv"], full["qkv"])
    for key in ("o", "o_bits", "y", "oprod"):
        assert np.array_equal(part[key], full[key][tok]), key
    lse_full = full["lse"].transpose(0, 2, 1).reshape(B * N, H)
    assert np.array_equal(part["lse"], lse_full[tok])


def test_fold_identity_with_exact_scales():
    """With gamma a power of two per column, gamma * W is exact in the dtype and
    the folded layer equals LN(x) W^T + b (the identity the fold rests on)."""
    w = gen.block_inputs(2, 6, 2, 32, "bf16", 51)
    rng = np.random.default_rng(3)
    gamma = (2.0 ** rng.integers(-2, 3, size=w.C)).astype(np.float32)
    wf, bf = ob.fold_weights(gamma, w.beta, w.w_qkv, w.b_qkv, "bf16")
    W = gen.bits_to_float(w.w_qkv, "bf16").astype(np.float64)
    assert np.array_equal(gen.bits_to_float(wf, "bf16").astype(np.float64), W * gamma)
    y_fold, _ = ob.ln_linear_folded(w.x, "bf16", wf, bf, w.eps)
    y_def, _, _ = ob.ln_linear(w.x, "bf16", gamma, w.beta, w.w_qkv, w.b_qkv, w.eps)
    assert np.allclose(y_fold, y_def, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_fold_rounds_like_a_float32_product(dtype):
    """W' is gamma * w formed in float32 and rounded to the dtype: equal to
    torch's / numpy's rounding of the float32 product."""
    w = gen.block_inputs(1, 4, 2, 32, dtype, 52)
    wf, _ = ob.fold_weights(w.gamma, w.beta, w.w_qkv, None, dtype)
    prod32 = gen.bits_to_float(w.w_qkv, dtype) * w.gamma[None, :]
    assert prod32.dtype == np.float32
    assert np.array_equal(wf, gen.round_bits(prod32, dtype))


def test_folded_block_close_to_the_definition():
    """The folded block differs from the definition only by the dtype rounding
    of gamma W: within u |xhat| . |gamma W| on qkv."""
    B, N, H, Hkv, d = 2, 8, 2, 1, 32
    w = gen.block_inputs(B, N, H, d, "f16", 53, Hkv=Hkv)
    args = (w.x, "f16", w.gamma, w.beta, w.w_qkv, w.b_qkv, w.w_o, w.b_o, B, N, H, Hkv, d, w.eps,
            w.scale, False)
    a = ob.prenorm_attention(*args)
    f = ob.prenorm_attention(*args, folded=True)
    _, absprod, _ = ob.ln_linear(w.x, "f16", w.gamma, w.beta, w.w_qkv, w.b_qkv, w.eps)
    assert np.all(np.abs(a["qkv"] - f["qkv"]) <= 2.0 ** -11 * absprod * (1 + 1e-9))
    assert not np.array_equal(a["qkv"], f["qkv"])
