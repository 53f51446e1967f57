"""GPU parity of the pre-LayerNorm attention block (fa_ln_stats,
fa_ln_fold_weights, fa_ln_linear, fa_linear, fa_prenorm_attention) against the
fp64 oracle (``oracle.block``), through the C ABI binding.

Bars, derived from the arithmetic (u = 2^-8 for bf16, 2^-11 for f16, the unit
roundoff of the 16-bit dtype; e = 2^-24 for fp32):
  * statistics: Welford's merges in fp32, |d mean| <= 64 e max|x| and
    |d rstd| / rstd <= 64 e (1 + |mean| rstd);
  * LayerNorm-ed dense layer: the folded weights gamma W rounded to the dtype
    (u |xhat| . |gamma W|), fp32 accumulation of the un-centred products and the
    folded sums (4 (K + 64) e rstd (|x| + |mean|) . |gamma W| (1 + |mean| rstd)
    + |beta| . |W| + |b|), one rounding of y (u |y|);
  * dense layer with residual: fp32 accumulation 2 (K + 4) e (|a| . |W| + |b| +
    |res|), one rounding u |y|;
  * the block's Q/K/V stage against the folded oracle (the same stored
    gamma W as the library's fold): the fp32 terms and the rounding of y only;
  * the block's attention stage against the plain definition: the attention
    bar (max 1e-2, mean 1e-3 on O, 1e-3 max(1, |LSE|)) plus half an ulp of the
    16-bit O, each element's bar widened by the exact effect of the library's
    one rounding that the definition lacks (gamma W stored in the dtype): the
    oracle evaluates the block in both forms and takes the difference.  The
    folded form is also checked at the plain attention bar;
  * the block output against the definition: the O bar carried through W_o
    (1e-2 |W_o| row sums, mean 1e-3), the dense-layer bar and the same
    fold effect on y.
"""
import math

import numpy as np
import pytest

import fa_inputs as gen
import oracle
from oracle import block as ob
from parity import compare, host_cores

pytestmark = pytest.mark.gpu

E32 = 2.0 ** -24


def _u(dtype):
    return 2.0 ** -8 if dtype == "bf16" else 2.0 ** -11


def _dev(bits, dtype):
    return gen.to_torch(bits, dtype).cuda()


def _f32dev(a):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()


def _host(t, dtype):
    import torch

    a = t.detach().cpu()
    if a.dtype == torch.float32:
        return a.numpy().astype(np.float64)
    return gen.bits_to_float(a.view(torch.int16).numpy().view(np.uint16), dtype).astype(np.float64)


def _check(what, got, ref, bound):
    err = np.abs(got - ref)
    ratio = float((err / bound).max()) if err.size else 0.0
    print(f"{what}: max|d|={err.max() if err.size else 0:.3e} worst err/bound={ratio:.3f}", flush=True)
    assert np.all(np.isfinite(got)), what
    assert np.all(err <= bound), (what, ratio)


def ln_linear_bound(w, x_bits, gamma, beta, wbits, bias, dtype, y_ref, absprod, rawprod):
    x = gen.bits_to_float(x_bits, dtype).astype(np.float64)
    mean, rstd = ob.layernorm_stats(x_bits, dtype, w.eps)
    W = gen.bits_to_float(wbits, dtype).astype(np.float64)
    K = x.shape[1]
    u = _u(dtype)
    bw = np.abs(beta.astype(np.float64)) @ np.abs(W).T
    babs = 0.0 if bias is None else np.abs(bias.astype(np.float64))[None, :]
    amp = (1.0 + np.abs(mean) * rstd)[:, None]
    return (1.0 + 1e-3) * u * (absprod + np.abs(y_ref)) + \
        4.0 * (K + 64) * E32 * (rawprod * amp + bw[None, :] + babs) + 1e-7


def folded_bound(w, x_bits, dtype, y_ref, rawprod):
    """The LayerNorm-ed layer against the folded oracle (the same stored
    gamma W): fp32 accumulation and the final rounding only."""
    x = gen.bits_to_float(x_bits, dtype).astype(np.float64)
    mean, rstd = ob.layernorm_stats(x_bits, dtype, w.eps)
    W = gen.bits_to_float(w.w_qkv, dtype).astype(np.float64)
    K = x.shape[1]
    bw = np.abs(w.beta.astype(np.float64)) @ np.abs(W).T + np.abs(w.b_qkv.astype(np.float64))
    amp = (1.0 + np.abs(mean) * rstd)[:, None]
    return (1.0 + 1e-3) * _u(dtype) * np.abs(y_ref) + 4.0 * (K + 64) * E32 * (rawprod * amp + bw[None, :]) + 1e-7


def check_stats(x_bits, dtype, eps, mean, rstd, what):
    m_ref, r_ref = ob.layernorm_stats(x_bits, dtype, eps)
    x = gen.bits_to_float(x_bits, dtype).astype(np.float64)
    _check(what + " mean", mean, m_ref, 64 * E32 * np.abs(x).max(axis=1) + 1e-30)
    _check(what + " rstd", rstd, r_ref, 64 * E32 * r_ref * (1.0 + np.abs(m_ref) * r_ref))


# ---------------------------------------------------------- statistics ---

@pytest.mark.parametrize("T,C,dtype,offset", [
    (37, 64, "bf16", 1.0),
    (300, 1024, "f16", 1.0),
    (5, 4104, "bf16", 3.0),      # rows of 513 chunks: lanes with 8 and 9 chunks
    (64, 1024, "f16", 200.0),    # offset 100x the spread
    (3, 8, "bf16", 1.0),         # one chunk: 63 empty lanes in the merge
])
def test_ln_stats_parity(T, C, dtype, offset):
    import flashattention_forward_03_amd as fa

    H = C // 8
    w = gen.block_inputs(1, T, H, 8, dtype, 9000 + C + T, row_offset=offset)
    mean, rstd = fa.ln_stats(_dev(w.x, dtype), w.eps)
    check_stats(w.x, dtype, w.eps, _host(mean, dtype), _host(rstd, dtype), f"stats T{T} C{C} {dtype}")


def test_ln_stats_constant_row():
    """A constant row: mean exact, var 0, rstd = 1/sqrt(eps)."""
    import flashattention_forward_03_amd as fa

    x = np.full((4, 256), gen.round_bits(np.array([3.5], np.float32), "bf16")[0], np.uint16)
    mean, rstd = fa.ln_stats(_dev(x, "bf16"), 1e-5)
    assert np.all(_host(mean, "bf16") == 3.5)
    assert np.allclose(_host(rstd, "bf16"), 1 / math.sqrt(1e-5), rtol=64 * E32)


# ----------------------------------------------------- LN dense layer ---

@pytest.mark.parametrize("T,C,N,dtype,offset", [
    (300, 256, 768, "bf16", 1.0),    # ragged token tile, 3 feature tiles
    (257, 192, 264, "f16", 1.0),     # odd k-step count (3), ragged feature tile of 8
    (1000, 1024, 3072, "bf16", 1.0), # the encoder's hidden size
    (128, 512, 512, "f16", 30.0),    # large row offsets
    (1, 64, 8, "bf16", 1.0),         # one token, one k-step, one 8-wide feature group
])
def test_ln_linear_parity(T, C, N, dtype, offset):
    import flashattention_forward_03_amd as fa

    rng = np.random.default_rng(T * 7 + C)
    w = gen.block_inputs(1, T, C // 64, 64, dtype, 9100 + T + C, row_offset=offset)
    wbits = gen.round_bits(rng.standard_normal((N, C), dtype=np.float32) / np.float32(math.sqrt(C)),
                           dtype)
    bias = (0.05 * rng.standard_normal(N)).astype(np.float32)
    x = _dev(w.x, dtype)
    folded = fa.ln_fold_weights(_f32dev(w.gamma), _f32dev(w.beta), _dev(wbits, dtype), _f32dev(bias))
    mean, rstd = fa.ln_stats(x, w.eps)
    y = fa.ln_linear(x, mean, rstd, folded)
    y_ref, absprod, rawprod = ob.ln_linear(w.x, dtype, w.gamma, w.beta, wbits, bias, w.eps)
    bound = ln_linear_bound(w, w.x, w.gamma, w.beta, wbits, bias, dtype, y_ref, absprod, rawprod)
    _check(f"ln_linear T{T} C{C} N{N} {dtype}", _host(y, dtype), y_ref, bound)


def test_ln_fold_outputs():
    """The fold's sums: colsum is the row sum of the folded weights (exact
    inputs, fp32 sum), bias_folded = bias + W beta."""
    import flashattention_forward_03_amd as fa

    rng = np.random.default_rng(77)
    N, C = 40, 4104
    wbits = gen.round_bits(rng.standard_normal((N, C), dtype=np.float32), "bf16")
    g = (1 + 0.2 * rng.standard_normal(C)).astype(np.float32)
    b = rng.standard_normal(C).astype(np.float32)
    bias = rng.standard_normal(N).astype(np.float32)
    wf, bf, cs = fa.ln_fold_weights(_f32dev(g), _f32dev(b), _dev(wbits, "bf16"), _f32dev(bias))
    W = gen.bits_to_float(wbits, "bf16").astype(np.float64)
    wf_h = _host(wf, "bf16")
    # each folded weight is gamma * w rounded once to bf16: within half an ulp
    gw = W * g.astype(np.float64)[None, :]
    assert np.all(np.abs(wf_h - gw) <= 2.0 ** -8 * np.abs(gw) * (1 + 1e-6))
    _check("colsum", _host(cs, "bf16"), wf_h.sum(axis=1), 2 * C * E32 * np.abs(wf_h).sum(axis=1))
    ref_b = bias + W @ b.astype(np.float64)
    _check("bias_folded", _host(bf, "bf16"), ref_b,
           2 * C * E32 * (np.abs(W) @ np.abs(b.astype(np.float64)) + np.abs(bias)) + 1e-7)
    # NULL bias: bias_folded = W beta
    _, bf0, _ = fa.ln_fold_weights(_f32dev(g), _f32dev(b), _dev(wbits, "bf16"), None)
    _check("bias_folded (no bias)", _host(bf0, "bf16"), W @ b.astype(np.float64),
           2 * C * E32 * (np.abs(W) @ np.abs(b.astype(np.float64))) + 1e-7)


# -------------------------------------------------------- dense layer ---

@pytest.mark.parametrize("M,K,N,dtype,with_bias,with_res", [
    (257, 64, 72, "bf16", True, True),
    (1000, 1024, 1024, "f16", True, True),
    (300, 320, 520, "bf16", False, True),
    (33, 128, 256, "f16", True, False),
    (512, 192, 264, "bf16", False, False),
])
def test_linear_parity(M, K, N, dtype, with_bias, with_res):
    import flashattention_forward_03_amd as fa

    rng = np.random.default_rng(M + K + N)
    a = gen.round_bits(rng.standard_normal((M, K), dtype=np.float32), dtype)
    wbits = gen.round_bits(rng.standard_normal((N, K), dtype=np.float32) / np.float32(math.sqrt(K)),
                           dtype)
    bias = (0.1 * rng.standard_normal(N)).astype(np.float32) if with_bias else None
    res = gen.round_bits(rng.standard_normal((M, N), dtype=np.float32), dtype) if with_res else None
    y = fa.linear(_dev(a, dtype), _dev(wbits, dtype), None if bias is None else _f32dev(bias),
                  None if res is None else _dev(res, dtype))
    y_ref, absprod = ob.linear(a, dtype, wbits, bias, res)
    extra = 0.0
    if bias is not None:
        extra = extra + np.abs(bias.astype(np.float64))[None, :]
    if res is not None:
        extra = extra + np.abs(gen.bits_to_float(res, dtype).astype(np.float64))
    bound = (1 + 1e-3) * _u(dtype) * np.abs(y_ref) + 2 * (K + 4) * E32 * (absprod + extra) + 1e-7
    _check(f"linear M{M} K{K} N{N} {dtype}", _host(y, dtype), y_ref, bound)


def test_linear_identity_weights_copy_exactly():
    """W = I, no bias: y = a bit for bit (one product per output, exact)."""
    import flashattention_forward_03_amd as fa

    rng = np.random.default_rng(3)
    a = gen.round_bits(rng.standard_normal((300, 128), dtype=np.float32), "f16")
    eye = gen.float_to_bits_exact(np.eye(128, dtype=np.float32), "f16")
    y = fa.linear(_dev(a, "f16"), _dev(eye, "f16"))
    assert np.array_equal(_host(y, "f16"), gen.bits_to_float(a, "f16").astype(np.float64))


# ---------------------------------------------------------- the block ---

def run_block(w, workspace=None):
    import torch

    import flashattention_forward_03_amd as fa

    tdt = torch.float16 if w.dtype == "f16" else torch.bfloat16
    x = _dev(w.x, w.dtype)
    folded = fa.ln_fold_weights(_f32dev(w.gamma), _f32dev(w.beta), _dev(w.w_qkv, w.dtype),
                                _f32dev(w.b_qkv))
    kl = None if w.kv_lens is None else torch.from_numpy(w.kv_lens).cuda()
    y, ws = fa.prenorm_attention(x, folded, _dev(w.w_o, w.dtype), _f32dev(w.b_o), B=w.B, N=w.N,
                                 H=w.H, H_kv=w.Hkv, eps=w.eps, scale=w.scale, causal=w.causal,
                                 kv_lens=kl, workspace=workspace)
    torch.cuda.synchronize()
    views = fa.prenorm_workspace_views(ws, w.B, w.N, w.H, w.Hkv, w.d, tdt)
    return y, views, (x, folded, kl)


def check_block(w, y, views, ref, tokens=None):
    import torch

    dt = w.dtype
    sel = slice(None) if tokens is None else tokens
    pick = (lambda t: t) if tokens is None else (lambda t: t[torch.from_numpy(tokens).cuda()])
    # stage 1: the LayerNorm-ed Q/K/V projection, against the definition (with
    # the rounding of gamma W in the bar) and against the folded layer
    xs = w.x[sel]
    qkv = _host(pick(views["qkv"]), dt)
    y_q, absprod, rawprod = ob.ln_linear(xs, dt, w.gamma, w.beta, w.w_qkv, w.b_qkv, w.eps)
    bound = ln_linear_bound(w, xs, w.gamma, w.beta, w.w_qkv, w.b_qkv, dt, y_q, absprod, rawprod)
    _check("block qkv (definition)", qkv, y_q, bound)
    wf, bf = ob.fold_weights(w.gamma, w.beta, w.w_qkv, w.b_qkv, dt)
    y_f, raw_f = ob.ln_linear_folded(xs, dt, wf, bf, w.eps)
    _check("block qkv (folded)", qkv, y_f, folded_bound(w, xs, dt, y_f, raw_f))
    # stage 2: attention, held to the plain definition.  The library's one
    # deviation from it is the 16-bit rounding of gamma W (the fold); its
    # effect on O and LSE is evaluated exactly by the oracle (the same block in
    # both forms, both in fp64 from the inputs) and widens the forward's bar
    # element by element.  The folded form is a secondary check at the
    # forward's own bar.
    o = _host(pick(views["o"]), dt)
    lse_all = _host(views["lse"], dt)
    H = w.H
    if tokens is None:
        lse = lse_all.transpose(0, 2, 1).reshape(w.T, H)
        to_rows = lambda a: a.transpose(0, 2, 1).reshape(w.T, H)
    else:
        b, n = tokens // w.N, tokens % w.N
        lse = lse_all[b, :, n]
        to_rows = lambda a: a
    p, f = ref["plain"], ref["folded"]
    lse_p, lse_f = to_rows(p["lse"]), to_rows(f["lse"])
    fold_o = np.abs(f["o"] - p["o"])
    fold_lse = np.abs(lse_f - lse_p)
    o_err = np.maximum(np.abs(o - p["o"]) - _u(dt) / 2 * np.abs(p["o"]) - fold_o, 0.0)
    fin = np.isfinite(lse_p)
    assert np.array_equal(np.isfinite(lse), fin), "block attention: -inf LSE rows differ"
    lse_err = np.maximum(np.abs(lse[fin] - lse_p[fin]) - fold_lse[fin], 0.0) / \
        np.maximum(1.0, np.abs(lse_p[fin]))
    raw = dict(max_abs=float(np.abs(o - p["o"]).max()), mean_abs=float(np.abs(o - p["o"]).mean()),
               lse_rel=float((np.abs(lse[fin] - lse_p[fin]) / np.maximum(1.0, np.abs(lse_p[fin]))).max()),
               fold_o_max=float(fold_o.max()), fold_lse_max=float(fold_lse[fin].max(initial=0.0)))
    print("block attention vs the definition", raw, flush=True)
    assert np.all(np.isfinite(o)), "block attention: non-finite O"
    assert o_err.max() <= 1e-2 and o_err.mean() <= 1e-3 and lse_err.max(initial=0.0) <= 1e-3, \
        ("block attention vs the definition", float(o_err.max()), float(o_err.mean()),
         float(lse_err.max(initial=0.0)))
    compare(o.reshape(-1, w.d), lse.reshape(-1), f["o"].reshape(-1, w.d), lse_f.reshape(-1),
            "block attention (folded form)", out_dtype=dt)
    # stage 3: output layer + residual against the definition: the O bar
    # carried through W_o, the dense-layer bar, and the fold's effect on y
    Wo = np.abs(gen.bits_to_float(w.w_o, dt).astype(np.float64))
    x = np.abs(gen.bits_to_float(xs, dt).astype(np.float64))
    u = _u(dt)
    fold_y = np.abs(f["y"] - p["y"])
    carried = 1e-2 * Wo.sum(axis=1)[None, :] + u * p["oprod"]
    bound = carried + (1 + 1e-3) * u * np.abs(p["y"]) + \
        2 * (w.C + 4) * E32 * (p["oprod"] + np.abs(w.b_o)[None, :] + x) + fold_y + 1e-7
    got = _host(pick(y), dt)
    _check("block y (definition)", got, p["y"], bound)
    mean_bar = float((1e-3 * Wo.sum(axis=1)).mean() + u * np.abs(p["y"]).mean()
                     + u * p["oprod"].mean() + fold_y.mean())
    err = float(np.abs(got - p["y"]).mean())
    print(f"block y mean|d|={err:.3e} bar={mean_bar:.3e} (fold effect {fold_y.mean():.3e})", flush=True)
    assert err <= mean_bar


def block_refs(w, tokens=None, nthreads=0):
    """The oracle's block in its plain form (the definition) and in its folded
    form (gamma W stored in the dtype)."""
    args = (w.x, w.dtype, w.gamma, w.beta, w.w_qkv, w.b_qkv, w.w_o, w.b_o, w.B, w.N, w.H, w.Hkv,
            w.d, w.eps, w.scale, w.causal, w.kv_lens)
    return {"plain": ob.prenorm_attention(*args, tokens=tokens, nthreads=nthreads, folded=False),
            "folded": ob.prenorm_attention(*args, tokens=tokens, nthreads=nthreads, folded=True)}


@pytest.mark.parametrize("B,N,H,Hkv,d,dtype,causal,lens", [
    (2, 300, 4, 4, 64, "bf16", False, None),
    (2, 257, 4, 2, 64, "f16", True, None),        # grouped K/V heads, causal
    (3, 200, 2, 1, 128, "bf16", False, (1, 200)), # multi-query, key padding, d = 128
    (1, 129, 8, 8, 32, "f16", True, None),        # d = 32
])
def test_block_parity(B, N, H, Hkv, d, dtype, causal, lens):
    w = gen.block_inputs(B, N, H, d, dtype, 9300 + B * 100 + H * 10 + Hkv, Hkv=Hkv, causal=causal,
                         kv_len_range=lens)
    y, views, _ = run_block(w)
    check_block(w, y, views, block_refs(w))


def test_block_equals_its_stages_bitwise():
    """The block is exactly ln_stats -> ln_linear -> the strided forward with a
    16-bit O -> linear with the residual."""
    import torch

    import flashattention_forward_03_amd as fa

    w = gen.block_inputs(2, 150, 4, 64, "bf16", 9400, Hkv=2, causal=True)
    y, views, (x, folded, _) = run_block(w)
    mean, rstd = fa.ln_stats(x, w.eps)
    qkv = fa.ln_linear(x, mean, rstd, folded)
    H, Hkv, d, N, B = w.H, w.Hkv, w.d, w.N, w.B
    heads = qkv.view(B, N, H + 2 * Hkv, d)
    q = heads[:, :, :H].transpose(1, 2)
    k = heads[:, :, H:H + Hkv].transpose(1, 2)
    v = heads[:, :, H + Hkv:].transpose(1, 2)
    o = torch.empty((B, N, H, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    fa.forward(q, k, v, scale=w.scale, causal=True, out=(o.transpose(1, 2), lse))
    y2 = fa.linear(o.view(B * N, H * d), _dev(w.w_o, "bf16"), _f32dev(w.b_o), x)
    torch.cuda.synchronize()
    assert torch.equal(qkv, views["qkv"]) and torch.equal(o.view(B * N, -1), views["o"])
    assert torch.equal(lse, views["lse"]) and torch.equal(y, y2)


def test_block_full_size_sampled():
    """The encoder block at B8 N4096, 16 heads of 64 (hidden 1024): the oracle's
    Q/K/V projection of every token, attention and output layer on 512
    sampled tokens (all heads of each)."""
    name = "prenorm_block_b8_n4096_h16_d64_bf16"
    w = gen.block_workload(name)
    y, views, _ = run_block(w)
    rng = np.random.default_rng(w.seed)
    tokens = np.sort(rng.choice(w.T, size=512, replace=False))
    tokens = np.concatenate([[0, w.N - 1, w.T - 1], tokens])
    check_block(w, y, views, block_refs(w, tokens=tokens, nthreads=host_cores()), tokens=tokens)
