"""Pins for the fp64 oracle: each check is fixed by the mathematics, a library
routine, a brute force or a closed form, never by the oracle itself.

Runs on the CPU only.
"""
import math

import numpy as np
import pytest

import fa_inputs as gen
import oracle
from oracle import brute


def _draw(rng, shape, dtype, scale=1.0):
    return gen.round_bits(rng.standard_normal(shape).astype(np.float32) * scale, dtype)


def _f(bits, dtype):
    return gen.bits_to_float(bits, dtype).astype(np.float64)


# ------------------------------------------------------------ decoding ----

def test_widen_f16_every_pattern_matches_numpy():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    mine = oracle.widen(bits, "f16")
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], ref[~nan])
    assert np.array_equal(np.signbit(mine[~nan]), np.signbit(ref[~nan]))


def test_widen_bf16_every_pattern_matches_torch():
    import torch

    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    mine = oracle.widen(bits, "bf16")
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], ref[~nan])


# --------------------------------------------------------- brute force ----

def _brute_case(rng, B, H, Nq, Nk, d, dtype, causal, kv_lens, scale):
    q = _draw(rng, (B, H, Nq, d), dtype)
    k = _draw(rng, (B, H, Nk, d), dtype)
    v = _draw(rng, (B, H, Nk, d), dtype)
    o, lse = oracle.attention_fwd(q, k, v, dtype, scale, causal, kv_lens)
    qf, kf, vf = _f(q, dtype), _f(k, dtype), _f(v, dtype)
    for b in range(B):
        for h in range(H):
            bo, bl = brute.attention(qf[b, h].tolist(), kf[b, h].tolist(), vf[b, h].tolist(),
                                     scale, causal,
                                     None if kv_lens is None else int(kv_lens[b]))
            bo, bl = np.array(bo), np.array(bl)
            fin = np.isfinite(bl)
            assert np.array_equal(fin, np.isfinite(lse[b, h]))
            assert np.all(lse[b, h][~fin] == -np.inf)
            assert np.max(np.abs(lse[b, h][fin] - bl[fin]), initial=0) <= 1e-12
            assert np.max(np.abs(o[b, h] - bo), initial=0) <= 1e-12


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_oracle_matches_brute_force(seed, dtype, causal):
    rng = np.random.default_rng(seed + 100 * causal)
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 3))
    Nq, Nk, d = int(rng.integers(1, 9)), int(rng.integers(1, 9)), int(rng.integers(1, 9))
    kv_lens = None
    if seed % 2:
        kv_lens = rng.integers(0, Nk + 2, size=B).astype(np.int32)   # includes 0 and > Nk
    _brute_case(rng, B, H, Nq, Nk, d, dtype, causal, kv_lens, 1.0 / math.sqrt(d))


def test_oracle_matches_brute_force_square_causal_padded():
    rng = np.random.default_rng(7)
    _brute_case(rng, 2, 2, 8, 8, 8, "bf16", True, np.array([8, 3], np.int32), 0.35)


# --------------------------------------------------------- closed forms ---

@pytest.mark.parametrize("causal", [False, True])
def test_constant_v_gives_that_constant(causal):
    rng = np.random.default_rng(1)
    q = _draw(rng, (2, 2, 16, 8), "bf16")
    k = _draw(rng, (2, 2, 16, 8), "bf16")
    for c in [2.0, -0.5, 0.7109375]:
        v = gen.float_to_bits_exact(np.full((2, 2, 16, 8), c, np.float32), "bf16")
        o, _ = oracle.attention_fwd(q, k, v, "bf16", 0.3, causal, np.array([16, 9], np.int32))
        # the probabilities sum to one up to a few fp64 roundings
        assert np.max(np.abs(o - c)) <= 16 * 2.0 ** -52 * abs(c)


def _zero_q_case(Nq, Nk, causal, kv_lens, B=2):
    rng = np.random.default_rng(3)
    d = 4
    q = np.zeros((B, 1, Nq, d), np.uint16)
    k = _draw(rng, (B, 1, Nk, d), "f16")
    v = _draw(rng, (B, 1, Nk, d), "f16")
    o, lse = oracle.attention_fwd(q, k, v, "f16", 0.5, causal, kv_lens)
    vf = _f(v, "f16")
    for b in range(B):
        n_b = Nk if kv_lens is None else min(int(kv_lens[b]), Nk)
        for i in range(Nq):
            n = n_b
            if causal:
                n = min(n, max(0, i + Nk - Nq + 1))
            if n == 0:
                assert lse[b, 0, i] == -np.inf and np.all(o[b, 0, i] == 0)
                continue
            assert abs(lse[b, 0, i] - math.log(n)) <= 1e-14
            np.testing.assert_allclose(o[b, 0, i], vf[b, 0, :n].mean(axis=0), rtol=0,
                                       atol=1e-14)


def test_zero_q_uniform_attention_noncausal():
    _zero_q_case(5, 7, False, None)


def test_zero_q_uniform_attention_causal_square():
    _zero_q_case(9, 9, True, None)


def test_zero_q_uniform_attention_causal_bottom_right():
    _zero_q_case(4, 10, True, None)      # Nq < Nk: row i sees keys j <= i + 6
    _zero_q_case(10, 4, True, None)      # Nq > Nk: first rows see nothing


def test_zero_q_uniform_attention_padding():
    _zero_q_case(6, 12, False, np.array([12, 5], np.int32))
    _zero_q_case(12, 12, True, np.array([7, 0], np.int32))


def test_causal_row0_is_v0():
    rng = np.random.default_rng(5)
    q = _draw(rng, (1, 3, 32, 16), "bf16")
    k = _draw(rng, (1, 3, 32, 16), "bf16")
    v = _draw(rng, (1, 3, 32, 16), "bf16")
    o, lse = oracle.attention_fwd(q, k, v, "bf16", 0.25, True)
    qf, kf, vf = _f(q, "bf16"), _f(k, "bf16"), _f(v, "bf16")
    assert np.array_equal(o[0, :, 0], vf[0, :, 0])
    s00 = 0.25 * np.einsum("ht,ht->h", qf[0, :, 0], kf[0, :, 0])
    np.testing.assert_allclose(lse[0, :, 0], s00, rtol=0, atol=1e-14)


def test_single_query_causal_equals_noncausal():
    rng = np.random.default_rng(6)
    q = _draw(rng, (2, 2, 1, 16), "f16")
    k = _draw(rng, (2, 2, 40, 16), "f16")
    v = _draw(rng, (2, 2, 40, 16), "f16")
    a = oracle.attention_fwd(q, k, v, "f16", 0.25, True)
    b = oracle.attention_fwd(q, k, v, "f16", 0.25, False)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_two_key_worked_case():
    # d=1, scale=1, q=1, k=(0,1): P=(1/(1+e), e/(1+e)), LSE=ln(1+e)
    q = gen.float_to_bits_exact(np.ones((1, 1, 1, 1), np.float32), "f16")
    k = gen.float_to_bits_exact(np.array([0.0, 1.0], np.float32).reshape(1, 1, 2, 1), "f16")
    v0, v1 = 3.0, -5.0
    v = gen.float_to_bits_exact(np.array([v0, v1], np.float32).reshape(1, 1, 2, 1), "f16")
    o, lse = oracle.attention_fwd(q, k, v, "f16", 1.0, False)
    e = math.e
    assert abs(o[0, 0, 0, 0] - (v0 + e * v1) / (1 + e)) <= 1e-15
    assert abs(lse[0, 0, 0] - math.log(1 + e)) <= 1e-15


def test_shift_of_keys_shifts_lse_only():
    """Adding u to every key adds scale*q_i.u to every score of row i: O is
    unchanged and LSE moves by exactly that amount.  u is chosen so that the
    shifted scores reach ~+100 (exp overflows float32 there without a max shift)."""
    rng = np.random.default_rng(8)
    B, H, N, d = 1, 2, 24, 8
    # values on a 1/16 grid, |x| <= 4, so K+u stays exact in f16
    grid = lambda shape: np.round(rng.uniform(-4, 4, shape) * 16) / 16
    qf = grid((B, H, N, d)).astype(np.float32)
    kf = grid((B, H, N, d)).astype(np.float32)
    vf = grid((B, H, N, d)).astype(np.float32)
    u = np.full(d, 50.0, np.float32)
    q = gen.float_to_bits_exact(qf, "f16")
    k = gen.float_to_bits_exact(kf, "f16")
    k2 = gen.float_to_bits_exact(kf + u, "f16")
    v = gen.float_to_bits_exact(vf, "f16")
    scale = 0.5
    for causal in (False, True):
        o1, l1 = oracle.attention_fwd(q, k, v, "f16", scale, causal)
        o2, l2 = oracle.attention_fwd(q, k2, v, "f16", scale, causal)
        shift = scale * (qf.astype(np.float64) @ u.astype(np.float64))
        np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12)
        np.testing.assert_allclose(l2, l1 + shift, rtol=1e-14, atol=1e-12)
        assert np.max(l2) > 100


def test_needle_key_selects_its_value():
    rng = np.random.default_rng(9)
    B, H, N, d = 1, 1, 64, 16
    qf = gen.bits_to_float(_draw(rng, (B, H, N, d), "bf16"), "bf16")
    kf = gen.bits_to_float(_draw(rng, (B, H, N, d), "bf16"), "bf16") * 0.01
    i, jstar = 40, 17
    kf[0, 0, jstar] = qf[0, 0, i] * 64.0            # exact in bf16 (power-of-two scale)
    q = gen.float_to_bits_exact(qf, "bf16")
    k = gen.round_bits(kf, "bf16")
    v = _draw(rng, (B, H, N, d), "bf16")
    o, _ = oracle.attention_fwd(q, k, v, "bf16", 1.0, True)
    np.testing.assert_allclose(o[0, 0, i], _f(v, "bf16")[0, 0, jstar], atol=1e-9)


def test_affine_in_v():
    rng = np.random.default_rng(10)
    B, H, N, d = 2, 2, 20, 8
    q = _draw(rng, (B, H, N, d), "f16")
    k = _draw(rng, (B, H, N, d), "f16")
    grid = lambda: (np.round(rng.uniform(-8, 8, (B, H, N, d)) * 8) / 8).astype(np.float32)
    v1f, v2f = grid(), grid()
    v1 = gen.float_to_bits_exact(v1f, "f16")
    v2 = gen.float_to_bits_exact(v2f, "f16")
    vc = gen.float_to_bits_exact(2 * v1f - 3 * v2f + 1.0, "f16")
    kl = np.array([20, 11], np.int32)
    o1, l1 = oracle.attention_fwd(q, k, v1, "f16", 0.4, True, kl)
    o2, _ = oracle.attention_fwd(q, k, v2, "f16", 0.4, True, kl)
    oc, lc = oracle.attention_fwd(q, k, vc, "f16", 0.4, True, kl)
    np.testing.assert_allclose(oc, 2 * o1 - 3 * o2 + 1.0, rtol=0, atol=1e-12)
    assert np.array_equal(lc, l1)


def test_split_keys_combine_by_lse_rule():
    """Attention over all keys equals the LSE-weighted merge of attention over
    two disjoint key blocks (the recurrence that online softmax and split-KV
    decode both rest on)."""
    rng = np.random.default_rng(11)
    B, H, Nq, Nk, d = 1, 2, 5, 30, 16
    q = _draw(rng, (B, H, Nq, d), "bf16")
    k = _draw(rng, (B, H, Nk, d), "bf16")
    v = _draw(rng, (B, H, Nk, d), "bf16")
    cut = 13
    of, lf = oracle.attention_fwd(q, k, v, "bf16", 0.25, False)
    o1, l1 = oracle.attention_fwd(q, k[:, :, :cut], v[:, :, :cut], "bf16", 0.25, False)
    o2, l2 = oracle.attention_fwd(q, k[:, :, cut:], v[:, :, cut:], "bf16", 0.25, False)
    m = np.maximum(l1, l2)
    w1, w2 = np.exp(l1 - m), np.exp(l2 - m)
    om = (w1[..., None] * o1 + w2[..., None] * o2) / (w1 + w2)[..., None]
    lm = m + np.log(w1 + w2)
    np.testing.assert_allclose(om, of, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lm, lf, rtol=0, atol=1e-12)


def test_identity_v_gives_scipy_softmax_rows():
    """With V = identity (d = Nk) each output row is the softmax of the scaled
    score row itself; compare with scipy's softmax and logsumexp."""
    from scipy.special import logsumexp, softmax

    rng = np.random.default_rng(12)
    N = 16
    q = _draw(rng, (1, 1, N, N), "f16")
    k = _draw(rng, (1, 1, N, N), "f16")
    v = gen.float_to_bits_exact(np.eye(N, dtype=np.float32).reshape(1, 1, N, N), "f16")
    scale = 0.3
    o, lse = oracle.attention_fwd(q, k, v, "f16", scale, False)
    s = scale * (_f(q, "f16")[0, 0] @ _f(k, "f16")[0, 0].T)
    np.testing.assert_allclose(o[0, 0], softmax(s, axis=1), rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse[0, 0], logsumexp(s, axis=1), rtol=0, atol=1e-13)
    np.testing.assert_allclose(o[0, 0].sum(axis=1), 1.0, rtol=0, atol=1e-14)


def test_row_subset_matches_full_rows():
    w = gen.fwd_inputs(2, 3, 40, 40, 16, "bf16", 77, causal=True, scale=0.125,
                       kv_len_range=(10, 40))
    o, lse = oracle.attention_fwd(w.q, w.k, w.v, "bf16", w.scale, True, w.kv_lens)
    rows = np.array([239, 0, 5, 119, 120, 77], np.int64)
    os_, ls_ = oracle.attention_fwd(w.q, w.k, w.v, "bf16", w.scale, True, w.kv_lens, rows=rows)
    assert np.array_equal(os_, o.reshape(-1, 16)[rows])
    assert np.array_equal(ls_, lse.reshape(-1)[rows])


def test_thread_count_does_not_change_bits():
    w = gen.fwd_inputs(2, 3, 33, 47, 16, "f16", 78, causal=True, scale=0.2)
    a = oracle.attention_fwd(w.q, w.k, w.v, "f16", w.scale, True, nthreads=1)
    b = oracle.attention_fwd(w.q, w.k, w.v, "f16", w.scale, True, nthreads=5)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ---------------------------------------------------------------- decode ---

def _tiny_decode(identity=False, seed=21):
    return gen.decode_inputs(3, 2, 8, (1, 37), "bf16", seed, page_size=4, num_pages=64,
                             identity_pages=identity)


def test_decode_matches_brute_force():
    inp = _tiny_decode()
    o, lse = oracle.decode(inp.q, inp.k, inp.v, inp.seq_off, "bf16", inp.scale)
    qf, kf, vf = _f(inp.q, "bf16"), _f(inp.k, "bf16"), _f(inp.v, "bf16")
    for s in range(inp.S):
        a, b = inp.seq_off[s], inp.seq_off[s + 1]
        for h in range(inp.H):
            bo, bl = brute.attention([qf[s, h].tolist()], kf[a:b, h].tolist(),
                                     vf[a:b, h].tolist(), inp.scale)
            assert abs(bl[0] - lse[s, h]) <= 1e-12
            assert np.max(np.abs(np.array(bo[0]) - o[s, h])) <= 1e-12


def test_decode_zero_query_is_mean_of_cache():
    inp = _tiny_decode(seed=22)
    qz = np.zeros_like(inp.q)
    o, lse = oracle.decode(qz, inp.k, inp.v, inp.seq_off, "bf16", inp.scale)
    vf = _f(inp.v, "bf16")
    for s in range(inp.S):
        a, b = inp.seq_off[s], inp.seq_off[s + 1]
        np.testing.assert_allclose(o[s], vf[a:b].mean(axis=0), atol=1e-14, rtol=0)
        np.testing.assert_allclose(lse[s], math.log(b - a), atol=1e-14, rtol=0)


def test_page_pool_round_trip():
    inp = _tiny_decode(seed=23)
    nan_bf16 = 0x7FC0
    for which, src in (("k", inp.k), ("v", inp.v)):
        pool = gen.build_pool_host(inp, which, fill_bits=nan_bf16)
        assert np.array_equal(gen.gather_logical(pool, inp), src)
        used = np.zeros(pool.shape[0] * pool.shape[2], bool)
        phys, row = gen.page_slots(inp)
        used[phys * inp.page_size + row] = True
        slots = pool.transpose(0, 2, 1, 3).reshape(-1, inp.H, inp.d)
        assert np.all(slots[~used] == nan_bf16)
    # each logical page maps to a distinct physical page
    t = inp.page_table[inp.page_table >= 0]
    assert len(np.unique(t)) == len(t)


def test_decode_on_gathered_pool_equals_logical():
    inp = _tiny_decode(seed=24)
    kp = gen.build_pool_host(inp, "k")
    vp = gen.build_pool_host(inp, "v")
    a = oracle.decode(inp.q, inp.k, inp.v, inp.seq_off, "bf16", inp.scale)
    b = oracle.decode(inp.q, gen.gather_logical(kp, inp), gen.gather_logical(vp, inp),
                      inp.seq_off, "bf16", inp.scale)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_decode_equals_forward_with_one_query():
    inp = _tiny_decode(seed=25)
    o, lse = oracle.decode(inp.q, inp.k, inp.v, inp.seq_off, "bf16", inp.scale)
    for s in range(inp.S):
        a, b = inp.seq_off[s], inp.seq_off[s + 1]
        kk = np.ascontiguousarray(inp.k[a:b].transpose(1, 0, 2))[None]
        vv = np.ascontiguousarray(inp.v[a:b].transpose(1, 0, 2))[None]
        fo, fl = oracle.attention_fwd(inp.q[s][None, :, None, :], kk, vv, "bf16", inp.scale,
                                      True)
        np.testing.assert_allclose(fo[0, :, 0], o[s], atol=1e-15, rtol=0)
        np.testing.assert_allclose(fl[0, :, 0], lse[s], atol=1e-15, rtol=0)


# ------------------------------------------------- grouped-query heads ---
# MQA / GQA (llm-kernel-lib page, "Ablation Study"): K/V carry Hkv heads and
# query head h reads K/V head h // (H // Hkv).

@pytest.mark.parametrize("H,Hkv", [(4, 2), (6, 3), (4, 1), (8, 2)])
@pytest.mark.parametrize("causal", [False, True])
def test_gqa_forward_matches_brute_force_with_head_map(H, Hkv, causal):
    rng = np.random.default_rng(40 + H + 10 * Hkv + causal)
    B, Nq, Nk, d = 2, 5, 7, 4
    q = _draw(rng, (B, H, Nq, d), "bf16")
    k = _draw(rng, (B, Hkv, Nk, d), "bf16")
    v = _draw(rng, (B, Hkv, Nk, d), "bf16")
    kv_lens = np.array([7, 4], np.int32)
    o, lse = oracle.attention_fwd(q, k, v, "bf16", 0.5, causal, kv_lens)
    qf, kf, vf = _f(q, "bf16"), _f(k, "bf16"), _f(v, "bf16")
    g = H // Hkv
    for b in range(B):
        for h in range(H):
            bo, bl = brute.attention(qf[b, h].tolist(), kf[b, h // g].tolist(),
                                     vf[b, h // g].tolist(), 0.5, causal, int(kv_lens[b]))
            assert np.max(np.abs(np.array(bl) - lse[b, h])) <= 1e-12
            assert np.max(np.abs(np.array(bo) - o[b, h])) <= 1e-12


@pytest.mark.parametrize("Hkv", [1, 2, 4])
def test_gqa_forward_equals_mha_on_repeated_heads(Hkv):
    inp = gen.fwd_inputs(2, 8, 33, 40, 16, "f16", 50 + Hkv, causal=True, Hkv=Hkv,
                         kv_len_range=(20, 40))
    g = 8 // Hkv
    a = oracle.attention_fwd(inp.q, inp.k, inp.v, "f16", inp.scale, True, inp.kv_lens)
    b = oracle.attention_fwd(inp.q, np.repeat(inp.k, g, axis=1), np.repeat(inp.v, g, axis=1),
                             "f16", inp.scale, True, inp.kv_lens)
    # the same per-head arithmetic on the same K/V rows: identical bits
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_mqa_equal_query_heads_give_equal_outputs():
    rng = np.random.default_rng(60)
    q1 = _draw(rng, (1, 1, 9, 8), "bf16")
    q = np.repeat(q1, 4, axis=1)
    k = _draw(rng, (1, 1, 11, 8), "bf16")
    v = _draw(rng, (1, 1, 11, 8), "bf16")
    o, lse = oracle.attention_fwd(q, k, v, "bf16", 0.4, False)
    for h in range(1, 4):
        assert np.array_equal(o[0, h], o[0, 0]) and np.array_equal(lse[0, h], lse[0, 0])


def test_gqa_decode_matches_brute_force_with_head_map():
    inp = gen.decode_inputs(3, 6, 8, (1, 37), "bf16", 61, page_size=4, num_pages=64, Hkv=2)
    o, lse = oracle.decode(inp.q, inp.k, inp.v, inp.seq_off, "bf16", inp.scale)
    qf, kf, vf = _f(inp.q, "bf16"), _f(inp.k, "bf16"), _f(inp.v, "bf16")
    for s in range(inp.S):
        a, b = inp.seq_off[s], inp.seq_off[s + 1]
        for h in range(inp.H):
            bo, bl = brute.attention([qf[s, h].tolist()], kf[a:b, h // 3].tolist(),
                                     vf[a:b, h // 3].tolist(), inp.scale)
            assert abs(bl[0] - lse[s, h]) <= 1e-12
            assert np.max(np.abs(np.array(bo[0]) - o[s, h])) <= 1e-12


@pytest.mark.parametrize("Hkv", [1, 2, 4])
def test_gqa_decode_equals_mha_on_repeated_heads(Hkv):
    inp = gen.decode_inputs(4, 8, 16, (1, 70), "f16", 62 + Hkv, page_size=8, num_pages=64,
                            Hkv=Hkv)
    g = 8 // Hkv
    a = oracle.decode(inp.q, inp.k, inp.v, inp.seq_off, "f16", inp.scale)
    b = oracle.decode(inp.q, np.repeat(inp.k, g, axis=1), np.repeat(inp.v, g, axis=1),
                      inp.seq_off, "f16", inp.scale)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_gqa_pool_round_trip():
    inp = gen.decode_inputs(3, 8, 8, (1, 37), "bf16", 63, page_size=4, num_pages=64, Hkv=2)
    for which, src in (("k", inp.k), ("v", inp.v)):
        pool = gen.build_pool_host(inp, which)
        assert pool.shape == (64, 2, 4, 8)
        assert np.array_equal(gen.gather_logical(pool, inp), src)


def test_gqa_rejects_head_counts_that_do_not_divide():
    with pytest.raises(ValueError):
        gen.fwd_inputs(1, 6, 4, 4, 8, "bf16", 0, causal=False, Hkv=4)
    with pytest.raises(ValueError):
        gen.decode_inputs(1, 6, 8, (1, 4), "bf16", 0, Hkv=4)


# ------------------------------------------------------------- backward ---
# Gradients of the attention for an output gradient dO (gpu-inference page,
# section 02: row term D, dK/dV, dQ).  Pinned by central differences of an
# independent numpy forward, and by closed forms and invariants.

def _np_forward(q, k, v, scale, causal, kv_len=None):
    """Plain numpy attention on float64 [N, d] arrays (definition only)."""
    Nq, Nk = q.shape[0], k.shape[0]
    s = scale * (q @ k.T)
    n = Nk if kv_len is None else kv_len
    mask = np.broadcast_to(np.arange(Nk)[None, :] < n, (Nq, Nk))
    if causal:
        mask = mask & (np.arange(Nk)[None, :] <= np.arange(Nq)[:, None] + Nk - Nq)
    s = np.where(mask, s, -np.inf)
    out = np.zeros((Nq, v.shape[1]))
    for i in range(Nq):
        if not mask[i].any():
            continue
        e = np.exp(s[i] - s[i][mask[i]].max())
        out[i] = (e / e.sum()) @ v
    return out


@pytest.mark.parametrize("causal,kv_len,Nq,Nk", [(False, None, 5, 6), (True, None, 6, 6),
                                                 (True, 4, 4, 7), (True, None, 7, 4),
                                                 (False, 3, 5, 6)])
def test_backward_matches_finite_differences(causal, kv_len, Nq, Nk):
    rng = np.random.default_rng(70 + Nq + 10 * Nk + causal)
    d, scale = 4, 0.7
    q = _draw(rng, (1, 1, Nq, d), "bf16")
    k = _draw(rng, (1, 1, Nk, d), "bf16")
    v = _draw(rng, (1, 1, Nk, d), "bf16")
    g = _draw(rng, (1, 1, Nq, d), "bf16")
    kl = None if kv_len is None else np.array([kv_len], np.int32)
    dq, dk, dv, delta = oracle.attention_bwd(q, k, v, g, "bf16", scale, causal, kl)
    qf, kf, vf, gf = (_f(x, "bf16")[0, 0] for x in (q, k, v, g))

    def loss(qx, kx, vx):
        return float(np.sum(gf * _np_forward(qx, kx, vx, scale, causal, kv_len)))

    h = 1e-6
    for name, x, grad in (("q", qf, dq[0, 0]), ("k", kf, dk[0, 0]), ("v", vf, dv[0, 0])):
        fd = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"q": (xp, kf, vf), "k": (qf, xp, vf), "v": (qf, kf, xp)}[name]
            args_m = {"q": (xm, kf, vf), "k": (qf, xm, vf), "v": (qf, kf, xm)}[name]
            fd[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        assert np.max(np.abs(fd - grad)) <= 1e-7, name
    # the row term is dO . O
    o = _np_forward(qf, kf, vf, scale, causal, kv_len)
    np.testing.assert_allclose(delta[0, 0], np.sum(gf * o, axis=1), atol=1e-13, rtol=0)


def test_backward_constant_v_gives_zero_q_and_k_gradients():
    rng = np.random.default_rng(80)
    q = _draw(rng, (1, 2, 9, 8), "bf16")
    k = _draw(rng, (1, 2, 11, 8), "bf16")
    row = _draw(rng, (1, 2, 1, 8), "bf16")
    v = np.repeat(row, 11, axis=2)
    g = _draw(rng, (1, 2, 9, 8), "bf16")
    dq, dk, dv, delta = oracle.attention_bwd(q, k, v, g, "bf16", 0.5, True)
    # O_i = v for every row, so dP_ij = dO_i . v = D_i and dS = 0
    assert np.max(np.abs(dq)) <= 1e-13 and np.max(np.abs(dk)) <= 1e-13
    np.testing.assert_allclose(delta[0], np.einsum("hid,hd->hi", _f(g, "bf16")[0],
                                                   _f(row, "bf16")[0, :, 0]), atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_invariants(causal):
    """Rows of P sum to one: sum_j dV_j = sum_i dO_i over rows that see a key;
    rows of dS sum to zero: sum_j dK_j = 0."""
    w = gen.fwd_inputs(2, 3, 13, 17, 8, "f16", 81 + causal, causal=causal, kv_len_range=(1, 17))
    g = gen.fwd_inputs(2, 3, 13, 17, 8, "f16", 91, causal=causal).q
    dq, dk, dv, _ = oracle.attention_bwd(w.q, w.k, w.v, g, "f16", w.scale, causal, w.kv_lens)
    gf = _f(g, "f16")
    for b in range(2):
        n = int(w.kv_lens[b])
        seen = np.array([min(n, i + 17 - 13 + 1) if causal else n for i in range(13)]) > 0
        np.testing.assert_allclose(dv[b].sum(axis=1), gf[b][:, seen].sum(axis=1), atol=1e-12)
        np.testing.assert_allclose(dk[b].sum(axis=1), 0.0, atol=1e-12)
        assert np.all(dq[b][:, ~seen] == 0)


def test_backward_gqa_sums_the_group_of_mha_gradients():
    w = gen.fwd_inputs(2, 6, 10, 12, 8, "bf16", 95, causal=True, Hkv=2)
    g = gen.fwd_inputs(2, 6, 10, 12, 8, "bf16", 96, causal=True).q
    dq, dk, dv, delta = oracle.attention_bwd(w.q, w.k, w.v, g, "bf16", w.scale, True)
    kr, vr = np.repeat(w.k, 3, axis=1), np.repeat(w.v, 3, axis=1)
    dq2, dk2, dv2, delta2 = oracle.attention_bwd(w.q, kr, vr, g, "bf16", w.scale, True)
    np.testing.assert_allclose(dq, dq2, atol=1e-14, rtol=0)
    np.testing.assert_allclose(delta, delta2, atol=1e-14, rtol=0)
    np.testing.assert_allclose(dk, dk2.reshape(2, 2, 3, 12, 8).sum(axis=2), atol=1e-12, rtol=0)
    np.testing.assert_allclose(dv, dv2.reshape(2, 2, 3, 12, 8).sum(axis=2), atol=1e-12, rtol=0)


def test_backward_group_subset_equals_full():
    w = gen.fwd_inputs(2, 4, 9, 9, 8, "bf16", 97, causal=False, Hkv=2)
    g = gen.fwd_inputs(2, 4, 9, 9, 8, "bf16", 98, causal=False).q
    full = oracle.attention_bwd(w.q, w.k, w.v, g, "bf16", w.scale, False)
    part = oracle.attention_bwd(w.q, w.k, w.v, g, "bf16", w.scale, False, groups=[3, 0])
    # groups 0 = (b0, kv head 0) -> query heads 0, 1; 3 = (b1, kv head 1) -> 2, 3
    assert np.array_equal(part[0][0, :2], full[0][0, :2]) and np.isnan(part[0][0, 2:]).all()
    assert np.array_equal(part[0][1, 2:], full[0][1, 2:])
    assert np.array_equal(part[1][0, 0], full[1][0, 0]) and np.array_equal(part[2][1, 1], full[2][1, 1])
    assert np.isnan(part[1][0, 1]).all()


# ------------------------------------------------------- paged cache append ---

def test_kv_append_then_gather_is_the_logical_cache():
    """Prefill in chunks, then one decode token per sequence: reading every
    sequence back through its page table gives its tokens in order."""
    from oracle import cache

    inp = gen.decode_inputs(3, 4, 8, (1, 45), "bf16", 130, page_size=16, num_pages=32, Hkv=2)
    kp = np.zeros((32, 2, 16, 8), np.uint16)
    vp = np.zeros_like(kp)
    # prefill each sequence in two chunks, interleaved across sequences
    chunks = []
    for s in range(inp.S):
        a, b = int(inp.seq_off[s]), int(inp.seq_off[s + 1])
        mid = a + (b - a) // 2
        chunks += [(s, a, mid), (s, mid, b)]
    for s, a, b in sorted(chunks, key=lambda c: c[1] - c[0]):
        base = int(inp.seq_off[s])
        n = cache.kv_append(kp, vp, inp.page_table, np.full(b - a, s), np.arange(a, b) - base,
                            inp.k[a:b], inp.v[a:b])
        assert n == b - a
    assert np.array_equal(gen.gather_logical(kp, inp), inp.k)
    assert np.array_equal(gen.gather_logical(vp, inp), inp.v)


def test_kv_append_skips_out_of_range_tokens():
    from oracle import cache

    kp = np.zeros((4, 1, 16, 8), np.uint16)
    vp = np.zeros_like(kp)
    table = np.array([[2, -1], [7, 1]], np.int32)   # page 7 does not exist
    new = np.arange(5 * 8, dtype=np.uint16).reshape(5, 1, 8) + 1
    n = cache.kv_append(kp, vp, table, np.array([0, 0, 1, 2, 1]), np.array([3, 16, 0, 0, 20]),
                        new, new)
    assert n == 2                       # (0, 3) -> page 2; (1, 20) -> page 1 row 4
    assert np.array_equal(kp[2, 0, 3], new[0, 0]) and np.array_equal(kp[1, 0, 4], new[4, 0])
    assert int(np.count_nonzero(kp)) == 16
