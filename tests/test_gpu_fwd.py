"""GPU parity of fa_fwd against the fp64 oracle (through the C ABI binding)."""
import math

import numpy as np
import pytest

import fa_inputs as gen
import oracle
from parity import compare, device_tensors, gpu_forward, host_cores

pytestmark = [pytest.mark.gpu, pytest.mark.usefixtures("fwd_kernel")]


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import flashattention_forward_03_amd as fa

    fa.load_library()


def full_parity(w, what):
    o, lse = gpu_forward(w)
    o_ref, lse_ref = oracle.attention_fwd(w.q, w.k, w.v, w.dtype, w.scale, w.causal, w.kv_lens)
    stats = compare(o, lse, o_ref, lse_ref, what)
    print(what, stats, flush=True)
    return stats


# ----------------------------------------------------- the named workloads

@pytest.mark.parametrize("name", [
    "fwd_b1h1_n256_d64_f16",
    "fwd_b1h1_n2048_d64_f16",
    "fwd_causal_b8h16_n512_d64_bf16",
    "fwd_causal_b8h16_n1024_d64_bf16",
])
def test_workload_full_parity(name):
    full_parity(gen.fwd_workload(name), name)


@pytest.mark.parametrize("name", [
    "fwd_causal_b8h16_n2048_d64_bf16",
    "fwd_causal_b8h16_n4096_d64_bf16",
    "fwd_padded_b8h16_n2048_d64_bf16",
])
def test_workload_full_size_parity(name):
    """The full-size launches the benchmark times, every output element against
    the oracle (run on all host cores), at the max / mean / LSE bar."""
    w = gen.fwd_workload(name)
    o, lse = gpu_forward(w)
    o_ref, lse_ref = oracle.attention_fwd(w.q, w.k, w.v, w.dtype, w.scale, w.causal, w.kv_lens,
                                          nthreads=host_cores())
    stats = compare(o, lse, o_ref, lse_ref, name)
    print(name, "all", lse.size, "rows", stats, flush=True)


def test_head_groups_of_a_long_launch():
    """A causal launch of 8192 workgroups (B256 H16 N256: 4096 heads, 2 query
    tiles each) takes each XCD's heads in four groups; every element against the
    oracle, with padding so that the groups see different key counts."""
    w = gen.fwd_inputs(256, 16, 256, 256, 64, "bf16", seed=9300, causal=True, kv_len_range=(1, 256))
    o, lse = gpu_forward(w)
    o_ref, lse_ref = oracle.attention_fwd(w.q, w.k, w.v, w.dtype, w.scale, w.causal, w.kv_lens,
                                          nthreads=host_cores())
    print("head groups B256 H16 N256", compare(o, lse, o_ref, lse_ref, "head groups"), flush=True)


def test_eight_head_groups_of_a_long_launch():
    """A causal launch of 16384 workgroups (B512 H16 N256: 8192 heads) takes
    each XCD's heads in eight groups, the most the mapping makes; every element
    against the oracle, with padding."""
    w = gen.fwd_inputs(512, 16, 256, 256, 64, "bf16", seed=9310, causal=True, kv_len_range=(1, 256))
    o, lse = gpu_forward(w)
    o_ref, lse_ref = oracle.attention_fwd(w.q, w.k, w.v, w.dtype, w.scale, w.causal, w.kv_lens,
                                          nthreads=host_cores())
    print("head groups B512 H16 N256", compare(o, lse, o_ref, lse_ref, "eight head groups"), flush=True)


# ------------------------------------------------ ragged and edge shapes

@pytest.mark.parametrize("B,H,Nq,Nk,d,dtype,causal,lens", [
    (1, 1, 1, 1, 64, "bf16", False, None),
    (2, 3, 300, 300, 64, "bf16", True, None),          # ragged query and key tails
    (2, 3, 300, 300, 64, "f16", False, None),
    (1, 2, 77, 333, 64, "bf16", True, None),           # Nq < Nk: bottom-right diagonal
    (1, 2, 333, 77, 64, "f16", True, None),            # Nq > Nk: leading rows see nothing
    (3, 2, 200, 250, 64, "bf16", False, (0, 250)),     # padding incl. kv_len 0
    (3, 2, 256, 256, 64, "bf16", True, (1, 256)),      # padding + causal
    (2, 2, 129, 65, 128, "bf16", False, None),         # d = 128
    (2, 2, 260, 260, 128, "f16", True, None),
    (2, 2, 192, 192, 128, "bf16", True, (60, 192)),
    (1, 1, 64, 5, 64, "bf16", False, None),            # Nk smaller than one key tile
])
def test_ragged_shapes(B, H, Nq, Nk, d, dtype, causal, lens):
    w = gen.fwd_inputs(B, H, Nq, Nk, d, dtype, seed=B * 1000 + Nq + Nk + d, causal=causal,
                       scale=1.0 / math.sqrt(d), kv_len_range=lens)
    full_parity(w, f"B{B} H{H} Nq{Nq} Nk{Nk} d{d} {dtype} causal={causal} lens={lens}")


@pytest.mark.parametrize("Nk", [32, 33, 64, 96, 97, 128, 161])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("extra_q", [0, 37])
def test_tile_count_boundaries(Nk, causal, extra_q):
    """Key counts around whole tiles: the kernel runs its unchecked iterations
    for the tiles below min(tiles - 2, the wave's tiles, the first masked
    tile) and checked ones after, so these counts put that split at every
    phase of the three-slot ring; extra query rows move the causal diagonal."""
    Nq = Nk + extra_q
    w = gen.fwd_inputs(1, 2, Nq, Nk, 64, "bf16", seed=9100 + Nk + 7 * extra_q + causal,
                       causal=causal, scale=0.125)
    full_parity(w, f"Nq{Nq} Nk{Nk} causal={causal}")


def test_zero_keys_gives_zero_output_and_minus_inf_lse():
    import torch

    import flashattention_forward_03_amd as fa

    q = torch.randn(2, 2, 70, 64, device="cuda").to(torch.bfloat16)
    k = torch.empty(2, 2, 0, 64, device="cuda", dtype=torch.bfloat16)
    o, lse = fa.forward(q, k, k, causal=False)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


def test_empty_batch_is_a_no_op():
    import torch

    import flashattention_forward_03_amd as fa

    q = torch.empty(0, 4, 16, 64, device="cuda", dtype=torch.float16)
    o, lse = fa.forward(q, q, q)
    assert o.shape == (0, 4, 16, 64) and lse.shape == (0, 4, 16)


# ----------------------------------------------------- invariants on GPU

@pytest.mark.parametrize("dtype,p_ulp", [("bf16", 2.0 ** -9), ("f16", 2.0 ** -11)])
def test_constant_v_rows_reproduce_the_constant(dtype, p_ulp):
    """O = sum(p~ v) / sum(p) with p~ the 16-bit-rounded probabilities that
    feed the MFMA and l summed in fp32: for constant V = c every row is
    c * sum(p~)/sum(p), within |c| * (half an ulp of the 16-bit type)."""
    w = gen.fwd_inputs(2, 4, 512, 512, 64, dtype, 901, causal=True, scale=0.125)
    w.v[...] = gen.float_to_bits_exact(np.full(w.v.shape, -1.5, np.float32), dtype)
    o, _ = gpu_forward(w)
    assert np.max(np.abs(o + 1.5)) <= 1.5 * p_ulp * (1 + 1e-3)


def test_causal_row0_equals_v0_and_zero_q_is_mean():
    w = gen.fwd_inputs(1, 2, 256, 256, 64, "bf16", 902, causal=True, scale=0.125)
    o, lse = gpu_forward(w)
    vf = gen.bits_to_float(w.v, "bf16")
    assert np.max(np.abs(o[0, :, 0] - vf[0, :, 0])) <= 1e-6
    w.q[...] = 0
    o, lse = gpu_forward(w)
    i = np.arange(256)
    np.testing.assert_allclose(lse[0], np.broadcast_to(np.log(i + 1.0), (2, 256)), atol=1e-5)
    means = np.cumsum(vf[0].astype(np.float64), axis=1) / (i + 1.0)[None, :, None]
    assert np.max(np.abs(o[0] - means)) <= 1e-5


def test_large_scores_stay_finite_and_shift_lse():
    """Keys shifted by u: every score of row i grows by scale*q_i.u (64 to 512,
    where exp overflows fp32 without the max shift); O is unchanged and LSE
    moves by exactly that amount."""
    B, H, N, d = 1, 2, 200, 64
    rng = np.random.default_rng(903)
    # quarter grid: q in [0.25, 2] (so q.u > 0), k in [-2, 2]; k + 32 stays exact in bf16
    qf = (np.round(rng.uniform(0.25, 2, (B, H, N, d)) * 4) / 4).astype(np.float32)
    kf = (np.round(rng.uniform(-2, 2, (B, H, N, d)) * 4) / 4).astype(np.float32)
    u = np.full(d, 32.0, np.float32)
    w = gen.fwd_inputs(B, H, N, N, d, "bf16", 903, causal=True, scale=0.125)
    w.q[...] = gen.float_to_bits_exact(qf, "bf16")
    w.k[...] = gen.float_to_bits_exact(kf, "bf16")
    o1, l1 = gpu_forward(w)
    w.k[...] = gen.float_to_bits_exact(kf + u, "bf16")
    o2, l2 = gpu_forward(w)
    shift = 0.125 * (qf.astype(np.float64) @ u.astype(np.float64))
    assert np.all(np.isfinite(o2))
    assert np.max(np.abs(o2 - o1)) <= 1e-2
    assert np.max(np.abs(l2 - (l1 + shift)) / np.maximum(1, np.abs(l1 + shift))) <= 1e-3
    o_ref, l_ref = oracle.attention_fwd(w.q, w.k, w.v, "bf16", 0.125, True)
    compare(o2, l2, o_ref, l_ref, "shifted keys")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_running_max_moves_mid_row(dtype):
    """Keys step up in every coordinate at each 64-key tile, so with positive
    queries a row's maximum score grows by ~6.5 (bf16) / ~3.2 (f16) log2 units
    per tile: the probabilities formed against a stale maximum pass the 2^32 /
    2^15 bound every few tiles and the exact update (new maximum, rescale of O
    and l) runs in the middle of every row, many times.  O and LSE must still
    match the oracle."""
    B, H, N, d = 1, 2, 640, 64
    rng = np.random.default_rng(905)
    qf = (np.round(rng.uniform(0.25, 2, (B, H, N, d)) * 4) / 4).astype(np.float32)
    step = 0.5 if dtype == "bf16" else 0.25          # grid on which k stays exact
    kf = (np.round(rng.uniform(-2, 2, (B, H, N, d)) / step) * step).astype(np.float32)
    kf += (step * (np.arange(N) // 64)).astype(np.float32)[None, None, :, None]
    for causal, lens in ((True, None), (False, (N - 100, N))):
        w = gen.fwd_inputs(B, H, N, N, d, dtype, 905, causal=causal, scale=0.125, kv_len_range=lens)
        w.q[...] = gen.float_to_bits_exact(qf, dtype)
        w.k[...] = gen.float_to_bits_exact(kf, dtype)
        # V halved (exact): with a few dominant keys per row, the 16-bit rounding
        # of P alone puts ~|v|*2^-9 into O; the test is about the maximum
        w.v[...] = gen.round_bits(gen.bits_to_float(w.v, dtype) * 0.5, dtype)
        o, lse = gpu_forward(w)
        o_ref, lse_ref = oracle.attention_fwd(w.q, w.k, w.v, dtype, 0.125, causal, w.kv_lens)
        print(dtype, "causal" if causal else "padded", compare(o, lse, o_ref, lse_ref, "moving max"),
              flush=True)


def test_bitwise_deterministic():
    import torch

    import flashattention_forward_03_amd as fa

    w = gen.fwd_inputs(2, 4, 640, 640, 64, "bf16", 904, causal=True, scale=0.125)
    q, k, v, _ = device_tensors(w)
    o1, l1 = fa.forward(q, k, v, causal=True)
    o2, l2 = fa.forward(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
