"""GPU parity of the attention backward (fa_bwd through the binding) against the
fp64 oracle's gradients: dQ, dK, dV and the row term D.

The backward's inputs O and LSE come from the oracle's forward (rounded to
fp32), so each check sees the backward's own arithmetic only; the tests
marked end-to-end feed it the GPU forward's O and LSE instead, as a training
step would (their D then also carries the forward's rounding of O)."""
import math

import numpy as np
import pytest

import fa_inputs as gen
import oracle
from parity import compare_grad, device_tensors

pytestmark = pytest.mark.gpu


def _run(w, g_bits, fwd="oracle"):
    import torch

    import flashattention_forward_03_amd as fa

    q, k, v, kl = device_tensors(w)
    g = gen.to_torch(g_bits, w.dtype).cuda()
    if fwd == "gpu":
        o, lse = fa.forward(q, k, v, scale=w.scale, causal=w.causal, kv_lens=kl)
    else:
        o_ref, lse_ref = oracle.attention_fwd(w.q, w.k, w.v, w.dtype, w.scale, w.causal, w.kv_lens)
        o = torch.from_numpy(o_ref.astype(np.float32)).cuda()
        lse = torch.from_numpy(lse_ref.astype(np.float32)).cuda()
    dq, dk, dv, delta = fa.backward(q, k, v, o, lse, g, scale=w.scale, causal=w.causal,
                                    kv_lens=kl)
    torch.cuda.synchronize()
    return tuple(x.cpu().numpy() for x in (dq, dk, dv, delta))


def _dout(w, seed):
    rng = np.random.default_rng(seed)
    return gen.round_bits(rng.standard_normal(w.q.shape, dtype=np.float32), w.dtype)


def _check(w, g, what, groups=None, fwd="oracle"):
    got = _run(w, g, fwd)
    ref = oracle.attention_bwd(w.q, w.k, w.v, g, w.dtype, w.scale, w.causal, w.kv_lens,
                               groups=groups)
    out = {}
    for name, x, r in zip(("dq", "dk", "dv", "delta"), got, ref):
        sel = ~np.isnan(r)
        out[name] = compare_grad(x[sel], r[sel], f"{what} {name}")
    print(what, out, flush=True)


@pytest.mark.parametrize("B,H,Hkv,Nq,Nk,dtype,causal,lens", [
    (1, 2, 2, 128, 128, "bf16", True, None),
    (2, 4, 2, 200, 200, "bf16", True, (50, 200)),     # grouped heads, padding
    (2, 3, 3, 160, 300, "f16", False, None),           # Nq < Nk, ragged
    (1, 2, 1, 300, 130, "bf16", True, None),           # Nq > Nk: leading rows see nothing
    (1, 2, 2, 77, 333, "f16", True, None),             # bottom-right diagonal
    (2, 2, 2, 1, 100, "bf16", False, (0, 100)),        # one query row; kv_len 0
    (1, 1, 1, 64, 5, "bf16", False, None),             # Nk smaller than a tile
    (2, 8, 1, 96, 96, "f16", True, None),              # multi-query
])
def test_backward_parity(B, H, Hkv, Nq, Nk, dtype, causal, lens):
    w = gen.fwd_inputs(B, H, Nq, Nk, 64, dtype, seed=11000 + B * 100 + Nq + Nk, causal=causal,
                       kv_len_range=lens, Hkv=Hkv)
    _check(w, _dout(w, 11500 + Nq), f"bwd B{B} H{H}/{Hkv} Nq{Nq} Nk{Nk} {dtype} causal={causal} "
                                    f"lens={lens}")


@pytest.mark.parametrize("H,Hkv,Nq,Nk,causal", [
    (2, 2, 33, 33, True),
    (2, 2, 134, 97, True),     # more query rows than keys: rows past the diagonal
    (2, 2, 97, 161, False),
    (4, 1, 161, 161, True),    # four query heads per K/V head: the dK/dV pass walks 4 heads
    (4, 2, 70, 97, False),
    (3, 1, 96, 64, True),
])
def test_backward_tile_boundaries(H, Hkv, Nq, Nk, causal):
    """Key and query counts around whole 32-row tiles, with groups of query
    heads, for the passes' unchecked and checked iterations and for the
    (query head, query tile) counters of the dK/dV pass."""
    w = gen.fwd_inputs(1, H, Nq, Nk, 64, "bf16", seed=11900 + H * 10 + Nq + Nk, causal=causal,
                       Hkv=Hkv)
    _check(w, _dout(w, 11950 + Nq + Nk), f"bwd H{H}/{Hkv} Nq{Nq} Nk{Nk} causal={causal}")


def test_backward_constant_v():
    """Equal V rows: O is that row everywhere, dS = 0, so dQ = dK = 0."""
    w = gen.fwd_inputs(1, 2, 150, 150, 64, "bf16", seed=11600, causal=True)
    w.v[:] = w.v[:, :, :1, :]
    dq, dk, dv, _ = _run(w, _dout(w, 11601))
    assert np.max(np.abs(dq)) <= 1e-2 and np.max(np.abs(dk)) <= 1e-2


def test_backward_deterministic():
    w = gen.fwd_inputs(2, 4, 300, 300, 64, "bf16", seed=11700, causal=True, Hkv=2)
    g = _dout(w, 11701)
    a = _run(w, g)
    b = _run(w, g)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_backward_full_size_sampled_heads():
    """End-to-end: the causal B8 H16 N4096 d64 backward (the launch the bench
    times) on the GPU forward's O and LSE; the oracle computes the full
    gradients of two (batch, head) pairs."""
    w = gen.fwd_workload("fwd_causal_b8h16_n4096_d64_bf16")
    g = _dout(w, 11800)
    _check(w, g, "bwd full size", groups=[0, 8 * 16 - 1], fwd="gpu")


@pytest.mark.parametrize("B,H,Hkv,Nq,Nk,dtype,causal,lens", [
    (1, 2, 2, 128, 128, "bf16", True, None),
    (2, 4, 2, 200, 200, "f16", True, (50, 200)),      # grouped heads, padding
    (2, 3, 3, 160, 300, "bf16", False, None),          # Nq < Nk, ragged
    (1, 2, 1, 300, 130, "f16", True, None),            # Nq > Nk: leading rows see nothing
    (2, 2, 2, 1, 100, "bf16", False, (0, 100)),        # one query row; kv_len 0
    (1, 1, 1, 64, 5, "bf16", False, None),             # Nk smaller than a tile
])
def test_backward_parity_d128(B, H, Hkv, Nq, Nk, dtype, causal, lens):
    w = gen.fwd_inputs(B, H, Nq, Nk, 128, dtype, seed=12000 + B * 100 + Nq + Nk, causal=causal,
                       kv_len_range=lens, Hkv=Hkv)
    _check(w, _dout(w, 12500 + Nq), f"bwd d128 B{B} H{H}/{Hkv} Nq{Nq} Nk{Nk} {dtype} "
                                    f"causal={causal} lens={lens}")


def test_backward_d128_sampled_heads():
    """A causal B4 H16 N2048 d128 backward; the oracle computes the full
    gradients of two (batch, head) pairs."""
    w = gen.fwd_inputs(4, 16, 2048, 2048, 128, "bf16", seed=12900, causal=True)
    _check(w, _dout(w, 12901), "bwd d128 B4 H16 N2048", groups=[0, 4 * 16 - 1])


def test_backward_d128_end_to_end():
    """End-to-end at d = 128: the GPU forward's O and LSE into the backward."""
    w = gen.fwd_inputs(2, 4, 250, 250, 128, "bf16", seed=12950, causal=True, Hkv=2)
    _check(w, _dout(w, 12951), "bwd d128 end-to-end", fwd="gpu")


@pytest.mark.parametrize("d,H,Hkv,Nq,Nk,dtype,causal,lens", [
    (8, 2, 2, 100, 100, "bf16", True, None),           # one 8-column group on the d = 64 tiles
    (32, 4, 2, 161, 97, "f16", False, (40, 97)),       # grouped heads, padding
    (48, 2, 1, 130, 200, "bf16", True, None),
    (72, 2, 2, 97, 97, "bf16", True, None),            # just past 64: the d = 128 tiles
    (96, 3, 3, 70, 150, "f16", True, (0, 150)),        # kv_len 0 in one batch
    (120, 4, 1, 120, 64, "bf16", False, None),         # multi-query
])
def test_backward_head_dims(d, H, Hkv, Nq, Nk, dtype, causal, lens):
    """Head dims other than 64 and 128, on the padded tiles: every gradient
    element against the oracle (the columns past d are neither read nor
    written)."""
    w = gen.fwd_inputs(2, H, Nq, Nk, d, dtype, seed=13000 + d + Nq, causal=causal, kv_len_range=lens,
                       Hkv=Hkv, scale=1.0 / math.sqrt(d))
    _check(w, _dout(w, 13500 + d), f"bwd d{d} H{H}/{Hkv} Nq{Nq} Nk{Nk} {dtype} causal={causal} lens={lens}")
    _check(w, _dout(w, 13600 + d), f"bwd d{d} end-to-end", fwd="gpu")


def test_backward_head_groups_of_a_long_launch():
    """Both passes of a launch of 8192 workgroups (B256 H16 N256, causal, with
    padding) take each XCD's heads in four groups; the oracle computes the full
    gradients of heads from several groups and XCDs."""
    w = gen.fwd_inputs(256, 16, 256, 256, 64, "bf16", seed=13700, causal=True, kv_len_range=(1, 256))
    _check(w, _dout(w, 13701), "bwd head groups B256 H16 N256", groups=[0, 1, 7, 8, 15, 16, 2047, 2048, 4095],
           fwd="gpu")


def test_backward_eight_head_groups():
    """Both passes of a launch of 16384 workgroups (B512 H16 N256, causal, with
    padding) take each XCD's heads in eight groups; full gradients of K/V heads
    from the first, second and last groups of two XCDs and from the middle."""
    w = gen.fwd_inputs(512, 16, 256, 256, 64, "bf16", seed=13710, causal=True, kv_len_range=(1, 256))
    _check(w, _dout(w, 13711), "bwd eight head groups B512 H16 N256",
           groups=[0, 127, 128, 1023, 1024, 5000, 8191], fwd="gpu")


@pytest.mark.parametrize("Nq,Nk", [(0, 70), (70, 0)])
def test_backward_empty_side(Nq, Nk):
    """No query rows: dK = dV = 0 (no row sees the keys).  No keys: dQ = 0 and
    D = 0 (the forward's O is 0 for rows without keys)."""
    import torch

    import flashattention_forward_03_amd as fa

    B, H, d = 2, 2, 64
    q = torch.randn(B, H, Nq, d, device="cuda").to(torch.bfloat16)
    k = torch.randn(B, H, Nk, d, device="cuda").to(torch.bfloat16)
    v = torch.randn(B, H, Nk, d, device="cuda").to(torch.bfloat16)
    g = torch.randn(B, H, Nq, d, device="cuda").to(torch.bfloat16)
    o = torch.zeros(B, H, Nq, d, device="cuda")
    lse = torch.full((B, H, Nq), float("-inf"), device="cuda")
    dq, dk, dv, delta = fa.backward(q, k, v, o, lse, g, causal=False)
    torch.cuda.synchronize()
    for name, x in (("dq", dq), ("dk", dk), ("dv", dv), ("delta", delta)):
        assert not torch.any(x != 0), f"{name} not zero"
