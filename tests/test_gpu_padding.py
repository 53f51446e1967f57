"""Padded keys must not reach the outputs.

The gpu-inference page (section 02) combines the padding mask with the causal
mask before the softmax: a key j >= kv_len[b] carries zero probability. The
rows [kv_len, Nk) of K and V are still caller memory, and whatever is stored
there must not change O, LSE or any gradient. These tests store NaN and
+/-Inf bit patterns in those rows. Each result must then be bitwise equal to
the run whose padding holds finite N(0, 1) values, and must match the oracle.
The oracle itself reads only valid keys.

Covered: the forward (contiguous, [B, N, H, d] strided views, grouped-query
K/V heads, head dims whose key tiles are 32 and 64 rows) and the backward
(the dK/dV and dQ passes)."""
import math

import numpy as np
import pytest

import fa_inputs as gen
import oracle
from parity import compare, compare_grad

pytestmark = [pytest.mark.gpu, pytest.mark.usefixtures("fwd_kernel")]

# IEEE bit patterns: quiet NaN, +Inf, -Inf
POISON = {"bf16": (0x7FC0, 0x7F80, 0xFF80), "f16": (0x7E00, 0x7C00, 0xFC00)}


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import flashattention_forward_03_amd as fa

    fa.load_library()


def _poisoned(w):
    """Copies of K and V whose padded rows cycle through NaN, +Inf, -Inf."""
    k, v = w.k.copy(), w.v.copy()
    pats = POISON[w.dtype]
    for b, n in enumerate(w.kv_lens):
        for j in range(int(n), k.shape[2]):
            k[b, :, j, :] = pats[j % 3]
            v[b, :, j, :] = pats[(j + 1) % 3]
    return k, v


def _inputs(B, H, Hkv, N, d, dtype, causal, lens, seed):
    w = gen.fwd_inputs(B, H, N, N, d, dtype, seed=seed, causal=causal,
                       scale=1.0 / math.sqrt(d), Hkv=Hkv)
    w.kv_lens = np.asarray(lens, np.int32)
    return w


def _dev(bits, dtype, bshd):
    t = gen.to_torch(np.ascontiguousarray(bits.transpose(0, 2, 1, 3) if bshd else bits), dtype).cuda()
    return t.transpose(1, 2) if bshd else t


def _forward(w, k_bits, v_bits, bshd=False):
    import torch

    import flashattention_forward_03_amd as fa

    q = _dev(w.q, w.dtype, bshd)
    k = _dev(k_bits, w.dtype, bshd)
    v = _dev(v_bits, w.dtype, bshd)
    kl = torch.from_numpy(w.kv_lens).cuda()
    o, lse = fa.forward(q, k, v, scale=w.scale, causal=w.causal, kv_lens=kl)
    torch.cuda.synchronize()
    return o.cpu().numpy(), lse.cpu().numpy()


# kv_lens cover: a partial last key tile, a length below one tile, a whole
# number of tiles, zero, and the full length
@pytest.mark.parametrize("B,H,Hkv,N,d,dtype,causal,lens,bshd", [
    (4, 2, 2, 200, 64, "bf16", False, (137, 1, 96, 200), False),
    (4, 2, 2, 200, 64, "bf16", True, (137, 33, 64, 0), False),
    (3, 2, 2, 260, 64, "f16", False, (250, 31, 129), False),
    (3, 4, 1, 230, 64, "bf16", False, (101, 229, 7), False),       # multi-query K/V
    (3, 4, 2, 230, 64, "bf16", True, (170, 65, 229), True),        # grouped heads, strided
    (3, 2, 2, 200, 128, "bf16", False, (150, 3, 199), False),
    (3, 2, 2, 200, 96, "f16", False, (150, 70, 5), False),         # 64-key tiles
    (3, 2, 2, 200, 32, "bf16", True, (190, 63, 129), False),       # 64-key tiles
])
def test_forward_ignores_poisoned_padding(B, H, Hkv, N, d, dtype, causal, lens, bshd):
    w = _inputs(B, H, Hkv, N, d, dtype, causal, lens, seed=13000 + N + d + 7 * Hkv + causal)
    o0, l0 = _forward(w, w.k, w.v, bshd)
    kp, vp = _poisoned(w)
    o1, l1 = _forward(w, kp, vp, bshd)
    assert np.array_equal(o0.view(np.uint32), o1.view(np.uint32)), "O depends on padded K/V rows"
    assert np.array_equal(l0.view(np.uint32), l1.view(np.uint32)), "LSE depends on padded K/V rows"
    o_ref, l_ref = oracle.attention_fwd(w.q, kp, vp, w.dtype, w.scale, w.causal, w.kv_lens)
    print(f"poisoned padding d{d} {dtype} causal={causal} lens={lens} bshd={bshd}",
          compare(o1, l1, o_ref, l_ref, "poisoned padding"), flush=True)


@pytest.mark.parametrize("B,H,Hkv,N,d,dtype,causal,lens", [
    (3, 2, 2, 200, 64, "bf16", False, (137, 1, 200)),
    (3, 4, 2, 230, 64, "f16", True, (170, 33, 0)),
    (2, 2, 2, 180, 128, "bf16", True, (150, 97)),
])
def test_backward_ignores_poisoned_padding(B, H, Hkv, N, d, dtype, causal, lens):
    import torch

    import flashattention_forward_03_amd as fa

    w = _inputs(B, H, Hkv, N, d, dtype, causal, lens, seed=13500 + N + d + causal)
    rng = np.random.default_rng(13600 + N)
    g = gen.to_torch(gen.round_bits(rng.standard_normal(w.q.shape, dtype=np.float32), dtype),
                     dtype).cuda()
    kl = torch.from_numpy(w.kv_lens).cuda()

    def run(k_bits, v_bits):
        q = gen.to_torch(w.q, dtype).cuda()
        k = gen.to_torch(k_bits, dtype).cuda()
        v = gen.to_torch(v_bits, dtype).cuda()
        o, lse = fa.forward(q, k, v, scale=w.scale, causal=causal, kv_lens=kl)
        grads = fa.backward(q, k, v, o, lse, g, scale=w.scale, causal=causal, kv_lens=kl)
        torch.cuda.synchronize()
        return [x.cpu().numpy() for x in grads]

    clean = run(w.k, w.v)
    kp, vp = _poisoned(w)
    dirty = run(kp, vp)
    for name, a, b in zip(("dq", "dk", "dv", "delta"), clean, dirty):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"{name} depends on padded K/V"
    dq, dk, dv, _ = dirty
    for b, n in enumerate(lens):
        assert not np.any(dk[b, :, n:]) and not np.any(dv[b, :, n:]), "padded keys got gradients"
    ref = oracle.attention_bwd(w.q, kp, vp, gen.round_bits(
        np.random.default_rng(13600 + N).standard_normal(w.q.shape, dtype=np.float32), dtype),
        dtype, w.scale, causal, w.kv_lens, groups=None)
    out = {}
    for name, x, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref[:3]):
        sel = np.isfinite(r)
        out[name] = compare_grad(x[sel], r[sel], f"poisoned bwd {name}")
    print(f"poisoned bwd d{d} {dtype} causal={causal} lens={lens}", out, flush=True)


@pytest.mark.parametrize("causal", [False, True])
def test_out_of_range_kv_lens_are_clamped(causal):
    """kv_lens outside [0, Nk] act as their clamped values (negative: no key,
    above Nk: every key), bitwise, in the forward and in the backward."""
    import torch

    import flashattention_forward_03_amd as fa

    N = 150
    w = _inputs(4, 2, 2, N, 64, "bf16", causal, (-7, N + 100, 97, 1 << 30), seed=13900 + causal)
    clamped = np.clip(w.kv_lens, 0, N).astype(np.int32)
    g = gen.to_torch(gen.round_bits(np.random.default_rng(13901).standard_normal(w.q.shape, dtype=np.float32),
                                    "bf16"), "bf16").cuda()
    q, k, v = (gen.to_torch(x, "bf16").cuda() for x in (w.q, w.k, w.v))

    def run(lens):
        kl = torch.from_numpy(np.asarray(lens, np.int32)).cuda()
        o, lse = fa.forward(q, k, v, scale=w.scale, causal=causal, kv_lens=kl)
        grads = fa.backward(q, k, v, o, lse, g, scale=w.scale, causal=causal, kv_lens=kl)
        torch.cuda.synchronize()
        return [x.cpu().numpy() for x in (o, lse, *grads)]

    raw, ref = run(w.kv_lens), run(clamped)
    for name, a, b in zip(("o", "lse", "dq", "dk", "dv", "delta"), raw, ref):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"{name}: kv_lens not clamped"
    o_ref, l_ref = oracle.attention_fwd(w.q, w.k, w.v, w.dtype, w.scale, causal, clamped)
    print(f"clamped kv_lens causal={causal}", compare(raw[0], raw[1], o_ref, l_ref, "clamped kv_lens"), flush=True)
