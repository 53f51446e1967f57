"""Randomised GPU parity sweep: forward and decode launches with shapes,
layouts, masks and head groupings drawn from fixed seeds, each compared over
every output element with the fp64 oracle at the same bar as the named cases
(the gradients at the backward's bar).

The draws cover what the named tests fix one at a time, in combination:
batch, query and K/V heads (grouped-query and multi-query), Nq != Nk both
ways, ragged tails, head dims 8..128, both 16-bit types, causal and key
padding (including empty sequences), [B, N, H, d] views and 16-bit O for the
forward; sequence counts, lengths from 0, head groups and both head dims for
the decode; for the backward, head dims 8..128, grouped heads,
padding, both masks, and O/LSE from either the oracle or the GPU forward.
Each case prints its parameters before it runs, so a failing draw names
itself."""
import math

import numpy as np
import pytest

import fa_inputs as gen
import oracle
from parity import compare, compare_grad
from test_gpu_decode import ref_decode, run_decode

pytestmark = pytest.mark.gpu

TORCH_DT = {"f16": "float16", "bf16": "bfloat16", "f32": "float32"}


def _fwd_case(seed):
    rng = np.random.default_rng(seed)
    Hkv = int(rng.choice([1, 2, 3, 4]))
    H = Hkv * int(rng.choice([1, 2, 3, 4]))
    B = int(rng.integers(1, 4))
    Nq = int(rng.integers(1, 600))
    Nk = Nq if rng.random() < 0.4 else int(rng.integers(1, 600))
    d = 8 * int(rng.integers(1, 17))
    return dict(B=B, H=H, Hkv=Hkv, Nq=Nq, Nk=Nk, d=d,
                dtype=str(rng.choice(["f16", "bf16"])),
                causal=bool(rng.random() < 0.5),
                padded=bool(rng.random() < 0.4),
                layout=str(rng.choice(["bhsd", "bshd"])),
                out=str(rng.choice(["f32", "f32", "bf16", "f16"])))


def _dev(bits, dtype, layout):
    """[B, H, N, d] bits as a device tensor, stored [B, N, H, d] for 'bshd'."""
    if layout == "bshd":
        return gen.to_torch(np.ascontiguousarray(bits.transpose(0, 2, 1, 3)), dtype).cuda().transpose(1, 2)
    return gen.to_torch(bits, dtype).cuda()


@pytest.mark.parametrize("seed", range(40))
def test_random_forward(seed, fwd_kernel):
    import torch

    import flashattention_forward_03_amd as fa

    c = _fwd_case(31000 + seed)
    print(f"forward case {seed} ({fwd_kernel} kernel): {c}", flush=True)
    w = gen.fwd_inputs(c["B"], c["H"], c["Nq"], c["Nk"], c["d"], c["dtype"], seed=32000 + seed,
                       causal=c["causal"], scale=1.0 / math.sqrt(c["d"]),
                       kv_len_range=(0, c["Nk"]) if c["padded"] else None, Hkv=c["Hkv"])
    q = _dev(w.q, w.dtype, c["layout"])
    k = _dev(w.k, w.dtype, c["layout"])
    v = _dev(w.v, w.dtype, c["layout"])
    kl = None if w.kv_lens is None else torch.from_numpy(w.kv_lens).cuda()
    odt = getattr(torch, TORCH_DT[c["out"]])
    B, H, Nq, d = c["B"], c["H"], c["Nq"], c["d"]
    if c["layout"] == "bshd":
        o = torch.empty((B, Nq, H, d), dtype=odt, device="cuda").transpose(1, 2)
    else:
        o = torch.empty((B, H, Nq, d), dtype=odt, device="cuda")
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device="cuda")
    fa.forward(q, k, v, scale=w.scale, causal=w.causal, kv_lens=kl, out=(o, lse), out_dtype=odt)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_fwd(w.q, w.k, w.v, w.dtype, w.scale, w.causal, w.kv_lens)
    stats = compare(o.float().cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, f"case {seed}",
                    out_dtype=c["out"])
    print(f"  {stats}", flush=True)


def _dec_case(seed):
    rng = np.random.default_rng(seed)
    Hkv = int(rng.choice([1, 2, 4, 8]))
    group = int(rng.choice([1, 2, 3, 4, 6, 8, 16, 24, 32]))
    while Hkv * group > 64:
        group //= 2
    lo = int(rng.choice([0, 1, 17, 500]))
    hi = lo + int(rng.integers(1, 3000))
    return dict(S=int(rng.integers(1, 40)), H=Hkv * group, Hkv=Hkv,
                d=int(rng.choice([64, 128])), lens=(lo, hi),
                dtype=str(rng.choice(["f16", "bf16"])))


@pytest.mark.parametrize("seed", range(24))
def test_random_decode(seed):
    c = _dec_case(33000 + seed)
    print(f"decode case {seed}: {c}", flush=True)
    num_pages = max(64, int(np.ceil(c["S"] * (c["lens"][1] + 15) / 16 * 1.25)))
    inp = gen.decode_inputs(c["S"], c["H"], c["d"], c["lens"], c["dtype"], seed=34000 + seed,
                            page_size=16, num_pages=num_pages, Hkv=c["Hkv"])
    o, lse = run_decode(inp)
    o_ref, lse_ref = ref_decode(inp)
    stats = compare(o, lse, o_ref, lse_ref, f"decode case {seed}")
    print(f"  {stats}", flush=True)


def _bwd_case(seed):
    rng = np.random.default_rng(seed)
    Hkv = int(rng.choice([1, 2, 4]))
    H = Hkv * int(rng.choice([1, 2])) if Hkv == 4 else Hkv * int(rng.choice([1, 2, 4]))
    Nq = int(rng.integers(1, 400))
    Nk = Nq if rng.random() < 0.4 else int(rng.integers(1, 400))
    return dict(B=int(rng.integers(1, 3)), H=H, Hkv=Hkv, Nq=Nq, Nk=Nk,
                d=8 * int(rng.integers(1, 17)), dtype=str(rng.choice(["f16", "bf16"])),
                causal=bool(rng.random() < 0.5), padded=bool(rng.random() < 0.4),
                fwd=str(rng.choice(["oracle", "gpu"])))


@pytest.mark.parametrize("seed", range(24))
def test_random_backward(seed):
    import torch

    import flashattention_forward_03_amd as fa

    c = _bwd_case(35000 + seed)
    print(f"backward case {seed}: {c}", flush=True)
    w = gen.fwd_inputs(c["B"], c["H"], c["Nq"], c["Nk"], c["d"], c["dtype"], seed=36000 + seed,
                       causal=c["causal"], scale=1.0 / math.sqrt(c["d"]),
                       kv_len_range=(0, c["Nk"]) if c["padded"] else None, Hkv=c["Hkv"])
    g_bits = gen.round_bits(np.random.default_rng(37000 + seed).standard_normal(w.q.shape, dtype=np.float32),
                            c["dtype"])
    q, k, v = (gen.to_torch(x, w.dtype).cuda() for x in (w.q, w.k, w.v))
    kl = None if w.kv_lens is None else torch.from_numpy(w.kv_lens).cuda()
    g = gen.to_torch(g_bits, w.dtype).cuda()
    if c["fwd"] == "gpu":
        o, lse = fa.forward(q, k, v, scale=w.scale, causal=w.causal, kv_lens=kl)
    else:
        o_ref, lse_ref = oracle.attention_fwd(w.q, w.k, w.v, w.dtype, w.scale, w.causal, w.kv_lens)
        o = torch.from_numpy(o_ref.astype(np.float32)).cuda()
        lse = torch.from_numpy(lse_ref.astype(np.float32)).cuda()
    got = fa.backward(q, k, v, o, lse, g, scale=w.scale, causal=w.causal, kv_lens=kl)
    torch.cuda.synchronize()
    ref = oracle.attention_bwd(w.q, w.k, w.v, g_bits, w.dtype, w.scale, w.causal, w.kv_lens)
    stats = {name: compare_grad(x.cpu().numpy(), r, f"backward case {seed} {name}")
             for name, x, r in zip(("dq", "dk", "dv", "delta"), got, ref)}
    print(f"  {stats}", flush=True)
