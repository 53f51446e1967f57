"""GPU parity of the generalised forward (fa_fwd_ex through the binding): head
dims other than 64 / 128, strided layouts ([B, N, H, d] activations, a fused
QKV buffer, K/V shared across the batch) and a 16-bit O, against the fp64
oracle on the logical [B, H, N, d] tensors."""
import math

import numpy as np
import pytest

import fa_inputs as gen
import oracle
from parity import compare, gpu_forward, host_cores

pytestmark = [pytest.mark.gpu, pytest.mark.usefixtures("fwd_kernel")]

TORCH_DT = {"f16": "float16", "bf16": "bfloat16", "f32": "float32"}


def _tdt(name):
    import torch

    return getattr(torch, TORCH_DT[name])


def _bshd(bits, dtype):
    """Device tensor stored [B, N, H, d], returned as a [B, H, N, d] view."""
    x = gen.to_torch(np.ascontiguousarray(bits.transpose(0, 2, 1, 3)), dtype).cuda()
    return x.transpose(1, 2)


def _run(w, q, k, v, out_dtype="f32", o_layout="bhsd"):
    import torch

    import flashattention_forward_03_amd as fa

    B, H, Nq, Nk, d = w.shape
    kl = None if w.kv_lens is None else torch.from_numpy(w.kv_lens).cuda()
    if o_layout == "bshd":
        o = torch.empty((B, Nq, H, d), dtype=_tdt(out_dtype), device="cuda").transpose(1, 2)
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device="cuda")
        out = (o, lse)
    else:
        out = None
    o, lse = fa.forward(q, k, v, scale=w.scale, causal=w.causal, kv_lens=kl, out=out,
                        out_dtype=_tdt(out_dtype))
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


def _ref(w):
    return oracle.attention_fwd(w.q, w.k, w.v, w.dtype, w.scale, w.causal, w.kv_lens)


# ------------------------------------------------------------ head dims

@pytest.mark.parametrize("d", [32, 48, 80, 96, 120, 8])
@pytest.mark.parametrize("causal", [False, True])
def test_head_dims(d, causal):
    dtype = "bf16" if d % 16 else "f16"
    w = gen.fwd_inputs(2, 3, 257, 300, d, dtype, seed=9000 + d + causal, causal=causal,
                       scale=1.0 / math.sqrt(d), kv_len_range=(1, 300))
    o, lse = gpu_forward(w)
    what = f"d={d} {dtype} causal={causal}"
    print(what, compare(o, lse, *_ref(w), what), flush=True)


@pytest.mark.parametrize("d", [32, 96, 128])
def test_head_dims_full_size(d):
    """B8 H16 N4096 causal bf16 at d = 32 / 96 / 128 (launches the bench times):
    every output element against the oracle."""
    w = gen.fwd_inputs(8, 16, 4096, 4096, d, "bf16", seed=9100 + d, causal=True,
                       scale=1.0 / math.sqrt(d))
    o, lse = gpu_forward(w)
    o_ref, lse_ref = oracle.attention_fwd(w.q, w.k, w.v, w.dtype, w.scale, True, None,
                                          nthreads=host_cores())
    print(d, compare(o, lse, o_ref, lse_ref, f"d={d}"), flush=True)


# ------------------------------------------------------------- 16-bit O

@pytest.mark.parametrize("out_dtype", ["bf16", "f16"])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_16bit_output(out_dtype, dtype):
    w = gen.fwd_inputs(2, 4, 300, 300, 64, dtype, seed=9200, causal=True,
                       kv_len_range=(50, 300))
    from parity import device_tensors

    q, k, v, _ = device_tensors(w)
    o16, lse16 = _run(w, q, k, v, out_dtype=out_dtype)
    what = f"O {out_dtype} from {dtype}"
    print(what, compare(o16, lse16, *_ref(w), what, out_dtype=out_dtype), flush=True)


def test_16bit_output_is_the_rounded_fp32_output():
    """The 16-bit epilogue rounds the same fp32 O to nearest even, bit for bit."""
    import torch

    from parity import device_tensors

    w = gen.fwd_inputs(2, 4, 200, 200, 80, "bf16", seed=9300, causal=False)
    q, k, v, _ = device_tensors(w)
    o32, l32 = _run(w, q, k, v, out_dtype="f32")
    for od in ("bf16", "f16"):
        o16, l16 = _run(w, q, k, v, out_dtype=od)
        want = torch.from_numpy(o32).to(_tdt(od)).float().numpy()
        assert np.array_equal(o16, want), od
        assert np.array_equal(l16, l32)


# ------------------------------------------------------------ strided layouts

@pytest.mark.parametrize("causal,dtype,d", [(True, "bf16", 64), (False, "f16", 128),
                                            (True, "bf16", 80)])
def test_bshd_layout(causal, dtype, d):
    w = gen.fwd_inputs(2, 4, 333, 333, d, dtype, seed=9400 + d, causal=causal,
                       scale=1.0 / math.sqrt(d), kv_len_range=(100, 333))
    q, k, v = (_bshd(x, dtype) for x in (w.q, w.k, w.v))
    assert not q.is_contiguous()
    o, lse = _run(w, q, k, v, o_layout="bshd")
    what = f"bshd {dtype} d={d} causal={causal}"
    print(what, compare(o, lse, *_ref(w), what), flush=True)


def test_fused_qkv_buffer_gqa_16bit_out():
    """q, k, v as views of one [B, N, H + 2*H_kv, d] projection output; 2 K/V
    heads for 8 query heads; d = 96; O written bf16 into a [B, N, H, d] buffer."""
    import torch

    B, H, Hkv, N, d = 2, 8, 2, 290, 96
    w = gen.fwd_inputs(B, H, N, N, d, "bf16", seed=9500, causal=True, Hkv=Hkv,
                       scale=1.0 / math.sqrt(d))
    buf = np.concatenate([w.q.transpose(0, 2, 1, 3), w.k.transpose(0, 2, 1, 3),
                          w.v.transpose(0, 2, 1, 3)], axis=2)        # [B, N, H+2Hkv, d]
    t = gen.to_torch(np.ascontiguousarray(buf), "bf16").cuda()
    q = t[:, :, :H].transpose(1, 2)
    k = t[:, :, H:H + Hkv].transpose(1, 2)
    v = t[:, :, H + Hkv:].transpose(1, 2)
    assert q.stride() == (N * (H + 2 * Hkv) * d, d, (H + 2 * Hkv) * d, 1)
    o, lse = _run(w, q, k, v, out_dtype="bf16", o_layout="bshd")
    print("fused qkv", compare(o, lse, *_ref(w), "fused qkv", out_dtype="bf16"), flush=True)
    del t, torch


def test_kv_shared_across_batch():
    """K/V batch stride 0: every batch entry attends to the same K/V."""
    import torch

    w1 = gen.fwd_inputs(1, 4, 200, 260, 64, "f16", seed=9600, causal=False)
    q = gen.fwd_inputs(3, 4, 200, 260, 64, "f16", seed=9601, causal=False).q
    w = gen.FwdInputs(q, np.repeat(w1.k, 3, axis=0), np.repeat(w1.v, 3, axis=0), "f16",
                      w1.scale, False, None, 9601)
    kk = gen.to_torch(w1.k, "f16").cuda().expand(3, -1, -1, -1)
    vv = gen.to_torch(w1.v, "f16").cuda().expand(3, -1, -1, -1)
    assert kk.stride(0) == 0
    qq = gen.to_torch(q, "f16").cuda()
    o, lse = _run(w, qq, kk, vv)
    print("shared kv", compare(o, lse, *_ref(w), "shared kv"), flush=True)
    del torch


def test_bshd_headline_full_size():
    """The headline causal B8 H16 N4096 d64 launch on [B, N, H, d] buffers with a
    bf16 O (the variant the bench times): every output element."""
    w = gen.fwd_workload("fwd_causal_b8h16_n4096_d64_bf16")
    q, k, v = (_bshd(x, "bf16") for x in (w.q, w.k, w.v))
    o, lse = _run(w, q, k, v, out_dtype="bf16", o_layout="bshd")
    o_ref, lse_ref = oracle.attention_fwd(w.q, w.k, w.v, w.dtype, w.scale, True, None,
                                          nthreads=host_cores())
    print("bshd headline", compare(o, lse, o_ref, lse_ref, "bshd headline", out_dtype="bf16"),
          flush=True)
