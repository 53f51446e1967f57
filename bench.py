#!/usr/bin/env python3
"""Benchmark of the exact-attention hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic inputs
already resident in HBM:
  * fa_fwd on the causal B=8, H=16, N=4096, d=64 bf16 forward (the workload
    the headline TFLOP/s is quoted on), and
  * fa_decode_paged on the decode batch (32 sequences x 32 heads, d=128,
    lengths uniform in [512, 8192], 16-token pages scattered over a
    65536-page pool), and
  * fa_decode_paged_gqa on the same kind of batch with 32 query heads over
    8 K/V heads (grouped-query attention).
Each kernel is bracketed by HIP events on the stream it is launched on.

Prints ONE JSON line.  ``value`` is forward TFLOP/s: nominal FLOPs
4*B*H*Nq*Nk*d, halved for causal, over the forward's median launch time in
the timed steps (HIP events); ``fwd`` also gives p10 / p90 / mean.
``roofline`` is the forward kernel against the dense bf16 MFMA peak;
``decode`` and ``decode_gqa`` carry the decode GB/s against the 8 TB/s HBM
peak.
``configs`` times every configuration of the workloads one by one (20 warmup
+ 200 launches each by default, median / p10 / p90): the f16 B1 H1 N256 and
N2048 forwards, the causal B8 H16 d64 sweep N = 512 / 1024 / 2048 / 4096, the
padded B8 H16 N2048 encoder shape (nominal and effective FLOPs) and the
decode batch; beside each, the fp64 oracle's wall time on the host cores
(one thread too for the B1 H1 configs and the decode) and the parity of the
GPU output over every element.  ``cpu_baseline`` is the oracle on the
headline workload (every row, all host cores up to 16).
``backward`` times fa_bwd (the dQ pass with the row term D, then the dK/dV pass) on the headline
shape outside the step: nominal FLOPs 2.5x the forward's (five products of
the forward's size against two).
``kv_append`` times fa_kv_append writing the whole grouped-query decode batch
(every cached token's K and V rows) into its pages, against the 8 TB/s peak
on the bytes read plus written.
``variants`` times generalised forward launches outside the step (head dims
32 / 96 / 128, [B, N, H, d] inputs with a bf16 O, 4 K/V heads) on the same
causal B8 H16 N4096 shape, each against the bf16 MFMA peak.
All the timings outside the step use the same protocol as ``configs``.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import fa_inputs as gen  # noqa: E402

FWD_WORKLOAD = "fwd_causal_b8h16_n4096_d64_bf16"
DEC_WORKLOAD = "decode_paged_s32h32_d128_bf16"
GQA_WORKLOAD = "decode_paged_s32h32kv8_d128_bf16"

# MI355X published peaks (dense, no sparsity)
PEAK_BF16_TFLOPS = 2516.6   # 256 CUs x 4096 FLOP/clk/CU x 2.4 GHz
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_fwd_causal_b8h16_n4096_d64.json")
DEC_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_decode_paged_s32h32_d128.json")
GQA_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_decode_paged_s32h32kv8_d128.json")


def attention_flops(B, H, Nq, Nk, d, causal):
    """Nominal FLOPs: 4*B*H*Nq*Nk*d, halved for causal (gpu-inference page,
    section 02: symmetric accounting; work skipped at the diagonal is not
    credited and work done on the diagonal tiles is not counted twice)."""
    f = 4.0 * B * H * Nq * Nk * d
    return f * 0.5 if causal else f


def decode_bytes(kv_lens, H, d, elem=2, with_io=True, Hkv=None):
    """Algorithmic bytes of one decode call: every cached K and V element once
    (Hkv heads of them), plus q, o (fp32), lse (fp32) of the H query heads, the
    page-table entries used and kv_lens."""
    Hkv = H if Hkv is None else Hkv
    tokens = int(np.sum(kv_lens))
    b = 2 * tokens * Hkv * d * elem
    if with_io:
        S = len(kv_lens)
        pages = int(np.sum((np.asarray(kv_lens) + 15) // 16))
        b += S * H * d * elem + S * H * d * 4 + S * H * 4 + pages * 4 + S * 4
    return b


def fwd_bytes(B, H, Nq, Nk, d, elem=2):
    """Compulsory HBM bytes of the forward: Q, K, V once, O (fp32) and LSE once."""
    return B * H * (Nq + 2 * Nk) * d * elem + B * H * Nq * d * 4 + B * H * Nq * 4


def effective_flops(B, H, Nq, Nk, d, causal, kv_lens=None):
    """FLOPs over the (row, key) pairs the mask leaves valid: 4*d per pair.
    For key padding: 4*H*d*Nq*sum_b kv_len_b (non-causal); for causal, each
    row i counts min(i+1+Nk-Nq, kv_len) keys."""
    lens = np.full(B, Nk, np.int64) if kv_lens is None else np.asarray(kv_lens, np.int64)
    if not causal:
        return 4.0 * H * d * Nq * float(lens.sum())
    i = np.arange(Nq, dtype=np.int64)
    tot = 0
    for n in lens:
        tot += int(np.clip(np.minimum(i + 1 + Nk - Nq, n), 0, None).sum())
    return 4.0 * H * d * float(tot)


def launch_stats(ms):
    """Median, p10, p90 and mean of per-launch times (ms)."""
    ms = np.asarray(ms, np.float64)
    return {"median_ms": float(np.median(ms)), "p10_ms": float(np.percentile(ms, 10)),
            "p90_ms": float(np.percentile(ms, 90)), "mean_ms": float(ms.mean()),
            "launches": int(ms.size)}


def event_times(fn, warmup, launches):
    """Per-launch times (ms) of fn() over `launches` launches after `warmup`
    untimed ones: each launch bracketed by HIP events on the current stream
    (the stream the library launches on)."""
    import torch

    for _ in range(warmup):
        fn()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(launches)]
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) for a, b in evs])


FWD_SOURCES = ("fa_fwd.hip", "fa_tile.h", "fa_common.h")


def kernel_digest(sources=FWD_SOURCES):
    """Digest of the kernel sources and of the flags the first one (the
    kernel's own file) is compiled with."""
    from flashattention_forward_03_amd import build as fa_build

    h = hashlib.sha256()
    for name in sources:
        with open(os.path.join(ROOT, "flashattention_forward_03_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    h.update(" ".join(fa_build.flags_for(sources[0])).replace(ROOT, "").encode())
    return h.hexdigest()[:16]


DEC_SOURCES = ("fa_decode.hip", "fa_tile.h", "fa_common.h")


def measured_traffic(path=TRAFFIC_FILE, sources=FWD_SOURCES):
    """HBM bytes per launch from the committed rocprofv3 counter runs, or None
    if they were taken on a different version of the kernel sources."""
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_digest") != kernel_digest(sources):
        return None
    return t.get("bytes_per_launch")


def _counter_means(csv_path, counter):
    import csv
    import collections

    vals = collections.defaultdict(list)
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                vals[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in vals.items()}


def record_traffic(d, copy_bytes):
    """Turn rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs (KiB per dispatch) of
    this benchmark and of a plain copy of copy_bytes into bytes per launch:
    each counter is scaled by (bytes the copy moves) / (what it reads for the
    copy).  Expects run dirs <d>/{fwd,gqa,copy}_{FETCH_SIZE,WRITE_SIZE}/ holding
    run_counter_collection.csv: fwd_* from a run with --no-gqa (forward and
    decode), gqa_* from a run with --gqa-only (see the profile notes for the
    commands)."""
    def one(sub, counter):
        return _counter_means(os.path.join(d, sub, "run_counter_collection.csv"), counter)

    factor = {}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        copy = [v for k, v in one("copy_" + c, c).items() if "copyBuffer" in k]
        factor[c] = copy_bytes / (copy[0] * 1024.0)
    out = {}
    for label, run, match, path, sources in (
            ("fwd", "fwd_", "fwd_kernel", TRAFFIC_FILE, FWD_SOURCES),
            ("decode", "fwd_", "decode_", DEC_TRAFFIC_FILE, DEC_SOURCES),
            ("decode_gqa", "gqa_", "decode_", GQA_TRAFFIC_FILE, DEC_SOURCES)):
        if not os.path.isdir(os.path.join(d, run + "FETCH_SIZE")):
            continue
        rec = {"kernel_digest": kernel_digest(sources), "calibration": factor}
        total = 0.0
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            kib = sum(v for k, v in one(run + c, c).items() if match in k)
            rec[c + "_KiB_raw"] = kib
            rec[c + "_bytes"] = kib * 1024.0 * factor[c]
            total += rec[c + "_bytes"]
        rec["bytes_per_launch"] = total
        with open(path, "w") as f:
            json.dump(rec, f, indent=1)
        out[label] = rec
    print(json.dumps(out, indent=1))


# The pages' workload configurations: name -> config number.  Config 3 is the
# causal sweep (the headline is its N = 4096 point); config 5 is the decode.
FWD_CONFIGS = (
    ("fwd_b1h1_n256_d64_f16", "1"),
    ("fwd_b1h1_n2048_d64_f16", "2"),
    ("fwd_causal_b8h16_n512_d64_bf16", "3"),
    ("fwd_causal_b8h16_n1024_d64_bf16", "3"),
    ("fwd_causal_b8h16_n2048_d64_bf16", "3"),
    (FWD_WORKLOAD, "3"),
    ("fwd_padded_b8h16_n2048_d64_bf16", "4"),
)
SINGLE_THREAD_CONFIGS = ("1", "2", "5")


def _parity(o, lse, o_ref, lse_ref):
    """max / mean |dO| and max |dLSE| / max(1, |LSE|) over every element."""
    err = np.abs(np.asarray(o, np.float64) - o_ref)
    fin = np.isfinite(lse_ref)
    lse = np.asarray(lse, np.float64)
    lrel = np.abs(lse[fin] - lse_ref[fin]) / np.maximum(1.0, np.abs(lse_ref[fin]))
    return {"max_abs": float(err.max(initial=0.0)), "mean_abs": float(err.mean()),
            "lse_rel": float(lrel.max(initial=0.0))}


def time_fwd_configs(fa, dev, warmup, launches, with_oracle, cores, headline=None):
    """Every forward configuration: GPU time per launch (median, p10, p90 over
    `launches` after `warmup`, HIP events), nominal TFLOP/s (and effective
    TFLOP/s over the unmasked pairs), and, with_oracle, the fp64 oracle's wall
    time on all `cores` (single-threaded too for configs 1 and 2) with the
    parity of the GPU output over every element.  ``headline``: the headline
    workload's (inputs, device tensors) to reuse."""
    import torch

    out = {}
    for name, cfg in FWD_CONFIGS:
        print(f"[bench] config {cfg}: {name}", file=sys.stderr, flush=True)
        if headline is not None and name == FWD_WORKLOAD:
            w, (q, k, v) = headline
        else:
            w = gen.fwd_workload(name)
            q, k, v = (gen.to_torch(x, w.dtype).to(dev) for x in (w.q, w.k, w.v))
        B, H, Nq, Nk, d = w.shape
        kl = None if w.kv_lens is None else torch.from_numpy(w.kv_lens).to(dev)
        o = torch.empty((B, H, Nq, d), dtype=torch.float32, device=dev)
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=dev)
        fa.forward(q, k, v, scale=w.scale, causal=w.causal, kv_lens=kl, out=(o, lse))   # checked call
        # the timed launches go straight to the C entry point with the arguments
        # the checked call validated, so that the small configurations' times
        # are the library's and not the Python argument checks'
        args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, Nq, Nk, d,
                float(w.scale), int(w.causal), None if kl is None else kl.data_ptr(),
                fa.FA_DTYPE_BF16 if w.dtype == "bf16" else fa.FA_DTYPE_F16,
                torch.cuda.current_stream().cuda_stream)

        def call():
            rc = fa.fa_fwd(*args)
            if rc != fa.FA_OK:
                raise RuntimeError(f"fa_fwd: {fa.fa_status_str(rc)}")
        st = launch_stats(event_times(call, warmup, launches))
        nom = attention_flops(B, H, Nq, Nk, d, w.causal)
        eff = effective_flops(B, H, Nq, Nk, d, w.causal, w.kv_lens)
        sec = st["median_ms"] / 1e3
        rec = {"config": cfg, "shape": {"B": B, "H": H, "Nq": Nq, "Nk": Nk, "d": d},
               "dtype": w.dtype, "causal": w.causal, "padded": w.kv_lens is not None,
               "seed": w.seed, "gpu": st, "flops_nominal": nom, "flops_effective": eff,
               "TFLOP/s": nom / sec / 1e12, "TFLOP/s_effective": eff / sec / 1e12,
               "frac": nom / sec / 1e12 / PEAK_BF16_TFLOPS, "workgroups": (Nq + 127) // 128 * B * H}
        if with_oracle:
            import oracle

            o_h, l_h = o.cpu().numpy(), lse.cpu().numpy()
            t0 = time.perf_counter()
            o_ref, l_ref = oracle.attention_fwd(w.q, w.k, w.v, w.dtype, w.scale, w.causal,
                                                w.kv_lens, nthreads=cores)
            dt = time.perf_counter() - t0
            rec["oracle"] = {"seconds": dt, "threads": cores, "TFLOP/s": eff / dt / 1e12,
                             "rows": B * H * Nq}
            if cfg in SINGLE_THREAD_CONFIGS:
                t0 = time.perf_counter()
                oracle.attention_fwd(w.q, w.k, w.v, w.dtype, w.scale, w.causal, w.kv_lens,
                                     nthreads=1)
                rec["oracle"]["seconds_1_thread"] = time.perf_counter() - t0
            rec["parity"] = _parity(o_h, l_h, o_ref, l_ref)
            del o_ref, l_ref
        out[name] = rec
        del o, lse
        if headline is None or name != FWD_WORKLOAD:
            del q, k, v
    return out


def oracle_decode_times(dec, o_gpu, lse_gpu, cores):
    """The decode batch through the fp64 oracle (all cores, then one thread),
    and the parity of the GPU output over every element."""
    import oracle

    t0 = time.perf_counter()
    o_ref, l_ref = oracle.decode(dec.q, dec.k, dec.v, dec.seq_off, dec.dtype, dec.scale,
                                 nthreads=cores)
    dt = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.decode(dec.q, dec.k, dec.v, dec.seq_off, dec.dtype, dec.scale, nthreads=1)
    dt1 = time.perf_counter() - t0
    flops = 4.0 * dec.q.shape[1] * dec.q.shape[2] * float(np.sum(dec.kv_lens))
    return {"seconds": dt, "threads": cores, "seconds_1_thread": dt1, "TFLOP/s": flops / dt / 1e12,
            "parity": _parity(o_gpu, lse_gpu, o_ref, l_ref)}


def cpu_baseline_from(rec):
    """The bench's cpu_baseline: the oracle on the headline workload (every
    row), from its config record."""
    B, H, Nq = rec["shape"]["B"], rec["shape"]["H"], rec["shape"]["Nq"]
    orc = rec["oracle"]
    return {"value": orc["TFLOP/s"], "unit": "TFLOP/s", "cores": orc["threads"], "kind": "oracle",
            "sample": f"all {B * H * Nq} query rows ({FWD_WORKLOAD}), fp64, {orc['seconds']:.1f} s",
            "seconds": orc["seconds"], "sample_parity": rec["parity"]}


# Generalised forward launches on the headline shape (causal B8 H16 N4096):
# name -> (d, K/V heads, inputs stored [B, N, H, d], O dtype)
VARIANTS = {
    "fwd_causal_b8h16_n4096_d128_bf16": (128, 16, False, "f32"),
    "fwd_causal_b8h16_n4096_d96_bf16": (96, 16, False, "f32"),
    "fwd_causal_b8h16_n4096_d32_bf16": (32, 16, False, "f32"),
    "fwd_causal_b8h16_n4096_d64_bf16_bshd_obf16": (64, 16, True, "bf16"),
    "fwd_causal_b8h16kv4_n4096_d64_bf16": (64, 4, False, "f32"),
}


def time_variants(fa, dev, steps, warmup):
    """Per variant: average launch time over `steps` launches (HIP events on
    the launch stream) after `warmup`, and TFLOP/s against the bf16 peak.
    Inputs are N(0, 1) from a seeded device generator (timing only; the
    parity tests cover these launch configurations)."""
    import torch

    B, H, N = 8, 16, 4096
    out = {}
    g = torch.Generator(device=dev)
    for i, (name, (d, hkv, bshd, odt)) in enumerate(VARIANTS.items()):
        g.manual_seed(7000 + i)

        def draw(heads):
            shape = (B, N, heads, d) if bshd else (B, heads, N, d)
            x = torch.randn(shape, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
            return x.transpose(1, 2) if bshd else x

        q, k, v = draw(H), draw(hkv), draw(hkv)
        otd = {"f32": torch.float32, "bf16": torch.bfloat16}[odt]
        o = torch.empty((B, N, H, d) if bshd else (B, H, N, d), dtype=otd, device=dev)
        o = o.transpose(1, 2) if bshd else o
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
        scale = 1.0 / math.sqrt(d)
        st = launch_stats(event_times(
            lambda: fa.forward(q, k, v, scale=scale, causal=True, out=(o, lse)), warmup, steps))
        tf = attention_flops(B, H, N, N, d, True) / (st["median_ms"] / 1e3) / 1e12
        out[name] = dict(st, **{"TFLOP/s": tf, "frac": tf / PEAK_BF16_TFLOPS, "d": d, "H_kv": hkv,
                                "layout": "bshd" if bshd else "bhsd", "o_dtype": odt})
        del q, k, v, o, lse
    return out


def time_append(fa, dev, gq, kp, vp, pt, steps, warmup):
    """fa_kv_append of every token of the grouped-query decode batch into its
    pages (rewriting the pools with their own contents); average over `steps`
    launches with HIP events.  Bytes: the new rows read plus the rows written."""
    import torch

    kn = gen.to_torch(gq.k, gq.dtype).to(dev)
    vn = gen.to_torch(gq.v, gq.dtype).to(dev)
    seq = torch.from_numpy(np.repeat(np.arange(gq.S, dtype=np.int32), gq.kv_lens)).to(dev)
    pos = torch.from_numpy(np.concatenate([np.arange(n, dtype=np.int32)
                                           for n in gq.kv_lens])).to(dev)
    st = launch_stats(event_times(lambda: fa.kv_append(kn, vn, seq, pos, kp, vp, pt), warmup, steps))
    T = int(gq.kv_lens.sum())
    nbytes = 2 * 2 * T * gq.Hkv * gq.d * 2 + 2 * T * 4 + T * 4   # K+V read and written; ids
    gbs = nbytes / (st["median_ms"] / 1e3) / 1e9
    return dict(st, **{"workload": GQA_WORKLOAD, "tokens": T, "bytes": nbytes, "GB/s": gbs,
                       "frac": gbs / PEAK_HBM_GBS})


def time_backward(fa, dev, q, k, v, o, lse, w, steps, warmup):
    """fa_bwd on the headline forward's inputs, O and LSE, with a seeded N(0, 1)
    output gradient; average launch time over `steps` (HIP events)."""
    import torch

    g = torch.Generator(device=dev)
    g.manual_seed(8000)
    dout = torch.randn(q.shape, generator=g, device=dev, dtype=torch.float32).to(q.dtype)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    fa.forward(q, k, v, scale=w.scale, causal=w.causal, out=(o, lse))
    outs = (torch.empty_like(o), torch.empty(k.shape, dtype=torch.float32, device=dev),
            torch.empty(v.shape, dtype=torch.float32, device=dev),
            torch.empty((2,) + tuple(lse.shape), dtype=torch.float32, device=dev))
    st = launch_stats(event_times(
        lambda: fa.backward(q, k, v, o, lse, dout, scale=w.scale, causal=w.causal, out=outs),
        warmup, steps))
    flops = 2.5 * attention_flops(B, H, Nq, Nk, d, w.causal)
    tf = flops / (st["median_ms"] / 1e3) / 1e12
    return dict(st, **{"workload": FWD_WORKLOAD, "TFLOP/s": tf, "frac": tf / PEAK_BF16_TFLOPS,
                       "flops": flops})


def time_decode_groups(fa, dev, steps, warmup):
    """The grouped-query decode batch with wider groups (the S32 H32 d128 batch
    drawn with 4 K/V heads: 8 query heads each, and with 1: multi-query),
    which take the matrix-core decode kernel; average over `steps` launches
    (HIP events), GB/s on the same algorithmic bytes as `decode`."""
    import torch

    out = {}
    for hkv in (4, 1):
        w = gen.decode_workload(GQA_WORKLOAD, Hkv=hkv)
        kp = gen.build_pool_device(w, "k", dev)
        vp = gen.build_pool_device(w, "v", dev)
        q = gen.to_torch(w.q, w.dtype).to(dev)
        pt = torch.from_numpy(w.page_table).to(dev)
        kl = torch.from_numpy(w.kv_lens).to(dev)
        wsb = fa.fa_decode_workspace_bytes(w.S, w.H, w.d, w.page_table.shape[1], 16)
        ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
        o = torch.empty((w.S, w.H, w.d), dtype=torch.float32, device=dev)
        lse = torch.empty((w.S, w.H), dtype=torch.float32, device=dev)
        call = lambda: fa.decode_paged(q, kp, vp, pt, kl, scale=w.scale, workspace=ws, out=(o, lse))
        st = launch_stats(event_times(call, warmup, steps))
        nb = decode_bytes(w.kv_lens, w.H, w.d, Hkv=hkv)
        gbs = nb / (st["median_ms"] / 1e3) / 1e9
        out[f"h32_kv{hkv}"] = dict(st, **{"H": w.H, "H_kv": hkv, "bytes": nb, "GB/s": gbs,
                                          "frac": gbs / PEAK_HBM_GBS, "tokens": int(w.kv_lens.sum())})
        del kp, vp
    return out


BLOCK_WORKLOAD = "prenorm_block_b8_n4096_h16_d64_bf16"


def time_block(fa, dev, steps, warmup):
    """The pre-LayerNorm attention block (fa_prenorm_attention) on its encoder
    workload, and each of its stages alone (the same kernels through their own
    entry points): average over `steps` launches with HIP events after
    `warmup`.  FLOPs: 2 T C (H + 2 H_kv) d for the Q/K/V layer, 2 T C^2 for
    the output layer, the attention forward's count for the attention."""
    import torch

    w = gen.block_workload(BLOCK_WORKLOAD)
    tdt = torch.bfloat16
    x = gen.to_torch(w.x, w.dtype).to(dev)
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)
    folded = fa.ln_fold_weights(f32(w.gamma), f32(w.beta), gen.to_torch(w.w_qkv, w.dtype).to(dev),
                                f32(w.b_qkv))
    w_o = gen.to_torch(w.w_o, w.dtype).to(dev)
    b_o = f32(w.b_o)
    T, C, d, H, Hkv, N, B = w.T, w.C, w.d, w.H, w.Hkv, w.N, w.B
    R = (H + 2 * Hkv) * d
    kw = dict(B=B, N=N, H=H, H_kv=Hkv, eps=w.eps, scale=w.scale, causal=w.causal)
    y, ws = fa.prenorm_attention(x, folded, w_o, b_o, **kw)
    views = fa.prenorm_workspace_views(ws, B, N, H, Hkv, d, tdt)
    qkv, o_flat, lse = views["qkv"], views["o"], views["lse"]
    heads = qkv.view(B, N, H + 2 * Hkv, d)
    q, k, v = (heads[:, :, :H].transpose(1, 2), heads[:, :, H:H + Hkv].transpose(1, 2),
               heads[:, :, H + Hkv:].transpose(1, 2))
    o4 = o_flat.view(B, N, H, d).transpose(1, 2)
    mean, rstd = views["mean"], views["rstd"]
    stages = {
        "ln_stats": lambda: fa.ln_stats(x, w.eps),
        "qkv_gemm": lambda: fa.ln_linear(x, mean, rstd, folded, out=qkv),
        "attention": lambda: fa.forward(q, k, v, scale=w.scale, causal=w.causal, out=(o4, lse)),
        "out_gemm": lambda: fa.linear(o_flat, w_o, b_o, x, out=y),
        "block": lambda: fa.prenorm_attention(x, folded, w_o, b_o, workspace=ws, out=y, **kw),
    }
    res = {}
    for name, fn in stages.items():
        res[name] = launch_stats(event_times(fn, warmup, steps))["median_ms"]
    fl_qkv = 2.0 * T * C * R
    fl_out = 2.0 * T * C * C
    fl_att = attention_flops(B, H, N, N, d, w.causal)
    tfs = lambda fl, ms: fl / (ms / 1e3) / 1e12
    out = {"workload": BLOCK_WORKLOAD, "tokens": T, "block_ms": res["block"],
           "tokens/s": T / (res["block"] / 1e3),
           "TFLOP/s": tfs(fl_qkv + fl_out + fl_att, res["block"]),
           "stages_ms": {k: res[k] for k in ("ln_stats", "qkv_gemm", "attention", "out_gemm")},
           "qkv_gemm_TFLOP/s": tfs(fl_qkv, res["qkv_gemm"]),
           "out_gemm_TFLOP/s": tfs(fl_out, res["out_gemm"]),
           "attention_TFLOP/s": tfs(fl_att, res["attention"]),
           "ln_stats_GB/s": T * C * 2 / (res["ln_stats"] / 1e3) / 1e9}
    out["qkv_gemm_frac"] = out["qkv_gemm_TFLOP/s"] / PEAK_BF16_TFLOPS
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="0 skips the fp64 oracle timings (cpu_baseline and the per-config "
                         "oracle wall times); any other value runs them")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-configuration timings (and with them the oracle)")
    ap.add_argument("--config-launches", type=int, default=200,
                    help="timed launches per configuration")
    ap.add_argument("--config-warmup", type=int, default=20,
                    help="untimed launches before each configuration's timed ones")
    ap.add_argument("--no-decode", action="store_true", help="time the forward only")
    ap.add_argument("--no-gqa", action="store_true", help="skip the grouped-query decode")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the generalised forward launches timed after the steps")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the backward timed after the steps")
    ap.add_argument("--no-append", action="store_true",
                    help="skip the paged-cache append timed after the steps")
    ap.add_argument("--no-block", action="store_true",
                    help="skip the pre-LayerNorm attention block timed after the steps")
    ap.add_argument("--block-only", action="store_true",
                    help="only time the pre-LayerNorm attention block (for its profiles) and exit")
    ap.add_argument("--gqa-only", action="store_true",
                    help="only run the grouped-query decode (for its counter runs) and exit")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run a plain device copy of this many bytes (HBM counter "
                         "calibration for rocprofv3 FETCH_SIZE / WRITE_SIZE) and exit")
    ap.add_argument("--record-traffic", metavar="DIR",
                    help="write the profiles/traffic_*.json files from rocprofv3 counter "
                         "runs in DIR (CPU only) and exit")
    args = ap.parse_args()
    if args.record_traffic:
        record_traffic(args.record_traffic, args.copy_bytes or (1 << 30))
        return
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              "(the path shards by batch/head with no communication; see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import flashattention_forward_03_amd as fa

    fa.load_library()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if args.copy_bytes:
        src = torch.ones(args.copy_bytes // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": args.copy_bytes, "launches": 3}), flush=True)
        return
    if args.block_only:
        print(json.dumps({"prenorm_block": time_block(fa, dev, args.steps, args.warmup)}),
              flush=True)
        return
    if args.gqa_only:
        gq = gen.decode_workload(GQA_WORKLOAD)
        pools = (gen.build_pool_device(gq, "k", dev), gen.build_pool_device(gq, "v", dev))
        g_q = gen.to_torch(gq.q, gq.dtype).to(dev)
        g_pt = torch.from_numpy(gq.page_table).to(dev)
        g_kl = torch.from_numpy(gq.kv_lens).to(dev)
        for _ in range(args.warmup + args.steps):
            fa.decode_paged(g_q, *pools, g_pt, g_kl, scale=gq.scale)
        torch.cuda.synchronize()
        print(json.dumps({"gqa_only": GQA_WORKLOAD, "launches": args.warmup + args.steps}),
              flush=True)
        return

    print(f"[bench] generating {FWD_WORKLOAD}", file=sys.stderr, flush=True)
    w = gen.fwd_workload(FWD_WORKLOAD)
    B, H, Nq, Nk, d = w.shape
    q, k, v = (gen.to_torch(x, w.dtype).to(dev) for x in (w.q, w.k, w.v))
    o = torch.empty((B, H, Nq, d), dtype=torch.float32, device=dev)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=dev)
    fflops = attention_flops(B, H, Nq, Nk, d, w.causal)

    dec = None
    if not args.no_decode:
        print(f"[bench] generating {DEC_WORKLOAD}", file=sys.stderr, flush=True)
        dec = gen.decode_workload(DEC_WORKLOAD)
        kp = gen.build_pool_device(dec, "k", dev)
        vp = gen.build_pool_device(dec, "v", dev)
        dq = gen.to_torch(dec.q, dec.dtype).to(dev)
        dpt = torch.from_numpy(dec.page_table).to(dev)
        dkl = torch.from_numpy(dec.kv_lens).to(dev)
        do = torch.empty((dec.S, dec.H, dec.d), dtype=torch.float32, device=dev)
        dlse = torch.empty((dec.S, dec.H), dtype=torch.float32, device=dev)
        ws_bytes = fa.fa_decode_workspace_bytes(dec.S, dec.H, dec.d, dec.page_table.shape[1], 16)
        ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
        dbytes = decode_bytes(dec.kv_lens, dec.H, dec.d)

    gq = None
    if not args.no_decode and not args.no_gqa:
        print(f"[bench] generating {GQA_WORKLOAD}", file=sys.stderr, flush=True)
        gq = gen.decode_workload(GQA_WORKLOAD)
        g_kp = gen.build_pool_device(gq, "k", dev)
        g_vp = gen.build_pool_device(gq, "v", dev)
        g_q = gen.to_torch(gq.q, gq.dtype).to(dev)
        g_pt = torch.from_numpy(gq.page_table).to(dev)
        g_kl = torch.from_numpy(gq.kv_lens).to(dev)
        g_o = torch.empty((gq.S, gq.H, gq.d), dtype=torch.float32, device=dev)
        g_lse = torch.empty((gq.S, gq.H), dtype=torch.float32, device=dev)
        g_wsb = fa.fa_decode_workspace_bytes(gq.S, gq.H, gq.d, gq.page_table.shape[1], 16)
        g_ws = torch.empty(max(g_wsb, 16), dtype=torch.uint8, device=dev)
        gbytes = decode_bytes(gq.kv_lens, gq.H, gq.d, Hkv=gq.Hkv)

    def step(evs=None):
        if evs is not None:
            evs[0].record()
        fa.forward(q, k, v, scale=w.scale, causal=True, out=(o, lse))
        if evs is not None:
            evs[1].record()
        if dec is not None:
            fa.decode_paged(dq, kp, vp, dpt, dkl, scale=dec.scale, workspace=ws, out=(do, dlse))
            if evs is not None:
                evs[2].record()
        if gq is not None:
            fa.decode_paged(g_q, g_kp, g_vp, g_pt, g_kl, scale=gq.scale, workspace=g_ws,
                            out=(g_o, g_lse))
            if evs is not None:
                evs[3].record()

    print("[bench] warmup", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    print("[bench] timing", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    fwd_ms = np.array([e[0].elapsed_time(e[1]) for e in events])
    fwd_st = launch_stats(fwd_ms)
    fwd_s = fwd_st["median_ms"] / 1e3
    tflops = fflops / fwd_s / 1e12
    cores = min(16, len(os.sched_getaffinity(0)))
    result = {
        "metric": "attention fwd TFLOP/s (causal B8 H16 d64 N4096) + % MFMA peak; decode GB/s",
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": elapsed * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": FWD_WORKLOAD, "B": B, "H": H, "Nq": Nq, "Nk": Nk, "d": d,
                   "causal": True, "decode_workload": None if dec is None else DEC_WORKLOAD,
                   "decode_gqa_workload": None if gq is None else GQA_WORKLOAD},
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": tflops / PEAK_BF16_TFLOPS,
                     "traffic": measured_traffic()},
        "peak_basis": {"bf16_mfma_TFLOP/s": PEAK_BF16_TFLOPS,
                       "derivation": "256 CUs x 4096 bf16 FLOP/clk/CU x 2.4 GHz (dense)",
                       "hbm_GB/s": PEAK_HBM_GBS},
        "fwd": dict(fwd_st, flops=fflops, compulsory_bytes=fwd_bytes(B, H, Nq, Nk, d),
                    value_basis="median launch time over the timed steps"),
    }
    if dec is not None:
        dec_st = launch_stats([e[1].elapsed_time(e[2]) for e in events])
        gbs = dbytes / (dec_st["median_ms"] / 1e3) / 1e9
        result["decode"] = dict(dec_st, **{
            "GB/s": gbs, "bytes": dbytes, "tokens": int(dec.kv_lens.sum()),
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": gbs / PEAK_HBM_GBS,
                         "traffic": measured_traffic(DEC_TRAFFIC_FILE, DEC_SOURCES)}})
    if gq is not None:
        g_st = launch_stats([e[2].elapsed_time(e[3]) for e in events])
        g_gbs = gbytes / (g_st["median_ms"] / 1e3) / 1e9
        result["decode_gqa"] = dict(g_st, **{
            "GB/s": g_gbs, "bytes": gbytes, "tokens": int(gq.kv_lens.sum()), "H": gq.H,
            "H_kv": gq.Hkv,
            "roofline": {"bound": "hbm", "achieved": g_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": g_gbs / PEAK_HBM_GBS,
                         "traffic": measured_traffic(GQA_TRAFFIC_FILE, DEC_SOURCES)}})
    with_oracle = args.cpu_seconds > 0
    if not args.no_configs:
        # every configuration of the pages' workloads, one by one (20 warmup +
        # 200 launches each, median / p10 / p90), with the oracle timed beside
        # each on the host cores
        cfgs = time_fwd_configs(fa, dev, args.config_warmup, args.config_launches, with_oracle,
                                cores, headline=(w, (q, k, v)))
        if dec is not None:
            call = lambda: fa.decode_paged(dq, kp, vp, dpt, dkl, scale=dec.scale, workspace=ws,
                                           out=(do, dlse))
            st = launch_stats(event_times(call, args.config_warmup, args.config_launches))
            rec = {"config": "5", "gpu": st, "bytes": dbytes,
                   "GB/s": dbytes / (st["median_ms"] / 1e3) / 1e9, "seed": dec.seed}
            rec["frac"] = rec["GB/s"] / PEAK_HBM_GBS
            if with_oracle:
                print("[bench] config 5: oracle", file=sys.stderr, flush=True)
                rec["oracle"] = oracle_decode_times(dec, do.cpu().numpy(), dlse.cpu().numpy(), cores)
            cfgs[DEC_WORKLOAD] = rec
        result["configs"] = cfgs
        if with_oracle:
            result["cpu_baseline"] = cpu_baseline_from(cfgs[FWD_WORKLOAD])
    if not args.no_backward:
        print("[bench] backward", file=sys.stderr, flush=True)
        result["backward"] = time_backward(fa, dev, q, k, v, o, lse, w, args.config_launches,
                                           args.config_warmup)
    if gq is not None and not args.no_variants:
        print("[bench] decode with wider query-head groups", file=sys.stderr, flush=True)
        result["decode_groups"] = time_decode_groups(fa, dev, args.config_launches,
                                                     args.config_warmup)
    if gq is not None and not args.no_append:
        print("[bench] kv append", file=sys.stderr, flush=True)
        result["kv_append"] = time_append(fa, dev, gq, g_kp, g_vp, g_pt, args.config_launches,
                                          args.config_warmup)
    if not args.no_variants:
        print("[bench] forward variants", file=sys.stderr, flush=True)
        result["variants"] = time_variants(fa, dev, args.config_launches, args.config_warmup)
    if not args.no_block:
        print("[bench] pre-LayerNorm block", file=sys.stderr, flush=True)
        result["prenorm_block"] = time_block(fa, dev, args.config_launches, args.config_warmup)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
