"""The library on the caller's stream, and inside a captured HIP graph.

Every entry point launches only on the stream it is given and never
synchronises, so a side stream must give the same bits as the default one,
and a graph captured from the calls must replay them.  The graph holds the
forward (tiled and split-key kernels), the backward, and the decode entry
point that allocates nothing (its scratch is a fixed device array, so the
graph needs no workspace).  Each replay follows eager work that rewrites the
inputs, and is checked bit for bit against an eager run on the same inputs."""
import numpy as np
import pytest

import fa_inputs as gen
from parity import compare
import oracle

pytestmark = pytest.mark.gpu


def _fwd_inputs(seed, Nq=300, causal=True):
    return gen.fwd_inputs(2, 4, Nq, Nq, 64, "bf16", seed=seed, causal=causal, Hkv=2)


def _dev(w):
    import torch

    return (gen.to_torch(w.q, w.dtype).cuda(), gen.to_torch(w.k, w.dtype).cuda(),
            gen.to_torch(w.v, w.dtype).cuda())


def test_side_stream_gives_the_default_stream_bits():
    import torch

    import flashattention_forward_03_amd as fa

    w = _fwd_inputs(15000)
    q, k, v = _dev(w)
    o0, l0 = fa.forward(q, k, v, scale=w.scale, causal=True)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()   # default priority
    with torch.cuda.stream(side):
        o1, l1 = fa.forward(q, k, v, scale=w.scale, causal=True)
        g = torch.ones_like(q)
        d1 = fa.backward(q, k, v, o1, l1, g, scale=w.scale, causal=True)
    side.synchronize()
    d0 = fa.backward(q, k, v, o0, l0, g, scale=w.scale, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    for a, b in zip(d0, d1):
        assert torch.equal(a, b)


@pytest.mark.parametrize("kernel", ["tiled", "split", "split8"])
def test_graph_capture_replays_match_eager_runs(kernel, monkeypatch):
    import torch

    import flashattention_forward_03_amd as fa

    monkeypatch.setenv("FA_FWD_SPLIT", {"tiled": "0", "split": "1", "split8": "8"}[kernel])
    w = _fwd_inputs(15100)
    q, k, v = _dev(w)
    B, H, N, d = q.shape
    o = torch.empty(B, H, N, d, dtype=torch.float32, device="cuda")
    lse = torch.empty(B, H, N, dtype=torch.float32, device="cuda")
    g = gen.to_torch(gen.round_bits(np.random.default_rng(15101).standard_normal(w.q.shape, dtype=np.float32),
                                    "bf16"), "bf16").cuda()
    dq = torch.empty_like(o)
    dk = torch.empty(k.shape, dtype=torch.float32, device="cuda")
    dv = torch.empty_like(dk)
    delta = torch.empty(2, B, H, N, dtype=torch.float32, device="cuda")

    inp = gen.decode_inputs(6, 8, 128, (1, 900), "bf16", seed=15102, page_size=16, num_pages=512, Hkv=2)
    kp = gen.build_pool_device(inp, "k", "cuda")
    vp = gen.build_pool_device(inp, "v", "cuda")
    dqv = gen.to_torch(inp.q, "bf16").cuda()
    pt = torch.from_numpy(inp.page_table).cuda()
    kl = torch.from_numpy(inp.kv_lens).cuda()
    S, Hd, dd = inp.q.shape
    do = torch.empty(S, Hd, dd, dtype=torch.float32, device="cuda")
    dl = torch.empty(S, Hd, dtype=torch.float32, device="cuda")

    def step(stream_handle):
        fa.forward(q, k, v, scale=w.scale, causal=True, out=(o, lse))
        fa.backward(q, k, v, o, lse, g, scale=w.scale, causal=True, out=(dq, dk, dv, delta))
        st = fa.fa_decode_paged_noalloc(dqv.data_ptr(), kp.data_ptr(), vp.data_ptr(), pt.data_ptr(),
                                        kl.data_ptr(), do.data_ptr(), dl.data_ptr(), S, Hd, 2, dd, 16,
                                        inp.page_table.shape[1], kp.shape[0], float(inp.scale),
                                        fa.FA_DTYPE_BF16, stream_handle)
        assert st == fa.FA_OK, fa.fa_status_str(st)

    def outputs():
        return [x.clone() for x in (o, lse, dq, dk, dv, do, dl)]

    step(torch.cuda.current_stream().cuda_stream)   # warm up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()

    rng = np.random.default_rng(15103)
    for replay in range(3):
        # eager work between replays: new inputs written in place
        q.copy_(gen.to_torch(gen.round_bits(rng.standard_normal(w.q.shape, dtype=np.float32), "bf16"),
                             "bf16").cuda())
        dqv.copy_(gen.to_torch(gen.round_bits(rng.standard_normal(inp.q.shape, dtype=np.float32), "bf16"),
                               "bf16").cuda())
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = outputs()
        step(torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        want = outputs()
        for i, (a, b) in enumerate(zip(got, want)):
            assert torch.equal(a, b), f"replay {replay}: output {i} differs from the eager run"
    # the last replay's forward also against the oracle
    qb = q.cpu().view(torch.int16).numpy().view(np.uint16)
    o_ref, lse_ref = oracle.attention_fwd(qb, w.k, w.v, "bf16", w.scale, True, None)
    compare(o.cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, f"graph replay ({kernel} kernel)")
