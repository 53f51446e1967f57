"""GPU checks of the paged KV cache append (fa_kv_append) against the oracle's
plain scatter, and the prefill -> decode -> append loop with the host page
allocator against the fp64 oracle decode."""
import numpy as np
import pytest

import fa_inputs as gen
import oracle
from oracle import cache
from parity import compare

pytestmark = pytest.mark.gpu

NAN_BF16 = 0x7FC0


def _t(x):
    import torch

    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _bits(t):
    import numpy as _np
    import torch

    return t.view(torch.int16).cpu().numpy().view(_np.uint16)


def test_append_matches_scatter_bitwise_including_skipped_tokens():
    import torch

    import flashattention_forward_03_amd as fa

    rng = np.random.default_rng(140)
    P, Hkv, d, S, maxp, T = 40, 2, 128, 5, 6, 300
    table = rng.permutation(P)[: S * maxp].reshape(S, maxp).astype(np.int32)
    table[0, 5] = -1            # unused entry
    table[1, 4] = 77            # out of range page
    seq = rng.integers(-1, S + 1, size=T).astype(np.int32)       # includes -1 and S
    pos = rng.integers(-2, maxp * 16 + 3, size=T).astype(np.int32)
    # one write per (seq, pos): duplicates would race
    _, first = np.unique(np.stack([seq, pos]), axis=1, return_index=True)
    seq, pos = seq[np.sort(first)], pos[np.sort(first)]
    T = len(seq)
    kn = gen.round_bits(rng.standard_normal((T, Hkv, d), dtype=np.float32), "bf16")
    vn = gen.round_bits(rng.standard_normal((T, Hkv, d), dtype=np.float32), "bf16")
    kp = np.full((P, Hkv, 16, d), NAN_BF16, np.uint16)
    vp = kp.copy()
    kdev = gen.to_torch(kp, "bf16").cuda()
    vdev = gen.to_torch(vp, "bf16").cuda()
    fa.kv_append(gen.to_torch(kn, "bf16").cuda(), gen.to_torch(vn, "bf16").cuda(), _t(seq),
                 _t(pos), kdev, vdev, _t(table))
    torch.cuda.synchronize()
    n = cache.kv_append(kp, vp, table, seq, pos, kn, vn)
    assert 0 < n < T
    assert np.array_equal(_bits(kdev), kp) and np.array_equal(_bits(vdev), vp)


def test_prefill_decode_append_loop_with_pager():
    """Prefill each sequence in chunks through the allocator's pages, then five
    decode steps that each append one token per sequence (finished sequences
    release their pages, a new one reuses them); every step's decode is held
    to the oracle on the logical cache."""
    import torch

    import flashattention_forward_03_amd as fa

    S, H, Hkv, d = 4, 8, 2, 128
    rng = np.random.default_rng(141)
    pager = fa.Pager(num_pages=96, max_seqs=S, max_pages_per_seq=24)
    kp = torch.zeros((96, Hkv, 16, d), dtype=torch.bfloat16, device="cuda")
    vp = torch.zeros_like(kp)
    lens = rng.integers(100, 300, size=S)
    logical_k = [np.zeros((0, Hkv, d), np.uint16) for _ in range(S)]
    logical_v = [np.zeros((0, Hkv, d), np.uint16) for _ in range(S)]

    def append(s, kn, vn):
        start = logical_k[s].shape[0]
        pager.reserve(s, start + kn.shape[0])
        table = _t(pager.table())
        n = kn.shape[0]
        fa.kv_append(gen.to_torch(kn, "bf16").cuda(), gen.to_torch(vn, "bf16").cuda(),
                     _t(np.full(n, s, np.int32)), _t(np.arange(start, start + n, dtype=np.int32)),
                     kp, vp, table)
        logical_k[s] = np.concatenate([logical_k[s], kn])
        logical_v[s] = np.concatenate([logical_v[s], vn])

    def draw(n):
        return gen.round_bits(rng.standard_normal((n, Hkv, d), dtype=np.float32), "bf16")

    for s in range(S):                       # chunked prefill, 64 tokens a chunk
        for a in range(0, int(lens[s]), 64):
            n = min(64, int(lens[s]) - a)
            append(s, draw(n), draw(n))
    for step in range(5):
        if step == 2:                        # sequence 1 ends; its pages go to a new one
            pager.release(1)
            logical_k[1] = logical_k[1][:0]
            logical_v[1] = logical_v[1][:0]
            append(1, draw(40), draw(40))
        for s in range(S):
            append(s, draw(1), draw(1))
        q = gen.round_bits(rng.standard_normal((S, H, d), dtype=np.float32), "bf16")
        kl = np.array([x.shape[0] for x in logical_k], np.int32)
        table = _t(pager.table())
        o, lse = fa.decode_paged(gen.to_torch(q, "bf16").cuda(), kp, vp, table, _t(kl),
                                 scale=d ** -0.5)
        torch.cuda.synchronize()
        off = np.zeros(S + 1, np.int64)
        off[1:] = np.cumsum(kl)
        ro, rl = oracle.decode(q, np.concatenate(logical_k), np.concatenate(logical_v), off,
                               "bf16", d ** -0.5)
        compare(o.cpu().numpy(), lse.cpu().numpy(), ro, rl, f"step {step}")
    pager.close()


def test_full_batch_prefill_equals_the_input_pools():
    """Appending the whole decode batch (32 sequences, 8 K/V heads, d = 128,
    ~138k tokens) through its page table reproduces the pools the input module
    builds, bit for bit (the launch the bench times)."""
    import torch

    import flashattention_forward_03_amd as fa

    inp = gen.decode_workload("decode_paged_s32h32kv8_d128_bf16")
    want_k = gen.build_pool_device(inp, "k", "cuda")
    kp = torch.zeros_like(want_k)
    vp = torch.zeros_like(want_k)
    seq = np.repeat(np.arange(inp.S, dtype=np.int32), inp.kv_lens)
    pos = np.concatenate([np.arange(n, dtype=np.int32) for n in inp.kv_lens])
    fa.kv_append(gen.to_torch(inp.k, "bf16").cuda(), gen.to_torch(inp.v, "bf16").cuda(), _t(seq),
                 _t(pos), kp, vp, _t(inp.page_table))
    torch.cuda.synchronize()
    assert torch.equal(kp.view(torch.int16), want_k.view(torch.int16))
    del want_k
    want_v = gen.build_pool_device(inp, "v", "cuda")
    assert torch.equal(vp.view(torch.int16), want_v.view(torch.int16))
