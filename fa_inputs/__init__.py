"""Seeded synthetic inputs for the attention forward and paged decode.

This module is shared by the tests, the benchmark and the fp64 oracle's
callers.  It draws random numbers, rounds them to the storage dtype and lays
them out (including the paged KV pool and its page table).  It holds none of
the attention arithmetic: no dot products, no softmax, no reductions.

Recipe (every workload):
  * ``rng = numpy.random.default_rng(seed)`` (PCG64).
  * Values are i.i.d. N(0, 1) drawn as float32 with ``rng.standard_normal``,
    then rounded to the storage dtype with round-to-nearest-even:
    f16 through numpy's ``astype(float16)``, bf16 through torch's CPU
    ``to(bfloat16)``.  Tensors carry raw 16-bit patterns (``uint16``) so
    that both sides decode the very same bits.
  * Forward draw order: Q ``[B, H, Nq, d]``, K, V (each ``[B, Hkv, Nk, d]``
    row-major; Hkv = H unless grouped-query heads are asked for), then the
    key lengths ``integers(lo, hi, endpoint=True)`` when a padding range is
    given.
  * Decode draw order: lengths ``kv_len[S]`` (inclusive range), q ``[S, H, d]``,
    K then V for all cached tokens concatenated over sequences
    (``[sum(kv_len), Hkv, d]``), then the page placement: a seeded permutation
    of the page pool; sequence s's p-th logical page goes to
    ``perm[sum_{s'<s} ceil(kv_len[s']/page) + p]``.
  * Pre-LayerNorm block draw order (``block_inputs``): per-row offsets and
    scales, the activations, LayerNorm gamma and beta, the Q/K/V weights and
    biases, the output weights and bias (recipe in its docstring).

The workloads are the attention shapes of the pages (the forward at N=2048,
d=64 of the flash-attention recipe, a causal B8 H16 d64 sweep, an encoder
shape with per-sequence key padding, decode over a paged cache, and the
encoder block of the BERT-large runs: hidden 1024 = 16 heads x 64).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

DTYPES = ("f16", "bf16")


def round_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to f16/bf16 (RNE) and return the uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        import torch

        out = np.empty(x.shape, dtype=np.uint16)
        flat_in = x.reshape(-1)
        flat_out = out.reshape(-1)
        step = 1 << 24
        for s in range(0, flat_in.size, step):
            t = torch.from_numpy(flat_in[s:s + step]).to(torch.bfloat16)
            flat_out[s:s + step] = t.view(torch.int16).numpy().view(np.uint16)
        return out
    raise ValueError(f"unknown dtype {dtype!r}")


def bits_to_float(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of f16/bf16 bit patterns to float32 (both embed exactly)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float32)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << 16).view(np.float32)
    raise ValueError(f"unknown dtype {dtype!r}")


def float_to_bits_exact(x: np.ndarray, dtype: str) -> np.ndarray:
    """Bits of values already on the dtype grid; raises if any value is not."""
    bits = round_bits(x, dtype)
    if not np.array_equal(bits_to_float(bits, dtype), np.asarray(x, np.float32)):
        raise ValueError("values are not exactly representable in " + dtype)
    return bits


def to_torch(bits: np.ndarray, dtype: str):
    """A CPU torch tensor of the f16/bf16 dtype sharing the given bit patterns."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.float16 if dtype == "f16" else torch.bfloat16)


# ---------------------------------------------------------------- forward ---

@dataclasses.dataclass
class FwdInputs:
    q: np.ndarray            # uint16 [B, H, Nq, d]
    k: np.ndarray            # uint16 [B, Hkv, Nk, d]
    v: np.ndarray            # uint16 [B, Hkv, Nk, d]
    dtype: str
    scale: float
    causal: bool
    kv_lens: Optional[np.ndarray]   # int32 [B] or None (all Nk keys valid)
    seed: int

    @property
    def shape(self):
        B, H, Nq, d = self.q.shape
        return B, H, Nq, self.k.shape[2], d

    @property
    def Hkv(self):
        return self.k.shape[1]


def fwd_inputs(B: int, H: int, Nq: int, Nk: int, d: int, dtype: str, seed: int, *,
               causal: bool, scale: Optional[float] = None,
               kv_len_range: Optional[tuple] = None, Hkv: Optional[int] = None) -> FwdInputs:
    Hkv = H if Hkv is None else Hkv
    if Hkv < 1 or H % Hkv:
        raise ValueError("H must be a multiple of Hkv")
    rng = np.random.default_rng(seed)
    q = round_bits(rng.standard_normal((B, H, Nq, d), dtype=np.float32), dtype)
    k = round_bits(rng.standard_normal((B, Hkv, Nk, d), dtype=np.float32), dtype)
    v = round_bits(rng.standard_normal((B, Hkv, Nk, d), dtype=np.float32), dtype)
    kv_lens = None
    if kv_len_range is not None:
        lo, hi = kv_len_range
        kv_lens = rng.integers(lo, hi, size=B, endpoint=True).astype(np.int32)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    return FwdInputs(q, k, v, dtype, float(scale), bool(causal), kv_lens, seed)


# ----------------------------------------------------------------- decode ---

@dataclasses.dataclass
class DecodeInputs:
    q: np.ndarray            # uint16 [S, H, d]
    k: np.ndarray            # uint16 [T, Hkv, d], sequences concatenated
    v: np.ndarray            # uint16 [T, Hkv, d]
    seq_off: np.ndarray      # int64 [S+1]; sequence s owns tokens seq_off[s]:seq_off[s+1]
    kv_lens: np.ndarray      # int32 [S]
    page_table: np.ndarray   # int32 [S, max_pages]; -1 where unused
    num_pages: int
    page_size: int
    dtype: str
    scale: float
    seed: int

    @property
    def S(self):
        return self.q.shape[0]

    @property
    def H(self):
        return self.q.shape[1]

    @property
    def Hkv(self):
        return self.k.shape[1]

    @property
    def d(self):
        return self.q.shape[2]


def pages_per_seq(kv_lens: np.ndarray, page_size: int) -> np.ndarray:
    return (np.asarray(kv_lens, np.int64) + page_size - 1) // page_size


def decode_inputs(S: int, H: int, d: int, len_range: tuple, dtype: str, seed: int, *,
                  page_size: int = 16, num_pages: int = 1 << 16,
                  max_pages: Optional[int] = None, scale: Optional[float] = None,
                  identity_pages: bool = False, Hkv: Optional[int] = None) -> DecodeInputs:
    """Draw one decode batch.  ``identity_pages`` keeps the same draws but lays
    the sequences' pages out contiguously (page p of the pool in logical order).
    ``Hkv``: number of K/V heads (default H)."""
    Hkv = H if Hkv is None else Hkv
    if Hkv < 1 or H % Hkv:
        raise ValueError("H must be a multiple of Hkv")
    rng = np.random.default_rng(seed)
    lo, hi = len_range
    kv_lens = rng.integers(lo, hi, size=S, endpoint=True).astype(np.int32)
    q = round_bits(rng.standard_normal((S, H, d), dtype=np.float32), dtype)
    T = int(kv_lens.sum())
    k = round_bits(rng.standard_normal((T, Hkv, d), dtype=np.float32), dtype)
    v = round_bits(rng.standard_normal((T, Hkv, d), dtype=np.float32), dtype)
    perm = rng.permutation(num_pages).astype(np.int64)
    if identity_pages:
        perm = np.arange(num_pages, dtype=np.int64)
    npg = pages_per_seq(kv_lens, page_size)
    if max_pages is None:
        max_pages = int(-(-hi // page_size))
    if int(npg.max(initial=0)) > max_pages:
        raise ValueError("max_pages too small for the drawn lengths")
    if int(npg.sum()) > num_pages:
        raise ValueError("page pool too small for the drawn lengths")
    table = np.full((S, max_pages), -1, dtype=np.int32)
    start = 0
    for s in range(S):
        n = int(npg[s])
        table[s, :n] = perm[start:start + n]
        start += n
    seq_off = np.zeros(S + 1, dtype=np.int64)
    seq_off[1:] = np.cumsum(kv_lens.astype(np.int64))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    return DecodeInputs(q, k, v, seq_off, kv_lens, table, num_pages, page_size,
                        dtype, float(scale), seed)


def page_slots(inp: DecodeInputs):
    """For every cached token (concatenated order): (physical page, row in page)."""
    phys = np.empty(inp.k.shape[0], dtype=np.int64)
    row = np.empty(inp.k.shape[0], dtype=np.int64)
    for s in range(inp.S):
        a, b = int(inp.seq_off[s]), int(inp.seq_off[s + 1])
        t = np.arange(b - a, dtype=np.int64)
        phys[a:b] = inp.page_table[s, t // inp.page_size]
        row[a:b] = t % inp.page_size
    return phys, row


def build_pool_host(inp: DecodeInputs, which: str, fill_bits: int = 0) -> np.ndarray:
    """Scatter the logical K (or V) into a host pool ``[num_pages, Hkv, page, d]``.

    Slots not holding a cached token keep ``fill_bits`` (0 = +0.0; a NaN
    pattern for the poison test).  Only for small pools: the full-size pool
    is built on the device by :func:`build_pool_device`.
    """
    src = inp.k if which == "k" else inp.v
    pool = np.full((inp.num_pages, inp.Hkv, inp.page_size, inp.d), fill_bits, dtype=np.uint16)
    phys, row = page_slots(inp)
    pool[phys, :, row, :] = src
    return pool


def build_pool_device(inp: DecodeInputs, which: str, device, fill_bits: int = 0):
    """Same layout as :func:`build_pool_host`, assembled in device memory by torch."""
    import torch

    tdt = torch.float16 if inp.dtype == "f16" else torch.bfloat16
    pool = torch.empty((inp.num_pages, inp.Hkv, inp.page_size, inp.d), dtype=torch.int16,
                       device=device)
    pool.fill_(int(np.array(fill_bits, np.uint16).view(np.int16)))
    phys, row = page_slots(inp)
    src = inp.k if which == "k" else inp.v
    phys_t = torch.from_numpy(phys).to(device)
    row_t = torch.from_numpy(row).to(device)
    step = 1 << 16
    for a in range(0, src.shape[0], step):
        chunk = torch.from_numpy(src[a:a + step].view(np.int16)).to(device)
        pool[phys_t[a:a + step], :, row_t[a:a + step], :] = chunk
    return pool.view(tdt)


def gather_logical(pool: np.ndarray, inp: DecodeInputs) -> np.ndarray:
    """Read the cached tokens back out of a host pool through the page table."""
    phys, row = page_slots(inp)
    return pool[phys, :, row, :]


# ------------------------------------------------------ pre-LN block ---

@dataclasses.dataclass
class BlockInputs:
    """One pre-LayerNorm attention block: activations, LayerNorm parameters and
    the two dense layers (weights output-major, as a dense layer's matrix)."""
    x: np.ndarray            # uint16 [B*N, C]   (token t = b*N + n), C = H*d
    gamma: np.ndarray        # float32 [C]
    beta: np.ndarray         # float32 [C]
    w_qkv: np.ndarray        # uint16 [(H + 2*Hkv)*d, C]  rows: Q heads, K heads, V heads
    b_qkv: np.ndarray        # float32 [(H + 2*Hkv)*d]
    w_o: np.ndarray          # uint16 [C, H*d]
    b_o: np.ndarray          # float32 [C]
    B: int
    N: int
    H: int
    Hkv: int
    d: int
    dtype: str
    eps: float
    scale: float
    causal: bool
    kv_lens: Optional[np.ndarray]   # int32 [B] or None
    seed: int

    @property
    def C(self):
        return self.H * self.d

    @property
    def T(self):
        return self.B * self.N


def block_inputs(B: int, N: int, H: int, d: int, dtype: str, seed: int, *,
                 Hkv: Optional[int] = None, causal: bool = False, eps: float = 1e-5,
                 scale: Optional[float] = None, row_offset: float = 1.0,
                 kv_len_range: Optional[tuple] = None) -> BlockInputs:
    """Draw one block's inputs.

    Draw order: per-row offsets ``uniform(-row_offset, row_offset)`` [T] and
    scales ``uniform(0.5, 2)`` [T], z ~ N(0, 1) [T, C] (x = offset + scale * z,
    a residual stream whose rows differ in mean and spread), gamma = 1 +
    0.1 N(0, 1), beta = 0.1 N(0, 1), W_qkv = N(0, 1) / sqrt(C), b_qkv =
    0.02 N(0, 1), W_o = N(0, 1) / sqrt(H*d), b_o = 0.02 N(0, 1), then the
    key lengths when a padding range is given.  Weights and x are rounded to
    the 16-bit dtype; gamma, beta and the biases stay float32.
    """
    Hkv = H if Hkv is None else Hkv
    if Hkv < 1 or H % Hkv:
        raise ValueError("H must be a multiple of Hkv")
    T, C = B * N, H * d
    R = (H + 2 * Hkv) * d
    rng = np.random.default_rng(seed)
    off = rng.uniform(-row_offset, row_offset, size=T).astype(np.float32)
    scl = rng.uniform(0.5, 2.0, size=T).astype(np.float32)
    z = rng.standard_normal((T, C), dtype=np.float32)
    x = round_bits(off[:, None] + scl[:, None] * z, dtype)
    gamma = (1.0 + 0.1 * rng.standard_normal(C, dtype=np.float32)).astype(np.float32)
    beta = (0.1 * rng.standard_normal(C, dtype=np.float32)).astype(np.float32)
    w_qkv = round_bits(rng.standard_normal((R, C), dtype=np.float32) / np.float32(math.sqrt(C)),
                       dtype)
    b_qkv = (0.02 * rng.standard_normal(R, dtype=np.float32)).astype(np.float32)
    w_o = round_bits(rng.standard_normal((C, H * d), dtype=np.float32)
                     / np.float32(math.sqrt(H * d)), dtype)
    b_o = (0.02 * rng.standard_normal(C, dtype=np.float32)).astype(np.float32)
    kv_lens = None
    if kv_len_range is not None:
        lo, hi = kv_len_range
        kv_lens = rng.integers(lo, hi, size=B, endpoint=True).astype(np.int32)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    return BlockInputs(x, gamma, beta, w_qkv, b_qkv, w_o, b_o, B, N, H, Hkv, d, dtype,
                       float(eps), float(scale), bool(causal), kv_lens, seed)


# -------------------------------------------------------------- workloads ---

# Named workloads: the forward shapes and the decode batch the measurements
# are quoted on.  Seeds are 1000*workload + sub-index.
FWD_WORKLOADS = {
    "fwd_b1h1_n256_d64_f16": dict(B=1, H=1, Nq=256, Nk=256, d=64, dtype="f16",
                                  causal=False, scale=0.125, seed=1000),
    "fwd_b1h1_n2048_d64_f16": dict(B=1, H=1, Nq=2048, Nk=2048, d=64, dtype="f16",
                                   causal=False, scale=0.125, seed=2000),
    "fwd_causal_b8h16_n512_d64_bf16": dict(B=8, H=16, Nq=512, Nk=512, d=64, dtype="bf16",
                                           causal=True, scale=0.125, seed=3000),
    "fwd_causal_b8h16_n1024_d64_bf16": dict(B=8, H=16, Nq=1024, Nk=1024, d=64,
                                            dtype="bf16", causal=True, scale=0.125,
                                            seed=3001),
    "fwd_causal_b8h16_n2048_d64_bf16": dict(B=8, H=16, Nq=2048, Nk=2048, d=64,
                                            dtype="bf16", causal=True, scale=0.125,
                                            seed=3002),
    "fwd_causal_b8h16_n4096_d64_bf16": dict(B=8, H=16, Nq=4096, Nk=4096, d=64,
                                            dtype="bf16", causal=True, scale=0.125,
                                            seed=3003),
    "fwd_padded_b8h16_n2048_d64_bf16": dict(B=8, H=16, Nq=2048, Nk=2048, d=64,
                                            dtype="bf16", causal=False, scale=0.125,
                                            kv_len_range=(1024, 2048), seed=4000),
    # grouped-query heads: 16 query heads over 4 K/V heads
    "fwd_causal_b8h16kv4_n4096_d64_bf16": dict(B=8, H=16, Hkv=4, Nq=4096, Nk=4096, d=64,
                                               dtype="bf16", causal=True, scale=0.125,
                                               seed=3004),
}

# The encoder block of the pages' BERT-large runs (hidden 1024 = 16 heads x 64),
# at the attention workload's batch and length, non-causal as an encoder is.
BLOCK_WORKLOADS = {
    "prenorm_block_b8_n4096_h16_d64_bf16": dict(B=8, N=4096, H=16, d=64, dtype="bf16",
                                                causal=False, seed=6000),
}

DECODE_WORKLOADS = {
    "decode_paged_s32h32_d128_bf16": dict(S=32, H=32, d=128, len_range=(512, 8192),
                                          dtype="bf16", page_size=16, num_pages=1 << 16,
                                          scale=1.0 / math.sqrt(128), seed=5000),
    # the same batch with grouped-query heads: 32 query heads over 8 K/V heads
    "decode_paged_s32h32kv8_d128_bf16": dict(S=32, H=32, Hkv=8, d=128, len_range=(512, 8192),
                                             dtype="bf16", page_size=16, num_pages=1 << 16,
                                             scale=1.0 / math.sqrt(128), seed=5001),
}


def fwd_workload(name: str) -> FwdInputs:
    w = dict(FWD_WORKLOADS[name])
    B, H, Nq, Nk, d = (w.pop(x) for x in ("B", "H", "Nq", "Nk", "d"))
    dtype = w.pop("dtype")
    seed = w.pop("seed")
    return fwd_inputs(B, H, Nq, Nk, d, dtype, seed, **w)


def decode_workload(name: str, **over) -> DecodeInputs:
    w = dict(DECODE_WORKLOADS[name])
    w.update(over)
    S, H, d = w.pop("S"), w.pop("H"), w.pop("d")
    len_range, dtype, seed = w.pop("len_range"), w.pop("dtype"), w.pop("seed")
    return decode_inputs(S, H, d, len_range, dtype, seed, **w)


def block_workload(name: str, **over) -> BlockInputs:
    w = dict(BLOCK_WORKLOADS[name])
    w.update(over)
    B, N, H, d = w.pop("B"), w.pop("N"), w.pop("H"), w.pop("d")
    dtype, seed = w.pop("dtype"), w.pop("seed")
    return block_inputs(B, N, H, d, dtype, seed, **w)
