"""The seeded input generator: determinism, rounding and page placement."""
import numpy as np

import fa_inputs as gen


def test_same_seed_same_bits():
    a = gen.fwd_inputs(2, 2, 17, 19, 8, "bf16", 5, causal=True, kv_len_range=(3, 19))
    b = gen.fwd_inputs(2, 2, 17, 19, 8, "bf16", 5, causal=True, kv_len_range=(3, 19))
    for x, y in [(a.q, b.q), (a.k, b.k), (a.v, b.v), (a.kv_lens, b.kv_lens)]:
        assert np.array_equal(x, y)
    c = gen.fwd_inputs(2, 2, 17, 19, 8, "bf16", 6, causal=True)
    assert not np.array_equal(a.q, c.q)


def test_bf16_rounding_is_round_to_nearest_even():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(200000).astype(np.float32)
    # include exact ties: low 16 bits == 0x8000
    u = x.view(np.uint32).copy()
    u[:1000] = (u[:1000] & 0xFFFF0000) | 0x8000
    x = u.view(np.float32)
    ref = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    assert np.array_equal(gen.round_bits(x, "bf16"), ref)


def test_f16_rounding_matches_ieee_cast():
    x = np.array([1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 65504.0, 6.0e-8, -2.5], np.float32)
    bits = gen.round_bits(x, "f16")
    # ties to even: 1+2^-11 -> 1.0 ; 1+3*2^-11 -> 1+2^-9
    assert gen.bits_to_float(bits, "f16").tolist() == [1.0, 1.0 + 2.0 ** -9, 65504.0,
                                                       np.float32(np.float16(6.0e-8)), -2.5]


def test_padding_lengths_inclusive_range():
    lens = np.concatenate([gen.fwd_inputs(64, 1, 1, 8, 1, "f16", s, causal=False,
                                          kv_len_range=(2, 4)).kv_lens for s in range(20)])
    assert set(lens.tolist()) == {2, 3, 4}


def test_decode_page_table_layout():
    inp = gen.decode_inputs(5, 2, 8, (1, 40), "f16", 3, page_size=4, num_pages=128)
    npg = gen.pages_per_seq(inp.kv_lens, 4)
    assert inp.page_table.shape == (5, 10)
    for s in range(5):
        assert np.all(inp.page_table[s, :npg[s]] >= 0)
        assert np.all(inp.page_table[s, npg[s]:] == -1)
    ident = gen.decode_inputs(5, 2, 8, (1, 40), "f16", 3, page_size=4, num_pages=128,
                              identity_pages=True)
    assert np.array_equal(ident.k, inp.k) and np.array_equal(ident.kv_lens, inp.kv_lens)
    flat = ident.page_table[ident.page_table >= 0]
    assert np.array_equal(flat, np.arange(flat.size))
