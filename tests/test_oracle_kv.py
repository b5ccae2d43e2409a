"""Pins of the oracle's NVFP4 KV cache (CPU only)."""

from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import formats as F
from oracle import kvcache as KV
from oracle import nvfp4 as Q


def _bf16(x):
    return F.bf16_bits_to_f64(synth.to_bf16_bits(np.asarray(x, np.float32)))


def test_exact_mean_matches_fractions():
    rng = np.random.default_rng(0)
    k = _bf16(rng.standard_normal((37, 3, 16)) * np.exp2(rng.integers(-30, 12, (37, 3, 16))))
    mu = KV.chunk_mean(k)
    for h in range(3):
        for d in range(16):
            s = sum(Fraction(float(v)) for v in k[:, h, d])
            assert mu[h, d] == F.round_fraction_to_binary(s / 37, F.F32)
    c = KV.ChunkQ(k, k)
    for t in range(0, 37, 6):
        for h in range(3):
            for d in range(16):
                want = F.round_fraction_to_binary(Fraction(float(k[t, h, d])) - Fraction(float(mu[h, d])), F.F32)
                assert c.kp[t, h, d] == want


def test_constant_chunk_mean_and_zero_codes():
    k = np.full((40, 2, 32), 3.25)
    v = _bf16(np.random.default_rng(1).standard_normal((40, 2, 32)))
    c = KV.ChunkQ(k, v)
    assert np.all(c.mu == 3.25)
    assert np.all(c.kp == 0.0) and not np.any(np.signbit(c.kp))
    assert c.s_gk == 1.0 and np.all(c.k_codes == 0) and np.all(c.k_scales == 0)


def test_known_offset_is_recovered_exactly():
    # K = off + (+e, -e) pairs: the exact mean is off, and K' = +-e
    off = np.random.default_rng(2).integers(-32, 33, (2, 16)) / 4.0
    e = np.array([0.5, -0.5] * 10)[:, None, None]
    k = off[None] + e * np.ones((20, 2, 16))
    assert np.array_equal(_bf16(k), k)
    assert np.array_equal(KV.chunk_mean(k), off)


def test_mean_subtraction_centres_each_channel():
    kb, _ = synth.kv_chunk(t=300, h=2, d=32)
    k = F.bf16_bits_to_f64(kb)
    c = KV.ChunkQ(k, k)
    # |sum_t K'| is at most T * (half ulp of mu + half ulp of K') -- tiny next to sum |K'|
    s = np.abs(np.sum(c.kp, axis=0))
    assert np.all(s <= 1e-3 * np.sum(np.abs(c.kp), axis=0))


def _small_pool(rng, layers=2, pages=6, chunks=3, h=2, d=32, p=16):
    n_phys = layers * pages
    table = rng.permutation(n_phys).reshape(layers, pages)
    return KV.KVPool(layers, h, d, p, pages, chunks, table, n_phys)


def test_page_chunk_metadata_for_straddling_writes():
    rng = np.random.default_rng(3)
    pool = _small_pool(rng)
    kb, vb = synth.kv_chunk(t=40, h=2, d=32, seed_k=5, seed_v=6, seed_off=7)
    k, v = F.bf16_bits_to_f64(kb), F.bf16_bits_to_f64(vb)
    pool.write_chunk(1, 0, k[:24], v[:24], 0)        # tokens 0..23: pages 0, 1 (half)
    pool.write_chunk(1, 1, k[24:], v[24:], 24)       # tokens 24..39: page 1 (rest), 2
    assert pool.page_chunk[1, 0].tolist() == [0, 16]
    assert pool.page_chunk[1, 1].tolist() == [0, 8]  # slots 0..7 chunk 0, 8..15 chunk 1
    assert pool.page_chunk[1, 2].tolist() == [1, 16]


def test_page_chunk_metadata_does_not_depend_on_stale_entries():
    # a chunk starting inside a page records the page's earlier slots as the
    # previous chunk's, whatever the table held before; chunk 0 cannot start
    # inside a page (its earlier slots would belong to no chunk)
    rng = np.random.default_rng(3)
    pool = _small_pool(rng)
    pool.page_chunk[0] = 2                           # stale entries from an earlier use
    kb, vb = synth.kv_chunk(t=40, h=2, d=32, seed_k=5, seed_v=6, seed_off=7)
    k, v = F.bf16_bits_to_f64(kb), F.bf16_bits_to_f64(vb)
    pool.write_chunk(0, 0, k[:24], v[:24], 0)
    pool.write_chunk(0, 1, k[24:], v[24:], 24)
    assert pool.page_chunk[0, :3].tolist() == [[0, 16], [0, 8], [1, 16]]
    with pytest.raises(ValueError):
        pool.write_chunk(1, 0, k[:24], v[:24], 5)


def test_dequant_matches_fraction_brute_force_and_is_shuffle_invariant():
    rng = np.random.default_rng(4)
    pool = _small_pool(rng, p=16)
    kb, vb = synth.kv_chunk(t=40, h=2, d=32, seed_k=8, seed_v=9, seed_off=10)
    k, v = F.bf16_bits_to_f64(kb), F.bf16_bits_to_f64(vb)
    c0 = pool.write_chunk(0, 0, k[:24], v[:24], 0)
    c1 = pool.write_chunk(0, 1, k[24:], v[24:], 24)
    pages = [2, 0, 1]
    kh, vh = pool.dequant_pages(0, pages)
    # brute force per element from the chunk objects (token-indexed, independent of paging)
    for out_i, lp in enumerate(pages):
        for slot in range(16):
            tok = lp * 16 + slot
            if tok >= 40:
                continue
            c, i = (c0, tok) if tok < 24 else (c1, tok - 24)
            for hh in range(2):
                for dd in range(0, 32, 5):
                    code = c.k_codes[i, hh, dd // 2]
                    code = code & 0xF if dd % 2 == 0 else code >> 4
                    q = Fraction(F.e2m1_decode(code))
                    sb = Fraction(F.e4m3_decode(c.k_scales[i, hh, dd // 16]))
                    exact = q * sb * Fraction(c.s_gk) + Fraction(c.mu[hh, dd])
                    assert kh[out_i * 16 + slot, hh, dd] == F.round_fraction_to_binary(exact, F.BF16)
                    code = c.v_codes[i, hh, dd // 2]
                    code = code & 0xF if dd % 2 == 0 else code >> 4
                    exact = Fraction(F.e2m1_decode(code)) * Fraction(F.e4m3_decode(c.v_scales[i, hh, dd // 16])) \
                        * Fraction(c.s_gv)
                    assert vh[out_i * 16 + slot, hh, dd] == F.round_fraction_to_binary(exact, F.BF16)
    # a different physical placement gives the same window
    pool2 = _small_pool(np.random.default_rng(99), p=16)
    pool2.write_chunk(0, 0, k[:24], v[:24], 0)
    pool2.write_chunk(0, 1, k[24:], v[24:], 24)
    kh2, vh2 = pool2.dequant_pages(0, pages)
    assert np.array_equal(kh, kh2) and np.array_equal(vh, vh2)
    # the window equals the matching slices of the whole-cache dequant
    ka, va = pool.dequant_pages(0, [0, 1, 2])
    assert np.array_equal(kh[16:32], ka[:16]) and np.array_equal(vh[:16], va[32:48])


def test_round_trip_error_bound():
    kb, vb = synth.kv_chunk(t=64, h=2, d=32)
    k, v = F.bf16_bits_to_f64(kb), F.bf16_bits_to_f64(vb)
    pool = _small_pool(np.random.default_rng(5), pages=4, p=16)
    c = pool.write_chunk(0, 0, k, v, 0)
    kh, vh = pool.dequant_pages(0, [0, 1, 2, 3])
    # |K^ - K| <= half the largest E2M1 gap (1.0) * s_b * s_g + bf16/fp32 rounding slack
    sbk = np.repeat(F.E4M3_GRID[c.k_scales], 16, axis=-1) * c.s_gk
    assert np.all(np.abs(kh - k) <= 1.0 * sbk + np.abs(k) * 2.0 ** -8 + 1e-6)
    sbv = np.repeat(F.E4M3_GRID[c.v_scales], 16, axis=-1) * c.s_gv
    assert np.all(np.abs(vh - v) <= 1.0 * sbv + np.abs(v) * 2.0 ** -8)


def test_page_bytes_and_compression_ratio():
    pool = KV.KVPool(1, 24, 128, 256, 1, 1, [0], 1)
    assert pool.page_bytes == 884736
    bf16_bytes = 2 * 24 * 256 * 128 * 2
    assert abs(bf16_bytes / pool.page_bytes - 3.6) < 0.05
