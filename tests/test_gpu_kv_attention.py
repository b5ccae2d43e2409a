"""GPU parity of nvfp4_kv_attention (fused attention over the NVFP4 pages)
against the oracle's window attention.

The oracle builds its own pool from the same seeded inputs (oracle write
path) and computes O in fp64.  Tolerance, from the device's arithmetic: the
logits and sums are fp32 (relative error ~1e-6 here), the softmax weights
enter the P V product rounded to bf16 (each within 2^-9 relative, so
|dO| <= 2^-9 sum_j w_j |V^_j|) and O is rounded once to bf16 (2^-9 |O|).  The
test allows four times the first term and twice the second:
    |O - O_ref| <= 2^-7 sum_j w_j |V^_j| + 2^-8 |O_ref| + 1e-30.
"""

import math

import numpy as np
import pytest
import torch

import synth
from helpers import bf16_tensor, dev
from oracle import formats as F
from oracle import kvcache as KV

pytestmark = pytest.mark.gpu

import w4a4_gemm_amd as nv  # noqa: E402


def _pair(h, p, max_pages, max_chunks, table, n_phys, d=128):
    gpu = nv.KVCache(1, h, d, p, max_pages, max_chunks, table, n_phys, device=dev())
    ora = KV.KVPool(1, h, d, p, max_pages, max_chunks, np.asarray(table), n_phys)
    return gpu, ora


def _write(gpu, ora, chunk, kb, vb, start):
    nv.nvfp4_kv_quantize(gpu, 0, chunk, bf16_tensor(kb), bf16_tensor(vb), start)
    ora.write_chunk(0, chunk, F.bf16_bits_to_f64(kb), F.bf16_bits_to_f64(vb), start)


def _check(gpu, ora, pages, last, qb, scale, n_phys):
    lp = torch.tensor(pages, dtype=torch.int32, device=dev())
    out = nv.nvfp4_kv_attention(gpu, 0, lp, last, bf16_tensor(qb), scale)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy().astype(np.float64)
    ref, wabs = KV.attention(ora, 0, pages, last, F.bf16_bits_to_f64(qb), scale, n_phys)
    bound = 2.0 ** -7 * wabs + 2.0 ** -8 * np.abs(ref) + 1e-30
    err = np.abs(o - ref)
    worst = float(np.max(err / bound))
    assert worst <= 1.0, f"worst error / bound = {worst}"
    return worst


def test_ragged_queries_partial_last_page():
    h, p = 3, 64
    table = np.random.default_rng(3).permutation(8).astype(np.int32)[None, :]
    gpu, ora = _pair(h, p, 8, 1, table, 8)
    kb, vb = synth.kv_chunk(t=300, h=h, d=128, seed_k=81, seed_v=82, seed_off=83)
    _write(gpu, ora, 0, kb, vb, 0)                          # pages 0..4, last holds 44 tokens
    qb = synth.attn_queries(200, h, 128, seed=84)           # 200 rows: two query blocks, ragged
    _check(gpu, ora, [0, 1, 2, 3, 4], 300 - 4 * p, qb, 1 / math.sqrt(128), 8)


def test_two_chunks_unmapped_page_and_order():
    h, p = 2, 128
    table = np.array([[5, 2, 7, 0, -1, 3, 1, 4]], dtype=np.int32)   # logical page 4 unmapped
    gpu, ora = _pair(h, p, 8, 2, table, 8)
    kb, vb = synth.kv_chunk(t=600, h=h, d=128, seed_k=85, seed_v=86, seed_off=87)
    _write(gpu, ora, 0, kb[:200], vb[:200], 0)              # chunk 0: pages 0, 1 (72 slots)
    _write(gpu, ora, 1, kb[200:500], vb[200:500], 200)      # chunk 1: rest of page 1, 2, 3 (116)
    qb = synth.attn_queries(130, h, 128, seed=88)
    # page 1 holds both chunks; page 4 is unmapped and contributes nothing
    _check(gpu, ora, [3, 1, 4, 0, 2], 128, qb, 0.09, 8)
    _check(gpu, ora, [1, 0, 3], 500 - 3 * p, qb, 0.09, 8)


def test_single_key_and_empty_window():
    h, p = 1, 64
    gpu, ora = _pair(h, p, 2, 1, np.array([[1, 0]], dtype=np.int32), 2)
    kb, vb = synth.kv_chunk(t=64, h=h, d=128, seed_k=89, seed_v=90, seed_off=91)
    _write(gpu, ora, 0, kb, vb, 0)
    qb = synth.attn_queries(5, h, 128, seed=92)
    _check(gpu, ora, [0], 1, qb, 0.5, 2)                    # one key: O = V^[0] up to rounding
    lp = torch.zeros(0, dtype=torch.int32, device=dev())
    out = nv.nvfp4_kv_attention(gpu, 0, lp, 0, bf16_tensor(qb), 0.5)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0            # no valid key -> 0


def test_large_logits_stay_finite():
    # sharp softmax: queries scaled up so logits reach a few hundred
    h, p = 2, 64
    gpu, ora = _pair(h, p, 4, 1, np.arange(4, dtype=np.int32)[None, :], 4)
    kb, vb = synth.kv_chunk(t=256, h=h, d=128, seed_k=93, seed_v=94, seed_off=95)
    _write(gpu, ora, 0, kb, vb, 0)
    qb = synth.attn_queries(64, h, 128, seed=96, std=8.0)
    _check(gpu, ora, [0, 1, 2, 3], 64, qb, 1 / math.sqrt(128), 4)


def test_dit_heads_window_of_the_written_chunk():
    # 24 heads x 128, 256-token pages: a 7040-token chunk and 160 of its queries
    h, p = 24, 256
    table = synth.page_permutation(28, 33)[None, :]
    gpu, ora = _pair(h, p, 28, 1, table, 28)
    kb, vb = synth.kv_chunk()
    _write(gpu, ora, 0, kb, vb, 0)
    qb = synth.attn_queries(160, h, 128, seed=97)
    _check(gpu, ora, list(range(28)), 7040 - 27 * p, qb, 1 / math.sqrt(128), 28)


def test_split_window_with_an_empty_split():
    # 20 blocks for a 1-block query grid: the window is split over workgroups,
    # and the first half of the listed pages is unmapped (that split sees no key)
    h, p = 2, 64
    table = np.array([[-1] * 10 + list(range(10))], dtype=np.int32)
    gpu, ora = _pair(h, p, 20, 1, table, 10)
    assert nv.nvfp4_workspace_bytes(nv.OP_KV_ATTENTION, 50, h, 20 * p) > 0
    kb, vb = synth.kv_chunk(t=10 * p, h=h, d=128, seed_k=98, seed_v=99, seed_off=100)
    _write(gpu, ora, 0, kb, vb, 10 * p)                     # logical pages 10..19
    qb = synth.attn_queries(50, h, 128, seed=101)
    _check(gpu, ora, list(range(20)), p, qb, 1 / math.sqrt(128), 10)


@pytest.mark.parametrize("scale", [-0.2, 0.0])
def test_negative_and_zero_scale(scale):
    # a negative scale prefers the keys least aligned with q; scale 0 averages V^
    h, p = 2, 64
    gpu, ora = _pair(h, p, 6, 1, np.array([[4, 1, 5, 0, 2, 3]], dtype=np.int32), 6)
    kb, vb = synth.kv_chunk(t=330, h=h, d=128, seed_k=102, seed_v=103, seed_off=104)
    _write(gpu, ora, 0, kb, vb, 0)
    qb = synth.attn_queries(40, h, 128, seed=105)
    _check(gpu, ora, [0, 1, 2, 3, 4, 5], 330 - 5 * p, qb, scale, 6)


@pytest.mark.slow
def test_long_context_window_full_size_sampled():
    """The measured launch: 880 queries x 24 heads over the 68-page window (4 sink
    pages + the last 16384 tokens) of a 65536-token layer in shuffled pages, split
    over workgroups and merged; sampled queries checked against the oracle."""
    r = synth.LongContextKV(n_layers=1)
    gpu = nv.KVCache(r.L, r.H, r.D, r.P, r.pages_per_layer, len(r.chunks), r.page_table,
                     r.n_phys, device=dev())
    ora = KV.KVPool(1, r.H, r.D, r.P, r.pages_per_layer, len(r.chunks),
                    np.arange(r.pages_per_layer)[None, :], r.pages_per_layer)
    window = r.window()
    win_tokens = set()
    for pg in window:
        win_tokens.update((pg * r.P, pg * r.P + r.P - 1))
    for c in range(len(r.chunks)):
        start, kb, vb = r.chunk(0, c)
        nv.nvfp4_kv_quantize(gpu, 0, c, bf16_tensor(kb), bf16_tensor(vb), start)
        # the oracle needs only the chunks that hold window pages
        if any(start <= t < start + len(kb) for t in win_tokens) or any(
                start <= pg * r.P < start + len(kb) for pg in window):
            ora.write_chunk(0, c, F.bf16_bits_to_f64(kb), F.bf16_bits_to_f64(vb), start)
        print(f"[attention full size] chunk {c} written", flush=True)
    assert nv.nvfp4_workspace_bytes(nv.OP_KV_ATTENTION, 880, r.H, len(window) * r.P) > 0
    qb = synth.attn_queries(880, r.H, r.D, seed=50)
    scale = 1 / math.sqrt(r.D)
    lp = torch.tensor(window, dtype=torch.int32, device=dev())
    out = nv.nvfp4_kv_attention(gpu, 0, lp, r.P, bf16_tensor(qb), scale)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy().astype(np.float64)
    rows = np.unique(np.concatenate([[0, 127, 128, 879],
                                     np.random.default_rng(106).choice(880, 20, replace=False)]))
    ref, wabs = KV.attention(ora, 0, window, r.P, F.bf16_bits_to_f64(qb[rows]), scale,
                             r.pages_per_layer)
    bound = 2.0 ** -7 * wabs + 2.0 ** -8 * np.abs(ref) + 1e-30
    assert float(np.max(np.abs(o[rows] - ref) / bound)) <= 1.0


def test_head_dim_64_two_chunks_ragged_queries():
    # head_dim 64: two chunks share page 1, logical page 7 (listed, never written)
    # is unmapped, the last listed page is partial and 200 queries leave the
    # second query block ragged
    h, p, d = 3, 64, 64
    table = np.array([[4, 0, 6, 2, 5, 1, 3, -1]], dtype=np.int32)
    gpu, ora = _pair(h, p, 8, 2, table, 8, d=d)
    kb, vb = synth.kv_chunk(t=400, h=h, d=d, seed_k=102, seed_v=103, seed_off=104)
    _write(gpu, ora, 0, kb[:100], vb[:100], 0)              # chunk 0: page 0, 36 slots of page 1
    _write(gpu, ora, 1, kb[100:400], vb[100:400], 100)      # chunk 1: rest of page 1 .. page 6
    qb = synth.attn_queries(200, h, d, seed=105)
    _check(gpu, ora, [0, 1, 2, 3, 7, 4, 5, 6], 400 - 6 * p, qb, 1 / math.sqrt(d), 8)
    _check(gpu, ora, [3, 1, 0], p, qb, 0.2, 8)


@pytest.mark.parametrize("d", [128, 64])
def test_many_splits_merge(d):
    # one query block of 2 heads over 160 shuffled pages: the window is split
    # more than 8 ways, so the merge reads its splits in several rounds after
    # a first pass for the maxima; a chunk boundary falls inside a block
    h, p, n_pages, n_q = 2, 64, 160, 40
    table = synth.page_permutation(n_pages, 111)[None, :]
    gpu, ora = _pair(h, p, n_pages, 2, table, n_pages, d=d)
    ws = nv.nvfp4_workspace_bytes(nv.OP_KV_ATTENTION, n_q, h, n_pages * p)
    splits = ws // (n_q * h * (128 + 2) * 4)
    assert splits > 8, splits
    kb, vb = synth.kv_chunk(t=n_pages * p, h=h, d=d, seed_k=112, seed_v=113, seed_off=114)
    cut = n_pages * p // 2 + 32
    _write(gpu, ora, 0, kb[:cut], vb[:cut], 0)
    _write(gpu, ora, 1, kb[cut:], vb[cut:], cut)
    qb = synth.attn_queries(n_q, h, d, seed=115)
    order = [int(x) for x in synth.page_permutation(n_pages, 116)]
    _check(gpu, ora, order, p, qb, 1 / math.sqrt(d), n_pages)


def test_v_scale_with_midpoint_products():
    # max|V| = 1.0390625: products q s_b s_gV round (in fp32) onto bf16
    # midpoints, so every page takes the V decode with the exact fix-up
    h, p = 2, 64
    table = np.arange(12, dtype=np.int32)[None, :]
    gpu, ora = _pair(h, p, 12, 1, table, 12)
    kb, vb = synth.kv_chunk(t=12 * p, h=h, d=128, seed_k=120, seed_v=121, seed_off=122)
    v = F.bf16_bits_to_f64(vb)
    v = v * 2.0 ** -int(np.ceil(np.log2(np.max(np.abs(v)) + 1e-30)))   # |v| <= 1, exact
    v.flat[5] = 1.0390625
    _write(gpu, ora, 0, kb, F.f64_to_bf16_bits(v), 0)
    qb = synth.attn_queries(70, h, 128, seed=123)
    _check(gpu, ora, list(range(12)), p, qb, 1 / math.sqrt(128), 12)


def test_head_dim_64_split_window():
    # a one-block query grid over 24 pages: the window is split over workgroups
    # and merged by the combine kernel (one channel per lane at head_dim 64)
    h, p, d = 2, 64, 64
    table = synth.page_permutation(24, 106)[None, :]
    gpu, ora = _pair(h, p, 24, 1, table, 24, d=d)
    assert nv.nvfp4_workspace_bytes(nv.OP_KV_ATTENTION, 40, h, 24 * p) > 0
    kb, vb = synth.kv_chunk(t=24 * p, h=h, d=d, seed_k=107, seed_v=108, seed_off=109)
    _write(gpu, ora, 0, kb, vb, 0)
    qb = synth.attn_queries(40, h, d, seed=110)
    _check(gpu, ora, list(range(24)), p, qb, 1 / math.sqrt(d), 24)


def test_pages_beyond_4gib():
    """A 4.4 GB pool (5000 pages of 24 heads x 256 tokens, 885 KB each) whose listed
    pages lie past 2^31 and 2^32 bytes, two of them straddling those offsets: the
    written bytes and the window read are bit-exact and the attention is within the
    tolerance.  The oracle keeps a small pool of its own: where a page is placed
    changes no value."""
    h, d, p = 24, 128, 256
    n_phys = 5000
    gtab = np.array([[4999, 2427, 4860, 0, 4998, 4854]], dtype=np.int32)
    gpu = nv.KVCache(1, h, d, p, 6, 2, gtab, n_phys, device=dev())
    ora = KV.KVPool(1, h, d, p, 6, 2, np.arange(6, dtype=np.int32)[None, :], 6)
    pb = gpu.page_bytes
    assert 2427 * pb < 2 ** 31 < 2428 * pb and 4854 * pb < 2 ** 32 < 4855 * pb
    kb, vb = synth.kv_chunk(t=1400, h=h, d=d, seed_k=124, seed_v=125, seed_off=126)
    _write(gpu, ora, 0, kb[:700], vb[:700], 0)
    _write(gpu, ora, 1, kb[700:], vb[700:], 700)              # pages 2 (from slot 188) .. 5
    torch.cuda.synchronize()
    for lp in range(6):
        g = gpu.pool[int(gtab[0, lp])].cpu().numpy()
        assert np.array_equal(g, ora.pool[lp]), f"page {lp}: {np.sum(g != ora.pool[lp])} bytes"
    pages = [3, 5, 0, 4, 1, 2]
    lp = torch.tensor(pages, dtype=torch.int32, device=dev())
    kh, vh = nv.nvfp4_kv_dequant_blocks(gpu, 0, lp)
    torch.cuda.synchronize()
    ko, vo = ora.dequant_pages(0, pages)
    assert np.array_equal(kh.float().cpu().numpy().astype(np.float64), ko)
    assert np.array_equal(vh.float().cpu().numpy().astype(np.float64), vo)
    qb = synth.attn_queries(300, h, d, seed=127)
    order = [0, 1, 2, 3, 4, 5]
    _check(gpu, ora, order, 1400 - 5 * p, qb, 1 / math.sqrt(d), 6)


def test_seeded_config_sweep():
    """12 seeded caches: 1-6 heads, head_dim 64 or 128, pages of 64, 128 or 256 tokens,
    1-3 chunks of random lengths (every chunk after the first at least a page) in a
    shuffled table with spare physical pages.  Pool bytes, means, scales and page->chunk
    entries and a window read in random page order are bit-exact; the attention over
    the window (random query count) is within the tolerance."""
    rng = np.random.default_rng(79)
    for i in range(12):
        h, d, p = int(rng.integers(1, 7)), int(rng.choice([64, 128])), int(rng.choice([64, 128, 256]))
        n_chunks = int(rng.integers(1, 4))
        lens = [int(rng.integers(1, 3 * p))] + [int(rng.integers(p, 3 * p)) for _ in range(n_chunks - 1)]
        total = sum(lens)
        n_pages = -(-total // p)
        n_phys = n_pages + int(rng.integers(0, 4))
        table = rng.permutation(n_phys)[:n_pages].astype(np.int32)[None, :]
        n_q = int(rng.integers(1, 601))
        print(f"[sweep {i}] heads {h} head_dim {d} page {p} chunks {lens} queries {n_q}", flush=True)
        gpu, ora = _pair(h, p, n_pages, n_chunks, table, n_phys, d=d)
        kb, vb = synth.kv_chunk(t=total, h=h, d=d, seed_k=200 + i, seed_v=300 + i, seed_off=400 + i)
        start = 0
        for c, n in enumerate(lens):
            _write(gpu, ora, c, kb[start:start + n], vb[start:start + n], start)
            start += n
        torch.cuda.synchronize()
        for lp in range(n_pages):
            g = gpu.pool[int(table[0, lp])].cpu().numpy()
            assert np.array_equal(g, ora.pool[int(table[0, lp])]), (i, lp)
        for name in ("k_mean", "k_gscale", "v_gscale", "page_chunk"):
            assert np.array_equal(getattr(gpu, name)[0].cpu().numpy(), getattr(ora, name)[0]), (i, name)
        order = [int(x) for x in rng.permutation(n_pages)]
        lp = torch.tensor(order, dtype=torch.int32, device=dev())
        kh, vh = nv.nvfp4_kv_dequant_blocks(gpu, 0, lp)
        torch.cuda.synchronize()
        ko, vo = ora.dequant_pages(0, order)
        assert np.array_equal(kh.float().cpu().numpy().astype(np.float64), ko), i
        assert np.array_equal(vh.float().cpu().numpy().astype(np.float64), vo), i
        window = [x for x in order if x != n_pages - 1] + [n_pages - 1]
        qb = synth.attn_queries(n_q, h, d, seed=500 + i)
        _check(gpu, ora, window, total - (n_pages - 1) * p, qb, 1 / math.sqrt(d), n_phys)
