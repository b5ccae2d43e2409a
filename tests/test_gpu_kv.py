"""GPU parity of nvfp4_kv_quantize / nvfp4_kv_dequant_blocks against the oracle.

Bit-exact: the pool bytes (codes and scale bytes of every written slot), the
K means, the per-chunk global scales, the page->chunk table and every
dequantized bf16 value.
"""

import numpy as np
import pytest
import torch

import synth
from helpers import bf16_tensor, dev
from oracle import formats as F
from oracle import kvcache as KV

pytestmark = pytest.mark.gpu

import w4a4_gemm_amd as nv  # noqa: E402


def _pair(n_layers, h, d, p, max_pages, max_chunks, table, n_phys):
    gpu = nv.KVCache(n_layers, h, d, p, max_pages, max_chunks, table, n_phys, device=dev())
    ora = KV.KVPool(n_layers, h, d, p, max_pages, max_chunks, np.asarray(table), n_phys)
    return gpu, ora


def _write(gpu, ora, layer, chunk, kb, vb, start):
    nv.nvfp4_kv_quantize(gpu, layer, chunk, bf16_tensor(kb), bf16_tensor(vb), start)
    ora.write_chunk(layer, chunk, F.bf16_bits_to_f64(kb), F.bf16_bits_to_f64(vb), start)


def _compare_state(gpu, ora, layer, chunks, pages):
    torch.cuda.synchronize()
    assert np.array_equal(gpu.k_mean[layer, chunks].cpu().numpy(), ora.k_mean[layer, chunks])
    assert np.array_equal(gpu.k_gscale[layer, chunks].cpu().numpy(), ora.k_gscale[layer, chunks])
    assert np.array_equal(gpu.v_gscale[layer, chunks].cpu().numpy(), ora.v_gscale[layer, chunks])
    assert np.array_equal(gpu.page_chunk[layer, pages].cpu().numpy(), ora.page_chunk[layer, pages])
    gpt = gpu.page_table.cpu().numpy()
    for lp in pages:
        g = gpu.pool[int(gpt[layer, lp])].cpu().numpy()
        o = ora.pool[int(ora.page_table[layer, lp])]
        bad = np.nonzero(g != o)[0]
        assert bad.size == 0, f"page {lp}: {bad.size} bytes differ, first at {bad[:4]}"


def _compare_dequant(gpu, ora, layer, pages):
    lp = torch.tensor(pages, dtype=torch.int32, device=dev())
    kh, vh = nv.nvfp4_kv_dequant_blocks(gpu, layer, lp)
    torch.cuda.synchronize()
    ko, vo = ora.dequant_pages(layer, pages)
    kg = kh.float().cpu().numpy().astype(np.float64)
    vg = vh.float().cpu().numpy().astype(np.float64)
    assert np.array_equal(kg, ko), f"K^: {np.sum(kg != ko)} values differ"
    assert np.array_equal(vg, vo), f"V^: {np.sum(vg != vo)} values differ"


def test_two_chunks_straddling_a_page():
    h, d, p = 4, 128, 256
    table = np.random.default_rng(1).permutation(10).astype(np.int32)[None, :]
    gpu, ora = _pair(1, h, d, p, 10, 3, table, 10)
    kb, vb = synth.kv_chunk(t=1100, h=h, d=d, seed_k=3, seed_v=4, seed_off=5)
    _write(gpu, ora, 0, 0, kb[:600], vb[:600], 0)          # pages 0, 1, 2 (first 88 slots)
    _write(gpu, ora, 0, 1, kb[600:], vb[600:], 600)        # page 2 (rest), 3, 4 (part)
    _compare_state(gpu, ora, 0, [0, 1], list(range(5)))
    _compare_dequant(gpu, ora, 0, [2, 0, 4, 2, 1, 3])


@pytest.mark.parametrize("d", [64, 80, 256])
def test_other_head_dims(d):
    h, p = 3, 64
    table = np.arange(8, dtype=np.int32)[::-1].copy()[None, :]
    gpu, ora = _pair(1, h, d, p, 8, 2, table, 8)
    kb, vb = synth.kv_chunk(t=300, h=h, d=d, seed_k=6, seed_v=7, seed_off=8)
    _write(gpu, ora, 0, 0, kb[:150], vb[:150], 0)
    _write(gpu, ora, 0, 1, kb[150:], vb[150:], 150)
    _compare_state(gpu, ora, 0, [0, 1], list(range(5)))
    _compare_dequant(gpu, ora, 0, [4, 1, 0])


def test_constant_chunk_and_layers():
    # a constant K chunk (mean exact, K' = 0, s_gK = 1) in layer 1 of a 2-layer cache
    h, d, p = 2, 128, 128
    table = np.random.default_rng(2).permutation(8).astype(np.int32).reshape(2, 4)
    gpu, ora = _pair(2, h, d, p, 4, 1, table, 8)
    kb = synth.to_bf16_bits(np.full((256, h, d), 2.75, np.float32))
    _, vb = synth.kv_chunk(t=256, h=h, d=d)
    _write(gpu, ora, 1, 0, kb, vb, 0)
    _compare_state(gpu, ora, 1, [0], [0, 1])
    _compare_dequant(gpu, ora, 1, [1, 0])
    assert float(gpu.k_gscale[1, 0].cpu()) == 1.0


def test_k_mean_exact_over_wide_ranges():
    """K means of channels whose values span more binades than an fp64 sum keeps:
    the stats pass flags them and the finalize sums them exactly as integers
    (design reading 18).  Head 0 channel 0 mixes +-2^50 and 2^-50, 2^-60 values;
    channel 1 alternates +-2^100 (they cancel) with tiny values between, so its
    mean comes from the tiny ones alone; head 1 channel 5 mixes +-1 with a bf16
    subnormal, so its mean is an fp32 subnormal."""
    h, d, p, t = 2, 64, 64, 300
    table = np.arange(5, dtype=np.int32)[None, :]
    gpu, ora = _pair(1, h, d, p, 5, 1, table, 5)
    kb, vb = synth.kv_chunk(t=t, h=h, d=d, seed_k=11, seed_v=12, seed_off=13)
    k = synth.bf16_bits_to_f32(kb).astype(np.float64).reshape(t, h, d)
    rng = np.random.default_rng(14)
    k[:, 0, 0] = rng.choice([1.5 * 2.0 ** 50, -1.25 * 2.0 ** 50, 1.125 * 2.0 ** -50,
                             -1.75 * 2.0 ** -60], size=t)
    k[:, 0, 1] = np.where(np.arange(t) % 2 == 0, 2.0 ** 100, -(2.0 ** 100))
    k[10:20, 0, 1] = np.array([1, 3, 5, 7, 9, 11, 13, 15, 17, 19]) * 2.0 ** -100
    k[:, 1, 5] = np.where(np.arange(t) % 2 == 0, 1.0, -1.0)
    k[100:104, 1, 5] = 2.0 ** -130                        # bf16 subnormals
    kb2 = synth.to_bf16_bits(k.astype(np.float32)).reshape(kb.shape)
    assert np.array_equal(synth.bf16_bits_to_f32(kb2).astype(np.float64).reshape(t, h, d), k)
    # an fp64 running sum in token order loses the small terms of channel 1
    import math
    assert sum(k[:, 0, 1]) != math.fsum(k[:, 0, 1])
    _write(gpu, ora, 0, 0, kb2, vb, 0)
    _compare_state(gpu, ora, 0, [0], list(range(5)))
    _compare_dequant(gpu, ora, 0, [0, 3, 4])
    mu = gpu.k_mean[0, 0].cpu().numpy().reshape(h, d)
    assert mu[0, 1] != 0.0 and abs(mu[0, 1]) < 2.0 ** -90
    assert 0.0 < mu[1, 5] < 2.0 ** -126                    # an fp32 subnormal


def test_k_mean_exact_full_chunk_with_tiny_values():
    """The step's 7040-token chunk with three lone tiny K values (2^-40, -2^-35 and a bf16
    subnormal) among values near 1-10: those channels fail the fp64 exactness test, so
    their means come from the wave-wide integer sum; every mean, scale and page byte must
    still match the oracle bit for bit."""
    h, d, p = synth.KV_HEADS, synth.KV_HEAD_DIM, synth.KV_PAGE
    table = synth.page_permutation(28, 33)[None, :]
    gpu, ora = _pair(1, h, d, p, 28, 1, table, 28)
    kb, vb = synth.kv_chunk()
    k = synth.bf16_bits_to_f32(kb)
    k[123, 5, 17] = 2.0 ** -40
    k[4000, 20, 100] = -(2.0 ** -35)
    k[77, 0, 0] = 2.0 ** -130
    kb2 = synth.to_bf16_bits(k)
    # the channels the finalize must take the exact path for (its test, on the host)
    t = kb2.shape[0]
    mag = (kb2.reshape(t, -1).astype(np.uint32) << 16) & 0x7FFFFFFF
    emax = (mag.max(axis=0) >> 23).astype(np.int64)
    emin = (np.where(mag == 0, 0xFFFFFFFF, mag).min(axis=0) >> 23).astype(np.int64)
    flagged = np.nonzero(emax - np.maximum(emin, 1) + int(np.ceil(np.log2(t))) > 45)[0]
    assert {5 * d + 17, 20 * d + 100, 0} <= set(flagged.tolist())
    _write(gpu, ora, 0, 0, kb2, vb, 0)
    _compare_state(gpu, ora, 0, [0], list(range(28)))
    _compare_dequant(gpu, ora, 0, [0, 5, 27])


def _midpoint_significands(g):
    """How many of the 16 significands a of q s_b ({1, 1.5} x (1 + m/8)) give
    RN32(a g) exactly on a bf16 midpoint while a g itself is not (fp64 holds
    a g exactly): for such a scale the V^ decode needs its exact fix-up."""
    g = np.float32(g)
    n = 0
    for i in range(16):
        a = (1.5 if i & 8 else 1.0) * (1.0 + (i & 7) * 0.125)
        pf = np.float32(np.float64(a) * np.float64(g))
        if (int(pf.view(np.uint32)) & 0xFFFF) == 0x8000 and np.float64(pf) != a * np.float64(g):
            n += 1
    return n


def test_v_products_on_bf16_midpoints():
    # max|V| = 1.0390625 gives s_gV = RN32(1.0390625 / 2688), for which some
    # products q s_b s_gV round (in fp32) onto a bf16 midpoint: the window read
    # must still give V^ = RN_bf16(q s_b s_gV) with one rounding
    h, d, p = 2, 128, 64
    table = np.arange(12, dtype=np.int32)[None, :]
    gpu, ora = _pair(1, h, d, p, 12, 1, table, 12)
    kb, vb = synth.kv_chunk(t=12 * p, h=h, d=d, seed_k=120, seed_v=121, seed_off=122)
    v = F.bf16_bits_to_f64(vb)
    v = v * 2.0 ** -int(np.ceil(np.log2(np.max(np.abs(v)) + 1e-30)))   # |v| <= 1, exact
    v.flat[5] = 1.0390625
    _write(gpu, ora, 0, 0, kb, F.f64_to_bf16_bits(v), 0)
    _compare_state(gpu, ora, 0, [0], list(range(12)))
    sgv = float(ora.v_gscale[0, 0])
    assert _midpoint_significands(sgv) > 0, sgv
    _compare_dequant(gpu, ora, 0, list(range(12)))
    _compare_dequant(gpu, ora, 0, [11, 3, 0, 7])


def test_invalid_listed_pages_give_zeros():
    h, d, p = 2, 64, 32
    gpu, ora = _pair(1, h, d, p, 4, 1, np.array([[0, 1, 2, 3]], np.int32), 4)
    kb, vb = synth.kv_chunk(t=64, h=h, d=d)
    _write(gpu, ora, 0, 0, kb, vb, 0)
    lp = torch.tensor([0, 7, -1], dtype=torch.int32, device=dev())
    kh, vh = nv.nvfp4_kv_dequant_blocks(gpu, 0, lp)
    torch.cuda.synchronize()
    assert torch.count_nonzero(kh[p:]) == 0 and torch.count_nonzero(vh[p:]) == 0


def test_kv_write_full_chunk():
    """One layer's new chunk at full size: 7040 tokens x 24 heads x 128, 256-token
    pages from a shuffled table (28 pages, the last one half full)."""
    h, d, p = synth.KV_HEADS, synth.KV_HEAD_DIM, synth.KV_PAGE
    table = synth.page_permutation(28, 33)[None, :]
    gpu, ora = _pair(1, h, d, p, 28, 1, table, 28)
    kb, vb = synth.kv_chunk()
    _write(gpu, ora, 0, 0, kb, vb, 0)
    _compare_state(gpu, ora, 0, [0], list(range(28)))
    _compare_dequant(gpu, ora, 0, [27, 0, 13])


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_long_context_window_sampled():
    """30 layers x 65536 tokens in shuffled 256-token pages; the attention window
    (4 sink pages + the most recent 16384 tokens) of every layer is dequantized in
    one launch per layer.  One layer is checked in full against an oracle cache
    built from the same chunks; every layer's window is checked by properties."""
    r = synth.LongContextKV()
    gpu = nv.KVCache(r.L, r.H, r.D, r.P, r.pages_per_layer, len(r.chunks), r.page_table,
                     r.n_phys, device=dev())
    for layer in range(r.L):
        for c in range(len(r.chunks)):
            start, kb, vb = r.chunk(layer, c)
            nv.nvfp4_kv_quantize(gpu, layer, c, bf16_tensor(kb), bf16_tensor(vb), start)
        print(f"[long-context] layer {layer} written", flush=True)
    window = r.window()
    lp = torch.tensor(window, dtype=torch.int32, device=dev())
    check = 17
    ora = KV.KVPool(1, r.H, r.D, r.P, r.pages_per_layer, len(r.chunks),
                    np.arange(r.pages_per_layer)[None, :], r.pages_per_layer)
    for c in range(len(r.chunks)):
        start, kb, vb = r.chunk(check, c)
        ora.write_chunk(0, c, F.bf16_bits_to_f64(kb), F.bf16_bits_to_f64(vb), start)
        print(f"[long-context] oracle chunk {c} of layer {check}", flush=True)
    kh, vh = nv.nvfp4_kv_dequant_blocks(gpu, check, lp)
    torch.cuda.synchronize()
    ko, vo = ora.dequant_pages(0, window)
    assert np.array_equal(kh.float().cpu().numpy().astype(np.float64), ko)
    assert np.array_equal(vh.float().cpu().numpy().astype(np.float64), vo)
    assert np.array_equal(gpu.k_mean[check].cpu().numpy(), ora.k_mean[0])
    # every layer: finite output, V^ within the format's error of V for a sink page
    for layer in range(r.L):
        kh, vh = nv.nvfp4_kv_dequant_blocks(gpu, layer, lp)
        assert torch.isfinite(kh.float()).all() and torch.isfinite(vh.float()).all()
        _, kb, vb = r.chunk(layer, 0)
        v0 = torch.from_numpy(F.bf16_bits_to_f64(vb[:r.P]).astype(np.float32))
        err = (vh[:r.P].float().cpu() - v0).abs().max().item()
        sgv = float(gpu.v_gscale[layer, 0].cpu())
        assert err <= 448 * sgv * 1.05          # one E2M1 step of the largest scale + bf16
