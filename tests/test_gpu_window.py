"""GPU parity of nvfp4_kv_window_pages against the oracle's page-list reading
(bit-exact: the list, its length and the last page's valid tokens)."""

import numpy as np
import pytest
import torch

from oracle.window import window_pages

pytestmark = pytest.mark.gpu

import w4a4_gemm_amd as nv  # noqa: E402


def test_long_context_window():
    pages, last = nv.nvfp4_kv_window_pages(65536, 256, 1024, 0, 0, 16384)
    ref, ref_last = window_pages(65536, 256, 1024, 0, 0, 16384)
    assert pages.cpu().tolist() == ref and last == ref_last


def test_random_windows():
    rng = np.random.default_rng(11)
    buf = torch.full((4096,), -7, dtype=torch.int32, device="cuda")
    for _ in range(300):
        P = int(rng.choice([64, 128, 256]))
        T = int(rng.integers(0, 200000))
        G, s0, S, W = (int(v) for v in rng.integers(0, 60000, size=4))
        ref, ref_last = window_pages(T, P, G, s0, S, W)
        if len(ref) > buf.numel():
            continue
        pages, last = nv.nvfp4_kv_window_pages(T, P, G, s0, S, W, pages=buf)
        assert pages.cpu().tolist() == ref and last == ref_last, (T, P, G, s0, S, W)


def test_shot_change_rebinds_only_the_shot_sink():
    # two shots: the shot sink moves from 0 to 40000; the global sink and window stay
    a, _ = nv.nvfp4_kv_window_pages(60000, 256, 1024, 0, 1760, 8192)
    b, _ = nv.nvfp4_kv_window_pages(60000, 256, 1024, 40000, 1760, 8192)
    sa, sb = set(a.cpu().tolist()), set(b.cpu().tolist())
    assert set(window_pages(60000, 256, 1024, 0, 0, 8192)[0]) <= sa & sb
    assert sb - sa == set(range(40000 // 256, -(-41760 // 256)))


def test_window_list_feeds_attention():
    """The device list goes straight into nvfp4_kv_attention (no host round trip);
    the result matches the oracle's attention over the oracle's list."""
    import math

    import synth
    from helpers import bf16_tensor, dev
    from oracle import formats as F
    from oracle import kvcache as KV

    h, p, n_pages = 2, 64, 24
    table = np.random.default_rng(5).permutation(n_pages).astype(np.int32)[None, :]
    gpu = nv.KVCache(1, h, 128, p, n_pages, 1, table, n_pages, device=dev())
    ora = KV.KVPool(1, h, 128, p, n_pages, 1, np.asarray(table), n_pages)
    T = 1500
    kb, vb = synth.kv_chunk(t=T, h=h, d=128, seed_k=95, seed_v=96, seed_off=97)
    nv.nvfp4_kv_quantize(gpu, 0, 0, bf16_tensor(kb), bf16_tensor(vb), 0)
    ora.write_chunk(0, 0, F.bf16_bits_to_f64(kb), F.bf16_bits_to_f64(vb), 0)
    # global sink 100, shot sink [700, 790), window 300: pages 0-1, 10-12, 18-23
    pages, last = nv.nvfp4_kv_window_pages(T, p, 100, 700, 90, 300)
    ref_pages, ref_last = window_pages(T, p, 100, 700, 90, 300)
    assert pages.cpu().tolist() == ref_pages and last == ref_last
    qb = synth.attn_queries(70, h, 128, seed=98)
    scale = 1 / math.sqrt(128)
    out = nv.nvfp4_kv_attention(gpu, 0, pages, last, bf16_tensor(qb), scale)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy().astype(np.float64)
    ref, wabs = KV.attention(ora, 0, ref_pages, ref_last, F.bf16_bits_to_f64(qb), scale, n_pages)
    # bound of the attention parity tests (bf16 weights into P V, one bf16 rounding of O)
    bound = 2.0 ** -7 * wabs + 2.0 ** -8 * np.abs(ref) + 1e-30
    assert float(np.max(np.abs(o - ref) / bound)) <= 1.0
