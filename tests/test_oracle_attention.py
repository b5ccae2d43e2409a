"""Pins of the oracle's window attention (CPU, no GPU).

The oracle defines O = softmax(scale q K^T) V over the valid keys of a listed
window of the paged NVFP4 cache (oracle/kvcache.py, attention).  It is pinned
to torch's float64 scaled-dot-product attention on the same K^, V^ (a
library routine of the same definition), to closed forms (one key, equal
logits, two keys), and to invariances (page order, masking = truncation,
unmapped pages contribute nothing).
"""

import math

import numpy as np
import pytest
import torch

import synth
from oracle import formats as F
from oracle import kvcache as KV

pytestmark = pytest.mark.filterwarnings("ignore")

H, D, P = 2, 128, 64


def _pool(tokens=150, n_pages=4, seed=0):
    kb, vb = synth.kv_chunk(t=tokens, h=H, d=D, seed_k=70 + seed, seed_v=71 + seed, seed_off=72 + seed)
    table = np.arange(n_pages)[None, :]
    pool = KV.KVPool(1, H, D, P, n_pages, 1, table, n_pages)
    pool.write_chunk(0, 0, F.bf16_bits_to_f64(kb), F.bf16_bits_to_f64(vb), 0)
    return pool


def _q(n_q, seed=5):
    return F.bf16_bits_to_f64(synth.attn_queries(n_q, H, D, seed=seed))


def test_matches_torch_sdpa_float64():
    pool = _pool()
    q = _q(7)
    pages, last = [0, 1, 2], 150 - 2 * P
    scale = 1.0 / math.sqrt(D)
    out, _ = KV.attention(pool, 0, pages, last, q, scale)
    k, v, mask = KV.window_keys(pool, 0, pages, last, 4)
    kt = torch.from_numpy(k[mask]).permute(1, 0, 2)[None]      # [1, H, n, D]
    vt = torch.from_numpy(v[mask]).permute(1, 0, 2)[None]
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
    ref = ref[0].permute(1, 0, 2).numpy()
    assert np.max(np.abs(out - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_single_key_returns_its_value():
    pool = _pool()
    q = _q(3)
    out, _ = KV.attention(pool, 0, [0], 1, q, 0.3)
    _, v = pool.dequant_pages(0, [0])
    assert np.array_equal(out, np.broadcast_to(v[0], out.shape))


def test_equal_logits_average_the_values():
    pool = _pool()
    q = np.zeros((2, H, D))                       # every logit 0
    out, _ = KV.attention(pool, 0, [0, 1], 40, q, 1.0)
    _, v = pool.dequant_pages(0, [0, 1])
    keep = np.r_[np.arange(P), P + np.arange(40)]
    assert np.max(np.abs(out - v[keep].mean(axis=0)[None])) <= 1e-14 * np.max(np.abs(v))


def test_two_keys_logistic_weights():
    pool = _pool()
    q = _q(4)
    scale = 0.125
    out, _ = KV.attention(pool, 0, [0], 2, q, scale)
    k, v = pool.dequant_pages(0, [0])
    for h in range(H):
        d = scale * (q[:, h] @ (k[1, h] - k[0, h]))            # logit difference
        w1 = 1.0 / (1.0 + np.exp(-d))
        ref = (1 - w1)[:, None] * v[0, h][None] + w1[:, None] * v[1, h][None]
        assert np.max(np.abs(out[:, h] - ref)) <= 1e-13 * np.max(np.abs(v))


def test_page_order_and_unmapped_pages():
    pool = _pool(tokens=4 * P, n_pages=4, seed=1)
    q = _q(5, seed=9)
    a, _ = KV.attention(pool, 0, [0, 1, 2, 3], P, q, 0.1)
    b, _ = KV.attention(pool, 0, [2, 0, 1, 3], P, q, 0.1)
    assert np.max(np.abs(a - b)) <= 1e-12 * np.max(np.abs(a))
    pool.page_table[0, 1] = -1                                  # unmap logical page 1
    c, _ = KV.attention(pool, 0, [0, 1, 2, 3], P, q, 0.1)
    pool.page_table[0, 1] = 1
    d, _ = KV.attention(pool, 0, [0, 2, 3], P, q, 0.1)
    assert np.max(np.abs(c - d)) <= 1e-12 * np.max(np.abs(d))


def test_masking_equals_truncation():
    pool = _pool()
    q = _q(3, seed=11)
    a, _ = KV.attention(pool, 0, [0, 1], 10, q, 0.09)
    k, v, mask = KV.window_keys(pool, 0, [0, 1], 10, 4)
    assert mask.sum() == P + 10
    assert not mask[P + 10:].any()
