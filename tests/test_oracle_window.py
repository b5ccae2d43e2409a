"""Pins of the window page-list reading (oracle/window.py), CPU only."""

import numpy as np

import synth
from oracle.window import window_pages


def test_long_context_window_matches_the_bench_list():
    # 65536 cached tokens, 256-token pages: 1024-token global sink + 16384 recent tokens
    lc = synth.LongContextKV()
    pages, last = window_pages(65536, 256, 1024, 0, 0, 16384)
    assert pages == lc.window()
    assert last == 256 and len(pages) == 68


def test_hand_cases():
    # partial last page, sink and window overlapping
    assert window_pages(1000, 256, 300, 0, 0, 500) == ([0, 1, 2, 3], 1000 - 768)
    # shot sink inside the window adds nothing
    assert window_pages(4096, 256, 256, 3800, 100, 512) == ([0, 14, 15], 256)
    # shot sink between global sink and window, straddling pages 3 and 4 (tokens
    # 1000..1029); ranges round outward to whole pages
    assert window_pages(4096, 256, 10, 1000, 30, 1) == ([0, 3, 4, 15], 256)
    # empty cache
    assert window_pages(0, 256, 1024, 0, 100, 4096) == ([], 0)
    # shot sink reaching past the cached length is clipped
    assert window_pages(700, 256, 0, 600, 500, 0) == ([2], 700 - 512)


def test_brute_force_token_membership():
    rng = np.random.default_rng(7)
    for _ in range(200):
        P = int(rng.choice([64, 128, 256]))
        T = int(rng.integers(0, 5000))
        G, s0, S, W = (int(v) for v in rng.integers(0, 3000, size=4))
        pages, last = window_pages(T, P, G, s0, S, W)
        # a page is listed iff one of its tokens lies in a range
        for p in range(-(-T // P) if T else 0):
            toks = range(p * P, min(T, p * P + P))
            inside = any(t < G or s0 <= t < s0 + S or t >= T - W for t in toks)
            assert (p in pages) == inside
        assert pages == sorted(set(pages))
        if pages:
            assert 1 <= last <= P
