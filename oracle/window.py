"""Multi-shot sink window -> logical page list (test infrastructure only).

What the page fixes (techwalker.com LongLive-2.0 report summary, section 六):
generation attends to a sliding window of recent content; a global sink
always keeps the first frames of the video in view; a shot sink keeps the
first frames of the current shot and is re-bound to the new shot's start at
a scene change; the two sinks are laid over the sliding window, and the shot
sink is recorded as two pointers (start, length) without copying data.

Readings (the page is silent on these):

* The three parts are token ranges of the cached sequence of length T:
  global sink [0, G), shot sink [start, start + S), window [T - W, T), each
  clipped to [0, T).
* The cache is paged, so the window handed to the KV kernels is the list of
  logical pages that contain at least one token of the union, in increasing
  order, each once (ranges round outward to whole pages).
* The last listed page holds min(P, T - P * last) valid tokens.
"""


def window_pages(total_tokens, page_tokens, global_sink, shot_start, shot_sink, window):
    """(pages, last_page_tokens) of the union of the three token ranges."""
    T, P = total_tokens, page_tokens
    tokens = set()
    for a, b in ((0, global_sink), (shot_start, shot_start + shot_sink), (T - window, T)):
        a, b = max(a, 0), min(b, T)
        tokens.update(range(a, b))
    pages = sorted({t // P for t in tokens})
    last = min(P, T - P * pages[-1]) if pages else 0
    return pages, last
