"""NVFP4 KV cache -- exact CPU oracle (test infrastructure only).

What the pages fix (techwalker.com LongLive-2.0 report summary, section 四,
second key): the KV cache is stored in NVFP4; K first gets a simple mean
subtraction so its values concentrate, then is quantized; a parallel kernel
decompresses many cache blocks of a time window at once.  The zuobiaodaohang
LongLive blog (section "NVFP4：数据体积砍到 1/4") adds that the quantized KV
cache is updated in place.  Video is generated in chunks of 8 latent frames
(techwalker summary, section 三), which is the granularity of a KV write.

Readings (the pages are silent on these):

* The mean is taken per (head, channel) over the tokens of one written chunk,
  and stored in fp32:  mu = RN32(S / T)  with S the exact sum.
* K' = RN32(K - mu); K' and V are NVFP4-quantized along head_dim (blocks of 16),
  each with one fp32 global scale per (layer, chunk) -- "per tensor" read as
  one chunk's K (or V) of one layer.
* Dequantization adds the mean back with one rounding:
  K^ = RN_bf16(q s_b s_gK + mu),  V^ = RN_bf16(q s_b s_gV).
* Paged storage: pages of ``page_tokens`` tokens; a page table maps
  (layer, logical page) -> physical page.  Page byte layout:
  K codes [H][P][D/2], K scales [H][P][D/16], V codes [H][P][D/2],
  V scales [H][P][D/16].  Per (layer, logical page) a pair {c_first, split}:
  slots [0, split) belong to chunk c_first, slots [split, P) to c_first + 1.
"""

from fractions import Fraction

import numpy as np

from . import formats as F
from . import nvfp4 as Q


def exact_column_sums(x: np.ndarray) -> list:
    """Exact sums over axis 0 of bf16 numbers (given as fp64), as Fractions.

    Every bf16 number is m * 2^e with an integer |m| < 2^8.  The integers m
    are summed per (exponent, column) bin -- exact, as each bin total is an
    integer below 2^8 * rows < 2^53 -- and the bins of a column are then
    combined as exact rationals.
    """
    x = np.asarray(x, dtype=np.float64)
    rows = x.shape[0]
    flat = x.reshape(rows, -1)
    ncols = flat.shape[1]
    assert rows < 2**44
    f, e = np.frexp(flat)
    m = np.ldexp(f, 8)
    assert np.array_equal(np.rint(m), m), "inputs must be bf16 numbers"
    ex = (e - 8).astype(np.int64)
    emin = int(ex.min()) if ex.size else 0
    nexp = int(ex.max()) - emin + 1 if ex.size else 1
    col = np.broadcast_to(np.arange(ncols), flat.shape)
    bins = np.bincount(((ex - emin) * ncols + col).reshape(-1),
                       weights=m.reshape(-1), minlength=nexp * ncols)
    bins = bins.reshape(nexp, ncols)
    sums = []
    for j in range(ncols):
        s = Fraction(0)
        for u in np.nonzero(bins[:, j])[0]:
            s += int(bins[u, j]) * Fraction(2) ** int(u + emin)
        sums.append(s)
    return sums


def chunk_mean(k: np.ndarray) -> np.ndarray:
    """mu[h, d] = RN32(exact mean over tokens) for K[T, H, D] of bf16 numbers."""
    t, h, d = k.shape
    sums = exact_column_sums(k.reshape(t, h * d))
    mu = np.array([F.round_fraction_to_binary(s / t, F.F32) for s in sums])
    return mu.reshape(h, d)


class ChunkQ:
    """Quantized chunk: per-token codes/scales for K' and V, plus mu and scales."""

    def __init__(self, k, v):
        k = np.asarray(k, dtype=np.float64)
        v = np.asarray(v, dtype=np.float64)
        t, h, d = k.shape
        assert d % Q.BLOCK == 0 and v.shape == k.shape
        self.mu = chunk_mean(k)                                  # [H, D]
        self.kp = F.round_sum_to_binary(k, -self.mu[None], F.F32)  # K' = RN32(K - mu)
        kq = Q.quantize(self.kp.reshape(t * h, d))
        vq = Q.quantize(v.reshape(t * h, d))
        self.s_gk, self.s_gv = kq.s_g, vq.s_g
        self.k_codes = kq.packed.reshape(t, h, d // 2)
        self.k_scales = kq.scales.reshape(t, h, d // 16)
        self.v_codes = vq.packed.reshape(t, h, d // 2)
        self.v_scales = vq.scales.reshape(t, h, d // 16)


class KVPool:
    """Host model of the paged NVFP4 KV cache (same byte layout as the device pool)."""

    def __init__(self, n_layers, n_heads, head_dim, page_tokens, max_pages,
                 max_chunks, page_table, n_phys_pages):
        self.L, self.H, self.D, self.P = n_layers, n_heads, head_dim, page_tokens
        self.max_pages, self.max_chunks = max_pages, max_chunks
        self.page_table = np.asarray(page_table, dtype=np.int64).reshape(n_layers, max_pages)
        self.page_bytes = 2 * n_heads * page_tokens * (head_dim // 2 + head_dim // 16)
        self.pool = np.zeros((n_phys_pages, self.page_bytes), dtype=np.uint8)
        self.page_chunk = np.zeros((n_layers, max_pages, 2), dtype=np.int64)
        self.k_mean = np.zeros((n_layers, max_chunks, n_heads, head_dim))
        self.k_gscale = np.zeros((n_layers, max_chunks))
        self.v_gscale = np.zeros((n_layers, max_chunks))

    # byte offsets of the four regions inside a page
    def _regions(self):
        h, p, d = self.H, self.P, self.D
        kc = 0
        ks = kc + h * p * d // 2
        vc = ks + h * p * d // 16
        vs = vc + h * p * d // 2
        return kc, ks, vc, vs

    def page_view(self, phys):
        kc, ks, vc, vs = self._regions()
        h, p, d = self.H, self.P, self.D
        pg = self.pool[phys]
        return (pg[kc:ks].reshape(h, p, d // 2), pg[ks:vc].reshape(h, p, d // 16),
                pg[vc:vs].reshape(h, p, d // 2), pg[vs:].reshape(h, p, d // 16))

    def write_chunk(self, layer, chunk_id, k, v, start_token) -> ChunkQ:
        """Quantize one chunk and store it in place (pages, mu, scales, page_chunk)."""
        if chunk_id == 0 and start_token % self.P:
            # a chunk that starts inside a page shares it with the chunk before
            # it; the first chunk of a layer has none
            raise ValueError("chunk 0 must start on a page boundary")
        c = ChunkQ(k, v)
        t = k.shape[0]
        self.k_mean[layer, chunk_id] = c.mu
        self.k_gscale[layer, chunk_id] = c.s_gk
        self.v_gscale[layer, chunk_id] = c.s_gv
        for i in range(t):
            pos = start_token + i
            lp, slot = divmod(pos, self.P)
            kcv, ksv, vcv, vsv = self.page_view(self.page_table[layer, lp])
            kcv[:, slot] = c.k_codes[i]
            ksv[:, slot] = c.k_scales[i]
            vcv[:, slot] = c.v_codes[i]
            vsv[:, slot] = c.v_scales[i]
        first = start_token // self.P
        last = (start_token + t - 1) // self.P
        for lp in range(first, last + 1):
            if lp == first and start_token % self.P:
                # slots before the chunk's first token belong to the chunk
                # written just before it (chunks of a layer are written in order)
                self.page_chunk[layer, lp] = (chunk_id - 1, start_token % self.P)
            else:
                self.page_chunk[layer, lp] = (chunk_id, self.P)
        return c

    def dequant_pages(self, layer, logical_pages):
        """K^, V^ for the listed logical pages, as bf16 numbers in fp64, [n*P, H, D]."""
        outs_k, outs_v = [], []
        slots = np.arange(self.P)
        for lp in logical_pages:
            kcv, ksv, vcv, vsv = self.page_view(self.page_table[layer, lp])
            c0, split = self.page_chunk[layer, lp]
            ch = np.minimum(np.where(slots < split, c0, c0 + 1), self.max_chunks - 1)
            k_qsb = _qsb(kcv, ksv)                      # [H, P, D]
            v_qsb = _qsb(vcv, vsv)
            sgk = self.k_gscale[layer, ch][None, :, None]
            sgv = self.v_gscale[layer, ch][None, :, None]
            mu = self.k_mean[layer, ch].transpose(1, 0, 2)   # [H, P, D]
            khat = F.round_sum_to_binary(k_qsb * sgk, mu, F.BF16)
            vhat = F.round_f64_to_binary(v_qsb * sgv, F.BF16)
            outs_k.append(khat.transpose(1, 0, 2))
            outs_v.append(vhat.transpose(1, 0, 2))
        return np.concatenate(outs_k), np.concatenate(outs_v)


def window_keys(pool, layer, logical_pages, last_page_tokens, n_phys_pages):
    """K^, V^ [n, H, D] and the key mask [n] of a listed window.

    Reading (the pages say only that many cache blocks of a time window are
    decompressed in parallel): a listed page contributes all its slots, except
    the last listed page, which contributes its first ``last_page_tokens``;
    a listed page that is not mapped (page table entry outside the pool, or a
    logical index outside the table) contributes no keys.
    """
    P = pool.P
    keys_k, keys_v, mask = [], [], []
    for i, lp in enumerate(logical_pages):
        n_valid = last_page_tokens if i == len(logical_pages) - 1 else P
        mapped = 0 <= lp < pool.max_pages and 0 <= pool.page_table[layer, lp] < n_phys_pages
        if mapped:
            k, v = pool.dequant_pages(layer, [lp])
        else:
            k = np.zeros((P, pool.H, pool.D))
            v = np.zeros((P, pool.H, pool.D))
        keys_k.append(k)
        keys_v.append(v)
        mask.append((np.arange(P) < n_valid) & mapped)
    return np.concatenate(keys_k), np.concatenate(keys_v), np.concatenate(mask)


def attention(pool, layer, logical_pages, last_page_tokens, q, scale, n_phys_pages=None):
    """Attention of queries q [n_q, H, D] over the valid keys of a listed window.

    O[n, h] = sum_j softmax_j(scale * q[n, h] . K^[j, h]) V^[j, h] over the
    valid keys j (see window_keys), computed in fp64 (the definition; the
    device's result is compared within a tolerance).  Reading: every query
    sees every valid key of the window (no causal mask: the window is the
    context the new chunk attends to).  No valid key -> O = 0.
    """
    if n_phys_pages is None:
        n_phys_pages = pool.pool.shape[0]
    k, v, mask = window_keys(pool, layer, logical_pages, last_page_tokens, n_phys_pages)
    k, v = k[mask], v[mask]
    n_q, H, D = q.shape
    out = np.zeros((n_q, H, D))
    weight_abs_v = np.zeros((n_q, H, D))
    if k.shape[0] == 0:
        return out, weight_abs_v
    for h in range(H):
        logits = scale * (q[:, h, :] @ k[:, h, :].T)             # [n_q, n_keys]
        logits -= logits.max(axis=1, keepdims=True)
        w = np.exp(logits)
        w /= w.sum(axis=1, keepdims=True)
        out[:, h, :] = w @ v[:, h, :]
        weight_abs_v[:, h, :] = w @ np.abs(v[:, h, :])
    return out, weight_abs_v


def _qsb(codes, scales):
    """q * s_b (exact fp64) for [H, P, D/2] codes and [H, P, D/16] scale bytes."""
    h, p, half = codes.shape
    lo = codes & 0xF
    hi = codes >> 4
    c = np.empty((h, p, half * 2), dtype=np.uint8)
    c[..., 0::2] = lo
    c[..., 1::2] = hi
    q = F.E2M1_MAGNITUDES[c & 7]
    q = np.where(c & 8, -q, q)
    return q * np.repeat(F.E4M3_GRID[scales], Q.BLOCK, axis=-1)
