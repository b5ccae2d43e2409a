"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the bench.

This module only draws random numbers and rounds samples to the input dtype
(bf16 via torch's round-to-nearest-even conversion).  It holds none of the
NVFP4 arithmetic, and neither imports the oracle nor the product library.

Workload recipes (DiT-shaped tensors of a 5B video model; the pages name the
model -- techwalker.com LongLive-2.0 report summary, section 七, Wan2.2-TI2V-5B
-- but not its dimensions, so the shapes below are the stated workload sizes):

* tiny:       X fp32 [256 x 1024] ~ N(0, 1) with 0.5% of entries (chosen without
              replacement) multiplied by 30; W fp32 [256 x 1024] ~ N(0, 0.02).
* attn proj:  X bf16 [4096 x 3072] ~ N(0, 1) with 8 fixed channels x20 (applied
              before the bf16 rounding); W bf16 [3072 x 3072] ~ N(0, 0.02).
* ffn pair:   X bf16 [8192 x 3072] (attn-proj distribution); W1 [14336 x 3072],
              W2 [3072 x 14336] ~ N(0, 0.02).
* kv write:   K, V bf16 [7040 x 24 x 128] ~ N(0, 1); K gets a per-(head,
              channel) offset ~ N(0, 3) before the bf16 rounding.
* kv read:    30 layers x 65536 tokens written as 9 chunks of 7040 tokens and
              one of 2176; per-(layer, head, channel) K offsets; physical pages
              a random permutation.

N(m, s) means mean m and standard deviation s.  Random numbers come from
numpy's PCG64 (``numpy.random.default_rng(seed)``), so both sides of every
comparison see the same bytes.
"""

import numpy as np
import torch

# ------------------------------------------------------------------ helpers


def to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """fp32 samples -> bf16 bit patterns (uint16), torch RNE conversion."""
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 values (exact widening)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_f32(shape, std, seed) -> np.ndarray:
    return np.random.default_rng(seed).standard_normal(shape, dtype=np.float32) * np.float32(std)


# ------------------------------------------------------------------ GEMM-side tensors


def entry_outliers_f32(rows, cols, seed, idx_seed, frac=0.005, factor=30.0):
    """N(0,1) fp32 with round(frac * rows * cols) entries multiplied by ``factor``."""
    x = normal_f32((rows, cols), 1.0, seed)
    n = int(round(frac * rows * cols))
    idx = np.random.default_rng(idx_seed).choice(rows * cols, size=n, replace=False)
    x.reshape(-1)[idx] *= np.float32(factor)
    return x


def channel_outliers_bf16(rows, cols, seed, ch_seed, n_ch=8, factor=20.0):
    """N(0,1) with ``n_ch`` fixed channels (columns) scaled before the bf16 round."""
    x = normal_f32((rows, cols), 1.0, seed)
    ch = np.random.default_rng(ch_seed).choice(cols, size=min(n_ch, cols), replace=False)
    x[:, ch] *= np.float32(factor)
    return to_bf16_bits(x)


def weights_bf16(rows, cols, seed, std=0.02):
    return to_bf16_bits(normal_f32((rows, cols), std, seed))


def tiny(rows=256, cols=1024, n=256):
    """Tiny round-trip + GEMM case (fp32 inputs)."""
    return {
        "x": entry_outliers_f32(rows, cols, seed=0, idx_seed=2),
        "w": normal_f32((n, cols), 0.02, seed=1),
    }


def attn_proj(m=4096, k=3072, n=3072):
    """Attention projection: activations with channel outliers, NVFP4-bound weights."""
    return {
        "x": channel_outliers_bf16(m, k, seed=10, ch_seed=12),
        "w": weights_bf16(n, k, seed=11),
    }


def ffn_pair(m=8192, d=3072, f=14336):
    """FFN up/down pair; the input has the attention-projection distribution."""
    return {
        "x": channel_outliers_bf16(m, d, seed=20, ch_seed=23),
        "w1": weights_bf16(f, d, seed=21),
        "w2": weights_bf16(d, f, seed=22),
    }


# ------------------------------------------------------------------ KV-cache tensors

KV_HEADS = 24
KV_HEAD_DIM = 128
KV_PAGE = 256
KV_CHUNK = 7040            # 8 latent frames x 880 tokens


def kv_chunk(t=KV_CHUNK, h=KV_HEADS, d=KV_HEAD_DIM, seed_k=30, seed_v=31, seed_off=32,
             offset=None):
    """One chunk of new K, V (bf16 bits, [T, H, D]); K has a per-(h, d) offset."""
    if offset is None:
        offset = normal_f32((h, d), 3.0, seed_off)
    k = normal_f32((t, h, d), 1.0, seed_k) + offset[None]
    v = normal_f32((t, h, d), 1.0, seed_v)
    return to_bf16_bits(k), to_bf16_bits(v)


def page_permutation(n, seed):
    return np.random.default_rng(seed).permutation(n).astype(np.int32)


class LongContextKV:
    """Recipe of the long-context cache: layers x tokens in chunks, shuffled pages.

    Chunk c of layer l:  K = bf16(Z_k[c] + off[l]),  V = bf16(Z_v[c]), where
    Z_k[c], Z_v[c] ~ N(0, 1) are drawn once per chunk index (seeds 1000 + 2c and
    1001 + 2c) and off[l] ~ N(0, 3) per (head, channel) (seed 40 + 100 l).
    Physical pages: a permutation of layers * pages (seed 41).
    """

    def __init__(self, n_layers=30, tokens=65536, chunk=KV_CHUNK, h=KV_HEADS,
                 d=KV_HEAD_DIM, page=KV_PAGE):
        self.L, self.N, self.C, self.H, self.D, self.P = n_layers, tokens, chunk, h, d, page
        self.pages_per_layer = -(-tokens // page)
        self.n_phys = n_layers * self.pages_per_layer
        self.page_table = page_permutation(self.n_phys, 41).reshape(n_layers, self.pages_per_layer)
        starts = list(range(0, tokens, chunk))
        self.chunks = [(s, min(chunk, tokens - s)) for s in starts]
        self._z = {}

    def _base(self, c, t):
        key = (c, t)
        if key not in self._z:
            self._z[key] = (normal_f32((t, self.H, self.D), 1.0, 1000 + 2 * c),
                            normal_f32((t, self.H, self.D), 1.0, 1001 + 2 * c))
        return self._z[key]

    def offset(self, layer):
        return normal_f32((self.H, self.D), 3.0, 40 + 100 * layer)

    def chunk(self, layer, c):
        """(start_token, K bits, V bits) of chunk c of a layer."""
        start, t = self.chunks[c]
        zk, zv = self._base(c, t)
        return start, to_bf16_bits(zk + self.offset(layer)[None]), to_bf16_bits(zv)

    def chunk_torch(self, layer, c, device):
        """The same recipe drawn with torch's generator on ``device``: fast, but the
        values differ from :meth:`chunk`.  For timing runs, where only the shapes
        and the distribution matter."""
        start, t = self.chunks[c]
        g = torch.Generator(device=device)
        g.manual_seed(1000 + 2 * c)
        zk = torch.randn((t, self.H, self.D), generator=g, device=device)
        g.manual_seed(1001 + 2 * c)
        zv = torch.randn((t, self.H, self.D), generator=g, device=device)
        off = torch.from_numpy(self.offset(layer)).to(device)
        return start, (zk + off).to(torch.bfloat16), zv.to(torch.bfloat16)

    def window(self, sink_pages=4, recent_tokens=16384):
        """Logical pages of the attention window: sink pages + the most recent tokens."""
        last = self.pages_per_layer
        recent = recent_tokens // self.P
        return list(range(sink_pages)) + list(range(last - recent, last))


def attn_queries(n_q, h=KV_HEADS, d=KV_HEAD_DIM, seed=50, std=1.0) -> np.ndarray:
    """Queries [n_q, h, d] as bf16 bits (normal, so q.k / sqrt(d) is O(1))."""
    return to_bf16_bits(normal_f32((n_q, h, d), std, seed))


# ------------------------------------------------------------------ adaLN producer

ADALN_ROWS_PER_GROUP = 880        # one latent frame of tokens per modulation pair


def adaln_modulation(n_groups, cols, seed=70, std=0.25):
    """(shift, scale) fp32 [n_groups, cols] ~ N(0, std): one pair per latent frame."""
    rng = np.random.default_rng(seed)
    shift = rng.standard_normal((n_groups, cols), dtype=np.float32) * np.float32(std)
    scale = rng.standard_normal((n_groups, cols), dtype=np.float32) * np.float32(std)
    return shift, scale


def adaln_input(m=4096, k=3072, seed=72, dtype="bf16"):
    """Residual stream entering a DiT block [m, k]: attn-proj distribution
    (N(0,1), 8 channels x20), as bf16 bits or fp32, plus its modulation."""
    x32 = normal_f32((m, k), 1.0, seed)
    ch = np.random.default_rng(seed + 1).choice(k, size=min(8, k), replace=False)
    x32[:, ch] *= np.float32(20.0)
    groups = -(-m // ADALN_ROWS_PER_GROUP)
    shift, scale = adaln_modulation(groups, k, seed=seed + 2)
    x = to_bf16_bits(x32) if dtype == "bf16" else x32
    return {"x": x, "shift": shift, "scale": scale, "rows_per_group": ADALN_ROWS_PER_GROUP}
