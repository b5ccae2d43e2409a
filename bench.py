"""Benchmark of the NVFP4 hot path on one MI355X.

One step is one pass of the whole hot path over resident synthetic inputs:

  attn proj   quantize X bf16 [4096 x 3072] (amax + fused scale/encode), then
              W4A4 GEMM with the pre-quantized W [3072 x 3072] -> bf16 [4096 x 3072]
  dequantize  X's NVFP4 back to bf16 [4096 x 3072]
  ffn pair    quantize X [8192 x 3072]; GEMM1 with W1 [14336 x 3072] -> Y1 bf16 with
              the fused output amax; requantize Y1 (one read, amax given); GEMM2
              with W2 [3072 x 14336] -> bf16 [8192 x 3072]
  kv write    one layer's new chunk K, V bf16 [7040 x 24 x 128]: K mean, K', NVFP4
              into 256-token pages of a shuffled page table
  kv read     30 layers x 65536 cached tokens: the window of every layer (4 sink
              pages + the most recent 16384 tokens = 68 pages) dequantized to bf16
              with the K means added back, one launch per layer

The metric is the whole step as a percentage of the MI355X roofline: the time
the step's algorithmic work takes at the roofline (HBM 8 TB/s for the
bandwidth kernels -- one read of every input and one write of every output --
and the 2.5 PFLOP/s dense fp16 MFMA peak for the GEMMs, which run on the
fp16 MFMA) divided by the
measured step time.  Per-op rates (GB/s, TFLOP/s) and fractions are reported
alongside, plus the roofline of the dominant kernel (the FFN GEMM1 launch)
and the CPU oracle's rate on a bounded sample of the same work.  Per-op times
are in-step (inputs cold in the Infinity Cache: the step streams GBs between
reuses); hot_ms is the same op repeated back to back, and copy_frac is a
bandwidth op's in-step rate over a measured 1 GiB device copy (hbm_copy_gbps).

usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
       python bench.py --only OP [--reps N]     one op of the step, N times (profiling)
       python bench.py --copy-bytes B [--reps N] a plain device copy of B bytes, N times
                                                 (calibrates the HBM byte counters)

roofline.traffic is the HBM traffic of one FFN GEMM1 launch as measured by
rocprofv3 counters (profiles/ffn_gemm1_hbm_traffic.md); it is reported only
while the GEMM source is the one those counters were taken with, else null.
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_BPS = 8.0e12               # MI355X HBM3E peak, bytes/s
MFMA_F16_FLOPS = 2.5e15        # MI355X dense fp16 (and bf16) MFMA peak, FLOP/s
GEMM_SOURCE = os.path.join(ROOT, "w4a4_gemm_amd", "csrc", "gemm.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "ffn_gemm1_hbm_traffic.md")
METRIC = "W4A4 GEMM TFLOPS + quant/dequant/KV GB/s, as % of MI355X roofline"

NV_ELEM = 0.5625               # NVFP4 bytes per element (4-bit code + E4M3 per 16)
ATTN_QUERIES = 880             # one latent frame of queries for the fused window attention


# ------------------------------------------------------------------ workload accounting

def op_table():
    """Algorithmic bytes / FLOPs of every op in one step."""
    a_m, a_k, a_n = 4096, 3072, 3072
    f_m, f_d, f_f = 8192, 3072, 14336
    kv_t, kv_h, kv_d = 7040, 24, 128
    layers, win_pages, page = 30, 68, 256
    page_bytes = 2 * kv_h * page * (kv_d // 2 + kv_d // 16)
    kv_elems = kv_t * kv_h * kv_d
    win_elems = win_pages * page * kv_h * kv_d          # per K (or V) per layer
    return {
        "attn_quantize": {"bytes": a_m * a_k * (2 + NV_ELEM) + 4},
        "attn_gemm": {"flops": 2 * a_m * a_n * a_k},
        "attn_dequantize": {"bytes": a_m * a_k * (NV_ELEM + 2) + 4},
        "ffn_quantize": {"bytes": f_m * f_d * (2 + NV_ELEM) + 4},
        "ffn_gemm1": {"flops": 2 * f_m * f_f * f_d},
        "ffn_requantize": {"bytes": f_m * f_f * (2 + NV_ELEM) + 4},
        "ffn_gemm2": {"flops": 2 * f_m * f_d * f_f},
        "kv_write": {"bytes": 2 * kv_elems * 2 + 2 * kv_elems * NV_ELEM + kv_h * kv_d * 4 + 8},
        "kv_read": {"bytes": layers * (win_pages * page_bytes + 2 * win_elems * 2),
                    "compressed_bytes": layers * win_pages * page_bytes},
    }


def next_op_table():
    """Algorithmic work of the rows measured beside the step."""
    keys = 68 * 256
    m, k, groups = 8192, 3072, -(-8192 // 880)
    return {"kv_attention": {"flops": 4 * ATTN_QUERIES * keys * 128 * 24,
                             "compressed_bytes": 68 * 2 * 24 * 256 * (64 + 8),
                             "workload": (f"{ATTN_QUERIES} queries x 24 heads x 128 over a 68-page "
                                          "window (17408 keys), pages read as NVFP4; bf16 MFMA")},
            # wgrad of FFN GEMM1, dW1 [14336 x 3072] = dY1^T X over 8192 tokens
            "wgrad_quantize_t": {"bytes": 8192 * 14336 * (2 + NV_ELEM) + 4,
                                 "workload": ("dY1 8192x14336 bf16 -> NVFP4 of dY1^T "
                                              "(blocks along the tokens), tiled scales")},
            "wgrad_gemm": {"flops": 2 * 14336 * 3072 * 8192,
                           "workload": ("FFN GEMM1 wgrad M14336 N3072 K8192 (tokens), "
                                        "both operands transposed-quantized, fp32 out")},
            # host merge of three page ranges + one small launch writing the list
            "window_pages": {"bytes": 68 * 4, "launch_bound": True,
                             "workload": ("global sink 1024 + window 16384 of 65536 cached tokens "
                                          "-> 68-page list on the device (launch-bound)")},
            # x read once, NVFP4 written, row stats written, modulation read once
            "adaln_quantize": {"bytes": m * k * (2 + NV_ELEM) + 4 + 8 * m + 2 * groups * k * 4,
                               "workload": ("FFN input 8192x3072 bf16: LayerNorm + adaLN modulate "
                                            "(880-row groups) + NVFP4, tiled scales")}}


def roofline_seconds(op):
    if "flops" in op:
        return op["flops"] / MFMA_F16_FLOPS
    return op["bytes"] / HBM_BPS


# ------------------------------------------------------------------ GPU step

class Workload:
    """Device inputs and outputs of the step's ops; ``groups`` limits the build to
    the ops being run (None: everything, as the full bench needs)."""

    GROUPS = ("attn", "ffn", "kvw", "kvr", "adaln", "wgrad")
    # op -> the input groups it needs
    NEEDS = {"attn_quantize": ("attn",), "attn_gemm": ("attn",), "attn_dequantize": ("attn",),
             "ffn_quantize": ("ffn",), "ffn_gemm1": ("ffn",), "ffn_requantize": ("ffn",),
             "ffn_gemm2": ("ffn",), "kv_write": ("kvw",), "kv_read": ("kvr",),
             "kv_attention": ("kvr",), "window_pages": ("kvr",), "adaln_quantize": ("adaln",),
             "wgrad_quantize_t": ("ffn", "wgrad"), "wgrad_gemm": ("ffn", "wgrad")}

    def __init__(self, dev, groups=None):
        import torch
        import synth
        import w4a4_gemm_amd as nv
        self.nv, self.torch, self.dev, self.synth = nv, torch, dev, synth
        groups = set(self.GROUPS if groups is None else groups)
        for g in self.GROUPS:
            if g in groups:
                getattr(self, "_build_" + g)()
        self._ops = self.ops() if groups >= {"attn", "ffn", "kvw", "kvr"} else None
        torch.cuda.synchronize()

    def _bf16(self, bits):
        torch = self.torch
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
            torch.bfloat16).to(self.dev)

    def _build_attn(self):
        nv, torch, dev = self.nv, self.torch, self.dev
        a = self.synth.attn_proj()
        self.ax = self._bf16(a["x"])
        self.aw = nv.nvfp4_quantize(self._bf16(a["w"]))              # weights pre-quantized
        self.axq = nv.NVFP4Tensor(4096, 3072, nv.SCALES_TILED, device=dev)
        self.ay = torch.empty((4096, 3072), dtype=torch.bfloat16, device=dev)
        self.adq = torch.empty((4096, 3072), dtype=torch.bfloat16, device=dev)
        self.aws = torch.empty(nv.nvfp4_workspace_bytes(nv.OP_QUANTIZE, 4096, 3072, 0),
                               dtype=torch.uint8, device=dev)

    def _build_ffn(self):
        nv, torch, dev = self.nv, self.torch, self.dev
        f = self.synth.ffn_pair()
        self.fx = self._bf16(f["x"])
        self.fw1 = nv.nvfp4_quantize(self._bf16(f["w1"]))
        self.fw2 = nv.nvfp4_quantize(self._bf16(f["w2"]))
        del f
        self.fxq = nv.NVFP4Tensor(8192, 3072, nv.SCALES_TILED, device=dev)
        self.fy1 = torch.empty((8192, 14336), dtype=torch.bfloat16, device=dev)
        self.fy1q = nv.NVFP4Tensor(8192, 14336, nv.SCALES_TILED, device=dev)
        self.fy2 = torch.empty((8192, 3072), dtype=torch.bfloat16, device=dev)
        self.famax = torch.zeros(1, dtype=torch.float32, device=dev)
        self.fws = torch.empty(nv.nvfp4_workspace_bytes(nv.OP_QUANTIZE, 8192, 3072, 0),
                               dtype=torch.uint8, device=dev)
        # the requantize's input as the step produces it
        nv.nvfp4_quantize(self.fx, out=self.fxq, workspace=self.fws)
        nv.nvfp4_gemm_w4a4(self.fxq, self.fw1, out=self.fy1, y_amax=self.famax)

    def _build_kvw(self):
        nv, dev = self.nv, self.dev
        kb, vb = self.synth.kv_chunk()
        self.kv_k, self.kv_v = self._bf16(kb), self._bf16(vb)
        table = self.synth.page_permutation(28, 33)[None, :]
        self.kv_w = nv.KVCache(1, 24, 128, 256, 28, 1, table, 28, device=dev)
        self.kv_ws = self.kv_w.workspace(7040)

    def _build_kvr(self):
        nv, torch, dev = self.nv, self.torch, self.dev
        r = self.synth.LongContextKV()
        self.lc = nv.KVCache(r.L, r.H, r.D, r.P, r.pages_per_layer, len(r.chunks), r.page_table,
                             r.n_phys, device=dev)
        lc_ws = self.lc.workspace(max(n for _, n in r.chunks))
        for layer in range(r.L):
            for c in range(len(r.chunks)):
                start, k, v = r.chunk_torch(layer, c, dev)
                nv.nvfp4_kv_quantize(self.lc, layer, c, k, v, start, workspace=lc_ws)
        self.lc_layers = r.L
        self.window = torch.tensor(r.window(), dtype=torch.int32, device=dev)
        n = self.window.numel() * r.P
        self.kh = torch.empty((n, r.H, r.D), dtype=torch.bfloat16, device=dev)
        self.vh = torch.empty((n, r.H, r.D), dtype=torch.bfloat16, device=dev)
        # next row (not part of the step): one 880-token latent frame's queries
        # attending to layer 0's window, read straight from the NVFP4 pages
        self.attn_q = self._bf16(self.synth.attn_queries(ATTN_QUERIES, r.H, r.D, seed=50))
        self.attn_out = torch.empty_like(self.attn_q)
        self.attn_last = r.P
        self.win_pages = torch.empty(256, dtype=torch.int32, device=dev)

    def _build_adaln(self):
        nv, torch, dev = self.nv, self.torch, self.dev
        # next row: the FFN input produced by LayerNorm + adaLN + NVFP4 in one kernel pair
        d = self.synth.adaln_input(m=8192, k=3072, seed=72)
        self.ln_x = self._bf16(d["x"])
        self.ln_shift = torch.from_numpy(d["shift"]).to(dev)
        self.ln_scale = torch.from_numpy(d["scale"]).to(dev)
        self.ln_rpg = d["rows_per_group"]
        self.ln_q = nv.NVFP4Tensor(8192, 3072, nv.SCALES_TILED, device=dev)
        self.ln_stats = torch.empty((8192, 2), dtype=torch.float32, device=dev)
        self.ln_ws = torch.empty(nv.nvfp4_workspace_bytes(nv.OP_ADALN_QUANTIZE, 8192, 3072, 0),
                                 dtype=torch.uint8, device=dev)

    def _build_wgrad(self):
        nv, torch, dev = self.nv, self.torch, self.dev
        # next row: wgrad of FFN GEMM1 on transposed-quantized operands
        gen = torch.Generator(device=dev).manual_seed(90)
        self.wg_dy = (torch.randn((8192, 14336), generator=gen, device=dev) * 1e-3).to(
            torch.bfloat16)
        self.wg_dyq = nv.NVFP4Tensor(14336, 8192, nv.SCALES_TILED, device=dev)
        self.wg_xq = nv.nvfp4_quantize_transposed(self.fx)
        self.wg_out = torch.empty((14336, 3072), dtype=torch.float32, device=dev)
        self.wg_ws = torch.empty(nv.nvfp4_workspace_bytes(nv.OP_QUANTIZE, 8192, 14336, 0),
                                 dtype=torch.uint8, device=dev)
        nv.nvfp4_quantize_transposed(self.wg_dy, out=self.wg_dyq, workspace=self.wg_ws)

    def ops(self):
        """The step's ops in order, as (name, callable) pairs."""
        nv = self.nv

        def ffn_gemm1():
            nv.nvfp4_gemm_w4a4(self.fxq, self.fw1, out=self.fy1, y_amax=self.famax)

        def ffn_quantize():
            nv.nvfp4_quantize(self.fx, out=self.fxq, workspace=self.fws)
            self.famax.zero_()             # GEMM1 folds max|Y1| into a zeroed float

        def kv_read():
            for layer in range(self.lc_layers):
                nv.nvfp4_kv_dequant_blocks(self.lc, layer, self.window, self.kh, self.vh)

        return [
            ("attn_quantize", lambda: nv.nvfp4_quantize(self.ax, out=self.axq, workspace=self.aws)),
            ("attn_gemm", lambda: nv.nvfp4_gemm_w4a4(self.axq, self.aw, out=self.ay)),
            ("attn_dequantize", lambda: nv.nvfp4_dequantize(self.axq, out=self.adq)),
            ("ffn_quantize", ffn_quantize),
            ("ffn_gemm1", ffn_gemm1),
            ("ffn_requantize", lambda: nv.nvfp4_quantize(self.fy1, out=self.fy1q, amax=self.famax)),
            ("ffn_gemm2", lambda: nv.nvfp4_gemm_w4a4(self.fy1q, self.fw2, out=self.fy2)),
            ("kv_write", lambda: nv.nvfp4_kv_quantize(self.kv_w, 0, 0, self.kv_k, self.kv_v, 0,
                                                      workspace=self.kv_ws)),
            ("kv_read", kv_read),
        ]

    def next_ops(self):
        """Rows built beyond the step, measured on their own."""
        nv = self.nv
        return [("kv_attention", lambda: nv.nvfp4_kv_attention(
                    self.lc, 0, self.window, self.attn_last, self.attn_q, 1.0 / 128 ** 0.5,
                    out=self.attn_out)),
                ("wgrad_quantize_t", lambda: nv.nvfp4_quantize_transposed(
                    self.wg_dy, out=self.wg_dyq, workspace=self.wg_ws)),
                ("wgrad_gemm", lambda: nv.nvfp4_gemm_w4a4(self.wg_dyq, self.wg_xq,
                                                          out=self.wg_out)),
                ("window_pages", lambda: nv.nvfp4_kv_window_pages(
                    65536, 256, 1024, 0, 0, 16384, pages=self.win_pages)),
                ("adaln_quantize", lambda: nv.nvfp4_adaln_quantize(
                    self.ln_x, self.ln_shift, self.ln_scale, self.ln_rpg, 1e-6, out=self.ln_q,
                    row_stats=self.ln_stats, workspace=self.ln_ws))]

    def step(self, ev=None):
        """One pass of the hot path.  ``ev(name)`` records a timing event boundary."""
        mark = ev or (lambda name: None)
        for name, fn in self._ops:
            mark(name)
            fn()
        mark(None)


def run_gpu(steps, warmup):
    import torch
    dev = torch.device("cuda", 0)
    wl = Workload(dev)
    for _ in range(warmup):
        wl.step()
    torch.cuda.synchronize()

    # whole-step wall time over exactly `steps` steps
    t0 = time.perf_counter()
    for _ in range(steps):
        wl.step()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps

    # per-op durations from events on the launch stream (a separate, equal pass);
    # the steps are enqueued back to back and synchronised once, so no op's
    # interval includes the host's launch latency after a synchronisation
    names = list(op_table())
    acc = {n: 0.0 for n in names}
    per_step = []
    for _ in range(steps):
        evs = []

        def ev(name, evs=evs):
            e = torch.cuda.Event(enable_timing=True)
            e.record()
            evs.append((name, e))
        wl.step(ev)
        per_step.append(evs)
    torch.cuda.synchronize()
    for evs in per_step:
        for (n, a), (_, b) in zip(evs[:-1], evs[1:]):
            acc[n] += a.elapsed_time(b) * 1e-3
    per_op = {n: acc[n] / steps for n in names}
    # each op of the step repeated back to back: its inputs stay in the 256 MB
    # Infinity Cache where they fit (the step streams GBs between reuses)
    hot = {}
    for n, fn in wl._ops:
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        hot[n] = a.elapsed_time(b) * 1e-3 / steps
    nxt = {}
    for n, fn in wl.next_ops():
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        nxt[n] = a.elapsed_time(b) * 1e-3 / steps
    return wall, per_op, hot, nxt, copy_bytes_per_second(torch)


def copy_bytes_per_second(torch, nbytes=1 << 30, reps=5):
    """A plain 1 GiB device copy (read + write bytes per second): the
    measured reference for the bandwidth-bound ops."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) * 1e-3)
    del src, dst
    return 2 * nbytes / sorted(ts)[reps // 2]


# ------------------------------------------------------------------ CPU oracle baseline

def cpu_baseline(ops):
    """Time the oracle on a bounded sample of every op; extrapolate a step."""
    import synth
    from oracle import formats as F
    from oracle import kvcache as KV
    from oracle import nvfp4 as Q
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    host_cores = len(os.sched_getaffinity(0))

    # sample sizes chosen for roughly 10-30 s of oracle work on the host
    q_rows, g_rows, kv_tok, kv_pages = 2048, 512, 7040, 28
    a = synth.attn_proj()
    x = F.bf16_bits_to_f64(a["x"][:q_rows])               # activation rows
    t = time.perf_counter()
    xq = Q.quantize(x)
    t_q = (time.perf_counter() - t) / x.size              # s per element
    t = time.perf_counter()
    Q.dequantize(xq, "bf16")
    t_dq = (time.perf_counter() - t) / x.size
    wq = Q.quantize(F.bf16_bits_to_f64(a["w"]))
    xg = Q.NVFP4(xq.packed[:g_rows], xq.scales[:g_rows], xq.s_g)  # g_rows x 3072 x 3072 product
    t = time.perf_counter()
    Q.gemm(xg, wq)
    t_gemm = (time.perf_counter() - t) / (2 * g_rows * 3072 * 3072)   # s per FLOP
    kb, vb = synth.kv_chunk(t=kv_tok)
    pool = KV.KVPool(1, 24, 128, 256, kv_pages, 1, np.arange(kv_pages)[None, :], kv_pages)
    t = time.perf_counter()
    pool.write_chunk(0, 0, F.bf16_bits_to_f64(kb), F.bf16_bits_to_f64(vb), 0)
    t_kvw = (time.perf_counter() - t) / kb.size           # per element of K (K and V done)
    t = time.perf_counter()
    pool.dequant_pages(0, list(range(kv_pages)))
    t_kvr = (time.perf_counter() - t) / kv_pages          # per page

    est = {
        "attn_quantize": t_q * 4096 * 3072,
        "attn_gemm": t_gemm * ops["attn_gemm"]["flops"],
        "attn_dequantize": t_dq * 4096 * 3072,
        "ffn_quantize": t_q * 8192 * 3072,
        "ffn_gemm1": t_gemm * ops["ffn_gemm1"]["flops"],
        "ffn_requantize": t_q * 8192 * 14336,
        "ffn_gemm2": t_gemm * ops["ffn_gemm2"]["flops"],
        "kv_write": t_kvw * 7040 * 24 * 128,
        "kv_read": t_kvr * 68 * 30,
    }
    step = sum(est.values())
    roof = sum(roofline_seconds(o) for o in ops.values())

    # the rows measured beside the step: oracle per-unit times on small samples
    from oracle import adaln as A
    from oracle import training as T
    from oracle import window as W
    nxt_ops = next_op_table()
    qa = F.bf16_bits_to_f64(synth.attn_queries(32, 24, 128, seed=50))
    t = time.perf_counter()
    KV.attention(pool, 0, list(range(kv_pages)), kv_tok - 256 * (kv_pages - 1), qa,
                 1 / 128 ** 0.5)
    t_attn = (time.perf_counter() - t) / (4 * 32 * kv_tok * 128 * 24)   # per FLOP
    d = synth.adaln_input(m=256, k=3072)
    xa = F.bf16_bits_to_f64(d["x"])
    t = time.perf_counter()
    A.adaln_quantize(xa, d["shift"][:1].astype(np.float64), d["scale"][:1].astype(np.float64),
                     880, 1e-6)
    t_ln = (time.perf_counter() - t) / xa.size
    t = time.perf_counter()
    T.quantize_transposed(x[:1024])
    t_qt = (time.perf_counter() - t) / (1024 * 3072)
    t = time.perf_counter()
    W.window_pages(65536, 256, 1024, 0, 0, 16384)
    t_win = time.perf_counter() - t
    nxt = {
        "kv_attention": t_attn * nxt_ops["kv_attention"]["flops"],
        "wgrad_quantize_t": t_qt * 8192 * 14336,
        "wgrad_gemm": t_gemm * nxt_ops["wgrad_gemm"]["flops"],
        "adaln_quantize": t_ln * 8192 * 3072,
        "window_pages": t_win,
    }
    return {
        "value": 100.0 * roof / step,
        "unit": "% of MI355X roofline (whole step, extrapolated)",
        "cores": int(blas_threads),
        "host_cores": host_cores,
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": (f"oracle timed on {q_rows}x3072 activation rows (quantize, bf16 dequantize), a "
                   f"{g_rows}x3072x3072 exact GEMM, a {kv_tok}-token KV chunk write and "
                   f"{kv_pages} KV pages read; "
                   "per-unit times scaled to the full step; elementwise numpy is single-"
                   "threaded, the GEMM's fp64 BLAS uses `cores` threads of the `host_cores` "
                   "cores available to the process; the rows beside "
                   "the step: attention of 32 queries over those 28 pages, LayerNorm + adaLN + "
                   "NVFP4 of 256 x 3072, transposed quantize of 1024 x 3072, the exact GEMM's "
                   "per-FLOP time, and the whole window page list"),
        "step_seconds_estimate": step,
        "next_ops_seconds_estimate": nxt,
    }


def cpu_model():
    """The host CPU's model name (Linux /proc/cpuinfo), or the platform's processor string."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


# ------------------------------------------------------------------ measured traffic

def source_sha256(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic():
    """HBM bytes of one FFN GEMM1 launch from the committed counter summary, or
    None when it is missing or was taken with a different GEMM source."""
    try:
        fields = {}
        with open(TRAFFIC_FILE) as f:
            for line in f:
                if line.startswith("- ") and ":" in line:
                    k, v = line[2:].split(":", 1)
                    fields[k.strip()] = v.strip().strip("`")
        if fields.get("gemm.hip sha256") != source_sha256(GEMM_SOURCE):
            return None
        return int(fields["HBM bytes per launch"])
    except (OSError, KeyError, ValueError):
        return None


def run_only(name, reps, warmup):
    import torch
    wl = Workload(torch.device("cuda", 0), groups=Workload.NEEDS[name])
    fn = dict(wl.ops() + wl.next_ops())[name]
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        fn()
    torch.cuda.synchronize()
    print(json.dumps({"op": name, "reps": reps,
                      "ms_per_rep": round((time.perf_counter() - t0) / reps * 1e3, 4)}), flush=True)


def run_copy(nbytes, reps):
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "reps": reps}), flush=True)


# ------------------------------------------------------------------ main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default=None, help="run one op of the step (profiling)")
    ap.add_argument("--copy-bytes", type=int, default=0, help="plain copy (counter calibration)")
    ap.add_argument("--reps", type=int, default=5)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the hot path runs on one MI355X; see the sharding notes).", file=sys.stderr)
        sys.exit(2)
    if args.copy_bytes:
        run_copy(args.copy_bytes, args.reps)
        return
    if args.only:
        run_only(args.only, args.reps, args.warmup)
        return

    ops = op_table()
    wall, per_op, hot, nxt, copy_bps = run_gpu(args.steps, args.warmup)
    roof = sum(roofline_seconds(o) for o in ops.values())

    per = {}
    for n, o in ops.items():
        s = per_op[n]
        rec = {"ms": round(s * 1e3, 4), "roofline_frac": round(roofline_seconds(o) / s, 4),
               "hot_ms": round(hot[n] * 1e3, 4)}
        if "flops" in o:
            rec["tflops"] = round(o["flops"] / s / 1e12, 2)
        else:
            rec["gbps"] = round(o["bytes"] / s / 1e9, 1)
            rec["copy_frac"] = round(o["bytes"] / s / copy_bps, 4)
        if "compressed_bytes" in o:
            rec["gbps_compressed_read"] = round(o["compressed_bytes"] / s / 1e9, 1)
        per[n] = rec

    nxt_rec = {}
    for n, o in next_op_table().items():
        t = nxt[n]
        rec = {"ms": round(t * 1e3, 4), "workload": o["workload"], "in_step": False}
        if o.get("launch_bound"):
            rec["us_per_call"] = round(t * 1e6, 2)           # no meaningful roofline
        elif "flops" in o:
            rec["roofline_frac"] = round(roofline_seconds(o) / t, 4)
            rec["tflops"] = round(o["flops"] / t / 1e12, 2)
        else:
            rec["roofline_frac"] = round(roofline_seconds(o) / t, 4)
            rec["gbps"] = round(o["bytes"] / t / 1e9, 1)
        nxt_rec[n] = rec

    g1 = per_op["ffn_gemm1"]
    line = {
        "metric": METRIC,
        "value": round(100.0 * roof / wall, 3),
        "unit": "% of MI355X roofline (whole step)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": ("DiT block hot path: attn proj quantize+GEMM 4096x3072x3072, dequantize, "
                         "FFN pair 8192x3072->14336->3072 with requant, KV chunk write "
                         "7040x24x128, KV window read 30 layers x 68 pages of 256 tokens"),
            "roofline_seconds_per_step": roof,
        },
        "roofline": {
            "kernel": "gemm_w4a4_kernel (FFN GEMM1 launch, M8192 N14336 K3072, fp16 MFMA, bf16 out)",
            "bound": "mfma",
            "achieved": round(ops["ffn_gemm1"]["flops"] / g1 / 1e12, 2),
            "peak": MFMA_F16_FLOPS / 1e12,
            "unit": "TFLOP/s",
            "frac": round(ops["ffn_gemm1"]["flops"] / g1 / MFMA_F16_FLOPS, 4),
            "traffic": measured_traffic(),
        },
        "hbm_copy_gbps": round(copy_bps / 1e9, 1),
        "per_op": per,
        "next_ops": nxt_rec,
    }
    if not args.no_cpu_baseline:
        cb = cpu_baseline(ops)
        for n, t_cpu in cb.pop("next_ops_seconds_estimate").items():
            if n in nxt_rec:
                nxt_rec[n]["oracle_seconds_estimate"] = t_cpu
                nxt_rec[n]["gpu_speedup_vs_oracle"] = round(t_cpu / nxt[n], 1)
        line["cpu_baseline"] = cb
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
