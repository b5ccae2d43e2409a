"""Shared helpers of the GPU parity tests: moving seeded inputs to the device and
reading the library's outputs back into the oracle's representation."""

import numpy as np
import torch

from oracle import formats as F
from oracle import nvfp4 as Q


def dev():
    return torch.device("cuda", 0)


def bf16_tensor(bits: np.ndarray) -> torch.Tensor:
    """bf16 bit patterns (uint16 numpy) -> bf16 CUDA tensor."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to(dev())


def f32_tensor(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev())


def to_oracle(t) -> Q.NVFP4:
    """Library NVFP4Tensor -> oracle NVFP4 (row-major scales)."""
    torch.cuda.synchronize()
    packed = t.codes.cpu().numpy()
    flat = t.scales.cpu().numpy()
    sc = Q.unlayout_scales(flat, t.rows, t.cols, t.layout)
    return Q.NVFP4(packed, sc, float(t.global_scale.cpu().numpy()[0]))


def from_oracle(q: Q.NVFP4, layout):
    """Oracle NVFP4 -> library NVFP4Tensor on the device (same bytes)."""
    import w4a4_gemm_amd as nv
    rows, cols = q.shape
    return nv.NVFP4Tensor(
        rows, cols, layout,
        codes=torch.from_numpy(np.ascontiguousarray(q.packed)).to(dev()),
        scales=torch.from_numpy(q.scales_in(layout)).to(dev()),
        global_scale=torch.tensor([q.s_g], dtype=torch.float32, device=dev()))


def assert_same_nvfp4(got: Q.NVFP4, want: Q.NVFP4):
    assert got.s_g == want.s_g, f"s_g {got.s_g!r} != {want.s_g!r}"
    bad_s = np.argwhere(got.scales != want.scales)
    assert bad_s.size == 0, f"{len(bad_s)} scale bytes differ, first at {bad_s[:3].tolist()}"
    bad_c = np.argwhere(got.packed != want.packed)
    assert bad_c.size == 0, f"{len(bad_c)} code bytes differ, first at {bad_c[:3].tolist()}"


def bf16_out_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def f64_of_bits(bits):
    return F.bf16_bits_to_f64(bits)
