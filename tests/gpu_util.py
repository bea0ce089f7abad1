"""Helpers for the GPU parity tests: device upload, guarded outputs, tolerance checks.

Inputs come from synth/ (seeded), expected values from oracle/ only; the HIP path
is reached through the gemm_affine_u4_amd binding of the C ABI."""
from __future__ import annotations

import sys

import numpy as np
import torch

GUARD = 2048          # sentinel elements on each side of every output
SENTINEL_BF16 = 0x7FC1
SENTINEL_F32 = np.float32(np.nan).view(np.uint32) | np.uint32(0x1234)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint32:
        return torch.from_numpy(a.view(np.int32)).cuda()
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda()
    return torch.from_numpy(a).cuda()


def dev_weight(w):
    return dev(w.codes), dev(w.scales), dev(w.biases)


class Guarded:
    """An output buffer with sentinel bands on both sides; .t is the contiguous middle."""

    def __init__(self, shape, f32: bool):
        n = int(np.prod(shape))
        self.f32 = f32
        if f32:
            self.buf = torch.full((n + 2 * GUARD,), 0, dtype=torch.int32, device="cuda")
            self.buf.fill_(int(SENTINEL_F32.view(np.int32)))
            self.t = self.buf[GUARD:GUARD + n].view(torch.float32).view(shape)
        else:
            self.buf = torch.full((n + 2 * GUARD,), SENTINEL_BF16, dtype=torch.int16, device="cuda")
            self.t = self.buf[GUARD:GUARD + n].view(shape)
        self.n = n

    def poison(self):
        """Overwrite the payload with NaN patterns (stale values must not survive a call)."""
        if self.f32:
            self.buf[GUARD:GUARD + self.n].fill_(int(np.array(0x7FC00000, np.uint32).view(np.int32)))
        else:
            self.buf[GUARD:GUARD + self.n].fill_(0x7FC0)

    def check_guards(self):
        b = self.buf.cpu().numpy()
        want = int(SENTINEL_F32.view(np.int32)) if self.f32 else np.int16(SENTINEL_BF16)
        assert np.all(b[:GUARD] == want), "write below the output buffer"
        assert np.all(b[GUARD + self.n:] == want), "write past the output buffer"

    def values(self) -> np.ndarray:
        """fp32 values (f32 mode) or bf16 bit patterns (bf16 mode)."""
        self.check_guards()
        if self.f32:
            return self.t.cpu().numpy().astype(np.float64)
        return self.t.cpu().numpy().view(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def bf16_term(M: int, K: int, heavy_tailed: bool = False) -> bool:
    """Whether a check adds the oracle's bf16-weight term (`bf16_weights`): only where the
    prefill GEMM runs (M > 8), which rounds each dequantized weight to bf16, and only where
    the stated 1e-3 rule alone can be narrower than that one rounding: at short K (K < 512)
    for a few elements per million, and at any K where the terms of a row are heavy-tailed
    (fp8 e4m3 codes, whose values span 2^-9 .. 448, or activations spread over six decades):
    a few large terms then carry the sum and their rounding errors do not average out (seen
    with fp8 at K = 640: 1.08 times the stated rule, matching the bf16-weight product
    computed in fp64).  Elsewhere the rounding errors of a row largely cancel and every check
    uses the stated rule alone."""
    return M > 8 and (K < 512 or heavy_tailed)


def assert_within(gpu, ref, tol, what: str):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    tol = np.broadcast_to(np.asarray(tol, np.float64), ref.shape)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite GPU output"
    err = np.abs(gpu - ref)
    bad = err > tol
    if np.any(bad):
        i = np.flatnonzero(bad.ravel())[:5]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside tolerance; first idx {i.tolist()} "
                             f"gpu {gpu.ravel()[i].tolist()} ref {ref.ravel()[i].tolist()} "
                             f"tol {tol.ravel()[i].tolist()}")
    ratio = float(np.max(err / np.maximum(tol, 1e-300))) if err.size else 0.0
    say(f"  {what}: {err.size} values within tolerance (max err/tol = {ratio:.3g})")
    return ratio


def rne_bits_of(f32_values: np.ndarray) -> np.ndarray:
    """torch's fp32 -> bf16 cast of the GPU's own fp32 output (for the bf16 == RNE(fp32) check)."""
    t = torch.from_numpy(np.asarray(f32_values, np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
