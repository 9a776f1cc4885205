"""Tolerance checks shared by the GPU parity tests.

fp32 output:  max|Y_gpu - Y_ref| <= 1e-4 * rms(Y_ref)       (Y_ref: the float64 oracle)
bf16 output:  max(|Y_gpu - Y_ref| - ulp_bf16(Y_ref)/2) <= 1e-2 * rms(Y_ref)
              and Y_gpu,bf16 == RNE_bf16(Y_gpu,fp32) bit for bit where both exist.

The bf16 bound removes the half-ulp that rounding a perfect result to
bfloat16 already costs: with Gaussian outputs the largest |Y| sit in a binade
whose half-ulp exceeds 1e-2 * rms, so the plain bound would fail even for an
exactly rounded result.  The plain (literal) figure is still reported.
"""
import numpy as np
import torch

from oracle import tpf_oracle as O

F32_TOL = 1e-4
BF16_TOL = 1e-2


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().double().numpy()


def bits16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def rms(ref: np.ndarray) -> float:
    return float(np.sqrt(np.mean(np.square(ref)))) if ref.size else 0.0


def half_ulp_bf16(ref: np.ndarray) -> np.ndarray:
    _, e = np.frexp(ref)
    return np.ldexp(1.0, np.maximum(e - 9, -134))


def f32_error(got: torch.Tensor, ref: np.ndarray) -> float:
    d = np.abs(to_f64(got) - ref)
    r = rms(ref)
    return float(d.max() / r) if r > 0 else float(d.max())


def assert_f32(got: torch.Tensor, ref: np.ndarray, what: str = "") -> float:
    assert got.dtype == torch.float32
    err = f32_error(got, ref)
    assert err <= F32_TOL, f"{what}: fp32 max|d|/rms = {err:.3e} > {F32_TOL}"
    return err


def bf16_errors(got: torch.Tensor, ref: np.ndarray):
    d = np.abs(to_f64(got) - ref)
    r = rms(ref) or 1.0
    literal = float(d.max() / r)
    aware = float(np.max(d - half_ulp_bf16(ref)) / r)
    return literal, aware


def assert_bf16(got: torch.Tensor, ref: np.ndarray, what: str = ""):
    assert got.dtype == torch.bfloat16
    literal, aware = bf16_errors(got, ref)
    assert aware <= BF16_TOL, f"{what}: bf16 max(|d|-ulp/2)/rms = {aware:.3e} > {BF16_TOL} (literal {literal:.3e})"
    return literal, aware


def assert_bf16_is_rne_of_f32(got16: torch.Tensor, got32: torch.Tensor, what: str = ""):
    want = O.round_to_bf16_bits(to_f64(got32))
    have = bits16(got16)
    bad = int(np.count_nonzero(want != have))
    assert bad == 0, f"{what}: {bad} bf16 outputs differ from RNE of the fp32 output"


def assert_bitwise(a: torch.Tensor, b: torch.Tensor, what: str = ""):
    assert a.dtype == b.dtype and a.shape == b.shape, what
    ok = torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))
    if not ok:
        diff = int((a != b).sum())
        raise AssertionError(f"{what}: not bit-identical ({diff} elements differ)")
