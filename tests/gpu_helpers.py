"""Shared helpers of the GPU parity tests: device transfer and the acceptance rules.

Acceptance (from the method's integer/float split):
  * int8 codes, scales, packed bytes, weight scales and int32 accumulators:
    bit-exact;
  * fp32 outputs: for every token row, max |y - y_ref| <= 1e-5 * max |y_ref|,
    and rows whose reference is all zero must be exactly zero;
  * bf16 outputs: the same rule with 8e-3.
"""
import numpy as np
import pytest
import torch

from bit_ternary_weight_amd import synth

F32_TOL = 1e-5
BF16_TOL = 8e-3

requires_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="no HIP device")


def dev():
    return torch.device("cuda:0")


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev()).view(torch.bfloat16)


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def f32_of_bf16(bits: np.ndarray) -> np.ndarray:
    return synth.bf16_to_f32(bits)


# Output guards.  Every output buffer a GPU test hands to the library is
# pre-filled with a byte pattern no correct result can hold, and is followed
# by a canary tail.  After the call, no element may still hold the pattern
# (an element never written) and the tail must be intact (no write past the
# end).  The patterns: NaN for fp32 / bf16 (0xFF bytes); 0x80 bytes for int8
# codes (-128 is unreachable: |x * a| < 127.5) and int32 accumulators
# (0x80808080: |A| <= 127 K is far below it); 0xFF for packed bytes (field
# value 3 is never produced).
_FILL = {torch.float32: 0xFF, torch.bfloat16: 0xFF, torch.int8: 0x80, torch.int32: 0x80, torch.uint8: 0xFF}
_TAIL = 512
_CANARY = 0xA5


class Guarded:
    """A device tensor of `shape` / `dtype` inside a pre-filled buffer with a
    canary tail (see above); .t is the tensor, .check() the assertions."""

    def __init__(self, shape, dtype, fill=None):
        n = 1
        for d in shape:
            n *= int(d)
        esz = torch.tensor([], dtype=dtype).element_size()
        self.nbytes = n * esz
        self.raw = torch.empty(self.nbytes + _TAIL, dtype=torch.uint8, device=dev())
        # fill: a byte of the caller's choosing for outputs where every byte
        # value is legal (the caller then compares runs with two fills); only
        # the tail is checked
        self.fill = fill
        self.raw[:self.nbytes].fill_(_FILL[dtype] if fill is None else fill)
        self.raw[self.nbytes:].fill_(_CANARY)
        self.dtype = dtype
        self.t = self.raw[:self.nbytes].view(dtype).view(*shape) if n else torch.empty(shape, dtype=dtype,
                                                                                        device=dev())

    def check(self, what="output"):
        tail = self.raw[self.nbytes:]
        assert bool((tail == _CANARY).all()), f"{what}: bytes written past the end of the buffer"
        if self.nbytes == 0 or self.fill is not None:
            return
        t = self.t
        if self.dtype in (torch.float32, torch.bfloat16):
            left = int(torch.isnan(t).sum())
        elif self.dtype == torch.int8:
            left = int((t == -128).sum())
        elif self.dtype == torch.int32:
            left = int((t == -2139062144).sum())
        else:
            left = int((t == 0xFF).sum())
        assert left == 0, f"{what}: {left} elements never written"


def guarded(shape, dtype=torch.float32, fill=None) -> Guarded:
    return Guarded(shape, dtype, fill)


def assert_rows_close(y: np.ndarray, ref: np.ndarray, tol: float, what: str = "y"):
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    assert y.shape == ref.shape, (y.shape, ref.shape)
    rmax = np.abs(ref).max(axis=1)
    err = np.abs(y - ref).max(axis=1)
    zero = rmax == 0
    assert (err[zero] == 0).all(), f"{what}: rows with all-zero reference are not exactly zero"
    bad = np.nonzero(err[~zero] > tol * rmax[~zero])[0]
    assert bad.size == 0, f"{what}: {bad.size} rows out of tolerance, worst rel {np.max(err[~zero] / rmax[~zero]):.3e}"


def max_ulp_diff(y: np.ndarray, ref: np.ndarray) -> int:
    a = np.ascontiguousarray(y, np.float32).view(np.int32).astype(np.int64)
    b = np.ascontiguousarray(ref, np.float32).view(np.int32).astype(np.int64)
    a = np.where(a < 0, -(a & 0x7FFFFFFF), a)
    b = np.where(b < 0, -(b & 0x7FFFFFFF), b)
    return int(np.abs(a - b).max()) if a.size else 0


def assert_exact(got: np.ndarray, ref: np.ndarray, what: str):
    got = np.asarray(got)
    ref = np.asarray(ref)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    if not np.array_equal(got, ref):
        idx = np.argwhere(got != ref)
        raise AssertionError(f"{what}: {idx.shape[0]} mismatches, first at {idx[0].tolist()}: "
                             f"got {got[tuple(idx[0])]} want {ref[tuple(idx[0])]}")
