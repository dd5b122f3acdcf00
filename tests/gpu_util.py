"""Helpers for the GPU parity tests: host<->device moves, poison guards, and
the comparison rules for floating-point outputs."""
import sys

import numpy as np
import pytest
import torch

from oracle import f32_to_bf16_bits_ref, bf16_bits_to_f32_ref

POISON_BYTE = 0x7F


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def say(msg):
    """Name the case on stdout before a GPU step, so a crash log shows it."""
    print(msg, flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


def dev(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


class Guarded:
    """An output tensor with poisoned guard bands on both sides.

    The view handed to the kernel is contiguous and 256-byte aligned; after the
    call, `check()` asserts the guard bands still hold the poison and returns
    the view's contents (every in-range element must have been overwritten,
    which the value comparison then shows)."""

    def __init__(self, shape, dtype, device, guard_bytes=4096):
        esize = torch.empty((), dtype=dtype).element_size()
        self.n = int(np.prod(shape))
        self.g = guard_bytes // esize
        raw = torch.full(((self.n + 2 * self.g) * esize,), POISON_BYTE, dtype=torch.uint8,
                         device=device)
        self.buf = raw.view(dtype)
        self.view = self.buf[self.g:self.g + self.n].view(*shape)

    def check(self):
        b = self.buf.view(torch.uint8)
        esize = self.buf.element_size()
        head = b[: self.g * esize]
        tail = b[(self.g + self.n) * esize:]
        assert bool((head == POISON_BYTE).all()), "write before the output"
        assert bool((tail == POISON_BYTE).all()), "write past the output"
        return host(self.view)


def check_fp32(y32: np.ndarray, y64: np.ndarray, mag: np.ndarray, canon: np.ndarray, strict=True):
    """FP32 outputs: within 1e-5 of the magnitude sum (the reading of "1e-5
    relative" that stays meaningful under cancellation: it equals the plain
    relative error when the terms do not cancel), and, for the kernels that
    keep the stated group order, bit-identical to the oracle's float32 replay."""
    y32 = np.asarray(y32, np.float32)
    err = np.abs(y32.astype(np.float64) - y64)
    bad = err > 1e-5 * mag
    assert not bad.any(), f"{bad.sum()} elements beyond 1e-5*mag; worst {np.max(err / np.maximum(mag, 1e-300))}"
    if strict:
        neq = y32.view(np.uint32) != np.asarray(canon, np.float32).view(np.uint32)
        assert not neq.any(), f"{neq.sum()} of {neq.size} differ from the stated float32 order"


def check_bf16(yb: np.ndarray, y64: np.ndarray, mag: np.ndarray, canon: np.ndarray, strict=True):
    """BF16 outputs: equal to RNE(fl32(y64)) or one of its BF16 neighbours
    (1 ulp); where the terms cancel so far that float32 rounding alone exceeds
    that, |y - y64| <= 1e-5*mag + half a BF16 ulp. Strict: bit-identical to the
    oracle's float32 replay rounded to BF16."""
    yb = np.asarray(yb, np.uint16)
    ref = f32_to_bf16_bits_ref(y64.astype(np.float32)).astype(np.int32)
    # distance in BF16 ulps via the ordered integer encoding of the bit patterns
    def ordered(b):
        b = b.astype(np.int32)
        return np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF)
    ulps = np.abs(ordered(yb) - ordered(ref))
    yv = bf16_bits_to_f32_ref(yb).astype(np.float64)
    half_ulp = np.abs(bf16_bits_to_f32_ref(ref.astype(np.uint16)).astype(np.float64)) * 2.0 ** -8
    ok = (ulps <= 1) | (np.abs(yv - y64) <= 1e-5 * mag + half_ulp)
    assert ok.all(), f"{(~ok).sum()} BF16 outputs beyond 1 ulp"
    if strict:
        neq = yb != np.asarray(canon, np.uint16)
        assert not neq.any(), f"{neq.sum()} of {neq.size} BF16 outputs differ from the stated order"
