"""Helpers for the GPU parity tests: numpy <-> device tensors, sentinels."""
import sys

import numpy as np
import torch

DEV = "cuda:0"


def note(msg: str) -> None:
    """Name the case before a GPU step (flushed, so a crash still shows it)."""
    print(f"[gpu] {msg}", file=sys.stderr, flush=True)


def bf16_dev(x_bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def i32_dev(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, np.int32))).to(DEV)


def u8_dev(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, np.uint8))).to(DEV)


def filled_u8(shape, value=0xA5) -> torch.Tensor:
    return torch.full(shape, value, dtype=torch.uint8, device=DEV)


def filled_f32(shape, value=-7.0) -> torch.Tensor:
    return torch.full(shape, value, dtype=torch.float32, device=DEV)


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def assert_bytes_equal(got: np.ndarray, ref: np.ndarray, what: str) -> None:
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    if not np.array_equal(got, ref):
        bad = np.argwhere(got != ref)
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} mismatches; first at {i}: got {got[i]!r} ref {ref[i]!r}")


def assert_f32_bits_equal(got: np.ndarray, ref: np.ndarray, what: str) -> None:
    assert_bytes_equal(np.asarray(got, np.float32).view(np.uint32), np.asarray(ref, np.float32).view(np.uint32),
                       what)


def e8m0_rows_to_k4(sc: np.ndarray) -> np.ndarray:
    """Row-major e8m0 scales [R, NB] in the K4 layout of include/fp8moe.h: [ceil(NB/4), R, 4], byte
    (r, b) at [b // 4, r, b % 4], the bytes past block NB - 1 of a row zero."""
    R, NB = sc.shape
    G = (NB + 3) // 4
    padded = np.zeros((R, 4 * G), np.uint8)
    padded[:, :NB] = sc
    return np.ascontiguousarray(padded.reshape(R, G, 4).transpose(1, 0, 2))


def ulp_key(bits: np.ndarray) -> np.ndarray:
    """bf16 bits -> integers ordered like the values (both zeros -> 0)."""
    b = bits.astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def assert_within_one_ulp(got: np.ndarray, ref: np.ndarray, what: str) -> None:
    """bf16 results of an fp32 evaluation with its own exponential against the exact values rounded
    once: at most one bf16 ulp apart, on at most a fraction 2^-11 of the elements (at least one
    allowed).  The fraction: the fp32 evaluation (exponential, add, divide and up to six products
    and sums) stays within a relative error eps = 2^-20 of the exact value; an element flips only if
    its exact value v lies within eps*v of a bf16 rounding midpoint, and with the bf16 spacing
    h > v*2^-8 that happens for a fraction at most 2*eps*v/h < 2^-11 of values spread over the
    spacing."""
    import math
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    d = np.abs(ulp_key(got) - ulp_key(ref))
    if d.size:
        i = np.unravel_index(np.argmax(d), d.shape)
        assert d.max() <= 1, f"{what}: {int((d > 1).sum())} elements beyond 1 bf16 ulp; worst at {i}: " \
                             f"got {got[i]:#06x} ref {ref[i]:#06x}"
        note(f"{what}: {int((d > 0).sum())} of {d.size} elements one bf16 ulp off ({(d > 0).mean():.3e})")
        allowed = math.ceil(d.size * 2.0 ** -11)
        assert int((d > 0).sum()) <= allowed, \
            f"{what}: {int((d > 0).sum())} elements off by one ulp, more than {allowed} ({d.size} * 2^-11)"
