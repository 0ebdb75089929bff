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
