"""Small numpy/torch conversions shared by the tests (no method arithmetic)."""
import numpy as np
import torch


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def torch_bf16_to_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def bits_to_torch_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)


def all_bf16_bits() -> np.ndarray:
    return np.arange(65536, dtype=np.uint32).astype(np.uint16)


def e4m3_ordinal(codes: np.ndarray) -> np.ndarray:
    """Signed position of an E4M3 code on the number line (+0 and -0 both 0)."""
    c = codes.astype(np.int32)
    mag = c & 0x7F
    return np.where(c & 0x80, -mag, mag)
