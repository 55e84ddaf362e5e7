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


# ------------------------------------------------------------ parity rates
# (config, direction, layout) -> merged oracle.parity.Stats of every fused
# comparison recorded in this session; printed at the end of the run (and
# written as JSON to $MXFP8_PARITY_RATES when that is set) by conftest.py.
PARITY_RATES = {}


def record_rates(config: str, direction: str, st) -> None:
    from oracle.parity import layout_parts

    for lay, part in layout_parts(st).items():
        key = (config, direction, lay)
        PARITY_RATES[key] = PARITY_RATES[key].merge(part) if key in PARITY_RATES else part
