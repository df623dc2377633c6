"""bfloat16 bit patterns -> float64 (exact). Oracle-only helper."""
import numpy as np


def to_f64(bits: np.ndarray) -> np.ndarray:
    """A bf16 value is the top 16 bits of the float32 with the same value."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def to_f32(bits: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)
