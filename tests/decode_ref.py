"""Independent decoders used by the oracle's pin tests.

These derive the formats from their bit-field definitions (OCP MX: e2m1 is a
minifloat with 1 sign, 2 exponent and 1 mantissa bit, exponent bias 1;
e8m0 is a biased exponent) and from torch's own float8_e8m0fnu cast. They are
written separately from the oracle's literal table so a wrong table entry,
sign or nibble order in either shows up as a mismatch.
"""
import numpy as np
import torch


def e2m1_from_bits(code: int) -> float:
    sign = -1.0 if (code >> 3) & 1 else 1.0
    exp = (code >> 1) & 0x3
    man = code & 0x1
    bias = 1
    if exp == 0:  # subnormal: 2^(1 - bias) * (man / 2)
        mag = 2.0 ** (1 - bias) * (man / 2.0)
    else:         # normal: 2^(exp - bias) * (1 + man / 2)
        mag = 2.0 ** (exp - bias) * (1.0 + man / 2.0)
    return sign * mag if mag != 0 else (-0.0 if sign < 0 else 0.0)


E2M1_TABLE = np.array([e2m1_from_bits(c) for c in range(16)], dtype=np.float64)


def e8m0_torch(b: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(b, dtype=np.uint8)).view(torch.float8_e8m0fnu)
    return t.to(torch.float32).numpy().astype(np.float64)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    """[..., K/2] bytes -> [..., K] codes, byte j -> (k = 2j low, 2j+1 high)."""
    lo = packed & 0x0F
    hi = packed >> 4
    return np.stack([lo, hi], axis=-1).reshape(*packed.shape[:-1], packed.shape[-1] * 2)


def dequant_mxfp4(w: np.ndarray, s: np.ndarray) -> np.ndarray:
    codes = unpack_nibbles(w)
    vals = E2M1_TABLE[codes]
    K = codes.shape[-1]
    scale = e8m0_torch(s).reshape(*s.shape[:-1], K // 32, 1)
    return (vals.reshape(*codes.shape[:-1], K // 32, 32) * scale).reshape(codes.shape)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(b, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


def dequant_int4g32(w: np.ndarray, s_bf16: np.ndarray) -> np.ndarray:
    codes = unpack_nibbles(w).astype(np.int64)
    q = np.where(codes >= 8, codes - 16, codes).astype(np.float64)
    K = codes.shape[-1]
    scale = bf16_bits_to_f64(s_bf16).reshape(*s_bf16.shape[:-1], K // 32, 1)
    return (q.reshape(*codes.shape[:-1], K // 32, 32) * scale).reshape(codes.shape)
