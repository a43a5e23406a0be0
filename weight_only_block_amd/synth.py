"""Seeded synthetic inputs for the block-quantized decode GEMV.

This module only draws random numbers and stores them in the canonical input
formats (int8 codes; 4-bit codes packed two per byte with the even element in
the low nibble; fp16 and bf16 bit patterns rounded to nearest even).  It holds
none of the GEMV's arithmetic and is the one piece of code that both the HIP
path's tests/benchmarks and the CPU oracle consume.

Workload shapes (decode, one token, weights stored row-major [N][K]):
  q8_small      Q8G64 N=K=1024
  qwen3_0.6b    Q8G64 hidden 1024: q 1024->2048, k/v 1024->1024, o 2048->1024,
                gate/up 1024->3072, down 3072->1024
  q4_k2560      Q4G32 gate/up 2560->9216, down 9216->2560, m = 1 and 4
  lm_head       Q8G64 K=2560, N=151936 (vocabulary rows)
  moe_experts   Q4G32, 128 experts, gate/up 4096->1536, down 1536->4096,
                8 distinct expert ids per token
  lm_head_q8g128  the lm_head in Q8G128
  w8a16_qwen3_14b_tp4  per-output-channel int8 (fp32 row scale) at Qwen3-14B
                TP4 rank-local shapes
Value distributions: int8 codes uniform in [-127, 127]; 4-bit codes uniform
in 0..15; scales uniform in [1e-3, 2e-2] then fp16; Q4 mins uniform in
[-0.1, 0] then fp16; activations N(0, 1) float32 then bf16.
"""
from __future__ import annotations

import numpy as np

Q8_GROUP = 64
Q4_GROUP = 32


def rng_for(*key: int) -> np.random.Generator:
    """Independent stream per (workload, matrix, ...) key."""
    return np.random.default_rng(list(key))


def to_fp16_bits(values) -> np.ndarray:
    """float -> IEEE binary16 bit patterns (numpy rounds to nearest even)."""
    return np.asarray(values, dtype=np.float32).astype(np.float16).view(np.uint16)


def to_bf16_bits(values) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even on the bits.
    Inputs here are finite, so no NaN special case is needed."""
    u = np.ascontiguousarray(values, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def pack_nibbles(c: np.ndarray) -> np.ndarray:
    """[..., K] codes 0..15 -> [..., K/2] bytes, even k in the low nibble."""
    c = np.asarray(c, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def q8g64_weights(rng: np.random.Generator, N: int, K: int):
    """(q [N][K] int8 in [-127,127], scale [N][K/64] fp16 bits)."""
    q = rng.integers(-127, 128, size=(N, K), dtype=np.int8)
    s = to_fp16_bits(rng.uniform(1e-3, 2e-2, size=(N, K // Q8_GROUP)))
    return q, s


def q8g128_weights(rng: np.random.Generator, N: int, K: int):
    """(q [N][K] int8 in [-127,127], scale [N][K/128] fp16 bits)."""
    q = rng.integers(-127, 128, size=(N, K), dtype=np.int8)
    s = to_fp16_bits(rng.uniform(1e-3, 2e-2, size=(N, K // 128)))
    return q, s


def q8pc_weights(rng: np.random.Generator, N: int, K: int):
    """(q [N][K] int8 in [-127,127], scale [N] as fp32 bit patterns).  A
    per-output-channel symmetric scale spans the row's whole range, so it is
    drawn from the same interval as the group scales."""
    q = rng.integers(-127, 128, size=(N, K), dtype=np.int8)
    s = rng.uniform(1e-3, 2e-2, size=N).astype(np.float32).view(np.uint32)
    return q, s


def q4g32_weights(rng: np.random.Generator, N: int, K: int):
    """(codes [N][K/2] packed, scale [N][K/32] fp16 bits, min [N][K/32] fp16 bits)."""
    c = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    codes = pack_nibbles(c)
    del c
    s = to_fp16_bits(rng.uniform(1e-3, 2e-2, size=(N, K // Q4_GROUP)))
    mn = to_fp16_bits(rng.uniform(-0.1, 0.0, size=(N, K // Q4_GROUP)))
    return codes, s, mn


def activations(rng: np.random.Generator, m: int, K: int) -> np.ndarray:
    """[m][K] bf16 bits drawn from N(0, 1)."""
    return to_bf16_bits(rng.standard_normal(size=(m, K), dtype=np.float32))


def expert_ids(rng: np.random.Generator, n_experts: int = 128, n_slots: int = 8) -> np.ndarray:
    """Distinct expert ids, uniform without replacement (int32)."""
    return rng.choice(n_experts, size=n_slots, replace=False).astype(np.int32)


# Workload catalogue: name -> list of matrices (label, format, N, K).
QWEN3_06B_LAYER = [
    ("q", "q8g64", 2048, 1024),
    ("k", "q8g64", 1024, 1024),
    ("v", "q8g64", 1024, 1024),
    ("o", "q8g64", 1024, 2048),
    ("gate", "q8g64", 3072, 1024),
    ("up", "q8g64", 3072, 1024),
    ("down", "q8g64", 1024, 3072),
]
Q4_K2560 = [
    ("gate", "q4g32", 9216, 2560),
    ("up", "q4g32", 9216, 2560),
    ("down", "q4g32", 2560, 9216),
]
LM_HEAD = ("lm_head", "q8g64", 151936, 2560)
# Per-output-channel W8A16 at Qwen3-14B TP4 rank-local decode shapes:
# QKV 5120->1792, O 1280->5120, gate/up 5120->8704, down 4352->5120.
W8A16_QWEN3_14B_TP4 = [
    ("qkv", "q8pc", 1792, 5120),
    ("o", "q8pc", 5120, 1280),
    ("gate", "q8pc", 8704, 5120),
    ("up", "q8pc", 8704, 5120),
    ("down", "q8pc", 5120, 4352),
]
MOE = {"n_experts": 128, "n_slots": 8,
       "gate": (1536, 4096), "up": (1536, 4096), "down": (4096, 1536)}

WORKLOAD_IDS = {"q8_small": 0, "qwen3_0.6b": 1, "q4_k2560": 2, "lm_head": 3, "moe_experts": 4,
                "lm_head_q8g128": 5, "w8a16_qwen3_14b_tp4": 6}


def bytes_q8g64(N: int, K: int) -> int:
    """Algorithmic weight bytes: int8 codes plus one fp16 scale per 64."""
    return N * K + 2 * N * (K // Q8_GROUP)


def bytes_q8g128(N: int, K: int) -> int:
    """Algorithmic weight bytes: int8 codes plus one fp16 scale per 128."""
    return N * K + 2 * N * (K // 128)


def bytes_q8pc(N: int, K: int) -> int:
    """Algorithmic weight bytes: int8 codes plus one fp32 scale per row."""
    return N * K + 4 * N


def bytes_q4g32(N: int, K: int) -> int:
    """Algorithmic weight bytes: packed nibbles plus fp16 scale and min per 32."""
    return N * K // 2 + 4 * N * (K // Q4_GROUP)
