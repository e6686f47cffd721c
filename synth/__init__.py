"""Seeded synthetic inputs for context-parallel attention workloads.

This module is shared by the fp64 oracle and by the GPU path, and by nothing
else of the method: it holds no attention, split or merge arithmetic. It only
turns (seed, tensor id, flat element index) into a number, and it describes
the workload shapes.

Generator definition (identical on every backend):

  mix(x)   for a 32-bit unsigned x:  x ^= x >> 16; x = (x * 0x21F0AAAD) mod 2^32;
                                     x ^= x >> 15; x = (x * 0x735A2D97) mod 2^32;
                                     x ^= x >> 15
  keys     k1 = mix(seed ^ 0x1B873593), k2 = mix(k1 ^ tensor_id), k3 = mix(k2 ^ 0x2545F491)
  element  i (int64 flat index into the tensor in its global, row-major order):
           h1 = mix(mix((i mod 2^32) ^ k2) ^ (i >> 32) ^ k3);  h2 = mix(h1 ^ k1)
           u  = lo16(h1) + hi16(h1) + lo16(h2) + hi16(h2)          (integer in [0, 262140])
           x  = fp32(u - 131070) * fp32(UNIT)                      (one fp32 multiply, RNE)
           value = x * scale  (scale a power of two, exact), then RNE to bf16 for bf16 tensors.

mix is the "lowbias32" integer hash published in C. Wellons' hash-prospector
(xorshift 16, multiply, xorshift 15, multiply, xorshift 15; first multiplier
0x21F0AAAD), with the top bit of its second multiplier cleared (0x735A2D97 in
place of 0xD35A2D97) so that the products below fit signed 64-bit integers.

u is a sum of four independent 16-bit uniforms (Irwin-Hall with n = 4), so x has
mean 0 and variance 1 and a near-normal shape with tails cut at about 3.46. Every
step is integer arithmetic or one correctly rounded fp32 multiply, so numpy on the
CPU and torch on the GPU produce the same bits; a CPU test checks numpy against
torch-on-CPU and a GPU test checks numpy against torch-on-GPU.

The multipliers are both below 2^31, so every product of a 32-bit value with
them stays below 2^63 and fits a signed 64-bit integer exactly (torch has no
unsigned 64-bit arithmetic).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

M32 = 0xFFFFFFFF
_C1 = 0x21F0AAAD
_C2 = 0x735A2D97
# 1 / sqrt(var(u)) with var(u) = (2^32 - 1) / 3, as an fp32 constant.
UNIT = np.float32(1.0 / math.sqrt((2.0 ** 32 - 1.0) / 3.0))

TENSOR_Q, TENSOR_K, TENSOR_V = 0, 1, 2


def _mix_int(x: int) -> int:
    x &= M32
    x ^= x >> 16
    x = (x * _C1) & M32
    x ^= x >> 15
    x = (x * _C2) & M32
    x ^= x >> 15
    return x


def _keys(seed: int, tensor_id: int):
    k1 = _mix_int(seed ^ 0x1B873593)
    k2 = _mix_int(k1 ^ tensor_id)
    k3 = _mix_int(k2 ^ 0x2545F491)
    return k1, k2, k3


def _mix_np(x: np.ndarray) -> np.ndarray:
    # uint32 arithmetic wraps modulo 2^32, which is the definition above.
    x = x ^ (x >> np.uint32(16))
    x = x * np.uint32(_C1)
    x = x ^ (x >> np.uint32(15))
    x = x * np.uint32(_C2)
    x = x ^ (x >> np.uint32(15))
    return x


def _unit_from_index(i: np.ndarray, k1: int, k2: int, k3: int) -> np.ndarray:
    """Unit-variance fp32 values for an array of uint64 flat indices."""
    hi = (i >> np.uint64(32)).astype(np.uint32)
    lo = i.astype(np.uint32)            # low 32 bits
    h1 = _mix_np(_mix_np(lo ^ np.uint32(k2)) ^ hi ^ np.uint32(k3))
    h2 = _mix_np(h1 ^ np.uint32(k1))
    m16 = np.uint32(0xFFFF)
    u = ((h1 & m16).astype(np.int32) + (h1 >> np.uint32(16)).astype(np.int32)
         + (h2 & m16).astype(np.int32) + (h2 >> np.uint32(16)).astype(np.int32))
    return (u - 131070).astype(np.float32) * UNIT


def unit_values_np(seed: int, tensor_id: int, start: int, count: int) -> np.ndarray:
    """fp32 unit-variance values for flat indices [start, start + count)."""
    k1, k2, k3 = _keys(seed, tensor_id)
    out = np.empty(count, dtype=np.float32)
    step = 1 << 20
    for pos in range(0, count, step):
        n = min(step, count - pos)
        i = np.arange(n, dtype=np.uint64) + np.uint64(start + pos)
        out[pos:pos + n] = _unit_from_index(i, k1, k2, k3)
    return out


def values_at_np(seed: int, tensor_id: int, index: np.ndarray, scale: float, dtype: str) -> np.ndarray:
    """Values at arbitrary flat indices (any shape); same numbers as values_np."""
    k1, k2, k3 = _keys(seed, tensor_id)
    idx = np.asarray(index, dtype=np.int64)
    flat = idx.reshape(-1)
    x = np.empty(flat.size, dtype=np.float32)
    step = 1 << 20
    for pos in range(0, flat.size, step):
        x[pos:pos + step] = _unit_from_index(flat[pos:pos + step].astype(np.uint64), k1, k2, k3)
    x = x * np.float32(scale)
    if dtype == "bf16":
        return f32_to_bf16_bits(x).reshape(idx.shape)
    if dtype == "f32":
        return x.reshape(idx.shape)
    raise ValueError(f"unknown dtype {dtype!r}")


def head_slice_np(seed: int, tensor_id: int, shape: Sequence[int], head: int, scale: float, dtype: str,
                  row_start: int = 0, rows: Optional[int] = None) -> np.ndarray:
    """x[row_start:row_start+rows, head, :] of a synthetic [T, H, D] tensor, i.e.
    one head of a token-major tensor, as [rows, 1, D]."""
    T, H, D = (int(s) for s in shape)
    if rows is None:
        rows = T - row_start
    out = np.empty((rows, 1, D), dtype=np.uint16 if dtype == "bf16" else np.float32)
    step = max(1, (1 << 20) // D)
    d = np.arange(D, dtype=np.int64)
    for r0 in range(0, rows, step):
        r = np.arange(row_start + r0, row_start + min(rows, r0 + step), dtype=np.int64)
        idx = (r[:, None] * H + head) * D + d[None, :]
        out[r0:r0 + r.size, 0, :] = values_at_np(seed, tensor_id, idx, scale, dtype)
    return out


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 with round-to-nearest-even; returns the uint16 bit patterns.
    Inputs here are always finite."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def values_np(seed: int, tensor_id: int, start: int, count: int, scale: float, dtype: str) -> np.ndarray:
    """Flat slice of a synthetic tensor. dtype 'bf16' returns uint16 bit patterns,
    'f32' returns float32."""
    x = unit_values_np(seed, tensor_id, start, count) * np.float32(scale)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "f32":
        return x
    raise ValueError(f"unknown dtype {dtype!r}")


def tensor_np(seed: int, tensor_id: int, shape: Sequence[int], scale: float, dtype: str,
              row_start: int = 0, rows: Optional[int] = None) -> np.ndarray:
    """Rows [row_start, row_start + rows) of a synthetic tensor of the given full shape
    (row = first dimension), as numpy (uint16 bits for bf16)."""
    shape = tuple(int(s) for s in shape)
    inner = int(np.prod(shape[1:], dtype=np.int64)) if len(shape) > 1 else 1
    if rows is None:
        rows = shape[0] - row_start
    flat = values_np(seed, tensor_id, row_start * inner, rows * inner, scale, dtype)
    return flat.reshape((rows,) + shape[1:])


# ---------------------------------------------------------------- torch backend

def _mix_torch(x):
    x = x ^ (x >> 16)
    x = (x * _C1) & M32
    x = x ^ (x >> 15)
    x = (x * _C2) & M32
    x = x ^ (x >> 15)
    return x


def values_torch(seed: int, tensor_id: int, start: int, count: int, scale: float, dtype: str,
                 device, out=None, chunk: int = 1 << 27):
    """Same values as values_np, computed with torch int64 ops on `device`.
    Returns a 1-D torch tensor (bfloat16 or float32); fills `out` if given."""
    import torch
    k1, k2, k3 = _keys(seed, tensor_id)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    if dtype not in ("bf16", "f32"):
        raise ValueError(f"unknown dtype {dtype!r}")
    if out is None:
        out = torch.empty(count, dtype=tdt, device=device)
    unit = torch.tensor(float(UNIT), dtype=torch.float32, device=device)
    sc = torch.tensor(float(np.float32(scale)), dtype=torch.float32, device=device)
    pos = 0
    while pos < count:
        n = min(chunk, count - pos)
        i = torch.arange(start + pos, start + pos + n, dtype=torch.int64, device=device)
        lo = i & M32
        hi = i >> 32
        h1 = _mix_torch(_mix_torch(lo ^ k2) ^ hi ^ k3)
        h2 = _mix_torch(h1 ^ k1)
        u = (h1 & 0xFFFF) + (h1 >> 16) + (h2 & 0xFFFF) + (h2 >> 16)
        del i, lo, hi, h1, h2
        x = (u - 131070).to(torch.float32)
        del u
        x = torch.mul(x, unit)
        x = torch.mul(x, sc)
        out[pos:pos + n].copy_(x.to(tdt))
        del x
        pos += n
    return out


def tensor_torch(seed: int, tensor_id: int, shape: Sequence[int], scale: float, dtype: str,
                 device, row_start: int = 0, rows: Optional[int] = None):
    import torch
    shape = tuple(int(s) for s in shape)
    inner = int(np.prod(shape[1:], dtype=np.int64)) if len(shape) > 1 else 1
    if rows is None:
        rows = shape[0] - row_start
    flat = values_torch(seed, tensor_id, row_start * inner, rows * inner, scale, dtype, device)
    return flat.view((rows,) + shape[1:])


# ---------------------------------------------------------------- workloads

@dataclass
class PrefillWorkload:
    name: str
    seqlens: List[int]
    cp: int
    n_hq: int
    n_kv: int
    head_dim: int
    dtype: str          # 'f32' or 'bf16'
    scale_in: float     # multiplies the unit-variance values
    seed: int
    rank_only: Optional[int] = None   # None: every rank; r: only rank r's share is the workload

    @property
    def total_tokens(self) -> int:
        return int(sum(self.seqlens))

    @property
    def cu_seqlens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.seqlens)]).astype(np.int64)

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


@dataclass
class DecodeWorkload:
    name: str
    batch: int
    kv_len: int
    cp: int
    n_hq: int
    n_kv: int
    head_dim: int
    dtype: str
    scale_in: float
    seed: int

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


# Lengths of the packed varlen batch: six draws, uniform over the multiples of 8
# in [2048, 16384] (numpy default_rng(4).integers(256, 2049, 6) * 8, recorded here
# so the workload does not depend on numpy's generator version).
VARLEN_LENGTHS = [12464, 15568, 14688, 9376, 15536, 16048]

WORKLOADS = {
    "tiny": PrefillWorkload("tiny prefill S=256 cp=2 2 heads d64 fp32", [256], 2, 2, 2, 64, "f32", 1.0, 0),
    "gqa": PrefillWorkload("GQA prefill S=32768 cp=8 32q/8kv d128 bf16", [32768], 8, 32, 8, 128, "bf16", 0.5, 1),
    "long": PrefillWorkload("long-context prefill S=1048576 cp=8 rank 0 share 32q/8kv d128 bf16",
                            [1048576], 8, 32, 8, 128, "bf16", 0.5, 2, rank_only=0),
    "decode": DecodeWorkload("pass-Q decode b=8 kv_len=1048576 cp=8 32q/8kv d128 bf16",
                             8, 1048576, 8, 32, 8, 128, "bf16", 1.0, 3),
    "varlen": PrefillWorkload("wide-head varlen prefill 6 seqs cp=4 64 heads d512 bf16",
                              list(VARLEN_LENGTHS), 4, 64, 64, 512, "bf16", 0.5, 4),
}
