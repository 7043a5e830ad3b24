"""Seeded synthetic workloads shared by the tests, the bench and the oracle checks.

This module holds shapes and random-number recipes only. It contains none of
the attention arithmetic, so both sides of a parity check (the fp64 CPU oracle
and the HIP library) can draw identical inputs from it without sharing code.

Recipes
-------
* ``tiny_fp32``: the worked example printed on "ALiBi in Attention: Complete
  Implementation" (mbrenndoerfer.com), section with the seed-42 test: legacy
  ``np.random.seed(42)``, then ``randn(4, 8, 16) * 0.5`` for Q, K and V in that
  order, fp32 on the device.
* bf16 forward workloads: ``np.random.default_rng(seed)`` drawing fp32 standard
  normals for q, then k, then v; each is rounded to bf16 by round-to-nearest-even
  (torch's ``.to(torch.bfloat16)``).
* decode workload: the 16 GiB KV cache is too large to draw on the host, so it
  is drawn on the device by a seeded ``torch.Generator``; the oracle receives
  copies of the same device values.
"""
from __future__ import annotations

import dataclasses

import numpy as np


@dataclasses.dataclass(frozen=True)
class FwdWorkload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str  # "f32" or "bf16"
    causal: bool = True
    seed: int = 42

    @property
    def shape(self):
        return (self.B, self.H, self.N, self.d)


@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    name: str
    B: int
    H: int
    L: int
    d: int
    seed: int = 42


# The five workloads of the ALiBi attention hot path plus the N=4096, d=128
# performance shape. Sizes follow the pages' workloads: the 4-head, 8-token,
# 16-dim seed-42 example; an 8-head 1024-token layer; a 12-head, 768-wide
# decoder layer at 2048 tokens; 16 heads at the extrapolated 16384-token
# length; and a 32x32-head decode step over a 32768-token KV cache.
TINY_FP32 = FwdWorkload("tiny_fp32_B1_H4_N8_d16", 1, 4, 8, 16, "f32")
FWD_B8_H8_N1024_D64 = FwdWorkload("fwd_bf16_B8_H8_N1024_d64", 8, 8, 1024, 64, "bf16")
FWD_B4_H12_N2048_D64 = FwdWorkload("fwd_bf16_B4_H12_N2048_d64", 4, 12, 2048, 64, "bf16")
FWD_B1_H16_N16384_D128 = FwdWorkload("fwd_bf16_B1_H16_N16384_d128", 1, 16, 16384, 128, "bf16")
FWD_B8_H16_N4096_D128 = FwdWorkload("fwd_bf16_B8_H16_N4096_d128", 8, 16, 4096, 128, "bf16")
DECODE_B32_H32_L32768_D128 = DecodeWorkload("decode_bf16_B32_H32_L32768_d128", 32, 32, 32768, 128)

FWD_WORKLOADS = [FWD_B8_H8_N1024_D64, FWD_B4_H12_N2048_D64, FWD_B1_H16_N16384_D128,
                 FWD_B8_H16_N4096_D128]


def tiny_example_qkv():
    """Q, K, V of the printed seed-42 example, as fp32 arrays of shape (4, 8, 16)."""
    rs = np.random.RandomState(42)
    q = rs.randn(4, 8, 16) * 0.5
    k = rs.randn(4, 8, 16) * 0.5
    v = rs.randn(4, 8, 16) * 0.5
    return q.astype(np.float32), k.astype(np.float32), v.astype(np.float32)


def tiny_example_qkv_f64():
    """The same draw as :func:`tiny_example_qkv` but kept in fp64 (the page's own precision)."""
    rs = np.random.RandomState(42)
    q = rs.randn(4, 8, 16) * 0.5
    k = rs.randn(4, 8, 16) * 0.5
    v = rs.randn(4, 8, 16) * 0.5
    return q, k, v


def gaussian_f32(shape, seed, scale=1.0):
    """One fp32 standard-normal array from ``default_rng(seed)``."""
    rng = np.random.default_rng(seed)
    return (rng.standard_normal(shape, dtype=np.float32) * np.float32(scale)).astype(np.float32)


def gaussian_qkv_f32(shape, seed=42, scale=1.0, kv_shape=None):
    """q, then k, then v from one ``default_rng(seed)`` stream, fp32."""
    rng = np.random.default_rng(seed)
    kv_shape = shape if kv_shape is None else kv_shape
    q = rng.standard_normal(shape, dtype=np.float32) * np.float32(scale)
    k = rng.standard_normal(kv_shape, dtype=np.float32) * np.float32(scale)
    v = rng.standard_normal(kv_shape, dtype=np.float32) * np.float32(scale)
    return q, k, v


def to_bf16_tensor(a):
    """fp32 numpy array -> torch bf16 CPU tensor (round to nearest even)."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def gaussian_qkv_bf16(shape, seed=42, scale=1.0, kv_shape=None):
    """bf16 (torch CPU tensors) q, k, v by the default_rng recipe."""
    q, k, v = gaussian_qkv_f32(shape, seed, scale, kv_shape)
    return to_bf16_tensor(q), to_bf16_tensor(k), to_bf16_tensor(v)


def device_gaussian_bf16(shape, seed, device="cuda"):
    """A bf16 standard-normal tensor drawn on the device by a seeded torch.Generator.

    Used for the KV cache of the decode workload, which is too large to draw on
    the host. The draw is fp32 then rounded to bf16 (round to nearest even).
    """
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    # Fill in slabs so the fp32 temporary stays small.
    flat = out.view(shape[0], -1)
    for b in range(shape[0]):
        flat[b].copy_(torch.randn(flat.shape[1], generator=g, device=device, dtype=torch.float32))
    return out
