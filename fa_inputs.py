"""Seeded synthetic inputs for attention forward, shared by the oracle tests,
the GPU parity tests and the bench.

This module draws random numbers and rounds them to the storage dtype. It
holds none of the attention arithmetic, so both the HIP path and the CPU
oracle can consume its tensors without sharing any of the method.

Recipe (the pages build every workload with ``torch.randn`` and state no
seed; see "How to optimise a Triton FlashAttention-2 kernel step by step with
a profiler", "A small program to profile" and "The sweep"):

* a CPU ``torch.Generator`` seeded with ``seed``;
* fp32 standard-normal draws for q, then k, then v, each of shape
  ``[B, H, N, d]`` (contiguous, row-major);
* each rounded to the storage dtype with ``Tensor.to`` (round to nearest even;
  fp32 keeps the draws as they are);
* for the heavy-tailed variant, q is multiplied by ``q_scale`` after rounding.
  A power-of-two ``q_scale`` (4 for the long-context case) is exact in
  fp16/bf16 at these magnitudes.
"""

import torch

DTYPES = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}


def as_torch_dtype(dtype):
    if isinstance(dtype, torch.dtype):
        return dtype
    return DTYPES[dtype]


def make_qkv(B, H, N, d, dtype, seed, q_scale=1.0):
    """Return CPU tensors ``(q, k, v)`` of shape ``[B, H, N, d]`` in ``dtype``."""
    dt = as_torch_dtype(dtype)
    g = torch.Generator().manual_seed(int(seed))
    shape = (B, H, N, d)
    q = torch.randn(shape, generator=g, dtype=torch.float32).to(dt)
    k = torch.randn(shape, generator=g, dtype=torch.float32).to(dt)
    v = torch.randn(shape, generator=g, dtype=torch.float32).to(dt)
    if q_scale != 1.0:
        q = (q.float() * float(q_scale)).to(dt)
    return q, k, v


def sample_rows(N, head=128, tail=128, stride=97):
    """Deterministic row subset of a length-``N`` sequence: the first ``head``
    rows, the last ``tail`` rows and every ``stride``-th row, sorted and unique.
    Used where a full oracle pass at a large size would take too long."""
    rows = set(range(min(head, N)))
    rows.update(range(max(0, N - tail), N))
    rows.update(range(0, N, stride))
    return sorted(rows)
