"""Seeded generators for the KDA workloads.

The pages describe small-batch Kimi K3 decode (batch 1-64, an FP32 SSM cache,
speculative drafts verified and committed, mixed spec / non-spec batches) but
print no tensors. The five named workloads below are synthetic stand-ins with
the shapes of that decode path:

  tiny           B=1, H=4,  dk=dv=64,  256 sequential single-token steps, zero state
  b1_latency     B=1, H=32, dk=dv=128, 1024 sequential single-token steps, zero state
  b64_bandwidth  B=64, H=32, dk=dv=128, one single-token step, 256-slot cache
  spec_verify    B=16, H=32, dk=dv=128, 8 draft tokens each, 256-slot cache
  mixed          B=64 packed: 40 single-token rows then 24 rows of 4 tokens,
                 512-slot cache, output gate
  prefill_8k     B=1, H=32, dk=dv=128, one 8000-token prompt from a zero state
                 (the state after token 7680 is the checkpoint)

Draw order from ``numpy.random.Generator(PCG64(seed))`` (all float32 standard
normal unless noted), shaped ``[steps][n_tok][H][.]``:
  1. q_raw, k_raw, v, a_raw (last dim dk), b_raw (no last dim)
  2. gate (last dim dv), only when the output gate is on
  3. the state cache, N(0, std) float32, in slot chunks
  4. the slot permutation ``rng.permutation(num_slots)``
  5. accepted lengths ``rng.integers(1, T_b + 1)`` per row with T_b > 1
Derived inputs:
  k = k_raw / |k_raw|_2 ; q = q_raw / |q_raw|_2 / sqrt(dk)  (float64, then bf16 RNE)
  alpha = exp(-softplus(a_raw)) ; beta = sigmoid(b_raw)      (float64, then float32)
The raw projections themselves are kept too, for the raw-input mode: q_raw and
k_raw as bf16 (RNE of the float32 draws), a_raw and b_raw as float32.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); return the bit patterns."""
    a = np.ascontiguousarray(x, dtype=np.float32)
    if not np.all(np.isfinite(a)):
        raise ValueError("bf16 conversion expects finite inputs")
    u = a.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class Workload:
    """One seeded workload. Arrays are host numpy arrays in the library's layouts.

    q, k: uint16 bf16 bits [steps][n_tok][H][dk]; v: [steps][n_tok][H][dv]
    alpha: float32 [steps][n_tok][H][dk]; beta: float32 [steps][n_tok][H]
    gate: uint16 bf16 bits [steps][n_tok][H][dv] or None
    q_raw, k_raw: uint16 bf16 bits like q, k; a_raw: float32 like alpha; b_raw: like beta
    cache: float32 [num_slots][H][dv][dk] (value column j holds its dk key channels)
    slot_ids: int32 [B]; slot_tables: int32 [num_slots // B][B], disjoint, first == slot_ids
    cu_seqlens: int32 [B + 1]; accepted: int32 [B] (0 for rows with one token) or None
    """

    name: str
    B: int
    H: int
    dk: int
    dv: int
    steps: int
    cu_seqlens: np.ndarray
    T_max: int
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    alpha: np.ndarray
    beta: np.ndarray
    gate: Optional[np.ndarray]
    cache: np.ndarray
    slot_ids: np.ndarray
    slot_tables: np.ndarray
    accepted: Optional[np.ndarray]
    seed: int
    q_raw: Optional[np.ndarray] = None
    k_raw: Optional[np.ndarray] = None
    a_raw: Optional[np.ndarray] = None
    b_raw: Optional[np.ndarray] = None

    @property
    def n_tok(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def num_slots(self) -> int:
        return int(self.cache.shape[0])

    @property
    def seqlens(self) -> np.ndarray:
        return np.diff(self.cu_seqlens).astype(np.int32)


def make(B: int, H: int, dk: int, dv: int, *, seqlens=None, steps: int = 1,
         num_slots: Optional[int] = None, state_std: float = 0.0, gate: bool = False,
         seed: int = 0, name: str = "custom") -> Workload:
    """Draw a workload of the given shape (draw order in the module docstring).

    ``seqlens`` gives the tokens per row (default: one each); rows are packed
    contiguously in batch order. ``num_slots`` defaults to B.
    """
    if seqlens is None:
        seqlens = [1] * B
    seqlens = np.asarray(seqlens, dtype=np.int64)
    if seqlens.shape != (B,) or np.any(seqlens < 0):
        raise ValueError("seqlens must hold B non-negative lengths")
    cu = np.zeros(B + 1, dtype=np.int32)
    cu[1:] = np.cumsum(seqlens)
    n_tok = int(cu[-1])
    T_max = int(seqlens.max()) if B > 0 else 1
    if num_slots is None:
        num_slots = B
    if num_slots < B:
        raise ValueError("num_slots must be >= B")

    rng = np.random.Generator(np.random.PCG64(seed))
    lead = (steps, n_tok, H)
    q_raw = rng.standard_normal(lead + (dk,), dtype=np.float32)
    k_raw = rng.standard_normal(lead + (dk,), dtype=np.float32)
    v_raw = rng.standard_normal(lead + (dv,), dtype=np.float32)
    a_raw = rng.standard_normal(lead + (dk,), dtype=np.float32)
    b_raw = rng.standard_normal(lead, dtype=np.float32)
    g_raw = rng.standard_normal(lead + (dv,), dtype=np.float32) if gate else None

    cache = np.zeros((num_slots, H, dv, dk), dtype=np.float32)
    if state_std != 0.0:
        chunk = 8
        for s0 in range(0, num_slots, chunk):
            s1 = min(num_slots, s0 + chunk)
            blk = rng.standard_normal((s1 - s0, H, dv, dk), dtype=np.float32)
            cache[s0:s1] = blk * np.float32(state_std)

    perm = rng.permutation(num_slots).astype(np.int32)
    slot_ids = perm[:B].copy()
    n_tables = max(1, num_slots // B) if B > 0 else 1
    slot_tables = perm[: n_tables * B].reshape(n_tables, B).copy() if B > 0 else np.zeros((1, 0), np.int32)

    accepted = None
    if B > 0 and T_max > 1:
        accepted = np.zeros(B, dtype=np.int32)
        multi = seqlens > 1
        if np.any(multi):
            accepted[multi] = rng.integers(1, seqlens[multi] + 1).astype(np.int32)

    k64 = k_raw.astype(np.float64)
    k64 /= np.linalg.norm(k64, axis=-1, keepdims=True)
    q64 = q_raw.astype(np.float64)
    q64 /= np.linalg.norm(q64, axis=-1, keepdims=True) * np.sqrt(dk)
    alpha = np.exp(-np.logaddexp(0.0, a_raw.astype(np.float64))).astype(np.float32)
    beta = (1.0 / (1.0 + np.exp(-b_raw.astype(np.float64)))).astype(np.float32)

    return Workload(
        name=name, B=B, H=H, dk=dk, dv=dv, steps=steps, cu_seqlens=cu, T_max=T_max,
        q=f32_to_bf16_bits(q64.astype(np.float32)),
        k=f32_to_bf16_bits(k64.astype(np.float32)),
        v=f32_to_bf16_bits(v_raw),
        alpha=alpha, beta=beta,
        gate=f32_to_bf16_bits(g_raw) if gate else None,
        cache=cache, slot_ids=slot_ids, slot_tables=slot_tables,
        accepted=accepted, seed=seed,
        q_raw=f32_to_bf16_bits(q_raw), k_raw=f32_to_bf16_bits(k_raw), a_raw=a_raw, b_raw=b_raw,
    )


WORKLOADS = {
    "tiny": dict(B=1, H=4, dk=64, dv=64, steps=256),
    "b1_latency": dict(B=1, H=32, dk=128, dv=128, steps=1024),
    "b64_bandwidth": dict(B=64, H=32, dk=128, dv=128, num_slots=256, state_std=0.02),
    "spec_verify": dict(B=16, H=32, dk=128, dv=128, seqlens=[8] * 16, num_slots=256, state_std=0.02),
    "mixed": dict(B=64, H=32, dk=128, dv=128, seqlens=[1] * 40 + [4] * 24, num_slots=512,
                  state_std=0.02, gate=True),
    "prefill_8k": dict(B=1, H=32, dk=128, dv=128, seqlens=[8000], num_slots=1),
}


def make_workload(name: str, seed: int = 0) -> Workload:
    """Draw one of the named workloads (see the module docstring)."""
    return make(name=name, seed=seed, **WORKLOADS[name])
