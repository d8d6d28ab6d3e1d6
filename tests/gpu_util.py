"""Helpers for the GPU parity tests: device copies of seeded workloads and error metrics."""

from __future__ import annotations

import sys

import numpy as np
import torch

SENTINEL_BITS = 0x7FC0DEAD


def log(msg: str) -> None:
    """Name the case before each GPU step (flushed, so a failing run still shows it)."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def dev():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    return torch.device("cuda", 0)


def bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev()).view(torch.bfloat16)


def f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev())


def i32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev())


def bits(t: torch.Tensor) -> np.ndarray:
    """Host copy of a float32 / bf16 tensor as raw integer bits."""
    a = t.detach().cpu()
    if a.dtype == torch.float32:
        return a.view(torch.int32).numpy().view(np.uint32)
    if a.dtype in (torch.bfloat16, torch.int16):
        return a.view(torch.int16).numpy().view(np.uint16)
    return a.numpy()


def sentinel(shape) -> torch.Tensor:
    return torch.full(shape, SENTINEL_BITS, dtype=torch.int32, device=dev()).view(torch.float32)


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    if nb < 1e-30:
        return float(np.linalg.norm(a - b))
    return float(np.linalg.norm(a - b) / nb)


def _worst_group(a, b, group_axes: int) -> float:
    """Largest relative L2 error over the sub-arrays formed by the last ``group_axes`` axes."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    if a.ndim <= group_axes or a.size == 0:
        return rel_l2(a, b)
    n = int(np.prod(a.shape[a.ndim - group_axes:]))
    a = a.reshape(-1, n)
    b = b.reshape(-1, n)
    num = np.linalg.norm(a - b, axis=1)
    den = np.linalg.norm(b, axis=1)
    err = np.where(den < 1e-30, num, num / np.maximum(den, 1e-300))
    return float(err.max())


def out_rel(a, b, name: str = "") -> float:
    """Error of outputs shaped [..., dv]: the larger of the whole-array relative L2 and the worst
    single (token, head) vector's, so that one wrong head cannot hide in the norm of thousands."""
    whole, worst = rel_l2(a, b), _worst_group(a, b, 1)
    if name:
        log(f"  {name}: rel-L2 {whole:.3e}, worst (token, head) {worst:.3e}")
    return max(whole, worst)


def state_rel(a, b, name: str = "") -> float:
    """Error of states shaped [..., dv, dk]: the larger of the whole-array relative Frobenius
    error and the worst single head's."""
    whole, worst = rel_l2(a, b), _worst_group(a, b, 2)
    if name:
        log(f"  {name}: rel-Frobenius {whole:.3e}, worst head {worst:.3e}")
    return max(whole, worst)


def step_inputs(w, step: int):
    """Device tensors of one step's token arrays."""
    d = dict(q=bf16(w.q[step]), k=bf16(w.k[step]), v=bf16(w.v[step]),
             alpha=f32(w.alpha[step]), beta=f32(w.beta[step]))
    if w.gate is not None:
        d["gate"] = bf16(w.gate[step])
    return d


def replay_buffers(B, T_max, H, dk, dv):
    z = dict(device=dev())
    return dict(k=torch.zeros(B, T_max, H, dk, dtype=torch.bfloat16, **z),
                v=torch.zeros(B, T_max, H, dv, dtype=torch.bfloat16, **z),
                alpha=torch.zeros(B, T_max, H, dk, dtype=torch.float32, **z),
                beta=torch.zeros(B, T_max, H, dtype=torch.float32, **z))


def raw_step_inputs(w, step: int):
    """Device tensors of one step's raw projections (q, k, alpha, beta before preparation)."""
    d = dict(q=bf16(w.q_raw[step]), k=bf16(w.k_raw[step]), v=bf16(w.v[step]),
             alpha=f32(w.a_raw[step]), beta=f32(w.b_raw[step]))
    if w.gate is not None:
        d["gate"] = bf16(w.gate[step])
    return d
