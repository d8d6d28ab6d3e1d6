"""CPU oracle for the KDA recurrent-state step (numpy front end over kda_oracle.c).

TEST INFRASTRUCTURE. Only the test suite, the package's smoke check and the
benchmark's CPU-baseline leg may import this package. It never imports the GPU
package and the GPU package never imports it.

Definition followed (the pages name the KDA recurrent state and its FP32 SSM
cache but do not write the update; the gated delta rule with per-channel decay
is the reading taken): per head, per token,
    S <- Diag(alpha) S ;  S <- S + beta k (v - S^T k)^T ;  o = S^T q
with S of shape dk x dv. The C file's header gives layouts, modes, the commit
definition (ReplaySSM, "Kimi K3 performance optimization in vLLM") and the
error bits.

Parity pins: brute force in exact rationals on tiny heads, closed forms
(alpha = 0, beta = 0, one-hot write-then-read, associative recall, output-gate
constants), linearity, permutation equivariance, slot/row handling and
hand-worked examples under tests/golden/. See tests/test_oracle_*.py.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

from . import build as _build

REPLAY = 0
PER_POSITION = 1

ERR_SLOT = 1
ERR_SEQLEN = 2
ERR_ACCEPTED = 4
ERR_CKPT = 8

_lib = None


def _load(path: Optional[str] = None):
    global _lib
    if path is None and _lib is not None:
        return _lib
    p = path or _build.LIB
    if not os.path.exists(p):
        _build.build(out=p)
    lib = ctypes.CDLL(p)
    P = ctypes.c_void_p
    i32, i64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    lib.kda_oracle_unit.argtypes = [P, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                    P, P, P, P, P, ctypes.c_int, P, P]
    lib.kda_oracle_unit.restype = None
    lib.kda_oracle_epilogue.argtypes = [P, ctypes.c_int, P, P, f64, P]
    lib.kda_oracle_epilogue.restype = None
    lib.kda_oracle_decode.argtypes = [P, i64, i64, P, i32, i32, i32, i32,
                                      P, P, P, P, P, P, P, P, f64, i32, i32, i32]
    lib.kda_oracle_decode.restype = ctypes.c_int
    lib.kda_oracle_verify.argtypes = [P, i64, i64, P, P, i32, i32, i32, i32, i32, i32,
                                      P, P, P, P, P, P, P, P, f64, i32, i32,
                                      P, P, P, P, P, i32, i32, i32]
    lib.kda_oracle_verify.restype = ctypes.c_int
    lib.kda_oracle_commit.argtypes = [P, i64, i64, P, P, P, i32, i32, i32, i32, i32, i32,
                                      P, P, P, P, i32, i32, i32]
    lib.kda_oracle_commit.restype = ctypes.c_int
    lib.kda_oracle_prefill.argtypes = [P, i64, i64, P, P, i32, i32, i32, i32, i32,
                                       P, P, P, P, P, P, P, P, i32, i32, i32]
    lib.kda_oracle_prefill.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def load_variant(path: str):
    """Load a separately built copy of the oracle (used to check that pins catch planted mistakes)."""
    return _load(path)


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    """Contiguous array of the given dtype (no copy when already so)."""
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=dtype)


def default_threads() -> int:
    """Threads for the batch drivers: the CPUs this process may use, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def unit(S0, q, k, v, alpha, beta, *, state_fp32: bool = True, lib=None):
    """Run one head over n tokens in double precision.

    S0: [dk][dv] (row i = key channel); q, k, alpha: [n][dk]; v: [n][dv]; beta: [n]
    (q may be None: no read-out). Returns (o [n][dv] or None, S_final [dk][dv],
    S_tok [n][dk][dv]).
    """
    lib = lib or _load()
    S = np.array(S0, dtype=np.float64, order="C", copy=True)
    dk, dv = S.shape
    k = _c(k, np.float64).reshape(-1, dk)
    n = k.shape[0]
    q = None if q is None else _c(q, np.float64).reshape(n, dk)
    v = _c(v, np.float64).reshape(n, dv)
    a = _c(alpha, np.float64).reshape(n, dk)
    b = _c(beta, np.float64).reshape(n)
    o = np.empty((n, dv), np.float64) if q is not None else None
    S_tok = np.empty((n, dk, dv), np.float64)
    lib.kda_oracle_unit(_ptr(S), dk, dv, n, _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b),
                        int(state_fp32), _ptr(o), _ptr(S_tok))
    return o, S, S_tok


def epilogue(o, g, w=None, eps: float = 1e-6, lib=None):
    """Output gate for one head: o / sqrt(mean(o^2) + eps) * w * sigmoid(g), in double."""
    lib = lib or _load()
    o = _c(o, np.float64)
    g = _c(g, np.float64)
    w = _c(w, np.float64)
    y = np.empty_like(o)
    lib.kda_oracle_epilogue(_ptr(o), o.shape[0], _ptr(g), _ptr(w), float(eps), _ptr(y))
    return y


def _slot_stride(cache: np.ndarray) -> int:
    return int(np.prod(cache.shape[1:]))


def decode(cache, slot_ids, q, k, v, alpha, beta, *, out=None, gate=None, weight=None,
           eps: float = 1e-6, prologue: bool = False, state_fp32: bool = True,
           nthreads: Optional[int] = None, lib=None):
    """Single-token step for B rows, in place on ``cache`` [num_slots][H][dv][dk] float32.

    q, k: uint16 bf16 bits [B][H][dk]; v (and gate): [B][H][dv]; alpha [B][H][dk];
    beta [B][H]. Returns (out [B][H][dv] float32, error bits).
    """
    lib = lib or _load()
    assert cache.dtype == np.float32 and cache.flags.c_contiguous
    num_slots, H, dv, dk = cache.shape
    slot_ids = _c(slot_ids, np.int32)
    B = slot_ids.shape[0]
    q, k, v, gate = (_c(x, np.uint16) for x in (q, k, v, gate))
    alpha, beta, weight = (_c(x, np.float32) for x in (alpha, beta, weight))
    if out is None:
        out = np.full((B, H, dv), np.nan, np.float32)
    rc = lib.kda_oracle_decode(_ptr(cache), num_slots, _slot_stride(cache), _ptr(slot_ids),
                               B, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                               _ptr(out), _ptr(gate), _ptr(weight), float(eps), int(bool(prologue)),
                               int(state_fp32), nthreads or default_threads())
    if rc < 0:
        raise ValueError("oracle decode: invalid arguments")
    return out, rc


def verify(cache, slot_ids, cu_seqlens, T_max, q, k, v, alpha, beta, *, mode=REPLAY,
           t1_inplace: bool = False, out=None, gate=None, weight=None, eps: float = 1e-6,
           replay=None, draft=None, prologue: bool = False, state_fp32: bool = True,
           nthreads: Optional[int] = None, lib=None):
    """Packed speculative chunk. Token arrays are [n_tok][H][.]; row b owns
    tokens [cu[b], cu[b+1]). Returns (out, replay dict or None, draft or None, error bits).
    replay buffers are rk [B][T_max][H][dk] (uint16), rv [B][T_max][H][dv] (uint16),
    ralpha [B][T_max][H][dk], rbeta [B][T_max][H]; draft is [B][T_max][H][dv][dk].
    """
    lib = lib or _load()
    assert cache.dtype == np.float32 and cache.flags.c_contiguous
    num_slots, H, dv, dk = cache.shape
    slot_ids = _c(slot_ids, np.int32)
    cu = _c(cu_seqlens, np.int32)
    B = slot_ids.shape[0]
    n_tok = int(k.shape[0])
    q, k, v, gate = (_c(x, np.uint16) for x in (q, k, v, gate))
    alpha, beta, weight = (_c(x, np.float32) for x in (alpha, beta, weight))
    if out is None:
        out = np.full((n_tok, H, dv), np.nan, np.float32)
    if mode == REPLAY and replay is None:
        replay = dict(
            rk=np.zeros((B, T_max, H, dk), np.uint16), rv=np.zeros((B, T_max, H, dv), np.uint16),
            ralpha=np.zeros((B, T_max, H, dk), np.float32), rbeta=np.zeros((B, T_max, H), np.float32))
    if mode == PER_POSITION and draft is None:
        draft = np.zeros((B, T_max, H, dv, dk), np.float32)
    rb = replay or {}
    rc = lib.kda_oracle_verify(_ptr(cache), num_slots, _slot_stride(cache), _ptr(slot_ids), _ptr(cu),
                               B, int(T_max), n_tok, H, dk, dv,
                               _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(out),
                               _ptr(gate), _ptr(weight), float(eps), int(mode), int(bool(t1_inplace)),
                               _ptr(rb.get("rk")), _ptr(rb.get("rv")), _ptr(rb.get("ralpha")),
                               _ptr(rb.get("rbeta")), _ptr(draft if mode == PER_POSITION else None),
                               int(bool(prologue)), int(state_fp32), nthreads or default_threads())
    if rc < 0:
        raise ValueError("oracle verify: invalid arguments")
    return out, (replay if mode == REPLAY else None), (draft if mode == PER_POSITION else None), rc


def commit(cache, slot_ids, cu_seqlens, accepted_len, T_max, k, v, alpha, beta, *,
           prologue: bool = False, state_fp32: bool = True, nthreads: Optional[int] = None, lib=None):
    """Slot of row b <- state after the first accepted_len[b] tokens of row b's chunk
    (in place on ``cache``). Returns the error bits."""
    lib = lib or _load()
    assert cache.dtype == np.float32 and cache.flags.c_contiguous
    num_slots, H, dv, dk = cache.shape
    slot_ids = _c(slot_ids, np.int32)
    cu = _c(cu_seqlens, np.int32)
    acc = _c(accepted_len, np.int32)
    B = slot_ids.shape[0]
    n_tok = int(k.shape[0])
    k, v = (_c(x, np.uint16) for x in (k, v))
    alpha, beta = (_c(x, np.float32) for x in (alpha, beta))
    rc = lib.kda_oracle_commit(_ptr(cache), num_slots, _slot_stride(cache), _ptr(slot_ids), _ptr(cu),
                               _ptr(acc), B, int(T_max), n_tok, H, dk, dv,
                               _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), int(bool(prologue)),
                               int(state_fp32), nthreads or default_threads())
    if rc < 0:
        raise ValueError("oracle commit: invalid arguments")
    return rc


def prefill(cache, slot_ids, cu_seqlens, q, k, v, alpha, beta, *, ckpt_pos=None, out=None,
            prologue: bool = False, state_fp32: bool = True, nthreads: Optional[int] = None, lib=None):
    """Whole prompts in one pass (in place on ``cache``). Token arrays are [n_tok][H][.];
    row b owns tokens [cu[b], cu[b+1]). Returns (out [n_tok][H][dv], ckpt [B][H][dv][dk]
    or None, error bits); ckpt[b] is the state after the first ckpt_pos[b] tokens."""
    lib = lib or _load()
    assert cache.dtype == np.float32 and cache.flags.c_contiguous
    num_slots, H, dv, dk = cache.shape
    slot_ids = _c(slot_ids, np.int32)
    cu = _c(cu_seqlens, np.int32)
    B = slot_ids.shape[0]
    n_tok = int(k.shape[0])
    q, k, v = (_c(x, np.uint16) for x in (q, k, v))
    alpha, beta = (_c(x, np.float32) for x in (alpha, beta))
    pos = _c(ckpt_pos, np.int32)
    ckpt = np.full((B, H, dv, dk), np.nan, np.float32) if pos is not None else None
    if out is None:
        out = np.full((n_tok, H, dv), np.nan, np.float32)
    rc = lib.kda_oracle_prefill(_ptr(cache), num_slots, _slot_stride(cache), _ptr(slot_ids), _ptr(cu),
                                B, n_tok, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                _ptr(out), _ptr(pos), _ptr(ckpt), int(bool(prologue)), int(state_fp32),
                                nthreads or default_threads())
    if rc < 0:
        raise ValueError("oracle prefill: invalid arguments")
    return out, ckpt, rc
