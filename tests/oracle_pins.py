"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Each ``check_*`` takes the oracle's ctypes library (the built one, or a copy
with a planted mistake) and raises AssertionError when the oracle disagrees
with the fact it checks. The facts:
  * hand-worked examples (tests/golden/), exact;
  * exact rational brute force of the matrix form (tests/brute.py) on tiny
    heads, through the single-head routine and through the batch drivers;
  * closed forms: alpha = 0 erases the state, beta = 0 gives a pure decay,
    one-hot write-then-read returns v, associative recall, the output gate's
    constants, the raw-input preparation on inputs where it is exact or has a
    hand-derived value;
  * structure: linearity, column permutation equivariance, commit equals
    step-by-step, slot / row / error handling, fp32 state storage.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np

import oracle
import synth
from brute import brute_run, to_float

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
DYADIC = np.array([-2, -1.5, -1, -0.75, -0.5, -0.25, 0, 0.25, 0.5, 0.75, 1, 1.5, 2], np.float64)
GATES = np.array([0, 0.25, 0.5, 0.75, 1], np.float64)


def _rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / nb if nb > 1e-300 else np.linalg.norm(a - b)


def _bf(x):
    return synth.f32_to_bf16_bits(np.asarray(x, np.float32))


def _head_cache(S0):
    """One slot, one head: the cache layout stores value column j's key channels contiguously."""
    S0 = np.asarray(S0, np.float32)
    return np.ascontiguousarray(S0.T[None, None, :, :])


# ---------------------------------------------------------------- golden files

def check_golden_steps(lib):
    with open(os.path.join(GOLDEN, "hand_worked_steps.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        S0 = np.array(case["S0"], np.float64)
        toks = case["tokens"]
        n = len(toks)
        q = np.array([t["q"] for t in toks], np.float64)
        k = np.array([t["k"] for t in toks], np.float64)
        v = np.array([t["v"] for t in toks], np.float64)
        a = np.array([t["alpha"] for t in toks], np.float64)
        b = np.array([t["beta"] for t in toks], np.float64)
        for fp32 in (False, True):
            o, S, S_tok = oracle.unit(S0, q, k, v, a, b, state_fp32=fp32, lib=lib)
            for t in range(n):
                assert np.array_equal(S_tok[t], np.array(toks[t]["S"], np.float64)), case["name"]
                assert np.array_equal(o[t], np.array(toks[t]["o"], np.float64)), case["name"]
        # the same through the batch decode driver and the cache layout
        cache = _head_cache(S0)
        for t in range(n):
            out, rc = oracle.decode(cache, [0], _bf(q[t])[None, None], _bf(k[t])[None, None],
                                    _bf(v[t])[None, None], a[t].astype(np.float32)[None, None],
                                    np.array([[b[t]]], np.float32), lib=lib)
            assert rc == 0
            assert np.array_equal(cache[0, 0].T, np.array(toks[t]["S"], np.float32)), case["name"]
            assert np.array_equal(out[0, 0], np.array(toks[t]["o"], np.float32)), case["name"]


def check_golden_gate(lib):
    with open(os.path.join(GOLDEN, "hand_worked_output_gate.json")) as f:
        cases = json.load(f)["cases"]
    ln3 = math.log(3.0)
    for case in cases:
        g = [ln3 if x == "ln3" else -ln3 if x == "-ln3" else x for x in case["g"]]
        y = oracle.epilogue(np.array(case["o"], np.float64), np.array(g, np.float64),
                            None if case["w"] is None else np.array(case["w"], np.float64),
                            eps=case["eps"], lib=lib)
        assert _rel(y, case["y"]) < 1e-15, case["name"]


# ---------------------------------------------------------------- brute force

def _dyadic_tokens(rng, dk, dv, n):
    q = rng.choice(DYADIC, (n, dk))
    k = rng.choice(DYADIC, (n, dk))
    v = rng.choice(DYADIC, (n, dv))
    a = rng.choice(GATES, (n, dk))
    b = rng.choice(GATES, n)
    return q, k, v, a, b


def check_brute_unit(lib):
    rng = np.random.Generator(np.random.PCG64(1234))
    shapes = [(1, 1), (2, 3), (3, 2), (4, 4), (1, 4), (4, 1), (3, 3), (2, 4)]
    for dk, dv in shapes:
        for n in (1, 3, 6):
            S0 = rng.choice(DYADIC, (dk, dv))
            q, k, v, a, b = _dyadic_tokens(rng, dk, dv, n)
            states, outs = brute_run(S0, list(zip(q, k, v, a, b)))
            Sx = np.array(to_float(states))
            ox = np.array(to_float(outs))
            o64, _, S64 = oracle.unit(S0, q, k, v, a, b, state_fp32=False, lib=lib)
            assert _rel(S64, Sx) <= 1e-13 and _rel(o64, ox) <= 1e-13, (dk, dv, n)
            o32, _, S32 = oracle.unit(S0, q, k, v, a, b, state_fp32=True, lib=lib)
            assert _rel(S32, Sx) <= 1e-6 and _rel(o32, ox) <= 1e-6, (dk, dv, n)


def _unit_tokens(w, rows, h):
    """(q, k, v, alpha, beta) of head h for the given packed token rows, as exact floats."""
    qf = synth.bf16_bits_to_f32(w.q[0])
    kf = synth.bf16_bits_to_f32(w.k[0])
    vf = synth.bf16_bits_to_f32(w.v[0])
    return [(qf[r, h], kf[r, h], vf[r, h], w.alpha[0][r, h], w.beta[0][r, h]) for r in rows]


def check_brute_batch(lib):
    # verify (both modes) + commit on a ragged packed chunk with an empty row and spare slots
    w = synth.make(4, 2, 3, 4, seqlens=[2, 0, 3, 1], num_slots=6, state_std=0.5, seed=7)
    cu, T_max = w.cu_seqlens, w.T_max
    acc = np.array([2, 0, 1, 1], np.int32)
    ref = {}
    for b in range(w.B):
        s = w.slot_ids[b]
        for h in range(w.H):
            S0 = w.cache[s, h].T.astype(np.float64)
            ref[b, h] = brute_run(S0, _unit_tokens(w, range(cu[b], cu[b + 1]), h))
    for mode in (oracle.REPLAY, oracle.PER_POSITION):
        cache = w.cache.copy()
        out, rb, draft, rc = oracle.verify(cache, w.slot_ids, cu, T_max, w.q[0], w.k[0], w.v[0],
                                           w.alpha[0], w.beta[0], mode=mode, lib=lib)
        assert rc == 0
        assert np.array_equal(cache, w.cache)  # verify never writes committed slots
        for b in range(w.B):
            for h in range(w.H):
                states, outs = ref[b, h]
                for t in range(cu[b + 1] - cu[b]):
                    assert _rel(out[cu[b] + t, h], to_float(outs[t])) <= 1e-6, (b, h, t)
                    if mode == oracle.PER_POSITION:
                        assert _rel(draft[b, t, h].T, to_float(states[t])) <= 1e-6, (b, h, t)
                    else:
                        r = cu[b] + t
                        assert np.array_equal(rb["rk"][b, t, h], w.k[0][r, h])
                        assert np.array_equal(rb["rv"][b, t, h], w.v[0][r, h])
                        assert np.array_equal(rb["ralpha"][b, t, h], w.alpha[0][r, h])
                        assert rb["rbeta"][b, t, h] == w.beta[0][r, h]
    cache = w.cache.copy()
    rc = oracle.commit(cache, w.slot_ids, cu, acc, T_max, w.k[0], w.v[0], w.alpha[0], w.beta[0], lib=lib)
    assert rc == 0
    for b in range(w.B):
        s = w.slot_ids[b]
        for h in range(w.H):
            if acc[b] == 0:
                assert np.array_equal(cache[s, h], w.cache[s, h])
            else:
                assert _rel(cache[s, h].T, to_float(ref[b, h][0][acc[b] - 1])) <= 1e-6, (b, h)
    untouched = np.setdiff1d(np.arange(w.num_slots), w.slot_ids)
    assert np.array_equal(cache[untouched], w.cache[untouched])

    # single-token decode on a non-square head
    d = synth.make(3, 2, 4, 3, num_slots=5, state_std=0.5, seed=8)
    cache = d.cache.copy()
    out, rc = oracle.decode(cache, d.slot_ids, d.q[0], d.k[0], d.v[0], d.alpha[0], d.beta[0], lib=lib)
    assert rc == 0
    for b in range(d.B):
        s = d.slot_ids[b]
        for h in range(d.H):
            states, outs = brute_run(d.cache[s, h].T.astype(np.float64), _unit_tokens(d, [b], h))
            assert _rel(cache[s, h].T, to_float(states[0])) <= 1e-6, (b, h)
            assert _rel(out[b, h], to_float(outs[0])) <= 1e-6, (b, h)


def check_prefill_brute(lib):
    """Prefill through the batch driver: outputs, final slot states and the in-pass
    checkpoints against exact brute force, for empty, short and checkpoint-0 rows."""
    w = synth.make(4, 2, 3, 4, seqlens=[6, 0, 3, 5], num_slots=6, state_std=0.5, seed=19)
    pos = np.array([2, 0, 3, 0], np.int32)
    cache = w.cache.copy()
    out, ckpt, rc = oracle.prefill(cache, w.slot_ids, w.cu_seqlens, w.q[0], w.k[0], w.v[0], w.alpha[0],
                                   w.beta[0], ckpt_pos=pos, lib=lib)
    assert rc == 0
    cu = w.cu_seqlens
    for b in range(w.B):
        s = w.slot_ids[b]
        for h in range(w.H):
            S0 = w.cache[s, h].T.astype(np.float64)
            states, outs = brute_run(S0, _unit_tokens(w, range(cu[b], cu[b + 1]), h))
            for t in range(cu[b + 1] - cu[b]):
                assert _rel(out[cu[b] + t, h], to_float(outs[t])) <= 1e-6, (b, h, t)
            final = to_float(states[-1]) if states else S0
            assert _rel(cache[s, h].T, final) <= 1e-6, (b, h)
            at = pos[b]
            expect = S0 if at == 0 else to_float(states[at - 1])
            assert _rel(ckpt[b, h].T, expect) <= 1e-6, (b, h)
    untouched = np.setdiff1d(np.arange(w.num_slots), w.slot_ids)
    assert np.array_equal(cache[untouched], w.cache[untouched])
    # a checkpoint past the row: error bit 8, row skipped, others done
    cache = w.cache.copy()
    _, _, rc = oracle.prefill(cache, w.slot_ids, w.cu_seqlens, w.q[0], w.k[0], w.v[0], w.alpha[0],
                              w.beta[0], ckpt_pos=np.array([7, 0, 3, 0], np.int32), lib=lib)
    assert rc == oracle.ERR_CKPT
    assert np.array_equal(cache[w.slot_ids[0]], w.cache[w.slot_ids[0]])
    assert not np.array_equal(cache[w.slot_ids[2]], w.cache[w.slot_ids[2]])

    # ckpt_pos < 0 asks for no export: that row's checkpoint keeps its contents,
    # and its outputs and final state are those of the plain run
    pos = np.array([-1, -1, 1, -5], np.int32)
    cache = w.cache.copy()
    out2, ckpt2, rc = oracle.prefill(cache, w.slot_ids, w.cu_seqlens, w.q[0], w.k[0], w.v[0], w.alpha[0],
                                     w.beta[0], ckpt_pos=pos, lib=lib)
    assert rc == 0
    for b in range(w.B):
        s = w.slot_ids[b]
        for h in range(w.H):
            S0 = w.cache[s, h].T.astype(np.float64)
            states, outs = brute_run(S0, _unit_tokens(w, range(cu[b], cu[b + 1]), h))
            for t in range(cu[b + 1] - cu[b]):
                assert _rel(out2[cu[b] + t, h], to_float(outs[t])) <= 1e-6, (b, h, t)
            final = to_float(states[-1]) if states else S0
            assert _rel(cache[s, h].T, final) <= 1e-6, (b, h)
            if pos[b] < 0:
                assert np.all(np.isnan(ckpt2[b, h])), (b, h)
            else:
                assert _rel(ckpt2[b, h].T, to_float(states[pos[b] - 1])) <= 1e-6, (b, h)


# ---------------------------------------------------------------- closed forms

def check_write_then_read(lib):
    rng = np.random.Generator(np.random.PCG64(5))
    dk = dv = 8
    for i in (0, 3, 7):
        for random_state in (False, True):
            S0 = (rng.standard_normal((dk, dv)) * 0.02).astype(np.float32) if random_state \
                else np.zeros((dk, dv), np.float32)
            cache = _head_cache(S0)
            k = np.zeros(dk, np.float32)
            k[i] = 1.0
            v = synth.bf16_bits_to_f32(_bf(rng.standard_normal(dv)))
            q = np.zeros(dk, np.float32)
            q[i] = 1.0
            out, rc = oracle.decode(cache, [0], _bf(q)[None, None], _bf(k)[None, None], _bf(v)[None, None],
                                    np.ones((1, 1, dk), np.float32), np.ones((1, 1), np.float32), lib=lib)
            assert rc == 0
            S = cache[0, 0].T
            assert np.array_equal(S[i], v)            # row i now holds v exactly
            assert np.array_equal(out[0, 0], v)       # and reading it back with k gives v
            others = np.arange(dk) != i
            assert np.array_equal(S[others], S0[others])
    # a general unit key, in double: S^T k = v after the write (beta = 1, alpha = 1)
    for _ in range(5):
        S0 = rng.standard_normal((dk, dv))
        k = rng.standard_normal(dk)
        k /= np.linalg.norm(k)
        v = rng.standard_normal(dv)
        _, S, _ = oracle.unit(S0, None, k[None], v[None], np.ones((1, dk)), np.ones(1),
                              state_fp32=False, lib=lib)
        assert np.linalg.norm(S.T @ k - v) <= 1e-12 * (np.linalg.norm(S0) + np.linalg.norm(v))


def check_alpha_zero(lib):
    rng = np.random.Generator(np.random.PCG64(6))
    dk, dv = 5, 3
    S0 = rng.standard_normal((dk, dv))
    k = rng.standard_normal((1, dk))
    v = rng.standard_normal((1, dv))
    b = np.array([0.375])
    a = np.zeros((1, dk))
    for fp32 in (False, True):
        _, S_a, _ = oracle.unit(S0, None, k, v, a, b, state_fp32=fp32, lib=lib)
        _, S_z, _ = oracle.unit(np.zeros((dk, dv)), None, k, v, a, b, state_fp32=fp32, lib=lib)
        assert np.array_equal(S_a, S_z)
    _, S_a, _ = oracle.unit(S0, None, k, v, a, b, state_fp32=False, lib=lib)
    assert _rel(S_a, b[0] * np.outer(k[0], v[0])) <= 1e-15


def check_beta_zero(lib):
    rng = np.random.Generator(np.random.PCG64(7))
    dk, dv, n = 6, 4, 5
    S0 = rng.standard_normal((dk, dv))
    q = rng.standard_normal((n, dk))
    k = rng.standard_normal((n, dk))
    v = rng.standard_normal((n, dv))
    a = rng.uniform(0.0, 1.0, (n, dk))
    o, S, _ = oracle.unit(S0, q, k, v, a, np.zeros(n), state_fp32=False, lib=lib)
    assert _rel(S, np.prod(a, axis=0)[:, None] * S0) <= 1e-14
    assert _rel(o[-1], S.T @ q[-1]) <= 1e-14
    S0f = S0.astype(np.float32).astype(np.float64)
    o, S, _ = oracle.unit(S0f, q, k, v, np.ones((n, dk)), np.zeros(n), state_fp32=True, lib=lib)
    assert np.array_equal(S, S0f)
    for t in range(n):
        assert _rel(o[t], np.matmul(q[t], S0f)) <= 1e-15


def check_associative_recall(lib):
    rng = np.random.Generator(np.random.PCG64(8))
    dk, dv = 8, 5
    perm = rng.permutation(dk)
    n = 6
    keys = np.eye(dk)[perm[:n]]
    vals = synth.bf16_bits_to_f32(_bf(rng.standard_normal((n, dv)))).astype(np.float64)
    q = np.tile(np.eye(dk)[perm[0]], (n, 1))
    o, S, _ = oracle.unit(np.zeros((dk, dv)), q, keys, vals, np.ones((n, dk)), np.ones(n),
                          state_fp32=True, lib=lib)
    for t in range(n):
        assert np.array_equal(S.T @ keys[t], vals[t])
    assert np.array_equal(o[-1], vals[0])


def check_linearity(lib):
    rng = np.random.Generator(np.random.PCG64(9))
    dk, dv, n = 5, 6, 7
    S0 = rng.standard_normal((dk, dv))
    q = rng.standard_normal((n, dk))
    k = rng.standard_normal((n, dk)) / math.sqrt(dk)
    v = rng.standard_normal((n, dv))
    a = rng.uniform(0.2, 1.0, (n, dk))
    b = rng.uniform(0.0, 1.0, n)
    o1, S1, _ = oracle.unit(S0, q, k, v, a, b, state_fp32=False, lib=lib)
    o2, S2, _ = oracle.unit(S0, q, k, np.zeros_like(v), a, b, state_fp32=False, lib=lib)
    o3, S3, _ = oracle.unit(np.zeros_like(S0), q, k, v, a, b, state_fp32=False, lib=lib)
    assert _rel(S1, S2 + S3) <= 1e-12
    assert _rel(o1, o2 + o3) <= 1e-12


def check_gate_closed_form(lib):
    rng = np.random.Generator(np.random.PCG64(10))
    dv = 16
    for c in (2.5, -0.75, 1e-3):
        for eps in (0.0, 1e-6, 0.5):
            g = rng.standard_normal(dv)
            w = rng.uniform(0.5, 2.0, dv)
            y = oracle.epilogue(np.full(dv, c), g, w, eps=eps, lib=lib)
            sig = np.array([1.0 / (1.0 + math.exp(-x)) for x in g])
            expect = math.copysign(1.0, c) / math.sqrt(1.0 + eps / (c * c)) * w * sig
            assert _rel(y, expect) <= 1e-14
    o = rng.standard_normal(dv)
    y = oracle.epilogue(o, np.zeros(dv), None, eps=0.0, lib=lib)
    rms = math.sqrt(sum(x * x for x in o) / dv)
    assert _rel(y, o / rms * 0.5) <= 1e-14
    # the batch drivers apply the gate to the read-out of each (token, head)
    d = synth.make(3, 2, 8, 16, num_slots=4, state_std=0.3, gate=True, seed=11)
    weight = rng.uniform(0.5, 2.0, 16).astype(np.float32)
    plain, _ = oracle.decode(d.cache.copy(), d.slot_ids, d.q[0], d.k[0], d.v[0], d.alpha[0], d.beta[0], lib=lib)
    gated, _ = oracle.decode(d.cache.copy(), d.slot_ids, d.q[0], d.k[0], d.v[0], d.alpha[0], d.beta[0],
                             gate=d.gate[0], weight=weight, eps=1e-6, lib=lib)
    gf = synth.bf16_bits_to_f32(d.gate[0])
    for b in range(d.B):
        for h in range(d.H):
            o = plain[b, h].astype(np.float64)
            rms = math.sqrt(float(np.mean(o * o)) + 1e-6)
            sig = 1.0 / (1.0 + np.exp(-gf[b, h].astype(np.float64)))
            assert _rel(gated[b, h], o / rms * weight * sig) <= 1e-6, (b, h)


def _prologue_case():
    """Raw projections whose normalization and activations have closed forms.

    Head 0: k along channels 0 and 70 as (3, 4) -> (0.6, 0.8); q along channels 0
    and 100 as (3, 4) -> (0.6, 0.8) / sqrt(128); a = 0 on even channels and ln 3 on
    odd ones -> alpha = 1/(1 + e^a) = 1/2 and 1/4; b = ln 3 -> beta = 3/4; v = 0.
    Head 1: zero key (normalizes to zero), q = 2 e_5 -> e_5 / sqrt(128), a = ln 3,
    b = 0, v nonzero (must not reach the state). The state starts at all ones.
    """
    dk, dv, H = 128, 4, 2
    ln3 = math.log(3.0)
    q = np.zeros((1, H, dk), np.float32)
    k = np.zeros((1, H, dk), np.float32)
    v = np.zeros((1, H, dv), np.float32)
    a = np.zeros((1, H, dk), np.float32)
    b = np.zeros((1, H), np.float32)
    k[0, 0, 0], k[0, 0, 70] = 3.0, 4.0
    q[0, 0, 0], q[0, 0, 100] = 3.0, 4.0
    a[0, 0, 1::2] = ln3
    b[0, 0] = ln3
    q[0, 1, 5] = 2.0
    a[0, 1, :] = ln3
    v[0, 1] = [1.0, 2.0, 3.0, 4.0]
    # hand-derived result of one token
    S = np.ones((H, dk, dv))
    S[0, 0::2] = 0.5
    S[0, 1::2] = 0.25
    d = 0.75 * (0.0 - (0.6 * 0.5 + 0.8 * 0.5))      # beta (v - S^T k) = -0.525
    S[0, 0] = 0.5 + 0.6 * d
    S[0, 70] = 0.5 + 0.8 * d
    S[1] = 0.25
    o = np.zeros((H, dv))
    o[0] = (0.6 * S[0, 0] + 0.8 * S[0, 100]) / math.sqrt(dk)
    o[1] = S[1, 5] / math.sqrt(dk)
    cache = np.ones((1, H, dv, dk), np.float32)
    return dict(q=_bf(q), k=_bf(k), v=_bf(v), a=a, b=b, S=S, o=o, cache=cache)


def check_prologue_closed_form(lib):
    """Raw-input mode through every batch driver against the hand-derived state and
    read-out of one token; the replay buffer keeps the raw inputs."""
    c = _prologue_case()
    cu = np.array([0, 1], np.int32)

    def state(cache):
        return cache[0].transpose(0, 2, 1)

    cache = c["cache"].copy()
    out, rc = oracle.decode(cache, [0], c["q"], c["k"], c["v"], c["a"], c["b"], prologue=True, lib=lib)
    assert rc == 0
    assert _rel(state(cache), c["S"]) <= 1e-7
    assert _rel(out[0], c["o"]) <= 1e-7
    assert np.all(state(cache)[1] == np.float32(0.25))          # zero key: a pure decay
    cache = c["cache"].copy()
    out, rb, _, rc = oracle.verify(cache, [0], cu, 1, c["q"], c["k"], c["v"], c["a"], c["b"],
                                   mode=oracle.REPLAY, prologue=True, lib=lib)
    assert rc == 0
    assert _rel(out[0], c["o"]) <= 1e-7
    assert np.array_equal(cache, c["cache"])
    assert np.array_equal(rb["rk"][0], c["k"]) and np.array_equal(rb["ralpha"][0], c["a"])
    assert np.array_equal(rb["rbeta"][0], c["b"])
    rc = oracle.commit(cache, [0], cu, np.array([1], np.int32), 1, rb["rk"][0], rb["rv"][0],
                       rb["ralpha"][0], rb["rbeta"][0], prologue=True, lib=lib)
    assert rc == 0
    assert _rel(state(cache), c["S"]) <= 1e-7
    cache = c["cache"].copy()
    out, ckpt, rc = oracle.prefill(cache, [0], cu, c["q"], c["k"], c["v"], c["a"], c["b"],
                                   ckpt_pos=np.array([1], np.int32), prologue=True, lib=lib)
    assert rc == 0
    assert _rel(out[0], c["o"]) <= 1e-7
    assert _rel(state(cache), c["S"]) <= 1e-7
    assert np.array_equal(ckpt[0], cache[0])


def check_prologue_prepared_equivalence(lib):
    """Raw inputs whose preparation has an exact value give what the prepared inputs
    passed directly give, to within the fp32 rounding of the state (the 1e-12 in the
    norms moves the prepared values by about 1e-14): a one-hot key, a query of norm
    8 with dk = 64 (the scale is 1/64), a = 0 (alpha = 1/2) and b = 0 (beta = 1/2),
    over several tokens."""
    w = synth.make(2, 3, 64, 8, steps=4, num_slots=3, state_std=0.1, seed=23)
    rng = np.random.Generator(np.random.PCG64(24))
    cache_raw, cache_prep = w.cache.copy(), w.cache.copy()
    for t in range(4):
        k = np.zeros((w.B, w.H, 64), np.float32)
        q = np.zeros((w.B, w.H, 64), np.float32)
        for bh in np.ndindex(w.B, w.H):
            k[bh][rng.integers(64)] = rng.choice([-2.0, 0.5, 3.0])
            q[bh][rng.permutation(64)[:4]] = 4.0 * rng.choice([-1.0, 1.0], 4)
        kp = k / np.abs(k).max(axis=-1, keepdims=True)
        zeros_a = np.zeros((w.B, w.H, 64), np.float32)
        zeros_b = np.zeros((w.B, w.H), np.float32)
        o1, rc1 = oracle.decode(cache_raw, w.slot_ids, _bf(q), _bf(k), w.v[t], zeros_a, zeros_b,
                                prologue=True, lib=lib)
        o2, rc2 = oracle.decode(cache_prep, w.slot_ids, _bf(q / 64.0), _bf(kp), w.v[t],
                                np.full_like(zeros_a, 0.5), np.full_like(zeros_b, 0.5), lib=lib)
        assert rc1 == 0 and rc2 == 0
        assert _rel(cache_raw, cache_prep) <= 1e-6, t
        assert _rel(o1, o2) <= 1e-6, t


def check_inplace_rows(lib):
    """The single-token rows of a mixed batch ("Kimi K3 performance optimization in
    vLLM", section "Zero-copy mixed KDA batching"): with t1_inplace, a row of one
    token takes its step on the slot itself (exact brute force of the matrix form)
    and leaves no replay or draft entry, while the multi-token rows keep their slots
    and fill their buffers, in both modes. Without the flag every row is speculative."""
    w = synth.make(5, 2, 3, 4, seqlens=[1, 3, 1, 2, 1], num_slots=7, state_std=0.5, seed=31)
    cu, T_max, H = w.cu_seqlens, w.T_max, w.H
    nan = np.array([0x7FC0DEAD], np.uint32).view(np.float32)[0]
    ref = {}
    for b in range(w.B):
        for h in range(H):
            S0 = w.cache[w.slot_ids[b], h].T.astype(np.float64)
            ref[b, h] = brute_run(S0, _unit_tokens(w, range(cu[b], cu[b + 1]), h))
    for inplace in (True, False):
        for mode in (oracle.REPLAY, oracle.PER_POSITION):
            cache = w.cache.copy()
            rb = dict(rk=np.full((w.B, T_max, H, w.dk), 0xDEAD, np.uint16),
                      rv=np.full((w.B, T_max, H, w.dv), 0xDEAD, np.uint16),
                      ralpha=np.full((w.B, T_max, H, w.dk), nan, np.float32),
                      rbeta=np.full((w.B, T_max, H), nan, np.float32))
            draft = np.full((w.B, T_max, H, w.dv, w.dk), nan, np.float32)
            out, rb, draft, rc = oracle.verify(cache, w.slot_ids, cu, T_max, w.q[0], w.k[0], w.v[0],
                                               w.alpha[0], w.beta[0], mode=mode, t1_inplace=inplace,
                                               replay=rb if mode == oracle.REPLAY else None,
                                               draft=draft if mode == oracle.PER_POSITION else None, lib=lib)
            assert rc == 0
            for b in range(w.B):
                s, Tb = w.slot_ids[b], cu[b + 1] - cu[b]
                in_place = inplace and Tb == 1
                for h in range(H):
                    states, outs = ref[b, h]
                    for t in range(Tb):
                        assert _rel(out[cu[b] + t, h], to_float(outs[t])) <= 1e-6, (b, h, t)
                    if in_place:
                        assert _rel(cache[s, h].T, to_float(states[0])) <= 1e-6, (b, h, mode)
                    else:
                        assert np.array_equal(cache[s, h], w.cache[s, h]), (b, h, mode)
                    for t in range(T_max):
                        written = not in_place and t < Tb
                        if mode == oracle.PER_POSITION:
                            d = draft[b, t, h]
                            if written:
                                assert _rel(d.T, to_float(states[t])) <= 1e-6, (b, t, h)
                            else:
                                assert np.all(d.view(np.uint32) == 0x7FC0DEAD), (b, t, h)
                        else:
                            if written:
                                r = cu[b] + t
                                assert np.array_equal(rb["rk"][b, t, h], w.k[0][r, h])
                                assert np.array_equal(rb["rv"][b, t, h], w.v[0][r, h])
                                assert np.array_equal(rb["ralpha"][b, t, h], w.alpha[0][r, h])
                                assert rb["rbeta"][b, t, h] == w.beta[0][r, h]
                            else:
                                assert np.all(rb["rk"][b, t, h] == 0xDEAD), (b, t, h)
                                assert np.all(rb["rv"][b, t, h] == 0xDEAD), (b, t, h)
                                assert np.all(rb["ralpha"][b, t, h].view(np.uint32) == 0x7FC0DEAD)
                                assert rb["rbeta"][b, t, h].view(np.uint32) == 0x7FC0DEAD
            untouched = np.setdiff1d(np.arange(w.num_slots), w.slot_ids)
            assert np.array_equal(cache[untouched], w.cache[untouched])


def check_gate_every_token(lib):
    """The output gate ("Hyper Optimizing Kimi K3 in vLLM", section "Finding time
    between operators") applies to the read-out of every token of a multi-token row.
    Closed form: with k = q = e_0, beta = 1 and alpha_0 = 0, the decay erases key row
    0 before each write, so the write stores v_t there exactly and the read-out is
    o_t = v_t. With v_t = c_t * 1 and gate 0 the gated output is
    sign(c_t) / sqrt(1 + eps / c_t^2) * w / 2, for every token t."""
    rng = np.random.Generator(np.random.PCG64(32))
    dk, dv, H = 4, 8, 2
    lens = [4, 1, 3]
    B, n_tok = len(lens), sum(lens)
    cu = np.zeros(B + 1, np.int32)
    cu[1:] = np.cumsum(lens)
    c = np.array([3.0, -0.5, 2.0, -1.25, 0.75, 1.5, -4.0, 0.25])[:n_tok]
    e0 = np.zeros(dk, np.float32)
    e0[0] = 1.0
    q = np.tile(_bf(e0), (n_tok, H, 1))
    v = _bf(np.broadcast_to(c[:, None, None], (n_tok, H, dv)))
    alpha = rng.uniform(0.25, 1.0, (n_tok, H, dk)).astype(np.float32)
    alpha[:, :, 0] = 0.0
    beta = np.ones((n_tok, H), np.float32)
    gate = np.zeros((n_tok, H, dv), np.uint16)            # bf16 +0
    weight = rng.uniform(0.5, 2.0, dv).astype(np.float32)
    eps = 1e-6
    cache0 = (rng.standard_normal((4, H, dv, dk)) * 0.3).astype(np.float32)
    slots = np.array([2, 0, 3], np.int32)
    for mode in (oracle.REPLAY, oracle.PER_POSITION):
        plain, _, _, rc = oracle.verify(cache0.copy(), slots, cu, max(lens), q, q, v, alpha, beta,
                                        mode=mode, lib=lib)
        assert rc == 0
        assert np.array_equal(plain, np.broadcast_to(c[:, None, None], plain.shape).astype(np.float32))
        gated, _, _, rc = oracle.verify(cache0.copy(), slots, cu, max(lens), q, q, v, alpha, beta,
                                        mode=mode, gate=gate, weight=weight, eps=eps, lib=lib)
        assert rc == 0
        for t in range(n_tok):
            expect = math.copysign(1.0, c[t]) / math.sqrt(1.0 + eps / (c[t] * c[t])) * weight * 0.5
            for h in range(H):
                assert _rel(gated[t, h], expect) <= 1e-7, (t, h)
    # random inputs: every token's gated output is the gate applied to its own read-out
    w = synth.make(3, 2, 8, 16, seqlens=[3, 1, 4], num_slots=4, state_std=0.3, gate=True, seed=33)
    plain, _, _, _ = oracle.verify(w.cache.copy(), w.slot_ids, w.cu_seqlens, w.T_max, w.q[0], w.k[0],
                                   w.v[0], w.alpha[0], w.beta[0], lib=lib)
    gated, _, _, _ = oracle.verify(w.cache.copy(), w.slot_ids, w.cu_seqlens, w.T_max, w.q[0], w.k[0],
                                   w.v[0], w.alpha[0], w.beta[0], gate=w.gate[0], eps=1e-6, lib=lib)
    gf = synth.bf16_bits_to_f32(w.gate[0]).astype(np.float64)
    for r in range(w.n_tok):
        for h in range(w.H):
            o = plain[r, h].astype(np.float64)
            rms = math.sqrt(float(np.mean(o * o)) + 1e-6)
            assert _rel(gated[r, h], o / rms / (1.0 + np.exp(-gf[r, h]))) <= 1e-6, (r, h)


# ---------------------------------------------------------------- structure

def check_commit_equals_steps(lib):
    w = synth.make(3, 2, 8, 4, seqlens=[4, 4, 4], num_slots=5, state_std=0.1, seed=12)
    cu = w.cu_seqlens
    acc = np.array([1, 3, 4], np.int32)
    # step by step with the single-token driver
    steps = w.cache.copy()
    outs = np.zeros((w.n_tok, w.H, w.dv), np.float32)
    per_pos = {}
    for t in range(4):
        rows = cu[:-1] + t
        o, rc = oracle.decode(steps, w.slot_ids, w.q[0][rows], w.k[0][rows], w.v[0][rows],
                              w.alpha[0][rows], w.beta[0][rows], lib=lib)
        assert rc == 0
        outs[rows] = o
        per_pos[t] = steps[w.slot_ids].copy()
    out, _, draft, rc = oracle.verify(w.cache.copy(), w.slot_ids, cu, 4, w.q[0], w.k[0], w.v[0],
                                      w.alpha[0], w.beta[0], mode=oracle.PER_POSITION, lib=lib)
    assert rc == 0
    assert np.array_equal(out, outs)
    for t in range(4):
        assert np.array_equal(draft[:, t], per_pos[t])
    cache = w.cache.copy()
    rc = oracle.commit(cache, w.slot_ids, cu, acc, 4, w.k[0], w.v[0], w.alpha[0], w.beta[0], lib=lib)
    assert rc == 0
    for b in range(w.B):
        assert np.array_equal(cache[w.slot_ids[b]], per_pos[acc[b] - 1][b])


def check_column_permutation(lib):
    rng = np.random.Generator(np.random.PCG64(13))
    dk, dv, n = 6, 7, 4
    S0 = rng.standard_normal((dk, dv)).astype(np.float32).astype(np.float64)
    q = rng.standard_normal((n, dk))
    k = rng.standard_normal((n, dk))
    v = rng.standard_normal((n, dv))
    a = rng.uniform(0, 1, (n, dk))
    b = rng.uniform(0, 1, n)
    p = rng.permutation(dv)
    o1, S1, _ = oracle.unit(S0, q, k, v, a, b, state_fp32=True, lib=lib)
    o2, S2, _ = oracle.unit(S0[:, p], q, k, v[:, p], a, b, state_fp32=True, lib=lib)
    assert np.array_equal(S1[:, p], S2)
    assert np.array_equal(o1[:, p], o2)


def check_slot_handling(lib):
    w = synth.make(6, 3, 8, 8, num_slots=10, state_std=0.1, seed=14)
    sentinel = np.array([0x7FC0DEAD], np.uint32).view(np.float32)[0]
    slots = w.slot_ids.copy()
    slots[2] = -1                      # padding row
    cache = w.cache.copy()
    out = np.full((w.B, w.H, w.dv), sentinel, np.float32)
    out, rc = oracle.decode(cache, slots, w.q[0], w.k[0], w.v[0], w.alpha[0], w.beta[0], out=out, lib=lib)
    assert rc == 0
    assert np.array_equal(out[2].view(np.uint32), np.full((w.H, w.dv), 0x7FC0DEAD, np.uint32))
    untouched = np.setdiff1d(np.arange(w.num_slots), slots[slots >= 0])
    assert np.array_equal(cache[untouched].view(np.uint32), w.cache[untouched].view(np.uint32))
    live = slots[slots >= 0]
    assert not np.array_equal(cache[live], w.cache[live])
    # permuting (rows, slot ids) permutes the outputs; the cache ends up identical
    p = np.random.Generator(np.random.PCG64(15)).permutation(w.B)
    cache2 = w.cache.copy()
    out2, rc = oracle.decode(cache2, slots[p], w.q[0][p], w.k[0][p], w.v[0][p], w.alpha[0][p],
                             w.beta[0][p], lib=lib)
    assert rc == 0
    assert np.array_equal(cache2.view(np.uint32), cache.view(np.uint32))
    keep = slots[p] >= 0
    assert np.array_equal(out2[keep], out[p][keep])
    # a slot id past the cache: error bit 1, the row is skipped, other rows proceed
    bad = w.slot_ids.copy()
    bad[1] = w.num_slots
    cache3 = w.cache.copy()
    out3 = np.full((w.B, w.H, w.dv), sentinel, np.float32)
    out3, rc = oracle.decode(cache3, bad, w.q[0], w.k[0], w.v[0], w.alpha[0], w.beta[0], out=out3, lib=lib)
    assert rc == oracle.ERR_SLOT
    assert np.all(out3[1].view(np.uint32) == 0x7FC0DEAD)
    same_rows = [0, 3, 4, 5]           # rows with the same slot in both runs
    assert np.array_equal(out3[same_rows], out[same_rows])
    # bad token ranges: error bit 2; accepted length past the row: error bit 4
    v = synth.make(3, 2, 8, 8, seqlens=[2, 3, 1], num_slots=4, state_std=0.1, seed=16)
    cu_bad = v.cu_seqlens.copy()
    cu_bad[2] = cu_bad[1] - 1          # row 1 decreasing
    cache4 = v.cache.copy()
    _, _, _, rc = oracle.verify(cache4, v.slot_ids, cu_bad, 3, v.q[0], v.k[0], v.v[0], v.alpha[0],
                                v.beta[0], lib=lib)
    assert rc & oracle.ERR_SEQLEN
    _, _, _, rc = oracle.verify(v.cache.copy(), v.slot_ids, v.cu_seqlens, 2, v.q[0], v.k[0], v.v[0],
                                v.alpha[0], v.beta[0], lib=lib)
    assert rc == oracle.ERR_SEQLEN   # row 1 has 3 tokens > T_max 2
    cache5 = v.cache.copy()
    rc = oracle.commit(cache5, v.slot_ids, v.cu_seqlens, np.array([2, 4, 1], np.int32), 3,
                       v.k[0], v.v[0], v.alpha[0], v.beta[0], lib=lib)
    assert rc == oracle.ERR_ACCEPTED
    assert np.array_equal(cache5[v.slot_ids[1]], v.cache[v.slot_ids[1]])
    assert not np.array_equal(cache5[v.slot_ids[0]], v.cache[v.slot_ids[0]])


def check_fp32_state_storage(lib):
    rng = np.random.Generator(np.random.PCG64(17))
    dk, dv, n = 6, 5, 8
    S0 = (rng.standard_normal((dk, dv)) * 0.1).astype(np.float32).astype(np.float64)
    q = rng.standard_normal((n, dk))
    k = rng.standard_normal((n, dk)) / math.sqrt(dk)
    v = rng.standard_normal((n, dv))
    a = rng.uniform(0.5, 1, (n, dk))
    b = rng.uniform(0, 1, n)
    _, _, S32 = oracle.unit(S0, q, k, v, a, b, state_fp32=True, lib=lib)
    _, _, S64 = oracle.unit(S0, q, k, v, a, b, state_fp32=False, lib=lib)
    assert np.array_equal(S32, S32.astype(np.float32).astype(np.float64))
    assert not np.array_equal(S64, S64.astype(np.float32).astype(np.float64))
    assert _rel(S32, S64) <= 1e-6


def check_bounded_state(lib):
    # sanity (not parity): with beta in [0, 1], |k| = 1, alpha in [0, 1] the state's
    # spectral norm grows by at most beta |v| per token
    rng = np.random.Generator(np.random.PCG64(18))
    dk, dv, n = 8, 8, 20
    S = rng.standard_normal((dk, dv))
    q = rng.standard_normal((n, dk))
    k = rng.standard_normal((n, dk))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((n, dv))
    a = rng.uniform(0, 1, (n, dk))
    b = rng.uniform(0, 1, n)
    _, _, S_tok = oracle.unit(S, q, k, v, a, b, state_fp32=False, lib=lib)
    prev = np.linalg.norm(S, 2)
    for t in range(n):
        cur = np.linalg.norm(S_tok[t], 2)
        assert cur <= prev + b[t] * np.linalg.norm(v[t]) + 1e-12
        prev = cur


CHECKS = [
    check_golden_steps, check_golden_gate, check_brute_unit, check_brute_batch, check_prefill_brute,
    check_write_then_read, check_alpha_zero, check_beta_zero, check_associative_recall,
    check_linearity, check_gate_closed_form, check_commit_equals_steps,
    check_column_permutation, check_slot_handling, check_fp32_state_storage, check_bounded_state,
    check_prologue_closed_form, check_prologue_prepared_equivalence,
    check_inplace_rows, check_gate_every_token,
]
