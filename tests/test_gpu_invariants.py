"""The recurrence's exact invariants, run through every GPU kernel.

Each holds exactly in real arithmetic and, by the argument in each test's
docstring, exactly in the kernels' floating point too, so most checks compare
with IEEE equality (-0 == +0) rather than a tolerance:
  * alpha = 0 on every key channel at a row's first token erases the committed
    state: every output and state that follows equals the same run from a zero
    state (decode, both verify forms, both buffer modes, the replay commit, both
    prefill forms); zeros on scattered (token, channel) pairs match the oracle;
  * beta = 0 is a pure decay: a single rounding of alpha * s per token, so the
    states equal the oracle's bit for bit wherever the recurrence itself stores
    them (decode, per-position verify, replay commit, recurrent prefill), and
    the chunk forms agree to rounding;
  * beta = 1, alpha = 1 and distinct one-hot keys from a zero state write each
    v_t into its own key row exactly, so a one-hot query returns an earlier v
    exactly, through chunks of 8 tokens (verify) and across the 32-token chunk
    boundary of the chunk prefill.
"""

import numpy as np
import pytest
import torch

import gated_delta_rule_98_amd as K
import oracle
import synth
from gpu_util import dev, f32, i32, log, out_rel, replay_buffers, sentinel, state_rel, step_inputs

pytestmark = pytest.mark.gpu

OUT_TOL = 1e-4
STATE_TOL = 1e-3
H, D, T = 4, 128, 8
VERIFY_FORMS = (K.KDA_VERIFY_RECURRENT, K.KDA_VERIFY_CHUNKED)


def _outputs_and_states(w, cache0, acc):
    """Run w (rows of T tokens) from cache0 through every kernel; return a dict of host arrays."""
    x = step_inputs(w, 0)
    slots = i32(w.slot_ids)
    cu = i32(w.cu_seqlens)
    res = {}
    # decode, token by token
    c = f32(cache0)
    outs = []
    for t in range(w.T_max):
        r = torch.from_numpy((w.cu_seqlens[:-1] + t).astype(np.int64)).to(dev())
        tok = {n: x[n][r].contiguous() for n in ("q", "k", "v", "alpha", "beta")}
        o = torch.empty(w.B, w.H, w.dv, device=dev())
        K.kda_decode_step(c, slots, tok["q"], tok["k"], tok["v"], tok["alpha"], tok["beta"], o)
        outs.append(o)
    torch.cuda.synchronize()
    res["decode_out"] = torch.stack(outs, 1).reshape(w.n_tok, w.H, w.dv).cpu().numpy()
    res["decode_state"] = c.cpu().numpy()[w.slot_ids]
    # verify in both forms, replay mode, then the replay commit
    for form in VERIFY_FORMS:
        c = f32(cache0)
        out = sentinel((w.n_tok, w.H, w.dv))
        rb = replay_buffers(w.B, w.T_max, w.H, w.dk, w.dv)
        K.kda_verify_chunk(c, slots, cu, w.T_max, x["q"], x["k"], x["v"], x["alpha"], x["beta"], out,
                           mode=K.KDA_REPLAY, replay=rb, verify_form=form)
        K.kda_replay_commit(c, slots, cu, i32(acc), w.T_max, w.n_tok, mode=K.KDA_REPLAY, replay=rb)
        torch.cuda.synchronize()
        res[f"verify{form}_out"] = out.cpu().numpy()
        res[f"commit{form}_state"] = c.cpu().numpy()[w.slot_ids]
    # per-position verify: the state after every draft token
    c = f32(cache0)
    out = sentinel((w.n_tok, w.H, w.dv))
    draft = torch.zeros(w.B, w.T_max, w.H, w.dv, w.dk, device=dev())
    K.kda_verify_chunk(c, slots, cu, w.T_max, x["q"], x["k"], x["v"], x["alpha"], x["beta"], out,
                       mode=K.KDA_PER_POSITION, draft=draft)
    torch.cuda.synchronize()
    res["perpos_out"] = out.cpu().numpy()
    res["perpos_draft"] = draft.cpu().numpy()
    # both prefill forms over the same rows, checkpoint after half the row
    pos = i32(np.full(w.B, w.T_max // 2, np.int32))
    for name, fn in (("prefill", K.kda_prefill), ("prefill_chunked", K.kda_prefill_chunked)):
        c = f32(cache0)
        out = sentinel((w.n_tok, w.H, w.dv))
        ckpt = sentinel((w.B, w.H, w.dv, w.dk))
        fn(c, slots, cu, x["q"], x["k"], x["v"], x["alpha"], x["beta"], out, ckpt_pos=pos, ckpt=ckpt)
        torch.cuda.synchronize()
        res[f"{name}_out"] = out.cpu().numpy()
        res[f"{name}_state"] = c.cpu().numpy()[w.slot_ids]
        res[f"{name}_ckpt"] = ckpt.cpu().numpy()
    return res


def _workload(seed, seqlen=T, B=4, state_std=0.5):
    return synth.make(B, H, D, D, seqlens=[seqlen] * B, num_slots=B + 2, state_std=state_std, seed=seed)


def test_alpha_zero_erases_the_state():
    """alpha = 0 on every channel at each row's first token: Diag(0) S0 = 0 exactly (S0 finite),
    so the recurrent kernels continue from an exact zero state, and the chunk forms multiply
    S0 only by decay products that contain that factor, all exactly zero. Every output and
    state equals the same run from a zero cache."""
    w = _workload(51)
    w.alpha[0][w.cu_seqlens[:-1]] = 0.0
    acc = np.array([1, 3, 8, 5], np.int32)
    log("alpha = 0 at the first token: random committed states")
    a = _outputs_and_states(w, w.cache, acc)
    log("alpha = 0 at the first token: zero committed states")
    z = _outputs_and_states(w, np.zeros_like(w.cache), acc)
    for key in a:
        assert np.array_equal(a[key], z[key]), key
    # and against the oracle from the random states
    ref_out, _, _, rc = oracle.verify(w.cache.copy(), w.slot_ids, w.cu_seqlens, w.T_max, w.q[0], w.k[0], w.v[0],
                                      w.alpha[0], w.beta[0])
    assert rc == 0
    assert out_rel(a[f"verify{K.KDA_VERIFY_CHUNKED}_out"], ref_out, "chunk verify outputs") <= OUT_TOL


def test_scattered_alpha_zeros_match_the_oracle():
    """alpha = 0 on a random fifth of the (token, channel) pairs, through every kernel, against
    the oracle (which the erasure closed form pins)."""
    w = _workload(52, state_std=0.05)
    mask = np.random.Generator(np.random.PCG64(53)).random(w.alpha[0].shape) < 0.2
    w.alpha[0][mask] = 0.0
    acc = np.array([8, 2, 7, 4], np.int32)
    log("scattered alpha zeros")
    g = _outputs_and_states(w, w.cache, acc)
    ref_out, _, ref_draft, rc = oracle.verify(w.cache.copy(), w.slot_ids, w.cu_seqlens, w.T_max, w.q[0], w.k[0],
                                              w.v[0], w.alpha[0], w.beta[0], mode=oracle.PER_POSITION)
    assert rc == 0
    for key in ("decode_out", "perpos_out", "prefill_out", "prefill_chunked_out") + tuple(
            f"verify{f}_out" for f in VERIFY_FORMS):
        assert out_rel(g[key], ref_out, key) <= OUT_TOL
    assert state_rel(g["perpos_draft"], ref_draft, "per-position states") <= STATE_TOL
    cache_h = w.cache.copy()
    assert oracle.commit(cache_h, w.slot_ids, w.cu_seqlens, acc, w.T_max, w.k[0], w.v[0], w.alpha[0],
                         w.beta[0]) == 0
    for form in VERIFY_FORMS:
        assert state_rel(g[f"commit{form}_state"], cache_h[w.slot_ids], "committed states") <= STATE_TOL
    cache_p = w.cache.copy()
    _, ref_ckpt, rc = oracle.prefill(cache_p, w.slot_ids, w.cu_seqlens, w.q[0], w.k[0], w.v[0], w.alpha[0],
                                     w.beta[0], ckpt_pos=np.full(w.B, w.T_max // 2, np.int32))
    assert rc == 0
    for name in ("prefill", "prefill_chunked"):
        assert state_rel(g[f"{name}_state"], cache_p[w.slot_ids], f"{name} final states") <= STATE_TOL
        assert state_rel(g[f"{name}_ckpt"], ref_ckpt, f"{name} checkpoints") <= STATE_TOL


def test_beta_zero_is_a_pure_decay():
    """beta = 0 on rows 0 and 2: the write adds k * 0, so each token leaves fl(alpha * s), one
    rounding of a product that is exact in double; the oracle's state is then bit-identical
    wherever a kernel stores the recurrence's own state. Rows 1 and 3 keep random beta."""
    w = _workload(54, state_std=0.05)
    zero_rows = [0, 2]
    for b in zero_rows:
        w.beta[0][w.cu_seqlens[b]:w.cu_seqlens[b + 1]] = 0.0
    acc = np.array([8, 3, 5, 8], np.int32)
    log("beta = 0 rows")
    g = _outputs_and_states(w, w.cache, acc)
    ref_out, _, ref_draft, rc = oracle.verify(w.cache.copy(), w.slot_ids, w.cu_seqlens, w.T_max, w.q[0], w.k[0],
                                              w.v[0], w.alpha[0], w.beta[0], mode=oracle.PER_POSITION)
    assert rc == 0
    for key in ("decode_out", "perpos_out", "prefill_out", "prefill_chunked_out") + tuple(
            f"verify{f}_out" for f in VERIFY_FORMS):
        assert out_rel(g[key], ref_out, key) <= OUT_TOL
    decayed = w.cache[w.slot_ids].astype(np.float64)
    cache_h = w.cache.copy()
    assert oracle.commit(cache_h, w.slot_ids, w.cu_seqlens, acc, w.T_max, w.k[0], w.v[0], w.alpha[0],
                         w.beta[0]) == 0
    cache_p = w.cache.copy()
    assert oracle.prefill(cache_p, w.slot_ids, w.cu_seqlens, w.q[0], w.k[0], w.v[0], w.alpha[0], w.beta[0])[2] == 0
    cache_d = w.cache.copy()
    assert oracle.commit(cache_d, w.slot_ids, w.cu_seqlens, np.full(w.B, w.T_max, np.int32), w.T_max, w.k[0], w.v[0],
                         w.alpha[0], w.beta[0]) == 0
    for b in zero_rows:
        s = w.slot_ids[b]
        assert np.array_equal(g["decode_state"][b], cache_d[s]), b
        assert np.array_equal(g["prefill_state"][b], cache_p[s]), b
        assert np.array_equal(g["perpos_draft"][b], ref_draft[b]), b
        for form in VERIFY_FORMS:
            assert np.array_equal(g[f"commit{form}_state"][b], cache_h[s]), (b, form)
        # the closed form Diag(prod alpha) S0, to the rounding of the per-token products
        prod = np.prod(w.alpha[0][w.cu_seqlens[b]:w.cu_seqlens[b + 1]].astype(np.float64), axis=0)   # [H][dk]
        expect = decayed[b] * prod[:, None, :]
        assert state_rel(g["prefill_chunked_state"][b], expect, "chunk prefill pure decay") <= 1e-5
    assert state_rel(g["prefill_chunked_state"], cache_p[w.slot_ids], "chunk prefill states") <= STATE_TOL


def _one_hot_rows(seed, seqlen, B=4):
    """Distinct one-hot keys per (row, head), alpha = beta = 1, zero state; token t's query is the
    key of an earlier token r_t <= t, so o_t = v_{r_t} exactly."""
    w = synth.make(B, H, D, D, seqlens=[seqlen] * B, num_slots=B + 2, state_std=0.0, seed=seed)
    rng = np.random.Generator(np.random.PCG64(seed + 1))
    k = np.zeros((w.n_tok, H, D), np.float32)
    q = np.zeros((w.n_tok, H, D), np.float32)
    src = np.zeros((w.n_tok, H), np.int64)
    keys = np.zeros((w.n_tok, H), np.int64)
    for b in range(B):
        for h in range(H):
            perm = rng.permutation(D)[:seqlen]
            for t in range(seqlen):
                r = w.cu_seqlens[b] + t
                keys[r, h] = perm[t]
                k[r, h, perm[t]] = 1.0
                rt = rng.integers(0, t + 1)
                q[r, h, perm[rt]] = 1.0
                src[r, h] = w.cu_seqlens[b] + rt
    w.k = synth.f32_to_bf16_bits(k)[None]
    w.q = synth.f32_to_bf16_bits(q)[None]
    w.alpha = np.ones_like(w.alpha)
    w.beta = np.ones_like(w.beta)
    return w, src, keys


def _expected_state(w, keys, b, n):
    """State of row b after its first n tokens, in the cache layout [H][dv][dk]."""
    v = synth.bf16_bits_to_f32(w.v[0])
    S = np.zeros((H, D, D), np.float32)
    for t in range(n):
        r = w.cu_seqlens[b] + t
        for h in range(H):
            S[h, :, keys[r, h]] = v[r, h]
    return S


def test_one_hot_write_then_read():
    """beta = 1, alpha = 1, distinct one-hot keys, zero state: u = S^T k reads an empty row, so
    the write stores v exactly; the chunk forms' coupling A is exactly zero (distinct keys), so
    their solve is the identity and their products add exact zeros. Every output equals the v
    its query names, and every stored state holds exactly the accepted v's, through T = 8
    verify chunks and a 40-token prefill that crosses the 32-token chunk boundary."""
    w, src, keys = _one_hot_rows(55, T)
    vf = synth.bf16_bits_to_f32(w.v[0])
    acc = np.array([8, 1, 4, 6], np.int32)
    log("one-hot write-then-read, rows of 8 tokens")
    g = _outputs_and_states(w, w.cache, acc)
    expect_out = np.take_along_axis(vf, src[:, :, None], axis=0)
    for key in ("decode_out", "perpos_out", "prefill_out", "prefill_chunked_out") + tuple(
            f"verify{f}_out" for f in VERIFY_FORMS):
        assert np.array_equal(g[key], expect_out), key
    for b in range(w.B):
        full = _expected_state(w, keys, b, T)
        assert np.array_equal(g["decode_state"][b], full), b
        assert np.array_equal(g["prefill_state"][b], full), b
        assert np.array_equal(g["prefill_chunked_state"][b], full), b
        half = _expected_state(w, keys, b, T // 2)
        assert np.array_equal(g["prefill_ckpt"][b], half), b
        assert np.array_equal(g["prefill_chunked_ckpt"][b], half), b
        for form in VERIFY_FORMS:
            assert np.array_equal(g[f"commit{form}_state"][b], _expected_state(w, keys, b, acc[b])), (b, form)
        for t in range(T):
            assert np.array_equal(g["perpos_draft"][b, t], _expected_state(w, keys, b, t + 1)), (b, t)
    # a longer prompt through both prefill forms: 40 tokens cross the 32-token chunk boundary
    p, psrc, pkeys = _one_hot_rows(56, 40, B=2)
    x = step_inputs(p, 0)
    for name, fn in (("prefill", K.kda_prefill), ("prefill_chunked", K.kda_prefill_chunked)):
        log(f"one-hot write-then-read, 40-token {name}")
        c = f32(p.cache)
        out = sentinel((p.n_tok, H, D))
        ckpt = sentinel((p.B, H, D, D))
        fn(c, i32(p.slot_ids), i32(p.cu_seqlens), x["q"], x["k"], x["v"], x["alpha"], x["beta"], out,
           ckpt_pos=i32([33, 7]), ckpt=ckpt)
        torch.cuda.synchronize()
        pv = synth.bf16_bits_to_f32(p.v[0])
        assert np.array_equal(out.cpu().numpy(), np.take_along_axis(pv, psrc[:, :, None], axis=0)), name
        got = c.cpu().numpy()
        ck = ckpt.cpu().numpy()
        for b, at in enumerate((33, 7)):
            assert np.array_equal(got[p.slot_ids[b]], _expected_state(p, pkeys, b, 40)), (name, b)
            assert np.array_equal(ck[b], _expected_state(p, pkeys, b, at)), (name, b)
