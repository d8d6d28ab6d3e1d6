"""GPU parity of the raw-input mode and the bf16 output, through the C ABI.

Raw inputs: q, k, alpha, beta are the raw projections and every kernel prepares
them (q/k L2 normalization with 1/sqrt(dk) on q, alpha = exp(-softplus(a)),
beta = sigmoid(b)) before the recurrence. Checked against the oracle's
raw-input mode at the usual tolerances (each step's output within 1e-4
relative L2, states within 1e-3 relative Frobenius), and bit for bit across
ops: n decode steps, verify drafts, replay commit and the prefill checkpoint
all give the same state bits, and every tile width gives the same bits.

bf16 output: each output is the round-to-nearest-even bf16 of the fp32 output
the same call computes without the flag, bit for bit, for decode, verify (with
and without the output gate) and prefill.
"""

import numpy as np
import pytest
import torch

import gated_delta_rule_98_amd as K
import oracle
import synth
from gpu_util import (bits, dev, f32, i32, log, raw_step_inputs, out_rel, state_rel, replay_buffers, sentinel,
                      step_inputs)

pytestmark = pytest.mark.gpu

OUT_TOL = 1e-4
STATE_TOL = 1e-3


def _decode_run(w, tile_w=0, steps=None):
    cache_d = f32(w.cache)
    slots_d = i32(w.slot_ids)
    steps = w.steps if steps is None else steps
    outs = torch.empty(steps, w.B, w.H, w.dv, device=dev())
    for s in range(steps):
        x = raw_step_inputs(w, s)
        K.kda_decode_step(cache_d, slots_d, x["q"], x["k"], x["v"], x["alpha"], x["beta"], outs[s],
                          tile_w=tile_w, raw_inputs=True)
    torch.cuda.synchronize()
    return cache_d, outs


def _oracle_decode_run(w, steps=None):
    cache_h = w.cache.copy()
    steps = w.steps if steps is None else steps
    outs = []
    for s in range(steps):
        o, rc = oracle.decode(cache_h, w.slot_ids, w.q_raw[s], w.k_raw[s], w.v[s], w.a_raw[s], w.b_raw[s],
                              prologue=True)
        assert rc == 0
        outs.append(o)
    return cache_h, outs


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (64, 128)])
def test_decode_raw_inputs_match_oracle_and_widths_agree(dk, dv):
    w = synth.make(8, 4, dk, dv, steps=12, num_slots=11, state_std=0.02, seed=31)
    ref_cache, ref_outs = _oracle_decode_run(w)
    first = None
    for tile_w in (0, 2, 4, 16, 64):
        if tile_w > dv or (tile_w == 2 and dk != 128):
            continue
        log(f"raw decode dk={dk} dv={dv} tile_w={tile_w}: {w.steps} steps")
        cache_d, outs = _decode_run(w, tile_w)
        got = cache_d.cpu().numpy()
        worst = max(out_rel(outs[s].cpu().numpy(), ref_outs[s]) for s in range(w.steps))
        serr = state_rel(got[w.slot_ids], ref_cache[w.slot_ids])
        log(f"  worst step rel-L2 (worst of whole, per head) {worst:.3e}, state rel-Frobenius (worst of whole, per head) {serr:.3e}")
        assert worst <= OUT_TOL and serr <= STATE_TOL
        untouched = np.setdiff1d(np.arange(w.num_slots), w.slot_ids)
        assert np.array_equal(got[untouched].view(np.uint32), w.cache[untouched].view(np.uint32))
        if first is None:
            first = (bits(cache_d), bits(outs))
        else:
            assert np.array_equal(bits(cache_d), first[0]) and np.array_equal(bits(outs), first[1])


def test_b1_latency_raw_inputs_1024_steps():
    w = synth.make_workload("b1_latency")
    log("raw decode b1_latency: 1024 steps")
    cache_d, outs = _decode_run(w)
    ref_cache, ref_outs = _oracle_decode_run(w)
    outs_h = outs.cpu().numpy()
    worst = max(out_rel(outs_h[s], ref_outs[s]) for s in range(w.steps))
    serr = state_rel(cache_d.cpu().numpy(), ref_cache)
    log(f"  worst step rel-L2 (worst of whole, per head) {worst:.3e}, state rel-Frobenius (worst of whole, per head) after 1024 steps {serr:.3e}")
    assert worst <= OUT_TOL and serr <= STATE_TOL


def test_raw_inputs_states_bit_identical_across_ops():
    """n raw decode steps == verify drafts == replay commit == prefill checkpoint, bit for bit."""
    w = synth.make(6, 4, 128, 128, seqlens=[8] * 6, num_slots=9, state_std=0.02, seed=32)
    acc = w.accepted
    x = raw_step_inputs(w, 0)
    cu = w.cu_seqlens
    slots_d = i32(w.slot_ids)
    dec_d = f32(w.cache)
    dec_out = torch.empty(w.n_tok, w.H, w.dv, device=dev())
    per_pos = []
    for t in range(8):
        r = torch.from_numpy((cu[:-1] + t).astype(np.int64)).to(dev())
        tok = {n: x[n][r].contiguous() for n in ("q", "k", "v", "alpha", "beta")}
        o = torch.empty(w.B, w.H, w.dv, device=dev())
        log(f"raw single-token step {t}")
        K.kda_decode_step(dec_d, slots_d, tok["q"], tok["k"], tok["v"], tok["alpha"], tok["beta"], o,
                          raw_inputs=True)
        dec_out[r] = o
        per_pos.append(bits(dec_d)[w.slot_ids])
    # per-position drafts
    log("raw verify, per-position mode")
    cache_p = f32(w.cache)
    out_p = sentinel((w.n_tok, w.H, w.dv))
    draft = torch.zeros(w.B, 8, w.H, w.dv, w.dk, device=dev())
    K.kda_verify_chunk(cache_p, slots_d, i32(cu), 8, x["q"], x["k"], x["v"], x["alpha"], x["beta"], out_p,
                       mode=K.KDA_PER_POSITION, draft=draft, raw_inputs=True)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out_p), bits(dec_out))
    d = bits(draft)
    for t in range(8):
        assert np.array_equal(d[:, t], per_pos[t]), t
    # replay buffer holds the raw inputs; the raw commit rebuilds the accepted states
    log("raw verify, replay mode, then raw replay commit")
    cache_r = f32(w.cache)
    rb = replay_buffers(w.B, 8, w.H, w.dk, w.dv)
    out_r = sentinel((w.n_tok, w.H, w.dv))
    K.kda_verify_chunk(cache_r, slots_d, i32(cu), 8, x["q"], x["k"], x["v"], x["alpha"], x["beta"], out_r,
                       mode=K.KDA_REPLAY, replay=rb, raw_inputs=True)
    K.kda_replay_commit(cache_r, slots_d, i32(cu), i32(acc), 8, w.n_tok, mode=K.KDA_REPLAY, replay=rb,
                        raw_inputs=True)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out_r), bits(dec_out))
    assert np.array_equal(bits(rb["k"]), w.k_raw[0].reshape(w.B, 8, w.H, w.dk))
    assert np.array_equal(bits(rb["alpha"]), w.a_raw[0].reshape(w.B, 8, w.H, w.dk).view(np.uint32))
    assert np.array_equal(bits(rb["beta"]), w.b_raw[0].reshape(w.B, 8, w.H).view(np.uint32))
    got = bits(cache_r)[w.slot_ids]
    for b in range(w.B):
        assert np.array_equal(got[b], per_pos[acc[b] - 1][b]), b
    # prefill with the checkpoint at the accepted length
    log("raw prefill with checkpoints")
    cache_f = f32(w.cache)
    out_f = sentinel((w.n_tok, w.H, w.dv))
    ckpt = sentinel((w.B, w.H, w.dv, w.dk))
    K.kda_prefill(cache_f, slots_d, i32(cu), x["q"], x["k"], x["v"], x["alpha"], x["beta"], out_f,
                  ckpt_pos=i32(acc), ckpt=ckpt, raw_inputs=True)
    torch.cuda.synchronize()
    assert np.array_equal(bits(cache_f)[w.slot_ids], per_pos[7])
    c = bits(ckpt)
    for b in range(w.B):
        assert np.array_equal(c[b], per_pos[acc[b] - 1][b]), b
    assert out_rel(out_f.cpu().numpy(), dec_out.cpu().numpy()) <= 1e-5
    # and all of it against the oracle's raw-input mode
    ref_out, ref_ckpt, rc = oracle.prefill(w.cache.copy(), w.slot_ids, cu, w.q_raw[0], w.k_raw[0], w.v[0],
                                           w.a_raw[0], w.b_raw[0], ckpt_pos=acc, prologue=True)
    assert rc == 0
    assert out_rel(out_f.cpu().numpy(), ref_out) <= OUT_TOL
    assert state_rel(ckpt.cpu().numpy(), ref_ckpt) <= STATE_TOL


def test_raw_inputs_with_output_gate():
    w = synth.make(5, 4, 128, 128, seqlens=[1, 4, 1, 3, 4], num_slots=7, state_std=0.02, gate=True, seed=33)
    x = raw_step_inputs(w, 0)
    weight = np.linspace(0.5, 1.5, w.dv).astype(np.float32)
    log("raw verify with output gate, in-place single-token rows")
    cache_d = f32(w.cache)
    out = sentinel((w.n_tok, w.H, w.dv))
    rb = replay_buffers(w.B, w.T_max, w.H, w.dk, w.dv)
    K.kda_verify_chunk(cache_d, i32(w.slot_ids), i32(w.cu_seqlens), w.T_max, x["q"], x["k"], x["v"],
                       x["alpha"], x["beta"], out, mode=K.KDA_REPLAY, t1_inplace=True, replay=rb,
                       gate=x["gate"], weight=f32(weight), eps=1e-6, raw_inputs=True)
    torch.cuda.synchronize()
    cache_h = w.cache.copy()
    ref, _, _, rc = oracle.verify(cache_h, w.slot_ids, w.cu_seqlens, w.T_max, w.q_raw[0], w.k_raw[0], w.v[0],
                                  w.a_raw[0], w.b_raw[0], mode=oracle.REPLAY, t1_inplace=True, gate=w.gate[0],
                                  weight=weight, eps=1e-6, prologue=True)
    assert rc == 0
    err = out_rel(out.cpu().numpy(), ref)
    serr = state_rel(cache_d.cpu().numpy(), cache_h)
    log(f"  outputs rel-L2 (worst of whole, per head) {err:.3e}, in-place states rel-Frobenius (worst of whole, per head) {serr:.3e}")
    assert err <= OUT_TOL and serr <= STATE_TOL
    # gated single-token step
    w1 = synth.make(6, 4, 128, 128, num_slots=6, state_std=0.02, gate=True, seed=34)
    x1 = raw_step_inputs(w1, 0)
    log("raw decode with output gate")
    cache_d = f32(w1.cache)
    out = sentinel((w1.B, w1.H, w1.dv))
    K.kda_decode_step(cache_d, i32(w1.slot_ids), x1["q"], x1["k"], x1["v"], x1["alpha"], x1["beta"], out,
                      gate=x1["gate"], weight=f32(weight), eps=1e-6, raw_inputs=True)
    torch.cuda.synchronize()
    cache_h = w1.cache.copy()
    ref, rc = oracle.decode(cache_h, w1.slot_ids, w1.q_raw[0], w1.k_raw[0], w1.v[0], w1.a_raw[0], w1.b_raw[0],
                            gate=w1.gate[0], weight=weight, eps=1e-6, prologue=True)
    assert rc == 0
    assert out_rel(out.cpu().numpy(), ref) <= OUT_TOL
    assert state_rel(cache_d.cpu().numpy(), cache_h) <= STATE_TOL


def _bf16_of(t: torch.Tensor) -> np.ndarray:
    return synth.f32_to_bf16_bits(t.cpu().numpy())


@pytest.mark.parametrize("raw", [False, True])
def test_bf16_output_is_rounded_fp32_output(raw):
    w = synth.make(6, 4, 128, 128, seqlens=[1, 5, 3, 1, 8, 2], num_slots=8, state_std=0.02, gate=True, seed=35)
    x = raw_step_inputs(w, 0) if raw else step_inputs(w, 0)
    slots_d, cu_d = i32(w.slot_ids), i32(w.cu_seqlens)
    rows = torch.from_numpy(w.cu_seqlens[:-1].astype(np.int64)).to(dev())
    first = {n: x[n][rows].contiguous() for n in ("q", "k", "v", "alpha", "beta", "gate")}
    for gate in (False, True):
        g = first["gate"] if gate else None
        for tw in (0,) if gate else (0, 2):
            log(f"bf16 output: decode gate={gate} raw={raw} tile_w={tw}")
            outs = []
            for o in (torch.empty(w.B, w.H, w.dv, device=dev()),
                      torch.empty(w.B, w.H, w.dv, device=dev(), dtype=torch.bfloat16)):
                cache_d = f32(w.cache)
                K.kda_decode_step(cache_d, slots_d, first["q"], first["k"], first["v"], first["alpha"],
                                  first["beta"], o, gate=g, raw_inputs=raw, tile_w=tw)
                outs.append(o)
            torch.cuda.synchronize()
            assert np.array_equal(bits(outs[1]), _bf16_of(outs[0]))
        log(f"bf16 output: verify gate={gate} raw={raw}")
        outs = []
        for o in (torch.empty(w.n_tok, w.H, w.dv, device=dev()),
                  torch.empty(w.n_tok, w.H, w.dv, device=dev(), dtype=torch.bfloat16)):
            cache_d = f32(w.cache)
            K.kda_verify_chunk(cache_d, slots_d, cu_d, w.T_max, x["q"], x["k"], x["v"], x["alpha"], x["beta"],
                               o, mode=K.KDA_PER_POSITION, t1_inplace=True,
                               draft=torch.zeros(w.B, w.T_max, w.H, w.dv, w.dk, device=dev()),
                               gate=x["gate"] if gate else None, raw_inputs=raw)
            outs.append(o)
        torch.cuda.synchronize()
        assert np.array_equal(bits(outs[1]), _bf16_of(outs[0]))
    log(f"bf16 output: prefill raw={raw}")
    outs = []
    for o in (torch.empty(w.n_tok, w.H, w.dv, device=dev()),
              torch.empty(w.n_tok, w.H, w.dv, device=dev(), dtype=torch.bfloat16)):
        cache_d = f32(w.cache)
        K.kda_prefill(cache_d, slots_d, cu_d, x["q"], x["k"], x["v"], x["alpha"], x["beta"], o, raw_inputs=raw)
        outs.append(o)
    torch.cuda.synchronize()
    assert np.array_equal(bits(outs[1]), _bf16_of(outs[0]))
    # and the rounded output against the oracle (bf16 spacing is 2^-8 relative)
    ref, _, rc = oracle.prefill(w.cache.copy(), w.slot_ids, w.cu_seqlens,
                                w.q_raw[0] if raw else w.q[0], w.k_raw[0] if raw else w.k[0], w.v[0],
                                w.a_raw[0] if raw else w.alpha[0], w.b_raw[0] if raw else w.beta[0],
                                prologue=raw)
    assert rc == 0
    got = synth.bf16_bits_to_f32(bits(outs[1]))
    assert out_rel(got, ref) <= 2.0 ** -8


def test_raw_replay_commit_both_staging_orders():
    """Raw-input replay commit in both staging orders (the state tile first at 2048 workgroups,
    the inputs first at 8192: 16 rows x 32 heads at 32 and 8 columns per workgroup): the same
    bits, and the oracle's raw-input commit within the state tolerance."""
    w = synth.make(16, 32, 128, 128, seqlens=[8] * 16, num_slots=20, state_std=0.02, seed=36)
    x = raw_step_inputs(w, 0)
    cu, acc = w.cu_seqlens, w.accepted
    cache_v = f32(w.cache)
    rb = replay_buffers(w.B, 8, w.H, w.dk, w.dv)
    out = sentinel((w.n_tok, w.H, w.dv))
    log("raw verify (replay mode) for the commit orders")
    K.kda_verify_chunk(cache_v, i32(w.slot_ids), i32(cu), 8, x["q"], x["k"], x["v"], x["alpha"], x["beta"], out,
                       mode=K.KDA_REPLAY, replay=rb, raw_inputs=True)
    got = []
    for tw in (32, 8):
        cache_c = f32(w.cache)
        log(f"raw replay commit, tile_w={tw}")
        K.kda_replay_commit(cache_c, i32(w.slot_ids), i32(cu), i32(acc), 8, w.n_tok, mode=K.KDA_REPLAY, replay=rb,
                            raw_inputs=True, tile_w=tw)
        torch.cuda.synchronize()
        got.append(bits(cache_c))
    assert np.array_equal(got[0], got[1])
    ref = w.cache.copy()
    assert oracle.commit(ref, w.slot_ids, cu, acc, 8, w.k_raw[0], w.v[0], w.a_raw[0], w.b_raw[0], prologue=True) == 0
    assert state_rel(got[0].view(np.float32)[w.slot_ids], ref[w.slot_ids]) <= STATE_TOL
