"""GPU parity of kda_verify_chunk and kda_replay_commit against the CPU oracle.

Covers the speculative-verify workload (B=16, H=32, d=128, 8 drafts, accepted
length uniform in 1..8) in both buffer modes, the mixed zero-copy batch (40
single-token rows updated in place plus 24 rows of 4 verified tokens, output
gate, 512-slot cache), ragged and empty rows, device-side errors, and the bit
identities: both commit modes leave the same slot bits, equal to that many
single-token steps, and verify outputs equal the single-token outputs.
"""

import numpy as np
import pytest
import torch

import gated_delta_rule_98_amd as K
import oracle
import synth
from gpu_util import (SENTINEL_BITS, bits, dev, f32, i32, log, out_rel, state_rel, replay_buffers, sentinel,
                      step_inputs)

pytestmark = pytest.mark.gpu

OUT_TOL = 1e-4
STATE_TOL = 1e-3


def _verify(w, cache_d, mode, *, t1_inplace=False, gate=False, weight=None, tile_w=0, slots=None, cu=None,
            dev_err=None, form=0):
    x = step_inputs(w, 0)
    slots = w.slot_ids if slots is None else slots
    cu = w.cu_seqlens if cu is None else cu
    out = sentinel((w.n_tok, w.H, w.dv))
    rb = replay_buffers(w.B, w.T_max, w.H, w.dk, w.dv) if mode == K.KDA_REPLAY else None
    draft = torch.zeros(w.B, w.T_max, w.H, w.dv, w.dk, device=dev()) if mode == K.KDA_PER_POSITION else None
    K.kda_verify_chunk(cache_d, i32(slots), i32(cu), w.T_max, x["q"], x["k"], x["v"], x["alpha"], x["beta"],
                       out, mode=mode, t1_inplace=t1_inplace, replay=rb, draft=draft,
                       gate=x["gate"] if gate else None, weight=weight, eps=1e-6, dev_err=dev_err,
                       tile_w=tile_w, verify_form=form)
    return out, rb, draft


def _commit(w, cache_d, mode, acc, rb, draft, *, tile_w=0, slots=None, cu=None, dev_err=None):
    slots = w.slot_ids if slots is None else slots
    cu = w.cu_seqlens if cu is None else cu
    K.kda_replay_commit(cache_d, i32(slots), i32(cu), i32(acc), w.T_max, w.n_tok, mode=mode, replay=rb,
                        draft=draft, dev_err=dev_err, tile_w=tile_w)


def _oracle_verify(w, mode, **kw):
    return oracle.verify(w.cache.copy(), kw.pop("slots", w.slot_ids), kw.pop("cu", w.cu_seqlens), w.T_max,
                         w.q[0], w.k[0], w.v[0], w.alpha[0], w.beta[0], mode=mode, **kw)


@pytest.mark.parametrize("B", [16, 64], ids=["b16", "b64"])
def test_spec_verify_both_modes_and_commit(B):
    """The speculative-verify workload (B=16) and the same at B=64, where the chunk form issues
    its state with its inputs and the replay commit its inputs before the state."""
    if B == 16:
        w = synth.make_workload("spec_verify")
    else:
        w = synth.make(B, 32, 128, 128, seqlens=[8] * B, num_slots=256, state_std=0.02, seed=64,
                       name="spec_verify_b64")
    acc = w.accepted
    results = {}
    for mode in (K.KDA_REPLAY, K.KDA_PER_POSITION):
        cache_d = f32(w.cache)
        log(f"spec_verify B={w.B}: verify mode {mode}")
        out, rb, draft = _verify(w, cache_d, mode)
        torch.cuda.synchronize()
        assert np.array_equal(bits(cache_d), w.cache.view(np.uint32))   # verify wrote no slot
        ref_out, ref_rb, ref_draft, rc = _oracle_verify(w, mode)
        assert rc == 0
        err = out_rel(out.cpu().numpy(), ref_out)
        log(f"  outputs rel-L2 (worst of whole, per head) {err:.3e}")
        assert err <= OUT_TOL
        if mode == K.KDA_REPLAY:
            assert np.array_equal(bits(rb["k"]), ref_rb["rk"])
            assert np.array_equal(bits(rb["v"]), ref_rb["rv"])
            assert np.array_equal(bits(rb["alpha"]), ref_rb["ralpha"].view(np.uint32))
            assert np.array_equal(bits(rb["beta"]), ref_rb["rbeta"].view(np.uint32))
        else:
            d = draft.cpu().numpy()
            derr = state_rel(d, ref_draft)
            log(f"  per-position states rel-Frobenius (worst of whole, per head) {derr:.3e}")
            assert derr <= STATE_TOL
        log(f"spec_verify B={w.B}: commit mode {mode}")
        _commit(w, cache_d, mode, acc, rb, draft)
        torch.cuda.synchronize()
        results[mode] = (bits(out), bits(cache_d))
    # both modes: the same committed slot bits; outputs agree to rounding (replay mode
    # computes them in chunk form, per-position mode token by token)
    assert out_rel(results[0][0].view(np.float32), results[1][0].view(np.float32)) <= 1e-5
    assert np.array_equal(results[0][1], results[1][1])
    cache_h = w.cache.copy()
    assert oracle.commit(cache_h, w.slot_ids, w.cu_seqlens, acc, w.T_max, w.k[0], w.v[0], w.alpha[0],
                         w.beta[0]) == 0
    got = results[0][1].view(np.float32)
    serr = state_rel(got[w.slot_ids], cache_h[w.slot_ids])
    log(f"  committed states rel-Frobenius (worst of whole, per head) {serr:.3e}")
    assert serr <= STATE_TOL
    untouched = np.setdiff1d(np.arange(w.num_slots), w.slot_ids)
    assert np.array_equal(results[0][1][untouched], w.cache[untouched].view(np.uint32))


def test_commit_equals_single_token_steps_bitwise():
    """Replay commit of a tokens == a calls of kda_decode_step; verify outputs == decode outputs."""
    w = synth.make_workload("spec_verify")
    acc = w.accepted
    x = step_inputs(w, 0)
    steps_d = f32(w.cache)     # only the accepted prefix of each row (others padded with slot -1)
    all_d = f32(w.cache)       # every draft token of every row
    dec_out = torch.empty(w.n_tok, w.H, w.dv, device=dev())
    for t in range(w.T_max):
        r = torch.from_numpy((w.cu_seqlens[:-1] + t).astype(np.int64)).to(dev())
        tok = {n: x[n][r].contiguous() for n in ("q", "k", "v", "alpha", "beta")}
        masked = np.where(acc > t, w.slot_ids, -1).astype(np.int32)
        o = torch.empty(w.B, w.H, w.dv, device=dev())
        log(f"single-token step {t}")
        K.kda_decode_step(steps_d, i32(masked), tok["q"], tok["k"], tok["v"], tok["alpha"], tok["beta"], o)
        K.kda_decode_step(all_d, i32(w.slot_ids), tok["q"], tok["k"], tok["v"], tok["alpha"], tok["beta"], o)
        dec_out[r] = o
    for form in (K.KDA_VERIFY_RECURRENT, K.KDA_VERIFY_CHUNKED):
        cache_r = f32(w.cache)
        log(f"verify (form {form}) + replay commit")
        out, rb, _ = _verify(w, cache_r, K.KDA_REPLAY, form=form)
        _commit(w, cache_r, K.KDA_REPLAY, acc, rb, None)
        torch.cuda.synchronize()
        assert np.array_equal(bits(cache_r), bits(steps_d))
        if form == K.KDA_VERIFY_RECURRENT:
            assert np.array_equal(bits(out), bits(dec_out))
        else:
            assert out_rel(out.cpu().numpy(), dec_out.cpu().numpy()) <= 1e-5
    # both staging orders of the replay commit: at this shape (16 rows x 32 heads) 32-column
    # tiles give 2048 workgroups (state tile first), 16 and 8 columns 4096 and 8192 (inputs first)
    cache_v = f32(w.cache)
    _, rb, _ = _verify(w, cache_v, K.KDA_REPLAY)
    for tw in (32, 16, 8):
        cache_c = f32(w.cache)
        log(f"replay commit, tile_w={tw}")
        _commit(w, cache_c, K.KDA_REPLAY, acc, rb, None, tile_w=tw)
        torch.cuda.synchronize()
        assert np.array_equal(bits(cache_c), bits(steps_d)), tw


def test_mixed_batch_inplace_gate_and_commit():
    """40 single-token rows in place + 24 rows of 4 verified tokens, output gate, then commit."""
    w = synth.make_workload("mixed")
    weight = np.random.Generator(np.random.PCG64(31)).uniform(0.5, 2.0, w.dv).astype(np.float32)
    cache_d = f32(w.cache)
    acc = w.accepted.copy()              # 0 for the single-token rows (already updated in place)
    log("mixed: verify with in-place singles, replay buffers, output gate")
    out, rb, _ = _verify(w, cache_d, K.KDA_REPLAY, t1_inplace=True, gate=True, weight=f32(weight))
    torch.cuda.synchronize()
    cache_h = w.cache.copy()
    ref_out, ref_rb, _, rc = oracle.verify(cache_h, w.slot_ids, w.cu_seqlens, w.T_max, w.q[0], w.k[0], w.v[0],
                                           w.alpha[0], w.beta[0], mode=oracle.REPLAY, t1_inplace=True,
                                           gate=w.gate[0], weight=weight, eps=1e-6)
    assert rc == 0
    err = out_rel(out.cpu().numpy(), ref_out)
    log(f"  gated outputs rel-L2 (worst of whole, per head) {err:.3e}")
    assert err <= OUT_TOL
    got = cache_d.cpu().numpy()
    singles = w.slot_ids[:40]
    multi = w.slot_ids[40:]
    assert state_rel(got[singles], cache_h[singles]) <= STATE_TOL
    assert np.array_equal(got[multi].view(np.uint32), w.cache[multi].view(np.uint32))
    # replay rows only for the multi-token rows; single rows leave the buffer alone
    rk = bits(rb["k"])
    assert np.array_equal(rk[40:], ref_rb["rk"][40:])
    assert np.all(rk[:40] == 0)
    log("mixed: commit")
    _commit(w, cache_d, K.KDA_REPLAY, acc, rb, None)
    torch.cuda.synchronize()
    assert oracle.commit(cache_h, w.slot_ids, w.cu_seqlens, acc, w.T_max, w.k[0], w.v[0], w.alpha[0],
                         w.beta[0]) == 0
    got = cache_d.cpu().numpy()
    serr = state_rel(got[w.slot_ids], cache_h[w.slot_ids])
    log(f"  committed states rel-Frobenius (worst of whole, per head) {serr:.3e}")
    assert serr <= STATE_TOL
    untouched = np.setdiff1d(np.arange(w.num_slots), w.slot_ids)
    assert np.array_equal(got[untouched].view(np.uint32), w.cache[untouched].view(np.uint32))


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 128), (128, 64), (64, 64)])
def test_ragged_rows_both_modes(dk, dv):
    seqlens = [3, 0, 1, 16, 5, 2, 7]
    w = synth.make(7, 3, dk, dv, seqlens=seqlens, num_slots=11, state_std=0.05, seed=32)
    slots = w.slot_ids.copy()
    slots[4] = -1                                   # a padding row with tokens
    acc = np.array([2, 0, 1, 16, 3, 1, 7], np.int32)
    res = {}
    for mode in (K.KDA_REPLAY, K.KDA_PER_POSITION):
        cache_d = f32(w.cache)
        log(f"ragged dk={dk} dv={dv} mode={mode}")
        out, rb, draft = _verify(w, cache_d, mode, slots=slots)
        ref_out, _, _, rc = _oracle_verify(w, mode, slots=slots)
        assert rc == 0
        torch.cuda.synchronize()
        o = out.cpu().numpy()
        live = np.concatenate([np.arange(w.cu_seqlens[b], w.cu_seqlens[b + 1]) for b in range(7) if b != 4])
        pad_rows = np.arange(w.cu_seqlens[4], w.cu_seqlens[5])
        assert np.all(bits(out)[pad_rows] == SENTINEL_BITS)
        assert out_rel(o[live], ref_out[live]) <= OUT_TOL
        _commit(w, cache_d, mode, acc, rb, draft, slots=slots)
        torch.cuda.synchronize()
        res[mode] = (bits(out), bits(cache_d))
    o0, o1 = res[0][0].view(np.float32), res[1][0].view(np.float32)
    live_rows = ~np.isnan(o1).any(axis=(1, 2))
    assert out_rel(o0[live_rows], o1[live_rows]) <= 1e-5
    assert np.array_equal(res[0][0][~live_rows], res[1][0][~live_rows])     # padding rows untouched
    assert np.array_equal(res[0][1], res[1][1])
    cache_h = w.cache.copy()
    assert oracle.commit(cache_h, slots, w.cu_seqlens, acc, w.T_max, w.k[0], w.v[0], w.alpha[0], w.beta[0]) == 0
    got = res[0][1].view(np.float32)
    live_slots = slots[[0, 2, 3, 5, 6]]
    assert state_rel(got[live_slots], cache_h[live_slots]) <= STATE_TOL
    assert np.array_equal(res[0][1][slots[1]], w.cache[slots[1]].view(np.uint32))   # accepted 0
    others = np.setdiff1d(np.arange(w.num_slots), live_slots)
    assert np.array_equal(res[0][1][others], w.cache[others].view(np.uint32))


@pytest.mark.parametrize("mode", [0, 1])
def test_verify_tile_widths_are_bit_identical(mode):
    w = synth.make(4, 5, 128, 128, seqlens=[4, 1, 3, 2], num_slots=6, state_std=0.05, seed=33)
    acc = np.array([3, 1, 3, 2], np.int32)
    first = None
    for tw in (4, 8, 16, 32, 64, 128):
        cache_d = f32(w.cache)
        log(f"verify tile widths mode={mode} W={tw}")
        out, rb, draft = _verify(w, cache_d, mode, tile_w=tw)
        _commit(w, cache_d, mode, acc, rb, draft, tile_w=tw)
        torch.cuda.synchronize()
        got = (bits(out), bits(cache_d), bits(draft) if draft is not None else bits(rb["v"]))
        if first is None:
            first = got
        else:
            for a, b in zip(got, first):
                assert np.array_equal(a, b), tw


def test_device_errors_skip_only_their_rows():
    w = synth.make(4, 2, 64, 64, seqlens=[2, 3, 1, 2], num_slots=6, state_std=0.05, seed=34)
    # a decreasing range in row 1 (and so row 2 starts before it ends)
    cu_bad = w.cu_seqlens.copy()
    cu_bad[2] = cu_bad[1] - 1
    cache_d = f32(w.cache)
    err = torch.zeros(1, dtype=torch.int32, device=dev())
    log("device error: bad row range")
    out, rb, _ = _verify(w, cache_d, K.KDA_REPLAY, cu=cu_bad, dev_err=err)
    torch.cuda.synchronize()
    ref_out, _, _, rc = _oracle_verify(w, K.KDA_REPLAY, cu=cu_bad)
    assert int(err.item()) == rc and rc & K.KDA_DEVERR_SEQLEN
    for b in range(w.B):
        lo, hi = cu_bad[b], cu_bad[b + 1]
        if lo >= 0 and hi >= lo and hi - lo <= w.T_max and hi <= w.n_tok:
            assert out_rel(out.cpu().numpy()[lo:hi], ref_out[lo:hi]) <= OUT_TOL
    # accepted length past the row: bit 4, that slot unchanged, the others committed
    cache_d = f32(w.cache)
    out, rb, _ = _verify(w, cache_d, K.KDA_REPLAY)
    err.zero_()
    acc = np.array([2, 4, 1, 1], np.int32)
    log("device error: accepted length past the row")
    _commit(w, cache_d, K.KDA_REPLAY, acc, rb, None, dev_err=err)
    torch.cuda.synchronize()
    cache_h = w.cache.copy()
    rc = oracle.commit(cache_h, w.slot_ids, w.cu_seqlens, acc, w.T_max, w.k[0], w.v[0], w.alpha[0], w.beta[0])
    assert int(err.item()) == rc == K.KDA_DEVERR_ACCEPTED
    got = cache_d.cpu().numpy()
    assert np.array_equal(got[w.slot_ids[1]].view(np.uint32), w.cache[w.slot_ids[1]].view(np.uint32))
    ok = w.slot_ids[[0, 2, 3]]
    assert state_rel(got[ok], cache_h[ok]) <= STATE_TOL
    # slot past the cache in verify and commit: bit 1
    slots = w.slot_ids.copy()
    slots[3] = w.num_slots
    err.zero_()
    cache_d = f32(w.cache)
    log("device error: slot past the cache")
    out, rb, _ = _verify(w, cache_d, K.KDA_REPLAY, slots=slots, dev_err=err)
    _commit(w, cache_d, K.KDA_REPLAY, np.array([1, 1, 1, 1], np.int32), rb, None, slots=slots, dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == K.KDA_DEVERR_SLOT


def test_empty_chunk_is_a_no_op():
    cache = torch.zeros(3, 2, 64, 64, device=dev())
    e16 = torch.empty(0, 2, 64, dtype=torch.bfloat16, device=dev())
    log("empty chunk")
    K.kda_verify_chunk(cache, i32([0, 1, 2]), i32([0, 0, 0, 0]), 4, e16, e16, e16,
                       torch.empty(0, 2, 64, device=dev()), torch.empty(0, 2, device=dev()),
                       torch.empty(0, 2, 64, device=dev()), mode=K.KDA_PER_POSITION,
                       draft=torch.zeros(3, 4, 2, 64, 64, device=dev()))
    torch.cuda.synchronize()
    assert float(cache.abs().sum()) == 0.0


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (128, 64), (64, 128)])
@pytest.mark.parametrize("seqlens", [[1, 2, 3, 5, 7, 8, 9, 11, 13, 15, 16, 4], [1, 2, 3, 5, 7, 8, 6, 4, 8]],
                         ids=["upto16", "upto8"])
def test_chunked_form_matches_oracle_and_recurrent_form(dk, dv, seqlens):
    """Replay-mode verify in chunk form (MFMA products with the committed state):
    ragged lengths with a padding row, decays spanning (0, 1). Up to 8 tokens the
    kernel stacks keys and queries in one product; longer rows take two."""
    w = synth.make(len(seqlens), 6, dk, dv, seqlens=seqlens, num_slots=16, state_std=0.05, seed=51)
    slots = w.slot_ids.copy()
    slots[3] = -1
    ref_out, ref_rb, _, rc = _oracle_verify(w, K.KDA_REPLAY, slots=slots)
    assert rc == 0
    live = np.concatenate([np.arange(w.cu_seqlens[b], w.cu_seqlens[b + 1]) for b in range(w.B) if b != 3])
    pad = np.arange(w.cu_seqlens[3], w.cu_seqlens[4])
    outs = {}
    for form in (K.KDA_VERIFY_CHUNKED, K.KDA_VERIFY_RECURRENT):
        cache_d = f32(w.cache)
        log(f"chunked vs recurrent dk={dk} dv={dv}: form {form}")
        out, rb, _ = _verify(w, cache_d, K.KDA_REPLAY, slots=slots, form=form)
        torch.cuda.synchronize()
        o = out.cpu().numpy()
        err = out_rel(o[live], ref_out[live])
        log(f"  outputs rel-L2 (worst of whole, per head) vs oracle {err:.3e}")
        assert err <= OUT_TOL
        assert np.all(bits(out)[pad] == SENTINEL_BITS)
        assert np.array_equal(bits(cache_d), w.cache.view(np.uint32))
        for key, rk in (("k", "rk"), ("v", "rv")):
            got = bits(rb[key])
            for b in range(w.B):
                if b != 3:
                    n = w.seqlens[b]
                    assert np.array_equal(got[b, :n], ref_rb[rk][b, :n])
        outs[form] = o
    assert out_rel(outs[K.KDA_VERIFY_CHUNKED][live], outs[K.KDA_VERIFY_RECURRENT][live]) <= 1e-5


@pytest.mark.parametrize("seqlens", [[16, 16, 9], [8, 8, 5]], ids=["upto16", "upto8"])
def test_chunked_form_with_extreme_decays(seqlens):
    """Decays near 0 and exactly 1 in the same chunk: running products stay finite."""
    w = synth.make(3, 4, 128, 128, seqlens=seqlens, num_slots=4, state_std=0.05, seed=52)
    rng = np.random.Generator(np.random.PCG64(53))
    alpha = w.alpha.copy()
    c = w.cu_seqlens
    alpha[0, c[0]:c[1]] = np.where(rng.random(alpha[0, c[0]:c[1]].shape) < 0.3, 1e-30, alpha[0, c[0]:c[1]])
    alpha[0, c[1]:c[2]] = 1.0
    alpha[0, c[2]:] = 1e-7
    w.alpha = alpha.astype(np.float32)
    ref_out, _, _, rc = _oracle_verify(w, K.KDA_REPLAY)
    assert rc == 0
    cache_d = f32(w.cache)
    log("chunked form, extreme decays")
    out, _, _ = _verify(w, cache_d, K.KDA_REPLAY, form=K.KDA_VERIFY_CHUNKED)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.all(np.isfinite(o))
    assert out_rel(o, ref_out) <= OUT_TOL


@pytest.mark.parametrize("B,T,expect", [(16, 8, K.KDA_VERIFY_CHUNKED), (4, 8, K.KDA_VERIFY_CHUNKED),
                                         (2, 8, K.KDA_VERIFY_RECURRENT), (8, 6, K.KDA_VERIFY_CHUNKED),
                                         (4, 6, K.KDA_VERIFY_RECURRENT), (16, 4, K.KDA_VERIFY_RECURRENT)])
def test_auto_form_choice(B, T, expect):
    """The automatic form is the chunk form from 7 tokens at 128 (row, head) groups and from 5
    tokens at 256 groups, the recurrent form otherwise (both are deterministic, so the outputs
    match bit for bit)."""
    w = synth.make(B, 32, 128, 128, seqlens=[T] * B, num_slots=B, state_std=0.05, seed=60 + B + T)
    outs = {}
    for form in (K.KDA_VERIFY_AUTO, expect):
        cache_d = f32(w.cache)
        log(f"auto form B={B} T={T}: form {form}")
        out, _, _ = _verify(w, cache_d, K.KDA_REPLAY, form=form)
        torch.cuda.synchronize()
        outs[form] = bits(out)
    assert np.array_equal(outs[K.KDA_VERIFY_AUTO], outs[expect])


def test_chunked_form_rejected_where_it_does_not_apply():
    w = synth.make(2, 2, 128, 128, seqlens=[2, 3], num_slots=3, state_std=0.05, seed=54)
    cache_d = f32(w.cache)
    for kw in (dict(mode=K.KDA_PER_POSITION), dict(mode=K.KDA_REPLAY, t1_inplace=True),
               dict(mode=K.KDA_REPLAY, gate=True), dict(mode=K.KDA_REPLAY, tile_w=32)):
        mode = kw.pop("mode")
        if kw.get("gate"):
            w.gate = synth.make(2, 2, 128, 128, seqlens=[2, 3], gate=True, seed=55).gate
        with pytest.raises(K.KdaError) as e:
            _verify(w, cache_d, mode, form=K.KDA_VERIFY_CHUNKED, **kw)
        assert e.value.status == K.KDA_ERR_UNSUPPORTED


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64)])
@pytest.mark.parametrize("tmax", [8, 16])
def test_chunked_form_state_load_orders_agree(dk, dv, tmax):
    """The chunk form issues the state behind the inputs' first writes within one round of
    resident workgroups and right behind the input requests for larger grids; both orders give
    the same bits. 16 live rows of 32 heads (512 groups: one round) against the same rows
    followed by 32 padding rows (1536 groups)."""
    rng = np.random.default_rng(61 + tmax)
    seqlens = list(rng.integers(1, tmax + 1, 16)) + [1] * 32
    seqlens[0] = tmax
    w = synth.make(48, 32, dk, dv, seqlens=seqlens, num_slots=64, state_std=0.05, seed=62)
    slots = w.slot_ids.copy()
    slots[16:] = -1
    x = step_inputs(w, 0)
    n16 = int(w.cu_seqlens[16])
    res = []
    for B in (16, 48):
        n_tok = n16 if B == 16 else w.n_tok
        out = sentinel((n_tok, w.H, dv))
        rb = replay_buffers(B, w.T_max, w.H, dk, dv)
        cache_d = f32(w.cache)
        log(f"chunk form, state load order: B={B} dk={dk} dv={dv} T_max={w.T_max}")
        K.kda_verify_chunk(cache_d, i32(slots[:B]), i32(w.cu_seqlens[:B + 1]), w.T_max,
                           *(x[n][:n_tok].contiguous() for n in ("q", "k", "v", "alpha", "beta")), out,
                           mode=K.KDA_REPLAY, replay=rb, verify_form=K.KDA_VERIFY_CHUNKED)
        torch.cuda.synchronize()
        res.append((bits(out), {k: bits(v)[:16] for k, v in rb.items()}))
        if B == 48:
            assert np.all(res[-1][0][n16:] == SENTINEL_BITS)
            assert np.array_equal(bits(cache_d), w.cache.view(np.uint32))
    assert np.array_equal(res[0][0], res[1][0][:n16])
    for k in res[0][1]:
        assert np.array_equal(res[0][1][k], res[1][1][k]), k
    ref_out, _, _, rc = _oracle_verify(w, K.KDA_REPLAY, slots=slots)
    assert rc == 0
    assert out_rel(res[0][0].view(np.float32), ref_out[:n16]) <= OUT_TOL


@pytest.mark.parametrize("mode", [0, 1], ids=["replay", "per_position"])
def test_commit_without_cu_seqlens_equals_steps(mode):
    """kda_replay_commit with cu_seqlens NULL takes T_b = T_max for every row and ignores
    n_tok (the commit reads only its buffers): with n_tok = 0 the committed slots equal
    accepted_len[b] single-token steps bit for bit."""
    w = synth.make_workload("spec_verify")
    acc = w.accepted
    x = step_inputs(w, 0)
    steps_d = f32(w.cache)
    for t in range(w.T_max):
        r = torch.from_numpy((w.cu_seqlens[:-1] + t).astype(np.int64)).to(dev())
        tok = {n: x[n][r].contiguous() for n in ("q", "k", "v", "alpha", "beta")}
        masked = np.where(acc > t, w.slot_ids, -1).astype(np.int32)
        log(f"single-token step {t}")
        K.kda_decode_step(steps_d, i32(masked), tok["q"], tok["k"], tok["v"], tok["alpha"], tok["beta"],
                          torch.empty(w.B, w.H, w.dv, device=dev()))
    cache_d = f32(w.cache)
    log(f"verify mode {mode}, then commit with cu_seqlens NULL and n_tok 0")
    _, rb, draft = _verify(w, cache_d, mode)
    err = torch.zeros(1, dtype=torch.int32, device=dev())
    K.kda_replay_commit(cache_d, i32(w.slot_ids), None, i32(acc), w.T_max, 0, mode=mode, replay=rb, draft=draft,
                        dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert np.array_equal(bits(cache_d), bits(steps_d))
    # an accepted length past T_max is still caught without cu_seqlens
    bad = acc.copy()
    bad[3] = w.T_max + 1
    cache_b = f32(w.cache)
    K.kda_replay_commit(cache_b, i32(w.slot_ids), None, i32(bad), w.T_max, 0, mode=mode, replay=rb, draft=draft,
                        dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == K.KDA_DEVERR_ACCEPTED
    got = bits(cache_b)
    assert np.array_equal(got[w.slot_ids[3]], w.cache[w.slot_ids[3]].view(np.uint32))
    others = np.delete(w.slot_ids, 3)
    assert np.array_equal(got[others], bits(steps_d)[others])


def test_mixed_batch_shuffled_order():
    """The mixed batch's stress order: 40 single-token rows and 24 four-token rows interleaved
    at random, single-token rows in place, output gate with a random weight, then the commit,
    against the oracle; untouched slots bit-exact."""
    rng = np.random.Generator(np.random.PCG64(41))
    lens = np.array([1] * 40 + [4] * 24)[rng.permutation(64)]
    w = synth.make(64, 32, 128, 128, seqlens=lens, num_slots=512, state_std=0.02, gate=True, seed=42,
                   name="mixed_shuffled")
    weight = rng.uniform(0.5, 2.0, w.dv).astype(np.float32)
    acc = w.accepted.copy()               # 0 for the single-token rows
    cache_d = f32(w.cache)
    log("mixed shuffled: verify with in-place singles, gate, weight")
    out, rb, _ = _verify(w, cache_d, K.KDA_REPLAY, t1_inplace=True, gate=True, weight=f32(weight))
    torch.cuda.synchronize()
    cache_h = w.cache.copy()
    ref_out, ref_rb, _, rc = oracle.verify(cache_h, w.slot_ids, w.cu_seqlens, w.T_max, w.q[0], w.k[0], w.v[0],
                                           w.alpha[0], w.beta[0], mode=oracle.REPLAY, t1_inplace=True,
                                           gate=w.gate[0], weight=weight, eps=1e-6)
    assert rc == 0
    assert out_rel(out.cpu().numpy(), ref_out, "gated outputs") <= OUT_TOL
    single = lens == 1
    got = cache_d.cpu().numpy()
    assert state_rel(got[w.slot_ids[single]], cache_h[w.slot_ids[single]], "in-place states") <= STATE_TOL
    multi = w.slot_ids[~single]
    assert np.array_equal(got[multi].view(np.uint32), w.cache[multi].view(np.uint32))
    rk = bits(rb["k"])
    assert np.array_equal(rk[~single], ref_rb["rk"][~single])
    assert np.all(rk[single] == 0)
    log("mixed shuffled: commit")
    _commit(w, cache_d, K.KDA_REPLAY, acc, rb, None)
    torch.cuda.synchronize()
    assert oracle.commit(cache_h, w.slot_ids, w.cu_seqlens, acc, w.T_max, w.k[0], w.v[0], w.alpha[0],
                         w.beta[0]) == 0
    got = cache_d.cpu().numpy()
    assert state_rel(got[w.slot_ids], cache_h[w.slot_ids], "committed states") <= STATE_TOL
    untouched = np.setdiff1d(np.arange(w.num_slots), w.slot_ids)
    assert np.array_equal(got[untouched].view(np.uint32), w.cache[untouched].view(np.uint32))
