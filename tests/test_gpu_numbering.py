"""GPU parity across the workgroup numberings.

Kernels whose rows carry unequal work (verify, both commits, both prefill
forms) deal the (row, head) groups out to the 8 XCDs in turn when there is a
multiple of 8 groups, and otherwise take contiguous ranges. Verify numbers
the groups head-major (split by the batch size); the commits and prefill
deal heads x, x + 8, ... of every row to XCD x when the head count is a
multiple of 8 (split by the batch size) and take groups in row order
otherwise (split by the head count). Each split is a shift for a power of two
and a division otherwise. These shapes reach every combination, with ragged
rows, an empty row and a padding row, and each result is checked against the
oracle: outputs within 1e-4 relative L2, states within 1e-3 relative
Frobenius, untouched slots bit-exact.
"""

import numpy as np
import pytest
import torch

import gated_delta_rule_98_amd as K
import oracle
import synth
from gpu_util import SENTINEL_BITS, bits, dev, f32, i32, log, out_rel, state_rel, replay_buffers, sentinel, step_inputs

pytestmark = pytest.mark.gpu

OUT_TOL = 1e-4
STATE_TOL = 1e-3

# (B, H): 24 groups in row order with H = 3 and H = 6 (division) and H = 4
# (shift); heads dealt with B = 2 (shift) and B = 3 (division); 15 and 21 in
# contiguous ranges. Verify's head-major split divides by B = 6 and 3 and
# shifts by the others.
SHAPES = [(8, 3), (4, 6), (6, 4), (2, 8), (3, 16), (5, 3), (7, 3)]


def _workload(B, H, seed, max_len=12):
    rng = np.random.default_rng(seed)
    seqlens = [int(x) for x in rng.integers(1, max_len + 1, size=B)]
    seqlens[1 % B] = 0                               # an empty row
    w = synth.make(B, H, 64, 64, seqlens=seqlens, num_slots=B + 3, state_std=0.05, seed=seed)
    slots = w.slot_ids.copy()
    slots[B - 1] = -1                                # a padding row with tokens
    return w, slots


def _live(w, slots):
    rows = [b for b in range(w.B) if slots[b] >= 0]
    return np.concatenate([np.arange(w.cu_seqlens[b], w.cu_seqlens[b + 1]) for b in rows] + [np.zeros(0, int)])


def _check_state(w, slots, cache_d, cache_h):
    got = cache_d.cpu().numpy()
    live_slots = slots[slots >= 0]
    serr = state_rel(got[live_slots], cache_h[live_slots])
    others = np.setdiff1d(np.arange(w.num_slots), live_slots)
    assert np.array_equal(got[others].view(np.uint32), w.cache[others].view(np.uint32))
    return serr


@pytest.mark.parametrize("B,H", SHAPES)
def test_verify_and_commit_across_numberings(B, H):
    w, slots = _workload(B, H, seed=100 + 8 * B + H)
    T = w.T_max
    acc = np.array([min(n, 1 + b % 3) for b, n in enumerate(w.seqlens)], np.int32)
    x = step_inputs(w, 0)
    live = _live(w, slots)
    for mode in (K.KDA_REPLAY, K.KDA_PER_POSITION):
        log(f"numbering B={B} H={H} verify mode {mode}")
        cache_d = f32(w.cache)
        out = sentinel((w.n_tok, H, w.dv))
        rb = replay_buffers(B, T, H, w.dk, w.dv) if mode == K.KDA_REPLAY else None
        draft = torch.zeros(B, T, H, w.dv, w.dk, device=dev()) if mode == K.KDA_PER_POSITION else None
        K.kda_verify_chunk(cache_d, i32(slots), i32(w.cu_seqlens), T, x["q"], x["k"], x["v"], x["alpha"],
                           x["beta"], out, mode=mode, replay=rb, draft=draft)
        K.kda_replay_commit(cache_d, i32(slots), i32(w.cu_seqlens), i32(acc), T, w.n_tok, mode=mode, replay=rb,
                            draft=draft)
        torch.cuda.synchronize()
        ref_out, _, _, rc = oracle.verify(w.cache.copy(), slots, w.cu_seqlens, T, w.q[0], w.k[0], w.v[0],
                                          w.alpha[0], w.beta[0], mode=mode)
        assert rc == 0
        err = out_rel(out.cpu().numpy()[live], ref_out[live])
        pad = np.arange(w.cu_seqlens[B - 1], w.cu_seqlens[B])
        assert np.all(bits(out)[pad] == SENTINEL_BITS)
        cache_h = w.cache.copy()
        assert oracle.commit(cache_h, slots, w.cu_seqlens, acc, T, w.k[0], w.v[0], w.alpha[0], w.beta[0]) == 0
        serr = _check_state(w, slots, cache_d, cache_h)
        log(f"  outputs rel-L2 (worst of whole, per head) {err:.3e}, committed states rel-Frobenius (worst of whole, per head) {serr:.3e}")
        assert err <= OUT_TOL and serr <= STATE_TOL


@pytest.mark.parametrize("B,H", SHAPES)
@pytest.mark.parametrize("chunked", [False, True])
def test_prefill_across_numberings(B, H, chunked):
    w, slots = _workload(B, H, seed=200 + 8 * B + H, max_len=70)
    x = step_inputs(w, 0)
    pos = np.array([min(n, 5 + 7 * b) if b % 2 == 0 else -1 for b, n in enumerate(w.seqlens)], np.int32)
    log(f"numbering B={B} H={H} prefill chunked={chunked}")
    cache_d = f32(w.cache)
    out = sentinel((w.n_tok, H, w.dv))
    ckpt = sentinel((B, H, w.dv, w.dk))
    fn = K.kda_prefill_chunked if chunked else K.kda_prefill
    fn(cache_d, i32(slots), i32(w.cu_seqlens), x["q"], x["k"], x["v"], x["alpha"], x["beta"], out,
       ckpt_pos=i32(pos), ckpt=ckpt)
    torch.cuda.synchronize()
    cache_h = w.cache.copy()
    ref_out, ref_ckpt, rc = oracle.prefill(cache_h, slots, w.cu_seqlens, w.q[0], w.k[0], w.v[0], w.alpha[0],
                                           w.beta[0], ckpt_pos=pos)
    assert rc == 0
    live = _live(w, slots)
    err = out_rel(out.cpu().numpy()[live], ref_out[live])
    serr = _check_state(w, slots, cache_d, cache_h)
    log(f"  outputs rel-L2 (worst of whole, per head) {err:.3e}, states rel-Frobenius (worst of whole, per head) {serr:.3e}")
    assert err <= OUT_TOL and serr <= STATE_TOL
    ck = ckpt.cpu().numpy()
    for b in range(B):
        if slots[b] >= 0 and pos[b] >= 0:
            assert state_rel(ck[b], ref_ckpt[b]) <= STATE_TOL, b
        else:
            assert np.all(bits(ckpt)[b] == SENTINEL_BITS), b
