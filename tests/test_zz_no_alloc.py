"""kda_prefill_chunked_noalloc: the chunk prefill on the library's static per-GPU scratch.

Two calls in a row, the second smaller than the first (the scratch keeps the
first call's contents), each against kda_prefill_chunked with a workspace of
its own (bit for bit: the same kernels on the same inputs) and against the CPU
oracle (outputs within 1e-4 relative L2, states within 1e-3 relative
Frobenius, per head as well). A call past the scratch limit is refused before
anything is enqueued.
"""

import numpy as np
import pytest
import torch

import gated_delta_rule_98_amd as K
import oracle
import synth
from gpu_util import bits, dev, f32, i32, log, out_rel, sentinel, state_rel, step_inputs

pytestmark = pytest.mark.gpu

OUT_TOL = 1e-4
STATE_TOL = 1e-3


def _run(fn, w, pos):
    x = step_inputs(w, 0)
    cache = f32(w.cache)
    out = sentinel((w.n_tok, w.H, w.dv))
    ckpt = sentinel((w.B, w.H, w.dv, w.dk))
    err = torch.zeros(1, dtype=torch.int32, device=dev())
    fn(cache, i32(w.slot_ids), i32(w.cu_seqlens), x["q"], x["k"], x["v"], x["alpha"], x["beta"], out,
       ckpt_pos=i32(pos), ckpt=ckpt, dev_err=err)
    torch.cuda.synchronize()
    return dict(out=bits(out), cache=bits(cache), ckpt=bits(ckpt), err=int(err.item()))


def test_noalloc_matches_workspace_entry_point():
    calls = [
        ("3 rows of 1000, 37 and 700 tokens, H=32, d=128",
         synth.make(3, 32, 128, 128, seqlens=[1000, 37, 700], num_slots=5, state_std=0.02, seed=71),
         np.array([640, 0, 333], np.int32)),
        ("2 rows of 90 and 5 tokens, H=8, dk=64, dv=128",
         synth.make(2, 8, 64, 128, seqlens=[90, 5], num_slots=3, state_std=0.02, seed=72),
         np.array([32, -1], np.int32)),
    ]
    for name, w, pos in calls:
        need = K.kda_prefill_chunked_workspace(w.B, w.n_tok, w.H, w.dk, w.dv)
        assert need <= K.KDA_NOALLOC_SCRATCH_BYTES
        log(f"no-alloc chunk prefill: {name} ({need / 2**20:.1f} MiB of scratch)")
        got = _run(K.kda_prefill_chunked_noalloc, w, pos)
        log(f"workspace chunk prefill: {name}")
        ref = _run(K.kda_prefill_chunked, w, pos)
        assert got["err"] == ref["err"] == 0
        for key in ("out", "cache", "ckpt"):
            assert np.array_equal(got[key], ref[key]), (name, key)
        cache_h = w.cache.copy()
        ref_out, ref_ckpt, rc = oracle.prefill(cache_h, w.slot_ids, w.cu_seqlens, w.q[0], w.k[0], w.v[0],
                                               w.alpha[0], w.beta[0], ckpt_pos=pos)
        assert rc == 0
        assert out_rel(got["out"].view(np.float32), ref_out, "outputs") <= OUT_TOL
        cache = got["cache"].view(np.float32)
        assert state_rel(cache[w.slot_ids], cache_h[w.slot_ids], "final states") <= STATE_TOL
        ck = got["ckpt"].view(np.float32)
        live = pos >= 0
        assert state_rel(ck[live], ref_ckpt[live], "checkpoints") <= STATE_TOL
        assert np.all(got["ckpt"][~live] == 0x7FC0DEAD)
        others = np.setdiff1d(np.arange(w.num_slots), w.slot_ids)
        assert np.array_equal(got["cache"][others], w.cache[others].view(np.uint32))


def test_noalloc_refuses_a_call_past_the_scratch():
    """A prompt whose workspace exceeds the static scratch: KDA_ERR_TOO_LARGE, nothing enqueued."""
    H, d = 32, 128
    n_tok = 4096
    assert K.kda_prefill_chunked_workspace(1, n_tok, H, d, d) > K.KDA_NOALLOC_SCRATCH_BYTES
    cache = torch.zeros(1, H, d, d, device=dev())
    q = torch.zeros(n_tok, H, d, dtype=torch.bfloat16, device=dev())
    alpha = torch.ones(n_tok, H, d, device=dev())
    beta = torch.zeros(n_tok, H, device=dev())
    out = sentinel((n_tok, H, d))
    log("no-alloc chunk prefill past the scratch limit")
    with pytest.raises(K.KdaError) as e:
        K.kda_prefill_chunked_noalloc(cache, i32([0]), i32([0, n_tok]), q, q, q, alpha, beta, out)
    assert e.value.status == K.KDA_ERR_TOO_LARGE
    torch.cuda.synchronize()
    assert np.all(bits(out) == 0x7FC0DEAD)
