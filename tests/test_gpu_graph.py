"""The library's launches captured in a HIP graph replay exactly like eager launches.

Nothing the library enqueues is a memset or a host synchronization, so a caller
may capture it. Each replay here is preceded by eager work (restoring the state
cache) and followed by a synchronization, and every replay is compared bit for
bit with the eager run.
"""

import numpy as np
import pytest
import torch

import gated_delta_rule_98_amd as K
import synth
from gpu_util import bits, dev, f32, i32, log, replay_buffers, step_inputs

pytestmark = pytest.mark.gpu


def test_decode_verify_commit_graph_replays_match_eager():
    steps = 6
    w = synth.make(4, 8, 128, 128, steps=steps, num_slots=6, state_std=0.05, seed=41)
    v = synth.make(3, 8, 128, 128, seqlens=[4, 2, 3], num_slots=5, state_std=0.05, seed=42)
    xs = [step_inputs(w, s) for s in range(steps)]
    xv = step_inputs(v, 0)
    cache_w, cache_v = f32(w.cache), f32(v.cache)
    init_w, init_v = cache_w.clone(), cache_v.clone()
    slots_w, slots_v = i32(w.slot_ids), i32(v.slot_ids)
    cu, acc = i32(v.cu_seqlens), i32(v.accepted)
    out_w = torch.empty(steps, w.B, w.H, w.dv, device=dev())
    out_v = torch.empty(v.n_tok, v.H, v.dv, device=dev())
    rb = replay_buffers(v.B, v.T_max, v.H, v.dk, v.dv)

    def work():
        for s in range(steps):
            x = xs[s]
            K.kda_decode_step(cache_w, slots_w, x["q"], x["k"], x["v"], x["alpha"], x["beta"], out_w[s])
        K.kda_verify_chunk(cache_v, slots_v, cu, v.T_max, xv["q"], xv["k"], xv["v"], xv["alpha"], xv["beta"],
                           out_v, mode=K.KDA_REPLAY, replay=rb)
        K.kda_replay_commit(cache_v, slots_v, cu, acc, v.T_max, v.n_tok, mode=K.KDA_REPLAY, replay=rb)

    log("graph: eager reference")
    work()
    torch.cuda.synchronize()
    ref = [bits(t) for t in (cache_w, out_w, cache_v, out_v, rb["k"])]

    cache_w.copy_(init_w)
    cache_v.copy_(init_v)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    log("graph: capture")
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            work()
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    for r in range(3):
        cache_w.copy_(init_w)          # eager work between replays
        cache_v.copy_(init_v)
        out_w.zero_()
        out_v.zero_()
        torch.cuda.synchronize()
        log(f"graph: replay {r}")
        graph.replay()
        torch.cuda.synchronize()
        got = [bits(t) for t in (cache_w, out_w, cache_v, out_v, rb["k"])]
        for a, b in zip(got, ref):
            assert np.array_equal(a, b), f"replay {r}"
