#!/usr/bin/env python3
"""Benchmark of the KDA fp32 recurrent-state decode step on one MI355X.

Headline: single-token decode at B=64, H=32, dk=dv=128 (the batch-64 end of the
pages' batch 1-64 decode, "Hyper Optimizing Kimi K3 in vLLM"), over a 256-slot
fp32 state cache (512 MiB). Each step runs on the next of four disjoint
64-slot tables, so a slot is revisited only after 384 MiB of other state has
streamed through the 256 MB Infinity Cache: the state comes from HBM.

Prints one JSON line on stdout:
  value         decode steps per second (K steps bracketed by synchronizations)
  roofline      HBM bytes the step must move per launch / the kernel's average
                duration (HIP events on its stream, median of 3 timed regions) vs
                8 TB/s; beside it the rate of a plain in-place read-modify-write of
                the same state bytes (the ceiling probe, libkda_ceiling.so)
  cpu_baseline  the CPU oracle on this host's cores (all of them, and one), on a
                bounded sample, median of 3
  breakdown     the batch sweep, the B=1 1024-step latency path (plain launches and
                one captured HIP graph), the speculative verify + commit in both
                buffer modes and the mixed gated batch, each with its own
                algorithmic bytes and GB/s
Progress goes to stderr.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
METRIC = "KDA decode steps/s + achieved HBM GB/s (fp32 state), B=1..64, H=32, dk=dv=128"
COUNTERS_FILE = os.path.join(ROOT, "profiles", "kda_decode_b64_counters.txt")
# the sources the decode kernel is compiled from: the counters hold only while these are unchanged
KERNEL_SOURCES = [os.path.join(ROOT, "gated_delta_rule_98_amd", "csrc", f) for f in ("kda_engine.h", "kda_decode.hip")]


def kernel_source_sha256():
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        h.update(os.path.basename(path).encode() + b"\0")
        h.update(open(path, "rb").read())
    return h.hexdigest()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------- bytes

def decode_bytes(B, H, dk, dv):
    """HBM bytes one single-token step must move: state read + write, inputs, output, slot ids."""
    per_head = 2 * dk * dv * 4 + (2 * dk + dv) * 2 + dk * 4 + 4 + dv * 4
    return B * H * per_head + B * 4


def verify_bytes(n_tok, B, H, dk, dv, mode, T_max):
    """Verify: state read once per row, per-token inputs and outputs, plus the replay copy
    (REPLAY) or the per-token state writes (PER_POSITION)."""
    state = B * H * dk * dv * 4
    tok_in = n_tok * H * ((2 * dk + dv) * 2 + dk * 4 + 4)
    tok_out = n_tok * H * dv * 4
    meta = B * 4 + (B + 1) * 4
    if mode == 0:
        extra = n_tok * H * (dk * 2 + dv * 2 + dk * 4 + 4)
    else:
        extra = n_tok * H * dk * dv * 4
    return state + tok_in + tok_out + meta + extra


def mixed_verify_bytes(seqlens, H, dk, dv):
    """Mixed batch with the output gate: single-token rows read and write their state in place;
    longer rows read it once and copy their inputs to the replay buffer; every token reads its
    inputs and gate and writes its output."""
    seqlens = np.asarray(seqlens)
    n_tok = int(seqlens.sum())
    singles = int(np.sum(seqlens == 1))
    multi = int(np.sum(seqlens > 1))
    multi_tok = int(seqlens[seqlens > 1].sum())
    state = (2 * singles + multi) * H * dk * dv * 4
    per_tok = H * ((2 * dk + dv) * 2 + dk * 4 + 4 + dv * 2 + dv * 4)
    replay = multi_tok * H * (dk * 2 + dv * 2 + dk * 4 + 4)
    return state + n_tok * per_tok + replay + len(seqlens) * 8 + 4 + dv * 4


def commit_bytes(accepted, H, dk, dv, mode):
    live = int(np.count_nonzero(accepted))
    state = live * H * dk * dv * 4
    if mode == 0:
        toks = int(np.sum(accepted)) * H * (dk * 2 + dv * 2 + dk * 4 + 4)
        return 2 * state + toks + len(accepted) * 8
    return 2 * state + len(accepted) * 8


# ----------------------------------------------------------------------------- GPU helpers

class Dev:
    def __init__(self):
        import torch

        self.torch = torch
        self.dev = torch.device("cuda", 0)

    def bf(self, a):
        t = self.torch
        return t.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(self.dev).view(t.bfloat16)

    def f(self, a):
        return self.torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(self.dev)

    def i(self, a):
        return self.torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(self.dev)

    def sync(self):
        self.torch.cuda.synchronize()

    def event(self):
        return self.torch.cuda.Event(enable_timing=True)


def timed_region(D, launch, n):
    """Run launch(i) for i < n between two events; returns total ms."""
    D.sync()
    a, b = D.event(), D.event()
    a.record()
    for i in range(n):
        launch(i)
    b.record()
    D.sync()
    return a.elapsed_time(b)


def per_launch_ms(D, launch, n):
    """Average duration of one launch: an event pair around each launch on the launch stream."""
    evs = [(D.event(), D.event()) for _ in range(n)]
    D.sync()
    for i in range(n):
        evs[i][0].record()
        launch(i)
        evs[i][1].record()
    D.sync()
    return float(np.mean([s.elapsed_time(e) for s, e in evs]))


def graph_ms(D, launch, n, replays=3):
    """GPU time per launch: n launches captured once in a HIP graph, replayed; the median of
    3 timed sets of `replays` replays."""
    torch = D.torch
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            for i in range(n):
                launch(i)
    torch.cuda.current_stream().wait_stream(stream)
    graph.replay()
    D.sync()
    times = []
    for _ in range(3):
        a, b = D.event(), D.event()
        a.record()
        for _ in range(replays):
            graph.replay()
        b.record()
        D.sync()
        times.append(a.elapsed_time(b) / (n * replays))
    return float(np.median(times))


# ----------------------------------------------------------------------------- workloads

def decode_setup(D, K, synth, B, seed=0):
    w = synth.make(B, 32, 128, 128, num_slots=256, state_std=0.02, seed=seed, name=f"decode_b{B}")
    cache = D.f(w.cache)
    tables = [D.i(t) for t in w.slot_tables]
    x = dict(q=D.bf(w.q[0]), k=D.bf(w.k[0]), v=D.bf(w.v[0]), alpha=D.f(w.alpha[0]), beta=D.f(w.beta[0]))
    out = D.torch.empty(B, 32, 128, device=D.dev)

    def launch(i, hot=False):
        K.kda_decode_step(cache, tables[0 if hot else i % len(tables)], x["q"], x["k"], x["v"], x["alpha"],
                          x["beta"], out)

    return w, launch, (cache, tables, x, out)


def headline(D, K, synth, steps, warmup):
    B = 64
    w, launch, keep = decode_setup(D, K, synth, B)
    nbytes = decode_bytes(B, 32, 128, 128)
    log(f"headline: B={B} H=32 d=128, {len(w.slot_tables)} rotating slot tables, {steps} steps after {warmup} warmup")
    for i in range(warmup):
        launch(i)
    D.sync()
    # three timed regions of K launches each; the median region gives the figure
    regions = [timed_region(D, launch, steps) / steps for _ in range(3)]
    ms_step = float(np.median(regions))
    # the K launches of a region run back to back on one stream with no other work, so
    # the region's average is the kernel's average duration (rocprofv3 agrees to ~1%)
    kernel_ms = ms_step
    pairs_ms = per_launch_ms(D, launch, min(steps, 200))
    hot_ms = timed_region(D, lambda i: launch(i, hot=True), min(steps, 200)) / min(steps, 200)
    log(f"headline: regions {', '.join(f'{r * 1e3:.2f}' for r in regions)} us/step; median "
        f"{ms_step * 1e3:.2f} us/step ({nbytes / kernel_ms / 1e6:.1f} GB/s); "
        f"event pair per launch {pairs_ms * 1e3:.2f} us; same table every step (cache-resident) {hot_ms * 1e3:.2f} us")
    return dict(w=w, ms_step=ms_step, kernel_ms=kernel_ms, pairs_ms=pairs_ms, hot_ms=hot_ms, bytes=nbytes,
                regions_ms=regions, tile=K.kda_query_variant(B, 32, 128, 128))


def batch_sweep(D, K, synth, reps):
    rows = []
    for B in (1, 2, 4, 8, 16, 32, 64):
        w, launch, keep = decode_setup(D, K, synth, B, seed=B)
        for i in range(10):
            launch(i)
        ms = graph_ms(D, launch, reps)
        eager = timed_region(D, launch, reps) / reps
        nb = decode_bytes(B, 32, 128, 128)
        tw, th = K.kda_query_variant(B, 32, 128, 128)
        rows.append(dict(B=B, tile_w=tw, threads=th, us_per_step=round(ms * 1e3, 3),
                         us_per_step_eager_python=round(eager * 1e3, 3), steps_per_s=round(1e3 / ms, 1),
                         tokens_per_s=round(B * 1e3 / ms, 1), algorithmic_bytes=nb,
                         gbs=round(nb / ms / 1e6, 1), frac_of_peak=round(nb / ms / 1e6 / PEAK_HBM_GBS, 4)))
        log(f"sweep B={B}: {ms * 1e3:.2f} us/step in a HIP graph ({nb / ms / 1e6:.0f} GB/s), "
            f"{eager * 1e3:.2f} us/step launched eagerly from Python")
        del keep
    return rows


def b1_latency(D, K, synth):
    """B=1, H=32, d=128: 1024 sequential single-token steps, each on the state the previous
    step wrote. Launched eagerly from Python, and as one captured HIP graph."""
    torch = D.torch
    w = synth.make_workload("b1_latency")
    cache = D.f(w.cache)
    slots = D.i(w.slot_ids)
    q, k, v = D.bf(w.q), D.bf(w.k), D.bf(w.v)
    al, be = D.f(w.alpha), D.f(w.beta)
    out = torch.empty(w.steps, 1, 32, 128, device=D.dev)

    def step(s):
        K.kda_decode_step(cache, slots, q[s], k[s], v[s], al[s], be[s], out[s])

    for s in range(16):
        step(s)
    D.sync()
    plain_ms = timed_region(D, step, w.steps) / w.steps
    g_ms = graph_ms(D, step, w.steps, replays=2)
    log(f"b1_latency: {plain_ms * 1e3:.2f} us/step launched from Python, {g_ms * 1e3:.2f} us/step in a HIP graph")
    return dict(B=1, steps=w.steps, us_per_step_eager_python=round(plain_ms * 1e3, 3),
                us_per_step_graph=round(g_ms * 1e3, 3), tile_w=K.kda_query_variant(1, 32, 128, 128)[0])


def raw_inputs_decode(D, K, synth, reps):
    """Single-token step from raw projections (q/k normalization and the alpha / beta
    activations inside the kernel) against the prepared-input step, at B=1 and B=64,
    with a bf16 output too; and, for scale, the same preparation done by separate
    torch kernels ahead of the prepared-input step."""
    torch = D.torch
    rows = []
    for B in (1, 64):
        w = synth.make(B, 32, 128, 128, num_slots=256, state_std=0.02, seed=40 + B, name=f"raw_b{B}")
        cache = D.f(w.cache)
        tables = [D.i(t) for t in w.slot_tables]
        prep = dict(q=D.bf(w.q[0]), k=D.bf(w.k[0]), v=D.bf(w.v[0]), alpha=D.f(w.alpha[0]), beta=D.f(w.beta[0]))
        raw = dict(q=D.bf(w.q_raw[0]), k=D.bf(w.k_raw[0]), v=prep["v"], alpha=D.f(w.a_raw[0]),
                   beta=D.f(w.b_raw[0]))
        out = torch.empty(B, 32, 128, device=D.dev)
        out16 = torch.empty(B, 32, 128, device=D.dev, dtype=torch.bfloat16)
        tmp = {}

        def run(x, o, flag):
            return lambda i: K.kda_decode_step(cache, tables[i % len(tables)], x["q"], x["k"], x["v"],
                                               x["alpha"], x["beta"], o, raw_inputs=flag)

        def unfused(i):
            tmp["k"] = torch.nn.functional.normalize(raw["k"].float(), dim=-1, eps=1e-6).to(torch.bfloat16)
            tmp["q"] = (torch.nn.functional.normalize(raw["q"].float(), dim=-1, eps=1e-6)
                        * (128 ** -0.5)).to(torch.bfloat16)
            tmp["alpha"] = torch.exp(-torch.nn.functional.softplus(raw["alpha"]))
            tmp["beta"] = torch.sigmoid(raw["beta"])
            K.kda_decode_step(cache, tables[i % len(tables)], tmp["q"], tmp["k"], raw["v"], tmp["alpha"],
                              tmp["beta"], out)

        graph, eager = {}, {}
        for name, fn in (("prepared_inputs", run(prep, out, False)), ("raw_inputs_fused", run(raw, out, True)),
                         ("raw_inputs_fused_bf16_out", run(raw, out16, True)),
                         ("torch_preparation_then_step", unfused)):
            for i in range(10):
                fn(i)
            eager[name] = round(timed_region(D, fn, reps) / reps * 1e3, 3)
            if name != "torch_preparation_then_step":   # torch's own kernels stay out of graphs
                graph[name] = round(graph_ms(D, fn, reps) * 1e3, 3)
        rows.append(dict(B=B, us_per_step_graph=graph, us_per_step_eager_python=eager))
        log(f"raw inputs B={B}: graph " + ", ".join(f"{k} {v:.2f}" for k, v in graph.items())
            + " us; eager " + ", ".join(f"{k} {v:.2f}" for k, v in eager.items()) + " us")
    return rows


def _replay_bufs(torch, dev, B, T, H, dk, dv):
    return dict(k=torch.zeros(B, T, H, dk, dtype=torch.bfloat16, device=dev),
                v=torch.zeros(B, T, H, dv, dtype=torch.bfloat16, device=dev),
                alpha=torch.zeros(B, T, H, dk, device=dev), beta=torch.zeros(B, T, H, device=dev))


def spec_verify(D, K, synth, reps, B=16):
    """B rows of 8 draft tokens (B=16: the speculative-verify workload). Each launch takes the
    next of the disjoint slot tables (16 at B=16, 4 at B=64) and of 4 replay / 2 per-position
    buffers, so state and buffers come from HBM."""
    torch = D.torch
    if B == 16:
        w = synth.make_workload("spec_verify")
    else:
        w = synth.make(B, 32, 128, 128, seqlens=[8] * B, num_slots=256, state_std=0.02, seed=B,
                       name=f"spec_verify_b{B}")
    H, d, T = 32, 128, w.T_max
    cache = D.f(w.cache)
    tables = [D.i(t) for t in w.slot_tables]
    cu, acc = D.i(w.cu_seqlens), D.i(w.accepted)
    x = dict(q=D.bf(w.q[0]), k=D.bf(w.k[0]), v=D.bf(w.v[0]), alpha=D.f(w.alpha[0]), beta=D.f(w.beta[0]))
    out = torch.empty(w.n_tok, H, d, device=D.dev)
    rbs = [_replay_bufs(torch, D.dev, w.B, T, H, d, d) for _ in range(4)]
    drafts = [torch.zeros(w.B, T, H, d, d, device=D.dev) for _ in range(2)]
    res = {}
    for mode, name in ((0, "replay"), (1, "per_position")):
        def verify(i):
            K.kda_verify_chunk(cache, tables[i % len(tables)], cu, T, x["q"], x["k"], x["v"], x["alpha"], x["beta"],
                               out, mode=mode, replay=rbs[i % 4] if mode == 0 else None,
                               draft=drafts[i % 2] if mode == 1 else None)

        def commit(i):
            K.kda_replay_commit(cache, tables[i % len(tables)], cu, acc, T, w.n_tok, mode=mode,
                                replay=rbs[i % 4] if mode == 0 else None, draft=drafts[i % 2] if mode == 1 else None)

        def pair(i):
            verify(i)
            commit(i)

        for i in range(8):
            pair(i)
        # kernel times from HIP-graph replays: launched one by one from Python, a call
        # costs more host time (~15 us) than these kernels take on the GPU
        v_ms = graph_ms(D, verify, reps)
        c_ms = graph_ms(D, commit, reps)
        p_ms = graph_ms(D, pair, reps)
        vb = verify_bytes(w.n_tok, w.B, H, d, d, mode, T)
        cb = commit_bytes(w.accepted, H, d, d, mode)
        res[name] = dict(verify_us=round(v_ms * 1e3, 3), verify_bytes=vb, verify_gbs=round(vb / v_ms / 1e6, 1),
                         commit_us=round(c_ms * 1e3, 3), commit_bytes=cb, commit_gbs=round(cb / c_ms / 1e6, 1),
                         verify_plus_commit_us=round(p_ms * 1e3, 3), total_bytes=vb + cb,
                         verify_form="automatic (chunk form at this shape)" if mode == 0 else "recurrent",
                         recurrent_tile_w=K.kda_query_variant(w.B, H, d, d, T_max=T, op=K.KDA_OP_VERIFY)[0])
        log(f"spec_verify B={w.B} {name}: verify {v_ms * 1e3:.2f} us ({vb / v_ms / 1e6:.0f} GB/s), "
            f"commit {c_ms * 1e3:.2f} us ({cb / c_ms / 1e6:.0f} GB/s), verify+commit {p_ms * 1e3:.2f} us")

    # replay-mode verify in each form explicitly: the automatic choice above is the chunk
    # form (MFMA products with the committed state) at this shape
    vb = verify_bytes(w.n_tok, w.B, H, d, d, 0, T)
    for form, name in ((K.KDA_VERIFY_CHUNKED, "chunk"), (K.KDA_VERIFY_RECURRENT, "recurrent")):
        def verify_form(i, form=form):
            K.kda_verify_chunk(cache, tables[i % len(tables)], cu, T, x["q"], x["k"], x["v"], x["alpha"],
                               x["beta"], out, mode=0, replay=rbs[i % 4], verify_form=form)

        for i in range(8):
            verify_form(i)
        f_ms = graph_ms(D, verify_form, reps)
        res[f"replay_{name}_form"] = dict(verify_us=round(f_ms * 1e3, 3), verify_gbs=round(vb / f_ms / 1e6, 1))
        log(f"spec_verify B={w.B} replay, {name} form: verify {f_ms * 1e3:.2f} us")
    return res


def spec_verify_small(D, K, synth, reps, batches=(1, 4)):
    """Speculative verify at small batch: B rows of 8 draft tokens (H=32, d=128), replay mode,
    verify and commit (5 accepted per row) timed in HIP graphs, 16 disjoint slot tables."""
    torch = D.torch
    res = {}
    for B in batches:
        T = 8
        w = synth.make(B, 32, 128, 128, seqlens=[T] * B, num_slots=16 * B, state_std=0.02, seed=B,
                       name=f"spec_b{B}")
        cache = D.f(w.cache)
        tables = [D.i(t) for t in w.slot_tables]
        cu = D.i(w.cu_seqlens)
        acc_h = np.full(B, 5, np.int32)
        acc = D.i(acc_h)
        x = dict(q=D.bf(w.q[0]), k=D.bf(w.k[0]), v=D.bf(w.v[0]), alpha=D.f(w.alpha[0]), beta=D.f(w.beta[0]))
        out = torch.empty(w.n_tok, 32, 128, device=D.dev)
        rbs = [_replay_bufs(torch, D.dev, B, T, 32, 128, 128) for _ in range(4)]

        def verify(i):
            K.kda_verify_chunk(cache, tables[i % len(tables)], cu, T, x["q"], x["k"], x["v"], x["alpha"], x["beta"],
                               out, mode=0, replay=rbs[i % 4])

        def commit(i):
            K.kda_replay_commit(cache, tables[i % len(tables)], cu, acc, T, w.n_tok, mode=0, replay=rbs[i % 4])

        for i in range(8):
            verify(i)
            commit(i)
        v_ms = graph_ms(D, verify, reps)
        c_ms = graph_ms(D, commit, reps)
        vb = verify_bytes(w.n_tok, B, 32, 128, 128, 0, T)
        cb = commit_bytes(acc_h, 32, 128, 128, 0)
        res[f"b{B}"] = dict(verify_us=round(v_ms * 1e3, 3), commit_us=round(c_ms * 1e3, 3),
                            verify_gbs=round(vb / v_ms / 1e6, 1), commit_gbs=round(cb / c_ms / 1e6, 1),
                            tile_w=K.kda_query_variant(B, 32, 128, 128, T_max=T, op=K.KDA_OP_VERIFY)[0])
        log(f"spec_verify B={B} T=8 (HIP graph): verify {v_ms * 1e3:.2f} us, commit {c_ms * 1e3:.2f} us")
    return res


def mixed(D, K, synth, reps):
    """40 single-token rows (in place) + 24 rows of 4 verified tokens, output gate, then the
    commit of the 24; 8 disjoint slot tables over the 512-slot cache, 2 replay buffers."""
    torch = D.torch
    w = synth.make_workload("mixed")
    H, d, T = 32, 128, w.T_max
    cache = D.f(w.cache)
    tables = [D.i(t) for t in w.slot_tables]
    cu, acc = D.i(w.cu_seqlens), D.i(w.accepted)
    x = dict(q=D.bf(w.q[0]), k=D.bf(w.k[0]), v=D.bf(w.v[0]), alpha=D.f(w.alpha[0]), beta=D.f(w.beta[0]),
             gate=D.bf(w.gate[0]))
    out = torch.empty(w.n_tok, H, d, device=D.dev)
    rbs = [_replay_bufs(torch, D.dev, w.B, T, H, d, d) for _ in range(2)]

    def verify(i):
        K.kda_verify_chunk(cache, tables[i % len(tables)], cu, T, x["q"], x["k"], x["v"], x["alpha"], x["beta"], out,
                           mode=0, t1_inplace=True, replay=rbs[i % 2], gate=x["gate"], eps=1e-6)

    def commit(i):
        K.kda_replay_commit(cache, tables[i % len(tables)], cu, acc, T, w.n_tok, mode=0, replay=rbs[i % 2])

    def pair(i):
        verify(i)
        commit(i)

    for i in range(8):
        pair(i)
    v_ms = graph_ms(D, verify, reps)
    c_ms = graph_ms(D, commit, reps)
    p_ms = graph_ms(D, pair, reps)
    vb = mixed_verify_bytes(w.seqlens, H, d, d)
    cb = commit_bytes(w.accepted, H, d, d, 0)
    log(f"mixed: verify {v_ms * 1e3:.2f} us ({vb / v_ms / 1e6:.0f} GB/s), commit {c_ms * 1e3:.2f} us "
        f"({cb / c_ms / 1e6:.0f} GB/s), verify+commit {p_ms * 1e3:.2f} us")
    return dict(verify_us=round(v_ms * 1e3, 3), verify_bytes=vb, verify_gbs=round(vb / v_ms / 1e6, 1),
                commit_us=round(c_ms * 1e3, 3), commit_bytes=cb, commit_gbs=round(cb / c_ms / 1e6, 1),
                verify_plus_commit_us=round(p_ms * 1e3, 3))


def prefill_8k(D, K, synth, reps, tile_w=0, chunked=False):
    """One 8000-token prompt, H=32, d=128, from a zero state, exporting the state after token
    7680 in the same pass (the in-loop checkpoint of the pages' long-prompt prefill); the
    recurrent kernel, or the chunk form (its two kernels, with a preallocated workspace)."""
    torch = D.torch
    w = synth.make_workload("prefill_8k")
    H, d = 32, 128
    cache = D.f(w.cache)
    slots, cu = D.i(w.slot_ids), D.i(w.cu_seqlens)
    x = dict(q=D.bf(w.q[0]), k=D.bf(w.k[0]), v=D.bf(w.v[0]), alpha=D.f(w.alpha[0]), beta=D.f(w.beta[0]))
    out = torch.empty(w.n_tok, H, d, device=D.dev)
    pos = D.i([7680])
    ckpt = torch.empty(1, H, d, d, device=D.dev)

    ws_bytes = K.kda_prefill_chunked_workspace(1, w.n_tok, H, d, d) if chunked else 0
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=D.dev) if chunked else None

    def run(i):
        if chunked:
            K.kda_prefill_chunked(cache, slots, cu, x["q"], x["k"], x["v"], x["alpha"], x["beta"], out,
                                  ckpt_pos=pos, ckpt=ckpt, workspace=ws)
        else:
            K.kda_prefill(cache, slots, cu, x["q"], x["k"], x["v"], x["alpha"], x["beta"], out, ckpt_pos=pos,
                          ckpt=ckpt, tile_w=tile_w)

    run(0)
    ms = timed_region(D, run, reps) / reps
    n = w.n_tok
    nbytes = n * H * ((2 * d + d) * 2 + d * 4 + 4 + d * 4) + 3 * H * d * d * 4 + 16
    flops = n * H * 7 * d * d
    form = "chunked" if chunked else "recurrent"
    log(f"prefill 8000 tokens ({form}): {ms * 1e3:.1f} us ({n / ms * 1e3:.0f} tok/s, "
        f"{flops / ms / 1e9:.2f} TFLOP/s of recurrence work)")
    res = dict(form=form, tokens=n, heads=H, us=round(ms * 1e3, 2), tokens_per_s=round(n / ms * 1e3, 1),
               algorithmic_bytes=nbytes, gbs=round(nbytes / ms / 1e6, 1), flops=flops,
               tflops=round(flops / ms / 1e9, 3), checkpoint_at=7680)
    if chunked:
        res["workspace_bytes"] = ws_bytes
        # fp32 state; its products with W, [Gamma q] and Kt on bfloat16 MFMA, three per fp32 product
        res["state_products"] = "bf16 MFMA, split fp32 operands (hi*hi + hi*lo + lo*hi)"
    else:
        res["tile_w"] = K.kda_query_variant(1, H, d, d, T_max=n, op=K.KDA_OP_PREFILL, tile_w=tile_w)[0]
    return res


def state_transfer(D, K, synth, reps):
    """Pack / unpack the states of 64 slots x 32 heads (128 MiB) between the slot cache and a
    contiguous buffer on the GPU, and in pinned host memory over PCIe."""
    torch = D.torch
    w = synth.make(64, 32, 128, 128, num_slots=256, state_std=0.02, seed=81)
    cache = D.f(w.cache)
    tables = [D.i(t) for t in w.slot_tables]
    nbytes = 64 * 32 * 128 * 128 * 4
    dbuf = torch.empty(64, 32, 128, 128, device=D.dev)
    hbuf = torch.empty(64, 32, 128, 128, pin_memory=True)
    res = {}
    for name, buf, op in (("pack_device", dbuf, K.kda_state_pack), ("unpack_device", dbuf, K.kda_state_unpack),
                          ("pack_pinned_host", hbuf, K.kda_state_pack),
                          ("unpack_pinned_host", hbuf, K.kda_state_unpack)):
        n = reps if "device" in name else max(2, reps // 20)
        op(cache, tables[0], buf)
        ms = timed_region(D, lambda i: op(cache, tables[i % len(tables)], buf), n) / n
        # a copy reads and writes the bytes once; over PCIe the host side is what counts
        moved = 2 * nbytes if "device" in name else nbytes
        res[name] = dict(us=round(ms * 1e3, 2), bytes=moved, gbs=round(moved / ms / 1e6, 1))
        log(f"state transfer {name}: {ms * 1e3:.1f} us ({moved / ms / 1e6:.0f} GB/s)")
    return res


def _ceiling_lib():
    import ctypes

    from gated_delta_rule_98_amd import build

    if not os.path.exists(build.CEILING_LIB):
        raise RuntimeError(f"{build.CEILING_LIB} is missing: run __graft_entry__.build() first")
    lib = ctypes.CDLL(build.CEILING_LIB)
    P, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.kda_ceiling_rmw.argtypes = [P, i64, P]
    lib.kda_ceiling_copy.argtypes = [P, P, i64, P]
    lib.kda_ceiling_read.argtypes = [P, i64, P, P]
    for fn in (lib.kda_ceiling_rmw, lib.kda_ceiling_copy, lib.kda_ceiling_read):
        fn.restype = ctypes.c_int
    return lib


def ceiling(D, reps=200):
    """The HBM rate of plain streams with the single-token step's state access shape (one
    128-bit access per lane, one wave per workgroup, non-temporal): an in-place
    read-modify-write of 128 MiB (the B=64 step's state bytes, read and written), a 128 MiB
    copy and a 128 MiB read, each rotating over the four 128 MiB regions of a 512 MiB buffer
    so that the data comes from HBM. Median of 3 timed regions of `reps` launches."""
    lib = _ceiling_lib()
    torch = D.torch
    region = (128 << 20) // 4
    buf = torch.ones(4 * region, device=D.dev)
    sink = torch.zeros(64, device=D.dev)
    stream = torch.cuda.current_stream().cuda_stream
    base = buf.data_ptr()

    def rmw(i):
        assert lib.kda_ceiling_rmw(base + (i % 4) * region * 4, region, stream) == 0

    def copy(i):
        assert lib.kda_ceiling_copy(base + (i % 4) * region * 4, base + ((i + 2) % 4) * region * 4, region,
                                    stream) == 0

    def read(i):
        assert lib.kda_ceiling_read(base + (i % 4) * region * 4, region, sink.data_ptr(), stream) == 0

    res = {}
    for name, fn, moved in (("rmw_in_place", rmw, 2 * region * 4), ("copy", copy, 2 * region * 4),
                            ("read", read, region * 4)):
        for i in range(20):
            fn(i)
        ms = float(np.median([timed_region(D, fn, reps) / reps for _ in range(3)]))
        res[name] = dict(us=round(ms * 1e3, 3), bytes=moved, gbs=round(moved / ms / 1e6, 1))
        log(f"ceiling {name}: {ms * 1e3:.2f} us for {moved} B ({moved / ms / 1e6:.0f} GB/s)")
    # the same read-modify-write at the state sizes of the smaller configurations, timed like
    # them (HIP-graph replays): the B=16 step's 32 MiB and the 48 MiB the mixed batch commits
    # (24 rows x 32 heads); a single round of workgroups reads, then writes, so the
    # attainable rate falls with the size
    for mib in (32, 48):
        sub = (mib << 20) // 4
        nreg = 4 * region // sub

        def rmw_sub(i, sub=sub, nreg=nreg):
            # the stream current at the call: a graph capture runs on its own stream
            cur = torch.cuda.current_stream().cuda_stream
            assert lib.kda_ceiling_rmw(base + (i % nreg) * sub * 4, sub, cur) == 0

        for i in range(20):
            rmw_sub(i)
        ms = graph_ms(D, rmw_sub, reps)
        res[f"rmw_in_place_{mib}mib"] = dict(us=round(ms * 1e3, 3), bytes=2 * sub * 4,
                                             gbs=round(2 * sub * 4 / ms / 1e6, 1))
        log(f"ceiling rmw_in_place_{mib}mib: {ms * 1e3:.2f} us for {2 * sub * 4} B "
            f"({2 * sub * 4 / ms / 1e6:.0f} GB/s)")
    del buf
    return res


def copy_calibration(D, reps=5):
    """Plain device copies of known size, 256 MiB read and 256 MiB written each (the ceiling
    probe's copy_kernel), for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE."""
    lib = _ceiling_lib()
    n = (256 << 20) // 4
    buf = D.torch.ones(2 * n, device=D.dev)
    stream = D.torch.cuda.current_stream().cuda_stream
    for _ in range(reps):
        assert lib.kda_ceiling_copy(buf.data_ptr(), buf.data_ptr() + n * 4, n, stream) == 0
    D.sync()
    log(f"copy calibration: {reps} copies of {n * 4} bytes (copy_kernel)")


# ----------------------------------------------------------------------------- CPU baseline

def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _rate(fn, seconds, max_calls=100000):
    """Calls of fn per second over at least one call and about `seconds` of wall time."""
    n = 0
    t0 = time.perf_counter()
    while n < max_calls:
        fn(n)
        n += 1
        if time.perf_counter() - t0 >= seconds:
            break
    return n / (time.perf_counter() - t0), n


def cpu_baseline(w, seconds_scale=1.0):
    """The CPU oracle (as it stands: fp64 arithmetic, fp32 state, one thread per (row, head)
    item list) on this host: the B=64 H=32 d=128 single-token step on every core this process
    may use and on one core, and the B=1 H=32 d=128 step (the 1024-step latency path's unit
    of work) on every core and on one. Each figure is the median of 3 samples; about 20 s of
    CPU time in all."""
    import oracle
    import synth

    cores = len(os.sched_getaffinity(0))
    b1 = synth.make(1, 32, 128, 128, num_slots=1, seed=5, name="b1")
    res = {}
    for key, work, threads, seconds in (("b64_all_cores", w, cores, 3.0), ("b64_one_core", w, 1, 2.0),
                                        ("b1_all_cores", b1, cores, 1.0), ("b1_one_core", b1, 1, 1.0)):
        cache = work.cache.copy()

        def step(n, work=work, cache=cache, threads=threads):
            table = work.slot_tables[n % len(work.slot_tables)]
            oracle.decode(cache, table, work.q[0], work.k[0], work.v[0], work.alpha[0], work.beta[0],
                          nthreads=threads)

        samples = [_rate(step, seconds * seconds_scale) for _ in range(3)]
        rates = [r for r, _ in samples]
        res[key] = dict(steps_per_s=round(float(np.median(rates)), 3),
                        us_per_step=round(1e6 / float(np.median(rates)), 1),
                        samples_steps_per_s=[round(r, 3) for r in rates], threads=threads,
                        steps_per_sample=[n for _, n in samples])
        log(f"cpu baseline {key}: {', '.join(f'{r:.2f}' for r in rates)} steps/s on {threads} thread(s)")
    nbytes = decode_bytes(64, 32, 128, 128)
    main = res["b64_all_cores"]
    return dict(value=main["steps_per_s"], unit="steps/s", cores=cores, kind="oracle",
                sample="median of 3 samples of ~3 s each: single-token steps of the B=64 H=32 d=128 workload "
                       "(4 rotating slot tables) on every core this process may use; fp64 arithmetic with "
                       "fp32 state",
                gbs=round(nbytes * main["steps_per_s"] / 1e9, 3), cpu_count=os.cpu_count(), affinity_cores=cores,
                cpu_model=_cpu_model(), one_core_steps_per_s=res["b64_one_core"]["steps_per_s"],
                b1_us_per_step_all_cores=res["b1_all_cores"]["us_per_step"],
                b1_us_per_step_one_core=res["b1_one_core"]["us_per_step"], detail=res)


# ----------------------------------------------------------------------------- counters

def stored_traffic(tile, key="hbm_bytes_per_launch"):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken on
    the current decode kernel source and the same launch shape: FETCH_SIZE + WRITE_SIZE scaled
    by a plain copy's counts (hbm_bytes_per_launch), or the TCC_EA0 read and write request
    counts times their sizes (request_bytes_per_launch)."""
    if not os.path.exists(COUNTERS_FILE):
        return None
    fields = {}
    for line in open(COUNTERS_FILE):
        if ":" in line and not line.startswith("#"):
            name, val = line.split(":", 1)
            fields[name.strip()] = val.strip()
    if fields.get("kernel_source_sha256") != kernel_source_sha256():
        return None
    if fields.get("launch") != f"tile_w {tile[0]}, threads {tile[1]}":
        return None
    try:
        return int(float(fields[key]))
    except (KeyError, ValueError):
        return None


def size_ceiling_fracs(breakdown):
    """The B=16 replay commit and the mixed batch's commit against the in-place
    read-modify-write ceiling measured at their own state sizes."""
    c = breakdown.get("hbm_ceiling") or {}
    sv = (breakdown.get("spec_verify_b16_t8") or {}).get("replay")
    if sv and "rmw_in_place_32mib" in c:
        sv["commit_frac_of_size_ceiling"] = round(sv["commit_gbs"] / c["rmw_in_place_32mib"]["gbs"], 4)
    mx = breakdown.get("mixed_b64_gated")
    if mx and "rmw_in_place_48mib" in c:
        mx["commit_frac_of_size_ceiling"] = round(mx["commit_gbs"] / c["rmw_in_place_48mib"]["gbs"], 4)


# ----------------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    # 2000 warmup steps (~90 ms): with 50 the timed region ran ~2% slower on MI355X, before the
    # GPU settled into its steady state
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=2000)
    ap.add_argument("--no-breakdown", action="store_true", help="headline only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the ceiling probe (ceiling fields null), for short profiling runs")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run plain device copies of 256 MiB (copy_kernel, for counter scaling)")
    ap.add_argument("--only", default="",
                    help="comma-separated breakdown parts to run (default: all), e.g. spec_verify,mixed")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: the KDA state step is independent per (sequence, head), "
              "so a multi-GPU run is this kernel on each GPU's share with no exchange; "
              "run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import gated_delta_rule_98_amd as K
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    K.load_library()
    D = Dev()
    log(f"device: {torch.cuda.get_device_name(0)}; library {K.LIB_PATH}")

    h = headline(D, K, synth, args.steps, args.warmup)
    breakdown = None
    if not args.no_breakdown:
        parts = dict(
            decode_batch_sweep=lambda: batch_sweep(D, K, synth, reps=256),
            b1_latency_1024_steps=lambda: b1_latency(D, K, synth),
            spec_verify_b16_t8=lambda: spec_verify(D, K, synth, reps=200),
            spec_verify_b64_t8=lambda: spec_verify(D, K, synth, reps=50, B=64),
            spec_verify_small_batch=lambda: spec_verify_small(D, K, synth, reps=200),
            mixed_b64_gated=lambda: mixed(D, K, synth, reps=200),
            prefill_8k_checkpoint=lambda: prefill_8k(D, K, synth, reps=5),
            prefill_8k_checkpoint_chunked=lambda: prefill_8k(D, K, synth, reps=5, chunked=True),
            state_transfer_64x32_heads=lambda: state_transfer(D, K, synth, reps=100),
            raw_inputs_decode=lambda: raw_inputs_decode(D, K, synth, reps=200),
            hbm_ceiling=lambda: ceiling(D),
        )
        only = [p for p in args.only.split(",") if p]
        unknown = [p for p in only if not any(name.startswith(p) for name in parts)]
        if unknown:
            print(f"unknown breakdown part(s) {unknown}; parts: {list(parts)}", file=sys.stderr)
            sys.exit(2)
        breakdown = {name: fn() for name, fn in parts.items() if not only or any(name.startswith(p) for p in only)}
        breakdown["headline_same_table_kernel_us"] = round(h["hot_ms"] * 1e3, 3)
        size_ceiling_fracs(breakdown)
    if args.copy_calibration:
        copy_calibration(D)
    if breakdown and "hbm_ceiling" in breakdown:
        ceil = breakdown["hbm_ceiling"]
    else:
        ceil = None if args.no_ceiling else ceiling(D)
    cpu = None if args.no_cpu_baseline else cpu_baseline(h["w"])

    achieved = h["bytes"] / h["kernel_ms"] / 1e6
    line = {
        "metric": METRIC,
        "value": round(1e3 / h["ms_step"], 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(h["ms_step"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "single-token KDA decode, B=64, H=32, dk=dv=128, fp32 state in a 256-slot "
                               "cache, 4 rotating disjoint slot tables",
                   "global_batch": 64, "heads": 32, "dk": 128, "dv": 128, "tile_w": h["tile"][0],
                   "threads": h["tile"][1], "tokens_per_s": round(64 * 1e3 / h["ms_step"], 1)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": stored_traffic(h["tile"]),
                     "traffic_from_requests": stored_traffic(h["tile"], "request_bytes_per_launch"),
                     "algorithmic_bytes_per_launch": h["bytes"],
                     "kernel_us": round(h["kernel_ms"] * 1e3, 3),
                     "kernel_us_regions": [round(r * 1e3, 3) for r in h["regions_ms"]],
                     "kernel_us_event_pair_per_launch": round(h["pairs_ms"] * 1e3, 3),
                     "ceiling_gbs": ceil["rmw_in_place"]["gbs"] if ceil else None,
                     "ceiling_kernel": "in-place read-modify-write of the same 256 MiB of state traffic "
                                       "(libkda_ceiling.so rmw_kernel), median of 3 regions",
                     "frac_of_ceiling": round(achieved / ceil["rmw_in_place"]["gbs"], 4) if ceil else None},
        "cpu_baseline": cpu,
        "breakdown": breakdown,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
