"""The shared input generator: bf16 rounding against torch's own cast, determinism, shapes."""

import numpy as np
import torch

import synth


def test_bf16_rounding_matches_torch():
    rng = np.random.Generator(np.random.PCG64(0))
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * s for s in (1e-30, 1e-3, 1, 1e30)])
    ties = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -1.0 - 2.0 ** -8], np.float32)  # exact halfway cases
    x = np.concatenate([x, ties])
    ours = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(synth.bf16_bits_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_workloads_are_deterministic_and_shaped():
    a = synth.make_workload("tiny")
    b = synth.make_workload("tiny")
    for f in ("q", "k", "v", "alpha", "beta", "cache", "slot_ids"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
    assert a.q.shape == (256, 1, 4, 64) and a.cache.shape == (1, 4, 64, 64)
    m = synth.make(5, 2, 8, 16, seqlens=[1, 3, 0, 2, 1], num_slots=9, state_std=0.02, gate=True)
    assert list(m.cu_seqlens) == [0, 1, 4, 4, 6, 7] and m.T_max == 3
    assert m.q.shape == (1, 7, 2, 8) and m.v.shape == (1, 7, 2, 16) and m.gate.shape == (1, 7, 2, 16)
    assert len(set(m.slot_ids.tolist())) == 5 and m.slot_ids.max() < 9
    assert m.accepted[0] == 0 and 1 <= m.accepted[1] <= 3 and m.accepted[2] == 0 and 1 <= m.accepted[3] <= 2
    assert m.q_raw.shape == m.q.shape and m.q_raw.dtype == np.uint16 and m.k_raw.shape == m.k.shape
    assert m.a_raw.shape == m.alpha.shape and m.a_raw.dtype == np.float32 and m.b_raw.shape == m.beta.shape
    assert np.array_equal(synth.make(5, 2, 8, 16, seqlens=[1, 3, 0, 2, 1], num_slots=9, state_std=0.02,
                                     gate=True).a_raw, m.a_raw)
    kf = synth.bf16_bits_to_f32(m.k).astype(np.float64)
    assert np.allclose(np.linalg.norm(kf, axis=-1), 1.0, atol=1e-2)
    assert np.all((m.alpha > 0) & (m.alpha < 1)) and np.all((m.beta > 0) & (m.beta < 1))
    assert abs(float(np.std(m.cache)) - 0.02) < 2e-3
    # rotation tables for a cache larger than the batch are disjoint and cover the cache
    w = synth.make(4, 1, 8, 8, num_slots=16, state_std=0.02)
    assert w.slot_tables.shape == (4, 4)
    assert sorted(w.slot_tables.ravel().tolist()) == list(range(16))
    assert np.array_equal(w.slot_tables[0], w.slot_ids)
