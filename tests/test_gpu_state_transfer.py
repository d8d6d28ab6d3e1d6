"""kda_state_pack / kda_state_unpack: bit-exact head- and column-range copies between
the slot cache and a contiguous buffer on the GPU or in pinned host memory."""

import numpy as np
import pytest
import torch

import gated_delta_rule_98_amd as K
import synth
from gpu_util import SENTINEL_BITS, bits, dev, f32, i32, log

pytestmark = pytest.mark.gpu


def _cache(num_slots=12, H=6, d=128, seed=71):
    w = synth.make(1, H, d, d, num_slots=num_slots, state_std=1.0, seed=seed)
    return w.cache


@pytest.mark.parametrize("pinned", [False, True])
def test_pack_full_and_ranges(pinned):
    cache_h = _cache()
    cache_d = f32(cache_h)
    slots = np.array([7, -1, 3, 11], np.int32)
    for heads, cols in ((None, None), ((1, 4), None), (None, (32, 96)), ((5, 6), (0, 64))):
        h0, h1 = heads or (0, 6)
        c0, c1 = cols or (0, 128)
        shape = (4, h1 - h0, c1 - c0, 128)
        if pinned:
            buf = torch.empty(shape, dtype=torch.float32, pin_memory=True)
            buf.view(torch.int32).fill_(SENTINEL_BITS)
        else:
            buf = torch.full(shape, SENTINEL_BITS, dtype=torch.int32, device=dev()).view(torch.float32)
        log(f"pack heads={heads} cols={cols} pinned={pinned}")
        K.kda_state_pack(cache_d, i32(slots), buf, heads=heads, cols=cols)
        torch.cuda.synchronize()
        got = buf.view(torch.int32).numpy().view(np.uint32) if pinned else bits(buf)
        for b, s in enumerate(slots):
            if s < 0:
                assert np.all(got[b] == SENTINEL_BITS)
            else:
                assert np.array_equal(got[b], cache_h[s, h0:h1, c0:c1].view(np.uint32))


@pytest.mark.parametrize("pinned", [False, True])
def test_round_trip_into_other_slots(pinned):
    src_h = _cache(seed=72)
    dst_h = _cache(seed=73)
    src_d, dst_d = f32(src_h), f32(dst_h)
    from_slots = np.array([2, 9, 5], np.int32)
    to_slots = np.array([0, 10, 4], np.int32)
    shape = (3, 6, 128, 128)
    buf = torch.empty(shape, dtype=torch.float32, pin_memory=True) if pinned else \
        torch.empty(shape, dtype=torch.float32, device=dev())
    log(f"round trip pinned={pinned}")
    K.kda_state_pack(src_d, i32(from_slots), buf)
    K.kda_state_unpack(dst_d, i32(to_slots), buf)
    torch.cuda.synchronize()
    got = bits(dst_d)
    assert np.array_equal(got[to_slots], src_h[from_slots].view(np.uint32))
    others = np.setdiff1d(np.arange(12), to_slots)
    assert np.array_equal(got[others], dst_h[others].view(np.uint32))


def test_unpack_column_range_and_errors():
    cache_h = _cache(seed=74)
    cache_d = f32(cache_h)
    buf = torch.randn(2, 2, 16, 128, device=dev())
    err = torch.zeros(1, dtype=torch.int32, device=dev())
    log("unpack a head/column range, one slot past the cache")
    K.kda_state_unpack(cache_d, i32([6, 12]), buf, heads=(3, 5), cols=(112, 128), dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == K.KDA_DEVERR_SLOT
    got = cache_d.cpu().numpy()
    expect = cache_h.copy()
    expect[6, 3:5, 112:128] = buf[0].cpu().numpy()
    assert np.array_equal(got.view(np.uint32), expect.view(np.uint32))
