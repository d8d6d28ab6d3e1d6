"""The C ABI on the host: the library loads, exports what include/kda.h declares,
reports launch shapes, and rejects bad arguments before anything is enqueued.

The argument checks below hand the library fake (never dereferenced) device
addresses. Every call is built to fail a host check, so nothing is launched; as
a second guard the module only runs where no GPU is visible.
"""

import ctypes
import os
import re

import pytest
import torch

from gated_delta_rule_98_amd import kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"^(?:int|const char \*)\s*(kda_\w+)\s*\(", text, flags=re.M)


def test_header_declares_the_boundary():
    assert set(declared_functions()) == {"kda_decode_step", "kda_verify_chunk", "kda_replay_commit",
                                         "kda_prefill", "kda_prefill_chunked", "kda_prefill_chunked_workspace",
                                         "kda_prefill_chunked_noalloc",
                                         "kda_state_pack", "kda_state_unpack",
                                         "kda_query_variant", "kda_status_str"}


def test_library_exports_every_declared_symbol():
    lib = kda.load_library()
    for name in declared_functions():
        assert getattr(lib, name) is not None, name
    out = os.popen(f"nm -D --defined-only {kda.LIB_PATH}").read()
    for name in declared_functions():
        assert re.search(rf"\bT {name}\b", out), name


def test_python_binding_has_the_same_names():
    import gated_delta_rule_98_amd as pkg
    for name in declared_functions():
        assert callable(getattr(pkg, name)), name


def test_query_variant_launch_shapes():
    q = kda.kda_query_variant
    D, V, CR, CC = kda.KDA_OP_DECODE, kda.KDA_OP_VERIFY, kda.KDA_OP_COMMIT_REPLAY, kda.KDA_OP_COMMIT_COPY
    # single-token step: widest tile with >= 256 workgroups; a pure stream past 1024
    assert q(1, 32, 128, 128) == (16, 256)          # 256 workgroups
    assert q(2, 32, 128, 128) == (32, 256)
    assert q(4, 32, 128, 128) == (64, 256)
    assert q(16, 32, 128, 128) == (128, 256)        # 512 heads: two 128-column workgroups per CU
    assert q(12, 32, 128, 128) == (64, 256)         # 768 workgroups
    assert q(32, 16, 128, 128) == (128, 256) and q(8, 64, 128, 128) == (128, 256)
    assert q(32, 32, 128, 128) == (2, 64)
    assert q(64, 32, 128, 128) == (2, 64)           # 65536 one-wave workgroups of column pairs
    assert q(64, 32, 64, 64) == (4, 64)             # dk = 64: 4 columns, one float4 per lane
    assert q(64, 32, 64, 128) == (4, 64)
    # column pairs: only the single-token step at dk = 128, without the gate
    assert q(3, 5, 128, 128, tile_w=2) == (2, 64) and q(3, 5, 128, 64, tile_w=2) == (2, 64)
    for bad in (dict(dk=64), dict(op=V, T_max=4), dict(op=CR, T_max=4), dict(op=CC, T_max=4),
                dict(op=kda.KDA_OP_PREFILL, T_max=100), dict(epilogue=True)):
        args = dict(B=3, H=5, dk=128, dv=128, tile_w=2)
        args.update(bad)
        with pytest.raises(kda.KdaError) as e:
            q(**args)
        assert e.value.status == kda.KDA_ERR_UNSUPPORTED, bad
    assert q(1, 4, 64, 64) == (16, 256)
    # verify / replay commit: 32 columns while >= 512 workgroups
    assert q(16, 32, 128, 128, T_max=8, op=V) == (32, 256)
    assert q(16, 32, 128, 128, T_max=8, op=CR) == (32, 256)
    assert q(24, 32, 128, 128, T_max=8, op=CR) == (16, 256)   # from 768 heads: 16 columns
    assert q(64, 32, 128, 128, T_max=8, op=CR) == (16, 256)
    assert q(2, 32, 128, 128, T_max=8, op=V) == (32, 256)
    assert q(1, 32, 128, 128, T_max=8, op=V) == (16, 256)
    assert q(8, 32, 128, 128, T_max=8, op=CR) == (16, 256)
    assert q(1, 4, 128, 128, T_max=8, op=CR) == (8, 128)
    assert q(1, 4, 128, 128, T_max=8, op=V) == (8, 128)
    assert q(16, 32, 128, 128, T_max=8, op=CC) == (16, 256)
    P = kda.KDA_OP_PREFILL
    assert q(1, 32, 128, 128, T_max=8000, op=P) == (16, 256)     # prompts of any length
    assert q(64, 32, 128, 128, T_max=100, op=P) == (32, 256)
    assert q(1, 32, 128, 128, T_max=100, op=P, tile_w=32) == (32, 256)
    with pytest.raises(kda.KdaError):
        q(1, 32, 128, 128, T_max=100, op=P, tile_w=64)
    # the output gate needs the whole head in one workgroup
    assert q(64, 32, 128, 128, epilogue=True) == (128, 1024)   # decode: 16 waves x 2 slabs
    assert q(64, 32, 128, 128, T_max=4, epilogue=True, op=V) == (128, 1024)   # verify: 16 waves x 2 slabs
    assert q(64, 32, 128, 64, epilogue=True) == (64, 512)
    assert q(64, 32, 128, 64, T_max=4, epilogue=True, op=V) == (64, 512)
    for w, threads in ((4, 64), (8, 128), (16, 256), (32, 256), (64, 256), (128, 256)):
        assert q(3, 5, 128, 128, tile_w=w) == (w, threads)
    for bad in (dict(tile_w=24), dict(tile_w=256), dict(epilogue=True, tile_w=64)):
        with pytest.raises(kda.KdaError) as e:
            q(2, 2, 128, 128, **bad)
        assert e.value.status == kda.KDA_ERR_UNSUPPORTED
    with pytest.raises(kda.KdaError) as e:
        q(2, 2, 128, 64, tile_w=128)
    assert e.value.status == kda.KDA_ERR_UNSUPPORTED
    for bad in (dict(dk=96), dict(dv=32), dict(T_max=17), dict(T_max=0)):
        args = dict(B=2, H=2, dk=128, dv=128, T_max=1)
        args.update(bad)
        with pytest.raises(kda.KdaError) as e:
            q(**args)
        assert e.value.status == kda.KDA_ERR_UNSUPPORTED
    for bad in (dict(H=0), dict(op=7), dict(op=CC, epilogue=True)):
        args = dict(B=2, H=2, dk=128, dv=128)
        args.update(bad)
        with pytest.raises(kda.KdaError) as e:
            q(**args)
        assert e.value.status == kda.KDA_ERR_INVALID


def test_status_strings():
    assert kda.kda_status_str(0) == "ok"
    for code in (-1, -2, -3, -4, -5):
        assert kda.kda_status_str(code) not in ("ok", "unknown status")
    assert kda.kda_status_str(7) == "unknown status"


gpu_visible = torch.cuda.device_count() > 0
needs_no_gpu = pytest.mark.skipif(gpu_visible, reason="hands fake device addresses to the library")

A = 0x10000          # fake, 256-byte aligned device addresses (never dereferenced)
P = ctypes.c_void_p


def _decode(**over):
    d = dict(cache=A, num_slots=8, slot_stride=2 * 128 * 128, slot_ids=A, B=4, H=2, dk=128, dv=128,
             q=A, k=A, v=A, alpha=A, beta=A, out=A, epi=None, dev_err=None, opts=None, stream=None)
    d.update(over)
    return kda.load_library().kda_decode_step(*d.values())


def _verify(**over):
    d = dict(cache=A, num_slots=8, slot_stride=2 * 128 * 128, slot_ids=A, cu=A, B=4, T_max=4, n_tok=9,
             H=2, dk=128, dv=128, q=A, k=A, v=A, alpha=A, beta=A, out=A, epi=None, mode=0, t1=0,
             rb=None, draft=None, dev_err=None, opts=None, stream=None)
    d.update(over)
    return kda.load_library().kda_verify_chunk(*d.values())


def _commit(**over):
    d = dict(cache=A, num_slots=8, slot_stride=2 * 128 * 128, slot_ids=A, cu=None, acc=A, B=4, T_max=4,
             n_tok=9, H=2, dk=128, dv=128, mode=1, rb=None, draft=None, dev_err=None, opts=None, stream=None)
    d.update(over)
    return kda.load_library().kda_replay_commit(*d.values())


@needs_no_gpu
def test_decode_host_checks():
    E = kda
    assert _decode(B=0) == E.KDA_OK                                   # empty batch: nothing enqueued
    assert _decode(B=-1) == E.KDA_ERR_INVALID
    assert _decode(H=0) == E.KDA_ERR_INVALID
    assert _decode(cache=None) == E.KDA_ERR_INVALID
    assert _decode(slot_ids=None) == E.KDA_ERR_INVALID
    assert _decode(q=None) == E.KDA_ERR_INVALID
    assert _decode(out=None) == E.KDA_ERR_INVALID
    assert _decode(num_slots=-1) == E.KDA_ERR_INVALID
    assert _decode(slot_stride=2 * 128 * 128 - 4) == E.KDA_ERR_INVALID
    assert _decode(dk=96) == E.KDA_ERR_UNSUPPORTED
    assert _decode(dv=256) == E.KDA_ERR_UNSUPPORTED
    assert _decode(cache=A + 4) == E.KDA_ERR_ALIGN
    assert _decode(slot_stride=2 * 128 * 128 + 2) == E.KDA_ERR_ALIGN
    assert _decode(alpha=A + 8) == E.KDA_ERR_ALIGN
    assert _decode(q=A + 2) == E.KDA_ERR_ALIGN
    assert _decode(k=A + 4) == E.KDA_ERR_ALIGN
    assert _decode(beta=A + 2) == E.KDA_ERR_ALIGN
    assert _decode(dev_err=A + 2) == E.KDA_ERR_ALIGN
    gate_null = kda.kda_epilogue(None, None, 1e-6)
    assert _decode(epi=ctypes.byref(gate_null)) == E.KDA_ERR_INVALID
    neg_eps = kda.kda_epilogue(A, None, -1.0)
    assert _decode(epi=ctypes.byref(neg_eps)) == E.KDA_ERR_INVALID
    nan_eps = kda.kda_epilogue(A, None, float("nan"))
    assert _decode(epi=ctypes.byref(nan_eps)) == E.KDA_ERR_INVALID
    gate_mis = kda.kda_epilogue(A + 2, None, 1e-6)
    assert _decode(epi=ctypes.byref(gate_mis)) == E.KDA_ERR_ALIGN
    assert _decode(opts=ctypes.byref(kda.kda_options(24, 0))) == E.KDA_ERR_UNSUPPORTED
    ok_gate = kda.kda_epilogue(A, None, 1e-6)
    assert _decode(epi=ctypes.byref(ok_gate), opts=ctypes.byref(kda.kda_options(64, 0))) == E.KDA_ERR_UNSUPPORTED
    # option flags: unknown bits are rejected; a bf16 output needs 2-byte alignment only
    assert _decode(opts=ctypes.byref(kda.kda_options(0, 0, 8))) == E.KDA_ERR_INVALID
    assert _decode(out=A + 2) == E.KDA_ERR_ALIGN
    assert _decode(out=A + 1, opts=ctypes.byref(kda.kda_options(0, 0, E.KDA_OUT_BF16))) == E.KDA_ERR_ALIGN
    # passes every host check: only the launch itself fails without a device
    assert _decode(out=A + 2, opts=ctypes.byref(kda.kda_options(0, 0, E.KDA_OUT_BF16))) == E.KDA_ERR_HIP
    assert _decode(opts=ctypes.byref(kda.kda_options(0, 0, E.KDA_RAW_INPUTS | E.KDA_OUT_BF16))) == E.KDA_ERR_HIP


@needs_no_gpu
def test_verify_host_checks():
    E = kda
    rb = kda.kda_replay_buf(A, A, A, A)
    assert _verify(B=0) == E.KDA_OK
    assert _verify(n_tok=0) == E.KDA_OK
    assert _verify(n_tok=-1) == E.KDA_ERR_INVALID
    assert _verify(mode=2) == E.KDA_ERR_INVALID
    assert _verify(T_max=0) == E.KDA_ERR_UNSUPPORTED
    assert _verify(T_max=17) == E.KDA_ERR_UNSUPPORTED
    assert _verify(cu=None, rb=ctypes.byref(rb)) == E.KDA_ERR_INVALID
    assert _verify(mode=0, rb=None) == E.KDA_ERR_INVALID                      # replay buffer required
    assert _verify(mode=0, rb=ctypes.byref(kda.kda_replay_buf(A, None, A, A))) == E.KDA_ERR_INVALID
    assert _verify(mode=0, rb=ctypes.byref(kda.kda_replay_buf(A, A, A + 8, A))) == E.KDA_ERR_ALIGN
    assert _verify(mode=1, draft=None) == E.KDA_ERR_INVALID                   # draft required
    assert _verify(mode=1, draft=A + 4) == E.KDA_ERR_ALIGN
    assert _verify(mode=1, draft=A, cache=A + 8) == E.KDA_ERR_ALIGN
    assert _verify(mode=1, draft=A, dk=64, dv=96) == E.KDA_ERR_UNSUPPORTED
    # the chunk form takes neither raw inputs nor a bf16 output
    rb_ok = ctypes.byref(rb)
    for flags in (E.KDA_RAW_INPUTS, E.KDA_OUT_BF16):
        opts = ctypes.byref(kda.kda_options(0, E.KDA_VERIFY_CHUNKED, flags))
        assert _verify(mode=0, rb=rb_ok, opts=opts) == E.KDA_ERR_UNSUPPORTED
    assert _verify(mode=0, rb=rb_ok, opts=ctypes.byref(kda.kda_options(0, 0, 8))) == E.KDA_ERR_INVALID


@needs_no_gpu
def test_commit_host_checks():
    E = kda
    assert _commit(B=0) == E.KDA_OK
    assert _commit(acc=None, draft=A) == E.KDA_ERR_INVALID
    assert _commit(mode=1, draft=None) == E.KDA_ERR_INVALID
    assert _commit(mode=0, rb=None) == E.KDA_ERR_INVALID
    assert _commit(mode=3, draft=A) == E.KDA_ERR_INVALID
    assert _commit(mode=1, draft=A + 4) == E.KDA_ERR_ALIGN
    assert _commit(mode=1, draft=A, acc=A + 2) == E.KDA_ERR_ALIGN
    assert _commit(mode=1, draft=A, T_max=32) == E.KDA_ERR_UNSUPPORTED
    assert _commit(mode=1, draft=A, slot_stride=100) == E.KDA_ERR_INVALID
    assert _commit(mode=1, draft=A, opts=ctypes.byref(kda.kda_options(0, 0, 16))) == E.KDA_ERR_INVALID
    # a bf16-output flag carried over from the verify call is accepted and ignored
    assert _commit(mode=1, draft=A, opts=ctypes.byref(kda.kda_options(0, 0, E.KDA_OUT_BF16))) == E.KDA_ERR_HIP


def _prefill(**over):
    d = dict(cache=A, num_slots=8, slot_stride=2 * 128 * 128, slot_ids=A, cu=A, B=4, n_tok=90, H=2, dk=128,
             dv=128, q=A, k=A, v=A, alpha=A, beta=A, out=A, ckpt_pos=None, ckpt=None, dev_err=None, opts=None,
             stream=None)
    d.update(over)
    return kda.load_library().kda_prefill(*d.values())


@needs_no_gpu
def test_prefill_host_checks():
    E = kda
    assert _prefill(B=0) == E.KDA_OK
    assert _prefill(n_tok=0) == E.KDA_OK                     # no tokens, no checkpoint: nothing to do
    assert _prefill(n_tok=-1) == E.KDA_ERR_INVALID
    assert _prefill(cu=None) == E.KDA_ERR_INVALID
    assert _prefill(q=None) == E.KDA_ERR_INVALID
    assert _prefill(ckpt_pos=A, ckpt=None) == E.KDA_ERR_INVALID
    assert _prefill(ckpt_pos=A, ckpt=A + 4) == E.KDA_ERR_ALIGN
    assert _prefill(dk=96) == E.KDA_ERR_UNSUPPORTED
    assert _prefill(opts=ctypes.byref(kda.kda_options(64, 0))) == E.KDA_ERR_UNSUPPORTED
    assert _prefill(alpha=A + 4) == E.KDA_ERR_ALIGN
    assert _prefill(opts=ctypes.byref(kda.kda_options(0, 0, 8))) == E.KDA_ERR_INVALID
    assert _prefill(out=A + 2) == E.KDA_ERR_ALIGN
    assert _prefill(out=A + 2, opts=ctypes.byref(kda.kda_options(0, 0, E.KDA_OUT_BF16))) == E.KDA_ERR_HIP


def _prefill_chunked(**over):
    d = dict(cache=A, num_slots=8, slot_stride=2 * 128 * 128, slot_ids=A, cu=A, B=4, n_tok=90, H=2, dk=128,
             dv=128, q=A, k=A, v=A, alpha=A, beta=A, out=A, ckpt_pos=None, ckpt=None, ws=A, ws_bytes=1 << 40,
             dev_err=None, opts=None, stream=None)
    d.update(over)
    return kda.load_library().kda_prefill_chunked(*d.values())


@needs_no_gpu
def test_prefill_chunked_host_checks():
    E = kda
    lib = kda.load_library()
    nbytes = ctypes.c_size_t(0)
    assert lib.kda_prefill_chunked_workspace(4, 90, 2, 128, 128, ctypes.byref(nbytes)) == E.KDA_OK
    # (ceil(90 / 32) + 2 * 4) chunks x 2 heads x (3 * 32 * 128 + 32 * 128 + 32 * 32 + 128) floats,
    # then the chunk map: int32 first chunk of each row (B + 1) and row of each chunk (11), to 16 B
    data = 11 * 2 * (3 * 32 * 128 + 32 * 128 + 32 * 32 + 128) * 4
    assert nbytes.value == (data + (4 + 1 + 11) * 4 + 15) // 16 * 16
    assert lib.kda_prefill_chunked_workspace(4, 90, 2, 96, 128, ctypes.byref(nbytes)) == E.KDA_ERR_UNSUPPORTED
    assert lib.kda_prefill_chunked_workspace(4, -1, 2, 128, 128, ctypes.byref(nbytes)) == E.KDA_ERR_INVALID
    assert lib.kda_prefill_chunked_workspace(4, 90, 2, 128, 128, None) == E.KDA_ERR_INVALID
    assert _prefill_chunked(B=0) == E.KDA_OK
    assert _prefill_chunked(n_tok=0) == E.KDA_OK
    assert _prefill_chunked(ws=None) == E.KDA_ERR_INVALID
    assert _prefill_chunked(ws_bytes=1000) == E.KDA_ERR_INVALID              # workspace too small
    assert _prefill_chunked(ws=A + 4) == E.KDA_ERR_ALIGN
    assert _prefill_chunked(cu=None) == E.KDA_ERR_INVALID
    assert _prefill_chunked(dk=96) == E.KDA_ERR_UNSUPPORTED
    assert _prefill_chunked(opts=ctypes.byref(kda.kda_options(32, 0, 0))) == E.KDA_ERR_UNSUPPORTED
    assert _prefill_chunked(opts=ctypes.byref(kda.kda_options(0, 0, 8))) == E.KDA_ERR_INVALID
    assert _prefill_chunked(ckpt_pos=A, ckpt=None) == E.KDA_ERR_INVALID
    assert _prefill_chunked(out=A + 2) == E.KDA_ERR_ALIGN
    # passes every host check: only the launch fails without a device
    assert _prefill_chunked(out=A + 2, opts=ctypes.byref(kda.kda_options(16, 0, E.KDA_OUT_BF16))) == E.KDA_ERR_HIP


def _prefill_noalloc(**over):
    d = dict(cache=A, num_slots=8, slot_stride=2 * 128 * 128, slot_ids=A, cu=A, B=4, n_tok=90, H=2, dk=128,
             dv=128, q=A, k=A, v=A, alpha=A, beta=A, out=A, ckpt_pos=None, ckpt=None, dev_err=None, opts=None,
             stream=None)
    d.update(over)
    return kda.load_library().kda_prefill_chunked_noalloc(*d.values())


@needs_no_gpu
def test_prefill_chunked_noalloc_host_checks():
    """The static-scratch variant: the size limit and the argument checks come before any
    device call; a call that passes them needs the device (the scratch address lookup)."""
    E = kda
    per_chunk_head = (3 * 32 * 128 + 32 * 128 + 32 * 32 + 128) * 4
    limit_chunks = E.KDA_NOALLOC_SCRATCH_BYTES // (32 * per_chunk_head)      # chunks at H = 32
    fits = (limit_chunks - 2) * 32                                          # tokens of one row (B = 1)
    assert _prefill_noalloc(B=0) == E.KDA_OK
    assert _prefill_noalloc(n_tok=0) == E.KDA_OK
    assert _prefill_noalloc(dk=96) == E.KDA_ERR_UNSUPPORTED
    assert _prefill_noalloc(n_tok=-1) == E.KDA_ERR_INVALID
    assert _prefill_noalloc(B=1, H=32, slot_stride=32 * 128 * 128, n_tok=fits + 32) == E.KDA_ERR_TOO_LARGE
    assert _prefill_noalloc(B=1, H=32, slot_stride=32 * 128 * 128, n_tok=1 << 30) == E.KDA_ERR_TOO_LARGE
    # within the limit every host check passes; without a device the scratch lookup fails
    assert _prefill_noalloc(B=1, H=32, slot_stride=32 * 128 * 128, n_tok=fits) == E.KDA_ERR_HIP
    assert fits >= 3600


@needs_no_gpu
def test_duplicate_slot_check():
    """KDA_CHECK_SLOTS reads a host-readable slot table before anything is enqueued and
    rejects two rows naming the same slot; padding rows may repeat. Without the flag the
    table is never read on the host (a fake device address passes)."""
    import numpy as np
    E = kda
    dup = np.array([3, 1, -1, 3], np.int32)
    pad = np.array([3, -1, 1, -1], np.int32)
    chk = ctypes.byref(kda.kda_options(0, 0, E.KDA_CHECK_SLOTS))
    for call in (lambda **kw: _decode(**kw), lambda **kw: _verify(mode=1, draft=A, **kw),
                 lambda **kw: _commit(mode=1, draft=A, **kw),
                 lambda **kw: _prefill(**kw), lambda **kw: _prefill_chunked(**kw),
                 lambda **kw: _prefill_noalloc(**kw)):
        assert call(slot_ids=dup.ctypes.data, opts=chk) == E.KDA_ERR_INVALID
        # distinct ids (padding repeated) pass the check; only the launch fails without a device
        assert call(slot_ids=pad.ctypes.data, opts=chk) == E.KDA_ERR_HIP
    assert _decode(opts=ctypes.byref(kda.kda_options(0, 0, 8))) == E.KDA_ERR_INVALID   # unknown flag bit


def _pack(**over):
    d = dict(cache=A, num_slots=8, slot_stride=4 * 128 * 128, slot_ids=A, B=4, H=4, dk=128, dv=128, head0=0,
             nheads=4, col0=0, ncols=128, buf=A, dev_err=None, stream=None)
    d.update(over)
    return kda.load_library().kda_state_pack(*d.values())


@needs_no_gpu
def test_state_transfer_host_checks():
    E = kda
    assert _pack(B=0) == E.KDA_OK
    assert _pack(nheads=0) == E.KDA_OK
    assert _pack(ncols=0) == E.KDA_OK
    assert _pack(head0=2, nheads=3) == E.KDA_ERR_INVALID
    assert _pack(col0=100, ncols=29) == E.KDA_ERR_INVALID
    assert _pack(head0=-1) == E.KDA_ERR_INVALID
    assert _pack(buf=None) == E.KDA_ERR_INVALID
    assert _pack(buf=A + 8) == E.KDA_ERR_ALIGN
    assert _pack(dk=32) == E.KDA_ERR_UNSUPPORTED
    assert kda.load_library().kda_state_unpack(A, 8, 4 * 128 * 128, A, 4, 4, 128, 128, 0, 4, 0, 128, None,
                                               None, None) == E.KDA_ERR_INVALID
