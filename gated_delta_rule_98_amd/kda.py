"""Python binding of the KDA C ABI (include/kda.h): argument marshalling only.

Each function has the name of the C entry point it calls, takes torch tensors
that already live on the GPU, passes their device pointers and the current
HIP stream, and raises KdaError on a non-zero status. Every step of the
computation runs in the HIP kernels of libkda.so; there is no other path. If
the library is missing, importing the package still works but the first call
raises, naming the build command.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkda.so")

KDA_OK = 0
KDA_ERR_INVALID = -1
KDA_ERR_UNSUPPORTED = -2
KDA_ERR_ALIGN = -3
KDA_ERR_HIP = -4
KDA_ERR_TOO_LARGE = -5

KDA_NOALLOC_SCRATCH_BYTES = 256 << 20   # the library's static workspace of kda_prefill_chunked_noalloc

KDA_REPLAY = 0
KDA_PER_POSITION = 1

KDA_OP_DECODE = 0
KDA_OP_VERIFY = 1
KDA_OP_COMMIT_REPLAY = 2
KDA_OP_COMMIT_COPY = 3
KDA_OP_PREFILL = 4

KDA_VERIFY_AUTO = 0
KDA_VERIFY_RECURRENT = 1
KDA_VERIFY_CHUNKED = 2

KDA_DEVERR_SLOT = 1
KDA_DEVERR_SEQLEN = 2
KDA_DEVERR_ACCEPTED = 4
KDA_DEVERR_CKPT = 8

KDA_RAW_INPUTS = 1
KDA_OUT_BF16 = 2
KDA_CHECK_SLOTS = 4


class KdaError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {kda_status_str(status)} ({status})")
        self.status = status


class kda_epilogue(ctypes.Structure):
    _fields_ = [("gate", ctypes.c_void_p), ("weight", ctypes.c_void_p), ("eps", ctypes.c_float)]


class kda_replay_buf(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("alpha", ctypes.c_void_p),
                ("beta", ctypes.c_void_p)]


class kda_options(ctypes.Structure):
    _fields_ = [("tile_w", ctypes.c_int32), ("verify_form", ctypes.c_int32), ("flags", ctypes.c_int32)]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libkda.so (once). Raises FileNotFoundError when it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise FileNotFoundError(
            f"{path} is missing: build it with `python gated_delta_rule_98_amd/build.py`")
    lib = ctypes.CDLL(path)
    P, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.kda_decode_step.argtypes = [P, i64, i64, P, i32, i32, i32, i32, P, P, P, P, P, P, P, P, P, P]
    lib.kda_decode_step.restype = ctypes.c_int
    lib.kda_verify_chunk.argtypes = [P, i64, i64, P, P, i32, i32, i32, i32, i32, i32,
                                     P, P, P, P, P, P, P, i32, i32, P, P, P, P, P]
    lib.kda_verify_chunk.restype = ctypes.c_int
    lib.kda_replay_commit.argtypes = [P, i64, i64, P, P, P, i32, i32, i32, i32, i32, i32, i32,
                                      P, P, P, P, P]
    lib.kda_replay_commit.restype = ctypes.c_int
    lib.kda_prefill.argtypes = [P, i64, i64, P, P, i32, i32, i32, i32, i32, P, P, P, P, P, P, P, P, P, P, P]
    lib.kda_prefill.restype = ctypes.c_int
    lib.kda_prefill_chunked.argtypes = [P, i64, i64, P, P, i32, i32, i32, i32, i32, P, P, P, P, P, P, P, P,
                                        P, ctypes.c_size_t, P, P, P]
    lib.kda_prefill_chunked.restype = ctypes.c_int
    lib.kda_prefill_chunked_noalloc.argtypes = [P, i64, i64, P, P, i32, i32, i32, i32, i32, P, P, P, P, P, P,
                                                P, P, P, P, P]
    lib.kda_prefill_chunked_noalloc.restype = ctypes.c_int
    lib.kda_prefill_chunked_workspace.argtypes = [i32, i32, i32, i32, i32, ctypes.POINTER(ctypes.c_size_t)]
    lib.kda_prefill_chunked_workspace.restype = ctypes.c_int
    for name in ("kda_state_pack", "kda_state_unpack"):
        fn = getattr(lib, name)
        fn.argtypes = [P, i64, i64, P, i32, i32, i32, i32, i32, i32, i32, i32, P, P, P]
        fn.restype = ctypes.c_int
    lib.kda_query_variant.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32,
                                      ctypes.POINTER(i32), ctypes.POINTER(i32)]
    lib.kda_query_variant.restype = ctypes.c_int
    lib.kda_status_str.argtypes = [i32]
    lib.kda_status_str.restype = ctypes.c_char_p
    _lib = lib
    return lib


def kda_status_str(status: int) -> str:
    return load_library().kda_status_str(int(status)).decode()


def kda_query_variant(B: int, H: int, dk: int, dv: int, T_max: int = 1, epilogue: bool = False,
                      tile_w: int = 0, op: int = KDA_OP_DECODE) -> Tuple[int, int]:
    """(tile width, threads per workgroup) that operation ``op`` launches for this shape."""
    w, t = ctypes.c_int32(0), ctypes.c_int32(0)
    rc = load_library().kda_query_variant(op, B, H, dk, dv, T_max, int(bool(epilogue)), tile_w,
                                          ctypes.byref(w), ctypes.byref(t))
    if rc != KDA_OK:
        raise KdaError(rc, "kda_query_variant")
    return w.value, t.value


# ------------------------------------------------------------------ marshalling

_BF16_TYPES = (torch.bfloat16, torch.int16, torch.uint16)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _dev(t: torch.Tensor, name: str, dtypes, ndim: Optional[int] = None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _shape(t: Optional[torch.Tensor], name: str, shape) -> None:
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _replay(replay: Optional[dict], B: int, T_max: int, H: int, dk: int, dv: int):
    if replay is None:
        return None
    for key, d, shape in (("k", _BF16_TYPES, (B, T_max, H, dk)), ("v", _BF16_TYPES, (B, T_max, H, dv)),
                          ("alpha", (torch.float32,), (B, T_max, H, dk)),
                          ("beta", (torch.float32,), (B, T_max, H))):
        _dev(replay[key], f"replay {key}", d)
        _shape(replay[key], f"replay {key}", shape)
    return kda_replay_buf(replay["k"].data_ptr(), replay["v"].data_ptr(), replay["alpha"].data_ptr(),
                          replay["beta"].data_ptr())


def _cache(cache: torch.Tensor):
    """cache: float32 [num_slots, H, dv, dk]; each slot contiguous, slots at stride(0)."""
    if cache.device.type != "cuda" or cache.dtype != torch.float32 or cache.dim() != 4:
        raise ValueError("cache must be a float32 GPU tensor [num_slots, H, dv, dk]")
    ns, H, dv, dk = cache.shape
    if cache.stride()[1:] != (dv * dk, dk, 1):
        raise ValueError("each cache slot must be contiguous [H, dv, dk]")
    return ns, cache.stride(0), H, dv, dk


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _epilogue(gate, weight, eps):
    if gate is None:
        return None
    _dev(gate, "gate", _BF16_TYPES)
    if weight is not None:
        _dev(weight, "weight", (torch.float32,), 1)
    return kda_epilogue(gate.data_ptr(), _ptr(weight), float(eps))


def _opts(tile_w: int, verify_form: int = 0, flags: int = 0):
    if not (tile_w or verify_form or flags):
        return None
    return kda_options(int(tile_w), int(verify_form), int(flags))


def _flags(raw_inputs: bool, out: Optional[torch.Tensor] = None) -> int:
    """Option flags: raw inputs on request, bf16 output when out holds bf16."""
    f = KDA_RAW_INPUTS if raw_inputs else 0
    if out is not None and out.dtype in _BF16_TYPES:
        f |= KDA_OUT_BF16
    return f


def _ref(x):
    return None if x is None else ctypes.byref(x)


def kda_decode_step(cache: torch.Tensor, slot_ids: torch.Tensor, q, k, v, alpha, beta,
                    out: torch.Tensor, *, gate=None, weight=None, eps: float = 1e-6,
                    dev_err: Optional[torch.Tensor] = None, tile_w: int = 0, raw_inputs: bool = False,
                    stream=None) -> None:
    """One token per row, state updated in place.

    cache float32 [num_slots, H, dv, dk]; slot_ids int32 [B]; q, k bf16 [B, H, dk];
    v bf16 [B, H, dv]; alpha float32 [B, H, dk]; beta float32 [B, H]; out float32 or
    bf16 [B, H, dv]; gate bf16 [B, H, dv] (optional output gate), weight float32 [dv].
    raw_inputs: q, k, alpha, beta are raw projections, prepared in the kernel.
    """
    ns, stride, H, dv, dk = _cache(cache)
    _dev(slot_ids, "slot_ids", (torch.int32,), 1)
    B = slot_ids.shape[0]
    for name, t, d in (("q", q, _BF16_TYPES), ("k", k, _BF16_TYPES), ("v", v, _BF16_TYPES),
                       ("alpha", alpha, (torch.float32,)), ("beta", beta, (torch.float32,)),
                       ("out", out, (torch.float32,) + _BF16_TYPES)):
        _dev(t, name, d)
    for name, t, shape in (("q", q, (B, H, dk)), ("k", k, (B, H, dk)), ("v", v, (B, H, dv)),
                           ("alpha", alpha, (B, H, dk)), ("beta", beta, (B, H)), ("out", out, (B, H, dv)),
                           ("gate", gate, (B, H, dv)), ("weight", weight, (dv,))):
        _shape(t, name, shape)
    if dev_err is not None:
        _dev(dev_err, "dev_err", (torch.int32,))
    epi = _epilogue(gate, weight, eps)
    rc = load_library().kda_decode_step(
        cache.data_ptr(), ns, stride, slot_ids.data_ptr(), B, H, dk, dv,
        q.data_ptr(), k.data_ptr(), v.data_ptr(), alpha.data_ptr(), beta.data_ptr(), out.data_ptr(),
        _ref(epi), _ptr(dev_err), _ref(_opts(tile_w, 0, _flags(raw_inputs, out))), _stream(stream))
    if rc != KDA_OK:
        raise KdaError(rc, "kda_decode_step")


def kda_verify_chunk(cache: torch.Tensor, slot_ids: torch.Tensor, cu_seqlens: torch.Tensor,
                     T_max: int, q, k, v, alpha, beta, out: torch.Tensor, *, mode: int = KDA_REPLAY,
                     t1_inplace: bool = False, replay: Optional[dict] = None,
                     draft: Optional[torch.Tensor] = None, gate=None, weight=None, eps: float = 1e-6,
                     dev_err: Optional[torch.Tensor] = None, tile_w: int = 0, verify_form: int = 0,
                     raw_inputs: bool = False, stream=None) -> None:
    """Packed speculative chunk; token arrays are [n_tok, H, .], row b owns tokens
    [cu[b], cu[b+1]). replay = dict(k, v, alpha, beta) with shapes [B, T_max, H, .]
    (mode KDA_REPLAY); draft float32 [B, T_max, H, dv, dk] (mode KDA_PER_POSITION).
    out is float32 or bf16; raw_inputs as for kda_decode_step (the replay buffer then
    holds the raw inputs and the commit needs raw_inputs too)."""
    ns, stride, H, dv, dk = _cache(cache)
    _dev(slot_ids, "slot_ids", (torch.int32,), 1)
    _dev(cu_seqlens, "cu_seqlens", (torch.int32,), 1)
    B = slot_ids.shape[0]
    if cu_seqlens.shape[0] != B + 1:
        raise ValueError("cu_seqlens must have B + 1 entries")
    for name, t, d in (("q", q, _BF16_TYPES), ("k", k, _BF16_TYPES), ("v", v, _BF16_TYPES),
                       ("alpha", alpha, (torch.float32,)), ("beta", beta, (torch.float32,)),
                       ("out", out, (torch.float32,) + _BF16_TYPES)):
        _dev(t, name, d)
    n_tok = k.shape[0]
    for name, t, shape in (("q", q, (n_tok, H, dk)), ("k", k, (n_tok, H, dk)), ("v", v, (n_tok, H, dv)),
                           ("alpha", alpha, (n_tok, H, dk)), ("beta", beta, (n_tok, H)),
                           ("out", out, (n_tok, H, dv)), ("gate", gate, (n_tok, H, dv)),
                           ("weight", weight, (dv,)), ("draft", draft, (B, T_max, H, dv, dk))):
        _shape(t, name, shape)
    rb = _replay(replay, B, T_max, H, dk, dv)
    if draft is not None:
        _dev(draft, "draft", (torch.float32,))
    if dev_err is not None:
        _dev(dev_err, "dev_err", (torch.int32,))
    epi = _epilogue(gate, weight, eps)
    rc = load_library().kda_verify_chunk(
        cache.data_ptr(), ns, stride, slot_ids.data_ptr(), cu_seqlens.data_ptr(), B, int(T_max),
        n_tok, H, dk, dv, q.data_ptr(), k.data_ptr(), v.data_ptr(), alpha.data_ptr(), beta.data_ptr(),
        out.data_ptr(), _ref(epi), int(mode), int(bool(t1_inplace)), _ref(rb), _ptr(draft),
        _ptr(dev_err), _ref(_opts(tile_w, verify_form, _flags(raw_inputs, out))), _stream(stream))
    if rc != KDA_OK:
        raise KdaError(rc, "kda_verify_chunk")


def kda_replay_commit(cache: torch.Tensor, slot_ids: torch.Tensor, cu_seqlens: Optional[torch.Tensor],
                      accepted_len: torch.Tensor, T_max: int, n_tok: int, *, mode: int = KDA_REPLAY,
                      replay: Optional[dict] = None, draft: Optional[torch.Tensor] = None,
                      dev_err: Optional[torch.Tensor] = None, tile_w: int = 0, raw_inputs: bool = False,
                      stream=None) -> None:
    """Slot of row b <- state after the first accepted_len[b] tokens of its verified chunk.
    raw_inputs must match the verify call that filled the replay buffer (mode KDA_REPLAY)."""
    ns, stride, H, dv, dk = _cache(cache)
    _dev(slot_ids, "slot_ids", (torch.int32,), 1)
    _dev(accepted_len, "accepted_len", (torch.int32,), 1)
    B = slot_ids.shape[0]
    if cu_seqlens is not None:
        _dev(cu_seqlens, "cu_seqlens", (torch.int32,), 1)
        _shape(cu_seqlens, "cu_seqlens", (B + 1,))
    rb = _replay(replay, B, T_max, H, dk, dv)
    if draft is not None:
        _dev(draft, "draft", (torch.float32,))
        _shape(draft, "draft", (B, T_max, H, dv, dk))
    if dev_err is not None:
        _dev(dev_err, "dev_err", (torch.int32,))
    rc = load_library().kda_replay_commit(
        cache.data_ptr(), ns, stride, slot_ids.data_ptr(), _ptr(cu_seqlens), accepted_len.data_ptr(),
        B, int(T_max), int(n_tok), H, dk, dv, int(mode), _ref(rb), _ptr(draft), _ptr(dev_err),
        _ref(_opts(tile_w, 0, _flags(raw_inputs))), _stream(stream))
    if rc != KDA_OK:
        raise KdaError(rc, "kda_replay_commit")


def kda_prefill(cache: torch.Tensor, slot_ids: torch.Tensor, cu_seqlens: torch.Tensor, q, k, v, alpha, beta,
                out: torch.Tensor, *, ckpt_pos: Optional[torch.Tensor] = None, ckpt: Optional[torch.Tensor] = None,
                dev_err: Optional[torch.Tensor] = None, tile_w: int = 0, raw_inputs: bool = False,
                stream=None) -> None:
    """Whole prompts in one pass with an in-pass checkpoint. Token arrays are [n_tok, H, .];
    row b owns tokens [cu[b], cu[b+1]); ckpt_pos int32 [B], ckpt float32 [B, H, dv, dk].
    out is float32 or bf16; raw_inputs as for kda_decode_step."""
    ns, stride, H, dv, dk = _cache(cache)
    _dev(slot_ids, "slot_ids", (torch.int32,), 1)
    _dev(cu_seqlens, "cu_seqlens", (torch.int32,), 1)
    B = slot_ids.shape[0]
    _shape(cu_seqlens, "cu_seqlens", (B + 1,))
    for name, t, d in (("q", q, _BF16_TYPES), ("k", k, _BF16_TYPES), ("v", v, _BF16_TYPES),
                       ("alpha", alpha, (torch.float32,)), ("beta", beta, (torch.float32,)),
                       ("out", out, (torch.float32,) + _BF16_TYPES)):
        _dev(t, name, d)
    n_tok = k.shape[0]
    for name, t, shape in (("q", q, (n_tok, H, dk)), ("k", k, (n_tok, H, dk)), ("v", v, (n_tok, H, dv)),
                           ("alpha", alpha, (n_tok, H, dk)), ("beta", beta, (n_tok, H)),
                           ("out", out, (n_tok, H, dv))):
        _shape(t, name, shape)
    if ckpt_pos is not None:
        _dev(ckpt_pos, "ckpt_pos", (torch.int32,), 1)
        _shape(ckpt_pos, "ckpt_pos", (B,))
        if ckpt is None:
            raise ValueError("ckpt_pos needs a ckpt buffer")
    if ckpt is not None:
        _dev(ckpt, "ckpt", (torch.float32,))
        _shape(ckpt, "ckpt", (B, H, dv, dk))
    if dev_err is not None:
        _dev(dev_err, "dev_err", (torch.int32,))
    rc = load_library().kda_prefill(
        cache.data_ptr(), ns, stride, slot_ids.data_ptr(), cu_seqlens.data_ptr(), B, n_tok, H, dk, dv,
        q.data_ptr(), k.data_ptr(), v.data_ptr(), alpha.data_ptr(), beta.data_ptr(), out.data_ptr(),
        _ptr(ckpt_pos), _ptr(ckpt), _ptr(dev_err), _ref(_opts(tile_w, 0, _flags(raw_inputs, out))),
        _stream(stream))
    if rc != KDA_OK:
        raise KdaError(rc, "kda_prefill")


def kda_prefill_chunked_workspace(B: int, n_tok: int, H: int, dk: int, dv: int) -> int:
    """Workspace bytes kda_prefill_chunked needs for these sizes."""
    n = ctypes.c_size_t(0)
    rc = load_library().kda_prefill_chunked_workspace(B, n_tok, H, dk, dv, ctypes.byref(n))
    if rc != KDA_OK:
        raise KdaError(rc, "kda_prefill_chunked_workspace")
    return n.value


def _prefill_chunked_checks(cache, slot_ids, cu_seqlens, q, k, v, alpha, beta, out, ckpt_pos, ckpt, dev_err):
    """Shape and dtype checks shared by both chunk-prefill calls; returns (B, n_tok, H, dk, dv, ns, stride)."""
    ns, stride, H, dv, dk = _cache(cache)
    _dev(slot_ids, "slot_ids", (torch.int32,), 1)
    _dev(cu_seqlens, "cu_seqlens", (torch.int32,), 1)
    B = slot_ids.shape[0]
    _shape(cu_seqlens, "cu_seqlens", (B + 1,))
    for name, t, d in (("q", q, _BF16_TYPES), ("k", k, _BF16_TYPES), ("v", v, _BF16_TYPES),
                       ("alpha", alpha, (torch.float32,)), ("beta", beta, (torch.float32,)),
                       ("out", out, (torch.float32,) + _BF16_TYPES)):
        _dev(t, name, d)
    n_tok = k.shape[0]
    for name, t, shape in (("q", q, (n_tok, H, dk)), ("k", k, (n_tok, H, dk)), ("v", v, (n_tok, H, dv)),
                           ("alpha", alpha, (n_tok, H, dk)), ("beta", beta, (n_tok, H)),
                           ("out", out, (n_tok, H, dv))):
        _shape(t, name, shape)
    if ckpt_pos is not None:
        _dev(ckpt_pos, "ckpt_pos", (torch.int32,), 1)
        _shape(ckpt_pos, "ckpt_pos", (B,))
        if ckpt is None:
            raise ValueError("ckpt_pos needs a ckpt buffer")
    if ckpt is not None:
        _dev(ckpt, "ckpt", (torch.float32,))
        _shape(ckpt, "ckpt", (B, H, dv, dk))
    if dev_err is not None:
        _dev(dev_err, "dev_err", (torch.int32,))
    return B, n_tok, H, dk, dv, ns, stride


def kda_prefill_chunked(cache: torch.Tensor, slot_ids: torch.Tensor, cu_seqlens: torch.Tensor, q, k, v, alpha,
                        beta, out: torch.Tensor, *, ckpt_pos: Optional[torch.Tensor] = None,
                        ckpt: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                        dev_err: Optional[torch.Tensor] = None, tile_w: int = 0, raw_inputs: bool = False,
                        stream=None) -> None:
    """Chunk form of kda_prefill: same arguments plus a device workspace (any dtype, at least
    kda_prefill_chunked_workspace() bytes); None allocates one for the call."""
    B, n_tok, H, dk, dv, ns, stride = _prefill_chunked_checks(cache, slot_ids, cu_seqlens, q, k, v, alpha, beta,
                                                              out, ckpt_pos, ckpt, dev_err)
    if workspace is None:
        workspace = torch.empty(kda_prefill_chunked_workspace(B, n_tok, H, dk, dv), dtype=torch.uint8,
                                device=cache.device)
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    rc = load_library().kda_prefill_chunked(
        cache.data_ptr(), ns, stride, slot_ids.data_ptr(), cu_seqlens.data_ptr(), B, n_tok, H, dk, dv,
        q.data_ptr(), k.data_ptr(), v.data_ptr(), alpha.data_ptr(), beta.data_ptr(), out.data_ptr(),
        _ptr(ckpt_pos), _ptr(ckpt), workspace.data_ptr(), workspace.numel() * workspace.element_size(),
        _ptr(dev_err), _ref(_opts(tile_w, 0, _flags(raw_inputs, out))), _stream(stream))
    if rc != KDA_OK:
        raise KdaError(rc, "kda_prefill_chunked")


def kda_prefill_chunked_noalloc(cache: torch.Tensor, slot_ids: torch.Tensor, cu_seqlens: torch.Tensor, q, k, v,
                                alpha, beta, out: torch.Tensor, *, ckpt_pos: Optional[torch.Tensor] = None,
                                ckpt: Optional[torch.Tensor] = None, dev_err: Optional[torch.Tensor] = None,
                                tile_w: int = 0, raw_inputs: bool = False, stream=None) -> None:
    """kda_prefill_chunked on the library's static per-GPU workspace: nothing is allocated
    (KdaError KDA_ERR_TOO_LARGE past KDA_NOALLOC_SCRATCH_BYTES). Calls that overlap on one GPU race."""
    B, n_tok, H, dk, dv, ns, stride = _prefill_chunked_checks(cache, slot_ids, cu_seqlens, q, k, v, alpha, beta,
                                                              out, ckpt_pos, ckpt, dev_err)
    rc = load_library().kda_prefill_chunked_noalloc(
        cache.data_ptr(), ns, stride, slot_ids.data_ptr(), cu_seqlens.data_ptr(), B, n_tok, H, dk, dv,
        q.data_ptr(), k.data_ptr(), v.data_ptr(), alpha.data_ptr(), beta.data_ptr(), out.data_ptr(),
        _ptr(ckpt_pos), _ptr(ckpt), _ptr(dev_err), _ref(_opts(tile_w, 0, _flags(raw_inputs, out))),
        _stream(stream))
    if rc != KDA_OK:
        raise KdaError(rc, "kda_prefill_chunked_noalloc")


def _state_copy(name, cache, slot_ids, buf, heads, cols, dev_err, stream):
    ns, stride, H, dv, dk = _cache(cache)
    _dev(slot_ids, "slot_ids", (torch.int32,), 1)
    B = slot_ids.shape[0]
    head0, nheads = (0, H) if heads is None else (int(heads[0]), int(heads[1]) - int(heads[0]))
    col0, ncols = (0, dv) if cols is None else (int(cols[0]), int(cols[1]) - int(cols[0]))
    if not isinstance(buf, torch.Tensor) or buf.dtype != torch.float32 or not buf.is_contiguous():
        raise TypeError("buf must be a contiguous float32 tensor")
    if buf.device.type != "cuda" and not buf.is_pinned():
        raise ValueError("buf must be on the GPU or in pinned host memory")
    _shape(buf, "buf", (B, nheads, ncols, dk))
    if dev_err is not None:
        _dev(dev_err, "dev_err", (torch.int32,))
    rc = getattr(load_library(), name)(cache.data_ptr(), ns, stride, slot_ids.data_ptr(), B, H, dk, dv, head0,
                                       nheads, col0, ncols, buf.data_ptr(), _ptr(dev_err), _stream(stream))
    if rc != KDA_OK:
        raise KdaError(rc, name)


def kda_state_pack(cache: torch.Tensor, slot_ids: torch.Tensor, buf: torch.Tensor, *, heads=None, cols=None,
                   dev_err: Optional[torch.Tensor] = None, stream=None) -> None:
    """buf[b] <- heads [h0, h1) x value columns [c0, c1) of slot slot_ids[b]; buf float32
    [B, h1 - h0, c1 - c0, dk] on the GPU or in pinned host memory."""
    _state_copy("kda_state_pack", cache, slot_ids, buf, heads, cols, dev_err, stream)


def kda_state_unpack(cache: torch.Tensor, slot_ids: torch.Tensor, buf: torch.Tensor, *, heads=None, cols=None,
                     dev_err: Optional[torch.Tensor] = None, stream=None) -> None:
    """The inverse of kda_state_pack: slots <- buf."""
    _state_copy("kda_state_unpack", cache, slot_ids, buf, heads, cols, dev_err, stream)
