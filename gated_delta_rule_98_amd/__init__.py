"""KDA fp32 recurrent-state decode, speculative verify and replay commit on MI355X.

The computation lives in hand-written HIP kernels for gfx950 behind the C ABI
of include/kda.h (libkda.so, built in this directory). This package is the thin
torch-facing binding of that library.
"""

from .kda import (  # noqa: F401
    KDA_CHECK_SLOTS,
    KDA_DEVERR_ACCEPTED,
    KDA_DEVERR_CKPT,
    KDA_DEVERR_SEQLEN,
    KDA_DEVERR_SLOT,
    KDA_ERR_ALIGN,
    KDA_ERR_HIP,
    KDA_ERR_INVALID,
    KDA_ERR_TOO_LARGE,
    KDA_ERR_UNSUPPORTED,
    KDA_OK,
    KDA_OP_COMMIT_COPY,
    KDA_OP_COMMIT_REPLAY,
    KDA_OP_DECODE,
    KDA_OP_PREFILL,
    KDA_OP_VERIFY,
    KDA_OUT_BF16,
    KDA_PER_POSITION,
    KDA_RAW_INPUTS,
    KDA_REPLAY,
    KDA_VERIFY_AUTO,
    KDA_VERIFY_CHUNKED,
    KDA_VERIFY_RECURRENT,
    KDA_NOALLOC_SCRATCH_BYTES,
    LIB_PATH,
    KdaError,
    kda_decode_step,
    kda_prefill,
    kda_prefill_chunked,
    kda_prefill_chunked_noalloc,
    kda_prefill_chunked_workspace,
    kda_query_variant,
    kda_replay_commit,
    kda_state_pack,
    kda_state_unpack,
    kda_status_str,
    kda_verify_chunk,
    load_library,
)
