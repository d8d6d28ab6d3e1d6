/*
 * kda.h - C ABI of the KDA recurrent-state library for MI355X (gfx950).
 *
 * The operation. Kimi K3's small-batch decode carries, per layer and per
 * attention head, a KDA recurrent state held in an FP32 SSM cache ("Kimi K3
 * vLLM optimization: NVIDIA decode speed-up 1.68x", section "What the upstream
 * tests actually show"; "Kimi K3 performance optimization in vLLM", opening
 * paragraph). The pages do not write the update out; this library takes KDA to
 * be the gated delta rule with per-channel decay. Per head, with the state S a
 * dk x dv matrix (row i = key channel, column j = value channel), one token
 * applies
 *     S <- Diag(alpha) S ;   S <- S + beta k (v - S^T k)^T ;   o = S^T q .
 * Speculative verify and commit follow ReplaySSM ("Kimi K3 performance
 * optimization in vLLM", section "ReplaySSM for state reconstruction"): the
 * draft tokens are evaluated without writing the committed state, their inputs
 * are buffered, and the commit rebuilds only the accepted state. Mixed batches
 * are packed contiguously and outputs are written straight to each row's
 * offset (same page, section "Zero-copy mixed KDA batching"). The launch shape
 * is chosen from the batch size and the per-GPU head count ("Hyper Optimizing
 * Kimi K3 in vLLM", section "Finding time between operators").
 *
 * Layouts. All arrays are contiguous, row-major, in device memory unless
 * marked "host". bf16 arrays hold raw bfloat16 bit patterns (uint16_t).
 *   cache   float  slot s at cache + s * slot_stride, laid out [H][dv][dk]:
 *                  element (i, j) of head h is cache[s*slot_stride + (h*dv + j)*dk + i]
 *                  (each value column's dk key channels are contiguous)
 *   q, k    bf16   [rows][H][dk]   (q is used as given: any 1/sqrt(dk) scale is the caller's)
 *   v       bf16   [rows][H][dv]
 *   alpha   float  [rows][H][dk]   decay per key channel
 *   beta    float  [rows][H]       write strength per head
 *   out     float  [rows][H][dv]  (bf16 with KDA_OUT_BF16)
 * where rows is B for kda_decode_step and n_tok for kda_verify_chunk.
 *
 * Supported shapes: dk, dv in {64, 128}; 1 <= T_max <= 16.
 *
 * Ownership and ordering. The caller allocates and frees every buffer. The
 * library allocates no device memory, keeps no state between calls and never
 * synchronizes: each call validates its arguments on the host, enqueues its
 * kernels on `stream` (a hipStream_t; NULL = the null stream) and returns.
 * Buffers must stay valid until the stream has passed the call. Calls are
 * reentrant. Within one call, slot ids must be distinct (KDA_CHECK_SLOTS checks
 * it on the host), and no output buffer may overlap an input or another output.
 *
 * Rows and slots. slot_ids[b] < 0 marks a padding row: its state is neither
 * read nor written and its output rows keep their contents (its inputs may
 * still be read). A slot id >= num_slots is a device-side error (below).
 *
 * Errors. Every entry point returns KDA_OK or a negative KDA_ERR_* code. The
 * host checks run before anything is enqueued; on an error nothing is
 * enqueued. Device-side errors are OR-ed into *dev_err (optional, int32 in
 * device memory, which the caller zeroes) and the offending row is skipped in
 * full while the other rows proceed:
 *   KDA_DEVERR_SLOT      slot id >= num_slots
 *   KDA_DEVERR_SEQLEN    row b's token range [cu[b], cu[b+1]) is decreasing, leaves
 *                        [0, n_tok] or is longer than T_max
 *   KDA_DEVERR_ACCEPTED  accepted_len[b] outside [0, T_b]
 *   KDA_DEVERR_CKPT      kda_prefill: checkpoint position past the row
 * The library never falls back to another path: an unsupported shape is
 * reported (KDA_ERR_UNSUPPORTED) and left to the caller.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum kda_status {
    KDA_OK = 0,
    KDA_ERR_INVALID = -1,     /* null required pointer, negative size, bad mode, unknown option flag,
                                 slot_stride too small */
    KDA_ERR_UNSUPPORTED = -2, /* dk or dv not in {64, 128}, T_max outside [1, 16], illegal tile width,
                                 grid too large */
    KDA_ERR_ALIGN = -3,       /* cache / alpha / draft / replay alpha not 16-byte aligned, slot_stride
                                 not a multiple of 4, bf16 input arrays not 8-byte aligned, out / beta
                                 not 4-byte aligned (bf16 out: 2-byte) */
    KDA_ERR_HIP = -4,         /* the HIP runtime rejected a launch */
    KDA_ERR_TOO_LARGE = -5    /* kda_prefill_chunked_noalloc: the call needs more workspace than
                                 KDA_NOALLOC_SCRATCH_BYTES */
};

enum kda_mode { KDA_REPLAY = 0, KDA_PER_POSITION = 1 };

enum kda_device_error {
    KDA_DEVERR_SLOT = 1,
    KDA_DEVERR_SEQLEN = 2,
    KDA_DEVERR_ACCEPTED = 4,
    KDA_DEVERR_CKPT = 8 /* kda_prefill: ckpt_pos[b] > T_b */
};

/* Operations, for kda_query_variant. */
enum kda_op {
    KDA_OP_DECODE = 0,        /* kda_decode_step */
    KDA_OP_VERIFY = 1,        /* kda_verify_chunk */
    KDA_OP_COMMIT_REPLAY = 2, /* kda_replay_commit, mode KDA_REPLAY */
    KDA_OP_COMMIT_COPY = 3,   /* kda_replay_commit, mode KDA_PER_POSITION */
    KDA_OP_PREFILL = 4        /* kda_prefill */
};

/* Output gate fused into the read-out, per (token, head) over the whole value
 * vector: y = o / sqrt(mean_j o_j^2 + eps) * weight * sigmoid(gate). It is the
 * gating fused at the output of "Hyper Optimizing Kimi K3 in vLLM", section
 * "Finding time between operators". Host struct; pointers are device memory. */
typedef struct kda_epilogue {
    const uint16_t *gate; /* bf16 [rows][H][dv], required */
    const float *weight;  /* [dv], or NULL for all ones */
    float eps;            /* >= 0 */
} kda_epilogue;

/* ReplaySSM input buffer, indexed by batch row b and draft position t.
 * Host struct; pointers are device memory. The caller keeps the batch order
 * between kda_verify_chunk and kda_replay_commit. */
typedef struct kda_replay_buf {
    uint16_t *k;  /* bf16 [B][T_max][H][dk] */
    uint16_t *v;  /* bf16 [B][T_max][H][dv] */
    float *alpha; /* [B][T_max][H][dk] */
    float *beta;  /* [B][T_max][H] */
} kda_replay_buf;

/* How kda_verify_chunk computes its outputs.
 *   KDA_VERIFY_RECURRENT: token by token on the state, the same arithmetic as
 *     kda_decode_step (outputs bit-identical to successive decode steps).
 *   KDA_VERIFY_CHUNKED: the chunk form of the same recurrence. Decays are
 *     accumulated per key channel, the state products (decayed keys and queries
 *     times the committed state) run on MFMA, and the coupling between the
 *     chunk's tokens is a small triangular solve. It needs no state until the
 *     commit, so it serves KDA_REPLAY rows that are not updated in place and
 *     have no output gate. Outputs agree with the recurrent form to rounding;
 *     replay buffers and committed states are identical.
 *   KDA_VERIFY_AUTO: the faster form on MI355X: the chunk form where it applies,
 *     with tile_w = 0 and either T_max >= 7 and B * H >= 128 or T_max >= 5 and
 *     B * H >= 256; the recurrent form otherwise (fewer tokens or (row, head)
 *     groups leave the chunk form's per-group latency exposed). */
enum kda_verify_form { KDA_VERIFY_AUTO = 0, KDA_VERIFY_RECURRENT = 1, KDA_VERIFY_CHUNKED = 2 };

/* Option flags (kda_options.flags, OR-ed).
 *   KDA_RAW_INPUTS: q, k, alpha and beta hold the raw projections (same types and
 *     layouts) and every token is prepared in the kernel before the recurrence, the
 *     normalization and gate activations that otherwise run as separate small
 *     kernels ("Hyper Optimizing Kimi K3 in vLLM", section "Finding time between
 *     operators"):
 *         k <- k / sqrt(sum_i k_i^2 + 1e-12)
 *         q <- q / sqrt(sum_i q_i^2 + 1e-12) / sqrt(dk)
 *         alpha_i <- exp(-softplus(alpha_i)) = 1 / (1 + exp(alpha_i))
 *         beta <- sigmoid(beta) = 1 / (1 + exp(-beta))
 *     in fp32 with the hardware exp2, reciprocal and reciprocal square root. Every
 *     op prepares the same way, so states stay bit-identical across decode,
 *     verify, commit and prefill. Replay buffers hold the raw inputs, and
 *     kda_replay_commit in KDA_REPLAY mode must get the flag when the verify did.
 *   KDA_OUT_BF16: out is bf16 [rows][H][dv] (2-byte aligned), each output rounded
 *     to nearest even from the fp32 value the call computes otherwise.
 *   KDA_CHECK_SLOTS: a debug check of the rule that slot ids are distinct within
 *     one call. slot_ids must then be host-readable memory that the device can
 *     also read (pinned host memory, hipHostMalloc): before anything is
 *     enqueued the library reads it on the host and returns KDA_ERR_INVALID if
 *     two rows name the same slot (padding rows, < 0, are exempt). The check
 *     takes O(B^2) host time and allocates nothing. Any entry point that takes
 *     kda_options accepts it.
 * kda_replay_commit ignores KDA_OUT_BF16 (it has no output) and, in
 * KDA_PER_POSITION mode, KDA_RAW_INPUTS. The chunk form of verify takes neither
 * KDA_RAW_INPUTS nor KDA_OUT_BF16 (KDA_ERR_UNSUPPORTED). Other bits are
 * KDA_ERR_INVALID. */
enum kda_flag { KDA_RAW_INPUTS = 1, KDA_OUT_BF16 = 2, KDA_CHECK_SLOTS = 4 };

/* Launch options (host struct, may be NULL = all zero). */
typedef struct kda_options {
    int32_t tile_w;      /* value columns per workgroup of the recurrent kernels: 0 = chosen from
                            (B, H); otherwise one of 4, 8, 16, 32, 64, 128 with tile_w <= dv (and
                            tile_w == dv with the gate), or 2 for kda_decode_step at dk = 128
                            without the gate (column pairs). Results are bit-identical for every
                            legal width. */
    int32_t verify_form; /* a kda_verify_form; KDA_VERIFY_CHUNKED where it does not apply is
                            KDA_ERR_UNSUPPORTED */
    int32_t flags;       /* kda_flag bits */
} kda_options;

/*
 * Single-token decode step for B rows. Row b reads token b of q, k, v, alpha,
 * beta, updates the state of slot slot_ids[b] in place (all H heads) and
 * writes out[b] (the gated y when epi != NULL).
 */
int kda_decode_step(float *cache, int64_t num_slots, int64_t slot_stride,
                    const int32_t *slot_ids, int32_t B, int32_t H, int32_t dk, int32_t dv,
                    const uint16_t *q, const uint16_t *k, const uint16_t *v,
                    const float *alpha, const float *beta, void *out,
                    const kda_epilogue *epi, int32_t *dev_err,
                    const kda_options *opts, void *stream);

/*
 * Speculative verify over a packed chunk ("ReplaySSM for state
 * reconstruction"; "Zero-copy mixed KDA batching"). Row b owns tokens
 * [cu_seqlens[b], cu_seqlens[b+1]) of the packed [n_tok] arrays; its T_b tokens
 * run in order from the slot's committed state and out[cu_seqlens[b] + t] gets
 * token t's read-out. The committed slot is not written, except that rows with
 * T_b == 1 are updated in place when t1_inplace != 0 (the non-speculative
 * members of a mixed batch).
 *   mode KDA_REPLAY:       token t's k, v, alpha, beta are copied bit for bit to
 *                          rb at [b][t] (rb required, draft ignored)
 *   mode KDA_PER_POSITION: the state after token t is written to draft at [b][t],
 *                          float [B][T_max][H][dv][dk] (draft required, rb ignored)
 * In-place rows write neither. Positions t >= T_b are left untouched. With
 * B == 0 or n_tok == 0 nothing is enqueued.
 */
int kda_verify_chunk(float *cache, int64_t num_slots, int64_t slot_stride,
                     const int32_t *slot_ids, const int32_t *cu_seqlens,
                     int32_t B, int32_t T_max, int32_t n_tok, int32_t H, int32_t dk, int32_t dv,
                     const uint16_t *q, const uint16_t *k, const uint16_t *v,
                     const float *alpha, const float *beta, void *out,
                     const kda_epilogue *epi, int32_t mode, int32_t t1_inplace,
                     const kda_replay_buf *rb, float *draft, int32_t *dev_err,
                     const kda_options *opts, void *stream);

/*
 * Commit the accepted prefix ("ReplaySSM for state reconstruction"): the slot
 * of row b becomes the state after the first accepted_len[b] tokens of the
 * chunk that kda_verify_chunk evaluated for row b. accepted_len[b] == 0 leaves
 * the slot unchanged (use it for rows already updated in place).
 *   mode KDA_REPLAY:       reload the slot, replay the buffered inputs of rb, store once
 *   mode KDA_PER_POSITION: copy draft[b][accepted_len[b] - 1] into the slot
 * Both modes leave bit-identical slots, equal bit for bit to accepted_len[b]
 * successive kda_decode_step calls. cu_seqlens bounds accepted_len by each
 * row's token count T_b (a bad range sets KDA_DEVERR_SEQLEN, as in verify). It
 * may be NULL: then T_b = T_max for every row and n_tok is not used.
 */
int kda_replay_commit(float *cache, int64_t num_slots, int64_t slot_stride,
                      const int32_t *slot_ids, const int32_t *cu_seqlens,
                      const int32_t *accepted_len, int32_t B, int32_t T_max, int32_t n_tok,
                      int32_t H, int32_t dk, int32_t dv, int32_t mode,
                      const kda_replay_buf *rb, const float *draft, int32_t *dev_err,
                      const kda_options *opts, void *stream);

/*
 * Prefill with an in-pass checkpoint ("Kimi K3 performance optimization in
 * vLLM", section "Internal KDA prefix checkpoint": one pass over the whole
 * prompt that also exports the state at an earlier token). Row b runs its
 * prompt, tokens [cu_seqlens[b], cu_seqlens[b+1]) of the packed [n_tok] arrays
 * (any length), from the state in slot slot_ids[b] (zero it for a fresh
 * prompt, or copy a checkpoint into it to resume); out[cu_seqlens[b] + t] gets
 * token t's read-out and the final state is written back to the slot. With
 * ckpt_pos (int32 [B], may be NULL), the state after the first ckpt_pos[b]
 * tokens (0 = before the prompt, < 0 = none) is written to ckpt
 * (float [B][H][dv][dk]) during the same pass; ckpt_pos[b] > T_b sets
 * KDA_DEVERR_CKPT and skips the row. The states match that many
 * kda_decode_step calls bit for bit; outputs agree to rounding (the read-out
 * is taken on the decayed state plus (k . q) delta). kda_options.tile_w may be
 * 16 or 32. With B == 0, or n_tok == 0 and no ckpt_pos, nothing is enqueued.
 */
int kda_prefill(float *cache, int64_t num_slots, int64_t slot_stride,
                const int32_t *slot_ids, const int32_t *cu_seqlens,
                int32_t B, int32_t n_tok, int32_t H, int32_t dk, int32_t dv,
                const uint16_t *q, const uint16_t *k, const uint16_t *v,
                const float *alpha, const float *beta, void *out,
                const int32_t *ckpt_pos, float *ckpt, int32_t *dev_err,
                const kda_options *opts, void *stream);

/*
 * Chunk form of kda_prefill (the same call plus a workspace): each row's prompt
 * is cut into chunks of 32 tokens (first at ckpt_pos[b] when it falls strictly
 * inside the row, so the checkpoint lies on a chunk boundary). A first kernel
 * prepares every (chunk, head) in parallel: the decay products inside the
 * chunk, the lower-triangular system of the delta rule solved once per chunk,
 * and the matrices that turn the chunk's effect on the state into dense
 * products. A second kernel runs each (row, head, 16 value columns) through its
 * chunks in order with those products on MFMA. The state is fp32 throughout,
 * but its products with the chunk matrices are taken on the bfloat16 matrix
 * cores as three products of split fp32 operands (hi = RNE(x), lo = RNE(x -
 * hi)), each within about 1.2e-5 of |a||b|: outputs stay within 1e-4 relative
 * L2 per (token, head) of the exact recurrence and states far within 1e-3
 * relative Frobenius, where kda_prefill's products are fp32. Outputs and states
 * therefore agree with kda_prefill to that accuracy (not bit for bit).
 * Arguments, layouts, flags and
 * device errors are kda_prefill's; kda_options.tile_w may be 0 or 16.
 * workspace: device memory of at least kda_prefill_chunked_workspace() bytes,
 * 16-byte aligned, owned by the caller; its contents need no initialization
 * and are dead when the stream has passed the call. A smaller workspace is
 * KDA_ERR_INVALID.
 */
int kda_prefill_chunked(float *cache, int64_t num_slots, int64_t slot_stride,
                        const int32_t *slot_ids, const int32_t *cu_seqlens,
                        int32_t B, int32_t n_tok, int32_t H, int32_t dk, int32_t dv,
                        const uint16_t *q, const uint16_t *k, const uint16_t *v,
                        const float *alpha, const float *beta, void *out,
                        const int32_t *ckpt_pos, float *ckpt,
                        void *workspace, size_t workspace_bytes, int32_t *dev_err,
                        const kda_options *opts, void *stream);

/* Host only. Workspace bytes kda_prefill_chunked needs for these sizes
 * (written to *bytes): about 2.1 KB per (token, head) at dk = dv = 128. */
int kda_prefill_chunked_workspace(int32_t B, int32_t n_tok, int32_t H, int32_t dk, int32_t dv,
                                  size_t *bytes);

/*
 * kda_prefill_chunked without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). The workspace is a static device array of
 * KDA_NOALLOC_SCRATCH_BYTES owned by the library: each GPU the library runs on
 * holds its own copy until the process ends, and the call allocates nothing.
 * Arguments, layouts, flags, results and device errors are kda_prefill_chunked's.
 * A call whose kda_prefill_chunked_workspace() size exceeds
 * KDA_NOALLOC_SCRATCH_BYTES returns KDA_ERR_TOO_LARGE and enqueues nothing (at
 * H = 32, dk = dv = 128 and B = 1 the limit is a prompt of about 3,700 tokens).
 * Every call on one GPU uses that GPU's one array: calls that can overlap on
 * one GPU (other streams, other host threads) race and must be serialized by
 * the caller. The array keeps the last call's contents; nothing in it needs to
 * start at zero. The first call on each device looks the array's device
 * address up (hipGetSymbolAddress) with that device current.
 */
#define KDA_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)

int kda_prefill_chunked_noalloc(float *cache, int64_t num_slots, int64_t slot_stride,
                                const int32_t *slot_ids, const int32_t *cu_seqlens,
                                int32_t B, int32_t n_tok, int32_t H, int32_t dk, int32_t dv,
                                const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                const float *alpha, const float *beta, void *out,
                                const int32_t *ckpt_pos, float *ckpt, int32_t *dev_err,
                                const kda_options *opts, void *stream);

/*
 * State transfer for prefill/decode disaggregation and offload ("Kimi K3
 * performance optimization in vLLM", section "Prefill/Decode disaggregation
 * and hybrid state offload": the KDA state is split by head and by dimension,
 * and boundary states are stored outside the GPU). For every row b with
 * slot_ids[b] >= 0, kda_state_pack copies heads [head0, head0 + nheads) and
 * value columns [col0, col0 + ncols) of slot slot_ids[b] to
 * buf[b][nheads][ncols][dk] (float, contiguous), and kda_state_unpack copies
 * them back. Bit-exact copies. buf is device memory or pinned host memory
 * mapped for the device (hipHostMalloc); the kernel reads or writes it
 * directly. Padding rows (slot < 0) leave their part of buf (pack) or the
 * cache (unpack) untouched; slot >= num_slots sets KDA_DEVERR_SLOT. Ranges
 * outside [0, H) or [0, dv) are KDA_ERR_INVALID; an empty range enqueues
 * nothing.
 */
int kda_state_pack(const float *cache, int64_t num_slots, int64_t slot_stride,
                   const int32_t *slot_ids, int32_t B, int32_t H, int32_t dk, int32_t dv,
                   int32_t head0, int32_t nheads, int32_t col0, int32_t ncols,
                   float *buf, int32_t *dev_err, void *stream);

int kda_state_unpack(float *cache, int64_t num_slots, int64_t slot_stride,
                     const int32_t *slot_ids, int32_t B, int32_t H, int32_t dk, int32_t dv,
                     int32_t head0, int32_t nheads, int32_t col0, int32_t ncols,
                     const float *buf, int32_t *dev_err, void *stream);

/*
 * Host only. Reports the launch shape operation op (a kda_op) would use for
 * these sizes (tile_w value columns per workgroup, threads per workgroup),
 * chosen from the batch size and head count when requested_tile_w == 0 (the
 * scheduling by batch size and per-GPU head count of "Hyper Optimizing Kimi K3
 * in vLLM", section "Finding time between operators"). For KDA_OP_VERIFY it is
 * the shape of the recurrent form; where the automatic choice takes the chunk
 * form instead (see kda_verify_form), that kernel runs dv columns and 4 * dv
 * threads per workgroup. For KDA_OP_COMMIT_REPLAY it assumes full rows:
 * kda_replay_commit with cu_seqlens whose n_tok is under 3/4 of B * T_max
 * (rows mostly short or empty) runs one workgroup of dv columns per head
 * instead. Returns KDA_ERR_UNSUPPORTED for shapes the library
 * does not run, KDA_ERR_INVALID for an unknown op or non-positive sizes.
 */
int kda_query_variant(int32_t op, int32_t B, int32_t H, int32_t dk, int32_t dv, int32_t T_max,
                      int32_t epilogue, int32_t requested_tile_w,
                      int32_t *tile_w, int32_t *threads);

/* Host only. Static message text for a kda_status code. */
const char *kda_status_str(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
