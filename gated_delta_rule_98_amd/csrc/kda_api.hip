// kda_api.hip - the C ABI of include/kda.h: host-side argument checks, the
// launch shape from (B, H), and dispatch to the kernel tables of the kernel
// files. Every entry point validates on the host, then enqueues on the
// caller's stream; nothing here allocates or synchronizes.

#include <string.h>

#include <mutex>

#include "kda_chunk.h"
#include "kda_engine.h"

using namespace kda;

// Static scratch of kda_prefill_chunked_noalloc: the chunk-prefill workspace for
// callers that cannot allocate. Every GPU the library runs on holds its own copy
// until the process ends. Host code never uses this name as an address: the
// per-device address comes from hipGetSymbolAddress (scratch_for_current_device).
static __device__ __align__(256) float scratch[KDA_NOALLOC_SCRATCH_BYTES / sizeof(float)];

namespace {

enum Kind { KIND_DECODE, KIND_VERIFY, KIND_COMMIT_REPLAY, KIND_COMMIT_COPY, KIND_PREFILL };

struct Launch {
  int W, waves, C;  // C = 0: column pairs (decode_pair_kernel), one float4 per lane
};

// Legal tile widths and their (waves, slabs per lane). Two columns per
// workgroup is the column-pair layout of the single-token step at dk = 128.
bool launch_of_width(int W, Launch *l) {
  switch (W) {
    case 2: *l = {2, 1, 0}; return true;
    case 4: *l = {4, 1, 1}; return true;
    case 8: *l = {8, 2, 1}; return true;
    case 16: *l = {16, 4, 1}; return true;
    case 32: *l = {32, 4, 2}; return true;
    case 64: *l = {64, 4, 4}; return true;
    case 128: *l = {128, 4, 8}; return true;
  }
  return false;
}

bool dims_supported(int dk, int dv) { return (dk == 64 || dk == 128) && (dv == 64 || dv == 128); }

// Launch shape from the batch size and the per-GPU head count. Measured on
// MI355X with cold state (fp32, d = 128, H = 32):
//  * single-token step: the widest tile (64, 32 or 16 columns) that still gives
//    at least 256 workgroups, i.e. one per CU, so a small batch spreads its state
//    over the whole chip; once that would exceed 1024 workgroups the step is a
//    pure stream and one-wave workgroups sustain the highest rate: column pairs
//    at dk = 128, 4 columns at dk = 64 (one float4 of state per lane either way);
//    at exactly 512 heads of 128 columns, 128-column tiles (two per CU);
//  * verify (T tokens per row, VALU-heavy): 32 columns while that gives at
//    least 256 workgroups, 16 below that, then 8;
//  * replay commit (accepted lengths uniform in 1..T): 32 columns at 512 to 767
//    heads (B = 16, T = 8: 12.6 us against 13.9 us for 16 columns), 16 columns
//    from 768 heads (B = 64, T = 8: 47.9 us against 49.4 us for 32) and below
//    512 heads while that gives 256 workgroups, then 8; a batch whose tokens
//    fill under 3/4 of B x T_max (rows mostly short or empty, as a mixed batch
//    whose single-token rows were committed in place) takes one workgroup per
//    head: fewer workgroups that only find nothing to do (the 64-row mixed
//    batch: 17.4 us against 19.7 us for 32 columns);
//  * per-position copy commit: 16 columns.
int choose_width(Kind kind, int64_t rows, int H, int dk, int dv, bool gate, int requested, Launch *l,
                 bool sparse_rows = false) {
  if (gate) {
    // the gate's RMS norm spans the whole head: one workgroup owns all dv columns,
    // with two slabs per lane (1024 threads at dv = 128) to keep registers low
    if (requested != 0 && requested != dv) return KDA_ERR_UNSUPPORTED;
    if (dv != 64 && dv != 128) return KDA_ERR_UNSUPPORTED;
    const int C = kind == KIND_DECODE ? kGateSlabsDecode : kGateSlabsVerify;
    *l = {dv, dv / (4 * C), C};
    return KDA_OK;
  }
  if (kind == KIND_PREFILL) {
    // 256-thread workgroups (the staging is spread over them): 16 or 32 columns
    const int W = requested != 0 ? requested : ((int64_t)rows * H * (dv / 16) > 2048 ? 32 : 16);
    if ((W != 16 && W != 32) || W > dv) return KDA_ERR_UNSUPPORTED;
    return launch_of_width(W, l) ? KDA_OK : KDA_ERR_UNSUPPORTED;
  }
  if (requested != 0) {
    if (requested > dv || dv % requested != 0 || !launch_of_width(requested, l)) return KDA_ERR_UNSUPPORTED;
    if (l->C == 0 && (kind != KIND_DECODE || dk != 128)) return KDA_ERR_UNSUPPORTED;
    return KDA_OK;
  }
  const int64_t heads = rows * H;
  int W = 16;
  switch (kind) {
    case KIND_DECODE:
      for (int cand : {64, 32, 16}) {
        if (cand <= dv && heads * (dv / cand) >= 256) {
          W = cand;
          break;
        }
      }
      if (heads * (dv / W) > 1024) W = dk == 128 ? 2 : 4;
      // exactly two 128-column workgroups per CU (512 on MI355X's 256 CUs): measured
      // 7-9% faster than 64 columns at H = 16, 32 and 64
      if (dv == 128 && heads == 512) W = 128;
      break;
    case KIND_VERIFY:
      W = 8;
      for (int cand : {32, 16}) {
        if (cand <= dv && heads * (dv / cand) >= 256) {
          W = cand;
          break;
        }
      }
      break;
    case KIND_COMMIT_REPLAY:
      W = 8;
      if (sparse_rows)
        W = dv;
      else if (heads >= 768)
        W = 16;
      else if (heads * (dv / 32) >= 2048)
        W = 32;
      else if (heads * (dv / 16) >= 256)
        W = 16;
      break;
    case KIND_COMMIT_COPY:
    case KIND_PREFILL:
      W = 16;
      break;
  }
  return launch_of_width(W, l) ? KDA_OK : KDA_ERR_UNSUPPORTED;
}

bool aligned(const void *p, uintptr_t n) { return ((uintptr_t)p % n) == 0; }

int launch_fn(const void *fn, int64_t blocks, int threads, size_t shmem, Args &a, void *stream) {
  if (!fn) return KDA_ERR_UNSUPPORTED;
  void *args[] = {&a};
  const hipError_t e = hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(threads), args, shmem,
                                       (hipStream_t)stream);
  return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

int launch(Kind kind, bool gate, int dk, const Launch &l, int64_t units, size_t shmem, Args &a,
           void *stream) {
  if (units > 0x7fffffff) return KDA_ERR_UNSUPPORTED;
  const int io = (a.raw ? kIoRaw : 0) | (a.out_bf16 ? kIoBf16 : 0);
  const void *fn = nullptr;
  switch (kind) {
    case KIND_DECODE:
      fn = l.C == 0 ? (dk == 128 && !gate ? decode_pair_kernel_for(io) : nullptr) : decode_kernel_for(dk, l.C, gate, io);
      break;
    case KIND_VERIFY: fn = verify_kernel_for(dk, l.C, gate, io, a.mode == KDA_PER_POSITION); break;
    case KIND_COMMIT_REPLAY:
      // staging before the state tile once the grid exceeds one round of resident
      // workgroups (8 per CU at these shapes, 2048 on MI355X's 256 CUs)
      fn = gate ? nullptr : commit_replay_kernel_for(dk, l.C, units > 2048);
      break;
    case KIND_COMMIT_COPY: fn = gate ? nullptr : commit_copy_kernel_for(dk, l.C); break;
    case KIND_PREFILL: fn = gate ? nullptr : prefill_kernel_for(dk, l.C, io); break;
  }
  return launch_fn(fn, units, 64 * l.waves, shmem, a, stream);
}

int check_cache(const float *cache, int64_t num_slots, int64_t slot_stride, int H, int dk, int dv) {
  if (!cache || num_slots < 0) return KDA_ERR_INVALID;
  if (slot_stride < (int64_t)H * dv * dk) return KDA_ERR_INVALID;
  if (!aligned(cache, 16) || slot_stride % 4 != 0) return KDA_ERR_ALIGN;
  return KDA_OK;
}

int check_inputs(const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *alpha,
                 const float *beta, const void *out, bool need_q, bool out_bf16) {
  if ((need_q && !q) || !k || !v || !alpha || !beta || (need_q && !out)) return KDA_ERR_INVALID;
  if ((q && !aligned(q, 8)) || !aligned(k, 8) || !aligned(v, 8) || !aligned(alpha, 16) ||
      !aligned(beta, 4) || (out && !aligned(out, out_bf16 ? 2 : 4)))
    return KDA_ERR_ALIGN;
  return KDA_OK;
}

// The option flags of a call: unknown bits are an error; `used` are the ones the
// op acts on (the others it accepts and ignores).
int read_flags(const kda_options *opts, int32_t used, Args &a) {
  const int32_t f = opts ? opts->flags : 0;
  if (f & ~(int32_t)(KDA_RAW_INPUTS | KDA_OUT_BF16 | KDA_CHECK_SLOTS)) return KDA_ERR_INVALID;
  a.raw = (f & used & KDA_RAW_INPUTS) ? 1 : 0;
  a.out_bf16 = (f & used & KDA_OUT_BF16) ? 1 : 0;
  return KDA_OK;
}

// KDA_CHECK_SLOTS: read the slot table on the host (the caller has put it in
// host-readable memory) and reject a batch in which two rows name the same
// slot. Quadratic in B and allocation-free; padding rows (< 0) are exempt.
int check_slots(const kda_options *opts, const int32_t *slot_ids, int32_t B) {
  if (!opts || !(opts->flags & KDA_CHECK_SLOTS)) return KDA_OK;
  for (int32_t i = 1; i < B; ++i) {
    const int32_t s = slot_ids[i];
    if (s < 0) continue;
    for (int32_t j = 0; j < i; ++j)
      if (slot_ids[j] == s) return KDA_ERR_INVALID;
  }
  return KDA_OK;
}

int check_gate(const kda_epilogue *epi) {
  if (!epi) return KDA_OK;
  if (!epi->gate || !(epi->eps >= 0.0f) || epi->eps > 3.0e38f) return KDA_ERR_INVALID;
  if (!aligned(epi->gate, 8) || (epi->weight && !aligned(epi->weight, 4))) return KDA_ERR_ALIGN;
  return KDA_OK;
}

int check_replay_buf(const kda_replay_buf *rb) {
  if (!rb || !rb->k || !rb->v || !rb->alpha || !rb->beta) return KDA_ERR_INVALID;
  if (!aligned(rb->k, 8) || !aligned(rb->v, 8) || !aligned(rb->alpha, 16) || !aligned(rb->beta, 4))
    return KDA_ERR_ALIGN;
  return KDA_OK;
}

#define KDA_TRY(expr)          \
  do {                         \
    const int rc_ = (expr);    \
    if (rc_ != KDA_OK) return rc_; \
  } while (0)

}  // namespace

// Device address of `scratch` on the current device, looked up once per device
// (with that device current) and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

int scratch_for_current_device(void **ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return KDA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return KDA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return KDA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return KDA_OK;
}

// Chunks the chunk form of prefill can meet: each row is cut at most once (at
// its checkpoint) and then into chunks, so at most ceil(n_tok / L) + 2 B.
int64_t prefill_chunk_bound(int64_t B, int64_t n_tok) {
  return (n_tok + kChunkTokens - 1) / kChunkTokens + 2 * B;
}

// Workspace of the chunk form: the per-(chunk, head) data, then the chunk map
// (int32 first chunk of each row [B + 1] and row of each chunk [chunks]),
// rounded up to 16 bytes.
size_t prefill_chunk_ws_data_bytes(int64_t B, int64_t n_tok, int H, int dk, int dv) {
  return (size_t)prefill_chunk_bound(B, n_tok) * (size_t)H * prefill_chunk_ws_floats(dk, dv) * sizeof(float);
}

size_t prefill_chunk_ws_bytes(int64_t B, int64_t n_tok, int H, int dk, int dv) {
  const size_t map = ((size_t)B + 1 + (size_t)prefill_chunk_bound(B, n_tok)) * sizeof(int32_t);
  return (prefill_chunk_ws_data_bytes(B, n_tok, H, dk, dv) + map + 15) / 16 * 16;
}

extern "C" {

int kda_prefill_chunked_workspace(int32_t B, int32_t n_tok, int32_t H, int32_t dk, int32_t dv, size_t *bytes) {
  if (!bytes || B < 0 || n_tok < 0 || H <= 0 || dk <= 0 || dv <= 0) return KDA_ERR_INVALID;
  if (!dims_supported(dk, dv)) return KDA_ERR_UNSUPPORTED;
  *bytes = prefill_chunk_ws_bytes(B, n_tok, H, dk, dv);
  return KDA_OK;
}

int kda_prefill_chunked(float *cache, int64_t num_slots, int64_t slot_stride, const int32_t *slot_ids,
                        const int32_t *cu_seqlens, int32_t B, int32_t n_tok, int32_t H, int32_t dk, int32_t dv,
                        const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *alpha,
                        const float *beta, void *out, const int32_t *ckpt_pos, float *ckpt, void *workspace,
                        size_t workspace_bytes, int32_t *dev_err, const kda_options *opts, void *stream) {
  Args f;
  memset(&f, 0, sizeof f);
  if (B < 0 || H <= 0 || dk <= 0 || dv <= 0 || n_tok < 0) return KDA_ERR_INVALID;
  KDA_TRY(read_flags(opts, KDA_RAW_INPUTS | KDA_OUT_BF16, f));
  if (!dims_supported(dk, dv)) return KDA_ERR_UNSUPPORTED;
  if (opts && opts->tile_w != 0 && opts->tile_w != 16) return KDA_ERR_UNSUPPORTED;
  if (B == 0 || (n_tok == 0 && !ckpt_pos)) return KDA_OK;
  if (!slot_ids || !cu_seqlens) return KDA_ERR_INVALID;
  KDA_TRY(check_slots(opts, slot_ids, B));
  KDA_TRY(check_cache(cache, num_slots, slot_stride, H, dk, dv));
  if (n_tok > 0) KDA_TRY(check_inputs(q, k, v, alpha, beta, out, true, f.out_bf16));
  if (ckpt_pos) {
    if (!ckpt) return KDA_ERR_INVALID;
    if (!aligned(ckpt, 16) || !aligned(ckpt_pos, 4)) return KDA_ERR_ALIGN;
  }
  if (!aligned(cu_seqlens, 4) || (dev_err && !aligned(dev_err, 4))) return KDA_ERR_ALIGN;
  const int64_t chunks = prefill_chunk_bound(B, n_tok);
  const size_t need = prefill_chunk_ws_bytes(B, n_tok, H, dk, dv);
  if (!workspace || workspace_bytes < need) return KDA_ERR_INVALID;
  if (!aligned(workspace, 16)) return KDA_ERR_ALIGN;
  const int64_t prep_blocks = chunks * H, state_blocks = (int64_t)B * H * (dv / 16);
  if (prep_blocks > 0x7fffffff || state_blocks > 0x7fffffff) return KDA_ERR_UNSUPPORTED;

  ChunkArgs a;
  memset(&a, 0, sizeof a);
  a.cache = cache;
  a.num_slots = num_slots;
  a.slot_stride = slot_stride;
  a.slot_ids = slot_ids;
  a.cu = cu_seqlens;
  a.ckpt_pos = ckpt_pos;
  a.q = q;
  a.k = k;
  a.v = v;
  a.alpha = alpha;
  a.beta = beta;
  a.out = static_cast<float *>(out);
  a.ckpt = ckpt;
  a.ws = static_cast<float *>(workspace);
  a.cbase = reinterpret_cast<int32_t *>(static_cast<char *>(workspace) +
                                        prefill_chunk_ws_data_bytes(B, n_tok, H, dk, dv));
  a.crow = a.cbase + B + 1;
  a.dev_err = dev_err;
  a.B = B;
  a.H = H;
  a.n_tok = n_tok;
  a.ws_chunks = (int32_t)chunks;
  a.ntile = dv / 16;
  a.raw = f.raw;
  a.out_bf16 = f.out_bf16;
  void *args[] = {&a};
  if (B > 1) {  // one row's chunks are numbered from 0 without the map
    const hipError_t e = hipLaunchKernel(prefill_chunk_map_kernel(), dim3(1), dim3(kChunkMapThreads), args, 0,
                                         (hipStream_t)stream);
    if (e != hipSuccess) return KDA_ERR_HIP;
  }
  if (n_tok > 0) {
    const hipError_t e = hipLaunchKernel(prefill_chunk_prep_kernel_for(dk, dv), dim3((unsigned)prep_blocks),
                                         dim3(kChunkPrepThreads), args, 0, (hipStream_t)stream);
    if (e != hipSuccess) return KDA_ERR_HIP;
  }
  const hipError_t e = hipLaunchKernel(prefill_chunk_state_kernel_for(dk, dv), dim3((unsigned)state_blocks),
                                       dim3(kChunkStateThreads), args, 0, (hipStream_t)stream);
  return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

int kda_prefill_chunked_noalloc(float *cache, int64_t num_slots, int64_t slot_stride, const int32_t *slot_ids,
                                const int32_t *cu_seqlens, int32_t B, int32_t n_tok, int32_t H, int32_t dk,
                                int32_t dv, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                const float *alpha, const float *beta, void *out, const int32_t *ckpt_pos,
                                float *ckpt, int32_t *dev_err, const kda_options *opts, void *stream) {
  size_t need = 0;
  KDA_TRY(kda_prefill_chunked_workspace(B, n_tok, H, dk, dv, &need));
  if (B == 0 || (n_tok == 0 && !ckpt_pos)) return KDA_OK;
  if (need > KDA_NOALLOC_SCRATCH_BYTES) return KDA_ERR_TOO_LARGE;
  if (!slot_ids || !cu_seqlens) return KDA_ERR_INVALID;
  KDA_TRY(check_slots(opts, slot_ids, B));
  void *ws = nullptr;
  KDA_TRY(scratch_for_current_device(&ws));
  return kda_prefill_chunked(cache, num_slots, slot_stride, slot_ids, cu_seqlens, B, n_tok, H, dk, dv, q, k, v,
                             alpha, beta, out, ckpt_pos, ckpt, ws, KDA_NOALLOC_SCRATCH_BYTES, dev_err, opts, stream);
}

int kda_prefill(float *cache, int64_t num_slots, int64_t slot_stride, const int32_t *slot_ids,
                const int32_t *cu_seqlens, int32_t B, int32_t n_tok, int32_t H, int32_t dk, int32_t dv,
                const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *alpha,
                const float *beta, void *out, const int32_t *ckpt_pos, float *ckpt, int32_t *dev_err,
                const kda_options *opts, void *stream) {
  Args a;
  memset(&a, 0, sizeof a);
  if (B < 0 || H <= 0 || dk <= 0 || dv <= 0 || n_tok < 0) return KDA_ERR_INVALID;
  KDA_TRY(read_flags(opts, KDA_RAW_INPUTS | KDA_OUT_BF16, a));
  if (!dims_supported(dk, dv)) return KDA_ERR_UNSUPPORTED;
  if (B == 0 || (n_tok == 0 && !ckpt_pos)) return KDA_OK;
  if (!slot_ids || !cu_seqlens) return KDA_ERR_INVALID;
  KDA_TRY(check_slots(opts, slot_ids, B));
  KDA_TRY(check_cache(cache, num_slots, slot_stride, H, dk, dv));
  if (n_tok > 0) KDA_TRY(check_inputs(q, k, v, alpha, beta, out, true, a.out_bf16));
  if (ckpt_pos) {
    if (!ckpt) return KDA_ERR_INVALID;
    if (!aligned(ckpt, 16) || !aligned(ckpt_pos, 4)) return KDA_ERR_ALIGN;
  }
  if (!aligned(cu_seqlens, 4) || (dev_err && !aligned(dev_err, 4))) return KDA_ERR_ALIGN;
  Launch l;
  KDA_TRY(choose_width(KIND_PREFILL, B, H, dk, dv, false, opts ? opts->tile_w : 0, &l));

  a.cache = cache;
  a.num_slots = num_slots;
  a.slot_stride = slot_stride;
  a.slot_ids = slot_ids;
  a.cu = cu_seqlens;
  a.q = q;
  a.k = k;
  a.v = v;
  a.alpha = alpha;
  a.beta = beta;
  a.out = static_cast<float *>(out);
  a.ckpt_pos = ckpt_pos;
  a.ckpt = ckpt;
  a.dev_err = dev_err;
  a.B = B;
  a.H = H;
  a.dv = dv;
  a.n_tok = n_tok;
  a.ntile = dv / l.W;
  const int64_t units = (int64_t)B * H * a.ntile;
  if (units > 0x7fffffff) return KDA_ERR_UNSUPPORTED;
  const int io = (a.raw ? kIoRaw : 0) | (a.out_bf16 ? kIoBf16 : 0);
  const void *fn = prefill_kernel_for(dk, l.C, io);
  return launch_fn(fn, units, 256, prefill_lds_bytes(dk, l.W), a, stream);
}

int kda_decode_step(float *cache, int64_t num_slots, int64_t slot_stride, const int32_t *slot_ids,
                    int32_t B, int32_t H, int32_t dk, int32_t dv, const uint16_t *q,
                    const uint16_t *k, const uint16_t *v, const float *alpha, const float *beta,
                    void *out, const kda_epilogue *epi, int32_t *dev_err,
                    const kda_options *opts, void *stream) {
  Args a;
  memset(&a, 0, sizeof a);
  if (B < 0 || H <= 0 || dk <= 0 || dv <= 0) return KDA_ERR_INVALID;
  KDA_TRY(read_flags(opts, KDA_RAW_INPUTS | KDA_OUT_BF16, a));
  if (!dims_supported(dk, dv)) return KDA_ERR_UNSUPPORTED;
  if (B == 0) return KDA_OK;
  if (!slot_ids) return KDA_ERR_INVALID;
  KDA_TRY(check_slots(opts, slot_ids, B));
  KDA_TRY(check_cache(cache, num_slots, slot_stride, H, dk, dv));
  KDA_TRY(check_inputs(q, k, v, alpha, beta, out, true, a.out_bf16));
  KDA_TRY(check_gate(epi));
  if (dev_err && !aligned(dev_err, 4)) return KDA_ERR_ALIGN;
  Launch l;
  KDA_TRY(choose_width(KIND_DECODE, B, H, dk, dv, epi != nullptr, opts ? opts->tile_w : 0, &l));

  a.cache = cache;
  a.num_slots = num_slots;
  a.slot_stride = slot_stride;
  a.slot_ids = slot_ids;
  a.q = q;
  a.k = k;
  a.v = v;
  a.alpha = alpha;
  a.beta = beta;
  a.out = static_cast<float *>(out);
  a.gate = epi ? epi->gate : nullptr;
  a.weight = epi ? epi->weight : nullptr;
  a.eps = epi ? epi->eps : 0.0f;
  a.dev_err = dev_err;
  a.B = B;
  a.H = H;
  a.dv = dv;
  a.T_max = 1;
  a.n_tok = B;
  a.ntile = dv / l.W;
  const int64_t units = (int64_t)B * H * a.ntile;
  if (units > 0x7fffffff) return KDA_ERR_UNSUPPORTED;
  return launch(KIND_DECODE, epi != nullptr, dk, l, units, 0, a, stream);
}

int kda_verify_chunk(float *cache, int64_t num_slots, int64_t slot_stride, const int32_t *slot_ids,
                     const int32_t *cu_seqlens, int32_t B, int32_t T_max, int32_t n_tok, int32_t H,
                     int32_t dk, int32_t dv, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                     const float *alpha, const float *beta, void *out, const kda_epilogue *epi,
                     int32_t mode, int32_t t1_inplace, const kda_replay_buf *rb, float *draft,
                     int32_t *dev_err, const kda_options *opts, void *stream) {
  Args a;
  memset(&a, 0, sizeof a);
  if (B < 0 || H <= 0 || dk <= 0 || dv <= 0 || n_tok < 0) return KDA_ERR_INVALID;
  if (mode != KDA_REPLAY && mode != KDA_PER_POSITION) return KDA_ERR_INVALID;
  KDA_TRY(read_flags(opts, KDA_RAW_INPUTS | KDA_OUT_BF16, a));
  if (!dims_supported(dk, dv) || T_max < 1 || T_max > kMaxT) return KDA_ERR_UNSUPPORTED;
  if (B == 0 || n_tok == 0) return KDA_OK;  // no tokens: nothing to read or write
  if (!slot_ids || !cu_seqlens) return KDA_ERR_INVALID;
  KDA_TRY(check_slots(opts, slot_ids, B));
  KDA_TRY(check_cache(cache, num_slots, slot_stride, H, dk, dv));
  KDA_TRY(check_inputs(q, k, v, alpha, beta, out, true, a.out_bf16));
  KDA_TRY(check_gate(epi));
  if (mode == KDA_REPLAY) KDA_TRY(check_replay_buf(rb));
  if (mode == KDA_PER_POSITION) {
    if (!draft) return KDA_ERR_INVALID;
    if (!aligned(draft, 16)) return KDA_ERR_ALIGN;
  }
  if (dev_err && !aligned(dev_err, 4)) return KDA_ERR_ALIGN;
  const int form = opts ? opts->verify_form : KDA_VERIFY_AUTO;
  if (form != KDA_VERIFY_AUTO && form != KDA_VERIFY_RECURRENT && form != KDA_VERIFY_CHUNKED)
    return KDA_ERR_INVALID;
  const bool chunk_fits = mode == KDA_REPLAY && !t1_inplace && epi == nullptr && !a.raw && !a.out_bf16;
  if (form == KDA_VERIFY_CHUNKED && (!chunk_fits || (opts && opts->tile_w != 0))) return KDA_ERR_UNSUPPORTED;
  // Automatic choice, from graph-timed runs on MI355X at H = 32, d = 128 with every row
  // holding T tokens (us, chunk / recurrent): the chunk form wins from 7 tokens at 128 or
  // more (row, head) groups (T = 8: B = 4 6.2 / 6.7, B = 16 11.1 / 15.5, B = 64 38.2 /
  // 48.6) and at 5 or 6 tokens from 256 groups (T = 6: B = 8 6.5 / 8.1, B = 64 37.1 /
  // 40.5); with fewer tokens or groups its per-group latency loses (T = 8, B = 2: 5.9 /
  // 5.1; T = 4, B = 64: 36.0 / 31.3; T = 2, B = 16: 9.7 / 8.0).
  const int64_t groups = (int64_t)B * H;
  const bool auto_chunk = (T_max >= 7 && groups >= 128) || (T_max >= 5 && groups >= 256);
  const bool chunked = form == KDA_VERIFY_CHUNKED ||
                       (form == KDA_VERIFY_AUTO && chunk_fits && (!opts || opts->tile_w == 0) && auto_chunk);
  Launch l;
  if (chunked) {
    l = {dv, dv / 16, 0};
  } else {
    KDA_TRY(choose_width(KIND_VERIFY, B, H, dk, dv, epi != nullptr, opts ? opts->tile_w : 0, &l));
  }

  a.cache = cache;
  a.num_slots = num_slots;
  a.slot_stride = slot_stride;
  a.slot_ids = slot_ids;
  a.cu = cu_seqlens;
  a.q = q;
  a.k = k;
  a.v = v;
  a.alpha = alpha;
  a.beta = beta;
  a.out = static_cast<float *>(out);
  a.gate = epi ? epi->gate : nullptr;
  a.weight = epi ? epi->weight : nullptr;
  a.eps = epi ? epi->eps : 0.0f;
  a.dev_err = dev_err;
  if (mode == KDA_REPLAY) {
    a.rk = rb->k;
    a.rv = rb->v;
    a.ralpha = rb->alpha;
    a.rbeta = rb->beta;
  } else {
    a.draft = draft;
  }
  a.B = B;
  a.H = H;
  a.dv = dv;
  a.T_max = T_max;
  a.n_tok = n_tok;
  a.ntile = dv / l.W;
  a.mode = mode;
  a.t1_inplace = t1_inplace ? 1 : 0;
  const int64_t units = (int64_t)B * H * a.ntile;
  if (chunked) {
    if (units > 0x7fffffff) return KDA_ERR_UNSUPPORTED;
    const void *fn = verify_chunk_kernel_for(dk, dv, T_max, units);
    return launch_fn(fn, units, 64 * l.waves, chunk_verify_lds_bytes(dk, dv, T_max), a, stream);
  }
  return launch(KIND_VERIFY, epi != nullptr, dk, l, units, staged_bytes(dk, T_max, l.W, epi != nullptr), a,
                stream);
}

int kda_replay_commit(float *cache, int64_t num_slots, int64_t slot_stride, const int32_t *slot_ids,
                      const int32_t *cu_seqlens, const int32_t *accepted_len, int32_t B,
                      int32_t T_max, int32_t n_tok, int32_t H, int32_t dk, int32_t dv, int32_t mode,
                      const kda_replay_buf *rb, const float *draft, int32_t *dev_err,
                      const kda_options *opts, void *stream) {
  Args a;
  memset(&a, 0, sizeof a);
  if (B < 0 || H <= 0 || dk <= 0 || dv <= 0 || n_tok < 0) return KDA_ERR_INVALID;
  if (mode != KDA_REPLAY && mode != KDA_PER_POSITION) return KDA_ERR_INVALID;
  KDA_TRY(read_flags(opts, mode == KDA_REPLAY ? KDA_RAW_INPUTS : 0, a));
  if (!dims_supported(dk, dv) || T_max < 1 || T_max > kMaxT) return KDA_ERR_UNSUPPORTED;
  if (B == 0) return KDA_OK;
  if (!slot_ids || !accepted_len) return KDA_ERR_INVALID;
  KDA_TRY(check_slots(opts, slot_ids, B));
  KDA_TRY(check_cache(cache, num_slots, slot_stride, H, dk, dv));
  if (mode == KDA_REPLAY) KDA_TRY(check_replay_buf(rb));
  if (mode == KDA_PER_POSITION) {
    if (!draft) return KDA_ERR_INVALID;
    if (!aligned(draft, 16)) return KDA_ERR_ALIGN;
  }
  if (!aligned(accepted_len, 4) || (cu_seqlens && !aligned(cu_seqlens, 4)) ||
      (dev_err && !aligned(dev_err, 4)))
    return KDA_ERR_ALIGN;
  Launch l;
  // rows mostly short or empty: the packed tokens fill under 3/4 of B x T_max
  const bool sparse_rows = cu_seqlens && 4 * (int64_t)n_tok < 3 * (int64_t)B * T_max;
  KDA_TRY(choose_width(mode == KDA_REPLAY ? KIND_COMMIT_REPLAY : KIND_COMMIT_COPY, B, H, dk, dv, false,
                       opts ? opts->tile_w : 0, &l, sparse_rows));

  a.cache = cache;
  a.num_slots = num_slots;
  a.slot_stride = slot_stride;
  a.slot_ids = slot_ids;
  a.cu = cu_seqlens;
  a.accepted = accepted_len;
  a.dev_err = dev_err;
  if (mode == KDA_REPLAY) {
    a.rk = rb->k;
    a.rv = rb->v;
    a.ralpha = rb->alpha;
    a.rbeta = rb->beta;
  } else {
    a.draft = const_cast<float *>(draft);
  }
  a.B = B;
  a.H = H;
  a.dv = dv;
  a.T_max = T_max;
  a.n_tok = n_tok;
  a.ntile = dv / l.W;
  a.mode = mode;
  if (mode == KDA_REPLAY) {
    return launch(KIND_COMMIT_REPLAY, false, dk, l, (int64_t)B * H * a.ntile, staged_bytes(dk, T_max, l.W, false), a,
                  stream);
  }
  return launch(KIND_COMMIT_COPY, false, dk, l, (int64_t)B * H * a.ntile, 0, a, stream);
}

int kda_query_variant(int32_t op, int32_t B, int32_t H, int32_t dk, int32_t dv, int32_t T_max,
                      int32_t epilogue, int32_t requested_tile_w, int32_t *tile_w, int32_t *threads) {
  if (B < 0 || H <= 0 || dk <= 0 || dv <= 0) return KDA_ERR_INVALID;
  Kind kind;
  switch (op) {
    case KDA_OP_DECODE: kind = KIND_DECODE; break;
    case KDA_OP_VERIFY: kind = KIND_VERIFY; break;
    case KDA_OP_COMMIT_REPLAY: kind = KIND_COMMIT_REPLAY; break;
    case KDA_OP_COMMIT_COPY: kind = KIND_COMMIT_COPY; break;
    case KDA_OP_PREFILL: kind = KIND_PREFILL; break;
    default: return KDA_ERR_INVALID;
  }
  if (!dims_supported(dk, dv) || T_max < 1 || (kind != KIND_PREFILL && T_max > kMaxT)) return KDA_ERR_UNSUPPORTED;
  if (epilogue && kind != KIND_DECODE && kind != KIND_VERIFY) return KDA_ERR_INVALID;
  Launch l;
  KDA_TRY(choose_width(kind, B, H, dk, dv, epilogue != 0, requested_tile_w, &l));
  if (tile_w) *tile_w = l.W;
  if (threads) *threads = 64 * l.waves;
  return KDA_OK;
}

static int state_copy(bool pack, float *cache, int64_t num_slots, int64_t slot_stride, const int32_t *slot_ids,
                      int32_t B, int32_t H, int32_t dk, int32_t dv, int32_t head0, int32_t nheads, int32_t col0,
                      int32_t ncols, float *buf, int32_t *dev_err, void *stream) {
  if (B < 0 || H <= 0 || dk <= 0 || dv <= 0) return KDA_ERR_INVALID;
  if (head0 < 0 || nheads < 0 || head0 + nheads > H || col0 < 0 || ncols < 0 || col0 + ncols > dv)
    return KDA_ERR_INVALID;
  if (!dims_supported(dk, dv)) return KDA_ERR_UNSUPPORTED;
  if (B == 0 || nheads == 0 || ncols == 0) return KDA_OK;
  if (!slot_ids || !buf) return KDA_ERR_INVALID;
  KDA_TRY(check_cache(cache, num_slots, slot_stride, H, dk, dv));
  if (!aligned(buf, 16) || (dev_err && !aligned(dev_err, 4))) return KDA_ERR_ALIGN;
  const int lanes = state_copy_lanes();
  const int parts = (ncols * dk / 4 + lanes - 1) / lanes;
  const int64_t blocks = (int64_t)B * nheads * parts;
  if (blocks > 0x7fffffff) return KDA_ERR_UNSUPPORTED;
  PackArgs p;
  p.cache = cache;
  p.num_slots = num_slots;
  p.slot_stride = slot_stride;
  p.slot_ids = slot_ids;
  p.buf = buf;
  p.dev_err = dev_err;
  p.H = H;
  p.dk = dk;
  p.dv = dv;
  p.head0 = head0;
  p.nheads = nheads;
  p.col0 = col0;
  p.ncols = ncols;
  p.parts = parts;
  void *args[] = {&p};
  const void *fn = state_copy_kernel_for(pack);
  const hipError_t e = hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(lanes), args, 0, (hipStream_t)stream);
  return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

int kda_state_pack(const float *cache, int64_t num_slots, int64_t slot_stride, const int32_t *slot_ids,
                   int32_t B, int32_t H, int32_t dk, int32_t dv, int32_t head0, int32_t nheads, int32_t col0,
                   int32_t ncols, float *buf, int32_t *dev_err, void *stream) {
  return state_copy(true, const_cast<float *>(cache), num_slots, slot_stride, slot_ids, B, H, dk, dv, head0,
                    nheads, col0, ncols, buf, dev_err, stream);
}

int kda_state_unpack(float *cache, int64_t num_slots, int64_t slot_stride, const int32_t *slot_ids, int32_t B,
                     int32_t H, int32_t dk, int32_t dv, int32_t head0, int32_t nheads, int32_t col0,
                     int32_t ncols, const float *buf, int32_t *dev_err, void *stream) {
  return state_copy(false, cache, num_slots, slot_stride, slot_ids, B, H, dk, dv, head0, nheads, col0, ncols,
                    const_cast<float *>(buf), dev_err, stream);
}

const char *kda_status_str(int32_t status) {
  switch (status) {
    case KDA_OK: return "ok";
    case KDA_ERR_INVALID: return "invalid argument";
    case KDA_ERR_UNSUPPORTED: return "unsupported shape or launch width";
    case KDA_ERR_ALIGN: return "misaligned pointer or stride";
    case KDA_ERR_HIP: return "HIP launch failed";
    case KDA_ERR_TOO_LARGE: return "the call needs more than the library's static scratch holds";
  }
  return "unknown status";
}

}  // extern "C"

