// kda_chunk.h - interface of the chunk forms of prefill (kda_prefill_chunk.hip)
// and verify (kda_verify_chunk.hip) to the C ABI in kda_api.hip.

#pragma once

#include <stddef.h>
#include <stdint.h>

namespace kda {

constexpr int kChunkTokens = 32;  // tokens per chunk of the chunk form of prefill
// Threads of a precompute workgroup (8 waves; measured on MI355X against 4 and
// 16 at d = 128).
constexpr int kChunkPrepThreads = 512;
// Threads of a state-pass workgroup: four recurrence waves and two waves that
// finish the outputs (measured on MI355X against eight waves, two of them only
// keeping the barrier count: 694 against 704 us for an 8000-token prefill).
constexpr int kChunkStateThreads = 384;

// Arguments of both chunk-prefill kernels.
struct ChunkArgs {
  float *cache;
  int64_t num_slots, slot_stride;
  const int32_t *slot_ids, *cu, *ckpt_pos;
  const uint16_t *q, *k, *v;
  const float *alpha, *beta;
  float *out;  // fp32, or bf16 when out_bf16
  float *ckpt;
  float *ws;
  int32_t *cbase;  // [B + 1] first chunk of each row (workspace tail; the map kernel writes it)
  int32_t *crow;   // [ws_chunks] row of each chunk, -1 past the last (likewise)
  int32_t *dev_err;
  int32_t B, H, n_tok, ws_chunks, ntile, raw, out_bf16;
};

// Floats of workspace per (chunk, head).
size_t prefill_chunk_ws_floats(int dk, int dv);
// Kernel handles: the chunk map, the per-chunk precompute and the sequential
// pass over chunks.
const void *prefill_chunk_map_kernel();
constexpr int kChunkMapThreads = 1024;
const void *prefill_chunk_prep_kernel_for(int dk, int dv);
const void *prefill_chunk_state_kernel_for(int dk, int dv);

// Chunk form of verify: one workgroup of dv / 16 waves per (row, head), its
// dynamic LDS bytes, and the kernel handle (dk, dv in {64, 128}, T_max <= 16).
size_t chunk_verify_lds_bytes(int dk, int dv, int T_max);
const void *verify_chunk_kernel_for(int dk, int dv, int T_max, int64_t groups);  // groups = B * H

}  // namespace kda
