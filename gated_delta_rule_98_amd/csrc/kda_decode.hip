// kda_decode.hip - the single-token decode step (kda_decode_step).

#include "kda_engine.h"

namespace kda {
namespace {

// Single-token step, in place. Inputs go straight to registers: a lane's key
// channels are fixed, so it loads exactly the k, q, alpha it uses.
template <int DK, int C, bool GATE, int IO>
__global__ __launch_bounds__(GATE ? 1024 : 256) void decode_kernel(Args a) {
  constexpr int NV = DK / 64;
  constexpr bool RAW = IO & kIoRaw, BF16 = IO & kIoBf16;
  const Unit u = unit_of_block(a.ntile, a.H);
  const int32_t slot = a.slot_ids[u.b];
  if (slot < 0) return;
  if (slot >= a.num_slots) {
    report(a.dev_err, u, KDA_DEVERR_SLOT);
    return;
  }
  const Lane L = lane_geometry();
  const int W = C * L.slab;
  const int64_t th = (int64_t)u.b * a.H + u.h;
  float *S = a.cache + (int64_t)slot * a.slot_stride + ((int64_t)u.h * a.dv + (int64_t)u.tile * W) * DK;

  float4 s[C][NV];
  load_tile<DK, C, kDecodeLoadStream>(s, S, L);
  float4 kk[NV], qq[NV], aa[NV];
#pragma unroll
  for (int e = 0; e < NV; ++e) {
    const int64_t off = th * DK + 4 * L.r + 64 * e;
    kk[e] = unpack_bf16x4(*reinterpret_cast<const uint2 *>(a.k + off));
    qq[e] = unpack_bf16x4(*reinterpret_cast<const uint2 *>(a.q + off));
    aa[e] = *reinterpret_cast<const float4 *>(a.alpha + off);
  }
  const int64_t vbase = th * a.dv + (int64_t)u.tile * W;
  float vj[C];
#pragma unroll
  for (int c = 0; c < C; ++c) vj[c] = bf16_to_f32(a.v[vbase + L.col0 + c * L.slab]);
  float beta = a.beta[th];
  if constexpr (RAW) {
    prep_normalize<NV>(kk, 1.0f);
    prep_normalize<NV>(qq, 1.0f / __builtin_sqrtf((float)DK));
    prep_decay<NV>(aa);
    beta = prep_beta(beta);
  }
  float gj = 0.0f, wj = 1.0f;
  if constexpr (GATE) {
    const int j = L.col0 + (L.r < C ? L.r : 0) * L.slab;
    gj = bf16_to_f32(a.gate[vbase + j]);
    if (a.weight) wj = a.weight[j];
  }

  token_update<NV, C>(s, aa, kk, vj, beta);
  float o[C];
  token_readout<NV, C>(s, qq, o);
  store_tile<DK, C, kDecodeStoreStream>(S, s, L);
  if constexpr (GATE) {
    __shared__ float part[kMaxWaves];
    __shared__ float raw[kMaxDv];
    store_cols<C>(raw, L, o);
    gate_partial<C>(o, part);
    __syncthreads();
    if (L.r < C) {
      const int j = L.col0 + L.r * L.slab;
      put_out(a, BF16, vbase + j, gate_apply(a, part, raw[j], gj, wj));
    }
  } else {
    store_out<C>(a, BF16, vbase, L, o);
  }
}

}  // namespace

template <int DK, int C, bool GATE>
struct decode_table {
  template <int IO>
  static const void *get() { return (const void *)decode_kernel<DK, C, GATE, IO>; }
};

template <int DK>
const void *decode_for(int C, bool gate, int io) {
  if (gate) return C == kGateSlabsDecode ? io_variant<decode_table<DK, kGateSlabsDecode, true>>(io) : nullptr;
  switch (C) {
    case 1: return io_variant<decode_table<DK, 1, false>>(io);
    case 2: return io_variant<decode_table<DK, 2, false>>(io);
    case 4: return io_variant<decode_table<DK, 4, false>>(io);
    case 8: return io_variant<decode_table<DK, 8, false>>(io);
  }
  return nullptr;
}

const void *decode_kernel_for(int dk, int C, bool gate, int io) {
  return dk == 64 ? decode_for<64>(C, gate, io) : dk == 128 ? decode_for<128>(C, gate, io) : nullptr;
}

}  // namespace kda
