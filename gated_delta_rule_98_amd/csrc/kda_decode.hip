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
  const Lane L = lane_geometry();
  const int W = C * L.slab;
  const int64_t th = (int64_t)u.b * a.H + u.h;
  const int64_t vbase = th * a.dv + (int64_t)u.tile * W;
  float4 kk[NV], qq[NV], aa[NV];
  float vj[C];
  float beta;
  auto load_inputs = [&]() {
#pragma unroll
    for (int e = 0; e < NV; ++e) {
      const int64_t off = th * DK + 4 * L.r + 64 * e;
      kk[e] = unpack_bf16x4(*reinterpret_cast<const uint2 *>(a.k + off));
      qq[e] = unpack_bf16x4(*reinterpret_cast<const uint2 *>(a.q + off));
      aa[e] = *reinterpret_cast<const float4 *>(a.alpha + off);
    }
#pragma unroll
    for (int c = 0; c < C; ++c) vj[c] = bf16_to_f32(a.v[vbase + L.col0 + c * L.slab]);
    beta = a.beta[th];
  };
  // With one or two slabs per lane the inputs go out first, while the slot id
  // returns (the scheduling barrier keeps the compiler from sinking them behind
  // the state load); with more slabs the state tile goes first (measured on
  // MI355X: inputs first was 7% slower at 128 columns per workgroup).
  constexpr bool kInputsFirst = C <= 2;
  if constexpr (kInputsFirst) {
    load_inputs();
    __builtin_amdgcn_sched_barrier(0);
  }
  const int32_t slot = a.slot_ids[u.b];
  if (slot < 0) return;
  if (slot >= a.num_slots) {
    report(a.dev_err, u, KDA_DEVERR_SLOT);
    return;
  }
  float *S = a.cache + (int64_t)slot * a.slot_stride + ((int64_t)u.h * a.dv + (int64_t)u.tile * W) * DK;

  float4 s[C][NV];
  load_tile<DK, C, kDecodeLoadStream>(s, S, L);
  if constexpr (!kInputsFirst) load_inputs();
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

// Single-token step at dk = 128 in column pairs: one wave per two value columns,
// one float4 of state per lane, so each wave reads and writes one contiguous
// 1 KiB span (the large-batch stream shape). The inputs do not depend on the
// slot, so they are requested before the slot id and are in flight while it
// returns; the scheduling barrier keeps the compiler from sinking them behind
// the state load. The arithmetic is decode_kernel's, operation for operation
// (pair_dot reproduces lane_dot and row16_sum), so states and outputs are the
// same bits as every other tile width.
template <int IO>
__global__ __launch_bounds__(64) void decode_pair_kernel(Args a) {
  constexpr bool RAW = IO & kIoRaw, BF16 = IO & kIoBf16;
  const Unit u = unit_of_block(a.ntile, a.H);
  const int lane = threadIdx.x & 63, ch = 4 * (lane & 31);
  const int64_t th = (int64_t)u.b * a.H + u.h;
  const int64_t col = th * a.dv + (int64_t)u.tile * 2 + (lane >> 5);
  const uint2 k2 = *reinterpret_cast<const uint2 *>(a.k + th * 128 + ch);
  const uint2 q2 = *reinterpret_cast<const uint2 *>(a.q + th * 128 + ch);
  float4 aa = *reinterpret_cast<const float4 *>(a.alpha + th * 128 + ch);
  const uint32_t vbits = a.v[col];
  float beta = a.beta[th];
  __builtin_amdgcn_sched_barrier(0);
  const int32_t slot = a.slot_ids[u.b];
  if (slot < 0) return;
  if (slot >= a.num_slots) {
    report(a.dev_err, u, KDA_DEVERR_SLOT);
    return;
  }
  float *S = a.cache + (int64_t)slot * a.slot_stride + ((int64_t)u.h * a.dv + (int64_t)u.tile * 2) * 128;
  float4 s = ld4<kDecodeLoadStream>(S + 4 * lane);
  float4 kk = unpack_bf16x4(k2), qq = unpack_bf16x4(q2);
  if constexpr (RAW) {
    // prep_normalize and prep_decay on the pair layout
    const float fk = __builtin_amdgcn_rsqf(pair_dot(kk, kk) + 1e-12f) * 1.0f;
    const float fq = __builtin_amdgcn_rsqf(pair_dot(qq, qq) + 1e-12f) * (1.0f / __builtin_sqrtf(128.0f));
    kk = make_float4(kk.x * fk, kk.y * fk, kk.z * fk, kk.w * fk);
    qq = make_float4(qq.x * fq, qq.y * fq, qq.z * fq, qq.w * fq);
    aa = make_float4(prep_sigmoid_neg(aa.x), prep_sigmoid_neg(aa.y), prep_sigmoid_neg(aa.z),
                     prep_sigmoid_neg(aa.w));
    beta = prep_beta(beta);
  }
  const float vj = bf16_to_f32(vbits);

  s.x = s.x * aa.x;
  s.y = s.y * aa.y;
  s.z = s.z * aa.z;
  s.w = s.w * aa.w;
  const float d = beta * (vj - pair_dot(s, kk));
  s.x = __builtin_fmaf(kk.x, d, s.x);
  s.y = __builtin_fmaf(kk.y, d, s.y);
  s.z = __builtin_fmaf(kk.z, d, s.z);
  s.w = __builtin_fmaf(kk.w, d, s.w);
  const float o = pair_dot(s, qq);
  st4<kDecodeStoreStream>(S + 4 * lane, s);
  if ((lane & 31) == 0) put_out(a, BF16, col, o);
}

}  // namespace

struct decode_pair_table {
  template <int IO>
  static const void *get() { return (const void *)decode_pair_kernel<IO>; }
};

const void *decode_pair_kernel_for(int io) { return io_variant<decode_pair_table>(io); }

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
