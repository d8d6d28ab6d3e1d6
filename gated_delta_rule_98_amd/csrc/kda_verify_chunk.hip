// kda_verify_chunk.hip - the chunk form of speculative verify (KDA_VERIFY_CHUNKED).

#include "kda_engine.h"

namespace kda {
namespace {

// ----------------------------------------------------------------------------
// Chunk form of verify (outputs only), MFMA for the state products
// ----------------------------------------------------------------------------
//
// For the T_b <= 16 tokens of a row, with S0 the committed state, G_t the
// running product of the decays up to and including token t, and
// D(s, t) = k_s * prod_{s < r <= t} alpha_r (the key of token s as the decayed
// state sees it at token t):
//   u_t     = S0^T (G_t k_t) + sum_{s<t} (k_t . D(s,t)) delta_s
//   delta_t = beta_t (v_t - u_t)
//   o_t     = S0^T (G_t q_t) + sum_{s<=t} (q_t . D(s,t)) delta_s
// which is the token-by-token recurrence unrolled over the chunk. The two
// products with S0 are a [2 x 16, dk] x [dk, W] matrix product on MFMA; the
// coupling coefficients come from running products (no division, so any decay
// in (0, 1] is safe); delta is a forward substitution per value column.
//
// Workgroup: 4 waves, W = 64 value columns, wave w owns columns 16w..16w+15.
// The state is held in the v_mfma_f32_16x16x4f32 accumulator layout: for the
// 16x16 block of channels 16cb..16cb+15 and the wave's columns, lane
// (j = lane % 16, g = lane / 16) holds channels 16cb + 4g .. + 3 of column j,
// one 128-bit load from the [dv][dk] cache. As the B operand of step
// (cb, e) that lane supplies channel 16cb + 4g + e; the A operand uses the same
// channel order, so the contraction over dk is complete.

constexpr int kChunkRows = 16;  // MFMA row block: tokens per chunk

// LDS of the chunk kernel, in floats.
struct ChunkLds {
  float *k, *q, *a;  // [T_max][DK] staged inputs
  float *v;          // [T_max][kChunkW]
  float *beta;       // [kChunkRows]
  float *kp, *qp;    // [DK / 4][kChunkRows][4]: G_t k_t and G_t q_t, 4 channels per entry
  float *cA, *cB;    // [kChunkRows][kChunkRows] coupling coefficients
  float *u0, *o0;    // [kChunkRows][kChunkW] products with S0
  __device__ ChunkLds(float *base, int T_max, int dk) {
    k = base;
    q = k + T_max * dk;
    a = q + T_max * dk;
    v = a + T_max * dk;
    beta = v + T_max * kChunkW;
    kp = beta + kChunkRows;
    qp = kp + dk * kChunkRows;
    cA = qp + dk * kChunkRows;
    cB = cA + kChunkRows * kChunkRows;
    u0 = cB + kChunkRows * kChunkRows;
    o0 = u0 + kChunkRows * kChunkW;
  }
};


template <int DK>
__global__ __launch_bounds__(256) void verify_chunk_kernel(Args a) {
  constexpr int NCB = DK / 16;  // 16-channel blocks
  constexpr int CPT = DK / 16;  // channels per thread in the coupling pass
  extern __shared__ float4 lds_dyn[];
  const Unit u = unit_of_block_rows(a.ntile, a.H, a.B);
  const int32_t slot = a.slot_ids[u.b];
  if (slot < 0) return;
  if (slot >= a.num_slots) {
    report(a.dev_err, u, KDA_DEVERR_SLOT);
    return;
  }
  int64_t row0;
  int Tb;
  if (!row_range(a, u.b, row0, Tb)) {
    report(a.dev_err, u, KDA_DEVERR_SEQLEN);
    return;
  }
  if (Tb == 0) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int j = lane & 15, g = lane >> 4;

  // committed state of the wave's 16 columns, in accumulator layout (issued first)
  const float *Scol = a.cache + (int64_t)slot * a.slot_stride +
                      ((int64_t)u.h * a.dv + (int64_t)u.tile * kChunkW + 16 * wave + j) * DK + 4 * g;
  float4 sreg[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) sreg[cb] = ld4<kVerifyLoadStream>(Scol + 16 * cb);

  ChunkLds L(reinterpret_cast<float *>(lds_dyn), a.T_max, DK);
  // stage the row's inputs and copy them to the replay buffer
  for (int idx = threadIdx.x; idx < Tb * (DK / 4); idx += blockDim.x) {
    const int t = idx / (DK / 4), i = (idx % (DK / 4)) * 4;
    const int64_t off = ((row0 + t) * a.H + u.h) * DK + i;
    const uint2 kb = *reinterpret_cast<const uint2 *>(a.k + off);
    const uint2 qb = *reinterpret_cast<const uint2 *>(a.q + off);
    const float4 al = *reinterpret_cast<const float4 *>(a.alpha + off);
    *reinterpret_cast<float4 *>(L.k + t * DK + i) = unpack_bf16x4(kb);
    *reinterpret_cast<float4 *>(L.q + t * DK + i) = unpack_bf16x4(qb);
    *reinterpret_cast<float4 *>(L.a + t * DK + i) = al;
    if (u.tile == 0) {
      const int64_t d = (((int64_t)u.b * a.T_max + t) * a.H + u.h) * DK + i;
      *reinterpret_cast<uint2 *>(a.rk + d) = kb;
      *reinterpret_cast<float4 *>(a.ralpha + d) = al;
    }
  }
  for (int idx = threadIdx.x; idx < Tb * kChunkW; idx += blockDim.x) {
    const int t = idx / kChunkW, jj = idx % kChunkW;
    const uint16_t vb = a.v[((row0 + t) * a.H + u.h) * a.dv + (int64_t)u.tile * kChunkW + jj];
    L.v[t * kChunkW + jj] = bf16_to_f32(vb);
    a.rv[(((int64_t)u.b * a.T_max + t) * a.H + u.h) * a.dv + (int64_t)u.tile * kChunkW + jj] = vb;
  }
  if ((int)threadIdx.x < kChunkRows) {
    float bt = 0.0f;
    if ((int)threadIdx.x < Tb) {
      bt = a.beta[(row0 + threadIdx.x) * a.H + u.h];
      if (u.tile == 0) a.rbeta[((int64_t)u.b * a.T_max + threadIdx.x) * a.H + u.h] = bt;
    }
    L.beta[threadIdx.x] = bt;
  }
  __syncthreads();

  // G_t k_t and G_t q_t (rows t >= T_b are zero), one thread per channel
  if ((int)threadIdx.x < DK) {
    const int i = threadIdx.x;
    float G = 1.0f;
    for (int t = 0; t < kChunkRows; ++t) {
      float kp = 0.0f, qp = 0.0f;
      if (t < Tb) {
        G = G * L.a[t * DK + i];
        kp = G * L.k[t * DK + i];
        qp = G * L.q[t * DK + i];
      }
      L.kp[((i >> 2) * kChunkRows + t) * 4 + (i & 3)] = kp;
      L.qp[((i >> 2) * kChunkRows + t) * 4 + (i & 3)] = qp;
    }
  }
  // coupling coefficients: thread (s, c) carries D(s, t) over its CPT channels
  // as t advances; a 16-lane row shares s and sums over the channel chunks
  {
    const int s = threadIdx.x >> 4, c = threadIdx.x & 15;
    float d[CPT];
#pragma unroll
    for (int e = 0; e < CPT; ++e) d[e] = s < Tb ? L.k[s * DK + c * CPT + e] : 0.0f;
    for (int t = 0; t < Tb; ++t) {
      const bool after = t > s;
      float pa = 0.0f, pb = 0.0f;
#pragma unroll
      for (int e = 0; e < CPT; ++e) {
        const int ch = t * DK + c * CPT + e;
        d[e] = after ? d[e] * L.a[ch] : d[e];
        pa = __builtin_fmaf(L.k[ch], d[e], pa);
        pb = __builtin_fmaf(L.q[ch], d[e], pb);
      }
      pa = row16_sum(pa);
      pb = row16_sum(pb);
      if (c == 0 && s < Tb) {
        if (after) L.cA[t * kChunkRows + s] = pa;
        if (t >= s) L.cB[t * kChunkRows + s] = pb;
      }
    }
  }
  __syncthreads();

  // U0 = [G k] S0 and O0 = [G q] S0 for the wave's 16 columns
  v4f accU = {0.0f, 0.0f, 0.0f, 0.0f}, accO = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const v4f ak = *reinterpret_cast<const v4f *>(L.kp + ((4 * cb + g) * kChunkRows + j) * 4);
    const v4f aq = *reinterpret_cast<const v4f *>(L.qp + ((4 * cb + g) * kChunkRows + j) * 4);
    const v4f b = {sreg[cb].x, sreg[cb].y, sreg[cb].z, sreg[cb].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      accU = __builtin_amdgcn_mfma_f32_16x16x4f32(ak[e], b[e], accU, 0, 0, 0);
      accO = __builtin_amdgcn_mfma_f32_16x16x4f32(aq[e], b[e], accO, 0, 0, 0);
    }
  }
  // accumulator layout: lane (j, g) holds rows (tokens) 4g .. 4g + 3 of column j
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    L.u0[(4 * g + r) * kChunkW + 16 * wave + j] = accU[r];
    L.o0[(4 * g + r) * kChunkW + 16 * wave + j] = accO[r];
  }
  __syncthreads();

  // forward substitution and outputs, one lane per value column
  if (lane < 16) {
    const int col = 16 * wave + lane;
    float delta[kChunkRows];
#pragma unroll
    for (int t = 0; t < kChunkRows; ++t) {
      if (t < Tb) {
        float acc = L.v[t * kChunkW + col] - L.u0[t * kChunkW + col];
#pragma unroll
        for (int s2 = 0; s2 < t; ++s2) acc = __builtin_fmaf(-L.cA[t * kChunkRows + s2], delta[s2], acc);
        delta[t] = L.beta[t] * acc;
        float o = L.o0[t * kChunkW + col];
#pragma unroll
        for (int s2 = 0; s2 <= t; ++s2) o = __builtin_fmaf(L.cB[t * kChunkRows + s2], delta[s2], o);
        a.out[((row0 + t) * a.H + u.h) * a.dv + (int64_t)u.tile * kChunkW + col] = o;
      }
    }
  }
}

}  // namespace

size_t chunk_lds_bytes(int dk, int T_max) {
  const size_t floats = (size_t)3 * T_max * dk + (size_t)T_max * kChunkW + kChunkRows +
                        (size_t)2 * dk * kChunkRows + 2 * kChunkRows * kChunkRows + 2 * kChunkRows * kChunkW;
  return (floats * sizeof(float) + 15) / 16 * 16;
}

const void *verify_chunk_kernel_for(int dk) {
  return dk == 64 ? (const void *)verify_chunk_kernel<64> : dk == 128 ? (const void *)verify_chunk_kernel<128> : nullptr;
}

}  // namespace kda
