// kda_verify.hip - speculative verify, token by token (kda_verify_chunk), and
// both commit modes (kda_replay_commit).

#include "kda_engine.h"

namespace kda {
namespace {

// LDS staging for a chunk of tokens: k, q, alpha as float [T_max][DK], the
// tile's v as float [T_max][W], beta [T_max], and with the output gate the
// tile's gate as float [T_max][W].
template <int DK>
struct Staged {
  float *k, *q, *a, *v, *beta, *g;
  __device__ Staged(float *base, int T_max, int W) {
    k = base;
    q = k + T_max * DK;
    a = q + T_max * DK;
    v = a + T_max * DK;
    beta = v + T_max * W;
    g = beta + T_max;
  }
};


// Speculative verify over a packed chunk: T_b tokens with the state in
// registers; outputs per token; the committed slot stays untouched unless the
// row is a single in-place token.
template <int DK, int C, bool GATE, int IO>
__global__ __launch_bounds__(GATE ? 1024 : 256) void verify_kernel(Args a) {
  constexpr int NV = DK / 64;
  constexpr bool RAW = IO & kIoRaw, BF16 = IO & kIoBf16;
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
  const bool inplace = Tb == 1 && a.t1_inplace;
  const bool replay = !inplace && a.mode == KDA_REPLAY;
  const bool perpos = !inplace && a.mode == KDA_PER_POSITION;
  const Lane L = lane_geometry();
  const int W = C * L.slab;
  Staged<DK> st(reinterpret_cast<float *>(lds_dyn), a.T_max, W);
  // the state tile is requested first, so its HBM latency overlaps the staging
  float *S = a.cache + (int64_t)slot * a.slot_stride + ((int64_t)u.h * a.dv + (int64_t)u.tile * W) * DK;
  float4 s[C][NV];
  load_tile<DK, C, kVerifyLoadStream>(s, S, L);

  // stage the chunk's inputs; in replay mode also copy them to the buffer
  for (int idx = threadIdx.x; idx < Tb * (DK / 4); idx += blockDim.x) {
    const int t = idx / (DK / 4), i = (idx % (DK / 4)) * 4;
    const int64_t off = ((row0 + t) * a.H + u.h) * DK + i;
    const uint2 kb = *reinterpret_cast<const uint2 *>(a.k + off);
    const uint2 qb = *reinterpret_cast<const uint2 *>(a.q + off);
    const float4 al = *reinterpret_cast<const float4 *>(a.alpha + off);
    *reinterpret_cast<float4 *>(st.k + t * DK + i) = unpack_bf16x4(kb);
    *reinterpret_cast<float4 *>(st.q + t * DK + i) = unpack_bf16x4(qb);
    *reinterpret_cast<float4 *>(st.a + t * DK + i) = al;
    if (replay && u.tile == 0) {
      const int64_t d = (((int64_t)u.b * a.T_max + t) * a.H + u.h) * DK + i;
      *reinterpret_cast<uint2 *>(a.rk + d) = kb;
      *reinterpret_cast<float4 *>(a.ralpha + d) = al;
    }
  }
  for (int idx = threadIdx.x; idx < Tb * W; idx += blockDim.x) {
    const int t = idx / W, jj = idx % W;
    const uint16_t vb = a.v[((row0 + t) * a.H + u.h) * a.dv + (int64_t)u.tile * W + jj];
    st.v[t * W + jj] = bf16_to_f32(vb);
    if (replay) a.rv[(((int64_t)u.b * a.T_max + t) * a.H + u.h) * a.dv + (int64_t)u.tile * W + jj] = vb;
    if constexpr (GATE) st.g[t * W + jj] = bf16_to_f32(a.gate[((row0 + t) * a.H + u.h) * a.dv + (int64_t)u.tile * W + jj]);
  }
  if ((int)threadIdx.x < Tb) {
    const float bt = a.beta[(row0 + threadIdx.x) * a.H + u.h];
    st.beta[threadIdx.x] = bt;
    if (replay && u.tile == 0) a.rbeta[((int64_t)u.b * a.T_max + threadIdx.x) * a.H + u.h] = bt;
  }
  __syncthreads();
  if constexpr (RAW) {
    prep_staged<DK>(st.k, st.q, st.a, st.beta, Tb);
    __syncthreads();
  }

  __shared__ float part[GATE ? kMaxT * kMaxWaves : 1];
  __shared__ float raw[GATE ? kMaxT * kMaxDv : 1];

  for (int t = 0; t < Tb; ++t) {
    float4 kk[NV], qq[NV], aa[NV];
#pragma unroll
    for (int e = 0; e < NV; ++e) {
      const int i = t * DK + 4 * L.r + 64 * e;
      kk[e] = *reinterpret_cast<const float4 *>(st.k + i);
      qq[e] = *reinterpret_cast<const float4 *>(st.q + i);
      aa[e] = *reinterpret_cast<const float4 *>(st.a + i);
    }
    float vj[C];
#pragma unroll
    for (int c = 0; c < C; ++c) vj[c] = st.v[t * W + L.col0 + c * L.slab];
    token_update<NV, C>(s, aa, kk, vj, st.beta[t]);
    float o[C];
    token_readout<NV, C>(s, qq, o);
    const int64_t obase = ((row0 + t) * a.H + u.h) * a.dv + (int64_t)u.tile * W;
    if constexpr (GATE) {
      // keep the raw read-out in LDS; the whole chunk is normalized after the loop
      store_cols<C>(raw + t * kMaxDv, L, o);
      gate_partial<C>(o, part + t * kMaxWaves);
    } else {
      store_out<C>(a, BF16, obase, L, o);
    }
    if (perpos) {
      float *D = a.draft + ((((int64_t)u.b * a.T_max + t) * a.H + u.h) * a.dv + (int64_t)u.tile * W) * DK;
      store_tile<DK, C, kVerifyStoreStream>(D, s, L);
    }
  }
  if (inplace) store_tile<DK, C, kVerifyStoreStream>(S, s, L);
  if constexpr (GATE) {
    // one barrier for the whole chunk, then each lane finishes its column per token
    __syncthreads();
    if (L.r < C) {
      const int j = L.col0 + L.r * L.slab;
      const float wj = a.weight ? a.weight[j] : 1.0f;
      for (int t = 0; t < Tb; ++t) {
        const int64_t obase = ((row0 + t) * a.H + u.h) * a.dv + (int64_t)u.tile * W;
        put_out(a, BF16, obase + j, gate_apply(a, part + t * kMaxWaves, raw[t * kMaxDv + j], st.g[t * W + j], wj));
      }
    }
  }
}

// ----------------------------------------------------------------------------
// Commit
// ----------------------------------------------------------------------------

// Row checks shared by the commit kernels; returns the accepted length, or -1
// when the row does not run.
__device__ __forceinline__ int commit_row(const Args &a, const Unit &u, int32_t &slot) {
  slot = a.slot_ids[u.b];
  if (slot < 0) return -1;
  if (slot >= a.num_slots) {
    report(a.dev_err, u, KDA_DEVERR_SLOT);
    return -1;
  }
  int Tb = a.T_max;
  if (a.cu) {
    int64_t row0;
    if (!row_range(a, u.b, row0, Tb)) {
      report(a.dev_err, u, KDA_DEVERR_SEQLEN);
      return -1;
    }
  }
  const int n = a.accepted[u.b];
  if (n < 0 || n > Tb) {
    report(a.dev_err, u, KDA_DEVERR_ACCEPTED);
    return -1;
  }
  return n;
}

// ReplaySSM commit: reload the committed state, replay the first n buffered
// tokens with the same column engine, store once.
template <int DK, int C>
__global__ __launch_bounds__(256) void commit_replay_kernel(Args a) {
  constexpr int NV = DK / 64;
  extern __shared__ float4 lds_dyn[];
  const Unit u = unit_of_block_rows(a.ntile, a.H, a.B);
  int32_t slot;
  const int n = commit_row(a, u, slot);
  if (n <= 0) return;
  const Lane L = lane_geometry();
  const int W = C * L.slab;
  Staged<DK> st(reinterpret_cast<float *>(lds_dyn), a.T_max, W);
  // the state tile is requested first, so its HBM latency overlaps the staging
  float *S = a.cache + (int64_t)slot * a.slot_stride + ((int64_t)u.h * a.dv + (int64_t)u.tile * W) * DK;
  float4 s[C][NV];
  load_tile<DK, C, kCommitLoadStream>(s, S, L);
  for (int idx = threadIdx.x; idx < n * (DK / 4); idx += blockDim.x) {
    const int t = idx / (DK / 4), i = (idx % (DK / 4)) * 4;
    const int64_t d = (((int64_t)u.b * a.T_max + t) * a.H + u.h) * DK + i;
    *reinterpret_cast<float4 *>(st.k + t * DK + i) = unpack_bf16x4(*reinterpret_cast<const uint2 *>(a.rk + d));
    *reinterpret_cast<float4 *>(st.a + t * DK + i) = *reinterpret_cast<const float4 *>(a.ralpha + d);
  }
  for (int idx = threadIdx.x; idx < n * W; idx += blockDim.x) {
    const int t = idx / W, jj = idx % W;
    st.v[t * W + jj] = bf16_to_f32(a.rv[(((int64_t)u.b * a.T_max + t) * a.H + u.h) * a.dv + (int64_t)u.tile * W + jj]);
  }
  if ((int)threadIdx.x < n) st.beta[threadIdx.x] = a.rbeta[((int64_t)u.b * a.T_max + threadIdx.x) * a.H + u.h];
  __syncthreads();
  if (a.raw) {
    prep_staged<DK>(st.k, nullptr, st.a, st.beta, n);
    __syncthreads();
  }

  for (int t = 0; t < n; ++t) {
    float4 kk[NV], aa[NV];
#pragma unroll
    for (int e = 0; e < NV; ++e) {
      const int i = t * DK + 4 * L.r + 64 * e;
      kk[e] = *reinterpret_cast<const float4 *>(st.k + i);
      aa[e] = *reinterpret_cast<const float4 *>(st.a + i);
    }
    float vj[C];
#pragma unroll
    for (int c = 0; c < C; ++c) vj[c] = st.v[t * W + L.col0 + c * L.slab];
    token_update<NV, C>(s, aa, kk, vj, st.beta[t]);
  }
  store_tile<DK, C, kCommitStoreStream>(S, s, L);
}

// Per-position commit: copy the state saved after the last accepted token.
template <int DK, int C>
__global__ __launch_bounds__(256) void commit_copy_kernel(Args a) {
  constexpr int NV = DK / 64;
  const Unit u = unit_of_block_rows(a.ntile, a.H, a.B);
  int32_t slot;
  const int n = commit_row(a, u, slot);
  if (n <= 0) return;
  const Lane L = lane_geometry();
  const int W = C * L.slab;
  const float *D = a.draft + ((((int64_t)u.b * a.T_max + (n - 1)) * a.H + u.h) * a.dv + (int64_t)u.tile * W) * DK;
  float *S = a.cache + (int64_t)slot * a.slot_stride + ((int64_t)u.h * a.dv + (int64_t)u.tile * W) * DK;
  float4 s[C][NV];
  load_tile<DK, C, kCopyLoadStream>(s, D, L);
  store_tile<DK, C, kCopyStoreStream>(S, s, L);
}

}  // namespace

// Dynamic LDS bytes for Staged<dk>, rounded up to 16.
size_t staged_bytes(int dk, int T_max, int W, bool gate) {
  return ((size_t)T_max * (3 * dk + W + 1 + (gate ? W : 0)) * sizeof(float) + 15) / 16 * 16;
}

template <int DK, int C, bool GATE>
struct verify_table {
  template <int IO>
  static const void *get() { return (const void *)verify_kernel<DK, C, GATE, IO>; }
};

template <int DK>
const void *verify_for(int C, bool gate, int io) {
  if (gate) return C == kGateSlabsVerify ? io_variant<verify_table<DK, kGateSlabsVerify, true>>(io) : nullptr;
  switch (C) {
    case 1: return io_variant<verify_table<DK, 1, false>>(io);
    case 2: return io_variant<verify_table<DK, 2, false>>(io);
    case 4: return io_variant<verify_table<DK, 4, false>>(io);
    case 8: return io_variant<verify_table<DK, 8, false>>(io);
  }
  return nullptr;
}

const void *verify_kernel_for(int dk, int C, bool gate, int io) {
  return dk == 64 ? verify_for<64>(C, gate, io) : dk == 128 ? verify_for<128>(C, gate, io) : nullptr;
}

template <int DK>
const void *commit_for(bool replay, int C) {
  switch (C) {
    case 1: return replay ? (const void *)commit_replay_kernel<DK, 1> : (const void *)commit_copy_kernel<DK, 1>;
    case 2: return replay ? (const void *)commit_replay_kernel<DK, 2> : (const void *)commit_copy_kernel<DK, 2>;
    case 4: return replay ? (const void *)commit_replay_kernel<DK, 4> : (const void *)commit_copy_kernel<DK, 4>;
    case 8: return replay ? (const void *)commit_replay_kernel<DK, 8> : (const void *)commit_copy_kernel<DK, 8>;
  }
  return nullptr;
}

const void *commit_replay_kernel_for(int dk, int C) {
  return dk == 64 ? commit_for<64>(true, C) : dk == 128 ? commit_for<128>(true, C) : nullptr;
}

const void *commit_copy_kernel_for(int dk, int C) {
  return dk == 64 ? commit_for<64>(false, C) : dk == 128 ? commit_for<128>(false, C) : nullptr;
}

}  // namespace kda
