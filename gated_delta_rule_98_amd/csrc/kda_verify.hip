// kda_verify.hip - speculative verify, token by token (kda_verify_chunk), and
// both commit modes (kda_replay_commit).

#include "kda_engine.h"

namespace kda {
namespace {

// LDS staging for a chunk of tokens. Each token's k, alpha and q sit in one
// record of 3 * DK floats, so a lane reaches all three from one pointer with
// constant offsets and moves to the next token with one add. The tile's v is
// [T_max][W] with each lane's C columns side by side (column col0 + c * slab
// at col0 * C + c), beta is [T_max], and with the output gate the tile's gate
// is [T_max][W] in column order.
template <int DK>
struct Staged {
  static constexpr int kRec = 3 * DK;
  float *rec, *v, *beta, *g;
  __device__ Staged(float *base, int T_max, int W) {
    rec = base;
    v = rec + T_max * kRec;
    beta = v + T_max * W;
    g = beta + T_max;
  }
  __device__ float *k(int t) const { return rec + t * kRec; }
  __device__ float *a(int t) const { return rec + t * kRec + DK; }
  __device__ float *q(int t) const { return rec + t * kRec + 2 * DK; }
};

// Position of tile column jj in the staged v: the lane owning it reads its C
// columns as one vector.
template <int C>
__device__ __forceinline__ int v_slot(int jj, int slab) {
  const int sh = __builtin_ctz(slab);  // slab = 4 * waves, a power of two
  return (jj & (slab - 1)) * C + (jj >> sh);
}

// LDS pointers in the local address space: the token loops step them with
// plain 32-bit adds and reach k, alpha and q through constant offsets.
typedef __attribute__((address_space(3))) const float lds_float;
typedef float lds_v2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ lds_float *to_lds(const float *p) { return (lds_float *)p; }
__device__ __forceinline__ float4 lds_f4(lds_float *p) {
  const v4f x = *(__attribute__((address_space(3))) const v4f *)p;
  return make_float4(x.x, x.y, x.z, x.w);
}

// The C staged v values of this lane's columns for one token.
template <int C>
__device__ __forceinline__ void load_v(lds_float *p, float (&vj)[C]) {
  if constexpr (C % 4 == 0) {
#pragma unroll
    for (int c = 0; c < C; c += 4) {
      const float4 x = lds_f4(p + c);
      vj[c] = x.x;
      vj[c + 1] = x.y;
      vj[c + 2] = x.z;
      vj[c + 3] = x.w;
    }
  } else if constexpr (C == 2) {
    const lds_v2 x = *(__attribute__((address_space(3))) const lds_v2 *)p;
    vj[0] = x.x;
    vj[1] = x.y;
  } else {
#pragma unroll
    for (int c = 0; c < C; ++c) vj[c] = p[c];
  }
}

// Speculative verify over a packed chunk: T_b tokens with the state in
// registers; outputs per token; the committed slot stays untouched unless the
// row is a single in-place token. Lane r of each 16-lane row keeps token r's
// outputs (the row's read-outs are equal in all its lanes), so outputs, and
// the gate, are written once after the token loop. PERPOS instantiates the
// per-position mode (each mode's loop alone keeps the register count down).
template <int DK, int C, bool GATE, int IO, bool PERPOS>
__global__ __launch_bounds__(GATE ? 1024 : 256) void verify_kernel(Args a) {
  constexpr int NV = DK / 64;
  constexpr bool RAW = IO & kIoRaw, BF16 = IO & kIoBf16;
  extern __shared__ float4 lds_dyn[];
  const Unit u = unit_of_block_headmajor(a.ntile, a.H, a.B);
  const Lane L = lane_geometry();
  int32_t slot;
  int64_t row0;
  int Tb;
  if (!row_slot_range(a, u, slot, row0, Tb)) return;
  if (Tb == 0) return;
  const bool inplace = Tb == 1 && a.t1_inplace;
  const bool replay = !inplace && !PERPOS;
  const int W = C * L.slab;
  Staged<DK> st(reinterpret_cast<float *>(lds_dyn), a.T_max, W);
  float *S = a.cache + (int64_t)slot * a.slot_stride + ((int64_t)u.h * a.dv + (int64_t)u.tile * W) * DK;
  // Vector loads complete in issue order. The first round of staging loads is
  // issued before the state tile, so writing the staging to LDS waits for the
  // inputs alone; each wave then waits for its own tile after the barrier
  // instead of the whole workgroup waiting for its slowest tile.
  const int nkq = Tb * (DK / 4);
  const int jj = threadIdx.x & (W - 1), sv = v_slot<C>(jj, L.slab);  // blockDim.x is a multiple of W
  const int tsh = __builtin_ctz(W), tstep = blockDim.x >> tsh, tv0 = threadIdx.x >> tsh;
  // Each array's part for this row and head starts at a uniform (scalar) base;
  // threads add 32-bit offsets (a token's stride times at most 16 tokens).
  const uint32_t kq_tok = (uint32_t)a.H * DK, v_tok = (uint32_t)a.H * a.dv;
  const int64_t kq0 = (row0 * a.H + u.h) * DK, v0 = (row0 * a.H + u.h) * a.dv + (int64_t)u.tile * W;
  const uint16_t *kbase = a.k + kq0, *qbase = a.q + kq0, *vbase = a.v + v0;
  const float *abase = a.alpha + kq0, *bbase = a.beta + row0 * a.H + u.h;
  auto kq_off = [&](int idx) { return (uint32_t)(idx / (DK / 4)) * kq_tok + (uint32_t)(idx % (DK / 4)) * 4; };
  auto v_off = [&](int t) { return (uint32_t)t * v_tok + (uint32_t)jj; };
  // (unconditional loads at clamped, in-bounds indices: straight-line code
  // keeps the compiler from waiting for them before the state loads go out)
  const uint32_t off0 = kq_off(min((int)threadIdx.x, nkq - 1));
  const uint2 kb0 = *reinterpret_cast<const uint2 *>(kbase + off0);
  const uint2 qb0 = *reinterpret_cast<const uint2 *>(qbase + off0);
  const float4 al0 = *reinterpret_cast<const float4 *>(abase + off0);
  const uint32_t voff0 = v_off(min(tv0, Tb - 1));
  const uint16_t vb0 = vbase[voff0];
  const uint16_t gb0 = GATE ? a.gate[v0 + voff0] : (uint16_t)0;
  const float bt0 = bbase[(uint32_t)min((int)threadIdx.x, Tb - 1) * (uint32_t)a.H];
  __builtin_amdgcn_sched_barrier(0);  // keep the issue order: inputs, then state
  float4 s[C][NV];
  load_tile<DK, C, kVerifyLoadStream>(s, S, L);

  // stage the chunk's inputs; in replay mode also copy them to the buffer. The
  // copies of the first round go out at the end of the kernel: stores share the
  // load counter, and a store issued behind the state loads can make a later
  // wait (for a staging load, or for a register the store still reads) wait
  // for the state too.
  auto put_kq = [&](int idx, uint2 kb, uint2 qb, float4 al) {
    const int t = idx / (DK / 4), i = (idx % (DK / 4)) * 4;
    *reinterpret_cast<float4 *>(st.k(t) + i) = unpack_bf16x4(kb);
    *reinterpret_cast<float4 *>(st.q(t) + i) = unpack_bf16x4(qb);
    *reinterpret_cast<float4 *>(st.a(t) + i) = al;
  };
  const int64_t r0 = (int64_t)u.b * a.T_max * a.H + u.h;  // replay buffer: row b, token 0, head h
  auto copy_kq = [&](int idx, uint2 kb, float4 al) {
    if (replay && u.tile == 0) {
      const uint32_t d = kq_off(idx);
      *reinterpret_cast<uint2 *>(a.rk + r0 * DK + d) = kb;
      *reinterpret_cast<float4 *>(a.ralpha + r0 * DK + d) = al;
    }
  };
  auto put_v = [&](int t, uint16_t vb, uint16_t gb) {
    st.v[t * W + sv] = bf16_to_f32(vb);
    if constexpr (GATE) st.g[t * W + jj] = bf16_to_f32(gb);
  };
  auto copy_v = [&](int t, uint16_t vb) {
    if (replay) a.rv[r0 * a.dv + (int64_t)u.tile * W + v_off(t)] = vb;
  };
  if ((int)threadIdx.x < nkq) put_kq(threadIdx.x, kb0, qb0, al0);
  if (tv0 < Tb) put_v(tv0, vb0, gb0);
  if ((int)threadIdx.x < Tb) st.beta[threadIdx.x] = bt0;
  // further rounds (more than blockDim.x staging items)
  for (int idx = threadIdx.x + blockDim.x; idx < nkq; idx += blockDim.x) {
    const uint32_t off = kq_off(idx);
    const uint2 kb = *reinterpret_cast<const uint2 *>(kbase + off), qb = *reinterpret_cast<const uint2 *>(qbase + off);
    const float4 al = *reinterpret_cast<const float4 *>(abase + off);
    put_kq(idx, kb, qb, al);
    copy_kq(idx, kb, al);
  }
  for (int t = tv0 + tstep; t < Tb; t += tstep) {
    const uint16_t vb = vbase[v_off(t)];
    put_v(t, vb, GATE ? a.gate[v0 + v_off(t)] : (uint16_t)0);
    copy_v(t, vb);
  }
  __syncthreads();
  if constexpr (RAW) {
    prep_staged<DK, Staged<DK>::kRec>(st.k(0), st.q(0), st.a(0), st.beta, Tb);
    __syncthreads();
  }

  float keep[C];
#pragma unroll
  for (int c = 0; c < C; ++c) keep[c] = 0.0f;
  const lds_float *pk = to_lds(st.rec) + 4 * L.r;
  const lds_float *pv = to_lds(st.v) + L.col0 * C;
  for (int t = 0; t < Tb; ++t) {
    float4 kk[NV], qq[NV], aa[NV];
#pragma unroll
    for (int e = 0; e < NV; ++e) {
      kk[e] = lds_f4(pk + 64 * e);
      aa[e] = lds_f4(pk + DK + 64 * e);
      qq[e] = lds_f4(pk + 2 * DK + 64 * e);
    }
    float vj[C];
    load_v<C>(pv, vj);
    token_update<NV, C>(s, aa, kk, vj, st.beta[t]);
    float o[C];
    token_readout<NV, C>(s, qq, o);
    const bool mine = L.r == t;
#pragma unroll
    for (int c = 0; c < C; ++c) keep[c] = mine ? o[c] : keep[c];
    if constexpr (PERPOS) {
      if (!inplace) {
        float *D = a.draft + ((((int64_t)u.b * a.T_max + t) * a.H + u.h) * a.dv + (int64_t)u.tile * W) * DK;
        store_tile<DK, C, kVerifyStoreStream>(D, s, L);
      }
    }
    pk += Staged<DK>::kRec;
    pv += W;
  }
  if (inplace) store_tile<DK, C, kVerifyStoreStream>(S, s, L);
  // outputs: lane r writes token r's columns at uniform base v0 plus a 32-bit offset
  float *out32 = a.out + v0;
  uint16_t *out16 = reinterpret_cast<uint16_t *>(a.out) + v0;
  const uint32_t ooff = (uint32_t)L.r * v_tok + (uint32_t)L.col0;
  auto put_o = [&](uint32_t off, float y) {
    if constexpr (BF16)
      out16[off] = f32_to_bf16(y);
    else
      out32[off] = y;
  };
  if constexpr (GATE) {
    // the gate's sum of squares over the head: per lane, then over the wave's
    // four rows (in the order (row 0 + row 1) + (row 2 + row 3)), then over the
    // waves after one barrier
    __shared__ float part[kMaxT * kMaxWaves];
    float ss = keep[0] * keep[0];
#pragma unroll
    for (int c = 1; c < C; ++c) ss = __builtin_fmaf(keep[c], keep[c], ss);
    ss = ss + __shfl_xor(ss, 16);
    ss = ss + __shfl_xor(ss, 32);
    if ((threadIdx.x & 63) < Tb) part[(threadIdx.x & 63) * kMaxWaves + (threadIdx.x >> 6)] = ss;
    __syncthreads();
    if (L.r < Tb) {
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const int j = L.col0 + c * L.slab;
        const float wj = a.weight ? a.weight[j] : 1.0f;
        put_o(ooff + c * L.slab, gate_apply(a, part + L.r * kMaxWaves, keep[c], st.g[L.r * W + j], wj));
      }
    }
  } else {
    if (L.r < Tb) {
#pragma unroll
      for (int c = 0; c < C; ++c) put_o(ooff + c * L.slab, keep[c]);
    }
  }
  // the first round's replay copies (see the staging above). With prepared
  // inputs they are read back from LDS (each staged value came from a bf16 or
  // fp32 input exactly; the bf16 ones return to their bits by truncation), so
  // no register stays live across the token loop; raw inputs were prepared in
  // place, so that variant keeps the raw values in registers.
  if ((int)threadIdx.x < nkq) {
    if constexpr (RAW) {
      copy_kq(threadIdx.x, kb0, al0);
    } else {
      const int t = threadIdx.x / (DK / 4), i = (threadIdx.x % (DK / 4)) * 4;
      const float4 kf = *reinterpret_cast<const float4 *>(st.k(t) + i);
      const uint2 kb = {(__float_as_uint(kf.x) >> 16) | (__float_as_uint(kf.y) & 0xffff0000u),
                        (__float_as_uint(kf.z) >> 16) | (__float_as_uint(kf.w) & 0xffff0000u)};
      copy_kq(threadIdx.x, kb, *reinterpret_cast<const float4 *>(st.a(t) + i));
    }
  }
  if (tv0 < Tb) copy_v(tv0, (uint16_t)(__float_as_uint(st.v[tv0 * W + sv]) >> 16));
  if ((int)threadIdx.x < Tb && replay && u.tile == 0)
    a.rbeta[r0 + (uint32_t)threadIdx.x * (uint32_t)a.H] = RAW ? bt0 : st.beta[threadIdx.x];
}


// ----------------------------------------------------------------------------
// Commit
// ----------------------------------------------------------------------------

// Row checks shared by the commit kernels; returns the accepted length, or -1
// when the row does not run.
__device__ __forceinline__ int commit_row(const Args &a, const Unit &u, int32_t &slot) {
  // The row's slot id, token range and accepted length are requested together
  // and checked after one wait: checked one by one, each load waited behind
  // the previous check's branch, a chain of scalar round trips ahead of the
  // state load.
  slot = a.slot_ids[u.b];
  int n = a.accepted[u.b];
  int32_t c0 = 0, c1 = a.T_max;
  if (a.cu) {
    c0 = a.cu[u.b];
    c1 = a.cu[u.b + 1];
  }
  wait_uniform3(slot, n, c0);
  const bool bad_slot = slot >= a.num_slots;
  // Without cu_seqlens every row's range is [0, T_max): it indexes no packed
  // array (the commit reads only its buffers), so n_tok does not bound it.
  const bool bad_range = a.cu && (c0 < 0 || c1 < c0 || c1 > a.n_tok || c1 - c0 > a.T_max);
  const bool bad_n = n < 0 || n > c1 - c0;
  if (slot < 0 || bad_slot || bad_range || bad_n) {
    if (slot >= 0) report(a.dev_err, u, bad_slot ? KDA_DEVERR_SLOT : bad_range ? KDA_DEVERR_SEQLEN : KDA_DEVERR_ACCEPTED);
    return -1;
  }
  return n;
}

// ReplaySSM commit: reload the committed state, replay the first n buffered
// tokens with the same column engine, store once.
//
// Staging order. With FIRST, every thread's first item of each input (k and
// alpha, v, beta) is requested before the state tile, at clamped, in-bounds
// indices, so the staging writes wait for the inputs alone and each wave then
// waits for its own tile in the token loop; otherwise the tile goes first and
// its latency overlaps the staging loads. Measured on MI355X: inputs first is
// faster once the grid takes more than one round of resident workgroups, and
// slower when all of them fit at once (B = 16, T = 8).
template <int DK, int C, bool FIRST>
__global__ __launch_bounds__(256) void commit_replay_kernel(Args a) {
  constexpr int NV = DK / 64;
  extern __shared__ float4 lds_dyn[];
  const Unit u = unit_of_block_rows(a.ntile, a.H, a.B);
  const Lane L = lane_geometry();
  int32_t slot;
  const int n = commit_row(a, u, slot);
  if (n <= 0) return;
  const int W = C * L.slab;
  Staged<DK> st(reinterpret_cast<float *>(lds_dyn), a.T_max, W);
  float *S = a.cache + (int64_t)slot * a.slot_stride + ((int64_t)u.h * a.dv + (int64_t)u.tile * W) * DK;
  const int tid = threadIdx.x, nkq = n * (DK / 4);
  const int vsh = __builtin_ctz(W), tstep = blockDim.x >> vsh, tv = tid >> vsh;
  const int jj = tid & (W - 1), sv = v_slot<C>(jj, L.slab);
  const int64_t row_h = (int64_t)u.b * a.T_max * a.H + u.h;  // (row, token 0, head) in [B][T_max][H]
  auto kq_at = [&](int idx) { return (row_h + (int64_t)(idx / (DK / 4)) * a.H) * DK + (idx % (DK / 4)) * 4; };
  auto v_at = [&](int t) { return (row_h + (int64_t)t * a.H) * a.dv + (int64_t)u.tile * W + jj; };
  auto put_kq = [&](int idx, uint2 kb, float4 al) {
    const int t = idx / (DK / 4), i = (idx % (DK / 4)) * 4;
    *reinterpret_cast<float4 *>(st.k(t) + i) = unpack_bf16x4(kb);
    *reinterpret_cast<float4 *>(st.a(t) + i) = al;
  };
  float4 s[C][NV];
  int idx1 = tid, tv1 = tv;  // first items the loops below still stage
  if constexpr (FIRST) {
    const int i0 = min(tid, nkq - 1);
    const uint2 kb = *reinterpret_cast<const uint2 *>(a.rk + kq_at(i0));
    const float4 al = *reinterpret_cast<const float4 *>(a.ralpha + kq_at(i0));
    const uint16_t vb = a.rv[v_at(min(tv, n - 1))];
    const float bt = a.rbeta[row_h + (int64_t)min(tid, n - 1) * a.H];
    __builtin_amdgcn_sched_barrier(0);  // keep the issue order: inputs, then state
    load_tile<DK, C, kCommitLoadStream>(s, S, L);
    if (tid < nkq) put_kq(tid, kb, al);
    if (tv < n) st.v[tv * W + sv] = bf16_to_f32(vb);
    if (tid < n) st.beta[tid] = bt;
    idx1 = tid + blockDim.x;
    tv1 = tv + tstep;
  } else {
    load_tile<DK, C, kCommitLoadStream>(s, S, L);
  }
  for (int idx = idx1; idx < nkq; idx += blockDim.x)
    put_kq(idx, *reinterpret_cast<const uint2 *>(a.rk + kq_at(idx)),
           *reinterpret_cast<const float4 *>(a.ralpha + kq_at(idx)));
  for (int t = tv1; t < n; t += tstep) st.v[t * W + sv] = bf16_to_f32(a.rv[v_at(t)]);
  if constexpr (!FIRST) {
    if (tid < n) st.beta[tid] = a.rbeta[row_h + (int64_t)tid * a.H];
  }
  __syncthreads();
  if (a.raw) {
    prep_staged<DK, Staged<DK>::kRec>(st.k(0), nullptr, st.a(0), st.beta, n);
    __syncthreads();
  }

  const lds_float *pk = to_lds(st.rec) + 4 * L.r;
  const lds_float *pv = to_lds(st.v) + L.col0 * C;
  for (int t = 0; t < n; ++t) {
    float4 kk[NV], aa[NV];
#pragma unroll
    for (int e = 0; e < NV; ++e) {
      kk[e] = lds_f4(pk + 64 * e);
      aa[e] = lds_f4(pk + DK + 64 * e);
    }
    float vj[C];
    load_v<C>(pv, vj);
    token_update<NV, C>(s, aa, kk, vj, st.beta[t]);
    pk += Staged<DK>::kRec;
    pv += W;
  }
  store_tile<DK, C, kCommitStoreStream>(S, s, L);
}

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

template <int DK, int C, bool GATE, bool PERPOS>
struct verify_table {
  template <int IO>
  static const void *get() { return (const void *)verify_kernel<DK, C, GATE, IO, PERPOS>; }
};

template <int DK, bool PERPOS>
const void *verify_for(int C, bool gate, int io) {
  if (gate)
    return C == kGateSlabsVerify ? io_variant<verify_table<DK, kGateSlabsVerify, true, PERPOS>>(io) : nullptr;
  switch (C) {
    case 1: return io_variant<verify_table<DK, 1, false, PERPOS>>(io);
    case 2: return io_variant<verify_table<DK, 2, false, PERPOS>>(io);
    case 4: return io_variant<verify_table<DK, 4, false, PERPOS>>(io);
    case 8: return io_variant<verify_table<DK, 8, false, PERPOS>>(io);
  }
  return nullptr;
}

const void *verify_kernel_for(int dk, int C, bool gate, int io, bool perpos) {
  if (dk == 64) return perpos ? verify_for<64, true>(C, gate, io) : verify_for<64, false>(C, gate, io);
  if (dk == 128) return perpos ? verify_for<128, true>(C, gate, io) : verify_for<128, false>(C, gate, io);
  return nullptr;
}

template <int DK, bool FIRST>
const void *commit_replay_for(int C) {
  switch (C) {
    case 1: return (const void *)commit_replay_kernel<DK, 1, FIRST>;
    case 2: return (const void *)commit_replay_kernel<DK, 2, FIRST>;
    case 4: return (const void *)commit_replay_kernel<DK, 4, FIRST>;
    case 8: return (const void *)commit_replay_kernel<DK, 8, FIRST>;
  }
  return nullptr;
}

template <int DK>
const void *commit_copy_for(int C) {
  switch (C) {
    case 1: return (const void *)commit_copy_kernel<DK, 1>;
    case 2: return (const void *)commit_copy_kernel<DK, 2>;
    case 4: return (const void *)commit_copy_kernel<DK, 4>;
    case 8: return (const void *)commit_copy_kernel<DK, 8>;
  }
  return nullptr;
}

const void *commit_replay_kernel_for(int dk, int C, bool inputs_first) {
  if (dk == 64) return inputs_first ? commit_replay_for<64, true>(C) : commit_replay_for<64, false>(C);
  if (dk == 128) return inputs_first ? commit_replay_for<128, true>(C) : commit_replay_for<128, false>(C);
  return nullptr;
}

const void *commit_copy_kernel_for(int dk, int C) {
  return dk == 64 ? commit_copy_for<64>(C) : dk == 128 ? commit_copy_for<128>(C) : nullptr;
}

}  // namespace kda
