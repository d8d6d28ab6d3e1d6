// kda_prefill.hip - whole prompts in one pass with an in-pass checkpoint (kda_prefill).

#include "kda_engine.h"

namespace kda {
namespace {

// ----------------------------------------------------------------------------
// Prefill with an in-pass checkpoint
// ----------------------------------------------------------------------------
//
// One pass over each row's whole prompt from its slot ("Internal KDA prefix
// checkpoint"): outputs for every token, the final state written back, and the
// state after the first ckpt_pos[b] tokens exported inside the same loop.
// Tokens are staged through LDS in chunks of kPrefillChunk, double-buffered:
// the next chunk's loads are in flight while the current chunk computes.
// Workgroups are 256 threads (W = 16 or 32 value columns). The state update is
// the single-token step's, so a checkpoint after n tokens equals n decode steps
// bit for bit.

constexpr int kPrefillChunk = 16;

template <int DK>
struct PrefillBuf {
  float *k, *q, *a, *v, *beta, *kq;
  __device__ PrefillBuf(float *base, int W) {
    k = base;
    q = k + kPrefillChunk * DK;
    a = q + kPrefillChunk * DK;
    v = a + kPrefillChunk * DK;
    beta = v + kPrefillChunk * W;
    kq = beta + kPrefillChunk;
  }
};

// floats of one staging buffer: k, q, alpha, the tile's v, beta and k . q per token
template <int DK>
__host__ __device__ constexpr int prefill_buf_floats(int W) {
  return kPrefillChunk * (3 * DK + W + 2);
}


// A chunk's inputs held in registers between the global loads and the LDS writes.
template <int DK, int W>
struct PrefillRegs {
  static constexpr int MK = kPrefillChunk * (DK / 4) / 256;  // k/q/alpha quads per thread
  static constexpr int MV = (kPrefillChunk * W + 255) / 256;  // v entries per thread
  uint2 k[MK], q[MK];
  float4 a[MK];
  uint16_t v[MV];
  float beta;
};

template <int DK, int W>
__device__ __forceinline__ void prefill_fetch(const Args &a, int64_t row0, int n, int h, int tile,
                                              PrefillRegs<DK, W> &r) {
#pragma unroll
  for (int m = 0; m < PrefillRegs<DK, W>::MK; ++m) {
    const int idx = threadIdx.x + 256 * m;
    const int t = idx / (DK / 4), i = (idx % (DK / 4)) * 4;
    if (t < n) {
      const int64_t off = ((row0 + t) * a.H + h) * DK + i;
      r.k[m] = *reinterpret_cast<const uint2 *>(a.k + off);
      r.q[m] = *reinterpret_cast<const uint2 *>(a.q + off);
      r.a[m] = *reinterpret_cast<const float4 *>(a.alpha + off);
    }
  }
#pragma unroll
  for (int m = 0; m < PrefillRegs<DK, W>::MV; ++m) {
    const int idx = threadIdx.x + 256 * m;
    const int t = idx / W, jj = idx % W;
    if (t < n && idx < kPrefillChunk * W)
      r.v[m] = a.v[((row0 + t) * a.H + h) * a.dv + (int64_t)tile * W + jj];
  }
  if ((int)threadIdx.x < n) r.beta = a.beta[(row0 + threadIdx.x) * a.H + h];
}

template <int DK, int W>
__device__ __forceinline__ void prefill_stage(const PrefillRegs<DK, W> &r, int n, PrefillBuf<DK> &B) {
#pragma unroll
  for (int m = 0; m < PrefillRegs<DK, W>::MK; ++m) {
    const int idx = threadIdx.x + 256 * m;
    const int t = idx / (DK / 4), i = (idx % (DK / 4)) * 4;
    if (t < n) {
      *reinterpret_cast<float4 *>(B.k + t * DK + i) = unpack_bf16x4(r.k[m]);
      *reinterpret_cast<float4 *>(B.q + t * DK + i) = unpack_bf16x4(r.q[m]);
      *reinterpret_cast<float4 *>(B.a + t * DK + i) = r.a[m];
    }
  }
#pragma unroll
  for (int m = 0; m < PrefillRegs<DK, W>::MV; ++m) {
    const int idx = threadIdx.x + 256 * m;
    const int t = idx / W;
    if (t < n && idx < kPrefillChunk * W) B.v[idx] = bf16_to_f32(r.v[m]);
  }
  if ((int)threadIdx.x < n) B.beta[threadIdx.x] = r.beta;
}

// One token's inputs for a lane, read from the staged chunk.
template <int NV, int C>
struct PrefillToken {
  float4 k[NV], q[NV], a[NV];
  float v[C], beta, kq;
};

template <int DK, int C>
__device__ __forceinline__ void prefill_token_read(const PrefillBuf<DK> &B, int t, int W, const Lane &L,
                                                   PrefillToken<DK / 64, C> &x) {
#pragma unroll
  for (int e = 0; e < DK / 64; ++e) {
    const int i = t * DK + 4 * L.r + 64 * e;
    x.k[e] = *reinterpret_cast<const float4 *>(B.k + i);
    x.q[e] = *reinterpret_cast<const float4 *>(B.q + i);
    x.a[e] = *reinterpret_cast<const float4 *>(B.a + i);
  }
#pragma unroll
  for (int c = 0; c < C; ++c) x.v[c] = B.v[t * W + L.col0 + c * L.slab];
  x.beta = B.beta[t];
  x.kq = B.kq[t];
}

template <int DK, int C, bool BF16>
__device__ __forceinline__ void prefill_token_step(const Args &a, float4 (&s)[C][DK / 64],
                                                   const PrefillToken<DK / 64, C> &x, int64_t row, const Unit &u,
                                                   int W, const Lane &L) {
  float o[C];
  token_fused<DK / 64, C>(s, x.a, x.k, x.q, x.v, x.beta, x.kq, o);
  store_out<C>(a, BF16, (row * a.H + u.h) * a.dv + (int64_t)u.tile * W, L, o);
}

template <int DK, int C, int IO>
__global__ __launch_bounds__(256) void prefill_kernel(Args a) {
  constexpr int NV = DK / 64;
  constexpr bool RAW = IO & kIoRaw, BF16 = IO & kIoBf16;
  constexpr int W = 16 * C;  // 4 waves x 4 columns x C slabs
  extern __shared__ float4 lds_dyn[];
  const Unit u = unit_of_block_rows(a.ntile, a.H, a.B);
  const int32_t slot = a.slot_ids[u.b];
  if (slot < 0) return;
  if (slot >= a.num_slots) {
    report(a.dev_err, u, KDA_DEVERR_SLOT);
    return;
  }
  const int32_t c0 = a.cu[u.b], c1 = a.cu[u.b + 1];
  if (c0 < 0 || c1 < c0 || c1 > a.n_tok) {
    report(a.dev_err, u, KDA_DEVERR_SEQLEN);
    return;
  }
  const int Tb = c1 - c0;
  const int ck = a.ckpt_pos ? a.ckpt_pos[u.b] : -1;
  if (ck > Tb) {
    report(a.dev_err, u, KDA_DEVERR_CKPT);
    return;
  }
  if (Tb == 0 && ck != 0) return;
  const Lane L = lane_geometry();
  float *S = a.cache + (int64_t)slot * a.slot_stride + ((int64_t)u.h * a.dv + (int64_t)u.tile * W) * DK;
  float *CK = ck >= 0 ? a.ckpt + (((int64_t)u.b * a.H + u.h) * a.dv + (int64_t)u.tile * W) * DK : nullptr;
  float4 s[C][NV];
  load_tile<DK, C, kVerifyLoadStream>(s, S, L);
  if (ck == 0) store_tile<DK, C, kVerifyStoreStream>(CK, s, L);
  if (Tb == 0) return;

  // the two LDS buffers are addressed from the shared base each chunk (an array of
  // buffer views indexed at run time would live in scratch and lose the LDS address space)
  float *const lds = reinterpret_cast<float *>(lds_dyn);
  constexpr int kBufFloats = prefill_buf_floats<DK>(W);
  const int nchunks = (Tb + kPrefillChunk - 1) / kPrefillChunk;
  PrefillRegs<DK, W> regs;
  prefill_fetch<DK, W>(a, c0, min(kPrefillChunk, Tb), u.h, u.tile, regs);
  for (int ci = 0; ci < nchunks; ++ci) {
    const int t0 = ci * kPrefillChunk;
    const int n = min(kPrefillChunk, Tb - t0);
    PrefillBuf<DK> B(lds + (ci & 1) * kBufFloats, W);
    prefill_stage<DK, W>(regs, n, B);
    __syncthreads();
    if (ci + 1 < nchunks)
      prefill_fetch<DK, W>(a, c0 + t0 + kPrefillChunk, min(kPrefillChunk, Tb - t0 - kPrefillChunk), u.h, u.tile,
                           regs);
    // k . q per token, once per workgroup: thread (t, chunk of DK / 16 channels), a
    // 16-lane row per token. Raw inputs are prepared in the same pass (one row per
    // token, the column engine's channel layout) and k . q taken on the prepared values.
    if constexpr (RAW) {
      const int t = threadIdx.x >> 4, r = threadIdx.x & 15;
      if (t < n) {
        float4 kk[NV], qq[NV], aa[NV];
#pragma unroll
        for (int e = 0; e < NV; ++e) {
          const int i = t * DK + 4 * r + 64 * e;
          kk[e] = *reinterpret_cast<const float4 *>(B.k + i);
          qq[e] = *reinterpret_cast<const float4 *>(B.q + i);
          aa[e] = *reinterpret_cast<const float4 *>(B.a + i);
        }
        prep_normalize<NV>(kk, 1.0f);
        prep_normalize<NV>(qq, 1.0f / __builtin_sqrtf((float)DK));
        prep_decay<NV>(aa);
        const float kq = row16_sum(lane_dot<NV>(kk, qq));
#pragma unroll
        for (int e = 0; e < NV; ++e) {
          const int i = t * DK + 4 * r + 64 * e;
          *reinterpret_cast<float4 *>(B.k + i) = kk[e];
          *reinterpret_cast<float4 *>(B.q + i) = qq[e];
          *reinterpret_cast<float4 *>(B.a + i) = aa[e];
        }
        if (r == 0) {
          B.kq[t] = kq;
          B.beta[t] = prep_beta(B.beta[t]);
        }
      }
    } else {
      constexpr int CPT = DK / 16;
      const int t = threadIdx.x >> 4, c = threadIdx.x & 15;
      float p = 0.0f;
      if (t < n) {
#pragma unroll
        for (int e = 0; e < CPT; ++e) p = __builtin_fmaf(B.k[t * DK + c * CPT + e], B.q[t * DK + c * CPT + e], p);
      }
      p = row16_sum(p);
      if (c == 0 && t < n) B.kq[t] = p;
    }
    __syncthreads();
    // tokens in pairs: the second token's LDS reads are issued before the first computes
    PrefillToken<NV, C> ta, tb;
    prefill_token_read<DK, C>(B, 0, W, L, ta);
    for (int t = 0; t < n; t += 2) {
      const bool pair = t + 1 < n;
      if (pair) prefill_token_read<DK, C>(B, t + 1, W, L, tb);
      prefill_token_step<DK, C, BF16>(a, s, ta, c0 + t0 + t, u, W, L);
      if (t0 + t + 1 == ck) store_tile<DK, C, kVerifyStoreStream>(CK, s, L);
      if (!pair) break;
      if (t + 2 < n) prefill_token_read<DK, C>(B, t + 2, W, L, ta);
      prefill_token_step<DK, C, BF16>(a, s, tb, c0 + t0 + t + 1, u, W, L);
      if (t0 + t + 2 == ck) store_tile<DK, C, kVerifyStoreStream>(CK, s, L);
    }
  }
  store_tile<DK, C, kVerifyStoreStream>(S, s, L);
}

}  // namespace

size_t prefill_lds_bytes(int dk, int W) {
  const int floats = dk == 64 ? prefill_buf_floats<64>(W) : prefill_buf_floats<128>(W);
  return (2 * (size_t)floats * sizeof(float) + 15) / 16 * 16;
}

template <int DK, int C>
struct prefill_table {
  template <int IO>
  static const void *get() { return (const void *)prefill_kernel<DK, C, IO>; }
};

const void *prefill_kernel_for(int dk, int C, int io) {
  if (dk == 64) return C == 1 ? io_variant<prefill_table<64, 1>>(io) : C == 2 ? io_variant<prefill_table<64, 2>>(io) : nullptr;
  if (dk == 128) return C == 1 ? io_variant<prefill_table<128, 1>>(io) : C == 2 ? io_variant<prefill_table<128, 2>>(io) : nullptr;
  return nullptr;
}

}  // namespace kda
