// kda.hip - HIP kernels for gfx950 and the C ABI declared in include/kda.h.
//
// The KDA recurrent-state step (taken as the gated delta rule with per-channel
// decay; the pages name the KDA recurrent state and its FP32 SSM cache in
// "Kimi K3 performance optimization in vLLM" and "Kimi K3 vLLM optimization:
// NVIDIA decode speed-up 1.68x", but do not write the update): per head,
//     S <- Diag(alpha) S ;  S <- S + beta k (v - S^T k)^T ;  o = S^T q .
//
// Work decomposition. One workgroup per (row, head, tile of W value columns).
// The cache stores each value column's dk key channels contiguously, so a tile
// is one contiguous span of W * dk floats. A column is owned by 16 lanes (one
// DPP row): lane r holds key channels 4r..4r+3 and, for dk = 128, also
// 64+4r..64+4r+3, as float4 registers. S^T k and S^T q are therefore a
// per-lane partial followed by a 16-lane DPP butterfly that leaves the same
// bits in every lane, and the rank-1 write needs no exchange at all. A wave
// covers 4 columns per slab; a lane holds C slabs, so W = 4 * waves * C.
//
// Bit-exactness. Every kernel runs the same column engine (token_update /
// token_readout) with explicit FMAs, the build disables contraction, and the
// reduction tree depends only on the lane's position in its row. The state
// after a token is therefore identical bit for bit across decode, verify,
// both commit modes and every tile width.
//
// Memory. At one token per row the step moves 2 * dk * dv * 4 bytes of state
// per head and ~1.3 KB of inputs, so it is HBM-bound: loads and stores are
// 128-bit and fully coalesced (each 16-lane row reads 256 contiguous bytes),
// and all of a lane's state loads are issued before the first use.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include "kda.h"

namespace {

constexpr int kMaxT = 16;
constexpr int kMaxWaves = 16;  // waves in the largest (1024-thread) workgroup
constexpr int kMaxDv = 128;
// Slabs per lane when the output gate makes one workgroup own all dv columns
// (waves = dv / (4 * slabs)); measured on MI355X.
constexpr int kGateSlabsDecode = 2;
constexpr int kGateSlabsVerify = 4;

struct Args {
  float *cache;
  int64_t num_slots, slot_stride;
  const int32_t *slot_ids;
  const int32_t *cu;       // packed row offsets [B + 1] (verify; commit may pass NULL)
  const int32_t *accepted; // commit
  const uint16_t *q, *k, *v, *gate;
  const float *alpha, *beta, *weight;
  float *out;
  int32_t *dev_err;
  uint16_t *rk, *rv;
  float *ralpha, *rbeta, *draft;
  const int32_t *ckpt_pos;  // prefill
  float *ckpt;
  float eps;
  int32_t B, H, dv, T_max, n_tok, ntile, mode, t1_inplace;
  int32_t raw;       // q, k, alpha, beta are raw projections (KDA_RAW_INPUTS)
  int32_t out_bf16;  // out holds bf16 (KDA_OUT_BF16)
};

// ----------------------------------------------------------------------------
// Column engine
// ----------------------------------------------------------------------------

__device__ __forceinline__ float bf16_to_f32(uint32_t bits) { return __uint_as_float(bits << 16); }

__device__ __forceinline__ float4 unpack_bf16x4(uint2 u) {
  return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                     __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over the 16 lanes of a DPP row. Each stage adds two partial sums that are
// the same pair in every lane (only the operand order differs), so all 16
// lanes end with identical bits.
__device__ __forceinline__ float row16_sum(float x) {
  x = x + dpp_f32<0xB1>(x);   // quad_perm(1,0,3,2): partner lane ^ 1
  x = x + dpp_f32<0x4E>(x);   // quad_perm(2,3,0,1): partner lane ^ 2
  x = x + dpp_f32<0x141>(x);  // row_half_mirror: the other quad of the half-row
  x = x + dpp_f32<0x140>(x);  // row_mirror: the other half of the row
  return x;
}

// This lane's share of dot(s, x) over its key channels, in a fixed order.
template <int NV>
__device__ __forceinline__ float lane_dot(const float4 (&s)[NV], const float4 (&x)[NV]) {
  float p = s[0].x * x[0].x;
  p = __builtin_fmaf(s[0].y, x[0].y, p);
  p = __builtin_fmaf(s[0].z, x[0].z, p);
  p = __builtin_fmaf(s[0].w, x[0].w, p);
#pragma unroll
  for (int e = 1; e < NV; ++e) {
    p = __builtin_fmaf(s[e].x, x[e].x, p);
    p = __builtin_fmaf(s[e].y, x[e].y, p);
    p = __builtin_fmaf(s[e].z, x[e].z, p);
    p = __builtin_fmaf(s[e].w, x[e].w, p);
  }
  return p;
}

// One token on C columns: decay rows by alpha, u = S^T k, S += k * beta (v - u).
template <int NV, int C>
__device__ __forceinline__ void token_update(float4 (&s)[C][NV], const float4 (&a)[NV],
                                             const float4 (&k)[NV], const float (&vj)[C],
                                             float beta) {
  float u[C];
#pragma unroll
  for (int c = 0; c < C; ++c) {
#pragma unroll
    for (int e = 0; e < NV; ++e) {
      s[c][e].x = s[c][e].x * a[e].x;
      s[c][e].y = s[c][e].y * a[e].y;
      s[c][e].z = s[c][e].z * a[e].z;
      s[c][e].w = s[c][e].w * a[e].w;
    }
    u[c] = lane_dot<NV>(s[c], k);
  }
#pragma unroll
  for (int c = 0; c < C; ++c) u[c] = row16_sum(u[c]);
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const float d = beta * (vj[c] - u[c]);
#pragma unroll
    for (int e = 0; e < NV; ++e) {
      s[c][e].x = __builtin_fmaf(k[e].x, d, s[c][e].x);
      s[c][e].y = __builtin_fmaf(k[e].y, d, s[c][e].y);
      s[c][e].z = __builtin_fmaf(k[e].z, d, s[c][e].z);
      s[c][e].w = __builtin_fmaf(k[e].w, d, s[c][e].w);
    }
  }
}

// Read-out on the updated state: o = S^T q, in every lane of the column's row.
template <int NV, int C>
__device__ __forceinline__ void token_readout(const float4 (&s)[C][NV], const float4 (&q)[NV],
                                              float (&o)[C]) {
#pragma unroll
  for (int c = 0; c < C; ++c) o[c] = lane_dot<NV>(s[c], q);
#pragma unroll
  for (int c = 0; c < C; ++c) o[c] = row16_sum(o[c]);
}

// One token on C columns with the read-out taken in the same pass as u:
// o = S_dec^T q + (k . q) delta, where S_dec is the decayed state. The state
// arithmetic (decay, u, delta, rank-1 write) is exactly token_update's, so the
// state matches the single-token step bit for bit; the read-out equals
// S_new^T q up to rounding, and its dot product no longer waits for the write.
template <int NV, int C>
__device__ __forceinline__ void token_fused(float4 (&s)[C][NV], const float4 (&a)[NV], const float4 (&k)[NV],
                                            const float4 (&q)[NV], const float (&vj)[C], float beta,
                                            float kq, float (&o)[C]) {
  float u[C], p[C];
#pragma unroll
  for (int c = 0; c < C; ++c) {
#pragma unroll
    for (int e = 0; e < NV; ++e) {
      s[c][e].x = s[c][e].x * a[e].x;
      s[c][e].y = s[c][e].y * a[e].y;
      s[c][e].z = s[c][e].z * a[e].z;
      s[c][e].w = s[c][e].w * a[e].w;
    }
    u[c] = lane_dot<NV>(s[c], k);
    p[c] = lane_dot<NV>(s[c], q);
  }
#pragma unroll
  for (int c = 0; c < C; ++c) {
    u[c] = row16_sum(u[c]);
    p[c] = row16_sum(p[c]);
  }
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const float d = beta * (vj[c] - u[c]);
#pragma unroll
    for (int e = 0; e < NV; ++e) {
      s[c][e].x = __builtin_fmaf(k[e].x, d, s[c][e].x);
      s[c][e].y = __builtin_fmaf(k[e].y, d, s[c][e].y);
      s[c][e].z = __builtin_fmaf(k[e].z, d, s[c][e].z);
      s[c][e].w = __builtin_fmaf(k[e].w, d, s[c][e].w);
    }
    o[c] = __builtin_fmaf(kq, d, p[c]);
  }
}

// ----------------------------------------------------------------------------
// Raw-input preparation
// ----------------------------------------------------------------------------
//
// With raw projections as inputs, each (token, head) is prepared before the
// recurrence: k and q are divided by their L2 norm over all dk channels (q is
// also scaled by 1/sqrt(dk)), alpha = exp(-softplus(a)) = 1 / (1 + e^a) and
// beta = sigmoid(b) = 1 / (1 + e^-b). It is the normalization and gate
// activation work that otherwise runs as separate small kernels ahead of the
// recurrence, fused in ("Hyper Optimizing Kimi K3 in vLLM", section "Finding
// time between operators"). Every op prepares through these functions on a
// 16-lane row with the column engine's channel layout, so the prepared values,
// and the states built from them, are the same bits in decode, verify, commit
// and prefill. The hardware exp2, reciprocal and reciprocal square root are
// each within about one ulp; exp's argument is a * log2(e) rounded to fp32.

constexpr float kLog2e = 1.44269504088896341f;

// x scaled by scale / sqrt(sum over the row's channels of x^2 + 1e-12)
template <int NV>
__device__ __forceinline__ void prep_normalize(float4 (&x)[NV], float scale) {
  const float f = __builtin_amdgcn_rsqf(row16_sum(lane_dot<NV>(x, x)) + 1e-12f) * scale;
#pragma unroll
  for (int e = 0; e < NV; ++e) {
    x[e].x = x[e].x * f;
    x[e].y = x[e].y * f;
    x[e].z = x[e].z * f;
    x[e].w = x[e].w * f;
  }
}

// 1 / (1 + e^x)
__device__ __forceinline__ float prep_sigmoid_neg(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x * kLog2e));
}

template <int NV>
__device__ __forceinline__ void prep_decay(float4 (&a)[NV]) {
#pragma unroll
  for (int e = 0; e < NV; ++e) {
    a[e].x = prep_sigmoid_neg(a[e].x);
    a[e].y = prep_sigmoid_neg(a[e].y);
    a[e].z = prep_sigmoid_neg(a[e].z);
    a[e].w = prep_sigmoid_neg(a[e].w);
  }
}

__device__ __forceinline__ float prep_beta(float b) { return prep_sigmoid_neg(-b); }

// In-place preparation of tokens [0, n) staged in LDS as float [t][DK] for k,
// alpha (and q when non-null) and beta [t]: one 16-lane row per token. Must be
// reached by the whole workgroup between two barriers.
template <int DK>
__device__ __forceinline__ void prep_staged(float *k, float *q, float *al, float *beta, int n) {
  constexpr int NV = DK / 64;
  const int rows = blockDim.x >> 4, r = threadIdx.x & 15;
  for (int t = threadIdx.x >> 4; t < n; t += rows) {
    float4 kk[NV], qq[NV], aa[NV];
#pragma unroll
    for (int e = 0; e < NV; ++e) {
      const int i = t * DK + 4 * r + 64 * e;
      kk[e] = *reinterpret_cast<const float4 *>(k + i);
      aa[e] = *reinterpret_cast<const float4 *>(al + i);
      if (q) qq[e] = *reinterpret_cast<const float4 *>(q + i);
    }
    prep_normalize<NV>(kk, 1.0f);
    prep_decay<NV>(aa);
    if (q) prep_normalize<NV>(qq, 1.0f / __builtin_sqrtf((float)DK));
#pragma unroll
    for (int e = 0; e < NV; ++e) {
      const int i = t * DK + 4 * r + 64 * e;
      *reinterpret_cast<float4 *>(k + i) = kk[e];
      *reinterpret_cast<float4 *>(al + i) = aa[e];
      if (q) *reinterpret_cast<float4 *>(q + i) = qq[e];
    }
    if (r == 0) beta[t] = prep_beta(beta[t]);
  }
}

// ----------------------------------------------------------------------------
// Work decomposition
// ----------------------------------------------------------------------------

struct Unit {
  int b, h, tile;
};

// Workgroups are dispatched round-robin over the 8 XCDs (workgroup n runs on
// XCD n % 8). Renumber them so each XCD gets a contiguous range of units: the
// tiles of one head then share their L2 for the head's k, q, alpha and beta.
__device__ __forceinline__ Unit unit_of_block(int ntile, int H) {
  const int n = blockIdx.x, N = gridDim.x;
  const int xcd = n & 7, local = n >> 3, per = N >> 3, rem = N & 7;
  const int u = xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
  Unit r;
  r.tile = u % ntile;
  const int bh = u / ntile;
  r.h = bh % H;
  r.b = bh / H;
  return r;
}

struct Lane {
  int r;     // position in the 16-lane row: key channels 4r..4r+3 (+ 64)
  int col0;  // tile-local value column of slab 0
  int slab;  // columns per slab = 4 * waves; slab c holds column col0 + c * slab
};

__device__ __forceinline__ Lane lane_geometry() {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  Lane L;
  L.r = lane & 15;
  L.col0 = wave * 4 + (lane >> 4);
  L.slab = (blockDim.x >> 6) * 4;
  return L;
}

__device__ __forceinline__ void report(int32_t *dev_err, const Unit &u, int bit) {
  if (dev_err && u.tile == 0 && u.h == 0 && threadIdx.x == 0) atomicOr(dev_err, bit);
}

__device__ __forceinline__ bool row_range(const Args &a, int b, int64_t &row0, int &Tb) {
  const int32_t c0 = a.cu[b], c1 = a.cu[b + 1];
  if (c0 < 0 || c1 < c0 || c1 > a.n_tok || c1 - c0 > a.T_max) return false;
  row0 = c0;
  Tb = c1 - c0;
  return true;
}

// 128-bit state accesses. STREAM marks an access that should not be kept in
// the caches (the "nt" hint): each state tile is touched once per call, and on
// MI355X streaming both the read and the write-back of the state measurably
// raises the sustained HBM rate of the single-token step.
typedef float v4f __attribute__((ext_vector_type(4)));

template <bool STREAM>
__device__ __forceinline__ float4 ld4(const float *p) {
  if constexpr (STREAM) {
    const v4f t = __builtin_nontemporal_load(reinterpret_cast<const v4f *>(p));
    return make_float4(t.x, t.y, t.z, t.w);
  } else {
    return *reinterpret_cast<const float4 *>(p);
  }
}

template <bool STREAM>
__device__ __forceinline__ void st4(float *p, const float4 &x) {
  if constexpr (STREAM) {
    const v4f t = {x.x, x.y, x.z, x.w};
    __builtin_nontemporal_store(t, reinterpret_cast<v4f *>(p));
  } else {
    *reinterpret_cast<float4 *>(p) = x;
  }
}

template <int DK, int C, bool STREAM>
__device__ __forceinline__ void load_tile(float4 (&s)[C][DK / 64], const float *base, const Lane &L) {
#pragma unroll
  for (int c = 0; c < C; ++c)
#pragma unroll
    for (int e = 0; e < DK / 64; ++e)
      s[c][e] = ld4<STREAM>(base + (int64_t)(L.col0 + c * L.slab) * DK + 4 * L.r + 64 * e);
}

template <int DK, int C, bool STREAM>
__device__ __forceinline__ void store_tile(float *base, const float4 (&s)[C][DK / 64], const Lane &L) {
#pragma unroll
  for (int c = 0; c < C; ++c)
#pragma unroll
    for (int e = 0; e < DK / 64; ++e)
      st4<STREAM>(base + (int64_t)(L.col0 + c * L.slab) * DK + 4 * L.r + 64 * e, s[c][e]);
}

// Cache policy of each state stream (measured on MI355X).
constexpr bool kDecodeLoadStream = true;    // slot state read by the single-token step
constexpr bool kDecodeStoreStream = true;   // slot state written back by it
constexpr bool kVerifyLoadStream = true;    // committed state read by verify
constexpr bool kVerifyStoreStream = true;   // per-position states and in-place rows written by verify
constexpr bool kCommitLoadStream = true;    // committed state reloaded by the replay commit
constexpr bool kCommitStoreStream = true;   // rebuilt state written by the replay commit
constexpr bool kCopyLoadStream = false;     // per-position state read by the copy commit
constexpr bool kCopyStoreStream = false;    // committed state written by the copy commit

__device__ __forceinline__ float readlane_f32(float x, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}

// Output gate over the head's whole value vector (the workgroup spans all of dv):
// y = o / sqrt(mean(o^2) + eps) * weight * sigmoid(gate).
//
// gate_partial: the wave's sum of squares of its columns' outputs (its four
// column groups in a fixed order), written to part[wave] by lane 0.
template <int C>
__device__ __forceinline__ void gate_partial(const float (&o)[C], float *part) {
  float ss = o[0] * o[0];
#pragma unroll
  for (int c = 1; c < C; ++c) ss = __builtin_fmaf(o[c], o[c], ss);
  const float wave_ss = (readlane_f32(ss, 0) + readlane_f32(ss, 16)) + (readlane_f32(ss, 32) + readlane_f32(ss, 48));
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = wave_ss;
}

// gate_apply: after a barrier, y for one column from the head's wave partials
// (summed over the waves in a fixed order), its raw output oc, its gate g and
// its weight w.
__device__ __forceinline__ float gate_apply(const Args &a, const float *part, float oc, float g, float w) {
  const int waves = blockDim.x >> 6;
  float tot = part[0];
  for (int i = 1; i < waves; ++i) tot += part[i];
  const float inv_rms = 1.0f / sqrtf(tot / (float)a.dv + a.eps);
  return oc * inv_rms * w * (1.0f / (1.0f + expf(-g)));
}

// Writes the C column outputs of each 16-lane row to dst[col0 + c * slab]: lane
// r == c stores column c (every lane of the row holds all C values).
template <int C>
__device__ __forceinline__ void store_cols(float *dst, const Lane &L, const float (&o)[C]) {
#pragma unroll
  for (int c = 0; c < C; ++c)
    if (L.r == c) dst[L.col0 + c * L.slab] = o[c];
}

// fp32 to bf16, round to nearest even (NaN stays a quiet NaN)
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  const uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// Output element idx of out: bf16 or fp32. Kernels on the hot paths pass a
// compile-time bf16 (a run-time choice costs them registers and occupancy).
__device__ __forceinline__ void put_out(const Args &a, bool bf16, int64_t idx, float y) {
  if (bf16)
    reinterpret_cast<uint16_t *>(a.out)[idx] = f32_to_bf16(y);
  else
    a.out[idx] = y;
}

// store_cols into out at element base
template <int C>
__device__ __forceinline__ void store_out(const Args &a, bool bf16, int64_t base, const Lane &L,
                                          const float (&o)[C]) {
#pragma unroll
  for (int c = 0; c < C; ++c)
    if (L.r == c) put_out(a, bf16, base + L.col0 + c * L.slab, o[c]);
}

// Input/output variant of the decode and verify kernels: bit 0 = raw inputs,
// bit 1 = bf16 output.
constexpr int kIoRaw = 1, kIoBf16 = 2;

// ----------------------------------------------------------------------------
// Kernels
// ----------------------------------------------------------------------------

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

// Dynamic LDS bytes for Staged<dk>, rounded up to 16.
inline size_t staged_bytes(int dk, int T_max, int W, bool gate) {
  return ((size_t)T_max * (3 * dk + W + 1 + (gate ? W : 0)) * sizeof(float) + 15) / 16 * 16;
}

// Speculative verify over a packed chunk: T_b tokens with the state in
// registers; outputs per token; the committed slot stays untouched unless the
// row is a single in-place token.
template <int DK, int C, bool GATE, int IO>
__global__ __launch_bounds__(GATE ? 1024 : 256) void verify_kernel(Args a) {
  constexpr int NV = DK / 64;
  constexpr bool RAW = IO & kIoRaw, BF16 = IO & kIoBf16;
  extern __shared__ float4 lds_dyn[];
  const Unit u = unit_of_block(a.ntile, a.H);
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

  float *S = a.cache + (int64_t)slot * a.slot_stride + ((int64_t)u.h * a.dv + (int64_t)u.tile * W) * DK;
  float4 s[C][NV];
  load_tile<DK, C, kVerifyLoadStream>(s, S, L);
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

inline size_t prefill_lds_bytes(int dk, int W) {
  const int floats = dk == 64 ? prefill_buf_floats<64>(W) : prefill_buf_floats<128>(W);
  return (2 * (size_t)floats * sizeof(float) + 15) / 16 * 16;
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

template <int DK, int C>
__device__ __forceinline__ void prefill_token_step(const Args &a, float4 (&s)[C][DK / 64],
                                                   const PrefillToken<DK / 64, C> &x, int64_t row, const Unit &u,
                                                   int W, const Lane &L) {
  float o[C];
  token_fused<DK / 64, C>(s, x.a, x.k, x.q, x.v, x.beta, x.kq, o);
  store_out<C>(a, a.out_bf16 != 0, (row * a.H + u.h) * a.dv + (int64_t)u.tile * W, L, o);
}

template <int DK, int C>
__global__ __launch_bounds__(256) void prefill_kernel(Args a) {
  constexpr int NV = DK / 64;
  constexpr int W = 16 * C;  // 4 waves x 4 columns x C slabs
  extern __shared__ float4 lds_dyn[];
  const Unit u = unit_of_block(a.ntile, a.H);
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
    if (a.raw) {
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
      prefill_token_step<DK, C>(a, s, ta, c0 + t0 + t, u, W, L);
      if (t0 + t + 1 == ck) store_tile<DK, C, kVerifyStoreStream>(CK, s, L);
      if (!pair) break;
      if (t + 2 < n) prefill_token_read<DK, C>(B, t + 2, W, L, ta);
      prefill_token_step<DK, C>(a, s, tb, c0 + t0 + t + 1, u, W, L);
      if (t0 + t + 2 == ck) store_tile<DK, C, kVerifyStoreStream>(CK, s, L);
    }
  }
  store_tile<DK, C, kVerifyStoreStream>(S, s, L);
}

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

constexpr int kChunkW = 64;     // value columns per workgroup of the chunk kernel
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

inline size_t chunk_lds_bytes(int dk, int T_max) {
  const size_t floats = (size_t)3 * T_max * dk + (size_t)T_max * kChunkW + kChunkRows +
                        (size_t)2 * dk * kChunkRows + 2 * kChunkRows * kChunkRows + 2 * kChunkRows * kChunkW;
  return (floats * sizeof(float) + 15) / 16 * 16;
}

template <int DK>
__global__ __launch_bounds__(256) void verify_chunk_kernel(Args a) {
  constexpr int NCB = DK / 16;  // 16-channel blocks
  constexpr int CPT = DK / 16;  // channels per thread in the coupling pass
  extern __shared__ float4 lds_dyn[];
  const Unit u = unit_of_block(a.ntile, a.H);
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
  const Unit u = unit_of_block(a.ntile, a.H);
  int32_t slot;
  const int n = commit_row(a, u, slot);
  if (n <= 0) return;
  const Lane L = lane_geometry();
  const int W = C * L.slab;
  Staged<DK> st(reinterpret_cast<float *>(lds_dyn), a.T_max, W);
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

  float *S = a.cache + (int64_t)slot * a.slot_stride + ((int64_t)u.h * a.dv + (int64_t)u.tile * W) * DK;
  float4 s[C][NV];
  load_tile<DK, C, kCommitLoadStream>(s, S, L);
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
  const Unit u = unit_of_block(a.ntile, a.H);
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

// ----------------------------------------------------------------------------
// State transfer (pack / unpack)
// ----------------------------------------------------------------------------
//
// For prefill/decode disaggregation and offload ("Prefill/Decode
// disaggregation and hybrid state offload": the KDA state is split by head
// and by dimension and boundary states are kept outside the GPU): the heads
// [head0, head0 + nheads) and value columns [col0, col0 + ncols) of each row's
// slot are copied to or from buf[b][nheads][ncols][dk]. Within one head the
// selected columns are one contiguous span of ncols * dk floats, so each
// workgroup streams one (row, head) span with 128-bit accesses. buf may be
// pinned host memory: the kernel then reads or writes it over PCIe directly.

struct PackArgs {
  float *cache;
  int64_t num_slots, slot_stride;
  const int32_t *slot_ids;
  float *buf;
  int32_t *dev_err;
  int32_t H, dk, dv, head0, nheads, col0, ncols;
};

template <bool PACK>
__global__ __launch_bounds__(256) void state_copy_kernel(PackArgs p) {
  const int b = blockIdx.x / p.nheads, hh = blockIdx.x % p.nheads;
  const int32_t slot = p.slot_ids[b];
  if (slot < 0) return;
  if (slot >= p.num_slots) {
    if (p.dev_err && hh == 0 && threadIdx.x == 0) atomicOr(p.dev_err, KDA_DEVERR_SLOT);
    return;
  }
  float *src = p.cache + (int64_t)slot * p.slot_stride + ((int64_t)(p.head0 + hh) * p.dv + p.col0) * p.dk;
  float *dst = p.buf + ((int64_t)b * p.nheads + hh) * (int64_t)p.ncols * p.dk;
  if (!PACK) {
    float *t = src;
    src = dst;
    dst = t;
  }
  const int n4 = p.ncols * p.dk / 4;
  for (int i = threadIdx.x; i < n4; i += blockDim.x)
    reinterpret_cast<float4 *>(dst)[i] = reinterpret_cast<const float4 *>(src)[i];
}

// ----------------------------------------------------------------------------
// Host side: checks, launch shape, dispatch
// ----------------------------------------------------------------------------

enum Kind { KIND_DECODE, KIND_VERIFY, KIND_COMMIT_REPLAY, KIND_COMMIT_COPY, KIND_PREFILL };

// Gated launches use a fixed number of slabs per lane for each op (see
// choose_width); only those are instantiated with the gate.
// The four input/output variants of one decode or verify kernel.
template <int DK, int C, bool GATE>
struct decode_table {
  template <int IO>
  static const void *get() { return (const void *)decode_kernel<DK, C, GATE, IO>; }
};
template <int DK, int C, bool GATE>
struct verify_table {
  template <int IO>
  static const void *get() { return (const void *)verify_kernel<DK, C, GATE, IO>; }
};
template <class T>
const void *io_variant(int io) {
  switch (io) {
    case 0: return T::template get<0>();
    case kIoRaw: return T::template get<kIoRaw>();
    case kIoBf16: return T::template get<kIoBf16>();
    case kIoRaw | kIoBf16: return T::template get<kIoRaw | kIoBf16>();
  }
  return nullptr;
}

template <int DK, int C>
const void *kernel_for(Kind kind, bool gate, int io) {
  if constexpr (C == kGateSlabsDecode)
    if (gate && kind == KIND_DECODE) return io_variant<decode_table<DK, C, true>>(io);
  if constexpr (C == kGateSlabsVerify)
    if (gate && kind == KIND_VERIFY) return io_variant<verify_table<DK, C, true>>(io);
  if (gate) return nullptr;
  switch (kind) {
    case KIND_DECODE:
      return io_variant<decode_table<DK, C, false>>(io);
    case KIND_VERIFY:
      return io_variant<verify_table<DK, C, false>>(io);
    case KIND_COMMIT_REPLAY:
      return (const void *)commit_replay_kernel<DK, C>;
    case KIND_COMMIT_COPY:
      return (const void *)commit_copy_kernel<DK, C>;
    case KIND_PREFILL:
      return nullptr;  // launched directly by kda_prefill
  }
  return nullptr;
}

template <int DK>
const void *kernel_for_c(Kind kind, bool gate, int io, int C) {
  switch (C) {
    case 1: return kernel_for<DK, 1>(kind, gate, io);
    case 2: return kernel_for<DK, 2>(kind, gate, io);
    case 4: return kernel_for<DK, 4>(kind, gate, io);
    case 8: return kernel_for<DK, 8>(kind, gate, io);
  }
  return nullptr;
}

struct Launch {
  int W, waves, C;
};

// Legal tile widths and their (waves, slabs per lane).
bool launch_of_width(int W, Launch *l) {
  switch (W) {
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
//    pure stream and one-wave workgroups of 4 columns sustain the highest rate;
//  * verify and replay commit (T tokens per row, VALU-heavy): 32 columns while
//    that gives at least 512 workgroups, narrower tiles below that;
//  * per-position copy commit: 16 columns.
int choose_width(Kind kind, int64_t rows, int H, int dv, bool gate, int requested, Launch *l) {
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
      if (heads * (dv / W) > 1024) W = 4;
      break;
    case KIND_VERIFY:
    case KIND_COMMIT_REPLAY:
      W = 8;
      for (int cand : {32, 16}) {
        if (cand <= dv && heads * (dv / cand) >= 512) {
          W = cand;
          break;
        }
      }
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
  const void *fn = dk == 64 ? kernel_for_c<64>(kind, gate, io, l.C) : kernel_for_c<128>(kind, gate, io, l.C);
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
  if (f & ~(int32_t)(KDA_RAW_INPUTS | KDA_OUT_BF16)) return KDA_ERR_INVALID;
  a.raw = (f & used & KDA_RAW_INPUTS) ? 1 : 0;
  a.out_bf16 = (f & used & KDA_OUT_BF16) ? 1 : 0;
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

extern "C" {

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
  KDA_TRY(check_cache(cache, num_slots, slot_stride, H, dk, dv));
  if (n_tok > 0) KDA_TRY(check_inputs(q, k, v, alpha, beta, out, true, a.out_bf16));
  if (ckpt_pos) {
    if (!ckpt) return KDA_ERR_INVALID;
    if (!aligned(ckpt, 16) || !aligned(ckpt_pos, 4)) return KDA_ERR_ALIGN;
  }
  if (!aligned(cu_seqlens, 4) || (dev_err && !aligned(dev_err, 4))) return KDA_ERR_ALIGN;
  Launch l;
  KDA_TRY(choose_width(KIND_PREFILL, B, H, dv, false, opts ? opts->tile_w : 0, &l));

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
  const void *fn = nullptr;
  if (dk == 64) fn = l.C == 1 ? (const void *)prefill_kernel<64, 1> : (const void *)prefill_kernel<64, 2>;
  else fn = l.C == 1 ? (const void *)prefill_kernel<128, 1> : (const void *)prefill_kernel<128, 2>;
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
  KDA_TRY(check_cache(cache, num_slots, slot_stride, H, dk, dv));
  KDA_TRY(check_inputs(q, k, v, alpha, beta, out, true, a.out_bf16));
  KDA_TRY(check_gate(epi));
  if (dev_err && !aligned(dev_err, 4)) return KDA_ERR_ALIGN;
  Launch l;
  KDA_TRY(choose_width(KIND_DECODE, B, H, dv, epi != nullptr, opts ? opts->tile_w : 0, &l));

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
  const bool chunk_fits = mode == KDA_REPLAY && !t1_inplace && epi == nullptr && dv % kChunkW == 0 &&
                          !a.raw && !a.out_bf16;
  if (form == KDA_VERIFY_CHUNKED && (!chunk_fits || (opts && opts->tile_w != 0))) return KDA_ERR_UNSUPPORTED;
  // Measured on MI355X (B=16, H=32, d=128, 8 drafts): the chunk form takes ~31 us against
  // ~19 us token by token, so the automatic choice is the recurrent kernel.
  const bool chunked = form == KDA_VERIFY_CHUNKED;
  Launch l;
  if (chunked) {
    l = {kChunkW, 4, 0};
  } else {
    KDA_TRY(choose_width(KIND_VERIFY, B, H, dv, epi != nullptr, opts ? opts->tile_w : 0, &l));
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
    const void *fn = dk == 64 ? (const void *)verify_chunk_kernel<64> : (const void *)verify_chunk_kernel<128>;
    return launch_fn(fn, units, 256, chunk_lds_bytes(dk, T_max), a, stream);
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
  KDA_TRY(choose_width(mode == KDA_REPLAY ? KIND_COMMIT_REPLAY : KIND_COMMIT_COPY, B, H, dv, false,
                       opts ? opts->tile_w : 0, &l));

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
  KDA_TRY(choose_width(kind, B, H, dv, epilogue != 0, requested_tile_w, &l));
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
  const int64_t blocks = (int64_t)B * nheads;
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
  void *args[] = {&p};
  const void *fn = pack ? (const void *)state_copy_kernel<true> : (const void *)state_copy_kernel<false>;
  const hipError_t e = hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(256), args, 0, (hipStream_t)stream);
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
  }
  return "unknown status";
}

}  // extern "C"
