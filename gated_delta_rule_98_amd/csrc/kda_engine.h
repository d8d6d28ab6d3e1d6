// kda_engine.h - device building blocks shared by every KDA kernel (gfx950),
// and the internal interface between the kernel files and the C ABI in
// kda_api.hip.
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

#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kda.h"

namespace kda {

constexpr int kMaxT = 16;
constexpr int kMaxWaves = 16;  // waves in the largest (1024-thread) workgroup
constexpr int kMaxDv = 128;
// Slabs per lane when the output gate makes one workgroup own all dv columns
// (waves = dv / (4 * slabs)); measured on MI355X.
constexpr int kGateSlabsDecode = 2;
constexpr int kGateSlabsVerify = 2;

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

// Column pairs (the single-token step's stream shape at dk = 128): a column is
// owned by 32 lanes, an even DPP row and the odd row after it; lane r of the
// even row holds key channels 4r..4r+3 and lane r of the odd row 64+4r..64+4r+3,
// one float4 each, so a wave covers two columns, one contiguous 1 KiB span.
// gfx950's v_permlane16_swap exchanges rows 2m and 2m+1 of two registers; with
// the same register twice, its first result holds the even row's value in both
// rows and its second the odd row's.
__device__ __forceinline__ float from_even_row(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]);
}

__device__ __forceinline__ float from_odd_row(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[1]);
}

// dot(s, x) over a column pair's 128 channels with the same operations, in the
// same order, as row16_sum(lane_dot<2>(s, x)): the even row's four-term chain
// moves to the odd row, which continues it over its own channels and runs the
// butterfly; every lane receives the odd row's total. The even row's second
// chain and butterfly are discarded.
__device__ __forceinline__ float pair_dot(const float4 &s, const float4 &x) {
  float p = s.x * x.x;
  p = __builtin_fmaf(s.y, x.y, p);
  p = __builtin_fmaf(s.z, x.z, p);
  p = __builtin_fmaf(s.w, x.w, p);
  p = from_even_row(p);
  p = __builtin_fmaf(s.x, x.x, p);
  p = __builtin_fmaf(s.y, x.y, p);
  p = __builtin_fmaf(s.z, x.z, p);
  p = __builtin_fmaf(s.w, x.w, p);
  return from_odd_row(row16_sum(p));
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

// In-place preparation of tokens [0, n) staged in LDS as float [t][STRIDE]
// (first DK used) for k, alpha (and q when non-null) and beta [t]: one 16-lane
// row per token. Must be
// reached by the whole workgroup between two barriers.
template <int DK, int STRIDE = DK>
__device__ __forceinline__ void prep_staged(float *k, float *q, float *al, float *beta, int n) {
  constexpr int NV = DK / 64;
  const int rows = blockDim.x >> 4, r = threadIdx.x & 15;
  for (int t = threadIdx.x >> 4; t < n; t += rows) {
    float4 kk[NV], qq[NV], aa[NV];
#pragma unroll
    for (int e = 0; e < NV; ++e) {
      const int i = t * STRIDE + 4 * r + 64 * e;
      kk[e] = *reinterpret_cast<const float4 *>(k + i);
      aa[e] = *reinterpret_cast<const float4 *>(al + i);
      if (q) qq[e] = *reinterpret_cast<const float4 *>(q + i);
    }
    prep_normalize<NV>(kk, 1.0f);
    prep_decay<NV>(aa);
    if (q) prep_normalize<NV>(qq, 1.0f / __builtin_sqrtf((float)DK));
#pragma unroll
    for (int e = 0; e < NV; ++e) {
      const int i = t * STRIDE + 4 * r + 64 * e;
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

// x / d and x % d for a uniform d: shifts when d is a power of two (tile counts
// always are, head counts usually), so the unit numbering stays on the scalar
// unit instead of an emulated division in vector registers.
__device__ __forceinline__ void divmod_uniform(int x, int d, int &q, int &m) {
  if ((d & (d - 1)) == 0) {
    q = x >> __builtin_ctz(d);
    m = x & (d - 1);
  } else {
    q = x / d;
    m = x - q * d;
  }
}

__device__ __forceinline__ Unit unit_of_index(int u, int ntile, int H) {
  Unit r;
  int bh;
  divmod_uniform(u, ntile, bh, r.tile);
  divmod_uniform(bh, H, r.b, r.h);
  return r;
}

// Workgroups are dispatched round-robin over the 8 XCDs (workgroup n runs on
// XCD n % 8). Renumber them so each XCD gets a contiguous range of units: the
// tiles of one head then share their L2 for the head's k, q, alpha and beta.
__device__ __forceinline__ Unit unit_of_block(int ntile, int H) {
  const int n = blockIdx.x, N = gridDim.x;
  const int xcd = n & 7, local = n >> 3, per = N >> 3, rem = N & 7;
  const int u = xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
  return unit_of_index(u, ntile, H);
}

// For kernels whose rows carry unequal work (varying token counts, rows that
// skip): deal the (row, head) groups out to the XCDs in turn, so every XCD gets
// an equal share of each row while a group's tiles still share one L2. With a
// multiple of 8 heads, XCD x takes heads x, x + 8, ... of every row, in an
// order where the row varies fastest, so the groups resident at any moment mix
// every kind of row: memory-bound single-token rows overlap VALU-bound
// multi-token ones instead of running before them. Other head counts take
// groups 8j + x in row order; counts of groups that are not a multiple of 8
// use the contiguous numbering above.
__device__ __forceinline__ Unit unit_of_block_rows(int ntile, int H, int B) {
  if ((B * H) & 7) return unit_of_block(ntile, H);
  const int n = blockIdx.x, xcd = n & 7;
  int j, tile;
  divmod_uniform(n >> 3, ntile, j, tile);
  Unit r;
  r.tile = tile;
  if ((H & 7) == 0) {
    int jh;
    divmod_uniform(j, B, jh, r.b);
    r.h = (jh << 3) | xcd;
  } else {
    divmod_uniform((j << 3) | xcd, H, r.b, r.h);
  }
  return r;
}

// Verify's numbering: groups dealt to the XCDs in turn, head-major (group
// 8j + x is head (8j + x) / B of row (8j + x) % B), so XCD x takes whole rows
// x, x + 8, ... (each slot's heads together in HBM) and the rows it holds
// alternate in its dispatch order. Measured on the mixed batch (40 single-token
// rows then 24 four-token rows, output gate): 43.1 us against 45.5 us for the
// numbering above and 46.4 us for row order. Counts of groups that are not a
// multiple of 8 use the contiguous numbering.
__device__ __forceinline__ Unit unit_of_block_headmajor(int ntile, int H, int B) {
  if ((B * H) & 7) return unit_of_block(ntile, H);
  const int n = blockIdx.x;
  int j;
  Unit r;
  divmod_uniform(n >> 3, ntile, j, r.tile);
  divmod_uniform((j << 3) | (n & 7), B, r.h, r.b);
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

// An empty statement that takes three wave-uniform values in scalar registers:
// every use of them then follows it, so the loads that produce them are all
// issued first and waited for once (without it the compiler may place a use,
// and the wait it needs, between two of the loads).
__device__ __forceinline__ void wait_uniform3(int32_t &x, int32_t &y, int32_t &z) {
  asm volatile("" : "+s"(x), "+s"(y), "+s"(z));
}

// A row's slot id and packed token range, requested together and checked after
// one wait (checked one at a time, each load waits behind the previous check's
// branch: a chain of scalar round trips ahead of the state load). False for a
// row to skip: padding (slot < 0, nothing reported), a slot past the cache or
// a bad token range (reported to dev_err).
__device__ __forceinline__ bool row_slot_range(const Args &a, const Unit &u, int32_t &slot, int64_t &row0,
                                               int &Tb) {
  slot = a.slot_ids[u.b];
  int32_t c0 = a.cu[u.b], c1 = a.cu[u.b + 1];
  wait_uniform3(slot, c0, c1);
  const bool bad_slot = slot >= a.num_slots;
  const bool bad_range = c0 < 0 || c1 < c0 || c1 > a.n_tok || c1 - c0 > a.T_max;
  if (slot < 0 || bad_slot || bad_range) {
    if (slot >= 0) report(a.dev_err, u, bad_slot ? KDA_DEVERR_SLOT : KDA_DEVERR_SEQLEN);
    return false;
  }
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

// Arguments of the state pack / unpack kernel.
struct PackArgs {
  float *cache;
  int64_t num_slots, slot_stride;
  const int32_t *slot_ids;
  float *buf;
  int32_t *dev_err;
  int32_t H, dk, dv, head0, nheads, col0, ncols;
  int32_t parts;  // workgroups per (row, head) span
};

// ----------------------------------------------------------------------------
// Kernel tables
// ----------------------------------------------------------------------------
//
// Each kernel file instantiates its kernels and returns the host handle of one
// instantiation (for hipLaunchKernel), or nullptr for a combination it does
// not build. `io` is a kIo* bit set; `C` is the number of slabs per lane.

// The four input/output variants of one kernel: T::get<IO>() for IO in 0..3.
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

const void *decode_kernel_for(int dk, int C, bool gate, int io);    // kda_decode.hip
const void *decode_pair_kernel_for(int io);                         // kda_decode.hip, dk = 128
const void *verify_kernel_for(int dk, int C, bool gate, int io, bool perpos);  // kda_verify.hip
const void *commit_replay_kernel_for(int dk, int C, bool inputs_first);  // kda_verify.hip
const void *commit_copy_kernel_for(int dk, int C);                  // kda_verify.hip
const void *prefill_kernel_for(int dk, int C, int io);              // kda_prefill.hip
const void *state_copy_kernel_for(bool pack);                       // kda_state.hip
int state_copy_lanes();                                             // kda_state.hip: lanes per workgroup

// Dynamic LDS bytes of the kernels that take it.
size_t staged_bytes(int dk, int T_max, int W, bool gate);           // verify, replay commit
size_t prefill_lds_bytes(int dk, int W);                            // prefill

}  // namespace kda
