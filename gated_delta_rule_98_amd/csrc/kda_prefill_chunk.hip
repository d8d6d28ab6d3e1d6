// kda_prefill_chunk.hip - the chunk form of prefill (kda_prefill_chunked).
//
// The prompt of each row is cut into chunks of L = 32 tokens (a row with a
// checkpoint strictly inside it is cut at the checkpoint first, so the state
// there falls on a chunk boundary). Within a chunk, with S0 the state entering
// it, Gamma_t the product of the decays of tokens 1..t of the chunk and
// D(t, s) = prod_{s < r <= t} alpha_r (elementwise over key channels), the
// token-by-token recurrence unrolls to
//   u_t     = S0^T (Gamma_t k_t) + sum_{s<t} A_ts delta_s,  A_ts = sum_i k_t,i D(t,s)_i k_s,i
//   delta_t = beta_t (v_t - u_t)
//   o_t     = S0^T (Gamma_t q_t) + sum_{s<=t} B_ts delta_s, B_ts = sum_i q_t,i D(t,s)_i k_s,i
//   S_L     = Diag(Gamma_L) S0 + sum_s (k_s D(L,s)) delta_s^T
// Solving the lower-triangular system once per chunk, T = (I + Diag(beta) A)^-1
// Diag(beta), gives delta = U - W S0 with W = T [Gamma k] and U = T V: every
// product with the state becomes a dense matrix product.
//
// Three kernels. A one-workgroup map numbers the chunks of all rows. The
// precompute runs once per (chunk, head), all chunks in parallel, and leaves
// W, U, [Gamma q], the keys decayed to the chunk end, B and Gamma_L in a
// caller-provided workspace, each in the order the state pass reads it. The
// state pass runs per (row, head, 16 value columns) through the row's chunks
// in order, with the state in MFMA accumulator registers:
//   delta = U - W S0 ;  o = [Gamma q] S0 + B delta ;  S0 <- Diag(Gamma_L) S0 + Kt^T delta
// The products with the state run on four waves split by key channel, and two
// other waves finish the outputs a barrier later.
//
// Products with the state on the bfloat16 matrix cores. gfx950 has no
// reduced-precision fp32 (xf32) MFMA, and its fp32 one, v_mfma_f32_16x16x4f32,
// issues every 32 cycles for 1,024 multiply-adds, while v_mfma_f32_16x16x32_bf16
// issues every 16 cycles for 8,192 (both measured on MI355X). Each fp32 operand
// x is split into bfloat16 parts, hi = RNE(x) and lo = RNE(x - hi) (x - hi is
// exact), so that x = hi + lo to within 2^-18 |x|, and a product is taken as
// a_lo b_hi + a_hi b_lo + a_hi b_hi with fp32 accumulation: each term is exact
// in fp32 and the dropped a_lo b_lo is below 2^-18 |a b|, so a product is off
// by at most about 3 2^-18 (1.2e-5) of |a b|, where fp32 products are off by
// 2^-24. The state itself stays fp32 in the accumulators. The precompute writes
// W, [Gamma q] and Kt already split; the state pass splits S0 and delta (three
// bfloat16 products replace eight fp32 ones per 16 x 16 x 32 block; measured on
// MI355X, 8000-token prefill 704-726 -> 613-620 us). The output finish (B delta)
// stays on fp32 MFMA.
//
// Decay products never divide. A chunk is two sub-blocks of 16 tokens. With
// P_t the product over its own sub-block up to and including t, and R_s the
// product over its sub-block after s:
//   * across sub-blocks (t in block 1, s in block 0) D(t, s) = P_t R_s, so A
//     and B there are MFMA products of [P k] and [P q] with [R k];
//   * inside a sub-block D(t, s) is carried as a running product;
//   * Gamma_t = (product of the earlier sub-blocks) P_t and the decay to the
//     chunk end is R_s (product of the later sub-blocks).
// Any decay in (0, 1] is safe: a product only underflows where the true value
// does. The results equal the token-by-token recurrence up to rounding (not bit
// for bit: the kernel of kda_prefill gives bit-identical states).

#include "kda_chunk.h"
#include "kda_engine.h"

namespace kda {
namespace {

constexpr int kCL = kChunkTokens;  // tokens per chunk
constexpr int kSB = 16;            // sub-block: the MFMA row block
static_assert(kCL == 2 * kSB, "the chunk is two sub-blocks");

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// (x0, x1) to packed bfloat16 pairs: hi = RNE(x) and lo = RNE(x - hi), element
// 0 in the low half of each word
__device__ __forceinline__ void split_pair(float x0, float x1, uint32_t &hi, uint32_t &lo) {
  hi = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){x0, x1}, bf16x2));
  const float r0 = x0 - __builtin_bit_cast(float, hi << 16);
  const float r1 = x1 - __builtin_bit_cast(float, hi & 0xffff0000u);
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){r0, r1}, bf16x2));
}

// The split of N floats as N/2 hi words then N/2 lo words
template <int N>
__device__ __forceinline__ void split_n(const float (&x)[N], uint32_t (&w)[N]) {
#pragma unroll
  for (int i = 0; i < N / 2; ++i) split_pair(x[2 * i], x[2 * i + 1], w[i], w[N / 2 + i]);
}

// 16-byte slot s of the split of N floats (N = 8: s = 0 the hi, 1 the lo parts;
// N = 4: s = 0, hi then lo)
template <int N>
__device__ __forceinline__ float4 split_slot(const float (&x)[N], int s) {
  uint32_t w[N];
  split_n<N>(x, w);
  if constexpr (N == 8) {
    return s == 0 ? make_float4(__builtin_bit_cast(float, w[0]), __builtin_bit_cast(float, w[1]),
                                __builtin_bit_cast(float, w[2]), __builtin_bit_cast(float, w[3]))
                  : make_float4(__builtin_bit_cast(float, w[N / 2]), __builtin_bit_cast(float, w[N / 2 + 1]),
                                __builtin_bit_cast(float, w[N / 2 + 2]), __builtin_bit_cast(float, w[N / 2 + 3]));
  } else {
    return make_float4(__builtin_bit_cast(float, w[0]), __builtin_bit_cast(float, w[1]),
                       __builtin_bit_cast(float, w[2]), __builtin_bit_cast(float, w[3]));
  }
}

// Workspace of one (chunk, head), in floats.
template <int DK, int DV>
struct ChunkWs {
  static constexpr int W = 0;               // [kCL][DK]  T [Gamma k]
  static constexpr int QD = W + kCL * DK;   // [kCL][DK]  Gamma q
  static constexpr int KT = QD + kCL * DK;  // [kCL][DK]  k_s decayed to the chunk end
  static constexpr int U = KT + kCL * DK;   // [kCL][DV]  T v
  static constexpr int BM = U + kCL * DV;   // [kCL][kCL]  B
  static constexpr int GL = BM + kCL * kCL; // [DK]  Gamma_L
  static constexpr int FLOATS = GL + DK;
  static_assert(FLOATS % 4 == 0, "float4 alignment of every (chunk, head)");
};

// Every array but Gamma_L is stored in the order in which the state pass
// reads it, so that each load instruction of a wave reads one contiguous
// block (1 KB for 16-byte loads) instead of a piece of each of 16 rows. With
// wave w of the state pass holding key channels [w DK/4, (w + 1) DK/4) and
// lane (j, g) = (lane % 16, lane / 16):
//   W, [Gamma q]  [rt][s][w][lane]: token 16 rt + j at the lane's channels
//                 w DK/4 + 16 (i / 4) + 4 g + i % 4, i < DK / 16
//   Kt            [ct][s][w][lane]: key channel w DK/4 + 16 ct + j at tokens 4 i + g, i < 8
//   B             [h][rb][lane][4]: row 16 rb + j, entries 4 (4 h + e) + g (fp32)
//   U             [tile][h][lane][4]: value column 16 tile + j, tokens 4 (4 h + e) + g (fp32)
// W, [Gamma q] and Kt hold the bfloat16 split of their n = 8 (n = 4 for W and
// [Gamma q] at DK = 64) values per lane: the n hi parts, then the n lo parts,
// each pair packed low half first, 16 bytes per slot s (ct < DK / 64, h and rb
// < 2, e < 4 the float of the float4).

// Chunks of one row.// Chunks of one row. nch = 0 for a row that does not run (padding, or any
// device error; the state pass reports those).
struct ChunkRow {
  int nch, n1, s1, Tb;  // chunks, chunks before the checkpoint cut, the cut, tokens
};

__device__ __forceinline__ ChunkRow chunk_row(const ChunkArgs &a, int b) {
  ChunkRow r = {0, 0, 0, 0};
  const int32_t slot = a.slot_ids[b];
  if (slot < 0 || slot >= a.num_slots) return r;
  const int32_t c0 = a.cu[b], c1 = a.cu[b + 1];
  if (c0 < 0 || c1 < c0 || c1 > a.n_tok) return r;
  const int Tb = c1 - c0;
  const int ck = a.ckpt_pos ? a.ckpt_pos[b] : -1;
  if (ck > Tb) return r;
  r.Tb = Tb;
  r.s1 = (ck > 0 && ck < Tb) ? ck : Tb;
  r.n1 = (r.s1 + kCL - 1) / kCL;
  r.nch = r.n1 + (Tb - r.s1 + kCL - 1) / kCL;
  return r;
}

// ----------------------------------------------------------------------------
// Chunk map, one workgroup: the first chunk of every row (an exclusive prefix
// sum of the rows' chunk counts) and the row of every chunk, so that each
// precompute workgroup finds its row and each state-pass workgroup its first
// chunk with one lookup. Chunks past the last row's map to -1.
// ----------------------------------------------------------------------------

__global__ __launch_bounds__(kChunkMapThreads) void chunk_map_kernel(ChunkArgs a) {
  __shared__ int32_t part[kChunkMapThreads];
  __shared__ int32_t run;
  const int tid = threadIdx.x;
  if (tid == 0) run = 0;
  __syncthreads();
  for (int b0 = 0; b0 < a.B; b0 += kChunkMapThreads) {
    const int b = b0 + tid;
    const int n = b < a.B ? chunk_row(a, b).nch : 0;
    part[tid] = n;
    __syncthreads();
    // inclusive scan of the tile (Hillis-Steele over LDS)
    for (int d = 1; d < kChunkMapThreads; d <<= 1) {
      const int add = tid >= d ? part[tid - d] : 0;
      __syncthreads();
      part[tid] += add;
      __syncthreads();
    }
    const int first = run + part[tid] - n;
    if (b < a.B) a.cbase[b] = first;
    // the chunk -> row table for this tile's rows: chunk run + c belongs to the
    // first row whose inclusive sum exceeds c (a binary search in LDS)
    const int tile_total = part[kChunkMapThreads - 1];
    for (int c = tid; c < tile_total; c += kChunkMapThreads) {
      int lo = 0, hi = kChunkMapThreads - 1;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (part[mid] > c)
          hi = mid;
        else
          lo = mid + 1;
      }
      if (run + c < a.ws_chunks) a.crow[run + c] = b0 + lo;
    }
    __syncthreads();
    if (tid == kChunkMapThreads - 1) run += part[tid];
    __syncthreads();
  }
  const int total = run;
  if (tid == 0) a.cbase[a.B] = total;
  for (int c = total + tid; c < a.ws_chunks; c += kChunkMapThreads) a.crow[c] = -1;
}

// Token range [t0, t0 + n) of chunk j of a row.
__device__ __forceinline__ void chunk_tokens(const ChunkRow &r, int j, int &t0, int &n) {
  if (j < r.n1) {
    t0 = j * kCL;
    n = min(kCL, r.s1 - t0);
  } else {
    t0 = r.s1 + (j - r.n1) * kCL;
    n = min(kCL, r.Tb - t0);
  }
}

// ----------------------------------------------------------------------------
// Precompute, one workgroup per (chunk, head)
// ----------------------------------------------------------------------------

// Raw-input preparation of staged tokens [0, n) held at row pitch PK: the
// engine's per-row routines on one 16-lane row per token.
template <int DK, int PK>
__device__ __forceinline__ void prep_rows(float *k, float *q, float *al, float *beta, int n) {
  constexpr int NV = DK / 64;
  const int rows = blockDim.x >> 4, r = threadIdx.x & 15;
  for (int t = threadIdx.x >> 4; t < n; t += rows) {
    float4 kk[NV], qq[NV], aa[NV];
#pragma unroll
    for (int e = 0; e < NV; ++e) {
      const int i = t * PK + 4 * r + 64 * e;
      kk[e] = *reinterpret_cast<const float4 *>(k + i);
      qq[e] = *reinterpret_cast<const float4 *>(q + i);
      aa[e] = *reinterpret_cast<const float4 *>(al + i);
    }
    prep_normalize<NV>(kk, 1.0f);
    prep_normalize<NV>(qq, 1.0f / __builtin_sqrtf((float)DK));
    prep_decay<NV>(aa);
#pragma unroll
    for (int e = 0; e < NV; ++e) {
      const int i = t * PK + 4 * r + 64 * e;
      *reinterpret_cast<float4 *>(k + i) = kk[e];
      *reinterpret_cast<float4 *>(q + i) = qq[e];
      *reinterpret_cast<float4 *>(al + i) = aa[e];
    }
    if (r == 0) beta[t] = prep_beta(beta[t]);
  }
}

template <int DK, int DV>
__global__ __launch_bounds__(kChunkPrepThreads) void prefill_chunk_prep_kernel(ChunkArgs a) {
  using WS = ChunkWs<DK, DV>;
  constexpr int CPT = DK / 16;  // channels per lane when a 16-lane row spans DK
  // Rows of k, q and alpha are padded by 4 floats: the MFMA operand reads of 16
  // rows at once then start 4 banks apart and cover every bank once per 8 lanes.
  constexpr int PK = DK + 4;
  __shared__ float kb[kCL * PK];  // k, then [P k]
  __shared__ float qb[kCL * PK];  // q, then [P q]
  __shared__ float ab[kCL * PK];  // alpha, then [R k]
  __shared__ float vb[kCL * DV];
  __shared__ float bet[kCL];
  __shared__ float Am[kCL * kCL];        // A (strictly lower)
  __shared__ float Tm[kCL * (kCL + 1)];  // T, rows padded by one float against bank conflicts
  __shared__ float Bl[kCL * kCL];        // B, written out in one coalesced pass
  __shared__ float gb[2 * DK];           // product of each sub-block's decays

  // Chunks are prepared last to first: the state pass starts at the first, and
  // the workspace written last is the part most likely still held in the
  // memory-side cache when it starts (measured on MI355X: 4% off the state pass
  // of an 8000-token prompt).
  const int c = (int)(gridDim.x / a.H) - 1 - (int)(blockIdx.x / a.H), h = blockIdx.x % a.H;
  // the row and chunk this workgroup prepares, from the chunk map (a single row
  // needs none: its chunks are numbered from 0)
  int b = 0, jc = c;
  if (a.B > 1) {
    b = a.crow[c];
    if (b < 0) return;
    jc = c - a.cbase[b];
  }
  const ChunkRow r = chunk_row(a, b);
  if (jc >= r.nch) return;
  int t0, n;
  chunk_tokens(r, jc, t0, n);
  const int64_t row0 = (int64_t)a.cu[b] + t0;
  float *ws = a.ws + ((int64_t)c * a.H + h) * WS::FLOATS;

  // stage the chunk; tokens past its end are k = q = v = 0, alpha = 1, beta = 0.
  // Every load is issued before the first LDS write.
  constexpr int NT = kChunkPrepThreads, NWAVES = NT / 64;
  constexpr int NK = kCL * (DK / 4) / NT;  // staging rounds of k, q and alpha
  constexpr int NVI = kCL * (DV / 4), NVL = (NVI + NT - 1) / NT;  // and of v
  static_assert(NK >= 1 && kCL * (DK / 4) == NT * NK, "whole staging rounds of k, q and alpha");
  uint2 kr[NK], qr[NK], vr[NVL];
  float4 ar[NK];
#pragma unroll
  for (int m = 0; m < NK; ++m) {
    const int idx = threadIdx.x + NT * m, t = idx / (DK / 4), i = (idx % (DK / 4)) * 4;
    kr[m] = qr[m] = make_uint2(0u, 0u);
    ar[m] = make_float4(1.0f, 1.0f, 1.0f, 1.0f);
    if (t < n) {
      const int64_t off = ((row0 + t) * a.H + h) * DK + i;
      kr[m] = *reinterpret_cast<const uint2 *>(a.k + off);
      qr[m] = *reinterpret_cast<const uint2 *>(a.q + off);
      ar[m] = *reinterpret_cast<const float4 *>(a.alpha + off);
    }
  }
#pragma unroll
  for (int m = 0; m < NVL; ++m) {
    const int idx = threadIdx.x + NT * m, t = idx / (DV / 4), j = (idx % (DV / 4)) * 4;
    vr[m] = make_uint2(0u, 0u);
    if (idx < NVI && t < n) vr[m] = *reinterpret_cast<const uint2 *>(a.v + ((row0 + t) * a.H + h) * DV + j);
  }
  if ((int)threadIdx.x < kCL) bet[threadIdx.x] = (int)threadIdx.x < n ? a.beta[(row0 + threadIdx.x) * a.H + h] : 0.0f;
#pragma unroll
  for (int m = 0; m < NK; ++m) {
    const int idx = threadIdx.x + NT * m, t = idx / (DK / 4), i = (idx % (DK / 4)) * 4;
    *reinterpret_cast<float4 *>(kb + t * PK + i) = unpack_bf16x4(kr[m]);
    *reinterpret_cast<float4 *>(qb + t * PK + i) = unpack_bf16x4(qr[m]);
    *reinterpret_cast<float4 *>(ab + t * PK + i) = ar[m];
  }
#pragma unroll
  for (int m = 0; m < NVL; ++m) {
    const int idx = threadIdx.x + NT * m, t = idx / (DV / 4), j = (idx % (DV / 4)) * 4;
    if (idx < NVI) *reinterpret_cast<float4 *>(vb + t * DV + j) = unpack_bf16x4(vr[m]);
  }
  __syncthreads();
  if (a.raw) {
    prep_rows<DK, PK>(kb, qb, ab, bet, n);
    __syncthreads();
  }

  // inside each sub-block: A and B by running products. Row (s, 16 lanes) of
  // sub-block o carries D(t, s) over its lane's channels 4 cl + 64 e4 .. + 3 as t
  // advances and sums over the row; the 32 rows of 16 lanes cover both sub-blocks.
  // A wave starts at the first token past its rows (the steps before it only fed
  // discarded sums), and the second sub-block's rows run in reverse order, so
  // that the two waves on a SIMD (w and w + 4) need 18 steps together instead of
  // up to 30: this pass is bound by VALU issue. Each step reads token t's k, q and
  // alpha with 128-bit LDS reads before any arithmetic and applies alpha_t as a
  // factor (1 up to s, exact), so no read waits behind a per-lane branch.
  if ((int)threadIdx.x < 2 * kSB * 16) {
    static_assert(CPT % 4 == 0, "whole float4 per lane");
    const int o = (threadIdx.x >> 8) * kSB, r = (threadIdx.x >> 4) & 15, cl = threadIdx.x & 15;
    const int s = o == 0 ? r : kSB - 1 - r;
    const int s_min = __builtin_amdgcn_readfirstlane(o == 0 ? (r & ~3) : kSB - 1 - (r | 3));
    auto ld_row = [&](const float *x, int t, float (&y)[CPT]) {
#pragma unroll
      for (int e4 = 0; e4 < CPT / 4; ++e4) {
        const float4 v = *reinterpret_cast<const float4 *>(x + (o + t) * PK + 4 * cl + 64 * e4);
        y[4 * e4] = v.x;
        y[4 * e4 + 1] = v.y;
        y[4 * e4 + 2] = v.z;
        y[4 * e4 + 3] = v.w;
      }
    };
    float d[CPT], qs[CPT];
    ld_row(kb, s, d);
    ld_row(qb, s, qs);
    float pd = 0.0f;
#pragma unroll
    for (int e = 0; e < CPT; ++e) pd = __builtin_fmaf(qs[e], d[e], pd);
    pd = row16_sum(pd);
    if (cl == 0) Bl[(o + s) * kCL + o + s] = pd;
    for (int t = s_min + 1; t < kSB; ++t) {
      const bool after = t > s;  // D(t, s) starts at k_s and takes alpha_t only past s
      float kt[CPT], qt[CPT], at[CPT];
      ld_row(kb, t, kt);
      ld_row(qb, t, qt);
      ld_row(ab, t, at);
      float pa = 0.0f, pb = 0.0f;
#pragma unroll
      for (int e = 0; e < CPT; ++e) {
        d[e] = d[e] * (after ? at[e] : 1.0f);
        pa = __builtin_fmaf(kt[e], d[e], pa);
        pb = __builtin_fmaf(qt[e], d[e], pb);
      }
      pa = row16_sum(pa);
      pb = row16_sum(pb);
      if (cl == 0 && after) {
        Am[(o + t) * kCL + o + s] = pa;
        Bl[(o + t) * kCL + o + s] = pb;
      }
    }
  }
  __syncthreads();

  // per (key channel, sub-block), all threads: [P k] and [P q] in place of k and q and
  // [R k] in place of alpha, for the thread's own sub-block
  {
    const int i = threadIdx.x % DK, J = threadIdx.x / DK;  // sub-blocks J = 0, 1 (the other threads idle)
    if (J < 2) {
      const int o = J * kSB;
      float kf[kSB];
      float P = 1.0f;
#pragma unroll
      for (int t = 0; t < kSB; ++t) {
        P = P * ab[(o + t) * PK + i];
        kf[t] = kb[(o + t) * PK + i] * P;
        qb[(o + t) * PK + i] = qb[(o + t) * PK + i] * P;
      }
      gb[J * DK + i] = P;
      float R = 1.0f;
#pragma unroll
      for (int t = kSB - 1; t >= 0; --t) {
        const float kr2 = kb[(o + t) * PK + i] * R;
        R = R * ab[(o + t) * PK + i];
        ab[(o + t) * PK + i] = kr2;
        kb[(o + t) * PK + i] = kf[t];
      }
    }
  }
  __syncthreads();
  // Gamma q = [P q] x (earlier sub-blocks), keys decayed to the chunk end = [R k] x
  // (later sub-blocks), both split to bfloat16 parts, and Gamma_L, to the workspace
  // in its read order, one 16-byte slot per thread and step
  constexpr int CPW = DK / 4, NCT = CPW / 16;
  for (int d4 = threadIdx.x; d4 < kCL * DK / 4; d4 += blockDim.x) {
    const int lane = d4 & 63, w = (d4 >> 6) & 3, r2 = d4 >> 8, j = lane & 15, g = lane >> 4;
    {
      const int t = 16 * (r2 / NCT) + j;
      float x[4 * NCT];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const int i0 = w * CPW + 16 * ct + 4 * g;
        float4 qf = *reinterpret_cast<const float4 *>(qb + t * PK + i0);
        if (t >= kSB) {  // uniform over the wave
          qf.x *= gb[i0];
          qf.y *= gb[i0 + 1];
          qf.z *= gb[i0 + 2];
          qf.w *= gb[i0 + 3];
        }
        x[4 * ct] = qf.x;
        x[4 * ct + 1] = qf.y;
        x[4 * ct + 2] = qf.z;
        x[4 * ct + 3] = qf.w;
      }
      *reinterpret_cast<float4 *>(ws + WS::QD + 4 * d4) = split_slot<4 * NCT>(x, r2 % NCT);
    }
    {
      const int i = w * CPW + 16 * (r2 >> 1) + j;
      const float gk = gb[DK + i];
      float kv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int tok = 4 * e + g;
        const float y = ab[tok * PK + i];
        kv[e] = tok < kSB ? y * gk : y;
      }
      *reinterpret_cast<float4 *>(ws + WS::KT + 4 * d4) = split_slot<8>(kv, r2 & 1);
    }
  }
  if ((int)threadIdx.x < DK) ws[WS::GL + threadIdx.x] = gb[threadIdx.x] * gb[DK + threadIdx.x];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, m = lane & 15, g = lane >> 4;
  // across the sub-blocks: A (wave 0) and B (wave 1) for t in block 1, s in block 0,
  // [P k]_t . [R k]_s and [P q]_t . [R k]_s over DK on MFMA
  if (wave < 2) {
    const float *arow = (wave == 0 ? kb : qb) + (kSB + m) * PK;  // A operand: row t = kSB + m
    const float *brow = ab + m * PK;                             // B operand: column s = m
    v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int cb = 0; cb < DK / 16; ++cb) {
      const float4 av = *reinterpret_cast<const float4 *>(arow + 16 * cb + 4 * g);
      const float4 bv = *reinterpret_cast<const float4 *>(brow + 16 * cb + 4 * g);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av.x, bv.x, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av.y, bv.y, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av.z, bv.z, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av.w, bv.w, acc, 0, 0, 0);
    }
    // accumulator: lane (m, g) holds rows 4g .. 4g + 3 (t = kSB + 4g + e) of column s = m
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = kSB + 4 * g + e;
      if (wave == 0)
        Am[t * kCL + m] = acc[e];
      else
        Bl[t * kCL + m] = acc[e];
    }
  }
  __syncthreads();
  // B to the workspace in its read order, zero above the diagonal
  for (int d = threadIdx.x; d < kCL * kCL; d += blockDim.x) {
    const int e = d & 3, lane = (d >> 2) & 63, rb = (d >> 8) & 1, h = d >> 9;
    const int t = 16 * rb + (lane & 15), s = 4 * (4 * h + e) + (lane >> 4);
    ws[WS::BM + d] = s > t ? 0.0f : Bl[t * kCL + s];
  }

  // X = (I + Diag(beta) A)^-1 by 16 x 16 blocks: the two diagonal blocks by forward
  // substitution (one column per thread), then X10 = -X11 (Diag(beta) A)10 X00,
  // into Tm; the products below read T = X Diag(beta) as X_ts beta_s.
  if ((int)threadIdx.x < 2 * kSB) {
    const int J = threadIdx.x / kSB, col = threadIdx.x % kSB, o = J * kSB;
    // Every row's sum is formed and the entries above and on the diagonal are
    // selected afterwards, so no read waits behind a per-lane branch; row t + 1
    // of A is read while row t is summed.
    float x[kSB], arow[kSB], nrow[kSB];
#pragma unroll
    for (int t = 0; t < kSB; ++t) {
      if (t + 1 < kSB) {
#pragma unroll
        for (int s2 = 0; s2 <= t; ++s2) nrow[s2] = Am[(o + t + 1) * kCL + o + s2];
      }
      const float bt = bet[o + t];
      float acc = 0.0f;
#pragma unroll
      for (int s2 = 0; s2 < t; ++s2) acc = __builtin_fmaf(arow[s2], x[s2], acc);
      float xt = -bt * acc;
      asm volatile("" : "+v"(xt));  // computed here, not sunk into a branch of the select
      x[t] = t == col ? 1.0f : (t < col ? 0.0f : xt);
#pragma unroll
      for (int s2 = 0; s2 <= t; ++s2) arow[s2] = nrow[s2];
    }
#pragma unroll
    for (int t = 0; t < kSB; ++t) Tm[(o + t) * (kCL + 1) + o + col] = x[t];
  }
  __syncthreads();
  if ((int)threadIdx.x < kSB * kSB) {
    const int t = threadIdx.x / kSB, col = threadIdx.x % kSB;  // one (t, col) of the 16 x 16 block each
    float y = 0.0f;
#pragma unroll
    for (int s2 = 0; s2 < kSB; ++s2) y = __builtin_fmaf(Am[(kSB + t) * kCL + s2], Tm[s2 * (kCL + 1) + col], y);
    Bl[t * kSB + col] = bet[kSB + t] * y;  // (Diag(beta) A)10 X00; B is already in the workspace
  }
  __syncthreads();
  if ((int)threadIdx.x < kSB * kSB) {
    const int t = threadIdx.x / kSB, col = threadIdx.x % kSB;
    float x10 = 0.0f;
#pragma unroll
    for (int u2 = 0; u2 < kSB; ++u2)
      x10 = __builtin_fmaf(Tm[(kSB + t) * (kCL + 1) + kSB + u2], Bl[u2 * kSB + col], x10);
    Tm[(kSB + t) * (kCL + 1) + col] = -x10;
    Tm[t * (kCL + 1) + kSB + col] = 0.0f;
  }
  __syncthreads();

  // W = T [Gamma k] and U = T V: 16 x 16 output tiles spread over the waves
  constexpr int TW = DK / 16, TU = DV / 16;
  for (int tile = wave; tile < 2 * TW; tile += NWAVES) {
    const int rt = tile & 1, ct = tile >> 1;
    float av[kCL / 4], bv[kCL / 4];
#pragma unroll
    for (int ks = 0; ks < kCL / 4; ++ks) {
      const int tok = 4 * ks + g;
      av[ks] = Tm[(16 * rt + m) * (kCL + 1) + tok] * bet[tok];
      // [Gamma k] = [P k] times the product of the earlier sub-blocks (one for block 0)
      bv[ks] = ks < kSB / 4 ? kb[tok * PK + 16 * ct + m] : kb[tok * PK + 16 * ct + m] * gb[16 * ct + m];
    }
    v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < kCL / 4; ++ks) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[ks], bv[ks], acc, 0, 0, 0);
    // W to the rows of [P q], free since the products across sub-blocks
#pragma unroll
    for (int e = 0; e < 4; ++e) qb[(16 * rt + 4 * g + e) * PK + 16 * ct + m] = acc[e];
  }
  for (int tile = wave; tile < 2 * TU; tile += NWAVES) {
    const int rt = tile & 1, ct = tile >> 1;
    float av[kCL / 4], bv[kCL / 4];
#pragma unroll
    for (int ks = 0; ks < kCL / 4; ++ks) {
      const int tok = 4 * ks + g;
      av[ks] = Tm[(16 * rt + m) * (kCL + 1) + tok] * bet[tok];
      bv[ks] = vb[tok * DV + 16 * ct + m];
    }
    v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < kCL / 4; ++ks) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[ks], bv[ks], acc, 0, 0, 0);
#pragma unroll
    for (int e = 0; e < 4; ++e) ws[WS::U + ct * (kCL * 16) + (rt * 64 + e * 16 + m) * 4 + g] = acc[e];
  }
  __syncthreads();
  for (int d4 = threadIdx.x; d4 < kCL * DK / 4; d4 += blockDim.x) {
    const int lane = d4 & 63, w = (d4 >> 6) & 3, r2 = d4 >> 8;
    const int t = 16 * (r2 / NCT) + (lane & 15);
    float x[4 * NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const float4 v = *reinterpret_cast<const float4 *>(qb + t * PK + w * CPW + 16 * ct + 4 * (lane >> 4));
      x[4 * ct] = v.x;
      x[4 * ct + 1] = v.y;
      x[4 * ct + 2] = v.z;
      x[4 * ct + 3] = v.w;
    }
    *reinterpret_cast<float4 *>(ws + WS::W + 4 * d4) = split_slot<4 * NCT>(x, r2 % NCT);
  }
}

// ----------------------------------------------------------------------------
// State pass, one workgroup per (row, head, 16 value columns)
// ----------------------------------------------------------------------------
//
// Wave w holds key channels [w DK/4, (w+1) DK/4) of the 16 columns in the
// accumulator layout: lane (j, g) holds channels 16 ct + 4g .. + 3 (of its
// quarter) of column j. The products with the state are split over the waves
// along DK and summed in LDS.

__device__ __forceinline__ void put_chunk_out(const ChunkArgs &a, int64_t idx, float y) {
  if (a.out_bf16)
    reinterpret_cast<uint16_t *>(a.out)[idx] = f32_to_bf16(y);
  else
    a.out[idx] = y;
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x8 as_bf16x8(float4 v) {
  return __builtin_bit_cast(bf16x8, (u32x4){__builtin_bit_cast(uint32_t, v.x), __builtin_bit_cast(uint32_t, v.y),
                                            __builtin_bit_cast(uint32_t, v.z), __builtin_bit_cast(uint32_t, v.w)});
}

// acc + A B over K = 32 (the bfloat16 parts of A in two 16-byte slots, hi then
// lo; B as split_n words), small terms first
__device__ __forceinline__ v4f split_mma32(float4 a_hi, float4 a_lo, const uint32_t (&b)[8], v4f acc) {
  const bf16x8 ah = as_bf16x8(a_hi), al = as_bf16x8(a_lo);
  const bf16x8 bh = __builtin_bit_cast(bf16x8, (u32x4){b[0], b[1], b[2], b[3]});
  const bf16x8 bl = __builtin_bit_cast(bf16x8, (u32x4){b[4], b[5], b[6], b[7]});
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc, 0, 0, 0);
}

// the same over K = 16, A's hi and lo parts in one slot
__device__ __forceinline__ v4f split_mma16(float4 a, const uint32_t (&b)[4], v4f acc) {
  const s16x4 ah = __builtin_bit_cast(s16x4, (u32x2){__builtin_bit_cast(uint32_t, a.x), __builtin_bit_cast(uint32_t, a.y)});
  const s16x4 al = __builtin_bit_cast(s16x4, (u32x2){__builtin_bit_cast(uint32_t, a.z), __builtin_bit_cast(uint32_t, a.w)});
  const s16x4 bh = __builtin_bit_cast(s16x4, (u32x2){b[0], b[1]});
  const s16x4 bl = __builtin_bit_cast(s16x4, (u32x2){b[2], b[3]});
  acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(al, bh, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, bl, acc, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, bh, acc, 0, 0, 0);
}

// A S0 over a wave's NCT 16-channel tiles (A one row block of W or [Gamma q])
template <int NCT>
__device__ __forceinline__ v4f state_mma(const float4 (&a)[NCT], const uint32_t (&sw)[4 * NCT]) {
  const v4f z = {0.0f, 0.0f, 0.0f, 0.0f};
  if constexpr (NCT == 2)
    return split_mma32(a[0], a[1], sw, z);
  else
    return split_mma16(a[0], sw, z);
}

template <class WS>
__device__ __forceinline__ const float *chunk_ws(const ChunkArgs &a, int c, int h) {
  return a.ws + ((int64_t)c * a.H + h) * WS::FLOATS;
}

template <class WS>
__device__ __forceinline__ float4 ws4(const float *w, int off) {
  return *reinterpret_cast<const float4 *>(w + off);
}

// One workgroup per (row, head, 16 value columns), six waves in two roles.
// Wave q < 4 carries the recurrence over key channels [q DK/4, (q + 1) DK/4):
//   W S0 and [Gamma q] S0 over its channels -> (barrier)
//   -> delta = U - sum of the four W S0 partials
//   -> S0 <- Diag(Gamma_L) S0 + Kt^T delta
// holding the state in the accumulator layout (lane (j, g) has channels
// q DK/4 + 16 ct + 4 g .. + 3 of column j), at the higher priority. Waves 4
// and 5 finish each chunk's outputs, o = [Gamma q] S0 + B delta, one barrier
// later. (With the [Gamma q] S0
// products on side waves sharing the SIMDs, the side waves' path was the longer
// one: measured on MI355X, 8000 tokens 735 -> 710 us with them moved here.) One
// barrier per chunk; a buffer is written again only after the barrier that
// follows its last read.
template <int DK, int DV>
__global__ __launch_bounds__(kChunkStateThreads) void prefill_chunk_state_kernel(ChunkArgs a) {
  using WS = ChunkWs<DK, DV>;
  constexpr int CPW = DK / 4;    // key channels per wave
  constexpr int NCT = CPW / 16;  // 16-channel tiles per wave
  static_assert(kChunkStateThreads == 384, "four recurrence waves and two finishing waves");
  // W S0 partials in the reading lanes' layout: [parity][wave][row block][lane][c]
  // holds token 4 (4 rb + c) + g, column j of lane (j, g), so that each lane reads
  // the partials it needs as float4s.
  __shared__ float4 pdp[2][4][2][64];
  // [Gamma q] S0 partials, accumulator layout, by chunk index mod 3: written
  // before barrier jc and read by the output finish after barrier jc + 1, while
  // the recurrence waves already write those of chunk jc + 1 (the chunk loop is
  // unrolled three times, so the index is static there)
  __shared__ v4f pop[3][4][2][64];
  __shared__ float4 dlt[2][2][64];        // delta, B-operand layout: [parity][h][lane] holds ks = 4 h + c

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
  const int ck = a.ckpt_pos ? a.ckpt_pos[u.b] : -1;
  if (ck > c1 - c0) {
    report(a.dev_err, u, KDA_DEVERR_CKPT);
    return;
  }
  const ChunkRow r = chunk_row(a, u.b);
  const int cbase = a.B > 1 ? a.cbase[u.b] : 0;
  if (cbase + r.nch > a.ws_chunks) {  // only with rows that overlap in cu_seqlens
    report(a.dev_err, u, KDA_DEVERR_SEQLEN);
    return;
  }
  if (r.nch == 0 && ck != 0) return;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), q = wave & 3;
  const int lane = threadIdx.x & 63, j = lane & 15, g = lane >> 4;
  const int n0 = 16 * u.tile;
  const int coff = CPW * q + 4 * g;  // first channel of this lane in tile 0
  const int last = r.nch - 1;

  if (wave < 4) {
    // ---- recurrence waves ----
    __builtin_amdgcn_s_setprio(2);
    float *S = a.cache + (int64_t)slot * a.slot_stride + ((int64_t)u.h * DV + n0 + j) * DK + coff;
    float *CK = ck >= 0 ? a.ckpt + (((int64_t)u.b * a.H + u.h) * DV + n0 + j) * DK + coff : nullptr;
    float4 s[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) s[ct] = ld4<kVerifyLoadStream>(S + 16 * ct);
    if (ck == 0) {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) st4<kVerifyStoreStream>(CK + 16 * ct, s[ct]);
    }
    // The operands of the chunk two ahead are read while this one computes, in
    // two batches that each follow a burst of products (a load issue that waits
    // for queue space then holds up no product): W and Kt behind the products
    // with S0, [Gamma q], Gamma_L and U behind the update (other splits measured
    // slower). Three operand sets rotate (the loop body is unrolled three times),
    // so no register copy waits for a load early; one chunk ahead, the loads'
    // latency still reached the products (measured on MI355X: 8000 tokens 790 ->
    // 740 us).
    // Past the last chunk the last one is read again, so every load is
    // unconditional.
    struct Ops {
      float4 wv[2][NCT], qv[2][NCT], kt[NCT][2], gl[NCT], uv[2];
    };
    auto load_wk = [&](Ops &o, const float *w) {
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) o.wv[rt][ct] = ws4<WS>(w, WS::W + (((rt * NCT + ct) * 4 + q) * 64 + lane) * 4);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int h = 0; h < 2; ++h) o.kt[ct][h] = ws4<WS>(w, WS::KT + (((ct * 2 + h) * 4 + q) * 64 + lane) * 4);
    };
    auto load_gu = [&](Ops &o, const float *w) {
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) o.qv[rt][ct] = ws4<WS>(w, WS::QD + (((rt * NCT + ct) * 4 + q) * 64 + lane) * 4);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) o.gl[ct] = ws4<WS>(w, WS::GL + coff + 16 * ct);
#pragma unroll
      for (int h = 0; h < 2; ++h) o.uv[h] = ws4<WS>(w, WS::U + u.tile * (kCL * 16) + (h * 64 + lane) * 4);
    };
    auto step = [&](int jc, int ps, const Ops &cur, Ops &nxt) {
      const int p = jc & 1;
      // S0 split to the B operand of the products over this wave's channels: slot i
      // of lane (j, g) is channel 16 (i / 4) + 4 g + i % 4 of the quarter, where the
      // accumulator layout already has it (no data moves between lanes)
      float sv[4 * NCT];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        sv[4 * ct] = s[ct].x;
        sv[4 * ct + 1] = s[ct].y;
        sv[4 * ct + 2] = s[ct].z;
        sv[4 * ct + 3] = s[ct].w;
      }
      uint32_t sw[4 * NCT];
      split_n<4 * NCT>(sv, sw);
      // W S0, then [Gamma q] S0 (for the output finish one barrier later)
      v4f pd[2], po[2];
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) pd[rt] = state_mma<NCT>(cur.wv[rt], sw);
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) po[rt] = state_mma<NCT>(cur.qv[rt], sw);
      const float *wn = chunk_ws<WS>(a, cbase + min(jc + 2, last), u.h);
      load_wk(nxt, wn);
      // this lane's accumulator element e (token 16 rt + 4 g + e, column j) is element
      // g of lane (j, e)'s float4
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int e = 0; e < 4; ++e) reinterpret_cast<float *>(&pdp[p][q][rt][e * 16 + j])[g] = pd[rt][e];
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) pop[ps][q][rt][lane] = po[rt];
      __syncthreads();

      // delta = U - W S0 at this lane's B-operand positions (token 4 ks + g, column
      // j), the partials summed over the waves in a fixed order
      float4 pv[4][2];
#pragma unroll
      for (int w4 = 0; w4 < 4; ++w4)
#pragma unroll
        for (int h = 0; h < 2; ++h) pv[w4][h] = pdp[p][w4][h][lane];
      float dv[8];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        dv[4 * h] = cur.uv[h].x - (((pv[0][h].x + pv[1][h].x) + pv[2][h].x) + pv[3][h].x);
        dv[4 * h + 1] = cur.uv[h].y - (((pv[0][h].y + pv[1][h].y) + pv[2][h].y) + pv[3][h].y);
        dv[4 * h + 2] = cur.uv[h].z - (((pv[0][h].z + pv[1][h].z) + pv[2][h].z) + pv[3][h].z);
        dv[4 * h + 3] = cur.uv[h].w - (((pv[0][h].w + pv[1][h].w) + pv[2][h].w) + pv[3][h].w);
      }
      if (wave == 0) {
#pragma unroll
        for (int h = 0; h < 2; ++h) dlt[p][h][lane] = make_float4(dv[4 * h], dv[4 * h + 1], dv[4 * h + 2], dv[4 * h + 3]);
      }

      // S0 <- Diag(Gamma_L) S0 + Kt^T delta over this wave's channels (delta split:
      // slot i of lane (j, g) is token 4 i + g, where dv already has it)
      uint32_t dw[8];
      split_n<8>(dv, dw);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        v4f acc = {s[ct].x * cur.gl[ct].x, s[ct].y * cur.gl[ct].y, s[ct].z * cur.gl[ct].z, s[ct].w * cur.gl[ct].w};
        acc = split_mma32(cur.kt[ct][0], cur.kt[ct][1], dw, acc);
        s[ct] = make_float4(acc[0], acc[1], acc[2], acc[3]);
      }
      load_gu(nxt, wn);
      int t0, n;
      chunk_tokens(r, jc, t0, n);
      if (ck > 0 && t0 + n == ck) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) st4<kVerifyStoreStream>(CK + 16 * ct, s[ct]);
      }
    };
    Ops o0, o1, o2;
    if (r.nch > 0) {
      load_wk(o0, chunk_ws<WS>(a, cbase, u.h));
      load_gu(o0, chunk_ws<WS>(a, cbase, u.h));
      load_wk(o1, chunk_ws<WS>(a, cbase + min(1, last), u.h));
      load_gu(o1, chunk_ws<WS>(a, cbase + min(1, last), u.h));
    }
    for (int jc = 0; jc < r.nch; jc += 3) {
      step(jc, 0, o0, o2);
      if (jc + 1 < r.nch) step(jc + 1, 1, o1, o0);
      if (jc + 2 < r.nch) step(jc + 2, 2, o2, o1);
    }
    __syncthreads();
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) st4<kVerifyStoreStream>(S + 16 * ct, s[ct]);
    return;
  }

  // ---- finishing waves ----
  // Wave 4 finishes row block 1 (tokens 16..31, B over all 32 deltas) and wave 5
  // row block 0 (tokens 0..15, whose B has no entries past token 15).
  const int rb = wave == 5 ? 0 : 1;
  // B of the chunk two ahead is read while this one finishes (three sets rotate)
  struct BOps {
    float4 bq[2];
  };
  float4 bprev[2];
  auto load_b = [&](BOps &o, const float *w) {
#pragma unroll
    for (int h = 0; h < 2; ++h) o.bq[h] = ws4<WS>(w, WS::BM + ((h * 2 + rb) * 64 + lane) * 4);
  };
  // the outputs of chunk jc, after the barrier that follows its delta
  auto finish = [&](int jc) {
    const int p = jc & 1, ps = jc % 3;
    v4f acc = ((pop[ps][0][rb][lane] + pop[ps][1][rb][lane]) + pop[ps][2][rb][lane]) + pop[ps][3][rb][lane];
    const float bm[8] = {bprev[0].x, bprev[0].y, bprev[0].z, bprev[0].w,
                         bprev[1].x, bprev[1].y, bprev[1].z, bprev[1].w};
    const float4 d0 = dlt[p][0][lane];
    const float dd0[4] = {d0.x, d0.y, d0.z, d0.w};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(bm[ks], dd0[ks], acc, 0, 0, 0);
    if (rb == 1) {  // row block 1 also takes the deltas of tokens 16..31
      const float4 d1 = dlt[p][1][lane];
      const float dd1[4] = {d1.x, d1.y, d1.z, d1.w};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(bm[4 + ks], dd1[ks], acc, 0, 0, 0);
    }
    int t0, n;
    chunk_tokens(r, jc, t0, n);
    // this lane's rows: tokens 16 rb + 4 g + e, column n0 + j; one base per chunk
    const int tok0 = 16 * rb + 4 * g;
    const int64_t row_stride = (int64_t)a.H * DV;
    const int64_t o0 = (((int64_t)c0 + t0 + tok0) * a.H + u.h) * DV + n0 + j;
    if (n == kCL) {  // a full chunk: every row is live
#pragma unroll
      for (int e = 0; e < 4; ++e) put_chunk_out(a, o0 + e * row_stride, acc[e]);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (tok0 + e < n) put_chunk_out(a, o0 + e * row_stride, acc[e]);
    }
  };
  auto side_step = [&](int jc, const BOps &cur, BOps &nxt) {
    __syncthreads();
    if (jc > 0) finish(jc - 1);
    bprev[0] = cur.bq[0];
    bprev[1] = cur.bq[1];
    load_b(nxt, chunk_ws<WS>(a, cbase + min(jc + 2, last), u.h));
  };
  BOps b0, b1, b2;
  if (r.nch > 0) {
    load_b(b0, chunk_ws<WS>(a, cbase, u.h));
    load_b(b1, chunk_ws<WS>(a, cbase + min(1, last), u.h));
  }
  for (int jc = 0; jc < r.nch; jc += 3) {
    side_step(jc, b0, b2);
    if (jc + 1 < r.nch) side_step(jc + 1, b1, b0);
    if (jc + 2 < r.nch) side_step(jc + 2, b2, b1);
  }
  __syncthreads();
  if (r.nch > 0) finish(last);
}

}  // namespace

size_t prefill_chunk_ws_floats(int dk, int dv) {
  if (dk == 64) return dv == 64 ? ChunkWs<64, 64>::FLOATS : ChunkWs<64, 128>::FLOATS;
  return dv == 64 ? ChunkWs<128, 64>::FLOATS : ChunkWs<128, 128>::FLOATS;
}

const void *prefill_chunk_map_kernel() { return (const void *)chunk_map_kernel; }

const void *prefill_chunk_prep_kernel_for(int dk, int dv) {
  if (dk == 64) return dv == 64 ? (const void *)prefill_chunk_prep_kernel<64, 64> : (const void *)prefill_chunk_prep_kernel<64, 128>;
  if (dk == 128) return dv == 64 ? (const void *)prefill_chunk_prep_kernel<128, 64> : (const void *)prefill_chunk_prep_kernel<128, 128>;
  return nullptr;
}

const void *prefill_chunk_state_kernel_for(int dk, int dv) {
  if (dk == 64) return dv == 64 ? (const void *)prefill_chunk_state_kernel<64, 64> : (const void *)prefill_chunk_state_kernel<64, 128>;
  if (dk == 128) return dv == 64 ? (const void *)prefill_chunk_state_kernel<128, 64> : (const void *)prefill_chunk_state_kernel<128, 128>;
  return nullptr;
}

}  // namespace kda
