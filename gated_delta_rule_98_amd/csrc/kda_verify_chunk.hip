// kda_verify_chunk.hip - the chunk form of speculative verify (KDA_VERIFY_CHUNKED).

#include "kda_chunk.h"
#include "kda_engine.h"

namespace kda {
namespace {

// ----------------------------------------------------------------------------
// Chunk form of verify (outputs only), MFMA for the products with the state
// ----------------------------------------------------------------------------
//
// For the T_b <= 16 tokens of a row, with S0 the committed state, G_t the
// running product of the decays up to and including token t, and
// D(s, t) = k_s * prod_{s < r <= t} alpha_r (the key of token s as the decayed
// state sees it at token t), the token-by-token recurrence unrolls to
//   u_t     = S0^T (G_t k_t) + sum_{s<t} A_ts delta_s,   A_ts = k_t . D(s, t)
//   delta_t = beta_t (v_t - u_t)
//   o_t     = S0^T (G_t q_t) + sum_{s<=t} B_ts delta_s,  B_ts = q_t . D(s, t)
// and over the chunk, with the tokens as rows, U0 = [G k] S0 and O0 = [G q] S0,
//   delta = M (V - U0),  M = (I + diag(beta) A)^{-1} diag(beta)
//   O     = O0 + N (V - U0),  N = B M.
// A, B, M and N are T_b x T_b and belong to the (row, head); the coupling
// coefficients come from running products (no division, so any decay in
// (0, 1] is safe) and M from a forward substitution per column. Everything
// per value column is then matrix products on MFMA: U0 and O0 contract the
// state over dk, and N (V - U0) contracts the chunk's tokens.
//
// Workgroup: one (row, head), all dv columns, dv / 16 waves; wave w owns
// columns 16w..16w+15. The state is held in the v_mfma_f32_16x16x4f32 layout:
// for the 16x16 block of channels 16cb..16cb+15 and the wave's columns, lane
// (j = lane % 16, g = lane / 16) holds channels 16cb + 4g .. + 3 of column j,
// one 128-bit load from the [dv][dk] cache. As the B operand of step (cb, e)
// that lane supplies channel 16cb + 4g + e; the A operand (row j of the
// decayed keys or queries) uses the same channel order, so the contraction
// over dk is complete. Products come back with lane (j, g) holding rows
// 4g..4g+3 of column j, which is again a B operand: step e of the product over
// tokens takes token 4g + e from register e of lane (j, g), so N (V - U0)
// needs no data movement between lanes.
//
// This kernel serves rows of up to 16 tokens (T_max > 8): the decayed keys and
// the decayed queries take one 16-row A operand each. Rows of at most 8 tokens
// have the kernel below it.

constexpr int kCoupleThreads = 256;  // threads of the coupling pass
constexpr int kNStride = 20;         // row stride of the N operand (conflict-free 128-bit reads)

// LDS of the chunk kernel, in floats. Row strides are padded by 4 floats so
// that the 16 rows read by a 16-lane group for an MFMA operand, and the token
// rows of v read by the four lane groups, fall on different banks.
template <int DK, int W>
struct VcLds {
  static constexpr int P = DK + 4;   // row stride of the A operand
  static constexpr int VS = W + 4;   // row stride of the staged v
  float *k, *a, *q;  // [T_max][DK] staged inputs
  float *v;          // [T_max][VS]
  float *beta;       // [16]
  float *am;         // [2R][P]: rows 0..R-1 are G_t k_t, rows R..2R-1 are G_t q_t
  float *cA, *cB;    // [16][16] coupling coefficients (row t, column s)
  float *nm;         // [16][kNStride]: the N operand, in output-row order
  __device__ VcLds(float *base, int T_max, int R) {
    k = base;
    a = k + T_max * DK;
    q = a + T_max * DK;
    v = q + T_max * DK;
    beta = v + T_max * VS;
    am = beta + 16;
    cA = am + 2 * R * P;
    cB = cA + 256;
    nm = cB + 256;
  }
};

// Sum over groups of LPR (16 or 32) consecutive lanes, valid in the group's
// last lane (with 32, row_bcast:15 adds the even row's sum into the odd row).
template <int LPR>
__device__ __forceinline__ float group_sum(float x) {
  x = row16_sum(x);
  if constexpr (LPR == 32)
    x = x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x142, 0xA, 0xF, false));
  return x;
}

template <int DK, int NW, bool EARLY>
__global__ __launch_bounds__(64 * NW, 4) void verify_chunk_kernel(Args a) {
  constexpr int NT = 64 * NW, W = 16 * NW, NCB = DK / 16;
  constexpr int R = 16;  // token rows of each half of the A operand
  using Lds = VcLds<DK, W>;
  static_assert(2 * DK <= NT, "one decay thread per channel of k and q");
  extern __shared__ float4 lds_dyn[];
  const Unit u = unit_of_block_rows(1, a.H, a.B);
  int32_t slot;
  int64_t row0;
  int Tb;
  if (!row_slot_range(a, u, slot, row0, Tb)) return;
  if (Tb == 0) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int j = lane & 15, g = lane >> 4;
  Lds L(reinterpret_cast<float *>(lds_dyn), a.T_max, R);

  // Inputs of this row and head start at uniform bases; threads add 32-bit
  // offsets. Staging items: 4 channels of k, q and alpha of one token, or 4
  // columns of v of one token.
  const uint32_t kq_tok = (uint32_t)a.H * DK, v_tok = (uint32_t)a.H * a.dv;
  const int64_t kq0 = (row0 * a.H + u.h) * DK, v0 = (row0 * a.H + u.h) * a.dv;
  const uint16_t *kbase = a.k + kq0, *qbase = a.q + kq0, *vbase = a.v + v0;
  const float *abase = a.alpha + kq0, *bbase = a.beta + row0 * a.H + u.h;
  const int nkq = Tb * (DK / 4), nv = Tb * (W / 4);
  auto kq_off = [&](int idx) { return (uint32_t)(idx / (DK / 4)) * kq_tok + (uint32_t)(idx % (DK / 4)) * 4; };
  auto v_off = [&](int idx) { return (uint32_t)(idx / (W / 4)) * v_tok + (uint32_t)(idx % (W / 4)) * 4; };
  // Vector loads complete in issue order: the first round of staging loads
  // (unconditional, at clamped in-bounds items) goes out before the state, so
  // the decay and coupling passes wait for the inputs alone and run while the
  // state is still on its way.
  const uint32_t ko0 = kq_off(min(tid, nkq - 1)), vo0 = v_off(min(tid, nv - 1));
  const uint2 kb0 = *reinterpret_cast<const uint2 *>(kbase + ko0);
  const uint2 qb0 = *reinterpret_cast<const uint2 *>(qbase + ko0);
  const float4 al0 = *reinterpret_cast<const float4 *>(abase + ko0);
  const uint2 vb0 = *reinterpret_cast<const uint2 *>(vbase + vo0);
  const float bt0 = bbase[(uint32_t)min(tid, Tb - 1) * (uint32_t)a.H];
  auto put_kq = [&](int idx, uint2 kb, uint2 qb, float4 al) {
    const int t = idx / (DK / 4), i = (idx % (DK / 4)) * 4;
    *reinterpret_cast<float4 *>(L.k + t * DK + i) = unpack_bf16x4(kb);
    *reinterpret_cast<float4 *>(L.q + t * DK + i) = unpack_bf16x4(qb);
    *reinterpret_cast<float4 *>(L.a + t * DK + i) = al;
  };
  auto put_v = [&](int idx, uint2 vb) {
    const int t = idx / (W / 4), c = (idx % (W / 4)) * 4;
    *reinterpret_cast<float4 *>(L.v + t * Lds::VS + c) = unpack_bf16x4(vb);
  };
  // With EARLY (grids of several rounds of resident workgroups), the state
  // goes out right behind the input requests and is in flight over the decay,
  // coupling and solve passes. Otherwise it is requested only before the state
  // products: its registers are then not live over the passes (61 VGPRs
  // against ~100, so twice the workgroups fit on a CU), and within one round a
  // block's inputs do not queue in HBM behind every other block's state.
  const float *Scol = a.cache + (int64_t)slot * a.slot_stride + (int64_t)u.h * a.dv * DK +
                      (uint32_t)((16 * wave + j) * DK + 4 * g);
  float4 sreg[NCB];
  auto load_state = [&]() {
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) sreg[cb] = ld4<kVerifyLoadStream>(Scol + 16 * cb);
  };
  if constexpr (EARLY) load_state();
  if (tid < nkq) put_kq(tid, kb0, qb0, al0);
  if (tid < nv) put_v(tid, vb0);
  if (tid < Tb) L.beta[tid] = bt0;
  for (int idx = tid + NT; idx < nkq; idx += NT) {
    const uint32_t off = kq_off(idx);
    put_kq(idx, *reinterpret_cast<const uint2 *>(kbase + off), *reinterpret_cast<const uint2 *>(qbase + off),
           *reinterpret_cast<const float4 *>(abase + off));
  }
  for (int idx = tid + NT; idx < nv; idx += NT) put_v(idx, *reinterpret_cast<const uint2 *>(vbase + v_off(idx)));
  __syncthreads();

  // The passes below run over all R token rows without branches (rows past
  // the row's tokens read the last token, at a uniform clamped index, and their
  // results are dropped by selects), so their loads issue together and their
  // reductions interleave.
  const int last = Tb - 1;
  // Decayed keys and queries G_t k_t, G_t q_t: one thread per channel of k or
  // q; rows T_b..R-1 are zero.
  auto decay_pass = [&](int p) {
    const int i = p % DK;
    const bool isq = p >= DK;
    const float *x = isq ? L.q : L.k;
    float *dst = L.am + (isq ? R * Lds::P : 0) + i;
    float av[R], xv[R];
#pragma unroll
    for (int t = 0; t < R; ++t) {
      const int tt = min(t, last);
      av[t] = L.a[tt * DK + i];
      xv[t] = x[tt * DK + i];
    }
    float G = 1.0f;
#pragma unroll
    for (int t = 0; t < R; ++t) {
      G = G * av[t];
      dst[t * Lds::P] = t < Tb ? G * xv[t] : 0.0f;
    }
  };
  // Coupling coefficients: thread (s, c) carries D(s, t) over its channels as
  // t advances; a group of LPR lanes shares s and sums over its channels.
  auto coupling_pass = [&](int p) {
    constexpr int LPR = kCoupleThreads / R, CPT = DK / LPR, VEC = CPT < 4 ? CPT : 4;
    const int s = p / LPR, c = p % LPR;
    int ch[CPT];
#pragma unroll
    for (int e = 0; e < CPT; ++e) ch[e] = VEC * c + VEC * LPR * (e / VEC) + e % VEC;
    float d[CPT];
#pragma unroll
    for (int e = 0; e < CPT; ++e) d[e] = L.k[min(s, last) * DK + ch[e]];
    // token rows of k, q and alpha are read LA rows ahead of their use (a ring
    // of LA + 1 rows in registers; the scheduling barrier keeps the compiler
    // from hoisting every row's loads at once)
    constexpr int LA = 1;
    float kr[LA + 1][CPT], qr[LA + 1][CPT], ar[LA + 1][CPT];
    auto load_row = [&](int t) {
      const int x0 = min(t, last) * DK, r = t % (LA + 1);
#pragma unroll
      for (int e = 0; e < CPT; ++e) {
        kr[r][e] = L.k[x0 + ch[e]];
        qr[r][e] = L.q[x0 + ch[e]];
        ar[r][e] = L.a[x0 + ch[e]];
      }
    };
#pragma unroll
    for (int t = 0; t < LA; ++t) load_row(t);
    // Partial dots of row t are summed over the group during row t + 1.
    auto finish = [&](int t, float pa, float pb) {
      pa = group_sum<LPR>(pa);
      pb = group_sum<LPR>(pb);
      if (c == LPR - 1 && s < Tb && t < Tb) {
        if (t > s) L.cA[t * 16 + s] = pa;
        if (t >= s) L.cB[t * 16 + s] = pb;
      }
    };
    float pa[R], pb[R];
#pragma unroll
    for (int t = 0; t < R; ++t) {
      if (t + LA < R) load_row(t + LA);
      const int r = t % (LA + 1);
      const bool after = t > s;
      pa[t] = 0.0f;
      pb[t] = 0.0f;
#pragma unroll
      for (int e = 0; e < CPT; ++e) {
        d[e] = after ? d[e] * ar[r][e] : d[e];
        pa[t] = __builtin_fmaf(kr[r][e], d[e], pa[t]);
        pb[t] = __builtin_fmaf(qr[r][e], d[e], pb[t]);
      }
      if (t > 0) finish(t - 1, pa[t - 1], pb[t - 1]);
      __builtin_amdgcn_sched_barrier(0);
    }
    finish(R - 1, pa[R - 1], pb[R - 1]);
  };
  if constexpr (NT >= 2 * DK + kCoupleThreads) {
    if (tid < 2 * DK) decay_pass(tid);
    if (tid >= NT - kCoupleThreads) coupling_pass(tid - (NT - kCoupleThreads));
  } else {
    if (tid < 2 * DK) decay_pass(tid);
    if (tid < kCoupleThreads) coupling_pass(tid);
  }
  __syncthreads();

  // M and N, one lane per column c, written as the A operand of the product
  // over tokens: row i of the operand is output row i of that product (O0
  // enters it as the accumulator). The coefficients are spread over the wave's lanes (entry t * R + s in lane
  // (t * R + s) % 64) and broadcast with readlane, so the substitution waits
  // for LDS once. Entries outside the row's tokens (never written) and beta
  // past them are zero, so rows t >= T_b come out as m = n = 0 without
  // branches.
  if (wave == NW - 1) {
    constexpr int PER = R * R / 64;
    float ca[PER], cbv[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int x = e * 64 + lane, tt = x / R, ss = x % R;
      const float va = L.cA[tt * 16 + ss], vb = L.cB[tt * 16 + ss];
      ca[e] = tt < Tb && ss < tt ? va : 0.0f;
      cbv[e] = tt < Tb && ss <= tt ? vb : 0.0f;
    }
    const float bt = L.beta[min(lane, last)];
    const float bl = lane < Tb ? bt : 0.0f;
    auto bcast = [](float v, int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l)); };
    const int c = lane & 15;
    float m[R], n[R];
#pragma unroll
    for (int t = 0; t < R; ++t) {
      float x = t == c ? 1.0f : 0.0f;
#pragma unroll
      for (int s = 0; s < t; ++s) x = __builtin_fmaf(-bcast(ca[(t * R + s) / 64], (t * R + s) % 64), m[s], x);
      m[t] = bcast(bl, t) * x;
      n[t] = 0.0f;
#pragma unroll
      for (int s = 0; s <= t; ++s) n[t] = __builtin_fmaf(bcast(cbv[(t * R + s) / 64], (t * R + s) % 64), m[s], n[t]);
    }
    // (written after the substitution: an LDS write inside it would make the
    // next row's wait for the coefficients wait for the write too)
    if (lane < 16) {
#pragma unroll
      for (int t = 0; t < R; ++t) {
        L.nm[t * kNStride + c] = n[t];
      }
    }
  }

  // this lane's v for the product over tokens (rows 4g..4g+3 of its column;
  // rows past the row's tokens read the last token and are dropped below)
  const int col = 16 * wave + j;
  float vv[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) vv[r] = L.v[min(4 * g + r, last) * Lds::VS + col];

  if constexpr (!EARLY) load_state();

  // U0 and O0 for the wave's 16 columns
  v4f acc = {0.0f, 0.0f, 0.0f, 0.0f}, accO = {0.0f, 0.0f, 0.0f, 0.0f};
  const float *ar = L.am + j * Lds::P + 4 * g;
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const v4f ak = *reinterpret_cast<const v4f *>(ar + 16 * cb);
    const v4f b = {sreg[cb].x, sreg[cb].y, sreg[cb].z, sreg[cb].w};
    const v4f aq = *reinterpret_cast<const v4f *>(ar + 16 * Lds::P + 16 * cb);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(ak[e], b[e], acc, 0, 0, 0);
      accO = __builtin_amdgcn_mfma_f32_16x16x4f32(aq[e], b[e], accO, 0, 0, 0);
    }
  }
  __syncthreads();

  // X = V - U0 on the key rows (zero past the row's tokens), then
  // O = O0 + N X. Lane (j, g) holds rows 4g..4g+3 of column j.
  float xb[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int t = 4 * g + r;
    xb[r] = t < Tb ? vv[r] - acc[r] : 0.0f;
  }
  v4f o = accO;
  const v4f nrow = *reinterpret_cast<const v4f *>(L.nm + j * kNStride + 4 * g);
#pragma unroll
  for (int e = 0; e < 4; ++e) o = __builtin_amdgcn_mfma_f32_16x16x4f32(nrow[e], xb[e], o, 0, 0, 0);
  float *out = a.out + v0 + col;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int t = 4 * g + r;
    if (t < Tb) out[(uint32_t)t * v_tok] = o[r];
  }

  // Replay buffers, read back from LDS: each staged value came from a bf16 or
  // fp32 input exactly, and the bf16 ones return to their bits by truncation.
  const int64_t r0 = (int64_t)u.b * a.T_max * a.H + u.h;  // row b, token 0, head h
  auto to_bf16x4 = [](float4 f) {
    return uint2{(__float_as_uint(f.x) >> 16) | (__float_as_uint(f.y) & 0xffff0000u),
                 (__float_as_uint(f.z) >> 16) | (__float_as_uint(f.w) & 0xffff0000u)};
  };
  for (int idx = tid; idx < nkq; idx += NT) {
    const int t = idx / (DK / 4), i = (idx % (DK / 4)) * 4;
    const uint32_t d = kq_off(idx);
    *reinterpret_cast<uint2 *>(a.rk + r0 * DK + d) = to_bf16x4(*reinterpret_cast<const float4 *>(L.k + t * DK + i));
    *reinterpret_cast<float4 *>(a.ralpha + r0 * DK + d) = *reinterpret_cast<const float4 *>(L.a + t * DK + i);
  }
  for (int idx = tid; idx < nv; idx += NT) {
    const int t = idx / (W / 4), c = (idx % (W / 4)) * 4;
    *reinterpret_cast<uint2 *>(a.rv + r0 * a.dv + v_off(idx)) =
        to_bf16x4(*reinterpret_cast<const float4 *>(L.v + t * Lds::VS + c));
  }
  if (tid < Tb) a.rbeta[r0 + (int64_t)tid * a.H] = L.beta[tid];
}

// ----------------------------------------------------------------------------
// Rows of at most 8 tokens: the solve folded into the token product
// ----------------------------------------------------------------------------
//
// The A operand of the state products holds the decayed keys and queries
// interleaved: operand row 4p + r is G_t k_t for token t = 2p + r (r < 2) and
// G_t q_t for token t = 2p + r - 2 (r >= 2). A lane (j, p) of the products
// thus receives u0 of tokens 2p, 2p + 1 in accumulator registers 0, 1 and o0
// of the same tokens in registers 2, 3, and registers 0, 1 are the B operand
// of a product over tokens whose step e takes token 2p + e: two MFMAs cover 8
// tokens. With X = diag(beta) (V - U0), L = diag(beta) A (strictly lower) and
// the coupling operand [-L ; B] interleaved like the products' rows, the delta
// of the chunk solves (I + L) delta = X, and the rounds
//   Y <- [X ; O0] + [-L ; B] delta,   delta <- key rows of Y
// starting from delta = X are exact for the rows of tokens 0..k after k + 1
// rounds (L is strictly lower triangular, so round k recomputes row k from
// rows 0..k-1 as forward substitution does). After T_b rounds the query rows
// of Y are O0 + B delta = O. Each round is two dependent MFMAs per wave; no
// wave runs a substitution while the others wait at a barrier.
//
// Memory order. A wave that requests its whole state tile stalls at those
// loads until the memory pipeline accepts them (at the CU's share of the HBM
// rate), and in-order issue holds up everything behind them; requested
// together with the inputs, the tile also delays the inputs, which the chain
// needs first. So the inputs are staged first, each wave then requests the
// first kVc8Ahead of its 8 column blocks, runs its part of the decay and
// coupling passes while they are in flight, and streams the remaining blocks
// kVc8Ahead ahead of the products that consume them. Measured on MI355X
// (H = 32, d = 128, T = 8, HIP graphs): B = 64 37.9 us, B = 16 11.1 us,
// B = 4 6.2 us, against 39.7, 11.6 and 7.4 us with the whole tile requested
// with the inputs or after the passes; 2 or 8 blocks ahead were slower.
constexpr int kC8Stride = 12;  // row stride of the [16][8] coupling operand (conflict-free 64-bit reads)
constexpr int kVc8Ahead = 4;   // state column blocks in flight ahead of their products

template <int DK, int W>
struct Vc8Lds {
  static constexpr int P = DK + 4;  // row stride of the A operand of the state products
  static constexpr int VS = W + 4;  // row stride of the staged v
  float *k, *a, *q;                 // [T_max][DK] staged inputs
  float *v;                         // [T_max][VS]
  float *beta;                      // [16]
  float *am;                        // [16][P]: interleaved G_t k_t and G_t q_t rows
  float *cm;                        // [16][kC8Stride]: interleaved -L and B rows, columns s = 0..7
  __device__ Vc8Lds(float *base, int T_max) {
    k = base;
    a = k + T_max * DK;
    q = a + T_max * DK;
    v = q + T_max * DK;
    beta = v + T_max * VS;
    am = beta + 16;
    cm = am + 16 * P;
  }
};

// operand row of token t's key (its query: + 2)
__device__ __forceinline__ int c8_row(int t) { return 4 * (t >> 1) + (t & 1); }

template <int DK, int NW>
__global__ __launch_bounds__(64 * NW, 2) void verify_chunk8_kernel(Args a) {
  constexpr int NT = 64 * NW, W = 16 * NW, NCB = DK / 16, R = 8;
  using Lds = Vc8Lds<DK, W>;
  static_assert(2 * DK <= NT, "one decay thread per channel of k and q");
  extern __shared__ float4 lds_dyn[];
  const Unit u = unit_of_block_rows(1, a.H, a.B);
  int32_t slot;
  int64_t row0;
  int Tb;
  if (!row_slot_range(a, u, slot, row0, Tb)) return;
  if (Tb == 0) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int j = lane & 15, g = lane >> 4;
  Lds L(reinterpret_cast<float *>(lds_dyn), a.T_max);

  // inputs of this row and head start at uniform bases; staging items are 4
  // channels of k, q and alpha of one token, or 4 columns of v of one token
  const uint32_t kq_tok = (uint32_t)a.H * DK, v_tok = (uint32_t)a.H * a.dv;
  const int64_t kq0 = (row0 * a.H + u.h) * DK, v0 = (row0 * a.H + u.h) * a.dv;
  const uint16_t *kbase = a.k + kq0, *qbase = a.q + kq0, *vbase = a.v + v0;
  const float *abase = a.alpha + kq0, *bbase = a.beta + row0 * a.H + u.h;
  const int nkq = Tb * (DK / 4), nv = Tb * (W / 4);
  auto kq_off = [&](int idx) { return (uint32_t)(idx / (DK / 4)) * kq_tok + (uint32_t)(idx % (DK / 4)) * 4; };
  auto v_off = [&](int idx) { return (uint32_t)(idx / (W / 4)) * v_tok + (uint32_t)(idx % (W / 4)) * 4; };
  const uint32_t ko0 = kq_off(min(tid, nkq - 1)), vo0 = v_off(min(tid, nv - 1));
  const uint2 kb0 = *reinterpret_cast<const uint2 *>(kbase + ko0);
  const uint2 qb0 = *reinterpret_cast<const uint2 *>(qbase + ko0);
  const float4 al0 = *reinterpret_cast<const float4 *>(abase + ko0);
  const uint2 vb0 = *reinterpret_cast<const uint2 *>(vbase + vo0);
  const float bt0 = bbase[(uint32_t)min(tid, Tb - 1) * (uint32_t)a.H];
  auto put_kq = [&](int idx, uint2 kb, uint2 qb, float4 al) {
    const int t = idx / (DK / 4), i = (idx % (DK / 4)) * 4;
    *reinterpret_cast<float4 *>(L.k + t * DK + i) = unpack_bf16x4(kb);
    *reinterpret_cast<float4 *>(L.q + t * DK + i) = unpack_bf16x4(qb);
    *reinterpret_cast<float4 *>(L.a + t * DK + i) = al;
  };
  auto put_v = [&](int idx, uint2 vb) {
    const int t = idx / (W / 4), c = (idx % (W / 4)) * 4;
    *reinterpret_cast<float4 *>(L.v + t * Lds::VS + c) = unpack_bf16x4(vb);
  };
  if (tid < nkq) put_kq(tid, kb0, qb0, al0);
  if (tid < nv) put_v(tid, vb0);
  if (tid < Tb) L.beta[tid] = bt0;
  for (int idx = tid + NT; idx < nkq; idx += NT) {
    const uint32_t off = kq_off(idx);
    put_kq(idx, *reinterpret_cast<const uint2 *>(kbase + off), *reinterpret_cast<const uint2 *>(qbase + off),
           *reinterpret_cast<const float4 *>(abase + off));
  }
  for (int idx = tid + NT; idx < nv; idx += NT) put_v(idx, *reinterpret_cast<const uint2 *>(vbase + v_off(idx)));
  __syncthreads();

  // the state in the v_mfma_f32_16x16x4f32 B layout: lane (j, g) holds channels
  // 16 cb + 4 g .. + 3 of column 16 wave + j, one 128-bit load per block cb
  const float *Scol = a.cache + (int64_t)slot * a.slot_stride + (int64_t)u.h * a.dv * DK +
                      (uint32_t)((16 * wave + j) * DK + 4 * g);
  float4 sreg[NCB];
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int cb = 0; cb < kVc8Ahead; ++cb) sreg[cb] = ld4<kVerifyLoadStream>(Scol + 16 * cb);
  __builtin_amdgcn_sched_barrier(0);

  // Both passes run over all 8 token rows without branches: rows past the
  // row's tokens read the last token at a clamped index and their results
  // are dropped by selects.
  const int last = Tb - 1;
  // decayed keys and queries, one thread per channel of k or q, in the
  // interleaved row order; rows of tokens T_b..7 are zero
  auto decay_pass = [&](int p) {
    const int i = p % DK;
    const bool isq = p >= DK;
    const float *x = isq ? L.q : L.k;
    float *dst = L.am + (isq ? 2 : 0) * Lds::P + i;
    float av[R], xv[R];
#pragma unroll
    for (int t = 0; t < R; ++t) {
      const int tt = min(t, last);
      av[t] = L.a[tt * DK + i];
      xv[t] = x[tt * DK + i];
    }
    float G = 1.0f;
#pragma unroll
    for (int t = 0; t < R; ++t) {
      G = G * av[t];
      dst[c8_row(t) * Lds::P] = t < Tb ? G * xv[t] : 0.0f;
    }
  };
  // coupling coefficients: group s of 32 lanes carries D(s, t) over its
  // channels as t advances (running products, no division); the group's last
  // lane writes column s of the interleaved operand: -beta_t A_ts on token t's
  // key row (t > s), B_ts on its query row (t >= s), zero elsewhere
  auto coupling_pass = [&](int p) {
    constexpr int LPR = 32, CPT = DK / LPR, VEC = CPT < 4 ? CPT : 4;
    const int s = p / LPR, c = p % LPR;
    int ch[CPT];
#pragma unroll
    for (int e = 0; e < CPT; ++e) ch[e] = VEC * c + VEC * LPR * (e / VEC) + e % VEC;
    float d[CPT];
#pragma unroll
    for (int e = 0; e < CPT; ++e) d[e] = L.k[min(s, last) * DK + ch[e]];
    // token rows are read LA rows ahead of their use (a ring of LA + 1 rows in
    // registers; the scheduling barrier keeps the compiler from hoisting every
    // row's loads at once)
    constexpr int LA = 2;
    float kr[LA + 1][CPT], qr[LA + 1][CPT], ar[LA + 1][CPT];
    auto load_row = [&](int t) {
      const int x0 = min(t, last) * DK, r = t % (LA + 1);
#pragma unroll
      for (int e = 0; e < CPT; ++e) {
        kr[r][e] = L.k[x0 + ch[e]];
        qr[r][e] = L.q[x0 + ch[e]];
        ar[r][e] = L.a[x0 + ch[e]];
      }
    };
#pragma unroll
    for (int t = 0; t < LA; ++t) load_row(t);
    float pa[R], pb[R];
#pragma unroll
    for (int t = 0; t < R; ++t) {
      if (t + LA < R) load_row(t + LA);
      const int r = t % (LA + 1);
      const bool after = t > s;
      pa[t] = 0.0f;
      pb[t] = 0.0f;
#pragma unroll
      for (int e = 0; e < CPT; ++e) {
        d[e] = after ? d[e] * ar[r][e] : d[e];
        pa[t] = __builtin_fmaf(kr[r][e], d[e], pa[t]);
        pb[t] = __builtin_fmaf(qr[r][e], d[e], pb[t]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // the 16 sums of each group run together, interleaved
#pragma unroll
    for (int t = 0; t < R; ++t) {
      pa[t] = group_sum<LPR>(pa[t]);
      pb[t] = group_sum<LPR>(pb[t]);
    }
    if (c == LPR - 1) {
      const bool live_s = s < Tb;
      float bt[R];
#pragma unroll
      for (int t = 0; t < R; ++t) bt[t] = L.beta[min(t, last)];
#pragma unroll
      for (int t = 0; t < R; ++t) {
        const bool live = live_s && t < Tb;
        L.cm[c8_row(t) * kC8Stride + s] = live && t > s ? -bt[t] * pa[t] : 0.0f;
        L.cm[(c8_row(t) + 2) * kC8Stride + s] = live && t >= s ? pb[t] : 0.0f;
      }
    }
  };
  if constexpr (NT >= 2 * DK + kCoupleThreads) {
    if (tid < 2 * DK) decay_pass(tid);
    if (tid >= NT - kCoupleThreads) coupling_pass(tid - (NT - kCoupleThreads));
  } else {
    if (tid < 2 * DK) decay_pass(tid);
    if (tid < kCoupleThreads) coupling_pass(tid);
  }
  __syncthreads();

  // this lane's tokens 2g, 2g + 1 of column col: v and beta (beta zero past T_b)
  const int col = 16 * wave + j;
  float xv[2], bv[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int t = 2 * g + r;
    xv[r] = L.v[min(t, last) * Lds::VS + col];
    bv[r] = t < Tb ? L.beta[min(t, last)] : 0.0f;
  }
  // this lane's part of the coupling operand: row j, tokens 2g, 2g + 1
  const float2 cop = *reinterpret_cast<const float2 *>(L.cm + j * kC8Stride + 2 * g);

  // U0 and O0, each column block as it arrives, the later blocks requested
  // kVc8Ahead ahead of their use. Blocks 2m and 2m + 1 are the two halves of
  // one 128-byte line of each column and are requested together: requested
  // apart, the streaming load let the line leave L2 between the halves (4.6%
  // more HBM reads than the state at B = 64, by the TCC_EA0 request counts).
  static_assert(kVc8Ahead % 2 == 0, "line halves requested together");
  v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
  const float *ar = L.am + j * Lds::P + 4 * g;
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    if (cb % 2 == 0 && cb + kVc8Ahead + 1 < NCB) {
      __builtin_amdgcn_sched_barrier(0);
      sreg[cb + kVc8Ahead] = ld4<kVerifyLoadStream>(Scol + 16 * (cb + kVc8Ahead));
      sreg[cb + kVc8Ahead + 1] = ld4<kVerifyLoadStream>(Scol + 16 * (cb + kVc8Ahead + 1));
      __builtin_amdgcn_sched_barrier(0);
    }
    const v4f ak = *reinterpret_cast<const v4f *>(ar + 16 * cb);
    const v4f b = {sreg[cb].x, sreg[cb].y, sreg[cb].z, sreg[cb].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(ak[e], b[e], acc, 0, 0, 0);
  }
  // [X ; O0] and the rounds
  const v4f c0 = {bv[0] * (xv[0] - acc[0]), bv[1] * (xv[1] - acc[1]), acc[2], acc[3]};
  v4f y = c0;
  for (int it = 0; it < Tb; ++it) {
    const float d0 = y[0], d1 = y[1];
    y = __builtin_amdgcn_mfma_f32_16x16x4f32(cop.x, d0, c0, 0, 0, 0);
    y = __builtin_amdgcn_mfma_f32_16x16x4f32(cop.y, d1, y, 0, 0, 0);
  }
  float *out = a.out + v0 + col;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int t = 2 * g + r;
    if (t < Tb) out[(uint32_t)t * v_tok] = y[2 + r];
  }

  // Replay buffers, read back from LDS: each staged value came from a bf16 or
  // fp32 input exactly, and the bf16 ones return to their bits by truncation.
  const int64_t r0 = (int64_t)u.b * a.T_max * a.H + u.h;  // row b, token 0, head h
  auto to_bf16x4 = [](float4 f) {
    return uint2{(__float_as_uint(f.x) >> 16) | (__float_as_uint(f.y) & 0xffff0000u),
                 (__float_as_uint(f.z) >> 16) | (__float_as_uint(f.w) & 0xffff0000u)};
  };
  for (int idx = tid; idx < nkq; idx += NT) {
    const int t = idx / (DK / 4), i = (idx % (DK / 4)) * 4;
    const uint32_t d = kq_off(idx);
    *reinterpret_cast<uint2 *>(a.rk + r0 * DK + d) = to_bf16x4(*reinterpret_cast<const float4 *>(L.k + t * DK + i));
    *reinterpret_cast<float4 *>(a.ralpha + r0 * DK + d) = *reinterpret_cast<const float4 *>(L.a + t * DK + i);
  }
  for (int idx = tid; idx < nv; idx += NT) {
    const int t = idx / (W / 4), c = (idx % (W / 4)) * 4;
    *reinterpret_cast<uint2 *>(a.rv + r0 * a.dv + v_off(idx)) =
        to_bf16x4(*reinterpret_cast<const float4 *>(L.v + t * Lds::VS + c));
  }
  if (tid < Tb) a.rbeta[r0 + (int64_t)tid * a.H] = L.beta[tid];
}

template <int DK, int NW>
const void *pick(int T_max, bool early) {
  if (T_max <= 8) return (const void *)verify_chunk8_kernel<DK, NW>;
  return early ? (const void *)verify_chunk_kernel<DK, NW, true> : (const void *)verify_chunk_kernel<DK, NW, false>;
}

}  // namespace

size_t chunk_verify_lds_bytes(int dk, int dv, int T_max) {
  if (T_max <= 8)
    return ((size_t)3 * T_max * dk + (size_t)T_max * (dv + 4) + 16 + 16 * (dk + 4) + 16 * kC8Stride) * sizeof(float);
  const size_t floats = (size_t)3 * T_max * dk + (size_t)T_max * (dv + 4) + 16 + 2 * 16 * (dk + 4) + 2 * 256 +
                        16 * kNStride;
  return floats * sizeof(float);
}

const void *verify_chunk_kernel_for(int dk, int dv, int T_max, int64_t groups) {
  // rows of up to 16 tokens, more than one round of resident workgroups: 16
  // waves per CU at that kernel's ~100-120 VGPRs, i.e. 4096 / NW workgroups on
  // MI355X's 256 CUs
  const int nw = dv / 16;
  const bool early = groups > 4096 / nw;
  if (dk == 64) return dv == 64 ? pick<64, 4>(T_max, early) : dv == 128 ? pick<64, 8>(T_max, early) : nullptr;
  if (dk == 128) return dv == 64 ? pick<128, 4>(T_max, early) : dv == 128 ? pick<128, 8>(T_max, early) : nullptr;
  return nullptr;
}

}  // namespace kda
