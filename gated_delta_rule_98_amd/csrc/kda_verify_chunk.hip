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
// With up to 8 tokens the decayed keys (rows 0..7) and queries (rows 8..15)
// share one 16-row A operand, so one product chain gives U0 and O0 together;
// longer rows use one 16-row chain for each.

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

template <int DK, int NW, bool STACK, bool EARLY>
__global__ __launch_bounds__(64 * NW, 4) void verify_chunk_kernel(Args a) {
  constexpr int NT = 64 * NW, W = 16 * NW, NCB = DK / 16;
  constexpr int R = STACK ? 8 : 16;  // token rows of each half of the A operand
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
    constexpr int LA = STACK ? 2 : 1;
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
    // Partial dots of row t are summed over the group: with 8 rows all at
    // the end (16 independent reductions interleave); with 16 rows during row
    // t + 1 (fewer registers).
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
      if constexpr (!STACK) {
        if (t > 0) finish(t - 1, pa[t - 1], pb[t - 1]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (STACK) {
#pragma unroll
      for (int t = 0; t < R; ++t) {
        pa[t] = group_sum<LPR>(pa[t]);
        pb[t] = group_sum<LPR>(pb[t]);
      }
      if (c == LPR - 1 && s < Tb) {
#pragma unroll
        for (int t = 0; t < R; ++t) {
          if (t < Tb && t > s) L.cA[t * 16 + s] = pa[t];
          if (t < Tb && t >= s) L.cB[t * 16 + s] = pb[t];
        }
      }
    } else {
      finish(R - 1, pa[R - 1], pb[R - 1]);
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

  // M and N, one lane per column c, written as the A operand of the product
  // over tokens: row i of the operand is output row i of that product (with
  // stacked halves, output rows 8..15 are the queries' rows, and operand
  // columns 8..15 meet O0, which enters as the accumulator instead). The
  // coefficients are spread over the wave's lanes (entry t * R + s in lane
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
        L.nm[(STACK ? R + t : t) * kNStride + c] = n[t];
        if constexpr (STACK) L.nm[t * kNStride + c] = 0.0f;
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
    if constexpr (STACK) {
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(ak[e], b[e], acc, 0, 0, 0);
    } else {
      const v4f aq = *reinterpret_cast<const v4f *>(ar + 16 * Lds::P + 16 * cb);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(ak[e], b[e], acc, 0, 0, 0);
        accO = __builtin_amdgcn_mfma_f32_16x16x4f32(aq[e], b[e], accO, 0, 0, 0);
      }
    }
  }
  __syncthreads();

  // X = V - U0 on the key rows (zero past the row's tokens), then
  // O = O0 + N X. Lane (j, g) holds rows 4g..4g+3 of column j.
  float xb[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int t = 4 * g + r;
    xb[r] = t < Tb && t < R ? vv[r] - acc[r] : 0.0f;
  }
  v4f o = STACK ? acc : accO;
  const v4f nrow = *reinterpret_cast<const v4f *>(L.nm + j * kNStride + 4 * g);
#pragma unroll
  for (int e = 0; e < 4; ++e) o = __builtin_amdgcn_mfma_f32_16x16x4f32(nrow[e], xb[e], o, 0, 0, 0);
  float *out = a.out + v0 + col;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int t = STACK ? 4 * g + r - R : 4 * g + r;
    if (t >= 0 && t < Tb) out[(uint32_t)t * v_tok] = o[r];
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
const void *pick(bool stack, bool early) {
  if (early)
    return stack ? (const void *)verify_chunk_kernel<DK, NW, true, true>
                 : (const void *)verify_chunk_kernel<DK, NW, false, true>;
  return stack ? (const void *)verify_chunk_kernel<DK, NW, true, false>
               : (const void *)verify_chunk_kernel<DK, NW, false, false>;
}

}  // namespace

size_t chunk_verify_lds_bytes(int dk, int dv, int T_max) {
  const size_t R = T_max <= 8 ? 8 : 16;
  const size_t floats = (size_t)3 * T_max * dk + (size_t)T_max * (dv + 4) + 16 + 2 * R * (dk + 4) + 2 * 256 +
                        16 * kNStride;
  return floats * sizeof(float);
}

const void *verify_chunk_kernel_for(int dk, int dv, int T_max, int64_t groups) {
  const bool stack = T_max <= 8;
  // more than one round of resident workgroups: 16 waves per CU at these
  // kernels' ~100-120 VGPRs, i.e. 4096 / NW workgroups on MI355X's 256 CUs
  const int nw = dv / 16;
  const bool early = groups > 4096 / nw;
  if (dk == 64) return dv == 64 ? pick<64, 4>(stack, early) : dv == 128 ? pick<64, 8>(stack, early) : nullptr;
  if (dk == 128) return dv == 64 ? pick<128, 4>(stack, early) : dv == 128 ? pick<128, 8>(stack, early) : nullptr;
  return nullptr;
}

}  // namespace kda
