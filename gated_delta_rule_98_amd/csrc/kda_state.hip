// kda_state.hip - head- and column-range state transfer (kda_state_pack / kda_state_unpack).

#include "kda_engine.h"

namespace kda {
namespace {

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

}  // namespace

const void *state_copy_kernel_for(bool pack) {
  return pack ? (const void *)state_copy_kernel<true> : (const void *)state_copy_kernel<false>;
}

}  // namespace kda
