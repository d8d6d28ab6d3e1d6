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
// selected columns are one contiguous span of ncols * dk floats. Each
// workgroup is one wave that moves 64 float4 (1 KiB) of one (row, head) span,
// so there are many small workgroups in flight. Measured on MI355X for 64 rows
// x 32 heads, d = 128 (128 MiB each way): pack 39.3 us and unpack 41.0 us,
// where one 256-lane workgroup looping over each whole span took 44.2 and
// 52.9 us. Several float4 per lane (2 to 8, wave counts 1 to 16) came out
// equal or slower, and streaming (nontemporal) hints cost 2-4 us here. buf
// may be pinned host memory: the kernel then reads or writes it over PCIe.

constexpr int kCopyLanes = 64;

template <bool PACK>
__global__ __launch_bounds__(kCopyLanes) void state_copy_kernel(PackArgs p) {
  const int span = blockIdx.x / p.parts, part = blockIdx.x % p.parts;
  const int b = span / p.nheads, hh = span % p.nheads;
  const int32_t slot = p.slot_ids[b];
  if (slot < 0) return;
  if (slot >= p.num_slots) {
    if (p.dev_err && hh == 0 && part == 0 && threadIdx.x == 0) atomicOr(p.dev_err, KDA_DEVERR_SLOT);
    return;
  }
  const int i = part * kCopyLanes + threadIdx.x;
  if (i >= p.ncols * p.dk / 4) return;
  float *src = p.cache + (int64_t)slot * p.slot_stride + ((int64_t)(p.head0 + hh) * p.dv + p.col0) * p.dk;
  float *dst = p.buf + ((int64_t)b * p.nheads + hh) * (int64_t)p.ncols * p.dk;
  if (!PACK) {
    float *t = src;
    src = dst;
    dst = t;
  }
  reinterpret_cast<float4 *>(dst)[i] = reinterpret_cast<const float4 *>(src)[i];
}

}  // namespace

int state_copy_lanes() { return kCopyLanes; }

const void *state_copy_kernel_for(bool pack) {
  return pack ? (const void *)state_copy_kernel<true> : (const void *)state_copy_kernel<false>;
}

}  // namespace kda
