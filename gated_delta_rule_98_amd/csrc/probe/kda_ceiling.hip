// kda_ceiling.hip - HBM ceiling probes for the benchmark (libkda_ceiling.so).
//
// Not part of the KDA library or its C ABI: plain streams over device memory
// with the access shape of the single-token step's state traffic (one 128-bit
// access per lane, one wave per workgroup, non-temporal hints), so that the
// benchmark can report the rate a kernel with no arithmetic reaches on the same
// bytes. Every call checks its sizes on the host, enqueues one kernel on
// `stream` and returns 0, or returns -1 for bad arguments and -4 when the
// launch fails. n counts floats and must be a positive multiple of 256.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

// in place: x <- x * (1 - 2^-24), read and written once
__global__ __launch_bounds__(64) void rmw_kernel(v4f *p) {
  const int64_t i = (int64_t)blockIdx.x * 64 + threadIdx.x;
  v4f x = __builtin_nontemporal_load(p + i);
  x = x * 0.99999994f;
  __builtin_nontemporal_store(x, p + i);
}

__global__ __launch_bounds__(64) void copy_kernel(const v4f *src, v4f *dst) {
  const int64_t i = (int64_t)blockIdx.x * 64 + threadIdx.x;
  __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

// read only; the sum is stored only if it equals a value no finite input of
// the benchmark produces, so the loads cannot be removed
__global__ __launch_bounds__(64) void read_kernel(const v4f *p, float *sink) {
  const int64_t i = (int64_t)blockIdx.x * 64 + threadIdx.x;
  const v4f x = __builtin_nontemporal_load(p + i);
  const float s = x.x + x.y + x.z + x.w;
  if (s == -1234.5678f) sink[threadIdx.x] = s;
}

int grid_of(int64_t n, unsigned *grid) {
  if (n <= 0 || n % 256 != 0 || n / 256 > 0x7fffffff) return -1;
  *grid = (unsigned)(n / 256);
  return 0;
}

}  // namespace

extern "C" {

int kda_ceiling_rmw(float *p, int64_t n, void *stream) {
  unsigned grid;
  if (!p || grid_of(n, &grid)) return -1;
  hipLaunchKernelGGL(rmw_kernel, dim3(grid), dim3(64), 0, (hipStream_t)stream, reinterpret_cast<v4f *>(p));
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int kda_ceiling_copy(const float *src, float *dst, int64_t n, void *stream) {
  unsigned grid;
  if (!src || !dst || grid_of(n, &grid)) return -1;
  hipLaunchKernelGGL(copy_kernel, dim3(grid), dim3(64), 0, (hipStream_t)stream,
                     reinterpret_cast<const v4f *>(src), reinterpret_cast<v4f *>(dst));
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int kda_ceiling_read(const float *p, int64_t n, float *sink, void *stream) {
  unsigned grid;
  if (!p || !sink || grid_of(n, &grid)) return -1;
  hipLaunchKernelGGL(read_kernel, dim3(grid), dim3(64), 0, (hipStream_t)stream, reinterpret_cast<const v4f *>(p),
                     sink);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
