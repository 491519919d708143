// Streaming-read reference kernel: reads a buffer once with the same 16-byte
// nontemporal loads the attention uses for the cache, with two workgroups per
// compute unit, so a benchmark can state the attention's bandwidth against
// what a plain read achieves on the same device. Not part of the decode path.
#include "../../include/mlra.h"
#include "common.h"

namespace mlra {
namespace {

constexpr int kReadThreads = 256;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const u32x4_t gu32x4_t;

__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const u32x4_t* src, int64_t n,
                                                                   uint32_t* sink) {
  __shared__ uint32_t red[kReadThreads];
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kReadThreads;
  int64_t i = static_cast<int64_t>(blockIdx.x) * kReadThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const u32x4_t a = __builtin_nontemporal_load((gu32x4_t*)(src + i));
    const u32x4_t b = __builtin_nontemporal_load((gu32x4_t*)(src + i + stride));
    const u32x4_t c = __builtin_nontemporal_load((gu32x4_t*)(src + i + 2 * stride));
    const u32x4_t d = __builtin_nontemporal_load((gu32x4_t*)(src + i + 3 * stride));
    const u32x4_t x = a ^ b ^ c ^ d;
    acc ^= x[0] ^ x[1] ^ x[2] ^ x[3];
  }
  for (; i < n; i += stride) {
    const u32x4_t a = __builtin_nontemporal_load((gu32x4_t*)(src + i));
    acc ^= a[0] ^ a[1] ^ a[2] ^ a[3];
  }
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int s = kReadThreads / 2; s > 0; s >>= 1) {
    if (threadIdx.x < s) red[threadIdx.x] ^= red[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0];
}

int read_workgroups() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  return 2 * n;
}

}  // namespace
}  // namespace mlra

extern "C" int mlra_stream_read(const void* src, size_t bytes, void* sink, size_t sink_bytes,
                                void* stream) {
  using namespace mlra;
  if (!src || !sink || bytes % 16 != 0) return MLRA_ERR_INVALID_ARG;
  const int wg = read_workgroups();
  if (sink_bytes < sizeof(uint32_t) * static_cast<size_t>(wg)) return MLRA_ERR_INVALID_ARG;
  stream_read_kernel<<<wg, kReadThreads, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const u32x4_t*>(src), static_cast<int64_t>(bytes / 16), static_cast<uint32_t*>(sink));
  return hipGetLastError() == hipSuccess ? MLRA_OK : MLRA_ERR_HIP;
}
