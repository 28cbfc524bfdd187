// Measurement-support kernels: a streaming read (achievable HBM bandwidth)
// and a cache-flushing writer.  Not part of the attention path.
#include <hip/hip_runtime.h>

#include "pa_device.h"
#include "pagedattn.h"
#include "pagedattn_bench.h"

namespace pa {
namespace {

constexpr int kReadGrid = 8192;   // one wavefront each; ~32 per compute unit
constexpr int kReadThreads = 256;  // fill kernel block
constexpr int kUnroll = 8;         // 1 KB loads in flight per wavefront

// Each wavefront streams one contiguous range: every load instruction reads
// 1 KB (64 lanes x 16 B, consecutive), kUnroll of them in flight.
__global__ __launch_bounds__(64) void stream_read_kernel(const u32x4* __restrict__ src, size_t n16,
                                                         uint32_t* sink) {
  const int lane = threadIdx.x;
  const size_t per = ((n16 + gridDim.x - 1) / gridDim.x + 63) & ~(size_t)63;
  const size_t begin = (size_t)blockIdx.x * per;
  const size_t end = begin + per < n16 ? begin + per : n16;
  uint32_t acc = 0;
  size_t i = begin + lane;
  for (; i + (kUnroll - 1) * 64 < end; i += kUnroll * 64) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * 64);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < end; i += 64) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, off, 64);
  if (lane == 0 && acc != 0u) atomicXor(sink, acc);
}

__global__ __launch_bounds__(kReadThreads) void fill_kernel(u32x4* __restrict__ dst, size_t n16, uint32_t value) {
  const size_t stride = (size_t)gridDim.x * kReadThreads;
  const u32x4 v = {value, value, value, value};
  for (size_t i = (size_t)blockIdx.x * kReadThreads + threadIdx.x; i < n16; i += stride)
    __builtin_nontemporal_store(v, dst + i);
}

int check(const void* p, size_t bytes) {
  if (!p) return PA_ERR_NULL;
  if ((bytes & 15) || (reinterpret_cast<uintptr_t>(p) & 15)) return PA_ERR_SIZE;
  return PA_OK;
}

}  // namespace
}  // namespace pa

extern "C" int pa_bench_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  int st = pa::check(src, bytes);
  if (st) return st;
  if (!sink) return PA_ERR_NULL;
  if (bytes == 0) return PA_OK;
  hipLaunchKernelGGL(pa::stream_read_kernel, dim3(pa::kReadGrid), dim3(64), 0,
                     static_cast<hipStream_t>(stream), static_cast<const pa::u32x4*>(src), bytes / 16, sink);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? PA_OK : (int)e;
}

extern "C" int pa_bench_fill(void* dst, size_t bytes, uint32_t value, void* stream) {
  int st = pa::check(dst, bytes);
  if (st) return st;
  if (bytes == 0) return PA_OK;
  hipLaunchKernelGGL(pa::fill_kernel, dim3(pa::kReadGrid), dim3(pa::kReadThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<pa::u32x4*>(dst), bytes / 16, value);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? PA_OK : (int)e;
}
