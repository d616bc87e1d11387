// Measurement probes for the benchmark's ceiling modes, built into their own
// library (libtaprobes.so) so the product library carries none of them:
//
//   ta_probe_read   a plain streaming read of a buffer (16-byte nontemporal
//                   loads, eight in flight per thread, XOR-folded so the loads
//                   stay live): the practical HBM read rate a read-bound kernel
//                   can reach on this GPU at a given size.
//   ta_probe_empty  a kernel that does nothing: launch-to-launch cost of a grid
//                   of a given size, the floor under any one-launch call.
//
// Neither is on the tree attention path.  Both return 0, or the HIP error.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#define PROBE_API extern "C" __attribute__((visibility("default")))

namespace {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 8;

__global__ __launch_bounds__(kReadThreads) void read_kernel(const u32x4_t* __restrict__ src,
                                                            size_t n16, unsigned* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * kReadThreads;
  size_t i = (size_t)blockIdx.x * kReadThreads + threadIdx.x;
  unsigned acc = 0;
  for (; i + (kReadUnroll - 1) * stride < n16; i += kReadUnroll * stride) {
    u32x4_t v[kReadUnroll];
#pragma unroll
    for (int k = 0; k < kReadUnroll; ++k) v[k] = __builtin_nontemporal_load(src + i + k * stride);
#pragma unroll
    for (int k = 0; k < kReadUnroll; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  for (; i < n16; i += stride) {
    const u32x4_t v = __builtin_nontemporal_load(src + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  // One word per thread would be a second stream; a per-block fold is enough
  // to keep every load live.
  acc = __reduce_xor_sync(~0ull, acc);
  if ((threadIdx.x & 63) == 0) atomicXor(sink + blockIdx.x, acc);
}

__global__ void empty_kernel() {}

}  // namespace

// src: device buffer of `bytes` bytes (16-byte aligned; bytes a multiple of
// 16); sink: device array of `grid` uint32 (XOR-accumulated, any content);
// grid: workgroups of 256 threads (1 .. 2^20).  Asynchronous on `stream`.
PROBE_API int ta_probe_read(const void* src, size_t bytes, void* sink, int grid, void* stream) {
  if (!src || !sink || grid < 1 || grid > (1 << 20) || bytes % 16 != 0 ||
      (reinterpret_cast<uintptr_t>(src) & 15) != 0)
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(read_kernel, dim3((unsigned)grid), dim3(kReadThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4_t*>(src),
                     bytes / 16, static_cast<unsigned*>(sink));
  return (int)hipGetLastError();
}

// An empty grid of `grid` workgroups of `block` threads (1 .. 1024).
PROBE_API int ta_probe_empty(int grid, int block, void* stream) {
  if (grid < 1 || grid > (1 << 20) || block < 1 || block > 1024) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(empty_kernel, dim3((unsigned)grid), dim3((unsigned)block), 0,
                     static_cast<hipStream_t>(stream));
  return (int)hipGetLastError();
}
