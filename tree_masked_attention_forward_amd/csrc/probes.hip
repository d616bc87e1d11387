// Measurement probes for the benchmark's ceiling modes, built into their own
// library (libtaprobes.so) so the product library carries none of them:
//
//   ta_probe_read   a plain streaming read of a buffer (16-byte nontemporal
//                   loads, eight in flight per thread, XOR-folded so the loads
//                   stay live): the practical HBM read rate a read-bound kernel
//                   can reach on this GPU at a given size.
//   ta_probe_empty  a kernel that does nothing: launch-to-launch cost of a grid
//                   of a given size, the floor under any one-launch call.
//   ta_probe_mfma   back-to-back independent v_mfma_f32_32x32x16_bf16 chains:
//                   the matrix units' sustained bf16 rate.
//   ta_probe_valu   independent fp32 FMA or exp2 chains: VALU issue rates.
//
// None is on the tree attention path.  Each returns 0, or the HIP error.
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

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// Four independent chains of v_mfma_f32_32x32x16_bf16 per wave, `iters` steps
// each: enough independent work to keep a SIMD's matrix unit issuing.
__global__ __launch_bounds__(512) void mfma_kernel(int iters, float* __restrict__ sink) {
  bf16x8_t a, b;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    a[k] = (__bf16)(0.001f * (threadIdx.x + k));
    b[k] = (__bf16)(0.002f * (threadIdx.x - k));
  }
  f32x16_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float t = 0.f;
#pragma unroll
  for (int v = 0; v < 16; ++v) t += c0[v] + c1[v] + c2[v] + c3[v];
  if (t == 1.2345f) sink[blockIdx.x] = t;   // keeps the chains live; never true in practice
}

// VALU rates: eight independent fp32 FMA chains (op = 0) or exp2 chains
// (op = 1) per thread, `iters` steps each.
__global__ __launch_bounds__(512) void valu_kernel(int iters, int op, float* __restrict__ sink) {
  float x[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) x[k] = 0.5f + 1e-3f * (threadIdx.x + k);
  if (op == 0) {
    for (int i = 0; i < iters; ++i)
#pragma unroll
      for (int k = 0; k < 8; ++k) x[k] = __builtin_fmaf(x[k], 0.999f, 1e-4f);
  } else {
    for (int i = 0; i < iters; ++i)
#pragma unroll
      for (int k = 0; k < 8; ++k) x[k] = __builtin_amdgcn_exp2f(-x[k]);
  }
  float t = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) t += x[k];
  if (t == 1.2345f) sink[blockIdx.x] = t;
}

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

// grid workgroups of 512 threads (8 waves, two per SIMD), each wave issuing
// 4 * iters MFMAs of 32x32x16 (32768 flops each).  sink: grid floats.
PROBE_API int ta_probe_mfma(int grid, int iters, void* sink, void* stream) {
  if (grid < 1 || grid > (1 << 20) || iters < 1 || !sink) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_kernel, dim3((unsigned)grid), dim3(512), 0,
                     static_cast<hipStream_t>(stream), iters, static_cast<float*>(sink));
  return (int)hipGetLastError();
}

// grid workgroups of 512 threads, each thread running 8 * iters FMAs (op 0)
// or exp2s (op 1).  sink: grid floats.
PROBE_API int ta_probe_valu(int grid, int iters, int op, void* sink, void* stream) {
  if (grid < 1 || grid > (1 << 20) || iters < 1 || (op != 0 && op != 1) || !sink)
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(valu_kernel, dim3((unsigned)grid), dim3(512), 0,
                     static_cast<hipStream_t>(stream), iters, op, static_cast<float*>(sink));
  return (int)hipGetLastError();
}
