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
//   ta_probe_lds    16-byte LDS reads with no bank conflicts (op 0), or the
//                   same reads each feeding a v_mfma_f32_32x32x16_bf16 as its
//                   A operand, eight per 32x128 tile as the attention's score
//                   step does (op 1): the LDS read rate, and the matrix rate
//                   when every operand tile comes from LDS.
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

// LDS reads.  Each wave walks 64 KB of LDS in 1 KB steps (lane i reads bytes
// 16i .. 16i+15 of the step: consecutive lanes, consecutive banks); eight
// reads per iteration, each from its own KB.  op 0 XOR-folds the data; op 1
// passes each read to an MFMA (two accumulator chains, B operand fixed in
// registers), the pattern of the attention's score step.
constexpr int kLdsProbeBytes = 64 * 1024;

__global__ __launch_bounds__(512) void lds_kernel(int iters, int op, float* __restrict__ sink) {
  __shared__ __align__(16) unsigned char buf[kLdsProbeBytes];
  for (int i = threadIdx.x * 16; i < kLdsProbeBytes; i += 512 * 16)
    *reinterpret_cast<u32x4_t*>(buf + i) =
        u32x4_t{(unsigned)i, (unsigned)i * 3u, (unsigned)i ^ 0x3c00u, 0x3c003c00u};
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  unsigned off = (unsigned)(wave * 8 * 1024) % kLdsProbeBytes;
  u32x4_t acc = {0u, 0u, 0u, 0u};
  bf16x8_t b;
#pragma unroll
  for (int k = 0; k < 8; ++k) b[k] = (__bf16)(0.001f * (lane + k));
  f32x16_t c0 = {}, c1 = {};
  for (int i = 0; i < iters; ++i) {
    u32x4_t v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
      v[k] = *reinterpret_cast<const u32x4_t*>(buf + ((off + k * 1024u) % kLdsProbeBytes) + lane * 16);
    if (op == 0) {
#pragma unroll
      for (int k = 0; k < 8; ++k) acc ^= v[k];
    } else {
#pragma unroll
      for (int k = 0; k < 8; k += 2) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, v[k]), b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, v[k + 1]), b, c1,
                                                     0, 0, 0);
      }
    }
    off = (off + 8u * 1024u) % kLdsProbeBytes;
  }
  float t = (float)(acc.x ^ acc.y ^ acc.z ^ acc.w);
#pragma unroll
  for (int v = 0; v < 16; ++v) t += c0[v] + c1[v];
  if (t == 1.2345f) sink[blockIdx.x] = t;   // keeps the work live; never true in practice
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

// grid workgroups of 512 threads (8 waves, two per SIMD), each wave issuing
// 8 * iters 16-byte LDS reads (1 KB per wave instruction), op 0 alone, op 1
// each feeding one 32x32x16 MFMA.  sink: grid floats.
PROBE_API int ta_probe_lds(int grid, int iters, int op, void* sink, void* stream) {
  if (grid < 1 || grid > (1 << 20) || iters < 1 || (op != 0 && op != 1) || !sink)
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(lds_kernel, dim3((unsigned)grid), dim3(512), 0,
                     static_cast<hipStream_t>(stream), iters, op, static_cast<float*>(sink));
  return (int)hipGetLastError();
}
