// Peak probes for the roofline denominators, measured on the GPU the
// projector runs on (measurement only; not part of the projector's path):
// sustained read bandwidth from HBM, from the Infinity Cache (MALL) and from
// L2, the fp32 fused multiply-add rate without packed math (the only fp32
// form the projector's kernels use), and the LDS 64-bit integer atomic rate
// (the adjoint's accumulator).  Declared in include/tp_peaks.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/tp_peaks.h"

namespace {

constexpr int kThreads = 256;

// Read n16 16-byte elements `passes` times, split into `regions` equal
// regions: workgroup b reads region b % regions (with 8 regions and the
// round-robin dispatch of workgroups over the 8 XCDs, each XCD reads only
// its own region).  Pass p reads element (i + p * rot) mod (region size) at
// thread i, so consecutive lanes stay coalesced while the data a CU touches
// changes from pass to pass (its L1 never holds what the next pass reads
// when rot is large).  The XOR of everything read is stored only if it
// equals a value it practically never takes, which keeps every load live.
__global__ __launch_bounds__(kThreads) void k_read(const uint4* __restrict__ buf, uint64_t n16, int64_t passes,
                                                    uint64_t rot, int regions, uint32_t* sink) {
  const uint32_t r = blockIdx.x % (uint32_t)regions, lb = blockIdx.x / (uint32_t)regions;
  const uint64_t per = n16 / (uint64_t)regions;
  const uint4* base = buf + (uint64_t)r * per;
  const uint64_t stride = (uint64_t)(gridDim.x / (uint32_t)regions) * kThreads;
  const uint64_t t0 = (uint64_t)lb * kThreads + threadIdx.x;
  const uint64_t step = rot % per;
  uint32_t acc = 0;
  uint64_t off = 0;
  for (int64_t p = 0; p < passes; ++p) {
#pragma unroll 4
    for (uint64_t i = t0; i < per; i += stride) {
      uint64_t j = i + off;
      j = j >= per ? j - per : j;
      const uint4 v = base[j];
      acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    off += step;
    off = off >= per ? off - per : off;
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

// Eight independent fp32 FMA chains per thread, iters steps each (2 flops
// per FMA).  The result is stored only under a condition the chains never
// meet, so nothing is dead.
__global__ __launch_bounds__(kThreads) void k_fma(int64_t iters, float* sink) {
  float a[8];
  const float m = 1.0f - 1e-7f * (float)(threadIdx.x & 7), c = 1e-7f;
#pragma unroll
  for (int k = 0; k < 8; ++k) a[k] = 1.0f + 0.125f * (float)k;
#pragma unroll 4
  for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < 8; ++k) a[k] = fmaf(a[k], m, c);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) s += a[k];
  if (s == -1.0f) sink[blockIdx.x] = s;
}

// 64-bit integer adds to LDS, each lane to its own slot (no bank conflicts,
// no address shared within an instruction), eight per iteration.
__global__ __launch_bounds__(kThreads) void k_lds_add(int64_t iters, unsigned long long* sink) {
  __shared__ unsigned long long slots[8 * kThreads];
  for (int k = 0; k < 8; ++k) slots[k * kThreads + threadIdx.x] = 0ull;
  __syncthreads();
  const unsigned long long v = 1ull + threadIdx.x;
  for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < 8; ++k) atomicAdd(&slots[k * kThreads + threadIdx.x], v);
  }
  __syncthreads();
  unsigned long long s = 0;
  for (int k = 0; k < 8; ++k) s += slots[k * kThreads + threadIdx.x];
  if (s == 0ull) sink[blockIdx.x] = s;
}

int launch_status() { return hipGetLastError() == hipSuccess ? 0 : -3; }

}  // namespace

extern "C" {

int tpk_threads_per_block(void) { return kThreads; }

int tpk_read(const void* buf, uint64_t n16, int64_t passes, uint64_t rot, int regions, int blocks,
             uint32_t* sink, void* stream) {
  if (!buf || !sink || n16 == 0 || passes <= 0 || blocks <= 0) return -1;
  if (regions != 1 && regions != 8) return -1;
  if (n16 % (uint64_t)regions != 0 || blocks % regions != 0) return -1;
  if ((reinterpret_cast<uintptr_t>(buf) & 15u) != 0) return -1;
  hipLaunchKernelGGL(k_read, dim3((unsigned)blocks), dim3(kThreads), 0, (hipStream_t)stream,
                     static_cast<const uint4*>(buf), n16, passes, rot, regions, sink);
  return launch_status();
}

int tpk_fma(int64_t iters, int blocks, float* sink, void* stream) {
  if (!sink || iters <= 0 || blocks <= 0) return -1;
  hipLaunchKernelGGL(k_fma, dim3((unsigned)blocks), dim3(kThreads), 0, (hipStream_t)stream, iters, sink);
  return launch_status();
}

int tpk_lds_add(int64_t iters, int blocks, unsigned long long* sink, void* stream) {
  if (!sink || iters <= 0 || blocks <= 0) return -1;
  hipLaunchKernelGGL(k_lds_add, dim3((unsigned)blocks), dim3(kThreads), 0, (hipStream_t)stream, iters, sink);
  return launch_status();
}

}  // extern "C"
