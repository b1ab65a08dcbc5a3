// Test helper (not part of the codec): leaves every CU's LDS and its waves' vector
// registers holding a chosen pattern, so that the first workgroups of the next
// kernel start on dirty state instead of what a clean preceding kernel left.
// A kernel that reads an LDS word or a register lane it never wrote in this
// workgroup would then see the pattern.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint32_t kThreads = 1024;
constexpr uint32_t kLdsBytes = 64 * 1024;  // per workgroup (dynamic LDS)
constexpr uint32_t kRegs = 96;             // registers per thread held at the pattern at once

__global__ void __launch_bounds__(kThreads) dirty_kernel(uint32_t *sink, uint32_t pattern) {
  extern __shared__ uint32_t lds[];
  constexpr uint32_t n = kLdsBytes / 4;
  for (uint32_t i = threadIdx.x; i < n; i += kThreads) lds[i] = pattern;
  __syncthreads();
  uint32_t r[kRegs];
#pragma unroll
  for (uint32_t k = 0; k < kRegs; ++k) r[k] = lds[(threadIdx.x + 37u * k) % n];
  // every value is live in its own register at this point (an empty asm that
  // takes them all as operands; no instruction is emitted)
#pragma unroll
  for (uint32_t k = 0; k < kRegs; k += 8)
    asm volatile("" : "+v"(r[k]), "+v"(r[k + 1]), "+v"(r[k + 2]), "+v"(r[k + 3]), "+v"(r[k + 4]), "+v"(r[k + 5]),
                 "+v"(r[k + 6]), "+v"(r[k + 7]));
  uint32_t x = 0;
#pragma unroll
  for (uint32_t k = 0; k < kRegs; ++k) x += r[k] ^ k;
  sink[(uint64_t)blockIdx.x * kThreads + threadIdx.x] = x;
}

// Counts, per workgroup, the words of its (never written) LDS that hold the
// pattern: what the next kernel's workgroups find there.
__global__ void __launch_bounds__(256) peek_kernel(uint32_t *count, uint32_t pattern) {
  extern __shared__ uint32_t lds[];
  constexpr uint32_t n = kLdsBytes / 4;
  uint32_t c = 0;
  for (uint32_t i = threadIdx.x; i < n; i += 256) c += lds[i] == pattern ? 1u : 0u;
  atomicAdd(&count[blockIdx.x], c);
}

}  // namespace

// count: device array of `blocks` zeroed words.
extern "C" __attribute__((visibility("default"))) int dirty_peek_lds(uint32_t *count, uint32_t blocks,
                                                                    uint32_t pattern, void *stream) {
  if (!count || blocks == 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(peek_kernel, dim3(blocks), dim3(256), kLdsBytes, (hipStream_t)stream, count, pattern);
  return (int)hipGetLastError();
}

// sink: device buffer of dirty_sink_bytes(blocks) bytes; blocks: workgroups of 1024
// threads (two per CU fill every wave slot's registers and 128 KB of its LDS).
extern "C" __attribute__((visibility("default"))) uint64_t dirty_sink_bytes(uint32_t blocks) {
  return (uint64_t)blocks * kThreads * 4u;
}

extern "C" __attribute__((visibility("default"))) int dirty_device_state(void *sink, uint32_t blocks,
                                                                        uint32_t pattern, void *stream) {
  if (!sink || blocks == 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(dirty_kernel, dim3(blocks), dim3(kThreads), kLdsBytes, (hipStream_t)stream,
                     static_cast<uint32_t *>(sink), pattern);
  return (int)hipGetLastError();
}
