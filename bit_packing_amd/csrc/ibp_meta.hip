// ibp_meta.hip -- step 1 of the IBP codec on gfx950: Mask and Bitval from a
// sample batch ("Riduzione del Collo di Bottiglia della Memoria GPU con la
// Compressione Lossless per il ML", section "Algoritmo Core", Preprocessing).
//
// A bit position is invariant when its majority value holds in at least k of the
// n samples; k arrives precomputed from T.  Counting is integer-only, so the GPU
// and any other exact implementation agree on every count.
#include "ibp_device.h"

namespace ibp {
namespace {

using namespace dev;

// Per-position one-counts: a wavefront takes 64 consecutive samples per step, one
// per lane, and counts position b with one ballot: the ballot of bit b over the 64
// lanes is column b of the step's 64 x W bit matrix, and its popcount goes to a
// wave-uniform counter.  The counters stay scalar, so no wavefront ends with W
// shuffle reductions (2^20-chunk sample of 64-bit ids: 23.1 -> 18.0 us; 10,000
// 512-byte rows: 15.7 -> 12.7 us).  Workgroups of kMetaThreads threads, so that the
// at most kMetaMaxBlocks workgroups (one row of partials each) still give every SIMD
// several wavefronts.  A wavefront counts at most ceil(n / (kMetaMaxBlocks *
// kMetaThreads / 64)) samples, below 2^32 for any sample that fits in memory.
template <typename T>
__global__ void __launch_bounds__(kMetaThreads) count_ones_kernel(MetaArgs a) {
  constexpr uint32_t W = sizeof(T) * 8;
  constexpr uint32_t kU = 4;  // steps whose loads are in flight together
  constexpr uint32_t kWaves = kMetaThreads / kWave;
  __shared__ uint32_t red[kWaves][W];
  const T *in = static_cast<const T *>(a.in);
  const uint32_t lane = lane_id(), wave = uniform(threadIdx.x / kWave);
  uint32_t c[W];  // wave-uniform
#pragma unroll
  for (uint32_t b = 0; b < W; ++b) c[b] = 0;
  const uint64_t step = (uint64_t)gridDim.x * kMetaThreads;  // samples per step of all wavefronts
  for (uint64_t base = ((uint64_t)blockIdx.x * kWaves + wave) * kWave; base < a.n; base += kU * step) {
    T v[kU];
#pragma unroll
    for (uint32_t u = 0; u < kU; ++u) {
      const uint64_t i = base + u * step + lane;
      v[u] = i < a.n ? in[i] : (T)0;  // lanes past the sample add no ones
    }
#pragma unroll
    for (uint32_t u = 0; u < kU; ++u) {
#pragma unroll
      for (uint32_t b = 0; b < W; ++b) c[b] += popc(ballot(((v[u] >> b) & 1u) != 0));
    }
  }
  uint32_t mine = 0;  // lane b: counter b
#pragma unroll
  for (uint32_t b = 0; b < W; ++b) mine = lane == b ? c[b] : mine;
  if (lane < W) red[wave][lane] = mine;
  __syncthreads();
  if (threadIdx.x < W) {
    uint64_t s = 0;
    for (uint32_t w = 0; w < kWaves; ++w) s += red[w][threadIdx.x];
    a.partial[(uint64_t)blockIdx.x * W + threadIdx.x] = s;
  }
}

// One workgroup: wavefront w sums every fourth row of partial counts (lane b =
// position b), the four sums meet in LDS, and wavefront 0 applies the threshold;
// the ballots of its per-lane verdicts are Mask and Bitval.
__global__ void __launch_bounds__(kBlock) meta_finish_kernel(MetaArgs a) {
  __shared__ uint64_t red[kWavesPerBlock][kWave];
  const uint32_t b = lane_id(), part = uniform(threadIdx.x / kWave);
  uint64_t c1 = 0;
  if (b < a.W) {
#pragma unroll 8
    for (uint32_t j = part; j < a.blocks; j += kWavesPerBlock) c1 += a.partial[(uint64_t)j * a.W + b];
  }
  red[part][b] = c1;
  __syncthreads();
  if (part != 0) return;
  c1 = 0;
  for (uint32_t w = 0; w < kWavesPerBlock; ++w) c1 += red[w][b];
  const uint64_t c0 = a.n - c1;
  const uint64_t majority = c1 > c0 ? c1 : c0;
  const bool invariant = b < a.W && majority >= a.k;
  const uint64_t mask = ballot(invariant);
  const uint64_t bitval = ballot(invariant && c1 > c0);
  a.result[b] = b < a.W ? c1 : 0;
  if (b == 0) {
    a.result[64] = mask;
    a.result[65] = bitval;
  }
}

// Position-dependent metadata, step 1 per chunk position of a row: thread
// (i, g) counts position i over sample rows g, g + RG, g + 2 RG, ... in W
// register counters and adds them to counts[i W + b] (64-bit atomics; every
// thread of a wavefront handles a different position or row group).
template <typename T>
__global__ void __launch_bounds__(kBlock) count_ones_pos_kernel(MetaArgs a, uint32_t S, uint32_t RG) {
  constexpr uint32_t W = sizeof(T) * 8;
  const uint64_t t = (uint64_t)blockIdx.x * kBlock + threadIdx.x;
  if (t >= (uint64_t)S * RG) return;
  const uint32_t i = (uint32_t)(t % S), g = (uint32_t)(t / S);
  const T *in = static_cast<const T *>(a.in);
  uint32_t c[W];
#pragma unroll
  for (uint32_t b = 0; b < W; ++b) c[b] = 0;
  for (uint64_t r = g; r < a.n; r += RG) {
    const T v = in[r * S + i];
#pragma unroll
    for (uint32_t b = 0; b < W; ++b) c[b] += (uint32_t)((v >> b) & 1u);
  }
#pragma unroll
  for (uint32_t b = 0; b < W; ++b)
    if (c[b]) atomicAdd(reinterpret_cast<unsigned long long *>(&a.partial[(uint64_t)i * W + b]), (unsigned long long)c[b]);
}

// One thread per position: the threshold rule over its counts gives Mask_i, Bitval_i.
__global__ void __launch_bounds__(kBlock) meta_pos_finish_kernel(MetaArgs a, uint32_t S, uint64_t *mask,
                                                                 uint64_t *bitval) {
  const uint32_t i = blockIdx.x * kBlock + threadIdx.x;
  if (i >= S) return;
  uint64_t m = 0, bv = 0;
  for (uint32_t b = 0; b < a.W; ++b) {
    const uint64_t c1 = a.partial[(uint64_t)i * a.W + b], c0 = a.n - c1;
    if ((c1 > c0 ? c1 : c0) >= a.k) {
      m |= 1ull << b;
      if (c1 > c0) bv |= 1ull << b;
    }
  }
  mask[i] = m;
  bitval[i] = bv;
}

}  // namespace

hipError_t launch_meta_pos(const MetaArgs &a, uint32_t S, uint64_t *d_mask, uint64_t *d_bitval, hipStream_t s) {
  hipError_t e = launch_zero(a.partial, (uint64_t)S * a.W, s);
  if (e != hipSuccess) return e;
  const uint64_t want = (65536u + S - 1) / S;
  const uint32_t RG = (uint32_t)(want < a.n ? want : a.n);
  const uint64_t threads = (uint64_t)S * RG;
  const dim3 grid((uint32_t)((threads + kBlock - 1) / kBlock));
  if (a.W == 16)
    hipLaunchKernelGGL(count_ones_pos_kernel<uint16_t>, grid, dim3(kBlock), 0, s, a, S, RG);
  else if (a.W == 32)
    hipLaunchKernelGGL(count_ones_pos_kernel<uint32_t>, grid, dim3(kBlock), 0, s, a, S, RG);
  else
    hipLaunchKernelGGL(count_ones_pos_kernel<uint64_t>, grid, dim3(kBlock), 0, s, a, S, RG);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(meta_pos_finish_kernel, dim3((S + kBlock - 1) / kBlock), dim3(kBlock), 0, s, a, S, d_mask, d_bitval);
  return hipGetLastError();
}

hipError_t launch_meta(const MetaArgs &a, hipStream_t s) {
  if (a.n) {
    if (a.W == 16)
      hipLaunchKernelGGL(count_ones_kernel<uint16_t>, dim3(a.blocks), dim3(kMetaThreads), 0, s, a);
    else if (a.W == 32)
      hipLaunchKernelGGL(count_ones_kernel<uint32_t>, dim3(a.blocks), dim3(kMetaThreads), 0, s, a);
    else
      hipLaunchKernelGGL(count_ones_kernel<uint64_t>, dim3(a.blocks), dim3(kMetaThreads), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(meta_finish_kernel, dim3(1), dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

}  // namespace ibp
