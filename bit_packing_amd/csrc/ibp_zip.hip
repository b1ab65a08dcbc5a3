// ibp_zip.hip -- the comparison codec: exponent coding of BF16 tensors as on the
// page "ZipCCL: Efficient Lossless Data Compression of Communication Collectives
// for Accelerating LLM Training", section 2 (Metodologia), A and B, on one GPU
// and without collectives.
//
// A BF16 word splits into a sign-mantissa byte and its 8-bit exponent.  The 7
// exponents of a table derived from the tensor's standard deviation get 3-bit
// codes 1..7; any other exponent gets code 0 and is stored whole, in element
// order, in an escape array.  Per block of 4096 elements the codes are kept as
// three bit planes of 4096 bits; eoff[j] counts the escapes before block j.
//
// Both kernels run one 256-thread workgroup per block; thread t handles the two
// groups of 8 consecutive elements [q*2048 + 8t, +8), q = 0, 1, so sign-mantissa
// bytes, plane bytes and BF16 words move as 8-, 1- and 16-byte accesses.  The
// escapes of a thread are ranked by a block scan of two 16-bit counts packed in
// one word (group 0 low, group 1 high), and the block's first escape by a
// decoupled look-back over the blocks (compression) or by eoff (decompression).
#include "ibp_device.h"

namespace ibp {
namespace {

using namespace dev;

constexpr uint32_t kGroup = 8;                          // consecutive elements per thread and group
constexpr uint32_t kHalf = kZipBlock / 2;               // elements per group pass
constexpr uint32_t kPlane = kZipBlock / 8;              // bytes per code plane

// Inclusive scan of v over the workgroup (256 threads); *total gets the sum.
__device__ __forceinline__ uint32_t block_scan(uint32_t v, uint32_t lane, uint32_t wave, uint32_t *wsum,
                                               uint32_t *total) {
  const uint32_t x = wave_incl_scan(v);
  if (lane == kWave - 1) wsum[wave] = x;
  __syncthreads();
  uint32_t pre = 0, all = 0;
#pragma unroll
  for (uint32_t w = 0; w < kWavesPerBlock; ++w) {
    const uint32_t s = wsum[w];
    if (w < wave) pre += s;
    all += s;
  }
  *total = all;
  return pre + x;
}

__global__ void __launch_bounds__(kBlock) zip_encode_kernel(ZipArgs a) {
  __shared__ uint8_t lut[256];  // exponent -> code
  __shared__ uint32_t wsum[kWavesPerBlock];
  __shared__ uint64_t s_excl;
  __shared__ uint32_t s_failed;
  const uint32_t tid = threadIdx.x, lane = lane_id(), wave = uniform(tid / kWave);
  lut[tid] = 0;
  __syncthreads();
  if (tid < 7) lut[a.table[tid]] = (uint8_t)(tid + 1);
  __syncthreads();
  const uint64_t j = blockIdx.x;  // grid == nblk; the look-back relies on workgroup order
  const uint64_t e0 = j * kZipBlock;
  const uint32_t nb = (uint32_t)min((uint64_t)kZipBlock, a.n - e0);

  uint32_t ex[2][kGroup / 4];  // exponents, four per word
  uint32_t smw[2][2];          // sign-mantissa bytes, four per word
  uint32_t pbv[2][3];          // plane bytes
  uint32_t escm = 0;           // bit q*8 + k: element k of group q is an escape
  uint32_t packed = 0;         // escape counts: group 0 low 16 bits, group 1 high
#pragma unroll
  for (uint32_t q = 0; q < 2; ++q) {
    const uint32_t t0 = q * kHalf + kGroup * tid;
    uint16_t u[kGroup];
    if (t0 + kGroup <= nb) {
      const uint4 w = *reinterpret_cast<const uint4 *>(a.in + e0 + t0);
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (uint32_t k = 0; k < kGroup; ++k) u[k] = (uint16_t)(ws[k / 2] >> (16 * (k % 2)));
    } else {
#pragma unroll
      for (uint32_t k = 0; k < kGroup; ++k) u[k] = t0 + k < nb ? a.in[e0 + t0 + k] : (uint16_t)0;
    }
    smw[q][0] = smw[q][1] = 0;
    pbv[q][0] = pbv[q][1] = pbv[q][2] = 0;
    ex[q][0] = ex[q][1] = 0;
#pragma unroll
    for (uint32_t k = 0; k < kGroup; ++k) {
      const uint32_t v = u[k], e = (v >> 7) & 0xFFu;
      const uint32_t sbyte = ((v >> 8) & 0x80u) | (v & 0x7Fu);
      const bool valid = t0 + k < nb;
      const uint32_t c = valid ? lut[e] : 0u;
      smw[q][k / 4] |= sbyte << (8 * (k % 4));
      ex[q][k / 4] |= e << (8 * (k % 4));
      pbv[q][0] |= (c & 1u) << k;
      pbv[q][1] |= ((c >> 1) & 1u) << k;
      pbv[q][2] |= ((c >> 2) & 1u) << k;
      if (valid && c == 0u) {
        escm |= 1u << (q * kGroup + k);
        packed += 1u << (16 * q);
      }
    }
  }
  // the block's escape count first, published at once for the successors' look-back
  uint32_t total;
  const uint32_t incl = block_scan(packed, lane, wave, wsum, &total);
  const uint32_t excl_t = incl - packed;
  const uint32_t tot0 = total & 0xFFFFu, agg = tot0 + (total >> 16);
  if (tid == 0) lookback_publish(a.status, j, agg);
  // then the sign-mantissa bytes and code planes, which need no offset
#pragma unroll
  for (uint32_t q = 0; q < 2; ++q) {
    const uint32_t t0 = q * kHalf + kGroup * tid;
    uint8_t *smo = a.sm + e0 + t0;
    if (t0 + kGroup <= nb) {
      *reinterpret_cast<uint2 *>(smo) = make_uint2(smw[q][0], smw[q][1]);
    } else {
      for (uint32_t k = 0; t0 + k < nb; ++k) smo[k] = (uint8_t)(smw[q][k / 4] >> (8 * (k % 4)));
    }
    uint8_t *cp = a.codes + j * (3 * kPlane) + q * (kHalf / 8) + tid;
    cp[0] = (uint8_t)pbv[q][0];
    cp[kPlane] = (uint8_t)pbv[q][1];
    cp[2 * kPlane] = (uint8_t)pbv[q][2];
  }
  if (wave == 0) {
    bool timed_out = false;
    const uint64_t excl = lookback_exclusive(a.status, a.control, a.err, j, agg, lane, timed_out);
    if (lane == 0) {
      s_excl = excl;
      s_failed = timed_out ? 1u : 0u;
    }
  }
  __syncthreads();
  if (s_failed != 0u) return;  // no valid escape offset: nothing more is stored
  const uint64_t base = s_excl;
  if (tid == 0) {
    a.eoff[j] = base;
    if (j == a.nblk - 1) a.eoff[a.nblk] = base + agg;
  }
#pragma unroll
  for (uint32_t q = 0; q < 2; ++q) {
    uint64_t r = base + (q == 0 ? (excl_t & 0xFFFFu) : tot0 + (excl_t >> 16));
#pragma unroll
    for (uint32_t k = 0; k < kGroup; ++k)
      if ((escm >> (q * kGroup + k)) & 1u) a.esc[r++] = (uint8_t)(ex[q][k / 4] >> (8 * (k % 4)));
  }
}

// Bits 0..3 of x spread to bit 0 of bytes 0..3 (bit k -> bit 8k): the shifted
// copies x, x << 7, x << 14, x << 21 do not overlap, so the product has no carries.
__device__ __forceinline__ uint32_t spread4(uint32_t x) { return __umul24(x & 0xFu, 0x00204081u) & 0x01010101u; }

// Bytes i of the result: 0 if byte i of x is 0, else 0x80 (bytes of x at most 0x7F).
__device__ __forceinline__ uint32_t nonzero_bytes(uint32_t x) { return (x + 0x7F7F7F7Fu) & 0x80808080u; }

// BF16 words of two elements from their sign-mantissa and exponent bytes placed
// in the low bytes of the 16-bit halves of sp and ep.
__device__ __forceinline__ uint32_t bf16_pair(uint32_t sp, uint32_t ep) {
  return ((sp << 8) & 0x80008000u) | (ep << 7) | (sp & 0x007F007Fu);
}

__global__ void __launch_bounds__(kBlock) zip_decode_kernel(ZipArgs a) {
  __shared__ uint32_t wsum[kWavesPerBlock];
  const uint32_t tid = threadIdx.x, lane = lane_id(), wave = uniform(tid / kWave);
  // exponent of code c in byte c of (thi:tlo); byte 0 (escape) is 0
  const uint32_t tlo = ((uint32_t)a.table[0] << 8) | ((uint32_t)a.table[1] << 16) | ((uint32_t)a.table[2] << 24);
  const uint32_t thi = (uint32_t)a.table[3] | ((uint32_t)a.table[4] << 8) | ((uint32_t)a.table[5] << 16) |
                       ((uint32_t)a.table[6] << 24);
  const uint64_t j = blockIdx.x;
  const uint64_t e0 = j * kZipBlock;
  const uint32_t nb = (uint32_t)min((uint64_t)kZipBlock, a.n - e0);
  // every load that does not depend on the escape ranks is issued first
  const uint64_t E0 = a.eoff[j], E1 = a.eoff[j + 1];
  uint32_t pb[2][3];
  uint32_t sm[2][2];
#pragma unroll
  for (uint32_t q = 0; q < 2; ++q) {
    const uint32_t t0 = q * kHalf + kGroup * tid;
    const uint8_t *cp = a.codes + j * (3 * kPlane) + q * (kHalf / 8) + tid;
    pb[q][0] = cp[0];
    pb[q][1] = cp[kPlane];
    pb[q][2] = cp[2 * kPlane];
    sm[q][0] = sm[q][1] = 0;
    if (t0 + kGroup <= nb) {
      const uint2 w = *reinterpret_cast<const uint2 *>(a.sm + e0 + t0);
      sm[q][0] = w.x;
      sm[q][1] = w.y;
    } else {
      for (uint32_t k = 0; t0 + k < nb; ++k) sm[q][k / 4] |= (uint32_t)a.sm[e0 + t0 + k] << (8 * (k % 4));
    }
  }
  // codes of elements 4h..4h+3 of group q as the bytes of cb[q][h], and the escapes
  // (code 0 of an element inside the block) as 0x80 bytes of esc[q][h]
  uint32_t cb[2][2], esc[2][2];
  uint32_t packed = 0;
#pragma unroll
  for (uint32_t q = 0; q < 2; ++q) {
    const uint32_t t0 = q * kHalf + kGroup * tid;
    const uint32_t valid = nb > t0 ? min(nb - t0, kGroup) : 0u;  // elements of the group inside the block
    uint32_t n = 0;
#pragma unroll
    for (uint32_t h = 0; h < 2; ++h) {
      cb[q][h] = spread4(pb[q][0] >> (4 * h)) | (spread4(pb[q][1] >> (4 * h)) << 1) |
                 (spread4(pb[q][2] >> (4 * h)) << 2);
      const uint32_t vh = valid > 4 * h ? min(valid - 4 * h, 4u) : 0u;  // valid elements of this word
      const uint32_t in_block = vh >= 4 ? 0xFFFFFFFFu : ((1u << (8 * vh)) - 1u);
      esc[q][h] = ~nonzero_bytes(cb[q][h]) & 0x80808080u & in_block;
      n += __builtin_popcount(esc[q][h]);
    }
    packed += n << (16 * q);
  }
  uint32_t total;
  const uint32_t incl = block_scan(packed, lane, wave, wsum, &total);
  const uint32_t excl_t = incl - packed;
  const uint32_t tot0 = total & 0xFFFFu, agg = tot0 + (total >> 16);
  if (E1 < E0 || E1 - E0 != agg || E1 > a.esc_bytes) {
    if (tid == 0 && a.err) atomicOr(a.err, IBP_DEVERR_CORRUPT);
    return;  // block not decoded
  }
#pragma unroll
  for (uint32_t q = 0; q < 2; ++q) {
    const uint32_t t0 = q * kHalf + kGroup * tid;
    if (t0 >= nb) continue;
    // exponents: table bytes by code, then this thread's escapes (consecutive in the
    // escape array per group) in element order
    uint32_t ex[2];
    uint64_t r = E0 + (q == 0 ? (excl_t & 0xFFFFu) : tot0 + (excl_t >> 16));
#pragma unroll
    for (uint32_t h = 0; h < 2; ++h) {
      ex[h] = __builtin_amdgcn_perm(thi, tlo, cb[q][h]);
      for (uint32_t m = esc[q][h]; m; m &= m - 1u) {
        const uint32_t sh = (uint32_t)__builtin_ctz(m) - 7u;  // 8 * (byte index)
        ex[h] |= (uint32_t)a.esc[r++] << sh;
      }
    }
    // pairs of elements: sign-mantissa and exponent bytes moved to the 16-bit halves
    const uint32_t w0 = bf16_pair(__builtin_amdgcn_perm(0u, sm[q][0], 0x0C010C00u), __builtin_amdgcn_perm(0u, ex[0], 0x0C010C00u));
    const uint32_t w1 = bf16_pair(__builtin_amdgcn_perm(0u, sm[q][0], 0x0C030C02u), __builtin_amdgcn_perm(0u, ex[0], 0x0C030C02u));
    const uint32_t w2 = bf16_pair(__builtin_amdgcn_perm(0u, sm[q][1], 0x0C010C00u), __builtin_amdgcn_perm(0u, ex[1], 0x0C010C00u));
    const uint32_t w3 = bf16_pair(__builtin_amdgcn_perm(0u, sm[q][1], 0x0C030C02u), __builtin_amdgcn_perm(0u, ex[1], 0x0C030C02u));
    uint16_t *o = a.out + e0 + t0;
    if (t0 + kGroup <= nb) {
      *reinterpret_cast<uint4 *>(o) = make_uint4(w0, w1, w2, w3);
    } else {
      const uint32_t w[4] = {w0, w1, w2, w3};
      for (uint32_t k = 0; t0 + k < nb; ++k) o[k] = (uint16_t)(w[k / 2] >> (16 * (k % 2)));
    }
  }
}

}  // namespace

hipError_t launch_zip_encode(const ZipArgs &a, hipStream_t s) {
  if (a.nblk == 0) return hipSuccess;
  if (a.nblk > 0x7FFFFFFFull) return hipErrorInvalidValue;
  // clear the control words and status words (a kernel, not a memset node)
  hipError_t e = launch_zero(reinterpret_cast<uint64_t *>(a.control), a.nblk + 1, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(zip_encode_kernel, dim3((uint32_t)a.nblk), dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_zip_decode(const ZipArgs &a, hipStream_t s) {
  if (a.nblk == 0) return hipSuccess;
  if (a.nblk > 0x7FFFFFFFull) return hipErrorInvalidValue;
  hipLaunchKernelGGL(zip_decode_kernel, dim3((uint32_t)a.nblk), dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

}  // namespace ibp
