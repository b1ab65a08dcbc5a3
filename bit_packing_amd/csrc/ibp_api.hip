// ibp_api.hip -- the extern "C" entry points declared in include/ibp.h.
//
// Every argument is checked here, on the host, before any HIP call; then the
// launch geometry and the workspace layout are derived and the kernels in
// ibp_meta.hip, ibp_encode.hip, ibp_decode.hip and ibp_slots.hip are enqueued on the caller's stream.
#include <math.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "ibp.h"
#include "ibp_internal.h"

namespace {

using namespace ibp;

uint64_t full_bits(uint32_t W) { return W >= 64 ? ~0ull : ((1ull << W) - 1ull); }

bool width_ok(uint32_t W) { return W == 16 || W == 32 || W == 64; }

uint32_t log2_if_pow2(uint32_t S) {
  if (S == 0 || (S & (S - 1u))) return kNotPow2;
  uint32_t l = 0;
  while ((1u << l) != S) ++l;
  return l;
}

bool aligned(const void *p, uint64_t a) { return ((uintptr_t)p % a) == 0; }

// x * y, false when the product does not fit 64 bits
bool mul_ok(uint64_t x, uint64_t y, uint64_t *out) { return !__builtin_mul_overflow(x, y, out); }

// Look-back polls of one unpublished predecessor before a compressing tile gives
// up (see lookback_finish); lowered only by tests of that path.
constexpr uint32_t kDefaultWaitLimit = 1u << 20;
std::atomic<uint32_t> g_wait_limit{kDefaultWaitLimit};
constexpr uint64_t kDefaultHalvesMin = 1ull << 23;  // chunks; see ibp_set_halves_min_chunks
std::atomic<uint64_t> g_halves_min{kDefaultHalvesMin};

// Mask/Bitval -> kernel parameters: popcount and the runs of free positions.
bool make_params(const ibp_meta_t *m, CodecParams *p) {
  if (!m || !width_ok(m->W) || m->reserved != 0) return false;
  const uint64_t full = full_bits(m->W);
  if ((m->mask & ~full) || (m->bitval & ~m->mask)) return false;
  memset(p, 0, sizeof(*p));
  p->mask = m->mask;
  p->bitval = m->bitval;
  p->W = m->W;
  p->pc = (uint32_t)__builtin_popcountll(m->mask);
  const uint64_t F = ~m->mask & full;
  uint32_t n = 0, cum = 0;
  for (uint32_t b = 0; b < m->W;) {
    if (!((F >> b) & 1ull)) {
      ++b;
      continue;
    }
    const uint32_t start = b;
    while (b < m->W && ((F >> b) & 1ull)) ++b;
    const uint32_t len = b - start;
    p->runs.pmask[n] = full_bits(len) << cum;
    p->runs.shift[n] = start - cum;
    cum += len;
    ++n;
  }
  p->runs.n = n;
  return true;
}

// Bits per segment can never exceed S * (W + 1); total bits must fit the 62-bit
// look-back value field.
bool total_fits(uint64_t n_chunks, uint32_t W) {
  return n_chunks < (1ull << 55) && n_chunks * (uint64_t)(W + 1) < (1ull << 62);
}

uint32_t meta_blocks(uint64_t n) {
  // about four samples per thread: one round of four in-flight steps per wavefront
  const uint64_t want = (n + (uint64_t)kMetaThreads * 4 - 1) / ((uint64_t)kMetaThreads * 4);
  return (uint32_t)(want < 1 ? 1 : (want > kMetaMaxBlocks ? kMetaMaxBlocks : want));
}

uint32_t enc_segs_per_tile(uint32_t S, bool pos, bool pair, uint32_t W, uint32_t halves = 1, bool big = false) {
  const uint32_t tile = enc_tile_chunks(pos, pair, W, halves, big);
  return S >= tile ? 1u : tile / S;
}

uint64_t enc_tiles(uint64_t n_chunks, uint32_t S, bool pos, bool pair, uint32_t W) {
  const uint64_t nseg = (n_chunks + S - 1) / S;
  const uint32_t G = enc_segs_per_tile(S, pos, pair, W);
  return (nseg + G - 1) / G;
}

uint32_t dec_units_per_tile(uint32_t S) {
  uint32_t G = S >= kDecTileChunks ? 1u : kDecTileChunks / S;
  return G > kDecMaxUnits ? kDecMaxUnits : G;
}

int status_of(hipError_t e) { return e == hipSuccess ? IBP_OK : IBP_ERR_DEVICE; }

// Device-visible address of the byte range [p, p + bytes), or nullptr when the
// range does not lie inside one device allocation or one pinned host allocation.
// Pageable host memory and stray pointers are refused here instead of being
// handed to a kernel, where they would fault the GPU.  Pinned host memory is
// returned through its device mapping (the zero-copy path).
const void *device_range(const void *p, uint64_t bytes, bool *is_host = nullptr) {
  if (is_host) *is_host = false;
  if (bytes == 0) return p;
  if (!p) return nullptr;
  hipPointerAttribute_t at;
  if (hipPointerGetAttributes(&at, p) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  const char *dev;
  if (at.type == hipMemoryTypeDevice || at.type == hipMemoryTypeManaged) {
    dev = static_cast<const char *>(p);
  } else if (at.type == hipMemoryTypeHost && at.devicePointer) {
    if (is_host) *is_host = true;
    const char *hp = at.hostPointer ? static_cast<const char *>(at.hostPointer) : static_cast<const char *>(p);
    dev = static_cast<const char *>(at.devicePointer) + (static_cast<const char *>(p) - hp);
  } else {
    return nullptr;
  }
  // the allocation that holds q must also hold [q, q + bytes): 1 yes, 0 no, -1 unknown
  auto inside = [bytes](const void *q) -> int {
    hipDeviceptr_t base = nullptr;
    size_t size = 0;
    if (hipMemGetAddressRange(&base, &size, (hipDeviceptr_t)q) != hipSuccess) {
      (void)hipGetLastError();
      return -1;
    }
    const uintptr_t b = (uintptr_t)base, a = (uintptr_t)q;
    return (a >= b && bytes <= size && a - b <= size - bytes) ? 1 : 0;
  };
  int in = inside(dev);
  // pinned host memory: the range may be known under its host address instead
  if (in < 0 && at.type == hipMemoryTypeHost) in = inside(p);
  return in == 1 ? dev : nullptr;
}

template <typename P> bool view(P *&p, uint64_t bytes, bool *is_host = nullptr) {
  const void *d = device_range(p, bytes, is_host);
  if (bytes && !d) return false;
  p = const_cast<P *>(static_cast<const P *>(d));
  return true;
}

// Workspace of ibp_compress_noalloc, for callers that cannot allocate: a file-scope
// device array (each GPU the library runs on holds its own copy until the process
// ends), shared by every such call on that GPU.  Its device address on each GPU is
// resolved once, with that GPU current, by hipGetSymbolAddress; host code uses only
// that address (the array's name is not a device address in host code).
constexpr uint64_t kScratchBytes = IBP_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

void *scratch_of_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

IBP_API const char *ibp_status_str(int status) {
  switch (status) {
    case IBP_OK: return "IBP_OK";
    case IBP_ERR_INVALID_ARG: return "IBP_ERR_INVALID_ARG";
    case IBP_ERR_SIZE: return "IBP_ERR_SIZE";
    case IBP_ERR_CAPACITY: return "IBP_ERR_CAPACITY";
    case IBP_ERR_DEVICE: return "IBP_ERR_DEVICE";
    default: return "IBP_ERR_UNKNOWN";
  }
}

IBP_API uint32_t ibp_set_wait_limit(uint32_t polls) {
  return g_wait_limit.exchange(polls == 0xFFFFFFFFu ? kDefaultWaitLimit : polls);
}

IBP_API uint64_t ibp_set_halves_min_chunks(uint64_t n_chunks) {
  return g_halves_min.exchange(n_chunks == ~0ull ? kDefaultHalvesMin : n_chunks);
}

IBP_API uint64_t ibp_num_segments(uint64_t n_chunks, uint32_t S) {
  return S ? (n_chunks + S - 1) / S : 0;
}

IBP_API uint64_t ibp_max_stream_bytes(uint64_t n_chunks, uint32_t W) {
  const uint64_t bytes = (n_chunks * (uint64_t)(W + 1) + 7) / 8;
  return (bytes + 15) & ~15ull;
}

IBP_API uint64_t ibp_stream_bytes(uint64_t total_bits) { return (((total_bits + 7) / 8) + 15) & ~15ull; }

IBP_API uint64_t ibp_metadata_workspace_bytes(uint64_t n_sample_chunks, uint32_t W) {
  const uint64_t w = width_ok(W) ? W : 64;
  return ((uint64_t)meta_blocks(n_sample_chunks) * w + 66) * 8;
}

IBP_API uint64_t ibp_compress_workspace_bytes(uint64_t n_chunks, uint32_t S) {
  if (S == 0) return 0;
  const uint64_t t = enc_tiles(n_chunks, S, true, false, 32);  // the smallest tiles (position metadata, W > 16)
  return t ? 8 + 8 * (status_words(t) + t) : 8;  // control, status words, hand-over words
}

IBP_API int ibp_build_metadata(const void *d_samples, uint64_t n_sample_chunks, uint32_t W, double T,
                               ibp_meta_t *meta_out, uint64_t *counts_out, void *d_workspace,
                               uint64_t workspace_bytes, void *hip_stream) {
  if (!width_ok(W) || !meta_out || !d_workspace || !(T > 0.5 && T <= 1.0)) return IBP_ERR_INVALID_ARG;
  if (n_sample_chunks == 0 || !d_samples || !aligned(d_samples, W / 8) || !aligned(d_workspace, 8))
    return IBP_ERR_INVALID_ARG;
  if (n_sample_chunks >= (1ull << 40)) return IBP_ERR_SIZE;
  if (workspace_bytes < ibp_metadata_workspace_bytes(n_sample_chunks, W)) return IBP_ERR_CAPACITY;
  if (!view(d_samples, n_sample_chunks * (W / 8)) || !view(d_workspace, ibp_metadata_workspace_bytes(n_sample_chunks, W)))
    return IBP_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  MetaArgs a;
  a.in = d_samples;
  a.n = n_sample_chunks;
  a.W = W;
  a.blocks = meta_blocks(n_sample_chunks);
  a.partial = static_cast<uint64_t *>(d_workspace);
  a.result = a.partial + (uint64_t)a.blocks * W;
  // k = ceil(round(T * 10^6) * n / 10^6), exactly, in 128-bit integers
  const uint64_t tppm = (uint64_t)(T * 1e6 + 0.5);
  const unsigned __int128 num = (unsigned __int128)tppm * n_sample_chunks;
  a.k = (uint64_t)((num + 999999u) / 1000000u);
  hipError_t e = launch_meta(a, s);
  if (e != hipSuccess) return IBP_ERR_DEVICE;
  uint64_t host[66];
  e = hipMemcpyAsync(host, a.result, sizeof(host), hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return IBP_ERR_DEVICE;
  e = hipStreamSynchronize(s);
  if (e != hipSuccess) return IBP_ERR_DEVICE;
  meta_out->W = W;
  meta_out->reserved = 0;
  meta_out->mask = host[64];
  meta_out->bitval = host[65];
  if (counts_out)
    for (uint32_t b = 0; b < W; ++b) counts_out[b] = host[b];
  return IBP_OK;
}

// ws_is_scratch: d_workspace is this library's own device array (ibp_compress_noalloc),
// known to be device memory of kScratchBytes bytes; it is not looked up.
static int compress_common(const CodecParams &p, const uint64_t *pmask, const uint64_t *pbitval, const void *d_in,
                           uint64_t n_bytes, uint32_t S, void *d_stream, uint64_t stream_capacity,
                           uint64_t *d_offsets, void *d_workspace, uint64_t workspace_bytes, uint32_t *d_err_word,
                           void *hip_stream, bool ws_is_scratch = false) {
  if (S == 0 || S > IBP_MAX_S || !d_offsets) return IBP_ERR_INVALID_ARG;
  const uint32_t cb = p.W / 8;
  if (n_bytes % cb) return IBP_ERR_SIZE;
  const uint64_t n = n_bytes / cb;
  if (n && (!d_in || !d_stream || !d_workspace)) return IBP_ERR_INVALID_ARG;
  if (!aligned(d_in, cb) || !aligned(d_stream, 16) || !aligned(d_offsets, 8) || !aligned(d_workspace, 8))
    return IBP_ERR_INVALID_ARG;
  if (!total_fits(n, p.W)) return IBP_ERR_SIZE;
  if (stream_capacity < ibp_max_stream_bytes(n, p.W)) return IBP_ERR_CAPACITY;
  if (workspace_bytes < ibp_compress_workspace_bytes(n, S)) return IBP_ERR_CAPACITY;
  const uint64_t nseg = (n + S - 1) / S;
  if (!view(d_in, n_bytes) || !view(d_stream, ibp_max_stream_bytes(n, p.W)) || !view(d_offsets, 8 * (nseg + 1)) ||
      (!ws_is_scratch && !view(d_workspace, n ? ibp_compress_workspace_bytes(n, S) : 0)) ||
      !view(d_err_word, d_err_word ? 4 : 0))
    return IBP_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  if (n == 0) return status_of(launch_zero(d_offsets, 1, s));  // offset table = {0}
  EncodeArgs a;
  a.pmask = pmask;
  a.pbitval = pbitval;
  a.in = d_in;
  a.stream = static_cast<uint32_t *>(d_stream);
  a.off = d_offsets;
  a.control = static_cast<uint32_t *>(d_workspace);
  a.status = reinterpret_cast<uint64_t *>(static_cast<uint8_t *>(d_workspace) + 8);
  // W = 16 with one Mask reads chunk pairs as 32-bit words when the segments are
  // whole 64-chunk blocks and the input allows it
  a.pair = (p.W == 16 && !pmask && S % kWave == 0 && aligned(d_in, 4)) ? 1u : 0u;
  a.halves = n >= g_halves_min.load() ? enc_halves(pmask != nullptr, a.pair != 0u, p.W, S) : 1u;
  a.big = !pmask && enc_big(p.W, a.halves, p.pc) ? 1u : 0u;
  a.G = enc_segs_per_tile(S, pmask != nullptr, a.pair != 0u, p.W, a.halves, a.big != 0u);
  a.ntiles = (nseg + a.G - 1) / a.G;  // at most the workspace's tile count (its tiles are the smallest)
  a.st_lg = status_lg(a.ntiles);
  a.tails = a.status + status_words(a.ntiles);
  a.err = d_err_word;
  a.n_chunks = n;
  a.nseg = nseg;
  a.S = S;
  a.s_log2 = log2_if_pow2(S);
  a.tile_chunks = a.G * S;
  if (a.halves == 2 && a.tile_chunks != enc_tile_chunks(pmask != nullptr, false, p.W, 2, a.big != 0u))
    return IBP_ERR_INVALID_ARG;
  // image (one half's when halves == 2) from the 16-byte block of the first bit
  a.obuf_dw = ((127 + a.tile_chunks / a.halves * (p.W + 1) + 31) / 32 + 2 + 3) & ~3u;
  a.wait_limit = g_wait_limit.load();
  return status_of(launch_encode(a, p, s));
}

IBP_API int ibp_compress(const ibp_meta_t *meta, const void *d_in, uint64_t n_bytes, uint32_t S,
                         void *d_stream, uint64_t stream_capacity, uint64_t *d_offsets,
                         void *d_workspace, uint64_t workspace_bytes, uint32_t *d_err_word,
                         void *hip_stream) {
  CodecParams p;
  if (!make_params(meta, &p)) return IBP_ERR_INVALID_ARG;
  return compress_common(p, nullptr, nullptr, d_in, n_bytes, S, d_stream, stream_capacity, d_offsets, d_workspace,
                         workspace_bytes, d_err_word, hip_stream);
}

IBP_API int ibp_compress_noalloc(const ibp_meta_t *meta, const void *d_in, uint64_t n_bytes, uint32_t S,
                                 void *d_stream, uint64_t stream_capacity, uint64_t *d_offsets,
                                 uint32_t *d_err_word, void *hip_stream) {
  CodecParams p;
  if (!make_params(meta, &p)) return IBP_ERR_INVALID_ARG;
  if (S == 0 || S > IBP_MAX_S) return IBP_ERR_INVALID_ARG;
  const uint32_t cb = p.W / 8;
  if (n_bytes % cb) return IBP_ERR_SIZE;
  if (!total_fits(n_bytes / cb, p.W)) return IBP_ERR_SIZE;
  if (ibp_compress_workspace_bytes(n_bytes / cb, S) > kScratchBytes) return IBP_ERR_CAPACITY;
  void *ws = nullptr;
  if (n_bytes) {
    ws = scratch_of_current_device();
    if (!ws) return IBP_ERR_DEVICE;
  }
  return compress_common(p, nullptr, nullptr, d_in, n_bytes, S, d_stream, stream_capacity, d_offsets, ws,
                         kScratchBytes, d_err_word, hip_stream, true);
}

// Position-dependent metadata: W/S checks, device tables of S words each.
static bool pos_params(const ibp_pos_meta_t *m, CodecParams *p, const uint64_t **mask, const uint64_t **bitval) {
  if (!m || !width_ok(m->W) || m->S == 0 || m->S > IBP_MAX_S || !m->mask || !m->bitval) return false;
  if (!aligned(m->mask, 8) || !aligned(m->bitval, 8)) return false;
  *mask = m->mask;
  *bitval = m->bitval;
  if (!view(*mask, 8ull * m->S) || !view(*bitval, 8ull * m->S)) return false;
  memset(p, 0, sizeof(*p));
  p->W = m->W;
  return true;
}

IBP_API uint64_t ibp_metadata_pos_workspace_bytes(uint32_t S, uint32_t W) {
  const uint64_t w = width_ok(W) ? W : 64;
  return 8ull * S * w;
}

IBP_API int ibp_build_metadata_pos(const void *d_samples, uint64_t n_rows, uint32_t S, uint32_t W, double T,
                                   uint64_t *d_mask, uint64_t *d_bitval, uint64_t *counts_out, void *d_workspace,
                                   uint64_t workspace_bytes, void *hip_stream) {
  if (!width_ok(W) || S == 0 || S > IBP_MAX_S || !(T > 0.5 && T <= 1.0)) return IBP_ERR_INVALID_ARG;
  if (n_rows == 0 || !d_samples || !d_mask || !d_bitval || !d_workspace) return IBP_ERR_INVALID_ARG;
  if (!aligned(d_samples, W / 8) || !aligned(d_mask, 8) || !aligned(d_bitval, 8) || !aligned(d_workspace, 8))
    return IBP_ERR_INVALID_ARG;
  if (n_rows >= (1ull << 32) || n_rows * S >= (1ull << 40)) return IBP_ERR_SIZE;
  if (workspace_bytes < ibp_metadata_pos_workspace_bytes(S, W)) return IBP_ERR_CAPACITY;
  if (!view(d_samples, n_rows * S * (W / 8)) || !view(d_mask, 8ull * S) || !view(d_bitval, 8ull * S) ||
      !view(d_workspace, ibp_metadata_pos_workspace_bytes(S, W)))
    return IBP_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  MetaArgs a;
  a.in = d_samples;
  a.n = n_rows;
  a.W = W;
  a.blocks = 0;
  a.partial = static_cast<uint64_t *>(d_workspace);
  a.result = nullptr;
  const uint64_t tppm = (uint64_t)(T * 1e6 + 0.5);
  const unsigned __int128 num = (unsigned __int128)tppm * n_rows;
  a.k = (uint64_t)((num + 999999u) / 1000000u);
  hipError_t e = launch_meta_pos(a, S, d_mask, d_bitval, s);
  if (e != hipSuccess) return IBP_ERR_DEVICE;
  if (counts_out) {
    e = hipMemcpyAsync(counts_out, a.partial, 8ull * S * W, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return IBP_ERR_DEVICE;
  }
  return IBP_OK;
}

IBP_API int ibp_compress_pos(const ibp_pos_meta_t *meta, const void *d_in, uint64_t n_bytes, void *d_stream,
                             uint64_t stream_capacity, uint64_t *d_offsets, void *d_workspace,
                             uint64_t workspace_bytes, uint32_t *d_err_word, void *hip_stream) {
  CodecParams p;
  const uint64_t *pm, *pb;
  if (!pos_params(meta, &p, &pm, &pb)) return IBP_ERR_INVALID_ARG;
  return compress_common(p, pm, pb, d_in, n_bytes, meta->S, d_stream, stream_capacity, d_offsets,
                         d_workspace, workspace_bytes, d_err_word, hip_stream);
}

static int decode_common(const CodecParams &p, const uint64_t *pmask, const uint64_t *pbitval, const void *stream_in,
                         uint64_t stream_bytes, const uint64_t *d_offsets, uint64_t nseg, uint32_t S,
                         const int64_t *d_ids, uint64_t n_units, uint64_t n_chunks, void *d_out,
                         uint32_t *d_err_word, void *hip_stream, bool gather) {
  if (S == 0 || S > IBP_MAX_S || !d_offsets) return IBP_ERR_INVALID_ARG;
  const uint32_t cb = p.W / 8;
  if (n_chunks && (!d_out || !stream_in)) return IBP_ERR_INVALID_ARG;
  if (gather && n_units && !d_ids) return IBP_ERR_INVALID_ARG;
  if (!aligned(stream_in, 16) || !aligned(d_out, cb) || !aligned(d_offsets, 8) || !aligned(d_ids, 8))
    return IBP_ERR_INVALID_ARG;
  if (nseg >= (1ull << 55) / S) return IBP_ERR_SIZE;  // keeps 8 (nseg + 1) and nseg S exact
  if (!total_fits(n_chunks, p.W) || (gather && !total_fits(nseg * (uint64_t)S, p.W))) return IBP_ERR_SIZE;
  if (n_units == 0) return IBP_OK;
  bool host_stream = false;
  if (!view(stream_in, stream_bytes, &host_stream) || !view(d_offsets, 8 * (nseg + 1)) || !view(d_ids, gather ? 8 * n_units : 0) ||
      !view(d_out, n_chunks * cb) || !view(d_err_word, d_err_word ? 4 : 0))
    return IBP_ERR_INVALID_ARG;
  DecodeArgs a;
  a.pmask = pmask;
  a.pbitval = pbitval;
  a.stream = static_cast<const uint8_t *>(stream_in);
  a.stream_bytes = stream_bytes;
  a.off = d_offsets;
  a.ids = d_ids;
  a.out = d_out;
  a.err = d_err_word;
  a.n_chunks = n_chunks;
  a.n_units = n_units;
  a.nseg = nseg;
  a.S = S;
  a.s_log2 = log2_if_pow2(S);
  // Rows read over PCIe go one per wavefront: more independent read streams keep
  // more host reads in flight.  From HBM a wavefront takes about 512 chunks of a
  // contiguous stream, and about 1024 chunks, at most kGatherMaxRows rows, of a
  // gather (its dependent id -> offset -> row reads favour one wave generation).
  // A contiguous stream with one Mask takes 512 chunks per wavefront; from 2^24
  // chunks on, 512 * 64 / W (the same ~4 KB of staging at every W), which spreads
  // the per-tile setup over more chunks (sparse W = 32 data: 197 -> 159 us per
  // 128M chunks; W = 16: 969 -> 865 us per 1G chunks), while smaller inputs keep
  // more wavefronts.
  if (gather) {
    a.G = host_stream ? 1u : (S >= 2 * kDecTileChunks / kGatherMaxRows ? (S >= 2 * kDecTileChunks ? 1u : 2 * kDecTileChunks / S)
                                                                       : kGatherMaxRows);
  } else if (pmask) {
    a.G = dec_units_per_tile(S);
  } else {
    const uint32_t tile = n_chunks >= (1ull << 24) ? kDecTileChunks * (64u / p.W) : kDecTileChunks;
    a.G = S >= tile ? 1u : (tile / S > kDecMaxUnits ? kDecMaxUnits : tile / S);
  }
  const uint32_t tile_chunks = a.G * S;
  if (gather) {
    a.slot_dw = ((S * (p.W + 1) + 127) / 128 + 1) * 4;
    a.sb_magic = (uint32_t)(((1ull << 32) + a.slot_dw / 4 - 1) / (a.slot_dw / 4));
    a.stage_dw = a.G * a.slot_dw + 4;
  } else {
    a.slot_dw = 0;
    a.sb_magic = 0;
    a.stage_dw = 4 * ((tile_chunks * (p.W + 1) + 254) / 128) + 8;
  }
  uint32_t per_unit = 3 * a.G;
  if (gather) per_unit += (a.G & 1u) + 3 * a.G;  // 8-byte aligned first-block table + block counts
  a.wave_dw = (a.stage_dw + per_unit + 3) & ~3u;
  if (pmask) return status_of(launch_decode_pos(a, p, static_cast<hipStream_t>(hip_stream)));
  return status_of(launch_decode(a, p, gather, static_cast<hipStream_t>(hip_stream)));
}

IBP_API int ibp_decompress(const ibp_meta_t *meta, const void *stream_in, uint64_t stream_bytes,
                           const uint64_t *d_offsets, uint64_t n_chunks, uint32_t S, void *d_out,
                           uint32_t *d_err_word, void *hip_stream) {
  CodecParams p;
  if (!make_params(meta, &p)) return IBP_ERR_INVALID_ARG;
  const uint64_t nseg = ibp_num_segments(n_chunks, S);
  return decode_common(p, nullptr, nullptr, stream_in, stream_bytes, d_offsets, nseg, S, nullptr, nseg, n_chunks,
                       d_out, d_err_word, hip_stream, false);
}

IBP_API int ibp_decompress_pos(const ibp_pos_meta_t *meta, const void *stream_in, uint64_t stream_bytes,
                               const uint64_t *d_offsets, uint64_t n_chunks, void *d_out, uint32_t *d_err_word,
                               void *hip_stream) {
  CodecParams p;
  const uint64_t *pm, *pb;
  if (!pos_params(meta, &p, &pm, &pb)) return IBP_ERR_INVALID_ARG;
  const uint64_t nseg = ibp_num_segments(n_chunks, meta->S);
  return decode_common(p, pm, pb, stream_in, stream_bytes, d_offsets, nseg, meta->S, nullptr, nseg,
                       n_chunks, d_out, d_err_word, hip_stream, false);
}

IBP_API int ibp_decompress_gather(const ibp_meta_t *meta, const void *stream_in, uint64_t stream_bytes,
                                  const uint64_t *d_offsets, uint64_t n_segments, uint32_t S,
                                  const int64_t *d_ids, uint64_t n_ids, void *d_out,
                                  uint32_t *d_err_word, void *hip_stream) {
  CodecParams p;
  if (!make_params(meta, &p)) return IBP_ERR_INVALID_ARG;
  if (S != 0 && n_ids > (1ull << 55) / S) return IBP_ERR_SIZE;
  return decode_common(p, nullptr, nullptr, stream_in, stream_bytes, d_offsets, n_segments, S, d_ids, n_ids,
                       n_ids * (uint64_t)S, d_out, d_err_word, hip_stream, true);
}

IBP_API int ibp_gather_raw(const void *src, uint64_t row_bytes, uint64_t n_rows, const int64_t *d_ids,
                           uint64_t n_ids, void *d_out, uint32_t *d_err_word, void *hip_stream) {
  if (row_bytes == 0 || row_bytes % 16) return IBP_ERR_SIZE;
  uint64_t src_bytes = 0, out_bytes = 0, id_bytes = 0;
  if (!mul_ok(row_bytes, n_rows, &src_bytes) || !mul_ok(row_bytes, n_ids, &out_bytes) || !mul_ok(8, n_ids, &id_bytes))
    return IBP_ERR_SIZE;
  if (n_ids && (!src || !d_ids || !d_out)) return IBP_ERR_INVALID_ARG;
  if (!aligned(src, 16) || !aligned(d_out, 16) || !aligned(d_ids, 8)) return IBP_ERR_INVALID_ARG;
  if (n_ids == 0) return IBP_OK;
  if (n_rows == 0) return IBP_ERR_SIZE;  // every id would be out of range
  if (!view(src, src_bytes) || !view(d_ids, id_bytes) || !view(d_out, out_bytes) ||
      !view(d_err_word, d_err_word ? 4 : 0))
    return IBP_ERR_INVALID_ARG;
  RawGatherArgs a;
  a.src = static_cast<const uint8_t *>(src);
  a.ids = d_ids;
  a.out = static_cast<uint8_t *>(d_out);
  a.err = d_err_word;
  a.row_blocks = row_bytes / 16;
  a.n_rows = n_rows;
  a.n_ids = n_ids;
  return status_of(launch_raw_gather(a, static_cast<hipStream_t>(hip_stream)));
}

}  // extern "C"

// ------------------------------------------------------------------ fixed-slot layout

extern "C" {

IBP_API uint64_t ibp_slot_flag_words(uint64_t n_rows) { return (n_rows + 63) / 64; }

IBP_API int ibp_compress_slots(const ibp_meta_t *meta, const void *d_in, uint64_t n_rows, uint32_t S,
                               void *slots, uint64_t slots_bytes, uint64_t *d_flags, uint32_t *d_err_word,
                               void *hip_stream) {
  CodecParams p;
  if (!make_params(meta, &p) || S == 0 || S > IBP_MAX_S) return IBP_ERR_INVALID_ARG;
  const uint64_t row_bytes = (uint64_t)S * (p.W / 8);
  if (row_bytes % 16) return IBP_ERR_SIZE;
  if (n_rows && (!d_in || !slots || !d_flags)) return IBP_ERR_INVALID_ARG;
  if (!aligned(d_in, 16) || !aligned(slots, 16) || !aligned(d_flags, 8)) return IBP_ERR_INVALID_ARG;
  if (n_rows >= (1ull << 40)) return IBP_ERR_SIZE;
  if (slots_bytes < n_rows * row_bytes) return IBP_ERR_CAPACITY;
  if (n_rows == 0) return IBP_OK;
  bool flags_host = false;
  if (!view(d_in, n_rows * row_bytes) || !view(slots, n_rows * row_bytes) ||
      !view(d_flags, 8 * ibp_slot_flag_words(n_rows), &flags_host) || flags_host ||
      !view(d_err_word, d_err_word ? 4 : 0))
    return IBP_ERR_INVALID_ARG;
  SlotArgs a{};
  a.in = d_in;
  a.slots = static_cast<uint8_t *>(slots);
  a.flags = d_flags;
  a.err = d_err_word;
  a.n_rows = n_rows;
  a.n_units = n_rows;
  a.S = S;
  a.s_log2 = log2_if_pow2(S);
  a.G = dec_units_per_tile(S);
  a.row_bytes = (uint32_t)row_bytes;
  a.img_dw = ((S * (p.W + 1) + 31) / 32 + 2 + 3) & ~3u;
  a.wave_dw = (a.G * a.img_dw + a.G + 1 + 3) & ~3u;
  return status_of(launch_encode_slots(a, p, static_cast<hipStream_t>(hip_stream)));
}

IBP_API int ibp_decompress_gather_slots(const ibp_meta_t *meta, const void *slots, uint64_t slots_bytes,
                                        uint64_t n_rows, uint32_t S, const uint64_t *d_flags, const int64_t *d_ids,
                                        uint64_t n_ids, void *d_out, uint32_t *d_err_word, void *hip_stream) {
  CodecParams p;
  if (!make_params(meta, &p) || S == 0 || S > IBP_MAX_S) return IBP_ERR_INVALID_ARG;
  const uint64_t row_bytes = (uint64_t)S * (p.W / 8);
  if (row_bytes % 16) return IBP_ERR_SIZE;
  if (n_ids && (!slots || !d_flags || !d_ids || !d_out)) return IBP_ERR_INVALID_ARG;
  if (!aligned(slots, 16) || !aligned(d_out, 16) || !aligned(d_flags, 8) || !aligned(d_ids, 8))
    return IBP_ERR_INVALID_ARG;
  if (n_rows >= (1ull << 40) || n_ids >= (1ull << 40)) return IBP_ERR_SIZE;
  if (slots_bytes < n_rows * row_bytes) return IBP_ERR_CAPACITY;
  if (n_ids == 0) return IBP_OK;
  bool slots_host = false, flags_host = false;
  if (!view(slots, n_rows * row_bytes, &slots_host) || !view(d_flags, 8 * ibp_slot_flag_words(n_rows), &flags_host) ||
      flags_host || !view(d_ids, 8 * n_ids) || !view(d_out, n_ids * row_bytes) ||
      !view(d_err_word, d_err_word ? 4 : 0))
    return IBP_ERR_INVALID_ARG;
  SlotArgs a{};
  a.slots = static_cast<uint8_t *>(const_cast<void *>(slots));
  a.flags = const_cast<uint64_t *>(d_flags);
  a.ids = d_ids;
  a.out = d_out;
  a.err = d_err_word;
  a.n_rows = n_rows;
  a.n_units = n_ids;
  a.S = S;
  a.s_log2 = log2_if_pow2(S);
  a.G = slots_host ? 1u : dec_units_per_tile(S);  // one row per wavefront over PCIe, as for the packed gather
  a.row_bytes = (uint32_t)row_bytes;
  const uint32_t row_blocks = (uint32_t)(row_bytes / 16);
  a.img_dw = row_blocks * 4 + 4;
  // First round of loads: the blocks of the shortest compressed row (every chunk
  // matching: S + S (W - popcount(Mask)) bits), at least its header and four
  // blocks, rounded up to whole 128-byte lines of the slot when slots start on
  // lines (host memory is read in 128-byte requests, so the rest of a line costs
  // nothing).  A row longer than that takes a second round.  When most rows are
  // near the shortest length, as on dense data, the slot is read in one round.
  {
    const uint32_t min_bits = S + S * (p.W - p.pc);
    uint32_t h = (min_bits + 127) / 128;
    const uint32_t hdr = (S + 127) / 128;
    if (h < hdr) h = hdr;
    if (h < 4) h = 4;
    if (row_bytes % 128 == 0) h = (h + 7) & ~7u;
    a.head_blocks = h < row_blocks ? h : row_blocks;
  }
  a.wave_dw = (a.G * a.img_dw + 8 * a.G + (a.G & 1u) + 3) & ~3u;
  return status_of(launch_decode_slots(a, p, static_cast<hipStream_t>(hip_stream)));
}

// ------------------------------------------------------------------ comparison codec: BF16 exponent coding

// Mass of BF16 exponent e under N(0, sigma^2): |x| in [2^(e-127), 2^(e-126)) for a
// normal exponent, |x| < 2^-126 for e = 0 (zero and subnormals), none for e = 255.
static double zip_exponent_mass(int e, double sigma) {
  const double d = sigma * sqrt(2.0);
  if (e == 0) return erf(ldexp(1.0, -126) / d);
  if (e == 255) return 0.0;
  return erf(ldexp(1.0, e - 126) / d) - erf(ldexp(1.0, e - 127) / d);
}

IBP_API int ibp_zip_table_from_sigma(double sigma, uint8_t *table_out) {
  if (!table_out || !(sigma > 0.0) || !isfinite(sigma)) return IBP_ERR_INVALID_ARG;
  double mass[256];
  for (int e = 0; e < 256; ++e) mass[e] = zip_exponent_mass(e, sigma);
  bool taken[256] = {false};
  for (int k = 0; k < 7; ++k) {  // largest mass first; equal masses: smaller exponent first
    int best = -1;
    for (int e = 0; e < 256; ++e)
      if (!taken[e] && (best < 0 || mass[e] > mass[best])) best = e;
    taken[best] = true;
    table_out[k] = (uint8_t)best;
  }
  return IBP_OK;
}

IBP_API uint64_t ibp_zip_blocks(uint64_t n) { return (n + kZipBlock - 1) / kZipBlock; }
IBP_API uint64_t ibp_zip_codes_bytes(uint64_t n) { return ibp_zip_blocks(n) * (3 * kZipBlock / 8); }
IBP_API uint64_t ibp_zip_workspace_bytes(uint64_t n) {
  // control word, then the look-back status words of the compressor's workgroups
  return n ? 8 + 8 * status_words((ibp_zip_blocks(n) + kZipWG - 1) / kZipWG) : 8;
}

static bool zip_table_ok(const uint8_t *t) {
  if (!t) return false;
  for (int a = 0; a < 7; ++a)
    for (int b = a + 1; b < 7; ++b)
      if (t[a] == t[b]) return false;
  return true;
}

IBP_API int ibp_zip_compress(const uint8_t *table, const void *d_in, uint64_t n, uint8_t *d_sm, uint8_t *d_codes,
                             uint8_t *d_esc, uint64_t esc_capacity, uint64_t *d_eoff, void *d_workspace,
                             uint64_t workspace_bytes, uint32_t *d_err_word, void *hip_stream) {
  if (!zip_table_ok(table) || !d_eoff) return IBP_ERR_INVALID_ARG;
  if (n >= (1ull << 40)) return IBP_ERR_SIZE;
  if (n && (!d_in || !d_sm || !d_codes || !d_esc || !d_workspace)) return IBP_ERR_INVALID_ARG;
  if (!aligned(d_in, 16) || !aligned(d_sm, 8) || !aligned(d_eoff, 8) || !aligned(d_workspace, 8))
    return IBP_ERR_INVALID_ARG;
  if (esc_capacity < n || workspace_bytes < ibp_zip_workspace_bytes(n)) return IBP_ERR_CAPACITY;
  const uint64_t nblk = ibp_zip_blocks(n);
  if (!view(d_in, 2 * n) || !view(d_sm, n) || !view(d_codes, ibp_zip_codes_bytes(n)) || !view(d_esc, n) ||
      !view(d_eoff, 8 * (nblk + 1)) || !view(d_workspace, n ? ibp_zip_workspace_bytes(n) : 0) ||
      !view(d_err_word, d_err_word ? 4 : 0))
    return IBP_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  if (n == 0) return status_of(launch_zero(d_eoff, 1, s));
  ZipArgs a;
  memset(&a, 0, sizeof(a));
  a.in = static_cast<const uint16_t *>(d_in);
  a.sm = d_sm;
  a.codes = d_codes;
  a.esc = d_esc;
  a.eoff = d_eoff;
  a.control = static_cast<uint32_t *>(d_workspace);
  a.status = reinterpret_cast<uint64_t *>(static_cast<uint8_t *>(d_workspace) + 8);
  a.err = d_err_word;
  a.n = n;
  a.nblk = nblk;
  for (int k = 0; k < 7; ++k) a.table[k] = table[k];
  a.wait_limit = g_wait_limit.load();
  a.st_lg = status_lg((nblk + kZipWG - 1) / kZipWG);
  return status_of(launch_zip_encode(a, s));
}

IBP_API int ibp_zip_decompress(const uint8_t *table, const uint8_t *d_sm, const uint8_t *d_codes,
                               const uint8_t *d_esc, uint64_t esc_bytes, const uint64_t *d_eoff, uint64_t n,
                               void *d_out, uint32_t *d_err_word, void *hip_stream) {
  if (!zip_table_ok(table) || !d_eoff) return IBP_ERR_INVALID_ARG;
  if (n >= (1ull << 40)) return IBP_ERR_SIZE;
  if (n && (!d_sm || !d_codes || !d_out)) return IBP_ERR_INVALID_ARG;
  if (esc_bytes && !d_esc) return IBP_ERR_INVALID_ARG;
  if (!aligned(d_out, 16) || !aligned(d_sm, 8) || !aligned(d_eoff, 8)) return IBP_ERR_INVALID_ARG;
  const uint64_t nblk = ibp_zip_blocks(n);
  if (!view(d_sm, n) || !view(d_codes, ibp_zip_codes_bytes(n)) || !view(d_esc, esc_bytes) ||
      !view(d_eoff, 8 * (nblk + 1)) || !view(d_out, 2 * n) || !view(d_err_word, d_err_word ? 4 : 0))
    return IBP_ERR_INVALID_ARG;
  if (n == 0) return IBP_OK;
  ZipArgs a;
  memset(&a, 0, sizeof(a));
  a.out = static_cast<uint16_t *>(d_out);
  a.sm = const_cast<uint8_t *>(d_sm);
  a.codes = const_cast<uint8_t *>(d_codes);
  a.esc = const_cast<uint8_t *>(d_esc);
  a.esc_bytes = esc_bytes;
  a.eoff = const_cast<uint64_t *>(d_eoff);
  a.err = d_err_word;
  a.n = n;
  a.nblk = nblk;
  for (int k = 0; k < 7; ++k) a.table[k] = table[k];
  return status_of(launch_zip_decode(a, static_cast<hipStream_t>(hip_stream)));
}

}  // extern "C"
