/*
 * ibp_oracle.c -- plain, slow CPU oracle of the Invariant Bit Packing (IBP) codec.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
 * benchmark's CPU-baseline leg load this library.  The GPU library never links,
 * includes or calls it, and the two share no source, header, table or helper.
 *
 * Source of the method: the IBP technical summary "Riduzione del Collo di
 * Bottiglia della Memoria GPU con la Compressione Lossless per il ML"
 * (gist.science, paper 2605.30728), section "Algoritmo Core":
 *   step 1 "Preprocessing"   -> ibpo_count_ones, ibpo_threshold, ibpo_meta_from_counts
 *   step 2 "Compressione"    -> ibpo_offsets, ibpo_encode, ibpo_encode_segment
 *   step 3 "Decompressione"  -> ibpo_decode, ibpo_decode_gather
 * and, from section "Integrazione del Sistema", the fixed-slot layout
 * (ibpo_encode_slots, ibpo_decode_slots_gather), plus the position-dependent
 * metadata variant (ibpo_build_meta_pos, ibpo_offsets_pos, ibpo_encode_pos,
 * ibpo_decode_pos; readings R11-R13 below).  The comparison codec of the page
 * "ZipCCL: Efficient Lossless Data Compression of Communication Collectives for
 * Accelerating LLM Training" (gist.science, paper 2604.27844), section 2
 * (Metodologia) A and B, is at the end (ibpo_zip_table, ibpo_zip_encode,
 * ibpo_zip_decode; readings Z1-Z6).
 *
 * The page fixes the idea, not a bit layout.  Where it is silent this file takes
 * these readings (the same list, with reasons, is kept in the design notes):
 *   R1  A sample unit and a chunk are both W-bit words; byte input is read as
 *       consecutive little-endian W/8-byte words.
 *   R2  Bit b is invariant when its majority value occurs in at least k of the N
 *       samples, k = ceil(Tppm * N / 10^6) with Tppm = round(T * 10^6), and
 *       0.5 < T <= 1 so that the majority value is unique.  Bitval holds that
 *       majority value on Mask positions and 0 elsewhere.
 *   R3  A chunk participates (is compressed) exactly when all of its Mask bits
 *       equal Bitval; its payload is then its non-Mask bits in increasing
 *       position order packed from bit 0 (a parallel bit extract), W - popcount(Mask)
 *       bits long.  A chunk that does not participate keeps all W bits.
 *   R4  Participation bit 1 means "compressed".  The participation bits of the
 *       m chunks of a segment are written first, in chunk order, as an m-bit
 *       header; the payloads follow back to back in chunk order.  The bit count
 *       is the same as one prefix bit per chunk.
 *   R5  Segments hold S consecutive chunks (the last may hold fewer), are
 *       bit-contiguous with no padding, and are located by a table of nseg+1
 *       uint64 bit offsets, off[0] = 0, off[nseg] = total bits.
 *   R6  Stream bit q is bit (q mod 8) of byte q/8; a field is written low bit
 *       first.  Unused high bits of the last byte are 0.
 *   R7  Decoding rebuilds a compressed chunk as deposit(payload, ~Mask) OR Bitval
 *       and a raw chunk as its W payload bits; a segment whose decoded length
 *       differs from its offset span is reported as corrupt.
 */
#include <stdint.h>
#include <string.h>
#include <math.h>

#define IBPO_OK 0
#define IBPO_EARG 1      /* bad argument (W, S, T, mask, value range, NULL) */
#define IBPO_ESIZE 2     /* byte count not a whole number of chunks, bad id */
#define IBPO_ECAP 3      /* output buffer too small */
#define IBPO_ECORRUPT 5  /* offset table and stream disagree */

/* ------------------------------------------------------------------ */
/* chunk access                                                        */
/* ------------------------------------------------------------------ */

/* Low W bits set. */
static uint64_t low_bits(unsigned W) { return W >= 64 ? ~0ull : ((1ull << W) - 1ull); }

/* Bit b of x. */
static unsigned bit_of(uint64_t x, unsigned b) { return (unsigned)((x >> b) & 1ull); }

/* Chunk i of a source: either an array of uint64 values (one chunk each, any W)
 * or a byte array read as little-endian W/8-byte words (R1). */
static uint64_t chunk_at(const void *src, int is_bytes, unsigned W, uint64_t i) {
  if (!is_bytes) return ((const uint64_t *)src)[i];
  const uint8_t *p = (const uint8_t *)src + i * (uint64_t)(W / 8);
  uint64_t v = 0;
  for (unsigned j = 0; j < W / 8; ++j) v |= (uint64_t)p[j] << (8 * j);
  return v;
}

static void chunk_put(void *dst, int is_bytes, unsigned W, uint64_t i, uint64_t v) {
  if (!is_bytes) { ((uint64_t *)dst)[i] = v; return; }
  uint8_t *p = (uint8_t *)dst + i * (uint64_t)(W / 8);
  for (unsigned j = 0; j < W / 8; ++j) p[j] = (uint8_t)(v >> (8 * j));
}

static int width_ok(unsigned W, int is_bytes) {
  if (W < 1 || W > 64) return 0;
  if (is_bytes && (W % 8) != 0) return 0;
  return 1;
}

/* Number of set bits, one position at a time. */
static unsigned count_set(uint64_t x, unsigned W) {
  unsigned c = 0;
  for (unsigned b = 0; b < W; ++b) c += bit_of(x, b);
  return c;
}

/* ------------------------------------------------------------------ */
/* step 1: metadata (Algoritmo Core, Preprocessing)                    */
/* ------------------------------------------------------------------ */

/* k = ceil(Tppm * N / 10^6), Tppm = round(T * 10^6) (R2).  Returns 0 when T is
 * outside (0.5, 1] or N == 0. */
uint64_t ibpo_threshold(uint64_t N, double T) {
  if (!(T > 0.5 && T <= 1.0) || N == 0) return 0;
  uint64_t tppm = (uint64_t)llround(T * 1e6);
  unsigned __int128 num = (unsigned __int128)tppm * N;
  unsigned __int128 k = (num + 999999u) / 1000000u;
  return (uint64_t)k;
}

/* c1[b] = number of samples whose bit b is 1, for b < W. */
int ibpo_count_ones(const void *samples, int is_bytes, uint64_t N, unsigned W, uint64_t *c1) {
  if (!width_ok(W, is_bytes) || !c1 || (N && !samples)) return IBPO_EARG;
  for (unsigned b = 0; b < W; ++b) c1[b] = 0;
  for (uint64_t j = 0; j < N; ++j) {
    uint64_t s = chunk_at(samples, is_bytes, W, j);
    for (unsigned b = 0; b < W; ++b) c1[b] += bit_of(s, b);
  }
  return IBPO_OK;
}

/* Mask and Bitval from per-position one-counts over N samples (R2). */
int ibpo_meta_from_counts(const uint64_t *c1, uint64_t N, unsigned W, double T,
                          uint64_t *mask, uint64_t *bitval) {
  if (W < 1 || W > 64 || !c1 || !mask || !bitval) return IBPO_EARG;
  uint64_t k = ibpo_threshold(N, T);
  if (k == 0) return IBPO_EARG;
  uint64_t m = 0, bv = 0;
  for (unsigned b = 0; b < W; ++b) {
    if (c1[b] > N) return IBPO_EARG;
    uint64_t ones = c1[b], zeros = N - c1[b];
    uint64_t majority = ones > zeros ? ones : zeros;
    if (majority >= k) {
      m |= 1ull << b;
      if (ones > zeros) bv |= 1ull << b;
    }
  }
  *mask = m;
  *bitval = bv;
  return IBPO_OK;
}

int ibpo_build_meta(const void *samples, int is_bytes, uint64_t N, unsigned W, double T,
                    uint64_t *mask, uint64_t *bitval, uint64_t *c1_out) {
  uint64_t c1[64];
  int rc = ibpo_count_ones(samples, is_bytes, N, W, c1);
  if (rc) return rc;
  rc = ibpo_meta_from_counts(c1, N, W, T, mask, bitval);
  if (rc) return rc;
  if (c1_out)
    for (unsigned b = 0; b < W; ++b) c1_out[b] = c1[b];
  return IBPO_OK;
}

/* ------------------------------------------------------------------ */
/* step 2: compression (Algoritmo Core, Compressione)                  */
/* ------------------------------------------------------------------ */

/* Parallel bit extract: the bits of v at the set positions of F, in increasing
 * position order, packed from bit 0 (R3). */
static uint64_t extract_bits(uint64_t v, uint64_t F, unsigned W) {
  uint64_t out = 0;
  unsigned t = 0;
  for (unsigned b = 0; b < W; ++b)
    if (bit_of(F, b)) { out |= (uint64_t)bit_of(v, b) << t; ++t; }
  return out;
}

/* Parallel bit deposit: bit t of x goes to the t-th set position of F (R7). */
static uint64_t deposit_bits(uint64_t x, uint64_t F, unsigned W) {
  uint64_t out = 0;
  unsigned t = 0;
  for (unsigned b = 0; b < W; ++b)
    if (bit_of(F, b)) { out |= (uint64_t)bit_of(x, t) << b; ++t; }
  return out;
}

/* Does the chunk match the invariant bits?  Every Mask position must hold its
 * Bitval value. */
static int participates(uint64_t v, uint64_t mask, uint64_t bitval) {
  return ((v ^ bitval) & mask) == 0;
}

/* Set stream bits q .. q+L-1 to bits 0 .. L-1 of x (R6).  The target bits must be 0. */
static void put_bits(uint8_t *stream, uint64_t q, uint64_t x, unsigned L) {
  for (unsigned j = 0; j < L; ++j)
    if (bit_of(x, j)) stream[(q + j) >> 3] |= (uint8_t)(1u << ((q + j) & 7));
}

/* Read stream bits q .. q+L-1 as an L-bit field (R6). */
static uint64_t get_bits(const uint8_t *stream, uint64_t q, unsigned L) {
  uint64_t x = 0;
  for (unsigned j = 0; j < L; ++j)
    x |= (uint64_t)((stream[(q + j) >> 3] >> ((q + j) & 7)) & 1u) << j;
  return x;
}

static int meta_ok(unsigned W, uint64_t mask, uint64_t bitval) {
  uint64_t full = low_bits(W);
  return (mask & ~full) == 0 && (bitval & ~mask) == 0;
}

static int values_ok(const void *src, int is_bytes, uint64_t n, unsigned W) {
  if (is_bytes || W == 64) return 1;
  for (uint64_t i = 0; i < n; ++i)
    if (((const uint64_t *)src)[i] >> W) return 0;
  return 1;
}

/* Bits of segment k: m header bits plus each chunk's payload length (R3, R4). */
static uint64_t segment_bits(const void *src, int is_bytes, uint64_t n, unsigned W,
                             uint64_t mask, uint64_t bitval, uint64_t S, uint64_t k) {
  unsigned pc = count_set(mask, W);
  uint64_t first = k * S, last = first + S < n ? first + S : n;
  uint64_t bits = last - first;
  for (uint64_t i = first; i < last; ++i)
    bits += participates(chunk_at(src, is_bytes, W, i), mask, bitval) ? (uint64_t)(W - pc) : W;
  return bits;
}

/* off[0..nseg]: bit offset of each segment and the total (R5). */
int ibpo_offsets(const void *src, int is_bytes, uint64_t n, unsigned W, uint64_t mask,
                 uint64_t bitval, uint64_t S, uint64_t *off) {
  if (!width_ok(W, is_bytes) || S == 0 || !off || (n && !src) || !meta_ok(W, mask, bitval))
    return IBPO_EARG;
  if (!values_ok(src, is_bytes, n, W)) return IBPO_EARG;
  uint64_t nseg = (n + S - 1) / S;
  off[0] = 0;
  for (uint64_t k = 0; k < nseg; ++k)
    off[k + 1] = off[k] + segment_bits(src, is_bytes, n, W, mask, bitval, S, k);
  return IBPO_OK;
}

/* Write segment k at stream bit q: header, then payloads (R3, R4). */
static uint64_t write_segment(uint8_t *stream, uint64_t q, const void *src, int is_bytes,
                              uint64_t n, unsigned W, uint64_t mask, uint64_t bitval,
                              uint64_t S, uint64_t k) {
  uint64_t F = ~mask & low_bits(W);
  unsigned pc = count_set(mask, W);
  uint64_t first = k * S, last = first + S < n ? first + S : n;
  for (uint64_t i = first; i < last; ++i) {
    unsigned p = (unsigned)participates(chunk_at(src, is_bytes, W, i), mask, bitval);
    put_bits(stream, q, p, 1);
    q += 1;
  }
  for (uint64_t i = first; i < last; ++i) {
    uint64_t v = chunk_at(src, is_bytes, W, i);
    if (participates(v, mask, bitval)) {
      put_bits(stream, q, extract_bits(v, F, W), W - pc);
      q += W - pc;
    } else {
      put_bits(stream, q, v, W);
      q += W;
    }
  }
  return q;
}

/* Compress n chunks: fills off[0..nseg] and stream[0 .. ceil(total/8)). */
int ibpo_encode(const void *src, int is_bytes, uint64_t n, unsigned W, uint64_t mask,
                uint64_t bitval, uint64_t S, uint64_t *off, uint8_t *stream, uint64_t cap) {
  int rc = ibpo_offsets(src, is_bytes, n, W, mask, bitval, S, off);
  if (rc) return rc;
  uint64_t nseg = (n + S - 1) / S;
  uint64_t total = off[nseg];
  uint64_t nbytes = (total + 7) / 8;
  if (nbytes > cap) return IBPO_ECAP;
  if (nbytes && !stream) return IBPO_EARG;
  if (nbytes) memset(stream, 0, nbytes);
  for (uint64_t k = 0; k < nseg; ++k) {
    uint64_t end = write_segment(stream, off[k], src, is_bytes, n, W, mask, bitval, S, k);
    if (end != off[k + 1]) return IBPO_ECORRUPT; /* cannot happen: same lengths */
  }
  return IBPO_OK;
}

/* Segment k alone, written from bit 0 of buf (for spot checks at large sizes). */
int ibpo_encode_segment(const void *src, int is_bytes, uint64_t n, unsigned W, uint64_t mask,
                        uint64_t bitval, uint64_t S, uint64_t k, uint8_t *buf, uint64_t cap,
                        uint64_t *bits) {
  if (!width_ok(W, is_bytes) || S == 0 || !bits || !src || !meta_ok(W, mask, bitval))
    return IBPO_EARG;
  uint64_t nseg = (n + S - 1) / S;
  if (k >= nseg) return IBPO_ESIZE;
  uint64_t b = segment_bits(src, is_bytes, n, W, mask, bitval, S, k);
  if ((b + 7) / 8 > cap || !buf) return IBPO_ECAP;
  memset(buf, 0, (b + 7) / 8);
  write_segment(buf, 0, src, is_bytes, n, W, mask, bitval, S, k);
  *bits = b;
  return IBPO_OK;
}

/* ------------------------------------------------------------------ */
/* step 3: decompression (Algoritmo Core, Decompressione)              */
/* ------------------------------------------------------------------ */

/* Decode the m chunks of the segment at bits [a, b) into dst chunks d0 .. d0+m-1 (R7). */
static int read_segment(const uint8_t *stream, uint64_t a, uint64_t b, uint64_t m, unsigned W,
                        uint64_t mask, uint64_t bitval, void *dst, int is_bytes, uint64_t d0) {
  uint64_t F = ~mask & low_bits(W);
  unsigned pc = count_set(mask, W);
  if (b < a || b - a < m) return IBPO_ECORRUPT;
  uint64_t q = a + m;
  for (uint64_t i = 0; i < m; ++i) {
    unsigned p = (unsigned)get_bits(stream, a + i, 1);
    unsigned L = p ? W - pc : W;
    if (q + L > b) return IBPO_ECORRUPT;
    uint64_t x = get_bits(stream, q, L);
    q += L;
    chunk_put(dst, is_bytes, W, d0 + i, p ? (deposit_bits(x, F, W) | bitval) : x);
  }
  return q == b ? IBPO_OK : IBPO_ECORRUPT;
}

/* Decompress n chunks into dst, given the stream and its offset table. */
int ibpo_decode(const uint8_t *stream, uint64_t stream_bytes, const uint64_t *off, uint64_t n,
                unsigned W, uint64_t mask, uint64_t bitval, uint64_t S, void *dst, int is_bytes) {
  if (!width_ok(W, is_bytes) || S == 0 || !off || (n && (!dst || !stream)) ||
      !meta_ok(W, mask, bitval))
    return IBPO_EARG;
  uint64_t nseg = (n + S - 1) / S;
  if (off[nseg] > stream_bytes * 8) return IBPO_ECORRUPT;
  for (uint64_t k = 0; k < nseg; ++k) {
    uint64_t first = k * S, m = (first + S < n ? first + S : n) - first;
    if (off[k] > off[k + 1]) return IBPO_ECORRUPT;
    int rc = read_segment(stream, off[k], off[k + 1], m, W, mask, bitval, dst, is_bytes, first);
    if (rc) return rc;
  }
  return IBPO_OK;
}

/* Row j of dst (S chunks) = segment ids[j] of a stream of nseg full segments. */
int ibpo_decode_gather(const uint8_t *stream, uint64_t stream_bytes, const uint64_t *off,
                       uint64_t nseg, uint64_t S, const int64_t *ids, uint64_t n_ids,
                       unsigned W, uint64_t mask, uint64_t bitval, void *dst, int is_bytes) {
  if (!width_ok(W, is_bytes) || S == 0 || !off || (n_ids && (!ids || !dst || !stream)) ||
      !meta_ok(W, mask, bitval))
    return IBPO_EARG;
  for (uint64_t j = 0; j < n_ids; ++j) {
    int64_t id = ids[j];
    if (id < 0 || (uint64_t)id >= nseg) return IBPO_ESIZE;
    uint64_t a = off[id], b = off[id + 1];
    if (b < a || b > stream_bytes * 8) return IBPO_ECORRUPT;
    int rc = read_segment(stream, a, b, S, W, mask, bitval, dst, is_bytes, j * S);
    if (rc) return rc;
  }
  return IBPO_OK;
}

/* ------------------------------------------------------------------ */
/* fixed-slot layout (Integrazione del Sistema, PCIe transfer mode)    */
/* ------------------------------------------------------------------ */
/*
 * The in-place layout of the IBP page's PCIe transfer compression: every row of
 * S chunks keeps a fixed slot of row_bytes = S*W/8 bytes (its uncompressed size)
 * and only the used part of a slot is read.  Readings:
 *   R8  Row r's slot starts at byte r*row_bytes.  If the row's segment encoding
 *       (header of S participation bits, then the payloads: the same bits as a
 *       segment of the packed stream) is shorter than S*W bits, the slot holds
 *       those bits from its bit 0 and flag r is 1; otherwise it holds the raw row
 *       and flag r is 0.
 *   R9  Flags are a bit vector in 64-bit words: bit r%64 of word r/64.
 *   R10 The used length of a compressed slot is not stored: it follows from the
 *       header, S + sum over chunks of (participating ? W - popcount(Mask) : W).
 * This oracle zeroes the unused tail of every slot; a reader never looks at it.
 */

/* Slots and flags of n_rows rows of S chunks (byte input, W a multiple of 8). */
int ibpo_encode_slots(const void *src, uint64_t n_rows, unsigned W, uint64_t mask, uint64_t bitval,
                      uint64_t S, uint8_t *slots, uint64_t *flags) {
  if (!width_ok(W, 1) || S == 0 || (n_rows && (!src || !slots || !flags)) || !meta_ok(W, mask, bitval))
    return IBPO_EARG;
  const uint64_t row_bytes = S * (W / 8), row_bits = S * W, n = n_rows * S;
  for (uint64_t w = 0; w < (n_rows + 63) / 64; ++w) flags[w] = 0;
  for (uint64_t r = 0; r < n_rows; ++r) {
    uint8_t *slot = slots + r * row_bytes;
    memset(slot, 0, row_bytes);
    uint64_t bits = segment_bits(src, 1, n, W, mask, bitval, S, r);
    if (bits < row_bits) {
      write_segment(slot, 0, src, 1, n, W, mask, bitval, S, r);
      flags[r / 64] |= 1ull << (r % 64);
    } else {
      for (uint64_t i = 0; i < S; ++i) chunk_put(slot, 1, W, i, chunk_at(src, 1, W, r * S + i));
    }
  }
  return IBPO_OK;
}

/* Used bits of slot r: from its header when compressed, else the whole row. */
uint64_t ibpo_slot_bits(const uint8_t *slots, uint64_t r, unsigned W, uint64_t mask, uint64_t S,
                        const uint64_t *flags) {
  const uint8_t *slot = slots + r * S * (W / 8);
  if (!((flags[r / 64] >> (r % 64)) & 1ull)) return S * W;
  unsigned pc = count_set(mask, W);
  uint64_t bits = S;
  for (uint64_t i = 0; i < S; ++i) bits += get_bits(slot, i, 1) ? (uint64_t)(W - pc) : W;
  return bits;
}

/* Row j of dst = row ids[j] read from its slot. */
int ibpo_decode_slots_gather(const uint8_t *slots, uint64_t n_rows, unsigned W, uint64_t mask,
                             uint64_t bitval, uint64_t S, const uint64_t *flags, const int64_t *ids,
                             uint64_t n_ids, void *dst, int is_bytes) {
  if (!width_ok(W, 1) || S == 0 || (n_ids && (!slots || !flags || !ids || !dst)) || !meta_ok(W, mask, bitval))
    return IBPO_EARG;
  const uint64_t row_bytes = S * (W / 8);
  for (uint64_t j = 0; j < n_ids; ++j) {
    int64_t id = ids[j];
    if (id < 0 || (uint64_t)id >= n_rows) return IBPO_ESIZE;
    const uint8_t *slot = slots + (uint64_t)id * row_bytes;
    if ((flags[id / 64] >> (id % 64)) & 1ull) {
      uint64_t bits = ibpo_slot_bits(slots, (uint64_t)id, W, mask, S, flags);
      if (bits >= S * W) return IBPO_ECORRUPT;
      int rc = read_segment(slot, 0, bits, S, W, mask, bitval, dst, is_bytes, j * S);
      if (rc) return rc;
    } else {
      for (uint64_t i = 0; i < S; ++i) chunk_put(dst, is_bytes, W, j * S + i, chunk_at(slot, 1, W, i));
    }
  }
  return IBPO_OK;
}

/* ------------------------------------------------------------------ */
/* position-dependent metadata (Algoritmo Core, Preprocessing: a      */
/* fixed-size metadata block "of the order of kilobytes")             */
/* ------------------------------------------------------------------ */
/*
 * Variant where chunk position i inside a segment (row) has its own Mask_i and
 * Bitval_i, i = 0 .. S-1.  Readings:
 *   R11 A sample unit is a whole row of S chunks; the statistics of position i
 *       are taken over the i-th chunk of every sample row, with the rule of R2
 *       and N = number of sample rows.
 *   R12 The stream layout is that of R4-R6: a participating chunk at position i
 *       carries W - popcount(Mask_i) payload bits (the bits outside Mask_i).
 *   R13 A short last segment of m < S chunks uses positions 0 .. m-1.
 */

/* Mask_i, Bitval_i (and optionally the one-counts c1[i*W + b]) from n_rows sample rows. */
int ibpo_build_meta_pos(const void *samples, int is_bytes, uint64_t n_rows, unsigned W, uint64_t S, double T,
                        uint64_t *mask, uint64_t *bitval, uint64_t *c1) {
  if (!width_ok(W, is_bytes) || S == 0 || n_rows == 0 || !samples || !mask || !bitval) return IBPO_EARG;
  for (uint64_t i = 0; i < S; ++i) {
    uint64_t c[64] = {0};
    for (uint64_t r = 0; r < n_rows; ++r) {
      uint64_t v = chunk_at(samples, is_bytes, W, r * S + i);
      for (unsigned b = 0; b < W; ++b) c[b] += bit_of(v, b);
    }
    int rc = ibpo_meta_from_counts(c, n_rows, W, T, &mask[i], &bitval[i]);
    if (rc) return rc;
    if (c1)
      for (unsigned b = 0; b < W; ++b) c1[i * W + b] = c[b];
  }
  return IBPO_OK;
}

static int meta_pos_ok(unsigned W, const uint64_t *mask, const uint64_t *bitval, uint64_t S) {
  for (uint64_t i = 0; i < S; ++i)
    if (!meta_ok(W, mask[i], bitval[i])) return 0;
  return 1;
}

/* Bits of segment k when position i uses Mask_i / Bitval_i (R12, R13). */
static uint64_t segment_bits_pos(const void *src, int is_bytes, uint64_t n, unsigned W, const uint64_t *mask,
                                 const uint64_t *bitval, uint64_t S, uint64_t k) {
  uint64_t first = k * S, last = first + S < n ? first + S : n;
  uint64_t bits = last - first;
  for (uint64_t c = first; c < last; ++c) {
    uint64_t i = c - first;
    bits += participates(chunk_at(src, is_bytes, W, c), mask[i], bitval[i]) ? (uint64_t)(W - count_set(mask[i], W))
                                                                            : W;
  }
  return bits;
}

int ibpo_offsets_pos(const void *src, int is_bytes, uint64_t n, unsigned W, const uint64_t *mask,
                     const uint64_t *bitval, uint64_t S, uint64_t *off) {
  if (!width_ok(W, is_bytes) || S == 0 || !off || (n && !src) || !mask || !bitval || !meta_pos_ok(W, mask, bitval, S))
    return IBPO_EARG;
  if (!values_ok(src, is_bytes, n, W)) return IBPO_EARG;
  uint64_t nseg = (n + S - 1) / S;
  off[0] = 0;
  for (uint64_t k = 0; k < nseg; ++k) off[k + 1] = off[k] + segment_bits_pos(src, is_bytes, n, W, mask, bitval, S, k);
  return IBPO_OK;
}

/* Segment k at stream bit q: header, then each chunk's payload under its position's metadata. */
static uint64_t write_segment_pos(uint8_t *stream, uint64_t q, const void *src, int is_bytes, uint64_t n,
                                  unsigned W, const uint64_t *mask, const uint64_t *bitval, uint64_t S,
                                  uint64_t k) {
  uint64_t first = k * S, last = first + S < n ? first + S : n;
  for (uint64_t c = first; c < last; ++c) {
    uint64_t i = c - first;
    put_bits(stream, q, (uint64_t)participates(chunk_at(src, is_bytes, W, c), mask[i], bitval[i]), 1);
    q += 1;
  }
  for (uint64_t c = first; c < last; ++c) {
    uint64_t i = c - first, v = chunk_at(src, is_bytes, W, c);
    if (participates(v, mask[i], bitval[i])) {
      unsigned L = W - count_set(mask[i], W);
      put_bits(stream, q, extract_bits(v, ~mask[i] & low_bits(W), W), L);
      q += L;
    } else {
      put_bits(stream, q, v, W);
      q += W;
    }
  }
  return q;
}

int ibpo_encode_pos(const void *src, int is_bytes, uint64_t n, unsigned W, const uint64_t *mask,
                    const uint64_t *bitval, uint64_t S, uint64_t *off, uint8_t *stream, uint64_t cap) {
  int rc = ibpo_offsets_pos(src, is_bytes, n, W, mask, bitval, S, off);
  if (rc) return rc;
  uint64_t nseg = (n + S - 1) / S;
  uint64_t nbytes = (off[nseg] + 7) / 8;
  if (nbytes > cap) return IBPO_ECAP;
  if (nbytes && !stream) return IBPO_EARG;
  if (nbytes) memset(stream, 0, nbytes);
  for (uint64_t k = 0; k < nseg; ++k)
    if (write_segment_pos(stream, off[k], src, is_bytes, n, W, mask, bitval, S, k) != off[k + 1]) return IBPO_ECORRUPT;
  return IBPO_OK;
}

/* Decode the m chunks of the segment at bits [a, b) under per-position metadata. */
static int read_segment_pos(const uint8_t *stream, uint64_t a, uint64_t b, uint64_t m, unsigned W,
                            const uint64_t *mask, const uint64_t *bitval, void *dst, int is_bytes, uint64_t d0) {
  if (b < a || b - a < m) return IBPO_ECORRUPT;
  uint64_t q = a + m;
  for (uint64_t i = 0; i < m; ++i) {
    unsigned p = (unsigned)get_bits(stream, a + i, 1);
    unsigned L = p ? W - count_set(mask[i], W) : W;
    if (q + L > b) return IBPO_ECORRUPT;
    uint64_t x = get_bits(stream, q, L);
    q += L;
    chunk_put(dst, is_bytes, W, d0 + i, p ? (deposit_bits(x, ~mask[i] & low_bits(W), W) | bitval[i]) : x);
  }
  return q == b ? IBPO_OK : IBPO_ECORRUPT;
}

int ibpo_decode_pos(const uint8_t *stream, uint64_t stream_bytes, const uint64_t *off, uint64_t n, unsigned W,
                    const uint64_t *mask, const uint64_t *bitval, uint64_t S, void *dst, int is_bytes) {
  if (!width_ok(W, is_bytes) || S == 0 || !off || (n && (!dst || !stream)) || !mask || !bitval ||
      !meta_pos_ok(W, mask, bitval, S))
    return IBPO_EARG;
  uint64_t nseg = (n + S - 1) / S;
  if (off[nseg] > stream_bytes * 8) return IBPO_ECORRUPT;
  for (uint64_t k = 0; k < nseg; ++k) {
    uint64_t first = k * S, m = (first + S < n ? first + S : n) - first;
    if (off[k] > off[k + 1]) return IBPO_ECORRUPT;
    int rc = read_segment_pos(stream, off[k], off[k + 1], m, W, mask, bitval, dst, is_bytes, first);
    if (rc) return rc;
  }
  return IBPO_OK;
}

/* ------------------------------------------------------------------ */
/* second codec for comparison: ZipCCL exponent coding of BF16        */
/* (ZipCCL page, section 2 "Metodologia": A. Gaussian insight,         */
/* B. exponent coding)                                                 */
/* ------------------------------------------------------------------ */
/*
 * Readings (the page gives the idea, not a layout):
 *   Z1 A BF16 element u (16 bits) splits into its exponent e = bits 14..7 and a
 *      sign-mantissa byte sm = (sign << 7) | mantissa (bits 15 and 6..0).
 *   Z2 The exponent table comes from the standard deviation sigma alone (no
 *      histogram): under N(0, sigma^2) exponent e in 1..254 has mass
 *      P(2^(e-127) <= |x| < 2^(e-126)), e = 0 the mass P(|x| < 2^-126), e = 255
 *      none.  The 7 exponents of largest mass (ties: smaller e first) get codes
 *      1..7 in decreasing order of mass.
 *   Z3 An element whose exponent is in the table gets its code; any other gets
 *      code 0 and its exponent goes, in element order, to the escape array.
 *   Z4 Elements are grouped in blocks of 4096.  Block j stores its codes as three
 *      bit planes of 4096 bits (plane p = bit p of every code, element t of the
 *      block at plane bit t, LSB-first bytes), 1536 bytes per block, unused bits 0.
 *   Z5 Outputs: sm[n] bytes, codes[nblk * 1536] bytes, esc[E] bytes, and
 *      eoff[nblk + 1] = escapes before each block (eoff[nblk] = E).
 *   Z6 Decoding: e = code ? table[code - 1] : esc[eoff[j] + rank of the element
 *      among the block's escapes]; u = ((sm & 0x80) << 8) | (e << 7) | (sm & 0x7F).
 */
#define ZIP_BLOCK 4096u
#define ZIP_PLANE_BYTES (ZIP_BLOCK / 8u)

static double zip_mass(unsigned e, double sigma) {
  /* P(a <= |x| < b) for x ~ N(0, sigma^2) = erf(b / (sigma sqrt2)) - erf(a / (sigma sqrt2)) */
  const double s = sigma * sqrt(2.0);
  if (e == 0) return erf(ldexp(1.0, -126) / s);
  if (e >= 255) return 0.0;
  return erf(ldexp(1.0, (int)e - 126) / s) - erf(ldexp(1.0, (int)e - 127) / s);
}

int ibpo_zip_table(double sigma, uint8_t table[7]) {
  if (!(sigma > 0.0) || !table) return IBPO_EARG;
  int used[256] = {0};
  for (int k = 0; k < 7; ++k) {
    int best = -1;
    double bm = -1.0;
    for (int e = 0; e < 256; ++e) {
      if (used[e]) continue;
      double m = zip_mass((unsigned)e, sigma);
      if (m > bm) { /* strictly greater: ties keep the smaller exponent */
        bm = m;
        best = e;
      }
    }
    used[best] = 1;
    table[k] = (uint8_t)best;
  }
  return IBPO_OK;
}

static unsigned zip_code(unsigned e, const uint8_t table[7]) {
  for (unsigned k = 0; k < 7; ++k)
    if (table[k] == e) return k + 1;
  return 0;
}

static int zip_table_ok(const uint8_t table[7]) {
  for (int a = 0; a < 7; ++a)
    for (int b = a + 1; b < 7; ++b)
      if (table[a] == table[b]) return 0;
  return 1;
}

/* Encode n BF16 words.  codes must hold ceil(n/4096)*1536 bytes, esc n bytes,
 * eoff ceil(n/4096)+1 words; *n_esc receives E. */
int ibpo_zip_encode(const uint16_t *x, uint64_t n, const uint8_t table[7], uint8_t *sm, uint8_t *codes,
                    uint8_t *esc, uint64_t *eoff, uint64_t *n_esc) {
  if ((n && (!x || !sm || !codes || !esc)) || !table || !eoff || !n_esc || !zip_table_ok(table)) return IBPO_EARG;
  const uint64_t nblk = (n + ZIP_BLOCK - 1) / ZIP_BLOCK;
  memset(codes, 0, nblk * 3 * ZIP_PLANE_BYTES);
  uint64_t E = 0;
  for (uint64_t j = 0; j < nblk; ++j) {
    eoff[j] = E;
    for (uint64_t t = 0; t < ZIP_BLOCK && j * ZIP_BLOCK + t < n; ++t) {
      const uint64_t i = j * ZIP_BLOCK + t;
      const unsigned u = x[i];
      const unsigned e = (u >> 7) & 0xFFu;
      sm[i] = (uint8_t)(((u >> 8) & 0x80u) | (u & 0x7Fu));
      const unsigned c = zip_code(e, table);
      for (unsigned p = 0; p < 3; ++p)
        if ((c >> p) & 1u) codes[j * 3 * ZIP_PLANE_BYTES + p * ZIP_PLANE_BYTES + t / 8] |= (uint8_t)(1u << (t % 8));
      if (c == 0) esc[E++] = (uint8_t)e;
    }
  }
  eoff[nblk] = E;
  *n_esc = E;
  return IBPO_OK;
}

int ibpo_zip_decode(const uint8_t *sm, const uint8_t *codes, const uint8_t *esc, uint64_t n_esc, const uint64_t *eoff,
                    uint64_t n, const uint8_t table[7], uint16_t *out) {
  if ((n && (!sm || !codes || !out || !eoff)) || !table || !zip_table_ok(table)) return IBPO_EARG;
  const uint64_t nblk = (n + ZIP_BLOCK - 1) / ZIP_BLOCK;
  for (uint64_t j = 0; j < nblk; ++j) {
    uint64_t k = eoff[j];
    for (uint64_t t = 0; t < ZIP_BLOCK && j * ZIP_BLOCK + t < n; ++t) {
      const uint64_t i = j * ZIP_BLOCK + t;
      unsigned c = 0;
      for (unsigned p = 0; p < 3; ++p)
        c |= (unsigned)((codes[j * 3 * ZIP_PLANE_BYTES + p * ZIP_PLANE_BYTES + t / 8] >> (t % 8)) & 1u) << p;
      unsigned e;
      if (c) {
        e = table[c - 1];
      } else {
        if (k >= n_esc || !esc) return IBPO_ECORRUPT;
        e = esc[k++];
      }
      out[i] = (uint16_t)(((sm[i] & 0x80u) << 8) | (e << 7) | (sm[i] & 0x7Fu));
    }
    if (k != eoff[j + 1]) return IBPO_ECORRUPT;
  }
  return IBPO_OK;
}
