// sps_bsc.hip -- the Block-Sparse CSR codec on gfx950: compressed column
// indices for an item corpus kept in HBM, decoded on the device before the
// corpus is prepared.
//
// Format (§3.2 of "稀疏嵌入批量相似度计算的工程化实践"): a column d is the pair
// (block = d / 1024, offset = d % 1024). Per row, the block ids (ascending in
// a canonical row) are stored as differences from the previous entry's block
// id, the first from 0, each an unsigned base-128 varint (7 value bits per
// byte, least significant group first, high bit set on all bytes of a value
// but its last); bptr[r] is the byte position of row r's varints. The 10-bit
// offsets are packed in entry order over the whole matrix, least significant
// bit first (entry k at bits 10k .. 10k + 9). indptr and values are the CSR's.
//
// The encoder runs one wave per row: the lanes take 64 consecutive entries
// of the row at a time, so every load and store of a row is contiguous. The
// decoder runs one thread per row (a wave per row for rows of more than 256
// entries) and gathers a wave's indices in LDS to store them contiguously.
// Every access is bounded by the buffer sizes the host passes, whatever the
// contents.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sps_device.h"
#include "sps_internal.h"

namespace sps {

constexpr int kRowsPerBlock = 4;  // waves (rows) per 256-thread workgroup

__device__ __forceinline__ int varint_len(uint32_t v) {
  return 1 + (v >= (1u << 7)) + (v >= (1u << 14)) + (v >= (1u << 21)) + (v >= (1u << 28));
}

__device__ __forceinline__ void row_range(const int32_t *__restrict__ ptr, int64_t r, int64_t hi,
                                          int64_t &b, int64_t &e) {
  b = clamp64(ptr[r], 0, hi);
  e = clamp64(ptr[r + 1], b, hi);
}

// WRITE = false: bptr[r + 1] = the varint bytes of row r (scanned afterwards).
// WRITE = true: the varint bytes of row r at blocks[bptr[r] ...], none past cap.
template <bool WRITE>
__global__ __launch_bounds__(256) void bsc_encode_rows_kernel(int64_t n_rows, int64_t nnz,
                                                              const int32_t *__restrict__ indptr,
                                                              const int32_t *__restrict__ indices,
                                                              int32_t *__restrict__ bptr,
                                                              uint8_t *__restrict__ blocks,
                                                              int64_t cap) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (r >= n_rows) return;  // uniform per wave
  int64_t e0, e1;
  row_range(indptr, r, nnz, e0, e1);
  int64_t pos = WRITE ? clamp64(bptr[r], 0, cap) : 0;
  uint32_t prev_last = 0;  // block id of the entry before this window
  for (int64_t w0 = e0; w0 < e1; w0 += 64) {
    const int64_t k = w0 + lane;
    const bool valid = k < e1;
    const uint32_t blk = valid ? (uint32_t)indices[k] >> 10 : 0u;
    uint32_t prev = (uint32_t)__shfl_up((int)blk, 1, 64);
    if (lane == 0) prev = prev_last;
    const uint32_t delta = blk - prev;
    const int nb = valid ? varint_len(delta) : 0;
    const int incl = wave_incl_scan_dpp(nb);
    if (WRITE && valid) {
      const int64_t o = pos + (incl - nb);
      uint32_t v = delta;
      for (int j = 0; j < nb; ++j) {
        if (o + j < cap) blocks[o + j] = (uint8_t)((v & 0x7Fu) | (j + 1 < nb ? 0x80u : 0u));
        v >>= 7;
      }
    }
    pos += __builtin_amdgcn_readlane(incl, 63);
    prev_last = (uint32_t)__builtin_amdgcn_readlane((int)blk, 63);  // last window only if partial
  }
  if (!WRITE && lane == 0) bptr[r + 1] = (int32_t)pos;
}

// 32-bit word j of the offset stream: bits 32j .. 32j + 31 hold the offsets
// of entries floor(32j / 10) .. floor((32j + 31) / 10) (at most four), each
// shifted to its place; the words past the stream's last entry are zero.
__global__ __launch_bounds__(256) void bsc_pack_offsets_kernel(int64_t nnz,
                                                               const int32_t *__restrict__ indices,
                                                               uint32_t *__restrict__ words,
                                                               int64_t n_words) {
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= n_words) return;
  const int64_t b0 = 32 * j;
  uint32_t w = 0;
  for (int64_t k = b0 / 10; k <= (b0 + 31) / 10 && k < nnz; ++k) {
    const uint32_t off = (uint32_t)indices[k] & 1023u;
    const int64_t sh = 10 * k - b0;  // -9 .. 31
    w |= sh >= 0 ? off << sh : off >> (-sh);
  }
  words[j] = w;
}

// Column indices from the varint bytes and the offsets. One thread decodes
// one row: a row of the pages corpus holds about 43 entries in about 100
// bytes, so a row per lane keeps every lane busy with no cross-lane step, and
// the thread reads its row's bytes through two 64-bit register windows (the
// varint bytes and the offset bits), each refilled word by word from a
// WordStream of 16-byte loads. Its indices are stored four at a time. Rows of
// more than kThreadRowMax entries are decoded by the whole wave instead
// (decode_row_wave), so that one long row does not hold up a lane for its
// length.
constexpr int kThreadRowMax = 256;

// bytes a .. a + 3 of buf[0 .. n) as a little-endian word (bytes outside the
// buffer read as 0); buf + a is 4-byte aligned, so a word wholly inside is
// one aligned load and the others are read byte by byte within the buffer
__device__ __forceinline__ uint32_t ld_word(const uint8_t *__restrict__ buf, int64_t n,
                                            int64_t a) {
  if (a >= 0 && a + 4 <= n) return *reinterpret_cast<const uint32_t *>(buf + a);
  uint32_t w = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (a + i >= 0 && a + i < n) w |= (uint32_t)buf[a + i] << (8 * i);
  return w;
}

// The little-endian words of buf[0 .. n) from a 4-byte aligned position on,
// read 16 bytes at a time with the next 16 loaded ahead: a thread that walks
// its row's bytes word by word then sends one request to the L1 per four
// words (the L1 cannot hold the lines of every lane of every wave, so each
// request tends to go on to the L2).
struct WordStream {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
  const uint8_t *buf;
  int64_t n;
  int64_t next;  // position of the next 16-byte load
  u32x4 q, qn;   // the current 16 bytes and the next
  int qi;        // words of q already taken
  __device__ __forceinline__ u32x4 ld16(int64_t a) const {
    if (a >= 0 && a + 16 <= n) return *reinterpret_cast<const u32x4_a4 *>(buf + a);
    const u32x4 w = {ld_word(buf, n, a), ld_word(buf, n, a + 4), ld_word(buf, n, a + 8),
                     ld_word(buf, n, a + 12)};
    return w;
  }
  __device__ __forceinline__ void init(const uint8_t *b, int64_t size, int64_t a) {
    buf = b;
    n = size;
    q = ld16(a);
    qn = ld16(a + 16);
    next = a + 32;
    qi = 0;
  }
  __device__ __forceinline__ uint32_t word() {
    const uint32_t w = qi == 0 ? q.x : (qi == 1 ? q.y : (qi == 2 ? q.z : q.w));
    if (++qi == 4) {
      q = qn;
      qn = ld16(next);
      next += 16;
      qi = 0;
    }
    return w;
  }
};

// Row entries [e0, e1) from its varint bytes [p0, p1), by one thread; entry
// e goes to out[e - base]. Returns true when the bytes do not hold exactly the row's entries, or a
// value takes more than 3 bytes (the indices are then unspecified).
__device__ __forceinline__ bool decode_row_thread(int64_t e0, int64_t e1, int64_t p0, int64_t p1,
                                                  const uint8_t *__restrict__ blocks,
                                                  int64_t n_bytes,
                                                  const uint8_t *__restrict__ offsets,
                                                  int64_t n_off, int32_t *__restrict__ out,
                                                  int64_t base) {
  // varint bytes: bw holds the next two words of the row's word stream (from
  // the word at ba on); the next byte is byte bo (0..3) of bw
  const int64_t mb = (int64_t)(reinterpret_cast<uintptr_t>(blocks) & 3u);
  const int64_t ba = ((p0 + mb) & ~(int64_t)3) - mb;
  WordStream bs;
  bs.init(blocks, n_bytes, ba);
  uint64_t bw = (uint64_t)bs.word();
  bw |= (uint64_t)bs.word() << 32;
  int32_t bo = (int32_t)(p0 - ba);
  int64_t left = p1 - p0;  // the row's bytes not yet taken
  // offset bits: ow holds the next two words of the offsets' word stream
  // (from the word at oa on); the next offset starts at bit ob (0..31) of ow
  const int64_t mo = (int64_t)(reinterpret_cast<uintptr_t>(offsets) & 3u);
  const int64_t bit0 = 10 * e0;
  const int64_t oa = (((bit0 >> 3) + mo) & ~(int64_t)3) - mo;
  WordStream os;
  os.init(offsets, n_off, oa);
  uint64_t ow = (uint64_t)os.word();
  ow |= (uint64_t)os.word() << 32;
  int32_t ob = (int32_t)(bit0 - 8 * oa);
  uint32_t blk = 0;
  bool bad = false;
  auto next = [&]() -> int32_t {
    // the value's bytes are among bytes bo .. bo + 2 of the window; its
    // length is where the first clear high bit is (3 at most for an int32
    // column), taken with selects rather than a loop over the bytes
    const uint32_t w = (uint32_t)(bw >> (8 * bo));
    const uint32_t b0 = w & 0xFFu, b1 = (w >> 8) & 0xFFu, b2 = (w >> 16) & 0xFFu;
    const int32_t len = b0 < 0x80u ? 1 : (b1 < 0x80u ? 2 : 3);
    uint32_t v = b0 & 0x7Fu;
    v |= len > 1 ? (b1 & 0x7Fu) << 7 : 0u;
    v |= len > 2 ? (b2 & 0x7Fu) << 14 : 0u;
    // a fourth byte, or a value running past the row's bytes
    bad = bad || (len == 3 && b2 >= 0x80u) || len > left;
    left -= len;
    bo += len;
    if (bo >= 4) {  // bo was <= 3, so one word of the window is used up
      bw = (bw >> 32) | ((uint64_t)bs.word() << 32);
      bo -= 4;
    }
    blk += v;
    const uint32_t off = (uint32_t)(ow >> ob) & 1023u;
    ob += 10;
    if (ob >= 32) {
      ow = (ow >> 32) | ((uint64_t)os.word() << 32);
      ob -= 32;
    }
    return (int32_t)(blk * 1024u + off);
  };
  typedef int32_t i32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
  int64_t e = e0;
  for (; e + 4 <= e1; e += 4) {
    i32x4_a4 x;
    x.x = next();
    x.y = next();
    x.z = next();
    x.w = next();
    *reinterpret_cast<i32x4_a4 *>(out + (e - base)) = x;
  }
  for (; e < e1; ++e) out[e - base] = next();
  return bad || left != 0;
}

// The same for one row by the whole wave (any length). Lane i of a 64-byte
// window takes byte i: the ballot of "last byte of a value" flags gives each
// byte its value (the number of value ends before it) and its place in that
// value; a wave scan of (byte & 0x7f) << 7 place, carried across windows, is
// at every value's last byte the running sum of the differences, i.e. that
// entry's block id. Its 10-bit offset is taken from the row's first 64
// offset bytes by lane shuffles (or loaded, past them). Returns the same flag
// as decode_row_thread, in every lane.
__device__ bool decode_row_wave(int64_t e0, int64_t e1, int64_t p0, int64_t p1,
                                const uint8_t *__restrict__ blocks,
                                const uint8_t *__restrict__ offsets,
                                int32_t *__restrict__ indices) {
  const int lane = threadIdx.x & 63;
  const uint64_t lt = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  const int64_t ob0 = (10 * e0) >> 3;
  const int64_t ob1 = (10 * e1 + 7) >> 3;  // <= ceil(10 nnz / 8)
  const uint32_t wo = ob0 + lane < ob1 ? (uint32_t)offsets[ob0 + lane] : 0u;
  const int64_t ne = e1 - e0;
  bool bad = false;
  uint32_t carry = 0;  // sum of all contributions of the earlier windows
  int64_t got = 0;     // values ended in the earlier windows
  int place0 = 0;      // bytes of an unfinished value before this window
  for (int64_t w0 = p0; w0 < p1; w0 += 64) {
    const int64_t i = w0 + lane;
    const bool valid = i < p1;
    const uint32_t b = valid ? (uint32_t)blocks[i] : 0u;
    const bool last = valid && (b & 0x80u) == 0;
    const uint64_t mask = __ballot(last);
    const uint64_t below = mask & lt;
    const int place = below ? lane - (63 - __clzll(below)) - 1 : lane + place0;
    uint32_t c = 0;
    if (valid) {
      // an int32 column has a block id below 2^21: three bytes at most
      if (place <= 2) c = (b & 0x7Fu) << (7 * place);
      else bad = true;
    }
    const uint32_t incl = (uint32_t)wave_incl_scan_dpp((int32_t)c);
    // this lane's entry (if its byte ends a value) and its offset bytes,
    // taken from the window by every lane (shuffles read all lanes)
    const int64_t k = got + __popcll(below);
    const int64_t e = e0 + k;
    const int64_t bit = 10 * e;
    const int64_t rel = (bit >> 3) - ob0;
    const int src = rel >= 0 && rel < 63 ? (int)rel : 0;
    const uint32_t lo_w = (uint32_t)__shfl((int)wo, src, 64);
    const uint32_t hi_w = (uint32_t)__shfl((int)wo, src + 1, 64);
    if (last) {
      if (k < ne) {
        uint32_t w;
        if (rel >= 0 && rel < 63) w = lo_w | (hi_w << 8);
        else w = (uint32_t)offsets[bit >> 3] | ((uint32_t)offsets[(bit >> 3) + 1] << 8);
        indices[e] = (int32_t)((carry + incl) * 1024u + ((w >> (bit & 7)) & 1023u));
      } else {
        bad = true;
      }
    }
    carry += (uint32_t)__builtin_amdgcn_readlane((int32_t)incl, 63);
    got += __popcll(mask);
    // a full window ends with clz(mask) bytes of a value that goes on
    place0 = mask ? __clzll(mask) : (place0 < (1 << 20) ? place0 + 64 : place0);
  }
  if (p1 > p0 && (blocks[p1 - 1] & 0x80u)) bad = true;  // the row ends inside a value
  if (got != ne) bad = true;
  return __ballot(bad) != 0;
}

// Staged entries per wave: a wave's 64 rows of the pages corpus hold about
// 2,750 entries. Its indices are gathered in LDS and stored as one contiguous
// range, so that every store instruction writes whole lines: lanes storing
// their own rows instead write 64 partial lines each, which the L2 fetches
// and writes back over and over (12x the algorithmic reads, 2.8x the writes).
constexpr int kStage = 3072;

__global__ __launch_bounds__(256) void bsc_decode_kernel(int64_t n_rows, int64_t nnz,
                                                         const int32_t *__restrict__ indptr,
                                                         const int32_t *__restrict__ bptr,
                                                         int64_t n_bytes,
                                                         const uint8_t *__restrict__ blocks,
                                                         const uint8_t *__restrict__ offsets,
                                                         int32_t *__restrict__ indices,
                                                         int32_t *__restrict__ status) {
  __shared__ int32_t stage[4][kStage];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t rw = (int64_t)blockIdx.x * blockDim.x + 64 * wv;  // the wave's first row
  const int64_t r = rw + lane;
  const int64_t n_off = (10 * nnz + 7) >> 3;
  // the row's entry and byte ranges, clamped to the buffers (all below 2^31)
  int32_t e0 = 0, e1 = 0, p0 = 0, p1 = 0;
  if (r < n_rows) {
    e0 = (int32_t)clamp64(indptr[r], 0, nnz);
    e1 = (int32_t)clamp64(indptr[r + 1], e0, nnz);
    p0 = (int32_t)clamp64(bptr[r], 0, n_bytes);
    p1 = (int32_t)clamp64(bptr[r + 1], p0, n_bytes);
  }
  const bool mine = r < n_rows && e1 - e0 <= kThreadRowMax;
  // staged: the wave's rows are all short and follow each other, and their
  // entries [first, last) fit the wave's stage
  const int nv = rw < n_rows ? (int)(n_rows - rw < 64 ? n_rows - rw : 64) : 0;
  const int32_t first = __builtin_amdgcn_readlane(e0, 0);
  const int32_t last = __builtin_amdgcn_readlane(e1, nv > 0 ? nv - 1 : 0);
  const int32_t e0_next = __shfl_down(e0, 1, 64);
  const bool breaks = (lane < nv - 1 && e1 != e0_next) || (r < n_rows && !mine);
  const bool staged = nv > 0 && __ballot(breaks) == 0ull && last - first <= kStage;
  bool bad = false;
  if (mine) {
    if (staged)
      bad = decode_row_thread(e0, e1, p0, p1, blocks, n_bytes, offsets, n_off, stage[wv], first);
    else
      bad = decode_row_thread(e0, e1, p0, p1, blocks, n_bytes, offsets, n_off, indices, 0);
  }
  __syncthreads();  // (the stage is the wave's own; every wave reaches this)
  if (staged) {
    typedef int32_t i32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
    typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
    const int32_t n = last - first;
    for (int32_t k = 4 * lane; k < n; k += 256) {
      if (k + 4 <= n) {
        *reinterpret_cast<i32x4_a4 *>(indices + first + k) =
            *reinterpret_cast<const i32x4 *>(&stage[wv][k]);
      } else {
        for (int32_t j = k; j < n; ++j) indices[first + j] = stage[wv][j];
      }
    }
  }
  // the wave's long rows, one at a time (never in a staged wave)
  for (uint64_t m = __ballot(r < n_rows && !mine); m != 0ull; m &= m - 1ull) {
    const int j = __builtin_ctzll(m);
    const bool b = decode_row_wave(__builtin_amdgcn_readlane(e0, j),
                                   __builtin_amdgcn_readlane(e1, j),
                                   __builtin_amdgcn_readlane(p0, j),
                                   __builtin_amdgcn_readlane(p1, j), blocks, offsets, indices);
    if (lane == 0) bad = bad || b;
  }
  if (__ballot(bad) && lane == 0 && status != nullptr) atomicOr(status, 1);
}

hipError_t launch_bsc_row_bytes(int64_t n_rows, int64_t nnz, const int32_t *indptr,
                                const int32_t *indices, int32_t *bptr, hipStream_t s) {
  hipError_t e = launch_fill_i32(bptr, 1, 0, s);
  if (e != hipSuccess || n_rows == 0) return e;
  const unsigned blocks = (unsigned)((n_rows + kRowsPerBlock - 1) / kRowsPerBlock);
  hipLaunchKernelGGL(bsc_encode_rows_kernel<false>, dim3(blocks), dim3(256), 0, s, n_rows, nnz,
                     indptr, indices, bptr, nullptr, (int64_t)0);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return launch_scan_inplace(bptr + 1, n_rows, s);
}

hipError_t launch_bsc_encode(int64_t n_rows, int64_t nnz, const int32_t *indptr,
                             const int32_t *indices, const int32_t *bptr, uint8_t *blocks,
                             int64_t block_bytes, uint32_t *offset_words, int64_t n_words,
                             hipStream_t s) {
  hipError_t e;
  if (n_rows > 0) {
    const unsigned nb = (unsigned)((n_rows + kRowsPerBlock - 1) / kRowsPerBlock);
    hipLaunchKernelGGL(bsc_encode_rows_kernel<true>, dim3(nb), dim3(256), 0, s, n_rows, nnz,
                       indptr, indices, const_cast<int32_t *>(bptr), blocks, block_bytes);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (n_words > 0) {
    hipLaunchKernelGGL(bsc_pack_offsets_kernel, dim3((unsigned)((n_words + 255) / 256)),
                       dim3(256), 0, s, nnz, indices, offset_words, n_words);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_bsc_decode(int64_t n_rows, int64_t nnz, const int32_t *indptr,
                             const int32_t *bptr, int64_t n_bytes, const uint8_t *blocks,
                             const uint8_t *offsets, int32_t *indices, int32_t *status,
                             hipStream_t s) {
  if (n_rows == 0) return hipSuccess;
  const unsigned nb = (unsigned)((n_rows + 255) / 256);
  hipLaunchKernelGGL(bsc_decode_kernel, dim3(nb), dim3(256), 0, s, n_rows, nnz, indptr, bptr,
                     n_bytes, blocks, offsets, indices, status);
  return hipGetLastError();
}

}  // namespace sps
