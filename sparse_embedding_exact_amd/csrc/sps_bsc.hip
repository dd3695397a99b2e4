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
// All kernels are wave64 with one wave per row: the lanes of a wave take 64
// consecutive entries (encode) or bytes (decode) of the row at a time, so
// every load and store of a row is contiguous. Every access is bounded by
// the buffer sizes the host passes, whatever the contents.
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

// Column indices from the varint bytes and the offsets, kDecRows rows per
// wave. The rows' bounds come with one load, and the first 64 varint bytes
// and 64 offset bytes of every row are loaded together before any row is
// decoded, so a wave waits for two dependent loads per kDecRows rows rather
// than three per row. Lane i of a 64-byte window takes byte i: the ballot of
// "last byte of a value" flags gives each byte its value (the number of
// value ends before it) and its place in that value; a wave scan of
// (byte & 0x7f) << 7 place, carried across windows, is at every value's last
// byte the running sum of the differences, i.e. that entry's block id. Its
// 10-bit offset is taken from the row's offset window by lane shuffles (or
// loaded, past the window).
constexpr int kDecRows = 4;
__global__ __launch_bounds__(256) void bsc_decode_kernel(int64_t n_rows, int64_t nnz,
                                                         const int32_t *__restrict__ indptr,
                                                         const int32_t *__restrict__ bptr,
                                                         int64_t n_bytes,
                                                         const uint8_t *__restrict__ blocks,
                                                         const uint8_t *__restrict__ offsets,
                                                         int32_t *__restrict__ indices,
                                                         int32_t *__restrict__ status) {
  const int lane = threadIdx.x & 63;
  const int64_t rbase = ((int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6)) * kDecRows;
  if (rbase >= n_rows) return;  // uniform per wave
  // lanes 0 .. kDecRows: the row pointers of rows rbase .. rbase + kDecRows
  const int64_t rl = rbase + lane < n_rows ? rbase + lane : n_rows;
  const int32_t ipl = lane <= kDecRows ? indptr[rl] : 0;
  const int32_t bpl = lane <= kDecRows ? bptr[rl] : 0;
  int64_t e0[kDecRows], e1[kDecRows], p0[kDecRows], p1[kDecRows], ob0[kDecRows];
  uint32_t wb[kDecRows], wo[kDecRows];
#pragma unroll
  for (int j = 0; j < kDecRows; ++j) {
    const bool row_ok = rbase + j < n_rows;
    const int64_t a = clamp64(__builtin_amdgcn_readlane(ipl, j), 0, nnz);
    const int64_t c = clamp64(__builtin_amdgcn_readlane(ipl, j + 1), a, nnz);
    const int64_t pa = clamp64(__builtin_amdgcn_readlane(bpl, j), 0, n_bytes);
    const int64_t pc = clamp64(__builtin_amdgcn_readlane(bpl, j + 1), pa, n_bytes);
    e0[j] = a;
    e1[j] = row_ok ? c : a;
    p0[j] = pa;
    p1[j] = row_ok ? pc : pa;
    ob0[j] = (10 * e0[j]) >> 3;
    const int64_t ob1 = (10 * e1[j] + 7) >> 3;  // <= ceil(10 nnz / 8)
    wb[j] = p0[j] + lane < p1[j] ? (uint32_t)blocks[p0[j] + lane] : 0u;
    wo[j] = ob0[j] + lane < ob1 ? (uint32_t)offsets[ob0[j] + lane] : 0u;
  }
  const uint64_t lt = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  bool bad = false;
#pragma unroll
  for (int j = 0; j < kDecRows; ++j) {
    const int64_t ne = e1[j] - e0[j];
    uint32_t carry = 0;  // sum of all contributions of the earlier windows
    int64_t got = 0;     // values ended in the earlier windows
    int place0 = 0;      // bytes of an unfinished value before this window
    for (int64_t w0 = p0[j]; w0 < p1[j]; w0 += 64) {
      const int64_t i = w0 + lane;
      const bool valid = i < p1[j];
      const uint32_t b = w0 == p0[j] ? wb[j] : (valid ? (uint32_t)blocks[i] : 0u);
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
      const int64_t e = e0[j] + k;
      const int64_t bit = 10 * e;
      const int64_t rel = (bit >> 3) - ob0[j];
      const int src = rel >= 0 && rel < 63 ? (int)rel : 0;
      const uint32_t lo_w = (uint32_t)__shfl((int)wo[j], src, 64);
      const uint32_t hi_w = (uint32_t)__shfl((int)wo[j], src + 1, 64);
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
    if (p1[j] > p0[j] && (blocks[p1[j] - 1] & 0x80u)) bad = true;  // the row ends inside a value
    if (got != ne) bad = true;
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
  const int64_t per_block = (int64_t)kRowsPerBlock * kDecRows;
  const unsigned nb = (unsigned)((n_rows + per_block - 1) / per_block);
  hipLaunchKernelGGL(bsc_decode_kernel, dim3(nb), dim3(256), 0, s, n_rows, nnz, indptr, bptr,
                     n_bytes, blocks, offsets, indices, status);
  return hipGetLastError();
}

}  // namespace sps
