// sf_layout.hip -- block-scale bytes rewritten from one layout into another
// (LINEAR, TILED, 128 x 4; sf_offset in common.hpp defines all three).
//
// HBM-bound copy: one thread per 4-byte word of the destination, which it
// writes whole (padding included); its four bytes are gathered from the
// source through the source layout's offset.  Consecutive threads write
// consecutive words, so the stores are coalesced; the gathers of a wave stay
// inside a few source tiles or rows and are served from L2.
#include <stdint.h>

#include "common.hpp"
#include "launch.hpp"

namespace lowbit {
namespace {

constexpr int kRelayoutThreads = 256;

// Thread t writes destination bytes [4t, 4t + 4): byte i holds row[i], block
// kb[i] of the operand, or padding (row >= rows or kb >= nblk), written zero.
template <int LS, int LD>
__global__ __launch_bounds__(kRelayoutThreads) void sf_relayout_kernel(const uint8_t* __restrict__ src,
                                                                        uint8_t* __restrict__ dst, int fmt,
                                                                        int64_t rows, int64_t nblk,
                                                                        int64_t total, int word_store) {
  const int64_t off = (int64_t(blockIdx.x) * kRelayoutThreads + threadIdx.x) * 4;
  if (off >= total) return;
  int64_t row[4], kb[4];
  if constexpr (LD == kLinear) {
    // row-major: the four bytes may run over the end of a row (nblk < 4 too)
    int64_t r = off / nblk, c = off - r * nblk;
    for (int i = 0; i < 4; ++i) {
      row[i] = r;
      kb[i] = c;
      if (++c == nblk) { c = 0; ++r; }
    }
  } else if constexpr (LD == kSwz128) {
    // 512-byte tiles of 128 rows x 4 blocks; a word is one row's 4 blocks
    const int64_t tiles_k = (nblk + 3) >> 2, tile = off >> 9, rt = tile / tiles_k;
    const int in = int(off & 511);
    const int64_t r = (rt << 7) + (((in >> 2) & 3) << 5) + (in >> 4);
    for (int i = 0; i < 4; ++i) {
      row[i] = r;
      kb[i] = ((tile - rt * tiles_k) << 2) + i;
    }
  } else {
    // 256-byte groups of 32 rows x 8 blocks; word h*32 + r is row r's half h,
    // its bytes ordered per format as sf_offset places them
    const int64_t ktiles = (nblk + 7) >> 3, grp = off >> 8, rg = grp / ktiles;
    const int word = int(off & 255) >> 2, h = word >> 5;
    const int64_t r = (rg << 5) + (word & 31), k0 = (grp - rg * ktiles) << 3;
    for (int i = 0; i < 4; ++i) {
      row[i] = r;
      kb[i] = k0 + (fmt == kNVFP4 ? 4 * h + i : 4 * (i >> 1) + 2 * h + (i & 1));
    }
  }
  uint32_t w = 0;
  for (int i = 0; i < 4; ++i) {
    const bool held = off + i < total && row[i] < rows && kb[i] < nblk;
    const uint32_t b = held ? uint32_t(src[sf_offset(fmt, LS, row[i], kb[i], nblk)]) : 0u;
    w |= b << (8 * i);
  }
  if (word_store && off + 4 <= total) {
    *reinterpret_cast<uint32_t*>(dst + off) = w;
  } else {
    for (int i = 0; i < 4; ++i)
      if (off + i < total) dst[off + i] = uint8_t(w >> (8 * i));
  }
}

template <int LS>
hipError_t relayout_from(const uint8_t* src, uint8_t* dst, int ld, int fmt, int64_t rows, int64_t nblk,
                         int64_t total, unsigned grid, int word_store, hipStream_t s) {
  if (ld == kLinear)
    hipLaunchKernelGGL((sf_relayout_kernel<LS, kLinear>), dim3(grid), dim3(kRelayoutThreads), 0, s, src, dst,
                       fmt, rows, nblk, total, word_store);
  else if (ld == kTiled)
    hipLaunchKernelGGL((sf_relayout_kernel<LS, kTiled>), dim3(grid), dim3(kRelayoutThreads), 0, s, src, dst,
                       fmt, rows, nblk, total, word_store);
  else
    hipLaunchKernelGGL((sf_relayout_kernel<LS, kSwz128>), dim3(grid), dim3(kRelayoutThreads), 0, s, src, dst,
                       fmt, rows, nblk, total, word_store);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_sf_relayout(const uint8_t* src, int ls, uint8_t* dst, int ld, int64_t rows, int64_t nblk,
                              int fmt, hipStream_t s) {
  const int64_t total = sf_bytes_of(ld, rows, nblk);
  if (total <= 0) return hipSuccess;
  if (total > kRelayoutMaxBytes) return hipErrorInvalidValue;
  const unsigned grid = unsigned((total + 4 * kRelayoutThreads - 1) / (4 * kRelayoutThreads));
  const int word_store = (reinterpret_cast<uintptr_t>(dst) & 3) == 0;
  if (ls == kLinear) return relayout_from<kLinear>(src, dst, ld, fmt, rows, nblk, total, grid, word_store, s);
  if (ls == kTiled) return relayout_from<kTiled>(src, dst, ld, fmt, rows, nblk, total, grid, word_store, s);
  return relayout_from<kSwz128>(src, dst, ld, fmt, rows, nblk, total, grid, word_store, s);
}

}  // namespace lowbit
