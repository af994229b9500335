// Key compression: one micro-block key per four indexer keys.
//
// Method: the indexer compresses keys four at a time (page "Qwen's
// million-token window has a 2,048-token keyhole", section "A million-token
// window with a selective view").  The operator is not printed; the block key
// is the sum of its four token keys, formed exactly and rounded once to bf16.
//
// HBM-bound streaming pass: each thread owns one 16-byte chunk (8 dims) of
// one block and reads the four 128-byte rows of that block at that chunk, so
// a wavefront reads 8 whole blocks (4 KiB) with every load fully coalesced and
// writes 8 whole compressed rows (1 KiB).  Sums are taken in float64 in row
// order, which is exact for any bf16 inputs of sane range, and narrowed with
// one round-to-nearest-even.
#include "common.h"
#include "internal.h"

namespace qsa {
namespace {

__global__ __launch_bounds__(256) void compress_kernel(const uint16_t* __restrict__ k_idx,
                                                       const int32_t* __restrict__ lens,
                                                       const int32_t* __restrict__ first_block,
                                                       uint16_t* __restrict__ k_cmp, int Lmax) {
  const int b = blockIdx.y;
  const int len = guard(lens[b], 0, Lmax);
  const int nb = len >> 2;
  const int fb = first_block ? guard(first_block[b], 0, nb) : 0;
  const size_t nbp = (size_t)(Lmax >> 2);
  const uint4* src = reinterpret_cast<const uint4*>(k_idx + (size_t)b * Lmax * kIdxDim);
  uint4* dst = reinterpret_cast<uint4*>(k_cmp + (size_t)b * nbp * kIdxDim);
  const long long end = (long long)nb * 8;
  const long long stride = (long long)gridDim.x * blockDim.x;
  for (long long g = (long long)fb * 8 + (long long)blockIdx.x * blockDim.x + threadIdx.x;
       g < end; g += stride) {
    const long long j = g >> 3;
    const int c = (int)(g & 7);
    // row 4j at chunk c; rows are 8 uint4 apart
    const uint4 o = compress_chunk(src + j * 32 + c);
    dst[j * 8 + c] = o;
  }
}

}  // namespace

hipError_t launch_compress(const Dims& d, const uint16_t* k_idx, const int32_t* lens,
                           const int32_t* first_block, uint16_t* k_cmp, hipStream_t s) {
  if (d.B == 0) return hipSuccess;
  // Grid-stride: enough workgroups to keep HBM busy on a full rebuild, few
  // enough that an incremental call (one new block per sequence) is cheap.
  const long long chunks = (long long)(d.Lmax / 4) * 8;
  long long wg = (chunks + 255) / 256;
  const long long cap = first_block ? 256 : 2048;
  if (wg > cap) wg = cap;
  if (wg < 1) wg = 1;
  QSA_LAUNCH(compress_kernel, dim3((unsigned)wg, (unsigned)d.B), dim3(256), 0, s, k_idx,
                     lens, first_block, k_cmp, d.Lmax);
  return hipGetLastError();
}

}  // namespace qsa
