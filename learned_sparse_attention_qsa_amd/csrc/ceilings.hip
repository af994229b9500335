// Memory-system ceilings of the part, measured with the access patterns of the
// QSA path (not part of the method): a cold streaming read of a buffer the
// size of one decode step's compressed-key scan, and random gathers of the
// pieces the sparse attention reads (one KV head's 256-byte K or V row, one
// token's 1 KiB row of all four KV heads, one micro-block's 4 KiB of four
// consecutive token rows).  The kernels only read; each folds what it read
// into one word so the loads cannot be dropped.  A last probe times LDS
// atomic adds by how many lanes share an address, 32-bit integer and float32.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qsa_ceilings.h"
#include "internal.h"

namespace qsa {
namespace {

// Workgroup w reads the w-th of gridDim.x equal contiguous pieces, eight
// 16-byte loads per thread in flight.
__global__ __launch_bounds__(512) void ceil_stream_kernel(const uint4* __restrict__ p, size_t n16,
                                                          uint32_t* __restrict__ sink) {
  constexpr int U = 8;
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t b0 = (size_t)blockIdx.x * per;
  const size_t b1 = b0 + per < n16 ? b0 + per : n16;
  uint32_t acc = 0;
  for (size_t i = b0 + threadIdx.x; i < b1; i += (size_t)blockDim.x * U) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t k = i + (size_t)u * blockDim.x;
      v[u] = k < b1 ? p[k] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;  // practically never: keeps the loads
}

// Piece i is row_bytes bytes at byte offset off[i] * row_bytes of base.
// A group of row_bytes / 16 lanes reads one piece; each thread has four
// pieces in flight.
__global__ __launch_bounds__(256) void ceil_gather_kernel(const uint4* __restrict__ base,
                                                          const int64_t* __restrict__ off,
                                                          int64_t n_pieces, int row16,
                                                          uint32_t* __restrict__ sink) {
  constexpr int U = 4;
  const int lanes = row16 < (int)blockDim.x ? row16 : (int)blockDim.x;
  const int per_pass = (int)blockDim.x / lanes;    // pieces one pass of the workgroup covers
  const int sub = (int)threadIdx.x / lanes, l = (int)threadIdx.x % lanes;
  const int chunks = row16 / lanes;                // 16-byte loads per lane per piece
  uint32_t acc = 0;
  for (int64_t p0 = (int64_t)blockIdx.x * per_pass * U; p0 < n_pieces;
       p0 += (int64_t)gridDim.x * per_pass * U) {
    for (int c = 0; c < chunks; ++c) {
      uint4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t pi = p0 + (int64_t)u * per_pass + sub;
        v[u] = pi < n_pieces ? base[off[pi] * row16 + (int64_t)c * lanes + l]
                             : make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

// Every thread adds 1 iters times to the LDS word of its address group
// (lane / share, rotated by 64 words per step), 32-bit integer or float32.
template <typename T>
__global__ __launch_bounds__(256) void ceil_lds_atomic_kernel(int share, int iters,
                                                              uint32_t* __restrict__ sink) {
  __shared__ T h[1024];
  for (int i = threadIdx.x; i < 1024; i += blockDim.x) h[i] = (T)0;
  __syncthreads();
  const int a = ((int)threadIdx.x >> 6) * 64 + ((int)threadIdx.x & 63) / share;
  for (int i = 0; i < iters; ++i) atomicAdd(&h[(a + i * 64) & 1023], (T)1);
  __syncthreads();
  if (threadIdx.x == 0 && h[0] == (T)-1) sink[blockIdx.x] = 1u;  // practically never
}

}  // namespace
}  // namespace qsa

extern "C" {

qsa_status qsa_ceil_stream_read(const void* buf, size_t bytes, int32_t workgroups, uint32_t* sink,
                                void* stream) {
  if (!buf || !sink) return QSA_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(buf) & 15u) != 0 || (bytes & 15u) != 0) return QSA_ERR_ALIGN;
  if (workgroups < 1 || workgroups > (1 << 20)) return QSA_ERR_SHAPE;
  if (bytes == 0) return QSA_OK;
  QSA_LAUNCH(qsa::ceil_stream_kernel, dim3((unsigned)workgroups), dim3(512), 0,
             static_cast<hipStream_t>(stream), static_cast<const uint4*>(buf), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? QSA_OK : QSA_ERR_HIP;
}

qsa_status qsa_ceil_gather(const void* base, const int64_t* row_index, int64_t n_rows,
                           int32_t row_bytes, int32_t workgroups, uint32_t* sink, void* stream) {
  if (!base || !row_index || !sink) return QSA_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(base) & 15u) != 0 ||
      (reinterpret_cast<uintptr_t>(row_index) & 7u) != 0)
    return QSA_ERR_ALIGN;
  if (row_bytes < 16 || row_bytes > 16384 || (row_bytes & (row_bytes - 1)) != 0 || n_rows < 0 ||
      workgroups < 1 || workgroups > (1 << 20))
    return QSA_ERR_SHAPE;
  if (n_rows == 0) return QSA_OK;
  QSA_LAUNCH(qsa::ceil_gather_kernel, dim3((unsigned)workgroups), dim3(256), 0,
             static_cast<hipStream_t>(stream), static_cast<const uint4*>(base), row_index, n_rows,
             row_bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? QSA_OK : QSA_ERR_HIP;
}

qsa_status qsa_ceil_lds_atomic(int32_t f32, int32_t share, int32_t workgroups, int32_t iters,
                               uint32_t* sink, void* stream) {
  if (!sink) return QSA_ERR_NULL;
  if ((f32 != 0 && f32 != 1) || (share != 1 && share != 2 && share != 4 && share != 16 &&
                                 share != 64) ||
      workgroups < 1 || workgroups > (1 << 20) || iters < 1 || iters > 4096)
    return QSA_ERR_SHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (f32)
    QSA_LAUNCH(qsa::ceil_lds_atomic_kernel<float>, dim3((unsigned)workgroups), dim3(256), 0, s,
               share, iters, sink);
  else
    QSA_LAUNCH(qsa::ceil_lds_atomic_kernel<uint32_t>, dim3((unsigned)workgroups), dim3(256), 0, s,
               share, iters, sink);
  return hipGetLastError() == hipSuccess ? QSA_OK : QSA_ERR_HIP;
}

}  // extern "C"
