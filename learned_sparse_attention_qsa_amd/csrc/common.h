// Device-side helpers shared by the QSA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qsa {

constexpr int kIdxHeads = 4;
constexpr int kIdxDim = 64;
constexpr int kBlock = 4;
constexpr int kTopK = 512;
constexpr int kHeadDim = 128;
constexpr int kMaxTok = kTopK * kBlock + kBlock;  // 2052
constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

__device__ __forceinline__ uint4 zero_u4() { return make_uint4(0u, 0u, 0u, 0u); }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bf16, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// float64 -> bf16 with a single rounding to nearest even.  The double is first
// narrowed to float with round-to-odd (truncate, then set the last bit when
// inexact); with 16 spare bits that makes the second rounding exact.
__device__ __forceinline__ uint32_t f64_to_bf16(double d) {
  float f = (float)d;
  double back = (double)f;
  uint32_t u = __float_as_uint(f);
  if (back != d && !__builtin_isnan(d)) {
    if (__builtin_fabs(back) > __builtin_fabs(d)) u -= 1u;  // undo rounding away from zero
    u |= 1u;
  }
  return f32_to_bf16(__uint_as_float(u));
}

// One 16-byte chunk (8 dims) of a compressed block key: the same chunk of
// the block's four token keys (rows[0], rows[8], rows[16], rows[24]: rows of
// 64 bf16 are 8 chunks apart) summed in float64 in token order, which is
// exact for any bf16 inputs of sane range, then rounded once to bf16.
__device__ __forceinline__ uint4 compress_chunk(const uint4* rows) {
  const uint4 r[4] = {rows[0], rows[8], rows[16], rows[24]};
  double s[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const uint32_t x[4] = {r[t].x, r[t].y, r[t].z, r[t].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s[2 * i] += (double)bf16_lo(x[i]);
      s[2 * i + 1] += (double)bf16_hi(x[i]);
    }
  }
  uint4 o;
  o.x = f64_to_bf16(s[0]) | (f64_to_bf16(s[1]) << 16);
  o.y = f64_to_bf16(s[2]) | (f64_to_bf16(s[3]) << 16);
  o.z = f64_to_bf16(s[4]) | (f64_to_bf16(s[5]) << 16);
  o.w = f64_to_bf16(s[6]) | (f64_to_bf16(s[7]) << 16);
  return o;
}

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// ---- guards on caller-supplied values
// A length outside [Nq, Lmax], a selected block outside [0, bt), a selection
// count other than min(bt, 512), a page id outside the pool or a first block
// past the completed ones is a caller bug.  Kernels clamp such values so that
// no access leaves its buffer.  Builds with QSA_DEBUG also count every value
// a guard caught, in a device counter per source file that the library's
// qsa_debug_guard_hits() collects and clears.
#ifdef QSA_DEBUG
namespace {
__device__ unsigned int g_guard_hits;
}
__device__ __forceinline__ void guard_hit() { atomicAdd(&g_guard_hits, 1u); }
void register_guard_counter(hipError_t (*read_and_clear)(unsigned int*));
namespace {
hipError_t read_and_clear_guard_hits(unsigned int* out) {
  hipError_t e = hipMemcpyFromSymbol(out, HIP_SYMBOL(g_guard_hits), sizeof(unsigned int));
  if (e != hipSuccess) return e;
  const unsigned int zero = 0u;
  return hipMemcpyToSymbol(HIP_SYMBOL(g_guard_hits), &zero, sizeof(unsigned int));
}
const bool g_guard_registered = (register_guard_counter(&read_and_clear_guard_hits), true);
}  // namespace
#else
__device__ __forceinline__ void guard_hit() {}
#endif

// x clamped to [lo, hi]; a value outside is a caught caller bug.
__device__ __forceinline__ int guard(int x, int lo, int hi) {
  const int c = clampi(x, lo, hi);
#ifdef QSA_DEBUG
  if (c != x) guard_hit();
#endif
  return c;
}

// A sequence length: clamped to [0, Lmax]; outside [Nq, Lmax] is caught.
__device__ __forceinline__ int guard_len(int x, int Nq, int Lmax) {
#ifdef QSA_DEBUG
  if (x < Nq || x > Lmax) guard_hit();
#else
  (void)Nq;
#endif
  return clampi(x, 0, Lmax);
}

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63u); }

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int l = lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// 64-bit selection key: larger is better.  Score bits (non-negative float, so
// the unsigned order of the bits is the numeric order) in the high word, the
// complement of the block id in the low word, so equal scores prefer the
// lower block id and all keys of one query are distinct.
__device__ __forceinline__ uint64_t make_key(uint32_t score_bits, uint32_t j) {
  return ((uint64_t)score_bits << 32) | (uint64_t)(0xffffffffu - j);
}
__device__ __forceinline__ uint32_t key_block(uint64_t key) { return 0xffffffffu - (uint32_t)key; }

// max(0, x) for a non-NaN float as one integer max on its bit pattern: a
// set sign bit reads as a negative int, so every negative value and -0
// become +0.  (fmaxf would first quiet possible NaNs, doubling the cost.)
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// Sum over the four indexer heads of max(0, x); the result is +0 or positive,
// so its bit pattern orders like its value.
__device__ __forceinline__ float relu_sum(float a, float b, float c, float d) {
  return (relu(a) + relu(b)) + (relu(c) + relu(d));
}
__device__ __forceinline__ uint32_t relu_sum_bits(float a, float b, float c, float d) {
  return __float_as_uint(relu_sum(a, b, c, d)) & 0x7fffffffu;
}

}  // namespace qsa
