// Indexer scoring and top-k selection.
//
// Method (page "Qwen's million-token window has a 2,048-token keyhole"):
// the indexer has four query heads and one shared key head, scores the
// compressed blocks and ranks them (section "A million-token window with a
// selective view"); each query keeps at most 512 micro-blocks (opening
// section).  Readings: score s_j = sum_h max(0, q_h . k_cmp[j]); candidates
// are the completed blocks j < bt = floor(t/4); ties go to the lower block id.
//
// Selection order.  A candidate is the 64-bit key (score bits << 32 | ~j):
// scores are non-negative floats (so their bit patterns order like their
// values) and the complemented id makes every key of a query distinct, with
// equal scores preferring lower ids.  The selection is the 512 largest keys.
//
// Two engines, with bit-identical results:
//
//  TABLE (few queries, decode-shaped): one streaming pass scores every block
//  with MFMA (16x16x32, 4 queries x 4 heads per tile), writes the fp32 score
//  table and a per-query 2048-bin histogram of the score's top bits.  A
//  second pass picks, from the histogram, the highest bin whose cumulative
//  count from the top reaches 512 and appends every key in or above it to a
//  candidate list (its size is known from the histogram).  A select kernel
//  then finds the exact 512th key in LDS.  Cost over the bare k_cmp scan: the
//  score table (4 B per query per block) written once and read once.
//
//  STREAM (many queries, prefill-shaped): a workgroup holds 64 queries x 4
//  heads stationary in registers and streams the compressed keys through LDS
//  in tiles of 64 blocks, MFMA 32x32x16.  Each query keeps a threshold tau =
//  score of the 512th best key seen so far; because blocks arrive in
//  ascending id order, a new block can only enter the top 512 if its score
//  is strictly greater than tau (an equal score loses the tie to an earlier
//  block).  Survivors are appended to a per-query list in HBM; when a list
//  nears its capacity the owning wavefront selects its top 512 in place and
//  raises tau.  No score table is written.
//
// Both engines finish with the same LDS radix select; rows the fast path
// cannot hold (extreme ties in the table engine) are finished by an exact
// fallback that recomputes or re-reads the whole row.
#include "common.h"
#include "internal.h"

namespace qsa {
namespace {

constexpr int kHistBins = 2048;    // table engine: bins of (score bits >> 20)
constexpr int kTableSlice = 2048;  // blocks per table-engine workgroup
constexpr int kSelCap = 8192;      // candidates a select workgroup holds in LDS
constexpr int kListCap = 2048;     // stream engine: list capacity per query
constexpr int kStreamTile = 64;    // blocks per key tile (stream engine)
constexpr int kStreamQ = 64;       // queries per stream workgroup (16 per wavefront)
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// One wavefront: given a 256-bin histogram h (bin = digit) and a rank k >= 1
// counted from the largest digit, find the digit holding the k-th largest
// element and the number of elements in strictly larger digits.  The caller
// guarantees sum(h) >= k.
__device__ __forceinline__ void wave_find_digit(const uint32_t* h, uint32_t k, uint32_t& digit,
                                                uint32_t& above) {
  const int l = lane_id();
  const uint32_t c0 = h[4 * l], c1 = h[4 * l + 1], c2 = h[4 * l + 2], c3 = h[4 * l + 3];
  const uint32_t mine = c0 + c1 + c2 + c3;
  uint32_t S = mine;  // inclusive suffix sum over lanes
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t o = __shfl_down(S, off);
    if (l + off < 64) S += o;
  }
  const uint64_t m = __ballot(S >= k);
  const int L = 63 - __clzll((long long)m);
  uint32_t cum = __shfl(S, L) - __shfl(mine, L);
  const uint32_t b3 = __shfl(c3, L), b2 = __shfl(c2, L), b1 = __shfl(c1, L);
  uint32_t d;
  if (cum + b3 >= k) {
    d = 3;
  } else {
    cum += b3;
    if (cum + b2 >= k) {
      d = 2;
    } else {
      cum += b2;
      if (cum + b1 >= k) {
        d = 1;
      } else {
        cum += b1;
        d = 0;
      }
    }
  }
  digit = 4u * (uint32_t)L + d;
  above = cum;
}

// Whole workgroup (blockDim.x threads): the k-th largest of n distinct keys in
// LDS, by most-significant-digit radix select over eight 8-bit digits.
__device__ uint64_t block_kth_largest(const uint64_t* keys, int n, uint32_t k, uint32_t* hist,
                                      uint32_t* bcast) {
  uint64_t prefix = 0, pmask = 0;
  const int tid = threadIdx.x;
  for (int shift = 56; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += blockDim.x) hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += blockDim.x) {
      const uint64_t key = keys[i];
      if ((key & pmask) == prefix) atomicAdd(&hist[(uint32_t)(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      uint32_t d, above;
      wave_find_digit(hist, k, d, above);
      if (tid == 0) {
        bcast[0] = d;
        bcast[1] = above;
      }
    }
    __syncthreads();
    k -= bcast[1];
    prefix |= (uint64_t)bcast[0] << shift;
    pmask |= 0xffull << shift;
  }
  return prefix;
}

// 512 ints in LDS, ascending; needs exactly 256 threads.
__device__ void bitonic_sort_512(int32_t* a) {
  const int tid = threadIdx.x;
  for (int k = 2; k <= 512; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      const int i = ((tid & ~(j - 1)) << 1) | (tid & (j - 1));
      const int p = i | j;
      const bool up = (i & k) == 0;
      const int32_t x = a[i], y = a[p];
      if ((x > y) == up) {
        a[i] = y;
        a[p] = x;
      }
      __syncthreads();
    }
  }
}

__device__ __forceinline__ int query_t(int len, int Nq, int q) { return len - Nq + q; }

// Rows whose candidates all fit the budget: keep every block.
__device__ __forceinline__ bool write_trivial(int t, int32_t* srow, int32_t* n_sel_row) {
  if (t >= 0 && (t >> 2) > kTopK) return false;
  const int bt = t < 0 ? 0 : (t >> 2);
  for (int i = threadIdx.x; i < kTopK; i += blockDim.x) srow[i] = i < bt ? i : -1;
  if (threadIdx.x == 0) *n_sel_row = bt;
  return true;
}

__global__ void fill_u32_kernel(uint32_t* p, size_t n, uint32_t v) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = v;
}

// ------------------------------------------------------------------ select
// One workgroup per query: exact top-512 of the candidate list of the row.
__global__ __launch_bounds__(256) void select_kernel(const uint64_t* __restrict__ cand,
                                                     const uint32_t* __restrict__ cand_cnt,
                                                     const int32_t* __restrict__ lens,
                                                     int32_t* __restrict__ sel,
                                                     int32_t* __restrict__ n_sel,
                                                     uint32_t* __restrict__ overflow, int Lmax,
                                                     int Nq, int cap) {
  __shared__ uint64_t keys[kSelCap];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t bcast[2];
  __shared__ int32_t outb[kTopK];
  __shared__ uint32_t outn;
  const int q = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const size_t row = (size_t)b * Nq + q;
  const int t = query_t(clampi(lens[b], 0, Lmax), Nq, q);
  int32_t* srow = sel + row * kTopK;
  if (write_trivial(t, srow, n_sel + row)) {
    if (tid == 0) overflow[row] = 0;
    return;
  }
  const uint32_t n = cand_cnt[row];
  if (n > (uint32_t)cap || n > (uint32_t)kSelCap || n < (uint32_t)kTopK) {
    if (tid == 0) overflow[row] = 1;
    return;
  }
  if (tid == 0) {
    overflow[row] = 0;
    outn = 0;
  }
  const uint64_t* src = cand + row * (size_t)cap;
  for (uint32_t i = tid; i < n; i += blockDim.x) keys[i] = src[i];
  __syncthreads();
  const uint64_t kth = block_kth_largest(keys, (int)n, kTopK, hist, bcast);
  for (uint32_t i = tid; i < n; i += blockDim.x) {
    const uint64_t key = keys[i];
    if (key >= kth) outb[atomicAdd(&outn, 1u)] = (int32_t)key_block(key);
  }
  __syncthreads();
  bitonic_sort_512(outb);
  for (int i = tid; i < kTopK; i += blockDim.x) srow[i] = outb[i];
  if (tid == 0) n_sel[row] = kTopK;
}

// ------------------------------------------------------------------ fallback
// Exact top-512 straight from the whole row, for rows flagged by select_kernel.
// kRecompute: recompute scores from q_idx / k_cmp (stream engine, no table);
// otherwise read the score table.  Output comes out in ascending order because
// the final pass walks the blocks in order.
template <bool kRecompute>
__global__ __launch_bounds__(256) void select_fallback_kernel(
    const uint32_t* __restrict__ table, const uint16_t* __restrict__ q_idx,
    const uint16_t* __restrict__ k_cmp, const int32_t* __restrict__ lens,
    const uint32_t* __restrict__ overflow, int32_t* __restrict__ sel, int32_t* __restrict__ n_sel,
    int Lmax, int Nq) {
  __shared__ float qf[kIdxHeads * kIdxDim];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t bcast[2];
  __shared__ uint32_t wsum[4];
  const int q = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const size_t row = (size_t)b * Nq + q;
  if (overflow[row] == 0) return;
  const int nbp = Lmax >> 2;
  const int t = query_t(clampi(lens[b], 0, Lmax), Nq, q);
  const int bt = t >> 2;  // > 512, guaranteed by the flag
  const uint32_t* trow = table + row * (size_t)nbp;
  const uint16_t* kc = k_cmp + (size_t)b * nbp * kIdxDim;
  if (kRecompute) {
    for (int i = tid; i < kIdxHeads * kIdxDim; i += blockDim.x)
      qf[i] = __uint_as_float((uint32_t)q_idx[row * kIdxHeads * kIdxDim + i] << 16);
    __syncthreads();
  }
  auto key_of = [&](int j) -> uint64_t {
    uint32_t bits;
    if (kRecompute) {
      float d[4] = {0.f, 0.f, 0.f, 0.f};
      const uint16_t* kr = kc + (size_t)j * kIdxDim;
      for (int e = 0; e < kIdxDim; ++e) {
        const float kv = __uint_as_float((uint32_t)kr[e] << 16);
#pragma unroll
        for (int h = 0; h < 4; ++h) d[h] = fmaf(qf[h * kIdxDim + e], kv, d[h]);
      }
      bits = relu_sum_bits(d[0], d[1], d[2], d[3]);
    } else {
      bits = trow[j];
    }
    return make_key(bits, (uint32_t)j);
  };
  uint64_t prefix = 0, pmask = 0;
  uint32_t k = kTopK;
  for (int shift = 56; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += blockDim.x) hist[i] = 0;
    __syncthreads();
    for (int j = tid; j < bt; j += blockDim.x) {
      const uint64_t key = key_of(j);
      if ((key & pmask) == prefix) atomicAdd(&hist[(uint32_t)(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      uint32_t d, above;
      wave_find_digit(hist, k, d, above);
      if (tid == 0) {
        bcast[0] = d;
        bcast[1] = above;
      }
    }
    __syncthreads();
    k -= bcast[1];
    prefix |= (uint64_t)bcast[0] << shift;
    pmask |= 0xffull << shift;
    __syncthreads();
  }
  const uint64_t kth = prefix;
  int32_t* srow = sel + row * kTopK;
  const int lane = lane_id(), wave = tid >> 6;
  uint32_t written = 0;
  for (int base = 0; base < bt; base += blockDim.x) {
    const int j = base + tid;
    const bool keep = j < bt && key_of(j) >= kth;
    const uint64_t m = __ballot(keep);
    if (lane == 0) wsum[wave] = (uint32_t)__popcll(m);
    __syncthreads();
    uint32_t off = written;
    for (int w = 0; w < wave; ++w) off += wsum[w];
    if (keep) srow[off + (uint32_t)__popcll(m & lanemask_lt())] = j;
    for (int w = 0; w < 4; ++w) written += wsum[w];
    __syncthreads();
  }
  if (tid == 0) n_sel[row] = kTopK;
}

// ------------------------------------------------------------------ TABLE
// Grid (slices, ceil(Nq/4), B); 4 wavefronts; each wavefront scores 4
// consecutive 16-block column tiles per step.
__global__ __launch_bounds__(256) void score_table_kernel(const uint16_t* __restrict__ q_idx,
                                                          const uint16_t* __restrict__ k_cmp,
                                                          const int32_t* __restrict__ lens,
                                                          uint32_t* __restrict__ scores,
                                                          uint32_t* __restrict__ ghist, int Lmax,
                                                          int Nq) {
  __shared__ uint32_t hist[4 * kHistBins];
  const int slice = blockIdx.x, q0 = blockIdx.y * 4, b = blockIdx.z;
  const int len = clampi(lens[b], 0, Lmax);
  const int nbp = Lmax >> 2;
  const int t_last = query_t(len, Nq, min(q0 + 3, Nq - 1));
  if (t_last < 4) return;
  const int j_begin = slice * kTableSlice;
  const int j_end = min(j_begin + kTableSlice, t_last >> 2);
  if (j_begin >= j_end) return;
  for (int i = threadIdx.x; i < 4 * kHistBins; i += blockDim.x) hist[i] = 0;

  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int r = lane & 15, kc = lane >> 4;
  // A operand: row r = (query r/4, head r%4); k chunk kc (dims kc*8.., 32+kc*8..)
  bf16x8 a0 = as_bf16x8(zero_u4()), a1 = a0;
  const int qa = q0 + (r >> 2);
  if (qa < Nq) {
    const uint4* p = reinterpret_cast<const uint4*>(
        q_idx + (((size_t)b * Nq + qa) * kIdxHeads + (r & 3)) * kIdxDim);
    a0 = as_bf16x8(p[kc]);
    a1 = as_bf16x8(p[4 + kc]);
  }
  // Output of the 16x16 tile: lane holds block column r for query q0+kc, all heads.
  const int qo = q0 + kc;
  const int t_o = query_t(len, Nq, qo);
  const int bt_o = (qo < Nq && t_o >= 0) ? (t_o >> 2) : 0;
  const int lim = min(bt_o, j_end);
  uint32_t* srow = scores + ((size_t)b * Nq + min(qo, Nq - 1)) * nbp;
  uint32_t* myhist = hist + kc * kHistBins;
  const uint4* kb = reinterpret_cast<const uint4*>(k_cmp + (size_t)b * nbp * kIdxDim);
  __syncthreads();

  constexpr int U = 4;
  for (int jt = j_begin + wave * 16 * U; jt < j_end; jt += 64 * U) {
    uint4 bv[U][2];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = jt + u * 16 + r;
      if (j < j_end) {
        bv[u][0] = kb[(size_t)j * 8 + kc];
        bv[u][1] = kb[(size_t)j * 8 + 4 + kc];
      } else {
        bv[u][0] = zero_u4();
        bv[u][1] = zero_u4();
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      acc = mfma16(a0, as_bf16x8(bv[u][0]), acc);
      acc = mfma16(a1, as_bf16x8(bv[u][1]), acc);
      const int jo = jt + u * 16 + r;
      if (jo < lim) {
        const uint32_t bits = relu_sum_bits(acc[0], acc[1], acc[2], acc[3]);
        srow[jo] = bits;
        atomicAdd(&myhist[bits >> 20], 1u);
      }
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 4 * kHistBins; i += blockDim.x) {
    const int qq = i / kHistBins;
    const uint32_t c = hist[i];
    if (c != 0 && q0 + qq < Nq)
      atomicAdd(&ghist[((size_t)b * Nq + q0 + qq) * kHistBins + (i % kHistBins)], c);
  }
}

// Same grid as score_table_kernel.  Appends the keys at or above each
// query's threshold bin to the query's candidate list.
__global__ __launch_bounds__(256) void table_filter_kernel(const uint32_t* __restrict__ scores,
                                                           const uint32_t* __restrict__ ghist,
                                                           const int32_t* __restrict__ lens,
                                                           uint64_t* __restrict__ cand,
                                                           uint32_t* __restrict__ cand_cnt,
                                                           int Lmax, int Nq, int cap) {
  __shared__ uint32_t bins[4][kHistBins];
  __shared__ int thr[4];
  const int slice = blockIdx.x, q0 = blockIdx.y * 4, b = blockIdx.z;
  const int len = clampi(lens[b], 0, Lmax);
  const int nbp = Lmax >> 2;
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int j_begin = slice * kTableSlice;
  {
    const int qq = q0 + wave;
    int m = -1;  // -1: nothing to append for this query
    const int t = query_t(len, Nq, qq);
    if (qq < Nq && t >= 0 && (t >> 2) > kTopK && j_begin < (t >> 2)) {
      const size_t row = (size_t)b * Nq + qq;
      const uint4* h4 = reinterpret_cast<const uint4*>(ghist + row * kHistBins);
      uint4* s4 = reinterpret_cast<uint4*>(bins[wave]);
      for (int i = lane; i < kHistBins / 4; i += 64) s4[i] = h4[i];
      wave_sync_lds();
      const uint32_t* hb = bins[wave] + lane * 32;
      uint32_t mine = 0;
      for (int i = 0; i < 32; ++i) mine += hb[i];
      uint32_t S = mine;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t o = __shfl_down(S, off);
        if (lane + off < 64) S += o;
      }
      const uint64_t msk = __ballot(S >= (uint32_t)kTopK);
      const int L = 63 - __clzll((long long)msk);
      uint32_t cum = __shfl(S, L) - __shfl(mine, L);
      int mb = 0;
      uint32_t total = 0;
      if (lane == L) {
        for (int i = 31; i >= 0; --i) {
          cum += hb[i];
          if (cum >= (uint32_t)kTopK) {
            mb = L * 32 + i;
            total = cum;
            break;
          }
        }
      }
      mb = __shfl(mb, L);
      total = __shfl(total, L);
      m = total <= (uint32_t)cap ? mb : -1;
    }
    if (lane == 0) thr[wave] = m;
  }
  __syncthreads();
  for (int qi = 0; qi < 4; ++qi) {
    const int m = thr[qi];
    if (m < 0) continue;
    const int qq = q0 + qi;
    const size_t row = (size_t)b * Nq + qq;
    const int bt = query_t(len, Nq, qq) >> 2;
    const int j_end = min(j_begin + kTableSlice, bt);
    const uint32_t* srow = scores + row * nbp;
    uint64_t* crow = cand + row * (size_t)cap;
    for (int base = j_begin + wave * 64; base < j_end; base += 256) {
      const int j = base + lane;
      uint32_t bits = 0;
      bool pred = false;
      if (j < j_end) {
        bits = srow[j];
        pred = (int)(bits >> 20) >= m;
      }
      const uint64_t mask = __ballot(pred);
      if (mask != 0) {
        const int leader = __ffsll((long long)mask) - 1;
        uint32_t pos0 = 0;
        if (lane == leader) pos0 = atomicAdd(&cand_cnt[row], (uint32_t)__popcll(mask));
        pos0 = __shfl(pos0, leader);
        if (pred) crow[pos0 + (uint32_t)__popcll(mask & lanemask_lt())] = make_key(bits, (uint32_t)j);
      }
    }
  }
}

// ------------------------------------------------------------------ STREAM
// In-place: keep the 512 largest of the n (> 512) distinct keys of `list`
// at its front; returns the 512th largest key.  One wavefront; hist is a
// 256-entry LDS scratch of that wavefront.
__device__ uint64_t wave_compact(uint64_t* list, uint32_t n, uint32_t* hist) {
  const int lane = lane_id();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  uint64_t prefix = 0, pmask = 0;
  uint32_t k = kTopK;
  for (int shift = 56; shift >= 0; shift -= 8) {
#pragma unroll
    for (int i = 0; i < 4; ++i) hist[4 * lane + i] = 0;
    wave_sync_lds();
    for (uint32_t i = lane; i < n; i += 64) {
      const uint64_t key = list[i];
      if ((key & pmask) == prefix) atomicAdd(&hist[(uint32_t)(key >> shift) & 255u], 1u);
    }
    wave_sync_lds();
    uint32_t d, above;
    wave_find_digit(hist, k, d, above);
    k -= above;
    prefix |= (uint64_t)d << shift;
    pmask |= 0xffull << shift;
    wave_sync_lds();
  }
  uint32_t w = 0;
  for (uint32_t base = 0; base < n; base += 64) {
    const uint32_t i = base + lane;
    const uint64_t key = i < n ? list[i] : 0ull;
    const bool keep = i < n && key >= prefix;
    const uint64_t m = __ballot(keep);
    if (keep) list[w + (uint32_t)__popcll(m & lanemask_lt())] = key;
    w += (uint32_t)__popcll(m);
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  return prefix;
}

// Grid (ceil(Nq/64), B); 4 wavefronts x 16 queries.
__global__ __launch_bounds__(256) void score_stream_kernel(const uint16_t* __restrict__ q_idx,
                                                           const uint16_t* __restrict__ k_cmp,
                                                           const int32_t* __restrict__ lens,
                                                           uint64_t* __restrict__ lists,
                                                           uint32_t* __restrict__ list_cnt,
                                                           int Lmax, int Nq) {
  __shared__ uint4 ktile[2][kStreamTile * 8];
  __shared__ int32_t s_tau[kStreamQ];
  __shared__ uint32_t s_cnt[kStreamQ];
  __shared__ uint32_t s_hist[4][256];

  const int qbase = blockIdx.x * kStreamQ, b = blockIdx.y;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int len = clampi(lens[b], 0, Lmax);
  const int nbp = Lmax >> 2;
  const int t_last = query_t(len, Nq, min(qbase + kStreamQ - 1, Nq - 1));
  const int bt_wg = t_last >= 0 ? (t_last >> 2) : 0;
  if (tid < kStreamQ) {
    s_tau[tid] = -1;
    s_cnt[tid] = 0;
  }
  const int wq0 = qbase + wave * 16;

  // Stationary A fragments: 2 row tiles x 4 k-steps.  Row (lane & 31) of row
  // tile rt is query wq0 + rt*8 + row/4, head row%4; k chunk lane >> 5.
  bf16x8 A[2][4];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int qa = wq0 + rt * 8 + ((lane & 31) >> 2);
    const uint4* p = reinterpret_cast<const uint4*>(
        q_idx + (((size_t)b * Nq + min(qa, Nq - 1)) * kIdxHeads + (lane & 3)) * kIdxDim);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      A[rt][ks] = as_bf16x8(qa < Nq ? p[ks * 2 + (lane >> 5)] : zero_u4());
  }
  // Output queries of this lane: (rt, c) -> local query rt*8 + c*2 + (lane >> 5).
  int btq[2][4];
  uint64_t* lrow[2][4];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int qq = wq0 + rt * 8 + c * 2 + (lane >> 5);
      const int t = query_t(len, Nq, qq);
      btq[rt][c] = (qq < Nq && t >= 0) ? (t >> 2) : 0;
      lrow[rt][c] = lists + ((size_t)b * Nq + min(qq, Nq - 1)) * kListCap;
    }

  const uint4* kb = reinterpret_cast<const uint4*>(k_cmp + (size_t)b * nbp * kIdxDim);
  const int ntiles = (bt_wg + kStreamTile - 1) / kStreamTile;
  uint4 nxt[2];
  auto fetch = [&](int tile) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int e = tid + 256 * u;
      const int j = tile * kStreamTile + (e >> 3);
      nxt[u] = j < bt_wg ? kb[(size_t)j * 8 + (e & 7)] : zero_u4();
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int e = tid + 256 * u;
      const int row = e >> 3, ch = e & 7;
      ktile[buf][row * 8 + (ch ^ (row & 7))] = nxt[u];
    }
  };
  if (ntiles > 0) {
    fetch(0);
    stash(0);
  }
  __syncthreads();

  for (int tile = 0; tile < ntiles; ++tile) {
    const int buf = tile & 1;
    const bool has_next = tile + 1 < ntiles;
    if (has_next) fetch(tile + 1);

    f32x16 acc[2][2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[rt][ct][i] = 0.f;
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const int row = ct * 32 + (lane & 31);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int ch = ks * 2 + (lane >> 5);
        const bf16x8 bf = as_bf16x8(ktile[buf][row * 8 + (ch ^ (row & 7))]);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) acc[rt][ct] = mfma32(A[rt][ks], bf, acc[rt][ct]);
      }
    }

    const int j0 = tile * kStreamTile;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int lq = wave * 16 + rt * 8 + c * 2 + (lane >> 5);
        const int tau = s_tau[lq];
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          const int j = j0 + ct * 32 + (lane & 31);
          const uint32_t bits = relu_sum_bits(acc[rt][ct][4 * c], acc[rt][ct][4 * c + 1],
                                              acc[rt][ct][4 * c + 2], acc[rt][ct][4 * c + 3]);
          if (j < btq[rt][c] && (int)bits > tau) {
            const uint32_t slot = atomicAdd(&s_cnt[lq], 1u);
            lrow[rt][c][slot] = make_key(bits, (uint32_t)j);
          }
        }
      }
    wave_sync_lds();
    // Lists close to capacity: select their top 512 and raise the threshold.
    for (int i = 0; i < 16; ++i) {
      const int lq = wave * 16 + i;
      const uint32_t n = s_cnt[lq];
      if (n > (uint32_t)(kListCap - 2 * kStreamTile)) {
        const int qq = qbase + lq;
        uint64_t* list = lists + ((size_t)b * Nq + qq) * kListCap;
        const uint64_t kth = wave_compact(list, n, s_hist[wave]);
        if (lane == 0) {
          s_cnt[lq] = kTopK;
          s_tau[lq] = (int)(uint32_t)(kth >> 32);
        }
        wave_sync_lds();
      }
    }
    if (has_next) stash(buf ^ 1);
    __syncthreads();
  }
  if (tid < kStreamQ && qbase + tid < Nq) list_cnt[(size_t)b * Nq + qbase + tid] = s_cnt[tid];
}

}  // namespace

// ------------------------------------------------------------------ host side

TopkPath choose_topk_path(const Dims& d, uint32_t flags) {
  if (flags & 1u) return TopkPath::kTable;
  if (flags & 2u) return TopkPath::kStream;
  const double table_bytes = (double)d.B * d.Nq * (d.Lmax / 4) * 4.0;
  return (d.Nq <= 64 && table_bytes <= 512.0 * 1024 * 1024) ? TopkPath::kTable
                                                             : TopkPath::kStream;
}

namespace {
struct TableWs {
  uint32_t* scores;
  uint32_t* ghist;
  uint32_t* cand_cnt;
  uint32_t* overflow;
  uint64_t* cand;
};
struct StreamWs {
  uint64_t* lists;
  uint32_t* cnt;
  uint32_t* overflow;
};
TableWs carve_table(const Dims& d, void* ws, size_t* total) {
  Carve c{static_cast<char*>(ws), 0};
  const size_t rows = (size_t)d.B * d.Nq;
  TableWs w;
  w.scores = c.take<uint32_t>(rows * (size_t)(d.Lmax / 4));
  w.ghist = c.take<uint32_t>(rows * kHistBins + rows);  // histogram, then counts
  w.cand_cnt = w.ghist ? w.ghist + rows * kHistBins : nullptr;
  w.overflow = c.take<uint32_t>(rows);
  w.cand = c.take<uint64_t>(rows * kSelCap);
  if (total) *total = c.off;
  return w;
}
StreamWs carve_stream(const Dims& d, void* ws, size_t* total) {
  Carve c{static_cast<char*>(ws), 0};
  const size_t rows = (size_t)d.B * d.Nq;
  StreamWs w;
  w.lists = c.take<uint64_t>(rows * kListCap);
  w.cnt = c.take<uint32_t>(rows);
  w.overflow = c.take<uint32_t>(rows);
  if (total) *total = c.off;
  return w;
}
}  // namespace

size_t topk_workspace_bytes(const Dims& d, TopkPath path) {
  size_t total = 0;
  if (path == TopkPath::kTable)
    carve_table(d, nullptr, &total);
  else
    carve_stream(d, nullptr, &total);
  return total;
}

hipError_t launch_index_topk(const Dims& d, TopkPath path, const uint16_t* q_idx,
                             const uint16_t* k_cmp, const int32_t* lens, int32_t* sel,
                             int32_t* n_sel, void* ws, hipStream_t s) {
  if (d.B == 0 || d.Nq == 0) return hipSuccess;
  const size_t rows = (size_t)d.B * d.Nq;
  const dim3 grid_q((unsigned)d.Nq, (unsigned)d.B);
  if (path == TopkPath::kTable) {
    TableWs w = carve_table(d, ws, nullptr);
    const size_t nz = rows * kHistBins + rows;
    QSA_LAUNCH(fill_u32_kernel, dim3((unsigned)std::min<size_t>((nz + 255) / 256, 4096)),
                       dim3(256), 0, s, w.ghist, nz, 0u);
    const unsigned slices = (unsigned)((d.Lmax / 4 + kTableSlice - 1) / kTableSlice);
    const dim3 grid(slices, (unsigned)((d.Nq + 3) / 4), (unsigned)d.B);
    QSA_LAUNCH(score_table_kernel, grid, dim3(256), 0, s, q_idx, k_cmp, lens, w.scores,
                       w.ghist, d.Lmax, d.Nq);
    QSA_LAUNCH(table_filter_kernel, grid, dim3(256), 0, s, w.scores, w.ghist, lens,
                       w.cand, w.cand_cnt, d.Lmax, d.Nq, kSelCap);
    QSA_LAUNCH(select_kernel, grid_q, dim3(256), 0, s, w.cand, w.cand_cnt, lens, sel,
                       n_sel, w.overflow, d.Lmax, d.Nq, kSelCap);
    QSA_LAUNCH(select_fallback_kernel<false>, grid_q, dim3(256), 0, s, w.scores, q_idx,
                       k_cmp, lens, w.overflow, sel, n_sel, d.Lmax, d.Nq);
  } else {
    StreamWs w = carve_stream(d, ws, nullptr);
    const dim3 grid((unsigned)((d.Nq + kStreamQ - 1) / kStreamQ), (unsigned)d.B);
    QSA_LAUNCH(score_stream_kernel, grid, dim3(256), 0, s, q_idx, k_cmp, lens, w.lists,
                       w.cnt, d.Lmax, d.Nq);
    QSA_LAUNCH(select_kernel, grid_q, dim3(256), 0, s, w.lists, w.cnt, lens, sel, n_sel,
                       w.overflow, d.Lmax, d.Nq, kListCap);
    QSA_LAUNCH(select_fallback_kernel<true>, grid_q, dim3(256), 0, s, nullptr, q_idx,
                       k_cmp, lens, w.overflow, sel, n_sel, d.Lmax, d.Nq);
  }
  return hipGetLastError();
}

}  // namespace qsa
