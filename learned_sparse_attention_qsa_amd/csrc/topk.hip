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
//  with MFMA (16x16x32, 4 queries x 4 heads per tile) and writes the fp32
//  score table plus, for every 16-block group, the group's best score.  The
//  512 largest group maxima belong to 512 distinct blocks, so the 512th
//  largest group maximum is a lower bound of the row's 512th best score; a
//  small per-row radix pass finds it (rounded down to 22 significant bits)
//  from the group maxima alone.  A filter pass appends every key whose score
//  reaches that bound (typically a few percent more than 512 keys) to a
//  candidate list, and a select kernel sorts them in LDS.  Cost over the
//  bare k_cmp scan: the score table (4 B per query per block) written once
//  and read once.
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

constexpr int kHistBins = 2048;    // radix bins of 11 bits (table threshold)
constexpr int kTableSlice = 1024;  // blocks per scoring workgroup (table engine)
constexpr int kFilterSlice = 2048; // blocks per filter workgroup (table engine)
constexpr int kGroup = 16;         // blocks per group maximum (table engine)
constexpr int kSelCap = 8192;      // candidates a select workgroup holds in LDS
constexpr int kHistW = 256;        // stream engine: threshold-tracking bins per query
constexpr int kHyst = 64;          // stream engine: new counts between threshold updates
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

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, m);
  const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), m);
  return ((uint64_t)hi << 32) | lo;
}

// Bitonic sort, descending, of N = 256 * NPT 64-bit values; thread t holds
// elements t*NPT .. t*NPT + NPT - 1 in v.  Exchanges within a thread use
// registers, within a wavefront lane shuffles, across wavefronts the LDS
// buffer xch (N values); only those last stages need barriers.  256 threads.
template <int NPT>
__device__ __forceinline__ void block_sort_desc(uint64_t (&v)[NPT], uint64_t* xch) {
  constexpr int N = 256 * NPT;
  const int t = threadIdx.x;
  // fully unrolled: j must be a compile-time constant for the register cases
#pragma unroll
  for (int k = 2; k <= N; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      if (j < NPT) {
#pragma unroll
        for (int s = 0; s < NPT; ++s) {
          if (s & j) continue;
          const int i = t * NPT + s;
          const bool desc = (i & k) == 0;
          const uint64_t a = v[s], b = v[s | j];
          const bool sw = (a < b) == desc;
          v[s] = sw ? b : a;
          v[s | j] = sw ? a : b;
        }
      } else {
        uint64_t o[NPT];
        if (j < 64 * NPT) {
#pragma unroll
          for (int s = 0; s < NPT; ++s) o[s] = shfl_xor_u64(v[s], j / NPT);
        } else {
          __syncthreads();
#pragma unroll
          for (int s = 0; s < NPT; ++s) xch[t * NPT + s] = v[s];
          __syncthreads();
#pragma unroll
          for (int s = 0; s < NPT; ++s) o[s] = xch[(t * NPT + s) ^ j];
        }
#pragma unroll
        for (int s = 0; s < NPT; ++s) {
          const int i = t * NPT + s;
          const bool desc = (i & k) == 0;
          const bool keep_max = ((i & j) == 0) == desc;
          v[s] = keep_max ? (v[s] > o[s] ? v[s] : o[s]) : (v[s] < o[s] ? v[s] : o[s]);
        }
      }
    }
  }
}

// Select's finish for at most 256 * NPT candidates held in v (0 = empty, below
// every key): sort them (descending), then sort the block ids of the first 512
// ascending into outb.  xch: LDS scratch of 256 * NPT keys.
template <int NPT>
__device__ __forceinline__ void finish_sorted(uint64_t (&v)[NPT], uint64_t* xch, int32_t* outb) {
  const int t = threadIdx.x;
  block_sort_desc<NPT>(v, xch);
  __syncthreads();
  // the 512 best keys sit at positions 0..511: pass their ids through LDS
  // and sort them ascending (as complemented ids, descending)
#pragma unroll
  for (int s = 0; s < NPT; ++s) {
    const int i = t * NPT + s;
    if (i < kTopK) outb[i] = (int32_t)key_block(v[s]);
  }
  __syncthreads();
  uint64_t w[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) w[s] = 0xffffffffull - (uint32_t)outb[2 * t + s];
  block_sort_desc<2>(w, xch);
#pragma unroll
  for (int s = 0; s < 2; ++s) outb[2 * t + s] = (int32_t)(0xffffffffu - (uint32_t)w[s]);
  __syncthreads();
}

// The same for n <= 256 * NPT candidates in keys[0..n) (LDS, also the scratch).
template <int NPT>
__device__ __forceinline__ void finish_small(uint64_t* keys, uint32_t n, int32_t* outb) {
  const int t = threadIdx.x;
  uint64_t v[NPT];
#pragma unroll
  for (int s = 0; s < NPT; ++s) {
    const uint32_t i = (uint32_t)(t * NPT + s);
    v[s] = i < n ? keys[i] : 0ull;
  }
  finish_sorted<NPT>(v, keys, outb);
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

// One wavefront: per-lane counts c[0..3] of bins 4*lane .. 4*lane+3 (bin
// order = value order); find the highest bin whose suffix count (that bin and
// every bin above it) reaches k.  Returns the bin and its suffix count.  The
// caller guarantees the total reaches k.
__device__ __forceinline__ void wave_suffix_bin4(uint32_t c0, uint32_t c1, uint32_t c2,
                                                 uint32_t c3, uint32_t k, int& bin,
                                                 uint32_t& suffix) {
  const int l = lane_id();
  const uint32_t mine = c0 + c1 + c2 + c3;
  uint32_t S = mine;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t o = __shfl_down(S, off);
    if (l + off < 64) S += o;
  }
  const uint64_t m = __ballot(S >= k);
  const int L = 63 - __clzll((long long)m);
  uint32_t cum = __shfl(S, L) - __shfl(mine, L);
  const uint32_t b3 = __shfl(c3, L), b2 = __shfl(c2, L), b1 = __shfl(c1, L), b0 = __shfl(c0, L);
  int d;
  if (cum + b3 >= k) {
    d = 3;
    cum += b3;
  } else if (cum + b3 + b2 >= k) {
    d = 2;
    cum += b3 + b2;
  } else if (cum + b3 + b2 + b1 >= k) {
    d = 1;
    cum += b3 + b2 + b1;
  } else {
    d = 0;
    cum += b3 + b2 + b1 + b0;
  }
  bin = 4 * L + d;
  suffix = cum;
}

// One wavefront, a kHistBins-bin histogram h (LDS or global): the highest bin
// whose suffix count reaches k, and that suffix count.
__device__ __forceinline__ void wave_suffix_bin_2048(const uint32_t* h, uint32_t k, int& bin,
                                                     uint32_t& suffix) {
  const int lane = lane_id();
  // lane holds bins [32*lane, 32*lane+32); rotated order keeps LDS reads
  // conflict-free
  uint32_t mine = 0;
#pragma unroll 8
  for (int i = 0; i < 32; ++i) mine += h[32 * lane + ((i + lane) & 31)];
  uint32_t S = mine;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t o = __shfl_down(S, off);
    if (lane + off < 64) S += o;
  }
  const uint64_t m = __ballot(S >= k);
  const int L = 63 - __clzll((long long)m);
  const uint32_t above = __shfl(S, L) - __shfl(mine, L);
  // lanes 0..31 take one bin of lane L's range each; suffix within it
  const int i = lane & 31;
  uint32_t c = lane < 32 ? h[32 * L + i] : 0u;
  uint32_t T = c;
#pragma unroll
  for (int off = 1; off < 32; off <<= 1) {
    const uint32_t o = __shfl_down(T, off);
    if (i + off < 32) T += o;
  }
  const uint64_t m2 = __ballot(lane < 32 && above + T >= k);
  const int I = 63 - __clzll((long long)m2);
  bin = 32 * L + I;
  suffix = above + __shfl(T, I);
}

// ------------------------------------------------------------------ select
// Exact top-512 of one query straight from its whole row, walking the blocks
// in order (so the output comes out ascending).  Slow path for rows whose
// candidate list does not fit the fast path.  kRecompute: no score table
// exists (stream engine), scores are recomputed from q_idx and k_cmp.
template <bool kRecompute>
__device__ void select_whole_row(const uint32_t* trow, const uint16_t* qrow, const uint16_t* kc,
                                 int bt, int32_t* srow, float* qf, uint32_t* hist,
                                 uint32_t* bcast, uint32_t* wsum) {
  const int tid = threadIdx.x;
  if (kRecompute) {
    for (int i = tid; i < kIdxHeads * kIdxDim; i += blockDim.x)
      qf[i] = __uint_as_float((uint32_t)qrow[i] << 16);
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
}

// One workgroup per query row.  Fast path: the row's candidates (nsub
// segments of up to seg_cap keys, segment lengths in cand_cnt; only keys whose
// score reaches the row's final threshold, when one is given) go to LDS, a
// radix select finds the 512th key and the winners are sorted.  Rows with too
// few or too many candidates take the exact whole-row path.
template <bool kRecompute>
__global__ __launch_bounds__(256) void select_kernel(
    const uint64_t* __restrict__ cand, const uint32_t* __restrict__ cand_cnt, int nsub,
    int seg_cap, const int32_t* __restrict__ tau_final, const uint32_t* __restrict__ table,
    int tstride, const uint16_t* __restrict__ q_idx, const uint16_t* __restrict__ k_cmp,
    const int32_t* __restrict__ lens, int32_t* __restrict__ sel, int32_t* __restrict__ n_sel,
    int Lmax, int Nq) {
  __shared__ uint64_t keys[kSelCap];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t bcast[2];
  __shared__ int32_t outb[kTopK];
  __shared__ uint32_t outn;
  __shared__ uint32_t bad;
  __shared__ float qf[kIdxHeads * kIdxDim];
  __shared__ uint32_t wsum[4];
  const int q = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const size_t row = (size_t)b * Nq + q;
  // threads_per_seg threads walk each segment; the segment length is read
  // before (and independently of) lens
  const int tps = blockDim.x / nsub;
  const int seg = tid / tps, sub = tid % tps;
  const uint32_t n_seg_raw = seg < nsub ? cand_cnt[row * nsub + seg] : 0u;
  const int t = query_t(clampi(lens[b], 0, Lmax), Nq, q);
  int32_t* srow = sel + row * kTopK;
  if (write_trivial(t, srow, n_sel + row)) return;
  const int bt = t >> 2;
  const int tau = tau_final ? tau_final[row] : -1;
  if (tid == 0) {
    outn = 0;
    bad = 0;
  }
  __syncthreads();
  const int lane = lane_id();
  uint32_t n_seg = 0;
  if (seg < nsub) {
    n_seg = n_seg_raw;
    if (n_seg > (uint32_t)seg_cap) {
      atomicOr(&bad, 1u);
      n_seg = seg_cap;
    }
  }
  const uint64_t* src = cand + (row * nsub + (seg < nsub ? seg : 0)) * (size_t)seg_cap;
  if (nsub == 1 && n_seg <= 1024u && cand_cnt[row] <= (uint32_t)seg_cap) {
    // short list: straight into registers, 4 keys per thread, then sort
    uint64_t v[4];
    int mine = 0;
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
      const uint32_t i = (uint32_t)(tid * 4 + s2);
      const uint64_t key = i < n_seg ? src[i] : 0ull;
      const bool keep = i < n_seg && (int)(uint32_t)(key >> 32) >= tau;
      v[s2] = keep ? key : 0ull;
      mine += keep ? 1 : 0;
    }
    atomicAdd(&outn, (uint32_t)mine);
    __syncthreads();
    if (outn >= (uint32_t)kTopK) {
      finish_sorted<4>(v, keys, outb);
      for (int i = tid; i < kTopK; i += blockDim.x) srow[i] = outb[i];
      if (tid == 0) n_sel[row] = kTopK;
      return;
    }
    // too few: the exact whole-row path below
    __syncthreads();
    if (tid == 0) {
      outn = 0;
      bad = 1;
    }
    __syncthreads();
  }
  uint32_t longest = n_seg;
  for (int off = 32; off >= 1; off >>= 1) longest = max(longest, (uint32_t)__shfl_xor((int)longest, off));
  for (uint32_t i0 = 0; i0 < longest; i0 += 8 * tps) {
    uint64_t kv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint32_t i = i0 + u * tps + sub;
      kv[u] = (seg < nsub && i < n_seg) ? src[i] : 0ull;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint32_t i = i0 + u * tps + sub;
      const bool keep = seg < nsub && i < n_seg && (int)(uint32_t)(kv[u] >> 32) >= tau;
      const uint64_t m = __ballot(keep);
      if (m == 0) continue;
      const int leader = __ffsll((long long)m) - 1;
      uint32_t p0 = 0;
      if (lane == leader) p0 = atomicAdd(&outn, (uint32_t)__popcll(m));
      p0 = __shfl(p0, leader);
      const uint32_t p = p0 + (uint32_t)__popcll(m & lanemask_lt());
      if (keep && p < (uint32_t)kSelCap) keys[p] = kv[u];
    }
  }
  __syncthreads();
  const uint32_t n = outn;
  const bool ok = bad == 0 && n >= (uint32_t)kTopK && n <= (uint32_t)kSelCap;
  __syncthreads();
  if (ok) {
    if (n <= 2048u) {
      // few candidates: sort them all, keep the first 512, sort their ids
      if (n <= 1024u)
        finish_small<4>(keys, n, outb);
      else
        finish_small<8>(keys, n, outb);
      for (int i = tid; i < kTopK; i += blockDim.x) srow[i] = outb[i];
      if (tid == 0) n_sel[row] = kTopK;
      return;
    } else {
      const uint64_t kth = block_kth_largest(keys, (int)n, kTopK, hist, bcast);
      if (tid == 0) outn = 0;
      __syncthreads();
      for (uint32_t i = tid; i < n; i += blockDim.x) {
        const uint64_t key = keys[i];
        if (key >= kth) outb[atomicAdd(&outn, 1u)] = (int32_t)key_block(key);
      }
      __syncthreads();
    }
    bitonic_sort_512(outb);
    for (int i = tid; i < kTopK; i += blockDim.x) srow[i] = outb[i];
    if (tid == 0) n_sel[row] = kTopK;
    return;
  }
  const int nbp = Lmax >> 2;
  select_whole_row<kRecompute>(table + (kRecompute ? 0 : row * (size_t)tstride),
                               q_idx + row * kIdxHeads * kIdxDim,
                               k_cmp + (size_t)b * nbp * kIdxDim, bt, srow, qf, hist, bcast, wsum);
  if (tid == 0) n_sel[row] = kTopK;
}

// ------------------------------------------------------------------ TABLE
// Grid (ceil(Lmax/4 / kTableSlice), ceil(Nq/4), B), 256 threads.  Wavefront w
// scores blocks [j_begin + 256 w, + 256) in two batches of eight 16-block
// tiles.  MFMA 16x16x32: A = 16 rows (query r/4, head r%4), B = 16 blocks;
// the lane (r, kc) receives block r of the tile for query q0 + kc, all four
// heads.  A tile is also one group: its maximum over the 16 lanes of a query
// goes to gmax.
__global__ __launch_bounds__(256) void score_table_kernel(const uint16_t* __restrict__ q_idx,
                                                          const uint16_t* __restrict__ k_cmp,
                                                          const int32_t* __restrict__ lens,
                                                          uint32_t* __restrict__ scores,
                                                          int tstride,
                                                          uint32_t* __restrict__ gmax,
                                                          int gstride, int Lmax, int Nq) {
  const int slice = blockIdx.x, q0 = blockIdx.y * 4, b = blockIdx.z;
  const int len = clampi(lens[b], 0, Lmax);
  const int nbp = Lmax >> 2;
  const int t_last = query_t(len, Nq, min(q0 + 3, Nq - 1));
  const int j_begin = slice * kTableSlice;
  const int j_end = min(j_begin + kTableSlice, t_last >= 0 ? (t_last >> 2) : 0);
  if (j_begin >= j_end) return;

  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int r = lane & 15, kc = lane >> 4;
  bf16x8 a0 = as_bf16x8(zero_u4()), a1 = a0;
  const int qa = q0 + (r >> 2);
  if (qa < Nq) {
    const uint4* p = reinterpret_cast<const uint4*>(
        q_idx + (((size_t)b * Nq + qa) * kIdxHeads + (r & 3)) * kIdxDim);
    a0 = as_bf16x8(p[kc]);
    a1 = as_bf16x8(p[4 + kc]);
  }
  const int qo = q0 + kc;
  const int t_o = query_t(len, Nq, qo);
  const int bt_o = (qo < Nq && t_o >= 0) ? (t_o >> 2) : 0;
  const int lim = min(bt_o, j_end);
  const size_t orow = (size_t)b * Nq + min(qo, Nq - 1);
  uint32_t* srow = scores + orow * tstride;
  uint32_t* grow = gmax + orow * gstride;
  const uint4* kb = reinterpret_cast<const uint4*>(k_cmp + (size_t)b * nbp * kIdxDim);

  constexpr int U = 8;
#pragma unroll 1
  for (int batch = 0; batch < 2; ++batch) {
    const int jt = j_begin + wave * (2 * U * 16) + batch * (U * 16);
    if (jt >= j_end) break;
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
      const int j0 = jt + u * 16;
      const int jo = j0 + r;
      // masked blocks count as score +0 in the group maximum: they can only
      // lower the bound, which stays valid
      const uint32_t bits = jo < lim ? relu_sum_bits(acc[0], acc[1], acc[2], acc[3]) : 0u;
      if (jo < lim) srow[jo] = bits;
      uint32_t gm = bits;
      gm = max(gm, (uint32_t)__shfl_xor((int)gm, 8));
      gm = max(gm, (uint32_t)__shfl_xor((int)gm, 4));
      gm = max(gm, (uint32_t)__shfl_xor((int)gm, 2));
      gm = max(gm, (uint32_t)__shfl_xor((int)gm, 1));
      if (r == 0 && j0 < lim && qo < Nq) grow[j0 / kGroup] = gm;
    }
  }
}

// One workgroup (1,024 threads) per query row: a lower bound tau of the
// row's 512th best score from its group maxima.  With G >= 512 groups the
// 512th largest group maximum is such a bound (512 distinct blocks reach it);
// two 11-bit radix passes find it to 22 bits, rounded down (still a lower
// bound).  First every thread keeps its two largest maxima: when every thread
// has two, the smallest of those 2,048 numbers is itself a valid bound, so
// only maxima at or above it need counting.  Rows with fewer than 512 groups
// keep every candidate (tau = 0).  Each thread reads 16 maxima per chunk
// (four 16-byte loads in flight); later passes re-read them from the L2.
constexpr int kThrThreads = 1024;

__device__ __forceinline__ void load_group_chunk(const uint32_t* g, int G, int c, uint32_t (&x)[16]) {
  const uint4* g4 = reinterpret_cast<const uint4*>(g);
  const int n4 = (G + 3) >> 2;
  uint4 v[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int i = (c * 4 + u) * kThrThreads + (int)threadIdx.x;
    v[u] = i < n4 ? g4[i] : zero_u4();
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int e = 4 * ((c * 4 + u) * kThrThreads + (int)threadIdx.x);
    x[4 * u + 0] = v[u].x;
    x[4 * u + 1] = e + 1 < G ? v[u].y : 0u;
    x[4 * u + 2] = e + 2 < G ? v[u].z : 0u;
    x[4 * u + 3] = e + 3 < G ? v[u].w : 0u;
  }
}
__device__ __forceinline__ bool group_valid(int G, int c, int k) {
  const int u = k >> 2, e = k & 3;
  return 4 * ((c * 4 + u) * kThrThreads + (int)threadIdx.x) + e < G;
}

__global__ __launch_bounds__(kThrThreads) void table_threshold_kernel(
    const uint32_t* __restrict__ gmax, int gstride, const int32_t* __restrict__ lens,
    uint32_t* __restrict__ thr, int Lmax, int Nq) {
  __shared__ uint32_t hist[kHistBins];
  __shared__ uint32_t s_cut;
  __shared__ int s_bin;
  __shared__ uint32_t s_above;
  const int row = blockIdx.x, b = row / Nq, q = row % Nq, tid = threadIdx.x;
  const int t = query_t(clampi(lens[b], 0, Lmax), Nq, q);
  const int bt = t >= 0 ? (t >> 2) : 0;
  const int G = (bt + kGroup - 1) / kGroup;
  if (bt <= kTopK || G < kTopK) {
    if (tid == 0) thr[row] = 0u;
    return;
  }
  const uint32_t* g = gmax + (size_t)row * gstride;
  const int nchunks = (G + 16 * kThrThreads - 1) / (16 * kThrThreads);
  uint32_t m1 = 0, m2 = 0;
  for (int c = 0; c < nchunks; ++c) {
    uint32_t x[16];
    load_group_chunk(g, G, c, x);
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const uint32_t v = group_valid(G, c, k) ? x[k] : 0u;
      m2 = v >= m1 ? m1 : max(m2, v);
      m1 = max(m1, v);
    }
  }
  if (tid == 0) s_cut = 0xffffffffu;
  for (int i = tid; i < kHistBins; i += blockDim.x) hist[i] = 0u;
  __syncthreads();
  // A thread with fewer than two maxima reports 0, which makes the cut 0: then
  // every maximum is counted (always valid).
  uint32_t wm = m2;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) wm = min(wm, (uint32_t)__shfl_xor((int)wm, off));
  if ((tid & 63) == 0) atomicMin(&s_cut, wm);
  __syncthreads();
  const uint32_t cut = s_cut;
  for (int c = 0; c < nchunks; ++c) {
    uint32_t x[16];
    load_group_chunk(g, G, c, x);
#pragma unroll
    for (int k = 0; k < 16; ++k)
      if (group_valid(G, c, k) && x[k] >= cut) atomicAdd(&hist[x[k] >> 20], 1u);
  }
  __syncthreads();
  if (tid < 64) {
    int bin;
    uint32_t sfx;
    wave_suffix_bin_2048(hist, kTopK, bin, sfx);
    if (tid == 0) {
      s_bin = bin;
      s_above = sfx - hist[bin];
    }
  }
  __syncthreads();
  const uint32_t bin1 = (uint32_t)s_bin;
  const uint32_t k2 = (uint32_t)kTopK - s_above;
  for (int i = tid; i < kHistBins; i += blockDim.x) hist[i] = 0u;
  __syncthreads();
  for (int c = 0; c < nchunks; ++c) {
    uint32_t x[16];
    load_group_chunk(g, G, c, x);
#pragma unroll
    for (int k = 0; k < 16; ++k)
      if (group_valid(G, c, k) && (x[k] >> 20) == bin1)
        atomicAdd(&hist[(x[k] >> 9) & (kHistBins - 1)], 1u);
  }
  __syncthreads();
  if (tid < 64) {
    int bin2;
    uint32_t sfx;
    wave_suffix_bin_2048(hist, k2, bin2, sfx);
    if (tid == 0) thr[row] = (bin1 << 20) | ((uint32_t)bin2 << 9);
  }
}

// Grid (nslices, ceil(Nq/4), B); workgroup w reads blocks [w * fslice, +
// fslice) of 4 rows (fslice a multiple of kFilterSlice) and writes the keys
// whose score reaches the row's bound to its own segment of the row's
// candidate list (segment w, fslice keys: it cannot overflow), and the count
// to cand_cnt[row][w].  No global atomics: candidates are rare (about 512 of
// a row's blocks) and contended counters would serialize them.
__global__ __launch_bounds__(256) void table_filter_kernel(const uint32_t* __restrict__ scores,
                                                           int tstride,
                                                           const uint32_t* __restrict__ thr,
                                                           const int32_t* __restrict__ lens,
                                                           uint64_t* __restrict__ cand,
                                                           uint32_t* __restrict__ cand_cnt,
                                                           int Lmax, int Nq, int fslice) {
  __shared__ uint32_t s_cnt[4];
  const int slice = blockIdx.x, q0 = blockIdx.y * 4, b = blockIdx.z;
  const int nslices = gridDim.x;
  const int len = clampi(lens[b], 0, Lmax);
  const int tid = threadIdx.x;
  if (tid < 4) s_cnt[tid] = 0u;
  int jend[4];
  uint32_t tau[4];
#pragma unroll
  for (int qi = 0; qi < 4; ++qi) {
    const int qq = min(q0 + qi, Nq - 1);
    const int t = query_t(len, Nq, qq);
    const int bt = t >= 0 ? (t >> 2) : 0;
    // rows with at most 512 candidates are finished by the select kernel alone
    const bool live = q0 + qi < Nq && bt > kTopK;
    jend[qi] = live ? min((slice + 1) * fslice, bt) : 0;
    tau[qi] = live ? thr[(size_t)b * Nq + qq] : 0u;
  }
  __syncthreads();
  for (int j_begin = slice * fslice; j_begin < (slice + 1) * fslice; j_begin += kFilterSlice) {
    // all loads first: 4 rows x 2 passes of 1024 blocks, 4 blocks per thread
    uint4 v[4][2];
#pragma unroll
    for (int qi = 0; qi < 4; ++qi) {
      const uint32_t* srow = scores + ((size_t)b * Nq + min(q0 + qi, Nq - 1)) * tstride;
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int j4 = j_begin + p * 1024 + tid * 4;
        v[qi][p] = j4 < jend[qi] ? *reinterpret_cast<const uint4*>(srow + j4) : zero_u4();
      }
    }
#pragma unroll
    for (int qi = 0; qi < 4; ++qi) {
      uint32_t pm = 0;  // bit (p*4+e): element passes
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const uint32_t e4[4] = {v[qi][p].x, v[qi][p].y, v[qi][p].z, v[qi][p].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = j_begin + p * 1024 + tid * 4 + e;
          pm |= (j < jend[qi] && e4[e] >= tau[qi] ? 1u : 0u) << (p * 4 + e);
        }
      }
      if (pm == 0) continue;
      const size_t row = (size_t)b * Nq + q0 + qi;
      uint32_t pos = atomicAdd(&s_cnt[qi], (uint32_t)__popc(pm));
      uint64_t* seg = cand + (row * nslices + slice) * (size_t)fslice;
      while (pm) {
        const int bit = __ffs(pm) - 1;
        pm &= pm - 1;
        const int p = bit >> 2, e = bit & 3;
        const uint4 a = p ? v[qi][1] : v[qi][0];  // (selects, not a dynamic register index)
        const uint32_t sc = e == 0 ? a.x : e == 1 ? a.y : e == 2 ? a.z : a.w;
        seg[pos++] = make_key(sc, (uint32_t)(j_begin + p * 1024 + tid * 4 + e));
      }
    }
  }
  __syncthreads();
  if (tid < 4 && q0 + tid < Nq) cand_cnt[((size_t)b * Nq + q0 + tid) * nslices + slice] = s_cnt[tid];
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

// Stream engine, per query: threshold tau (a score; below 0 = accept all)
// and a 256-bin histogram of the appended scores at bf16 resolution, bin i =
// (score bits >> 16) - base (the last bin also holds everything above;
// scores below the base go to a spare 257th bin that is never read).  Every
// counted element has score bits >= base<<16 and was appended; so if the
// bins from m up hold >= 512 counts, at least 512 blocks seen so far score
// >= (base+m)<<16, and any later block scoring no more than that is beaten by
// all of them (an equal score loses on the higher block id): tau can rise to
// (base+m)<<16.
//
// Survivors are first queued in LDS (one 8-byte entry: score, local query,
// block id) by the scoring lanes; once per tile the queue is drained with
// all 64 lanes busy: list slot, list store, histogram update.  That keeps
// the per-survivor work of the scoring pass to a handful of instructions.
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kRing = 8;        // LDS tile slots of the stream engine
constexpr int kListCap = 16384; // candidate list entries per query
// survivors one tile can add to a wavefront's queue, plus fewer than 64 held over
constexpr int kQueue = kStreamTile * 16 + 64;
constexpr int kHistWords = kHistW / 2 + 1;  // 256 packed bins + the spare bin

// Barriers of the stream engine: no wait on vector-memory stores, so list
// appends stay in flight across tiles.
__device__ __forceinline__ void stream_barrier_compute() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
// Loader: the tiles up to two past the one just consumed must have landed;
// the (kRing - 3) later tiles (8 loads each) may still be in flight.
__device__ __forceinline__ void stream_barrier_loader() {
  asm volatile("s_waitcnt vmcnt(40) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
static_assert(8 * (kRing - 3) == 40, "loader wait count");

// Loader wavefront: copy one 64-block tile of compressed keys straight from
// HBM into ring slot `slot` (8 KiB, eight 16-byte-per-lane DMA loads).  The
// slot is stored swizzled: block row r, 16-byte chunk c lives at r*8 + (c ^ (r&7)).
// Rows past bt_wg load row 0 instead (their scores are masked by the consumer).
__device__ __forceinline__ void dma_tile(uint4* slot, const uint4* kb, int tile, int bt_wg) {
  const int lane = lane_id();
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int s16 = i * 64 + lane;
    const int row = s16 >> 3;
    const int ch = (s16 & 7) ^ (row & 7);
    int j = tile * kStreamTile + row;
    if (j >= bt_wg) j = 0;
    __builtin_amdgcn_global_load_lds(kb + (size_t)j * 8 + ch, (lds_void_t*)(slot + i * 64), 16, 0, 0);
  }
}

// B fragments (compressed keys) of one 32-block half (column tile ct) of a
// 64-block tile, read from the LDS ring.
__device__ __forceinline__ void load_b(const uint4* kt, int ct, bf16x8 (&bf)[4]) {
  const int lane = lane_id();
  const int row = ct * 32 + (lane & 31);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int ch = ks * 2 + (lane >> 5);
    bf[ks] = as_bf16x8(kt[row * 8 + (ch ^ (row & 7))]);
  }
}

// Scores of one 32-block half for the wavefront's 16 queries x 4 heads.
__device__ __forceinline__ void mma_half(const bf16x8 (&bf)[4], const bf16x8 (&A)[2][4],
                                         f32x16 (&acc)[2]) {
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[rt][i] = 0.f;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) acc[rt] = mfma32(A[rt][ks], bf[ks], acc[rt]);
}

__device__ __forceinline__ int rdl(int v, int lane) { return __builtin_amdgcn_readlane(v, lane); }

// Per-wavefront state.  Slot (rt, c) of a lane scores local query
// rt*8 + c*2 + (lane >> 5); the lane keeps a copy of that query's tau.
struct Stream {
  float tau_l[2][4];
  int tau_v, base_v, trig_v;  // lane q < 16: query q's tau bits, base, next update point
  int tq0;                    // position of local query (lane >> 5)
  int nq_left;                // queries of the batch from local query (lane >> 5) on
  uint64_t* lists;            // list of local query 0; query q at + q * kListCap
  uint32_t (*h)[kHistWords];  // the wavefront's 16 histograms
  uint32_t* hc;               // 16 counts currently in the histograms
  uint32_t* cnt;              // 16 list lengths
  uint32_t* mx;               // 16 best scores seen before the base is set
  uint32_t* rs;               // 256-word radix scratch
  uint64_t* queue;            // kQueue survivors of the current tile
};

__device__ __forceinline__ int slot_query(int rt, int c) { return rt * 8 + c * 2 + (lane_id() >> 5); }


// Filter one 32-block half against tau; queue the survivors behind the qn
// already queued this tile.  kFull: every block of the tile is below every
// query's own block.  Returns the new queue length.
template <bool kFull>
__device__ __forceinline__ int stream_epilogue(Stream& st, const f32x16 (&acc)[2], int tile, int ct,
                                               int qn) {
  const int lane = lane_id();
  const int j = tile * kStreamTile + ct * 32 + (lane & 31);
  float sc[2][4];
  bool pass[2][4];
  uint64_t any = 0;
  // scores and pass tests of all 8 slots first, without branches, so the
  // compiler can interleave them
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      sc[rt][c] = relu_sum(acc[rt][4 * c], acc[rt][4 * c + 1], acc[rt][4 * c + 2],
                           acc[rt][4 * c + 3]);
      bool p = sc[rt][c] > st.tau_l[rt][c];
      if (!kFull) {
        const int off = rt * 8 + c * 2;
        const int tq = st.tq0 + off;
        p = p && off < st.nq_left && tq >= 0 && j < (tq >> 2);
      }
      pass[rt][c] = p;
      any |= __ballot(p);
    }
  if (any == 0) return qn;
  const uint32_t tag = (uint32_t)j | ((uint32_t)(lane >> 5) << 28);
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint64_t m = __ballot(pass[rt][c]);
      if (pass[rt][c]) {
        const uint32_t pos = __builtin_amdgcn_mbcnt_hi(
            (uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, (uint32_t)qn));
        st.queue[pos] = ((uint64_t)__float_as_uint(sc[rt][c]) << 32) |
                        (uint64_t)(tag + ((uint32_t)(rt * 8 + c * 2) << 28));
      }
      qn += __popcll(m);
    }
  return qn;
}

// Drain the tile's queue: append every survivor to its query's list and
// count it in the histogram (first tile: only track the best score).
template <bool kFirst>
__device__ __forceinline__ void stream_drain(Stream& st, int qn) {
  const int lane = lane_id();
  wave_sync_lds();
  for (int i0 = 0; i0 < qn; i0 += 64) {
    const int i = i0 + lane;
    const uint64_t e = st.queue[min(i, qn - 1)];
    const uint32_t bits = (uint32_t)(e >> 32);
    const uint32_t lo = (uint32_t)e;
    const int q = (int)(lo >> 28);
    const uint32_t j = lo & 0x0fffffffu;
    // (a lane-crossing read takes its value only from active lanes: do it
    // before the tail lanes drop out)
    const int qbase = kFirst ? 0 : __shfl(st.base_v, q);
    if (i < qn) {
      const uint32_t pos = atomicAdd(&st.cnt[q], 1u);
      // (the upkeep compacts a list before it can fill: pos < kListCap)
      st.lists[(size_t)q * kListCap + min(pos, (uint32_t)kListCap - 1)] = make_key(bits, j);
      if (kFirst) {
        atomicMax(&st.mx[q], bits);
      } else {
        const int bin = (int)(bits >> 16) - qbase;
        const int bb = bin < 0 ? kHistW : min(bin, kHistW - 1);
        atomicAdd(&st.h[q][bb >> 1], 1u << ((bb & 1) * 16));
        atomicAdd(&st.hc[q], bin < 0 ? 0u : 1u);
      }
    }
  }
  wave_sync_lds();
}

// New tau / base of local query i: refresh the lanes' copies.
__device__ __forceinline__ void stream_set_query(Stream& st, int i, int tau_bits, int base) {
  const int lane = lane_id();
  if (lane == i) {
    st.tau_v = tau_bits;
    st.base_v = base;
  }
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (slot_query(rt, c) == i) st.tau_l[rt][c] = __uint_as_float((uint32_t)tau_bits);
}

// Raise tau of local query i from its histogram (one wavefront).
__device__ __forceinline__ void stream_raise_tau(Stream& st, int i) {
  const int lane = lane_id();
  uint32_t* h = st.h[i];
  const uint32_t w0 = h[2 * lane], w1 = h[2 * lane + 1];
  int m;
  uint32_t total;
  wave_suffix_bin4(w0 & 0xffffu, w0 >> 16, w1 & 0xffffu, w1 >> 16, kTopK, m, total);
  if (m > 0) {
    uint32_t nw[2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      uint32_t packed = 0;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int src = 4 * lane + 2 * half + e + m;
        uint32_t cc = 0;
        if (src < kHistW) cc = (h[src >> 1] >> ((src & 1) * 16)) & 0xffffu;
        packed |= cc << (16 * e);
      }
      nw[half] = packed;
    }
    wave_sync_lds();
    h[2 * lane] = nw[0];
    h[2 * lane + 1] = nw[1];
  }
  const int nb = rdl(st.base_v, i) + m;
  const int nt = max(nb << 16, rdl(st.tau_v, i));
  if (lane == 0) st.hc[i] = total;
  if (lane == i) st.trig_v = (int)total + kHyst;
  stream_set_query(st, i, nt, nb);
  wave_sync_lds();
}

// Rare: the list of local query i is nearly full.  Keep its 512 best keys,
// set tau to the exact 512th score and rebuild the histogram from them.
__device__ __forceinline__ void stream_compact(Stream& st, int i) {
  const int lane = lane_id();
  uint64_t* list = st.lists + (size_t)i * kListCap;
  const uint32_t n = st.cnt[i];
  const uint64_t kth = wave_compact(list, n, st.rs);
  const int tau_bits = (int)(uint32_t)(kth >> 32);
  const int base = tau_bits >> 16;
  st.h[i][2 * lane] = 0u;
  st.h[i][2 * lane + 1] = 0u;
  if (lane == 0) st.h[i][kHistW / 2] = 0u;
  wave_sync_lds();
  for (int k2 = lane; k2 < kTopK; k2 += 64) {
    const uint32_t sb = (uint32_t)(list[k2] >> 32);
    const int bin = min((int)(sb >> 16) - base, kHistW - 1);
    atomicAdd(&st.h[i][bin >> 1], 1u << ((bin & 1) * 16));
  }
  if (lane == 0) {
    st.hc[i] = kTopK;
    st.cnt[i] = kTopK;
  }
  if (lane == i) st.trig_v = kTopK + kHyst;
  stream_set_query(st, i, max(tau_bits, rdl(st.tau_v, i)), base);
  wave_sync_lds();
}

// After a tile: raise tau where enough new counts arrived, compact nearly
// full lists (rare).
__device__ __forceinline__ void stream_upkeep(Stream& st) {
  const int lane = lane_id();
  const uint32_t hc = lane < 16 ? st.hc[lane] : 0u;
  const uint32_t cnt = lane < 16 ? st.cnt[lane] : 0u;
  uint64_t r = __ballot(lane < 16 && (int)hc >= st.trig_v);
  while (r) {
    const int i = __builtin_ctzll(r);
    r &= r - 1;
    stream_raise_tau(st, i);
  }
  // one tile adds at most 64 entries to a list
  uint64_t f = __ballot(lane < 16 && cnt > (uint32_t)(kListCap - 2 * kStreamTile));
  while (f) {
    const int i = __builtin_ctzll(f);
    f &= f - 1;
    stream_compact(st, i);
  }
}

// One tile k: MFMAs of its second half, filter of its first half (computed
// in the previous step), MFMAs of the next tile's first half, filter of the
// second half; then, once a full wavefront's worth of survivors is queued
// (or on the first tile), the queue drain and the per-query upkeep; barrier.
template <bool kFirst, bool kFull>
__device__ __forceinline__ void stream_step(Stream& st, const bf16x8 (&A)[2][4],
                                            uint4 (*ring)[kStreamTile * 8], f32x16 (&accA)[2],
                                            f32x16 (&accB)[2], int k, int ntiles, int& qn) {
  const int lane = lane_id();
  bf16x8 bf[4], bn[4];
  load_b(ring[k % kRing], 1, bf);
  // (the slot of tile k+1 is always LDS of the ring; unused past the end)
  load_b(ring[(k + 1) % kRing], 0, bn);
  mma_half(bf, A, accB);
  qn = stream_epilogue<kFull>(st, accA, k, 0, qn);
  // (unconditional, also past the last tile: a conditional update would make
  // the compiler copy the accumulators, and the copies wait for the MFMAs)
  mma_half(bn, A, accA);
  qn = stream_epilogue<kFull>(st, accB, k, 1, qn);
  if (kFirst) {
    if (qn > 0) stream_drain<true>(st, qn);
    qn = 0;
    // histogram base: one octave below the best score of the first tile
    wave_sync_lds();
    const int base = lane < 16 ? max(0, (int)(st.mx[lane] >> 16) - 128) : 0;
    for (int i = 0; i < 16; ++i) stream_set_query(st, i, (int)0xbf800000u, rdl(base, i));
  } else if (qn >= 64) {
    stream_drain<false>(st, qn);
    qn = 0;
    stream_upkeep(st);
  }
  stream_barrier_compute();
}

// Grid (ceil(Nq/64), B); 5 wavefronts: 4 compute wavefronts x 16 queries and
// one loader wavefront feeding an 8-slot LDS ring of key tiles.  Compute
// wavefronts run tile k+1's MFMAs before tile k's filtering (double-buffered
// accumulators), so matrix and vector work overlap.
__global__ __launch_bounds__(320) void score_stream_kernel(const uint16_t* __restrict__ q_idx,
                                                           const uint16_t* __restrict__ k_cmp,
                                                           const int32_t* __restrict__ lens,
                                                           uint64_t* __restrict__ lists,
                                                           uint32_t* __restrict__ list_cnt,
                                                           int32_t* __restrict__ tau_out, int Lmax,
                                                           int Nq) {
  __shared__ uint4 ring[kRing][kStreamTile * 8];
  __shared__ uint32_t s_h[kStreamQ][kHistWords];
  __shared__ uint32_t s_hc[kStreamQ];
  __shared__ uint32_t s_mx[kStreamQ];
  __shared__ uint32_t s_cnt[kStreamQ];
  __shared__ uint32_t s_rs[4][256];
  __shared__ uint64_t s_queue[4][kQueue];

  const int qbase = blockIdx.x * kStreamQ, b = blockIdx.y;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int len = clampi(lens[b], 0, Lmax);
  const int nbp = Lmax >> 2;
  const int t_last = query_t(len, Nq, min(qbase + kStreamQ - 1, Nq - 1));
  const int bt_wg = t_last >= 0 ? (t_last >> 2) : 0;
  const int ntiles = (bt_wg + kStreamTile - 1) / kStreamTile;
  const uint4* kb = reinterpret_cast<const uint4*>(k_cmp + (size_t)b * nbp * kIdxDim);
  for (int i = tid; i < kStreamQ * kHistWords; i += blockDim.x) (&s_h[0][0])[i] = 0u;
  if (tid < kStreamQ) {
    s_hc[tid] = 0u;
    s_mx[tid] = 0u;
    s_cnt[tid] = 0u;
  }

  if (wave == 4) {
    // ---------------- loader
    for (int t = 0; t < kRing - 1; ++t) dma_tile(ring[t], kb, t, bt_wg);
    stream_barrier_loader();
    for (int k = 0; k < ntiles; ++k) {
      dma_tile(ring[(k + kRing - 1) % kRing], kb, k + kRing - 1, bt_wg);
      stream_barrier_loader();
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no DMA may outlive the workgroup
    return;
  }

  // ---------------- compute wavefronts
  const int wq0 = qbase + wave * 16;
  Stream st;
  st.h = &s_h[wave * 16];
  st.hc = &s_hc[wave * 16];
  st.mx = &s_mx[wave * 16];
  st.cnt = &s_cnt[wave * 16];
  st.rs = s_rs[wave];
  st.queue = s_queue[wave];
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
  int bt_min = 0x7fffffff;
  st.tq0 = query_t(len, Nq, wq0 + (lane >> 5));
  st.nq_left = Nq - wq0 - (lane >> 5);
  // (lists of rows past the batch are never written: their slots never pass)
  st.lists = lists + ((size_t)b * Nq + wq0) * kListCap;
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int qq = wq0 + slot_query(rt, c);
      const int t = query_t(len, Nq, qq);
      bt_min = min(bt_min, (qq < Nq && t >= 0) ? (t >> 2) : 0);
      st.tau_l[rt][c] = -1.f;
    }
  // tiles entirely below every query's own block need no causal mask
  for (int off = 32; off >= 1; off >>= 1) bt_min = min(bt_min, __shfl_xor(bt_min, off));
  st.tau_v = (int)0xbf800000u;  // bits of -1.0f (as int: negative, below every score)
  st.base_v = 0;
  st.trig_v = kTopK + kHyst;
  // Settle the A-fragment loads now, so no wait on vector memory (which
  // would also wait for the list appends) is needed inside the tile loop.
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
  stream_barrier_compute();

  // Pipeline over 32-block halves: the MFMAs of the next half run, and its
  // key fragments are read from LDS, while the current half is filtered.
  // Three loops: the first tile, the tiles below every query's own block
  // (no causal mask), and the last tiles (masked).
  f32x16 accA[2], accB[2];
  int qn = 0;  // survivors queued, not yet drained
  if (ntiles > 0) {
    bf16x8 bf[4];
    load_b(ring[0], 0, bf);
    mma_half(bf, A, accA);
  }
  const int nfull = min(ntiles, bt_min / kStreamTile);
  if (ntiles > 0) {
    if (nfull > 0)
      stream_step<true, true>(st, A, ring, accA, accB, 0, ntiles, qn);
    else
      stream_step<true, false>(st, A, ring, accA, accB, 0, ntiles, qn);
  }
  for (int k = 1; k < nfull; ++k) stream_step<false, true>(st, A, ring, accA, accB, k, ntiles, qn);
  for (int k = max(1, nfull); k < ntiles; ++k)
    stream_step<false, false>(st, A, ring, accA, accB, k, ntiles, qn);
  if (qn > 0) stream_drain<false>(st, qn);
  wave_sync_lds();
  if (lane < 16 && wq0 + lane < Nq) list_cnt[(size_t)b * Nq + wq0 + lane] = st.cnt[lane];
  if (lane < 16 && wq0 + lane < Nq) tau_out[(size_t)b * Nq + wq0 + lane] = st.tau_v;
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
int table_stride(const Dims& d) { return ((d.Lmax / 4) + 3) & ~3; }
int group_stride(const Dims& d) { return (((d.Lmax / 4) + kGroup - 1) / kGroup + 3) & ~3; }
// Filter slices: at most 256 per row (the select kernel walks one segment per
// thread pair or more), each a multiple of kFilterSlice blocks.
int filter_slice(const Dims& d) {
  const long long nbp = d.Lmax / 4;
  const long long per = (nbp + 255) / 256;
  return (int)((per + kFilterSlice - 1) / kFilterSlice * kFilterSlice);
}
int filter_slices(const Dims& d) { return (int)((d.Lmax / 4 + filter_slice(d) - 1) / filter_slice(d)); }
struct TableWs {
  uint32_t* scores;
  uint32_t* gmax;
  uint32_t* thr;
  uint32_t* cand_cnt;  // [rows][filter slices], written by the filter
  uint64_t* cand;      // [rows][filter slices][filter slice]
};
struct StreamWs {
  uint64_t* lists;
  uint32_t* cnt;
  int32_t* tau;
};
TableWs carve_table(const Dims& d, void* ws, size_t* total) {
  Carve c{static_cast<char*>(ws), 0};
  const size_t rows = (size_t)d.B * d.Nq;
  TableWs w;
  w.scores = c.take<uint32_t>(rows * (size_t)table_stride(d));
  w.gmax = c.take<uint32_t>(rows * (size_t)group_stride(d));
  w.thr = c.take<uint32_t>(rows);
  w.cand_cnt = c.take<uint32_t>(rows * filter_slices(d));
  w.cand = c.take<uint64_t>(rows * (size_t)filter_slices(d) * filter_slice(d));
  if (total) *total = c.off;
  return w;
}
StreamWs carve_stream(const Dims& d, void* ws, size_t* total) {
  Carve c{static_cast<char*>(ws), 0};
  const size_t rows = (size_t)d.B * d.Nq;
  StreamWs w;
  w.lists = c.take<uint64_t>(rows * kListCap);
  w.cnt = c.take<uint32_t>(rows);
  w.tau = c.take<int32_t>(rows);
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

void topk_zero_range(const Dims& d, TopkPath path, void* ws, uint32_t** ptr, size_t* n) {
  if (path == TopkPath::kTable) {
    (void)ws;  // nothing to clear: every count is written by the filter
    *ptr = nullptr;
    *n = 0;
  } else {
    *ptr = nullptr;
    *n = 0;
  }
}

hipError_t launch_index_topk(const Dims& d, TopkPath path, const uint16_t* q_idx,
                             const uint16_t* k_cmp, const int32_t* lens, int32_t* sel,
                             int32_t* n_sel, void* ws, bool ws_zeroed, hipStream_t s) {
  if (d.B == 0 || d.Nq == 0) return hipSuccess;
  const dim3 grid_q((unsigned)d.Nq, (unsigned)d.B);
  if (path == TopkPath::kTable) {
    TableWs w = carve_table(d, ws, nullptr);
    const int ts = table_stride(d), gs = group_stride(d);
    const int fs = filter_slice(d), nfs = filter_slices(d);
    const size_t rows = (size_t)d.B * d.Nq;
    (void)ws_zeroed;
    const unsigned qg = (unsigned)((d.Nq + 3) / 4);
    const dim3 grid_s((unsigned)((d.Lmax / 4 + kTableSlice - 1) / kTableSlice), qg, (unsigned)d.B);
    QSA_LAUNCH(score_table_kernel, grid_s, dim3(256), 0, s, q_idx, k_cmp, lens, w.scores, ts,
               w.gmax, gs, d.Lmax, d.Nq);
    QSA_LAUNCH(table_threshold_kernel, dim3((unsigned)rows), dim3(kThrThreads), 0, s, w.gmax, gs,
               lens, w.thr, d.Lmax, d.Nq);
    QSA_LAUNCH(table_filter_kernel, dim3((unsigned)nfs, qg, (unsigned)d.B), dim3(256), 0, s,
               w.scores, ts, w.thr, lens, w.cand, w.cand_cnt, d.Lmax, d.Nq, fs);
    QSA_LAUNCH(select_kernel<false>, grid_q, dim3(256), 0, s, w.cand, w.cand_cnt, nfs, fs,
               (const int32_t*)nullptr, w.scores, ts, q_idx, k_cmp, lens, sel, n_sel, d.Lmax,
               d.Nq);
  } else {
    StreamWs w = carve_stream(d, ws, nullptr);
    const dim3 grid((unsigned)((d.Nq + kStreamQ - 1) / kStreamQ), (unsigned)d.B);
    QSA_LAUNCH(score_stream_kernel, grid, dim3(320), 0, s, q_idx, k_cmp, lens, w.lists, w.cnt,
               w.tau, d.Lmax, d.Nq);
    QSA_LAUNCH(select_kernel<true>, grid_q, dim3(256), 0, s, w.lists, w.cnt, 1, kListCap,
               (const int32_t*)w.tau, (const uint32_t*)nullptr, 0, q_idx, k_cmp, lens, sel, n_sel,
               d.Lmax, d.Nq);
  }
  return hipGetLastError();
}

}  // namespace qsa
