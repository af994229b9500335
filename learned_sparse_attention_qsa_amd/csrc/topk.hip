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
// Three engines, with bit-identical results:
//
//  TABLE (few queries, decode-shaped): one streaming pass scores every block
//  with MFMA (16x16x32, 4 queries x 4 heads per tile) and writes the fp32
//  score table plus, for every 16-block group, the group's best score.  Any
//  value that 512 group maxima reach is reached by 512 distinct blocks, so it
//  bounds the row's 512th best score from below.  One workgroup per row then
//  finds such a bound from the group maxima, lists the groups that reach it,
//  reads only those groups' scores back from the table (typically 700 of
//  the row's 16,384 groups at 1M context), and finds the exact top 512 among
//  the blocks that reach it by histogram passes, with no sort: the list is
//  built in ascending block order and compacted in place.  Cost over the
//  bare k_cmp scan: the score table (4 B per query per block) written once.
//
//  STREAM (many queries, prefill-shaped): a workgroup holds 64 queries x 4
//  heads stationary in registers and streams a fragment-ordered copy of the
//  compressed keys straight into registers in tiles of 32 blocks, MFMA
//  32x32x16.  A first pass over 1/32 of the tiles sets each query's bound
//  tau (the lower bin edge of its 40th best sample score); the second pass
//  keeps the blocks scoring strictly above tau (about 1,400 per query).  If
//  at least 512 blocks pass, no block at or below tau can be in the top 512;
//  the select kernel checks this, finds the 512th key by an LDS radix select
//  and sorts the winners' ids.  No score table is written.
//
//  SCAN (few queries at contexts whose score table would not fit): every
//  workgroup bounds its queries from the same 1,024 sample blocks of the
//  sequence, streams its slice with MFMA 16x16x32 and keeps the blocks
//  reaching the bound in a per-slice segment, written in ascending block
//  order; one workgroup per row then finds the exact top 512 in the
//  concatenated segments, already ascending, with no sort.
//
// Rows whose candidates cannot be trusted or held (an overflow, too few
// candidates, or very many equal scores) are finished by an exact fallback
// that recomputes or re-reads the whole row.

#include "common.h"
#include "internal.h"

namespace qsa {
namespace {

constexpr int kHistBins = 2048;    // histogram bins of the table engine's pick
constexpr int kGroup = 16;         // blocks per group maximum (table engine)
constexpr int kSelCap = 4096;      // candidates a select workgroup holds in LDS (a stream list)
constexpr int kHistW = 256;        // stream engine: sample-histogram bins per query
constexpr int kStreamQ = 64;       // queries per stream workgroup (two groups of 32)
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

// Histogram increment of bin d for every lane with `active`: the lanes that
// share the first active lane's bin add their count with one LDS atomic, the
// others one each.  Keys that agree on a digit (the leading digits of similar
// scores) then cost one atomic per wavefront instead of 64 on one address,
// and diverse digits cost no more than plain atomics.  Every lane of the
// wavefront must reach the call (active may differ per lane).
__device__ __forceinline__ void hist_add_wave(uint32_t* hist, uint32_t d, bool active) {
  const uint64_t act = __ballot(active);
  if (act == 0) return;
  const int leader = __builtin_amdgcn_readfirstlane(__ffsll((long long)act) - 1);
  const uint32_t dl = (uint32_t)__builtin_amdgcn_readlane((int)d, leader);
  const bool same = active && d == dl;
  const uint64_t m = __ballot(same);
  if (lane_id() == leader) atomicAdd(&hist[dl], (uint32_t)__popcll(m));
  if (active && !same) atomicAdd(&hist[d], 1u);
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
// LDS, by most-significant-digit radix select over 8-bit digits.  Once the
// digit's bin holds exactly the keys still needed, the k-th largest is the
// smallest of them and the remaining digits are skipped (one pass for the
// minimum instead).  bcast: 3 words of LDS, mn: one 64-bit LDS word.
__device__ uint64_t block_kth_largest(const uint64_t* keys, int n, uint32_t k, uint32_t* hist,
                                      uint32_t* bcast, uint64_t* mn) {
  uint64_t prefix = 0, pmask = 0;
  const int tid = threadIdx.x;
  for (int shift = 56; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += blockDim.x) hist[i] = 0;
    __syncthreads();
    for (int i0 = 0; i0 < n; i0 += blockDim.x) {
      const int i = i0 + tid;
      const uint64_t key = i < n ? keys[i] : 0ull;
      hist_add_wave(hist, (uint32_t)(key >> shift) & 255u, i < n && (key & pmask) == prefix);
    }
    __syncthreads();
    if (tid < 64) {
      uint32_t d, above;
      wave_find_digit(hist, k, d, above);
      if (tid == 0) {
        bcast[0] = d;
        bcast[1] = above;
        bcast[2] = hist[d];
        *mn = ~0ull;
      }
    }
    __syncthreads();
    k -= bcast[1];
    prefix |= (uint64_t)bcast[0] << shift;
    pmask |= 0xffull << shift;
    if (bcast[2] == k && shift > 0) {
      // every key with this prefix is among the k largest: the k-th is the
      // smallest of them (reduced per wavefront, then one atomic each)
      uint64_t m = ~0ull;
      for (int i = tid; i < n; i += blockDim.x) {
        const uint64_t key = keys[i];
        if ((key & pmask) == prefix) m = key < m ? key : m;
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)m, off);
        const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(m >> 32), off);
        const uint64_t o = ((uint64_t)hi << 32) | lo;
        m = o < m ? o : m;
      }
      if ((tid & 63) == 0 && m != ~0ull) atomicMin(mn, m);
      __syncthreads();
      return *mn;
    }
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

// ------------------------------------------------------------------ select
// Exact top-512 of one query straight from its whole row.  Slow path for
// rows whose candidate list does not fit the fast path (very many equal or
// near-equal scores).  kRecompute: no score table exists (stream engine),
// scores are recomputed from q_idx and k_cmp.  The 512th best key is
// (v, the lowest indices among scores equal to v): an LDS radix select over
// the 32 score bits (four passes of 8 bits, each ending early once the
// chosen digit's bin holds exactly the keys still needed, or once every
// score left in play is equal) gives v's prefix and how many of the scores
// equal to it are needed; a last walk over the blocks in ascending order
// keeps every higher score and the first that many equal ones, and stops
// once 512 are kept (an all-equal row ends after its first 512 blocks).
// hist: 256 words; bcast: 6 words; wsum: two words per wavefront.
template <bool kRecompute>
__device__ void select_whole_row(const uint32_t* trow, const uint16_t* qrow, const uint16_t* kc,
                                 int bt, int32_t* srow, float* qf, uint32_t* hist,
                                 uint32_t* bcast, uint32_t* wsum) {
  const int tid = threadIdx.x;
  const int nw = (int)(blockDim.x >> 6);
  if (kRecompute) {
    for (int i = tid; i < kIdxHeads * kIdxDim; i += blockDim.x)
      qf[i] = __uint_as_float((uint32_t)qrow[i] << 16);
    __syncthreads();
  }
  // score bits of block j (dims accumulated in order, as a scalar dot would)
  auto score_of = [&](int j) -> uint32_t {
    if (!kRecompute) return trow[j];
    const uint4* kr = reinterpret_cast<const uint4*>(kc + (size_t)j * kIdxDim);
    // (an opaque copy of the query pointer, so that the 256 query values are
    // read from LDS per block instead of being held in registers)
    typedef __attribute__((address_space(3))) const float lds_float;
    lds_float* qv = (lds_float*)qf;
    asm volatile("" : "+v"(qv));
    float d0 = 0.f, d1 = 0.f, d2 = 0.f, d3 = 0.f;
#pragma unroll 2
    for (int c = 0; c < kIdxDim / 8; ++c) {
      const uint4 u = kr[c];
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t h = w[e >> 1];
        const float kv = __uint_as_float((e & 1) ? (h & 0xffff0000u) : (h << 16));
        const int dd = c * 8 + e;
        d0 = fmaf(qv[dd], kv, d0);
        d1 = fmaf(qv[kIdxDim + dd], kv, d1);
        d2 = fmaf(qv[2 * kIdxDim + dd], kv, d2);
        d3 = fmaf(qv[3 * kIdxDim + dd], kv, d3);
      }
    }
    return relu_sum_bits(d0, d1, d2, d3);
  };
  uint32_t prefix = 0, pmask = 0;
  uint32_t k = kTopK;  // keys still needed among those matching the prefix
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += blockDim.x) hist[i] = 0;
    if (tid == 0) {
      bcast[4] = 0xffffffffu;  // min, max of the scores matching the prefix
      bcast[5] = 0u;
    }
    __syncthreads();
    uint32_t mn = 0xffffffffu, mx = 0u;
    for (int j0 = 0; j0 < bt; j0 += blockDim.x) {
      const int j = j0 + tid;
      const uint32_t sb = j < bt ? score_of(j) : 0u;
      const bool in = j < bt && (sb & pmask) == prefix;
      hist_add_wave(hist, (sb >> shift) & 255u, in);
      if (in) {
        mn = min(mn, sb);
        mx = max(mx, sb);
      }
    }
    for (int off = 32; off >= 1; off >>= 1) {
      mn = min(mn, (uint32_t)__shfl_xor((int)mn, off));
      mx = max(mx, (uint32_t)__shfl_xor((int)mx, off));
    }
    if ((tid & 63) == 0) {
      atomicMin(&bcast[4], mn);
      atomicMax(&bcast[5], mx);
    }
    __syncthreads();
    if (tid < 64) {
      uint32_t d, above;
      wave_find_digit(hist, k, d, above);
      if (tid == 0) {
        bcast[0] = d;
        bcast[1] = above;
        bcast[2] = hist[d];
      }
    }
    __syncthreads();
    if (bcast[4] == bcast[5]) {  // every score in play is the same value
      prefix = bcast[4];
      pmask = 0xffffffffu;
      __syncthreads();
      break;
    }
    k -= bcast[1];
    prefix |= bcast[0] << shift;
    pmask |= 0xffu << shift;
    const bool exact = bcast[2] == k;  // the bin holds exactly the keys needed
    __syncthreads();
    if (exact) break;
  }
  // blocks in ascending order: every score above the prefix range, and the
  // first k of those inside it
  const int lane = lane_id(), wave = tid >> 6;
  uint32_t kept = 0, eq_seen = 0;
  for (int base = 0; base < bt && kept < (uint32_t)kTopK; base += blockDim.x) {
    const int j = base + tid;
    uint32_t sb = 0;
    if (j < bt) sb = score_of(j);
    const bool in = j < bt;
    const bool gt = in && (sb & pmask) > prefix;
    const bool eq = in && (sb & pmask) == prefix;
    const uint64_t mg = __ballot(gt), me = __ballot(eq);
    if (lane == 0) {
      wsum[2 * wave] = (uint32_t)__popcll(mg);
      wsum[2 * wave + 1] = (uint32_t)__popcll(me);
    }
    __syncthreads();
    uint32_t eq_before = eq_seen, eq_all = 0, kept_before = kept;
    for (int w = 0; w < nw; ++w) {
      if (w < wave) eq_before += wsum[2 * w + 1];
      eq_all += wsum[2 * w + 1];
    }
    const uint32_t my_eq = eq_before + (uint32_t)__popcll(me & lanemask_lt());
    const bool keep = gt || (eq && my_eq < k);
    // kept in this chunk: every gt, and the equal ones still needed
    const uint64_t mk = __ballot(keep);
    __syncthreads();
    if (lane == 0) wsum[2 * wave] = (uint32_t)__popcll(mk);
    __syncthreads();
    uint32_t kept_all = 0;
    for (int w = 0; w < nw; ++w) {
      if (w < wave) kept_before += wsum[2 * w];
      kept_all += wsum[2 * w];
    }
    if (keep) {
      const uint32_t pos = kept_before + (uint32_t)__popcll(mk & lanemask_lt());
      if (pos < (uint32_t)kTopK) srow[pos] = j;
    }
    kept += kept_all;
    eq_seen += eq_all;
    __syncthreads();
  }
}

// One workgroup per query row.  Fast path: the row's candidates (nsub
// segments of up to seg_cap keys, segment lengths in cand_cnt; only keys whose
// score reaches the row's final threshold, when one is given) go to LDS, a
// radix select finds the 512th key and the winners' ids are sorted.  (A full
// sort of the candidates costs about twice as much at the ~1,400 candidates
// of a 1M-context row.)  Rows with too few or too many candidates take the
// exact whole-row path.
template <bool kRecompute>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void select_kernel(
    const uint64_t* __restrict__ cand, const uint32_t* __restrict__ cand_cnt, int nsub,
    int seg_cap, const int32_t* __restrict__ tau_final, const uint32_t* __restrict__ table,
    int tstride, const uint16_t* __restrict__ q_idx, const uint16_t* __restrict__ k_cmp,
    const int32_t* __restrict__ lens, int32_t* __restrict__ sel, int32_t* __restrict__ n_sel,
    int Lmax, int Nq) {
  __shared__ uint64_t keys[kSelCap];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t bcast[6];
  __shared__ uint64_t s_min;
  __shared__ int32_t outb[kTopK];
  __shared__ uint32_t outn;
  __shared__ uint32_t bad;
  __shared__ float qf[kIdxHeads * kIdxDim];
  __shared__ uint32_t wsum[8];
  const int q = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const size_t row = (size_t)b * Nq + q;
  // threads_per_seg threads walk each segment; the segment length is read
  // before (and independently of) lens
  const int tps = blockDim.x / nsub;
  const int seg = tid / tps, sub = tid % tps;
  const uint32_t n_seg_raw = seg < nsub ? cand_cnt[row * nsub + seg] : 0u;
  const int t = query_t(guard_len(lens[b], Nq, Lmax), Nq, q);
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
    // the 512th best key by an LDS radix select, then the keys at or above
    // it (exactly 512: keys are distinct) and their ids sorted ascending
    const uint64_t kth = block_kth_largest(keys, (int)n, kTopK, hist, bcast, &s_min);
    if (tid == 0) outn = 0;
    __syncthreads();
    for (uint32_t i = tid; i < n; i += blockDim.x) {
      const uint64_t key = keys[i];
      if (key >= kth) outb[atomicAdd(&outn, 1u)] = (int32_t)key_block(key);
    }
    __syncthreads();
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
// Grid (ceil(Lmax/4 / (4 kSpan)), ceil(Nq/4), B), 256 threads: a slice of
// 4 kSpan blocks per workgroup, the span chosen so that the grid fills the
// chip (256 at long contexts, shorter below).  Wavefront w scores blocks
// [j_begin + kSpan w, + kSpan) in batches of up to eight 16-block tiles.
// MFMA 16x16x32: A = 16 rows (query r/4, head r%4), B = 16 blocks;
// the lane (r, kc) receives block r of the tile for query q0 + kc, all four
// heads.  A tile is also one group: its maximum over the 16 lanes of a query
// goes to gmax.
//
// With k_idx given (one workgroup row covers all of a sequence's queries),
// the pass also compresses the sequence's new blocks [first_block, len/4):
// each workgroup writes those of its slice to k_cmp before scoring them
// (the vector L1 is shared by the workgroup's wavefronts, so a barrier
// orders the writes before the reads).
template <int kSpan>
__global__ __launch_bounds__(256) void score_table_kernel(const uint16_t* __restrict__ q_idx,
                                                          uint16_t* __restrict__ k_cmp,
                                                          const int32_t* __restrict__ lens,
                                                          uint32_t* __restrict__ scores,
                                                          int tstride,
                                                          uint32_t* __restrict__ gmax,
                                                          int gstride, int Lmax, int Nq,
                                                          const uint16_t* __restrict__ k_idx,
                                                          const int32_t* __restrict__ first_block) {
  const int slice = blockIdx.x, q0 = blockIdx.y * 4, b = blockIdx.z;
  const int len = guard_len(lens[b], Nq, Lmax);
  const int nbp = Lmax >> 2;
  const int t_last = query_t(len, Nq, min(q0 + 3, Nq - 1));
  constexpr int kSlice = 4 * kSpan;
  const int j_begin = slice * kSlice;
  const int j_end = min(j_begin + kSlice, t_last >= 0 ? (t_last >> 2) : 0);
  if (k_idx != nullptr) {
    const int nb = len >> 2;
    const int fb = first_block ? guard(first_block[b], 0, nb) : 0;
    const long long c0 = (long long)max(fb, j_begin) * 8;
    const long long c1 = (long long)min(nb, j_begin + kSlice) * 8;
    if (c0 < c1) {  // (uniform over the workgroup)
      const uint4* src = reinterpret_cast<const uint4*>(k_idx + (size_t)b * Lmax * kIdxDim);
      uint4* dst = reinterpret_cast<uint4*>(k_cmp + (size_t)b * nbp * kIdxDim);
      for (long long g = c0 + threadIdx.x; g < c1; g += blockDim.x)
        dst[g] = compress_chunk(src + (g >> 3) * 32 + (g & 7));
      __syncthreads();
    }
  }
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

  constexpr int U = kSpan >= 128 ? 8 : kSpan / 16;  // tiles per batch
  constexpr int kBatches = kSpan / (16 * U);
  static_assert(kBatches * U * 16 == kSpan, "whole batches per wavefront");
#pragma unroll 1
  for (int batch = 0; batch < kBatches; ++batch) {
    const int jt = j_begin + wave * kSpan + batch * (U * 16);
    if (jt >= j_end) break;
    // Unconditional loads (a block past the slice re-reads the slice's last
    // one; its score is masked below): with per-lane conditions the
    // compiler's wait before the first MFMA covers nearly the whole batch.
    uint4 bv[U][2];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = min(jt + u * 16 + r, j_end - 1);
      bv[u][0] = kb[(size_t)j * 8 + kc];
      bv[u][1] = kb[(size_t)j * 8 + 4 + kc];
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

// ------------------------------------------------------------------ PICK
// Table engine, after the scoring pass: one workgroup (1,024 threads) per
// query row turns the row's group maxima and score table into its selection.
// Scores are non-negative, so bins of a linear scale order them; every
// decision below is taken on such bins or on exact score bits.
//
//  1. bound: with G >= 512 groups, any value that 512 group maxima reach is
//     reached by 512 distinct blocks, so it is a lower bound of the row's
//     512th best score.  Each thread holds 16 consecutive maxima; a histogram
//     of the per-thread maxima finds the bin of their 512th largest, and the
//     smallest per-thread maximum in that bin or above is the bound bv.
//  2. candidate groups: the groups whose maximum reaches bv, listed in
//     ascending order by a block-wide prefix count.
//  3. candidates: the blocks of those groups whose score reaches bv,
//     read from the score table 16 B at a time, listed in ascending order
//     (typically 600 to 800).
//  4. cutoff: the exact 512th best key among the candidates.  A finer scale
//     over the candidates' range finds its bin; a bin holding one score value
//     (the usual case for integer scores) settles it, otherwise passes over
//     the score bits, 11 at a time, do.
//  5. output: blocks above the cutoff, plus the lowest-index blocks at the
//     cutoff score, compacted in list order, which is ascending.
// Rows of at most kPickCand blocks skip steps 2 and 3: every block is a
// candidate, read straight from the table.  A row whose candidate groups or
// blocks exceed the LDS lists (many equal scores) is finished by the exact
// whole-row select.
constexpr int kPickThreads = 1024;
constexpr int kPickWaves = kPickThreads / 64;  // 16: one lane of a 16-lane row each
constexpr int kPickGroups = 2048;  // candidate groups a row keeps in LDS
constexpr int kPickCand = 2048;    // candidate blocks a row keeps in LDS (2 per thread)
constexpr int kPickRounds = kPickGroups / (kPickThreads / 4);
constexpr int kPickDirectGroups = 1536;  // rows of fewer groups (and > kPickCand blocks): bound from block scores
static_assert(kPickWaves == 16, "per-wavefront values are combined within one 16-lane row");

// Wavefront primitives on DPP lane moves, which need no LDS traffic.
// Controls: row_shr:n = 0x110 + n, row_bcast:15 = 0x142, row_bcast:31 =
// 0x143.  Lanes whose source is outside the row, or whose row is masked off,
// receive `old`.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ uint32_t dpp_mov(uint32_t old, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, kCtrl, kRowMask, 0xf, false);
}
__device__ __forceinline__ uint32_t lane_read(uint32_t v, int l) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, l);
}
// Inclusive prefix sum within each row of 16 lanes.
__device__ __forceinline__ uint32_t row_incl_sum(uint32_t v) {
  v += dpp_mov<0x111, 0xf>(0u, v);
  v += dpp_mov<0x112, 0xf>(0u, v);
  v += dpp_mov<0x114, 0xf>(0u, v);
  v += dpp_mov<0x118, 0xf>(0u, v);
  return v;
}
// Inclusive prefix sum over the wavefront.
__device__ __forceinline__ uint32_t wave_incl_sum(uint32_t v) {
  v = row_incl_sum(v);
  v += dpp_mov<0x142, 0xa>(0u, v);
  v += dpp_mov<0x143, 0xc>(0u, v);
  return v;
}
// Running maximum / minimum: lane 15 of each row holds its row's, lane 63
// the wavefront's.
__device__ __forceinline__ uint32_t row_scan_max(uint32_t v) {
  v = max(v, dpp_mov<0x111, 0xf>(v, v));
  v = max(v, dpp_mov<0x112, 0xf>(v, v));
  v = max(v, dpp_mov<0x114, 0xf>(v, v));
  v = max(v, dpp_mov<0x118, 0xf>(v, v));
  return v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = row_scan_max(v);
  v = max(v, dpp_mov<0x142, 0xa>(v, v));
  v = max(v, dpp_mov<0x143, 0xc>(v, v));
  return lane_read(v, 63);
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, dpp_mov<0x111, 0xf>(v, v));
  v = min(v, dpp_mov<0x112, 0xf>(v, v));
  v = min(v, dpp_mov<0x114, 0xf>(v, v));
  v = min(v, dpp_mov<0x118, 0xf>(v, v));
  v = min(v, dpp_mov<0x142, 0xa>(v, v));
  v = min(v, dpp_mov<0x143, 0xc>(v, v));
  return lane_read(v, 63);
}
// After every wavefront w has stored a count in slot[w] (and a barrier): the
// sum over the wavefronts below `wave` and the total.  `wave` is uniform.
__device__ __forceinline__ void waves_prefix(const uint32_t* slot, int wave, uint32_t& below,
                                             uint32_t& total) {
  const uint32_t sc = row_incl_sum(slot[threadIdx.x & 15]);
  total = lane_read(sc, 15);
  const uint32_t incl = lane_read(sc, wave > 0 ? wave - 1 : 0);
  below = wave > 0 ? incl : 0u;
}

// Whole workgroup of kPickThreads: over kHistBins bins in LDS (bin order =
// value order), the highest bin whose suffix count reaches k (the caller
// guarantees the total does), the count in the bins above it and its own
// count.  Thread t owns bins 2t and 2t+1.  Ends past a barrier.
__device__ __forceinline__ void pick_suffix_find(const uint32_t* h, uint32_t k, uint32_t* wtot,
                                                 uint4* res, uint32_t& bin, uint32_t& above,
                                                 uint32_t& count) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint2 c = reinterpret_cast<const uint2*>(h)[tid];
  const uint32_t mine = c.x + c.y;
  const uint32_t P = wave_incl_sum(mine);  // lanes up to this one
  const uint32_t wt = lane_read(P, 63);
  if (lane == 0) wtot[wave] = wt;
  __syncthreads();
  const uint32_t sc = row_incl_sum(wtot[lane & 15]);
  const uint32_t hi = lane_read(sc, 15) - lane_read(sc, wave);  // wavefronts above
  const uint32_t suf1 = hi + (wt - P) + c.y;  // suffix count from bin 2t+1
  const uint32_t suf0 = suf1 + c.x;           // from bin 2t
  if (suf1 >= k && suf1 - c.y < k)
    res[0] = make_uint4(2 * tid + 1, suf1 - c.y, c.y, 0u);
  else if (suf0 >= k && suf1 < k)
    res[0] = make_uint4(2 * tid, suf1, c.x, 0u);
  __syncthreads();
  const uint4 r = res[0];
  bin = r.x;
  above = r.y;
  count = r.z;
}

// Shift that maps spans up to `span` into kHistBins bins.
__device__ __forceinline__ uint32_t pick_shift(uint32_t span) {
  const uint32_t top = span >> 11;
  return top == 0 ? 0u : 32u - (uint32_t)__clz((int)top);
}

// Bin of a score on the linear scale (x - lo) * scale, clamped to the
// histogram; non-decreasing in x.
__device__ __forceinline__ uint32_t lin_bin(uint32_t bits, float lo, float scale) {
  const float f = (__uint_as_float(bits) - lo) * scale;
  return f > 0.f ? min((uint32_t)f, (uint32_t)(kHistBins - 1)) : 0u;
}

// This thread's 16 group maxima of chunk c (groups 16 (1024 c + t) .. + 15)
// and a mask of the valid ones (group < G).
__device__ __forceinline__ uint32_t pick_chunk(const uint4* g4, int n4, int G, int c,
                                               const uint4 (&first)[4], uint32_t (&x)[16]) {
  const int i4 = 4 * (c * kPickThreads + (int)threadIdx.x);
  uint4 v[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) v[u] = c == 0 ? first[u] : (i4 + u < n4 ? g4[i4 + u] : zero_u4());
  uint32_t vm = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    x[4 * u + 0] = v[u].x;
    x[4 * u + 1] = v[u].y;
    x[4 * u + 2] = v[u].z;
    x[4 * u + 3] = v[u].w;
#pragma unroll
    for (int e = 0; e < 4; ++e) vm |= (4 * (i4 + u) + e < G ? 1u : 0u) << (4 * u + e);
  }
  return vm;
}

__global__ __launch_bounds__(kPickThreads) void table_pick_kernel(
    const uint32_t* __restrict__ scores, int tstride, const uint32_t* __restrict__ gmax,
    int gstride, const int32_t* __restrict__ lens, int32_t* __restrict__ sel,
    int32_t* __restrict__ n_sel, int Lmax, int Nq) {
  __shared__ __align__(16) uint32_t hist[kHistBins];
  __shared__ uint32_t glist[kPickGroups];
  __shared__ uint32_t cbits[kPickCand];
  __shared__ uint32_t cj[kPickCand];
  __shared__ uint32_t wred[2][kPickWaves];
  __shared__ uint32_t wcnt[kPickRounds][kPickWaves];
  __shared__ uint32_t wtot[kPickWaves];
  __shared__ uint4 res[1];
  __shared__ uint32_t wsum[2 * kPickWaves];
  __shared__ uint32_t bcast[6];
  __shared__ uint32_t s_bv;
  __shared__ uint32_t s_mm[2];
  const int row = blockIdx.x, b = row / Nq, q = row - b * Nq, tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // the first chunk of group maxima is requested before lens arrives (a row
  // holds gstride >= G entries, gstride a multiple of 4)
  const uint4* g4 = reinterpret_cast<const uint4*>(gmax + (size_t)row * gstride);
  const int n4 = gstride >> 2;
  uint4 first[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int i = 4 * tid + u;
    first[u] = i < n4 ? g4[i] : zero_u4();
  }
  hist[tid] = 0u;
  hist[tid + kPickThreads] = 0u;
  if (tid == 0) {
    s_bv = 0xffffffffu;
    s_mm[0] = 0xffffffffu;
    s_mm[1] = 0u;
  }
  const int t = query_t(guard_len(lens[b], Nq, Lmax), Nq, q);
  int32_t* srow = sel + (size_t)row * kTopK;
  if (write_trivial(t, srow, n_sel + row)) return;
  const int bt = t >> 2;
  const int G = (bt + kGroup - 1) / kGroup;
  const int nchunks = (G + 16 * kPickThreads - 1) / (16 * kPickThreads);
  const uint32_t* trow = scores + (size_t)row * tstride;
  // Rows of at most kPickCand blocks: every block is a candidate, read
  // straight from the table (two per thread, requested now) instead of
  // through the candidate groups; the bound below stays 0 for them.
  const bool small = bt <= kPickCand;  // (uniform)
  uint32_t sm[2] = {0u, 0u};
  if (small) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int i = 2 * tid + e;
      sm[e] = i < bt ? trow[i] : 0u;
    }
  }

  // ---- 1. bound: bv, a value that at least 512 group maxima reach
  uint32_t m1 = 0;
  bool any = false;
  for (int c = 0; c < nchunks; ++c) {
    uint32_t x[16];
    const uint32_t vm = pick_chunk(g4, n4, G, c, first, x);
#pragma unroll
    for (int k = 0; k < 16; ++k) m1 = ((vm >> k) & 1u) ? max(m1, x[k]) : m1;
    any = any || vm != 0u;
  }
  {
    const uint32_t wmax = wave_max_u32(m1);
    const uint32_t nany = (uint32_t)__popcll(__ballot(any));
    if (lane == 0) {
      wred[0][wave] = wmax;
      wred[1][wave] = nany;
    }
  }
  __syncthreads();
  const uint32_t rowmax = lane_read(row_scan_max(wred[0][lane & 15]), 15);
  const uint32_t nthr = lane_read(row_incl_sum(wred[1][lane & 15]), 15);
  const float rowmax_f = __uint_as_float(rowmax);
  const float scale = rowmax != 0u ? 2047.0f / rowmax_f : 0.f;
  uint32_t bv = 0;
  if (G < kPickDirectGroups && bt > kPickCand) {
    // Too few groups for their maxima to bound the 512th score tightly (with
    // 512 groups the bound is the smallest maximum) while the row's blocks
    // exceed the candidate list: the bound comes from the block scores
    // themselves (a linear histogram of the row's scores, then the smallest
    // score in the bin of the 512th best or above).
    for (int j = tid; j < bt; j += kPickThreads) atomicAdd(&hist[lin_bin(trow[j], 0.f, scale)], 1u);
    __syncthreads();
    uint32_t bin_a, ab, cn;
    pick_suffix_find(hist, kTopK, wtot, res, bin_a, ab, cn);
    uint32_t mn = 0xffffffffu;
    for (int j = tid; j < bt; j += kPickThreads) {
      const uint32_t x = trow[j];
      if (lin_bin(x, 0.f, scale) >= bin_a) mn = min(mn, x);
    }
    mn = wave_min_u32(mn);
    if (lane == 0 && mn != 0xffffffffu) atomicMin(&s_bv, mn);
    __syncthreads();
    bv = s_bv;
  } else if (G >= kTopK) {
    // With >= 512 threads holding maxima, their per-thread maxima (distinct
    // groups) are counted, else every maximum; the smallest counted value in
    // the bins from the one holding the 512th largest up is reached by >= 512
    // groups.
    const bool per_thread = nthr >= (uint32_t)kTopK;
    if (per_thread) {
      if (any) atomicAdd(&hist[lin_bin(m1, 0.f, scale)], 1u);
    } else {
      for (int c = 0; c < nchunks; ++c) {
        uint32_t x[16];
        const uint32_t vm = pick_chunk(g4, n4, G, c, first, x);
#pragma unroll
        for (int k = 0; k < 16; ++k)
          if ((vm >> k) & 1u) atomicAdd(&hist[lin_bin(x[k], 0.f, scale)], 1u);
      }
    }
    __syncthreads();
    uint32_t bin_a, ab, cn;
    pick_suffix_find(hist, kTopK, wtot, res, bin_a, ab, cn);
    uint32_t mn = 0xffffffffu;
    if (per_thread) {
      if (any && lin_bin(m1, 0.f, scale) >= bin_a) mn = m1;
    } else {
      for (int c = 0; c < nchunks; ++c) {
        uint32_t x[16];
        const uint32_t vm = pick_chunk(g4, n4, G, c, first, x);
#pragma unroll
        for (int k = 0; k < 16; ++k)
          if (((vm >> k) & 1u) && lin_bin(x[k], 0.f, scale) >= bin_a) mn = min(mn, x[k]);
      }
    }
    mn = wave_min_u32(mn);
    if (lane == 0 && mn != 0xffffffffu) atomicMin(&s_bv, mn);
    __syncthreads();
    bv = s_bv;
  }

  // ---- 2. candidate groups, ascending
  uint32_t ng = 0;
  for (int c = 0; c < (small ? 0 : nchunks); ++c) {
    uint32_t x[16];
    const uint32_t vm = pick_chunk(g4, n4, G, c, first, x);
    uint32_t keep = 0;
#pragma unroll
    for (int k = 0; k < 16; ++k) keep |= (((vm >> k) & 1u) && x[k] >= bv ? 1u : 0u) << k;
    const uint32_t cnt = (uint32_t)__popc(keep);
    const uint32_t P = wave_incl_sum(cnt);
    if (c > 0) __syncthreads();  // wtot of the previous chunk has been read
    if (lane == 0) wtot[wave] = lane_read(P, 63);
    __syncthreads();
    uint32_t below, all;
    waves_prefix(wtot, wave, below, all);
    uint32_t p = ng + below + P - cnt;
    const uint32_t gi0 = 16u * (uint32_t)(c * kPickThreads + tid);
    while (keep) {
      const int k = __ffs(keep) - 1;
      keep &= keep - 1;
      if (p < (uint32_t)kPickGroups) glist[p] = gi0 + (uint32_t)k;
      ++p;
    }
    ng += all;
  }
  __syncthreads();

  // ---- 3. candidate blocks of those groups, ascending
  uint32_t n = small ? (uint32_t)bt : 0u;
  if (!small && ng <= (uint32_t)kPickGroups) {
    const int rounds = (int)((ng + kPickThreads / 4 - 1) / (kPickThreads / 4));
    const int quarter = tid & 3;
    uint4 v[kPickRounds];
    int j0[kPickRounds];
#pragma unroll
    for (int r = 0; r < kPickRounds; ++r) {
      const uint32_t slot = (uint32_t)(r * (kPickThreads / 4) + (tid >> 2));
      j0[r] = slot < ng ? (int)(glist[slot] * kGroup) + 4 * quarter : bt;
      v[r] = (r < rounds && j0[r] < bt) ? *reinterpret_cast<const uint4*>(trow + j0[r])
                                        : zero_u4();
    }
    uint32_t keep[kPickRounds], pre[kPickRounds];
#pragma unroll
    for (int r = 0; r < kPickRounds; ++r) {
      keep[r] = 0;
      pre[r] = 0;
      if (r >= rounds) continue;
      const uint32_t e4[4] = {v[r].x, v[r].y, v[r].z, v[r].w};
      uint32_t tot = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool k = j0[r] + e < bt && e4[e] >= bv;
        keep[r] |= (k ? 1u : 0u) << e;
        const uint64_t m = __ballot(k);
        pre[r] += (uint32_t)__popcll(m & lanemask_lt());
        tot += (uint32_t)__popcll(m);
      }
      if (lane == 0) wcnt[r][wave] = tot;
    }
    __syncthreads();
    // lane 16 i + w reads round (4 h + i)'s count of wavefront w: one row per round
    uint32_t sc[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
      sc[h] = rounds > 4 * h ? row_incl_sum(wcnt[4 * h + (lane >> 4)][lane & 15]) : 0u;
    uint32_t base = 0;
#pragma unroll
    for (int r = 0; r < kPickRounds; ++r) {
      if (r >= rounds) continue;
      const uint32_t s = sc[r >> 2];
      const int r16 = 16 * (r & 3);
      const uint32_t all = lane_read(s, r16 + 15);
      const uint32_t before = wave > 0 ? lane_read(s, r16 + (wave > 0 ? wave - 1 : 0)) : 0u;
      uint32_t p = base + before + pre[r];
      const uint32_t e4[4] = {v[r].x, v[r].y, v[r].z, v[r].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if ((keep[r] >> e) & 1u) {
          if (p < (uint32_t)kPickCand) {
            cbits[p] = e4[e];
            cj[p] = (uint32_t)(j0[r] + e);
          }
          ++p;
        }
      }
      base += all;
    }
    n = base;
  }
  __syncthreads();

  if (ng > (uint32_t)kPickGroups || n > (uint32_t)kPickCand) {
    // too many candidates for the lists (many equal scores): exact slow path
    select_whole_row<false>(trow, nullptr, nullptr, bt, srow, nullptr, hist, bcast, wsum);
    if (tid == 0) n_sel[row] = kTopK;
    return;
  }

  // ---- 4. the exact 512th best key among the n candidates
  uint32_t mb[2], mj[2];
  bool mv[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const uint32_t i = 2u * (uint32_t)tid + e;
    mv[e] = i < n;
    mb[e] = mv[e] ? (small ? sm[e] : cbits[i]) : 0u;
    mj[e] = mv[e] ? (small ? i : cj[i]) : 0u;
  }
  // the candidates' scale: [bv, rowmax]
  const float lo4 = __uint_as_float(bv);
  const float scale4 = rowmax_f > lo4 ? 2047.0f / (rowmax_f - lo4) : 0.f;
  uint32_t fb[2];
  hist[tid] = 0u;
  hist[tid + kPickThreads] = 0u;
  __syncthreads();
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    fb[e] = lin_bin(mb[e], lo4, scale4);
    if (mv[e]) atomicAdd(&hist[fb[e]], 1u);
  }
  __syncthreads();
  uint32_t cb, above, cnt;
  pick_suffix_find(hist, kTopK, wtot, res, cb, above, cnt);
  uint32_t k = (uint32_t)kTopK - above;  // still to take from bin cb
  // within bin cb: keep bits >= keep_from, and `ties` blocks at tie_bits
  uint32_t keep_from = 0, tie_bits = 0xffffffffu, ties = 0;
  if (cnt != k) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      if (mv[e] && fb[e] == cb) {
        atomicMin(&s_mm[0], mb[e]);
        atomicMax(&s_mm[1], mb[e]);
      }
    }
    __syncthreads();
    const uint32_t mn = s_mm[0], mx = s_mm[1];
    if (mn == mx) {
      keep_from = mn + 1;
      tie_bits = mn;
      ties = k;
    } else {
      // several score values share the bin: refine on the bits
      uint32_t lo = mn, width = mx - mn + 1u;
      uint32_t s = pick_shift(mx - mn);
      for (;;) {
        hist[tid] = 0u;
        hist[tid + kPickThreads] = 0u;
        __syncthreads();
#pragma unroll
        for (int e = 0; e < 2; ++e)
          if (mv[e] && fb[e] == cb && mb[e] >= lo && mb[e] - lo < width)
            atomicAdd(&hist[(mb[e] - lo) >> s], 1u);
        __syncthreads();
        uint32_t bn, ab2, cn2;
        pick_suffix_find(hist, k, wtot, res, bn, ab2, cn2);
        k -= ab2;
        lo += bn << s;
        if (cn2 == k) {  // the whole bin is kept
          keep_from = lo;
          break;
        }
        if (s == 0) {  // one score value: keep k of its blocks, lowest first
          keep_from = lo + 1;
          tie_bits = lo;
          ties = k;
          break;
        }
        width = 1u << s;
        s = s > 11 ? s - 11 : 0u;
      }
    }
  }

  // ---- 5. compaction in list order (ascending block ids)
  uint32_t gk[2], tk[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    gk[e] = mv[e] && (fb[e] > cb || (fb[e] == cb && mb[e] >= keep_from)) ? 1u : 0u;
    tk[e] = mv[e] && !gk[e] && fb[e] == cb && mb[e] == tie_bits ? 1u : 0u;
  }
  const uint32_t mine = (gk[0] + gk[1]) | ((tk[0] + tk[1]) << 16);
  const uint32_t S = wave_incl_sum(mine);
  // (the last find's reads of wtot are behind its barrier)
  if (lane == 0) wtot[wave] = lane_read(S, 63);
  __syncthreads();
  uint32_t before, all;
  waves_prefix(wtot, wave, before, all);
  uint32_t P = before + S - mine;  // exclusive prefix of this thread
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const uint32_t A = P & 0xffffu, T = P >> 16;
    const uint32_t pos = A + min(T, ties);
    if ((gk[e] || (tk[e] && T < ties)) && pos < (uint32_t)kTopK) srow[pos] = (int32_t)mj[e];
    P += gk[e] | (tk[e] << 16);
  }
  if (tid == 0) n_sel[row] = kTopK;
}

// ------------------------------------------------------------------ STREAM
// Stream engine.  A workgroup takes 64 queries in two groups of 32 and has
// 8 wavefronts, four per group (two per SIMD).  Wavefront w holds the A
// fragments of the 32 queries of group w / 4 (32 queries x 4 heads = 4 row
// tiles x 4 k-steps, stationary in registers) and walks the 32-block column
// tiles c with c mod 4 = w mod 4, loading each tile's B fragments
// (compressed keys) straight from memory into registers one tile ahead:
// every block is read by two wavefronts, and the scan needs no LDS staging
// and no barriers.  MFMA 32x32x16; the 32 queries form two halves of 16
// whose MFMAs and epilogues alternate (one half's epilogue runs under the
// other half's MFMAs), and the second wavefront on each SIMD fills the
// gaps.  Two phases over the same pipeline:
//
//  1. sample: about every 32nd column tile (c = 128 i + 33 p for the four
//     parities p).  The first sample tile of each parity sets each query's
//     histogram base (3 octaves below its best score there); then every
//     sample tile, the first ones again included, goes into the query's
//     histogram (256 bins, 64 per octave; higher scores count in the top
//     bin), and its bound tau is the lower edge of the bin holding its
//     kSampleRank-th best sample score.
//  2. filter: every tile; a block is a candidate if its score is strictly
//     above tau.  A lane with a candidate among its 8 scores queues one LDS
//     record of them; records are drained 64 at a time into the queries'
//     lists in HBM.
//
// tau is an estimate, so the result is verified, not assumed: if at least
// 512 blocks score strictly above tau, every block at or below tau is beaten
// by 512 others and the list holds the whole top 512; the select kernel then
// finishes exactly.  Otherwise (or if a list overflowed) that row takes the
// exact whole-row path.  With 1/32 of the blocks sampled and rank 40, about
// 40 x 32 = 1,280 blocks per query pass (plus those of the part of a bin
// below the 40th sample), and the bound fails only when over 40 of the
// samples lie above the true 512th score, about 1e-7 per query for
// independent scores.
constexpr int kListCap = 4096;    // candidate list entries per query
constexpr int kColTile = 32;      // blocks per MFMA column tile
constexpr int kPar = 4;           // column-tile parities: wavefronts per group of 32 queries
constexpr int kStreamWaves = 2 * kPar;
// sample column tiles: c = 128 i + 33 p for parity p (each parity's own
// tiles, about every 32nd tile)
constexpr int kSampleStride = 32 * kPar;
constexpr int kSampleStep = 33;
static_assert(kSampleStep % kPar == 1 && kSampleStep * (kPar - 1) < kSampleStride, "sample tiles");
constexpr int kSampleRank = 40;   // tau: the 40th best sample score (bin edge)
// sample histogram: bins of (score bits >> 17), i.e. 64 per octave, 256 bins =
// 4 octaves from a base 3 octaves (192 bins) below the best of the first
// tiles; higher samples count in the top bin
constexpr int kSampleShift = 17;
constexpr int kSampleBase = 192;
// records one position can add to a wavefront's queue (one per lane and
// half), plus fewer than 64 held over
constexpr int kQueue = 2 * 64 + 64;
constexpr int kHistWords = kHistW / 2 + 1;  // 256 packed 16-bit bins + the spare bin

__device__ __forceinline__ void stream_barrier() {
  // no wait on vector memory: the key prefetch stays in flight
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// The stream scorer reads the compressed keys in fragment order: a copy in
// which column tile c (32 blocks) is 4 KiB laid out as [k-step ks][lane l],
// 16 bytes each, lane l holding block 32c + (l & 31), dims 16 ks + 8 (l >> 5)
// .. + 8 -- the 32x32x16 MFMA's B operand.  A wavefront's fragment load then
// reads 1 KiB of consecutive bytes (8 cache lines) where the row-major cache
// needs 32 lines, which kept the texture path busy 92 % of the scan.
// frag_order_kernel writes the copy: one thread per 16-byte chunk of the
// sequence's blocks below its last query's own block.
constexpr int kFragTile = kColTile * 8;  // 16-byte chunks per column tile
__global__ __launch_bounds__(256) void frag_order_kernel(const uint4* __restrict__ src,
                                                         uint4* __restrict__ dst,
                                                         const int32_t* __restrict__ lens,
                                                         int Lmax, int Nq, int ncol_pad) {
  const int b = blockIdx.y;
  const int i = blockIdx.x * 256 + threadIdx.x;  // chunk index in the sequence
  const int j = i >> 3, d8 = i & 7;
  const int len = guard_len(lens[b], Nq, Lmax);
  const int nb = len > 0 ? ((len - 1) >> 2) : 0;  // blocks below the last query's own block
  if (j >= nb) return;
  const int nbp = Lmax >> 2;
  const uint4 v = src[(size_t)b * nbp * 8 + i];
  const int c = j >> 5, r = j & 31, ks = d8 >> 1, half = d8 & 1;
  dst[((size_t)b * ncol_pad + c) * kFragTile + ks * 64 + half * 32 + r] = v;
}

// B fragments of column tile c from the fragment-ordered copy (kb: the
// sequence's first tile), through a buffer resource over the tile.  A tile
// with no block below bt_g (the prefetch past the last one) gets a resource
// of size 0 and reads zeros; a partial tile is read whole: it lies inside the
// copy, and a column of the MFMA's B operand only reaches the scores of its
// own block, which are masked for blocks at or past bt_g whatever the bytes
// held there.  The masking is scalar work, so the lane offset voff (lane x
// 16 within a k-step) stays one loop-invariant register: rewriting an
// address register per tile made the compiler wait for the loads in flight
// that used it.
constexpr uint32_t kBufferConfig = 0x00020000u;  // raw 32-bit buffer, no swizzle
__device__ __forceinline__ void load_cols(const uint4* kb, int c, int bt_g, uint32_t voff,
                                          uint4 (&bv)[4]) {
  // (every operand is wavefront-uniform; readfirstlane lets the compiler
  // keep the descriptor in scalar registers, with no waterfall loop; the
  // 1 KiB k-steps go in the scalar offset)
  const int nrec = __builtin_amdgcn_readfirstlane(c * kColTile < bt_g ? kFragTile * 16 : 0);
  const uint64_t a = reinterpret_cast<uint64_t>(kb + (size_t)c * kFragTile);
  const uint64_t au = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(a >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      reinterpret_cast<void*>(au), (short)0, nrec, (int)kBufferConfig);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    bv[ks] =
        __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 1024 * ks, 0));
}

// MFMAs of half kHalf (row tiles 2 kHalf, 2 kHalf + 1) against one column tile.
template <int kHalf>
__device__ __forceinline__ void mma_rows(const uint4 (&bv)[4], const bf16x8 (&A)[4][4],
                                         f32x16 (&acc)[2]) {
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[r][i] = 0.f;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int r = 0; r < 2; ++r) acc[r] = mfma32(A[2 * kHalf + r][ks], as_bf16x8(bv[ks]), acc[r]);
}

__device__ __forceinline__ int rdl(int v, int lane) { return __builtin_amdgcn_readlane(v, lane); }

// Per-wavefront state.  Slot (rt, c) of a lane scores local query
// rt*8 + c*2 + (lane >> 5) of the group (0..31).
struct Stream {
  float tau_l[4][4];          // filter bound of the slot's query (phase 2)
  int base_l[4][4];           // histogram base of the slot's query (phase 1)
  int tq0;                    // position of local query (lane >> 5)
  int nq_left;                // queries of the batch from local query (lane >> 5) on
  uint64_t* lists;            // list of local query 0; query q at + q * kListCap
  uint32_t (*h)[kHistWords];  // the group's 32 sample histograms
  uint32_t* cnt;              // the group's 32 list lengths
  uint32_t* mx;               // the group's 32 best scores of the first sample tiles
  // this wavefront's records not yet drained (see filter_epilogue): 48 bytes
  // each, the scores of slots 0..3, of slots 4..7, then column tile << 7 |
  // half << 6 | lane
  uint4* rec;
  const int32_t* tau;         // the group's 32 bounds (LDS)
  uint32_t voff;              // byte offset of this lane's B fragment within a key tile
};

__device__ __forceinline__ int slot_off(int rt, int c) { return rt * 8 + c * 2; }

// Causal / batch mask of slot (rt, c) for block j.
__device__ __forceinline__ bool slot_valid(const Stream& st, int rt, int c, int j) {
  const int off = slot_off(rt, c);
  const int tq = st.tq0 + off;
  return (off < st.nq_left) & (tq >= 0) & (j < (tq >> 2));
}

// Phase 1 epilogue of one half: histogram the sample scores (the first sample
// tiles: track each query's best score instead).
template <bool kFirst, int kHalf>
__device__ __forceinline__ void sample_epilogue(Stream& st, const f32x16 (&acc)[2], int col) {
  const int lane = lane_id();
  const int j = col * kColTile + (lane & 31);
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int rt = 2 * kHalf + r;
      const uint32_t bits =
          relu_sum_bits(acc[r][4 * c], acc[r][4 * c + 1], acc[r][4 * c + 2], acc[r][4 * c + 3]);
      const bool valid = slot_valid(st, rt, c, j);
      const int q = slot_off(rt, c) + (lane >> 5);
      if (kFirst) {
        if (valid) atomicMax(&st.mx[q], bits);
      } else {
        const int bin = (int)(bits >> kSampleShift) - st.base_l[rt][c];
        if (valid && bin >= 0) {
          const int bb = min(bin, kHistW - 1);
          atomicAdd(&st.h[q][bb >> 1], 1u << ((bb & 1) * 16));
        }
      }
    }
}

// The filter's test value of a block: u = max(s01 + s23, s01, s23) with
// s01 = max(a + b, a, b) and s23 = max(c + d, c, d).  relu(x) + relu(y) =
// max(x + y, x, y, 0), with the same rounding as the sum of the relu'd
// values wherever it is not 0, so relu(u) is the block's score bit for bit
// and, for a bound tau >= 0 or tau = -inf, u > tau exactly when the score
// is.  Three 3-input maxima and three adds: one instruction fewer than four
// relus and three adds.
__device__ __forceinline__ float max3f(float x, float y, float z) {
  return __builtin_fmaxf(__builtin_fmaxf(x, y), z);
}
__device__ __forceinline__ float relu_sum_test(float a, float b, float c, float d) {
  const float s01 = max3f(a + b, a, b), s23 = max3f(c + d, c, d);
  return max3f(s01 + s23, s01, s23);
}

// Phase 2 epilogue of one half: the scores and the enqueue.  Survivors are
// rare (about 1 score in 200), so the scan only records where they are: a
// lane with any of its 8 slots above its query's bound appends one record
// (the 8 scores and the tile, half and lane they belong to) behind the qn
// already queued, its place a masked bit count of the wavefront's mask of
// such lanes.  No per-slot work, no branch but the skip of an empty half.
// The drain later re-tests the 8 scores of each record.  kFull: every block
// of the tile is below every query's own block; otherwise masked slots
// score -inf.
template <bool kFull, int kHalf>
__device__ __forceinline__ int filter_epilogue(Stream& st, const f32x16 (&acc)[2], int col,
                                               int qn) {
  const int lane = lane_id();
  const int j = col * kColTile + (lane & 31);
  float sc[8];
  // the mask of lanes to record, as the OR of the comparisons' own lane
  // masks (scalar work), and the branch taken on it directly: no per-lane
  // flag is materialised in a vector register
  uint64_t m = 0;
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int rt = 2 * kHalf + r;
      float v = relu_sum_test(acc[r][4 * c], acc[r][4 * c + 1], acc[r][4 * c + 2], acc[r][4 * c + 3]);
      if (!kFull) v = slot_valid(st, rt, c, j) ? v : kNegInf;
      sc[r * 4 + c] = v;
      m |= __builtin_amdgcn_ballot_w64(v > st.tau_l[rt][c]);
    }
  if (__builtin_amdgcn_inverse_ballot_w64(m)) {
    const uint32_t at =
        __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    // (the queue's end is scalar; a full-rate 24-bit multiply for the lane's place)
    uint4* rp = (st.rec + 3 * qn) + __umul24(at, 3u);
    rp[0] = make_uint4(__float_as_uint(sc[0]), __float_as_uint(sc[1]), __float_as_uint(sc[2]),
                       __float_as_uint(sc[3]));
    rp[1] = make_uint4(__float_as_uint(sc[4]), __float_as_uint(sc[5]), __float_as_uint(sc[6]),
                       __float_as_uint(sc[7]));
    reinterpret_cast<uint32_t*>(rp + 2)[0] =
        ((uint32_t)col << 7) | (uint32_t)(kHalf << 6) | (uint32_t)lane;
  }
  // (uniform: readfirstlane keeps the queue count scalar)
  return __builtin_amdgcn_readfirstlane(qn + (int)__popcll(m));
}

// Append the survivors of the qn queued records to their queries' lists, one
// record per lane: slot k of a record from lane l of half h scores block
// 32 tile + l % 32 for local query (2h + k/4) * 8 + (k%4) * 2 + l/32.
__device__ __forceinline__ void stream_drain(Stream& st, int qn) {
  const int lane = lane_id();
  qn = __builtin_amdgcn_readfirstlane(qn);
  wave_sync_lds();
  for (int i0 = 0; i0 < qn; i0 += 64) {
    const int i = i0 + lane;
    if (i < qn) {
      const uint4 lo = st.rec[3 * i], hi = st.rec[3 * i + 1];
      const uint32_t at = st.rec[3 * i + 2].x;
      const float sc[8] = {__uint_as_float(lo.x), __uint_as_float(lo.y), __uint_as_float(lo.z),
                           __uint_as_float(lo.w), __uint_as_float(hi.x), __uint_as_float(hi.y),
                           __uint_as_float(hi.z), __uint_as_float(hi.w)};
      const uint32_t j = ((at >> 7) * kColTile) | (at & 31u);
      const int qb = (int)((at >> 6) & 1u) * 16 + (int)((at >> 5) & 1u);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int q = qb + (k >> 2) * 8 + (k & 3) * 2;
        if (sc[k] > __int_as_float(st.tau[q])) {
          const uint32_t pos = atomicAdd(&st.cnt[q], 1u);
          // a list that overflows keeps counting: the select kernel sees it
          if (pos < (uint32_t)kListCap)
            st.lists[(size_t)q * kListCap + pos] = make_key(__float_as_uint(relu(sc[k])), j);
        }
      }
    }
  }
  wave_sync_lds();
}

// Phase epilogue of one half, by phase: 0 the first sample tiles, 1 a sample
// tile, 2 a filter tile below every query's own block, 3 a masked filter
// tile.
template <int kPhase, int kHalf>
__device__ __forceinline__ void epilogue(Stream& st, const f32x16 (&acc)[2], int col, int& qn) {
  if (kPhase <= 1)
    sample_epilogue<kPhase == 0, kHalf>(st, acc, col);
  else
    qn = filter_epilogue<kPhase == 2, kHalf>(st, acc, col, qn);
}

// One position of a wavefront's scan: column tile `col`, its B fragments in
// bv[kBuf].  Issues the loads of the next position's tile (`colf`), then
// half 0's MFMAs, the epilogue of the previous position's half 1 (when
// `prev`: column `colp`), half 1's MFMAs and half 0's epilogue.  A drain of
// the survivor queue goes first, so that its stores precede the loads.
template <int kPhase, int kBuf, bool kPrev>
__device__ __forceinline__ void stream_pos(Stream& st, const bf16x8 (&A)[4][4],
                                           uint4 (&bv)[2][4], f32x16 (&accX)[2],
                                           f32x16 (&accY)[2], int col, int colp, int colf,
                                           const uint4* kb, int bt_g, int& qn) {
  if (kPhase >= 2 && qn >= 64) {
    stream_drain(st, qn);
    qn = 0;
  }
  load_cols(kb, colf, bt_g, st.voff, bv[kBuf ^ 1]);
  mma_rows<0>(bv[kBuf], A, accX);
  if (kPrev) epilogue<kPhase, 1>(st, accY, colp, qn);
  mma_rows<1>(bv[kBuf], A, accY);
  epilogue<kPhase, 0>(st, accX, col, qn);
}

// Position i of a phase's scan, its key tile in buffer kBuf.  Filter phases:
// position i >= ns scans column tile kPar (i - ns) + par; sample phases:
// i < ns, tile kSampleStride i + kSampleStep par, and the position after the
// last sample one is the first filter tile.
template <int kPhase, bool kPrev, int kBuf>
__device__ __forceinline__ void stream_pos_at(Stream& st, const bf16x8 (&A)[4][4],
                                              uint4 (&bv)[2][4], f32x16 (&accX)[2],
                                              f32x16 (&accY)[2], int i, int ns, int par,
                                              const uint4* kb, int bt_g, int& qn, int& colp) {
  const int col = kPhase >= 2 ? kPar * (i - ns) + par : i * kSampleStride + kSampleStep * par;
  const int colf = kPhase >= 2 ? col + kPar : (i + 1 < ns ? col + kSampleStride : par);
  stream_pos<kPhase, kBuf, kPrev>(st, A, bv, accX, accY, col, colp, colf, kb, bt_g, qn);
  colp = col;
}

// Positions [i0, i1) of a phase whose first position uses buffer kB0: the
// first one (no pending half), then pairs of straight-line positions, so
// that the buffers never move between registers.
template <int kPhase, int kB0>
__device__ __forceinline__ void stream_positions(Stream& st, const bf16x8 (&A)[4][4],
                                                 uint4 (&bv)[2][4], f32x16 (&accX)[2],
                                                 f32x16 (&accY)[2], int i0, int i1, int ns,
                                                 int par, const uint4* kb, int bt_g, int& qn,
                                                 int& colp) {
  stream_pos_at<kPhase, false, kB0>(st, A, bv, accX, accY, i0, ns, par, kb, bt_g, qn, colp);
  int i = i0 + 1;
  for (; i + 1 < i1; i += 2) {
    stream_pos_at<kPhase, true, kB0 ^ 1>(st, A, bv, accX, accY, i, ns, par, kb, bt_g, qn, colp);
    stream_pos_at<kPhase, true, kB0>(st, A, bv, accX, accY, i + 1, ns, par, kb, bt_g, qn, colp);
  }
  if (i < i1)
    stream_pos_at<kPhase, true, kB0 ^ 1>(st, A, bv, accX, accY, i, ns, par, kb, bt_g, qn, colp);
}

// Positions [i0, i1) of one phase, then the last position's half-1 epilogue.
// The queue holds at most 63 + 2 x 64 records after a position and 63 + 64
// after that last epilogue, within kQueue.
template <int kPhase>
__device__ __forceinline__ void stream_phase(Stream& st, const bf16x8 (&A)[4][4],
                                             uint4 (&bv)[2][4], f32x16 (&accX)[2],
                                             f32x16 (&accY)[2], int i0, int i1, int ns, int par,
                                             const uint4* kb, int bt_g, int& qn, int& colp) {
  if (i1 <= i0) return;
  // (position i uses buffer i & 1; positions are straight-line code, so that
  // the compiler interleaves epilogues with MFMAs)
  if (i0 & 1)
    stream_positions<kPhase, 1>(st, A, bv, accX, accY, i0, i1, ns, par, kb, bt_g, qn, colp);
  else
    stream_positions<kPhase, 0>(st, A, bv, accX, accY, i0, i1, ns, par, kb, bt_g, qn, colp);
  if (kPhase >= 2 && qn >= 64) {  // room for the pending half's survivors
    stream_drain(st, qn);
    qn = 0;
  }
  epilogue<kPhase, 1>(st, accY, colp, qn);
}

// After the sample phase: the bound of local query q (lane q of the wavefront
// computing it), from its histogram.
__device__ __forceinline__ int query_bound(const Stream& st, int q, bool fits) {
  const int lane = lane_id();
  const uint32_t* h = st.h[q];
  const uint32_t w0 = h[2 * lane], w1 = h[2 * lane + 1];
  uint32_t total = (w0 & 0xffffu) + (w0 >> 16) + (w1 & 0xffffu) + (w1 >> 16);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) total += (uint32_t)__shfl_xor((int)total, off);
  if (fits) return (int)0xff800000u;  // -inf: the whole row fits the list, keep every block
  if (total < (uint32_t)kSampleRank) return 0;  // too few samples above the base: keep every positive score
  int m;
  uint32_t sfx;
  wave_suffix_bin4(w0 & 0xffffu, w0 >> 16, w1 & 0xffffu, w1 >> 16, kSampleRank, m, sfx);
  return (max(0, (int)(st.mx[q] >> kSampleShift) - kSampleBase) + m) << kSampleShift;  // bin edge
}

// Grid (ceil(Nq/64), B); kStreamWaves = 8 wavefronts: kPar = 4 per group of
// 32 queries, one per column-tile parity.
__global__ __launch_bounds__(64 * kStreamWaves) void score_stream_kernel(const uint16_t* __restrict__ q_idx,
                                                           const uint4* __restrict__ k_frag,
                                                           const int32_t* __restrict__ lens,
                                                           uint64_t* __restrict__ lists,
                                                           uint32_t* __restrict__ list_cnt,
                                                           int32_t* __restrict__ tau_out, int Lmax,
                                                           int Nq) {
  __shared__ uint32_t s_h[kStreamQ][kHistWords];
  __shared__ uint32_t s_mx[kStreamQ];
  __shared__ uint32_t s_cnt[kStreamQ];
  __shared__ int32_t s_tau[kStreamQ];
  __shared__ uint4 s_rec[kStreamWaves][3 * kQueue];

  const int qbase = blockIdx.x * kStreamQ, b = blockIdx.y;
  const int tid = threadIdx.x, lane = lane_id();
  // (wavefront-uniform, so that the scan's loop control stays scalar)
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave / kPar, par = wave % kPar;
  const int len = guard_len(lens[b], Nq, Lmax);
  const int nbp = Lmax >> 2;
  const int gq0 = qbase + grp * 32;  // first query of the group
  const int t_last = query_t(len, Nq, min(gq0 + 31, Nq - 1));
  const int bt_g = (gq0 < Nq && t_last >= 0) ? (t_last >> 2) : 0;  // blocks the group scans
  const int ncol = (bt_g + kColTile - 1) / kColTile;
  // this wavefront's positions: ns sample tiles, then nf filter tiles
  // (the scan's bounds are wavefront-uniform: readfirstlane keeps its loop
  // control and column arithmetic scalar)
  const int ns = __builtin_amdgcn_readfirstlane(
      ncol > kSampleStep * par ? (ncol - 1 - kSampleStep * par) / kSampleStride + 1 : 0);
  const int nf = __builtin_amdgcn_readfirstlane(ncol > par ? (ncol - 1 - par) / kPar + 1 : 0);
  const uint4* kb = k_frag + (size_t)b * ((nbp + kColTile - 1) / kColTile) * kFragTile;
  for (int i = tid; i < kStreamQ * kHistWords; i += blockDim.x) (&s_h[0][0])[i] = 0u;
  if (tid < kStreamQ) {
    s_mx[tid] = 0u;
    s_cnt[tid] = 0u;
  }

  Stream st;
  st.h = &s_h[grp * 32];
  st.mx = &s_mx[grp * 32];
  st.cnt = &s_cnt[grp * 32];
  st.rec = s_rec[wave];
  st.tau = &s_tau[grp * 32];
  st.voff = (uint32_t)(lane * 16);
  // Stationary A fragments: 4 row tiles x 4 k-steps.  Row (lane & 31) of row
  // tile rt is query gq0 + rt*8 + row/4, head row%4; k chunk lane >> 5.
  bf16x8 A[4][4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    const int qa = gq0 + rt * 8 + ((lane & 31) >> 2);
    const uint4* p = reinterpret_cast<const uint4*>(
        q_idx + (((size_t)b * Nq + min(qa, Nq - 1)) * kIdxHeads + (lane & 3)) * kIdxDim);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      A[rt][ks] = as_bf16x8(qa < Nq ? p[ks * 2 + (lane >> 5)] : zero_u4());
  }
  // The A fragments only feed MFMAs: keep them in accumulation registers, so
  // that the MFMA results (read by the vector epilogue) fit in VGPRs.
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) asm volatile("" : "+a"(A[rt][ks]));
  int bt_min = 0x7fffffff;
  st.tq0 = query_t(len, Nq, gq0 + (lane >> 5));
  st.nq_left = Nq - gq0 - (lane >> 5);
  // (lists of rows past the batch are never written: their slots never pass)
  st.lists = lists + ((size_t)b * Nq + gq0) * kListCap;
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int qq = gq0 + slot_off(rt, c) + (lane >> 5);
      const int t = query_t(len, Nq, qq);
      bt_min = min(bt_min, (qq < Nq && t >= 0) ? (t >> 2) : 0);
      st.base_l[rt][c] = 0;
      st.tau_l[rt][c] = 0.f;
    }
  // tiles entirely below every query's own block need no causal mask
  for (int off = 32; off >= 1; off >>= 1) bt_min = min(bt_min, __shfl_xor(bt_min, off));
  // full filter positions: column tiles kPar m + par with (kPar m + par + 1) * 32 <= bt_min
  const int nfull = __builtin_amdgcn_readfirstlane(
      min(nf, max(0, (bt_min / kColTile - par + kPar - 1) / kPar)));
  // lane q < 32: own block of local query q
  const int tl = query_t(len, Nq, gq0 + lane);
  const int bt_q_lane = (lane < 32 && gq0 + lane < Nq && tl >= 0) ? (tl >> 2) : 0;
  // B fragments of the first position (the first sample tile, or with no
  // sample tiles the first filter tile)
  uint4 bv[2][4];
  load_cols(kb, ns > 0 ? kSampleStep * par : par, bt_g, st.voff, bv[0]);
  stream_barrier();  // LDS initialised

  f32x16 accX[2], accY[2];
  int qn = 0;  // survivors queued, not yet drained
  int colp = 0;
  // phase 0: the first sample tile of each parity (column tiles 0 .. kPar - 1)
  stream_phase<0>(st, A, bv, accX, accY, 0, min(ns, 1), ns, par, kb, bt_g, qn, colp);
  stream_barrier();
  // histogram base: three octaves below the best score of those tiles
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int c = 0; c < 4; ++c)
      st.base_l[rt][c] =
          max(0, (int)(st.mx[slot_off(rt, c) + (lane >> 5)] >> kSampleShift) - kSampleBase);
  // every sample tile into the histograms, the first one of this parity
  // again (its fragments reloaded into buffer 0; buffer 1 already holds the
  // next position's)
  if (ns > 0) load_cols(kb, kSampleStep * par, bt_g, st.voff, bv[0]);
  stream_phase<1>(st, A, bv, accX, accY, 0, ns, ns, par, kb, bt_g, qn, colp);
  stream_barrier();
  // bounds: wavefront of parity par computes local queries [kQp par, kQp par + kQp)
  {
    constexpr int kQp = 32 / kPar;
    int tau_v = 0;
    for (int i = 0; i < kQp; ++i) {
      const int q = kQp * par + i;
      const int bound = query_bound(st, q, rdl(bt_q_lane, q) <= kListCap);
      if (lane == i) tau_v = bound;
    }
    if (lane < kQp) s_tau[grp * 32 + kQp * par + lane] = tau_v;
  }
  stream_barrier();
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int c = 0; c < 4; ++c)
      st.tau_l[rt][c] = __int_as_float(s_tau[grp * 32 + slot_off(rt, c) + (lane >> 5)]);
  stream_phase<2>(st, A, bv, accX, accY, ns, ns + nfull, ns, par, kb, bt_g, qn, colp);
  stream_phase<3>(st, A, bv, accX, accY, ns + nfull, ns + nf, ns, par, kb, bt_g, qn, colp);
  if (qn > 0) stream_drain(st, qn);
  // no key load may outlive the workgroup (the prefetch runs past the end)
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  stream_barrier();
  if (tid < kStreamQ && qbase + tid < Nq) {
    list_cnt[(size_t)b * Nq + qbase + tid] = s_cnt[tid];
    // every list entry scores strictly above the bound: the select kernel
    // keeps keys at or above it, i.e. all of them
    tau_out[(size_t)b * Nq + qbase + tid] = s_tau[tid];
  }
}

// ------------------------------------------------------------------ SCAN
// Scan engine (decode-shaped calls: a few queries per sequence over a long
// context).  One pass over the compressed keys keeps only the blocks that can
// be in a row's top 512, and a per-row select finishes exactly; no score
// table is written.
//
// scan_filter_kernel: grid (n_slices, ceil(Nq/4), B), 512 threads.  A
// workgroup holds the 4 queries x 4 heads of one query group as the MFMA A
// operand (16x16x32: the lane (r, kc) receives block r of a 16-block tile
// for query kc, all four heads) and handles one slice of the sequence's
// blocks:
//  1. at once, before lens or first_block are known, it requests the first
//     two batches of its slice's tiles and the 1,024 sample blocks (every
//     (Lmax/4/1,024)-th block: the same for every workgroup of the
//     sequence), so the memory system is busy from the start; once lens and
//     first_block arrive, blocks past the query group's own blocks are
//     masked and blocks not yet in the cache (j >= first_block, k_idx given)
//     are compressed in registers from k_idx instead (and written to the
//     cache by the lanes that scan them);
//  2. each query's bound tau is the lower edge of the bin (64 bins per
//     octave of the score) holding its 12th best valid sample score (samples
//     below the group's first query's own block): every workgroup of a row
//     derives the same tau;
//  3. it streams the slice (wavefront w takes the 16-block tiles w, w + 8,
//     ..., four tiles per batch with the next batch's loads in flight) and
//     appends every block scoring >= tau to the row's LDS list, then writes
//     the list as the row's segment for this slice, with its length (which
//     may exceed the segment's capacity: the select sees that).
// Rows whose group's first query has fewer than 2,048 candidate blocks, or
// fewer than 12 valid samples, keep every block (tau = 0).
//
// Why the result is exact.  Every candidate scores >= tau.  If the row's
// candidates number at least 512 (and no segment overflowed), at least 512
// blocks score >= tau, so the row's 512th best score is >= tau and every
// block of its top 512 is a candidate.  Otherwise the select takes the exact
// whole-row path.  With 1,024 samples spread over n blocks, the bound lies
// above the 512th best block only if 12 samples fall among the top 512
// (expected 1,024 x 512 / n: 2 at n = 262,144), about 2e-6 per row for
// independent scores; the candidates then number about 12 n / 1,024 (3,072
// at n = 262,144) plus the blocks in the bound's bin.
constexpr int kScanWaves = 8;
constexpr int kScanThreads = 64 * kScanWaves;
constexpr int kScanSegCap = 512;       // candidates a row keeps per slice
constexpr int kScanSampleN = 1024;     // sample blocks per sequence
constexpr int kScanSampleRank = 12;    // tau: the bin of the 12th best sample score
constexpr int kScanSampleMin = 2048;   // fewer candidate blocks: keep every block
constexpr int kScanSampleShift = 17;   // sample bins: score bits >> 17 (64 per octave)
constexpr int kScanU = 4;              // 16-block tiles per wavefront batch
constexpr int kScanCandCap = 8192;     // candidates a select workgroup holds in LDS
constexpr int kScanMaxSlices = 2048;   // slices a select workgroup can walk
constexpr int kScanMaxSliceBlocks = 8192;
constexpr int kScanBmWords = kScanMaxSliceBlocks / 32;  // a slice's bitmap, 32-bit words

// One wavefront: the lower edge (as float bits) of the bin, 64 per octave,
// holding the k-th largest of the 16 values each lane holds (non-negative
// float bits), over the 256 bins below and including the largest value's;
// 0 when fewer than k values lie in those bins.  h: this wavefront's
// 256-word LDS histogram.
__device__ uint32_t wave_kth_bin_edge(const uint32_t (&v)[16], uint32_t k, uint32_t* h) {
  const int lane = lane_id();
  uint32_t mx = 0u;
#pragma unroll
  for (int e = 0; e < 16; ++e) mx = max(mx, v[e]);
  const int top = (int)(wave_max_u32(mx) >> kScanSampleShift);
  const int base = max(0, top - 255);
#pragma unroll
  for (int i = 0; i < 4; ++i) h[lane + 64 * i] = 0u;
  wave_sync_lds();
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int bin = (int)(v[e] >> kScanSampleShift) - base;
    if (bin >= 0) atomicAdd(&h[bin], 1u);
  }
  wave_sync_lds();
  const uint32_t c0 = h[4 * lane], c1 = h[4 * lane + 1], c2 = h[4 * lane + 2], c3 = h[4 * lane + 3];
  uint32_t tot = c0 + c1 + c2 + c3;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) tot += (uint32_t)__shfl_xor((int)tot, off);
  if (tot < k) return 0u;
  int bin;
  uint32_t sfx;
  wave_suffix_bin4(c0, c1, c2, c3, k, bin, sfx);
  return (uint32_t)(base + bin) << kScanSampleShift;
}

__global__ __launch_bounds__(kScanThreads) void scan_filter_kernel(
    const uint16_t* __restrict__ q_idx, uint16_t* __restrict__ k_cmp,
    const int32_t* __restrict__ lens, const uint16_t* __restrict__ k_idx,
    const int32_t* __restrict__ first_block, uint64_t* __restrict__ seg,
    uint32_t* __restrict__ seg_cnt, int Lmax, int Nq, int slice_blocks, int n_slices) {
  __shared__ uint64_t s_seg[4][kScanSegCap];
  __shared__ uint32_t s_samp[4][kScanSampleN];
  __shared__ uint32_t s_hist[4][256];
  __shared__ uint32_t s_cnt[4];
  __shared__ uint32_t s_tau[4];
  __shared__ __align__(8) uint32_t s_bm[4][kScanBmWords];  // candidates of the slice, per query
  __shared__ uint32_t s_bmpre[4][kScanBmWords];
  __shared__ uint32_t s_bmsum[kScanWaves];
  const int slice = blockIdx.x, q0 = blockIdx.y * 4, b = blockIdx.z;
  const int tid = threadIdx.x, lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, kc = lane >> 4;
  const int nbp = Lmax >> 2;
  const int j_begin = slice * slice_blocks;
  const int j_cap = min(j_begin + slice_blocks, nbp);  // the slice, as far as the cache goes
  const int samp_stride = max(1, nbp / kScanSampleN);
  const uint4* src = reinterpret_cast<const uint4*>(k_idx + (size_t)b * Lmax * kIdxDim);
  uint4* kb = reinterpret_cast<uint4*>(k_cmp + (size_t)b * nbp * kIdxDim);

  // 1. requests that need neither lens nor first_block: the query group's
  // fragments and the lane's sample blocks first (they are needed first and
  // the waits count loads in order), then the slice's first two batches
  // (tiles w + 8 (4 bi + u), lane (r, kc): dims 8 kc .. and 32 + 8 kc .. of
  // block r).  Loads are unconditional, from addresses clamped into the
  // cache: a block past the range reads some other block, and its score is
  // masked where it is used (each MFMA output column depends on its own block
  // only).  (Conditional loads would make the compiler wait for every load in
  // flight.)
  // (A rows of queries past the batch repeat the last query; their lanes'
  // results are never kept)
  const uint4* qp = reinterpret_cast<const uint4*>(
      q_idx + (((size_t)b * Nq + min(q0 + (r >> 2), Nq - 1)) * kIdxHeads + (r & 3)) * kIdxDim);
  const bf16x8 a0 = as_bf16x8(qp[kc]), a1 = as_bf16x8(qp[4 + kc]);
  constexpr int kSampT = kScanSampleN / (16 * kScanWaves);  // sample tiles per wavefront
  uint4 sA[kSampT][2];
#pragma unroll
  for (int tt = 0; tt < kSampT; ++tt) {
    const int j = min((wave * (kScanSampleN / kScanWaves) + tt * 16 + r) * samp_stride, nbp - 1);
    sA[tt][0] = kb[(size_t)j * 8 + kc];
    sA[tt][1] = kb[(size_t)j * 8 + 4 + kc];
  }
  uint4 bA[kScanU][2], bB[kScanU][2];
  auto load = [&](uint4 (&bv)[kScanU][2], int bi) {
#pragma unroll
    for (int u = 0; u < kScanU; ++u) {
      const int j = min(j_begin + (wave + kScanWaves * (kScanU * bi + u)) * 16 + r, nbp - 1);
      bv[u][0] = kb[(size_t)j * 8 + kc];
      bv[u][1] = kb[(size_t)j * 8 + 4 + kc];
    }
  };
  load(bA, 0);
  load(bB, 1);
  if (tid < 4) s_cnt[tid] = 0u;

  // the group's queries ascend in position: its first and last valid one
  const int len = guard_len(lens[b], Nq, Lmax);
  const int nb = len >> 2;
  const int t_first = query_t(len, Nq, q0);
  const int t_last = query_t(len, Nq, min(q0 + 3, Nq - 1));
  const int bt_min = t_first >= 0 ? (t_first >> 2) : 0;
  const int bt_g = t_last >= 0 ? (t_last >> 2) : 0;
  const int qo = q0 + kc;  // this lane's query
  const int t_o = query_t(len, Nq, qo);
  const int bt_o = (qo < Nq && t_o >= 0) ? (t_o >> 2) : 0;
  const int j_end = min(j_begin + slice_blocks, bt_g);
  const bool active = j_begin < j_end;  // (uniform)
  int fb = nb;  // blocks from fb on are not in the cache yet
  if (k_idx != nullptr) fb = first_block ? guard(first_block[b], 0, nb) : 0;
  // blocks not yet in the cache, compressed here: in the prefetched batches
  // (then written to the cache) and among the samples
  auto fix_new = [&](uint4 (&bv)[kScanU][2], int bi) {
#pragma unroll
    for (int u = 0; u < kScanU; ++u) {
      const int j = j_begin + (wave + kScanWaves * (kScanU * bi + u)) * 16 + r;
      if (j >= fb && j < j_end) {
        bv[u][0] = compress_chunk(src + (size_t)j * 32 + kc);
        bv[u][1] = compress_chunk(src + (size_t)j * 32 + 4 + kc);
        kb[(size_t)j * 8 + kc] = bv[u][0];
        kb[(size_t)j * 8 + 4 + kc] = bv[u][1];
      }
    }
  };
  if (fb < j_end && active) {  // (uniform)
    fix_new(bA, 0);
    fix_new(bB, 1);
  }
  // the slice's new blocks the scan does not cover
  if (k_idx != nullptr) {
    const long long c0 = (long long)max(fb, active ? j_end : j_begin) * 8;
    const long long c1 = (long long)min(nb, j_cap) * 8;
    for (long long g = c0 + tid; g < c1; g += kScanThreads)
      kb[g] = compress_chunk(src + (g >> 3) * 32 + (g & 7));
  }

  // 2. the bound tau of each query of the group
  const bool sampled = active && bt_min >= kScanSampleMin;  // (uniform)
  if (sampled) {
#pragma unroll
    for (int tt = 0; tt < kSampT; ++tt) {
      const int i = wave * (kScanSampleN / kScanWaves) + tt * 16 + r;
      const int j = i * samp_stride;
      uint4 b0 = sA[tt][0], b1 = sA[tt][1];
      if (j >= fb && j < bt_min) {  // not in the cache yet: compress it here
        b0 = compress_chunk(src + (size_t)j * 32 + kc);
        b1 = compress_chunk(src + (size_t)j * 32 + 4 + kc);
      }
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      acc = mfma16(a0, as_bf16x8(b0), acc);
      acc = mfma16(a1, as_bf16x8(b1), acc);
      // samples at or past the group's first own block count as 0
      s_samp[kc][i] = j < bt_min ? relu_sum_bits(acc[0], acc[1], acc[2], acc[3]) : 0u;
    }
  }
  __syncthreads();  // samples in LDS
  if (wave < 4) {
    uint32_t tau = 0u;  // keep every block
    if (sampled) {
      uint32_t v[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) v[e] = s_samp[wave][lane * 16 + e];
      tau = wave_kth_bin_edge(v, kScanSampleRank, s_hist[wave]);
    }
    if (lane == 0) s_tau[wave] = tau;
  }
  __syncthreads();

  // 3. the scan of [j_begin, j_end)
  if (active) {
    const uint32_t tau_o = s_tau[kc];
    const int lim = min(bt_o, j_end);  // this lane's query's candidates in the slice
    const int ntiles = (j_end - j_begin + 15) >> 4;
    constexpr int kStep = kScanWaves * kScanU;  // tiles per batch of the workgroup
    const int nbatch =
        __builtin_amdgcn_readfirstlane(ntiles > wave ? (ntiles - wave + kStep - 1) / kStep : 0);
    auto load_fix = [&](uint4 (&bv)[kScanU][2], int bi) {
      load(bv, bi);
      if (fb < j_end) fix_new(bv, bi);  // (uniform)
    };
    auto proc = [&](const uint4 (&bv)[kScanU][2], int bi) {
#pragma unroll
      for (int u = 0; u < kScanU; ++u) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = mfma16(a0, as_bf16x8(bv[u][0]), acc);
        acc = mfma16(a1, as_bf16x8(bv[u][1]), acc);
        const int j = j_begin + (wave + kScanWaves * (kScanU * bi + u)) * 16 + r;
        const uint32_t bits = relu_sum_bits(acc[0], acc[1], acc[2], acc[3]);
        const bool pass = j < lim && bits >= tau_o;
        const uint64_t m = __ballot(pass);
        if (m == 0) continue;
        const uint32_t mq = (uint32_t)(m >> (16 * kc)) & 0xffffu;
        uint32_t base = 0;
        if (r == 0 && mq != 0u) base = atomicAdd(&s_cnt[kc], (uint32_t)__popc(mq));
        base = (uint32_t)__shfl((int)base, lane & 48);
        const uint32_t pos = base + (uint32_t)__popc(mq & ((1u << r) - 1u));
        if (pass && pos < (uint32_t)kScanSegCap) s_seg[kc][pos] = make_key(bits, (uint32_t)j);
      }
    };
    for (int bi = 0; bi < nbatch; bi += 2) {
      proc(bA, bi);
      if (bi + 2 < nbatch) load_fix(bA, bi + 2);
      if (bi + 1 >= nbatch) break;
      proc(bB, bi + 1);
      if (bi + 3 < nbatch) load_fix(bB, bi + 3);
    }
  }
  // 4. the group's segments of this slice (an empty one when nothing was
  // scanned), each in ascending block order: a candidate's place is the
  // number of the query's candidates below it in the slice, counted on a
  // bitmap of the slice's blocks (the appends above come in no fixed order).
  // A row's segments in slice order then list its candidates ascending.
  // Overflowed segments are left unordered: their rows take the exact path.
#pragma unroll
  for (int i = tid; i < 4 * kScanBmWords; i += kScanThreads) (&s_bm[0][0])[i] = 0u;
  __syncthreads();
  const int q = tid >> 7, qt = tid & 127;  // 128 threads per query
  const uint32_t n = s_cnt[q];
  const bool ordered = n <= (uint32_t)kScanSegCap;  // (uniform per query)
  if (ordered)
    for (uint32_t i = qt; i < n; i += 128) {
      const uint32_t o = key_block(s_seg[q][i]) - (uint32_t)j_begin;
      atomicOr(&s_bm[q][o >> 5], 1u << (o & 31));
    }
  __syncthreads();
  {
    // exclusive prefix of the word popcounts, two words per thread
    const uint2 w = reinterpret_cast<const uint2*>(s_bm[q])[qt];
    const uint32_t c0 = (uint32_t)__popc(w.x), own = c0 + (uint32_t)__popc(w.y);
    const uint32_t incl = wave_incl_sum(own);
    if (lane == 63) s_bmsum[tid >> 6] = incl;
    __syncthreads();
    const uint32_t below = (tid & 64) ? s_bmsum[(tid >> 6) - 1] : 0u;  // other wavefront of q
    const uint32_t ex = below + incl - own;
    s_bmpre[q][2 * qt] = ex;
    s_bmpre[q][2 * qt + 1] = ex + c0;
  }
  __syncthreads();
  if (q0 + q < Nq) {
    const size_t sidx = ((size_t)b * Nq + q0 + q) * n_slices + slice;
    if (qt == 0) seg_cnt[sidx] = n;
    const uint32_t nk = min(n, (uint32_t)kScanSegCap);
    for (uint32_t i = qt; i < nk; i += 128) {
      const uint64_t key = s_seg[q][i];
      uint32_t at = i;
      if (ordered) {
        const uint32_t o = key_block(key) - (uint32_t)j_begin;
        at = s_bmpre[q][o >> 5] + (uint32_t)__popc(s_bm[q][o >> 5] & ((1u << (o & 31)) - 1u));
      }
      seg[sidx * kScanSegCap + at] = key;
    }
  }
}
static_assert(kScanThreads == 4 * 128 && kScanBmWords == 2 * 128,
              "segment order: 128 threads and 256 bitmap words per query");

// Block-wide exclusive prefix sum of one value per thread (512 threads) and
// the total; s_red: kScanWaves words.  Ends past a barrier.
__device__ __forceinline__ uint32_t block_excl_sum(uint32_t v, uint32_t* s_red, uint32_t& total) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const uint32_t incl = wave_incl_sum(v);
  __syncthreads();  // s_red free
  if (lane == 63) s_red[wave] = incl;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kScanWaves; ++w) {
    const uint32_t x = s_red[w];
    before += w < wave ? x : 0u;
    all += x;
  }
  total = all;
  return before + incl - v;
}

// Per row (grid (Nq, B), 512 threads): the row's candidates from its slices'
// segments into LDS, then
//  * the cut: a 2,048-bin linear histogram of the candidates' scores over
//    [lowest, highest] finds the bin holding the 512th best; while that bin
//    holds several score values it is narrowed by histograms of its score
//    bits, 11 at a time, until one value v remains (usually at once): the
//    winners are the scores above v and the lowest-id candidates scoring v;
//  * the order: the list is already ascending in block id (each segment is
//    ordered by the filter, and the segments follow the slices), so a prefix
//    count of the ties keeps the first (lowest-id) ones needed and a prefix
//    count of the kept entries writes them in list order: no sort.
// Rows with too few candidates (tau above the 512th best score), an
// overflowed segment or more candidates than the LDS list holds take the
// exact whole-row path.
__global__ __launch_bounds__(kScanThreads) void scan_select_kernel(
    const uint64_t* __restrict__ seg, const uint32_t* __restrict__ seg_cnt,
    const uint16_t* __restrict__ q_idx, const uint16_t* __restrict__ k_cmp,
    const int32_t* __restrict__ lens, int32_t* __restrict__ sel, int32_t* __restrict__ n_sel,
    int Lmax, int Nq, int slice_blocks, int n_slices) {
  __shared__ __align__(16) uint64_t keys[kScanCandCap];
  __shared__ uint32_t s_pre[kScanMaxSlices + 1];
  __shared__ uint32_t hist[kHistBins];
  __shared__ uint32_t s_red[2 * kScanWaves];
  __shared__ uint32_t bcast[8];
  __shared__ uint32_t s_bad;
  __shared__ uint32_t s_mm[4];
  __shared__ float qf[kIdxHeads * kIdxDim];
  const int q = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, lane = lane_id();
  const int wave = tid >> 6;
  const size_t row = (size_t)b * Nq + q;
  const uint32_t* cnt = seg_cnt + row * n_slices;
  const uint64_t* rseg = seg + row * n_slices * (size_t)kScanSegCap;
  const int t = query_t(guard_len(lens[b], Nq, Lmax), Nq, q);
  int32_t* srow = sel + row * kTopK;
  if (write_trivial(t, srow, n_sel + row)) return;
  const int bt = t >> 2;
  const int n_used = min(n_slices, (bt + slice_blocks - 1) / slice_blocks);  // (<= kScanMaxSlices)
  if (tid == 0) {
    s_bad = 0u;
    s_mm[0] = 0xffffffffu;
    s_mm[1] = 0u;
    s_mm[2] = 0xffffffffu;
    s_mm[3] = 0u;
  }
  __syncthreads();
  // exclusive prefix of the segment lengths, 512 at a time
  uint32_t carry = 0;
  for (int s0 = 0; s0 < n_used; s0 += kScanThreads) {
    const int s = s0 + tid;
    uint32_t c = s < n_used ? cnt[s] : 0u;
    const bool over = c > (uint32_t)kScanSegCap;
    if (over) c = 0u;
    if (__ballot(over) != 0 && lane == 0) s_bad = 1u;
    uint32_t tot;
    const uint32_t ex = block_excl_sum(c, s_red, tot);
    if (s < n_used) s_pre[s] = carry + ex;
    carry += tot;
  }
  const uint32_t total = carry;
  if (tid == 0) s_pre[n_used] = total;
  __syncthreads();
  const bool ok = s_bad == 0u && total >= (uint32_t)kTopK && total <= (uint32_t)kScanCandCap;
  if (!ok) {
    const int nbp = Lmax >> 2;
    select_whole_row<true>(nullptr, q_idx + row * kIdxHeads * kIdxDim,
                           k_cmp + (size_t)b * nbp * kIdxDim, bt, srow, qf, hist, bcast, s_red);
    if (tid == 0) n_sel[row] = kTopK;
    return;
  }
  // ---- the candidates into LDS: wavefront w copies segments w, w + 8, ...,
  // four at a time, the first 128 entries of each with two independent loads
  // per lane (segments hold about 50 on average), any rest one by one
  for (int s0 = wave; s0 < n_used; s0 += 4 * kScanWaves) {
    uint64_t v[4][2];
    uint32_t n4[4], o4[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int s = s0 + kScanWaves * k;
      n4[k] = s < n_used ? s_pre[s + 1] - s_pre[s] : 0u;
      o4[k] = s < n_used ? s_pre[s] : 0u;
      // (unconditional loads inside the row's segment storage; entries past
      // a segment's length are not kept)
      const size_t sb = (size_t)min(s, n_used - 1) * kScanSegCap;
#pragma unroll
      for (int m = 0; m < 2; ++m) v[k][m] = rseg[sb + lane + 64 * m];
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const uint32_t i = (uint32_t)(lane + 64 * m);
        if (i < n4[k]) keys[o4[k] + i] = v[k][m];
      }
      const int s = s0 + kScanWaves * k;
      for (uint32_t i = 128 + lane; i < n4[k]; i += 64) keys[o4[k] + i] = rseg[(size_t)s * kScanSegCap + i];
    }
  }
  for (int i = tid; i < kHistBins; i += kScanThreads) hist[i] = 0u;
  __syncthreads();
  // the lowest and highest candidate score
  {
    uint32_t lo = 0xffffffffu, hi = 0u;
    for (uint32_t e = tid; e < total; e += kScanThreads) {
      const uint32_t sc = (uint32_t)(keys[e] >> 32);
      lo = min(lo, sc);
      hi = max(hi, sc);
    }
    lo = wave_min_u32(lo);
    hi = wave_max_u32(hi);
    if (lane == 0) {
      atomicMin(&s_mm[0], lo);
      atomicMax(&s_mm[1], hi);
    }
  }
  __syncthreads();
  const uint32_t lo = s_mm[0], hi = s_mm[1];
  // ---- the cut: the bin of a 2,048-bin linear histogram over [lowest,
  // highest] that holds the 512th best score
  const float lo_f = __uint_as_float(lo);
  const float scale = hi > lo ? 2047.0f / (__uint_as_float(hi) - lo_f) : 0.f;
  for (uint32_t e = tid; e < total; e += kScanThreads)
    atomicAdd(&hist[lin_bin((uint32_t)(keys[e] >> 32), lo_f, scale)], 1u);
  __syncthreads();
  uint32_t cb, above;
  {
    // thread t owns bins 4t .. 4t + 3; suffix counts from the top
    const uint4 c = reinterpret_cast<const uint4*>(hist)[tid];
    const uint32_t own = c.x + c.y + c.z + c.w;
    uint32_t tot;
    const uint32_t ex = block_excl_sum(own, s_red, tot);
    const uint32_t cc[4] = {c.x, c.y, c.z, c.w};
    uint32_t sfx = tot - ex - own;  // bins above this thread's four
#pragma unroll
    for (int i = 3; i >= 0; --i) {
      if (sfx < (uint32_t)kTopK && sfx + cc[i] >= (uint32_t)kTopK) {
        bcast[0] = (uint32_t)(4 * tid + i);
        bcast[1] = sfx;
      }
      sfx += cc[i];
    }
    __syncthreads();
    cb = bcast[0];
    above = bcast[1];
  }
  // The cut bin's lowest and highest score; while it holds several values,
  // narrow it: a histogram of (bits - lowest) >> shift over the candidates
  // in it (11 bits at a time) finds the sub-bin holding the cut, until one
  // value remains.  Then v is that value and `need` the candidates scoring
  // exactly v that are kept.
  uint32_t need = kTopK - above;  // still to take from the cut bin
  uint32_t blo = 0u, bhi = 0xffffffffu;  // the cut bin's score range (bits), inclusive
  bool first = true;
  for (;;) {
    uint32_t bmn = 0xffffffffu, bmx = 0u;
    for (uint32_t e = tid; e < total; e += kScanThreads) {
      const uint32_t sc = (uint32_t)(keys[e] >> 32);
      const bool in = first ? lin_bin(sc, lo_f, scale) == cb : (sc >= blo && sc <= bhi);
      if (in) {
        bmn = min(bmn, sc);
        bmx = max(bmx, sc);
      }
    }
    bmn = wave_min_u32(bmn);
    bmx = wave_max_u32(bmx);
    if (lane == 0) {
      atomicMin(&s_mm[2], bmn);
      atomicMax(&s_mm[3], bmx);
    }
    for (int i = tid; i < kHistBins; i += kScanThreads) hist[i] = 0u;
    __syncthreads();
    blo = s_mm[2];
    bhi = s_mm[3];
    first = false;
    if (blo == bhi) break;  // (uniform) one value: v = blo
    const uint32_t span = bhi - blo;
    const uint32_t shift = pick_shift(span);  // (span >> shift) < 2048
    for (uint32_t e = tid; e < total; e += kScanThreads) {
      const uint32_t sc = (uint32_t)(keys[e] >> 32);
      if (sc >= blo && sc <= bhi) atomicAdd(&hist[(sc - blo) >> shift], 1u);
    }
    __syncthreads();
    {
      const uint4 c = reinterpret_cast<const uint4*>(hist)[tid];
      const uint32_t own = c.x + c.y + c.z + c.w;
      uint32_t tot;
      const uint32_t ex = block_excl_sum(own, s_red, tot);
      const uint32_t cc[4] = {c.x, c.y, c.z, c.w};
      uint32_t sfx = tot - ex - own;
#pragma unroll
      for (int i = 3; i >= 0; --i) {
        if (sfx < need && sfx + cc[i] >= need) {
          bcast[0] = (uint32_t)(4 * tid + i);
          bcast[1] = sfx;
        }
        sfx += cc[i];
      }
      if (tid == 0) {
        s_mm[2] = 0xffffffffu;
        s_mm[3] = 0u;
      }
      __syncthreads();
    }
    const uint32_t sub = bcast[0];
    need -= bcast[1];  // the sub-bins above the cut's are kept whole
    // the cut sub-bin's range: [blo + sub << shift, blo + (sub + 1) << shift - 1]
    const uint32_t nlo = blo + (sub << shift);
    bhi = min(bhi, nlo + ((1u << shift) - 1u));
    blo = nlo;
  }
  // winners: every score above v; ties: exactly v, of which the `need`
  // lowest-id ones are kept
  const uint32_t v = blo;
  auto is_win = [&](uint64_t key) -> bool { return (uint32_t)(key >> 32) > v; };
  auto is_tie = [&](uint64_t key) -> bool { return (uint32_t)(key >> 32) == v; };
  // ---- the winners in list order, which is ascending block order (each
  // segment is ordered and the segments follow the slices): thread t walks
  // the run [t per, t per + per) of the list; a prefix count of the ties
  // keeps the first `need` of them (the lowest ids), a prefix count of the
  // kept entries places them
  const uint32_t per = (total + kScanThreads - 1) / kScanThreads;  // <= kScanCandCap / 512
  const uint32_t e0 = min(total, (uint32_t)tid * per), e1 = min(total, e0 + per);
  uint32_t ntie = 0;
  for (uint32_t e = e0; e < e1; ++e) ntie += is_tie(keys[e]) ? 1u : 0u;
  uint32_t tot;
  const uint32_t tie0 = block_excl_sum(ntie, s_red, tot);
  uint32_t nkeep = 0;
  {
    uint32_t tr = tie0;
    for (uint32_t e = e0; e < e1; ++e) {
      const uint64_t key = keys[e];
      const bool tie = is_tie(key);
      nkeep += (is_win(key) || (tie && tr < need)) ? 1u : 0u;
      tr += tie ? 1u : 0u;
    }
  }
  uint32_t pos = block_excl_sum(nkeep, s_red, tot);
  {
    uint32_t tr = tie0;
    for (uint32_t e = e0; e < e1; ++e) {
      const uint64_t key = keys[e];
      const bool tie = is_tie(key);
      if (is_win(key) || (tie && tr < need)) {
        if (pos < (uint32_t)kTopK) srow[pos] = (int32_t)key_block(key);
        ++pos;
      }
      tr += tie ? 1u : 0u;
    }
  }
  if (tid == 0) n_sel[row] = kTopK;
}


}  // namespace

// ------------------------------------------------------------------ host side

namespace {
// Slices of the scan engine: about one workgroup per compute unit over the
// batch's (sequence, query group) pairs, at most kScanMaxSliceBlocks blocks
// each (so that a slice's expected candidates stay far below a segment's
// capacity), a multiple of the 16-block tile.
struct ScanGeom {
  int slice_blocks, n_slices;
};
ScanGeom scan_geom(const Dims& d) {
  const long long nbp = d.Lmax / 4;
  const long long groups = (long long)d.B * ((d.Nq + 3) / 4);
  const long long want = groups > 0 ? (256 + groups - 1) / groups : 1;
  long long sb = (nbp + want - 1) / want;
  if (sb > kScanMaxSliceBlocks) sb = kScanMaxSliceBlocks;
  sb = (sb + 15) / 16 * 16;
  if (sb < 16) sb = 16;
  return {(int)sb, (int)((nbp + sb - 1) / sb)};
}
bool scan_fits(const Dims& d) { return d.Nq <= 64 && scan_geom(d).n_slices <= kScanMaxSlices; }
}  // namespace

// Automatic choice: decode-shaped calls (at most 64 queries per sequence)
// take the table engine while its score table fits 512 MiB (at a 1M-token
// context, batch 4 x 4: 67.5 us per step against 70.0 us for the scan
// engine, whose sampled bound costs more latency at the start of its pass
// than the table's write and read-back), longer contexts the scan engine, whose
// workspace grows with the slices instead of the context; prefill-shaped
// calls the stream engine.
TopkPath choose_topk_path(const Dims& d, uint32_t flags) {
  if (flags & 1u) return TopkPath::kTable;
  if (flags & 2u) return TopkPath::kStream;
  if (flags & 4u) return scan_fits(d) ? TopkPath::kScan : TopkPath::kStream;
  const double table_bytes = (double)d.B * d.Nq * (d.Lmax / 4) * 4.0;
  if (d.Nq <= 64 && table_bytes <= 512.0 * 1024 * 1024) return TopkPath::kTable;
  return scan_fits(d) ? TopkPath::kScan : TopkPath::kStream;
}

namespace {
int table_stride(const Dims& d) { return ((d.Lmax / 4) + 3) & ~3; }
int group_stride(const Dims& d) { return (((d.Lmax / 4) + kGroup - 1) / kGroup + 3) & ~3; }
struct TableWs {
  uint32_t* scores;  // [rows][table stride] score bits
  uint32_t* gmax;    // [rows][group stride] group maxima
};
struct StreamWs {
  uint64_t* lists;
  uint32_t* cnt;
  int32_t* tau;
  uint4* frag;  // [B][column tiles][kFragTile] fragment-ordered compressed keys
};
TableWs carve_table(const Dims& d, void* ws, size_t* total) {
  Carve c{static_cast<char*>(ws), 0};
  const size_t rows = (size_t)d.B * d.Nq;
  TableWs w;
  w.scores = c.take<uint32_t>(rows * (size_t)table_stride(d));
  w.gmax = c.take<uint32_t>(rows * (size_t)group_stride(d));
  if (total) *total = c.off;
  return w;
}
struct ScanWs {
  uint64_t* seg;     // [rows][n_slices][kScanSegCap] candidate keys
  uint32_t* cnt;     // [rows][n_slices] segment lengths
};
ScanWs carve_scan(const Dims& d, void* ws, size_t* total) {
  Carve c{static_cast<char*>(ws), 0};
  const size_t rows = (size_t)d.B * d.Nq;
  const ScanGeom g = scan_geom(d);
  ScanWs w;
  w.seg = c.take<uint64_t>(rows * (size_t)g.n_slices * kScanSegCap);
  w.cnt = c.take<uint32_t>(rows * (size_t)g.n_slices);
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
  w.frag = c.take<uint4>((size_t)d.B * ((d.Lmax / 4 + kColTile - 1) / kColTile) * kFragTile);
  if (total) *total = c.off;
  return w;
}
}  // namespace

size_t topk_workspace_bytes(const Dims& d, TopkPath path) {
  size_t total = 0;
  if (path == TopkPath::kTable)
    carve_table(d, nullptr, &total);
  else if (path == TopkPath::kScan)
    carve_scan(d, nullptr, &total);
  else
    carve_stream(d, nullptr, &total);
  return total;
}

hipError_t launch_table_score(const Dims& d, const uint16_t* q_idx, uint16_t* k_cmp,
                              const int32_t* lens, void* ws, hipStream_t s,
                              const CompressFuse* fuse) {
  if (d.B == 0 || d.Nq == 0) return hipSuccess;
  if (fuse && !topk_can_fuse_compress(d, TopkPath::kTable)) return hipErrorInvalidValue;
  TableWs w = carve_table(d, ws, nullptr);
  const unsigned qg = (unsigned)((d.Nq + 3) / 4);
  // the longest span (256 blocks per wavefront) that still gives about two
  // workgroups per compute unit
  const long long nbp = d.Lmax / 4, rows = (long long)qg * d.B;
  int span = 256;
  while (span > 64 && ((nbp + 4 * span - 1) / (4 * span)) * rows < 512) span /= 2;
  const dim3 grid((unsigned)((nbp + 4 * span - 1) / (4 * span)), qg, (unsigned)d.B);
#define QSA_TABLE_SCORE(S)                                                                    \
  QSA_LAUNCH(score_table_kernel<S>, grid, dim3(256), 0, s, q_idx, k_cmp, lens, w.scores,     \
             table_stride(d), w.gmax, group_stride(d), d.Lmax, d.Nq,                        \
             fuse ? fuse->k_idx : nullptr, fuse ? fuse->first_block : nullptr)
  if (span == 256) QSA_TABLE_SCORE(256);
  else if (span == 128) QSA_TABLE_SCORE(128);
  else QSA_TABLE_SCORE(64);
#undef QSA_TABLE_SCORE
  return hipGetLastError();
}

hipError_t launch_table_pick(const Dims& d, const int32_t* lens, int32_t* sel, int32_t* n_sel,
                             void* ws, hipStream_t s) {
  if (d.B == 0 || d.Nq == 0) return hipSuccess;
  TableWs w = carve_table(d, ws, nullptr);
  QSA_LAUNCH(table_pick_kernel, dim3((unsigned)((size_t)d.B * d.Nq)), dim3(kPickThreads), 0, s,
             w.scores, table_stride(d), w.gmax, group_stride(d), lens, sel, n_sel, d.Lmax, d.Nq);
  return hipGetLastError();
}

bool topk_can_fuse_compress(const Dims& d, TopkPath path) {
  // one scoring workgroup per slice and sequence: each new block is written once
  return (path == TopkPath::kTable || path == TopkPath::kScan) && d.Nq <= 4;
}

hipError_t launch_index_topk(const Dims& d, TopkPath path, const uint16_t* q_idx,
                             uint16_t* k_cmp, const int32_t* lens, int32_t* sel,
                             int32_t* n_sel, void* ws, hipStream_t s,
                             const CompressFuse* fuse) {
  if (fuse && !topk_can_fuse_compress(d, path)) return hipErrorInvalidValue;
  if (d.B == 0 || d.Nq == 0) return hipSuccess;
  const dim3 grid_q((unsigned)d.Nq, (unsigned)d.B);
  if (path == TopkPath::kTable) {
    const hipError_t e = launch_table_score(d, q_idx, k_cmp, lens, ws, s, fuse);
    if (e != hipSuccess) return e;
    return launch_table_pick(d, lens, sel, n_sel, ws, s);
  } else if (path == TopkPath::kScan) {
    ScanWs w = carve_scan(d, ws, nullptr);
    const ScanGeom g = scan_geom(d);
    const dim3 grid((unsigned)g.n_slices, (unsigned)((d.Nq + 3) / 4), (unsigned)d.B);
    QSA_LAUNCH(scan_filter_kernel, grid, dim3(kScanThreads), 0, s, q_idx, k_cmp, lens,
               fuse ? fuse->k_idx : nullptr, fuse ? fuse->first_block : nullptr, w.seg, w.cnt,
               d.Lmax, d.Nq, g.slice_blocks, g.n_slices);
    QSA_LAUNCH(scan_select_kernel, grid_q, dim3(kScanThreads), 0, s, (const uint64_t*)w.seg,
               (const uint32_t*)w.cnt, q_idx, (const uint16_t*)k_cmp, lens, sel, n_sel, d.Lmax,
               d.Nq, g.slice_blocks, g.n_slices);
  } else {
    StreamWs w = carve_stream(d, ws, nullptr);
    const int nbp = d.Lmax / 4;
    const int ncol_pad = (nbp + kColTile - 1) / kColTile;
    QSA_LAUNCH(frag_order_kernel, dim3((unsigned)(((size_t)nbp * 8 + 255) / 256), (unsigned)d.B),
               dim3(256), 0, s, reinterpret_cast<const uint4*>(k_cmp), w.frag, lens, d.Lmax,
               d.Nq, ncol_pad);
    const dim3 grid((unsigned)((d.Nq + kStreamQ - 1) / kStreamQ), (unsigned)d.B);
    QSA_LAUNCH(score_stream_kernel, grid, dim3(64 * kStreamWaves), 0, s, q_idx,
               (const uint4*)w.frag, lens, w.lists, w.cnt, w.tau, d.Lmax, d.Nq);
    QSA_LAUNCH(select_kernel<true>, grid_q, dim3(256), 0, s, w.lists, w.cnt, 1, kListCap,
               (const int32_t*)w.tau, (const uint32_t*)nullptr, 0, q_idx, k_cmp, lens, sel, n_sel,
               d.Lmax, d.Nq);
  }
  return hipGetLastError();
}

}  // namespace qsa
