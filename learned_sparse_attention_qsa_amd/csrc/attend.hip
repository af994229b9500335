// Core attention over the selected tokens (sparse) and over the whole
// causal context (dense comparator).
//
// Method (page "Qwen's million-token window has a 2,048-token keyhole"):
// core attention runs only over the expanded token positions (section "A
// million-token window with a selective view"); the dense baseline the pages
// compare against is grouped-query attention (section "Three speed claims,
// three different experiments").  Query head h reads KV head floor(h/G).
//
// Layout of the work.  A wavefront owns one KV head and up to 16 query heads
// of that group (the sparse kernel: the heads of one query; the dense decode
// kernel: 16 (query, head) columns of one sequence, the workgroup's
// wavefronts sharing the K/V stream; the dense prefill kernel, which stages
// 64-token K/V tiles in LDS, is described at its definition).  It walks the
// tokens in tiles of 32:
//   * S^T = K Q^T with MFMA 16x16x32: K rows are gathered straight from HBM
//     into the A operand (each lane loads 16 contiguous bytes of one row),
//     the stationary Q fragment is the B operand;
//   * online softmax in fp32 registers (exp2 domain), one running max and sum
//     per query head;
//   * O^T += V^T P with MFMA: P already sits in the B-operand layout, V goes
//     through a per-wavefront LDS tile and is read back transposed.
// Long token ranges are split across workgroups; partial (o, lse) pairs are
// merged by merge_kernel.  Paged K/V: the same kernels read token rows
// through a page table (pool row = table[b][t / page] * page +
// t mod page).  The file also holds the indexer's training target (dense
// attention mass pooled per micro-block) and the recall of a selection.
#include "common.h"
#include "internal.h"

namespace qsa {
namespace {

constexpr int kTile = 32;        // tokens per step
constexpr int kVStride = 136;    // LDS row stride (elements) of a V tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Eight probabilities (finite, >= 0) as an MFMA operand: hardware
// round-to-nearest-even conversion, pairwise.
__device__ __forceinline__ bf16x8 pack8_rne(const float* p) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  uint4 u;
  u.x = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){p[0], p[1]}, bf16x2));
  u.y = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){p[2], p[3]}, bf16x2));
  u.z = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){p[4], p[5]}, bf16x2));
  u.w = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){p[6], p[7]}, bf16x2));
  return as_bf16x8(u);
}

// Maximum over the four lanes L, L^16, L^32, L^48 (one MFMA output column):
// the gfx950 row-swap moves, no LDS round trip.
__device__ __forceinline__ float max_over_rows(float x) {
  const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
  x = fmaxf(__uint_as_float(s32[0]), __uint_as_float(s32[1]));
  const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
  return fmaxf(__uint_as_float(s16[0]), __uint_as_float(s16[1]));
}

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* lens;
  const int32_t* sel;
  const int32_t* n_sel;
  uint16_t* out;
  float* lse;
  float* part_o;    // [rows][Hq][n_split][128] when n_split > 1
  float* part_lse;  // [rows][Hq][n_split]
  int B, Lmax, Nq, Hq, Hkv, G;
  float scale_log2;
  int split_tokens, n_split;
  int tail_last;  // 1: the last split also takes the query's own block
  // paged K/V (pt != null): token tok of sequence b is row
  // pt[b * max_pages + tok / page] * page + tok % page of a pool of n_pages
  // pages of `page` tokens (page = 1 << page_shift)
  const int32_t* pt;
  int page_shift, max_pages, n_pages;
};

// Paged K/V: the pool row of token tok of sequence b (ids clamped into the pool).
__device__ __forceinline__ int pool_row(const AttnArgs& a, int b, int tok) {
  const int page = guard(a.pt[(size_t)b * a.max_pages + (tok >> a.page_shift)], 0, a.n_pages - 1);
  return (page << a.page_shift) + (tok & ((1 << a.page_shift) - 1));
}

// Element offset of token tok's row (all KV heads) of sequence b in K or V.
__device__ __forceinline__ long long kv_off(const AttnArgs& a, int b, int tok) {
  if (a.pt == nullptr) return ((long long)b * a.Lmax + tok) * a.Hkv * kHeadDim;
  return (long long)pool_row(a, b, tok) * a.Hkv * kHeadDim;
}

// Running softmax state of one wavefront: 16 query columns (one per lane
// column), 128 output dims as 8 tiles of 16.
struct Run {
  float m, l;
  f32x4 o[8];
};

__device__ __forceinline__ void run_init(Run& r) {
  r.m = kNegInf;
  r.l = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) r.o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// One 32-token step.  kf: K fragments of the two 16-token halves (A operand
// layout); z: scaled logits of this lane's 8 tokens (kNegInf when masked);
// vt: this wavefront's V tile in LDS (token-major, kVStride).
__device__ __forceinline__ void softmax_pv(Run& r, float* z, const uint16_t* vt) {
  const int lane = lane_id();
  float tmax = z[0];
#pragma unroll
  for (int e = 1; e < 8; ++e) tmax = fmaxf(tmax, z[e]);
  tmax = max_over_rows(tmax);
  const float m_new = fmaxf(r.m, tmax);
  // A column with every logit masked so far keeps m = -inf; guard the exp2.
  const float m_use = m_new == kNegInf ? 0.f : m_new;
  const float alpha = __builtin_amdgcn_exp2f(r.m - m_use);
  float p[8];
  float ps = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    p[e] = __builtin_amdgcn_exp2f(z[e] - m_use);
    ps += p[e];
  }
  r.l = r.l * alpha + ps;
  r.m = m_new;
  const bf16x8 pf = pack8_rne(p);
  const int g = lane >> 4;
  const int dl = lane & 15;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    const uint16_t* col = vt + dt * 16 + dl;
    uint4 u;
    u.x = (uint32_t)col[(4 * g + 0) * kVStride] | ((uint32_t)col[(4 * g + 1) * kVStride] << 16);
    u.y = (uint32_t)col[(4 * g + 2) * kVStride] | ((uint32_t)col[(4 * g + 3) * kVStride] << 16);
    u.z = (uint32_t)col[(16 + 4 * g + 0) * kVStride] |
          ((uint32_t)col[(16 + 4 * g + 1) * kVStride] << 16);
    u.w = (uint32_t)col[(16 + 4 * g + 2) * kVStride] |
          ((uint32_t)col[(16 + 4 * g + 3) * kVStride] << 16);
    r.o[dt] = r.o[dt] * alpha;
    r.o[dt] = mfma16(as_bf16x8(u), pf, r.o[dt]);
  }
}

// A 32-token tile of one KV head, in registers: the K fragments of the two
// 16-token halves (MFMA A-operand layout: lane -> token lane&15, 16 bytes at
// dims ks*32 + (lane>>4)*8) and the V rows (v[i]: lane -> token 4i + lane/16,
// 16 bytes at dims (lane&15)*8, so that 16 lanes read one 256-byte row).
struct KVTile {
  uint4 k[2][4];
  uint4 v[8];
};

// kv_row(kk) returns the element offset of token-list entry kk's row for this
// KV head, or -1 when kk is past the end of the range.
template <typename RowOf>
__device__ __forceinline__ void load_tile(KVTile& t, const uint16_t* kbase, const uint16_t* vbase,
                                          int k0, RowOf row_of) {
  const int lane = lane_id();
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const long long off = row_of(k0 + s * 16 + (lane & 15));
    const uint4* kp = reinterpret_cast<const uint4*>(kbase + (off < 0 ? 0 : off));
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) t.k[s][ks] = off >= 0 ? kp[ks * 4 + (lane >> 4)] : zero_u4();
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const long long off = row_of(k0 + 4 * i + (lane >> 4));
    const uint4* vp = reinterpret_cast<const uint4*>(vbase + (off < 0 ? 0 : off)) + (lane & 15);
    t.v[i] = off >= 0 ? *vp : zero_u4();
  }
}

__device__ __forceinline__ void stash_v(uint16_t* vt, const KVTile& t) {
  const int lane = lane_id();
#pragma unroll
  for (int i = 0; i < 8; ++i)
    *reinterpret_cast<uint4*>(vt + (4 * i + (lane >> 4)) * kVStride + (lane & 15) * 8) = t.v[i];
}

// Logits of this lane's 8 tokens (two 16-token halves x 4 rows of the MFMA
// output), already scaled to the exp2 domain.
__device__ __forceinline__ void qk_logits(const KVTile& t, const bf16x8* qf, float scale_log2,
                                          float* z) {
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) acc = mfma16(as_bf16x8(t.k[s][ks]), qf[ks], acc);
#pragma unroll
    for (int i = 0; i < 4; ++i) z[s * 4 + i] = acc[i] * scale_log2;
  }
}

// Final per-column reduction and store.  Column c = lane & 15.
__device__ __forceinline__ void finish(const Run& r, bool col_valid, uint16_t* out_row,
                                       float* lse_ptr, float* po, float* pl, bool partial) {
  const int lane = lane_id();
  float l = r.l;
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const float lse_v = l > 0.f ? (r.m + __log2f(l)) * kLn2 : kNegInf;
  if (!col_valid) return;
  const int g = lane >> 4;
  if (partial) {
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      float4 w = make_float4(r.o[dt][0] * inv, r.o[dt][1] * inv, r.o[dt][2] * inv, r.o[dt][3] * inv);
      *reinterpret_cast<float4*>(po + dt * 16 + g * 4) = w;
    }
    if (g == 0) *pl = lse_v;
  } else {
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      uint2 w;
      w.x = f32_to_bf16(r.o[dt][0] * inv) | (f32_to_bf16(r.o[dt][1] * inv) << 16);
      w.y = f32_to_bf16(r.o[dt][2] * inv) | (f32_to_bf16(r.o[dt][3] * inv) << 16);
      *reinterpret_cast<uint2*>(out_row + dt * 16 + g * 4) = w;
    }
    if (g == 0 && lse_ptr) *lse_ptr = lse_v;
  }
}

// ------------------------------------------------------------------ sparse
// A unit is (query row, KV head g, chunk of <= 16 query heads of g's
// group); unit u = (q * Hkv + g) * hchunks + hc.  Grid (Nq * Hkv * hchunks /
// kUnits, n_split, B): one workgroup per kUnits consecutive units of one
// query and one token split.  Wavefront w serves unit w mod kUnits and takes
// every (kWaves / kUnits)-th 32-token tile of the split from tile
// w / kUnits on, with its own online softmax; the wavefronts of a unit are
// merged in LDS.  With kUnits = 4 the four KV heads of a query sit in one
// workgroup and read their 256-byte pieces of each token's 1 KiB K and V
// rows in step, so a row is fetched whole.  With one split the result is
// final; otherwise the workgroup writes a partial (o, lse) that merge_kernel
// combines.  (A merge by the last workgroup to arrive would need a
// device-scope fence per workgroup, and on this chip such a fence writes
// back the whole L2 of its XCD.)  kMulti false: every wavefront has at most
// one 32-token tile.  kUnits > 1 needs G <= 16 (one head chunk per KV head).
template <bool kMulti, int kWaves, int kUnits>
__global__ __launch_bounds__(64 * kWaves) void sparse_attend_kernel(AttnArgs a) {
  constexpr int kThreads = 64 * kWaves;
  constexpr int kWpu = kWaves / kUnits;      // wavefronts per unit
  constexpr int kSelPer = kTopK / kThreads;  // selection entries each thread prefetches
  static_assert(kWaves % kUnits == 0, "whole wavefronts per unit");
  __shared__ int32_t s_sel[kTopK];
  __shared__ __align__(16) uint16_t s_v[kWaves][kTile * kVStride];  // V tiles; then merge scratch
  __shared__ float s_m[kWaves][16], s_l[kWaves][16], s_f[kWaves][16], s_inv[kUnits][16];
  const int split = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int wu = wave % kUnits, wi = wave / kUnits;  // unit of this wavefront, rank in it
  const int unit = blockIdx.x * kUnits + wu;
  const int hchunks = (a.G + 15) >> 4;
  const int q = unit / (a.Hkv * hchunks);
  const int g = (unit / hchunks) % a.Hkv, hc = unit % hchunks;
  const size_t row = (size_t)b * a.Nq + q;
  const int len = guard_len(a.lens[b], a.Nq, a.Lmax);
  const int t = len - a.Nq + q;
  const int k_begin = split * a.split_tokens;
  // This split's slice of the selection, loaded before n_sel is known (the
  // loads do not wait on each other): blocks [kb0, kb0 + split_tokens / 4).
  const int kb0 = k_begin >> 2;
  const int nsb = min(a.split_tokens >> 2, kTopK - kb0);  // <= 512 = kSelPer per thread
  int32_t my_sel[kSelPer];
#pragma unroll
  for (int i = 0; i < kSelPer; ++i)
    my_sel[i] = tid + kThreads * i < nsb ? a.sel[row * kTopK + kb0 + tid + kThreads * i] : 0;
  const int h0 = g * a.G + hc * 16;
  const int nh = min(16, a.G - hc * 16);
  const int col = lane & 15;
  bf16x8 qf[4];
  {
    const uint4* qp =
        reinterpret_cast<const uint4*>(a.q + (row * a.Hq + h0 + min(col, nh - 1)) * kHeadDim);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[ks] = as_bf16x8(col < nh ? qp[ks * 4 + (lane >> 4)] : zero_u4());
  }
  int ns = 0, ntok = 0, bt = 0;
  if (t >= 0) {
    bt = t >> 2;
    ns = guard(a.n_sel[row], 0, bt < kTopK ? bt : kTopK);
    ntok = 4 * ns + (t - 4 * bt) + 1;
  }
  const uint16_t* kbase = a.k + g * kHeadDim;
  const uint16_t* vbase = a.v + g * kHeadDim;
  // With tail_last, the query's own block (tokens 4 bt .. t, known from lens
  // alone) is wavefront 0's extra tile in the last split: its rows are
  // requested now, before the selection arrives, and it is processed ahead
  // of the selected tiles, so that it does not add a round trip at the end.
  const bool own_tail = kMulti && a.tail_last && split == a.n_split - 1 && wi == 0 && t >= 0;
  KVTile tail;
  if (own_tail)
    load_tile(tail, kbase, vbase, 0, [&](int kk) -> long long {
      const int tok = 4 * (t >> 2) + kk;
      return tok <= t ? kv_off(a, b, tok) : -1;
    });
  // ids outside [0, bt) are a caller bug: clamped so no access leaves the
  // row.  Paged K/V with pages of 4 tokens or more: a block lies inside one
  // page, so its id is replaced here, once, by the pool row of its first
  // token, and the tiles read rows without a table lookup.
  const bool paged4 = a.pt != nullptr && a.page_shift >= 2;
#pragma unroll
  for (int i = 0; i < kSelPer; ++i) {
    const int e = tid + kThreads * i;
    if (e < nsb && kb0 + e < ns) {
      const int j = guard(my_sel[i], 0, bt - 1);
      s_sel[e] = paged4 ? pool_row(a, b, 4 * j) : j;
    }
  }
  __syncthreads();
  // the selected tokens of this split (with tail_last the query's own block
  // is handled apart, above; otherwise it follows the selected ones)
  const int k_end = a.tail_last ? min(4 * ns, k_begin + a.split_tokens)
                                : min(ntok, k_begin + a.split_tokens);
  auto row_of = [&](int kk) -> long long {
    if (kk >= k_end) return -1;
    if (kk < 4 * ns) {
      const int e = s_sel[(kk >> 2) - kb0];
      return paged4 ? ((long long)e + (kk & 3)) * a.Hkv * kHeadDim : kv_off(a, b, 4 * e + (kk & 3));
    }
    return kv_off(a, b, 4 * bt + (kk - 4 * ns));
  };
  uint16_t* vt = s_v[wave];
  Run r;
  run_init(r);
  KVTile cur;
  const int first = k_begin + wi * kTile;
  if (first < k_end) load_tile(cur, kbase, vbase, first, row_of);
  if (own_tail) {
    stash_v(vt, tail);
    float z[8];
    qk_logits(tail, qf, a.scale_log2, z);
    const int n_own = t - 4 * bt + 1;  // 1..4 tokens
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (s2 * 16 + (lane >> 4) * 4 + i >= n_own) z[s2 * 4 + i] = kNegInf;
    wave_sync_lds();
    softmax_pv(r, z, vt);
    wave_sync_lds();
  }
  for (int k0 = first; k0 < k_end; k0 += kWpu * kTile) {
    stash_v(vt, cur);
    KVTile nxt;
    if (kMulti && k0 + kWpu * kTile < k_end)
      load_tile(nxt, kbase, vbase, k0 + kWpu * kTile, row_of);
    float z[8];
    qk_logits(cur, qf, a.scale_log2, z);
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (k0 + s * 16 + (lane >> 4) * 4 + i >= k_end) z[s * 4 + i] = kNegInf;
    wave_sync_lds();
    softmax_pv(r, z, vt);
    wave_sync_lds();
    if (!kMulti) break;
    cur = nxt;
  }
  // ---- merge the wavefronts (LDS)
  float l = r.l;
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  __syncthreads();  // every wavefront is done with its V tile: reuse s_v
  // [kWaves][16][kOStride]: a column's 128 floats padded to 132 so that the
  // 16 columns' float4 stores of one wavefront hit distinct banks
  constexpr int kOStride = kHeadDim + 4;
  static_assert(kOStride * 16 * 4 <= kTile * kVStride * 2, "merge scratch fits the V tiles");
  float* O = reinterpret_cast<float*>(&s_v[0][0]);
  {
    const int gq = lane >> 4;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
      *reinterpret_cast<float4*>(O + (wave * 16 + col) * kOStride + dt * 16 + gq * 4) =
          make_float4(r.o[dt][0], r.o[dt][1], r.o[dt][2], r.o[dt][3]);
    if (lane < 16) {
      s_m[wave][lane] = r.m;
      s_l[wave][lane] = l;
    }
  }
  __syncthreads();
  const bool partial = a.n_split > 1;
  // first query head of unit uu of this workgroup (every unit of a workgroup
  // has the same nh: kUnits > 1 only with one head chunk per KV head)
  auto head0 = [&](int uu) -> int {
    const int un = blockIdx.x * kUnits + uu;
    return ((un / hchunks) % a.Hkv) * a.G + (un % hchunks) * 16;
  };
  if (tid < 16 * kUnits) {
    const int uu = tid >> 4, c = tid & 15;
    float M = kNegInf;
    for (int j = 0; j < kWpu; ++j) M = fmaxf(M, s_m[uu + kUnits * j][c]);
    float L = 0.f;
    for (int j = 0; j < kWpu; ++j) {
      const int w = uu + kUnits * j;
      const float f = (M == kNegInf || s_m[w][c] == kNegInf) ? 0.f : exp2f(s_m[w][c] - M);
      s_f[w][c] = f;
      L += f * s_l[w][c];
    }
    s_inv[uu][c] = L > 0.f ? 1.f / L : 0.f;
    const float lse_v = L > 0.f ? (M + __log2f(L)) * kLn2 : kNegInf;
    if (c < nh) {
      const size_t rh = row * a.Hq + head0(uu) + c;
      if (partial)
        a.part_lse[rh * a.n_split + split] = lse_v;
      else if (a.lse)
        a.lse[rh] = lse_v;
    }
  }
  __syncthreads();
  for (int i = tid; i < kUnits * nh * kHeadDim; i += blockDim.x) {
    const int uu = kUnits == 1 ? 0 : i / (nh * kHeadDim);
    const int rem = i - uu * nh * kHeadDim;
    const int c = rem >> 7, d = rem & 127;
    float o = 0.f;
#pragma unroll
    for (int j = 0; j < kWpu; ++j) {
      const int w = uu + kUnits * j;
      o += s_f[w][c] * O[(w * 16 + c) * kOStride + d];
    }
    o *= s_inv[uu][c];
    const size_t rh = row * a.Hq + head0(uu) + c;
    if (partial)
      a.part_o[(rh * a.n_split + split) * kHeadDim + d] = o;
    else
      a.out[rh * kHeadDim + d] = (uint16_t)f32_to_bf16(o);
  }
}

// ------------------------------------------------------------------ dense
// Column units: chunk cc of 16 (query, head) columns of KV head g is unit
// g * cchunks + cc, cchunks = ceil(Nq*G/16).  Grid (n_split, ceil(units / 8),
// B); a workgroup holds up to eight wavefronts, one per unit, and each walks
// all tokens 0..len-1 of the split range with a causal mask per column.  The
// wavefronts of a workgroup read the same tokens in step: the chunks of one
// KV head share its rows, and the KV heads' rows of a token are adjacent
// 256-byte pieces of one 1 KiB row, so each token's K and V cross the fabric
// once, as whole rows.  Always writes partials (merged by merge_kernel).
constexpr int kDenseWaves = 8;
// kPaged: K/V rows through the page table.  The page ids of a tile's 32
// tokens (lane x holds token T + x's) are loaded one tile ahead of the
// tile's own loads, and each lane takes its rows' ids by shuffle, so the
// table adds no round trip to the tile pipeline.
template <bool kPaged>
__global__ __launch_bounds__(64 * kDenseWaves) void dense_decode_kernel(AttnArgs a) {
  __shared__ __align__(16) uint16_t s_vw[kDenseWaves][kTile * kVStride];
  const int split = blockIdx.x, b = blockIdx.z;
  const int cchunks = (a.Nq * a.G + 15) >> 4;
  const int wave = threadIdx.x >> 6;
  const int u = blockIdx.y * kDenseWaves + wave;
  if (u >= a.Hkv * cchunks) return;  // (no workgroup barrier below)
  const int g = u / cchunks, cc = u % cchunks;
  uint16_t* s_v = s_vw[wave];
  const int lane = lane_id();
  const int len = guard_len(a.lens[b], a.Nq, a.Lmax);
  const int col = lane & 15;
  const int c = cc * 16 + col;  // (query, head) column
  const bool col_valid = c < a.Nq * a.G;
  const int qi = col_valid ? c / a.G : 0;
  const int h = g * a.G + (col_valid ? c % a.G : 0);
  const int tq = len - a.Nq + qi;  // last visible token of this column
  const size_t row = (size_t)b * a.Nq + qi;
  bf16x8 qf[4];
  {
    const uint4* qp = reinterpret_cast<const uint4*>(a.q + (row * a.Hq + h) * kHeadDim);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      qf[ks] = as_bf16x8(col_valid && tq >= 0 ? qp[ks * 4 + (lane >> 4)] : zero_u4());
  }
  // the last token any column of this chunk may see
  const int c_last = min(cc * 16 + 15, a.Nq * a.G - 1);
  const int t_hi = len - a.Nq + c_last / a.G;
  const int k_begin = split * a.split_tokens;
  const int k_end = min(t_hi + 1, k_begin + a.split_tokens);
  const uint16_t* kbase = a.k + g * kHeadDim;
  const uint16_t* vbase = a.v + g * kHeadDim;
  auto row_of = [&](int kk) -> long long { return kk < k_end ? kv_off(a, b, kk) : -1; };
  // (the id is checked where it is used, so that nothing waits for the
  // load early)
  auto page_ids = [&](int T) -> int {
    const int tok = min(T + (lane & 31), k_end - 1);
    return a.pt[(size_t)b * a.max_pages + (tok >> a.page_shift)];
  };
  auto paged_row = [&](int T, int pe) {
    return [&, T, pe](int kk) -> long long {
      const int page = guard(__shfl(pe, (kk - T) & 31), 0, a.n_pages - 1);
      if (kk >= k_end) return -1;
      return (((long long)page << a.page_shift) + (kk & ((1 << a.page_shift) - 1))) * a.Hkv *
             kHeadDim;
    };
  };
  Run r;
  run_init(r);
  KVTile cur, nxt;
  int pe_nxt = 0;  // page ids of the tile after the one in flight
  if (k_begin < k_end) {
    if constexpr (kPaged) {
      load_tile(cur, kbase, vbase, k_begin, paged_row(k_begin, page_ids(k_begin)));
      pe_nxt = page_ids(k_begin + kTile);
    } else {
      load_tile(cur, kbase, vbase, k_begin, row_of);
    }
  }
  for (int k0 = k_begin; k0 < k_end; k0 += kTile) {
    stash_v(s_v, cur);
    int pe_after = 0;
    if constexpr (kPaged) {
      if (k0 + kTile < k_end) load_tile(nxt, kbase, vbase, k0 + kTile, paged_row(k0 + kTile, pe_nxt));
      // (unconditional: past the end it reads the last token's id; a
      // conditional load would be waited for at the iteration's end)
      pe_after = page_ids(k0 + 2 * kTile);
    } else {
      if (k0 + kTile < k_end) load_tile(nxt, kbase, vbase, k0 + kTile, row_of);
    }
    float z[8];
    qk_logits(cur, qf, a.scale_log2, z);
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kk = k0 + s * 16 + (lane >> 4) * 4 + i;
        if (kk >= k_end || kk > tq) z[s * 4 + i] = kNegInf;
      }
    wave_sync_lds();
    softmax_pv(r, z, s_v);
    wave_sync_lds();
    cur = nxt;
    pe_nxt = pe_after;
  }
  float* po = a.part_o + (((row * a.Hq) + h) * a.n_split + split) * kHeadDim;
  float* pl = a.part_lse + ((row * a.Hq) + h) * a.n_split + split;
  finish(r, col_valid, nullptr, nullptr, po, pl, true);
}

// ------------------------------------------------------------------ teacher
// The indexer's training target: dense attention probabilities pooled per
// micro-block and averaged over the query heads,
//   T[b][i][j] = (1/Hq) sum_h sum_{s in block j, s <= t} exp(scale q_h.k_s - lse_h)
// with lse_h the dense causal log-sum-exp of head h (from the dense pass).
// Same grid and column units as dense_decode_kernel, K only: a lane's eight
// logits of a 32-token tile (qk_logits) are the four tokens of one
// micro-block in each 16-token half, so the lane sums them into its
// column's mass of that block; the columns of one query (G consecutive
// lanes when G divides 16) are summed across lanes and one lane adds the
// result to T, which the launcher clears first.
__global__ __launch_bounds__(64 * kDenseWaves) void block_teacher_kernel(AttnArgs a,
                                                                         const float* __restrict__ lse_dense,
                                                                         float* __restrict__ teacher) {
  const int split = blockIdx.x, b = blockIdx.z;
  const int cchunks = (a.Nq * a.G + 15) >> 4;
  const int wave = threadIdx.x >> 6;
  const int u = blockIdx.y * kDenseWaves + wave;
  if (u >= a.Hkv * cchunks) return;  // (no workgroup barrier below)
  const int g = u / cchunks, cc = u % cchunks;
  const int lane = lane_id();
  const int len = guard_len(a.lens[b], a.Nq, a.Lmax);
  const int col = lane & 15;
  const int c = cc * 16 + col;  // (query, head) column
  const bool col_valid = c < a.Nq * a.G;
  const int qi = col_valid ? c / a.G : 0;
  const int h = g * a.G + (col_valid ? c % a.G : 0);
  const int tq = len - a.Nq + qi;
  const size_t row = (size_t)b * a.Nq + qi;
  bf16x8 qf[4];
  {
    const uint4* qp = reinterpret_cast<const uint4*>(a.q + (row * a.Hq + h) * kHeadDim);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      qf[ks] = as_bf16x8(col_valid && tq >= 0 ? qp[ks * 4 + (lane >> 4)] : zero_u4());
  }
  const float lse2 = col_valid && tq >= 0 ? lse_dense[row * a.Hq + h] * kLog2e : 0.f;
  const int c_last = min(cc * 16 + 15, a.Nq * a.G - 1);
  const int t_hi = len - a.Nq + c_last / a.G;
  const int k_begin = split * a.split_tokens;  // a multiple of 32
  const int k_end = min(t_hi + 1, k_begin + a.split_tokens);
  const uint16_t* kbase = a.k + g * kHeadDim;
  const int nbp = a.Lmax >> 2;
  const bool grouped = a.G <= 16 && (16 % a.G) == 0;
  const float inv_hq = 1.0f / (float)a.Hq;
  KVTile cur;
  auto load_k = [&](KVTile& t, int k0) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int kk = k0 + s * 16 + (lane & 15);
      const uint4* kp = reinterpret_cast<const uint4*>(kbase + kv_off(a, b, min(kk, len > 0 ? len - 1 : 0)));
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) t.k[s][ks] = kk < k_end ? kp[ks * 4 + (lane >> 4)] : zero_u4();
    }
  };
  if (k_begin < k_end) load_k(cur, k_begin);
  for (int k0 = k_begin; k0 < k_end; k0 += kTile) {
    KVTile nxt;
    if (k0 + kTile < k_end) load_k(nxt, k0 + kTile);
    float z[8];
    qk_logits(cur, qf, a.scale_log2, z);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int tok0 = k0 + s * 16 + (lane >> 4) * 4;  // the block's first token
      float m = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kk = tok0 + i;
        m += (col_valid && kk <= tq && kk < k_end) ? exp2f(z[s * 4 + i] - lse2) : 0.f;
      }
      m *= inv_hq;
      const int jb = tok0 >> 2;
      if (grouped) {
        // sum over the G lanes of the query (consecutive lanes of the row)
        for (int off = 1; off < a.G; off <<= 1) m += __shfl_xor(m, off);
        if ((col % a.G) == 0 && col_valid && tok0 <= tq && m != 0.f)
          atomicAdd(&teacher[row * nbp + jb], m);
      } else if (col_valid && tok0 <= tq && m != 0.f) {
        atomicAdd(&teacher[row * nbp + jb], m);
      }
    }
    cur = nxt;
  }
}

// ------------------------------------------------------------------ dense prefill
// Dense causal GQA over positions 0..t of every query (the comparator of a
// prefill chunk, contiguous or paged K/V).  Grid (ceil(Nq / QW), Hkv, B),
// 512 threads: one KV head g and QW = floor(256 / G) consecutive queries,
// whose (query, head) columns the 8 wavefronts hold 32 apiece (two 16-column
// MFMA groups sharing every K and V operand).  The workgroup walks tokens
// 0 .. t of its last query in 64-token tiles staged once in LDS for all its
// wavefronts: K row-major (the A operand of S^T = K Q^T), V transposed to
// dims x tokens so that the A operand of O^T += V^T P is two 8-byte reads.
// The next tile's global loads are issued before the current tile's MFMA
// work.  Causal masking is per column (tokens after its query).
constexpr int kPrefWaves = 8;
constexpr int kPrefTok = 64;
constexpr int kPrefVtStride = 72;  // elements per transposed-V row (one dim)


// Position of token tau (0..31 of a 32-token half) in a transposed V row:
// the eight tokens one lane group g = (tau >> 2) & 3 feeds to the PV MFMA
// (4g..4g+3 and 16+4g..16+4g+3) are stored contiguously, so the A operand
// is one 16-byte read.
__device__ __forceinline__ int vt_pos(int tau) {
  return (((tau >> 2) & 3) << 3) | ((tau >> 4) << 2) | (tau & 3);
}

// kPaged: K/V through the page table.  The page ids of the rows an
// iteration requests at its end are loaded at its start, so the table read
// completes under the iteration's MFMA work; a page id carried from one
// iteration to the next would instead make the compiler wait, at the loop's
// back edge, for every load issued before it (the row prefetches too).
template <bool kPaged>
__global__ __launch_bounds__(64 * kPrefWaves) void dense_prefill_kernel(AttnArgs a) {
  __shared__ __align__(16) uint16_t s_k[2][kPrefTok * kVStride];
  __shared__ __align__(16) uint16_t s_vt[2][kHeadDim * kPrefVtStride];
  const int qt = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = lane_id();
  const int qw = 16 * 2 * kPrefWaves / a.G;  // queries per workgroup
  const int len = guard_len(a.lens[b], a.Nq, a.Lmax);
  const float c2 = a.scale_log2;
  bf16x8 qf[2][4];
  int tq[2];
  bool cv[2];
  size_t rh[2];  // (row, head) index of each column group's column
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int c = wave * 32 + j * 16 + (lane & 15);
    const int qi = qt * qw + c / a.G;
    cv[j] = c < qw * a.G && qi < a.Nq;
    tq[j] = len - a.Nq + qi;
    rh[j] = ((size_t)b * a.Nq + (cv[j] ? qi : 0)) * a.Hq + g * a.G + c % a.G;
    const uint4* qp = reinterpret_cast<const uint4*>(a.q + rh[j] * kHeadDim);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      qf[j][ks] = as_bf16x8(cv[j] && tq[j] >= 0 ? qp[ks * 4 + (lane >> 4)] : zero_u4());
  }
  const int q_last = min(qt * qw + qw - 1, a.Nq - 1);
  const int t_hi = len - a.Nq + q_last;  // the workgroup's last token
  const int t_lo = len - a.Nq + qt * qw; // its first query's last token
  const int n_tiles = t_hi >= 0 ? t_hi / kPrefTok + 1 : 0;
  // A thread's share of a tile: token 64 i + lane, 16-byte pieces wave and
  // wave + 8 of its K or V row (a token past t_hi reads t_hi's row, which
  // the masks then ignore).
  auto row_ptr = [&](const uint16_t* base, int i) -> const uint4* {
    const int tok = min(i * kPrefTok + lane, t_hi);
    const long long row = kPaged ? (long long)pool_row(a, b, tok) : (long long)b * a.Lmax + tok;
    return reinterpret_cast<const uint4*>(base + row * a.Hkv * kHeadDim + (long long)g * kHeadDim);
  };
  // paged: the page id of this thread's token of tile i (a load, checked
  // only where it is used, so that nothing waits for it early), and the row
  // of that token given its page id
  auto page_of = [&](int i) -> int {
    const int tok = min(i * kPrefTok + lane, t_hi);
    return a.pt[(size_t)b * a.max_pages + (tok >> a.page_shift)];
  };
  auto row_in = [&](const uint16_t* base, int i, int page) -> const uint4* {
    const int tok = min(i * kPrefTok + lane, t_hi);
    page = guard(page, 0, a.n_pages - 1);
    const long long r = ((long long)page << a.page_shift) + (tok & ((1 << a.page_shift) - 1));
    return reinterpret_cast<const uint4*>(base + r * a.Hkv * kHeadDim + (long long)g * kHeadDim);
  };

  const int vcol = (lane & 32) | vt_pos(lane & 31);  // this thread's token in a V^T row
  auto stash_k = [&](int buf, uint4 r0, uint4 r1) {
    *reinterpret_cast<uint4*>(&s_k[buf][lane * kVStride + wave * 8]) = r0;
    *reinterpret_cast<uint4*>(&s_k[buf][lane * kVStride + (wave + 8) * 8]) = r1;
  };
  auto stash_v1 = [&](int buf, int piece, uint4 r) {
    uint16_t* d = &s_vt[buf][piece * 8 * kPrefVtStride + vcol];
    d[0 * kPrefVtStride] = (uint16_t)r.x;
    d[1 * kPrefVtStride] = (uint16_t)(r.x >> 16);
    d[2 * kPrefVtStride] = (uint16_t)r.y;
    d[3 * kPrefVtStride] = (uint16_t)(r.y >> 16);
    d[4 * kPrefVtStride] = (uint16_t)r.z;
    d[5 * kPrefVtStride] = (uint16_t)(r.z >> 16);
    d[6 * kPrefVtStride] = (uint16_t)r.w;
    d[7 * kPrefVtStride] = (uint16_t)(r.w >> 16);
  };
  auto stash_v = [&](int buf, uint4 r0, uint4 r1) {
    stash_v1(buf, wave, r0);
    stash_v1(buf, wave + 8, r1);
  };
  // S^T of tile i from K buffer `buf`: z[j][4 qr + e] is token 64 i + 16 qr +
  // 4 (lane >> 4) + e of column group j, raw logits, causally masked on or
  // past the diagonal.
  auto qk = [&](int buf, int i, float (&z)[2][16]) {
    const uint16_t* sk = s_k[buf];
#pragma unroll
    for (int qr = 0; qr < 4; ++qr) {
      uint4 kf[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        kf[ks] = *reinterpret_cast<const uint4*>(
            &sk[(qr * 16 + (lane & 15)) * kVStride + ks * 32 + (lane >> 4) * 8]);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) acc = mfma16(as_bf16x8(kf[ks]), qf[j][ks], acc);
#pragma unroll
        for (int e = 0; e < 4; ++e) z[j][qr * 4 + e] = acc[e];
      }
    }
    const int k0 = i * kPrefTok;
    if (k0 + kPrefTok - 1 > t_lo) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int kk = k0 + (e >> 2) * 16 + (lane >> 4) * 4 + (e & 3);
          if (!cv[j] || kk > tq[j]) z[j][e] = kNegInf;
        }
    }
  };
  // running softmax per column group: m in the exp2 domain, l, O^T tiles
  float m[2] = {kNegInf, kNegInf}, l[2] = {0.f, 0.f};
  f32x4 o[2][8];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[j][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Software pipeline over tiles i = 0 .. n_tiles-1, one barrier per tile.
  // Iteration i computes S of tile i+1 (K buffer (i+1)&1) while it finishes
  // the softmax and PV of tile i (V buffer i&1), then stores K(i+2) into K
  // buffer i&1 and V(i+1) into V buffer (i+1)&1, both last read in iteration
  // i-1, and requests K(i+3) and V(i+2) from memory.
  float z[2][16], zn[2][16];
  uint4 rk0 = zero_u4(), rk1 = zero_u4(), rv0 = zero_u4(), rv1 = zero_u4();
  if (n_tiles > 0) {
    const uint4* kp = row_ptr(a.k, 0);
    const uint4* vp = row_ptr(a.v, 0);
    const uint4* kp1 = row_ptr(a.k, 1);
    stash_k(0, kp[wave], kp[wave + 8]);
    stash_v(0, vp[wave], vp[wave + 8]);
    stash_k(1, kp1[wave], kp1[wave + 8]);
  }
  // Every path into the loop has the Q fragments in registers: without this
  // wait the compiler, merging the paths, waits for every load in flight at
  // the first MFMA of each iteration.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0) only
  __syncthreads();
  if (n_tiles > 0) {
    qk(0, 0, z);
    const uint4* kp = row_ptr(a.k, 2);
    const uint4* vp = row_ptr(a.v, 1);
    rk0 = kp[wave];
    rk1 = kp[wave + 8];
    rv0 = vp[wave];
    rv1 = vp[wave + 8];
  }
  for (int i = 0; i < n_tiles; ++i) {
    const int cur = i & 1;
    // paged: ids of the rows requested at the end of this iteration (a tile
    // past the last reads the last token's id, unused)
    int pg_k = 0, pg_v = 0;
    if (kPaged) {
      pg_k = page_of(i + 3);
      pg_v = page_of(i + 2);
    }
    if (i + 1 < n_tiles) qk(cur ^ 1, i + 1, zn);
    float alpha[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      float tmax = z[j][0];
#pragma unroll
      for (int e = 1; e < 16; ++e) tmax = fmaxf(tmax, z[j][e]);
      tmax = max_over_rows(tmax);
      const float m_new = fmaxf(m[j], tmax * c2);
      // a column with every logit masked so far keeps m = -inf
      const float m_use = m_new == kNegInf ? 0.f : m_new;
      alpha[j] = __builtin_amdgcn_exp2f(m[j] - m_use);
      m[j] = m_new;
      float ps = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        z[j][e] = __builtin_amdgcn_exp2f(fmaf(z[j][e], c2, -m_use));
        ps += z[j][e];
      }
      l[j] = l[j] * alpha[j] + ps;
    }
    // the running maximum rarely moves once a few tiles are in: rescale O
    // only when it did for some column of the wavefront
    if (__ballot(alpha[0] != 1.f || alpha[1] != 1.f) != 0) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) o[j][dt] = o[j][dt] * alpha[j];
    }
    const uint16_t* svt = s_vt[cur];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const bf16x8 pf0 = pack8_rne(&z[0][h2 * 8]);
      const bf16x8 pf1 = pack8_rne(&z[1][h2 * 8]);
      const uint16_t* base = &svt[(lane & 15) * kPrefVtStride + h2 * 32 + 8 * (lane >> 4)];
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const bf16x8 u =
            as_bf16x8(*reinterpret_cast<const uint4*>(base + dt * 16 * kPrefVtStride));
        o[0][dt] = mfma16(u, pf0, o[0][dt]);
        o[1][dt] = mfma16(u, pf1, o[1][dt]);
      }
    }
    // Stores and loads are unconditional: tiles past the last read the last
    // token's rows and fill buffers no later iteration reads.  (Conditional
    // ones make the compiler's wait counts conservative at the merges, down
    // to waiting for every load in flight.)
    stash_k(cur, rk0, rk1);
    stash_v(cur ^ 1, rv0, rv1);
    {
      const uint4* kp = kPaged ? row_in(a.k, i + 3, pg_k) : row_ptr(a.k, i + 3);
      rk0 = kp[wave];
      rk1 = kp[wave + 8];
      const uint4* vp = kPaged ? row_in(a.v, i + 2, pg_v) : row_ptr(a.v, i + 2);
      rv0 = vp[wave];
      rv1 = vp[wave + 8];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) z[j][e] = zn[j][e];
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    Run r;
    r.m = m[j];
    r.l = l[j];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) r.o[dt] = o[j][dt];
    finish(r, cv[j], a.out + rh[j] * kHeadDim, a.lse ? a.lse + rh[j] : nullptr, nullptr, nullptr,
           false);
  }
}

__global__ void fill_f32_kernel(float* __restrict__ p, size_t n, float v) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = v;
}

// Share of the teacher's mass on the positions a row attends to: its kept
// blocks and its own block.  One workgroup (256 threads) per row.
__global__ __launch_bounds__(256) void teacher_recall_kernel(const float* __restrict__ teacher,
                                                             const int32_t* __restrict__ lens,
                                                             const int32_t* __restrict__ sel,
                                                             const int32_t* __restrict__ n_sel,
                                                             float* __restrict__ recall, int Lmax,
                                                             int Nq) {
  __shared__ float wsum[4];
  const int q = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const size_t row = (size_t)b * Nq + q;
  const int t = guard_len(lens[b], Nq, Lmax) - Nq + q;
  const int nbp = Lmax >> 2;
  float acc = 0.f;
  if (t >= 0) {
    const int bt = t >> 2;
    const int ns = guard(n_sel[row], 0, min(bt, kTopK));
    const float* tr = teacher + row * nbp;
    for (int i = tid; i < ns; i += blockDim.x) acc += tr[guard(sel[row * kTopK + i], 0, bt - 1)];
    if (tid == 0) acc += tr[bt];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
  if ((tid & 63) == 0) wsum[tid >> 6] = acc;
  __syncthreads();
  if (tid == 0) recall[row] = t >= 0 ? (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]) : 0.f;
}

// ------------------------------------------------------------------ merge
// Grid (Hq, Nq, B), 128 threads (one per output dim).  Combines the n_split
// partial (o, lse) pairs of one (query, head): o = sum_s e^(lse_s - M) o_s /
// sum_s e^(lse_s - M).  Up to kChunk partials: every load goes out at once,
// unconditionally (slots past n_split re-read the last partial and weigh 0),
// so they share one round trip; more partials are walked kChunk at a time.
template <int kChunk>
__global__ __launch_bounds__(128) void merge_kernel(const float* __restrict__ part_o,
                                                    const float* __restrict__ part_lse,
                                                    uint16_t* __restrict__ out,
                                                    float* __restrict__ lse, int Nq, int Hq,
                                                    int n_split) {
  const int h = blockIdx.x, q = blockIdx.y, b = blockIdx.z, d = threadIdx.x;
  const size_t rh = ((size_t)b * Nq + q) * Hq + h;
  const float* pl = part_lse + rh * n_split;
  const float* po = part_o + rh * n_split * kHeadDim + d;
  // A chunk's lse values and outputs are requested together (one memory
  // round trip per chunk, one in all for n_split <= kChunk); a later chunk
  // with a larger maximum rescales the sums so far.
  float M = kNegInf, acc = 0.f, sw = 0.f;
  for (int s0 = 0; s0 < n_split; s0 += kChunk) {
    float w[kChunk], v[kChunk];
#pragma unroll
    for (int s = 0; s < kChunk; ++s) {
      const int si = min(s0 + s, n_split - 1);
      w[s] = pl[si];
      v[s] = po[(size_t)si * kHeadDim];
    }
    float Mc = M;
#pragma unroll
    for (int s = 0; s < kChunk; ++s) Mc = fmaxf(Mc, w[s]);
    if (Mc == kNegInf) continue;  // nothing attended so far
    if (Mc > M) {
      const float r = __expf(M - Mc);  // 0 while M is -inf
      acc *= r;
      sw *= r;
      M = Mc;
    }
#pragma unroll
    for (int s = 0; s < kChunk; ++s) {
      const float e = (s0 + s < n_split && w[s] != kNegInf) ? __expf(w[s] - M) : 0.f;
      sw += e;
      acc += e * v[s];
    }
  }
  const float o = sw > 0.f ? acc / sw : 0.f;
  out[rh * kHeadDim + d] = (uint16_t)f32_to_bf16(o);
  if (lse && d == 0) lse[rh] = sw > 0.f ? M + __logf(sw) : kNegInf;
}

hipError_t launch_merge(const float* part_o, const float* part_lse, uint16_t* out, float* lse,
                        const Dims& d, int n_split, hipStream_t s) {
  const dim3 grid((unsigned)d.Hq, (unsigned)d.Nq, (unsigned)d.B);
  if (n_split <= 4)
    QSA_LAUNCH(merge_kernel<4>, grid, dim3(128), 0, s, part_o, part_lse, out, lse, d.Nq, d.Hq,
               n_split);
  else if (n_split <= 8)
    QSA_LAUNCH(merge_kernel<8>, grid, dim3(128), 0, s, part_o, part_lse, out, lse, d.Nq, d.Hq,
               n_split);
  else
    QSA_LAUNCH(merge_kernel<16>, grid, dim3(128), 0, s, part_o, part_lse, out, lse, d.Nq, d.Hq,
               n_split);
  return hipGetLastError();
}

int sparse_units(const Dims& d) {
  const int G = d.Hq / d.Hkv;
  return d.Nq * d.Hkv * ((G + 15) / 16);
}

// Workgroups a decode-sized sparse attention aims for: one per compute unit,
// each wavefront walking four or more 32-token tiles with the next one's
// loads in flight (fewer, longer splits also leave merge_kernel fewer
// partials).
constexpr int kSparseTargetWG = 256;

// Units of one query that share a workgroup: for batches with enough rows
// to fill the chip without splits, the four KV heads of a group of four when
// each KV head's query heads fit one chunk (eight wavefronts, two per KV
// head; 7 % faster on the 16K-query chunk than a workgroup per KV head),
// else one.  (Decode-sized batches split the token list instead; there the
// grouping was slower: more splits for the same number of workgroups.)
int sparse_group(const Dims& d) {
  const int G = d.Hq / d.Hkv;
  if (G > 16 || d.Hkv % 4 != 0) return 1;
  return (long long)d.B * sparse_units(d) / 4 >= kSparseTargetWG ? 4 : 1;
}

int sparse_splits(const Dims& d, int* split_tokens, int* tail_last) {
  // Decode-sized batches have few (query, KV head) units: split their token
  // lists so that about kSparseTargetWG workgroups share the gather.  Splits
  // of one tile per wavefront leave the query's own block (<= 4 tokens) to a
  // split of its own; longer splits take it into the last one.
  constexpr int kSelTok = kTopK * kBlock;
  if (sparse_group(d) > 1) {  // whole token lists
    *split_tokens = kMaxTok;
    *tail_last = 0;
    return 1;
  }
  const long long units = (long long)d.B * sparse_units(d);
  int st = kMaxTok;
  if (units < kSparseTargetWG) {
    const long long want = (kSparseTargetWG + units - 1) / units;
    st = (int)(kSelTok / want) / (4 * kTile) * (4 * kTile);
    if (st < 4 * kTile) st = 4 * kTile;
  }
  *split_tokens = st;
  if (st >= kSelTok) {
    *tail_last = 0;
    return 1;
  }
  if (st <= 4 * kTile) {
    *tail_last = 0;
    return (kMaxTok + st - 1) / st;
  }
  *tail_last = 1;
  return (kSelTok + st - 1) / st;
}

int dense_splits(const Dims& d, int* split_tokens) {
  // About 8K wavefronts in total, at least 256 tokens each.
  const long long cchunks = ((long long)d.Nq * (d.Hq / d.Hkv) + 15) / 16;
  const long long units = (long long)d.B * d.Hkv * cchunks;
  long long n_split = (8192 + units - 1) / units;
  const long long max_split = (d.Lmax + 255) / 256;
  if (n_split > max_split) n_split = max_split;
  if (n_split < 1) n_split = 1;
  long long st = (d.Lmax + n_split - 1) / n_split;
  st = (st + kTile - 1) / kTile * kTile;
  *split_tokens = (int)st;
  return (int)((d.Lmax + st - 1) / st);
}

}  // namespace

AttendLayout attend_layout(const Dims& d) {
  AttendLayout l{};
  int st, tl;
  const int ns = sparse_splits(d, &st, &tl);
  if (ns > 1) {
    const size_t rh = (size_t)d.B * d.Nq * d.Hq;
    l.partial_floats = rh * ns * kHeadDim;
    l.lse_floats = rh * ns;
  }
  return l;
}

namespace {
void set_paging(AttnArgs& a, const Paged* pg) {
  a.pt = pg ? pg->page_table : nullptr;
  a.page_shift = pg ? pg->page_shift : 0;
  a.max_pages = pg ? pg->max_pages : 0;
  a.n_pages = pg ? pg->n_pages : 0;
}
}  // namespace

hipError_t launch_sparse_attend(const Dims& d, const uint16_t* q, const uint16_t* k,
                                const uint16_t* v, const int32_t* lens, const int32_t* sel,
                                const int32_t* n_sel, uint16_t* out, float* lse, float* part_o,
                                float* part_lse, hipStream_t s, const Paged* pg) {
  if (d.B == 0 || d.Nq == 0) return hipSuccess;
  AttnArgs a{};
  set_paging(a, pg);
  a.q = q;
  a.k = k;
  a.v = v;
  a.lens = lens;
  a.sel = sel;
  a.n_sel = n_sel;
  a.out = out;
  a.lse = lse;
  a.B = d.B;
  a.Lmax = d.Lmax;
  a.Nq = d.Nq;
  a.Hq = d.Hq;
  a.Hkv = d.Hkv;
  a.G = d.Hq / d.Hkv;
  a.scale_log2 = d.scale * kLog2e;
  a.n_split = sparse_splits(d, &a.split_tokens, &a.tail_last);
  if (a.n_split > 1) {
    a.part_o = part_o;
    a.part_lse = part_lse;
  }
  const int grp = sparse_group(d);
  const dim3 grid((unsigned)(sparse_units(d) / grp), (unsigned)a.n_split, (unsigned)d.B);
  if (grp > 1)  // four KV heads per workgroup, two wavefronts each, one split
    QSA_LAUNCH_AS("sparse_attend_kernel<true>", (sparse_attend_kernel<true, 8, 4>), grid,
                  dim3(512), 0, s, a);
  else if (a.split_tokens <= 4 * kTile)
    QSA_LAUNCH_AS("sparse_attend_kernel<false>", (sparse_attend_kernel<false, 4, 1>), grid,
                  dim3(256), 0, s, a);
  else if (a.n_split > 1)  // decode-sized: eight wavefronts walk a split's tiles
    QSA_LAUNCH_AS("sparse_attend_kernel<true>", (sparse_attend_kernel<true, 8, 1>), grid,
                  dim3(512), 0, s, a);
  else
    QSA_LAUNCH_AS("sparse_attend_kernel<true>", (sparse_attend_kernel<true, 4, 1>), grid,
                  dim3(256), 0, s, a);
  if (a.n_split > 1) return launch_merge(part_o, part_lse, out, lse, d, a.n_split, s);
  return hipGetLastError();
}

size_t teacher_workspace_bytes(const Dims& d) {
  Carve c{nullptr, 0};
  c.take<char>(dense_workspace_bytes(d));
  c.take<uint16_t>((size_t)d.B * d.Nq * d.Hq * kHeadDim);  // dense output (unused)
  c.take<float>((size_t)d.B * d.Nq * d.Hq);                // dense lse
  return c.off;
}

hipError_t launch_block_teacher(const Dims& d, const uint16_t* q, const uint16_t* k,
                                const uint16_t* v, const int32_t* lens, float* teacher, void* ws,
                                hipStream_t s) {
  if (d.B == 0 || d.Nq == 0) return hipSuccess;
  Carve c{static_cast<char*>(ws), 0};
  void* dws = c.take<char>(dense_workspace_bytes(d));
  uint16_t* dout = c.take<uint16_t>((size_t)d.B * d.Nq * d.Hq * kHeadDim);
  float* dlse = c.take<float>((size_t)d.B * d.Nq * d.Hq);
  hipError_t e = launch_dense_decode(d, q, k, v, lens, dout, dlse, dws, s);
  if (e != hipSuccess) return e;
  const size_t nt = (size_t)d.B * d.Nq * (d.Lmax / 4);
  QSA_LAUNCH(fill_f32_kernel, dim3(1024), dim3(256), 0, s, teacher, nt, 0.f);
  AttnArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.lens = lens;
  a.B = d.B;
  a.Lmax = d.Lmax;
  a.Nq = d.Nq;
  a.Hq = d.Hq;
  a.Hkv = d.Hkv;
  a.G = d.Hq / d.Hkv;
  a.scale_log2 = d.scale * kLog2e;
  a.n_split = dense_splits(d, &a.split_tokens);
  const int units = d.Hkv * ((d.Nq * a.G + 15) / 16);
  const int waves = units < kDenseWaves ? units : kDenseWaves;
  QSA_LAUNCH(block_teacher_kernel,
             dim3((unsigned)a.n_split, (unsigned)((units + kDenseWaves - 1) / kDenseWaves),
                  (unsigned)d.B),
             dim3(64 * (unsigned)waves), 0, s, a, (const float*)dlse, teacher);
  return hipGetLastError();
}

hipError_t launch_teacher_recall(const Dims& d, const float* teacher, const int32_t* lens,
                                 const int32_t* sel, const int32_t* n_sel, float* recall,
                                 hipStream_t s) {
  if (d.B == 0 || d.Nq == 0) return hipSuccess;
  QSA_LAUNCH(teacher_recall_kernel, dim3((unsigned)d.Nq, (unsigned)d.B), dim3(256), 0, s, teacher,
             lens, sel, n_sel, recall, d.Lmax, d.Nq);
  return hipGetLastError();
}

size_t dense_workspace_bytes(const Dims& d) {
  int st;
  const int ns = dense_splits(d, &st);
  Carve c{nullptr, 0};
  const size_t rh = (size_t)d.B * d.Nq * d.Hq;
  c.take<float>(rh * ns * kHeadDim);
  c.take<float>(rh * ns);
  return c.off;
}

hipError_t launch_dense_decode(const Dims& d, const uint16_t* q, const uint16_t* k,
                               const uint16_t* v, const int32_t* lens, uint16_t* out,
                               float* lse, void* ws, hipStream_t s, const Paged* pg) {
  if (d.B == 0 || d.Nq == 0) return hipSuccess;
  AttnArgs a{};
  set_paging(a, pg);
  a.q = q;
  a.k = k;
  a.v = v;
  a.lens = lens;
  a.out = out;
  a.lse = lse;
  a.B = d.B;
  a.Lmax = d.Lmax;
  a.Nq = d.Nq;
  a.Hq = d.Hq;
  a.Hkv = d.Hkv;
  a.G = d.Hq / d.Hkv;
  a.scale_log2 = d.scale * kLog2e;
  a.n_split = dense_splits(d, &a.split_tokens);
  Carve c{static_cast<char*>(ws), 0};
  const size_t rh = (size_t)d.B * d.Nq * d.Hq;
  a.part_o = c.take<float>(rh * a.n_split * kHeadDim);
  a.part_lse = c.take<float>(rh * a.n_split);
  const int units = d.Hkv * ((d.Nq * a.G + 15) / 16);
  const int waves = units < kDenseWaves ? units : kDenseWaves;
  const dim3 grid((unsigned)a.n_split, (unsigned)((units + kDenseWaves - 1) / kDenseWaves),
                  (unsigned)d.B);
  if (a.pt)
    QSA_LAUNCH(dense_decode_kernel<true>, grid, dim3(64 * (unsigned)waves), 0, s, a);
  else
    QSA_LAUNCH(dense_decode_kernel<false>, grid, dim3(64 * (unsigned)waves), 0, s, a);
  return launch_merge(a.part_o, a.part_lse, out, lse, d, a.n_split, s);
}

hipError_t launch_dense_prefill(const Dims& d, const uint16_t* q, const uint16_t* k,
                                const uint16_t* v, const int32_t* lens, uint16_t* out, float* lse,
                                hipStream_t s, const Paged* pg) {
  if (d.B == 0 || d.Nq == 0) return hipSuccess;
  AttnArgs a{};
  set_paging(a, pg);
  a.q = q;
  a.k = k;
  a.v = v;
  a.lens = lens;
  a.out = out;
  a.lse = lse;
  a.B = d.B;
  a.Lmax = d.Lmax;
  a.Nq = d.Nq;
  a.Hq = d.Hq;
  a.Hkv = d.Hkv;
  a.G = d.Hq / d.Hkv;
  a.scale_log2 = d.scale * kLog2e;
  const int qw = 16 * 2 * kPrefWaves / a.G;
  const dim3 grid((unsigned)((d.Nq + qw - 1) / qw), (unsigned)d.Hkv, (unsigned)d.B);
  if (a.pt)
    QSA_LAUNCH(dense_prefill_kernel<true>, grid, dim3(64 * kPrefWaves), 0, s, a);
  else
    QSA_LAUNCH(dense_prefill_kernel<false>, grid, dim3(64 * kPrefWaves), 0, s, a);
  return hipGetLastError();
}

}  // namespace qsa
