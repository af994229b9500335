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
// of that group (the sparse kernel: the heads of one query; the dense kernel:
// 32 (query, head) rows of one sequence, all queries sharing the K/V stream).
// It walks the tokens in tiles of 32:
//   * S^T = K Q^T with MFMA 16x16x32: K rows are gathered straight from HBM
//     into the A operand (each lane loads 16 contiguous bytes of one row),
//     the stationary Q fragment is the B operand;
//   * online softmax in fp32 registers (exp2 domain), one running max and sum
//     per query head;
//   * O^T += V^T P with MFMA: P already sits in the B-operand layout, V goes
//     through a per-wavefront LDS tile and is read back transposed.
// Long token ranges are split across workgroups; partial (o, lse) pairs are
// merged by merge_kernel.
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

__device__ __forceinline__ bf16x8 pack8(const float* p) {
  uint4 u;
  u.x = f32_to_bf16(p[0]) | (f32_to_bf16(p[1]) << 16);
  u.y = f32_to_bf16(p[2]) | (f32_to_bf16(p[3]) << 16);
  u.z = f32_to_bf16(p[4]) | (f32_to_bf16(p[5]) << 16);
  u.w = f32_to_bf16(p[6]) | (f32_to_bf16(p[7]) << 16);
  return as_bf16x8(u);
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
};

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
  tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
  tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
  const float m_new = fmaxf(r.m, tmax);
  // A column with every logit masked so far keeps m = -inf; guard the exp2.
  const float m_use = m_new == kNegInf ? 0.f : m_new;
  const float alpha = exp2f(r.m - m_use);
  float p[8];
  float ps = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    p[e] = exp2f(z[e] - m_use);
    ps += p[e];
  }
  r.l = r.l * alpha + ps;
  r.m = m_new;
  const bf16x8 pf = pack8(p);
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
  const int len = clampi(a.lens[b], 0, a.Lmax);
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
    ns = clampi(a.n_sel[row], 0, bt < kTopK ? bt : kTopK);
    ntok = 4 * ns + (t - 4 * bt) + 1;
  }
  const size_t kv_seq = (size_t)b * a.Lmax * a.Hkv;
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
      return tok <= t ? (long long)(kv_seq + (size_t)tok * a.Hkv) * kHeadDim : -1;
    });
  // ids outside [0, bt) are a caller bug: clamped so no access leaves the row
#pragma unroll
  for (int i = 0; i < kSelPer; ++i) {
    const int e = tid + kThreads * i;
    if (e < nsb && kb0 + e < ns) s_sel[e] = clampi(my_sel[i], 0, bt - 1);
  }
  __syncthreads();
  // the selected tokens of this split (with tail_last the query's own block
  // is handled apart, above; otherwise it follows the selected ones)
  const int k_end = a.tail_last ? min(4 * ns, k_begin + a.split_tokens)
                                : min(ntok, k_begin + a.split_tokens);
  auto row_of = [&](int kk) -> long long {
    if (kk >= k_end) return -1;
    const int tok = kk < 4 * ns ? 4 * s_sel[(kk >> 2) - kb0] + (kk & 3) : 4 * bt + (kk - 4 * ns);
    return (long long)(kv_seq + (size_t)tok * a.Hkv) * kHeadDim;
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
  float* O = reinterpret_cast<float*>(&s_v[0][0]);  // [kWaves][16][128]
  {
    const int gq = lane >> 4;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
      *reinterpret_cast<float4*>(O + (wave * 16 + col) * kHeadDim + dt * 16 + gq * 4) =
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
      o += s_f[w][c] * O[(w * 16 + c) * kHeadDim + d];
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
  const int len = clampi(a.lens[b], 0, a.Lmax);
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
  const size_t kv_seq = (size_t)b * a.Lmax * a.Hkv;
  const uint16_t* kbase = a.k + g * kHeadDim;
  const uint16_t* vbase = a.v + g * kHeadDim;
  auto row_of = [&](int kk) -> long long {
    return kk < k_end ? (long long)(kv_seq + (size_t)kk * a.Hkv) * kHeadDim : -1;
  };
  Run r;
  run_init(r);
  KVTile cur, nxt;
  if (k_begin < k_end) load_tile(cur, kbase, vbase, k_begin, row_of);
  for (int k0 = k_begin; k0 < k_end; k0 += kTile) {
    stash_v(s_v, cur);
    if (k0 + kTile < k_end) load_tile(nxt, kbase, vbase, k0 + kTile, row_of);
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
  }
  float* po = a.part_o + (((row * a.Hq) + h) * a.n_split + split) * kHeadDim;
  float* pl = a.part_lse + ((row * a.Hq) + h) * a.n_split + split;
  finish(r, col_valid, nullptr, nullptr, po, pl, true);
}

__global__ void fill_words_kernel(uint32_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

// ------------------------------------------------------------------ merge
// Grid (Hq, Nq, B), 128 threads (one per output dim).  Combines the n_split
// partial (o, lse) pairs of one (query, head): o = sum_s e^(lse_s - M) o_s /
// sum_s e^(lse_s - M).  Loads go out 32 splits at a time so that their
// latencies overlap.
__global__ __launch_bounds__(128) void merge_kernel(const float* __restrict__ part_o,
                                                    const float* __restrict__ part_lse,
                                                    uint16_t* __restrict__ out,
                                                    float* __restrict__ lse, int Nq, int Hq,
                                                    int n_split) {
  constexpr int kChunk = 32;
  const int h = blockIdx.x, q = blockIdx.y, b = blockIdx.z, d = threadIdx.x;
  const size_t rh = ((size_t)b * Nq + q) * Hq + h;
  const float* pl = part_lse + rh * n_split;
  const float* po = part_o + rh * n_split * kHeadDim + d;
  float M = kNegInf;
  float acc = 0.f, sw = 0.f;
  if (n_split <= kChunk) {
    // every partial in one round of loads
    float w[kChunk], v[kChunk];
#pragma unroll
    for (int s = 0; s < kChunk; ++s) {
      const bool ok = s < n_split;
      w[s] = ok ? pl[s] : kNegInf;
      v[s] = ok ? po[(size_t)s * kHeadDim] : 0.f;
    }
#pragma unroll
    for (int s = 0; s < kChunk; ++s) M = fmaxf(M, w[s]);
    if (M != kNegInf) {
#pragma unroll
      for (int s = 0; s < kChunk; ++s) {
        const float e = w[s] == kNegInf ? 0.f : __expf(w[s] - M);
        sw += e;
        acc += e * v[s];
      }
    }
  } else {
    for (int s0 = 0; s0 < n_split; s0 += kChunk) {
#pragma unroll
      for (int s = 0; s < kChunk; ++s)
        if (s0 + s < n_split) M = fmaxf(M, pl[s0 + s]);
    }
  }
  if (n_split > kChunk && M != kNegInf) {
    for (int s0 = 0; s0 < n_split; s0 += kChunk) {
      float w[kChunk], v[kChunk];
#pragma unroll
      for (int s = 0; s < kChunk; ++s) {
        const bool ok = s0 + s < n_split;
        w[s] = ok ? pl[s0 + s] : kNegInf;
        v[s] = ok ? po[(size_t)(s0 + s) * kHeadDim] : 0.f;
      }
#pragma unroll
      for (int s = 0; s < kChunk; ++s) {
        const float e = w[s] == kNegInf ? 0.f : __expf(w[s] - M);
        sw += e;
        acc += e * v[s];
      }
    }
  }
  const float o = sw > 0.f ? acc / sw : 0.f;
  out[rh * kHeadDim + d] = (uint16_t)f32_to_bf16(o);
  if (lse && d == 0) lse[rh] = sw > 0.f ? M + __logf(sw) : kNegInf;
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

hipError_t launch_sparse_attend(const Dims& d, const uint16_t* q, const uint16_t* k,
                                const uint16_t* v, const int32_t* lens, const int32_t* sel,
                                const int32_t* n_sel, uint16_t* out, float* lse, float* part_o,
                                float* part_lse, hipStream_t s) {
  if (d.B == 0 || d.Nq == 0) return hipSuccess;
  AttnArgs a{};
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
  if (a.n_split > 1)
    QSA_LAUNCH(merge_kernel, dim3((unsigned)d.Hq, (unsigned)d.Nq, (unsigned)d.B), dim3(128), 0, s,
               part_o, part_lse, out, lse, d.Nq, d.Hq, a.n_split);
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
                               float* lse, void* ws, hipStream_t s) {
  if (d.B == 0 || d.Nq == 0) return hipSuccess;
  AttnArgs a{};
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
  QSA_LAUNCH(dense_decode_kernel,
             dim3((unsigned)a.n_split, (unsigned)((units + kDenseWaves - 1) / kDenseWaves),
                  (unsigned)d.B),
             dim3(64 * (unsigned)waves), 0, s, a);
  QSA_LAUNCH(merge_kernel, dim3((unsigned)d.Hq, (unsigned)d.Nq, (unsigned)d.B), dim3(128), 0, s,
             a.part_o, a.part_lse, out, lse, d.Nq, d.Hq, a.n_split);
  return hipGetLastError();
}

}  // namespace qsa
