// Gradients of the QSA layer: the indexer and the model are trained together
// (page "Qwen's million-token window has a 2,048-token keyhole", section "The
// indexer is trained, not bolted on"), so both the sparse attention and the
// indexer's scoring need a backward pass.
//
//  * sparse attention over each query's token list (its kept micro-blocks and
//    its own block): with p the softmax of z = scale q_h . k_s, dp_s =
//    dO_h . v_s, D_h = dO_h . O_h and ds_s = p_s (dp_s - D_h),
//      dq_h = scale sum_s ds_s k_s,  dk_s += scale ds_s q_h,  dv_s += p_s dO_h;
//    tokens are shared by the heads of a group and by queries, so dk and dv
//    are float32 sums added atomically;
//  * indexer scores s_j = sum_h max(0, q_h . kc_j): given g = dL/ds,
//      dq_h = sum_j g_j [q_h . kc_j > 0] kc_j,  dkc_j = sum_h g_j [q_h . kc_j > 0] q_h;
//  * compression (a sum of four keys): every key of a block receives the
//    block's gradient.
// Float32 arithmetic throughout (plain vector math; the forward pass's MFMA
// tiles are not reused here).
#include "common.h"
#include "internal.h"

namespace qsa {
namespace {

constexpr int kBwdThreads = 256;
constexpr int kBwdTile = 64;    // tokens per step
constexpr int kBwdHeads = 16;   // query heads per workgroup (one chunk of a group)
constexpr float kLog2eB = 1.4426950408889634f;

__device__ __forceinline__ float bf(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }

// Grid (Nq, Hkv * hchunks, B), 256 threads: one query row, one KV head g and
// up to 16 of its query heads.
__global__ __launch_bounds__(kBwdThreads) void sparse_attend_bwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ lens, const int32_t* __restrict__ sel,
    const int32_t* __restrict__ n_sel, const uint16_t* __restrict__ out,
    const float* __restrict__ lse, const uint16_t* __restrict__ d_out, float* __restrict__ dq,
    float* __restrict__ dk, float* __restrict__ dv, int Lmax, int Nq, int Hq, int Hkv,
    float scale) {
  __shared__ float s_q[kBwdHeads][kHeadDim];
  __shared__ float s_do[kBwdHeads][kHeadDim];
  __shared__ float s_D[kBwdHeads], s_lse2[kBwdHeads];
  __shared__ int32_t s_sel[kTopK];
  __shared__ __align__(16) uint16_t s_k[kBwdTile][kHeadDim];
  __shared__ __align__(16) uint16_t s_v[kBwdTile][kHeadDim];
  __shared__ float s_p[kBwdTile][kBwdHeads], s_ds[kBwdTile][kBwdHeads];
  __shared__ int32_t s_tok[kBwdTile];
  const int qi = blockIdx.x, b = blockIdx.z, tid = threadIdx.x;
  const int G = Hq / Hkv, hchunks = (G + kBwdHeads - 1) / kBwdHeads;
  const int g = blockIdx.y / hchunks, hc = blockIdx.y % hchunks;
  const int h0 = g * G + hc * kBwdHeads, nh = min(kBwdHeads, G - hc * kBwdHeads);
  const size_t row = (size_t)b * Nq + qi;
  const int len = guard_len(lens[b], Nq, Lmax);
  const int t = len - Nq + qi;
  int ns = 0, ntok = 0, bt = 0;
  if (t >= 0) {
    bt = t >> 2;
    ns = guard(n_sel[row], 0, min(bt, kTopK));
    ntok = 4 * ns + (t - 4 * bt) + 1;
  }
  // the heads' q, dO, D = dO . O and lse (exp2 domain)
  for (int i = tid; i < nh * kHeadDim; i += kBwdThreads) {
    const int h = i >> 7, d = i & 127;
    const size_t off = (row * Hq + h0 + h) * kHeadDim + d;
    s_q[h][d] = bf(q[off]);
    s_do[h][d] = bf(d_out[off]);
  }
  for (int i = tid; i < ns; i += kBwdThreads) s_sel[i] = guard(sel[row * kTopK + i], 0, bt - 1);
  if (tid < kBwdHeads * 16) {
    // 16 lanes per head: partial dot products of dO and O
    const int h = tid >> 4, part = tid & 15;
    float acc = 0.f;
    if (h < nh) {
      const size_t off = (row * Hq + h0 + h) * kHeadDim;
      for (int d = part; d < kHeadDim; d += 16) acc += bf(d_out[off + d]) * bf(out[off + d]);
    }
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
    if (part == 0 && h < nh) {
      s_D[h] = acc;
      s_lse2[h] = lse[row * Hq + h0 + h] * kLog2eB;
    }
  }
  __syncthreads();
  const float sl2 = scale * kLog2eB;
  // dq accumulators: thread (d = tid & 127, half = tid >> 7) holds heads half, half + 2, ...
  const int dd = tid & 127, half = tid >> 7;
  float acc_dq[kBwdHeads / 2];
#pragma unroll
  for (int i = 0; i < kBwdHeads / 2; ++i) acc_dq[i] = 0.f;
  const size_t kv_seq = (size_t)b * Lmax * Hkv;
  for (int k0 = 0; k0 < ntok; k0 += kBwdTile) {
    // the tile's token ids and K/V rows of head g
    if (tid < kBwdTile) {
      const int kk = k0 + tid;
      int tok = -1;
      if (kk < ntok) tok = kk < 4 * ns ? 4 * s_sel[kk >> 2] + (kk & 3) : 4 * bt + (kk - 4 * ns);
      s_tok[tid] = tok;
    }
    __syncthreads();
    for (int i = tid; i < kBwdTile * 16; i += kBwdThreads) {
      const int r = i >> 4, c = i & 15;  // row, 16-byte chunk
      const int tok = s_tok[r];
      uint4 kv = zero_u4(), vv = zero_u4();
      if (tok >= 0) {
        const size_t off = (kv_seq + (size_t)tok * Hkv + g) * kHeadDim;
        kv = reinterpret_cast<const uint4*>(k + off)[c];
        vv = reinterpret_cast<const uint4*>(v + off)[c];
      }
      reinterpret_cast<uint4*>(&s_k[r][0])[c] = kv;
      reinterpret_cast<uint4*>(&s_v[r][0])[c] = vv;
    }
    __syncthreads();
    // p and ds of (token, head) pairs: thread -> token tid & 63, heads (tid >> 6) + 4 i
    {
      const int r = tid & 63, hb = tid >> 6;
      const bool live = s_tok[r] >= 0;
      for (int h = hb; h < kBwdHeads; h += 4) {
        float z = 0.f, dp = 0.f;
        if (h < nh && live) {
#pragma unroll 8
          for (int d = 0; d < kHeadDim; ++d) {
            z = fmaf(s_q[h][d], bf(s_k[r][d]), z);
            dp = fmaf(s_do[h][d], bf(s_v[r][d]), dp);
          }
        }
        const float p = (h < nh && live) ? exp2f(z * sl2 - s_lse2[h]) : 0.f;
        s_p[r][h] = p;
        s_ds[r][h] = (h < nh && live) ? p * (dp - s_D[h]) : 0.f;
      }
    }
    __syncthreads();
    // dq: thread (dd, half) over the tile's tokens
#pragma unroll
    for (int i = 0; i < kBwdHeads / 2; ++i) {
      const int h = half + 2 * i;
      if (h >= nh) continue;
      float a = 0.f;
      for (int r = 0; r < kBwdTile; ++r) a = fmaf(s_ds[r][h], bf(s_k[r][dd]), a);
      acc_dq[i] += a;
    }
    // dk, dv of the tile's tokens: thread (dd, half) over 32 tokens each
    for (int r = half * 32; r < half * 32 + 32; ++r) {
      const int tok = s_tok[r];
      if (tok < 0) continue;
      float ak = 0.f, av = 0.f;
      for (int h = 0; h < nh; ++h) {
        ak = fmaf(s_ds[r][h], s_q[h][dd], ak);
        av = fmaf(s_p[r][h], s_do[h][dd], av);
      }
      const size_t off = (kv_seq + (size_t)tok * Hkv + g) * kHeadDim + dd;
      atomicAdd(&dk[off], scale * ak);
      atomicAdd(&dv[off], av);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < kBwdHeads / 2; ++i) {
    const int h = half + 2 * i;
    if (h < nh) dq[(row * Hq + h0 + h) * kHeadDim + dd] = scale * acc_dq[i];
  }
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Grid (n_slices, ceil(Nq / kQ), B), 256 threads (four wavefronts): the
// blocks of one slice against up to kQ queries of one sequence.  Each
// wavefront takes 64-block tiles of the slice in turn:
//  1. block side, on the matrix cores: the products q_h . kc_j of the kQ x 4
//     (query, head) rows and the tile's blocks, 16 x 16 per pair of
//     16x16x32 bf16 MFMA steps (bf16 inputs, float32 sums).  A lane then
//     holds the four heads of one query for one block and keeps
//     w = g (product > 0 and the block a candidate of the query) or 0;
//     the w rows and the tile's keys go to the wavefront's LDS;
//  2. dimension side, float32 FMA: a lane owns kDL = 16 / kQ consecutive
//     dimensions of every (64 / kDL)-th block; per block j it sums
//     w_j,r q_r,d over the rows r into dkc_j,d, added to dk_cmp as one
//     row (a plain read-add-write when this workgroup is the row's only
//     writer, atomic adds otherwise), and adds w_j,r kc_j,d to its dq_r,d
//     registers.
// The lanes' dq are summed in LDS and added to dq_idx at the end.
template <int kQ>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(kQ <= 4 ? 2 : 1)))
void index_scores_bwd_kernel(
    const uint16_t* __restrict__ q_idx, const uint16_t* __restrict__ k_cmp,
    const int32_t* __restrict__ lens, const float* __restrict__ g_scores,
    float* __restrict__ dq_idx, float* __restrict__ dk_cmp, int Lmax, int Nq, int slice_blocks) {
  constexpr int kR = kQ * kIdxHeads;   // (query, head) rows
  constexpr int kMT = kR / 16;         // 16-row MFMA tiles
  constexpr int kDL = 16 / kQ;         // dimensions per lane on the dimension side
  constexpr int kG = kIdxDim / kDL;    // lanes per block on the dimension side
  constexpr int kKRow = 9;             // LDS key row: 64 bf16 + 16 bytes of stagger, in uint4
  constexpr int kWRow = kR / 4;        // LDS w row, in float4
  constexpr int kWaves = kBwdThreads / 64;
  __shared__ uint4 s_k[kWaves][64 * kKRow];
  __shared__ f32x4 s_w[kWaves][64 * kWRow];
  __shared__ float s_dq[kR * kIdxDim];
  const int slice = blockIdx.x, q0 = blockIdx.y * kQ, b = blockIdx.z, tid = threadIdx.x;
  const int nq = min(kQ, Nq - q0);
  const int len = guard_len(lens[b], Nq, Lmax);
  const int nbp = Lmax >> 2;
  const int t_last = len - Nq + q0 + nq - 1;
  const int j0 = slice * slice_blocks, j1 = min(j0 + slice_blocks, t_last >> 2);
  if (j1 <= j0) return;  // (uniform over the workgroup)
  for (int i = tid; i < kR * kIdxDim; i += kBwdThreads) s_dq[i] = 0.f;

  const int lane = lane_id(), wave = tid >> 6;
  const int r = lane & 15, kc = lane >> 4;
  // block side: A fragments (row 16 mt + r = query 4 mt + r / 4, head r % 4,
  // dimensions 8 kc.. and 32 + 8 kc..) and this lane's query 4 mt + kc
  bf16x8 qa[kMT][2];
  int lim[kMT];
  const size_t qrow0 = (size_t)b * Nq + q0;
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt) {
    const int qq = 4 * mt + (r >> 2);
    uint4 u0 = zero_u4(), u1 = zero_u4();
    if (qq < nq) {
      const uint4* p =
          reinterpret_cast<const uint4*>(q_idx + ((qrow0 + qq) * kIdxHeads + (r & 3)) * kIdxDim);
      u0 = p[kc];
      u1 = p[4 + kc];
    }
    qa[mt][0] = as_bf16x8(u0);
    qa[mt][1] = as_bf16x8(u1);
    const int qw = 4 * mt + kc;
    lim[mt] = qw < nq ? min((len - Nq + q0 + qw) >> 2, j1) : 0;
  }
  // dimension side: this lane's dimensions d0.. of every row
  const int d0 = (lane % kG) * kDL, js = lane / kG;
  float qv[kR][kDL], dq[kR][kDL];
#pragma unroll
  for (int rr = 0; rr < kR; ++rr)
#pragma unroll
    for (int e = 0; e < kDL; ++e) {
      qv[rr][e] = rr / kIdxHeads < nq ? bf(q_idx[(qrow0 * kIdxHeads + rr) * kIdxDim + d0 + e]) : 0.f;
      dq[rr][e] = 0.f;
    }
  __syncthreads();

  const uint4* kb = reinterpret_cast<const uint4*>(k_cmp + (size_t)b * nbp * kIdxDim);
  const float* gb = g_scores + qrow0 * nbp;
  float* dkb = dk_cmp + (size_t)b * nbp * kIdxDim;
  const bool sole = gridDim.y == 1;
  uint4* sk = s_k[wave];
  f32x4* sw = s_w[wave];
  const int ntiles = (j1 - j0 + 63) >> 6;
  // the tile's keys and g values, loaded one tile ahead
  uint4 bv[4][2];
  float gv[kMT][4];
  auto load_tile = [&](int jt) {
    // Unconditional key loads: a block past the slice re-reads its last one
    // and gets w = 0.
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int j = min(jt + nt * 16 + r, j1 - 1);
      bv[nt][0] = kb[(size_t)j * 8 + kc];
      bv[nt][1] = kb[(size_t)j * 8 + 4 + kc];
    }
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int j = jt + nt * 16 + r;
        gv[mt][nt] = j < lim[mt] ? gb[(size_t)(4 * mt + kc) * nbp + j] : 0.f;
      }
  };
  if (wave < ntiles) load_tile(j0 + wave * 64);
#pragma unroll 1
  for (int tile = wave; tile < ntiles; tile += kWaves) {
    const int jt = j0 + tile * 64;
    wave_sync_lds();  // the previous tile's LDS reads are done
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      sk[(nt * 16 + r) * kKRow + kc] = bv[nt][0];
      sk[(nt * 16 + r) * kKRow + 4 + kc] = bv[nt][1];
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = mfma16(qa[mt][0], as_bf16x8(bv[nt][0]), acc);
        acc = mfma16(qa[mt][1], as_bf16x8(bv[nt][1]), acc);
        const float g = gv[mt][nt];
        f32x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = acc[i] > 0.f ? g : 0.f;
        sw[(nt * 16 + r) * kWRow + 4 * mt + kc] = w;
      }
    }
    wave_sync_lds();
    if (tile + kWaves < ntiles) load_tile(jt + kWaves * 64);
    const uint16_t* skh = reinterpret_cast<const uint16_t*>(sk);
    // Dimension side.  With a sole writer, the dk_cmp values of a row are
    // read two rows ahead of its add.
    auto fetch = [&](int jl, float (&v)[kDL]) {
      const int j = jt + jl;
#pragma unroll
      for (int e = 0; e < kDL; ++e) v[e] = 0.f;
      if (sole && j < j1) {
        const float* src = dkb + (size_t)j * kIdxDim + d0;
#pragma unroll
        for (int e = 0; e < kDL; ++e) v[e] = src[e];
      }
    };
    auto row = [&](int jl, const float (&cur)[kDL]) {
      const int j = jt + jl;
      float kv[kDL], dk[kDL];
#pragma unroll
      for (int e = 0; e < kDL; ++e) {
        kv[e] = bf(skh[jl * kKRow * 8 + d0 + e]);
        dk[e] = 0.f;
      }
#pragma unroll
      for (int c = 0; c < kWRow; ++c) {
        const f32x4 w4 = sw[jl * kWRow + c];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int e = 0; e < kDL; ++e) {
            dq[4 * c + i][e] = fmaf(w4[i], kv[e], dq[4 * c + i][e]);
            dk[e] = fmaf(w4[i], qv[4 * c + i][e], dk[e]);
          }
      }
      if (j < j1) {
        float* dst = dkb + (size_t)j * kIdxDim + d0;
        if (sole) {
#pragma unroll
          for (int e = 0; e < kDL; ++e) dst[e] = cur[e] + dk[e];
        } else {
#pragma unroll
          for (int e = 0; e < kDL; ++e)
            if (dk[e] != 0.f) atomicAdd(&dst[e], dk[e]);
        }
      }
    };
    constexpr int kRows = 64 / kDL;  // rows per lane per tile (even)
    float pre0[kDL], pre1[kDL], cur[kDL];
    fetch(js, pre0);
    fetch(kDL + js, pre1);
#pragma unroll 1
    for (int jj = 0; jj < kRows; jj += 2) {
#pragma unroll
      for (int e = 0; e < kDL; ++e) cur[e] = pre0[e];
      if (jj + 2 < kRows) fetch((jj + 2) * kDL + js, pre0);
      row(jj * kDL + js, cur);
#pragma unroll
      for (int e = 0; e < kDL; ++e) cur[e] = pre1[e];
      if (jj + 3 < kRows) fetch((jj + 3) * kDL + js, pre1);
      row((jj + 1) * kDL + js, cur);
    }
  }
#pragma unroll
  for (int rr = 0; rr < kR; ++rr)
#pragma unroll
    for (int e = 0; e < kDL; ++e)
      if (dq[rr][e] != 0.f) atomicAdd(&s_dq[rr * kIdxDim + d0 + e], dq[rr][e]);
  __syncthreads();
  float* dqb = dq_idx + qrow0 * kIdxHeads * kIdxDim;
  for (int i = tid; i < nq * kIdxHeads * kIdxDim; i += kBwdThreads) {
    const float x = s_dq[i];
    if (x != 0.f) atomicAdd(&dqb[i], x);
  }
}

// dk_idx[b][4j + r][:] += dk_cmp[b][j][:] for the completed blocks j < lens[b]/4.
__global__ __launch_bounds__(256) void compress_bwd_kernel(const float* __restrict__ dk_cmp,
                                                           const int32_t* __restrict__ lens,
                                                           float* __restrict__ dk_idx, int Lmax) {
  const int b = blockIdx.y;
  const int nb = guard(lens[b], 0, Lmax) >> 2;
  const size_t n = (size_t)nb * 4 * kIdxDim;
  const float* src = dk_cmp + (size_t)b * (Lmax >> 2) * kIdxDim;
  float* dst = dk_idx + (size_t)b * Lmax * kIdxDim;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x) {
    const size_t tok = i / kIdxDim, d = i % kIdxDim;
    dst[i] += src[(tok >> 2) * kIdxDim + d];
  }
}

}  // namespace

hipError_t launch_sparse_attend_bwd(const Dims& d, const uint16_t* q, const uint16_t* k,
                                    const uint16_t* v, const int32_t* lens, const int32_t* sel,
                                    const int32_t* n_sel, const uint16_t* out, const float* lse,
                                    const uint16_t* d_out, float* dq, float* dk, float* dv,
                                    hipStream_t s) {
  if (d.B == 0 || d.Nq == 0) return hipSuccess;
  const int G = d.Hq / d.Hkv;
  const int hchunks = (G + kBwdHeads - 1) / kBwdHeads;
  QSA_LAUNCH(sparse_attend_bwd_kernel, dim3((unsigned)d.Nq, (unsigned)(d.Hkv * hchunks), (unsigned)d.B),
             dim3(kBwdThreads), 0, s, q, k, v, lens, sel, n_sel, out, lse, d_out, dq, dk, dv,
             d.Lmax, d.Nq, d.Hq, d.Hkv, d.scale);
  return hipGetLastError();
}

hipError_t launch_index_scores_bwd(const Dims& d, const uint16_t* q_idx, const uint16_t* k_cmp,
                                   const int32_t* lens, const float* g_scores, float* dq_idx,
                                   float* dk_cmp, hipStream_t s) {
  if (d.B == 0 || d.Nq == 0) return hipSuccess;
  const int nbp = d.Lmax / 4;
  const int slice = 1024;
  const unsigned n_slices = (unsigned)((nbp + slice - 1) / slice);
#define QSA_IBWD(KQ)                                                                           \
  QSA_LAUNCH(index_scores_bwd_kernel<KQ>,                                                      \
             dim3(n_slices, (unsigned)((d.Nq + (KQ)-1) / (KQ)), (unsigned)d.B), dim3(kBwdThreads), \
             0, s, q_idx, k_cmp, lens, g_scores, dq_idx, dk_cmp, d.Lmax, d.Nq, slice)
  if (d.Nq <= 4)
    QSA_IBWD(4);
  else if (d.Nq <= 8)
    QSA_IBWD(8);
  else
    QSA_IBWD(16);
#undef QSA_IBWD
  return hipGetLastError();
}

hipError_t launch_compress_bwd(const Dims& d, const float* dk_cmp, const int32_t* lens,
                               float* dk_idx, hipStream_t s) {
  if (d.B == 0) return hipSuccess;
  QSA_LAUNCH(compress_bwd_kernel, dim3(1024, (unsigned)d.B), dim3(256), 0, s, dk_cmp, lens, dk_idx,
             d.Lmax);
  return hipGetLastError();
}

}  // namespace qsa
