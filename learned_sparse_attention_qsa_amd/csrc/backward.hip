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

// Grid (n_slices, ceil(Nq / 16), B), 256 threads: the blocks of one slice
// against up to 16 queries of one sequence.  Thread per block: the four
// heads' dot products, the gradient's mask, dkc of the block (registers,
// added to dk_cmp at the end) and dq (LDS, added to dq_idx at the end).
constexpr int kIbwdQ = 16;
__global__ __launch_bounds__(kBwdThreads) void index_scores_bwd_kernel(
    const uint16_t* __restrict__ q_idx, const uint16_t* __restrict__ k_cmp,
    const int32_t* __restrict__ lens, const float* __restrict__ g_scores,
    float* __restrict__ dq_idx, float* __restrict__ dk_cmp, int Lmax, int Nq, int slice_blocks) {
  __shared__ float s_q[kIbwdQ][kIdxHeads][kIdxDim];
  __shared__ float s_dq[kIbwdQ][kIdxHeads][kIdxDim];
  const int slice = blockIdx.x, q0 = blockIdx.y * kIbwdQ, b = blockIdx.z, tid = threadIdx.x;
  const int nq = min(kIbwdQ, Nq - q0);
  const int len = guard_len(lens[b], Nq, Lmax);
  const int nbp = Lmax >> 2;
  for (int i = tid; i < kIbwdQ * kIdxHeads * kIdxDim; i += kBwdThreads) {
    const int qq = i / (kIdxHeads * kIdxDim), rem = i % (kIdxHeads * kIdxDim);
    (&s_q[0][0][0])[i] =
        qq < nq ? bf(q_idx[((size_t)b * Nq + q0 + qq) * kIdxHeads * kIdxDim + rem]) : 0.f;
    (&s_dq[0][0][0])[i] = 0.f;
  }
  __syncthreads();
  const int t_last = len - Nq + q0 + nq - 1;
  const int bt_max = t_last >= 0 ? (t_last >> 2) : 0;
  const int j0 = slice * slice_blocks, j1 = min(j0 + slice_blocks, bt_max);
  for (int j = j0 + tid; j < j1; j += kBwdThreads) {
    float kc[kIdxDim];
    const uint4* kr = reinterpret_cast<const uint4*>(k_cmp + ((size_t)b * nbp + j) * kIdxDim);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const uint4 u = kr[c];
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kc[8 * c + 2 * e] = bf16_lo(w[e]);
        kc[8 * c + 2 * e + 1] = bf16_hi(w[e]);
      }
    }
    float dkc[kIdxDim];
#pragma unroll
    for (int d = 0; d < kIdxDim; ++d) dkc[d] = 0.f;
    for (int qq = 0; qq < nq; ++qq) {
      const int t = len - Nq + q0 + qq;
      if (t < 0 || j >= (t >> 2)) continue;  // not a candidate of this query
      const float gj = g_scores[((size_t)b * Nq + q0 + qq) * nbp + j];
      if (gj == 0.f) continue;
#pragma unroll
      for (int h = 0; h < kIdxHeads; ++h) {
        float dot = 0.f;
#pragma unroll
        for (int d = 0; d < kIdxDim; ++d) dot = fmaf(s_q[qq][h][d], kc[d], dot);
        if (dot > 0.f) {
#pragma unroll
          for (int d = 0; d < kIdxDim; ++d) {
            dkc[d] = fmaf(gj, s_q[qq][h][d], dkc[d]);
            atomicAdd(&s_dq[qq][h][d], gj * kc[d]);
          }
        }
      }
    }
    float* dst = dk_cmp + ((size_t)b * nbp + j) * kIdxDim;
#pragma unroll
    for (int d = 0; d < kIdxDim; ++d)
      if (dkc[d] != 0.f) atomicAdd(&dst[d], dkc[d]);
  }
  __syncthreads();
  for (int i = tid; i < nq * kIdxHeads * kIdxDim; i += kBwdThreads) {
    const float x = (&s_dq[0][0][0])[i];
    if (x != 0.f) atomicAdd(&dq_idx[((size_t)b * Nq + q0) * kIdxHeads * kIdxDim + i], x);
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
  QSA_LAUNCH(index_scores_bwd_kernel,
             dim3(n_slices, (unsigned)((d.Nq + kIbwdQ - 1) / kIbwdQ), (unsigned)d.B),
             dim3(kBwdThreads), 0, s, q_idx, k_cmp, lens, g_scores, dq_idx, dk_cmp, d.Lmax, d.Nq,
             slice);
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
