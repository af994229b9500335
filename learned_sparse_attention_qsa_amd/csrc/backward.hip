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
// The products q . k, dO . v and q_h . kc_j run on the matrix cores (bf16
// inputs, exact products, float32 sums); every gradient sum is float32 vector
// FMA.
#include <algorithm>

#include "common.h"
#include "internal.h"

namespace qsa {
namespace {

constexpr int kBwdThreads = 256;
constexpr int kBwdTile = 64;    // tokens per step
constexpr float kLog2eB = 1.4426950408889634f;

__device__ __forceinline__ float bf(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Grid (Nq * kAbChunks, Hkv * hchunks, B), 256 threads: one chunk of up to
// 256 entries of one query's token list, one KV head g and up to kH of its
// query heads (rows of the 16-row MFMA tiles past the group's heads are
// zero).  Per 64-token tile:
//  1. wavefront w, tokens 16 w .. 16 w + 15, on the matrix cores: the logits
//     z = q_h . k_s and dp_s = dO_h . v_s of the 16 x 16 (head, token) pairs
//     in four 16x16x32 bf16 steps each (bf16 inputs, float32 sums); a lane
//     holds four heads of one token and forms p = exp(scale z - lse) and
//     ds = p (dp - D_h), stored in LDS with the tile's keys and token ids;
//  2. float32 FMA: a thread owns kDT = 32 / kH dimensions, 128 / kDT
//     apart, and every (256 kDT / 128)-th token of the tile and adds ds k
//     into its dq registers and scale sum_h ds q_h, sum_h p dO_h into dk,
//     dv (atomic adds, as a token can be read by several queries and head
//     chunks; the lanes of one add cover whole 128-byte lines).
// dq is summed over the workgroup (shuffles, then LDS) and added to dq, which
// a fill kernel clears first (the chunks of one query add into the same rows).
constexpr int kAbChunk = 256;                                  // token list entries per workgroup
constexpr int kAbChunks = (kMaxTok + kAbChunk - 1) / kAbChunk;  // chunks per query
constexpr int kAbKRow = kHeadDim / 8 + 1;                      // LDS key row in uint4 (staggered)

template <int kH>
__global__ __launch_bounds__(kBwdThreads) void sparse_attend_bwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ lens, const int32_t* __restrict__ sel,
    const int32_t* __restrict__ n_sel, const uint16_t* __restrict__ out,
    const float* __restrict__ lse, const uint16_t* __restrict__ d_out, float* __restrict__ dq,
    float* __restrict__ dk, float* __restrict__ dv, int Lmax, int Nq, int Hq, int Hkv,
    float scale) {
  constexpr int kDT = 32 / kH;                   // dimensions per thread in the FMA phase
  constexpr int kTPT = kHeadDim / kDT;           // threads per token
  constexpr int kTG = kBwdThreads / kTPT;        // token groups
  __shared__ uint4 s_k[kBwdTile * kAbKRow];
  __shared__ f32x4 s_p[kBwdTile * kH / 4], s_ds[kBwdTile * kH / 4];
  __shared__ int32_t s_tok[kBwdTile];
  __shared__ int32_t s_sel[kAbChunk / kBlock];
  __shared__ float s_D[16], s_lse2[16];
  __shared__ float s_part[kBwdThreads / 64][kH * kHeadDim];
  __shared__ uint4 s_qd[2 * kH * kHeadDim / 8];
  const int qi = blockIdx.x / kAbChunks, chunk = blockIdx.x % kAbChunks;
  const int b = blockIdx.z, tid = threadIdx.x;
  const int G = Hq / Hkv, hchunks = (G + kH - 1) / kH;
  const int g = blockIdx.y / hchunks, hc = blockIdx.y % hchunks;
  const int h0 = g * G + hc * kH, nh = min(kH, G - hc * kH);
  const size_t row = (size_t)b * Nq + qi;
  const int len = guard_len(lens[b], Nq, Lmax);
  const int t = len - Nq + qi;
  const int bt = t >> 2;
  const int ns = guard(n_sel[row], 0, min(bt, kTopK));
  const int ntok = 4 * ns + (t - 4 * bt) + 1;
  const int c0 = chunk * kAbChunk, c1 = min(c0 + kAbChunk, ntok);
  if (c0 >= c1) return;  // (uniform over the workgroup)
  for (int i = tid; i < kAbChunk / kBlock; i += kBwdThreads) {
    const int j = (c0 >> 2) + i;
    s_sel[i] = j < ns ? guard(sel[row * kTopK + j], 0, bt - 1) : 0;
  }
  // Loads below are unconditional (rows clamped to the chunk's heads, values
  // masked after), so that each group of them costs one memory round trip.
  {
    // 16 lanes per head, eight dimensions each: partial dot products of dO and O
    const int h = tid >> 4, part = tid & 15;
    const size_t off = (row * Hq + h0 + min(h, nh - 1)) * kHeadDim + 8 * part;
    const uint4 a = *reinterpret_cast<const uint4*>(d_out + off);
    const uint4 o = *reinterpret_cast<const uint4*>(out + off);
    const float l2 = lse[row * Hq + h0 + min(h, nh - 1)] * kLog2eB;
    const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, ow[4] = {o.x, o.y, o.z, o.w};
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc = fmaf(bf16_lo(aw[i]), bf16_lo(ow[i]), acc);
      acc = fmaf(bf16_hi(aw[i]), bf16_hi(ow[i]), acc);
    }
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
    if (part == 0) {
      s_D[h] = h < nh ? acc : 0.f;
      s_lse2[h] = h < nh ? l2 : 0.f;
    }
  }
  const int lane = lane_id(), wave = tid >> 6;
  const int r = lane & 15, kc = lane >> 4;
  // A fragments: head r, dimensions 32 ks + 8 kc ..
  bf16x8 qa[4], da[4];
  {
    const uint4* pq = reinterpret_cast<const uint4*>(q + (row * Hq + h0 + min(r, nh - 1)) * kHeadDim);
    const uint4* pd =
        reinterpret_cast<const uint4*>(d_out + (row * Hq + h0 + min(r, nh - 1)) * kHeadDim);
    uint4 uq[4], ud[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      uq[ks] = pq[4 * ks + kc];
      ud[ks] = pd[4 * ks + kc];
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      qa[ks] = as_bf16x8(r < nh ? uq[ks] : zero_u4());
      da[ks] = as_bf16x8(r < nh ? ud[ks] : zero_u4());
    }
  }
  // FMA side: this thread's dimensions d0 + e kTPT (e < kDT) and token group
  const int d0 = tid % kTPT, tg = tid / kTPT;
  // the chunk's q and dO rows, staged in LDS for the FMA side
  for (int i = tid; i < 2 * kH * (kHeadDim / 8); i += kBwdThreads) {
    const int src = i / (kH * (kHeadDim / 8)), rem = i % (kH * (kHeadDim / 8));
    const int h = rem / (kHeadDim / 8), c = rem % (kHeadDim / 8);
    const uint16_t* p = (src ? d_out : q) + (row * Hq + h0 + min(h, nh - 1)) * kHeadDim;
    s_qd[i] = reinterpret_cast<const uint4*>(p)[c];
  }
  __syncthreads();
  float qr[kH][kDT], dr[kH][kDT], acc_dq[kH][kDT];
  {
    const uint16_t* sq = reinterpret_cast<const uint16_t*>(s_qd);
#pragma unroll
    for (int h = 0; h < kH; ++h)
#pragma unroll
      for (int e = 0; e < kDT; ++e) {
        const int off = h * kHeadDim + d0 + e * kTPT;
        qr[h][e] = h < nh ? bf(sq[off]) : 0.f;
        dr[h][e] = h < nh ? bf(sq[kH * kHeadDim + off]) : 0.f;
        acc_dq[h][e] = 0.f;
      }
  }
  float Dl[4], L2[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    Dl[i] = s_D[4 * kc + i];
    L2[i] = s_lse2[4 * kc + i];
  }
  const float sl2 = scale * kLog2eB;
  const size_t kv_seq = (size_t)b * Lmax * Hkv;
  const uint4* k4 = reinterpret_cast<const uint4*>(k);
  const uint4* v4 = reinterpret_cast<const uint4*>(v);
  const uint16_t* skh = reinterpret_cast<const uint16_t*>(s_k);
  const float* spf = reinterpret_cast<const float*>(s_p);
  const float* sdf = reinterpret_cast<const float*>(s_ds);
  // the lane's token of a tile and its K and V pieces, loaded one tile ahead
  const int rl = wave * 16 + r;
  int tok = 0;
  uint4 kb[4], vb[4];
  auto load_kv = [&](int k0) {
    const int kk = k0 + rl;
    // a dead slot reads the own block's first token (ds = p = 0 there)
    tok = kk >= c1 ? 4 * bt
          : kk < 4 * ns ? 4 * s_sel[(kk - c0) >> 2] + (kk & 3)
                        : 4 * bt + (kk - 4 * ns);
    const size_t rb = (kv_seq + (size_t)tok * Hkv + g) * (kHeadDim / 8);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      kb[ks] = k4[rb + 4 * ks + kc];
      vb[ks] = v4[rb + 4 * ks + kc];
    }
  };
  load_kv(c0);
  for (int k0 = c0; k0 < c1; k0 += kBwdTile) {
    {
      const bool live = k0 + rl < c1;
      f32x4 z = {0.f, 0.f, 0.f, 0.f}, dp = z;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        z = mfma16(qa[ks], as_bf16x8(kb[ks]), z);
        dp = mfma16(da[ks], as_bf16x8(vb[ks]), dp);
        s_k[rl * kAbKRow + 4 * ks + kc] = kb[ks];
      }
      if (4 * kc < kH) {
        f32x4 pv, dsv;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool on = live && 4 * kc + i < nh;
          const float p = on ? exp2f(z[i] * sl2 - L2[i]) : 0.f;
          pv[i] = p;
          dsv[i] = on ? p * (dp[i] - Dl[i]) : 0.f;
        }
        s_p[rl * (kH / 4) + kc] = pv;
        s_ds[rl * (kH / 4) + kc] = dsv;
      }
      if (kc == 0) s_tok[rl] = live ? tok : -1;
    }
    __syncthreads();
    if (k0 + kBwdTile < c1) load_kv(k0 + kBwdTile);
#pragma unroll 2
    for (int jr = tg; jr < kBwdTile; jr += kTG) {
      const int tk = s_tok[jr];
      if (tk < 0) continue;
      float kv[kDT], ak[kDT], av[kDT];
#pragma unroll
      for (int e = 0; e < kDT; ++e) {
        kv[e] = bf(skh[jr * kAbKRow * 8 + d0 + e * kTPT]);
        ak[e] = 0.f;
        av[e] = 0.f;
      }
#pragma unroll
      for (int h = 0; h < kH; ++h) {
        const float ds = sdf[jr * kH + h], p = spf[jr * kH + h];
#pragma unroll
        for (int e = 0; e < kDT; ++e) {
          acc_dq[h][e] = fmaf(ds, kv[e], acc_dq[h][e]);
          ak[e] = fmaf(ds, qr[h][e], ak[e]);
          av[e] = fmaf(p, dr[h][e], av[e]);
        }
      }
      const size_t off = (kv_seq + (size_t)tk * Hkv + g) * kHeadDim + d0;
#pragma unroll
      for (int e = 0; e < kDT; ++e) {
        atomicAdd(&dk[off + e * kTPT], scale * ak[e]);
        atomicAdd(&dv[off + e * kTPT], av[e]);
      }
    }
    __syncthreads();
  }
  // dq: the lanes of a wavefront that share dimensions summed by shuffles,
  // each wavefront's sums stored in its own LDS region, the regions summed
  // by the workgroup (LDS atomic adds from lanes that share an address cost
  // far more)
  constexpr int kLPW = 64 / kTPT;  // token groups per wavefront
#pragma unroll
  for (int h = 0; h < kH; ++h)
#pragma unroll
    for (int e = 0; e < kDT; ++e)
#pragma unroll
      for (int m = kTPT; m < 64; m <<= 1) acc_dq[h][e] += __shfl_xor(acc_dq[h][e], m);
  const int gw = lane / kTPT;
#pragma unroll
  for (int h = 0; h < kH; ++h)
    if (h % kLPW == gw) {
#pragma unroll
      for (int e = 0; e < kDT; ++e) s_part[wave][h * kHeadDim + d0 + e * kTPT] = acc_dq[h][e];
    }
  __syncthreads();
  for (int i = tid; i < nh * kHeadDim; i += kBwdThreads) {
    float x = 0.f;
#pragma unroll
    for (int w = 0; w < kBwdThreads / 64; ++w) x += s_part[w][i];
    atomicAdd(&dq[(row * Hq + h0) * kHeadDim + i], scale * x);
  }
}

__global__ void zero_f32_kernel(float* __restrict__ p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0.f;
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16k16(s16x4 a, s16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// bf16 bits of x rounded to nearest even (finite x).
__device__ __forceinline__ uint32_t bf16_rne_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// x = hi + mid + lo, each part a bf16 rounded to nearest even from what the
// previous parts leave (each subtraction is exact); the three parts carry 24
// significant bits, so their products with a bf16 value, summed in float32,
// match float32 arithmetic on x.
__device__ __forceinline__ void split3_bf16(float x, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  hi = bf16_rne_bits(x);
  const float r1 = x - __uint_as_float(hi << 16);
  mid = bf16_rne_bits(r1);
  lo = bf16_rne_bits(r1 - __uint_as_float(mid << 16));
}

// Grid (n_slices, ceil(Nq / kQ), B), 256 threads (four wavefronts): the
// blocks of one slice against up to kQ queries of one sequence.  Each
// wavefront takes 64-block tiles of the slice in turn:
//  1. on the matrix cores: the products q_r . kc_j of the kQ x 4 (query,
//     head) rows r and the tile's blocks, 16 x 16 per pair of 16x16x32 bf16
//     MFMA steps.  A lane then holds four heads of one query for one block
//     and keeps w = g (product > 0 and the block a candidate of the query)
//     or 0; that is the A fragment layout of a 16x16x16 step with blocks as
//     rows, so dkc_j,d = sum_r w_j,r q_r,d follows from three such steps per
//     16 rows r (w split into three bf16 parts; q is bf16) with no exchange
//     between lanes.  The B fragments give lane column c the dimension
//     4 c + n of column tile n, so a lane ends with four consecutive
//     dimensions of four blocks, added to dk_cmp 16 bytes at a time (a
//     read-add-write, the old values read one tile ahead, when this
//     workgroup is the rows' only writer; atomic adds otherwise).  The w
//     rows and the tile's keys go to the wavefront's LDS;
//  2. float32 FMA: a lane owns kDL = 16 / kQ consecutive dimensions of
//     every kDL-th block of the tile (from its lane group's offset) and adds
//     w_j,r kc_j,d to its dq_r,d registers.
// The lanes' dq are summed (shuffles, then LDS) and added to dq_idx at the end.
template <int kQ>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(kQ <= 4 ? 2 : 1)))
void index_scores_bwd_kernel(
    const uint16_t* __restrict__ q_idx, const uint16_t* __restrict__ k_cmp,
    const int32_t* __restrict__ lens, const float* __restrict__ g_scores,
    float* __restrict__ dq_idx, float* __restrict__ dk_cmp, int Lmax, int Nq, int slice_blocks) {
  constexpr int kR = kQ * kIdxHeads;   // (query, head) rows
  constexpr int kMT = kR / 16;         // 16-row MFMA tiles
  constexpr int kDL = 16 / kQ;         // dimensions per lane in the dq sums
  constexpr int kG = kIdxDim / kDL;    // lanes per block in the dq sums
  constexpr int kKRow = 9;             // LDS key row: 64 bf16 + 16 bytes of stagger, in uint4
  constexpr int kWRow = kR / 4;        // LDS w row, in float4
  constexpr int kWaves = kBwdThreads / 64;
  __shared__ uint4 s_k[kWaves][64 * kKRow];
  __shared__ f32x4 s_w[kWaves][64 * kWRow];
  const int slice = blockIdx.x, q0 = blockIdx.y * kQ, b = blockIdx.z, tid = threadIdx.x;
  const int nq = min(kQ, Nq - q0);
  const int len = guard_len(lens[b], Nq, Lmax);
  const int nbp = Lmax >> 2;
  const int t_last = len - Nq + q0 + nq - 1;
  const int j0 = slice * slice_blocks, j1 = min(j0 + slice_blocks, t_last >> 2);
  if (j1 <= j0) return;  // (uniform over the workgroup)

  const int lane = lane_id(), wave = tid >> 6;
  const int r = lane & 15, kc = lane >> 4;
  const size_t qrow0 = (size_t)b * Nq + q0;
  // (unconditional loads, rows clamped to the workgroup's queries and
  // masked after: one memory round trip for all of them)
  // products: A fragments (row 16 mt + r = query 4 mt + r / 4, head r % 4,
  // dimensions 8 kc.. and 32 + 8 kc..) and this lane's query 4 mt + kc;
  // dk_cmp: B fragments (rows 16 mt + 4 kc + i, dimension 4 r + n)
  bf16x8 qa[kMT][2];
  s16x4 qb[kMT][4];
  int lim[kMT];
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt) {
    const int qq = 4 * mt + (r >> 2);
    const uint4* p = reinterpret_cast<const uint4*>(
        q_idx + ((qrow0 + min(qq, nq - 1)) * kIdxHeads + (r & 3)) * kIdxDim);
    const uint4 u0 = p[kc], u1 = p[4 + kc];
    qa[mt][0] = as_bf16x8(qq < nq ? u0 : zero_u4());
    qa[mt][1] = as_bf16x8(qq < nq ? u1 : zero_u4());
    const int qw = 4 * mt + kc;
    lim[mt] = qw < nq ? min((len - Nq + q0 + qw) >> 2, j1) : 0;
    uint2 qd[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      qd[i] = *reinterpret_cast<const uint2*>(
          q_idx + (qrow0 * kIdxHeads + min(16 * mt + 4 * kc + i, kIdxHeads * nq - 1)) * kIdxDim +
          4 * r);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool on = (16 * mt + 4 * kc + i) / kIdxHeads < nq;
      qb[mt][0][i] = on ? (short)(qd[i].x & 0xffffu) : (short)0;
      qb[mt][1][i] = on ? (short)(qd[i].x >> 16) : (short)0;
      qb[mt][2][i] = on ? (short)(qd[i].y & 0xffffu) : (short)0;
      qb[mt][3][i] = on ? (short)(qd[i].y >> 16) : (short)0;
    }
  }
  // dq sums: this lane's dimensions d0.. of every row
  const int d0 = (lane % kG) * kDL, js = lane / kG;
  float dq[kR][kDL];
#pragma unroll
  for (int rr = 0; rr < kR; ++rr)
#pragma unroll
    for (int e = 0; e < kDL; ++e) dq[rr][e] = 0.f;
  __syncthreads();

  const uint4* kb = reinterpret_cast<const uint4*>(k_cmp + (size_t)b * nbp * kIdxDim);
  const float* gb = g_scores + qrow0 * nbp;
  float* dkb = dk_cmp + (size_t)b * nbp * kIdxDim;
  const bool sole = gridDim.y == 1;
  uint4* sk = s_k[wave];
  f32x4* sw = s_w[wave];
  const int ntiles = (j1 - j0 + 63) >> 6;
  // the tile's keys, g values and (sole writer) dk_cmp values, loaded one
  // tile ahead
  uint4 bv[4][2];
  float gv[kMT][4];
  f32x4 old[4][4];
  auto load_tile = [&](int jt) {
    // Unconditional loads: a block past the slice re-reads its last one and
    // gets w = 0 (and no add).
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
    if (sole) {
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = min(jt + nt * 16 + 4 * kc + i, j1 - 1);
          old[nt][i] = *reinterpret_cast<const f32x4*>(dkb + (size_t)j * kIdxDim + 4 * r);
        }
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
      f32x4 dk[4];
#pragma unroll
      for (int n = 0; n < 4; ++n) dk[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = mfma16(qa[mt][0], as_bf16x8(bv[nt][0]), acc);
        acc = mfma16(qa[mt][1], as_bf16x8(bv[nt][1]), acc);
        const float g = gv[mt][nt];
        f32x4 w;
        s16x4 wh, wm, wl;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          w[i] = acc[i] > 0.f ? g : 0.f;
          uint32_t h, m, l;
          split3_bf16(w[i], h, m, l);
          wh[i] = (short)h;
          wm[i] = (short)m;
          wl[i] = (short)l;
        }
        sw[(nt * 16 + r) * kWRow + 4 * mt + kc] = w;
#pragma unroll
        for (int n = 0; n < 4; ++n) {
          dk[n] = mfma16k16(wh, qb[mt][n], dk[n]);
          dk[n] = mfma16k16(wm, qb[mt][n], dk[n]);
          dk[n] = mfma16k16(wl, qb[mt][n], dk[n]);
        }
      }
      // dk[n][i]: block jt + 16 nt + 4 kc + i, dimension 4 r + n
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = jt + nt * 16 + 4 * kc + i;
        if (j < j1) {
          float* dst = dkb + (size_t)j * kIdxDim + 4 * r;
          if (sole) {
            f32x4 o = old[nt][i];
#pragma unroll
            for (int n = 0; n < 4; ++n) o[n] += dk[n][i];
            *reinterpret_cast<f32x4*>(dst) = o;
          } else {
#pragma unroll
            for (int n = 0; n < 4; ++n)
              if (dk[n][i] != 0.f) atomicAdd(&dst[n], dk[n][i]);
          }
        }
      }
    }
    wave_sync_lds();
    if (tile + kWaves < ntiles) load_tile(jt + kWaves * 64);
    const uint16_t* skh = reinterpret_cast<const uint16_t*>(sk);
#pragma unroll 2
    for (int jj = 0; jj < 64 / kDL; ++jj) {
      const int jl = jj * kDL + js;
      float kv[kDL];
#pragma unroll
      for (int e = 0; e < kDL; ++e) kv[e] = bf(skh[jl * kKRow * 8 + d0 + e]);
#pragma unroll
      for (int c = 0; c < kWRow; ++c) {
        const f32x4 w4 = sw[jl * kWRow + c];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int e = 0; e < kDL; ++e) dq[4 * c + i][e] = fmaf(w4[i], kv[e], dq[4 * c + i][e]);
      }
    }
  }
  // dq: the kDL lanes of a dimension group summed by shuffles, each
  // wavefront's sums stored in its own LDS region (its w rows are done with),
  // the four regions summed by the workgroup.  (LDS atomic adds from lanes
  // that share an address cost far more than this.)
#pragma unroll
  for (int rr = 0; rr < kR; ++rr)
#pragma unroll
    for (int e = 0; e < kDL; ++e)
#pragma unroll
      for (int m = kG; m < 64; m <<= 1) dq[rr][e] += __shfl_xor(dq[rr][e], m);
  float* part = reinterpret_cast<float*>(sw);  // kR x 64 floats
  wave_sync_lds();
#pragma unroll
  for (int rr = 0; rr < kR; ++rr)
    if (js == rr % kDL) {
#pragma unroll
      for (int e = 0; e < kDL; ++e) part[rr * kIdxDim + d0 + e] = dq[rr][e];
    }
  __syncthreads();
  float* dqb = dq_idx + qrow0 * kIdxHeads * kIdxDim;
  const float* parts = reinterpret_cast<const float*>(&s_w[0][0]);
  for (int i = tid; i < nq * kIdxHeads * kIdxDim; i += kBwdThreads) {
    float x = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) x += parts[w * kR * kIdxDim + i];
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
  const size_t nq_el = (size_t)d.B * d.Nq * d.Hq * kHeadDim;
  QSA_LAUNCH(zero_f32_kernel, dim3((unsigned)std::min<size_t>((nq_el + 255) / 256, 1024)),
             dim3(256), 0, s, dq, nq_el);
  const int G = d.Hq / d.Hkv;
  const dim3 block(kBwdThreads);
  if (G <= 8) {
    const dim3 grid((unsigned)(d.Nq * kAbChunks), (unsigned)d.Hkv, (unsigned)d.B);
    QSA_LAUNCH(sparse_attend_bwd_kernel<8>, grid, block, 0, s, q, k, v, lens, sel, n_sel, out,
               lse, d_out, dq, dk, dv, d.Lmax, d.Nq, d.Hq, d.Hkv, d.scale);
  } else {
    const dim3 grid((unsigned)(d.Nq * kAbChunks), (unsigned)(d.Hkv * ((G + 15) / 16)),
                    (unsigned)d.B);
    QSA_LAUNCH(sparse_attend_bwd_kernel<16>, grid, block, 0, s, q, k, v, lens, sel, n_sel, out,
               lse, d_out, dq, dk, dv, d.Lmax, d.Nq, d.Hq, d.Hkv, d.scale);
  }
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
