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

// Stage the V rows of 32 tokens into LDS: lane -> token lane/2, half lane&1.
__device__ __forceinline__ void stage_v(uint16_t* vt, const uint16_t* vrow, bool valid) {
  const int lane = lane_id();
  const uint4* src = reinterpret_cast<const uint4*>(vrow) + (lane & 1) * 8;
  uint4* dst = reinterpret_cast<uint4*>(vt + (lane >> 1) * kVStride + (lane & 1) * 64);
  uint4 buf[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) buf[i] = valid ? src[i] : zero_u4();
#pragma unroll
  for (int i = 0; i < 8; ++i) dst[i] = buf[i];
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
// Grid (n_split, Nq, B); 4 wavefronts; wavefront w takes work items
// w, w+4, ... where item = (kv head, chunk of 16 query heads).
__global__ __launch_bounds__(256) void sparse_attend_kernel(AttnArgs a) {
  __shared__ int32_t s_sel[kTopK];
  __shared__ __align__(16) uint16_t s_v[4][kTile * kVStride];
  const int split = blockIdx.x, q = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const size_t row = (size_t)b * a.Nq + q;
  const int len = clampi(a.lens[b], 0, a.Lmax);
  const int t = len - a.Nq + q;
  int ns = 0, ntok = 0, bt = 0;
  if (t >= 0) {
    bt = t >> 2;
    ns = clampi(a.n_sel[row], 0, bt < kTopK ? bt : kTopK);
    ntok = 4 * ns + (t - 4 * bt) + 1;
  }
  for (int i = tid; i < ns; i += blockDim.x)
    s_sel[i] = clampi(a.sel[row * kTopK + i], 0, bt - 1);  // ids outside [0, bt) are a caller bug
  __syncthreads();
  const int k_begin = split * a.split_tokens;
  const int k_end = min(ntok, k_begin + a.split_tokens);
  const int hchunks = (a.G + 15) >> 4;
  const int items = a.Hkv * hchunks;
  uint16_t* vt = s_v[wave];
  auto tok_at = [&](int kk) -> int {
    return kk < 4 * ns ? 4 * s_sel[kk >> 2] + (kk & 3) : 4 * bt + (kk - 4 * ns);
  };
  const size_t kv_seq = (size_t)b * a.Lmax * a.Hkv;
  for (int item = wave; item < items; item += 4) {
    const int g = item / hchunks, hc = item % hchunks;
    const int h0 = g * a.G + hc * 16;
    const int nh = min(16, a.G - hc * 16);
    const int col = lane & 15;
    bf16x8 qf[4];
    {
      const uint4* qp = reinterpret_cast<const uint4*>(a.q + (row * a.Hq + h0 + min(col, nh - 1)) * kHeadDim);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) qf[ks] = as_bf16x8(col < nh ? qp[ks * 4 + (lane >> 4)] : zero_u4());
    }
    Run r;
    run_init(r);
    for (int k0 = k_begin; k0 < k_end; k0 += kTile) {
      uint4 kf[2][4];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int kk = k0 + s * 16 + (lane & 15);
        const bool valid = kk < k_end;
        const uint4* kp = reinterpret_cast<const uint4*>(
            a.k + ((kv_seq + (size_t)(valid ? tok_at(kk) : 0) * a.Hkv) + g) * kHeadDim);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) kf[s][ks] = valid ? kp[ks * 4 + (lane >> 4)] : zero_u4();
      }
      {
        const int kk = k0 + (lane >> 1);
        const bool valid = kk < k_end;
        stage_v(vt, a.v + ((kv_seq + (size_t)(valid ? tok_at(kk) : 0) * a.Hkv) + g) * kHeadDim,
                valid);
      }
      float z[8];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) acc = mfma16(as_bf16x8(kf[s][ks]), qf[ks], acc);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int kk = k0 + s * 16 + (lane >> 4) * 4 + i;
          z[s * 4 + i] = kk < k_end ? acc[i] * a.scale_log2 : kNegInf;
        }
      }
      wave_sync_lds();
      softmax_pv(r, z, vt);
      wave_sync_lds();
    }
    const int h = h0 + col;
    const bool partial = a.n_split > 1;
    float* po = partial ? a.part_o + (((row * a.Hq) + h) * a.n_split + split) * kHeadDim : nullptr;
    float* pl = partial ? a.part_lse + ((row * a.Hq) + h) * a.n_split + split : nullptr;
    finish(r, col < nh, a.out + (row * a.Hq + h) * kHeadDim, a.lse ? a.lse + row * a.Hq + h : nullptr,
           po, pl, partial);
  }
}

// ------------------------------------------------------------------ dense
// Grid (n_split, Hkv * ceil(Nq*G/16), B); one wavefront per workgroup, 16
// (query, head) columns, all tokens 0..len-1 of the split range, causal mask
// per column.  Always writes partials.
__global__ __launch_bounds__(64) void dense_decode_kernel(AttnArgs a) {
  __shared__ __align__(16) uint16_t s_v[kTile * kVStride];
  const int split = blockIdx.x, b = blockIdx.z;
  const int cchunks = (a.Nq * a.G + 15) >> 4;
  const int g = blockIdx.y / cchunks, cc = blockIdx.y % cchunks;
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
  Run r;
  run_init(r);
  for (int k0 = k_begin; k0 < k_end; k0 += kTile) {
    uint4 kf[2][4];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int kk = k0 + s * 16 + (lane & 15);
      const bool valid = kk < k_end;
      const uint4* kp = reinterpret_cast<const uint4*>(
          a.k + ((kv_seq + (size_t)(valid ? kk : 0) * a.Hkv) + g) * kHeadDim);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kf[s][ks] = valid ? kp[ks * 4 + (lane >> 4)] : zero_u4();
    }
    {
      const int kk = k0 + (lane >> 1);
      const bool valid = kk < k_end;
      stage_v(s_v, a.v + ((kv_seq + (size_t)(valid ? kk : 0) * a.Hkv) + g) * kHeadDim, valid);
    }
    float z[8];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) acc = mfma16(as_bf16x8(kf[s][ks]), qf[ks], acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kk = k0 + s * 16 + (lane >> 4) * 4 + i;
        z[s * 4 + i] = (kk < k_end && kk <= tq) ? acc[i] * a.scale_log2 : kNegInf;
      }
    }
    wave_sync_lds();
    softmax_pv(r, z, s_v);
    wave_sync_lds();
  }
  float* po = a.part_o + (((row * a.Hq) + h) * a.n_split + split) * kHeadDim;
  float* pl = a.part_lse + ((row * a.Hq) + h) * a.n_split + split;
  finish(r, col_valid, nullptr, nullptr, po, pl, true);
}

// ------------------------------------------------------------------ merge
// Grid (Hq, Nq, B), 128 threads (one per output dim).
__global__ __launch_bounds__(128) void merge_kernel(const float* __restrict__ part_o,
                                                    const float* __restrict__ part_lse,
                                                    uint16_t* __restrict__ out,
                                                    float* __restrict__ lse, int Nq, int Hq,
                                                    int n_split) {
  const int h = blockIdx.x, q = blockIdx.y, b = blockIdx.z, d = threadIdx.x;
  const size_t rh = ((size_t)b * Nq + q) * Hq + h;
  const float* pl = part_lse + rh * n_split;
  const float* po = part_o + rh * n_split * kHeadDim;
  float M = kNegInf;
  for (int s = 0; s < n_split; ++s) M = fmaxf(M, pl[s]);
  float acc = 0.f, sw = 0.f;
  if (M != kNegInf) {
    for (int s = 0; s < n_split; ++s) {
      const float w = __expf(pl[s] - M);
      sw += w;
      acc += w * po[(size_t)s * kHeadDim + d];
    }
  }
  const float o = sw > 0.f ? acc / sw : 0.f;
  out[rh * kHeadDim + d] = (uint16_t)f32_to_bf16(o);
  if (lse && d == 0) lse[rh] = sw > 0.f ? M + __logf(sw) : kNegInf;
}

int sparse_splits(const Dims& d, int* split_tokens) {
  // Enough workgroups to cover the chip for decode-sized batches; one split
  // (no merge) when there are already many query rows.
  const long long rows = (long long)d.B * d.Nq;
  int n_split = 1;
  if (rows < 1024) {
    n_split = (int)((1024 + rows - 1) / rows);
    const int max_split = (kMaxTok + kTile - 1) / kTile;
    if (n_split > max_split) n_split = max_split;
  }
  int st = (kMaxTok + n_split - 1) / n_split;
  st = (st + kTile - 1) / kTile * kTile;
  n_split = (kMaxTok + st - 1) / st;
  *split_tokens = st;
  return n_split;
}

int dense_splits(const Dims& d, int* split_tokens) {
  // About 8K single-wavefront workgroups in total, at least 256 tokens each.
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

size_t attend_workspace_bytes(const Dims& d) {
  int st;
  const int ns = sparse_splits(d, &st);
  if (ns <= 1) return 0;
  Carve c{nullptr, 0};
  const size_t rh = (size_t)d.B * d.Nq * d.Hq;
  c.take<float>(rh * ns * kHeadDim);
  c.take<float>(rh * ns);
  return c.off;
}

hipError_t launch_sparse_attend(const Dims& d, const uint16_t* q, const uint16_t* k,
                                const uint16_t* v, const int32_t* lens, const int32_t* sel,
                                const int32_t* n_sel, uint16_t* out, float* lse, void* ws,
                                hipStream_t s) {
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
  a.n_split = sparse_splits(d, &a.split_tokens);
  if (a.n_split > 1) {
    Carve c{static_cast<char*>(ws), 0};
    const size_t rh = (size_t)d.B * d.Nq * d.Hq;
    a.part_o = c.take<float>(rh * a.n_split * kHeadDim);
    a.part_lse = c.take<float>(rh * a.n_split);
  }
  QSA_LAUNCH(sparse_attend_kernel, dim3((unsigned)a.n_split, (unsigned)d.Nq, (unsigned)d.B),
                     dim3(256), 0, s, a);
  if (a.n_split > 1)
    QSA_LAUNCH(merge_kernel, dim3((unsigned)d.Hq, (unsigned)d.Nq, (unsigned)d.B), dim3(128),
                       0, s, a.part_o, a.part_lse, out, lse, d.Nq, d.Hq, a.n_split);
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
  const int cchunks = (d.Nq * a.G + 15) / 16;
  QSA_LAUNCH(dense_decode_kernel,
                     dim3((unsigned)a.n_split, (unsigned)(d.Hkv * cchunks), (unsigned)d.B), dim3(64),
                     0, s, a);
  QSA_LAUNCH(merge_kernel, dim3((unsigned)d.Hq, (unsigned)d.Nq, (unsigned)d.B), dim3(128), 0,
                     s, a.part_o, a.part_lse, out, lse, d.Nq, d.Hq, a.n_split);
  return hipGetLastError();
}

}  // namespace qsa
