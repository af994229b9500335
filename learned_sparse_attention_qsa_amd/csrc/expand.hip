// Expansion of the kept micro-blocks back to token positions.
//
// Method: the winners are expanded back to token positions and the
// unfinished block at the sequence tail is added (page "Qwen's million-token
// window has a 2,048-token keyhole", opening section and section "A
// million-token window with a selective view").  Reading: the tail is the
// query's own block, tokens 4*bt .. t.
//
// One workgroup per query row; each thread writes whole 16-byte groups of
// four tokens, so the 2052-entry row (8 KiB) is written with full-width
// coalesced stores.
#include "common.h"
#include "internal.h"

namespace qsa {
namespace {

__global__ __launch_bounds__(128) void expand_kernel(const int32_t* __restrict__ lens,
                                                     const int32_t* __restrict__ sel,
                                                     const int32_t* __restrict__ n_sel,
                                                     int32_t* __restrict__ tok,
                                                     int32_t* __restrict__ n_tok, int Lmax,
                                                     int Nq) {
  const int q = blockIdx.x;
  const int b = blockIdx.y;
  const size_t row = (size_t)b * Nq + q;
  const int t = guard_len(lens[b], Nq, Lmax) - Nq + q;
  int ns = 0, nt = 0, bt = 0;
  if (t >= 0) {
    bt = t >> 2;
    ns = guard(n_sel[row], 0, bt < kTopK ? bt : kTopK);
    nt = 4 * ns + (t - 4 * bt) + 1;
  }
  int4* out = reinterpret_cast<int4*>(tok + row * kMaxTok);
  const int32_t* srow = sel + row * kTopK;
  for (int g = threadIdx.x; g < kMaxTok / 4; g += blockDim.x) {
    int4 w;
    if (g < ns) {
      const int id = srow[g];  // (ids outside [0, bt) are expanded as given)
#ifdef QSA_DEBUG
      if (id < 0 || id >= bt) guard_hit();
#endif
      const int base = 4 * id;
      w = make_int4(base, base + 1, base + 2, base + 3);
    } else {
      int e[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int k = 4 * g + i;
        e[i] = (k < nt) ? 4 * bt + (k - 4 * ns) : -1;
      }
      w = make_int4(e[0], e[1], e[2], e[3]);
    }
    out[g] = w;
  }
  if (threadIdx.x == 0) n_tok[row] = nt;
}

}  // namespace

hipError_t launch_expand(const Dims& d, const int32_t* lens, const int32_t* sel,
                         const int32_t* n_sel, int32_t* tok, int32_t* n_tok, hipStream_t s) {
  if (d.B == 0 || d.Nq == 0) return hipSuccess;
  QSA_LAUNCH(expand_kernel, dim3((unsigned)d.Nq, (unsigned)d.B), dim3(128), 0, s, lens,
                     sel, n_sel, tok, n_tok, d.Lmax, d.Nq);
  return hipGetLastError();
}

}  // namespace qsa
