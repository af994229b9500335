// Host-side launch interface between the C ABI (api.cpp) and the kernel
// translation units.  Every launcher enqueues on `stream`, never allocates or
// synchronises, and returns hipGetLastError() of its launches.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qsa {

struct Dims {
  int B, Lmax, Nq, Hq, Hkv;
  float scale;
};

// ---- compress.hip
hipError_t launch_compress(const Dims& d, const uint16_t* k_idx, const int32_t* lens,
                           const int32_t* first_block, uint16_t* k_cmp, hipStream_t s);

// ---- expand.hip
hipError_t launch_expand(const Dims& d, const int32_t* lens, const int32_t* sel,
                         const int32_t* n_sel, int32_t* tok, int32_t* n_tok, hipStream_t s);

// ---- topk.hip
enum class TopkPath { kTable, kStream, kScan };
TopkPath choose_topk_path(const Dims& d, uint32_t flags);
size_t topk_workspace_bytes(const Dims& d, TopkPath path);
// Key compression folded into the scoring pass (qsa_forward): the blocks from
// first_block[b] (all when null) to floor(lens[b]/4) are compressed from
// k_idx and written to k_cmp by the pass that scores them.
struct CompressFuse {
  const uint16_t* k_idx;
  const int32_t* first_block;
};
// Whether launch_index_topk can take the compression over (else it is a
// separate launch_compress before it).
bool topk_can_fuse_compress(const Dims& d, TopkPath path);
// The table engine's two passes on their own (launch_index_topk runs both):
// scoring (score table and group maxima in ws) and the per-row pick.
hipError_t launch_table_score(const Dims& d, const uint16_t* q_idx, uint16_t* k_cmp,
                              const int32_t* lens, void* ws, hipStream_t s,
                              const CompressFuse* fuse);
hipError_t launch_table_pick(const Dims& d, const int32_t* lens, int32_t* sel, int32_t* n_sel,
                             void* ws, hipStream_t s);
hipError_t launch_index_topk(const Dims& d, TopkPath path, const uint16_t* q_idx,
                             uint16_t* k_cmp, const int32_t* lens, int32_t* sel,
                             int32_t* n_sel, void* ws, hipStream_t s,
                             const CompressFuse* fuse = nullptr);

// ---- attend.hip
// Paged K/V: token tok of sequence b is row page_table[b * max_pages + tok /
// page] * page + tok % page of a pool of n_pages pages (page = 1 << page_shift).
struct Paged {
  const int32_t* page_table;
  int page_shift, max_pages, n_pages;
};
// Scratch of the sparse attention when a query row is split over several
// workgroups: partial outputs and log-sum-exps.
struct AttendLayout {
  size_t partial_floats, lse_floats;
};
AttendLayout attend_layout(const Dims& d);
hipError_t launch_sparse_attend(const Dims& d, const uint16_t* q, const uint16_t* k,
                                const uint16_t* v, const int32_t* lens, const int32_t* sel,
                                const int32_t* n_sel, uint16_t* out, float* lse, float* part_o,
                                float* part_lse, hipStream_t s, const Paged* pg = nullptr);
size_t dense_workspace_bytes(const Dims& d);
// The indexer's training target (dense attention mass per micro-block, over
// the heads) and the share of it a selection keeps.
size_t teacher_workspace_bytes(const Dims& d);
hipError_t launch_block_teacher(const Dims& d, const uint16_t* q, const uint16_t* k,
                                const uint16_t* v, const int32_t* lens, float* teacher, void* ws,
                                hipStream_t s);
hipError_t launch_teacher_recall(const Dims& d, const float* teacher, const int32_t* lens,
                                 const int32_t* sel, const int32_t* n_sel, float* recall,
                                 hipStream_t s);
hipError_t launch_dense_decode(const Dims& d, const uint16_t* q, const uint16_t* k,
                               const uint16_t* v, const int32_t* lens, uint16_t* out,
                               float* lse, void* ws, hipStream_t s, const Paged* pg = nullptr);
hipError_t launch_dense_prefill(const Dims& d, const uint16_t* q, const uint16_t* k,
                                const uint16_t* v, const int32_t* lens, uint16_t* out, float* lse,
                                hipStream_t s, const Paged* pg = nullptr);

// ---- backward.hip
hipError_t launch_sparse_attend_bwd(const Dims& d, const uint16_t* q, const uint16_t* k,
                                    const uint16_t* v, const int32_t* lens, const int32_t* sel,
                                    const int32_t* n_sel, const uint16_t* out, const float* lse,
                                    const uint16_t* d_out, float* dq, float* dk, float* dv,
                                    hipStream_t s);
hipError_t launch_index_scores_bwd(const Dims& d, const uint16_t* q_idx, const uint16_t* k_cmp,
                                   const int32_t* lens, const float* g_scores, float* dq_idx,
                                   float* dk_cmp, hipStream_t s);
hipError_t launch_compress_bwd(const Dims& d, const float* dk_cmp, const int32_t* lens,
                               float* dk_idx, hipStream_t s);

// Profiling hook: when a caller has attached HIP events (qsa_profile_attach),
// profile_events hands out the next start/stop pair and every launch carries
// them in its own dispatch packet, so the recorded interval is the kernel's
// execution alone (no separate marker packets on the stream).
bool profile_events(const char* name, hipEvent_t* start, hipEvent_t* stop);
void profile_commit();

// Workspace carving: aligned bump allocation inside the caller's buffer.
struct Carve {
  char* base;
  size_t off;
  template <typename T>
  T* take(size_t count) {
    off = (off + 255) & ~size_t(255);
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += count * sizeof(T);
    return p;
  }
};

}  // namespace qsa

#define QSA_LAUNCH_AS(name, kernel, grid, block, shmem, stream, ...)                       \
  do {                                                                                    \
    hipEvent_t qsa_start_ = nullptr, qsa_stop_ = nullptr;                                 \
    const bool qsa_timed_ = ::qsa::profile_events(name, &qsa_start_, &qsa_stop_);         \
    hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream, qsa_start_, qsa_stop_, 0u,  \
                          __VA_ARGS__);                                                   \
    if (qsa_timed_) ::qsa::profile_commit();                                              \
  } while (0)
// The same with the kernel's spelling as the recorded name.
#define QSA_LAUNCH(kernel, grid, block, shmem, stream, ...) \
  QSA_LAUNCH_AS(#kernel, kernel, grid, block, shmem, stream, __VA_ARGS__)
