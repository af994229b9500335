// C ABI of libqsa: argument validation, workspace sizing and kernel dispatch.
// Every entry point checks what the host can see before it launches anything,
// returns a status code, and never throws, allocates, frees or synchronises
// (except the opt-in QSA_CHECK validation of device `lens`).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../../include/qsa.h"
#include "internal.h"

using qsa::Dims;

// ---------------------------------------------------------------- profiling
namespace {
constexpr int kMaxProfiled = 1024;
thread_local void** t_events = nullptr;
thread_local int t_cap = 0;
thread_local int t_count = 0;
thread_local const char* t_names[kMaxProfiled];
}  // namespace

namespace qsa {
bool profile_events(const char* name, hipEvent_t* start, hipEvent_t* stop) {
  if (!t_events || t_count >= kMaxProfiled || 2 * t_count + 1 >= t_cap) return false;
  *start = static_cast<hipEvent_t>(t_events[2 * t_count]);
  *stop = static_cast<hipEvent_t>(t_events[2 * t_count + 1]);
  t_names[t_count] = name;
  return true;
}
void profile_commit() { ++t_count; }

#ifdef QSA_DEBUG
// Guard counters of the source files (debug builds register one per file).
namespace {
std::vector<hipError_t (*)(unsigned int*)>& guard_counters() {
  static std::vector<hipError_t (*)(unsigned int*)> v;
  return v;
}
}  // namespace
void register_guard_counter(hipError_t (*read_and_clear)(unsigned int*)) {
  guard_counters().push_back(read_and_clear);
}
#endif
}  // namespace qsa

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_ok[kMaxDevices];  // 0 unknown, 1 gfx950, -1 other

qsa_status check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return QSA_ERR_DEVICE;
  if (dev < 0 || dev >= kMaxDevices) return QSA_ERR_DEVICE;
  int st = g_arch_ok[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return QSA_ERR_DEVICE;
    st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    g_arch_ok[dev].store(st, std::memory_order_relaxed);
  }
  return st == 1 ? QSA_OK : QSA_ERR_DEVICE;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

qsa_status check_shape(const qsa_shape* s, Dims* d) {
  if (!s) return QSA_ERR_NULL;
  if (s->batch < 0 || s->n_query < 0 || s->max_len <= 0 || (s->max_len % 4) != 0)
    return QSA_ERR_SHAPE;
  if (s->n_query > s->max_len || s->max_len > (1 << 30)) return QSA_ERR_SHAPE;
  if (s->q_heads < 1 || s->kv_heads < 1 || (s->q_heads % s->kv_heads) != 0) return QSA_ERR_SHAPE;
  if (s->q_heads / s->kv_heads > 64) return QSA_ERR_SHAPE;
  if (s->batch > 65535 || s->n_query > (1 << 24) || s->q_heads > 65535) return QSA_ERR_SHAPE;
  if ((s->flags & ~7u) != 0 || (s->flags & (s->flags - 1u)) != 0) return QSA_ERR_SHAPE;
  d->B = s->batch;
  d->Lmax = s->max_len;
  d->Nq = s->n_query;
  d->Hq = s->q_heads;
  d->Hkv = s->kv_heads;
  d->scale = s->scale > 0.f ? s->scale : 1.0f / std::sqrt((float)QSA_HEAD_DIM);
  return QSA_OK;
}

// Opt-in synchronous validation of the device-side lens array.
qsa_status check_lens(const Dims& d, const int32_t* lens, hipStream_t stream) {
  const char* env = std::getenv("QSA_CHECK");
  if (!env || env[0] != '1' || d.B == 0) return QSA_OK;
  std::vector<int32_t> h(d.B);
  if (hipMemcpyAsync(h.data(), lens, sizeof(int32_t) * d.B, hipMemcpyDeviceToHost, stream) !=
      hipSuccess)
    return QSA_ERR_HIP;
  if (hipStreamSynchronize(stream) != hipSuccess) return QSA_ERR_HIP;
  for (int b = 0; b < d.B; ++b)
    if (h[b] < d.Nq || h[b] > d.Lmax) return QSA_ERR_SHAPE;
  return QSA_OK;
}

// Workspace of qsa_sparse_attend: partial outputs of split query rows.
struct AttendPtrs {
  float* part_o;
  float* part_lse;
};
size_t carve_attend_partials(const Dims& d, char* base, AttendPtrs* p) {
  qsa::Carve c{base, 0};
  const qsa::AttendLayout l = qsa::attend_layout(d);
  p->part_o = l.partial_floats ? c.take<float>(l.partial_floats) : nullptr;
  p->part_lse = l.lse_floats ? c.take<float>(l.lse_floats) : nullptr;
  return c.off;
}
size_t carve_attend(const Dims& d, void* ws, AttendPtrs* p) {
  return carve_attend_partials(d, static_cast<char*>(ws), p);
}

// Workspace of qsa_forward: selection, then one region shared by the top-k
// engine and (afterwards) the attention partials.
struct ForwardPtrs {
  int32_t* sel;
  int32_t* n_sel;
  AttendPtrs att;
  void* shared;
};
size_t carve_forward(const Dims& d, uint32_t flags, void* ws, ForwardPtrs* p) {
  qsa::Carve c{static_cast<char*>(ws), 0};
  const size_t rows = (size_t)d.B * d.Nq;
  p->sel = c.take<int32_t>(rows * QSA_TOPK);
  p->n_sel = c.take<int32_t>(rows);
  char* shared = c.take<char>(0);
  p->shared = shared;
  const size_t a = qsa::topk_workspace_bytes(d, qsa::choose_topk_path(d, flags));
  const size_t b = carve_attend_partials(d, shared, &p->att);
  c.off += a > b ? a : b;
  return c.off;
}

size_t ws_bytes_for(const Dims& d, uint32_t flags, int32_t op) {
  switch (op) {
    case QSA_OP_COMPRESS:
    case QSA_OP_EXPAND:
      return 0;
    case QSA_OP_INDEX_TOPK:
      return qsa::topk_workspace_bytes(d, qsa::choose_topk_path(d, flags));
    case QSA_OP_SPARSE_ATTEND: {
      AttendPtrs p;
      return carve_attend(d, nullptr, &p);
    }
    case QSA_OP_FORWARD: {
      ForwardPtrs p;
      return carve_forward(d, flags, nullptr, &p);
    }
    case QSA_OP_DENSE_DECODE:
      return qsa::dense_workspace_bytes(d);
    case QSA_OP_BLOCK_TEACHER:
      return qsa::teacher_workspace_bytes(d);
    default:
      return 0;
  }
}

qsa_status check_ws(const Dims& d, uint32_t flags, int32_t op, const void* ws, size_t ws_bytes) {
  const size_t need = ws_bytes_for(d, flags, op);
  if (need == 0) return QSA_OK;
  if (!ws || ws_bytes < need) return QSA_ERR_WORKSPACE;
  if (!aligned16(ws)) return QSA_ERR_ALIGN;
  return QSA_OK;
}

qsa_status hip_status(hipError_t e) { return e == hipSuccess ? QSA_OK : QSA_ERR_HIP; }

#define QSA_TRY(expr)            \
  do {                           \
    qsa_status st_ = (expr);     \
    if (st_ != QSA_OK) return st_; \
  } while (0)

qsa_status need(const void* p) {
  if (!p) return QSA_ERR_NULL;
  return aligned16(p) ? QSA_OK : QSA_ERR_ALIGN;
}

qsa_status need_i32(const void* p) {
  if (!p) return QSA_ERR_NULL;
  return (reinterpret_cast<uintptr_t>(p) & 3u) == 0 ? QSA_OK : QSA_ERR_ALIGN;
}

// Host-visible checks of a page descriptor; fills the kernels' form.
qsa_status check_paged(const Dims& d, const qsa_paged_kv* kv, qsa::Paged* pg) {
  if (!kv) return QSA_ERR_NULL;
  QSA_TRY(need_i32(kv->page_table));
  const int32_t ps = kv->page_size;
  if (ps < 1 || ps > (1 << 20) || (ps & (ps - 1)) != 0) return QSA_ERR_SHAPE;
  if (kv->max_pages < 1 || kv->n_pages < 1) return QSA_ERR_SHAPE;
  if ((int64_t)kv->max_pages * ps < d.Lmax) return QSA_ERR_SHAPE;
  if ((int64_t)kv->n_pages * ps > INT32_MAX) return QSA_ERR_SHAPE;  // pool rows are int32
  pg->page_table = kv->page_table;
  pg->page_shift = __builtin_ctz((unsigned)ps);
  pg->max_pages = kv->max_pages;
  pg->n_pages = kv->n_pages;
  return QSA_OK;
}

}  // namespace

namespace {
qsa_status forward_impl(const qsa_shape* shape, const uint16_t* q_idx, const uint16_t* k_idx,
                        uint16_t* k_cmp, const int32_t* first_block, const uint16_t* q,
                        const uint16_t* k, const uint16_t* v, const qsa_paged_kv* kv,
                        const int32_t* lens, uint16_t* out, float* lse, int32_t* sel_out,
                        int32_t* n_sel_out, void* ws, size_t ws_bytes, void* stream) {
  Dims d;
  QSA_TRY(check_shape(shape, &d));
  if (d.B == 0) return QSA_OK;
  qsa::Paged pg{};
  if (kv) QSA_TRY(check_paged(d, kv, &pg));
  QSA_TRY(need(q_idx));
  QSA_TRY(need(k_idx));
  QSA_TRY(need(k_cmp));
  if (first_block) QSA_TRY(need_i32(first_block));
  QSA_TRY(need(q));
  QSA_TRY(need(k));
  QSA_TRY(need(v));
  QSA_TRY(need_i32(lens));
  QSA_TRY(need(out));
  if (lse) QSA_TRY(need_i32(lse));
  if (sel_out) QSA_TRY(need(sel_out));
  if (n_sel_out) QSA_TRY(need_i32(n_sel_out));
  if ((sel_out == nullptr) != (n_sel_out == nullptr)) return QSA_ERR_NULL;
  QSA_TRY(check_ws(d, shape->flags, QSA_OP_FORWARD, ws, ws_bytes));
  QSA_TRY(check_device());
  hipStream_t s = static_cast<hipStream_t>(stream);
  QSA_TRY(check_lens(d, lens, s));
  ForwardPtrs p;
  carve_forward(d, shape->flags, ws, &p);
  int32_t* sel = sel_out ? sel_out : p.sel;
  int32_t* n_sel = sel_out ? n_sel_out : p.n_sel;
  const qsa::TopkPath path = qsa::choose_topk_path(d, shape->flags);
  // decode-shaped calls compress inside the scoring pass; others first
  const bool fuse = d.Nq > 0 && qsa::topk_can_fuse_compress(d, path);
  if (!fuse) QSA_TRY(hip_status(qsa::launch_compress(d, k_idx, lens, first_block, k_cmp, s)));
  if (d.Nq == 0) return QSA_OK;
  const qsa::CompressFuse cf{k_idx, first_block};
  QSA_TRY(hip_status(qsa::launch_index_topk(d, path, q_idx, k_cmp, lens, sel, n_sel, p.shared,
                                            s, fuse ? &cf : nullptr)));
  return hip_status(qsa::launch_sparse_attend(d, q, k, v, lens, sel, n_sel, out, lse, p.att.part_o,
                                              p.att.part_lse, s, kv ? &pg : nullptr));
}

qsa_status sparse_attend_impl(const qsa_shape* shape, const uint16_t* q, const uint16_t* k,
                              const uint16_t* v, const qsa_paged_kv* kv, const int32_t* lens,
                              const int32_t* sel, const int32_t* n_sel, uint16_t* out, float* lse,
                              void* ws, size_t ws_bytes, void* stream) {
  Dims d;
  QSA_TRY(check_shape(shape, &d));
  if (d.B == 0 || d.Nq == 0) return QSA_OK;
  qsa::Paged pg{};
  if (kv) QSA_TRY(check_paged(d, kv, &pg));
  QSA_TRY(need(q));
  QSA_TRY(need(k));
  QSA_TRY(need(v));
  QSA_TRY(need_i32(lens));
  QSA_TRY(need(sel));
  QSA_TRY(need_i32(n_sel));
  QSA_TRY(need(out));
  if (lse) QSA_TRY(need_i32(lse));
  QSA_TRY(check_ws(d, shape->flags, QSA_OP_SPARSE_ATTEND, ws, ws_bytes));
  QSA_TRY(check_device());
  hipStream_t s = static_cast<hipStream_t>(stream);
  QSA_TRY(check_lens(d, lens, s));
  AttendPtrs p;
  carve_attend(d, ws, &p);
  return hip_status(qsa::launch_sparse_attend(d, q, k, v, lens, sel, n_sel, out, lse, p.part_o,
                                              p.part_lse, s, kv ? &pg : nullptr));
}

qsa_status dense_decode_impl(const qsa_shape* shape, const uint16_t* q, const uint16_t* k,
                             const uint16_t* v, const qsa_paged_kv* kv, const int32_t* lens,
                             uint16_t* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
  Dims d;
  QSA_TRY(check_shape(shape, &d));
  if (d.B == 0 || d.Nq == 0) return QSA_OK;
  qsa::Paged pg{};
  if (kv) QSA_TRY(check_paged(d, kv, &pg));
  QSA_TRY(need(q));
  QSA_TRY(need(k));
  QSA_TRY(need(v));
  QSA_TRY(need_i32(lens));
  QSA_TRY(need(out));
  if (lse) QSA_TRY(need_i32(lse));
  QSA_TRY(check_ws(d, shape->flags, QSA_OP_DENSE_DECODE, ws, ws_bytes));
  QSA_TRY(check_device());
  hipStream_t s = static_cast<hipStream_t>(stream);
  QSA_TRY(check_lens(d, lens, s));
  return hip_status(qsa::launch_dense_decode(d, q, k, v, lens, out, lse, ws, s, kv ? &pg : nullptr));
}
}  // namespace

extern "C" {

qsa_status qsa_profile_attach(void** events, int32_t n_events) {
  if (!events || n_events < 2) return QSA_ERR_NULL;
  t_events = events;
  t_cap = n_events;
  t_count = 0;
  return QSA_OK;
}

int32_t qsa_profile_detach(void) {
  const int n = t_count;
  t_events = nullptr;
  t_cap = 0;
  return n;
}

int32_t qsa_debug_build(void) {
#ifdef QSA_DEBUG
  return 1;
#else
  return 0;
#endif
}

qsa_status qsa_debug_guard_hits(uint64_t* hits) {
  if (!hits) return QSA_ERR_NULL;
  *hits = 0;
#ifdef QSA_DEBUG
  QSA_TRY(check_device());
  if (hipDeviceSynchronize() != hipSuccess) return QSA_ERR_HIP;
  for (auto read_and_clear : qsa::guard_counters()) {
    unsigned int v = 0;
    if (read_and_clear(&v) != hipSuccess) return QSA_ERR_HIP;
    *hits += v;
  }
#endif
  return QSA_OK;
}

const char* qsa_profile_kernel_name(int32_t i) {
  if (i < 0 || i >= t_count || i >= kMaxProfiled) return "";
  return t_names[i];
}

size_t qsa_workspace_bytes(const qsa_shape* shape, int32_t op) {
  Dims d;
  if (check_shape(shape, &d) != QSA_OK) return 0;
  return ws_bytes_for(d, shape->flags, op);
}

const char* qsa_status_string(qsa_status status) {
  switch (status) {
    case QSA_OK:
      return "ok";
    case QSA_ERR_NULL:
      return "a required pointer is NULL";
    case QSA_ERR_ALIGN:
      return "a pointer is not 16-byte aligned";
    case QSA_ERR_SHAPE:
      return "unsupported or inconsistent shape";
    case QSA_ERR_WORKSPACE:
      return "workspace missing or too small";
    case QSA_ERR_DEVICE:
      return "current device is not an MI355X (gfx950)";
    case QSA_ERR_HIP:
      return "HIP runtime error";
    case QSA_ERR_SCRATCH:
      return "shape needs more scratch memory than qsa_forward_noalloc holds";
    default:
      return "unknown status";
  }
}

qsa_status qsa_compress_keys(const qsa_shape* shape, const uint16_t* k_idx, const int32_t* lens,
                             const int32_t* first_block, uint16_t* k_cmp, void* stream) {
  Dims d;
  QSA_TRY(check_shape(shape, &d));
  if (d.B == 0) return QSA_OK;
  QSA_TRY(need(k_idx));
  QSA_TRY(need_i32(lens));
  QSA_TRY(need(k_cmp));
  if (first_block) QSA_TRY(need_i32(first_block));
  QSA_TRY(check_device());
  hipStream_t s = static_cast<hipStream_t>(stream);
  QSA_TRY(check_lens(d, lens, s));
  return hip_status(
      qsa::launch_compress(d, k_idx, lens, first_block, k_cmp, s));
}

qsa_status qsa_index_topk(const qsa_shape* shape, const uint16_t* q_idx, const uint16_t* k_cmp,
                          const int32_t* lens, int32_t* sel, int32_t* n_sel, void* ws,
                          size_t ws_bytes, void* stream) {
  Dims d;
  QSA_TRY(check_shape(shape, &d));
  if (d.B == 0 || d.Nq == 0) return QSA_OK;
  QSA_TRY(need(q_idx));
  QSA_TRY(need(k_cmp));
  QSA_TRY(need_i32(lens));
  QSA_TRY(need(sel));
  QSA_TRY(need_i32(n_sel));
  QSA_TRY(check_ws(d, shape->flags, QSA_OP_INDEX_TOPK, ws, ws_bytes));
  QSA_TRY(check_device());
  hipStream_t s = static_cast<hipStream_t>(stream);
  QSA_TRY(check_lens(d, lens, s));
  // (no compression is fused here, so k_cmp is only read)
  return hip_status(qsa::launch_index_topk(d, qsa::choose_topk_path(d, shape->flags), q_idx,
                                           const_cast<uint16_t*>(k_cmp), lens, sel, n_sel, ws,
                                           s));
}

qsa_status qsa_expand_blocks(const qsa_shape* shape, const int32_t* lens, const int32_t* sel,
                             const int32_t* n_sel, int32_t* tok, int32_t* n_tok, void* stream) {
  Dims d;
  QSA_TRY(check_shape(shape, &d));
  if (d.B == 0 || d.Nq == 0) return QSA_OK;
  QSA_TRY(need_i32(lens));
  QSA_TRY(need(sel));
  QSA_TRY(need_i32(n_sel));
  QSA_TRY(need(tok));
  QSA_TRY(need_i32(n_tok));
  QSA_TRY(check_device());
  hipStream_t s = static_cast<hipStream_t>(stream);
  QSA_TRY(check_lens(d, lens, s));
  return hip_status(qsa::launch_expand(d, lens, sel, n_sel, tok, n_tok, s));
}

qsa_status qsa_sparse_attend(const qsa_shape* shape, const uint16_t* q, const uint16_t* k,
                             const uint16_t* v, const int32_t* lens, const int32_t* sel,
                             const int32_t* n_sel, uint16_t* out, float* lse, void* ws,
                             size_t ws_bytes, void* stream) {
  return sparse_attend_impl(shape, q, k, v, nullptr, lens, sel, n_sel, out, lse, ws, ws_bytes,
                            stream);
}

qsa_status qsa_forward(const qsa_shape* shape, const uint16_t* q_idx, const uint16_t* k_idx,
                       uint16_t* k_cmp, const int32_t* first_block, const uint16_t* q,
                       const uint16_t* k, const uint16_t* v, const int32_t* lens, uint16_t* out,
                       float* lse, int32_t* sel_out, int32_t* n_sel_out, void* ws,
                       size_t ws_bytes, void* stream) {
  return forward_impl(shape, q_idx, k_idx, k_cmp, first_block, q, k, v, nullptr, lens, out, lse,
                      sel_out, n_sel_out, ws, ws_bytes, stream);
}

qsa_status qsa_forward_paged(const qsa_shape* shape, const uint16_t* q_idx,
                             const uint16_t* k_idx, uint16_t* k_cmp, const int32_t* first_block,
                             const uint16_t* q, const uint16_t* k_pool, const uint16_t* v_pool,
                             const qsa_paged_kv* kv, const int32_t* lens, uint16_t* out,
                             float* lse, int32_t* sel_out, int32_t* n_sel_out, void* ws,
                             size_t ws_bytes, void* stream) {
  if (!kv) return QSA_ERR_NULL;
  return forward_impl(shape, q_idx, k_idx, k_cmp, first_block, q, k_pool, v_pool, kv, lens, out,
                      lse, sel_out, n_sel_out, ws, ws_bytes, stream);
}

qsa_status qsa_sparse_attend_paged(const qsa_shape* shape, const uint16_t* q,
                                   const uint16_t* k_pool, const uint16_t* v_pool,
                                   const qsa_paged_kv* kv, const int32_t* lens,
                                   const int32_t* sel, const int32_t* n_sel, uint16_t* out,
                                   float* lse, void* ws, size_t ws_bytes, void* stream) {
  if (!kv) return QSA_ERR_NULL;
  return sparse_attend_impl(shape, q, k_pool, v_pool, kv, lens, sel, n_sel, out, lse, ws,
                            ws_bytes, stream);
}

qsa_status qsa_dense_gqa_decode_paged(const qsa_shape* shape, const uint16_t* q,
                                      const uint16_t* k_pool, const uint16_t* v_pool,
                                      const qsa_paged_kv* kv, const int32_t* lens,
                                      uint16_t* out, float* lse, void* ws, size_t ws_bytes,
                                      void* stream) {
  if (!kv) return QSA_ERR_NULL;
  return dense_decode_impl(shape, q, k_pool, v_pool, kv, lens, out, lse, ws, ws_bytes, stream);
}

qsa_status qsa_dense_gqa_prefill(const qsa_shape* shape, const uint16_t* q, const uint16_t* k,
                                 const uint16_t* v, const qsa_paged_kv* kv, const int32_t* lens,
                                 uint16_t* out, float* lse, void* stream) {
  Dims d;
  QSA_TRY(check_shape(shape, &d));
  if (d.B == 0 || d.Nq == 0) return QSA_OK;
  qsa::Paged pg{};
  if (kv) QSA_TRY(check_paged(d, kv, &pg));
  QSA_TRY(need(q));
  QSA_TRY(need(k));
  QSA_TRY(need(v));
  QSA_TRY(need_i32(lens));
  QSA_TRY(need(out));
  if (lse) QSA_TRY(need_i32(lse));
  QSA_TRY(check_device());
  hipStream_t s = static_cast<hipStream_t>(stream);
  QSA_TRY(check_lens(d, lens, s));
  return hip_status(qsa::launch_dense_prefill(d, q, k, v, lens, out, lse, s, kv ? &pg : nullptr));
}

qsa_status qsa_dense_gqa_decode(const qsa_shape* shape, const uint16_t* q, const uint16_t* k,
                                const uint16_t* v, const int32_t* lens, uint16_t* out, float* lse,
                                void* ws, size_t ws_bytes, void* stream) {
  return dense_decode_impl(shape, q, k, v, nullptr, lens, out, lse, ws, ws_bytes, stream);
}

qsa_status qsa_block_teacher(const qsa_shape* shape, const uint16_t* q, const uint16_t* k,
                             const uint16_t* v, const int32_t* lens, float* teacher, void* ws,
                             size_t ws_bytes, void* stream) {
  Dims d;
  QSA_TRY(check_shape(shape, &d));
  if (d.B == 0 || d.Nq == 0) return QSA_OK;
  QSA_TRY(need(q));
  QSA_TRY(need(k));
  QSA_TRY(need(v));
  QSA_TRY(need_i32(lens));
  QSA_TRY(need(teacher));
  QSA_TRY(check_ws(d, shape->flags, QSA_OP_BLOCK_TEACHER, ws, ws_bytes));
  QSA_TRY(check_device());
  hipStream_t s = static_cast<hipStream_t>(stream);
  QSA_TRY(check_lens(d, lens, s));
  return hip_status(qsa::launch_block_teacher(d, q, k, v, lens, teacher, ws, s));
}

qsa_status qsa_teacher_recall(const qsa_shape* shape, const int32_t* lens, const float* teacher,
                              const int32_t* sel, const int32_t* n_sel, float* recall,
                              void* stream) {
  Dims d;
  QSA_TRY(check_shape(shape, &d));
  if (d.B == 0 || d.Nq == 0) return QSA_OK;
  QSA_TRY(need_i32(lens));
  QSA_TRY(need(teacher));
  QSA_TRY(need(sel));
  QSA_TRY(need_i32(n_sel));
  QSA_TRY(need_i32(recall));
  QSA_TRY(check_device());
  hipStream_t s = static_cast<hipStream_t>(stream);
  QSA_TRY(check_lens(d, lens, s));
  return hip_status(qsa::launch_teacher_recall(d, teacher, lens, sel, n_sel, recall, s));
}

qsa_status qsa_sparse_attend_backward(const qsa_shape* shape, const uint16_t* q,
                                      const uint16_t* k, const uint16_t* v, const int32_t* lens,
                                      const int32_t* sel, const int32_t* n_sel,
                                      const uint16_t* out, const float* lse,
                                      const uint16_t* d_out, float* dq, float* dk, float* dv,
                                      void* stream) {
  Dims d;
  QSA_TRY(check_shape(shape, &d));
  if (d.B == 0 || d.Nq == 0) return QSA_OK;
  QSA_TRY(need(q));
  QSA_TRY(need(k));
  QSA_TRY(need(v));
  QSA_TRY(need_i32(lens));
  QSA_TRY(need(sel));
  QSA_TRY(need_i32(n_sel));
  QSA_TRY(need(out));
  QSA_TRY(need_i32(lse));
  QSA_TRY(need(d_out));
  QSA_TRY(need(dq));
  QSA_TRY(need(dk));
  QSA_TRY(need(dv));
  QSA_TRY(check_device());
  hipStream_t s = static_cast<hipStream_t>(stream);
  QSA_TRY(check_lens(d, lens, s));
  return hip_status(
      qsa::launch_sparse_attend_bwd(d, q, k, v, lens, sel, n_sel, out, lse, d_out, dq, dk, dv, s));
}

qsa_status qsa_index_scores_backward(const qsa_shape* shape, const uint16_t* q_idx,
                                     const uint16_t* k_cmp, const int32_t* lens,
                                     const float* d_scores, float* dq_idx, float* dk_cmp,
                                     void* stream) {
  Dims d;
  QSA_TRY(check_shape(shape, &d));
  if (d.B == 0 || d.Nq == 0) return QSA_OK;
  QSA_TRY(need(q_idx));
  QSA_TRY(need(k_cmp));
  QSA_TRY(need_i32(lens));
  QSA_TRY(need(d_scores));
  QSA_TRY(need(dq_idx));
  QSA_TRY(need(dk_cmp));
  QSA_TRY(check_device());
  hipStream_t s = static_cast<hipStream_t>(stream);
  QSA_TRY(check_lens(d, lens, s));
  return hip_status(qsa::launch_index_scores_bwd(d, q_idx, k_cmp, lens, d_scores, dq_idx, dk_cmp, s));
}

qsa_status qsa_compress_keys_backward(const qsa_shape* shape, const int32_t* lens,
                                      const float* dk_cmp, float* dk_idx, void* stream) {
  Dims d;
  QSA_TRY(check_shape(shape, &d));
  if (d.B == 0) return QSA_OK;
  QSA_TRY(need_i32(lens));
  QSA_TRY(need(dk_cmp));
  QSA_TRY(need(dk_idx));
  QSA_TRY(check_device());
  hipStream_t s = static_cast<hipStream_t>(stream);
  QSA_TRY(check_lens(d, lens, s));
  return hip_status(qsa::launch_compress_bwd(d, dk_cmp, lens, dk_idx, s));
}

}  // extern "C"
