// C ABI of the local MoE expert layer: argument checks, workspace layout, and the
// ordered launches of the kernels on the caller's stream. Nothing here allocates,
// frees, synchronises or reads device memory.
#include <limits.h>

#include <atomic>
#include <mutex>

#include "../../include/moe.h"
#include "kernels.h"

using namespace moe;

namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
inline size_t elem_size(moe_dtype dt) { return dt == MOE_BF16 ? 2 : 4; }

bool meta_ok(const moe_metadata *m) {
  if (!m) return false;
  if (m->N < 0 || m->K < 1 || m->K > MOE_MAX_TOPK || m->E < 1 || m->E > MOE_MAX_EXPERTS)
    return false;
  const int64_t NK = (int64_t)m->N * m->K;
  if (NK >= INT32_MAX) return false;
  if (m->capacity < 0) return false;
  if (!m->expert_frequency || !m->expert_frequency_offset ||
      !m->num_activated_expert_per_token_offset || !m->status)
    return false;
  if (m->capacity > 0 &&
      (!m->x_gather_idx || !m->s_scatter_idx || !m->s_reverse_scatter_idx || !m->router_scores))
    return false;
  if ((int64_t)meta_blocks(NK) * (m->E + 1) >= INT32_MAX) return false;
  return true;
}

// H and I in whole 16-byte bf16 chunks; the GEMM tiles at their edges may be partial
bool dims_ok(int32_t H, int32_t I) {
  return H > 0 && I > 0 && H % 8 == 0 && I % 8 == 0 && H <= (1 << 20) && I <= (1 << 20);
}

struct FwdWs {
  size_t a, y, total;
};
FwdWs fwd_layout(const moe_metadata *m, int32_t H, int32_t I, moe_dtype dt) {
  const size_t es = elem_size(dt), cap = (size_t)m->capacity;
  FwdWs w;
  w.a = 0;
  w.y = align_up(cap * I * es);
  w.total = w.y + align_up(cap * H * es);
  return w;
}
struct BwdWs {
  size_t dh, aw, dxg, partial, total;
};
BwdWs bwd_layout(const moe_metadata *m, int32_t H, int32_t I, moe_dtype dt) {
  const size_t es = elem_size(dt), cap = (size_t)m->capacity;
  BwdWs w;
  w.dh = 0;
  w.aw = w.dh + align_up(cap * 2 * I * es);
  w.dxg = w.aw + align_up(cap * I * es);
  w.partial = w.dxg + align_up(cap * H * es);
  w.total = w.partial + align_up(cap * (size_t)((I + kGemmBN - 1) / kGemmBN) * sizeof(float));
  return w;
}

// ---- diagnostics: events around the launches of one kernel. The hook belongs to the
// host thread that armed it (thread-local): launches made by other threads never read
// or advance it, so arming it in one thread cannot race with another thread's calls.
struct TimingHook {
  int kernel = -1;
  hipEvent_t const *events = nullptr;
  int n = 0, i = 0;
};
thread_local TimingHook g_hook;

struct Bracket {  // records the start event on construction, the end event on destruction
  hipStream_t st;
  bool on;
  int slot;
  Bracket(moe_kernel_id k, hipStream_t s) : st(s), on(false), slot(0) {
    if (g_hook.events && g_hook.kernel == (int)k && g_hook.i < g_hook.n) {
      on = true;
      slot = g_hook.i++;
      (void)hipEventRecord(g_hook.events[2 * slot], st);
    }
  }
  ~Bracket() {
    if (on) (void)hipEventRecord(g_hook.events[2 * slot + 1], st);
  }
};

GemmArgs base_args(const moe_metadata *m) {
  GemmArgs g = {};
  g.foff = m->expert_frequency_offset;
  g.E = m->E;
  g.cap = m->capacity;
  return g;
}

moe_status gemm(GemmKind kind, moe_kernel_id id, const GemmArgs &g, moe_dtype dt,
                hipStream_t st) {
  if ((dt == MOE_BF16 ? gemm_grid(kind, g) : gemm_grid_f32(kind, g)) < 0) return MOE_EUNSUPPORTED;
  Bracket b(id, st);
  hipError_t err = dt == MOE_BF16 ? launch_gemm_bf16(kind, g, st) : launch_gemm_f32(kind, g, st);
  return err == hipSuccess ? MOE_OK : MOE_EHIP;
}

// ---- the library-owned scratch of the allocation-free metadata build. A file-scope
// device array: each GPU the library runs on holds its own copy, at its own address,
// until the process ends. In host code `scratch` is only a stand-in for the symbol;
// the device address of the current GPU's copy is looked up once per device
// (hipGetSymbolAddress, with that device current) and kept, and only that address is
// ever passed to kernels.
constexpr int kMaxDevices = 64;
static __device__ __align__(256) int32_t scratch[MOE_NOALLOC_SCRATCH_BYTES / sizeof(int32_t)];
std::atomic<int32_t *> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

int32_t *scratch_of_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  int32_t *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (!p) {
    void *addr = nullptr;
    if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || !addr) return nullptr;
    p = (int32_t *)addr;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace

namespace moe {
static MetaOut meta_out(const moe_metadata *meta) {
  MetaOut o;
  o.expert_frequency = meta->expert_frequency;
  o.expert_frequency_offset = meta->expert_frequency_offset;
  o.x_gather_idx = meta->x_gather_idx;
  o.s_scatter_idx = meta->s_scatter_idx;
  o.s_reverse_scatter_idx = meta->s_reverse_scatter_idx;
  o.tok_off = meta->num_activated_expert_per_token_offset;
  o.router_scores = meta->router_scores;
  o.status = meta->status;
  return o;
}
}  // namespace moe

namespace {
// The metadata launches (one to three) over an argument-checked metadata object and a
// workspace of at least meta_workspace_bytes(N*K, E) bytes. None of the workspace needs
// to start zeroed: every cell the kernels read was written earlier in the same build
// (the one-launch build reads none).
moe_status enqueue_metadata(const int32_t *topk_idx, const float *topk_weights,
                            const moe_metadata *meta, int32_t *ws, hipStream_t st) {
  const MetaOut o = meta_out(meta);
  const int64_t NK = (int64_t)meta->N * meta->K;
  // up to 2048 slots: one workgroup builds everything (one launch); few chunks and
  // experts: the scatter pass sums the chunk counts itself (two launches); else three
  const int mode = meta_solo(NK) ? kMetaSolo : meta_fused_scan(NK, meta->E) ? kMetaFused
                                                                           : kMetaScanned;
  hipError_t err = hipSuccess;
  if (mode != kMetaSolo) {
    Bracket b(MOE_KERNEL_META_HIST, st);
    err = launch_meta_hist(topk_idx, meta->N, meta->K, meta->E, ws, st);
  }
  if (err != hipSuccess) return MOE_EHIP;
  if (mode == kMetaScanned) {
    Bracket b(MOE_KERNEL_META_SCAN, st);
    err = launch_meta_scan(meta->N, meta->K, meta->E, ws, st);
  }
  if (err != hipSuccess) return MOE_EHIP;
  Bracket b(MOE_KERNEL_META_SCATTER, st);
  err = launch_meta_scatter(topk_idx, topk_weights, meta->N, meta->K, meta->E, meta->capacity,
                            ws, o, st, mode);
  return err == hipSuccess ? MOE_OK : MOE_EHIP;
}
}  // namespace

extern "C" {

size_t moe_build_metadata_workspace(int32_t N, int32_t K, int32_t E) {
  if (N < 0 || K < 1 || E < 1) return 0;
  return meta_workspace_bytes((int64_t)N * K, E);
}

size_t moe_expert_forward_workspace(const moe_metadata *meta, int32_t H, int32_t I,
                                    moe_dtype dt) {
  if (!meta || H <= 0 || I <= 0 || meta->capacity < 0) return 0;
  return fwd_layout(meta, H, I, dt).total;
}

size_t moe_expert_backward_workspace(const moe_metadata *meta, int32_t H, int32_t I,
                                     moe_dtype dt) {
  if (!meta || H <= 0 || I <= 0 || meta->capacity < 0) return 0;
  return bwd_layout(meta, H, I, dt).total;
}

moe_status moe_build_metadata(const int32_t *topk_idx, const float *topk_weights,
                              const moe_metadata *meta, void *workspace, size_t workspace_bytes,
                              void *stream) {
  if (!meta_ok(meta)) return MOE_EINVAL;
  const int64_t NK = (int64_t)meta->N * meta->K;
  if (NK > 0 && (!topk_idx || !topk_weights)) return MOE_EINVAL;
  const size_t need = meta_workspace_bytes(NK, meta->E);
  if (workspace_bytes < need || !workspace) return MOE_ENOSPC;
  return enqueue_metadata(topk_idx, topk_weights, meta, (int32_t *)workspace,
                          (hipStream_t)stream);
}

moe_status moe_build_metadata_noalloc(const int32_t *topk_idx, const float *topk_weights,
                                      const moe_metadata *meta, void *stream) {
  if (!meta_ok(meta)) return MOE_EINVAL;
  const int64_t NK = (int64_t)meta->N * meta->K;
  if (NK > 0 && (!topk_idx || !topk_weights)) return MOE_EINVAL;
  if (meta_workspace_bytes(NK, meta->E) > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ENOSPC;
  int32_t *ws = scratch_of_current_device();
  if (!ws) return MOE_EHIP;
  return enqueue_metadata(topk_idx, topk_weights, meta, ws, (hipStream_t)stream);
}

size_t moe_route_workspace(int32_t N, int32_t K, int32_t E) {
  if (N < 0 || K < 1 || E < 1) return 0;
  const int64_t NK = (int64_t)N * K;
  return align_up(meta_workspace_bytes(NK, E)) + route_ws_floats(NK, E) * sizeof(float);
}

moe_status moe_route(const void *logits, moe_dtype logits_dtype, moe_route_mode mode,
                     int32_t renormalize, int32_t *topk_idx, float *topk_weights,
                     float *aux_loss, const moe_metadata *meta, void *workspace,
                     size_t workspace_bytes, void *stream) {
  if (!meta_ok(meta)) return MOE_EINVAL;
  if (logits_dtype != MOE_BF16 && logits_dtype != MOE_FP32) return MOE_EUNSUPPORTED;
  if (mode != MOE_ROUTE_SOFTMAX_TOPK && mode != MOE_ROUTE_TOPK_SOFTMAX) return MOE_EUNSUPPORTED;
  if (meta->K > meta->E) return MOE_EINVAL;
  const int N = meta->N, K = meta->K, E = meta->E;
  const int64_t NK = (int64_t)N * K;
  if (NK > 0 && (!logits || !topk_idx || !topk_weights)) return MOE_EINVAL;
  const size_t need = moe_route_workspace(N, K, E);
  if (workspace_bytes < need || !workspace) return MOE_ENOSPC;
  int32_t *mws = (int32_t *)workspace;
  float *ppart = (float *)((char *)workspace + align_up(meta_workspace_bytes(NK, E)));
  float *psum = ppart + (size_t)meta_blocks(NK) * E;  // [E] after the [E][nblk] columns
  MetaOut o = meta_out(meta);
  const bool want_p = aux_loss != nullptr && N > 0;
  if (aux_loss) {
    o.aux = aux_loss;
    o.psum = want_p ? psum : nullptr;  // N = 0: the loss is 0
    o.aux_scale = want_p ? (float)((double)E / ((double)N * (double)K * (double)N)) : 0.0f;
  }
  hipStream_t st = (hipStream_t)stream;
  hipError_t err;
  {
    Bracket b(MOE_KERNEL_ROUTE, st);
    err = N > 0 ? launch_route_hist(logits, logits_dtype == MOE_BF16, N, E, K, (int)mode,
                                    renormalize != 0, want_p, topk_idx, topk_weights, mws,
                                    ppart, st)
                : launch_meta_hist(topk_idx, N, K, E, mws, st);  // empty histogram
  }
  if (err != hipSuccess) return MOE_EHIP;
  {
    Bracket b(MOE_KERNEL_META_SCAN, st);
    err = launch_meta_scan(N, K, E, mws, st, want_p ? ppart : nullptr, psum);
  }
  if (err != hipSuccess) return MOE_EHIP;
  Bracket b(MOE_KERNEL_META_SCATTER, st);
  err = launch_meta_scatter(topk_idx, topk_weights, N, K, E, meta->capacity, mws, o, st);
  return err == hipSuccess ? MOE_OK : MOE_EHIP;
}

moe_status moe_expert_forward(const moe_metadata *meta, const void *x, const void *w_up,
                              const void *w_down, int32_t H, int32_t I, moe_dtype dt,
                              moe_gateup_layout layout, void *h_save, void *out,
                              void *workspace, size_t workspace_bytes, void *stream) {
  if (!meta_ok(meta)) return MOE_EINVAL;
  if (dt != MOE_BF16 && dt != MOE_FP32) return MOE_EUNSUPPORTED;
  if (layout != MOE_GATEUP_INTERLEAVED && layout != MOE_GATEUP_CONCAT) return MOE_EUNSUPPORTED;
  if (!dims_ok(H, I)) return MOE_EUNSUPPORTED;
  if (meta->N > 0 && (!x || !w_up || !w_down || !out)) return MOE_EINVAL;
  const FwdWs L = fwd_layout(meta, H, I, dt);
  if (workspace_bytes < L.total || (L.total > 0 && !workspace)) return MOE_ENOSPC;
  if (meta->N == 0) return MOE_OK;
  hipStream_t st = (hipStream_t)stream;
  char *ws = (char *)workspace;
  void *a = ws + L.a, *y = ws + L.y;

  GemmArgs g = base_args(meta);
  // h = x_g W_up, a = SwiGLU(h)
  g.N = 2 * I;
  g.K = H;
  g.A = x;
  g.lda = H;
  g.a_rows = meta->x_gather_idx;
  g.B = w_up;
  g.ldb = 2 * I;
  g.b_es = (int64_t)H * 2 * I;
  g.C = h_save;
  g.ldc = 2 * I;
  g.C2 = a;
  g.ldc2 = I;
  g.gu_concat = layout == MOE_GATEUP_CONCAT;
  moe_status s = gemm(kUpSwiGLU, MOE_KERNEL_UP_SWIGLU, g, dt, st);
  if (s != MOE_OK) return s;
  // y = a W_down
  g = base_args(meta);
  g.N = H;
  g.K = I;
  g.A = a;
  g.lda = I;
  g.B = w_down;
  g.ldb = H;
  g.b_es = (int64_t)I * H;
  g.C = y;
  g.ldc = H;
  s = gemm(kDown, MOE_KERNEL_DOWN, g, dt, st);
  if (s != MOE_OK) return s;
  // out = sum_q w_q y[s_rev[q]]
  Bracket b(MOE_KERNEL_COMBINE, st);
  hipError_t err = launch_combine(dt == MOE_BF16, y, meta->num_activated_expert_per_token_offset,
                                  meta->s_reverse_scatter_idx, meta->router_scores, meta->N, H,
                                  meta->capacity, out, st);
  return err == hipSuccess ? MOE_OK : MOE_EHIP;
}

moe_status moe_expert_backward(const moe_metadata *meta, const int32_t *topk_idx,
                               const void *x, const void *w_up, const void *w_down,
                               const void *h_saved, const void *dout, int32_t H, int32_t I,
                               moe_dtype dt, moe_gateup_layout layout, void *dx, void *dw_up,
                               void *dw_down, float *d_topk_weights, void *workspace,
                               size_t workspace_bytes, void *stream) {
  if (!meta_ok(meta)) return MOE_EINVAL;
  if (dt != MOE_BF16 && dt != MOE_FP32) return MOE_EUNSUPPORTED;
  if (layout != MOE_GATEUP_INTERLEAVED && layout != MOE_GATEUP_CONCAT) return MOE_EUNSUPPORTED;
  if (!dims_ok(H, I)) return MOE_EUNSUPPORTED;
  if (!w_up || !w_down || !dw_up || !dw_down) return MOE_EINVAL;
  if (meta->N > 0 && (!topk_idx || !x || !dout || !dx || !d_topk_weights)) return MOE_EINVAL;
  if (meta->capacity > 0 && !h_saved) return MOE_EINVAL;
  const BwdWs L = bwd_layout(meta, H, I, dt);
  if (workspace_bytes < L.total || (L.total > 0 && !workspace)) return MOE_ENOSPC;
  hipStream_t st = (hipStream_t)stream;
  char *ws = (char *)workspace;
  void *dh = ws + L.dh, *aw = ws + L.aw, *dxg = ws + L.dxg;
  float *partial = (float *)(ws + L.partial);

  // da_u = dout_g W_down^T; epilogue: dh, w*a, per-tile dscore partials
  GemmArgs g = base_args(meta);
  g.N = I;
  g.K = H;
  g.A = dout;
  g.lda = H;
  g.a_rows = meta->x_gather_idx;
  g.B = w_down;
  g.ldb = H;
  g.b_es = (int64_t)I * H;
  g.C = dh;
  g.ldc = 2 * I;
  g.C2 = aw;
  g.ldc2 = I;
  g.Hs = h_saved;
  g.ldh = 2 * I;
  g.scores = meta->router_scores;
  g.s_scatter = meta->s_scatter_idx;
  g.partial = partial;
  g.gu_concat = layout == MOE_GATEUP_CONCAT;  // dh takes W_up's column order
  if (dt == MOE_BF16) {  // one dscore partial per column tile of this GEMM
    int bm, bn, bk;
    gemm_tile(kDownBwd, g, &bm, &bn, &bk);
    g.n_ntiles = (I + bn - 1) / bn;
  } else {
    g.n_ntiles = (I + kGemmBN - 1) / kGemmBN;
  }
  const int nnt = g.n_ntiles;
  moe_status s = MOE_OK;
  if (meta->N > 0 && (s = gemm(kDownBwd, MOE_KERNEL_DOWN_BWD, g, dt, st)) != MOE_OK) return s;
  // dW_down[e] = (w a)^T dout_g over the expert's rows
  g = base_args(meta);
  g.M = I;
  g.N = H;
  g.A = aw;
  g.lda = I;
  g.B = dout;
  g.ldb = H;
  g.b_rows = meta->x_gather_idx;
  g.C = dw_down;
  g.ldc = H;
  g.c_es = (int64_t)I * H;
  if ((s = gemm(kWeightGrad, MOE_KERNEL_WGRAD_DOWN, g, dt, st)) != MOE_OK) return s;
  // dxg = dh W_up^T
  g = base_args(meta);
  g.N = H;
  g.K = 2 * I;
  g.A = dh;
  g.lda = 2 * I;
  g.B = w_up;
  g.ldb = 2 * I;
  g.b_es = (int64_t)H * 2 * I;
  g.C = dxg;
  g.ldc = H;
  if (meta->N > 0 && (s = gemm(kUpBwd, MOE_KERNEL_UP_BWD, g, dt, st)) != MOE_OK) return s;
  // dW_up[e] = x_g^T dh over the expert's rows
  g = base_args(meta);
  g.M = H;
  g.N = 2 * I;
  g.A = x;
  g.lda = H;
  g.a_rows = meta->x_gather_idx;
  g.B = dh;
  g.ldb = 2 * I;
  g.C = dw_up;
  g.ldc = 2 * I;
  g.c_es = (int64_t)H * 2 * I;
  if ((s = gemm(kWeightGrad, MOE_KERNEL_WGRAD_UP, g, dt, st)) != MOE_OK) return s;
  if (meta->N == 0) return MOE_OK;
  // dx = sum_q dxg[s_rev[q]], and d_topk_weights from the partials
  Bracket b(MOE_KERNEL_COMBINE_DX, st);
  hipError_t err = launch_combine_dscore(
      dt == MOE_BF16, dxg, meta->num_activated_expert_per_token_offset,
      meta->s_reverse_scatter_idx, meta->N, H, meta->capacity, dx, topk_idx, meta->K, meta->E,
      partial, nnt, d_topk_weights, st);
  return err == hipSuccess ? MOE_OK : MOE_EHIP;
}

moe_status moe_time_kernel(moe_kernel_id kernel, void *const *events, int32_t n_launches,
                           int32_t *n_recorded) {
  if (n_recorded) *n_recorded = g_hook.i;
  if (events && ((int)kernel < 0 || (int)kernel >= MOE_KERNEL_COUNT || n_launches < 0))
    return MOE_EINVAL;
  for (int i = 0; events && i < 2 * n_launches; i++)
    if (!events[i]) return MOE_EINVAL;
  g_hook.kernel = (int)kernel;
  g_hook.events = (hipEvent_t const *)events;
  g_hook.n = events ? n_launches : 0;
  g_hook.i = 0;
  return MOE_OK;
}

const char *moe_kernel_name(moe_kernel_id k) {
  static const char *names[MOE_KERNEL_COUNT] = {
      "meta_hist", "meta_scan", "meta_scatter", "up_swiglu", "down", "combine", "down_bwd",
      "wgrad_down", "up_bwd", "wgrad_up", "combine_dx", "route"};
  return ((int)k >= 0 && (int)k < MOE_KERNEL_COUNT) ? names[(int)k] : "unknown";
}

const char *moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument";
    case MOE_ENOSPC: return "workspace too small";
    case MOE_EUNSUPPORTED: return "unsupported shape, dtype or layout";
    case MOE_EHIP: return "HIP launch failed";
  }
  return "unknown status";
}

}  // extern "C"
