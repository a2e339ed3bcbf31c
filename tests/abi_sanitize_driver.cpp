// Host-side check of the C ABI layer (csrc/api.hip, csrc/schedule.hip) on the CPU,
// built with AddressSanitizer and UndefinedBehaviorSanitizer against stub launchers.
//
// Every "device" buffer is a host allocation of exactly the size include/moe.h
// documents (workspaces: exactly what the *_workspace queries return). The stub
// launchers read or write every element of every extent the ABI hands them, derived
// from the launch arguments the way the kernels use them, so a wrong workspace layout,
// a short query or an extent computed from the wrong size is an out-of-bounds access
// the sanitizer reports. Argument errors, edge shapes and the size arithmetic at the
// limits (1024 experts, 64 slots, N*K near 2^31, H = I = 2^20) run through the same
// build. `plant` makes one stub write one element past an output, which the test
// expects the sanitizer to catch.
#include <hip/hip_runtime.h>

#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "../token_routing_grouped_amd/csrc/kernels.h"
#include "moe.h"

static bool g_dry = false;    // stubs touch nothing (size arithmetic at huge shapes)
static bool g_plant = false;  // the combine stub writes one element too many
static int g_launches = 0;
static int g_checks = 0;

hipError_t hipGetDevice(int *d) {
  *d = 0;
  return hipSuccess;
}
hipError_t hipGetSymbolAddress(void **p, const void *sym) {
  *p = (void *)sym;
  return hipSuccess;
}
hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipSuccess; }

static volatile unsigned char g_sink;
static void rd(const void *p, size_t bytes) {
  if (g_dry || bytes == 0) return;
  if (!p) {
    fprintf(stderr, "read of %zu bytes through a null pointer\n", bytes);
    abort();
  }
  const unsigned char *c = (const unsigned char *)p;
  unsigned char s = 0;
  for (size_t i = 0; i < bytes; i++) s ^= c[i];
  g_sink = s;
}
static void wr(void *p, size_t bytes) {
  if (g_dry || bytes == 0) return;
  if (!p) {
    fprintf(stderr, "write of %zu bytes through a null pointer\n", bytes);
    abort();
  }
  memset(p, 0x5a, bytes);
}

namespace moe {

hipError_t launch_meta_hist(const int32_t *topk_idx, int N, int K, int E, int32_t *ws,
                            hipStream_t) {
  g_launches++;
  const int64_t NK = (int64_t)N * K;
  const MetaWs L = meta_ws_layout(NK, E);
  rd(topk_idx, (size_t)NK * 4);
  wr(ws + L.hist, (size_t)(E + 2) * L.nblk * 4);
  return hipSuccess;
}

hipError_t launch_meta_scan(int N, int K, int E, int32_t *ws, hipStream_t, const float *fcol,
                            float *fsum) {
  g_launches++;
  const MetaWs L = meta_ws_layout((int64_t)N * K, E);
  rd(ws + L.hist, (size_t)(E + 2) * L.nblk * 4);
  wr(ws + L.pre, (size_t)(E + 2) * L.nblk * 4);
  wr(ws + L.tot, (size_t)(E + 2) * 4);
  if (L.nseg > 1) wr(ws + L.seg, (size_t)(2 * E + 2) * L.nseg * 4);
  if (fcol) {
    rd(fcol, (size_t)E * L.nblk * 4);
    wr(fsum, (size_t)E * 4);
  }
  return hipSuccess;
}

bool meta_fused_scan(int64_t NK, int E) {  // same rules as the library's
  return meta_items(NK) == 2 && E + 2 <= 36 && meta_blocks(NK) <= 256;
}
bool meta_solo(int64_t NK) { return NK <= kMetaSoloSlots; }

hipError_t launch_meta_scatter(const int32_t *topk_idx, const float *topk_weights, int N, int K,
                               int E, int capacity, const int32_t *ws, const MetaOut &o,
                               hipStream_t, int mode) {
  g_launches++;
  const int64_t NK = (int64_t)N * K;
  const MetaWs L = meta_ws_layout(NK, E);
  rd(topk_idx, (size_t)NK * 4);
  rd(topk_weights, (size_t)NK * 4);
  if (mode == kMetaSolo) {  // reads no workspace
    if (!meta_solo(NK) || o.aux) return hipErrorInvalidValue;
  } else if (mode == kMetaFused) {
    if (!meta_fused_scan(NK, E) || o.aux) return hipErrorInvalidValue;
    rd(ws + L.hist, (size_t)(E + 2) * L.nblk * 4);
  } else {
    rd(ws + L.pre, (size_t)(E + 2) * L.nblk * 4);
    rd(ws + L.tot, (size_t)(E + 2) * 4);
  }
  wr(o.expert_frequency, (size_t)E * 4);
  wr(o.expert_frequency_offset, (size_t)(E + 1) * 4);
  wr(o.tok_off, (size_t)(N + 1) * 4);
  wr(o.status, 4);
  const size_t c = (size_t)capacity * 4;
  wr(o.x_gather_idx, c);
  wr(o.s_scatter_idx, c);
  wr(o.s_reverse_scatter_idx, c);
  wr(o.router_scores, c);
  if (o.aux) wr(o.aux, 4);
  if (o.psum) rd(o.psum, (size_t)E * 4);
  return hipSuccess;
}

hipError_t launch_route_hist(const void *logits, bool bf16, int N, int E, int K, int, int,
                             bool want_p, int32_t *topk_idx, float *topk_w, int32_t *meta_ws,
                             float *ppart, hipStream_t) {
  g_launches++;
  const int64_t NK = (int64_t)N * K;
  const MetaWs L = meta_ws_layout(NK, E);
  rd(logits, (size_t)N * E * (bf16 ? 2 : 4));
  wr(topk_idx, (size_t)NK * 4);
  wr(topk_w, (size_t)NK * 4);
  wr(meta_ws + L.hist, (size_t)(E + 2) * L.nblk * 4);
  if (want_p) wr(ppart, (size_t)E * L.nblk * 4);
  return hipSuccess;
}

static hipError_t gemm_touch(GemmKind kind, const GemmArgs &g, size_t es) {
  g_launches++;
  const size_t cap = (size_t)g.cap;
  rd(g.foff, (size_t)(g.E + 1) * 4);
  switch (kind) {
    case kUpSwiGLU:  // A = x gathered (caller tensor), B = W_up, C = h_save or null, C2 = a
      rd(g.a_rows, cap * 4);
      rd(g.B, (size_t)g.E * g.b_es * es);
      if (g.C) wr(g.C, cap * g.ldc * es);
      wr(g.C2, cap * g.ldc2 * es);
      break;
    case kDown:  // A = a, B = W_down, C = y
      rd(g.A, cap * g.lda * es);
      rd(g.B, (size_t)g.E * g.b_es * es);
      wr(g.C, cap * g.ldc * es);
      break;
    case kDownBwd:  // A = dout gathered, B = W_down, C = dh, C2 = w*a, Hs = h, partials
      rd(g.a_rows, cap * 4);
      rd(g.B, (size_t)g.E * g.b_es * es);
      rd(g.Hs, cap * g.ldh * es);
      rd(g.scores, cap * 4);
      rd(g.s_scatter, cap * 4);
      wr(g.C, cap * g.ldc * es);
      wr(g.C2, cap * g.ldc2 * es);
      wr(g.partial, cap * (size_t)g.n_ntiles * 4);
      break;
    case kUpBwd:  // A = dh, B = W_up, C = dxg
      rd(g.A, cap * g.lda * es);
      rd(g.B, (size_t)g.E * g.b_es * es);
      wr(g.C, cap * g.ldc * es);
      break;
    case kWeightGrad:  // one operand gathered through a row map, the other by position
      if (g.a_rows) rd(g.a_rows, cap * 4); else rd(g.A, cap * g.lda * es);
      if (g.b_rows) rd(g.b_rows, cap * 4); else rd(g.B, cap * g.ldb * es);
      wr(g.C, (size_t)g.E * g.c_es * es);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipSuccess;
}
hipError_t launch_gemm_bf16(GemmKind kind, const GemmArgs &g, hipStream_t) {
  if (gemm_grid(kind, g) < 0) return hipErrorInvalidValue;
  return gemm_touch(kind, g, 2);
}
hipError_t launch_gemm_f32(GemmKind kind, const GemmArgs &g, hipStream_t) {
  if (gemm_grid_f32(kind, g) < 0) return hipErrorInvalidValue;
  return gemm_touch(kind, g, 4);
}

hipError_t launch_combine(bool bf16, const void *y, const int32_t *tok_off, const int32_t *s_rev,
                          const float *scores, int N, int H, int cap, void *out, hipStream_t) {
  g_launches++;
  const size_t es = bf16 ? 2 : 4;
  rd(y, (size_t)cap * H * es);
  rd(tok_off, (size_t)(N + 1) * 4);
  rd(s_rev, (size_t)cap * 4);
  if (scores) rd(scores, (size_t)cap * 4);
  wr(out, (size_t)N * H * es + (g_plant ? es : 0));
  return hipSuccess;
}

hipError_t launch_combine_dscore(bool bf16, const void *dxg, const int32_t *tok_off,
                                 const int32_t *s_rev, int N, int H, int cap, void *dx,
                                 const int32_t *topk_idx, int K, int, const float *partial,
                                 int n_ntiles, float *dtw, hipStream_t s) {
  launch_combine(bf16, dxg, tok_off, s_rev, nullptr, N, H, cap, dx, s);
  rd(topk_idx, (size_t)N * K * 4);
  rd(partial, (size_t)cap * n_ntiles * 4);
  wr(dtw, (size_t)N * K * 4);
  return hipSuccess;
}

}  // namespace moe

// ---- cases -----------------------------------------------------------------

#define EXPECT(call, want)                                                              \
  do {                                                                                  \
    const int got_ = (int)(call);                                                       \
    g_checks++;                                                                         \
    if (got_ != (int)(want)) {                                                          \
      fprintf(stderr, "%s:%d: %s returned %d, expected %d\n", __FILE__, __LINE__, #call, \
              got_, (int)(want));                                                       \
      exit(3);                                                                          \
    }                                                                                   \
  } while (0)

struct Buf {  // one exactly sized host allocation standing for a device buffer
  std::vector<unsigned char> *v = nullptr;
  void *p = nullptr;
  explicit Buf(size_t bytes) {
    if (bytes) {
      v = new std::vector<unsigned char>(bytes);
      p = v->data();
    }
  }
  ~Buf() { delete v; }
  Buf(const Buf &) = delete;
  Buf &operator=(const Buf &) = delete;
};

struct Meta {  // metadata arrays at their documented sizes
  Buf freq, foff, xg, ss, sr, toff, rs, st;
  moe_metadata m;
  Meta(int N, int K, int E, int cap)
      : freq((size_t)E * 4), foff((size_t)(E + 1) * 4), xg((size_t)cap * 4),
        ss((size_t)cap * 4), sr((size_t)cap * 4), toff((size_t)(N + 1) * 4),
        rs((size_t)cap * 4), st(4) {
    m = {N, K, E, cap, (int32_t *)freq.p, (int32_t *)foff.p, (int32_t *)xg.p,
         (int32_t *)ss.p, (int32_t *)sr.p, (int32_t *)toff.p, (float *)rs.p,
         (uint32_t *)st.p};
  }
};

// metadata, router, forward (with and without h_save), backward, allocation-free build
static void full_case(int N, int K, int E, int cap, int H, int I, moe_dtype dt,
                      moe_gateup_layout lay) {
  Meta M(N, K, E, cap);
  const size_t es = dt == MOE_BF16 ? 2 : 4;
  Buf idx((size_t)N * K * 4), w((size_t)N * K * 4);
  Buf mws(moe_build_metadata_workspace(N, K, E));
  EXPECT(moe_build_metadata((int32_t *)idx.p, (float *)w.p, &M.m, mws.p,
                            moe_build_metadata_workspace(N, K, E), nullptr),
         MOE_OK);
  if (moe_build_metadata_workspace(N, K, E) <= (size_t)MOE_NOALLOC_SCRATCH_BYTES)
    EXPECT(moe_build_metadata_noalloc((int32_t *)idx.p, (float *)w.p, &M.m, nullptr), MOE_OK);
  if (K <= E) {
    Buf logits((size_t)N * E * es), aux(4);
    Buf rws(moe_route_workspace(N, K, E));
    EXPECT(moe_route(logits.p, dt, MOE_ROUTE_TOPK_SOFTMAX, 1, (int32_t *)idx.p, (float *)w.p,
                     (float *)aux.p, &M.m, rws.p, moe_route_workspace(N, K, E), nullptr),
           MOE_OK);
    EXPECT(moe_route(logits.p, dt, MOE_ROUTE_SOFTMAX_TOPK, 0, (int32_t *)idx.p, (float *)w.p,
                     nullptr, &M.m, rws.p, moe_route_workspace(N, K, E), nullptr),
           MOE_OK);
  }
  Buf x((size_t)N * H * es), wu((size_t)E * H * 2 * I * es), wd((size_t)E * I * H * es);
  Buf out((size_t)N * H * es), h((size_t)cap * 2 * I * es);
  const size_t fws = moe_expert_forward_workspace(&M.m, H, I, dt);
  Buf fw(fws);
  EXPECT(moe_expert_forward(&M.m, x.p, wu.p, wd.p, H, I, dt, lay, h.p, out.p, fw.p, fws, nullptr),
         MOE_OK);
  EXPECT(moe_expert_forward(&M.m, x.p, wu.p, wd.p, H, I, dt, lay, nullptr, out.p, fw.p, fws,
                            nullptr),
         MOE_OK);
  const size_t bws = moe_expert_backward_workspace(&M.m, H, I, dt);
  Buf bw(bws), dout((size_t)N * H * es), dx((size_t)N * H * es), dwu((size_t)E * H * 2 * I * es),
      dwd((size_t)E * I * H * es), dtw((size_t)N * K * 4);
  EXPECT(moe_expert_backward(&M.m, (int32_t *)idx.p, x.p, wu.p, wd.p, h.p, dout.p, H, I, dt, lay,
                             dx.p, dwu.p, dwd.p, (float *)dtw.p, bw.p, bws, nullptr),
         MOE_OK);
}

static void argument_errors() {
  Meta M(8, 2, 4, 16);
  Buf idx(64), w(64), x(8 * 128 * 2), wu(4 * 128 * 256 * 2), wd(4 * 128 * 128 * 2);
  Buf out(8 * 128 * 2), h(16 * 256 * 2);
  const size_t mws_n = moe_build_metadata_workspace(8, 2, 4);
  Buf mws(mws_n);
  EXPECT(moe_build_metadata(nullptr, nullptr, nullptr, nullptr, 0, nullptr), MOE_EINVAL);
  EXPECT(moe_build_metadata(nullptr, (float *)w.p, &M.m, mws.p, mws_n, nullptr), MOE_EINVAL);
  EXPECT(moe_build_metadata((int32_t *)idx.p, (float *)w.p, &M.m, mws.p, mws_n - 1, nullptr),
         MOE_ENOSPC);
  EXPECT(moe_build_metadata((int32_t *)idx.p, (float *)w.p, &M.m, nullptr, mws_n, nullptr),
         MOE_ENOSPC);
  moe_metadata bad = M.m;
  bad.K = 0;
  EXPECT(moe_build_metadata((int32_t *)idx.p, (float *)w.p, &bad, mws.p, mws_n, nullptr),
         MOE_EINVAL);
  bad = M.m;
  bad.K = MOE_MAX_TOPK + 1;
  EXPECT(moe_build_metadata_noalloc((int32_t *)idx.p, (float *)w.p, &bad, nullptr), MOE_EINVAL);
  bad = M.m;
  bad.E = MOE_MAX_EXPERTS + 1;
  EXPECT(moe_build_metadata_noalloc((int32_t *)idx.p, (float *)w.p, &bad, nullptr), MOE_EINVAL);
  bad = M.m;
  bad.capacity = -1;
  EXPECT(moe_build_metadata((int32_t *)idx.p, (float *)w.p, &bad, mws.p, mws_n, nullptr),
         MOE_EINVAL);
  bad = M.m;
  bad.x_gather_idx = nullptr;
  EXPECT(moe_build_metadata((int32_t *)idx.p, (float *)w.p, &bad, mws.p, mws_n, nullptr),
         MOE_EINVAL);
  bad = M.m;
  bad.status = nullptr;
  EXPECT(moe_build_metadata((int32_t *)idx.p, (float *)w.p, &bad, mws.p, mws_n, nullptr),
         MOE_EINVAL);
  const size_t fws = moe_expert_forward_workspace(&M.m, 128, 128, MOE_BF16);
  Buf fw(fws);
  EXPECT(moe_expert_forward(&M.m, x.p, wu.p, wd.p, 100, 128, MOE_BF16, MOE_GATEUP_INTERLEAVED,
                            h.p, out.p, fw.p, fws, nullptr),
         MOE_EUNSUPPORTED);  // H not a multiple of 8
  EXPECT(moe_expert_forward(&M.m, x.p, wu.p, wd.p, 128, 12, MOE_FP32, MOE_GATEUP_INTERLEAVED,
                            h.p, out.p, fw.p, fws, nullptr),
         MOE_EUNSUPPORTED);  // I not a multiple of 8
  EXPECT(moe_expert_forward(&M.m, x.p, wu.p, wd.p, 128, 0, MOE_BF16, MOE_GATEUP_INTERLEAVED,
                            h.p, out.p, fw.p, fws, nullptr),
         MOE_EUNSUPPORTED);
  EXPECT(moe_expert_forward(&M.m, x.p, wu.p, wd.p, 128, 128, (moe_dtype)7,
                            MOE_GATEUP_INTERLEAVED, h.p, out.p, fw.p, fws, nullptr),
         MOE_EUNSUPPORTED);
  EXPECT(moe_expert_forward(&M.m, x.p, wu.p, wd.p, 128, 128, MOE_BF16, (moe_gateup_layout)2, h.p,
                            out.p, fw.p, fws, nullptr),
         MOE_EUNSUPPORTED);
  EXPECT(moe_expert_forward(&M.m, x.p, wu.p, wd.p, 128, 128, MOE_BF16, MOE_GATEUP_INTERLEAVED,
                            h.p, out.p, fw.p, fws - 1, nullptr),
         MOE_ENOSPC);
  EXPECT(moe_expert_forward(&M.m, nullptr, wu.p, wd.p, 128, 128, MOE_BF16,
                            MOE_GATEUP_INTERLEAVED, h.p, out.p, fw.p, fws, nullptr),
         MOE_EINVAL);
  const size_t bws = moe_expert_backward_workspace(&M.m, 128, 128, MOE_BF16);
  Buf bw(bws);
  EXPECT(moe_expert_backward(&M.m, (int32_t *)idx.p, x.p, wu.p, wd.p, nullptr, x.p, 128, 128,
                             MOE_BF16, MOE_GATEUP_INTERLEAVED, x.p, wu.p, wd.p, (float *)w.p,
                             bw.p, bws, nullptr),
         MOE_EINVAL);  // saved activations missing
  EXPECT(moe_expert_backward(&M.m, (int32_t *)idx.p, x.p, wu.p, wd.p, h.p, x.p, 128, 128,
                             MOE_BF16, MOE_GATEUP_INTERLEAVED, x.p, wu.p, wd.p, (float *)w.p,
                             bw.p, bws - 1, nullptr),
         MOE_ENOSPC);
  Buf lg(8 * 4 * 4);
  const size_t rws = moe_route_workspace(8, 2, 4);
  Buf rw(rws);
  bad = M.m;
  bad.K = 5;  // K > E
  EXPECT(moe_route(lg.p, MOE_FP32, MOE_ROUTE_SOFTMAX_TOPK, 0, (int32_t *)idx.p, (float *)w.p,
                   nullptr, &bad, rw.p, 1 << 20, nullptr),
         MOE_EINVAL);
  EXPECT(moe_route(lg.p, MOE_FP32, (moe_route_mode)9, 0, (int32_t *)idx.p, (float *)w.p, nullptr,
                   &M.m, rw.p, rws, nullptr),
         MOE_EUNSUPPORTED);
  EXPECT(moe_route(lg.p, MOE_FP32, MOE_ROUTE_SOFTMAX_TOPK, 0, (int32_t *)idx.p, (float *)w.p,
                   nullptr, &M.m, rw.p, rws - 1, nullptr),
         MOE_ENOSPC);
  // the timing hook's argument checks, and its use around real launches
  void *ev[4] = {(void *)16, (void *)16, (void *)16, nullptr};
  EXPECT(moe_time_kernel((moe_kernel_id)99, ev, 1, nullptr), MOE_EINVAL);
  EXPECT(moe_time_kernel(MOE_KERNEL_META_SCATTER, ev, 2, nullptr), MOE_EINVAL);  // a null event
  EXPECT(moe_time_kernel(MOE_KERNEL_META_SCATTER, ev, 1, nullptr), MOE_OK);
  EXPECT(moe_build_metadata((int32_t *)idx.p, (float *)w.p, &M.m, mws.p, mws_n, nullptr), MOE_OK);
  EXPECT(moe_build_metadata((int32_t *)idx.p, (float *)w.p, &M.m, mws.p, mws_n, nullptr), MOE_OK);
  int32_t n = -1;
  EXPECT(moe_time_kernel(MOE_KERNEL_META_SCATTER, nullptr, 0, &n), MOE_OK);
  EXPECT(n, 1);  // the second build's launch was past the one bracketed slot
  if (strcmp(moe_status_string(MOE_ENOSPC), "workspace too small") != 0) exit(4);
  if (strcmp(moe_kernel_name((moe_kernel_id)-1), "unknown") != 0) exit(4);
}

// size arithmetic at the limits, with the stubs touching nothing
static void limits() {
  // N*K just below and at 2^31
  Meta M(0, 64, 1024, 0);
  M.m.N = (1 << 25) - 1;  // N*K = 2^31 - 64
  EXPECT(moe_build_metadata((int32_t *)16, (float *)16, &M.m, (void *)16, 1, nullptr),
         MOE_ENOSPC);
  if (moe_build_metadata_workspace(M.m.N, 64, 1024) == 0) exit(5);
  if (moe_route_workspace(M.m.N, 64, 1024) == 0) exit(5);
  EXPECT(moe_build_metadata_noalloc((int32_t *)16, (float *)16, &M.m, nullptr), MOE_ENOSPC);
  M.m.N = 1 << 25;  // N*K = 2^31
  EXPECT(moe_build_metadata((int32_t *)16, (float *)16, &M.m, (void *)16, 1, nullptr),
         MOE_EINVAL);
  // H = I = 2^20 with 1024 experts: every size query and grid in 64-bit arithmetic; the
  // weight-gradient grid exceeds the launch limit and is refused
  g_dry = true;
  Meta B(1 << 12, 8, 1024, 1 << 15);
  const int H = 1 << 20, I = 1 << 20;
  const size_t fws = moe_expert_forward_workspace(&B.m, H, I, MOE_BF16);
  const size_t bws = moe_expert_backward_workspace(&B.m, H, I, MOE_FP32);
  if (fws < (size_t)(1 << 15) * (size_t)(H + I) * 2 || bws <= fws) exit(6);
  EXPECT(moe_expert_forward(&B.m, (void *)16, (void *)16, (void *)16, H, I, MOE_BF16,
                            MOE_GATEUP_INTERLEAVED, (void *)16, (void *)16, (void *)16, fws,
                            nullptr),
         MOE_OK);
  EXPECT(moe_expert_backward(&B.m, (int32_t *)16, (void *)16, (void *)16, (void *)16, (void *)16,
                             (void *)16, H, I, MOE_FP32, MOE_GATEUP_INTERLEAVED, (void *)16,
                             (void *)16, (void *)16, (float *)16, (void *)16, bws, nullptr),
         MOE_EUNSUPPORTED);
  const size_t bws16 = moe_expert_backward_workspace(&B.m, H, I, MOE_BF16);
  EXPECT(moe_expert_backward(&B.m, (int32_t *)16, (void *)16, (void *)16, (void *)16, (void *)16,
                             (void *)16, H, I, MOE_BF16, MOE_GATEUP_CONCAT, (void *)16,
                             (void *)16, (void *)16, (float *)16, (void *)16, bws16, nullptr),
         MOE_EUNSUPPORTED);
  g_dry = false;
}

int main(int argc, char **argv) {
  g_plant = argc > 1 && strcmp(argv[1], "plant") == 0;
  if (g_plant) {
    full_case(16, 2, 4, 32, 128, 128, MOE_BF16, MOE_GATEUP_INTERLEAVED);
    printf("plant: not caught\n");
    return 0;
  }
  argument_errors();
  for (int d = 0; d < 2; d++)
    for (int l = 0; l < 2; l++) {
      const moe_dtype dt = d ? MOE_FP32 : MOE_BF16;
      const moe_gateup_layout lay = l ? MOE_GATEUP_CONCAT : MOE_GATEUP_INTERLEAVED;
      full_case(64, 4, 8, 64 * 4, 128, 128, dt, lay);  // capacity = N*K
      full_case(64, 4, 8, 100, 256, 384, dt, lay);     // capacity below N*K
      full_case(0, 2, 4, 0, 128, 128, dt, lay);        // N = 0
      full_case(16, 2, 4, 0, 128, 128, dt, lay);       // capacity = 0
      full_case(50, 4, 5, 200, 200, 72, dt, lay);      // partial edge tiles
      full_case(9, 2, 3, 18, 8, 8, dt, lay);           // the smallest H and I
      full_case(8, 8, 32, 40, 256, 136, dt, lay);      // decode-sized (32-row tiles)
    }
  full_case(4, 64, 1024, 256, 128, 128, MOE_BF16, MOE_GATEUP_INTERLEAVED);  // the limits
  full_case(1, 1, 1, 1, 128, 128, MOE_BF16, MOE_GATEUP_INTERLEAVED);
  full_case(3000, 8, 64, 24000, 128, 128, MOE_BF16, MOE_GATEUP_CONCAT);  // several chunks
  full_case((1 << 18) + 5, 8, 2, 1000, 128, 128, MOE_BF16, MOE_GATEUP_INTERLEAVED);  // > 2^21
  limits();
  printf("abi ok: %d checks, %d stub launches\n", g_checks, g_launches);
  return 0;
}
