// Drives the library through include/moe.h alone, from plain C++ with the HIP runtime
// (no Python, no torch): reads one case's inputs from a directory, builds the routing
// metadata, runs the forward and the backward on the default stream, and writes every
// output back to the same directory. The test that runs it compares the outputs with the
// oracle; this program does no arithmetic of its own.
//
// usage: abi_gpu_driver <dir> N H I E K capacity
// inputs (raw little-endian): x.bin [N,H] bf16 bits, w_up.bin [E,H,2I], w_down.bin [E,I,H],
//   dout.bin [N,H], topk_idx.bin [N,K] int32, topk_weights.bin [N,K] fp32
// outputs: the metadata arrays (<name>.out), out.out [N,H], h.out [capacity,2I], dx.out,
//   dw_up.out, dw_down.out, dtw.out [N,K] fp32
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <string>
#include <vector>

#include "moe.h"

namespace {

std::string g_dir;

bool read_file(const char *name, std::vector<char> &buf, size_t bytes) {
  const std::string path = g_dir + "/" + name;
  FILE *f = std::fopen(path.c_str(), "rb");
  if (!f) {
    std::fprintf(stderr, "cannot open %s\n", path.c_str());
    return false;
  }
  buf.resize(bytes);
  const size_t got = bytes ? std::fread(buf.data(), 1, bytes, f) : 0;
  std::fclose(f);
  if (got != bytes) {
    std::fprintf(stderr, "%s: %zu bytes, expected %zu\n", path.c_str(), got, bytes);
    return false;
  }
  return true;
}

bool write_file(const char *name, const void *dev, size_t bytes) {
  std::vector<char> host(bytes);
  if (bytes && hipMemcpy(host.data(), dev, bytes, hipMemcpyDeviceToHost) != hipSuccess) {
    std::fprintf(stderr, "copy of %s failed\n", name);
    return false;
  }
  const std::string path = g_dir + "/" + name;
  FILE *f = std::fopen(path.c_str(), "wb");
  if (!f) return false;
  const size_t put = bytes ? std::fwrite(host.data(), 1, bytes, f) : 0;
  std::fclose(f);
  return put == bytes;
}

// device buffer of at least one byte (a zero-size request still gets a valid pointer)
void *dev_alloc(size_t bytes) {
  void *p = nullptr;
  if (hipMalloc(&p, bytes ? bytes : 1) != hipSuccess) {
    std::fprintf(stderr, "hipMalloc(%zu) failed\n", bytes);
    std::exit(3);
  }
  return p;
}

void *dev_from_file(const char *name, size_t bytes) {
  std::vector<char> buf;
  if (!read_file(name, buf, bytes)) std::exit(4);
  void *p = dev_alloc(bytes);
  if (bytes && hipMemcpy(p, buf.data(), bytes, hipMemcpyHostToDevice) != hipSuccess) {
    std::fprintf(stderr, "upload of %s failed\n", name);
    std::exit(3);
  }
  return p;
}

}  // namespace

#define MOE_CHECK(call)                                                              \
  do {                                                                               \
    const moe_status s_ = (call);                                                    \
    if (s_ != MOE_OK) {                                                              \
      std::fprintf(stderr, "%s: %s\n", #call, moe_status_string(s_));                \
      return 2;                                                                      \
    }                                                                                \
  } while (0)

int main(int argc, char **argv) {
  if (argc != 8) {
    std::fprintf(stderr, "usage: %s <dir> N H I E K capacity\n", argv[0]);
    return 1;
  }
  g_dir = argv[1];
  const int32_t N = std::atoi(argv[2]), H = std::atoi(argv[3]), I = std::atoi(argv[4]),
                E = std::atoi(argv[5]), K = std::atoi(argv[6]), cap = std::atoi(argv[7]);
  const size_t nk = (size_t)N * K, bf = 2;

  void *x = dev_from_file("x.bin", (size_t)N * H * bf);
  void *w_up = dev_from_file("w_up.bin", (size_t)E * H * 2 * I * bf);
  void *w_down = dev_from_file("w_down.bin", (size_t)E * I * H * bf);
  void *dout = dev_from_file("dout.bin", (size_t)N * H * bf);
  auto *idx = (int32_t *)dev_from_file("topk_idx.bin", nk * 4);
  auto *wts = (float *)dev_from_file("topk_weights.bin", nk * 4);

  moe_metadata m = {};
  m.N = N;
  m.K = K;
  m.E = E;
  m.capacity = cap;
  m.expert_frequency = (int32_t *)dev_alloc((size_t)E * 4);
  m.expert_frequency_offset = (int32_t *)dev_alloc((size_t)(E + 1) * 4);
  m.x_gather_idx = (int32_t *)dev_alloc((size_t)cap * 4);
  m.s_scatter_idx = (int32_t *)dev_alloc((size_t)cap * 4);
  m.s_reverse_scatter_idx = (int32_t *)dev_alloc((size_t)cap * 4);
  m.num_activated_expert_per_token_offset = (int32_t *)dev_alloc((size_t)(N + 1) * 4);
  m.router_scores = (float *)dev_alloc((size_t)cap * 4);
  m.status = (uint32_t *)dev_alloc(4);

  const size_t wsm = moe_build_metadata_workspace(N, K, E);
  void *ws_meta = dev_alloc(wsm);
  MOE_CHECK(moe_build_metadata(idx, wts, &m, ws_meta, wsm, nullptr));

  void *h = dev_alloc((size_t)cap * 2 * I * bf);
  void *out = dev_alloc((size_t)N * H * bf);
  const size_t wsf = moe_expert_forward_workspace(&m, H, I, MOE_BF16);
  void *ws_fwd = dev_alloc(wsf);
  MOE_CHECK(moe_expert_forward(&m, x, w_up, w_down, H, I, MOE_BF16, MOE_GATEUP_INTERLEAVED, h,
                               out, ws_fwd, wsf, nullptr));

  void *dx = dev_alloc((size_t)N * H * bf);
  void *dw_up = dev_alloc((size_t)E * H * 2 * I * bf);
  void *dw_down = dev_alloc((size_t)E * I * H * bf);
  auto *dtw = (float *)dev_alloc(nk * 4);
  const size_t wsb = moe_expert_backward_workspace(&m, H, I, MOE_BF16);
  void *ws_bwd = dev_alloc(wsb);
  MOE_CHECK(moe_expert_backward(&m, idx, x, w_up, w_down, h, dout, H, I, MOE_BF16,
                                MOE_GATEUP_INTERLEAVED, dx, dw_up, dw_down, dtw, ws_bwd, wsb,
                                nullptr));
  if (hipDeviceSynchronize() != hipSuccess) {
    std::fprintf(stderr, "device synchronisation failed\n");
    return 3;
  }

  const bool ok =
      write_file("expert_frequency.out", m.expert_frequency, (size_t)E * 4) &&
      write_file("expert_frequency_offset.out", m.expert_frequency_offset, (size_t)(E + 1) * 4) &&
      write_file("x_gather_idx.out", m.x_gather_idx, (size_t)cap * 4) &&
      write_file("s_scatter_idx.out", m.s_scatter_idx, (size_t)cap * 4) &&
      write_file("s_reverse_scatter_idx.out", m.s_reverse_scatter_idx, (size_t)cap * 4) &&
      write_file("num_activated_expert_per_token_offset.out",
                 m.num_activated_expert_per_token_offset, (size_t)(N + 1) * 4) &&
      write_file("router_scores.out", m.router_scores, (size_t)cap * 4) &&
      write_file("status.out", m.status, 4) &&
      write_file("out.out", out, (size_t)N * H * bf) &&
      write_file("h.out", h, (size_t)cap * 2 * I * bf) &&
      write_file("dx.out", dx, (size_t)N * H * bf) &&
      write_file("dw_up.out", dw_up, (size_t)E * H * 2 * I * bf) &&
      write_file("dw_down.out", dw_down, (size_t)E * I * H * bf) &&
      write_file("dtw.out", dtw, nk * 4);
  if (!ok) return 4;
  std::printf("abi_gpu_driver: N=%d H=%d I=%d E=%d K=%d capacity=%d ok\n", N, H, I, E, K, cap);
  return 0;
}
