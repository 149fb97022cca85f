// A host-only driver of the libmha C ABI, built with the address and
// undefined-behaviour sanitizers on the host code (tests/test_host_sanitizers.py).
//
// Every call here either fails validation on the host, is a zero-size no-op,
// asks for a route, or -- only when the environment has no GPU -- passes
// validation and must fail at its first HIP call with MHA_ERR_HIP.  Host
// buffers stand in for device pointers; no kernel is ever launched.  Any
// sanitizer report aborts the process; a wrong status returns 1.

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "mha.h"

static int failures = 0;

static void expect(int got, int want, const char* what) {
  if (got != want) {
    std::fprintf(stderr, "FAIL %s: status %d, expected %d (%s)\n", what, got, want, mha_last_error());
    ++failures;
  }
}

int main(int argc, char** argv) {
  const bool no_device = argc > 1 && std::strcmp(argv[1], "--no-device") == 0;
  // 256-byte aligned host memory standing in for device buffers
  std::vector<unsigned char> mem(8 << 20);
  uintptr_t base = (reinterpret_cast<uintptr_t>(mem.data()) + 255) & ~(uintptr_t)255;
  auto at = [&](size_t off) { return reinterpret_cast<void*>(base + off); };
  void* Q = at(0);
  void* K = at(1 << 20);
  void* V = at(2 << 20);
  void* O = at(3 << 20);
  const float nan = std::nanf("");

  // ---- mha_sdpa validation
  expect(mha_sdpa(Q, K, V, O, 7, 1, 1, 8, 8, 64, 64, 0.125f, 0, nullptr, nullptr), MHA_ERR_DTYPE, "dtype");
  expect(mha_sdpa(Q, K, V, O, MHA_BF16, -1, 1, 8, 8, 64, 64, 0.125f, 0, nullptr, nullptr), MHA_ERR_SHAPE, "B<0");
  expect(mha_sdpa(Q, K, V, O, MHA_BF16, 1, 1, 8, 9, 64, 64, 0.125f, MHA_MASK_CAUSAL, nullptr, nullptr),
         MHA_ERR_SHAPE, "causal n_q != n_k");
  expect(mha_sdpa(Q, K, V, O, MHA_BF16, 1, 1, 8, 8, 64, 64, INFINITY, 0, nullptr, nullptr),
         MHA_ERR_INVALID_ARG, "inf scale");
  expect(mha_sdpa(Q, K, V, O, MHA_BF16, 0, 1, 8, 8, 64, 64, nan, 0, nullptr, nullptr), MHA_OK, "NaN scale, B 0");
  expect(mha_sdpa(Q, K, V, O, MHA_BF16, 1, 1, 8, 8, 48, 48, 0.125f, 0, nullptr, nullptr),
         MHA_ERR_UNSUPPORTED, "d 48");
  expect(mha_sdpa(nullptr, K, V, O, MHA_BF16, 1, 1, 8, 8, 64, 64, 0.125f, 0, nullptr, nullptr),
         MHA_ERR_INVALID_ARG, "null Q");
  expect(mha_sdpa(Q, at((1 << 20) + 8), V, O, MHA_BF16, 1, 1, 8, 8, 64, 64, 0.125f, 0, nullptr, nullptr),
         MHA_ERR_INVALID_ARG, "misaligned K");
  expect(mha_sdpa(Q, K, V, at(64), MHA_BF16, 1, 1, 8, 8, 64, 64, 0.125f, 0, nullptr, nullptr),
         MHA_ERR_ALIAS, "O overlaps Q");
  expect(mha_sdpa(Q, K, V, O, MHA_BF16, 1, 1, (int64_t)1 << 31, 8, 64, 64, 0.125f, 0, nullptr, nullptr),
         MHA_ERR_SHAPE, "n_q too large");

  // ---- strided forms
  mha_sdpa_strides st;
  for (int i = 0; i < 3; ++i) st.q[i] = st.k[i] = st.v[i] = st.o[i] = 0;
  const int64_t contig[3] = {8 * 64, 8 * 64, 64};
  for (int i = 0; i < 3; ++i) st.q[i] = st.k[i] = st.v[i] = st.o[i] = contig[i];
  expect(mha_sdpa_strided(Q, K, V, O, nullptr, MHA_BF16, 1, 1, 8, 8, 64, 64, 0.125f, 0, nullptr, nullptr),
         MHA_ERR_INVALID_ARG, "null strides");
  st.k[2] = 68;
  expect(mha_sdpa_strided(Q, K, V, O, &st, MHA_BF16, 1, 1, 8, 8, 64, 64, 0.125f, 0, nullptr, nullptr),
         MHA_ERR_INVALID_ARG, "unaligned stride");
  st.k[2] = 64;
  st.o[2] = 32;
  expect(mha_sdpa_strided(Q, K, V, O, &st, MHA_BF16, 1, 1, 8, 8, 64, 64, 0.125f, 0, nullptr, nullptr),
         MHA_ERR_INVALID_ARG, "overlapping output rows");
  st.o[2] = 64;
  st.q[0] = 1 << 14;
  expect(mha_sdpa_strided(Q, K, V, at(2 * 64 * 8), &st, MHA_BF16, 2, 1, 8, 8, 64, 64, 0.125f, 0, nullptr,
                          nullptr),
         MHA_ERR_ALIAS, "O inside Q's span");
  st.q[0] = 8 * 64;
  expect(mha_sdpa_window_strided(Q, K, V, O, &st, MHA_BF16, 1, 1, 8, 8, 64, 64, 0.125f, -1, 2, nullptr,
                                 nullptr),
         MHA_ERR_INVALID_ARG, "window reach < 0");

  // ---- routes
  mha_route r;
  expect(mha_sdpa_route(MHA_BF16, 4, 8, 4096, 4096, 64, 64, MHA_MASK_NONE, 0, 0, 0, &r), MHA_OK, "route");
  if (r.kernel != MHA_KERNEL_BLOCKS || r.waves != 8 || r.workgroups != 256) {
    std::fprintf(stderr, "FAIL route [4,8,4096,64]: kernel %d waves %d wgs %lld\n", r.kernel, r.waves,
                 (long long)r.workgroups);
    ++failures;
  }
  expect(mha_sdpa_route(MHA_BF16, 4, 8, 4096, 4096, 64, 64, MHA_MASK_NONE, 1, 4095, 0, &r), MHA_OK,
         "route window");
  if (r.mask_kind != MHA_MASK_CAUSAL) {
    std::fprintf(stderr, "FAIL window reaching back to every key is not the causal mask\n");
    ++failures;
  }
  expect(mha_sdpa_route(MHA_BF16, 1, 1, 8, 8, 64, 64, 0, 0, 0, 0, nullptr), MHA_ERR_INVALID_ARG, "null route");

  // ---- mha_forward and friends
  void* W[4] = {at(4 << 20), at(5 << 20), at(6 << 20), at(7 << 20)};
  void* out = at(3 << 20);
  expect(mha_forward(Q, nullptr, W[0], W[1], W[2], W[3], out, MHA_F32, 2, 8, 8, 128, 2, 0, nullptr, nullptr,
                     0, nullptr),
         MHA_ERR_UNSUPPORTED, "forward f32");
  expect(mha_forward(Q, nullptr, W[0], W[1], W[2], W[3], out, MHA_BF16, 2, 8, 8, 129, 2, 0, nullptr, nullptr,
                     0, nullptr),
         MHA_ERR_SHAPE, "forward d_model % h");
  expect(mha_forward(Q, nullptr, W[0], W[1], W[2], W[3], out, MHA_BF16, 2, 8, 8, 128, 2, 0, nullptr,
                     at((2 << 20) + 256), 16, nullptr),
         MHA_ERR_WORKSPACE, "forward small workspace");
  expect(mha_forward(Q, nullptr, W[0], W[1], W[2], W[3], Q, MHA_BF16, 2, 8, 8, 128, 2, 0, nullptr, nullptr, 0,
                     nullptr),
         MHA_ERR_ALIAS, "forward out == x_q");
  expect(mha_forward_noalloc(Q, nullptr, W[0], W[1], W[2], W[3], out, MHA_BF16, 16, 512, 512, 1024, 16, 0,
                             nullptr, nullptr),
         MHA_ERR_WORKSPACE, "noalloc oversized");
  expect(mha_forward_noalloc(Q, nullptr, W[0], W[1], W[2], W[3], out, MHA_BF16, 0, 8, 8, 128, 2, 0, nullptr,
                             nullptr),
         MHA_OK, "noalloc B 0");
  expect(mha_add_norm(Q, K, V, O, -1.f, out, MHA_BF16, 4, 64, nullptr), MHA_ERR_INVALID_ARG, "add_norm eps");
  expect(mha_add_norm(Q, K, W[0], W[1], 1e-5f, at(32), MHA_BF16, 4, 64, nullptr), MHA_ERR_ALIAS,
         "add_norm partial overlap");
  expect(mha_forward_add_norm(Q, nullptr, W[0], W[1], W[2], W[3], nullptr, W[1], 1e-5f, out, MHA_BF16, 2, 8, 8,
                              128, 2, 0, nullptr, nullptr, 0, nullptr),
         MHA_ERR_INVALID_ARG, "forward_add_norm null gamma");
  if (mha_forward_workspace_size(8, 384, 512, 1024, 16, MHA_BF16) == 0) {
    std::fprintf(stderr, "FAIL workspace size\n");
    ++failures;
  }
  if (std::strncmp(mha_status_string(MHA_ERR_HIP), "MHA_ERR_HIP", 11) != 0 || mha_status_string(-99) == nullptr) {
    std::fprintf(stderr, "FAIL status strings\n");
    ++failures;
  }

  // ---- valid calls with no device: the first HIP call fails, cleanly
  if (no_device) {
    expect(mha_sdpa(Q, K, V, O, MHA_BF16, 1, 1, 8, 8, 64, 64, 0.125f, 0, nullptr, nullptr), MHA_ERR_HIP,
           "sdpa without a device");
    expect(mha_sdpa_strided(Q, K, V, O, &st, MHA_F32, 1, 1, 8, 8, 64, 64, nan, MHA_MASK_CAUSAL, nullptr,
                            nullptr),
           MHA_ERR_HIP, "strided sdpa without a device");
    expect(mha_forward(Q, nullptr, W[0], W[1], W[2], W[3], out, MHA_BF16, 2, 8, 8, 128, 2, 0, nullptr,
                       at((2 << 20) + 256), 1 << 20, nullptr),
           MHA_ERR_HIP, "forward without a device");
    expect(mha_forward_noalloc(Q, nullptr, W[0], W[1], W[2], W[3], out, MHA_BF16, 2, 8, 8, 128, 2, 0, nullptr,
                               nullptr),
           MHA_ERR_HIP, "noalloc without a device");
  }
  if (failures) return 1;
  std::printf("abi driver: all checks passed%s\n", no_device ? " (including no-device calls)" : "");
  return 0;
}
