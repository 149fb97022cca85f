// Restricted attention (a window around each query position) with the flash
// kernel of sdpa_fwd_kernel.h, bf16 / fp16: nickwang.xyz "Lire « Attention
// Is All You Need »" §4, Table 1 ("Auto-attention restreinte") and the text
// after it -- attention limited to a neighbourhood of the output position,
// O(r·n·d) work for a neighbourhood of size r.  The waves per workgroup come
// from the route (sdpa_route.cpp).  Key c is visible to query r
// iff r − win_left <= c <= r + win_right; the centred neighbourhood of size
// 2w + 1 is win_left = win_right = w.  Only the key tiles inside some row's
// window are loaded and computed, so the work (and the time) scales with the
// window, not with n_k.

#include "sdpa_fwd_kernel.h"

namespace mha {

namespace {

template <int DT, int DH, int NW>
hipError_t launch_win_nw(const SdpaArgs& a, hipStream_t st) {
  const int64_t nqb = (a.n_q + NW * 64 - 1) / (NW * 64);
  const int64_t grid = nqb * a.B * a.H;
  hipLaunchKernelGGL((sdpa_fwd_kernel<DT, DH, false, NW, false, true>), dim3((unsigned)grid),
                     dim3(NW * 64), 0, st, a);
  return hipGetLastError();
}

template <int DT, int DH>
hipError_t launch_win(const SdpaArgs& a, int waves, hipStream_t st) {
  switch (waves) {
    case 1: return launch_win_nw<DT, DH, 1>(a, st);
    case 2: return launch_win_nw<DT, DH, 2>(a, st);
    case 4: return launch_win_nw<DT, DH, 4>(a, st);
    default: return hipErrorInvalidValue;
  }
}

template <int DT>
hipError_t launch_win_dim(const SdpaArgs& a, int waves, int d, hipStream_t st) {
  switch (d) {
    case 16: return launch_win<DT, 16>(a, waves, st);
    case 32: return launch_win<DT, 32>(a, waves, st);
    case 64: return launch_win<DT, 64>(a, waves, st);
    case 128: return launch_win<DT, 128>(a, waves, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_sdpa_window(const SdpaArgs& a, const SdpaRoute& r, int dtype, int d, hipStream_t st) {
  if (r.kernel != SDPA_K_WINDOW) return hipErrorInvalidValue;
  if (dtype == DT_BF16) return launch_win_dim<DT_BF16>(a, r.waves, d, st);
  if (dtype == DT_F16) return launch_win_dim<DT_F16>(a, r.waves, d, st);
  return hipErrorInvalidValue;
}

}  // namespace mha
