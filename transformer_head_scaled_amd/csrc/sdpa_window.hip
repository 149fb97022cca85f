// Restricted attention (a window around each query position) with the flash
// kernel of sdpa_fwd_kernel.h, bf16 / fp16: nickwang.xyz "Lire « Attention
// Is All You Need »" §4, Table 1 ("Auto-attention restreinte") and the text
// after it -- attention limited to a neighbourhood of the output position,
// O(r·n·d) work for a neighbourhood of size r.  Key c is visible to query r
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

// Waves per workgroup: as for the plain kernel, but at most two while the
// window spans fewer than 2048 keys besides the row itself.  A workgroup
// loads the key tiles of all its rows' windows and every wave takes part in
// every step, so a wave idles through the tiles only its neighbours see,
// with nothing to cover the next tile's load; 128 rows a workgroup halve
// that.  Measured on [4,8,4096,64], reach w on both sides, four waves
// against two: w 0 36.7 / 25.3 µs, 64 41.2 / 31.6, 256 55.4 / 41.8, 1024
// 97.9 / 88.9, 2048 141.8 / 145.3 (one wave: slower from w 64 on).
int window_waves(const SdpaArgs& a) {
  const int w = waves_per_wg(a.n_q, (int64_t)a.B * a.H, false);
  return (w > 2 && (int64_t)a.win_left + a.win_right < 2048) ? 2 : w;
}

template <int DT, int DH>
hipError_t launch_win(const SdpaArgs& a, hipStream_t st) {
  switch (window_waves(a)) {
    case 1: return launch_win_nw<DT, DH, 1>(a, st);
    case 2: return launch_win_nw<DT, DH, 2>(a, st);
    default: return launch_win_nw<DT, DH, 4>(a, st);
  }
}

template <int DT>
hipError_t launch_win_dim(const SdpaArgs& a, int d, hipStream_t st) {
  switch (d) {
    case 16: return launch_win<DT, 16>(a, st);
    case 32: return launch_win<DT, 32>(a, st);
    case 64: return launch_win<DT, 64>(a, st);
    case 128: return launch_win<DT, 128>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_sdpa_window(const SdpaArgs& a, int dtype, int d, hipStream_t st) {
  if (dtype == DT_BF16) return launch_win_dim<DT_BF16>(a, d, st);
  if (dtype == DT_F16) return launch_win_dim<DT_F16>(a, d, st);
  return hipErrorInvalidValue;
}

}  // namespace mha
