// libmha host layer: argument validation, workspace layout, dispatch.
//
// Implements the C ABI declared in include/mha.h.  Every check runs before
// the first enqueue, so an error never leaves partial output.

#include "mha.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <utility>

#include "kernels.h"

// mha_forward for n_q, n_k <= 64 at head dimension 64 without a causal mask:
// 1 runs the projections and the attention of each head in one launch
// (mha_short.hip), 0 keeps them separate
#ifndef MHA_SHORT_FUSED
#define MHA_SHORT_FUSED 1
#endif

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return MHA_OK;
}

bool trace_on() {
  static const int on = [] {
    const char* e = std::getenv("MHA_TRACE");
    return (e && *e && std::strcmp(e, "0") != 0) ? 1 : 0;
  }();
  return on != 0;
}

size_t elem_size(int dtype) { return dtype == MHA_F32 ? 4 : 2; }

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

Range range_of(const void* p, size_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Range{a, a + bytes};
}

bool overlap(Range a, Range b) {
  if (a.lo == a.hi || b.lo == b.hi) return false;
  return a.lo < b.hi && b.lo < a.hi;
}

constexpr int64_t kMaxRows = (int64_t)1 << 30;  // rows per sequence (int32 indexing in kernels)
// The MFMA kernels address one head's K/V through a buffer resource with a
// 32-bit byte range.
constexpr int64_t kMaxBufferBytes = ((int64_t)1 << 31) - 1;
// No operand may span more bytes than this (far beyond any device's memory);
// it also keeps the byte arithmetic on shapes and strides clear of overflow.
constexpr int64_t kMaxSpanBytes = (int64_t)1 << 46;

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct WsLayout {
  size_t q, k, v, concat, total;
  // mha_forward_add_norm: the fp32 x + concat·Wo rows, written after the
  // attention has consumed Q/K/V, so at offset 0 when that region is large
  // enough (it must not reach the concat, which the same GEMM reads)
  size_t z, total_an;
};

WsLayout ws_layout(int64_t B, int64_t n_q, int64_t n_k, int64_t d_model, int dtype) {
  const size_t es = elem_size(dtype);
  WsLayout w;
  w.q = 0;
  w.k = align256(w.q + (size_t)(B * n_q * d_model) * es);
  w.v = align256(w.k + (size_t)(B * n_k * d_model) * es);
  w.concat = align256(w.v + (size_t)(B * n_k * d_model) * es);
  w.total = align256(w.concat + (size_t)(B * n_q * d_model) * es);
  const size_t zbytes = align256((size_t)(B * n_q * d_model) * 4);
  w.z = zbytes <= w.concat ? 0 : w.total;
  w.total_an = w.z + zbytes > w.total ? w.z + zbytes : w.total;
  return w;
}

// The sizes mha_forward accepts (non-negative ones): rows per sequence for
// int32 indexing, rows per launch for the GEMMs' int32 M, and the product
// B·n·d_model, which ws_layout forms in 64 bits.
bool forward_sizes_in_range(int64_t B, int64_t n_q, int64_t n_k, int64_t d_model) {
  return n_q <= kMaxRows && n_k <= kMaxRows && B <= 65535 && d_model <= 65536 &&
         B * n_q <= ((int64_t)1 << 31) - 1 && B * n_k <= ((int64_t)1 << 31) - 1;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

int hip_fail(hipError_t e, const char* what) {
  return fail(MHA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// The workspace of mha_forward_noalloc: a device array of this library, one
// copy on every GPU that loads it, held until the process ends.  Its name in
// host code is only a stand-in for the symbol; the device address comes from
// hipGetSymbolAddress, once per device, and is what the kernels receive.
static __device__ __align__(256) unsigned char scratch[MHA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// this device's address of `scratch` (looked up on the first call on it)
int scratch_on_current_device(const char* fn, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, fn);
  if (dev < 0 || dev >= kMaxDevices) return fail(MHA_ERR_HIP, "%s: device %d out of range", fn, dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, fn);
    if (!p) return fail(MHA_ERR_HIP, "%s: no device address for the scratch array", fn);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MHA_OK;
}

}  // namespace

extern "C" {

const char* mha_status_string(int status) {
  switch (status) {
    case MHA_OK: return "MHA_OK";
    case MHA_ERR_INVALID_ARG: return "MHA_ERR_INVALID_ARG: invalid argument";
    case MHA_ERR_SHAPE: return "MHA_ERR_SHAPE: inconsistent or out-of-range sizes";
    case MHA_ERR_DTYPE: return "MHA_ERR_DTYPE: unknown dtype";
    case MHA_ERR_UNSUPPORTED: return "MHA_ERR_UNSUPPORTED: valid but not implemented";
    case MHA_ERR_WORKSPACE: return "MHA_ERR_WORKSPACE: workspace too small";
    case MHA_ERR_ALIAS: return "MHA_ERR_ALIAS: output overlaps an input";
    case MHA_ERR_HIP: return "MHA_ERR_HIP: HIP runtime error";
    default: return "unknown libmha status";
  }
}

const char* mha_last_error(void) { return g_err; }

int mha_version(void) { return 300; }

// The sizes of one attention call, validated (dtype, shapes, scale, window)
// and brought to the form the launch uses: a NaN scale becomes 1/sqrt(d_k), a
// window that reaches every key is dropped, and one that reaches every
// earlier key and no later one becomes the causal mask.
struct SdpaSizes {
  int32_t dtype;
  int64_t B, h, n_q, n_k, d_k, d_v;
  float scale;
  int32_t mask_kind;
  bool window;
  int64_t left, right;  // reaches, clamped to [0, n_q] and [0, n_k]
};

static int sdpa_sizes(const char* fn, SdpaSizes& z) {
  if (z.dtype != MHA_F32 && z.dtype != MHA_BF16 && z.dtype != MHA_F16)
    return fail(MHA_ERR_DTYPE, "%s: dtype %d", fn, (int)z.dtype);
  if (z.mask_kind != MHA_MASK_NONE && z.mask_kind != MHA_MASK_CAUSAL)
    return fail(MHA_ERR_INVALID_ARG, "%s: mask_kind %d", fn, (int)z.mask_kind);
  if (z.B < 0 || z.h < 0 || z.n_q < 0 || z.n_k < 0 || z.d_k <= 0 || z.d_v <= 0)
    return fail(MHA_ERR_SHAPE, "%s: negative or zero size", fn);
  if (z.n_q > kMaxRows || z.n_k > kMaxRows || z.B > 65535 || z.h > 65535 || z.B * z.h > (int64_t)1 << 24)
    return fail(MHA_ERR_SHAPE, "%s: size beyond the supported range", fn);
  if (z.mask_kind == MHA_MASK_CAUSAL && z.n_q != z.n_k)
    return fail(MHA_ERR_SHAPE, "%s: causal mask needs n_q == n_k (%lld vs %lld)", fn,
                (long long)z.n_q, (long long)z.n_k);
  // NaN: the pages' scale 1/sqrt(d_k)
  if (std::isnan(z.scale)) z.scale = 1.0f / std::sqrt((float)z.d_k);
  if (!std::isfinite(z.scale)) return fail(MHA_ERR_INVALID_ARG, "%s: scale is infinite", fn);
  if (z.window && (z.left < 0 || z.right < 0))
    return fail(MHA_ERR_INVALID_ARG, "%s: window reaches must be >= 0 (%lld, %lld)", fn,
                (long long)z.left, (long long)z.right);
  if (z.window && z.left >= z.n_q - 1 && z.right >= z.n_k - 1) z.window = false;
  if (z.window && z.left >= z.n_q - 1 && z.right == 0 && z.n_q == z.n_k) {
    z.window = false;
    z.mask_kind = MHA_MASK_CAUSAL;
  }
  if (!z.window) z.left = z.right = 0;
  if (z.left > z.n_q) z.left = z.n_q;
  if (z.right > z.n_k) z.right = z.n_k;
  const int64_t d = z.d_k;
  if (z.dtype == MHA_F32) {
    if (z.d_k != z.d_v || (d != 16 && d != 32 && d != 64 && d != 128))
      return fail(MHA_ERR_UNSUPPORTED, "%s: f32 needs d_k == d_v in {16,32,64,128}", fn);
  } else if (z.d_k != z.d_v || (d != 16 && d != 32 && d != 64 && d != 128 && d != 256 && d != 512)) {
    return fail(MHA_ERR_UNSUPPORTED, "%s: bf16/f16 needs d_k == d_v in {16,32,64,128,256,512}", fn);
  } else if (z.window && d > 128) {
    return fail(MHA_ERR_UNSUPPORTED, "%s: the window needs d_k <= 128", fn);
  }
  return MHA_OK;
}

static mha::SdpaRoute route_of(const SdpaSizes& z) {
  return mha::sdpa_route(z.dtype, z.mask_kind == MHA_MASK_CAUSAL, z.window, z.B, z.h, z.n_q, z.n_k,
                         (int)z.d_k, z.left, z.right);
}

// One [B, h, n, d] operand: element strides of batch, head and row (the d
// axis contiguous).
struct Operand {
  const void* p;
  int64_t sb, sh, sr;
  int64_t n, d;
};

// bytes from an operand's first element to one past its last (B, h, n >= 1),
// in 128 bits so that no shape or stride the checks let through overflows
static __int128 span_bytes(const Operand& t, int64_t B, int64_t h, size_t es) {
  return ((__int128)t.sb * (B - 1) + (__int128)t.sh * (h - 1) + (__int128)t.sr * (t.n - 1) + t.d) *
         (__int128)es;
}
// [lo, hi) bytes an operand can touch (its span checked against kMaxSpanBytes)
static Range span_of(const Operand& t, int64_t B, int64_t h, size_t es) {
  return range_of(t.p, (size_t)span_bytes(t, B, h, es));
}

// Distinct (batch, head, row) of an output land on distinct elements: the
// dimensions, ordered by stride, each step past everything inside the
// previous ones.
static bool rows_disjoint(const Operand& o, int64_t B, int64_t h) {
  struct Dim { int64_t stride, size; } dims[3] = {{o.sr, o.n}, {o.sh, h}, {o.sb, B}};
  for (int i = 0; i < 3; ++i)
    for (int j = i + 1; j < 3; ++j)
      if (dims[j].stride < dims[i].stride) std::swap(dims[i], dims[j]);
  __int128 extent = o.d;  // elements spanned by the dimensions so far
  for (const Dim& dm : dims) {
    if (dm.size <= 1) continue;
    if (dm.stride < extent) return false;
    extent = (__int128)dm.stride * (dm.size - 1) + extent;
  }
  return true;
}

static bool reverse_grid() {
  const char* e = std::getenv("MHA_GRID_ORDER");
  return e && std::strcmp(e, "reverse") == 0;
}

// mha_sdpa, mha_sdpa_window and their strided forms.  st: element strides
// ([batch, head, row] of Q, K, V, O), or NULL for contiguous tensors.
static int sdpa_impl(const char* fn, const void* Q, const void* K, const void* V, void* O,
                     const mha_sdpa_strides* st, SdpaSizes z, const int32_t* seq_lens,
                     void* stream) {
  int rc = sdpa_sizes(fn, z);
  if (rc != MHA_OK) return rc;
  const int64_t B = z.B, h = z.h, n_q = z.n_q, n_k = z.n_k, d_k = z.d_k, d_v = z.d_v;
  Operand q{Q, h * n_q * d_k, n_q * d_k, d_k, n_q, d_k}, k{K, h * n_k * d_k, n_k * d_k, d_k, n_k, d_k},
      v{V, h * n_k * d_v, n_k * d_v, d_v, n_k, d_v}, o{O, h * n_q * d_v, n_q * d_v, d_v, n_q, d_v};
  const size_t es = elem_size(z.dtype);
  if (st) {
    Operand* ops[4] = {&q, &k, &v, &o};
    const int64_t* s3[4] = {st->q, st->k, st->v, st->o};
    const int64_t align = 16 / (int64_t)es;  // rows start on 16 bytes
    for (int i = 0; i < 4; ++i) {
      for (int j = 0; j < 3; ++j)
        if (s3[i][j] < 0 || s3[i][j] > kMaxSpanBytes / (int64_t)es || s3[i][j] % align != 0)
          return fail(MHA_ERR_INVALID_ARG,
                      "%s: strides must be >= 0, below 2^46 bytes and multiples of %lld elements "
                      "(operand %d, stride %lld)",
                      fn, (long long)align, i, (long long)s3[i][j]);
      ops[i]->sb = s3[i][0], ops[i]->sh = s3[i][1], ops[i]->sr = s3[i][2];
    }
    if (!rows_disjoint(o, B, h))
      return fail(MHA_ERR_INVALID_ARG, "%s: O strides make output rows overlap", fn);
  }
  if (B > 0 && h > 0) {
    const bool big = (n_q > 0 && (span_bytes(q, B, h, es) > kMaxSpanBytes ||
                                  span_bytes(o, B, h, es) > kMaxSpanBytes)) ||
                     (n_k > 0 && (span_bytes(k, B, h, es) > kMaxSpanBytes ||
                                  span_bytes(v, B, h, es) > kMaxSpanBytes));
    if (big) return fail(MHA_ERR_SHAPE, "%s: an operand spans more than 2^46 bytes", fn);
  }
  if (z.dtype != MHA_F32 && n_k > 0 &&
      ((__int128)n_k * k.sr * (int64_t)es > kMaxBufferBytes ||
       (__int128)n_k * v.sr * (int64_t)es > kMaxBufferBytes))
    return fail(MHA_ERR_UNSUPPORTED, "%s: one head's K/V rows span more than 2 GiB (n_k %lld)", fn,
                (long long)n_k);
  if (B == 0 || h == 0 || n_q == 0) return ok();
  if (!Q || !O || ((!K || !V) && n_k > 0))
    return fail(MHA_ERR_INVALID_ARG, "%s: null tensor pointer", fn);
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) ||
      (reinterpret_cast<uintptr_t>(seq_lens) & 3) != 0)
    return fail(MHA_ERR_INVALID_ARG, "%s: tensors must be 16-byte aligned", fn);
  const Range ro = span_of(o, B, h, es);
  if (overlap(ro, span_of(q, B, h, es)) || (n_k > 0 && overlap(ro, span_of(k, B, h, es))) ||
      (n_k > 0 && overlap(ro, span_of(v, B, h, es))) ||
      (seq_lens && overlap(ro, range_of(seq_lens, (size_t)B * 4))))
    return fail(MHA_ERR_ALIAS, "%s: O overlaps an input", fn);

  mha::SdpaArgs a{};
  a.Q = Q, a.K = K, a.V = V, a.O = O;
  a.q_sb = q.sb, a.q_sh = q.sh, a.q_sr = q.sr;
  a.k_sb = k.sb, a.k_sh = k.sh, a.k_sr = k.sr;
  a.v_sb = v.sb, a.v_sh = v.sh, a.v_sr = v.sr;
  a.o_sb = o.sb, a.o_sh = o.sh, a.o_sr = o.sr;
  a.B = (int32_t)B, a.H = (int32_t)h, a.n_q = (int32_t)n_q, a.n_k = (int32_t)n_k;
  // c is clamped away from 0: for |scale| this small every visible weight
  // is exp2(~0) = 1 in fp32 (the uniform softmax scale 0 defines), while
  // masked scores (-inf) still give exactly 0
  a.c = std::fmax(std::fabs(z.scale) * 1.4426950408889634f, 1e-30f);
  a.neg = z.scale < 0.f ? 1 : 0;
  a.lens = seq_lens;
  a.window = z.window ? 1 : 0;
  a.win_left = (int32_t)z.left;
  a.win_right = (int32_t)z.right;
  a.reverse = reverse_grid() ? 1 : 0;
  const mha::SdpaRoute r = route_of(z);
  if (trace_on()) {
    double vis = z.mask_kind == MHA_MASK_CAUSAL ? 0.5 * n_q * (n_q + 1) : (double)n_q * n_k;
    if (z.window) {
      vis = 0.0;
      for (int64_t row = 0; row < n_q; ++row) {
        const int64_t lo = row - z.left > 0 ? row - z.left : 0;
        const int64_t hi = row + z.right < n_k - 1 ? row + z.right : n_k - 1;
        if (hi >= lo) vis += (double)(hi - lo + 1);
      }
    }
    std::fprintf(stderr,
                 "[libmha] %s dtype=%d B=%lld h=%lld n_q=%lld n_k=%lld d=%lld mask=%d window=%lld,%lld "
                 "lens=%s strided=%d kernel=%d waves=%d rows/wg=%d wgs=%lld flops(visible)=%.4g "
                 "bytes=%.4g\n",
                 fn, (int)z.dtype, (long long)B, (long long)h, (long long)n_q, (long long)n_k,
                 (long long)d_k, (int)z.mask_kind, z.window ? (long long)z.left : -1LL,
                 z.window ? (long long)z.right : -1LL, seq_lens ? "yes" : "no", st ? 1 : 0, r.kernel,
                 r.waves, r.rows, (long long)r.workgroups, 4.0 * d_k * vis * B * h,
                 (double)es * B * h * (2 * n_q * d_k + 2 * n_k * d_k));
  }
  const hipError_t e = mha::launch_sdpa(a, r, z.dtype, z.mask_kind == MHA_MASK_CAUSAL, (int)d_k,
                                        z.scale, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, fn);
  return ok();
}

int mha_sdpa(const void* Q, const void* K, const void* V, void* O, int32_t dtype, int64_t B,
             int64_t h, int64_t n_q, int64_t n_k, int64_t d_k, int64_t d_v, float scale,
             int32_t mask_kind, const int32_t* seq_lens, void* stream) {
  return sdpa_impl("mha_sdpa", Q, K, V, O, nullptr,
                   SdpaSizes{dtype, B, h, n_q, n_k, d_k, d_v, scale, mask_kind, false, 0, 0},
                   seq_lens, stream);
}

int mha_sdpa_strided(const void* Q, const void* K, const void* V, void* O,
                     const mha_sdpa_strides* strides, int32_t dtype, int64_t B, int64_t h,
                     int64_t n_q, int64_t n_k, int64_t d_k, int64_t d_v, float scale,
                     int32_t mask_kind, const int32_t* seq_lens, void* stream) {
  if (!strides) return fail(MHA_ERR_INVALID_ARG, "mha_sdpa_strided: null strides");
  return sdpa_impl("mha_sdpa_strided", Q, K, V, O, strides,
                   SdpaSizes{dtype, B, h, n_q, n_k, d_k, d_v, scale, mask_kind, false, 0, 0},
                   seq_lens, stream);
}

int mha_sdpa_window(const void* Q, const void* K, const void* V, void* O, int32_t dtype,
                    int64_t B, int64_t h, int64_t n_q, int64_t n_k, int64_t d_k, int64_t d_v,
                    float scale, int64_t left, int64_t right, const int32_t* seq_lens,
                    void* stream) {
  return sdpa_impl("mha_sdpa_window", Q, K, V, O, nullptr,
                   SdpaSizes{dtype, B, h, n_q, n_k, d_k, d_v, scale, MHA_MASK_NONE, true, left, right},
                   seq_lens, stream);
}

int mha_sdpa_window_strided(const void* Q, const void* K, const void* V, void* O,
                            const mha_sdpa_strides* strides, int32_t dtype, int64_t B, int64_t h,
                            int64_t n_q, int64_t n_k, int64_t d_k, int64_t d_v, float scale,
                            int64_t left, int64_t right, const int32_t* seq_lens, void* stream) {
  if (!strides) return fail(MHA_ERR_INVALID_ARG, "mha_sdpa_window_strided: null strides");
  return sdpa_impl("mha_sdpa_window_strided", Q, K, V, O, strides,
                   SdpaSizes{dtype, B, h, n_q, n_k, d_k, d_v, scale, MHA_MASK_NONE, true, left, right},
                   seq_lens, stream);
}

int mha_sdpa_route(int32_t dtype, int64_t B, int64_t h, int64_t n_q, int64_t n_k, int64_t d_k,
                   int64_t d_v, int32_t mask_kind, int32_t windowed, int64_t left, int64_t right,
                   mha_route* route) {
  if (!route) return fail(MHA_ERR_INVALID_ARG, "mha_sdpa_route: null route");
  SdpaSizes z{dtype, B, h, n_q, n_k, d_k, d_v, 1.f, mask_kind, windowed != 0, left, right};
  const int rc = sdpa_sizes("mha_sdpa_route", z);
  if (rc != MHA_OK) return rc;
  const mha::SdpaRoute r = route_of(z);
  route->kernel = r.kernel;
  route->waves = r.waves;
  route->rows_per_workgroup = r.rows;
  route->mask_kind = z.mask_kind;
  route->workgroups = (B == 0 || h == 0 || n_q == 0) ? 0 : r.workgroups;
  return ok();
}

size_t mha_forward_workspace_size(int64_t B, int64_t n_q, int64_t n_k, int64_t d_model,
                                  int32_t h, int32_t dtype) {
  if (B < 0 || n_q < 0 || n_k < 0 || d_model <= 0 || h <= 0 || d_model % h != 0) return 0;
  if (!forward_sizes_in_range(B, n_q, n_k, d_model)) return 0;
  if (dtype != MHA_F32 && dtype != MHA_BF16 && dtype != MHA_F16) return 0;
  return ws_layout(B, n_q, n_k, d_model, dtype).total;
}

// The sublayer; with an_gamma set (mha_forward_add_norm) also its Add &
// Norm: the output projection's epilogue adds the residual x_q and writes
// fp32 rows to the workspace, which the normalisation reads.
static int forward_impl(const char* fn, const void* x_q, const void* x_kv, const void* Wq,
                        const void* Wk, const void* Wv, const void* Wo, const void* an_gamma,
                        const void* an_beta, float an_eps, void* out, int32_t dtype, int64_t B,
                        int64_t n_q, int64_t n_k, int64_t d_model, int32_t h, int32_t mask_kind,
                        const int32_t* kv_lens, void* workspace, size_t workspace_bytes,
                        void* stream, bool noalloc = false) {
  const bool an = an_gamma != nullptr || an_beta != nullptr;
  if (dtype != MHA_F32 && dtype != MHA_BF16 && dtype != MHA_F16)
    return fail(MHA_ERR_DTYPE, "%s: dtype %d", fn, (int)dtype);
  if (mask_kind != MHA_MASK_NONE && mask_kind != MHA_MASK_CAUSAL)
    return fail(MHA_ERR_INVALID_ARG, "%s: mask_kind %d", fn, (int)mask_kind);
  if (B < 0 || n_q < 0 || n_k < 0 || d_model <= 0 || h <= 0)
    return fail(MHA_ERR_SHAPE, "%s: negative or zero size", fn);
  if (d_model % h != 0)
    return fail(MHA_ERR_SHAPE, "%s: d_model %lld not divisible by h %d", fn,
                (long long)d_model, (int)h);
  if (!forward_sizes_in_range(B, n_q, n_k, d_model))
    return fail(MHA_ERR_SHAPE, "%s: size beyond the supported range", fn);
  const bool self = (x_kv == nullptr || x_kv == x_q);
  if (self && n_k != n_q)
    return fail(MHA_ERR_SHAPE, "%s: self-attention needs n_k == n_q", fn);
  if (mask_kind == MHA_MASK_CAUSAL && n_q != n_k)
    return fail(MHA_ERR_SHAPE, "%s: causal mask needs n_q == n_k", fn);
  if (dtype == MHA_F32) return fail(MHA_ERR_UNSUPPORTED, "%s: f32 is not implemented", fn);
  const int64_t d = d_model / h;
  if (d != 16 && d != 32 && d != 64 && d != 128 && d != 256 && d != 512)
    return fail(MHA_ERR_UNSUPPORTED, "%s: head dim %lld (needs 16, 32, 64, 128, 256 or 512)", fn,
                (long long)d);
  if (d_model % 64 != 0)  // the projection GEMMs tile N and K by 64
    return fail(MHA_ERR_UNSUPPORTED, "%s: d_model %lld is not a multiple of 64", fn,
                (long long)d_model);
  if (n_k * d * 2 > kMaxBufferBytes)
    return fail(MHA_ERR_UNSUPPORTED, "%s: one head's K/V exceeds 2 GiB (n_k %lld)", fn,
                (long long)n_k);
  if (an) {
    if (!std::isfinite(an_eps) || an_eps < 0.f)
      return fail(MHA_ERR_INVALID_ARG, "%s: eps must be finite and >= 0", fn);
    if (d_model > mha::kAddNormMaxD)
      return fail(MHA_ERR_UNSUPPORTED, "%s: d_model %lld above %d", fn, (long long)d_model,
                  mha::kAddNormMaxD);
  }
  if (B == 0 || n_q == 0) return ok();
  if (an && (!an_gamma || !an_beta || !aligned16(an_gamma) || !aligned16(an_beta)))
    return fail(MHA_ERR_INVALID_ARG, "%s: gamma and beta must be 16-byte aligned device pointers", fn);
  if (!x_q || !Wq || !Wk || !Wv || !Wo || !out)
    return fail(MHA_ERR_INVALID_ARG, "%s: null tensor pointer", fn);
  if (!aligned16(x_q) || !aligned16(x_kv) || !aligned16(Wq) || !aligned16(Wk) ||
      !aligned16(Wv) || !aligned16(Wo) || !aligned16(out) ||
      (reinterpret_cast<uintptr_t>(kv_lens) & 3) != 0)
    return fail(MHA_ERR_INVALID_ARG, "%s: tensors must be 16-byte aligned", fn);
  const size_t es = elem_size(dtype);
  const WsLayout L = ws_layout(B, n_q, n_k, d_model, dtype);
  const size_t ws_need = an ? L.total_an : L.total;
  if (workspace && workspace_bytes < ws_need)
    return fail(MHA_ERR_WORKSPACE, "%s: workspace %zu bytes, needs %zu", fn, workspace_bytes,
                ws_need);
  if (noalloc && ws_need > (size_t)MHA_NOALLOC_SCRATCH_BYTES)
    return fail(MHA_ERR_WORKSPACE, "%s: these sizes need %zu bytes of scratch, above its %zu", fn,
                ws_need, (size_t)MHA_NOALLOC_SCRATCH_BYTES);
  if (workspace && (reinterpret_cast<uintptr_t>(workspace) & 255) != 0)
    return fail(MHA_ERR_INVALID_ARG, "%s: workspace not 256-byte aligned", fn);
  const size_t wbytes = (size_t)(d_model * d_model) * es;
  const Range ro = range_of(out, (size_t)(B * n_q * d_model) * es);
  if (overlap(ro, range_of(x_q, (size_t)(B * n_q * d_model) * es)) ||
      (!self && overlap(ro, range_of(x_kv, (size_t)(B * n_k * d_model) * es))) ||
      overlap(ro, range_of(Wq, wbytes)) || overlap(ro, range_of(Wk, wbytes)) ||
      overlap(ro, range_of(Wv, wbytes)) || overlap(ro, range_of(Wo, wbytes)) ||
      (kv_lens && overlap(ro, range_of(kv_lens, (size_t)B * 4))) ||
      (workspace && overlap(ro, range_of(workspace, ws_need))) ||
      (an && (overlap(ro, range_of(an_gamma, (size_t)d_model * es)) ||
              overlap(ro, range_of(an_beta, (size_t)d_model * es)))))
    return fail(MHA_ERR_ALIAS, "%s: out overlaps an input or the workspace", fn);

  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  bool owned = false;
  if (noalloc) {  // every argument is valid: the scratch array of this device
    void* p = nullptr;
    const int rc = scratch_on_current_device(fn, &p);
    if (rc != MHA_OK) return rc;
    ws = (char*)p;
    if (overlap(ro, range_of(ws, ws_need)))
      return fail(MHA_ERR_ALIAS, "%s: out overlaps the library's scratch array", fn);
  }
  if (!ws) {
    const hipError_t e = hipMallocAsync((void**)&ws, ws_need, st);
    if (e != hipSuccess) return hip_fail(e, "workspace allocation");
    owned = true;
  }
  const void* xkv = self ? x_q : x_kv;
  void* q_ws = ws + L.q;
  void* k_ws = ws + L.k;
  void* v_ws = ws + L.v;
  void* c_ws = ws + L.concat;

  // (1) projections, head-split store [B, h, n, d]
  mha::GemmArgs g{};
  g.N = (int32_t)d_model;
  g.K = (int32_t)d_model;
  auto split = [&](const void* A, const void* W, void* C, int64_t n) {
    mha::GemmProblem p{};
    p.A = A, p.W = W, p.C = C;
    p.lda = d_model, p.ldw = d_model;
    p.M = (int32_t)(B * n), p.rows_per_b = (int32_t)n, p.head_dim = (int32_t)d;
    p.c_sb = h * n * d, p.c_st = d, p.c_sh = n * d;
    return p;
  };
  g.nprob = 0;
  // short sequences: projections and attention of each head in one launch
  const bool fused = MHA_SHORT_FUSED && d == 64 && n_q <= 64 && n_k >= 1 && n_k <= 64 &&
                     mask_kind == MHA_MASK_NONE;
  if (n_k > 0 && !fused) {
    g.prob[g.nprob++] = split(x_q, Wq, q_ws, n_q);
    g.prob[g.nprob++] = split(xkv, Wk, k_ws, n_k);
    g.prob[g.nprob++] = split(xkv, Wv, v_ws, n_k);
  }
  hipError_t e = hipSuccess;
  if (trace_on())
    std::fprintf(stderr,
                 "[libmha] forward dtype=%d B=%lld n_q=%lld n_k=%lld d_model=%lld h=%d mask=%d "
                 "lens=%s self=%d ws=%zu%s%s\n",
                 (int)dtype, (long long)B, (long long)n_q, (long long)n_k, (long long)d_model,
                 (int)h, (int)mask_kind, kv_lens ? "yes" : "no", self ? 1 : 0, L.total,
                 owned ? " (allocated)" : "", fused ? " fused projections+attention" : "");
  if (g.nprob) e = mha::launch_gemm(g, dtype, st);

  if (fused) {  // (1) + (2) in one launch, into the concat
    mha::ShortArgs a{};
    a.xq = x_q, a.xkv = xkv, a.Wq = Wq, a.Wk = Wk, a.Wv = Wv, a.C = c_ws, a.lens = kv_lens;
    a.B = (int32_t)B, a.H = h, a.n_q = (int32_t)n_q, a.n_k = (int32_t)n_k;
    a.d_model = (int32_t)d_model, a.self = self ? 1 : 0;
    a.c = (1.0f / std::sqrt((float)d)) * 1.4426950408889634f;
    e = mha::launch_mha_short(a, dtype, st);
  }
  // (2) attention per head; output in the concat layout [B, n_q, h·d]
  if (e == hipSuccess && !fused) {
    mha::SdpaArgs a{};
    a.Q = q_ws, a.K = k_ws, a.V = v_ws, a.O = c_ws;
    a.q_sr = d, a.q_sh = n_q * d, a.q_sb = h * n_q * d;
    a.k_sr = d, a.k_sh = n_k * d, a.k_sb = h * n_k * d;
    a.v_sr = d, a.v_sh = n_k * d, a.v_sb = h * n_k * d;
    a.o_sr = d_model, a.o_sh = d, a.o_sb = n_q * d_model;
    a.B = (int32_t)B, a.H = h, a.n_q = (int32_t)n_q, a.n_k = (int32_t)n_k;
    const float scale = 1.0f / std::sqrt((float)d);
    a.c = scale * 1.4426950408889634f;
    a.neg = 0;
    a.lens = kv_lens;
    const mha::SdpaRoute r = mha::sdpa_route(dtype, mask_kind == MHA_MASK_CAUSAL, false, B, h, n_q,
                                             n_k, (int)d, 0, 0);
    e = mha::launch_sdpa(a, r, dtype, mask_kind == MHA_MASK_CAUSAL, (int)d, scale, st);
  }
  // (3) out = concat · Wo
  if (e == hipSuccess) {
    mha::GemmArgs o{};
    o.N = (int32_t)d_model;
    o.K = (int32_t)d_model;
    o.nprob = 1;
    mha::GemmProblem& p = o.prob[0];
    p.A = c_ws, p.W = Wo, p.C = an ? (void*)(ws + L.z) : out;
    p.lda = d_model, p.ldw = d_model;
    p.M = (int32_t)(B * n_q), p.rows_per_b = (int32_t)(B * n_q), p.head_dim = (int32_t)d_model;
    p.c_sb = 0, p.c_st = d_model, p.c_sh = 0;
    if (an) p.R = x_q, p.ldr = d_model;  // z = x_q + concat·Wo, fp32
    e = mha::launch_gemm(o, dtype, st);
  }
  // (4) Add & Norm: out = LayerNorm(z)
  if (an && e == hipSuccess) {
    mha::AddNormArgs a{};
    a.z = ws + L.z, a.gamma = an_gamma, a.beta = an_beta, a.out = out;
    a.rows = B * n_q, a.d = (int32_t)d_model, a.eps = an_eps;
    e = mha::launch_add_norm(a, dtype, true, st);
  }
  if (owned) {
    const hipError_t e2 = hipFreeAsync(ws, st);
    if (e == hipSuccess) e = e2;
  }
  if (e != hipSuccess) return hip_fail(e, fn);
  return ok();
}

int mha_forward(const void* x_q, const void* x_kv, const void* Wq, const void* Wk,
                const void* Wv, const void* Wo, void* out, int32_t dtype, int64_t B,
                int64_t n_q, int64_t n_k, int64_t d_model, int32_t h, int32_t mask_kind,
                const int32_t* kv_lens, void* workspace, size_t workspace_bytes, void* stream) {
  return forward_impl("mha_forward", x_q, x_kv, Wq, Wk, Wv, Wo, nullptr, nullptr, 0.f, out, dtype,
                      B, n_q, n_k, d_model, h, mask_kind, kv_lens, workspace, workspace_bytes,
                      stream);
}

int mha_forward_noalloc(const void* x_q, const void* x_kv, const void* Wq, const void* Wk,
                        const void* Wv, const void* Wo, void* out, int32_t dtype, int64_t B,
                        int64_t n_q, int64_t n_k, int64_t d_model, int32_t h, int32_t mask_kind,
                        const int32_t* kv_lens, void* stream) {
  return forward_impl("mha_forward_noalloc", x_q, x_kv, Wq, Wk, Wv, Wo, nullptr, nullptr, 0.f, out,
                      dtype, B, n_q, n_k, d_model, h, mask_kind, kv_lens, nullptr, 0, stream,
                      /*noalloc=*/true);
}

int mha_forward_add_norm(const void* x_q, const void* x_kv, const void* Wq, const void* Wk,
                         const void* Wv, const void* Wo, const void* gamma, const void* beta,
                         float eps, void* out, int32_t dtype, int64_t B, int64_t n_q, int64_t n_k,
                         int64_t d_model, int32_t h, int32_t mask_kind, const int32_t* kv_lens,
                         void* workspace, size_t workspace_bytes, void* stream) {
  if (!gamma || !beta) return fail(MHA_ERR_INVALID_ARG, "mha_forward_add_norm: null gamma or beta");
  return forward_impl("mha_forward_add_norm", x_q, x_kv, Wq, Wk, Wv, Wo, gamma, beta, eps, out,
                      dtype, B, n_q, n_k, d_model, h, mask_kind, kv_lens, workspace,
                      workspace_bytes, stream);
}

size_t mha_forward_add_norm_workspace_size(int64_t B, int64_t n_q, int64_t n_k, int64_t d_model,
                                           int32_t h, int32_t dtype) {
  if (mha_forward_workspace_size(B, n_q, n_k, d_model, h, dtype) == 0) return 0;
  return ws_layout(B, n_q, n_k, d_model, dtype).total_an;
}

int mha_add_norm(const void* x, const void* sub, const void* gamma, const void* beta, float eps,
                 void* out, int32_t dtype, int64_t rows, int64_t d_model, void* stream) {
  if (dtype != MHA_F32 && dtype != MHA_BF16 && dtype != MHA_F16)
    return fail(MHA_ERR_DTYPE, "mha_add_norm: dtype %d", (int)dtype);
  if (rows < 0 || d_model <= 0) return fail(MHA_ERR_SHAPE, "mha_add_norm: negative or zero size");
  if (rows > ((int64_t)1 << 33)) return fail(MHA_ERR_SHAPE, "mha_add_norm: rows beyond the supported range");
  if (d_model % 4 != 0 || d_model > mha::kAddNormMaxD)
    return fail(MHA_ERR_UNSUPPORTED, "mha_add_norm: d_model %lld (needs a multiple of 4, at most %d)",
                (long long)d_model, mha::kAddNormMaxD);
  if (!std::isfinite(eps) || eps < 0.f)
    return fail(MHA_ERR_INVALID_ARG, "mha_add_norm: eps must be finite and >= 0");
  if (rows == 0) return ok();
  if (!x || !sub || !gamma || !beta || !out)
    return fail(MHA_ERR_INVALID_ARG, "mha_add_norm: null pointer");
  if (!aligned16(x) || !aligned16(sub) || !aligned16(gamma) || !aligned16(beta) || !aligned16(out))
    return fail(MHA_ERR_INVALID_ARG, "mha_add_norm: tensors must be 16-byte aligned");
  const size_t es = elem_size(dtype);
  const size_t rb = (size_t)(rows * d_model) * es;
  const Range ro = range_of(out, rb);
  // in place (out == x or out == sub) is allowed: a row is read whole
  // before it is written; any other overlap is not
  if ((out != x && overlap(ro, range_of(x, rb))) || (out != sub && overlap(ro, range_of(sub, rb))) ||
      overlap(ro, range_of(gamma, (size_t)d_model * es)) ||
      overlap(ro, range_of(beta, (size_t)d_model * es)))
    return fail(MHA_ERR_ALIAS, "mha_add_norm: out partially overlaps x or sub, or overlaps gamma/beta");
  mha::AddNormArgs a{};
  a.x = x, a.sub = sub, a.gamma = gamma, a.beta = beta, a.out = out;
  a.rows = rows, a.d = (int32_t)d_model, a.eps = eps;
  const hipError_t e = mha::launch_add_norm(a, dtype, false, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "mha_add_norm launch");
  return ok();
}

}  // extern "C"
