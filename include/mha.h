/*
 * libmha -- the multi-head attention sublayer of the Transformer on AMD
 * Instinct MI355X (gfx950).  C ABI.
 *
 * Page references (title, section):
 *   [N] nickwang.xyz, "Lire « Attention Is All You Need » : l'article
 *       original du Transformer"
 *   [A] agi-iri.ru, "Attention Is All You Need (на русском)"
 *   [M] ml-canon.vercel.app, "32 Transformer"
 *
 * Conventions shared by every call
 * --------------------------------
 * - Pointers named Q, K, V, O, x_*, W*, out, seq_lens, kv_lens and
 *   workspace are DEVICE pointers (memory of the current HIP device).  The
 *   caller owns every buffer; the library keeps no pointer after a call
 *   returns.
 * - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *   stream).  A status of MHA_OK means the work was validated and enqueued;
 *   faults inside a kernel surface at the caller's next synchronisation.
 * - A call only enqueues kernels on `stream`: no synchronisation, no copy
 *   and no memset.  Unless noted, a call also allocates nothing, so it can
 *   be captured into a HIP graph.  The exceptions are mha_forward and
 *   mha_forward_add_norm given no workspace: they allocate stream-ordered.
 *   Each replay writes what the eager call writes, bit for bit.
 * - Every argument is validated on the host before anything is enqueued, so
 *   an error return never leaves partial output.  Device-side key lengths
 *   cannot be read without a synchronisation; the kernels clamp each one to
 *   [0, n_k].
 * - Tensor pointers must be 16-byte aligned and key-length arrays 4-byte
 *   aligned (MHA_ERR_INVALID_ARG otherwise).
 * - All tensors of a call share one dtype; the output has the input dtype.
 *   Products accumulate in fp32; each output element is rounded once
 *   (round to nearest even).
 * - B = 0, h = 0 or n_q = 0 is a successful no-op.  n_k = 0 or a key length
 *   of 0 gives all-zero output rows (a row with nothing visible).
 * - The library's only mutable state is the device address of the scratch
 *   array of mha_forward_noalloc (looked up once per device, under a lock);
 *   concurrent calls on different streams are safe as long as their buffers
 *   do not overlap (mha_forward_noalloc: see there).
 * - Setting the environment variable MHA_TRACE=1 logs every dispatch
 *   (kernel, grid, algorithmic bytes and flops) to stderr.
 *   MHA_GRID_ORDER=reverse launches the attention workgroups in the opposite
 *   order (a check that results do not depend on it; they are bitwise the
 *   same).
 */
#ifndef LIBMHA_MHA_H
#define LIBMHA_MHA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types.  BF16 and F16 are 2-byte storage; F32 is 4-byte. */
typedef enum { MHA_F32 = 0, MHA_BF16 = 1, MHA_F16 = 2 } mha_dtype;

/* MHA_MASK_CAUSAL: query r sees keys c <= r, the position itself included
 * ([A] §3.2.1; [N] "Trois usages de l'attention dans le modèle", decoder
 * self-attention).  Only defined for n_q == n_k. */
typedef enum { MHA_MASK_NONE = 0, MHA_MASK_CAUSAL = 1 } mha_mask_kind;

/* Status codes. */
enum {
  MHA_OK = 0,
  MHA_ERR_INVALID_ARG = -1, /* null pointer, non-finite scale, bad enum   */
  MHA_ERR_SHAPE = -2,       /* negative/oversized dims, causal n_q != n_k,
                               self-attention n_q != n_k, d_model % h != 0 */
  MHA_ERR_DTYPE = -3,       /* dtype value outside mha_dtype               */
  MHA_ERR_UNSUPPORTED = -4, /* valid but not implemented: head dim, or F32
                               in mha_forward                               */
  MHA_ERR_WORKSPACE = -5,   /* workspace given but smaller than required   */
  MHA_ERR_ALIAS = -6,       /* output overlaps an input or the workspace   */
  MHA_ERR_HIP = -7          /* a HIP runtime call failed (no device, launch
                               failure, allocation failure)                 */
};

/*
 * Scaled dot-product attention, [N] §3.2.1 eq. (1):
 *   O = softmax(scale · Q·Kᵀ + mask) · V, one independent softmax per query
 *   row, masked scores set to -inf before the softmax (weight exactly 0).
 *
 * Layouts (row-major, contiguous):
 *   Q [B, h, n_q, d_k]   K [B, h, n_k, d_k]   V [B, h, n_k, d_v]
 *   O [B, h, n_q, d_v]  (written)
 * seq_lens: NULL, or device int32[B]: batch b uses only its first
 *   seq_lens[b] keys (key padding; clamped to [0, n_k]).  Masked K/V rows
 *   are never read, so their contents (NaN included) have no effect.  A
 *   key masked for a query row (causal, window, padding) has no effect on
 *   that row, even where its value row holds NaN or ±inf; a row that sees
 *   such a key takes its NaN or infinity, as the formula does.
 * scale: any finite float, or NaN for the pages' 1/sqrt(d_k) (computed by
 *   the library in fp32); ±inf is MHA_ERR_INVALID_ARG.
 * Supported: BF16/F16 with d_k = d_v in {16, 32, 64, 128, 256, 512} and
 *   n_k·d_k·2 bytes < 2 GiB (MFMA kernels); F32 with d_k = d_v in {16, 32,
 *   64, 128}.  The head-dimension variants are those of [N] Table 3 row (A)
 *   (d_model fixed, h and d_k = d_model / h varied, down to h = 1).
 * O must not overlap Q, K, V or seq_lens (MHA_ERR_ALIAS).
 */
int mha_sdpa(const void* Q, const void* K, const void* V, void* O, int32_t dtype, int64_t B,
             int64_t h, int64_t n_q, int64_t n_k, int64_t d_k, int64_t d_v, float scale,
             int32_t mask_kind, const int32_t* seq_lens, void* stream);

/*
 * Element strides of the four operands of mha_sdpa_strided and
 * mha_sdpa_window_strided, each [batch, head, row] (the d axis is always
 * contiguous).  A caller's x·W^Q of shape [B, n, h·d] viewed as [B, h, n, d]
 * without a copy has strides {n·h·d, d, h·d} -- the head split of [M] "32
 * Transformer" (the sketch's view and transpose of the projected rows).
 * Strides must be >= 0 and multiples of 8 elements for BF16/F16 (4 for F32),
 * so that every row starts on 16 bytes; 0 repeats an operand (for example one
 * K/V head shared by all query heads).  O's strides must keep distinct
 * (batch, head, row) on distinct elements; and with BF16/F16 a head's n_k
 * K (V) rows must span less than 2 GiB (n_k · row stride · 2 bytes).
 */
typedef struct {
  int64_t q[3], k[3], v[3], o[3];
} mha_sdpa_strides;

/*
 * mha_sdpa on strided operands: the same computation, arguments and errors,
 * with each operand at element (b, i, r, j) = base + b·s[0] + i·s[1] + r·s[2]
 * + j.  O must not overlap the memory any input can touch (the span from its
 * base to its last element), MHA_ERR_ALIAS otherwise.  strides: a host
 * pointer, read during the call; NULL is MHA_ERR_INVALID_ARG.
 */
int mha_sdpa_strided(const void* Q, const void* K, const void* V, void* O,
                     const mha_sdpa_strides* strides, int32_t dtype, int64_t B, int64_t h,
                     int64_t n_q, int64_t n_k, int64_t d_k, int64_t d_v, float scale,
                     int32_t mask_kind, const int32_t* seq_lens, void* stream);

/*
 * Restricted attention, [N] §4 (Table 1, "Auto-attention restreinte", and
 * the text after it): attention limited to a neighbourhood of the output
 * position.  As mha_sdpa without a mask kind, plus the window: key c is
 * visible to query r iff r - left <= c <= r + right (positions are absolute
 * indices; left, right >= 0, else MHA_ERR_INVALID_ARG).  The centred
 * neighbourhood of size 2w + 1 is left = right = w; left >= n_q - 1 with
 * right = 0 is the causal mask; seq_lens masks keys as in mha_sdpa.  A row
 * whose window holds no valid key gives 0.  Only the key tiles inside some
 * row's window are read.  Supported: as mha_sdpa with d_k <= 128.
 */
int mha_sdpa_window(const void* Q, const void* K, const void* V, void* O, int32_t dtype,
                    int64_t B, int64_t h, int64_t n_q, int64_t n_k, int64_t d_k, int64_t d_v,
                    float scale, int64_t left, int64_t right, const int32_t* seq_lens,
                    void* stream);

/* mha_sdpa_window on strided operands, as mha_sdpa_strided. */
int mha_sdpa_window_strided(const void* Q, const void* K, const void* V, void* O,
                            const mha_sdpa_strides* strides, int32_t dtype, int64_t B, int64_t h,
                            int64_t n_q, int64_t n_k, int64_t d_k, int64_t d_v, float scale,
                            int64_t left, int64_t right, const int32_t* seq_lens, void* stream);

/*
 * The kernel an attention call runs on, for the same arguments as mha_sdpa
 * (windowed = 0) or mha_sdpa_window (windowed != 0; left, right its reaches);
 * no device is needed.  Validation and status codes as those calls (sizes
 * only: no pointers).  route (host) receives the kernel, its waves per
 * workgroup, query rows per workgroup and grid size, and the mask kind the
 * call runs with (a window that reaches every earlier key and no later one
 * runs as the causal mask).
 */
enum {
  MHA_KERNEL_F32 = 0,     /* fp32, one or four lanes per query row           */
  MHA_KERNEL_BLOCKS = 1,  /* MFMA flash kernel, two 32-row blocks per wave   */
  MHA_KERNEL_PAIRS = 2,   /* MFMA flash kernel, one 32-row block per wave,
                             two key tiles per step                          */
  MHA_KERNEL_SPLIT = 3,   /* MFMA flash kernel, waves split the keys         */
  MHA_KERNEL_DECODE = 4,  /* one query row, no matrix cores                  */
  MHA_KERNEL_WINDOW = 5,  /* MFMA flash kernel, restricted window            */
  MHA_KERNEL_WIDE = 6     /* d_k 256, 512: 4 waves split the head dimension
                             of a 32-row block; 8 waves: unmasked, two
                             blocks; causal d_k 512, two groups split keys  */
};
typedef struct {
  int32_t kernel, waves, rows_per_workgroup, mask_kind;
  int64_t workgroups;
} mha_route;
int mha_sdpa_route(int32_t dtype, int64_t B, int64_t h, int64_t n_q, int64_t n_k, int64_t d_k,
                   int64_t d_v, int32_t mask_kind, int32_t windowed, int64_t left, int64_t right,
                   mha_route* route);

/*
 * Multi-head attention sublayer, [N] §3.2.2 ("Attention multi-têtes"):
 *   out = Concat(head_1, ..., head_h) · Wo,
 *   head_i = Attention(x_q·Wq_i, x_kv·Wk_i, x_kv·Wv_i) with scale 1/sqrt(d_k).
 * No bias, no dropout, no residual/normalisation (outside the sublayer).
 *
 * Layouts (row-major, contiguous):
 *   x_q  [B, n_q, d_model]            queries' source (decoder side)
 *   x_kv [B, n_k, d_model] or NULL    keys'/values' source; NULL or == x_q
 *                                     means self-attention (n_k must equal n_q);
 *                                     the encoder output for cross-attention
 *   Wq, Wk, Wv [d_model, h·d_k]       multiplied on the right (x·W); head i
 *                                     owns columns [i·d_k, (i+1)·d_k)
 *   Wo [h·d_k, d_model]               row blocks in the same head order
 *   out [B, n_q, d_model]             (written)
 * d_k = d_v = d_model / h.  Supported: BF16/F16 with d_k in {16, 32, 64,
 *   128, 256, 512} and d_model a multiple of 64.
 * mask_kind: NONE (encoder self / cross) or CAUSAL (decoder self).
 * kv_lens: NULL or device int32[B], key padding as in mha_sdpa.
 * workspace: device memory of at least mha_forward_workspace_size() bytes,
 *   256-byte aligned, used for the projected Q/K/V and the concat of heads;
 *   its contents are undefined afterwards.  NULL: the library allocates and
 *   frees stream-ordered (hipMallocAsync / hipFreeAsync) inside the call.
 * out must not overlap any input or the workspace (MHA_ERR_ALIAS).
 */
int mha_forward(const void* x_q, const void* x_kv, const void* Wq, const void* Wk,
                const void* Wv, const void* Wo, void* out, int32_t dtype, int64_t B,
                int64_t n_q, int64_t n_k, int64_t d_model, int32_t h, int32_t mask_kind,
                const int32_t* kv_lens, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes mha_forward needs for these sizes (0 for invalid sizes and
   for sizes mha_forward rejects as beyond its supported range). */
size_t mha_forward_workspace_size(int64_t B, int64_t n_q, int64_t n_k, int64_t d_model,
                                  int32_t h, int32_t dtype);

/*
 * mha_forward for callers that cannot allocate: code being captured into a
 * HIP graph, tight serving loops, harnesses that forbid allocation.  Same
 * computation, arguments (no workspace) and errors as mha_forward; it calls
 * no allocating routine.  Its workspace is a scratch array inside the
 * library, MHA_NOALLOC_SCRATCH_BYTES (32 MiB) on every GPU the library runs
 * on, held until the process ends: sizes whose mha_forward_workspace_size()
 * exceeds it return MHA_ERR_WORKSPACE (the big-model cross-attention
 * sub-layer, B 8, n_q 384, n_k 512, d_model 1024, needs 29.4 MB).  Every
 * call on one GPU shares that GPU's array (each call fully writes what it
 * reads from it, so no clearing is needed): calls that overlap in time on one
 * GPU -- on different streams, or from different threads -- race and must
 * be serialised by the caller.  The array's device address is looked up on
 * the first call on each device (a HIP runtime query, not an allocation).
 */
#define MHA_NOALLOC_SCRATCH_BYTES (32u << 20)
int mha_forward_noalloc(const void* x_q, const void* x_kv, const void* Wq, const void* Wk,
                        const void* Wv, const void* Wo, void* out, int32_t dtype, int64_t B,
                        int64_t n_q, int64_t n_k, int64_t d_model, int32_t h, int32_t mask_kind,
                        const int32_t* kv_lens, void* stream);

/*
 * Residual connection and layer normalisation ("Add & Norm"), [N] the
 * section on the encoder and decoder stacks (paper §3.1): every sub-layer's
 * output is LayerNorm(x + Sublayer(x)), normalisation after the addition.
 * LayerNorm (not written out on the pages; the standard definition) acts on
 * each row of d_model features on its own:
 *   z = x + sub,  mu = mean(z),  var = mean((z - mu)^2),
 *   out = gamma ⊙ (z - mu) / sqrt(var + eps) + beta.
 * Sums and normalisation in fp32, output rounded once to dtype.
 *
 * mha_add_norm: x, sub, out [rows, d_model] row-major, contiguous; gamma,
 *   beta [d_model]; all of dtype (F32, BF16 or F16), device pointers,
 *   16-byte aligned.  out may be x or sub (in place); any other overlap of
 *   out with an input is MHA_ERR_ALIAS.  eps finite and >= 0 (eps = 0 gives
 *   NaN for a constant row, as the formula does).  Supported: d_model a
 *   multiple of 4, at most 4096.  rows = 0 is a no-op.
 */
int mha_add_norm(const void* x, const void* sub, const void* gamma, const void* beta, float eps,
                 void* out, int32_t dtype, int64_t rows, int64_t d_model, void* stream);

/*
 * The attention sub-layer with its Add & Norm:
 *   out = LayerNorm(x_q + MultiHead(x_q, x_kv, x_kv))
 * (the residual is the query-side input: for encoder-decoder attention the
 * decoder stream).  Arguments as mha_forward, plus gamma and beta [d_model]
 * (dtype) and eps as in mha_add_norm; d_model at most 4096.  The output
 * projection adds the residual in its epilogue and keeps x_q + concat·Wo in
 * fp32 (workspace) for the normalisation, so out is rounded once.
 * workspace: at least mha_forward_add_norm_workspace_size() bytes (or NULL:
 * allocated stream-ordered inside the call).
 */
int mha_forward_add_norm(const void* x_q, const void* x_kv, const void* Wq, const void* Wk,
                         const void* Wv, const void* Wo, const void* gamma, const void* beta,
                         float eps, void* out, int32_t dtype, int64_t B, int64_t n_q, int64_t n_k,
                         int64_t d_model, int32_t h, int32_t mask_kind, const int32_t* kv_lens,
                         void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes mha_forward_add_norm needs (0 for invalid sizes and for
   sizes beyond the supported range, as mha_forward_workspace_size). */
size_t mha_forward_add_norm_workspace_size(int64_t B, int64_t n_q, int64_t n_k, int64_t d_model,
                                           int32_t h, int32_t dtype);

/* Static description of a status code (never NULL). */
const char* mha_status_string(int status);

/* Thread-local detail of the last error returned on this thread ("" if
 * none).  Valid until the next libmha call on the same thread. */
const char* mha_last_error(void);

/* Library ABI version: major * 10000 + minor * 100 + patch. */
int mha_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBMHA_MHA_H */
