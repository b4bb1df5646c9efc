/*
 * iskv.h -- C ABI of the MI355X (gfx950) iS-KV compressed KV cache.
 *
 * Method: page "iS-KV: Online Low-Rank KV Cache Compression via
 * Block-Incremental SVD". Each K and each V stream of every
 * (batch, layer, kv-head) keeps
 *   - an exact window of the most recent rows at input precision
 *     (section "Architecture Overview"), and
 *   - a low-rank history C = U Sigma (n x k), sigma (k) and basis B (d x k),
 *     k <= r, updated block by block: the oldest b window rows F are folded
 *     in with one core SVD of Z = [Sigma 0; FB FP], and both the basis and
 *     every stored row's coordinates are rotated and truncated
 *     (section "Block-Incremental Decoding Updates"; equations for Z,
 *     SVD_r(Z), U+ and B+).
 * Decode attention runs on the factors: a history row's score is
 * (C B_K^T) q = C (B_K^T q), and the weighted history values are
 * (p^T C_V) B_V^T, which equals dense attention over the reconstruction of
 * section "Reconstruction and Storage".
 *
 * Conventions for every entry point:
 *   - All data pointers are DEVICE pointers (HIP device memory) unless the
 *     argument says "host". Layouts are row-major and dense.
 *   - `stream` is a hipStream_t passed as void*; NULL means the default
 *     stream. All device work is enqueued on it, in call order; pointers
 *     must stay valid until that work has completed. No entry point
 *     synchronizes except iskv_status.
 *   - The library never allocates device memory: the caller owns the
 *     workspace (sized by iskv_workspace_bytes) and every input/output.
 *     The handle owns host metadata only and is released by iskv_destroy.
 *   - Return value: ISKV_OK (0) or a negative iskv_status. Argument,
 *     capacity and workspace errors are detected on the host before anything
 *     is enqueued and leave the state unchanged. A failed kernel launch
 *     poisons the handle (ISKV_ERR_POISONED from then on). Numeric trouble
 *     inside kernels (core SVD iteration cap, non-finite values) sets sticky
 *     device flags read by iskv_status.
 *   - Counters n (history rows), e (window rows) and k (rank) are kept per
 *     layer; all sequences of a batch advance in lockstep.
 *   - Calls that overlap on the same handle from several host threads race;
 *     serialize them.
 */
#ifndef ISKV_H_
#define ISKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ISKV_API __attribute__((visibility("default")))

typedef enum {
  ISKV_OK = 0,
  ISKV_ERR_ARG = -1,       /* invalid argument or configuration */
  ISKV_ERR_WORKSPACE = -2, /* workspace too small or misaligned */
  ISKV_ERR_CAPACITY = -3,  /* max_tokens would be exceeded */
  ISKV_ERR_HIP = -4,       /* a HIP runtime call failed */
  ISKV_ERR_NUMERIC = -5,   /* returned by iskv_status when a numeric flag is set */
  ISKV_ERR_POISONED = -6,  /* an earlier launch failed; the handle is unusable */
  ISKV_ERR_STATE = -7,     /* call not valid in the current state (e.g. empty cache) */
  ISKV_ERR_SCRATCH = -8    /* the call would need more than the static scratch array */
} iskv_status_code;

/* Bytes of the library's static device array used by iskv_decode_attn_static. */
#define ISKV_STATIC_SCRATCH_BYTES (16u << 20)

/* ISKV_I8 (coordinates only): low-bit history storage, the direction the
 * page's section "Conclusion" names (integration with quantization) with no
 * format given. The history keeps U = C Sigma^-1, the factor the equation for
 * U+ rotates, as int8 codes with one fp32 scale per row: for a row u,
 * scale = max|u| / 127 and code = round-half-even(127 u / max|u|) (a zero row
 * has scale 0); history row i is reconstructed as (code_i * scale_i) Sigma B^T.
 * Every fold stores the rotated old rows and the new rows again. Requires
 * kv_dtype ISKV_BF16, ranks that are multiples of 8, (ncap + 65536) * r < 2^31
 * and the joint update mode. */
typedef enum { ISKV_F32 = 0, ISKV_BF16 = 1, ISKV_I8 = 2 } iskv_dtype;

/* Numeric status flags (bit mask returned by iskv_status). */
#define ISKV_FLAG_SWEEP_CAP 0x1u /* a core SVD stopped at its sweep cap */
#define ISKV_FLAG_NONFINITE 0x2u /* a core produced a non-finite singular value */

/* Update modes. ISKV_MODE_JOINT is the method; the other two are the
 * ablations the pages discuss, for measuring what the joint update buys
 * (section "The Basis Drift Problem", section "Ablation Study"). */
#define ISKV_MODE_JOINT 0        /* basis and every stored row's coordinates rotated together */
#define ISKV_MODE_FIXED_COORDS 1 /* basis updated, stored rows keep their coordinates (drift) */
#define ISKV_MODE_FIXED_BASIS 2  /* once a basis exists it is kept; new rows are stored as
                                    their projections F B, rank and sigma stay */

typedef struct {
  int32_t batch;       /* sequences, >= 1 */
  int32_t layers;      /* >= 1 */
  int32_t kv_heads;    /* >= 1 */
  int32_t q_heads;     /* multiple of kv_heads; query head h reads kv head h / (q_heads/kv_heads) */
  int32_t head_dim;    /* d; must be 128 */
  int32_t block;       /* b, rows per fold; 1 <= b <= 128 */
  int32_t rank_k;      /* r_K, rank budget of keys; 1 <= r_K <= 128 */
  int32_t rank_v;      /* r_V, rank budget of values; 1 <= r_V <= 128 */
  int32_t window;      /* w >= 0: exact rows kept after a fold; w + 2b <= 4096 */
  int32_t max_tokens;  /* per-sequence capacity: n + e <= max_tokens */
  int32_t coord_dtype; /* iskv_dtype of C = U Sigma (ISKV_I8: of U, see above); B and sigma are always fp32 */
  int32_t kv_dtype;    /* iskv_dtype of incoming rows, window, queries and outputs */
} iskv_config;

typedef struct iskv_ctx *iskv_t;

/* Bytes of device workspace needed for `cfg`; 0 if cfg is invalid. */
ISKV_API size_t iskv_workspace_bytes(const iskv_config *cfg);

/* Validate cfg, carve the caller's device workspace `dev_ws` (>= 256-byte
 * aligned, ws_bytes >= iskv_workspace_bytes(cfg)) and clear it on `stream`.
 * On success *out (host) receives a new handle with every layer empty. */
ISKV_API int iskv_init(const iskv_config *cfg, void *dev_ws, size_t ws_bytes, void *stream, iskv_t *out);

/* Forget all tokens (host counters only; state memory is overwritten as the
 * cache refills) and clear the numeric flags on `stream`. */
ISKV_API int iskv_reset(iskv_t h, void *stream);

/* Select the update mode used by later folds of every layer (one of the
 * ISKV_MODE_* values; ISKV_ERR_ARG otherwise, and for any mode other than
 * ISKV_MODE_JOINT with ISKV_I8 coordinates). Host state only; takes effect
 * with the next fold. */
ISKV_API int iskv_set_mode(iskv_t h, int32_t mode);

/* Timing hooks for profiling the fold. `events` is a host array of four
 * hipEvent_t handles (passed as void*) created by the caller; from now on
 * every fold enqueues hipEventRecord(events[0]) before its ingest copy,
 * events[1] before the core kernel, events[2] before the coordinate rewrite
 * and events[3] after it, on the call's stream (when a call folds several
 * layer runs, the events of the last run remain). NULL turns the hooks off.
 * The library neither creates nor destroys the events; they must stay valid
 * while the hooks are on. ISKV_ERR_ARG if a handle is NULL. */
ISKV_API int iskv_set_fold_events(iskv_t h, void *const *events);

/* Append `nrows` (1..b) new K and V rows per sequence and kv head to layers
 * layer0 .. layer0+nlayers-1. k_rows, v_rows: [batch][nlayers][kv_heads][nrows][d]
 * in kv_dtype. Rows enter the exact window; when a layer's window then holds
 * >= w + b rows, its oldest b rows are folded into the history (at most one
 * fold per call). Section "Block-Incremental Decoding Updates". */
ISKV_API int iskv_append_block(iskv_t h, const void *k_rows, const void *v_rows, int32_t nrows,
                      int32_t layer0, int32_t nlayers, void *stream);

/* One-shot prompt compression (section "Prefill Compression"; key and value
 * protection not modelled): the nrows (>= 1) rows per sequence and kv head
 * of layers layer0..layer0+nlayers-1 are factorised at once by a truncated
 * SVD and become the whole history, k = min(r, nrows, d) per stream
 * (section "Theoretical Foundation"); the window stays empty. k_rows,
 * v_rows: [batch][nlayers][kv_heads][nrows][d] in kv_dtype, device memory,
 * read only. Requires every such layer to be empty (n == 0 and e == 0, else
 * ISKV_ERR_STATE) and nrows <= ncap = floor(max_tokens / b) * b, the history
 * capacity in whole blocks (else ISKV_ERR_CAPACITY). nrows need not be a
 * multiple of b. Later appends fold into this history as usual. Long
 * prompts (nrows >= 1024, 16-byte aligned rows) are factorised through the
 * fp64 Gram matrix, kept in these layers' own (empty) coordinate storage when
 * it holds 192 KiB per stream; no memory is allocated. */
ISKV_API int iskv_prefill_oneshot(iskv_t h, const void *k_rows, const void *v_rows, int32_t nrows,
                                  int32_t layer0, int32_t nlayers, void *stream);

/* Prompt compression without a window: fold exactly b rows per sequence and
 * kv head straight into the history of layers layer0..layer0+nlayers-1.
 * Requires every such layer's window to be empty (e == 0). Layout as in
 * iskv_append_block with nrows = b. */
ISKV_API int iskv_prefill_block(iskv_t h, const void *k_rows, const void *v_rows, int32_t layer0,
                       int32_t nlayers, void *stream);

/* Single-token decode attention over history factors plus the exact window
 * for layers layer0..layer0+nlayers-1. Section "Reconstruction and Storage"
 * defines the cached rows X~ (history rows U Sigma B^T, window rows exact);
 * the output is softmax attention over X~, evaluated on the factors
 * (C_K B_K^T q = C_K (B_K^T q) and p^T C_V B_V^T = (p^T C_V) B_V^T): for
 * every query head,
 *   out = softmax(scale * [C_K (B_K^T q); K_win q]) applied to [C_V B_V^T; V_win].
 * q: [batch][nlayers][q_heads][d] in kv_dtype; out: same shape in fp32 (the
 * compute type; rounding it to bf16 would cost up to 2^-8 relative). Every
 * layer in range must hold at least one token (else ISKV_ERR_STATE). */
ISKV_API int iskv_decode_attn(iskv_t h, const void *q, float *out, int32_t layer0, int32_t nlayers,
                     float scale, void *stream);

/* Allocation-free iskv_decode_attn, for callers that cannot allocate device
 * memory or call an allocating routine (code under HIP graph capture, tight
 * serving loops, harnesses that forbid it). Same arguments, layouts and
 * results as iskv_decode_attn (to rounding: the history of each unit is split
 * over several workgroups whose partial softmax sums are merged by
 * log-sum-exp). The partials live in a static device array of
 * ISKV_STATIC_SCRATCH_BYTES owned by the library, one per GPU, held until the
 * process ends; nothing in it needs clearing (each call writes every partial
 * it reads). Calls that overlap on one GPU (any handle, any stream) race on
 * that array: serialize them. Requires bf16 or int8 (ISKV_I8) coordinates,
 * bf16 rows and ranks that are multiples of 8 (else ISKV_ERR_ARG); a call whose partials exceed
 * the array (units x splits x g x (2 + r_V + d) floats, at least one split per
 * unit) returns ISKV_ERR_SCRATCH; ISKV_ERR_HIP if the array's device address
 * could not be obtained at iskv_init. All checks happen before anything is
 * enqueued. This function calls no hipMalloc, hipFree or other allocating
 * routine. */
ISKV_API int iskv_decode_attn_static(iskv_t h, const void *q, float *out, int32_t layer0, int32_t nlayers,
                                     float scale, void *stream);

/* One decode step in one call: append one new K and V row per sequence and
 * kv head (as iskv_append_block with nrows = 1), then decode attention over
 * the updated cache (as iskv_decode_attn), for layers layer0..layer0+nlayers-1.
 * k_rows, v_rows: [batch][nlayers][kv_heads][1][d]; q, out as in
 * iskv_decode_attn. Results are those of the two calls in sequence. When the
 * append does not fold and the bf16 matrix-core decode applies (bf16
 * coordinates and rows, ranks multiples of 8, 16-byte aligned q and rows,
 * window in LDS), a single launch copies the new rows into the window ring
 * and attends over them; otherwise the two calls run. Errors: as the two
 * calls; argument and capacity errors leave the state unchanged. Sections
 * "Block-Incremental Decoding Updates" and "Reconstruction and Storage". */
ISKV_API int iskv_append_decode(iskv_t h, const void *k_rows, const void *v_rows, const void *q, float *out,
                                int32_t layer0, int32_t nlayers, float scale, void *stream);

/* Reconstruction of one unit (section "Reconstruction and Storage"):
 * dev_out [(n+e) x d] fp32 = history rows C B^T, then the window rows
 * oldest first. which: 0 = K, 1 = V. */
ISKV_API int iskv_reconstruct(iskv_t h, int32_t which, int32_t batch, int32_t layer, int32_t head,
                     float *dev_out, void *stream);

/* Host-known counters of a layer (no device access): history rows n, window
 * rows e, key rank k_k and value rank k_v. Pointers are host pointers. */
ISKV_API int iskv_counts(iskv_t h, int32_t layer, int32_t *n, int32_t *e, int32_t *k_k, int32_t *k_v);

/* Copy one unit's state out (device to device): C [n x r] in coord_dtype
 * (columns >= k are zero; with ISKV_I8 the int8 codes of U, whose per-row
 * scales iskv_export_scales copies), sigma [r] fp32, Bt [r x d] fp32 (row j = basis
 * vector j), window [e x d] in kv_dtype oldest first. Any pointer may be NULL
 * to skip that part. */
ISKV_API int iskv_export_state(iskv_t h, int32_t which, int32_t batch, int32_t layer, int32_t head, void *C,
                      float *sigma, float *Bt, void *window, void *stream);

/* Set a layer's counters (host), e.g. before importing a checkpoint (a
 * state exported by iskv_export_state, or one a caller builds, such as a
 * one-shot factorisation of any number of rows). Requires
 * 0 <= n <= floor(max_tokens / b) * b, k_k <= min(r_K, n, d),
 * k_v <= min(r_V, n, d), k > 0 exactly when n > 0, 0 <= e < w + b and
 * n + e <= max_tokens; the window ring restarts at slot 0. */
ISKV_API int iskv_set_counts(iskv_t h, int32_t layer, int32_t n, int32_t e, int32_t k_k, int32_t k_v);

/* Copy one unit's state in (device to device), layouts as iskv_export_state,
 * with the layer's current counters; NULL pointers leave that part as is.
 * The caller is responsible for the state being a valid factorization
 * (orthonormal Bt rows, zero C columns >= k). */
ISKV_API int iskv_import_state(iskv_t h, int32_t which, int32_t batch, int32_t layer, int32_t head,
                      const void *C, const float *sigma, const float *Bt, const void *window,
                      void *stream);

/* ISKV_I8 coordinates only (else ISKV_ERR_ARG): copy one unit's per-row
 * scales of U out, scales [n] fp32 device memory, n = the layer's history rows
 * (see ISKV_I8 for their meaning). Section "Reconstruction and Storage" (the
 * stored history) with the int8 reading above. */
ISKV_API int iskv_export_scales(iskv_t h, int32_t which, int32_t batch, int32_t layer, int32_t head,
                                float *scales, void *stream);

/* ISKV_I8 coordinates only: copy one unit's per-row scales in (device to
 * device), layout as iskv_export_scales, with the layer's current counters;
 * to be used with iskv_import_state. */
ISKV_API int iskv_import_scales(iskv_t h, int32_t which, int32_t batch, int32_t layer, int32_t head,
                                const float *scales, void *stream);

/* Per-unit statistics of each unit's most recent fold (device to device):
 * sweeps [units] int32 = core SVD sweeps; discarded [units] fp32 = energy
 * (sum of squared singular values) dropped by truncation. Units are ordered
 * [layers][batch][kv_heads]. Either pointer may be NULL. */
ISKV_API int iskv_fold_stats(iskv_t h, int32_t which, int32_t *sweeps, float *discarded, void *stream);

/* Synchronize `stream` and read the sticky numeric flags (host *flags).
 * Returns ISKV_ERR_NUMERIC if any flag is set, else ISKV_OK. */
ISKV_API int iskv_status(iskv_t h, void *stream, uint32_t *flags);

/* Release the handle (host memory only; the workspace stays the caller's). */
ISKV_API int iskv_destroy(iskv_t h);

/* Static description of a status code. */
ISKV_API const char *iskv_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* ISKV_H_ */
