/*
 * darkprf.h - C ABI of the MI355X (gfx950) DARKFormer positive-random-feature
 * attention forward pass.
 *
 * What is computed (package README "Data-Aware Random Feature Kernels for
 * Transformers (DARKformer)", darkformer-pytorch 0.1.0):
 *   - section "Kernel", scaled-kernel equation: q and k are scaled by
 *     d_h^(-1/4) inside the library; callers pass unscaled tensors;
 *   - section "Kernel", feature-map equation: for a scaled row x,
 *     phi(x)_j = exp(omega_j^T M x - x^T M^T M x / 2) / sqrt(m);
 *   - section "Kernel", attention equation: out = Phi(Q)(Phi(K)^T V) /
 *     Phi(Q)(Phi(K)^T 1), evaluated associatively;
 *   - section "Self-attention": a boolean key mask (nonzero = valid token),
 *     combined with the causal constraint when causal;
 *   - section "Encoder-decoder model and generation": recurrent statistics
 *     S = sum phi(k) v^T and z = sum phi(k), updated per appended token; a
 *     state is tied to the projection that produced it and a redraw is
 *     rejected;
 *   - section "Mixed precision": reductions accumulate in fp32 and results are
 *     returned in the input dtype.
 *
 * Conventions shared by every entry point:
 *   - Ownership: every pointer is owned by the caller.  Device pointers must
 *     stay valid until the work queued on `stream` has finished.  The library
 *     allocates no device memory and keeps no state between calls; it is safe
 *     to call from several host threads on different streams.
 *   - Asynchrony: compute calls only queue kernels on `stream` (a hipStream_t;
 *     NULL = the default stream) and never synchronise.
 *   - Errors: argument errors are detected on the host, before anything is
 *     queued, and returned as a status; nothing is launched in that case.  A
 *     failed launch is reported as DARK_ERR_HIP.  Nothing throws or aborts.
 *   - Layout: q, k, v and out are addressed as base + b*str[0] + h*str[1] +
 *     l*str[2] + e (elements, e = 0..d_h-1 contiguous).  Device pointers and
 *     every stride must give 16-byte aligned rows.
 *   - dtype: q, k, v and out share desc->dtype.  M, omega and the recurrent
 *     state are fp32.
 */
#ifndef DARKPRF_H
#define DARKPRF_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DARK_OK = 0,
  DARK_ERR_INVALID_ARG = 1,  /* a pointer, size, stride or alignment is wrong */
  DARK_ERR_UNSUPPORTED = 2,  /* a valid combination this build does not serve */
  DARK_ERR_WORKSPACE = 3,    /* workspace missing or smaller than required */
  DARK_ERR_STALE_STATE = 4,  /* recurrent state made with another projection */
  DARK_ERR_HIP = 5           /* the HIP runtime reported an error */
} dark_status;

typedef enum { DARK_F32 = 0, DARK_BF16 = 1 } dark_dtype;

typedef struct {
  int32_t B;          /* batch (number of sequences) */
  int32_t H;          /* query heads */
  int32_t H_kv;       /* key/value heads; H % H_kv == 0; query head h reads kv head h*H_kv/H */
  int32_t L;          /* sequence length (1 for a decode step) */
  int32_t d_h;        /* head dimension: 16, 32, 64, 128 or 256 */
  int32_t m;          /* number of random features, a positive multiple of 16 */
  int32_t r;          /* geometry rank (rows of M, width of omega), 1..256 */
  int32_t dtype;      /* dark_dtype of q, k, v and out */
  int32_t causal;     /* 0: every valid key is visible; 1: key j visible to query t iff j <= t */
  int32_t m_per_head; /* 1: M is [H][r][d_h]; 0: one M [r][d_h] shared by all heads */
  int64_t q_str[3];   /* element strides of q over (b, h, l) */
  int64_t k_str[3];   /* element strides of k over (b, h_kv, l) */
  int64_t v_str[3];   /* element strides of v over (b, h_kv, l) */
  int64_t o_str[3];   /* element strides of out over (b, h, l) */
  uint64_t proj_tag;  /* identifies omega; see dark_prf_proj_tag and dark_prf_proj_tag_per_head */
  int32_t omega_per_head; /* 1: omega is [H][m][r], one projection per query head; 0: one [m][r] shared */
} dark_prf_desc;

/*
 * dark_prf_omega - the random projection omega [m][r] (fp32, row-major, host
 * memory) for a seed.  README section "Kernel" (each omega_j standard
 * Gaussian), section "Self-attention" (orthogonal Gaussian blocks by default,
 * independent Gaussian features otherwise) and section "Projection lifecycle"
 * (a seed makes the projection reproducible).
 *   orthogonal == 0: i.i.d. N(0, 1) entries.
 *   orthogonal != 0: ceil(m / r) blocks of r rows; each block is a Haar
 *     rotation (QR of a Gaussian r x r matrix with the sign of diag(R) moved
 *     into Q) whose rows are rescaled by the norms of independent Gaussian
 *     r-vectors; the last block keeps its first m - r*(blocks-1) rows.
 * Gaussians come from Box-Muller over the SplitMix64 stream of `seed`; the
 * arithmetic is fp64 and the result is rounded once to fp32.  Deterministic
 * for a seed on any machine with IEEE fp64 libm.  Returns
 * DARK_ERR_INVALID_ARG for m < 1, r < 1 or omega_host == NULL.
 */
dark_status dark_prf_omega(uint64_t seed, int32_t m, int32_t r, int32_t orthogonal,
                           float* omega_host);

/*
 * Per-head projections (the projection drawn once per query head instead of
 * once per module; the README keeps the projection a library choice next to
 * the per-head geometry of section "Self-attention").  Head h uses the
 * projection of seed dark_prf_head_seed(seed, h), built exactly as
 * dark_prf_omega builds it, so one seed still makes every head reproducible
 * (section "Projection lifecycle").
 *   dark_prf_head_seed: SplitMix64's finaliser over seed + (h + 1) *
 *     0xD1B54A32D192ED03 (an odd constant other than the redraw sequence's).
 *   dark_prf_omega_per_head: omega_host [H][m][r] (fp32, host memory), head h
 *     equal to dark_prf_omega(dark_prf_head_seed(seed, h), m, r, orthogonal).
 *     DARK_ERR_INVALID_ARG for H < 1, m < 1, r < 1 or omega_host == NULL.
 *   dark_prf_proj_tag_per_head: the tag of the H projections together; it
 *     differs from dark_prf_proj_tag(seed, ...) and between head counts, so a
 *     state made with shared projections is rejected by per-head calls and
 *     the other way round.
 * A call uses per-head projections when desc->omega_per_head = 1: omega is
 * then [H][m][r] contiguous and every query head h uses omega[h] for its
 * queries and for the keys it reads (with GQA, the keys of K/V head
 * h*H_kv/H as seen by h, as with per-head geometry).
 */
uint64_t dark_prf_head_seed(uint64_t seed, int32_t h);
dark_status dark_prf_omega_per_head(uint64_t seed, int32_t H, int32_t m, int32_t r, int32_t orthogonal,
                                    float* omega_host);
uint64_t dark_prf_proj_tag_per_head(uint64_t seed, int32_t H, int32_t m, int32_t r, int32_t orthogonal);

/*
 * dark_prf_omega_device - the same projection as dark_prf_omega, generated on
 * the device into omega [m][r] (fp32, row-major, device memory) on `stream`
 * (README section "Projection lifecycle": a redraw replaces the projection;
 * with this call it stays on the device).  The same stream and construction
 * as dark_prf_omega; the fp64 arithmetic runs in a different order, so results
 * agree with the host's to within an ulp of fp32 or two, not bit for bit.
 * Orthogonal blocks use one workgroup each (fp64 Householder QR in the
 * workspace).  1 <= r <= 256.
 *   dark_prf_omega_device_workspace_bytes: device workspace needed (0 for
 *     i.i.d. entries, and for invalid m or r).
 * Returns DARK_ERR_INVALID_ARG for m < 1, r outside 1..256 or omega == NULL,
 * DARK_ERR_WORKSPACE for a missing or short workspace (it must be 8-byte
 * aligned).
 */
size_t dark_prf_omega_device_workspace_bytes(int32_t m, int32_t r, int32_t orthogonal);
dark_status dark_prf_omega_device(uint64_t seed, int32_t m, int32_t r, int32_t orthogonal,
                                  float* omega, void* workspace, size_t ws_bytes, void* stream);

/*
 * dark_prf_proj_tag - a 64-bit tag naming the projection (seed, m, r,
 * orthogonal).  Store it in desc->proj_tag; states exported by dark_prf_fwd
 * are valid only for calls that carry the same tag.
 */
uint64_t dark_prf_proj_tag(uint64_t seed, int32_t m, int32_t r, int32_t orthogonal);

/*
 * dark_prf_workspace_bytes - device workspace that dark_prf_fwd needs for this
 * descriptor (0 if the descriptor is invalid).  The workspace holds the
 * bf16/fp32 operand copies of M and omega and the partial or per-chunk
 * feature-space states; its contents need no initialisation.
 */
size_t dark_prf_workspace_bytes(const dark_prf_desc* desc);

/*
 * dark_prf_fwd - linear-mode attention over a whole sequence (README section
 * "Kernel", attention equation; section "Self-attention" for mask and causal).
 *   q     [B][H][L][d_h]     (strides q_str), dtype
 *   k, v  [B][H_kv][L][d_h]  (strides k_str, v_str), dtype
 *   M     fp32 [H][r][d_h] when m_per_head, else [r][d_h], contiguous
 *   omega fp32 [m][r], contiguous (e.g. from dark_prf_omega), or [H][m][r]
 *         when desc->omega_per_head (e.g. from dark_prf_omega_per_head)
 *   mask  uint8 [B][L] contiguous, nonzero = valid key, or NULL (all valid);
 *         masked positions are removed as keys; their query rows are still
 *         computed
 *   out   [B][H][L][d_h] (strides o_str), dtype; a row with no visible valid
 *         key is 0
 *   S_out fp32 [B][H][m][d_h] contiguous or NULL; z_out fp32 [B][H][m]
 *         contiguous or NULL: the recurrent state after the last token
 *         (causal only; either both or neither), i.e. S = sum_j phi(k_j) v_j^T
 *         and z = sum_j phi(k_j) over valid keys, ready for
 *         dark_prf_decode_step
 *   workspace, ws_bytes: device scratch of at least dark_prf_workspace_bytes
 * All device pointers are read or written on `stream` only.
 * Precision (bf16 inputs): the feature exponent and |u|^2 from fp16 operands
 * (u and omega, or x with omega M and M, each rounded once to fp16, clamped to
 * +-65504; u itself from bf16 hi/lo parts of M where it is formed) in matrix
 * products with fp32 accumulation; features rounded to bf16 for the
 * contractions, states and sums fp32.  Inputs whose entries (or projections) exceed the fp16 range are
 * outside the supported range.  fp32 inputs: fp32 throughout.
 */
dark_status dark_prf_fwd(const dark_prf_desc* desc, const void* q, const void* k,
                         const void* v, const float* M, const float* omega,
                         const uint8_t* mask, void* out, float* S_out, float* z_out,
                         void* workspace, size_t ws_bytes, void* stream);

/*
 * dark_prf_fwd_noalloc - dark_prf_fwd for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same computation, with the workspace taken from a
 * static device array of DARK_PRF_SCRATCH_BYTES that the library holds on
 * every GPU it runs on until the process ends.  Arguments as for dark_prf_fwd
 * without workspace and ws_bytes.  The call allocates and frees nothing.
 *   - The first call on a device looks up that device's copy of the array
 *     (hipGetSymbolAddress); `stream` must belong to the current device, else
 *     DARK_ERR_INVALID_ARG.
 *   - A call whose dark_prf_workspace_bytes(desc) exceeds
 *     DARK_PRF_SCRATCH_BYTES returns DARK_ERR_WORKSPACE and queues nothing.
 *   - Every call on one GPU shares that GPU's array, whose contents persist
 *     between calls and need no initialisation: calls that overlap in time on
 *     one GPU (several streams, several host threads) race on it and must be
 *     serialised by the caller, e.g. by queueing them on one stream.
 */
#define DARK_PRF_SCRATCH_BYTES (64u << 20)
dark_status dark_prf_fwd_noalloc(const dark_prf_desc* desc, const void* q, const void* k,
                                 const void* v, const float* M, const float* omega,
                                 const uint8_t* mask, void* out, float* S_out, float* z_out,
                                 void* stream);

/*
 * dark_prf_decode_step - append one token to every sequence and emit its
 * output (README section "Encoder-decoder model and generation": recurrent
 * statistics updated per appended token).  desc->B = N sequences, desc->L = 1,
 * desc->causal = 1.
 *   q [N][H][d_h], k, v [N][H_kv][d_h] (strides q_str/k_str/v_str over
 *     (n, h, -); the l-stride is unused), dtype
 *   S fp32 [N][H][m][d_h], z fp32 [N][H][m]: updated in place,
 *     S += phi(k) v^T, z += phi(k); the output reads the updated state:
 *     out = phi(q)^T S / phi(q)^T z (0 when the denominator is 0)
 *   state_tag: the proj_tag the state was made with; it must equal
 *     desc->proj_tag, else DARK_ERR_STALE_STATE and nothing is queued
 *   out [N][H][d_h] (strides o_str), dtype
 */
dark_status dark_prf_decode_step(const dark_prf_desc* desc, const void* q, const void* k,
                                 const void* v, const float* M, const float* omega,
                                 float* S, float* z, uint64_t state_tag, void* out,
                                 void* stream);

/*
 * Cross-attention (README section "Cross-attention": queries attend to a
 * context of another length; query and context masks are separate; there is
 * no causal option.  Section "Encoder-decoder model and generation": decoder
 * cross-attention projects and summarises the encoded source once per layer,
 * and every decoder step reuses that summary).  Two calls: the summary of a
 * context, then any number of query batches against it.  Query head h uses
 * geometry M_h and reads context K/V head h*H_kv/H, as in dark_prf_fwd.
 *
 * dark_prf_context_state - the summary of a context.  desc->L = context
 * length L_k, desc->causal = 0; q_str and o_str are not used.
 *   k, v  [B][H_kv][L_k][d_h]  (strides k_str, v_str), dtype
 *   M, omega as for dark_prf_fwd
 *   context_mask uint8 [B][L_k] contiguous, nonzero = valid context token, or
 *     NULL (all valid); masked tokens are removed as keys
 *   S_out fp32 [B][H][m][d_h], z_out fp32 [B][H][m], contiguous (both
 *     required): S = sum_j phi(k_j) v_j^T and z = sum_j phi(k_j) over the
 *     valid context tokens (all zero when L_k = 0); tagged, like any exported
 *     state, with desc->proj_tag
 *   workspace, ws_bytes: at least dark_prf_workspace_bytes(desc)
 * Returns DARK_ERR_INVALID_ARG for causal != 0 or a missing S_out / z_out.
 */
dark_status dark_prf_context_state(const dark_prf_desc* desc, const void* k, const void* v,
                                   const float* M, const float* omega,
                                   const uint8_t* context_mask, float* S_out, float* z_out,
                                   void* workspace, size_t ws_bytes, void* stream);

/*
 * dark_prf_cross_fwd - queries against a context summary.  desc->L = query
 * length L_q, desc->causal = 0; desc->H, H_kv, d_h, m, r, m_per_head and dtype
 * as for the dark_prf_context_state call that made the summary; k_str and
 * v_str are not used.
 *   q   [B][H][L_q][d_h] (strides q_str), dtype
 *   M, omega as for dark_prf_fwd (the same as for the summary)
 *   S fp32 [B][H][m][d_h], z fp32 [B][H][m], contiguous: the summary (read
 *     only; S is rounded to the input dtype for the products, z stays fp32)
 *   state_tag: the proj_tag the summary was made with; it must equal
 *     desc->proj_tag, else DARK_ERR_STALE_STATE and nothing is queued
 *   query_mask uint8 [B][L_q] contiguous, nonzero = valid query, or NULL;
 *     a masked query row is written as 0
 *   out [B][H][L_q][d_h] (strides o_str), dtype: out_t = phi(q_t)^T S /
 *     phi(q_t)^T z (0 when the denominator is 0)
 *   workspace, ws_bytes: at least dark_prf_workspace_bytes(desc)
 */
dark_status dark_prf_cross_fwd(const dark_prf_desc* desc, const void* q, const float* M,
                               const float* omega, const float* S, const float* z,
                               uint64_t state_tag, const uint8_t* query_mask, void* out,
                               void* workspace, size_t ws_bytes, void* stream);

/*
 * Exact learned-kernel attention (README section "Attention modes": the exact
 * mode evaluates the learned kernel with exact softmax attention, applying the
 * geometry to queries and keys before scaled dot-product attention; "auto"
 * uses it up to a caller-chosen sequence length and the linear mode beyond).
 * With u = d_h^(-1/4) M_h x for every query and key row:
 *   out_t = sum_j w_tj v_j / sum_j w_tj,  w_tj = exp(u_t . u_j),
 * over the keys j that are valid under `mask` and, when desc->causal, j <= t;
 * a row with no such key is 0.  This is the m -> infinity limit of
 * dark_prf_fwd on the same inputs.  Computed with a row-maximum shift and
 * fp32 accumulation; for bf16 inputs the scores u_t . u_j come from u rounded
 * once to fp16 (clamped to +-65504) in fp16 matrix products, and the weights
 * are rounded to the input dtype for the products with V.  omega and desc->m
 * are not used (m must still be valid).
 *
 * dark_prf_exact_workspace_bytes - device workspace dark_prf_exact_fwd needs
 * (M' and the projected rows of q and k); 0 for an invalid descriptor.
 *
 * dark_prf_exact_fwd - arguments as for dark_prf_fwd (q, k, v, M, mask, out,
 * strides and GQA head map); workspace of at least
 * dark_prf_exact_workspace_bytes(desc).
 */
size_t dark_prf_exact_workspace_bytes(const dark_prf_desc* desc);
dark_status dark_prf_exact_fwd(const dark_prf_desc* desc, const void* q, const void* k,
                               const void* v, const float* M, const uint8_t* mask, void* out,
                               void* workspace, size_t ws_bytes, void* stream);

/*
 * "auto" attention mode (README section "Attention modes": exact attention up
 * to and including a caller-chosen sequence length, linear attention beyond
 * it).  With L = desc->L:
 *   L <= exact_threshold: dark_prf_exact_fwd (omega is not used);
 *   L >  exact_threshold: dark_prf_fwd without state export.
 * exact_threshold >= 0 (0: always linear).  No recurrent state is exported:
 * the README keeps full-prefix decoding for the auto and exact modes.
 *   dark_prf_auto_mode: 1 if the call takes the exact path, 0 if the linear
 *     one, -1 for an invalid descriptor or a negative threshold.
 *   dark_prf_auto_workspace_bytes: the workspace of the path taken (0 if
 *     invalid).
 *   dark_prf_auto_fwd: arguments as for dark_prf_fwd without S_out and z_out;
 *     DARK_ERR_INVALID_ARG for a negative threshold; otherwise the status of
 *     the path taken.
 */
int32_t dark_prf_auto_mode(const dark_prf_desc* desc, int32_t exact_threshold);
size_t dark_prf_auto_workspace_bytes(const dark_prf_desc* desc, int32_t exact_threshold);
dark_status dark_prf_auto_fwd(const dark_prf_desc* desc, int32_t exact_threshold, const void* q,
                              const void* k, const void* v, const float* M, const float* omega,
                              const uint8_t* mask, void* out, void* workspace, size_t ws_bytes,
                              void* stream);

/*
 * Projection lifecycle (README section "Projection lifecycle"): a projection
 * stays unchanged unless a redraw is requested; a positive redraw interval
 * redraws after that many training forwards, and evaluation forwards do not
 * advance the schedule; a fixed projection ignores ordinary manual and
 * scheduled redraws, and a forced redraw applies once while fixed; a seed
 * makes the initial projection reproducible; "deterministic" fixes the
 * projection at construction.  Host-side state only: after a redraw the
 * caller regenerates omega from `seed` (dark_prf_omega or
 * dark_prf_omega_device) and uses the new `tag`, so recurrent states and
 * cross-attention summaries made with the old projection are rejected.
 * Draw k uses seed mix(base_seed, k) (SplitMix64's finaliser over base_seed +
 * k * golden ratio; draw 0 uses base_seed itself).  Not thread-safe: one
 * object per module.
 */
typedef struct {
  uint64_t base_seed;  /* the projection seed of draw 0 */
  uint64_t seed;       /* seed of the current draw */
  uint64_t tag;        /* dark_prf_proj_tag(seed, m, r, orthogonal) */
  int64_t draw;        /* index of the current draw (0 = initial) */
  int64_t forwards;    /* training forwards since the current draw */
  int32_t m, r, orthogonal;
  int32_t interval;    /* redraw after this many training forwards; <= 0: never */
  int32_t fixed;       /* 1: ordinary redraws are ignored */
} dark_prf_projection;

/* dark_prf_projection_init - draw 0 from `seed`; DARK_ERR_INVALID_ARG for
 * p == NULL, m < 1 or r < 1. */
dark_status dark_prf_projection_init(dark_prf_projection* p, uint64_t seed, int32_t m, int32_t r,
                                     int32_t orthogonal, int32_t redraw_interval,
                                     int32_t deterministic);
/* dark_prf_projection_forward - call once before each forward.  Training
 * forwards (training != 0) count toward the interval: when the count has
 * reached it and the projection is not fixed, the projection is redrawn first
 * and the count restarts.  Returns 1 if a redraw happened (the caller must
 * regenerate omega), 0 if not, -1 for p == NULL. */
int32_t dark_prf_projection_forward(dark_prf_projection* p, int32_t training);
/* dark_prf_projection_redraw - a manual redraw; ignored while fixed unless
 * force != 0.  Returns 1 if a redraw happened, 0 if not, -1 for p == NULL. */
int32_t dark_prf_projection_redraw(dark_prf_projection* p, int32_t force);
/* dark_prf_projection_fix - fixed != 0 fixes the projection, 0 unfixes it. */
dark_status dark_prf_projection_fix(dark_prf_projection* p, int32_t fixed);

/*
 * Backward pass of dark_prf_fwd: gradients of a scalar loss with respect to
 * q, k, v and the geometry M, given dout = d loss / d out.  README section
 * "Kernel" has M learned (and the DARKFormer abstract pages finetune the q-k-v
 * projections with the projection covariance, Figure 4); omega is a fixed
 * draw and gets no gradient.  The pages give no backward formulas: these are
 * the chain rule through out = N / D, N = W V, D = W 1 with
 * W[t][j] = phi(q_t) . phi(k_j) over the visible keys (mask, causal), the
 * feature map phi and u = d_h^(-1/4) M_h x.  A query row with no visible key
 * (out fixed at 0) gets no gradient; a masked key gets dk = dv = 0.
 *
 * dark_prf_bwd_workspace_bytes - device workspace dark_prf_bwd needs for
 * desc; 0 for an invalid descriptor, and 0 for B = 0 (dark_prf_bwd then
 * only zeroes dM and takes no workspace).  It holds the fp32 features, the
 * per-chunk states and the intermediate gradients, and grows linearly in
 * B*H*L (with the chunk length C = 64, or 128 for causal calls with
 * d_h >= 128, and L rounded up to a multiple of C); size the workspace with
 * this call rather than from a formula.
 *
 * dark_prf_bwd - arguments as for dark_prf_fwd, plus:
 *   dout  [B][H][L][d_h] (strides o_str), dtype
 *   dq    [B][H][L][d_h] (strides q_str), dtype, overwritten
 *   dk, dv [B][H_kv][L][d_h] (strides k_str, v_str), dtype, overwritten; with
 *         H_kv < H they sum over the query heads that share the key/value head
 *   dM    fp32, shaped like M ([H][r][d_h] or [r][d_h], contiguous),
 *         overwritten; a shared M sums over heads; summed over the batch
 *   workspace, ws_bytes: at least dark_prf_bwd_workspace_bytes(desc)
 * Intermediates are fp32.  The products run on the fp32 matrix cores, except
 * that for bf16 inputs the plain matrix products (not the feature exponents
 * and not the intra-chunk scores) run on the bf16 matrix cores with each fp32
 * operand split into a bf16 high part and a bf16 remainder (three products,
 * about 16 significant bits per operand).  dq, dk and dv are rounded to the
 * input dtype once at the end.  Error codes as for dark_prf_fwd.
 */
size_t dark_prf_bwd_workspace_bytes(const dark_prf_desc* desc);
dark_status dark_prf_bwd(const dark_prf_desc* desc, const void* q, const void* k, const void* v,
                         const float* M, const float* omega, const uint8_t* mask, const void* dout,
                         void* dq, void* dk, void* dv, float* dM, void* workspace, size_t ws_bytes,
                         void* stream);

/* dark_prf_status_str - a static, human-readable name of a status. */
const char* dark_prf_status_str(dark_status status);

/*
 * Diagnostics: GPU time of each kernel the library launches, taken with HIP
 * events recorded on the caller's stream around every launch.  Not needed for
 * computation and off by default; while on, each launch costs two event
 * records.  Process-wide; the two calls are serialised by a lock.
 *   dark_prf_timing_begin: start recording (drops anything recorded before).
 *   dark_prf_timing_end: wait for the recorded events, write the summed
 *     milliseconds and the launch count of every kernel kind into
 *     ms[DARK_KERNEL_KINDS] and launches[DARK_KERNEL_KINDS] (host arrays),
 *     and stop recording.  Returns DARK_ERR_INVALID_ARG for NULL arrays and
 *     DARK_ERR_HIP if an event failed.
 * Kernel kinds: 0 operand preparation of M and omega, 1 key-side feature
 * state, 2 state sum / prefix scan, 3 query-side output, 4 decode step,
 * 5 exponent shift pass (the per-token maxima of the folded exponent),
 * 6 backward matrix products, 7 backward element-wise passes and chunk scans.
 */
#define DARK_KERNEL_KINDS 8
dark_status dark_prf_timing_begin(void);
dark_status dark_prf_timing_end(double* ms, int32_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* DARKPRF_H */
