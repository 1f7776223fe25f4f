/*
 * stc.h -- C ABI of the spectral transform KV-cache codec for MI355X (gfx950).
 *
 * What the codec computes (sources are cited by page title and section):
 *
 *  - Calibration. Per stream (one layer / batch / KV head / K-or-V), the
 *    uncentred second moment of representative tokens is diagonalised; the
 *    tokens are coded in its energy-ordered orthonormal eigenbasis.
 *    ("Sintesi Tecnica: SPECTRA", gist.science, "Metodologia" observations 1
 *    and 3, "La Pipeline di SPECTRA" step 1; Dutch ablation summary
 *    "Technisch Overzicht: Ablatie ...", "Experimentele Opstelling",
 *    SpectralQuant: a per-head eigenbasis calibrated on representative tokens.)
 *  - Allocation. Integer bits per latent channel by reverse water-filling on
 *    the eigenvalues; 0-bit channels are dropped. (SPECTRA summary,
 *    "Metodologia" observation 2, "La Pipeline" step 2.)
 *  - Encode. Each token is projected onto the basis, each kept channel is
 *    scalar-quantized independently and the codes are appended to the stream.
 *    (SPECTRA summary, "La Pipeline" step 3.)
 *  - Decode / attention. Codes are unpacked, dequantized and rotated back; a
 *    decode-step attention reads the packed K/V directly. (SPECTRA summary,
 *    "La Pipeline" step 3 and "Significato e Rivendicazioni"; SPECTRA abstract,
 *    arxivdaily.com: the cache is re-read in full at every generated token.)
 *  - Comparison path. A randomized Walsh-Hadamard rotation with a fixed
 *    Lloyd-Max codebook on every channel (Dutch ablation summary,
 *    "Experimentele Opstelling", TurboQuant).
 *
 * Readings of the pages fixed by this library (the pages leave them open):
 *  - second moment over the first n_calib tokens, no mean removed;
 *  - eigenvalues descending; each eigenvector's largest-magnitude entry made
 *    positive (lowest row index on a tie);
 *  - water-filling is the greedy integer allocation under the model
 *    D_j(b) = lambda_j 4^-b with widths 0..8, ties to the lowest channel,
 *    total bits per token B = floor(avg_bits * d + 0.5);
 *  - a kept channel j with L = 2^b_j levels uses the midrise uniform quantizer
 *    with step delta_j = sqrt(lambda_j) * delta*(b_j), delta*(b) being the
 *    MSE-optimal step for a unit Gaussian; the code is the number of
 *    thresholds t_k = fl32((k - L/2) delta_j), k = 1..L-1, with t_k <= fl32(c)
 *    (NaN -> 0); the level of code q is (q - (L-1)/2) delta_j;
 *  - packed format F1: token t occupies stream bits [t*B, (t+1)*B); kept
 *    channels in ascending index take bits [o_j, o_j + b_j), least
 *    significant bit first; stream bit i is bit (i & 7) of byte (i >> 3); a
 *    stream of n tokens is ceil(n*B/8) bytes, zero-padded to a multiple of 16;
 *  - decode output is rounded to the stream dtype (bf16: round to nearest even);
 *  - the Walsh-Hadamard path stores each token's L2 norm as fp32 next to the
 *    codes, rotates y = H D (x / |x|) / sqrt(d) (H Sylvester order, D = +-1)
 *    and codes every channel with 3 bits against the fp32 midpoints of an
 *    8-entry fp32 codebook.
 *
 * Conventions for every call:
 *  - d must be 128 on the GPU path (STC_EUNSUPPORTED otherwise).
 *  - All buffers are owned by the caller. Pointers named *_dev are device
 *    memory (HBM) of the current HIP device; all other pointers are host
 *    memory. The library allocates no device memory.
 *  - Arguments are validated before any device work; on an error nothing is
 *    written and the status says why (see stc_last_error for a message).
 *  - Device work is enqueued on the given stream and is asynchronous unless a
 *    call says it synchronizes. Asynchronous faults surface at the caller's
 *    next synchronization.
 *  - A state is a device blob of stc_state_bytes() bytes (256-byte aligned)
 *    plus a host stc_head_info written by the same call. Batched calls take
 *    an array of states laid out back to back (stride stc_state_bytes()).
 */
#ifndef STC_H
#define STC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* stc_stream_t; /* a hipStream_t; NULL = default stream */

typedef int32_t stc_status;
enum {
  STC_OK = 0,
  STC_EINVAL = -1,       /* null pointer, bad size, stride or alignment */
  STC_EUNSUPPORTED = -2, /* d != 128, unknown dtype or transform */
  STC_EBUDGET = -3,      /* bit vector does not sum to the budget, a width > 8,
                            or budget > 8 d */
  STC_EWORKSPACE = -4,   /* workspace too small */
  STC_EDEVICE = -5       /* a HIP call failed */
};

enum { STC_F32 = 0, STC_BF16 = 1 };                                   /* K/V dtype */
enum { STC_XFORM_EIGEN = 0, STC_XFORM_IDENTITY = 1, STC_XFORM_RHT = 2 }; /* transform */

#define STC_D 128
#define STC_MAX_BITS 8
#define STC_RHT_BITS 3
#define STC_SKETCH_BITS 128  /* bits of the key residual sketch per token (Walsh-Hadamard path) */

/* Host-side summary of a state, written by the calls that build one. */
typedef struct {
  int32_t d;            /* head dimension (128) */
  int32_t xform;        /* STC_XFORM_* */
  int32_t total_bits;   /* B, bits per token record */
  int32_t n_kept;       /* channels with a non-zero width */
  uint8_t bits[STC_D];  /* width of each latent channel (0..8) */
  double lambda[STC_D]; /* second-moment eigenvalues (EIGEN), diagonal (IDENTITY) */
  double steps[STC_D];  /* quantizer step of each kept channel (0 if dropped) */
  int32_t sketch_bits;  /* RHT states: bits of the key residual sketch per token (0: none) */
} stc_head_info;

/* ------------------------------------------------------------ sizes */
size_t stc_state_bytes(void);
/* ceil(n_tokens * total_bits / 8) rounded up to a multiple of 16 (format F1). */
size_t stc_packed_bytes(int32_t total_bits, int64_t n_tokens);
/* Workspace of stc_attend_compressed_batched: the per-split partial results
 * (written by one kernel, merged by the next) and the per-pair score weights
 * of the packed-bit kernel (written by a kernel that runs before it). It
 * needs no initialisation and can be reused by later calls of any shape in
 * stream order (not by calls that run at the same time). */
size_t stc_attend_workspace_bytes(int64_t n_pairs, int32_t group, int64_t n_tokens);

/* ------------------------------------------------------- host math
 * These run on the host only and need no GPU.                        */

/* floor(avg_bits * d + 0.5). */
int32_t stc_total_bits(float avg_bits, int32_t d);

/* MSE-optimal step of the 2^bits-level midrise uniform quantizer for N(0,1),
 * bits in 1..8 (returns NaN otherwise). */
double stc_delta_star(int32_t bits);

/* Greedy reverse water-filling: total_bits bits over d channels, one at a time
 * to argmax lambda_j 2^(-2 b_j) among b_j < 8 (lambda <= 0 counts as 0; ties
 * to the lowest j). bits_out[d]. STC_EBUDGET if total_bits > 8 d or < 0. */
stc_status stc_water_fill(int32_t d, const double* lambda, int32_t total_bits, uint8_t* bits_out);

/* Allocation variants, all calibrate-time choices feeding the same
 * quantizer, format and kernels (pass the result as `bits` to
 * stc_calibrate_head / stc_state_init):
 *  GREEDY       stc_water_fill (param unused);
 *  OPERATIONAL  greedy on the quantizer's own distortion: each bit to
 *               argmax lambda_j (eps(b_j) - eps(b_j + 1)), eps(b) the MSE of
 *               the b-bit quantizer on a unit Gaussian, eps(0) = 1 (SPECTRA
 *               summary, "La Pipeline" step 2; param unused);
 *  GROUPED      one width per group of param adjacent channels (param
 *               divides d), greedy on the group variance sums, param bits per
 *               step while at least param bits remain ("Raggruppamento");
 *  FLOOR        param bits on every channel, the rest greedy (ablation
 *               summary, "Opslag vs. Kwaliteit": tail floor);
 *  GAP          spectral-gap pruning: d_eff = 1 + the first j with
 *               lambda_j >= param * lambda_{j+1} (param > 1; a positive
 *               lambda_j before a non-positive one counts), channels from
 *               d_eff on get 0 bits, the others share min(budget, 8 d_eff)
 *               greedily (ablation summary, d_eff).
 * Ties to the lowest index, lambda <= 0 counts as 0. Errors: STC_EBUDGET for
 * a budget outside [0, 8d], STC_EINVAL for a bad variant or param. */
enum { STC_ALLOC_GREEDY = 0, STC_ALLOC_OPERATIONAL = 1, STC_ALLOC_GROUPED = 2, STC_ALLOC_FLOOR = 3,
       STC_ALLOC_GAP = 4 };
stc_status stc_allocate_bits(int32_t d, const double* lambda, int32_t total_bits, int32_t variant,
                             double param, uint8_t* bits_out);

/* Symmetric eigendecomposition A = U diag(lambda) U^T (cyclic Jacobi, fp64),
 * lambda descending, columns sign-fixed as above. A, U row-major d*d. */
stc_status stc_eigh(int32_t d, const double* a, double* u_out, double* lambda_out);

/* Lloyd's algorithm on training samples for a `levels`-entry scalar codebook:
 * start at the sample quantiles (k+1/2)/levels (linear interpolation between
 * order statistics), thresholds = midpoints, centroids = cell means (a sample
 * equal to a threshold joins the upper cell); stop once no centroid moves by
 * tol or more, or after max_iter rounds. centroids_out[levels], ascending. */
stc_status stc_lloyd_max(const double* samples, int64_t n, int32_t levels, double tol,
                         int32_t max_iter, double* centroids_out, int32_t* iters_out);

/* ------------------------------------------------------- states */

/* Build a state from a given basis (EIGEN: u row-major d*d, column j = latent
 * channel j; IDENTITY: u must be NULL), its variances and a bit vector.
 * steps NULL: steps_j = sqrt(max(lambda_j,0)) * delta*(b_j); otherwise the
 * given steps are used (e.g. to reproduce another implementation's state).
 * Fills *info and state_dev; synchronizes `stream`. */
stc_status stc_state_init(int32_t d, int32_t xform, const double* u, const double* lambda,
                          const uint8_t* bits, const double* steps, stc_head_info* info,
                          void* state_dev, stc_stream_t stream);

/* stc_state_init plus a selective residual sketch of the keys (SpectralQuant
 * applies its QJL sketch only on the leading effective dimensions; ablation
 * summary, "Experimentele Opstelling"): sketch[i*d + j] = S_ij (host fp32, finite,
 * STC_SKETCH_BITS x d). The sketch covers r = c - c_hat on the kept channels
 * with a positive step (latent basis; 0 elsewhere): stc_sketch_kv_batched
 * writes sign(S r) and |r| per token, stc_attend_compressed_sketch_batched
 * adds sqrt(pi/2)/STC_SKETCH_BITS |r_t| (S U^T q).z_t to each score. The
 * sketch matrices take the place of the state's fp32 threshold table (which
 * no kernel reads). Synchronizes `stream`. */
stc_status stc_state_init_sketch(int32_t d, int32_t xform, const double* u, const double* lambda,
                                 const uint8_t* bits, const double* steps, const float* sketch,
                                 stc_head_info* info, void* state_dev, stc_stream_t stream);

/* Build a Walsh-Hadamard state: signs[d] in {-1,+1}, codebook[8] fp32
 * ascending. Fills *info and state_dev; synchronizes `stream`. */
stc_status stc_rht_state_init(int32_t d, const int8_t* signs, const float* codebook,
                              stc_head_info* info, void* state_dev, stc_stream_t stream);

/* A Walsh-Hadamard state whose keys also carry a 1-bit Johnson-Lindenstrauss
 * sketch of their residual (TQ-QKV; ablation summary, "Experimentele
 * Opstelling" and "Belangrijkste Bijdragen" 1): sketch[i*d + j] = S_ij, the
 * STC_SKETCH_BITS x d Gaussian matrix of the stream (host fp32, finite). The
 * encode then also writes z = sign(S r) of r = x - K_hat (STC_SKETCH_BITS
 * bits per token, one per row, 1 = non-negative) and |r| (fp32), and the
 * attention adds sqrt(pi/2)/m |r_t| (S q).z_t to each score. Synchronizes
 * `stream`. */
stc_status stc_rht_sketch_state_init(int32_t d, const int8_t* signs, const float* codebook,
                                     const float* sketch, stc_head_info* info, void* state_dev,
                                     stc_stream_t stream);

/* Calibrate one stream (SPECTRA summary, "Metodologia" observations 1-3 and
 * "La Pipeline di SPECTRA" steps 1-2: the basis diagonalises the second
 * moment of representative tokens, bits follow the eigenvalues by reverse
 * water-filling; ablation summary, "Experimentele Opstelling": one such
 * eigenbasis per head): second moment of the first n_calib tokens of x_dev
 * ([n][ld] of dtype, row t at x_dev + t*ld elements) computed on the GPU in
 * fp64, eigendecomposition on the host (EIGEN) or its diagonal (IDENTITY),
 * water-filling of floor(avg_bits*d+0.5) bits unless `bits` (host, d widths)
 * is given, then as stc_state_init. Synchronizes `stream`. */
stc_status stc_calibrate_head(int32_t d, int64_t n_calib, const void* x_dev, int32_t dtype,
                              int64_t ld, float avg_bits, const uint8_t* bits, int32_t xform,
                              stc_head_info* info, void* state_dev, stc_stream_t stream);

/* Calibrate n_streams heads in one call (same SPECTRA summary passages as
 * stc_calibrate_head): stream s takes the first n_calib rows at
 * x_dev + s * x_stream_stride elements (row stride ld, dtype STC_BF16 or
 * STC_F32), its widths by stc_water_fill of avg_bits, and its state goes to
 * states_dev + s * stc_state_bytes() (256-byte aligned; the layout of the
 * batched calls) with its summary in infos[s]. One launch forms every second
 * moment; the eigenbases, widths and blobs are then built on host threads
 * and uploaded, 256 streams at a time (host memory stays near 160 MB). Each state equals the one stc_calibrate_head would
 * build from the same rows. Synchronizes `stream`. A failing stream (a
 * non-finite second moment, ...) returns its status, names the stream in
 * stc_last_error and leaves the states undefined. */
stc_status stc_calibrate_heads_batched(int32_t d, int64_t n_streams, int64_t n_calib,
                                       const void* x_dev, int32_t dtype, int64_t ld,
                                       int64_t x_stream_stride, float avg_bits, int32_t xform,
                                       stc_head_info* infos, void* states_dev, stc_stream_t stream);

/* Read back a state's basis as fp32, row-major d*d (u[i*d+j] = U_ij).
 * Synchronizes `stream`. */
stc_status stc_state_basis(const void* state_dev, float* u_out, stc_stream_t stream);

/* ---------------------------------------------------------- codec
 * Batched layout: stream s uses state (state_of_stream_dev ? map[s] : s) of
 * the states array; its tokens are x_dev + s*x_stream_stride (elements), row t
 * at + t*ld; its packed bytes are packed_dev + s*packed_stream_stride; its
 * norms (Walsh-Hadamard states only) norms_dev + s*n_tokens. All streams of a
 * call have n_tokens tokens and use states of one family (all EIGEN/IDENTITY,
 * or all RHT). infos[n_states] are the host summaries of the states, used for
 * validation (packed_stream_stride must hold the largest stream) and to size
 * and choose the kernels' on-chip layouts: each must be the one
 * stc_calibrate_head or stc_state_init gave for its state; one that disagrees with
 * its state is undefined behaviour.
 * x rows must be 16-byte aligned (ld*elem and x_stream_stride*elem multiples
 * of 16); packed_stream_stride a multiple of 16.
 * A map entry outside [0, n_states) is read on the device only, so the call
 * still returns STC_OK: its stream is never coded with another state (encode,
 * append and sketch leave its bytes untouched, decode writes NaN rows, the
 * attention calls write NaN outputs); stc_check_state_map reports such
 * entries on the host.                                                   */

/* Encode: project every token onto its stream's basis, quantize each kept
 * channel on its own and pack the codes as F1 records (SPECTRA summary, "La
 * Pipeline di SPECTRA" step 3: tokens are projected into the latent space and
 * quantized per token). Walsh-Hadamard states also write each token's fp32
 * norm to norms_dev + s*n_tokens (ablation summary, "Experimentele
 * Opstelling": the rotated unit vector meets a data-independent codebook). */
stc_status stc_encode_kv_batched(const void* states_dev, int64_t n_states,
                                 const int32_t* state_of_stream_dev, const stc_head_info* infos,
                                 int64_t n_streams, int64_t n_tokens, const void* x_dev,
                                 int32_t dtype, int64_t ld, int64_t x_stream_stride,
                                 void* packed_dev, int64_t packed_stream_stride,
                                 float* norms_dev, stc_stream_t stream);

/* Decode: unpack, dequantize (level (q - (L-1)/2) step) and rotate back,
 * x_hat = U c_hat, rounded to dtype into x_out_dev + s*x_stream_stride, row t
 * at + t*ld (SPECTRA summary, "La Pipeline di SPECTRA" step 3: keys and
 * values are rebuilt on the fly). Walsh-Hadamard states read the norms at
 * norms_dev + s*n_tokens. */
stc_status stc_decode_kv_batched(const void* states_dev, int64_t n_states,
                                 const int32_t* state_of_stream_dev, const stc_head_info* infos,
                                 int64_t n_streams, int64_t n_tokens, const void* packed_dev,
                                 int64_t packed_stream_stride, const float* norms_dev,
                                 void* x_out_dev, int32_t dtype, int64_t ld,
                                 int64_t x_stream_stride, stc_stream_t stream);

/* Append m tokens to streams that already hold n_old (the cache is
 * append-only, each token quantized on its own when it arrives: SPECTRA
 * summary, "La Pipeline", steps 2-3). x row r of stream s is its token
 * n_old + r; the records go to stream bits [(n_old + r) B, (n_old + r + 1) B).
 * Bits of the first n_old records are kept, every byte from there up to
 * packed_bytes(B, n_old + m) is rewritten (F1 zero padding included), so
 * after the call the stream equals one encode of all n_old + m tokens.
 * packed_stream_stride must hold n_old + m tokens; Walsh-Hadamard norms go to
 * norms_dev + s*norms_stream_stride + n_old + r. Same layout rules and errors
 * as stc_encode_kv_batched; m = 0 does nothing. */
stc_status stc_append_kv_batched(const void* states_dev, int64_t n_states,
                                 const int32_t* state_of_stream_dev, const stc_head_info* infos,
                                 int64_t n_streams, int64_t n_old, int64_t m, const void* x_dev,
                                 int32_t dtype, int64_t ld, int64_t x_stream_stride,
                                 void* packed_dev, int64_t packed_stream_stride,
                                 float* norms_dev, int64_t norms_stream_stride, stc_stream_t stream);

/* stc_append_kv_batched (n_old = 0: a plain encode) for Walsh-Hadamard
 * states built by stc_rht_sketch_state_init, bf16 tokens, also writing each
 * token's key residual sketch (STC_SKETCH_BITS / 8 bytes at sketch_dev +
 * s*sketch_stream_stride + t*16, row i at bit i, 1 = non-negative,
 * sign(0) = +1) and |r| (fp32 at rnorm_dev + s*rnorm_stream_stride + t).
 * Streams whose state has no sketch matrix get codes and norms only (their
 * sketch bytes and residual norms are not written); STC_EINVAL if no state
 * of the array has one. */
stc_status stc_append_rht_sketch_batched(const void* states_dev, int64_t n_states,
                                        const int32_t* state_of_stream_dev, const stc_head_info* infos,
                                        int64_t n_streams, int64_t n_old, int64_t m, const void* x_dev,
                                        int64_t ld, int64_t x_stream_stride, void* packed_dev,
                                        int64_t packed_stream_stride, float* norms_dev,
                                        int64_t norms_stream_stride, void* sketch_dev,
                                        int64_t sketch_stream_stride, float* rnorm_dev,
                                        int64_t rnorm_stream_stride, stc_stream_t stream);

/* The selective residual sketch of tokens [n_old, n_old + m) of eigen /
 * identity streams (bf16 tokens, x row r = token n_old + r) whose states
 * were built by stc_state_init_sketch: recomputes the cells and codes the
 * encode gives those tokens (it does not read the packed stream), then writes
 * sign(S r) (STC_SKETCH_BITS / 8 bytes at sketch_dev + s*sketch_stream_stride
 * + t*16, row i at bit i, 1 = non-negative) and |r| (fp32 at rnorm_dev +
 * s*rnorm_stream_stride + t). Streams whose state has no sketch matrix are
 * left untouched; STC_EINVAL if no state has one. */
stc_status stc_sketch_kv_batched(const void* states_dev, int64_t n_states,
                                const int32_t* state_of_stream_dev, const stc_head_info* infos,
                                int64_t n_streams, int64_t n_old, int64_t m, const void* x_dev,
                                int64_t ld, int64_t x_stream_stride, void* sketch_dev,
                                int64_t sketch_stream_stride, float* rnorm_dev,
                                int64_t rnorm_stream_stride, stc_stream_t stream);

/* The same for one stream (encode: SPECTRA summary, "La Pipeline di
 * SPECTRA" step 3, projection and per-token quantization; decode: the same
 * step, reconstruction on the fly). */
stc_status stc_encode_kv(const stc_head_info* info, const void* state_dev, int64_t n_tokens,
                         const void* x_dev, int32_t dtype, int64_t ld, void* packed_dev,
                         float* norms_dev, stc_stream_t stream);
stc_status stc_decode_kv(const stc_head_info* info, const void* state_dev, int64_t n_tokens,
                         const void* packed_dev, const float* norms_dev, void* x_out_dev,
                         int32_t dtype, int64_t ld, stc_stream_t stream);

/* Quantize and pack given latent coefficients (fp32 [n][128], row stride
 * 128) with an EIGEN/IDENTITY state: the encode path without the
 * projection. For bit-exact checks of the quantizer and the format. */
stc_status stc_quantize_pack_f32(const stc_head_info* info, const void* state_dev, int64_t n_tokens,
                                 const float* coeffs_dev, void* packed_dev, stc_stream_t stream);

/* ------------------------------------------------------ attention
 * (SPECTRA summary, "La Pipeline di SPECTRA" step 3 and "Significato e
 * Rivendicazioni": standard attention over the rebuilt keys and values, the
 * latent form of it being the same arithmetic; SPECTRA abstract: the cache
 * is read in full at every generated token.)
 * One decode step for n_pairs KV heads (pair p: K stream with state
 * k_state_of_pair[p] and bytes k_packed_dev + p*packed_pair_stride, V stream
 * likewise), each shared by `group` query heads (1..16):
 *   out[p][h][:] = sum_t softmax_t(scale * q[p][h] . K_hat_t) V_hat_t
 * over all n_tokens cached tokens, with K_hat/V_hat the exact reconstructions
 * of the packed codes (never materialised: scores are taken in the latent
 * basis and the weighted code average is rotated back once). q_dev, out_dev:
 * fp32 [n_pairs][group][128]. EIGEN/IDENTITY states only. ws_dev: at least
 * stc_attend_workspace_bytes(n_pairs, group, n_tokens) bytes, 256-aligned
 * (see stc_attend_workspace_bytes). */
stc_status stc_attend_compressed_batched(const void* states_dev, int64_t n_states,
                                         const int32_t* k_state_of_pair_dev,
                                         const int32_t* v_state_of_pair_dev,
                                         const stc_head_info* infos, int64_t n_pairs,
                                         int64_t n_tokens, const void* k_packed_dev,
                                         const void* v_packed_dev, int64_t packed_pair_stride,
                                         int32_t group, const float* q_dev, float* out_dev,
                                         float scale, void* ws_dev, size_t ws_bytes,
                                         stc_stream_t stream);

/* For callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): stc_attend_compressed_batched
 * without a workspace argument. The split partials go to a static device
 * array of the library (stc_attend_noalloc_max_bytes() bytes, one copy per
 * device, held until the process ends); a call needing more
 * (stc_attend_workspace_bytes of its shape) fails with STC_EWORKSPACE before
 * any device work. The call allocates nothing. Calls that overlap on one
 * device share the array and race: serialize them (one stream, or events). */
stc_status stc_attend_compressed_batched_noalloc(const void* states_dev, int64_t n_states,
                                                 const int32_t* k_state_of_pair_dev,
                                                 const int32_t* v_state_of_pair_dev,
                                                 const stc_head_info* infos, int64_t n_pairs,
                                                 int64_t n_tokens, const void* k_packed_dev,
                                                 const void* v_packed_dev, int64_t packed_pair_stride,
                                                 int32_t group, const float* q_dev, float* out_dev,
                                                 float scale, stc_stream_t stream);
size_t stc_attend_noalloc_max_bytes(void);

/* stc_attend_compressed_batched with the keys' selective residual sketch
 * (from stc_sketch_kv_batched; pair p's at k_sketch_dev + p*sketch_pair_stride,
 * 16 bytes per token, and |r| at k_rnorm_dev + p*rnorm_pair_stride): every
 * score gains sqrt(pi/2)/STC_SKETCH_BITS |r_t| (S U_K^T q).z_t. */
stc_status stc_attend_compressed_sketch_batched(const void* states_dev, int64_t n_states,
                                                const int32_t* k_state_of_pair_dev,
                                                const int32_t* v_state_of_pair_dev,
                                                const stc_head_info* infos, int64_t n_pairs,
                                                int64_t n_tokens, const void* k_packed_dev,
                                                const void* v_packed_dev, int64_t packed_pair_stride,
                                                const void* k_sketch_dev, const float* k_rnorm_dev,
                                                int64_t sketch_pair_stride, int64_t rnorm_pair_stride,
                                                int32_t group, const float* q_dev, float* out_dev,
                                                float scale, void* ws_dev, size_t ws_bytes,
                                                stc_stream_t stream);

/* One KV head (the same step as stc_attend_compressed_batched, same pages). */
stc_status stc_attend_compressed(const stc_head_info* k_info, const void* k_state_dev,
                                 const stc_head_info* v_info, const void* v_state_dev,
                                 int64_t n_tokens, const void* k_packed_dev,
                                 const void* v_packed_dev, int32_t group, const float* q_dev,
                                 float* out_dev, float scale, void* ws_dev, size_t ws_bytes,
                                 stc_stream_t stream);

/* One decode step over Walsh-Hadamard caches (the TurboQuant-style
 * comparison path; ablation summary, "Regime-Specifieke Prestaties"): as
 * stc_attend_compressed_batched, with K_hat_t = |k_t| D H y_hat_t / sqrt(d)
 * and V_hat_t likewise, y_hat the codebook values of the 3-bit codes. The
 * per-token norms written by the RHT encode are k_norms_dev +
 * p*norms_pair_stride (and v_norms_dev likewise), fp32. Scores are taken
 * against H D q (never reconstructing K_hat), the softmax-weighted values are
 * accumulated in the rotated basis and rotated back once. With k_sketch_dev
 * (keys encoded by stc_append_rht_sketch_batched; their states built by
 * stc_rht_sketch_state_init) each score gains the residual estimate
 * sqrt(pi/2)/STC_SKETCH_BITS |r_t| (S q).z_t, the sketch of pair p at
 * k_sketch_dev + p*sketch_pair_stride (16 bytes per token) and |r| at
 * k_rnorm_dev + p*rnorm_pair_stride; NULL: no correction (a K state built
 * without the sketch matrix contributes none either). RHT states only
 * (STC_EUNSUPPORTED otherwise); ws_dev as for stc_attend_compressed_batched. */
stc_status stc_attend_rht_batched(const void* states_dev, int64_t n_states,
                                  const int32_t* k_state_of_pair_dev,
                                  const int32_t* v_state_of_pair_dev, const stc_head_info* infos,
                                  int64_t n_pairs, int64_t n_tokens, const void* k_packed_dev,
                                  const float* k_norms_dev, const void* v_packed_dev,
                                  const float* v_norms_dev, int64_t packed_pair_stride,
                                  int64_t norms_pair_stride, const void* k_sketch_dev,
                                  const float* k_rnorm_dev, int64_t sketch_pair_stride,
                                  int64_t rnorm_pair_stride, int32_t group, const float* q_dev,
                                  float* out_dev, float scale, void* ws_dev, size_t ws_bytes,
                                  stc_stream_t stream);

/* One generation step for n_pairs KV heads: append the new K token
 * k_new_dev[p][128] and V token v_new_dev[p][128] (dtype STC_BF16 or
 * STC_F32, rows of 128 elements) to pair p's packed K and V streams, which
 * hold n_old tokens and have room for n_old + 1, then attend as
 * stc_attend_compressed_batched over all n_old + 1 tokens. The new token's
 * records are those a full encode would write (the stream is append-only),
 * and attention reads them back from the packed cache like every other
 * token. EIGEN/IDENTITY states only; ws_dev as for
 * stc_attend_compressed_batched with n_old + 1 tokens; the new-token rows
 * must be 16-byte aligned. With bf16 rows the launches on `stream` are
 * those of the attention call alone: its first launch (per-KV-head score
 * weights) also forms and appends the two records, which the next launch
 * reads; fp32 rows take one launch more for the appends. */
stc_status stc_decode_step_batched(const void* states_dev, int64_t n_states,
                                   const int32_t* k_state_of_pair_dev,
                                   const int32_t* v_state_of_pair_dev, const stc_head_info* infos,
                                   int64_t n_pairs, int64_t n_old, const void* k_new_dev,
                                   const void* v_new_dev, int32_t dtype, void* k_packed_dev,
                                   void* v_packed_dev, int64_t packed_pair_stride, int32_t group,
                                   const float* q_dev, float* out_dev, float scale, void* ws_dev,
                                   size_t ws_bytes, stc_stream_t stream);

/* Check a state map on the host: copies n entries of map_dev to the host
 * (synchronizes `stream`) and returns STC_EINVAL, naming the first entry
 * outside [0, n_states) in stc_last_error, if there is one. For callers that
 * want the device-side behaviour above reported before they rely on it. */
stc_status stc_check_state_map(const int32_t* map_dev, int64_t n, int64_t n_states, stc_stream_t stream);

/* Kernel of the Walsh-Hadamard encode without the residual sketch (TurboQuant
 * ablation summary, "Experimentele Opstelling": a random sign flip and a
 * Walsh-Hadamard transform before the fixed 3-bit codebook). Both kernels
 * write the same records and norms up to fp32 summation order:
 *   STC_RHT_ENCODE_MFMA       the transform as a +-1 matrix on the matrix
 *                             cores (exact in bf16, fp32 sums)
 *   STC_RHT_ENCODE_BUTTERFLY  the fast transform as fp32 butterflies in
 *                             registers (one cross-lane swap stage)
 * The choice is process-wide and applies to launches issued after the call;
 * any other kind returns STC_EINVAL. The sketch encode always uses the
 * matrix cores (its sketch is a dense product). */
#define STC_RHT_ENCODE_MFMA 0
#define STC_RHT_ENCODE_BUTTERFLY 1
stc_status stc_set_rht_encode_kernel(int32_t kind);
int32_t stc_get_rht_encode_kernel(void);

/* Debug builds (libstc_debug.so, compiled with -DSTC_DEBUG): the kernels
 * check the indices they compute (LDS stream words, record byte ranges inside
 * a stream's capacity, staging offsets, value rows); a failed check sets one
 * bit of a device word and skips the access it guards. stc_debug_flags
 * synchronizes `stream`, stores the word in *flags and clears it; bits:
 * 0 encode stream word, 1 encode copy-out range, 2 decode stream word,
 * 3 decode record range, 4 attention staging, 5 attention value rows,
 * 6 generation-step append range, 7 Walsh-Hadamard encode range. Release
 * builds have no checks: *flags = 0. stc_debug_build returns 1 for a debug
 * build, else 0. */
int32_t stc_debug_build(void);
stc_status stc_debug_flags(uint32_t* flags, stc_stream_t stream);

/* Measurement helper: a plain streaming copy of `bytes` (a multiple of 16;
 * both buffers 16-byte aligned, not overlapping) on `stream`, with 16-byte
 * loads and non-temporal stores: the practical ceiling of a read + write
 * pattern against which the codec kernels' rates are read (it computes
 * nothing of the method). STC_EINVAL on a bad size or pointer. */
stc_status stc_stream_copy(void* dst_dev, const void* src_dev, int64_t bytes, stc_stream_t stream);

/* ------------------------------------------------------ diagnostics */
const char* stc_status_str(stc_status s);
/* Message of the last error on the calling thread ("" if none). */
const char* stc_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* STC_H */
