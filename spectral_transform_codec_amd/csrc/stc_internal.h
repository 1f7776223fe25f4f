// Internal layout of the device state blob and helpers shared by the host
// code and the HIP kernels of libstc. Not part of the public ABI.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "../../include/stc.h"

namespace stc {

constexpr int D = STC_D;
constexpr size_t STATE_BYTES = 512u * 1024u;

// Byte offsets of the regions of one state blob.
constexpr size_t OFF_HDR = 0;                        // DevHdr
constexpr size_t OFF_U32 = 8192;                     // float U[i][j], row-major (64 KiB)
constexpr size_t OFF_UT_HI = OFF_U32 + 65536;        // bf16 U[i][j] * yscale_j at [R][i], j = enc_row_channel(R), high part
constexpr size_t OFF_UT_LO = OFF_UT_HI + 32768;      // the low parts
constexpr size_t OFF_W_HI = OFF_UT_LO + 32768;       // bf16 W[enc_row_channel(R)][j] at [R][j], W = U diag(step)
constexpr size_t OFF_W_LO = OFF_W_HI + 32768;
constexpr size_t OFF_THR = OFF_W_LO + 32768;         // float thresholds, up to 128*255
// Walsh-Hadamard states with a key residual sketch reuse the threshold area:
// P = S D H / sqrt(d) as bf16 hi / lo rows (sketch row i at [R][j], i =
// enc_row_channel(R)) and S^T fp32 ([j][i] = S_ij) for S q.
constexpr size_t OFF_SKP_HI = OFF_THR;
constexpr size_t OFF_SKP_LO = OFF_THR + 32768;
constexpr size_t OFF_SKT32 = OFF_THR + 65536;
constexpr size_t OFF_GRAM = OFF_THR + 131072;        // double second moment [i][j]
// Value columns of the attention kernel (eigen / identity states): each kept
// channel's code cut at the record's byte boundaries, in record order; column
// c holds the bits of record byte `row` selected by `mask2` (the mask in both
// 16-bit halves of a word), and its fragment, read as an fp16 subnormal,
// times `fac` is that fragment's contribution to the channel's code.
// vch[j] = first column of channel j | number of its columns << 16.
constexpr size_t OFF_ATTV = OFF_GRAM + 131072;
constexpr int ATT_MAX_VCOLS = 256;
struct AttVCol {
  uint32_t row;
  uint32_t mask2;
  float fac;
  uint32_t chan;
};
constexpr size_t OFF_ATTVCH = OFF_ATTV + ATT_MAX_VCOLS * sizeof(AttVCol);
// fp16 W rows (the W_HI order) scaled by 2^e16, e16 = 13 - floor(log2 max |W|):
// the single-pass decode of low budgets
constexpr size_t OFF_W16 = (OFF_ATTVCH + D * sizeof(uint32_t) + 255) / 256 * 256;
static_assert(OFF_W16 + 32768 <= STATE_BYTES, "state layout overflows the blob");

// Quantizer fast path for a channel with L levels: y = c * fl(1/step) +
// (L/2 + eps_L) in fp32 with eps_L = L * 2^-21. Against the exact count of
// fp32 thresholds t_k = fl((k - L/2) step) <= c, y deviates by less than
// L * 2^-21.5 (fp32 rounding of 1/step, of the fma, and of t_k, each relative
// 2^-24 on magnitudes <= 2L), so floor(y) clamped to [0, L-1] is exact
// whenever fract(y) >= 2 eps_L; otherwise the thresholds decide. Ties
// (c == t_k) give y ~ k + eps_L and so go up, as the count does.
inline constexpr float quant_eps(int levels) { return (float)levels * (1.0f / 2097152.0f); }

struct alignas(16) DevHdr {
  int32_t xform;
  int32_t total_bits;
  int32_t n_kept;
  int32_t nmax16;       // 16 * ceil((last kept channel + 1) / 16): encode N extent
  int32_t kmax32;       // 32 * ceil((last kept channel + 1) / 32): decode K extent
  int32_t sketch_bits;  // Walsh-Hadamard states: key residual sketch bits per token (0: none)
  int32_t n_vcols;      // eigen / identity: value columns of the attention kernel (OFF_ATTV)
  int32_t pad;
  uint8_t bits[D];
  uint16_t off[D];      // bit offset of channel j inside a token record
  float inv_step[D];    // fl32(1 / step_j); 0 for a dropped channel or a zero step
  float ybias[D];       // L_j/2 + quant_eps(L_j) for a kept channel, 0.5 for a dropped one
  int32_t lm1[D];       // L_j - 1 (0 if dropped)
  int32_t thr_base[D];  // index of t_1 of channel j in the threshold table
  float bias[D];        // decode: sum_j U_ij step_j (L_j - 1)/2, natural dim order
  float step32[D];      // fl32(step_j)
  float halfspan[D];    // (L_j - 1) / 2
  float sign[D];        // Walsh-Hadamard diagonal (+-1)
  float cb[8];          // Walsh-Hadamard codebook
  float cb_thr[8];      // its 7 midpoint thresholds (last entry unused)
  uint32_t bits4[D / 8];  // widths again, 4 bits each: channel j in bits 4(j%8).. of word j/8
  // Unpack plan. Quarter q covers channels [32q, 32q+32); its codes start at
  // record bit qoff[q]. Output dword i of quarter q (channels 32q+4i..+3)
  // reads the 64-bit window of quarter-relative words k, k+1 at bit s:
  //   plan[q][i] = k | s << 5 | b0 << 10 | b1 << 14 | b2 << 18 | b3 << 22.
  // qwords[q] = record-aligned words a quarter needs (max k + 2).
  uint32_t plan[4][8];
  uint32_t qoff[4];
  uint32_t qwords[4];
  double step64[D];     // step_j in fp64: thresholds are fl32((k - L/2) * step64[j])
  // Token encode: the basis rows are stored scaled by yscale_j = 1/step_j
  // (2^100 for a zero step, 0 for a dropped channel), so that the projection
  // gives the coordinate in quantizer cells directly; the code is
  // clamp(floor(x.U_j yscale_j + yhalf_j), 0, L_j - 1), yhalf_j = L_j/2
  // (L_j - 1/2 for a zero step, where every threshold is 0).
  float yhalf[D];
  // Walsh-Hadamard attention: the codebook as byte planes for v_perm lookups
  // (code c selects byte c of the 8-byte plane held in words 2i, 2i+1):
  // planes 0/1 low/high bytes of bf16(cb), 2/3 of bf16(cb - bf16(cb)),
  // 4/5 of fp16(cb)
  uint32_t cbt[12];
  float bias16[D];      // decode with fp16 W: sum_j W16_ij 2^-e16 (L_j - 1)/2, natural dim order
  uint32_t code16;      // fp16 pair (2^-e16, 2^-e16): the codes' scale in that decode
};
static_assert(sizeof(DevHdr) <= OFF_U32, "header too large");


// Encode basis rows (bf16 U^T hi/lo) are stored permuted for the 32x32
// encode MFMA (A = basis rows, M = channels): output row 8i + 4h + j of row
// block b lands in lane half h, register 4i + j. Stored row R = 32b + 8i +
// 4h + j holds latent channel 64h + 16b + 4i + j, so lane half h holds
// channels [64h, 64h + 64) of its token, four consecutive channels per i.
inline constexpr int enc_row_channel(int R) {
  return 64 * ((R >> 2) & 1) + 16 * (R >> 5) + 4 * ((R >> 3) & 3) + (R & 3);
}

inline size_t packed_bytes(int64_t total_bits, int64_t n) {
  int64_t nb = (n * total_bits + 7) / 8;
  return (size_t)((nb + 15) / 16 * 16);
}

// Attention split geometry (tokens per workgroup) as a function of the call's
// shape; shared by the workspace-size query and the launcher.
constexpr int ATT_TILE = 256;
// `round`: workgroups resident at once (256 CUs times the kernel's workgroups
// per CU); the workspace covers every kernel's split count (ATT_ROUNDS).
constexpr int64_t ATT_ROUNDS[3] = {256, 768, 1024};
inline int64_t att_split_tokens(int64_t n_pairs, int64_t n_tokens, int64_t round) {
  // at least one round of workgroups; among up to twice the fewest splits
  // per pair, the count that fills the last round best; a pair has at most
  // one split per tile
  const int64_t tiles = (n_tokens + ATT_TILE - 1) / ATT_TILE;
  int64_t s0 = (round + n_pairs - 1) / n_pairs;
  if (s0 > tiles) s0 = tiles;
  if (s0 < 1) s0 = 1;
  int64_t best = s0;
  double best_fill = 0.0;
  for (int64_t s = s0; s <= 2 * s0 && s <= tiles; ++s) {
    const int64_t wg = n_pairs * s;
    const double fill = (double)wg / (double)(((wg + round - 1) / round) * round);
    if (fill > best_fill + 1e-9) {
      best_fill = fill;
      best = s;
    }
  }
  const int64_t per = (tiles + best - 1) / best;
  return per * ATT_TILE;
}
inline int64_t att_n_splits(int64_t n_pairs, int64_t n_tokens, int64_t round) {
  int64_t s = att_split_tokens(n_pairs, n_tokens, round);
  return (n_tokens + s - 1) / s;
}
constexpr int ATT_PART_FLOATS = D + 2;              // per (pair, split, head): acc[128], m, l
// per pair, after a launch's partials: the packed-bit kernel's score weights
// a [8 heads][128] and the 8 per-head scales (padded to whole 128-byte lines)
constexpr int ATT_PREP_FLOATS = 8 * D + 32;
// floats of one (pair, split) partial block: group x (acc, m, l), padded to
// whole 128-byte lines so that no line is written by two workgroups
__host__ __device__ inline int64_t att_part_stride(int group) {
  return ((int64_t)group * ATT_PART_FLOATS + 31) / 32 * 32;
}
// Attention workspace: the split partials of one launch, which covers at
// most ATT_MAX_PAIRS pairs (launches of one call reuse it in stream order),
// then the per-pair score weights of the packed-bit kernel.
constexpr int64_t ATT_MAX_PAIRS = 16384;
inline int64_t att_partial_floats(int64_t np, int64_t n_tokens, int group, int64_t round) {
  return np * att_n_splits(np, n_tokens, round) * att_part_stride(group);
}
inline int64_t att_launch_floats(int64_t np, int64_t n_tokens, int group) {
  int64_t most = 0;
  for (int64_t round : ATT_ROUNDS) {
    const int64_t f = att_partial_floats(np, n_tokens, group, round) + np * ATT_PREP_FLOATS;
    most = f > most ? f : most;
  }
  return most;
}

// Host-side launchers implemented in stc_kernels.hip.
struct EncodeLaunch {
  const unsigned char* states;
  const int32_t* map;
  int64_t n_states;
  int64_t n_streams, n_tokens, ld, x_stride, packed_stride;
  const void* x;
  unsigned char* packed;
  float* norms;
  int mode;       // 0 bf16 tokens, 1 fp32 tokens, 2 fp32 latent coefficients
  int max_bits;   // largest total_bits of the states used
  int64_t n_old = 0;         // tokens already in the streams (append); n_tokens new ones follow
  int64_t norms_stride = 0;  // Walsh-Hadamard norms: elements between streams
  unsigned char* sketch = nullptr;  // Walsh-Hadamard key residual sketch (16 bytes per token) or null
  float* rnorm = nullptr;           // |r| per token
  int64_t sketch_stride = 0, rnorm_stride = 0;
  bool rec = false;  // every record is 0 or 32 * 2^s bits: the slot layout
};
struct DecodeLaunch {
  const unsigned char* states;
  const int32_t* map;
  int64_t n_states;
  int64_t n_streams, n_tokens, ld, x_stride, packed_stride;
  const unsigned char* packed;
  const float* norms;
  void* x;
  int f32out;
  int max_bits;
  bool w16 = false;  // bf16 output from the fp16 W rows in one pass (low budgets; see decode_w16_ok)
};
struct AttendLaunch {
  const unsigned char* k_states;
  const int32_t* k_map;
  const unsigned char* v_states;
  const int32_t* v_map;
  int64_t n_states;
  int64_t n_pairs, n_tokens, packed_stride;
  const unsigned char* k_packed;
  const unsigned char* v_packed;
  int group;
  const float* q;
  float* out;
  float scale;
  unsigned char* ws;
  int max_bits;
  const float* k_norms = nullptr;  // Walsh-Hadamard caches: per-token norms
  const float* v_norms = nullptr;
  int64_t norms_stride = 0;       // elements between pairs
  bool rht = false;
  const unsigned char* k_sketch = nullptr;  // Walsh-Hadamard keys: residual sketch and |r|, or null
  const float* k_rnorm = nullptr;
  int64_t sketch_stride = 0, rnorm_stride = 0;
  bool rec = false;  // every record is 0 or 32 * 2^s bits: one word-aligned LDS slot per record
  int att_chunks = 3;  // 1 KiB loads that cover one 32-token block of any stream (its records may
                       // start 4, 8 or 12 bytes past a 16-byte boundary)
  int max_vcols = 256;  // value columns of the states at most (code fragments cut at record bytes)
  bool rec256 = false;  // every record is 256 bits
  // generation step: new K and V rows [pair][128] appended as token n_tokens - 1
  // before the attention reads the caches (eigen / identity states, no sketch)
  const void* k_new = nullptr;
  const void* v_new = nullptr;
  int new_f32 = 0;
};

// second moments of n_streams streams (rows x + s * x_stride, elements) into
// gram + s * gram_stride (doubles), one launch
int launch_gram(const void* x, int dtype, int64_t ld, int64_t x_stride, int64_t n_calib, int64_t n_streams,
                double* gram, int64_t gram_stride, void* stream);
int launch_encode_eigen(const EncodeLaunch& a, void* stream);
int launch_decode_eigen(const DecodeLaunch& a, void* stream);
int launch_encode_rht(const EncodeLaunch& a, void* stream);
// Walsh-Hadamard encode kernel: 0 the +-1 matrix on the matrix cores, 1 the
// register butterfly (stc_set_rht_encode_kernel)
int rht_encode_kernel();
// debug builds: read and clear the device check word (synchronizes stream);
// release builds: 0
int read_debug_flags(unsigned* out, void* stream);
int launch_stream_copy(void* dst, const void* src, int64_t bytes, void* stream);
int debug_build();
int launch_sketch_eigen(const EncodeLaunch& a, void* stream);
int launch_decode_rht(const DecodeLaunch& a, void* stream);
int launch_attend(const AttendLaunch& a, void* stream);
// The static device scratch of the attention entry point that allocates
// nothing: its size, and its address on the current device (looked up once
// per device; nonzero on failure).
size_t attend_scratch_bytes();
int attend_scratch(void** ptr);

}  // namespace stc
