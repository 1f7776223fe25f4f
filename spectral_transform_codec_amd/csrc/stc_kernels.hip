// HIP kernels of libstc for gfx950 (MI355X, CDNA4, wave64).
//
// What they compute is fixed by the pages (cited by title and section):
//  - second moment of calibration tokens: "Sintesi Tecnica: SPECTRA"
//    (gist.science), "Metodologia" observation 3 (G = E[h^T h]);
//  - projection onto the latent basis, per-token quantization, append to the
//    packed cache: same page, "La Pipeline di SPECTRA" steps 2-3;
//  - unpack / dequantize / rotate back, and attention over the rebuilt K/V:
//    "La Pipeline" step 3 and "Significato e Rivendicazioni";
//  - randomized Walsh-Hadamard + fixed codebook: "Technisch Overzicht:
//    Ablatie, ..." (gist.science), "Experimentele Opstelling" (TurboQuant).
// Readings of the pages (quantizer, bit layout F1, ...) are listed in
// include/stc.h; this file implements exactly those.
//
// Hardware mapping:
//  - projection and reconstruction are dense 128-wide contractions on the
//    matrix cores (v_mfma_f32_32x32x16_bf16, 32 tokens per wave). The basis
//    is split into bf16 high and low parts (two passes; three for fp32
//    tokens) so the fp32 result carries ~16 significant bits of the basis,
//    enough for code parity with the fp64 definition. Codes are exact small
//    integers in bf16. The bf16 decode of budgets up to 2 bits per value
//    takes one fp16 pass (v_mfma_f32_32x32x16_f16) with the basis scaled by
//    a power of two and codes scaled back exactly.
//  - bit packing and unpacking go through a per-wave LDS stream, which
//    turns the variable-length records into coalesced HBM accesses and
//    moves codes between the matrix-core layouts and the records.
//  - attention reads the packed records straight into the matrix cores:
//    scores from the K record bits on int8 MFMAs, softmax weights times the
//    V codes on fp16 MFMAs, records staged to LDS by buffer loads.
//  - the Walsh-Hadamard encode runs either as a +-1 matrix on the matrix
//    cores or as fp32 butterflies in registers (two lanes per token, one
//    cross-lane swap stage); its decode runs the butterflies one token per
//    lane.
#include <hip/hip_runtime.h>

#include <mutex>

#include "stc_internal.h"

namespace stc {

// Debug builds (-DSTC_DEBUG, libstc_debug.so): device-side checks of the
// indices the kernels compute (LDS stream words, record byte ranges inside a
// stream's capacity, staging offsets, value rows). A failed check sets its
// bit in stc_debug_word (a vector atomic) and the access it guards is
// skipped, so the launch completes; stc_debug_flags reads and clears the
// word. Release builds compile every check to `true`.
enum : unsigned {
  DBG_ENC_STREAM = 0,   // encode: LDS stream word of a group
  DBG_ENC_RANGE = 1,    // encode: copy-out past the stream's capacity
  DBG_DEC_STREAM = 2,   // decode: LDS stream word of a group
  DBG_DEC_RANGE = 3,    // decode: record bytes past the stream
  DBG_ATT_STAGE = 4,    // attention: staged record words past a staging buffer
  DBG_ATT_VROW = 5,     // attention: value row past the wave's rows
  DBG_APPEND = 6,       // generation step: record words past the stream's capacity
  DBG_RHT_RANGE = 7,    // Walsh-Hadamard encode: record past the stream's capacity
};
#ifdef STC_DEBUG
__device__ unsigned stc_debug_word;
__device__ __forceinline__ bool dbg_check(bool ok, unsigned bit) {
  if (__builtin_expect(ok, 1)) return true;
  __hip_atomic_fetch_or(&stc_debug_word, 1u << bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return false;
}
#define STC_CHECK(cond, bit) dbg_check((cond), (bit))
#else
#define STC_CHECK(cond, bit) true
#endif

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr float LOG2E = 1.4426950408889634f;

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
typedef float f32x16 __attribute__((ext_vector_type(16)));
__device__ __forceinline__ f32x16 mfma32_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
// Two floats rounded to bf16 (nearest even), packed low / high: one
// v_cvt_pk_bf16_f32.
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}
// Two floats that bf16 holds exactly (here integers below 2^8, whose fp32
// low halves are zero) as a bf16 pair: the two high halves, one byte permute.
__device__ __forceinline__ unsigned bf16_pair_exact(float lo, float hi) {
  return __builtin_amdgcn_perm(__builtin_bit_cast(unsigned, hi), __builtin_bit_cast(unsigned, lo), 0x07060302u);
}

__device__ __forceinline__ long long packed_len(long long total_bits, long long n) {
  const long long nb = (n * total_bits + 7) / 8;
  return (nb + 15) / 16 * 16;
}

// State of stream s: map[s] (or s without a map); -1 when the entry lies
// outside [0, n_states). Such a stream is never read from its state: encode
// and append leave its records untouched, decode writes NaN rows, attention
// writes NaN outputs (stc_check_state_map reports the entry on the host).
__device__ __forceinline__ long long state_index(const int32_t* map, long long s, long long n_states) {
  const long long si = map ? (long long)map[s] : s;
  return (si < 0 || si >= n_states) ? -1 : si;
}

// Workgroup -> work mapping that keeps consecutive logical workgroups on one
// XCD (hardware dispatches blockIdx round-robin over the 8 XCDs), so the
// workgroups sharing a stream's basis share an L2.
__device__ __forceinline__ int xcd_logical(int b, int grid) {
  return (grid % 8 == 0) ? (b % 8) * (grid / 8) + b / 8 : b;
}

// ======================================================================
// Second moment (calibration): one workgroup per stream (blockIdx.x; rows
// at x + stream * x_stride, the result at gram + stream * gram_stride), fp64
// accumulation of exact fp32 products in token order. Thread (ti, tj) owns
// entries (ti + 16u, tj + 16v), so (a, b) and (b, a) see identical sums.
// ======================================================================
__global__ void __launch_bounds__(256) k_gram(const void* x0, int dtype, long long ld, long long x_stride, long long n,
                                              double* gram0, long long gram_stride) {
  const long long sidx = blockIdx.x;
  const void* x = static_cast<const unsigned char*>(x0) + sidx * x_stride * (dtype == STC_F32 ? 4 : 2);
  double* gram = gram0 + sidx * gram_stride;
  __shared__ float sx[64][132];
  const int tid = threadIdx.x, ti = tid >> 4, tj = tid & 15;
  double acc[8][8];
#pragma unroll
  for (int u = 0; u < 8; ++u)
#pragma unroll
    for (int v = 0; v < 8; ++v) acc[u][v] = 0.0;
  for (long long t0 = 0; t0 < n; t0 += 64) {
    const int cnt = (int)((n - t0) < 64 ? (n - t0) : 64);
    for (int i = tid; i < 64 * 128; i += 256) {
      const int r = i >> 7, c = i & 127;
      float v = 0.0f;
      if (r < cnt) {
        if (dtype == STC_F32) v = static_cast<const float*>(x)[(t0 + r) * ld + c];
        else v = __uint_as_float((unsigned)static_cast<const unsigned short*>(x)[(t0 + r) * ld + c] << 16);
      }
      sx[r][c] = v;
    }
    __syncthreads();
    for (int r = 0; r < cnt; ++r) {
      double xa[8], xb[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) { xa[u] = (double)sx[r][ti + 16 * u]; xb[u] = (double)sx[r][tj + 16 * u]; }
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int v = 0; v < 8; ++v) acc[u][v] = __builtin_fma(xa[u], xb[v], acc[u][v]);
    }
    __syncthreads();
  }
  const double inv_n = 1.0 / (double)n;
#pragma unroll
  for (int u = 0; u < 8; ++u)
#pragma unroll
    for (int v = 0; v < 8; ++v) gram[(ti + 16 * u) * 128 + tj + 16 * v] = acc[u][v] / (double)n;
  (void)inv_n;
}

int read_debug_flags(unsigned* out, void* stream) {
#ifdef STC_DEBUG
  hipStream_t s = (hipStream_t)stream;
  unsigned zero = 0u;
  if (hipMemcpyFromSymbolAsync(out, HIP_SYMBOL(stc_debug_word), sizeof(unsigned), 0, hipMemcpyDeviceToHost, s) !=
          hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return 1;
  if (hipMemcpyToSymbolAsync(HIP_SYMBOL(stc_debug_word), &zero, sizeof(unsigned), 0, hipMemcpyHostToDevice, s) !=
          hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return 1;
  return 0;
#else
  (void)stream;
  *out = 0u;
  return 0;
#endif
}

int debug_build() {
#ifdef STC_DEBUG
  return 1;
#else
  return 0;
#endif
}

int launch_gram(const void* x, int dtype, int64_t ld, int64_t x_stride, int64_t n_calib, int64_t n_streams,
                double* gram, int64_t gram_stride, void* stream) {
  hipLaunchKernelGGL(k_gram, dim3((unsigned)n_streams), dim3(256), 0, (hipStream_t)stream, x, dtype, (long long)ld,
                     (long long)x_stride, (long long)n_calib, gram, (long long)gram_stride);
  return hipGetLastError() != hipSuccess;
}

// ======================================================================
// Encode (eigen / identity): project -> quantize -> pack.
// A workgroup of 16 waves shares the basis (bf16 hi/lo rows, permuted) and
// the quantizer tables in LDS; each wave encodes blocks of 32 tokens on its
// own, with no workgroup barrier between blocks (four waves per SIMD hide
// each other's memory and MFMA latency).
//  1. MFMA 32x32x16 with A = basis rows (M = channels), B = the block's
//     tokens: lane (h, t) receives channels [64h, 64h + 64) of token t,
//     sixteen per row block, four consecutive channels per register group.
//  2. Each value is quantized in registers and shifted to its bit offset
//     inside its group of four channels (adjacent in the record): one word
//     per group.
//  3. Each group word is ORed into the wave's LDS bit stream at bit
//     t*B + offset (one pad word per 32 keeps lanes on distinct banks; a
//     spill past a 32-word block lands in that pad word and is folded back
//     on the way out).
//  4. The wave copies its stream (32 records, 4B bytes) to HBM and clears it.
// ======================================================================
constexpr int ENC_WAVES = 16;
constexpr int ENC_THREADS = 64 * ENC_WAVES;
constexpr int ENC_BT = 32;                       // tokens per wave block
constexpr int UROW = 272;                        // bytes per LDS basis row (256 + 16 pad)
constexpr int CROW = 144;                        // bytes per LDS code row (128 + 16 pad)
constexpr int EST_WORDS = 32 * 33 + 8;           // wave stream: 32 x 1024 bits + pad words + tail
constexpr size_t ENC_LDS = 2 * 128 * UROW + 8 * 128 * 4 + (size_t)ENC_WAVES * EST_WORDS * 4;

struct EncK {
  const unsigned char* states;
  const int32_t* map;
  long long n_states, n_tokens, ld, x_stride, packed_stride;
  const void* x;
  unsigned char* packed;
  long long blocks_per_stream, total_blocks, blocks_per_wg;
  long long n_old, blk0;  // tokens already in the streams; first (absolute) 32-token block
  long long norms_stride;
  unsigned char* sketch;  // selective residual sketch (16 bytes per token) and |r|
  float* rnorm;
  long long sketch_stride, rnorm_stride;
  int grid;
};

__device__ __forceinline__ unsigned est_idx(unsigned w) { return w + (w >> 5); }
// est_idx(P >> 5) for a stream bit P < 2^24 (a wave block's stream is at
// most 32 x 1024 bits): w + floor(w / 32) = floor(33 w / 32), one 24-bit
// multiply (written as such: the compiler would expand 33 w into shifts and
// masks, two instructions more per group)
__device__ __forceinline__ unsigned est_idx_bit(unsigned P) {
  unsigned r;
  asm("v_lshrrev_b32 %0, 5, %1\n\tv_mul_u32_u24 %0, 33, %0\n\tv_lshrrev_b32 %0, 5, %0" : "=&v"(r) : "v"(P));
  return r;
}

// LDS (address space 3) byte pointers, used where a per-lane base must stay
// one register so that reads can take constant offsets.
typedef __attribute__((address_space(3))) unsigned char lds_u8;
__device__ __forceinline__ unsigned lds_offset(unsigned char* p) {
  return (unsigned)(uintptr_t)(lds_u8*)p;
}
__device__ __forceinline__ const lds_u8* lds_ptr(unsigned off) { return (const lds_u8*)(uintptr_t)off; }
#define LDS_AT(T, p) (*(const __attribute__((address_space(3))) T*)(p))

// Copy a wave stream of `nbytes` bytes (a multiple of 4*CW) to dst with
// CW-word stores, folding the pad words back in; then clear `clear` words.
template <int CW>
__device__ __forceinline__ void est_copy_out(unsigned* str, unsigned char* dst, long long nbytes, unsigned clear,
                                             int lane) {
  typedef unsigned vec __attribute__((ext_vector_type(CW)));
  const int nchunk = (int)(nbytes / (4 * CW));
  for (int c = lane; c < nchunk; c += 64) {
    vec v;
#pragma unroll
    for (int e = 0; e < CW; ++e) {
      const unsigned w = (unsigned)(CW * c + e);
      unsigned x = str[est_idx(w)];
      if ((w & 31u) == 0u && w > 0u) x |= str[est_idx(w - 1) + 1];
      v[e] = x;
    }
    reinterpret_cast<vec*>(dst)[c] = v;
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);
  __builtin_amdgcn_wave_barrier();
  for (unsigned i = lane; i < clear; i += 64) str[i] = 0u;
}

// Slot layout (records of 32 * 2^sh bits): word w of the block sits at
// w + (w >> sh), one pad word after each record; records never spill into
// their pad, so the copy needs no folding.
template <int CW>
__device__ __forceinline__ void rec_copy_out(unsigned* str, unsigned char* dst, long long nbytes, unsigned clear,
                                             int lane, unsigned sh) {
  typedef unsigned vec __attribute__((ext_vector_type(CW)));
  const int nchunk = (int)(nbytes / (4 * CW));
  for (int c = lane; c < nchunk; c += 64) {
    vec v;
#pragma unroll
    for (int e = 0; e < CW; ++e) {
      const unsigned w = (unsigned)(CW * c + e);
      v[e] = str[w + (w >> sh)];
    }
    reinterpret_cast<vec*>(dst)[c] = v;
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);
  __builtin_amdgcn_wave_barrier();
  for (unsigned i = lane; i < clear; i += 64) str[i] = 0u;
}

// MODE 0: bf16 tokens, 1: fp32 tokens, 2: fp32 latent coefficients [n][128].
// REC (MODE 0 and 1): every record is 32 * 2^s bits, staged in the slot
// layout, so a group's word and shift are table entries.
template <int MODE, bool REC>
__global__ void __launch_bounds__(ENC_THREADS, 1) k_encode_eigen(EncK a) {
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* sUhi = smem;
  float* sInv = reinterpret_cast<float*>(smem + 2 * 128 * UROW);  // then yb, L-1, pos, band, group offset, fp64 step
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t32 = lane & 31, h = lane >> 5;
  unsigned* sStr = reinterpret_cast<unsigned*>(sInv + 8 * 128) + wave * EST_WORDS;
  const int lw = xcd_logical(blockIdx.x, a.grid);
  const long long b_begin = (long long)lw * a.blocks_per_wg;
  long long b_end = b_begin + a.blocks_per_wg;
  if (b_end > a.total_blocks) b_end = a.total_blocks;
  // the call writes tokens [n0, n) of each stream: x row r holds token n0 + r
  const long long n0 = a.n_old, m = a.n_tokens, n = n0 + m;

  for (int i = lane; i < EST_WORDS; i += 64) sStr[i] = 0u;

  // x row of lane t in the block at token tok0: rbase + rlane (clamped to
  // the call's rows [0, m))
  auto x_row = [&](long long tok0, long long& rbase, unsigned& rlane) {
    rbase = tok0 - n0 > 0 ? tok0 - n0 : 0;
    long long r = tok0 + t32 - n0 - rbase;
    if (r < 0) r = 0;
    if (r > m - 1 - rbase) r = m - 1 - rbase;
    rlane = (unsigned)r;
  };
  // B fragments (tokens) of a block: pf[ks] = token t, dims 16ks + 8h .. +7
  bf16x8 pf[8];
  auto load_frags = [&](long long s2, long long tt2) {
    long long rbase;
    unsigned r;
    x_row(tt2 * ENC_BT, rbase, r);
    const unsigned short* base = static_cast<const unsigned short*>(a.x) + s2 * a.x_stride + rbase * a.ld;
    const unsigned ro = r * (unsigned)a.ld + 8u * (unsigned)h;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      pf[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(base + ro + 16 * ks));
  };

  for (long long seg = b_begin; seg < b_end;) {
    const long long s = seg / a.blocks_per_stream;
    long long seg_end = (s + 1) * a.blocks_per_stream;
    if (seg_end > b_end) seg_end = b_end;
    const long long si = state_index(a.map, s, a.n_states);
    if (si < 0) {  // (uniform over the workgroup) no state: records untouched
      seg = seg_end;
      continue;
    }
    const unsigned char* st = a.states + (size_t)si * STATE_BYTES;
    const DevHdr* hdr = reinterpret_cast<const DevHdr*>(st + OFF_HDR);
    const unsigned B = (unsigned)__builtin_amdgcn_readfirstlane(hdr->total_bits);
    __syncthreads();  // every wave is done with the previous basis
    if (MODE != 2) {
      const u32x4* ghi = reinterpret_cast<const u32x4*>(st + OFF_UT_HI);
      const u32x4* glo = reinterpret_cast<const u32x4*>(st + OFF_UT_LO);
      for (int i = tid; i < 128 * 16; i += ENC_THREADS) {
        const int row = i >> 4, c = i & 15;
        *reinterpret_cast<u32x4*>(sUhi + row * UROW + c * 16) = ghi[i];
        *reinterpret_cast<u32x4*>(sUhi + 128 * UROW + row * UROW + c * 16) = glo[i];
      }
    }
    if (tid < 128) {
      if (MODE == 2) {
        sInv[tid] = hdr->inv_step[tid];
        sInv[128 + tid] = hdr->ybias[tid];
        sInv[256 + tid] = (float)hdr->lm1[tid];
        reinterpret_cast<unsigned*>(sInv)[384 + tid] = (unsigned)hdr->off[tid] - (unsigned)hdr->off[tid & ~3];
        sInv[512 + tid] = 2.0f * quant_eps(hdr->lm1[tid] + 1);  // guard band of the fast path
        reinterpret_cast<unsigned*>(sInv)[640 + tid] = (unsigned)hdr->off[tid & ~3];  // record offset of the group
        reinterpret_cast<double*>(sInv + 768)[tid] = hdr->step64[tid];
      } else {
        sInv[tid] = hdr->yhalf[tid];
        sInv[128 + tid] = (float)hdr->lm1[tid];
        reinterpret_cast<unsigned*>(sInv)[256 + tid] = (unsigned)hdr->off[tid] - (unsigned)hdr->off[tid & ~3];
        // group record offset; entries 4g + 1, 4g + 2: the byte offset of
        // its word in a record slot and the shift inside it
        const unsigned go = (unsigned)hdr->off[tid & ~3];
        reinterpret_cast<unsigned*>(sInv)[384 + tid] = (tid & 3) == 1 ? (go >> 5) << 2 : ((tid & 3) == 2 ? go & 31u : go);
      }
    }
    __syncthreads();
    if (B > 0) {
      const long long P_len = packed_len((long long)B, n);
      const unsigned cw_kind = (B & 3u) == 0u ? 4u : ((B & 1u) == 0u ? 2u : 1u);
      const unsigned rsh = (unsigned)__builtin_ctz((B >> 5) | 64u);  // REC: log2 of the words a record
      const unsigned clear = REC ? 32u * ((B >> 5) + 1u) + 2u : est_idx(B + 4u) + 2u;
      // bf16 tokens: a block's fragments are requested as soon as the
      // previous block's last MFMA has read its own (same registers), so the
      // load runs under that block's last quantization and copy-out
      if (MODE == 0 && seg + wave < seg_end) load_frags(s, seg + wave - s * a.blocks_per_stream + a.blk0);
      for (long long blk = seg + wave; blk < seg_end; blk += ENC_WAVES) {
        const long long tt = blk - s * a.blocks_per_stream + a.blk0;  // absolute block of the stream
        const long long tok0 = tt * ENC_BT;
        long long rbase;
        unsigned trow;
        x_row(tok0, rbase, trow);
        bf16x8 xl[8];
        auto& xh = pf;
        if (MODE == 1) {
          const float* row = static_cast<const float*>(a.x) + s * a.x_stride + rbase * a.ld + trow * (unsigned)a.ld;
#pragma unroll
          for (int ks = 0; ks < 8; ++ks) {
            const f32x4 v0 = *reinterpret_cast<const f32x4*>(row + 16 * ks + 8 * h);
            const f32x4 v1 = *reinterpret_cast<const f32x4*>(row + 16 * ks + 8 * h + 4);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float f = e < 4 ? v0[e] : v1[e - 4];
              const __bf16 hi = (__bf16)f;
              xh[ks][e] = hi;
              xl[ks][e] = (__bf16)(f - (float)hi);
            }
          }
        }
        // opaque per-lane LDS bases: every table read is base + constant
        unsigned ub = lds_offset(sUhi + t32 * UROW + 16 * h);
        unsigned pb = lds_offset(reinterpret_cast<unsigned char*>(sInv + 64 * h));
        asm volatile("" : "+v"(ub), "+v"(pb));
        const lds_u8* uL = lds_ptr(ub);
        const lds_u8* pL = lds_ptr(pb);
        const bool tok_ok = tok0 + t32 >= n0 && tok0 + t32 < n;
        const unsigned tB = (unsigned)t32 * B;
        unsigned rb = REC ? t32 * ((B >> 5) + 1u) * 4u : 0u;  // REC: byte offset of the lane's slot
        if (REC) asm volatile("" : "+v"(rb));
        unsigned char* sRec = reinterpret_cast<unsigned char*>(sStr) + rb;
        // ---- 3: OR a group word into the stream at record bit tB + goff; a
        // lane whose token is outside the call ORs zero (no branch, so that
        // this work can overlap the next row block's MFMA chain). gt: the
        // group's offset, word byte offset and shift (REC) from the table.
        auto put_group = [&](unsigned word, u32x4 gt) {
          unsigned* dst;
          unsigned long long v;
          if (REC) {
            v = (unsigned long long)(tok_ok ? word : 0u) << gt[2];
            dst = reinterpret_cast<unsigned*>(sRec + gt[1]);
          } else {
            const unsigned P = tB + gt[0];
            v = (unsigned long long)(tok_ok ? word : 0u) << (P & 31u);
            dst = sStr + est_idx_bit(P);
          }
          if (!STC_CHECK((unsigned)(dst - sStr) + 1u < (unsigned)EST_WORDS, DBG_ENC_STREAM)) return;
          __hip_atomic_fetch_or(dst, (unsigned)v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
          __hip_atomic_fetch_or(dst + 1, (unsigned)(v >> 32), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        };
        if (MODE != 2) {
          // ---- 1: channels 64h + 16mb + 4i + j of token t in acc[4i + j].
          // The chain starts from yhalf_j, so that it ends on the cell
          // coordinate x.U_j yscale_j + yhalf_j itself.
          auto chain_init = [&](const int mb, f32x16& acc) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const f32x4 yh = LDS_AT(f32x4, pL + 4 * (16 * mb + 4 * i));
#pragma unroll
              for (int j = 0; j < 4; ++j) acc[4 * i + j] = yh[j];
            }
          };
          // The basis rows of chain step i = 8 mb + ks are read LA steps
          // ahead of their MFMAs, and a scheduling barrier keeps the reads
          // there: left to itself the compiler issues each read right before
          // its MFMA and waits for it. (fp32 tokens, three MFMAs per step,
          // keep LA = 0: their registers would not hold the extra rows.)
          constexpr int LA = MODE == 0 ? 1 : 0;
          bf16x8 ahr[LA + 1], alr[LA + 1];
          auto readA = [&](const int i) {
            const int off = 32 * (i >> 3) * UROW + 32 * (i & 7);
            ahr[i % (LA + 1)] = LDS_AT(bf16x8, uL + off);
            alr[i % (LA + 1)] = LDS_AT(bf16x8, uL + 128 * UROW + off);
          };
          auto chain_step = [&](const int mb, const int ks, f32x16& acc) {
            const int i = 8 * mb + ks;
            if (i + LA < 32) readA(i + LA);
            if (LA > 0) __builtin_amdgcn_sched_barrier(0);
            acc = mfma32_bf16(ahr[i % (LA + 1)], xh[ks], acc);
            acc = mfma32_bf16(alr[i % (LA + 1)], xh[ks], acc);
            if (MODE == 1) acc = mfma32_bf16(ahr[i % (LA + 1)], xl[ks], acc);
          };
          // ---- 2: the code is floor(acc) clamped to [0, L-1], per group of
          // four channels
          auto quant_group = [&](const int mb, const int i, const f32x16& acc) {
            const int coff = 4 * (16 * mb + 4 * i);  // byte offset of the group in a table
            const f32x4 lm = LDS_AT(f32x4, pL + 512 + coff);
            const u32x4 pos = LDS_AT(u32x4, pL + 1024 + coff);
            u32x4 gt;
            if (REC) gt = LDS_AT(u32x4, pL + 1536 + coff);
            else gt[0] = LDS_AT(unsigned, pL + 1536 + coff);
            unsigned q[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) q[j] = (unsigned)__builtin_amdgcn_fmed3f(acc[4 * i + j], 0.0f, lm[j]);
            put_group(q[0] | (q[1] << pos[1]) | (q[2] << pos[2]) | (q[3] << pos[3]), gt);
          };
          // Two accumulators, interleaved in program order: while the chain
          // of row block mb + 1 runs on the MFMA unit, row block mb is
          // quantized (one group of four channels per two steps).
          f32x16 acc0, acc1;
          // bf16 tokens: the wave's MFMA chains run at raised priority, so
          // that the SIMD's arbiter favours waves that keep the matrix core
          // fed over waves in their copy-out (measured about 1% faster)
          if (MODE == 0) __builtin_amdgcn_s_setprio(1);
#pragma unroll
          for (int i = 0; i < LA; ++i) readA(i);
          chain_init(0, acc0);
#pragma unroll
          for (int ks = 0; ks < 8; ++ks) chain_step(0, ks, acc0);
#pragma unroll
          for (int mb = 0; mb < 4; ++mb) {
            f32x16& cur = (mb & 1) ? acc1 : acc0;
            f32x16& nxt = (mb & 1) ? acc0 : acc1;
            if (mb < 3) chain_init(mb + 1, nxt);
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
              if (mb < 3) chain_step(mb + 1, ks, nxt);
              if (ks & 1) quant_group(mb, ks >> 1, cur);
            }
            if (MODE == 0 && mb == 2 && blk + ENC_WAVES < seg_end) load_frags(s, tt + ENC_WAVES);
            if (MODE == 0 && mb == 2) __builtin_amdgcn_s_setprio(0);  // the chains are done
          }
        } else {
#pragma unroll
          for (int mb = 0; mb < 4; ++mb) {
            // ---- 1: latent coefficients of channels 64h + 16mb + 4i + j
            f32x16 acc;
            const float* cf = static_cast<const float*>(a.x) + (rbase + trow) * 128 + 64 * h + 16 * mb;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const f32x4 v = *reinterpret_cast<const f32x4*>(cf + 4 * i);
#pragma unroll
              for (int j = 0; j < 4; ++j) acc[4 * i + j] = v[j];
            }
            // ---- 2: per group of four channels
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int coff = 4 * (16 * mb + 4 * i);  // byte offset of the group in a table
              unsigned q[4];
              // y = c/step + L/2 + eps_L; outside the guard band next to an
              // integer, floor(y) clamped to [0, L-1] is the exact threshold
              // count; inside it, or for NaN or a zero step, the fp32
              // thresholds decide.
              const f32x4 inv = LDS_AT(f32x4, pL + coff);
              const f32x4 yb = LDS_AT(f32x4, pL + 512 + coff);
              const f32x4 lm = LDS_AT(f32x4, pL + 1024 + coff);
              const u32x4 pos = LDS_AT(u32x4, pL + 1536 + coff);
              const f32x4 band = LDS_AT(f32x4, pL + 2048 + coff);
              const unsigned goff = LDS_AT(unsigned, pL + 2560 + coff);
              bool need = false;
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const float y = __builtin_fmaf(acc[4 * i + j], inv[j], yb[j]);
                q[j] = (unsigned)__builtin_amdgcn_fmed3f(y, 0.0f, lm[j]);
                need |= !(__builtin_amdgcn_fractf(y) >= band[j]);
              }
              if (__any(need)) {
                // exact decision against the thresholds t_k = fl32((k - L/2) step),
                // k = 1..L-1, rebuilt here from the fp64 step exactly as the
                // state builder forms them; the fast result is off by at most
                // one level
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                  const float c = acc[4 * i + j];
                  const float y = __builtin_fmaf(c, inv[j], yb[j]);
                  if (!(__builtin_amdgcn_fractf(y) >= band[j])) {
                    const int lm1 = (int)lm[j];
                    int qq = (int)q[j];
                    if (c != c) {
                      qq = 0;
                    } else if (inv[j] == 0.0f) {
                      qq = c >= 0.0f ? lm1 : 0;  // zero step: every threshold is 0
                    } else {
                      // fp64 table entry of channel 64h + 16mb + 4i + j (pL covers 64h floats)
                      const double s64 = LDS_AT(double, pL + 3072 + 256 * h + 2 * coff + 8 * j);
                      const double half = (double)((lm1 + 1) >> 1);
                      if (qq > 0 && c < (float)(((double)qq - half) * s64)) qq -= 1;
                      else if (qq < lm1 && c >= (float)(((double)(qq + 1) - half) * s64)) qq += 1;
                    }
                    q[j] = (unsigned)qq;
                  }
                }
              }
              u32x4 gt;
              gt[0] = goff;
              put_group(q[0] | (q[1] << pos[1]) | (q[2] << pos[2]) | (q[3] << pos[3]), gt);
            }
          }
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's ORs have landed
        __builtin_amdgcn_wave_barrier();
        // ---- 4: stream -> HBM, then clear it. The last block of a stream
        // also writes the zero padding up to the 16-byte boundary.
        const long long start = tt * 4LL * (long long)B;
        long long nbytes = 4LL * (long long)B;
        if (tok0 + ENC_BT >= n || nbytes > P_len - start) nbytes = P_len - start;
        unsigned char* dst = a.packed + s * a.packed_stride + start;
        if (tok0 < n0) {
          // an append's first block: the words holding bits of the records
          // already in the stream keep them
          const unsigned oldbits = (unsigned)((n0 - tok0) * (long long)B);
          const unsigned wold = (oldbits + 31u) >> 5;
          const unsigned* old = reinterpret_cast<const unsigned*>(dst);
          for (unsigned w2 = lane; w2 < wold; w2 += 64) {
            const unsigned rb = oldbits - 32u * w2;  // old bits in this word (all of them if >= 32)
            sStr[REC ? w2 + (w2 >> rsh) : est_idx(w2)] |= old[w2] & (rb >= 32u ? ~0u : (1u << rb) - 1u);
          }
          __builtin_amdgcn_s_waitcnt(0xc07f);
          __builtin_amdgcn_wave_barrier();
        }
        if (!STC_CHECK(a.packed_stride == 0 || start + nbytes <= a.packed_stride, DBG_ENC_RANGE)) nbytes = 0;
        if (REC) rec_copy_out<4>(sStr, dst, nbytes, clear, lane, rsh);  // (records of 32 * 2^s bits: whole words)
        else if (cw_kind == 4u) est_copy_out<4>(sStr, dst, nbytes, clear, lane);
        else if (cw_kind == 2u) est_copy_out<2>(sStr, dst, nbytes, clear, lane);
        else est_copy_out<1>(sStr, dst, nbytes, clear, lane);
      }
    }
    seg = seg_end;
  }
}

// ======================================================================
// Selective residual sketch of eigen / identity keys (tokens bf16): a wave
// takes 32-token blocks, recomputes the cell coordinates y = x U/step + L/2
// with the encode's scaled basis and its codes q = clamp(floor y), keeps
// r = step (y - q - 1/2) = c - c_hat on the kept channels (the step table is
// 0 elsewhere), and writes the signs of S r (rows permuted like the encode
// basis, hi / lo MFMA chains against r hi / lo) and |r| per token.
// ======================================================================
constexpr int SKE_WAVES = 8;
constexpr int SKE_BPW = 4;  // blocks per wave
constexpr size_t SKE_LDS = 4 * 128 * UROW + 3 * 128 * 4;

__global__ void __launch_bounds__(64 * SKE_WAVES, 2) k_sketch_eigen(EncK a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const long long s = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t32 = lane & 31, h = lane >> 5;
  const long long m = a.n_tokens;  // x rows of the call; row j is token n_old + j of the stream
  const long long si = state_index(a.map, s, a.n_states);
  if (si < 0) return;  // no state: sketch bits and norms untouched
  const unsigned char* st = a.states + (size_t)si * STATE_BYTES;
  const DevHdr* hdr = reinterpret_cast<const DevHdr*>(st + OFF_HDR);
  if (hdr->sketch_bits == 0) return;  // the whole workgroup: no sketch matrix for this stream
  float* sTb = reinterpret_cast<float*>(smem + 4 * 128 * UROW);  // L/2, L - 1, step (per channel)
  for (int i = tid; i < 128 * 16; i += 64 * SKE_WAVES) {
    const int row = i >> 4, c = i & 15;
    *reinterpret_cast<u32x4*>(smem + row * UROW + c * 16) = reinterpret_cast<const u32x4*>(st + OFF_UT_HI)[i];
    *reinterpret_cast<u32x4*>(smem + (128 + row) * UROW + c * 16) = reinterpret_cast<const u32x4*>(st + OFF_UT_LO)[i];
    *reinterpret_cast<u32x4*>(smem + (256 + row) * UROW + c * 16) = reinterpret_cast<const u32x4*>(st + OFF_SKP_HI)[i];
    *reinterpret_cast<u32x4*>(smem + (384 + row) * UROW + c * 16) = reinterpret_cast<const u32x4*>(st + OFF_SKP_LO)[i];
  }
  if (tid < 128) {
    sTb[tid] = hdr->yhalf[tid];
    sTb[128 + tid] = (float)hdr->lm1[tid];
    sTb[256 + tid] = hdr->step32[tid];
  }
  __syncthreads();
  unsigned ub = lds_offset(smem + t32 * UROW + 16 * h);                // basis rows: cols 16ks + 8h ..
  unsigned pb = lds_offset(smem + 256 * UROW + t32 * UROW + 128 * h);  // S rows: cols 64h + 8ks ..
  unsigned tb = lds_offset(reinterpret_cast<unsigned char*>(sTb + 64 * h));
  asm volatile("" : "+v"(ub), "+v"(pb), "+v"(tb));
  const lds_u8* uL = lds_ptr(ub);
  const lds_u8* pL = lds_ptr(pb);
  const lds_u8* tL = lds_ptr(tb);
  const long long nblk = (m + ENC_BT - 1) / ENC_BT;
  const long long b0 = ((long long)blockIdx.x * SKE_WAVES + wave) * SKE_BPW;
  for (long long blk = b0; blk < b0 + SKE_BPW && blk < nblk; ++blk) {
    const long long tok0 = blk * ENC_BT;
    const unsigned last = (unsigned)(m - 1 - tok0);
    const unsigned r = (unsigned)t32 < last ? (unsigned)t32 : last;
    const unsigned short* row = static_cast<const unsigned short*>(a.x) + s * a.x_stride + (tok0 + r) * a.ld;
    bf16x8 xf[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      xf[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(row + 16 * ks + 8 * h));
    u32x4 rh[8], rl[8];  // r of channels 64h + 8ks + i, bf16 hi / lo
    float ee = 0.0f;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      f32x16 acc;  // from yhalf, as the encode accumulates
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x4 yh = LDS_AT(f32x4, tL + 4 * (16 * mb + 4 * i));
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[4 * i + j] = yh[j];
      }
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const int off = 32 * mb * UROW + 32 * ks;
        acc = mfma32_bf16(LDS_AT(bf16x8, uL + off), xf[ks], acc);
        acc = mfma32_bf16(LDS_AT(bf16x8, uL + 128 * UROW + off), xf[ks], acc);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int coff = 4 * (16 * mb + 4 * i);
        const f32x4 lm = LDS_AT(f32x4, tL + 512 + coff);
        const f32x4 stp = LDS_AT(f32x4, tL + 1024 + coff);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int e = 4 * i + j;
          const float y = acc[e];
          const float q = (float)(unsigned)__builtin_amdgcn_fmed3f(y, 0.0f, lm[j]);
          const float rv = stp[j] == 0.0f ? 0.0f : stp[j] * (y - q - 0.5f);
          ee = __builtin_fmaf(rv, rv, ee);
          const __bf16 hi = (__bf16)rv;
          const __bf16 lo = (__bf16)(rv - (float)hi);
          const int ks = 2 * mb + (e >> 3), k2 = (e & 7) >> 1;
          const unsigned hv = __builtin_bit_cast(unsigned short, hi), lv = __builtin_bit_cast(unsigned short, lo);
          if (e & 1) {
            rh[ks][k2] |= hv << 16;
            rl[ks][k2] |= lv << 16;
          } else {
            rh[ks][k2] = hv;
            rl[ks][k2] = lv;
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    unsigned zw[2] = {0u, 0u};
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      f32x16 acc;
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[e] = 0.0f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const bf16x8 ph = LDS_AT(bf16x8, pL + 32 * mb * UROW + 16 * ks);
        const bf16x8 pl = LDS_AT(bf16x8, pL + 128 * UROW + 32 * mb * UROW + 16 * ks);
        acc = mfma32_bf16(ph, __builtin_bit_cast(bf16x8, rh[ks]), acc);
        acc = mfma32_bf16(ph, __builtin_bit_cast(bf16x8, rl[ks]), acc);
        acc = mfma32_bf16(pl, __builtin_bit_cast(bf16x8, rh[ks]), acc);
      }
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (acc[e] >= 0.0f) zw[mb >> 1] |= 1u << (16 * (mb & 1) + e);
      __builtin_amdgcn_sched_barrier(0);
    }
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(ee), __float_as_uint(ee), false, false);
      const unsigned s_lo = sw[0], s_hi = sw[1];
      ee = __uint_as_float(s_lo) + __uint_as_float(s_hi);
    }
    if (tok0 + t32 < m) {
      const long long tk = a.n_old + tok0 + t32;
      *reinterpret_cast<u32x2*>(a.sketch + s * a.sketch_stride + tk * 16 + 8 * h) = (u32x2){zw[0], zw[1]};
      if (h == 0) a.rnorm[s * a.rnorm_stride + tk] = sqrtf(ee);
    }
  }
}

int launch_sketch_eigen(const EncodeLaunch& L, void* stream) {
  static bool attr = false;
  if (!attr) {
    if (hipFuncSetAttribute((const void*)k_sketch_eigen, hipFuncAttributeMaxDynamicSharedMemorySize, (int)SKE_LDS) !=
        hipSuccess)
      return 1;
    attr = true;
  }
  EncK a{};
  a.states = L.states;
  a.map = L.map;
  a.n_states = L.n_states;
  a.n_tokens = L.n_tokens;
  a.ld = L.ld;
  a.x_stride = L.x_stride;
  a.x = L.x;
  a.n_old = L.n_old;
  a.sketch = L.sketch;
  a.rnorm = L.rnorm;
  a.sketch_stride = L.sketch_stride;
  a.rnorm_stride = L.rnorm_stride;
  const long long nblk = (L.n_tokens + ENC_BT - 1) / ENC_BT;
  dim3 grid((unsigned)((nblk + SKE_WAVES * SKE_BPW - 1) / (SKE_WAVES * SKE_BPW)), (unsigned)L.n_streams);
  hipLaunchKernelGGL(k_sketch_eigen, grid, dim3(64 * SKE_WAVES), SKE_LDS, (hipStream_t)stream, a);
  return hipGetLastError() != hipSuccess;
}

static bool g_enc_attr_done = false, g_dec_attr_done = false, g_att_attr_done = false;

int launch_encode_eigen(const EncodeLaunch& L, void* stream) {
  if (!g_enc_attr_done) {
    for (const void* k : {(const void*)k_encode_eigen<0, false>, (const void*)k_encode_eigen<1, false>,
                          (const void*)k_encode_eigen<2, false>, (const void*)k_encode_eigen<0, true>,
                          (const void*)k_encode_eigen<1, true>})
      if (hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)ENC_LDS) != hipSuccess) return 1;
    g_enc_attr_done = true;
  }
  EncK a;
  a.states = L.states;
  a.map = L.map;
  a.n_states = L.n_states;
  a.n_tokens = L.n_tokens;
  a.ld = L.ld;
  a.x_stride = L.x_stride;
  a.packed_stride = L.packed_stride;
  a.x = L.x;
  a.packed = L.packed;
  a.n_old = L.n_old;
  a.blk0 = L.n_old / ENC_BT;
  a.norms_stride = L.norms_stride;
  a.blocks_per_stream = (L.n_old + L.n_tokens + ENC_BT - 1) / ENC_BT - a.blk0;
  a.total_blocks = a.blocks_per_stream * L.n_streams;
  int dev = 0, cus = 256;
  (void)hipGetDevice(&dev);
  (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  // one workgroup per CU, or per block when there are fewer blocks than CUs
  // (short appends: each workgroup then stages one state for one block)
  long long grid = a.total_blocks < cus ? a.total_blocks : cus;
  a.blocks_per_wg = (a.total_blocks + grid - 1) / grid;
  grid = (a.total_blocks + a.blocks_per_wg - 1) / a.blocks_per_wg;
  a.grid = (int)grid;
  hipStream_t s = (hipStream_t)stream;
  if (L.mode == 0 && L.rec) hipLaunchKernelGGL((k_encode_eigen<0, true>), dim3(grid), dim3(ENC_THREADS), ENC_LDS, s, a);
  else if (L.mode == 0) hipLaunchKernelGGL((k_encode_eigen<0, false>), dim3(grid), dim3(ENC_THREADS), ENC_LDS, s, a);
  else if (L.mode == 1 && L.rec) hipLaunchKernelGGL((k_encode_eigen<1, true>), dim3(grid), dim3(ENC_THREADS), ENC_LDS, s, a);
  else if (L.mode == 1) hipLaunchKernelGGL((k_encode_eigen<1, false>), dim3(grid), dim3(ENC_THREADS), ENC_LDS, s, a);
  else hipLaunchKernelGGL((k_encode_eigen<2, false>), dim3(grid), dim3(ENC_THREADS), ENC_LDS, s, a);
  return hipGetLastError() != hipSuccess;
}

// ======================================================================
// Variable-width unpack, one quarter record (32 channels) per lane.
// Stage: the lane loads the HBM dwords covering its quarter record, aligns
// them to the record's first bit and stores them in a column of an LDS array
// (word k of task t at col[k * ntask + t]: consecutive lanes hit consecutive
// banks). Unpack: for each group of 4 channels the state's plan names the
// word pair and bit shift holding the group; one 64-bit window read gives 4
// codes. No read depends on another, so they pipeline; the plan is uniform.
// ======================================================================
constexpr int QW_MAX = 9;    // record-aligned words a quarter can need (256 bits + shift)

struct QPlan {
  unsigned e[8];
  unsigned off;
  unsigned nw;
};
__device__ __forceinline__ QPlan load_qplan(const DevHdr* hdr, int q) {
  QPlan r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r.e[i] = __builtin_amdgcn_readfirstlane(hdr->plan[q][i]);
  r.off = __builtin_amdgcn_readfirstlane(hdr->qoff[q]);
  r.nw = __builtin_amdgcn_readfirstlane(hdr->qwords[q]);
  return r;
}

// HBM dwords [d0, d0 + nw] of a stream of sdw >= 1 dwords (zero past the end
// or when !valid). Addresses are clamped instead of branched on, so the loads
// issue back to back.
__device__ __forceinline__ void load_quarter_raw(const unsigned* g, unsigned long long d0, unsigned long long sdw,
                                                 bool valid, unsigned nw, unsigned raw[QW_MAX + 1]) {
  const unsigned long long last = sdw - 1;
#pragma unroll
  for (int k = 0; k <= QW_MAX; ++k) {
    if ((unsigned)k <= nw) {
      const unsigned long long idx = d0 + k;
      const unsigned v = g[idx < last ? idx : last];
      raw[k] = (valid && idx <= last) ? v : 0u;
    } else {
      raw[k] = 0u;
    }
  }
}

__device__ __forceinline__ void stage_quarter(const unsigned raw[QW_MAX + 1], unsigned sh, unsigned nw, unsigned* col,
                                              int ntask) {
#pragma unroll
  for (int k = 0; k < QW_MAX; ++k)
    if ((unsigned)k < nw) col[k * ntask] = __builtin_amdgcn_alignbit(raw[k + 1], raw[k], sh);
}

__device__ __forceinline__ void unpack_quarter(const unsigned* col, int ntask, const QPlan& P, unsigned out[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const unsigned e = P.e[i];
    const unsigned k = e & 31u, sft = (e >> 5) & 31u;
    const unsigned b0 = (e >> 10) & 15u, b1 = (e >> 14) & 15u, b2 = (e >> 18) & 15u, b3 = (e >> 22) & 15u;
    const unsigned lo = col[k * ntask], hi = col[(k + 1) * ntask];
    const unsigned w = __builtin_amdgcn_alignbit(hi, lo, sft);
    unsigned v = __builtin_amdgcn_ubfe(w, 0u, b0);
    v |= __builtin_amdgcn_ubfe(w, b0, b1) << 8;
    v |= __builtin_amdgcn_ubfe(w, b0 + b1, b2) << 16;
    v |= __builtin_amdgcn_ubfe(w, b0 + b1 + b2, b3) << 24;
    out[i] = v;
  }
}

// ======================================================================
// Decode (eigen / identity): unpack -> MFMA with W = U diag(step) -> bias.
// x_hat_i = sum_j W_ij q_j - bias_i,  bias_i = sum_j W_ij (L_j - 1)/2,
// i.e. sum_j U_ij step_j (q_j - (L_j - 1)/2) with q the raw codes.
// A workgroup of 16 waves shares W (bf16 hi/lo rows, permuted) and the unpack
// tables in LDS; each wave decodes blocks of 32 tokens on its own:
//  1. The block's records (32 B bits) go from HBM into the wave's LDS stream
//     (word w at w + w/32; the pad slot after each 32 words repeats the next
//     word, so the word after k is always at idx(k) + 1).
//  2. Lane (h, t) takes channels [64h, 64h + 64) of token t: per group of four
//     channels one 64-bit window at the group's record bit holds the four
//     codes (offsets and widths from the tables); codes are exact in bf16.
//  3. MFMA 32x32x16 with A = W rows (M = output dims, stored so that lane half
//     h receives dims [64h, 64h + 64)) and B = codes (K = channels; lane half
//     h supplies the channels of its own half record), minus the bias, rounded
//     to the output dtype: each lane stores one 128-byte (bf16) or two
//     (fp32) whole row halves.
// ======================================================================
constexpr int DEC_WAVES = 16;
constexpr int DEC_THREADS = 64 * DEC_WAVES;
constexpr int DEC_BT = 32;
constexpr size_t DEC_LDS = 2 * 128 * UROW + 4 * 128 * 4 + (size_t)DEC_WAVES * EST_WORDS * 4;

struct DecK {
  const unsigned char* states;
  const int32_t* map;
  long long n_states, n_tokens, ld, x_stride, packed_stride;
  const unsigned char* packed;
  void* x;
  long long blocks_per_stream, total_blocks, blocks_per_wg;
  int grid;
};

// HBM bytes [0, nbytes) of a block (32 records of at most 64*NW bits, 4-byte
// aligned) -> wave stream, in two steps so that every load of a block is in
// flight at once: est_load issues dword loads (lane l takes words l, l + 64,
// ..; 256 contiguous bytes per instruction, scalar base) into NW registers;
// est_store writes them with the word following each 32-word run repeated in
// the pad slot before it.
// (a global-memory pointer held in scalar registers: the loads take it as
// their base and a 32-bit per-lane offset, with no 64-bit address math)
typedef __attribute__((address_space(1))) const unsigned gbl_u32;
__device__ __forceinline__ gbl_u32* uniform_ptr(const unsigned char* p) {
  const unsigned long long v = (unsigned long long)(uintptr_t)p;
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)v), hi = __builtin_amdgcn_readfirstlane((unsigned)(v >> 32));
  return reinterpret_cast<gbl_u32*>((uintptr_t)(((unsigned long long)hi << 32) | lo));
}
// (The chunk tests are uniform; only a ragged last chunk tests per lane.
// Word c = lane + 64k sits at est_idx(c) = est_idx(lane) + 66k.)
template <int NW>
__device__ __forceinline__ void est_load(unsigned (&w)[NW], const unsigned char* src, long long nbytes, int lane) {
  const int nw = (int)(nbytes >> 2);
  gbl_u32* s32 = uniform_ptr(src);
#pragma unroll
  for (int k = 0; k < NW; ++k) {
    const int c = lane + 64 * k;
    if (64 * k + 64 <= nw) w[k] = s32[(unsigned)c];
    else if (64 * k < nw) w[k] = c < nw ? s32[(unsigned)c] : 0u;
    else w[k] = 0u;
  }
}
template <int NW>
__device__ __forceinline__ void est_store(unsigned* str, const unsigned (&w)[NW], long long nbytes, int lane) {
  const int nw = (int)(nbytes >> 2);
  unsigned* base = str + est_idx((unsigned)lane);
  const bool pad = (lane & 31) == 0;  // lanes 0 and 32 start a 32-word run
#pragma unroll
  for (int k = 0; k < NW; ++k) {
    if (64 * k >= nw) break;
    if (64 * k + 64 <= nw || lane + 64 * k < nw) {
      base[66 * k] = w[k];
      if (pad && (lane != 0 || k > 0)) base[66 * k - 1] = w[k];
    }
  }
}

// REC layout: word c = lane + 64k of a block of 32 records of 32 * 2^sh bits
// (sh <= 5) goes to c + (c >> sh), so record T starts at word T (2^sh + 1):
// one pad word after each record keeps the lanes' reads on distinct banks.
template <int NW>
__device__ __forceinline__ void rec_store(unsigned* str, const unsigned (&w)[NW], long long nbytes, int lane,
                                          unsigned sh) {
  const int nw = (int)(nbytes >> 2);
  const unsigned stride = 64u + (64u >> sh);
  unsigned* base = str + lane + ((unsigned)lane >> sh);
#pragma unroll
  for (int k = 0; k < NW; ++k) {
    if (64 * k >= nw) break;
    if (64 * k + 64 <= nw || lane + 64 * k < nw) base[k * stride] = w[k];
  }
}

// W16: one MFMA pass with the fp16 W rows and fp16 codes (bf16 output of low
// budgets; the host decides), else the bf16 hi and lo passes.
template <int F32OUT, int NW, bool W16>
__global__ void __launch_bounds__(DEC_THREADS, 1) k_decode_eigen(DecK a) {
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* sWhi = smem;
  unsigned* sTab = reinterpret_cast<unsigned*>(smem + 2 * 128 * UROW);  // goff, pos, width, bias
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t32 = lane & 31, h = lane >> 5;
  unsigned* sStr = sTab + 4 * 128 + wave * EST_WORDS;
  const int lw = xcd_logical(blockIdx.x, a.grid);
  const long long b_begin = (long long)lw * a.blocks_per_wg;
  long long b_end = b_begin + a.blocks_per_wg;
  if (b_end > a.total_blocks) b_end = a.total_blocks;
  const long long n = a.n_tokens;

  for (long long seg = b_begin; seg < b_end;) {
    const long long s = seg / a.blocks_per_stream;
    long long seg_end = (s + 1) * a.blocks_per_stream;
    if (seg_end > b_end) seg_end = b_end;
    const long long si = state_index(a.map, s, a.n_states);
    if (si < 0) {  // (uniform over the workgroup) no state: NaN rows
      for (long long blk = seg + wave; blk < seg_end; blk += DEC_WAVES) {
        const long long tok0 = (blk - s * a.blocks_per_stream) * DEC_BT;
        for (int i = lane; i < DEC_BT * 128; i += 64) {
          const long long tok = tok0 + (i >> 7);
          if (tok >= n) break;
          if (F32OUT) static_cast<float*>(a.x)[s * a.x_stride + tok * a.ld + (i & 127)] = __builtin_nanf("");
          else static_cast<unsigned short*>(a.x)[s * a.x_stride + tok * a.ld + (i & 127)] = 0x7FC0u;
        }
      }
      seg = seg_end;
      continue;
    }
    const unsigned char* st = a.states + (size_t)si * STATE_BYTES;
    const DevHdr* hdr = reinterpret_cast<const DevHdr*>(st + OFF_HDR);
    const unsigned B = (unsigned)__builtin_amdgcn_readfirstlane(hdr->total_bits);
    __syncthreads();  // every wave is done with the previous state
    {
      const u32x4* ghi = reinterpret_cast<const u32x4*>(st + (W16 ? OFF_W16 : OFF_W_HI));
      const u32x4* glo = reinterpret_cast<const u32x4*>(st + OFF_W_LO);
      for (int i = tid; i < 128 * 16; i += DEC_THREADS) {
        const int row = i >> 4, c = i & 15;
        *reinterpret_cast<u32x4*>(sWhi + row * UROW + c * 16) = ghi[i];
        if (!W16) *reinterpret_cast<u32x4*>(sWhi + 128 * UROW + row * UROW + c * 16) = glo[i];
      }
    }
    if (tid < 128) {
      sTab[tid] = tid < 32 ? (unsigned)hdr->off[4 * tid] : 0u;              // record offset of group tid
      sTab[128 + tid] = (unsigned)hdr->off[tid] - (unsigned)hdr->off[tid & ~3];  // offset in the group
      sTab[256 + tid] = (unsigned)hdr->bits[tid];                            // width
      reinterpret_cast<float*>(sTab)[384 + tid] = -(W16 ? hdr->bias16[tid] : hdr->bias[tid]);  // natural dim order
    }
    __syncthreads();
    const long long P_len = packed_len((long long)B, n);
    const unsigned cw_kind = (B & 3u) == 0u ? 4u : ((B & 1u) == 0u ? 2u : 1u);
    // bytes of a block's records (the stream's last block may be short)
    auto rec_bytes = [&](long long tt2, long long& start) {
      start = tt2 * 4LL * (long long)B;
      const long long nb0 = 4LL * (long long)B;
      const long long nb = nb0 > P_len - start ? P_len - start : nb0;
      return STC_CHECK(a.packed_stride == 0 || start + nb <= a.packed_stride, DBG_DEC_RANGE) ? nb : 0LL;
    };
    // NW <= 4 (records of at most 256 bits): the next block's records are
    // requested as soon as the current ones are in LDS, into the same
    // registers, so the load runs under this block's work
    constexpr bool PREF = NW <= 4;
    unsigned wr[NW];
    if (PREF && B > 0 && seg + wave < seg_end) {
      long long st0;
      const long long nb0 = rec_bytes(seg + wave - s * a.blocks_per_stream, st0);
      est_load<NW>(wr, a.packed + s * a.packed_stride + st0, nb0, lane);
    }
    for (long long blk = seg + wave; blk < seg_end; blk += DEC_WAVES) {
      const long long tt = blk - s * a.blocks_per_stream;
      const long long tok0 = tt * DEC_BT;
      // ---- 1: records -> LDS stream
      if (B > 0) {
        long long start;
        const long long nbytes = rec_bytes(tt, start);
        if (!PREF) est_load<NW>(wr, a.packed + s * a.packed_stride + start, nbytes, lane);
        est_store<NW>(sStr, wr, nbytes, lane);
        if (PREF && blk + DEC_WAVES < seg_end) {
          long long st2;
          const long long nb2 = rec_bytes(tt + DEC_WAVES, st2);
          est_load<NW>(wr, a.packed + s * a.packed_stride + st2, nb2, lane);
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
        __builtin_amdgcn_wave_barrier();
      }
      // ---- 2: codes of channels 64h + 8ks + i as bf16 (B fragments)
      unsigned tb = lds_offset(reinterpret_cast<unsigned char*>(sTab + 64 * h));
      unsigned wb = lds_offset(sWhi + t32 * UROW + 128 * h);
      asm volatile("" : "+v"(tb), "+v"(wb));
      const lds_u8* tL = lds_ptr(tb);
      const lds_u8* wL = lds_ptr(wb);
      const unsigned tB = (unsigned)t32 * B;
      // W16: the codes' scale 2^-e16 (exact products in fp16)
      const f16x2 cscale = __builtin_bit_cast(f16x2, (unsigned)__builtin_amdgcn_readfirstlane(hdr->code16));
      u32x4 cf[8];
      // groups (channels 64h + 4g .. +3) four at a time: the four record
      // offsets in one read, the position and width tables and then the
      // eight stream words requested together, so that a batch waits on LDS
      // twice instead of once per read
      const lds_u8* tG = lds_ptr(lds_offset(reinterpret_cast<unsigned char*>(sTab + 16 * h)));
      // (two at a time in the fp32-output and 16-word instances, whose
      // registers would not hold four)
      constexpr int GB = (F32OUT || NW > 8) ? 2 : 4;
#pragma unroll
      for (int gb = 0; gb < 16; gb += GB) {
        // (a state without kept channels, B = 0, has all-zero tables: it
        // reads the stream's first two words and extracts zero-width codes)
        const u32x4 go = LDS_AT(u32x4, tG + 4 * (gb & ~3));
        u32x4 pos[GB], wid[GB];
#pragma unroll
        for (int k = 0; k < GB; ++k) {
          pos[k] = LDS_AT(u32x4, tL + 512 + 16 * (gb + k));
          wid[k] = LDS_AT(u32x4, tL + 1024 + 16 * (gb + k));
        }
        unsigned P[GB], lo[GB], hi[GB];
#pragma unroll
        for (int k = 0; k < GB; ++k) {
          P[k] = tB + go[(gb & 3) + k];
          const unsigned ix = est_idx_bit(P[k]);
          if (STC_CHECK(ix + 1u < (unsigned)EST_WORDS, DBG_DEC_STREAM)) {
            lo[k] = sStr[ix];
            hi[k] = sStr[ix + 1];
          } else {
            lo[k] = hi[k] = 0u;
          }
        }
#pragma unroll
        for (int k = 0; k < GB; ++k) {
          const int g = gb + k;
          const unsigned w = __builtin_amdgcn_alignbit(hi[k], lo[k], P[k] & 31u);
          unsigned code[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) code[j] = __builtin_amdgcn_ubfe(w, pos[k][j], wid[k][j]);
#pragma unroll
          for (int j = 0; j < 2; ++j)
            cf[g >> 1][2 * (g & 1) + j] =
                W16 ? __builtin_bit_cast(unsigned, (f16x2){(_Float16)(unsigned short)code[2 * j],
                                                           (_Float16)(unsigned short)code[2 * j + 1]} *
                                                       cscale)
                    : bf16_pair_exact((float)code[2 * j], (float)code[2 * j + 1]);
        }
      }
      // ---- 3: reconstruct dims 64h + 16ob + r of token t
      const long long tok = tok0 + t32;
      const bool tok_ok = tok < n;
      u32x4 pk[4][2];  // bf16 output, dims 64h + 16ob + 8c .. +7 in pk[ob][c]
      // the rows of W for chain step i = 8 ob + ks, read DLA steps ahead of
      // their MFMA (kept there by a scheduling barrier, as in the encode;
      // the bf16 hi / lo pair keeps DLA = 0: its registers would not hold
      // the extra rows)
      constexpr int DLA = W16 ? 1 : 0;
      u32x4 whr[DLA + 1], wlr[DLA + 1];
      auto readW = [&](const int i) {
        const int off = 32 * (i >> 3) * UROW + 16 * (i & 7);
        whr[i % (DLA + 1)] = LDS_AT(u32x4, wL + off);
        if (!W16) wlr[i % (DLA + 1)] = LDS_AT(u32x4, wL + 128 * UROW + off);
      };
#pragma unroll
      for (int i = 0; i < DLA; ++i) readW(i);
#pragma unroll
      for (int ob = 0; ob < 4; ++ob) {
        // the accumulator starts at -bias
        f32x16 acc;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4 nb = LDS_AT(f32x4, tL + 1536 + 64 * ob + 16 * q4);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[4 * q4 + e] = nb[e];
        }
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          const int i = 8 * ob + ks;
          if (i + DLA < 32) readW(i + DLA);
          if (DLA > 0) __builtin_amdgcn_sched_barrier(0);
          if (W16) {
            acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, whr[i % (DLA + 1)]),
                                                         __builtin_bit_cast(f16x8, cf[ks]), acc, 0, 0, 0);
          } else {
            acc = mfma32_bf16(__builtin_bit_cast(bf16x8, whr[i % (DLA + 1)]), __builtin_bit_cast(bf16x8, cf[ks]), acc);
            acc = mfma32_bf16(__builtin_bit_cast(bf16x8, wlr[i % (DLA + 1)]), __builtin_bit_cast(bf16x8, cf[ks]), acc);
          }
        }
        if (F32OUT) {
          if (tok_ok) {
            float* o = static_cast<float*>(a.x) + s * a.x_stride + tok * a.ld + 64 * h + 16 * ob;
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
              __builtin_nontemporal_store((f32x4){acc[4 * q4], acc[4 * q4 + 1], acc[4 * q4 + 2], acc[4 * q4 + 3]},
                                          reinterpret_cast<f32x4*>(o) + q4);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float v0 = acc[2 * e];
            const float v1 = acc[2 * e + 1];
            pk[ob][e >> 2][e & 3] = pack_bf16x2(v0, v1);
          }
        }
      }
      if (!F32OUT) {
        // Two rounds through the LDS stream (free once the codes are out):
        // the lanes of half r put their 128-byte row halves (one cache line
        // each) into rows of 33 words, then the wave writes the 32 lines with
        // 16-byte stores, eight lanes per line. The reconstructed rows are
        // stored non-temporally: they are not read back by this library, and
        // cached dirty lines would be written back during the launches after.
        const int nrow = (int)(n - tok0 < DEC_BT ? n - tok0 : DEC_BT);
        unsigned short* obase = static_cast<unsigned short*>(a.x) + s * a.x_stride + tok0 * a.ld;
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          __builtin_amdgcn_s_waitcnt(0xc07f);
          __builtin_amdgcn_wave_barrier();
          if (h == r) {
#pragma unroll
            for (int ob = 0; ob < 4; ++ob)
#pragma unroll
              for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int e = 0; e < 4; ++e) sStr[33 * t32 + 8 * ob + 4 * c + e] = pk[ob][c][e];
          }
          __builtin_amdgcn_s_waitcnt(0xc07f);
          __builtin_amdgcn_wave_barrier();
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int row = 8 * k + (lane >> 3), c = lane & 7;
            if (row < nrow) {
              const u32x4 v = (u32x4){sStr[33 * row + 4 * c], sStr[33 * row + 4 * c + 1], sStr[33 * row + 4 * c + 2],
                                      sStr[33 * row + 4 * c + 3]};
              __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(obase + row * a.ld + 64 * r + 8 * c));
            }
          }
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);
        __builtin_amdgcn_wave_barrier();
      }
    }
    seg = seg_end;
  }
}

int launch_decode_eigen(const DecodeLaunch& L, void* stream) {
  if (!g_dec_attr_done) {
    for (const void* k : {(const void*)k_decode_eigen<0, 8, false>, (const void*)k_decode_eigen<1, 8, false>,
                          (const void*)k_decode_eigen<0, 16, false>, (const void*)k_decode_eigen<1, 16, false>,
                          (const void*)k_decode_eigen<0, 8, true>, (const void*)k_decode_eigen<0, 16, true>,
                          (const void*)k_decode_eigen<0, 4, true>, (const void*)k_decode_eigen<0, 4, false>})
      if (hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)DEC_LDS) != hipSuccess) return 1;
    g_dec_attr_done = true;
  }
  DecK a;
  a.states = L.states;
  a.map = L.map;
  a.n_states = L.n_states;
  a.n_tokens = L.n_tokens;
  a.ld = L.ld;
  a.x_stride = L.x_stride;
  a.packed_stride = L.packed_stride;
  a.packed = L.packed;
  a.x = L.x;
  a.blocks_per_stream = (L.n_tokens + DEC_BT - 1) / DEC_BT;
  a.total_blocks = a.blocks_per_stream * L.n_streams;
  int dev = 0, cus = 256;
  (void)hipGetDevice(&dev);
  (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  // one workgroup per CU, or per block when there are fewer blocks than CUs
  // (short appends: each workgroup then stages one state for one block)
  long long grid = a.total_blocks < cus ? a.total_blocks : cus;
  a.blocks_per_wg = (a.total_blocks + grid - 1) / grid;
  grid = (a.total_blocks + a.blocks_per_wg - 1) / a.blocks_per_wg;
  a.grid = (int)grid;
  hipStream_t s = (hipStream_t)stream;
  // records of up to 512 bits: 8 staging words per lane, else 16
  const bool small = L.max_bits <= 512;
  if (L.f32out) {
    if (small) hipLaunchKernelGGL((k_decode_eigen<1, 8, false>), dim3(grid), dim3(DEC_THREADS), DEC_LDS, s, a);
    else hipLaunchKernelGGL((k_decode_eigen<1, 16, false>), dim3(grid), dim3(DEC_THREADS), DEC_LDS, s, a);
  } else if (L.w16) {
    if (L.max_bits <= 256) hipLaunchKernelGGL((k_decode_eigen<0, 4, true>), dim3(grid), dim3(DEC_THREADS), DEC_LDS, s, a);
    else if (small) hipLaunchKernelGGL((k_decode_eigen<0, 8, true>), dim3(grid), dim3(DEC_THREADS), DEC_LDS, s, a);
    else hipLaunchKernelGGL((k_decode_eigen<0, 16, true>), dim3(grid), dim3(DEC_THREADS), DEC_LDS, s, a);
  } else {
    if (L.max_bits <= 256) hipLaunchKernelGGL((k_decode_eigen<0, 4, false>), dim3(grid), dim3(DEC_THREADS), DEC_LDS, s, a);
    else if (small) hipLaunchKernelGGL((k_decode_eigen<0, 8, false>), dim3(grid), dim3(DEC_THREADS), DEC_LDS, s, a);
    else hipLaunchKernelGGL((k_decode_eigen<0, 16, false>), dim3(grid), dim3(DEC_THREADS), DEC_LDS, s, a);
  }
  return hipGetLastError() != hipSuccess;
}

// ======================================================================
// Walsh-Hadamard path. Encode: the rotation x -> H D x is a dense +-1
// matrix, exact in bf16, so it runs as MFMA chains like the eigen path, with
// the 3-bit codebook in place of the per-channel uniform quantizer. Decode:
// one token per lane, codebook values -> FWHT butterflies -> scale by
// |x|/sqrt(d) -> signs.
// ======================================================================
struct RhtK {
  const unsigned char* states;
  const int32_t* map;
  long long n_states, n_tokens, ld, x_stride, packed_stride;
  const void* x;
  void* xo;
  unsigned char* packed;
  const unsigned char* packed_in;
  float* norms;
  const float* norms_in;
  long long n_old, norms_stride;  // encode: tokens already in the streams; norms row stride
  unsigned char* sketch;          // key residual sketch: 16 bytes per token, stream stride sketch_stride
  float* rnorm;                   // |r| per token, stream stride rnorm_stride
  long long sketch_stride, rnorm_stride;
  int f32out;
};

__device__ __forceinline__ void fwht128(float v[128]) {
#pragma unroll
  for (int h = 1; h < 128; h <<= 1)
#pragma unroll
    for (int i = 0; i < 128; ++i)
      if (!(i & h)) {
        const float x0 = v[i], x1 = v[i + h];
        v[i] = x0 + x1;
        v[i + h] = x0 - x1;
      }
}

// 3-bit code of a rotated value c: the count of the sorted scaled
// thresholds T_0 <= .. <= T_6 that are <= c, by binary search.
__device__ __forceinline__ unsigned rht_code(float c, const float T[7]) {
  const bool b2 = c >= T[3];
  const float t1 = b2 ? T[5] : T[1];
  const bool b1 = c >= t1;
  const float ta = b1 ? T[6] : T[4], tb = b1 ? T[2] : T[0];
  const float t0 = b2 ? ta : tb;
  const bool b0 = c >= t0;
  return (b2 ? 4u : 0u) | (b1 ? 2u : 0u) | (b0 ? 1u : 0u);
}

// Encode: a wave takes blocks of 32 tokens. The rotation H D x is one
// 32x32x16 MFMA chain per 32 channels against the +-1 rows of H D (exact in
// bf16, so the products are exact and only the fp32 sums round); lane (h, t)
// receives channels [64h, 64h + 64) of token t, whose 3-bit codes fill
// words 6h .. 6h + 5 of the token's 48-byte record. The norm comes from the
// lane's 64 input values and the other half's, and the code of a value c is
// the count of scaled thresholds t_k |x| sqrt(d) <= c.
constexpr int RHT_WAVES = 4;
constexpr int RHT_BPW = 4;  // blocks per wave
constexpr size_t RHT_LDS = 128 * UROW;
// With the key residual sketch (SKETCH): 8 waves, and P = S D H / sqrt(d)
// (bf16 hi / lo rows) plus the codebook next to the basis in LDS. Each value
// leaves e' = c - y_hat |x| sqrt(d) = |x| sqrt(d) (y - y_hat) in the rotated
// basis; S r = P e' / sqrt(d) has the sign of P e', and |r| = |e'| / sqrt(d).
constexpr int RHTS_WAVES = 8;
constexpr size_t RHTS_LDS = 3 * 128 * UROW + 32;

template <bool SKETCH>
__global__ void __launch_bounds__(SKETCH ? 64 * RHTS_WAVES : 64 * RHT_WAVES, SKETCH ? 2 : 4)
    k_rht_encode(RhtK a) {
  constexpr int NWV = SKETCH ? RHTS_WAVES : RHT_WAVES;
  extern __shared__ __align__(16) unsigned char smem[];
  const long long s = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t32 = lane & 31, h = lane >> 5;
  const long long n = a.n_tokens;  // x rows of the call; row j is token n_old + j of the stream
  const long long si = state_index(a.map, s, a.n_states);
  if (si < 0) return;  // no state: records, norms and sketch untouched
  const unsigned char* st = a.states + (size_t)si * STATE_BYTES;
  const DevHdr* hdr = reinterpret_cast<const DevHdr*>(st + OFF_HDR);
  {
    const u32x4* g = reinterpret_cast<const u32x4*>(st + OFF_UT_HI);
    for (int i = tid; i < 128 * 16; i += 64 * NWV) {
      const int row = i >> 4, c = i & 15;
      *reinterpret_cast<u32x4*>(smem + row * UROW + c * 16) = g[i];
      if (SKETCH) {
        *reinterpret_cast<u32x4*>(smem + (128 + row) * UROW + c * 16) = reinterpret_cast<const u32x4*>(st + OFF_SKP_HI)[i];
        *reinterpret_cast<u32x4*>(smem + (256 + row) * UROW + c * 16) = reinterpret_cast<const u32x4*>(st + OFF_SKP_LO)[i];
      }
    }
    if (SKETCH && tid < 8) reinterpret_cast<float*>(smem + 3 * 128 * UROW)[tid] = hdr->cb[tid];
  }
  float thr[7];
#pragma unroll
  for (int k = 0; k < 7; ++k) thr[k] = hdr->cb_thr[k];
  __syncthreads();
  unsigned ub = lds_offset(smem + t32 * UROW + 16 * h);
  asm volatile("" : "+v"(ub));
  const lds_u8* uL = lds_ptr(ub);
  unsigned pb = lds_offset(smem + 128 * UROW + t32 * UROW + 128 * h);  // P rows: lane reads cols 64h + 8ks ..
  asm volatile("" : "+v"(pb));
  const lds_u8* pL = lds_ptr(pb);
  const float* sCb = reinterpret_cast<const float*>(smem + 3 * 128 * UROW);
  const long long nblk = (n + ENC_BT - 1) / ENC_BT;
  const long long b0 = ((long long)blockIdx.x * NWV + wave) * RHT_BPW;
  for (long long blk = b0; blk < b0 + RHT_BPW && blk < nblk; ++blk) {
    const long long tok0 = blk * ENC_BT;
    const unsigned last = (unsigned)(n - 1 - tok0);
    const unsigned r = (unsigned)t32 < last ? (unsigned)t32 : last;
    const unsigned short* row = static_cast<const unsigned short*>(a.x) + s * a.x_stride + (tok0 + r) * a.ld;
    bf16x8 xf[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      xf[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(row + 16 * ks + 8 * h));
    // squared norm: this lane's 64 values, then the other half's
    float ss = 0.0f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const u32x4 w = __builtin_bit_cast(u32x4, xf[ks]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = __uint_as_float(w[e] << 16), hi = __uint_as_float(w[e] & 0xffff0000u);
        ss = __builtin_fmaf(lo, lo, ss);
        ss = __builtin_fmaf(hi, hi, ss);
      }
    }
    {
      // element 0: the low half's sum, element 1: the high half's, in every lane
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(ss), __float_as_uint(ss), false, false);
      const unsigned s_lo = sw[0], s_hi = sw[1];
      ss = __uint_as_float(s_lo) + __uint_as_float(s_hi);
    }
    const float nu = sqrtf(ss);
    const float sc = nu * 11.313708498984761f;
    float T[7];
#pragma unroll
    for (int k = 0; k < 7; ++k) T[k] = nu > 0.0f ? thr[k] * sc : thr[k];
    unsigned w[6] = {0u, 0u, 0u, 0u, 0u, 0u};
    // SKETCH: e' of channels 64h + 8ks + i as bf16 hi / lo B fragments, |e'|^2
    u32x4 eh[8], el[8];
    float ee = 0.0f;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      f32x16 acc;
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[e] = 0.0f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) acc = mfma32_bf16(LDS_AT(bf16x8, uL + 32 * mb * UROW + 32 * ks), xf[ks], acc);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float c = acc[e];
        const unsigned q = rht_code(c, T);
        const int bp = 3 * (16 * mb + e);  // bit of channel 64h + 16mb + e in the half record
        w[bp >> 5] |= q << (bp & 31);
        if ((bp & 31) > 29) w[(bp >> 5) + 1] |= q >> (32 - (bp & 31));
        if (SKETCH) {
          const float ep = __builtin_fmaf(-sCb[q], sc, c);  // c - y_hat |x| sqrt(d)
          ee = __builtin_fmaf(ep, ep, ee);
          const __bf16 hi = (__bf16)ep;
          const __bf16 lo = (__bf16)(ep - (float)hi);
          // channel 64h + 16mb + e is element e % 8 of fragment 2mb + e / 8
          const int ks = 2 * mb + (e >> 3), k2 = (e & 7) >> 1;
          const unsigned hv = __builtin_bit_cast(unsigned short, hi), lv = __builtin_bit_cast(unsigned short, lo);
          if (e & 1) {
            eh[ks][k2] |= hv << 16;
            el[ks][k2] |= lv << 16;
          } else {
            eh[ks][k2] = hv;
            el[ks][k2] = lv;
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);  // one row block's accumulators live at a time
    }
    if (tok0 + t32 < n && STC_CHECK(a.packed_stride == 0 || (a.n_old + tok0 + t32 + 1) * 48 <= a.packed_stride,
                                    DBG_RHT_RANGE)) {
      const long long tk = a.n_old + tok0 + t32;
      u32x2* dst = reinterpret_cast<u32x2*>(a.packed + s * a.packed_stride + tk * 48 + 24 * h);
      dst[0] = (u32x2){w[0], w[1]};
      dst[1] = (u32x2){w[2], w[3]};
      dst[2] = (u32x2){w[4], w[5]};
      if (h == 0) a.norms[s * a.norms_stride + tk] = nu;
    }
    if (SKETCH && hdr->sketch_bits != 0) {
      // sign bits of P e' for sketch rows 64h + 16mb + e of token t
      unsigned zw[2] = {0u, 0u};
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        f32x16 acc;
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[e] = 0.0f;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          const bf16x8 ph = LDS_AT(bf16x8, pL + 32 * mb * UROW + 16 * ks);
          const bf16x8 pl = LDS_AT(bf16x8, pL + 128 * UROW + 32 * mb * UROW + 16 * ks);
          acc = mfma32_bf16(ph, __builtin_bit_cast(bf16x8, eh[ks]), acc);
          acc = mfma32_bf16(ph, __builtin_bit_cast(bf16x8, el[ks]), acc);
          acc = mfma32_bf16(pl, __builtin_bit_cast(bf16x8, eh[ks]), acc);
        }
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (acc[e] >= 0.0f) zw[mb >> 1] |= 1u << (16 * (mb & 1) + e);
        __builtin_amdgcn_sched_barrier(0);
      }
      {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(ee), __float_as_uint(ee), false, false);
        const unsigned s_lo = sw[0], s_hi = sw[1];
        ee = __uint_as_float(s_lo) + __uint_as_float(s_hi);
      }
      if (tok0 + t32 < n) {
        const long long tk = a.n_old + tok0 + t32;
        *reinterpret_cast<u32x2*>(a.sketch + s * a.sketch_stride + tk * 16 + 8 * h) = (u32x2){zw[0], zw[1]};
        if (h == 0) a.rnorm[s * a.rnorm_stride + tk] = sqrtf(ee) * 0.08838834764831845f;
      }
    }
  }
}

// Butterfly encode (no matrix product): the same blocks of 32 tokens per
// wave and the same input fragments, lane (h, t) holding channels
// 16 ks + 8 h + i (ks, i < 8) of token t. The signs D flip bf16 sign bits
// by one XOR per value pair (masks per half in LDS); the fast Walsh-Hadamard
// transform then runs in fp32 registers: the butterflies of channel bits 0,
// 1, 2, 4, 5 and 6 inside the lane (64 values), then one permlane32 swap per
// register pair trades channel bit 6 for bit 3 between the two halves of
// the wave, and the bit-3 butterfly finishes inside the lane. Afterwards
// lane (h, t) holds channels 64 h + [0, 64) of token t, the half record it
// writes, exactly as the matrix-core kernel does; the quantizer and the
// record layout are the same.
constexpr int RHTB_WAVES = 4;
__global__ void __launch_bounds__(64 * RHTB_WAVES, 4) k_rht_encode_bfly(RhtK a) {
  __shared__ __align__(16) unsigned smask[2][32];
  const long long s = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t32 = lane & 31, h = lane >> 5;
  const long long n = a.n_tokens;
  const long long si = state_index(a.map, s, a.n_states);
  if (si < 0) return;  // no state: records and norms untouched
  const DevHdr* hdr = reinterpret_cast<const DevHdr*>(a.states + (size_t)si * STATE_BYTES + OFF_HDR);
  if (tid < 64) {
    // word k of half hh: channels c0 = 16 (k / 4) + 8 hh + 2 (k % 4) and c0 + 1 (bf16 sign bits 15, 31)
    const int hh = tid >> 5, k = tid & 31;
    const int c0 = 16 * (k >> 2) + 8 * hh + 2 * (k & 3);
    smask[hh][k] = (hdr->sign[c0] < 0.0f ? 0x8000u : 0u) | (hdr->sign[c0 + 1] < 0.0f ? 0x80000000u : 0u);
  }
  float thr[7];
#pragma unroll
  for (int k = 0; k < 7; ++k) thr[k] = hdr->cb_thr[k];
  __syncthreads();
  const u32x4* mrow = reinterpret_cast<const u32x4*>(&smask[h][0]);
  const long long nblk = (n + ENC_BT - 1) / ENC_BT;
  const long long b0 = ((long long)blockIdx.x * RHTB_WAVES + wave) * RHT_BPW;
  for (long long blk = b0; blk < b0 + RHT_BPW && blk < nblk; ++blk) {
    const long long tok0 = blk * ENC_BT;
    const unsigned last = (unsigned)(n - 1 - tok0);
    const unsigned r = (unsigned)t32 < last ? (unsigned)t32 : last;
    const unsigned short* row = static_cast<const unsigned short*>(a.x) + s * a.x_stride + (tok0 + r) * a.ld;
    u32x4 xw[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) xw[ks] = *reinterpret_cast<const u32x4*>(row + 16 * ks + 8 * h);
    float ss = 0.0f;
    // v[8 ks + i]: channel 16 ks + 8 h + i; D and the bit-0 butterfly on each bf16 pair
    float v[64];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const u32x4 m = mrow[ks];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const unsigned w = xw[ks][e];
        const float x0 = __uint_as_float(w << 16), x1 = __uint_as_float(w & 0xffff0000u);
        ss = __builtin_fmaf(x0, x0, ss);
        ss = __builtin_fmaf(x1, x1, ss);
        const unsigned ws = w ^ m[e];
        const float y0 = __uint_as_float(ws << 16), y1 = __uint_as_float(ws & 0xffff0000u);
        v[8 * ks + 2 * e] = y0 + y1;
        v[8 * ks + 2 * e + 1] = y0 - y1;
      }
    }
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(ss), __float_as_uint(ss), false, false);
      const unsigned s_lo = sw[0], s_hi = sw[1];
      ss = __uint_as_float(s_lo) + __uint_as_float(s_hi);
    }
    // channel bits 1, 2 (register bits 1, 2) and 4, 5, 6 (register bits 3, 4, 5)
#pragma unroll
    for (int hb = 2; hb < 64; hb <<= 1)
#pragma unroll
      for (int i = 0; i < 64; ++i)
        if (!(i & hb)) {
          const float p = v[i], q = v[i + hb];
          v[i] = p + q;
          v[i + hb] = p - q;
        }
    // channel bit 3 across the halves: lower lanes receive the pair of v[i]
    // (channel bit 6 clear), upper lanes that of v[i + 32]; afterwards v[i]
    // is channel 64 h + 16 (i / 8) + i % 8 and v[i + 32] the same + 8
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[i]), __float_as_uint(v[i + 32]), false,
                                                        false);
      const float p = __uint_as_float(sw[0]), q = __uint_as_float(sw[1]);
      v[i] = p + q;
      v[i + 32] = p - q;
    }
    const float nu = sqrtf(ss);
    const float sc = nu * 11.313708498984761f;
    float T[7];
#pragma unroll
    for (int k = 0; k < 7; ++k) T[k] = nu > 0.0f ? thr[k] * sc : thr[k];
    unsigned w[6] = {0u, 0u, 0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      const int jl = 16 * ((i & 31) >> 3) + 8 * (i >> 5) + (i & 7);  // channel 64 h + jl
      const unsigned q = rht_code(v[i], T);
      const int bp = 3 * jl;
      w[bp >> 5] |= q << (bp & 31);
      if ((bp & 31) > 29) w[(bp >> 5) + 1] |= q >> (32 - (bp & 31));
      if ((i & 7) == 7) __builtin_amdgcn_sched_barrier(0);  // compare masks of 8 values live at a time
    }
    if (tok0 + t32 < n && STC_CHECK(a.packed_stride == 0 || (a.n_old + tok0 + t32 + 1) * 48 <= a.packed_stride,
                                    DBG_RHT_RANGE)) {
      const long long tk = a.n_old + tok0 + t32;
      u32x2* dst = reinterpret_cast<u32x2*>(a.packed + s * a.packed_stride + tk * 48 + 24 * h);
      dst[0] = (u32x2){w[0], w[1]};
      dst[1] = (u32x2){w[2], w[3]};
      dst[2] = (u32x2){w[4], w[5]};
      if (h == 0) a.norms[s * a.norms_stride + tk] = nu;
    }
  }
}

// 128 tokens per workgroup; the reconstructed rows go through LDS so that the
// HBM stores are whole consecutive rows (per-lane row stores leave cache
// lines partly written and multiply the write traffic).
constexpr int RHTD_T = 128;
__global__ void __launch_bounds__(RHTD_T) k_rht_decode(RhtK a) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ float scb[8];
  const long long s = blockIdx.y;
  const int t = threadIdx.x;
  const long long si = state_index(a.map, s, a.n_states);
  if (si < 0) {  // no state: NaN rows
    const long long tok = (long long)blockIdx.x * RHTD_T + t;
    if (tok < a.n_tokens)
      for (int i = 0; i < 128; ++i) {
        if (a.f32out) static_cast<float*>(a.xo)[s * a.x_stride + tok * a.ld + i] = __builtin_nanf("");
        else static_cast<unsigned short*>(a.xo)[s * a.x_stride + tok * a.ld + i] = 0x7FC0u;
      }
    return;
  }
  const DevHdr* hdr = reinterpret_cast<const DevHdr*>(a.states + (size_t)si * STATE_BYTES);
  if (t < 8) scb[t] = hdr->cb[t];
  __syncthreads();
  const long long tok0 = (long long)blockIdx.x * RHTD_T;
  const long long tok = tok0 + t;
  const int rowb = a.f32out ? 512 + 16 : 256 + 16;  // LDS row bytes
  if (tok < a.n_tokens) {
    const u32x4* src = reinterpret_cast<const u32x4*>(a.packed_in + s * a.packed_stride + tok * 48);
    unsigned w[12];
    {
      const u32x4 w0 = src[0], w1 = src[1], w2 = src[2];
#pragma unroll
      for (int e = 0; e < 4; ++e) { w[e] = w0[e]; w[4 + e] = w1[e]; w[8 + e] = w2[e]; }
    }
    float v[128];
#pragma unroll
    for (int i = 0; i < 128; ++i) {
      const int bp = 3 * i;
      unsigned q = w[bp >> 5] >> (bp & 31);
      if ((bp & 31) > 29) q |= w[(bp >> 5) + 1] << (32 - (bp & 31));
      v[i] = scb[q & 7u];
    }
    fwht128(v);
    const float m = a.norms_in[s * a.n_tokens + tok] * 0.08838834764831845f;  // |x| / sqrt(128)
    unsigned char* row = smem + t * rowb;
    if (a.f32out) {
#pragma unroll
      for (int c = 0; c < 32; ++c)
        *reinterpret_cast<f32x4*>(row + 16 * c) =
            (f32x4){v[4 * c] * m * hdr->sign[4 * c], v[4 * c + 1] * m * hdr->sign[4 * c + 1],
                    v[4 * c + 2] * m * hdr->sign[4 * c + 2], v[4 * c + 3] * m * hdr->sign[4 * c + 3]};
    } else {
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        u32x4 pk;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 8 * c + 2 * e;
          pk[e] = pack_bf16x2(v[i] * m * hdr->sign[i], v[i + 1] * m * hdr->sign[i + 1]);
        }
        *reinterpret_cast<u32x4*>(row + 16 * c) = pk;
      }
    }
  }
  __syncthreads();
  // whole rows out: consecutive threads take consecutive 16-byte chunks of a row
  const int cpr = a.f32out ? 32 : 16;
  const long long ntok = (a.n_tokens - tok0) < RHTD_T ? (a.n_tokens - tok0) : RHTD_T;
  const int esz = a.f32out ? 4 : 2;
  unsigned char* obase = static_cast<unsigned char*>(a.xo) + (s * a.x_stride + tok0 * a.ld) * esz;
  for (int i = t; i < ntok * cpr; i += RHTD_T) {
    const int r = i / cpr, c = i - r * cpr;
    __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(smem + r * rowb + 16 * c),
                                reinterpret_cast<u32x4*>(obase + ((long long)r * a.ld) * esz + 16 * c));
  }
}

int launch_encode_rht(const EncodeLaunch& L, void* stream) {
  RhtK a{};
  a.states = L.states;
  a.map = L.map;
  a.n_states = L.n_states;
  a.n_tokens = L.n_tokens;
  a.ld = L.ld;
  a.x_stride = L.x_stride;
  a.packed_stride = L.packed_stride;
  a.x = L.x;
  a.packed = L.packed;
  a.norms = L.norms;
  a.n_old = L.n_old;
  a.norms_stride = L.norms_stride;
  a.sketch = L.sketch;
  a.rnorm = L.rnorm;
  a.sketch_stride = L.sketch_stride;
  a.rnorm_stride = L.rnorm_stride;
  const long long nblk = (L.n_tokens + ENC_BT - 1) / ENC_BT;
  if (L.sketch) {
    static bool attr = false;
    if (!attr) {
      if (hipFuncSetAttribute((const void*)k_rht_encode<true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)RHTS_LDS) != hipSuccess)
        return 1;
      attr = true;
    }
    dim3 grid((unsigned)((nblk + RHTS_WAVES * RHT_BPW - 1) / (RHTS_WAVES * RHT_BPW)), (unsigned)L.n_streams);
    hipLaunchKernelGGL(k_rht_encode<true>, grid, dim3(64 * RHTS_WAVES), RHTS_LDS, (hipStream_t)stream, a);
  } else if (rht_encode_kernel() == 1) {
    dim3 grid((unsigned)((nblk + RHTB_WAVES * RHT_BPW - 1) / (RHTB_WAVES * RHT_BPW)), (unsigned)L.n_streams);
    hipLaunchKernelGGL(k_rht_encode_bfly, grid, dim3(64 * RHTB_WAVES), 0, (hipStream_t)stream, a);
  } else {
    dim3 grid((unsigned)((nblk + RHT_WAVES * RHT_BPW - 1) / (RHT_WAVES * RHT_BPW)), (unsigned)L.n_streams);
    hipLaunchKernelGGL(k_rht_encode<false>, grid, dim3(64 * RHT_WAVES), RHT_LDS, (hipStream_t)stream, a);
  }
  return hipGetLastError() != hipSuccess;
}

int launch_decode_rht(const DecodeLaunch& L, void* stream) {
  RhtK a{};
  a.states = L.states;
  a.map = L.map;
  a.n_states = L.n_states;
  a.n_tokens = L.n_tokens;
  a.ld = L.ld;
  a.x_stride = L.x_stride;
  a.packed_stride = L.packed_stride;
  a.packed_in = L.packed;
  a.norms_in = L.norms;
  a.xo = L.x;
  a.f32out = L.f32out;
  dim3 grid((unsigned)((L.n_tokens + RHTD_T - 1) / RHTD_T), (unsigned)L.n_streams);
  const size_t lds = (size_t)RHTD_T * (L.f32out ? 512 + 16 : 256 + 16);
  static bool attr = false;
  if (!attr) {
    if (hipFuncSetAttribute((const void*)k_rht_decode, hipFuncAttributeMaxDynamicSharedMemorySize,
                              RHTD_T * (512 + 16)) != hipSuccess) return 1;
    attr = true;
  }
  hipLaunchKernelGGL(k_rht_decode, grid, dim3(RHTD_T), lds, (hipStream_t)stream, a);
  return hipGetLastError() != hipSuccess;
}

// ======================================================================
// Decode-step attention over the packed cache.
// Scores in the latent basis: s_t = sum_j a_j q_tj with a_j = (U_K^T q)_j
// step_j scale log2(e) and q_tj the raw codes; the dropped offset
// -sum_j a_j (L_j - 1)/2 is the same for every token and cancels in the
// softmax. Values: the softmax-weighted average of the raw V codes is
// accumulated per split, merged across splits with log-sum-exp, then
// dequantized and rotated back once: o = U_V (step * (avg code - halfspan)).
//  k_att_main: one workgroup per (split, pair). It builds the a table (bf16
//   hi/lo) in LDS; then each wave takes 32-token blocks of the split on its
//   own: K and V records to LDS, K half records extracted per lane, scores
//   by one MFMA chain (hi rows 0..15 and lo rows 16..31 of the table
//   against the K codes), online softmax, P (fp16) x V codes (fp16) on MFMA
//   with the V codes byte-transposed into a [channel][token] buffer. At the
//   end the waves' (acc, m, l) are merged into the split's partial.
//  k_att_combine (the next launch on the stream, so every split's partial
//   is in memory): one workgroup per (pair, query head): merge the splits,
//   dequantize, rotate back.
// ======================================================================
struct AttK {
  const unsigned char* k_states;
  const int32_t* k_map;
  const unsigned char* v_states;
  const int32_t* v_map;
  long long n_states, n_pairs, n_tokens, packed_stride;
  const unsigned char* k_packed;
  const unsigned char* v_packed;
  int group;
  const float* q;
  float* out;
  float scale;
  unsigned char* ws;
  long long split_tokens, n_splits;
  int stream_words, region_words;
  long long pair_base;  // first pair of this launch (maps, caches, q, out); ws is per launch
  const float* k_norms;  // Walsh-Hadamard caches: per-token norms, pair stride norms_stride
  const float* v_norms;
  long long norms_stride;
  const unsigned char* k_sketch;  // key residual sketch (16 bytes per token) and |r|, or null
  const float* k_rnorm;
  long long sketch_stride, rnorm_stride;
  float* prep;  // per pair of the launch: score weights and head scales (k_att2_prep), ATT_PREP_FLOATS each
  // generation step: pair p's new K and V token rows (128 elements, bf16 or
  // fp32) appended as token n_tokens - 1 before the scores are formed; null
  // for a plain attention call
  const void* k_new;
  const void* v_new;
  int new_f32;
  // packed-bit kernel with one split per pair: each workgroup forms its
  // pair's output itself (the merge kernel is not launched)
  int direct;
};

constexpr int ATT_WAVES_MAX = 16;
constexpr int ATT_THREADS = 64 * ATT_WAVES_MAX;
constexpr int ATT_BT = 32;                       // tokens per wave block
constexpr int AROW = 272;                        // bytes per a-table row (rows 0..15 hi, 16..31 lo)
// [channel][token] V bytes: 8 dwords a channel (4 tokens a dword), channels
// 64..127 32 dwords further on and the dword index XOR 4 on channels with
// bit 3 set, so that the quad-transposed writes (64 lanes: 2 halves x 4
// channels x 8 token quads) and the P.V reads (16 channels x 4 token quads)
// each touch 64 distinct banks
constexpr int VT_ROW = 8;
constexpr int VT_WORDS = 128 * VT_ROW + 32;
__device__ __forceinline__ int vt_index(int c, int j) { return c * VT_ROW + ((c >> 6) << 5) + (j ^ (((c >> 3) & 1) << 2)); }
constexpr int P_ROWH = 36;                       // fp16 per row of P [head][token]
constexpr int P_WORDS = 16 * P_ROWH / 2;
constexpr int ATT_FIXED_BYTES = 32 * AROW + 6 * 128 * 4 + 64;  // a table, unpack tables, codebook planes
// Words of one wave's region: the K and V record streams (reused for the
// transposed V codes once both are extracted), P, and per-head alpha.
// (a block's 32 records with one pad word per 32-word run, or, in the REC
// layout, one pad word per record)
__host__ __device__ constexpr int att_stream_words(int max_bits) {
  return max_bits + ((max_bits >> 5) > 32 ? (max_bits >> 5) : 32) + 8;
}
__host__ __device__ constexpr int att_region_words(int max_bits) {
  return (2 * att_stream_words(max_bits) > VT_WORDS ? 2 * att_stream_words(max_bits) : VT_WORDS) + P_WORDS + 32;
}

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

// 4 unsigned byte codes c -> 4 fp16 c: two byte permutes give 1024 + c
// (0x64xx in fp16, exact), two packed fp16 subtractions remove the 1024
// (exact: the results are integers below 2^8). P.V then accumulates p c, whose
// fp32 rounding scales with the codes, not with an offset (a near-uniform
// softmax over many tokens averages the codes to within a small fraction of
// one level, which an offset of 1024 in the sums would swamp).
__device__ __forceinline__ f16x4 bytes_to_f16x4(unsigned v) {
  const unsigned lo = __builtin_amdgcn_perm(v, 0x64646464u, 0x00050004u);
  const unsigned hi = __builtin_amdgcn_perm(v, 0x64646464u, 0x00070006u);
  const f16x2 off = {(_Float16)1024.0f, (_Float16)1024.0f};
  const f16x2 a = __builtin_bit_cast(f16x2, lo) - off, b = __builtin_bit_cast(f16x2, hi) - off;
  return __builtin_bit_cast(f16x4, (u32x2){__builtin_bit_cast(unsigned, a), __builtin_bit_cast(unsigned, b)});
}

// Four codes (bytes of c, each 0..7) -> four 16-bit table entries, from the
// low-byte plane (l0: entries 0..3, l1: 4..7) and the high-byte plane
// (h0, h1): entries of codes 0, 1 in the first word, 2, 3 in the second.
__device__ __forceinline__ u32x2 lut16x4(unsigned c, unsigned l0, unsigned l1, unsigned h0, unsigned h1) {
  const unsigned lo = __builtin_amdgcn_perm(l1, l0, c);
  const unsigned hi = __builtin_amdgcn_perm(h1, h0, c);
  return (u32x2){__builtin_amdgcn_perm(hi, lo, 0x05010400u), __builtin_amdgcn_perm(hi, lo, 0x07030602u)};
}

// 4x4 byte transpose across the 4 lanes of a quad: lane e holds byte c of
// token e in byte c; afterwards lane e holds byte e of tokens 0..3.
__device__ __forceinline__ unsigned quad_transpose_bytes(unsigned x, int e) {
  const unsigned p1 = (unsigned)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false);  // lane e^1
  const unsigned y = __builtin_amdgcn_perm(p1, x, (e & 1) ? 0x03070105u : 0x06020400u);
  const unsigned p2 = (unsigned)__builtin_amdgcn_mov_dpp((int)y, 0x4E, 0xF, 0xF, false);  // lane e^2
  return __builtin_amdgcn_perm(p2, y, (e & 2) ? 0x03020706u : 0x05040100u);
}

// Max / sum over the 32 lanes of each half wave (DPP within 16-lane rows,
// then a row swap).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
// Both 16-lane rows of each half wave side by side: element 0 holds the
// value of row 2k, element 1 that of row 2k + 1, in every lane of the half.
__device__ __forceinline__ auto row_swap(float x) {
  const unsigned a = __builtin_bit_cast(unsigned, x);
  return __builtin_amdgcn_permlane16_swap(a, a, false, false);
}
__device__ __forceinline__ float half_max(float x) {
  x = fmaxf(x, dpp_f<0xB1>(x));   // quad_perm [1,0,3,2]
  x = fmaxf(x, dpp_f<0x4E>(x));   // quad_perm [2,3,0,1]
  x = fmaxf(x, dpp_f<0x141>(x));  // row_half_mirror
  x = fmaxf(x, dpp_f<0x140>(x));  // row_mirror
  const auto r = row_swap(x);
  const unsigned r0 = r[0], r1 = r[1];  // (a bit cast of a vector element reads element 0)
  return fmaxf(__builtin_bit_cast(float, r0), __builtin_bit_cast(float, r1));
}
// Max over the 16 lanes of each row (DPP within the row).
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp_f<0xB1>(x));   // quad_perm [1,0,3,2]
  x = fmaxf(x, dpp_f<0x4E>(x));   // quad_perm [2,3,0,1]
  x = fmaxf(x, dpp_f<0x141>(x));  // row_half_mirror
  return fmaxf(x, dpp_f<0x140>(x));  // row_mirror
}
__device__ __forceinline__ float half_sum(float x) {
  x += dpp_f<0xB1>(x);
  x += dpp_f<0x4E>(x);
  x += dpp_f<0x141>(x);
  x += dpp_f<0x140>(x);
  const auto r = row_swap(x);
  const unsigned r0 = r[0], r1 = r[1];
  return __builtin_bit_cast(float, r0) + __builtin_bit_cast(float, r1);
}

// Per-lane unpack tables of a state: group record offset (entry 4g + 1:
// the byte offset of the word that holds it), offset inside the group,
// width (128 each).
__device__ __forceinline__ void att_tables(const DevHdr* hd, unsigned* tab, int c) {
  const unsigned go = (unsigned)hd->off[c & ~3];
  tab[c] = (c & 3) == 1 ? (go >> 5) << 2 : go;
  tab[128 + c] = (unsigned)hd->off[c] - (unsigned)hd->off[c & ~3];
  tab[256 + c] = (unsigned)hd->bits[c];
}

// The four codes of group g (channels 64h + 4g .. +3) of the record at bit
// tB of an LDS stream, as bytes of one word.
// 32-bit window of the lane's record at stream bit P; sb = the stream's LDS
// base as one register, so that the address is one shift-add
__device__ __forceinline__ unsigned att_window(const lds_u8* sb, unsigned P) {
  const lds_u8* p = sb + (est_idx_bit(P) << 2);
  return __builtin_amdgcn_alignbit(LDS_AT(unsigned, p + 4), LDS_AT(unsigned, p), P & 31u);
}
// REC layout (records of 32 * 2^s bits, each on its own word-aligned slot
// of the wave's stream): str is the lane's record, and the group's word and
// bit offsets are uniform, so the window is one add and one funnel shift.
// Otherwise str is the stream and tB the bit where the lane's record starts.
template <bool REC>
__device__ __forceinline__ unsigned att_group_window(const lds_u8* str, const lds_u8* tL, unsigned tB, int g) {
  if (REC) {
    const u32x2 t = LDS_AT(u32x2, tL + 16 * g);
    const lds_u8* p = str + t[1];
    return __builtin_amdgcn_alignbit(LDS_AT(unsigned, p + 4), LDS_AT(unsigned, p), t[0] & 31u);
  }
  return att_window(str, tB + LDS_AT(unsigned, tL + 16 * g));
}
// the four codes of group g as floats (exact)
template <bool REC>
__device__ __forceinline__ void att_group_codes(const lds_u8* str, const lds_u8* tL, unsigned tB, int g,
                                                float c[4]) {
  const unsigned w = att_group_window<REC>(str, tL, tB, g);
  const u32x4 pos = LDS_AT(u32x4, tL + 512 + 16 * g);
  const u32x4 wid = LDS_AT(u32x4, tL + 1024 + 16 * g);
#pragma unroll
  for (int j = 0; j < 4; ++j) c[j] = (float)__builtin_amdgcn_ubfe(w, pos[j], wid[j]);
}
template <bool REC>
__device__ __forceinline__ unsigned att_group_bytes(const lds_u8* str, const lds_u8* tL, unsigned tB, int g) {
  const unsigned w = att_group_window<REC>(str, tL, tB, g);
  const u32x4 pos = LDS_AT(u32x4, tL + 512 + 16 * g);
  const u32x4 wid = LDS_AT(u32x4, tL + 1024 + 16 * g);
  const unsigned c0 = __builtin_amdgcn_ubfe(w, pos[0], wid[0]), c1 = __builtin_amdgcn_ubfe(w, pos[1], wid[1]);
  const unsigned c2 = __builtin_amdgcn_ubfe(w, pos[2], wid[2]), c3 = __builtin_amdgcn_ubfe(w, pos[3], wid[3]);
  // bytes (c0, c1, 0, 0) and (c2, c3, 0, 0), then (c0, c1, c2, c3)
  return __builtin_amdgcn_perm(__builtin_amdgcn_perm(c3, c2, 0x0C0C0400u), __builtin_amdgcn_perm(c1, c0, 0x0C0C0400u),
                               0x05040100u);
}


// RHT: a Walsh-Hadamard cache. Its state stores U = D H / sqrt(d) with unit
// steps, so the score table and the split merge are the eigen ones; the
// codes are looked up in the codebook (bf16 high and low parts for the
// scores, fp16 for P.V), scores are scaled by the key's norm and P by the
// value's norm over the largest value norm of the wave's block (the scale
// is carried in the accumulators and restored at the merge).
// SKETCH (RHT only): keys carry the 1-bit residual sketch; a second table
// holds S q scale log2(e) sqrt(pi/2)/m (hi / lo) and each score gains
// |r_t| times its product with the token's signs, one more MFMA chain.
// Split merge, after the main kernel has written every split's partial:
// per (query head, V channel j) the splits' (acc_j, m, l) merge with
// log-sum-exp weights (fp32 weights, fp64 sums, batches of 8 splits with all
// loads in flight), the mean code is dequantized, and o = U_V chat is formed
// for every head.
//  k_att_combine: one 256-thread workgroup per pair (many pairs): each
//   thread merges whole elements, then thread (half, i) sums its half of row
//   i of U_V (read once per pair, 16 floats at a time) against every head's
//   codes and the two halves are added through LDS.
//  k_att_combine_head: one 1024-thread workgroup per (pair, query head) (few
//   pairs with many splits): eight threads per channel merge interleaved
//   eighths of the splits, the eighths are merged in a fixed order, and eight
//   threads per output dim sum sixteen inputs each.
constexpr int CMB_THREADS = 256;
constexpr int CMB_BATCH = 8;
constexpr int CMBH_THREADS = 1024;
// dynamic LDS of k_att_combine: mean codes [g][128], half sums [2][g][128]
__host__ __device__ constexpr size_t cmb_lds_bytes(int g) { return (size_t)3 * g * 128 * 4; }

// Merge splits s0, s0 + step, ... (< S) of element j of a head's partials ph:
// running maximum M and the sums A (weighted codes) and L (weights).
__device__ __forceinline__ void cmb_merge(const float* ph, int S, int s0, int step, long long PS, int j, float& M,
                                          double& A, double& L) {
  M = -INFINITY;
  A = 0.0;
  L = 0.0;
  for (int sb = s0; sb < S; sb += CMB_BATCH * step) {
    float mv[CMB_BATCH], lv[CMB_BATCH], av[CMB_BATCH];
#pragma unroll
    for (int r = 0; r < CMB_BATCH; ++r) {
      const int s2 = sb + r * step;
      const long long sc = s2 < S ? s2 : s0;  // (past the end: a repeat that gets weight 0)
      mv[r] = ph[sc * PS + 128];
      lv[r] = ph[sc * PS + 129];
      av[r] = ph[sc * PS + j];
    }
    float Mc = M;
#pragma unroll
    for (int r = 0; r < CMB_BATCH; ++r) Mc = fmaxf(Mc, mv[r]);  // repeats change no maximum
    if (Mc != -INFINITY) {
      if (M != -INFINITY && M != Mc) {
        const double sc = (double)exp2f(M - Mc);
        A *= sc;
        L *= sc;
      }
#pragma unroll
      for (int r = 0; r < CMB_BATCH; ++r) {
        const float f = (sb + r * step < S && mv[r] != -INFINITY) ? exp2f(mv[r] - Mc) : 0.0f;
        A += (double)(f * av[r]);
        L += (double)(f * lv[r]);
      }
      M = Mc;
    }
  }
}

// Mean code of V channel j from the merged sums: step_j (A / L - (L_j - 1)/2),
// 0 for a dropped channel.
__device__ __forceinline__ float cmb_code(const DevHdr* hv, int j, double A, double L) {
  return hv->bits[j] ? (float)((double)hv->step32[j] * (A / L - (double)hv->halfspan[j])) : 0.0f;
}

// o = U_V chat for every head of a pair, from the mean codes sC [g][128]:
// thread (half, i) of the first CMB_THREADS sums its half of row i of U_V
// (16 floats at a time) against every head's codes; the halves are added
// through sQ [2][g][128] and written to out [g][128]. Every thread of the
// workgroup calls it (it holds a barrier).
__device__ __forceinline__ void cmb_rotate(const float* sC, float* sQ, const unsigned char* vst, int g, float* out,
                                           int t) {
  if (t < CMB_THREADS) {
    const int i = t & 127, half = t >> 7;
    const f32x4* urow = reinterpret_cast<const f32x4*>(vst + OFF_U32) + i * 32 + half * 16;  // U[i][64 half ..]
    float o[16];
#pragma unroll
    for (int hh = 0; hh < 16; ++hh) o[hh] = 0.0f;
#pragma unroll
    for (int jc = 0; jc < 4; ++jc) {
      f32x4 u[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) u[r] = urow[4 * jc + r];
#pragma unroll
      for (int hh = 0; hh < 16; ++hh) {
        if (hh < g) {
          const f32x4* c4 = reinterpret_cast<const f32x4*>(sC + hh * 128 + 64 * half + 16 * jc);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const f32x4 c = c4[r];
#pragma unroll
            for (int e = 0; e < 4; ++e) o[hh] = __builtin_fmaf(u[r][e], c[e], o[hh]);
          }
        }
      }
    }
#pragma unroll
    for (int hh = 0; hh < 16; ++hh)
      if (hh < g) sQ[(half * g + hh) * 128 + i] = o[hh];
  }
  __syncthreads();
  if (t < CMB_THREADS) {
    for (int e = t; e < g * 128; e += CMB_THREADS) {
      const int hh = e >> 7, ii = e & 127;
      out[hh * 128 + ii] = sQ[hh * 128 + ii] + sQ[(g + hh) * 128 + ii];
    }
  }
}

__global__ void __launch_bounds__(CMB_THREADS) k_att_combine(AttK a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int g = a.group;
  float* sC = reinterpret_cast<float*>(smem);  // dequantized mean codes [head][128]
  float* sQ = sC + g * 128;                    // half sums [2][head][128]
  const long long p = blockIdx.x;
  const long long pg = a.pair_base + p;
  const int t = threadIdx.x;
  const int S = (int)a.n_splits;
  const long long PS = att_part_stride(g);
  const long long ksi = state_index(a.k_map, pg, a.n_states), vsi = state_index(a.v_map, pg, a.n_states);
  if (ksi < 0 || vsi < 0) {  // no state for the pair (the main kernel wrote no partial): NaN
    for (int e = t; e < g * 128; e += CMB_THREADS) a.out[pg * g * 128 + e] = __builtin_nanf("");
    return;
  }
  const unsigned char* vst = a.v_states + (size_t)vsi * STATE_BYTES;
  const DevHdr* hv = reinterpret_cast<const DevHdr*>(vst);
  for (int e = t; e < g * 128; e += CMB_THREADS) {
    const int hh = e >> 7, j = e & 127;
    const float* ph = reinterpret_cast<const float*>(a.ws) + p * (long long)S * PS + hh * ATT_PART_FLOATS;
    float M;
    double A, L;
    cmb_merge(ph, S, 0, 1, PS, j, M, A, L);
    sC[hh * 128 + j] = cmb_code(hv, j, A, L);
  }
  __syncthreads();
  cmb_rotate(sC, sQ, vst, g, a.out + pg * g * 128, t);
}

__global__ void __launch_bounds__(CMBH_THREADS) k_att_combine_head(AttK a) {
  __shared__ float sM[8][128];
  __shared__ double sA[8][128], sL[8][128];
  __shared__ __align__(16) float sC[128];
  __shared__ float sR[8][128];
  const int g = a.group;
  const long long p = blockIdx.x;
  const int hh = blockIdx.y;
  const long long pg = a.pair_base + p;
  const int t = threadIdx.x;
  const int S = (int)a.n_splits;
  const long long PS = att_part_stride(g);
  const long long ksi = state_index(a.k_map, pg, a.n_states), vsi = state_index(a.v_map, pg, a.n_states);
  if (ksi < 0 || vsi < 0) {  // no state for the pair: NaN
    if (t < 128) a.out[(pg * g + hh) * 128 + t] = __builtin_nanf("");
    return;
  }
  const unsigned char* vst = a.v_states + (size_t)vsi * STATE_BYTES;
  const DevHdr* hv = reinterpret_cast<const DevHdr*>(vst);
  const int j = t & 127, eighth = t >> 7;
  // row i = j of U_V, inputs 16 eighth .. + 15, requested before the merge
  const f32x4* urow = reinterpret_cast<const f32x4*>(vst + OFF_U32) + j * 32 + eighth * 4;
  f32x4 u[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) u[r] = urow[r];
  {
    const float* ph = reinterpret_cast<const float*>(a.ws) + p * (long long)S * PS + hh * ATT_PART_FLOATS;
    float M;
    double A, L;
    cmb_merge(ph, S, eighth, 8, PS, j, M, A, L);
    sM[eighth][j] = M;
    sA[eighth][j] = A;
    sL[eighth][j] = L;
  }
  __syncthreads();
  if (t < 128) {
    float M = -INFINITY;
#pragma unroll
    for (int e = 0; e < 8; ++e) M = fmaxf(M, sM[e][t]);
    double A = 0.0, L = 0.0;
    if (M != -INFINITY) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float me = sM[e][t];
        if (me != -INFINITY) {
          const double f = (double)exp2f(me - M);
          A += f * sA[e][t];
          L += f * sL[e][t];
        }
      }
    }
    sC[t] = cmb_code(hv, t, A, L);
  }
  __syncthreads();
  float o = 0.0f;
  const f32x4* c4 = reinterpret_cast<const f32x4*>(sC + 16 * eighth);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const f32x4 c = c4[r];
#pragma unroll
    for (int e = 0; e < 4; ++e) o = __builtin_fmaf(u[r][e], c[e], o);
  }
  sR[eighth][j] = o;
  __syncthreads();
  if (t < 128) {
    float r = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) r += sR[e][t];
    a.out[(pg * g + hh) * 128 + t] = r;
  }
}

template <int NW, bool RHT, bool SKETCH, bool REC>
__global__ void __launch_bounds__(ATT_THREADS, 1) k_att_main(AttK a) {
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* sA = smem;                                        // a table [32][AROW]
  unsigned* sTab = reinterpret_cast<unsigned*>(smem + 32 * AROW);  // K tables, V tables, codebook planes
  unsigned char* sA2 = reinterpret_cast<unsigned char*>(sTab + 6 * 128 + 16);  // SKETCH: sign table [32][AROW]
  unsigned* sReg0 = sTab + 6 * 128 + 16 + (SKETCH ? 32 * AROW / 4 : 0);       // wave regions
  const int nwav = (int)(blockDim.x >> 6);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t32 = lane & 31, h = lane >> 5;
  const int c16 = lane & 15, g4 = lane >> 4;
  const long long sp = blockIdx.x, p = blockIdx.y;  // split, pair within this launch
  const long long pg = a.pair_base + p;
  const long long n = a.n_tokens;
  const int g = a.group;
  const bool two_rows = g > 8;  // query heads 8..15 in use
  const long long ksi = state_index(a.k_map, pg, a.n_states), vsi = state_index(a.v_map, pg, a.n_states);
  if (ksi < 0 || vsi < 0) return;  // (the whole workgroup) the merge writes NaN for this pair
  const unsigned char* kst = a.k_states + (size_t)ksi * STATE_BYTES;
  const unsigned char* vst = a.v_states + (size_t)vsi * STATE_BYTES;
  const DevHdr* hk = reinterpret_cast<const DevHdr*>(kst);
  const DevHdr* hv = reinterpret_cast<const DevHdr*>(vst);
  const unsigned Bk = (unsigned)__builtin_amdgcn_readfirstlane(hk->total_bits);
  const unsigned Bv = (unsigned)__builtin_amdgcn_readfirstlane(hv->total_bits);
  const int SW = a.stream_words;
  unsigned* sKs = sReg0 + wave * a.region_words;  // K stream
  unsigned* sVs = sKs + SW;                        // V stream
  unsigned* sVT = sKs;                             // [channel][token] V bytes, after extraction
  _Float16* sP = reinterpret_cast<_Float16*>(sKs + (2 * SW > VT_WORDS ? 2 * SW : VT_WORDS));
  float* sAl = reinterpret_cast<float*>(sP + 16 * P_ROWH);  // alpha per head
  float* sM = sAl + 16;                                     // running max per head
  const long long t_begin = sp * a.split_tokens;
  long long t_end = t_begin + a.split_tokens;
  if (t_end > n) t_end = n;

  // the records of a wave block go HBM -> registers (wk, wv) -> the wave's
  // streams; the wave's first block is requested before the a table is built
  const long long PkL = packed_len((long long)Bk, n), PvL = packed_len((long long)Bv, n);
  const unsigned char* gk = a.k_packed + pg * a.packed_stride;
  const unsigned char* gv = a.v_packed + pg * a.packed_stride;
  unsigned wk[NW], wv[NW];
  long long nbk = 0, nbv = 0;
  auto load_records = [&](long long tok0) {
    const long long blk = tok0 / ATT_BT;
    const long long stk = blk * 4LL * (long long)Bk, stv = blk * 4LL * (long long)Bv;
    nbk = 4LL * (long long)Bk;
    nbv = 4LL * (long long)Bv;
    if (nbk > PkL - stk) nbk = PkL - stk;
    if (nbv > PvL - stv) nbv = PvL - stv;
    est_load<NW>(wk, gk + stk, Bk ? nbk : 0, lane);  // K and V loads in flight together
    est_load<NW>(wv, gv + stv, Bv ? nbv : 0, lane);
  };
  const long long t_first = t_begin + (long long)wave * ATT_BT;
  if (t_first < t_end) load_records(t_first);

  if (tid < 128) {
    att_tables(hk, sTab, tid);
    att_tables(hv, sTab + 384, tid);
    if (RHT && tid < 12) sTab[768 + tid] = tid < 8 ? hk->cbt[tid] : hv->cbt[tid];  // K: bf16 hi/lo, V: fp16
  }
  // Score A operand: a_hj = (U_K^T q_h)_j step_j scale log2(e) as bf16 high
  // (rows 0..15) and low (rows 16..31) parts. Thread (part, j) sums rows
  // part, part + 8, .. of column j of U_K; the parts are added through LDS
  // scratch in the wave regions, which the blocks reuse afterwards.
  {
    float* sqT = reinterpret_cast<float*>(sReg0);  // q transposed [128][16], zero for heads >= g
    float* red = sqT + 128 * 16;                    // [nparts][16][128]
    const int j = tid & 127, part = tid >> 7;
    const int nparts = (int)(blockDim.x >> 7);
    const float* qp = a.q + pg * g * 128;
    const int rows = (128 + nparts - 1) / nparts;  // rows per part: 16 or 22 (1024 or 768 threads)
    for (int e = tid; e < 128 * 16; e += blockDim.x) {
      const int r = e >> 4, hh = e & 15;
      sqT[e] = hh < g ? qp[hh * 128 + r] : 0.0f;
    }
    for (int tab = 0; tab < (SKETCH ? 2 : 1); ++tab) {
    // tab 0: U_K (scores), tab 1: S^T (sketch products)
    const float* u = reinterpret_cast<const float*>(kst + (tab == 0 ? OFF_U32 : OFF_SKT32));
    float ur[22];
#pragma unroll
    for (int k = 0; k < 22; ++k) {
      // issued together: rows past the part's share load row 127 and count 0
      const int row = part + k * nparts;
      const float v = u[(row < 127 ? row : 127) * 128 + j];
      ur[k] = (k < rows && row < 128) ? v : 0.0f;
    }
    __syncthreads();
    float acc[16];
#pragma unroll
    for (int hh = 0; hh < 16; ++hh) acc[hh] = 0.0f;
#pragma unroll
    for (int k = 0; k < 22; ++k) {
      if (k < rows) {
        const int row = part + k * nparts;
        const f32x4* q4 = reinterpret_cast<const f32x4*>(sqT + (row < 127 ? row : 127) * 16);
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
          const f32x4 qv = q4[c4];
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[4 * c4 + e] = __builtin_fmaf(ur[k], qv[e], acc[4 * c4 + e]);
        }
      }
    }
#pragma unroll
    for (int hh = 0; hh < 16; ++hh) red[(part * 16 + hh) * 128 + j] = acc[hh];
    __syncthreads();
    unsigned char* dstA = tab == 0 ? sA : sA2;
    for (int e = tid; e < 16 * 128; e += blockDim.x) {
      const int hh = e >> 7, c = e & 127;
      float val = 0.0f;
      if (hh < g && (tab == 1 || hk->bits[c] > 0)) {
        float sum = 0.0f;
        for (int pt = 0; pt < nparts; ++pt) sum += red[(pt * 16 + hh) * 128 + c];
        val = tab == 0 ? sum * hk->step32[c] * a.scale * LOG2E
                       : sum * (a.scale * LOG2E * 1.2533141373155003f / (float)STC_SKETCH_BITS);  // sqrt(pi/2)/m
      }
      const __bf16 hi = (__bf16)val;
      const __bf16 lo = (__bf16)(val - (float)hi);
      *reinterpret_cast<__bf16*>(dstA + hh * AROW + 2 * c) = hi;
      *reinterpret_cast<__bf16*>(dstA + (16 + hh) * AROW + 2 * c) = lo;
    }
    __syncthreads();
    }
  }

  // per-wave online softmax state: heads H = 8i + 4h + j in the score
  // layout (m replicated over the half, l partial per lane); the value
  // accumulators in the P.V layout (heads 4*g4 + r, channel 16nb + c16)
  float l_run[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) l_run[i][j] = 0.0f;
  if (lane < 16) sM[lane] = -INFINITY;
  if (!two_rows) {
    // heads 8..15 unused: their P rows stay 0 and their alpha 1 (the
    // blocks only write rows 0..7 then)
#pragma unroll
    for (int j = 0; j < 4; ++j) sP[(8 + 4 * h + j) * P_ROWH + t32] = (_Float16)0.0f;
    if (lane < 8) sAl[8 + lane] = 1.0f;
  }
  f32x4 acc_o[8];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) acc_o[nb] = (f32x4){0.f, 0.f, 0.f, 0.f};
  float vscale = 1.0f;  // RHT: acc_o is in units of the current block's largest value norm

  // REC: records of 32 * 2^s bits (or none), each on its own slot
  const unsigned shk = Bk ? (unsigned)__builtin_ctz(Bk >> 5) : 0u, shv = Bv ? (unsigned)__builtin_ctz(Bv >> 5) : 0u;
  const unsigned rk4 = Bk ? ((Bk >> 5) + 1u) * 4u : 0u, rv4 = Bv ? ((Bv >> 5) + 1u) * 4u : 0u;
  auto store_records = [&]() {
    if (REC) {
      rec_store<NW>(sKs, wk, Bk ? nbk : 0, lane, shk);
      rec_store<NW>(sVs, wv, Bv ? nbv : 0, lane, shv);
    } else {
      est_store<NW>(sKs, wk, Bk ? nbk : 0, lane);
      est_store<NW>(sVs, wv, Bv ? nbv : 0, lane);
    }
  };
  if (t_first < t_end) store_records();  // (the a-table build is done with the wave regions)
  for (long long tok0 = t_first; tok0 < t_end; tok0 += (long long)nwav * ATT_BT) {
    // ---- records -> the wave's streams
    if (tok0 != t_first) {
      load_records(tok0);
      store_records();
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
    unsigned kb = lds_offset(reinterpret_cast<unsigned char*>(sTab + 64 * h));
    unsigned ab = lds_offset(sA + t32 * AROW + 128 * h);
    unsigned ksb = lds_offset(reinterpret_cast<unsigned char*>(sKs)) + (REC ? (unsigned)t32 * rk4 : 0u);
    unsigned vsb = lds_offset(reinterpret_cast<unsigned char*>(sVs)) + (REC ? (unsigned)t32 * rv4 : 0u);
    asm volatile("" : "+v"(kb), "+v"(ab), "+v"(ksb), "+v"(vsb));
    const lds_u8* kSL = lds_ptr(ksb);
    const lds_u8* vSL = lds_ptr(vsb);
    const lds_u8* kL = lds_ptr(kb);
    const lds_u8* vL = kL + 1536;
    const lds_u8* aL = lds_ptr(ab);
    const bool tok_ok = tok0 + t32 < t_end;
    // RHT: the norms of the lane's token
    float nk = 1.0f, nv = 0.0f;
    if (RHT && tok_ok) {
      nk = a.k_norms[pg * a.norms_stride + tok0 + t32];
      nv = a.v_norms[pg * a.norms_stride + tok0 + t32];
    }
    // ---- scores: channels 64h + 8ks + i of token t as bf16 B fragments
    float sc[2][4];
    {
      f32x16 acc;
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[e] = 0.0f;
      const unsigned tB = (unsigned)t32 * Bk;
      u32x4 cbh, cbl;  // RHT: codebook planes (bf16 high parts, low parts)
      if (RHT) {
        cbh = LDS_AT(u32x4, kL - 64 * 4 * h + 768 * 4);
        cbl = LDS_AT(u32x4, kL - 64 * 4 * h + 772 * 4);
      }
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        if (RHT) {
          u32x4 fh, fl;
#pragma unroll
          for (int hg = 0; hg < 2; ++hg) {
            const unsigned v = att_group_bytes<false>(kSL, kL, tB, 2 * ks + hg);
            const u32x2 vh = lut16x4(v, cbh[0], cbh[1], cbh[2], cbh[3]);
            const u32x2 vl = lut16x4(v, cbl[0], cbl[1], cbl[2], cbl[3]);
            fh[2 * hg] = vh[0]; fh[2 * hg + 1] = vh[1];
            fl[2 * hg] = vl[0]; fl[2 * hg + 1] = vl[1];
          }
          const bf16x8 at = LDS_AT(bf16x8, aL + 16 * ks);
          acc = mfma32_bf16(at, __builtin_bit_cast(bf16x8, fh), acc);
          acc = mfma32_bf16(at, __builtin_bit_cast(bf16x8, fl), acc);
        } else {
          // codes straight to bf16 (exact); a stream without kept channels
          // (Bk = 0) reads its all-zero tables and gives code 0
          u32x4 bf;
#pragma unroll
          for (int hg = 0; hg < 2; ++hg) {
            float c[4];
            att_group_codes<REC>(kSL, kL, tB, 2 * ks + hg, c);
            bf[2 * hg] = bf16_pair_exact(c[0], c[1]);
            bf[2 * hg + 1] = bf16_pair_exact(c[2], c[3]);
          }
          acc = mfma32_bf16(LDS_AT(bf16x8, aL + 16 * ks), __builtin_bit_cast(bf16x8, bf), acc);
        }
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int H = 8 * i + 4 * h + j;
          sc[i][j] = (tok_ok && H < g) ? (acc[4 * i + j] + acc[4 * (i + 2) + j]) * nk : -INFINITY;
        }
      if (SKETCH) {
        // + |r_t| (S q) . z_t: the lane's 64 signs (rows 64h .. 64h + 63) as +-1 bf16
        u32x2 zb = (u32x2){0u, 0u};
        float rn = 0.0f;
        if (tok_ok) {
          zb = *reinterpret_cast<const u32x2*>(a.k_sketch + pg * a.sketch_stride + (tok0 + t32) * 16 + 8 * h);
          rn = a.k_rnorm[pg * a.rnorm_stride + tok0 + t32];
        }
        unsigned zab = lds_offset(sA2 + t32 * AROW + 128 * h);
        asm volatile("" : "+v"(zab));
        const lds_u8* zL = lds_ptr(zab);
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[e] = 0.0f;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          const unsigned byte = (zb[ks >> 2] >> (8 * (ks & 3))) & 0xffu;
          u32x4 zf;
#pragma unroll
          for (int k2 = 0; k2 < 4; ++k2) {
            const unsigned x2 = byte >> (2 * k2);
            zf[k2] = 0xBF80BF80u - ((x2 & 1u) << 15) - ((x2 & 2u) << 30);  // bit 1 -> +1, 0 -> -1
          }
          acc = mfma32_bf16(LDS_AT(bf16x8, zL + 16 * ks), __builtin_bit_cast(bf16x8, zf), acc);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) sc[i][j] += (acc[4 * i + j] + acc[4 * (i + 2) + j]) * rn;
      }
    }
    // RHT: P is stored as p * |v_t| / (largest |v| of the block), at most 1
    float pscale = 1.0f, vratio = 1.0f;
    if (RHT) {
      float vm = half_max(nv);
      vm = vm > 0.0f ? vm : 1.0f;
      pscale = nv / vm;
      vratio = vscale / vm;  // rescales acc_o from the previous block's units
      vscale = vm;
    }
    // ---- online softmax; P (fp16) -> sP[head][token], alpha -> sAl
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if (i == 1 && !two_rows) break;
      const f32x4 mold = *reinterpret_cast<const f32x4*>(sM + 8 * i + 4 * h);
      // When every score of the block is at most 2^8 above its head's running
      // maximum, that maximum stays the reference (weights <= 2^8, exact
      // enough in fp16; the merges use the same reference), so no block
      // maximum, no alpha and no rescale are needed.
      bool slow = false;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (8 * i + 4 * h + j < g) slow |= !(sc[i][j] <= mold[j] + 8.0f);
      if (!__any(slow)) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int H = 8 * i + 4 * h + j;
          const float pv = H < g ? __builtin_amdgcn_exp2f(sc[i][j] - mold[j]) : 0.0f;
          const _Float16 ph = (_Float16)(RHT ? pv * pscale : pv);
          l_run[i][j] += RHT ? pv : (float)ph;
          sP[H * P_ROWH + t32] = ph;
          if (t32 == 0) sAl[H] = 1.0f;
        }
        continue;
      }
      f32x4 mnw;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int H = 8 * i + 4 * h + j;
        const float mx = half_max(sc[i][j]);
        const float mnew = fmaxf(mold[j], mx);
        // arguments <= 0: the hardware exp2 (results below 2^-126 flush to 0)
        const float alpha = (mnew == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(mold[j] - mnew);
        const float pv = (mnew == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(sc[i][j] - mnew);
        const _Float16 ph = (_Float16)(RHT ? pv * pscale : pv);
        l_run[i][j] = l_run[i][j] * alpha + (RHT ? pv : (float)ph);
        mnw[j] = mnew;
        sP[H * P_ROWH + t32] = ph;
        if (t32 == 0) sAl[H] = alpha;
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // every lane has read the old maxima
      __builtin_amdgcn_wave_barrier();
      if (t32 == 0) *reinterpret_cast<f32x4*>(sM + 8 * i + 4 * h) = mnw;
    }
    // ---- V codes of the lane's 16 groups (bytes), then -> [channel][token]
    // (quads of lanes = 4 consecutive tokens)
    unsigned gvb[16];
    {
      const unsigned tB = (unsigned)t32 * Bv;
#pragma unroll
      for (int gg = 0; gg < 16; ++gg) gvb[gg] = att_group_bytes<REC>(vSL, vL, tB, gg);  // all 0 if Bv = 0 (zero widths)
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
    {
      const int e = t32 & 3;
#pragma unroll
      for (int gg = 0; gg < 16; ++gg) {
        const unsigned tq = quad_transpose_bytes(gvb[gg], e);
        sVT[vt_index(64 * h + 4 * gg + e, t32 >> 2)] = tq;
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
    // ---- rescale and accumulate P x V: heads 4*g4 + r, channels 16nb + c16
    {
      f32x4 al = *reinterpret_cast<const f32x4*>(sAl + 4 * g4);
      if (RHT) al *= vratio;
      // (once the running maxima settle, every alpha is 1: skip the rescale)
      if (!__all(al[0] == 1.0f && al[1] == 1.0f && al[2] == 1.0f && al[3] == 1.0f)) {
#pragma unroll
        for (int nb = 0; nb < 8; ++nb)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc_o[nb][r] *= al[r];
      }
      u32x4 cbv;  // RHT: fp16 codebook planes
      if (RHT) cbv = *reinterpret_cast<const u32x4*>(sTab + 776);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const f16x4 pa = *reinterpret_cast<const f16x4*>(sP + c16 * P_ROWH + 16 * kt + 4 * g4);
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) {
          const unsigned vb = sVT[vt_index(16 * nb + c16, 4 * kt + g4)];
          f16x4 vf;
          if (RHT) vf = __builtin_bit_cast(f16x4, lut16x4(vb, cbv[0], cbv[1], cbv[2], cbv[3]));
          else vf = bytes_to_f16x4(vb);
          acc_o[nb] = __builtin_amdgcn_mfma_f32_16x16x16f16(pa, vf, acc_o[nb], 0, 0, 0);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
  }
  // ---- l over the half's tokens; the maxima out of LDS before it is reused
  float mfin[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      l_run[i][j] = half_sum(l_run[i][j]);
      mfin[i][j] = sM[8 * i + 4 * h + j];
    }
  // ---- merge the waves, four heads at a time: scratch [wave][4][130]
  __syncthreads();
  float* red = reinterpret_cast<float*>(sReg0);
  float* part = reinterpret_cast<float*>(a.ws) + (p * a.n_splits + sp) * att_part_stride(g);
  for (int c4 = 0; c4 * 4 < g; ++c4) {
    float* mine = red + wave * 4 * ATT_PART_FLOATS;
    // m, l of heads 4*c4 .. +3: H = 8i + 4h + j
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int H = 8 * i + 4 * h + j;
        if (t32 == 0 && (H >> 2) == c4) {
          mine[(H & 3) * ATT_PART_FLOATS + 128] = mfin[i][j];
          mine[(H & 3) * ATT_PART_FLOATS + 129] = l_run[i][j];
        }
      }
    if (g4 == c4) {
#pragma unroll
      for (int nb = 0; nb < 8; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r) mine[r * ATT_PART_FLOATS + 16 * nb + c16] = RHT ? acc_o[nb][r] * vscale : acc_o[nb][r];
    }
    __syncthreads();
    const int nh = g - 4 * c4 < 4 ? g - 4 * c4 : 4;
    for (int e = tid; e < nh * 128; e += blockDim.x) {
      const int hh = e >> 7, jj = e & 127;
      float M = -INFINITY;
      for (int w = 0; w < nwav; ++w) M = fmaxf(M, red[(w * 4 + hh) * ATT_PART_FLOATS + 128]);
      float A = 0.0f, Ls = 0.0f;
      for (int w = 0; w < nwav; ++w) {
        const float* rw = red + (w * 4 + hh) * ATT_PART_FLOATS;
        const float f = (rw[128] == -INFINITY) ? 0.0f : exp2f(rw[128] - M);
        A += f * rw[jj];
        Ls += f * rw[129];
      }
      float* ph = part + (4 * c4 + hh) * ATT_PART_FLOATS;
      ph[jj] = A;
      if (jj == 0) { ph[128] = M; ph[129] = Ls; }
    }
    if (4 * (c4 + 1) < g) __syncthreads();
  }
}

// ======================================================================
// Decode-step attention over eigen / identity caches with the packed bits
// fed to the matrix cores (k_att2; one workgroup per (KV head, token split),
// the same split partials and merge kernel as k_att_main).
//
// Scores. A K record is a string of B bits and the score is linear in them:
// record bit c, bit k of channel j's code, carries a_j 2^k with
// a_j = (U_K^T q)_j step_j scale log2(e). Each lane holds half of its token's
// record, realigned to bit 0, and turns each record word w into eight int8
// operand words with one AND each: w & (0x01010101 << r) and
// (w >> 4) & (0x01010101 << r), r = 0..3, whose byte q is bit 8q + r (or
// 8q + 4 + r) of w times 2^r. The weights a_j 2^k 2^-r, scaled by a power of
// two per query head, are split into three int8 parts that sit in rows
// 4H + p (p = 0..2) of the 32x32x32 int8 MFMA, so the accumulators are exact
// integers and a lane finds the three parts of heads H = 2i + h (h its half
// of the wave) in accumulators 4i .. 4i + 2.
// Values. Each lane quad (four consecutive tokens) transposes its V record
// words by byte and splits each result into the bytes of tokens (0, 2) and of
// tokens (1, 3), each byte in the low half of a 16-bit field; both words go to
// LDS rows [record byte][token quad]. A value column is the fragment of one
// channel's code that lies in one record byte: lane (column, token octet)
// reads the four words of two quads of the column's row and masks the
// fragment in place. Each 16-bit half is then an fp16 subnormal fragment
// * 2^(shift - 24), exact, and the words are the B operand of the fp16
// 16x16x32 MFMA against P (the softmax weights stored in the same token
// order). When the waves merge, the columns of each channel are added with
// their scales 2^(24 - shift + offset of the fragment in the code), which
// gives the split partials in code units.
// ======================================================================
constexpr int AT2_PST = 136;  // fp16 per token octet of P ([octet][16 heads][8] + 8 pad: octets 4 banks apart)
constexpr int AT2_BT = 32;    // tokens per wave block
// Word offset of value row r ([quad][tokens 0,2 | 1,3], 16 words). For records
// of at most 256 bits, 24 r + 12 (r >> 2) + 8 (r >> 3): the 8-byte writes of
// four rows by 16 lanes fall in 32 different banks and the 16-byte reads of
// consecutive rows spread over the 64 (this layout measured faster than
// octet-major rows, whose writes conflict); longer records: 16 r, to fit the
// LDS.
__host__ __device__ constexpr unsigned at2_vrow(int R2M, unsigned r) {
  return R2M <= 4 ? 24u * r + 12u * (r >> 2) + 8u * (r >> 3) : 16u * r;
}
// Workgroups per CU of k_att2<R2M, .., NCH, W, SWZ, G4>: four for the
// four-wave instances whose registers fit 128 per lane (256-bit records with
// groups up to 4; records of at most 96-bit halves), else three (four waves)
// or one (eight waves).
__host__ __device__ constexpr int at2_occ(int R2M, int NCH, int W, bool SWZ, bool G4) {
  return W == 4 ? (NCH == 1 && ((SWZ && G4) || R2M == 3) ? 4 : 3) : 1;
}
// stages of the record ring of one wave (blocks in flight: stages - 1): two
// at four workgroups per CU, to fit the LDS
__host__ __device__ constexpr int at2_nst(int NCH, int OCC) { return NCH == 1 && OCC < 4 ? 3 : 2; }
// value rows of at most 256-bit records at four workgroups per CU: 16 r
// words, to fit the LDS
__host__ __device__ constexpr unsigned at2_vrowo(int R2M, int OCC, unsigned r) {
  return OCC == 4 && R2M == 4 ? 16u * r : at2_vrow(R2M, r);
}
// weight-table rows: three per head of the instance, then one of zeros
__host__ __device__ constexpr int at2_trows(bool G4) { return G4 ? 13 : 25; }
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

// byte of a score-weight row that holds record bit c: record word dw = c >> 5
// (the i-th word of lane half dw >= R2, each half's words R2M apart), operand
// half (c & 7) >> 2, operand word c & 3, byte (c >> 3) & 3
__device__ __forceinline__ unsigned at2_tab_off(unsigned c, unsigned R2, unsigned R2M) {
  const unsigned dw = c >> 5, hh = dw >= R2 ? 1u : 0u;
  return (dw - hh * R2 + hh * R2M) * 32u + ((c & 7u) >> 2) * 16u + (c & 3u) * 4u + ((c >> 3) & 3u);
}
// The same for the 16x16x64 layout of 256-bit records and groups up to 4:
// word dw of a record is taken by k-block dw >> 1 at steps 2 (dw & 1) and
// 2 (dw & 1) + 1 (its two operand halves); a row holds [step][k-block][16].
__device__ __forceinline__ unsigned at2_tab_off16(unsigned c) {
  const unsigned dw = c >> 5, kk = (c & 7u) >> 2;
  return (2u * (dw & 1u) + kk) * 64u + (dw >> 1) * 16u + (c & 3u) * 4u + ((c >> 3) & 3u);
}
// The unscaled score from the three parts' accumulators: the integer
// 2^14 p0 + 2^7 p1 + p2 is S times the score, and S (at most 2^20 over the
// largest weight |a_j| 2^(b_j - 1)) keeps it within 2^28 for 128 channels,
// so the int32 sum is exact and one conversion rounds it.
__device__ __forceinline__ float at2_score(int p0, int p1, int p2) {
  int x = p0 * 128 + p1;
  asm("" : "+v"(x));  // (kept as two shift-adds, not reassociated into three operations)
  return (float)(x * 128 + p2);
}
// position of token t of a block in the P / value-operand order: inside each
// group of four tokens the order is 0, 2, 1, 3
__device__ __forceinline__ int at2_pos(int t) { return (t & ~3) | ((t & 1) << 1) | ((t >> 1) & 1); }

// The int8 operand words of record word w: half kk of its eight.
__device__ __forceinline__ u32x4 at2_bits(unsigned w, int kk) {
  const unsigned x = kk ? (w >> 4) : w;
  return (u32x4){x & 0x01010101u, x & 0x02020202u, x & 0x04040404u, x & 0x08080808u};
}

// Record byte 4i + e of the four tokens of a lane quad (e = lane & 3, x the
// lane's record word i), split by token parity: .x = bytes of tokens 0 and 2
// in bits 0-7 and 16-23, .y = those of tokens 1 and 3 (two DPP moves and
// three byte permutes).
__device__ __forceinline__ u32x2 at2_quad_split(unsigned x, unsigned sel1, unsigned sel_e, unsigned sel_o) {
  const unsigned p1 = (unsigned)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false);  // lane e^1
  const unsigned y = __builtin_amdgcn_perm(p1, x, sel1);
  const unsigned p2 = (unsigned)__builtin_amdgcn_mov_dpp((int)y, 0x4E, 0xF, 0xF, false);  // lane e^2
  return (u32x2){__builtin_amdgcn_perm(p2, y, sel_e), __builtin_amdgcn_perm(p2, y, sel_o)};
}

// Staging modes: AT2_GEN, the block's bytes from the 16-byte boundary at or
// below its start, in order; AT2_SWZ (256-bit records), chunk q of half h of
// token t at slot t + 32 h + 64 q; AT2_DIRECT (half records of at most 96
// bits), slot t + 32 h holds the 16 bytes from the word that holds the first
// bit of half h of token t.
constexpr int AT2_GEN = 0, AT2_SWZ = 1, AT2_DIRECT = 2;
// A lane's half record from a wave's staging buffer: R2 words from record bit
// 32 R2 h of token t, realigned to bit 0 (AT2_GEN: the block's records start
// at bit `off` of the buffer; AT2_DIRECT: off is the lane's bit shift). Words
// past the half record hold other bits, which meet zero weights and columns
// that never read them.
template <int R2M, int MODE>
__device__ __forceinline__ void at2_read(unsigned (&r)[R2M], const unsigned* buf, unsigned off, unsigned B, int R2,
                                         int t, int h, unsigned lim) {
  if (MODE == AT2_DIRECT) {
    // slot t + 32 h holds the 16 bytes from the word that holds the half
    // record's first bit; off is that bit's position in the word
    const u32x4 v = *reinterpret_cast<const u32x4*>(buf + 4 * (t + 32 * h));
    const unsigned x[4] = {v[0], v[1], v[2], v[3]};
#pragma unroll
    for (int j = 0; j < R2M; ++j) r[j] = __builtin_amdgcn_alignbit(x[j + 1], x[j], off);
    return;
  }
  if (MODE == AT2_SWZ) {
#pragma unroll
    for (int j = 0; j < R2M; j += 4) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(buf + 4 * (t + 32 * h + 64 * (j >> 2)));
      r[j] = v[0]; r[j + 1] = v[1]; r[j + 2] = v[2]; r[j + 3] = v[3];
    }
    return;
  }
  const unsigned P = off + (unsigned)t * B + 32u * (unsigned)R2 * (unsigned)h;
  const unsigned* w = buf + (P >> 5);
  const unsigned sh = P & 31u;
  unsigned x[R2M + 1];
  if (!STC_CHECK((P >> 5) + R2M < lim, DBG_ATT_STAGE)) w = buf;
#pragma unroll
  for (int j = 0; j <= R2M; ++j) x[j] = w[j];
#pragma unroll
  for (int j = 0; j < R2M; ++j) r[j] = __builtin_amdgcn_alignbit(x[j + 1], x[j], sh);
}

// Request the records of block blk of one stream (4 B bytes from byte 4 B blk)
// into a wave's staging buffer: NCH buffer loads of 16 bytes per lane
// straight to LDS, from the 16-byte boundary at or below the block's first
// byte (returned in bits, the offset of the records in the buffer). Load c of
// a lane reads rel[c] bytes past that boundary (at2_stage_rel) through a
// buffer resource whose range ends at the block's last byte (256-bit records:
// at the block's end) and at the stream's plen bytes: lanes past it read
// zeros and move no data. A stream of no bytes (or a request past a split's
// end) passes plen 0.
template <int NCH, int MODE>
__device__ __forceinline__ unsigned at2_stage(const unsigned char* stream, unsigned blk, unsigned B, unsigned plen,
                                              unsigned* buf, const unsigned (&rel)[NCH]) {
  // (streams of this kernel hold fewer than 2^31 bytes: 32-bit scalar arithmetic)
  const unsigned start = blk * 4u * B;
  // AT2_DIRECT: the resource starts at the block (4-byte aligned) and reaches
  // 16 bytes past it (the lanes' 16-byte windows), or the stream's end
  const unsigned base = MODE == AT2_DIRECT ? start : start & ~15u;
  int lim = (int)plen - (int)base;  // bytes past base that the lanes may read (uniform)
  if (MODE == AT2_GEN && lim > (int)(start - base + 4u * B)) lim = (int)(start - base + 4u * B);
  if (MODE == AT2_DIRECT && lim > (int)(4u * B + 16u)) lim = (int)(4u * B + 16u);
  // (scalar clamps: the first value passes readfirstlane, so that the two are
  // not merged into one vector med3)
  lim = __builtin_amdgcn_readfirstlane(lim < 0 ? 0 : lim);
  if (MODE != AT2_DIRECT && lim > 1024 * NCH + 16) lim = 1024 * NCH + 16;  // (the loads reach no further)
#if defined(__HIP_DEVICE_COMPILE__)  // (buffer resources exist in the device pass only)
  // (uniform by construction; readfirstlane keeps the resource in scalar registers)
  const unsigned long long ad = (unsigned long long)(stream + (lim > 0 ? base : 0u));
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)ad), hi = __builtin_amdgcn_readfirstlane((unsigned)(ad >> 32));
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(((unsigned long long)hi << 32) | lo), (short)0, __builtin_amdgcn_readfirstlane(lim), 0x00020000);
#pragma unroll
  for (int c = 0; c < NCH; ++c)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(buf + 256 * c), 16, rel[c],
                                             0, 0, 0);
#endif
  return (start - base) * 8u;
}
// Per-lane byte offsets of at2_stage's loads: AT2_GEN, 16 lane + 1024 c;
// AT2_SWZ, slot lane takes chunk 2 t + h + c (t = lane & 31, h = lane >> 5),
// so that the 16-byte reads of 16 consecutive lanes cover 64 banks (in block
// order they would pair up); AT2_DIRECT, the word that holds bit t B + 32 R2 h
// (sh: that bit's position in the word).
template <int NCH, int MODE>
__device__ __forceinline__ void at2_stage_rel(unsigned (&rel)[NCH], unsigned& sh, int lane, unsigned B, int R2) {
  const unsigned P = (unsigned)(lane & 31) * B + 32u * (unsigned)R2 * (unsigned)(lane >> 5);
  sh = P & 31u;
#pragma unroll
  for (int c = 0; c < NCH; ++c)
    rel[c] = MODE == AT2_SWZ      ? 16u * (unsigned)(2 * (lane & 31) + (lane >> 5) + c)
             : MODE == AT2_DIRECT ? 4u * (P >> 5)
                                  : 1024u * c + 16u * (unsigned)lane;
}


// Score weights of the packed-bit kernel, once per pair (its splits share
// them): a_j = (U_K^T q)_j step_j scale log2(e) for the group's heads (0 for
// dropped channels and heads past the group), and per head the power of two
// S that scales the largest weight max_j |a_j| 2^(b_j - 1) to at most 2^20.
// 1024 threads: thread (part, j) sums rows part, part + 8, .. of U_K for
// channel j and all eight heads (its 16 loads in flight at once); the eight
// parts are added through LDS.
constexpr int PREP_PARTS = 2;  // (256 threads: many workgroups per CU)
// Generation-step append, one wave per stream: the record of one token is
// formed exactly as k_encode_eigen forms it (the same MFMA chain on the same
// basis rows, the token in every column of the block, the same quantizer and
// group words), so the appended bytes equal those of an encode of the whole
// stream. It is written over the stream's words from the record's first bit
// to the 16-byte end of the stream; the bits of earlier records in its first
// word are kept. sbuf: 64 words of LDS for this wave.
template <bool F32>
__device__ void append_record(const unsigned char* st, const void* x, unsigned char* stream, long long n_old,
                              long long stride, unsigned* sbuf, int lane) {
  const DevHdr* hdr = reinterpret_cast<const DevHdr*>(st + OFF_HDR);
  const unsigned B = (unsigned)__builtin_amdgcn_readfirstlane(hdr->total_bits);
  if (B == 0) return;  // no kept channel: the stream has no bytes
  const int t32 = lane & 31, h = lane >> 5;
  bf16x8 xh[8], xl[8];
  if (F32) {
    const float* row = static_cast<const float*>(x);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const f32x4 v0 = *reinterpret_cast<const f32x4*>(row + 16 * ks + 8 * h);
      const f32x4 v1 = *reinterpret_cast<const f32x4*>(row + 16 * ks + 8 * h + 4);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float f = e < 4 ? v0[e] : v1[e - 4];
        const __bf16 hi = (__bf16)f;
        xh[ks][e] = hi;
        xl[ks][e] = (__bf16)(f - (float)hi);
      }
    }
  } else {
    const unsigned short* row = static_cast<const unsigned short*>(x);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) xh[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(row + 16 * ks + 8 * h));
  }
  sbuf[lane] = 0u;
  __builtin_amdgcn_s_waitcnt(0xc07f);
  __builtin_amdgcn_wave_barrier();
  const long long P0 = n_old * (long long)B;
  const unsigned sh0 = (unsigned)(P0 & 31);
  const unsigned char* uh = st + OFF_UT_HI + t32 * 256 + 16 * h;
  const unsigned char* ul = st + OFF_UT_LO + t32 * 256 + 16 * h;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    // channels 64h + 16mb + 4i + j of the token in acc[4i + j] (rows of the
    // basis permuted by the state builder), the chain started from yhalf
    f32x16 acc;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[4 * i + j] = hdr->yhalf[64 * h + 16 * mb + 4 * i + j];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const bf16x8 ah = *reinterpret_cast<const bf16x8*>(uh + 32 * mb * 256 + 32 * ks);
      const bf16x8 al = *reinterpret_cast<const bf16x8*>(ul + 32 * mb * 256 + 32 * ks);
      acc = mfma32_bf16(ah, xh[ks], acc);
      acc = mfma32_bf16(al, xh[ks], acc);
      if (F32) acc = mfma32_bf16(ah, xl[ks], acc);
    }
    if (t32 == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c0 = 64 * h + 16 * mb + 4 * i;
        const unsigned goff = (unsigned)hdr->off[c0];
        unsigned word = 0u;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const unsigned q = (unsigned)__builtin_amdgcn_fmed3f(acc[4 * i + j], 0.0f, (float)hdr->lm1[c0 + j]);
          word |= q << ((unsigned)hdr->off[c0 + j] - goff);
        }
        const unsigned rb = sh0 + goff;
        const unsigned long long v = (unsigned long long)word << (rb & 31u);
        __hip_atomic_fetch_or(sbuf + (rb >> 5), (unsigned)v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        __hip_atomic_fetch_or(sbuf + (rb >> 5) + 1, (unsigned)(v >> 32), __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_WORKGROUP);
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // one row block's basis rows in registers at a time
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);
  __builtin_amdgcn_wave_barrier();
  const long long w0 = P0 >> 5;
  const int nw = (int)(packed_len((long long)B, n_old + 1) / 4 - w0);  // <= 33 + 3 words
  unsigned* s32 = reinterpret_cast<unsigned*>(stream);
  if (lane < nw && STC_CHECK(stride == 0 || 4 * (w0 + nw) <= stride, DBG_APPEND)) {
    unsigned v = sbuf[lane];
    if (lane == 0 && sh0 != 0u) v |= s32[w0] & ((1u << sh0) - 1u);
    s32[w0 + lane] = v;
  }
}

// The appends of a generation step, K on wave 0 and V on wave 1 (streams
// without a state are left as they are). F32: fp32 token rows (else bf16).
template <bool F32>
__device__ __forceinline__ void att_append_pair(const AttK& a, long long pg, long long ksi, long long vsi,
                                                unsigned (*sbuf)[64], int tid) {
  const int wave = tid >> 6, lane = tid & 63;
  const long long n_old = a.n_tokens - 1;
  const long long si = wave == 0 ? ksi : vsi;
  if (wave > 1 || si < 0) return;
  const unsigned char* st = (wave == 0 ? a.k_states : a.v_states) + (size_t)si * STATE_BYTES;
  unsigned char* stream = const_cast<unsigned char*>(wave == 0 ? a.k_packed : a.v_packed) + pg * a.packed_stride;
  const unsigned char* x = static_cast<const unsigned char*>(wave == 0 ? a.k_new : a.v_new) + pg * 128 * (F32 ? 4 : 2);
  append_record<F32>(st, x, stream, n_old, a.packed_stride, sbuf[wave], lane);
}

// The appends in a launch of their own: fp32 token rows (their three-pass
// chain needs more registers than the prep kernel's 1024 threads leave), or
// attention instances without the prep launch.
__global__ void __launch_bounds__(128) k_att_append(AttK a) {
  __shared__ unsigned sbuf[2][64];
  const long long pg = a.pair_base + blockIdx.x;
  const long long ksi = state_index(a.k_map, pg, a.n_states), vsi = state_index(a.v_map, pg, a.n_states);
  if (a.new_f32) att_append_pair<true>(a, pg, ksi, vsi, sbuf, threadIdx.x);
  else att_append_pair<false>(a, pg, ksi, vsi, sbuf, threadIdx.x);
}

// APPEND: a generation step's bf16 new-token rows are appended first.
template <bool APPEND>
__global__ void __launch_bounds__(128 * PREP_PARTS) k_att2_prep(AttK a) {
  __shared__ __align__(16) float sqT[128 * 8];   // q^T [128][8]
  __shared__ float red[PREP_PARTS][8][128];
  __shared__ float wmax[8][2];
  const int tid = threadIdx.x;
  const long long p = blockIdx.x, pg = a.pair_base + p;
  const int g = a.group;
  const long long ksi = state_index(a.k_map, pg, a.n_states), vsi = state_index(a.v_map, pg, a.n_states);
  __shared__ unsigned sapp[2][64];
  // generation step: the new token's K and V records go into the caches
  // first (the main kernel, the next launch, reads them with the rest)
  if (APPEND) att_append_pair<false>(a, pg, ksi, vsi, sapp, tid);
  if (ksi < 0 || vsi < 0) return;  // (the main kernel writes nothing for this pair either)
  const unsigned char* kst = a.k_states + (size_t)ksi * STATE_BYTES;
  const DevHdr* hk = reinterpret_cast<const DevHdr*>(kst);
  const int j = tid & 127, part = tid >> 7;
  const float* u = reinterpret_cast<const float*>(kst + OFF_U32);
  const float* qp = a.q + pg * g * 128;
  for (int e = tid; e < 128 * 8; e += 128 * PREP_PARTS) {
    const int r = e >> 3, hh = e & 7;
    sqT[e] = hh < g ? qp[hh * 128 + r] : 0.0f;
  }
  __syncthreads();
  // thread (part, j): rows part + PREP_PARTS k of column j of U_K, in chunks
  // of 16 rows (loads of a chunk in flight together)
  constexpr int RPP = 128 / PREP_PARTS;
  float acc[8];
#pragma unroll
  for (int hh = 0; hh < 8; ++hh) acc[hh] = 0.0f;
#pragma unroll
  for (int k0 = 0; k0 < RPP; k0 += 16) {
    float ur[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) ur[k] = u[(part + PREP_PARTS * (k0 + k)) * 128 + j];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const f32x4* q4 = reinterpret_cast<const f32x4*>(sqT + (part + PREP_PARTS * (k0 + k)) * 8);
      const f32x4 q0 = q4[0], q1 = q4[1];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[e] = __builtin_fmaf(ur[k], q0[e], acc[e]);
        acc[4 + e] = __builtin_fmaf(ur[k], q1[e], acc[4 + e]);
      }
    }
  }
#pragma unroll
  for (int hh = 0; hh < 8; ++hh) red[part][hh][j] = acc[hh];
  __syncthreads();
  float* pre = a.prep + p * ATT_PREP_FLOATS;
  {
    // thread (half, c): channel c of heads 4 half .. 4 half + 3; the two
    // waves of a half hold channels 0..63 and 64..127
    const int c = tid & 127, half = tid >> 7;
    const unsigned b = hk->bits[c];
    const float f = hk->step32[c] * a.scale * LOG2E;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int hh = 4 * half + r;
      float v = 0.0f;
      if (hh < g && b > 0) {
        float sum = 0.0f;
#pragma unroll
        for (int pt = 0; pt < PREP_PARTS; ++pt) sum += red[pt][hh][c];
        v = sum * f;
      }
      pre[hh * 128 + c] = v;
      // the largest weight of the head: max over c of |a_c| 2^(b_c - 1)
      float m = b > 0 ? fabsf(v) * (float)(1u << (b - 1)) : 0.0f;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
      if ((tid & 63) == 0) wmax[hh][(tid >> 6) & 1] = m;
    }
  }
  __syncthreads();
  if (tid < 8) {
    const float M = fmaxf(wmax[tid][0], wmax[tid][1]);
    int ex = 0;
    frexpf(M, &ex);
    pre[8 * 128 + tid] = M > 0.0f ? ldexpf(1.0f, 20 - ex) : 1.0f;
  }
}

// Dynamic LDS of k_att2<R2M, NT, NCH, W, .., G4>: the score weights, the
// value column table and the per-head scales, then the larger of the prologue
// scratch, the W wave regions and the merge scratch.
__host__ __device__ constexpr size_t at2_lds_bytes(int R2M, int NT, int NCH, int W, bool SWZ, bool G4) {
  const int occ = at2_occ(R2M, NCH, W, SWZ, G4);
  const size_t fixed =
      (size_t)at2_trows(G4) * (64 * R2M + 16) + ATT_MAX_VCOLS * 8 + 8 * 4 + 128 * 4 + ATT_MAX_VCOLS * 4 + 16 * 4;
  const size_t pro = (size_t)8 * 128 * 4 + 2 * 64 * R2M + 8 * 4;
  const size_t vwords = (size_t)at2_vrowo(R2M, occ, 8 * R2M - 1) + 16;
  const size_t waves = (size_t)W * (2 * at2_nst(NCH, occ) * 256 * NCH + vwords + 4 * AT2_PST / 2 + 16) * 4;
  const size_t merge = (size_t)W * 8 * (16 * NT + 4) * 4;
  const size_t big = pro > waves ? (pro > merge ? pro : merge) : (waves > merge ? waves : merge);
  return fixed + big;
}

// R2M: record words per half record at most (records of at most 64 R2M bits);
// NT: value tiles (columns <= 16 NT); NCH: 1 KiB loads per stream and block;
// W: waves; SWZ: every record is 256 bits (R2M = 4, NCH = 1); G4: group <= 4
// (a lane's heads are 2i + h for i < 2, otherwise i < 4).
template <int R2M, int NT, int NCH, int W, bool SWZ, bool G4>
__global__ void __launch_bounds__(64 * W, at2_occ(R2M, NCH, W, SWZ, G4)) k_att2(AttK a) {
  static_assert(!SWZ || (R2M == 4 && NCH == 1), "256-bit records: four words per half, one load per block");
  extern __shared__ __align__(16) unsigned char smem[];
  // S16: 256-bit records and groups up to 4 take the scores from 16x16x64
  // MFMAs (rows 4H + p: the four heads fill them), lane (c16, g4) holding
  // head g4 for tokens c16 and 16 + c16; otherwise 32x32x32, lane (t32, h)
  // holding heads 2i + h for token t32
  constexpr bool S16 = SWZ && G4;
  constexpr int MODE = SWZ ? AT2_SWZ : (R2M <= 3 && NCH == 1 ? AT2_DIRECT : AT2_GEN);
  constexpr int NHL = G4 ? 2 : 4;              // score slots per lane
  constexpr int NH = G4 ? 4 : 8;               // heads of the weight table
  constexpr int TABW = 64 * R2M;               // bytes of a score-weight row (record bits <= 64 R2M)
  constexpr int TROW = TABW + 16;              // row stride: rows 4 banks apart, so 16 lanes' reads hit 64 banks
  constexpr int TROWS = at2_trows(G4);         // rows 3H + p of head H, part p; then a row of zeros
  constexpr int OCC = at2_occ(R2M, NCH, W, SWZ, G4);
  constexpr int VWORDS = (int)at2_vrowo(R2M, OCC, 8 * R2M - 1) + 16;  // value rows: 4 R2M record bytes per lane half
  constexpr int SWORDS = 256 * NCH;            // words of one staging buffer
  constexpr int NST = at2_nst(NCH, OCC);       // ring stages (blocks in flight: NST - 1)
  constexpr int WREG = 2 * NST * SWORDS + VWORDS + 4 * AT2_PST / 2 + 16;  // words per wave region
  static_assert(3 * NH + 1 == TROWS, "weight-table rows");
  static_assert(WREG % 4 == 0 && (TROWS * TROW) % 16 == 0, "16-byte aligned LDS regions");
  signed char* sA = reinterpret_cast<signed char*>(smem);            // [TROWS][TROW]
  u32x2* sVc = reinterpret_cast<u32x2*>(smem + TROWS * TROW);        // [256] (row word offset, mask2)
  float* sInvS = reinterpret_cast<float*>(sVc + ATT_MAX_VCOLS);     // [8]
  unsigned* sVch = reinterpret_cast<unsigned*>(sInvS + 8);          // [128] channel: first column | count << 16
  float* sFac = reinterpret_cast<float*>(sVch + 128);                // [256] column scale 2^(24 - shift + offset)
  unsigned* sOnes = reinterpret_cast<unsigned*>(sFac + ATT_MAX_VCOLS);  // [16] fp16 pairs (1, 1): the sum column
  unsigned* sReg0 = sOnes + 16;                                         // wave regions / prologue scratch
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t32 = lane & 31, h = lane >> 5;
  const int c16 = lane & 15, g4 = lane >> 4;
  const long long sp = blockIdx.x, p = blockIdx.y;
  const long long pg = a.pair_base + p;
  const long long n = a.n_tokens;
  const int g = a.group;
  const long long ksi = state_index(a.k_map, pg, a.n_states), vsi = state_index(a.v_map, pg, a.n_states);
  if (ksi < 0 || vsi < 0) {  // (the whole workgroup) no state: NaN, written here or by the merge
    if (a.direct)
      for (int e = tid; e < g * 128; e += blockDim.x) a.out[pg * g * 128 + e] = __builtin_nanf("");
    return;
  }
  const unsigned char* kst = a.k_states + (size_t)ksi * STATE_BYTES;
  const unsigned char* vst = a.v_states + (size_t)vsi * STATE_BYTES;
  const DevHdr* hk = reinterpret_cast<const DevHdr*>(kst);
  const DevHdr* hv = reinterpret_cast<const DevHdr*>(vst);
  const unsigned Bk = (unsigned)__builtin_amdgcn_readfirstlane(hk->total_bits);
  const unsigned Bv = (unsigned)__builtin_amdgcn_readfirstlane(hv->total_bits);
  const int R2k = (int)((((Bk + 31u) >> 5) + 1u) >> 1), R2v = (int)((((Bv + 31u) >> 5) + 1u) >> 1);
  const int ncols = __builtin_amdgcn_readfirstlane(hv->n_vcols);
  const long long t_begin = sp * a.split_tokens;
  long long t_end = t_begin + a.split_tokens;
  if (t_end > n) t_end = n;

  // ------------------------------------------------------------ prologue
  {
    // the pair's score weights a [8][128] and head scales (k_att2_prep)
    float* sAf = reinterpret_cast<float*>(sReg0);                             // a [8][128]
    unsigned short* sBit = reinterpret_cast<unsigned short*>(sAf + 8 * 128);  // [TABW] record bit -> j | k << 8
    float* sS = reinterpret_cast<float*>(sBit + TABW);                        // [8] per-head scales
    const float* pre = a.prep + p * ATT_PREP_FLOATS;
    for (int i = tid; i < TROWS * TROW / 16; i += blockDim.x) reinterpret_cast<u32x4*>(sA)[i] = (u32x4){0u, 0u, 0u, 0u};
    for (int i = tid; i < TABW; i += blockDim.x) sBit[i] = 0xFFFFu;
    for (int e = tid; e < 8 * 128 / 4; e += blockDim.x)
      reinterpret_cast<f32x4*>(sAf)[e] = reinterpret_cast<const f32x4*>(pre)[e];
    if (tid < 8) {
      sS[tid] = pre[8 * 128 + tid];
      sInvS[tid] = 1.0f / pre[8 * 128 + tid];
    }
    __syncthreads();
    if (tid < 128) {
      const unsigned b = hk->bits[tid], o = hk->off[tid];
      for (unsigned k = 0; k < b; ++k) sBit[o + k] = (unsigned short)(tid | (k << 8));
    }
    if (tid < ATT_MAX_VCOLS) {
      const AttVCol* vc = reinterpret_cast<const AttVCol*>(vst + OFF_ATTV);
      u32x2 e = (u32x2){0u, 0u};
      if (tid < ncols) {
        // record byte k of lane half hh sits in value row k - 4 R2v hh + 4 R2M hh
        const unsigned row = vc[tid].row, hh = row >= 4u * (unsigned)R2v ? 1u : 0u;
        e = (u32x2){at2_vrowo(R2M, OCC, row - 4u * (unsigned)R2v * hh + 4u * R2M * hh), vc[tid].mask2};
      }
      sVc[tid] = e;
      sFac[tid] = tid < ncols ? vc[tid].fac : 0.0f;
      if (tid < 128) sVch[tid] = reinterpret_cast<const unsigned*>(vst + OFF_ATTVCH)[tid];
      if (tid < 16) sOnes[tid] = 0x3C003C00u;
    }
    __syncthreads();
    // int8 parts of round(S_h a_j 2^(k - (c & 3))): rows 3h + p
    for (int e = tid; e < NH * TABW; e += blockDim.x) {
      const int hh = e / TABW, c = e - hh * TABW;
      const unsigned bj = sBit[c];
      if (hh < g && bj != 0xFFFFu && (unsigned)c < Bk) {
        const int jj = bj & 255, k = bj >> 8;
        const float w = sAf[hh * 128 + jj] * ldexpf(sS[hh], k - (c & 3));
        const int A = (int)rintf(w);
        const int a2 = ((A + 64) & 127) - 64;
        const int r1 = (A - a2) >> 7;
        const int a1 = ((r1 + 64) & 127) - 64;
        const int a0 = (r1 - a1) >> 7;
        const unsigned o = S16 ? at2_tab_off16((unsigned)c) : at2_tab_off((unsigned)c, (unsigned)R2k, (unsigned)R2M);
        sA[(3 * hh) * TROW + o] = (signed char)a0;
        sA[(3 * hh + 1) * TROW + o] = (signed char)a1;
        sA[(3 * hh + 2) * TROW + o] = (signed char)a2;
      }
    }
    __syncthreads();
  }

  // wave regions: NST staging buffers per stream, value rows, P, alpha
  unsigned* sStage = sReg0 + wave * WREG;                                 // [stage][K, V][SWORDS]
  unsigned* sV = sStage + 2 * NST * SWORDS;                               // value rows (at2_vrow)
  _Float16* sP = reinterpret_cast<_Float16*>(sV + VWORDS);                // P [4 octets][16 heads][8] (+ pad)
  float* sAl = reinterpret_cast<float*>(sP + 4 * AT2_PST);               // alpha per head [16]
  for (int i = lane; i < 4 * AT2_PST / 2; i += 64) reinterpret_cast<unsigned*>(sP)[i] = 0u;
  if (lane < 16) sAl[lane] = 1.0f;
  // per head of the lane (H = 2i + h): running max, its threshold of the
  // fast path in unscaled score units, the scales. (The running sum of P is
  // the value column ncols, whose operand is fp16 1 for every token.)
  float mold[NHL], thr[NHL], invS[NHL];
  bool hval[NHL];
#pragma unroll
  for (int i = 0; i < NHL; ++i) {
    const int H = S16 ? g4 : 2 * i + h;
    invS[i] = sInvS[H];
    mold[i] = -INFINITY;
    thr[i] = -INFINITY;
    hval[i] = H < g;
  }
  f32x4 acc_v[NT];
#pragma unroll
  for (int T = 0; T < NT; ++T) acc_v[T] = (f32x4){0.f, 0.f, 0.f, 0.f};
  // value columns of this lane: LDS address of the four words it reads and
  // the fragment mask (columns past the state's have mask 0; column ncols
  // reads the ones)
  unsigned vaddr[NT], vmask[NT];
  {
    const unsigned vb0 = lds_offset(reinterpret_cast<unsigned char*>(sV));
    const unsigned ones = lds_offset(reinterpret_cast<unsigned char*>(sOnes));
#pragma unroll
    for (int T = 0; T < NT; ++T) {
      const u32x2 cm = sVc[16 * T + c16];
      const bool sumcol = 16 * T + c16 == ncols;
      vaddr[T] = sumcol ? ones + 16u * (unsigned)g4 : vb0 + 4u * (cm[0] + 4u * (unsigned)g4);
      vmask[T] = sumcol ? 0xFFFFFFFFu : cm[1];
      asm volatile("" : "+v"(vaddr[T]), "+v"(vmask[T]));
    }
  }
  // LDS address of the lane's score-weight row. 16x16x64: lane row c16 =
  // 4H + p holds part p of head H, k-block g4; 32x32x32: lane row t32 = 4H + p,
  // half h. Table row 3H + p, or the zero row for p = 3 and heads past the
  // table.
  unsigned abase;
  {
    const int rr = S16 ? c16 : t32;
    const int trow = ((rr & 3) == 3 || (rr >> 2) >= NH) ? 3 * NH : 3 * (rr >> 2) + (rr & 3);
    abase = lds_offset(reinterpret_cast<unsigned char*>(sA) + trow * TROW + (S16 ? g4 * 16 : h * R2M * 32));
    asm volatile("" : "+v"(abase));
  }
  const unsigned PkL = (unsigned)packed_len((long long)Bk, n), PvL = (unsigned)packed_len((long long)Bv, n);
  const unsigned char* gk = a.k_packed + pg * a.packed_stride;
  const unsigned char* gv = a.v_packed + pg * a.packed_stride;
  const int e4 = t32 & 3;
  const unsigned sel1 = (e4 & 1) ? 0x03070105u : 0x06020400u;
  const unsigned sel_e = (e4 & 2) ? 0x0C020C06u : 0x0C040C00u;
  const unsigned sel_o = (e4 & 2) ? 0x0C030C07u : 0x0C050C01u;
  const unsigned pos = (unsigned)at2_pos(t32);
  bool resc = false;  // (uniform) a rescale of the value accumulators is pending
  // the wave's blocks: tok0 = t_begin + 32 (wave + W k) (token counts below
  // 2^31: 32-bit scalar arithmetic). The records of the next NST - 1 blocks
  // are requested (straight to LDS) before the current one is processed;
  // past the split's end the requests are of nothing (plen 0), so that every
  // step issues 2 NCH loads
  const int stride = W * AT2_BT;
  const int tend = (int)t_end;
  int tok0 = (int)t_begin + wave * AT2_BT;
  unsigned offk[NST], offv[NST];
  unsigned krel[NCH], vrel[NCH], ksh, vsh;
  at2_stage_rel<NCH, MODE>(krel, ksh, lane, Bk, R2k);
  at2_stage_rel<NCH, MODE>(vrel, vsh, lane, Bv, R2v);
  __builtin_amdgcn_s_waitcnt(0xc07f);
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int st = 0; st < NST - 1; ++st) {
    const int tb = tok0 + st * stride;
    const bool real = tb < tend;
    unsigned* buf = sStage + st * 2 * SWORDS;
    offk[st] = at2_stage<NCH, MODE>(gk, real ? (unsigned)tb / AT2_BT : 0u, Bk, real ? PkL : 0u, buf, krel);
    offv[st] = at2_stage<NCH, MODE>(gv, real ? (unsigned)tb / AT2_BT : 0u, Bv, real ? PvL : 0u, buf + SWORDS, vrel);
  }
  int cur = 0;  // ring stage of the current block
  for (; tok0 < tend; tok0 += stride) {
    {
      const int tb = tok0 + (NST - 1) * stride;
      const bool real = tb < tend;
      unsigned* buf = sStage + (cur == 0 ? NST - 1 : cur - 1) * 2 * SWORDS;
      offk[NST - 1] = at2_stage<NCH, MODE>(gk, real ? (unsigned)tb / AT2_BT : 0u, Bk, real ? PkL : 0u, buf, krel);
      offv[NST - 1] =
          at2_stage<NCH, MODE>(gv, real ? (unsigned)tb / AT2_BT : 0u, Bv, real ? PvL : 0u, buf + SWORDS, vrel);
    }
    // the current block's loads are done once at most the later blocks' remain
    __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * NCH * (NST - 1)));  // vmcnt(2 NCH (NST - 1))
    __builtin_amdgcn_wave_barrier();
    const bool tail = tok0 + AT2_BT > tend;  // (uniform) the split ends inside this block
    unsigned rk[R2M], rv[R2M];
    const unsigned* bk = sStage + cur * 2 * SWORDS;
    at2_read<R2M, MODE>(rv, bk + SWORDS, MODE == AT2_DIRECT ? vsh : offv[0], Bv, R2v, t32, h, SWORDS);
    if constexpr (!S16) at2_read<R2M, MODE>(rk, bk, MODE == AT2_DIRECT ? ksh : offk[0], Bk, R2k, t32, h, SWORDS);
#pragma unroll
    for (int st = 0; st < NST - 1; ++st) {
      offk[st] = offk[st + 1];
      offv[st] = offv[st + 1];
    }
    cur = cur == NST - 1 ? 0 : cur + 1;
    // ---- value records -> LDS rows [record byte][token quad][parity]
#pragma unroll
    for (int i = 0; i < R2M; ++i) {
      const u32x2 y = at2_quad_split(rv[i], sel1, sel_e, sel_o);
      const unsigned row = (unsigned)(4 * (i + h * R2M) + e4);
      const unsigned vo = at2_vrowo(R2M, OCC, row) + 2 * (t32 >> 2);
      if (STC_CHECK(vo + 2u <= (unsigned)VWORDS, DBG_ATT_VROW)) *reinterpret_cast<u32x2*>(sV + vo) = y;
    }
    // ---- scores: int8 MFMAs, A = weights (rows 4H + p), B = the record bits
    float su[NHL];  // unscaled scores of the lane's slots (-inf past the split)
    if constexpr (S16) {
      const lds_u8* aL = lds_ptr(abase);
      u32x4 av[4];
#pragma unroll
      for (int st = 0; st < 4; ++st) av[st] = LDS_AT(u32x4, aL + 64 * st);
      // token 16 G + c16: words 2 g4, 2 g4 + 1 of its record (chunk g4 >> 1,
      // staged at slot token + 32 (g4 >> 1))
      u32x2 kw[2];
      {
        unsigned ka = lds_offset(reinterpret_cast<unsigned char*>(const_cast<unsigned*>(bk))) +
                      4u * (4u * (unsigned)(c16 + 32 * (g4 >> 1)) + 2u * (unsigned)(g4 & 1));
        kw[0] = LDS_AT(u32x2, lds_ptr(ka));
        // (an opaque address: the two 8-byte reads stay separate; merged
        // into one two-address read they would conflict)
        asm volatile("" : "+v"(ka));
        kw[1] = LDS_AT(u32x2, lds_ptr(ka + 256u));
      }
#pragma unroll
      for (int G = 0; G < 2; ++G) {
        i32x4 a16 = (i32x4){0, 0, 0, 0};
#pragma unroll
        for (int st = 0; st < 4; ++st)
          a16 = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, av[st]),
                                                      __builtin_bit_cast(i32x4, at2_bits(kw[G][st >> 1], st & 1)), a16,
                                                      0, 0, 0);
        su[G] = at2_score(a16[0], a16[1], a16[2]);
        if (tail && tok0 + 16 * G + c16 >= tend) su[G] = -INFINITY;
      }
    } else {
      i32x16 acc;
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[e] = 0;
      const lds_u8* aL = lds_ptr(abase);
      // (all of the block's weight reads are issued first, so that their
      // latencies overlap; words past a half record meet zero weights)
      u32x4 av[2 * R2M];
#pragma unroll
      for (int e = 0; e < 2 * R2M; ++e) av[e] = LDS_AT(u32x4, aL + 16 * e);
#pragma unroll
      for (int i = 0; i < R2M; ++i) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
          acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, av[2 * i + kk]),
                                                      __builtin_bit_cast(i32x4, at2_bits(rk[i], kk)), acc, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < NHL; ++i) {
        su[i] = at2_score(acc[4 * i], acc[4 * i + 1], acc[4 * i + 2]);
      }
      if (tail) {  // (uniform) tokens past the split
#pragma unroll
        for (int i = 0; i < NHL; ++i)
          if (tok0 + t32 >= tend) su[i] = -INFINITY;
      }
    }
    bool slow = false;
#pragma unroll
    for (int i = 0; i < NHL; ++i) slow |= hval[i] && !(su[i] <= thr[i]);
    // ---- online softmax. A score above its head's max + 8 (log2 units)
    // raises the max first (rare once the max has settled): alpha =
    // 2^(m_old - m_new) rescales the value accumulators before P x V.
    if (__builtin_amdgcn_ballot_w64(slow) != 0) {
      float mx16 = 0.0f;
      if constexpr (S16) mx16 = row16_max(fmaxf(su[0], su[1]) * invS[0]);
#pragma unroll
      for (int i = 0; i < NHL; ++i) {
        const float mx = S16 ? mx16 : half_max(su[i] * invS[i]);
        const float mnew = fmaxf(mold[i], mx);
        // (no token of the head so far: max 0, every P and sum so far 0)
        const float mset = mnew == -INFINITY ? 0.0f : mnew;
        const float alpha = mold[i] == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(mold[i] - mset);
        // (a copy after the last use of the old max, which alpha's operand
        // makes it: the running max keeps one register through the loop,
        // with no moves on the fast path)
        asm volatile("v_mov_b32 %0, %1" : "=v"(mold[i]) : "v"(mset), "v"(alpha));
        thr[i] = (mset + 8.0f) / invS[i];
        if (S16 ? (c16 == 0 && i == 0) : t32 == 0) sAl[S16 ? g4 : 2 * i + h] = alpha;
      }
      resc = true;
    }
    // P (fp16) -> sP[octet][head][8]
#pragma unroll
    for (int i = 0; i < NHL; ++i) {
      const _Float16 ph = (_Float16)__builtin_amdgcn_exp2f(__builtin_fmaf(su[i], invS[i], -mold[i]));
      if constexpr (S16) {
        const unsigned ps = (unsigned)at2_pos(16 * i + c16);
        sP[(ps >> 3) * AT2_PST + g4 * 8 + (ps & 7)] = ph;
      } else {
        sP[(pos >> 3) * AT2_PST + (2 * i + h) * 8 + (pos & 7)] = ph;
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // the wave's value rows, P and alpha are in LDS
    __builtin_amdgcn_wave_barrier();
    // ---- rescale and accumulate P x V: heads 4 g4 + r, columns 16 T + c16
    {
      if (resc) {
        const f32x4 al = *reinterpret_cast<const f32x4*>(sAl + 4 * g4);
#pragma unroll
        for (int T = 0; T < NT; ++T)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc_v[T][r] *= al[r];
        // (every slow block writes the alphas of all the lanes' heads again;
        // those of other heads stay 1)
        resc = false;
      }
      const f16x8 pa = *reinterpret_cast<const f16x8*>(sP + g4 * AT2_PST + c16 * 8);  // 16 lanes: 64 banks
      u32x4 vv[NT];
#pragma unroll
      for (int T = 0; T < NT; ++T) vv[T] = LDS_AT(u32x4, lds_ptr(vaddr[T]));
#pragma unroll
      for (int T = 0; T < NT; ++T) {
        const unsigned m = vmask[T];
        const u32x4 vb = (u32x4){vv[T][0] & m, vv[T][1] & m, vv[T][2] & m, vv[T][3] & m};
        acc_v[T] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa, __builtin_bit_cast(f16x8, vb), acc_v[T], 0, 0, 0);
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the requests past the end have landed before LDS is reused
  // ---- merge the waves: scratch [wave][8 heads][CST]
  constexpr int CST = 16 * NT + 4;
  __syncthreads();
  float* red = reinterpret_cast<float*>(sReg0);
  float* part = reinterpret_cast<float*>(a.ws) + (p * a.n_splits + sp) * att_part_stride(g);
  const bool cols_ok = ncols < 16 * NT;  // (the launch chose NT from the states' column counts, plus the sum column)
  {
    float* mine = red + wave * 8 * CST;
#pragma unroll
    for (int i = 0; i < NHL; ++i) {
      if constexpr (S16) {
        if (c16 == 0 && i == 0) mine[g4 * CST + 16 * NT] = mold[0];
      } else {
        if (t32 == 0) mine[(2 * i + h) * CST + 16 * NT] = mold[i];
      }
    }
    if (g4 < 2) {
#pragma unroll
      for (int T = 0; T < NT; ++T)
#pragma unroll
        for (int r = 0; r < 4; ++r) mine[(4 * g4 + r) * CST + 16 * T + c16] = acc_v[T][r];
    }
  }
  __syncthreads();
  // the split's partial (acc, m, l) per head; with one split per pair
  // (direct), the mean codes, as the merge would form them from this one
  // partial (weight exp2(m - m) = 1; nothing merged for a split without
  // tokens)
  constexpr int NE = 8 * 128 / (64 * W);  // elements per thread at most
  float code[NE];
#pragma unroll
  for (int k = 0; k < NE; ++k) {
    const int e = tid + 64 * W * k;
    if (e >= g * 128) break;
    const int hh = e >> 7, jj = e & 127;
    const unsigned cc = sVch[jj];
    const int c0 = (int)(cc & 0xFFFFu), nc = (int)(cc >> 16);
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < W; ++w) M = fmaxf(M, red[(w * 8 + hh) * CST + 16 * NT]);
    float A = 0.0f, Ls = 0.0f;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const float* rw = red + (w * 8 + hh) * CST;
      const float mw = rw[16 * NT];
      const float f = (mw == -INFINITY) ? 0.0f : exp2f(mw - M);
      float v = 0.0f;
      for (int k2 = 0; k2 < nc; ++k2)
        if (c0 + k2 < 16 * NT) v += sFac[c0 + k2] * rw[c0 + k2];
      A += f * v;
      Ls += f * rw[ncols];  // (the sum column)
    }
    if (!cols_ok) A = __builtin_nanf("");
    if (a.direct) {
      code[k] = M == -INFINITY ? cmb_code(hv, jj, 0.0, 0.0) : cmb_code(hv, jj, (double)A, (double)Ls);
    } else {
      float* ph = part + hh * ATT_PART_FLOATS;
      ph[jj] = A;
      if (jj == 0) { ph[128] = M; ph[129] = Ls; }
    }
  }
  if (a.direct) {  // (uniform)
    static_assert((size_t)3 * 8 * 128 <= (size_t)W * 8 * CST, "mean codes and half sums fit the merge scratch");
    float* sC = red;            // [g][128] mean codes
    float* sQ = red + g * 128;  // [2][g][128] half sums
    __syncthreads();            // every thread is done reading the wave partials
#pragma unroll
    for (int k = 0; k < NE; ++k) {
      const int e = tid + 64 * W * k;
      if (e < g * 128) sC[e] = code[k];
    }
    __syncthreads();
    cmb_rotate(sC, sQ, vst, g, a.out + pg * g * 128, tid);
  }
}

// Partials area of stc_attend_compressed_batched_noalloc: a file-scope device
// array, one copy on every device the library runs on, held until the process
// ends. Host code uses the address hipGetSymbolAddress gives on the current
// device (looked up once per device), never the array's name. Calls that
// overlap on one device share it and race; the partials need no clearing
// (the main kernel writes every one the merge reads).
constexpr size_t ATT_SCRATCH_BYTES = (size_t)32 << 20;
static __device__ __align__(256) unsigned char scratch[ATT_SCRATCH_BYTES];

size_t attend_scratch_bytes() { return ATT_SCRATCH_BYTES; }

int attend_scratch(void** ptr) {
  static std::mutex mu;
  static void* per_device[64] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 1;
  std::lock_guard<std::mutex> lock(mu);
  if (!per_device[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return 1;
    per_device[dev] = p;
  }
  *ptr = per_device[dev];
  return 0;
}

template <int R2M, int NT, int NCH, int W, bool SWZ, bool G4>
static int at2_attr() {
  return hipFuncSetAttribute((const void*)k_att2<R2M, NT, NCH, W, SWZ, G4>, hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)at2_lds_bytes(R2M, NT, NCH, W, SWZ, G4)) != hipSuccess;
}
template <int R2M, int NT, int NCH, int W, bool SWZ, bool G4>
static void at2_launch(dim3 grid, hipStream_t s, const AttK& a) {
  static_assert(at2_lds_bytes(R2M, NT, NCH, W, SWZ, G4) * at2_occ(R2M, NCH, W, SWZ, G4) <= 160 * 1024, "k_att2 LDS");
  hipLaunchKernelGGL((k_att2<R2M, NT, NCH, W, SWZ, G4>), grid, dim3(64 * W), at2_lds_bytes(R2M, NT, NCH, W, SWZ, G4),
                     s, a);
}

typedef void (*AttKernel)(AttK);
// variant: [RHT+sketch, sketch, sketch >512, RHT, -, >512] x [stream, REC]
static const AttKernel kAttKernels[6][2] = {
    {k_att_main<8, true, true, false>, k_att_main<8, true, true, false>},
    {k_att_main<8, false, true, false>, k_att_main<8, false, true, true>},
    {k_att_main<16, false, true, false>, k_att_main<16, false, true, true>},
    {k_att_main<8, true, false, false>, k_att_main<8, true, false, false>},
    {k_att_main<8, false, false, false>, k_att_main<8, false, false, true>},
    {k_att_main<16, false, false, false>, k_att_main<16, false, false, true>},
};

int launch_attend(const AttendLaunch& L, void* stream) {
  if (!g_att_attr_done) {
    for (const auto& row : kAttKernels)
      for (AttKernel k : row)
        if (hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) !=
            hipSuccess)
          return 1;
    if (hipFuncSetAttribute((const void*)k_att_combine, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)cmb_lds_bytes(16)) != hipSuccess)
      return 1;
    if (at2_attr<4, 10, 1, 4, true, true>() || at2_attr<4, 10, 1, 4, true, false>() ||
        at2_attr<3, 8, 1, 4, false, false>() || at2_attr<4, 8, 1, 4, false, false>() ||
        at2_attr<4, 10, 1, 4, false, false>() ||
        at2_attr<4, 10, 1, 4, false, true>() || at2_attr<4, 10, 2, 8, false, false>() ||
        at2_attr<8, 12, 3, 8, false, false>())
      return 1;
    g_att_attr_done = true;
  }
  AttK a{};
  a.k_states = L.k_states;
  a.k_map = L.k_map;
  a.v_states = L.v_states;
  a.v_map = L.v_map;
  a.n_states = L.n_states;
  a.n_pairs = L.n_pairs;
  a.n_tokens = L.n_tokens;
  a.packed_stride = L.packed_stride;
  a.k_packed = L.k_packed;
  a.v_packed = L.v_packed;
  a.group = L.group;
  a.q = L.q;
  a.out = L.out;
  a.scale = L.scale;
  a.ws = L.ws;
  a.k_norms = L.k_norms;
  a.v_norms = L.v_norms;
  a.norms_stride = L.norms_stride;
  a.k_sketch = L.k_sketch;
  a.k_rnorm = L.k_rnorm;
  a.sketch_stride = L.sketch_stride;
  a.rnorm_stride = L.rnorm_stride;
  a.k_new = L.k_new;
  a.v_new = L.v_new;
  a.new_f32 = L.new_f32;
  a.stream_words = att_stream_words(L.max_bits);
  a.region_words = att_region_words(L.max_bits);
  const bool sketch = L.k_sketch != nullptr;
  const size_t fixed = ATT_FIXED_BYTES + (sketch ? 32 * AROW : 0);
  int waves = ATT_WAVES_MAX;
  while (waves > 12 && fixed + (size_t)waves * a.region_words * 4 > 160 * 1024) waves -= 4;
  // (records of at most 1024 bits always leave room for 12 waves; the
  // a-table build assumes 12 or 16)
  if (fixed + (size_t)waves * a.region_words * 4 > 160 * 1024) return 1;
  hipStream_t s = (hipStream_t)stream;
  // the packed-bit kernel's instance (-1: the older kernel): value columns
  // plus the sum column fit the tiles; token counts and stream bytes below
  // 2^31 for its 32-bit arithmetic
  const bool small = L.n_tokens < (1LL << 30) && L.n_tokens * (long long)L.max_bits / 8 < (1LL << 31) - 65536;
  int inst = -1;
  if (!sketch && !L.rht && L.group <= 8 && L.max_bits <= 512 && L.max_vcols <= 191 && small) {
    const bool g4 = L.group <= 4;
    if (L.max_bits <= 256 && L.att_chunks <= 1) {
      if (L.rec256) inst = g4 ? 0 : 1;
      else if (!g4 && L.max_vcols <= 127 && L.max_bits <= 192) inst = 2;
      else if (!g4 && L.max_vcols <= 127) inst = 3;
      else inst = g4 ? 4 : 5;
    } else {
      inst = L.max_bits <= 256 ? 6 : 7;
    }
  }
  static constexpr int kOcc[8] = {at2_occ(4, 1, 4, true, true),   at2_occ(4, 1, 4, true, false),
                                  at2_occ(3, 1, 4, false, false), at2_occ(4, 1, 4, false, false),
                                  at2_occ(4, 1, 4, false, true),  at2_occ(4, 1, 4, false, false),
                                  at2_occ(4, 2, 8, false, false), at2_occ(8, 3, 8, false, false)};
  // one round of workgroups: the CUs times the instance's workgroups per CU
  // (the older family: one per CU)
  const int64_t round = inst >= 0 ? (kOcc[inst] == 4 ? ATT_ROUNDS[2] : kOcc[inst] == 3 ? ATT_ROUNDS[1] : ATT_ROUNDS[0])
                                  : ATT_ROUNDS[0];
  for (long long c0 = 0; c0 < L.n_pairs; c0 += ATT_MAX_PAIRS) {
    const long long np = L.n_pairs - c0 < ATT_MAX_PAIRS ? L.n_pairs - c0 : ATT_MAX_PAIRS;
    a.pair_base = c0;
    a.n_pairs = np;
    a.split_tokens = att_split_tokens(np, L.n_tokens, round);
    a.n_splits = att_n_splits(np, L.n_tokens, round);
    const size_t att_lds = fixed + (size_t)waves * a.region_words * 4;
    const dim3 grid((unsigned)a.n_splits, (unsigned)np);
    a.direct = inst >= 0 && a.n_splits == 1;
    if (inst >= 0) {
      a.prep = reinterpret_cast<float*>(a.ws) + att_partial_floats(np, L.n_tokens, L.group, round);
      if (L.k_new && L.new_f32) hipLaunchKernelGGL(k_att_append, dim3((unsigned)np), dim3(128), 0, s, a);
      if (L.k_new && !L.new_f32) hipLaunchKernelGGL(k_att2_prep<true>, dim3((unsigned)np), dim3(128 * PREP_PARTS), 0, s, a);
      else hipLaunchKernelGGL(k_att2_prep<false>, dim3((unsigned)np), dim3(128 * PREP_PARTS), 0, s, a);
      switch (inst) {
        case 0: at2_launch<4, 10, 1, 4, true, true>(grid, s, a); break;
        case 1: at2_launch<4, 10, 1, 4, true, false>(grid, s, a); break;
        case 2: at2_launch<3, 8, 1, 4, false, false>(grid, s, a); break;
        case 3: at2_launch<4, 8, 1, 4, false, false>(grid, s, a); break;
        case 4: at2_launch<4, 10, 1, 4, false, true>(grid, s, a); break;
        case 5: at2_launch<4, 10, 1, 4, false, false>(grid, s, a); break;
        case 6: at2_launch<4, 10, 2, 8, false, false>(grid, s, a); break;
        default: at2_launch<8, 12, 3, 8, false, false>(grid, s, a); break;
      }
    } else {
      if (L.k_new) hipLaunchKernelGGL(k_att_append, dim3((unsigned)np), dim3(128), 0, s, a);
      const int var = sketch ? (L.rht ? 0 : (L.max_bits <= 512 ? 1 : 2)) : (L.rht ? 3 : (L.max_bits <= 512 ? 4 : 5));
      hipLaunchKernelGGL(kAttKernels[var][L.rec && !L.rht ? 1 : 0], grid, dim3(64 * waves), att_lds, s, a);
    }
    // the splits' partials -> out, once every split has written its own
    // (the packed-bit kernel with one split per pair has written out itself);
    // few pairs with many splits: a workgroup per (pair, query head), the
    // splits merged eight ways; else a workgroup per pair
    if (a.direct) continue;
    if (np <= 64 && a.n_splits >= 16)
      hipLaunchKernelGGL(k_att_combine_head, dim3((unsigned)np, (unsigned)L.group), dim3(CMBH_THREADS), 0, s, a);
    else
      hipLaunchKernelGGL(k_att_combine, dim3((unsigned)np), dim3(CMB_THREADS), cmb_lds_bytes(L.group), s, a);
  }
  return hipGetLastError() != hipSuccess;
}

}  // namespace stc
