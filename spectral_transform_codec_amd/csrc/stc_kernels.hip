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
//  - projection and reconstruction are dense 128-wide contractions on bf16
//    MFMA (v_mfma_f32_16x16x32_bf16). The basis is split into bf16 high and
//    low parts (two MFMA passes; three for fp32 tokens) so the fp32 result
//    carries ~16 significant bits of the basis, enough for code parity with
//    the fp64 definition. Codes are exact small integers in bf16.
//  - bit packing / unpacking run one token per lane with the per-channel
//    widths in scalar registers (uniform control flow), going through LDS to
//    change between the MFMA layouts and the token-per-lane layout, and to
//    turn the variable-length records into coalesced 128-bit HBM accesses.
//  - the Walsh-Hadamard butterfly runs in registers, one token per lane.
#include <hip/hip_runtime.h>

#include "stc_internal.h"

namespace stc {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr float LOG2E = 1.4426950408889634f;

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ long long packed_len(long long total_bits, long long n) {
  const long long nb = (n * total_bits + 7) / 8;
  return (nb + 15) / 16 * 16;
}

__device__ __forceinline__ long long state_index(const int32_t* map, long long s, long long n_states) {
  long long si = map ? (long long)map[s] : s;
  return si < 0 ? 0 : (si >= n_states ? n_states - 1 : si);
}

// Workgroup -> work mapping that keeps consecutive logical workgroups on one
// XCD (hardware dispatches blockIdx round-robin over the 8 XCDs), so the
// workgroups sharing a stream's basis share an L2.
__device__ __forceinline__ int xcd_logical(int b, int grid) {
  return (grid % 8 == 0) ? (b % 8) * (grid / 8) + b / 8 : b;
}

// 8 unsigned bytes -> 8 bf16 (exact: codes are integers < 256)
__device__ __forceinline__ bf16x8 bytes_to_bf16x8(u32x2 v) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (__bf16)(float)((v[i >> 2] >> (8 * (i & 3))) & 0xffu);
  return r;
}
__device__ __forceinline__ f16x8 bytes_to_f16x8(u32x2 v) {
  f16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (_Float16)(float)((v[i >> 2] >> (8 * (i & 3))) & 0xffu);
  return r;
}

// Widths (and the record offset) of the 64 channels [64h, 64h+64) of a state,
// forced into scalar registers: the pack/unpack loops branch on them, and a
// per-channel vector load there would serialise a cache round trip per channel.
struct HalfW {
  unsigned w[16];  // byte k of w[i] = width of channel 64h + 4i + k
  unsigned off;    // record bit offset of channel 64h
};
__device__ __forceinline__ HalfW load_half_widths(const DevHdr* hdr, int h) {
  HalfW r;
  const unsigned* bw = reinterpret_cast<const unsigned*>(hdr->bits) + 16 * h;
#pragma unroll
  for (int i = 0; i < 16; ++i) r.w[i] = __builtin_amdgcn_readfirstlane(bw[i]);
  r.off = __builtin_amdgcn_readfirstlane((unsigned)hdr->off[64 * h]);
  return r;
}
__device__ __forceinline__ int width_of(const HalfW& W, int jj) { return (W.w[jj >> 2] >> (8 * (jj & 3))) & 0xff; }

// OR a 32-bit record word into an LDS bit stream at bit (32*d + sh).
__device__ __forceinline__ void stage_or(unsigned* stage, unsigned d, unsigned sh, unsigned w) {
  atomicOr(&stage[d], w << sh);
  if (sh) atomicOr(&stage[d + 1], w >> (32u - sh));
}

// Exact code of a flagged element: the count of thresholds t_k <= c, found
// from the fast estimate q (off by at most one level) with two comparisons.
__device__ __noinline__ int quant_slow(float c, float inv, int lm1, int q, const float* thr) {
  if (c != c) return 0;
  if (inv == 0.0f) return c >= 0.0f ? lm1 : 0;  // zero step: every threshold is 0
  if (q > 0 && c < thr[q - 1]) return q - 1;
  if (q < lm1 && c >= thr[q]) return q + 1;
  return q;
}

// ======================================================================
// Second moment (calibration): one workgroup per stream, fp64 accumulation
// of exact fp32 products in token order. Thread (ti, tj) owns entries
// (ti + 16u, tj + 16v), so (a, b) and (b, a) see identical sums.
// ======================================================================
__global__ void __launch_bounds__(256) k_gram(const void* x, int dtype, long long ld, long long n, double* gram) {
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

int launch_gram(const void* x, int dtype, int64_t ld, int64_t n_calib, double* gram, void* stream) {
  hipLaunchKernelGGL(k_gram, dim3(1), dim3(256), 0, (hipStream_t)stream, x, dtype, (long long)ld,
                     (long long)n_calib, gram);
  return hipGetLastError() != hipSuccess;
}

// ======================================================================
// Encode (eigen / identity): project -> quantize -> pack.
// One persistent workgroup of 8 waves per CU; a tile is 256 tokens of one
// stream. Phase A: each wave projects 32 tokens onto the kept channels with
// MFMA (B operand = basis rows staged in LDS) and quantizes in the MFMA
// output layout (one channel per lane). Phase B: one token (half record) per
// lane packs its codes with the widths in scalar registers into an LDS bit
// stream. Phase C: the tile's bytes go to HBM as 128-bit stores.
// ======================================================================
constexpr int ENC_T = 256;
constexpr int ENC_THREADS = 512;
constexpr int UROW = 272;  // bytes per LDS basis row (256 + 16 pad against bank conflicts)
constexpr int CROW = 144;  // bytes per LDS code row (128 + 16 pad)
constexpr int STAGE_BYTES = 32 * 1024 + 64;
constexpr size_t ENC_LDS = 2 * 128 * UROW + ENC_T * CROW + STAGE_BYTES;

struct EncK {
  const unsigned char* states;
  const int32_t* map;
  long long n_states, n_tokens, ld, x_stride, packed_stride;
  const void* x;
  unsigned char* packed;
  long long tiles_per_stream, total_tiles, tiles_per_wg;
  int grid;
};

// MODE 0: bf16 tokens, 1: fp32 tokens, 2: fp32 latent coefficients [n][128].
template <int MODE>
__global__ void __launch_bounds__(ENC_THREADS, 1) k_encode_eigen(EncK a) {
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* sUhi = smem;
  unsigned char* sUlo = smem + 128 * UROW;
  unsigned char* sCode = smem + 2 * 128 * UROW;
  unsigned* sStage = reinterpret_cast<unsigned*>(smem + 2 * 128 * UROW + ENC_T * CROW);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, g4 = lane >> 4;
  const int lw = xcd_logical(blockIdx.x, a.grid);
  const long long t_begin = (long long)lw * a.tiles_per_wg;
  long long t_end = t_begin + a.tiles_per_wg;
  if (t_end > a.total_tiles) t_end = a.total_tiles;
  const long long n = a.n_tokens;

  for (int i = tid; i < STAGE_BYTES / 4; i += ENC_THREADS) sStage[i] = 0u;

  long long cur = -1;
  const DevHdr* hdr = nullptr;
  const float* thr = nullptr;
  float p_inv[8], p_yb[8];
  int p_lm1[8], p_tb[8];
  int nt_cnt = 0, B = 0;
  HalfW HW = {};

  for (long long tile = t_begin; tile < t_end; ++tile) {
    const long long s = tile / a.tiles_per_stream;
    const long long tt = tile - s * a.tiles_per_stream;
    if (s != cur) {
      cur = s;
      const unsigned char* st = a.states + (size_t)state_index(a.map, s, a.n_states) * STATE_BYTES;
      hdr = reinterpret_cast<const DevHdr*>(st + OFF_HDR);
      thr = reinterpret_cast<const float*>(st + OFF_THR);
      nt_cnt = hdr->nmax16 >> 4;
      B = hdr->total_bits;
      HW = load_half_widths(hdr, wave >> 2);
      __syncthreads();  // every wave is done with the previous basis
      if (MODE != 2) {
        const u32x4* ghi = reinterpret_cast<const u32x4*>(st + OFF_UT_HI);
        const u32x4* glo = reinterpret_cast<const u32x4*>(st + OFF_UT_LO);
        const int chunks = hdr->nmax16 * 16;
        for (int i = tid; i < chunks; i += ENC_THREADS) {
          const int row = i >> 4, c = i & 15;
          *reinterpret_cast<u32x4*>(sUhi + row * UROW + c * 16) = ghi[i];
          *reinterpret_cast<u32x4*>(sUlo + row * UROW + c * 16) = glo[i];
        }
      }
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        const int j = 16 * nt + r16;
        p_inv[nt] = hdr->inv_step[j];
        p_yb[nt] = hdr->ybias[j];
        p_lm1[nt] = hdr->lm1[j];
        p_tb[nt] = hdr->thr_base[j];
      }
      __syncthreads();
    }
    if (B == 0) continue;
    const long long tok0 = tt * ENC_T;

    // ---------------- phase A: project + quantize, codes -> LDS rows
    unsigned cw[2][2][4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < 4; ++r) cw[mt][h][r] = 0u;
    {
      bf16x8 ah[2][4], al[2][4];
      if (MODE != 2) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          long long tok = tok0 + 32 * wave + 16 * mt + r16;
          if (tok > n - 1) tok = n - 1;
          if (MODE == 0) {
            const unsigned short* row =
                static_cast<const unsigned short*>(a.x) + s * a.x_stride + tok * a.ld;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
              ah[mt][ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(row + 32 * ks + 8 * g4));
          } else {
            const float* row = static_cast<const float*>(a.x) + s * a.x_stride + tok * a.ld;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
              const f32x4 v0 = *reinterpret_cast<const f32x4*>(row + 32 * ks + 8 * g4);
              const f32x4 v1 = *reinterpret_cast<const f32x4*>(row + 32 * ks + 8 * g4 + 4);
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                const float f = e < 4 ? v0[e] : v1[e - 4];
                const __bf16 hi = (__bf16)f;
                ah[mt][ks][e] = hi;
                al[mt][ks][e] = (__bf16)(f - (float)hi);
              }
            }
          }
        }
      }
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        if (nt < nt_cnt) {
          f32x4 acc[2];
          if (MODE == 2) {
            const float* cf = static_cast<const float*>(a.x);
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                long long tok = tok0 + 32 * wave + 16 * mt + 4 * g4 + r;
                if (tok > n - 1) tok = n - 1;
                acc[mt][r] = cf[tok * 128 + 16 * nt + r16];
              }
          } else {
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) acc[mt] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
              const int off = (16 * nt + r16) * UROW + (32 * ks + 8 * g4) * 2;
              const bf16x8 bh = *reinterpret_cast<const bf16x8*>(sUhi + off);
              const bf16x8 bl = *reinterpret_cast<const bf16x8*>(sUlo + off);
#pragma unroll
              for (int mt = 0; mt < 2; ++mt) {
                acc[mt] = mfma_bf16(ah[mt][ks], bh, acc[mt]);
                acc[mt] = mfma_bf16(ah[mt][ks], bl, acc[mt]);
                if (MODE == 1) acc[mt] = mfma_bf16(al[mt][ks], bh, acc[mt]);
              }
            }
          }
          // Quantize. y = c/step + L/2 + EPS; away from integers floor(y) is
          // the exact threshold count (the fp32 error of y is < 2^-15 while
          // the guard band is 2^-13 wide); near an integer, or for NaN or a
          // zero step, the exact thresholds decide.
          const float inv = p_inv[nt], yb = p_yb[nt];
          const int lm1 = p_lm1[nt];
          int q[2][4];
          unsigned flags = 0u;
#pragma unroll
          for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float y = __builtin_fmaf(acc[mt][r], inv, yb);
              const float yc = fminf(fmaxf(y, -1.0f), 511.0f);
              int q0 = (int)floorf(yc);
              q0 = q0 < 0 ? 0 : (q0 > lm1 ? lm1 : q0);
              q[mt][r] = q0;
              const float fr = __builtin_amdgcn_fractf(y);
              if (!(fr >= QFLAG)) flags |= 1u << (4 * mt + r);
            }
          if (__any(flags != 0u)) {
            const float* tc = thr + p_tb[nt];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
              for (int r = 0; r < 4; ++r)
                if (flags & (1u << (4 * mt + r))) q[mt][r] = quant_slow(acc[mt][r], inv, lm1, q[mt][r], tc);
          }
#pragma unroll
          for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) cw[mt][nt >> 2][r] |= (unsigned)q[mt][r] << (8 * (nt & 3));
        }
      }
    }
    // code row of a token: dword (16h + c) holds channels 64h + 16k + c in byte k
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tl = 32 * wave + 16 * mt + 4 * g4 + r;
#pragma unroll
        for (int h = 0; h < 2; ++h)
          *reinterpret_cast<unsigned*>(sCode + tl * CROW + 4 * (16 * h + r16)) = cw[mt][h][r];
      }
    __syncthreads();

    // ---------------- phase B: pack (half a record per lane) into the LDS stream
    {
      const int h = wave >> 2;
      const int tl = 64 * (wave & 3) + lane;
      if (tok0 + tl < n) {
        unsigned c16[16];
        const unsigned* crow = reinterpret_cast<const unsigned*>(sCode + tl * CROW + 64 * h);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const u32x4 v = *reinterpret_cast<const u32x4*>(crow + 4 * i);
          c16[4 * i] = v[0]; c16[4 * i + 1] = v[1]; c16[4 * i + 2] = v[2]; c16[4 * i + 3] = v[3];
        }
        const unsigned S = (unsigned)tl * (unsigned)B + HW.off;
        const unsigned d0 = S >> 5, sh = S & 31u;
        unsigned acc = 0u, k = 0u;
        int pos = 0;
#pragma unroll
        for (int jj = 0; jj < 64; ++jj) {
          const int bw = width_of(HW, jj);
          if (bw) {
            const unsigned code = (c16[jj & 15] >> (8 * (jj >> 4))) & 0xffu;
            acc |= code << pos;
            if (pos + bw >= 32) {
              stage_or(sStage, d0 + k, sh, acc);
              ++k;
              acc = code >> (32 - pos);
              pos += bw - 32;
            } else {
              pos += bw;
            }
          }
        }
        if (pos > 0) stage_or(sStage, d0 + k, sh, acc);
      }
    }
    __syncthreads();

    // ---------------- phase C: tile bytes -> HBM, then clear the stage
    {
      const long long P = packed_len(B, n);
      const long long start = tt * 32LL * B;
      long long nb = 32LL * B;
      if (nb > P - start) nb = P - start;
      u32x4* dst = reinterpret_cast<u32x4*>(a.packed + s * a.packed_stride + start);
      u32x4* src = reinterpret_cast<u32x4*>(sStage);
      const int nchunk = (int)(nb >> 4);
      for (int i = tid; i < nchunk; i += ENC_THREADS) dst[i] = src[i];
      const int zchunk = 2 * B + 1;
      for (int i = tid; i < zchunk; i += ENC_THREADS) src[i] = (u32x4){0u, 0u, 0u, 0u};
    }
    __syncthreads();
  }
}

static bool g_enc_attr_done = false, g_dec_attr_done = false, g_att_attr_done = false;

int launch_encode_eigen(const EncodeLaunch& L, void* stream) {
  if (!g_enc_attr_done) {
    (void)hipFuncSetAttribute((const void*)k_encode_eigen<0>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)ENC_LDS);
    (void)hipFuncSetAttribute((const void*)k_encode_eigen<1>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)ENC_LDS);
    (void)hipFuncSetAttribute((const void*)k_encode_eigen<2>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)ENC_LDS);
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
  a.tiles_per_stream = (L.n_tokens + ENC_T - 1) / ENC_T;
  a.total_tiles = a.tiles_per_stream * L.n_streams;
  int dev = 0, cus = 256;
  (void)hipGetDevice(&dev);
  (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  long long grid = a.total_tiles < cus ? a.total_tiles : cus;
  a.tiles_per_wg = (a.total_tiles + grid - 1) / grid;
  grid = (a.total_tiles + a.tiles_per_wg - 1) / a.tiles_per_wg;
  a.grid = (int)grid;
  hipStream_t s = (hipStream_t)stream;
  if (L.mode == 0) hipLaunchKernelGGL(k_encode_eigen<0>, dim3(grid), dim3(ENC_THREADS), ENC_LDS, s, a);
  else if (L.mode == 1) hipLaunchKernelGGL(k_encode_eigen<1>, dim3(grid), dim3(ENC_THREADS), ENC_LDS, s, a);
  else hipLaunchKernelGGL(k_encode_eigen<2>, dim3(grid), dim3(ENC_THREADS), ENC_LDS, s, a);
  return hipGetLastError() != hipSuccess;
}

// ======================================================================
// Decode (eigen / identity): unpack -> MFMA with W = U diag(step) -> bias.
// x_hat_i = sum_j W_ij q_j - bias_i,  bias_i = sum_j W_ij (L_j - 1)/2,
// i.e. sum_j U_ij step_j (q_j - (L_j - 1)/2) with q the raw codes.
// Phase A: the tile's packed bytes -> LDS. Phase B: one half record per lane
// unpacks codes (uniform widths) to LDS rows. Phase C: each wave rebuilds 32
// tokens x 128 dims (A = W rows from LDS, B = codes), then stores bf16/fp32.
// ======================================================================
constexpr int DEC_T = 256;
constexpr int DEC_THREADS = 512;
constexpr int PK_BYTES = 32 * 1024 + 64;
constexpr size_t DEC_LDS = 2 * 128 * UROW + DEC_T * CROW + PK_BYTES;

struct DecK {
  const unsigned char* states;
  const int32_t* map;
  long long n_states, n_tokens, ld, x_stride, packed_stride;
  const unsigned char* packed;
  void* x;
  long long tiles_per_stream, total_tiles, tiles_per_wg;
  int grid;
};

// Unpack the 64 codes of channels [64h, 64h+64) of token tl from the LDS
// stream `P32` (bit 0 = first bit of the tile) into 16 dwords, natural order.
__device__ __forceinline__ void unpack_half(const unsigned* P32, const HalfW& W, unsigned tl, int B,
                                            unsigned cw[16]) {
#pragma unroll
  for (int i = 0; i < 16; ++i) cw[i] = 0u;
  const unsigned S = tl * (unsigned)B + W.off;
  const unsigned d0 = S >> 5, sh = S & 31u;
  const unsigned r0 = P32[d0], r1 = P32[d0 + 1], r2 = P32[d0 + 2];
  unsigned cur = __builtin_amdgcn_alignbit(r1, r0, sh);
  unsigned nxt = __builtin_amdgcn_alignbit(r2, r1, sh);
  unsigned raw = r2, k = d0 + 3;
  int pos = 0;
#pragma unroll
  for (int jj = 0; jj < 64; ++jj) {
    // bits [pos, pos + bw) of the 64-bit window nxt:cur (bw = 0 gives 0)
    const int bw = width_of(W, jj);
    const unsigned code = __builtin_amdgcn_ubfe(__builtin_amdgcn_alignbit(nxt, cur, (unsigned)pos), 0u, (unsigned)bw);
    cw[jj >> 2] |= code << (8 * (jj & 3));
    pos += bw;
    if (pos >= 32) {
      pos -= 32;
      cur = nxt;
      const unsigned rn = P32[k++];
      nxt = __builtin_amdgcn_alignbit(rn, raw, sh);
      raw = rn;
    }
  }
}

template <int F32OUT>
__global__ void __launch_bounds__(DEC_THREADS, 1) k_decode_eigen(DecK a) {
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* sWhi = smem;
  unsigned char* sWlo = smem + 128 * UROW;
  unsigned char* sCode = smem + 2 * 128 * UROW;
  unsigned* sPk = reinterpret_cast<unsigned*>(smem + 2 * 128 * UROW + DEC_T * CROW);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, g4 = lane >> 4;
  const int lw = xcd_logical(blockIdx.x, a.grid);
  const long long t_begin = (long long)lw * a.tiles_per_wg;
  long long t_end = t_begin + a.tiles_per_wg;
  if (t_end > a.total_tiles) t_end = a.total_tiles;
  const long long n = a.n_tokens;

  long long cur = -1;
  const DevHdr* hdr = nullptr;
  int ks_cnt = 0, B = 0;
  HalfW HW = {};

  for (long long tile = t_begin; tile < t_end; ++tile) {
    const long long s = tile / a.tiles_per_stream;
    const long long tt = tile - s * a.tiles_per_stream;
    if (s != cur) {
      cur = s;
      const unsigned char* st = a.states + (size_t)state_index(a.map, s, a.n_states) * STATE_BYTES;
      hdr = reinterpret_cast<const DevHdr*>(st + OFF_HDR);
      ks_cnt = hdr->kmax32 >> 5;
      B = hdr->total_bits;
      HW = load_half_widths(hdr, wave >> 2);
      __syncthreads();
      const u32x4* ghi = reinterpret_cast<const u32x4*>(st + OFF_W_HI);
      const u32x4* glo = reinterpret_cast<const u32x4*>(st + OFF_W_LO);
      const int cpr = hdr->kmax32 / 8;  // 16-byte chunks per row used
      for (int i = tid; i < 128 * cpr; i += DEC_THREADS) {
        const int row = i / cpr, c = i - row * cpr;
        *reinterpret_cast<u32x4*>(sWhi + row * UROW + c * 16) = ghi[row * 16 + c];
        *reinterpret_cast<u32x4*>(sWlo + row * UROW + c * 16) = glo[row * 16 + c];
      }
      __syncthreads();
    }
    const long long tok0 = tt * DEC_T;
    // ---------------- phase A: packed tile -> LDS
    {
      const long long P = packed_len(B, n);
      const long long start = tt * 32LL * B;
      long long nb = 32LL * B;
      if (nb > P - start) nb = P - start;
      const u32x4* src = reinterpret_cast<const u32x4*>(a.packed + s * a.packed_stride + start);
      u32x4* dst = reinterpret_cast<u32x4*>(sPk);
      const int nchunk = (int)(nb >> 4);
      const int zend = 2 * B + 2;
      for (int i = tid; i < zend; i += DEC_THREADS) dst[i] = i < nchunk ? src[i] : (u32x4){0u, 0u, 0u, 0u};
    }
    __syncthreads();
    // ---------------- phase B: unpack to code rows (natural channel order)
    {
      const int h = wave >> 2;
      const int tl = 64 * (wave & 3) + lane;
      unsigned cw[16];
      if (tok0 + tl < n && B > 0) {
        unpack_half(sPk, HW, (unsigned)tl, B, cw);
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) cw[i] = 0u;
      }
      u32x4* crow = reinterpret_cast<u32x4*>(sCode + tl * CROW + 64 * h);
#pragma unroll
      for (int i = 0; i < 4; ++i) crow[i] = (u32x4){cw[4 * i], cw[4 * i + 1], cw[4 * i + 2], cw[4 * i + 3]};
    }
    __syncthreads();
    // ---------------- phase C: MFMA reconstruction + store
    {
      bf16x8 bfr[2][4];
#pragma unroll
      for (int nt2 = 0; nt2 < 2; ++nt2)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          if (ks < ks_cnt) {
            const u32x2 v = *reinterpret_cast<const u32x2*>(sCode + (32 * wave + 16 * nt2 + r16) * CROW + 32 * ks + 8 * g4);
            bfr[nt2][ks] = bytes_to_bf16x8(v);
          }
        }
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        f32x4 acc[2][2];
#pragma unroll
        for (int sI = 0; sI < 2; ++sI)
#pragma unroll
          for (int nt2 = 0; nt2 < 2; ++nt2) acc[sI][nt2] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int sI = 0; sI < 2; ++sI) {
          const int mt = 2 * p + sI;
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            if (ks < ks_cnt) {
              const int off = (16 * mt + r16) * UROW + (32 * ks + 8 * g4) * 2;
              const bf16x8 wh = *reinterpret_cast<const bf16x8*>(sWhi + off);
              const bf16x8 wl = *reinterpret_cast<const bf16x8*>(sWlo + off);
#pragma unroll
              for (int nt2 = 0; nt2 < 2; ++nt2) {
                acc[sI][nt2] = mfma_bf16(wh, bfr[nt2][ks], acc[sI][nt2]);
                acc[sI][nt2] = mfma_bf16(wl, bfr[nt2][ks], acc[sI][nt2]);
              }
            }
          }
        }
        const int dbase = 32 * p + 8 * g4;
        const f32x4 b0 = *reinterpret_cast<const f32x4*>(hdr->bias + dbase);
        const f32x4 b1 = *reinterpret_cast<const f32x4*>(hdr->bias + dbase + 4);
#pragma unroll
        for (int nt2 = 0; nt2 < 2; ++nt2) {
          const long long tok = tok0 + 32 * wave + 16 * nt2 + r16;
          if (tok < n) {
            float v[8];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              v[r] = acc[0][nt2][r] - b0[r];
              v[4 + r] = acc[1][nt2][r] - b1[r];
            }
            if (F32OUT) {
              float* o = static_cast<float*>(a.x) + s * a.x_stride + tok * a.ld + dbase;
              *reinterpret_cast<f32x4*>(o) = (f32x4){v[0], v[1], v[2], v[3]};
              *reinterpret_cast<f32x4*>(o + 4) = (f32x4){v[4], v[5], v[6], v[7]};
            } else {
              unsigned short* o = static_cast<unsigned short*>(a.x) + s * a.x_stride + tok * a.ld + dbase;
              u32x4 w;
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const unsigned lo = __builtin_bit_cast(unsigned short, (__bf16)v[2 * e]);
                const unsigned hi = __builtin_bit_cast(unsigned short, (__bf16)v[2 * e + 1]);
                w[e] = lo | (hi << 16);
              }
              *reinterpret_cast<u32x4*>(o) = w;
            }
          }
        }
      }
    }
    __syncthreads();
  }
}

int launch_decode_eigen(const DecodeLaunch& L, void* stream) {
  if (!g_dec_attr_done) {
    (void)hipFuncSetAttribute((const void*)k_decode_eigen<0>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)DEC_LDS);
    (void)hipFuncSetAttribute((const void*)k_decode_eigen<1>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)DEC_LDS);
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
  a.tiles_per_stream = (L.n_tokens + DEC_T - 1) / DEC_T;
  a.total_tiles = a.tiles_per_stream * L.n_streams;
  int dev = 0, cus = 256;
  (void)hipGetDevice(&dev);
  (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  long long grid = a.total_tiles < cus ? a.total_tiles : cus;
  a.tiles_per_wg = (a.total_tiles + grid - 1) / grid;
  grid = (a.total_tiles + a.tiles_per_wg - 1) / a.tiles_per_wg;
  a.grid = (int)grid;
  hipStream_t s = (hipStream_t)stream;
  if (L.f32out) hipLaunchKernelGGL(k_decode_eigen<1>, dim3(grid), dim3(DEC_THREADS), DEC_LDS, s, a);
  else hipLaunchKernelGGL(k_decode_eigen<0>, dim3(grid), dim3(DEC_THREADS), DEC_LDS, s, a);
  return hipGetLastError() != hipSuccess;
}

// ======================================================================
// Walsh-Hadamard path: one token per lane, the 128 values in registers.
// Encode: signs -> norm -> FWHT butterflies -> scale by 1/(|x| sqrt(d)) ->
// 3-bit codebook cell (count of midpoint thresholds <= y) -> 48-byte record.
// Decode: codebook values -> FWHT -> scale by |x|/sqrt(d) -> signs.
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

__global__ void __launch_bounds__(256) k_rht_encode(RhtK a) {
  const long long s = blockIdx.y;
  const long long tok = (long long)blockIdx.x * 256 + threadIdx.x;
  if (tok >= a.n_tokens) return;
  const DevHdr* hdr =
      reinterpret_cast<const DevHdr*>(a.states + (size_t)state_index(a.map, s, a.n_states) * STATE_BYTES);
  const unsigned short* row = static_cast<const unsigned short*>(a.x) + s * a.x_stride + tok * a.ld;
  float v[128];
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(row + 8 * c);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[8 * c + 2 * e] = __uint_as_float(w[e] << 16);
      v[8 * c + 2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
    }
  }
  float ss = 0.0f;
#pragma unroll
  for (int i = 0; i < 128; ++i) {
    v[i] *= hdr->sign[i];
    ss = __builtin_fmaf(v[i], v[i], ss);
  }
  fwht128(v);
  const float nu = sqrtf(ss);
  const float inv = nu > 0.0f ? 1.0f / (nu * 11.313708498984761f) : 0.0f;
  float t[7];
#pragma unroll
  for (int k = 0; k < 7; ++k) t[k] = hdr->cb_thr[k];
  unsigned w[12];
#pragma unroll
  for (int i = 0; i < 12; ++i) w[i] = 0u;
#pragma unroll
  for (int i = 0; i < 128; ++i) {
    const float y = v[i] * inv;
    unsigned q = 0;
#pragma unroll
    for (int k = 0; k < 7; ++k) q += (y >= t[k]) ? 1u : 0u;
    const int bp = 3 * i;
    w[bp >> 5] |= q << (bp & 31);
    if ((bp & 31) > 29) w[(bp >> 5) + 1] |= q >> (32 - (bp & 31));
  }
  u32x4* dst = reinterpret_cast<u32x4*>(a.packed + s * a.packed_stride + tok * 48);
  dst[0] = (u32x4){w[0], w[1], w[2], w[3]};
  dst[1] = (u32x4){w[4], w[5], w[6], w[7]};
  dst[2] = (u32x4){w[8], w[9], w[10], w[11]};
  a.norms[s * a.n_tokens + tok] = nu;
}

__global__ void __launch_bounds__(256) k_rht_decode(RhtK a) {
  __shared__ float scb[8];
  const long long s = blockIdx.y;
  const DevHdr* hdr =
      reinterpret_cast<const DevHdr*>(a.states + (size_t)state_index(a.map, s, a.n_states) * STATE_BYTES);
  if (threadIdx.x < 8) scb[threadIdx.x] = hdr->cb[threadIdx.x];
  __syncthreads();
  const long long tok = (long long)blockIdx.x * 256 + threadIdx.x;
  if (tok >= a.n_tokens) return;
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
  if (a.f32out) {
    float* o = static_cast<float*>(a.xo) + s * a.x_stride + tok * a.ld;
#pragma unroll
    for (int c = 0; c < 32; ++c)
      *reinterpret_cast<f32x4*>(o + 4 * c) =
          (f32x4){v[4 * c] * m * hdr->sign[4 * c], v[4 * c + 1] * m * hdr->sign[4 * c + 1],
                  v[4 * c + 2] * m * hdr->sign[4 * c + 2], v[4 * c + 3] * m * hdr->sign[4 * c + 3]};
  } else {
    unsigned short* o = static_cast<unsigned short*>(a.xo) + s * a.x_stride + tok * a.ld;
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      u32x4 pk;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 8 * c + 2 * e;
        const unsigned lo = __builtin_bit_cast(unsigned short, (__bf16)(v[i] * m * hdr->sign[i]));
        const unsigned hi = __builtin_bit_cast(unsigned short, (__bf16)(v[i + 1] * m * hdr->sign[i + 1]));
        pk[e] = lo | (hi << 16);
      }
      *reinterpret_cast<u32x4*>(o + 8 * c) = pk;
    }
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
  dim3 grid((unsigned)((L.n_tokens + 255) / 256), (unsigned)L.n_streams);
  hipLaunchKernelGGL(k_rht_encode, grid, dim3(256), 0, (hipStream_t)stream, a);
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
  dim3 grid((unsigned)((L.n_tokens + 255) / 256), (unsigned)L.n_streams);
  hipLaunchKernelGGL(k_rht_decode, grid, dim3(256), 0, (hipStream_t)stream, a);
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
//  k_att_prologue: a -> bf16 hi/lo table per pair.
//  k_att_main: one workgroup per (split, pair); 256-token tiles; K and V
//   records unpacked one token per lane into LDS; scores = MFMA(a, K codes);
//   online softmax per wave; P (fp16) x V codes (fp16) on MFMA.
//  k_att_combine: merge splits, dequantize, rotate back (fp64).
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
};

__global__ void __launch_bounds__(256) k_att_prologue(AttK a) {
  const long long p = blockIdx.x;
  const unsigned char* st = a.k_states + (size_t)state_index(a.k_map, p, a.n_states) * STATE_BYTES;
  const DevHdr* hk = reinterpret_cast<const DevHdr*>(st);
  const float* u = reinterpret_cast<const float*>(st + OFF_U32);
  const float* q = a.q + p * a.group * 128;
  unsigned short* tab = reinterpret_cast<unsigned short*>(a.ws + p * ATT_QTAB_BYTES);
  for (int e = threadIdx.x; e < 16 * 128; e += 256) {
    const int h = e >> 7, j = e & 127;
    float val = 0.0f;
    if (h < a.group && hk->bits[j] > 0) {
      float acc = 0.0f;
      for (int i = 0; i < 128; ++i) acc = __builtin_fmaf(u[i * 128 + j], q[h * 128 + i], acc);
      val = acc * hk->step32[j] * a.scale * LOG2E;
    }
    const __bf16 hi = (__bf16)val;
    const __bf16 lo = (__bf16)(val - (float)hi);
    tab[e] = __builtin_bit_cast(unsigned short, hi);
    tab[16 * 128 + e] = __builtin_bit_cast(unsigned short, lo);
  }
}

constexpr int ATT_THREADS = 256;
constexpr int AKP = 32 * 1024 + 64;     // packed K tile bytes (max)
constexpr int VCROW = ATT_TILE + 16;    // bytes per LDS row of transposed V codes
constexpr int PROW = 72;                // fp16 per LDS row of P (64 tokens + pad)
constexpr size_t ATT_LDS = 2 * (size_t)AKP + ATT_TILE * CROW + 128 * VCROW + 4 * 16 * PROW * 2;

__device__ __forceinline__ float grp16_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 1));
  v = fmaxf(v, __shfl_xor(v, 2));
  v = fmaxf(v, __shfl_xor(v, 4));
  v = fmaxf(v, __shfl_xor(v, 8));
  return v;
}
__device__ __forceinline__ float grp16_sum(float v) {
  v += __shfl_xor(v, 1);
  v += __shfl_xor(v, 2);
  v += __shfl_xor(v, 4);
  v += __shfl_xor(v, 8);
  return v;
}

__device__ __forceinline__ void load_tile_bytes(const unsigned char* src_stream, long long total_bits, long long n,
                                                long long tt, unsigned* dst32, int tid, int nthreads) {
  const long long P = packed_len(total_bits, n);
  const long long start = tt * 32LL * total_bits;
  long long nb = 32LL * total_bits;
  if (nb > P - start) nb = P - start;
  const u32x4* src = reinterpret_cast<const u32x4*>(src_stream + start);
  u32x4* dst = reinterpret_cast<u32x4*>(dst32);
  const int nchunk = (int)(nb >> 4);
  const int zend = (int)(2 * total_bits + 2);
  for (int i = tid; i < zend; i += nthreads) dst[i] = i < nchunk ? src[i] : (u32x4){0u, 0u, 0u, 0u};
}

__global__ void __launch_bounds__(ATT_THREADS, 1) k_att_main(AttK a) {
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned* sKp = reinterpret_cast<unsigned*>(smem);
  unsigned* sVp = reinterpret_cast<unsigned*>(smem + AKP);
  unsigned char* sKc = smem + 2 * AKP;
  unsigned char* sVc = sKc + ATT_TILE * CROW;
  _Float16* sP = reinterpret_cast<_Float16*>(sVc + 128 * VCROW);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, g4 = lane >> 4;
  const long long sp = blockIdx.x, p = blockIdx.y;
  const long long n = a.n_tokens;
  const unsigned char* kst = a.k_states + (size_t)state_index(a.k_map, p, a.n_states) * STATE_BYTES;
  const unsigned char* vst = a.v_states + (size_t)state_index(a.v_map, p, a.n_states) * STATE_BYTES;
  const DevHdr* hk = reinterpret_cast<const DevHdr*>(kst);
  const DevHdr* hv = reinterpret_cast<const DevHdr*>(vst);
  const int Bk = hk->total_bits, Bv = hv->total_bits;
  const int ksK = hk->kmax32 >> 5;
  const int ntV = hv->nmax16 >> 4;
  const unsigned char* kpk = a.k_packed + p * a.packed_stride;
  const unsigned char* vpk = a.v_packed + p * a.packed_stride;
  const HalfW KW0 = load_half_widths(hk, 0), KW1 = load_half_widths(hk, 1);
  const HalfW VW0 = load_half_widths(hv, 0), VW1 = load_half_widths(hv, 1);

  // score A operand: a (bf16 hi/lo), rows = query heads (padded to 16)
  bf16x8 ahi[4], alo[4];
  {
    const unsigned short* tab = reinterpret_cast<const unsigned short*>(a.ws + p * ATT_QTAB_BYTES);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      ahi[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(tab + r16 * 128 + 32 * ks + 8 * g4));
      alo[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(tab + 2048 + r16 * 128 + 32 * ks + 8 * g4));
    }
  }
  float m_run[4], l_run[4];
  f32x4 acc_o[8];
#pragma unroll
  for (int r = 0; r < 4; ++r) { m_run[r] = -INFINITY; l_run[r] = 0.0f; }
#pragma unroll
  for (int i = 0; i < 8; ++i) acc_o[i] = (f32x4){0.f, 0.f, 0.f, 0.f};

  const long long t_begin = sp * a.split_tokens;
  long long t_end = t_begin + a.split_tokens;
  if (t_end > n) t_end = n;

  for (long long tok0 = t_begin; tok0 < t_end; tok0 += ATT_TILE) {
    const long long tt = tok0 / ATT_TILE;
    if (Bk > 0) load_tile_bytes(kpk, Bk, n, tt, sKp, tid, ATT_THREADS);
    if (Bv > 0) load_tile_bytes(vpk, Bv, n, tt, sVp, tid, ATT_THREADS);
    __syncthreads();
    // unpack one token per thread
    {
      const int tl = tid;
      const bool valid = tok0 + tl < t_end;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        unsigned cw[16];
        if (valid && Bk > 0) unpack_half(sKp, h ? KW1 : KW0, (unsigned)tl, Bk, cw);
        else {
#pragma unroll
          for (int i = 0; i < 16; ++i) cw[i] = 0u;
        }
        u32x4* krow = reinterpret_cast<u32x4*>(sKc + tl * CROW + 64 * h);
#pragma unroll
        for (int i = 0; i < 4; ++i) krow[i] = (u32x4){cw[4 * i], cw[4 * i + 1], cw[4 * i + 2], cw[4 * i + 3]};
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        unsigned cw[16];
        if (valid && Bv > 0) unpack_half(sVp, h ? VW1 : VW0, (unsigned)tl, Bv, cw);
        else {
#pragma unroll
          for (int i = 0; i < 16; ++i) cw[i] = 0u;
        }
#pragma unroll
        for (int jj = 0; jj < 64; ++jj) sVc[(64 * h + jj) * VCROW + tl] = (unsigned char)((cw[jj >> 2] >> (8 * (jj & 3))) & 0xffu);
      }
    }
    __syncthreads();
    // scores for this wave's 64 tokens
    f32x4 sc[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      sc[nt] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        if (ks < ksK) {
          const u32x2 v = *reinterpret_cast<const u32x2*>(sKc + (64 * wave + 16 * nt + r16) * CROW + 32 * ks + 8 * g4);
          const bf16x8 b = bytes_to_bf16x8(v);
          sc[nt] = mfma_bf16(ahi[ks], b, sc[nt]);
          sc[nt] = mfma_bf16(alo[ks], b, sc[nt]);
        }
      }
      const long long tok = tok0 + 64 * wave + 16 * nt + r16;
      if (tok >= t_end) sc[nt] = (f32x4){-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    }
    // online softmax (per wave); lane rows are heads 4*g4 + r
    _Float16* myP = sP + wave * 16 * PROW;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float mt = fmaxf(fmaxf(sc[0][r], sc[1][r]), fmaxf(sc[2][r], sc[3][r]));
      mt = grp16_max(mt);
      const float mnew = fmaxf(m_run[r], mt);
      const float alpha = (mnew == -INFINITY) ? 1.0f : exp2f(m_run[r] - mnew);
      float ls = 0.0f;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const float pv = (mnew == -INFINITY) ? 0.0f : exp2f(sc[nt][r] - mnew);
        const _Float16 ph = (_Float16)pv;
        ls += (float)ph;
        myP[(4 * g4 + r) * PROW + 16 * nt + r16] = ph;
      }
      l_run[r] = l_run[r] * alpha + ls;
      m_run[r] = mnew;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc_o[i][r] *= alpha;
    }
    __syncthreads();
    // P x V codes
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2) {
      const f16x8 pa = *reinterpret_cast<const f16x8*>(myP + r16 * PROW + 32 * ks2 + 8 * g4);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (i < ntV) {
          const u32x2 v = *reinterpret_cast<const u32x2*>(sVc + (16 * i + r16) * VCROW + 64 * wave + 32 * ks2 + 8 * g4);
          acc_o[i] = mfma_f16(pa, bytes_to_f16x8(v), acc_o[i]);
        }
      }
    }
    __syncthreads();
  }
  // merge the four waves: reuse the K code rows as scratch
  float* red = reinterpret_cast<float*>(sKc);  // [4 waves][16 heads][130]
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float lsum = grp16_sum(l_run[r]);
    const int hrow = 4 * g4 + r;
    float* base = red + (wave * 16 + hrow) * ATT_PART_FLOATS;
#pragma unroll
    for (int i = 0; i < 8; ++i) base[16 * i + r16] = acc_o[i][r];
    if (r16 == 0) { base[128] = m_run[r]; base[129] = lsum; }
  }
  __syncthreads();
  float* part = reinterpret_cast<float*>(a.ws + a.n_pairs * ATT_QTAB_BYTES) +
                ((p * a.n_splits + sp) * a.group) * ATT_PART_FLOATS;
  for (int e = tid; e < a.group * 128; e += ATT_THREADS) {
    const int h = e >> 7, j = e & 127;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, red[(w * 16 + h) * ATT_PART_FLOATS + 128]);
    float A = 0.0f, Ls = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = red[(w * 16 + h) * ATT_PART_FLOATS + 128];
      const float f = (mw == -INFINITY) ? 0.0f : exp2f(mw - M);
      A += f * red[(w * 16 + h) * ATT_PART_FLOATS + j];
      Ls += f * red[(w * 16 + h) * ATT_PART_FLOATS + 129];
    }
    part[h * ATT_PART_FLOATS + j] = A;
    if (j == 0) { part[h * ATT_PART_FLOATS + 128] = M; part[h * ATT_PART_FLOATS + 129] = Ls; }
  }
}

// One workgroup per (pair, query head): merge the splits' (acc, m, l) with
// log-sum-exp weights (fp32 weights, fp64 sums), take the softmax-weighted
// mean code of every V channel, dequantize it and rotate back with U_V.
__global__ void __launch_bounds__(128) k_att_combine(AttK a) {
  __shared__ float chat[128];
  const long long p = blockIdx.x / a.group;
  const int h = (int)(blockIdx.x - p * a.group);
  const int j = threadIdx.x;
  const unsigned char* vst = a.v_states + (size_t)state_index(a.v_map, p, a.n_states) * STATE_BYTES;
  const DevHdr* hv = reinterpret_cast<const DevHdr*>(vst);
  const float* u = reinterpret_cast<const float*>(vst + OFF_U32);
  const float* ps0 = reinterpret_cast<const float*>(a.ws + a.n_pairs * ATT_QTAB_BYTES) +
                     ((p * a.n_splits) * a.group + h) * ATT_PART_FLOATS;
  const long long sstride = (long long)a.group * ATT_PART_FLOATS;
  float M = -INFINITY;
  for (long long s = 0; s < a.n_splits; ++s) M = fmaxf(M, ps0[s * sstride + 128]);
  double A = 0.0, L = 0.0;
  for (long long s = 0; s < a.n_splits; ++s) {
    const float* ps = ps0 + s * sstride;
    const float ms = ps[128];
    const float f = (ms == -INFINITY) ? 0.0f : exp2f(ms - M);
    A += (double)(f * ps[j]);
    L += (double)(f * ps[129]);
  }
  chat[j] = hv->bits[j] ? (float)((double)hv->step32[j] * (A / L - (double)hv->halfspan[j])) : 0.0f;
  __syncthreads();
  float o = 0.0f;
#pragma unroll 8
  for (int k = 0; k < 128; ++k) o = __builtin_fmaf(u[j * 128 + k], chat[k], o);
  a.out[(p * a.group + h) * 128 + j] = o;
}

int launch_attend(const AttendLaunch& L, void* stream) {
  if (!g_att_attr_done) {
    (void)hipFuncSetAttribute((const void*)k_att_main, hipFuncAttributeMaxDynamicSharedMemorySize, (int)ATT_LDS);
    g_att_attr_done = true;
  }
  AttK a;
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
  a.split_tokens = att_split_tokens(L.n_pairs, L.n_tokens);
  a.n_splits = att_n_splits(L.n_pairs, L.n_tokens);
  hipStream_t s = (hipStream_t)stream;
  hipLaunchKernelGGL(k_att_prologue, dim3((unsigned)L.n_pairs), dim3(256), 0, s, a);
  hipLaunchKernelGGL(k_att_main, dim3((unsigned)a.n_splits, (unsigned)L.n_pairs), dim3(ATT_THREADS), ATT_LDS, s, a);
  hipLaunchKernelGGL(k_att_combine, dim3((unsigned)(L.n_pairs * L.group)), dim3(128), 0, s, a);
  return hipGetLastError() != hipSuccess;
}

}  // namespace stc
