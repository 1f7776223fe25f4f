// Host side of libstc: argument validation, the calibration math that runs on
// the CPU (eigendecomposition, water-filling, quantizer steps, Lloyd-Max), the
// construction of device state blobs, and the C ABI entry points.
//
// Sources, by page title and section (the pages are web summaries):
//  - "Sintesi Tecnica: SPECTRA" (gist.science), "Metodologia: SPECTRA"
//    observations 1-3 and "La Pipeline di SPECTRA" steps 1-3.
//  - "Technisch Overzicht: Ablatie, Statistische Inferentie en Validatie voor
//    KV-Cache Compressie" (gist.science), "Experimentele Opstelling".
// The readings taken where the pages are silent are listed in include/stc.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <limits>
#include <numeric>
#include <string>
#include <thread>
#include <vector>

#include "stc_internal.h"

using namespace stc;

namespace {
std::atomic<int> g_rht_encode_kernel{STC_RHT_ENCODE_BUTTERFLY};
}
int stc::rht_encode_kernel() { return g_rht_encode_kernel.load(std::memory_order_relaxed); }

namespace {

thread_local std::string g_err;

stc_status fail(stc_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

stc_status ok() {
  g_err.clear();
  return STC_OK;
}

stc_status hip_check(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(STC_EDEVICE, "%s: %s", what, hipGetErrorString(e));
  return STC_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// ------------------------------------------------------------ bf16 helpers
uint16_t bf16_bits_rne(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);  // NaN stays NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
// IEEE binary16 bits of fp32 f, round to nearest even (NaN stays NaN,
// values from 65520 up become infinity, subnormal halves below 2^-14).
uint16_t f16_bits_rne(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  const uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return sign | 0x7e00u;
  if (a >= 0x477ff000u) return sign | 0x7c00u;
  if (a < 0x38800000u) {
    float av;
    std::memcpy(&av, &a, 4);
    return sign | (uint16_t)std::nearbyint(av * 16777216.0f);  // units of 2^-24
  }
  uint32_t r = a - 0x38000000u;  // exponent bias 127 -> 15
  r += 0xfffu + ((r >> 13) & 1u);
  return sign | (uint16_t)(r >> 13);
}
double bf16_value(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return (double)f;
}
// fp16 bits of a double, rounded to nearest even (|v| < 65520; subnormals kept).
uint16_t fp16_bits_rne(double v) {
  const uint16_t sign = std::signbit(v) ? 0x8000u : 0u;
  const double a = std::fabs(v);
  if (a == 0.0) return sign;
  int e = 0;
  const double m = std::frexp(a, &e);  // a = m 2^e, m in [0.5, 1)
  if (e - 1 < -14) return (uint16_t)(sign | (uint16_t)std::nearbyint(std::ldexp(a, 24)));  // k 2^-24 (k = 1024: the least normal)
  double k = std::nearbyint(m * 2048.0);  // 1024 .. 2048
  if (k == 2048.0) {
    k = 1024.0;
    ++e;
  }
  return (uint16_t)(sign | (uint16_t)((e - 1 + 15) << 10) | (uint16_t)(k - 1024.0));
}
double fp16_value(uint16_t b) {
  const int ex = (b >> 10) & 31, mant = b & 1023;
  const double v = ex == 0 ? std::ldexp((double)mant, -24) : std::ldexp(1024.0 + mant, ex - 25);
  return (b & 0x8000u) ? -v : v;
}
// hi + lo split of a double into two bf16 values (hi = RNE(v), lo = RNE(v - hi)).
void split_bf16(double v, uint16_t* hi, uint16_t* lo) {
  *hi = bf16_bits_rne((float)v);
  *lo = bf16_bits_rne((float)(v - bf16_value(*hi)));
}

// ------------------------------------------------ MSE-optimal uniform step
// Slope of the MSE of the 2^b-level midrise uniform quantizer with step
// delta on N(0,1). By symmetry only the cells of the non-negative half are
// summed: cell i = [i delta, (i+1) delta) (the last one open) with level
// (i + 1/2) delta. The moving cell edges contribute nothing because each edge
// is the midpoint of its two levels, so the slope is
//   -4 sum_i m_i ( int_cell x phi(x) dx - m_i delta P(cell) ),  m_i = i + 1/2.
double mse_slope(double delta, int levels) {
  const double inv_sqrt2pi = 0.39894228040143267794;
  const int half = levels / 2;
  double acc = 0.0;
  for (int i = 0; i < half; ++i) {
    const double a = i * delta;
    const bool last = (i == half - 1);
    const double b = last ? 0.0 : (i + 1) * delta;
    const double phia = inv_sqrt2pi * std::exp(-0.5 * a * a);
    const double phib = last ? 0.0 : inv_sqrt2pi * std::exp(-0.5 * b * b);
    const double qa = 0.5 * std::erfc(a / std::sqrt(2.0));
    const double qb = last ? 0.0 : 0.5 * std::erfc(b / std::sqrt(2.0));
    const double m = i + 0.5;
    acc += m * ((phia - phib) - m * delta * (qa - qb));
  }
  return -4.0 * acc;
}

double delta_star_impl(int bits) {
  const int levels = 1 << bits;
  double lo = 1e-6, hi = 4.0;  // slope < 0 at lo, > 0 at hi for every b in 1..8
  for (int it = 0; it < 400; ++it) {
    const double mid = 0.5 * (lo + hi);
    if (mid <= lo || mid >= hi) break;
    if (mse_slope(mid, levels) < 0.0) lo = mid; else hi = mid;
  }
  return 0.5 * (lo + hi);
}

// --------------------------------------------------------- cyclic Jacobi
// Golub & Van Loan, cyclic Jacobi: sweep over all (p, q), p < q, annihilating
// a_pq with the rotation from the symmetric 2x2 Schur decomposition, until a
// sweep finds every off-diagonal entry negligible next to its diagonal pair.
void jacobi_eigh(int n, std::vector<double>& a, std::vector<double>& v) {
  v.assign((size_t)n * n, 0.0);
  for (int i = 0; i < n; ++i) v[(size_t)i * n + i] = 1.0;
  for (int sweep = 0; sweep < 60; ++sweep) {
    bool rotated = false;
    for (int p = 0; p < n - 1; ++p) {
      for (int q = p + 1; q < n; ++q) {
        const double apq = a[(size_t)p * n + q];
        const double app = a[(size_t)p * n + p];
        const double aqq = a[(size_t)q * n + q];
        if (apq == 0.0) continue;
        const double g = 100.0 * std::fabs(apq);
        if (sweep > 3 && std::fabs(app) + g == std::fabs(app) && std::fabs(aqq) + g == std::fabs(aqq)) {
          a[(size_t)p * n + q] = a[(size_t)q * n + p] = 0.0;
          continue;
        }
        rotated = true;
        const double theta = (aqq - app) / (2.0 * apq);
        double t;
        if (std::fabs(theta) > 1e150) {
          t = 0.5 / theta;
        } else {
          t = (theta >= 0.0 ? 1.0 : -1.0) / (std::fabs(theta) + std::sqrt(theta * theta + 1.0));
        }
        const double c = 1.0 / std::sqrt(t * t + 1.0);
        const double s = t * c;
        for (int k = 0; k < n; ++k) {  // columns p, q
          const double akp = a[(size_t)k * n + p], akq = a[(size_t)k * n + q];
          a[(size_t)k * n + p] = c * akp - s * akq;
          a[(size_t)k * n + q] = s * akp + c * akq;
        }
        for (int k = 0; k < n; ++k) {  // rows p, q
          const double apk = a[(size_t)p * n + k], aqk = a[(size_t)q * n + k];
          a[(size_t)p * n + k] = c * apk - s * aqk;
          a[(size_t)q * n + k] = s * apk + c * aqk;
        }
        a[(size_t)p * n + q] = a[(size_t)q * n + p] = 0.0;
        for (int k = 0; k < n; ++k) {
          const double vkp = v[(size_t)k * n + p], vkq = v[(size_t)k * n + q];
          v[(size_t)k * n + p] = c * vkp - s * vkq;
          v[(size_t)k * n + q] = s * vkp + c * vkq;
        }
      }
    }
    if (!rotated) break;
  }
}

// Sort eigenpairs by descending eigenvalue (stable), then make the
// largest-magnitude entry of every column positive (lowest row on a tie).
void sort_and_fix_signs(int n, const std::vector<double>& diag, const std::vector<double>& v,
                        double* u_out, double* lam_out) {
  std::vector<int> order(n);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(), [&](int x, int y) { return diag[x] > diag[y]; });
  for (int j = 0; j < n; ++j) {
    const int src = order[j];
    lam_out[j] = diag[src];
    int kmax = 0;
    double vmax = -1.0;
    for (int i = 0; i < n; ++i) {
      const double m = std::fabs(v[(size_t)i * n + src]);
      if (m > vmax) { vmax = m; kmax = i; }
    }
    const double sgn = v[(size_t)kmax * n + src] < 0.0 ? -1.0 : 1.0;
    for (int i = 0; i < n; ++i) u_out[(size_t)i * n + j] = sgn * v[(size_t)i * n + src];
  }
}

// ------------------------------------------------------ unpack plan
// For each quarter of 32 channels and each group of 4 consecutive channels,
// where the group's codes sit relative to the quarter's first code bit: the
// quarter-relative 32-bit word k holding its first bit, the shift s inside
// it, and the 4 widths. 4 codes span at most 32 bits, so one 64-bit window
// (words k, k+1) always holds the whole group.
void fill_unpack_plan(DevHdr* h) {
  for (int q = 0; q < 4; ++q) {
    const uint32_t q0 = h->off[32 * q];
    h->qoff[q] = q0;
    uint32_t kmax = 0;
    for (int i = 0; i < 8; ++i) {
      const int c = 32 * q + 4 * i;
      const uint32_t rel = h->off[c] - q0;
      const uint32_t k = rel >> 5, sft = rel & 31;
      kmax = std::max(kmax, k);
      h->plan[q][i] = k | sft << 5 | (uint32_t)h->bits[c] << 10 | (uint32_t)h->bits[c + 1] << 14 |
                      (uint32_t)h->bits[c + 2] << 18 | (uint32_t)h->bits[c + 3] << 22;
    }
    h->qwords[q] = kmax + 2;
  }
}

// ------------------------------------------------------ state construction
stc_status build_eigen_blob(int d, int xform, const double* u, const double* lambda,
                            const uint8_t* bits, const double* steps_in, stc_head_info* info,
                            std::vector<unsigned char>& blob) {
  blob.assign(STATE_BYTES, 0);
  DevHdr* h = reinterpret_cast<DevHdr*>(blob.data() + OFF_HDR);
  float* u32 = reinterpret_cast<float*>(blob.data() + OFF_U32);
  uint16_t* ut_hi = reinterpret_cast<uint16_t*>(blob.data() + OFF_UT_HI);
  uint16_t* ut_lo = reinterpret_cast<uint16_t*>(blob.data() + OFF_UT_LO);
  uint16_t* w_hi = reinterpret_cast<uint16_t*>(blob.data() + OFF_W_HI);
  uint16_t* w_lo = reinterpret_cast<uint16_t*>(blob.data() + OFF_W_LO);
  float* thr = reinterpret_cast<float*>(blob.data() + OFF_THR);

  std::vector<double> ud((size_t)d * d, 0.0);
  if (xform == STC_XFORM_IDENTITY) {
    for (int i = 0; i < d; ++i) ud[(size_t)i * d + i] = 1.0;
  } else {
    for (size_t k = 0; k < (size_t)d * d; ++k) ud[k] = u[k];
  }
  double steps[D];
  int total = 0, n_kept = 0, last = -1, nthr = 0;
  for (int j = 0; j < d; ++j) {
    const int b = bits[j];
    total += b;
    if (b > 0) { ++n_kept; last = j; }
    if (b == 0) steps[j] = 0.0;
    else if (steps_in) steps[j] = steps_in[j];
    else steps[j] = std::sqrt(std::max(lambda[j], 0.0)) * delta_star_impl(b);
  }
  h->xform = xform;
  h->total_bits = total;
  h->n_kept = n_kept;
  h->nmax16 = last < 0 ? 0 : 16 * ((last + 16) / 16);
  h->kmax32 = last < 0 ? 0 : 32 * ((last + 32) / 32);
  int off = 0;
  for (int j = 0; j < d; ++j) {
    const int b = bits[j];
    h->bits[j] = (uint8_t)b;
    h->off[j] = (uint16_t)off;
    off += b;
    if (b > 0) {
      const int L = 1 << b;
      h->inv_step[j] = steps[j] > 0.0 ? (float)(1.0 / steps[j]) : 0.0f;
      h->ybias[j] = (float)(L / 2) + quant_eps(L);
      h->lm1[j] = L - 1;
      h->thr_base[j] = nthr;
      for (int k = 1; k < L; ++k) thr[nthr++] = (float)(((double)k - (double)(L / 2)) * steps[j]);
      h->step32[j] = (float)steps[j];
      h->step64[j] = steps[j];
      h->halfspan[j] = 0.5f * (float)(L - 1);
      h->yhalf[j] = steps[j] > 0.0 ? (float)(L / 2) : (float)L - 0.5f;
    } else {
      h->inv_step[j] = 0.0f;
      h->ybias[j] = 0.5f;
      h->lm1[j] = 0;
      h->thr_base[j] = 0;
      h->step32[j] = 0.0f;
      h->halfspan[j] = 0.0f;
    }
  }
  for (int i = 0; i < d; ++i) {
    double bias = 0.0;
    for (int j = 0; j < d; ++j) {
      const double uij = ud[(size_t)i * d + j];
      u32[i * D + j] = (float)uij;
      if (bits[j] > 0) bias += uij * steps[j] * 0.5 * (double)((1 << bits[j]) - 1);
    }
    h->bias[i] = (float)bias;
  }
  for (int R = 0; R < D; ++R) {
    const int j = enc_row_channel(R);
    if (j >= d) continue;
    const double ys = bits[j] == 0 ? 0.0 : (steps[j] > 0.0 ? 1.0 / steps[j] : 0x1p100);
    for (int i = 0; i < d; ++i) split_bf16(ud[(size_t)i * d + j] * ys, &ut_hi[R * D + i], &ut_lo[R * D + i]);
  }
  for (int j = 0; j < d; ++j) h->bits4[j / 8] |= (uint32_t)bits[j] << (4 * (j % 8));
  fill_unpack_plan(h);
  {
    // attention value columns: each code cut at the record's byte boundaries
    AttVCol* vc = reinterpret_cast<AttVCol*>(blob.data() + OFF_ATTV);
    uint32_t* vch = reinterpret_cast<uint32_t*>(blob.data() + OFF_ATTVCH);
    int nc = 0;
    for (int j = 0; j < d; ++j) {
      const int first = nc;
      int bit = h->off[j], z = 0, rem = bits[j];
      while (rem > 0) {
        const int s = bit & 7, w = std::min(8 - s, rem);
        const uint32_t m = ((1u << w) - 1u) << s;
        vc[nc].row = (uint32_t)(bit >> 3);
        vc[nc].mask2 = m | (m << 16);
        vc[nc].fac = std::ldexp(1.0f, 24 - s + z);
        vc[nc].chan = (uint32_t)j;
        ++nc;
        bit += w;
        z += w;
        rem -= w;
      }
      vch[j] = (uint32_t)first | ((uint32_t)(nc - first) << 16);
    }
    h->n_vcols = nc;
  }
  // fp16 W scaled by 2^e16 so that its largest entry lies in [2^13, 2^14);
  // the codes enter that decode scaled by 2^-e16 (exact in fp16 for e16 in
  // [-7, 24]; other scales leave the region unused, see decode_w16_ok)
  uint16_t* w16 = reinterpret_cast<uint16_t*>(blob.data() + OFF_W16);
  double wmax = 0.0;
  for (int i = 0; i < d; ++i)
    for (int j = 0; j < d; ++j) wmax = std::max(wmax, std::fabs(ud[(size_t)i * d + j] * steps[j]));
  int e16 = 0;
  if (wmax > 0.0) {
    std::frexp(wmax, &e16);  // wmax = m 2^e16, m in [0.5, 1)
    e16 = 14 - e16;
  }
  const bool w16_range = e16 >= -7 && e16 <= 24;
  for (int R = 0; R < D; ++R) {
    const int i = enc_row_channel(R);  // output dim of stored row R (same permutation as the encode basis)
    double b16 = 0.0;
    for (int j = 0; j < d; ++j) {
      const double wij = ud[(size_t)i * d + j] * steps[j];
      split_bf16(wij, &w_hi[R * D + j], &w_lo[R * D + j]);
      w16[R * D + j] = w16_range ? fp16_bits_rne(std::ldexp(wij, e16)) : 0;
      if (bits[j] > 0) b16 += std::ldexp(fp16_value(w16[R * D + j]), -e16) * 0.5 * (double)((1 << bits[j]) - 1);
    }
    if (i < D) h->bias16[i] = (float)b16;
  }
  {
    const uint32_t c = w16_range ? fp16_bits_rne(std::ldexp(1.0, -e16)) : 0u;
    h->code16 = c | (c << 16);
  }
  if (info) {
    info->d = d;
    info->xform = xform;
    info->total_bits = total;
    info->n_kept = n_kept;
    info->sketch_bits = 0;
    for (int j = 0; j < d; ++j) {
      info->bits[j] = bits[j];
      info->lambda[j] = lambda ? lambda[j] : 0.0;
      info->steps[j] = steps[j];
    }
  }
  return STC_OK;
}

stc_status upload(const std::vector<unsigned char>& blob, void* state_dev, stc_stream_t stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  stc_status st = hip_check(hipMemcpyAsync(state_dev, blob.data(), blob.size(), hipMemcpyHostToDevice, s),
                            "state upload");
  if (st) return st;
  return hip_check(hipStreamSynchronize(s), "state upload sync");
}

stc_status check_state_ptr(const void* p, const char* name) {
  if (!p) return fail(STC_EINVAL, "%s is NULL", name);
  if (!aligned(p, 256)) return fail(STC_EINVAL, "%s must be 256-byte aligned", name);
  return STC_OK;
}

int elem_size(int32_t dtype) { return dtype == STC_F32 ? 4 : 2; }

}  // namespace

extern "C" {

const char* stc_status_str(stc_status s) {
  switch (s) {
    case STC_OK: return "ok";
    case STC_EINVAL: return "invalid argument";
    case STC_EUNSUPPORTED: return "unsupported";
    case STC_EBUDGET: return "bit budget";
    case STC_EWORKSPACE: return "workspace too small";
    case STC_EDEVICE: return "device error";
    default: return "unknown status";
  }
}

const char* stc_last_error(void) { return g_err.c_str(); }

size_t stc_state_bytes(void) { return STATE_BYTES; }

size_t stc_packed_bytes(int32_t total_bits, int64_t n_tokens) {
  if (total_bits < 0 || n_tokens < 0) return 0;
  return packed_bytes(total_bits, n_tokens);
}

size_t stc_attend_workspace_bytes(int64_t n_pairs, int32_t group, int64_t n_tokens) {
  if (n_pairs <= 0 || n_tokens <= 0 || group <= 0) return 256;
  // one launch covers at most ATT_MAX_PAIRS pairs; launches reuse the area,
  // which holds the larger of a full launch's and the last launch's needs
  const int64_t np = n_pairs < ATT_MAX_PAIRS ? n_pairs : ATT_MAX_PAIRS;
  const int64_t last = n_pairs % ATT_MAX_PAIRS;
  int64_t floats = att_launch_floats(np, n_tokens, group);
  if (last) floats = std::max(floats, att_launch_floats(last, n_tokens, group));
  const size_t bytes = (size_t)floats * sizeof(float);
  return (bytes + 255) / 256 * 256;
}

int32_t stc_total_bits(float avg_bits, int32_t d) {
  return (int32_t)std::floor((double)avg_bits * d + 0.5);
}

double stc_delta_star(int32_t bits) {
  if (bits < 1 || bits > STC_MAX_BITS) return std::numeric_limits<double>::quiet_NaN();
  static double cache[STC_MAX_BITS + 1] = {0};
  if (cache[bits] == 0.0) cache[bits] = delta_star_impl(bits);
  return cache[bits];
}

stc_status stc_water_fill(int32_t d, const double* lambda, int32_t total_bits, uint8_t* bits_out) {
  if (d <= 0 || !lambda || !bits_out) return fail(STC_EINVAL, "water_fill: bad arguments");
  if (total_bits < 0 || total_bits > STC_MAX_BITS * d)
    return fail(STC_EBUDGET, "water_fill: budget %d outside [0, %d]", total_bits, STC_MAX_BITS * d);
  std::vector<int> b(d, 0);
  for (int it = 0; it < total_bits; ++it) {
    int best = -1;
    double bestv = -1.0;
    for (int j = 0; j < d; ++j) {
      if (b[j] >= STC_MAX_BITS) continue;
      const double lam = lambda[j] > 0.0 ? lambda[j] : 0.0;
      const double g = std::ldexp(lam, -2 * b[j]);
      if (g > bestv) { bestv = g; best = j; }
    }
    b[best] += 1;
  }
  for (int j = 0; j < d; ++j) bits_out[j] = (uint8_t)b[j];
  return ok();
}

// MSE of the midrise uniform quantizer with `levels` levels and step delta
// on N(0, 1): both halves of sum over cells of int (x - level)^2 phi(x) dx,
// with int_a^b x^2 phi = [Q(x) ... ] written through Q = upper tail, phi.
double gauss_uniform_mse(double delta, int levels) {
  const double inv_sqrt2pi = 0.39894228040143267794;
  const int half = levels / 2;
  double acc = 0.0;
  for (int i = 0; i < half; ++i) {
    const double a = i * delta;
    const bool last = (i == half - 1);
    const double b = (i + 1) * delta;
    const double y = (i + 0.5) * delta;
    const double phia = inv_sqrt2pi * std::exp(-0.5 * a * a);
    const double phib = last ? 0.0 : inv_sqrt2pi * std::exp(-0.5 * b * b);
    const double qa = 0.5 * std::erfc(a / std::sqrt(2.0));
    const double qb = last ? 0.0 : 0.5 * std::erfc(b / std::sqrt(2.0));
    const double pr = qa - qb;                              // P(a <= x < b)
    const double m1 = phia - phib;                          // int x phi
    const double m2 = pr + a * phia - (last ? 0.0 : b * phib);  // int x^2 phi
    acc += m2 - 2.0 * y * m1 + y * y * pr;
  }
  return 2.0 * acc;
}

// Distortion of a unit Gaussian channel at b bits (1 when dropped).
static double eps_bits(int b) {
  static double tab[STC_MAX_BITS + 1] = {-1.0};
  if (tab[0] < 0.0) {
    tab[0] = 1.0;
    for (int k = 1; k <= STC_MAX_BITS; ++k) tab[k] = gauss_uniform_mse(delta_star_impl(k), 1 << k);
  }
  return tab[b];
}

stc_status stc_allocate_bits(int32_t d, const double* lambda, int32_t total_bits, int32_t variant, double param,
                             uint8_t* bits_out) {
  if (d <= 0 || !lambda || !bits_out) return fail(STC_EINVAL, "allocate_bits: bad arguments");
  if (total_bits < 0 || total_bits > STC_MAX_BITS * d)
    return fail(STC_EBUDGET, "allocate_bits: budget %d outside [0, %d]", total_bits, STC_MAX_BITS * d);
  std::vector<double> lam(d);
  for (int j = 0; j < d; ++j) lam[j] = lambda[j] > 0.0 ? lambda[j] : 0.0;
  std::vector<int> b(d, 0);
  // one bit at a time to the channel of largest gain (lowest index on ties)
  auto greedy = [&](int first, int last, int nbits, auto gain) {
    for (int it = 0; it < nbits; ++it) {
      int best = -1;
      double bestv = -1.0;
      for (int j = first; j < last; ++j) {
        if (b[j] >= STC_MAX_BITS) continue;
        const double g = gain(j);
        if (g > bestv) { bestv = g; best = j; }
      }
      if (best < 0) break;
      b[best] += 1;
    }
  };
  auto rd_gain = [&](int j) { return std::ldexp(lam[j], -2 * b[j]); };
  switch (variant) {
    case STC_ALLOC_GREEDY:
      greedy(0, d, total_bits, rd_gain);
      break;
    case STC_ALLOC_OPERATIONAL:
      greedy(0, d, total_bits, [&](int j) { return lam[j] * (eps_bits(b[j]) - eps_bits(b[j] + 1)); });
      break;
    case STC_ALLOC_GROUPED: {
      const int G = (int)param;
      if (param != (double)G || G < 1 || d % G) return fail(STC_EINVAL, "allocate_bits: group size %g", param);
      const int ng = d / G;
      std::vector<double> lg(ng, 0.0);
      std::vector<int> bg(ng, 0);
      for (int j = 0; j < d; ++j) lg[j / G] += lam[j];
      for (int left = total_bits; left >= G; left -= G) {
        int best = -1;
        double bestv = -1.0;
        for (int k = 0; k < ng; ++k) {
          if (bg[k] >= STC_MAX_BITS) continue;
          const double g = std::ldexp(lg[k], -2 * bg[k]);
          if (g > bestv) { bestv = g; best = k; }
        }
        if (best < 0) break;
        bg[best] += 1;
      }
      for (int j = 0; j < d; ++j) b[j] = bg[j / G];
      break;
    }
    case STC_ALLOC_FLOOR: {
      const int f = (int)param;
      if (param != (double)f || f < 0 || f > STC_MAX_BITS || f * d > total_bits)
        return fail(STC_EINVAL, "allocate_bits: floor %g with budget %d", param, total_bits);
      for (int j = 0; j < d; ++j) b[j] = f;
      greedy(0, d, total_bits - f * d, rd_gain);
      break;
    }
    case STC_ALLOC_GAP: {
      if (!(param > 1.0)) return fail(STC_EINVAL, "allocate_bits: gap ratio %g must exceed 1", param);
      int d_eff = d;
      for (int j = 0; j + 1 < d; ++j)
        if (lam[j] > 0.0 && (lam[j + 1] <= 0.0 || lam[j] >= param * lam[j + 1])) { d_eff = j + 1; break; }
      greedy(0, d_eff, std::min(total_bits, STC_MAX_BITS * d_eff), rd_gain);
      break;
    }
    default:
      return fail(STC_EINVAL, "allocate_bits: unknown variant %d", variant);
  }
  for (int j = 0; j < d; ++j) bits_out[j] = (uint8_t)b[j];
  return ok();
}

stc_status stc_eigh(int32_t d, const double* a, double* u_out, double* lambda_out) {
  if (d <= 0 || !a || !u_out || !lambda_out) return fail(STC_EINVAL, "eigh: bad arguments");
  for (size_t k = 0; k < (size_t)d * d; ++k)
    if (!std::isfinite(a[k])) return fail(STC_EINVAL, "eigh: entry %zu is not finite", k);
  std::vector<double> m(a, a + (size_t)d * d), v;
  // symmetrize exactly (the input is symmetric up to rounding at most)
  for (int i = 0; i < d; ++i)
    for (int j = i + 1; j < d; ++j) m[(size_t)j * d + i] = m[(size_t)i * d + j];
  jacobi_eigh(d, m, v);
  std::vector<double> diag(d);
  for (int i = 0; i < d; ++i) diag[i] = m[(size_t)i * d + i];
  sort_and_fix_signs(d, diag, v, u_out, lambda_out);
  return ok();
}

stc_status stc_lloyd_max(const double* samples, int64_t n, int32_t levels, double tol, int32_t max_iter,
                         double* centroids_out, int32_t* iters_out) {
  if (!samples || n < 2 || levels < 2 || !centroids_out) return fail(STC_EINVAL, "lloyd_max: bad arguments");
  std::vector<double> y(samples, samples + n);
  std::sort(y.begin(), y.end());
  std::vector<long double> pre((size_t)n + 1, 0.0L);
  for (int64_t i = 0; i < n; ++i) pre[i + 1] = pre[i] + (long double)y[i];
  std::vector<double> c(levels), nc(levels), t(levels - 1);
  for (int k = 0; k < levels; ++k) {  // sample quantile (k + 1/2)/levels, linear interpolation
    const double p = (k + 0.5) / levels;
    const double hpos = (double)(n - 1) * p;
    const int64_t lo = (int64_t)std::floor(hpos);
    const double frac = hpos - (double)lo;
    const double a = y[lo], b = y[std::min<int64_t>(lo + 1, n - 1)];
    c[k] = frac >= 0.5 ? b - (b - a) * (1.0 - frac) : a + (b - a) * frac;
  }
  int it = 0;
  for (it = 1; it <= max_iter; ++it) {
    for (int k = 0; k < levels - 1; ++k) t[k] = 0.5 * (c[k] + c[k + 1]);
    int64_t start = 0;
    double moved = 0.0;
    for (int k = 0; k < levels; ++k) {
      const int64_t end = (k == levels - 1) ? n : (int64_t)(std::lower_bound(y.begin(), y.end(), t[k]) - y.begin());
      const int64_t cnt = end - start;
      nc[k] = cnt > 0 ? (double)((pre[end] - pre[start]) / (long double)cnt) : c[k];
      moved = std::max(moved, std::fabs(nc[k] - c[k]));
      start = end;
    }
    c = nc;
    if (moved < tol) break;
  }
  for (int k = 0; k < levels; ++k) centroids_out[k] = c[k];
  if (iters_out) *iters_out = std::min(it, max_iter);
  return ok();
}

stc_status stc_state_init(int32_t d, int32_t xform, const double* u, const double* lambda,
                          const uint8_t* bits, const double* steps, stc_head_info* info,
                          void* state_dev, stc_stream_t stream) {
  if (d != D) return fail(STC_EUNSUPPORTED, "state_init: d=%d (only %d is supported)", d, D);
  if (xform != STC_XFORM_EIGEN && xform != STC_XFORM_IDENTITY)
    return fail(STC_EUNSUPPORTED, "state_init: xform %d", xform);
  if (xform == STC_XFORM_EIGEN && !u) return fail(STC_EINVAL, "state_init: EIGEN needs a basis");
  if (xform == STC_XFORM_IDENTITY && u) return fail(STC_EINVAL, "state_init: IDENTITY takes no basis");
  if (!lambda || !bits || !info) return fail(STC_EINVAL, "state_init: NULL lambda/bits/info");
  if (stc_status s = check_state_ptr(state_dev, "state_dev")) return s;
  for (int j = 0; j < d; ++j)
    if (bits[j] > STC_MAX_BITS) return fail(STC_EBUDGET, "state_init: width %d > 8 at channel %d", bits[j], j);
  if (steps)
    for (int j = 0; j < d; ++j)
      if (bits[j] && !(steps[j] >= 0.0 && std::isfinite(steps[j])))
        return fail(STC_EINVAL, "state_init: bad step at channel %d", j);
  std::vector<unsigned char> blob;
  build_eigen_blob(d, xform, u, lambda, bits, steps, info, blob);
  if (stc_status s = upload(blob, state_dev, stream)) return s;
  return ok();
}

stc_status stc_state_init_sketch(int32_t d, int32_t xform, const double* u, const double* lambda,
                                 const uint8_t* bits, const double* steps, const float* sketch,
                                 stc_head_info* info, void* state_dev, stc_stream_t stream) {
  if (!sketch) return fail(STC_EINVAL, "state_init_sketch: NULL sketch matrix");
  for (int k = 0; k < STC_SKETCH_BITS * D; ++k)
    if (!std::isfinite(sketch[k])) return fail(STC_EINVAL, "state_init_sketch: sketch entry %d not finite", k);
  if (d != D) return fail(STC_EUNSUPPORTED, "state_init_sketch: d=%d (only %d is supported)", d, D);
  if (xform != STC_XFORM_EIGEN && xform != STC_XFORM_IDENTITY)
    return fail(STC_EUNSUPPORTED, "state_init_sketch: xform %d", xform);
  if (xform == STC_XFORM_EIGEN && !u) return fail(STC_EINVAL, "state_init_sketch: EIGEN needs a basis");
  if (xform == STC_XFORM_IDENTITY && u) return fail(STC_EINVAL, "state_init_sketch: IDENTITY takes no basis");
  if (!lambda || !bits || !info) return fail(STC_EINVAL, "state_init_sketch: NULL lambda/bits/info");
  if (stc_status s = check_state_ptr(state_dev, "state_dev")) return s;
  for (int j = 0; j < d; ++j)
    if (bits[j] > STC_MAX_BITS) return fail(STC_EBUDGET, "state_init_sketch: width %d > 8 at channel %d", bits[j], j);
  if (steps)
    for (int j = 0; j < d; ++j)
      if (bits[j] && !(steps[j] >= 0.0 && std::isfinite(steps[j])))
        return fail(STC_EINVAL, "state_init_sketch: bad step at channel %d", j);
  std::vector<unsigned char> blob;
  build_eigen_blob(d, xform, u, lambda, bits, steps, info, blob);
  // the sketch replaces the fp32 threshold table (which no kernel reads): S rows
  // (latent channel order) permuted like the encode basis, bf16 hi / lo, and
  // M^T = (S U^T)^T fp32 for the attention's S U^T q
  DevHdr* h = reinterpret_cast<DevHdr*>(blob.data() + OFF_HDR);
  h->sketch_bits = STC_SKETCH_BITS;
  uint16_t* p_hi = reinterpret_cast<uint16_t*>(blob.data() + OFF_SKP_HI);
  uint16_t* p_lo = reinterpret_cast<uint16_t*>(blob.data() + OFF_SKP_LO);
  float* mt = reinterpret_cast<float*>(blob.data() + OFF_SKT32);
  for (int R = 0; R < STC_SKETCH_BITS; ++R) {
    const int i = enc_row_channel(R);
    for (int j = 0; j < D; ++j) split_bf16((double)sketch[i * D + j], &p_hi[R * D + j], &p_lo[R * D + j]);
  }
  for (int k = 0; k < D; ++k)
    for (int i = 0; i < STC_SKETCH_BITS; ++i) {
      double acc = 0.0;  // M_ik = sum_j S_ij U_kj
      for (int j = 0; j < D; ++j) acc += (double)sketch[i * D + j] * (u ? u[(size_t)k * D + j] : (k == j ? 1.0 : 0.0));
      mt[k * STC_SKETCH_BITS + i] = (float)acc;
    }
  info->sketch_bits = STC_SKETCH_BITS;
  if (stc_status s = upload(blob, state_dev, stream)) return s;
  return ok();
}

static stc_status rht_state_build(int32_t d, const int8_t* signs, const float* codebook, const float* sketch,
                                  stc_head_info* info, void* state_dev, stc_stream_t stream) {
  if (d != D) return fail(STC_EUNSUPPORTED, "rht_state_init: d=%d (only %d is supported)", d, D);
  if (!signs || !codebook || !info) return fail(STC_EINVAL, "rht_state_init: NULL argument");
  if (stc_status s = check_state_ptr(state_dev, "state_dev")) return s;
  for (int i = 0; i < d; ++i)
    if (signs[i] != 1 && signs[i] != -1) return fail(STC_EINVAL, "rht_state_init: sign %d is not +-1", i);
  for (int k = 0; k < 8; ++k)
    if (!std::isfinite(codebook[k]) || (k && !(codebook[k] > codebook[k - 1])))
      return fail(STC_EINVAL, "rht_state_init: codebook must be finite and increasing");
  std::vector<unsigned char> blob(STATE_BYTES, 0);
  DevHdr* h = reinterpret_cast<DevHdr*>(blob.data());
  h->xform = STC_XFORM_RHT;
  h->total_bits = STC_RHT_BITS * d;
  h->n_kept = d;
  h->nmax16 = d;
  h->kmax32 = d;
  for (int j = 0; j < d; ++j) {
    h->bits[j] = STC_RHT_BITS;
    h->bits4[j / 8] |= (uint32_t)STC_RHT_BITS << (4 * (j % 8));
    h->off[j] = (uint16_t)(STC_RHT_BITS * j);
    h->sign[j] = (float)signs[j];
  }
  fill_unpack_plan(h);
  // encode basis: row R holds output channel j = enc_row_channel(R) of
  // H D, entries H[j][i] sign_i = +-1 (exact in bf16; no low part)
  uint16_t* ut_hi = reinterpret_cast<uint16_t*>(blob.data() + OFF_UT_HI);
  for (int R = 0; R < D; ++R) {
    const int j = enc_row_channel(R);
    for (int i = 0; i < D; ++i) {
      const int hsign = (__builtin_popcount((unsigned)(i & j)) & 1) ? -1 : 1;
      ut_hi[R * D + i] = hsign * signs[i] > 0 ? 0x3F80u : 0xBF80u;
    }
  }
  // attention reads a Walsh-Hadamard cache through the eigen machinery:
  // U = D H / sqrt(d) (U_ij = sign_i H[i][j] / sqrt(d); H is symmetric), unit
  // steps and no level offset, so the latent code average is the average of
  // codebook values and U rotates it back
  float* u32 = reinterpret_cast<float*>(blob.data() + OFF_U32);
  const double rs = 1.0 / std::sqrt((double)D);
  for (int i = 0; i < D; ++i)
    for (int j = 0; j < D; ++j) {
      const int hsign = (__builtin_popcount((unsigned)(i & j)) & 1) ? -1 : 1;
      u32[i * D + j] = (float)(hsign * signs[i] * rs);
    }
  for (int j = 0; j < D; ++j) {
    h->step32[j] = 1.0f;
    h->step64[j] = 1.0;
    h->halfspan[j] = 0.0f;
  }
  for (int k = 0; k < 8; ++k) {
    const uint16_t hi = bf16_bits_rne(codebook[k]);
    const uint16_t lo = bf16_bits_rne(codebook[k] - bf16_value(hi));
    const uint16_t hf = f16_bits_rne(codebook[k]);
    const uint16_t v[3] = {hi, lo, hf};
    for (int t = 0; t < 3; ++t) {
      h->cbt[4 * t + (k >> 2)] |= (uint32_t)(v[t] & 0xFF) << (8 * (k & 3));
      h->cbt[4 * t + 2 + (k >> 2)] |= (uint32_t)(v[t] >> 8) << (8 * (k & 3));
    }
  }
  for (int k = 0; k < 8; ++k) h->cb[k] = codebook[k];
  for (int k = 0; k < 7; ++k) h->cb_thr[k] = (float)(0.5 * ((double)codebook[k] + (double)codebook[k + 1]));
  if (sketch) {
    // key residual sketch: z = sign(S r), r = x - K_hat = |x| D H (y - y_hat) / sqrt(d),
    // so S r = |x| P e with P = S D H / sqrt(d) and e = y - y_hat in the rotated
    // basis; P rows permuted like the encode basis, S^T for the attention's S q
    h->sketch_bits = STC_SKETCH_BITS;
    uint16_t* p_hi = reinterpret_cast<uint16_t*>(blob.data() + OFF_SKP_HI);
    uint16_t* p_lo = reinterpret_cast<uint16_t*>(blob.data() + OFF_SKP_LO);
    float* st32 = reinterpret_cast<float*>(blob.data() + OFF_SKT32);
    const double rs = 1.0 / std::sqrt((double)D);
    for (int R = 0; R < STC_SKETCH_BITS; ++R) {
      const int i = enc_row_channel(R);
      for (int j = 0; j < D; ++j) {
        double acc = 0.0;  // (S D H)_ij = sum_k S_ik sign_k H[k][j]
        for (int k = 0; k < D; ++k) {
          const int hsign = (__builtin_popcount((unsigned)(k & j)) & 1) ? -1 : 1;
          acc += (double)sketch[i * D + k] * signs[k] * hsign;
        }
        split_bf16(acc * rs, &p_hi[R * D + j], &p_lo[R * D + j]);
      }
    }
    for (int i = 0; i < STC_SKETCH_BITS; ++i)
      for (int j = 0; j < D; ++j) st32[j * STC_SKETCH_BITS + i] = sketch[i * D + j];
  }
  info->d = d;
  info->xform = STC_XFORM_RHT;
  info->total_bits = h->total_bits;
  info->n_kept = d;
  info->sketch_bits = sketch ? STC_SKETCH_BITS : 0;
  for (int j = 0; j < d; ++j) {
    info->bits[j] = STC_RHT_BITS;
    info->lambda[j] = 0.0;
    info->steps[j] = 0.0;
  }
  if (stc_status s = upload(blob, state_dev, stream)) return s;
  return ok();
}

stc_status stc_rht_state_init(int32_t d, const int8_t* signs, const float* codebook, stc_head_info* info,
                              void* state_dev, stc_stream_t stream) {
  return rht_state_build(d, signs, codebook, nullptr, info, state_dev, stream);
}

stc_status stc_rht_sketch_state_init(int32_t d, const int8_t* signs, const float* codebook, const float* sketch,
                                     stc_head_info* info, void* state_dev, stc_stream_t stream) {
  if (!sketch) return fail(STC_EINVAL, "rht_sketch_state_init: NULL sketch matrix");
  for (int k = 0; k < STC_SKETCH_BITS * D; ++k)
    if (!std::isfinite(sketch[k])) return fail(STC_EINVAL, "rht_sketch_state_init: sketch entry %d not finite", k);
  return rht_state_build(d, signs, codebook, sketch, info, state_dev, stream);
}

}  // extern "C"

namespace {

// Calibration arguments shared by the single and batched calls; budget out.
stc_status check_calibration(const char* who, int32_t d, int64_t n_calib, const void* x_dev, int32_t dtype,
                             int64_t ld, float avg_bits, const uint8_t* bits, int32_t xform, int32_t* budget) {
  if (d != D) return fail(STC_EUNSUPPORTED, "%s: d=%d (only %d is supported)", who, d, D);
  if (xform != STC_XFORM_EIGEN && xform != STC_XFORM_IDENTITY)
    return fail(STC_EUNSUPPORTED, "%s: xform %d (use stc_rht_state_init for RHT)", who, xform);
  if (dtype != STC_F32 && dtype != STC_BF16) return fail(STC_EUNSUPPORTED, "%s: dtype %d", who, dtype);
  if (!x_dev) return fail(STC_EINVAL, "%s: NULL argument", who);
  if (n_calib <= 0) return fail(STC_EINVAL, "%s: n_calib must be positive", who);
  if (ld < d) return fail(STC_EINVAL, "%s: ld < d", who);
  if (!aligned(x_dev, 16) || (ld * elem_size(dtype)) % 16)
    return fail(STC_EINVAL, "%s: x rows must be 16-byte aligned", who);
  if (!(avg_bits >= 0.0f) || !std::isfinite(avg_bits)) return fail(STC_EBUDGET, "%s: bad budget", who);
  *budget = stc_total_bits(avg_bits, d);
  if (*budget > STC_MAX_BITS * d) return fail(STC_EBUDGET, "%s: budget %d > %d", who, *budget, STC_MAX_BITS * d);
  if (bits) {
    int sum = 0;
    for (int j = 0; j < d; ++j) {
      if (bits[j] > STC_MAX_BITS) return fail(STC_EBUDGET, "%s: width > 8 at channel %d", who, j);
      sum += bits[j];
    }
    if (sum != *budget) return fail(STC_EBUDGET, "%s: widths sum to %d, budget is %d", who, sum, *budget);
  }
  return STC_OK;
}

// Host part of a calibration: second moment g (d x d) -> basis, widths,
// state blob (with g kept in its scratch region) and summary.
stc_status state_from_gram(const char* who, const double* g, int32_t xform, int32_t budget, const uint8_t* bits,
                           stc_head_info* info, std::vector<unsigned char>& blob) {
  const int d = D;
  for (int i = 0; i < d * d; ++i)
    if (!std::isfinite(g[i]))
      return fail(STC_EINVAL, "%s: the second moment is not finite (NaN or Inf among the tokens)", who);
  std::vector<double> u((size_t)d * d), lam(d);
  if (xform == STC_XFORM_EIGEN) {
    if (stc_status st = stc_eigh(d, g, u.data(), lam.data())) return st;
  } else {
    for (int j = 0; j < d; ++j) lam[j] = g[(size_t)j * d + j];
  }
  std::vector<uint8_t> b(d);
  if (bits) std::copy(bits, bits + d, b.begin());
  else if (stc_status st = stc_water_fill(d, lam.data(), budget, b.data())) return st;
  if (stc_status st = build_eigen_blob(d, xform, xform == STC_XFORM_EIGEN ? u.data() : nullptr, lam.data(), b.data(),
                                       nullptr, info, blob))
    return st;
  std::memcpy(blob.data() + OFF_GRAM, g, (size_t)d * d * sizeof(double));
  return STC_OK;
}

}  // namespace

extern "C" {

stc_status stc_calibrate_head(int32_t d, int64_t n_calib, const void* x_dev, int32_t dtype, int64_t ld,
                              float avg_bits, const uint8_t* bits, int32_t xform, stc_head_info* info,
                              void* state_dev, stc_stream_t stream) {
  int32_t budget = 0;
  if (stc_status s = check_calibration("calibrate_head", d, n_calib, x_dev, dtype, ld, avg_bits, bits, xform, &budget))
    return s;
  if (!info) return fail(STC_EINVAL, "calibrate_head: NULL argument");
  if (stc_status s = check_state_ptr(state_dev, "state_dev")) return s;
  // second moment on the GPU (fp64), into the state's scratch region
  double* gram_dev = reinterpret_cast<double*>(static_cast<unsigned char*>(state_dev) + OFF_GRAM);
  if (launch_gram(x_dev, dtype, ld, 0, n_calib, 1, gram_dev, 0, stream))
    return fail(STC_EDEVICE, "gram launch: %s", hipGetErrorString(hipGetLastError()));
  std::vector<double> g((size_t)d * d);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (stc_status st = hip_check(hipMemcpyAsync(g.data(), gram_dev, g.size() * sizeof(double), hipMemcpyDeviceToHost, s), "gram download")) return st;
  if (stc_status st = hip_check(hipStreamSynchronize(s), "gram sync")) return st;
  std::vector<unsigned char> blob;
  if (stc_status st = state_from_gram("calibrate_head", g.data(), xform, budget, bits, info, blob)) return st;
  if (stc_status st = upload(blob, state_dev, stream)) return st;
  return ok();
}

stc_status stc_calibrate_heads_batched(int32_t d, int64_t n_streams, int64_t n_calib, const void* x_dev,
                                       int32_t dtype, int64_t ld, int64_t x_stream_stride, float avg_bits,
                                       int32_t xform, stc_head_info* infos, void* states_dev, stc_stream_t stream) {
  int32_t budget = 0;
  if (stc_status s = check_calibration("calibrate_heads_batched", d, n_calib, x_dev, dtype, ld, avg_bits, nullptr,
                                       xform, &budget))
    return s;
  if (n_streams < 0) return fail(STC_EINVAL, "calibrate_heads_batched: negative stream count");
  if (n_streams == 0) return ok();
  if (!infos) return fail(STC_EINVAL, "calibrate_heads_batched: NULL infos");
  if (stc_status s = check_state_ptr(states_dev, "states_dev")) return s;
  if (n_streams > 1 && (x_stream_stride < (n_calib - 1) * ld + D || (x_stream_stride * elem_size(dtype)) % 16))
    return fail(STC_EINVAL, "calibrate_heads_batched: x stream stride must cover n_calib rows and keep 16-byte "
                            "alignment");
  if (n_streams > (1 << 20)) return fail(STC_EINVAL, "calibrate_heads_batched: at most 2^20 streams");
  // every stream's second moment in one launch, into each state's scratch region
  unsigned char* base = static_cast<unsigned char*>(states_dev);
  if (launch_gram(x_dev, dtype, ld, x_stream_stride, n_calib, n_streams,
                  reinterpret_cast<double*>(base + OFF_GRAM), (int64_t)(STATE_BYTES / sizeof(double)), stream))
    return fail(STC_EDEVICE, "gram launch: %s", hipGetErrorString(hipGetLastError()));
  // the host part in chunks of at most 256 streams (host memory stays near
  // 160 MB whatever the batch): download the chunk's second moments, build
  // its eigenbases, widths and blobs on worker threads, upload its states
  const size_t dd = (size_t)D * D;
  constexpr int64_t CHUNK = 256;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  // the lazily filled step tables, before the workers read them
  for (int b = 1; b <= STC_MAX_BITS; ++b) (void)stc_delta_star(b);
  const unsigned hw = std::thread::hardware_concurrency();
  std::vector<double> g(dd * (size_t)std::min(n_streams, CHUNK));
  std::vector<unsigned char> all((size_t)std::min(n_streams, CHUNK) * STATE_BYTES);
  for (int64_t c0 = 0; c0 < n_streams; c0 += CHUNK) {
    const int64_t nc = std::min(CHUNK, n_streams - c0);
    if (stc_status st = hip_check(hipMemcpy2DAsync(g.data(), dd * sizeof(double), base + c0 * STATE_BYTES + OFF_GRAM,
                                                   STATE_BYTES, dd * sizeof(double), (size_t)nc,
                                                   hipMemcpyDeviceToHost, hs),
                                  "gram download"))
      return st;
    if (stc_status st = hip_check(hipStreamSynchronize(hs), "gram sync")) return st;
    // streams spread over worker threads; each worker keeps the first failure it meets
    const int64_t n_thr = std::min<int64_t>(nc, std::max(1u, std::min(hw, 16u)));
    std::atomic<int64_t> next{0};
    std::vector<stc_status> thr_status((size_t)n_thr, STC_OK);
    std::vector<std::string> thr_msg((size_t)n_thr);
    auto work = [&](int64_t t) {
      std::vector<unsigned char> blob;
      for (int64_t i = next.fetch_add(1); i < nc; i = next.fetch_add(1)) {
        stc_status st = state_from_gram("calibrate_heads_batched", g.data() + dd * (size_t)i, xform, budget, nullptr,
                                        &infos[c0 + i], blob);
        if (st) {
          thr_status[(size_t)t] = st;
          thr_msg[(size_t)t] = "stream " + std::to_string(c0 + i) + ": " + stc_last_error();
          next.store(nc);
          return;
        }
        std::memcpy(all.data() + (size_t)i * STATE_BYTES, blob.data(), STATE_BYTES);
      }
    };
    std::vector<std::thread> pool;
    for (int64_t t = 1; t < n_thr; ++t) pool.emplace_back(work, t);
    work(0);
    for (auto& th : pool) th.join();
    for (int64_t t = 0; t < n_thr; ++t)
      if (thr_status[(size_t)t]) return fail(thr_status[(size_t)t], "%s", thr_msg[(size_t)t].c_str());
    if (stc_status st = hip_check(hipMemcpyAsync(base + c0 * STATE_BYTES, all.data(), (size_t)nc * STATE_BYTES,
                                                 hipMemcpyHostToDevice, hs),
                                  "state upload"))
      return st;
    if (stc_status st = hip_check(hipStreamSynchronize(hs), "state upload sync")) return st;
  }
  return ok();
}

stc_status stc_state_basis(const void* state_dev, float* u_out, stc_stream_t stream) {
  if (stc_status s = check_state_ptr(state_dev, "state_dev")) return s;
  if (!u_out) return fail(STC_EINVAL, "state_basis: NULL output");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (stc_status st = hip_check(hipMemcpyAsync(u_out, static_cast<const unsigned char*>(state_dev) + OFF_U32,
                                               (size_t)D * D * sizeof(float), hipMemcpyDeviceToHost, s), "basis download")) return st;
  if (stc_status st = hip_check(hipStreamSynchronize(s), "basis sync")) return st;
  return ok();
}

stc_status stc_set_rht_encode_kernel(int32_t kind) {
  if (kind != STC_RHT_ENCODE_MFMA && kind != STC_RHT_ENCODE_BUTTERFLY)
    return fail(STC_EINVAL, "set_rht_encode_kernel: kind %d", (int)kind);
  g_rht_encode_kernel.store(kind, std::memory_order_relaxed);
  return ok();
}

int32_t stc_get_rht_encode_kernel(void) { return g_rht_encode_kernel.load(std::memory_order_relaxed); }

int32_t stc_debug_build(void) { return debug_build(); }

stc_status stc_stream_copy(void* dst_dev, const void* src_dev, int64_t bytes, stc_stream_t stream) {
  if (bytes < 0 || bytes % 16) return fail(STC_EINVAL, "stream_copy: bytes must be a non-negative multiple of 16");
  if (bytes == 0) return ok();
  if (!dst_dev || !src_dev || !aligned(dst_dev, 16) || !aligned(src_dev, 16))
    return fail(STC_EINVAL, "stream_copy: NULL or misaligned buffer");
  if (launch_stream_copy(dst_dev, src_dev, bytes, stream))
    return fail(STC_EDEVICE, "stream_copy launch: %s", hipGetErrorString(hipGetLastError()));
  return ok();
}

stc_status stc_debug_flags(uint32_t* flags, stc_stream_t stream) {
  if (!flags) return fail(STC_EINVAL, "debug_flags: NULL output");
  unsigned f = 0u;
  if (read_debug_flags(&f, stream)) return fail(STC_EDEVICE, "debug_flags: %s", hipGetErrorString(hipGetLastError()));
  *flags = f;
  return ok();
}

stc_status stc_check_state_map(const int32_t* map_dev, int64_t n, int64_t n_states, stc_stream_t stream) {
  if (n < 0 || n_states < 0) return fail(STC_EINVAL, "check_state_map: negative size");
  if (n == 0) return ok();
  if (!map_dev) return fail(STC_EINVAL, "check_state_map: NULL map");
  std::vector<int32_t> m((size_t)n);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (stc_status st = hip_check(hipMemcpyAsync(m.data(), map_dev, (size_t)n * sizeof(int32_t), hipMemcpyDeviceToHost, s),
                                "map download")) return st;
  if (stc_status st = hip_check(hipStreamSynchronize(s), "map sync")) return st;
  for (int64_t i = 0; i < n; ++i)
    if (m[(size_t)i] < 0 || m[(size_t)i] >= n_states)
      return fail(STC_EINVAL, "check_state_map: entry %lld is %d, outside [0, %lld)", (long long)i, m[(size_t)i],
                  (long long)n_states);
  return ok();
}

// Every record 0 or 32 * 2^s bits long (s = 0..5): the attention kernel then
// stages each record on a word-aligned slot of its own.
static bool records_word_pow2(const stc_head_info* infos, int64_t n) {
  for (int64_t i = 0; i < n; ++i) {
    const int b = infos[i].total_bits;
    if (b == 0) continue;
    if ((b & 31) || ((b >> 5) & ((b >> 5) - 1))) return false;
  }
  return true;
}

// ------------------------------------------------------------- codec calls
static stc_status check_batch(const char* who, const void* states_dev, int64_t n_states,
                              const stc_head_info* infos, int64_t n_streams, int64_t n_tokens,
                              int64_t packed_stride, bool* is_rht, int* max_bits) {
  if (stc_status s = check_state_ptr(states_dev, "states_dev")) return s;
  if (!infos) return fail(STC_EINVAL, "%s: NULL infos", who);
  if (n_states <= 0 || n_streams <= 0) return fail(STC_EINVAL, "%s: need at least one state and stream", who);
  if (n_tokens < 0) return fail(STC_EINVAL, "%s: negative token count", who);
  if (n_tokens > (int64_t)1 << 31) return fail(STC_EINVAL, "%s: more than 2^31 tokens per stream", who);
  int mb = 0;
  bool rht = infos[0].xform == STC_XFORM_RHT;
  for (int64_t i = 0; i < n_states; ++i) {
    const stc_head_info& f = infos[i];
    if (f.d != D) return fail(STC_EUNSUPPORTED, "%s: state %lld has d=%d", who, (long long)i, f.d);
    if ((f.xform == STC_XFORM_RHT) != rht) return fail(STC_EINVAL, "%s: states mix RHT and eigen families", who);
    if (f.xform < 0 || f.xform > 2) return fail(STC_EUNSUPPORTED, "%s: xform %d", who, f.xform);
    if (f.total_bits < 0 || f.total_bits > STC_MAX_BITS * D) return fail(STC_EBUDGET, "%s: total_bits %d", who, f.total_bits);
    mb = std::max(mb, f.total_bits);
  }
  if (packed_stride % 16) return fail(STC_EINVAL, "%s: packed stride must be a multiple of 16", who);
  if (n_streams > 1 && (size_t)packed_stride < packed_bytes(mb, n_tokens))
    return fail(STC_EINVAL, "%s: packed stride %lld < %zu bytes", who, (long long)packed_stride, packed_bytes(mb, n_tokens));
  *is_rht = rht;
  *max_bits = mb;
  return STC_OK;
}

// Encode tokens [n_old, n_old + m) of every stream (x row r = token n_old + r).
static stc_status encode_impl(const char* who, const void* states_dev, int64_t n_states, const int32_t* map,
                              const stc_head_info* infos, int64_t n_streams, int64_t n_old, int64_t m,
                              const void* x_dev, int32_t dtype, int64_t ld, int64_t x_stream_stride,
                              void* packed_dev, int64_t packed_stream_stride, float* norms_dev,
                              int64_t norms_stream_stride, stc_stream_t stream, void* sketch_dev = nullptr,
                              int64_t sketch_stream_stride = 0, float* rnorm_dev = nullptr,
                              int64_t rnorm_stream_stride = 0) {
  bool rht = false;
  int mb = 0;
  if (n_old < 0 || m < 0) return fail(STC_EINVAL, "%s: negative token count", who);
  if (stc_status s = check_batch(who, states_dev, n_states, infos, n_streams, n_old + m, packed_stream_stride,
                                 &rht, &mb)) return s;
  if (dtype != STC_F32 && dtype != STC_BF16) return fail(STC_EUNSUPPORTED, "%s: dtype %d", who, dtype);
  if (rht && dtype != STC_BF16) return fail(STC_EUNSUPPORTED, "%s: the RHT path takes bf16 tokens", who);
  if (m == 0) return ok();
  if (!x_dev || !packed_dev) return fail(STC_EINVAL, "%s: NULL buffer", who);
  if (rht && !norms_dev) return fail(STC_EINVAL, "%s: RHT states need a norms buffer", who);
  if (rht && n_streams > 1 && norms_stream_stride < n_old + m)
    return fail(STC_EINVAL, "%s: norms stream stride %lld < %lld tokens", who, (long long)norms_stream_stride,
                (long long)(n_old + m));
  const int es = elem_size(dtype);
  if (ld < D || !aligned(x_dev, 16) || (ld * es) % 16 || (x_stream_stride * es) % 16)
    return fail(STC_EINVAL, "%s: x rows must be >= 128 elements and 16-byte aligned", who);
  if (n_streams > 1 && x_stream_stride < (m - 1) * ld + D)
    return fail(STC_EINVAL, "%s: x stream stride too small", who);
  if (!aligned(packed_dev, 16)) return fail(STC_EINVAL, "%s: packed buffer must be 16-byte aligned", who);
  if (rht && !aligned(norms_dev, 4)) return fail(STC_EINVAL, "%s: norms misaligned", who);
  if (sketch_dev) {
    if (!rht) return fail(STC_EUNSUPPORTED, "%s: the residual sketch needs Walsh-Hadamard states", who);
    // the map lives on the device: streams whose state has no sketch matrix get codes and
    // norms only (their sketch bytes and residual norms are left as they are)
    bool any = false;
    for (int64_t i = 0; i < n_states; ++i) any = any || infos[i].sketch_bits == STC_SKETCH_BITS;
    if (!any) return fail(STC_EINVAL, "%s: no state has a sketch matrix", who);
    if (!rnorm_dev || !aligned(sketch_dev, 8) || !aligned(rnorm_dev, 4) || sketch_stream_stride % 8)
      return fail(STC_EINVAL, "%s: sketch needs 8-byte aligned bytes and a norms buffer", who);
    if (n_streams > 1 && (sketch_stream_stride < (n_old + m) * (STC_SKETCH_BITS / 8) ||
                          rnorm_stream_stride < n_old + m))
      return fail(STC_EINVAL, "%s: sketch or residual norm stride too small", who);
  }
  EncodeLaunch a{static_cast<const unsigned char*>(states_dev), map, n_states, n_streams, m, ld,
                 x_stream_stride, packed_stream_stride, x_dev, static_cast<unsigned char*>(packed_dev), norms_dev,
                 dtype == STC_F32 ? 1 : 0, mb, n_old, norms_stream_stride,
                 static_cast<unsigned char*>(sketch_dev), rnorm_dev, sketch_stream_stride, rnorm_stream_stride};
  a.rec = records_word_pow2(infos, n_states);
  const int rc = rht ? launch_encode_rht(a, stream) : launch_encode_eigen(a, stream);
  if (rc) return fail(STC_EDEVICE, "%s launch: %s", who, hipGetErrorString(hipGetLastError()));
  return ok();
}

stc_status stc_encode_kv_batched(const void* states_dev, int64_t n_states, const int32_t* map,
                                 const stc_head_info* infos, int64_t n_streams, int64_t n_tokens,
                                 const void* x_dev, int32_t dtype, int64_t ld, int64_t x_stream_stride,
                                 void* packed_dev, int64_t packed_stream_stride, float* norms_dev,
                                 stc_stream_t stream) {
  return encode_impl("encode_kv", states_dev, n_states, map, infos, n_streams, 0, n_tokens, x_dev, dtype, ld,
                     x_stream_stride, packed_dev, packed_stream_stride, norms_dev, n_tokens, stream);
}

stc_status stc_append_rht_sketch_batched(const void* states_dev, int64_t n_states, const int32_t* map,
                                        const stc_head_info* infos, int64_t n_streams, int64_t n_old, int64_t m,
                                        const void* x_dev, int64_t ld, int64_t x_stream_stride, void* packed_dev,
                                        int64_t packed_stream_stride, float* norms_dev, int64_t norms_stream_stride,
                                        void* sketch_dev, int64_t sketch_stream_stride, float* rnorm_dev,
                                        int64_t rnorm_stream_stride, stc_stream_t stream) {
  if (!sketch_dev && m > 0) return fail(STC_EINVAL, "append_rht_sketch: NULL sketch buffer");
  return encode_impl("append_rht_sketch", states_dev, n_states, map, infos, n_streams, n_old, m, x_dev, STC_BF16,
                     ld, x_stream_stride, packed_dev, packed_stream_stride, norms_dev, norms_stream_stride, stream,
                     sketch_dev, sketch_stream_stride, rnorm_dev, rnorm_stream_stride);
}

stc_status stc_sketch_kv_batched(const void* states_dev, int64_t n_states, const int32_t* map,
                                const stc_head_info* infos, int64_t n_streams, int64_t n_old, int64_t m,
                                const void* x_dev, int64_t ld, int64_t x_stream_stride, void* sketch_dev,
                                int64_t sketch_stream_stride, float* rnorm_dev, int64_t rnorm_stream_stride,
                                stc_stream_t stream) {
  bool rht = false;
  int mb = 0;
  if (n_old < 0 || m < 0) return fail(STC_EINVAL, "sketch_kv: negative token count");
  if (stc_status s = check_batch("sketch_kv", states_dev, n_states, infos, n_streams, n_old + m, (int64_t)1 << 40,
                                 &rht, &mb))  // no packed stream here
    return s;
  if (rht) return fail(STC_EUNSUPPORTED, "sketch_kv: eigen/identity states (Walsh-Hadamard: append_rht_sketch)");
  bool any = false;
  for (int64_t i = 0; i < n_states; ++i) any = any || infos[i].sketch_bits == STC_SKETCH_BITS;
  if (!any) return fail(STC_EINVAL, "sketch_kv: no state has a sketch matrix");
  if (m == 0) return ok();
  if (!x_dev || !sketch_dev || !rnorm_dev) return fail(STC_EINVAL, "sketch_kv: NULL buffer");
  if (ld < D || !aligned(x_dev, 16) || (ld * 2) % 16 || (x_stream_stride * 2) % 16)
    return fail(STC_EINVAL, "sketch_kv: x rows must be >= 128 bf16 and 16-byte aligned");
  if (n_streams > 1 && x_stream_stride < (m - 1) * ld + D) return fail(STC_EINVAL, "sketch_kv: x stream stride too small");
  if (!aligned(sketch_dev, 8) || !aligned(rnorm_dev, 4) || sketch_stream_stride % 8)
    return fail(STC_EINVAL, "sketch_kv: misaligned sketch or norms");
  if (n_streams > 1 && (sketch_stream_stride < (n_old + m) * (STC_SKETCH_BITS / 8) || rnorm_stream_stride < n_old + m))
    return fail(STC_EINVAL, "sketch_kv: sketch or residual norm stride too small");
  EncodeLaunch a{static_cast<const unsigned char*>(states_dev), map, n_states, n_streams, m, ld, x_stream_stride, 0,
                 x_dev, nullptr, nullptr, 0, mb, n_old, 0,
                 static_cast<unsigned char*>(sketch_dev), rnorm_dev, sketch_stream_stride, rnorm_stream_stride};
  if (launch_sketch_eigen(a, stream)) return fail(STC_EDEVICE, "sketch_kv launch: %s", hipGetErrorString(hipGetLastError()));
  return ok();
}

stc_status stc_append_kv_batched(const void* states_dev, int64_t n_states, const int32_t* map,
                                 const stc_head_info* infos, int64_t n_streams, int64_t n_old, int64_t m,
                                 const void* x_dev, int32_t dtype, int64_t ld, int64_t x_stream_stride,
                                 void* packed_dev, int64_t packed_stream_stride, float* norms_dev,
                                 int64_t norms_stream_stride, stc_stream_t stream) {
  return encode_impl("append_kv", states_dev, n_states, map, infos, n_streams, n_old, m, x_dev, dtype, ld,
                     x_stream_stride, packed_dev, packed_stream_stride, norms_dev, norms_stream_stride, stream);
}

// Decode in one fp16 pass (W 2^e16 rounded to fp16, codes times 2^-e16,
// instead of a bf16 hi + lo pair) when every state's budget is at most 2 bits
// per value and its largest kept step lies in [2^-7, 2^20] (then max |W|,
// between max step / sqrt(128) and max step, gives e16 in [-7, 24], where
// the scaled codes are exact in fp16). Each entry's relative error 2^-11,
// against a bias computed from the same fp16 entries, moves the
// reconstruction MSE by less than 1e-4 of the quantization MSE on the
// spiked-Gaussian workloads at these budgets (bf16 output, whose own rounding
// is 2^-9); higher budgets, whose quantization error is smaller, keep the
// pair.
static bool decode_w16_ok(const stc_head_info* infos, int64_t n) {
  for (int64_t k = 0; k < n; ++k) {
    if (infos[k].total_bits > 2 * D) return false;
    double smax = 0.0;
    for (int j = 0; j < infos[k].d && j < D; ++j)
      if (infos[k].bits[j] > 0) smax = std::max(smax, infos[k].steps[j]);
    if (smax > 0.0 && (smax < 0.0078125 || smax > 1048576.0)) return false;
  }
  return n > 0;
}

stc_status stc_decode_kv_batched(const void* states_dev, int64_t n_states, const int32_t* map,
                                 const stc_head_info* infos, int64_t n_streams, int64_t n_tokens,
                                 const void* packed_dev, int64_t packed_stream_stride, const float* norms_dev,
                                 void* x_out_dev, int32_t dtype, int64_t ld, int64_t x_stream_stride,
                                 stc_stream_t stream) {
  bool rht = false;
  int mb = 0;
  if (stc_status s = check_batch("decode_kv", states_dev, n_states, infos, n_streams, n_tokens,
                                 packed_stream_stride, &rht, &mb)) return s;
  if (dtype != STC_F32 && dtype != STC_BF16) return fail(STC_EUNSUPPORTED, "decode_kv: dtype %d", dtype);
  if (n_tokens == 0) return ok();
  if (!x_out_dev || !packed_dev) return fail(STC_EINVAL, "decode_kv: NULL buffer");
  if (rht && !norms_dev) return fail(STC_EINVAL, "decode_kv: RHT states need the norms");
  const int es = elem_size(dtype);
  if (ld < D || !aligned(x_out_dev, 16) || (ld * es) % 16 || (x_stream_stride * es) % 16)
    return fail(STC_EINVAL, "decode_kv: output rows must be >= 128 elements and 16-byte aligned");
  if (n_streams > 1 && x_stream_stride < (n_tokens - 1) * ld + D)
    return fail(STC_EINVAL, "decode_kv: output stream stride too small");
  if (!aligned(packed_dev, 16)) return fail(STC_EINVAL, "decode_kv: packed buffer must be 16-byte aligned");
  DecodeLaunch a{static_cast<const unsigned char*>(states_dev), map, n_states, n_streams, n_tokens, ld,
                 x_stream_stride, packed_stream_stride, static_cast<const unsigned char*>(packed_dev), norms_dev,
                 x_out_dev, dtype == STC_F32 ? 1 : 0, mb};
  a.w16 = !rht && dtype == STC_BF16 && decode_w16_ok(infos, n_states);
  const int rc = rht ? launch_decode_rht(a, stream) : launch_decode_eigen(a, stream);
  if (rc) return fail(STC_EDEVICE, "decode_kv launch: %s", hipGetErrorString(hipGetLastError()));
  return ok();
}

stc_status stc_encode_kv(const stc_head_info* info, const void* state_dev, int64_t n_tokens, const void* x_dev,
                         int32_t dtype, int64_t ld, void* packed_dev, float* norms_dev, stc_stream_t stream) {
  return stc_encode_kv_batched(state_dev, 1, nullptr, info, 1, n_tokens, x_dev, dtype, ld, 0, packed_dev,
                               (int64_t)packed_bytes(info ? info->total_bits : 0, n_tokens), norms_dev, stream);
}

stc_status stc_decode_kv(const stc_head_info* info, const void* state_dev, int64_t n_tokens, const void* packed_dev,
                         const float* norms_dev, void* x_out_dev, int32_t dtype, int64_t ld, stc_stream_t stream) {
  return stc_decode_kv_batched(state_dev, 1, nullptr, info, 1, n_tokens, packed_dev,
                               (int64_t)packed_bytes(info ? info->total_bits : 0, n_tokens), norms_dev, x_out_dev,
                               dtype, ld, 0, stream);
}

stc_status stc_quantize_pack_f32(const stc_head_info* info, const void* state_dev, int64_t n_tokens,
                                 const float* coeffs_dev, void* packed_dev, stc_stream_t stream) {
  bool rht = false;
  int mb = 0;
  if (stc_status s = check_batch("quantize_pack_f32", state_dev, 1, info, 1, n_tokens,
                                 (int64_t)packed_bytes(info ? info->total_bits : 0, n_tokens), &rht, &mb)) return s;
  if (rht) return fail(STC_EUNSUPPORTED, "quantize_pack_f32: eigen/identity states only");
  if (n_tokens == 0) return ok();
  if (!coeffs_dev || !packed_dev || !aligned(coeffs_dev, 16) || !aligned(packed_dev, 16))
    return fail(STC_EINVAL, "quantize_pack_f32: NULL or misaligned buffer");
  EncodeLaunch a{static_cast<const unsigned char*>(state_dev), nullptr, 1, 1, n_tokens, D, 0,
                 (int64_t)packed_bytes(mb, n_tokens), coeffs_dev, static_cast<unsigned char*>(packed_dev),
                 nullptr, 2, mb, 0, 0};
  if (launch_encode_eigen(a, stream)) return fail(STC_EDEVICE, "quantize_pack launch: %s", hipGetErrorString(hipGetLastError()));
  return ok();
}

// 1 KiB loads that cover one 32-token block (4 B bytes) of every state's
// stream, the block starting up to 12 bytes past a 16-byte boundary when
// 4 B is not a multiple of 16.
static int attend_chunks(const stc_head_info* infos, int64_t n) {
  int c = 1;
  for (int64_t i = 0; i < n; ++i) {
    const int64_t bytes = 4LL * infos[i].total_bits;
    const int64_t span = bytes + ((bytes & 15) ? 12 : 0);
    c = std::max(c, (int)((span + 1023) / 1024));
  }
  return c;
}

// Value columns of the attention kernels: the pieces of the kept codes cut at
// the record's byte boundaries (the largest count over the states).
static int attend_vcols(const stc_head_info* infos, int64_t n) {
  int most = 0;
  for (int64_t i = 0; i < n; ++i) {
    int off = 0, nc = 0;
    for (int j = 0; j < infos[i].d && j < STC_D; ++j) {
      const int b = infos[i].bits[j];
      if (b > 0) nc += (off + b - 1) / 8 - off / 8 + 1;
      off += b;
    }
    most = std::max(most, nc);
  }
  return most;
}

static bool records_256(const stc_head_info* infos, int64_t n) {
  for (int64_t i = 0; i < n; ++i)
    if (infos[i].total_bits != 256) return false;
  return n > 0;
}

// The eigen attention with a given partials area (the caller's workspace, or
// the library's static scratch for the entry point that allocates nothing).
static stc_status attend_eigen(const char* who, const void* states_dev, int64_t n_states, const int32_t* k_map,
                               const int32_t* v_map, const stc_head_info* infos, int64_t n_pairs, int64_t n_tokens,
                               const void* k_packed_dev, const void* v_packed_dev, int64_t packed_pair_stride,
                               int32_t group, const float* q_dev, float* out_dev, float scale, void* ws_dev,
                               size_t ws_bytes, bool scratch, stc_stream_t stream,
                               const void* k_new = nullptr, const void* v_new = nullptr, int new_f32 = 0) {
  bool rht = false;
  int mb = 0;
  if (stc_status s = check_batch("attend_compressed", states_dev, n_states, infos, n_pairs, n_tokens,
                                 packed_pair_stride, &rht, &mb)) return s;
  if (rht) return fail(STC_EUNSUPPORTED, "%s: eigen/identity states only", who);
  if (group < 1 || group > 16) return fail(STC_EUNSUPPORTED, "%s: group %d outside 1..16", who, group);
  if (n_tokens <= 0) return fail(STC_EINVAL, "%s: need at least one cached token", who);
  if (!k_packed_dev || !v_packed_dev || !q_dev || !out_dev || (!scratch && !ws_dev))
    return fail(STC_EINVAL, "%s: NULL buffer", who);
  if (!aligned(k_packed_dev, 16) || !aligned(v_packed_dev, 16) || !aligned(q_dev, 16) || !aligned(out_dev, 16) ||
      (!scratch && !aligned(ws_dev, 256)))
    return fail(STC_EINVAL, "%s: misaligned buffer", who);
  if (!std::isfinite(scale)) return fail(STC_EINVAL, "%s: scale must be finite", who);
  const size_t need = stc_attend_workspace_bytes(n_pairs, group, n_tokens);
  if (scratch) {
    if (need > attend_scratch_bytes())
      return fail(STC_EWORKSPACE, "%s: the call needs %zu bytes of partials, the static scratch holds %zu", who, need,
                  attend_scratch_bytes());
    if (attend_scratch(&ws_dev)) return fail(STC_EDEVICE, "%s: scratch address: %s", who,
                                             hipGetErrorString(hipGetLastError()));
  } else if (ws_bytes < need) {
    return fail(STC_EWORKSPACE, "%s: workspace %zu < %zu", who, ws_bytes, need);
  }
  const unsigned char* st = static_cast<const unsigned char*>(states_dev);
  AttendLaunch a{st, k_map, st, v_map, n_states, n_pairs, n_tokens, packed_pair_stride,
                 static_cast<const unsigned char*>(k_packed_dev), static_cast<const unsigned char*>(v_packed_dev),
                 group, q_dev, out_dev, scale, static_cast<unsigned char*>(ws_dev), mb};
  a.rec = records_word_pow2(infos, n_states);
  a.att_chunks = attend_chunks(infos, n_states);
  a.max_vcols = attend_vcols(infos, n_states);
  a.rec256 = records_256(infos, n_states);
  a.k_new = k_new;
  a.v_new = v_new;
  a.new_f32 = new_f32;
  if (launch_attend(a, stream)) return fail(STC_EDEVICE, "attend launch: %s", hipGetErrorString(hipGetLastError()));
  return ok();
}

stc_status stc_attend_compressed_batched(const void* states_dev, int64_t n_states, const int32_t* k_map,
                                         const int32_t* v_map, const stc_head_info* infos, int64_t n_pairs,
                                         int64_t n_tokens, const void* k_packed_dev, const void* v_packed_dev,
                                         int64_t packed_pair_stride, int32_t group, const float* q_dev,
                                         float* out_dev, float scale, void* ws_dev, size_t ws_bytes,
                                         stc_stream_t stream) {
  return attend_eigen("attend_compressed", states_dev, n_states, k_map, v_map, infos, n_pairs, n_tokens, k_packed_dev,
                      v_packed_dev, packed_pair_stride, group, q_dev, out_dev, scale, ws_dev, ws_bytes, false, stream);
}

stc_status stc_attend_compressed_batched_noalloc(const void* states_dev, int64_t n_states, const int32_t* k_map,
                                                 const int32_t* v_map, const stc_head_info* infos, int64_t n_pairs,
                                                 int64_t n_tokens, const void* k_packed_dev, const void* v_packed_dev,
                                                 int64_t packed_pair_stride, int32_t group, const float* q_dev,
                                                 float* out_dev, float scale, stc_stream_t stream) {
  return attend_eigen("attend_compressed_noalloc", states_dev, n_states, k_map, v_map, infos, n_pairs, n_tokens,
                      k_packed_dev, v_packed_dev, packed_pair_stride, group, q_dev, out_dev, scale, nullptr, 0, true,
                      stream);
}

size_t stc_attend_noalloc_max_bytes(void) { return attend_scratch_bytes(); }

stc_status stc_attend_compressed_sketch_batched(const void* states_dev, int64_t n_states, const int32_t* k_map,
                                                const int32_t* v_map, const stc_head_info* infos, int64_t n_pairs,
                                                int64_t n_tokens, const void* k_packed_dev, const void* v_packed_dev,
                                                int64_t packed_pair_stride, const void* k_sketch_dev,
                                                const float* k_rnorm_dev, int64_t sketch_pair_stride,
                                                int64_t rnorm_pair_stride, int32_t group, const float* q_dev,
                                                float* out_dev, float scale, void* ws_dev, size_t ws_bytes,
                                                stc_stream_t stream) {
  bool rht = false;
  int mb = 0;
  if (stc_status s = check_batch("attend_sketch", states_dev, n_states, infos, n_pairs, n_tokens, packed_pair_stride,
                                 &rht, &mb)) return s;
  if (rht) return fail(STC_EUNSUPPORTED, "attend_sketch: eigen/identity states (Walsh-Hadamard: attend_rht)");
  if (group < 1 || group > 16) return fail(STC_EUNSUPPORTED, "attend_sketch: group %d outside 1..16", group);
  if (n_tokens <= 0) return fail(STC_EINVAL, "attend_sketch: need at least one cached token");
  if (!k_packed_dev || !v_packed_dev || !q_dev || !out_dev || !ws_dev || !k_sketch_dev || !k_rnorm_dev)
    return fail(STC_EINVAL, "attend_sketch: NULL buffer");
  if (!aligned(k_packed_dev, 16) || !aligned(v_packed_dev, 16) || !aligned(q_dev, 16) || !aligned(out_dev, 16) ||
      !aligned(ws_dev, 256) || !aligned(k_sketch_dev, 8) || !aligned(k_rnorm_dev, 4) || sketch_pair_stride % 8)
    return fail(STC_EINVAL, "attend_sketch: misaligned buffer");
  if (n_pairs > 1 && (sketch_pair_stride < n_tokens * (STC_SKETCH_BITS / 8) || rnorm_pair_stride < n_tokens))
    return fail(STC_EINVAL, "attend_sketch: sketch or residual norm stride too small");
  bool any = false;
  for (int64_t i = 0; i < n_states; ++i) any = any || infos[i].sketch_bits == STC_SKETCH_BITS;
  if (!any) return fail(STC_EINVAL, "attend_sketch: no state has a sketch matrix");
  if (!std::isfinite(scale)) return fail(STC_EINVAL, "attend_sketch: scale must be finite");
  const size_t need = stc_attend_workspace_bytes(n_pairs, group, n_tokens);
  if (ws_bytes < need) return fail(STC_EWORKSPACE, "attend_sketch: workspace %zu < %zu", ws_bytes, need);
  const unsigned char* st = static_cast<const unsigned char*>(states_dev);
  AttendLaunch a{st, k_map, st, v_map, n_states, n_pairs, n_tokens, packed_pair_stride,
                 static_cast<const unsigned char*>(k_packed_dev), static_cast<const unsigned char*>(v_packed_dev),
                 group, q_dev, out_dev, scale, static_cast<unsigned char*>(ws_dev), mb, nullptr, nullptr, 0, false,
                 static_cast<const unsigned char*>(k_sketch_dev), k_rnorm_dev, sketch_pair_stride, rnorm_pair_stride};
  a.rec = records_word_pow2(infos, n_states);
  if (launch_attend(a, stream)) return fail(STC_EDEVICE, "attend_sketch launch: %s", hipGetErrorString(hipGetLastError()));
  return ok();
}

stc_status stc_attend_rht_batched(const void* states_dev, int64_t n_states, const int32_t* k_map,
                                  const int32_t* v_map, const stc_head_info* infos, int64_t n_pairs,
                                  int64_t n_tokens, const void* k_packed_dev, const float* k_norms_dev,
                                  const void* v_packed_dev, const float* v_norms_dev, int64_t packed_pair_stride,
                                  int64_t norms_pair_stride, const void* k_sketch_dev, const float* k_rnorm_dev,
                                  int64_t sketch_pair_stride, int64_t rnorm_pair_stride, int32_t group,
                                  const float* q_dev, float* out_dev, float scale, void* ws_dev, size_t ws_bytes,
                                  stc_stream_t stream) {
  bool rht = false;
  int mb = 0;
  if (stc_status s = check_batch("attend_rht", states_dev, n_states, infos, n_pairs, n_tokens, packed_pair_stride,
                                 &rht, &mb)) return s;
  if (!rht) return fail(STC_EUNSUPPORTED, "attend_rht: Walsh-Hadamard states only");
  if (group < 1 || group > 16) return fail(STC_EUNSUPPORTED, "attend_rht: group %d outside 1..16", group);
  if (n_tokens <= 0) return fail(STC_EINVAL, "attend_rht: need at least one cached token");
  if (!k_packed_dev || !v_packed_dev || !k_norms_dev || !v_norms_dev || !q_dev || !out_dev || !ws_dev)
    return fail(STC_EINVAL, "attend_rht: NULL buffer");
  if (!aligned(k_packed_dev, 16) || !aligned(v_packed_dev, 16) || !aligned(q_dev, 16) || !aligned(out_dev, 16) ||
      !aligned(ws_dev, 256) || !aligned(k_norms_dev, 4) || !aligned(v_norms_dev, 4))
    return fail(STC_EINVAL, "attend_rht: misaligned buffer");
  if (n_pairs > 1 && norms_pair_stride < n_tokens)
    return fail(STC_EINVAL, "attend_rht: norms stride %lld < %lld tokens", (long long)norms_pair_stride,
                (long long)n_tokens);
  if (!std::isfinite(scale)) return fail(STC_EINVAL, "attend_rht: scale must be finite");
  if (k_sketch_dev) {
    // the K states need the sketch matrix (V states have none; the maps live on the device,
    // so only its presence in the array is checked: a K state without one adds nothing)
    bool any = false;
    for (int64_t i = 0; i < n_states; ++i) any = any || infos[i].sketch_bits == STC_SKETCH_BITS;
    if (!any) return fail(STC_EINVAL, "attend_rht: a sketch is given but no state has a sketch matrix");
    if (!k_rnorm_dev || !aligned(k_sketch_dev, 8) || !aligned(k_rnorm_dev, 4) || sketch_pair_stride % 8)
      return fail(STC_EINVAL, "attend_rht: sketch needs 8-byte aligned bytes and the residual norms");
    if (n_pairs > 1 && (sketch_pair_stride < n_tokens * (STC_SKETCH_BITS / 8) || rnorm_pair_stride < n_tokens))
      return fail(STC_EINVAL, "attend_rht: sketch or residual norm stride too small");
  }
  const size_t need = stc_attend_workspace_bytes(n_pairs, group, n_tokens);
  if (ws_bytes < need) return fail(STC_EWORKSPACE, "attend_rht: workspace %zu < %zu", ws_bytes, need);
  const unsigned char* st = static_cast<const unsigned char*>(states_dev);
  AttendLaunch a{st, k_map, st, v_map, n_states, n_pairs, n_tokens, packed_pair_stride,
                 static_cast<const unsigned char*>(k_packed_dev), static_cast<const unsigned char*>(v_packed_dev),
                 group, q_dev, out_dev, scale, static_cast<unsigned char*>(ws_dev), mb,
                 k_norms_dev, v_norms_dev, norms_pair_stride, true,
                 static_cast<const unsigned char*>(k_sketch_dev), k_rnorm_dev, sketch_pair_stride, rnorm_pair_stride};
  if (launch_attend(a, stream)) return fail(STC_EDEVICE, "attend_rht launch: %s", hipGetErrorString(hipGetLastError()));
  return ok();
}

stc_status stc_attend_compressed(const stc_head_info* k_info, const void* k_state_dev, const stc_head_info* v_info,
                                 const void* v_state_dev, int64_t n_tokens, const void* k_packed_dev,
                                 const void* v_packed_dev, int32_t group, const float* q_dev, float* out_dev,
                                 float scale, void* ws_dev, size_t ws_bytes, stc_stream_t stream) {
  if (!k_info || !v_info) return fail(STC_EINVAL, "attend_compressed: NULL info");
  bool rht = false;
  int mbk = 0, mbv = 0;
  const int64_t stride = 0;
  if (stc_status s = check_batch("attend_compressed", k_state_dev, 1, k_info, 1, n_tokens, stride, &rht, &mbk)) return s;
  if (rht) return fail(STC_EUNSUPPORTED, "attend_compressed: eigen/identity states only");
  if (stc_status s = check_batch("attend_compressed", v_state_dev, 1, v_info, 1, n_tokens, stride, &rht, &mbv)) return s;
  if (rht) return fail(STC_EUNSUPPORTED, "attend_compressed: eigen/identity states only");
  if (group < 1 || group > 16) return fail(STC_EUNSUPPORTED, "attend_compressed: group %d outside 1..16", group);
  if (n_tokens <= 0) return fail(STC_EINVAL, "attend_compressed: need at least one cached token");
  if (!k_packed_dev || !v_packed_dev || !q_dev || !out_dev || !ws_dev)
    return fail(STC_EINVAL, "attend_compressed: NULL buffer");
  if (!aligned(k_packed_dev, 16) || !aligned(v_packed_dev, 16) || !aligned(q_dev, 16) || !aligned(out_dev, 16) ||
      !aligned(ws_dev, 256))
    return fail(STC_EINVAL, "attend_compressed: misaligned buffer");
  if (!std::isfinite(scale)) return fail(STC_EINVAL, "attend_compressed: scale must be finite");
  const size_t need = stc_attend_workspace_bytes(1, group, n_tokens);
  if (ws_bytes < need) return fail(STC_EWORKSPACE, "attend_compressed: workspace %zu < %zu", ws_bytes, need);
  AttendLaunch a{static_cast<const unsigned char*>(k_state_dev), nullptr, static_cast<const unsigned char*>(v_state_dev),
                 nullptr, 1, 1, n_tokens, 0, static_cast<const unsigned char*>(k_packed_dev),
                 static_cast<const unsigned char*>(v_packed_dev), group, q_dev, out_dev, scale,
                 static_cast<unsigned char*>(ws_dev), std::max(mbk, mbv)};
  a.rec = records_word_pow2(k_info, 1) && records_word_pow2(v_info, 1);
  a.att_chunks = std::max(attend_chunks(k_info, 1), attend_chunks(v_info, 1));
  a.max_vcols = std::max(attend_vcols(k_info, 1), attend_vcols(v_info, 1));
  a.rec256 = records_256(k_info, 1) && records_256(v_info, 1);
  if (launch_attend(a, stream)) return fail(STC_EDEVICE, "attend launch: %s", hipGetErrorString(hipGetLastError()));
  return ok();
}

stc_status stc_decode_step_batched(const void* states_dev, int64_t n_states, const int32_t* k_map,
                                   const int32_t* v_map, const stc_head_info* infos, int64_t n_pairs,
                                   int64_t n_old, const void* k_new_dev, const void* v_new_dev, int32_t dtype,
                                   void* k_packed_dev, void* v_packed_dev, int64_t packed_pair_stride,
                                   int32_t group, const float* q_dev, float* out_dev, float scale, void* ws_dev,
                                   size_t ws_bytes, stc_stream_t stream) {
  bool rht = false;
  int mb = 0;
  if (n_old < 0) return fail(STC_EINVAL, "decode_step: negative token count");
  if (stc_status s = check_batch("decode_step", states_dev, n_states, infos, n_pairs, n_old + 1, packed_pair_stride,
                                 &rht, &mb)) return s;
  if (rht) return fail(STC_EUNSUPPORTED, "decode_step: eigen/identity states only");
  if (group < 1 || group > 16) return fail(STC_EUNSUPPORTED, "decode_step: group %d outside 1..16", group);
  if (!q_dev || !out_dev || !ws_dev) return fail(STC_EINVAL, "decode_step: NULL buffer");
  if (!std::isfinite(scale)) return fail(STC_EINVAL, "decode_step: scale must be finite");
  if (dtype != STC_F32 && dtype != STC_BF16) return fail(STC_EUNSUPPORTED, "decode_step: dtype %d", dtype);
  if (n_pairs > 0 && (!k_new_dev || !v_new_dev)) return fail(STC_EINVAL, "decode_step: NULL new-token rows");
  if (!aligned(k_new_dev, 16) || !aligned(v_new_dev, 16))
    return fail(STC_EINVAL, "decode_step: new-token rows must be 16-byte aligned");
  const size_t need = stc_attend_workspace_bytes(n_pairs, group, n_old + 1);
  if (ws_bytes < need) return fail(STC_EWORKSPACE, "decode_step: workspace %zu < %zu", ws_bytes, need);
  // the new K and V token of every KV head are appended by the attention's
  // first launch, then attention runs over all n_old + 1 tokens
  return attend_eigen("decode_step", states_dev, n_states, k_map, v_map, infos, n_pairs, n_old + 1, k_packed_dev,
                      v_packed_dev, packed_pair_stride, group, q_dev, out_dev, scale, ws_dev, ws_bytes, false, stream,
                      k_new_dev, v_new_dev, dtype == STC_F32 ? 1 : 0);
}

}  // extern "C"
