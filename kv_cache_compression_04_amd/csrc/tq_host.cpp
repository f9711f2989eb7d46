// Host side of libtq: argument checking, the seeded matrices (Pi, S, S'),
// the Lloyd-Max codebook, the per-(parameters, device) cache and the C ABI
// entry points declared in include/tq.h.
//
// The pages describe the method; this file supplies the one-off set-up it
// needs:
//   * "谷歌TurboQuant如何绕过内存墙？重新审视它的技术突破", 第一阶段: a random
//     rotation makes every coordinate follow one known Beta-shaped law, so a
//     Lloyd-Max codebook for that law is computed once and reused.
//   * "TurboQuant 与 AI 效率革命：当旧数学遇到新智能", section 四: a random
//     rotation P (generated once and reused), a JL projection S in R^{m x d}.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <thread>
#include <tuple>
#include <vector>

#include "tq_internal.h"

namespace tq {

// --------------------------------------------------------------------------
// errors
// --------------------------------------------------------------------------
static thread_local std::string g_last_error;

void set_error(const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
}

#define TQ_HIP_CHECK(expr)                                                  \
  do {                                                                      \
    hipError_t e_ = (expr);                                                 \
    if (e_ != hipSuccess) {                                                 \
      set_error("%s failed: %s", #expr, hipGetErrorString(e_));            \
      return TQ_ERR_HIP;                                                    \
    }                                                                       \
  } while (0)

// --------------------------------------------------------------------------
// SplitMix64 (Steele, Lea & Flood 2014): word k of the stream seeded with
// `seed` is mix(seed + (k + 1) * golden_gamma).  Gaussians by Box-Muller on
// word pairs (2p, 2p + 1) for counter pair p; even counter -> cosine branch.
// --------------------------------------------------------------------------
static inline uint64_t sm64(uint64_t seed, uint64_t k) {
  uint64_t z = seed + (k + 1) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static void seeded_gaussian(uint64_t seed, int64_t rows, int64_t cols,
                            std::vector<double> &out) {
  const int64_t n = rows * cols;
  out.assign(n, 0.0);
  const double two53 = 1.0 / 9007199254740992.0;
  for (int64_t c = 0; c < n; c += 2) {
    const uint64_t pair = (uint64_t)c / 2;
    const double u1 = ((double)(sm64(seed, 2 * pair) >> 11) + 1.0) * two53;
    const double u2 = (double)(sm64(seed, 2 * pair + 1) >> 11) * two53;
    const double rad = std::sqrt(-2.0 * std::log(u1));
    const double ang = 2.0 * M_PI * u2;
    out[c] = rad * std::cos(ang);
    if (c + 1 < n) out[c + 1] = rad * std::sin(ang);
  }
}

// --------------------------------------------------------------------------
// Pi: Q of G = QR with diag(R) > 0, by Householder reflections.
// G row-major d x d in, Pi row-major d x d out (y = Pi x).
// --------------------------------------------------------------------------
static void rotation_from_gaussian(int d, const std::vector<double> &g,
                                   std::vector<double> &pi) {
  // column-major working copy: a[j*d + i] = G[i][j]
  std::vector<double> a((size_t)d * d), vs((size_t)d * d, 0.0), rdiag(d);
  for (int i = 0; i < d; ++i)
    for (int j = 0; j < d; ++j) a[(size_t)j * d + i] = g[(size_t)i * d + j];
  for (int k = 0; k < d; ++k) {
    double *col = &a[(size_t)k * d];
    double nrm = 0.0;
    for (int i = k; i < d; ++i) nrm += col[i] * col[i];
    nrm = std::sqrt(nrm);
    const double alpha = col[k] > 0 ? -nrm : nrm;  // reflect away from x0
    double *v = &vs[(size_t)k * d];
    for (int i = k; i < d; ++i) v[i] = col[i];
    v[k] -= alpha;
    double vn = 0.0;
    for (int i = k; i < d; ++i) vn += v[i] * v[i];
    vn = std::sqrt(vn);
    if (vn > 0)
      for (int i = k; i < d; ++i) v[i] /= vn;
    rdiag[k] = alpha;
    // A[k:, j] -= 2 v (v . A[k:, j]) for j >= k
    for (int j = k; j < d; ++j) {
      double *cj = &a[(size_t)j * d];
      double dot = 0.0;
      for (int i = k; i < d; ++i) dot += v[i] * cj[i];
      dot *= 2.0;
      for (int i = k; i < d; ++i) cj[i] -= dot * v[i];
    }
  }
  // Q = H_0 H_1 ... H_{d-1} I, accumulated backwards; column-major q.
  std::vector<double> q((size_t)d * d, 0.0);
  for (int i = 0; i < d; ++i) q[(size_t)i * d + i] = 1.0;
  for (int k = d - 1; k >= 0; --k) {
    const double *v = &vs[(size_t)k * d];
    for (int j = k; j < d; ++j) {
      double *cj = &q[(size_t)j * d];
      double dot = 0.0;
      for (int i = k; i < d; ++i) dot += v[i] * cj[i];
      dot *= 2.0;
      for (int i = k; i < d; ++i) cj[i] -= dot * v[i];
    }
  }
  // positive diagonal: G = (Q D)(D R) with D = sign(diag R)
  pi.assign((size_t)d * d, 0.0);
  for (int j = 0; j < d; ++j) {
    const double s = rdiag[j] < 0 ? -1.0 : 1.0;
    for (int i = 0; i < d; ++i) pi[(size_t)i * d + j] = s * q[(size_t)j * d + i];
  }
}

// --------------------------------------------------------------------------
// Lloyd-Max codebook for f_d(x) ∝ (1-x^2)^((d-3)/2).  Cell masses come from
// the regularised incomplete beta function ((X+1)/2 ~ Beta(a, a),
// a = (d-1)/2), evaluated by its continued fraction (DLMF 8.17.22) with the
// modified Lentz method; cell first moments from the antiderivative
// -C (1-x^2)^((d-1)/2) / (d-1).
// --------------------------------------------------------------------------
typedef long double ld;

static ld ibeta_cf(ld a, ld b, ld y) {
  const ld tiny = 1e-300L, eps = 1e-19L;
  ld f = 1.0L, c = 1.0L, dd = 0.0L;
  for (int i = 0; i <= 4000; ++i) {
    const int m = i / 2;
    ld num;
    if (i == 0) {
      num = 1.0L;
    } else if (i % 2 == 0) {
      num = (m * (b - m) * y) / ((a + 2 * m - 1) * (a + 2 * m));
    } else {
      num = -((a + m) * (a + b + m) * y) / ((a + 2 * m) * (a + 2 * m + 1));
    }
    dd = 1.0L + num * dd;
    if (std::fabs(dd) < tiny) dd = tiny;
    dd = 1.0L / dd;
    c = 1.0L + num / c;
    if (std::fabs(c) < tiny) c = tiny;
    const ld cd = c * dd;
    f *= cd;
    if (std::fabs(1.0L - cd) < eps) break;
  }
  return f - 1.0L;
}

// upper tail P(X >= x) for 0 <= x <= 1 = I_{(1-x)/2}(a, a)
static ld coord_tail(int d, ld x) {
  const ld a = (d - 1) / 2.0L;
  const ld y = (1.0L - x) / 2.0L;
  if (y <= 0) return 0.0L;
  const ld lbeta = std::lgamma(a) + std::lgamma(a) - std::lgamma(2 * a);
  const ld front = std::exp(a * std::log(y) + a * std::log1p(-y) - lbeta) / a;
  return front * ibeta_cf(a, a, y);
}

static ld coord_moment_antider(int d, ld x) {
  const ld logc = std::lgamma(d / 2.0L) - 0.5L * std::log((ld)M_PI) -
                  std::lgamma((d - 1) / 2.0L);
  const ld w = 1.0L - x * x;
  if (w <= 0) return 0.0L;
  return -std::exp(logc + ((d - 1) / 2.0L) * std::log(w)) / (d - 1);
}

static void lloyd_max_codebook(int d, int nbits, std::vector<double> &cent) {
  const int L = 1 << nbits, half = L / 2;
  std::vector<ld> c(half), nc(half), e(half + 1);
  const ld span = std::min<ld>(3.0L / std::sqrt((ld)d), 1.0L);
  for (int j = 0; j < half; ++j) c[j] = (j + 0.5L) * span / half;
  ld prev = 1.0L;
  for (int it = 0; it < 100000; ++it) {
    e[0] = 0.0L;
    e[half] = 1.0L;
    for (int j = 1; j < half; ++j) e[j] = 0.5L * (c[j - 1] + c[j]);
    ld delta = 0.0L;
    for (int j = 0; j < half; ++j) {
      const ld mass = coord_tail(d, e[j]) - coord_tail(d, e[j + 1]);
      const ld mom = coord_moment_antider(d, e[j + 1]) - coord_moment_antider(d, e[j]);
      nc[j] = mom / mass;
      delta = std::max(delta, std::fabs(nc[j] - c[j]));
    }
    c.swap(nc);
    // converged, or stalled at the rounding floor of long double
    if (delta <= 1e-17L * c[half - 1]) break;
    if (delta < 1e-15L * c[half - 1] && delta >= prev) break;
    prev = delta;
  }
  cent.resize(L);
  for (int j = 0; j < half; ++j) {
    cent[half + j] = (double)c[j];
    cent[half - 1 - j] = -(double)c[j];
  }
}

static void build_codebook(int d, int nbits, Codebook &cb) {
  std::memset(&cb, 0, sizeof(cb));
  cb.nbits = nbits;
  if (nbits == 0) return;
  std::vector<double> cent;
  lloyd_max_codebook(d, nbits, cent);
  const int L = 1 << nbits;
  for (int j = 0; j < L; ++j) cb.c[j] = (float)cent[j];
  for (int j = 0; j + 1 < L; ++j)
    cb.t[j] = (float)(0.5 * ((double)cb.c[j] + (double)cb.c[j + 1]));
  cb.t[L / 2 - 1] = 0.0f;
  // c[idx] = sum over odd subsets S of the planes of coef_S * prod_{k in S} sigma_k,
  // sigma_k = 2 bit_k(idx) - 1 (the even subsets vanish because c is odd).
  int np = 0;
  while (np < kMaxParts && part_mask_ct(nbits, np) != 0) {
    cb.part_mask[np] = part_mask_ct(nbits, np);
    ++np;
  }
  cb.nparts = np;
  for (int s = 0; s < np; ++s) {
    double acc = 0.0;
    for (int idx = 0; idx < L; ++idx) {
      int sign = 1;
      for (int k = 0; k < nbits; ++k)
        if (cb.part_mask[s] >> k & 1) sign *= ((idx >> k) & 1) ? 1 : -1;
      acc += sign * (double)cb.c[idx];
    }
    cb.coef[s] = acc / L;
  }
}

// --------------------------------------------------------------------------
// argument checks
// --------------------------------------------------------------------------
static int mse_bits(const tq_params *p) { return p->mode == TQ_MODE_PROD ? p->b - 1 : p->b; }

static tq_status check_params(const tq_params *p) {
  if (!p) {
    set_error("params is NULL");
    return TQ_ERR_INVALID_ARG;
  }
  if (p->mode != TQ_MODE_PROD && p->mode != TQ_MODE_MSE) {
    set_error("mode %d is neither TQ_MODE_PROD nor TQ_MODE_MSE", p->mode);
    return TQ_ERR_INVALID_ARG;
  }
  if (p->d < 128 || p->d > 1024 || p->d % 128) {
    set_error("d = %d: must be a multiple of 128 in [128, 1024]", p->d);
    return p->d > 0 ? TQ_ERR_UNSUPPORTED : TQ_ERR_INVALID_ARG;
  }
  if (p->mode == TQ_MODE_PROD && (p->m < 128 || p->m > 1024 || p->m % 128)) {
    set_error("m = %d: must be a multiple of 128 in [128, 1024]", p->m);
    return p->m > 0 ? TQ_ERR_UNSUPPORTED : TQ_ERR_INVALID_ARG;
  }
  const int B = mse_bits(p);
  if (p->b < 1 || B > 4) {
    set_error("b = %d out of range for mode %d", p->b, p->mode);
    return p->b < 1 ? TQ_ERR_INVALID_ARG : TQ_ERR_UNSUPPORTED;
  }
  return TQ_OK;
}

static bool aligned16(const void *ptr) { return ((uintptr_t)ptr & 15u) == 0; }

// --------------------------------------------------------------------------
// host matrices and device cache
// --------------------------------------------------------------------------
static void host_matrices(const tq_params *p, std::vector<double> *pi,
                          std::vector<double> *s) {
  if (pi) {
    std::vector<double> g;
    seeded_gaussian(p->seed_pi, p->d, p->d, g);
    rotation_from_gaussian(p->d, g, *pi);
  }
  if (s) seeded_gaussian(p->seed_s, p->m, p->d, *s);
}

static uint16_t bf16_bits(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  const uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;  // round to nearest even
  return (uint16_t)(u >> 16);
}

static double bf16_value(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return (double)f;
}

// IEEE binary16 bits of v (round to nearest even, subnormals kept, |v| well
// inside the finite range).
static uint16_t f16_bits(double v) {
  const uint16_t sign = std::signbit(v) ? 0x8000u : 0u;
  double a = std::fabs(v);
  if (a == 0.0) return sign;
  int e;
  std::frexp(a, &e);                                  // a = f 2^e, f in [0.5, 1)
  const int lsb = e - 11 < -24 ? -24 : e - 11;        // weight of the last kept bit
  const double k = std::nearbyint(std::ldexp(a, -lsb));  // exact scaling, RNE
  a = std::ldexp(k, lsb);
  if (a < 0x1p-14) return (uint16_t)(sign | (uint16_t)k);  // subnormal (k < 1024)
  std::frexp(a, &e);
  const uint32_t field = (uint32_t)(e + 14);          // biased exponent of a in [2^(e-1), 2^e)
  const uint32_t mant = (uint32_t)(std::ldexp(a, 11 - e) - 1024.0);
  return (uint16_t)(sign | (field << 10) | mant);
}

static double f16_value(uint16_t h) {
  const int field = (h >> 10) & 31, mant = h & 1023;
  const double a = field == 0 ? std::ldexp((double)mant, -24)
                              : std::ldexp((double)(mant + 1024), field - 25);
  return (h & 0x8000u) ? -a : a;
}

// Split a 128 x 128 row-major double matrix into hi/lo bf16 fragments.
// col_of(kt, lanegroup, e) gives the matrix column that element e of a lane
// in lane group `lanegroup` holds within column block kt.
template <typename ColOf>
static void make_fragments(const std::vector<double> &mat, ColOf col_of,
                           std::vector<uint16_t> &hi, std::vector<uint16_t> &lo) {
  hi.assign(kFragElems, 0);
  lo.assign(kFragElems, 0);
  size_t o = 0;
  for (int nt = 0; nt < 8; ++nt)
    for (int kt = 0; kt < 4; ++kt)
      for (int l = 0; l < 64; ++l)
        for (int e = 0; e < 8; ++e, ++o) {
          const int row = 16 * nt + (l & 15);
          const int col = col_of(kt, l >> 4, e);
          const double v = mat[(size_t)row * 128 + col];
          const uint16_t h = bf16_bits((float)v);
          hi[o] = h;
          lo[o] = bf16_bits((float)(v - bf16_value(h)));
        }
}

// The same fragment order with scale * mat split into fp16 hi + lo (the hi
// part keeps 11 significant bits, the lo part the next 11, so hi + lo carries
// scale * mat to about 2^-23 relative; the encode kernels take the power of
// two `scale` back out of their results).
template <typename ColOf>
static void make_fragments_f16(const std::vector<double> &mat, double scale, ColOf col_of,
                               std::vector<uint16_t> &hi, std::vector<uint16_t> &lo) {
  hi.assign(kFragElems, 0);
  lo.assign(kFragElems, 0);
  size_t o = 0;
  for (int nt = 0; nt < 8; ++nt)
    for (int kt = 0; kt < 4; ++kt)
      for (int l = 0; l < 64; ++l)
        for (int e = 0; e < 8; ++e, ++o) {
          const int row = 16 * nt + (l & 15);
          const int col = col_of(kt, l >> 4, e);
          const double v = scale * mat[(size_t)row * 128 + col];
          const uint16_t h = f16_bits(v);
          hi[o] = h;
          lo[o] = f16_bits(v - f16_value(h));
        }
}

// Split kEncScale * (an R x K row-major double matrix) into the general-shape
// GEMM fragments, fp16 hi + lo: uint4 [K/32 block kt][R/16 tile nt][hi, lo][lane],
// element e of lane l = mat[16 nt + l % 16][col_of(kt, l / 16, e)].
template <typename ColOf>
static void make_gemm_fragments(const std::vector<double> &mat, int R, int K, ColOf col_of,
                                std::vector<uint4> &out) {
  const int NT = R / 16, KT = K / 32;
  out.assign((size_t)KT * NT * 2 * 64, make_uint4(0, 0, 0, 0));
  for (int kt = 0; kt < KT; ++kt)
    for (int nt = 0; nt < NT; ++nt)
      for (int l = 0; l < 64; ++l) {
        uint16_t h[8], lo[8];
        for (int e = 0; e < 8; ++e) {
          const double v = kEncScale * mat[(size_t)(16 * nt + (l & 15)) * K + col_of(kt, l >> 4, e)];
          h[e] = f16_bits(v);
          lo[e] = f16_bits(v - f16_value(h[e]));
        }
        uint4 vh, vl;
        std::memcpy(&vh, h, 16);
        std::memcpy(&vl, lo, 16);
        const size_t o = (((size_t)kt * NT + nt) * 2) * 64 + l;
        out[o] = vh;
        out[o + 64] = vl;
      }
}

template <typename T>
static tq_status upload(T **dst, const std::vector<T> &src) {
  TQ_HIP_CHECK(hipMalloc((void **)dst, src.size() * sizeof(T)));
  TQ_HIP_CHECK(hipMemcpy(*dst, src.data(), src.size() * sizeof(T), hipMemcpyHostToDevice));
  return TQ_OK;
}

static tq_status build_derived(const tq_params *p, int dev, Derived *D) {
  D->p = *p;
  D->device = dev;
  D->B = mse_bits(p);
  build_codebook(p->d, D->B, D->cb);
  const bool prod = p->mode == TQ_MODE_PROD;
  std::vector<double> pi, s;
  host_matrices(p, &pi, prod ? &s : nullptr);
  std::vector<float> f(pi.begin(), pi.end());
  tq_status st = upload(&D->pi32, f);
  if (st) return st;
  if ((st = upload(&D->pi64, pi))) return st;
  if (prod) {
    f.assign(s.begin(), s.end());
    if ((st = upload(&D->s32, f))) return st;
    if ((st = upload(&D->s64, s))) return st;
  }
  // S' = S Pi^T (m x d): the second projection acts on the residual in the
  // rotated domain, S r = S Pi^T (Pi r)
  std::vector<double> sp;
  if (prod) {
    const int d = p->d, m = p->m;
    sp.assign((size_t)m * d, 0.0);
    for (int r = 0; r < m; ++r)
      for (int c = 0; c < d; ++c) {
        double acc = 0.0;
        for (int j = 0; j < d; ++j) acc += s[(size_t)r * d + j] * pi[(size_t)c * d + j];
        sp[(size_t)r * d + c] = acc;
      }
  }
  if (is_d128(*p)) {
    std::vector<uint16_t> hi, lo;
    // GEMM 1 (Pi x): element e of lane group g in block kt is column 32 kt + 8 g + e
    const auto col1 = [](int kt, int g, int e) { return 32 * kt + 8 * g + e; };
    make_fragments_f16(pi, kEncScale, col1, hi, lo);
    if ((st = upload(&D->pi16_hi, hi)) || (st = upload(&D->pi16_lo, lo))) return st;
    // (bf16 split of Pi for the PolarQuant encoder)
    make_fragments(pi, col1, hi, lo);
    if ((st = upload(&D->pi_hi, hi)) || (st = upload(&D->pi_lo, lo))) return st;
    if (prod) {
      // S' is consumed against the residual held in the layout of the first
      // GEMM's output: element e of lane group g in block kt is coordinate
      // 32 kt + 16 (e / 4) + 4 g + e % 4.
      make_fragments_f16(sp, kEncScale,
                         [](int kt, int g, int e) { return 32 * kt + 16 * (e / 4) + 4 * g + e % 4; }, hi,
                         lo);
      if ((st = upload(&D->sp16_hi, hi)) || (st = upload(&D->sp16_lo, lo))) return st;
    }
    // column sums of Pi and S and the largest row norm of S
    std::vector<float> qs(256, 0.f);
    double smax = 0.0;
    for (int c = 0; c < 128; ++c) {
      double a = 0.0, b = 0.0;
      for (int r = 0; r < 128; ++r) {
        a += pi[(size_t)r * 128 + c];
        if (prod) b += s[(size_t)r * 128 + c];
      }
      qs[c] = (float)a;
      qs[128 + c] = (float)b;
    }
    if (prod)
      for (int r = 0; r < 128; ++r) {
        double n2 = 0.0;
        for (int c = 0; c < 128; ++c) n2 += s[(size_t)r * 128 + c] * s[(size_t)r * 128 + c];
        smax = std::max(smax, std::sqrt(n2));
      }
    D->smax = std::nextafter((float)smax, INFINITY);  // a bound: never below the true norm
    if ((st = upload(&D->qsums, qs))) return st;
    // the query preparation's matrix, column-major: qmat[c][r] = Pi[r][c]
    // for r < 128 and S[r - 128][c] for r >= 128 (zero in mse mode), so the
    // threads of one column read one contiguous kilobyte
    std::vector<float> qm((size_t)128 * 256, 0.f);
    for (int c = 0; c < 128; ++c)
      for (int r = 0; r < 128; ++r) {
        qm[(size_t)c * 256 + r] = (float)pi[(size_t)r * 128 + c];
        if (prod) qm[(size_t)c * 256 + 128 + r] = (float)s[(size_t)r * 128 + c];
      }
    if ((st = upload(&D->qmat, qm))) return st;
  } else {
    // same column maps, general shapes, K-block-major fragments
    std::vector<uint4> fr;
    make_gemm_fragments(pi, p->d, p->d, [](int kt, int g, int e) { return 32 * kt + 8 * g + e; }, fr);
    if ((st = upload(&D->pi_frag, fr))) return st;
    if (prod) {
      make_gemm_fragments(sp, p->m, p->d,
                          [](int kt, int g, int e) { return 32 * kt + 16 * (e / 4) + 4 * g + e % 4; }, fr);
      if ((st = upload(&D->sp_frag, fr))) return st;
    }
  }
  return TQ_OK;
}

static void free_derived(Derived *D) {
  int cur = 0;
  (void)hipGetDevice(&cur);
  (void)hipSetDevice(D->device);
  (void)hipFree(D->pi32);
  (void)hipFree(D->s32);
  (void)hipFree(D->pi64);
  (void)hipFree(D->s64);
  (void)hipFree(D->pi_hi);
  (void)hipFree(D->pi_lo);
  (void)hipFree(D->pi16_hi);
  (void)hipFree(D->pi16_lo);
  (void)hipFree(D->sp16_hi);
  (void)hipFree(D->sp16_lo);
  (void)hipFree(D->qsums);
  (void)hipFree(D->qmat);
  (void)hipFree(D->pi_frag);
  (void)hipFree(D->sp_frag);
  (void)hipSetDevice(cur);
  delete D;
}

typedef std::tuple<int, int, int, int, uint64_t, uint64_t, int> CacheKey;
static std::mutex g_cache_mu;
static std::map<CacheKey, Derived *> g_cache;

const Derived *find_derived(const tq_params *p) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  const int m = p->mode == TQ_MODE_PROD ? p->m : 0;
  const uint64_t ss = p->mode == TQ_MODE_PROD ? p->seed_s : 0;
  CacheKey key(p->d, p->b, m, p->mode, p->seed_pi, ss, dev);
  std::lock_guard<std::mutex> lock(g_cache_mu);
  auto it = g_cache.find(key);
  return it == g_cache.end() ? nullptr : it->second;
}

tq_status get_derived(const tq_params *p, const Derived **out) {
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev <= 0) {
    set_error("no HIP device available");
    return TQ_ERR_HIP;
  }
  int dev = 0;
  TQ_HIP_CHECK(hipGetDevice(&dev));
  const int m = p->mode == TQ_MODE_PROD ? p->m : 0;
  const uint64_t ss = p->mode == TQ_MODE_PROD ? p->seed_s : 0;
  CacheKey key(p->d, p->b, m, p->mode, p->seed_pi, ss, dev);
  std::lock_guard<std::mutex> lock(g_cache_mu);
  auto it = g_cache.find(key);
  if (it != g_cache.end()) {
    *out = it->second;
    return TQ_OK;
  }
  Derived *D = new Derived();
  tq_status st = build_derived(p, dev, D);
  if (st != TQ_OK) {
    free_derived(D);
    return st;
  }
  g_cache[key] = D;
  *out = D;
  return TQ_OK;
}


}  // namespace tq

// ============================================================================
// C ABI
namespace tq {

// --------------------------------------------------------------------------
// PolarQuant codebooks.  Level 1: the angle of a coordinate pair is uniform on
// [0, 2 pi), whose Lloyd-Max quantiser is the uniform grid.  Level l >= 2:
// the angle between two radii of k = 2^(l-1) coordinates each has density
// Gamma(k) / (2^(k-2) Gamma(k/2)^2) sin^(k-1)(2 theta) on [0, pi/2]; the
// Lloyd-Max iteration takes cell masses and first moments by composite
// Simpson quadrature in long double.
// --------------------------------------------------------------------------
static ld polar_pdf(int k, ld t) {
  const ld s = std::sin(2.0L * t);
  if (s <= 0.0L) return k == 1 ? std::exp(std::lgamma(1.0L) + std::log(2.0L) - 2.0L * std::lgamma(0.5L)) : 0.0L;
  const ld logc = std::lgamma((ld)k) - (k - 2) * std::log(2.0L) - 2.0L * std::lgamma(k / 2.0L);
  return std::exp(logc + (k - 1) * std::log(s));
}

static void polar_cell(int k, ld a, ld b, ld &m0, ld &m1) {
  const int n = 2048;  // even
  const ld h = (b - a) / n;
  ld s0 = 0.0L, s1 = 0.0L;
  for (int i = 0; i <= n; ++i) {
    const ld t = a + h * i;
    const ld w = (i == 0 || i == n) ? 1.0L : (i % 2 ? 4.0L : 2.0L);
    const ld f = polar_pdf(k, t);
    s0 += w * f;
    s1 += w * t * f;
  }
  m0 = s0 * h / 3.0L;
  m1 = s1 * h / 3.0L;
}

static void polar_codebook(int level, int nbits, std::vector<double> &cent, std::vector<double> &bnd) {
  const int L = 1 << nbits;
  cent.assign(L, 0.0);
  bnd.assign(L - 1, 0.0);
  const ld pi = 3.14159265358979323846264338327950288L;
  if (level == 1) {
    const ld step = 2.0L * pi / L;
    for (int j = 0; j < L; ++j) cent[j] = (double)((j + 0.5L) * step);
    for (int j = 1; j < L; ++j) bnd[j - 1] = (double)(j * step);
    return;
  }
  const int k = 1 << (level - 1);
  const ld lo = 0.0L, hi = pi / 2.0L;
  // start: equal steps over pi/4 +- 2 standard deviations of the law
  ld m0, m1, var = 0.0L;
  {
    const int n = 4096;
    const ld h = (hi - lo) / n;
    for (int i = 0; i <= n; ++i) {
      const ld t = lo + h * i;
      const ld w = (i == 0 || i == n) ? 1.0L : (i % 2 ? 4.0L : 2.0L);
      var += w * (t - pi / 4) * (t - pi / 4) * polar_pdf(k, t);
    }
    var *= h / 3.0L;
  }
  const ld half = std::min<ld>(2.0L * std::sqrt(var), pi / 4);
  std::vector<ld> c(L), nc(L), e(L + 1);
  for (int j = 0; j < L; ++j) c[j] = pi / 4 - half + (2.0L * half) * (j + 0.5L) / L;
  ld prev = 1.0L;
  for (int it = 0; it < 100000; ++it) {
    e[0] = lo;
    e[L] = hi;
    for (int j = 1; j < L; ++j) e[j] = 0.5L * (c[j - 1] + c[j]);
    ld delta = 0.0L;
    for (int j = 0; j < L; ++j) {
      polar_cell(k, e[j], e[j + 1], m0, m1);
      nc[j] = m1 / m0;
      delta = std::max(delta, std::fabs(nc[j] - c[j]));
    }
    c.swap(nc);
    if (delta <= 1e-17L) break;
    if (delta < 1e-14L && delta >= prev) break;
    prev = delta;
  }
  for (int j = 0; j < L; ++j) cent[j] = (double)c[j];
  for (int j = 1; j < L; ++j) bnd[j - 1] = 0.5 * (cent[j - 1] + cent[j]);
}

// Kernel constants for d = 128, bits1 = 4, bits = 2 (built once).
static const PolarTables &polar_tables() {
  static PolarTables T;
  static std::once_flag once;
  std::call_once(once, [] {
    std::memset(&T, 0, sizeof(T));
    std::vector<double> c, b;
    polar_codebook(1, 4, c, b);
    for (int j = 0; j < 16; ++j) {
      T.c1[j] = (float)std::cos(c[j]);
      T.s1[j] = (float)std::sin(c[j]);
    }
    for (int j = 0; j < 3; ++j) {  // boundaries pi/8, pi/4, 3 pi/8 inside a quadrant
      T.dc1[j] = (float)std::cos(b[j]);
      T.ds1[j] = (float)std::sin(b[j]);
    }
    T.tau1[0] = (float)std::tan(b[0]);
    T.tau1[1] = (float)std::tan(b[2]);
    for (int lev = 2; lev <= 7; ++lev) {
      polar_codebook(lev, 2, c, b);
      const double tb = std::tan(b[0]);
      T.tau[lev - 2] = (float)(tb * tb);
      for (int j = 0; j < 4; ++j) {
        T.cl[lev - 2][j] = (float)std::cos(c[j]);
        T.sl[lev - 2][j] = (float)std::sin(c[j]);
      }
      for (int j = 0; j < 3; ++j) {
        const double cj = std::cos(b[j]), sj = std::sin(b[j]);
        T.dC[lev - 2][j] = (float)(cj * cj);
        T.dS[lev - 2][j] = (float)(sj * sj);
      }
    }
  });
  return T;
}

// The tables on the current device (uploaded on first use, freed by
// tq_release_cache).
static std::mutex g_polar_mu;
static std::map<int, PolarTables *> g_polar_dev;

static tq_status polar_tables_device(const PolarTables **out) {
  int dev = 0;
  TQ_HIP_CHECK(hipGetDevice(&dev));
  const PolarTables &host = polar_tables();
  std::lock_guard<std::mutex> lock(g_polar_mu);
  auto it = g_polar_dev.find(dev);
  if (it == g_polar_dev.end()) {
    PolarTables *d = nullptr;
    TQ_HIP_CHECK(hipMalloc((void **)&d, sizeof(PolarTables)));
    const hipError_t e = hipMemcpy(d, &host, sizeof(PolarTables), hipMemcpyHostToDevice);
    if (e != hipSuccess) {
      (void)hipFree(d);
      set_error("hipMemcpy of the polar tables failed: %s", hipGetErrorString(e));
      return TQ_ERR_HIP;
    }
    it = g_polar_dev.emplace(dev, d).first;
  }
  *out = it->second;
  return TQ_OK;
}

static void polar_tables_release() {
  std::lock_guard<std::mutex> lock(g_polar_mu);
  for (auto &kv : g_polar_dev) {
    int cur = 0;
    (void)hipGetDevice(&cur);
    (void)hipSetDevice(kv.first);
    (void)hipFree(kv.second);
    (void)hipSetDevice(cur);
  }
  g_polar_dev.clear();
}

static tq_status check_polar(const tq_polar_params *p, const char *fn) {
  if (!p) {
    set_error("%s: params is NULL", fn);
    return TQ_ERR_INVALID_ARG;
  }
  if (p->d < 4 || (p->d & (p->d - 1)) || p->bits1 < 1 || p->bits1 > 6 || p->bits < 1 || p->bits > 6 ||
      p->reserved != 0) {
    set_error("%s: need d a power of two >= 4, 1 <= bits1, bits <= 6, reserved = 0", fn);
    return TQ_ERR_INVALID_ARG;
  }
  if (p->d != 128 || p->bits1 != 4 || p->bits != 2) {
    set_error("%s: device kernels are built for d = 128, bits1 = 4, bits = 2", fn);
    return TQ_ERR_UNSUPPORTED;
  }
  return TQ_OK;
}

// the TurboQuant parameters whose cache entry holds the rotation of seed_pi
static tq_params polar_rotation_params(const tq_polar_params *p) {
  tq_params t;
  t.d = p->d;
  t.b = 1;
  t.m = 128;
  t.mode = TQ_MODE_MSE;
  t.seed_pi = p->seed_pi;
  t.seed_s = 0;
  return t;
}

// --------------------------------------------------------------------------
// Mixed bit widths: two TurboQuant groups of one head (d = 128), the n_out
// outlier channels and the rest.
// --------------------------------------------------------------------------
static int split_n_out(const tq_split_params *p) { return p->n_out == 0 ? 64 : p->n_out; }

static tq_status check_split(const tq_split_params *p, const char *fn) {
  if (!p) {
    set_error("%s: params is NULL", fn);
    return TQ_ERR_INVALID_ARG;
  }
  if (p->b_out != p->b_rest + 1 || p->b_rest < 1 || p->b_rest > 4) {
    set_error("%s: need b_out = b_rest + 1, 1 <= b_rest <= 4", fn);
    return TQ_ERR_INVALID_ARG;
  }
  if (p->n_out != 0 && (p->n_out <= 0 || p->n_out >= 128 || p->n_out % 32 != 0)) {
    set_error("%s: n_out must be 32, 64 or 96 (0 selects 64)", fn);
    return TQ_ERR_INVALID_ARG;
  }
  if (p->d != 128) {
    set_error("%s: built for d = 128", fn);
    return TQ_ERR_UNSUPPORTED;
  }
  bool seen[128] = {false};
  for (int i = 0; i < 128; ++i) {
    const int c = p->channels[i];
    if (c < 0 || c >= 128 || seen[c]) {
      set_error("%s: channels must be a permutation of 0 .. 127", fn);
      return TQ_ERR_INVALID_ARG;
    }
    seen[c] = true;
  }
  if (p->b_rest != 2 && p->b_rest != 3) {
    set_error("%s: device kernels are built for b_rest = 2 or 3", fn);
    return TQ_ERR_UNSUPPORTED;
  }
  return TQ_OK;
}

static tq_status build_split(const tq_split_params *p, int dev, SplitDerived *D) {
  D->device = dev;
  const int b[2] = {p->b_out, p->b_rest};
  D->DG[0] = split_n_out(p);
  D->DG[1] = 128 - D->DG[0];
  const size_t cb_off = split_codebook_offset(D->DG);
  std::vector<float> mat(cb_off + 32, 0.f), proj(256 * 128, 0.f);
  size_t moff[2][2];  // offsets of Pi_g and S'_g in mat
  moff[0][0] = 0;
  moff[0][1] = (size_t)D->DG[0] * D->DG[0];
  moff[1][0] = 2 * moff[0][1];
  moff[1][1] = moff[1][0] + (size_t)D->DG[1] * D->DG[1];
  for (int g = 0; g < 2; ++g) {
    const int n = D->DG[g], coff = g ? D->DG[0] : 0;
    D->B[g] = b[g] - 1;  // prod mode: b - 1 Lloyd-Max bits + the QJL bit
    std::vector<double> gs, pi, sm;
    seeded_gaussian(p->seed_pi + g, n, n, gs);
    rotation_from_gaussian(n, gs, pi);
    seeded_gaussian(p->seed_s + g, n, n, sm);
    for (int r = 0; r < n; ++r)
      for (int k = 0; k < n; ++k) {
        mat[moff[g][0] + (size_t)r * n + k] = (float)pi[(size_t)r * n + k];
        double sp = 0.0;  // S' = S Pi^T: S r = S' (Pi r)
        for (int j = 0; j < n; ++j) sp += sm[(size_t)r * n + j] * pi[(size_t)k * n + j];
        mat[moff[g][1] + (size_t)r * n + k] = (float)sp;
        const int ch = p->channels[coff + k];
        proj[(size_t)(coff + r) * 128 + ch] = (float)pi[(size_t)r * n + k];
        proj[(size_t)(128 + coff + r) * 128 + ch] = (float)sm[(size_t)r * n + k];
      }
    Codebook cb;
    build_codebook(n, D->B[g], cb);
    for (int j = 0; j < (1 << D->B[g]); ++j) mat[cb_off + 8 * g + j] = cb.c[j];
    for (int j = 0; j + 1 < (1 << D->B[g]); ++j) mat[cb_off + 16 + 8 * g + j] = cb.t[j];
  }
  // bf16 hi / lo fragments of each group's matrices for the encode MFMAs:
  // [nt (DG/16)][kt (DG/32)][lane (64)][e (8)], element (lane, e) =
  // M[16 nt + lane % 16][col(kt, lane / 16, e)].  Pi: col = 32 kt + 8 g + e
  // (the gathered keys); S': col = 32 kt + 16 (e / 4) + 4 g + e % 4 (the
  // residual in the layout of the first product's output); g = lane / 16.
  std::vector<uint16_t> frag;
  for (int g = 0; g < 2; ++g) {
    const int n = D->DG[g];
    for (int m = 0; m < 2; ++m) {
      const float *src = &mat[moff[g][m]];
      std::vector<uint16_t> hi, lo;
      for (int nt = 0; nt < n / 16; ++nt)
        for (int kt = 0; kt < n / 32; ++kt)
          for (int l = 0; l < 64; ++l)
            for (int e = 0; e < 8; ++e) {
              const int gg = l >> 4;
              const int col = m == 0 ? 32 * kt + 8 * gg + e : 32 * kt + 16 * (e / 4) + 4 * gg + e % 4;
              const double v = src[(size_t)(16 * nt + (l & 15)) * n + col];
              const uint16_t h = bf16_bits((float)v);
              hi.push_back(h);
              lo.push_back(bf16_bits((float)(v - bf16_value(h))));
            }
      frag.insert(frag.end(), hi.begin(), hi.end());
      frag.insert(frag.end(), lo.begin(), lo.end());
    }
  }
  std::vector<int32_t> ch(p->channels, p->channels + 128);
  tq_status st;
  if ((st = upload(&D->mat, mat)) || (st = upload(&D->proj, proj)) || (st = upload(&D->chan, ch)) ||
      (st = upload(&D->frag, frag)))
    return st;
  return TQ_OK;
}

static std::mutex g_split_mu;
static std::map<std::pair<std::string, int>, SplitDerived *> g_split;

static tq_status get_split(const tq_split_params *p, const SplitDerived **out) {
  int dev = 0;
  TQ_HIP_CHECK(hipGetDevice(&dev));
  const std::string key(reinterpret_cast<const char *>(p), sizeof(tq_split_params));
  std::lock_guard<std::mutex> lock(g_split_mu);
  auto it = g_split.find({key, dev});
  if (it == g_split.end()) {
    SplitDerived *D = new SplitDerived();
    const tq_status st = build_split(p, dev, D);
    if (st) {
      (void)hipFree(D->mat);
      (void)hipFree(D->proj);
      (void)hipFree(D->chan);
      (void)hipFree(D->frag);
      delete D;
      return st;
    }
    it = g_split.emplace(std::make_pair(key, dev), D).first;
  }
  *out = it->second;
  return TQ_OK;
}

static void split_release() {
  std::lock_guard<std::mutex> lock(g_split_mu);
  int cur = 0;
  (void)hipGetDevice(&cur);
  for (auto &kv : g_split) {
    (void)hipSetDevice(kv.first.second);
    (void)hipFree(kv.second->mat);
    (void)hipFree(kv.second->proj);
    (void)hipFree(kv.second->chan);
    (void)hipFree(kv.second->frag);
    delete kv.second;
  }
  (void)hipSetDevice(cur);
  g_split.clear();
}

}  // namespace tq

// ============================================================================
using namespace tq;

extern "C" {

const char *tq_status_string(tq_status s) {
  switch (s) {
    case TQ_OK: return "TQ_OK";
    case TQ_ERR_INVALID_ARG: return "TQ_ERR_INVALID_ARG";
    case TQ_ERR_UNSUPPORTED: return "TQ_ERR_UNSUPPORTED";
    case TQ_ERR_ALIGNMENT: return "TQ_ERR_ALIGNMENT";
    case TQ_ERR_HIP: return "TQ_ERR_HIP";
    case TQ_ERR_NO_MEMORY: return "TQ_ERR_NO_MEMORY";
  }
  return "TQ_ERR_UNKNOWN";
}

const char *tq_last_error(void) { return g_last_error.c_str(); }

int32_t tq_layout_version(void) { return TQ_LAYOUT_VERSION; }

tq_status tq_make_codebook(int32_t d, int32_t b, int32_t mode, float *centroids,
                           float *boundaries) {
  if (mode != TQ_MODE_PROD && mode != TQ_MODE_MSE) {
    set_error("bad mode %d", mode);
    return TQ_ERR_INVALID_ARG;
  }
  const int B = mode == TQ_MODE_PROD ? b - 1 : b;
  if (d < 3 || b < 1 || B > 4) {
    set_error("tq_make_codebook: d = %d, b = %d out of range", d, b);
    return TQ_ERR_INVALID_ARG;
  }
  if (B == 0) return TQ_OK;
  if (!centroids || !boundaries) {
    set_error("tq_make_codebook: NULL output");
    return TQ_ERR_INVALID_ARG;
  }
  Codebook cb;
  build_codebook(d, B, cb);
  std::memcpy(centroids, cb.c, sizeof(float) * (1 << B));
  std::memcpy(boundaries, cb.t, sizeof(float) * ((1 << B) - 1));
  return TQ_OK;
}

tq_status tq_codes_bytes(const tq_params *p, int64_t n, size_t out[4]) {
  tq_status st = check_params(p);
  if (st) return st;
  if (n < 0 || !out) {
    set_error("tq_codes_bytes: n < 0 or NULL output");
    return TQ_ERR_INVALID_ARG;
  }
  const int B = mse_bits(p);
  const bool prod = p->mode == TQ_MODE_PROD;
  out[0] = (size_t)n * (p->d / 32) * B * 4;
  out[1] = prod ? (size_t)n * (p->m / 32) * 4 : 0;
  out[2] = (size_t)n * 4;
  out[3] = prod ? (size_t)n * 4 : 0;
  return TQ_OK;
}

tq_status tq_export_matrices(const tq_params *p, float *pi, float *s) {
  tq_status st = check_params(p);
  if (st) return st;
  std::vector<double> vpi, vs;
  const bool prod = p->mode == TQ_MODE_PROD;
  host_matrices(p, pi ? &vpi : nullptr, (s && prod) ? &vs : nullptr);
  if (pi)
    for (size_t i = 0; i < vpi.size(); ++i) pi[i] = (float)vpi[i];
  if (s && prod)
    for (size_t i = 0; i < vs.size(); ++i) s[i] = (float)vs[i];
  return TQ_OK;
}

static tq_status check_codes(const tq_params *p, const tq_codes &c) {
  const bool prod = p->mode == TQ_MODE_PROD;
  const int B = p->mode == TQ_MODE_PROD ? p->b - 1 : p->b;
  if ((B > 0 && !c.idx) || !c.knorm || (prod && (!c.sgn || !c.rnorm))) {
    set_error("code array missing");
    return TQ_ERR_INVALID_ARG;
  }
  if ((B > 0 && !aligned16(c.idx)) || !aligned16(c.knorm) ||
      (prod && (!aligned16(c.sgn) || !aligned16(c.rnorm)))) {
    set_error("code arrays must be 16-byte aligned");
    return TQ_ERR_ALIGNMENT;
  }
  return TQ_OK;
}

tq_status tq_encode_workspace_bytes(const tq_params *p, int64_t n, size_t *bytes) {
  tq_status st = check_params(p);
  if (st) return st;
  if (n < 0 || !bytes) {
    set_error("tq_encode_workspace_bytes: n < 0 or NULL output");
    return TQ_ERR_INVALID_ARG;
  }
  *bytes = encode_workspace_bytes(*p, n);
  return TQ_OK;
}

tq_status tq_encode(const tq_params *p, const void *x, int32_t dtype, int64_t n,
                    tq_codes codes, void *workspace, size_t ws_bytes, void *stream) {
  tq_status st = check_params(p);
  if (st) return st;
  if (n < 0 || (dtype != TQ_F32 && dtype != TQ_BF16)) {
    set_error("tq_encode: n < 0 or bad dtype");
    return TQ_ERR_INVALID_ARG;
  }
  if (n == 0) return TQ_OK;
  if (!x) {
    set_error("tq_encode: x is NULL");
    return TQ_ERR_INVALID_ARG;
  }
  if ((st = check_codes(p, codes))) return st;
  if (!aligned16(x) || (workspace && !aligned16(workspace))) {
    set_error("tq_encode: x and workspace must be 16-byte aligned");
    return TQ_ERR_ALIGNMENT;
  }
  const size_t need = encode_workspace_bytes(*p, n);
  if (need > 0 && (!workspace || ws_bytes < need)) {
    set_error("tq_encode: workspace too small (%zu < %zu)", workspace ? ws_bytes : (size_t)0, need);
    return TQ_ERR_NO_MEMORY;
  }
  const Derived *D = nullptr;
  if ((st = get_derived(p, &D))) return st;
  return launch_encode(*D, x, dtype, n, codes, workspace, ws_bytes, (hipStream_t)stream);
}

tq_status tq_score_workspace_bytes(const tq_params *p, int64_t n_kv, int64_t g,
                                   size_t *bytes) {
  tq_status st = check_params(p);
  if (st) return st;
  if (n_kv < 0 || g < 1 || !bytes) {
    set_error("tq_score_workspace_bytes: bad n_kv/g/bytes");
    return TQ_ERR_INVALID_ARG;
  }
  *bytes = score_workspace_bytes(*p, n_kv, g);
  return TQ_OK;
}

tq_status tq_score(const tq_params *p, const float *q, int64_t n_kv, int64_t g,
                   tq_codes codes, int64_t seq, float *logits, void *workspace,
                   size_t ws_bytes, void *stream) {
  tq_status st = check_params(p);
  if (st) return st;
  if (n_kv < 0 || g < 1 || seq < 0) {
    set_error("tq_score: bad n_kv/g/seq");
    return TQ_ERR_INVALID_ARG;
  }
  if (n_kv == 0 || seq == 0) return TQ_OK;
  if (!q || !logits || !workspace) {
    set_error("tq_score: NULL q/logits/workspace");
    return TQ_ERR_INVALID_ARG;
  }
  if ((st = check_codes(p, codes))) return st;
  if (!aligned16(q) || !aligned16(logits) || !aligned16(workspace)) {
    set_error("tq_score: pointers must be 16-byte aligned");
    return TQ_ERR_ALIGNMENT;
  }
  if (ws_bytes < score_workspace_bytes(*p, n_kv, g)) {
    set_error("tq_score: workspace too small (%zu < %zu)", ws_bytes,
              score_workspace_bytes(*p, n_kv, g));
    return TQ_ERR_NO_MEMORY;
  }
  const Derived *D = nullptr;
  if ((st = get_derived(p, &D))) return st;
  return launch_score(*D, q, n_kv, g, codes, seq, logits, workspace, (hipStream_t)stream);
}

tq_status tq_attend_workspace_bytes(const tq_params *kp, const tq_params *vp,
                                    int64_t batch, int64_t n_kv, int64_t g,
                                    int64_t seq, size_t *bytes) {
  tq_status st = check_params(kp);
  if (st) return st;
  if ((st = check_params(vp))) return st;
  if (batch < 0 || n_kv < 0 || g < 1 || seq < 0 || !bytes) {
    set_error("tq_attend_workspace_bytes: bad sizes");
    return TQ_ERR_INVALID_ARG;
  }
  Derived K, V;
  K.p = *kp;
  K.B = mse_bits(kp);
  K.cb.nparts = K.B == 0 ? 0 : (K.B == 1 ? 1 : K.B == 2 ? 2 : K.B == 3 ? 4 : 8);
  V.p = *vp;
  V.B = mse_bits(vp);
  V.cb.nparts = V.B == 0 ? 0 : (V.B == 1 ? 1 : V.B == 2 ? 2 : V.B == 3 ? 4 : 8);
  *bytes = attend_workspace_bytes(K, V, batch, n_kv, g, seq);
  return TQ_OK;
}

tq_status tq_attend(const tq_params *kp, const tq_params *vp, const float *q,
                    int64_t batch, int64_t n_kv, int64_t g, tq_codes kcodes,
                    tq_codes vcodes, int64_t seq, float scale, float *out,
                    void *workspace, size_t ws_bytes, void *stream) {
  tq_status st = check_params(kp);
  if (st) return st;
  if ((st = check_params(vp))) return st;
  if (kp->mode != TQ_MODE_PROD || vp->mode != TQ_MODE_MSE || kp->d != vp->d) {
    set_error("tq_attend: keys must be prod mode, values mse mode, same d");
    return TQ_ERR_INVALID_ARG;
  }
  if (batch < 0 || n_kv < 0 || g < 1 || seq < 0) {
    set_error("tq_attend: bad sizes");
    return TQ_ERR_INVALID_ARG;
  }
  if (batch == 0 || n_kv == 0) return TQ_OK;
  if (seq == 0) {
    set_error("tq_attend: softmax over an empty sequence");
    return TQ_ERR_INVALID_ARG;
  }
  if (!q || !out || !workspace) {
    set_error("tq_attend: NULL q/out/workspace");
    return TQ_ERR_INVALID_ARG;
  }
  if ((st = check_codes(kp, kcodes)) || (st = check_codes(vp, vcodes))) return st;
  if (!aligned16(q) || !aligned16(out) || !aligned16(workspace)) {
    set_error("tq_attend: pointers must be 16-byte aligned");
    return TQ_ERR_ALIGNMENT;
  }
  if (!is_d128(*kp) || !is_d128(*vp)) {
    set_error("tq_attend: device kernels are built for d = m = 128 only");
    return TQ_ERR_UNSUPPORTED;
  }
  const Derived *K = nullptr, *V = nullptr;
  if ((st = get_derived(kp, &K)) || (st = get_derived(vp, &V))) return st;
  if (ws_bytes < attend_workspace_bytes(*K, *V, batch, n_kv, g, seq)) {
    set_error("tq_attend: workspace too small");
    return TQ_ERR_NO_MEMORY;
  }
  if (!(scale > 0.0f)) scale = 1.0f / std::sqrt((float)kp->d);
  return launch_attend(*K, *V, q, batch, n_kv, g, kcodes, vcodes, seq, scale, out,
                       workspace, (hipStream_t)stream);
}

tq_status tq_attend_noalloc(const tq_params *kp, const tq_params *vp, const float *q,
                            int64_t batch, int64_t n_kv, int64_t g, tq_codes kcodes,
                            tq_codes vcodes, int64_t seq, float scale, float *out, void *stream) {
  tq_status st = check_params(kp);
  if (st) return st;
  if ((st = check_params(vp))) return st;
  if (kp->mode != TQ_MODE_PROD || vp->mode != TQ_MODE_MSE || kp->d != vp->d) {
    set_error("tq_attend_noalloc: keys must be prod mode, values mse mode, same d");
    return TQ_ERR_INVALID_ARG;
  }
  if (batch < 0 || n_kv < 0 || g < 1 || seq < 0) {
    set_error("tq_attend_noalloc: bad sizes");
    return TQ_ERR_INVALID_ARG;
  }
  if (batch == 0 || n_kv == 0) return TQ_OK;
  if (seq == 0) {
    set_error("tq_attend_noalloc: softmax over an empty sequence");
    return TQ_ERR_INVALID_ARG;
  }
  if (!q || !out) {
    set_error("tq_attend_noalloc: NULL q/out");
    return TQ_ERR_INVALID_ARG;
  }
  if ((st = check_codes(kp, kcodes)) || (st = check_codes(vp, vcodes))) return st;
  if (!aligned16(q) || !aligned16(out)) {
    set_error("tq_attend_noalloc: pointers must be 16-byte aligned");
    return TQ_ERR_ALIGNMENT;
  }
  if (!is_d128(*kp) || !is_d128(*vp)) {
    set_error("tq_attend_noalloc: device kernels are built for d = m = 128 only");
    return TQ_ERR_UNSUPPORTED;
  }
  // scratch needed, against the fixed size of the device array
  size_t need = 0;
  if ((st = tq_attend_workspace_bytes(kp, vp, batch, n_kv, g, seq, &need))) return st;
  if (need > kNoAllocScratchBytes) {
    set_error("tq_attend_noalloc: these sizes need %zu bytes of scratch, more than the %zu bytes "
              "of the no-allocation scratch array; use tq_attend with a caller workspace",
              need, (size_t)kNoAllocScratchBytes);
    return TQ_ERR_UNSUPPORTED;
  }
  // the parameter caches must exist already: building them allocates
  const Derived *K = find_derived(kp), *V = find_derived(vp);
  if (!K || !V) {
    set_error("tq_attend_noalloc: the rotation/codebook cache of these parameters is not built on "
              "this device; any earlier call with the same parameters (tq_encode of the keys and of "
              "the values, tq_attend) builds it");
    return TQ_ERR_INVALID_ARG;
  }
  void *ws = nullptr;
  if ((st = noalloc_scratch(&ws))) return st;
  if (!(scale > 0.0f)) scale = 1.0f / std::sqrt((float)kp->d);
  return launch_attend(*K, *V, q, batch, n_kv, g, kcodes, vcodes, seq, scale, out, ws,
                       (hipStream_t)stream);
}

tq_status tq_encode_slots(const tq_params *p, const void *x, int32_t dtype, int64_t n,
                          const int64_t *slots, int64_t capacity, tq_codes codes, void *stream) {
  tq_status st = check_params(p);
  if (st) return st;
  if (n < 0 || capacity < 0 || (dtype != TQ_F32 && dtype != TQ_BF16)) {
    set_error("tq_encode_slots: n < 0, capacity < 0 or bad dtype");
    return TQ_ERR_INVALID_ARG;
  }
  if (n == 0) return TQ_OK;
  if (!x || !slots) {
    set_error("tq_encode_slots: x or slots is NULL");
    return TQ_ERR_INVALID_ARG;
  }
  if ((st = check_codes(p, codes))) return st;
  if (!aligned16(x)) {
    set_error("tq_encode_slots: x must be 16-byte aligned");
    return TQ_ERR_ALIGNMENT;
  }
  if (!is_d128(*p)) {
    set_error("tq_encode_slots: built for d = m = 128 (the attention shape)");
    return TQ_ERR_UNSUPPORTED;
  }
  const Derived *D = nullptr;
  if ((st = get_derived(p, &D))) return st;
  return launch_encode(*D, x, dtype, n, codes, nullptr, 0, (hipStream_t)stream, slots, capacity);
}

tq_status tq_attend_paged_workspace_bytes(const tq_params *kp, const tq_params *vp,
                                          int64_t batch, int64_t n_kv, int64_t g,
                                          int64_t max_pages, size_t *bytes) {
  if (max_pages < 0 || max_pages > (int64_t(1) << 40)) {
    set_error("tq_attend_paged_workspace_bytes: bad max_pages");
    return TQ_ERR_INVALID_ARG;
  }
  return tq_attend_workspace_bytes(kp, vp, batch, n_kv, g, max_pages * TQ_PAGE_POSITIONS, bytes);
}

tq_status tq_attend_paged(const tq_params *kp, const tq_params *vp, const float *q,
                          int64_t batch, int64_t n_kv, int64_t g, tq_codes kcodes,
                          tq_codes vcodes, int64_t num_pages, const int32_t *block_table,
                          int64_t max_pages, const int32_t *seq_lens, float scale, float *out,
                          void *workspace, size_t ws_bytes, void *stream) {
  tq_status st = check_params(kp);
  if (st) return st;
  if ((st = check_params(vp))) return st;
  if (kp->mode != TQ_MODE_PROD || vp->mode != TQ_MODE_MSE || kp->d != vp->d) {
    set_error("tq_attend_paged: keys must be prod mode, values mse mode, same d");
    return TQ_ERR_INVALID_ARG;
  }
  if (batch < 0 || n_kv < 0 || g < 1 || num_pages < 0 || max_pages < 0) {
    set_error("tq_attend_paged: bad sizes");
    return TQ_ERR_INVALID_ARG;
  }
  if (batch == 0 || n_kv == 0) return TQ_OK;
  if (num_pages == 0 || max_pages == 0) {
    set_error("tq_attend_paged: softmax over an empty sequence");
    return TQ_ERR_INVALID_ARG;
  }
  if (!q || !out || !workspace || !block_table || !seq_lens) {
    set_error("tq_attend_paged: NULL q/out/workspace/block_table/seq_lens");
    return TQ_ERR_INVALID_ARG;
  }
  if ((st = check_codes(kp, kcodes)) || (st = check_codes(vp, vcodes))) return st;
  if (!aligned16(q) || !aligned16(out) || !aligned16(workspace)) {
    set_error("tq_attend_paged: pointers must be 16-byte aligned");
    return TQ_ERR_ALIGNMENT;
  }
  if (!is_d128(*kp) || !is_d128(*vp)) {
    set_error("tq_attend_paged: device kernels are built for d = m = 128 only");
    return TQ_ERR_UNSUPPORTED;
  }
  if (max_pages >= (int64_t(1) << 28) / TQ_PAGE_POSITIONS) {
    set_error("tq_attend_paged: max_pages * %d must stay below 2^28", TQ_PAGE_POSITIONS);
    return TQ_ERR_UNSUPPORTED;
  }
  const Derived *K = nullptr, *V = nullptr;
  if ((st = get_derived(kp, &K)) || (st = get_derived(vp, &V))) return st;
  const int64_t seq_max = max_pages * TQ_PAGE_POSITIONS;
  if (ws_bytes < attend_workspace_bytes(*K, *V, batch, n_kv, g, seq_max)) {
    set_error("tq_attend_paged: workspace too small");
    return TQ_ERR_NO_MEMORY;
  }
  if (!(scale > 0.0f)) scale = 1.0f / std::sqrt((float)kp->d);
  return launch_attend(*K, *V, q, batch, n_kv, g, kcodes, vcodes, seq_max, scale, out, workspace,
                       (hipStream_t)stream, block_table, max_pages, num_pages, seq_lens);
}

tq_status tq_decode(const tq_params *p, tq_codes codes, int64_t n, float *out, void *stream) {
  tq_status st = check_params(p);
  if (st) return st;
  if (n < 0) {
    set_error("tq_decode: n < 0");
    return TQ_ERR_INVALID_ARG;
  }
  if (n == 0) return TQ_OK;
  if (!out) {
    set_error("tq_decode: out is NULL");
    return TQ_ERR_INVALID_ARG;
  }
  const int B = mse_bits(p);
  if ((B > 0 && !codes.idx) || !codes.knorm) {
    set_error("tq_decode: idx/knorm missing");
    return TQ_ERR_INVALID_ARG;
  }
  if ((B > 0 && !aligned16(codes.idx)) || !aligned16(codes.knorm) || !aligned16(out)) {
    set_error("tq_decode: pointers must be 16-byte aligned");
    return TQ_ERR_ALIGNMENT;
  }
  if (p->d != 128) {
    set_error("tq_decode: device kernels are built for d = 128 only");
    return TQ_ERR_UNSUPPORTED;
  }
  const Derived *D = nullptr;
  if ((st = get_derived(p, &D))) return st;
  return launch_decode(*D, codes, n, out, (hipStream_t)stream);
}

tq_status tq_search_workspace_bytes(const tq_params *p, int64_t nq, int64_t n, int32_t k,
                                    size_t *bytes) {
  tq_status st = check_params(p);
  if (st) return st;
  if (nq < 0 || n < 0 || k < 1 || k > 32 || !bytes) {
    set_error("tq_search_workspace_bytes: bad nq/n/k");
    return TQ_ERR_INVALID_ARG;
  }
  *bytes = search_workspace_bytes(*p, nq, n, k);
  return TQ_OK;
}

tq_status tq_search(const tq_params *p, const float *q, int64_t nq, tq_codes codes, int64_t n,
                    int32_t k, int64_t *out_idx, float *out_val, void *workspace,
                    size_t ws_bytes, void *stream) {
  tq_status st = check_params(p);
  if (st) return st;
  if (nq < 0 || n < 0 || k < 1 || k > 32 || (nq > 0 && k > n)) {
    set_error("tq_search: need nq >= 0, 1 <= k <= 32, k <= n");
    return TQ_ERR_INVALID_ARG;
  }
  if (nq == 0) return TQ_OK;
  if (!q || !out_idx || !workspace) {
    set_error("tq_search: NULL q/out_idx/workspace");
    return TQ_ERR_INVALID_ARG;
  }
  if ((st = check_codes(p, codes))) return st;
  if (!aligned16(q) || !aligned16(workspace) || !aligned16(out_idx) || (out_val && !aligned16(out_val))) {
    set_error("tq_search: pointers must be 16-byte aligned");
    return TQ_ERR_ALIGNMENT;
  }
  const size_t need = search_workspace_bytes(*p, nq, n, k);
  if (ws_bytes < need) {
    set_error("tq_search: workspace too small (%zu < %zu)", ws_bytes, need);
    return TQ_ERR_NO_MEMORY;
  }
  const Derived *D = nullptr;
  if ((st = get_derived(p, &D))) return st;
  return launch_search(*D, q, nq, codes, n, k, out_idx, out_val, workspace, (hipStream_t)stream);
}

tq_status tq_polar_make_codebook(int32_t d, int32_t level, int32_t nbits, float *centroids,
                                 float *boundaries) {
  int levels = 0;
  while ((1 << (levels + 1)) <= d) ++levels;
  if (d < 4 || (d & (d - 1)) || level < 1 || level > levels || nbits < 1 || nbits > 6 || !centroids ||
      (nbits > 0 && !boundaries)) {
    set_error("tq_polar_make_codebook: need d a power of two >= 4, 1 <= level <= log2 d, 1 <= nbits <= 6");
    return TQ_ERR_INVALID_ARG;
  }
  std::vector<double> c, b;
  polar_codebook(level, nbits, c, b);
  for (size_t j = 0; j < c.size(); ++j) centroids[j] = (float)c[j];
  for (size_t j = 0; j < b.size(); ++j) boundaries[j] = (float)b[j];
  return TQ_OK;
}

tq_status tq_polar_encode(const tq_polar_params *p, const void *x, int32_t dtype, int64_t n,
                          tq_polar_codes codes, void *stream) {
  tq_status st = check_polar(p, "tq_polar_encode");
  if (st) return st;
  if (n < 0 || (dtype != TQ_F32 && dtype != TQ_BF16)) {
    set_error("tq_polar_encode: n < 0 or bad dtype");
    return TQ_ERR_INVALID_ARG;
  }
  if (n == 0) return TQ_OK;
  if (!x || !codes.pq || !codes.radius) {
    set_error("tq_polar_encode: NULL x/pq/radius");
    return TQ_ERR_INVALID_ARG;
  }
  if (!aligned16(x) || !aligned16(codes.pq) || !aligned16(codes.radius)) {
    set_error("tq_polar_encode: pointers must be 16-byte aligned");
    return TQ_ERR_ALIGNMENT;
  }
  const tq_params tp = polar_rotation_params(p);
  const Derived *D = nullptr;
  if ((st = get_derived(&tp, &D))) return st;
  const PolarTables *T = nullptr;
  if ((st = polar_tables_device(&T))) return st;
  return launch_polar_encode(*D, T, x, dtype, n, codes, (hipStream_t)stream);
}

tq_status tq_polar_score_workspace_bytes(const tq_polar_params *p, int64_t n_kv, int64_t g,
                                         size_t *bytes) {
  tq_status st = check_polar(p, "tq_polar_score_workspace_bytes");
  if (st) return st;
  if (n_kv < 0 || g < 1 || !bytes) {
    set_error("tq_polar_score_workspace_bytes: bad sizes");
    return TQ_ERR_INVALID_ARG;
  }
  *bytes = polar_score_workspace_bytes(n_kv * g);
  return TQ_OK;
}

tq_status tq_polar_score(const tq_polar_params *p, const float *q, int64_t n_kv, int64_t g,
                         tq_polar_codes codes, int64_t seq, float *logits, void *workspace,
                         size_t ws_bytes, void *stream) {
  tq_status st = check_polar(p, "tq_polar_score");
  if (st) return st;
  if (n_kv < 0 || g < 1 || seq < 0) {
    set_error("tq_polar_score: bad sizes");
    return TQ_ERR_INVALID_ARG;
  }
  if (n_kv == 0 || seq == 0) return TQ_OK;
  if (!q || !logits || !workspace || !codes.pq || !codes.radius) {
    set_error("tq_polar_score: NULL q/logits/workspace/pq/radius");
    return TQ_ERR_INVALID_ARG;
  }
  if (!aligned16(q) || !aligned16(workspace) || !aligned16(codes.pq) || !aligned16(codes.radius)) {
    set_error("tq_polar_score: pointers must be 16-byte aligned");
    return TQ_ERR_ALIGNMENT;
  }
  if (ws_bytes < polar_score_workspace_bytes(n_kv * g)) {
    set_error("tq_polar_score: workspace too small");
    return TQ_ERR_NO_MEMORY;
  }
  const tq_params tp = polar_rotation_params(p);
  const Derived *D = nullptr;
  if ((st = get_derived(&tp, &D))) return st;
  const PolarTables *T = nullptr;
  if ((st = polar_tables_device(&T))) return st;
  return launch_polar_score(*D, T, q, n_kv, g, codes, seq, logits, workspace, (hipStream_t)stream);
}

tq_status tq_split_words(const tq_split_params *p, int32_t *words) {
  tq_status st = check_split(p, "tq_split_words");
  if (st) return st;
  if (!words) {
    set_error("tq_split_words: words is NULL");
    return TQ_ERR_INVALID_ARG;
  }
  // b planes per group (b - 1 index planes and the sign plane), d_g / 32 words each
  const int n_out = split_n_out(p);
  *words = p->b_out * (n_out / 32) + p->b_rest * ((128 - n_out) / 32);
  return TQ_OK;
}

tq_status tq_split_encode(const tq_split_params *p, const void *x, int32_t dtype, int64_t n,
                          tq_split_codes codes, void *stream) {
  tq_status st = check_split(p, "tq_split_encode");
  if (st) return st;
  if (n < 0 || (dtype != TQ_F32 && dtype != TQ_BF16)) {
    set_error("tq_split_encode: n < 0 or bad dtype");
    return TQ_ERR_INVALID_ARG;
  }
  if (n == 0) return TQ_OK;
  if (!x || !codes.words || !codes.norms) {
    set_error("tq_split_encode: NULL x/words/norms");
    return TQ_ERR_INVALID_ARG;
  }
  if (!aligned16(x) || !aligned16(codes.words) || !aligned16(codes.norms)) {
    set_error("tq_split_encode: pointers must be 16-byte aligned");
    return TQ_ERR_ALIGNMENT;
  }
  const SplitDerived *D = nullptr;
  if ((st = get_split(p, &D))) return st;
  return launch_split_encode(*D, x, dtype, n, codes, (hipStream_t)stream);
}

tq_status tq_split_score_workspace_bytes(const tq_split_params *p, int64_t n_kv, int64_t g,
                                         size_t *bytes) {
  tq_status st = check_split(p, "tq_split_score_workspace_bytes");
  if (st) return st;
  if (n_kv < 0 || g < 1 || !bytes) {
    set_error("tq_split_score_workspace_bytes: bad sizes");
    return TQ_ERR_INVALID_ARG;
  }
  *bytes = split_score_workspace_bytes(n_kv * g);
  return TQ_OK;
}

tq_status tq_split_score(const tq_split_params *p, const float *q, int64_t n_kv, int64_t g,
                         tq_split_codes codes, int64_t seq, float *logits, void *workspace,
                         size_t ws_bytes, void *stream) {
  tq_status st = check_split(p, "tq_split_score");
  if (st) return st;
  if (n_kv < 0 || g < 1 || seq < 0) {
    set_error("tq_split_score: bad sizes");
    return TQ_ERR_INVALID_ARG;
  }
  if (n_kv == 0 || seq == 0) return TQ_OK;
  if (!q || !logits || !workspace || !codes.words || !codes.norms) {
    set_error("tq_split_score: NULL q/logits/workspace/words/norms");
    return TQ_ERR_INVALID_ARG;
  }
  if (!aligned16(q) || !aligned16(workspace) || !aligned16(codes.words) || !aligned16(codes.norms)) {
    set_error("tq_split_score: pointers must be 16-byte aligned");
    return TQ_ERR_ALIGNMENT;
  }
  if (ws_bytes < split_score_workspace_bytes(n_kv * g)) {
    set_error("tq_split_score: workspace too small");
    return TQ_ERR_NO_MEMORY;
  }
  const SplitDerived *D = nullptr;
  if ((st = get_split(p, &D))) return st;
  return launch_split_score(*D, q, n_kv, g, codes, seq, logits, workspace, (hipStream_t)stream);
}

tq_status tq_release_cache(void) {
  polar_tables_release();
  split_release();
  std::lock_guard<std::mutex> lock(g_cache_mu);
  for (auto &kv : g_cache) free_derived(kv.second);
  g_cache.clear();
  return TQ_OK;
}

}  // extern "C"
