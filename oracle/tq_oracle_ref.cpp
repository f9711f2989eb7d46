// Plain, slow CPU oracle of the TurboQuant hot path in C++ (a second
// implementation beside the numpy oracle in tq_oracle.py).
//
// TEST INFRASTRUCTURE ONLY.  Built into oracle/libtqref.so and loaded by
// tests/ (to cross-check the numpy oracle) and by the cpu_baseline leg of
// bench.py.  It shares no code with the GPU library and includes nothing
// from it; every step is written out here in scalar loops with long double
// accumulation, one vector at a time.
//
// What it computes (pages cited by title and section):
//   "谷歌TurboQuant如何绕过内存墙？重新审视它的技术突破", 2.TurboQuant到底做了什么？
//     第一阶段: rotate by a random orthogonal Pi, then quantise each
//               coordinate with the Lloyd-Max codebook of the known
//               coordinate law of a rotated unit vector;
//     第二阶段: with b bits, b-1 go to that quantiser and one QJL sign bit
//               per projection row to the residual.
//   "TurboQuant 与 AI 效率革命：当旧数学遇到新智能", 三 (非对称估计器: the inner
//     product from sign bits, sqrt(pi/2)/m * ||r|| * <S q, sign(S r)>; 零开销的
//     秘密: norms stored as 32-bit floats) and 四 (三段论: rotation, then the
//     signs of S times the residual).
//   yeyulingfeng.com explainer, "TurboQuant：6倍压缩，零损失": attention over
//     the compressed cache, here softmax over the logits of the keys' codes
//     weighting the MSE reconstructions of the values.
// Readings where the pages are silent (the same as the numpy oracle's):
//   random numbers: SplitMix64 words, Gaussians by Box-Muller on word pairs
//     (element (i, j) of an R x C matrix is counter i C + j; pair c / 2 takes
//     u1 = (top 53 bits of word c - c % 2 + 1) * 2^-53 in (0, 1] and
//     u2 = top 53 bits of the next word * 2^-53; even c the cosine branch);
//   Pi: Q of the QR factorisation of a seeded Gaussian with diag(R) > 0, here
//     by Gram-Schmidt on the columns, orthogonalised twice (which yields
//     diag(R) > 0 directly); y = Pi x;
//   S: i.i.d. N(0, 1), m x d;
//   codebook: Lloyd-Max for f_d(x) proportional to (1 - x^2)^((d - 3) / 2) on
//     [-1, 1], run on the positive half and mirrored; exchanged as float32
//     centroids and float32 boundaries fp32((c_j + c_j+1) / 2) taken in double;
//   index = #{j : fp32(u_i) >= t_j}; residual r = x - ||x|| Pi^T c[idx] in the
//     original domain; sign bit = [fp32((S r)_j) >= 0]; norms float32; a zero
//     vector has u = 0, r = 0;
//   prod mode: b - 1 Lloyd-Max bits and m signs; mse mode: b bits;
//   attention: softmax temperature 1 / sqrt(d) unless one is given, values
//     in mse mode.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

namespace {

typedef long double ld;

uint64_t splitmix_word(uint64_t seed, uint64_t k) {
  uint64_t z = seed + (k + 1) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

double gaussian_at(uint64_t seed, uint64_t c) {
  const uint64_t pair = c / 2;
  const uint64_t w1 = splitmix_word(seed, 2 * pair), w2 = splitmix_word(seed, 2 * pair + 1);
  const double u1 = ((double)(w1 >> 11) + 1.0) * 0x1p-53;
  const double u2 = (double)(w2 >> 11) * 0x1p-53;
  const double rad = std::sqrt(-2.0 * std::log(u1));
  const double ang = 2.0 * M_PI * u2;
  return (c % 2 == 0) ? rad * std::cos(ang) : rad * std::sin(ang);
}

// ---- Gauss-Legendre rule (nodes by Newton's method on P_n) -------------
struct GaussLegendre {
  std::vector<ld> x, w;
  explicit GaussLegendre(int n) : x(n), w(n) {
    for (int i = 0; i < n; ++i) {
      ld z = std::cos(M_PI * (i + 0.75L) / (n + 0.5L));
      ld dp = 0;
      for (int it = 0; it < 100; ++it) {
        ld p0 = 1, p1 = z;  // P_0, P_1
        for (int k = 2; k <= n; ++k) {
          const ld p2 = ((2 * k - 1) * z * p1 - (k - 1) * p0) / k;
          p0 = p1;
          p1 = p2;
        }
        dp = n * (z * p1 - p0) / (z * z - 1);  // P_n'(z)
        const ld dz = p1 / dp;
        z -= dz;
        if (std::fabs(dz) < 1e-19L) break;
      }
      x[i] = z;
      w[i] = 2 / ((1 - z * z) * dp * dp);
    }
  }
};

const GaussLegendre &rule() {
  static const GaussLegendre gl(20);
  return gl;
}

// f_d on [0, 1]: exp(log normaliser + (d - 3) / 2 * log(1 - x^2))
struct Density {
  int d;
  ld logc, alpha;
  explicit Density(int d_) : d(d_) {
    logc = std::lgamma((ld)d / 2) - 0.5L * std::log((ld)M_PI) - std::lgamma(((ld)d - 1) / 2);
    alpha = ((ld)d - 3) / 2;
  }
  ld operator()(ld x) const {
    if (alpha == 0) return std::exp(logc);
    const ld one_m = 1 - x * x;
    if (one_m <= 0) return 0;
    return std::exp(logc + alpha * std::log(one_m));
  }
};

// integral over [a, b] of f(x) and of x f(x): panels of at most an eighth
// of the coordinate's standard deviation, plus points 1 - 2^-k near x = 1
// (the (1 - x^2)^alpha end for small d)
void moments(const Density &f, ld a, ld b, ld &mass, ld &mom) {
  mass = mom = 0;
  if (b <= a) return;
  std::vector<ld> pts;
  const ld width = 1 / (8 * std::sqrt((ld)f.d));
  const int np = (int)std::ceil((b - a) / width);
  for (int i = 0; i <= np; ++i) pts.push_back(a + (b - a) * i / np);
  for (int k = 1; k < 64; ++k) {
    const ld e = 1 - std::ldexp((ld)1, -k);
    if (e > a && e < b) pts.push_back(e);
  }
  std::sort(pts.begin(), pts.end());
  const GaussLegendre &gl = rule();
  for (size_t i = 0; i + 1 < pts.size(); ++i) {
    const ld lo = pts[i], hi = pts[i + 1];
    if (hi <= lo) continue;
    const ld h = (hi - lo) / 2, mid = (hi + lo) / 2;
    for (size_t k = 0; k < gl.x.size(); ++k) {
      const ld xx = mid + h * gl.x[k], fx = f(xx);
      mass += h * gl.w[k] * fx;
      mom += h * gl.w[k] * xx * fx;
    }
  }
}

// Lloyd-Max with 2^B levels (float32 exchange form)
void lloyd_max(int d, int B, float *c32, float *t32) {
  const int L = 1 << B, half = L / 2;
  const Density f(d);
  std::vector<ld> c(half), e(half + 1);
  const ld sigma = 1 / std::sqrt((ld)d);
  const ld span = std::min<ld>(3 * sigma, 1);
  for (int j = 0; j < half; ++j) c[j] = (j + 0.5L) * span / half;
  for (int it = 0; it < 200000; ++it) {
    e[0] = 0;
    e[half] = 1;
    for (int j = 1; j < half; ++j) e[j] = (c[j - 1] + c[j]) / 2;
    ld delta = 0;
    for (int j = 0; j < half; ++j) {
      ld mass, mom;
      moments(f, e[j], e[j + 1], mass, mom);
      const ld nc = mom / mass;
      delta = std::max<ld>(delta, std::fabs(nc - c[j]));
      c[j] = nc;
    }
    if (delta <= 1e-16L * c[half - 1]) break;
  }
  for (int j = 0; j < half; ++j) {
    c32[half + j] = (float)c[j];
    c32[half - 1 - j] = -(float)c[j];
  }
  for (int j = 0; j + 1 < L; ++j) t32[j] = (float)(((double)c32[j] + (double)c32[j + 1]) / 2);
  t32[half - 1] = 0.f;
}

struct Ctx {
  int d, b, m, mode, B;
  std::vector<double> pi;  // [d][d], y = Pi x
  std::vector<double> s;   // [m][d]
  std::vector<float> c, t;
};

void build_rotation(int d, uint64_t seed, std::vector<double> &pi) {
  // columns of G, orthonormalised in turn (twice), become the columns of Pi
  std::vector<ld> q((size_t)d * d);  // column-major: q[j * d + i] = Pi[i][j]
  for (int j = 0; j < d; ++j) {
    std::vector<ld> v(d);
    for (int i = 0; i < d; ++i) v[i] = gaussian_at(seed, (uint64_t)i * d + j);
    for (int pass = 0; pass < 2; ++pass)
      for (int k = 0; k < j; ++k) {
        ld dot = 0;
        for (int i = 0; i < d; ++i) dot += q[(size_t)k * d + i] * v[i];
        for (int i = 0; i < d; ++i) v[i] -= dot * q[(size_t)k * d + i];
      }
    ld nrm = 0;
    for (int i = 0; i < d; ++i) nrm += v[i] * v[i];
    nrm = std::sqrt(nrm);
    for (int i = 0; i < d; ++i) q[(size_t)j * d + i] = v[i] / nrm;
  }
  pi.assign((size_t)d * d, 0.0);
  for (int i = 0; i < d; ++i)
    for (int j = 0; j < d; ++j) pi[(size_t)i * d + j] = (double)q[(size_t)j * d + i];
}

void encode_one(const Ctx &C, const double *x, int32_t *idx, uint8_t *sign, float *knorm,
                float *rnorm, double *z) {
  const int d = C.d, m = C.m;
  ld ss = 0;
  for (int i = 0; i < d; ++i) ss += (ld)x[i] * x[i];
  const double nu = (double)std::sqrt(ss);
  *knorm = (float)nu;
  std::vector<double> recon(d, 0.0);
  if (C.B > 0) {
    const int L = 1 << C.B;
    std::vector<int> id(d);
    for (int i = 0; i < d; ++i) {
      ld y = 0;
      for (int j = 0; j < d; ++j) y += (ld)C.pi[(size_t)i * d + j] * x[j];
      const double u = nu > 0 ? (double)(y / nu) : 0.0;
      const float u32 = (float)u;
      int k = 0;
      for (int j = 0; j + 1 < L; ++j) k += u32 >= C.t[j] ? 1 : 0;
      id[i] = k;
      idx[i] = k;
    }
    // x~ = nu Pi^T c[idx]
    for (int j = 0; j < d; ++j) {
      ld a = 0;
      for (int i = 0; i < d; ++i) a += (ld)C.pi[(size_t)i * d + j] * (ld)C.c[id[i]];
      recon[j] = (double)(nu * a);
    }
  }
  if (C.mode == 0) {  // prod: QJL signs of the residual
    std::vector<double> r(d);
    ld rr = 0;
    for (int j = 0; j < d; ++j) {
      r[j] = nu > 0 ? x[j] - recon[j] : 0.0;
      rr += (ld)r[j] * r[j];
    }
    *rnorm = (float)std::sqrt(rr);
    for (int k = 0; k < m; ++k) {
      ld a = 0;
      for (int j = 0; j < d; ++j) a += (ld)C.s[(size_t)k * d + j] * r[j];
      const double zz = (double)a;
      if (z) z[k] = zz;
      sign[k] = (float)zz >= 0.f ? 1 : 0;
    }
  }
}

}  // namespace

extern "C" {

// Parameters and derived matrices; returns an opaque context (NULL on bad
// arguments).  mode 0 = prod (b - 1 Lloyd-Max bits + m signs), 1 = mse.
void *tqref_create(int d, int b, int m, int mode, uint64_t seed_pi, uint64_t seed_s) {
  if (d < 2 || b < 1 || b > 5 || (mode != 0 && mode != 1) || (mode == 0 && m < 1)) return nullptr;
  Ctx *C = new Ctx;
  C->d = d;
  C->b = b;
  C->m = mode == 0 ? m : 0;
  C->mode = mode;
  C->B = mode == 0 ? b - 1 : b;
  build_rotation(d, seed_pi, C->pi);
  if (mode == 0) {
    C->s.resize((size_t)m * d);
    for (int i = 0; i < m; ++i)
      for (int j = 0; j < d; ++j) C->s[(size_t)i * d + j] = gaussian_at(seed_s, (uint64_t)i * d + j);
  }
  if (C->B > 0) {
    C->c.resize(1 << C->B);
    C->t.resize((1 << C->B) - 1);
    lloyd_max(d, C->B, C->c.data(), C->t.data());
  }
  return C;
}

void tqref_destroy(void *ctx) { delete static_cast<Ctx *>(ctx); }

// Gaussian matrix of the reading above, rows x cols, row-major.
void tqref_gaussian(uint64_t seed, int64_t rows, int64_t cols, double *out) {
  for (int64_t c = 0; c < rows * cols; ++c) out[c] = gaussian_at(seed, (uint64_t)c);
}

// Copies of the context's Pi [d][d], S [m][d] (if any) and codebook
// (centroids [2^B], boundaries [2^B - 1]); NULL skips an output.
void tqref_matrices(const void *ctx, double *pi, double *s, float *c, float *t) {
  const Ctx &C = *static_cast<const Ctx *>(ctx);
  if (pi) std::memcpy(pi, C.pi.data(), C.pi.size() * sizeof(double));
  if (s && !C.s.empty()) std::memcpy(s, C.s.data(), C.s.size() * sizeof(double));
  if (c && !C.c.empty()) std::memcpy(c, C.c.data(), C.c.size() * sizeof(float));
  if (t && !C.t.empty()) std::memcpy(t, C.t.data(), C.t.size() * sizeof(float));
}

// Encodes n rows of x [n][d]: idx [n][d] (B > 0), sign [n][m] and rnorm [n]
// (prod mode), knorm [n], z [n][m] (raw S r, may be NULL).  Vectors are
// split over `threads` std::threads (1 = the calling thread only).
void tqref_encode(const void *ctx, const double *x, int64_t n, int32_t *idx, uint8_t *sign,
                  float *knorm, float *rnorm, double *z, int threads) {
  const Ctx &C = *static_cast<const Ctx *>(ctx);
  auto work = [&](int64_t lo, int64_t hi) {
    for (int64_t v = lo; v < hi; ++v)
      encode_one(C, x + v * C.d, C.B > 0 ? idx + v * C.d : nullptr, C.mode == 0 ? sign + v * C.m : nullptr,
                 knorm + v, C.mode == 0 ? rnorm + v : nullptr, z ? z + v * C.m : nullptr);
  };
  if (threads <= 1) {
    work(0, n);
    return;
  }
  std::vector<std::thread> pool;
  for (int t = 0; t < threads; ++t) pool.emplace_back(work, n * t / threads, n * (t + 1) / threads);
  for (auto &th : pool) th.join();
}

// Logits [n_kv * g][seq] of queries q [n_kv * g][d] against the codes of
// n_kv * seq keys (query head h reads KV head h / g):
//   knorm * <Pi q, c[idx]> + sqrt(pi/2) / m * rnorm * <S q, s>, s = +-1.
void tqref_score(const void *ctx, const double *q, int64_t n_kv, int64_t g, const int32_t *idx,
                 const uint8_t *sign, const float *knorm, const float *rnorm, int64_t seq, double *logits,
                 int threads) {
  const Ctx &C = *static_cast<const Ctx *>(ctx);
  const int d = C.d, m = C.m;
  const int64_t nq = n_kv * g;
  std::vector<double> qt((size_t)nq * d), qs((size_t)nq * (m > 0 ? m : 1));
  for (int64_t h = 0; h < nq; ++h) {
    for (int i = 0; i < d; ++i) {
      ld a = 0;
      for (int j = 0; j < d; ++j) a += (ld)C.pi[(size_t)i * d + j] * q[h * d + j];
      qt[h * d + i] = (double)a;
    }
    for (int k = 0; k < m; ++k) {
      ld a = 0;
      for (int j = 0; j < d; ++j) a += (ld)C.s[(size_t)k * d + j] * q[h * d + j];
      qs[h * m + k] = (double)a;
    }
  }
  const ld kq = m > 0 ? std::sqrt((ld)M_PI / 2) / m : 0;
  auto work = [&](int64_t lo, int64_t hi) {
    for (int64_t h = lo; h < hi; ++h) {
      const int64_t kv = h / g;
      for (int64_t p = 0; p < seq; ++p) {
        const int64_t v = kv * seq + p;
        ld l = 0;
        if (C.B > 0) {
          ld a = 0;
          for (int i = 0; i < d; ++i) a += (ld)qt[h * d + i] * (ld)C.c[idx[v * d + i]];
          l += (ld)knorm[v] * a;
        }
        if (C.mode == 0) {
          ld a = 0;
          for (int k = 0; k < m; ++k) a += sign[v * m + k] ? (ld)qs[h * m + k] : -(ld)qs[h * m + k];
          l += kq * (ld)rnorm[v] * a;
        }
        logits[h * seq + p] = (double)l;
      }
    }
  };
  if (threads <= 1) {
    work(0, nq);
    return;
  }
  std::vector<std::thread> pool;
  for (int t = 0; t < threads; ++t) pool.emplace_back(work, nq * t / threads, nq * (t + 1) / threads);
  for (auto &th : pool) th.join();
}

// Decode attention over compressed K and V, as the numpy oracle reads it:
// for each batch entry bi and query head h (KV head h / g), logits from the
// K codes (as tqref_score) times `scale` (<= 0 selects 1 / sqrt(d)), weights
// softmax over all seq positions (the largest logit subtracted), output
//   out[bi][h] = sum_p w_p v~_p,   v~_p = ||v_p|| Pi_V^T c_V[idx_p]
// with each value reconstructed in the original domain first.  kctx is a
// prod- or mse-mode context of dimension d, vctx an mse-mode context of
// dimension dv; the codes of batch entry bi, KV head k, position p are row
// (bi n_kv + k) seq + p.  q [batch][n_kv g][d], out [batch][n_kv g][dv].
void tqref_attend(const void *kctx, const void *vctx, const double *q, int64_t batch, int64_t n_kv,
                  int64_t g, int64_t seq, const int32_t *kidx, const uint8_t *ksign, const float *knorm,
                  const float *krnorm, const int32_t *vidx, const float *vnorm, double scale, double *out,
                  int threads) {
  const Ctx &K = *static_cast<const Ctx *>(kctx);
  const Ctx &V = *static_cast<const Ctx *>(vctx);
  const int d = K.d, dv = V.d;
  if (!(scale > 0)) scale = 1.0 / std::sqrt((double)d);
  const int64_t nq = n_kv * g;
  std::vector<double> logits((size_t)nq * seq);
  for (int64_t bi = 0; bi < batch; ++bi) {
    const int64_t k0 = bi * n_kv * seq;  // first key row of this batch entry
    tqref_score(kctx, q + bi * nq * d, n_kv, g, K.B > 0 ? kidx + k0 * d : nullptr,
                K.mode == 0 ? ksign + k0 * K.m : nullptr, knorm + k0, K.mode == 0 ? krnorm + k0 : nullptr,
                seq, logits.data(), threads);
    // the values of this batch entry, reconstructed one at a time
    std::vector<double> vrec((size_t)n_kv * seq * dv);
    for (int64_t r = 0; r < n_kv * seq; ++r) {
      const int32_t *ix = vidx + (k0 + r) * dv;
      for (int j = 0; j < dv; ++j) {
        ld a = 0;
        for (int i = 0; i < dv; ++i) a += (ld)V.pi[(size_t)i * dv + j] * (ld)V.c[ix[i]];
        vrec[(size_t)r * dv + j] = (double)((ld)vnorm[k0 + r] * a);
      }
    }
    for (int64_t h = 0; h < nq; ++h) {
      const int64_t kv = h / g;
      const double *lh = logits.data() + h * seq;
      ld mx = -INFINITY;
      for (int64_t p = 0; p < seq; ++p) mx = std::max<ld>(mx, (ld)lh[p] * scale);
      std::vector<ld> w(seq);
      ld wsum = 0;
      for (int64_t p = 0; p < seq; ++p) {
        w[p] = std::exp((ld)lh[p] * scale - mx);
        wsum += w[p];
      }
      for (int j = 0; j < dv; ++j) {
        ld a = 0;
        for (int64_t p = 0; p < seq; ++p) a += w[p] * (ld)vrec[(size_t)(kv * seq + p) * dv + j];
        out[(bi * nq + h) * dv + j] = (double)(a / wsum);
      }
    }
  }
}

// Top-k search: for each of nq queries q [nq][d], the k of the n coded
// vectors with the largest logit (as tqref_score, every query against the
// same n vectors), in descending order of logit, ties to the lower index.
// out_idx / out_val [nq][k]; k <= n.  A plain running list per query: each
// logit is compared with the list's last entry and, if it beats it, inserted
// in place.
void tqref_search(const void *ctx, const double *q, int64_t nq, const int32_t *idx, const uint8_t *sign,
                  const float *knorm, const float *rnorm, int64_t n, int64_t k, int64_t *out_idx,
                  double *out_val, int threads) {
  const Ctx &C = *static_cast<const Ctx *>(ctx);
  for (int64_t i = 0; i < nq; ++i) {
    std::vector<double> row(n);
    tqref_score(ctx, q + i * C.d, 1, 1, idx, sign, knorm, rnorm, n, row.data(), threads);
    std::vector<int64_t> li;
    std::vector<double> lv;
    for (int64_t v = 0; v < n; ++v) {
      // strictly larger logits go first; an equal logit comes after (v is
      // larger than every index already listed)
      if ((int64_t)li.size() == k && !(row[v] > lv.back())) continue;
      int64_t pos = (int64_t)li.size();
      while (pos > 0 && row[v] > lv[pos - 1]) --pos;
      li.insert(li.begin() + pos, v);
      lv.insert(lv.begin() + pos, row[v]);
      if ((int64_t)li.size() > k) {
        li.pop_back();
        lv.pop_back();
      }
    }
    for (int64_t j = 0; j < k; ++j) {
      out_idx[i * k + j] = li[j];
      out_val[i * k + j] = lv[j];
    }
  }
}

}  // extern "C"
