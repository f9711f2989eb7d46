// Device side of libtq: the gfx950 kernels of the TurboQuant hot path and
// their launchers.
//
// Method (pages cited by title and section):
//   "谷歌TurboQuant如何绕过内存墙？重新审视它的技术突破", 2.TurboQuant到底做了什么？
//     第一阶段: rotate, then scalar-quantise every coordinate with a Lloyd-Max
//               codebook for the known Beta-shaped coordinate law;
//     第二阶段: with b bits, b-1 go to that quantiser and 1 to a QJL sign
//               transform of the residual.
//   "TurboQuant 与 AI 效率革命：当旧数学遇到新智能", 三 非对称估计器 (inner
//     products from sign bits: sqrt(pi/2)/m * ||k|| * <S q, sign(S k)>) and
//     四 三段论 (rotation P, then sign(S * residual)).
//
// Design notes for gfx950 (wave64, MFMA, 160 KB LDS):
//   * encode: both projections are dense 128 x 128 contractions per vector and
//     run on bf16 MFMA (v_mfma_f32_16x16x32_bf16).  Bucket decisions need the
//     rotated coordinates to ~1e-7, so the matrices are split hi + lo in bf16
//     (and float32 inputs / the residual too), giving float32-level products.
//     The whole bf16 split of Pi and S' = S Pi^T lives in LDS (128 KB) for the
//     life of a persistent workgroup.  The first GEMM's output registers are
//     already the second GEMM's operand layout, so the residual never leaves
//     registers, and each lane packs its own 32-bit words of index planes and
//     sign bits (the packed layout follows the MFMA output layout).
//   * score: logits from packed codes are integer dot products of bit planes
//     with the query.  A symmetric codebook is an odd multilinear function of
//     the +-1 bit signs, so c[idx] is a short sum of coefficient * (parity of
//     a subset of planes); the QJL term is a plain +-1 dot product.  Bits
//     become int8 MFMA operands with one AND per 4 bytes (bit k of every byte,
//     weight 2^k, -128 for k = 7); the query side carries the weights 2^-k and
//     is split into four balanced base-128 int8 limbs that fill the 16 MFMA
//     rows (4 queries x 4 limbs).  int32 accumulation is exact.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "tq_internal.h"

namespace tq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

#define TQ_LAUNCH_CHECK()                                                   \
  do {                                                                      \
    hipError_t e_ = hipGetLastError();                                      \
    if (e_ != hipSuccess) {                                                 \
      set_error("kernel launch failed: %s", hipGetErrorString(e_));        \
      return TQ_ERR_HIP;                                                    \
    }                                                                       \
  } while (0)

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// float -> bf16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// ===========================================================================
// Encode, d = m = 128
// ===========================================================================
constexpr int kEncWaves = 8;          // waves per workgroup
constexpr int kEncCT = 2;             // 16-vector column tiles per wave batch
constexpr int kEncBatch = 16 * kEncCT;  // vectors per wave batch
constexpr int kFragU4 = kFragElems / 8;  // uint4 per fragment matrix (2048)

// X^T fragment of one 16-vector column tile, column block kt: lane (v, g)
// holds x[v][32 kt + 8 g .. + 7]; hi/lo bf16 split for float32 inputs.
template <bool XBF16>
__device__ __forceinline__ void load_x_frag(const void *__restrict__ x, int64_t row, bool valid,
                                            int kt, int g, uint4 &hi, uint4 &lo, float &sumsq) {
  if (XBF16) {
    const uint4 *p = reinterpret_cast<const uint4 *>(
        reinterpret_cast<const uint16_t *>(x) + row * 128 + 32 * kt + 8 * g);
    hi = valid ? *p : make_uint4(0, 0, 0, 0);
    const uint32_t w[4] = {hi.x, hi.y, hi.z, hi.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a = bf16_to_f32(w[i] & 0xFFFFu), b = bf16_to_f32(w[i] >> 16);
      sumsq += a * a + b * b;
    }
  } else {
    const float4 *p = reinterpret_cast<const float4 *>(
        reinterpret_cast<const float *>(x) + row * 128 + 32 * kt + 8 * g);
    float4 a = valid ? p[0] : make_float4(0, 0, 0, 0);
    float4 b = valid ? p[1] : make_float4(0, 0, 0, 0);
    const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    uint32_t h[8], l[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      sumsq += v[i] * v[i];
      h[i] = bf16_rne(v[i]);
      l[i] = bf16_rne(v[i] - bf16_to_f32(h[i]));
    }
    hi = make_uint4(h[0] | h[1] << 16, h[2] | h[3] << 16, h[4] | h[5] << 16, h[6] | h[7] << 16);
    lo = make_uint4(l[0] | l[1] << 16, l[2] | l[3] << 16, l[4] | l[5] << 16, l[6] | l[7] << 16);
  }
}

template <int B, bool PROD, bool XBF16>
__global__ __launch_bounds__(kEncWaves * 64) void encode128_kernel(
    const void *__restrict__ x, int64_t n, const uint4 *__restrict__ pi_hi,
    const uint4 *__restrict__ pi_lo, const uint4 *__restrict__ sp_hi,
    const uint4 *__restrict__ sp_lo, Codebook cb, uint32_t *__restrict__ idx_out,
    uint32_t *__restrict__ sgn_out, float *__restrict__ knorm_out,
    float *__restrict__ rnorm_out) {
  constexpr int kMats = PROD ? 4 : 2;
  __shared__ uint4 lds[kMats * kFragU4];
  for (int i = threadIdx.x; i < kFragU4; i += blockDim.x) {
    lds[i] = pi_hi[i];
    lds[kFragU4 + i] = pi_lo[i];
    if (PROD) {
      lds[2 * kFragU4 + i] = sp_hi[i];
      lds[3 * kFragU4 + i] = sp_lo[i];
    }
  }
  __syncthreads();
  const uint4 *Phi = lds, *Plo = lds + kFragU4, *Shi = lds + 2 * kFragU4,
              *Slo = lds + 3 * kFragU4;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int vcol = lane & 15;  // vector within a column tile
  const int g = lane >> 4;     // lane group: coordinates 4 g .. 4 g + 3 of every 16
  const int64_t nbatch = (n + kEncBatch - 1) / kEncBatch;

  for (int64_t batch = (int64_t)blockIdx.x * kEncWaves + wave; batch < nbatch;
       batch += (int64_t)gridDim.x * kEncWaves) {
    const int64_t v0 = batch * kEncBatch;
    uint4 xh[kEncCT][4], xl[kEncCT][4];
    float nu[kEncCT], inv[kEncCT];
#pragma unroll
    for (int ct = 0; ct < kEncCT; ++ct) {
      const int64_t row = v0 + 16 * ct + vcol;
      const bool valid = row < n;
      float ss = 0.f;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) load_x_frag<XBF16>(x, row, valid, kt, g, xh[ct][kt], xl[ct][kt], ss);
      ss += __shfl_xor(ss, 16);
      ss += __shfl_xor(ss, 32);
      nu[ct] = sqrtf(ss);
      inv[ct] = nu[ct] > 0.f ? 1.0f / nu[ct] : 0.f;
    }

    // Coordinates are processed in 4 blocks of 32 (kt2).  For each block:
    //  GEMM 1 rows 32 kt2 .. +31 (row tiles nt = 2 kt2, 2 kt2 + 1):
    //    Y^T = Pi X^T, rows = rotated coordinates, columns = vectors;
    //    lane (vcol, g) holds y[coordinate 16 nt + 4 g + i][vector 16 ct + vcol]
    //  bucketise those coordinates, pack their index bits, form the residual
    //  GEMM 2 contribution of K block kt2: Z^T += S'[:, block] rho^T[block, :]
    uint32_t planes[kEncCT][B > 0 ? B : 1];
    float rsq[kEncCT];
    f32x4 acc2[8][kEncCT];
#pragma unroll
    for (int ct = 0; ct < kEncCT; ++ct) {
      rsq[ct] = 0.f;
#pragma unroll
      for (int p = 0; p < (B > 0 ? B : 1); ++p) planes[ct][p] = 0u;
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) acc2[nt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll 1
    for (int kt2 = 0; kt2 < 4; ++kt2) {
      f32x4 acc[2][kEncCT];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int ct = 0; ct < kEncCT; ++ct) acc[h][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int nt = 2 * kt2 + h;
          const bf16x8 ah = as_bf16x8(Phi[(nt * 4 + kt) * 64 + lane]);
          const bf16x8 al = as_bf16x8(Plo[(nt * 4 + kt) * 64 + lane]);
#pragma unroll
          for (int ct = 0; ct < kEncCT; ++ct) {
            const bf16x8 bh = as_bf16x8(xh[ct][kt]);
            acc[h][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc[h][ct], 0, 0, 0);
            acc[h][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc[h][ct], 0, 0, 0);
            if (!XBF16)
              acc[h][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, as_bf16x8(xl[ct][kt]), acc[h][ct], 0, 0, 0);
          }
        }
      }
      uint32_t rh[kEncCT][4], rl[kEncCT][4];  // residual of this block as bf16 pairs
#pragma unroll
      for (int ct = 0; ct < kEncCT; ++ct) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          float rho[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float u = acc[h][ct][i] * inv[ct];
            float r = u;
            if (B > 0) {
              int idx = 0;
              float c = cb.c[0];
#pragma unroll
              for (int j = 0; j < (1 << B) - 1; ++j) {
                const bool ge = u >= cb.t[j];
                idx += ge ? 1 : 0;
                c = ge ? cb.c[j + 1] : c;
              }
              const int bit = 4 * (2 * kt2 + h) + i;
#pragma unroll
              for (int p = 0; p < B; ++p) planes[ct][p] |= (uint32_t)((idx >> p) & 1) << bit;
              r = u - c;
            }
            r = nu[ct] > 0.f ? r : 0.f;
            rsq[ct] += r * r;
            rho[i] = r;
          }
          // element e of the GEMM-2 operand for block kt2 is coordinate
          // 32 kt2 + 16 (e / 4) + 4 g + e % 4, i.e. e = 4 h + i
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const uint32_t h0 = bf16_rne(rho[2 * hh]), h1 = bf16_rne(rho[2 * hh + 1]);
            const uint32_t l0 = bf16_rne(rho[2 * hh] - bf16_to_f32(h0));
            const uint32_t l1 = bf16_rne(rho[2 * hh + 1] - bf16_to_f32(h1));
            rh[ct][2 * h + hh] = h0 | h1 << 16;
            rl[ct][2 * h + hh] = l0 | l1 << 16;
          }
        }
      }
      if (PROD) {
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
          const bf16x8 ah = as_bf16x8(Shi[(nt * 4 + kt2) * 64 + lane]);
          const bf16x8 al = as_bf16x8(Slo[(nt * 4 + kt2) * 64 + lane]);
#pragma unroll
          for (int ct = 0; ct < kEncCT; ++ct) {
            const bf16x8 bh = as_bf16x8(make_uint4(rh[ct][0], rh[ct][1], rh[ct][2], rh[ct][3]));
            const bf16x8 bl = as_bf16x8(make_uint4(rl[ct][0], rl[ct][1], rl[ct][2], rl[ct][3]));
            acc2[nt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc2[nt][ct], 0, 0, 0);
            acc2[nt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc2[nt][ct], 0, 0, 0);
            acc2[nt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc2[nt][ct], 0, 0, 0);
          }
        }
      }
    }
    // sign bits: acc2[nt][ct][i] = z[row 16 nt + 4 g + i][vector 16 ct + vcol]
    uint32_t sbits[kEncCT];
#pragma unroll
    for (int ct = 0; ct < kEncCT; ++ct) {
      uint32_t w = 0;
      if (PROD) {
#pragma unroll
        for (int nt = 0; nt < 8; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i) w |= (acc2[nt][ct][i] >= 0.f ? 1u : 0u) << (4 * nt + i);
      }
      sbits[ct] = w;
    }

    // ---- store
#pragma unroll
    for (int ct = 0; ct < kEncCT; ++ct) {
      const int64_t row = v0 + 16 * ct + vcol;
      float r2 = rsq[ct];
      r2 += __shfl_xor(r2, 16);
      r2 += __shfl_xor(r2, 32);
      if (row < n) {
        if (B > 0) {
          uint32_t *dst = idx_out + (row * 4 + g) * B;
#pragma unroll
          for (int p = 0; p < B; ++p) dst[p] = planes[ct][p];
        }
        if (PROD) sgn_out[row * 4 + g] = sbits[ct];
        if (g == 0) {
          knorm_out[row] = nu[ct];
          if (PROD) rnorm_out[row] = nu[ct] * sqrtf(r2);
        }
      }
    }
  }
}

template <int B, bool PROD>
static void launch_encode_t(const Derived &D, const void *x, int dtype, int64_t n,
                            tq_codes c, hipStream_t s, int grid) {
  const dim3 blk(kEncWaves * 64);
  const uint4 *ph = (const uint4 *)D.pi_hi, *pl = (const uint4 *)D.pi_lo;
  const uint4 *sh = (const uint4 *)D.sp_hi, *sl = (const uint4 *)D.sp_lo;
  if (dtype == TQ_BF16)
    encode128_kernel<B, PROD, true><<<grid, blk, 0, s>>>(x, n, ph, pl, sh, sl, D.cb, c.idx, c.sgn,
                                                         c.knorm, c.rnorm);
  else
    encode128_kernel<B, PROD, false><<<grid, blk, 0, s>>>(x, n, ph, pl, sh, sl, D.cb, c.idx, c.sgn,
                                                          c.knorm, c.rnorm);
}

static int num_cus(int dev) {
  static int cached[64] = {0};
  if (dev >= 0 && dev < 64 && cached[dev]) return cached[dev];
  int cu = 0;
  if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cu <= 0)
    cu = 256;
  if (dev >= 0 && dev < 64) cached[dev] = cu;
  return cu;
}

tq_status launch_encode(const Derived &D, const void *x, int dtype, int64_t n, tq_codes c,
                        hipStream_t s) {
  const int64_t nbatch = (n + kEncBatch - 1) / kEncBatch;
  const int64_t need = (nbatch + kEncWaves - 1) / kEncWaves;
  const int grid = (int)std::min<int64_t>(need, num_cus(D.device));
  const bool prod = D.p.mode == TQ_MODE_PROD;
  switch (D.B * 2 + (prod ? 1 : 0)) {
    case 0 * 2 + 1: launch_encode_t<0, true>(D, x, dtype, n, c, s, grid); break;
    case 1 * 2 + 1: launch_encode_t<1, true>(D, x, dtype, n, c, s, grid); break;
    case 2 * 2 + 1: launch_encode_t<2, true>(D, x, dtype, n, c, s, grid); break;
    case 3 * 2 + 1: launch_encode_t<3, true>(D, x, dtype, n, c, s, grid); break;
    case 4 * 2 + 1: launch_encode_t<4, true>(D, x, dtype, n, c, s, grid); break;
    case 1 * 2 + 0: launch_encode_t<1, false>(D, x, dtype, n, c, s, grid); break;
    case 2 * 2 + 0: launch_encode_t<2, false>(D, x, dtype, n, c, s, grid); break;
    case 3 * 2 + 0: launch_encode_t<3, false>(D, x, dtype, n, c, s, grid); break;
    case 4 * 2 + 0: launch_encode_t<4, false>(D, x, dtype, n, c, s, grid); break;
    default:
      set_error("tq_encode: unsupported B = %d", D.B);
      return TQ_ERR_UNSUPPORTED;
  }
  TQ_LAUNCH_CHECK();
  return TQ_OK;
}

// ===========================================================================
// Score, d = m = 128
// ===========================================================================
// Query operands, one block of 4 queries of one KV head ("query group"):
//   idx part: for part s (odd subset of planes) and half h2, MFMA 2 s + h2
//   sign part: MFMA 2 NP + h2
// Lane l (row = 4 jq + t: query jq, limb t; lane group kg = l / 16) dword w
// byte e multiplies the key bit at byte e, bit sl = 4 h2 + w of the key's
// plane word kg, i.e. coordinate 32 e + 16 (sl / 4) + 4 kg + sl % 4.
constexpr int kScoreWaves = 4;

__host__ __device__ constexpr int score_mfmas(int nparts, bool prod) {
  return 2 * nparts + (prod ? 2 : 0);
}

struct QConst {  // per query
  float idx_scale;  // 2^-E of the index part
  float idx_bias;   // sum_S coef_S * sum_c qt_c
  float sgn_scale;  // sqrt(pi/2)/m * 2^-E'
  float sgn_bias;   // sqrt(pi/2)/m * sum_r qs_r
};

// one workgroup per (KV head, query group)
template <bool PROD>
__global__ __launch_bounds__(256) void qprep128_kernel(const float *__restrict__ q, int64_t g,
                                                       int ngroups, const float *__restrict__ pi,
                                                       const float *__restrict__ s, Codebook cb,
                                                       int m, i32x4 *__restrict__ aops,
                                                       QConst *__restrict__ qc) {
  __shared__ float qin[4][128];
  __shared__ float qt[4][128];
  __shared__ float qs[4][128];
  __shared__ double red[4][4];
  __shared__ int expo[4][2];
  const int hg = blockIdx.x;
  const int h = hg / ngroups, grp = hg % ngroups;
  const int tid = threadIdx.x;
  for (int i = tid; i < 512; i += 256) {
    const int jq = i >> 7, c = i & 127;
    const int64_t qh = (int64_t)grp * 4 + jq;
    qin[jq][c] = qh < g ? q[((int64_t)h * g + qh) * 128 + c] : 0.f;
  }
  __syncthreads();
  for (int i = tid; i < 512; i += 256) {
    const int jq = i >> 7, c = i & 127;
    float a = 0.f, b = 0.f;
    for (int j = 0; j < 128; ++j) {
      a = fmaf(pi[c * 128 + j], qin[jq][j], a);
      if (PROD) b = fmaf(s[c * 128 + j], qin[jq][j], b);
    }
    qt[jq][c] = a;
    qs[jq][c] = b;
  }
  __syncthreads();
  const int NP = cb.nparts;
  if (tid < 4) {
    const int jq = tid;
    double mq = 0, ms = 0, sq = 0, ssum = 0, acoef = 0, amax = 0;
    for (int c = 0; c < 128; ++c) {
      mq = fmax(mq, fabs((double)qt[jq][c]));
      ms = fmax(ms, fabs((double)qs[jq][c]));
      sq += qt[jq][c];
      ssum += qs[jq][c];
    }
    for (int p = 0; p < NP; ++p) {
      acoef += cb.coef[p];
      amax = fmax(amax, fabs(cb.coef[p]));
    }
    // largest operand magnitude below 2^26 after scaling by 2^E
    int e1 = 0, e2 = 0;
    const double A1 = 2.0 * amax * mq, A2 = 2.0 * ms;
    int k;
    if (A1 > 0) { frexp(A1, &k); e1 = 26 - k; }
    if (A2 > 0) { frexp(A2, &k); e2 = 26 - k; }
    expo[jq][0] = e1;
    expo[jq][1] = e2;
    const double cq = sqrt(M_PI / 2.0) / m;
    QConst o;
    o.idx_scale = (float)ldexp(1.0, -e1);
    o.idx_bias = (float)(acoef * sq);
    o.sgn_scale = (float)(cq * ldexp(1.0, -e2));
    o.sgn_bias = (float)(cq * ssum);
    qc[(int64_t)hg * 4 + jq] = o;
    (void)red;
  }
  __syncthreads();
  const int NMF = score_mfmas(NP, PROD);
  for (int i = tid; i < NMF * 64; i += 256) {
    const int j = i >> 6, l = i & 63;
    const int row = l & 15, kg = l >> 4;
    const int jq = row >> 2, t = row & 3;
    const bool sgnpart = j >= 2 * NP;
    const int h2 = j & 1;
    const double coef = sgnpart ? 2.0 : 2.0 * cb.coef[j >> 1];
    const int E = expo[jq][sgnpart ? 1 : 0];
    int out[4];
    for (int w = 0; w < 4; ++w) {
      uint32_t packed = 0;
      const int sl = 4 * h2 + w;
      for (int e = 0; e < 4; ++e) {
        const int c = 32 * e + 16 * (sl >> 2) + 4 * kg + (sl & 3);
        const double v = coef * (double)(sgnpart ? qs[jq][c] : qt[jq][c]);
        long long Q = llrint(ldexp(v, E - sl));
        if (sl == 7) Q = -Q;
        // balanced base-128 digits, limb t
        long long digit = 0;
        for (int tt = 0; tt <= t; ++tt) {
          digit = ((Q + 64) & 127) - 64;
          Q = (Q - digit) / 128;
        }
        packed |= (uint32_t)(uint8_t)(int8_t)digit << (8 * e);
      }
      out[w] = (int)packed;
    }
    aops[((int64_t)hg * NMF + j) * 64 + l] = i32x4{out[0], out[1], out[2], out[3]};
  }
}

template <int B, bool PROD>
__global__ __launch_bounds__(kScoreWaves * 64) void score128_kernel(
    const i32x4 *__restrict__ aops, const QConst *__restrict__ qc,
    const uint32_t *__restrict__ idx, const uint32_t *__restrict__ sgn,
    const float *__restrict__ knorm, const float *__restrict__ rnorm, int64_t seq, int64_t g,
    int ngroups, int tiles_per_wave, Codebook cb, float *__restrict__ logits) {
  constexpr int NP = B == 0 ? 0 : (B == 1 ? 1 : B == 2 ? 2 : B == 3 ? 4 : 8);
  constexpr int NMF = score_mfmas(NP, PROD);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int hg = blockIdx.y;
  const int h = hg / ngroups, grp = hg % ngroups;
  const int kc = lane & 15, kg = lane >> 4;
  i32x4 A[NMF];
#pragma unroll
  for (int j = 0; j < NMF; ++j) A[j] = aops[((int64_t)hg * NMF + j) * 64 + lane];
  const QConst cst = qc[(int64_t)hg * 4 + kg];
  const int64_t qh = (int64_t)grp * 4 + kg;  // this lane's output query within the head
  const bool qvalid = qh < g;
  float *out = logits + ((int64_t)h * g + qh) * seq;

  const int64_t tiles = (seq + 15) / 16;
  const int64_t t0 = ((int64_t)blockIdx.x * kScoreWaves + wave) * tiles_per_wave;
  const int64_t t1 = t0 + tiles_per_wave < tiles ? t0 + tiles_per_wave : tiles;
  for (int64_t tile = t0; tile < t1; ++tile) {
    const int64_t pos = tile * 16 + kc;
    const bool valid = pos < seq;
    const int64_t vid = (int64_t)h * seq + (valid ? pos : 0);
    uint32_t pl[B > 0 ? B : 1];
#pragma unroll
    for (int p = 0; p < B; ++p) pl[p] = valid ? idx[(vid * 4 + kg) * B + p] : 0u;
    const uint32_t sw = PROD && valid ? sgn[vid * 4 + kg] : 0u;
    const float kn = valid ? knorm[vid] : 0.f;
    const float rn = PROD && valid ? rnorm[vid] : 0.f;
    i32x4 ai = {0, 0, 0, 0}, as = {0, 0, 0, 0};
#pragma unroll
    for (int sp = 0; sp < NP; ++sp) {
      uint32_t part = 0;
#pragma unroll
      for (int p = 0; p < B; ++p)
        if (cb.part_mask[sp] >> p & 1) part ^= pl[p];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const i32x4 bw = {(int)(part & (0x01010101u << (4 * h2 + 0))),
                          (int)(part & (0x01010101u << (4 * h2 + 1))),
                          (int)(part & (0x01010101u << (4 * h2 + 2))),
                          (int)(part & (0x01010101u << (4 * h2 + 3)))};
        ai = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[2 * sp + h2], bw, ai, 0, 0, 0);
      }
    }
    if (PROD) {
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const i32x4 bw = {(int)(sw & (0x01010101u << (4 * h2 + 0))),
                          (int)(sw & (0x01010101u << (4 * h2 + 1))),
                          (int)(sw & (0x01010101u << (4 * h2 + 2))),
                          (int)(sw & (0x01010101u << (4 * h2 + 3)))};
        as = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[2 * NP + h2], bw, as, 0, 0, 0);
      }
    }
    // lane (kc, kg) holds rows 4 kg + t (query kg, limb t) of column kc (this key)
    float li = 0.f, ls = 0.f;
    if (NP > 0) {
      const float vi = (float)ai[0] + 128.f * (float)ai[1] + 16384.f * (float)ai[2] +
                       2097152.f * (float)ai[3];
      li = kn * (vi * cst.idx_scale - cst.idx_bias);
    }
    if (PROD) {
      const float vs = (float)as[0] + 128.f * (float)as[1] + 16384.f * (float)as[2] +
                       2097152.f * (float)as[3];
      ls = rn * (vs * cst.sgn_scale - cst.sgn_bias);
    }
    if (valid && qvalid) out[pos] = li + ls;
  }
}

static int nparts_of(int B) { return B == 0 ? 0 : (B == 1 ? 1 : B == 2 ? 2 : B == 3 ? 4 : 8); }

size_t score_workspace_bytes(const Derived &D, int64_t n_kv, int64_t g) {
  const int64_t ngroups = (g + 3) / 4;
  const int NMF = score_mfmas(nparts_of(D.B), D.p.mode == TQ_MODE_PROD);
  return (size_t)n_kv * ngroups * ((size_t)NMF * 64 * sizeof(i32x4) + 4 * sizeof(QConst));
}

template <int B, bool PROD>
static void launch_score_t(const Derived &D, const float *q, int64_t n_kv, int64_t g,
                           tq_codes c, int64_t seq, float *logits, void *ws, hipStream_t s) {
  const int ngroups = (int)((g + 3) / 4);
  const int NMF = score_mfmas(nparts_of(B), PROD);
  i32x4 *aops = (i32x4 *)ws;
  QConst *qc = (QConst *)((char *)ws + (size_t)n_kv * ngroups * NMF * 64 * sizeof(i32x4));
  qprep128_kernel<PROD><<<dim3((unsigned)(n_kv * ngroups)), dim3(256), 0, s>>>(
      q, g, ngroups, D.pi32, D.s32, D.cb, D.p.m, aops, qc);
  const int64_t tiles = (seq + 15) / 16;
  const int tpw = 8;
  const int64_t chunks = (tiles + (int64_t)tpw * kScoreWaves - 1) / ((int64_t)tpw * kScoreWaves);
  score128_kernel<B, PROD><<<dim3((unsigned)chunks, (unsigned)(n_kv * ngroups)),
                             dim3(kScoreWaves * 64), 0, s>>>(aops, qc, c.idx, c.sgn, c.knorm,
                                                             c.rnorm, seq, g, ngroups, tpw, D.cb,
                                                             logits);
}

tq_status launch_score(const Derived &D, const float *q, int64_t n_kv, int64_t g, tq_codes c,
                       int64_t seq, float *logits, void *ws, hipStream_t s) {
  if ((uint64_t)n_kv * ((g + 3) / 4) > 65535u) {
    set_error("tq_score: n_kv * ceil(g/4) = %lld exceeds 65535", (long long)(n_kv * ((g + 3) / 4)));
    return TQ_ERR_UNSUPPORTED;
  }
  const bool prod = D.p.mode == TQ_MODE_PROD;
  switch (D.B * 2 + (prod ? 1 : 0)) {
    case 0 * 2 + 1: launch_score_t<0, true>(D, q, n_kv, g, c, seq, logits, ws, s); break;
    case 1 * 2 + 1: launch_score_t<1, true>(D, q, n_kv, g, c, seq, logits, ws, s); break;
    case 2 * 2 + 1: launch_score_t<2, true>(D, q, n_kv, g, c, seq, logits, ws, s); break;
    case 3 * 2 + 1: launch_score_t<3, true>(D, q, n_kv, g, c, seq, logits, ws, s); break;
    case 4 * 2 + 1: launch_score_t<4, true>(D, q, n_kv, g, c, seq, logits, ws, s); break;
    case 1 * 2 + 0: launch_score_t<1, false>(D, q, n_kv, g, c, seq, logits, ws, s); break;
    case 2 * 2 + 0: launch_score_t<2, false>(D, q, n_kv, g, c, seq, logits, ws, s); break;
    case 3 * 2 + 0: launch_score_t<3, false>(D, q, n_kv, g, c, seq, logits, ws, s); break;
    case 4 * 2 + 0: launch_score_t<4, false>(D, q, n_kv, g, c, seq, logits, ws, s); break;
    default:
      set_error("tq_score: unsupported B = %d", D.B);
      return TQ_ERR_UNSUPPORTED;
  }
  TQ_LAUNCH_CHECK();
  return TQ_OK;
}

// ===========================================================================
// Attend (not yet built on the device)
// ===========================================================================
size_t attend_workspace_bytes(const Derived &K, const Derived &V, int64_t batch, int64_t n_kv,
                              int64_t g, int64_t seq) {
  (void)K; (void)V; (void)batch; (void)n_kv; (void)g; (void)seq;
  return 16;
}

tq_status launch_attend(const Derived &K, const Derived &V, const float *q, int64_t batch,
                        int64_t n_kv, int64_t g, tq_codes k, tq_codes v, int64_t seq, float scale,
                        float *out, void *ws, hipStream_t s) {
  (void)K; (void)V; (void)q; (void)batch; (void)n_kv; (void)g; (void)k; (void)v; (void)seq;
  (void)scale; (void)out; (void)ws; (void)s;
  set_error("tq_attend: not built yet");
  return TQ_ERR_UNSUPPORTED;
}

}  // namespace tq
