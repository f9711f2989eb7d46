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
//     run on 16-bit MFMAs.  Bucket decisions need the rotated coordinates to
//     ~1e-7, so the matrices are split hi + lo (and float32 inputs and the
//     residual too), giving float32-level products: bfloat16 keys against the
//     bf16 split of Pi, float32 keys and the residual in fp16 hi + lo after a
//     power-of-two scaling of each vector (fp16 keeps 11 bits per piece).
//     The split matrices (Pi and S' = S Pi^T) live in LDS (128 KB) for the
//     life of a persistent workgroup.  The first GEMM's output registers are
//     already the second GEMM's operand layout, so the residual never leaves
//     registers, and each lane packs its own 32-bit words of index planes and
//     sign bits (the packed layout follows the MFMA output layout).
//   * score: logits from packed codes are integer dot products of bit planes
//     with the query.  A symmetric codebook is an odd multilinear function of
//     the +-1 bit signs, so c[idx] is a short sum of coefficient * (parity of
//     a subset of planes); the QJL term is a plain +-1 dot product.  Bits
//     become int8 MFMA operands with one AND per 4 bytes (bit k of every byte,
//     weight 2^(k mod 4)); the query side carries the weights 2^-(k mod 4) and
//     is split into four balanced base-128 int8 limbs that fill the 16 MFMA
//     rows (4 queries x 4 limbs).  int32 accumulation is exact.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>
#include <type_traits>

#include "tq_internal.h"

namespace tq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define TQ_LAUNCH_CHECK()                                                   \
  do {                                                                      \
    hipError_t e_ = hipGetLastError();                                      \
    if (e_ != hipSuccess) {                                                 \
      set_error("kernel launch failed: %s", hipGetErrorString(e_));        \
      return TQ_ERR_HIP;                                                    \
    }                                                                       \
  } while (0)

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// float -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// (a, b) -> packed hi = bf16(a) | bf16(b) << 16 and lo = bf16 of the remainders
__device__ __forceinline__ void split2(float a, float b, uint32_t &hi, uint32_t &lo) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 h = {(__bf16)a, (__bf16)b};
  const uint32_t hb = __builtin_bit_cast(uint32_t, h);
  const bf16x2 l = {(__bf16)(a - __uint_as_float(hb << 16)), (__bf16)(b - __uint_as_float(hb & 0xFFFF0000u))};
  hi = hb;
  lo = __builtin_bit_cast(uint32_t, l);
}

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ f16x8 as_f16x8(uint4 v) { return __builtin_bit_cast(f16x8, v); }

// two floats -> packed fp16, rounded toward zero (one v_cvt_pkrtz_f16_f32)
__device__ __forceinline__ uint32_t pk_f16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a, b));
}

// (a, b) -> packed fp16 hi and the packed fp16 of the remainders a - hi,
// b - hi (exact in float32): hi + lo carries a, b to about 2^-21 relative
__device__ __forceinline__ void split2h(float a, float b, uint32_t &hi, uint32_t &lo) {
  hi = pk_f16(a, b);
  const f16x2 h = __builtin_bit_cast(f16x2, hi);
  lo = pk_f16(a - (float)h[0], b - (float)h[1]);
}

// The same split in three instructions: the remainders a - hi, b - hi are
// formed and rounded to fp16 by one mixed-precision fma each (hi read as
// fp16, a and b as float32), written straight into the halves of lo.
__device__ __forceinline__ void split2h_mix(float a, float b, uint32_t &hi, uint32_t &lo) {
  hi = pk_f16(a, b);
  uint32_t l;
  asm("v_fma_mixlo_f16 %0, -%1, 1.0, %2 op_sel_hi:[1,0,0]\n\t"
      "v_fma_mixhi_f16 %0, -%1, 1.0, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
      : "=&v"(l)
      : "v"(hi), "v"(a), "v"(b));
  lo = l;
}

// Streaming accesses: packed codes that a call reads once and outputs it
// writes once go through the non-temporal path, so they do not displace
// reused data from the caches (measured: the 32-layer score call ~7% faster).
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t nt_load(const uint32_t *p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ float nt_load(const float *p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ u32x2 nt_load2(const uint32_t *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
}
__device__ __forceinline__ u32x4 nt_load4(const uint32_t *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}
__device__ __forceinline__ void nt_store(float *p, float v) { __builtin_nontemporal_store(v, p); }

// Raw buffer loads (non-temporal): a descriptor covers one region of `bytes`
// bytes; the address is the descriptor's base + a per-lane offset + a
// wave-uniform (scalar) offset, so a load whose offsets are loop constants
// costs no vector instruction.  The range check covers the per-lane offset
// only (a load whose per-lane offset lies past the region returns zeros); a
// scalar offset is used only where every access is known to be in range.
constexpr int kBufWord3 = 0x00020000;  // descriptor word 3 for raw dword loads
typedef __amdgpu_buffer_rsrc_t bufrsrc;
__device__ __forceinline__ bufrsrc buf_rsrc(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, kBufWord3);
}
__device__ __forceinline__ uint32_t buf_ld1(bufrsrc r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 2);
}
// N consecutive dwords
template <int N>
__device__ __forceinline__ void buf_ldn(bufrsrc r, uint32_t voff, uint32_t soff, uint32_t *out) {
  if constexpr (N == 1) {
    out[0] = __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 2);
  } else if constexpr (N == 2) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, 2);
    out[0] = v[0];
    out[1] = v[1];
  } else if constexpr (N == 3) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b96(r, (int)voff, (int)soff, 2);
    out[0] = v[0];
    out[1] = v[1];
    out[2] = v[2];
  } else {
    static_assert(N == 4, "1 to 4 dwords");
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 2);
    out[0] = v[0];
    out[1] = v[1];
    out[2] = v[2];
    out[3] = v[3];
  }
}

// Power-of-two scale of one encoded vector: with e the exponent of its norm
// nu (nu = f 2^e, f in [0.5, 1)), the kernels feed x 2^(1-e) (norm in [1, 2))
// to fp16 MFMAs against kEncScale times the matrices, so rotated coordinates
// and residuals come out multiplied by 2^(kEncScaleLog2 + 1 - e).  Returns
// that exponent (0 for a zero vector, whose inputs are all zero anyway).
__device__ __forceinline__ int enc_scale_exp(float nu) {
  return nu > 0.f ? kEncScaleLog2 + 1 - __builtin_amdgcn_frexp_expf(nu) : 0;
}

// a * b - c in one v_fma_f32 with a negated third operand (left to itself the
// compiler moves the negation into an integer XOR of c's sign)
__device__ __forceinline__ float fma_negc(float a, float b, float c) {
  float r;
  asm("v_fma_f32 %0, %1, %2, -%3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// w = 2 w + (bit of this lane in mask): one v_addc with the lane mask as
// carry-in, which shifts a compare result into a packed word.
__device__ __forceinline__ uint32_t shift_in(uint32_t w, uint64_t mask) {
  uint32_t r;
  uint64_t carry_out;
  asm("v_addc_co_u32_e64 %0, %1, %2, %2, %3" : "=v"(r), "=s"(carry_out) : "v"(w), "s"(mask));
  return r;
}

// ===========================================================================
// Encode, d = m = 128
// ===========================================================================
constexpr int kEncWaves = 16;         // waves per workgroup
constexpr int kEncCT = 1;             // 16-vector column tiles per wave batch
constexpr int kEncBatch = 16 * kEncCT;  // vectors per wave batch
constexpr int kFragU4 = kFragElems / 8;  // uint4 per fragment matrix (2048)

// X^T fragment of one 16-vector column tile, column block kt: lane (v, g)
// holds x[v][32 kt + 8 g .. + 7], as loaded (8 bf16 in raw[0], or 8 float32
// in raw[0], raw[1]), and adds their squares to sumsq.
template <bool XBF16>
__device__ __forceinline__ void load_x_raw(const void *__restrict__ x, int64_t row, bool valid,
                                           int kt, int g, uint4 (&raw)[2], float &sumsq) {
  if (XBF16) {
    const uint4 *p = reinterpret_cast<const uint4 *>(
        reinterpret_cast<const uint16_t *>(x) + row * 128 + 32 * kt + 8 * g);
    raw[0] = valid ? *p : make_uint4(0, 0, 0, 0);
    const uint32_t w[4] = {raw[0].x, raw[0].y, raw[0].z, raw[0].w};
    // squares of both bfloat16 halves in one v_dot2 each (the products are exact in float32)
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bf16x2 v = __builtin_bit_cast(bf16x2, w[i]);
      sumsq = __builtin_amdgcn_fdot2_f32_bf16(v, v, sumsq, false);
    }
  } else {
    const uint4 *p = reinterpret_cast<const uint4 *>(
        reinterpret_cast<const float *>(x) + row * 128 + 32 * kt + 8 * g);
    raw[0] = valid ? p[0] : make_uint4(0, 0, 0, 0);
    raw[1] = valid ? p[1] : make_uint4(0, 0, 0, 0);
    const uint32_t w[8] = {raw[0].x, raw[0].y, raw[0].z, raw[0].w, raw[1].x, raw[1].y, raw[1].z, raw[1].w};
#pragma unroll
    for (int i = 0; i < 8; ++i) sumsq = fmaf(__uint_as_float(w[i]), __uint_as_float(w[i]), sumsq);
  }
}

// bf16 MFMA operand of the same fragment (PolarQuant encoder): bf16 inputs
// as they are, float32 inputs split hi/lo.
template <bool XBF16>
__device__ __forceinline__ void load_x_frag(const void *__restrict__ x, int64_t row, bool valid,
                                            int kt, int g, uint4 &hi, uint4 &lo, float &sumsq) {
  uint4 raw[2];
  load_x_raw<XBF16>(x, row, valid, kt, g, raw, sumsq);
  if (XBF16) {
    hi = lo = raw[0];
  } else {
    const uint32_t w[8] = {raw[0].x, raw[0].y, raw[0].z, raw[0].w, raw[1].x, raw[1].y, raw[1].z, raw[1].w};
    uint32_t h[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) split2(__uint_as_float(w[2 * i]), __uint_as_float(w[2 * i + 1]), h[i], l[i]);
    hi = make_uint4(h[0], h[1], h[2], h[3]);
    lo = make_uint4(l[0], l[1], l[2], l[3]);
  }
}

// The fp16 MFMA operand of a loaded fragment, scaled by 2^sh (exact): bf16
// values fit fp16 exactly once the vector's norm is near 1; float32 values
// become fp16 hi + lo.
template <bool XBF16>
__device__ __forceinline__ void x_frag_f16(const uint4 (&raw)[2], int sh, uint4 &hi, uint4 &lo) {
  if (XBF16) {
    const uint32_t w[4] = {raw[0].x, raw[0].y, raw[0].z, raw[0].w};
    uint32_t h[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      h[i] = pk_f16(ldexpf(__uint_as_float(w[i] << 16), sh), ldexpf(__uint_as_float(w[i] & 0xFFFF0000u), sh));
    hi = make_uint4(h[0], h[1], h[2], h[3]);
    lo = hi;
  } else {
    const uint32_t w[8] = {raw[0].x, raw[0].y, raw[0].z, raw[0].w, raw[1].x, raw[1].y, raw[1].z, raw[1].w};
    uint32_t h[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      split2h(ldexpf(__uint_as_float(w[2 * i]), sh), ldexpf(__uint_as_float(w[2 * i + 1]), sh), h[i], l[i]);
    hi = make_uint4(h[0], h[1], h[2], h[3]);
    lo = make_uint4(l[0], l[1], l[2], l[3]);
  }
}

template <int B, bool PROD, bool XBF16>
__global__ __launch_bounds__(kEncWaves * 64) void encode128_kernel(
    const void *__restrict__ x, int64_t n, const uint4 *__restrict__ pi_hi,
    const uint4 *__restrict__ pi_lo, const uint4 *__restrict__ sp_hi,
    const uint4 *__restrict__ sp_lo, Codebook cb, uint32_t *__restrict__ idx_out,
    uint32_t *__restrict__ sgn_out, float *__restrict__ knorm_out,
    float *__restrict__ rnorm_out, const int64_t *__restrict__ slots, int64_t capacity) {
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
    float nu[kEncCT], ysc[kEncCT];
    int esh[kEncCT];
    // the codebook is odd: magnitudes only, scaled by ||x|| 2^esh
    constexpr int kHalf = B > 0 ? 1 << (B - 1) : 1;
    float cp[kEncCT][kHalf], tp[kEncCT][kHalf > 1 ? kHalf - 1 : 1];
#pragma unroll
    for (int ct = 0; ct < kEncCT; ++ct) {
      const int64_t row = v0 + 16 * ct + vcol;
      const bool valid = row < n;
      float ss = 0.f;
      uint4 raw[4][2];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) load_x_raw<XBF16>(x, row, valid, kt, g, raw[kt], ss);
      ss += __shfl_xor(ss, 16);
      ss += __shfl_xor(ss, 32);
      nu[ct] = sqrtf(ss);
      // x enters the fp16 MFMAs as x 2^(1-e) (norm in [1, 2)) against
      // kEncScale Pi, so y' = Pi x 2^esh; the codebook is scaled by the same
      // ||x|| 2^esh: y' is compared with t_j ||x|| 2^esh and the residual is
      // formed as y' - c ||x|| 2^esh = ||x|| 2^esh (u - c), with no division;
      // a zero vector gets y' = 0 and a zero residual
      esh[ct] = enc_scale_exp(nu[ct]);
      const float nus = ldexpf(nu[ct], esh[ct]);
      // bfloat16 keys enter a bf16 MFMA against the bf16 hi + lo split of Pi
      // as they are, so y = Pi x comes out unscaled: the boundaries are
      // scaled by ||x|| alone and the residual is brought to the fp16 scale
      // of GEMM 2 by the factor 2^esh inside its fma
      ysc[ct] = XBF16 ? ldexpf(1.f, esh[ct]) : 1.f;
      const float nut = XBF16 ? nu[ct] : nus;
      if (XBF16) {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) xh[ct][kt] = raw[kt][0];
      } else {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) x_frag_f16<XBF16>(raw[kt], esh[ct] - kEncScaleLog2, xh[ct][kt], xl[ct][kt]);
      }
#pragma unroll
      for (int j = 0; j < kHalf; ++j) cp[ct][j] = B > 0 ? cb.c[kHalf + j] * nus : 0.f;
      // (for a zero vector the unscaled boundaries reproduce the u = 0 decisions)
#pragma unroll
      for (int j = 0; j + 1 < kHalf; ++j) tp[ct][j] = nu[ct] > 0.f ? cb.t[kHalf + j] * nut : cb.t[kHalf + j];
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
    }
    // One 32-coordinate block kt2: GEMM 1 rows 32 kt2 .. +31, bucketise,
    // pack, residual, GEMM-2 contribution.  The first block starts the GEMM-2
    // accumulators from zero inside the MFMA (no register clearing).
#define TQ_ENC_BLOCK(KT2, FIRST)                                                                                                            \
  do {                                                                                                                                      \
    const uint4 *Pk_ = Phi + 2 * (KT2) * 4 * 64 + lane;                                                                                     \
    int so_ = (KT2) * 64; asm volatile("" : "+s"(so_));                                                                                     \
    const uint4 *Sk_ = Shi + so_ + lane;                                                                                                    \
        f32x4 acc[2][kEncCT];                                                                                                               \
  _Pragma("unroll")                                                                                                                         \
        for (int h = 0; h < 2; ++h)                                                                                                         \
  _Pragma("unroll")                                                                                                                         \
          for (int ct = 0; ct < kEncCT; ++ct) acc[h][ct] = f32x4{0.f, 0.f, 0.f, 0.f};                                                       \
  _Pragma("unroll")                                                                                                                         \
        for (int kt = 0; kt < 4; ++kt) {                                                                                                    \
  _Pragma("unroll")                                                                                                                         \
          for (int h = 0; h < 2; ++h) {                                                                                                     \
            const uint4 ah_ = Pk_[(h * 4 + kt) * 64];                                                                                      \
            const uint4 al_ = Pk_[kFragU4 + (h * 4 + kt) * 64];                                                                            \
  _Pragma("unroll")                                                                                                                         \
            for (int ct = 0; ct < kEncCT; ++ct) {                                                                                           \
              if (XBF16) {                                                                                                                  \
                const bf16x8 bh = as_bf16x8(xh[ct][kt]);                                                                                    \
                acc[h][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ah_), bh, acc[h][ct], 0, 0, 0);                              \
                acc[h][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(al_), bh, acc[h][ct], 0, 0, 0);                              \
              } else {                                                                                                                      \
                const f16x8 ah = as_f16x8(ah_), al = as_f16x8(al_), bh = as_f16x8(xh[ct][kt]);                                              \
                acc[h][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bh, acc[h][ct], 0, 0, 0);                                           \
                acc[h][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, bh, acc[h][ct], 0, 0, 0);                                           \
                acc[h][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, as_f16x8(xl[ct][kt]), acc[h][ct], 0, 0, 0);                         \
              }                                                                                                                             \
            }                                                                                                                               \
          }                                                                                                                                 \
        }                                                                                                                                   \
        uint32_t rh[kEncCT][4], rl[kEncCT][4];                                                                                              \
  _Pragma("unroll")                                                                                                                         \
        for (int ct = 0; ct < kEncCT; ++ct) {                                                                                               \
  _Pragma("unroll")                                                                                                                         \
          for (int h = 0; h < 2; ++h) {                                                                                                     \
            float rho[4];                                                                                                                   \
  _Pragma("unroll")                                                                                                                         \
            for (int i = 0; i < 4; ++i) {                                                                                                   \
              const float y = acc[h][ct][i];                                                                                                \
              float r = XBF16 ? y * ysc[ct] : y;                                                                                            \
              if (B > 0) {                                                                                                                  \
                const float a = fabsf(y);                                                                                                   \
                uint64_t gm[kHalf > 1 ? kHalf - 1 : 1];                                                                                     \
                float cm = cp[ct][0];                                                                                                       \
  _Pragma("unroll")                                                                                                                         \
                for (int j = 0; j < kHalf - 1; ++j) {                                                                                       \
                  const bool gj = a >= tp[ct][j];                                                                                           \
                  gm[j] = __builtin_amdgcn_ballot_w64(gj);                                                                                  \
                  cm = gj ? cp[ct][j + 1] : cm;                                                                                             \
                }                                                                                                                           \
  _Pragma("unroll")                                                                                                                         \
                for (int p = 0; p + 1 < B; ++p) {                                                                                           \
                  uint64_t mk = 0;                                                                                                          \
  _Pragma("unroll")                                                                                                                         \
                  for (int j = (1 << p) - 1; j < kHalf - 1; j += (1 << p)) mk ^= gm[j];                                                     \
                  planes[ct][p] = shift_in(planes[ct][p], mk);                                                                              \
                }                                                                                                                           \
                planes[ct][B - 1] = __builtin_amdgcn_alignbit(planes[ct][B - 1], __float_as_uint(y), 31);                                   \
                r = XBF16 ? fma_negc(y, ysc[ct], __builtin_copysignf(cm, y)) : y - __builtin_copysignf(cm, y);                              \
              }                                                                                                                             \
              rsq[ct] = fmaf(r, r, rsq[ct]);                                                                                                \
              rho[i] = r;                                                                                                                   \
            }                                                                                                                               \
  _Pragma("unroll")                                                                                                                         \
            for (int hh = 0; hh < 2; ++hh) split2h_mix(rho[2 * hh], rho[2 * hh + 1], rh[ct][2 * h + hh], rl[ct][2 * h + hh]);               \
          }                                                                                                                                 \
        }                                                                                                                                   \
        if (PROD) {                                                                                                                         \
  _Pragma("unroll")                                                                                                                         \
          for (int nt = 0; nt < 8; ++nt) {                                                                                                  \
            const f16x8 ah = as_f16x8(Sk_[nt * 4 * 64]);                                                                                    \
            const f16x8 al = as_f16x8(Sk_[kFragU4 + nt * 4 * 64]);                                                                          \
  _Pragma("unroll")                                                                                                                         \
            for (int ct = 0; ct < kEncCT; ++ct) {                                                                                           \
              const f16x8 bh = as_f16x8(make_uint4(rh[ct][0], rh[ct][1], rh[ct][2], rh[ct][3]));                                            \
              const f16x8 bl = as_f16x8(make_uint4(rl[ct][0], rl[ct][1], rl[ct][2], rl[ct][3]));                                            \
              acc2[nt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bh, (FIRST) ? f32x4{0.f, 0.f, 0.f, 0.f} : acc2[nt][ct], 0, 0, 0);   \
              acc2[nt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bl, acc2[nt][ct], 0, 0, 0);                                         \
              acc2[nt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, bh, acc2[nt][ct], 0, 0, 0);                                         \
            }                                                                                                                               \
          }                                                                                                                                 \
        }                                                                                                                                   \
  } while (0)
    TQ_ENC_BLOCK(0, true);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll 1
    for (int kt2 = 1; kt2 < 4; ++kt2) TQ_ENC_BLOCK(kt2, false);
#undef TQ_ENC_BLOCK
    // sign bits: acc2[nt][ct][i] = z[row 16 nt + 4 g + i][vector 16 ct + vcol],
    // shifted in from the highest row down so that row 4 nt + i lands at bit
    // 4 nt + i.  One v_alignbit per bit shifts in the float's sign bit (1 for
    // z < 0), and the word is complemented once at the end.  An exactly zero
    // z comes out of the MFMA accumulation as +0 (its first product starts
    // from +0), so it gets bit 1 as the z >= 0 rule says.
    uint32_t sbits[kEncCT];
#pragma unroll
    for (int ct = 0; ct < kEncCT; ++ct) {
      uint32_t w = 0;
      if (PROD) {
#pragma unroll
        for (int nt = 7; nt >= 0; --nt)
#pragma unroll
          for (int i = 3; i >= 0; --i) w = __builtin_amdgcn_alignbit(w, __float_as_uint(acc2[nt][ct][i]), 31);
        w = ~w;
      }
      sbits[ct] = w;
    }
    // index planes were shifted in from the lowest coordinate up: the top
    // plane holds the sign bits of y (1 for y < 0) and plane p < B - 1 the
    // XOR of its boundary masks, so plane p = (y >= 0) XNOR masks = sign XOR
    // masks, and the top plane (y >= 0) = NOT sign; then reverse them
#pragma unroll
    for (int ct = 0; ct < kEncCT; ++ct) {
      if (B > 0) {
        const uint32_t sw = planes[ct][B > 0 ? B - 1 : 0];
#pragma unroll
        for (int p = 0; p + 1 < B; ++p) planes[ct][p] ^= sw;
        planes[ct][B > 0 ? B - 1 : 0] = ~sw;
      }
#pragma unroll
      for (int p = 0; p < (B > 0 ? B : 1); ++p) planes[ct][p] = __builtin_bitreverse32(planes[ct][p]);
    }

    // ---- store
#pragma unroll
    for (int ct = 0; ct < kEncCT; ++ct) {
      const int64_t row = v0 + 16 * ct + vcol;
      float r2 = rsq[ct];
      r2 += __shfl_xor(r2, 16);
      r2 += __shfl_xor(r2, 32);
      // destination: the row itself, or its slot in a store (out-of-range
      // slots are skipped)
      const int64_t orow = slots != nullptr && row < n ? slots[row] : row;
      if (row < n && (slots == nullptr || (orow >= 0 && orow < capacity))) {
        if (B > 0) {
          uint32_t *dst = idx_out + (orow * 4 + g) * B;
#pragma unroll
          for (int p = 0; p < B; ++p) dst[p] = planes[ct][p];
        }
        if (PROD) sgn_out[orow * 4 + g] = sbits[ct];
        if (g == 0) {
          knorm_out[orow] = nu[ct];
          if (PROD) rnorm_out[orow] = ldexpf(sqrtf(r2), -esh[ct]);
        }
      }
    }
  }
}

template <int B, bool PROD>
static void launch_encode_t(const Derived &D, const void *x, int dtype, int64_t n,
                            tq_codes c, hipStream_t s, int grid, const int64_t *slots,
                            int64_t capacity) {
  const dim3 blk(kEncWaves * 64);
  const uint4 *ph = (const uint4 *)D.pi16_hi, *pl = (const uint4 *)D.pi16_lo;
  const uint4 *sh = (const uint4 *)D.sp16_hi, *sl = (const uint4 *)D.sp16_lo;
  if (dtype == TQ_BF16)  // bfloat16 keys: GEMM 1 on bf16 MFMAs against the bf16 split of Pi
    encode128_kernel<B, PROD, true><<<grid, blk, 0, s>>>(x, n, (const uint4 *)D.pi_hi, (const uint4 *)D.pi_lo,
                                                         sh, sl, D.cb, c.idx, c.sgn,
                                                         c.knorm, c.rnorm, slots, capacity);
  else
    encode128_kernel<B, PROD, false><<<grid, blk, 0, s>>>(x, n, ph, pl, sh, sl, D.cb, c.idx, c.sgn,
                                                          c.knorm, c.rnorm, slots, capacity);
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

static tq_status launch_encode128(const Derived &D, const void *x, int dtype, int64_t n, tq_codes c,
                                  hipStream_t s, const int64_t *slots, int64_t capacity) {
  const int64_t nbatch = (n + kEncBatch - 1) / kEncBatch;
  const int64_t need = (nbatch + kEncWaves - 1) / kEncWaves;
  // one workgroup per CU holds the 128 KB of prod-mode fragments; mse mode (64 KB) fits two
  const int per_cu = D.p.mode == TQ_MODE_PROD ? 1 : 2;
  const int grid = (int)std::min<int64_t>(need, (int64_t)num_cus(D.device) * per_cu);
  const bool prod = D.p.mode == TQ_MODE_PROD;
  switch (D.B * 2 + (prod ? 1 : 0)) {
    case 0 * 2 + 1: launch_encode_t<0, true>(D, x, dtype, n, c, s, grid, slots, capacity); break;
    case 1 * 2 + 1: launch_encode_t<1, true>(D, x, dtype, n, c, s, grid, slots, capacity); break;
    case 2 * 2 + 1: launch_encode_t<2, true>(D, x, dtype, n, c, s, grid, slots, capacity); break;
    case 3 * 2 + 1: launch_encode_t<3, true>(D, x, dtype, n, c, s, grid, slots, capacity); break;
    case 4 * 2 + 1: launch_encode_t<4, true>(D, x, dtype, n, c, s, grid, slots, capacity); break;
    case 1 * 2 + 0: launch_encode_t<1, false>(D, x, dtype, n, c, s, grid, slots, capacity); break;
    case 2 * 2 + 0: launch_encode_t<2, false>(D, x, dtype, n, c, s, grid, slots, capacity); break;
    case 3 * 2 + 0: launch_encode_t<3, false>(D, x, dtype, n, c, s, grid, slots, capacity); break;
    case 4 * 2 + 0: launch_encode_t<4, false>(D, x, dtype, n, c, s, grid, slots, capacity); break;
    default:
      set_error("tq_encode: unsupported B = %d", D.B);
      return TQ_ERR_UNSUPPORTED;
  }
  TQ_LAUNCH_CHECK();
  return TQ_OK;
}

// ===========================================================================
// Encode, general shapes (d, m multiples of 128 up to 1024)
// ===========================================================================
// Two tiled GEMMs with fused epilogues, run over chunks of at most kGenChunk
// vectors:
//   1: Y^T = Pi X^T.  The epilogue bucketises, packs the index planes, forms
//      the residual rho = y - ||x|| c[idx] and stores it as bf16 hi/lo pairs
//      already in the second GEMM's operand layout, plus per-row-block
//      partial sums of rho^2.
//   2: Z^T = S' rho^T.  The epilogue packs the sign bits and finishes ||r||.
// Workgroup tile: one 128-row block mt of the matrix x 128 vectors.  4 waves,
// each owning 32 vectors (two 16-vector column tiles) of all 128 rows, so a
// lane ends with whole 32-bit words of the packed layout (rows
// 128 mt + 16 nt + 4 g + i, nt < 8, i < 4, are word 4 mt + g, bit 4 nt + i).
// The matrix operand streams through LDS in 64-wide K stages (32 KB, double
// buffered); the vector operand goes from global memory straight to
// registers, one stage ahead.
constexpr int kGW = 4;                      // waves per workgroup
constexpr int kGCT = 2;                     // 16-vector column tiles per wave
constexpr int kGVec = kGW * 16 * kGCT;      // vectors per workgroup tile (128)
constexpr int kGKB = 2;                     // 32-wide K blocks per stage
constexpr int kGStage = kGKB * 8 * 2 * 64;  // uint4 per stage (32 KB)
constexpr int kGPer = kGStage / (kGW * 64); // uint4 per thread per stage
constexpr int64_t kGenChunk = 32768;        // vectors per GEMM pair

// Workgroup -> (vector tile, row block).  Workgroups are dispatched to the 8
// XCDs round robin; give each XCD a contiguous range of tiles, row block
// fastest, so the row blocks of one vector tile share that XCD's L2.
__device__ __forceinline__ void gen_tile(int64_t T, int MT, int64_t &vt, int &mt) {
  const int64_t bid = blockIdx.x;
  const int64_t t = (T % 8 == 0) ? (bid % 8) * (T / 8) + bid / 8 : bid;
  vt = t / MT;
  mt = (int)(t % MT);
}

// Copy one K stage of the matrix fragments (rows of block mt) to registers.
__device__ __forceinline__ void gen_load_a(const uint4 *__restrict__ fbase, int NT, int stage,
                                           int tid, u32x4 (&r)[kGPer]) {
#pragma unroll
  for (int j = 0; j < kGPer; ++j) {
    const int i = tid + j * kGW * 64;
    const int ktl = i >> 10, rest = i & 1023;
    r[j] = reinterpret_cast<const u32x4 *>(fbase)[(size_t)(kGKB * stage + ktl) * NT * 128 + rest];
  }
}

// Vector operand of one K stage for the first GEMM: lane (vcol, g) of column
// tile ct holds x[v][32 kt + 8 g .. + 7] (two uint4 of float32, or one of bf16).
template <bool XBF16>
__device__ __forceinline__ void gen_load_x(const void *__restrict__ x, int d, const int64_t (&vrow)[kGCT],
                                           const bool (&vok)[kGCT], int g, int stage,
                                           u32x4 (&r)[kGCT][kGKB][XBF16 ? 1 : 2]) {
#pragma unroll
  for (int ct = 0; ct < kGCT; ++ct)
#pragma unroll
    for (int kb = 0; kb < kGKB; ++kb) {
      const int col = 32 * (kGKB * stage + kb) + 8 * g;
      if (XBF16) {
        const u32x4 *p = reinterpret_cast<const u32x4 *>(
            reinterpret_cast<const uint16_t *>(x) + vrow[ct] * d + col);
        r[ct][kb][0] = vok[ct] ? p[0] : u32x4{0u, 0u, 0u, 0u};
      } else {
        const u32x4 *p = reinterpret_cast<const u32x4 *>(
            reinterpret_cast<const float *>(x) + vrow[ct] * d + col);
        r[ct][kb][0] = vok[ct] ? p[0] : u32x4{0u, 0u, 0u, 0u};
        r[ct][kb][XBF16 ? 0 : 1] = vok[ct] ? p[1] : u32x4{0u, 0u, 0u, 0u};
      }
    }
}

// Residual operand of one K stage for the second GEMM (bf16 hi, lo).
__device__ __forceinline__ void gen_load_rho(const uint4 *__restrict__ rho, int64_t stride,
                                             const int64_t (&vrow)[kGCT], int g, int stage,
                                             u32x4 (&r)[kGCT][kGKB][2]) {
#pragma unroll
  for (int ct = 0; ct < kGCT; ++ct)
#pragma unroll
    for (int kb = 0; kb < kGKB; ++kb) {
      const u32x4 *p = reinterpret_cast<const u32x4 *>(rho) +
                       (((size_t)(kGKB * stage + kb) * stride + vrow[ct]) * 4 + g) * 2;
      r[ct][kb][0] = p[0];
      r[ct][kb][1] = p[1];
    }
}

template <int B, bool PROD, bool XBF16>
__global__ __launch_bounds__(kGW * 64) void encode_gemm1_kernel(
    const void *__restrict__ x, int64_t n, int d, const uint4 *__restrict__ frag, Codebook cb,
    uint32_t *__restrict__ idx_out, const float *__restrict__ knorm, uint4 *__restrict__ rho,
    float *__restrict__ rsq_part, int64_t stride) {
  __shared__ u32x4 As[2][kGStage];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int vcol = lane & 15, g = lane >> 4;
  const int MT = d >> 7, NT = d >> 4, KT = d >> 5, S = KT / kGKB;
  const int64_t VT = (n + kGVec - 1) / kGVec;
  int64_t vt;
  int mt;
  gen_tile(VT * MT, MT, vt, mt);
  int64_t vrow[kGCT];
  bool vok[kGCT];
#pragma unroll
  for (int ct = 0; ct < kGCT; ++ct) {
    vrow[ct] = vt * kGVec + wave * (16 * kGCT) + 16 * ct + vcol;
    vok[ct] = vrow[ct] < n;
  }
  const uint4 *fbase = frag + (size_t)8 * mt * 128;
  // the norms (from the norm pass) and each vector's power-of-two scale
  float nu[kGCT];
  int esh[kGCT];
#pragma unroll
  for (int ct = 0; ct < kGCT; ++ct) {
    nu[ct] = vok[ct] ? knorm[vrow[ct]] : 0.f;
    esh[ct] = enc_scale_exp(nu[ct]);
  }

  // vector operand of one stage: lane (vcol, g) holds x[v][32 kt + 8 g .. + 7]
  constexpr int XU = XBF16 ? 1 : 2;
  u32x4 xr[kGCT][kGKB][XU], xn[kGCT][kGKB][XU];
  f32x4 acc[8][kGCT];
#pragma unroll
  for (int ct = 0; ct < kGCT; ++ct) {
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) acc[nt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  u32x4 ar[kGPer];
  gen_load_a(fbase, NT, 0, tid, ar);
  gen_load_x<XBF16>(x, d, vrow, vok, g, 0, xr);
#pragma unroll
  for (int j = 0; j < kGPer; ++j) As[0][tid + j * kGW * 64] = ar[j];
  __syncthreads();

#pragma unroll 1
  for (int st = 0; st < S; ++st) {
    const int cur = st & 1;
    if (st + 1 < S) {
      gen_load_a(fbase, NT, st + 1, tid, ar);
      gen_load_x<XBF16>(x, d, vrow, vok, g, st + 1, xn);
    }
#pragma unroll
    for (int kb = 0; kb < kGKB; ++kb) {
      f16x8 bh[kGCT], bl[kGCT];
#pragma unroll
      for (int ct = 0; ct < kGCT; ++ct) {
        // x 2^(1-e) as fp16 (hi + lo for float32 inputs)
        uint4 raw[2], h, l;
        raw[0] = make_uint4(xr[ct][kb][0][0], xr[ct][kb][0][1], xr[ct][kb][0][2], xr[ct][kb][0][3]);
        raw[1] = make_uint4(xr[ct][kb][XU - 1][0], xr[ct][kb][XU - 1][1], xr[ct][kb][XU - 1][2],
                            xr[ct][kb][XU - 1][3]);
        x_frag_f16<XBF16>(raw, esh[ct] - kEncScaleLog2, h, l);
        bh[ct] = as_f16x8(h);
        bl[ct] = as_f16x8(l);
      }
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        const f16x8 ah = __builtin_bit_cast(f16x8, As[cur][(kb * 8 + nt) * 128 + lane]);
        const f16x8 al = __builtin_bit_cast(f16x8, As[cur][(kb * 8 + nt) * 128 + 64 + lane]);
#pragma unroll
        for (int ct = 0; ct < kGCT; ++ct) {
          acc[nt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bh[ct], acc[nt][ct], 0, 0, 0);
          acc[nt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, bh[ct], acc[nt][ct], 0, 0, 0);
          if (!XBF16)
            acc[nt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bl[ct], acc[nt][ct], 0, 0, 0);
        }
      }
    }
    if (st + 1 < S) {
#pragma unroll
      for (int j = 0; j < kGPer; ++j) As[cur ^ 1][tid + j * kGW * 64] = ar[j];
#pragma unroll
      for (int ct = 0; ct < kGCT; ++ct)
#pragma unroll
        for (int kb = 0; kb < kGKB; ++kb)
#pragma unroll
          for (int u = 0; u < XU; ++u) xr[ct][kb][u] = xn[ct][kb][u];
    }
    __syncthreads();
  }

  // ---- epilogue: acc[nt][ct][i] = ||x|| 2^esh u at row 128 mt + 16 nt + 4 g + i
#pragma unroll
  for (int ct = 0; ct < kGCT; ++ct) {
    const float nus = ldexpf(nu[ct], esh[ct]);
    float cs[1 << B], ts[(1 << B) > 1 ? (1 << B) - 1 : 1];
#pragma unroll
    for (int j = 0; j < (1 << B); ++j) cs[j] = cb.c[j] * nus;
#pragma unroll
    for (int j = 0; j + 1 < (1 << B); ++j) ts[j] = nu[ct] > 0.f ? cb.t[j] * nus : cb.t[j];
    uint32_t planes[B > 0 ? B : 1];
#pragma unroll
    for (int p = 0; p < (B > 0 ? B : 1); ++p) planes[p] = 0u;
    float rsq = 0.f;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float y = acc[nt][ct][i];
        float r = y;
        if (B > 0) {
          // thermometer code, parity bits shifted in (see the d = 128 kernel)
          bool gj[(1 << B) > 1 ? (1 << B) - 1 : 1];
          float c = cs[0];
#pragma unroll
          for (int j = 0; j < (1 << B) - 1; ++j) {
            gj[j] = y >= ts[j];
            c = gj[j] ? cs[j + 1] : c;
          }
#pragma unroll
          for (int p = 0; p < B; ++p) {
            bool bit = false;
#pragma unroll
            for (int j = (1 << p) - 1; j < (1 << B) - 1; j += (1 << p)) bit ^= gj[j];
            planes[p] = planes[p] + planes[p] + (bit ? 1u : 0u);
          }
          r = y - c;
        }
        rsq = fmaf(r, r, rsq);
        acc[nt][ct][i] = r;
      }
    const int64_t v = vrow[ct];
    if (B > 0 && vok[ct]) {
      uint32_t *dst = idx_out + (v * (d >> 5) + 4 * mt + g) * B;
#pragma unroll
      for (int p = 0; p < B; ++p) dst[p] = __builtin_bitreverse32(planes[p]);
    }
    if (PROD) {
      rsq += __shfl_xor(rsq, 16);
      rsq += __shfl_xor(rsq, 32);
      if (g == 0) rsq_part[v * MT + mt] = rsq;
      // K block kt = 4 mt + kk of the second GEMM: element e of lane group g is
      // coordinate 32 kt + 16 (e / 4) + 4 g + e % 4 = row tile 2 kk + e / 4, i = e % 4
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        uint32_t h[4], l[4];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          split2h(acc[2 * kk + hh][ct][0], acc[2 * kk + hh][ct][1], h[2 * hh], l[2 * hh]);
          split2h(acc[2 * kk + hh][ct][2], acc[2 * kk + hh][ct][3], h[2 * hh + 1], l[2 * hh + 1]);
        }
        uint4 *dst = rho + (((size_t)(4 * mt + kk) * stride + v) * 4 + g) * 2;
        dst[0] = make_uint4(h[0], h[1], h[2], h[3]);
        dst[1] = make_uint4(l[0], l[1], l[2], l[3]);
      }
    }
  }
}

__global__ __launch_bounds__(kGW * 64) void encode_gemm2_kernel(
    const uint4 *__restrict__ rho, const float *__restrict__ rsq_part, int64_t n, int64_t stride,
    int d, int m, const uint4 *__restrict__ frag, const float *__restrict__ knorm,
    uint32_t *__restrict__ sgn_out, float *__restrict__ rnorm_out) {
  __shared__ u32x4 As[2][kGStage];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int vcol = lane & 15, g = lane >> 4;
  const int MT = m >> 7, NT = m >> 4, KT = d >> 5, S = KT / kGKB;
  const int64_t VT = (n + kGVec - 1) / kGVec;
  int64_t vt;
  int mt;
  gen_tile(VT * MT, MT, vt, mt);
  int64_t vrow[kGCT];
#pragma unroll
  for (int ct = 0; ct < kGCT; ++ct) vrow[ct] = vt * kGVec + wave * (16 * kGCT) + 16 * ct + vcol;
  const uint4 *fbase = frag + (size_t)8 * mt * 128;

  // residual operand of one stage (written for every vector of the padded tile)
  u32x4 xr[kGCT][kGKB][2], xn[kGCT][kGKB][2];

  f32x4 acc[8][kGCT];
#pragma unroll
  for (int ct = 0; ct < kGCT; ++ct)
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) acc[nt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  u32x4 ar[kGPer];
  gen_load_a(fbase, NT, 0, tid, ar);
  gen_load_rho(rho, stride, vrow, g, 0, xr);
#pragma unroll
  for (int j = 0; j < kGPer; ++j) As[0][tid + j * kGW * 64] = ar[j];
  __syncthreads();

#pragma unroll 1
  for (int st = 0; st < S; ++st) {
    const int cur = st & 1;
    if (st + 1 < S) {
      gen_load_a(fbase, NT, st + 1, tid, ar);
      gen_load_rho(rho, stride, vrow, g, st + 1, xn);
    }
#pragma unroll
    for (int kb = 0; kb < kGKB; ++kb) {
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        const f16x8 ah = __builtin_bit_cast(f16x8, As[cur][(kb * 8 + nt) * 128 + lane]);
        const f16x8 al = __builtin_bit_cast(f16x8, As[cur][(kb * 8 + nt) * 128 + 64 + lane]);
#pragma unroll
        for (int ct = 0; ct < kGCT; ++ct) {
          const f16x8 bh = __builtin_bit_cast(f16x8, xr[ct][kb][0]), bl = __builtin_bit_cast(f16x8, xr[ct][kb][1]);
          acc[nt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bh, acc[nt][ct], 0, 0, 0);
          acc[nt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bl, acc[nt][ct], 0, 0, 0);
          acc[nt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, bh, acc[nt][ct], 0, 0, 0);
        }
      }
    }
    if (st + 1 < S) {
#pragma unroll
      for (int j = 0; j < kGPer; ++j) As[cur ^ 1][tid + j * kGW * 64] = ar[j];
#pragma unroll
      for (int ct = 0; ct < kGCT; ++ct)
#pragma unroll
        for (int kb = 0; kb < kGKB; ++kb) {
          xr[ct][kb][0] = xn[ct][kb][0];
          xr[ct][kb][1] = xn[ct][kb][1];
        }
    }
    __syncthreads();
  }

  // ---- epilogue: sign bit of z at row 128 mt + 16 nt + 4 g + i -> word 4 mt + g, bit 4 nt + i
  const int QT = d >> 7;
#pragma unroll
  for (int ct = 0; ct < kGCT; ++ct) {
    const int64_t v = vrow[ct];
    if (v >= n) continue;
    uint32_t w = 0;
#pragma unroll
    for (int nt = 7; nt >= 0; --nt)
#pragma unroll
      for (int i = 3; i >= 0; --i) w = w + w + (acc[nt][ct][i] >= 0.f ? 1u : 0u);
    sgn_out[v * (m >> 5) + 4 * mt + g] = w;
    if (mt == 0 && g == 0) {
      float r2 = 0.f;
      for (int j = 0; j < QT; ++j) r2 += rsq_part[v * QT + j];
      rnorm_out[v] = ldexpf(sqrtf(r2), -enc_scale_exp(knorm[v]));
    }
  }
}

size_t encode_workspace_bytes(const tq_params &p, int64_t n) {
  if (is_d128(p) || p.mode != TQ_MODE_PROD || n <= 0) return 0;
  const int64_t nc = std::min<int64_t>((n + kGVec - 1) / kGVec * kGVec, kGenChunk);
  return (size_t)nc * (4 * (size_t)p.d + 4 * (size_t)(p.d / 128));
}

// Norms of the vectors of a chunk (general shapes), needed before the first
// GEMM because they fix each vector's fp16 scale: one wave per vector,
// float32 partial sums per lane combined across the wave.
template <bool XBF16>
__global__ __launch_bounds__(256) void vec_norm_kernel(const void *__restrict__ x, int64_t n, int d,
                                                       float *__restrict__ knorm) {
  const int lane = threadIdx.x & 63;
  const int64_t v = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (v >= n) return;  // wave-uniform
  float ss = 0.f;
  if (XBF16) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const uint4 *p = reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(x) + v * d);
    for (int i = lane; i < d / 8; i += 64) {
      const uint4 w = p[i];
      const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const bf16x2 b = __builtin_bit_cast(bf16x2, u[k]);
        ss = __builtin_amdgcn_fdot2_f32_bf16(b, b, ss, false);
      }
    }
  } else {
    const float4 *p = reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(x) + v * d);
    for (int i = lane; i < d / 4; i += 64) {
      const float4 a = p[i];
      ss = fmaf(a.x, a.x, ss);
      ss = fmaf(a.y, a.y, ss);
      ss = fmaf(a.z, a.z, ss);
      ss = fmaf(a.w, a.w, ss);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
  if (lane == 0) knorm[v] = sqrtf(ss);
}

template <int B, bool PROD>
static void launch_gemm1_t(const Derived &D, const void *x, int dtype, int64_t n, tq_codes c,
                           uint4 *rho, float *rsq, int64_t stride, hipStream_t s) {
  const int64_t grid = (n + kGVec - 1) / kGVec * (D.p.d / 128);
  const unsigned ngrid = (unsigned)((n + 3) / 4);
  if (dtype == TQ_BF16) {
    vec_norm_kernel<true><<<dim3(ngrid), dim3(256), 0, s>>>(x, n, D.p.d, c.knorm);
    encode_gemm1_kernel<B, PROD, true><<<dim3((unsigned)grid), dim3(kGW * 64), 0, s>>>(
        x, n, D.p.d, D.pi_frag, D.cb, c.idx, c.knorm, rho, rsq, stride);
  } else {
    vec_norm_kernel<false><<<dim3(ngrid), dim3(256), 0, s>>>(x, n, D.p.d, c.knorm);
    encode_gemm1_kernel<B, PROD, false><<<dim3((unsigned)grid), dim3(kGW * 64), 0, s>>>(
        x, n, D.p.d, D.pi_frag, D.cb, c.idx, c.knorm, rho, rsq, stride);
  }
}

static tq_status launch_encode_general(const Derived &D, const void *x, int dtype, int64_t n,
                                       tq_codes c, void *ws, hipStream_t s) {
  const bool prod = D.p.mode == TQ_MODE_PROD;
  const int d = D.p.d, m = D.p.m, B = D.B;
  const size_t esz = dtype == TQ_BF16 ? 2 : 4;
  // mse mode needs no workspace: one launch over all vectors
  const int64_t chunk = prod ? std::min<int64_t>((n + kGVec - 1) / kGVec * kGVec, kGenChunk) : n;
  uint4 *rho = (uint4 *)ws;
  float *rsq = prod ? (float *)((char *)ws + (size_t)chunk * 4 * d) : nullptr;
  for (int64_t c0 = 0; c0 < n; c0 += chunk) {
    const int64_t nc = std::min<int64_t>(chunk, n - c0);
    const void *xc = (const char *)x + (size_t)c0 * d * esz;
    tq_codes cc;
    cc.idx = B > 0 ? c.idx + (size_t)c0 * (d / 32) * B : nullptr;
    cc.sgn = prod ? c.sgn + (size_t)c0 * (m / 32) : nullptr;
    cc.knorm = c.knorm + c0;
    cc.rnorm = prod ? c.rnorm + c0 : nullptr;
    switch (B * 2 + (prod ? 1 : 0)) {
      case 0 * 2 + 1: launch_gemm1_t<0, true>(D, xc, dtype, nc, cc, rho, rsq, chunk, s); break;
      case 1 * 2 + 1: launch_gemm1_t<1, true>(D, xc, dtype, nc, cc, rho, rsq, chunk, s); break;
      case 2 * 2 + 1: launch_gemm1_t<2, true>(D, xc, dtype, nc, cc, rho, rsq, chunk, s); break;
      case 3 * 2 + 1: launch_gemm1_t<3, true>(D, xc, dtype, nc, cc, rho, rsq, chunk, s); break;
      case 4 * 2 + 1: launch_gemm1_t<4, true>(D, xc, dtype, nc, cc, rho, rsq, chunk, s); break;
      case 1 * 2 + 0: launch_gemm1_t<1, false>(D, xc, dtype, nc, cc, rho, rsq, chunk, s); break;
      case 2 * 2 + 0: launch_gemm1_t<2, false>(D, xc, dtype, nc, cc, rho, rsq, chunk, s); break;
      case 3 * 2 + 0: launch_gemm1_t<3, false>(D, xc, dtype, nc, cc, rho, rsq, chunk, s); break;
      case 4 * 2 + 0: launch_gemm1_t<4, false>(D, xc, dtype, nc, cc, rho, rsq, chunk, s); break;
      default:
        set_error("tq_encode: unsupported B = %d", B);
        return TQ_ERR_UNSUPPORTED;
    }
    TQ_LAUNCH_CHECK();
    if (prod) {
      const int64_t grid = (nc + kGVec - 1) / kGVec * (m / 128);
      encode_gemm2_kernel<<<dim3((unsigned)grid), dim3(kGW * 64), 0, s>>>(
          rho, rsq, nc, chunk, d, m, D.sp_frag, cc.knorm, cc.sgn, cc.rnorm);
      TQ_LAUNCH_CHECK();
    }
  }
  return TQ_OK;
}

tq_status launch_encode(const Derived &D, const void *x, int dtype, int64_t n, tq_codes c,
                        void *ws, size_t ws_bytes, hipStream_t s, const int64_t *slots,
                        int64_t capacity) {
  if (is_d128(D.p)) return launch_encode128(D, x, dtype, n, c, s, slots, capacity);
  if (slots != nullptr) {
    set_error("tq_encode_slots: built for d = m = 128");
    return TQ_ERR_UNSUPPORTED;
  }
  if (ws_bytes < encode_workspace_bytes(D.p, n)) {
    set_error("tq_encode: workspace too small");
    return TQ_ERR_NO_MEMORY;
  }
  if (D.p.mode == TQ_MODE_MSE &&
      ((n + kGVec - 1) / kGVec * (D.p.d / 128) > 0x7fffffffLL || (n + 3) / 4 > 0x7fffffffLL)) {
    set_error("tq_encode: too many vectors for one launch");
    return TQ_ERR_UNSUPPORTED;
  }
  return launch_encode_general(D, x, dtype, n, c, ws, s);
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

struct QConst {  // per query, float64 so that logits keep ~1e-8 relative accuracy
  double idx_scale;  // 2^-E of the index part
  double idx_bias;   // sum_S coef_S * sum_c qt_c
  double sgn_scale;  // sqrt(pi/2)/m * 2^-E'
  double sgn_bias;   // sqrt(pi/2)/m * sum_r qs_r
  float f[4];        // the same four in float32, for the plain-score epilogue
};

// The 8 bit slices of a packed word as int8 MFMA operands: slice s keeps bit s
// of every byte.  The upper four slices come from the word shifted by 4, so a
// set bit weighs 2^(s & 3) (1, 2, 4 or 8): one shift and eight ANDs per word.
// The query side carries the factor 2^-(s & 3) and so loses at most three of
// its 26 bits to the weight.
__device__ __forceinline__ void bit_slices(uint32_t w, i32x4 &lo4, i32x4 &hi4) {
  const uint32_t w4 = w >> 4;
  lo4 = i32x4{(int)(w & 0x01010101u), (int)(w & 0x02020202u), (int)(w & 0x04040404u),
              (int)(w & 0x08080808u)};
  hi4 = i32x4{(int)(w4 & 0x01010101u), (int)(w4 & 0x02020202u), (int)(w4 & 0x04040404u),
              (int)(w4 & 0x08080808u)};
}

// Integer sums of one 16-key tile: lane (kc, kg) of a wave, planes = the
// key's index words of lane group kg, sw = its sign word.  Output rows
// 4 kg + t of column kc are limb t of query kg: ai for the index part, as for
// the sign part.
template <int B, bool PROD, int NP>
__device__ __forceinline__ void tile_sums(const i32x4 *A, const uint32_t *planes, uint32_t sw,
                                          i32x4 &ai, i32x4 &as) {
  ai = i32x4{0, 0, 0, 0};
  as = i32x4{0, 0, 0, 0};
#pragma unroll
  for (int sp = 0; sp < NP; ++sp) {
    uint32_t part = 0;
#pragma unroll
    for (int p = 0; p < B; ++p)
      if (part_mask_ct(B, sp) >> p & 1) part ^= planes[p];
    i32x4 lo4, hi4;
    bit_slices(part, lo4, hi4);
    ai = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[2 * sp], lo4, ai, 0, 0, 0);
    ai = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[2 * sp + 1], hi4, ai, 0, 0, 0);
  }
  if (PROD) {
    i32x4 lo4, hi4;
    bit_slices(sw, lo4, hi4);
    as = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[2 * NP], lo4, as, 0, 0, 0);
    as = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[2 * NP + 1], hi4, as, 0, 0, 0);
  }
}

// Logit of (query kg, key kc) for one 16-key tile, in float32.  Each
// accumulated limb is below 2^19 in magnitude, so limbs 0 + 128 * 1 and
// 2 + 128 * 3 pair up exactly in int32; the two conversions, the final fma and
// the bias subtraction carry a few 2^-24 of the index part's magnitude, which
// exceeds the logit's own size by a factor of order sqrt(d), so the logit's
// relative error stays near 1e-6, far under a 1e-4 bar (attention: the
// softmax weights inherit it as a relative error of |logit| * 1e-6).
template <int B, bool PROD, int NP>
__device__ __forceinline__ float tile_logit_f32(const i32x4 *A, const uint32_t *planes, uint32_t sw,
                                                float kn, float rn, float si, float bi, float ss,
                                                float bs) {
  i32x4 ai, as;
  tile_sums<B, PROD, NP>(A, planes, sw, ai, as);
  float l = 0.f;
  if (NP > 0) {
    const float vi = fmaf((float)(ai[2] + (ai[3] << 7)), 16384.f, (float)(ai[0] + (ai[1] << 7)));
    l = kn * fmaf(vi, si, -bi);
  }
  if (PROD) {
    const float vs = fmaf((float)(as[2] + (as[3] << 7)), 16384.f, (float)(as[0] + (as[1] << 7)));
    l = fmaf(rn, fmaf(vs, ss, -bs), l);
  }
  return l;
}

// Balanced base-128 digit t (t = 0..3) of an integer |Q| < 2^26.
__device__ __forceinline__ int limb_of(int Q, int t) {
  int digit = 0;
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    if (tt > t) break;
    digit = ((Q + 64) & 127) - 64;
    Q = (Q - digit) >> 7;  // exact: Q - digit is a multiple of 128
  }
  return digit;
}

// Query preparation for the d = 128 kernels.  One workgroup of 1024 threads
// takes one query group (4 queries of one KV head); the call is latency-bound
// (a decode step has a few dozen groups), so the work of a group is spread
// over as many threads as it has independent pieces:
//   1. thread (quarter cq, row r) requests columns 32 cq .. 32 cq + 31 of row
//      r of [Pi; S] first (column-major copy: each column is one contiguous
//      kilobyte), then the group's queries land in LDS;
//   2. the thread forms its partial dot products with the 4 queries with
//      float64 accumulation; the four quarters are summed through LDS,
//      giving qt = Pi q and qs = S q rounded once to float32 (~6e-8 of each
//      value, below the operands' 26-bit quantisation step);
//   3. per query (one wave each): ||q||, u . q and v . q (u, v the column
//      sums of Pi and S) in float64; the exponents that put the largest
//      operand below 2^26 (|qt_c| <= ||q||, |qs_r| <= smax ||q||, smax the
//      largest row norm of S: one or two of the 26 bits spent on the bound),
//      and the constants (sum_c qt_c = u . q, sum_r qs_r = v . q);
//   4. the int8 operands of the score MFMAs.  MFMA j (part j / 2, half j % 2;
//      the sign part last) lane l = 16 kg + 4 jq + t holds limb t of query jq
//      at the coordinates of lane group kg; one thread computes the 16 scaled
//      values of (j, jq, kg) once and writes all four limbs.
constexpr int kQPThreads = 1024;

template <bool PROD>
__global__ __launch_bounds__(kQPThreads) void qprep128_kernel(
    const float *__restrict__ q, int64_t g, int ngroups, const float *__restrict__ qmat,
    const float *__restrict__ qsums, float smax, Codebook cb, int m, i32x4 *__restrict__ aops,
    QConst *__restrict__ qc) {
  constexpr int R = PROD ? 256 : 128;  // rows of [Pi; S] in use
  __shared__ float qs[4][128];           // the group's queries (missing ones zero)
  __shared__ double part[4][4][R];       // [quarter][query][row] partial projections
  __shared__ float qv[4][R];             // [query][row]: rows < 128 Pi q, the rest S q
  __shared__ int expo[4][2];
  const int tid = threadIdx.x;
  const int r = tid & 255, cq = tid >> 8;
  const int64_t hg = blockIdx.x;
  const int64_t h = hg / ngroups;
  const int grp = (int)(hg % ngroups);
  // 1. this thread's 32 matrix entries, then the queries
  float mv[32];
  if (r < R) {
#pragma unroll
    for (int k = 0; k < 32; ++k) mv[k] = qmat[(32 * cq + k) * 256 + r];
  }
  if (tid < 512) {
    const int j = tid >> 7, c = tid & 127;
    const int64_t qh = (int64_t)grp * 4 + j;
    qs[j][c] = qh < g ? q[(h * g + qh) * 128 + c] : 0.f;
  }
  __syncthreads();
  // 2. partial projections over this thread's quarter of the columns
  if (r < R) {
    double a[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int k = 0; k < 32; k += 4) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float4 qq = *reinterpret_cast<const float4 *>(&qs[j][32 * cq + k]);
        a[j] = fma((double)mv[k], (double)qq.x, a[j]);
        a[j] = fma((double)mv[k + 1], (double)qq.y, a[j]);
        a[j] = fma((double)mv[k + 2], (double)qq.z, a[j]);
        a[j] = fma((double)mv[k + 3], (double)qq.w, a[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) part[cq][j][r] = a[j];
  }
  // 3. per query j (wave j): norm, column-sum dots, exponents, constants
  if (tid < 256) {
    const int j = tid >> 6, lane = tid & 63;
    float ss = 0.f;
    double du = 0.0, dv = 0.0;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int c = lane + 64 * e;
      const float x = qs[j][c];
      ss = fmaf(x, x, ss);
      du = fma((double)qsums[c], (double)x, du);
      if (PROD) dv = fma((double)qsums[128 + c], (double)x, dv);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      ss += __shfl_xor(ss, off);
      du += __shfl_xor(du, off);
      if (PROD) dv += __shfl_xor(dv, off);
    }
    if (lane == 0) {
      const float qn = sqrtf(ss);
      double acoef = 0, amax = 0;
      for (int sp = 0; sp < cb.nparts; ++sp) {
        acoef += cb.coef[sp];
        amax = fmax(amax, fabs(cb.coef[sp]));
      }
      int e1 = 0, e2 = 0, k;
      const double A1 = 2.0 * amax * (double)qn, A2 = 2.0 * (double)smax * (double)qn;
      if (A1 > 0) { frexp(A1, &k); e1 = 26 - k; }
      if (PROD && A2 > 0) { frexp(A2, &k); e2 = 26 - k; }
      expo[j][0] = e1;
      expo[j][1] = e2;
      const double cqj = PROD ? sqrt(M_PI / 2.0) / m : 0.0;
      QConst o;
      o.idx_scale = ldexp(1.0, -e1);
      o.idx_bias = acoef * du;
      o.sgn_scale = cqj * ldexp(1.0, -e2);
      o.sgn_bias = cqj * dv;
      o.f[0] = (float)o.idx_scale;
      o.f[1] = (float)o.idx_bias;
      o.f[2] = (float)o.sgn_scale;
      o.f[3] = (float)o.sgn_bias;
      qc[hg * 4 + j] = o;
    }
  }
  __syncthreads();
  if (r < R) qv[cq][r] = (float)(((part[0][cq][r] + part[1][cq][r]) + part[2][cq][r]) + part[3][cq][r]);
  __syncthreads();
  // 4. operands: unit (j, jq, kg, w): word w of the four lanes 16 kg + 4 jq + t
  const int NMF = score_mfmas(cb.nparts, PROD);
  const int NP = cb.nparts;
  uint32_t *aw = reinterpret_cast<uint32_t *>(aops);
  for (int i = tid; i < NMF * 64; i += kQPThreads) {
    const int j = i >> 6, jq = (i >> 4) & 3, kg = (i >> 2) & 3, w = i & 3;
    const bool sgnpart = j >= 2 * NP;
    const int sl = 4 * (j & 1) + w;
    const float coef = sgnpart ? 2.f : (float)(2.0 * cb.coef[j >> 1]);
    const int E = expo[jq][sgnpart ? 1 : 0];
    const float *src = &qv[jq][sgnpart ? 128 : 0];
    uint32_t out[4] = {0u, 0u, 0u, 0u};  // limb t
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int cc = 32 * e + 16 * (sl >> 2) + 4 * kg + (sl & 3);
      // |Q| < 2^26, formed in float32: off by at most a few units of the
      // 2^26 scale, a ~1e-7 relative error in the logit
      int Q = (int)rintf(ldexpf(coef * src[cc], E - (sl & 3)));
#pragma unroll
      for (int t = 0; t < 4; ++t) {  // balanced base-128 digits, lowest first
        const int digit = ((Q + 64) & 127) - 64;
        Q = (Q - digit) >> 7;  // exact: Q - digit is a multiple of 128
        out[t] |= (uint32_t)(uint8_t)(int8_t)digit << (8 * e);
      }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) aw[((hg * NMF + j) * 64 + 16 * kg + 4 * jq + t) * 4 + w] = out[t];
  }
}

template <bool PROD>
static void launch_qprep128(const Derived &D, const float *q, int64_t g, int ngroups, int64_t nhg,
                            i32x4 *aops, QConst *qc, hipStream_t s) {
  qprep128_kernel<PROD><<<dim3((unsigned)nhg), dim3(kQPThreads), 0, s>>>(
      q, g, ngroups, D.qmat, D.qsums, D.smax, D.cb, D.p.m, aops, qc);
}

constexpr int kScoreU = 4;  // tiles per load batch (64 keys)
constexpr int kScoreH = 4;  // batches per wave, all requested before any is consumed

// The codes of kScoreU consecutive 16-key tiles as one lane holds them: its
// own index and sign words of every tile, and the norms of key `lane` of the
// batch (spread to the lanes that need them with ds_bpermute).
template <int BB>
struct ScoreBatch {
  uint32_t pl[kScoreU][BB];
  uint32_t sw[kScoreU];
  float kn, rn;
};

// Loads of a batch whose tiles all lie inside the sequence.  The bases are
// wave-uniform (scalar registers) and the lane offsets do not change between
// batches, so no vector address arithmetic is spent per tile.
template <int B, bool PROD>
__device__ __forceinline__ void score_load_full(ScoreBatch<(B > 0 ? B : 1)> &b,
                                                const uint32_t *idx_t, const uint32_t *sgn_t,
                                                const float *kn_t, const float *rn_t,
                                                uint32_t off_idx, uint32_t off_sgn, uint32_t lane) {
  constexpr int BB = B > 0 ? B : 1;
#pragma unroll
  for (int u = 0; u < kScoreU; ++u) {
    const uint32_t *ip = idx_t + (uint32_t)(u * 64 * BB) + off_idx;
    if constexpr (B == 1) {
      b.pl[u][0] = nt_load(ip);
    } else if constexpr (B == 2) {
      const u32x2 t = nt_load2(ip);
      b.pl[u][0] = t.x; b.pl[u][1] = t.y;
    } else if constexpr (B == 3) {
      b.pl[u][0] = nt_load(ip); b.pl[u][1] = nt_load(ip + 1); b.pl[u][2] = nt_load(ip + 2);
    } else if constexpr (B == 4) {
      const u32x4 t = nt_load4(ip);
      b.pl[u][0] = t.x; b.pl[u][1] = t.y; b.pl[u][2] = t.z; b.pl[u][3] = t.w;
    } else {
      b.pl[u][0] = 0u;
    }
    b.sw[u] = PROD ? nt_load(&sgn_t[(uint32_t)(u * 64) + off_sgn]) : 0u;
  }
  b.kn = nt_load(&kn_t[lane]);
  b.rn = PROD ? nt_load(&rn_t[lane]) : 0.f;
}

template <int B, bool PROD, int NP>
__device__ __forceinline__ void score_store_full(const ScoreBatch<(B > 0 ? B : 1)> &b,
                                                 const i32x4 *A, float si, float bi, float ss,
                                                 float bs, float *out_t, bool qvalid, int kc) {
  // One tile at a time (the scheduling barrier keeps the MFMA accumulators
  // of different tiles from being live together), and every logit computed
  // before the store branch so that no load is sunk into it.
  float l[kScoreU];
#pragma unroll
  for (int u = 0; u < kScoreU; ++u) {
    const int src = (16 * u + kc) * 4;  // byte address of lane 16 u + kc
    const float kn = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src, __builtin_bit_cast(int, b.kn)));
    const float rn = PROD ? __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src, __builtin_bit_cast(int, b.rn)))
                          : 0.f;
    l[u] = tile_logit_f32<B, PROD, NP>(A, b.pl[u], b.sw[u], kn, rn, si, bi, ss, bs);
    asm volatile("" ::"v"(l[u]));  // materialise here, not inside the branch below
    __builtin_amdgcn_sched_barrier(0);
  }
  if (qvalid) {
#pragma unroll
    for (int u = 0; u < kScoreU; ++u) nt_store(&out_t[u * 16], l[u]);
  }
}

template <int B, bool PROD>
__global__ __launch_bounds__(kScoreWaves * 64) void score128_kernel(
    const i32x4 *__restrict__ aops, const QConst *__restrict__ qc,
    const uint32_t *__restrict__ idx, const uint32_t *__restrict__ sgn,
    const float *__restrict__ knorm, const float *__restrict__ rnorm, int64_t seq, int64_t g,
    int ngroups, Codebook cb, float *__restrict__ logits) {
  constexpr int NP = B == 0 ? 0 : (B == 1 ? 1 : B == 2 ? 2 : B == 3 ? 4 : 8);
  constexpr int NMF = score_mfmas(NP, PROD);
  constexpr int BB = B > 0 ? B : 1;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hg = blockIdx.y;
  const int h = hg / ngroups, grp = hg % ngroups;
  const int kc = lane & 15, kg = lane >> 4;
  i32x4 A[NMF];
#pragma unroll
  for (int j = 0; j < NMF; ++j) A[j] = aops[((int64_t)hg * NMF + j) * 64 + lane];
  // float32 constants: no conversion, so nothing waits for these loads
  // before the first codes are requested
  const float4 cf = *reinterpret_cast<const float4 *>(qc[(int64_t)hg * 4 + kg].f);
  const float si = cf.x, bi = cf.y, ss = cf.z, bs = cf.w;
  const int64_t qh = (int64_t)grp * 4 + kg;  // this lane's output query within the head
  const bool qvalid = qh < g;
  float *out = logits + ((int64_t)h * g + (qvalid ? qh : 0)) * seq;
  const uint32_t *idx_h = idx + (int64_t)h * seq * 4 * BB;
  const uint32_t *sgn_h = sgn + (int64_t)h * seq * 4;
  const float *kn_h = knorm + (int64_t)h * seq;
  const float *rn_h = rnorm + (int64_t)h * seq;

  // Work of a wave: kScoreH consecutive batches of kScoreU tiles, whose loads
  // are all issued at once before the first is consumed (the codes are read
  // once; many short-lived waves on neighbouring tiles stream HBM best).
  // Batches past the last whole one load a clamped, in-bounds copy and are
  // not stored.  Tile indices within one head fit in 32 bits (seq < 2^35);
  // all of this is wave-uniform.
  const int tiles = (int)((seq + 15) / 16);
  const int nbf = (int)(seq / 16) / kScoreU;  // batches whose tiles are all full
  const int nw = (int)gridDim.x * kScoreWaves;
  const int j = (int)blockIdx.x * kScoreWaves + wave;
  const int bc = j * kScoreH;
  if (bc < nbf) {
    const uint32_t off_idx = (uint32_t)((kc * 4 + kg) * BB), off_sgn = (uint32_t)(kc * 4 + kg);
    ScoreBatch<BB> bt[kScoreH];
#pragma unroll
    for (int u = 0; u < kScoreH; ++u) {
      const int64_t t_ = (int64_t)(bc + u < nbf ? bc + u : nbf - 1) * kScoreU;
      score_load_full<B, PROD>(bt[u], idx_h + t_ * 64 * BB, sgn_h + t_ * 64, kn_h + t_ * 16,
                               rn_h + t_ * 16, off_idx, off_sgn, (uint32_t)lane);
    }
#pragma unroll
    for (int u = 0; u < kScoreH; ++u)
      if (bc + u < nbf)
        score_store_full<B, PROD, NP>(bt[u], A, si, bi, ss, bs,
                                      out + (int64_t)(bc + u) * (16 * kScoreU) + kc, qvalid, kc);
  }
  // The rest (fewer than a batch of tiles, the last one possibly partial),
  // taken by the last wave: positions are clamped into the sequence so every
  // load is in bounds; results of out-of-range positions are not stored.
  if (j != nw - 1) return;
  for (int tb = nbf * kScoreU; tb < tiles; tb += kScoreU) {
    uint32_t pl[kScoreU][BB], sw[kScoreU];
    float kn[kScoreU], rn[kScoreU];
#pragma unroll
    for (int u = 0; u < kScoreU; ++u) {
      const int64_t pos = (int64_t)(tb + u) * 16 + kc;
      const int64_t vp = pos < seq ? pos : seq - 1;
      const uint32_t *ip = idx_h + (vp * 4 + kg) * BB;
#pragma unroll
      for (int p = 0; p < BB; ++p) pl[u][p] = B > 0 ? ip[p] : 0u;
      sw[u] = PROD ? sgn_h[vp * 4 + kg] : 0u;
      kn[u] = kn_h[vp];
      rn[u] = PROD ? rn_h[vp] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kScoreU; ++u) {
      const float l = tile_logit_f32<B, PROD, NP>(A, pl[u], sw[u], kn[u], rn[u], si, bi, ss, bs);
      const int64_t pos = (int64_t)(tb + u) * 16 + kc;
      if (pos < seq && qvalid) out[pos] = l;
    }
  }
}

static int nparts_of(int B) { return B == 0 ? 0 : (B == 1 ? 1 : B == 2 ? 2 : B == 3 ? 4 : 8); }

static size_t score128_workspace_bytes(int B, bool prod, int64_t n_kv, int64_t g) {
  const int64_t ngroups = (g + 3) / 4;
  const int NMF = score_mfmas(nparts_of(B), prod);
  return (size_t)n_kv * ngroups * ((size_t)NMF * 64 * sizeof(i32x4) + 4 * sizeof(QConst));
}

template <int B, bool PROD>
static void launch_score_t(const Derived &D, const float *q, int64_t n_kv, int64_t g,
                           tq_codes c, int64_t seq, float *logits, void *ws, hipStream_t s) {
  const int ngroups = (int)((g + 3) / 4);
  const int NMF = score_mfmas(nparts_of(B), PROD);
  const int64_t nhg = n_kv * ngroups;
  i32x4 *aops = (i32x4 *)ws;
  QConst *qc = (QConst *)((char *)ws + (size_t)nhg * NMF * 64 * sizeof(i32x4));
  launch_qprep128<PROD>(D, q, g, ngroups, nhg, aops, qc, s);
  // Workgroups per (KV head, query group): enough waves for every batch.
  const int64_t nb = (seq + 16 * kScoreU - 1) / (16 * kScoreU);
  const int64_t chunks = std::max<int64_t>(1, (nb + kScoreH * kScoreWaves - 1) / (kScoreH * kScoreWaves));
  score128_kernel<B, PROD><<<dim3((unsigned)chunks, (unsigned)(n_kv * ngroups)),
                             dim3(kScoreWaves * 64), 0, s>>>(aops, qc, c.idx, c.sgn, c.knorm,
                                                             c.rnorm, seq, g, ngroups, D.cb, logits);
}

static tq_status launch_score128(const Derived &D, const float *q, int64_t n_kv, int64_t g,
                                 tq_codes c, int64_t seq, float *logits, void *ws, hipStream_t s) {
  if ((uint64_t)n_kv * ((g + 3) / 4) > 65535u) {
    set_error("tq_score: n_kv * ceil(g/4) = %lld exceeds 65535", (long long)(n_kv * ((g + 3) / 4)));
    return TQ_ERR_UNSUPPORTED;
  }
  if (seq >= (int64_t(1) << 34)) {  // tile indices within a head are 32-bit
    set_error("tq_score: seq = %lld exceeds 2^34", (long long)seq);
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
// Score and search, many queries and general shapes (d, m multiples of 128)
// ===========================================================================
// The same integer formulation as the d = 128 kernel, tiled for reuse: a
// workgroup scores blocks of kSMCodes codes against 4 QB queries (QB groups
// of 4).  The K dimension is walked in chunks of 128 coordinates; in chunk q,
// lane group kg of a code holds word 4 q + kg of each index plane and of the
// sign bits (the packed layout's own order, so the four lanes of a code read
// one contiguous run per chunk).  The query operands of one chunk (all parts,
// all QB groups) are staged in LDS, double buffered; every bit slice a wave
// builds from its codes feeds QB query groups.
//
// Search (top-k per query) runs the same kernel persistently over a segment
// of code blocks and keeps a running top-k list per query in LDS: a block's
// logits are merged into the list only for queries where some logit beats the
// list's current k-th entry, which after the first blocks is rare.  A small
// kernel merges the per-segment lists.
constexpr int kSMWaves = 8;
constexpr int kSMCT = 4;                          // 16-code tiles per wave
constexpr int kSMCodes = kSMWaves * kSMCT * 16;  // codes per block (512)
constexpr int kSMGroup = 4;                       // query blocks per L2 window
constexpr int kMaxChunks = 8;                     // 1024 / 128
constexpr int kQJR = 64, kQJQ = 16, kQJK = 64;    // projection tile: rows x queries x K

__host__ __device__ constexpr int nparts_ct(int B) {
  return B == 0 ? 0 : (B == 1 ? 1 : B == 2 ? 2 : B == 3 ? 4 : 8);
}
__host__ __device__ constexpr int sm_nj(int B, bool prod) { return 2 * nparts_ct(B) + (prod ? 2 : 0); }
// query groups per workgroup: as many as keep the LDS stages (QB NJ KB each,
// double buffered) and the registers (8 accumulators per group and code tile,
// plus the code words) within budget
// (K is the capacity of the search lists kept in LDS, 0 for plain scoring.)
__host__ __device__ constexpr int sm_qb(int B, bool prod, int K) {
  return sm_nj(B, prod) <= 10 ? 4 : 2;
}
__host__ __device__ constexpr int list_cap(int k) { return k <= 0 ? 0 : (k <= 8 ? 8 : (k <= 16 ? 16 : 32)); }

// Projections of every query, float64 sums: out[i][r] = sum_j M[r][j] q_i[j]
// with M = [Pi; S] (rows = d + m in prod mode, d in mse mode).  A workgroup
// computes a 64-row x 16-query tile; both operands pass through LDS in
// 64-wide K tiles.
__global__ __launch_bounds__(256) void qproj_kernel(const float *__restrict__ q, int64_t nq, int d,
                                                    int rows, const float *__restrict__ pi,
                                                    const float *__restrict__ s,
                                                    double *__restrict__ out) {
  __shared__ float Ms[kQJR][kQJK + 1];
  __shared__ double Qs[kQJQ][kQJK];
  const int tid = threadIdx.x;
  const int r0 = blockIdx.x * kQJR;
  const int64_t q0 = (int64_t)blockIdx.y * kQJQ;
  const int r = tid & 63, jq0 = (tid >> 6) * 4;
  double acc[4] = {0.0, 0.0, 0.0, 0.0};
  for (int j0 = 0; j0 < d; j0 += kQJK) {
    for (int i = tid; i < kQJR * kQJK / 4; i += 256) {
      const int rr = i >> 4, c4 = i & 15;
      const int gr = r0 + rr;
      const float *row = gr < d ? pi + (size_t)gr * d : s + (size_t)(gr - d) * d;
      const float4 v = reinterpret_cast<const float4 *>(row + j0)[c4];
      Ms[rr][4 * c4 + 0] = v.x;
      Ms[rr][4 * c4 + 1] = v.y;
      Ms[rr][4 * c4 + 2] = v.z;
      Ms[rr][4 * c4 + 3] = v.w;
    }
    for (int i = tid; i < kQJQ * kQJK; i += 256) {
      const int jq = i >> 6, c = i & 63;
      const int64_t qi = q0 + jq;
      Qs[jq][c] = qi < nq ? (double)q[qi * d + j0 + c] : 0.0;
    }
    __syncthreads();
#pragma unroll 8
    for (int j = 0; j < kQJK; ++j) {
      const double w = (double)Ms[r][j];
#pragma unroll
      for (int k = 0; k < 4; ++k) acc[k] = fma(w, Qs[jq0 + k][j], acc[k]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int64_t qi = q0 + jq0 + k;
    if (qi < nq) out[qi * rows + r0 + r] = acc[k];
  }
}

// Integer operands of every chunk for one group of 4 queries (layout
// [head][query block][chunk][group][operand j][lane]) and the per-query
// constants.  Operand j < 2 NP is part j / 2, half j % 2; the last two are
// the sign part.  Lane l (row 4 jq + t: query jq, limb t; lane group kg),
// dword w, byte e multiplies bit 8 e + sl (sl = 4 (j % 2) + w) of word
// W = 4 q + kg, i.e. coordinate 128 q + 32 e + 16 (sl / 4) + 4 kg + sl % 4.
template <bool PROD>
__global__ __launch_bounds__(256) void qops_kernel(const double *__restrict__ qproj, int64_t g,
                                                   int nqb, int QB, int d, int m, Codebook cb,
                                                   i32x4 *__restrict__ aops,
                                                   QConst *__restrict__ qc) {
  __shared__ double qv[2][4][1024];  // [0] = Pi q, [1] = S q
  __shared__ int expo[4][2];
  const int64_t gid = blockIdx.x;
  const int qb = (int)(gid % QB);
  const int64_t hq = gid / QB;  // head * nqb + query block
  const int64_t head = hq / nqb;
  const int qblk = (int)(hq % nqb);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int Qd = d >> 7, Md = PROD ? m >> 7 : 0, NCH = Qd > Md ? Qd : Md;
  const int NP = cb.nparts, NJ = 2 * NP + (PROD ? 2 : 0);
  const int rows = d + (PROD ? m : 0);
  for (int i = tid; i < 4 * rows; i += 256) {
    const int jq = i / rows, c = i - jq * rows;
    const int64_t qi = ((int64_t)qblk * QB + qb) * 4 + jq;
    const double v = qi < g ? qproj[(head * g + qi) * rows + c] : 0.0;
    if (c < d)
      qv[0][jq][c] = v;
    else
      qv[1][jq][c - d] = v;
  }
  __syncthreads();
  {
    // wave jq: max |qt|, max |qs|, sum qt, sum qs of query jq
    const int jq = wave;
    double mq = 0.0, ms = 0.0, sq = 0.0, ss = 0.0;
    for (int c = lane; c < d; c += 64) {
      mq = fmax(mq, fabs(qv[0][jq][c]));
      sq += qv[0][jq][c];
    }
    if (PROD)
      for (int c = lane; c < m; c += 64) {
        ms = fmax(ms, fabs(qv[1][jq][c]));
        ss += qv[1][jq][c];
      }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      mq = fmax(mq, __shfl_xor(mq, off));
      ms = fmax(ms, __shfl_xor(ms, off));
      sq += __shfl_xor(sq, off);
      ss += __shfl_xor(ss, off);
    }
    if (lane == 0) {
      double acoef = 0, amax = 0;
      for (int p = 0; p < NP; ++p) {
        acoef += cb.coef[p];
        amax = fmax(amax, fabs(cb.coef[p]));
      }
      // scale the largest operand magnitude below 2^26
      int e1 = 0, e2 = 0, k;
      const double A1 = 2.0 * amax * mq, A2 = 2.0 * ms;
      if (A1 > 0) { frexp(A1, &k); e1 = 26 - k; }
      if (A2 > 0) { frexp(A2, &k); e2 = 26 - k; }
      expo[jq][0] = e1;
      expo[jq][1] = e2;
      const double cq = PROD ? sqrt(M_PI / 2.0) / m : 0.0;
      QConst o;
      o.idx_scale = ldexp(1.0, -e1);
      o.idx_bias = acoef * sq;
      o.sgn_scale = cq * ldexp(1.0, -e2);
      o.sgn_bias = cq * ss;
      o.f[0] = (float)o.idx_scale;
      o.f[1] = (float)o.idx_bias;
      o.f[2] = (float)o.sgn_scale;
      o.f[3] = (float)o.sgn_bias;
      qc[hq * 4 * QB + qb * 4 + jq] = o;
    }
  }
  __syncthreads();
  for (int i = tid; i < NCH * NJ * 64; i += 256) {
    const int l = i & 63, jl = i >> 6;
    const int j = jl % NJ, qq = jl / NJ;
    const int row = l & 15, kg = l >> 4, jq = row >> 2, t = row & 3;
    const bool sgnpart = j >= 2 * NP;
    const int h2 = j & 1;
    const int nchunk = sgnpart ? Md : Qd;
    int out[4] = {0, 0, 0, 0};
    if (qq < nchunk) {
      const double coef = sgnpart ? 2.0 : 2.0 * cb.coef[j >> 1];
      const int E = expo[jq][sgnpart ? 1 : 0];
      const double *src = qv[sgnpart ? 1 : 0][jq];
      const int W = 4 * qq + kg, qp = W >> 2, kp = W & 3;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        uint32_t packed = 0;
        const int sl = 4 * h2 + w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int c = 128 * qp + 32 * e + 16 * (sl >> 2) + 4 * kp + (sl & 3);
          const int Q = (int)llrint(ldexp(coef * src[c], E - (sl & 3)));
          packed |= (uint32_t)(uint8_t)(int8_t)limb_of(Q, t) << (8 * e);
        }
        out[w] = (int)packed;
      }
    }
    aops[(((size_t)hq * NCH + qq) * QB + qb) * NJ * 64 + (size_t)j * 64 + l] =
        i32x4{out[0], out[1], out[2], out[3]};
  }
}

// Load n dwords (n <= N, n a runtime count) that start at a multiple of n
// dwords: vector loads when n is a multiple of 4, dword loads otherwise.
template <int N>
__device__ __forceinline__ void load_run(const uint32_t *__restrict__ p, int n, uint32_t (&r)[N]) {
  if ((n & 3) == 0) {
#pragma unroll
    for (int j = 0; j < N / 4; ++j)
      if (4 * j < n) {
        const u32x4 u = reinterpret_cast<const u32x4 *>(p)[j];
        r[4 * j] = u[0]; r[4 * j + 1] = u[1]; r[4 * j + 2] = u[2]; r[4 * j + 3] = u[3];
      }
  } else {
#pragma unroll
    for (int j = 0; j < N; ++j)
      if (j < n) r[j] = p[j];
  }
}

__device__ __forceinline__ bool better_vi(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

// max-update of a float in LDS (compare-and-swap on its bits)
__device__ __forceinline__ void lds_fmax(float *addr, float v) {
  int *ia = reinterpret_cast<int *>(addr);
  int old = *reinterpret_cast<volatile int *>(ia);
  while (__int_as_float(old) < v) {
    const int assumed = old;
    old = atomicCAS(ia, assumed, __float_as_int(v));
    if (old == assumed) break;
  }
}

// Running top-k lists (search), one per (wave, query), in LDS: descending,
// ties by lower index.  Insert (cv, ci) into the list of lane group kg
// (entries r and r + 16 sit with lane r of the group) when `has`
// (group-uniform); the last entry drops out.
template <int K>
__device__ __forceinline__ void group_insert(float *lv, int *li, int lane, int kg, int k, bool has,
                                             float cv, int ci) {
  constexpr int KR = K > 16 ? 2 : 1;
  const int r = lane & 15;
  float v[KR];
  int ix[KR];
#pragma unroll
  for (int j = 0; j < KR; ++j) {
    const int e = r + 16 * j;
    v[j] = e < k ? lv[e] : -INFINITY;
    ix[j] = e < k ? li[e] : 0x7fffffff;
  }
  int pos = 0;
#pragma unroll
  for (int j = 0; j < KR; ++j) {
    const bool bt = r + 16 * j < k && better_vi(v[j], ix[j], cv, ci);
    pos += __popc((uint32_t)(__ballot(bt) >> (16 * kg)) & 0xFFFFu);
  }
  // the entry before each slot
  float up[KR];
  int upi[KR];
  up[0] = __shfl(v[0], (lane + 63) & 63);
  upi[0] = __shfl(ix[0], (lane + 63) & 63);
  if (KR > 1) {
    const float a15 = __shfl(v[0], 16 * kg + 15);
    const int ai15 = __shfl(ix[0], 16 * kg + 15);
    const float b_ = __shfl(v[KR - 1], (lane + 63) & 63);
    const int bi_ = __shfl(ix[KR - 1], (lane + 63) & 63);
    up[KR - 1] = r == 0 ? a15 : b_;
    upi[KR - 1] = r == 0 ? ai15 : bi_;
  }
  if (has && pos < k) {
#pragma unroll
    for (int j = 0; j < KR; ++j) {
      const int e = r + 16 * j;
      if (e < k && e >= pos) {
        lv[e] = e == pos ? cv : up[j];
        li[e] = e == pos ? ci : upi[j];
      }
    }
  }
}

template <int B, bool PROD, bool TOPK, int K>
__global__ __launch_bounds__(kSMWaves * 64) void score_many_kernel(
    const i32x4 *__restrict__ aops, const QConst *__restrict__ qc,
    const uint32_t *__restrict__ idx, const uint32_t *__restrict__ sgn,
    const float *__restrict__ knorm, const float *__restrict__ rnorm, int64_t seq, int64_t g,
    int nqb, int nseg, int cps, int Qd, int Md, int k, float *__restrict__ logits,
    float *__restrict__ cand_v, int *__restrict__ cand_i) {
  constexpr int NP = nparts_ct(B);
  constexpr int NJ = sm_nj(B, PROD);
  constexpr int QB = sm_qb(B, PROD, TOPK ? K : 0);
  constexpr int NQ = 4 * QB;
  constexpr int BB = B > 0 ? B : 1;
  constexpr int kStage = QB * NJ * 64;               // i32x4 per chunk
  constexpr int kThreads = kSMWaves * 64;
  constexpr int kPer = (kStage + kThreads - 1) / kThreads;
  __shared__ i32x4 As[2][kStage];
  __shared__ QConst qcs[NQ];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kc = lane & 15, kg = lane >> 4;
  const int64_t head = blockIdx.y;
  // tile -> (query block, segment): XCD-contiguous ranges, then windows of
  // kSMGroup query blocks walked query block fastest, so a window of tiles
  // shares both its codes and its query operands in L2
  const int64_t T = (int64_t)nqb * nseg;
  const int64_t bid = blockIdx.x;
  const int64_t t = (T % 8 == 0) ? (bid % 8) * (T / 8) + bid / 8 : bid;
  const int64_t grp = t / ((int64_t)kSMGroup * nseg);
  const int64_t first = grp * kSMGroup;
  const int64_t gsz = (nqb - first) < kSMGroup ? (nqb - first) : kSMGroup;
  const int64_t within = t - grp * kSMGroup * nseg;
  const int qblk = (int)(first + within % gsz);
  const int64_t seg = within / gsz;
  const int NCH = Qd > Md ? Qd : Md;
  const i32x4 *ablk = aops + (size_t)(head * nqb + qblk) * NCH * kStage;
  const QConst *qch = qc + (size_t)(head * nqb + qblk) * NQ;
  const int D32 = 4 * Qd, M32 = 4 * Md;
  const uint32_t *idx_h = idx + (size_t)head * seq * D32 * BB;
  const uint32_t *sgn_h = PROD ? sgn + (size_t)head * seq * M32 : nullptr;
  const float *kn_h = knorm + head * seq;
  const float *rn_h = PROD ? rnorm + head * seq : nullptr;
  const int64_t ncb = (seq + kSMCodes - 1) / kSMCodes;
  const int64_t cb0 = seg * cps;
  const int64_t cb1 = (cb0 + cps) < ncb ? (cb0 + cps) : ncb;
  const int64_t nsteps = (cb1 > cb0 ? cb1 - cb0 : 0) * NCH;

  // search: this wave's running top-k list of each of the NQ queries
  // and, per query, the largest k-th entry over the waves: no code below it
  // can reach the workgroup's top k, so it is not even a candidate
  __shared__ float tlv[TOPK ? kSMWaves : 1][TOPK ? NQ : 1][TOPK ? K : 1];
  __shared__ int tli[TOPK ? kSMWaves : 1][TOPK ? NQ : 1][TOPK ? K : 1];
  __shared__ float tau_sh[TOPK ? NQ : 1];
  if constexpr (TOPK) {
    for (int i = lane; i < NQ * K; i += 64) {
      tlv[wave][i / K][i % K] = -INFINITY;
      tli[wave][i / K][i % K] = 0x7fffffff;
    }
    for (int i = tid; i < NQ; i += kThreads) tau_sh[i] = -INFINITY;
  }

  // One step = one 128-coordinate chunk q of one code block.  Lane group kg of
  // a code holds word 4 q + kg of each index plane and of the sign bits.  The
  // words and the query operands of the next step are fetched while this
  // step's MFMAs run; the operand stages alternate between two LDS buffers
  // across block boundaries.
  uint32_t wcur[kSMCT][BB], scur[kSMCT], wnx[kSMCT][BB], snx[kSMCT];
  auto code_of = [&](int64_t cbk, int ct) -> int64_t {
    const int64_t v = cbk * kSMCodes + wave * (16 * kSMCT) + 16 * ct + kc;
    return v < seq ? v : seq - 1;
  };
#define TQ_LOAD_WORDS(CBK, Q, W, S)                                                      \
  do {                                                                                   \
    _Pragma("unroll") for (int ct_ = 0; ct_ < kSMCT; ++ct_) {                            \
      const int64_t v_ = code_of((CBK), ct_);                                            \
      if (B > 0 && (Q) < Qd) {                                                           \
        const uint32_t *ip_ = idx_h + ((size_t)v_ * D32 + 4 * (Q) + kg) * BB;            \
        if constexpr (BB == 2) {                                                         \
          const uint2 u_ = *reinterpret_cast<const uint2 *>(ip_);                        \
          W[ct_][0] = u_.x;                                                              \
          W[ct_][BB - 1] = u_.y;                                                         \
        } else if constexpr (BB == 4) {                                                  \
          const u32x4 u_ = *reinterpret_cast<const u32x4 *>(ip_);                        \
          _Pragma("unroll") for (int p_ = 0; p_ < BB; ++p_) W[ct_][p_] = u_[p_ & 3];     \
        } else {                                                                         \
          _Pragma("unroll") for (int p_ = 0; p_ < BB; ++p_) W[ct_][p_] = ip_[p_];        \
        }                                                                                \
      }                                                                                  \
      if (PROD && (Q) < Md) S[ct_] = sgn_h[(size_t)v_ * M32 + 4 * (Q) + kg];             \
    }                                                                                    \
  } while (0)

  i32x4 ar[kPer];
  for (int i = tid; i < NQ; i += kThreads) qcs[i] = qch[i];
  if (nsteps > 0) {
    TQ_LOAD_WORDS(cb0, 0, wcur, scur);
#pragma unroll
    for (int j = 0; j < kPer; ++j)
      if (tid + j * kThreads < kStage) As[0][tid + j * kThreads] = ablk[tid + j * kThreads];
  }
  __syncthreads();

  i32x4 acc_i[kSMCT][QB], acc_s[kSMCT][QB];
#pragma unroll
  for (int ct = 0; ct < kSMCT; ++ct)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      acc_i[ct][qb] = i32x4{0, 0, 0, 0};
      acc_s[ct][qb] = i32x4{0, 0, 0, 0};
    }
  float kn[kSMCT], rn[kSMCT];

  int q = 0;
  int64_t cbk = cb0;
#pragma unroll 1
  for (int64_t st = 0; st < nsteps; ++st) {
    const int cur = (int)(st & 1);
    const bool more = st + 1 < nsteps;
    const bool last = q == NCH - 1;
    if (more) {
      const int qn = last ? 0 : q + 1;
      const int64_t cbn = last ? cbk + 1 : cbk;
#pragma unroll
      for (int j = 0; j < kPer; ++j)
        if (tid + j * kThreads < kStage) ar[j] = ablk[(size_t)qn * kStage + tid + j * kThreads];
      TQ_LOAD_WORDS(cbn, qn, wnx, snx);
    }
    if (last) {
#pragma unroll
      for (int ct = 0; ct < kSMCT; ++ct) {
        const int64_t v = code_of(cbk, ct);
        kn[ct] = kn_h[v];
        rn[ct] = PROD ? rn_h[v] : 0.f;
      }
    }
    if (NP > 0 && q < Qd) {
#pragma unroll
      for (int sp = 0; sp < NP; ++sp) {
        i32x4 lo4[kSMCT], hi4[kSMCT];
#pragma unroll
        for (int ct = 0; ct < kSMCT; ++ct) {
          uint32_t part = 0;
#pragma unroll
          for (int p = 0; p < BB; ++p)
            if (part_mask_ct(B, sp) >> p & 1) part ^= wcur[ct][p];
          bit_slices(part, lo4[ct], hi4[ct]);
        }
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const i32x4 a0 = As[cur][(qb * NJ + 2 * sp) * 64 + lane];
          const i32x4 a1 = As[cur][(qb * NJ + 2 * sp + 1) * 64 + lane];
#pragma unroll
          for (int ct = 0; ct < kSMCT; ++ct) {
            acc_i[ct][qb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, lo4[ct], acc_i[ct][qb], 0, 0, 0);
            acc_i[ct][qb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, hi4[ct], acc_i[ct][qb], 0, 0, 0);
          }
        }
      }
    }
    if (PROD && q < Md) {
      i32x4 lo4[kSMCT], hi4[kSMCT];
#pragma unroll
      for (int ct = 0; ct < kSMCT; ++ct) bit_slices(scur[ct], lo4[ct], hi4[ct]);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const i32x4 a0 = As[cur][(qb * NJ + 2 * NP) * 64 + lane];
        const i32x4 a1 = As[cur][(qb * NJ + 2 * NP + 1) * 64 + lane];
#pragma unroll
        for (int ct = 0; ct < kSMCT; ++ct) {
          acc_s[ct][qb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, lo4[ct], acc_s[ct][qb], 0, 0, 0);
          acc_s[ct][qb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, hi4[ct], acc_s[ct][qb], 0, 0, 0);
        }
      }
    }

    if (more) {
#pragma unroll
      for (int j = 0; j < kPer; ++j)
        if (tid + j * kThreads < kStage) As[cur ^ 1][tid + j * kThreads] = ar[j];
#pragma unroll
      for (int ct = 0; ct < kSMCT; ++ct) {
#pragma unroll
        for (int p = 0; p < BB; ++p) wcur[ct][p] = wnx[ct][p];
        scur[ct] = snx[ct];
      }
    }
    if (last) {
      // ---- epilogue of block cbk: lane (kc, kg) of tile (ct, qb) = query
      // 4 (QB qblk + qb) + kg, code cbk * kSMCodes + wave * 16 kSMCT + 16 ct + kc
      const int64_t vbase = cbk * kSMCodes + wave * (16 * kSMCT) + kc;
      // logit of tile (ct, qb), exact integer sums combined in float64
#define TQ_LOGIT(CT, QB_)                                                                    \
  ([&]() -> float {                                                                          \
    const QConst &cst_ = qcs[(QB_) * 4 + kg];                                                \
    double l_ = 0.0;                                                                         \
    if (NP > 0) {                                                                            \
      const i32x4 a_ = acc_i[CT][QB_];                                                       \
      const double v_ = (double)a_[0] + 128.0 * (double)a_[1] + 16384.0 * (double)a_[2] +    \
                        2097152.0 * (double)a_[3];                                           \
      l_ += (double)kn[CT] * (v_ * cst_.idx_scale - cst_.idx_bias);                          \
    }                                                                                        \
    if (PROD) {                                                                              \
      const i32x4 a_ = acc_s[CT][QB_];                                                       \
      const double v_ = (double)a_[0] + 128.0 * (double)a_[1] + 16384.0 * (double)a_[2] +    \
                        2097152.0 * (double)a_[3];                                           \
      l_ += (double)rn[CT] * (v_ * cst_.sgn_scale - cst_.sgn_bias);                          \
    }                                                                                        \
    return (float)l_;                                                                        \
  }())
      if constexpr (!TOPK) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const int64_t qi = ((int64_t)qblk * QB + qb) * 4 + kg;
#pragma unroll
          for (int ct = 0; ct < kSMCT; ++ct) {
            const float lf = TQ_LOGIT(ct, qb);
            const int64_t vpos = vbase + 16 * ct;
            if (qi < g && vpos < seq) logits[((size_t)head * g + qi) * seq + vpos] = lf;
          }
        }
      } else {
        // candidates beat their query's k-th entry; usually there are none
        // and the block costs a compare per logit and one ballot
        uint32_t pend = 0;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const float tv = tlv[wave][qb * 4 + kg][k - 1];
          const int ti = tli[wave][qb * 4 + kg][k - 1];
          const float ts = tau_sh[qb * 4 + kg];
#pragma unroll
          for (int ct = 0; ct < kSMCT; ++ct) {
            const int64_t vpos = vbase + 16 * ct;
            const float lf = TQ_LOGIT(ct, qb);
            if (vpos < seq && lf >= ts && better_vi(lf, (int)vpos, tv, ti)) pend |= 1u << (qb * kSMCT + ct);
          }
        }
        if (__ballot(pend != 0)) {
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int ct = 0; ct < kSMCT; ++ct) {
              // each lane group inserts its pending candidates one at a time
              const int bit = qb * kSMCT + ct;
              bool pd = (pend >> bit) & 1u;
              uint64_t bal = __ballot(pd);
              if (!bal) continue;
              const float lf = TQ_LOGIT(ct, qb);
              const int cidx = (int)(vbase + 16 * ct);
              float *lvq = &tlv[wave][qb * 4 + kg][0];
              int *liq = &tli[wave][qb * 4 + kg][0];
              while (bal) {
                const uint32_t gb = (uint32_t)(bal >> (16 * kg)) & 0xFFFFu;
                const bool has = gb != 0;
                const int src = 16 * kg + (has ? __ffs(gb) - 1 : 0);
                const float cv = __shfl(lf, src);
                const int ci = __shfl(cidx, src);
                group_insert<K>(lvq, liq, lane, kg, k, has, cv, ci);
                if (has && lane == src) pd = false;
                __builtin_amdgcn_wave_barrier();
                pd = pd && better_vi(lf, cidx, lvq[k - 1], liq[k - 1]);
                bal = __ballot(pd);
              }
            }
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            if ((lane & 15) == 0) lds_fmax(&tau_sh[qb * 4 + kg], tlv[wave][qb * 4 + kg][k - 1]);
        }
      }
#undef TQ_LOGIT
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int ct = 0; ct < kSMCT; ++ct) {
          acc_i[ct][qb] = i32x4{0, 0, 0, 0};
          acc_s[ct][qb] = i32x4{0, 0, 0, 0};
        }
    }
    if (last) {
      q = 0;
      ++cbk;
    } else {
      ++q;
    }
    __syncthreads();
  }
#undef TQ_LOAD_WORDS
  if constexpr (TOPK) {
    // this wave's lists -> candidates [head * g + query][segment][wave][k]
    for (int i = lane; i < NQ * k; i += 64) {
      const int qq = i / k, r = i % k;
      const int64_t qi = (int64_t)qblk * NQ + qq;
      if (qi < g) {
        const size_t o = ((((size_t)head * g + qi) * nseg + seg) * kSMWaves + wave) * k + r;
        cand_v[o] = tlv[wave][qq][r];
        cand_i[o] = tli[wave][qq][r];
      }
    }
  }
}

// Final top-k of each query from its segments' candidate lists: one wave per
// query; per-lane sorted lists, then k rounds of wave-wide arg-max.
template <int K>
__global__ __launch_bounds__(256) void topk_merge_kernel(const float *__restrict__ cand_v,
                                                         const int *__restrict__ cand_i,
                                                         int64_t nrows, int ncand, int k,
                                                         int64_t *__restrict__ out_idx,
                                                         float *__restrict__ out_val) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= nrows) return;
  const float *cv = cand_v + row * ncand;
  const int *ci = cand_i + row * ncand;
  float v[K];
  int id[K];
#pragma unroll
  for (int i = 0; i < K; ++i) { v[i] = -INFINITY; id[i] = 0x7fffffff; }
  for (int j = lane; j < ncand; j += 64) {
    float cvv = cv[j];
    int cii = ci[j];
    if (better_vi(cvv, cii, v[K - 1], id[K - 1])) {
#pragma unroll
      for (int i = 0; i < K; ++i) {
        if (better_vi(cvv, cii, v[i], id[i])) {
          const float tv = v[i];
          const int ti = id[i];
          v[i] = cvv; id[i] = cii;
          cvv = tv; cii = ti;
        }
      }
    }
  }
  int head = 0;
  for (int r = 0; r < k; ++r) {
    float hv = -INFINITY;
    int hi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < K; ++i)
      if (i == head) { hv = v[i]; hi = id[i]; }
    float bv = hv;
    int bi = hi, bl = lane;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      const int ol = __shfl_xor(bl, off);
      if (better_vi(ov, oi, bv, bi)) { bv = ov; bi = oi; bl = ol; }
    }
    if (lane == bl) ++head;
    if (lane == 0) {
      out_idx[row * k + r] = bi;
      if (out_val) out_val[row * k + r] = bv;
    }
  }
}

// ---- workspace layout and launchers
struct ManyLayout {
  int QB, NJ, NCH, nqb;
  size_t aops, qc, proj, cand_v, cand_i, total;  // byte offsets, total size
};

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static ManyLayout many_layout(const tq_params &p, int64_t n_kv, int64_t g, int nseg, int k) {
  ManyLayout L;
  const bool prod = p.mode == TQ_MODE_PROD;
  const int B = prod ? p.b - 1 : p.b;
  L.QB = sm_qb(B, prod, list_cap(k));
  L.NJ = sm_nj(B, prod);
  const int Qd = p.d / 128, Md = prod ? p.m / 128 : 0;
  L.NCH = Qd > Md ? Qd : Md;
  L.nqb = (int)((g + 4 * L.QB - 1) / (4 * L.QB));
  const size_t rows = p.d + (prod ? p.m : 0);
  size_t o = 0;
  L.aops = o;
  o = align256(o + (size_t)n_kv * L.nqb * L.NCH * L.QB * L.NJ * 64 * sizeof(i32x4));
  L.qc = o;
  o = align256(o + (size_t)n_kv * L.nqb * 4 * L.QB * sizeof(QConst));
  L.proj = o;
  o = align256(o + (size_t)n_kv * g * rows * sizeof(double));
  L.cand_v = o;
  o = align256(o + (size_t)n_kv * g * nseg * kSMWaves * k * sizeof(float));
  L.cand_i = o;
  o = align256(o + (size_t)n_kv * g * nseg * kSMWaves * k * sizeof(int));
  L.total = o;
  return L;
}

// Segments of code blocks per (head, query block): about four workgroups per
// CU in total, every segment non-empty.
static int many_segments(const tq_params &p, int64_t n_kv, int64_t g, int64_t n, int cus, int k) {
  const bool prod = p.mode == TQ_MODE_PROD;
  const int B = prod ? p.b - 1 : p.b;
  const int QB = sm_qb(B, prod, list_cap(k));
  const int64_t nqb = (g + 4 * QB - 1) / (4 * QB);
  const int64_t ncb = std::max<int64_t>(1, (n + kSMCodes - 1) / kSMCodes);
  int64_t nseg = std::max<int64_t>(1, (4LL * cus + n_kv * nqb - 1) / (n_kv * nqb));
  nseg = std::min<int64_t>(nseg, ncb);
  const int64_t cps = (ncb + nseg - 1) / nseg;
  return (int)((ncb + cps - 1) / cps);
}

static int search_segments(const tq_params &p, int64_t nq, int64_t n, int k) {
  return many_segments(p, 1, nq, n, 256, k);
}

size_t search_workspace_bytes(const tq_params &p, int64_t nq, int64_t n, int k) {
  return many_layout(p, 1, nq, search_segments(p, nq, n, k), k).total;
}

template <int B, bool PROD, bool TOPK, int K>
static void launch_many_t(const Derived &D, const float *q, int64_t n_kv, int64_t g, tq_codes c,
                          int64_t seq, float *logits, char *ws, int nseg, int k, hipStream_t s) {
  const ManyLayout L = many_layout(D.p, n_kv, g, nseg, k);
  const int rows = D.p.d + (PROD ? D.p.m : 0);
  double *proj = (double *)(ws + L.proj);
  i32x4 *aops = (i32x4 *)(ws + L.aops);
  QConst *qc = (QConst *)(ws + L.qc);
  qproj_kernel<<<dim3(rows / kQJR, (unsigned)((n_kv * g + kQJQ - 1) / kQJQ)), dim3(256), 0, s>>>(
      q, n_kv * g, D.p.d, rows, D.pi32, D.s32, proj);
  qops_kernel<PROD><<<dim3((unsigned)(n_kv * L.nqb * L.QB)), dim3(256), 0, s>>>(
      proj, g, L.nqb, L.QB, D.p.d, D.p.m, D.cb, aops, qc);
  const int64_t ncb = (seq + kSMCodes - 1) / kSMCodes;
  const int cps = (int)((ncb + nseg - 1) / nseg);
  score_many_kernel<B, PROD, TOPK, K>
      <<<dim3((unsigned)(L.nqb * nseg), (unsigned)n_kv), dim3(kSMWaves * 64), 0, s>>>(
          aops, qc, c.idx, c.sgn, c.knorm, c.rnorm, seq, g, L.nqb, nseg, cps, D.p.d / 128,
          PROD ? D.p.m / 128 : 0, k, logits, (float *)(ws + L.cand_v), (int *)(ws + L.cand_i));
}

template <bool TOPK, int K>
static tq_status launch_many(const Derived &D, const float *q, int64_t n_kv, int64_t g, tq_codes c,
                             int64_t seq, float *logits, char *ws, int nseg, int k, hipStream_t s) {
  const ManyLayout L = many_layout(D.p, n_kv, g, nseg, k);
  if (n_kv > 65535 || (int64_t)L.nqb * nseg > 0x7fffffffLL || n_kv * L.nqb * L.QB > 0x7fffffffLL ||
      seq > 0x7fffffffLL) {
    set_error("problem too large for one launch");
    return TQ_ERR_UNSUPPORTED;
  }
  const bool prod = D.p.mode == TQ_MODE_PROD;
  switch (D.B * 2 + (prod ? 1 : 0)) {
    case 0 * 2 + 1: launch_many_t<0, true, TOPK, K>(D, q, n_kv, g, c, seq, logits, ws, nseg, k, s); break;
    case 1 * 2 + 1: launch_many_t<1, true, TOPK, K>(D, q, n_kv, g, c, seq, logits, ws, nseg, k, s); break;
    case 2 * 2 + 1: launch_many_t<2, true, TOPK, K>(D, q, n_kv, g, c, seq, logits, ws, nseg, k, s); break;
    case 3 * 2 + 1: launch_many_t<3, true, TOPK, K>(D, q, n_kv, g, c, seq, logits, ws, nseg, k, s); break;
    case 4 * 2 + 1: launch_many_t<4, true, TOPK, K>(D, q, n_kv, g, c, seq, logits, ws, nseg, k, s); break;
    case 1 * 2 + 0: launch_many_t<1, false, TOPK, K>(D, q, n_kv, g, c, seq, logits, ws, nseg, k, s); break;
    case 2 * 2 + 0: launch_many_t<2, false, TOPK, K>(D, q, n_kv, g, c, seq, logits, ws, nseg, k, s); break;
    case 3 * 2 + 0: launch_many_t<3, false, TOPK, K>(D, q, n_kv, g, c, seq, logits, ws, nseg, k, s); break;
    case 4 * 2 + 0: launch_many_t<4, false, TOPK, K>(D, q, n_kv, g, c, seq, logits, ws, nseg, k, s); break;
    default:
      set_error("unsupported B = %d", D.B);
      return TQ_ERR_UNSUPPORTED;
  }
  TQ_LAUNCH_CHECK();
  return TQ_OK;
}

size_t score_workspace_bytes(const tq_params &p, int64_t n_kv, int64_t g) {
  const bool prod = p.mode == TQ_MODE_PROD;
  const int B = prod ? p.b - 1 : p.b;
  if (is_d128(p)) return score128_workspace_bytes(B, prod, n_kv, g);
  return many_layout(p, n_kv, g, 1, 0).total;
}

tq_status launch_search(const Derived &D, const float *q, int64_t nq, tq_codes c, int64_t n,
                        int k, int64_t *out_idx, float *out_val, void *ws, hipStream_t s) {
  const int nseg = search_segments(D.p, nq, n, k);
  tq_status st;
  if (k <= 8)
    st = launch_many<true, 8>(D, q, 1, nq, c, n, nullptr, (char *)ws, nseg, k, s);
  else if (k <= 16)
    st = launch_many<true, 16>(D, q, 1, nq, c, n, nullptr, (char *)ws, nseg, k, s);
  else
    st = launch_many<true, 32>(D, q, 1, nq, c, n, nullptr, (char *)ws, nseg, k, s);
  if (st != TQ_OK) return st;
  const ManyLayout L = many_layout(D.p, 1, nq, nseg, k);
  const float *cv = (const float *)((char *)ws + L.cand_v);
  const int *ci = (const int *)((char *)ws + L.cand_i);
  const dim3 grid((unsigned)((nq + 3) / 4)), blk(256);
  const int ncand = nseg * kSMWaves * k;
  if (k <= 8)
    topk_merge_kernel<8><<<grid, blk, 0, s>>>(cv, ci, nq, ncand, k, out_idx, out_val);
  else if (k <= 16)
    topk_merge_kernel<16><<<grid, blk, 0, s>>>(cv, ci, nq, ncand, k, out_idx, out_val);
  else
    topk_merge_kernel<32><<<grid, blk, 0, s>>>(cv, ci, nq, ncand, k, out_idx, out_val);
  TQ_LAUNCH_CHECK();
  return TQ_OK;
}

tq_status launch_score(const Derived &D, const float *q, int64_t n_kv, int64_t g, tq_codes c,
                       int64_t seq, float *logits, void *ws, hipStream_t s) {
  if (is_d128(D.p)) return launch_score128(D, q, n_kv, g, c, seq, logits, ws, s);
  const int nseg = many_segments(D.p, n_kv, g, seq, num_cus(D.device), 0);
  return launch_many<false, 1>(D, q, n_kv, g, c, seq, logits, (char *)ws, nseg, 0, s);
}

// ===========================================================================
// Attend, d = m = 128: flash-decoding split over the sequence
// ===========================================================================
// Each wave owns kAttKPW consecutive positions of one (batch, KV head, query
// group) and produces, per query, the running max m, the sum l of
// exp(logit - m) and the un-normalised rotated-domain output
//   o_rot[c] = sum_n exp(logit_n - m) ||v_n|| c_V[idx_n][c].
// Phase 1 computes the logits of its positions with the score MFMAs and keeps
// them in LDS.  Phase 2 turns them into weights w = exp(logit - m) ||v||.
// Phase 3 walks 64-position blocks: the value codebook is the odd multilinear
// expansion c_V[idx] = sum_S a_S sigma_S of the bit planes, so
//   o_rot[c] = sum_S sum_n (2 a_S w_n) bit_S,n,c - sum_S a_S sum_n w_n,
// an int8 MFMA with K running over positions: A = 2 a_S w_n quantised to four
// balanced int8 limbs (one power-of-two scale per query, one operand per part
// S, all parts into one accumulator), B = bit c of 4 consecutive positions
// per dword (a byte transpose of their index words with v_perm, then one AND
// per bit slice).  A merge kernel combines the splits and applies Pi_V^T once
// per query head.
constexpr int kAttKPW = 512;   // positions per wave
constexpr int kAttWaves = 4;
constexpr int kAttU = 8;       // key tiles whose loads are issued together
static_assert(kAttWaves == 4, "the in-workgroup merge gives wave j query j of a group of 4");

struct AttPartial {  // per (group, split, query): m, l, o_rot[128]
  float m, l, o[128];
};

// A paged code store (block_table == nullptr: the plain layout).  Page j of
// sequence b holds its positions 512 j .. 512 j + 511 (one attention split);
// vector (page, head, offset) of the store is (page * n_kv + head) * 512 +
// offset.  Sequence lengths are clamped into [1, max_pages * 512] and page
// ids into [0, num_pages), so no input makes a kernel leave the store.
struct PagedKV {
  const int32_t *block_table;  // [batch][max_pages]
  const int32_t *seq_lens;     // [batch]
  int64_t max_pages, num_pages;
  int32_t n_kv;
};

__device__ __forceinline__ int64_t paged_seq_len(const PagedKV &pg, int64_t b) {
  int64_t len = pg.seq_lens[b];
  const int64_t cap = pg.max_pages * kAttKPW;
  return len < 1 ? 1 : (len > cap ? cap : len);
}

template <int BK, int BV>
__global__ __launch_bounds__(kAttWaves * 64, 2) void attend128_kernel(
    const i32x4 *__restrict__ aops, const QConst *__restrict__ qc,
    const uint32_t *__restrict__ kidx, const uint32_t *__restrict__ ksgn,
    const float *__restrict__ knorm, const float *__restrict__ rnorm,
    const uint32_t *__restrict__ vidx, const float *__restrict__ vnorm, int64_t seq, int64_t g,
    int ngroups, int nsplit, float scale, Codebook kcb, Codebook vcb,
    AttPartial *__restrict__ part, PagedKV pg) {
  constexpr int NPK = BK == 0 ? 0 : (BK == 1 ? 1 : BK == 2 ? 2 : BK == 3 ? 4 : 8);
  constexpr int NPV = BV == 1 ? 1 : BV == 2 ? 2 : BV == 3 ? 4 : 8;
  constexpr int NMF = score_mfmas(NPK, true);
  constexpr int BKK = BK > 0 ? BK : 1;
  // Up to 4 parity parts share one quantisation of the weights and keep an
  // accumulator set each; 8 parts (4-bit values) would need 256 accumulator
  // registers, so there each part quantises its own scaled weights into one
  // shared accumulator set.
  constexpr bool SHARED = NPV <= 4;
  constexpr int NQ = SHARED ? 1 : NPV;   // quantised weight sets per block
  constexpr int NACC = SHARED ? NPV : 1;  // accumulator sets
  __shared__ __attribute__((aligned(16))) float lg[kAttWaves][4][kAttKPW];  // logits, then weights
  // one block of quantised weights: [set][query][limb][positions / 4]
  __shared__ __attribute__((aligned(16))) uint32_t limbs[kAttWaves][NQ][4][4][64 / 4];
  // value index words of a 64-position block, copied into LDS by the
  // memory unit (no registers) one block ahead of their use: two slots
  constexpr bool VDMA = SHARED;
  __shared__ __attribute__((aligned(16))) uint32_t vbuf[kAttWaves][2][VDMA ? 64 * 4 * BV : 4];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hg = blockIdx.y;  // (batch * n_kv + head) * ngroups + group
  const int hb = hg / ngroups;
  const int split = blockIdx.x * kAttWaves + wave;
  const int c16 = lane & 15, kg = lane >> 4;
  const int64_t p0 = (int64_t)split * kAttKPW;
  // The wave's positions p0 .. p0 + npos - 1 are the vectors vb + 0 .. npos - 1
  // of the code store: one contiguous run per (batch, KV head) in the plain
  // layout, one page of the block table in the paged one.
  // A wave past the end of its sequence computes nothing but still takes part
  // in the workgroup's merge of its waves' partial results below.
  int64_t vb = 0;
  bool active;
  if (pg.block_table) {
    const int64_t b = hb / pg.n_kv, h = hb % pg.n_kv;
    seq = paged_seq_len(pg, b);
    active = p0 < seq;
    if (active) {
      int64_t page = pg.block_table[b * pg.max_pages + split];
      page = page < 0 ? 0 : (page >= pg.num_pages ? pg.num_pages - 1 : page);  // never outside the store
      vb = (page * pg.n_kv + h) * kAttKPW;
    }
  } else {
    active = split < nsplit;
    vb = (int64_t)hb * seq + p0;
  }
  // this lane's 8 output coordinates of o_rot (query kg), and m, l of the query
  float ov[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float m_out = -INFINITY, l_out = 0.f;
  const int w = c16 >> 2, beta = c16 & 3;
  if (active) {
  const int npos = (int)(seq - p0 < kAttKPW ? seq - p0 : kAttKPW);

  // ---------------- phase 1: logits of this wave's positions
  float m;
  {
    i32x4 A[NMF];
#pragma unroll
    for (int j = 0; j < NMF; ++j) A[j] = aops[((int64_t)hg * NMF + j) * 64 + lane];
    const QConst cst = qc[(int64_t)hg * 4 + kg];
    // the wave's positions through buffer descriptors of exactly its npos
    // codes (positions past them read zeros, and their logits are -inf):
    // position 16 t + c16 at the lane's offset plus a per-tile scalar offset
    const bufrsrc rki = buf_rsrc(kidx + vb * 4 * BKK, (uint32_t)npos * 16u * BKK);
    const bufrsrc rks = buf_rsrc(ksgn + vb * 4, (uint32_t)npos * 16u);
    const bufrsrc rkn = buf_rsrc(knorm + vb, (uint32_t)npos * 4u);
    const bufrsrc rrn = buf_rsrc(rnorm + vb, (uint32_t)npos * 4u);
    const uint32_t oki = (uint32_t)(4 * c16 + kg) * 4u * BKK, oks = (uint32_t)(4 * c16 + kg) * 4u;
    const uint32_t okn = (uint32_t)c16 * 4u;
    // a full split passes each tile's offset as the scalar offset (every
    // access in range); the last split of a sequence adds it to the lane's
    // offset, where the range check turns positions past npos into zeros
    auto logits_of = [&](auto full_c) -> float {
      constexpr bool FULL = decltype(full_c)::value;
      auto ld = [&](auto n_c, bufrsrc r, uint32_t lane_off, uint32_t tile_off, uint32_t *out) {
        constexpr int N = decltype(n_c)::value;
        if constexpr (FULL)
          buf_ldn<N>(r, lane_off, tile_off, out);
        else
          buf_ldn<N>(r, lane_off + tile_off, 0u, out);
      };
      float mx = -INFINITY;
      for (int t0 = 0; t0 < kAttKPW / 16; t0 += kAttU) {
        uint32_t planes[kAttU][BKK], sw[kAttU], kr[kAttU], rr[kAttU];
#pragma unroll
        for (int u = 0; u < kAttU; ++u) {
          const uint32_t tile = (uint32_t)(t0 + u);
          if constexpr (BK > 0) ld(std::integral_constant<int, BK>{}, rki, oki, tile * 256u * BKK, planes[u]);
          ld(std::integral_constant<int, 1>{}, rks, oks, tile * 256u, &sw[u]);
          ld(std::integral_constant<int, 1>{}, rkn, okn, tile * 64u, &kr[u]);
          ld(std::integral_constant<int, 1>{}, rrn, okn, tile * 64u, &rr[u]);
        }
#pragma unroll
        for (int u = 0; u < kAttU; ++u) {
          const int pl = (t0 + u) * 16 + c16;
          const float lt = tile_logit_f32<BK, true, NPK>(A, planes[u], sw[u], __uint_as_float(kr[u]),
                                                         __uint_as_float(rr[u]), cst.f[0], cst.f[1], cst.f[2],
                                                         cst.f[3]);
          const float logit = (FULL || pl < npos) ? lt * scale : -INFINITY;
          lg[wave][kg][pl] = logit;
          mx = fmaxf(mx, logit);
        }
      }
      return mx;
    };
    float mx = npos == kAttKPW ? logits_of(std::true_type{}) : logits_of(std::false_type{});
    // max over the 16 lanes of this query (lanes 16 kg .. 16 kg + 15)
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    m = mx;
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();

  // ---------------- phase 2: weights w = exp(logit - m) * ||v||, in place
  // lane (c16, kg): query kg, positions 4 c16 + 64 r + {0..3}
  float lsum = 0.f, wmax = 0.f;
  {
    const bufrsrc rvn = buf_rsrc(vnorm + vb, (uint32_t)npos * 4u);
#pragma unroll
    for (int r = 0; r < kAttKPW / 64; ++r) {
      const int pl0 = 64 * r + 4 * c16;
      const float4 lv = *reinterpret_cast<const float4 *>(&lg[wave][kg][pl0]);
      const float lvv[4] = {lv.x, lv.y, lv.z, lv.w};
      uint32_t vnr[4];
      buf_ldn<4>(rvn, (uint32_t)c16 * 16u + (uint32_t)r * 256u, 0u, vnr);  // past npos: zeros
      float wv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int pl = pl0 + e;
        const float pe = pl < npos ? __expf(lvv[e] - m) : 0.f;
        lsum += pe;
        wv[e] = pe * __uint_as_float(vnr[e]);
        wmax = fmaxf(wmax, wv[e]);
      }
      *reinterpret_cast<float4 *>(&lg[wave][kg][pl0]) = make_float4(wv[0], wv[1], wv[2], wv[3]);
    }
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) {
      lsum += __shfl_xor(lsum, off);
      wmax = fmaxf(wmax, __shfl_xor(wmax, off));
    }
  }
  // one power-of-two scale per query: shared, w 2^E < 2^27 (4 unsigned
  // 7-bit limbs); per part, |2 a_S w| 2^E < 2^26 (4 balanced limbs)
  int E = 0;
  {
    double amax = 0.0;
#pragma unroll
    for (int sp = 0; sp < NPV; ++sp) amax = fmax(amax, fabs(vcb.coef[sp]));
    int k;
    const double A1 = SHARED ? (double)wmax : 2.0 * amax * (double)wmax;
    if (A1 > 0) { frexp(A1, &k); E = (SHARED ? 27 : 26) - k; }
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();

  // ---------------- phase 3: o_rot = sum_n w_n c_V[idx_n] as int8 MFMAs
  // B lane (c16 = (w, beta), kg) covers positions 16 kg + 4 gi + e of each
  // block: byte e of dword gi of D_beta is byte beta of index word w of
  // position 4 gi + e.  Slice s (bit s of every byte; a set bit weighs
  // 2^(s & 3)) is coordinate 32 beta + 16 (s / 4) + 4 w + s % 4.
  const uint32_t sel_lo = (uint32_t)(beta | (beta + 4) << 8 | 0x0C0C0000u);
  i32x4 acc[NACC][8];
#pragma unroll
  for (int a = 0; a < NACC; ++a)
#pragma unroll
    for (int sl = 0; sl < 8; ++sl) acc[a][sl] = i32x4{0, 0, 0, 0};
  // shared: sum of this lane's Q; per part: sum of Q / 2 * 2^-E
  double qsum = 0.0;
  const uint32_t *vi = vidx + vb * 4 * BV;
  const uint32_t woff = (uint32_t)w * (4u * BV);  // byte offset of index word w
  // value index words through a descriptor of the wave's npos codes; lane
  // (c16 = (w, beta), kg) reads word w of positions 16 kg + 4 gi + e of a
  // block: the lane's offset plus a scalar offset per load.  Quantisation of
  // one block: lane (c16, kg) takes query kg, positions 4 c16 .. 4 c16 + 3.
  const bufrsrc rvi = buf_rsrc(vi, (uint32_t)npos * 16u * BV);
  const uint32_t vlane = (uint32_t)(16 * kg) * (16u * BV) + woff;
  // block b's 64 * 16 BV bytes are contiguous: BV copies of 1 KB, lane l
  // taking bytes 16 l .. 16 l + 15 of each; positions past npos read zeros
  // (their weights are zero, so what a slot holds there never counts)
  auto copy_block = [&](int b) {
#pragma unroll
    for (int k = 0; k < BV; ++k)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rvi, (__attribute__((address_space(3))) void *)&vbuf[wave][b & 1][256 * k], 16,
          (int)((uint32_t)b * (1024u * BV) + 1024u * k + 16u * (uint32_t)lane), 0, 0, 2);
  };
  if constexpr (VDMA) copy_block(0);
  for (int blk = 0; blk < kAttKPW / 64; ++blk) {
    // V index words of this lane's 16 positions (issued first)
    uint32_t x[4][4][BV];
    if constexpr (VDMA) {
      // the copy of this block is the wave's only vector-memory operation
      // in flight here (the compiler does not track these copies itself)
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      const uint32_t *vb_ = &vbuf[wave][blk & 1][0];
#pragma unroll
      for (int gi = 0; gi < 4; ++gi)
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int p = 0; p < BV; ++p) x[gi][e][p] = vb_[(16 * kg + 4 * gi + e) * 4 * BV + w * BV + p];
    } else if (npos == kAttKPW) {  // every access in range: scalar offsets
#pragma unroll
      for (int gi = 0; gi < 4; ++gi)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          buf_ldn<BV>(rvi, vlane, (uint32_t)(blk * 64 + 4 * gi + e) * (16u * BV), x[gi][e]);
    } else {  // range-checked lane offsets: positions past npos read zeros
#pragma unroll
      for (int gi = 0; gi < 4; ++gi)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          buf_ldn<BV>(rvi, vlane + (uint32_t)(blk * 64 + 4 * gi + e) * (16u * BV), 0u, x[gi][e]);
    }
    {
      const float4 wv4 = *reinterpret_cast<const float4 *>(&lg[wave][kg][blk * 64 + 4 * c16]);
      const float wv[4] = {wv4.x, wv4.y, wv4.z, wv4.w};
      if constexpr (SHARED) {
        // Q = w 2^E rounded (0 <= Q < 2^27), limbs = its base-128 digits
        uint32_t lw[4] = {0u, 0u, 0u, 0u};
        uint32_t qs = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t Q = (uint32_t)rintf(ldexpf(wv[e], E));
          qs += Q;
#pragma unroll
          for (int t = 0; t < 4; ++t) lw[t] |= ((Q >> (7 * t)) & 127u) << (8 * e);
        }
        qsum += (double)qs;
#pragma unroll
        for (int t = 0; t < 4; ++t) limbs[wave][0][kg][t][c16] = lw[t];
      } else {
#pragma unroll
        for (int sp = 0; sp < NQ; ++sp) {
          // Q = 2 a_S w 2^E rounded in float32: any integer near it serves, as
          // the MFMA sum and the correction qsum use the same Q
          const float cf = (float)ldexp(2.0 * vcb.coef[sp], E);
          uint32_t lw[4] = {0u, 0u, 0u, 0u};
          int qs = 0;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            int Q = (int)rintf(cf * wv[e]);
            qs += Q;
#pragma unroll
            for (int t = 0; t < 4; ++t) {  // balanced base-128 digits, lowest first
              const int digit = ((Q + 64) & 127) - 64;
              Q = (Q - digit) >> 7;  // exact: Q - digit is a multiple of 128
              lw[t] |= (uint32_t)(digit & 0xFF) << (8 * e);
            }
          }
          qsum += ldexp(0.5 * (double)qs, -E);
#pragma unroll
          for (int t = 0; t < 4; ++t) limbs[wave][sp][kg][t][c16] = lw[t];
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    i32x4 Aw0;
    if constexpr (VDMA) {
      // every LDS read of this block is done before the next block's copy
      // is issued into the other slot
      Aw0 = *reinterpret_cast<const i32x4 *>(&limbs[wave][0][c16 >> 2][c16 & 3][4 * kg]);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      if (blk + 1 < kAttKPW / 64) copy_block(blk + 1);
    }
    // transpose: D[S][gi] = parity part S of the byte-beta transposes
    uint32_t D[NPV][4];
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      uint32_t pd[BV];
#pragma unroll
      for (int p = 0; p < BV; ++p) {
        const uint32_t lo = __builtin_amdgcn_perm(x[gi][1][p], x[gi][0][p], sel_lo);
        const uint32_t hi = __builtin_amdgcn_perm(x[gi][3][p], x[gi][2][p], sel_lo);
        pd[p] = lo | hi << 16;
      }
#pragma unroll
      for (int sp = 0; sp < NPV; ++sp) {
        uint32_t pt = 0;
#pragma unroll
        for (int p = 0; p < BV; ++p)
          if (part_mask_ct(BV, sp) >> p & 1) pt ^= pd[p];
        D[sp][gi] = pt;
      }
    }
#pragma unroll
    for (int sp = 0; sp < NPV; ++sp) {
      // A: rows (query c16 / 4, limb c16 % 4), positions 16 kg .. 16 kg + 15
      i32x4 Aw;
      if constexpr (VDMA)
        Aw = Aw0;
      else
        Aw = *reinterpret_cast<const i32x4 *>(&limbs[wave][SHARED ? 0 : sp][c16 >> 2][c16 & 3][4 * kg]);
      i32x4 lo4[4], hi4[4];
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        i32x4 a4, b4;
        bit_slices(D[sp][gi], a4, b4);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          lo4[k][gi] = a4[k];
          hi4[k][gi] = b4[k];
        }
      }
      i32x4 *ac = acc[SHARED ? sp : 0];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        ac[k] = __builtin_amdgcn_mfma_i32_16x16x64_i8(Aw, lo4[k], ac[k], 0, 0, 0);
        ac[4 + k] = __builtin_amdgcn_mfma_i32_16x16x64_i8(Aw, hi4[k], ac[4 + k], 0, 0, 0);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
  }
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) qsum += __shfl_xor(qsum, off);
  // ---------------- epilogue: lane (c16, kg) holds query kg, limbs t = 0..3
  // sum_n w_n c[idx_n] = sum_S a_S (2 sum_n w_n beta_S,n - sum_n w_n)
  {
    double asum = 0.0;
#pragma unroll
    for (int sp = 0; sp < NPV; ++sp) asum += vcb.coef[sp];
#pragma unroll
    for (int sl = 0; sl < 8; ++sl) {
      double v = 0.0;
#pragma unroll
      for (int a = 0; a < NACC; ++a) {
        const i32x4 r = acc[a][sl];
        const double ra = (double)r[0] + 128.0 * (double)r[1] + 16384.0 * (double)r[2] +
                          2097152.0 * (double)r[3];
        v += (SHARED ? 2.0 * vcb.coef[a] : 1.0) * ra;
      }
      // shared: (v 2^-(s&3) - a qsum) 2^-E; per part: v 2^-(E + s&3) - qsum
      ov[sl] = SHARED ? (float)ldexp(ldexp(v, -(sl & 3)) - asum * qsum, -E)
                      : (float)(ldexp(v, -E - (sl & 3)) - qsum);
    }
    m_out = m;
    l_out = lsum;
  }
  }  // active

  // ---------------- merge of the workgroup's waves (consecutive splits):
  // the waves' (m, l, o_rot) go through LDS (each wave's logit buffer, free
  // now) and wave j combines query j:  M = max m_w, L = sum l_w e^(m_w - M),
  // O = sum o_w e^(m_w - M).  Inactive waves carry m = -inf, l = 0, o = 0.
  {
    float *mine = &lg[wave][kg][0];
#pragma unroll
    for (int sl = 0; sl < 8; ++sl) mine[32 * beta + 16 * (sl >> 2) + 4 * w + (sl & 3)] = ov[sl];
    if (c16 == 0) {
      mine[128] = m_out;
      mine[129] = l_out;
    }
  }
  __syncthreads();
  {
    const int jq = wave;  // query of the group this wave combines
    const int64_t qh = (int64_t)(hg % ngroups) * 4 + jq;
    float mw[kAttWaves], M = -INFINITY;
#pragma unroll
    for (int v = 0; v < kAttWaves; ++v) {
      mw[v] = lg[v][jq][128];
      M = fmaxf(M, mw[v]);
    }
    float sc[kAttWaves], L = 0.f;
#pragma unroll
    for (int v = 0; v < kAttWaves; ++v) {
      sc[v] = M == -INFINITY ? 0.f : __expf(mw[v] - M);
      L = fmaf(lg[v][jq][129], sc[v], L);
    }
    float o0 = 0.f, o1 = 0.f;
#pragma unroll
    for (int v = 0; v < kAttWaves; ++v) {
      o0 = fmaf(lg[v][jq][lane], sc[v], o0);
      o1 = fmaf(lg[v][jq][64 + lane], sc[v], o1);
    }
    if (qh < g) {
      AttPartial *dst = part + ((int64_t)hg * gridDim.x + blockIdx.x) * 4 + jq;
      dst->o[lane] = o0;
      dst->o[64 + lane] = o1;
      if (lane == 0) {
        dst->m = M;
        dst->l = L;
      }
    }
  }
}

// Combine the partials of one query head and rotate back: out = Pi_V^T o_rot / L.
// Thread (c, grp) runs an online softmax over partials grp, grp + 8, ... for
// coordinate c (one pass; the loads do not wait on a reduction), the 8 groups
// are combined through LDS, and the rows of Pi_V this thread needs are loaded
// before any of it.
constexpr int kMergeThreads = 1024;
constexpr int kMergeGroups = kMergeThreads / 128;  // partial groups per coordinate
__global__ __launch_bounds__(kMergeThreads) void attend_merge_kernel(
    const AttPartial *__restrict__ part, int nsplit_max, int ngroups, int64_t g,
    const float *__restrict__ piv, float *__restrict__ out, PagedKV pg) {
  constexpr int R = 128 / kMergeGroups;  // rows of Pi_V per thread in the rotation
  __shared__ float gm[kMergeGroups], gl[kMergeGroups];
  __shared__ float orot[kMergeGroups][128];
  __shared__ float osum[128];
  const int hq = blockIdx.x;        // (batch * n_kv + head) * g + j
  const int64_t hb = hq / g, j = hq % g;
  const int64_t hg = hb * ngroups + j / 4;
  const int jq = (int)(j % 4);
  const int tid = threadIdx.x;
  const int c = tid & 127, grp = tid >> 7;
  float pv[R];
#pragma unroll
  for (int r = 0; r < R; ++r) pv[r] = piv[(grp * R + r) * 128 + c];
  const AttPartial *p = part + (int64_t)hg * nsplit_max * 4 + jq;
  // partials written for this sequence, one per workgroup of kAttWaves
  // splits (all of them in the plain layout)
  const int nsplit = pg.block_table
                         ? (int)((paged_seq_len(pg, hb / pg.n_kv) + kAttKPW * kAttWaves - 1) /
                                 (kAttKPW * kAttWaves))
                         : nsplit_max;
  float M = -INFINITY, L = 0.f, O = 0.f;
#pragma unroll 4
  for (int sidx = grp; sidx < nsplit; sidx += kMergeGroups) {
    const AttPartial *ps = p + (int64_t)sidx * 4;
    const float ms = ps->m, ls = ps->l, os = ps->o[c];
    const float mn = fmaxf(M, ms);
    const float a = M == -INFINITY ? 0.f : __expf(M - mn), b = __expf(ms - mn);
    L = fmaf(L, a, ls * b);
    O = fmaf(O, a, os * b);
    M = mn;
  }
  orot[grp][c] = O;
  if (c == 0) {
    gm[grp] = M;
    gl[grp] = L;
  }
  __syncthreads();
  if (tid < 128) {
    float Mx = -INFINITY;
#pragma unroll
    for (int k = 0; k < kMergeGroups; ++k) Mx = fmaxf(Mx, gm[k]);
    float Lt = 0.f, Ot = 0.f;
#pragma unroll
    for (int k = 0; k < kMergeGroups; ++k) {
      const float e = gm[k] == -INFINITY ? 0.f : __expf(gm[k] - Mx);
      Lt = fmaf(gl[k], e, Lt);
      Ot = fmaf(orot[k][tid], e, Ot);
    }
    osum[tid] = Ot / Lt;
  }
  __syncthreads();
  // out = Pi_V^T o_rot: thread (c, grp) sums rows grp R .. grp R + R - 1
  float o = 0.f;
#pragma unroll
  for (int r = 0; r < R; ++r) o = fmaf(pv[r], osum[grp * R + r], o);
  orot[grp][c] = o;  // every read of orot above is behind the barrier
  __syncthreads();
  if (tid < 128) {
    float t = 0.f;
#pragma unroll
    for (int k = 0; k < kMergeGroups; ++k) t += orot[k][tid];
    out[(int64_t)hq * 128 + tid] = t;
  }
}

static int nparts_of_(int B) { return B == 0 ? 0 : (B == 1 ? 1 : B == 2 ? 2 : B == 3 ? 4 : 8); }

size_t attend_workspace_bytes(const Derived &K, const Derived &V, int64_t batch, int64_t n_kv,
                              int64_t g, int64_t seq) {
  (void)V;
  const int64_t ngroups = (g + 3) / 4;
  const int64_t nhg = batch * n_kv * ngroups;
  const int64_t nsplit = (seq + kAttKPW - 1) / kAttKPW;
  const int NMF = score_mfmas(nparts_of_(K.B), true);
  return (size_t)nhg * ((size_t)NMF * 64 * sizeof(i32x4) + 4 * sizeof(QConst)) +
         (size_t)nhg * nsplit * 4 * sizeof(AttPartial) + 256;
}

template <int BK, int BV>
static void launch_attend_t(const Derived &K, const Derived &V, const float *q, int64_t batch,
                            int64_t n_kv, int64_t g, tq_codes k, tq_codes v, int64_t seq,
                            float scale, float *out, void *ws, hipStream_t s, const PagedKV &pg) {
  const int ngroups = (int)((g + 3) / 4);
  const int64_t nhg = batch * n_kv * ngroups;
  const int nsplit = (int)((seq + kAttKPW - 1) / kAttKPW);
  const int NMF = score_mfmas(nparts_of_(BK), true);
  i32x4 *aops = (i32x4 *)ws;
  QConst *qc = (QConst *)((char *)ws + (size_t)nhg * NMF * 64 * sizeof(i32x4));
  uintptr_t pp = (uintptr_t)((char *)qc + (size_t)nhg * 4 * sizeof(QConst));
  pp = (pp + 255) & ~(uintptr_t)255;
  AttPartial *part = (AttPartial *)pp;
  launch_qprep128<true>(K, q, g, ngroups, nhg, aops, qc, s);
  attend128_kernel<BK, BV><<<dim3((unsigned)((nsplit + kAttWaves - 1) / kAttWaves), (unsigned)nhg),
                             dim3(kAttWaves * 64), 0, s>>>(aops, qc, k.idx, k.sgn, k.knorm, k.rnorm,
                                                           v.idx, v.knorm, seq, g, ngroups, nsplit,
                                                           scale, K.cb, V.cb, part, pg);
  const int nblk = (nsplit + kAttWaves - 1) / kAttWaves;  // partials per query head
  attend_merge_kernel<<<dim3((unsigned)(batch * n_kv * g)), dim3(kMergeThreads), 0, s>>>(part, nblk, ngroups, g,
                                                                               V.pi32, out, pg);
}

tq_status launch_attend(const Derived &K, const Derived &V, const float *q, int64_t batch,
                        int64_t n_kv, int64_t g, tq_codes k, tq_codes v, int64_t seq, float scale,
                        float *out, void *ws, hipStream_t s, const int32_t *block_table,
                        int64_t max_pages, int64_t num_pages, const int32_t *seq_lens) {
  if ((uint64_t)batch * n_kv * ((g + 3) / 4) > 65535u || seq >= (1LL << 28)) {
    set_error("tq_attend: batch * n_kv * ceil(g/4) must be <= 65535 and seq < 2^28");
    return TQ_ERR_UNSUPPORTED;
  }
  // paged: seq = max_pages * 512 sizes the grid; each sequence's length is read on the device
  const PagedKV pg{block_table, seq_lens, max_pages, num_pages, (int32_t)n_kv};
  if (V.B < 1) {
    set_error("tq_attend: values need at least one Lloyd-Max bit");
    return TQ_ERR_UNSUPPORTED;
  }
  switch (K.B * 8 + V.B) {
#define TQ_ATT_CASE(bk, bv) \
    case bk * 8 + bv: launch_attend_t<bk, bv>(K, V, q, batch, n_kv, g, k, v, seq, scale, out, ws, s, pg); break;
    TQ_ATT_CASE(0, 1) TQ_ATT_CASE(0, 2) TQ_ATT_CASE(0, 3) TQ_ATT_CASE(0, 4)
    TQ_ATT_CASE(1, 1) TQ_ATT_CASE(1, 2) TQ_ATT_CASE(1, 3) TQ_ATT_CASE(1, 4)
    TQ_ATT_CASE(2, 1) TQ_ATT_CASE(2, 2) TQ_ATT_CASE(2, 3) TQ_ATT_CASE(2, 4)
    TQ_ATT_CASE(3, 1) TQ_ATT_CASE(3, 2) TQ_ATT_CASE(3, 3) TQ_ATT_CASE(3, 4)
    TQ_ATT_CASE(4, 1) TQ_ATT_CASE(4, 2) TQ_ATT_CASE(4, 3) TQ_ATT_CASE(4, 4)
#undef TQ_ATT_CASE
    default:
      set_error("tq_attend: unsupported bit widths");
      return TQ_ERR_UNSUPPORTED;
  }
  TQ_LAUNCH_CHECK();
  return TQ_OK;
}

// ===========================================================================
// Scratch of the no-allocation attention entry point: one file-scope device
// array per GPU (the module's own copy on each device), used in place of a
// caller workspace.  Host code never passes the array's name to a kernel: its
// device address is looked up once per device with hipGetSymbolAddress (with
// that device current) and kept here.  Nothing in it needs clearing: every
// byte a call reads was written earlier in the same call.
// ===========================================================================
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

tq_status noalloc_scratch(void **out) {
  static std::mutex mu;
  static void *ptr[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    set_error("no usable HIP device for the scratch array");
    return TQ_ERR_HIP;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (ptr[dev] == nullptr) {
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      set_error("hipGetSymbolAddress(scratch) failed on device %d: %s", dev, hipGetErrorString(e));
      return TQ_ERR_HIP;
    }
    ptr[dev] = p;
  }
  *out = ptr[dev];
  return TQ_OK;
}

// ===========================================================================
// Decode (MSE reconstruction), d = 128: x~ = ||x|| Pi^T c[idx]
// ===========================================================================
// 256 threads per workgroup, Pi (float32, 64 KB) in LDS; two vectors per
// round, one output coordinate per thread: x~_j = nu sum_c Pi[c][j] c[idx_c].
template <int B>
__global__ __launch_bounds__(256) void decode128_kernel(const uint32_t *__restrict__ idx,
                                                        const float *__restrict__ knorm,
                                                        int64_t n, const float *__restrict__ pi,
                                                        Codebook cb, float *__restrict__ out) {
  __shared__ float P[128][128];
  __shared__ float cv[2][128];
  const int tid = threadIdx.x;
  for (int i = tid; i < 128 * 32; i += 256)
    reinterpret_cast<float4 *>(&P[0][0])[i] = reinterpret_cast<const float4 *>(pi)[i];
  const int half = tid >> 7, j = tid & 127;
  for (int64_t v0 = (int64_t)blockIdx.x * 2; v0 < n; v0 += (int64_t)gridDim.x * 2) {
    const int64_t v = v0 + half;
    __syncthreads();  // P ready (first round) / cv consumed (later rounds)
    if (v < n) {
      // centroid of coordinate j: word 4 (j / 128) + (j / 4) % 4, bit 4 ((j % 128) / 16) + j % 4
      const int w = (j >> 2) & 3, bit = 4 * (j >> 4) + (j & 3);
      int id = 0;
#pragma unroll
      for (int p = 0; p < B; ++p) id |= (int)((idx[(v * 4 + w) * B + p] >> bit) & 1u) << p;
      cv[half][j] = cb.c[id];
    }
    __syncthreads();
    if (v < n) {
      float acc = 0.f;
#pragma unroll 8
      for (int c = 0; c < 128; ++c) acc = fmaf(P[c][j], cv[half][c], acc);
      out[v * 128 + j] = knorm[v] * acc;
    }
  }
}

__global__ void fill_zero_kernel(float *__restrict__ out, int64_t count) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count;
       i += (int64_t)gridDim.x * blockDim.x)
    out[i] = 0.f;
}

tq_status launch_decode(const Derived &D, tq_codes codes, int64_t n, float *out, hipStream_t s) {
  const int grid = (int)std::min<int64_t>((n + 1) / 2, 4LL * num_cus(D.device));
  switch (D.B) {
    case 0:
      // no Lloyd-Max bits (prod mode with b = 1): the reconstruction is zero
      // (a fill kernel rather than a memset, so the call stays capturable)
      fill_zero_kernel<<<grid, 256, 0, s>>>(out, n * 128);
      break;
    case 1: decode128_kernel<1><<<grid, 256, 0, s>>>(codes.idx, codes.knorm, n, D.pi32, D.cb, out); break;
    case 2: decode128_kernel<2><<<grid, 256, 0, s>>>(codes.idx, codes.knorm, n, D.pi32, D.cb, out); break;
    case 3: decode128_kernel<3><<<grid, 256, 0, s>>>(codes.idx, codes.knorm, n, D.pi32, D.cb, out); break;
    case 4: decode128_kernel<4><<<grid, 256, 0, s>>>(codes.idx, codes.knorm, n, D.pi32, D.cb, out); break;
    default:
      set_error("tq_decode: unsupported B = %d", D.B);
      return TQ_ERR_UNSUPPORTED;
  }
  TQ_LAUNCH_CHECK();
  return TQ_OK;
}

// ===========================================================================
// PolarQuant, d = 128 (level 1: 4 bits, levels 2..7: 2 bits)
// ===========================================================================
// Encode: the rotation is the TurboQuant GEMM 1 (bf16 hi/lo fragments of Pi
// in LDS), one 16-row tile nt at a time: lane (v, g) receives
// y[16 nt + 4 g + i] of vector v.  Levels 1 and 2 pair coordinates inside
// the lane; level 3 pairs lane groups g, g ^ 1 and level 4 g, g ^ 2 (one
// shuffle each); levels 5..7 pair the tiles nt inside the lane.  Every level
// >= 2 decision is taken on squared radii (theta >= t  <=>
// r_R^2 >= tan^2(t) r_L^2), so no square root or arctangent is needed;
// level 1 takes the quadrant from the signs and the sector within it from
// the turned pair against tan of the sub-sector boundaries.
constexpr int kPolWaves = 16;

__device__ __forceinline__ uint32_t polar_sector(float a, float b, float t8, float t38) {
  // quadrant q: psi in [q pi/2, (q + 1) pi/2); (a', b') = (a, b) turned back by q pi/2
  const bool q1 = a <= 0.f && b > 0.f, q2 = a < 0.f && b <= 0.f, q3 = a >= 0.f && b < 0.f;
  const float ap = q1 ? b : (q2 ? -a : (q3 ? -b : a));
  const float bp = q1 ? -a : (q2 ? -b : (q3 ? a : b));
  const uint32_t q = q1 ? 1u : (q2 ? 2u : (q3 ? 3u : 0u));
  // sub-sector: angle >= pi/8, pi/4, 3 pi/8  <=>  b' >= a' tan(boundary)
  const uint32_t sub = (bp >= ap * t8 ? 1u : 0u) + (bp >= ap ? 1u : 0u) + (bp >= ap * t38 ? 1u : 0u);
  const bool zero = a == 0.f && b == 0.f;  // the zero pair has angle 0
  return zero ? 0u : 4u * q + sub;
}

// Code of the angle between radii with squares sl (left) and sr (right):
// theta >= t  <=>  sr >= tan^2(t) sl.  The level's boundaries are t1, pi/4
// and pi/2 - t1 (tau = tan^2 t1; tan^2(pi/2 - t1) = 1 / tau).
__device__ __forceinline__ uint32_t polar_level_code(float sl, float sr, float tau) {
  const uint32_t c = (sr >= tau * sl ? 1u : 0u) + (sr >= sl ? 1u : 0u) + (tau * sr >= sl ? 1u : 0u);
  return sl + sr > 0.f ? c : 0u;
}

template <bool XBF16>
__global__ __launch_bounds__(kPolWaves * 64) void polar_encode128_kernel(
    const void *__restrict__ x, int64_t n, const uint4 *__restrict__ pi_hi,
    const uint4 *__restrict__ pi_lo, const PolarTables *__restrict__ T, uint32_t *__restrict__ pq,
    float *__restrict__ radius) {
  __shared__ uint4 lds[2 * kFragU4];
  for (int i = threadIdx.x; i < kFragU4; i += blockDim.x) {
    lds[i] = pi_hi[i];
    lds[kFragU4 + i] = pi_lo[i];
  }
  __syncthreads();
  const uint4 *Phi = lds + (threadIdx.x & 63), *Plo = lds + kFragU4 + (threadIdx.x & 63);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int vcol = lane & 15, g = lane >> 4;
  const int64_t nbatch = (n + 15) / 16;
  const float t8 = T->tau1[0], t38 = T->tau1[1];
  float tau[6];
#pragma unroll
  for (int i = 0; i < 6; ++i) tau[i] = T->tau[i];
  for (int64_t batch = (int64_t)blockIdx.x * kPolWaves + wave; batch < nbatch;
       batch += (int64_t)gridDim.x * kPolWaves) {
    const int64_t row = batch * 16 + vcol;
    const bool valid = row < n;
    uint4 xh[4], xl[4];
    float ss = 0.f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) load_x_frag<XBF16>(x, row, valid, kt, g, xh[kt], xl[kt], ss);
    ss += __shfl_xor(ss, 16);
    ss += __shfl_xor(ss, 32);
    uint32_t w1[2] = {0u, 0u}, w8 = 0u;
    float s2[8];
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const bf16x8 ah = as_bf16x8(Phi[(nt * 4 + kt) * 64]);
        const bf16x8 al = as_bf16x8(Plo[(nt * 4 + kt) * 64]);
        const bf16x8 bh = as_bf16x8(xh[kt]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc, 0, 0, 0);
        if (!XBF16) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, as_bf16x8(xl[kt]), acc, 0, 0, 0);
      }
      float sp[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const float a = acc[2 * i], b = acc[2 * i + 1];
        w1[nt >> 2] |= polar_sector(a, b, t8, t38) << (4 * (2 * (nt & 3) + i));
        sp[i] = fmaf(b, b, a * a);
      }
      w8 |= polar_level_code(sp[0], sp[1], tau[0]) << (2 * nt);
      s2[nt] = sp[0] + sp[1];
      // one tile's fragments in flight at a time (no hoisting of all 64 reads)
      __builtin_amdgcn_sched_barrier(0);
    }
    // level 3: node (nt, g / 2) pairs lane groups 2h, 2h + 1; kept by g = 2h
    // level 4: node nt pairs h = 0 (g < 2) and h = 1; kept by g = 1
    uint32_t hi3 = 0u, hi4 = 0u;
    float s4[8];
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const float o = __shfl_xor(s2[nt], 16);
      const float sl = (g & 1) ? o : s2[nt], sr = (g & 1) ? s2[nt] : o;
      hi3 |= polar_level_code(sl, sr, tau[1]) << (2 * nt);
      const float s3 = sl + sr;
      const float o3 = __shfl_xor(s3, 32);
      const float tl = (g & 2) ? o3 : s3, tr = (g & 2) ? s3 : o3;
      hi4 |= polar_level_code(tl, tr, tau[2]) << (2 * nt);
      s4[nt] = tl + tr;
    }
    // levels 5..7 inside the lane; kept by g = 3
    uint32_t hi5 = 0u;
    float s5[4], s6[2];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      hi5 |= polar_level_code(s4[2 * j], s4[2 * j + 1], tau[3]) << (2 * j);
      s5[j] = s4[2 * j] + s4[2 * j + 1];
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      hi5 |= polar_level_code(s5[2 * j], s5[2 * j + 1], tau[4]) << (8 + 2 * j);
      s6[j] = s5[2 * j] + s5[2 * j + 1];
    }
    hi5 |= polar_level_code(s6[0], s6[1], tau[5]) << 12;
    const uint32_t hi = g == 0 ? hi3 : (g == 1 ? hi4 : (g == 2 ? hi3 : hi5));
    w8 |= hi << 16;
    if (valid) {
      uint32_t *dst = pq + row * 12;
      *reinterpret_cast<uint2 *>(dst + 2 * g) = make_uint2(w1[0], w1[1]);
      dst[8 + g] = w8;
      if (g == 0) radius[row] = sqrtf(ss);
    }
  }
}

// Score: one key per thread and the (up to) 4 query heads of a group.  The
// tree is folded bottom-up: a level-1 node gives c q_2j + s q_2j+1 per query
// (looked up from a table of all 16 codes of every node, built per workgroup),
// a node above gives c f_left + s f_right, and the root times the radius is
// the logit <Pi q, y^>.  The rotated queries come from qproj_kernel (float64
// sums).
constexpr int kPolScoreThreads = 256;
constexpr int kPolKPT = 8;  // keys per thread
__global__ __launch_bounds__(kPolScoreThreads) void polar_score128_kernel(
    const double *__restrict__ qt, const uint32_t *__restrict__ pq, const float *__restrict__ radius,
    int64_t seq, int64_t g, int ngroups, const PolarTables *__restrict__ T, float *__restrict__ logits) {
  __shared__ float4 qs[128];
  __shared__ float4 L1[64][16];  // level-1 node j, code k: c_k q_2j + s_k q_2j+1 for the 4 queries
  __shared__ float2 tl[6][4];
  const int hg = blockIdx.y, h = hg / ngroups, grp = hg % ngroups;
  const int tid = threadIdx.x;
  if (tid < 128) {
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t qh = (int64_t)grp * 4 + j;
      v[j] = qh < g ? (float)qt[((int64_t)h * g + qh) * 128 + tid] : 0.f;
    }
    qs[tid] = make_float4(v[0], v[1], v[2], v[3]);
  }
  if (tid < 24) tl[tid / 4][tid % 4] = make_float2(T->cl[tid / 4][tid % 4], T->sl[tid / 4][tid % 4]);
  __syncthreads();
  // the level-1 products of every (node, code): 64 x 16 entries, a gather per
  // node below (16 entries of 16 bytes cover the 64 banks once: no conflicts)
  for (int e = tid; e < 64 * 16; e += kPolScoreThreads) {
    const int j = e >> 4, k = e & 15;
    const float c = T->c1[k], sn = T->s1[k];
    const float4 qa = qs[2 * j], qb = qs[2 * j + 1];
    L1[j][k] = make_float4(fmaf(c, qa.x, sn * qb.x), fmaf(c, qa.y, sn * qb.y), fmaf(c, qa.z, sn * qb.z),
                           fmaf(c, qa.w, sn * qb.w));
  }
  __syncthreads();
  // kPolKPT keys per thread amortise the level-1 table
#pragma unroll 1
  for (int kr = 0; kr < kPolKPT; ++kr) {
  const int64_t pos = ((int64_t)blockIdx.x * kPolKPT + kr) * kPolScoreThreads + tid;
  if (pos >= seq) break;  // no barrier follows
  const int64_t v = (int64_t)h * seq + pos;
  const u32x4 u0 = nt_load4(pq + v * 12), u1 = nt_load4(pq + v * 12 + 4), u2 = nt_load4(pq + v * 12 + 8);
  const uint32_t wd[12] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w, u2.x, u2.y, u2.z, u2.w};
  const float R = nt_load(&radius[v]);
  // Blocks of 32 coordinates (t2) one loop iteration at a time, so that the
  // query and table reads of one block are not all hoisted and held together;
  // the level-5 and level-6 left siblings wait in p5, p6.
  float p5[4] = {0.f, 0.f, 0.f, 0.f}, p6[4] = {0.f, 0.f, 0.f, 0.f}, f7[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
  for (int t2 = 0; t2 < 4; ++t2) {
    float f4[2][4];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int t = 2 * t2 + tt;
      float f3[2][4];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        float f2[2][4];
#pragma unroll
        for (int gg = 0; gg < 2; ++gg) {
          const int gl = 2 * hh + gg;
          const uint32_t w1 = t2 >= 2 ? wd[2 * gl + 1] : wd[2 * gl];
          float f1[2][4];
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const uint32_t code = (w1 >> (4 * (2 * (t & 3) + i))) & 15u;
            const float4 l1 = L1[8 * t + 2 * gl + i][code];
            f1[i][0] = l1.x;
            f1[i][1] = l1.y;
            f1[i][2] = l1.z;
            f1[i][3] = l1.w;
          }
          const float2 c2 = tl[0][(wd[8 + gl] >> (2 * t)) & 3u];
#pragma unroll
          for (int j = 0; j < 4; ++j) f2[gg][j] = fmaf(c2.x, f1[0][j], c2.y * f1[1][j]);
        }
        const float2 c3 = tl[1][(wd[8 + 2 * hh] >> (16 + 2 * t)) & 3u];
#pragma unroll
        for (int j = 0; j < 4; ++j) f3[hh][j] = fmaf(c3.x, f2[0][j], c3.y * f2[1][j]);
      }
      const float2 c4 = tl[2][(wd[9] >> (16 + 2 * t)) & 3u];
#pragma unroll
      for (int j = 0; j < 4; ++j) f4[tt][j] = fmaf(c4.x, f3[0][j], c4.y * f3[1][j]);
    }
    float f5[4];
    const float2 c5 = tl[3][(wd[11] >> (16 + 2 * t2)) & 3u];
#pragma unroll
    for (int j = 0; j < 4; ++j) f5[j] = fmaf(c5.x, f4[0][j], c5.y * f4[1][j]);
    if (t2 & 1) {
      float f6[4];
      const float2 c6 = tl[4][(wd[11] >> (24 + (t2 & 2))) & 3u];
#pragma unroll
      for (int j = 0; j < 4; ++j) f6[j] = fmaf(c6.x, p5[j], c6.y * f5[j]);
      if (t2 == 3) {
        const float2 c7 = tl[5][(wd[11] >> 28) & 3u];
#pragma unroll
        for (int j = 0; j < 4; ++j) f7[j] = fmaf(c7.x, p6[j], c7.y * f6[j]);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) p6[j] = f6[j];
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) p5[j] = f5[j];
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t qh = (int64_t)grp * 4 + j;
    if (qh < g) nt_store(&logits[((int64_t)h * g + qh) * seq + pos], R * f7[j]);
  }
  }  // keys of this thread
}

tq_status launch_polar_encode(const Derived &D, const PolarTables *T, const void *x, int dtype,
                              int64_t n, tq_polar_codes c, hipStream_t s) {
  const int64_t nbatch = (n + 15) / 16;
  const int64_t need = (nbatch + kPolWaves - 1) / kPolWaves;
  // 64 KB of fragments per workgroup: two workgroups per CU
  const int grid = (int)std::min<int64_t>(need, (int64_t)num_cus(D.device) * 2);
  const uint4 *ph = reinterpret_cast<const uint4 *>(D.pi_hi), *pl = reinterpret_cast<const uint4 *>(D.pi_lo);
  if (dtype == TQ_BF16)
    polar_encode128_kernel<true><<<grid, kPolWaves * 64, 0, s>>>(x, n, ph, pl, T, c.pq, c.radius);
  else
    polar_encode128_kernel<false><<<grid, kPolWaves * 64, 0, s>>>(x, n, ph, pl, T, c.pq, c.radius);
  TQ_LAUNCH_CHECK();
  return TQ_OK;
}

size_t polar_score_workspace_bytes(int64_t nq) { return (size_t)nq * 128 * sizeof(double); }

tq_status launch_polar_score(const Derived &D, const PolarTables *T, const float *q, int64_t n_kv,
                             int64_t g, tq_polar_codes c, int64_t seq, float *logits, void *ws,
                             hipStream_t s) {
  const int ngroups = (int)((g + 3) / 4);
  const int64_t nhg = n_kv * ngroups;
  const int64_t nblk = (seq + kPolKPT * kPolScoreThreads - 1) / (kPolKPT * kPolScoreThreads);
  if (nhg > 65535 || nblk > 0x7fffffffLL || n_kv * g > 0x7fffffffLL) {
    set_error("tq_polar_score: problem too large for one launch");
    return TQ_ERR_UNSUPPORTED;
  }
  if ((n_kv * g + kQJQ - 1) / kQJQ > 65535) {
    set_error("tq_polar_score: too many queries for one launch");
    return TQ_ERR_UNSUPPORTED;
  }
  double *qt = (double *)ws;
  qproj_kernel<<<dim3(128 / kQJR, (unsigned)((n_kv * g + kQJQ - 1) / kQJQ)), dim3(256), 0, s>>>(
      q, n_kv * g, 128, 128, D.pi32, nullptr, qt);
  polar_score128_kernel<<<dim3((unsigned)nblk, (unsigned)nhg), kPolScoreThreads, 0, s>>>(
      qt, c.pq, c.radius, seq, g, ngroups, T, logits);
  TQ_LAUNCH_CHECK();
  return TQ_OK;
}

// ===========================================================================
// Mixed bit widths: two TurboQuant groups of one head, d = 128: the DG0
// outlier channels and the other DG1 = 128 - DG0 (DG0 = 32, 64 or 96)
// ===========================================================================
// Encode: one wave per 16 vectors, the two channel groups in turn, as bf16
// hi / lo MFMAs like the d = 128 encoder: Y_g = Pi_g X_g with X_g the keys'
// channels of group g gathered into the B operand (lane (v, k) holds the
// group's channels 32 kt + 8 k .. + 7 of vector v), so lane (v, k) receives
// rotated coordinates 16 t + 4 k + i (t < DG / 16); bucketisation and the
// residual stay in registers, Z_g = S'_g rho_g reads the residual in that
// layout (S'_g's columns are arranged for it), and each lane holds the
// DG / 4 bits of its coordinates (16 t + 4 k + i at bit 4 t + i), which lane
// group 0 gathers into the plane's words (the field of lane group k starts at
// bit k DG / 4 of the plane).
constexpr int kSplitWaves = 16;
constexpr int kSplitRowB = 272;  // LDS bytes per staged bfloat16 row (256 + 16)

__host__ __device__ constexpr int split_frag_u4(int DG) { return (DG / 16) * (DG / 32) * 64; }

// The words of a plane from the four lane groups' fields of FB bits each
// (field k at bit k FB of the plane's bit string).
template <int FB, int NW>
__device__ __forceinline__ void pack_fields(const uint32_t (&f)[4], uint32_t (&w)[NW]) {
#pragma unroll
  for (int j = 0; j < NW; ++j) w[j] = 0u;
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int j = 0; j < NW; ++j) {
      const int pos = k * FB, lo = 32 * j;
      if (pos + FB <= lo || pos >= lo + 32) continue;
      if (pos >= lo)
        w[j] |= f[k] << (pos - lo);
      else
        w[j] |= f[k] >> (lo - pos);
    }
}

// One channel group g of dimension DG with B Lloyd-Max bits for the wave's 16
// vectors.  Fg: the group's fragments (Pi hi, Pi lo, S' hi, S' lo); goff: the
// group's first entry in the channel order; off: its first word.
template <bool XBF16, int B, int DG>
__device__ __forceinline__ void split_encode_group(
    const int g, const int goff, const void *__restrict__ x, const uint16_t *xrow, const int64_t rr,
    const int64_t row, const bool valid, const int lane, const int kg, const uint4 *Fg, const int *chs,
    const float (*cbc)[8], const float (*cbt)[8], const int off, const int W,
    uint32_t *__restrict__ words, float *__restrict__ norms) {
  constexpr int NT = DG / 16, NK = DG / 32, NW = DG / 32, FB = DG / 4;
  constexpr int FH = split_frag_u4(DG);
  constexpr int nbnd = (1 << B) - 1;
  const uint4 *Ph = Fg + lane, *Pl = Fg + FH + lane;
  const uint4 *Sh = Fg + 2 * FH + lane, *Sl = Fg + 3 * FH + lane;
  // B operand: the group's channels 32 kt + 8 kg + e of vector rr
  uint4 xh[NK], xl[NK];
  float ss = 0.f;
#pragma unroll
  for (int kt = 0; kt < NK; ++kt) {
    if (XBF16) {  // bfloat16 channels are the operand as they are: pairs packed, squares by v_dot2
      typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
      uint32_t h[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c0 = chs[goff + 32 * kt + 8 * kg + 2 * i], c1 = chs[goff + 32 * kt + 8 * kg + 2 * i + 1];
        h[i] = (uint32_t)xrow[c0] | (uint32_t)xrow[c1] << 16;
        const bf16x2 hv = __builtin_bit_cast(bf16x2, h[i]);
        ss = __builtin_amdgcn_fdot2_f32_bf16(hv, hv, ss, false);
      }
      xh[kt] = make_uint4(h[0], h[1], h[2], h[3]);
      xl[kt] = xh[kt];
    } else {
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int c = chs[goff + 32 * kt + 8 * kg + e];
        v[e] = reinterpret_cast<const float *>(x)[rr * 128 + c];
        ss = fmaf(v[e], v[e], ss);
      }
      uint32_t h[4], l[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) split2(v[2 * i], v[2 * i + 1], h[i], l[i]);
      xh[kt] = make_uint4(h[0], h[1], h[2], h[3]);
      xl[kt] = make_uint4(l[0], l[1], l[2], l[3]);
    }
  }
  ss += __shfl_xor(ss, 16);
  ss += __shfl_xor(ss, 32);
  const float nu = sqrtf(ss);
  f32x4 acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kt = 0; kt < NK; ++kt) {
      const bf16x8 ah = as_bf16x8(Ph[(nt * NK + kt) * 64]), al = as_bf16x8(Pl[(nt * NK + kt) * 64]);
      const bf16x8 bh = as_bf16x8(xh[kt]);
      acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc[nt], 0, 0, 0);
      acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc[nt], 0, 0, 0);
      if (!XBF16) acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, as_bf16x8(xl[kt]), acc[nt], 0, 0, 0);
    }
  }
  // buckets (decided on y against the boundaries scaled by ||x_g||; a zero
  // vector compares 0 with the unscaled ones), index bits, residual
  // y - c ||x_g|| with one rounding
  float tb[nbnd], cv[nbnd + 1];
#pragma unroll
  for (int j = 0; j < nbnd; ++j) tb[j] = nu > 0.f ? cbt[g][j] * nu : cbt[g][j];
#pragma unroll
  for (int j = 0; j <= nbnd; ++j) cv[j] = cbc[g][j];
  // The compares form a thermometer code g_0 >= g_1 >= ... (the boundaries
  // ascend), so bit p of the index k = #{j : g_j} is the parity of
  // #{m >= 1 : k >= m 2^p}, i.e. the XOR of g_{m 2^p - 1}: one XOR of compare
  // masks and one v_addc per plane bit, shifted in from the highest
  // coordinate down so that coordinate 4 nt + i lands at bit 4 nt + i.
  uint32_t pf[B + 1];
#pragma unroll
  for (int p = 0; p <= B; ++p) pf[p] = 0u;
  float rho[NT][4], rsq = 0.f;
#pragma unroll
  for (int nt = NT - 1; nt >= 0; --nt)
#pragma unroll
    for (int i = 3; i >= 0; --i) {
      const float y = acc[nt][i];
      uint64_t gm[nbnd];
      float cm = cv[0];
#pragma unroll
      for (int j = 0; j < nbnd; ++j) {
        const bool ge = y >= tb[j];
        gm[j] = __builtin_amdgcn_ballot_w64(ge);
        cm = ge ? cv[j + 1] : cm;
      }
#pragma unroll
      for (int p = 0; p < B; ++p) {
        uint64_t mk = 0;
#pragma unroll
        for (int mm = 1; mm * (1 << p) <= nbnd; ++mm) mk ^= gm[mm * (1 << p) - 1];
        pf[p] = shift_in(pf[p], mk);
      }
      const float r = fmaf(-cm, nu, y);
      rsq = fmaf(r, r, rsq);
      rho[nt][i] = r;
    }
  rsq += __shfl_xor(rsq, 16);
  rsq += __shfl_xor(rsq, 32);
  // Z = S' rho: K block kt element e of lane group kg = coordinate 32 kt + 16 (e / 4) + 4 kg + e % 4
  uint4 rh[NK], rl[NK];
#pragma unroll
  for (int kt = 0; kt < NK; ++kt) {
    uint32_t h[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e0 = 2 * i, e1 = 2 * i + 1;
      split2(rho[2 * kt + e0 / 4][e0 % 4], rho[2 * kt + e1 / 4][e1 % 4], h[i], l[i]);
    }
    rh[kt] = make_uint4(h[0], h[1], h[2], h[3]);
    rl[kt] = make_uint4(l[0], l[1], l[2], l[3]);
  }
  // sign bits from the highest row down, one v_alignbit each (the float's
  // sign bit shifted in; an exactly zero z comes out of the accumulation as
  // +0), complemented once within the field
#pragma unroll
  for (int nt = NT - 1; nt >= 0; --nt) {
    f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kt = 0; kt < NK; ++kt) {
      const bf16x8 ah = as_bf16x8(Sh[(nt * NK + kt) * 64]), al = as_bf16x8(Sl[(nt * NK + kt) * 64]);
      z = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, as_bf16x8(rh[kt]), z, 0, 0, 0);
      z = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, as_bf16x8(rl[kt]), z, 0, 0, 0);
      z = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, as_bf16x8(rh[kt]), z, 0, 0, 0);
    }
#pragma unroll
    for (int i = 3; i >= 0; --i) pf[B] = __builtin_amdgcn_alignbit(pf[B], __float_as_uint(z[i]), 31);
  }
  pf[B] = ~pf[B] & (4 * NT >= 32 ? 0xFFFFFFFFu : (1u << (4 * NT)) - 1u);
  // lane group 0 gathers the four fields of each plane (index planes, then
  // the sign plane) and writes the plane's words
  const int kc = lane & 15;
  uint32_t *dst = words + rr * W + off;
#pragma unroll
  for (int p = 0; p <= B; ++p) {
    uint32_t f[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) f[k] = __shfl(pf[p], kc + 16 * k);
    uint32_t wd[NW];
    pack_fields<FB, NW>(f, wd);
    if (valid && kg == 0) {
#pragma unroll
      for (int j = 0; j < NW; ++j) dst[p * NW + j] = wd[j];
    }
  }
  if (valid && kg == 0) {
    norms[row * 4 + 2 * g] = nu;
    norms[row * 4 + 2 * g + 1] = sqrtf(rsq);
  }
}

template <bool XBF16, int B0, int B1, int DG0>
__global__ __launch_bounds__(kSplitWaves * 64) void split_encode128_kernel(
    const void *__restrict__ x, int64_t n, const uint4 *__restrict__ frag, const float *__restrict__ cbk,
    const int32_t *__restrict__ chan, uint32_t *__restrict__ words, float *__restrict__ norms) {
  constexpr int DG1 = 128 - DG0;
  constexpr int FU0 = 4 * split_frag_u4(DG0), FU1 = 4 * split_frag_u4(DG1);
  constexpr int W = (B0 + 1) * (DG0 / 32) + (B1 + 1) * (DG1 / 32);
  __shared__ uint4 F[FU0 + FU1];  // group 0: Pi hi, lo, S' hi, lo; then group 1
  // bfloat16 keys: each wave's 16 rows, loaded whole (coalesced) and gathered
  // from here; rows padded to 272 bytes to spread the gathers over the banks
  __shared__ __attribute__((aligned(16))) unsigned char xs[XBF16 ? kSplitWaves : 1][16 * kSplitRowB];
  __shared__ int chs[128];
  __shared__ float cbc[2][8], cbt[2][8];
  for (int i = threadIdx.x; i < FU0 + FU1; i += blockDim.x) F[i] = frag[i];
  if (threadIdx.x < 128) chs[threadIdx.x] = chan[threadIdx.x];
  if (threadIdx.x < 32) {
    const int t = threadIdx.x;
    const float v = cbk[t];
    if (t < 16) cbc[t >> 3][t & 7] = v;
    else cbt[(t - 16) >> 3][(t - 16) & 7] = v;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int vcol = lane & 15, kg = lane >> 4;
  const int64_t nbatch = (n + 15) / 16;
  for (int64_t batch = (int64_t)blockIdx.x * kSplitWaves + wave; batch < nbatch;
       batch += (int64_t)gridDim.x * kSplitWaves) {
    const int64_t row = batch * 16 + vcol;
    const bool valid = row < n;
    const int64_t rr = valid ? row : n - 1;  // loads stay in bounds; results of rr != row are not stored
    const uint16_t *xrow = nullptr;
    if constexpr (XBF16) {
      // rows batch * 16 + r (clamped to n - 1, as rr is), 16 uint4 each; the
      // previous batch's gathers are done before the rows are overwritten
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
      const uint4 *src = reinterpret_cast<const uint4 *>(x);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int q = lane + 64 * i, r = q >> 4, c4 = q & 15;
        const int64_t gr = batch * 16 + r < n ? batch * 16 + r : n - 1;
        *reinterpret_cast<uint4 *>(&xs[wave][r * kSplitRowB + 16 * c4]) = src[gr * 16 + c4];
      }
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
      xrow = reinterpret_cast<const uint16_t *>(&xs[wave][vcol * kSplitRowB]);
    }
    split_encode_group<XBF16, B0, DG0>(0, 0, x, xrow, rr, row, valid, lane, kg, F, chs, cbc, cbt, 0, W,
                                       words, norms);
    __builtin_amdgcn_sched_barrier(0);
    split_encode_group<XBF16, B1, DG1>(1, DG0, x, xrow, rr, row, valid, lane, kg, F + FU0, chs, cbc, cbt,
                                       (B0 + 1) * (DG0 / 32), W, words, norms);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Score: one key per thread, the (up to) 4 query heads of a group.  Per
// workgroup, tables over chunks of coordinates: for a chunk of S coordinates
// of group g (S = 2, or 4 for 1-bit groups) and each combination `code` of
// their index bits, the sum of c_g[idx] (Pi_g q)_c over the chunk; for a
// chunk of 4 sign bits, the sum of (S_g q)_c over the set bits (the estimator
// takes 2 sum - total).  A key then costs one gather and four adds per chunk.
// The projections come from qproj_kernel (float64 sums).
constexpr int kSplitScoreThreads = 256;
constexpr int kSplitKPT = 16;  // keys per thread (the tables amortised over 4096 keys)

__host__ __device__ constexpr int split_chunk(int B) { return B >= 2 ? 2 : 4; }

template <int B0, int B1, int DG0>
__global__ __launch_bounds__(kSplitScoreThreads) void split_score128_kernel(
    const double *__restrict__ pq, const float *__restrict__ cbk, const uint32_t *__restrict__ words,
    const float *__restrict__ norms, int64_t seq, int64_t g, int ngroups, float kq0, float kq1,
    float *__restrict__ logits) {
  constexpr int DG1 = 128 - DG0;
  constexpr int W = (B0 + 1) * (DG0 / 32) + (B1 + 1) * (DG1 / 32);
  constexpr int S0 = split_chunk(B0), S1 = split_chunk(B1);
  constexpr int C0 = 1 << (B0 * S0), C1 = 1 << (B1 * S1);  // codes per chunk
  constexpr int N0 = DG0 / S0, N1 = DG1 / S1;               // chunks per group
  __shared__ float4 qs4[256];  // (Pi q)_c for c < 128 (group 0, then group 1), then (S q)_c
  __shared__ float4 TI0[N0 * C0], TI1[N1 * C1];
  __shared__ float4 TS0[DG0 / 4][16], TS1[DG1 / 4][16];  // sign chunk, code
  __shared__ float4 SS[2];
  const int hg = blockIdx.y, h = hg / ngroups, grp = hg % ngroups;
  const int tid = threadIdx.x;
  {
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t qh = (int64_t)grp * 4 + j;
      v[j] = qh < g ? (float)pq[((int64_t)h * g + qh) * 256 + tid] : 0.f;
    }
    qs4[tid] = make_float4(v[0], v[1], v[2], v[3]);
  }
  __syncthreads();
  for (int e = tid; e < N0 * C0 + N1 * C1; e += kSplitScoreThreads) {
    const bool g1 = e >= N0 * C0;
    const int ee = g1 ? e - N0 * C0 : e;
    const int S = g1 ? S1 : S0, B = g1 ? B1 : B0, C = g1 ? C1 : C0;
    const int chunk = ee / C, code = ee % C;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < S; ++j) {
      int idx = 0;
      for (int p = 0; p < B; ++p) idx |= ((code >> (p * S + j)) & 1) << p;
      const float cent = cbk[(g1 ? 8 : 0) + idx];
      const float4 q = qs4[(g1 ? DG0 : 0) + chunk * S + j];
      a.x = fmaf(cent, q.x, a.x); a.y = fmaf(cent, q.y, a.y); a.z = fmaf(cent, q.z, a.z); a.w = fmaf(cent, q.w, a.w);
    }
    if (g1) TI1[ee] = a;
    else TI0[ee] = a;
  }
  for (int e = tid; e < 32 * 16; e += kSplitScoreThreads) {
    const int chunk = e >> 4, code = e & 15;  // chunk 0 .. 31 over both groups
    const bool g1 = chunk >= DG0 / 4;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < 4; ++j)
      if ((code >> j) & 1) {
        const float4 q = qs4[128 + 4 * chunk + j];
        a.x += q.x; a.y += q.y; a.z += q.z; a.w += q.w;
      }
    if (g1) TS1[chunk - DG0 / 4][code] = a;
    else TS0[chunk][code] = a;
  }
  if (tid < 2) {
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    const int c0 = tid ? 128 + DG0 : 128, c1 = tid ? 256 : 128 + DG0;
    for (int c = c0; c < c1; ++c) {
      a.x += qs4[c].x; a.y += qs4[c].y; a.z += qs4[c].z; a.w += qs4[c].w;
    }
    SS[tid] = a;
  }
  __syncthreads();
  // kSplitKPT keys per thread amortise the tables
#pragma unroll 1
  for (int r = 0; r < kSplitKPT; ++r) {
  const int64_t pos = ((int64_t)blockIdx.x * kSplitKPT + r) * kSplitScoreThreads + tid;
  if (pos >= seq) break;  // no barrier follows
  const int64_t v = (int64_t)h * seq + pos;
  uint32_t wd[W];
#pragma unroll
  for (int i = 0; i < W; ++i) wd[i] = nt_load(&words[v * W + i]);
  const u32x4 nru = nt_load4(reinterpret_cast<const uint32_t *>(norms + v * 4));
  const float4 nr = make_float4(__uint_as_float(nru.x), __uint_as_float(nru.y), __uint_as_float(nru.z),
                                __uint_as_float(nru.w));
  float4 acc[2], accs[2];
#pragma unroll
  for (int gg = 0; gg < 2; ++gg) {
    acc[gg] = make_float4(0.f, 0.f, 0.f, 0.f);
    accs[gg] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  // one group at a time: plane word j holds bits 32 j .. 32 j + 31 of the
  // plane; its 4-bit group at bit 4 bq is coordinate 16 t + 4 k + (0..3)
  // with k = (32 j + 4 bq) / (DG / 4), t = ((32 j + 4 bq) % (DG / 4)) / 4.
  // One word per loop iteration (the gathers of an iteration are not all
  // hoisted together; words picked by wave-uniform selects).
  auto group = [&](auto gc) {
    constexpr int gg = decltype(gc)::value;
    constexpr int B = gg ? B1 : B0, S = gg ? S1 : S0, C = gg ? C1 : C0;
    constexpr int DG = gg ? DG1 : DG0, NW = DG / 32, FB = DG / 4;
    constexpr int off = gg ? (B0 + 1) * (DG0 / 32) : 0;
    const float4 *TI = gg ? TI1 : TI0;
    const float4(*TS)[16] = gg ? TS1 : TS0;
    auto pick = [&](int base, int j) -> uint32_t {  // an OR of masked words, not an indexed load
      uint32_t w = 0u;
#pragma unroll
      for (int jj = 0; jj < NW; ++jj) w |= wd[base + jj] & (j == jj ? 0xFFFFFFFFu : 0u);
      return w;
    };
#pragma unroll 1
    for (int j = 0; j < NW; ++j) {
      uint32_t pl[3];
#pragma unroll
      for (int p = 0; p < 3; ++p) pl[p] = p < B ? pick(off + p * NW, j) : 0u;
      const uint32_t sw = pick(off + B * NW, j);
#pragma unroll
      for (int bq = 0; bq < 8; ++bq) {
        const int pos = 32 * j + 4 * bq;
        const int c0 = 16 * ((pos % FB) / 4) + 4 * (pos / FB);
#pragma unroll
        for (int i0 = 0; i0 < 4; i0 += S) {
          uint32_t code = 0;
#pragma unroll
          for (int p = 0; p < 3; ++p)
            if (p < B) code |= ((pl[p] >> (4 * bq + i0)) & ((1u << S) - 1u)) << (p * S);
          const float4 tv = TI[((c0 + i0) / S) * C + code];
          acc[gg].x += tv.x; acc[gg].y += tv.y; acc[gg].z += tv.z; acc[gg].w += tv.w;
        }
        const float4 tv = TS[c0 / 4][(sw >> (4 * bq)) & 15u];
        accs[gg].x += tv.x; accs[gg].y += tv.y; accs[gg].z += tv.z; accs[gg].w += tv.w;
      }
    }
  };
  group(std::integral_constant<int, 0>{});
  group(std::integral_constant<int, 1>{});
  const float nrm[4] = {nr.x, nr.y, nr.z, nr.w};
  const float a0[4] = {acc[0].x, acc[0].y, acc[0].z, acc[0].w}, a1[4] = {acc[1].x, acc[1].y, acc[1].z, acc[1].w};
  const float s0[4] = {accs[0].x, accs[0].y, accs[0].z, accs[0].w};
  const float s1[4] = {accs[1].x, accs[1].y, accs[1].z, accs[1].w};
  const float t0[4] = {SS[0].x, SS[0].y, SS[0].z, SS[0].w}, t1[4] = {SS[1].x, SS[1].y, SS[1].z, SS[1].w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t qh = (int64_t)grp * 4 + j;
    if (qh < g) {
      const float l = nrm[0] * a0[j] + kq0 * nrm[1] * (2.f * s0[j] - t0[j]) + nrm[2] * a1[j] +
                      kq1 * nrm[3] * (2.f * s1[j] - t1[j]);
      nt_store(&logits[((int64_t)h * g + qh) * seq + pos], l);
    }
  }
  }  // keys of this thread
}

template <int B0, int B1, int DG0>
static void launch_split_encode_t(const SplitDerived &D, const void *x, bool bf, int64_t n, tq_split_codes c,
                                  hipStream_t s) {
  // as many workgroups as fit in the CUs' LDS at once (the fragments, and for
  // bfloat16 keys the staged rows): one per CU for bfloat16 keys, two for
  // float32 keys with 64 outlier channels
  constexpr size_t kLdsPerCU = 160 * 1024;
  const size_t lds = 16 * (size_t)(4 * split_frag_u4(DG0) + 4 * split_frag_u4(128 - DG0)) +
                     (bf ? (size_t)kSplitWaves * 16 * kSplitRowB : 0) + 1024;
  const int64_t per_cu = std::max<int64_t>(1, (int64_t)(kLdsPerCU / lds));
  const int64_t need = ((n + 15) / 16 + kSplitWaves - 1) / kSplitWaves;
  const int grid = (int)std::min<int64_t>(need, (int64_t)num_cus(D.device) * per_cu);
  const uint4 *fr = reinterpret_cast<const uint4 *>(D.frag);
  const float *cbk = D.mat + split_codebook_offset(D.DG);
  if (bf)
    split_encode128_kernel<true, B0, B1, DG0><<<grid, kSplitWaves * 64, 0, s>>>(x, n, fr, cbk, D.chan, c.words,
                                                                                 c.norms);
  else
    split_encode128_kernel<false, B0, B1, DG0><<<grid, kSplitWaves * 64, 0, s>>>(x, n, fr, cbk, D.chan, c.words,
                                                                                  c.norms);
}

template <int B0, int B1>
static tq_status launch_split_encode_b(const SplitDerived &D, const void *x, bool bf, int64_t n,
                                       tq_split_codes c, hipStream_t s) {
  switch (D.DG[0]) {
    case 32: launch_split_encode_t<B0, B1, 32>(D, x, bf, n, c, s); break;
    case 64: launch_split_encode_t<B0, B1, 64>(D, x, bf, n, c, s); break;
    case 96: launch_split_encode_t<B0, B1, 96>(D, x, bf, n, c, s); break;
    default:
      set_error("tq_split_encode: no kernel for %d outlier channels", D.DG[0]);
      return TQ_ERR_UNSUPPORTED;
  }
  return TQ_OK;
}

tq_status launch_split_encode(const SplitDerived &D, const void *x, int dtype, int64_t n,
                              tq_split_codes c, hipStream_t s) {
  const bool bf = dtype == TQ_BF16;
  tq_status st;
  if (D.B[0] == 2 && D.B[1] == 1)
    st = launch_split_encode_b<2, 1>(D, x, bf, n, c, s);
  else if (D.B[0] == 3 && D.B[1] == 2)
    st = launch_split_encode_b<3, 2>(D, x, bf, n, c, s);
  else {
    set_error("tq_split_encode: no kernel for Lloyd-Max bits (%d, %d)", D.B[0], D.B[1]);
    return TQ_ERR_UNSUPPORTED;
  }
  if (st != TQ_OK) return st;
  TQ_LAUNCH_CHECK();
  return TQ_OK;
}

size_t split_score_workspace_bytes(int64_t nq) { return (size_t)nq * 256 * sizeof(double); }

template <int B0, int B1>
static tq_status launch_split_score_b(const SplitDerived &D, const double *pq, tq_split_codes c, int64_t seq,
                                      int64_t g, int ngroups, dim3 grid, float *logits, hipStream_t s) {
  const float *cbk = D.mat + split_codebook_offset(D.DG);
  // the QJL constant sqrt(pi/2)/m of each group (m = its dimension)
  const float kq0 = (float)(std::sqrt(M_PI / 2.0) / D.DG[0]), kq1 = (float)(std::sqrt(M_PI / 2.0) / D.DG[1]);
  switch (D.DG[0]) {
    case 32:
      split_score128_kernel<B0, B1, 32><<<grid, kSplitScoreThreads, 0, s>>>(pq, cbk, c.words, c.norms, seq, g,
                                                                            ngroups, kq0, kq1, logits);
      break;
    case 64:
      split_score128_kernel<B0, B1, 64><<<grid, kSplitScoreThreads, 0, s>>>(pq, cbk, c.words, c.norms, seq, g,
                                                                            ngroups, kq0, kq1, logits);
      break;
    case 96:
      split_score128_kernel<B0, B1, 96><<<grid, kSplitScoreThreads, 0, s>>>(pq, cbk, c.words, c.norms, seq, g,
                                                                            ngroups, kq0, kq1, logits);
      break;
    default:
      set_error("tq_split_score: no kernel for %d outlier channels", D.DG[0]);
      return TQ_ERR_UNSUPPORTED;
  }
  return TQ_OK;
}

tq_status launch_split_score(const SplitDerived &D, const float *q, int64_t n_kv, int64_t g,
                             tq_split_codes c, int64_t seq, float *logits, void *ws, hipStream_t s) {
  const int ngroups = (int)((g + 3) / 4);
  const int64_t nhg = n_kv * ngroups;
  const int64_t nblk = (seq + kSplitKPT * kSplitScoreThreads - 1) / (kSplitKPT * kSplitScoreThreads);
  if (nhg > 65535 || nblk > 0x7fffffffLL || (n_kv * g + kQJQ - 1) / kQJQ > 65535) {
    set_error("tq_split_score: problem too large for one launch");
    return TQ_ERR_UNSUPPORTED;
  }
  double *pq = (double *)ws;
  qproj_kernel<<<dim3(256 / kQJR, (unsigned)((n_kv * g + kQJQ - 1) / kQJQ)), dim3(256), 0, s>>>(
      q, n_kv * g, 128, 256, D.proj, D.proj + 128 * 128, pq);
  const dim3 grid((unsigned)nblk, (unsigned)nhg);
  tq_status st;
  if (D.B[0] == 2 && D.B[1] == 1)
    st = launch_split_score_b<2, 1>(D, pq, c, seq, g, ngroups, grid, logits, s);
  else if (D.B[0] == 3 && D.B[1] == 2)
    st = launch_split_score_b<3, 2>(D, pq, c, seq, g, ngroups, grid, logits, s);
  else {
    set_error("tq_split_score: built for b_rest = 2 or 3");
    return TQ_ERR_UNSUPPORTED;
  }
  if (st != TQ_OK) return st;
  TQ_LAUNCH_CHECK();
  return TQ_OK;
}

}  // namespace tq

