// Internal declarations shared by the host side (tq_host.cpp) and the device
// side (tq_kernels.hip) of libtq.  Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/tq.h"

namespace tq {

constexpr int kMaxLevels = 16;  // 2^B with B <= 4
constexpr int kMaxParts = 8;    // odd subsets of B <= 4 bit planes

// Odd subsets of B bit planes, ordered by size then by mask value: the parts
// of the multilinear expansion of a symmetric codebook.  Shared by the host
// (coefficients) and the kernels (which planes to XOR), so both agree on the
// order; compile-time in the kernels.
__host__ __device__ constexpr int popcount_ct(uint32_t x) {
  int c = 0;
  for (; x; x >>= 1) c += (int)(x & 1u);
  return c;
}
__host__ __device__ constexpr uint32_t part_mask_ct(int B, int sp) {
  int np = 0;
  for (int size = 1; size <= B; size += 2)
    for (uint32_t mask = 1; mask < (1u << B); ++mask)
      if (popcount_ct(mask) == size) {
        if (np == sp) return mask;
        ++np;
      }
  return 0;
}

// Codebook in the form the kernels consume.  Passed by value as a kernel
// argument.
struct Codebook {
  int32_t nbits;                // B
  int32_t nparts;               // number of odd subsets of the B planes
  float c[kMaxLevels];          // fp32 centroids, ascending
  float t[kMaxLevels - 1];      // fp32 boundaries
  uint32_t part_mask[kMaxParts];  // planes XORed into each part
  double coef[kMaxParts];       // c[idx] = sum_S coef_S * prod_{k in S} (2 b_k - 1)
};

// Everything derived from one tq_params on one device.
struct Derived {
  tq_params p;
  int device;
  int B;  // Lloyd-Max bits
  Codebook cb;
  // device buffers
  float *pi32 = nullptr;       // [d][d]   Pi, row-major (y = Pi x)
  float *s32 = nullptr;        // [m][d]   S
  double *pi64 = nullptr;      // the same in float64 (query preparation)
  double *s64 = nullptr;
  uint16_t *pi_hi = nullptr;   // bf16 fragments of Pi (PolarQuant encoder)
  uint16_t *pi_lo = nullptr;
  // fp16 fragments of kEncScale * Pi and kEncScale * S' (S' = S Pi^T) for the
  // d = m = 128 encoder, hi + lo
  uint16_t *pi16_hi = nullptr;
  uint16_t *pi16_lo = nullptr;
  uint16_t *sp16_hi = nullptr;
  uint16_t *sp16_lo = nullptr;
  // query preparation (d = m = 128): the column sums of Pi and S (float
  // [2][128]: sum_c (Pi q)_c = u . q, sum_r (S q)_r = v . q) and the largest
  // row norm of S (|(S q)_r| <= smax ||q||)
  float *qsums = nullptr;
  float smax = 0.f;
  // float32 [128 columns][256 rows]: column c of Pi (rows 0..127) and of S
  // (rows 128..255), for the query preparation's coalesced projections
  float *qmat = nullptr;
  // General shapes (d, m multiples of 128 other than d = m = 128): GEMM
  // fragments [K/32 block kt][16-row tile nt][hi, lo][lane] of uint4 (8 fp16
  // of kEncScale * the matrix).
  uint4 *pi_frag = nullptr;    // Pi,  d x d
  uint4 *sp_frag = nullptr;    // S',  m x d
};

// True when the d = m = 128 kernels serve these parameters.
inline bool is_d128(const tq_params &p) {
  return p.d == 128 && (p.mode == TQ_MODE_MSE || p.m == 128);
}

// Returns the cache entry for (p, current device), building it on first use.
tq_status get_derived(const tq_params *p, const Derived **out);
// The cache entry if it exists already (allocates nothing), else nullptr.
const Derived *find_derived(const tq_params *p);

void set_error(const char *fmt, ...);

// Launchers (tq_kernels.hip).  Shapes are validated by the caller.
size_t encode_workspace_bytes(const tq_params &p, int64_t n);
// slots != nullptr (d = m = 128 only): vector i is stored at slot slots[i]
// of a store of `capacity` vectors; slots outside [0, capacity) are skipped.
tq_status launch_encode(const Derived &D, const void *x, int dtype, int64_t n,
                        tq_codes codes, void *ws, size_t ws_bytes, hipStream_t stream,
                        const int64_t *slots = nullptr, int64_t capacity = 0);
size_t score_workspace_bytes(const tq_params &p, int64_t n_kv, int64_t g);
tq_status launch_score(const Derived &D, const float *q, int64_t n_kv, int64_t g,
                       tq_codes codes, int64_t seq, float *logits, void *ws,
                       hipStream_t stream);
size_t attend_workspace_bytes(const Derived &K, const Derived &V, int64_t batch,
                              int64_t n_kv, int64_t g, int64_t seq);
// block_table == nullptr: the plain layout.  Otherwise a paged store (pages
// of 512 positions) and seq = max_pages * 512.
tq_status launch_attend(const Derived &K, const Derived &V, const float *q,
                        int64_t batch, int64_t n_kv, int64_t g, tq_codes k,
                        tq_codes v, int64_t seq, float scale, float *out,
                        void *ws, hipStream_t stream, const int32_t *block_table = nullptr,
                        int64_t max_pages = 0, int64_t num_pages = 0,
                        const int32_t *seq_lens = nullptr);

// Device address of this device's scratch array (tq_kernels.hip), looked up
// once per device with that device current.
constexpr size_t kNoAllocScratchBytes = TQ_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
tq_status noalloc_scratch(void **ptr);

tq_status launch_decode(const Derived &D, tq_codes codes, int64_t n, float *out,
                        hipStream_t stream);
size_t search_workspace_bytes(const tq_params &p, int64_t nq, int64_t n, int k);
tq_status launch_search(const Derived &D, const float *q, int64_t nq, tq_codes codes, int64_t n,
                        int k, int64_t *out_idx, float *out_val, void *ws, hipStream_t stream);

// PolarQuant constants for d = 128 (level-1 bits 4, later levels 2 bits), in
// the form the kernels consume (one device copy per GPU).
struct PolarTables {
  float c1[16], s1[16];      // cos, sin of the level-1 centroid angles
  float cl[6][4], sl[6][4];  // cos, sin of the level-(2 + i) centroid angles
  float dc1[3], ds1[3];      // cos, sin of the level-1 boundaries pi/8, pi/4, 3 pi/8 within a quadrant
  float dC[6][3], dS[6][3];  // cos^2, sin^2 of the level-(2 + i) boundaries
  // The encoder's decision constants: tan(pi/8), tan(3 pi/8) for level 1, and
  // tan^2 of the lowest boundary of each level >= 2 (the codebooks are
  // symmetric about pi/4, so the highest boundary is its complement and the
  // middle one is pi/4 itself).
  float tau1[2];
  float tau[6];
};
tq_status launch_polar_encode(const Derived &D, const PolarTables *T, const void *x, int dtype,
                              int64_t n, tq_polar_codes codes, hipStream_t stream);
size_t polar_score_workspace_bytes(int64_t nq);
tq_status launch_polar_score(const Derived &D, const PolarTables *T, const float *q, int64_t n_kv,
                             int64_t g, tq_polar_codes codes, int64_t seq, float *logits, void *ws,
                             hipStream_t stream);

// Mixed bit widths (two 64-channel groups), d = 128: device buffers of one
// tq_split_params on one device.
struct SplitDerived {
  int device;
  int B[2];             // Lloyd-Max bits of the groups
  int DG[2];            // group dimensions: n_out, 128 - n_out
  // fp32: Pi_0 [DG0][DG0], S'_0 = S_0 Pi_0^T, Pi_1 [DG1][DG1], S'_1; then,
  // at split_codebook_offset(), the codebooks: centroids [2][8], boundaries
  // [2][8] (ascending, unused entries 0)
  float *mat = nullptr;
  // fp32 [256][128]: rows 0..127 the rotations of group 0 then group 1, rows
  // 128..255 their JL matrices, on the original channels (the query
  // projections)
  float *proj = nullptr;
  int32_t *chan = nullptr;  // [128] channel order
  // bf16 MFMA fragments, per group Pi hi, Pi lo, S' hi, S' lo, each uint4
  // [DG/16 row tiles][DG/32 column blocks][64 lanes] (see build_split)
  uint16_t *frag = nullptr;
};
inline size_t split_codebook_offset(const int DG[2]) {
  return 2 * ((size_t)DG[0] * DG[0] + (size_t)DG[1] * DG[1]);
}
tq_status launch_split_encode(const SplitDerived &D, const void *x, int dtype, int64_t n,
                              tq_split_codes codes, hipStream_t stream);
size_t split_score_workspace_bytes(int64_t nq);
tq_status launch_split_score(const SplitDerived &D, const float *q, int64_t n_kv, int64_t g,
                             tq_split_codes codes, int64_t seq, float *logits, void *ws,
                             hipStream_t stream);

// The encoders' fp16 matrix fragments hold kEncScale times the matrix (Pi,
// S'), which keeps the lo parts of small entries out of the fp16 subnormals;
// the kernels scale every input vector by a power of two so that its norm is
// in [1, 2).  Both factors are powers of two, so they leave every decision
// unchanged and come back out exactly.
constexpr double kEncScale = 16.0;
constexpr int kEncScaleLog2 = 4;

// Fragment geometry of the d = m = 128 encode kernel: a 128 x 128 matrix is
// stored as [16-row tile nt][32-column block kt][lane][8] bf16 values; lane l
// covers row 16 nt + l % 16 and lane group l / 16.
constexpr int kFragElems = 128 * 128;

}  // namespace tq
