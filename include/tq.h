/*
 * tq.h -- C ABI of the MI355X (gfx950) TurboQuant hot path.
 *
 * The method (cited by page title and section):
 *   [P5] "谷歌TurboQuant如何绕过内存墙？重新审视它的技术突破", section
 *        "2.TurboQuant到底做了什么？": 第一阶段 (random rotation, then an
 *        MSE-optimal Lloyd-Max scalar quantiser for the known Beta-shaped law
 *        of a rotated coordinate, no per-block scale or zero point) and
 *        第二阶段 (b-1 MSE bits plus a 1-bit QJL transform of the residual,
 *        which makes the inner-product estimate unbiased).
 *   [P3] "TurboQuant 与 AI 效率革命：当旧数学遇到新智能", section 三
 *        (非对称估计器: sqrt(pi/2)/m * ||k|| * <S q, sign(S k)>; 零开销的秘密:
 *        m sign bits plus one 32-bit norm) and section 四 (三段论: rotation P,
 *        JL projection S in R^{m x d}, sign(S * residual)).
 *
 * Conventions for every entry point:
 *   - Return value is a tq_status; TQ_OK (0) on success.  Nothing throws
 *     across the ABI.  tq_last_error() gives a human-readable reason for the
 *     last failure on the calling thread.
 *   - Device pointers are caller-owned HIP device memory on the current
 *     device; host pointers are ordinary host memory.  Each argument below
 *     says which.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Device entry points only enqueue kernels on it and return; asynchronous
 *     faults surface at the caller's next synchronisation.
 *   - The library allocates device memory only for its per-(parameters,
 *     device) cache of the rotation, the JL matrix and the codebook (and, for
 *     the PolarQuant calls, one small table per device), built on the first
 *     call that needs them and freed by tq_release_cache().  The hot-path
 *     calls allocate nothing and record no memset (they can be captured in a
 *     HIP graph); scratch comes in through `workspace` (tq_attend_noalloc
 *     uses the library's own device array instead, see there).
 *   - Sizes: d and m must be multiples of 128 in [128, 1024].  tq_encode,
 *     tq_score and tq_search take every such shape; tq_attend, tq_decode,
 *     tq_encode_slots and tq_attend_paged are built for d == 128 (and
 *     m == 128 for prod-mode keys) and return TQ_ERR_UNSUPPORTED otherwise.  b in [1, 5] (prod) or [1, 4] (mse) with
 *     the number of Lloyd-Max bits B <= 4.  n == 0 (or seq == 0) is a no-op.
 *   - Device pointers must be 16-byte aligned (TQ_ERR_ALIGNMENT otherwise).
 *   - Inputs must be finite (precondition, not checked).
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TQ_LAYOUT_VERSION 1

typedef enum {
  TQ_OK = 0,
  TQ_ERR_INVALID_ARG = 1,  /* null pointer, negative size, bad enum        */
  TQ_ERR_UNSUPPORTED = 2,  /* valid for the method, not built for (d, m, b) */
  TQ_ERR_ALIGNMENT = 3,    /* device pointer not 16-byte aligned            */
  TQ_ERR_HIP = 4,          /* HIP runtime error or no usable device         */
  TQ_ERR_NO_MEMORY = 5,    /* cache allocation failed / workspace too small */
} tq_status;

/* prod: B = b-1 Lloyd-Max bits + m QJL sign bits (unbiased inner products);
 * mse : B = b Lloyd-Max bits only (reconstruction, used for values).       */
typedef enum { TQ_MODE_PROD = 0, TQ_MODE_MSE = 1 } tq_mode;

typedef enum { TQ_F32 = 0, TQ_BF16 = 1 } tq_dtype;

/* The problem statement: dimension d, total bits per coordinate b, number of
 * JL rows m, mode, and the seeds of the rotation Pi and of S.  Pi is the Q
 * factor (with positive diag(R)) of a d x d Gaussian drawn from seed_pi; S is
 * an m x d N(0,1) matrix drawn from seed_s.  Both Gaussians come from
 * SplitMix64 words: word k = mix(seed + (k+1) * 0x9E3779B97F4A7C15);
 * element (i, j) of an R x C matrix is counter c = i*C + j; counter pair
 * p = c/2 takes u1 = (w_2p >> 11 + 1) 2^-53 and u2 = (w_2p+1 >> 11) 2^-53,
 * even c -> sqrt(-2 ln u1) cos(2 pi u2), odd c -> the sine branch.        */
typedef struct {
  int32_t d;
  int32_t b;
  int32_t m;
  int32_t mode;     /* tq_mode */
  uint64_t seed_pi;
  uint64_t seed_s;
} tq_params;

/* Packed codes of n vectors, structure of arrays, all device memory owned by
 * the caller (sizes from tq_codes_bytes):
 *   idx   uint32 [n][d/32][B]  word w of plane j holds bit j of the indices
 *                              of 32 coordinates: coordinate
 *                              c = 128 q + 16 t + 4 k + i (t<8, k<4, i<4)
 *                              sits in word 4 q + k at bit 4 t + i.
 *                              NULL when B == 0.
 *   sgn   uint32 [n][m/32]     QJL sign bits, same word/bit map over the m
 *                              rows; bit set <=> (S r)_row >= 0.  prod only.
 *   knorm float  [n]           ||x||
 *   rnorm float  [n]           ||r||, r = x - ||x|| Pi^T c[idx].  prod only.
 * Vector v of a KV cache with n_kv heads and seq positions is
 * (batch * n_kv + head) * seq + pos.                                      */
typedef struct {
  uint32_t *idx;
  uint32_t *sgn;
  float *knorm;
  float *rnorm;
} tq_codes;

const char *tq_status_string(tq_status s);
const char *tq_last_error(void);
int32_t tq_layout_version(void);

/* Lloyd-Max codebook for the law of one coordinate of a randomly rotated
 * unit vector in R^d, density proportional to (1-x^2)^((d-3)/2) on [-1, 1]
 * ([P5] 第一阶段: the law is known, so the codebook is computed once).
 * Host only, pure.  centroids: host float[2^B] ascending; boundaries: host
 * float[2^B - 1], boundaries[j] = fp32((c_j + c_{j+1}) / 2) with the middle
 * one exactly 0.  B = b-1 (prod) or b (mse); B == 0 writes nothing.  d >= 3. */
tq_status tq_make_codebook(int32_t d, int32_t b, int32_t mode, float *centroids,
                           float *boundaries);

/* Byte sizes of the four code arrays for n vectors: out[0] idx, out[1] sgn,
 * out[2] knorm, out[3] rnorm (0 for an absent array).  Host only.          */
tq_status tq_codes_bytes(const tq_params *p, int64_t n, size_t out[4]);

/* The seeded matrices in float64-accurate form rounded to float32, for tests:
 * pi: host float[d*d] row-major (y = Pi x), s: host float[m*d] row-major.
 * Either pointer may be NULL.  Host only.                                  */
tq_status tq_export_matrices(const tq_params *p, float *pi, float *s);

/* Workspace bytes tq_encode needs for n vectors: 0 in mse mode and for
 * d == m == 128; otherwise it holds the residual of up to 32768 vectors at a
 * time, min(n rounded up to 128, 32768) * (4 d + 4 d / 128) bytes.
 * Host only.                                                               */
tq_status tq_encode_workspace_bytes(const tq_params *p, int64_t n, size_t *bytes);

/* Online encode of n vectors ([P5] 第一阶段 + 第二阶段; [P3] 四):
 *   nu = ||x||, u = Pi x / nu, idx_i = #{j : u_i >= boundary_j},
 *   prod: r = x - nu Pi^T c[idx], sign bits of S r, rnorm = ||r||.
 * x: device, row-major [n][d], dtype TQ_F32 or TQ_BF16.  codes: device
 * arrays sized by tq_codes_bytes.  workspace: device, at least
 * tq_encode_workspace_bytes(p, n) bytes (may be NULL when that is 0); its
 * contents are scratch, nothing needs clearing.  A zero vector encodes as
 * idx = 2^(B-1), all sign bits 1, both norms 0.                            */
tq_status tq_encode(const tq_params *p, const void *x, int32_t dtype, int64_t n,
                    tq_codes codes, void *workspace, size_t ws_bytes, void *stream);

/* Workspace bytes tq_score needs for n_kv*g queries.  Host only.           */
tq_status tq_score_workspace_bytes(const tq_params *p, int64_t n_kv, int64_t g,
                                   size_t *bytes);

/* Decode-time attention logits straight from the packed codes ([P3]
 * 非对称估计器 applied to the residual, plus the MSE part):
 *   logit[h][n] = knorm_n * <Pi q_h, c[idx_n]>
 *               + sqrt(pi/2)/m * rnorm_n * <S q_h, s_n>,  s = +-1,
 * query head h reads KV head h / g (grouped-query attention).
 * q: device float [n_kv*g][d]; codes: device, n_kv*seq vectors, KV head k
 * owning vectors k*seq .. k*seq+seq-1; logits: device float [n_kv*g][seq]
 * (unscaled).  workspace: device, >= tq_score_workspace_bytes.             */
tq_status tq_score(const tq_params *p, const float *q, int64_t n_kv, int64_t g,
                   tq_codes codes, int64_t seq, float *logits, void *workspace,
                   size_t ws_bytes, void *stream);

/* Workspace bytes tq_attend needs.  Host only.                             */
tq_status tq_attend_workspace_bytes(const tq_params *kp, const tq_params *vp,
                                    int64_t batch, int64_t n_kv, int64_t g,
                                    int64_t seq, size_t *bytes);

/* One decode step of attention over a compressed KV cache, the computation
 * whose speed-up over 32-bit keys the yeyulingfeng.com explainer reports for
 * 4-bit TurboQuant on H100 (section "TurboQuant：6倍压缩，零损失", and its
 * caveat that the speed-up is for attention, not end-to-end inference): the
 * logits are [P3] 非对称估计器 applied to the compressed keys (tq_score); the
 * values are the MSE reconstructions of [P5] 第一阶段 (mse mode):
 *   p = softmax(scale * logits) over all seq positions,
 *   out[b][h] = sum_n p_n * ||v_n|| * Pi_V^T c_V[idx_n].
 * The softmax temperature is not on the pages: scale <= 0 selects the usual
 * 1/sqrt(d).
 * kp: prod-mode parameters of the keys; vp: mse-mode parameters of the
 * values (same d).  q: device float [batch][n_kv*g][d]; kcodes / vcodes:
 * device, batch*n_kv*seq vectors each; out: device float [batch][n_kv*g][d].
 * workspace: device, >= the size above.                                  */
tq_status tq_attend(const tq_params *kp, const tq_params *vp, const float *q,
                    int64_t batch, int64_t n_kv, int64_t g, tq_codes kcodes,
                    tq_codes vcodes, int64_t seq, float scale, float *out,
                    void *workspace, size_t ws_bytes, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): tq_attend
 * with the same arguments except the workspace, which is replaced by a
 * file-scope device array of TQ_NOALLOC_SCRATCH_BYTES in the library (one per
 * GPU, held until the process ends).  Calls no hipMalloc, hipFree or other
 * allocating routine, records no memset, and needs nothing cleared.
 *   - Sizes whose workspace (tq_attend_workspace_bytes) exceeds
 *     TQ_NOALLOC_SCRATCH_BYTES return TQ_ERR_UNSUPPORTED (tq_last_error gives
 *     the bytes needed); nothing is launched.
 *   - The per-(parameters, device) cache of kp and vp must exist already on
 *     the current device (TQ_ERR_INVALID_ARG otherwise): any earlier call with
 *     the same parameters builds it, e.g. tq_encode of the keys and values.
 *   - Every call on one GPU shares that GPU's array: calls that overlap in
 *     time on one device (different streams, different host threads) race
 *     and give wrong outputs.  Calls on one stream are ordered and safe.  */
#define TQ_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
tq_status tq_attend_noalloc(const tq_params *kp, const tq_params *vp, const float *q,
                            int64_t batch, int64_t n_kv, int64_t g, tq_codes kcodes,
                            tq_codes vcodes, int64_t seq, float scale, float *out,
                            void *stream);

/* ---------------------------------------------------------------------------
 * Paged code cache for decoding.  The pages "TurboQuant压缩效果" (the kernel
 * decompresses the codes as it reads them, in registers) and
 * "刷屏的Google Research论文…", section 九 item 4 (at scale the rotation must be
 * generated once and reused) describe the serving setting: tokens are encoded
 * once into a cache that grows page by page, and every decode step attends
 * over it with the same (Pi, S) of the parameters' seeds.
 *
 * A store of num_pages pages holds num_pages * n_kv * TQ_PAGE_POSITIONS
 * vectors (one tq_codes set for keys, one for values); vector (page, head,
 * offset) is (page * n_kv + head) * TQ_PAGE_POSITIONS + offset.
 * ------------------------------------------------------------------------- */
#define TQ_PAGE_POSITIONS 512

/* Encodes n vectors like tq_encode and stores vector i at slot slots[i] of a
 * code store of `capacity` vectors (appending new tokens to a paged cache).
 * slots: device int64 [n], distinct (two equal slots race); slots outside
 * [0, capacity) are skipped.  Built for d = m = 128 (TQ_ERR_UNSUPPORTED
 * otherwise); no workspace.                                                */
tq_status tq_encode_slots(const tq_params *p, const void *x, int32_t dtype, int64_t n,
                          const int64_t *slots, int64_t capacity, tq_codes codes,
                          void *stream);

/* Workspace bytes tq_attend_paged needs.  Host only.                       */
tq_status tq_attend_paged_workspace_bytes(const tq_params *kp, const tq_params *vp,
                                          int64_t batch, int64_t n_kv, int64_t g,
                                          int64_t max_pages, size_t *bytes);

/* tq_attend over a paged store: sequence b has seq_lens[b] positions, and its
 * positions 512 j .. 512 j + 511 live in page block_table[b][j].
 * block_table: device int32 [batch][max_pages]; seq_lens: device int32
 * [batch], each in [1, max_pages * TQ_PAGE_POSITIONS] (clamped into that
 * range); page ids are clamped into [0, num_pages), so bad entries give wrong
 * rows, never an access outside the store.  q, out, scale and the parameters
 * as tq_attend.  max_pages * TQ_PAGE_POSITIONS < 2^28.                     */
tq_status tq_attend_paged(const tq_params *kp, const tq_params *vp, const float *q,
                          int64_t batch, int64_t n_kv, int64_t g, tq_codes kcodes,
                          tq_codes vcodes, int64_t num_pages, const int32_t *block_table,
                          int64_t max_pages, const int32_t *seq_lens, float scale, float *out,
                          void *workspace, size_t ws_bytes, void *stream);

/* MSE reconstruction of n vectors, x~ = ||x|| Pi^T c[idx] ([P5] 第一阶段: the
 * reconstruction whose squared error the Lloyd-Max codebook minimises).
 * Prod-mode codes decode their B = b-1 bit MSE part (the QJL bits carry no
 * reconstruction).  codes: device, n vectors; out: device float [n][d].    */
tq_status tq_decode(const tq_params *p, tq_codes codes, int64_t n, float *out,
                    void *stream);

/* Workspace bytes tq_search needs.  Host only.                             */
tq_status tq_search_workspace_bytes(const tq_params *p, int64_t nq, int64_t n,
                                    int32_t k, size_t *bytes);

/* Top-k search over compressed vectors: the vector-search use the
 * "TurboQuant压缩效果" transcript names beside the KV cache (compressing the
 * memory of vector search engines), scored with the same estimator as
 * tq_score ([P3] 非对称估计器): for each of nq queries, the k database vectors of
 * largest logit, in descending order, ties broken by the lower index.  The
 * logits are never materialised: workgroups keep running top-k lists over
 * segments of the database and a final pass merges them.
 * q: device float [nq][d]; codes: device, n vectors (n < 2^31); out_idx:
 * device int64 [nq][k]; out_val: device float [nq][k] (may be NULL), the
 * logits as tq_score computes them.  1 <= k <= 32 and k <= n.  workspace:
 * device, >= tq_search_workspace_bytes (query operands and candidate lists,
 * O(nq (d + m + k)) bytes).                                                */
tq_status tq_search(const tq_params *p, const float *q, int64_t nq, tq_codes codes,
                    int64_t n, int32_t k, int64_t *out_idx, float *out_val,
                    void *workspace, size_t ws_bytes, void *stream);

/* Frees every cached matrix/codebook on every device.  Not thread-safe with
 * concurrent calls into the library.                                       */
tq_status tq_release_cache(void);

/* ---------------------------------------------------------------------------
 * Outlier-channel mixed bit widths: the channels of a head are split into a
 * few outlier channels that get one bit more and the ordinary ones
 * ("TurboQuant压缩效果": 3 bits on the outlier channels, 2 on the great
 * majority, 2.5 and 3.5 bits per coordinate on average over 128 channels).
 * With b_out = b_rest + 1 the average is b_rest + n_out / 128: n_out = 64
 * gives the page's 2.5 / 3.5 bits, n_out = 32 a few outliers (2.25 / 3.25).
 * The split is made before the rotation; group 0 (the n_out outlier
 * channels) and group 1 (the other 128 - n_out) are each a prod-mode
 * TurboQuant instance of their own dimension d_g with m = d_g (rotation seed
 * seed_pi + g, JL seed seed_s + g), and the logit is the sum of the two
 * groups' estimators.
 *
 * channels: a permutation of 0 .. 127 whose first n_out entries are the
 * outlier channels (chosen by the caller, e.g. the channels of largest mean
 * square in a prompt's keys).
 *
 * Packed record (d = 128): tq_split_words() uint32 words per vector, group 0
 * then group 1; a group with B = b - 1 Lloyd-Max bits holds its B index
 * planes and then its sign plane, d_g / 32 words each.  Rotated coordinate
 * c = 16 t + 4 k + i of the group (t < d_g / 16; k, i < 4) is bit
 * k d_g / 4 + 4 t + i of the plane's bit string, bit j of which is bit
 * j % 32 of the plane's word j / 32 (d_g = 64: word k / 2, bit
 * 16 (k % 2) + 4 t + i).  Float32 norms [n][4]: ||x_0||, ||r_0||, ||x_1||,
 * ||r_1||.  At n_out = 64: 10 words + 16 bytes (56 bytes) at 2.5 bits, 14
 * words + 16 bytes (72 bytes) at 3.5 bits.
 * ------------------------------------------------------------------------- */
typedef struct {
  int32_t d;             /* 128 */
  int32_t b_out;         /* bits of the outlier channels: b_rest + 1 */
  int32_t b_rest;        /* 2 or 3 */
  int32_t n_out;         /* outlier channels: 32, 64 or 96 (0 selects 64) */
  uint64_t seed_pi;
  uint64_t seed_s;
  int32_t channels[128]; /* host copy of the channel order */
} tq_split_params;

typedef struct {
  uint32_t *words;  /* device uint32 [n][tq_split_words()] */
  float *norms;     /* device float32 [n][4] */
} tq_split_codes;

/* uint32 words per vector.  Host only.                                      */
tq_status tq_split_words(const tq_split_params *p, int32_t *words);

/* Encodes n vectors x (row-major [n][128], TQ_F32 or TQ_BF16, device,
 * 16-byte aligned).  Asynchronous on `stream`; no workspace.               */
tq_status tq_split_encode(const tq_split_params *p, const void *x, int32_t dtype, int64_t n,
                          tq_split_codes codes, void *stream);

/* Workspace bytes tq_split_score needs for n_kv * g queries.  Host only.   */
tq_status tq_split_score_workspace_bytes(const tq_split_params *p, int64_t n_kv, int64_t g,
                                         size_t *bytes);

/* Logits [n_kv * g][seq] (float32, device) of queries q [n_kv * g][128]
 * against the codes of n_kv * seq vectors (vector h * seq + pos); query head
 * j uses KV head j / g.  Asynchronous.                                      */
tq_status tq_split_score(const tq_split_params *p, const float *q, int64_t n_kv, int64_t g,
                         tq_split_codes codes, int64_t seq, float *logits, void *workspace,
                         size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * PolarQuant: the stage-1 variant in which the rotated vector becomes one
 * radius and d - 1 angles by a recursive polar transform, each angle
 * quantised with a fixed codebook of its known law ("TurboQuant 与 AI 效率革命：
 * 当旧数学遇到新智能", section 二, 极坐标的洞察 and 递归极坐标变换; bits per
 * level: "TurboQuant压缩效果", 4 bits at the first level and 2 after).
 *
 * y = Pi x with the TurboQuant rotation of seed_pi.  Level 1 pairs y_2j,
 * y_2j+1 into the angle atan2(y_2j+1, y_2j) in [0, 2 pi) (uniform law, bits1
 * bits, uniform grid); level l >= 2 pairs the level-(l-1) radii (2j, 2j+1)
 * into atan2(r_2j+1, r_2j) in [0, pi/2], whose law has density
 * Gamma(k) / (2^(k-2) Gamma(k/2)^2) sin^(k-1)(2 theta), k = 2^(l-1)
 * (Lloyd-Max codebook of `bits` bits).  A code is the number of boundaries at
 * or below the angle.  The logit of a query q is <Pi q, y^>, y^ rebuilt from
 * the radius ||x|| down the tree (r cos, r sin of the centroid angles).
 *
 * Packed record of one vector (d = 128, bits1 = 4, bits = 2): 12 uint32
 * words `pq` and the float32 radius, 52 bytes.  Level 1 node j = 8 t + 2 g + i
 * (coordinates 2j, 2j+1; t < 8, g < 4, i < 2): word 2 g + t / 4, bits
 * 4 (2 (t % 4) + i) .. + 3.  Level 2 node 4 t + g: word 8 + g, bits 2 t.
 * Level 3 node 2 t + h: word 8 + 2 h, bits 16 + 2 t.  Level 4 node t: word 9,
 * bits 16 + 2 t.  Level 5 node j: word 11, bits 16 + 2 j; level 6 node j:
 * word 11, bits 24 + 2 j; level 7: word 11, bits 28.  Other bits are zero.
 * ------------------------------------------------------------------------- */
typedef struct {
  int32_t d;        /* power of two; the device kernels take d = 128 */
  int32_t bits1;    /* bits of a level-1 angle (device: 4) */
  int32_t bits;     /* bits of an angle at levels >= 2 (device: 2) */
  int32_t reserved; /* 0 */
  uint64_t seed_pi; /* rotation seed (the TurboQuant Pi) */
} tq_polar_params;

typedef struct {
  uint32_t *pq;   /* device uint32 [n][12], caller-owned */
  float *radius;  /* device float32 [n] */
} tq_polar_codes;

/* Codebook of level `level` (1 .. log2 d) at nbits bits (1 .. 6): float32
 * centroids [2^nbits] and boundaries [2^nbits - 1], ascending, in radians.
 * Host only.                                                                */
tq_status tq_polar_make_codebook(int32_t d, int32_t level, int32_t nbits, float *centroids,
                                 float *boundaries);

/* Encodes n vectors x (row-major [n][128], TQ_F32 or TQ_BF16, device, 16-byte
 * aligned) into codes.  Asynchronous on `stream`; no workspace.
 * TQ_ERR_UNSUPPORTED unless d = 128, bits1 = 4, bits = 2.                  */
tq_status tq_polar_encode(const tq_polar_params *p, const void *x, int32_t dtype, int64_t n,
                          tq_polar_codes codes, void *stream);

/* Workspace bytes tq_polar_score needs for n_kv * g queries.  Host only.   */
tq_status tq_polar_score_workspace_bytes(const tq_polar_params *p, int64_t n_kv, int64_t g,
                                         size_t *bytes);

/* Logits [n_kv * g][seq] (float32, device) of queries q [n_kv * g][128]
 * (float32, device) against the codes of n_kv * seq vectors (vector
 * h * seq + pos); query head j uses KV head j / g.  Asynchronous; the caller's
 * workspace holds the rotated queries.                                      */
tq_status tq_polar_score(const tq_polar_params *p, const float *q, int64_t n_kv, int64_t g,
                         tq_polar_codes codes, int64_t seq, float *logits, void *workspace,
                         size_t ws_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H */
