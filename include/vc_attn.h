/*
 * vc_attn.h -- C ABI of the VC-Attention hot path on AMD Instinct MI355X
 * (gfx950): non-causal FP8 flash-attention forward with ExpCast-FP8 and
 * V-Smooth.
 *
 * Sources, cited by page title and place:
 *   [VC]  "VC-Attention: Value Smoothing and Softmax Casting for Low-bit
 *         Attention" (arXiv 2609.15810).
 *   [OVC] "Open-VC Attention: an open-source, error-tunable variant of
 *         VC-Attention" (machgen.ai blog).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers owned by the caller.  The
 *    library never allocates, frees or synchronises; every call only
 *    enqueues kernels on `stream` (a hipStream_t passed as void*; NULL is the
 *    default stream) and returns.  Calls are graph-capturable.
 *  - Shapes: B batches, H heads, S tokens, D head dim (D in {64, 128}).
 *    nblk = ceil(S / 128) key/query blocks, S_pad = 128 * nblk.
 *  - bf16 activations are described by vc_bshd: element (b, s, h, d) lives at
 *    ptr + b*sB + s*sS + h*sH + d (strides in elements, d contiguous).  The
 *    base and all three strides must be multiples of 8 elements (16 bytes),
 *    and the token stride sS below 2^30 elements (2 GiB; VC_ERR_SHAPE).
 *  - FP8 data is OCP E4M3 (E4M3FN: bias 7, max 448, no infinities), the
 *    format gfx950's matrix cores consume.
 *  - Packed FP8 operand layouts.  K and V (and K', R) are stored tile-major
 *    so that each 128-key tile is one contiguous block the attention kernel
 *    copies HBM -> LDS as is; inside a tile each 16-byte chunk is placed at
 *    a swizzled chunk index (this makes the kernel's LDS reads conflict-free)
 *    and V keys are ordered as the kernel's P.V operand consumes them:
 *      sw(r) = ((r >> 1) & 7) ^ ((r & 1) << 2)
 *      packed K, per (b, h): byte ((b*H + h)*nblk + j)*128*D + r*D
 *        + 16*(c ^ swK(r)) + e holds logical K code [128 j + r][16 c + e]
 *        (r < 128, c < D/16, e < 16), swK = sw for D = 128, sw & 3 for
 *        D = 64;
 *      packed V, per (b, h): byte ((b*H + h)*nblk + j)*D*128 + d*128
 *        + 16*(c ^ sw(d)) + e (c < 8, e < 16) holds the V code of channel d,
 *        key 128 j + kappa(16 c + e), kappa(p) = (p & 64)
 *        + 16*((p >> 2) & 3) + 4*((p >> 4) & 3) + (p & 3).
 *    Both occupy B*H*S_pad*D bytes, the same as the row-major forms.
 *  - Validation of every argument happens before anything is enqueued; on
 *    error nothing is written and a vc_status other than VC_OK is returned.
 *    A failed launch returns VC_ERR_HIP (from hipGetLastError, no sync).
 *    Device-side faults surface at the caller's next synchronisation.
 *  - NaN or Inf inputs are not checked; they propagate.
 *  - Entry points are thread-safe; concurrent calls must not share output
 *    buffers or workspaces.
 */
#ifndef VC_ATTN_H
#define VC_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VC_ABI_VERSION 7

typedef enum vc_status {
  VC_OK = 0,
  VC_ERR_NULL = 1,        /* a required pointer is NULL */
  VC_ERR_SHAPE = 2,       /* B, H, S or D out of range */
  VC_ERR_ALIGN = 3,       /* pointer or stride not 16-byte aligned */
  VC_ERR_UNSUPPORTED = 4, /* parameter outside the supported set */
  VC_ERR_WORKSPACE = 5,   /* workspace too small */
  VC_ERR_HIP = 6,         /* a HIP launch failed */
  VC_ERR_SCRATCH = 7      /* the shape needs more than the static scratch holds */
} vc_status;

typedef struct vc_shape {
  int32_t B, H, S, D;
} vc_shape;

/* bf16 tensor in [B, S, H, D] order with element strides (see above). */
typedef struct vc_bshd {
  const void* ptr;
  int64_t sB, sS, sH;
} vc_bshd;

typedef struct vc_bshd_out {
  void* ptr;
  int64_t sB, sS, sH;
} vc_bshd_out;

/* ABI version of the loaded library (VC_ABI_VERSION it was built with). */
int32_t vc_abi_version(void);

/* Static, human-readable name of a status code. */
const char* vc_status_str(int32_t status);

/* ----------------------------------------------------------------------- */

/*
 * Q/K preprocessing ahead of the quantisers ([VC] §3.4 "Fused Kernel and
 * Amortized Grouping" and Appendix B: rotary embedding, the key channel mean,
 * the QK Hadamard rotation, fused into the quantisers).  Applied per row in
 * this order, in fp32, before the pre-factor and the block scale:
 *   VC_PREP_ROPE:     pairs (2i, 2i+1) of a row at token position p become
 *                     (a c - b s, a s + b c), c = rope_cos[p][i],
 *                     s = rope_sin[p][i] (fp32 [S][D/2] device tables; for
 *                     V-Smooth's K' the position is the key's own, before the
 *                     gather);
 *   VC_PREP_K_CENTER: K only: minus the channel mean of the head's S keys
 *                     after RoPE (sums in 64-bit fixed point with 24 fraction
 *                     bits, mean = fl(sum / (S 2^24)) in fp64).  Softmax rows
 *                     do not change;
 *   VC_PREP_HADAMARD: the unnormalised Walsh-Hadamard transform over D,
 *                     radix-2 butterflies (a, b) -> (a + b, a - b) over strides
 *                     1, 2, ..., D/2; Q's pre-factor becomes G / D (exact), so
 *                     the scores do not change.
 * Q and K must be prepared alike (the same RoPE tables, the rotation on both)
 * for the attention to be the intended one: with V-Smooth, pass the same
 * vc_prep_params to vc_quantize (Q) and vc_smooth_group (K).
 * workspace: device, 8-byte aligned, >= vc_prep_workspace_size(shape) bytes,
 * needed with VC_PREP_K_CENTER when K is given (else may be NULL); its
 * contents on entry do not matter.
 */
#define VC_PREP_ROPE 1u
#define VC_PREP_HADAMARD 2u
#define VC_PREP_K_CENTER 4u

typedef struct vc_prep_params {
  uint32_t flags;        /* OR of VC_PREP_* (0: none) */
  const float* rope_cos; /* fp32 [S][D/2], with VC_PREP_ROPE */
  const float* rope_sin; /* fp32 [S][D/2], with VC_PREP_ROPE */
  void* workspace;
  size_t workspace_bytes;
} vc_prep_params;

/* Bytes of device workspace VC_PREP_K_CENTER needs: B*H*D*8. */
size_t vc_prep_workspace_size(const vc_shape* shape);

/*
 * vc_quantize -- FP8 operands for the attention kernel.
 * [OVC] "Scheduling around ExpCast" and "Fused input preparation": Q and K
 * take one E4M3 scale per 128-token block, V one scale per head; the packed
 * V is stored transposed with the key dimension contiguous ("Packed V").
 * [VC] §3.1: X_q = s_X * Xhat.  The blog folds softmax scale, log2 e and
 * ExpCast's factor 8 into the code's multiply-add; here they go into Q's
 * codes, and the Q/K block scales are powers of two, which the attention
 * kernel's block-scaled matrix product applies exactly.
 *
 * sm_scale: the softmax scale (0 selects 1/sqrt(D)); must be finite, >= 0.
 * G = 8 * fl(sm_scale * fl(log2 e)) (fp32; the factor 8 is exact), divided
 * by D with VC_PREP_HADAMARD.
 * prep: preprocessing (above), or NULL for none.
 * For each (b, h) and 128-token block j of Q (pre = G) and of K (pre = 1),
 * x the row after preprocessing:
 *   y = fl(x * pre); amax = max |y| over the block's valid rows;
 *   e = the smallest integer >= -127 with amax <= 448 * 2^e (e = 0 for a
 *   block of zeros); scale = 2^e; code = E4M3_rne(y * 2^-e).
 *   Q rows >= S are written as code 0; K rows >= S repeat the codes of
 *   row S - 1 (so the ragged last tile's max over all its rows is that of
 *   its valid rows -- the attention kernel relies on it when repair tiles
 *   follow that tile).  So Q * G ~= q8 * q_scale and K ~= k8 * k_scale.
 *   q8:           uint8 [B][H][S_pad][D] row-major
 *   k8:           packed K (B*H*S_pad*D bytes)
 *   q_scale, k_scale: fp32 [B][H][nblk] (powers of two)
 * For V: one amax per (b, h) over all S x D elements; s = amax / 448 (fp32),
 * code = E4M3_rne(x * (448 / amax)), s = 1 for zeros;
 *   v8:      packed V (B*H*S_pad*D bytes; keys >= S are code 0)
 *   v_scale: fp32 [B][H][D]          (the head's scale repeated over d)
 * Any of q, k, v may have ptr == NULL to skip that operand (its outputs are
 * then ignored and may be NULL).  q8/k8/v8 must be 16-byte aligned.
 */
int32_t vc_quantize(const vc_shape* shape, float sm_scale, const vc_prep_params* prep, const vc_bshd* q,
                    const vc_bshd* k, const vc_bshd* v, uint8_t* q8, float* q_scale, uint8_t* k8, float* k_scale,
                    uint8_t* v8, float* v_scale, void* stream);

/* ----------------------------------------------------------------------- */

typedef struct vc_group_params {
  int32_t clusters; /* k in [1, min(S, 8192 / D)] */
  int32_t iters;    /* Lloyd iterations, [1, 64] */
  uint64_t seed;    /* seeds the Forgy initialisation */
  uint32_t flags;   /* 0, VC_GROUP_WARM_START or VC_GROUP_REUSE_PERM */
} vc_group_params;

/* Warm start ([VC] §3.2, "Unbalanced clusters cost little": each step starts
 * from the previous step's centroids): `centroids` is read as the first
 * iterate instead of the Forgy draw, then overwritten with the result; the
 * seed is unused. */
#define VC_GROUP_WARM_START 1u
/* Permutation reuse ([VC] §3.4 and Appendix A: pi is computed once and
 * reused for the following steps of the window): no k-means and no sort;
 * `perm` is read (a permutation of [0, S) per (b, h)) and only step 3 runs
 * on the given K, V.  `centroids` and `labels` are not touched and may be
 * NULL; `clusters` and `iters` are not used but must still be valid. */
#define VC_GROUP_REUSE_PERM 2u

/* Bytes of device workspace vc_smooth_group needs for this shape. */
size_t vc_smooth_group_workspace_size(const vc_shape* shape, int32_t clusters);

/*
 * vc_smooth_group -- V-Smooth grouping, demeaning and residual quantisation.
 * [VC] §3.2 "Value-guided permutation" (Eq. 3), "Block demeaning" (Eq. 4),
 * "Unbalanced clusters cost little"; Appendix B (per-operand fused kernels,
 * means stored divided by the per-channel value scale).
 *
 * Per (b, h):
 *  1. k-means over the value tokens (Lloyd): centroids start at the values of
 *     `clusters` distinct tokens drawn by a partial Fisher-Yates shuffle fed
 *     by SplitMix64 with state seed + 0x9E3779B97F4A7C15 * (1 + b*H + h);
 *     each assignment takes argmin_c (|c|^2 - 2 v.c) with every dot product
 *     one fp32 fused-multiply-add chain over d = 0..D-1 (ties -> lowest c);
 *     each update is the member mean, summed in 64-bit fixed point with 24
 *     fraction bits (order independent); empty clusters keep their centroid.
 *     labels = the last assignment, centroids = after the last update.
 *  2. perm = stable argsort(labels)  (K' = K[perm], V' = V[perm]).
 *  3. For each 128-row block j of V': mu_j = bf16(mean of its valid rows);
 *     R = V' - 1 mu_j^T in fp32; per-channel s_R[d] = amax_d |R| / 448;
 *     r8 = E4M3_rne(R * (448 / amax_d)); the scaled mean m = mu_j[d] *
 *     (448 / amax_d) in fp32 is stored as a bf16 pair mu_split[j][d] =
 *     hi | lo << 16, hi = bf16_rne(m), lo = bf16_rne(m - hi) (m - hi is
 *     exact), the form the attention kernel's mean product reads.  K' is
 *     quantised per 128-row block as K in vc_quantize (power-of-two
 *     scales).
 * prep: K's preprocessing (vc_quantize), applied to each key of K' before
 * its block scale, or NULL for none.
 * With VC_GROUP_WARM_START, step 1 starts from the given centroids; with
 * VC_GROUP_REUSE_PERM, steps 1 and 2 are skipped and perm is an input.  The
 * two flags exclude each other (VC_ERR_UNSUPPORTED).
 * Outputs (all device, caller-owned):
 *   centroids fp32 [B][H][clusters][D]; labels, perm int32 [B][H][S];
 *   k8 packed K, k_scale fp32 [B][H][nblk];
 *   r8 packed V (the residual codes), r_scale fp32 [B][H][D];
 *   mu_bf16 uint16 [B][H][nblk][D]; mu_split uint32 [B][H][nblk][D].
 * workspace: >= vc_smooth_group_workspace_size(shape, clusters) bytes,
 * 256-byte aligned; its contents on entry do not matter.
 */
int32_t vc_smooth_group(const vc_shape* shape, const vc_bshd* k, const vc_bshd* v, const vc_group_params* p,
                        const vc_prep_params* prep, float* centroids, int32_t* labels, int32_t* perm, uint8_t* k8,
                        float* k_scale, uint8_t* r8, float* r_scale, uint16_t* mu_bf16, uint32_t* mu_split,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * vc_smooth_group_noalloc -- vc_smooth_group without a workspace argument,
 * for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, semantics and outputs as vc_smooth_group (bit for bit), with the
 * workspace (and, with VC_PREP_K_CENTER, the centring sums; prep->workspace
 * is then not used) taken from a static device array of
 * VC_GROUP_SCRATCH_BYTES that the library holds on every GPU it runs on
 * until the process ends.  The array of the calling thread's current device
 * is used, so `stream` must belong to that device; the call itself never
 * allocates or frees.  Its device address is looked up once per device, on
 * that device's first call (VC_ERR_HIP if the lookup fails).
 * Limits: vc_smooth_group_noalloc_bytes(shape, clusters, prep flags) must be
 * <= VC_GROUP_SCRATCH_BYTES (the Wan-shaped H = 40, S = 75600, D = 128 call
 * with 64 clusters needs about 5.7 MB; H = 48, S = 84672 about 7.3 MB), else
 * VC_ERR_SCRATCH and nothing is enqueued.
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (different streams, or threads without ordering) race and give wrong
 * results; calls ordered on one stream are safe.  Every part of the array a
 * call reads is written by that call first.
 */
#define VC_GROUP_SCRATCH_BYTES ((size_t)16 << 20)

/* Scratch bytes vc_smooth_group_noalloc needs (0 for an invalid shape). */
size_t vc_smooth_group_noalloc_bytes(const vc_shape* shape, int32_t clusters, uint32_t prep_flags);

int32_t vc_smooth_group_noalloc(const vc_shape* shape, const vc_bshd* k, const vc_bshd* v, const vc_group_params* p,
                                const vc_prep_params* prep, float* centroids, int32_t* labels, int32_t* perm,
                                uint8_t* k8, float* k_scale, uint8_t* r8, float* r_scale, uint16_t* mu_bf16,
                                uint32_t* mu_split, void* stream);

/* ----------------------------------------------------------------------- */

/*
 * V residual repair rows ([OVC] "Why V residual repair"; plain path only).
 * With one FP8 scale per head, token j keeps the residual
 * r_j = V_j - s * Vhat_j, s = amax / 448, Vhat_j = E4M3_rne(V_j * (448 / amax))
 * (per element, each operation rounded once in fp32).  The R tokens of
 * largest residual energy sum_d r_jd^2 (fp64, summed over d = 0..D-1 in
 * order; ties go to the lower token index) become repair rows: the key of
 * the token, prepared as K is (vc_quantize's prep, at the token's own
 * position), paired with the residual as a value row.  The pages pick
 * R = ceil(rho S) with rho = 0.5%; the caller passes R.
 *
 * vc_repair_prepare writes, per (b, h), with nrb = ceil(R / 128):
 *   idx      int32 [B][H][R]: the selected token indices, ascending;
 *   rk8      packed K tiles [B][H][nrb] (the packed K layout with nrb in
 *            place of nblk): repair row i < R holds key idx[i]; rows past R
 *            repeat key idx[R-1] (so a tile's max is that of its real rows);
 *   rk_scale fp32 [B][H][nrb]: power-of-two block scales as vc_quantize's;
 *   rv8      packed V tiles [B][H][nrb]: code E4M3_rne(r * (448 / amax)),
 *            the head's own V scale (so v_scale of vc_quantize applies);
 *            rows past R are code 0.
 * prep: K's preprocessing, as passed to vc_quantize (NULL for none).
 * rows: R in [0, S]; R = 0 writes nothing.
 * workspace: device, 256-byte aligned, >= vc_repair_workspace_size(shape)
 * bytes; its contents on entry do not matter.
 */
size_t vc_repair_workspace_size(const vc_shape* shape);
int32_t vc_repair_prepare(const vc_shape* shape, const vc_prep_params* prep, const vc_bshd* k, const vc_bshd* v,
                          int32_t rows, int32_t* idx, uint8_t* rk8, float* rk_scale, uint8_t* rv8, void* workspace,
                          size_t workspace_bytes, void* stream);

/* Repair rows for vc_attn_fwd (rows = 0 or a NULL pointer to this: none). */
typedef struct vc_repair_rows {
  int32_t rows;          /* R from vc_repair_prepare */
  const uint8_t* k8;     /* rk8 */
  const float* k_scale;  /* rk_scale */
  const uint8_t* v8;     /* rv8 */
} vc_repair_rows;

/* ----------------------------------------------------------------------- */

#define VC_ATTN_SEQUENTIAL 1u /* visit key blocks 0..nblk-1 instead of mid-window */

typedef struct vc_attn_params {
  float sm_scale;  /* softmax scale; 0 selects 1/sqrt(D) (vc_attn_fwd_bf16; the FP8
                      path takes it from q8, see vc_quantize; validated only) */
  int32_t window;  /* mid-window offset W >= 0 (default 2) */
  uint32_t flags;  /* VC_ATTN_SEQUENTIAL or 0 */
} vc_attn_params;

/*
 * vc_attn_fwd -- non-causal FP8 attention with ExpCast-FP8 (and V-Smooth's
 * mean restoration when mu_split != NULL).
 * [VC] §3.1 Eq. 1 (online softmax), §3.2 Eq. 6 (A <- aA + P_q R_q + r mu^T),
 * §3.3 Eq. 7 (c = clip_[0,120](Round(8(u+8)+56+beta)), beta = -0.35);
 * [OVC] "Scheduling around ExpCast" (true-score running max, scales folded
 * into the code arithmetic, 4 codes per register), "A consistent
 * denominator", "Mid-window key traversal".
 *
 * For each query row i (tile qt = i / 128) and key block t in the order
 *   start = min((qt | 1) + window, nblk - 1): start, start-1, ..., 0,
 *   start+1, ..., nblk-1
 * (query tiles 2p and 2p+1 are processed together and share one pass over
 * K/V -- [OVC] "A warp-specialized pipeline" -- so the start lies `window`
 * blocks past the pair's second diagonal block),
 * y = q_scale[qt] * k_scale[t] * (Q8 . K8) + (119.65 - 8 M) (matrix cores:
 * E8M0 block scales, fp32 accumulate starting at the offset), where
 * q_scale * k_scale * (Q8 . K8) / 8 is the log2-domain score because q8
 * carries G (vc_quantize) -- so sm_scale does not enter here;
 * M' = max(M, M + (max y - 119.65) / 8) (the first tile sets M from its
 * max); when M' > M the numerator and denominator are rescaled by
 * 2^(M - M') and y gains 8 (M - M');
 * code = Round(y) clipped below at 0 (an integer conversion, no
 * exponential, no FP8 cast); keys >= S get code 0;
 * A += P_code . V8 (matrix cores); r = sum of the decoded codes (the same
 * bytes, through the matrix cores against a tile of ones); l += r;
 * with V-Smooth A += r * (hi + lo) of mu_split[t], as the three bf16
 * products r_hi hi + r_hi lo + r_lo hi on the matrix cores (r_hi = bf16(r),
 * r_lo = bf16(r - r_hi)), once per 8 visited tiles.
 * repair (plain path only; with mu_split VC_ERR_UNSUPPORTED): after the
 * nblk key blocks, the ceil(R / 128) repair tiles of vc_repair_prepare are
 * visited in order, as above with their own key scales, except that l does
 * not grow (their keys are counted once already) and only repair rows < R
 * count towards the max.
 * Output: O = bf16((A / l) * v_scale[d]) written to `o` ([B,S,H,D] strided),
 * rows in the original query order.
 * Inputs are those of vc_quantize (plain path: q8 .. v_scale from it) or, for
 * V-Smooth, q8/q_scale from vc_quantize and k8/k_scale, v8 = r8,
 * v_scale = r_scale, mu_split from vc_smooth_group.  q_scale and k_scale
 * must be powers of two in [2^-127, 2^127] (as those calls write them).
 * Requires |scores| well below 2^17 in log2 units so the code never exceeds
 * 120 (the upper clip is then implicit).
 */
int32_t vc_attn_fwd(const vc_shape* shape, const vc_attn_params* p, const uint8_t* q8, const float* q_scale,
                    const uint8_t* k8, const float* k_scale, const uint8_t* v8, const float* v_scale,
                    const uint32_t* mu_split, const vc_repair_rows* repair, const vc_bshd_out* o, void* stream);

/* ----------------------------------------------------------------------- */

/*
 * The 4-bit path: V-Smooth at 4 bits without ExpCast ([VC] §4.1
 * "Implementation" -- 4 bits run V-Smooth alone -- and "Scope of ExpCast-FP8":
 * P is kept in a microscaled 4-bit format, for which no affine log-to-code
 * map exists).  The pages' format is NVFP4; gfx950's matrix cores take OCP
 * MXFP4: E2M1 elements (0, 0.5, 1, 1.5, 2, 3, 4, 6 and negatives) with one
 * E8M0 scale byte (2^(byte - 127)) per 32 elements.  A block's scale is the
 * smallest 2^e (e >= -127) with amax <= 6 * 2^e (2^0 for zeros); elements
 * are E2M1, round half to even, of x / 2^e.
 *
 * vc_quantize4 -- Q, K, V into MXFP4 (any of q or k/v may be NULL to skip;
 * k and v go together).  Q is multiplied first by fl32(sm_scale * fl32(log2
 * e)) (sm_scale 0 selects 1/sqrt(D)), so scores come out in log2 units.
 * With perm and mu_bf16 (V-Smooth, from vc_smooth_group) K and V are taken
 * through perm and V becomes the residual fl32(V' - mu_j) of [VC] §3.2
 * Eq. 4; without them (both NULL) the plain 4-bit path.
 * Layouts, per (b, h), nblk = ceil(S / 128), S_pad = 128 nblk:
 *   q4       uint8 [S_pad][D/2]: byte c = channels 2c (low nibble), 2c + 1;
 *   q4_scale uint8 [S_pad][D/32]: one E8M0 byte per 32 channels of a row;
 *   k4       per tile t, 64 D bytes: tile row 64 c + 32 b + 8 j + 4 h + v
 *            (c, b, h < 2, j, v < 4), D/2 bytes as q4, holds key
 *            128 t + 64 c + 32 h + 16 b + 4 j + v, its 16-byte chunk x at
 *            chunk x ^ sw4(r), sw4(r) = (r >> 2) & 3 for D = 128,
 *            (r >> 3) & 1 for D = 64;
 *   k4_scale per tile 512 bytes: byte (32 (x & 1) + (r & 31)) * 8
 *            + 2 (r >> 5) + (x >> 1) is the scale of tile row r, channels
 *            [32 x, 32 x + 32) (127 for x >= D/32);
 *   v4       per tile, D channel rows of 64 bytes: logical byte c of row d
 *            holds keys 128 t + 2c (low nibble) and 128 t + 2c + 1; the
 *            16-byte chunk c of row d sits at chunk c ^ ((d >> 2) & 3);
 *   v4_scale per tile 512 bytes: byte (32 (g & 1) + (d & 31)) * 8
 *            + 2 (d >> 5) + (g >> 1) is the scale of channel d, keys
 *            [128 t + 32 g, 128 t + 32 g + 32) (127 for d >= D);
 * rows / keys >= S are zero codes and do not enter any block maximum.
 * q4, k4, v4 16-byte aligned; k4_scale, v4_scale 8-byte; mu_bf16 16-byte.
 */
int32_t vc_quantize4(const vc_shape* shape, float sm_scale, const vc_bshd* q, const vc_bshd* k, const vc_bshd* v,
                     const int32_t* perm, const uint16_t* mu_bf16, uint8_t* q4, uint8_t* q4_scale, uint8_t* k4,
                     uint8_t* k4_scale, uint8_t* v4, uint8_t* v4_scale, void* stream);

/*
 * vc_attn_fwd4 -- non-causal 4-bit attention on vc_quantize4's operands,
 * keys in the order of vc_attn_fwd.  Per query row and key tile:
 * s = Q4 . K4 (block-scaled matrix cores, log2 units); M' = max(M, max s),
 * the numerator and denominator rescaled by 2^(M - M') on every increase;
 * p = 2^(s - M') (fp32); P in MXFP4 blocks of the tile's 32 consecutive
 * keys; l += sum of the dequantised P; A += P . V4 (block-scaled), and with
 * mu_bf16 (V-Smooth) A += r * mu_t, r the tile's sum of P.  Output
 * bf16(A / l) to `o`.  p->sm_scale is validated only (Q carries it).
 */
int32_t vc_attn_fwd4(const vc_shape* shape, const vc_attn_params* p, const uint8_t* q4, const uint8_t* q4_scale,
                     const uint8_t* k4, const uint8_t* k4_scale, const uint8_t* v4, const uint8_t* v4_scale,
                     const uint16_t* mu_bf16, const vc_bshd_out* o, void* stream);

/* ----------------------------------------------------------------------- */

/*
 * vc_pack_v_bf16 -- key-contiguous, tile-major copy of V for the BF16
 * baseline (B*H*S_pad*D bf16 values, keys >= S zero): per (b, h), tile j and
 * half hf in {0, 1}, element ((b*H + h)*nblk + j)*128*D + hf*64*D + d*64
 * + 8*(c ^ sw(d)) + e holds V[128 j + 64 hf + 8 c + e][d] (c < 8).
 * The FP8 path gets its packed V from vc_quantize; both preparations run
 * outside the timed attention call, as on the pages ([VC] Appendix A).
 */
int32_t vc_pack_v_bf16(const vc_shape* shape, const vc_bshd* v, uint16_t* vt, void* stream);

/*
 * vc_attn_fwd_bf16 -- in-house BF16 flash-attention baseline on the same
 * kernel skeleton as vc_attn_fwd (same tiling, traversal and epilogue):
 * BF16 matrix-core products, fp32 exp2 online softmax ([VC] §3.1 Eq. 1),
 * row sum of the bf16-rounded probabilities.  q, k bf16 [B,S,H,D] strided;
 * vt from vc_pack_v_bf16; o bf16 [B,S,H,D] strided.
 */
int32_t vc_attn_fwd_bf16(const vc_shape* shape, const vc_attn_params* p, const vc_bshd* q, const vc_bshd* k,
                         const uint16_t* vt, const vc_bshd_out* o, void* stream);

/*
 * vc_expcast_codes -- the ExpCast code map alone, for bit-exact checks
 * ([VC] §3.3 Eq. 7): codes[i] = min(120, Round_even_clamped0(fma(a[r], x[i],
 * b[r]))) with r = i / row_len: one fp32 fused multiply-add, then the
 * round-half-even integer conversion clamped at 0 (v_cvt_pk_u8_f32), then the
 * explicit upper clip.  It is a routine of its own: vc_attn_fwd forms the
 * pre-rounding value inside its score product instead (the accumulator
 * starts at the code offset) and applies the same conversion to it, so its
 * codes are observable only through its output.
 * x: fp32 [n]; a, b: fp32 [n / row_len]; codes: uint8 [n].  n % row_len == 0.
 */
int32_t vc_expcast_codes(const float* x, const float* a, const float* b, int64_t n, int32_t row_len,
                         uint8_t* codes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* VC_ATTN_H */
