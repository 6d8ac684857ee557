// vc_group.hip -- V-Smooth grouping on the GPU.
//
// [VC] §3.2 "Value-guided permutation": per (b, h) an online k-means over the
// value tokens gives labels z and pi = argsort(z); K and V are permuted
// together (Eq. 3).  "Block demeaning": each 128-row block of V' loses its
// mean, the residual goes through the per-channel E4M3 value quantiser
// (Eq. 4), and the means are stored divided by the per-channel scale
// (Appendix B).  "Unbalanced clusters cost little": plain Lloyd k-means.
//
// Labels / pi / codes are bit-identical to a sequential CPU run of the rule:
// each distance is one fp32 fmaf chain over d = 0..D-1 in a fixed order,
// ties to the lowest cluster.  The assignment computes the distances on the
// matrix cores and settles every token whose winner is not certain under a
// proven error bound with that exact chain (kmeans_assign_mx).  Cluster and
// block sums are 64-bit fixed point (24 fraction bits), which makes atomics
// order-independent; pi is a stable counting sort.
//
// Kernels per call: init (Forgy indices by partial Fisher-Yates on
// SplitMix64, centroids, norms, zeroed accumulators) -> iters x (assign and
// member sums, update; the last assignment also counts each 256-token
// chunk's labels) -> scan of the counts -> stable scatter -> apply pass 1
// (gather K, V by pi; K' per-block codes; block means; residual channel
// maxima) -> apply pass 2 (residual codes, key-contiguous; scaled means).
#include <algorithm>

#include "vc_common.hpp"
#include "vc_prep.hpp"
#include "vc_launch.hpp"

namespace vc {

namespace {

constexpr int kAssignTokens = 2048;  // tokens per assign workgroup
constexpr int kChunk = 256;          // tokens per histogram / scatter chunk
constexpr unsigned char kOpen = 0xff;  // label byte of a token not settled yet (k <= 255)

struct GroupWs {
  long long* sums;      // [BH][k][D]
  long long* counts;    // [BH][k]
  float* norms;         // [BH][k]
  int* hist;            // [BH][k][nchunk]
  unsigned* r_amax;     // [BH][D]
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

GroupWs carve(void* ws, const vc_shape& sh, int k, size_t* total) {
  const size_t BH = (size_t)sh.B * sh.H, nchunk = (sh.S + kChunk - 1) / kChunk;
  char* p = (char*)ws;
  GroupWs g;
  size_t off = 0;
  g.sums = (long long*)(p + off);
  off += align256(BH * k * sh.D * sizeof(long long));
  g.counts = (long long*)(p + off);
  off += align256(BH * k * sizeof(long long));
  g.norms = (float*)(p + off);
  off += align256(BH * k * sizeof(float));
  g.hist = (int*)(p + off);
  off += align256(BH * k * nchunk * sizeof(int));
  g.r_amax = (unsigned*)(p + off);
  off += align256(BH * sh.D * sizeof(unsigned));
  if (total) *total = off;
  return g;
}

VC_DEV uint64_t splitmix64_next(uint64_t& st) {
  uint64_t z = (st += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

VC_DEV long long fx24(float v) { return (long long)rint((double)v * 16777216.0); }

VC_DEV float fx24_mean(long long s, long long n) {
  return (float)(((double)s * (1.0 / 16777216.0)) / (double)n);
}

// fx24 of a bf16 value (its bit pattern b16) with |v| < 128: v * 2^24 is the
// bit pattern with 24 added to the exponent field (a zero or subnormal lands
// far below 1/2 and rounds to 0), rounded to nearest even in fp32 -- the
// same integer as fx24 -- and converted exactly (|v * 2^24| < 2^31).
VC_DEV long long fx24_small(u32 b16) {
  return (long long)(int)__builtin_rintf(__uint_as_float((b16 << 16) + (24u << 23)));
}

// Row t of a token-major tensor: one 32 x 32 -> 64-bit multiply-add.
VC_DEV const uint16_t* token_row(const uint16_t* base, int t, u32 rowB) {
  return (const uint16_t*)((const char*)base + (uint64_t)(u32)t * rowB);
}

// The oracle's assignment rule for one token: one fp32 fmaf chain per
// centroid over d = 0..D-1, distance fmaf(-2, dot, |c|^2), ties to the
// lowest cluster index.
template <int D>
VC_DEV int exact_label(const float (&x)[D], const float* __restrict__ cb, const float* __restrict__ nb, int k) {
  int best = 0;
  float bd = 0.0f;
  int c = 0;
  for (; c + 4 <= k; c += 4) {
    float d0 = 0.f, d1 = 0.f, d2 = 0.f, d3 = 0.f;
    const float* c0 = cb + (c + 0) * D;
    const float* c1 = cb + (c + 1) * D;
    const float* c2 = cb + (c + 2) * D;
    const float* c3 = cb + (c + 3) * D;
#pragma unroll
    for (int d = 0; d < D; ++d) {
      d0 = __builtin_fmaf(x[d], c0[d], d0);
      d1 = __builtin_fmaf(x[d], c1[d], d1);
      d2 = __builtin_fmaf(x[d], c2[d], d2);
      d3 = __builtin_fmaf(x[d], c3[d], d3);
    }
    float e0 = __builtin_fmaf(-2.0f, d0, nb[c + 0]);
    float e1 = __builtin_fmaf(-2.0f, d1, nb[c + 1]);
    float e2 = __builtin_fmaf(-2.0f, d2, nb[c + 2]);
    float e3 = __builtin_fmaf(-2.0f, d3, nb[c + 3]);
    if (c == 0 || e0 < bd) { bd = e0; best = c; }
    if (e1 < bd) { bd = e1; best = c + 1; }
    if (e2 < bd) { bd = e2; best = c + 2; }
    if (e3 < bd) { bd = e3; best = c + 3; }
  }
  for (; c < k; ++c) {
    const float* cc = cb + c * D;
    float d0 = 0.f;
#pragma unroll
    for (int d = 0; d < D; ++d) d0 = __builtin_fmaf(x[d], cc[d], d0);
    float e0 = __builtin_fmaf(-2.0f, d0, nb[c]);
    if (c == 0 || e0 < bd) { bd = e0; best = c; }
  }
  return best;
}

template <int D>
VC_DEV void load_row_f32(const uint16_t* row, float (&x)[D]) {
#pragma unroll
  for (int c8 = 0; c8 < D / 8; ++c8) {
    uint4 w = ((const uint4*)row)[c8];
    x[8 * c8 + 0] = bf16_lo(w.x);
    x[8 * c8 + 1] = bf16_hi(w.x);
    x[8 * c8 + 2] = bf16_lo(w.y);
    x[8 * c8 + 3] = bf16_hi(w.y);
    x[8 * c8 + 4] = bf16_lo(w.z);
    x[8 * c8 + 5] = bf16_hi(w.z);
    x[8 * c8 + 6] = bf16_lo(w.w);
    x[8 * c8 + 7] = bf16_hi(w.w);
  }
}

// A reduction over the four lane groups l, l^16, l^32, l^48 (the lanes that
// hold one token's MFMA outputs): row swaps of 16, then of 32 lanes.
template <class F>
VC_DEV u32 over_groups(u32 x, F f) {
  auto p16 = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = f(p16[0], p16[1]);
  auto p32 = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return f(p32[0], p32[1]);
}

// Forgy initialisation, centroids, norms; zero the accumulators.
template <int D>
__global__ __launch_bounds__(256) void group_init(const uint16_t* __restrict__ v, int64_t sB, int64_t sS, int64_t sH,
                                                  int S, int H, int k, uint64_t seed, int warm,
                                                  float* __restrict__ cent, GroupWs ws) {
  __shared__ int idx[256];
  __shared__ float cl[8192];  // the k x D centroids (k D <= 8192)
  const int h = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
  const int64_t bh = (int64_t)b * H + h;
  float* cb = cent + bh * k * D;
  for (int e = t; e < k * D; e += 256) ws.sums[bh * k * D + e] = 0;
  for (int e = t; e < k; e += 256) ws.counts[bh * k + e] = 0;
  for (int e = t; e < D; e += 256) ws.r_amax[bh * D + e] = 0u;
  if (warm) {
    // warm start: the caller's centroids are the first iterate
    for (int e = t; e < k * D; e += 256) cl[e] = cb[e];
  } else {
    if (t < 64) {
      // partial Fisher-Yates over the identity [0, S), the touched positions
      // kept in a small map (position -> value) spread over wave 0's lanes:
      // entry e in lane e % 64, slot e / 64 (at most 2 k <= 256 entries);
      // each lookup is one compare per slot and a ballot
      constexpr int NS = 4;
      int pos[NS], val[NS];
#pragma unroll
      for (int m = 0; m < NS; ++m) pos[m] = val[m] = -1;
      const int lane = t;
      int n = 0;
      // the draws need no map: SplitMix64's i-th output depends only on its
      // counter, so lane i computes draws i and 64 + i (k <= 128) up front
      const uint64_t st0 = seed + 0x9E3779B97F4A7C15ull * (uint64_t)(1 + bh);
      int jl[2] = {0, 0};
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int i = 64 * hh + lane;
        if (i < k) {
          uint64_t st = st0 + 0x9E3779B97F4A7C15ull * (uint64_t)i;
          const uint64_t r = splitmix64_next(st);
          jl[hh] = i + (int)(((r >> 32) * (uint64_t)(unsigned)(S - i)) >> 32);
        }
      }
      for (int i = 0; i < k; ++i) {
        const int j = i < 64 ? __shfl(jl[0], i) : __shfl(jl[1], i - 64);
        int ei = -1, ej = -1, ai = i, aj = j;
#pragma unroll
        for (int m = 0; m < NS; ++m) {
          const unsigned long long bi = __ballot(pos[m] == i), bj = __ballot(pos[m] == j);
          if (bi) {
            const int L = __builtin_ctzll(bi);
            ei = 64 * m + L;
            ai = __shfl(val[m], L);
          }
          if (bj) {
            const int L = __builtin_ctzll(bj);
            ej = 64 * m + L;
            aj = __shfl(val[m], L);
          }
        }
        if (ei < 0) {
          ei = n++;
#pragma unroll
          for (int m = 0; m < NS; ++m)
            if (ei == 64 * m + lane) pos[m] = i;
        }
        if (ej < 0 && j != i) {
          ej = n++;
#pragma unroll
          for (int m = 0; m < NS; ++m)
            if (ej == 64 * m + lane) pos[m] = j;
        }
#pragma unroll
        for (int m = 0; m < NS; ++m) {
          if (ei == 64 * m + lane) val[m] = aj;
          if (j != i && ej == 64 * m + lane) val[m] = ai;
        }
        if (lane == 0) idx[i] = aj;
      }
    }
    __syncthreads();
    const uint16_t* vb = v + b * sB + h * sH;
    constexpr int CPR = D / 8;  // 16-byte chunks per row
    for (int q = t; q < k * CPR; q += 256) {
      const int c = q / CPR, u = q % CPR;
      float x[8];
      unpack8(*(const uint4*)(vb + (int64_t)idx[c] * sS + 8 * u), x);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        cb[c * D + 8 * u + e] = x[e];
        cl[c * D + 8 * u + e] = x[e];
      }
    }
  }
  __syncthreads();
  // norms: one fmaf chain per centroid over d = 0..D-1, from LDS
  for (int c = t; c < k; c += 256) {
    float n2 = 0.0f;
    for (int d = 0; d < D; ++d) n2 = __builtin_fmaf(cl[c * D + d], cl[c * D + d], n2);
    ws.norms[bh * k + c] = n2;
  }
}

// Zeroes the per-channel residual amax of each (b, h): the only state the
// gather/means/residual passes need when the permutation is given.
__global__ __launch_bounds__(256) void amax_reset(int D, GroupWs ws) {
  const int64_t bh = blockIdx.x;
  for (int e = threadIdx.x; e < D; e += 256) ws.r_amax[bh * D + e] = 0u;
}

// Assignment on the matrix cores, with the exact rule's result.
//
// Every centroid component c is split into two bf16 parts, hi = bf16(c) and
// mid = bf16(c - hi) (c - hi is exact in fp32), so |c - hi - mid| <= 2^-16 |c|
// and bf16 products x_d * part are exact: v_mfma_f32_16x16x32_bf16 sums the
// 2D products of q ~ x . c in fp32.  However the matrix core orders and
// rounds that sum, it stays within gamma_{2D+8}(2^-23) (1 + 2^-6) S of
// x . (hi + mid), S = sum_d |x_d c_d| <= |x| |c| (each addition off by at
// most 2^-23 relative), and the dropped part adds at most 2^-16 S; the
// oracle's fmaf chain p stays within gamma_D(2^-24) S of x . c.  With
// a = fl(|c|^2 - 2q) and e the exact rule's fl(|c|^2 - 2p), for D <= 128
//   |a_c - e_c| <= 1.10e-4 |x| |c| + 2^-23 |a_c| + 2^-121.5 |x| + 2^-118
// (the last two terms: mid parts below the smallest normal bf16, 2^-126,
// and tiny products, should the matrix core flush them: at most
// 2 sum_d |x_d| 2^-126 <= 2 sqrt(D) |x| 2^-126 and 2D 2^-126), and the
// kernel takes more than that, twice the first two terms,
//   beta_c = |x| (|c| 1.0625 2^-12 + 2^-120) + |a_c| 2^-22 + 2^-96,
// with |x| and |c| rounded up.  The exact argmin c* then has
// a_c* - beta_c* <= e_c* <= e_c <= a_c + beta_c for every c, so it lies in
// {c : a_c - beta_c <= min_c' (a_c' + beta_c')}.  A token whose set has one
// member takes it; the others go on the workgroup's list in LDS and are
// settled at its end with the exact rule over their candidates only.
//
// Work: 512 threads, kAssignTokens tokens per workgroup; wave w takes 16 TBW
// tokens per step; lane (g, lr) loads channels 32 kc + 8 g .. + 7 of token
// 16 tb + lr (the B operand) and, after the products, holds centroids
// 16 cb + 4 g + v of that token.  Labels go to LDS, and the settled tokens'
// rows into the member sums (below) in the same step.
template <int D, int NCB>
__global__ __launch_bounds__(512) void kmeans_assign_mx(const uint16_t* __restrict__ v, int64_t sB, int64_t sS,
                                                        int64_t sH, int S, int H, int k,
                                                        const float* __restrict__ cent, int32_t* __restrict__ labels,
                                                        GroupWs ws, int last, int nchunk) {
  constexpr int NKC = D / 32;             // 32-channel chunks
  constexpr int NF = NCB * NKC * 2;       // A fragments (centroid block, chunk, part)
  constexpr int TBW = NCB <= 4 ? 4 : 2;   // 16-token blocks per wave step
  constexpr int KP = 16 * NCB;            // centroids, padded
  constexpr int LD = D + 1;               // member-sum row stride (bank spread)
  constexpr int NIT = kAssignTokens / (8 * 16 * TBW);
  constexpr int NW = (KP + 31) / 32;      // 32-bit words of a candidate set
  __shared__ uint4 cfrag[NF * 64];
  __shared__ unsigned long long lsum[KP * LD];
  __shared__ int lcnt[KP];
  __shared__ __attribute__((aligned(16))) float lnrm[KP], lbc[KP];
  // every token's label (k <= 255; kOpen while a token is open)
  __shared__ __attribute__((aligned(16))) unsigned char lbl[kAssignTokens];
  __shared__ unsigned short otok[kAssignTokens];  // open tokens (offset in the workgroup's range)
  __shared__ u32 omask[kAssignTokens * NW];       // and their candidate sets
  __shared__ unsigned lmisc[2];                   // max |c|^2 (bits), open-list length
  constexpr int NCH = kAssignTokens / kChunk;
  static_assert(kAssignTokens % kChunk == 0, "whole histogram chunks per workgroup");
  __shared__ int hcnt[NCH][KP];                   // last pass: label counts per 256-token chunk
  __shared__ uint4 stage[8][16 * (D / 8)];        // per wave: one 16-token block of rows
  // heads vary fastest over the grid: the workgroups running at one time
  // read whole [H, D] stripes of the token-major value tensor
  const int h = blockIdx.x, b = blockIdx.z, t = threadIdx.x;
  const int l = t & 63, lr = l & 15, g = l >> 4, w = t >> 6;
  const int64_t bh = (int64_t)b * H + h;
  const int base = blockIdx.y * kAssignTokens;
  const float* __restrict__ cb = cent + bh * k * D;
  for (int e = t; e < KP * LD; e += 512) lsum[e] = 0ull;
  for (int e = t; e < NCH * KP; e += 512) (&hcnt[0][0])[e] = 0;
  for (int c = t; c < KP; c += 512) {
    lcnt[c] = 0;
    const float n2 = c < k ? ws.norms[bh * k + c] : INFINITY;  // padded centroids never win
    lnrm[c] = n2;
    // >= |c| times the bound's factor, plus the flush allowance
    lbc[c] = __builtin_fmaf(__builtin_sqrtf(n2) * (1.0f + 0x1p-10f), 0x1.1p-12f, 0x1p-120f);
  }
  if (t < 2) lmisc[t] = 0u;
  for (int q = t; q < KP * (D / 8); q += 512) {
    const int c = q / (D / 8), u = q % (D / 8);  // centroid c, channels 8u .. 8u + 7
    u32 pw[2][4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      u32 lo16[2], hi16[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const float x = c < k ? cb[c * D + 8 * u + e + j] : 0.f;
        const uint16_t p0 = f32_to_bf16(x);
        const uint16_t p1 = f32_to_bf16(x - bf16_to_f32(p0));
        (j ? hi16 : lo16)[0] = p0;
        (j ? hi16 : lo16)[1] = p1;
      }
#pragma unroll
      for (int part = 0; part < 2; ++part) pw[part][e / 2] = lo16[part] | (hi16[part] << 16);
    }
    const int lane = (u & 3) * 16 + (c & 15);
#pragma unroll
    for (int part = 0; part < 2; ++part)
      cfrag[(((c >> 4) * NKC + (u >> 2)) * 2 + part) * 64 + lane] =
          make_uint4(pw[part][0], pw[part][1], pw[part][2], pw[part][3]);
  }
  __syncthreads();
  const uint16_t* vb = v + b * sB + h * sH;
  const u32 rowB = (u32)(2 * sS);  // bytes per token (below 2^31: checked at the boundary)
  const v4f zero4 = {0.f, 0.f, 0.f, 0.f};

  // Member sums, taken while the labels are made, from the rows already in
  // registers (V is read once).  Lanes form groups of D / 8 (lane c of a
  // group holds channels 8 c .. 8 c + 7 of a token); a group adds its tokens
  // into 64-bit fixed-point registers and moves them to the cluster's LDS
  // row only where the label changes.  A 16-token block reaches the groups
  // through a wave-private LDS stage: chunk q (channels 8 q .. 8 q + 7) of
  // row r sits at q ^ (r mod D / 8), so both the stage's writes and its
  // reads hit distinct banks.  In an LDS sum row, channel 8 c + e sits at
  // 8 c + ((e + c / 2) & 7): the 16 lanes of one flush hit 16 distinct bank
  // pairs.  Open tokens are added once settled.  Fixed-point sums are exact,
  // so the order of the additions does not matter.
  constexpr int LPT = D / 8;     // lanes per token
  constexpr int GPW = 64 / LPT;  // token groups per wave
  constexpr int TPG = 16 / GPW;  // tokens of a 16-token block per group
  const int grp = l / LPT, c = l % LPT;
  uint4* const stg = &stage[w][0];
  int cur = -1, run = 0;
  long long sacc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) sacc[e] = 0;
  auto flush = [&]() {
    unsigned long long* ls = lsum + cur * LD + 8 * c;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      atomicAdd(&ls[(e + (c >> 1)) & 7], (unsigned long long)sacc[e]);
      sacc[e] = 0;
    }
    if (c == 0) atomicAdd(&lcnt[cur], run);
    run = 0;
  };
  // one token's 8 channels of this lane, labelled L
  auto add_row = [&](const uint4& row, int L) {
    if (L != cur) {
      if (cur >= 0) flush();
      cur = L;
    }
    const u32 wd[4] = {row.x, row.y, row.z, row.w};
    u32 mx = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) mx = max(mx, max(wd[q] & 0x7fffu, (wd[q] >> 16) & 0x7fffu));
    if (mx < 0x4300u) {  // |x| < 128: the exponent shortcut
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        sacc[2 * q] += fx24_small(wd[q] & 0xffffu);
        sacc[2 * q + 1] += fx24_small(wd[q] >> 16);
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        sacc[2 * q] += fx24(bf16_lo(wd[q]));
        sacc[2 * q + 1] += fx24(bf16_hi(wd[q]));
      }
    }
    ++run;
  };

  for (int it = 0; it < NIT; ++it) {
    const int t0 = base + (it * 8 + w) * 16 * TBW;
    if (t0 >= S) break;
    uint4 xw[TBW][NKC];
#pragma unroll
    for (int tb = 0; tb < TBW; ++tb) {
      const uint16_t* row = token_row(vb, min(t0 + 16 * tb + lr, S - 1), rowB);  // rows past S: discarded
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) xw[tb][kc] = *(const uint4*)(row + 32 * kc + 8 * g);
    }
    v4f acc[NCB][TBW];
#pragma unroll
    for (int cbk = 0; cbk < NCB; ++cbk)
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
        for (int part = 0; part < 2; ++part) {
          const v8bf af = __builtin_bit_cast(v8bf, cfrag[((cbk * NKC + kc) * 2 + part) * 64 + l]);
#pragma unroll
          for (int tb = 0; tb < TBW; ++tb)
            acc[cbk][tb] = mfma_bf16(af, __builtin_bit_cast(v8bf, xw[tb][kc]),
                                     (kc == 0 && part == 0) ? zero4 : acc[cbk][tb]);
        }
#pragma unroll
    for (int tb = 0; tb < TBW; ++tb) {
      // |x|^2 straight from the packed pairs (v_dot2c_f32_bf16: exact bf16
      // products, within a relative 2^-19 of the square norm over the 16
      // accumulations; the factor 1 + 2^-10 below covers it, and 2^-59 any
      // squares below the smallest normal that the instruction may flush)
      float x2 = 0.f;
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        const u32 wd[4] = {xw[tb][kc].x, xw[tb][kc].y, xw[tb][kc].z, xw[tb][kc].w};
#pragma unroll
        for (int q = 0; q < 4; ++q)
          x2 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2bf, wd[q]), __builtin_bit_cast(v2bf, wd[q]), x2,
                                               false);
      }
      x2 = __uint_as_float(over_groups(__float_as_uint(x2), [](u32 x, u32 y) {
        return __float_as_uint(__uint_as_float(x) + __uint_as_float(y));
      }));
      const float xn = __builtin_fmaf(__builtin_sqrtf(x2), 1.0f + 0x1p-10f, 0x1p-59f);  // >= |x|
      float a[NCB][4], lo[NCB][4];
      float hmin = INFINITY;
#pragma unroll
      for (int cbk = 0; cbk < NCB; ++cbk) {
        const float4 bc = *(const float4*)&lbc[16 * cbk + 4 * g];
        const float4 nc = *(const float4*)&lnrm[16 * cbk + 4 * g];
        const float bcv[4] = {bc.x, bc.y, bc.z, bc.w}, ncv[4] = {nc.x, nc.y, nc.z, nc.w};
#pragma unroll
        for (int vv = 0; vv < 4; ++vv) {
          a[cbk][vv] = __builtin_fmaf(-2.0f, acc[cbk][tb][vv], ncv[vv]);
          const float beta = __builtin_fmaf(fabsf(a[cbk][vv]), 0x1p-22f, __builtin_fmaf(xn, bcv[vv], 0x1p-96f));
          lo[cbk][vv] = a[cbk][vv] - beta;  // NaN for padded centroids: never a candidate
          hmin = fminf(hmin, a[cbk][vv] + beta);
        }
      }
      hmin = __uint_as_float(over_groups(__float_as_uint(hmin), [](u32 x, u32 y) {
        return __float_as_uint(fminf(__uint_as_float(x), __uint_as_float(y)));
      }));
      // candidate set as bits c = 16 cb + 4 g + v, word c / 32
      u32 cm[NW];
#pragma unroll
      for (int q = 0; q < NW; ++q) cm[q] = 0u;
#pragma unroll
      for (int cbk = 0; cbk < NCB; ++cbk)
#pragma unroll
        for (int vv = 0; vv < 4; ++vv)
          if (lo[cbk][vv] <= hmin) cm[cbk / 2] |= 1u << ((16 * cbk + 4 * g + vv) & 31);
      int cnt = 0;
#pragma unroll
      for (int q = 0; q < NW; ++q) {
        cm[q] = over_groups(cm[q], [](u32 x, u32 y) { return x | y; });
        cnt += __builtin_popcount(cm[q]);
      }
      int idx = -1;
#pragma unroll
      for (int q = NW - 1; q >= 0; --q)
        if (cm[q]) idx = 32 * q + __builtin_ctz(cm[q]);
      const int tok = t0 + 16 * tb + lr;
      const bool decided = cnt == 1 && idx < k;
      if (tok < S && g == 0) {
        if (decided) {
          labels[bh * S + tok] = idx;
          lbl[tok - base] = (unsigned char)idx;
        } else {
          lbl[tok - base] = kOpen;
          const unsigned slot = atomicAdd(&lmisc[1], 1u);
          otok[slot] = (unsigned short)(tok - base);
#pragma unroll
          for (int q = 0; q < NW; ++q) omask[slot * NW + q] = cm[q];
        }
      }
      // the block's settled tokens into the member sums, through the stage
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) stg[lr * LPT + ((4 * kc + g) ^ (lr & (LPT - 1)))] = xw[tb][kc];
      // all of this group's labels (one LDS read) and rows first, then the sums
      const int r0 = TPG * grp, tk0 = t0 + 16 * tb + r0;
      const u32 lw = TPG == 4 ? *(const u32*)&lbl[tk0 - base] : (u32)*(const uint16_t*)&lbl[tk0 - base];
      uint4 rows[TPG];
#pragma unroll
      for (int j = 0; j < TPG; ++j) rows[j] = stg[(r0 + j) * LPT + (c ^ ((r0 + j) & (LPT - 1)))];
#pragma unroll
      for (int j = 0; j < TPG; ++j) {
        const int L = (int)((lw >> (8 * j)) & 0xffu);
        if (L != kOpen && tk0 + j < S) add_row(rows[j], L);  // not open, not past S
      }
    }
  }
  __syncthreads();
  // the open tokens: the exact rule over each one's candidates, in increasing
  // cluster index so that ties still go to the lowest
  const int nopen = (int)lmisc[1];
  const float* __restrict__ nb = ws.norms + bh * k;
  for (int i = t; i < nopen; i += 512) {
    const int tok = base + otok[i];
    float x[D];
    load_row_f32<D>(vb + (int64_t)tok * sS, x);
    int best = -1;
    float bd = 0.0f;
    for (int q = 0; q < NW; ++q) {
      u32 mk = omask[i * NW + q];
      while (mk) {
        const int c = 32 * q + __builtin_ctz(mk);
        mk &= mk - 1;
        if (c >= k) break;
        float d0 = 0.f;
#pragma unroll
        for (int d = 0; d < D; ++d) d0 = __builtin_fmaf(x[d], cb[c * D + d], d0);
        const float e0 = __builtin_fmaf(-2.0f, d0, nb[c]);
        if (best < 0 || e0 < bd) {
          bd = e0;
          best = c;
        }
      }
    }
    if (best < 0) best = exact_label<D>(x, cb, nb, k);  // an empty set cannot happen; stay exact regardless
    labels[bh * S + tok] = best;
    lbl[tok - base] = (unsigned char)best;
  }
  __syncthreads();
  // last pass: the label histogram of each 256-token chunk (the counting
  // sort's first step), written out after the next barrier
  if (last)
    for (int i = t; i < kAssignTokens && base + i < S; i += 512) atomicAdd(&hcnt[i / kChunk][lbl[i]], 1);
  // the open tokens' rows, now that their labels are settled
  for (int i = w * GPW + grp; i < nopen; i += 8 * GPW) {
    const int off = otok[i];
    add_row(*(const uint4*)token_row(vb + 8 * c, base + off, rowB), lbl[off]);
  }
  if (cur >= 0) flush();
  __syncthreads();
  unsigned long long* gs = (unsigned long long*)ws.sums + bh * k * D;
  for (int e = t; e < k * D; e += 512) {
    const int ch = e % D, cc = ch >> 3;  // channel 8 cc + (ch & 7) sits at 8 cc + ((ch + cc / 2) & 7)
    if (lcnt[e / D] > 0) atomicAdd(&gs[e], lsum[(e / D) * LD + 8 * cc + (((ch & 7) + (cc >> 1)) & 7)]);
  }
  for (int e = t; e < k; e += 512)
    if (lcnt[e] > 0) atomicAdd((unsigned long long*)&ws.counts[bh * k + e], (unsigned long long)lcnt[e]);
  if (last)
    for (int e = t; e < NCH * k; e += 512) {
      const int i = e / k, c = e % k, ch = blockIdx.y * NCH + i;
      if (ch < nchunk) ws.hist[(bh * k + c) * nchunk + ch] = hcnt[i][c];
    }
}

// Member means (empty clusters keep their centroid), norms, reset sums and
// counts: CPW centroids per workgroup, every element's loads issued at once.
constexpr int kUpdCentroids = 8;
template <int D>
__global__ __launch_bounds__(256) void kmeans_update(int k, float* __restrict__ cent, GroupWs ws) {
  constexpr int CPW = kUpdCentroids, PER = CPW * D / 256;
  __shared__ float cl[CPW * D];
  const int64_t bh = blockIdx.y;
  const int c0 = blockIdx.x * CPW, t = threadIdx.x;
  const int nc = min(CPW, k - c0);
  float* cb = cent + (bh * k + c0) * D;
  long long* sb = ws.sums + (bh * k + c0) * D;
  long long* nb = ws.counts + bh * k + c0;
  long long n[PER], sv[PER];
  float old[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = t + 256 * i;
    const bool in = e < nc * D;
    n[i] = in ? nb[e / D] : 0;
    sv[i] = in ? sb[e] : 0;
    old[i] = in ? cb[e] : 0.0f;
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = t + 256 * i;
    if (e < nc * D) {
      const float c = n[i] > 0 ? fx24_mean(sv[i], n[i]) : old[i];
      cb[e] = c;
      cl[e] = c;
      sb[e] = 0;
    }
  }
  __syncthreads();  // every count of this workgroup's centroids has been read
  if (t < nc) {
    float n2 = 0.0f;
    for (int d = 0; d < D; ++d) n2 = __builtin_fmaf(cl[t * D + d], cl[t * D + d], n2);
    ws.norms[bh * k + c0 + t] = n2;
    nb[t] = 0;
  }
}

// Exclusive scan of hist[bh] in (label, chunk) order, in place: tiles of
// 8192 counts go through LDS with coalesced loads and stores; each thread
// scans 8 consecutive counts, the 1024 partial sums are scanned in LDS, and
// the running total carries to the next tile.
__global__ __launch_bounds__(1024) void hist_scan(int k, int nchunk, GroupWs ws) {
  constexpr int PER = 8, TILE = 1024 * PER;
  __shared__ int tile[TILE];
  __shared__ int part[1024];
  const int64_t bh = blockIdx.x;
  const int t = threadIdx.x;
  int* hb = ws.hist + bh * k * nchunk;
  const int E = k * nchunk;
  int carry = 0;
  for (int b0 = 0; b0 < E; b0 += TILE) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = b0 + t + 1024 * i;
      tile[t + 1024 * i] = e < E ? hb[e] : 0;
    }
    __syncthreads();
    int s = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) s += tile[PER * t + j];
    part[t] = s;
    __syncthreads();
    for (int o = 1; o < 1024; o <<= 1) {
      const int x = t >= o ? part[t - o] : 0;
      __syncthreads();
      part[t] += x;
      __syncthreads();
    }
    int run = carry + part[t] - s;  // exclusive prefix of this thread's 8 counts
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int c = tile[PER * t + j];
      tile[PER * t + j] = run;
      run += c;
    }
    carry += part[1023];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = b0 + t + 1024 * i;
      if (e < E) hb[e] = tile[t + 1024 * i];
    }
    __syncthreads();  // the tile is reused
  }
}

__global__ __launch_bounds__(256) void label_scatter(const int32_t* __restrict__ labels, int S, int H, int k,
                                                     int nchunk, GroupWs ws, int32_t* __restrict__ perm) {
  __shared__ int wcnt[4][256];
  const int h = blockIdx.y, b = blockIdx.z, t = threadIdx.x, ch = blockIdx.x;
  const int w = t >> 6, lane = t & 63;
  const int64_t bh = (int64_t)b * H + h;
  for (int e = t; e < 4 * 256; e += 256) (&wcnt[0][0])[e] = 0;
  __syncthreads();
  const int tok = ch * kChunk + t;
  const bool valid = tok < S;
  const int L = valid ? labels[bh * S + tok] : 0;
  // lanes of this wave holding the same (valid) label
  unsigned long long same = __ballot(valid);
#pragma unroll
  for (int bit = 0; bit < 8; ++bit) {
    unsigned long long bal = __ballot((L >> bit) & 1);
    same &= ((L >> bit) & 1) ? bal : ~bal;
  }
  const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int rank_w = __popcll(same & lt);
  if (valid && rank_w == 0) wcnt[w][L] = __popcll(same);
  __syncthreads();
  if (valid) {
    int rank = rank_w;
    for (int w2 = 0; w2 < w; ++w2) rank += wcnt[w2][L];
    perm[bh * S + ws.hist[(bh * k + L) * nchunk + ch] + rank] = tok;
  }
}

// A gathered token index, clamped into [0, S) (negative values to 0).
VC_DEV int clamp_tok(int t, int S) { return min(max(t, 0), S - 1); }

template <int D>
struct ApplyMap {
  static constexpr int CPR = D / 8;         // 16-byte chunks per row
  static constexpr int RG = 256 / CPR;      // row groups
  static constexpr int RPT = kBlk / RG;     // rows per thread
};

// Pass 1: gather K and V by pi; K' per-block codes; block means; residual
// per-channel maxima.  PREP: the key preprocessing is on.  Without it every
// K and V row of the tile is loaded up front, raw, in one round trip; with
// it the keys are transformed in fp32 first and V follows.
template <int D, bool PREP>
__global__ __launch_bounds__(256) void group_apply1(const uint16_t* __restrict__ kx, int64_t kB, int64_t kS,
                                                    int64_t kH, const uint16_t* __restrict__ vx, int64_t vB,
                                                    int64_t vS, int64_t vH, int S, int H, int nblk,
                                                    const int32_t* __restrict__ perm, uint8_t* __restrict__ k8,
                                                    float* __restrict__ k_scale, uint16_t* __restrict__ mu_bf16,
                                                    GroupWs ws, PrepArgs pp) {
  using Mp = ApplyMap<D>;
  // partial sums and maxima, row group x channel; a lane's 8 channels sit
  // 16 apart (slot e * CPR + ch for channel 8 ch + e) so that the lanes of a
  // row group write consecutive words, and the rows are padded so that the
  // row groups of one wave start in different banks
  constexpr int PW = D + 16;
  __shared__ long long psum[Mp::RG][PW];
  __shared__ float pmax[Mp::RG][PW];
  __shared__ float red[4];
  __shared__ float mu_l[D];
  const int j = blockIdx.x, h = blockIdx.y, b = blockIdx.z, t = threadIdx.x;
  const int64_t bh = (int64_t)b * H + h;
  const int ch = t % Mp::CPR, rg = t / Mp::CPR;
  const int nvalid = min(kBlk, S - j * kBlk);
  // perm may be the caller's (VC_GROUP_REUSE_PERM): every gathered index is
  // clamped into [0, S), so a malformed permutation gives wrong codes, never
  // an access outside K, V or the RoPE tables.  Rows past the end of a
  // ragged last tile load the tile's last row and count as zero.
  int tok[Mp::RPT];
  bool ok[Mp::RPT];
#pragma unroll
  for (int r = 0; r < Mp::RPT; ++r) {
    const int row = rg * Mp::RPT + r;
    ok[r] = row < nvalid;
    tok[r] = clamp_tok(perm[bh * S + j * kBlk + min(row, nvalid - 1)], S);
  }
  const uint16_t* kb = kx + b * kB + h * kH;
  const uint16_t* vb = vx + b * vB + h * vH;
  uint4 vr[Mp::RPT];
  // ---- K' = K[pi], per-block E4M3 ----
  // With preprocessing ([VC] App. B: centring statistics, RoPE, gather,
  // Hadamard, mean subtraction), each gathered key is rotated at its original
  // position, centred by the head's channel mean and transformed, as in
  // vc_quantize's K path, before the block scale is taken.
  {
    uint8_t* kd = k8 + (bh * nblk * kBlk + (int64_t)j * kBlk) * D;
    auto store_codes = [&](int r, const float (&x)[8], float inv) {
      uint2 c;
      c.x = cvt4_fp8(x[0] * inv, x[1] * inv, x[2] * inv, x[3] * inv);
      c.y = cvt4_fp8(x[4] * inv, x[5] * inv, x[6] * inv, x[7] * inv);
      *(uint2*)(kd + kpack_off<D>(rg * Mp::RPT + r, ch >> 1) + (ch & 1) * 8) = c;
    };
    auto block_scale = [&](float m) {
      m = wave_max(m);
      if ((t & 63) == 0) red[t >> 6] = m;
      __syncthreads();
      m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
      // power-of-two block scale, as for vc_quantize's K
      const int e = pow2_block_exp(m);
      if (t == 0) k_scale[bh * nblk + j] = ldexpf(1.0f, e);
      return ldexpf(1.0f, -e);
    };
    if constexpr (!PREP) {
      uint4 kr[Mp::RPT];
#pragma unroll
      for (int r = 0; r < Mp::RPT; ++r) kr[r] = *(const uint4*)(kb + (int64_t)tok[r] * kS + ch * 8);
#pragma unroll
      for (int r = 0; r < Mp::RPT; ++r) vr[r] = *(const uint4*)(vb + (int64_t)tok[r] * vS + ch * 8);
      float m = 0.0f;
#pragma unroll
      for (int r = 0; r < Mp::RPT; ++r) {
        if (!ok[r]) kr[r] = make_uint4(0, 0, 0, 0);
        float x[8];
        unpack8(kr[r], x);
#pragma unroll
        for (int e2 = 0; e2 < 8; ++e2) m = fmaxf(m, fabsf(x[e2]));
      }
      const float inv = block_scale(m);
#pragma unroll
      for (int r = 0; r < Mp::RPT; ++r) {
        float x[8];
        unpack8(kr[r], x);
        store_codes(r, x, inv);
      }
    } else {
      float kv[Mp::RPT][8];
      float cm[8];
      if (pp.flags & kPrepCenter) {
#pragma unroll
        for (int e2 = 0; e2 < 8; ++e2) cm[e2] = fx24_mean_of(pp.ksum[bh * D + ch * 8 + e2], S);
      }
      float m = 0.0f;
#pragma unroll
      for (int r = 0; r < Mp::RPT; ++r) {
        unpack8(ok[r] ? *(const uint4*)(kb + (int64_t)tok[r] * kS + ch * 8) : make_uint4(0, 0, 0, 0), kv[r]);
        if (ok[r]) {
          if (pp.flags & kPrepRope)
            rope8(kv[r], pp.cs + (int64_t)tok[r] * (D / 2) + ch * 4, pp.sn + (int64_t)tok[r] * (D / 2) + ch * 4);
          if (pp.flags & kPrepCenter)
#pragma unroll
            for (int e2 = 0; e2 < 8; ++e2) kv[r][e2] -= cm[e2];
        }
        if (pp.flags & kPrepHadamard) fwht_row8<Mp::CPR>(kv[r], ch);  // every lane of the row takes part
#pragma unroll
        for (int e2 = 0; e2 < 8; ++e2) m = fmaxf(m, fabsf(kv[r][e2]));
      }
      const float inv = block_scale(m);
#pragma unroll
      for (int r = 0; r < Mp::RPT; ++r) store_codes(r, kv[r], inv);
#pragma unroll
      for (int r = 0; r < Mp::RPT; ++r) vr[r] = *(const uint4*)(vb + (int64_t)tok[r] * vS + ch * 8);
    }
  }
  // ---- V' block mean ----
#pragma unroll
  for (int r = 0; r < Mp::RPT; ++r)
    if (!ok[r]) vr[r] = make_uint4(0, 0, 0, 0);
  {
    long long ps[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    u32 mx = 0;
#pragma unroll
    for (int r = 0; r < Mp::RPT; ++r) {
      const u32 wd[4] = {vr[r].x, vr[r].y, vr[r].z, vr[r].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) mx = max(mx, max(wd[q] & 0x7fffu, (wd[q] >> 16) & 0x7fffu));
    }
    if (mx < 0x4300u) {  // every |x| < 128: the exponent shortcut
#pragma unroll
      for (int r = 0; r < Mp::RPT; ++r) {
        const u32 wd[4] = {vr[r].x, vr[r].y, vr[r].z, vr[r].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          ps[2 * q] += fx24_small(wd[q] & 0xffffu);
          ps[2 * q + 1] += fx24_small(wd[q] >> 16);
        }
      }
    } else {
#pragma unroll
      for (int r = 0; r < Mp::RPT; ++r) {
        float x[8];
        unpack8(vr[r], x);
#pragma unroll
        for (int e = 0; e < 8; ++e) ps[e] += fx24(x[e]);
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) psum[rg][e * Mp::CPR + ch] = ps[e];
  }
  __syncthreads();
  if (t < D) {
    // thread t sums slot t: channel 8 (t % CPR) + t / CPR
    const int c = (t % Mp::CPR) * 8 + t / Mp::CPR;
    long long s = 0;
    for (int q = 0; q < Mp::RG; ++q) s += psum[q][t];
    uint16_t mb = f32_to_bf16(fx24_mean(s, nvalid));
    mu_bf16[(bh * nblk + j) * D + c] = mb;
    mu_l[c] = bf16_to_f32(mb);
  }
  __syncthreads();
  // ---- residual channel maxima ----
  {
    float pm[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int r = 0; r < Mp::RPT; ++r)
      if (ok[r]) {
        float x[8];
        unpack8(vr[r], x);
#pragma unroll
        for (int e = 0; e < 8; ++e) pm[e] = fmaxf(pm[e], fabsf(x[e] - mu_l[ch * 8 + e]));
      }
#pragma unroll
    for (int e = 0; e < 8; ++e) pmax[rg][e * Mp::CPR + ch] = pm[e];
  }
  __syncthreads();
  if (t < D) {
    const int c = (t % Mp::CPR) * 8 + t / Mp::CPR;
    float m = 0.0f;
    for (int q = 0; q < Mp::RG; ++q) m = fmaxf(m, pmax[q][t]);
    atomicMax(&ws.r_amax[bh * D + c], __float_as_uint(m));
  }
}

// Pass 2: residual codes in the key-contiguous layout; scaled means as bf16
// (hi, lo) pairs: m = mu * 448 / amax in fp32, hi = bf16(m), lo = bf16(m - hi)
// (both round-half-even; m - hi is exact), stored hi | lo << 16.
template <int D>
__global__ __launch_bounds__(256) void group_apply2(const uint16_t* __restrict__ vx, int64_t vB, int64_t vS,
                                                    int64_t vH, int S, int H, int nblk,
                                                    const int32_t* __restrict__ perm,
                                                    const uint16_t* __restrict__ mu_bf16, GroupWs ws,
                                                    uint8_t* __restrict__ r8, float* __restrict__ r_scale,
                                                    u32* __restrict__ mu_split) {
  using Mp = ApplyMap<D>;
  // the packed tile in LDS, channel-major: channel d's 128 codes in V tile
  // position order at tile[d * LP ...] (rows 16-byte aligned)
  constexpr int LP = kBlk + 16;
  __shared__ __align__(16) uint8_t tile[D * LP];
  __shared__ float inv_l[D], mu_l[D];
  const int j = blockIdx.x, h = blockIdx.y, b = blockIdx.z, t = threadIdx.x;
  const int64_t bh = (int64_t)b * H + h;
  const int ch = t % Mp::CPR, rg = t / Mp::CPR;
  const int nvalid = min(kBlk, S - j * kBlk);
  // every row of the tile in one round trip: indices clamped as in pass 1,
  // rows past the end of a ragged last tile load the tile's last row.  The
  // per-channel loads come first (every lane issues them, so that the wait
  // for them leaves the row loads in flight).
  const int tc = t & (D - 1);
  const u32 amax_bits = ws.r_amax[bh * D + tc];
  const uint16_t mu_bits = mu_bf16[(bh * nblk + j) * D + tc];
  const uint16_t* vb = vx + b * vB + h * vH;
  uint4 w[Mp::RPT];
  {
    int tok[Mp::RPT];
#pragma unroll
    for (int r = 0; r < Mp::RPT; ++r)
      tok[r] = clamp_tok(perm[bh * S + j * kBlk + min(rg * Mp::RPT + r, nvalid - 1)], S);
#pragma unroll
    for (int r = 0; r < Mp::RPT; ++r) w[r] = *(const uint4*)(vb + (int64_t)tok[r] * vS + ch * 8);
  }
  asm volatile("" ::"v"(amax_bits), "v"(mu_bits));  // keeps the two loads ahead of the row loads
  if (t < D) {
    const float m = __uint_as_float(amax_bits);
    float s = 1.0f, inv = 1.0f;
    if (m > 0.0f) {
      s = m / 448.0f;
      inv = 448.0f / m;
    }
    inv_l[t] = inv;
    const float mu = bf16_to_f32(mu_bits);
    mu_l[t] = mu;
    const float ms = mu * inv;
    const uint16_t hi = f32_to_bf16(ms);
    const uint16_t lo = f32_to_bf16(ms - bf16_to_f32(hi));
    mu_split[(bh * nblk + j) * D + t] = (u32)hi | ((u32)lo << 16);
    if (j == 0) r_scale[bh * D + t] = s;
  }
  __syncthreads();
  // codes of this lane's rows (keys 8 rg + r) and channels (8 ch + e):
  // cw[r][0] holds channels 0..3 (byte e = channel e), cw[r][1] channels 4..7
  u32 cw[Mp::RPT][2];
#pragma unroll
  for (int r = 0; r < Mp::RPT; ++r) {
    const float* mu = mu_l + ch * 8;
    const float* iv = inv_l + ch * 8;
    cw[r][0] = cvt4_fp8((bf16_lo(w[r].x) - mu[0]) * iv[0], (bf16_hi(w[r].x) - mu[1]) * iv[1],
                        (bf16_lo(w[r].y) - mu[2]) * iv[2], (bf16_hi(w[r].y) - mu[3]) * iv[3]);
    cw[r][1] = cvt4_fp8((bf16_lo(w[r].z) - mu[4]) * iv[4], (bf16_hi(w[r].z) - mu[5]) * iv[5],
                        (bf16_lo(w[r].w) - mu[6]) * iv[6], (bf16_hi(w[r].w) - mu[7]) * iv[7]);
    if (rg * Mp::RPT + r >= nvalid) cw[r][0] = cw[r][1] = 0;
  }
  // 4 x 4 byte transposes: four rows' words (byte = channel) into four
  // channels' words (byte = row); keys k0 .. k0 + 3 (k0 a multiple of 4)
  // sit at the 4 consecutive tile positions starting at the position of k0
#pragma unroll
  for (int rq = 0; rq < Mp::RPT / 4; ++rq) {
    const int k0 = rg * Mp::RPT + 4 * rq;
    const int p0 = vkey_of_pos(k0);  // the key <-> position swap is its own inverse
#pragma unroll
    for (int cq = 0; cq < 2; ++cq) {
      const u32 x0 = cw[4 * rq][cq], x1 = cw[4 * rq + 1][cq], x2 = cw[4 * rq + 2][cq], x3 = cw[4 * rq + 3][cq];
      const u32 a_lo = __builtin_amdgcn_perm(x1, x0, 0x05010400u), a_hi = __builtin_amdgcn_perm(x1, x0, 0x07030602u);
      const u32 b_lo = __builtin_amdgcn_perm(x3, x2, 0x05010400u), b_hi = __builtin_amdgcn_perm(x3, x2, 0x07030602u);
      const u32 y[4] = {__builtin_amdgcn_perm(b_lo, a_lo, 0x05040100u), __builtin_amdgcn_perm(b_lo, a_lo, 0x07060302u),
                        __builtin_amdgcn_perm(b_hi, a_hi, 0x05040100u), __builtin_amdgcn_perm(b_hi, a_hi, 0x07060302u)};
#pragma unroll
      for (int e = 0; e < 4; ++e) *(u32*)(tile + (ch * 8 + 4 * cq + e) * LP + p0) = y[e];
    }
  }
  __syncthreads();
  uint8_t* ob = r8 + (bh * nblk + j) * (int64_t)D * kBlk;  // packed V tile j
  constexpr int TASKS = D * (kBlk / 16);
#pragma unroll
  for (int i = 0; i < TASKS / 256; ++i) {
    const int task = t + 256 * i, d = task / (kBlk / 16), c = task % (kBlk / 16);
    *(uint4*)(ob + vpack_off(d, c)) = *(const uint4*)(tile + d * LP + 16 * c);
  }
}

template <int D>
hipError_t launch_group_t(const vc_shape& sh, Bshd k, Bshd v, const vc_group_params& p, float* cent, int32_t* labels,
                          int32_t* perm, uint8_t* k8, float* k_scale, uint8_t* r8, float* r_scale,
                          uint16_t* mu_bf16, u32* mu_split, GroupWs ws, PrepArgs pp, hipStream_t st) {
  const int S = sh.S, H = sh.H, B = sh.B, kc = p.clusters;
  const int nblk = (S + kBlk - 1) / kBlk, nchunk = (S + kChunk - 1) / kChunk;
  const int BH = B * H;
  if (p.flags & VC_GROUP_REUSE_PERM) {
    // the caller's permutation: only the gather, block means and residual codes
    amax_reset<<<BH, 256, 0, st>>>(D, ws);
  } else {
    group_init<D><<<dim3(H, B), 256, 0, st>>>(v.p, v.sB, v.sS, v.sH, S, H, kc, p.seed,
                                              (p.flags & VC_GROUP_WARM_START) ? 1 : 0, cent, ws);
    const dim3 ga(H, (S + kAssignTokens - 1) / kAssignTokens, B);
    const int ncb = kc <= 16 ? 1 : kc <= 32 ? 2 : kc <= 64 ? 4 : 8;  // k <= 8192 / D
    auto assign = ncb == 1 ? kmeans_assign_mx<D, 1> : ncb == 2 ? kmeans_assign_mx<D, 2>
                  : ncb == 4 ? kmeans_assign_mx<D, 4> : kmeans_assign_mx<D, (D == 64 ? 8 : 4)>;
    const dim3 gu((kc + kUpdCentroids - 1) / kUpdCentroids, BH);
    for (int it = 0; it < p.iters; ++it) {
      // the last pass also counts each 256-token chunk's labels
      assign<<<ga, 512, 0, st>>>(v.p, v.sB, v.sS, v.sH, S, H, kc, cent, labels, ws, it == p.iters - 1 ? 1 : 0,
                                 nchunk);
      kmeans_update<D><<<gu, 256, 0, st>>>(kc, cent, ws);
    }
    hist_scan<<<BH, 1024, 0, st>>>(kc, nchunk, ws);
    label_scatter<<<dim3(nchunk, H, B), 256, 0, st>>>(labels, S, H, kc, nchunk, ws, perm);
  }
  auto apply1 = pp.flags ? group_apply1<D, true> : group_apply1<D, false>;
  apply1<<<dim3(nblk, H, B), 256, 0, st>>>(k.p, k.sB, k.sS, k.sH, v.p, v.sB, v.sS, v.sH, S, H, nblk, perm, k8, k_scale,
                                           mu_bf16, ws, pp);
  group_apply2<D><<<dim3(nblk, H, B), 256, 0, st>>>(v.p, v.sB, v.sS, v.sH, S, H, nblk, perm, mu_bf16, ws, r8,
                                                    r_scale, mu_split);
  return hipGetLastError();
}

}  // namespace

size_t group_workspace_bytes(const vc_shape& sh, int clusters) {
  size_t total = 0;
  carve(nullptr, sh, clusters, &total);
  return total;
}

hipError_t launch_smooth_group(const vc_shape& sh, Bshd k, Bshd v, const vc_group_params& p, float* centroids,
                               int32_t* labels, int32_t* perm, uint8_t* k8, float* k_scale, uint8_t* r8,
                               float* r_scale, uint16_t* mu_bf16, uint32_t* mu_split, void* ws, PrepArgs pp,
                               hipStream_t st) {
  GroupWs g = carve(ws, sh, p.clusters, nullptr);
  if (sh.D == 128)
    return launch_group_t<128>(sh, k, v, p, centroids, labels, perm, k8, k_scale, r8, r_scale, mu_bf16, mu_split, g,
                               pp, st);
  return launch_group_t<64>(sh, k, v, p, centroids, labels, perm, k8, k_scale, r8, r_scale, mu_bf16, mu_split, g, pp,
                            st);
}

}  // namespace vc
