// vc_group.hip -- V-Smooth grouping on the GPU.
//
// [VC] §3.2 "Value-guided permutation": per (b, h) an online k-means over the
// value tokens gives labels z and pi = argsort(z); K and V are permuted
// together (Eq. 3).  "Block demeaning": each 128-row block of V' loses its
// mean, the residual goes through the per-channel E4M3 value quantiser
// (Eq. 4), and the means are stored divided by the per-channel scale
// (Appendix B).  "Unbalanced clusters cost little": plain Lloyd k-means.
//
// Determinism by construction, so labels / pi / codes are bit-identical to a
// sequential CPU run: every distance is one fp32 fmaf chain over d = 0..D-1
// in a fixed order; cluster and block sums are 64-bit fixed point (24
// fraction bits), which makes atomics order-independent; pi is a stable
// counting sort.
//
// Kernels per call: init (Forgy indices by partial Fisher-Yates on
// SplitMix64, centroids, norms, zeroed accumulators) -> iters x (assign +
// LDS-accumulate, update) -> label histogram -> scan -> stable scatter ->
// apply pass 1 (gather K, V by pi; K' per-block codes; block means; residual
// channel maxima) -> apply pass 2 (residual codes, key-contiguous; scaled
// means).
#include "vc_common.hpp"
#include "vc_launch.hpp"

namespace vc {

namespace {

constexpr int kAssignTokens = 2048;  // tokens per assign workgroup
constexpr int kChunk = 256;          // tokens per histogram / scatter chunk

struct GroupWs {
  long long* sums;     // [BH][k][D]
  long long* counts;   // [BH][k]
  float* norms;        // [BH][k]
  int* hist;           // [BH][k][nchunk]
  unsigned* r_amax;    // [BH][D]
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

// Forgy initialisation, centroids, norms; zero the accumulators.
template <int D>
__global__ __launch_bounds__(256) void group_init(const uint16_t* __restrict__ v, int64_t sB, int64_t sS, int64_t sH,
                                                  int S, int H, int k, uint64_t seed, int warm,
                                                  float* __restrict__ cent, GroupWs ws) {
  __shared__ int mpos[512], mval[512];
  __shared__ int idx[256];
  const int h = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
  const int64_t bh = (int64_t)b * H + h;
  if (warm) {
    // warm start: the caller's centroids are the first iterate
    float* cb = cent + bh * k * D;
    for (int e = t; e < k * D; e += 256) ws.sums[bh * k * D + e] = 0;
    for (int e = t; e < k; e += 256) ws.counts[bh * k + e] = 0;
    for (int e = t; e < D; e += 256) ws.r_amax[bh * D + e] = 0u;
    for (int c = t; c < k; c += 256) {
      float n2 = 0.0f;
      for (int d = 0; d < D; ++d) n2 = __builtin_fmaf(cb[c * D + d], cb[c * D + d], n2);
      ws.norms[bh * k + c] = n2;
    }
    return;
  }
  if (t == 0) {
    // partial Fisher-Yates over the identity [0, S), the touched positions
    // kept in a small map (position -> value)
    int n = 0;
    uint64_t st = seed + 0x9E3779B97F4A7C15ull * (uint64_t)(1 + bh);
    for (int i = 0; i < k; ++i) {
      uint64_t r = splitmix64_next(st);
      int j = i + (int)(((r >> 32) * (uint64_t)(unsigned)(S - i)) >> 32);
      int ei = -1, ej = -1;
      for (int e = 0; e < n; ++e) {
        if (mpos[e] == i) ei = e;
        if (mpos[e] == j) ej = e;
      }
      int ai = ei >= 0 ? mval[ei] : i;
      int aj = ej >= 0 ? mval[ej] : j;
      if (ei < 0) { mpos[n] = i; ei = n++; }
      if (ej < 0 && j != i) { mpos[n] = j; ej = n++; }
      mval[ei] = aj;
      if (j != i) mval[ej] = ai;
      idx[i] = aj;
    }
  }
  __syncthreads();
  const uint16_t* vb = v + b * sB + h * sH;
  float* cb = cent + bh * k * D;
  for (int e = t; e < k * D; e += 256) {
    int c = e / D, d = e % D;
    cb[e] = bf16_to_f32(vb[(int64_t)idx[c] * sS + d]);
  }
  for (int e = t; e < k * D; e += 256) ws.sums[bh * k * D + e] = 0;
  for (int e = t; e < k; e += 256) ws.counts[bh * k + e] = 0;
  for (int e = t; e < D; e += 256) ws.r_amax[bh * D + e] = 0u;
  for (int c = t; c < k; c += 256) {
    float n2 = 0.0f;
    for (int d = 0; d < D; ++d) {
      float x = bf16_to_f32(vb[(int64_t)idx[c] * sS + d]);
      n2 = __builtin_fmaf(x, x, n2);
    }
    ws.norms[bh * k + c] = n2;
  }
}

// Zeroes the per-channel residual amax of each (b, h): the only state the
// gather/means/residual passes need when the permutation is given.
__global__ __launch_bounds__(256) void amax_reset(int D, GroupWs ws) {
  const int64_t bh = blockIdx.x;
  for (int e = threadIdx.x; e < D; e += 256) ws.r_amax[bh * D + e] = 0u;
}

// Assignment of kAssignTokens tokens, member sums accumulated in LDS and
// flushed with 64-bit atomics.
template <int D>
__global__ __launch_bounds__(256) void kmeans_assign(const uint16_t* __restrict__ v, int64_t sB, int64_t sS,
                                                     int64_t sH, int S, int H, int k,
                                                     const float* __restrict__ cent, int32_t* __restrict__ labels,
                                                     GroupWs ws) {
  __shared__ unsigned long long lsum[8192];  // k * D <= 8192
  __shared__ int lcnt[256];
  const int h = blockIdx.y, b = blockIdx.z, t = threadIdx.x;
  const int64_t bh = (int64_t)b * H + h;
  for (int e = t; e < k * D; e += 256) lsum[e] = 0ull;
  for (int e = t; e < k; e += 256) lcnt[e] = 0;
  __syncthreads();
  const uint16_t* vb = v + b * sB + h * sH;
  const float* __restrict__ cb = cent + bh * k * D;
  const float* __restrict__ nb = ws.norms + bh * k;
  for (int i = 0; i < kAssignTokens / 256; ++i) {
    const int tok = blockIdx.x * kAssignTokens + i * 256 + t;
    if (tok >= S) break;
    float x[D];
    const uint4* row = (const uint4*)(vb + (int64_t)tok * sS);
#pragma unroll
    for (int c8 = 0; c8 < D / 8; ++c8) {
      uint4 w = row[c8];
      x[8 * c8 + 0] = bf16_lo(w.x);
      x[8 * c8 + 1] = bf16_hi(w.x);
      x[8 * c8 + 2] = bf16_lo(w.y);
      x[8 * c8 + 3] = bf16_hi(w.y);
      x[8 * c8 + 4] = bf16_lo(w.z);
      x[8 * c8 + 5] = bf16_hi(w.z);
      x[8 * c8 + 6] = bf16_lo(w.w);
      x[8 * c8 + 7] = bf16_hi(w.w);
    }
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
    labels[bh * S + tok] = best;
    atomicAdd(&lcnt[best], 1);
    unsigned long long* ls = lsum + best * D;
#pragma unroll
    for (int d = 0; d < D; ++d) atomicAdd(&ls[d], (unsigned long long)fx24(x[d]));
  }
  __syncthreads();
  unsigned long long* gs = (unsigned long long*)ws.sums + bh * k * D;
  for (int e = t; e < k * D; e += 256)
    if (lcnt[e / D] > 0) atomicAdd(&gs[e], lsum[e]);
  for (int e = t; e < k; e += 256)
    if (lcnt[e] > 0) atomicAdd((unsigned long long*)&ws.counts[bh * k + e], (unsigned long long)lcnt[e]);
}

// Member means (empty clusters keep their centroid), norms, reset sums.
template <int D>
__global__ __launch_bounds__(256) void kmeans_update(int k, float* __restrict__ cent, GroupWs ws) {
  const int64_t bh = blockIdx.x;
  const int t = threadIdx.x;
  float* cb = cent + bh * k * D;
  long long* sb = ws.sums + bh * k * D;
  const long long* nb = ws.counts + bh * k;
  for (int e = t; e < k * D; e += 256) {
    long long n = nb[e / D];
    if (n > 0) cb[e] = fx24_mean(sb[e], n);
    sb[e] = 0;
  }
  __syncthreads();
  for (int c = t; c < k; c += 256) {
    float n2 = 0.0f;
    for (int d = 0; d < D; ++d) n2 = __builtin_fmaf(cb[c * D + d], cb[c * D + d], n2);
    ws.norms[bh * k + c] = n2;
  }
  __syncthreads();
  for (int c = t; c < k; c += 256) ws.counts[bh * k + c] = 0;
}

// Per-chunk label counts: hist[bh][c][chunk].
__global__ __launch_bounds__(256) void label_hist(const int32_t* __restrict__ labels, int S, int H, int k,
                                                  int nchunk, GroupWs ws) {
  __shared__ int cnt[256];
  const int h = blockIdx.y, b = blockIdx.z, t = threadIdx.x, ch = blockIdx.x;
  const int64_t bh = (int64_t)b * H + h;
  if (t < k) cnt[t] = 0;
  __syncthreads();
  const int tok = ch * kChunk + t;
  if (tok < S) atomicAdd(&cnt[labels[bh * S + tok]], 1);
  __syncthreads();
  if (t < k) ws.hist[(bh * k + t) * nchunk + ch] = cnt[t];
}

// Exclusive scan of hist[bh] in (label, chunk) order, in place.
__global__ __launch_bounds__(1024) void hist_scan(int k, int nchunk, GroupWs ws) {
  __shared__ int part[1024];
  const int64_t bh = blockIdx.x;
  const int t = threadIdx.x;
  int* hb = ws.hist + bh * k * nchunk;
  const int E = k * nchunk;
  const int per = (E + 1023) / 1024;
  const int e0 = t * per, e1 = min(E, e0 + per);
  int s = 0;
  for (int e = e0; e < e1; ++e) s += hb[e];
  part[t] = s;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    int x = t >= o ? part[t - o] : 0;
    __syncthreads();
    part[t] += x;
    __syncthreads();
  }
  int run = part[t] - s;  // exclusive prefix of this segment
  for (int e = e0; e < e1; ++e) {
    int c = hb[e];
    hb[e] = run;
    run += c;
  }
}

// Stable scatter: perm[offset(label, chunk) + rank within chunk] = token.
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

template <int D>
struct ApplyMap {
  static constexpr int CPR = D / 8;         // 16-byte chunks per row
  static constexpr int RG = 256 / CPR;      // row groups
  static constexpr int RPT = kBlk / RG;     // rows per thread
};

// Pass 1: gather K and V by pi; K' per-block codes; block means; residual
// per-channel maxima.
template <int D>
__global__ __launch_bounds__(256) void group_apply1(const uint16_t* __restrict__ kx, int64_t kB, int64_t kS,
                                                    int64_t kH, const uint16_t* __restrict__ vx, int64_t vB,
                                                    int64_t vS, int64_t vH, int S, int H, int nblk,
                                                    const int32_t* __restrict__ perm, uint8_t* __restrict__ k8,
                                                    float* __restrict__ k_scale, uint16_t* __restrict__ mu_bf16,
                                                    GroupWs ws) {
  using Mp = ApplyMap<D>;
  __shared__ long long psum[Mp::RG][D];
  __shared__ float pmax[Mp::RG][D];
  __shared__ float red[4];
  __shared__ float mu_l[D];
  const int j = blockIdx.x, h = blockIdx.y, b = blockIdx.z, t = threadIdx.x;
  const int64_t bh = (int64_t)b * H + h;
  const int ch = t % Mp::CPR, rg = t / Mp::CPR;
  const int nvalid = min(kBlk, S - j * kBlk);
  int tok[Mp::RPT];
#pragma unroll
  for (int r = 0; r < Mp::RPT; ++r) {
    int row = rg * Mp::RPT + r;
    tok[r] = row < nvalid ? perm[bh * S + j * kBlk + row] : -1;
  }
  // ---- K' = K[pi], per-block E4M3 ----
  {
    const uint16_t* kb = kx + b * kB + h * kH;
    uint4 kv[Mp::RPT];
    float m = 0.0f;
#pragma unroll
    for (int r = 0; r < Mp::RPT; ++r) {
      kv[r] = tok[r] >= 0 ? *(const uint4*)(kb + (int64_t)tok[r] * kS + ch * 8) : make_uint4(0, 0, 0, 0);
      m = fmaxf(m, fabsf(bf16_lo(kv[r].x)));
      m = fmaxf(m, fabsf(bf16_hi(kv[r].x)));
      m = fmaxf(m, fabsf(bf16_lo(kv[r].y)));
      m = fmaxf(m, fabsf(bf16_hi(kv[r].y)));
      m = fmaxf(m, fabsf(bf16_lo(kv[r].z)));
      m = fmaxf(m, fabsf(bf16_hi(kv[r].z)));
      m = fmaxf(m, fabsf(bf16_lo(kv[r].w)));
      m = fmaxf(m, fabsf(bf16_hi(kv[r].w)));
    }
    m = wave_max(m);
    if ((t & 63) == 0) red[t >> 6] = m;
    __syncthreads();
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    float s = 1.0f, inv = 1.0f;
    if (m > 0.0f) {
      s = m / 448.0f;
      inv = 448.0f / m;
    }
    if (t == 0) k_scale[bh * nblk + j] = s;
    uint8_t* kd = k8 + (bh * nblk * kBlk + (int64_t)j * kBlk) * D;
#pragma unroll
    for (int r = 0; r < Mp::RPT; ++r) {
      uint4 w = kv[r];
      uint2 c;
      c.x = cvt4_fp8(bf16_lo(w.x) * inv, bf16_hi(w.x) * inv, bf16_lo(w.y) * inv, bf16_hi(w.y) * inv);
      c.y = cvt4_fp8(bf16_lo(w.z) * inv, bf16_hi(w.z) * inv, bf16_lo(w.w) * inv, bf16_hi(w.w) * inv);
      *(uint2*)(kd + kpack_off<D>(rg * Mp::RPT + r, ch >> 1) + (ch & 1) * 8) = c;
    }
  }
  // ---- V' block mean ----
  const uint16_t* vb = vx + b * vB + h * vH;
  float xv[Mp::RPT][8];
  {
    long long ps[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int r = 0; r < Mp::RPT; ++r) {
      uint4 w = tok[r] >= 0 ? *(const uint4*)(vb + (int64_t)tok[r] * vS + ch * 8) : make_uint4(0, 0, 0, 0);
      xv[r][0] = bf16_lo(w.x); xv[r][1] = bf16_hi(w.x);
      xv[r][2] = bf16_lo(w.y); xv[r][3] = bf16_hi(w.y);
      xv[r][4] = bf16_lo(w.z); xv[r][5] = bf16_hi(w.z);
      xv[r][6] = bf16_lo(w.w); xv[r][7] = bf16_hi(w.w);
#pragma unroll
      for (int e = 0; e < 8; ++e) ps[e] += fx24(xv[r][e]);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) psum[rg][ch * 8 + e] = ps[e];
  }
  __syncthreads();
  if (t < D) {
    long long s = 0;
    for (int q = 0; q < Mp::RG; ++q) s += psum[q][t];
    uint16_t mb = f32_to_bf16(fx24_mean(s, nvalid));
    mu_bf16[(bh * nblk + j) * D + t] = mb;
    mu_l[t] = bf16_to_f32(mb);
  }
  __syncthreads();
  // ---- residual channel maxima ----
  {
    float pm[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int r = 0; r < Mp::RPT; ++r)
      if (tok[r] >= 0)
#pragma unroll
        for (int e = 0; e < 8; ++e) pm[e] = fmaxf(pm[e], fabsf(xv[r][e] - mu_l[ch * 8 + e]));
#pragma unroll
    for (int e = 0; e < 8; ++e) pmax[rg][ch * 8 + e] = pm[e];
  }
  __syncthreads();
  if (t < D) {
    float m = 0.0f;
    for (int q = 0; q < Mp::RG; ++q) m = fmaxf(m, pmax[q][t]);
    atomicMax(&ws.r_amax[bh * D + t], __float_as_uint(m));
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
  constexpr int LD = D + 4;
  __shared__ uint8_t tile[kBlk * LD];
  __shared__ float inv_l[D], mu_l[D];
  const int j = blockIdx.x, h = blockIdx.y, b = blockIdx.z, t = threadIdx.x;
  const int64_t bh = (int64_t)b * H + h;
  if (t < D) {
    float m = __uint_as_float(ws.r_amax[bh * D + t]);
    float s = 1.0f, inv = 1.0f;
    if (m > 0.0f) {
      s = m / 448.0f;
      inv = 448.0f / m;
    }
    inv_l[t] = inv;
    float mu = bf16_to_f32(mu_bf16[(bh * nblk + j) * D + t]);
    mu_l[t] = mu;
    const float ms = mu * inv;
    const uint16_t hi = f32_to_bf16(ms);
    const uint16_t lo = f32_to_bf16(ms - bf16_to_f32(hi));
    mu_split[(bh * nblk + j) * D + t] = (u32)hi | ((u32)lo << 16);
    if (j == 0) r_scale[bh * D + t] = s;
  }
  __syncthreads();
  const int ch = t % Mp::CPR, rg = t / Mp::CPR;
  const int nvalid = min(kBlk, S - j * kBlk);
  const uint16_t* vb = vx + b * vB + h * vH;
#pragma unroll
  for (int r = 0; r < Mp::RPT; ++r) {
    const int row = rg * Mp::RPT + r;
    u32 c0 = 0, c1 = 0;
    if (row < nvalid) {
      const int tk = perm[bh * S + j * kBlk + row];
      uint4 w = *(const uint4*)(vb + (int64_t)tk * vS + ch * 8);
      const float* mu = mu_l + ch * 8;
      const float* iv = inv_l + ch * 8;
      c0 = cvt4_fp8((bf16_lo(w.x) - mu[0]) * iv[0], (bf16_hi(w.x) - mu[1]) * iv[1], (bf16_lo(w.y) - mu[2]) * iv[2],
                    (bf16_hi(w.y) - mu[3]) * iv[3]);
      c1 = cvt4_fp8((bf16_lo(w.z) - mu[4]) * iv[4], (bf16_hi(w.z) - mu[5]) * iv[5], (bf16_lo(w.w) - mu[6]) * iv[6],
                    (bf16_hi(w.w) - mu[7]) * iv[7]);
    }
    *(u32*)(tile + row * LD + ch * 8) = c0;
    *(u32*)(tile + row * LD + ch * 8 + 4) = c1;
  }
  __syncthreads();
  uint8_t* ob = r8 + (bh * nblk + j) * (int64_t)D * kBlk;  // packed V tile j
  constexpr int TASKS = D * (kBlk / 16);
#pragma unroll
  for (int i = 0; i < TASKS / 256; ++i) {
    int task = t + 256 * i, d = task / (kBlk / 16), c = task % (kBlk / 16), k0 = c * 16;
    u32 wv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      wv[q] = (u32)tile[vkey_of_pos(k0 + 4 * q) * LD + d] | ((u32)tile[vkey_of_pos(k0 + 4 * q + 1) * LD + d] << 8) |
             ((u32)tile[vkey_of_pos(k0 + 4 * q + 2) * LD + d] << 16) |
             ((u32)tile[vkey_of_pos(k0 + 4 * q + 3) * LD + d] << 24);
    *(uint4*)(ob + vpack_off(d, c)) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
  }
}

template <int D>
hipError_t launch_group_t(const vc_shape& sh, Bshd k, Bshd v, const vc_group_params& p, float* cent, int32_t* labels,
                          int32_t* perm, uint8_t* k8, float* k_scale, uint8_t* r8, float* r_scale,
                          uint16_t* mu_bf16, u32* mu_split, GroupWs ws, hipStream_t st) {
  const int S = sh.S, H = sh.H, B = sh.B, kc = p.clusters;
  const int nblk = (S + kBlk - 1) / kBlk, nchunk = (S + kChunk - 1) / kChunk;
  const int BH = B * H;
  if (p.flags & VC_GROUP_REUSE_PERM) {
    // the caller's permutation: only the gather, block means and residual codes
    amax_reset<<<BH, 256, 0, st>>>(D, ws);
  } else {
    group_init<D><<<dim3(H, B), 256, 0, st>>>(v.p, v.sB, v.sS, v.sH, S, H, kc, p.seed,
                                              (p.flags & VC_GROUP_WARM_START) ? 1 : 0, cent, ws);
    const dim3 ga((S + kAssignTokens - 1) / kAssignTokens, H, B);
    for (int it = 0; it < p.iters; ++it) {
      kmeans_assign<D><<<ga, 256, 0, st>>>(v.p, v.sB, v.sS, v.sH, S, H, kc, cent, labels, ws);
      kmeans_update<D><<<BH, 256, 0, st>>>(kc, cent, ws);
    }
    label_hist<<<dim3(nchunk, H, B), 256, 0, st>>>(labels, S, H, kc, nchunk, ws);
    hist_scan<<<BH, 1024, 0, st>>>(kc, nchunk, ws);
    label_scatter<<<dim3(nchunk, H, B), 256, 0, st>>>(labels, S, H, kc, nchunk, ws, perm);
  }
  group_apply1<D><<<dim3(nblk, H, B), 256, 0, st>>>(k.p, k.sB, k.sS, k.sH, v.p, v.sB, v.sS, v.sH, S, H, nblk, perm,
                                                    k8, k_scale, mu_bf16, ws);
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
                               float* r_scale, uint16_t* mu_bf16, uint32_t* mu_split, void* ws, hipStream_t st) {
  GroupWs g = carve(ws, sh, p.clusters, nullptr);
  if (sh.D == 128)
    return launch_group_t<128>(sh, k, v, p, centroids, labels, perm, k8, k_scale, r8, r_scale, mu_bf16, mu_split, g,
                               st);
  return launch_group_t<64>(sh, k, v, p, centroids, labels, perm, k8, k_scale, r8, r_scale, mu_bf16, mu_split, g, st);
}

}  // namespace vc
