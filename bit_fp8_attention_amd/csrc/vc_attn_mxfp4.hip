// vc_attn_mxfp4.hip -- the 4-bit path: V-Smooth at 4 bits without ExpCast
// ([VC] §4.1 "Implementation": 4 bits run V-Smooth alone; "Scope of
// ExpCast-FP8": P is kept in a microscaled 4-bit format, for which no affine
// log-to-code map exists).  The pages' format is NVFP4; gfx950's matrix
// cores take OCP MXFP4: E2M1 elements with one E8M0 (power-of-two) scale per
// 32, applied by v_mfma_scale_f32_16x16x128_f8f6f4 from a per-lane byte.
//
// Block scale of 32 elements: the smallest 2^e (e >= -127) with
// amax <= 6 * 2^e (2^0 for zeros); elements E2M1_rne(x / 2^e)
// (v_cvt_scalef32_pk_fp4_f32, which divides by the scale and rounds half to
// even, saturating at 6 -- checked by a probe).  Q is multiplied first by
// fl(sm_scale * log2 e), so the score product is in log2 units.
//
// Layouts (per (b, h); nblk = ceil(S / 128) tiles of 128 keys):
//  - q4: row-major [S_pad][D/2] bytes, byte c = channels 2c (low nibble) and
//    2c + 1; q4_scale [S_pad][D/32] E8M0 bytes.
//  - k4: per tile 128 rows of D/2 bytes; tile row 16 t + 4 g + v holds key
//    32 g + 4 t + v of the tile, so that the S^T accumulator of MFMA block t,
//    register v, in lane group g holds key 32 g + 4 t + v: lane group g then
//    holds keys [32 g, 32 g + 32), one P block, in its own registers.  The
//    16-byte chunk c of row r sits at chunk c ^ k4swz(r), so that the 16 rows
//    a fragment read touches spread over all LDS banks.
//    k4_scale per tile 512 bytes [g][lr][t] (the scale of tile row 16 t + lr,
//    channel block g; 127 where g >= D/32).
//  - v4: per tile D channel rows of 64 bytes (keys 0..127 of the tile,
//    key 2c in the low nibble of byte c; 16-byte chunk c of row d at chunk
//    c ^ ((d >> 2) & 3)); v4_scale per tile 512 bytes
//    [g][lr][m] (the scale of channel 16 m + lr, keys [32 g, 32 g + 32)).
#include "vc_common.hpp"
#include "vc_launch.hpp"

namespace vc {

namespace {

VC_DEV int mx_block_exp(float amax) {
  if (!(amax > 0.0f)) return 0;
  int e = __builtin_amdgcn_frexp_expf(amax) - 4;  // amax in [2^(e+3), 2^(e+4)): below the answer
  if (e < -127) e = -127;
  while (amax > ldexpf(6.0f, e)) ++e;
  return e;
}

// mx_block_exp for a probability maximum p in [0, 1] (finite), without the
// loop: with p = m 2^f, m in [0.5, 1), the answer is f - 3, plus one when
// m > 0.75 (then 6 2^(f - 3) = 0.75 2^f < p), at least -127; 0 for p = 0
VC_DEV int mx_block_exp_prob(float p) {
  const int e = __builtin_amdgcn_frexp_expf(p) - 3 + (__builtin_amdgcn_frexp_mantf(p) > 0.75f ? 1 : 0);
  return p > 0.0f ? max(e, -127) : 0;
}

// 8 fp32 -> 8 E2M1 nibbles (one dword, element i in nibble i) at scale 2^e
VC_DEV u32 cvt8_fp4(const float (&x)[8], float scale) {
  u32 w = 0u;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[0], x[1], scale, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[2], x[3], scale, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[4], x[5], scale, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[6], x[7], scale, 3);
  return w;
}

// tile row holding key k of the tile (inverse of the row -> key map above)
VC_DEV int k4_row_of_key(int k) { return 16 * ((k & 31) >> 2) + 4 * (k >> 5) + (k & 3); }
// chunk swizzles: 4 rows of 64 bytes (2 of 32 at D = 64) fill the 256-byte
// bank width, so rows r and r + 4 (r + 8) would collide without them
template <int D>
VC_DEV int k4swz(int r) { return D == 128 ? (r >> 2) & 3 : (r >> 3) & 1; }
VC_DEV int v4swz(int d) { return (d >> 2) & 3; }

// ---- quantisers (HBM-bound) ----

// Q: one thread per (row, 32-channel block): 64 contiguous bytes in, 16 out.
template <int D>
__global__ __launch_bounds__(256) void q4_rows_kernel(const uint16_t* __restrict__ x, int64_t sB, int64_t sS,
                                                      int64_t sH, int S, int H, int S_pad, float pre,
                                                      uint8_t* __restrict__ q4, uint8_t* __restrict__ q4s) {
  constexpr int NB = D / 32;
  const int64_t item = (int64_t)blockIdx.x * 256 + threadIdx.x;  // over S_pad * NB
  const int h = blockIdx.y, b = blockIdx.z;
  if (item >= (int64_t)S_pad * NB) return;
  const int row = (int)(item / NB), blk = (int)(item % NB);
  const int64_t bh = (int64_t)b * H + h;
  float y[32];
  if (row < S) {
    const uint16_t* src = x + b * sB + h * sH + (int64_t)row * sS + 32 * blk;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint4 w = *(const uint4*)(src + 8 * c);
      const u32 ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        y[8 * c + 2 * i] = bf16_lo(ws[i]) * pre;
        y[8 * c + 2 * i + 1] = bf16_hi(ws[i]) * pre;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) y[i] = 0.0f;
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(y[i]));
  const int e = mx_block_exp(amax);
  const float sc = ldexpf(1.0f, e);
  u32 wd[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    float t[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) t[i] = y[8 * c + i];
    wd[c] = cvt8_fp4(t, sc);
  }
  *(uint4*)(q4 + (bh * S_pad + row) * (D / 2) + 16 * blk) = make_uint4(wd[0], wd[1], wd[2], wd[3]);
  q4s[(bh * S_pad + row) * NB + blk] = (uint8_t)(e + 127);
}

// K and V of one 128-key tile: keys taken through perm (V-Smooth's pi) when
// given, V minus the tile's block mean mu_bf16 when given (the residual of
// [VC] §3.2 Eq. 4, one fp32 subtraction).  256 threads.
template <int D>
__global__ __launch_bounds__(256) void kv4_tile_kernel(const uint16_t* __restrict__ k, int64_t kB, int64_t kS,
                                                       int64_t kH, const uint16_t* __restrict__ v, int64_t vB,
                                                       int64_t vS, int64_t vH, int S, int H, int nblk,
                                                       const int32_t* __restrict__ perm,
                                                       const uint16_t* __restrict__ mu, uint8_t* __restrict__ k4,
                                                       uint8_t* __restrict__ k4s, uint8_t* __restrict__ v4,
                                                       uint8_t* __restrict__ v4s) {
  constexpr int NB = D / 32;
  constexpr int TB = kBlk * D / 2;
  constexpr int LD = D + 1;
  __shared__ float vt[kBlk * LD];  // the tile's V (or residual) rows, fp32
  const int t = blockIdx.x, h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int64_t bh = (int64_t)b * H + h;
  uint8_t* kt = k4 + (bh * nblk + t) * TB;
  uint8_t* kts = k4s + (bh * nblk + t) * 512;
  uint8_t* vtp = v4 + (bh * nblk + t) * TB;
  uint8_t* vts = v4s + (bh * nblk + t) * 512;
  auto token = [&](int key) -> int {  // key index within the tile -> token, or -1
    const int pos = t * kBlk + key;
    if (pos >= S) return -1;
    if (!perm) return pos;
    int tok = perm[bh * S + pos];
    return tok < 0 ? 0 : (tok < S ? tok : S - 1);  // in bounds whatever the list holds
  };
  // K: one thread per (key, channel block)
  for (int item = tid; item < kBlk * NB; item += 256) {
    const int key = item / NB, blk = item % NB, tok = token(key);
    float y[32];
    if (tok >= 0) {
      const uint16_t* src = k + b * kB + h * kH + (int64_t)tok * kS + 32 * blk;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint4 w = *(const uint4*)(src + 8 * c);
        const u32 ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          y[8 * c + 2 * i] = bf16_lo(ws[i]);
          y[8 * c + 2 * i + 1] = bf16_hi(ws[i]);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 32; ++i) y[i] = 0.0f;
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(y[i]));
    const int e = mx_block_exp(amax);
    const float sc = ldexpf(1.0f, e);
    u32 wd[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float tt[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) tt[i] = y[8 * c + i];
      wd[c] = cvt8_fp4(tt, sc);
    }
    const int row = k4_row_of_key(key);
    *(uint4*)(kt + row * (D / 2) + 16 * (blk ^ k4swz<D>(row))) = make_uint4(wd[0], wd[1], wd[2], wd[3]);
    kts[(16 * blk + (row & 15)) * 8 + (row >> 4)] = (uint8_t)(e + 127);
  }
  // channel blocks the head dimension does not fill: scale 2^0
  for (int item = tid; item < (4 - NB) * 16 * 8; item += 256) kts[NB * 128 + item] = 127;
  // V: rows into LDS (fp32, minus the block mean), then one thread per
  // (channel, 32-key block)
  for (int item = tid; item < kBlk * (D / 8); item += 256) {
    const int key = item / (D / 8), ch = item % (D / 8), tok = token(key);
    float xv[8];
    if (tok >= 0) {
      const uint4 w = *(const uint4*)(v + b * vB + h * vH + (int64_t)tok * vS + 8 * ch);
      const u32 ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        xv[2 * i] = bf16_lo(ws[i]);
        xv[2 * i + 1] = bf16_hi(ws[i]);
      }
      if (mu) {
        const uint16_t* mr = mu + (bh * nblk + t) * D + 8 * ch;
#pragma unroll
        for (int i = 0; i < 8; ++i) xv[i] = xv[i] - bf16_to_f32(mr[i]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) xv[i] = 0.0f;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) vt[key * LD + 8 * ch + i] = xv[i];
  }
  __syncthreads();
  for (int item = tid; item < D * 4; item += 256) {
    const int d = item / 4, g = item % 4;
    const int lim = S - t * kBlk;  // valid keys of this tile (keys past S do not enter the max)
    float amax = 0.0f;
    for (int kk = 32 * g; kk < 32 * g + 32; ++kk)
      if (kk < lim) amax = fmaxf(amax, fabsf(vt[kk * LD + d]));
    const int e = mx_block_exp(amax);
    const float sc = ldexpf(1.0f, e);
    u32 wd[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float tt[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) tt[i] = vt[(32 * g + 8 * c + i) * LD + d];
      wd[c] = cvt8_fp4(tt, sc);
    }
    *(uint4*)(vtp + d * 64 + 16 * (g ^ v4swz(d))) = make_uint4(wd[0], wd[1], wd[2], wd[3]);
    vts[(16 * g + (d & 15)) * 8 + (d >> 4)] = (uint8_t)(e + 127);
  }
  for (int item = tid; item < 64 * 8; item += 256)  // channel blocks past D / 16: scale 2^0
    if ((item & 7) >= D / 16) vts[item] = 127;
}

// ---- attention ----
//
// One workgroup = one 128-query tile of one (b, h) (4 waves x 32 queries),
// two workgroups per CU: their barriers are independent, so one
// workgroup's VALU work overlaps the other's matrix-core work on each SIMD
// (with both tiles in one 8-wave workgroup the shared per-tile barrier kept
// the two waves of a SIMD in the same phase: 8-9% slower).  K/V tiles come
// in the mid-window order through a 2-stage LDS ring that the 4 waves fill
// with global_load_lds_dwordx4.  Per tile and 16-query sub-tile:
// S^T = K Q^T (scores in log2 units), the running max on the true scores,
// p = 2^(s - M) (v_exp_f32), one E8M0 block scale per lane (its 32 keys),
// E2M1 codes, row sum (ones x P^T) and A^T += V^T P^T on the block-scaled
// matrix cores, and with V-Smooth the block mean restored as A += r mu.

VC_DEV v4f mfma_fp4(v8i a, v8i b, v4f c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 4, 0, sa, 0, sb);
}

template <int D, bool VS>
__global__ __launch_bounds__(256, 2) void attn4_kernel(
    const uint8_t* __restrict__ q4, const uint8_t* __restrict__ q4s, const uint8_t* __restrict__ k4,
    const uint8_t* __restrict__ k4s, const uint8_t* __restrict__ v4, const uint8_t* __restrict__ v4s,
    const uint16_t* __restrict__ mu, uint16_t* __restrict__ o, int64_t oB, int64_t oS, int64_t oH, int S, int H,
    int nblk, int npair, int window, int sequential) {
  constexpr int NM = D / 16;
  constexpr int TB = kBlk * D / 2;  // bytes of a K or V tile
  constexpr int NB = D / 32;
  __shared__ __attribute__((aligned(1024))) uint8_t kst[2][TB];
  __shared__ __attribute__((aligned(1024))) uint8_t vst[2][TB];
  // V-Smooth: ring of the block-mean rows (bf16) of the last 16 visited tiles
  constexpr int MR = VS ? 16 : 1;
  __shared__ __attribute__((aligned(16))) uint16_t mring[MR][VS ? D : 8];

  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int pr = __builtin_amdgcn_readfirstlane(lin % npair);
  const int bh = __builtin_amdgcn_readfirstlane(lin / npair);
  const int tid = threadIdx.x, l = tid & 63, lr = l & 15, g = l >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wq = w & 3;
  const bool live = true;
  const int qt = pr;  // one query tile per workgroup
  const int64_t S_pad = (int64_t)nblk * kBlk;
  const int start = __builtin_amdgcn_readfirstlane(sequential ? 0 : min((qt | 1) + window, nblk - 1));
  auto tile_at = [&](int i) -> int { return sequential ? i : (i <= start ? start - i : i); };

  // Q fragments and scales of the wave's two 16-query sub-tiles
  v8i qf[2];
  int qsc[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int64_t qrow = (int64_t)bh * S_pad + qt * kBlk + 32 * wq + 16 * s + lr;
    uint4 qv = make_uint4(0, 0, 0, 0);
    int sc = 127;
    if (g < NB) {
      qv = *(const uint4*)(q4 + qrow * (D / 2) + 16 * g);
      sc = q4s[qrow * NB + g];
    }
    qf[s] = v8i{(int)qv.x, (int)qv.y, (int)qv.z, (int)qv.w, 0, 0, 0, 0};
    qsc[s] = sc;
  }

  // copies of tile i into stage st: each wave 1/8 of the K and of the V tile
  constexpr int CW = TB / 4;  // bytes per wave (2 KB at D = 128)
  const unsigned loff = (unsigned)l * 16u;
  auto issue = [&](int i, int st) {
    const int64_t t = (int64_t)bh * nblk + tile_at(i);
    const uint8_t* ks = k4 + t * TB + w * CW;
    const uint8_t* vs = v4 + t * TB + w * CW;
    if constexpr (CW == 2048) {  // two 1 KB blocks under one M0 each
      lds_dma16_kb<2>(ks + loff, &kst[st][w * CW]);
      lds_dma16_kb<2>(vs + loff, &vst[st][w * CW]);
    } else {
#pragma unroll
      for (int r = 0; r < (CW + 1023) / 1024; ++r) {
        if (l * 16 < CW - 1024 * r) {
          lds_dma16_raw(ks + 1024 * r + loff, &kst[st][w * CW + 1024 * r]);
          lds_dma16_raw(vs + 1024 * r + loff, &vst[st][w * CW + 1024 * r]);
        }
      }
    }
    if (VS && w == 0 && l < D / 8) lds_dma16_raw((const uint8_t*)(mu + t * D) + loff, &mring[i & (MR - 1)][0]);
  };
  // per-lane scale bytes of tile i: 8 K scales (blocks t8) and 8 V scales (blocks m)
  auto load_scales = [&](int i, uint2& ks, uint2& vs) {
    const int64_t t = (int64_t)bh * nblk + tile_at(i);
    ks = *(const uint2*)(k4s + t * 512 + l * 8);
    vs = *(const uint2*)(v4s + t * 512 + l * 8);
  };
  auto sbyte = [](const uint2& s, int k) -> int { return (int)(((k < 4 ? s.x : s.y) >> (8 * (k & 3))) & 0xffu); };

  const v8i ones = {0x22222222, 0x22222222, 0x22222222, 0x22222222, 0, 0, 0, 0};  // E2M1 1.0
  const v4f zero4 = {0.f, 0.f, 0.f, 0.f};
  // M: running max of the sub-tile's query (log2 units); the score product
  // starts its accumulator at -M, so it emits s - M directly (0 before the
  // first tile, which always sets M)
  float M[2] = {0.f, 0.f};
  v4f cinit[2] = {zero4, zero4};
  float L[2] = {0.f, 0.f};
  v4f O[2][NM];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int m = 0; m < NM; ++m) O[s][m] = zero4;

  // V-Smooth: row sums of the window slots 2g, 2g + 1 (lane group g), restored
  // every 8 tiles on the bf16 matrix cores as A += r mu^T: lane group g
  // carries its two slots in K slots 8g .. 8g + 7 as
  //   mean side: (mu0, 0, mu1, 0, mu0, 0, mu1, 0)   (mu is exact in bf16)
  //   sum side:  (r0.hi, r0.hi, r1.hi, r1.hi, r0.lo, 0, r1.lo, 0)
  float rb[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
  if (VS) {  // rows never written must read as finite zeros
    for (int e2 = tid; e2 < MR * D; e2 += 256) (&mring[0][0])[e2] = 0;
    __syncthreads();
  }

  uint2 ksc, vsc;
  issue(0, 0);
  load_scales(0, ksc, vsc);
  wait_vm();
  __syncthreads();
  for (int i = 0; i < nblk; ++i) {
    const int st = i & 1;
    uint2 ksn = ksc, vsn = vsc;
    if (i + 1 < nblk) {
      issue(i + 1, st ^ 1);  // stage st ^ 1 was last read in the previous iteration
      load_scales(i + 1, ksn, vsn);
    }
    const uint8_t* Kt = kst[st];
    const uint8_t* Vt = vst[st];
    // S^T = K Q^T: block t8 is tile rows 16 t8 + lr, channel block g
    v4f Sc[2][8];
    uint4 kv[8];
#pragma unroll
    for (int t8 = 0; t8 < 8; ++t8) {
      const int r = 16 * t8 + lr;
      kv[t8] = g < NB ? *(const uint4*)(Kt + r * (D / 2) + 16 * (g ^ k4swz<D>(r))) : make_uint4(0, 0, 0, 0);
    }
    const int t = tile_at(i);
    const bool ragged = t == nblk - 1 && (S % kBlk) != 0;  // keys past S: no probability
    v8i P[2];
    int pe[2];
    float lmx[2], rr[2];
    // one sub-tile (16 query rows) at a time: scores; running max and
    // rescale; probabilities and their codes; row sum and P.V.  Sub-tile 1's
    // scores come after sub-tile 0's rescale, and sub-tile 0's P.V after
    // sub-tile 1's, so each stretch between the rescale branches pairs one
    // sub-tile's matrix-core work with the other's VALU work
    auto qk = [&](int s) {
#pragma unroll
      for (int t8 = 0; t8 < 8; ++t8) {
        const v8i kf = {(int)kv[t8].x, (int)kv[t8].y, (int)kv[t8].z, (int)kv[t8].w, 0, 0, 0, 0};
        Sc[s][t8] = mfma_fp4(kf, qf[s], cinit[s], sbyte(ksc, t8), qsc[s]);
      }
    };
    auto mask = [&](int s) {
      if (ragged) {
        const int lim = S - t * kBlk;
#pragma unroll
        for (int t8 = 0; t8 < 8; ++t8)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            if (32 * g + 4 * t8 + v >= lim) Sc[s][t8][v] = -INFINITY;
      }
    };
    auto rescale = [&](int s) {
      float lm = -INFINITY;  // the lane's max (its 32 keys: one P block)
#pragma unroll
      for (int t8 = 0; t8 < 8; ++t8)
#pragma unroll
        for (int v = 0; v < 4; ++v) lm = fmaxf(lm, Sc[s][t8][v]);
      const float rm = max_over_groups(lm);  // the row's max of s - M
      const bool rise = i == 0 || rm > 0.0f;
      if (__any(rise)) {
        const float delta = rise ? -rm : 0.0f;  // M - M'
        if (i != 0) {
          const float alpha = __builtin_amdgcn_exp2f(delta);
          L[s] *= alpha;
          if (VS) {
            rb[s][0] *= alpha;
            rb[s][1] *= alpha;
          }
#pragma unroll
          for (int m = 0; m < NM; ++m) O[s][m] = O[s][m] * alpha;
        }
        M[s] -= delta;
        cinit[s] = v4f{-M[s], -M[s], -M[s], -M[s]};
        lm += delta;
#pragma unroll
        for (int t8 = 0; t8 < 8; ++t8) Sc[s][t8] = Sc[s][t8] + delta;
      }
      lmx[s] = lm;
    };
    auto probs = [&](int s) {
      const float pmax = __builtin_amdgcn_exp2f(lmx[s]);  // in [0, 1]: lmx <= 0
      const int e = mx_block_exp_prob(pmax);
      const float sc = ldexpf(1.0f, e);
      pe[s] = e + 127;
      // key 32 g + 4 t8 + v is nibble 4 t8 + v of the lane's P operand
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float p8[8];
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int v = 0; v < 4; ++v) p8[4 * u + v] = __builtin_amdgcn_exp2f(Sc[s][2 * q + u][v]);
        P[s][q] = (int)cvt8_fp4(p8, sc);
      }
      P[s][4] = P[s][5] = P[s][6] = P[s][7] = 0;
    };
    // V's fragments, read once for both sub-tiles
    v8i vf[NM];
    auto pv = [&](int s) {
      // row sum and A^T += V^T P^T
      rr[s] = mfma_fp4(ones, P[s], zero4, 127, pe[s])[0];
      L[s] += rr[s];
#pragma unroll
      for (int m = 0; m < NM; ++m) O[s][m] = mfma_fp4(vf[m], P[s], O[s][m], sbyte(vsc, m), pe[s]);
    };
    qk(0);
    mask(0);
    rescale(0);
    qk(1);
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const int d = 16 * m + lr;
      const uint4 vv = *(const uint4*)(Vt + d * 64 + 16 * (g ^ v4swz(d)));
      vf[m] = v8i{(int)vv.x, (int)vv.y, (int)vv.z, (int)vv.w, 0, 0, 0, 0};
    }
    probs(0);
    // sub-tile 0's codes stay ahead of sub-tile 1's branches, and its
    // conversion work is spread between sub-tile 1's score products
    asm volatile("" ::"v"(P[0][0]), "v"(P[0][1]), "v"(P[0][2]), "v"(P[0][3]), "v"(pe[0]));
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 12, 0);
    }
    mask(1);
    rescale(1);
    pv(0);
    probs(1);
    // and sub-tile 1's between sub-tile 0's row sum and P.V products
#pragma unroll
    for (int k = 0; k < 9; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 12, 0);
    }
    pv(1);
    if (VS) {
      const int slot = i & 7;
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        if (slot == 2 * g) rb[s2][0] = rr[s2];
        if (slot == 2 * g + 1) rb[s2][1] = rr[s2];
      }
      if (slot == 7 || i == nblk - 1) {
        v8bf Ar[2];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const __bf16 hi = (__bf16)rb[s2][jj];
            const __bf16 lo = (__bf16)(rb[s2][jj] - (float)hi);
            Ar[s2][2 * jj + 0] = hi;
            Ar[s2][2 * jj + 1] = hi;
            Ar[s2][4 + 2 * jj + 0] = lo;
            Ar[s2][4 + 2 * jj + 1] = (__bf16)0.0f;
            rb[s2][jj] = 0.f;
          }
        }
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          // window slot 2g + jj is visit i - slot + 2g + jj; slots past i hold
          // zero row sums, so whatever finite row the ring holds there adds nothing
          const u32 m0 = mring[(i - slot + 2 * g) & (MR - 1)][16 * m + lr];
          const u32 m1 = mring[(i - slot + 2 * g + 1) & (MR - 1)][16 * m + lr];
          const v8bf Bm = __builtin_bit_cast(v8bf, (v4u){m0, m1, m0, m1});
          O[0][m] = mfma_bf16(Bm, Ar[0], O[0][m]);
          O[1][m] = mfma_bf16(Bm, Ar[1], O[1][m]);
        }
      }
    }
    ksc = ksn;
    vsc = vsn;
    wait_vm();        // this wave's copies of tile i + 1 have landed
    __syncthreads();  // every wave is done with stage st and sees stage st ^ 1
  }

  if (!live) return;
  const int b = bh / H, h = bh % H;
  uint16_t* ob = o + b * oB + h * oH;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int q = qt * kBlk + 32 * wq + 16 * s + lr;
    if (q >= S) continue;
    const float inv = 1.0f / L[s];
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const int d = 16 * m + 4 * g;
      const u32 lo = (u32)f32_to_bf16(O[s][m][0] * inv) | ((u32)f32_to_bf16(O[s][m][1] * inv) << 16);
      const u32 hi = (u32)f32_to_bf16(O[s][m][2] * inv) | ((u32)f32_to_bf16(O[s][m][3] * inv) << 16);
      *(uint2*)(ob + (int64_t)q * oS + d) = make_uint2(lo, hi);
    }
  }
}

}  // namespace

hipError_t launch_quant4(const vc_shape& sh, float pre, Bshd q, Bshd k, Bshd v, const int32_t* perm,
                         const uint16_t* mu, uint8_t* q4, uint8_t* q4s, uint8_t* k4, uint8_t* k4s, uint8_t* v4,
                         uint8_t* v4s, hipStream_t st) {
  const int nblk = (sh.S + kBlk - 1) / kBlk, S_pad = nblk * kBlk;
  if (q.p) {
    const int64_t items = (int64_t)S_pad * (sh.D / 32);
    dim3 grid((unsigned)((items + 255) / 256), sh.H, sh.B);
    if (sh.D == 128)
      q4_rows_kernel<128><<<grid, 256, 0, st>>>(q.p, q.sB, q.sS, q.sH, sh.S, sh.H, S_pad, pre, q4, q4s);
    else
      q4_rows_kernel<64><<<grid, 256, 0, st>>>(q.p, q.sB, q.sS, q.sH, sh.S, sh.H, S_pad, pre, q4, q4s);
  }
  if (k.p) {
    dim3 grid(nblk, sh.H, sh.B);
    if (sh.D == 128)
      kv4_tile_kernel<128><<<grid, 256, 0, st>>>(k.p, k.sB, k.sS, k.sH, v.p, v.sB, v.sS, v.sH, sh.S, sh.H, nblk, perm,
                                                 mu, k4, k4s, v4, v4s);
    else
      kv4_tile_kernel<64><<<grid, 256, 0, st>>>(k.p, k.sB, k.sS, k.sH, v.p, v.sB, v.sS, v.sH, sh.S, sh.H, nblk, perm,
                                                mu, k4, k4s, v4, v4s);
  }
  return hipGetLastError();
}

hipError_t launch_attn4(const vc_shape& sh, int window, uint32_t flags, const uint8_t* q4, const uint8_t* q4s,
                        const uint8_t* k4, const uint8_t* k4s, const uint8_t* v4, const uint8_t* v4s,
                        const uint16_t* mu, BshdOut o, hipStream_t st) {
  const int nblk = (sh.S + kBlk - 1) / kBlk;
  const int npair = nblk;  // workgroups per head: one query tile each
  const int seq = (flags & VC_ATTN_SEQUENTIAL) ? 1 : 0;
  const unsigned n = (unsigned)((int64_t)npair * sh.H * sh.B);
  if (sh.D == 128) {
    if (mu)
      attn4_kernel<128, true><<<n, 256, 0, st>>>(q4, q4s, k4, k4s, v4, v4s, mu, o.p, o.sB, o.sS, o.sH, sh.S, sh.H,
                                                 nblk, npair, window, seq);
    else
      attn4_kernel<128, false><<<n, 256, 0, st>>>(q4, q4s, k4, k4s, v4, v4s, nullptr, o.p, o.sB, o.sS, o.sH, sh.S,
                                                  sh.H, nblk, npair, window, seq);
  } else {
    if (mu)
      attn4_kernel<64, true><<<n, 256, 0, st>>>(q4, q4s, k4, k4s, v4, v4s, mu, o.p, o.sB, o.sS, o.sH, sh.S, sh.H,
                                                nblk, npair, window, seq);
    else
      attn4_kernel<64, false><<<n, 256, 0, st>>>(q4, q4s, k4, k4s, v4, v4s, nullptr, o.p, o.sB, o.sS, o.sH, sh.S,
                                                 sh.H, nblk, npair, window, seq);
  }
  return hipGetLastError();
}

}  // namespace vc
