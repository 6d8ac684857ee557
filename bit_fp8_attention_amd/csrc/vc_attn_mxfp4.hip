// vc_attn_mxfp4.hip -- the 4-bit path: V-Smooth at 4 bits without ExpCast
// ([VC] §4.1 "Implementation": 4 bits run V-Smooth alone; "Scope of
// ExpCast-FP8": P is kept in a microscaled 4-bit format, for which no affine
// log-to-code map exists).  The pages' format is NVFP4; gfx950's matrix
// cores take OCP MXFP4: E2M1 elements with one E8M0 (power-of-two) scale per
// 32, applied by v_mfma_scale_f32_32x32x64_f8f6f4 from a per-lane byte.
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
//  - k4: per tile 128 rows of D/2 bytes; tile row 64 c + 32 b + 8 j + 4 h + v
//    holds key 64 c + 32 h + 16 b + 4 j + v of the tile, so that the S^T
//    accumulator of key block kb = 2 c + b, register 4 j + v, in lane half h
//    holds key 64 c + 32 h + 16 b + 4 j + v: lane half h then holds keys
//    [64 c + 32 h, 64 c + 32 h + 32), one P block, in its own registers, in
//    the order the P operand takes them.  The 16-byte chunk x of row r sits
//    at chunk x ^ k4swz(r), so that the 16 rows a fragment read touches
//    spread over all LDS banks.
//    k4_scale per tile 512 bytes [h][n][kb][cc] (the scale of tile row
//    32 kb + n, channels [64 cc + 32 h, 64 cc + 32 h + 32); 127 where that
//    block lies past D).
//  - v4: per tile D channel rows of 64 bytes (keys 0..127 of the tile,
//    key 2y in the low nibble of byte y; 16-byte chunk x of row d at chunk
//    x ^ ((d >> 2) & 3)); v4_scale per tile 512 bytes [h][n][cb][c] (the
//    scale of channel 32 cb + n, keys [64 c + 32 h, 64 c + 32 h + 32)).
//  The bytes of one lane (h = lane / 32, n = lane % 32) are its 8 scale
//  operands of a tile, read as one 8-byte load.
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

// mx_block_exp for a block's maximum p = 2^lm (finite), without the loop:
// with p = m 2^f, m in [0.5, 1), the answer is f - 3, plus one when
// m > 0.75 (then 6 2^(f - 3) = 0.75 2^f < p), at least -127; 0 for p = 0
VC_DEV int mx_block_exp_prob(float p) {
  const int e = __builtin_amdgcn_frexp_expf(p) - 3 + (__builtin_amdgcn_frexp_mantf(p) > 0.75f ? 1 : 0);
  return p > 0.0f ? max(e, -127) : 0;
}

// 8 fp32 -> 8 E2M1 nibbles (one dword, element i in nibble i) at scale 2^e
VC_DEV u32 cvt8_fp4(const float (&x)[8], float scale) {
  // the four conversions below write every byte of w: it starts from an
  // unset register (an empty asm defines it), not from a zero written first
  u32 w;
  asm volatile("" : "=v"(w));
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[0], x[1], scale, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[2], x[3], scale, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[4], x[5], scale, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[6], x[7], scale, 3);
  return w;
}

// tile row holding key k of the tile (inverse of the row -> key map above):
// key 64 c + 32 h + 16 b + 4 j + v sits in row 64 c + 32 b + 8 j + 4 h + v
VC_DEV int k4_row_of_key(int k) { return (k & 64) | ((k & 28) << 1) | ((k >> 3) & 4) | (k & 3); }
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
    kts[(32 * (blk & 1) + (row & 31)) * 8 + 2 * (row >> 5) + (blk >> 1)] = (uint8_t)(e + 127);
  }
  // D = 64 has one 64-channel chunk: the second chunk's bytes hold 2^0
  if (D == 64)
    for (int item = tid; item < 256; item += 256) kts[2 * item + 1] = 127;
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
    vts[(32 * (g & 1) + (d & 31)) * 8 + 2 * (d >> 5) + (g >> 1)] = (uint8_t)(e + 127);
  }
  for (int item = tid; item < 64 * 8; item += 256)  // channel blocks past D / 32: scale 2^0
    if ((item & 7) >= D / 16) vts[item] = 127;
}

// ---- attention ----
//
// One workgroup = one 128-query tile of one (b, h) (4 waves x 32 queries),
// two workgroups per CU: their barriers are independent, so one
// workgroup's VALU work overlaps the other's matrix-core work on each SIMD.
// K/V tiles come in the mid-window order through a 2-stage LDS ring that the
// 4 waves fill with global_load_lds_dwordx4.  The products are
// v_mfma_scale_f32_32x32x64_f8f6f4 (FP4 operands): a wave's 32 queries are
// one product's 32 columns, so lane l holds query l % 32 in both halves
// (h = l / 32) and each half carries 32 of a product's 64 K values.  Every
// product holds the SIMD's VALU issue for about the same few cycles
// whatever its size, so the 32x32 products, each twice the work of a
// 16x16x128 one, take half as many of those cycles.  Per tile:
// S^T = K Q^T (scores in log2 units; tile row 32 kb + 8 j + 4 h + v of key
// block kb lands in register 4 j + v of lane half h), the running max as
// an integer (rises within a headroom left unapplied), p = 2^(s - M)
// (v_exp_f32), one E8M0 scale per lane and
// 64-key chunk (its 32 keys: one P block), E2M1 codes, then the row sum
// (ones x P^T) and A^T += V^T P^T on the block-scaled matrix cores, and with
// V-Smooth the block mean restored as A += r mu.

typedef float v16f __attribute__((ext_vector_type(16)));

// how far a tile's max may exceed the running max before it is applied
// (log2 units)
constexpr float kHeadroom4 = 8.0f;

VC_DEV v16f mfma32_fp4(v8i a, v8i b, v16f c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 4, 4, 0, sa, 0, sb);
}
// the same product with the A operand's E8M0 scale taken as byte k of the
// 8 scale bytes s: the product's own byte select picks it out of its dword,
// so no instruction extracts it (k is a constant once the loops unroll)
VC_DEV v16f mfma32_fp4_sa(v8i a, v8i b, v16f c, const uint2& s, int k, int sb) {
  const int w = (int)(k < 4 ? s.x : s.y);
  switch (k & 3) {
    case 0: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 4, 4, 0, w, 0, sb);
    case 1: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 4, 4, 1, w, 0, sb);
    case 2: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 4, 4, 2, w, 0, sb);
    default: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 4, 4, 3, w, 0, sb);
  }
}
VC_DEV v16f mfma32_bf16(v8bf a, v8bf b, v16f c) { return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0); }

// max over the two 32-lane halves (lanes l and l ^ 32 hold the same query)
VC_DEV float max_over_halves(float x) {
  const int xi = __float_as_int(x);
  const auto p32 = __builtin_amdgcn_permlane32_swap(xi, xi, false, false);
  return __builtin_fmaxf(__int_as_float(p32[0]), __int_as_float(p32[1]));
}

template <int D, bool VS>
__global__ __launch_bounds__(256, 2) void attn4_kernel(
    const uint8_t* __restrict__ q4, const uint8_t* __restrict__ q4s, const uint8_t* __restrict__ k4,
    const uint8_t* __restrict__ k4s, const uint8_t* __restrict__ v4, const uint8_t* __restrict__ v4s,
    const uint16_t* __restrict__ mu, uint16_t* __restrict__ o, int64_t oB, int64_t oS, int64_t oH, int S, int H,
    int nblk, int npair, int window, int sequential) {
  constexpr int NC = D / 64;        // 64-channel chunks of the score product
  constexpr int NO = D / 32;        // 32-channel blocks of the output
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
  const int tid = threadIdx.x, l = tid & 63, n = l & 31, hh = l >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wq = w & 3;
  const int qt = pr;  // one query tile per workgroup
  const int64_t S_pad = (int64_t)nblk * kBlk;
  const int start = __builtin_amdgcn_readfirstlane(sequential ? 0 : min((qt | 1) + window, nblk - 1));
  auto tile_at = [&](int i) -> int { return sequential ? i : (i <= start ? start - i : i); };

  // Q fragments of the wave's 32 queries: chunk c, lane half hh holds
  // channels 64 c + 32 hh .. + 31 of query n, with their scale
  v8i qf[NC];
  int qsc[NC];
  {
    const int64_t qrow = (int64_t)bh * S_pad + qt * kBlk + 32 * wq + n;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const uint4 qv = *(const uint4*)(q4 + qrow * (D / 2) + 32 * c + 16 * hh);
      qf[c] = v8i{(int)qv.x, (int)qv.y, (int)qv.z, (int)qv.w, 0, 0, 0, 0};
      qsc[c] = q4s[qrow * NB + 2 * c + hh];
    }
  }

  // copies of tile i into stage st: each wave a quarter of the K and of the V tile
  constexpr int CW = TB / 4;  // bytes per wave (2 KB at D = 128)
  const unsigned loff = (unsigned)l * 16u;
  // (destinations as LDS addresses, taken once: a stage is an integer offset)
  const unsigned kst_a = lds_addr_of(kst), vst_a = lds_addr_of(vst), mring_a = lds_addr_of(mring);
  auto issue = [&](int i, int st) {
    const int64_t t = (int64_t)bh * nblk + tile_at(i);
    const uint8_t* ks = k4 + t * TB + w * CW;
    const uint8_t* vs = v4 + t * TB + w * CW;
    const unsigned kd = kst_a + (unsigned)(st * TB + w * CW), vd = vst_a + (unsigned)(st * TB + w * CW);
    if constexpr (CW == 2048) {  // two 1 KB blocks under one M0 each
      lds_dma16_kb_at<2>(ks + loff, kd);
      lds_dma16_kb_at<2>(vs + loff, vd);
    } else {
#pragma unroll
      for (int r = 0; r < (CW + 1023) / 1024; ++r) {
        if (l * 16 < CW - 1024 * r) {
          lds_dma16_at(ks + 1024 * r + loff, kd + 1024 * r);
          lds_dma16_at(vs + 1024 * r + loff, vd + 1024 * r);
        }
      }
    }
    if (VS && w == 0 && l < D / 8)
      lds_dma16_at((const uint8_t*)(mu + t * D) + loff, mring_a + (unsigned)((i & (MR - 1)) * (VS ? D : 8) * 2));
  };
  // per-lane scale bytes of tile i: K byte 2 kb + c, V byte 2 cb + c
  auto load_scales = [&](int i, uint2& ks, uint2& vs) {
    const int64_t t = (int64_t)bh * nblk + tile_at(i);
    ks = *(const uint2*)(k4s + t * 512 + l * 8);
    vs = *(const uint2*)(v4s + t * 512 + l * 8);
  };

  const v8i ones = {0x22222222, 0x22222222, 0x22222222, 0x22222222, 0, 0, 0, 0};  // E2M1 1.0
  v16f zero16;
#pragma unroll
  for (int e = 0; e < 16; ++e) zero16[e] = 0.f;
  // M: running max of query n (log2 units, an integer); the score product
  // starts its accumulator at -M, so it emits s - M directly (0 before the
  // first tile, which always sets M)
  float M = 0.f;
  v16f cinit = zero16;
  float L = 0.f;
  v16f O[NO];  // A^T: lane half hh holds channels 32 cb + 8 j + 4 hh + v of query n
#pragma unroll
  for (int cb = 0; cb < NO; ++cb) O[cb] = zero16;

  // V-Smooth: row sums of window slots 4 hh .. 4 hh + 3 (lane half hh),
  // restored every 8 tiles on the bf16 matrix cores as A += r mu^T: element
  // 2q / 2q + 1 of lane half hh carries slot 4 hh + q as
  //   mean side: (mu, mu)   (mu is exact in bf16)
  //   sum side:  (r.hi, r.lo)
  float rb[4] = {0.f, 0.f, 0.f, 0.f};
  const bool hi_half = hh != 0;
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
    // S^T = K Q^T: key block kb is tile rows 32 kb + n (A operand), chunk c
    v16f Sc[4];
    uint4 kv[4][NC];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int r = 32 * kb + n;
#pragma unroll
      for (int c = 0; c < NC; ++c) kv[kb][c] = *(const uint4*)(Kt + r * (D / 2) + 16 * ((2 * c + hh) ^ k4swz<D>(r)));
    }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const v8i kf = {(int)kv[kb][c].x, (int)kv[kb][c].y, (int)kv[kb][c].z, (int)kv[kb][c].w, 0, 0, 0, 0};
        Sc[kb] = mfma32_fp4_sa(kf, qf[c], c == 0 ? cinit : Sc[kb], ksc, 2 * kb + c, qsc[c]);
      }
    }
    // every K fragment read goes out before the first score product
    __builtin_amdgcn_sched_group_barrier(0x100, 4 * NC, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 4 * NC, 0);
    // V fragments of both chunks, read now so that their latency hides
    // behind the max and the probabilities: channel block cb is row
    // 32 cb + n, keys 64 cp + 32 hh .. + 31
    uint4 vf[2][NO];
#pragma unroll
    for (int cp = 0; cp < 2; ++cp)
#pragma unroll
      for (int cb = 0; cb < NO; ++cb) {
        const int d = 32 * cb + n;
        vf[cp][cb] = *(const uint4*)(Vt + d * 64 + 16 * ((2 * cp + hh) ^ v4swz(d)));
      }
    const int t = tile_at(i);
    if (t == nblk - 1 && (S % kBlk) != 0) {  // keys past S: no probability
      // opaque to the compiler, so the compares stay in this branch instead
      // of being hoisted out of the loop as 64 live lane masks
      int lim = S - t * kBlk;
      asm volatile("" : "+s"(lim));
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e)  // register e of block kb is key 64 (kb / 2) + 32 hh + 16 (kb % 2) + e
          if (64 * (kb >> 1) + 32 * hh + 16 * (kb & 1) + e >= lim) Sc[kb][e] = -INFINITY;
    }
    // the lane's max over each 64-key chunk (its 32 keys: one P block), the
    // row's max over both halves, and the rescale on an increase
    float lm[2];
#pragma unroll
    for (int cp = 0; cp < 2; ++cp) {
      float m = __builtin_fmaxf(Sc[2 * cp][0], Sc[2 * cp][1]);
#pragma unroll
      for (int e = 2; e < 32; e += 2)
        m = __builtin_fmaxf(__builtin_fmaxf(m, Sc[2 * cp + (e >> 4)][e & 15]), Sc[2 * cp + (e >> 4)][(e & 15) + 1]);
      lm[cp] = m;
    }
    // M is an integer (log2 units), the ceiling of the scores' max: a
    // rescale is then an exact power of two, and moving M by an integer n
    // moves each P block's exponent by n and none of its codes.  So a rise
    // of at most kHeadroom4 is left unapplied (p then stays below 2^9): the
    // output is the same, and most tiles skip the rescale ([OVC] "Mid-window
    // key traversal": without ExpCast a stale maximum has headroom)
    const float rm = max_over_halves(__builtin_fmaxf(lm[0], lm[1]));  // the row's max of s - M
    const bool rise = i == 0 || rm > kHeadroom4;
    if (__any(rise)) {
      const float delta = rise ? -__builtin_ceilf(rm) : 0.0f;  // M - M', an integer
      if (i != 0) {
        const float alpha = __builtin_ldexpf(1.0f, (int)delta);
        L *= alpha;
        if (VS) {
#pragma unroll
          for (int q = 0; q < 4; ++q) rb[q] *= alpha;
        }
#pragma unroll
        for (int cb = 0; cb < NO; ++cb) O[cb] = O[cb] * alpha;
      }
      M -= delta;
#pragma unroll
      for (int e = 0; e < 16; ++e) cinit[e] = -M;
      lm[0] += delta;
      lm[1] += delta;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) Sc[kb] = Sc[kb] + delta;
    }
    // probabilities and codes of chunk cp: element 8 q + e of the lane's P
    // operand is key 64 cp + 32 hh + 8 q + e, register 8 (q % 2) + e of
    // key block 2 cp + q / 2
    v8i P[2];
    int pe[2];
    auto probs = [&](int cp) {
      const float pmax = __builtin_amdgcn_exp2f(lm[cp]);  // below 2^9: lm <= the headroom
      const int e = mx_block_exp_prob(pmax);
      const float sc = ldexpf(1.0f, e);
      pe[cp] = e + 127;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float p8[8];
#pragma unroll
        for (int x = 0; x < 8; ++x) p8[x] = __builtin_amdgcn_exp2f(Sc[2 * cp + (q >> 1)][8 * (q & 1) + x]);
        P[cp][q] = (int)cvt8_fp4(p8, sc);
      }
      P[cp][4] = P[cp][5] = P[cp][6] = P[cp][7] = 0;
    };
    // row sum over both chunks and A^T += V^T P^T for chunk cp
    v16f rs;
    auto pv = [&](int cp) {
      rs = mfma32_fp4(ones, P[cp], cp == 0 ? zero16 : rs, 127, pe[cp]);
#pragma unroll
      for (int cb = 0; cb < NO; ++cb) {
        const uint4 vv = vf[cp][cb];
        const v8i a = {(int)vv.x, (int)vv.y, (int)vv.z, (int)vv.w, 0, 0, 0, 0};
        O[cb] = mfma32_fp4_sa(a, P[cp], O[cb], vsc, 2 * cb + cp, pe[cp]);
      }
    };
    probs(0);
    // chunk 0's codes stay ahead of chunk 1's conversions, so its products
    // can run beside them (the compiler's own placement of the products
    // measured faster than a fixed interleave)
    asm volatile("" ::"v"(P[0][0]), "v"(P[0][1]), "v"(P[0][2]), "v"(P[0][3]), "v"(pe[0]));
    pv(0);
    probs(1);
    pv(1);
    const float rr = rs[0];
    L += rr;
    if (VS) {
      const int slot = i & 7;
      // the lanes whose half carries this slot (a lane mask picked by a
      // scalar test, so the selects below need no per-lane compare)
      const bool mine = (slot >> 2) ? hi_half : !hi_half;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (mine && (slot & 3) == q) rb[q] = rr;
      if (slot == 7 || i == nblk - 1) {
        v8bf Br;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const __bf16 hi = (__bf16)rb[q];
          Br[2 * q] = hi;
          Br[2 * q + 1] = (__bf16)(rb[q] - (float)hi);
          rb[q] = 0.f;
        }
#pragma unroll
        for (int cb = 0; cb < NO; ++cb) {
          // window slot 4 hh + q is visit i - slot + 4 hh + q; slots past i
          // hold zero row sums, so whatever finite row the ring holds there
          // adds nothing
          v8bf Am;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const __bf16 m = __builtin_bit_cast(__bf16, mring[(i - slot + 4 * hh + q) & (MR - 1)][32 * cb + n]);
            Am[2 * q] = m;
            Am[2 * q + 1] = m;
          }
          O[cb] = mfma32_bf16(Am, Br, O[cb]);
        }
      }
    }
    ksc = ksn;
    vsc = vsn;
    wait_vm();        // this wave's copies of tile i + 1 have landed
    __syncthreads();  // every wave is done with stage st and sees stage st ^ 1
  }

  // the last products feed the stores below, which some lanes skip: use
  // every accumulator before that branch, so no product moves into it
  asm volatile("" ::"v"(L));
#pragma unroll
  for (int cb = 0; cb < NO; ++cb)
#pragma unroll
    for (int e = 0; e < 16; e += 4) asm volatile("" ::"v"(O[cb][e]), "v"(O[cb][e + 1]), "v"(O[cb][e + 2]), "v"(O[cb][e + 3]));
  const int b = bh / H, h = bh % H;
  uint16_t* ob = o + b * oB + h * oH;
  const int q = qt * kBlk + 32 * wq + n;
  if (q >= S) return;
  const float inv = 1.0f / L;
#pragma unroll
  for (int cb = 0; cb < NO; ++cb) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d = 32 * cb + 8 * j + 4 * hh;
      const u32 lo = (u32)f32_to_bf16(O[cb][4 * j] * inv) | ((u32)f32_to_bf16(O[cb][4 * j + 1] * inv) << 16);
      const u32 hi = (u32)f32_to_bf16(O[cb][4 * j + 2] * inv) | ((u32)f32_to_bf16(O[cb][4 * j + 3] * inv) << 16);
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
