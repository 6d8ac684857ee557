// vc_quantize.hip -- FP8 operand preparation (HBM-bound streaming kernels).
//
// [OVC] "Scheduling around ExpCast" / "Fused input preparation": Q and K are
// quantised to E4M3 with one scale per 128-token block, V with one scale per
// head, V written transposed with keys contiguous ("Packed V").  The Q/K
// block scales are powers of two, and Q is multiplied by G = 8 fl(sm_scale
// log2 e) first: the factors the blog folds into the code's multiply-add go
// into the FP8 operands and the matrix core's E8M0 block scales instead.  Three
// stream-ordered passes as on the blog: Q/K per block; V per-head maximum;
// V convert into the packed layout.  [VC] §3.1 gives X_q = s_X * Xhat.
//
// Each block kernel streams one 128-token x D tile: 256 threads, 16-byte
// loads (each row is D contiguous bf16), amax through a wave then LDS
// reduction, E4M3 conversion with the hardware round-half-even convert.
#include "vc_common.hpp"
#include "vc_prep.hpp"
#include "vc_vscale.hpp"
#include "vc_launch.hpp"

namespace vc {

namespace {

// amax over 8 bf16 packed in a uint4
VC_DEV float amax8(uint4 w, float m) {
  m = fmaxf(m, fabsf(bf16_lo(w.x)));
  m = fmaxf(m, fabsf(bf16_hi(w.x)));
  m = fmaxf(m, fabsf(bf16_lo(w.y)));
  m = fmaxf(m, fabsf(bf16_hi(w.y)));
  m = fmaxf(m, fabsf(bf16_lo(w.z)));
  m = fmaxf(m, fabsf(bf16_hi(w.z)));
  m = fmaxf(m, fabsf(bf16_lo(w.w)));
  m = fmaxf(m, fabsf(bf16_hi(w.w)));
  return m;
}

// 8 bf16 * inv -> 8 E4M3 bytes
VC_DEV uint2 codes8(uint4 w, float inv) {
  uint2 r;
  r.x = cvt4_fp8(bf16_lo(w.x) * inv, bf16_hi(w.x) * inv, bf16_lo(w.y) * inv, bf16_hi(w.y) * inv);
  r.y = cvt4_fp8(bf16_lo(w.z) * inv, bf16_hi(w.z) * inv, bf16_lo(w.w) * inv, bf16_hi(w.w) * inv);
  return r;
}

VC_DEV float block_max256(float m, float* red) {
  m = wave_max(m);
  int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  return m;
}

// Q or K: one workgroup per (block j, head h, batch b).  PACK writes the
// packed K layout (chunk-swizzled rows), otherwise plain row-major codes.
// With preprocessing ([VC] §3.4, App. B), each valid row is first rotated
// (RoPE at its position), centred (K: minus the head's channel mean, from the
// fixed-point sums of k_center_sums) and transformed by the unnormalised
// Walsh-Hadamard matrix, all in fp32.  Each element is then multiplied by
// pre (Q: G = 8 fl(sm_scale log2 e), over D with the rotation; K: 1); the
// block scale is the power of two pow2_block_exp picks for the products'
// amax (the max of the rounded products).
// GATHER: block j holds rows gat[128 j + r] (r < 128) of the head's tokens,
// the last listed row repeated past its end R ([OVC] "Why V residual
// repair": the keys of the repair rows, prepared as at their own positions);
// nblk then counts the output blocks.
template <int D, bool PACK, bool GATHER>
__global__ __launch_bounds__(256) void qk_block_quant(const uint16_t* __restrict__ x, int64_t sB, int64_t sS,
                                                      int64_t sH, int S, int H, int nblk, float pre, PrepArgs pp,
                                                      uint8_t* __restrict__ codes, float* __restrict__ scale,
                                                      const int32_t* __restrict__ gat, int R) {
  constexpr int CPR = D / 8;             // 16-byte chunks per row
  constexpr int NCH = kBlk * CPR / 256;  // chunks per thread
  __shared__ float red[4];
  const int j = blockIdx.x, h = blockIdx.y, b = blockIdx.z, t = threadIdx.x;
  const int64_t bh = (int64_t)b * H + h;
  const uint16_t* xb = x + b * sB + h * sH;
  const int ch = t % CPR;  // the same chunk for every row of this thread
  // token of block row r; K (PACK) rows past the end repeat the last row,
  // so a ragged tile's max over all its rows is that of its valid rows
  auto token = [&](int r) -> int {
    if constexpr (GATHER) {
      const int i = j * kBlk + r;
      const int tok = gat[bh * R + (i < R ? i : R - 1)];
      return tok < 0 ? 0 : (tok < S ? tok : S - 1);  // in bounds whatever the list holds
    } else if constexpr (PACK) {
      const int tok = j * kBlk + r;
      return tok < S ? tok : S - 1;
    } else {
      return j * kBlk + r;
    }
  };
  float xv[NCH][8];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int row = (t + 256 * i) / CPR, tok = token(row);
    unpack8(tok < S ? *(const uint4*)(xb + (int64_t)tok * sS + ch * 8) : make_uint4(0, 0, 0, 0), xv[i]);
  }
  if (pp.flags) {
    float cm[8];
    if (pp.flags & kPrepCenter) {
#pragma unroll
      for (int e2 = 0; e2 < 8; ++e2) cm[e2] = fx24_mean_of(pp.ksum[bh * D + ch * 8 + e2], S);
    }
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int row = (t + 256 * i) / CPR, tok = token(row);
      if (tok < S) {
        if (pp.flags & kPrepRope) rope8(xv[i], pp.cs + (int64_t)tok * (D / 2) + ch * 4, pp.sn + (int64_t)tok * (D / 2) + ch * 4);
        if (pp.flags & kPrepCenter)
#pragma unroll
          for (int e2 = 0; e2 < 8; ++e2) xv[i][e2] -= cm[e2];
      }
      if (pp.flags & kPrepHadamard) fwht_row8<CPR>(xv[i], ch);  // every lane of the row takes part
    }
  }
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < NCH; ++i)
#pragma unroll
    for (int e2 = 0; e2 < 8; ++e2) m = fmaxf(m, fabsf(xv[i][e2] * pre));
  m = block_max256(m, red);
  const int e = pow2_block_exp(m);
  const float p2 = ldexpf(1.0f, -e);
  if (t == 0) scale[bh * nblk + j] = ldexpf(1.0f, e);
  uint8_t* cb = codes + (bh * nblk * kBlk + (int64_t)j * kBlk) * D;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int row = (t + 256 * i) / CPR;
    const int off = PACK ? kpack_off<D>(row, ch >> 1) + (ch & 1) * 8 : row * D + ch * 8;
    auto f = [&](int e2) { return (xv[i][e2] * pre) * p2; };
    uint2 r;
    r.x = cvt4_fp8(f(0), f(1), f(2), f(3));
    r.y = cvt4_fp8(f(4), f(5), f(6), f(7));
    *(uint2*)(cb + off) = r;
  }
}

// K centring statistics: per (b, h), the fixed-point sums over all S keys of
// each channel after RoPE, added into ksum [B][H][D] (zeroed first).  One
// workgroup per (128-key block, head, batch), the same row/chunk map as
// qk_block_quant; the sums of a workgroup are combined in LDS first.
template <int D>
__global__ __launch_bounds__(256) void k_center_sums(const uint16_t* __restrict__ x, int64_t sB, int64_t sS,
                                                     int64_t sH, int S, int H, PrepArgs pp,
                                                     unsigned long long* __restrict__ ksum) {
  constexpr int CPR = D / 8;
  constexpr int NCH = kBlk * CPR / 256;
  constexpr int RG = 256 / CPR;
  __shared__ long long ps[RG][D];
  const int j = blockIdx.x, h = blockIdx.y, b = blockIdx.z, t = threadIdx.x;
  const int64_t bh = (int64_t)b * H + h;
  const uint16_t* xb = x + b * sB + h * sH;
  const int ch = t % CPR, rg = t / CPR;
  long long acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int row = (t + 256 * i) / CPR, tok = j * kBlk + row;
    if (tok < S) {
      float xv[8];
      unpack8(*(const uint4*)(xb + (int64_t)tok * sS + ch * 8), xv);
      if (pp.flags & kPrepRope) rope8(xv, pp.cs + (int64_t)tok * (D / 2) + ch * 4, pp.sn + (int64_t)tok * (D / 2) + ch * 4);
#pragma unroll
      for (int e2 = 0; e2 < 8; ++e2) acc[e2] += fx24_ll(xv[e2]);
    }
  }
#pragma unroll
  for (int e2 = 0; e2 < 8; ++e2) ps[rg][ch * 8 + e2] = acc[e2];
  __syncthreads();
  for (int d = t; d < D; d += 256) {
    long long sum = 0;
    for (int r = 0; r < RG; ++r) sum += ps[r][d];
    atomicAdd(ksum + bh * D + d, (unsigned long long)sum);  // two's complement: signed sums add exactly
  }
}

__global__ void zero_u64(unsigned long long* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0ull;
}

// V pass 1: per-(b,h) amax as ordered uint bits, accumulated into
// out[bh * stride] (zeroed beforehand).  256 tokens per workgroup.
template <int D>
__global__ __launch_bounds__(256) void v_amax(const uint16_t* __restrict__ x, int64_t sB, int64_t sS, int64_t sH,
                                              int S, int H, float* __restrict__ out, int stride) {
  constexpr int CPR = D / 8;
  constexpr int NCH = 256 * CPR / 256;
  __shared__ float red[4];
  const int h = blockIdx.y, b = blockIdx.z, t = threadIdx.x;
  const uint16_t* xb = x + b * sB + h * sH;
  float m = 0.0f;
#pragma unroll 4
  for (int i = 0; i < NCH; ++i) {
    int c = t + 256 * i, row = c / CPR, ch = c % CPR, tok = blockIdx.x * 256 + row;
    if (tok < S) m = amax8(*(const uint4*)(xb + (int64_t)tok * sS + ch * 8), m);
  }
  m = block_max256(m, red);
  if (t == 0) atomicMax((unsigned int*)(out + ((int64_t)b * H + h) * stride), __float_as_uint(m));
}

__global__ void v_amax_zero(float* out, int BH, int stride) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < BH) out[(int64_t)i * stride] = 0.0f;
}

// V pass 2: convert one 128-token block and write it as a packed V tile
// (channel rows of 128 key bytes, chunk-swizzled).
template <int D>
__global__ __launch_bounds__(256) void v_convert(const uint16_t* __restrict__ x, int64_t sB, int64_t sS, int64_t sH,
                                                 int S, int H, int nblk, const float* __restrict__ v_scale,
                                                 uint8_t* __restrict__ v8) {
  constexpr int CPR = D / 8;
  constexpr int NCH = kBlk * CPR / 256;
  constexpr int LD = D + 4;  // LDS row pitch in bytes (spreads banks on the transposed read)
  __shared__ uint8_t tile[kBlk * LD];
  const int j = blockIdx.x, h = blockIdx.y, b = blockIdx.z, t = threadIdx.x;
  const int64_t bh = (int64_t)b * H + h;
  const uint16_t* xb = x + b * sB + h * sH;
  float s, inv;
  scale_pair(v_scale[bh * D], s, inv);
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    int c = t + 256 * i, row = c / CPR, ch = c % CPR, tok = j * kBlk + row;
    uint4 w = tok < S ? *(const uint4*)(xb + (int64_t)tok * sS + ch * 8) : make_uint4(0, 0, 0, 0);
    uint2 cd = codes8(w, inv);
    *(u32*)(tile + row * LD + ch * 8) = cd.x;
    *(u32*)(tile + row * LD + ch * 8 + 4) = cd.y;
  }
  __syncthreads();
  uint8_t* ob = v8 + (bh * nblk + j) * (int64_t)D * kBlk;  // packed V tile j
  constexpr int TASKS = D * (kBlk / 16);
#pragma unroll
  for (int i = 0; i < TASKS / 256; ++i) {
    int task = t + 256 * i, d = task / (kBlk / 16), c = task % (kBlk / 16), k0 = c * 16;
    u32 w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      w[q] = (u32)tile[vkey_of_pos(k0 + 4 * q) * LD + d] | ((u32)tile[vkey_of_pos(k0 + 4 * q + 1) * LD + d] << 8) |
             ((u32)tile[vkey_of_pos(k0 + 4 * q + 2) * LD + d] << 16) |
             ((u32)tile[vkey_of_pos(k0 + 4 * q + 3) * LD + d] << 24);
    *(uint4*)(ob + vpack_off(d, c)) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// V pass 3: amax bits -> scale, repeated over the D channels.
__global__ void v_finalize(float* v_scale, int D) {
  const int64_t bh = blockIdx.x;
  float amax = v_scale[bh * D];
  __syncthreads();
  float s, inv;
  scale_pair(amax, s, inv);
  for (int d = threadIdx.x; d < D; d += blockDim.x) v_scale[bh * D + d] = s;
}

// bf16 V -> packed bf16 V for the baseline: per (b, h), tile j, half hf
// (64 keys): D rows of 64 keys, 8-key chunk c of row d at chunk
// c ^ (vswz(d) & 7).
template <int D>
__global__ __launch_bounds__(256) void v_pack_bf16(const uint16_t* __restrict__ x, int64_t sB, int64_t sS,
                                                   int64_t sH, int S, int H, int nblk, uint16_t* __restrict__ vt) {
  constexpr int CPR = D / 8;
  constexpr int NCH = kBlk * CPR / 256;
  constexpr int LD = D + 2;  // elements
  __shared__ uint16_t tile[kBlk * LD];
  const int j = blockIdx.x, h = blockIdx.y, b = blockIdx.z, t = threadIdx.x;
  const int64_t bh = (int64_t)b * H + h;
  const uint16_t* xb = x + b * sB + h * sH;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    int c = t + 256 * i, row = c / CPR, ch = c % CPR, tok = j * kBlk + row;
    uint4 w = tok < S ? *(const uint4*)(xb + (int64_t)tok * sS + ch * 8) : make_uint4(0, 0, 0, 0);
    u32* dst = (u32*)(tile + row * LD + ch * 8);
    dst[0] = w.x;
    dst[1] = w.y;
    dst[2] = w.z;
    dst[3] = w.w;
  }
  __syncthreads();
  uint16_t* ob = vt + (bh * nblk + j) * (int64_t)kBlk * D;  // tile j: two 64-key halves of D x 64
  constexpr int TASKS = D * (kBlk / 8);
#pragma unroll
  for (int i = 0; i < TASKS / 256; ++i) {
    int task = t + 256 * i, d = task / (kBlk / 8), k0 = (task % (kBlk / 8)) * 8;
    const int hf = k0 / 64, c = (k0 % 64) / 8;
    u32 w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) w[q] = (u32)tile[(k0 + 2 * q) * LD + d] | ((u32)tile[(k0 + 2 * q + 1) * LD + d] << 16);
    *(uint4*)(ob + hf * D * 64 + d * 64 + ((c ^ vswz(d)) & 7) * 8) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// The ExpCast code map alone (same byte routine as the attention kernel,
// plus the explicit upper clip at 120).
__global__ void expcast_codes_kernel(const float* __restrict__ x, const float* __restrict__ a,
                                     const float* __restrict__ b, int64_t n, int32_t row_len,
                                     uint8_t* __restrict__ codes) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  int64_t r = i / row_len;
  u32 w = VC_EXPCAST_BYTE(0u, a[r], x[i], b[r], 0);
  codes[i] = (uint8_t)min(w & 0xffu, 120u);
}

}  // namespace

hipError_t launch_k_center_sums(const vc_shape& sh, Bshd x, PrepArgs pp, unsigned long long* ksum, hipStream_t st) {
  const int nblk = (sh.S + kBlk - 1) / kBlk;
  const int64_t n = (int64_t)sh.B * sh.H * sh.D;
  zero_u64<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(ksum, n);
  dim3 grid(nblk, sh.H, sh.B);
  if (sh.D == 128)
    k_center_sums<128><<<grid, 256, 0, st>>>(x.p, x.sB, x.sS, x.sH, sh.S, sh.H, pp, ksum);
  else
    k_center_sums<64><<<grid, 256, 0, st>>>(x.p, x.sB, x.sS, x.sH, sh.S, sh.H, pp, ksum);
  return hipGetLastError();
}

namespace {
template <bool GATHER>
hipError_t qk_quant_t(const vc_shape& sh, Bshd x, float pre, PrepArgs pp, uint8_t* codes, float* scale, bool pack,
                      int nb, const int32_t* gat, int R, hipStream_t st) {
  dim3 grid(nb, sh.H, sh.B);
  if (sh.D == 128) {
    if (pack)
      qk_block_quant<128, true, GATHER><<<grid, 256, 0, st>>>(x.p, x.sB, x.sS, x.sH, sh.S, sh.H, nb, pre, pp, codes,
                                                               scale, gat, R);
    else
      qk_block_quant<128, false, GATHER><<<grid, 256, 0, st>>>(x.p, x.sB, x.sS, x.sH, sh.S, sh.H, nb, pre, pp, codes,
                                                                scale, gat, R);
  } else {
    if (pack)
      qk_block_quant<64, true, GATHER><<<grid, 256, 0, st>>>(x.p, x.sB, x.sS, x.sH, sh.S, sh.H, nb, pre, pp, codes,
                                                              scale, gat, R);
    else
      qk_block_quant<64, false, GATHER><<<grid, 256, 0, st>>>(x.p, x.sB, x.sS, x.sH, sh.S, sh.H, nb, pre, pp, codes,
                                                               scale, gat, R);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_qk_quant(const vc_shape& sh, Bshd x, float pre, PrepArgs pp, uint8_t* codes, float* scale,
                           bool pack, hipStream_t st) {
  const int nblk = (sh.S + kBlk - 1) / kBlk;
  return qk_quant_t<false>(sh, x, pre, pp, codes, scale, pack, nblk, nullptr, 0, st);
}

hipError_t launch_k_gather_quant(const vc_shape& sh, Bshd k, PrepArgs pp, const int32_t* idx, int R, uint8_t* k8,
                                 float* k_scale, hipStream_t st) {
  if (R <= 0) return hipSuccess;
  return qk_quant_t<true>(sh, k, 1.0f, pp, k8, k_scale, true, (R + kBlk - 1) / kBlk, idx, R, st);
}

hipError_t launch_v_amax(const vc_shape& sh, Bshd v, float* out, int stride, hipStream_t st) {
  const int BH = sh.B * sh.H;
  v_amax_zero<<<(BH + 255) / 256, 256, 0, st>>>(out, BH, stride);
  dim3 g1((sh.S + 255) / 256, sh.H, sh.B);
  if (sh.D == 128)
    v_amax<128><<<g1, 256, 0, st>>>(v.p, v.sB, v.sS, v.sH, sh.S, sh.H, out, stride);
  else
    v_amax<64><<<g1, 256, 0, st>>>(v.p, v.sB, v.sS, v.sH, sh.S, sh.H, out, stride);
  return hipGetLastError();
}

hipError_t launch_v_quant(const vc_shape& sh, Bshd v, uint8_t* v8, float* v_scale, hipStream_t st) {
  int nblk = (sh.S + kBlk - 1) / kBlk;
  const hipError_t e = launch_v_amax(sh, v, v_scale, sh.D, st);
  if (e != hipSuccess) return e;
  dim3 g2(nblk, sh.H, sh.B);
  if (sh.D == 128)
    v_convert<128><<<g2, 256, 0, st>>>(v.p, v.sB, v.sS, v.sH, sh.S, sh.H, nblk, v_scale, v8);
  else
    v_convert<64><<<g2, 256, 0, st>>>(v.p, v.sB, v.sS, v.sH, sh.S, sh.H, nblk, v_scale, v8);
  v_finalize<<<sh.B * sh.H, 128, 0, st>>>(v_scale, sh.D);
  return hipGetLastError();
}

hipError_t launch_pack_v_bf16(const vc_shape& sh, Bshd v, uint16_t* vt, hipStream_t st) {
  int nblk = (sh.S + kBlk - 1) / kBlk;
  dim3 grid(nblk, sh.H, sh.B);
  if (sh.D == 128)
    v_pack_bf16<128><<<grid, 256, 0, st>>>(v.p, v.sB, v.sS, v.sH, sh.S, sh.H, nblk, vt);
  else
    v_pack_bf16<64><<<grid, 256, 0, st>>>(v.p, v.sB, v.sS, v.sH, sh.S, sh.H, nblk, vt);
  return hipGetLastError();
}

hipError_t launch_expcast_codes(const float* x, const float* a, const float* b, int64_t n, int32_t row_len,
                                uint8_t* codes, hipStream_t st) {
  if (n == 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  expcast_codes_kernel<<<(unsigned)blocks, 256, 0, st>>>(x, a, b, n, row_len, codes);
  return hipGetLastError();
}

}  // namespace vc
