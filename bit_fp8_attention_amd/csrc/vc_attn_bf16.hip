// vc_attn_bf16.hip -- in-house BF16 flash-attention baseline on the same
// kernel skeleton as the FP8 ExpCast kernel: one workgroup per 128-query
// tile (4 waves x 32 queries), the same mid-window key order, K/V streamed
// HBM -> LDS with global_load_lds_dwordx4 and double-buffered, S^T = K Q^T so
// each lane holds one query's keys in the order the P.V operand needs, row
// sums through a matrix-core product against ones, the same epilogue.
//
// What differs is the arithmetic the pages contrast with ExpCast ([VC] §3.1
// Eq. 1, §3.3; [OVC] opening paragraph): BF16 matrix-core products
// (v_mfma_f32_16x16x32_bf16), and per score an fp32 exponential
// p = exp2(acc * scale * log2 e - m) followed by a cast to bf16.  Key tiles
// are processed as two 64-key halves so that the double-buffered bf16 tiles
// fit the same 64 KB of LDS per workgroup.
#include <type_traits>

#include "vc_common.hpp"
#include "vc_launch.hpp"

namespace vc {

namespace {

constexpr int kHalf = 64;  // keys per LDS stage

// K half-tile in LDS: 64 rows x 256 bytes; 16-byte chunk c of row r sits at
// chunk c ^ swb(r) (rows read together by a fragment differ in bits 0,1,3,4).
VC_DEV int swb(int r) { return (r & 3) | (((r >> 3) & 3) << 2); }

// Packed bf16 V (written by vc_pack_v_bf16): per (b, h), tile j, half hf: a
// contiguous block of D rows x 64 keys x 2 bytes; 16-byte chunk c (8 keys)
// of channel row d at chunk c ^ (vswz(d) & 7).
VC_DEV int vpack_bf16_off(int d, int c) { return d * 128 + ((c ^ vswz(d)) & 7) * 16; }

template <int D>
__global__ __launch_bounds__(256, 2) void attn_bf16_kernel(const uint16_t* __restrict__ q, int64_t qB, int64_t qS,
                                                           int64_t qH, const uint16_t* __restrict__ k, int64_t kB,
                                                           int64_t kS, int64_t kH, const uint16_t* __restrict__ vt,
                                                           uint16_t* __restrict__ o, int64_t oB, int64_t oS,
                                                           int64_t oH, int S, int H, int nblk, float c1, int window,
                                                           int sequential) {
  constexpr int NM = D / 16;          // channel blocks
  constexpr int NKC = D / 32;         // 32-wide d chunks of QK^T
  constexpr int KBYTES = kHalf * D * 2;
  constexpr int VBYTES = D * kHalf * 2;
  constexpr int NI = KBYTES / 1024 / 4;  // DMA copies per wave per operand
  // two separate LDS objects so the DMA into one does not make the compiler
  // wait before reads of the other
  __shared__ __attribute__((aligned(1024))) uint8_t lds0[KBYTES + VBYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t lds1[KBYTES + VBYTES];

  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int qt = __builtin_amdgcn_readfirstlane(lin % nblk);
  const int bh = __builtin_amdgcn_readfirstlane(lin / nblk);
  const int b = bh / H, h = bh % H;
  const int tid = threadIdx.x, l = tid & 63, lr = l & 15, g = l >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint16_t* qb = q + b * qB + h * qH;
  const uint16_t* kbp = k + b * kB + h * kH;
  const uint8_t* vb = (const uint8_t*)(vt + (int64_t)bh * nblk * kBlk * D);

  // the FP8 kernel's order: `window` blocks past the diagonal of the
  // query-tile pair (qt | 1)
  const int start = __builtin_amdgcn_readfirstlane(sequential ? 0 : min((qt | 1) + window, nblk - 1));
  auto tile_at = [&](int i) -> int { return sequential ? i : (i <= start ? start - i : i); };

  // per-lane DMA sources of the K half-tile: LDS byte p = (4r + w) KB + 16 l
  // holds K row p / 256, logical chunk (p % 256 / 16) ^ swb(row)
  int krow[NI], kcol[NI];
#pragma unroll
  for (int r = 0; r < NI; ++r) {
    const int p = (r * 4 + w) * 1024 + l * 16;
    krow[r] = p / (D * 2);
    kcol[r] = (((p % (D * 2)) / 16) ^ (D == 128 ? swb(krow[r]) : (swb(krow[r]) & 7))) * 8;
  }
  auto issue = [&](int step, uint8_t* buf) {
    const int t = tile_at(step >> 1), hf = step & 1;
    const int key0 = t * kBlk + hf * kHalf;
#pragma unroll
    for (int r = 0; r < NI; ++r) {
      const int key = min(key0 + krow[r], S - 1);  // rows past S are masked, any valid row will do
      lds_dma16(kbp + (int64_t)key * kS + kcol[r], buf + (r * 4 + w) * 1024);
    }
    const uint8_t* vsrc = vb + ((int64_t)t * 2 + hf) * VBYTES;
#pragma unroll
    for (int r = 0; r < NI; ++r)
      lds_dma16(vsrc + (r * 4 + w) * 1024 + l * 16, buf + KBYTES + (r * 4 + w) * 1024);
  };

  // Q^T fragments: sub-tile s, d chunk kc: lane holds query lr, d = 32 kc + 8 g .. + 7
  v8bf qf[2][NKC];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int qrow = min(qt * kBlk + 32 * w + 16 * s + lr, S - 1);
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      uint4 x = *(const uint4*)(qb + (int64_t)qrow * qS + 32 * kc + 8 * g);
      qf[s][kc] = __builtin_bit_cast(v8bf, x);
    }
  }

  // fragment lane bases: K block blk (16 keys) of the half-tile, lane row lr
  // holds key 32 (blk / 2) + 8 (lr / 4) + 4 (blk & 1) + lr % 4
  const v4f zero4 = {0.f, 0.f, 0.f, 0.f};
  v8bf ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (__bf16)1.0f;
  float M[2] = {-INFINITY, -INFINITY};
  float Lq[2] = {0.f, 0.f};
  v4f O[2][NM];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int m = 0; m < NM; ++m) O[s][m] = zero4;

  const int nsteps = 2 * nblk;
  const bool ragged = (S % kBlk) != 0;
  issue(0, lds0);

  auto step_body = [&](int st, uint8_t* cur, uint8_t* nxt, auto tail_tag) {
    constexpr bool TAIL = decltype(tail_tag)::value;
    wait_vm();
    __syncthreads();
    if (st + 1 < nsteps) issue(st + 1, nxt);
    const uint8_t* Kt = cur;
    const uint8_t* Vt = cur + KBYTES;
    const int key0 = tile_at(st >> 1) * kBlk + (st & 1) * kHalf;

    v4f Sc[2][4];
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
      const int row = 32 * (blk >> 1) + 8 * (lr >> 2) + 4 * (blk & 1) + (lr & 3);
      Sc[0][blk] = zero4;
      Sc[1][blk] = zero4;
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        const int ch = (4 * kc + g) ^ (D == 128 ? swb(row) : (swb(row) & 7));
        v8bf kf = __builtin_bit_cast(v8bf, *(const uint4*)(Kt + row * D * 2 + ch * 16));
        Sc[0][blk] = mfma_bf16(kf, qf[0][kc], Sc[0][blk]);
        Sc[1][blk] = mfma_bf16(kf, qf[1][kc], Sc[1][blk]);
      }
    }
    if constexpr (TAIL) {
      const int lim = S - key0;
#pragma unroll
      for (int blk = 0; blk < 4; ++blk)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (32 * (blk >> 1) + 8 * g + 4 * (blk & 1) + v >= lim) {
            Sc[0][blk][v] = -INFINITY;
            Sc[1][blk][v] = -INFINITY;
          }
    }
    v8bf P[2][2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      float mx = __builtin_fmaxf(Sc[s][0][0], Sc[s][0][1]);
#pragma unroll
      for (int e = 2; e < 16; e += 2)
        mx = __builtin_fmaxf(__builtin_fmaxf(mx, Sc[s][e >> 2][e & 3]), Sc[s][(e + 1) >> 2][(e + 1) & 3]);
      mx = max_over_groups(mx);
      const float Mn = __builtin_fmaxf(M[s], c1 * mx);
      if (__any(Mn > M[s])) {
        const float alpha = exp2f(M[s] - Mn);
        Lq[s] *= alpha;
        float a4[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) a4[v] = __shfl(alpha, 4 * g + v);
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
          for (int m = 0; m < NM; ++m) O[s][m][v] *= a4[v];
        M[s] = Mn;
      }
      const float nm = -M[s];
#pragma unroll
      for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            P[s][p][4 * hb + v] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(Sc[s][2 * p + hb][v], c1, nm));
    }
#pragma unroll
    for (int m = 0; m < NM; ++m) {
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        v8bf vf = __builtin_bit_cast(v8bf, *(const uint4*)(Vt + vpack_bf16_off(16 * m + lr, 4 * p + g)));
        O[0][m] = mfma_bf16(P[0][p], vf, O[0][m]);
        O[1][m] = mfma_bf16(P[1][p], vf, O[1][m]);
      }
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      v4f r = mfma_bf16(ones, P[s][0], zero4);
      r = mfma_bf16(ones, P[s][1], r);
      Lq[s] += r[0];
    }
  };

  // the ragged last tile is the first two steps or the last two
  const bool tail_first = ragged && tile_at(0) == nblk - 1;
  const bool tail_last = ragged && !tail_first;
  int s0 = 0, s1 = nsteps;
  if (tail_first) {
    step_body(0, lds0, lds1, std::true_type{});
    step_body(1, lds1, lds0, std::true_type{});
    s0 = 2;
  }
  if (tail_last) s1 = nsteps - 2;
  // s0, s1 and nsteps are even: even steps read lds0, odd steps lds1
  for (int st = s0; st < s1; st += 2) {
    step_body(st, lds0, lds1, std::false_type{});
    step_body(st + 1, lds1, lds0, std::false_type{});
  }
  if (tail_last) {
    step_body(nsteps - 2, lds0, lds1, std::true_type{});
    step_body(nsteps - 1, lds1, lds0, std::true_type{});
  }

  uint16_t* ob = o + b * oB + h * oH;
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int qi = qt * kBlk + 32 * w + 16 * s + 4 * g + v;
      const float lsum = __shfl(Lq[s], 4 * g + v);
      if (qi >= S) continue;
      const float inv = 1.0f / lsum;
#pragma unroll
      for (int m = 0; m < NM; ++m) ob[(int64_t)qi * oS + 16 * m + lr] = f32_to_bf16(O[s][m][v] * inv);
    }
}

}  // namespace

hipError_t launch_attn_bf16(const vc_shape& sh, float sm_scale, int window, uint32_t flags, Bshd q, Bshd k,
                            const uint16_t* vt, BshdOut o, hipStream_t st) {
  const float c1 = sm_scale * 1.44269504088896340736f;
  const int seq = (flags & VC_ATTN_SEQUENTIAL) ? 1 : 0;
  const int nblk = (sh.S + kBlk - 1) / kBlk;
  const int64_t n = (int64_t)nblk * sh.H * sh.B;
  if (sh.D == 128)
    attn_bf16_kernel<128><<<(unsigned)n, 256, 0, st>>>(q.p, q.sB, q.sS, q.sH, k.p, k.sB, k.sS, k.sH, vt, o.p, o.sB,
                                                        o.sS, o.sH, sh.S, sh.H, nblk, c1, window, seq);
  else
    attn_bf16_kernel<64><<<(unsigned)n, 256, 0, st>>>(q.p, q.sB, q.sS, q.sH, k.p, k.sB, k.sS, k.sH, vt, o.p, o.sB,
                                                       o.sS, o.sH, sh.S, sh.H, nblk, c1, window, seq);
  return hipGetLastError();
}

}  // namespace vc
