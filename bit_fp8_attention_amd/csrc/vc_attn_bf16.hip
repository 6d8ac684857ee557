// vc_attn_bf16.hip -- in-house BF16 flash-attention baseline on the same
// kernel skeleton as the FP8 ExpCast kernel: one workgroup of 8 waves holds
// two 128-query tiles of one (b, h) that share one K/V stream; the two
// 4-wave halves alternate a matrix-core phase and a VALU phase one phase
// apart (barrier ping-pong); K/V stream HBM -> LDS with global_load_lds into
// 4-stage rings, issued by half A in its VALU phase; fragments are read two
// MFMA pairs ahead;
// S^T = K Q^T; the output is accumulated transposed (V^T P^T) so rescales
// stay in the lane; row sums come from a matrix-core product against ones;
// the same mid-window key order and epilogue.
//
// What differs is the arithmetic the pages contrast with ExpCast ([VC] §3.1
// Eq. 1, §3.3; [OVC] opening paragraph): BF16 matrix-core products
// (v_mfma_f32_16x16x32_bf16), and per score an fp32 exponential
// p = exp2(acc * scale * log2 e - m) followed by a cast to bf16.  As in a
// BF16 FlashAttention-4 kernel, a rise of the running max m of at most
// kHeadroom is left unapplied ([OVC] "Mid-window key traversal": without
// ExpCast a stale maximum has headroom; the probabilities then stay below
// 2^9, where bf16 keeps the same relative precision).  A step is
// a 64-key half-tile, so the bf16 K and V stages (16 KB each) fill the same
// 128 KB of rings as the FP8 kernel's 128-key tiles.
#include "vc_common.hpp"
#include "vc_launch.hpp"

namespace vc {

namespace {

constexpr int kHalf = 64;  // keys per step
// how far a step's max may exceed the running max before it is applied
// (log2 units)
constexpr float kHeadroom = 8.0f;

// K half-tile in LDS: 64 rows x 2D bytes; 16-byte chunk c of row r sits at
// chunk c ^ swb(r) (rows read together by a fragment differ in bits 0,1,3,4).
VC_DEV int swb(int r) { return (r & 3) | (((r >> 3) & 3) << 2); }

// Packed bf16 V (written by vc_pack_v_bf16): per (b, h), tile j, half hf: a
// contiguous block of D rows x 64 keys x 2 bytes; 16-byte chunk c (8 keys)
// of channel row d at chunk c ^ (vswz(d) & 7).
VC_DEV int vpack_bf16_off(int d, int c) { return d * 128 + ((c ^ vswz(d)) & 7) * 16; }

template <int D>
__global__ __launch_bounds__(512, 1) void attn_bf16_kernel(const uint16_t* __restrict__ q, int64_t qB, int64_t qS,
                                                           int64_t qH, const uint16_t* __restrict__ k, int64_t kB,
                                                           int64_t kS, int64_t kH, const uint16_t* __restrict__ vt,
                                                           uint16_t* __restrict__ o, int64_t oB, int64_t oS,
                                                           int64_t oH, int S, int H, int nblk, int npair, float c1,
                                                           int window, int sequential) {
  constexpr int NM = D / 16;           // channel blocks
  constexpr int NKC = D / 32;          // 32-wide d chunks of QK^T
  constexpr int TB = kHalf * D * 2;    // bytes of one K or V half-tile
  constexpr int NI = TB / 1024 / 4;    // 1 KB copies per issuing wave per half-tile
  __shared__ __attribute__((aligned(1024))) uint8_t kring[4][TB];
  __shared__ __attribute__((aligned(1024))) uint8_t vring[4][TB];
  uint8_t* const kst0 = kring[0];
  uint8_t* const kst1 = kring[1];
  uint8_t* const vst0 = vring[0];
  uint8_t* const vst3 = vring[3];

  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int pr = __builtin_amdgcn_readfirstlane(lin % npair);
  const int bh = __builtin_amdgcn_readfirstlane(lin / npair);
  const int b = bh / H, h = bh % H;
  const int tid = threadIdx.x, l = tid & 63, lr = l & 15, g = l >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool hb = w >= 4;  // half B: one phase behind
  const int wq = w & 3;
  const bool live = 2 * pr + (hb ? 1 : 0) < nblk;
  const int qt = __builtin_amdgcn_readfirstlane(live ? 2 * pr + (hb ? 1 : 0) : nblk - 1);
  const int n = 2 * nblk;  // steps (64-key half-tiles)
  const uint16_t* qb = q + b * qB + h * qH;
  const uint16_t* kbp = k + b * kB + h * kH;
  const uint8_t* vb = (const uint8_t*)(vt + (int64_t)bh * nblk * kBlk * D);

  const int start = __builtin_amdgcn_readfirstlane(sequential ? 0 : min(2 * pr + 1 + window, nblk - 1));
  auto tile_at = [&](int i) -> int { return sequential ? i : (i <= start ? start - i : i); };

  // per-lane sources of the K half-tile copies of wave wq: LDS byte
  // p = (4r + wq) KB + 16 l holds K row p / (2D), logical chunk
  // (p % 2D / 16) ^ swb(row)
  int krow[NI], kcol[NI];
#pragma unroll
  for (int r = 0; r < NI; ++r) {
    const int p = (r * 4 + wq) * 1024 + l * 16;
    krow[r] = p / (D * 2);
    kcol[r] = (((p % (D * 2)) / 16) ^ (D == 128 ? swb(krow[r]) : (swb(krow[r]) & 7))) * 8;
  }
  // copy destinations as LDS addresses, taken once: a stage is an integer
  // offset from its ring
  const unsigned kring_a = lds_addr_of(kring), vring_a = lds_addr_of(vring);
  auto kdst = [&](int i) { return kring_a + (unsigned)((i & 3) * TB); };
  auto vdst = [&](int i) { return vring_a + (unsigned)((i & 3) * TB); };
  auto issue_k = [&](unsigned dst, int j) {
    const int key0 = tile_at(j >> 1) * kBlk + (j & 1) * kHalf;
#pragma unroll
    for (int r = 0; r < NI; ++r) {
      const int key = min(key0 + krow[r], S - 1);  // rows past S are masked; any valid row will do
      lds_dma16_at(kbp + (int64_t)key * kS + kcol[r], dst + (unsigned)((r * 4 + wq) * 1024));
    }
  };
  // V half-tiles are contiguous: the wave's NI consecutive 1 KB blocks under one M0
  auto issue_v = [&](unsigned dst, int j) {
    const uint8_t* vsrc = vb + ((int64_t)tile_at(j >> 1) * 2 + (j & 1)) * TB;
    lds_dma16_kb_at<NI>(vsrc + wq * NI * 1024 + l * 16, dst + (unsigned)(wq * NI * 1024));
  };
  constexpr int GRP = 2 * NI;  // copies per half-A wave per step
  // the stages of step i (i mod 4; picked at run time): a shift, as one
  // array per ring
  auto kst_of = [&](int i) -> uint8_t* { return kring[i & 3]; };
  auto vst_of = [&](int i) -> uint8_t* { return vring[i & 3]; };


  // the ragged last tile is steps 0, 1 or steps n - 2, n - 1
  const bool ragged = (S % kBlk) != 0;
  const bool tail_first = ragged && tile_at(0) == nblk - 1;
  const bool tail_last = ragged && !tail_first;

  if (!hb) {  // prologue (half A): K_0, V_0, K_1, then K_2, V_1; K_0 must have landed before M(0)
    issue_k(kdst(0), 0);
    issue_v(vdst(0), 0);
    if (1 < n) issue_k(kdst(1), 1);
    if (2 < n) issue_k(kdst(2), 2);
    if (1 < n) issue_v(vdst(1), 1);
    if (n >= 3)
      wait_vm_n<4 * NI>();
    else
      wait_vm();
  }

  // Q^T fragments: sub-tile s, d chunk kc: lane holds query lr, d = 32 kc + 8 g .. + 7
  v8bf qf[2][NKC];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int qrow = min(qt * kBlk + 32 * wq + 16 * s + lr, S - 1);
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      uint4 x = *(const uint4*)(qb + (int64_t)qrow * qS + 32 * kc + 8 * g);
      qf[s][kc] = __builtin_bit_cast(v8bf, x);
    }
  }
  float zq0;  // an opaque zero accumulator, as in the FP8 kernel
  asm volatile("v_mov_b32 %0, 0" : "=v"(zq0));
  const v4f zq = {zq0, zq0, zq0, zq0};
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
  v4f Sc[2][4];  // S^T of the current step: key block blk holds keys 32 (blk / 2) + 8 g + 4 (blk & 1) + v
  v8bf P[2][2];  // bf16 probabilities of the previous step, as the P.V B operand

  // ---- M phase: row sums of P_{j-1}, A^T += V_{j-1}^T P_{j-1}^T, then
  // S_j^T = K_j Q^T.  Fragment k: V block (m = k / 2, key half p = k % 2)
  // for k < 2 NM, then K (chunk kc, block blk) for k = 2 NM + 4 kc + blk;
  // each read two MFMA pairs ahead. ----
  auto mphase = [&](int j, const uint8_t* Kt, const uint8_t* Vt, auto pv_tag, auto qk_tag) {
    constexpr bool PV = decltype(pv_tag)::value;
    constexpr bool QK = decltype(qk_tag)::value;
    constexpr int NV = 2 * NM;
    constexpr int K0 = PV ? 0 : NV;
    constexpr int K1 = QK ? NV + 4 * NKC : NV;
    auto frag = [&](auto kk) -> v8bf {
      constexpr int k = decltype(kk)::value;
      if constexpr (k < NV) {
        return __builtin_bit_cast(v8bf, *(const uint4*)(Vt + vpack_bf16_off(16 * (k / 2) + lr, 4 * (k % 2) + g)));
      } else {
        constexpr int kc = (k - NV) / 4, blk = (k - NV) % 4;
        const int row = 32 * (blk >> 1) + 8 * (lr >> 2) + 4 * (blk & 1) + (lr & 3);
        const int ch = (4 * kc + g) ^ (D == 128 ? swb(row) : (swb(row) & 7));
        return __builtin_bit_cast(v8bf, *(const uint4*)(Kt + row * D * 2 + ch * 16));
      }
    };
    v8bf fr[3];
    if constexpr (K0 < K1) fr[K0 % 3] = frag(std::integral_constant<int, K0>{});
    if constexpr (K0 + 1 < K1) fr[(K0 + 1) % 3] = frag(std::integral_constant<int, K0 + 1>{});
    float rr[2] = {0.f, 0.f};
    if constexpr (PV) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        v4f r = mfma_bf16(ones, P[s][0], zq);
        r = mfma_bf16(ones, P[s][1], r);
        rr[s] = r[0];
      }
    }
    static_for<K0, K1>([&](auto kk) {
      constexpr int k = decltype(kk)::value;
      if constexpr (k + 2 < K1) fr[(k + 2) % 3] = frag(std::integral_constant<int, k + 2>{});
      const v8bf f = fr[k % 3];
      if constexpr (k < NV) {
        O[0][k / 2] = mfma_bf16(f, P[0][k % 2], O[0][k / 2]);
        O[1][k / 2] = mfma_bf16(f, P[1][k % 2], O[1][k / 2]);
      } else {
        constexpr int kc = (k - NV) / 4, blk = (k - NV) % 4;
        Sc[0][blk] = mfma_bf16(f, qf[0][kc], kc == 0 ? zq : Sc[0][blk]);
        Sc[1][blk] = mfma_bf16(f, qf[1][kc], kc == 0 ? zq : Sc[1][blk]);
      }
    });
    if constexpr (K0 < K1) {
      __builtin_amdgcn_sched_group_barrier(0x100, K0 + 1 < K1 ? 2 : 1, 0);
      if constexpr (PV) __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      static_for<K0, K1>([&](auto kk) {
        constexpr int k = decltype(kk)::value;
        if constexpr (k + 2 < K1) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      });
    }
    if constexpr (PV) {
      Lq[0] += rr[0];
      Lq[1] += rr[1];
    }
    (void)j;
  };

  // ---- V phase: running max, rescale, probabilities of step j; half A
  // then copies K_{j+3} and V_{j+2} ----
  auto vphase = [&](int j, bool tail) {
    if (tail) {
      const int lim = S - (tile_at(j >> 1) * kBlk + (j & 1) * kHalf);
#pragma unroll
      for (int blk = 0; blk < 4; ++blk)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (32 * (blk >> 1) + 8 * g + 4 * (blk & 1) + v >= lim) {
            Sc[0][blk][v] = -INFINITY;
            Sc[1][blk][v] = -INFINITY;
          }
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      float mx = __builtin_fmaxf(Sc[s][0][0], Sc[s][0][1]);
#pragma unroll
      for (int e = 2; e < 16; e += 2)
        mx = __builtin_fmaxf(__builtin_fmaxf(mx, Sc[s][e >> 2][e & 3]), Sc[s][(e + 1) >> 2][(e + 1) & 3]);
      mx = max_over_groups(mx);
      // the first step always applies (M = -inf before it)
      const float Mn = c1 * mx > M[s] + kHeadroom ? c1 * mx : M[s];
      if (__any(Mn > M[s])) {
        const float alpha = exp2f(M[s] - Mn);
        Lq[s] *= alpha;
#pragma unroll
        for (int m = 0; m < NM; ++m) O[s][m] = O[s][m] * alpha;  // the lane's own query
        M[s] = Mn;
      }
      const float nm = -M[s];
#pragma unroll
      for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int hb2 = 0; hb2 < 2; ++hb2)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            P[s][p][4 * hb2 + v] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(Sc[s][2 * p + hb2][v], c1, nm));
    }
    // half A: K_{j+3} and V_{j+2} into the stages of K_{j-1} and V_{j-2}
    // (read for the last time in half B's M(j - 1), one slot earlier), then
    // wait until only these and the previous step's copies are in flight,
    // so the barrier ending this slot publishes K_{j+1} and V_j
    if (!hb) {
      if (j + 3 < n) issue_k(kdst(j + 3), j + 3);
      if (j + 2 < n) issue_v(vdst(j + 2), j + 2);
      if (j + 3 < n)
        wait_vm_n<2 * GRP>();
      else
        wait_vm();
    }
  };

  phase_sync();
  if (hb) phase_sync();  // half B: one phase behind
  const std::true_type T{};
  const std::false_type F{};
  // steps 0 and 1 (the ragged tile's halves when it is visited first)
  mphase(0, kst0, vst3, F, T);
  phase_sync();
  vphase(0, tail_first);
  phase_sync();
  mphase(1, kst1, vst0, T, T);
  phase_sync();
  vphase(1, tail_first);
  phase_sync();
  // steady state, steps 2 .. n - 3.  The loop stays rolled with the stages
  // picked at run time (j mod 4): unrolled copies each kept the output
  // accumulators in registers of their own and spilled.
  for (int j = 2; j < n - 2; ++j) {
    mphase(j, kst_of(j), vst_of(j - 1), T, T);
    phase_sync();
    vphase(j, false);
    phase_sync();
  }
  // steps n - 2 and n - 1 (n >= 2 always; when n == 2 they are steps 0, 1 above)
  if (n > 2) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int jj = n - 2 + e;
      mphase(jj, kst_of(jj), vst_of(jj - 1), T, T);
      phase_sync();
      vphase(jj, tail_last);
      phase_sync();
    }
  }
  mphase(n, nullptr, vst_of(n - 1), T, F);  // the last P.V (V_{n-1})
  if (!hb) phase_sync();  // half A's extra barrier, matching half B's first
  wait_vm();              // no copy may outlive the workgroup's LDS

  if (!live) return;
  uint16_t* ob = o + b * oB + h * oH;
  // lane (g, lr) holds query lr of each sub-tile, channels 16m + 4g + v
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int qi = qt * kBlk + 32 * wq + 16 * s + lr;
    if (qi >= S) continue;
    const float inv = 1.0f / Lq[s];
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const int d = 16 * m + 4 * g;
      const u32 lo = (u32)f32_to_bf16(O[s][m][0] * inv) | ((u32)f32_to_bf16(O[s][m][1] * inv) << 16);
      const u32 hi = (u32)f32_to_bf16(O[s][m][2] * inv) | ((u32)f32_to_bf16(O[s][m][3] * inv) << 16);
      *(uint2*)(ob + (int64_t)qi * oS + d) = make_uint2(lo, hi);
    }
  }
}

}  // namespace

hipError_t launch_attn_bf16(const vc_shape& sh, float sm_scale, int window, uint32_t flags, Bshd q, Bshd k,
                            const uint16_t* vt, BshdOut o, hipStream_t st) {
  const float c1 = sm_scale * 1.44269504088896340736f;
  const int seq = (flags & VC_ATTN_SEQUENTIAL) ? 1 : 0;
  const int nblk = (sh.S + kBlk - 1) / kBlk;
  const int npair = (nblk + 1) / 2;
  const int64_t n = (int64_t)npair * sh.H * sh.B;
  if (sh.D == 128)
    attn_bf16_kernel<128><<<(unsigned)n, 512, 0, st>>>(q.p, q.sB, q.sS, q.sH, k.p, k.sB, k.sS, k.sH, vt, o.p, o.sB,
                                                        o.sS, o.sH, sh.S, sh.H, nblk, npair, c1, window, seq);
  else
    attn_bf16_kernel<64><<<(unsigned)n, 512, 0, st>>>(q.p, q.sB, q.sS, q.sH, k.p, k.sB, k.sS, k.sH, vt, o.p, o.sB,
                                                       o.sS, o.sH, sh.S, sh.H, nblk, npair, c1, window, seq);
  return hipGetLastError();
}

}  // namespace vc
