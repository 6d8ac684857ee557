// vc_attn_fp8.hip -- non-causal FP8 attention with ExpCast-FP8 and V-Smooth
// mean restoration, for gfx950 (CDNA4) matrix cores.
//
// Method ([VC] = VC-Attention paper, [OVC] = Open-VC blog):
//  - online softmax recurrence m', alpha, A <- alpha A + P V, l <- alpha l + P1
//    ([VC] §3.1 Eq. 1), running maximum on the true (dequantised) score and
//    every increase applied ([OVC] "Scheduling around ExpCast");
//  - each probability is the E4M3 code c = Round(8 g acc + 119.65 - 8 M')
//    ([VC] §3.3 Eq. 7, beta = -0.35).  [OVC] "Scheduling around ExpCast"
//    folds softmax scale, Q/K dequant scales, log2 e, the factor 8 and the
//    running maximum into one multiply-add per score; here they are folded
//    one step earlier, into the score product itself: Q's codes carry
//    8 sm_scale log2 e (vc_quantize), the power-of-two Q/K block scales enter
//    the matrix core as its E8M0 operands, and the accumulator starts at
//    119.65 - 8 M, so the product emits 8 g acc + 119.65 - 8 M directly and a
//    code is one integer conversion (v_cvt_pk_u8_f32: round half-even, clamp
//    at 0, byte into its slot of the operand register) -- no exponential, no
//    FP8 cast, no multiply-add.  Only a tile whose max rises adds the shift
//    8 (M - M') to its scores;
//  - the row sum is taken over the same bytes ([OVC] "A consistent
//    denominator") by a matrix-core product against a tile of ones;
//  - V-Smooth's block mean is restored in the same accumulator,
//    A += r mu^T ([VC] §3.2 Eq. 6), with mu stored divided by the per-channel
//    value scale so one epilogue multiply serves both terms ([VC] App. B);
//  - keys are visited mid-window ([OVC] "Mid-window key traversal").
//
// MI355X mapping:
//  - one workgroup = two 128-query tiles (each its own Q-scale block) of one
//    (b, h), 8 waves x 32 queries; the two 4-wave halves share one stream of
//    K/V tiles and run their matrix-core and VALU phases one phase apart
//    (barrier ping-pong), so on every SIMD one wave's products overlap the
//    other wave's codes;
//  - S^T = K Q^T on v_mfma_f32_16x16x128_f8f6f4 (K = D = 128): the output
//    puts one query and 4 keys in each lane; the packed V tile stores its keys
//    in exactly the order in which those accumulators hand them, as codes, to
//    the P.V product's B operand, so codes go from the accumulator to the PV
//    operand without any shuffle;
//  - K and V are stored tile-major and pre-swizzled (the packed layouts of
//    vc_attn.h), so each 16 KB tile streams HBM -> LDS as one straight copy
//    with global_load_lds_dwordx4 (no VGPR staging, no per-tile address
//    arithmetic; each issuing wave copies a contiguous quarter under one M0)
//    into 4-stage rings, and the 32-byte fragment reads from LDS are
//    bank-conflict free;
//  - workgroup ids are remapped so each XCD works on a contiguous range of
//    query tiles of one head, whose mid-window sweeps hit the same K/V in that
//    XCD's L2.
#include "vc_common.hpp"
#include "vc_launch.hpp"

#include <type_traits>

namespace vc {

namespace {

template <int D>
struct TileLds {
  // K tile: 128 rows (keys) x D bytes; V tile: D rows (channels) x 128 bytes (keys)
  static constexpr int KB = kBlk * D;
  static constexpr int VB = D * kBlk;
  static constexpr int BYTES = KB + VB;
};

// Fragment reads.  For MFMA block t8 the A-operand lane row i = lr holds
// key 16*t8 + lr: the 16 lanes of a group read 16 consecutive K rows, lane
// group g taking logical chunks g and g + 4 (for D = 64: chunk g and zeros),
// which also fixes which channels group g's 32 bytes carry -- Q is loaded
// with the same mapping.  The row swizzle depends on the row's bits 0-3,
// i.e. on lr alone, so every K read is a lane base + 16*t8*D.  For channel
// block m lane column lr holds channel 16m + lr, lane group g chunks g and
// g + 4 of its key row: every V read is a lane base + m*16*128.  The S^T
// accumulator of block t8 holds, in lane group g and register v, key
// 16*t8 + 4g + v -- the key the packed V tile stores at byte 4*t8 + v of
// group g's 32 bytes, so the codes feed P.V unshuffled.
template <int D>
struct FragBase {
  unsigned k0, k1;  // byte offsets of the two 16-byte K chunks (t8 = 0)
  unsigned v0, v1;  // byte offsets of the two 16-byte V chunks (m = 0)
  VC_DEV FragBase(int lr, int g) {
    k0 = kpack_off<D>(lr, g);
    k1 = D == 128 ? kpack_off<D>(lr, g + 4) : 0;
    v0 = vpack_off(lr, g);
    v1 = vpack_off(lr, g + 4);
  }
};

template <int D>
VC_DEV v8i kfrag(const uint8_t* kt, int t8, const FragBase<D>& fb) {
  uint4 lo = *(const uint4*)(kt + fb.k0 + 16 * t8 * D);
  uint4 hi = D == 128 ? *(const uint4*)(kt + fb.k1 + 16 * t8 * D) : make_uint4(0, 0, 0, 0);
  return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

template <int D>
VC_DEV v8i vfrag(const uint8_t* vt, int m, const FragBase<D>& fb) {
  uint4 lo = *(const uint4*)(vt + fb.v0 + m * 16 * kBlk);
  uint4 hi = *(const uint4*)(vt + fb.v1 + m * 16 * kBlk);
  return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// ---------------------------------------------------------------------------
// Two-query-tile ping-pong kernel.
//
// One workgroup of 8 waves holds two 128-query tiles of one (b, h) that share
// one stream of K/V tiles ([OVC] "A warp-specialized pipeline": each CTA holds
// two query tiles that alternate).  Half A (waves 0-3) takes query tile 2p,
// half B (waves 4-7) tile 2p + 1; waves w and w + 4 share a SIMD.  Each wave
// alternates two phases per key tile j:
//   M(j): matrix cores -- P_{j-1} V_{j-1}, the row sums of P_{j-1}, and
//         S_j^T = K_j Q^T;
//   V(j): VALU -- running max, rescale, ExpCast codes P_j.
// Half B runs one phase behind half A (one extra barrier at the start, A one
// at the end), so on every SIMD one wave's matrix-core chain runs while the
// other wave computes codes.  K and V tiles go through two 4-stage LDS rings
// (tile i in stage i mod 4), filled in the V phases: at V(j) the mean row
// j + 2, K_{j+3} and V_{j+2} go into the stages of K_{j-1} and V_{j-2},
// read for the last time in half B's M(j-1), one slot earlier; half A issues
// them all with V-Smooth, and on the plain path half B issues V_{j+2}.
// ---------------------------------------------------------------------------

template <int D, bool VS>
__global__ __launch_bounds__(512, 1) void attn_fp8_kernel(
    const uint8_t* __restrict__ q8, const float* __restrict__ q_scale, const uint8_t* __restrict__ k8,
    const float* __restrict__ k_scale, const uint8_t* __restrict__ v8, const float* __restrict__ v_scale,
    const u32* __restrict__ mu, const uint8_t* __restrict__ rk8, const float* __restrict__ rk_scale,
    const uint8_t* __restrict__ rv8, int nrb, uint16_t* __restrict__ o, int64_t oB, int64_t oS, int64_t oH, int S,
    int H, int nblk, int npair, int window, int sequential) {
  constexpr int NM = D / 16;             // channel blocks of the output
  constexpr int TB = kBlk * D;           // bytes of one K or V tile
  constexpr int NI = TB / 1024 / 4;      // 1 KB copies per issuing wave per tile
  // the K and V rings: four 16 KB stages each
  __shared__ __attribute__((aligned(1024))) uint8_t kring[4][TB];
  __shared__ __attribute__((aligned(1024))) uint8_t vring[4][TB];
  uint8_t* const kst0 = kring[0];
  uint8_t* const vst0 = vring[0];
  uint8_t* const vst3 = vring[3];
  // V-Smooth: ring of the scaled block-mean rows (bf16 hi | lo << 16 per
  // channel) of the last 16 visited tiles (one 8-tile restoration window
  // plus the rows in flight)
  constexpr int MR = VS ? 16 : 1;
  __shared__ __attribute__((aligned(1024))) u32 mring[MR][D];

  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int pr = __builtin_amdgcn_readfirstlane(lin % npair);
  const int bh = __builtin_amdgcn_readfirstlane(lin / npair);
  const int tid = threadIdx.x, l = tid & 63, lr = l & 15, g = l >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, kept scalar
  const bool hb = w >= 4;                                  // half B
  const int wq = w & 3;                                    // wave within the half
  // visits: the nblk regular key tiles, then (plain path) the nrb repair
  // tiles ([OVC] "Why V residual repair": visited last, numerator only)
  const int n = VS ? nblk : nblk + nrb;
  // with an odd number of query tiles, half B of the last pair repeats half
  // A's tile (it must take part in every barrier) and stores nothing
  const bool live = 2 * pr + (hb ? 1 : 0) < nblk;
  const int qt = __builtin_amdgcn_readfirstlane(live ? 2 * pr + (hb ? 1 : 0) : nblk - 1);
  const int64_t S_pad = (int64_t)nblk * kBlk;
  const uint8_t* qb = q8 + (int64_t)bh * S_pad * D;
  const uint8_t* kb = k8 + (int64_t)bh * S_pad * D;
  const uint8_t* vb = v8 + (int64_t)bh * D * S_pad;  // packed: tile t at + t * 128 * D
  const float* ksb = k_scale + (int64_t)bh * nblk;
  // repair tile r is visit nblk + r, and tile_at(i) = i past the regular
  // visits, so the repair bases of the copies are shifted down by nblk tiles
  // (integer arithmetic: the shifted address itself is never read) and a
  // visit's source is base(i) + tile_at(i) * TB either way
  const uint8_t* rkb = (const uint8_t*)((uintptr_t)(rk8 + (int64_t)bh * nrb * TB) - (uintptr_t)nblk * TB);
  const uint8_t* rvb = (const uint8_t*)((uintptr_t)(rv8 + (int64_t)bh * nrb * TB) - (uintptr_t)nblk * TB);
  // the key scales through plain pointers into the arguments, which keeps
  // their read a scalar load
  const float* rksb = rk_scale + (int64_t)bh * nrb;
  // E8M0 block scale of the query tile (Q's codes carry 8 sm_scale log2 e)
  const int sq = __builtin_amdgcn_readfirstlane(e8m0_of_pow2(q_scale[(int64_t)bh * nblk + qt]));

  // mid-window order of the pair: start a few tiles past the pair's diagonal
  const int start = __builtin_amdgcn_readfirstlane(sequential ? 0 : min(2 * pr + 1 + window, nblk - 1));
  auto tile_at = [&](int i) -> int { return sequential ? i : (i <= start ? start - i : i); };
  auto repair_visit = [&](int i) { return !VS && i >= nblk; };
  auto ksrc = [&](int i) { return (repair_visit(i) ? rkb : kb) + (int64_t)tile_at(i) * TB; };
  auto vsrc = [&](int i) { return (repair_visit(i) ? rvb : vb) + (int64_t)tile_at(i) * TB; };
  auto kscale = [&](int i) { return repair_visit(i) ? rksb[i - nblk] : ksb[tile_at(i)]; };

  const unsigned loff = (unsigned)l * 16u;
  // the stages of visit i (i mod 4; picked at run time).  One array per
  // ring, so a stage address is a shift of i mod 4; with a separate object
  // per stage it was a chain of scalar selects at the head of every M phase,
  // ahead of its first fragment read (2.7% slower with V-Smooth)
  auto kst_of = [&](int i) -> uint8_t* { return kring[i & 3]; };
  auto vst_of = [&](int i) -> uint8_t* { return vring[i & 3]; };

  // copies of an issuing wave wq: the tile's NI consecutive 1 KB blocks from
  // wq NI KB on, under one M0; with V-Smooth (half A) also bytes
  // [wq D, (wq + 1) D) of the tile's mean row (D / 16 lanes), issued first
  // in a group, so that a read of the ring waits for no tile
  // copy destinations as LDS addresses: the rings' addresses are taken once
  // and a stage is an integer offset from them
  const unsigned kring_a = lds_addr_of(kring), vring_a = lds_addr_of(vring), mring_a = lds_addr_of(mring);
  auto kdst = [&](int i) { return kring_a + (unsigned)((i & 3) * TB); };
  auto vdst = [&](int i) { return vring_a + (unsigned)((i & 3) * TB); };
  auto issue_mu = [&](int i) {
    if (VS) {
      const uint8_t* msrc = (const uint8_t*)(mu + ((int64_t)bh * nblk + tile_at(i)) * D) + wq * D;
      if (l < D / 16) lds_dma16_at(msrc + loff, mring_a + (unsigned)((i & (MR - 1)) * D * 4 + wq * D));
    }
  };
  auto issue_k = [&](unsigned dst, int i) { lds_dma16_kb_at<NI>(ksrc(i) + wq * NI * 1024 + loff, dst + wq * NI * 1024); };
  auto issue_v = [&](unsigned dst, int i) { lds_dma16_kb_at<NI>(vsrc(i) + wq * NI * 1024 + loff, dst + wq * NI * 1024); };
  constexpr int GRP_A = VS ? 2 * NI + 1 : NI;  // copies per half-A wave per V phase

  const FragBase<D> fb(lr, g);
  // visit of the ragged last key tile: first when the order starts there,
  // else visit nblk - 1 (the last regular one); -1 if S fills its tiles
  const int tail_visit = (S % kBlk) == 0 ? -1 : (tile_at(0) == nblk - 1 ? 0 : nblk - 1);

  if (VS) {  // rows never written must read as finite zeros
    u32* mz = &mring[0][0];
    for (int e = tid; e < MR * D; e += 512) mz[e] = 0u;
    __syncthreads();
  }
  // prologue (half A): mean row 0, K_0, V_0, K_1, then group -1 (mean row 1,
  // K_2, V_1); K_0 must have landed before M(0)
  if (!hb) {
    issue_mu(0);
    issue_k(kdst(0), 0);
    issue_v(vdst(0), 0);
    if (n > 1) issue_k(kdst(1), 1);
    if (1 < n) issue_mu(1);
    if (2 < n) issue_k(kdst(2), 2);
    if (1 < n) issue_v(vdst(1), 1);
    if (n >= 3)
      wait_vm_n<4 * NI + (VS ? 1 : 0)>();
    else
      wait_vm();
  }

  v8i qf[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int qrow = qt * kBlk + 32 * wq + 16 * s + lr;
    const uint8_t* qp = qb + (int64_t)qrow * D;
    const uint4 lo = *(const uint4*)(qp + 16 * g);
    const uint4 hi = D == 128 ? *(const uint4*)(qp + 64 + 16 * g) : make_uint4(0, 0, 0, 0);
    qf[s] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  }

  const v8i ones = {0x38383838, 0x38383838, 0x38383838, 0x38383838,
                    0x38383838, 0x38383838, 0x38383838, 0x38383838};  // E4M3 1.0
  const v4f zero4 = {0.f, 0.f, 0.f, 0.f};
  // code offset 119.65 - 8 M of query lr of each sub-tile, M its running max
  // (log2 units), and the S^T accumulator start holding it; 0 before the
  // first tile, which sets it from that tile's max
  float Bo[2] = {0.f, 0.f};
  float Lq[2] = {0.f, 0.f};             // running denominator of query lr
  v4f O[2][NM];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int m = 0; m < NM; ++m) O[s][m] = zero4;
  // V-Smooth: row sums of the window slots 2g, 2g + 1 that lane group g
  // feeds to the mean product
  float rb[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
  v4f Sc[2][8];                               // S^T of the current tile
  float pm[2];                                // max of its key blocks 0..5 (steady-state tiles)
  int skv = e8m0_of_pow2(kscale(0));          // E8M0 key scale of the current tile
  v4f cinit[2] = {zero4, zero4};
  v8i P[2];                                   // codes of the previous tile

  // ---- M phase: row sums of P_{j-1}, A^T += V_{j-1}^T P_{j-1}^T, then
  // S_j^T = K_j Q^T.  The output is accumulated transposed: the V fragment is
  // the A operand and the codes the B operand, so lane (g, lr) holds channels
  // 16m + 4g + v of query lr -- the query whose max, rescale factor and
  // denominator the lane already holds from S^T, so a rescale needs no
  // cross-lane movement.
  // Fragment k of a phase is V channel block k (k < NM), then K key block
  // k - NM; each is read from LDS two MFMA pairs ahead of its use, so the LDS
  // latency hides behind matrix-core work.  PV / QK are std::true_type or
  // std::false_type, so every index is a compile-time constant. ----
  auto mphase = [&](int j, const uint8_t* Kt, const uint8_t* Vt, auto pv_tag, auto qk_tag, auto pm_tag) {
    constexpr bool PV = decltype(pv_tag)::value;
    constexpr bool QK = decltype(qk_tag)::value;
    // PM: a tile with no masked keys; the running-max tree over its key
    // blocks 0..5 is built here, two MFMA pairs behind their products, on
    // VALU issue slots the matrix-core chain leaves free
    constexpr bool PM = QK && decltype(pm_tag)::value;
    constexpr int K0 = PV ? 0 : NM;
    constexpr int K1 = QK ? NM + 8 : NM;
    constexpr int KD = D == 128 ? 2 : 1;  // LDS reads of one K fragment
    auto frag = [&](auto kk) -> v8i {
      constexpr int k = decltype(kk)::value;
      if constexpr (k < NM)
        return vfrag<D>(Vt, k, fb);
      else
        return kfrag<D>(Kt, k - NM, fb);
    };
    auto nds = [](int k) { return k < NM ? 2 : KD; };
    v8i fr[3];
    if constexpr (K0 < K1) fr[K0 % 3] = frag(std::integral_constant<int, K0>{});
    if constexpr (K0 + 1 < K1) fr[(K0 + 1) % 3] = frag(std::integral_constant<int, K0 + 1>{});
    float rr[2] = {0.f, 0.f};
    v4f rsum[2];
    if constexpr (PV) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        rsum[s] = mfma_fp8(ones, P[s], zero4);
        rr[s] = rsum[s][0];
      }
    }
    static_for<K0, K1>([&](auto kk) {
      constexpr int k = decltype(kk)::value;
      if constexpr (k + 2 < K1) fr[(k + 2) % 3] = frag(std::integral_constant<int, k + 2>{});
      const v8i f = fr[k % 3];
      if constexpr (k < NM) {
        O[0][k] = mfma_fp8(f, P[0], O[0][k]);
        O[1][k] = mfma_fp8(f, P[1], O[1][k]);
      } else {
        Sc[0][k - NM] = mfma_fp8_scaled(f, qf[0], cinit[0], skv, sq);
        Sc[1][k - NM] = mfma_fp8_scaled(f, qf[1], cinit[1], skv, sq);
        if constexpr (PM && k - NM >= 2) {
          constexpr int t8 = k - NM - 2;
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            float m = __builtin_fmaxf(__builtin_fmaxf(t8 == 0 ? Sc[s][0][0] : pm[s], Sc[s][t8][t8 == 0 ? 1 : 0]),
                                      Sc[s][t8][t8 == 0 ? 2 : 1]);
            if (t8 == 0) {
              pm[s] = __builtin_fmaxf(m, Sc[s][0][3]);
            } else {
              pm[s] = __builtin_fmaxf(__builtin_fmaxf(m, Sc[s][t8][2]), Sc[s][t8][3]);
            }
          }
        }
      }
    });
    // issue order: the first two fragments' reads, the row sums, then per
    // fragment k the reads of k + 2 and the two products of k
    if constexpr (K0 < K1) {
      __builtin_amdgcn_sched_group_barrier(0x100, nds(K0) + (K0 + 1 < K1 ? nds(K0 + 1) : 0), 0);
      if constexpr (PV) __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      static_for<K0, K1>([&](auto kk) {
        constexpr int k = decltype(kk)::value;
        if constexpr (k + 2 < K1) __builtin_amdgcn_sched_group_barrier(0x100, nds(k + 2), 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      });
    }
    // with V-Smooth the row sums' whole results stay allocated through the
    // chain: with three of their four registers free, the compiler wrote into
    // one while the product was still in flight, which cost a hazard wait
    // (measured faster with V-Smooth, slightly slower on the plain path)
    if constexpr (PV && VS) asm volatile("" ::"v"(rsum[0]), "v"(rsum[1]));
    // keep the score products in this block, ahead of the mean-restoration
    // branch: the block-scaled products were otherwise moved below it, out
    // of the interleaving above
    if constexpr (QK)
      asm volatile("" ::"v"(Sc[0][0]), "v"(Sc[0][1]), "v"(Sc[0][2]), "v"(Sc[0][3]), "v"(Sc[0][4]), "v"(Sc[0][5]),
                   "v"(Sc[0][6]), "v"(Sc[0][7]), "v"(Sc[1][0]), "v"(Sc[1][1]), "v"(Sc[1][2]), "v"(Sc[1][3]),
                   "v"(Sc[1][4]), "v"(Sc[1][5]), "v"(Sc[1][6]), "v"(Sc[1][7]));
    if constexpr (PV) {
      const int i = j - 1;
      const int slot = i & 7;
      // repair rows: numerator only (a scalar 0 / 1 factor: rr * 1 is exact)
      const float keep = repair_visit(i) ? 0.0f : 1.0f;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        Lq[s] = __builtin_fmaf(rr[s], keep, Lq[s]);
        if (VS) {
          if (slot == 2 * g) rb[s][0] = rr[s];
          if (slot == 2 * g + 1) rb[s][1] = rr[s];
        }
      }
      // V-Smooth mean restoration for the 8-tile window ending at tile i.
      // Lane group g carries window slots 2g (mean pair m0, row sum r0) and
      // 2g + 1 (m1, r1) in K slots 8g .. 8g + 7 as
      //   mean side: (m0.hi, m0.lo, m1.hi, m1.lo, m0.hi, 0, m1.hi, 0)
      //   sum side:  (r0.hi, r0.hi, r1.hi, r1.hi, r0.lo, 0, r1.lo, 0)
      // i.e. r.hi * (hi + lo) + r.lo * hi per slot; the mean side is the two
      // stored pairs as read plus their hi halves
      if (VS && (slot == 7 || i == n - 1)) {
        v8bf Ar[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const __bf16 hi = (__bf16)rb[s][jj];
            const __bf16 lo = (__bf16)(rb[s][jj] - (float)hi);
            Ar[s][2 * jj + 0] = hi;
            Ar[s][2 * jj + 1] = hi;
            Ar[s][4 + 2 * jj + 0] = lo;
            Ar[s][4 + 2 * jj + 1] = (__bf16)0.0f;
            rb[s][jj] = 0.f;
          }
        }
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          // window slot 2g + jj is visit i - slot + 2g + jj; slots past i
          // hold zero row sums, so whatever finite row the ring holds there
          // adds nothing
          const u32 m0 = mring[(i - slot + 2 * g) & (MR - 1)][16 * m + lr];
          const u32 m1 = mring[(i - slot + 2 * g + 1) & (MR - 1)][16 * m + lr];
          const v8bf Bm = __builtin_bit_cast(v8bf, (v4u){m0, m1, m0 & 0xffffu, m1 & 0xffffu});
          O[0][m] = mfma_bf16(Bm, Ar[0], O[0][m]);
          O[1][m] = mfma_bf16(Bm, Ar[1], O[1][m]);
        }
      }
    }
  };

  // ---- V phase: running max, rescale, codes of tile j; half B then issues
  // the copies of K_{j+3} and V_{j+2} into the stages M(j) last read ----
  auto vphase = [&](int j, bool tail, auto pm_tag) {
    constexpr bool PM = decltype(pm_tag)::value;
    const int t = tile_at(j);
    if (tail) {
      const int lim = S - t * kBlk;  // valid keys in this tile
#pragma unroll
      for (int t8 = 0; t8 < 8; ++t8)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (16 * t8 + 4 * g + v >= lim) {
            Sc[0][t8][v] = -INFINITY;
            Sc[1][t8][v] = -INFINITY;
          }
    }
    // the lane's 32 scores of each sub-tile: a max tree of depth 4 (one
    // v_max3_f32 per two scores, as a chain would take, but 4 dependent
    // steps instead of 16), both sub-tiles before either rescale, so the
    // two trees and the two cross-lane reductions overlap
    float mx[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if constexpr (PM) {  // blocks 0..5 came from the M phase
        const float m = __builtin_fmaxf(__builtin_fmaxf(pm[s], Sc[s][6][0]), Sc[s][6][1]);
        const float m2 = __builtin_fmaxf(__builtin_fmaxf(m, Sc[s][6][2]), Sc[s][6][3]);
        const float m3 = __builtin_fmaxf(__builtin_fmaxf(m2, Sc[s][7][0]), Sc[s][7][1]);
        mx[s] = __builtin_fmaxf(__builtin_fmaxf(m3, Sc[s][7][2]), Sc[s][7][3]);
        continue;
      }
      auto x = [&](int e) { return Sc[s][e >> 2][e & 3]; };
      float u[11];
#pragma unroll
      for (int k = 0; k < 10; ++k) u[k] = __builtin_fmaxf(__builtin_fmaxf(x(3 * k), x(3 * k + 1)), x(3 * k + 2));
      u[10] = __builtin_fmaxf(x(30), x(31));
      const float w0 = __builtin_fmaxf(__builtin_fmaxf(u[0], u[1]), u[2]);
      const float w1 = __builtin_fmaxf(__builtin_fmaxf(u[3], u[4]), u[5]);
      const float w2 = __builtin_fmaxf(__builtin_fmaxf(u[6], u[7]), u[8]);
      const float w3 = __builtin_fmaxf(u[9], u[10]);
      mx[s] = __builtin_fmaxf(__builtin_fmaxf(__builtin_fmaxf(w0, w1), w2), w3);
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) mx[s] = max_over_groups(mx[s]);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      // Sc holds 8 g acc + Bo = 8 (score - M) + 119.65: the max rose iff the
      // tile's largest exceeds 119.65; the first tile always sets the offset
      const bool rise = j == 0 || mx[s] > 119.65f;
      if (__any(rise)) {
        const float delta = rise ? 119.65f - mx[s] : 0.0f;  // 8 (M - M'), 0 where the max held
        if (j != 0) {
          const float alpha = exp2f(delta * 0.125f);
          Lq[s] *= alpha;
          if (VS) {
            rb[s][0] *= alpha;
            rb[s][1] *= alpha;
          }
          // whole-vector multiplies (lane-wise: alpha is the lane's own query);
          // per-element updates led the register allocator to keep two copies
          // of the accumulators and spill
#pragma unroll
          for (int m = 0; m < NM; ++m) O[s][m] = O[s][m] * alpha;
        }
        Bo[s] += delta;
        cinit[s] = v4f{Bo[s], Bo[s], Bo[s], Bo[s]};
#pragma unroll
        for (int t8 = 0; t8 < 8; ++t8) Sc[s][t8] = Sc[s][t8] + delta;
      }
#pragma unroll
      for (int t8 = 0; t8 < 8; ++t8) {
        u32 wd = 0;
        wd = __builtin_amdgcn_cvt_pk_u8_f32(Sc[s][t8][0], 0, wd);
        wd = __builtin_amdgcn_cvt_pk_u8_f32(Sc[s][t8][1], 1, wd);
        wd = __builtin_amdgcn_cvt_pk_u8_f32(Sc[s][t8][2], 2, wd);
        wd = __builtin_amdgcn_cvt_pk_u8_f32(Sc[s][t8][3], 3, wd);
        P[s][t8] = (int)wd;
      }
    }
    // the next tile's key scale, a whole phase before it is needed
    if (j + 1 < n) skv = e8m0_of_pow2(kscale(j + 1));
    // The copies of V(j): mean row j + 2, K_{j+3}, V_{j+2}.  Half A issues
    // its share and then waits until only those of V(j - 1) and V(j) are in
    // flight, so the barrier ending this slot publishes the tiles read from
    // the next slot on (K_{j+1}, and V_j when half A copies V).  With
    // V-Smooth half A issues all of them; on the plain path half B copies
    // V_{j+2} (into V_{j-2}'s stage) and waits for it at the end of M(j + 1)
    // (the balance that measured fastest for each path: the issuing wave
    // stalls for several hundred cycles, and the mean flush lengthens the M
    // phases)
    if (!hb) {
      if (j + 2 < n) issue_mu(j + 2);
      if (j + 3 < n) issue_k(kdst(j + 3), j + 3);
      if (VS && j + 2 < n) issue_v(vdst(j + 2), j + 2);
      if (j + 3 < n)
        wait_vm_n<2 * GRP_A>();
      else
        wait_vm();
    } else if (!VS) {
      if (j + 2 < n) issue_v(vdst(j + 2), j + 2);
    }
  };

  // end of an M phase M(j) in half B (plain path): the V copies it issued
  // in V(j - 1) may stay in flight, V_j (issued in V(j - 2)) must have
  // landed (half A's next phase reads it)
  auto mwait = [&](int j) {
    if (!VS && hb) {
      if (j + 1 < n)
        wait_vm_n<NI>();
      else
        wait_vm();
    }
  };

  phase_sync();  // prologue copies visible
  if (hb) phase_sync();  // half B: one phase behind

  // j = 0 (may be the ragged tile; no P.V yet)
  mphase(0, kst0, vst3, std::false_type{}, std::true_type{}, std::false_type{});
  mwait(0);
  phase_sync();
  vphase(0, tail_visit == 0, std::false_type{});
  phase_sync();

  // steady state, rolled: stages picked at run time (j mod 4)
  {
    auto steady = [&](int j, auto mask_tag) {
      mphase(j, kst_of(j), vst_of(j - 1), std::true_type{}, std::true_type{}, std::true_type{});
      mwait(j);
      phase_sync();
      vphase(j, false, std::true_type{});
      // plain path with repair tiles: the ragged tile may fall in here.  The
      // running max above then covered its pad keys, harmless because
      // vc_quantize makes them copies of the last key; their codes are
      // cleared here so that the row sum counts only the valid keys
      if (decltype(mask_tag)::value && j == tail_visit) {
        const int lim = S - (nblk - 1) * kBlk;
#pragma unroll
        for (int t8 = 0; t8 < 8; ++t8) {
          const int k0 = 16 * t8 + 4 * g;  // key of byte 0 of register t8
          const u32 keep = k0 + 4 <= lim ? 0xffffffffu : (k0 >= lim ? 0u : (1u << (8 * (lim - k0))) - 1u);
          P[0][t8] = (int)((u32)P[0][t8] & keep);
          P[1][t8] = (int)((u32)P[1][t8] & keep);
        }
      }
      phase_sync();
    };
    // the loop with that check only where it can matter, so the common loop
    // carries no test
    if (!VS && tail_visit > 0 && tail_visit < n - 1) {
      for (int j = 1; j < n - 1; ++j) steady(j, std::true_type{});
    } else {
      for (int j = 1; j < n - 1; ++j) steady(j, std::false_type{});
    }
  }
  // j = n - 1 (may be the ragged tile); stages chosen at run time
  if (n >= 2) {
    mphase(n - 1, kst_of(n - 1), vst_of(n - 2), std::true_type{}, std::true_type{}, std::false_type{});
    mwait(n - 1);
    phase_sync();
    vphase(n - 1, tail_visit == n - 1, std::false_type{});
    phase_sync();
  }
  // M(n): the last P.V
  mphase(n, nullptr, vst_of(n - 1), std::true_type{}, std::false_type{}, std::false_type{});
  if (!hb) phase_sync();  // half A's extra barrier, matching half B's first
  wait_vm();              // no copy may outlive the workgroup's LDS

  // ---- epilogue: O = (A / l) * s_V, bf16, original query order -----------
  if (!live) return;
  const int b = bh / H, h = bh % H;
  const float* vsb = v_scale + (int64_t)bh * D;
  uint16_t* ob = o + b * oB + h * oH;
  // lane (g, lr) holds query lr of each sub-tile, channels 16m + 4g + v
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int q = qt * kBlk + 32 * wq + 16 * s + lr;
    if (q >= S) continue;
    const float inv = 1.0f / Lq[s];
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const int d = 16 * m + 4 * g;
      const float4 sv = *(const float4*)(vsb + d);
      const u32 lo = (u32)f32_to_bf16((O[s][m][0] * inv) * sv.x) | ((u32)f32_to_bf16((O[s][m][1] * inv) * sv.y) << 16);
      const u32 hi = (u32)f32_to_bf16((O[s][m][2] * inv) * sv.z) | ((u32)f32_to_bf16((O[s][m][3] * inv) * sv.w) << 16);
      *(uint2*)(ob + (int64_t)q * oS + d) = make_uint2(lo, hi);
    }
  }
}

template <int D, bool VS>
hipError_t launch_t(const vc_shape& sh, int window, int seq, const uint8_t* q8, const float* qs,
                    const uint8_t* k8, const float* ks, const uint8_t* v8, const float* vs, const u32* mu,
                    RepairTiles rp, BshdOut o, hipStream_t st) {
  const int nblk = (sh.S + kBlk - 1) / kBlk;
  const int npair = (nblk + 1) / 2;
  const int64_t n = (int64_t)npair * sh.H * sh.B;
  attn_fp8_kernel<D, VS><<<(unsigned)n, 512, 0, st>>>(q8, qs, k8, ks, v8, vs, mu, rp.k8, rp.k_scale, rp.v8, rp.nrb,
                                                          o.p, o.sB, o.sS, o.sH, sh.S, sh.H, nblk, npair, window, seq);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fp8(const vc_shape& sh, int window, uint32_t flags, const uint8_t* q8, const float* q_scale,
                           const uint8_t* k8, const float* k_scale, const uint8_t* v8, const float* v_scale,
                           const u32* mu_split, RepairTiles rp, BshdOut o, hipStream_t st) {
  const int seq = (flags & VC_ATTN_SEQUENTIAL) ? 1 : 0;
  const RepairTiles none{0, nullptr, nullptr, nullptr};
  if (sh.D == 128) {
    if (mu_split)
      return launch_t<128, true>(sh, window, seq, q8, q_scale, k8, k_scale, v8, v_scale, mu_split, none, o, st);
    return launch_t<128, false>(sh, window, seq, q8, q_scale, k8, k_scale, v8, v_scale, nullptr, rp, o, st);
  }
  if (mu_split) return launch_t<64, true>(sh, window, seq, q8, q_scale, k8, k_scale, v8, v_scale, mu_split, none, o, st);
  return launch_t<64, false>(sh, window, seq, q8, q_scale, k8, k_scale, v8, v_scale, nullptr, rp, o, st);
}

}  // namespace vc
