// vc_attn_fp8.hip -- non-causal FP8 attention with ExpCast-FP8 and V-Smooth
// mean restoration, for gfx950 (CDNA4) matrix cores.
//
// Method ([VC] = VC-Attention paper, [OVC] = Open-VC blog):
//  - online softmax recurrence m', alpha, A <- alpha A + P V, l <- alpha l + P1
//    ([VC] §3.1 Eq. 1), running maximum on the true (dequantised) score and
//    every increase applied ([OVC] "Scheduling around ExpCast");
//  - each probability is an E4M3 code from one fused multiply-add into which
//    softmax scale, Q/K dequant scales, log2 e, the factor 8 and the running
//    maximum are folded: c = Round(8 g acc + 119.65 - 8 M') ([VC] §3.3 Eq. 7,
//    beta = -0.35), rounded half-even and clamped at 0 by one integer
//    conversion (v_cvt_pk_u8_f32) that also drops the byte into its slot of
//    the matrix-core operand register -- no exponential, no FP8 cast;
//  - the row sum is taken over the same bytes ([OVC] "A consistent
//    denominator") by a matrix-core product against a tile of ones;
//  - V-Smooth's block mean is restored in the same accumulator,
//    A += r mu^T ([VC] §3.2 Eq. 6), with mu stored divided by the per-channel
//    value scale so one epilogue multiply serves both terms ([VC] App. B);
//  - keys are visited mid-window ([OVC] "Mid-window key traversal").
//
// MI355X mapping:
//  - one workgroup = one 128-query tile (the Q-scale block) of one (b, h):
//    4 waves x 32 queries (two 16-query sub-tiles per wave), two workgroups
//    per CU so that one wave's matrix-core chain overlaps another's VALU work;
//  - S^T = K Q^T on v_mfma_f32_16x16x128_f8f6f4 (K = D = 128): the output
//    puts one query and 4 keys in each lane; the packed V tile stores its keys
//    in exactly the order in which those accumulators hand them to the P.V
//    product's A operand, so codes go from the accumulator to the PV operand
//    without any shuffle;
//  - K and V are stored tile-major and pre-swizzled (the packed layouts of
//    vc_attn.h), so each 16 KB tile streams HBM -> LDS as one straight copy
//    with global_load_lds_dwordx4 (no VGPR staging, no per-tile address
//    arithmetic), double-buffered, and the 32-byte fragment reads from LDS
//    are bank-conflict free;
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

// Issue the asynchronous copies of key tile `t` (two contiguous 16 KB
// blocks in the packed layouts) into LDS buffer `buf`: wave w, copy r moves
// bytes [(4r + w) KB, +1 KB), lane l its 16 bytes at + 16 l.
template <int D>
VC_DEV void issue_tile(uint8_t* buf, const uint8_t* __restrict__ kb, const uint8_t* __restrict__ vb, int t, int w,
                       unsigned loff) {
  constexpr int NI = D * kBlk / 1024 / 4;  // copies per wave per operand
  const uint8_t* kt = kb + (int64_t)t * kBlk * D;
  const uint8_t* vt = vb + (int64_t)t * kBlk * D;
  uint8_t* vbuf = buf + TileLds<D>::KB;
#pragma unroll
  for (int r = 0; r < NI; ++r) {
    const int base = (r * 4 + w) * 1024;
    lds_dma16(kt + base + loff, buf + base);
    lds_dma16(vt + base + loff, vbuf + base);
  }
}

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

template <int D, bool VS>
__global__ __launch_bounds__(256, 2) void attn_fp8_kernel(
    const uint8_t* __restrict__ q8, const float* __restrict__ q_scale, const uint8_t* __restrict__ k8,
    const float* __restrict__ k_scale, const uint8_t* __restrict__ v8, const float* __restrict__ v_scale,
    const float* __restrict__ mu, uint16_t* __restrict__ o, int64_t oB, int64_t oS, int64_t oH, int S, int H,
    int nblk, float c1, int window, int sequential) {
  constexpr int NM = D / 16;  // channel blocks of the output
  // two separate LDS objects (not one array indexed by parity), so the
  // compiler can tell the buffer being filled by DMA from the one being read
  // and does not wait for the copy in flight before reading the other
  __shared__ __attribute__((aligned(1024))) uint8_t lds0[TileLds<D>::BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t lds1[TileLds<D>::BYTES];

  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int qt = __builtin_amdgcn_readfirstlane(lin % nblk);  // workgroup-uniform, kept scalar
  const int bh = __builtin_amdgcn_readfirstlane(lin / nblk);
  const int tid = threadIdx.x, l = tid & 63, lr = l & 15, g = l >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, kept scalar
  const int64_t S_pad = (int64_t)nblk * kBlk;
  const uint8_t* qb = q8 + (int64_t)bh * S_pad * D;
  const uint8_t* kb = k8 + (int64_t)bh * S_pad * D;
  const uint8_t* vb = v8 + (int64_t)bh * D * S_pad;  // packed: tile t at + t * 128 * D
  const float* ksb = k_scale + (int64_t)bh * nblk;
  const float c2 = c1 * q_scale[(int64_t)bh * nblk + qt];

  const int start = __builtin_amdgcn_readfirstlane(sequential ? 0 : min(qt + window, nblk - 1));
  auto tile_at = [&](int i) -> int { return sequential ? i : (i <= start ? start - i : i); };

  const unsigned loff = (unsigned)l * 16u;
  const FragBase<D> fb(lr, g);
  issue_tile<D>(lds0, kb, vb, tile_at(0), w, loff);

  // Q^T fragments (B operand), kept in registers for the whole kernel; lane
  // group g carries the channels of K chunks g and g + 4 (D = 64: chunk g).
  v8i qf[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int qrow = qt * kBlk + 32 * w + 16 * s + lr;
    const uint8_t* qp = qb + (int64_t)qrow * D;
    const uint4 lo = *(const uint4*)(qp + 16 * g);
    const uint4 hi = D == 128 ? *(const uint4*)(qp + 64 + 16 * g) : make_uint4(0, 0, 0, 0);
    qf[s] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  }

  const v8i ones = {0x38383838, 0x38383838, 0x38383838, 0x38383838,
                    0x38383838, 0x38383838, 0x38383838, 0x38383838};  // E4M3 1.0
  const v4f zero4 = {0.f, 0.f, 0.f, 0.f};
  float M[2] = {-INFINITY, -INFINITY};  // running max of query lr of each sub-tile (log2 units)
  float Lq[2] = {0.f, 0.f};             // running denominator of query lr
  v4f O[2][NM];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int m = 0; m < NM; ++m) O[s][m] = zero4;
  // V-Smooth: row sums of the last tiles of the current 8-tile window, kept
  // for the two window slots 2g, 2g+1 this lane feeds to the mean MFMA.
  float rb[2][2] = {{0.f, 0.f}, {0.f, 0.f}};

  const bool ragged = (S % kBlk) != 0;

  // One key tile; TAIL marks the last, ragged tile, whose keys >= S get
  // score -inf (code 0, no part in the maximum).  Instantiated twice so the
  // common tiles carry no masking selects.
  auto tile_body = [&](int i, uint8_t* cur, uint8_t* nxt, auto tail_tag) {
    constexpr bool TAIL = decltype(tail_tag)::value;
    const int t = tile_at(i);
    wait_vm();
    __syncthreads();
    if (i + 1 < nblk) issue_tile<D>(nxt, kb, vb, tile_at(i + 1), w, loff);
    const uint8_t* Kt = cur;
    const uint8_t* Vt = cur + TileLds<D>::KB;

    // ---- S^T = K Q^T ------------------------------------------------------
    v4f Sc[2][8];
#pragma unroll
    for (int t8 = 0; t8 < 8; ++t8) {
      v8i kf = kfrag<D>(Kt, t8, fb);
      Sc[0][t8] = mfma_fp8(kf, qf[0], zero4);
      Sc[1][t8] = mfma_fp8(kf, qf[1], zero4);
    }
    if constexpr (TAIL) {
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

    // ---- running max, rescale, codes ---------------------------------------
    const float gk = c2 * ksb[t];
    const float a8 = 8.0f * gk;
    v8i P[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      float mx = __builtin_fmaxf(Sc[s][0][0], Sc[s][0][1]);
#pragma unroll
      for (int e = 2; e < 32; e += 2)  // one v_max3_f32 per two scores
        mx = __builtin_fmaxf(__builtin_fmaxf(mx, Sc[s][e >> 2][e & 3]), Sc[s][(e + 1) >> 2][(e + 1) & 3]);
      mx = max_over_groups(mx);
      const float Mn = __builtin_fmaxf(M[s], gk * mx);
      if (__any(Mn > M[s])) {
        const float alpha = exp2f(M[s] - Mn);
        Lq[s] *= alpha;
        if (VS) {
          rb[s][0] *= alpha;
          rb[s][1] *= alpha;
        }
        float a4[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) a4[v] = __shfl(alpha, 4 * g + v);
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
          for (int m = 0; m < NM; ++m) O[s][m][v] *= a4[v];
        M[s] = Mn;
      }
      const float bb = 119.65f - 8.0f * M[s];
#pragma unroll
      for (int t8 = 0; t8 < 8; ++t8) {
        u32 wd = 0;
        wd = VC_EXPCAST_BYTE(wd, a8, Sc[s][t8][0], bb, 0);
        wd = VC_EXPCAST_BYTE(wd, a8, Sc[s][t8][1], bb, 1);
        wd = VC_EXPCAST_BYTE(wd, a8, Sc[s][t8][2], bb, 2);
        wd = VC_EXPCAST_BYTE(wd, a8, Sc[s][t8][3], bb, 3);
        P[s][t8] = (int)wd;
      }
    }

    // ---- A += P V -------------------------------------------------------------
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      v8i vf = vfrag<D>(Vt, m, fb);
      O[0][m] = mfma_fp8(P[0], vf, O[0][m]);
      O[1][m] = mfma_fp8(P[1], vf, O[1][m]);
    }
    // ---- row sums over the same bytes: ones x P^T puts query lr's sum in
    // every register of lane l (the layout of M, alpha and the mean MFMA) ----
    const int slot = i & 7;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const float r = mfma_fp8(ones, P[s], zero4)[0];
      Lq[s] += r;
      if (VS) {
        if (slot == 2 * g) rb[s][0] = r;
        if (slot == 2 * g + 1) rb[s][1] = r;
      }
    }
    // ---- V-Smooth mean restoration, A += sum_t r_t mu_t^T, for 8 tiles at a
    // time on the bf16 matrix cores: K slots (g, 4j + e) carry tile 2g + j of
    // the window with (r_hi, r_lo, r_hi, 0) x (mu_hi, mu_hi, mu_lo, 0) ----
    if (VS && (slot == 7 || i == nblk - 1)) {
      v8bf Ar[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const __bf16 hi = (__bf16)rb[s][j];
          const __bf16 lo = (__bf16)(rb[s][j] - (float)hi);
          Ar[s][4 * j + 0] = hi;
          Ar[s][4 * j + 1] = lo;
          Ar[s][4 * j + 2] = hi;
          Ar[s][4 * j + 3] = (__bf16)0.0f;
          rb[s][j] = 0.f;
        }
      }
      const int i0 = i - slot;  // visit index of window slot 0
      const float* mut[2];
      bool okj[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int iv = i0 + 2 * g + j;
        okj[j] = iv <= i;
        mut[j] = mu + ((int64_t)bh * nblk + tile_at(okj[j] ? iv : i)) * D;
      }
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        v8bf Bm;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const float mv = okj[j] ? mut[j][16 * m + lr] : 0.0f;
          const __bf16 hi = (__bf16)mv;
          const __bf16 lo = (__bf16)(mv - (float)hi);
          Bm[4 * j + 0] = hi;
          Bm[4 * j + 1] = hi;
          Bm[4 * j + 2] = lo;
          Bm[4 * j + 3] = (__bf16)0.0f;
        }
        O[0][m] = mfma_bf16(Ar[0], Bm, O[0][m]);
        O[1][m] = mfma_bf16(Ar[1], Bm, O[1][m]);
      }
    }
  };

  // The ragged last key tile is visited either first (mid-window start
  // clamped to the last block) or last; peel it so the loop body is unmasked.
  const bool tail_first = ragged && tile_at(0) == nblk - 1;
  const bool tail_last = ragged && !tail_first;
  int i0 = 0, i1 = nblk;
  if (tail_first) {
    tile_body(0, lds0, lds1, std::true_type{});
    i0 = 1;
  }
  if (tail_last) i1 = nblk - 1;
  // unrolled by two so each buffer is a fixed LDS object in each half
  int i = i0;
  if (i & 1) {
    if (i < i1) tile_body(i, lds1, lds0, std::false_type{});
    ++i;
  }
  for (; i + 1 < i1; i += 2) {
    tile_body(i, lds0, lds1, std::false_type{});
    tile_body(i + 1, lds1, lds0, std::false_type{});
  }
  if (i < i1) {
    tile_body(i, lds0, lds1, std::false_type{});
    ++i;
  }
  if (tail_last) {
    if ((nblk - 1) & 1)
      tile_body(nblk - 1, lds1, lds0, std::true_type{});
    else
      tile_body(nblk - 1, lds0, lds1, std::true_type{});
  }

  // ---- epilogue: O = (A / l) * s_V, bf16, original query order -----------
  const int b = bh / H, h = bh % H;
  const float* vsb = v_scale + (int64_t)bh * D;
  uint16_t* ob = o + b * oB + h * oH;
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int q = qt * kBlk + 32 * w + 16 * s + 4 * g + v;
      const float lsum = __shfl(Lq[s], 4 * g + v);
      if (q >= S) continue;
      const float inv = 1.0f / lsum;
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const int d = 16 * m + lr;
        ob[(int64_t)q * oS + d] = f32_to_bf16((O[s][m][v] * inv) * vsb[d]);
      }
    }
}

template <int D, bool VS>
hipError_t launch_t(const vc_shape& sh, float c1, int window, int seq, const uint8_t* q8, const float* qs,
                    const uint8_t* k8, const float* ks, const uint8_t* v8, const float* vs, const float* mu,
                    BshdOut o, hipStream_t st) {
  const int nblk = (sh.S + kBlk - 1) / kBlk;
  const int64_t n = (int64_t)nblk * sh.H * sh.B;
  attn_fp8_kernel<D, VS><<<(unsigned)n, 256, 0, st>>>(q8, qs, k8, ks, v8, vs, mu, o.p, o.sB, o.sS, o.sH, sh.S, sh.H,
                                                       nblk, c1, window, seq);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fp8(const vc_shape& sh, float sm_scale, int window, uint32_t flags, const uint8_t* q8,
                           const float* q_scale, const uint8_t* k8, const float* k_scale, const uint8_t* v8,
                           const float* v_scale, const float* mu_scaled, BshdOut o, hipStream_t st) {
  const float c1 = sm_scale * 1.44269504088896340736f;  // fl32(sm_scale * fl32(log2 e))
  const int seq = (flags & VC_ATTN_SEQUENTIAL) ? 1 : 0;
  if (sh.D == 128) {
    if (mu_scaled) return launch_t<128, true>(sh, c1, window, seq, q8, q_scale, k8, k_scale, v8, v_scale, mu_scaled, o, st);
    return launch_t<128, false>(sh, c1, window, seq, q8, q_scale, k8, k_scale, v8, v_scale, nullptr, o, st);
  }
  if (mu_scaled) return launch_t<64, true>(sh, c1, window, seq, q8, q_scale, k8, k_scale, v8, v_scale, mu_scaled, o, st);
  return launch_t<64, false>(sh, c1, window, seq, q8, q_scale, k8, k_scale, v8, v_scale, nullptr, o, st);
}

}  // namespace vc
