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
//    puts one query and 4 keys in each lane, and the K rows of each MFMA are
//    taken in the order that leaves lane group g holding keys 32g..32g+31 of
//    the tile, which is exactly the A-operand layout of the P.V product, so
//    codes go from the accumulator to the PV operand without any shuffle and
//    V is read key-contiguous;
//  - K and V tiles (16 KB each) stream HBM -> LDS with global_load_lds_dwordx4
//    (no VGPR staging), double-buffered, in an XOR-swizzled layout that makes
//    the 32-byte fragment reads bank-conflict free;
//  - workgroup ids are remapped so each XCD works on a contiguous range of
//    query tiles of one head, whose mid-window sweeps hit the same K/V in that
//    XCD's L2.
#include "vc_common.hpp"
#include "vc_launch.hpp"

namespace vc {

namespace {

// LDS swizzles (16-byte chunk index XOR), see the bank analysis in the design doc.
VC_DEV int kswz(int r) { return ((r & 3) ^ ((r >> 6) & 1)) | (((r >> 5) & 1) << 2); }
VC_DEV int vswz(int d) { return ((d >> 1) & 7) ^ ((d & 1) << 2); }

template <int D>
struct TileLds {
  // K tile: 128 rows (keys) x D bytes; V tile: D rows (channels) x 128 bytes (keys)
  static constexpr int KB = kBlk * D;
  static constexpr int VB = D * kBlk;
  static constexpr int BYTES = KB + VB;
};

template <int D>
VC_DEV int kchunk(int row, int c) {
  return D == 128 ? (c ^ kswz(row)) : (c ^ (kswz(row) & 3));
}

// Issue the asynchronous copies of key tile `t` into LDS buffer `buf`.
template <int D>
VC_DEV void issue_tile(uint8_t* buf, const uint8_t* __restrict__ kb, const uint8_t* __restrict__ vb, int64_t S_pad,
                       int t, int w, int l) {
  constexpr int NI = D * kBlk / 1024 / 4;  // 16-byte-per-lane wave instructions per wave per operand
  const uint8_t* kt = kb + (int64_t)t * kBlk * D;
#pragma unroll
  for (int r = 0; r < NI; ++r) {
    int base = (r * 4 + w) * 1024;
    int p = base + l * 16;
    int row = p / D, pch = (p % D) / 16;
    lds_dma16(kt + row * D + kchunk<D>(row, pch) * 16, buf + base);
  }
  const uint8_t* vt = vb + (int64_t)t * kBlk;
  uint8_t* vbuf = buf + TileLds<D>::KB;
#pragma unroll
  for (int r = 0; r < NI; ++r) {
    int base = (r * 4 + w) * 1024;
    int p = base + l * 16;
    int d = p / kBlk, pch = (p % kBlk) / 16;
    lds_dma16(vt + (int64_t)d * S_pad + ((pch ^ vswz(d)) * 16), vbuf + base);
  }
}

// K fragment (A operand) of MFMA block t8: lane row i = lr holds key
// 32*(i/4) + 4*t8 + i%4, bytes [32g, 32g+32) of its D.
template <int D>
VC_DEV v8i kfrag(const uint8_t* kt, int t8, int lr, int g) {
  int row = 32 * (lr >> 2) + 4 * t8 + (lr & 3);
  if (D == 64 && g >= 2) return v8i{0, 0, 0, 0, 0, 0, 0, 0};
  const uint8_t* rp = kt + row * D;
  uint4 lo = *(const uint4*)(rp + kchunk<D>(row, 2 * g) * 16);
  uint4 hi = *(const uint4*)(rp + kchunk<D>(row, 2 * g + 1) * 16);
  return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// V fragment (B operand) of channel block m: lane column lr is channel
// 16m + lr, bytes = keys [32g, 32g+32).
VC_DEV v8i vfrag(const uint8_t* vt, int m, int lr, int g) {
  int d = 16 * m + lr;
  const uint8_t* rp = vt + d * kBlk;
  uint4 lo = *(const uint4*)(rp + ((2 * g) ^ vswz(d)) * 16);
  uint4 hi = *(const uint4*)(rp + ((2 * g + 1) ^ vswz(d)) * 16);
  return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

template <int D, bool VS>
__global__ __launch_bounds__(256, 2) void attn_fp8_kernel(
    const uint8_t* __restrict__ q8, const float* __restrict__ q_scale, const uint8_t* __restrict__ k8,
    const float* __restrict__ k_scale, const uint8_t* __restrict__ v8, const float* __restrict__ v_scale,
    const float* __restrict__ mu, uint16_t* __restrict__ o, int64_t oB, int64_t oS, int64_t oH, int S, int H,
    int nblk, float c1, int window, int sequential) {
  constexpr int NM = D / 16;  // channel blocks of the output
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2][TileLds<D>::BYTES];

  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int qt = lin % nblk;
  const int bh = lin / nblk;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, lr = l & 15, g = l >> 4;
  const int64_t S_pad = (int64_t)nblk * kBlk;
  const uint8_t* qb = q8 + (int64_t)bh * S_pad * D;
  const uint8_t* kb = k8 + (int64_t)bh * S_pad * D;
  const uint8_t* vb = v8 + (int64_t)bh * D * S_pad;
  const float* ksb = k_scale + (int64_t)bh * nblk;
  const float c2 = c1 * q_scale[(int64_t)bh * nblk + qt];

  const int start = sequential ? 0 : min(qt + window, nblk - 1);
  auto tile_at = [&](int i) -> int { return sequential ? i : (i <= start ? start - i : i); };

  issue_tile<D>(lds[0], kb, vb, S_pad, tile_at(0), w, l);

  // Q^T fragments (B operand), kept in registers for the whole kernel.
  v8i qf[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int qrow = qt * kBlk + 32 * w + 16 * s + lr;
    if (D == 64 && g >= 2) {
      qf[s] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
    } else {
      const uint4* qp = (const uint4*)(qb + (int64_t)qrow * D + 32 * g);
      uint4 lo = qp[0], hi = qp[1];
      qf[s] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
  }

  const v8i ones = {0x38383838, 0x38383838, 0x38383838, 0x38383838,
                    0x38383838, 0x38383838, 0x38383838, 0x38383838};  // E4M3 1.0
  const v4f zero4 = {0.f, 0.f, 0.f, 0.f};
  float M[2] = {-INFINITY, -INFINITY};
  v4f O[2][NM];
  v4f L[2] = {zero4, zero4};
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int m = 0; m < NM; ++m) O[s][m] = zero4;

  const bool ragged = (S % kBlk) != 0;

  for (int i = 0; i < nblk; ++i) {
    const int t = tile_at(i);
    const int buf = i & 1;
    wait_vm();
    __syncthreads();
    if (i + 1 < nblk) issue_tile<D>(lds[buf ^ 1], kb, vb, S_pad, tile_at(i + 1), w, l);
    const uint8_t* Kt = lds[buf];
    const uint8_t* Vt = lds[buf] + TileLds<D>::KB;

    // ---- S^T = K Q^T ------------------------------------------------------
    v4f Sc[2][8];
#pragma unroll
    for (int t8 = 0; t8 < 8; ++t8) {
      v8i kf = kfrag<D>(Kt, t8, lr, g);
      Sc[0][t8] = mfma_fp8(kf, qf[0], zero4);
      Sc[1][t8] = mfma_fp8(kf, qf[1], zero4);
    }
    if (ragged && t == nblk - 1) {
      const int lim = S - t * kBlk;  // valid keys in this tile
#pragma unroll
      for (int t8 = 0; t8 < 8; ++t8)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (32 * g + 4 * t8 + v >= lim) {
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
      float mx = fmaxf(fmaxf(Sc[s][0][0], Sc[s][0][1]), fmaxf(Sc[s][0][2], Sc[s][0][3]));
#pragma unroll
      for (int t8 = 1; t8 < 8; ++t8)
        mx = fmaxf(mx, fmaxf(fmaxf(Sc[s][t8][0], Sc[s][t8][1]), fmaxf(Sc[s][t8][2], Sc[s][t8][3])));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float Mn = fmaxf(M[s], gk * mx);
      if (__any(Mn > M[s])) {
        const float alpha = exp2f(M[s] - Mn);
        float a4[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) a4[v] = __shfl(alpha, 4 * g + v);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          L[s][v] *= a4[v];
#pragma unroll
          for (int m = 0; m < NM; ++m) O[s][m][v] *= a4[v];
        }
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

    // ---- A += P V, row sums (and mean restoration) ------------------------
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      v8i vf = vfrag(Vt, m, lr, g);
      O[0][m] = mfma_fp8(P[0], vf, O[0][m]);
      O[1][m] = mfma_fp8(P[1], vf, O[1][m]);
    }
    if (VS) {
      const float* mut = mu + ((int64_t)bh * nblk + t) * D;
      float muv[NM];
#pragma unroll
      for (int m = 0; m < NM; ++m) muv[m] = mut[16 * m + lr];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        v4f r = mfma_fp8(P[s], ones, zero4);
        L[s] += r;
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
          for (int v = 0; v < 4; ++v) O[s][m][v] = __builtin_fmaf(r[v], muv[m], O[s][m][v]);
      }
    } else {
      L[0] = mfma_fp8(P[0], ones, L[0]);
      L[1] = mfma_fp8(P[1], ones, L[1]);
    }
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
      if (q >= S) continue;
      const float inv = 1.0f / L[s][v];
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
  attn_fp8_kernel<D, VS><<<(unsigned)n, 256, 0, st>>>(q8, qs, k8, ks, v8, vs, mu, o.p, o.sB, o.sS, o.sH, sh.S,
                                                       sh.H, nblk, c1, window, seq);
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
