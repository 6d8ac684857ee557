// vc_repair.hip -- Open-VC's V residual repair rows ([OVC] "Why V residual
// repair").  With one FP8 scale per head, token j keeps the residual
// r_j = V_j - s_V Vhat_j; the R tokens of largest energy sum_c r_jc^2 get a
// second value row holding that residual, paired with a copy of their key,
// in extra key tiles the attention kernel visits after all others (their
// products go into the numerator only: the denominator already counts these
// keys once).
//
// Four stream-ordered passes per call, all HBM-streaming except the select:
//   1. per-head amax of V (the quantiser's own kernel);
//   2. residual energies: coalesced residual tiles in LDS, then one thread
//      per token sums in fp64 over the channels in order; stored as their
//      IEEE bit patterns (for non-negative doubles the unsigned order of the
//      bits is the numeric order);
//   3. per head, one 1024-thread workgroup: radix select of the R-th largest
//      pattern T, eight 8-bit digits from the top; then one ordered sweep
//      over the tokens keeps every energy > T and the first (lowest-index)
//      ties == T, writing the kept indices in ascending order -- ties go to
//      the lower index, and the result does not depend on thread timing;
//   4. the repair tiles: keys gathered, prepared at their own positions and
//      quantised as power-of-two blocks (vc_quantize.hip, gather mode);
//      residual codes E4M3(r * 448 / amax) -- the head's own V scale, so the
//      attention epilogue's single multiply covers them -- written in the
//      packed V layout.  Rows past R repeat the last key with a zero residual:
//      the tile's max is that of its real rows and the copies add nothing.
#include "vc_common.hpp"
#include "vc_prep.hpp"
#include "vc_vscale.hpp"
#include "vc_launch.hpp"

namespace vc {

namespace {

// Pass 2: energies of one head's tokens, bits into energy [B][H][S].  One
// workgroup per 128-token block: coalesced 16-byte loads (16 lanes per row
// for D = 128), the fp32 residuals staged in LDS, then one thread per token
// sums its row's squares in fp64 in channel order (row pitch D + 1 floats:
// the 64 rows a wave reads at once sit in distinct banks).
template <int D>
__global__ __launch_bounds__(256) void r_energy(const uint16_t* __restrict__ x, int64_t sB, int64_t sS, int64_t sH,
                                                int S, int H, const float* __restrict__ amax,
                                                unsigned long long* __restrict__ energy) {
  constexpr int CPR = D / 8;
  constexpr int NCH = kBlk * CPR / 256;
  constexpr int LD = D + 1;
  __shared__ float rt[kBlk * LD];
  const int j = blockIdx.x, h = blockIdx.y, b = blockIdx.z, t = threadIdx.x;
  const int64_t bh = (int64_t)b * H + h;
  const uint16_t* xb = x + b * sB + h * sH;
  float s, inv;
  scale_pair(amax[bh], s, inv);
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = t + 256 * i, row = c / CPR, ch = c % CPR, tok = j * kBlk + row;
    float xv[8];
    unpack8(tok < S ? *(const uint4*)(xb + (int64_t)tok * sS + ch * 8) : make_uint4(0, 0, 0, 0), xv);
#pragma unroll
    for (int e2 = 0; e2 < 8; ++e2) rt[row * LD + ch * 8 + e2] = v_residual(xv[e2], s, inv);
  }
  __syncthreads();
  const int tok = j * kBlk + t;
  if (t < kBlk && tok < S) {
    double e = 0.0;
#pragma unroll 8
    for (int d = 0; d < D; ++d) {  // channels 0 .. D - 1 in order
      const double r = (double)rt[t * LD + d];
      e += r * r;  // the square is exact in fp64 (24-bit significands)
    }
    energy[bh * S + tok] = (unsigned long long)__double_as_longlong(e);
  }
}

// Pass 3: the R selected indices of one head, ascending, into idx [B][H][R].
constexpr int kSelT = 1024;
__global__ __launch_bounds__(kSelT) void r_select(const unsigned long long* __restrict__ energy, int S, int H, int R,
                                                  int32_t* __restrict__ idx) {
  __shared__ u32 hist[256];
  __shared__ u32 wtot[2][kSelT / 64];
  __shared__ unsigned long long s_pre;
  __shared__ int s_k;
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int64_t bh = (int64_t)blockIdx.y * H + blockIdx.x;
  const unsigned long long* e = energy + bh * S;
  // radix select: after the pass at digit `sh`, pre holds the top digits of
  // T and k how many of the energies matching pre (at those digits) still
  // have to be taken from the top
  unsigned long long pre = 0ull, msk = 0ull;
  int k = R;
  for (int sh = 56; sh >= 0; sh -= 8) {
    if (t < 256) hist[t] = 0u;
    __syncthreads();
    // four loads in flight per thread; lanes of a wave that fall in the
    // same bin add their count with one atomic (the top digits of the
    // energies are mostly shared, and same-address LDS atomics serialise)
    for (int j0 = t; j0 < S; j0 += 4 * kSelT) {
      unsigned long long xs[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) xs[u] = j0 + u * kSelT < S ? e[j0 + u * kSelT] : 0ull;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        bool act = j0 + u * kSelT < S && (xs[u] & msk) == pre;
        const u32 bin = (u32)(xs[u] >> sh) & 255u;
#pragma unroll
        for (int it = 0; it < 2; ++it) {
          const unsigned long long live = __ballot(act);
          if (live == 0ull) break;
          const int lead = __ffsll((long long)live) - 1;
          const u32 b0 = (u32)__shfl((int)bin, lead);
          const unsigned long long same = __ballot(act && bin == b0);
          if (lane == lead) atomicAdd(&hist[b0], (u32)__popcll(same));
          if (bin == b0) act = false;
        }
        if (act) atomicAdd(&hist[bin], 1u);
      }
    }
    __syncthreads();
    if (t == 0) {
      // the digit where the count from the top first reaches k; it exists
      // because at least k candidates match pre
      int above = 0, dsel = 0;
      for (int d = 255; d >= 0; --d) {
        const int c = (int)hist[d];
        if (above + c >= k) {
          dsel = d;
          break;
        }
        above += c;
      }
      s_pre = pre | ((unsigned long long)dsel << sh);
      s_k = k - above;
    }
    __syncthreads();
    pre = s_pre;
    k = s_k;
    msk |= 0xffull << sh;
  }
  // pre = T, the R-th largest; R - k energies exceed it, and the k
  // lowest-index ties are taken
  const unsigned long long lt = (1ull << lane) - 1ull;
  int eq_base = 0, sel_base = 0;
  for (int base = 0; base < S; base += kSelT) {
    const int j = base + t;
    const unsigned long long x = j < S ? e[j] : 0ull;
    const bool gt = j < S && x > pre, eq = j < S && x == pre;
    const unsigned long long beq = __ballot(eq);
    if (lane == 0) wtot[0][wv] = (u32)__popcll(beq);
    __syncthreads();
    int eq_before = 0, eq_all = 0;
    for (int w = 0; w < kSelT / 64; ++w) {
      const int c = (int)wtot[0][w];
      eq_before += w < wv ? c : 0;
      eq_all += c;
    }
    const bool sel = gt || (eq && eq_base + eq_before + __popcll(beq & lt) < k);
    const unsigned long long bs = __ballot(sel);
    if (lane == 0) wtot[1][wv] = (u32)__popcll(bs);
    __syncthreads();
    int s_before = 0, s_all = 0;
    for (int w = 0; w < kSelT / 64; ++w) {
      const int c = (int)wtot[1][w];
      s_before += w < wv ? c : 0;
      s_all += c;
    }
    const int pos = sel_base + s_before + __popcll(bs & lt);
    if (sel && pos < R) idx[bh * R + pos] = j;
    eq_base += eq_all;
    sel_base += s_all;
    __syncthreads();  // wtot is rewritten by the next chunk
  }
}

// Pass 4 (values): repair tile j of one head, residual codes in the packed V
// layout; rows past R are code 0.
template <int D>
__global__ __launch_bounds__(256) void r_pack_v(const uint16_t* __restrict__ x, int64_t sB, int64_t sS, int64_t sH,
                                                int S, int H, int R, int nrb, const float* __restrict__ amax,
                                                const int32_t* __restrict__ idx, uint8_t* __restrict__ rv8) {
  constexpr int CPR = D / 8;
  constexpr int NCH = kBlk * CPR / 256;
  constexpr int LD = D + 4;  // LDS row pitch in bytes
  __shared__ uint8_t tile[kBlk * LD];
  const int j = blockIdx.x, h = blockIdx.y, b = blockIdx.z, t = threadIdx.x;
  const int64_t bh = (int64_t)b * H + h;
  const uint16_t* xb = x + b * sB + h * sH;
  float s, inv;
  scale_pair(amax[bh], s, inv);
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = t + 256 * i, row = c / CPR, ch = c % CPR, ri = j * kBlk + row;
    u32 w0 = 0u, w1 = 0u;
    if (ri < R) {
      int tok = idx[bh * R + ri];
      tok = tok < 0 ? 0 : (tok < S ? tok : S - 1);  // in bounds whatever the list holds
      float xv[8];
      unpack8(*(const uint4*)(xb + (int64_t)tok * sS + ch * 8), xv);
      float r[8];
#pragma unroll
      for (int e2 = 0; e2 < 8; ++e2) r[e2] = v_residual(xv[e2], s, inv) * inv;
      w0 = cvt4_fp8(r[0], r[1], r[2], r[3]);
      w1 = cvt4_fp8(r[4], r[5], r[6], r[7]);
    }
    *(u32*)(tile + row * LD + ch * 8) = w0;
    *(u32*)(tile + row * LD + ch * 8 + 4) = w1;
  }
  __syncthreads();
  uint8_t* ob = rv8 + (bh * nrb + j) * (int64_t)D * kBlk;
  constexpr int TASKS = D * (kBlk / 16);
#pragma unroll
  for (int i = 0; i < TASKS / 256; ++i) {
    const int task = t + 256 * i, d = task / (kBlk / 16), c = task % (kBlk / 16), k0 = c * 16;
    u32 w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      w[q] = (u32)tile[vkey_of_pos(k0 + 4 * q) * LD + d] | ((u32)tile[vkey_of_pos(k0 + 4 * q + 1) * LD + d] << 8) |
             ((u32)tile[vkey_of_pos(k0 + 4 * q + 2) * LD + d] << 16) |
             ((u32)tile[vkey_of_pos(k0 + 4 * q + 3) * LD + d] << 24);
    *(uint4*)(ob + vpack_off(d, c)) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

}  // namespace

size_t repair_workspace_bytes(const vc_shape& sh) {
  const size_t BH = (size_t)sh.B * sh.H;
  return (BH * 4 + 255) / 256 * 256 + BH * (size_t)sh.S * 8;
}

hipError_t launch_repair_prepare(const vc_shape& sh, Bshd k, Bshd v, PrepArgs pp, int R, int32_t* idx, uint8_t* rk8,
                                 float* rk_scale, uint8_t* rv8, void* ws, hipStream_t st) {
  if (R <= 0) return hipSuccess;
  const int64_t BH = (int64_t)sh.B * sh.H;
  float* amax = (float*)ws;
  unsigned long long* energy = (unsigned long long*)((char*)ws + ((size_t)BH * 4 + 255) / 256 * 256);
  const int nrb = (R + kBlk - 1) / kBlk;
  hipError_t e = launch_v_amax(sh, v, amax, 1, st);
  if (e != hipSuccess) return e;
  dim3 ge((sh.S + kBlk - 1) / kBlk, sh.H, sh.B), gs(sh.H, sh.B), gp(nrb, sh.H, sh.B);
  if (sh.D == 128)
    r_energy<128><<<ge, 256, 0, st>>>(v.p, v.sB, v.sS, v.sH, sh.S, sh.H, amax, energy);
  else
    r_energy<64><<<ge, 256, 0, st>>>(v.p, v.sB, v.sS, v.sH, sh.S, sh.H, amax, energy);
  r_select<<<gs, kSelT, 0, st>>>(energy, sh.S, sh.H, R, idx);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = launch_k_gather_quant(sh, k, pp, idx, R, rk8, rk_scale, st)) != hipSuccess) return e;
  if (sh.D == 128)
    r_pack_v<128><<<gp, 256, 0, st>>>(v.p, v.sB, v.sS, v.sH, sh.S, sh.H, R, nrb, amax, idx, rv8);
  else
    r_pack_v<64><<<gp, 256, 0, st>>>(v.p, v.sB, v.sS, v.sH, sh.S, sh.H, R, nrb, amax, idx, rv8);
  return hipGetLastError();
}

}  // namespace vc
