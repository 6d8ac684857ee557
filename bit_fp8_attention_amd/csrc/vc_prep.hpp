// vc_prep.hpp -- device helpers of the fused Q/K preprocessing ([VC] §3.4
// "Fused Kernel and Amortized Grouping", Appendix B): rotary embedding, key
// centring statistics and the QK Hadamard rotation, applied ahead of the
// quantisers in vc_quantize.hip and vc_group.hip.
#pragma once
#include "vc_common.hpp"

namespace vc {

// 8 bf16 of a uint4 as fp32
VC_DEV void unpack8(uint4 w, float (&x)[8]) {
  x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x); x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
  x[4] = bf16_lo(w.z); x[5] = bf16_hi(w.z); x[6] = bf16_lo(w.w); x[7] = bf16_hi(w.w);
}

// ---- Q/K preprocessing ([VC] §3.4, App. B), on an 8-channel chunk of a
// row (channels 8 ch .. 8 ch + 7) held by one lane; a row's D / 8 chunks sit
// in D / 8 consecutive lanes (aligned) ----
// RoPE: pairs (2i, 2i+1) -> (a c - b s, a s + b c), cs / sn the row's table
// entries for the chunk's 4 pairs; fp32 products and sums, no contraction.
VC_DEV void rope8(float (&v)[8], const float* cs, const float* sn) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const float a = v[2 * p], b = v[2 * p + 1], c = cs[p], s = sn[p];
    const float ac = a * c, bs = b * s, as = a * s, bc = b * c;
    v[2 * p] = ac - bs;
    v[2 * p + 1] = as + bc;
  }
}
// Unnormalised Walsh-Hadamard transform of the row, radix-2 butterflies
// (a, b) -> (a + b, a - b) over strides 1, 2, ..., D/2 in that order: strides
// 1, 2, 4 inside the chunk, the rest across the lanes of the row (partner =
// lane ^ stride / 8; the lane with the stride bit set holds the b side).
template <int CPR>
VC_DEV void fwht_row8(float (&v)[8], int ch) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1)
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (!(i & h)) {
        const float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
#pragma unroll
  for (int m = 1; m < CPR; m <<= 1) {
    const bool upper = (ch & m) != 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float o = __shfl_xor(v[i], m);
      v[i] = upper ? o - v[i] : v[i] + o;
    }
  }
}
// 64-bit fixed point with 24 fraction bits, round half-even (exact sums in
// any order).
VC_DEV long long fx24_ll(float v) { return __double2ll_rn((double)v * 16777216.0); }
// The channel mean of centring from the head's fixed-point sum over S keys.
VC_DEV float fx24_mean_of(long long sum, int S) { return (float)((double)sum / ((double)S * 16777216.0)); }

}  // namespace vc
