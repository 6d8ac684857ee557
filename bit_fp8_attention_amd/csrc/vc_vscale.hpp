// vc_vscale.hpp -- the per-head V scale and its FP8 residual, shared by the V
// quantiser (vc_quantize.hip) and the repair rows (vc_repair.hip).
#pragma once
#include "vc_common.hpp"

namespace vc {

// One scale per head ([OVC] "Scheduling around ExpCast"): s = amax / 448 and
// the encode factor inv = 448 / amax, both rounded once in fp32; a head of
// zeros takes s = inv = 1.
VC_DEV void scale_pair(float amax, float& s, float& inv) {
  if (amax > 0.0f) {
    s = amax / 448.0f;
    inv = 448.0f / amax;
  } else {
    s = 1.0f;
    inv = 1.0f;
  }
}

// What a value keeps after the head's FP8 round trip ([OVC] "Why V residual
// repair"): r = v - s * dec(E4M3(v * inv)), each operation rounded once in
// fp32 (the build does not contract).
VC_DEV float v_residual(float v, float s, float inv) {
  const int c = __builtin_amdgcn_cvt_pk_fp8_f32(v * inv, 0.0f, 0, false);
  return v - s * __builtin_amdgcn_cvt_f32_fp8(c, 0);
}

}  // namespace vc
