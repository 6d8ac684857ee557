// vc_launch.hpp -- internal launchers (validated arguments only).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/vc_attn.h"

namespace vc {

struct Bshd {
  const uint16_t* p;
  int64_t sB, sS, sH;
};

struct BshdOut {
  uint16_t* p;
  int64_t sB, sS, sH;
};

// vc_quantize.hip
// Q/K preprocessing ahead of the quantiser (VC_PREP_* flags of vc_attn.h)
constexpr uint32_t kPrepRope = 1u, kPrepHadamard = 2u, kPrepCenter = 4u;
struct PrepArgs {
  uint32_t flags;         // 0: none
  const float* cs;        // RoPE tables fp32 [S][D/2] by token position
  const float* sn;
  const long long* ksum;  // K centring: fixed-point channel sums [B][H][D]
};
// pre: fp32 factor applied before quantising (Q: G = 8 fl(sm_scale log2 e), over D with the rotation; K: 1)
hipError_t launch_qk_quant(const vc_shape& sh, Bshd x, float pre, PrepArgs pp, uint8_t* codes, float* scale,
                           bool pack, hipStream_t st);
// K centring statistics into ksum (zeroed here first): sums over all keys after RoPE
hipError_t launch_k_center_sums(const vc_shape& sh, Bshd x, PrepArgs pp, unsigned long long* ksum, hipStream_t st);
hipError_t launch_v_quant(const vc_shape& sh, Bshd v, uint8_t* v8, float* v_scale, hipStream_t st);
// per-(b, h) amax of V into out[(b H + h) stride] (as ordered bits: zeroed, then atomically raised)
hipError_t launch_v_amax(const vc_shape& sh, Bshd v, float* out, int stride, hipStream_t st);
// K rows idx[(b H + h) R + i] (i < R; the last repeated to fill the block), prepared at their own
// positions, quantised as packed power-of-two blocks into ceil(R / 128) tiles per head
hipError_t launch_k_gather_quant(const vc_shape& sh, Bshd k, PrepArgs pp, const int32_t* idx, int R, uint8_t* k8,
                                 float* k_scale, hipStream_t st);
hipError_t launch_pack_v_bf16(const vc_shape& sh, Bshd v, uint16_t* vt, hipStream_t st);
hipError_t launch_expcast_codes(const float* x, const float* a, const float* b, int64_t n, int32_t row_len,
                                uint8_t* codes, hipStream_t st);

// vc_group.hip
size_t group_workspace_bytes(const vc_shape& sh, int clusters);
hipError_t launch_smooth_group(const vc_shape& sh, Bshd k, Bshd v, const vc_group_params& p, float* centroids,
                               int32_t* labels, int32_t* perm, uint8_t* k8, float* k_scale, uint8_t* r8,
                               float* r_scale, uint16_t* mu_bf16, uint32_t* mu_split, void* ws, PrepArgs pp,
                               hipStream_t st);

// vc_repair.hip
size_t repair_workspace_bytes(const vc_shape& sh);
hipError_t launch_repair_prepare(const vc_shape& sh, Bshd k, Bshd v, PrepArgs pp, int R, int32_t* idx, uint8_t* rk8,
                                 float* rk_scale, uint8_t* rv8, void* ws, hipStream_t st);

// vc_attn_fp8.hip
// Repair tiles visited after the regular ones (nrb = 0: none)
struct RepairTiles {
  int nrb;
  const uint8_t* k8;
  const float* k_scale;
  const uint8_t* v8;
};
// q8 / q_scale carry the softmax factor G (vc_quantize); Q/K scales are powers of two
hipError_t launch_attn_fp8(const vc_shape& sh, int window, uint32_t flags, const uint8_t* q8, const float* q_scale,
                           const uint8_t* k8, const float* k_scale, const uint8_t* v8, const float* v_scale,
                           const uint32_t* mu_split, RepairTiles rp, BshdOut o, hipStream_t st);

// vc_attn_mxfp4.hip (the 4-bit path)
// Q rows (times pre) into q4 / q4s; K and V (through perm, minus mu_bf16, when given) into the packed tiles
hipError_t launch_quant4(const vc_shape& sh, float pre, Bshd q, Bshd k, Bshd v, const int32_t* perm,
                         const uint16_t* mu, uint8_t* q4, uint8_t* q4s, uint8_t* k4, uint8_t* k4s, uint8_t* v4,
                         uint8_t* v4s, hipStream_t st);
hipError_t launch_attn4(const vc_shape& sh, int window, uint32_t flags, const uint8_t* q4, const uint8_t* q4s,
                        const uint8_t* k4, const uint8_t* k4s, const uint8_t* v4, const uint8_t* v4s,
                        const uint16_t* mu, BshdOut o, hipStream_t st);

// vc_attn_bf16.hip
hipError_t launch_attn_bf16(const vc_shape& sh, float sm_scale, int window, uint32_t flags, Bshd q, Bshd k,
                            const uint16_t* vt, BshdOut o, hipStream_t st);

}  // namespace vc
