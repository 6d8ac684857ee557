// vc_capi.hip -- the extern "C" entry points: argument validation, then
// dispatch to the launchers.  Nothing is enqueued unless every check passes.
#include <hip/hip_runtime.h>
#include <math.h>

#include "vc_launch.hpp"

namespace {

using vc::Bshd;
using vc::BshdOut;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int32_t check_shape(const vc_shape* sh) {
  if (!sh) return VC_ERR_NULL;
  if (sh->B < 1 || sh->H < 1 || sh->S < 1) return VC_ERR_SHAPE;
  if (sh->D != 64 && sh->D != 128) return VC_ERR_SHAPE;
  if (sh->S > (1 << 24)) return VC_ERR_SHAPE;
  // every index of an operand stays below 2^31 blocks / 2^62 bytes
  if ((int64_t)sh->B * sh->H * ((sh->S + 127) / 128) > 0x7fffffff) return VC_ERR_SHAPE;
  return VC_OK;
}

int32_t check_bshd(const vc_bshd* x) {
  if (!x || !x->ptr) return VC_ERR_NULL;
  if (!aligned16(x->ptr)) return VC_ERR_ALIGN;
  if ((x->sB % 8) || (x->sS % 8) || (x->sH % 8)) return VC_ERR_ALIGN;
  if (x->sB < 0 || x->sS < 0 || x->sH < 0) return VC_ERR_SHAPE;
  return VC_OK;
}

int32_t check_out(const vc_bshd_out* x) {
  if (!x || !x->ptr) return VC_ERR_NULL;
  if ((uintptr_t)x->ptr & 1u) return VC_ERR_ALIGN;
  if (x->sB < 0 || x->sS < 0 || x->sH < 0) return VC_ERR_SHAPE;
  return VC_OK;
}

Bshd as_bshd(const vc_bshd* x) { return Bshd{(const uint16_t*)x->ptr, x->sB, x->sS, x->sH}; }

int32_t hip_status(hipError_t e) { return e == hipSuccess ? VC_OK : VC_ERR_HIP; }

}  // namespace

extern "C" {

__attribute__((visibility("default"))) int32_t vc_abi_version(void) { return VC_ABI_VERSION; }

__attribute__((visibility("default"))) const char* vc_status_str(int32_t s) {
  switch (s) {
    case VC_OK: return "VC_OK";
    case VC_ERR_NULL: return "VC_ERR_NULL: a required pointer is NULL";
    case VC_ERR_SHAPE: return "VC_ERR_SHAPE: B, H, S or D out of range";
    case VC_ERR_ALIGN: return "VC_ERR_ALIGN: pointer or stride not 16-byte aligned";
    case VC_ERR_UNSUPPORTED: return "VC_ERR_UNSUPPORTED: parameter outside the supported set";
    case VC_ERR_WORKSPACE: return "VC_ERR_WORKSPACE: workspace too small";
    case VC_ERR_HIP: return "VC_ERR_HIP: a HIP launch failed";
    default: return "unknown vc_status";
  }
}

__attribute__((visibility("default"))) int32_t vc_quantize(const vc_shape* sh, float sm_scale, const vc_bshd* q,
                                                            const vc_bshd* k, const vc_bshd* v, uint8_t* q8,
                                                            float* q_scale, uint8_t* k8, float* k_scale,
                                                            uint8_t* v8, float* v_scale, void* stream) {
  int32_t e = check_shape(sh);
  if (e) return e;
  if (!(sm_scale >= 0.0f) || isinf(sm_scale)) return VC_ERR_UNSUPPORTED;
  const bool dq = q && q->ptr, dk = k && k->ptr, dv = v && v->ptr;
  if (dq) {
    if ((e = check_bshd(q))) return e;
    if (!q8 || !q_scale) return VC_ERR_NULL;
    if (!aligned16(q8)) return VC_ERR_ALIGN;
  }
  if (dk) {
    if ((e = check_bshd(k))) return e;
    if (!k8 || !k_scale) return VC_ERR_NULL;
    if (!aligned16(k8)) return VC_ERR_ALIGN;
  }
  if (dv) {
    if ((e = check_bshd(v))) return e;
    if (!v8 || !v_scale) return VC_ERR_NULL;
    if (!aligned16(v8) || ((uintptr_t)v_scale & 3u)) return VC_ERR_ALIGN;
  }
  hipStream_t st = (hipStream_t)stream;
  const float sm = sm_scale == 0.0f ? 1.0f / sqrtf((float)sh->D) : sm_scale;
  const float G = 8.0f * (sm * 1.44269504088896340736f);  // 8 fl(sm_scale * fl(log2 e)), exact times 8
  if (dq && (e = hip_status(vc::launch_qk_quant(*sh, as_bshd(q), G, q8, q_scale, false, st)))) return e;
  if (dk && (e = hip_status(vc::launch_qk_quant(*sh, as_bshd(k), 1.0f, k8, k_scale, true, st)))) return e;
  if (dv && (e = hip_status(vc::launch_v_quant(*sh, as_bshd(v), v8, v_scale, st)))) return e;
  return VC_OK;
}

__attribute__((visibility("default"))) size_t vc_smooth_group_workspace_size(const vc_shape* sh, int32_t clusters) {
  if (check_shape(sh) || clusters < 1) return 0;
  return vc::group_workspace_bytes(*sh, clusters);
}

__attribute__((visibility("default"))) int32_t vc_smooth_group(
    const vc_shape* sh, const vc_bshd* k, const vc_bshd* v, const vc_group_params* p, float* centroids,
    int32_t* labels, int32_t* perm, uint8_t* k8, float* k_scale, uint8_t* r8, float* r_scale, uint16_t* mu_bf16,
    uint32_t* mu_split, void* workspace, size_t workspace_bytes, void* stream) {
  int32_t e = check_shape(sh);
  if (e) return e;
  if ((e = check_bshd(k)) || (e = check_bshd(v))) return e;
  if (!p) return VC_ERR_NULL;
  if (p->flags & ~(VC_GROUP_WARM_START | VC_GROUP_REUSE_PERM)) return VC_ERR_UNSUPPORTED;
  if ((p->flags & VC_GROUP_WARM_START) && (p->flags & VC_GROUP_REUSE_PERM)) return VC_ERR_UNSUPPORTED;
  const bool reuse = (p->flags & VC_GROUP_REUSE_PERM) != 0;
  if ((!reuse && (!centroids || !labels)) || !perm || !k8 || !k_scale || !r8 || !r_scale || !mu_bf16 ||
      !mu_split || !workspace)
    return VC_ERR_NULL;
  const int kmax = 8192 / sh->D;
  if (p->clusters < 1 || p->clusters > kmax || p->clusters > sh->S) return VC_ERR_UNSUPPORTED;
  if (p->iters < 1 || p->iters > 64) return VC_ERR_UNSUPPORTED;
  if (!aligned16(k8) || !aligned16(r8) || ((uintptr_t)workspace & 255u)) return VC_ERR_ALIGN;
  if (((uintptr_t)centroids | (uintptr_t)labels | (uintptr_t)perm | (uintptr_t)k_scale | (uintptr_t)r_scale |
       (uintptr_t)mu_split) & 3u)
    return VC_ERR_ALIGN;
  if (((uintptr_t)mu_bf16) & 1u) return VC_ERR_ALIGN;
  if (workspace_bytes < vc::group_workspace_bytes(*sh, p->clusters)) return VC_ERR_WORKSPACE;
  return hip_status(vc::launch_smooth_group(*sh, as_bshd(k), as_bshd(v), *p, centroids, labels, perm, k8, k_scale,
                                            r8, r_scale, mu_bf16, mu_split, workspace, (hipStream_t)stream));
}

__attribute__((visibility("default"))) int32_t vc_attn_fwd(const vc_shape* sh, const vc_attn_params* p,
                                                            const uint8_t* q8, const float* q_scale,
                                                            const uint8_t* k8, const float* k_scale,
                                                            const uint8_t* v8, const float* v_scale,
                                                            const uint32_t* mu_split, const vc_bshd_out* o,
                                                            void* stream) {
  int32_t e = check_shape(sh);
  if (e) return e;
  if (!p || !q8 || !q_scale || !k8 || !k_scale || !v8 || !v_scale) return VC_ERR_NULL;
  if ((e = check_out(o))) return e;
  if (!aligned16(q8) || !aligned16(k8) || !aligned16(v8)) return VC_ERR_ALIGN;
  if (((uintptr_t)q_scale | (uintptr_t)k_scale | (uintptr_t)v_scale | (uintptr_t)mu_split) & 3u) return VC_ERR_ALIGN;
  if (p->window < 0 || (p->flags & ~VC_ATTN_SEQUENTIAL)) return VC_ERR_UNSUPPORTED;
  if (!(p->sm_scale >= 0.0f) || isinf(p->sm_scale)) return VC_ERR_UNSUPPORTED;
  BshdOut ob{(uint16_t*)o->ptr, o->sB, o->sS, o->sH};
  return hip_status(vc::launch_attn_fp8(*sh, p->window, p->flags, q8, q_scale, k8, k_scale, v8, v_scale,
                                        mu_split, ob, (hipStream_t)stream));
}

__attribute__((visibility("default"))) int32_t vc_pack_v_bf16(const vc_shape* sh, const vc_bshd* v, uint16_t* vt,
                                                               void* stream) {
  int32_t e = check_shape(sh);
  if (e) return e;
  if ((e = check_bshd(v))) return e;
  if (!vt) return VC_ERR_NULL;
  if (!aligned16(vt)) return VC_ERR_ALIGN;
  return hip_status(vc::launch_pack_v_bf16(*sh, as_bshd(v), vt, (hipStream_t)stream));
}

__attribute__((visibility("default"))) int32_t vc_attn_fwd_bf16(const vc_shape* sh, const vc_attn_params* p,
                                                                 const vc_bshd* q, const vc_bshd* k,
                                                                 const uint16_t* vt, const vc_bshd_out* o,
                                                                 void* stream) {
  int32_t e = check_shape(sh);
  if (e) return e;
  if (!p || !vt) return VC_ERR_NULL;
  if ((e = check_bshd(q)) || (e = check_bshd(k)) || (e = check_out(o))) return e;
  if (!aligned16(vt)) return VC_ERR_ALIGN;
  if (p->window < 0 || (p->flags & ~VC_ATTN_SEQUENTIAL)) return VC_ERR_UNSUPPORTED;
  if (!(p->sm_scale >= 0.0f) || isinf(p->sm_scale)) return VC_ERR_UNSUPPORTED;
  const float sm = p->sm_scale == 0.0f ? 1.0f / sqrtf((float)sh->D) : p->sm_scale;
  BshdOut ob{(uint16_t*)o->ptr, o->sB, o->sS, o->sH};
  return hip_status(vc::launch_attn_bf16(*sh, sm, p->window, p->flags, as_bshd(q), as_bshd(k), vt, ob,
                                         (hipStream_t)stream));
}

__attribute__((visibility("default"))) int32_t vc_expcast_codes(const float* x, const float* a, const float* b,
                                                                 int64_t n, int32_t row_len, uint8_t* codes,
                                                                 void* stream) {
  if (n < 0 || row_len < 1 || (n % row_len) != 0) return VC_ERR_SHAPE;
  if (n > 0 && (!x || !a || !b || !codes)) return VC_ERR_NULL;
  if (((uintptr_t)x | (uintptr_t)a | (uintptr_t)b) & 3u) return VC_ERR_ALIGN;
  return hip_status(vc::launch_expcast_codes(x, a, b, n, row_len, codes, (hipStream_t)stream));
}

}  // extern "C"
