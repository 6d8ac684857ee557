// vc_capi.hip -- the extern "C" entry points: argument validation, then
// dispatch to the launchers.  Nothing is enqueued unless every check passes.
#include <hip/hip_runtime.h>
#include <math.h>

#include <mutex>

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
  if (x->sS >= ((int64_t)1 << 30)) return VC_ERR_SHAPE;  // token stride below 2^31 bytes
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
    case VC_ERR_SCRATCH:
      return "VC_ERR_SCRATCH: the shape needs more than the library's static scratch (VC_GROUP_SCRATCH_BYTES)";
    default: return "unknown vc_status";
  }
}

// Validates a vc_prep_params (NULL = none) into PrepArgs; with_k: K is
// prepared in this call (the centring workspace is then needed).
static int32_t check_prep(const vc_shape* sh, const vc_prep_params* pp, bool with_k, vc::PrepArgs* out) {
  *out = vc::PrepArgs{0u, nullptr, nullptr, nullptr};
  if (!pp || !pp->flags) return VC_OK;
  if (pp->flags & ~(VC_PREP_ROPE | VC_PREP_HADAMARD | VC_PREP_K_CENTER)) return VC_ERR_UNSUPPORTED;
  if (pp->flags & VC_PREP_ROPE) {
    if (!pp->rope_cos || !pp->rope_sin) return VC_ERR_NULL;
    if (((uintptr_t)pp->rope_cos | (uintptr_t)pp->rope_sin) & 15u) return VC_ERR_ALIGN;
  }
  if (with_k && (pp->flags & VC_PREP_K_CENTER)) {
    if (!pp->workspace) return VC_ERR_NULL;
    if ((uintptr_t)pp->workspace & 7u) return VC_ERR_ALIGN;
    if (pp->workspace_bytes < (size_t)sh->B * sh->H * sh->D * 8) return VC_ERR_WORKSPACE;
  }
  *out = vc::PrepArgs{pp->flags, pp->rope_cos, pp->rope_sin, (const long long*)pp->workspace};
  return VC_OK;
}

__attribute__((visibility("default"))) size_t vc_prep_workspace_size(const vc_shape* sh) {
  if (check_shape(sh)) return 0;
  return (size_t)sh->B * sh->H * sh->D * 8;
}

__attribute__((visibility("default"))) int32_t vc_quantize(const vc_shape* sh, float sm_scale,
                                                            const vc_prep_params* prep, const vc_bshd* q,
                                                            const vc_bshd* k, const vc_bshd* v, uint8_t* q8,
                                                            float* q_scale, uint8_t* k8, float* k_scale,
                                                            uint8_t* v8, float* v_scale, void* stream) {
  int32_t e = check_shape(sh);
  if (e) return e;
  if (!(sm_scale >= 0.0f) || isinf(sm_scale)) return VC_ERR_UNSUPPORTED;
  vc::PrepArgs pa;
  if ((e = check_prep(sh, prep, k && k->ptr, &pa))) return e;
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
  float G = 8.0f * (sm * 1.44269504088896340736f);  // 8 fl(sm_scale * fl(log2 e)), exact times 8
  if (pa.flags & VC_PREP_HADAMARD) G /= (float)sh->D;  // exact: D is a power of two
  vc::PrepArgs pq = pa;
  pq.flags &= ~VC_PREP_K_CENTER;  // Q is not centred
  if (dq && (e = hip_status(vc::launch_qk_quant(*sh, as_bshd(q), G, pq, q8, q_scale, false, st)))) return e;
  if (dk && (pa.flags & VC_PREP_K_CENTER) &&
      (e = hip_status(vc::launch_k_center_sums(*sh, as_bshd(k), pa, (unsigned long long*)prep->workspace, st))))
    return e;
  if (dk && (e = hip_status(vc::launch_qk_quant(*sh, as_bshd(k), 1.0f, pa, k8, k_scale, true, st)))) return e;
  if (dv && (e = hip_status(vc::launch_v_quant(*sh, as_bshd(v), v8, v_scale, st)))) return e;
  return VC_OK;
}

__attribute__((visibility("default"))) size_t vc_smooth_group_workspace_size(const vc_shape* sh, int32_t clusters) {
  if (check_shape(sh) || clusters < 1) return 0;
  return vc::group_workspace_bytes(*sh, clusters);
}

}  // extern "C"

namespace {

// Checks shared by vc_smooth_group and vc_smooth_group_noalloc (everything
// but the workspace).
int32_t check_group(const vc_shape* sh, const vc_bshd* k, const vc_bshd* v, const vc_group_params* p,
                    float* centroids, int32_t* labels, int32_t* perm, uint8_t* k8, float* k_scale, uint8_t* r8,
                    float* r_scale, uint16_t* mu_bf16, uint32_t* mu_split) {
  int32_t e = check_shape(sh);
  if (e) return e;
  if ((e = check_bshd(k)) || (e = check_bshd(v))) return e;
  if (!p) return VC_ERR_NULL;
  if (p->flags & ~(VC_GROUP_WARM_START | VC_GROUP_REUSE_PERM)) return VC_ERR_UNSUPPORTED;
  if ((p->flags & VC_GROUP_WARM_START) && (p->flags & VC_GROUP_REUSE_PERM)) return VC_ERR_UNSUPPORTED;
  const bool reuse = (p->flags & VC_GROUP_REUSE_PERM) != 0;
  if ((!reuse && (!centroids || !labels)) || !perm || !k8 || !k_scale || !r8 || !r_scale || !mu_bf16 || !mu_split)
    return VC_ERR_NULL;
  const int kmax = 8192 / sh->D;
  if (p->clusters < 1 || p->clusters > kmax || p->clusters > sh->S) return VC_ERR_UNSUPPORTED;
  if (p->iters < 1 || p->iters > 64) return VC_ERR_UNSUPPORTED;
  if (!aligned16(k8) || !aligned16(r8)) return VC_ERR_ALIGN;
  if (((uintptr_t)centroids | (uintptr_t)labels | (uintptr_t)perm | (uintptr_t)k_scale | (uintptr_t)r_scale |
       (uintptr_t)mu_split) & 3u)
    return VC_ERR_ALIGN;
  if (((uintptr_t)mu_bf16) & 1u) return VC_ERR_ALIGN;
  return VC_OK;
}

int32_t run_group(const vc_shape* sh, const vc_bshd* k, const vc_bshd* v, const vc_group_params* p,
                  const vc_prep_params* prep, vc::PrepArgs pa, float* centroids, int32_t* labels, int32_t* perm,
                  uint8_t* k8, float* k_scale, uint8_t* r8, float* r_scale, uint16_t* mu_bf16, uint32_t* mu_split,
                  void* workspace, hipStream_t st) {
  int32_t e;
  if ((pa.flags & VC_PREP_K_CENTER) &&
      (e = hip_status(vc::launch_k_center_sums(*sh, as_bshd(k), pa, (unsigned long long*)pa.ksum, st))))
    return e;
  return hip_status(vc::launch_smooth_group(*sh, as_bshd(k), as_bshd(v), *p, centroids, labels, perm, k8, k_scale,
                                            r8, r_scale, mu_bf16, mu_split, workspace, pa, st));
}

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

// The no-allocation variant's scratch: one array per GPU the library runs
// on, held until the process ends.  In host code `scratch` names a host-side
// stand-in, never the device memory: its device address is taken once per
// device with hipGetSymbolAddress and only that pointer reaches kernels.
static __device__ __attribute__((aligned(256))) unsigned char scratch[VC_GROUP_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// Device address of the current device's scratch, looked up on the first
// call on that device.
int32_t scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return VC_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return VC_ERR_HIP;
    g_scratch_dev[dev] = ptr;
  }
  *out = g_scratch_dev[dev];
  return VC_OK;
}

}  // namespace

extern "C" {

__attribute__((visibility("default"))) int32_t vc_smooth_group(
    const vc_shape* sh, const vc_bshd* k, const vc_bshd* v, const vc_group_params* p, const vc_prep_params* prep,
    float* centroids, int32_t* labels, int32_t* perm, uint8_t* k8, float* k_scale, uint8_t* r8, float* r_scale,
    uint16_t* mu_bf16, uint32_t* mu_split, void* workspace, size_t workspace_bytes, void* stream) {
  int32_t e = check_group(sh, k, v, p, centroids, labels, perm, k8, k_scale, r8, r_scale, mu_bf16, mu_split);
  if (e) return e;
  if (!workspace) return VC_ERR_NULL;
  if ((uintptr_t)workspace & 255u) return VC_ERR_ALIGN;
  if (workspace_bytes < vc::group_workspace_bytes(*sh, p->clusters)) return VC_ERR_WORKSPACE;
  vc::PrepArgs pa;
  if ((e = check_prep(sh, prep, true, &pa))) return e;
  return run_group(sh, k, v, p, prep, pa, centroids, labels, perm, k8, k_scale, r8, r_scale, mu_bf16, mu_split,
                   workspace, (hipStream_t)stream);
}

__attribute__((visibility("default"))) size_t vc_smooth_group_noalloc_bytes(const vc_shape* sh, int32_t clusters,
                                                                            uint32_t prep_flags) {
  if (check_shape(sh) || clusters < 1) return 0;
  size_t n = round256(vc::group_workspace_bytes(*sh, clusters));
  if (prep_flags & VC_PREP_K_CENTER) n += round256((size_t)sh->B * sh->H * sh->D * 8);
  return n;
}

__attribute__((visibility("default"))) int32_t vc_smooth_group_noalloc(
    const vc_shape* sh, const vc_bshd* k, const vc_bshd* v, const vc_group_params* p, const vc_prep_params* prep,
    float* centroids, int32_t* labels, int32_t* perm, uint8_t* k8, float* k_scale, uint8_t* r8, float* r_scale,
    uint16_t* mu_bf16, uint32_t* mu_split, void* stream) {
  int32_t e = check_group(sh, k, v, p, centroids, labels, perm, k8, k_scale, r8, r_scale, mu_bf16, mu_split);
  if (e) return e;
  // the centring sums (VC_PREP_K_CENTER) follow the grouping workspace in
  // the scratch; prep->workspace is not used
  vc_prep_params pp{};
  if (prep) {
    pp = *prep;
    pp.workspace = nullptr;
    pp.workspace_bytes = 0;
  }
  const uint32_t pflags = prep ? prep->flags : 0u;
  const size_t gbytes = round256(vc::group_workspace_bytes(*sh, p->clusters));
  if (vc_smooth_group_noalloc_bytes(sh, p->clusters, pflags) > VC_GROUP_SCRATCH_BYTES) return VC_ERR_SCRATCH;
  // validate the preparation first with a stand-in centring buffer: no HIP
  // call happens before every argument is known to be good
  if (pflags & VC_PREP_K_CENTER) {
    pp.workspace = (void*)(uintptr_t)256;
    pp.workspace_bytes = (size_t)sh->B * sh->H * sh->D * 8;
  }
  vc::PrepArgs pa;
  if ((e = check_prep(sh, prep ? &pp : nullptr, true, &pa))) return e;
  void* base = nullptr;
  if ((e = scratch_on_current_device(&base))) return e;
  if (pflags & VC_PREP_K_CENTER) pa.ksum = (const long long*)((unsigned char*)base + gbytes);
  return run_group(sh, k, v, p, prep, pa, centroids, labels, perm, k8, k_scale, r8, r_scale, mu_bf16, mu_split,
                   base, (hipStream_t)stream);
}

__attribute__((visibility("default"))) int32_t vc_attn_fwd(const vc_shape* sh, const vc_attn_params* p,
                                                            const uint8_t* q8, const float* q_scale,
                                                            const uint8_t* k8, const float* k_scale,
                                                            const uint8_t* v8, const float* v_scale,
                                                            const uint32_t* mu_split,
                                                            const vc_repair_rows* repair, const vc_bshd_out* o,
                                                            void* stream) {
  int32_t e = check_shape(sh);
  if (e) return e;
  if (!p || !q8 || !q_scale || !k8 || !k_scale || !v8 || !v_scale) return VC_ERR_NULL;
  if ((e = check_out(o))) return e;
  if (!aligned16(q8) || !aligned16(k8) || !aligned16(v8)) return VC_ERR_ALIGN;
  if (((uintptr_t)q_scale | (uintptr_t)k_scale | (uintptr_t)v_scale | (uintptr_t)mu_split) & 3u) return VC_ERR_ALIGN;
  if (p->window < 0 || (p->flags & ~VC_ATTN_SEQUENTIAL)) return VC_ERR_UNSUPPORTED;
  if (!(p->sm_scale >= 0.0f) || isinf(p->sm_scale)) return VC_ERR_UNSUPPORTED;
  vc::RepairTiles rp{0, nullptr, nullptr, nullptr};
  if (repair && repair->rows != 0) {
    if (repair->rows < 0 || repair->rows > sh->S) return VC_ERR_SHAPE;
    if (mu_split) return VC_ERR_UNSUPPORTED;  // repair rows belong to the plain path
    if (!repair->k8 || !repair->k_scale || !repair->v8) return VC_ERR_NULL;
    if (!aligned16(repair->k8) || !aligned16(repair->v8) || ((uintptr_t)repair->k_scale & 3u)) return VC_ERR_ALIGN;
    rp = vc::RepairTiles{(repair->rows + 127) / 128, repair->k8, repair->k_scale, repair->v8};
  }
  BshdOut ob{(uint16_t*)o->ptr, o->sB, o->sS, o->sH};
  return hip_status(vc::launch_attn_fp8(*sh, p->window, p->flags, q8, q_scale, k8, k_scale, v8, v_scale,
                                        mu_split, rp, ob, (hipStream_t)stream));
}

__attribute__((visibility("default"))) size_t vc_repair_workspace_size(const vc_shape* sh) {
  if (check_shape(sh)) return 0;
  return vc::repair_workspace_bytes(*sh);
}

__attribute__((visibility("default"))) int32_t vc_repair_prepare(const vc_shape* sh, const vc_prep_params* prep,
                                                                  const vc_bshd* k, const vc_bshd* v, int32_t rows,
                                                                  int32_t* idx, uint8_t* rk8, float* rk_scale,
                                                                  uint8_t* rv8, void* workspace,
                                                                  size_t workspace_bytes, void* stream) {
  int32_t e = check_shape(sh);
  if (e) return e;
  if (rows < 0 || rows > sh->S) return VC_ERR_SHAPE;
  if ((e = check_bshd(k)) || (e = check_bshd(v))) return e;
  vc::PrepArgs pa;
  if ((e = check_prep(sh, prep, true, &pa))) return e;
  if (rows == 0) return VC_OK;
  if (!idx || !rk8 || !rk_scale || !rv8 || !workspace) return VC_ERR_NULL;
  if (!aligned16(rk8) || !aligned16(rv8) || ((uintptr_t)workspace & 255u)) return VC_ERR_ALIGN;
  if (((uintptr_t)idx | (uintptr_t)rk_scale) & 3u) return VC_ERR_ALIGN;
  if (workspace_bytes < vc::repair_workspace_bytes(*sh)) return VC_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  if ((pa.flags & VC_PREP_K_CENTER) &&
      (e = hip_status(vc::launch_k_center_sums(*sh, as_bshd(k), pa, (unsigned long long*)prep->workspace, st))))
    return e;
  return hip_status(vc::launch_repair_prepare(*sh, as_bshd(k), as_bshd(v), pa, rows, idx, rk8, rk_scale, rv8,
                                              workspace, st));
}

__attribute__((visibility("default"))) int32_t vc_quantize4(const vc_shape* sh, float sm_scale, const vc_bshd* q,
                                                             const vc_bshd* k, const vc_bshd* v,
                                                             const int32_t* perm, const uint16_t* mu_bf16,
                                                             uint8_t* q4, uint8_t* q4_scale, uint8_t* k4,
                                                             uint8_t* k4_scale, uint8_t* v4, uint8_t* v4_scale,
                                                             void* stream) {
  int32_t e = check_shape(sh);
  if (e) return e;
  if (!(sm_scale >= 0.0f) || isinf(sm_scale)) return VC_ERR_UNSUPPORTED;
  const bool dq = q && q->ptr, dk = k && k->ptr, dv = v && v->ptr;
  if (dk != dv) return VC_ERR_NULL;             // K and V go together
  if ((perm == nullptr) != (mu_bf16 == nullptr)) return VC_ERR_NULL;  // V-Smooth: both
  if (perm && !dk) return VC_ERR_NULL;
  if (dq) {
    if ((e = check_bshd(q))) return e;
    if (!q4 || !q4_scale) return VC_ERR_NULL;
    if (!aligned16(q4)) return VC_ERR_ALIGN;
  }
  if (dk) {
    if ((e = check_bshd(k)) || (e = check_bshd(v))) return e;
    if (!k4 || !k4_scale || !v4 || !v4_scale) return VC_ERR_NULL;
    if (!aligned16(k4) || !aligned16(v4) || (((uintptr_t)k4_scale | (uintptr_t)v4_scale) & 7u)) return VC_ERR_ALIGN;
    if (((uintptr_t)perm & 3u) || ((uintptr_t)mu_bf16 & 15u)) return VC_ERR_ALIGN;
  }
  const float sm = sm_scale == 0.0f ? 1.0f / sqrtf((float)sh->D) : sm_scale;
  const float pre = sm * 1.44269504088896340736f;  // fl(sm_scale * fl(log2 e)): scores in log2 units
  const Bshd none{nullptr, 0, 0, 0};
  return hip_status(vc::launch_quant4(*sh, pre, dq ? as_bshd(q) : none, dk ? as_bshd(k) : none,
                                      dv ? as_bshd(v) : none, perm, mu_bf16, q4, q4_scale, k4, k4_scale, v4,
                                      v4_scale, (hipStream_t)stream));
}

__attribute__((visibility("default"))) int32_t vc_attn_fwd4(const vc_shape* sh, const vc_attn_params* p,
                                                             const uint8_t* q4, const uint8_t* q4_scale,
                                                             const uint8_t* k4, const uint8_t* k4_scale,
                                                             const uint8_t* v4, const uint8_t* v4_scale,
                                                             const uint16_t* mu_bf16, const vc_bshd_out* o,
                                                             void* stream) {
  int32_t e = check_shape(sh);
  if (e) return e;
  if (!p || !q4 || !q4_scale || !k4 || !k4_scale || !v4 || !v4_scale) return VC_ERR_NULL;
  if ((e = check_out(o))) return e;
  if (!aligned16(q4) || !aligned16(k4) || !aligned16(v4)) return VC_ERR_ALIGN;
  if ((((uintptr_t)k4_scale | (uintptr_t)v4_scale) & 7u) || ((uintptr_t)mu_bf16 & 15u)) return VC_ERR_ALIGN;
  if (p->window < 0 || (p->flags & ~VC_ATTN_SEQUENTIAL)) return VC_ERR_UNSUPPORTED;
  if (!(p->sm_scale >= 0.0f) || isinf(p->sm_scale)) return VC_ERR_UNSUPPORTED;
  BshdOut ob{(uint16_t*)o->ptr, o->sB, o->sS, o->sH};
  return hip_status(vc::launch_attn4(*sh, p->window, p->flags, q4, q4_scale, k4, k4_scale, v4, v4_scale, mu_bf16,
                                     ob, (hipStream_t)stream));
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
