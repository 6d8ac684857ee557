// vc_common.hpp -- device helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "../../include/vc_attn.h"

#define VC_DEV __device__ __forceinline__

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef unsigned int u32;
typedef u32 v4u __attribute__((ext_vector_type(4)));

#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

namespace vc {

constexpr int kBlk = 128;  // key/query block: the FP8 scale granularity and the tile height

VC_DEV float bf16_lo(u32 w) { return __uint_as_float(w << 16); }
VC_DEV float bf16_hi(u32 w) { return __uint_as_float(w & 0xffff0000u); }
VC_DEV float bf16_to_f32(uint16_t h) { return __uint_as_float((u32)h << 16); }

// Round-to-nearest-even fp32 -> bf16 bits (finite inputs).
VC_DEV uint16_t f32_to_bf16(float f) {
  u32 u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Two fp32 -> two OCP E4M3 bytes (round-half-even) in the low 16 bits.
VC_DEV u32 cvt2_fp8(float a, float b) { return (u32)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false); }

// Four fp32 -> one dword of E4M3 bytes, byte i = x_i.
VC_DEV u32 cvt4_fp8(float x0, float x1, float x2, float x3) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, w, true);
  return (u32)w;
}

// One ExpCast code into byte `sel` of `word`: round-half-even of fma(a, x, b),
// clamped below at 0 by the integer conversion (v_cvt_pk_u8_f32).
#define VC_EXPCAST_BYTE(word, a, x, b, sel) __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf((a), (x), (b)), (sel), (word))

// Q/K block scale: the smallest power of two 2^e (e >= -127) with
// amax <= 448 * 2^e, 2^0 for a block of zeros -- a scale the block-scaled
// matrix-core product applies exactly, as its E8M0 operand e + 127.
VC_DEV int pow2_block_exp(float amax) {
  if (!(amax > 0.0f)) return 0;
  int e = __builtin_amdgcn_frexp_expf(amax) - 10;  // amax in [2^(e+9), 2^(e+10)): one step low
  if (e < -127) e = -127;
  while (amax > ldexpf(448.0f, e)) ++e;
  return e;
}
// The E8M0 byte of a power-of-two scale 2^e, e in [-127, 127]: the fp32
// exponent field (2^-127, the one subnormal, has field 0 = E8M0 2^-127).
VC_DEV int e8m0_of_pow2(float s) { return (__float_as_int(s) >> 23) & 0xff; }

// Packed FP8 operand layouts (see vc_attn.h): each 128-key tile of K and of
// V is one contiguous block, and inside it every 16-byte chunk sits at
// chunk index (logical ^ swizzle(row)).  The attention kernel's fragment
// reads have 16 lanes read 16 consecutive rows, lane group g taking logical
// chunks g and g + 4 -- a pattern measured free of LDS bank conflicts on
// gfx950 with this swizzle -- while the HBM -> LDS copy stays a straight
// 16 KB block copy.  Inside a V tile the keys are stored in the order the
// P.V operand wants: byte position p = 64 a + 16 g + 4 t + v of a channel
// row holds key 64 a + 16 t + 4 g + v, the key the S^T = K Q^T accumulator
// of MFMA block 4 a + t, register v, puts in lane group g.
VC_DEV int rswz(int r) { return ((r >> 1) & 7) ^ ((r & 1) << 2); }
VC_DEV int kswz(int r) { return rswz(r); }
VC_DEV int vswz(int d) { return rswz(d); }
VC_DEV int vkey_of_pos(int p) { return (p & 64) + 16 * ((p >> 2) & 3) + 4 * ((p >> 4) & 3) + (p & 3); }
template <int D>
VC_DEV int kchunk(int row, int c) {
  return D == 128 ? (c ^ kswz(row)) : (c ^ (kswz(row) & 3));
}
// byte offset of logical (row, 16-byte chunk c) inside a packed K tile
template <int D>
VC_DEV int kpack_off(int row, int c) { return row * D + kchunk<D>(row, c) * 16; }
// byte offset of logical (channel d, position chunk c) inside a packed V tile
VC_DEV int vpack_off(int d, int c) { return d * kBlk + ((c ^ vswz(d)) * 16); }

// Max over the 4 lanes l, l^16, l^32, l^48 (the 4 lane groups holding one
// query's keys) with gfx950's row-swap permutes: permlane16_swap exchanges
// 16-lane rows 1<->0 and 3<->2, permlane32_swap the two 32-lane halves; with
// both operands x, the max of the two results is the max over the pair.
VC_DEV float max_over_groups(float x) {
  int xi = __float_as_int(x);
  auto p16 = __builtin_amdgcn_permlane16_swap(xi, xi, false, false);
  x = __builtin_fmaxf(__int_as_float(p16[0]), __int_as_float(p16[1]));
  xi = __float_as_int(x);
  auto p32 = __builtin_amdgcn_permlane32_swap(xi, xi, false, false);
  return __builtin_fmaxf(__int_as_float(p32[0]), __int_as_float(p32[1]));
}

VC_DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// FP8 16x16x128 matrix-core product with fp32 accumulate (unscaled form).
VC_DEV v4f mfma_fp8(v8i a, v8i b, v4f c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

VC_DEV v4f mfma_bf16(v8bf a, v8bf b, v4f c) { return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0); }

// The same FP8 product with E8M0 block scales 2^(sa - 127) on A and
// 2^(sb - 127) on B (one scale for the whole operand here: every lane passes
// the same byte), fp32 accumulate onto c.
VC_DEV v4f mfma_fp8_scaled(v8i a, v8i b, v4f c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

// Asynchronous 16-byte global -> LDS copy: lane i lands at lds_base + 16 i.
VC_DEV void lds_dma16(const void* g, void* lds_base) {
  __builtin_amdgcn_global_load_lds(g, LDS_PTR(lds_base), 16, 0, 0);
}

// s_waitcnt with vmcnt = 0 and the other counters at their maxima.
VC_DEV void wait_vm() { __builtin_amdgcn_s_waitcnt(0x0f70); }

// The same 16-byte global -> LDS copy as lds_dma16 (lane i lands at
// lds_base + 16 i), issued as inline asm.  The hardware counts these copies
// on vmcnt only (an outstanding copy does not hold lgkmcnt, measured), but
// the compiler's wait insertion, seeing one, stops trusting partial lgkmcnt
// counts and drains every LDS read before its first use.  Hidden from it,
// the fragment reads get exact partial waits; the kernel orders the copies
// itself with explicit vmcnt waits and barriers.
VC_DEV void lds_dma16_at(const void* g, unsigned lds_addr) {
  const unsigned lds = __builtin_amdgcn_readfirstlane(lds_addr);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds) : "memory", "m0");
}

// The LDS address of a pointer into a __shared__ array.  The cast from a
// generic pointer tests it for null (a scalar compare and select each
// time), so a kernel that copies in a loop takes its arrays' addresses once
// and adds offsets in integer arithmetic.
VC_DEV unsigned lds_addr_of(const void* p) { return (unsigned)(uintptr_t)LDS_PTR(p); }

VC_DEV void lds_dma16_raw(const void* g, void* lds_base) { lds_dma16_at(g, lds_addr_of(lds_base)); }

// NB consecutive 1 KB copies under one M0: lane i of copy r reads
// g + 1024 r and lands at lds_base + 1024 r + 16 i.  The instruction's
// immediate offset moves the global and the LDS address alike, so the
// copies need one M0 write between them (a wave's copies issue about a
// quarter faster than with an M0 write before each, measured).
template <int NB>
VC_DEV void lds_dma16_kb_at(const void* g, unsigned lds_addr) {
  static_assert(NB == 2 || NB == 4, "2 or 4 KB per call");
  const unsigned lds = __builtin_amdgcn_readfirstlane(lds_addr);
  if constexpr (NB == 4)
    asm volatile(
        "s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off\n\tglobal_load_lds_dwordx4 %0, off offset:1024\n\t"
        "global_load_lds_dwordx4 %0, off offset:2048\n\tglobal_load_lds_dwordx4 %0, off offset:3072" ::"v"(g),
        "s"(lds)
        : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off\n\tglobal_load_lds_dwordx4 %0, off offset:1024" ::"v"(
                     g),
                 "s"(lds)
                 : "memory", "m0");
}

template <int NB>
VC_DEV void lds_dma16_kb(const void* g, void* lds_base) {
  lds_dma16_kb_at<NB>(g, lds_addr_of(lds_base));
}

// Compile-time loop: f(std::integral_constant<int, I>) for I in [B, E).
template <int B, int E, class F>
VC_DEV void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Barrier between phases: waits for this wave's own LDS reads and scalar
// loads only.  The copies in flight are waited for by the waves that issued
// them (a fence here would wait for every outstanding copy).  The barrier
// is inline asm with a memory clobber so the compiler moves no memory access
// across it, and the scheduling barriers pin every other instruction.
VC_DEV void phase_sync() {
  __builtin_amdgcn_sched_barrier(0);  // no instruction moves across a phase boundary
  // lgkmcnt(0), vmcnt and expcnt at their maxima; as a builtin, so the
  // compiler's own wait insertion knows every LDS and scalar load is done
  __builtin_amdgcn_s_waitcnt(0xc07f);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// s_waitcnt with vmcnt = N, other counters at their maxima (gfx9 encoding:
// vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
VC_DEV void wait_vm_n() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0f70);
}

// Blocks of 8 XCDs: workgroup ids are dealt round-robin to the XCDs, so
// remap them so that each XCD runs one contiguous range of logical tiles
// (neighbouring query tiles of one head share K/V in that XCD's L2).
VC_DEV int xcd_remap(int id, int n) {
  const int X = 8;
  int q = n / X, r = n % X;
  int xcd = id % X, slot = id / X;
  // XCD x owns logical ids [x*q + min(x, r), ...) of length q + (x < r)
  int start = xcd * q + (xcd < r ? xcd : r);
  return start + slot;
}

}  // namespace vc

#define VC_CHECK_LAUNCH()                     \
  do {                                        \
    if (hipGetLastError() != hipSuccess) return VC_ERR_HIP; \
  } while (0)
