// Device-side building blocks shared by the gfx950 kernels of the QLoRA layer.
//
// NF4 restore ("48GB GPU Fine-Tuning a 65B Model", section "Quantization Keeps
// the Patterns and Reduces Bits per Number"; reconstruction equation of the
// double-quantization paragraph on the first page, section "메모리 회계"):
//     s_hat = fl32(q2 * 2^-8 * S_g)          one rounding (q2 * 2^-8 is exact)
//     w_hat = bf16_rne(fl32(c[q] * s_hat))
// Per block of 64 weights the 16 possible restored values form a table. The
// kernels hold that table as four byte planes in registers and expand packed
// nibbles with v_perm_b32 byte selects (CDNA has no dynamically indexed
// registers), so no per-weight multiply or convert is needed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qlora {

constexpr int kBlock = 64;
constexpr int kGroup = 256;
// Split reductions count arriving workgroups per output tile in a fixed region
// at the start of the workspace (zero before first use, left zero by every
// kernel). A kernel whose tile count exceeds it runs without a split.
constexpr int64_t kMaxCounters = 16384;

// Codebook and decision thresholds, passed to kernels by value (kernel arguments
// live in SGPRs; they are only ever indexed with compile-time constants).
struct Nf4Consts {
  float code[16];
  float thr[15];
  float pad_;
};

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  // byte i of the result = byte sel.i of the 8-byte value {hi:lo} (lo = bytes 0..3)
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// Two float32 -> one dword of two bf16 (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  bf16x2 b = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, b);
}

__device__ __forceinline__ float bf16_lo_to_f32(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi_to_f32(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Restored block scale s_hat = fl32((q2 * 2^-8) * S).
__device__ __forceinline__ float restore_scale(uint32_t q2, float S) {
  float f = (float)q2 * 0.00390625f;  // exact
  return f * S;
}

// Byte planes of a block's 16-entry bf16 table t[j] = bf16(fl32(c[j] * s_hat)):
//   lo[k] = low bytes of t[4k..4k+3], hi[k] = high bytes of t[4k..4k+3].
struct Nf4Planes {
  uint32_t lo[4];
  uint32_t hi[4];
};

__device__ __forceinline__ Nf4Planes make_planes(const Nf4Consts &c, float sh) {
  uint32_t p[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) p[k] = pack_bf16x2(c.code[2 * k] * sh, c.code[2 * k + 1] * sh);
  Nf4Planes t;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    t.lo[k] = perm(p[2 * k + 1], p[2 * k], 0x06040200u);
    t.hi[k] = perm(p[2 * k + 1], p[2 * k], 0x07050301u);
  }
  return t;
}

// Look up four 16-entry byte tables at once: byte i of the result is plane
// entry q_i, where q_i = (sel.i & 7) + 8 * bit2(merge.i).
__device__ __forceinline__ uint32_t lookup4(const uint32_t pl[4], uint32_t sel, uint32_t merge) {
  uint32_t a = perm(pl[1], pl[0], sel);  // entries 0..7
  uint32_t b = perm(pl[3], pl[2], sel);  // entries 8..15
  return perm(b, a, merge);
}

// Expand one dword of packed codes (8 nibbles: element 2i in the low nibble of
// byte i) into 8 restored bf16 weights, returned in the slot order
//   [e0, e2, e4, e6, e1, e3, e5, e7]
// (the partner MFMA operand is permuted to the same order, see x_slots()).
__device__ __forceinline__ u32x4 expand8(const Nf4Planes &t, uint32_t c) {
  const uint32_t se = c & 0x07070707u;
  const uint32_t me = ((c >> 1) & 0x04040404u) | 0x03020100u;
  const uint32_t so = (c >> 4) & 0x07070707u;
  const uint32_t mo = ((c >> 5) & 0x04040404u) | 0x03020100u;
  const uint32_t lo_e = lookup4(t.lo, se, me);
  const uint32_t hi_e = lookup4(t.hi, se, me);
  const uint32_t lo_o = lookup4(t.lo, so, mo);
  const uint32_t hi_o = lookup4(t.hi, so, mo);
  u32x4 r;
  r[0] = perm(hi_e, lo_e, 0x05010400u);  // (e0, e2)
  r[1] = perm(hi_e, lo_e, 0x07030602u);  // (e4, e6)
  r[2] = perm(hi_o, lo_o, 0x05010400u);  // (e1, e3)
  r[3] = perm(hi_o, lo_o, 0x07030602u);  // (e5, e7)
  return r;
}

// Same expansion in natural element order (e0,e1), (e2,e3), ... for writing to memory.
__device__ __forceinline__ u32x4 expand8_natural(const Nf4Planes &t, uint32_t c) {
  u32x4 s = expand8(t, c);
  u32x4 r;
  r[0] = perm(s[2], s[0], 0x05040100u);  // (e0, e1)
  r[1] = perm(s[2], s[0], 0x07060302u);  // (e2, e3)
  r[2] = perm(s[3], s[1], 0x05040100u);  // (e4, e5)
  r[3] = perm(s[3], s[1], 0x07060302u);  // (e6, e7)
  return r;
}

// Permute 8 consecutive bf16 (natural order, 4 dwords) into the slot order of expand8().
__device__ __forceinline__ u32x4 x_slots(u32x4 x) {
  u32x4 r;
  r[0] = perm(x[1], x[0], 0x05040100u);  // (x0, x2)
  r[1] = perm(x[3], x[2], 0x05040100u);  // (x4, x6)
  r[2] = perm(x[1], x[0], 0x07060302u);  // (x1, x3)
  r[3] = perm(x[3], x[2], 0x07060302u);  // (x5, x7)
  return r;
}

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// Global loads of 16 bytes that bypass nothing special; kept as helpers so the
// kernels read as intent.
__device__ __forceinline__ u32x4 ld16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }
__device__ __forceinline__ void st16(void *p, u32x4 v) { *reinterpret_cast<u32x4 *>(p) = v; }

}  // namespace qlora
