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
// Where a weight keeps its block scales. Double quantization (the default): an
// 8-bit code q2 per block and a float32 S per group of 256 blocks, the scale of
// block k being restore_scale(q2[k], S[k >> 8]). Absmax-only storage (4.5 bits
// per weight, the variant without double quantization on the first page,
// section "메모리 회계"): the float32 block absmax s_k itself, read as
// S[k >> 0] with the code taken as 256, for which restore_scale gives
// fl32(1 * s_k) = s_k exactly. Kernels receive the shift (kDqShift or 0); with
// shift 0 their q2 buffer range is empty, so its loads return 0, and
// q2_or(0) = 256 is OR-ed into the code where it is used.
constexpr int kDqShift = 8;  // log2(kGroup)
__host__ __device__ inline uint32_t q2_or(int sshift) { return sshift ? 0u : 256u; }
__host__ __device__ inline int64_t scale_words(int64_t nblocks, int sshift) {
  return (nblocks + ((int64_t)1 << sshift) - 1) >> sshift;
}
// Split reductions count arriving workgroups per output tile in a fixed region
// at the start of the workspace (zero before first use, left zero by every
// kernel). Each tile's counter has a 128-byte line of its own: the workgroups
// of all tiles arrive and poll at about the same time, and counters that share
// a line serialize at one memory channel (measured: a third of a K-split
// gradient kernel's time). A kernel whose tile count exceeds kMaxTileCounters
// runs without a split. The last kSyncWords words of the region are reserved:
// the last of them counts the waits that ran out of time and took their
// fallback (the result is the same either way; see split_arrive and the skinny
// forward's exchange), the one before it overrides the wait limit (wait_limit).
constexpr int64_t kMaxCounters = 16384;
constexpr int64_t kSyncWords = 4;
constexpr int64_t kCounterStride = 32;  // 32-bit words per tile counter
constexpr int64_t kMaxTileCounters = (kMaxCounters - kSyncWords) / kCounterStride;
__host__ __device__ inline uint32_t *tile_counter(uint32_t *counters, int64_t tile) {
  return counters + tile * kCounterStride;
}

// The 16 NF4 levels as float32 bit patterns, ascending. Kernels that build
// restore tables take them as literal operands (no registers held across the
// loop). The host derives the same table from normal quantiles and checks it
// against this one, bit for bit, before it launches anything.
constexpr uint32_t kNf4CodeBits[16] = {
    0xbf800000u, 0xbf3239b1u, 0xbf066b2eu, 0xbeca329eu, 0xbe91a24bu, 0xbe3d353du, 0xbdba7869u, 0x00000000u,
    0x3da2fb01u, 0x3e24cadfu, 0x3e7c04dau, 0x3ead0336u, 0x3ee1a4b5u, 0x3f1007a9u, 0x3f3913b0u, 0x3f800000u};

// Codebook and decision thresholds, passed by value to the kernels that index
// them (kernel arguments live in SGPRs; only compile-time indices are used).
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

__device__ __forceinline__ float code_times(int j, float sh) {
  // fl32(c[j] * sh); c[0] = -1, c[7] = 0 and c[15] = 1 need no multiply
  if (j == 0) return -sh;
  if (j == 7) return 0.f;
  if (j == 15) return sh;
  return __uint_as_float(kNf4CodeBits[j]) * sh;
}

__device__ __forceinline__ Nf4Planes make_planes(float sh) {
  uint32_t p[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) p[k] = pack_bf16x2(code_times(2 * k, sh), code_times(2 * k + 1, sh));
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

// Expand one 32-bit word of packed codes into 8 restored bf16 weights in
// element order. Packing: the word covers 8 consecutive weights e0..e7 and byte
// i (i = 0..3) holds e_i in its low nibble and e_(i+4) in its high nibble, so
// the low nibbles select e0..e3 and the high nibbles e4..e7 with the same byte
// lanes, and one byte interleave of the low/high planes yields bf16 pairs.
// Cost: 7 selector ops + 12 table perms + 4 interleave perms per 8 weights.
__device__ __forceinline__ u32x4 expand8(const Nf4Planes &t, uint32_t c) {
  const uint32_t sa = c & 0x07070707u;
  const uint32_t ma = ((c >> 1) & 0x04040404u) | 0x03020100u;
  const uint32_t sb = (c >> 4) & 0x07070707u;
  const uint32_t mb = ((c >> 5) & 0x04040404u) | 0x03020100u;
  const uint32_t lo_a = lookup4(t.lo, sa, ma);  // low bytes of e0..e3
  const uint32_t hi_a = lookup4(t.hi, sa, ma);
  const uint32_t lo_b = lookup4(t.lo, sb, mb);  // low bytes of e4..e7
  const uint32_t hi_b = lookup4(t.hi, sb, mb);
  u32x4 r;
  r[0] = perm(hi_a, lo_a, 0x05010400u);  // (e0, e1)
  r[1] = perm(hi_a, lo_a, 0x07030602u);  // (e2, e3)
  r[2] = perm(hi_b, lo_b, 0x05010400u);  // (e4, e5)
  r[3] = perm(hi_b, lo_b, 0x07030602u);  // (e6, e7)
  return r;
}

// Bit offset of element e (0..7) inside its packed 32-bit word.
__device__ __forceinline__ int nibble_shift(int e) { return 8 * (e & 3) + 4 * (e >> 2); }

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

__device__ __forceinline__ u32x4 ld16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }
__device__ __forceinline__ void st16(void *p, u32x4 v) { *reinterpret_cast<u32x4 *>(p) = v; }

// ---------------------------------------------------------------------------
// Raw buffer loads. A buffer resource covers one tile-sized range; a lane whose
// byte offset is at or past the range reads zeros, so tails need no branches and
// every load of a loop body can be issued before the first use. Ranges are kept
// below 2^31 bytes (the callers rebase per tile), so kOOB is always outside.
// ---------------------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOOB = 0x80000000u;

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, int64_t bytes) {
  if (bytes < 0) bytes = 0;
  const int n = bytes >= 0x7fffffffll ? 0x7fffffff : (int)bytes;
  // word 3 = 0x00020000: 32-bit data format, the raw-buffer setting for gfx9 parts
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, n, 0x00020000);
}
__device__ __forceinline__ u32x4 bld16(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
// Device-coherent variant (sc1): reads data another workgroup published this launch.
__device__ __forceinline__ u32x4 bld16_dev(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 16);
}
__device__ __forceinline__ uint32_t bld32(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t bld32_dev(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 16);
}
__device__ __forceinline__ uint32_t bld8(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0);
}
// Loads at a per-lane offset plus a wave-uniform one (an SGPR operand), for
// addresses known to lie inside the range.
__device__ __forceinline__ u32x4 bld16s(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}
__device__ __forceinline__ uint32_t bld8s(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, voff, soff, 0);
}

// ---------------------------------------------------------------------------
// Cross-workgroup exchange inside one launch, without cache-wide fences: the
// producer writes with device-scope (sc1, write-through) stores, waits for them
// to complete, then bumps a device-scope counter; the consumer that sees the
// final count reads back with device-scope loads.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void st_dev(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float *p) {
  return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev_u32(uint32_t *p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_dev_u32(const uint32_t *p) {
  return __hip_atomic_load(const_cast<uint32_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add_dev_u32(uint32_t *p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t xchg_dev_u32(uint32_t *p, uint32_t v) {
  return __hip_atomic_exchange(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// How long a workgroup waits for others of its launch before it takes a path
// that needs no one else: 20000 ticks of the constant 100 MHz counter that
// wall_clock64() reads, about 200 us. Within one launch on an idle chip every
// wait ends in a few microseconds; the limit matters only when launches on
// other streams hold the compute units that the awaited workgroups need.
constexpr long long kWaitTicks = 20000;
// The limit in force for the launches on a workspace: the counter-region word
// just before the fallback count (`fallbacks - 1`) replaces kWaitTicks when it
// is nonzero. A testing aid: a limit of 1 tick sends every wait that does not
// succeed at once down its fallback path, whose results must equal the others.
__device__ __forceinline__ long long wait_limit(const uint32_t *fallbacks) {
  const uint32_t v = __hip_atomic_load(const_cast<uint32_t *>(fallbacks - 1), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  return v ? (long long)v : kWaitTicks;
}

// ---------------------------------------------------------------------------
// Combine of a tile whose reduction range is split over `parts` workgroups,
// with no wait that progress depends on. Every part stores its float32 partial
// (device scope, complete before it arrives) and the tile's sum is cut into
// `parts` shares, each summed over all partials in part order (so the result
// does not depend on who sums it). The tile's counter line holds:
//   word 0        arrivals (low 16 bits) and departures (high 16 bits)
//   word 1 + s    claim of share s (0 free, 1 taken)
// A part that arrives last knows every partial is stored; an earlier part
// polls for the last arrival until the wait limit passes. Whoever has seen all
// arrivals claims its own share (one atomic exchange) and sums it if the claim
// wins; the last arriver afterwards claims every share still free and sums
// those too. So every share is summed exactly once, by its own part when all
// parts run together, and by the last arriver for the parts that gave up
// waiting (a wait then costs time, never a wrong or missing result). The last
// part to depart clears the line for the next launch on the workspace.
// ---------------------------------------------------------------------------
constexpr uint32_t kDepart = 0x10000u;

// Thread-0 side of the arrival: returns the claimed-share mask of this part
// (own share only; the last arriver's sweep comes later) and whether it
// arrived last. `fallbacks` counts waits that ran out of time.
__device__ __forceinline__ uint32_t split_arrive(uint32_t *line, int part, int parts, bool &last,
                                                 uint32_t *fallbacks) {
  const uint32_t prev = add_dev_u32(line, 1u);
  last = (prev & 0xffffu) == (uint32_t)(parts - 1);
  bool ready = last;
  if (!last) {
    const long long t0 = wall_clock64(), limit = wait_limit(fallbacks);
    for (;;) {
      if ((ld_dev_u32(line) & 0xffffu) >= (uint32_t)parts) {
        ready = true;
        break;
      }
      if (wall_clock64() - t0 > limit) {
        add_dev_u32(fallbacks, 1u);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
  return ready && xchg_dev_u32(line + 1 + part, 1u) == 0u ? 1u << part : 0u;
}
// The last arriver's sweep, run by one whole wave (lane p claims share p, all
// in one round trip): the mask of the shares it won.
__device__ __forceinline__ uint32_t split_sweep(uint32_t *line, int part, int parts, int lane) {
  bool won = false;
  if (lane < parts && lane != part) won = xchg_dev_u32(line + 1 + lane, 1u) == 0u;
  return (uint32_t)__ballot(won);
}
// Thread 0, after every claim of this part is settled: count the departure;
// the last one out clears the line.
__device__ __forceinline__ void split_depart(uint32_t *line, int parts) {
  if ((add_dev_u32(line, kDepart) >> 16) == (uint32_t)(parts - 1)) {
    for (int p = 0; p < parts; ++p) st_dev_u32(line + 1 + p, 0u);
    st_dev_u32(line, 0u);
  }
}
// A 32-bit name of the running launch: the dispatch id (the queue's packet
// counter, which advances for every launch, graph replays included) mixed with
// the queue address; never zero. Read from registers set up at wave launch.
extern "C" __device__ uint64_t qlora_llvm_dispatch_id() __asm("llvm.amdgcn.dispatch.id");
__device__ __forceinline__ uint32_t launch_tag() {
  const uint64_t d = qlora_llvm_dispatch_id();
  const uint64_t q = (uint64_t)(uintptr_t)__builtin_amdgcn_queue_ptr();
  const uint32_t t = (uint32_t)d ^ (uint32_t)(q >> 8) ^ (uint32_t)(q >> 40);
  return t ? t : 1u;
}

// 64-bit device-scope store / load: naturally aligned, so a reader sees either
// the old or the new 8 bytes, never a mix (a value and its tag travel together).
__device__ __forceinline__ void st_dev_u64(uint64_t *p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_dev_u64(const uint64_t *p) {
  return __hip_atomic_load(const_cast<uint64_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Workgroup barrier that orders LDS accesses only. A plain __syncthreads() also
// waits for every outstanding global load and store of each wave, which would
// drain prefetches and device-scope publishes at every barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// s_waitcnt vmcnt(0): every load and store this wave issued has completed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

}  // namespace qlora
