// LDS tile helpers shared by the MFMA kernels (large-T contractions and the
// adapter products): typedefs for LDS pointers, scheduling pins, a barrier that
// leaves copies into LDS in flight, copies into LDS issued from asm, and the
// bank swizzle of 512-byte-row tiles read with ds_read_b64_tr_b16.
#pragma once

#include "common.h"

namespace qlora {

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

#define QLORA_SCHED_FENCE() __builtin_amdgcn_sched_barrier(0)

// Pin a value to this point of the instruction stream: an empty volatile asm
// that reads and rewrites it. Scheduling fences order only instructions with
// side effects; pure arithmetic would otherwise drift to its first use (or up
// to its inputs). Pinning a piece's inputs before it and its results after it
// keeps each restore piece between the MFMAs it was written between.
__device__ __forceinline__ void pin(uint32_t &x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(float &x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(u32x4 &x) { asm volatile("" : "+v"(x)); }

// Wait until at most N vector-memory operations of this wave are outstanding
// and all of its LDS operations are done, then join the workgroup barrier. One
// asm block with a memory clobber: no LDS access moves across it, and the
// copies into LDS still in flight (the newest N operations) are not waited for.
template <int N>
__device__ __forceinline__ void wait_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// 16-byte copies from memory into LDS (buffer_load ... lds; lane L lands at
// M0 + 16 L) issued from inline asm, for kernels that also read LDS with
// ds_read_b64_tr_b16: the compiler makes every such read wait for all copies
// into LDS it knows of, which would stall the first transposed read of a step
// until the next step's tile has landed. Copies it does not see impose no such
// wait; the kernel orders them itself (barrier waits with explicit counts) and
// waits for vmcnt(0) before issuing them, so that the counts the compiler
// keeps for its own loads never span a copy.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 rsrc_words(const void *base, int64_t bytes) {
  if (bytes < 0) bytes = 0;
  const uint64_t a = (uint64_t)(uintptr_t)base;
  const int n = bytes >= 0x7fffffffll ? 0x7fffffff : (int)bytes;
  // same descriptor as make_rsrc: 48-bit base, stride 0, range n, raw 32-bit format
  return i32x4{(int)(uint32_t)a, (int)((uint32_t)(a >> 32) & 0xffffu), n, 0x00020000};
}
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t *)p;
}
__device__ __forceinline__ void dma16_asm(const i32x4 &rs, uint32_t m0v, uint32_t voff, uint32_t soff) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, %3 offen lds"
      :
      : "s"(m0v), "v"(voff), "s"(rs), "s"(soff)
      : "memory");  // M0 is reserved (never allocated); nothing else in the kernels that use this reads it
}
// Tiles of 512-byte rows read with ds_read_b64_tr_b16 (dX weight tiles,
// token-major adapter operands): row o takes 512 bytes; its 16-byte chunk c
// (columns 8c .. 8c+7) sits at chunk position c ^ wswz(o). With this swizzle
// the restore stores (16 lanes: 8 rows x 2 blocks, one chunk each) and the
// transposed fragment reads (32 lanes: 4 rows x 4 chunks, 8 bytes each) both
// land on 64 distinct banks.
__device__ __forceinline__ int wswz(int o) { return ((o & 3) << 2) | ((o >> 1) & 3); }

}  // namespace qlora
