// Adapter products at large token counts (T > 64), bound by streaming the
// token-major operand once.
//
// First page, "QLoRA의 수식" and "명제 1": the adapter path s B A x (s = alpha/r)
// needs, besides the two weight-sized contractions,
//   u  = x A^T   [T, r]      (forward intermediate)
//   v  = dY B    [T, r]      (backward intermediate)
//   dA = s v^T x [r, d_in]   and   dB = s dY^T u [d_out, r]
// Each reads a [T, d] activation (tens of MB at T = 4096) against a rank-sized
// operand, so the kernels are built around reading that activation once, in
// wide coalesced rows, while the rank-sized operand is shared through LDS.
//
// k_lora_tall (u, v): out[T, r] = P[T, K] Q[r, K]^T. A workgroup owns 64 tokens
// and a K range; per K step the token tile and the Q tile (r_pad x 64) are
// copied into LDS several steps ahead, and wave w computes the column tiles
// w, w+4, ... of all 64 tokens with v_mfma_f32_16x16x32_bf16. K ranges of one
// token tile are summed by the last range to finish (fixed order,
// device-scope partials).
//
// k_lora_wgrad (dA, dB): C = s sum_t X[t, :]^T Y[t, :] or its transpose, X the
// bf16 [T, D] activation, Y the float32 [T, R] intermediate (split into bf16
// high and low parts: two MFMAs, ~2^-16 relative). A workgroup owns 256
// columns of D by 64 of R and a token range; per 64-token step the X tile
// (64 x 512 bytes) and the Y tile (64 x 256 bytes) are copied into LDS two
// steps ahead, and the Y tile is converted in place into two bf16 planes. Both MFMA operands need 8 consecutive tokens per lane, which
// ds_read_b64_tr_b16 gathers from the token-major tiles. Token ranges of one
// tile are summed cooperatively: every range stores its float32 tile and sums
// its share of rows over all ranges in range order once all have arrived; a
// range that stops waiting leaves its share to the last one to arrive
// (split_arrive in common.h), so no range depends on another being dispatched.
#include <type_traits>

#include "kernels.h"
#include "tiles.h"

namespace qlora {

// ---------------------------------------------------------------------------
// u = x A^T, v = dY B
// ---------------------------------------------------------------------------
constexpr int kTallT = 64;  // tokens per workgroup
constexpr int kTallMaxSplit = 16;

// A token tile (64 tokens x 64 K) and the matching Q tile (32 NCQ rows x 64 K)
// share one ring slot; both are copied straight into LDS (every wave issues
// 2 + NCQ copies of 1 KB per K step, so the copy counts, and with them the
// barrier's wait count, are the same on every wave and every step). Rows take
// 128 bytes; chunk c of row q sits at chunk position c ^ ((q >> 1) & 7), so
// the 16 rows of one fragment read fall on 16 distinct bank groups. The ring
// keeps RS - 1 K steps in flight: at these sizes a workgroup's whole share is
// a few hundred KB, so latency, not bandwidth, is what the depth has to hide.
__device__ __forceinline__ int qsw(int q) { return (q >> 1) & 7; }

template <int NCQ, int RS>
__global__ __launch_bounds__(256) void k_lora_tall(const uint16_t *__restrict__ P, const uint16_t *__restrict__ Q,
                                                   int64_t T, int64_t K, int r, int r_pad, float scale,
                                                   float *__restrict__ out_f32, uint16_t *__restrict__ out_bf16,
                                                   float *__restrict__ partial, uint32_t *__restrict__ counters,
                                                   int ksplit) {
  constexpr int kSlot = 8192 + 4096 * NCQ;  // P tile + Q tile
  constexpr int kNtw = NCQ >= 2 ? NCQ / 2 : 1;  // column tiles of 16 per wave
  constexpr int kAhead = RS - 1;                // K steps in flight
  extern __shared__ __attribute__((aligned(16))) uint8_t tsm[];  // [RS][kSlot]
  __shared__ int is_last;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int li = lane & 15, g = lane >> 4;
  const int tile = blockIdx.x, part = blockIdx.y;
  const int64_t t0 = (int64_t)tile * kTallT;
  const int nk = (int)((K + 63) / 64);
  const int k0 = nk * part / ksplit, k1 = nk * (part + 1) / ksplit;
  const int nt = r_pad / 16;

  const int64_t prow = T - t0 < kTallT ? T - t0 : kTallT;
  const rsrc_t pr = make_rsrc(P + t0 * K, prow * K * 2);
  const rsrc_t qr = make_rsrc(Q, (int64_t)r * K * 2);  // rows r and up read zeros
  // copy q of this wave: P rows 8 (2w + q) .. +7 (q < 2), then Q rows
  // 8 (NCQ w + q') .. +7; lane L takes row 8 gi + L/8, chunk position L%8
  uint32_t src[2 + NCQ];
  int c8[2 + NCQ];
#pragma unroll
  for (int q = 0; q < 2 + NCQ; ++q) {
    const int row = 8 * (q < 2 ? 2 * wave + q : NCQ * wave + q - 2) + (lane >> 3);
    c8[q] = 8 * ((lane & 7) ^ qsw(row));
    src[q] = (uint32_t)((row * K + c8[q]) * 2);
  }
  auto copy_step = [&](int kk) {
    uint8_t *slot = tsm + ((kk - k0) % RS) * kSlot;
    const int klim = (int)(K - (int64_t)kk * 64);  // chunks at or past K read zeros
#pragma unroll
    for (int q = 0; q < 2 + NCQ; ++q) {
      const uint32_t keep = (uint32_t)((c8[q] - klim) >> 31);
      const uint32_t off = ((src[q] + (uint32_t)(kk * 128)) & keep) | (kOOB & ~keep);
      uint8_t *dst = q < 2 ? slot + 1024 * (2 * wave + q) : slot + 8192 + 1024 * (NCQ * wave + q - 2);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(q < 2 ? pr : qr, (lds_void *)dst, 16, off, 0, 0, 0);
    }
  };

  f32x4 acc[4][kNtw];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < kNtw; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Steps past the range copy step k1-1 again into free slots: every step
  // issues the same copies.
#pragma unroll
  for (int a = 0; a < kAhead; ++a) copy_step(k0 + a < k1 ? k0 + a : k1 - 1);
  for (int kk = k0; kk < k1; ++kk) {
    // step kk's copies are the oldest outstanding: kAhead - 1 later steps' may fly
    wait_barrier<(kAhead - 1) * (2 + NCQ)>();
    copy_step(kk + kAhead < k1 ? kk + kAhead : k1 - 1);  // into the slot step kk-1 used
    const uint8_t *slot = tsm + ((kk - k0) % RS) * kSlot;
    // Every fragment of the step is read before the first MFMA, so the step
    // waits for LDS once.
    u32x4 a[2][4], b[2][kNtw];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * i + li;
        a[h][i] = *reinterpret_cast<const u32x4 *>(slot + row * 128 + (((4 * h + g) ^ qsw(row)) << 4));
      }
#pragma unroll
      for (int j = 0; j < kNtw; ++j) {
        const int ct = wave + 4 * j;  // column tile
        const int row = 16 * ct + li;
        b[h][j] = ct < nt ? *reinterpret_cast<const u32x4 *>(slot + 8192 + row * 128 + (((4 * h + g) ^ qsw(row)) << 4))
                          : u32x4{0u, 0u, 0u, 0u};  // (wave-uniform) no such tile
      }
    }
    // Unconditional MFMAs: a wave past the last column tile multiplies its
    // zero B fragment, so that accumulator stays zero and is never stored. (A
    // branch around them would make the compiler copy the accumulators out of
    // and back into the matrix registers around every group of four.)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int j = 0; j < kNtw; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i][j] = mfma16(a[h][i], b[h][j], acc[i][j]);
  }

  // lane (li, g): tokens 16i + 4g + e of token tile i, column 16 ct + li
  if (ksplit == 1) {
#pragma unroll
    for (int j = 0; j < kNtw; ++j) {
      const int ct = wave + 4 * j;
      if (ct >= nt) continue;
      const int col = 16 * ct + li;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t tt = t0 + 16 * i + 4 * g + e;
          if (tt < T) {
            if (out_f32 && col < r) out_f32[tt * r + col] = acc[i][j][e];
            if (out_bf16)
              out_bf16[tt * r_pad + col] = (uint16_t)(pack_bf16x2(col < r ? scale * acc[i][j][e] : 0.f, 0.f) & 0xffffu);
          }
        }
    }
    return;
  }
  float *pbase = partial + ((int64_t)tile * ksplit + part) * kTallT * r_pad;
#pragma unroll
  for (int j = 0; j < kNtw; ++j) {
    const int ct = wave + 4 * j;
    if (ct >= nt) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) st_dev(pbase + (16 * i + 4 * g + e) * r_pad + 16 * ct + li, acc[i][j][e]);
  }
  wait_vmem();
  __syncthreads();
  if (tid == 0) is_last = add_dev_u32(tile_counter(counters, tile), 1u) == (uint32_t)ksplit - 1u;
  __syncthreads();
  if (!is_last) return;
  // Sum the parts in part order. ksplit is a power of two; each thread takes
  // 16 / ksplit 4-float chunks at a time and issues every part's load of all
  // of them before the first is used (loads past the chunks read zeros), so
  // the sum costs one round trip per batch, not one per load.
  const rsrc_t prs = make_rsrc(partial + (int64_t)tile * ksplit * kTallT * r_pad,
                               (int64_t)ksplit * kTallT * r_pad * 4);
  auto combine = [&](auto ks_c) __attribute__((always_inline)) {
    constexpr int KS = decltype(ks_c)::value;
    constexpr int CPB = kTallMaxSplit / KS;
    const int nch = kTallT * r_pad / 4;
    for (int c0 = tid; c0 < nch; c0 += 256 * CPB) {
      u32x4 w[CPB][KS];
#pragma unroll
      for (int j = 0; j < CPB; ++j)
#pragma unroll
        for (int p = 0; p < KS; ++p) {
          const int c = c0 + 256 * j;
          w[j][p] = bld16_dev(prs, c < nch ? (uint32_t)((p * kTallT * r_pad + 4 * c) * 4) : kOOB);
        }
#pragma unroll
      for (int j = 0; j < CPB; ++j) {
        const int c = c0 + 256 * j;
        f32x4 v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int p = 0; p < KS; ++p)
          v += f32x4{__uint_as_float(w[j][p][0]), __uint_as_float(w[j][p][1]), __uint_as_float(w[j][p][2]),
                     __uint_as_float(w[j][p][3])};
        const int row = (4 * c) / r_pad, col0 = (4 * c) % r_pad;
        const int64_t tt = t0 + row;
        if (c < nch && tt < T) {
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int col = col0 + u;
            if (out_f32 && col < r) out_f32[tt * r + col] = v[u];
            if (out_bf16)
              out_bf16[tt * r_pad + col] = (uint16_t)(pack_bf16x2(col < r ? scale * v[u] : 0.f, 0.f) & 0xffffu);
          }
        }
      }
    }
  };
  switch (ksplit) {
    case 2: combine(std::integral_constant<int, 2>{}); break;
    case 4: combine(std::integral_constant<int, 4>{}); break;
    case 8: combine(std::integral_constant<int, 8>{}); break;
    default: combine(std::integral_constant<int, 16>{}); break;
  }
  if (tid == 0) st_dev_u32(tile_counter(counters, tile), 0u);
}

int lora_tall_ksplit(int64_t T, int64_t K) {
  const int cus = device_cu_count(current_device());
  const int64_t tiles = (T + kTallT - 1) / kTallT, nk = (K + 63) / 64;
  int64_t ks = cus / tiles;
  if (ks > nk / 4) ks = nk / 4;
  if (ks > kTallMaxSplit) ks = kTallMaxSplit;
  if (ks < 1) ks = 1;
  if (tiles > kMaxTileCounters) ks = 1;
  while (ks & (ks - 1)) ks &= ks - 1;  // a power of two (the combine batches loads by it)
  return (int)ks;
}

size_t lora_tall_partial_floats(int64_t T, int64_t K, int r_pad) {
  const int ks = lora_tall_ksplit(T, K);
  return ks > 1 ? (size_t)((T + kTallT - 1) / kTallT) * ks * kTallT * r_pad : 0;
}

template <int NCQ, int RS>
static hipError_t launch_tall(const uint16_t *P, const uint16_t *Q, int64_t T, int64_t K, int r, int r_pad,
                              float scale, float *out_f32, uint16_t *out_bf16, float *partial, uint32_t *counters,
                              hipStream_t st) {
  constexpr int kLds = RS * (8192 + 4096 * NCQ);
  static DeviceOnce once;
  const hipError_t e = once.run(current_device(), [] {
    return hipFuncSetAttribute(reinterpret_cast<const void *>(k_lora_tall<NCQ, RS>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, kLds);
  });
  if (e != hipSuccess) return e;
  const int ks = lora_tall_ksplit(T, K);
  const int64_t tiles = (T + kTallT - 1) / kTallT;
  k_lora_tall<NCQ, RS><<<dim3((unsigned)tiles, (unsigned)ks), dim3(256), kLds, st>>>(
      P, Q, T, K, r, r_pad, scale, out_f32, out_bf16, partial, counters, ks);
  return hipGetLastError();
}

hipError_t launch_lora_tall(const uint16_t *P, const uint16_t *Q, int64_t T, int64_t K, int r, int r_pad, float scale,
                            float *out_f32, uint16_t *out_bf16, float *partial, uint32_t *counters, hipStream_t st) {
  if (r_pad < 16 || r_pad > 256 || r_pad % 16 != 0) return hipErrorInvalidValue;
  if (r_pad <= 32) return launch_tall<1, 8>(P, Q, T, K, r, r_pad, scale, out_f32, out_bf16, partial, counters, st);
  if (r_pad <= 64) return launch_tall<2, 6>(P, Q, T, K, r, r_pad, scale, out_f32, out_bf16, partial, counters, st);
  if (r_pad <= 128) return launch_tall<4, 5>(P, Q, T, K, r, r_pad, scale, out_f32, out_bf16, partial, counters, st);
  return launch_tall<8, 3>(P, Q, T, K, r, r_pad, scale, out_f32, out_bf16, partial, counters, st);
}

// ---------------------------------------------------------------------------
// dA = s v^T x, dB = s dY^T u
// ---------------------------------------------------------------------------
constexpr int kWgD = 256;             // D columns per workgroup (64 per wave)
constexpr int kWgR = 64;              // R columns per workgroup
constexpr int kWgTok = 64;            // tokens per step
constexpr int kXTile = kWgTok * 512;  // bytes of one X tile (64 tokens x 256 bf16)
constexpr int kYPlane = kWgTok * 128; // bytes of one bf16 Y plane (64 tokens x 64)
constexpr int kWgSlot = kXTile + 2 * kYPlane;  // X tile + float32 Y tile (later its two planes)
constexpr int kWgRing = 3;            // two steps in flight
constexpr int kWgTileFloats = kWgD * kWgR;
constexpr size_t kWgLds = (size_t)kWgRing * kWgSlot;
constexpr int kWgMaxSplit = 16;
constexpr int kWgCopies = 8 + 4;      // 1 KB copies per wave per step: X, then Y

// Y planes: row t takes 128 bytes; chunk c sits at c ^ ysw(t), which keeps both
// the plane stores (32 lanes: 2 rows x 16 half-chunks) and the transposed reads
// (32 lanes: 4 rows x 4 chunks) on 64 distinct banks.
__device__ __forceinline__ int ysw(int t) { return 4 * ((t >> 1) & 1); }

// LDS-only workgroup barrier (copies into LDS may stay in flight).
__device__ __forceinline__ void lds_only_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <bool kYisA>
__global__ __launch_bounds__(256) void k_lora_wgrad(const uint16_t *__restrict__ X, const float *__restrict__ Y,
                                                    int64_t T, int64_t D, int64_t R, float scale,
                                                    float *__restrict__ C, float *__restrict__ partial,
                                                    uint32_t *__restrict__ counters, uint32_t *__restrict__ fallbacks,
                                                    int ksplit) {
  // Ring slot: [X tile 64 x 512 B][Y: float32 64 x 256 B as copied, then in
  // place the bf16 high plane (first 8 KB) and low plane (next 8 KB)].
  extern __shared__ __attribute__((aligned(16))) uint8_t wsm[];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int gr = (int)((R + kWgR - 1) / kWgR);
  const int tile = blockIdx.x, part = blockIdx.y;
  const int64_t d0 = (int64_t)(tile / gr) * kWgD, r0 = (int64_t)(tile % gr) * kWgR;
  const int nkt = (int)((T + kWgTok - 1) / kWgTok);
  const int k0 = nkt * part / ksplit, k1 = nkt * (part + 1) / ksplit;

  // X copies: wave w issues copies gi = 8w + q (q < 8) of token rows 2 gi,
  // 2 gi + 1; lane L fills row 2 gi + L/32, chunk position L%32 (wswz).
  uint32_t xsrc[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int row = 2 * (8 * wave + q) + (lane >> 5);
    const int c = (lane & 31) ^ wswz(row);
    const int64_t d = d0 + 8 * c;
    xsrc[q] = d < D ? (uint32_t)((row * D + d) * 2) : kOOB;  // columns past D read zeros
  }
  // Y copies: wave w issues copies gi = 4w + q (q < 4) of token rows 4 gi ..
  // 4 gi + 3 (256 bytes each, unswizzled); lane L fills row 4 gi + L/16,
  // columns 4 (L%16) .. +3.
  uint32_t ysrc[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = 4 * (4 * wave + q) + (lane >> 4);
    const int64_t col = r0 + 4 * (lane & 15);
    ysrc[q] = col < R ? (uint32_t)((row * R + col) * 4) : kOOB;  // columns past R read zeros
  }
  // Every step issues the same 12 copies per wave (steps past the range copy
  // its last step again into a free slot).
  auto copy_step = [&](int kt) {
    const int kc = kt < k1 ? kt : k1 - 1;
    const int64_t t0 = (int64_t)kc * kWgTok;
    const int64_t rows = T - t0 < kWgTok ? T - t0 : kWgTok;
    const uint32_t base = lds_addr(wsm + ((kt - k0) % kWgRing) * kWgSlot);
    const i32x4 xs = rsrc_words(X + t0 * D, rows * D * 2);
#pragma unroll
    for (int q = 0; q < 8; ++q) dma16_asm(xs, base + 1024u * (uint32_t)(8 * wave + q), xsrc[q], 0u);
    const i32x4 ys = rsrc_words(Y + t0 * R, rows * R * 4);
#pragma unroll
    for (int q = 0; q < 4; ++q) dma16_asm(ys, base + kXTile + 1024u * (uint32_t)(4 * wave + q), ysrc[q], 0u);
  };
  // float32 Y tile -> bf16 high and low planes, in place (reads, barrier, stores)
  auto split_y = [&](uint8_t *y) {
    u32x4 v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = *reinterpret_cast<const u32x4 *>(y + 16 * (tid + 256 * q));
    lds_only_barrier();
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = tid + 256 * q, t = c >> 4, c4 = c & 15;
      const float f0 = __uint_as_float(v[q][0]), f1 = __uint_as_float(v[q][1]);
      const float f2 = __uint_as_float(v[q][2]), f3 = __uint_as_float(v[q][3]);
      const uint32_t h0 = pack_bf16x2(f0, f1), h1 = pack_bf16x2(f2, f3);
      const uint32_t l0 = pack_bf16x2(f0 - bf16_lo_to_f32(h0), f1 - bf16_hi_to_f32(h0));
      const uint32_t l1 = pack_bf16x2(f2 - bf16_lo_to_f32(h1), f3 - bf16_hi_to_f32(h1));
      const int off = t * 128 + (((c4 >> 1) ^ ysw(t)) << 4) + (c4 & 1) * 8;
      *reinterpret_cast<u32x2 *>(y + off) = u32x2{h0, h1};
      *reinterpret_cast<u32x2 *>(y + kYPlane + off) = u32x2{l0, l1};
    }
    lds_only_barrier();
  };

  // Transposed fragment reads: lane u of group g addresses token row
  // 32(g/2) + 8s + u/4 (and four rows further down), columns 16(g%2) + 4(u%4)
  // of a 32-column tile; the lane then holds 8 consecutive tokens (token order
  // inside a step: slice s, lane half h covers tokens 32h + 8s .. +7, the same
  // for both operands) of column l%32. Row mod 8 does not depend on s.
  const int grp = lane >> 4, u16 = lane & 15;
  uint32_t xoff[2][2], yoff[2][2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int row = 32 * (grp >> 1) + (u16 >> 2) + 4 * hh;
      const int xc = 64 * wave + 32 * j + 16 * (grp & 1) + 4 * (u16 & 3);
      xoff[j][hh] = (uint32_t)(row * 512 + (((xc >> 3) ^ wswz(row)) << 4) + (xc & 7) * 2);
      const int yc = 32 * j + 16 * (grp & 1) + 4 * (u16 & 3);
      yoff[j][hh] = (uint32_t)(row * 128 + (((yc >> 3) ^ ysw(row)) << 4) + (yc & 7) * 2);
    }
  auto tr = [&](const uint8_t *base, uint32_t lo_off, uint32_t hi_off) {
    const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(base + lo_off));
    const v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(base + hi_off));
    const u32x2 a2 = __builtin_bit_cast(u32x2, a), b2 = __builtin_bit_cast(u32x2, b);
    return u32x4{a2[0], a2[1], b2[0], b2[1]};
  };

  // acc[a][b]: kYisA: a = R tile, b = this wave's D tile; else a = D tile, b = R tile
  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.f;

  copy_step(k0);
  copy_step(k0 + 1);
  for (int kt = k0; kt < k1; ++kt) {
    // step kt's copies are the oldest outstanding; every wave is done with step kt-1
    wait_barrier<kWgCopies>();
    copy_step(kt + 2);  // into the slot step kt-1 used
    uint8_t *sl = wsm + ((kt - k0) % kWgRing) * kWgSlot;
    split_y(sl + kXTile);
    const uint8_t *xs = sl, *yh = sl + kXTile, *yl = yh + kYPlane;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4 fx[2], fh[2], fl[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        fx[j] = tr(xs + 4096 * s, xoff[j][0], xoff[j][1]);
        fh[j] = tr(yh + 1024 * s, yoff[j][0], yoff[j][1]);
        fl[j] = tr(yl + 1024 * s, yoff[j][0], yoff[j][1]);
      }
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          if (kYisA) {
            acc[a][b] = mfma32(fh[a], fx[b], acc[a][b]);
            acc[a][b] = mfma32(fl[a], fx[b], acc[a][b]);
          } else {
            acc[a][b] = mfma32(fx[a], fh[b], acc[a][b]);
            acc[a][b] = mfma32(fx[a], fl[b], acc[a][b]);
          }
        }
    }
  }
  wait_vmem();  // the last steps' copies (never read) are done before anything else

  // Output tile: kYisA: rows R (64), columns D (256), C row pitch D; else rows
  // D (256), columns R (64), C row pitch R. Lane l, accumulator e of acc[a][b]
  // sits at row 32a + 8(e/4) + 4(l/32) + e%4 (+64w for D rows), column
  // 32b + l%32 (+64w for D columns).
  const int64_t M = kYisA ? R : D, N = kYisA ? D : R;
  const int64_t m0 = kYisA ? r0 : d0, n0 = kYisA ? d0 : r0;
  auto rc = [&](int a, int b, int e, int &row, int &col) {
    row = 32 * a + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3) + (kYisA ? 0 : 64 * wave);
    col = 32 * b + (lane & 31) + (kYisA ? 64 * wave : 0);
  };
  if (ksplit == 1) {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          int row, col;
          rc(a, b, e, row, col);
          if (m0 + row < M && n0 + col < N) C[(m0 + row) * N + n0 + col] = scale * acc[a][b][e];
        }
    return;
  }
  // Cooperative sum of the token ranges (see the file comment). A range's
  // float32 tile is stored in register order: 16-byte chunk
  // g = (((w 2 + a) 2 + b) 4 + e4) 64 + l holds acc[a][b][4 e4 .. 4 e4 + 3] of
  // lane l of wave w, so each store instruction writes 1 KB contiguously.
  const rsrc_t prs = make_rsrc(partial + (size_t)tile * ksplit * kWgTileFloats, (int64_t)ksplit * kWgTileFloats * 4);
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int g = (((wave * 2 + a) * 2 + b) * 4 + e4) * 64 + lane;
        const u32x4 v = {__float_as_uint(acc[a][b][4 * e4]), __float_as_uint(acc[a][b][4 * e4 + 1]),
                         __float_as_uint(acc[a][b][4 * e4 + 2]), __float_as_uint(acc[a][b][4 * e4 + 3])};
        __builtin_amdgcn_raw_buffer_store_b128(v, prs, (uint32_t)((part * kWgTileFloats + 4 * g) * 4), 0, 16);
      }
  wait_barrier<0>();  // every wave's stores have completed
  // Share p of the tile is chunks [p N / ksplit, (p+1) N / ksplit) (N chunks of
  // four rows of one column, in the accumulator layout above), summed over all
  // ranges in range order by whichever workgroup claims it (split_arrive).
  __shared__ uint32_t claim_lds[2];
  uint32_t *line = tile_counter(counters, tile);
  if (tid == 0) {
    bool last;
    claim_lds[0] = split_arrive(line, part, ksplit, last, fallbacks);
    claim_lds[1] = last ? 1u : 0u;
  }
  wait_barrier<0>();
  // ksplit is a power of two, so a share is 16 / ksplit chunks per thread:
  // every part's load of all of them goes out before the first is used.
  auto sum_shares_ks = [&](uint32_t mask, auto ks_c) __attribute__((always_inline)) {
    constexpr int KS = decltype(ks_c)::value;
    constexpr int CPB = kWgMaxSplit / KS;
    for (int sh = 0; sh < KS; ++sh) {
      if (!((mask >> sh) & 1u)) continue;
      const int glo = sh * (kWgTileFloats / 4) / KS, ghi = (sh + 1) * (kWgTileFloats / 4) / KS;
      for (int g0 = glo + tid; g0 < ghi; g0 += 256 * CPB) {
        u32x4 w[CPB][KS];
#pragma unroll
        for (int j = 0; j < CPB; ++j)
#pragma unroll
          for (int p = 0; p < KS; ++p) {
            const int g = g0 + 256 * j;
            w[j][p] = bld16_dev(prs, g < ghi ? (uint32_t)((p * kWgTileFloats + 4 * g) * 4) : kOOB);
          }
#pragma unroll
        for (int j = 0; j < CPB; ++j) {
          const int g = g0 + 256 * j;
          f32x4 v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int p = 0; p < KS; ++p)
            v += f32x4{__uint_as_float(w[j][p][0]), __uint_as_float(w[j][p][1]), __uint_as_float(w[j][p][2]),
                       __uint_as_float(w[j][p][3])};
          const int gl = g & 63, e4 = (g >> 6) & 3, b = (g >> 8) & 1, a = (g >> 9) & 1, gw = g >> 10;
          const int row = 32 * a + 8 * e4 + 4 * (gl >> 5) + (kYisA ? 0 : 64 * gw);
          const int col = 32 * b + (gl & 31) + (kYisA ? 64 * gw : 0);
          if (g < ghi && n0 + col < N) {
#pragma unroll
            for (int u = 0; u < 4; ++u)
              if (m0 + row + u < M) C[(m0 + row + u) * N + n0 + col] = scale * v[u];
          }
        }
      }
    }
  };
  auto sum_shares = [&](uint32_t mask) __attribute__((always_inline)) {
    switch (ksplit) {
      case 2: sum_shares_ks(mask, std::integral_constant<int, 2>{}); break;
      case 4: sum_shares_ks(mask, std::integral_constant<int, 4>{}); break;
      case 8: sum_shares_ks(mask, std::integral_constant<int, 8>{}); break;
      default: sum_shares_ks(mask, std::integral_constant<int, 16>{}); break;
    }
  };
  const uint32_t mine = claim_lds[0];
  const bool last = claim_lds[1] != 0u;
  sum_shares(mine);
  if (last) {
    wait_barrier<0>();  // every wave has read the claim words
    if (wave == 0) {
      const uint32_t m = split_sweep(line, part, ksplit, lane);
      if (lane == 0) claim_lds[0] = m;
    }
    wait_barrier<0>();
    sum_shares(claim_lds[0]);
  }
  if (tid == 0) split_depart(line, ksplit);
}

// Token split: as many ranges as keep all of a launch's workgroups resident at
// once (then the ranges of a tile share the combine), at least two 64-token
// steps each.
int lora_wgrad_ksplit(int64_t D, int64_t R, int64_t T) {
  const int cus = device_cu_count(current_device());
  const int64_t tiles = ((D + kWgD - 1) / kWgD) * ((R + kWgR - 1) / kWgR);
  const int64_t nkt = (T + kWgTok - 1) / kWgTok;
  int64_t ks = cus / (tiles > 0 ? tiles : 1);
  if (ks > nkt / 2) ks = nkt / 2;
  if (ks > kWgMaxSplit) ks = kWgMaxSplit;
  if (ks < 1) ks = 1;
  if (tiles > kMaxTileCounters) ks = 1;
  while (ks & (ks - 1)) ks &= ks - 1;  // a power of two (the share sums batch loads by it)
  return (int)ks;
}

size_t lora_wgrad_partial_floats(int64_t D, int64_t R, int64_t T) {
  const int ks = lora_wgrad_ksplit(D, R, T);
  const int64_t tiles = ((D + kWgD - 1) / kWgD) * ((R + kWgR - 1) / kWgR);
  return ks > 1 ? (size_t)tiles * ks * kWgTileFloats : 0;
}

hipError_t launch_lora_wgrad(const uint16_t *X, const float *Y, int64_t T, int64_t D, int64_t R, bool y_is_rows,
                             float scale, float *C, float *partial, uint32_t *counters, uint32_t *fallbacks,
                             hipStream_t st) {
  static DeviceOnce once;
  const hipError_t e = once.run(current_device(), [] {
    const hipError_t s = hipFuncSetAttribute(reinterpret_cast<const void *>(k_lora_wgrad<true>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)kWgLds);
    if (s != hipSuccess) return s;
    return hipFuncSetAttribute(reinterpret_cast<const void *>(k_lora_wgrad<false>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)kWgLds);
  });
  if (e != hipSuccess) return e;
  const int ks = lora_wgrad_ksplit(D, R, T);
  const int64_t tiles = ((D + kWgD - 1) / kWgD) * ((R + kWgR - 1) / kWgR);
  const dim3 grid((unsigned)tiles, (unsigned)ks);
  if (y_is_rows)
    k_lora_wgrad<true><<<grid, dim3(256), kWgLds, st>>>(X, Y, T, D, R, scale, C, partial, counters, fallbacks, ks);
  else
    k_lora_wgrad<false><<<grid, dim3(256), kWgLds, st>>>(X, Y, T, D, R, scale, C, partial, counters, fallbacks, ks);
  return hipGetLastError();
}

}  // namespace qlora
