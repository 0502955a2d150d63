// Large-T contractions with on-the-fly NF4 restore (bf16 MFMA, fp32 accumulate).
//
// Forward  h  = x W_hat^T + su B^T     (first page, "QLoRA의 수식")
// Backward dX = dY W_hat + sv A        (same section and "명제 1": the gradient
//                                       passes through the restored frozen W;
//                                       "48GB GPU Fine-Tuning a 65B Model",
//                                       "QLoRA Puts the Two Methods in Different
//                                       Places")
// The weight blocks are restored to bf16 tile by tile and discarded after use
// ("48GB...": each block is restored to bf16 for the multiplication, then
// discarded). The adapter term enters as extra K columns: [x | su] . [W_hat | B]^T
// and [dY | sv] . [W_hat ; A].
//
// Tiling: a 256-thread workgroup (four waves, one per SIMD) computes a 256 x 256
// output tile; wave w owns all 256 rows and columns 64w .. 64w+63 (8 x 2
// v_mfma_f32_32x32x16_bf16 tiles, 256 accumulators per lane). K advances 64 at
// a time. On gfx950 the matrix cores are starved first by LDS stores (they
// stall MFMA issue), then by LDS reads; VALU work co-issues with MFMAs almost
// for free. Hence:
//   * activation tiles (x, dY, su, sv) go from memory straight into LDS with
//     buffer_load ... lds (no registers, no LDS store instructions), two tiles
//     in a ring: the copy of step k+1 runs during step k;
//   * forward: a wave's B operand (8 consecutive K of one output row per lane)
//     is exactly one 32-bit word of packed codes, so each lane restores its own
//     fragments in registers from its codes and block scale; no weight tile
//     touches LDS and every weight is restored once per workgroup;
//   * dX: K = d_out runs across weight rows, so a lane's fragment needs one
//     nibble from each of 8 rows. The workgroup restores the 64 x 256 weight
//     tile of step k+1 into LDS during step k (one 64-weight block per lane)
//     and the waves read B fragments with ds_read_b64_tr_b16, which transposes
//     16-bit data across each 16 lanes;
//   * the K order inside a step is permuted the same way for both operands:
//     slice s, lane half h covers K columns 32h + 8s .. +7, so a lane's four
//     forward code words of a step are one 16-byte load;
//   * the restore and the fragment reads of the next slice are cut into pieces
//     of a few instructions, one after each MFMA, with scheduling fences that
//     keep the order; the one barrier per step sits in the middle of the last
//     slice so that the matrix core keeps working across it.
// The epilogue goes through LDS so that every lane writes 16-byte rows.
#include "kernels.h"
#include "tiles.h"

namespace qlora {

constexpr int kBM = 256, kBN = 256, kBK = 64;
constexpr int kThreads = 256;                 // four waves, one per SIMD
constexpr int kWN = 64;                       // output columns per wave
constexpr int kTile = kBM * kBK * 2;          // bytes of one swizzled 256 x 64 bf16 activation tile
constexpr int kWRow = kBN * 2;                // bytes per row of the dX [k][n] weight tile (unpadded)
constexpr int kWTile = kBK * kWRow;           // bytes of one dX weight tile
constexpr int kEP = kWN + 8;                  // epilogue staging pitch (bf16)
constexpr size_t kStageLds = (size_t)4 * kBM * kEP * 2;
constexpr size_t kFwdTiles = (size_t)2 * kTile;
constexpr size_t kDxTiles = (size_t)2 * kTile + (size_t)2 * kWTile;
constexpr size_t kFwdLds = kFwdTiles > kStageLds ? kFwdTiles : kStageLds;
constexpr size_t kDxLds = kDxTiles > kStageLds ? kDxTiles : kStageLds;

// Activation tiles in LDS: row r (0..255) takes 128 bytes at 128 r; its 16-byte
// chunk c (K columns 8c .. 8c+7) sits at chunk position c ^ swz(r), which puts
// the 16 rows of one fragment read on 16 distinct bank groups.
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

// Copies of rows 0..255, K columns k0 .. k0+63 of a bf16 matrix (row pitch
// `pitch` elements; the buffer range covers the valid rows, rows past it read
// zeros) into a swizzled tile. Wave w issues 8 copies of 1 KB (8 rows each);
// lane L fills row 8g + L/8, chunk position L%8. DmaOffs holds each lane's
// source byte offsets for k0 = 0; full tiles add 2 k0 as the scalar offset.
struct DmaOffs {
  uint32_t v[8];
};
__device__ __forceinline__ DmaOffs dma_offsets(int pitch, int wave, int lane) {
  DmaOffs o;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int r = 8 * (8 * wave + q) + (lane >> 3);
    o.v[q] = (uint32_t)(r * pitch + 8 * ((lane & 7) ^ swz(r))) * 2u;
  }
  return o;
}
// Tile with K columns k0 .. k0+63 all below klim: no per-lane checks.
__device__ __forceinline__ void dma_tile(rsrc_t src, const DmaOffs &o, int k0, uint8_t *tile, int wave) {
#pragma unroll
  for (int q = 0; q < 8; ++q)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (lds_void *)(tile + 1024 * (8 * wave + q)), 16, o.v[q],
                                             2 * k0, 0, 0);
}
// Tile reaching past klim (a K tail): chunks at or past klim read zeros.
__device__ __forceinline__ void dma_tile_tail(rsrc_t src, const DmaOffs &o, int k0, int klim, uint8_t *tile,
                                              int wave, int lane) {
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int r = 8 * (8 * wave + q) + (lane >> 3);
    const int c8 = 8 * ((lane & 7) ^ swz(r));
    const uint32_t keep = (uint32_t)((c8 - (klim - k0)) >> 31);  // all ones if k0 + c8 < klim
    const uint32_t off = ((o.v[q] + 2u * (uint32_t)k0) & keep) | (kOOB & ~keep);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (lds_void *)(tile + 1024 * (8 * wave + q)), 16, off, 0, 0, 0);
  }
}
// Checked copies (chunks at or past klim read zeros) from asm.
__device__ __forceinline__ void dma_tile_asm(const i32x4 &rs, const DmaOffs &o, int k0, int klim, uint8_t *tile,
                                             int wave, int lane) {
  const uint32_t base = lds_addr(tile);
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int r = 8 * (8 * wave + q) + (lane >> 3);
    const int c8 = 8 * ((lane & 7) ^ swz(r));
    const uint32_t keep = (uint32_t)((c8 - (klim - k0)) >> 31);  // all ones if k0 + c8 < klim
    const uint32_t off = ((o.v[q] + 2u * (uint32_t)k0) & keep) | (kOOB & ~keep);
    dma16_asm(rs, base + 1024u * (uint32_t)(8 * wave + q), off, 0u);
  }
}

__device__ __forceinline__ void dma_any(rsrc_t src, const DmaOffs &o, int k0, int klim, uint8_t *tile, int wave,
                                        int lane) {
  if (k0 + kBK <= klim)
    dma_tile(src, o, k0, tile, wave);
  else
    dma_tile_tail(src, o, k0, klim, tile, wave, lane);
}

// Byte offset (within a tile) of lane (m = l%32, h = l/32)'s A fragment of
// slice s in row tile 0; row tile i adds 4096 i. The fragment holds row m,
// K columns 32h + 8s .. +7 (chunk 4h + s).
__device__ __forceinline__ int a_off(int lane, int s) {
  const int m = lane & 31, h = lane >> 5;
  return m * 128 + (((4 * h + s) ^ swz(m)) << 4);
}

// Restore-table build of one 64-weight block cut into 3 pieces: products of
// the first and second half of the 16 levels, then the byte planes. The scale
// code is combined with q2o (the absmax-only marker) only after it is pinned:
// an OR of the raw loaded byte would be pure arithmetic that the compiler may
// hoist to the top of the step, where it would wait for the load there.
struct TableBuild {
  float sh;
  uint32_t p[8];
  __device__ __forceinline__ void run(int k, uint32_t q2, uint32_t q2o, float S, Nf4Planes &t) {
    if (k == 0) {
      pin(q2);
      pin(S);
      sh = restore_scale(q2 | q2o, S);
      pin(sh);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        p[u] = pack_bf16x2(code_times(2 * u, sh), code_times(2 * u + 1, sh));
        pin(p[u]);
      }
    } else if (k == 1) {
#pragma unroll
      for (int u = 4; u < 8; ++u) {
        p[u] = pack_bf16x2(code_times(2 * u, sh), code_times(2 * u + 1, sh));
        pin(p[u]);
      }
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        t.lo[u] = perm(p[2 * u + 1], p[2 * u], 0x06040200u);
        t.hi[u] = perm(p[2 * u + 1], p[2 * u], 0x07050301u);
        pin(t.lo[u]);
        pin(t.hi[u]);
      }
    }
  }
};

// The same table build cut into 7 pieces of 4 to 6 VALU instructions: the
// restored scale, two pairs of level products each (4), the low planes, the
// high planes.
struct TableBuild7 {
  float sh;
  uint32_t p[8];
  __device__ __forceinline__ void run(int k, uint32_t q2, uint32_t q2o, float S, Nf4Planes &t) {
    if (k == 0) {
      pin(q2);
      pin(S);
      sh = restore_scale(q2 | q2o, S);
      pin(sh);
    } else if (k <= 4) {
#pragma unroll
      for (int u = 2 * (k - 1); u < 2 * k; ++u) {
        p[u] = pack_bf16x2(code_times(2 * u, sh), code_times(2 * u + 1, sh));
        pin(p[u]);
      }
    } else if (k == 5) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        t.lo[u] = perm(p[2 * u + 1], p[2 * u], 0x06040200u);
        pin(t.lo[u]);
      }
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        t.hi[u] = perm(p[2 * u + 1], p[2 * u], 0x07050301u);
        pin(t.hi[u]);
      }
    }
  }
};

// expand8 cut into 4 pieces: selectors, low-plane lookups, high-plane
// lookups, interleave (the result is complete after piece 3).
struct Expand {
  uint32_t sa, ma, sb, mb, lo_a, hi_a, lo_b, hi_b;
  __device__ __forceinline__ void run(int ph, const Nf4Planes &t, uint32_t w, u32x4 &out) {
    if (ph == 0) {
      pin(w);
      sa = w & 0x07070707u;
      ma = ((w >> 1) & 0x04040404u) | 0x03020100u;
      sb = (w >> 4) & 0x07070707u;
      mb = ((w >> 5) & 0x04040404u) | 0x03020100u;
      pin(sa);
      pin(ma);
      pin(sb);
      pin(mb);
    } else if (ph == 1) {
      lo_a = lookup4(t.lo, sa, ma);
      hi_a = lookup4(t.hi, sa, ma);
      pin(lo_a);
      pin(hi_a);
    } else if (ph == 2) {
      lo_b = lookup4(t.lo, sb, mb);
      hi_b = lookup4(t.hi, sb, mb);
      pin(lo_b);
      pin(hi_b);
    } else {
      out[0] = perm(hi_a, lo_a, 0x05010400u);
      out[1] = perm(hi_a, lo_a, 0x07030602u);
      out[2] = perm(hi_b, lo_b, 0x05010400u);
      out[3] = perm(hi_b, lo_b, 0x07030602u);
      pin(out);
    }
  }
};

// expand8 cut into 8 pieces of 3 or 4 VALU instructions each, so that every
// MFMA of a slice carries at most about four (a single wave co-issues that
// many with a 32-cycle MFMA for free; one piece of 9 stalls the next MFMA):
// selectors (3 pieces), the four plane lookups, the interleave.
struct Expand8 {
  // (the code word is kept as pinned in piece 0: pure arithmetic on the loaded
  // word would otherwise drift up to the load's wait, all pieces at once)
  uint32_t c, x, sa, ma, sb, mb, lo_a, hi_a, lo_b, hi_b;
  __device__ __forceinline__ void run(int ph, const Nf4Planes &t, uint32_t w, u32x4 &out) {
    if (ph == 0) {
      c = w;
      pin(c);
      sa = c & 0x07070707u;
      x = (c >> 1) & 0x04040404u;
      pin(sa);
      pin(x);
    } else if (ph == 1) {
      ma = x | 0x03020100u;
      sb = (c >> 4) & 0x07070707u;
      pin(ma);
      pin(sb);
    } else if (ph == 2) {
      mb = ((c >> 5) & 0x04040404u) | 0x03020100u;
      pin(mb);
    } else if (ph == 3) {
      lo_a = lookup4(t.lo, sa, ma);
      pin(lo_a);
    } else if (ph == 4) {
      hi_a = lookup4(t.hi, sa, ma);
      pin(hi_a);
    } else if (ph == 5) {
      lo_b = lookup4(t.lo, sb, mb);
      pin(lo_b);
    } else if (ph == 6) {
      hi_b = lookup4(t.hi, sb, mb);
      pin(hi_b);
    } else {
      out[0] = perm(hi_a, lo_a, 0x05010400u);
      out[1] = perm(hi_a, lo_a, 0x07030602u);
      out[2] = perm(hi_b, lo_b, 0x05010400u);
      out[3] = perm(hi_b, lo_b, 0x07030602u);
      pin(out);
    }
  }
};

__device__ __forceinline__ void zero_acc(f32x16 (&acc)[8][2]) {
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
}

// Epilogue through LDS: a wave's 256 x 64 tile is staged as bf16 rows in this
// wave's region (pitch kEP), then written out so that each lane stores 16
// contiguous bytes. Lane l, accumulator e of MFMA tile (i, j) holds row
// 32i + 8(e/4) + 4(l/32) + e%4, column 32j + l%32.
__device__ __forceinline__ void stage_put4(uint16_t *stage, int lane, int i, int j, int e4, float a0, float a1,
                                           float a2, float a3) {
  const int rr = 32 * i + 8 * e4 + 4 * (lane >> 5), cc = 32 * j + (lane & 31);
  stage[rr * kEP + cc] = (uint16_t)(pack_bf16x2(a0, 0.f) & 0xffffu);
  stage[(rr + 1) * kEP + cc] = (uint16_t)(pack_bf16x2(a1, 0.f) & 0xffffu);
  stage[(rr + 2) * kEP + cc] = (uint16_t)(pack_bf16x2(a2, 0.f) & 0xffffu);
  stage[(rr + 3) * kEP + cc] = (uint16_t)(pack_bf16x2(a3, 0.f) & 0xffffu);
}
__device__ __forceinline__ void stage_acc(const f32x16 (&acc)[8][2], uint16_t *stage, int lane) {
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4)
        stage_put4(stage, lane, i, j, e4, acc[i][j][4 * e4], acc[i][j][4 * e4 + 1], acc[i][j][4 * e4 + 2],
                   acc[i][j][4 * e4 + 3]);
}
// Rows [rlo, rhi) of the staged tile -> `out` (row pitch ld; rows < mlim and
// columns < nlim of the output).
__device__ __forceinline__ void stage_store(const uint16_t *stage, int lane, uint16_t *out, int64_t ld,
                                            int64_t row0, int64_t col0, int64_t mlim, int64_t nlim, int rlo,
                                            int rhi) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  // 256 rows x 8 chunks of 8 bf16: lane takes chunk lane%8 of rows lane/8 + 8q
#pragma unroll 4
  for (int q = 0; q < 32; ++q) {
    const int rr = (lane >> 3) + 8 * q, ch = lane & 7;
    const int64_t m = row0 + rr, n = col0 + 8 * ch;
    if (rr >= rlo && rr < rhi && m < mlim && n < nlim) {
      const u32x4 v = *reinterpret_cast<const u32x4 *>(stage + rr * kEP + 8 * ch);
      if (n + 8 <= nlim) {
        st16(out + m * ld + n, v);
      } else {
        const uint16_t *s16 = reinterpret_cast<const uint16_t *>(&v);
        for (int u = 0; u < 8 && n + u < nlim; ++u) out[m * ld + n + u] = s16[u];
      }
    }
  }
}

// The 64 MFMAs of an adapter K tile (operands from LDS / registers, no overlap).
template <typename BFn>
__device__ __forceinline__ void plain_tile(f32x16 (&acc)[8][2], const uint8_t *atile, const int (&aoff)[4],
                                           BFn bfrag) {
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    u32x4 a[8], b[2];
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = *reinterpret_cast<const u32x4 *>(atile + aoff[s] + 4096 * i);
    bfrag(s, b);
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(a[i], b[j], acc[i][j]);
  }
}

// ---------------------------------------------------------------------------
// Work items and K-split tails
// ---------------------------------------------------------------------------
constexpr int kTileFloats = kBM * kBN;  // one float32 partial tile
constexpr int kMaxSplit = 8;

// Workgroup b < full runs one whole tile; otherwise part (b - full) % split of
// tail tile full + (b - full) / split, over K steps [k0, k1).
//
// Whole tiles are handed out XCD-aware. Consecutive workgroups go to the eight
// XCDs in turn (b % 8), and the workgroups of one XCD run at about the same
// time, each streaming its activation row tile and its weight column tile
// through that XCD's L2. XCD x therefore takes the x-th contiguous share of
// the tiles in an order that walks down kXcdRows row tiles before moving to
// the next column: the 32 tiles it holds at once span 2 row tiles x 16 column
// tiles instead of all 8 row tiles x 4 columns, which cuts what its L2 pulls
// in per step (one activation row tile is four times the bytes of one weight
// column tile). Tiles of an incomplete last row keep the linear order.
constexpr int kXcdRows = 2;
struct WorkItem {
  int tile, part, parts, k0, k1;
  int64_t m0, n0;
};
__device__ __forceinline__ int xcd_tile(int b, int gn, int full) {
  const int x = b & 7, i = b >> 3, q = full >> 3, rem8 = full & 7;
  const int L = x * q + (x < rem8 ? x : rem8) + i;  // a bijection of [0, full)
  const int rows = full / gn;                        // complete rows among the whole tiles
  if (L >= rows * gn) return L;
  const int g = L / (kXcdRows * gn), ha = rows - g * kXcdRows < kXcdRows ? rows - g * kXcdRows : kXcdRows;
  const int idx = L - g * kXcdRows * gn;
  return (g * kXcdRows + idx % ha) * gn + idx / ha;
}
__device__ __forceinline__ WorkItem work_item(int gn, int nk, int full, int split) {
  WorkItem w;
  const int b = blockIdx.x;
  if (b < full) {
    w.tile = xcd_tile(b, gn, full);
    w.part = 0;
    w.parts = 1;
    w.k0 = 0;
    w.k1 = nk;
  } else {
    const int p = b - full;
    w.tile = full + p / split;
    w.part = p % split;
    w.parts = split;
    w.k0 = w.part * nk / split;
    w.k1 = (w.part + 1) * nk / split;
  }
  w.m0 = (int64_t)(w.tile / gn) * kBM;
  w.n0 = (int64_t)(w.tile % gn) * kBN;
  return w;
}

// End of a K part of a tail tile (the combine protocol of split_arrive in
// common.h). Every part stores its float32 tile with device-scope stores and
// arrives; share p of the tile is row tiles [8p/parts, 8(p+1)/parts), summed
// over all parts in part order by whichever workgroup claims it, staged as
// bf16 and handed to store_rows(rlo, rhi). Wave w's accumulators sit at floats
// [16384 w, 16384 (w+1)) of a part's tile as 64 chunks of 1 KB, lane-major;
// each wave sums and stores its own 64 columns. No part depends on another
// part being dispatched: one that stops waiting leaves its share to the last
// arriver.
template <typename StoreRows>
__device__ __forceinline__ void split_combine(const f32x16 (&acc)[8][2], float *tile_parts, int part, int parts,
                                              uint32_t *line, uint32_t *fallbacks, uint16_t *stage, int tid,
                                              int wave, int lane, StoreRows store_rows) {
  __shared__ uint32_t claim_lds[2];
  const rsrc_t pr = make_rsrc(tile_parts, (int64_t)parts * kTileFloats * 4);
  const uint32_t lane_off = (uint32_t)(wave * (kTileFloats / 4) + 4 * lane) * 4u;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const u32x4 v = {__float_as_uint(acc[i][j][4 * e4]), __float_as_uint(acc[i][j][4 * e4 + 1]),
                         __float_as_uint(acc[i][j][4 * e4 + 2]), __float_as_uint(acc[i][j][4 * e4 + 3])};
        const uint32_t off = (uint32_t)(part * kTileFloats) * 4u + lane_off + (uint32_t)((i * 2 + j) * 4 + e4) * 1024u;
        __builtin_amdgcn_raw_buffer_store_b128(v, pr, off, 0, 16);
      }
  wait_barrier<0>();  // every wave's stores have completed
  if (tid == 0) {
    bool last;
    claim_lds[0] = split_arrive(line, part, parts, last, fallbacks);
    claim_lds[1] = last ? 1u : 0u;
  }
  wait_barrier<0>();
  auto sum_shares = [&](uint32_t mask) {
    for (int sh = 0; sh < parts; ++sh) {
      if (!((mask >> sh) & 1u)) continue;
      const int ilo = sh * 8 / parts, ihi = (sh + 1) * 8 / parts;
      for (int i = ilo; i < ihi; ++i) {
        f32x4 sum[2][4];
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int e4 = 0; e4 < 4; ++e4) sum[j][e4] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int p = 0; p < parts; ++p) {
          u32x4 v[2][4];
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4)
              v[j][e4] = bld16_dev(pr, (uint32_t)(p * kTileFloats) * 4u + lane_off + (uint32_t)((i * 2 + j) * 4 + e4) * 1024u);
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4)
#pragma unroll
              for (int u = 0; u < 4; ++u) sum[j][e4][u] += __uint_as_float(v[j][e4][u]);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int e4 = 0; e4 < 4; ++e4)
            stage_put4(stage, lane, i, j, e4, sum[j][e4][0], sum[j][e4][1], sum[j][e4][2], sum[j][e4][3]);
      }
      store_rows(32 * ilo, 32 * ihi);
    }
  };
  const uint32_t mine = claim_lds[0];
  const bool last = claim_lds[1] != 0u;
  sum_shares(mine);
  if (last) {
    wait_barrier<0>();  // every wave has read the claim words
    if (wave == 0) {
      const uint32_t m = split_sweep(line, part, parts, lane);
      if (lane == 0) claim_lds[0] = m;
    }
    wait_barrier<0>();
    sum_shares(claim_lds[0]);
  }
  if (tid == 0) split_depart(line, parts);
}

// ---------------------------------------------------------------------------
// Forward
// ---------------------------------------------------------------------------
// Codes of one K step held by one lane: for each of its two output rows
// (column tiles j = 0, 1) the four code words of its K half; and the scale
// code and group maximum of the block of row j = l / 32 only. Lanes l and
// l + 32 hold the same two rows, so each builds one of the two restore tables
// and v_permlane32_swap gives both lanes both (see share_tables).
struct FwdCodes {
  u32x4 c[2];
  uint32_t q2;
  float S;
};

// Table words of row j = l / 32 in every lane -> t[0] (row j = 0) and t[1]
// (row j = 1) in every lane: the swap hands lanes 0..31 the words of lanes
// 32..63 in its second result and lanes 32..63 those of lanes 0..31 in its
// first. Words k0 .. k0 + 3 of the eight (lo[0..3], hi[0..3]).
__device__ __forceinline__ void share_tables(const Nf4Planes &own, Nf4Planes (&t)[2], int k0) {
#pragma unroll
  for (int k = k0; k < k0 + 4; ++k) {
    const uint32_t w = k < 4 ? own.lo[k] : own.hi[k - 4];
    const auto sw = __builtin_amdgcn_permlane32_swap(w, w, false, false);
    uint32_t a = sw[0], b = sw[1];
    pin(a);
    pin(b);
    if (k < 4) {
      t[0].lo[k] = a;
      t[1].lo[k] = b;
    } else {
      t[0].hi[k - 4] = a;
      t[1].hi[k - 4] = b;
    }
  }
}

__global__ __launch_bounds__(kThreads) void k_gemm_fwd(const uint8_t *__restrict__ codes,
                                                       const uint8_t *__restrict__ qscale,
                                                       const float *__restrict__ smax, int64_t d_out, int64_t d_in,
                                                       const uint16_t *__restrict__ x, int64_t T,
                                                       const uint16_t *__restrict__ su, int r_pad,
                                                       const uint16_t *__restrict__ B, int r,
                                                       uint16_t *__restrict__ h, float *__restrict__ partial,
                                                       uint32_t *__restrict__ counters, int gn, int full,
                                                       int split, int sshift) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];  // [2][kTile] activation ring
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int half = lane >> 5, ml = lane & 31;
  const int64_t KB = d_in / kBlock;
  const int nk = (int)KB;
  const WorkItem wi = work_item(gn, nk, full, split);
  const int64_t m0 = wi.m0, n0 = wi.n0;
  const int k0 = wi.k0, k1 = wi.k1;
  const int nk_lora = r > 0 && wi.part == wi.parts - 1 ? (r_pad + kBK - 1) / kBK : 0;

  // Buffer ranges of this tile (rows past T / d_out read zeros).
  const int64_t mrows = T - m0 < kBM ? T - m0 : kBM;
  const int64_t nrows = d_out - n0 < kBN ? d_out - n0 : kBN;
  const rsrc_t xr = make_rsrc(x + m0 * d_in, mrows * d_in * 2);
  const rsrc_t cr = make_rsrc(codes + n0 * (d_in / 2), nrows * (d_in / 2));
  // absmax-only storage (sshift 0): an empty q2 range (loads return 0) and one scale per block
  const rsrc_t qr = make_rsrc(qscale + n0 * KB, sshift ? nrows * KB : 0);
  const rsrc_t sr = make_rsrc(smax, scale_words(d_out * KB, sshift) * 4);
  const uint32_t q2o = q2_or(sshift);

  int aoff[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) aoff[s] = a_off(lane, s);
  const DmaOffs xo = dma_offsets((int)d_in, wave, lane);

  // This lane's output rows (column tiles j = 0, 1) within the tile: byte
  // offsets of their code rows; the scale-code row and first block index of
  // row j = l / 32.
  uint32_t coff[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) coff[j] = (uint32_t)((kWN * wave + 32 * j + ml) * (d_in / 2)) + 16u * half;
  const int trow = kWN * wave + 32 * half + ml;
  const uint32_t qoff = (uint32_t)(trow * KB), blk0 = (uint32_t)((n0 + trow) * KB);
  auto issue_codes = [&](int kt, FwdCodes &C) {
    const int kc = kt < nk ? kt : nk - 1;  // steps past the end reload the last one (never used)
#pragma unroll
    for (int j = 0; j < 2; ++j) C.c[j] = bld16s(cr, coff[j], kc * (kBlock / 2));
    C.q2 = bld8s(qr, qoff, kc);
    C.S = __uint_as_float(bld32(sr, ((blk0 + (uint32_t)kc) >> sshift) * 4u));
  };

  f32x16 acc[8][2];
  zero_acc(acc);
  FwdCodes C0, C1;
  Nf4Planes t[2];
  u32x4 fa[2][8], fb[2][2];

  // Prologue: tile 0 in LDS, codes of steps 0 and 1 requested, tables and
  // fragments of step 0, slice 0 ready.
  dma_tile(xr, xo, k0 * kBK, smem, wave);
  issue_codes(k0, C0);
  issue_codes(k0 + 1, C1);
  wait_barrier<4>();
  {
    TableBuild tb;
    Nf4Planes own;
#pragma unroll
    for (int k = 0; k < 3; ++k) tb.run(k, C0.q2, q2o, C0.S, own);
    share_tables(own, t, 0);
    share_tables(own, t, 4);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) fb[0][j] = expand8(t[j], C0.c[j][0]);
#pragma unroll
  for (int i = 0; i < 8; ++i) fa[0][i] = *reinterpret_cast<const u32x4 *>(smem + aoff[0] + 4096 * i);

  // One K step. Tile kt is in ring slot P = kt & 1, its codes in Ccur; Cnext
  // holds the codes of step kt+1. Side work after MFMA q of slice s:
  //   s < 3 : A fragments of slice s+1 (q < 8); B fragments of slice s+1
  //           (one of 8 expand pieces after every MFMA: column tile 0 at
  //           q = 0..7, 1 at 8..15);
  //   s = 3 : codes of step kt+2 into Ccur (q = 0); this lane's table of
  //           step kt+1 (q = 1..3) and the swap that shares it (q = 4, 5);
  //           wait for tile kt+1 and barrier (q = 7); then the A and B
  //           fragments of step kt+1, slice 0 (q = 8..15).
  auto step = [&](int kt, const int P, FwdCodes &Ccur, FwdCodes &Cnext) {
    // (the last step copies its own tile again into the idle slot: no branch)
    dma_tile(xr, xo, (kt + 1 < k1 ? kt + 1 : kt) * kBK, smem + (P ^ 1) * kTile, wave);
    const uint8_t *cur = smem + P * kTile, *nxt = smem + (P ^ 1) * kTile;
    Expand8 ex;
    TableBuild7 tb;
    Nf4Planes own;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int i = q >> 1, j = q & 1;
        acc[i][j] = mfma32(fa[s & 1][i], fb[s & 1][j], acc[i][j]);
        QLORA_SCHED_FENCE();
        if (s < 3) {
          if (q < 8) fa[(s + 1) & 1][q] = *reinterpret_cast<const u32x4 *>(cur + aoff[s + 1] + 4096 * q);
          const int jj = q >> 3;
          ex.run(q & 7, t[jj], Ccur.c[jj][s + 1], fb[(s + 1) & 1][jj]);
        } else {
          if (q == 0) issue_codes(kt + 2, Ccur);
          if (q <= 6) tb.run(q, Cnext.q2, q2o, Cnext.S, own);
          if (q == 6 || q == 7) share_tables(own, t, 4 * (q - 6));
          if (q == 7) wait_barrier<4>();
          if (q >= 8) {
            fa[0][q - 8] = *reinterpret_cast<const u32x4 *>(nxt + aoff[0] + 4096 * (q - 8));
            const int jj = (q - 8) >> 2, ph = 2 * ((q - 8) & 3);
            ex.run(ph, t[jj], Cnext.c[jj][0], fb[0][jj]);
            ex.run(ph + 1, t[jj], Cnext.c[jj][0], fb[0][jj]);
          }
        }
        QLORA_SCHED_FENCE();
      }
    }
  };

  // Two steps per iteration (the register sets trade roles), no branch between them.
  int kt = k0;
  for (; kt + 1 < k1; kt += 2) {
    step(kt, 0, C0, C1);
    step(kt + 1, 1, C1, C0);
  }
  if (kt < k1) step(kt, 0, C0, C1);

  // Adapter K tile(s) (with the last K part of a split tile): su [T, r_pad] through LDS; B [d_out, r] fragments
  // straight from memory (lane: row of its column tile, K 32h + 8s .. +7).
  const rsrc_t ur = make_rsrc(su + m0 * r_pad, mrows * r_pad * 2);
  const rsrc_t br = make_rsrc(B + n0 * r, nrows * r * 2);
  for (int lt = 0; lt < nk_lora; ++lt) {
    const int j0 = lt * kBK;
    wait_barrier<0>();  // every wave is done with the ring
    dma_any(ur, dma_offsets(r_pad, wave, lane), j0, r_pad, smem, wave, lane);
    wait_barrier<0>();
    plain_tile(acc, smem, aoff, [&](int s, u32x4 (&b)[2]) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int row = kWN * wave + 32 * j + ml, col = j0 + 32 * half + 8 * s;
        b[j] = bld16(br, col < r ? (uint32_t)((row * r + col) * 2) : kOOB);
      }
    });
  }

  // Epilogue through LDS once every wave is done with the ring.
  wait_barrier<0>();
  uint16_t *stage = reinterpret_cast<uint16_t *>(smem) + wave * kBM * kEP;
  if (wi.parts > 1) {
    split_combine(acc, partial + (size_t)(wi.tile - full) * split * kTileFloats, wi.part, wi.parts,
                  tile_counter(counters, wi.tile - full), counters + kMaxCounters - 1, stage, tid, wave, lane,
                  [&](int rlo, int rhi) { stage_store(stage, lane, h, d_out, m0, n0 + kWN * wave, T, d_out, rlo, rhi); });
  } else {
    stage_acc(acc, stage, lane);
    stage_store(stage, lane, h, d_out, m0, n0 + kWN * wave, T, d_out, 0, kBM);
  }
}

// ---------------------------------------------------------------------------
// Backward dX
// ---------------------------------------------------------------------------
// Codes of one weight block (one lane's share of a 64 x 256 weight tile).
struct DxCodes {
  u32x4 c0, c1;
  uint32_t q2;
  float S;
};

// Restore of one block into a weight tile in 3 + 32 pieces: table, then per
// code word the four expand pieces, the last of which stores the 8 weights.
// Word m of the block goes to byte (wxor ^ 16 m) of the tile: the block's
// chunks are 8 consecutive positions whose order the swizzle permutes.
struct DxRestore {
  // 7 table pieces, then 6 pieces per code word (the selectors in two, the
  // low and high lookups of e0..e3 one each, those of e4..e7 together, the
  // interleave with the store), one per slot: after each MFMA of slices 0..2
  // and of slice 3 before its barrier.
  static constexpr int kPieces = 7 + 8 * 6;
  TableBuild7 tb;
  Nf4Planes t;
  uint32_t w, sa, ma, sb, mb, lo_a, hi_a, lo_b, hi_b;  // w: the word as pinned in its piece 0
  __device__ __forceinline__ void run(int k, const DxCodes &C, uint8_t *tile, uint32_t wxor, uint32_t q2o) {
    if (k < 7) {
      tb.run(k, C.q2, q2o, C.S, t);
      return;
    }
    if (k >= kPieces) return;
    const int m = (k - 7) / 6, ph = (k - 7) % 6;
    if (ph == 0) {
      w = m < 4 ? C.c0[m & 3] : C.c1[m & 3];
      pin(w);
      sa = w & 0x07070707u;
      ma = ((w >> 1) & 0x04040404u) | 0x03020100u;
      pin(sa);
      pin(ma);
    } else if (ph == 1) {
      sb = (w >> 4) & 0x07070707u;
      mb = ((w >> 5) & 0x04040404u) | 0x03020100u;
      pin(sb);
      pin(mb);
    } else if (ph == 2) {
      lo_a = lookup4(t.lo, sa, ma);
      pin(lo_a);
    } else if (ph == 3) {
      hi_a = lookup4(t.hi, sa, ma);
      pin(hi_a);
    } else if (ph == 4) {
      lo_b = lookup4(t.lo, sb, mb);
      hi_b = lookup4(t.hi, sb, mb);
      pin(lo_b);
      pin(hi_b);
    } else {
      u32x4 v;
      v[0] = perm(hi_a, lo_a, 0x05010400u);
      v[1] = perm(hi_a, lo_a, 0x07030602u);
      v[2] = perm(hi_b, lo_b, 0x05010400u);
      v[3] = perm(hi_b, lo_b, 0x07030602u);
      st16(tile + (wxor ^ (16u * m)), v);
    }
  }
};

__global__ __launch_bounds__(kThreads) void k_gemm_dx(const uint8_t *__restrict__ codes,
                                                      const uint8_t *__restrict__ qscale,
                                                      const float *__restrict__ smax, int64_t d_out, int64_t d_in,
                                                      const uint16_t *__restrict__ dY, int64_t T,
                                                      const uint16_t *__restrict__ sv, int r_pad,
                                                      const uint16_t *__restrict__ A, int r,
                                                      uint16_t *__restrict__ dX, float *__restrict__ partial,
                                                      uint32_t *__restrict__ counters, int gn, int full,
                                                      int split, int sshift) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint8_t *ring = smem;                                             // [2][kTile]     dY tiles [t][o]
  uint8_t *Bt = smem + 2 * kTile;                                   // [2][kWTile]    W_hat tiles [o][i]
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int64_t KB = d_in / kBlock;
  const int nk = (int)((d_out + kBK - 1) / kBK);
  const WorkItem wi = work_item(gn, nk, full, split);
  const int64_t m0 = wi.m0, n0 = wi.n0;  // n = input feature i
  const int k0 = wi.k0, k1 = wi.k1;
  const int nk_lora = r > 0 && wi.part == wi.parts - 1 ? (r_pad + kBK - 1) / kBK : 0;

  const int64_t mrows = T - m0 < kBM ? T - m0 : kBM;
  const i32x4 yr = rsrc_words(dY + m0 * d_out, mrows * d_out * 2);
  const DmaOffs yo = dma_offsets((int)d_out, wave, lane);

  int aoff[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) aoff[s] = a_off(lane, s);
  // B fragment of column tile j, slice s from a weight tile: lane gets column
  // 64w + 32j + l%32, K rows 32h + 8s .. +7. Within each 16 lanes
  // ds_read_b64_tr_b16 hands lane u element e of the 8 bytes that lane
  // 4e + u/4 addresses (its 16-bit element u%4); lane u of group g therefore
  // addresses K row 32(g/2) + 8s + u/4, columns 16(g%2) + 4(u%4) .. +3, and a
  // second read four rows further down gives elements 4..7. Row o mod 8 does
  // not depend on s, so the swizzled byte offsets (per j, per half) are fixed
  // per lane and slices add 4096 s.
  const int grp = lane >> 4, u16 = lane & 15;
  uint32_t boff[2][2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int row = 32 * (grp >> 1) + (u16 >> 2) + 4 * hh;
      const int col = kWN * wave + 32 * j + 16 * (grp & 1) + 4 * (u16 & 3);
      boff[j][hh] = (uint32_t)(row * kWRow + (((col >> 3) ^ wswz(row)) << 4) + (col & 7) * 2);
    }
  auto frag_b = [&](const uint8_t *bt, int s, int j) {
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(bt + boff[j][0] + 4096 * s));
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(bt + boff[j][1] + 4096 * s));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
    return u32x4{l2[0], l2[1], h2[0], h2[1]};
  };

  // weight tile: 64 rows o x 4 blocks of 64 columns i; lanes 16G + u take row
  // 8 (G % 8) + u % 8, block 2 (G / 8) + u / 8 (8 rows x 2 blocks per 16 lanes)
  const int wo = 8 * ((tid >> 4) & 7) + (tid & 7), wb = 2 * (tid >> 7) + ((tid >> 3) & 1);
  const uint32_t wxor = (uint32_t)(wo * kWRow + ((8 * wb ^ wswz(wo)) << 4));
  const int64_t kblk = n0 / kBlock + wb;
  const uint32_t q2o = q2_or(sshift);
  auto issue_codes = [&](int kt, DxCodes &C) {
    // weight rows k0..k0+63: ranges rebased per K tile (32-bit offsets stay small for any weight size)
    const int64_t k0 = (int64_t)kt * kBK;
    const int64_t orows = kt < nk ? (d_out - k0 < kBK ? d_out - k0 : kBK) : 0;
    const int64_t kr = kt < nk ? k0 : 0;
    const rsrc_t crr = make_rsrc(codes + kr * (d_in / 2), orows * (d_in / 2));
    const rsrc_t qrr = make_rsrc(qscale + kr * KB, sshift ? orows * KB : 0);
    const int64_t gb = (kr * KB) >> sshift;  // first scale word of the tile's rows
    const rsrc_t srr = make_rsrc(smax + gb, (scale_words(d_out * KB, sshift) - gb) * 4);
    // Rows past the tile's end fall outside the ranges and restore to zero
    // (scale code 0). Blocks past d_in (kblk >= KB) read the next row's
    // blocks: finite values that reach only output columns past d_in, which
    // are never stored.
    const uint32_t lblk = (uint32_t)(wo * KB + kblk);  // block index within the tile
    C.c0 = bld16(crr, lblk * 32u);
    C.c1 = bld16(crr, lblk * 32u + 16u);
    C.q2 = bld8(qrr, lblk);
    C.S = __uint_as_float(bld32(srr, (uint32_t)((((kr * KB) & ((1 << sshift) - 1)) + lblk) >> sshift) * 4u));
  };

  f32x16 acc[8][2];
  zero_acc(acc);
  DxCodes C0, C1;
  u32x4 fa[2][8], fb[2][2];

  // Prologue: dY tile 0 and weight tile 0 in LDS, codes of step 1 requested,
  // fragments of step 0, slice 0 ready.
  dma_tile_asm(yr, yo, k0 * kBK, (int)d_out, ring, wave, lane);
  issue_codes(k0, C0);
  issue_codes(k0 + 1, C1);
  {
    DxRestore rs;
#pragma unroll
    for (int k = 0; k < DxRestore::kPieces; ++k) rs.run(k, C0, Bt, wxor, q2o);
  }
  wait_barrier<4>();
#pragma unroll
  for (int i = 0; i < 8; ++i) fa[0][i] = *reinterpret_cast<const u32x4 *>(ring + aoff[0] + 4096 * i);
#pragma unroll
  for (int j = 0; j < 2; ++j) fb[0][j] = frag_b(Bt, 0, j);

  // One K step. Tiles of step kt are in slot P; Cnext holds the codes of step
  // kt+1, whose weight tile is restored into slot P^1 during this step; Ccur
  // (dead) receives the codes of step kt+2. Side work after MFMA q of slice s:
  //   s < 3 : A fragments of slice s+1 (q < 8), B fragments (q = 8, 10);
  //           restore piece 16s + q (55 pieces: slices 0..2 and slice 3 up to q = 6);
  //   s = 3 : restore pieces 48 + q (q < 7); wait for the copies and stores
  //           of step kt+1 and barrier (q = 7);
  //           A and B fragments of step kt+1, slice 0 (q = 8..15).
  auto step = [&](int kt, const int P, DxCodes &Ccur, DxCodes &Cnext) {
    wait_vmem();  // codes of step kt+1 (requested a step ago) are in; see dma16_asm
    dma_tile_asm(yr, yo, (kt + 1 < k1 ? kt + 1 : kt) * kBK, (int)d_out, ring + (P ^ 1) * kTile, wave, lane);
    issue_codes(kt + 2, Ccur);
    const uint8_t *cur = ring + P * kTile, *nxt = ring + (P ^ 1) * kTile;
    const uint8_t *bcur = Bt + P * kWTile;
    uint8_t *bnxt = Bt + (P ^ 1) * kWTile;
    DxRestore rs;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int i = q >> 1, j = q & 1;
        acc[i][j] = mfma32(fa[s & 1][i], fb[s & 1][j], acc[i][j]);
        QLORA_SCHED_FENCE();
        if (s < 3) {
          if (q < 8) fa[(s + 1) & 1][q] = *reinterpret_cast<const u32x4 *>(cur + aoff[s + 1] + 4096 * q);
          if (q == 8 || q == 10) fb[(s + 1) & 1][(q - 8) >> 1] = frag_b(bcur, s + 1, (q - 8) >> 1);
          rs.run(16 * s + q, Cnext, bnxt, wxor, q2o);
        } else {
          if (q < 7) rs.run(48 + q, Cnext, bnxt, wxor, q2o);
          if (q == 7) wait_barrier<4>();
          if (q >= 8) fa[0][q - 8] = *reinterpret_cast<const u32x4 *>(nxt + aoff[0] + 4096 * (q - 8));
          if (q == 12 || q == 14) fb[0][(q - 12) >> 1] = frag_b(bnxt, 0, (q - 12) >> 1);
        }
        QLORA_SCHED_FENCE();
      }
    }
  };

  // Two steps per iteration (the register sets trade roles), no branch between them.
  int kt = k0;
  for (; kt + 1 < k1; kt += 2) {
    step(kt, 0, C0, C1);
    step(kt + 1, 1, C1, C0);
  }
  if (kt < k1) step(kt, 0, C0, C1);

  const rsrc_t ar = make_rsrc(A, (int64_t)r * d_in * 2);
  for (int lt = 0; lt < nk_lora; ++lt) {
    const int j0 = lt * kBK;
    wait_barrier<0>();  // every wave is done with the ring and the weight tiles
    dma_tile_asm(rsrc_words(sv + m0 * r_pad, mrows * r_pad * 2), dma_offsets(r_pad, wave, lane), j0, r_pad, ring,
                 wave, lane);
    // A rows j0..j0+63, columns n0..n0+255 -> weight tile slot 0
#pragma unroll
    for (int q = 0; q < kBK * (kBN / 8) / kThreads; ++q) {
      const int e = q * kThreads + tid;
      const int jr = e / (kBN / 8), cc = (e % (kBN / 8)) * 8;
      const int64_t jj = j0 + jr, ii = n0 + cc;
      const uint32_t off = (jj < r && ii < d_in) ? (uint32_t)((jj * d_in + ii) * 2) : kOOB;
      st16(Bt + jr * kWRow + ((((cc >> 3) ^ wswz(jr))) << 4), bld16(ar, off));
    }
    wait_barrier<0>();
    plain_tile(acc, ring, aoff, [&](int s, u32x4 (&b)[2]) {
      b[0] = frag_b(Bt, s, 0);
      b[1] = frag_b(Bt, s, 1);
    });
  }

  wait_barrier<0>();
  uint16_t *stage = reinterpret_cast<uint16_t *>(smem) + wave * kBM * kEP;
  if (wi.parts > 1) {
    split_combine(acc, partial + (size_t)(wi.tile - full) * split * kTileFloats, wi.part, wi.parts,
                  tile_counter(counters, wi.tile - full), counters + kMaxCounters - 1, stage, tid, wave, lane,
                  [&](int rlo, int rhi) { stage_store(stage, lane, dX, d_in, m0, n0 + kWN * wave, T, d_in, rlo, rhi); });
  } else {
    stage_acc(acc, stage, lane);
    stage_store(stage, lane, dX, d_in, m0, n0 + kWN * wave, T, d_in, 0, kBM);
  }
}

static hipError_t set_lds_attrs() {
  static DeviceOnce once;
  return once.run(current_device(), [] {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(k_gemm_fwd),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kFwdLds);
    if (e != hipSuccess) return e;
    return hipFuncSetAttribute(reinterpret_cast<const void *>(k_gemm_dx),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)kDxLds);
  });
}

// Choose the K split of the tail tiles by a step count: whole tiles take nk
// steps per round of `cus` tiles; a round of parts takes ceil(nk/s) steps plus
// a fixed cost (prologue and epilogue of a short K range, storing a float32
// partial tile, waiting for the other parts and reading back a 1/s share of
// all of them), measured at about 24 steps.
GemmPlan gemm_plan(int64_t M, int64_t N, int64_t nk) {
  GemmPlan p{};
  p.gm = (int)((M + kBM - 1) / kBM);
  p.gn = (int)((N + kBN - 1) / kBN);
  p.nk = (int)nk;
  const int64_t tiles = (int64_t)p.gm * p.gn, cus = device_cu_count(current_device());
  const int64_t rounds = tiles / cus, rem = tiles % cus;
  int best = 1;
  int64_t best_cost = rounds * nk + (rem > 0 ? nk : 0);
  for (int s = 2; s <= kMaxSplit && s <= nk && rem > 0 && rem <= kMaxTileCounters; ++s) {
    // Cost in K steps of one tile. When the split tail shares rounds with other
    // work, each round pays for moving its partials through memory (24 steps
    // measured at the 13B/65B shapes). When the whole launch is one round of
    // split tiles, the combine is one tile's store and re-read per part, about
    // three steps.
    const int64_t cost = (rounds == 0 && rem * s <= cus)
                             ? (nk + s - 1) / s + 3
                             : rounds * nk + (rem * s + cus - 1) / cus * ((nk + s - 1) / s + 24);
    if (cost < best_cost) {
      best_cost = cost;
      best = s;
    }
  }
  p.split = best;
  p.rem = best > 1 ? (int)rem : 0;
  p.full = (int)(tiles - p.rem);
  return p;
}

size_t gemm_partial_floats(const GemmPlan &p) { return (size_t)p.rem * p.split * kTileFloats; }

hipError_t launch_gemm_fwd(const uint8_t *codes, const uint8_t *qscale, const float *smax, int64_t d_out,
                           int64_t d_in, const uint16_t *x, int64_t T, const uint16_t *su, int r_pad,
                           const uint16_t *B, int r, uint16_t *h, float *partial, uint32_t *counters,
                           hipStream_t st) {
  hipError_t e = set_lds_attrs();
  if (e != hipSuccess) return e;
  const GemmPlan p = gemm_plan(T, d_out, d_in / kBlock);
  if (p.rem > kMaxTileCounters) return hipErrorInvalidValue;
  const unsigned grid = (unsigned)(p.full + p.rem * p.split);
  // absmax-only storage: no scale codes (the kernel's q2 range is then empty)
  k_gemm_fwd<<<dim3(grid), dim3(kThreads), kFwdLds, st>>>(codes, qscale ? qscale : codes, smax, d_out, d_in, x, T, su,
                                                            r_pad, B, r, h, partial, counters, p.gn, p.full, p.split,
                                                            qscale ? kDqShift : 0);
  return hipGetLastError();
}

hipError_t launch_gemm_dx(const uint8_t *codes, const uint8_t *qscale, const float *smax, int64_t d_out,
                          int64_t d_in, const uint16_t *dY, int64_t T, const uint16_t *sv, int r_pad,
                          const uint16_t *A, int r, uint16_t *dX, float *partial, uint32_t *counters,
                          hipStream_t st) {
  hipError_t e = set_lds_attrs();
  if (e != hipSuccess) return e;
  const GemmPlan p = gemm_plan(T, d_in, (d_out + kBK - 1) / kBK);
  if (p.rem > kMaxTileCounters) return hipErrorInvalidValue;
  const unsigned grid = (unsigned)(p.full + p.rem * p.split);
  k_gemm_dx<<<dim3(grid), dim3(kThreads), kDxLds, st>>>(codes, qscale ? qscale : codes, smax, d_out, d_in, dY, T, sv,
                                                          r_pad, A, r, dX, partial, counters, p.gn, p.full, p.split,
                                                          qscale ? kDqShift : 0);
  return hipGetLastError();
}

}  // namespace qlora
