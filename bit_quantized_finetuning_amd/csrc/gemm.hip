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
// Tiling: a 256-thread workgroup computes a 256 x 256 output tile; its four
// waves each own 128 x 128 (4 x 4 v_mfma_f32_32x32x16_bf16 tiles, 256 fp32
// accumulators per lane, one wave per SIMD). K advances 64 at a time:
//   * global loads run two tiles ahead (two register sets in turn), so a tile's
//     codes and activations have a whole K step to arrive;
//   * LDS is double-buffered: while the MFMAs consume tile k, the same wave
//     restores tile k+1 (one 64-weight block per thread, one table per block)
//     into the other buffer. The restore is cut into pieces of a few VALU
//     instructions, one after each MFMA, with scheduling fences that keep the
//     order: each piece issues while the matrix core works on the MFMA before
//     it, so the restore runs in the shadow of the matrix cores;
//   * loop bodies are straight-line: tiles past the end load zeros (out-of-range
//     buffer offsets) and add nothing.
// Forward: W's K (= d_in) runs along a block, so a thread restores one whole
// block of one output row and the MFMA B operand is read straight from LDS.
// dX: K = d_out runs across blocks; the restored tile is stored [o][i] as
// restored and the B fragments (8 consecutive o for one i per lane) come from
// two ds_read_b64_tr_b16, which transpose 16-bit data across each 16 lanes.
// The epilogue goes through LDS so that every lane writes 16-byte rows.
#include "kernels.h"

namespace qlora {

constexpr int kBM = 256, kBN = 256, kBK = 64;
constexpr int kAP = kBK + 8;   // padded pitch (bf16) of [row][k] tiles: fragment reads free of bank conflicts
constexpr int kBTP = kBN + 16; // pitch of the dX [k][n] weight tile: the four rows of a transposed read 8 banks apart
constexpr int kEP = 128 + 8;   // epilogue staging pitch (bf16) of a wave's 128 x 128 tile

typedef short v4i16 __attribute__((ext_vector_type(4)));

// One wave's 128 x 128 fp32 tile -> bf16 rows of `out` (row pitch ld, rows < mlim,
// columns < nlim), staged through this wave's LDS region so that each lane
// stores 16 contiguous bytes. Lane l, accumulator e of tile (i, j) holds row
// 32i + 8(e/4) + 4(l/32) + e%4, column 32j + l%32.
__device__ __forceinline__ void store_tile_bf16(const f32x16 (&acc)[4][4], uint16_t *stage, int lane,
                                                uint16_t *out, int64_t ld, int64_t row0, int64_t col0,
                                                int64_t mlim, int64_t nlim) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int rr = 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3), cc = 32 * j + (lane & 31);
        stage[rr * kEP + cc] = (uint16_t)(pack_bf16x2(acc[i][j][e], 0.f) & 0xffffu);
      }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  // 128 rows x 16 chunks of 8 bf16: lane takes chunk lane%16 of rows lane/16 + 4q
#pragma unroll 4
  for (int q = 0; q < 32; ++q) {
    const int rr = (lane >> 4) + 4 * q, ch = lane & 15;
    const int64_t m = row0 + rr, n = col0 + 8 * ch;
    if (m < mlim && n < nlim) {
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

// Restore of one 64-weight block cut into 39 pieces of a few VALU instructions
// each, so that one piece can follow each MFMA of a K step: the piece issues
// while the matrix core works on that MFMA. piece(0..3): scale and table
// products; piece(4): byte planes; pieces 5 + 4m + 0..3: word m's selectors,
// low-nibble lookups, high-nibble lookups, interleave and LDS store; pieces
// 37, 38: the activation rows' LDS stores.
struct PieceRestore {
  float sh;
  uint32_t p[8];
  Nf4Planes t;
  uint32_t sa, ma, sb, mb, lo_a, hi_a, lo_b, hi_b;
  __device__ __forceinline__ void run(int k, uint32_t q2, float S, const u32x4 &c0, const u32x4 &c1, uint16_t *wdst,
                                      const u32x4 (&act)[8], uint16_t *const (&adst)[8]) {
    if (k < 4) {
      if (k == 0) sh = restore_scale(q2, S);
      p[2 * k] = pack_bf16x2(code_times(4 * k, sh), code_times(4 * k + 1, sh));
      p[2 * k + 1] = pack_bf16x2(code_times(4 * k + 2, sh), code_times(4 * k + 3, sh));
    } else if (k == 4) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        t.lo[j] = perm(p[2 * j + 1], p[2 * j], 0x06040200u);
        t.hi[j] = perm(p[2 * j + 1], p[2 * j], 0x07050301u);
      }
    } else if (k < 37) {
      const int m = (k - 5) >> 2, ph = (k - 5) & 3;
      const uint32_t c = m < 4 ? c0[m & 3] : c1[m & 3];
      if (ph == 0) {
        sa = c & 0x07070707u;
        ma = ((c >> 1) & 0x04040404u) | 0x03020100u;
        sb = (c >> 4) & 0x07070707u;
        mb = ((c >> 5) & 0x04040404u) | 0x03020100u;
      } else if (ph == 1) {
        lo_a = lookup4(t.lo, sa, ma);
        hi_a = lookup4(t.hi, sa, ma);
      } else if (ph == 2) {
        lo_b = lookup4(t.lo, sb, mb);
        hi_b = lookup4(t.hi, sb, mb);
      } else {
        u32x4 r;
        r[0] = perm(hi_a, lo_a, 0x05010400u);
        r[1] = perm(hi_a, lo_a, 0x07030602u);
        r[2] = perm(hi_b, lo_b, 0x05010400u);
        r[3] = perm(hi_b, lo_b, 0x07030602u);
        st16(wdst + 8 * m, r);
      }
    } else if (k < 39) {
      const int i0 = 4 * (k - 37);
#pragma unroll
      for (int i = 0; i < 4; ++i) st16(adst[i0 + i], act[i0 + i]);
    }
  }
};
#define QLORA_SCHED_FENCE() __builtin_amdgcn_sched_barrier(0)

// ---------------------------------------------------------------------------
// Forward
// ---------------------------------------------------------------------------
constexpr size_t kFwdLds = (size_t)2 * (kBM + kBN) * kAP * sizeof(uint16_t);

struct FwdRegs {
  u32x4 x[8];    // 8 rows x 8 bf16 of the activation tile
  u32x4 c0, c1;  // one 64-weight block of codes
  uint32_t q2;
  float S;
};

__global__ __launch_bounds__(256) void k_gemm_fwd(const uint8_t *__restrict__ codes,
                                                  const uint8_t *__restrict__ qscale,
                                                  const float *__restrict__ smax, int64_t d_out, int64_t d_in,
                                                  const uint16_t *__restrict__ x, int64_t T,
                                                  const uint16_t *__restrict__ su, int r_pad,
                                                  const uint16_t *__restrict__ B, int r,
                                                  uint16_t *__restrict__ h) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  uint16_t *As = smem;                        // [2][kBM][kAP]
  uint16_t *Bs = smem + 2 * kBM * kAP;        // [2][kBN][kAP]
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wm = wave & 1, wn = wave >> 1;
  const int64_t m0 = (int64_t)blockIdx.y * kBM, n0 = (int64_t)blockIdx.x * kBN;
  const int64_t KB = d_in / kBlock;
  const int nk = (int)KB;
  const int nk_lora = r > 0 ? (r_pad + kBK - 1) / kBK : 0;

  // Buffer ranges of this tile (rows past T / d_out read zeros).
  const int64_t mrows = T - m0 < kBM ? T - m0 : kBM;
  const int64_t nrows = d_out - n0 < kBN ? d_out - n0 : kBN;
  const rsrc_t xr = make_rsrc(x + m0 * d_in, mrows * d_in * 2);
  const rsrc_t cr = make_rsrc(codes + n0 * (d_in / 2), nrows * (d_in / 2));
  const rsrc_t qr = make_rsrc(qscale + n0 * KB, nrows * KB);
  const rsrc_t sr = make_rsrc(smax, ((d_out * KB + kGroup - 1) / kGroup) * 4);

  // x tile loader: 8 threads per row, 32 rows apart per step
  const int xr_ = tid >> 3, xc = (tid & 7) * 8;

  auto issue = [&](int kt, FwdRegs &R) {
    const bool in = kt < nk;  // tiles past the end read zeros
    const int64_t k0 = (int64_t)kt * kBK;
#pragma unroll
    for (int i = 0; i < 8; ++i) R.x[i] = bld16(xr, in ? (uint32_t)(((xr_ + 32 * i) * d_in + k0 + xc) * 2) : kOOB);
    const uint32_t coff = in ? (uint32_t)(tid * (d_in / 2) + (int64_t)kt * (kBlock / 2)) : kOOB;
    R.c0 = bld16(cr, coff);
    R.c1 = bld16(cr, in ? coff + 16 : kOOB);
    R.q2 = bld8(qr, in ? (uint32_t)(tid * KB + kt) : kOOB);
    R.S = __uint_as_float(bld32(sr, in ? (uint32_t)((((n0 + tid) * KB + kt) >> 8) * 4) : kOOB));
  };
  auto restore = [&](const FwdRegs &R, int buf) {
    uint16_t *as = As + buf * kBM * kAP;
#pragma unroll
    for (int i = 0; i < 8; ++i) st16(as + (xr_ + 32 * i) * kAP + xc, R.x[i]);
    const Nf4Planes t = make_planes(restore_scale(R.q2, R.S));
    uint16_t *bs = Bs + buf * kBN * kAP + tid * kAP;
#pragma unroll
    for (int m = 0; m < 4; ++m) st16(bs + 8 * m, expand8(t, R.c0[m]));
#pragma unroll
    for (int m = 0; m < 4; ++m) st16(bs + 32 + 8 * m, expand8(t, R.c1[m]));
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  auto compute = [&](int buf) {
    const uint16_t *as = As + buf * kBM * kAP + (wm * 128 + (lane & 31)) * kAP + 8 * (lane >> 5);
    const uint16_t *bs = Bs + buf * kBN * kAP + (wn * 128 + (lane & 31)) * kAP + 8 * (lane >> 5);
#pragma unroll
    for (int k16 = 0; k16 < kBK / 16; ++k16) {
      u32x4 a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = *reinterpret_cast<const u32x4 *>(as + i * 32 * kAP + 16 * k16);
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = *reinterpret_cast<const u32x4 *>(bs + j * 32 * kAP + 16 * k16);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma32(a[i], b[j], acc[i][j]);
    }
  };

  // One K step: the 64 MFMAs of LDS buffer `buf`, each followed by one piece
  // of the restore of register set R into buffer buf^1; the fragments of the
  // next 16-wide K slice are read while the current one's MFMAs run.
  auto frags = [&](int buf, int k16, u32x4 (&a)[4], u32x4 (&b)[4]) {
    const uint16_t *as = As + buf * kBM * kAP + (wm * 128 + (lane & 31)) * kAP + 8 * (lane >> 5) + 16 * k16;
    const uint16_t *bs = Bs + buf * kBN * kAP + (wn * 128 + (lane & 31)) * kAP + 8 * (lane >> 5) + 16 * k16;
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = *reinterpret_cast<const u32x4 *>(as + i * 32 * kAP);
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = *reinterpret_cast<const u32x4 *>(bs + j * 32 * kAP);
  };
  auto step = [&](int buf, const FwdRegs &R) {
    uint16_t *wdst = Bs + (buf ^ 1) * kBN * kAP + tid * kAP;
    uint16_t *adst[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) adst[i] = As + (buf ^ 1) * kBM * kAP + (xr_ + 32 * i) * kAP + xc;
    PieceRestore pr;
    u32x4 fa[2][4], fb[2][4];
    frags(buf, 0, fa[0], fb[0]);
#pragma unroll
    for (int k16 = 0; k16 < kBK / 16; ++k16) {
      if (k16 + 1 < kBK / 16) frags(buf, k16 + 1, fa[(k16 + 1) & 1], fb[(k16 + 1) & 1]);
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int i = q >> 2, j = q & 3;
        acc[i][j] = mfma32(fa[k16 & 1][i], fb[k16 & 1][j], acc[i][j]);
        QLORA_SCHED_FENCE();
        pr.run(16 * k16 + q, R.q2, R.S, R.c0, R.c1, wdst, R.x, adst);
        QLORA_SCHED_FENCE();
      }
    }
  };

  // Main K loop: tile kt in LDS buffer kt&1, tile kt+1 in registers, tile kt+2 in flight.
  FwdRegs R0, R1;
  issue(0, R0);
  issue(1, R1);
  restore(R0, 0);
  lds_barrier();
  for (int kt = 0; kt < nk; kt += 2) {
    issue(kt + 2, R0);
    step(0, R1);
    lds_barrier();
    issue(kt + 3, R1);
    step(1, R0);
    lds_barrier();
  }
  // (an odd K count ran one zero tile through buffer 1)

  // Adapter K tile(s): su [T, r_pad] and B [d_out, r], both K-contiguous bf16.
  const rsrc_t ur = make_rsrc(su + m0 * r_pad, mrows * r_pad * 2);
  const rsrc_t br = make_rsrc(B + n0 * r, nrows * r * 2);
  for (int lt = 0; lt < nk_lora; ++lt) {
    const int j0 = lt * kBK;
    uint16_t *as = As, *bs = Bs + tid * kAP;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t off = j0 + xc < r_pad ? (uint32_t)(((xr_ + 32 * i) * r_pad + j0 + xc) * 2) : kOOB;
      st16(as + (xr_ + 32 * i) * kAP + xc, bld16(ur, off));
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const uint32_t off = j0 + 8 * q < r ? (uint32_t)((tid * r + j0 + 8 * q) * 2) : kOOB;
      st16(bs + 8 * q, bld16(br, off));
    }
    lds_barrier();
    compute(0);
    lds_barrier();
  }

  // Epilogue through LDS (the tile buffers are free now): wave w stages its
  // 128 x 128 bf16 tile, then writes 16-byte rows of h.
  store_tile_bf16(acc, smem + wave * 128 * kEP, lane, h, d_out, m0 + wm * 128, n0 + wn * 128, T, d_out);
}

// ---------------------------------------------------------------------------
// Backward dX
// ---------------------------------------------------------------------------
constexpr size_t kDxLds = (size_t)2 * (kBM * kAP + kBK * kBTP) * sizeof(uint16_t);

struct DxRegs {
  u32x4 y[8];    // 8 rows x 8 bf16 of the dY tile
  u32x4 c0, c1;  // one 64-weight block of codes
  uint32_t q2;
  float S;
};

// B fragment of v_mfma_f32_32x32x16_bf16 from a [k][n] bf16 tile (n contiguous,
// pitch p): lane l gets column n0 + l%32, rows k0 + 8(l/32) .. + 7. Within each
// 16 lanes, ds_read_b64_tr_b16 hands lane j element e of the 8 bytes that lane
// 4e + j/4 addresses (its 16-bit element j%4); lane s therefore addresses row
// k + s/4, columns 4(s%4) .. + 3 of its group's 16 columns.
__device__ __forceinline__ u32x4 frag_b_tr(const uint16_t *t, int p, int k0, int n0, int lane) {
  const int grp = lane >> 4, s = lane & 15;
  const int k = k0 + 8 * (grp >> 1) + (s >> 2), n = n0 + 16 * (grp & 1) + 4 * (s & 3);
  typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(t + k * p + n));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(t + (k + 4) * p + n));
  const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
  return u32x4{l2[0], l2[1], h2[0], h2[1]};
}

__global__ __launch_bounds__(256) void k_gemm_dx(const uint8_t *__restrict__ codes,
                                                 const uint8_t *__restrict__ qscale,
                                                 const float *__restrict__ smax, int64_t d_out, int64_t d_in,
                                                 const uint16_t *__restrict__ dY, int64_t T,
                                                 const uint16_t *__restrict__ sv, int r_pad,
                                                 const uint16_t *__restrict__ A, int r,
                                                 uint16_t *__restrict__ dX) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  uint16_t *As = smem;                      // [2][kBM][kAP]   dY tile [t][o]
  uint16_t *Bt = smem + 2 * kBM * kAP;      // [2][kBK][kBTP]  W_hat tile [o][i]
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wm = wave & 1, wn = wave >> 1;
  const int64_t m0 = (int64_t)blockIdx.y * kBM, n0 = (int64_t)blockIdx.x * kBN;  // n = input feature i
  const int64_t KB = d_in / kBlock;
  const int nk = (int)((d_out + kBK - 1) / kBK);
  const int nk_lora = r > 0 ? (r_pad + kBK - 1) / kBK : 0;

  const int64_t mrows = T - m0 < kBM ? T - m0 : kBM;
  const rsrc_t yr = make_rsrc(dY + m0 * d_out, mrows * d_out * 2);

  const int xr_ = tid >> 3, xc = (tid & 7) * 8;
  const int wo = tid >> 2, wb = tid & 3;  // weight tile: row o, block b (64 columns)
  const int64_t kblk = n0 / kBlock + wb;

  auto issue = [&](int kt, DxRegs &R) {
    const int64_t k0 = (int64_t)kt * kBK;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bool ok = kt < nk && k0 + xc < d_out;
      R.y[i] = bld16(yr, ok ? (uint32_t)(((xr_ + 32 * i) * d_out + k0 + xc) * 2) : kOOB);
    }
    // weight rows k0..k0+63: ranges rebased per K tile (32-bit offsets stay small for any weight size)
    const int64_t orows = kt < nk ? (d_out - k0 < kBK ? d_out - k0 : kBK) : 0;
    const int64_t kr = kt < nk ? k0 : 0;
    const rsrc_t cr = make_rsrc(codes + kr * (d_in / 2), orows * (d_in / 2));
    const rsrc_t qr = make_rsrc(qscale + kr * KB, orows * KB);
    const int64_t gb = (kr * KB) >> 8;  // first group of the tile's rows
    const rsrc_t sr = make_rsrc(smax + gb, ((d_out * KB + kGroup - 1) / kGroup - gb) * 4);
    const bool ok = wo < orows && kblk < KB;
    const uint32_t lblk = (uint32_t)(wo * KB + kblk);  // block index within the tile
    R.c0 = bld16(cr, ok ? lblk * 32u : kOOB);
    R.c1 = bld16(cr, ok ? lblk * 32u + 16u : kOOB);
    R.q2 = bld8(qr, ok ? lblk : kOOB);
    R.S = __uint_as_float(bld32(sr, ok ? (uint32_t)((((kr * KB) & (kGroup - 1)) + lblk) >> 8) * 4u : kOOB));
  };
  auto restore = [&](const DxRegs &R, int buf) {
    uint16_t *as = As + buf * kBM * kAP;
#pragma unroll
    for (int i = 0; i < 8; ++i) st16(as + (xr_ + 32 * i) * kAP + xc, R.y[i]);
    const Nf4Planes t = make_planes(restore_scale(R.q2, R.S));
    uint16_t *bt = Bt + buf * kBK * kBTP + wo * kBTP + wb * 64;
#pragma unroll
    for (int m = 0; m < 4; ++m) st16(bt + 8 * m, expand8(t, R.c0[m]));
#pragma unroll
    for (int m = 0; m < 4; ++m) st16(bt + 32 + 8 * m, expand8(t, R.c1[m]));
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  auto compute = [&](int buf) {
    const uint16_t *as = As + buf * kBM * kAP + (wm * 128 + (lane & 31)) * kAP + 8 * (lane >> 5);
    const uint16_t *bt = Bt + buf * kBK * kBTP;
#pragma unroll
    for (int k16 = 0; k16 < kBK / 16; ++k16) {
      u32x4 a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = *reinterpret_cast<const u32x4 *>(as + i * 32 * kAP + 16 * k16);
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = frag_b_tr(bt, kBTP, 16 * k16, wn * 128 + j * 32, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma32(a[i], b[j], acc[i][j]);
    }
  };

  auto frags = [&](int buf, int k16, u32x4 (&a)[4], u32x4 (&b)[4]) {
    const uint16_t *as = As + buf * kBM * kAP + (wm * 128 + (lane & 31)) * kAP + 8 * (lane >> 5) + 16 * k16;
    const uint16_t *bt = Bt + buf * kBK * kBTP;
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = *reinterpret_cast<const u32x4 *>(as + i * 32 * kAP);
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = frag_b_tr(bt, kBTP, 16 * k16, wn * 128 + j * 32, lane);
  };
  auto step = [&](int buf, const DxRegs &R) {
    uint16_t *wdst = Bt + (buf ^ 1) * kBK * kBTP + wo * kBTP + wb * 64;
    uint16_t *adst[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) adst[i] = As + (buf ^ 1) * kBM * kAP + (xr_ + 32 * i) * kAP + xc;
    PieceRestore pr;
    u32x4 fa[2][4], fb[2][4];
    frags(buf, 0, fa[0], fb[0]);
#pragma unroll
    for (int k16 = 0; k16 < kBK / 16; ++k16) {
      if (k16 + 1 < kBK / 16) frags(buf, k16 + 1, fa[(k16 + 1) & 1], fb[(k16 + 1) & 1]);
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int i = q >> 2, j = q & 3;
        acc[i][j] = mfma32(fa[k16 & 1][i], fb[k16 & 1][j], acc[i][j]);
        QLORA_SCHED_FENCE();
        pr.run(16 * k16 + q, R.q2, R.S, R.c0, R.c1, wdst, R.y, adst);
        QLORA_SCHED_FENCE();
      }
    }
  };

  DxRegs R0, R1;
  issue(0, R0);
  issue(1, R1);
  restore(R0, 0);
  lds_barrier();
  for (int kt = 0; kt < nk; kt += 2) {
    issue(kt + 2, R0);
    step(0, R1);
    lds_barrier();
    issue(kt + 3, R1);
    step(1, R0);
    lds_barrier();
  }

  const rsrc_t vr = make_rsrc(sv + m0 * r_pad, mrows * r_pad * 2);
  const rsrc_t ar = make_rsrc(A, (int64_t)r * d_in * 2);
  for (int lt = 0; lt < nk_lora; ++lt) {
    const int j0 = lt * kBK;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t off = j0 + xc < r_pad ? (uint32_t)(((xr_ + 32 * i) * r_pad + j0 + xc) * 2) : kOOB;
      st16(As + (xr_ + 32 * i) * kAP + xc, bld16(vr, off));
    }
    // A rows j0..j0+63, columns n0..n0+255
#pragma unroll
    for (int q = 0; q < kBK * (kBN / 8) / 256; ++q) {
      const int e = q * 256 + tid;
      const int jr = e / (kBN / 8), cc = (e % (kBN / 8)) * 8;
      const int64_t j = j0 + jr, i = n0 + cc;
      const uint32_t off = (j < r && i < d_in) ? (uint32_t)((j * d_in + i) * 2) : kOOB;
      st16(Bt + jr * kBTP + cc, bld16(ar, off));
    }
    lds_barrier();
    compute(0);
    lds_barrier();
  }

  store_tile_bf16(acc, smem + wave * 128 * kEP, lane, dX, d_in, m0 + wm * 128, n0 + wn * 128, T, d_in);
}

static bool g_attr_set[64];

static hipError_t set_lds_attrs() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (g_attr_set[dev]) return hipSuccess;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(k_gemm_fwd),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)kFwdLds);
  if (e != hipSuccess) return e;
  e = hipFuncSetAttribute(reinterpret_cast<const void *>(k_gemm_dx), hipFuncAttributeMaxDynamicSharedMemorySize,
                          (int)kDxLds);
  if (e != hipSuccess) return e;
  g_attr_set[dev] = true;
  return hipSuccess;
}

hipError_t launch_gemm_fwd(const uint8_t *codes, const uint8_t *qscale, const float *smax, int64_t d_out,
                           int64_t d_in, const uint16_t *x, int64_t T, const uint16_t *su, int r_pad,
                           const uint16_t *B, int r, uint16_t *h, const Nf4Consts &c, hipStream_t st) {
  (void)c;
  hipError_t e = set_lds_attrs();
  if (e != hipSuccess) return e;
  dim3 grid((unsigned)((d_out + kBN - 1) / kBN), (unsigned)((T + kBM - 1) / kBM));
  k_gemm_fwd<<<grid, dim3(256), kFwdLds, st>>>(codes, qscale, smax, d_out, d_in, x, T, su, r_pad, B, r, h);
  return hipGetLastError();
}

hipError_t launch_gemm_dx(const uint8_t *codes, const uint8_t *qscale, const float *smax, int64_t d_out,
                          int64_t d_in, const uint16_t *dY, int64_t T, const uint16_t *sv, int r_pad,
                          const uint16_t *A, int r, uint16_t *dX, const Nf4Consts &c, hipStream_t st) {
  (void)c;
  hipError_t e = set_lds_attrs();
  if (e != hipSuccess) return e;
  dim3 grid((unsigned)((d_in + kBN - 1) / kBN), (unsigned)((T + kBM - 1) / kBM));
  k_gemm_dx<<<grid, dim3(256), kDxLds, st>>>(codes, qscale, smax, d_out, d_in, dY, T, sv, r_pad, A, r, dX);
  return hipGetLastError();
}

}  // namespace qlora
