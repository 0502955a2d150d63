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
// Tiling: a 512-thread workgroup computes a 256 x 256 output tile; its eight
// waves (two per SIMD) each own 128 x 64 (4 x 2 v_mfma_f32_32x32x16_bf16
// tiles). With two waves on a SIMD, one wave's restore VALU issues while the
// other's MFMAs occupy the matrix core. K advances 64 at a time:
//   * global loads run two tiles ahead (two register sets in turn), so a tile's
//     codes and activations have a whole K step to arrive;
//   * LDS is double-buffered: while the MFMAs consume tile k, the waves restore
//     tile k+1 into the other buffer, two lanes per 64-weight block (32 weights
//     each). The restore is cut into pieces of a few VALU instructions, one
//     after each MFMA, with scheduling fences that keep the order;
//   * loop bodies are straight-line: tiles past the end load zeros (out-of-range
//     buffer offsets) and add nothing.
// Forward: W's K (= d_in) runs along a block, so a restored block is one row of
// the K-contiguous weight tile and the MFMA B operand is read straight from LDS.
// dX: K = d_out runs across blocks; the restored tile is stored [o][i] as
// restored and the B fragments (8 consecutive o for one i per lane) come from
// two ds_read_b64_tr_b16, which transpose 16-bit data across each 16 lanes.
// The epilogue goes through LDS so that every lane writes 16-byte rows.
#include "kernels.h"

namespace qlora {

constexpr int kBM = 256, kBN = 256, kBK = 64;
constexpr int kWaves = 8, kThreads = 64 * kWaves;
constexpr int kWM = 128, kWN = 64;  // wave tile
constexpr int kAP = kBK + 8;   // padded pitch (bf16) of [row][k] tiles: fragment reads free of bank conflicts
constexpr int kBTP = kBN + 16; // pitch of the dX [k][n] weight tile: the four rows of a transposed read 8 banks apart
constexpr int kEP = kWN + 8;   // epilogue staging pitch (bf16) of a wave's 128 x 64 tile
constexpr size_t kStageLds = (size_t)kWaves * kWM * kEP * sizeof(uint16_t);

typedef short v4i16 __attribute__((ext_vector_type(4)));

// One wave's 128 x 64 fp32 tile -> bf16 rows of `out` (row pitch ld, rows < mlim,
// columns < nlim), staged through this wave's LDS region so that each lane
// stores 16 contiguous bytes. Lane l, accumulator e of tile (i, j) holds row
// 32i + 8(e/4) + 4(l/32) + e%4, column 32j + l%32.
__device__ __forceinline__ void store_tile_bf16(const f32x16 (&acc)[4][2], uint16_t *stage, int lane,
                                                uint16_t *out, int64_t ld, int64_t row0, int64_t col0,
                                                int64_t mlim, int64_t nlim) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int rr = 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3), cc = 32 * j + (lane & 31);
        stage[rr * kEP + cc] = (uint16_t)(pack_bf16x2(acc[i][j][e], 0.f) & 0xffffu);
      }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  // 128 rows x 8 chunks of 8 bf16: lane takes chunk lane%8 of rows lane/8 + 8q
#pragma unroll 4
  for (int q = 0; q < 16; ++q) {
    const int rr = (lane >> 3) + 8 * q, ch = lane & 7;
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

// Half of a 64-weight block's restore (4 packed words, 32 weights) and four
// activation chunks' LDS stores, cut into 25 pieces of a few VALU instructions
// so that one piece can follow each MFMA of a K step. pieces 0..3: scale and
// table products; 4: byte planes; 5 + 4m + 0..3: word m's selectors,
// low-nibble lookups, high-nibble lookups, interleave and LDS store;
// 21..24: the activation chunks.
constexpr int kPieces = 25;
struct PieceRestore {
  float sh;
  uint32_t p[8];
  Nf4Planes t;
  uint32_t sa, ma, sb, mb, lo_a, hi_a, lo_b, hi_b;
  __device__ __forceinline__ void run(int k, uint32_t q2, float S, const u32x4 &c, uint16_t *wdst,
                                      const u32x4 (&act)[4], uint16_t *const (&adst)[4]) {
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
    } else if (k < 21) {
      const int m = (k - 5) >> 2, ph = (k - 5) & 3;
      const uint32_t w = c[m];
      if (ph == 0) {
        sa = w & 0x07070707u;
        ma = ((w >> 1) & 0x04040404u) | 0x03020100u;
        sb = (w >> 4) & 0x07070707u;
        mb = ((w >> 5) & 0x04040404u) | 0x03020100u;
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
    } else if (k < kPieces) {
      st16(adst[k - 21], act[k - 21]);
    }
  }
};
#define QLORA_SCHED_FENCE() __builtin_amdgcn_sched_barrier(0)

// Register set of one K tile held by one lane: four 8-element activation
// chunks and half a block of codes with its scale code and group maximum.
struct TileRegs {
  u32x4 a[4];
  u32x4 c;
  uint32_t q2;
  float S;
};

// One K step of one wave: the 32 MFMAs of its 128 x 64 tile over LDS buffer
// `buf`, each followed by one restore piece of register set R. Fragments of
// the next 16-wide K slice are read while the current slice's MFMAs run: the
// B pair one slice ahead, each A fragment as soon as its two MFMAs are issued.
template <typename FragFn>
__device__ __forceinline__ void k_step(f32x16 (&acc)[4][2], const FragFn &frags, int buf, const TileRegs &R,
                                       uint16_t *wdst, uint16_t *const (&adst)[4]) {
  PieceRestore pr;
  u32x4 fa[4], fb[2][2];
  frags.a_all(buf, 0, fa);
  frags.b(buf, 0, fb[0]);
#pragma unroll
  for (int k16 = 0; k16 < kBK / 16; ++k16) {
    const bool more = k16 + 1 < kBK / 16;
    if (more) frags.b(buf, k16 + 1, fb[(k16 + 1) & 1]);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int i = q >> 1, j = q & 1;
      acc[i][j] = mfma32(fa[i], fb[k16 & 1][j], acc[i][j]);
      QLORA_SCHED_FENCE();
      pr.run(8 * k16 + q, R.q2, R.S, R.c, wdst, R.a, adst);
      if (j == 1 && more) fa[i] = frags.a(buf, k16 + 1, i);
      QLORA_SCHED_FENCE();
    }
  }
}

// The whole restore of register set R at once (before the first K step).
__device__ __forceinline__ void restore_all(const TileRegs &R, uint16_t *wdst, uint16_t *const (&adst)[4]) {
  PieceRestore pr;
#pragma unroll
  for (int k = 0; k < kPieces; ++k) pr.run(k, R.q2, R.S, R.c, wdst, R.a, adst);
}

// Adapter K slices: MFMAs over LDS buffer 0 without restore work.
template <typename FragFn>
__device__ __forceinline__ void k_plain(f32x16 (&acc)[4][2], const FragFn &frags) {
#pragma unroll
  for (int k16 = 0; k16 < kBK / 16; ++k16) {
    u32x4 a[4], b[2];
    frags.a_all(0, k16, a);
    frags.b(0, k16, b);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(a[i], b[j], acc[i][j]);
  }
}

__device__ __forceinline__ void zero_acc(f32x16 (&acc)[4][2]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
}

// Activation chunk i (< 4) of lane `tid`: row (tid + 512 i) / 8, columns 8 ((tid + 512 i) % 8) .. + 7.
__device__ __forceinline__ int act_row(int tid, int i) { return (tid + kThreads * i) >> 3; }
__device__ __forceinline__ int act_col(int tid) { return (tid & 7) * 8; }

// ---------------------------------------------------------------------------
// Forward
// ---------------------------------------------------------------------------
constexpr size_t kFwdTiles = (size_t)2 * (kBM + kBN) * kAP * sizeof(uint16_t);
constexpr size_t kFwdLds = kFwdTiles > kStageLds ? kFwdTiles : kStageLds;

__global__ __launch_bounds__(kThreads) void k_gemm_fwd(const uint8_t *__restrict__ codes,
                                                       const uint8_t *__restrict__ qscale,
                                                       const float *__restrict__ smax, int64_t d_out, int64_t d_in,
                                                       const uint16_t *__restrict__ x, int64_t T,
                                                       const uint16_t *__restrict__ su, int r_pad,
                                                       const uint16_t *__restrict__ B, int r,
                                                       uint16_t *__restrict__ h) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  uint16_t *As = smem;                        // [2][kBM][kAP]  x tile [t][k]
  uint16_t *Bs = smem + 2 * kBM * kAP;        // [2][kBN][kAP]  W_hat tile [n][k]
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

  const int wrow = tid >> 1, half = tid & 1;  // weight: tile row tid/2, half tid%2 of its block
  const int ac = act_col(tid);

  auto issue = [&](int kt, TileRegs &R) {
    const bool in = kt < nk;  // tiles past the end read zeros
    const int64_t k0 = (int64_t)kt * kBK;
#pragma unroll
    for (int i = 0; i < 4; ++i) R.a[i] = bld16(xr, in ? (uint32_t)((act_row(tid, i) * d_in + k0 + ac) * 2) : kOOB);
    R.c = bld16(cr, in ? (uint32_t)(wrow * (d_in / 2) + (int64_t)kt * (kBlock / 2) + 16 * half) : kOOB);
    R.q2 = bld8(qr, in ? (uint32_t)(wrow * KB + kt) : kOOB);
    R.S = __uint_as_float(bld32(sr, in ? (uint32_t)((((n0 + wrow) * KB + kt) >> 8) * 4) : kOOB));
  };
  auto dsts = [&](int buf, uint16_t *(&adst)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) adst[i] = As + buf * kBM * kAP + act_row(tid, i) * kAP + ac;
    return Bs + buf * kBN * kAP + wrow * kAP + 32 * half;
  };
  struct Frags {
    const uint16_t *as, *bs;  // this lane's fragment rows in buffer 0
    __device__ __forceinline__ u32x4 a(int buf, int k16, int i) const {
      return *reinterpret_cast<const u32x4 *>(as + buf * kBM * kAP + i * 32 * kAP + 16 * k16);
    }
    __device__ __forceinline__ void a_all(int buf, int k16, u32x4 (&f)[4]) const {
#pragma unroll
      for (int i = 0; i < 4; ++i) f[i] = a(buf, k16, i);
    }
    __device__ __forceinline__ void b(int buf, int k16, u32x4 (&f)[2]) const {
#pragma unroll
      for (int j = 0; j < 2; ++j)
        f[j] = *reinterpret_cast<const u32x4 *>(bs + buf * kBN * kAP + j * 32 * kAP + 16 * k16);
    }
  };
  const Frags frags{As + (wm * kWM + (lane & 31)) * kAP + 8 * (lane >> 5),
                    Bs + (wn * kWN + (lane & 31)) * kAP + 8 * (lane >> 5)};

  f32x16 acc[4][2];
  zero_acc(acc);

  // Main K loop: tile kt in LDS buffer kt&1, tile kt+1 in registers, tile kt+2 in flight.
  TileRegs R0, R1;
  uint16_t *adst[4];
  issue(0, R0);
  issue(1, R1);
  restore_all(R0, dsts(0, adst), adst);
  lds_barrier();
  for (int kt = 0; kt < nk; kt += 2) {
    issue(kt + 2, R0);
    k_step(acc, frags, 0, R1, dsts(1, adst), adst);
    lds_barrier();
    issue(kt + 3, R1);
    k_step(acc, frags, 1, R0, dsts(0, adst), adst);
    lds_barrier();
  }
  // (an odd K count ran one zero tile through buffer 1)

  // Adapter K tile(s): su [T, r_pad] and B [d_out, r], both K-contiguous bf16.
  const rsrc_t ur = make_rsrc(su + m0 * r_pad, mrows * r_pad * 2);
  const rsrc_t br = make_rsrc(B + n0 * r, nrows * r * 2);
  for (int lt = 0; lt < nk_lora; ++lt) {
    const int j0 = lt * kBK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = act_row(tid, i);
      const uint32_t off = j0 + ac < r_pad ? (uint32_t)((row * r_pad + j0 + ac) * 2) : kOOB;
      st16(As + row * kAP + ac, bld16(ur, off));
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int col = 32 * half + 8 * q;
      const uint32_t off = j0 + col < r ? (uint32_t)((wrow * r + j0 + col) * 2) : kOOB;
      st16(Bs + wrow * kAP + col, bld16(br, off));
    }
    lds_barrier();
    k_plain(acc, frags);
    lds_barrier();
  }

  // Epilogue through LDS (the tile buffers are free now).
  store_tile_bf16(acc, smem + wave * kWM * kEP, lane, h, d_out, m0 + wm * kWM, n0 + wn * kWN, T, d_out);
}

// ---------------------------------------------------------------------------
// Backward dX
// ---------------------------------------------------------------------------
constexpr size_t kDxTiles = (size_t)2 * (kBM * kAP + kBK * kBTP) * sizeof(uint16_t);
constexpr size_t kDxLds = kDxTiles > kStageLds ? kDxTiles : kStageLds;

__global__ __launch_bounds__(kThreads) void k_gemm_dx(const uint8_t *__restrict__ codes,
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

  const int ac = act_col(tid);
  // weight tile: 64 rows o x 4 blocks of 64 columns i; lane -> block tid/2 (row wo, block wb), half tid%2
  const int wblk = tid >> 1, half = tid & 1;
  const int wo = wblk >> 2, wb = wblk & 3;
  const int64_t kblk = n0 / kBlock + wb;

  auto issue = [&](int kt, TileRegs &R) {
    const int64_t k0 = (int64_t)kt * kBK;
    const bool aok = kt < nk && k0 + ac < d_out;
#pragma unroll
    for (int i = 0; i < 4; ++i) R.a[i] = bld16(yr, aok ? (uint32_t)((act_row(tid, i) * d_out + k0 + ac) * 2) : kOOB);
    // weight rows k0..k0+63: ranges rebased per K tile (32-bit offsets stay small for any weight size)
    const int64_t orows = kt < nk ? (d_out - k0 < kBK ? d_out - k0 : kBK) : 0;
    const int64_t kr = kt < nk ? k0 : 0;
    const rsrc_t cr = make_rsrc(codes + kr * (d_in / 2), orows * (d_in / 2));
    const rsrc_t qr = make_rsrc(qscale + kr * KB, orows * KB);
    const int64_t gb = (kr * KB) >> 8;  // first group of the tile's rows
    const rsrc_t sr = make_rsrc(smax + gb, ((d_out * KB + kGroup - 1) / kGroup - gb) * 4);
    // Rows past the tile's end fall outside the ranges and restore to zero
    // (scale code 0). Blocks past d_in (kblk >= KB) read the next row's
    // blocks: finite values that reach only output columns past d_in, which
    // are never stored.
    const uint32_t lblk = (uint32_t)(wo * KB + kblk);  // block index within the tile
    R.c = bld16(cr, lblk * 32u + 16u * half);
    R.q2 = bld8(qr, lblk);
    R.S = __uint_as_float(bld32(sr, (uint32_t)((((kr * KB) & (kGroup - 1)) + lblk) >> 8) * 4u));
  };
  auto dsts = [&](int buf, uint16_t *(&adst)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) adst[i] = As + buf * kBM * kAP + act_row(tid, i) * kAP + ac;
    return Bt + buf * kBK * kBTP + wo * kBTP + wb * 64 + 32 * half;
  };
  struct Frags {
    const uint16_t *as;  // this lane's A fragment rows in buffer 0
    const uint16_t *bt;  // the address this lane hands to the transposed reads of column tile 0, slice 0, buffer 0
    __device__ __forceinline__ u32x4 a(int buf, int k16, int i) const {
      return *reinterpret_cast<const u32x4 *>(as + buf * kBM * kAP + i * 32 * kAP + 16 * k16);
    }
    __device__ __forceinline__ void a_all(int buf, int k16, u32x4 (&f)[4]) const {
#pragma unroll
      for (int i = 0; i < 4; ++i) f[i] = a(buf, k16, i);
    }
    __device__ __forceinline__ void b(int buf, int k16, u32x4 (&f)[2]) const {
      typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint16_t *t = bt + buf * kBK * kBTP + 16 * k16 * kBTP + 32 * j;
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)t);
        const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(t + 4 * kBTP));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        f[j] = u32x4{l2[0], l2[1], h2[0], h2[1]};
      }
    }
  };
  // B fragment of v_mfma_f32_32x32x16_bf16 from the [k][n] weight tile: lane l
  // gets column n + l%32, rows k0 + 8(l/32) .. + 7. Within each 16 lanes,
  // ds_read_b64_tr_b16 hands lane j element e of the 8 bytes that lane
  // 4e + j/4 addresses (its 16-bit element j%4); lane s of group g therefore
  // addresses row 8(g/2) + s/4, columns 16(g%2) + 4(s%4) .. + 3, and a second
  // read four rows further down gives elements 4..7.
  const int tgrp = lane >> 4, ts = lane & 15;
  const Frags frags{As + (wm * kWM + (lane & 31)) * kAP + 8 * (lane >> 5),
                    Bt + (8 * (tgrp >> 1) + (ts >> 2)) * kBTP + wn * kWN + 16 * (tgrp & 1) + 4 * (ts & 3)};

  f32x16 acc[4][2];
  zero_acc(acc);

  TileRegs R0, R1;
  uint16_t *adst[4];
  issue(0, R0);
  issue(1, R1);
  restore_all(R0, dsts(0, adst), adst);
  lds_barrier();
  for (int kt = 0; kt < nk; kt += 2) {
    issue(kt + 2, R0);
    k_step(acc, frags, 0, R1, dsts(1, adst), adst);
    lds_barrier();
    issue(kt + 3, R1);
    k_step(acc, frags, 1, R0, dsts(0, adst), adst);
    lds_barrier();
  }

  const rsrc_t vr = make_rsrc(sv + m0 * r_pad, mrows * r_pad * 2);
  const rsrc_t ar = make_rsrc(A, (int64_t)r * d_in * 2);
  for (int lt = 0; lt < nk_lora; ++lt) {
    const int j0 = lt * kBK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = act_row(tid, i);
      const uint32_t off = j0 + ac < r_pad ? (uint32_t)((row * r_pad + j0 + ac) * 2) : kOOB;
      st16(As + row * kAP + ac, bld16(vr, off));
    }
    // A rows j0..j0+63, columns n0..n0+255
#pragma unroll
    for (int q = 0; q < kBK * (kBN / 8) / kThreads; ++q) {
      const int e = q * kThreads + tid;
      const int jr = e / (kBN / 8), cc = (e % (kBN / 8)) * 8;
      const int64_t j = j0 + jr, i = n0 + cc;
      const uint32_t off = (j < r && i < d_in) ? (uint32_t)((j * d_in + i) * 2) : kOOB;
      st16(Bt + jr * kBTP + cc, bld16(ar, off));
    }
    lds_barrier();
    k_plain(acc, frags);
    lds_barrier();
  }

  store_tile_bf16(acc, smem + wave * kWM * kEP, lane, dX, d_in, m0 + wm * kWM, n0 + wn * kWN, T, d_in);
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
  k_gemm_fwd<<<grid, dim3(kThreads), kFwdLds, st>>>(codes, qscale, smax, d_out, d_in, x, T, su, r_pad, B, r, h);
  return hipGetLastError();
}

hipError_t launch_gemm_dx(const uint8_t *codes, const uint8_t *qscale, const float *smax, int64_t d_out,
                          int64_t d_in, const uint16_t *dY, int64_t T, const uint16_t *sv, int r_pad,
                          const uint16_t *A, int r, uint16_t *dX, const Nf4Consts &c, hipStream_t st) {
  (void)c;
  hipError_t e = set_lds_attrs();
  if (e != hipSuccess) return e;
  dim3 grid((unsigned)((d_in + kBN - 1) / kBN), (unsigned)((T + kBM - 1) / kBM));
  k_gemm_dx<<<grid, dim3(kThreads), kDxLds, st>>>(codes, qscale, smax, d_out, d_in, dY, T, sv, r_pad, A, r, dX);
  return hipGetLastError();
}

}  // namespace qlora
