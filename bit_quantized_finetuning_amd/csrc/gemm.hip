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
// accumulators per lane). K advances 64 at a time through double-buffered LDS:
// the next tile's global loads are issued before the current tile's MFMAs, and
// its restore (one 64-weight block per thread, one table per block) is written
// to the other buffer afterwards. M rows of each 256-row tile are padded with
// 16 bytes to keep the 16-byte fragment reads free of bank conflicts.
//
// Forward: W's K (= d_in) runs along a block, so a thread restores one whole
// block of one output row and the MFMA B operand is read straight from LDS.
// dX: K = d_out runs across blocks; the restored tile is stored as [o][i] and
// the B fragments (8 consecutive o for one i per lane) are gathered with 16-bit
// LDS reads.
#include "kernels.h"

namespace qlora {

constexpr int kBM = 256, kBN = 256, kBK = 64;
constexpr int kAP = kBK + 8;   // padded pitch (bf16) of [row][k] tiles
constexpr int kBTP = kBN + 8;  // padded pitch of the dX [k][n] weight tile

// ---------------------------------------------------------------------------
// Forward
// ---------------------------------------------------------------------------
constexpr size_t kFwdLds = (size_t)2 * (kBM + kBN) * kAP * sizeof(uint16_t);

__global__ __launch_bounds__(256) void k_gemm_fwd(const uint8_t *__restrict__ codes,
                                                  const uint8_t *__restrict__ qscale,
                                                  const float *__restrict__ smax, int64_t d_out, int64_t d_in,
                                                  const uint16_t *__restrict__ x, int64_t T,
                                                  const uint16_t *__restrict__ su, int r_pad,
                                                  const uint16_t *__restrict__ B, int r,
                                                  uint16_t *__restrict__ h, Nf4Consts c) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  uint16_t *As = smem;                        // [2][kBM][kAP]
  uint16_t *Bs = smem + 2 * kBM * kAP;        // [2][kBN][kAP]
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wm = wave & 1, wn = wave >> 1;
  const int64_t m0 = (int64_t)blockIdx.y * kBM, n0 = (int64_t)blockIdx.x * kBN;
  const int64_t KB = d_in / kBlock;
  const int nk_main = (int)KB;
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
  u32x4 xa[8];
  u32x4 cw0, cw1;
  uint32_t q2;
  float S;

  auto load_main = [&](int kt) {
    const int64_t k0 = (int64_t)kt * kBK;
#pragma unroll
    for (int i = 0; i < 8; ++i) xa[i] = bld16(xr, (uint32_t)(((xr_ + 32 * i) * d_in + k0 + xc) * 2));
    const uint32_t coff = (uint32_t)(tid * (d_in / 2) + (int64_t)kt * (kBlock / 2));
    cw0 = bld16(cr, coff);
    cw1 = bld16(cr, coff + 16);
    q2 = bld8(qr, (uint32_t)(tid * KB + kt));
    S = __uint_as_float(bld32(sr, (uint32_t)((((n0 + tid) * KB + kt) >> 8) * 4)));
  };
  auto store_main = [&](int buf) {
    uint16_t *as = As + buf * kBM * kAP;
#pragma unroll
    for (int i = 0; i < 8; ++i) st16(as + (xr_ + 32 * i) * kAP + xc, xa[i]);
    const Nf4Planes t = make_planes(restore_scale(q2, S));
    uint16_t *bs = Bs + buf * kBN * kAP + tid * kAP;
#pragma unroll
    for (int m = 0; m < 4; ++m) st16(bs + 8 * m, expand8(t, cw0[m]));
#pragma unroll
    for (int m = 0; m < 4; ++m) st16(bs + 32 + 8 * m, expand8(t, cw1[m]));
  };
  // Adapter K tile: su [T, r_pad] and B [d_out, r], both K-contiguous bf16.
  const rsrc_t ur = make_rsrc(su + m0 * r_pad, mrows * r_pad * 2);
  const rsrc_t br = make_rsrc(B + n0 * r, nrows * r * 2);
  auto load_store_lora = [&](int lt, int buf) {
    const int j0 = lt * kBK;
    uint16_t *as = As + buf * kBM * kAP;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t off = j0 + xc < r_pad ? (uint32_t)(((xr_ + 32 * i) * r_pad + j0 + xc) * 2) : kOOB;
      st16(as + (xr_ + 32 * i) * kAP + xc, bld16(ur, off));
    }
    uint16_t *bs = Bs + buf * kBN * kAP + tid * kAP;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const uint32_t off = j0 + 8 * q < r ? (uint32_t)((tid * r + j0 + 8 * q) * 2) : kOOB;
      st16(bs + 8 * q, bld16(br, off));
    }
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

  if (nk_main > 0) {
    load_main(0);
    store_main(0);
  }
  __syncthreads();
  for (int kt = 0; kt < nk_main; ++kt) {
    const int buf = kt & 1;
    const bool more = kt + 1 < nk_main;
    if (more) load_main(kt + 1);
    compute(buf);
    if (more) store_main(buf ^ 1);
    __syncthreads();
  }
  for (int lt = 0; lt < nk_lora; ++lt) {
    const int buf = (nk_main + lt) & 1;
    load_store_lora(lt, buf);
    __syncthreads();
    compute(buf);
    __syncthreads();
  }

  // Epilogue: lane l, accumulator e of tile (i, j) is row 8*(e/4) + 4*(l/32) + e%4,
  // column l%32 of that 32 x 32 tile.
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t n = n0 + wn * 128 + j * 32 + (lane & 31);
      if (n >= d_out) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t m = m0 + wm * 128 + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        if (m < T) h[m * d_out + n] = (uint16_t)(pack_bf16x2(acc[i][j][e], 0.f) & 0xffffu);
      }
    }
}

// ---------------------------------------------------------------------------
// Backward dX
// ---------------------------------------------------------------------------
constexpr size_t kDxLds = (size_t)2 * (kBM * kAP + kBK * kBTP) * sizeof(uint16_t);

__device__ __forceinline__ uint32_t lds_pair(const uint16_t *p0, const uint16_t *p1) {
  return (uint32_t)*p0 | ((uint32_t)*p1 << 16);
}

__global__ __launch_bounds__(256) void k_gemm_dx(const uint8_t *__restrict__ codes,
                                                 const uint8_t *__restrict__ qscale,
                                                 const float *__restrict__ smax, int64_t d_out, int64_t d_in,
                                                 const uint16_t *__restrict__ dY, int64_t T,
                                                 const uint16_t *__restrict__ sv, int r_pad,
                                                 const uint16_t *__restrict__ A, int r,
                                                 uint16_t *__restrict__ dX, Nf4Consts c) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  uint16_t *As = smem;                      // [2][kBM][kAP]   dY tile [t][o]
  uint16_t *Bt = smem + 2 * kBM * kAP;      // [2][kBK][kBTP]  W_hat tile [o][i]
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wm = wave & 1, wn = wave >> 1;
  const int64_t m0 = (int64_t)blockIdx.y * kBM, n0 = (int64_t)blockIdx.x * kBN;  // n = input feature i
  const int64_t KB = d_in / kBlock;
  const int nk_main = (int)((d_out + kBK - 1) / kBK);
  const int nk_lora = r > 0 ? (r_pad + kBK - 1) / kBK : 0;

  const int64_t mrows = T - m0 < kBM ? T - m0 : kBM;
  const rsrc_t yr = make_rsrc(dY + m0 * d_out, mrows * d_out * 2);
  const rsrc_t sr = make_rsrc(smax, ((d_out * KB + kGroup - 1) / kGroup) * 4);

  const int xr_ = tid >> 3, xc = (tid & 7) * 8;
  const int wo = tid >> 2, wb = tid & 3;  // weight tile: row o, block b (64 columns)
  const int64_t kblk = n0 / kBlock + wb;
  u32x4 xa[8];
  u32x4 cw0, cw1;
  uint32_t q2;
  float S;

  auto load_main = [&](int kt) {
    const int64_t k0 = (int64_t)kt * kBK;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t off = k0 + xc < d_out ? (uint32_t)(((xr_ + 32 * i) * d_out + k0 + xc) * 2) : kOOB;
      xa[i] = bld16(yr, off);
    }
    // weight rows k0..k0+63 of this k tile, 4 blocks of columns per row
    const int64_t orows = d_out - k0 < kBK ? d_out - k0 : kBK;
    const rsrc_t cr = make_rsrc(codes + k0 * (d_in / 2), orows * (d_in / 2));
    const rsrc_t qr = make_rsrc(qscale + k0 * KB, orows * KB);
    const bool ok = kblk < KB;
    const uint32_t coff = ok ? (uint32_t)(wo * (d_in / 2) + kblk * (kBlock / 2)) : kOOB;
    cw0 = bld16(cr, coff);
    cw1 = bld16(cr, coff + 16);
    q2 = bld8(qr, ok ? (uint32_t)(wo * KB + kblk) : kOOB);
    S = __uint_as_float(bld32(sr, ok ? (uint32_t)((((k0 + wo) * KB + kblk) >> 8) * 4) : kOOB));
  };
  auto store_main = [&](int buf) {
    uint16_t *as = As + buf * kBM * kAP;
#pragma unroll
    for (int i = 0; i < 8; ++i) st16(as + (xr_ + 32 * i) * kAP + xc, xa[i]);
    const Nf4Planes t = make_planes(restore_scale(q2, S));
    uint16_t *bt = Bt + buf * kBK * kBTP + wo * kBTP + wb * 64;
#pragma unroll
    for (int m = 0; m < 4; ++m) st16(bt + 8 * m, expand8(t, cw0[m]));
#pragma unroll
    for (int m = 0; m < 4; ++m) st16(bt + 32 + 8 * m, expand8(t, cw1[m]));
  };
  const rsrc_t vr = make_rsrc(sv + m0 * r_pad, mrows * r_pad * 2);
  const rsrc_t ar = make_rsrc(A, (int64_t)r * d_in * 2);
  auto load_store_lora = [&](int lt, int buf) {
    const int j0 = lt * kBK;
    uint16_t *as = As + buf * kBM * kAP;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t off = j0 + xc < r_pad ? (uint32_t)(((xr_ + 32 * i) * r_pad + j0 + xc) * 2) : kOOB;
      st16(as + (xr_ + 32 * i) * kAP + xc, bld16(vr, off));
    }
    // A rows j0..j0+63, columns n0..n0+255
    uint16_t *bt = Bt + buf * kBK * kBTP;
#pragma unroll
    for (int q = 0; q < kBK * (kBN / 8) / 256; ++q) {
      const int e = q * 256 + tid;
      const int jr = e / (kBN / 8), cc = (e % (kBN / 8)) * 8;
      const int64_t j = j0 + jr, i = n0 + cc;
      const uint32_t off = (j < r && i < d_in) ? (uint32_t)((j * d_in + i) * 2) : kOOB;
      st16(bt + jr * kBTP + cc, bld16(ar, off));
    }
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
    const uint16_t *bt = Bt + buf * kBK * kBTP + (8 * (lane >> 5)) * kBTP + wn * 128 + (lane & 31);
#pragma unroll
    for (int k16 = 0; k16 < kBK / 16; ++k16) {
      u32x4 a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = *reinterpret_cast<const u32x4 *>(as + i * 32 * kAP + 16 * k16);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint16_t *p = bt + (16 * k16) * kBTP + j * 32;
#pragma unroll
        for (int e = 0; e < 4; ++e) b[j][e] = lds_pair(p + (2 * e) * kBTP, p + (2 * e + 1) * kBTP);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma32(a[i], b[j], acc[i][j]);
    }
  };

  load_main(0);
  store_main(0);
  __syncthreads();
  for (int kt = 0; kt < nk_main; ++kt) {
    const int buf = kt & 1;
    const bool more = kt + 1 < nk_main;
    if (more) load_main(kt + 1);
    compute(buf);
    if (more) store_main(buf ^ 1);
    __syncthreads();
  }
  for (int lt = 0; lt < nk_lora; ++lt) {
    const int buf = (nk_main + lt) & 1;
    load_store_lora(lt, buf);
    __syncthreads();
    compute(buf);
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t n = n0 + wn * 128 + j * 32 + (lane & 31);
      if (n >= d_in) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t m = m0 + wm * 128 + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        if (m < T) dX[m * d_in + n] = (uint16_t)(pack_bf16x2(acc[i][j][e], 0.f) & 0xffffu);
      }
    }
}

static bool g_attr_set = false;

static hipError_t set_lds_attrs() {
  if (g_attr_set) return hipSuccess;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(k_gemm_fwd),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)kFwdLds);
  if (e != hipSuccess) return e;
  e = hipFuncSetAttribute(reinterpret_cast<const void *>(k_gemm_dx), hipFuncAttributeMaxDynamicSharedMemorySize,
                          (int)kDxLds);
  if (e != hipSuccess) return e;
  g_attr_set = true;
  return hipSuccess;
}

hipError_t launch_gemm_fwd(const uint8_t *codes, const uint8_t *qscale, const float *smax, int64_t d_out,
                           int64_t d_in, const uint16_t *x, int64_t T, const uint16_t *su, int r_pad,
                           const uint16_t *B, int r, uint16_t *h, const Nf4Consts &c, hipStream_t st) {
  hipError_t e = set_lds_attrs();
  if (e != hipSuccess) return e;
  dim3 grid((unsigned)((d_out + kBN - 1) / kBN), (unsigned)((T + kBM - 1) / kBM));
  k_gemm_fwd<<<grid, dim3(256), kFwdLds, st>>>(codes, qscale, smax, d_out, d_in, x, T, su, r_pad, B, r, h, c);
  return hipGetLastError();
}

hipError_t launch_gemm_dx(const uint8_t *codes, const uint8_t *qscale, const float *smax, int64_t d_out,
                          int64_t d_in, const uint16_t *dY, int64_t T, const uint16_t *sv, int r_pad,
                          const uint16_t *A, int r, uint16_t *dX, const Nf4Consts &c, hipStream_t st) {
  hipError_t e = set_lds_attrs();
  if (e != hipSuccess) return e;
  dim3 grid((unsigned)((d_in + kBN - 1) / kBN), (unsigned)((T + kBM - 1) / kBM));
  k_gemm_dx<<<grid, dim3(256), kDxLds, st>>>(codes, qscale, smax, d_out, d_in, dY, T, sv, r_pad, A, r, dX, c);
  return hipGetLastError();
}

}  // namespace qlora
