// Forward for T <= 16 tokens in one launch: stream the 4.13-bit weight once.
//
// h[T, d_out] = x W_hat^T + s (x A^T) B^T   ("QLoRA의 수식" on the first page: the
// restored frozen base plus the adapter term, s = alpha/r).
//
// Every weight is used by at most 16 tokens, so the kernel is bound by the
// packed-weight stream (0.516 bytes per weight) and by the VALU work of the
// restore (~3.7 instructions per weight). Calls of this size are also dominated
// by launch, ramp and memory latency, so the design issues as many loads as
// possible up front and keeps the per-wave fixed work small.
//
// One grid of G workgroups of kW waves, one per CU (G = min(row tiles, CUs)):
//   * workgroup c streams row tiles c, c+G, c+2G, ... of 16 output rows. The
//     waves split K into 256-wide segments; in a segment lane (row, g) owns one
//     64-weight block (two 16-byte code loads), builds that block's restore
//     table once and feeds 8 v_mfma_f32_16x16x32_bf16 (tokens on M, padded to
//     16; rows on N). Each wave prefetches its next (row tile, segment) item
//     while computing the current one (two register stages in ping-pong). x is
//     staged once per workgroup in LDS when it fits (T x d_in bf16 <= 136 KB)
//     and is otherwise read per segment from global memory. At the end of a row
//     tile the waves reduce through LDS and write h; wave 0 first adds s*u B^T
//     as r_pad more K columns.
//   * the first P workgroups also produce the adapter intermediate at their
//     start: job (j, ks) computes columns 16j..16j+15 of u = x A^T over the
//     ks-th of ksp K slices, publishes the partial with device-scope stores and
//     bumps a counter; the last job raises a ready flag.
//   * s*u is formed once per workgroup: wave 0 issues the ready-flag load before
//     streaming; at the first row-tile end every thread sums its entries over
//     the ksp partials in slice order (deterministic) into LDS. The last
//     workgroup through resets the flag.
// The grid never exceeds one residency (one workgroup per CU), producer jobs
// come before any wait, and the spin is bounded anyway (timeout -> status word,
// never a hang). All per-lane offsets are 32-bit against buffer ranges rebased
// per row tile.
#include "kernels.h"

namespace qlora {

constexpr int kSpinLimit = 1 << 21;  // ~60 ms of s_sleep; only a safety net
constexpr int kMaxKsp = 8;           // K slices per adapter column tile
constexpr int kMaxRpad = 256;
constexpr int kXPad = 8;             // bf16 of padding per staged x row (rows 4 banks apart)
constexpr int kXLdsBytes = 136 * 1024;

struct GemvCodes {
  u32x4 c0, c1;  // 32 bytes of codes = one 64-weight block
  uint32_t q2;
  float S;
};
struct GemvX {
  u32x4 x[8];  // 64 bf16 of one token row (global-x path only)
};

template <int kW, bool kXL>
__global__ __launch_bounds__(64 * kW) void k_gemv_fwd(
    const uint8_t *__restrict__ codes, const uint8_t *__restrict__ qscale, const float *__restrict__ smax,
    int d_out, int d_in, const uint16_t *__restrict__ x, int T, const uint16_t *__restrict__ A,
    const uint16_t *__restrict__ B, int r, int r_pad, int ksp, float scale, uint16_t *__restrict__ h,
    float *__restrict__ u_out, float *__restrict__ upart, uint32_t *__restrict__ sync, Nf4Consts c) {
  constexpr int kThreads = 64 * kW;
  extern __shared__ __attribute__((aligned(16))) uint16_t x_l[];  // [T][d_in + kXPad] when kXL
  __shared__ float red[kW][256];
  __shared__ __attribute__((aligned(16))) uint16_t su_l[16 * kMaxRpad];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int li = lane & 15, g = lane >> 4;
  const int P = r > 0 ? (r_pad / 16) * ksp : 0;
  const int KB = d_in / kBlock;
  const int cid = blockIdx.x, G = gridDim.x;
  const rsrc_t xr = make_rsrc(x, (int64_t)T * d_in * 2);
  const int xpitch = d_in + kXPad;

  // ---------------- items: (row tile k, segment s) of this wave ----------------
  const int RT = (d_out + 15) / 16;
  const int nrt = cid < RT ? (RT - cid + G - 1) / G : 0;
  const int NS = (KB + 3) / 4;
  const int mseg = NS > wave ? (NS - wave + kW - 1) / kW : 0;  // my segments per row tile
  const uint32_t lane_code = (uint32_t)(li * (d_in / 2) + g * (kBlock / 2));
  const uint32_t lane_q2 = (uint32_t)(li * KB + g);
  const int64_t ngroups = ((int64_t)d_out * KB + kGroup - 1) / kGroup;

  auto load_codes = [&](int k, int s, GemvCodes &st) {
    const int row0 = (cid + k * G) * 16;
    const bool krow = k < nrt;
    const int rows = krow ? (d_out - row0 < 16 ? d_out - row0 : 16) : 0;
    const int kb0 = 4 * (wave + kW * s);  // first block of the segment
    const bool ok = kb0 + g < KB && li < rows;
    const int64_t rb = krow ? row0 : 0;
    const rsrc_t cr = make_rsrc(codes + rb * (d_in / 2), (int64_t)rows * (d_in / 2));
    const uint32_t coff = ok ? lane_code + (uint32_t)kb0 * (kBlock / 2) : kOOB;
    st.c0 = bld16(cr, coff);
    st.c1 = bld16(cr, coff + 16);
    const rsrc_t qr = make_rsrc(qscale + rb * KB, (int64_t)rows * KB);
    st.q2 = bld8(qr, ok ? lane_q2 + (uint32_t)kb0 : kOOB);
    // group maximum of block (row0 + li, kb0 + g), range rebased at the row tile's first group
    const int64_t blk0 = rb * KB;
    const rsrc_t sr = make_rsrc(smax + (blk0 >> 8), (ngroups - (blk0 >> 8)) * 4);
    const uint32_t rel = (uint32_t)(blk0 & (kGroup - 1)) + (uint32_t)(li * KB) + (uint32_t)(kb0 + g);
    st.S = __uint_as_float(bld32(sr, ok ? (rel >> 8) * 4 : kOOB));
  };
  auto load_x = [&](int s, GemvX &st) {
    const int kbl = 4 * (wave + kW * s) + g;
    const uint32_t xoff = kbl < KB ? (uint32_t)((li * d_in + kbl * kBlock) * 2) : kOOB;
#pragma unroll
    for (int m = 0; m < 8; ++m) st.x[m] = bld16(xr, xoff + 16 * m);
  };

  // ---------------- first loads, handshake read ----------------
  GemvCodes ca, cb;
  GemvX xa, xb;
  if (mseg > 0) {
    load_codes(0, 0, ca);
    if (!kXL) load_x(0, xa);
  }
  uint32_t ready = 1;
  u32x4 bpre[2] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
  const rsrc_t br = make_rsrc(B, (int64_t)d_out * r * 2);
  auto load_b = [&](int k) {
    const int row0 = (cid + k * G) * 16;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int j = 32 * q + 8 * g;
      const bool ok = j < r && row0 + li < d_out && k < nrt;
      bpre[q] = bld16(br, ok ? (uint32_t)(((row0 + li) * r + j) * 2) : kOOB);
    }
  };
  if (P > 0 && wave == 0) {
    ready = ld_dev_u32(&sync[1]);
    load_b(0);
  }

  // ---------------- adapter producer job (first P workgroups) ----------------
  if (cid < P) {
    const int j = cid / ksp, ks = cid % ksp;
    const int nrow = r - 16 * j < 16 ? r - 16 * j : 16;
    const rsrc_t ar = make_rsrc(A + (int64_t)16 * j * d_in, (int64_t)nrow * d_in * 2);
    const int nk32 = d_in / 32;
    const int kb = nk32 * ks / ksp, ke = nk32 * (ks + 1) / ksp;
    f32x4 pacc = {0.f, 0.f, 0.f, 0.f};
    for (int k0 = kb + wave; k0 < ke; k0 += 4 * kW) {
      u32x4 a[4], b[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int k32 = k0 + kW * s;
        const uint32_t off = k32 < ke ? (uint32_t)((li * d_in + k32 * 32 + 8 * g) * 2) : kOOB;
        a[s] = bld16(xr, off);
        b[s] = bld16(ar, off);
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) pacc = mfma16(a[s], b[s], pacc);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][(4 * g + i) * 16 + li] = pacc[i];
    __syncthreads();
    if (tid < 256) {
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < kW; ++w) v += red[w][tid];
      const int t = tid >> 4, col = 16 * j + (tid & 15);
      st_dev(upart + (ks * 16 + t) * r_pad + col, v);
    }
    wait_vmem();
    __syncthreads();
    if (tid == 0) {
      const uint32_t prev = add_dev_u32(&sync[0], 1u);
      if (prev == (uint32_t)P - 1u) {
        st_dev_u32(&sync[0], 0u);
        st_dev_u32(&sync[1], 1u);
      }
    }
  }

  // ---------------- stage x in LDS ----------------
  if (kXL) {
    for (int c0 = tid * 8; c0 < d_in; c0 += kThreads * 8) {
      u32x4 v[16];
#pragma unroll
      for (int t = 0; t < 16; ++t) v[t] = bld16(xr, t < T ? (uint32_t)((t * d_in + c0) * 2) : kOOB);
#pragma unroll
      for (int t = 0; t < 16; ++t)
        if (t < T) st16(x_l + t * xpitch + c0, v[t]);
    }
    __syncthreads();
  }

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int s, const GemvCodes &cs, const GemvX &xs) {
    const Nf4Planes t = make_planes(c, restore_scale(cs.q2, cs.S));
    // LDS path: token rows >= T only feed accumulator rows that are never stored,
    // and a block past the row end has an all-zero restore table, so both read
    // clamped in-range x without masking.
    const int kbl = 4 * (wave + kW * s) + g;
    const uint16_t *xp = x_l + (li < T ? li : 0) * xpitch + (kbl < KB ? kbl : KB - 1) * kBlock;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const u32x4 a = kXL ? *reinterpret_cast<const u32x4 *>(xp + 8 * m) : xs.x[m];
      acc = mfma16(a, expand8(t, m < 4 ? cs.c0[m] : cs.c1[m - 4]), acc);
    }
  };

  // Row-tile epilogue: adapter columns (wave 0), LDS reduce across waves, store h.
  auto epilogue = [&](int k) {
    const int row0 = (cid + k * G) * 16;
    const int rows = d_out - row0 < 16 ? d_out - row0 : 16;
    if (P > 0 && k == 0) {
      // s*u for all rows of this workgroup: wave 0 waits for the producers, then
      // every thread sums a few entries over the K-slice partials in slice order
      // (deterministic) and stages bf16 s*u in LDS.
      if (wave == 0) {
        int it = 0;
        while (ready == 0u) {
          if (++it > kSpinLimit) {
            st_dev_u32(&sync[3], 1u);
            break;
          }
          __builtin_amdgcn_s_sleep(1);
          ready = ld_dev_u32(&sync[1]);
        }
      }
      __syncthreads();
      const rsrc_t ur = make_rsrc(upart, (int64_t)ksp * 16 * r_pad * 4);
      for (int e = tid; e < 16 * r_pad; e += kThreads) {
        const int t = e / r_pad, col = e - t * r_pad;
        float pv[kMaxKsp];
#pragma unroll
        for (int q = 0; q < kMaxKsp; ++q)
          pv[q] = __uint_as_float(bld32_dev(ur, q < ksp ? (uint32_t)(((q * 16 + t) * r_pad + col) * 4) : kOOB));
        float v = 0.f;
#pragma unroll
        for (int q = 0; q < kMaxKsp; ++q) v += pv[q];
        if (u_out && cid == 0 && t < T && col < r) u_out[t * r + col] = v;
        su_l[e] = (uint16_t)(pack_bf16x2((t < T && col < r) ? scale * v : 0.f, 0.f) & 0xffffu);
      }
      wait_vmem();
      __syncthreads();
      if (tid == 0) {
        const uint32_t prev = add_dev_u32(&sync[2], 1u);
        if (prev == (uint32_t)G - 1u) {
          st_dev_u32(&sync[2], 0u);
          st_dev_u32(&sync[1], 0u);
        }
      }
    }
    if (P > 0 && wave == 0) {
      // adapter K columns of this row tile: a = s*u (LDS), b = B rows
      for (int j0 = 0; j0 < r_pad; j0 += 32) {
        const int j = j0 + 8 * g;
        const u32x4 a = j < r_pad ? *reinterpret_cast<const u32x4 *>(su_l + li * r_pad + j) : u32x4{0u, 0u, 0u, 0u};
        u32x4 b;
        if (j0 < 64) {
          b = bpre[j0 >> 5];
        } else {
          const bool ok = j < r && row0 + li < d_out;
          b = bld16(br, ok ? (uint32_t)(((row0 + li) * r + j) * 2) : kOOB);
        }
        acc = mfma16(a, b, acc);
      }
      if (k + 1 < nrt) load_b(k + 1);
    }
    // Lane (li, g) holds tokens 4g..4g+3 of row li.
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][(4 * g + i) * 16 + li] = acc[i];
    acc = f32x4{0.f, 0.f, 0.f, 0.f};
    __syncthreads();
    if (tid < 256) {
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < kW; ++w) v += red[w][tid];
      const int t = tid >> 4, rl = tid & 15;
      if (t < T && rl < rows) h[t * d_out + row0 + rl] = (uint16_t)(pack_bf16x2(v, 0.f) & 0xffffu);
    }
    __syncthreads();
  };

  if (mseg == 0) {
    for (int k = 0; k < nrt; ++k) epilogue(k);
  } else {
    // Two stages in ping-pong: compute one item while the next one's loads fly.
    int k = 0, s = 0;
    while (true) {
      int k2 = k, s2 = s + 1;
      if (s2 == mseg) { s2 = 0; ++k2; }
      load_codes(k2, s2, cb);
      if (!kXL) load_x(s2, xb);
      compute(s, ca, xa);
      if (s == mseg - 1) epilogue(k);
      k = k2, s = s2;
      if (k >= nrt) break;

      k2 = k, s2 = s + 1;
      if (s2 == mseg) { s2 = 0; ++k2; }
      load_codes(k2, s2, ca);
      if (!kXL) load_x(s2, xa);
      compute(s, cb, xb);
      if (s == mseg - 1) epilogue(k);
      k = k2, s = s2;
      if (k >= nrt) break;
    }
  }
  if (P > 0 && nrt == 0 && tid == 0) {
    // a workgroup without rows still takes part in the handshake count
    const uint32_t prev = add_dev_u32(&sync[2], 1u);
    if (prev == (uint32_t)G - 1u) {
      st_dev_u32(&sync[2], 0u);
      st_dev_u32(&sync[1], 0u);
    }
  }
}

#ifndef QLORA_GEMV_WAVES
#define QLORA_GEMV_WAVES 8
#endif
constexpr int kGvW = QLORA_GEMV_WAVES;  // waves per workgroup

int gemv_ksplit(int64_t d_in) {
  // one batch of <= 4 K steps per producer wave where possible
  int64_t ksp = (d_in / 32 + 4 * kGvW - 1) / (4 * kGvW);
  if (ksp < 1) ksp = 1;
  if (ksp > kMaxKsp) ksp = kMaxKsp;
  return (int)ksp;
}

static int g_gemv_cus[64];
static bool g_gemv_attr[64];

static int device_index() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return -1;
  return dev;
}

static int device_cus(int dev) {
  if (dev < 0) return 256;
  if (g_gemv_cus[dev] > 0) return g_gemv_cus[dev];
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) return 256;
  g_gemv_cus[dev] = cus;
  return cus;
}

hipError_t launch_gemv_fwd(const uint8_t *codes, const uint8_t *qscale, const float *smax, int64_t d_out,
                           int64_t d_in, const uint16_t *x, int64_t T, const uint16_t *A, const uint16_t *B, int r,
                           int r_pad, float scale, uint16_t *h, float *u_out, float *upart, uint32_t *sync,
                           const Nf4Consts &c, hipStream_t st) {
  if (r_pad > kMaxRpad) return hipErrorInvalidValue;
  const int dev = device_index();
  const int ksp = gemv_ksplit(d_in);
  const int P = r > 0 ? (r_pad / 16) * ksp : 0;
  const int64_t RT = (d_out + 15) / 16;
  // One workgroup per CU; the first P of them also produce x A^T. The grid never
  // exceeds one residency, so every workgroup runs concurrently.
  int64_t G = RT < device_cus(dev) ? RT : device_cus(dev);
  if (G < P) G = P;
  const size_t xbytes = (size_t)T * (d_in + kXPad) * 2;
  const int di = (int)d_in, dn = (int)d_out, Tt = (int)T;
  if (xbytes <= (size_t)kXLdsBytes) {
    if (dev >= 0 && !g_gemv_attr[dev]) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(k_gemv_fwd<kGvW, true>),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, kXLdsBytes);
      if (e != hipSuccess) return e;
      g_gemv_attr[dev] = true;
    }
    k_gemv_fwd<kGvW, true><<<dim3((unsigned)G), dim3(64 * kGvW), xbytes, st>>>(
        codes, qscale, smax, dn, di, x, Tt, A, B, r, r_pad, ksp, scale, h, u_out, upart, sync, c);
  } else {
    k_gemv_fwd<kGvW, false><<<dim3((unsigned)G), dim3(64 * kGvW), 0, st>>>(
        codes, qscale, smax, dn, di, x, Tt, A, B, r, r_pad, ksp, scale, h, u_out, upart, sync, c);
  }
  return hipGetLastError();
}

}  // namespace qlora
