// Forward for T <= 16 tokens: stream the 4.13-bit weight once from HBM.
//
// h[T, d_out] = x W_hat^T + su B^T   ("QLoRA의 수식": the restored frozen base
// plus the adapter term; su = bf16(alpha/r * x A^T) comes from k_lora_small).
//
// Every weight is used by at most 16 tokens, so the kernel is bound by the
// packed-weight stream (0.516 bytes per weight). Work decomposition:
//   * a workgroup (4 waves) owns 64 output rows and one K slice (ksplit slices
//     per row; the last workgroup of a row tile sums the slices in order);
//   * each wave takes all 64 rows (4 groups of 16 rows = the N side of
//     v_mfma_f32_16x16x32_bf16; tokens are the M side, padded to 16) over its
//     share of 256-wide K segments, so one x fragment feeds four MFMAs;
//   * in a segment, lane (row, g) owns one whole 64-weight block (its 32 bytes
//     of codes arrive as two 16-byte loads) and builds that block's 16-entry
//     restore table once; the 8 MFMAs of the segment take 8 weights per lane
//     each, expanded from nibbles with v_perm byte selects. The MFMA's K order
//     is permuted identically on both operands (x_slots / expand8).
#include "kernels.h"

namespace qlora {

__global__ __launch_bounds__(256) void k_gemv_fwd(const uint8_t *__restrict__ codes, const uint8_t *__restrict__ qscale,
                                                  const float *__restrict__ smax, int64_t d_out, int64_t d_in,
                                                  const uint16_t *__restrict__ x, int64_t T,
                                                  const uint16_t *__restrict__ su, int r_pad,
                                                  const uint16_t *__restrict__ B, int r, uint16_t *__restrict__ h,
                                                  float *__restrict__ partial, uint32_t *__restrict__ counters,
                                                  int ksplit, Nf4Consts c) {
  __shared__ float red[4][16][64];
  __shared__ int is_last;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, g = lane >> 4;
  const int64_t row0 = (int64_t)blockIdx.x * 64;
  const int split = blockIdx.y;
  const int64_t KB = d_in / kBlock;
  const int64_t NS = (KB + 3) / 4;
  const int64_t sb = NS * split / ksplit, se = NS * (split + 1) / ksplit;

  f32x4 acc[4];
#pragma unroll
  for (int rg = 0; rg < 4; ++rg) acc[rg] = f32x4{0.f, 0.f, 0.f, 0.f};

  const bool tok_ok = li < T;
  for (int64_t seg = sb + wave; seg < se; seg += 4) {
    const int64_t kblk = seg * 4 + g;
    const bool k_ok = kblk < KB;
    u32x4 xf[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      xf[m] = u32x4{0u, 0u, 0u, 0u};
      if (tok_ok && k_ok) xf[m] = x_slots(ld16(x + li * d_in + kblk * kBlock + 8 * m));
    }
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int64_t n = row0 + rg * 16 + li;
      u32x4 c0 = {0u, 0u, 0u, 0u}, c1 = {0u, 0u, 0u, 0u};
      float sh = 0.f;
      if (n < d_out && k_ok) {
        const uint8_t *cp = codes + n * (d_in / 2) + kblk * (kBlock / 2);
        c0 = ld16(cp);
        c1 = ld16(cp + 16);
        const int64_t blk = n * KB + kblk;
        sh = restore_scale(qscale[blk], smax[blk >> 8]);
      }
      const Nf4Planes t = make_planes(c, sh);
#pragma unroll
      for (int m = 0; m < 4; ++m) acc[rg] = mfma16(xf[m], expand8(t, c0[m]), acc[rg]);
#pragma unroll
      for (int m = 0; m < 4; ++m) acc[rg] = mfma16(xf[4 + m], expand8(t, c1[m]), acc[rg]);
    }
  }

  // Adapter term as extra K columns, added once per row tile (wave 0 of split 0;
  // the waves' accumulators are summed below).
  if (split == 0 && wave == 0 && r > 0) {
    for (int j0 = 0; j0 < r_pad; j0 += 32) {
      const int j = j0 + 8 * g;
      u32x4 a = {0u, 0u, 0u, 0u};
      if (j < r_pad) a = ld16(su + li * r_pad + j);
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int64_t n = row0 + rg * 16 + li;
        u32x4 b = {0u, 0u, 0u, 0u};
        if (n < d_out && j < r) b = ld16(B + n * r + j);
        acc[rg] = mfma16(a, b, acc[rg]);
      }
    }
  }

  // Lane (li, g) holds tokens 4g..4g+3 of row rg*16+li.
#pragma unroll
  for (int rg = 0; rg < 4; ++rg)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][4 * g + i][rg * 16 + li] = acc[rg][i];
  __syncthreads();

  const int tt = tid >> 4, n4 = (tid & 15) * 4;  // token, 4 consecutive rows
  f32x4 v;
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = red[0][tt][n4 + e] + red[1][tt][n4 + e] + red[2][tt][n4 + e] + red[3][tt][n4 + e];

  if (ksplit > 1) {
    float *pp = partial + ((int64_t)blockIdx.x * ksplit + split) * 1024;
    *reinterpret_cast<f32x4 *>(pp + tt * 64 + n4) = v;
    __threadfence();
    __syncthreads();
    if (tid == 0) {
      const uint32_t prev = atomicAdd(&counters[blockIdx.x], 1u);
      is_last = (prev == (uint32_t)ksplit - 1u);
    }
    __syncthreads();
    if (!is_last) return;
    __threadfence();
    const float *pb = partial + (int64_t)blockIdx.x * ksplit * 1024 + tt * 64 + n4;
    v = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < ksplit; ++s) {
      const f32x4 p = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(pb + (int64_t)s * 1024));
      v += p;
    }
    if (tid == 0) counters[blockIdx.x] = 0u;
  }
  if (tt < T) {
    const int64_t n = row0 + n4;
    uint16_t *hp = h + tt * d_out + n;
    if (n + 3 < d_out) {
      u32x2 o = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      *reinterpret_cast<u32x2 *>(hp) = o;
    } else {
      for (int e = 0; e < 4; ++e)
        if (n + e < d_out) hp[e] = (uint16_t)(pack_bf16x2(v[e], 0.f) & 0xffffu);
    }
  }
}

int gemv_ksplit(int64_t d_out, int64_t d_in) {
  const int64_t RT = (d_out + 63) / 64;
  const int64_t NS = (d_in / kBlock + 3) / 4;
  int ks = 1;
  if (RT > kMaxCounters) return 1;
  while (RT * ks * 2 <= 512 && 4 * ks * 2 <= NS) ks *= 2;
  return ks;
}

hipError_t launch_gemv_fwd(const uint8_t *codes, const uint8_t *qscale, const float *smax, int64_t d_out,
                           int64_t d_in, const uint16_t *x, int64_t T, const uint16_t *su, int r_pad,
                           const uint16_t *B, int r, uint16_t *h, float *partial, uint32_t *counters, int ksplit,
                           const Nf4Consts &c, hipStream_t st) {
  dim3 grid((unsigned)((d_out + 63) / 64), (unsigned)ksplit);
  k_gemv_fwd<<<grid, dim3(256), 0, st>>>(codes, qscale, smax, d_out, d_in, x, T, su, r_pad, B, r, h, partial,
                                         counters, ksplit, c);
  return hipGetLastError();
}

}  // namespace qlora
