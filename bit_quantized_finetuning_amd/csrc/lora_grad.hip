// Adapter gradients: dA = s v^T x and dB = s dY^T u (reduction over tokens).
//
// First page, "QLoRA의 수식" and "명제 1": the adapter path (alpha/r) B A x is
// fully differentiable and its gradients land on A and B only. With
// u = x A^T and v = dY B:
//     dA[r, d_in]  = s * sum_t v[t, :]^T x[t, :]
//     dB[d_out, r] = s * sum_t dY[t, :]^T u[t, :]
// Both are C[M, N] = s * sum_t P[t, m] Q[t, n] with P and Q stored token-major, so
// both MFMA operands need 8 consecutive tokens per lane: the 64-token tiles are
// staged in LDS as loaded and gathered with 16-bit reads. A float32 operand (v or
// u) is split into hi + lo bf16 parts (two MFMAs), which keeps the product
// accurate to ~2^-16 relative instead of bf16's 2^-8.
//
// These products are HBM-bound on their own (arithmetic intensity ~ r flop per
// byte). Tokens are split across workgroups; the last workgroup of an output
// tile (device-scope counter) adds the float32 partial tiles in split order, so
// the result is deterministic. Partials travel through device-scope stores and
// loads (no cache-wide fence); operand tails are read as zeros by buffer loads.
#include "kernels.h"

namespace qlora {

constexpr int kGT = 64;         // tile edge (M, N) and token step
constexpr int kGP = kGT + 8;    // LDS pitch (bf16)

template <bool kPf32, bool kQf32>
__global__ __launch_bounds__(256) void k_lora_grad(const void *__restrict__ Pv, int64_t M, const void *__restrict__ Qv,
                                                   int64_t N, int64_t T, float scale, float *__restrict__ C,
                                                   float *__restrict__ partial, uint32_t *__restrict__ counters,
                                                   int ksplit, int tiles_n) {
  __shared__ __attribute__((aligned(16))) uint16_t Ph[kGT * kGP], Pl[kPf32 ? kGT * kGP : 1];
  __shared__ __attribute__((aligned(16))) uint16_t Qh[kGT * kGP], Ql[kQf32 ? kGT * kGP : 1];
  __shared__ int is_last;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wm = wave & 1, wn = wave >> 1;
  const int tile = blockIdx.x, split = blockIdx.y;
  const int64_t m0 = (int64_t)(tile / tiles_n) * kGT, n0 = (int64_t)(tile % tiles_n) * kGT;
  const int64_t nkt = (T + kGT - 1) / kGT;
  const int64_t kb = nkt * split / ksplit, ke = nkt * (split + 1) / ksplit;

  const int lr = tid >> 2, lc = (tid & 3) * 16;  // loader: token row, 16 columns

  // Stage rows t0..t0+63 of a token-major operand (cols wide) as bf16 (hi [+ lo]).
  auto stage = [&](const void *src, bool f32, int64_t cols, int64_t c0, int64_t t0, uint16_t *hi, uint16_t *lo) {
    const int esz = f32 ? 4 : 2;
    const int64_t nrow = T - t0 < kGT ? T - t0 : kGT;
    const rsrc_t rs = make_rsrc(static_cast<const uint8_t *>(src) + t0 * cols * esz, nrow * cols * esz);
    uint16_t *dh = hi + lr * kGP + lc;
    if (f32) {
      f32x4 v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t cc = c0 + lc + 4 * q;
        const u32x4 w = bld16(rs, cc < cols ? (uint32_t)((lr * cols + cc) * 4) : kOOB);
        v[q] = f32x4{__uint_as_float(w[0]), __uint_as_float(w[1]), __uint_as_float(w[2]), __uint_as_float(w[3])};
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t h0 = pack_bf16x2(v[q][0], v[q][1]), h1 = pack_bf16x2(v[q][2], v[q][3]);
        uint32_t l0 = pack_bf16x2(v[q][0] - bf16_lo_to_f32(h0), v[q][1] - bf16_hi_to_f32(h0));
        uint32_t l1 = pack_bf16x2(v[q][2] - bf16_lo_to_f32(h1), v[q][3] - bf16_hi_to_f32(h1));
        *reinterpret_cast<u32x2 *>(dh + 4 * q) = u32x2{h0, h1};
        *reinterpret_cast<u32x2 *>(lo + lr * kGP + lc + 4 * q) = u32x2{l0, l1};
      }
    } else {
      u32x4 v[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int64_t cc = c0 + lc + 8 * q;
        v[q] = bld16(rs, cc < cols ? (uint32_t)((lr * cols + cc) * 2) : kOOB);
      }
#pragma unroll
      for (int q = 0; q < 2; ++q) st16(dh + 8 * q, v[q]);
    }
  };

  f32x16 acc;
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;

  // fragment: lane (x = l%32, g = l/32) takes rows 16*k16 + 8g + 0..7 of column x
  auto frag = [&](const uint16_t *base, int col0, int k16) {
    const uint16_t *p = base + (16 * k16 + 8 * (lane >> 5)) * kGP + col0 + (lane & 31);
    u32x4 f;
#pragma unroll
    for (int e = 0; e < 4; ++e) f[e] = (uint32_t)p[(2 * e) * kGP] | ((uint32_t)p[(2 * e + 1) * kGP] << 16);
    return f;
  };

  for (int64_t kt = kb; kt < ke; ++kt) {
    stage(Pv, kPf32, M, m0, kt * kGT, Ph, Pl);
    stage(Qv, kQf32, N, n0, kt * kGT, Qh, Ql);
    __syncthreads();
#pragma unroll
    for (int k16 = 0; k16 < kGT / 16; ++k16) {
      const u32x4 ah = frag(Ph, wm * 32, k16);
      const u32x4 bh = frag(Qh, wn * 32, k16);
      acc = mfma32(ah, bh, acc);
      if (kPf32) acc = mfma32(frag(Pl, wm * 32, k16), bh, acc);
      if (kQf32) acc = mfma32(ah, frag(Ql, wn * 32, k16), acc);
    }
    __syncthreads();
  }

  // lane l, accumulator e -> row wm*32 + 8(e/4) + 4(l/32) + e%4, column wn*32 + l%32
  const int cn = wn * 32 + (lane & 31);
  if (ksplit == 1) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int64_t m = m0 + wm * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3), n = n0 + cn;
      if (m < M && n < N) C[m * N + n] = scale * acc[e];
    }
    return;
  }
  float *pp = partial + ((int64_t)tile * ksplit + split) * (kGT * kGT);
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int rm = wm * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
    st_dev(pp + rm * kGT + cn, acc[e]);
  }
  wait_vmem();
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev = add_dev_u32(tile_counter(counters, tile), 1u);
    is_last = (prev == (uint32_t)ksplit - 1u);
  }
  __syncthreads();
  if (!is_last) return;
  const float *pb = partial + (int64_t)tile * ksplit * (kGT * kGT);
  for (int q = tid; q < kGT * kGT / 4; q += 256) {
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < ksplit; ++s) {
      const float *ps = pb + (int64_t)s * kGT * kGT + 4 * q;
      v += f32x4{ld_dev(ps), ld_dev(ps + 1), ld_dev(ps + 2), ld_dev(ps + 3)};
    }
    const int rm = (4 * q) / kGT, rn = (4 * q) % kGT;
    const int64_t m = m0 + rm;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t n = n0 + rn + e;
      if (m < M && n < N) C[m * N + n] = scale * v[e];
    }
  }
  if (tid == 0) st_dev_u32(tile_counter(counters, tile), 0u);
}

int lora_grad_tiles(int64_t M, int64_t N) { return (int)(((M + kGT - 1) / kGT) * ((N + kGT - 1) / kGT)); }

int lora_grad_ksplit(int64_t M, int64_t N, int64_t T) {
  const int64_t tiles = lora_grad_tiles(M, N);
  const int64_t nkt = (T + kGT - 1) / kGT;
  if (tiles > kMaxTileCounters) return 1;
  int64_t ks = (512 + tiles - 1) / tiles;
  if (ks > nkt / 2) ks = nkt / 2;
  if (ks < 1) ks = 1;
  return (int)ks;
}

size_t lora_grad_partial_floats(int64_t M, int64_t N, int64_t T) {
  const int ks = lora_grad_ksplit(M, N, T);
  return ks > 1 ? (size_t)lora_grad_tiles(M, N) * ks * kGT * kGT : 0;
}

hipError_t launch_lora_grad(const void *P, bool P_f32, int64_t M, const void *Q, bool Q_f32, int64_t N, int64_t T,
                            float scale, float *C, float *partial, uint32_t *counters, int ksplit, hipStream_t st) {
  const int tiles_n = (int)((N + kGT - 1) / kGT);
  dim3 grid((unsigned)lora_grad_tiles(M, N), (unsigned)ksplit);
  if (P_f32 && !Q_f32)
    k_lora_grad<true, false><<<grid, dim3(256), 0, st>>>(P, M, Q, N, T, scale, C, partial, counters, ksplit, tiles_n);
  else if (!P_f32 && Q_f32)
    k_lora_grad<false, true><<<grid, dim3(256), 0, st>>>(P, M, Q, N, T, scale, C, partial, counters, ksplit, tiles_n);
  else if (P_f32 && Q_f32)
    k_lora_grad<true, true><<<grid, dim3(256), 0, st>>>(P, M, Q, N, T, scale, C, partial, counters, ksplit, tiles_n);
  else
    k_lora_grad<false, false><<<grid, dim3(256), 0, st>>>(P, M, Q, N, T, scale, C, partial, counters, ksplit, tiles_n);
  return hipGetLastError();
}

}  // namespace qlora
