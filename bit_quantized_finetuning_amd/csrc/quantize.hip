// NF4 blockwise quantization with double quantization, and the standalone restore.
//
// Quantize ("48GB GPU Fine-Tuning a 65B Model", section "Quantization Keeps the
// Patterns and Reduces Bits per Number"): per block of 64 weights the scale is
// the largest |w|; each weight is divided by it and replaced by the index of the
// nearest of the 16 NF4 levels. Double quantization (first page, section
// "메모리 회계"): the block scales are re-coded to 8 bits against their group
// maximum so that they come back as (q2/256) * S.
//
// One workgroup owns one group of 256 blocks (16384 weights). Eight lanes share
// a block: each loads 8 consecutive weights (32 contiguous bytes of float32, the
// eight lanes together 256 contiguous bytes), the eight reduce the block absmax
// with lane shuffles, and each lane emits its weights' codes as one packed
// 32-bit word. All eight passes' loads are issued before any arithmetic. The
// block scales wait in LDS for the group maximum, then one thread per block
// writes its 8-bit scale code. The kernel streams 4 (or 2) bytes in and ~0.52
// bytes out per weight.
//
// Nearest level: the index is the number of the 15 float32 thresholds at or
// below x = w/s (x is in [-1, 1]). Instead of 15 comparisons per weight, x's
// float32 bits pick one of 64 buckets: sign, binade (2^-5 .. 1 in six steps,
// everything smaller in one) and the top two significand bits. No bucket
// holds more than one threshold, so the count is the bucket's base count
// plus one comparison with its threshold (+inf where it has none). The
// buckets are built per workgroup from the thresholds; checked against the
// plain count for every float32 in [-1, 1]. For absmax-only storage (sshift 0) each block's float32
// absmax is written as its scale instead, and there is no group step.
#include "kernels.h"

namespace qlora {

template <bool kBf16In>
__global__ __launch_bounds__(256) void k_quantize(const void *__restrict__ W, int64_t nblocks,
                                                  uint8_t *__restrict__ codes, uint8_t *__restrict__ qscale,
                                                  float *__restrict__ smax, uint32_t *__restrict__ flags,
                                                  int sshift, Nf4Consts c) {
  constexpr int esz = kBf16In ? 2 : 4;
  constexpr int kPasses = kGroup / 32;
  __shared__ float s_blk[kGroup];
  __shared__ float s_red[4];
  __shared__ float2 bucket[64];  // {threshold inside the bucket or +inf, count of thresholds below it}
  const int tid = threadIdx.x;
  const int64_t b0 = (int64_t)blockIdx.x * kGroup;
  const int nb = (int)(nblocks - b0 < kGroup ? nblocks - b0 : kGroup);
  const int l8 = tid & 7;
  const int slot = tid >> 3;  // 32 blocks per pass
  const rsrc_t wr = make_rsrc(static_cast<const uint8_t *>(W) + b0 * kBlock * esz, (int64_t)nb * kBlock * esz);

  u32x4 raw[kPasses][kBf16In ? 1 : 2];
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const int b = p * 32 + slot;
    const uint32_t off = b < nb ? (uint32_t)((b * kBlock + l8 * 8) * esz) : kOOB;
    raw[p][0] = bld16(wr, off);
    if (!kBf16In) raw[p][kBf16In ? 0 : 1] = bld16(wr, off + 16);
  }

  // Bucket b = sign * 32 + e * 4 + m covers magnitudes [lo, hi): e = 0 is
  // [0, 2^-5); e = 1 .. 6 the binade [2^(e-6), 2^(e-5)) cut into quarters by m.
  // A positive x in it has every threshold <= lo below it and can pass one in
  // (lo, hi); a negative x (in (-hi, -lo]) has every threshold <= -hi below it
  // and can pass one in (-hi, -lo].
  if (tid < 64) {
    const int sg = tid >> 5, e = (tid >> 2) & 7, m = tid & 3;
    float lo = 0.f, hi = 0.03125f;
    if (e > 0) {
      const float b = __builtin_ldexpf(1.f, e - 6);
      lo = b + 0.25f * b * (float)m;  // exact
      hi = b + 0.25f * b * (float)(m + 1);
    }
    float cand = __builtin_inff();
    int below = 0;
#pragma unroll
    for (int j = 0; j < 15; ++j) {
      const float t = c.thr[j];
      if (sg == 0) {
        below += t <= lo;
        if (t > lo && t < hi) cand = t;
      } else {
        below += t <= -hi;
        if (t > -hi && t <= -lo) cand = t;
      }
    }
    bucket[tid] = make_float2(cand, (float)below);
  }
  __syncthreads();

  uint32_t bad = 0;
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const int b = p * 32 + slot;
    float w[8];
    if (kBf16In) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        w[2 * e] = bf16_lo_to_f32(raw[p][0][e]);
        w[2 * e + 1] = bf16_hi_to_f32(raw[p][0][e]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        w[e] = __uint_as_float(raw[p][0][e]);
        w[4 + e] = __uint_as_float(raw[p][kBf16In ? 0 : 1][e]);
      }
    }
    float m = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      bad |= !__builtin_isfinite(w[e]);
      m = fmaxf(m, fabsf(w[e]));
    }
#pragma unroll
    for (int off = 1; off < 8; off <<= 1) m = fmaxf(m, __shfl_xor(m, off, 8));
    uint32_t word = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = m > 0.f ? w[e] / m : 0.f;  // IEEE float32 divide
      const uint32_t xb = __float_as_uint(x);
      const int be = min(max((int)((xb >> 23) & 0xffu) - 121, 0), 6);
      const float2 bk = bucket[((xb >> 31) << 5) | ((uint32_t)be << 2) | ((xb >> 21) & 3u)];
      const uint32_t q = (uint32_t)bk.y + (x >= bk.x ? 1u : 0u);
      word |= q << nibble_shift(e);
    }
    if (b < nb) {
      if (l8 == 0) s_blk[b] = m;
      *reinterpret_cast<uint32_t *>(codes + (b0 + b) * (kBlock / 2) + l8 * 4) = word;
    }
  }
  __syncthreads();

  const float s = tid < nb ? s_blk[tid] : 0.f;
  if (sshift == 0) {  // absmax-only storage: the block scales as they are
    if (tid < nb) smax[b0 + tid] = s;
    if (bad && flags) atomicOr(flags, 1u);
    return;
  }
  float S = s;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) S = fmaxf(S, __shfl_xor(S, off));
  if ((tid & 63) == 0) s_red[tid >> 6] = S;
  __syncthreads();
  S = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  if (tid < nb) {
    uint32_t q2 = 0;
    if (S > 0.f) {
      const float ratio = s / S;             // fl32(s / S)
      const float v = rintf(ratio * 256.f);  // exact scale, ties to even
      q2 = (uint32_t)fminf(v, 255.f);
    }
    qscale[b0 + tid] = (uint8_t)q2;
  }
  if (tid == 0) smax[blockIdx.x] = S;
  if (bad && flags) atomicOr(flags, 1u);
}

// Restore: one thread per 8 weights (one packed word). float32 output is the
// unrounded product c[q] * s_hat; bf16 output goes through the same byte-plane
// table expansion the matmul kernels use, so checking it bit for bit checks
// their dequantization as well.
template <bool kBf16Out>
__global__ __launch_bounds__(256) void k_dequantize(const uint32_t *__restrict__ codes,
                                                    const uint8_t *__restrict__ qscale,
                                                    const float *__restrict__ smax, int64_t n8,
                                                    void *__restrict__ out, int sshift, Nf4Consts c) {
  __shared__ float cb[16];
  if (threadIdx.x == 0) {
#pragma unroll
    for (int j = 0; j < 16; ++j) cb[j] = c.code[j];
  }
  __syncthreads();
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8; i += stride) {
    const uint32_t cw = codes[i];
    const int64_t blk = i >> 3;
    const float sh = sshift ? restore_scale(qscale[blk], smax[blk >> kDqShift]) : smax[blk];
    if (kBf16Out) {
      const Nf4Planes t = make_planes(sh);
      st16(static_cast<uint16_t *>(out) + i * 8, expand8(t, cw));
    } else {
      f32x4 a, b;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a[e] = cb[(cw >> nibble_shift(e)) & 15u] * sh;
        b[e] = cb[(cw >> nibble_shift(e + 4)) & 15u] * sh;
      }
      float *o = static_cast<float *>(out) + i * 8;
      *reinterpret_cast<f32x4 *>(o) = a;
      *reinterpret_cast<f32x4 *>(o + 4) = b;
    }
  }
}

hipError_t launch_quantize(const void *W, bool bf16_in, int64_t d_out, int64_t d_in, uint8_t *codes,
                           uint8_t *qscale, float *smax, uint32_t *flags, const Nf4Consts &c,
                           hipStream_t st) {
  const int64_t nblocks = d_out * d_in / kBlock;
  const int64_t ngroups = (nblocks + kGroup - 1) / kGroup;
  const int sshift = qscale ? kDqShift : 0;
  if (bf16_in)
    k_quantize<true><<<dim3((unsigned)ngroups), dim3(256), 0, st>>>(W, nblocks, codes, qscale, smax, flags, sshift,
                                                                    c);
  else
    k_quantize<false><<<dim3((unsigned)ngroups), dim3(256), 0, st>>>(W, nblocks, codes, qscale, smax, flags, sshift,
                                                                     c);
  return hipGetLastError();
}

hipError_t launch_dequantize(const uint8_t *codes, const uint8_t *qscale, const float *smax, int64_t d_out,
                             int64_t d_in, bool bf16_out, void *out, const Nf4Consts &c, hipStream_t st) {
  const int64_t n8 = d_out * d_in / 8;
  int64_t grid = (n8 + 255) / 256;
  if (grid > 65536) grid = 65536;
  const uint32_t *cw = reinterpret_cast<const uint32_t *>(codes);
  const int sshift = qscale ? kDqShift : 0;
  if (bf16_out)
    k_dequantize<true><<<dim3((unsigned)grid), dim3(256), 0, st>>>(cw, qscale, smax, n8, out, sshift, c);
  else
    k_dequantize<false><<<dim3((unsigned)grid), dim3(256), 0, st>>>(cw, qscale, smax, n8, out, sshift, c);
  return hipGetLastError();
}

}  // namespace qlora
