// NF4 blockwise quantization with double quantization, and the standalone restore.
//
// Quantize ("48GB GPU Fine-Tuning a 65B Model", section "Quantization Keeps the
// Patterns and Reduces Bits per Number"): per block of 64 weights the scale is
// the largest |w|; each weight is divided by it and replaced by the index of the
// nearest of the 16 NF4 levels. Double quantization (first page, section
// "메모리 회계"): the block scales are re-coded to 8 bits against their group
// maximum so that they come back as (q2/256) * S.
//
// One workgroup owns one group of 256 blocks (16384 weights): a 16-lane slice
// reduces the absmax of one 64-weight block (4 weights per lane, 256 contiguous
// bytes per slice for float32 input), writes that block's 32 bytes of codes, and
// parks the block scale in LDS; the workgroup then takes the group maximum and
// writes the 256 scale codes. The kernel is HBM-bound (4 or 2 bytes read per
// weight, 0.52 written).
#include "kernels.h"

namespace qlora {

template <bool kBf16In>
__global__ __launch_bounds__(256) void k_quantize(const void *__restrict__ W, int64_t nblocks,
                                                  uint8_t *__restrict__ codes, uint8_t *__restrict__ qscale,
                                                  float *__restrict__ smax, uint32_t *__restrict__ flags,
                                                  Nf4Consts c) {
  __shared__ float s_blk[kGroup];
  __shared__ float s_red[4];
  const int tid = threadIdx.x;
  const int64_t b0 = (int64_t)blockIdx.x * kGroup;
  const int nb = (int)(nblocks - b0 < kGroup ? nblocks - b0 : kGroup);
  const int l16 = tid & 15;
  const int slot = tid >> 4;
  uint32_t bad = 0;

  for (int pass = 0; pass < kGroup / 16; ++pass) {
    const int b = pass * 16 + slot;
    if (b >= nb) break;  // uniform across the 16-lane slice
    const int64_t e0 = (b0 + b) * kBlock + l16 * 4;
    float w[4];
    if (kBf16In) {
      const u32x2 v = *reinterpret_cast<const u32x2 *>(static_cast<const uint16_t *>(W) + e0);
      w[0] = bf16_lo_to_f32(v[0]);
      w[1] = bf16_hi_to_f32(v[0]);
      w[2] = bf16_lo_to_f32(v[1]);
      w[3] = bf16_hi_to_f32(v[1]);
    } else {
      const f32x4 v = *reinterpret_cast<const f32x4 *>(static_cast<const float *>(W) + e0);
      w[0] = v[0];
      w[1] = v[1];
      w[2] = v[2];
      w[3] = v[3];
    }
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bad |= !__builtin_isfinite(w[i]);
      m = fmaxf(m, fabsf(w[i]));
    }
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) m = fmaxf(m, __shfl_xor(m, off, 16));
    if (l16 == 0) s_blk[b] = m;

    uint32_t packed = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float x = m > 0.f ? w[i] / m : 0.f;  // IEEE float32 divide
      uint32_t q = 0;
#pragma unroll
      for (int j = 0; j < 15; ++j) q += (x >= c.thr[j]) ? 1u : 0u;
      packed |= q << (4 * i);
    }
    *reinterpret_cast<uint16_t *>(codes + (b0 + b) * (kBlock / 2) + l16 * 2) = (uint16_t)packed;
  }
  __syncthreads();

  const float s = tid < nb ? s_blk[tid] : 0.f;
  float S = s;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) S = fmaxf(S, __shfl_xor(S, off));
  if ((tid & 63) == 0) s_red[tid >> 6] = S;
  __syncthreads();
  S = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  if (tid < nb) {
    uint32_t q2 = 0;
    if (S > 0.f) {
      const float ratio = s / S;                 // fl32(s / S)
      const float v = rintf(ratio * 256.f);      // exact scale, ties to even
      q2 = (uint32_t)fminf(v, 255.f);
    }
    qscale[b0 + tid] = (uint8_t)q2;
  }
  if (tid == 0) smax[blockIdx.x] = S;
  if (bad && flags) atomicOr(flags, 1u);
}

// Restore: one thread per 8 weights (one dword of codes). float32 output is the
// unrounded product c[q] * s_hat; bf16 output goes through the same byte-plane
// table expansion the matmul kernels use, so checking it bit for bit checks
// their dequantization as well.
template <bool kBf16Out>
__global__ __launch_bounds__(256) void k_dequantize(const uint32_t *__restrict__ codes,
                                                    const uint8_t *__restrict__ qscale,
                                                    const float *__restrict__ smax, int64_t n8,
                                                    void *__restrict__ out, Nf4Consts c) {
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
    const float sh = restore_scale(qscale[blk], smax[blk >> 8]);
    if (kBf16Out) {
      const Nf4Planes t = make_planes(c, sh);
      st16(static_cast<uint16_t *>(out) + i * 8, expand8_natural(t, cw));
    } else {
      f32x4 a, b;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a[e] = cb[(cw >> (4 * e)) & 15u] * sh;
        b[e] = cb[(cw >> (4 * e + 16)) & 15u] * sh;
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
  if (bf16_in)
    k_quantize<true><<<dim3((unsigned)ngroups), dim3(256), 0, st>>>(W, nblocks, codes, qscale, smax, flags, c);
  else
    k_quantize<false><<<dim3((unsigned)ngroups), dim3(256), 0, st>>>(W, nblocks, codes, qscale, smax, flags, c);
  return hipGetLastError();
}

hipError_t launch_dequantize(const uint8_t *codes, const uint8_t *qscale, const float *smax, int64_t d_out,
                             int64_t d_in, bool bf16_out, void *out, const Nf4Consts &c, hipStream_t st) {
  const int64_t n8 = d_out * d_in / 8;
  int64_t grid = (n8 + 255) / 256;
  if (grid > 65536) grid = 65536;
  const uint32_t *cw = reinterpret_cast<const uint32_t *>(codes);
  if (bf16_out)
    k_dequantize<true><<<dim3((unsigned)grid), dim3(256), 0, st>>>(cw, qscale, smax, n8, out, c);
  else
    k_dequantize<false><<<dim3((unsigned)grid), dim3(256), 0, st>>>(cw, qscale, smax, n8, out, c);
  return hipGetLastError();
}

}  // namespace qlora
