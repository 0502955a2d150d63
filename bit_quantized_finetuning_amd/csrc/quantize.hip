// NF4 blockwise quantization with double quantization, and the standalone restore.
//
// Quantize ("48GB GPU Fine-Tuning a 65B Model", section "Quantization Keeps the
// Patterns and Reduces Bits per Number"): per block of 64 weights the scale is
// the largest |w|; each weight is divided by it and replaced by the index of the
// nearest of the 16 NF4 levels. Double quantization (first page, section
// "메모리 회계"): the block scales are re-coded to 8 bits against their group
// maximum so that they come back as (q2/256) * S.
//
// One launch quantizes up to kQuantizeJobs weights (a table of jobs passed as a
// kernel argument): their groups of 256 blocks (16384 weights) are numbered
// one after another, and persistent workgroups take groups blockIdx.x,
// blockIdx.x + gridDim.x, ... of that sequence, so small weights share the
// launch, its start-up and its tail with the large ones. Each workgroup
// builds its search table once.
// Eight lanes share a block: each loads 8 consecutive weights (32 contiguous
// bytes of float32, the eight lanes together 256 contiguous bytes), the eight
// reduce the block absmax, and each lane emits its weights' codes as one packed
// 32-bit word. All eight passes' loads of a group are issued at once; the next
// group's loads go out as soon as the current group's weights have been coded,
// so they fly while the group's scales are reduced and written. The block
// scales wait in LDS for the group maximum, then one thread per block writes
// its 8-bit scale code. The kernel streams 4 (or 2) bytes in and ~0.52 bytes
// out per weight.
//
// Nearest level: the index is the number of the 15 float32 thresholds at or
// below x = fl32(w / s) (x is in [-1, 1]). The float32 bits of x pick one of
// 2048 table entries (sign, exponent, top two significand bits): every entry
// covers a quarter binade (all magnitudes below 2^-5 share the entries of one
// bucket) holding at most one threshold t, and stores the count of thresholds
// below it, t (+inf if none) and a tolerance of 16 units in the last place of
// t. The index is then count + [x >= t].
//
// The quotient is not formed by the IEEE divide (about ten instructions) but
// as xa = w * rcp(s) (v_rcp_f32, within 1 ulp), which is within 4 ulp of
// fl32(w / s). No threshold lies within 64 ulp of a quarter-binade edge (a
// property of the 15 thresholds, checked on the host), so xa and the exact
// quotient fall on the same side of every threshold unless xa is within the
// tolerance of its entry's t; such weights, and blocks whose absmax is below
// 2^-100, are recomputed with the IEEE divide. The rule is checked against the
// plain count on the host, with the quotient perturbed by up to 4 ulp.
//
// For absmax-only storage (a job without scale codes) each block's float32 absmax is written as
// its scale instead, and there is no group step.
#include "kernels.h"

namespace qlora {

constexpr int kQTable = 2048;
constexpr int64_t kQuantizeGrid = 1024;

template <bool kBf16In>
__global__ __launch_bounds__(256) void k_quantize(QuantizeJobs J, uint32_t *__restrict__ flags, Nf4Consts c) {
  constexpr int esz = kBf16In ? 2 : 4;
  constexpr int kPasses = kGroup / 32;
  __shared__ float s_blk[kGroup];
  __shared__ float s_red[4];
  __shared__ float2 bucket[64];       // {threshold inside the bucket or +inf, count of thresholds below it}
  __shared__ u32x4 qtab[kQTable];     // {bits of t, bits of the tolerance, count, 0} per (sign, exponent, m2)
  const int tid = threadIdx.x;
  const int l8 = tid & 7;
  const int slot = tid >> 3;  // 32 blocks per pass
  const int64_t ngroups = J.gstart[J.n];  // groups of all jobs

  // The job holding group g, searched forward from job j (g only grows).
  auto job_of = [&](int64_t g, int j) {
    while (j + 1 < J.n && g >= J.gstart[j + 1]) ++j;
    return j;
  };
  u32x4 raw[kPasses][kBf16In ? 1 : 2];
  auto load_group = [&](int64_t g, int j) {
    const int64_t b0 = (g - J.gstart[j]) * kGroup;
    const int64_t nblocks = J.nblocks[j];
    const int nb = (int)(nblocks - b0 < kGroup ? nblocks - b0 : kGroup);
    const rsrc_t wr = make_rsrc(static_cast<const uint8_t *>(J.W[j]) + b0 * kBlock * esz, (int64_t)nb * kBlock * esz);
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
      const int b = p * 32 + slot;
      const uint32_t off = b < nb ? (uint32_t)((b * kBlock + l8 * 8) * esz) : kOOB;
      // non-temporal (aux 2): W is read once; with the codes' non-temporal stores the pass ran 3.7 % faster
      raw[p][0] = __builtin_amdgcn_raw_buffer_load_b128(wr, off, 0, 2);
      if (!kBf16In) raw[p][kBf16In ? 0 : 1] = __builtin_amdgcn_raw_buffer_load_b128(wr, off + 16, 0, 2);
    }
  };
  int64_t g = blockIdx.x;
  int j = 0;
  if (g < ngroups) {
    j = job_of(g, 0);
    load_group(g, j);
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
  // Entry i = (sign, exponent, m2) from bits 31, 30..23, 22..21 of x: its bucket,
  // with exponents below 122 in bucket e = 0 and above 127 (never reached) in e = 6.
  for (int i = tid; i < kQTable; i += 256) {
    const int sg = i >> 10, ex = (i >> 2) & 0xff, m2 = i & 3;
    const int e = min(max(ex - 121, 0), 6);
    const float2 bk = bucket[(sg << 5) | (e << 2) | (e == 0 ? 0 : m2)];
    const uint32_t tb = __float_as_uint(bk.x);
    const uint32_t texp = (tb >> 23) & 0xffu;
    // 16 ulp of t = 2^(texp - 127 - 23 + 4); none (0) where t is +inf
    const uint32_t tol = bk.x < __builtin_inff() ? (texp - 19u) << 23 : 0u;
    qtab[i] = u32x4{tb, tol, (uint32_t)bk.y, 0u};
  }
  __syncthreads();

  for (; g < ngroups; g += gridDim.x) {
    j = job_of(g, j);
    const int64_t gl = g - J.gstart[j];  // group of job j
    const int64_t b0 = gl * kGroup;
    const int64_t nblocks = J.nblocks[j];
    const int nb = (int)(nblocks - b0 < kGroup ? nblocks - b0 : kGroup);
    uint8_t *const codes = J.codes[j];
    uint8_t *const qscale = J.qscale[j];
    float *const smax = J.smax[j];
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
      // Block absmax as the largest magnitude bit pattern: for finite values the
      // order of |w|'s bits is the order of |w|; a NaN or inf makes it >= 0x7f800000.
      uint32_t mb = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) mb = max(mb, __float_as_uint(w[e]) & 0x7fffffffu);
      mb = max(mb, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mb, 0xB1, 0xF, 0xF, false));   // lanes ^ 1
      mb = max(mb, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mb, 0x4E, 0xF, 0xF, false));   // lanes ^ 2
      mb = max(mb, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mb, 0x141, 0xF, 0xF, false));  // other quad of 8
      bad |= mb >= 0x7f800000u;
      const float m = __uint_as_float(mb);
      const float rm = m > 0.f ? __builtin_amdgcn_rcpf(m) : 0.f;
      bool near = m > 0.f && m < 0x1p-100f;
      uint32_t word = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float xa = w[e] * rm;
        const u32x4 ent = qtab[__float_as_uint(xa) >> 21];
        const float d = xa - __uint_as_float(ent[0]);
        near |= fabsf(d) <= __uint_as_float(ent[1]);
        word |= (ent[2] + (d >= 0.f ? 1u : 0u)) << nibble_shift(e);
      }
      if (near) {  // rare: the exact quotient decides
        word = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = m > 0.f ? w[e] / m : 0.f;  // IEEE float32 divide
          const u32x4 ent = qtab[__float_as_uint(x) >> 21];
          word |= (ent[2] + (x >= __uint_as_float(ent[0]) ? 1u : 0u)) << nibble_shift(e);
        }
      }
      if (b < nb) {
        if (l8 == 0) s_blk[b] = m;
        // non-temporal: the codes are written once and not read back by this pass
        __builtin_nontemporal_store(word, reinterpret_cast<uint32_t *>(codes + (b0 + b) * (kBlock / 2) + l8 * 4));
      }
    }
    if (g + gridDim.x < ngroups) load_group(g + gridDim.x, job_of(g + gridDim.x, j));
    __syncthreads();

    const float s = tid < nb ? s_blk[tid] : 0.f;
    if (!qscale) {  // absmax-only storage: the block scales as they are
      if (tid < nb) smax[b0 + tid] = s;
    } else {
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
      if (tid == 0) smax[gl] = S;
    }
    if (bad && flags) atomicOr(flags, 1u);
    __syncthreads();  // s_blk and s_red are reused by the next group
  }
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

hipError_t launch_quantize(const QuantizeJobs &jobs, bool bf16_in, uint32_t *flags, const Nf4Consts &c,
                           hipStream_t st) {
  const int64_t ngroups = jobs.gstart[jobs.n];
  if (jobs.n < 1 || jobs.n > kQuantizeJobs || ngroups < 1) return hipErrorInvalidValue;
  // persistent workgroups: four per compute unit of a 256-CU part (their LDS
  // allows four), or one per group when there are fewer groups
  const unsigned grid = (unsigned)(ngroups < kQuantizeGrid ? ngroups : kQuantizeGrid);
  if (bf16_in)
    k_quantize<true><<<dim3(grid), dim3(256), 0, st>>>(jobs, flags, c);
  else
    k_quantize<false><<<dim3(grid), dim3(256), 0, st>>>(jobs, flags, c);
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
