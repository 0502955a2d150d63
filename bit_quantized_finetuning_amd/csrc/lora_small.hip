// Skinny LoRA products u = x A^T and v = dY B (N = r columns).
//
// The adapter path of the forward "QLoRA의 수식" (first page): the rank-r
// intermediate A x, here u = x A^T [T, r]; and of the backward, v = dY B [T, r]
// (the gradient of h with respect to the adapter intermediate).
//
// out[T, r] = P[T, K] . Q[r, K]^T with both operands K-contiguous (for v the
// caller passes Q = B^T). One workgroup (4 waves) owns 16 tokens and a K slice;
// the waves split the slice, each accumulating all r columns with
// v_mfma_f32_16x16x32_bf16, and reduce through LDS. With ksplit > 1 the K slices
// of a token tile land in a float32 partial buffer and the last workgroup to
// arrive (device-scope counter) sums them in fixed order, so results do not
// depend on scheduling. Outputs: float32 out (optional) and the bf16 copy of
// scale*out that the matmul kernels consume as extra K columns. Loads are raw
// buffer loads (rows past T and K steps past the slice read zeros), and partials
// travel through device-scope stores/loads, so no cache-wide fence is needed.
#include "kernels.h"

namespace qlora {

constexpr int kMaxNt = 16;  // r <= 256

__global__ __launch_bounds__(256) void k_lora_small(const uint16_t *__restrict__ P, const uint16_t *__restrict__ Q,
                                                    int64_t T, int64_t K, int r, int nt, float scale,
                                                    float *__restrict__ out_f32, uint16_t *__restrict__ out_bf16,
                                                    int r_pad, float *__restrict__ partial,
                                                    uint32_t *__restrict__ counters, int ksplit) {
  __shared__ float red[4][256];
  __shared__ int is_last;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int64_t t0 = (int64_t)blockIdx.x * 16;
  const int split = blockIdx.y;
  const int64_t nk32 = (K + 31) / 32;
  const int64_t kb = nk32 * split / ksplit, ke = nk32 * (split + 1) / ksplit;
  const int li = lane & 15, g = lane >> 4;

  f32x4 acc[kMaxNt];
#pragma unroll
  for (int j = 0; j < kMaxNt; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int64_t prow = T - t0 < 16 ? T - t0 : 16;
  const rsrc_t pr = make_rsrc(P + t0 * K, prow * K * 2);
  const rsrc_t qr = make_rsrc(Q, (int64_t)r * K * 2);
  // Two K steps per iteration, all loads first; steps past ke read zeros.
  for (int64_t k32 = kb + wave; k32 < ke; k32 += 8) {
    u32x4 a[2], b[2][kMaxNt];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int64_t kk = k32 + 4 * s;
      const int64_t k = kk * 32 + 8 * g;
      const bool ok = kk < ke && k < K;
      a[s] = bld16(pr, ok ? (uint32_t)((li * K + k) * 2) : kOOB);
#pragma unroll
      for (int j = 0; j < kMaxNt; ++j)
        if (j < nt) b[s][j] = bld16(qr, ok ? (uint32_t)(((16 * j + li) * K + k) * 2) : kOOB);
    }
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int j = 0; j < kMaxNt; ++j)
        if (j < nt) acc[j] = mfma16(a[s], b[s][j], acc[j]);
  }

  // Reduce the four waves; lane (li, g) of each wave holds rows 4g..4g+3, column li.
  float *pbase = partial + ((int64_t)blockIdx.x * ksplit + split) * 16 * r_pad;
  for (int j = 0; j < nt; ++j) {
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][lane * 4 + i] = acc[j][i];
    __syncthreads();
    {
      const float v = red[0][tid] + red[1][tid] + red[2][tid] + red[3][tid];
      // tid = lane*4 + i  ->  row 4*(lane/16) + i, col lane%16
      const int ln = tid >> 2, i = tid & 3;
      const int row = 4 * (ln >> 4) + i, col = 16 * j + (ln & 15);
      if (ksplit == 1) {
        const int64_t tt = t0 + row;
        if (tt < T && col < r && out_f32) out_f32[tt * r + col] = v;
        if (out_bf16 && col < r_pad) {
          const float sv = (tt < T && col < r) ? scale * v : 0.f;
          out_bf16[tt * r_pad + col] = (uint16_t)(pack_bf16x2(sv, 0.f) & 0xffffu);
        }
      } else {
        st_dev(pbase + row * r_pad + col, v);
      }
    }
    __syncthreads();
  }
  if (ksplit == 1) return;

  wait_vmem();
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev = add_dev_u32(tile_counter(counters, blockIdx.x), 1u);
    is_last = (prev == (uint32_t)ksplit - 1u);
  }
  __syncthreads();
  if (!is_last) return;
  const float *base = partial + (int64_t)blockIdx.x * ksplit * 16 * r_pad;
  for (int e = tid; e < 16 * r_pad; e += 256) {
    float v = 0.f;
    for (int s = 0; s < ksplit; ++s) v += ld_dev(base + (int64_t)s * 16 * r_pad + e);
    const int row = e / r_pad, col = e % r_pad;
    const int64_t tt = t0 + row;
    if (tt < T && col < r && out_f32) out_f32[tt * r + col] = v;
    if (out_bf16) {
      const float sv = (tt < T && col < r) ? scale * v : 0.f;
      out_bf16[tt * r_pad + col] = (uint16_t)(pack_bf16x2(sv, 0.f) & 0xffffu);
    }
  }
  if (tid == 0) st_dev_u32(tile_counter(counters, blockIdx.x), 0u);
}

// 32x32 tiles through LDS.
__global__ __launch_bounds__(256) void k_transpose_bf16(const uint16_t *__restrict__ src, int64_t rows, int64_t cols,
                                                        uint16_t *__restrict__ dst) {
  __shared__ uint16_t tile[32][33];
  const int64_t r0 = (int64_t)blockIdx.y * 32, c0 = (int64_t)blockIdx.x * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
  for (int i = ty; i < 32; i += 8) {
    const int64_t r = r0 + i, c = c0 + tx;
    tile[i][tx] = (r < rows && c < cols) ? src[r * cols + c] : (uint16_t)0;
  }
  __syncthreads();
  for (int i = ty; i < 32; i += 8) {
    const int64_t c = c0 + i, r = r0 + tx;
    if (c < cols && r < rows) dst[c * rows + r] = tile[tx][i];
  }
}

hipError_t launch_lora_small(const uint16_t *P, const uint16_t *Q, int64_t T, int64_t K, int r, float scale,
                             float *out_f32, uint16_t *out_bf16, int r_pad, float *partial, uint32_t *counters,
                             int ksplit, hipStream_t st) {
  const int nt = (r + 15) / 16;
  const int64_t tiles = (T + 15) / 16;
  k_lora_small<<<dim3((unsigned)tiles, (unsigned)ksplit), dim3(256), 0, st>>>(
      P, Q, T, K, r, nt, scale, out_f32, out_bf16, r_pad, partial, counters, ksplit);
  return hipGetLastError();
}

hipError_t launch_transpose_bf16(const uint16_t *src, int64_t rows, int64_t cols, uint16_t *dst, hipStream_t st) {
  dim3 grid((unsigned)((cols + 31) / 32), (unsigned)((rows + 31) / 32));
  k_transpose_bf16<<<grid, dim3(256), 0, st>>>(src, rows, cols, dst);
  return hipGetLastError();
}

}  // namespace qlora
