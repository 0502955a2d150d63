// Merge of a trained adapter into the restored weight, for export:
//
//     W_merged = bf16( W_hat + s B A ),   s = alpha / r
//
// "48GB GPU Fine-Tuning a 65B Model: Where QLoRA Saves GPU Memory", section
// "QLoRA Puts the Two Methods in Different Places": the trained A and B cannot
// be added to the 4-bit weights; they are merged into the restored 16-bit
// weights (or kept separately). W_hat is the same bf16 restore the forward and
// backward use (bit-exact with the dequantize entry point); the sum is formed
// in float32 and rounded once to bf16.
//
// One workgroup per 32 x 256 output tile (rows of d_out x columns of d_in):
//   * s B A over the tile is a rank-r product: four waves, each two
//     v_mfma_f32_32x32x16_bf16 accumulators (32 rows x 64 columns), stepping
//     through r 16 at a time. B rows are read straight into the MFMA A operand
//     (16 bytes per lane); the 16 x 256 slab of A is staged in LDS, because the
//     MFMA B operand needs 8 consecutive rank entries of one column.
//   * the float32 product goes through LDS so that each thread then owns 32
//     consecutive weights of one row = half a block: one 16-byte code load,
//     one restore table, four 8-weight expansions, four 16-byte stores.
// The kernel is bound by the bf16 output stream (2 bytes per weight written
// against 0.52 read); the product costs 2 r flops per weight on the matrix
// cores.
#include "kernels.h"

namespace qlora {

constexpr int kMgRows = 32;            // output rows (d_out) per workgroup
constexpr int kMgCols = 256;           // output columns (d_in) per workgroup
constexpr int kMgStep = 16;            // rank entries per MFMA step
constexpr int kMgAPitch = kMgCols + 8;  // bf16 per staged A row (rows 4 banks apart)
constexpr int kMgDPitch = kMgCols + 4;  // floats per staged product row

__global__ __launch_bounds__(256) void k_merge(const uint8_t *__restrict__ codes, const uint8_t *__restrict__ qscale,
                                               const float *__restrict__ smax, int64_t d_out, int64_t d_in,
                                               const uint16_t *__restrict__ A, const uint16_t *__restrict__ B, int r,
                                               float scale, uint16_t *__restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint16_t a_l[kMgStep * kMgAPitch];
  __shared__ __attribute__((aligned(16))) float d_l[kMgRows * kMgDPitch];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t n0 = (int64_t)blockIdx.y * kMgRows, k0 = (int64_t)blockIdx.x * kMgCols;
  const int rows = d_out - n0 < kMgRows ? (int)(d_out - n0) : kMgRows;

  f32x16 acc[2];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[t][e] = 0.f;

  if (r > 0) {
    // B rows n0 .. n0 + rows - 1 (r % 8 == 0: 8 rank entries are all in or all out)
    const rsrc_t br = make_rsrc(B + n0 * r, (int64_t)rows * r * 2);
    const rsrc_t ar = make_rsrc(A, (int64_t)r * d_in * 2);
    const int bl = lane & 31, bh = lane >> 5;
    for (int j0 = 0; j0 < r; j0 += kMgStep) {
      // A[j0 .. j0 + 15][k0 .. k0 + 255] -> a_l; 512 chunks of 8 bf16, two per thread
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int c = tid + 256 * q, jj = c >> 5, cc = (c & 31) * 8;
        const bool ok = j0 + jj < r && k0 + cc < d_in;
        st16(a_l + jj * kMgAPitch + cc, bld16(ar, ok ? (uint32_t)(((j0 + jj) * d_in + k0 + cc) * 2) : kOOB));
      }
      // MFMA A operand: row n0 + l % 32 of B, rank entries j0 + 8 (l / 32) .. + 7
      const int jb = j0 + 8 * bh;
      const u32x4 fb = bld16(br, (bl < rows && jb < r) ? (uint32_t)((bl * r + jb) * 2) : kOOB);
      __syncthreads();
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        // MFMA B operand: column 64 w + 32 t + l % 32 of the slab, rank entries 8 (l / 32) .. + 7
        const uint16_t *p = a_l + (8 * bh) * kMgAPitch + 64 * wave + 32 * t + bl;
        u32x4 fa;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          fa[e] = (uint32_t)p[(2 * e) * kMgAPitch] | ((uint32_t)p[(2 * e + 1) * kMgAPitch] << 16);
        acc[t] = mfma32(fb, fa, acc[t]);
      }
      __syncthreads();
    }
  }
  // Lane l, accumulator e of tile t holds row 8 (e / 4) + 4 (l / 32) + e % 4,
  // column 64 w + 32 t + l % 32.
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int row = 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3), col = 64 * wave + 32 * t + (lane & 31);
      d_l[row * kMgDPitch + col] = scale * acc[t][e];
    }
  __syncthreads();

  // Thread: row tid / 8, columns 32 (tid % 8) .. + 31 (half a block).
  const int row = tid >> 3, c0 = 32 * (tid & 7);
  const int64_t n = n0 + row, k = k0 + c0;
  if (row >= rows || k >= d_in) return;
  const int64_t e0 = n * d_in + k;  // first element; a multiple of 32
  const u32x4 cw = *reinterpret_cast<const u32x4 *>(codes + e0 / 2);
  const int64_t blk = e0 / kBlock;
  const Nf4Planes tab = make_planes(restore_scale(qscale[blk], smax[blk / kGroup]));
  const float *dp = d_l + row * kMgDPitch + c0;
  uint16_t *op = out + e0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const u32x4 wh = expand8(tab, cw[w]);  // 8 restored weights, element order
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float lo = bf16_lo_to_f32(wh[i]) + dp[8 * w + 2 * i];
      const float hi = bf16_hi_to_f32(wh[i]) + dp[8 * w + 2 * i + 1];
      o[i] = pack_bf16x2(lo, hi);
    }
    st16(op + 8 * w, o);
  }
}

hipError_t launch_merge(const uint8_t *codes, const uint8_t *qscale, const float *smax, int64_t d_out, int64_t d_in,
                        const uint16_t *A, const uint16_t *B, int r, float scale, uint16_t *out, hipStream_t st) {
  const dim3 grid((unsigned)((d_in + kMgCols - 1) / kMgCols), (unsigned)((d_out + kMgRows - 1) / kMgRows));
  k_merge<<<grid, dim3(256), 0, st>>>(codes, qscale, smax, d_out, d_in, A, B, r, scale, out);
  return hipGetLastError();
}

}  // namespace qlora
