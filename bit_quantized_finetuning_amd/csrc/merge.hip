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
// One workgroup per 256-column strip of kMgTiles row tiles of 32 rows:
//   * s B A over a tile is a rank-r product: four waves, each two
//     v_mfma_f32_32x32x16_bf16 accumulators (32 rows x 64 columns), stepping
//     through r 16 at a time. B rows are read straight into the MFMA A operand
//     (16 bytes per lane); the A slab (rank entries x 256 columns) is staged in
//     LDS, because the MFMA B operand needs 8 consecutive rank entries of one
//     column. For r <= 64 the slab is staged once and serves all the strip's
//     row tiles; a larger rank restages it in chunks of 64 per tile.
//   * the float32 product goes through LDS; the epilogue then gives each
//     thread four 8-weight words, consecutive threads on consecutive words of
//     a row, so every store instruction writes whole 512-byte row segments
//     (a thread owning half a block instead wrote 16 bytes per 64 and ran at
//     half the rate of the plain restore). Each word builds its block's
//     restore table; its codes and scales are loaded one tile ahead.
// The kernel is bound by the bf16 output stream (2 bytes per weight written
// against 0.52 read); the product costs 2 r flops per weight on the matrix
// cores.
#include "kernels.h"

namespace qlora {

constexpr int kMgRows = 32;             // rows (d_out) per row tile
constexpr int kMgCols = 256;            // columns (d_in) per workgroup
constexpr int kMgTiles = 4;             // row tiles per workgroup
constexpr int kMgStep = 16;             // rank entries per MFMA step
constexpr int kMgChunk = 64;            // rank entries staged at once
constexpr int kMgAPitch = kMgCols + 8;  // bf16 per staged A row (rows 4 banks apart)
constexpr int kMgDPitch = kMgCols + 4;  // floats per staged product row
constexpr size_t kMgALds = (size_t)kMgChunk * kMgAPitch * 2;
constexpr size_t kMgLds = kMgALds + (size_t)kMgRows * kMgDPitch * 4;

__global__ __launch_bounds__(256) void k_merge(const uint8_t *__restrict__ codes, const uint8_t *__restrict__ qscale,
                                               const float *__restrict__ smax, int64_t d_out, int64_t d_in,
                                               const uint16_t *__restrict__ A, const uint16_t *__restrict__ B, int r,
                                               float scale, uint16_t *__restrict__ out, int sshift) {
  extern __shared__ __attribute__((aligned(16))) uint8_t mg_lds[];
  uint16_t *a_l = reinterpret_cast<uint16_t *>(mg_lds);
  float *d_l = reinterpret_cast<float *>(mg_lds + kMgALds);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bl = lane & 31, bh = lane >> 5;
  const int64_t k0 = (int64_t)blockIdx.x * kMgCols;
  const int64_t nbase = (int64_t)blockIdx.y * kMgRows * kMgTiles;
  const rsrc_t ar = make_rsrc(A, (int64_t)r * d_in * 2);

  // rank entries j0 .. j0 + 63 of columns k0 .. k0 + 255 -> a_l; 2048 chunks of 8 bf16, eight per thread
  auto stage = [&](int j0) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int c = tid + 256 * q, jj = c >> 5, cc = (c & 31) * 8;
      const bool ok = j0 + jj < r && k0 + cc < d_in;
      st16(a_l + jj * kMgAPitch + cc, bld16(ar, ok ? (uint32_t)(((j0 + jj) * d_in + k0 + cc) * 2) : kOOB));
    }
  };
  const bool resident = r <= kMgChunk;
  if (resident && r > 0) {
    stage(0);
    __syncthreads();
  }

  // Epilogue ownership: words w = tid + 256 k (k = 0..3) of the tile's 32 rows x
  // 32 words: row w / 32, weights 8 (w % 32) .. + 7.
  // A tile's global loads: its B fragments for the first rank chunk and the
  // epilogue's codes and scales. They go out one tile ahead, so that each tile
  // waits for at most one memory round trip, and only for the first tile.
  constexpr int kSteps = kMgChunk / kMgStep;  // MFMA steps per chunk
  struct TileLoads {
    u32x4 fb[kSteps];
    uint32_t cw[4], q2[4];
    float S[4];
  };
  auto tile_rows = [&](int t) {
    const int64_t n0 = nbase + (int64_t)t * kMgRows;
    return n0 >= d_out ? 0 : (d_out - n0 < kMgRows ? (int)(d_out - n0) : kMgRows);
  };
  auto load_b = [&](int64_t n0, int rows, int jc, u32x4 (&fb)[kSteps]) {
    const rsrc_t br = make_rsrc(B + n0 * r, (int64_t)rows * r * 2);
#pragma unroll
    for (int i = 0; i < kSteps; ++i) {
      // MFMA A operand: row n0 + l % 32 of B, rank entries j + 8 (l / 32) .. + 7
      // (r % 8 == 0: 8 rank entries are all in or all out)
      const int jb = jc + kMgStep * i + 8 * bh;
      fb[i] = bld16(br, (bl < rows && jb < r) ? (uint32_t)((bl * r + jb) * 2) : kOOB);
    }
  };
  auto load_tile = [&](int t, TileLoads &L) {
    const int rows = tile_rows(t);
    const int64_t n0 = nbase + (int64_t)t * kMgRows;
    if (r > 0 && rows > 0) load_b(n0, rows, 0, L.fb);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int w = tid + 256 * k, row = w >> 5, c = 8 * (w & 31);
      const bool ev = row < rows && k0 + c < d_in;
      const int64_t e = ev ? (n0 + row) * d_in + k0 + c : 0;  // a multiple of 8
      L.cw[k] = ev ? *reinterpret_cast<const uint32_t *>(codes + e / 2) : 0u;
      L.q2[k] = ev ? (sshift ? (uint32_t)qscale[e / kBlock] : q2_or(0)) : 0u;
      L.S[k] = ev ? smax[(e / kBlock) >> sshift] : 0.f;
    }
  };

  TileLoads cur, nxt;
  load_tile(0, cur);
  for (int t = 0; t < kMgTiles; ++t) {
    const int rows = tile_rows(t);
    if (rows == 0) break;  // the same on every thread
    const int64_t n0 = nbase + (int64_t)t * kMgRows;
    if (t + 1 < kMgTiles && tile_rows(t + 1) > 0) load_tile(t + 1, nxt);

    f32x16 acc[2];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[u][e] = 0.f;
    for (int jc = 0; jc < r; jc += kMgChunk) {
      u32x4 fb[kSteps];
      if (jc == 0) {
#pragma unroll
        for (int i = 0; i < kSteps; ++i) fb[i] = cur.fb[i];
      } else {
        load_b(n0, rows, jc, fb);
      }
      if (!resident) {
        __syncthreads();  // the previous chunk's reads are done
        stage(jc);
        __syncthreads();
      }
#pragma unroll
      for (int i = 0; i < kSteps; ++i) {
        const int j = jc + kMgStep * i;
        if (j < r) {
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            // MFMA B operand: column 64 w + 32 u + l % 32 of the slab, rank entries j + 8 (l / 32) .. + 7
            const uint16_t *p = a_l + (kMgStep * i + 8 * bh) * kMgAPitch + 64 * wave + 32 * u + bl;
            u32x4 fa;
#pragma unroll
            for (int e = 0; e < 4; ++e)
              fa[e] = (uint32_t)p[(2 * e) * kMgAPitch] | ((uint32_t)p[(2 * e + 1) * kMgAPitch] << 16);
            acc[u] = mfma32(fb[i], fa, acc[u]);
          }
        }
      }
    }
    __syncthreads();  // the previous tile's epilogue has read d_l
    // Lane l, accumulator e of tile u holds row 8 (e / 4) + 4 (l / 32) + e % 4,
    // column 64 w + 32 u + l % 32.
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = 8 * (e >> 2) + 4 * bh + (e & 3), col = 64 * wave + 32 * u + bl;
        d_l[row * kMgDPitch + col] = scale * acc[u][e];
      }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int w = tid + 256 * k, row = w >> 5, c = 8 * (w & 31);
      if (row < rows && k0 + c < d_in) {
        const Nf4Planes tab = make_planes(restore_scale(cur.q2[k], cur.S[k]));
        const u32x4 wh = expand8(tab, cur.cw[k]);  // 8 restored weights, element order
        const float *dp = d_l + row * kMgDPitch + c;
        const f32x4 d0 = *reinterpret_cast<const f32x4 *>(dp);
        const f32x4 d1 = *reinterpret_cast<const f32x4 *>(dp + 4);
        const u32x4 o = {pack_bf16x2(bf16_lo_to_f32(wh[0]) + d0[0], bf16_hi_to_f32(wh[0]) + d0[1]),
                         pack_bf16x2(bf16_lo_to_f32(wh[1]) + d0[2], bf16_hi_to_f32(wh[1]) + d0[3]),
                         pack_bf16x2(bf16_lo_to_f32(wh[2]) + d1[0], bf16_hi_to_f32(wh[2]) + d1[1]),
                         pack_bf16x2(bf16_lo_to_f32(wh[3]) + d1[2], bf16_hi_to_f32(wh[3]) + d1[3])};
        st16(out + (n0 + row) * d_in + k0 + c, o);
      }
    }
    cur = nxt;
  }
}

static bool g_merge_attr[64];

hipError_t launch_merge(const uint8_t *codes, const uint8_t *qscale, const float *smax, int64_t d_out, int64_t d_in,
                        const uint16_t *A, const uint16_t *B, int r, float scale, uint16_t *out, hipStream_t st) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = -1;
  if (dev < 0 || dev >= 64 || !g_merge_attr[dev]) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(k_merge),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMgLds);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < 64) g_merge_attr[dev] = true;
  }
  const int64_t rows_per_wg = (int64_t)kMgRows * kMgTiles;
  const dim3 grid((unsigned)((d_in + kMgCols - 1) / kMgCols), (unsigned)((d_out + rows_per_wg - 1) / rows_per_wg));
  k_merge<<<grid, dim3(256), kMgLds, st>>>(codes, qscale, smax, d_out, d_in, A, B, r, scale, out,
                                           qscale ? kDqShift : 0);
  return hipGetLastError();
}

}  // namespace qlora
