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
// The kernel is bound by the bf16 output stream (2 bytes per weight written
// against 0.52 read), so it is laid out for many independent waves with their
// loads in flight, and no workgroup-wide step after the start:
//   * a workgroup owns one strip of 64 columns (one 64-weight block per row)
//     and 4 x kMgRT row tiles of 32 rows; wave w takes row tiles w, w + 4, ...;
//   * the strip's slice of A (r rank entries x 64 columns) is staged once in
//     LDS as it lies in memory, rank-major;
//   * per row tile a wave issues all its global loads at once, one tile ahead:
//     B rows (16 bytes per lane and 16 rank entries) and each lane's 16 bytes
//     of packed codes (half a row of the strip: 32 weights), its block's scale
//     code and group maximum;
//   * the product is formed transposed, (s B A)^T = A^T B^T, with
//     v_mfma_f32_32x32x16_bf16: the A side comes from LDS through
//     ds_read_b64_tr_b16 (8 consecutive rank entries of one column per lane),
//     the B rows are the other operand as loaded. Lane l then holds, for row
//     l % 32 of the tile, runs of 4 consecutive columns; one v_permlane32_swap
//     per accumulator pair gives lane l all 32 columns 32 (l / 32) .. +31 of
//     its row -- exactly the weights of its 16 code bytes;
//   * each lane builds its block's restore table once, restores the 32
//     weights, adds and rounds into the wave's LDS tile; the tile then goes
//     out with eight consecutive lanes on each 128-byte row, so every store
//     instruction writes whole lines (16-byte pieces of 64 different lines ran
//     at four fifths of the rate).
#include "kernels.h"
#include "tiles.h"

namespace qlora {

constexpr int kMgCols = 64;                   // columns (d_in) per strip: one block per row
constexpr int kMgRows = 32;                   // rows per row tile
constexpr int kMgWaves = 4;
constexpr int kMgRT = 2;                      // row tiles per wave
constexpr int kMgAPitch = kMgCols * 2 + 32;   // bytes per staged A row: 4 consecutive rows on distinct banks
constexpr int kMgOPitch = kMgCols * 2 + 16;   // bytes per row of a wave's output tile in LDS
constexpr int kMgOBytes = kMgRows * kMgOPitch;
constexpr int kMgMaxSteps = QLORA_MAX_RANK / 16;

// LDS for RS rank steps: 16 RS rank rows of A (those from r on are zero), then each wave's output tile
__host__ __device__ constexpr size_t mg_a_bytes(int rs) { return (size_t)(rs > 0 ? 16 * rs : 1) * kMgAPitch; }
__host__ __device__ constexpr size_t mg_lds(int rs) { return mg_a_bytes(rs) + (size_t)kMgWaves * kMgOBytes; }

template <int RS>  // rank steps of 16 (r <= 16 RS)
__global__ __launch_bounds__(256) void k_merge(const uint8_t *__restrict__ codes, const uint8_t *__restrict__ qscale,
                                               const float *__restrict__ smax, int64_t d_out, int64_t d_in,
                                               const uint16_t *__restrict__ A, const uint16_t *__restrict__ B, int r,
                                               float scale, uint16_t *__restrict__ out, int sshift, int strips,
                                               int groups) {
  extern __shared__ __attribute__((aligned(16))) uint8_t mg_smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ml = lane & 31, half = lane >> 5;
  uint8_t *o_w = mg_smem + mg_a_bytes(RS) + (size_t)wave * kMgOBytes;
  // Workgroup -> (strip, row group), XCD-aware: consecutive workgroups go to
  // the eight XCDs in turn, so XCD x (blockIdx % 8) takes the x-th eighth of
  // the tiles in the order (line group, row group, strip within the line
  // group). The four strips of a line group share every 128-byte line of
  // packed codes (32 bytes each); run on one XCD at about the same time they
  // read each line from HBM once, through that XCD's L2.
  const int64_t lgroups = (strips + 3) / 4, ntiles = lgroups * groups * 4;
  const int64_t per_xcd = (ntiles + 7) / 8;
  const int64_t L = (int64_t)(blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  const int64_t strip = (L / (groups * 4)) * 4 + (L & 3);
  if (L >= ntiles || strip >= strips) return;  // the whole workgroup, before any barrier
  const int64_t k0 = strip * kMgCols;
  const int64_t nbase = ((L >> 2) % groups) * (kMgRows * kMgWaves * kMgRT);
  const int64_t KB = d_in / kBlock;
  const uint32_t q2o = q2_or(sshift);

  // Loads of row tile t of this wave (rows n0 .. n0 + 31 of the strip).
  struct TileLoads {
    u32x4 fb[RS > 0 ? RS : 1];
    u32x4 cw;
    uint32_t q2;
    float S;
  };
  auto tile_row0 = [&](int t) { return nbase + (int64_t)kMgRows * (wave + kMgWaves * t); };
  auto load_tile = [&](int t, TileLoads &L) {
    const int64_t n0 = tile_row0(t);
    const int64_t rows = n0 >= d_out ? 0 : (d_out - n0 < kMgRows ? d_out - n0 : kMgRows);
    if (RS > 0) {
      const rsrc_t br = make_rsrc(B + n0 * r, rows * r * 2);
#pragma unroll
      for (int i = 0; i < RS; ++i) {
        // MFMA B operand: column l % 32 (row n0 + l % 32 of B), rank entries 16 i + 8 (l / 32) .. + 7
        // (r % 8 == 0: the 8 entries are all in or all out)
        const int jb = 16 * i + 8 * half;
        L.fb[i] = bld16(br, (ml < rows && jb < r) ? (uint32_t)((ml * r + jb) * 2) : kOOB);
      }
    }
    // codes of row n0 + l % 32, columns k0 + 32 (l / 32) .. + 31
    const rsrc_t cr = make_rsrc(codes + n0 * (d_in / 2), rows * (d_in / 2));
    L.cw = bld16(cr, ml < rows ? (uint32_t)(ml * (d_in / 2) + k0 / 2 + 16 * half) : kOOB);
    const int64_t blk = (n0 + ml) * KB + k0 / kBlock;  // the row's block in this strip
    const bool ok = ml < rows;
    L.q2 = ok && sshift ? (uint32_t)qscale[blk] : 0u;
    L.S = ok ? smax[blk >> sshift] : 0.f;
  };

  TileLoads cur, nxt;
  load_tile(0, cur);

  // A slice, rank rows 0 .. 16 RS - 1 (zero from r on) x 64 columns, as it lies in memory.
  if (RS > 0) {
    for (int e = tid; e < 16 * RS * (kMgCols / 8); e += 256) {
      const int j = e / (kMgCols / 8), c8 = (e % (kMgCols / 8)) * 8;
      const u32x4 v = j < r ? *reinterpret_cast<const u32x4 *>(A + (int64_t)j * d_in + k0 + c8) : u32x4{0u, 0u, 0u, 0u};
      st16(mg_smem + j * kMgAPitch + c8 * 2, v);
    }
    __syncthreads();
  }
  // MFMA A operand from the slice with ds_read_b64_tr_b16: within each 16 lanes,
  // lane u receives element e (e = 0..3) of the 8 bytes that lane 4e + u/4
  // addresses, its 16-bit element u % 4. Lane v of 16-lane group g therefore
  // addresses rank row 8 (g / 2) + v / 4 (+ 4 for the second read), columns
  // 16 (g % 2) + 4 (v % 4) .. + 3: lane u gets column 16 (g % 2) + u, i.e.
  // l % 32, and rank entries 8 (l / 32) .. + 7 over the two reads.
  const int grp = lane >> 4, u16 = lane & 15;
  const uint32_t aoff = (uint32_t)((8 * (grp >> 1) + (u16 >> 2)) * kMgAPitch + (16 * (grp & 1) + 4 * (u16 & 3)) * 2);
  auto frag_a = [&](int i, int jb) {
    const uint8_t *p = mg_smem + aoff + 16 * i * kMgAPitch + 64 * jb;
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(p));
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(p + 4 * kMgAPitch));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
    return u32x4{l2[0], l2[1], h2[0], h2[1]};
  };

  for (int t = 0; t < kMgRT; ++t) {
    const int64_t n0 = tile_row0(t);
    if (n0 >= d_out) break;  // wave-uniform
    if (t + 1 < kMgRT && tile_row0(t + 1) < d_out) load_tile(t + 1, nxt);

    f32x16 acc[2];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[u][e] = 0.f;
#pragma unroll
    for (int i = 0; i < RS; ++i)
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) acc[jb] = mfma32(frag_a(i, jb), cur.fb[i], acc[jb]);
    // Lane l, accumulator e of column block jb holds strip column 32 jb + 8 (e / 4) + 4 (l / 32) + e % 4 of
    // tile row l % 32. The swap hands lanes 0..31 the block-0 runs of lanes 32..63 (in acc[1]) and lanes 32..63
    // the block-1 runs of lanes 0..31 (in acc[0]): lane l then holds columns 32 (l / 32) + 8 k + 0..3 in
    // acc[0][4k .. 4k+3] and + 4..7 in acc[1][4k .. 4k+3].
    uint32_t d0[16], d1[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[0][e]), __float_as_uint(acc[1][e]),
                                                       false, false);
      d0[e] = sw[0];
      d1[e] = sw[1];
    }

    // Restore, add and round into the wave's LDS tile (row-major, 32 rows x 128 bytes), then store it so that
    // eight consecutive lanes write one whole 128-byte row: the lines go out whole instead of in 16-byte pieces.
    {
      const Nf4Planes tab = make_planes(restore_scale(cur.q2 | q2o, cur.S));
      uint8_t *rowp = o_w + ml * kMgOPitch + 64 * half;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const u32x4 wh = expand8(tab, cur.cw[k]);  // 8 restored weights, element order
        const float s0 = scale * __uint_as_float(d0[4 * k]), s1 = scale * __uint_as_float(d0[4 * k + 1]);
        const float s2 = scale * __uint_as_float(d0[4 * k + 2]), s3 = scale * __uint_as_float(d0[4 * k + 3]);
        const float s4 = scale * __uint_as_float(d1[4 * k]), s5 = scale * __uint_as_float(d1[4 * k + 1]);
        const float s6 = scale * __uint_as_float(d1[4 * k + 2]), s7 = scale * __uint_as_float(d1[4 * k + 3]);
        const u32x4 o = {pack_bf16x2(bf16_lo_to_f32(wh[0]) + s0, bf16_hi_to_f32(wh[0]) + s1),
                         pack_bf16x2(bf16_lo_to_f32(wh[1]) + s2, bf16_hi_to_f32(wh[1]) + s3),
                         pack_bf16x2(bf16_lo_to_f32(wh[2]) + s4, bf16_hi_to_f32(wh[2]) + s5),
                         pack_bf16x2(bf16_lo_to_f32(wh[3]) + s6, bf16_hi_to_f32(wh[3]) + s7)};
        st16(rowp + 16 * k, o);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int rr = 8 * k + (lane >> 3), ch = lane & 7;
      const u32x4 v = *reinterpret_cast<const u32x4 *>(o_w + rr * kMgOPitch + 16 * ch);
      if (n0 + rr < d_out) st16(out + (n0 + rr) * d_in + k0 + 8 * ch, v);
    }
    // the next tile's writes into the LDS tile come after every lane's reads
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
    cur = nxt;
  }
}

template <int RS>
static hipError_t set_merge_attr() {
  return hipFuncSetAttribute(reinterpret_cast<const void *>(k_merge<RS>), hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)mg_lds(RS));
}

hipError_t launch_merge(const uint8_t *codes, const uint8_t *qscale, const float *smax, int64_t d_out, int64_t d_in,
                        const uint16_t *A, const uint16_t *B, int r, float scale, uint16_t *out, hipStream_t st) {
  static DeviceOnce once;
  const hipError_t e = once.run(current_device(), [] {
    hipError_t s = set_merge_attr<0>();
    if (s == hipSuccess) s = set_merge_attr<1>();
    if (s == hipSuccess) s = set_merge_attr<2>();
    if (s == hipSuccess) s = set_merge_attr<4>();
    if (s == hipSuccess) s = set_merge_attr<8>();
    if (s == hipSuccess) s = set_merge_attr<kMgMaxSteps>();
    return s;
  });
  if (e != hipSuccess) return e;
  const int strips = (int)(d_in / kMgCols);
  const int64_t rows_per_wg = (int64_t)kMgRows * kMgWaves * kMgRT;
  const int64_t groups = (d_out + rows_per_wg - 1) / rows_per_wg;
  const int64_t ntiles = (strips + 3) / 4 * groups * 4;
  const dim3 grid((unsigned)((ntiles + 7) / 8 * 8));
  const int sshift = qscale ? kDqShift : 0;
  const int steps = (r + 15) / 16;
#define QLORA_MERGE_LAUNCH(RS)                                                                                     \
  k_merge<RS><<<grid, dim3(256), mg_lds(RS), st>>>(codes, qscale, smax, d_out, d_in, A, B, r, scale, out, \
                                                         sshift, strips, (int)groups)
  if (steps == 0)
    QLORA_MERGE_LAUNCH(0);
  else if (steps == 1)
    QLORA_MERGE_LAUNCH(1);
  else if (steps == 2)
    QLORA_MERGE_LAUNCH(2);
  else if (steps <= 4)
    QLORA_MERGE_LAUNCH(4);
  else if (steps <= 8)
    QLORA_MERGE_LAUNCH(8);
  else
    QLORA_MERGE_LAUNCH(kMgMaxSteps);
#undef QLORA_MERGE_LAUNCH
  return hipGetLastError();
}

}  // namespace qlora
