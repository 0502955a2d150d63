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
// against 0.52 read). Workgroups walk along the rows: each owns a band of 128
// rows and a run of 64-column strips (one 64-weight block per row per strip),
// so that the loads of the next strip fly while the current one is computed
// and stored, and every operand that does not change along the band is read
// once:
//   * wave w owns rows 32 w .. 32 w + 31 of the band; its slice of B (32 rows
//     x r) is loaded once into registers as the MFMA's B operand (16 bytes per
//     lane and 16 rank entries);
//   * per strip the slice of A (r rank entries x 64 columns, rank-major, as it
//     lies in memory) goes into one of two LDS buffers; it is loaded into
//     registers during the previous strip, so one barrier per strip makes it
//     visible and frees the buffer of the strip before;
//   * per strip each lane loads 16 bytes of packed codes (half a row of the
//     strip: 32 weights), its block's scale code and group maximum, also one
//     strip ahead;
//   * the product is formed transposed, (s B A)^T = A^T B^T, with
//     v_mfma_f32_32x32x16_bf16: the A side comes from LDS through
//     ds_read_b64_tr_b16 (8 consecutive rank entries of one column per lane),
//     the B rows are the other operand. Lane l then holds, for row l % 32 of
//     the wave's rows, runs of 4 consecutive columns; one v_permlane32_swap per
//     accumulator pair gives lane l all 32 columns 32 (l / 32) .. +31 of its
//     row -- exactly the weights of its 16 code bytes;
//   * each lane builds its block's restore table, restores the 32 weights
//     straight to float32, adds s (B A) with one fused multiply-add and
//     rounds into the wave's LDS tile; the tile then goes out with
//     eight consecutive lanes on each 128-byte row, so every store instruction
//     writes whole lines.
#include "kernels.h"
#include "tiles.h"

namespace qlora {

constexpr int kMgCols = 64;                   // columns (d_in) per strip: one block per row
constexpr int kMgRows = 32;                   // rows per wave
constexpr int kMgWaves = 4;
constexpr int kMgBand = kMgRows * kMgWaves;   // rows per workgroup
constexpr int kMgAPitch = kMgCols * 2 + 32;   // bytes per staged A row: 4 consecutive rows on distinct banks
constexpr int kMgOPitch = kMgCols * 2 + 16;   // bytes per row of a wave's output tile in LDS
constexpr int kMgOBytes = kMgRows * kMgOPitch;
constexpr int kMgMaxSteps = QLORA_MAX_RANK / 16;
constexpr int kMgTargetWgs = 1024;            // about four workgroups per CU of a 256-CU part

// LDS for RS rank steps: two buffers of 16 RS rank rows of A (those from r on
// are zero), then each wave's output tile
__host__ __device__ constexpr size_t mg_a_bytes(int rs) { return (size_t)(rs > 0 ? 16 * rs : 1) * kMgAPitch; }
__host__ __device__ constexpr size_t mg_lds(int rs) { return 2 * mg_a_bytes(rs) + (size_t)kMgWaves * kMgOBytes; }

template <int RS>  // rank steps of 16 (r <= 16 RS)
__global__ __launch_bounds__(256) void k_merge(const uint8_t *__restrict__ codes, const uint8_t *__restrict__ qscale,
                                               const float *__restrict__ smax, int64_t d_out, int64_t d_in,
                                               const uint16_t *__restrict__ A, const uint16_t *__restrict__ B, int r,
                                               float scale, uint16_t *__restrict__ out, int sshift, int strips,
                                               int chunk) {
  extern __shared__ __attribute__((aligned(16))) uint8_t mg_smem[];
  constexpr int kAPer = RS > 0 ? (16 * RS * (kMgCols / 8) + 255) / 256 : 1;  // 16-byte A pieces per thread
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ml = lane & 31, half = lane >> 5;
  uint8_t *o_w = mg_smem + 2 * mg_a_bytes(RS) + (size_t)wave * kMgOBytes;
  const int64_t nbands = (d_out + kMgBand - 1) / kMgBand;
  const int64_t band = blockIdx.x % nbands;  // neighbouring workgroups: the same strips of other bands
  const int s0 = (int)(blockIdx.x / nbands) * chunk;
  const int s1 = s0 + chunk < strips ? s0 + chunk : strips;
  if (s0 >= strips) return;  // the whole workgroup, before any barrier
  const int64_t n0 = band * kMgBand + (int64_t)kMgRows * wave;  // this wave's first row
  const int64_t rows = n0 >= d_out ? 0 : (d_out - n0 < kMgRows ? d_out - n0 : kMgRows);
  const bool row_ok = ml < rows;
  const int64_t KB = d_in / kBlock;
  const uint32_t q2o = q2_or(sshift);

  // B slice of this wave: MFMA B operand, column l % 32 (row n0 + l % 32 of B), rank entries
  // 16 i + 8 (l / 32) .. + 7 (r % 8 == 0: the 8 entries are all in or all out)
  u32x4 fb[RS > 0 ? RS : 1];
  if (RS > 0) {
    const rsrc_t br = make_rsrc(B + n0 * r, rows * r * 2);
#pragma unroll
    for (int i = 0; i < RS; ++i) {
      const int jb = 16 * i + 8 * half;
      fb[i] = bld16(br, (row_ok && jb < r) ? (uint32_t)((ml * r + jb) * 2) : kOOB);
    }
  }
  // Per strip: the A slice pieces of this thread (rank row j, columns c8 .. c8 + 7) and this lane's codes.
  struct StripLoads {
    u32x4 a[kAPer];
    u32x4 cw;
    uint32_t q2;
    float S;
  };
  const rsrc_t cr = make_rsrc(codes + n0 * (d_in / 2), rows * (d_in / 2));
  const rsrc_t ar = make_rsrc(A, (int64_t)r * d_in * 2);  // rank rows r and up read zeros
  auto load_strip = [&](int s, StripLoads &L) {
    const int64_t k0 = (int64_t)s * kMgCols;
    if (RS > 0) {
#pragma unroll
      for (int q = 0; q < kAPer; ++q) {
        const int e = tid + 256 * q, j = e / (kMgCols / 8), c8 = (e % (kMgCols / 8)) * 8;
        L.a[q] = bld16(ar, (e < 16 * RS * (kMgCols / 8) && j < r) ? (uint32_t)((j * d_in + k0 + c8) * 2) : kOOB);
      }
    }
    // codes of row n0 + l % 32, columns k0 + 32 (l / 32) .. + 31
    L.cw = bld16(cr, row_ok ? (uint32_t)(ml * (d_in / 2) + k0 / 2 + 16 * half) : kOOB);
    const int64_t blk = (n0 + ml) * KB + k0 / kBlock;  // the row's block in this strip
    L.q2 = row_ok && sshift ? (uint32_t)qscale[blk] : 0u;
    L.S = row_ok ? smax[blk >> sshift] : 0.f;
  };
  auto stage_a = [&](int s, const StripLoads &L) {
    uint8_t *buf = mg_smem + (s & 1) * mg_a_bytes(RS);
#pragma unroll
    for (int q = 0; q < kAPer; ++q) {
      const int e = tid + 256 * q, j = e / (kMgCols / 8), c8 = (e % (kMgCols / 8)) * 8;
      if (e < 16 * RS * (kMgCols / 8)) st16(buf + j * kMgAPitch + c8 * 2, L.a[q]);
    }
  };

  // MFMA A operand from the slice with ds_read_b64_tr_b16: within each 16 lanes,
  // lane u receives element e (e = 0..3) of the 8 bytes that lane 4e + u/4
  // addresses, its 16-bit element u % 4. Lane v of 16-lane group g therefore
  // addresses rank row 8 (g / 2) + v / 4 (+ 4 for the second read), columns
  // 16 (g % 2) + 4 (v % 4) .. + 3: lane u gets column 16 (g % 2) + u, i.e.
  // l % 32, and rank entries 8 (l / 32) .. + 7 over the two reads.
  const int grp = lane >> 4, u16 = lane & 15;
  const uint32_t aoff = (uint32_t)((8 * (grp >> 1) + (u16 >> 2)) * kMgAPitch + (16 * (grp & 1) + 4 * (u16 & 3)) * 2);
  auto frag_a = [&](const uint8_t *buf, int i, int jb) {
    const uint8_t *p = buf + aoff + 16 * i * kMgAPitch + 64 * jb;
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(p));
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(p + 4 * kMgAPitch));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
    return u32x4{l2[0], l2[1], h2[0], h2[1]};
  };

  StripLoads cur, nxt;
  load_strip(s0, cur);
  for (int s = s0; s < s1; ++s) {
    stage_a(s, cur);
    // A of strip s is visible; every wave is done with strip s - 1 (its buffer
    // takes strip s + 1) and with the output tile of strip s - 1.
    __syncthreads();
    if (s + 1 < s1) load_strip(s + 1, nxt);
    const uint8_t *buf = mg_smem + (s & 1) * mg_a_bytes(RS);
    const int64_t k0 = (int64_t)s * kMgCols;

    f32x16 acc[2];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[u][e] = 0.f;
#pragma unroll
    for (int i = 0; i < RS; ++i)
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) acc[jb] = mfma32(frag_a(buf, i, jb), fb[i], acc[jb]);
    // Lane l, accumulator e of column block jb holds strip column 32 jb + 8 (e / 4) + 4 (l / 32) + e % 4 of
    // row l % 32. The swap hands lanes 0..31 the block-0 runs of lanes 32..63 (in acc[1]) and lanes 32..63
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
    // eight consecutive lanes write one whole 128-byte row. The restore stops at the byte-plane lookups: one
    // more byte select per weight puts its low and high bf16 bytes into the top half of a zero word, which is
    // the restored weight as a float32, and one fused multiply-add forms w_hat + s (B A).
    {
      const Nf4Planes tab = make_planes(restore_scale(cur.q2 | q2o, cur.S));
      uint8_t *rowp = o_w + ml * kMgOPitch + 64 * half;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t c = cur.cw[k];
        const uint32_t sa = c & 0x07070707u, ma = ((c >> 1) & 0x04040404u) | 0x03020100u;
        const uint32_t sb = (c >> 4) & 0x07070707u, mb = ((c >> 5) & 0x04040404u) | 0x03020100u;
        const uint32_t lo_a = lookup4(tab.lo, sa, ma), hi_a = lookup4(tab.hi, sa, ma);  // e0..e3
        const uint32_t lo_b = lookup4(tab.lo, sb, mb), hi_b = lookup4(tab.hi, sb, mb);  // e4..e7
        float v[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // bytes 0, 1 zero (selector 12), byte 2 the low and byte 3 the high byte of weight e
          const uint32_t sel = 0x00000c0cu | ((uint32_t)e << 16) | ((uint32_t)(4 + e) << 24);
          v[e] = fmaf(scale, __uint_as_float(d0[4 * k + e]), __uint_as_float(perm(hi_a, lo_a, sel)));
          v[4 + e] = fmaf(scale, __uint_as_float(d1[4 * k + e]), __uint_as_float(perm(hi_b, lo_b, sel)));
        }
        const u32x4 o = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                         pack_bf16x2(v[6], v[7])};
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
      // non-temporal: the merged weight is written once (10 % faster than plain stores; non-temporal code
      // loads measured slower)
      if (rr < rows) __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(out + (n0 + rr) * d_in + k0 + 8 * ch));
    }
    cur = nxt;
    // (the next strip's writes into the output tile come after its barrier)
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
  const int64_t nbands = (d_out + kMgBand - 1) / kMgBand;
  // strips per workgroup: enough workgroups for about four per CU, runs of
  // four strips (whole 128-byte lines of codes), at least four
  int64_t chunk = (nbands * strips + kMgTargetWgs - 1) / kMgTargetWgs;
  chunk = (chunk + 3) / 4 * 4;
  if (chunk < 4) chunk = 4;
  if (chunk > strips) chunk = strips;
  const int64_t nchunks = (strips + chunk - 1) / chunk;
  const dim3 grid((unsigned)(nbands * nchunks));
  const int sshift = qscale ? kDqShift : 0;
  const int steps = (r + 15) / 16;
#define QLORA_MERGE_LAUNCH(RS)                                                                                     \
  k_merge<RS><<<grid, dim3(256), mg_lds(RS), st>>>(codes, qscale, smax, d_out, d_in, A, B, r, scale, out, \
                                                         sshift, strips, (int)chunk)
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
