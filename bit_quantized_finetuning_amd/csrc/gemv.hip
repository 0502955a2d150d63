// Forward for T <= 16 tokens in one launch: stream the 4.13-bit weight once.
//
// h[T, d_out] = x W_hat^T + s (x A^T) B^T   ("QLoRA의 수식" on the first page: the
// restored frozen base plus the adapter term, s = alpha/r).
//
// Every weight is used by at most 16 tokens, so the kernel is bound by the
// packed-weight stream (0.516 bytes per weight), by the VALU work of the
// restore (about 3.5 instructions per weight) and, at these sizes, by launch
// and memory latency. The design therefore issues its loads early, in the
// order they are needed, and keeps the per-item bookkeeping out of the VALU.
//
// One grid of G workgroups of kW waves, one per CU (G = min(row tiles, CUs)):
//   * workgroup c streams row tiles c, c+G, c+2G, ... of 16 output rows. The
//     waves split K into 256-wide segments; in a segment lane (row, g) owns one
//     64-weight block (two 16-byte code loads), builds that block's restore
//     table once and feeds 8 v_mfma_f32_16x16x32_bf16 (tokens on M, padded to
//     16; rows on N). Each wave prefetches its next (row tile, segment) item
//     while computing the current one (two register stages in ping-pong).
//   * x is staged in LDS when it fits (T x d_in bf16 <= 136 KB), each wave
//     staging just the segments it computes with, so no workgroup barrier
//     stands before the first item; the segment order is rotated per workgroup
//     so that the CUs, which all read all of x, spread over the L2 channels.
//     Otherwise x is read per segment from global memory. Loads go out in the
//     order they are needed (they complete in issue order).
//   * the first P = 4 r_pad/16 workgroups (dispatched first, and given the
//     fewest row tiles: workgroup c streams row tiles G-1-c, 2G-1-c, ...)
//     also produce the adapter intermediate: producer (j, ks) forms the
//     partial of columns 16j..16j+15 of u = x A^T over the ks-th quarter of K
//     (a single CU streams only a few tens of GB/s, so the A reads are
//     spread). Its A and x operands are its first loads and the job runs
//     before anything else, so each float32 partial is published early,
//     together with a tag in one 64-bit device-scope store. No counter or flag
//     sits between producer and reader.
//   * the tag names the launch: the dispatch id of the kernel (a per-queue
//     packet counter, new for every launch and every graph replay) mixed with
//     the queue's address. Every workgroup has it in registers from the start,
//     so nothing is read from memory or counted to agree on it. An entry left
//     by an earlier launch could only match after 2^32 launches on one queue,
//     or, across queues, with probability 2^-32 per change of queue.
//   * s*u is read once per workgroup: the loads go out before the last item of
//     the first row tile, and at that tile's end the entries are checked (and
//     re-read until their tags match), the four partials summed in slice order
//     and bf16(s*u) put in LDS; wave 0 then adds s*u B^T as r_pad more K
//     columns. The workgroup of row tile 0 writes float32 u for the backward.
//   * a reader that has waited the wait limit (kWaitTicks) for a partial forms it itself with
//     the producer's own code (same operands, same order of operations, so the
//     same bits) and publishes it as the producer would. The grid never
//     exceeds one residency and producers never wait, so on its own a launch
//     never gets there; when launches on other streams hold the compute units
//     a producer needs, this keeps every wait finite and every result exact.
//     Each such fallback is counted in a status word of the workspace.
//   * at the end of a row tile the waves reduce through LDS and write h.
// Buffer
// descriptors cover whole tensors (the launcher requires the packed codes to
// stay below 2^31 bytes); per-lane offsets are 32-bit and an out-of-range lane
// reads zero.
#include "kernels.h"

namespace qlora {

constexpr int kMaxRpad = 256;
constexpr int kXPad = 8;             // bf16 of padding per staged x row (rows 4 banks apart)
constexpr int kXLdsBytes = 136 * 1024;
constexpr int kABatch = 8;           // producer K steps (of 32) per wave per batch
constexpr int kKsp = 4;              // K slices of the adapter intermediate (one producer each)
constexpr int kPairsAhead = 2;       // s*u entries per thread read ahead (x kKsp partials)

struct GemvCodes {
  u32x4 c0, c1;  // 32 bytes of codes = one 64-weight block
  uint32_t q2;   // its scale code; with kQ4, the aligned word holding the
                 // codes of blocks 4j..4j+3 of the row (the byte is picked
                 // when used, so no loaded value is reshaped while in flight)
  float S;
};
struct GemvX {
  u32x4 x[8];  // 64 bf16 of one token row (global-x path only)
};

template <int kW, bool kXL, bool kQ4>
__global__ __launch_bounds__(64 * kW) void k_gemv_fwd(
    const uint8_t *__restrict__ codes, const uint8_t *__restrict__ qscale, const float *__restrict__ smax,
    int d_out, int d_in, const uint16_t *__restrict__ x, int T, const uint16_t *__restrict__ A,
    const uint16_t *__restrict__ B, int r, int r_pad, float scale, uint16_t *__restrict__ h,
    float *__restrict__ u_out, uint64_t *__restrict__ uex, uint32_t *__restrict__ sync, int sshift) {
#define QLORA_GEMV_CID blockIdx.x
#define QLORA_GEMV_G gridDim.x
#include "gemv_body.inc"
#undef QLORA_GEMV_CID
#undef QLORA_GEMV_G
}

// Independent weights in one launch: workgroups wg0[j] .. wg0[j+1]-1 run job j
// as a launch of that many workgroups for that weight alone would (the
// launch's fixed costs, its start and its last workgroups' tails, are paid
// once for all jobs). Every job has its own exchange buffer; the launch tag and
// the status words are shared.
template <int kW, bool kXL, bool kQ4>
__global__ __launch_bounds__(64 * kW) void k_gemv_fwd_many(GemvJobs J, uint32_t *__restrict__ sync) {
  const int b = blockIdx.x;
  int j = 0;
  while (j + 1 < J.n && b >= J.wg0[j + 1]) ++j;  // wave-uniform
  const uint8_t *__restrict__ codes = J.codes[j];
  const uint8_t *__restrict__ qscale = J.qscale[j];
  const float *__restrict__ smax = J.smax[j];
  const int d_out = J.d_out[j], d_in = J.d_in[j], T = J.T[j], r = J.r[j], r_pad = J.r_pad[j], sshift = J.sshift[j];
  const uint16_t *__restrict__ x = J.x[j];
  const uint16_t *__restrict__ A = J.A[j];
  const uint16_t *__restrict__ B = J.B[j];
  const float scale = J.scale[j];
  uint16_t *__restrict__ h = J.h[j];
  float *__restrict__ u_out = J.u_out[j];
  uint64_t *__restrict__ uex = J.uex[j];
  const int cid_j = b - J.wg0[j], G_j = J.wg0[j + 1] - J.wg0[j];
#define QLORA_GEMV_CID cid_j
#define QLORA_GEMV_G G_j
#include "gemv_body.inc"
#undef QLORA_GEMV_CID
#undef QLORA_GEMV_G
}

constexpr int kGvW = 8;  // waves per workgroup

static hipError_t set_gemv_attrs() {
  static DeviceOnce once;
  return once.run(current_device(), [] {
    for (const void *f : {reinterpret_cast<const void *>(k_gemv_fwd<kGvW, true, true>),
                          reinterpret_cast<const void *>(k_gemv_fwd<kGvW, true, false>),
                          reinterpret_cast<const void *>(k_gemv_fwd_many<kGvW, true, true>),
                          reinterpret_cast<const void *>(k_gemv_fwd_many<kGvW, true, false>)}) {
      hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, kXLdsBytes);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  });
}

bool gemv_supported(int64_t d_out, int64_t d_in, int64_t T) {
  // whole-tensor buffer ranges: packed codes (and the rows of one ragged tile) below 2^31 bytes
  return T >= 1 && T <= 16 && (d_out + 16) * d_in / 2 < ((int64_t)1 << 31);
}

hipError_t launch_gemv_fwd(const uint8_t *codes, const uint8_t *qscale, const float *smax, int64_t d_out,
                           int64_t d_in, const uint16_t *x, int64_t T, const uint16_t *A, const uint16_t *B, int r,
                           int r_pad, float scale, uint16_t *h, float *u_out, uint64_t *uex, uint32_t *sync,
                           hipStream_t st) {
  if (r_pad > kMaxRpad || !gemv_supported(d_out, d_in, T)) return hipErrorInvalidValue;
  const int P = r > 0 ? (r_pad / 16) * kKsp : 0;
  const int64_t RT = (d_out + 15) / 16;
  // One workgroup per CU; the first P of them also produce x A^T. The grid never
  // exceeds one residency, so on an otherwise idle chip every workgroup runs
  // concurrently (the kernel does not depend on it: see the file comment).
  const int64_t cus = device_cu_count(current_device());
  int64_t G = RT < cus ? RT : cus;
  if (G < P) G = P;
  const size_t xbytes = (size_t)T * (d_in + kXPad) * 2;
  const int di = (int)d_in, dn = (int)d_out, Tt = (int)T;
  const bool q4 = (d_in / kBlock) % 4 == 0;
  // absmax-only storage: no scale codes (the kernel's q2 range is then empty)
  const int sshift = qscale ? kDqShift : 0;
  const uint8_t *qs = qscale ? qscale : codes;
  if (xbytes <= (size_t)kXLdsBytes) {
    const hipError_t e = set_gemv_attrs();
    if (e != hipSuccess) return e;
    if (q4)
      k_gemv_fwd<kGvW, true, true><<<dim3((unsigned)G), dim3(64 * kGvW), xbytes, st>>>(
          codes, qs, smax, dn, di, x, Tt, A, B, r, r_pad, scale, h, u_out, uex, sync, sshift);
    else
      k_gemv_fwd<kGvW, true, false><<<dim3((unsigned)G), dim3(64 * kGvW), xbytes, st>>>(
          codes, qs, smax, dn, di, x, Tt, A, B, r, r_pad, scale, h, u_out, uex, sync, sshift);
  } else if (q4) {
    k_gemv_fwd<kGvW, false, true><<<dim3((unsigned)G), dim3(64 * kGvW), 0, st>>>(
        codes, qs, smax, dn, di, x, Tt, A, B, r, r_pad, scale, h, u_out, uex, sync, sshift);
  } else {
    k_gemv_fwd<kGvW, false, false><<<dim3((unsigned)G), dim3(64 * kGvW), 0, st>>>(
        codes, qs, smax, dn, di, x, Tt, A, B, r, r_pad, scale, h, u_out, uex, sync, sshift);
  }
  return hipGetLastError();
}

// Grouped launches. Jobs share a launch when they take the same kernel variant
// (x staged in LDS or not; blocks per row a multiple of 4 or not), at most
// kGemvJobs of them, and while their producers fill at most half of the compute
// units. Within a launch the compute units are shared out in proportion to
// each job's weight bytes, each job getting at least its producers and at most
// one workgroup per row tile, so that the grid stays within one residency.
static size_t gemv_xbytes(const GemvJob &j) { return (size_t)j.T * (j.d_in + kXPad) * 2; }
static int gemv_producers(const GemvJob &j) { return j.r > 0 ? (j.r_pad / 16) * kKsp : 0; }

static hipError_t launch_group(const GemvJob *const *g, int n, uint32_t *sync, bool xl, bool q4, int64_t cus,
                               hipStream_t st) {
  GemvJobs J{};
  J.n = n;
  int64_t wsum = 0, grid = 0;
  int64_t G[kGemvJobs], W[kGemvJobs], RT[kGemvJobs], lo[kGemvJobs];
  for (int i = 0; i < n; ++i) {
    RT[i] = (g[i]->d_out + 15) / 16;
    W[i] = RT[i] * (g[i]->d_in / kBlock);
    wsum += W[i];
  }
  for (int i = 0; i < n; ++i) {
    lo[i] = std::max<int64_t>(gemv_producers(*g[i]), 1);
    G[i] = std::max(lo[i], std::min(RT[i], cus * W[i] / wsum));
    grid += G[i];
  }
  // compute units left over go one at a time to the job with the most weight per workgroup
  while (grid < cus) {
    int best = -1;
    for (int i = 0; i < n; ++i)
      if (G[i] < RT[i] && (best < 0 || W[i] * G[best] > W[best] * G[i])) best = i;
    if (best < 0) break;
    ++G[best];
    ++grid;
  }
  // the producers' minimums can push the total past one residency (the launcher keeps them to half of it):
  // take workgroups back from the jobs with the least weight per workgroup
  while (grid > cus) {
    int best = -1;
    for (int i = 0; i < n; ++i)
      if (G[i] > lo[i] && (best < 0 || W[i] * G[best] < W[best] * G[i])) best = i;
    if (best < 0) break;
    --G[best];
    --grid;
  }
  size_t lds = 0;
  int64_t wg = 0;
  for (int i = 0; i < n; ++i) {
    const GemvJob &j = *g[i];
    J.codes[i] = j.codes;
    J.qscale[i] = j.qscale ? j.qscale : j.codes;  // absmax-only storage: no scale codes (an empty q2 range)
    J.smax[i] = j.smax;
    J.x[i] = j.x;
    J.A[i] = j.A;
    J.B[i] = j.B;
    J.h[i] = j.h;
    J.u_out[i] = j.u_out;
    J.uex[i] = j.uex;
    J.scale[i] = j.scale;
    J.d_out[i] = (int)j.d_out;
    J.d_in[i] = (int)j.d_in;
    J.T[i] = (int)j.T;
    J.r[i] = j.r;
    J.r_pad[i] = j.r_pad;
    J.sshift[i] = j.qscale ? kDqShift : 0;
    J.wg0[i] = (int)wg;
    wg += G[i];
    if (xl) lds = std::max(lds, gemv_xbytes(j));
  }
  J.wg0[n] = (int)wg;
  const dim3 grd((unsigned)wg), blk(64 * kGvW);
  if (xl && q4)
    k_gemv_fwd_many<kGvW, true, true><<<grd, blk, lds, st>>>(J, sync);
  else if (xl)
    k_gemv_fwd_many<kGvW, true, false><<<grd, blk, lds, st>>>(J, sync);
  else if (q4)
    k_gemv_fwd_many<kGvW, false, true><<<grd, blk, 0, st>>>(J, sync);
  else
    k_gemv_fwd_many<kGvW, false, false><<<grd, blk, 0, st>>>(J, sync);
  return hipGetLastError();
}

hipError_t launch_gemv_fwd_many(const GemvJob *jobs, int n, uint32_t *sync, hipStream_t st) {
  for (int i = 0; i < n; ++i)
    if (jobs[i].r_pad > kMaxRpad || !gemv_supported(jobs[i].d_out, jobs[i].d_in, jobs[i].T))
      return hipErrorInvalidValue;
  const hipError_t e = set_gemv_attrs();
  if (e != hipSuccess) return e;
  const int64_t cus = device_cu_count(current_device());
  for (int cls = 0; cls < 4; ++cls) {
    const bool xl = (cls & 2) != 0, q4 = (cls & 1) != 0;
    const GemvJob *g[kGemvJobs];
    int m = 0, prod = 0;
    for (int i = 0; i <= n; ++i) {
      const bool mine = i < n && (gemv_xbytes(jobs[i]) <= (size_t)kXLdsBytes) == xl &&
                        ((jobs[i].d_in / kBlock) % 4 == 0) == q4;
      const int p = mine ? std::max(gemv_producers(jobs[i]), 1) : 0;
      if (m > 0 && (i == n || (mine && (m == kGemvJobs || 2 * (prod + p) > cus)))) {
        const hipError_t le = launch_group(g, m, sync, xl, q4, cus, st);
        if (le != hipSuccess) return le;
        m = prod = 0;
      }
      if (mine) {
        g[m++] = &jobs[i];
        prod += p;
      }
    }
  }
  return hipSuccess;
}

}  // namespace qlora
