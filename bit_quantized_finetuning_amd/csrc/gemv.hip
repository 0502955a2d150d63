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
  // All kernel arguments in one scalar-memory round trip (left alone, the
  // compiler fetches them in dependent batches at first use).
  asm volatile("; kernel arguments" ::"s"(codes), "s"(qscale), "s"(smax), "s"(d_out), "s"(d_in), "s"(x), "s"(T),
               "s"(A), "s"(B), "s"(r), "s"(r_pad), "s"(scale), "s"(h), "s"(u_out), "s"(uex), "s"(sync),
               "s"(sshift), "s"(gridDim.x));
  constexpr int kThreads = 64 * kW;
  extern __shared__ __attribute__((aligned(16))) uint16_t x_l[];  // [T][d_in + kXPad] when kXL
  __shared__ float red[kW][256];
  __shared__ __attribute__((aligned(16))) uint16_t su_l[16 * kMaxRpad];
  __shared__ int poll_bad[2][kW];
  __shared__ int poll_late[2];
  __shared__ uint32_t miss[2];  // jobs with a partial not yet seen (bit j kKsp + ks)
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int li = lane & 15, g = lane >> 4;
  if (tid == 0) miss[0] = miss[1] = 0u;  // read only after later barriers (the fallback of the exchange)
  const int P = r > 0 ? (r_pad / 16) * kKsp : 0;
  const int KB = d_in / kBlock;
  const int cid = blockIdx.x, G = gridDim.x;
  const int xpitch = d_in + kXPad;
  const int RT = (d_out + 15) / 16;
  const int rt0 = G - 1 - cid;  // row tiles rt0, rt0 + G, ... (the producers, first, get the fewest)
  const int nrt = rt0 < RT ? (RT - rt0 + G - 1) / G : 0;
  const int NS = (KB + 3) / 4;
  // Segments seg = wv + kW s of every row tile belong to wave slot wv; the slot
  // is rotated per workgroup so that at any moment different workgroups read
  // different parts of x (every CU reads all of x).
  const int wv = (wave + cid) % kW;
  const int mseg = NS > wv ? (NS - wv + kW - 1) / kW : 0;  // my segments per row tile
  const int nblocks = d_out * KB;
  const rsrc_t cr = make_rsrc(codes, (int64_t)nblocks * (kBlock / 2));
  // absmax-only storage (sshift 0): an empty q2 range (loads return 0) and one scale per block
  const rsrc_t qr = make_rsrc(qscale, sshift ? nblocks : 0);
  const rsrc_t sr = make_rsrc(smax, scale_words(nblocks, sshift) * 4);
  const uint32_t q2o = q2_or(sshift);
  const rsrc_t xr = make_rsrc(x, (int64_t)T * d_in * 2);

  // Item (row tile k, segment s): lane (li, g) takes block g of the segment in
  // row 16 (c + kG) + li. Rows past d_out (ragged tile, k >= nrt) read zeros.
  auto load_codes = [&](int k, int s, GemvCodes &st) {
    const int row = (rt0 + k * G) * 16 + li;
    const int kb = 4 * (wv + kW * s) + g;
    const bool ok = row < d_out && kb < KB;
    const uint32_t blk = (uint32_t)row * (uint32_t)KB + (uint32_t)kb;
    st.c0 = bld16(cr, ok ? blk * 32u : kOOB);
    st.c1 = bld16(cr, ok ? blk * 32u + 16u : kOOB);
    // kQ4 (blocks per row a multiple of 4): the word of blocks kb - g .. kb - g + 3
    // lies in the row, so inside the tensor
    st.q2 = kQ4 ? bld32(qr, ok ? (blk & ~3u) : kOOB) : bld8(qr, ok ? blk : kOOB);
    st.S = __uint_as_float(bld32(sr, ok ? (blk >> sshift) * 4u : kOOB));
  };
  auto load_x = [&](int s, GemvX &st) {
    const int kb = 4 * (wv + kW * s) + g;
    const uint32_t xoff = kb < KB ? (uint32_t)((li * d_in + kb * kBlock) * 2) : kOOB;
#pragma unroll
    for (int m = 0; m < 8; ++m) st.x[m] = bld16(xr, xoff + 16 * m);
  };

  // ---------------- loads in the order they are needed ----------------
  // Loads complete in issue order, so everything a step waits for goes out
  // before the loads it does not need yet.

  // Job (j, ks) = id j kKsp + ks: the partial of u columns 16j..16j+15 over K
  // slice ks (A rows 16j..16j+15; steps of 32 split over the waves). A CU
  // streams only a few tens of GB/s on its own, so the A reads are spread over
  // kKsp producers per column tile. Producer workgroup c runs job c.
  const bool producer = P > 0 && cid < P;
  const int nk32 = d_in / 32;
  u32x4 ap[kABatch], xp[kABatch];
  auto a_issue = [&](int job, int b) {
    const int pj = job / kKsp, pks = job % kKsp;
    const int k32b = nk32 * pks / kKsp, k32e = nk32 * (pks + 1) / kKsp;
    const int arows = r - 16 * pj < 16 ? r - 16 * pj : 16;
    const rsrc_t ar = make_rsrc(A + (int64_t)16 * pj * d_in, (int64_t)arows * d_in * 2);
#pragma unroll
    for (int s = 0; s < kABatch; ++s) {
      const int k32 = k32b + wave + kW * (kABatch * b + s);
      const uint32_t off = k32 < k32e ? (uint32_t)((li * d_in + k32 * 32 + 8 * g) * 2) : kOOB;
      ap[s] = bld16(ar, off);
      xp[s] = bld16(xr, off);  // x row li has the same offsets as A row li
    }
  };

  // x staging, per wave: only the 256-column segments this wave computes with
  // (a producer workgroup stages all of x the same way, then joins up). Load i
  // of a segment covers tokens 2i, 2i+1: lane l takes token 2i + l/32,
  // columns 8 (l % 32) .. + 8. Two segments go per batch.
  constexpr int kXSeg = 2;
  u32x4 xs[kXSeg][8];
  auto x_addr = [&](int j, int i, int &t, int &col) {
    t = 2 * i + (lane >> 5);
    col = 256 * (wv + kW * j) + 8 * (lane & 31);
    return j < mseg && t < T && col < d_in;
  };
  auto x_issue = [&](int j0) {
#pragma unroll
    for (int jj = 0; jj < kXSeg; ++jj)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        int t, col;
        const bool ok = x_addr(j0 + jj, i, t, col);
        xs[jj][i] = bld16(xr, ok ? (uint32_t)((t * d_in + col) * 2) : kOOB);
      }
  };
  auto x_store = [&](int j0) {
#pragma unroll
    for (int jj = 0; jj < kXSeg; ++jj)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        int t, col;
        if (x_addr(j0 + jj, i, t, col)) st16(x_l + t * xpitch + col, xs[jj][i]);
      }
  };
  // A producer's own operands go out first: its job needs nothing else.
  if (producer) a_issue(cid, 0);
  if (kXL && mseg > 0) x_issue(0);

  // Items (row tile k, segment s) in order k * mseg + s, through a ring of
  // kStages register stages: kStages - 1 items are in flight while one is
  // computed. Two stages measure fastest: the restore (about 270 VALU
  // instructions per wave and item) and the fixed launch and first-load
  // latency bound this kernel, not the bytes in flight, and deeper rings
  // (3 or 4 stages, measured) only delay the first data. Items past the last
  // row tile read rows >= d_out, which load as zeros without touching memory.
  constexpr int kStages = 2;
  GemvCodes cq[kStages];
  GemvX xg[kXL ? 1 : kStages];
  auto advance = [&](int &k, int &s) {
    if (++s == mseg) {
      s = 0;
      ++k;
    }
  };
  int kl = 0, sl = 0;  // next item to load
  if (mseg > 0) {
#pragma unroll
    for (int j = 0; j + 1 < kStages; ++j) {
      load_codes(kl, sl, cq[j]);
      if (!kXL) load_x(sl, xg[j]);
      advance(kl, sl);
      // the stages go out in ring order (the waits count on it)
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  u32x4 bpre[2] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
  const rsrc_t br = make_rsrc(B, (int64_t)d_out * r * 2);
  auto load_b = [&](int k) {
    const int row = (rt0 + k * G) * 16 + li;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int j = 32 * q + 8 * g;
      const bool ok = j < r && row < d_out;
      bpre[q] = bld16(br, ok ? (uint32_t)((row * r + j) * 2) : kOOB);
    }
  };
  if (P > 0 && wave == 0) load_b(0);

  // ---------------- adapter producer job ----------------
  // The partial of columns 16j..16j+15 of u = x A^T over K slice ks, with the
  // loads of its first batch already issued: the waves split the slice and
  // reduce through LDS; each float32 value goes out with this launch's tag in
  // one 64-bit store. Nothing waits for those stores: a reader accepts an
  // entry once its tag matches. (Run by every wave of the workgroup.)
  const uint32_t tag = launch_tag();
  // The waves' partials of a job: reduce through LDS in wave order and publish with the tag.
  auto a_publish = [&](int job, const f32x4 &pacc) {
    const int pj = job / kKsp, pks = job % kKsp;
    // lane (li, g) holds u[4g + i][16j + li]
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][(4 * g + i) * 16 + li] = pacc[i];
    lds_barrier();
    if (tid < 256) {
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < kW; ++w) v += red[w][tid];
      const int t = tid >> 4, col = 16 * pj + (tid & 15);
      if (t < T) st_dev_u64(uex + (pks * 16 + t) * r_pad + col, (uint64_t)__float_as_uint(v) | ((uint64_t)tag << 32));
    }
    lds_barrier();
  };
  auto a_run = [&](int job) {
    const int pks = job % kKsp;
    const int k32b = nk32 * pks / kKsp, k32e = nk32 * (pks + 1) / kKsp;
    f32x4 pacc = {0.f, 0.f, 0.f, 0.f};
    for (int b = 0;; ++b) {
#pragma unroll
      for (int s = 0; s < kABatch; ++s)
        if (k32b + wave + kW * (kABatch * b + s) < k32e) pacc = mfma16(xp[s], ap[s], pacc);  // wave-uniform
      if (k32b + kABatch * kW * (b + 1) >= k32e) break;
      a_issue(job, b + 1);
    }
    a_publish(job, pacc);
  };
  // The same job one K step at a time, for the rare reader that forms a missing
  // partial itself: the same MFMA operands in the same order as a_run, so the
  // same bits, in a fraction of a_run's code (it sits in the epilogue, which the
  // item loop holds twice, and its size alone slowed every launch by 7 %).
  auto a_run_cold = [&](int job) {
    const int pj = job / kKsp, pks = job % kKsp;
    const int k32b = nk32 * pks / kKsp, k32e = nk32 * (pks + 1) / kKsp;
    const int arows = r - 16 * pj < 16 ? r - 16 * pj : 16;
    const rsrc_t ar = make_rsrc(A + (int64_t)16 * pj * d_in, (int64_t)arows * d_in * 2);
    f32x4 pacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
    for (int k32 = k32b + wave; k32 < k32e; k32 += kW) {
      const uint32_t off = (uint32_t)((li * d_in + k32 * 32 + 8 * g) * 2);
      pacc = mfma16(bld16(xr, off), bld16(ar, off), pacc);
    }
    a_publish(job, pacc);
  };
  // x comes straight from global memory (rows >= T read zeros), so the job
  // waits for nothing but its own loads, issued first.
  if (producer) a_run(cid);

  if (kXL && mseg > 0) {
    x_store(0);
    for (int j0 = kXSeg; j0 < mseg; j0 += kXSeg) {
      x_issue(j0);
      x_store(j0);
    }
  }
  // This wave reads back only what it wrote: order its LDS stores before its
  // loads without involving the other waves.
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");

  // ---------------- s*u exchange: read ahead, check at the first row-tile end ----------------
  // Thread tid owns entries (t, col) = tid + i kThreads of the T x r_pad
  // intermediate and reads their kKsp partials; the first kPairsAhead go out
  // before the last item of the first row tile. (A second round kept in
  // flight measured slower: every round reads all kKsp tagged partials, which
  // competes with the weight stream.)
  const int npair = T * r_pad;
  uint64_t pv0[kPairsAhead][kKsp];
  auto poll_load = [&](int i, uint64_t (&dst)[kKsp]) {
    const int p = tid + i * kThreads;
    const int t = p / r_pad, col = p - t * r_pad;
#pragma unroll
    for (int ks = 0; ks < kKsp; ++ks)
      dst[ks] = p < npair ? ld_dev_u64(uex + (ks * 16 + t) * r_pad + col) : ((uint64_t)tag << 32);
  };
  bool polled = false;
  auto poll_issue = [&](uint64_t (&pv)[kPairsAhead][kKsp]) {
#pragma unroll
    for (int i = 0; i < kPairsAhead; ++i) poll_load(i, pv[i]);
    polled = true;
  };

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int s, const GemvCodes &cs, const GemvX &xs2) {
    const Nf4Planes t = make_planes(restore_scale((kQ4 ? (cs.q2 >> (8 * g)) & 0xffu : cs.q2) | q2o, cs.S));
    // LDS path: token rows >= T only feed accumulator rows that are never stored,
    // and a block past the row end has an all-zero restore table, so both read
    // clamped, staged x without masking
    // (a block past the row end reads the segment's first block, which this wave staged)
    const int kbl = 4 * (wv + kW * s) + g;
    const uint16_t *xq = x_l + (li < T ? li : 0) * xpitch + (kbl < KB ? kbl : 4 * (wv + kW * s)) * kBlock;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const u32x4 a = kXL ? *reinterpret_cast<const u32x4 *>(xq + 8 * m) : xs2.x[m];
      acc = mfma16(a, expand8(t, m < 4 ? cs.c0[m] : cs.c1[m - 4]), acc);
    }
  };

  // Row-tile epilogue: adapter columns (wave 0), LDS reduce across waves, store h.
  auto epilogue = [&](int k) {
    const int row0 = (rt0 + k * G) * 16;
    const int rows = d_out - row0 < 16 ? d_out - row0 : 16;
    if (P > 0 && k == 0) {
      // bf16(s*u) rows t < T into LDS once every tag matches: u is the sum of
      // the kKsp partials in slice order (the same on every workgroup); the
      // workgroup of row tile 0 also writes float32 u. Rows t >= T of su_l
      // only feed accumulator rows that are never stored.
      // One round: write every entry whose partials all carry this launch's
      // tag, note in a register the jobs of those that do not, and (thread 0)
      // whether the wait has run out of time; returns whether any entry of the
      // workgroup was not ready (two flag rows in turn: a row is rewritten only
      // two barriers after it was last read). The job masks meet in LDS only
      // when the wait has run out.
      const long long t0 = wall_clock64(), limit = wait_limit(&sync[3]);
      uint64_t mymiss = 0;
      auto check = [&](const uint64_t (&pv)[kPairsAhead][kKsp], int it) {
        int bad = 0;
        mymiss = 0;
        for (int i = 0; i * kThreads < npair; ++i) {
          uint64_t e[kKsp];
          if (i < kPairsAhead) {
#pragma unroll
            for (int ks = 0; ks < kKsp; ++ks) e[ks] = pv[i < kPairsAhead ? i : 0][ks];
          } else {
            poll_load(i, e);
          }
          const int p = tid + i * kThreads;
          bool ok = true;
          float u = 0.f;
#pragma unroll
          for (int ks = 0; ks < kKsp; ++ks) {
            const bool oks = (uint32_t)(e[ks] >> 32) == tag;
            ok = ok && oks;
            const int job = ((p - (p / r_pad) * r_pad) >> 4) * kKsp + ks;
            mymiss |= oks ? 0ull : 1ull << job;
            u += __uint_as_float((uint32_t)e[ks]);
          }
          if (!ok) {
            bad = 1;
          } else if (p < npair) {
            const int t = p / r_pad, col = p - t * r_pad;
            su_l[t * r_pad + col] = (uint16_t)(pack_bf16x2(col < r ? scale * u : 0.f, 0.f) & 0xffffu);
            if (u_out && rt0 == 0 && col < r) u_out[t * r + col] = u;
          }
        }
        const int wbad = __builtin_amdgcn_readfirstlane(__ballot(bad) != 0ull ? 1 : 0);
        if (lane == 0) poll_bad[it & 1][wave] = wbad;
        if (tid == 0) poll_late[it & 1] = wall_clock64() - t0 > limit ? 1 : 0;
        lds_barrier();
        int any = 0;
#pragma unroll
        for (int w = 0; w < kW; ++w) any |= poll_bad[it & 1][w];
        return any != 0;
      };
      if (!polled) poll_issue(pv0);
      for (int it = 0;; ++it) {
        if (!check(pv0, it)) break;
        if (poll_late[it & 1]) {
          // form the missing partials here, exactly as their producers would,
          // and publish them; the next round then finds every entry
          if (mymiss) {
            atomicOr(&miss[0], (uint32_t)mymiss);
            atomicOr(&miss[1], (uint32_t)(mymiss >> 32));
          }
          lds_barrier();
          const uint32_t m0 = miss[0], m1 = miss[1];
          for (int job = 0; job < P; ++job) {
            if (!(((job < 32 ? m0 : m1) >> (job & 31)) & 1u)) continue;
            a_run_cold(job);
          }
          if (tid == 0) {
            miss[0] = miss[1] = 0u;
            add_dev_u32(&sync[3], 1u);
          }
          wait_vmem();  // the published entries are in memory before anyone polls again
          lds_barrier();
        } else {
          __builtin_amdgcn_s_sleep(2);
        }
        poll_issue(pv0);
      }
    }
    if (P > 0 && wave == 0) {
      // adapter K columns of this row tile: a = s*u (LDS), b = B rows
      for (int j0 = 0; j0 < r_pad; j0 += 32) {
        const int j = j0 + 8 * g;
        const u32x4 a = j < r_pad ? *reinterpret_cast<const u32x4 *>(su_l + li * r_pad + j) : u32x4{0u, 0u, 0u, 0u};
        u32x4 b;
        if (j0 < 64) {
          b = bpre[j0 >> 5];
        } else {
          const bool ok = j < r && row0 + li < d_out;
          b = bld16(br, ok ? (uint32_t)(((row0 + li) * r + j) * 2) : kOOB);
        }
        acc = mfma16(a, b, acc);
      }
      if (k + 1 < nrt) load_b(k + 1);
    }
    // Lane (li, g) holds tokens 4g..4g+3 of row li.
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][(4 * g + i) * 16 + li] = acc[i];
    acc = f32x4{0.f, 0.f, 0.f, 0.f};
    lds_barrier();
    if (tid < 256) {
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < kW; ++w) v += red[w][tid];
      const int t = tid >> 4, rl = tid & 15;
      if (t < T && rl < rows) h[t * d_out + row0 + rl] = (uint16_t)(pack_bf16x2(v, 0.f) & 0xffffu);
    }
    lds_barrier();
  };

  if (mseg == 0) {
    for (int k = 0; k < nrt; ++k) epilogue(k);
  } else {
    // The ring, unrolled kStages times so that every stage has fixed registers:
    // step u refills the stage freed by step u - 1, then computes stage u.
    // The loop has one exit, after a whole turn of the ring (the item count is
    // rounded up; items past the last row tile compute on zeros and skip the
    // epilogue), and the steps keep their order: then each stage's wait
    // covers only its own loads. (An exit inside the turn, or loads moved
    // across steps, makes the compiler wait for every stage at once.)
    const int nitems = nrt * mseg;
    int k = 0, s = 0;  // item being computed
    for (int i = 0; i < nitems; i += kStages) {
#pragma unroll
      for (int u = 0; u < kStages; ++u) {
        load_codes(kl, sl, cq[(u + kStages - 1) % kStages]);
        if (!kXL) load_x(sl, xg[(u + kStages - 1) % kStages]);
        advance(kl, sl);
        __builtin_amdgcn_sched_barrier(0);
        if (P > 0 && k == 0 && s == mseg - 1) poll_issue(pv0);
        compute(s, cq[u], xg[kXL ? 0 : u]);
        if (s == mseg - 1 && k < nrt) epilogue(k);
        advance(k, s);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
}

constexpr int kGvW = 8;  // waves per workgroup

static hipError_t set_gemv_attrs() {
  static DeviceOnce once;
  return once.run(current_device(), [] {
    for (const void *f : {reinterpret_cast<const void *>(k_gemv_fwd<kGvW, true, true>),
                          reinterpret_cast<const void *>(k_gemv_fwd<kGvW, true, false>)}) {
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

}  // namespace qlora
