// Internal host-side launchers of the gfx950 kernels. Called only by api.cpp after
// argument validation; every launcher enqueues on `st` and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "common.h"
#include "qlora.h"

namespace qlora {

// Per-device one-time set-up of a launcher (function attributes): the first
// call on a device runs `fn` under a once flag, every call returns its status.
// Safe to use from any number of host threads.
constexpr int kMaxDevices = 64;
struct DeviceOnce {
  std::once_flag flag[kMaxDevices];
  hipError_t status[kMaxDevices] = {};
  template <class F>
  hipError_t run(int dev, F &&fn) {
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::call_once(flag[dev], [&] { status[dev] = fn(); });
    return status[dev];
  }
};
// api.cpp: the current device (-1 if it cannot be read) and its compute-unit
// count (read once per device; 256 if the query fails).
int current_device();
int device_cu_count(int dev);

// api.cpp: the forward's argument checks, the workspace bytes one forward call
// touches, and its kernels on a checked workspace (used by the entry points of
// api.cpp and scratch.hip). r must already be 0 when A = B = NULL for the last two.
int validate_forward(const qlora_nf4_weight *W, const uint16_t *x, int64_t T, const uint16_t *A, const uint16_t *B,
                     int32_t r, uint16_t *h, float *u_out);
size_t forward_workspace_need(int64_t d_out, int64_t d_in, int64_t T, int r);
int enqueue_forward(const qlora_nf4_weight *W, const uint16_t *x, int64_t T, const uint16_t *A, const uint16_t *B,
                    int32_t r, float alpha, uint16_t *h, float *u_out, void *ws, hipStream_t stream);

// quantize.hip
// Up to kQuantizeJobs weights per launch, passed by value as a kernel
// argument (no device buffer): job i covers global groups
// [gstart[i], gstart[i+1]); qscale[i] == NULL selects absmax-only storage.
constexpr int kQuantizeJobs = 32;
struct QuantizeJobs {
  const void *W[kQuantizeJobs];
  uint8_t *codes[kQuantizeJobs];
  uint8_t *qscale[kQuantizeJobs];
  float *smax[kQuantizeJobs];
  int64_t nblocks[kQuantizeJobs];
  int64_t gstart[kQuantizeJobs + 1];
  int n;
};
hipError_t launch_quantize(const QuantizeJobs &jobs, bool bf16_in, uint32_t *flags, const Nf4Consts &c,
                           hipStream_t st);
hipError_t launch_dequantize(const uint8_t *codes, const uint8_t *qscale, const float *smax,
                             int64_t d_out, int64_t d_in, bool bf16_out, void *out, const Nf4Consts &c,
                             hipStream_t st);

// adamw.hip: one AdamW step over n float32 elements (see the kernel file).
// grad, master, m, v are device-accessible addresses (pinned host memory
// mapped for the device, or device memory); param (nullable, device) receives
// bf16(master). host_state: some operand is in host memory, so the step is
// bound by the host link rather than HBM.
struct AdamWArgs {
  float lr, b1, b2, one_minus_b1, one_minus_b2, eps, decay, c1, c2;
};
hipError_t launch_adamw(const float *grad, float *master, float *m, float *v, uint16_t *param, int64_t n,
                        const AdamWArgs &a, bool host_state, hipStream_t st);

// merge.hip: out[d_out, d_in] = bf16(W_hat + scale B A), A [r, d_in], B [d_out, r] bf16 (r may be 0).
hipError_t launch_merge(const uint8_t *codes, const uint8_t *qscale, const float *smax, int64_t d_out, int64_t d_in,
                        const uint16_t *A, const uint16_t *B, int r, float scale, uint16_t *out, hipStream_t st);

// lora_small.hip: out[T, r] = P[T, K] . Q^T with Q given as [r, K] (K contiguous).
// Writes out_f32 (nullable) and out_bf16 = bf16(scale * out) with row pitch r_pad
// (zero-filled up to r_pad, a multiple of 16). Uses `partial` (ksplit*16*r_pad f32
// per 16-token tile) and `counters` (one tile_counter per 16-token tile) when ksplit > 1.
hipError_t launch_lora_small(const uint16_t *P, const uint16_t *Q, int64_t T, int64_t K, int r,
                             float scale, float *out_f32, uint16_t *out_bf16, int r_pad, float *partial,
                             uint32_t *counters, int ksplit, hipStream_t st);
// B [rows, cols] bf16 -> Bt [cols, rows] bf16
hipError_t launch_transpose_bf16(const uint16_t *src, int64_t rows, int64_t cols, uint16_t *dst,
                                 hipStream_t st);

// gemv.hip: T <= 16, one launch:
// h[T, d_out] = x W_hat^T + scale (x A^T) B^T. u_out (nullable) receives x A^T
// [T, r]. uex is the [4, 16, r_pad] exchange buffer of tagged float32 partials
// of x A^T (one per quarter of K); sync points at four reserved words (word 3
// counts the workgroups whose wait for a partial ran out of time and which then
// formed it themselves; the result does not depend on it).
hipError_t launch_gemv_fwd(const uint8_t *codes, const uint8_t *qscale, const float *smax, int64_t d_out,
                           int64_t d_in, const uint16_t *x, int64_t T, const uint16_t *A, const uint16_t *B, int r,
                           int r_pad, float scale, uint16_t *h, float *u_out, uint64_t *uex, uint32_t *sync,
                           hipStream_t st);
// Whether the T <= 16 kernel takes these sizes (its buffer ranges cover whole tensors).
bool gemv_supported(int64_t d_out, int64_t d_in, int64_t T);
// Several independent T <= 16 forwards (launch_gemv_fwd's arguments, each with
// its own exchange buffer uex) in as few launches as their kernel variants
// allow; the status words `sync` are shared. The kernel argument of one launch:
// job j runs on workgroups wg0[j] .. wg0[j+1]-1.
struct GemvJob {
  const uint8_t *codes, *qscale;
  const float *smax;
  int64_t d_out, d_in;
  const uint16_t *x;
  int64_t T;
  const uint16_t *A, *B;
  int r, r_pad;
  float scale;
  uint16_t *h;
  float *u_out;
  uint64_t *uex;
};
constexpr int kGemvJobs = 8;
struct GemvJobs {
  const uint8_t *codes[kGemvJobs];
  const uint8_t *qscale[kGemvJobs];
  const float *smax[kGemvJobs];
  const uint16_t *x[kGemvJobs];
  const uint16_t *A[kGemvJobs];
  const uint16_t *B[kGemvJobs];
  uint16_t *h[kGemvJobs];
  float *u_out[kGemvJobs];
  uint64_t *uex[kGemvJobs];
  float scale[kGemvJobs];
  int d_out[kGemvJobs], d_in[kGemvJobs], T[kGemvJobs], r[kGemvJobs], r_pad[kGemvJobs], sshift[kGemvJobs];
  int wg0[kGemvJobs + 1];
  int n;
};
hipError_t launch_gemv_fwd_many(const GemvJob *jobs, int n, uint32_t *sync, hipStream_t st);

// gemm.hip: T > 16 (and any T the weight-streaming kernel does not take).
// Work split of one contraction over 256 x 256 output tiles (gm x gn of them,
// nk K steps of 64 each): tiles 0 .. full-1 run whole, one workgroup each; each
// of the remaining `rem` tiles is cut into `split` K ranges run by separate
// workgroups, which store their float32 partial tiles (gemm_partial_floats in
// total, in the workspace's shared scratch region) and sum the tile's rows in
// range order, one share each (split_arrive in common.h). Chosen so
// that the chip's last round of tiles is not left mostly idle; depends on the
// current device's compute-unit count.
struct GemmPlan {
  int gm, gn, nk, full, rem, split;
};
GemmPlan gemm_plan(int64_t M, int64_t N, int64_t nk);
size_t gemm_partial_floats(const GemmPlan &p);
hipError_t launch_gemm_fwd(const uint8_t *codes, const uint8_t *qscale, const float *smax, int64_t d_out,
                           int64_t d_in, const uint16_t *x, int64_t T, const uint16_t *su, int r_pad,
                           const uint16_t *B, int r, uint16_t *h, float *partial, uint32_t *counters,
                           hipStream_t st);
// dX[T, d_in] = dY W_hat + sv A (sv = bf16(s*v) [T, r_pad], A [r, d_in]).
hipError_t launch_gemm_dx(const uint8_t *codes, const uint8_t *qscale, const float *smax, int64_t d_out,
                          int64_t d_in, const uint16_t *dY, int64_t T, const uint16_t *sv, int r_pad,
                          const uint16_t *A, int r, uint16_t *dX, float *partial, uint32_t *counters,
                          hipStream_t st);

// lora_wide.hip: the adapter products for T >= kWideMinTokens.
constexpr int64_t kWideMinTokens = 65;
// out[T, r] = P[T, K] . Q[r, K]^T (u = x A^T, v = dY B with Q = B^T); writes
// out_f32 [T, r] (nullable) and out_bf16 = bf16(scale * out) [T, r_pad]
// (nullable, zero columns r .. r_pad-1). Uses `partial`
// (lora_tall_partial_floats) and `counters` (one tile_counter per 64-token tile).
hipError_t launch_lora_tall(const uint16_t *P, const uint16_t *Q, int64_t T, int64_t K, int r, int r_pad, float scale,
                            float *out_f32, uint16_t *out_bf16, float *partial, uint32_t *counters, hipStream_t st);
size_t lora_tall_partial_floats(int64_t T, int64_t K, int r_pad);
// X bf16 [T, D], Y float32 [T, R]. y_is_rows: C[R, D] = scale * Y^T X (dA);
// otherwise C[D, R] = scale * X^T Y (dB). Uses `partial`
// (lora_wgrad_partial_floats) and `counters` (one tile_counter per output tile); counts in
// *fallbacks the waits that ran out of time (the result does not depend on them).
hipError_t launch_lora_wgrad(const uint16_t *X, const float *Y, int64_t T, int64_t D, int64_t R, bool y_is_rows,
                             float scale, float *C, float *partial, uint32_t *counters, uint32_t *fallbacks,
                             hipStream_t st);
size_t lora_wgrad_partial_floats(int64_t D, int64_t R, int64_t T);

// lora_grad.hip: C[M, N] = scale * sum_t P[t, m] Q[t, n] over t < T.
// P and Q are each bf16 or f32 (an f32 operand is split into two bf16 terms).
hipError_t launch_lora_grad(const void *P, bool P_f32, int64_t M, const void *Q, bool Q_f32, int64_t N,
                            int64_t T, float scale, float *C, float *partial, uint32_t *counters,
                            int ksplit, hipStream_t st);
int lora_grad_ksplit(int64_t M, int64_t N, int64_t T);
size_t lora_grad_partial_floats(int64_t M, int64_t N, int64_t T);
int lora_grad_tiles(int64_t M, int64_t N);

}  // namespace qlora
