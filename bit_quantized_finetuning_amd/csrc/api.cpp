// C ABI of the QLoRA frozen-NF4 linear layer: validation, workspace layout and
// kernel dispatch. Every entry point validates all arguments on the host before
// enqueuing anything; the library allocates no memory.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

#include "qlora.h"
#include "kernels.h"

using namespace qlora;

namespace {

// ---------------------------------------------------------------------------
// NF4 codebook: normal quantiles with an exact zero, dense near zero ("48GB GPU
// Fine-Tuning a 65B Model", section "Quantization Keeps the Patterns..."):
// 8 positive levels Phi^-1(1/2 + (p - 1/2) j/8), j = 1..8, 7 negative levels
// -Phi^-1(1/2 + (p - 1/2) j/7), j = 1..7, and 0, with p = ((1-1/30)+(1-1/32))/2,
// divided by Phi^-1(p) so the extremes are exactly +-1, rounded to float32.
// The quantile is found by bisection on Phi(x) = erfc(-x/sqrt(2))/2 in double.
// ---------------------------------------------------------------------------
double normal_quantile(double p) {
  double lo = -12.0, hi = 12.0;
  for (int it = 0; it < 400; ++it) {
    const double mid = 0.5 * (lo + hi);
    if (mid <= lo || mid >= hi) break;
    if (0.5 * std::erfc(-mid / std::sqrt(2.0)) < p)
      lo = mid;
    else
      hi = mid;
  }
  return 0.5 * (lo + hi);
}

struct Tables {
  Nf4Consts c;
  Tables() {
    const double p = 0.5 * ((1.0 - 1.0 / 30.0) + (1.0 - 1.0 / 32.0));
    std::vector<double> v;
    for (int j = 1; j <= 8; ++j) v.push_back(normal_quantile(0.5 + (p - 0.5) * j / 8.0));
    for (int j = 1; j <= 7; ++j) v.push_back(-normal_quantile(0.5 + (p - 0.5) * j / 7.0));
    v.push_back(0.0);
    std::sort(v.begin(), v.end());
    const double top = normal_quantile(p);
    for (int j = 0; j < 16; ++j) c.code[j] = (float)(v[j] / top);
    // Decision thresholds: smallest float32 strictly above each midpoint of two
    // adjacent levels, so (x >= thr[j]) <=> (x > midpoint) for float32 x and the
    // nearest level wins with ties going to the lower index.
    for (int j = 0; j < 15; ++j) {
      const double m = 0.5 * ((double)c.code[j] + (double)c.code[j + 1]);
      float f = (float)m;
      if ((double)f <= m) f = std::nextafter(f, INFINITY);
      c.thr[j] = f;
    }
    c.pad_ = 0.f;
  }
};

const Nf4Consts &consts() {
  static const Tables t;
  return t.c;
}

// The restore kernels carry the levels as literals; they must equal the derived table.
bool literals_match() {
  static const bool ok = [] {
    for (int j = 0; j < 16; ++j) {
      uint32_t b;
      std::memcpy(&b, &consts().code[j], 4);
      if (b != kNf4CodeBits[j]) return false;
    }
    return true;
  }();
  return ok;
}

// Per-tile buffer ranges stay below 2^31 bytes with these bounds.
constexpr int64_t kMaxDim = (int64_t)1 << 20;
constexpr int64_t kMaxTokens = (int64_t)1 << 24;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

int validate_weight(const qlora_nf4_weight *W) {
  if (!literals_match()) return QLORA_ERR_INTERNAL;
  if (!W || !W->codes || !W->smax) return QLORA_ERR_NULL;  // qscale NULL: absmax-only storage
  if (W->d_out < 1 || W->d_in < QLORA_BLOCK || W->d_in % QLORA_BLOCK != 0 || W->d_out % 16 != 0)
    return QLORA_ERR_SHAPE;
  if (W->d_out > kMaxDim || W->d_in > kMaxDim) return QLORA_ERR_SHAPE;
  // block indices are 32-bit in the kernels
  if (W->d_out * W->d_in / QLORA_BLOCK >= ((int64_t)1 << 32)) return QLORA_ERR_SHAPE;
  // absmax-only storage: the kernels address the float32 block scales as one buffer range
  if (!W->qscale && W->d_out * W->d_in / QLORA_BLOCK * 4 >= ((int64_t)1 << 31)) return QLORA_ERR_SHAPE;
  if (!aligned16(W->codes) || (W->qscale && !aligned16(W->qscale)) || !aligned16(W->smax)) return QLORA_ERR_ALIGN;
  return QLORA_OK;
}

int rank_pad(int r) { return r > 0 ? (int)ceil_div(r, 16) * 16 : 0; }

int lora_small_ksplit(int64_t T, int64_t K) {
  if (T > 64) return 1;
  int64_t ks = ceil_div(K, 32) / 8;
  return (int)std::max<int64_t>(1, std::min<int64_t>(ks, 64));
}

// Workspace regions (byte offsets). The counter region is fixed (kMaxCounters
// u32 at offset 0, independent of the shapes) so that a workspace reused across
// calls of different sizes always finds its counters zero: every kernel that
// counts arriving workgroups resets its counters before it exits, and the calls
// of one stream run one kernel at a time.
struct Layout {
  size_t sx, su32, u, v, bt, partial, total;
};

Layout layout(int64_t d_out, int64_t d_in, int64_t T, int r) {
  Layout L{};
  const int rp = rank_pad(r);
  const int64_t T16 = std::max<int64_t>(16, ceil_div(T, 16) * 16);
  size_t off = align256((size_t)kMaxCounters * sizeof(uint32_t));
  L.sx = off;
  off = align256(off + (size_t)T16 * rp * 2);
  L.su32 = off;
  off = align256(off + (size_t)4 * 16 * rp * 8);  // tagged float32 partials of u (4 K slices)
  L.u = off;
  off = align256(off + (size_t)T * r * 4);
  L.v = off;
  off = align256(off + (size_t)T * r * 4);
  L.bt = off;
  off = align256(off + (size_t)r * d_out * 2);
  size_t pf = 0;
  if (r > 0 && T < kWideMinTokens) {
    pf = std::max(pf, (size_t)ceil_div(T, 16) * lora_small_ksplit(T, std::max(d_in, d_out)) * 16 * rp);
    pf = std::max(pf, lora_grad_partial_floats(r, d_in, T));
    pf = std::max(pf, lora_grad_partial_floats(d_out, r, T));
  }
  if (r > 0 && T >= kWideMinTokens) {
    pf = std::max(pf, lora_tall_partial_floats(T, d_in, rp));
    pf = std::max(pf, lora_tall_partial_floats(T, d_out, rp));
    pf = std::max(pf, lora_wgrad_partial_floats(d_in, r, T));
    pf = std::max(pf, lora_wgrad_partial_floats(d_out, r, T));
  }
  // K-split tail tiles of the large-T contractions (forward over d_in, dX over d_out)
  pf = std::max(pf, gemm_partial_floats(gemm_plan(T, d_out, d_in / kBlock)));
  pf = std::max(pf, gemm_partial_floats(gemm_plan(T, d_in, ceil_div(d_out, kBlock))));
  L.partial = off;
  off = align256(off + pf * 4);
  L.total = off;
  return L;
}

template <typename T>
T *at(void *ws, size_t off) {
  return reinterpret_cast<T *>(static_cast<uint8_t *>(ws) + off);
}

int hip_status(hipError_t e) { return e == hipSuccess ? QLORA_OK : QLORA_ERR_HIP; }

}  // namespace

namespace qlora {

int current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return -1;
  return dev;
}

int device_cu_count(int dev) {
  static DeviceOnce once;
  static int cus[kMaxDevices];
  if (dev < 0 || dev >= kMaxDevices) return 256;
  (void)once.run(dev, [&] {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) n = 256;
    cus[dev] = n;
    return hipSuccess;
  });
  return cus[dev];
}

// Argument checks of a forward call that do not involve the workspace.
int validate_forward(const qlora_nf4_weight *W, const uint16_t *x, int64_t T, const uint16_t *A, const uint16_t *B,
                     int32_t r, uint16_t *h, float *u_out) {
  int s = validate_weight(W);
  if (s) return s;
  if (!x || !h) return QLORA_ERR_NULL;
  if (T < 1 || r < 0 || r > QLORA_MAX_RANK || r % 8 != 0) return QLORA_ERR_SHAPE;
  if (T > kMaxTokens) return QLORA_ERR_SHAPE;
  if (!A && !B) r = 0;
  if (r > 0 && (!A || !B)) return QLORA_ERR_NULL;
  if (!aligned16(x) || !aligned16(h) || (r > 0 && (!aligned16(A) || !aligned16(B))) ||
      (u_out && !aligned16(u_out)))
    return QLORA_ERR_ALIGN;
  return QLORA_OK;
}

// Workspace bytes one forward call touches (its counters, intermediates and
// partials; qlora_workspace_bytes also covers the backward at the same sizes).
size_t forward_workspace_need(int64_t d_out, int64_t d_in, int64_t T, int r) {
  const Layout L = layout(d_out, d_in, T, r);
  // the weight-streaming kernel uses the counters and the tagged exchange only
  if (gemv_supported(d_out, d_in, T)) return L.u;
  // the tiled path: counters, s*u, and the partials of u = x A^T and of the contraction's split tail
  size_t pf = gemm_partial_floats(gemm_plan(T, d_out, d_in / kBlock));
  if (r > 0)
    pf = std::max(pf, T >= kWideMinTokens ? lora_tall_partial_floats(T, d_in, rank_pad(r))
                                          : (size_t)ceil_div(T, 16) * lora_small_ksplit(T, d_in) * 16 * rank_pad(r));
  return L.partial + pf * 4;
}

// The forward's kernels on a checked workspace (r already 0 when A = B = NULL).
int enqueue_forward(const qlora_nf4_weight *W, const uint16_t *x, int64_t T, const uint16_t *A, const uint16_t *B,
                    int32_t r, float alpha, uint16_t *h, float *u_out, void *ws, hipStream_t stream) {
  const int64_t d_out = W->d_out, d_in = W->d_in;
  const Layout L = layout(d_out, d_in, T, r);
  const int rp = rank_pad(r);
  const float sc = r > 0 ? alpha / (float)r : 0.f;
  if (gemv_supported(d_out, d_in, T))
    return hip_status(launch_gemv_fwd(W->codes, W->qscale, W->smax, d_out, d_in, x, T, A, B, r, rp, sc, h, u_out,
                                      at<uint64_t>(ws, L.su32), at<uint32_t>(ws, (kMaxCounters - kSyncWords) * 4),
                                      stream));
  uint16_t *su = at<uint16_t>(ws, L.sx);
  float *partial = at<float>(ws, L.partial);
  hipError_t e = hipSuccess;
  if (r > 0) {
    if (T >= kWideMinTokens) {
      e = launch_lora_tall(x, A, T, d_in, r, rp, sc, u_out, su, partial, at<uint32_t>(ws, 0), stream);
    } else {
      const int ks = lora_small_ksplit(T, d_in);
      e = launch_lora_small(x, A, T, d_in, r, sc, u_out, su, rp, partial, at<uint32_t>(ws, 0), ks, stream);
    }
    if (e != hipSuccess) return QLORA_ERR_HIP;
  }
  e = launch_gemm_fwd(W->codes, W->qscale, W->smax, d_out, d_in, x, T, su, rp, B, r, h, partial,
                      at<uint32_t>(ws, 0), stream);
  return hip_status(e);
}

}  // namespace qlora

extern "C" {

void qlora_nf4_codebook(float out[16]) {
  if (out) std::memcpy(out, consts().code, 16 * sizeof(float));
}

void qlora_nf4_thresholds(float out[15]) {
  if (out) std::memcpy(out, consts().thr, 15 * sizeof(float));
}

const char *qlora_status_string(int status) {
  switch (status) {
    case QLORA_OK: return "ok";
    case QLORA_ERR_NULL: return "a required pointer is NULL";
    case QLORA_ERR_SHAPE: return "invalid shape (need d_in % 64 == 0, d_out % 16 == 0, T >= 1, 0 <= r <= 256, r % 8 == 0)";
    case QLORA_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case QLORA_ERR_WORKSPACE: return "workspace too small";
    case QLORA_ERR_DTYPE: return "unknown dtype";
    case QLORA_ERR_HIP: return "HIP launch failed";
    case QLORA_ERR_INTERNAL: return "internal: the kernels' NF4 levels differ from the derived table";
    case QLORA_ERR_MEMORY: return "a pointer is neither device memory nor pinned host memory";
    case QLORA_ERR_VALUE: return "a hyperparameter is out of range (or step < 1)";
    case QLORA_ERR_SCRATCH: return "qlora_forward_noalloc takes T <= 16 only (its static scratch array holds that path)";
    default: return "unknown status";
  }
}

int qlora_workspace_fallbacks(const void *ws, uint32_t *count, hipStream_t stream) {
  if (!ws || !count) return QLORA_ERR_NULL;
  const void *word = static_cast<const uint8_t *>(ws) + (kMaxCounters - 1) * sizeof(uint32_t);
  if (hipMemcpyAsync(count, word, sizeof(uint32_t), hipMemcpyDeviceToHost, stream) != hipSuccess) return QLORA_ERR_HIP;
  return hip_status(hipStreamSynchronize(stream));
}

int qlora_workspace_set_wait_limit(void *ws, uint32_t ticks, hipStream_t stream) {
  if (!ws) return QLORA_ERR_NULL;
  void *word = static_cast<uint8_t *>(ws) + (kMaxCounters - 2) * sizeof(uint32_t);
  if (hipMemsetD32Async(word, (int)ticks, 1, stream) != hipSuccess) return QLORA_ERR_HIP;
  return hip_status(hipStreamSynchronize(stream));
}

size_t qlora_storage_bytes(int64_t d_out, int64_t d_in) {
  if (d_out < 1 || d_in < 1) return 0;
  const int64_t n = d_out * d_in, nb = n / QLORA_BLOCK;
  return (size_t)(n / 2 + nb + 4 * ceil_div(nb, QLORA_GROUP));
}

size_t qlora_storage_bytes_absmax(int64_t d_out, int64_t d_in) {
  if (d_out < 1 || d_in < 1) return 0;
  const int64_t n = d_out * d_in;
  return (size_t)(n / 2 + 4 * (n / QLORA_BLOCK));
}

size_t qlora_workspace_bytes(int64_t d_out, int64_t d_in, int64_t T, int32_t r) {
  if (d_out < 1 || d_in < 1 || T < 1 || r < 0 || r > QLORA_MAX_RANK) return 0;
  return layout(d_out, d_in, T, r).total;
}

int qlora_quantize_many(const void *const *W, int w_dtype, const qlora_nf4_weight *out, int32_t count,
                        uint32_t *flags, hipStream_t stream) {
  if (count < 0) return QLORA_ERR_SHAPE;
  if (count > 0 && (!W || !out)) return QLORA_ERR_NULL;
  // every job is checked before anything is launched
  for (int32_t i = 0; i < count; ++i) {
    if (!W[i]) return QLORA_ERR_NULL;
    const int s = validate_weight(&out[i]);
    if (s) return s;
    if (w_dtype != QLORA_F32 && w_dtype != QLORA_BF16) return QLORA_ERR_DTYPE;
    if (!aligned16(W[i]) || (flags && (reinterpret_cast<uintptr_t>(flags) & 3u))) return QLORA_ERR_ALIGN;
  }
  if (w_dtype != QLORA_F32 && w_dtype != QLORA_BF16) return QLORA_ERR_DTYPE;
  for (int32_t i0 = 0; i0 < count; i0 += kQuantizeJobs) {
    QuantizeJobs jobs{};
    jobs.n = (int)std::min<int32_t>(kQuantizeJobs, count - i0);
    int64_t g = 0;
    for (int k = 0; k < jobs.n; ++k) {
      const qlora_nf4_weight &o = out[i0 + k];
      jobs.W[k] = W[i0 + k];
      jobs.codes[k] = o.codes;
      jobs.qscale[k] = o.qscale;
      jobs.smax[k] = o.smax;
      jobs.nblocks[k] = o.d_out * o.d_in / QLORA_BLOCK;
      jobs.gstart[k] = g;
      g += ceil_div(jobs.nblocks[k], kGroup);
    }
    jobs.gstart[jobs.n] = g;
    const int s = hip_status(launch_quantize(jobs, w_dtype == QLORA_BF16, flags, consts(), stream));
    if (s) return s;
  }
  return QLORA_OK;
}

int qlora_quantize(const void *W, int w_dtype, const qlora_nf4_weight *out, uint32_t *flags, hipStream_t stream) {
  if (!W) return QLORA_ERR_NULL;
  const int s = validate_weight(out);  // (out may be NULL)
  if (s) return s;
  return qlora_quantize_many(&W, w_dtype, out, 1, flags, stream);
}

int qlora_dequantize(const qlora_nf4_weight *W, int out_dtype, void *out, hipStream_t stream) {
  int s = validate_weight(W);
  if (s) return s;
  if (!out) return QLORA_ERR_NULL;
  if (out_dtype != QLORA_F32 && out_dtype != QLORA_BF16) return QLORA_ERR_DTYPE;
  if (!aligned16(out)) return QLORA_ERR_ALIGN;
  return hip_status(launch_dequantize(W->codes, W->qscale, W->smax, W->d_out, W->d_in, out_dtype == QLORA_BF16, out,
                                      consts(), stream));
}

int qlora_merge(const qlora_nf4_weight *W, const uint16_t *A, const uint16_t *B, int32_t r, float alpha,
                uint16_t *out, hipStream_t stream) {
  int s = validate_weight(W);
  if (s) return s;
  if (!out) return QLORA_ERR_NULL;
  if (r < 0 || r > QLORA_MAX_RANK || r % 8 != 0) return QLORA_ERR_SHAPE;
  if (!A && !B) r = 0;
  if (r > 0 && (!A || !B)) return QLORA_ERR_NULL;
  if (!aligned16(out) || (r > 0 && (!aligned16(A) || !aligned16(B)))) return QLORA_ERR_ALIGN;
  const float sc = r > 0 ? alpha / (float)r : 0.f;
  return hip_status(launch_merge(W->codes, W->qscale, W->smax, W->d_out, W->d_in, r > 0 ? A : nullptr,
                                 r > 0 ? B : nullptr, r, sc, out, stream));
}

// A device-accessible address for a pointer into device memory or pinned host
// memory (*host is set for the latter); pageable host memory is refused (its
// lookup error is cleared so that it does not surface from a later call).
static int device_address(void *p, void **out, bool *host) {
  hipPointerAttribute_t at;
  if (hipPointerGetAttributes(&at, p) != hipSuccess) {
    (void)hipGetLastError();
    return QLORA_ERR_MEMORY;
  }
  if (at.type == hipMemoryTypeDevice || at.type == hipMemoryTypeManaged || at.isManaged) {
    *out = p;
    *host = false;
    return QLORA_OK;
  }
  if (at.type == hipMemoryTypeHost) {
    void *d = nullptr;
    if (hipHostGetDevicePointer(&d, p, 0) != hipSuccess || !d) {
      (void)hipGetLastError();
      return QLORA_ERR_MEMORY;
    }
    *out = d;
    *host = true;
    return QLORA_OK;
  }
  return QLORA_ERR_MEMORY;
}

int qlora_adamw_step(const qlora_adamw_hparams *hp, int64_t step, int64_t n, const float *grad, float *master,
                     float *m, float *v, uint16_t *param, hipStream_t stream) {
  if (!hp || !grad || !master || !m || !v) return QLORA_ERR_NULL;
  if (n < 0) return QLORA_ERR_SHAPE;
  if (step < 1 || !(hp->lr >= 0.f) || !(hp->beta1 >= 0.f && hp->beta1 < 1.f) ||
      !(hp->beta2 >= 0.f && hp->beta2 < 1.f) || !(hp->eps > 0.f) || !(hp->weight_decay >= 0.f))
    return QLORA_ERR_VALUE;
  if (!aligned16(grad) || !aligned16(master) || !aligned16(m) || !aligned16(v) || (param && !aligned16(param)))
    return QLORA_ERR_ALIGN;
  if (n == 0) return QLORA_OK;
  void *dg = nullptr, *dm = nullptr, *dmm = nullptr, *dv = nullptr, *dp = nullptr;
  bool hg = false, hm = false, hmm = false, hv = false, hp_ = false;
  int s;
  if ((s = device_address(const_cast<float *>(grad), &dg, &hg)) || (s = device_address(master, &dm, &hm)) ||
      (s = device_address(m, &dmm, &hmm)) || (s = device_address(v, &dv, &hv)) ||
      (param && (s = device_address(param, &dp, &hp_))))
    return s;
  AdamWArgs a;
  a.lr = hp->lr;
  a.b1 = hp->beta1;
  a.b2 = hp->beta2;
  a.one_minus_b1 = 1.f - hp->beta1;
  a.one_minus_b2 = 1.f - hp->beta2;
  a.eps = hp->eps;
  a.decay = 1.f - hp->lr * hp->weight_decay;
  a.c1 = (float)(1.0 - std::pow((double)hp->beta1, (double)step));
  a.c2 = (float)(1.0 - std::pow((double)hp->beta2, (double)step));
  return hip_status(launch_adamw(static_cast<const float *>(dg), static_cast<float *>(dm), static_cast<float *>(dmm),
                                 static_cast<float *>(dv), static_cast<uint16_t *>(dp), n, a,
                                 hg || hm || hmm || hv || hp_, stream));
}

int qlora_forward(const qlora_nf4_weight *W, const uint16_t *x, int64_t T, const uint16_t *A, const uint16_t *B,
                  int32_t r, float alpha, uint16_t *h, float *u_out, void *ws, size_t ws_bytes,
                  hipStream_t stream) {
  int s = validate_forward(W, x, T, A, B, r, h, u_out);
  if (s) return s;
  if (!A && !B) r = 0;
  const Layout L = layout(W->d_out, W->d_in, T, r);
  if (ws_bytes < L.total) return QLORA_ERR_WORKSPACE;
  if (!ws) return QLORA_ERR_NULL;
  if (!aligned16(ws)) return QLORA_ERR_ALIGN;
  return enqueue_forward(W, x, T, A, B, r, alpha, h, u_out, ws, stream);
}

// qlora_forward_many's workspace: the counter region, then one tagged exchange
// buffer per job, sized for the largest rank (4 K slices x 16 tokens x r_pad
// tagged float32 partials of u).
constexpr size_t kUexJobBytes = (size_t)4 * 16 * QLORA_MAX_RANK * 8;
static size_t many_uex_offset() { return align256((size_t)kMaxCounters * sizeof(uint32_t)); }

size_t qlora_forward_many_workspace_bytes(int32_t count) {
  if (count < 1 || count > QLORA_MAX_FORWARD_JOBS) return 0;
  return many_uex_offset() + (size_t)count * kUexJobBytes;
}

int qlora_forward_many(const qlora_forward_job *jobs, int32_t count, void *ws, size_t ws_bytes,
                       hipStream_t stream) {
  if (!jobs) return QLORA_ERR_NULL;
  if (count < 1 || count > QLORA_MAX_FORWARD_JOBS) return QLORA_ERR_SHAPE;
  for (int i = 0; i < count; ++i) {
    const qlora_forward_job &j = jobs[i];
    const int s = validate_forward(j.W, j.x, j.T, j.A, j.B, j.r, j.h, j.u_out);
    if (s) return s;
    if (j.T > 16 || !gemv_supported(j.W->d_out, j.W->d_in, j.T)) return QLORA_ERR_SHAPE;
  }
  if (ws_bytes < qlora_forward_many_workspace_bytes(count)) return QLORA_ERR_WORKSPACE;
  if (!ws) return QLORA_ERR_NULL;
  if (!aligned16(ws)) return QLORA_ERR_ALIGN;
  GemvJob g[QLORA_MAX_FORWARD_JOBS];
  for (int i = 0; i < count; ++i) {
    const qlora_forward_job &j = jobs[i];
    const int r = j.A || j.B ? j.r : 0;
    g[i] = GemvJob{j.W->codes, j.W->qscale, j.W->smax, j.W->d_out, j.W->d_in, j.x, j.T, j.A, j.B, r, rank_pad(r),
                   r > 0 ? j.alpha / (float)r : 0.f, j.h, j.u_out,
                   at<uint64_t>(ws, many_uex_offset() + (size_t)i * kUexJobBytes)};
  }
  return hip_status(launch_gemv_fwd_many(g, count, at<uint32_t>(ws, (kMaxCounters - kSyncWords) * 4), stream));
}

int qlora_backward(const qlora_nf4_weight *W, const uint16_t *x, const uint16_t *dY, int64_t T, const uint16_t *A,
                   const uint16_t *B, int32_t r, float alpha, const float *u_saved, uint16_t *dX, float *dA,
                   float *dB, void *ws, size_t ws_bytes, hipStream_t stream) {
  int s = validate_weight(W);
  if (s) return s;
  if (!dY) return QLORA_ERR_NULL;
  if (T < 1 || r < 0 || r > QLORA_MAX_RANK || r % 8 != 0) return QLORA_ERR_SHAPE;
  if (T > kMaxTokens) return QLORA_ERR_SHAPE;
  if (!A && !B) r = 0;
  if (r > 0 && (!A || !B)) return QLORA_ERR_NULL;
  if (r == 0 && (dA || dB)) return QLORA_ERR_SHAPE;
  if (dA && !x) return QLORA_ERR_NULL;
  if (dB && !u_saved && !x) return QLORA_ERR_NULL;
  if (!aligned16(dY) || (x && !aligned16(x)) || (r > 0 && (!aligned16(A) || !aligned16(B))) ||
      (u_saved && !aligned16(u_saved)) || (dX && !aligned16(dX)) || (dA && !aligned16(dA)) ||
      (dB && !aligned16(dB)))
    return QLORA_ERR_ALIGN;
  const int64_t d_out = W->d_out, d_in = W->d_in;
  const Layout L = layout(d_out, d_in, T, r);
  if (ws_bytes < L.total) return QLORA_ERR_WORKSPACE;
  if (!ws) return QLORA_ERR_NULL;
  if (!aligned16(ws)) return QLORA_ERR_ALIGN;
  if (!dX && !dA && !dB) return QLORA_OK;

  const int rp = rank_pad(r);
  const float sc = r > 0 ? alpha / (float)r : 0.f;
  uint16_t *sv = at<uint16_t>(ws, L.sx);
  float *v = at<float>(ws, L.v);
  float *partial = at<float>(ws, L.partial);
  uint32_t *cnt_small = at<uint32_t>(ws, 0);
  hipError_t e = hipSuccess;
  const float *u = u_saved;
  if (r > 0) {
    uint16_t *bt = at<uint16_t>(ws, L.bt);
    e = launch_transpose_bf16(B, d_out, r, bt, stream);
    if (e != hipSuccess) return QLORA_ERR_HIP;
    if (T >= kWideMinTokens)
      e = launch_lora_tall(dY, bt, T, d_out, r, rp, sc, v, sv, partial, cnt_small, stream);
    else
      e = launch_lora_small(dY, bt, T, d_out, r, sc, v, sv, rp, partial, cnt_small, lora_small_ksplit(T, d_out),
                            stream);
    if (e != hipSuccess) return QLORA_ERR_HIP;
  }
  if (dX) {
    e = launch_gemm_dx(W->codes, W->qscale, W->smax, d_out, d_in, dY, T, sv, rp, A, r, dX, partial,
                       at<uint32_t>(ws, 0), stream);
    if (e != hipSuccess) return QLORA_ERR_HIP;
  }
  const bool wide = T >= kWideMinTokens;
  uint32_t *fallbacks = at<uint32_t>(ws, (kMaxCounters - 1) * 4);
  if (dA) {
    if (wide)
      e = launch_lora_wgrad(x, v, T, d_in, r, true, sc, dA, partial, at<uint32_t>(ws, 0), fallbacks, stream);
    else
      e = launch_lora_grad(v, true, r, x, false, d_in, T, sc, dA, partial, at<uint32_t>(ws, 0),
                           lora_grad_ksplit(r, d_in, T), stream);
    if (e != hipSuccess) return QLORA_ERR_HIP;
  }
  if (dB) {
    if (!u) {
      float *uw = at<float>(ws, L.u);
      if (wide)
        e = launch_lora_tall(x, A, T, d_in, r, rp, 1.f, uw, nullptr, partial, cnt_small, stream);
      else
        e = launch_lora_small(x, A, T, d_in, r, 1.f, uw, nullptr, rp, partial, cnt_small,
                              lora_small_ksplit(T, d_in), stream);
      if (e != hipSuccess) return QLORA_ERR_HIP;
      u = uw;
    }
    if (wide)
      e = launch_lora_wgrad(dY, u, T, d_out, r, false, sc, dB, partial, at<uint32_t>(ws, 0), fallbacks, stream);
    else
      e = launch_lora_grad(dY, false, d_out, u, true, r, T, sc, dB, partial, at<uint32_t>(ws, 0),
                           lora_grad_ksplit(d_out, r, T), stream);
    if (e != hipSuccess) return QLORA_ERR_HIP;
  }
  return QLORA_OK;
}

}  // extern "C"
