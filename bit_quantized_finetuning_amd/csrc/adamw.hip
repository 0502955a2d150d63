// AdamW step for the adapter parameters with the optimizer state kept in host
// memory ("paged" state).
//
// First page ("QLoRA는 어떻게 65B 모델을 GPU 한 장에 올렸나"), the paged-optimizer
// entry of its memory accounting: the adapters' Adam state (m, v) is moved out
// to CPU pinned memory, and the update runs alongside the backward on another
// stream so that the transfers hide behind it. Here the state (m, v and a
// float32 master copy of the parameters) may live in pinned host memory: the
// kernel reads and writes it in place over the host link, and writes the bf16
// parameters the layer computes with to device memory. Nothing is copied in a
// separate step and the library allocates nothing.
//
// AdamW with decoupled weight decay (Loshchilov and Hutter, "Decoupled Weight
// Decay Regularization"), per element:
//     p <- p (1 - lr wd)
//     m <- b1 m + (1 - b1) g
//     v <- b2 v + (1 - b2) g^2
//     p <- p - lr (m / c1) / (sqrt(v / c2) + eps),  c1 = 1 - b1^t, c2 = 1 - b2^t
// in float32 (c1 and c2 are formed on the host in float64 and passed rounded).
// The kernel is bound by the host link when the state is in host memory (8
// bytes read and 8 written per element for m and v there, 16 and 12 with the
// master copy too) and by HBM otherwise.
//
// Grid: with all operands in device memory, enough workgroups to fill the chip
// (HBM bound). With state in host memory the step is link bound and meant to
// run beside the backward's kernels on another stream; there a few workgroups
// already keep enough requests in flight to saturate the link (32 x 256 lanes
// x 16 bytes per state stream per round trip), while every extra one occupies a
// CU slot, stalled on host latency, that the concurrent GEMM tiles wait for. On
// the 13B projections at 4096 tokens the cost of the paged update to the step
// fell from about 19 % with up to 2048 workgroups to about 12 % with 32 (16 and
// 8 were no better; more loads in flight per lane did not help either).
#include "kernels.h"

namespace qlora {

__device__ __forceinline__ void adamw_one(float &p, float &m, float &v, float g, const AdamWArgs &a) {
  p = p * a.decay;
  m = a.b1 * m + a.one_minus_b1 * g;
  v = a.b2 * v + a.one_minus_b2 * (g * g);
  const float mh = m / a.c1;
  const float vh = v / a.c2;
  p = p - a.lr * (mh / (sqrtf(vh) + a.eps));
}

__global__ __launch_bounds__(256) void k_adamw(const float *__restrict__ grad, float *__restrict__ master,
                                               float *__restrict__ m, float *__restrict__ v,
                                               uint16_t *__restrict__ param, int64_t n, AdamWArgs a) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t n4 = n / 4;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
    const f32x4 g = reinterpret_cast<const f32x4 *>(grad)[i];
    f32x4 p = reinterpret_cast<f32x4 *>(master)[i];
    f32x4 mm = reinterpret_cast<f32x4 *>(m)[i];
    f32x4 vv = reinterpret_cast<f32x4 *>(v)[i];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float pe = p[e], me = mm[e], ve = vv[e];
      adamw_one(pe, me, ve, g[e], a);
      p[e] = pe;
      mm[e] = me;
      vv[e] = ve;
    }
    reinterpret_cast<f32x4 *>(master)[i] = p;
    reinterpret_cast<f32x4 *>(m)[i] = mm;
    reinterpret_cast<f32x4 *>(v)[i] = vv;
    if (param) reinterpret_cast<u32x2 *>(param)[i] = u32x2{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
  }
  // the last n % 4 elements
  const int64_t i = 4 * n4 + (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) {
    float p = master[i], mm = m[i], vv = v[i];
    adamw_one(p, mm, vv, grad[i], a);
    master[i] = p;
    m[i] = mm;
    v[i] = vv;
    if (param) param[i] = (uint16_t)(pack_bf16x2(p, 0.f) & 0xffffu);
  }
}

constexpr int64_t kAdamWBlocksDevice = 2048;
constexpr int64_t kAdamWBlocksHost = 32;

hipError_t launch_adamw(const float *grad, float *master, float *m, float *v, uint16_t *param, int64_t n,
                        const AdamWArgs &a, bool host_state, hipStream_t st) {
  const int64_t cap = host_state ? kAdamWBlocksHost : kAdamWBlocksDevice;
  int64_t blocks = (n / 4 + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > cap) blocks = cap;
  k_adamw<<<dim3((unsigned)blocks), dim3(256), 0, st>>>(grad, master, m, v, param, n, a);
  return hipGetLastError();
}

}  // namespace qlora
