// AdamW step run by the host CPU: the page's own placement of the paged
// optimizer's update.
//
// First page ("QLoRA는 어떻게 65B 모델을 GPU 한 장에 올렸나"), the paged-optimizer
// entry of section "메모리 회계": the adapters' Adam state stays in pinned CPU
// memory and the CPU runs the optimizer step while the GPU continues with the
// backward. Here the caller copies the float32 gradients to host memory (a DMA
// copy, no compute unit involved), this function updates the float32 master
// copy, m and v in place and writes the bf16 parameters to a host buffer, and
// the caller copies those back to the device. The GPU's compute units never
// see the update.
//
// Per element, in float32, the same operations in the same order as the GPU
// kernel (adamw.hip): decoupled weight decay, then the moments, then the
// bias-corrected step; the bias corrections are formed in float64 and rounded
// to float32. Results agree with the kernel's to rounding (the kernel's
// compiler may contract a multiply-add into one fused operation; here, on a
// baseline x86-64 target, nothing is fused).
//
// The elements are split into contiguous chunks over a small pool of worker
// threads that lives for the process; a call waits for all of its chunks.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <condition_variable>
#include <cstring>
#include <functional>
#include <mutex>
#include <thread>
#include <vector>

#include "qlora.h"

namespace {

struct Args {
  float lr, b1, b2, one_minus_b1, one_minus_b2, eps, decay, c1, c2;
};

// bf16 of a float32 by round-to-nearest-even (a NaN stays a quiet NaN).
inline uint16_t to_bf16(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return (uint16_t)((u >> 16) | 0x0040u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

void update_range(const Args &a, int64_t lo, int64_t hi, const float *grad, float *master, float *m, float *v,
                  uint16_t *param) {
  for (int64_t i = lo; i < hi; ++i) {
    float p = master[i] * a.decay;
    const float g = grad[i];
    const float mm = a.b1 * m[i] + a.one_minus_b1 * g;
    const float vv = a.b2 * v[i] + a.one_minus_b2 * (g * g);
    const float mh = mm / a.c1;
    const float vh = vv / a.c2;
    p = p - a.lr * (mh / (std::sqrt(vh) + a.eps));
    master[i] = p;
    m[i] = mm;
    v[i] = vv;
    if (param) param[i] = to_bf16(p);
  }
}

// A fixed pool of worker threads; run() hands out `tasks` indices and returns
// once every task has finished. Calls from several host threads take turns.
class Pool {
 public:
  explicit Pool(int n) {
    for (int i = 0; i < n; ++i) workers_.emplace_back([this] { loop(); });
  }
  ~Pool() {
    {
      std::lock_guard<std::mutex> g(mu_);
      stop_ = true;
    }
    cv_.notify_all();
    for (auto &t : workers_) t.join();
  }
  int size() const { return (int)workers_.size(); }
  void run(int tasks, const std::function<void(int)> &fn) {
    std::lock_guard<std::mutex> call(call_mu_);
    {
      std::lock_guard<std::mutex> g(mu_);
      fn_ = &fn;
      next_ = 0;
      tasks_ = tasks;
      left_ = tasks;
      ++generation_;
    }
    cv_.notify_all();
    std::unique_lock<std::mutex> g(mu_);
    done_cv_.wait(g, [this] { return left_ == 0; });
    fn_ = nullptr;
  }

 private:
  void loop() {
    uint64_t seen = 0;
    for (;;) {
      std::unique_lock<std::mutex> g(mu_);
      cv_.wait(g, [&] { return stop_ || (generation_ != seen && next_ < tasks_); });
      if (stop_) return;
      seen = generation_;
      while (next_ < tasks_) {
        const int t = next_++;
        const std::function<void(int)> *fn = fn_;
        g.unlock();
        (*fn)(t);
        g.lock();
        if (--left_ == 0) done_cv_.notify_all();
      }
    }
  }
  std::vector<std::thread> workers_;
  std::mutex mu_, call_mu_;
  std::condition_variable cv_, done_cv_;
  const std::function<void(int)> *fn_ = nullptr;
  int next_ = 0, tasks_ = 0, left_ = 0;
  uint64_t generation_ = 0;
  bool stop_ = false;
};

Pool &pool() {
  static Pool p(std::max(1u, std::min(16u, std::thread::hardware_concurrency())));
  return p;
}

}  // namespace

extern "C" int qlora_adamw_step_host(const qlora_adamw_hparams *hp, int64_t step, int64_t n, const float *grad,
                                     float *master, float *m, float *v, uint16_t *param, int32_t threads) {
  if (!hp || !grad || !master || !m || !v) return QLORA_ERR_NULL;
  if (n < 0) return QLORA_ERR_SHAPE;
  if (step < 1 || !(hp->lr >= 0.f) || !(hp->beta1 >= 0.f && hp->beta1 < 1.f) ||
      !(hp->beta2 >= 0.f && hp->beta2 < 1.f) || !(hp->eps > 0.f) || !(hp->weight_decay >= 0.f))
    return QLORA_ERR_VALUE;
  if (n == 0) return QLORA_OK;
  Args a;
  a.lr = hp->lr;
  a.b1 = hp->beta1;
  a.b2 = hp->beta2;
  a.one_minus_b1 = 1.f - hp->beta1;
  a.one_minus_b2 = 1.f - hp->beta2;
  a.eps = hp->eps;
  a.decay = 1.f - hp->lr * hp->weight_decay;
  a.c1 = (float)(1.0 - std::pow((double)hp->beta1, (double)step));
  a.c2 = (float)(1.0 - std::pow((double)hp->beta2, (double)step));
  // chunks of at least 64 Ki elements, at most one per worker (or `threads` if smaller)
  int workers = pool().size();
  if (threads > 0) workers = std::min(workers, (int)threads);
  const int64_t chunk_min = 1 << 16;
  const int tasks = (int)std::max<int64_t>(1, std::min<int64_t>(workers, (n + chunk_min - 1) / chunk_min));
  if (tasks == 1) {
    update_range(a, 0, n, grad, master, m, v, param);
    return QLORA_OK;
  }
  const std::function<void(int)> fn = [&](int t) {
    const int64_t lo = n * t / tasks, hi = n * (t + 1) / tasks;
    update_range(a, lo, hi, grad, master, m, v, param);
  };
  pool().run(tasks, fn);
  return QLORA_OK;
}
