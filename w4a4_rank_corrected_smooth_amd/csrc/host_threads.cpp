#include "host_threads.h"

#include <sched.h>

namespace svdq {

static int cpus_in_affinity_mask() {
  cpu_set_t set;
  CPU_ZERO(&set);
  if (sched_getaffinity(0, sizeof(set), &set) == 0) {
    int c = CPU_COUNT(&set);
    if (c > 0) return c;
  }
  unsigned h = std::thread::hardware_concurrency();
  return h ? static_cast<int>(h) : 1;
}

ThreadPool &ThreadPool::get() {
  static ThreadPool pool(cpus_in_affinity_mask());
  return pool;
}

ThreadPool::ThreadPool(int n) : nthreads_(n < 1 ? 1 : n) {
  for (int i = 1; i < nthreads_; ++i) workers_.emplace_back([this] { worker_loop(); });
}

ThreadPool::~ThreadPool() {
  {
    std::lock_guard<std::mutex> lk(mu_);
    stop_ = true;
  }
  cv_job_.notify_all();
  for (auto &t : workers_) t.join();
}

void ThreadPool::drain() {
  for (;;) {
    int64_t b = next_.fetch_add(grain_);
    if (b >= n_) break;
    int64_t e = b + grain_ < n_ ? b + grain_ : n_;
    (*body_)(b, e);
  }
}

void ThreadPool::worker_loop() {
  // Every worker takes part in every epoch exactly once, and run() waits for
  // all of them, so no worker can wander into the next epoch's state.
  uint64_t seen = 0;
  for (;;) {
    {
      std::unique_lock<std::mutex> lk(mu_);
      cv_job_.wait(lk, [&] { return stop_ || epoch_ != seen; });
      if (stop_) return;
      seen = epoch_;
    }
    drain();
    {
      std::lock_guard<std::mutex> lk(mu_);
      if (++finished_ == nthreads_ - 1) cv_done_.notify_all();
    }
  }
}

void ThreadPool::run(int64_t n, int64_t grain,
                     const std::function<void(int64_t, int64_t)> &body) {
  if (n <= 0) return;
  if (grain < 1) grain = 1;
  if (nthreads_ == 1 || n <= grain) {
    body(0, n);
    return;
  }
  std::lock_guard<std::mutex> one_run(run_mu_);
  std::unique_lock<std::mutex> lk(mu_);
  body_ = &body;
  n_ = n;
  grain_ = grain;
  next_.store(0);
  finished_ = 0;
  ++epoch_;
  lk.unlock();
  cv_job_.notify_all();
  drain();
  lk.lock();
  cv_done_.wait(lk, [&] { return finished_ == nthreads_ - 1; });
  body_ = nullptr;
}

}  // namespace svdq
