// Minimal persistent thread pool for the offline (host) preparation steps.
// One pool per process, sized to the CPUs in the affinity mask.
#pragma once

#include <atomic>
#include <condition_variable>
#include <cstdint>
#include <functional>
#include <mutex>
#include <thread>
#include <vector>

namespace svdq {

class ThreadPool {
 public:
  static ThreadPool &get();
  int size() const { return nthreads_; }
  // Runs body(begin, end) over [0, n) split into chunks of `grain`, on all
  // threads including the caller; returns when every chunk is done.
  void run(int64_t n, int64_t grain, const std::function<void(int64_t, int64_t)> &body);
  ~ThreadPool();

 private:
  explicit ThreadPool(int n);
  void worker_loop();
  void drain();
  int nthreads_;
  std::vector<std::thread> workers_;
  std::mutex mu_;
  std::mutex run_mu_;  // one run() at a time; bodies must not call run()
  std::condition_variable cv_job_, cv_done_;
  const std::function<void(int64_t, int64_t)> *body_ = nullptr;
  int64_t n_ = 0, grain_ = 1;
  std::atomic<int64_t> next_{0};
  int finished_ = 0;
  uint64_t epoch_ = 0;
  bool stop_ = false;
};

inline void parallel_for(int64_t n, int64_t grain,
                         const std::function<void(int64_t, int64_t)> &body) {
  ThreadPool::get().run(n, grain, body);
}

}  // namespace svdq
