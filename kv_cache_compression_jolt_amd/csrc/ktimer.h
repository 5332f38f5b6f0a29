// Launch timing of selected kernels (a measurement hook behind
// jolt_kernel_timer / jolt_kernel_time): while a kernel's timer is on, every
// launch site of that kernel records a HIP event on its stream before and
// after the launch.  With no timer on, a KTimeScope costs one relaxed atomic load.
#pragma once
#include <hip/hip_runtime.h>

#include <stdint.h>

namespace jolt {

struct KTimer;
KTimer *ktimer_find(const char *kernel);           // nullptr unless the kernel's timer is on
void ktimer_record(KTimer *t, hipStream_t s, bool start);
hipError_t ktimer_enable(const char *kernel, bool on);
hipError_t ktimer_read(const char *kernel, double *total_ms, int64_t *launches);

class KTimeScope {
  public:
    KTimeScope(const char *kernel, hipStream_t s) : s_(s), t_(ktimer_find(kernel)) {
        if (t_) ktimer_record(t_, s_, true);
    }
    ~KTimeScope() {
        if (t_) ktimer_record(t_, s_, false);
    }
    KTimeScope(const KTimeScope &) = delete;
    KTimeScope &operator=(const KTimeScope &) = delete;

  private:
    hipStream_t s_;
    KTimer *t_;
};

}  // namespace jolt
