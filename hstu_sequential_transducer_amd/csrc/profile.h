// profile.h -- RAII bracket that records a HIP event pair around the kernels
// launched in its scope when hstu_profile_enable(1) is in effect.
#pragma once
#include <hip/hip_runtime.h>

class ProfScope {
  public:
    ProfScope(const char *name, hipStream_t st);
    ~ProfScope();
    ProfScope(const ProfScope &) = delete;
    ProfScope &operator=(const ProfScope &) = delete;

  private:
    const char *name_;
    hipStream_t st_;
    void *a_ = nullptr;
};
