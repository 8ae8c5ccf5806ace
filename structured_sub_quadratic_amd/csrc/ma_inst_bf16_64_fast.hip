// Kernels and launch sequence for bf16 inputs with head_dim 64, fast aggregate path.
#include "ma_launch.hpp"

namespace ma {

ma_status run_bf16_64_fast(const Plan& pl, const Bufs& b, hipStream_t st, void* const* events,
                              int n_events) {
  return run_t<bf16, 64, false>(pl, b, st, events, n_events);
}

}  // namespace ma
