// Kernels and launch sequence for bf16 inputs with head_dim 128, precise aggregate path.
#include "ma_launch.hpp"

namespace ma {

ma_status run_bf16_128_precise(const Plan& pl, const Bufs& b, hipStream_t st, void* const* events,
                              int n_events) {
  return run_t<bf16, 128, true>(pl, b, st, events, n_events);
}

}  // namespace ma
