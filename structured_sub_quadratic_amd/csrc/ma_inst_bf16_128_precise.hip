// Kernels and launch sequence for bf16 inputs with head_dim 128, precise aggregate path.
#include "ma_backward.hpp"

namespace ma {

ma_status run_bf16_128_precise(const Plan& pl, const Bufs& b, hipStream_t st, void* const* events,
                              int n_events) {
  return run_t<bf16, 128, true>(pl, b, st, events, n_events);
}

ma_status run_bwd_steps_bf16_128(const Plan& pl, const BwdBufs& b, hipStream_t st) {
  return run_bwd_steps_t<bf16, 128, true>(pl, b, st);
}

}  // namespace ma
