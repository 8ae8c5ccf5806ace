// Kernels and launch sequence for float inputs with head_dim 128.
#include "ma_backward.hpp"

namespace ma {

ma_status run_f32_128(const Plan& pl, const Bufs& b, hipStream_t st, void* const* events, int n_events) {
  return run_t<float, 128, true>(pl, b, st, events, n_events);
}

ma_status run_bwd_f32_128(const Plan& pl, const BwdBufs& b, hipStream_t st) {
  return run_bwd_t<float, 128, true>(pl, b, st);
}

}  // namespace ma
