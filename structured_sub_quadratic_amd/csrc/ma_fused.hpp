// Fused single-launch path for T = 1: [tile means ->] stage 1 -> stage 2 in
// one cooperative launch whose phases are separated by grid-wide barriers.
// Every workgroup walks the items of a phase with stride gridDim.x; the
// exchange (c, u, H_R) written in one phase is read in the next without a
// kernel boundary, so it is still warm in L2 / Infinity Cache, and the tail of
// one phase overlaps the start of the next only at the barrier.
//
// Source: MonarchAttention (scime summary "Key results": a fully-fused kernel
// for short sequences) -- the same idea, here for any size on one device.
#pragma once

#include <hip/hip_cooperative_groups.h>

#include "ma_aux_kernels.hpp"
#include "ma_stage_kernels.hpp"

namespace ma {

template <size_t A, size_t B> constexpr size_t cmax() { return A > B ? A : B; }

template <typename T, int D, int NQ1, int KTB, int NQ2, bool PRECISE, bool QSPLIT, bool PAD = false>
__global__ __launch_bounds__(THREADS) void fused_t1_kernel(QbarParams pq, Stage1Params p1, Stage2Params p2) {
  typedef Stage1Item<T, D, NQ1, KTB, true, PRECISE, QSPLIT, PAD> S1;
  typedef Stage2Item<T, D, NQ2, true, PRECISE, PAD> S2;
  typedef QbarItem<T, D> QB;
  constexpr size_t SZ = cmax<cmax<sizeof(typename S1::Smem), sizeof(typename S2::Smem)>(),
                             sizeof(typename QB::Smem)>();
  __shared__ __attribute__((aligned(16))) char buf[SZ];
  cooperative_groups::grid_group grid = cooperative_groups::this_grid();

  if (p1.c1 > 1 || PAD) {
    const int n0 = QB::items(pq);
    for (int it = blockIdx.x; it < n0; it += gridDim.x)
      QB::run(pq, *reinterpret_cast<typename QB::Smem*>(buf), it);
    grid.sync();
  }
  const int n1 = S1::items(p1);
  for (int it = blockIdx.x; it < n1; it += gridDim.x)
    S1::run(p1, *reinterpret_cast<typename S1::Smem*>(buf), it);
  grid.sync();
  const int n2 = S2::items(p2);
  for (int it = blockIdx.x; it < n2; it += gridDim.x)
    S2::run(p2, *reinterpret_cast<typename S2::Smem*>(buf), it);
}

}  // namespace ma
