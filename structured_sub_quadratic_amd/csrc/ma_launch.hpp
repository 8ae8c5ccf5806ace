// Launch sequence of one element type and head dimension, included by the
// per-type translation units (ma_inst_*.hip).
#pragma once

#include <algorithm>
#include <type_traits>

#include <hip/hip_ext.h>

#include "ma_plan.hpp"
#include "ma_aux_kernels.hpp"
#include "ma_stage_kernels.hpp"
#include "ma_fused.hpp"
#include "ma_async.hpp"

namespace ma {

inline unsigned grid1(size_t n) { return (unsigned)n; }

// Events that take the start and end time stamps of the launch in progress
// (set by the timed entry point around each launch, null otherwise).
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
inline LaunchEvents& launch_events() {
  static thread_local LaunchEvents ev;
  return ev;
}

// Every kernel launch of the forward goes through here: with launch events
// set, the kernel's own start and end are recorded with its dispatch
// (hipExtLaunchKernel), so nothing is queued between the launches.
template <class F, class... A>
inline void ma_launch(F kernel, dim3 grid, dim3 block, hipStream_t st, A... args) {
  const LaunchEvents& ev = launch_events();
  if (ev.start) hipExtLaunchKernelGGL(kernel, grid, block, 0, st, ev.start, ev.stop, 0, args...);
  else hipLaunchKernelGGL(kernel, grid, block, 0, st, args...);
}

// Workgroups of a persistent launch: two per compute unit of the current
// device (the persistent kernels are built for two resident workgroups).
inline size_t persistent_slots() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    cus = 256;
  return (size_t)2 * cus;
}

template <typename T> constexpr bool is_f32() { return std::is_same<T, float>::value; }


// Waves per workgroup of the direct-to-LDS kernels: 8 (128 query rows) unless
// 4 (64 rows) pads fewer rows.
inline int async_waves(int rows) {
  const int pad4 = (rows + 63) / 64 * 64 - rows, pad8 = (rows + 127) / 128 * 128 - rows;
  return pad8 <= pad4 ? 8 : 4;
}

// Stage 2: at head_dim 128 the 4-wave kernel holds one wave a SIMD (it
// needs more than 256 registers), so 8 waves win whenever there are more
// than 64 query rows, even with up to a quarter of them padding.
template <int D> inline int stage2_waves(int rows) {
  if (rows <= 64) return 4;
  return D == 128 ? 8 : async_waves(rows);
}

// Stage 2 of bf16 at head_dim 64 with 8 waves (b2 > 64, one row tile) takes
// a column of 65 to 128 keys as one chunk of 128 (fewer chunk switches); the
// staged and the fused copied-tile launches chunk alike, so they give the
// same result.
inline bool one_chunk2(const Plan& pl) {
  return pl.b2 > 64 && pl.c1 == 1 && pl.b1 * pl.c2 > KT && pl.b1 * pl.c2 <= 2 * KT && !pl.causal &&
         !pl.padded;
}

template <class K, class P>
void launch_persistent(K kernel, int threads, size_t items, const P& p, hipStream_t st) {
  const size_t g = resident_slots(kernel, threads, items);
  ma_launch(kernel, dim3(grid1(g)), dim3(threads), st, p);
}

// Query sub-tiles of 16 per wave: the choice (1 or 2) that pads the fewest
// query rows per workgroup group, preferring 2 (more MFMAs per LDS operand).
inline int pick_nq(int rows) {
  const int pad1 = (rows + 63) / 64 * 64 - rows, pad2 = (rows + 127) / 128 * 128 - rows;
  return pad2 <= pad1 ? 2 : 1;
}
template <typename T, int D> int stage1_nq(int slots) {
  if (D == 128 || is_f32<T>()) return 1;
  return pick_nq(slots);
}
template <typename T, int D> int stage2_nq(int rows) {
  if (is_f32<T>() && D == 128) return 1;     // two sub-tiles would spill
  return pick_nq(rows);
}

// Cooperative launch of a fused kernel: as many workgroups as can be resident
// at once (the grid-wide barriers need them all), at most one per item.
template <class K>
hipError_t launch_cooperative(K kernel, size_t items, void** args, hipStream_t st, int threads = THREADS) {
  int per_cu = 0, dev = 0, cus = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0);
  if (e != hipSuccess) return e;
  if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
  if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
  if (per_cu < 1 || cus < 1) return hipErrorInvalidConfiguration;
  const size_t g = std::max<size_t>(1, std::min<size_t>(items, (size_t)per_cu * cus));
  const LaunchEvents& ev = launch_events();
  if (ev.start && (e = hipEventRecord(ev.start, st)) != hipSuccess) return e;
  e = hipLaunchCooperativeKernel(reinterpret_cast<const void*>(kernel), dim3(grid1(g)), dim3(threads), args, 0,
                                 st);
  if (e == hipSuccess && ev.stop) e = hipEventRecord(ev.stop, st);
  return e;
}

template <typename T, int D, bool PRECISE>
hipError_t launch_one(const Plan& pl, const Bufs& b, LaunchKind kind, int step, hipStream_t st) {
  char* ws = b.ws;
  void* cx = ws + pl.off_cx;
  void* ux = ws + pl.off_ux;
  float* h2 = reinterpret_cast<float*>(ws + pl.off_h2);
  float* lser = reinterpret_cast<float*>(ws + pl.off_lser);
  float* lse2 = reinterpret_cast<float*>(ws + pl.off_lse2);
  float* qtil = pl.need_qtil ? reinterpret_cast<float*>(ws + pl.off_qtil) : nullptr;
  float* qbar = pl.need_qbar ? reinterpret_cast<float*>(ws + pl.off_qbar) : nullptr;
  void* qbar_lp = pl.need_qbar_lp ? ws + pl.off_qbar_lp : nullptr;
  const int S = (int)pl.S, N = (int)pl.N;
  switch (kind) {
    case L_FUSED: {
      if constexpr (!is_f32<T>()) {
        if (pl.c1 == 1 && !pl.padded && pl.b2 <= 128) {
          // copied-tile stages in one cooperative launch; both phases use
          // the stage-1 wave count
          const int nqs = pl.b2, ktb = pl.b2 <= 64 ? 64 : 128;
          const int nw = D == 64 ? async_waves(nqs) : 4, qg = nw * 16;
          Stage1Params p1{b.q, b.k, b.v, qtil, qbar, cx, ux, h2, lser, pl.map,
                          S, N, pl.b1, pl.b2, pl.c1, pl.c2, pl.sw, pl.rt, nqs, (nqs + qg - 1) / qg,
                          pl.sc2, 1, pl.xlo};
          p1.heads = pl.heads;
          p1.group = pl.group;
          // (stage 2 at head_dim 128 on the fast path: 32 rows a wave)
          const int qg2 = D == 128 && !PRECISE ? 2 * qg : qg;
          Stage2Params p2{b.q, b.y, cx, ux, h2, lse2, b.lse, pl.map,
                          S, N, pl.b1, pl.b2, pl.c1, pl.c2, pl.rt, pl.b1 * pl.c2, (pl.rt + qg2 - 1) / qg2,
                          pl.sc2, pl.xlo, pl.causal};
          const size_t items = std::max<size_t>((size_t)S * pl.b1 * p1.nqg, (size_t)S * pl.b2 * p2.nqg);
          void* args[] = {&p1, &p2};
          hipError_t e = hipSuccess;
          // with one row tile the query slots are the b2 positions of a
          // block, so head_dim 64 takes 4 waves exactly when the block fits
          // one 64-key tile, 8 waves otherwise
#define MA_FA(NW, KTB) e = launch_cooperative(fused_async_kernel<D, NW, KTB, PRECISE>, items, args, st, NW * WAVE)
          if constexpr (D == 64) {
            if (ktb == 64) MA_FA(4, 64);
            else if (one_chunk2(pl)) e = launch_cooperative(fused_async_kernel<D, 8, 128, PRECISE, 2 * KT>, items, args, st, 8 * WAVE);
            else MA_FA(8, 128);
          } else {
            if (ktb == 64) MA_FA(4, 64); else MA_FA(4, 128);
          }
#undef MA_FA
          if (e != hipSuccess) return e;
          break;
        }
      }
      // the bf16 tile means too (a backward that reuses this state reads them)
      QbarParams pq{b.q, qbar, pl.map, S, N, pl.b2, pl.c1, pl.rt, qbar_lp};
      const int nqs = pl.c1 * pl.b2;
      const int nq1 = stage1_nq<T, D>(nqs), qg1 = WAVES * nq1 * 16;
      Stage1Params p1{b.q, b.k, b.v, qtil, qbar, cx, ux, h2, lser, pl.map,
                      S, N, pl.b1, pl.b2, pl.c1, pl.c2, pl.sw, pl.rt, nqs, (nqs + qg1 - 1) / qg1,
                      pl.sc2, 1, pl.xlo};
      p1.heads = pl.heads;
      p1.group = pl.group;
      const int nq2 = stage2_nq<T, D>(pl.rt), qg2 = WAVES * nq2 * 16;
      Stage2Params p2{b.q, b.y, cx, ux, h2, lse2, b.lse, pl.map,
                      S, N, pl.b1, pl.b2, pl.c1, pl.c2, pl.rt, pl.b1 * pl.c2, (pl.rt + qg2 - 1) / qg2,
                      pl.sc2, pl.xlo, pl.causal};
      const size_t items = std::max<size_t>(std::max<size_t>((size_t)S * pl.c1 * pl.b2,
                                                             (size_t)S * pl.b1 * p1.nqg),
                                            (size_t)S * pl.b2 * pl.c1 * p2.nqg);
      void* args[] = {&pq, &p1, &p2};
      const bool ktb64 = pl.b2 <= 64 || (is_f32<T>() && D == 128);
      const bool qsplit = PRECISE && is_bf16<T>() && (pl.c1 > 1 || pl.padded);
      hipError_t e = hipSuccess;
      if (pl.padded) {     // one build: one query sub-tile a wave in both phases
        constexpr int KP = (is_f32<T>() && D == 128) ? 64 : 128;
        p1.nqg = (nqs + WAVES * 16 - 1) / (WAVES * 16);
        p2.nqg = (pl.rt + WAVES * 16 - 1) / (WAVES * 16);
        const size_t itp = std::max<size_t>(std::max<size_t>((size_t)S * pl.c1 * pl.b2,
                                                             (size_t)S * pl.b1 * p1.nqg),
                                            (size_t)S * pl.b2 * pl.c1 * p2.nqg);
        if (qsplit) e = launch_cooperative(fused_t1_kernel<T, D, 1, KP, 1, PRECISE, true, true>, itp, args, st);
        else e = launch_cooperative(fused_t1_kernel<T, D, 1, KP, 1, PRECISE, false, true>, itp, args, st);
        if (e != hipSuccess) return e;
        break;
      }
#define MA_F3(NQ1, KTB, NQ2, QS) e = launch_cooperative(fused_t1_kernel<T, D, NQ1, KTB, NQ2, PRECISE, QS>, items, args, st)
#define MA_F2(NQ1, KTB, NQ2) do { if (qsplit) MA_F3(NQ1, KTB, NQ2, true); else MA_F3(NQ1, KTB, NQ2, false); } while (0)
#define MA_F1(NQ1, KTB) do { if (nq2 == 1) MA_F2(NQ1, KTB, 1); else MA_F2(NQ1, KTB, 2); } while (0)
      if constexpr (D == 128) {
        if (ktb64) MA_F1(1, 64);
        else if constexpr (!is_f32<T>()) MA_F1(1, 128);
      } else {
        if (nq1 == 1 || is_f32<T>()) {
          if (ktb64) MA_F1(1, 64); else MA_F1(1, 128);
        } else if constexpr (!is_f32<T>()) {
          if (ktb64) MA_F1(2, 64); else MA_F1(2, 128);
        }
      }
#undef MA_F1
#undef MA_F2
#undef MA_F3
      if (e != hipSuccess) return e;
      break;
    }
    case L_QBAR: {
      QbarParams p{b.q, qbar, pl.map, S, N, pl.b2, pl.c1, pl.rt, qbar_lp};
      ma_launch((qbar_kernel<T, D>), dim3(grid1((size_t)S * pl.c1 * pl.b2)), dim3(256), st, p);
      break;
    }
    case L_STAGE1:
    case L_STAGE1_LAST: {
      const int nqs = pl.c1 * pl.b2;
      if constexpr (!is_f32<T>()) {
        const int ktb = pl.b2 <= 64 ? 64 : 128;
        // the copied-tile kernel serves the first step when its queries are
        // bf16 rows (rows of Q, and with tiles or padding the bf16 tile means
        // of the plain c path), and the later steps of untiled, unpadded runs,
        // whose fp32 queries q~ it reads into registers (QF builds); other
        // fp32 query sources stay on the register-staged kernels
        const bool qf = step > 0 && pl.c1 == 1 && pl.c2 == 1 && !pl.padded;
        if (pl.b2 <= 128 && ((step == 0 && ((pl.c1 == 1 && !pl.padded) || qbar_lp)) || qf)) {
          // head_dim 128 keeps 4 waves (two waves a SIMD would spill the
          // K|V sums)
          const int nw = D == 64 ? async_waves(nqs) : 4, qg = nw * 16;
          Stage1Params p{b.q, b.k, b.v, qtil, qbar, cx, ux, h2, lser, pl.map,
                         S, N, pl.b1, pl.b2, pl.c1, pl.c2, pl.sw, pl.rt, nqs, (nqs + qg - 1) / qg,
                         pl.sc2, step == 0 ? 1 : 0, pl.xlo, qbar_lp};
          p.heads = pl.heads;
          p.group = pl.group;
          const size_t items = (size_t)S * pl.b1 * p.nqg;
          const bool last = kind == L_STAGE1_LAST;
#define MA_A1Q(NW, KTB, U, Q) launch_persistent(stage1_async_kernel<D, NW, KTB, U, PRECISE, false, Q>, NW * WAVE, items, p, st)
#define MA_A1(NW, KTB, U) do { if (qf) MA_A1Q(NW, KTB, U, true); else MA_A1Q(NW, KTB, U, false); } while (0)
#define MA_A1U(NW, KTB) do { if (last) MA_A1(NW, KTB, true); else MA_A1(NW, KTB, false); } while (0)
#define MA_A1F(NW, KTB, U, Q) launch_persistent(stage1_async_kernel<D, NW, KTB, U, PRECISE, false, Q, true>, NW * WAVE, items, p, st)
#define MA_A1UF(NW, KTB) do { if (last) { if (qf) MA_A1F(NW, KTB, true, true); else MA_A1F(NW, KTB, true, false); } \
                              else { if (qf) MA_A1F(NW, KTB, false, true); else MA_A1F(NW, KTB, false, false); } } while (0)
#define MA_A1K(NW) do { if (ktb == 64) { if (full) MA_A1UF(NW, 64); else MA_A1U(NW, 64); } \
                        else if (full) MA_A1UF(NW, 128); else MA_A1U(NW, 128); } while (0)
#define MA_A1P(NW) do { if (last) MA_A1X(NW, true); else MA_A1X(NW, false); } while (0)
#define MA_A1X(NW, U) launch_persistent(stage1_async_kernel<D, NW, 128, U, PRECISE, true>, NW * WAVE, items, p, st)
          // blocks that fill their key tiles in one segment: a build with that path only
          const bool full = pl.c2 == 1 && pl.b2 == ktb;
          bool small = false;
          if constexpr (D == 64 && !PRECISE) {
            // one step over blocks of 65-128 keys: the whole block's softmax
            // in one pass, c and u in turn, two workgroups a CU
            if (last && step == 0 && nw == 8 && Stage1Pair<D>::serves(pl.b2, pl.c1, pl.c2, pl.padded)) {
              small = true;
              launch_persistent(stage1_pair_kernel<D, false>, 8 * WAVE, items, p, st);
            } else if (last && step == 0 && nw == 8 && qbar_lp &&
                       Stage1Pair<D, true>::serves(pl.b2, pl.c1, pl.c2, pl.padded)) {
              small = true;
              launch_persistent(stage1_pair_kernel<D, true>, 8 * WAVE, items, p, st);
            }
          }
          if constexpr (D == 128 && !PRECISE) {
            // one step over blocks of at most 64 keys: c and u in turn, two
            // workgroups a CU
            if (last && step == 0 && !pl.padded && pl.b2 <= KT && (pl.c1 == 1 || qbar_lp)) {
              small = true;
              launch_persistent(stage1_small_kernel<D>, 4 * WAVE, items, p, st);
            }
          }
          if (small) {
          } else if (pl.padded) {     // padded sequences: 128-key tiles only
            if (nw == 8) { if constexpr (D == 64) MA_A1P(8); }
            else MA_A1P(4);
          } else if constexpr (D == 64) { if (nw == 8) MA_A1K(8); else MA_A1K(4); }
          else MA_A1K(4);
#undef MA_A1
#undef MA_A1Q
#undef MA_A1U
#undef MA_A1F
#undef MA_A1UF
#undef MA_A1K
#undef MA_A1P
#undef MA_A1X
          break;
        }
      }
      const int nq = stage1_nq<T, D>(nqs);
      const int qg = WAVES * nq * 16;
      Stage1Params p{b.q, b.k, b.v, qtil, qbar, cx, ux, h2, lser, pl.map,
                     S, N, pl.b1, pl.b2, pl.c1, pl.c2, pl.sw, pl.rt, nqs, (nqs + qg - 1) / qg,
                     pl.sc2, step == 0 ? 1 : 0, pl.xlo};
      p.heads = pl.heads;
      p.group = pl.group;
      const size_t items1 = (size_t)S * pl.b1 * p.nqg;
      const dim3 grid(grid1(items1));
      const bool ktb64 = pl.b2 <= 64 || (is_f32<T>() && D == 128);
      const bool last = kind == L_STAGE1_LAST;
      // queries from fp32 rows (next-step queries, tile means) need the split
      const bool qsplit = PRECISE && is_bf16<T>() && (step > 0 || pl.c1 > 1 || pl.padded);
      if (pl.padded) {     // one build: one query sub-tile a wave, 128-key tiles
        constexpr int KP = (is_f32<T>() && D == 128) ? 64 : 128;
        const int qgp = WAVES * 16;
        p.nqg = (nqs + qgp - 1) / qgp;
        const dim3 gp(grid1((size_t)S * pl.b1 * p.nqg));
#define MA_S1P(U, QS) ma_launch((stage1_kernel<T, D, 1, KP, U, PRECISE, QS, true>), gp, dim3(THREADS), st, p)
        if (last) { if (qsplit) MA_S1P(true, true); else MA_S1P(true, false); }
        else { if (qsplit) MA_S1P(false, true); else MA_S1P(false, false); }
#undef MA_S1P
        break;
      }
      // persistent pipelined kernel when the whole block fits one LDS tile
      const bool persistent = pl.b2 <= (ktb64 ? 64 : 128);
      const dim3 pgrid(grid1(std::min<size_t>(items1, persistent_slots())));
#define MA_S1_K(NQ, KTB, U, QS)                                                                   \
  do {                                                                                            \
    if (persistent)                                                                               \
      ma_launch((stage1_persistent_kernel<T, D, NQ, KTB, U, PRECISE, QS>), pgrid, dim3(THREADS), st, p); \
    else                                                                                          \
      ma_launch((stage1_kernel<T, D, NQ, KTB, U, PRECISE, QS>), grid, dim3(THREADS), st, p); \
  } while (0)
#define MA_S1(NQ, KTB, U)                                                                         \
  do {                                                                                            \
    if (qsplit) MA_S1_K(NQ, KTB, U, true); else MA_S1_K(NQ, KTB, U, false);                      \
  } while (0)
      if constexpr (D == 128) {
        if (ktb64) {
          if (last) MA_S1(1, 64, true); else MA_S1(1, 64, false);
        } else if constexpr (!is_f32<T>()) {
          if (last) MA_S1(1, 128, true); else MA_S1(1, 128, false);
        }
      } else {
        if (nq == 1 || is_f32<T>()) {
          if (ktb64) { if (last) MA_S1(1, 64, true); else MA_S1(1, 64, false); }
          else { if (last) MA_S1(1, 128, true); else MA_S1(1, 128, false); }
        } else if constexpr (!is_f32<T>()) {
          if (ktb64) { if (last) MA_S1(2, 64, true); else MA_S1(2, 64, false); }
          else { if (last) MA_S1(2, 128, true); else MA_S1(2, 128, false); }
        }
      }
#undef MA_S1_K
#undef MA_S1
      break;
    }
    case L_STAGE2_STATS:
    case L_STAGE2_LAST: {
      if constexpr (!is_f32<T>()) {
        {
          // last step at head_dim 128 (bidirectional, unpadded, fast path): 4
          // waves of 32 rows, KC_R32-key chunks, two workgroups a CU
          const bool rows32 = D == 128 && !PRECISE && !pl.causal && !pl.padded && kind == L_STAGE2_LAST;
          const int nw = rows32 ? 4 : stage2_waves<D>(pl.rt), qg = rows32 ? 128 : nw * 16;
          Stage2Params p{b.q, b.y, cx, ux, h2, lse2, kind == L_STAGE2_LAST ? b.lse : nullptr, pl.map,
                         S, N, pl.b1, pl.b2, pl.c1, pl.c2, pl.rt, pl.b1 * pl.c2, (pl.rt + qg - 1) / qg,
                         pl.sc2, pl.xlo, pl.causal};
          const size_t items = (size_t)S * pl.b2 * pl.c1 * p.nqg;
          const bool last = kind == L_STAGE2_LAST;
#define MA_A2C(NW, PV, C) launch_persistent(stage2_async_kernel<D, NW, 1, PV, PRECISE, KT, false, C>, NW * WAVE, items, p, st)
#define MA_A2(NW, PV) do { if (pl.causal) MA_A2C(NW, PV, true); else MA_A2C(NW, PV, false); } while (0)
#define MA_A2P(NW, PV) launch_persistent(stage2_async_kernel<D, NW, 1, PV, PRECISE, KT, true>, NW * WAVE, items, p, st)
          if constexpr (D == 128 && !PRECISE) {
            if (rows32) launch_persistent(stage2_async_kernel<D, 4, 2, true, PRECISE, KC_R32, false, false>, 4 * WAVE, items, p, st);
          }
          if (rows32) {
          } else if (pl.padded) {
            bool col = false;
            if constexpr (D == 64 && !PRECISE) {
              // the last step over columns of 65-128 keys: one chunk an item
              if (last && nw == 8 && Stage2Col<D, true>::serves(pl.b2, pl.c1, pl.b1 * pl.c2, pl.causal, true)) {
                col = true;
                launch_persistent(stage2_col_kernel<D, true>, 8 * WAVE, items, p, st);
              }
            }
            if (col) {
            } else if (nw == 8) { if (last) MA_A2P(8, true); else MA_A2P(8, false); }
            else { if (last) MA_A2P(4, true); else MA_A2P(4, false); }
          } else if (nw == 8) {
            bool one = false;            // a column of up to 128 keys in one chunk
            if constexpr (D == 64) {
              if (one_chunk2(pl)) {
                one = true;
                // (one_chunk2: no causal mask)
                if (last && !PRECISE) launch_persistent(stage2_col_kernel<D, false>, 8 * WAVE, items, p, st);
                else if (last) launch_persistent(stage2_async_kernel<D, 8, 1, true, PRECISE, 2 * KT, false, false>, 8 * WAVE, items, p, st);
                else launch_persistent(stage2_async_kernel<D, 8, 1, false, PRECISE, 2 * KT, false, false>, 8 * WAVE, items, p, st);
              }
            }
            if (!one) { if (last) MA_A2(8, true); else MA_A2(8, false); }
          }
          else { if (last) MA_A2(4, true); else MA_A2(4, false); }
#undef MA_A2
#undef MA_A2C
#undef MA_A2P
          break;
        }
      }
      const int nq = stage2_nq<T, D>(pl.rt);
      const int qg = WAVES * nq * 16;
      Stage2Params p{b.q, b.y, cx, ux, h2, lse2, kind == L_STAGE2_LAST ? b.lse : nullptr, pl.map,
                     S, N, pl.b1, pl.b2, pl.c1, pl.c2, pl.rt, pl.b1 * pl.c2, (pl.rt + qg - 1) / qg,
                     pl.sc2, pl.xlo, pl.causal};
      const bool last = kind == L_STAGE2_LAST;
      if (pl.padded) {     // one build: one query sub-tile a wave
        p.nqg = (pl.rt + WAVES * 16 - 1) / (WAVES * 16);
        const dim3 gp(grid1((size_t)S * pl.b2 * pl.c1 * p.nqg));
        if (last) ma_launch((stage2_kernel<T, D, 1, true, PRECISE, true>), gp, dim3(THREADS), st, p);
        else ma_launch((stage2_kernel<T, D, 1, false, PRECISE, true>), gp, dim3(THREADS), st, p);
        break;
      }
      const size_t items2 = (size_t)S * pl.b2 * pl.c1 * p.nqg;
      const dim3 grid(grid1(items2));
      const int nkeys = pl.b1 * pl.c2;
      const int ktb = nkeys <= 64 ? 64 : 128;
      const bool persistent = nkeys <= ((is_f32<T>() && D == 128) ? 64 : 128);
      const dim3 pgrid(grid1(std::min<size_t>(items2, persistent_slots())));
#define MA_S2_P(NQ, PV)                                                                           \
  do {                                                                                            \
    if (ktb == 64)                                                                                \
      ma_launch((stage2_persistent_kernel<T, D, NQ, 64, PV, PRECISE>), pgrid, dim3(THREADS), st, p); \
    else if constexpr (!(is_f32<T>() && D == 128))                                                \
      ma_launch((stage2_persistent_kernel<T, D, NQ, 128, PV, PRECISE>), pgrid, dim3(THREADS), st, p); \
  } while (0)
#define MA_S2(NQ, PV)                                                                             \
  do {                                                                                            \
    if (persistent) MA_S2_P(NQ, PV);                                                              \
    else ma_launch((stage2_kernel<T, D, NQ, PV, PRECISE>), grid, dim3(THREADS), st, p); \
  } while (0)
      if (nq == 1) { if (last) MA_S2(1, true); else MA_S2(1, false); }
      else { if (last) MA_S2(2, true); else MA_S2(2, false); }
#undef MA_S2_P
#undef MA_S2
      break;
    }
    case L_STAGE2_ALPHA: {
      if constexpr (!is_f32<T>()) {
        // one workgroup per column (b1 <= 64 rows and keys, untiled)
        Stage2Params p{b.q, b.y, cx, ux, h2, lse2, nullptr, pl.map,
                       S, N, pl.b1, pl.b2, 1, 1, pl.rt, pl.b1, 1, pl.sc2, pl.xlo, 0};
        ma_launch((stage2_alpha_kernel<D, PRECISE>), dim3(grid1((size_t)S * pl.b2)), dim3(256), st,
                           p, qtil);
      }
      break;
    }
    case L_ALPHA:
    case L_EXPORT_L: {
      const int nkeys = pl.b1 * pl.c2;
      AlphaParams p{b.q, cx, h2, lse2, qbar, kind == L_ALPHA ? qtil : nullptr,
                    kind == L_EXPORT_L ? b.L : nullptr, pl.map,
                    S, N, pl.b1, pl.b2, pl.c1, pl.c2, pl.rt, nkeys, (nkeys + KT - 1) / KT, pl.sc2,
                    pl.xlo};
      p.beta_out = kind == L_ALPHA && pl.beta_out ? reinterpret_cast<float*>(ws + pl.off_beta) : nullptr;
      p.causal = pl.causal;
      const size_t wgs = (size_t)S * pl.b2 * pl.c1 * p.nkt;
      ma_launch((alpha_kernel<T, D, PRECISE>), dim3(grid1(wgs)), dim3(THREADS), st, p);
      break;
    }
    case L_EXPORT_R: {
      RExportParams p{b.q, b.k, qtil, qbar, lser, b.R, pl.map, S, N, pl.b1, pl.b2, pl.c1, pl.c2,
                      pl.sw, pl.rt, (int)pl.D, pl.sc2, step == 0 ? 1 : 0};
      p.heads = pl.heads;
      p.group = pl.group;
      const size_t total = (size_t)S * pl.b1 * pl.b2 * pl.c1 * pl.b2;
      ma_launch(r_export_kernel<T>, dim3(grid1((total + 255) / 256)), dim3(256), st, p);
      break;
    }
    case L_OBJECTIVE: {
      ObjectiveParams p{lse2, b.obj, pl.map};
      ma_launch(objective_kernel, dim3(S), dim3(256), st, p);
      break;
    }
  }
  return hipGetLastError();
}

template <typename T, int D, bool PRECISE>
ma_status run_t(const Plan& pl, const Bufs& b, hipStream_t st, void* const* events, int n_events) {
  ma_status status = MA_OK;
  for_each_launch(pl, b.L != nullptr, b.R != nullptr, b.obj != nullptr,
                  [&](int j, LaunchKind kind, int step) {
                    if (status != MA_OK) return;
                    if (events && 2 * j + 1 < n_events)
                      launch_events() = LaunchEvents{(hipEvent_t)events[2 * j], (hipEvent_t)events[2 * j + 1]};
                    const hipError_t e = launch_one<T, D, PRECISE>(pl, b, kind, step, st);
                    launch_events() = LaunchEvents{};
                    if (e != hipSuccess) status = MA_ERR_DEVICE;
                  });
  return status;
}


}  // namespace ma
