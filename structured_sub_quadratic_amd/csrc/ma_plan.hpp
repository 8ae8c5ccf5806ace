// Host-side plan of a MonarchAttention forward call: the workspace layout and
// the launch sequence, shared by the C ABI and the per-type launch units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/monarch_attn.h"
#include "ma_device.hpp"

namespace ma {

constexpr size_t ALIGN = 256;
inline size_t align_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

// Largest segment width (keys per R row): one segment must fit the stage-1
// LDS tile (128 keys; 64 for fp32 with head_dim 128, whose tiles are twice
// as large).
inline int max_segment(const ma_problem* p) {
  return (p->dtype == MA_F32 && p->head_dim == 128) ? 64 : 128;
}

struct Plan {
  int64_t S, N, D;
  int64_t G;           // grid positions b1*b2 (N, or more for a padded flat sequence)
  bool padded;
  int heads, group;    // query heads; query heads per K/V head
  int b1, b2, c1, c2, sw, rt, T;
  int dtype;
  float scale, sc2;
  GridMap map;
  size_t elt, xc_elt;
  size_t xlo;          // elements from the hi plane of split c to its lo plane (0: not split)
  bool precise;
  size_t off_cx, off_ux, off_h2, off_lser, off_lse2, off_qtil, off_qbar, off_qbar_lp, total;
  size_t off_dq2, off_dcx, off_dux, off_dhx, off_dkp, off_dvp, off_dlx, off_dqbar;   // backward only
  size_t off_dq2p;     // backward, columns of several key chunks: dq2_parts parts of the dQ sum
  int dq2_parts;
  // backward of T > 1: per-step forward state, T regions of step_bytes from
  // off_steps (offsets so_* inside one), the column sums beta of L, and the
  // gradients of the next queries (dq~ / dalpha rows and dbeta)
  size_t off_steps, step_bytes, so_cx, so_h2, so_lser, so_lse2, so_qtil, so_beta;
  size_t off_beta, off_dqt, off_dbt;
  bool beta_out;       // the alpha launch also stores beta at off_beta
  bool reuse_state;    // backward: the forward state is in the workspace already
  bool need_qbar, need_qtil;
  bool need_qbar_lp;   // tile means also in the input type (copied-tile first step)
  bool fused;        // single cooperative launch for T = 1
  bool fuse_alpha;   // steps before the last: L-update and next queries in one launch
  int causal;        // 0, or grid blocks per causal unit when that masks anything (< b1)
};

// The plan of step t of a T > 1 backward: the forward kernels read and write
// that step's state region.
inline Plan step_plan(const Plan& pl, int t) {
  Plan s = pl;
  const size_t base = pl.off_steps + (size_t)t * pl.step_bytes;
  s.off_cx = base + pl.so_cx;
  s.off_h2 = base + pl.so_h2;
  s.off_lser = base + pl.so_lser;
  s.off_lse2 = base + pl.so_lse2;
  s.off_qtil = base + pl.so_qtil;
  s.off_beta = base + pl.so_beta;
  return s;
}

// The launch sequence, shared by the real run, the launch count and the
// launch names.  `Launcher` is called once per kernel launch in order.
enum LaunchKind { L_FUSED, L_QBAR, L_STAGE1, L_STAGE1_LAST, L_STAGE2_STATS, L_STAGE2_LAST, L_ALPHA,
                  L_STAGE2_ALPHA, L_EXPORT_L, L_EXPORT_R, L_OBJECTIVE };

inline const char* launch_kind_name(LaunchKind k) {
  switch (k) {
    case L_FUSED: return "fused_t1";
    case L_QBAR: return "qbar";
    case L_STAGE1: return "stage1";
    case L_STAGE1_LAST: return "stage1_last";
    case L_STAGE2_STATS: return "stage2_stats";
    case L_STAGE2_LAST: return "stage2_last";
    case L_ALPHA: return "alpha";
    case L_STAGE2_ALPHA: return "stage2_alpha";
    case L_EXPORT_L: return "export_L";
    case L_EXPORT_R: return "export_R";
    case L_OBJECTIVE: return "objective";
  }
  return "?";
}

template <class F>
void for_each_launch(const Plan& pl, bool exp_L, bool exp_R, bool exp_obj, F&& f) {
  int j = 0;
  if (pl.fused) {
    f(j++, L_FUSED, 0);
  } else {
    // the fused L-update takes the zero-weight fallback (a column mean) itself
    if (pl.need_qbar && !pl.fuse_alpha) f(j++, L_QBAR, 0);
  }
  for (int step = 0; step < (pl.fused ? 0 : pl.T); ++step) {
    const bool last = step == pl.T - 1;
    f(j++, last ? L_STAGE1_LAST : L_STAGE1, step);
    if (!last && pl.fuse_alpha) {
      f(j++, L_STAGE2_ALPHA, step);
      continue;
    }
    f(j++, last ? L_STAGE2_LAST : L_STAGE2_STATS, step);
    if (!last) f(j++, L_ALPHA, step);
  }
  if (exp_L) f(j++, L_EXPORT_L, pl.T - 1);
  if (exp_R) f(j++, L_EXPORT_R, pl.T - 1);
  if (exp_obj) f(j++, L_OBJECTIVE, pl.T - 1);
}

struct Bufs {
  const void *q, *k, *v;
  void* y;
  char* ws;
  float *L, *R, *lse;
  double* obj;
};

struct BwdBufs {
  const void *q, *k, *v, *dy;
  void *dq, *dk, *dv;
  char* ws;
  const void* y;       // the forward's output, or null
};

// Largest blocks of the backward: the keys of a stage-1 block sit in LDS
// whole (b2 <= bwd_max_block); a stage-2 column of more keys walks them in
// chunks of that size.
inline int bwd_max_block(const ma_problem* p) {
  return (p->dtype == MA_F32 && p->head_dim == 128) ? 64 : 128;
}
// Keys of a stage-2 chunk of the backward: bf16 at head_dim 128 with T > 1
// reads c as two planes and keeps to 64.
inline int bwd_key_chunk(const ma_problem* p) {
  return (p->dtype == MA_BF16 && p->head_dim == 128 && p->steps > 1) ? 64 : bwd_max_block(p);
}

// Kernel-launch entry of one element type and head dimension (one
// translation unit each): runs the whole launch sequence of *pl on st.
typedef ma_status (*RunFn)(const Plan& pl, const Bufs& b, hipStream_t st, void* const* events,
                           int n_events);
ma_status run_bf16_64_precise(const Plan&, const Bufs&, hipStream_t, void* const*, int);
ma_status run_bf16_64_fast(const Plan&, const Bufs&, hipStream_t, void* const*, int);
ma_status run_bf16_128_precise(const Plan&, const Bufs&, hipStream_t, void* const*, int);
ma_status run_bf16_128_fast(const Plan&, const Bufs&, hipStream_t, void* const*, int);
ma_status run_f32_64(const Plan&, const Bufs&, hipStream_t, void* const*, int);
ma_status run_f32_128(const Plan&, const Bufs&, hipStream_t, void* const*, int);
ma_status run_bwd_bf16_64(const Plan&, const BwdBufs&, hipStream_t);
ma_status run_bwd_bf16_128(const Plan&, const BwdBufs&, hipStream_t);
ma_status run_bwd_f32_64(const Plan&, const BwdBufs&, hipStream_t);
ma_status run_bwd_f32_128(const Plan&, const BwdBufs&, hipStream_t);
ma_status run_bwd_steps_bf16_64(const Plan&, const BwdBufs&, hipStream_t);   // T > 1, split c
ma_status run_bwd_steps_bf16_128(const Plan&, const BwdBufs&, hipStream_t);

}  // namespace ma
