// C ABI of the MonarchAttention forward pass (see include/monarch_attn.h):
// host-side validation, workspace plan and the launch sequence.
#include "../../include/monarch_attn.h"
#include "ma_kernels.hpp"

#include <cmath>
#include <cstring>

namespace {

using namespace ma;

constexpr size_t ALIGN = 256;
inline size_t align_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

// Largest segment width (keys per R row) the stage-1 kernel streams.  The
// kernel itself streams any width; the bound keeps the exchange and the
// R export within the sizes validated so far.
constexpr int MAX_SEGMENT = 128;

struct Plan {
  int64_t S, N, D;
  int b1, b2, c1, c2, sw, rt, T;
  int dtype;
  float scale, sc2;
  GridMap map;
  size_t elt, xc_elt;
  bool precise;
  size_t off_cx, off_ux, off_h2, off_lser, off_lse2, off_qtil, off_qbar, total;
  bool need_qbar, need_qtil;
};

ma_status validate_problem(const ma_problem* p) {
  if (!p) return MA_ERR_INVALID_ARGUMENT;
  if (p->batch < 1 || p->heads < 1 || p->seq_len < 1 || p->head_dim < 1) return MA_ERR_INVALID_ARGUMENT;
  if (p->b1 < 1 || p->b2 < 1 || (int64_t)p->b1 * p->b2 != p->seq_len) return MA_ERR_INVALID_ARGUMENT;
  if (p->c1 < 1 || p->c2 < 1 || p->b1 % p->c1 != 0 || p->b2 % p->c2 != 0) return MA_ERR_INVALID_ARGUMENT;
  if (p->steps < 1) return MA_ERR_INVALID_ARGUMENT;
  if (!(std::isfinite(p->scale)) || p->scale < 0.f) return MA_ERR_INVALID_ARGUMENT;
  if (p->dtype != MA_F32 && p->dtype != MA_BF16) return MA_ERR_INVALID_ARGUMENT;
  if (p->layout < MA_LAYOUT_FLAT || p->layout > MA_LAYOUT_H_FW) return MA_ERR_INVALID_ARGUMENT;
  if (p->layout != MA_LAYOUT_FLAT) {
    const int64_t f = p->f, h = p->h, w = p->w;
    if (f < 1 || h < 1 || w < 1 || f * h * w != p->seq_len) return MA_ERR_INVALID_ARGUMENT;
    int64_t e1 = 0, e2 = 0;
    switch (p->layout) {
      case MA_LAYOUT_FH_W: e1 = f * h; e2 = w; break;
      case MA_LAYOUT_W_FH: e1 = w; e2 = f * h; break;
      case MA_LAYOUT_F_HW: e1 = f; e2 = h * w; break;
      case MA_LAYOUT_HW_F: e1 = h * w; e2 = f; break;
      case MA_LAYOUT_FW_H: e1 = f * w; e2 = h; break;
      case MA_LAYOUT_H_FW: e1 = h; e2 = f * w; break;
    }
    if (e1 != p->b1 || e2 != p->b2) return MA_ERR_INVALID_ARGUMENT;
  }
  if (p->head_dim != 64 && p->head_dim != 128) return MA_ERR_UNSUPPORTED;
  if (p->b2 / p->c2 > MAX_SEGMENT) return MA_ERR_UNSUPPORTED;
  const int64_t slices = p->batch * p->heads;
  if (slices > (int64_t)1 << 24 || p->seq_len > (int64_t)1 << 26) return MA_ERR_UNSUPPORTED;
  return MA_OK;
}

Plan make_plan(const ma_problem* p) {
  Plan pl;
  pl.S = p->batch * p->heads;
  pl.N = p->seq_len;
  pl.D = p->head_dim;
  pl.b1 = p->b1; pl.b2 = p->b2; pl.c1 = p->c1; pl.c2 = p->c2;
  pl.sw = p->b2 / p->c2;
  pl.rt = p->b1 / p->c1;
  pl.T = p->steps;
  pl.dtype = p->dtype;
  pl.scale = p->scale > 0.f ? p->scale : 1.f / std::sqrt((float)p->head_dim);
  pl.sc2 = pl.scale * LOG2E;
  pl.map.kind = p->layout;
  pl.map.b1 = p->b1; pl.map.b2 = p->b2;
  pl.map.h = p->h; pl.map.w = p->w; pl.map.hw = p->h * p->w;
  pl.elt = p->dtype == MA_F32 ? 4 : 2;
  pl.precise = p->dtype == MA_F32 || !(p->flags & MA_FLAG_FAST_AGGREGATE);
  pl.xc_elt = pl.precise ? 4 : 2;
  pl.need_qtil = p->steps > 1;
  pl.need_qbar = p->steps > 1 || p->c1 > 1;
  const size_t rows = (size_t)pl.S * pl.N * pl.c1 * pl.c2;   // exchange rows
  size_t off = 0;
  pl.off_cx = off;   off = align_up(off + rows * pl.D * pl.xc_elt);
  pl.off_ux = off;   off = align_up(off + rows * pl.D * pl.elt);
  pl.off_h2 = off;   off = align_up(off + rows * 4);
  pl.off_lser = off; off = align_up(off + rows * 4);
  pl.off_lse2 = off; off = align_up(off + (size_t)pl.S * pl.N * 4);
  pl.off_qtil = off; if (pl.need_qtil) off = align_up(off + rows * pl.D * 4);
  pl.off_qbar = off; if (pl.need_qbar) off = align_up(off + (size_t)pl.S * pl.c1 * pl.b2 * pl.D * 4);
  pl.total = off;
  return pl;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

// The launch sequence, shared by the real run, the launch count and the
// launch names.  `Launcher` is called once per kernel launch in order.
enum LaunchKind { L_QBAR, L_STAGE1, L_STAGE1_LAST, L_STAGE2_STATS, L_STAGE2_LAST, L_ALPHA,
                  L_EXPORT_L, L_EXPORT_R, L_OBJECTIVE };

const char* launch_kind_name(LaunchKind k) {
  switch (k) {
    case L_QBAR: return "qbar";
    case L_STAGE1: return "stage1";
    case L_STAGE1_LAST: return "stage1_last";
    case L_STAGE2_STATS: return "stage2_stats";
    case L_STAGE2_LAST: return "stage2_last";
    case L_ALPHA: return "alpha";
    case L_EXPORT_L: return "export_L";
    case L_EXPORT_R: return "export_R";
    case L_OBJECTIVE: return "objective";
  }
  return "?";
}

template <class F>
void for_each_launch(const Plan& pl, bool exp_L, bool exp_R, bool exp_obj, F&& f) {
  int j = 0;
  if (pl.need_qbar) f(j++, L_QBAR, 0);
  for (int step = 0; step < pl.T; ++step) {
    const bool last = step == pl.T - 1;
    f(j++, last ? L_STAGE1_LAST : L_STAGE1, step);
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

inline unsigned grid1(size_t n) { return (unsigned)n; }

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
  const int S = (int)pl.S, N = (int)pl.N;
  switch (kind) {
    case L_QBAR: {
      QbarParams p{b.q, qbar, pl.map, S, N, pl.b2, pl.c1, pl.rt, (int)pl.D};
      const size_t total = (size_t)S * pl.c1 * pl.b2 * pl.D;
      hipLaunchKernelGGL(qbar_kernel<T>, dim3(grid1((total + 255) / 256)), dim3(256), 0, st, p);
      break;
    }
    case L_STAGE1:
    case L_STAGE1_LAST: {
      constexpr int NQ = 1;
      const int qg = WAVES * NQ * 16;
      Stage1Params p{b.q, b.k, b.v, qtil, qbar, cx, ux, h2, lser, pl.map,
                     S, N, pl.b1, pl.b2, pl.c1, pl.c2, pl.sw, pl.rt, (pl.b2 + qg - 1) / qg,
                     pl.sc2, step == 0 ? 1 : 0};
      const size_t wgs = (size_t)S * pl.b1 * pl.c1 * pl.c2 * p.nqg;
      if (kind == L_STAGE1_LAST)
        hipLaunchKernelGGL((stage1_kernel<T, D, NQ, true, PRECISE>), dim3(grid1(wgs)), dim3(THREADS), 0, st, p);
      else
        hipLaunchKernelGGL((stage1_kernel<T, D, NQ, false, PRECISE>), dim3(grid1(wgs)), dim3(THREADS), 0, st, p);
      break;
    }
    case L_STAGE2_STATS:
    case L_STAGE2_LAST: {
      constexpr int NQ = 1;
      const int qg = WAVES * NQ * 16;
      Stage2Params p{b.q, b.y, cx, ux, h2, lse2, kind == L_STAGE2_LAST ? b.lse : nullptr, pl.map,
                     S, N, pl.b1, pl.b2, pl.c1, pl.c2, pl.rt, pl.b1 * pl.c2, (pl.rt + qg - 1) / qg,
                     pl.sc2};
      const size_t wgs = (size_t)S * pl.b2 * pl.c1 * p.nqg;
      if (kind == L_STAGE2_LAST)
        hipLaunchKernelGGL((stage2_kernel<T, D, NQ, true, PRECISE>), dim3(grid1(wgs)), dim3(THREADS), 0, st, p);
      else
        hipLaunchKernelGGL((stage2_kernel<T, D, NQ, false, PRECISE>), dim3(grid1(wgs)), dim3(THREADS), 0, st, p);
      break;
    }
    case L_ALPHA:
    case L_EXPORT_L: {
      const int nkeys = pl.b1 * pl.c2;
      AlphaParams p{b.q, cx, h2, lse2, qbar, kind == L_ALPHA ? qtil : nullptr,
                    kind == L_EXPORT_L ? b.L : nullptr, pl.map,
                    S, N, pl.b1, pl.b2, pl.c1, pl.c2, pl.rt, nkeys, (nkeys + KT - 1) / KT, pl.sc2};
      const size_t wgs = (size_t)S * pl.b2 * pl.c1 * p.nkt;
      hipLaunchKernelGGL((alpha_kernel<T, D, PRECISE>), dim3(grid1(wgs)), dim3(THREADS), 0, st, p);
      break;
    }
    case L_EXPORT_R: {
      RExportParams p{b.q, b.k, qtil, qbar, lser, b.R, pl.map, S, N, pl.b1, pl.b2, pl.c1, pl.c2,
                      pl.sw, pl.rt, (int)pl.D, pl.sc2, step == 0 ? 1 : 0};
      const size_t total = (size_t)S * pl.b1 * pl.b2 * pl.c1 * pl.b2;
      hipLaunchKernelGGL(r_export_kernel<T>, dim3(grid1((total + 255) / 256)), dim3(256), 0, st, p);
      break;
    }
    case L_OBJECTIVE: {
      ObjectiveParams p{lse2, b.obj, N};
      hipLaunchKernelGGL(objective_kernel, dim3(S), dim3(256), 0, st, p);
      break;
    }
  }
  return hipGetLastError();
}

template <typename T, int D, bool PRECISE>
ma_status run(const Plan& pl, const Bufs& b, hipStream_t st, void* const* events, int n_events) {
  ma_status status = MA_OK;
  if (events && n_events > 0 && hipEventRecord((hipEvent_t)events[0], st) != hipSuccess) return MA_ERR_DEVICE;
  for_each_launch(pl, b.L != nullptr, b.R != nullptr, b.obj != nullptr,
                  [&](int j, LaunchKind kind, int step) {
                    if (status != MA_OK) return;
                    if (launch_one<T, D, PRECISE>(pl, b, kind, step, st) != hipSuccess) { status = MA_ERR_DEVICE; return; }
                    if (events && j + 1 < n_events &&
                        hipEventRecord((hipEvent_t)events[j + 1], st) != hipSuccess)
                      status = MA_ERR_DEVICE;
                  });
  return status;
}

ma_status forward_impl(const ma_problem* p, const void* q, const void* k, const void* v, void* y,
                       const ma_exports* ex, void* workspace, size_t workspace_bytes, void* stream,
                       void* const* events, int32_t n_events) {
  ma_status s = validate_problem(p);
  if (s != MA_OK) return s;
  const Plan pl = make_plan(p);
  if (!q || !k || !v || !y) return MA_ERR_INVALID_ARGUMENT;
  auto misaligned = [](const void* x, uintptr_t a) { return ((uintptr_t)x % a) != 0; };
  if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(y, 16))
    return MA_ERR_INVALID_ARGUMENT;
  const size_t tbytes = (size_t)pl.S * pl.N * pl.D * pl.elt;
  if (overlaps(y, tbytes, q, tbytes) || overlaps(y, tbytes, k, tbytes) || overlaps(y, tbytes, v, tbytes))
    return MA_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < pl.total) return MA_ERR_WORKSPACE_TOO_SMALL;
  if (pl.total > 0) {
    if (!workspace || misaligned(workspace, ALIGN)) return MA_ERR_INVALID_ARGUMENT;
    if (overlaps(workspace, pl.total, q, tbytes) || overlaps(workspace, pl.total, k, tbytes) ||
        overlaps(workspace, pl.total, v, tbytes) || overlaps(workspace, pl.total, y, tbytes))
      return MA_ERR_INVALID_ARGUMENT;
  }
  Bufs b{q, k, v, y, static_cast<char*>(workspace), nullptr, nullptr, nullptr, nullptr};
  if (ex) {
    b.L = ex->L; b.R = ex->R; b.lse = ex->lse; b.obj = ex->objective;
    if ((b.L && misaligned(b.L, 4)) || (b.R && misaligned(b.R, 4)) || (b.lse && misaligned(b.lse, 4)) ||
        (b.obj && misaligned(b.obj, 8)))
      return MA_ERR_INVALID_ARGUMENT;
  }
  if (n_events < 0) return MA_ERR_INVALID_ARGUMENT;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (pl.dtype == MA_BF16) {
    if (pl.precise) {
      if (pl.D == 64) return run<bf16, 64, true>(pl, b, st, events, n_events);
      return run<bf16, 128, true>(pl, b, st, events, n_events);
    }
    if (pl.D == 64) return run<bf16, 64, false>(pl, b, st, events, n_events);
    return run<bf16, 128, false>(pl, b, st, events, n_events);
  }
  if (pl.D == 64) return run<float, 64, true>(pl, b, st, events, n_events);
  return run<float, 128, true>(pl, b, st, events, n_events);
}

}  // namespace

extern "C" {

ma_status monarch_attn_workspace_size(const ma_problem* p, size_t* bytes) {
  if (!bytes) return MA_ERR_INVALID_ARGUMENT;
  const ma_status s = validate_problem(p);
  if (s != MA_OK) return s;
  *bytes = make_plan(p).total;
  return MA_OK;
}

ma_status monarch_attn_forward(const ma_problem* p, const void* q, const void* k, const void* v,
                               void* y, const ma_exports* exports, void* workspace,
                               size_t workspace_bytes, void* stream) {
  return forward_impl(p, q, k, v, y, exports, workspace, workspace_bytes, stream, nullptr, 0);
}

ma_status monarch_attn_forward_timed(const ma_problem* p, const void* q, const void* k, const void* v,
                                     void* y, const ma_exports* exports, void* workspace,
                                     size_t workspace_bytes, void* stream, void* const* events,
                                     int32_t n_events) {
  return forward_impl(p, q, k, v, y, exports, workspace, workspace_bytes, stream, events, n_events);
}

int32_t monarch_attn_num_launches(const ma_problem* p) {
  if (validate_problem(p) != MA_OK) return -1;
  int32_t n = 0;
  for_each_launch(make_plan(p), false, false, false, [&](int, LaunchKind, int) { ++n; });
  return n;
}

const char* monarch_attn_launch_name(const ma_problem* p, int32_t j) {
  if (validate_problem(p) != MA_OK) return nullptr;
  const char* name = nullptr;
  for_each_launch(make_plan(p), false, false, false, [&](int jj, LaunchKind kind, int) {
    if (jj == j) name = launch_kind_name(kind);
  });
  return name;
}

ma_status monarch_attn_event_create(void** event) {
  if (!event) return MA_ERR_INVALID_ARGUMENT;
  hipEvent_t e;
  if (hipEventCreate(&e) != hipSuccess) return MA_ERR_DEVICE;
  *event = e;
  return MA_OK;
}

ma_status monarch_attn_event_destroy(void* event) {
  if (!event) return MA_ERR_INVALID_ARGUMENT;
  return hipEventDestroy((hipEvent_t)event) == hipSuccess ? MA_OK : MA_ERR_DEVICE;
}

ma_status monarch_attn_event_elapsed_ms(void* a, void* b, float* ms) {
  if (!a || !b || !ms) return MA_ERR_INVALID_ARGUMENT;
  if (hipEventSynchronize((hipEvent_t)b) != hipSuccess) return MA_ERR_DEVICE;
  return hipEventElapsedTime(ms, (hipEvent_t)a, (hipEvent_t)b) == hipSuccess ? MA_OK : MA_ERR_DEVICE;
}

const char* monarch_attn_status_string(ma_status s) {
  switch (s) {
    case MA_OK: return "ok";
    case MA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case MA_ERR_UNSUPPORTED: return "unsupported problem";
    case MA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MA_ERR_DEVICE: return "device error";
  }
  return "unknown status";
}

const char* monarch_attn_version(void) { return "0.1.0"; }

}  // extern "C"
