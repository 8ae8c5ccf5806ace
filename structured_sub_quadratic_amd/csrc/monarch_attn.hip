// C ABI of the MonarchAttention forward pass (see include/monarch_attn.h):
// host-side validation, the workspace plan and dispatch to the per-type
// launch units.
#include "ma_plan.hpp"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>

// Workspace of monarch_attn_forward_noalloc: one fixed device array, which
// every GPU the library runs on holds (its own copy, at its own address)
// from the load of this code object until the process ends.  In host code
// `scratch` is a host-side stand-in, never a device address: the device
// address comes from hipGetSymbolAddress, taken once per device with that
// device current, and only that address is passed on.
static __device__ __align__(256) char scratch[MONARCH_ATTN_SCRATCH_BYTES];

namespace {

using namespace ma;

constexpr int MAX_DEVICES = 64;
std::mutex scratch_mu;
void* scratch_at[MAX_DEVICES];      // device address of `scratch` per device, or null

// Device address of the current device's scratch array (looked up on the
// first call on that device).
ma_status device_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MA_ERR_DEVICE;
  if (dev < 0 || dev >= MAX_DEVICES) return MA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_at[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return MA_ERR_DEVICE;
    scratch_at[dev] = ptr;
  }
  *out = scratch_at[dev];
  return MA_OK;
}

ma_status validate_problem(const ma_problem* p) {
  if (!p) return MA_ERR_INVALID_ARGUMENT;
  if (p->batch < 1 || p->heads < 1 || p->seq_len < 1 || p->head_dim < 1) return MA_ERR_INVALID_ARGUMENT;
  if (p->b1 < 1 || p->b2 < 1) return MA_ERR_INVALID_ARGUMENT;
  if (p->c1 < 1 || p->c2 < 1 || p->b1 % p->c1 != 0 || p->b2 % p->c2 != 0) return MA_ERR_INVALID_ARGUMENT;
  const int64_t grid = (int64_t)p->b1 * p->b2;
  if (p->layout == MA_LAYOUT_FLAT) {
    // a flat sequence may be padded to the grid, as long as every key
    // segment keeps a real key
    if (grid < p->seq_len || grid - p->seq_len >= p->b2 / p->c2) return MA_ERR_INVALID_ARGUMENT;
  } else if (grid != p->seq_len) {
    return MA_ERR_INVALID_ARGUMENT;
  }
  if (p->steps < 1 || p->causal < 0) return MA_ERR_INVALID_ARGUMENT;
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
  const int64_t kvh = p->kv_heads ? p->kv_heads : p->heads;
  if (kvh < 1 || kvh > p->heads || p->heads % kvh != 0) return MA_ERR_INVALID_ARGUMENT;
  if (p->head_dim != 64 && p->head_dim != 128) return MA_ERR_UNSUPPORTED;
  if (p->b2 / p->c2 > max_segment(p)) return MA_ERR_UNSUPPORTED;
  const int64_t slices = p->batch * p->heads;
  if (slices > (int64_t)1 << 24 || grid > (int64_t)1 << 26) return MA_ERR_UNSUPPORTED;
  // work items and exchange rows are counted in 32 bits
  if (slices * grid * p->c1 * p->c2 > INT32_MAX) return MA_ERR_UNSUPPORTED;
  return MA_OK;
}

// backward: the forward state it recomputes takes the forward's default c
// path (bf16: plain for T = 1, split for T > 1), T > 1 keeps that state per
// step, and the workspace adds the gradient buffers
Plan make_plan(const ma_problem* p, bool backward = false) {
  Plan pl;
  pl.S = p->batch * p->heads;
  pl.heads = (int)p->heads;
  pl.group = (int)(p->heads / (p->kv_heads ? p->kv_heads : p->heads));
  pl.N = p->seq_len;
  pl.G = (int64_t)p->b1 * p->b2;
  pl.padded = pl.G != pl.N;
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
  pl.map.pre = (p->flags & MA_FLAG_PAD_FRONT) ? (int)(pl.G - pl.N) : 0;
  pl.map.n = (int)pl.N;
  pl.elt = p->dtype == MA_F32 ? 4 : 2;
  pl.precise = p->dtype == MA_F32 || (p->flags & MA_FLAG_PRECISE_AGGREGATE) ||
               (!(p->flags & MA_FLAG_FAST_AGGREGATE) && p->steps > 1);
  if (backward) pl.precise = p->dtype == MA_F32 || p->steps > 1;
  const bool steps_state = backward && p->steps > 1;   // per-step regions instead of one
  const bool tiled_bwd = backward && (p->c1 > 1 || p->c2 > 1);   // query gradients per exchange row
  pl.xc_elt = pl.precise ? 4 : 2;
  pl.need_qtil = p->steps > 1;
  // tile means: the zero-weight fallback (tiles other than the own one,
  // padding rows, zero column weight at later steps)
  pl.need_qbar = p->steps > 1 || p->c1 > 1 || pl.padded;
  pl.need_qbar_lp = pl.need_qbar && (p->c1 > 1 || pl.padded) && !pl.precise;
  pl.fused = !backward && p->steps == 1 && (p->flags & MA_FLAG_FORCE_FUSED) &&
             !(p->flags & MA_FLAG_FORCE_STAGED);
  // a causal unit of at least b1 blocks masks nothing
  pl.causal = p->causal < p->b1 ? p->causal : 0;
  // columns of at most 64 rows and keys (untiled, unpadded, bf16, no mask):
  // the steps before the last run the L-update and the next queries in one
  // launch
  pl.fuse_alpha = !backward && p->steps > 1 && p->dtype == MA_BF16 && p->c1 == 1 && p->c2 == 1 &&
                  !pl.padded && p->b1 <= 64 && pl.causal == 0;
  const size_t rows = (size_t)pl.S * pl.G * pl.c1 * pl.c2;   // exchange rows
  size_t off = 0;
  pl.xlo = (pl.precise && p->dtype == MA_BF16) ? rows * pl.D : 0;
  pl.beta_out = false;
  pl.reuse_state = backward && (p->flags & MA_FLAG_REUSE_FORWARD_STATE);
  pl.off_steps = pl.step_bytes = pl.so_cx = pl.so_h2 = pl.so_lser = pl.so_lse2 = pl.so_qtil = 0;
  pl.so_beta = pl.off_beta = pl.off_dqt = pl.off_dbt = 0;
  if (steps_state) {
    size_t so = 0;
    pl.so_cx = so;   so = align_up(so + rows * pl.D * pl.xc_elt);
    pl.so_h2 = so;   so = align_up(so + rows * 4);
    pl.so_lser = so; so = align_up(so + rows * 4);
    pl.so_lse2 = so; so = align_up(so + (size_t)pl.S * pl.G * 4);
    pl.so_qtil = so; so = align_up(so + rows * pl.D * 4);
    pl.so_beta = so; so = align_up(so + rows * 4);
    pl.step_bytes = so;
    pl.off_steps = off; off += (size_t)pl.T * so;
    const Plan last = step_plan(pl, pl.T - 1);   // the state the gradient kernels read first
    pl.off_cx = last.off_cx; pl.off_h2 = last.off_h2; pl.off_lser = last.off_lser;
    pl.off_lse2 = last.off_lse2; pl.off_qtil = last.off_qtil; pl.off_beta = last.off_beta;
  } else {
    pl.off_cx = off;   off = align_up(off + rows * pl.D * pl.xc_elt);
    pl.off_h2 = off;   off = align_up(off + rows * 4);
    pl.off_lser = off; off = align_up(off + rows * 4);
    pl.off_lse2 = off; off = align_up(off + (size_t)pl.S * pl.G * 4);
    pl.off_qtil = off; if (pl.need_qtil) off = align_up(off + rows * pl.D * 4);
  }
  pl.off_ux = off;   off = align_up(off + rows * pl.D * pl.elt);
  pl.off_qbar = off; if (pl.need_qbar) off = align_up(off + (size_t)pl.S * pl.c1 * pl.b2 * pl.D * 4);
  // tile means in bf16 for the copied-tile first step of the plain c path
  pl.off_qbar_lp = off;
  if (pl.need_qbar_lp) off = align_up(off + (size_t)pl.S * pl.c1 * pl.b2 * pl.D * pl.elt);
  pl.off_dq2 = pl.off_dcx = pl.off_dux = pl.off_dhx = pl.off_dkp = pl.off_dvp = pl.off_dlx = off;
  pl.off_dq2p = off;
  pl.dq2_parts = 0;
  pl.off_dqbar = off;
  if (backward) {
    pl.off_dq2 = off; off = align_up(off + (size_t)pl.S * pl.N * pl.D * 4);
    // stage-2 columns of several key chunks write one dQ part per chunk,
    // summed in chunk order (no atomics: the result does not depend on timing)
    const int nkeys = p->b1 * p->c2, nb = bwd_key_chunk(p);
    if (nkeys > nb) {
      pl.dq2_parts = (nkeys + nb - 1) / nb;
      pl.off_dq2p = off; off = align_up(off + (size_t)pl.dq2_parts * pl.S * pl.N * pl.D * 4);
    }
    pl.off_dcx = off; off = align_up(off + rows * pl.D * 4);
    pl.off_dux = off; off = align_up(off + rows * pl.D * 4);
    pl.off_dhx = off; off = align_up(off + rows * 4);
    pl.off_dlx = off; off = align_up(off + (size_t)pl.S * pl.G * 4);   // D of stage-2 rows
    if (pl.padded) { pl.off_dqbar = off; off = align_up(off + (size_t)pl.S * pl.b2 * pl.D * 4); }
    if (pl.group > 1 || steps_state) {   // per-query-head (and per-step summed) dK, dV in fp32
      pl.off_dkp = off; off = align_up(off + (size_t)pl.S * pl.N * pl.D * 4);
      pl.off_dvp = off; off = align_up(off + (size_t)pl.S * pl.N * pl.D * 4);
    }
    if (steps_state || tiled_bwd) { pl.off_dqt = off; off = align_up(off + rows * pl.D * 4); }
    if (steps_state) { pl.off_dbt = off; off = align_up(off + rows * 4); }
  }
  pl.total = off;
  return pl;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

// use_scratch: the workspace is the current device's scratch array (looked
// up after every other host check), not the caller's buffer
ma_status forward_impl(const ma_problem* p, const void* q, const void* k, const void* v, void* y,
                       const ma_exports* ex, void* workspace, size_t workspace_bytes, void* stream,
                       void* const* events, int32_t n_events, bool use_scratch = false) {
  ma_status s = validate_problem(p);
  if (s != MA_OK) return s;
  const Plan pl = make_plan(p);
  if (use_scratch) {
    // the cooperative launch's grid barrier keeps runtime-owned state
    if (pl.fused) return MA_ERR_UNSUPPORTED;
    if (pl.total > MONARCH_ATTN_SCRATCH_BYTES) return MA_ERR_WORKSPACE_TOO_SMALL;
    workspace_bytes = MONARCH_ATTN_SCRATCH_BYTES;
  }
  if (!q || !k || !v || !y) return MA_ERR_INVALID_ARGUMENT;
  auto misaligned = [](const void* x, uintptr_t a) { return ((uintptr_t)x % a) != 0; };
  if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(y, 16))
    return MA_ERR_INVALID_ARGUMENT;
  const size_t tbytes = (size_t)pl.S * pl.N * pl.D * pl.elt;
  const size_t kvbytes = tbytes / pl.group;
  if (overlaps(y, tbytes, q, tbytes) || overlaps(y, tbytes, k, kvbytes) || overlaps(y, tbytes, v, kvbytes))
    return MA_ERR_INVALID_ARGUMENT;
  if (ex) {
    if ((ex->L && misaligned(ex->L, 4)) || (ex->R && misaligned(ex->R, 4)) ||
        (ex->lse && misaligned(ex->lse, 4)) || (ex->objective && misaligned(ex->objective, 8)))
      return MA_ERR_INVALID_ARGUMENT;
  }
  if (n_events < 0) return MA_ERR_INVALID_ARGUMENT;
  if (use_scratch && (s = device_scratch(&workspace)) != MA_OK) return s;
  if (workspace_bytes < pl.total) return MA_ERR_WORKSPACE_TOO_SMALL;
  if (pl.total > 0) {
    if (!workspace || misaligned(workspace, ALIGN)) return MA_ERR_INVALID_ARGUMENT;
    if (overlaps(workspace, pl.total, q, tbytes) || overlaps(workspace, pl.total, k, kvbytes) ||
        overlaps(workspace, pl.total, v, kvbytes) || overlaps(workspace, pl.total, y, tbytes))
      return MA_ERR_INVALID_ARGUMENT;
  }
  Bufs b{q, k, v, y, static_cast<char*>(workspace), nullptr, nullptr, nullptr, nullptr};
  if (ex) { b.L = ex->L; b.R = ex->R; b.lse = ex->lse; b.obj = ex->objective; }
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (pl.dtype == MA_BF16) {
    if (pl.D == 64)
      return pl.precise ? run_bf16_64_precise(pl, b, st, events, n_events)
                        : run_bf16_64_fast(pl, b, st, events, n_events);
    return pl.precise ? run_bf16_128_precise(pl, b, st, events, n_events)
                      : run_bf16_128_fast(pl, b, st, events, n_events);
  }
  if (pl.D == 64) return run_f32_64(pl, b, st, events, n_events);
  return run_f32_128(pl, b, st, events, n_events);
}

// The backward covers stage-1 blocks whose keys fit LDS whole, any b1 (long
// stage-2 columns are walked in key chunks), grouped K/V, padding, and row
// tiles / key segments, at any T; bf16 at head_dim 128 with T > 1 keeps to
// 64-key blocks (its split c tiles).
ma_status validate_backward(const ma_problem* p) {
  const ma_status s = validate_problem(p);
  if (s != MA_OK) return s;
  const bool tiled = p->c1 != 1 || p->c2 != 1;
  if (p->b2 > bwd_max_block(p)) return MA_ERR_UNSUPPORTED;
  // bf16 at head_dim 128 with T > 1: its stage-1 blocks hold both c planes
  if (p->steps > 1 && p->dtype == MA_BF16 && p->head_dim == 128 && p->b2 > 64) return MA_ERR_UNSUPPORTED;
  return MA_OK;
}

ma_status backward_impl(const ma_problem* p, const void* q, const void* k, const void* v,
                        const void* y, const void* dy, void* dq, void* dk, void* dv, void* workspace,
                        size_t workspace_bytes, void* stream) {
  ma_status s = validate_backward(p);
  if (s != MA_OK) return s;
  const Plan pl = make_plan(p, true);
  if (pl.reuse_state) {     // the forward's state regions must be the backward's
    const Plan f = make_plan(p);
    if (pl.T != 1 || f.precise != pl.precise || f.off_cx != pl.off_cx || f.off_ux != pl.off_ux ||
        f.off_h2 != pl.off_h2 || f.off_lser != pl.off_lser || f.off_lse2 != pl.off_lse2 ||
        f.need_qbar != pl.need_qbar || f.off_qbar != pl.off_qbar ||
        f.need_qbar_lp != pl.need_qbar_lp || f.off_qbar_lp != pl.off_qbar_lp || f.xlo != pl.xlo)
      return MA_ERR_UNSUPPORTED;
  }
  const void* in[] = {q, k, v, dy};
  void* out[] = {dq, dk, dv};
  auto misaligned = [](const void* x, uintptr_t a) { return ((uintptr_t)x % a) != 0; };
  for (const void* x : in)
    if (!x || misaligned(x, 16)) return MA_ERR_INVALID_ARGUMENT;
  for (void* x : out)
    if (!x || misaligned(x, 16)) return MA_ERR_INVALID_ARGUMENT;
  if (y && misaligned(y, 16)) return MA_ERR_INVALID_ARGUMENT;
  const size_t tbytes = (size_t)pl.S * pl.N * pl.D * pl.elt;     // q, dy, dq
  const size_t kvbytes = tbytes / pl.group;                       // k, v, dk, dv
  const size_t isz[] = {tbytes, kvbytes, kvbytes, tbytes}, osz[] = {tbytes, kvbytes, kvbytes};
  for (int a = 0; a < 3; ++a) {
    for (int c = 0; c < 4; ++c)
      if (overlaps(out[a], osz[a], in[c], isz[c])) return MA_ERR_INVALID_ARGUMENT;
    if (y && overlaps(out[a], osz[a], y, tbytes)) return MA_ERR_INVALID_ARGUMENT;
    for (int c = a + 1; c < 3; ++c)
      if (overlaps(out[a], osz[a], out[c], osz[c])) return MA_ERR_INVALID_ARGUMENT;
  }
  if (workspace_bytes < pl.total) return MA_ERR_WORKSPACE_TOO_SMALL;
  if (!workspace || misaligned(workspace, ALIGN)) return MA_ERR_INVALID_ARGUMENT;
  for (int c = 0; c < 4; ++c)
    if (overlaps(workspace, pl.total, in[c], isz[c])) return MA_ERR_INVALID_ARGUMENT;
  for (int a = 0; a < 3; ++a)
    if (overlaps(workspace, pl.total, out[a], osz[a])) return MA_ERR_INVALID_ARGUMENT;
  if (y && overlaps(workspace, pl.total, y, tbytes)) return MA_ERR_INVALID_ARGUMENT;
  BwdBufs b{q, k, v, dy, dq, dk, dv, static_cast<char*>(workspace), y};
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (pl.dtype == MA_BF16)
    return pl.T > 1 ? (pl.D == 64 ? run_bwd_steps_bf16_64(pl, b, st) : run_bwd_steps_bf16_128(pl, b, st))
                    : pl.D == 64 ? run_bwd_bf16_64(pl, b, st) : run_bwd_bf16_128(pl, b, st);
  return pl.D == 64 ? run_bwd_f32_64(pl, b, st) : run_bwd_f32_128(pl, b, st);
}

}  // namespace

extern "C" {

ma_status monarch_attn_backward_workspace_size(const ma_problem* p, size_t* bytes) {
  if (!bytes) return MA_ERR_INVALID_ARGUMENT;
  const ma_status s = validate_backward(p);
  if (s != MA_OK) return s;
  *bytes = make_plan(p, true).total;
  return MA_OK;
}

ma_status monarch_attn_backward(const ma_problem* p, const void* q, const void* k, const void* v,
                                const void* y, const void* dy, void* dq, void* dk, void* dv,
                                void* workspace, size_t workspace_bytes, void* stream) {
  return backward_impl(p, q, k, v, y, dy, dq, dk, dv, workspace, workspace_bytes, stream);
}

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

ma_status monarch_attn_forward_noalloc(const ma_problem* p, const void* q, const void* k,
                                       const void* v, void* y, const ma_exports* exports,
                                       void* stream) {
  return forward_impl(p, q, k, v, y, exports, nullptr, 0, stream, nullptr, 0, true);
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
  if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return MA_ERR_DEVICE;
  *event = e;
  return MA_OK;
}

ma_status monarch_attn_event_destroy(void* event) {
  if (!event) return MA_ERR_INVALID_ARGUMENT;
  return hipEventDestroy((hipEvent_t)event) == hipSuccess ? MA_OK : MA_ERR_DEVICE;
}

ma_status monarch_attn_event_record(void* event, void* stream) {
  if (!event) return MA_ERR_INVALID_ARGUMENT;
  return hipEventRecord((hipEvent_t)event, (hipStream_t)stream) == hipSuccess ? MA_OK : MA_ERR_DEVICE;
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
