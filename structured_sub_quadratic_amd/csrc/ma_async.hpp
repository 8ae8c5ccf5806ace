// Stage kernels for bf16 whose LDS tiles are filled by direct global->LDS
// copies (global_load_lds, 16 bytes a lane) instead of register staging.
//
// Each persistent workgroup keeps two LDS buffers: while it computes on one,
// the copies of its next unit of work stream into the other, so the loads of
// a whole tile are in flight behind the arithmetic without holding any
// registers.  The two buffers are distinct LDS objects and the work loop is
// unrolled by two so that every access names its buffer statically: the
// compiler can then tell that the reads of one buffer do not depend on the
// copies in flight into the other and does not wait for them.  Tiles stay row-major (as they are in HBM); the 16-byte chunks
// of a row are XOR-swizzled by (row mod 8) so that the 16 rows an MFMA
// operand read touches fall in different banks.  The transposed value
// operand (V^T, K^T and U^T of the weighted sums) is read with the gfx950
// LDS transpose read ds_read_b64_tr_b16: within each 16-lane group, lane s
// addresses 4 elements of row s/4, and lane m receives element m%4 of the
// four rows read by lanes 4e + m/4 (e = 0..3), i.e. four consecutive keys of
// one head-dim column.
//
// Sources: MonarchAttention (scime summary "Approach": the steps are
// FlashAttention-like fused kernels over square-root-size blocks); the
// two-stage structure and the tiled variant follow MonarchRT ("Method").
#pragma once

#include <hip/hip_cooperative_groups.h>

#include "ma_stage_kernels.hpp"

namespace ma {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;

// Wait until every vector-memory operation of this wave has completed
// (direct-to-LDS copies included): vmcnt(0), other counters untouched.
__device__ inline void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }


// Copy 16 bytes at g into LDS at wave_base + 16 * lane (wave_base uniform).
//
// The copy is issued through inline assembly on purpose: the compiler then
// does not track it, so it cannot make LDS reads of the other buffer wait
// for it.  Ordering is explicit instead: every buffer is read only after
// wait_vmem() and a workgroup barrier, and refilled only after the next
// barrier.  The instruction writes no register; its address operands are
// read at issue.  M0 (the LDS base of the copy) is saved and restored
// around it; the nop covers the M0-write hazard of LDS-bound loads.
__device__ inline void copy16_to_lds(const void* g, void* wave_base) {
  // low 32 bits of a generic pointer into LDS = the LDS byte address
  const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)wave_base);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved) : "s"(lds), "v"(g) : "memory");
}

__device__ inline bf16x4 lds_read_tr4(const char* p) {
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)p);
  return __builtin_bit_cast(bf16x4, v);
}

// Row-major tile of bf16 rows of D elements with XOR-swizzled 16-byte chunks.
template <int D> struct SwzTile {
  static constexpr int RB = 2 * D;        // bytes per row
  static constexpr int CPR = D / 8;       // 16-byte chunks per row
  static_assert(CPR >= 8, "swizzle needs at least 8 chunks per row");
  __device__ static constexpr int offset(int row, int chunk) { return row * RB + ((chunk ^ (row & 7)) << 4); }

  // Fill rows [0, R) of the tile at lds from rowptr(r) (r clamped to
  // nvalid - 1), the NW waves of the workgroup sharing the copies.
  template <int R, int NW, class RowPtr>
  __device__ static inline void load(char* lds, RowPtr rowptr, int nvalid) {
    constexpr int NI = R * CPR / WAVE;    // wave-wide copies per tile
    static_assert((R * CPR) % WAVE == 0, "tile must be whole wave copies");
    const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE;
#pragma unroll 1
    for (int i0 = 0; i0 < NI; i0 += NW) {
      const int i = i0 + wave;
      if (NI % NW != 0 && i >= NI) break;
      const int slot = i * WAVE + lane;
      const int row = slot / CPR, cs = slot % CPR;
      const int c = cs ^ (row & 7);
      copy16_to_lds(rowptr(min(row, nvalid - 1)) + c * 8, lds + i * WAVE * 16);
    }
  }
};

// Score operand: key rows of swizzled tiles (hi, and lo when split).
template <int D> struct SwzKeys {
  typedef Mfma<bf16>::frag frag;
  static constexpr int NKS = D / 32;
  const char* hi;
  const char* lo;
  int off[NKS];       // this lane's byte offset in a 16-row sub-tile per k step
  __device__ inline SwzKeys(const char* h, const char* l) : hi(h), lo(l) {
    const int lane = threadIdx.x % WAVE, mrow = lane % 16, g = lane / 16;
#pragma unroll
    for (int k = 0; k < NKS; ++k) off[k] = SwzTile<D>::offset(mrow, 4 * k + g);
  }
  __device__ inline frag a(int mt, int ks_) const {
    return *reinterpret_cast<const frag*>(hi + mt * 16 * SwzTile<D>::RB + off[ks_]);
  }
  __device__ inline frag alo(int mt, int ks_) const {
    return *reinterpret_cast<const frag*>(lo + mt * 16 * SwzTile<D>::RB + off[ks_]);
  }
};

// Weighted-sum operand: the transposed value tiles.  Value sub-tiles
// dt < D/16 come from tile t0, the rest from t1 (stage 1 sums K and V).
template <int D> struct SwzValuesT {
  typedef Mfma<bf16>::frag frag;
  static constexpr int DPT = D / 16;      // value sub-tiles per tile
  const char* t0;
  const char* t1;
  int off[DPT];
  __device__ inline SwzValuesT(const char* a, const char* b) : t0(a), t1(b) {
    const int lane = threadIdx.x % WAVE, s = lane % 16, g = lane / 16;
    const int row = 4 * g + s / 4;        // key row read by this lane (mod 32)
#pragma unroll
    for (int dt = 0; dt < DPT; ++dt)
      off[dt] = SwzTile<D>::offset(row, 2 * dt + (s % 4) / 2) + 8 * (s % 2);
  }
  // keys {32kk+4g+r, 32kk+16+4g+r}, head-dim column 16*dt + lane%16
  __device__ inline frag at(int dt, int kk) const {
    const char* base = (dt < DPT ? t0 : t1) + kk * 32 * SwzTile<D>::RB + off[dt % DPT];
    const bf16x4 a = lds_read_tr4(base);
    const bf16x4 b = lds_read_tr4(base + 16 * SwzTile<D>::RB);
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  }
};

// A wave's 16-row output tile (accumulator layout: lane (q, g) holds
// elements 16*dt + 4*g .. +3 of row q) written to global memory as whole
// 16-byte row chunks through a per-wave LDS staging tile of 16 rows: lanes
// then cover complete rows, so each store instruction writes full lines
// instead of sixteen partial ones.  Ordering inside a wave needs no barrier.
template <int D> struct WaveRows {
  static constexpr int CPR = D / 8;          // 16-byte chunks per row
  static constexpr int RPI = WAVE / CPR;     // rows per store instruction
  static constexpr int BYTES = 16 * SwzTile<D>::RB;
  __device__ static inline void put(char* stg, const bf16x4 (&v)[D / 16]) {
    const int lane = threadIdx.x % WAVE, q = lane % 16, g = lane / 16;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
      *reinterpret_cast<bf16x4*>(stg + SwzTile<D>::offset(q, 2 * dt + g / 2) + 8 * (g % 2)) = v[dt];
  }
  // row(r) -> destination of row r (nullptr: skip)
  template <class RowPtr>
  __device__ static inline void drain(const char* stg, RowPtr row) {
    const int lane = threadIdx.x % WAVE, c = lane % CPR;
#pragma unroll
    for (int r0 = 0; r0 < 16; r0 += RPI) {
      const int r = r0 + lane / CPR;
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(stg + SwzTile<D>::offset(r, c));
      bf16* dst = row(r);
      if (dst) *reinterpret_cast<bf16x8*>(dst + c * 8) = v;
    }
  }
};

// Resident workgroups per CU of a kernel (cached) times the CU count.
template <class K>
inline size_t resident_slots(K kernel, int threads, size_t items) {
  static int per_cu = -1;
  if (per_cu < 0) {
    int v = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, kernel, threads, 0) != hipSuccess || v < 1) v = 1;
    per_cu = v;
  }
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    cus = 256;
  return std::max<size_t>(1, std::min<size_t>(items, (size_t)per_cu * cus));
}

// ---------------------------------------------------------------------------
// Stage 1 of the first step, whole block in one tile (b2 <= KTB).  The
// queries of block k are then bf16 rows: the rows (k, i) of Q (the same grid
// rows as its keys) and, when tiled, the tile means of the other row tiles
// kept in bf16 for the plain c path; they are copied into LDS with the keys
// and values.  Item = (slice, block k, query group of NW*16 slots
// t*b2 + i); NW waves of 16 queries each.  (Later steps and the split c path
// read fp32 query rows and use the register-staged kernels.)
// ---------------------------------------------------------------------------
template <int D, int NW, int KTB, bool WITH_U>
struct Stage1AsyncSmem {
  static constexpr int TILE = KTB * SwzTile<D>::RB;            // one K or V tile
  static constexpr int QOFF = (WITH_U ? 2 : 1) * TILE;         // query tile
  static constexpr int BUF = QOFF + NW * WaveRows<D>::BYTES;
};

// PAD: a padded flat sequence (padding positions clamped on load, padding
// keys masked, padding query positions read the tile means); the unpadded
// build keeps the plain row addressing.
// QF: a step after the first of an untiled, unpadded run; the queries are
// the fp32 next-step queries q~ (split into hi + lo when `split`), read from
// global memory into registers, and no query tile is copied.
template <int D, int NW, int KTB, bool WITH_U, bool PRECISE, bool PAD = false, bool QF = false>
struct Stage1Async {
  static constexpr int LDS_BYTES = 2 * Stage1AsyncSmem<D, NW, KTB, WITH_U>::BUF;

  __device__ static void run(const Stage1Params& p, char* lds) {
  typedef bf16 T;
  constexpr bool SPLITX = split_x<T, PRECISE>();
  constexpr int DV = WITH_U ? 2 * D : D;
  constexpr int QG = NW * 16;
  constexpr int NSPLIT = PRECISE ? D / 16 : 0;
  typedef FlashCore<T, D, DV, 1, KT, true, true, false, NSPLIT, QF> Core;
  typedef typename Core::frag frag;
  typedef Stage1AsyncSmem<D, NW, KTB, WITH_U> SM;
  char* const buf_a = lds;
  char* const buf_b = lds + SM::BUF;

  const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE, g = lane / 16;
  const int nitems = p.S * p.b1 * p.nqg;
  const int slot0 = wave * 16;            // this wave's first slot within a query group

  auto issue = [&](int item, char* b) {
    const int qg = item % p.nqg, k = (item / p.nqg) % p.b1, sl = item / (p.nqg * p.b1);
    const AxisMap am = p.map.template row_axis<PAD>(k);
    auto tok = [&](int r) -> int64_t { if constexpr (PAD) return am.at(r); else return am.raw(r); };
    const int kvs = kv_slice(sl, p.heads, p.group);
    const T* K = static_cast<const T*>(p.k) + (size_t)kvs * p.N * D;
    SwzTile<D>::template load<KTB, NW>(b, [&](int r) { return K + tok(r) * D; }, p.b2);
    if constexpr (WITH_U) {
      const T* V = static_cast<const T*>(p.v) + (size_t)kvs * p.N * D;
      SwzTile<D>::template load<KTB, NW>(b + SM::TILE, [&](int r) { return V + tok(r) * D; }, p.b2);
    }
    if constexpr (QF) return;     // queries come from q~ in global memory
    // slot = t*b2 + i: row (k, i) of Q in the own row tile t = k / rt, the
    // tile mean of (t, i) elsewhere (tiled first step) and at padding
    // positions (k, i)
    const T* Q = static_cast<const T*>(p.q) + (size_t)sl * p.N * D;
    const T* QB = p.qbar_lp ? static_cast<const T*>(p.qbar_lp) + (size_t)sl * p.c1 * p.b2 * D : Q;
    const int town = k / p.rt;
    SwzTile<D>::template load<QG, NW>(b + SM::QOFF, [&](int r) {
      const int slot = min(qg * QG + r, p.nqs - 1);
      const int t = slot / p.b2, i = slot - t * p.b2;
      if constexpr (PAD) return t == town && am.valid(i) ? Q + am.at(i) * D : QB + ((size_t)t * p.b2 + i) * D;
      else return t == town ? Q + am.raw(i) * D : QB + ((size_t)t * p.b2 + i) * D;
    }, QG);
  };

  Core core;

  // Outputs of one segment (c hi/lo, u, entropy, normaliser of this lane's
  // slot), held in registers until they are stored.  The last segment of an
  // item is stored only after the next item's copies have been issued, so
  // that the wait for those copies does not also wait for these stores.
  struct Out {
    bf16x4 c[D / 16], cl[SPLITX ? D / 16 : 1], u[WITH_U ? D / 16 : 1];
    float h2, lse;
    size_t xbase;       // exchange row of slot 0 of the item's query group
    int qg0;            // first slot of the query group
    bool any;
  };
  Out out;
  out.any = false;
  auto collect = [&](int qg, int k, int sl, int s) {
    float lse2[1], h2[1];
    core.finish(lse2, h2, p.sc2);
    out.xbase = x_row(p.b1, p.b2, p.c1, p.c2, sl, k, s, 0, 0);   // slot t*b2 + i -> xbase + slot
    out.qg0 = qg * QG;
    out.h2 = h2[0];
    out.lse = lse2[0];
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      const f32x4 v = core.o[0][dt];
      const bf16x4 h = __builtin_convertvector(v, bf16x4);
      out.c[dt] = h;
      if constexpr (SPLITX) out.cl[dt] = __builtin_convertvector(v - __builtin_convertvector(h, f32x4), bf16x4);
      if constexpr (WITH_U) out.u[dt] = __builtin_convertvector(core.o[0][D / 16 + dt], bf16x4);
    }
    out.any = true;
  };
  // stage: the wave's rows of the query tile of the current buffer, which
  // have been read into registers already
  auto flush = [&](char* cur) {
    if (!out.any) return;
    char* stg = cur + SM::QOFF + wave * WaveRows<D>::BYTES;
    auto rows = [&](T* base) {
      return [&, base](int r) -> T* {
        const int slot = out.qg0 + slot0 + r;
        return slot < p.nqs ? base + (out.xbase + slot) * D : nullptr;
      };
    };
    WaveRows<D>::put(stg, out.c);
    WaveRows<D>::drain(stg, rows(static_cast<T*>(p.cx)));
    if constexpr (SPLITX) {
      WaveRows<D>::put(stg, out.cl);
      WaveRows<D>::drain(stg, rows(static_cast<T*>(p.cx) + p.xlo));
    }
    if constexpr (WITH_U) {
      WaveRows<D>::put(stg, out.u);
      WaveRows<D>::drain(stg, rows(static_cast<T*>(p.ux)));
    }
    const int slot = out.qg0 + slot0 + lane % 16;
    if (g == 0 && slot < p.nqs) {
      p.h2x[out.xbase + slot] = out.h2;
      p.lser[out.xbase + slot] = out.lse;
    }
    out.any = false;
  };

  // item from buffer cur; the next item of this workgroup is copied into nxt
  auto step = [&](int item, char* cur, char* nxt) {
    const int qg = item % p.nqg, k = (item / p.nqg) % p.b1, sl = item / (p.nqg * p.b1);
    wait_vmem();
    __syncthreads();              // cur landed everywhere; nobody reads nxt any more
    if constexpr (QF) {
      core.load_queries([&](int) {
        const int slot = min(qg * QG + slot0 + lane % 16, p.nqs - 1);
        QSrc<T> r;
        r.t = nullptr;
        r.f = p.qtil + (((size_t)sl * p.b1 + k) * p.b2 + slot) * D;
        r.use_f = true;
        return r;
      }, Q_F32, PRECISE);
    } else {
#pragma unroll
      for (int ks_ = 0; ks_ < Core::NKS; ++ks_)
        core.qf[0][ks_] = *reinterpret_cast<const frag*>(
            cur + SM::QOFF + SwzTile<D>::offset(slot0 + lane % 16, 4 * ks_ + g));
    }
    if (item + (int)gridDim.x < nitems) issue(item + gridDim.x, nxt);
    flush(cur);                   // the previous item's last segment
    const char* vt = WITH_U ? cur + SM::TILE : cur;
    if constexpr (KTB == 2 * KT) {
      // (padded: blocks whose keys are all real)
      if (p.c2 == 1 && p.b2 == KTB && (!PAD || (p.map.key_lo(k) == 0 && p.map.key_hi(k) == KTB))) {
        // two full key tiles: both score products are issued before the
        // first softmax, so the second tile's MFMAs overlap the first
        // tile's exp and sums (the online-softmax updates keep their order)
        constexpr int OFF1 = KT * SwzTile<D>::RB;
        core.init();
        core.template scores_v<0>(SwzKeys<D>(cur, nullptr), 0, KT / 16);
        core.template scores_v<1>(SwzKeys<D>(cur + OFF1, nullptr), 0, KT / 16);
        core.template softmax_step<false, false, 0>(nullptr, p.sc2, 0, KT);
        core.template pv<false, 0>(SwzValuesT<D>(cur, vt), 0, KT);
        core.template softmax_step<false, false, 1>(nullptr, p.sc2, 0, KT);
        core.template pv<false, 1>(SwzValuesT<D>(cur + OFF1, vt + OFF1), 0, KT);
        collect(qg, k, sl, 0);
        return;
      }
    }
    for (int s = 0; s < p.c2; ++s) {
      int klo = s * p.sw, khi = klo + p.sw;
      if constexpr (PAD) {     // real keys of block k
        klo = max(klo, p.map.key_lo(k));
        khi = min(khi, p.map.key_hi(k));
      }
      core.init();
#pragma unroll 1
      for (int c0 = 0; c0 < KTB; c0 += KT) {
        if (c0 >= khi || c0 + KT <= klo) continue;
        const int lo = max(klo - c0, 0), hi = min(khi - c0, KT);
        const int off = c0 * SwzTile<D>::RB;
        core.scores_v(SwzKeys<D>(cur + off, nullptr), lo / 16, (hi + 15) / 16);
        const SwzValuesT<D> vv(cur + off, vt + off);
        if (lo == 0 && hi == KT) {
          core.template softmax_step<false, false>(nullptr, p.sc2, lo, hi);
          core.template pv<false>(vv, lo, hi);
        } else {
          core.template softmax_step<false, true>(nullptr, p.sc2, lo, hi);
          core.template pv<true>(vv, lo, hi);
        }
      }
      collect(qg, k, sl, s);
      if (s + 1 < p.c2) flush(cur);  // earlier segments: store now
    }
  };

  // Workgroup b takes items pos(b), pos(b) + G, ... where pos groups the
  // workgroups of one XCD on consecutive items.
  int item = (int)xcd_swizzle(blockIdx.x, gridDim.x);
  if (item >= nitems) return;
  issue(item, buf_a);
  char* last = buf_a;
  for (;;) {
    step(item, buf_a, buf_b);
    if ((item += gridDim.x) >= nitems) break;
    step(item, buf_b, buf_a);
    last = buf_b;
    if ((item += gridDim.x) >= nitems) break;
    last = buf_a;
  }
  flush(last);
  }
};

template <int D, int NW, int KTB, bool WITH_U, bool PRECISE, bool PAD = false, bool QF = false>
__global__ __launch_bounds__(NW * WAVE) void stage1_async_kernel(Stage1Params p) {
  typedef Stage1Async<D, NW, KTB, WITH_U, PRECISE, PAD, QF> S;
  __shared__ __attribute__((aligned(1024))) char lds[S::LDS_BYTES];
  S::run(p, lds);
}

// ---------------------------------------------------------------------------
// Stage 2.  Item = (slice, column i, row tile t, query group of NW*NQ*16
// rows); its b1*c2 keys are streamed in chunks of KT.  A workgroup walks the
// flat sequence of (item, chunk) units of its items, copying unit u+1 into
// the other buffer while unit u computes.
// ---------------------------------------------------------------------------
template <int D, bool KLO, bool WITH_PV, int KC>
struct Stage2AsyncSmem {
  static constexpr int TILE = KC * SwzTile<D>::RB;
  static constexpr int HI = 0;
  static constexpr int LO = TILE;
  static constexpr int U = (KLO ? 2 : 1) * TILE;
  static constexpr int BUF = U + (WITH_PV ? TILE : 0);
};

// PAD: a padded flat sequence (no output at padding positions).
template <int D, int NW, int NQ, bool WITH_PV, bool PRECISE, int KC = KT, bool PAD = false>
struct Stage2Async {
  typedef Stage2AsyncSmem<D, split_x<bf16, PRECISE>(), WITH_PV, KC> SM0;
  static constexpr int STG = WITH_PV ? NW * WaveRows<D>::BYTES : 0;
  static constexpr int LDS_BYTES = 2 * SM0::BUF + STG + 2 * KC * 4;

  __device__ static void run(const Stage2Params& p, char* lds) {
  typedef bf16 T;
  constexpr bool KLO = split_x<T, PRECISE>();
  constexpr int QG = NW * NQ * 16;
  typedef FlashCore<T, D, D, NQ, KC, false, WITH_PV, KLO, 0> Core;
  typedef typename Core::frag frag;
  typedef Stage2AsyncSmem<D, KLO, WITH_PV, KC> SM;
  char* const buf_a = lds;
  char* const buf_b = lds + SM::BUF;
  char* const stage_rows = lds + 2 * SM::BUF;
  float* const bias_a = reinterpret_cast<float*>(lds + 2 * SM::BUF + STG);
  float* const bias_b = bias_a + KC;

  const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE, g = lane / 16;
  const int nitems = p.S * p.b2 * p.c1 * p.nqg;
  const int nch = (p.nkeys + KC - 1) / KC;
  auto decode = [&](int item, int& sl, int& i, int& t, int& qg) {
    qg = item % p.nqg; item /= p.nqg;
    t = item % p.c1; item /= p.c1;
    i = item % p.b2;
    sl = item / p.b2;
  };
  auto row_of = [&](int qg, int n) { return qg * QG + wave * NQ * 16 + n * 16 + lane % 16; };

  frag qn[NQ][Core::NKS];
  typename Core::QLo qnl;
  float hn[KC / WAVE];          // bias of the unit in flight (last wave, KC/64 keys a lane)
  auto issue = [&](int item, int ch, char* b) {
    int sl, i, t, qg;
    decode(item, sl, i, t, qg);
    const size_t xs = x_stride(p.b2, p.c1);
    const size_t base = x_base(p.b1, p.b2, p.c1, p.c2, sl, t, i) + (size_t)ch * KC * xs;
    const int nvalid = min(KC, p.nkeys - ch * KC);
    const T* C = static_cast<const T*>(p.cx) + base * D;
    SwzTile<D>::template load<KC, NW>(b + SM::HI, [&](int r) { return C + (size_t)r * xs * D; }, nvalid);
    if constexpr (KLO)
      SwzTile<D>::template load<KC, NW>(b + SM::LO, [&](int r) { return C + p.xlo + (size_t)r * xs * D; }, nvalid);
    if constexpr (WITH_PV) {
      const T* U = static_cast<const T*>(p.ux) + base * D;
      SwzTile<D>::template load<KC, NW>(b + SM::U, [&](int r) { return U + (size_t)r * xs * D; }, nvalid);
    }
    if (wave == NW - 1) {
#pragma unroll
      for (int j = 0; j < KC / WAVE; ++j) hn[j] = p.h2x[base + (size_t)min(lane + WAVE * j, nvalid - 1) * xs];
    }
    if (ch == 0)
      Core::fetch_queries([&](int n) { return stage2_qsrc<T, D, PAD>(p, sl, i, t, row_of(qg, n)); },
                          Q_INPUT, qn, qnl);
  };

  // Workgroup b takes items pos(b), pos(b) + G, ... where pos groups the
  // workgroups of one XCD on consecutive items, so the query groups of one
  // column (consecutive items) read their shared key tiles through one L2.
  int item = (int)xcd_swizzle(blockIdx.x, gridDim.x);
  if (item >= nitems) return;
  int ch = 0;
  issue(item, 0, buf_a);
  Core core;

  // Outputs of an item (y rows and normalisers of this lane's queries),
  // stored after the next unit's copies are issued.
  struct Out {
    bf16x4 y[NQ][WITH_PV ? D / 16 : 1];
    float lse[NQ];
    int64_t tok[NQ];
    int l[NQ];
    bool valid[NQ];
    int sl, i;
    int l0, lend;       // grid rows of this wave's first query and of the row tile's end
    bool any;
  };
  Out out;
  out.any = false;
  char* stg = stage_rows + (WITH_PV ? wave * WaveRows<D>::BYTES : 0);
  auto flush = [&]() {
    if (!out.any) return;
    T* Y = static_cast<T*>(p.y) + (size_t)out.sl * p.N * D;
    if constexpr (WITH_PV) {
      const AxisMap am = p.map.template col_axis<PAD>(out.i);
#pragma unroll
      for (int n = 0; n < NQ; ++n) {
        WaveRows<D>::put(stg, out.y[n]);
        WaveRows<D>::drain(stg, [&](int r) -> T* {
          const int l = out.l0 + n * 16 + r;
          if constexpr (PAD) return l < out.lend && am.valid(l) ? Y + am.at(l) * D : nullptr;
          else return l < out.lend ? Y + am.raw(l) * D : nullptr;
        });
      }
    }
#pragma unroll
    for (int n = 0; n < NQ; ++n) {
      if (!out.valid[n]) continue;
      if (g == 0) {
        p.lse2[((size_t)out.sl * p.b2 + out.i) * p.b1 + out.l[n]] = out.lse[n];
        if (p.lse_out && (!PAD || out.tok[n] >= 0)) p.lse_out[(size_t)out.sl * p.N + out.tok[n]] = out.lse[n] * LN2;
      }
    }
    out.any = false;
  };
  // unit (item, ch) from buffer cur; the next unit is copied into nxt.
  // Returns false after the last unit of this workgroup.
  auto unit = [&](const char* cur, float* bias, char* nxt) -> bool {
    wait_vmem();
    if (wave == NW - 1) {
#pragma unroll
      for (int j = 0; j < KC / WAVE; ++j) bias[lane + WAVE * j] = hn[j];
    }
    __syncthreads();              // cur landed everywhere; nobody reads nxt any more
    if (ch == 0) {
      core.init();
      core.set_queries(qn, qnl);
    }
    int nitem = item, nchk = ch + 1;
    if (nchk == nch) { nitem = item + gridDim.x; nchk = 0; }
    if (nitem < nitems) issue(nitem, nchk, nxt);
    flush();

    const int nvalid = min(KC, p.nkeys - ch * KC);
    core.scores_v(SwzKeys<D>(cur + SM::HI, cur + SM::LO), 0, Core::MT);
    if (nvalid == KC) core.template softmax_step<true, false>(bias, p.sc2, 0, nvalid);
    else core.template softmax_step<true, true>(bias, p.sc2, 0, nvalid);
    if constexpr (WITH_PV) {
      const SwzValuesT<D> vv(cur + SM::U, cur + SM::U);
      if (nvalid == KC) core.template pv<false>(vv, 0, nvalid);
      else core.template pv<true>(vv, 0, nvalid);
    }
    if (ch == nch - 1) {
      int sl, i, t, qg;
      decode(item, sl, i, t, qg);
      float lse2[NQ], h2[NQ];
      core.finish(lse2, h2, p.sc2);
      const AxisMap am = p.map.template col_axis<PAD>(i);
      out.sl = sl;
      out.i = i;
      out.l0 = t * p.rt + row_of(qg, 0) - lane % 16;
      out.lend = t * p.rt + p.rt;
#pragma unroll
      for (int n = 0; n < NQ; ++n) {
        const int ll = row_of(qg, n);
        out.valid[n] = ll < p.rt;
        out.l[n] = t * p.rt + min(ll, p.rt - 1);
        if constexpr (PAD) out.tok[n] = am.valid(out.l[n]) ? am.at(out.l[n]) : -1;   // -1: padding row
        else out.tok[n] = am.raw(out.l[n]);
        out.lse[n] = lse2[n];
        if constexpr (WITH_PV) {
#pragma unroll
          for (int dt = 0; dt < D / 16; ++dt) out.y[n][dt] = __builtin_convertvector(core.o[n][dt], bf16x4);
        }
      }
      out.any = true;
    }
    if (nitem >= nitems) return false;
    item = nitem;
    ch = nchk;
    return true;
  };
  while (unit(buf_a, bias_a, buf_b) && unit(buf_b, bias_b, buf_a)) {
  }
  flush();
  }
};

template <int D, int NW, int NQ, bool WITH_PV, bool PRECISE, int KC = KT, bool PAD = false>
__global__ __launch_bounds__(NW * WAVE) void stage2_async_kernel(Stage2Params p) {
  typedef Stage2Async<D, NW, NQ, WITH_PV, PRECISE, KC, PAD> S;
  __shared__ __attribute__((aligned(1024))) char lds[S::LDS_BYTES];
  S::run(p, lds);
}

// ---------------------------------------------------------------------------
// Fused single launch for T = 1 (untiled): stage 1 over every block, a
// grid-wide barrier, stage 2 over every column, in one cooperative launch of
// resident persistent workgroups.  Removes the launch gap between the stages;
// the exchange written by phase 1 is read by phase 2 while it is still warm
// in the Infinity Cache.  Both phases use NW waves per workgroup.
// ---------------------------------------------------------------------------
template <int D, int NW, int KTB, bool PRECISE>
__global__ __launch_bounds__(NW * WAVE) void fused_async_kernel(Stage1Params p1, Stage2Params p2) {
  typedef Stage1Async<D, NW, KTB, true, PRECISE> S1;
  typedef Stage2Async<D, NW, 1, true, PRECISE> S2;
  constexpr int BYTES = S1::LDS_BYTES > S2::LDS_BYTES ? S1::LDS_BYTES : S2::LDS_BYTES;
  __shared__ __attribute__((aligned(1024))) char lds[BYTES];
  S1::run(p1, lds);
  __syncthreads();
  cooperative_groups::this_grid().sync();
  S2::run(p2, lds);
}

}  // namespace ma
