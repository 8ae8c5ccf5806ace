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

#include <map>
#include <mutex>
#include <utility>

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

// N (2 or 4) such copies of one wave in a row: g[j] -> LDS byte address
// lds[j] (uniform), M0 saved once.  Same ordering contract as above.
__device__ inline void copy16x2_to_lds(const void* g0, const void* g1, uint32_t l0, uint32_t l1) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %3, off\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %4, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved) : "s"(l0), "s"(l1), "v"(g0), "v"(g1) : "memory");
}
__device__ inline void copy16x4_to_lds(const void* g0, const void* g1, const void* g2, const void* g3,
                                       uint32_t l0, uint32_t l1, uint32_t l2, uint32_t l3) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %5, off\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %6, off\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %7, off\n\t"
      "s_mov_b32 m0, %4\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %8, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved) : "s"(l0), "s"(l1), "s"(l2), "s"(l3), "v"(g0), "v"(g1), "v"(g2), "v"(g3) : "memory");
}

__device__ inline bf16x4 lds_read_tr4(const char* p) {
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)p);
  return __builtin_bit_cast(bf16x4, v);
}

// Row-major tile of bf16 rows of D elements with XOR-swizzled 16-byte chunks:
// chunk c of row r sits at chunk c ^ swz(r).  The score operand reads one
// chunk from each of 16 consecutive rows, and the transposed value read two
// adjacent chunks (32 bytes) from each of 8 consecutive rows.  64-element
// rows (128 bytes) take r mod 8.  128-element rows (256 bytes, so every row
// starts on the same LDS bank) take 2 (r mod 8) + bit 3 of r: with r mod 8,
// rows 2j and 2j + 1 put their chunk pair on the same banks, which the
// bank-conflict counters showed in about half of the LDS cycles of the
// head_dim-128 kernels; the doubled index gives each of 8 rows a pair of
// its own and keeps 16 rows on 16 distinct chunks.
template <int D> struct SwzTile {
  static constexpr int RB = 2 * D;        // bytes per row
  static constexpr int CPR = D / 8;       // 16-byte chunks per row
  static_assert(CPR == 8 || CPR == 16, "swizzle for rows of 64 or 128 elements");
  __host__ __device__ static constexpr int swz(int row) {
    return CPR == 8 ? (row & 7) : (((row & 7) << 1) | ((row >> 3) & 1));
  }
  __device__ static constexpr int offset(int row, int chunk) { return row * RB + ((chunk ^ swz(row)) << 4); }

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
      const int c = cs ^ swz(row);
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

// Lanes of one wave exchanging data through LDS: the hardware runs a wave's
// LDS instructions in order, but the compiler reasons per lane and may
// reuse an earlier read of an address that this lane did not write in
// between (another lane's write is invisible to it without
// synchronisation).  A wavefront-scope release, a scheduling barrier and an
// acquire make the other lanes' writes visible and keep the accesses in
// program order.
__device__ inline void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// A wave's 16-row output tile (accumulator layout: lane (q, g) holds
// elements 16*dt + 4*g .. +3 of row q) written to global memory as whole
// 16-byte row chunks through a per-wave LDS staging tile of 16 rows: lanes
// then cover complete rows, so each store instruction writes full lines
// instead of sixteen partial ones.  The lanes meet at wave_sync() before
// the tile is written (the previous drain's reads are done) and before it
// is read.
template <int D> struct WaveRows {
  static constexpr int CPR = D / 8;          // 16-byte chunks per row
  static constexpr int RPI = WAVE / CPR;     // rows per store instruction
  static constexpr int BYTES = 16 * SwzTile<D>::RB;
  __device__ static inline void put(char* stg, const bf16x4 (&v)[D / 16]) {
    const int lane = threadIdx.x % WAVE, q = lane % 16, g = lane / 16;
    wave_sync();
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
      *reinterpret_cast<bf16x4*>(stg + SwzTile<D>::offset(q, 2 * dt + g / 2) + 8 * (g % 2)) = v[dt];
  }
  // row(r) -> destination of row r (nullptr: skip)
  template <class RowPtr>
  __device__ static inline void drain(const char* stg, RowPtr row) {
    const int lane = threadIdx.x % WAVE, c = lane % CPR;
    wave_sync();
#pragma unroll
    for (int r0 = 0; r0 < 16; r0 += RPI) {
      const int r = r0 + lane / CPR;
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(stg + SwzTile<D>::offset(r, c));
      bf16* dst = row(r);
      if (dst) *reinterpret_cast<bf16x8*>(dst + c * 8) = v;
    }
  }
};

// Resident workgroups per CU of a kernel on a device, cached per (kernel
// address, device): every instantiation of a kernel template has its own
// register and LDS footprint.
inline int cached_occupancy(const void* kernel, int dev, int threads) {
  static std::mutex mu;
  static std::map<std::pair<const void*, int>, int> cache;
  std::lock_guard<std::mutex> lock(mu);
  const auto key = std::make_pair(kernel, dev);
  const auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int v = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, kernel, threads, 0) != hipSuccess || v < 1) v = 1;
  cache.emplace(key, v);
  return v;
}

// Resident workgroups per CU of a kernel times the CU count, at most items.
template <class K>
inline size_t resident_slots(K kernel, int threads, size_t items) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    cus = 256;
  const int per_cu = cached_occupancy(reinterpret_cast<const void*>(kernel), dev, threads);
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
// FULL: every block fills the key tiles in one segment (b2 = KTB, c2 = 1,
// unpadded); the build holds that path only, whose one update per tile keeps
// the accumulators in place.
template <int D, int NW, int KTB, bool WITH_U, bool PRECISE, bool PAD = false, bool QF = false,
          bool FULL = false>
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

  // An item (slice, block k, query group qg), decoded once when its copies
  // are issued and handed to the step that computes it.
  struct It {
    int item, qg, k, sl;
  };
  auto decode = [&](int item) {
    It r;
    r.item = item;
    r.qg = item % p.nqg;
    const int q = item / p.nqg;
    r.k = q % p.b1;
    r.sl = q / p.b1;
    return r;
  };
  auto issue = [&](const It& it, char* b) {
    const int qg = it.qg, k = it.k, sl = it.sl;
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
    if (p.c1 == 1 && !PAD) {        // one row tile: slot i is row (k, i) of Q
      SwzTile<D>::template load<QG, NW>(b + SM::QOFF, [&](int r) {
        return Q + am.raw(min(qg * QG + r, p.nqs - 1)) * D;
      }, QG);
      return;
    }
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
  auto step = [&](const It& it, char* cur, char* nxt, It& next) {
    const int item = it.item, qg = it.qg, k = it.k, sl = it.sl;
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
    next.item = item + (int)gridDim.x;
    if (next.item < nitems) {
      next = decode(next.item);
      issue(next, nxt);
    }
    flush(cur);                   // the previous item's last segment
    const char* vt = WITH_U ? cur + SM::TILE : cur;
    if constexpr (KTB == 2 * KT) {
      // (padded: blocks whose keys are all real)
      if (FULL || (p.c2 == 1 && p.b2 == KTB && (!PAD || (p.map.key_lo(k) == 0 && p.map.key_hi(k) == KTB)))) {
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
    } else if constexpr (FULL) {
      core.init();
      core.scores_v(SwzKeys<D>(cur, nullptr), 0, KT / 16);
      core.template softmax_step<false, false>(nullptr, p.sc2, 0, KT);
      core.template pv<false>(SwzValuesT<D>(cur, vt), 0, KT);
      collect(qg, k, sl, 0);
      return;
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
  const int item0 = (int)xcd_swizzle(blockIdx.x, gridDim.x);
  if (item0 >= nitems) return;
  It ia = decode(item0), ib;
  issue(ia, buf_a);
  char* last = buf_a;
  for (;;) {
    step(ia, buf_a, buf_b, ib);
    if (ib.item >= nitems) break;
    step(ib, buf_b, buf_a, ia);
    last = buf_b;
    if (ia.item >= nitems) break;
    last = buf_a;
  }
  flush(last);
  }
};

template <int D, int NW, int KTB, bool WITH_U, bool PRECISE, bool PAD = false, bool QF = false,
          bool FULL = false>
__global__ __launch_bounds__(NW * WAVE) void stage1_async_kernel(Stage1Params p) {
  static_assert(!FULL || !PAD, "whole tiles: unpadded");
  typedef Stage1Async<D, NW, KTB, WITH_U, PRECISE, PAD, QF, FULL> S;
  __shared__ __attribute__((aligned(1024))) char lds[S::LDS_BYTES];
  S::run(p, lds);
}

// ---------------------------------------------------------------------------
// Stage 1 of a single step (u as well) for blocks of at most 64 keys at
// head_dim 128 (the video latent's 52-key blocks), first step on the plain c
// path, unpadded, with or without row tiles and key segments.  Four waves
// take 64 query slots (t, i) of a block k -- row (k, i) of Q on k's own row
// tile, the bf16 tile mean of (t, i) elsewhere -- and the K and V tiles of
// the next item stream into the other of two LDS buffers; each wave reads its
// query rows of the next item straight into registers.  Per key segment the
// weighted sums c = R K and u = R V run one after the other on the same
// probabilities, so only one 128-wide accumulator is live and two workgroups
// share a CU (two waves a SIMD).
// ---------------------------------------------------------------------------
template <int D>
struct Stage1SmallSmem {
  static constexpr int TILE = KT * SwzTile<D>::RB;       // one K or V tile (64 rows)
  static constexpr int BUF = 2 * TILE;
  static constexpr int LDS_BYTES = 2 * BUF + 4 * WaveRows<D>::BYTES;
};

template <int D>
__global__ __launch_bounds__(4 * WAVE, 2) void stage1_small_kernel(Stage1Params p) {
  typedef bf16 T;
  constexpr int NW = 4, QG = NW * 16;
  typedef FlashCore<T, D, D, 1, KT, true, true, false, 0> Core;
  typedef typename Core::frag frag;
  typedef Stage1SmallSmem<D> SM;
  __shared__ __attribute__((aligned(1024))) char lds[SM::LDS_BYTES];
  char* const buf_a = lds;
  char* const buf_b = lds + SM::BUF;
  const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE, g = lane / 16;
  char* const stg = lds + 2 * SM::BUF + wave * WaveRows<D>::BYTES;
  const int nitems = p.S * p.b1 * p.nqg;
  const int slot0 = wave * 16;                    // this wave's first slot within a query group
  struct It {
    int item, qg, k, sl;
  };
  auto decode = [&](int item) {
    It r;
    r.item = item;
    r.qg = item % p.nqg;
    const int q = item / p.nqg;
    r.k = q % p.b1;
    r.sl = q / p.b1;
    return r;
  };
  frag qn[Core::NKS];
  auto issue = [&](const It& it, char* b) {
    const AxisMap am = p.map.template row_axis<false>(it.k);
    const int kvs = kv_slice(it.sl, p.heads, p.group);
    const T* K = static_cast<const T*>(p.k) + (size_t)kvs * p.N * D;
    const T* V = static_cast<const T*>(p.v) + (size_t)kvs * p.N * D;
    SwzTile<D>::template load<KT, NW>(b, [&](int r) { return K + am.raw(r) * D; }, p.b2);
    SwzTile<D>::template load<KT, NW>(b + SM::TILE, [&](int r) { return V + am.raw(r) * D; }, p.b2);
    // slot (t, i): row (k, i) of Q on the own row tile, the tile mean of (t, i) elsewhere
    const int q = min(it.qg * QG + slot0 + lane % 16, p.nqs - 1);
    const int t = p.c1 == 1 ? 0 : q / p.b2, i = q - t * p.b2;
    const T* src = t == it.k / p.rt
        ? static_cast<const T*>(p.q) + ((size_t)it.sl * p.N + am.raw(i)) * D
        : static_cast<const T*>(p.qbar_lp) + ((size_t)it.sl * p.c1 * p.b2 + q) * D;
#pragma unroll
    for (int ks_ = 0; ks_ < Core::NKS; ++ks_) qn[ks_] = *reinterpret_cast<const frag*>(src + ks_ * 32 + g * 8);
  };
  Core core;
  // rows of the wave's 16 queries (o normalised) to exchange rows xb + slot
  auto store_rows = [&](T* x, size_t xb, int qg0) {
    bf16x4 v[D / 16];
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) v[dt] = __builtin_convertvector(core.o[0][dt], bf16x4);
    WaveRows<D>::put(stg, v);
    WaveRows<D>::drain(stg, [&](int r) -> T* {
      const int q = qg0 + slot0 + r;
      return q < p.nqs ? x + (xb + q) * D : nullptr;
    });
  };
  auto step = [&](const It& it, const char* cur, char* nxt, It& next) {
    wait_vmem();
    __syncthreads();              // cur landed everywhere; nobody reads nxt any more
#pragma unroll
    for (int ks_ = 0; ks_ < Core::NKS; ++ks_) core.qf[0][ks_] = qn[ks_];
    next.item = it.item + (int)gridDim.x;
    if (next.item < nitems) {
      next = decode(next.item);
      issue(next, nxt);
    }
    const int qg0 = it.qg * QG, q = qg0 + slot0 + lane % 16;
    const char* vt = cur + SM::TILE;
    for (int s = 0; s < p.c2; ++s) {
      const int klo = s * p.sw, khi = klo + p.sw;
      // (the masked path for every segment, whole tiles included: one code
      // path keeps the accumulators in place)
      core.init();
      core.scores_v(SwzKeys<D>(cur, nullptr), klo / 16, (khi + 15) / 16);
      core.template softmax_step<false, true>(nullptr, p.sc2, klo, khi);
      // c = R K
      core.template pv<true>(SwzValuesT<D>(cur, cur), klo, khi);
      float lse2[1], h2[1];
      core.finish(lse2, h2, p.sc2);
      const size_t xb = x_row(p.b1, p.b2, p.c1, p.c2, it.sl, it.k, s, 0, 0);   // slot t*b2 + i -> xb + slot
      store_rows(static_cast<T*>(p.cx), xb, qg0);
      if (g == 0 && q < p.nqs) {
        p.h2x[xb + q] = h2[0];
        p.lser[xb + q] = lse2[0];
      }
      // u = R V on the same probabilities
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) core.o[0][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
      core.template pv<true>(SwzValuesT<D>(vt, vt), klo, khi);
      const float inv = 1.f / wave_sum_x16x32(core.l[0]);
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) core.o[0][dt] *= inv;
      store_rows(static_cast<T*>(p.ux), xb, qg0);
    }
  };
  const int item0 = (int)xcd_swizzle(blockIdx.x, gridDim.x);
  if (item0 >= nitems) return;
  It ia = decode(item0), ib;
  issue(ia, buf_a);
  for (;;) {
    step(ia, buf_a, buf_b, ib);
    if (ib.item >= nitems) break;
    step(ib, buf_b, buf_a, ia);
    if (ia.item >= nitems) break;
  }
}

// ---------------------------------------------------------------------------
// Stage 1 of a single step (u as well) for blocks of 65-128 keys at
// head_dim 64 (the 128 x 128 grid of a 16K sequence), unpadded, one row tile
// and one segment.  Eight waves take the (up to) 128 query rows of block k;
// the block's K and V rows (two 64-key tiles each) of the next item stream
// into the other of two LDS buffers and each wave reads its query rows of
// the next item straight into registers.  All 128 scores of a row are held
// at once, so the softmax takes the row maximum over the whole block in one
// pass; then c = R K and u = R V run one after the other on the same
// probabilities with one 64-wide accumulator.  80 KB of LDS and at most 128
// registers a lane: two workgroups share a CU, four waves a SIMD.
// ---------------------------------------------------------------------------
// PAD: a padded flat sequence (padding positions clamped on load, the keys
// outside the block's real range masked, padding query slots read the bf16
// column means).
template <int D, bool PAD = false>
struct Stage1Pair {
  static constexpr int NW = 8, QG = NW * 16;
  static constexpr int HALF = KT * SwzTile<D>::RB;        // one 64-row tile
  static constexpr int TILE = 2 * HALF;                   // the K or V rows of a block
  static constexpr int BUF = 2 * TILE;
  static constexpr int LDS_BYTES = 2 * BUF + NW * WaveRows<D>::BYTES;

  // the launches this body serves
  __host__ __device__ static bool serves(int b2, int c1, int c2, bool padded) {
    return b2 > KT && b2 <= 2 * KT && c1 == 1 && c2 == 1 && padded == PAD;
  }

  __device__ static void run(const Stage1Params& p, char* lds) {
    typedef bf16 T;
    typedef FlashCore<T, D, D, 1, KT, true, true, false, 0> Core;
    typedef typename Core::frag frag;
    char* const buf_a = lds;
    char* const buf_b = lds + BUF;
    const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE, g = lane / 16;
    char* const stg = lds + 2 * BUF + wave * WaveRows<D>::BYTES;
    const int nitems = p.S * p.b1 * p.nqg;
    const int slot0 = wave * 16;
    struct It {
      int item, qg, k, sl;
    };
    auto decode = [&](int item) {
      It r;
      r.item = item;
      r.qg = item % p.nqg;
      const int q = item / p.nqg;
      r.k = q % p.b1;
      r.sl = q / p.b1;
      return r;
    };
    frag qn[Core::NKS];
    auto issue = [&](const It& it, char* b) {
      const AxisMap am = p.map.template row_axis<PAD>(it.k);
      auto tok = [&](int r) -> int64_t { if constexpr (PAD) return am.at(r); else return am.raw(r); };
      const int kvs = kv_slice(it.sl, p.heads, p.group);
      const T* K = static_cast<const T*>(p.k) + (size_t)kvs * p.N * D;
      const T* V = static_cast<const T*>(p.v) + (size_t)kvs * p.N * D;
      SwzTile<D>::template load<2 * KT, NW>(b, [&](int r) { return K + tok(r) * D; }, p.b2);
      SwzTile<D>::template load<2 * KT, NW>(b + TILE, [&](int r) { return V + tok(r) * D; }, p.b2);
      const int i = min(it.qg * QG + slot0 + lane % 16, p.nqs - 1);
      const T* src;
      if constexpr (PAD) {
        // a padding slot (k, i) takes the mean of the real rows of column i
        src = am.valid(i) ? static_cast<const T*>(p.q) + ((size_t)it.sl * p.N + am.at(i)) * D
                          : static_cast<const T*>(p.qbar_lp) + ((size_t)it.sl * p.b2 + i) * D;
      } else {
        src = static_cast<const T*>(p.q) + ((size_t)it.sl * p.N + am.raw(i)) * D;
      }
#pragma unroll
      for (int ks_ = 0; ks_ < Core::NKS; ++ks_) qn[ks_] = *reinterpret_cast<const frag*>(src + ks_ * 32 + g * 8);
    };
    Core core;
    auto store_rows = [&](T* x, size_t xb, int qg0) {
      bf16x4 v[D / 16];
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) v[dt] = __builtin_convertvector(core.o[0][dt], bf16x4);
      WaveRows<D>::put(stg, v);
      WaveRows<D>::drain(stg, [&](int r) -> T* {
        const int q = qg0 + slot0 + r;
        return q < p.nqs ? x + (xb + q) * D : nullptr;
      });
    };
    auto step = [&](const It& it, const char* cur, char* nxt, It& next) {
      wait_vmem();
      __syncthreads();              // cur landed everywhere; nobody reads nxt any more
#pragma unroll
      for (int ks_ = 0; ks_ < Core::NKS; ++ks_) core.qf[0][ks_] = qn[ks_];
      next.item = it.item + (int)gridDim.x;
      if (next.item < nitems) {
        next = decode(next.item);
        issue(next, nxt);
      }
      const int qg0 = it.qg * QG, q = qg0 + slot0 + lane % 16;
      core.template scores_v<0>(SwzKeys<D>(cur, nullptr), 0, Core::MT);
      core.template scores_v<1>(SwzKeys<D>(cur + HALF, nullptr), 0, Core::MT);
      // softmax over the block: keys 16 mt + 4 g + r of each tile; keys past
      // b2 (second tile) masked, and with padding the keys outside the
      // block's real range [klo, khi)
      {
        constexpr float MASKED = -1e30f;
        if constexpr (PAD) {
          // only the block holding padding positions masks keys here (a
          // pass of its own, so the other blocks run the unpadded code)
          const int klo = p.map.key_lo(it.k), khi = min(p.map.key_hi(it.k), p.b2);
          if (klo > 0 || khi < p.b2) {
#pragma unroll
            for (int mt = 0; mt < Core::MT; ++mt)
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const int key0 = mt * 16 + 4 * g + r, key1 = KT + key0;
                if (key0 < klo || key0 >= khi) core.s[0][mt][r] = MASKED;
                if (key1 < klo || key1 >= khi) core.s2[0][mt][r] = MASKED;
              }
          }
        }
        float zs[8 * Core::MT];
#pragma unroll
        for (int mt = 0; mt < Core::MT; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key1 = KT + mt * 16 + 4 * g + r;
            zs[4 * mt + r] = core.s[0][mt][r];
            const float z1 = key1 < p.b2 ? core.s2[0][mt][r] : MASKED;
            core.s2[0][mt][r] = z1;
            zs[4 * Core::MT + 4 * mt + r] = z1;
          }
        const float m = wave_max_x16x32(Core::tree_max(zs)) * p.sc2;   // base-2 units
        float ps[8 * Core::MT], pz[4 * Core::MT];
#pragma unroll
        for (int j = 0; j < 8 * Core::MT; ++j) ps[j] = __builtin_amdgcn_exp2f(fmaf(zs[j], p.sc2, -m));
#pragma unroll
        for (int j = 0; j < 4 * Core::MT; ++j) pz[j] = fmaf(ps[2 * j], zs[2 * j], ps[2 * j + 1] * zs[2 * j + 1]);
#pragma unroll
        for (int mt = 0; mt < Core::MT; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            core.s[0][mt][r] = ps[4 * mt + r];
            core.s2[0][mt][r] = ps[4 * Core::MT + 4 * mt + r];
          }
        core.m[0] = m;
        core.l[0] = Core::tree_sum(ps);
        core.e[0] = Core::tree_sum(pz);
      }
      const size_t xb = x_row(p.b1, p.b2, p.c1, p.c2, it.sl, it.k, 0, 0, 0);   // slot i -> xb + i
      // c = R K
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) core.o[0][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
      core.template pv<false, 0>(SwzValuesT<D>(cur, cur), 0, KT);
      core.template pv<false, 1>(SwzValuesT<D>(cur + HALF, cur + HALF), 0, KT);
      float lse2[1], h2[1];
      core.finish(lse2, h2, p.sc2);
      store_rows(static_cast<T*>(p.cx), xb, qg0);
      if (g == 0 && q < p.nqs) {
        p.h2x[xb + q] = h2[0];
        p.lser[xb + q] = lse2[0];
      }
      // u = R V on the same probabilities
      const char* vt = cur + TILE;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) core.o[0][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
      core.template pv<false, 0>(SwzValuesT<D>(vt, vt), 0, KT);
      core.template pv<false, 1>(SwzValuesT<D>(vt + HALF, vt + HALF), 0, KT);
      const float inv = 1.f / wave_sum_x16x32(core.l[0]);
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) core.o[0][dt] *= inv;
      store_rows(static_cast<T*>(p.ux), xb, qg0);
    };
    const int item0 = (int)xcd_swizzle(blockIdx.x, gridDim.x);
    if (item0 >= nitems) return;
    It ia = decode(item0), ib;
    issue(ia, buf_a);
    for (;;) {
      step(ia, buf_a, buf_b, ib);
      if (ib.item >= nitems) break;
      step(ib, buf_b, buf_a, ia);
      if (ia.item >= nitems) break;
    }
  }
};

template <int D, bool PAD>
__global__ __launch_bounds__(8 * WAVE, 4) void stage1_pair_kernel(Stage1Params p) {
  __shared__ __attribute__((aligned(1024))) char lds[Stage1Pair<D, PAD>::LDS_BYTES];
  Stage1Pair<D, PAD>::run(p, lds);
}

// ---------------------------------------------------------------------------
// Stage 2.  Item = (slice, column i, row tile t, query group of NW*NQ*16
// rows); its b1*c2 keys are streamed in chunks of KT.  A workgroup walks the
// flat sequence of (item, chunk) units of its items, copying unit u+1 into
// the other buffer while unit u computes.
// ---------------------------------------------------------------------------
// Key chunk of the stage-2 builds of 32 query rows a wave (head_dim 128):
// 64 keys, so a chunk's copies are issued a whole 64-key chunk of arithmetic
// ahead of their use (32-key chunks left the copy latency exposed).
constexpr int KC_R32 = KT;

template <int D, bool KLO, bool WITH_PV, int KC>
struct Stage2AsyncSmem {
  static constexpr int TILE = KC * SwzTile<D>::RB;
  static constexpr int HI = 0;
  static constexpr int LO = TILE;
  static constexpr int U = (KLO ? 2 : 1) * TILE;
  static constexpr int BUF = U + (WITH_PV ? TILE : 0);
};

// PAD: a padded flat sequence (no output at padding positions).
//
// The per-chunk path is kept short: the workgroup decodes an item (integer
// divisions, exchange offsets) once, when its first chunk is issued, and
// every lane's copy offsets within a full key chunk are computed once per
// launch, so a chunk's copies cost one address add each.  Each wave copies
// its own query rows of the next item into LDS with that item's first
// chunk (where LDS allows; otherwise it prefetches them into registers),
// and stores an item's outputs as soon as its last chunk is done, which
// keeps the registers for the arithmetic.
template <int D, int NW, int NQ, bool WITH_PV, bool PRECISE, int KC = KT, bool PAD = false, bool CAUSAL = true>
struct Stage2Async {
  typedef Stage2AsyncSmem<D, split_x<bf16, PRECISE>(), WITH_PV, KC> SM0;
  // y rows leave through a per-wave LDS staging tile (whole 16-byte row
  // chunks per store), except in the builds of 32 rows a wave, which store
  // straight from the accumulators (8 bytes a lane) and keep their LDS small
  // enough for two workgroups a CU
  static constexpr bool DIRECT_Y = WITH_PV && NQ > 1;
  static constexpr int STG = WITH_PV && !DIRECT_Y ? NW * WaveRows<D>::BYTES : 0;
  static constexpr int QROWS = NQ * 16 * SwzTile<D>::RB;        // one wave's query rows
  // Builds of 32 rows a wave (NQ > 1) read the next item's query rows into
  // the score operands as soon as the current item's last score product has
  // been issued (the operands are free from then on; the loads overlap that
  // chunk's softmax and weighted sum), so their LDS holds key chunks only;
  // bidirectional builds (one code path for every chunk).  Other builds
  // stage the queries in LDS where they fit (else prefetch them into
  // registers of their own).
  static constexpr bool QLATE = NQ > 1 && !CAUSAL;
  static constexpr bool QLDS = !QLATE && 2 * SM0::BUF + STG + NW * QROWS + 2 * KC * 4 <= 160 * 1024;
  static constexpr int LDS_BYTES = 2 * SM0::BUF + STG + (QLDS ? NW * QROWS : 0) + 2 * KC * 4;

  // An item (slice, column i, row tile t, query group qg) and its key chunks.
  struct Item {
    int item, sl, i, t, qg, nch;
    size_t base;        // exchange row of its first key
  };

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
  char* const qrows = lds + 2 * SM::BUF + STG;
  float* const bias_a = reinterpret_cast<float*>(lds + 2 * SM::BUF + STG + (QLDS ? NW * QROWS : 0));
  float* const bias_b = bias_a + KC;

  const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE, g = lane / 16;
  char* const qw = qrows + wave * QROWS;          // this wave's query rows (copied by the wave itself)
  const int nitems = p.S * p.b2 * p.c1 * p.nqg;
  const size_t xs = x_stride(p.b2, p.c1);                 // exchange rows between keys
  const size_t key_bytes = xs * D * sizeof(T);
  auto row_of = [&](int qg, int n) { return qg * QG + wave * NQ * 16 + n * 16 + lane % 16; };
  auto decode = [&](int item) {
    Item it;
    it.item = item;
    it.qg = item % p.nqg; item /= p.nqg;
    it.t = item % p.c1; item /= p.c1;
    it.i = item % p.b2;
    it.sl = item / p.b2;
    it.nch = (stage2_keys(p, it.t, it.qg * QG + QG) + KC - 1) / KC;
    it.base = x_base(p.b1, p.b2, p.c1, p.c2, it.sl, it.t, it.i);
    return it;
  };

  constexpr int CPR = D / 8, NI = KC * CPR / WAVE, NCW = (NI + NW - 1) / NW;
  static_assert((KC * CPR) % WAVE == 0, "tile must be whole wave copies");
  int crow[NCW];
  uint32_t ccol[NCW];
  size_t coff[NCW];
#pragma unroll
  for (int j = 0; j < NCW; ++j) {
    const int slot = (j * NW + wave) * WAVE + lane;
    crow[j] = slot / CPR;
    ccol[j] = (uint32_t)(((slot % CPR) ^ SwzTile<D>::swz(crow[j])) << 4);
    coff[j] = (size_t)crow[j] * key_bytes + ccol[j];
  }
  auto copy_tile = [&](char* dst, const char* src, int nvalid) {
    if constexpr (NI % NW == 0 && (NCW == 2 || NCW == 4)) {
      // a whole chunk: one address add a copy, the copies of the tile in
      // one block (copy j lands NW * WAVE * 16 bytes after copy j - 1)
      if (nvalid == KC) {
        constexpr uint32_t ST = NW * WAVE * 16;
        const uint32_t l0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(dst + wave * WAVE * 16));
        if constexpr (NCW == 2) copy16x2_to_lds(src + coff[0], src + coff[1], l0, l0 + ST);
        else copy16x4_to_lds(src + coff[0], src + coff[1], src + coff[2], src + coff[3], l0, l0 + ST,
                             l0 + 2 * ST, l0 + 3 * ST);
        return;
      }
    }
#pragma unroll
    for (int j = 0; j < NCW; ++j) {
      const int ii = j * NW + wave;
      if (NI % NW != 0 && ii >= NI) break;
      const size_t off = nvalid == KC ? coff[j] : (size_t)min(crow[j], nvalid - 1) * key_bytes + ccol[j];
      copy16_to_lds(src + off, dst + ii * WAVE * 16);
    }
  };
  // The wave's query rows into qw: copy j moves chunk (slot % CPR) of row
  // slot / CPR, slot = j * WAVE + lane, to the swizzled place of that chunk.
  constexpr int QCW = NQ * 16 * CPR / WAVE;
  auto copy_queries = [&](const Item& it) {
#pragma unroll
    for (int j = 0; j < QCW; ++j) {
      const int slot = j * WAVE + lane, r = slot / CPR, cs = slot % CPR;
      const int c = cs ^ SwzTile<D>::swz(r);
      const T* src = stage2_qsrc<T, D, PAD>(p, it.sl, it.i, it.t, it.qg * QG + wave * NQ * 16 + r).t;
      copy16_to_lds(src + c * 8, qw + j * WAVE * 16);
    }
  };

  frag qn[NQ][Core::NKS];
  typename Core::QLo qnl;
  float hn[(KC + WAVE - 1) / WAVE];   // bias of the unit in flight (last wave)
  auto issue = [&](const Item& it, int ch, char* b) {
    const size_t row0 = it.base + (size_t)ch * KC * xs;
    const int nvalid = min(KC, p.nkeys - ch * KC);
    const char* C = static_cast<const char*>(p.cx) + row0 * D * sizeof(T);
    copy_tile(b + SM::HI, C, nvalid);
    if constexpr (KLO) copy_tile(b + SM::LO, C + p.xlo * sizeof(T), nvalid);
    if constexpr (WITH_PV) copy_tile(b + SM::U, static_cast<const char*>(p.ux) + row0 * D * sizeof(T), nvalid);
    if (wave == NW - 1) {
#pragma unroll
      for (int j = 0; j < (KC + WAVE - 1) / WAVE; ++j)
        hn[j] = p.h2x[row0 + (size_t)min(min(lane + WAVE * j, KC - 1), nvalid - 1) * xs];
    }
    if (ch == 0) {
      if constexpr (QLDS) copy_queries(it);
      else if constexpr (!QLATE)
        Core::fetch_queries([&](int n) { return stage2_qsrc<T, D, PAD>(p, it.sl, it.i, it.t, row_of(it.qg, n)); },
                            Q_INPUT, qn, qnl);
    }
  };
  // QLATE: the item's query rows straight into the score operands
  auto load_queries = [&](Core& core, const Item& it) {
    Core::fetch_queries([&](int n) { return stage2_qsrc<T, D, PAD>(p, it.sl, it.i, it.t, row_of(it.qg, n)); },
                        Q_INPUT, core.qf, qnl);
  };

  const int item0 = (int)xcd_swizzle(blockIdx.x, gridDim.x);
  if (item0 >= nitems) return;
  Item cur = decode(item0), nx = cur;
  int ch = 0;
  issue(cur, 0, buf_a);
  Core core;
  if constexpr (QLATE) load_queries(core, cur);
  char* stg = stage_rows + (STG ? wave * WaveRows<D>::BYTES : 0);

  // y rows and normalisers of the item just finished
  auto store = [&]() {
    float lse2[NQ], h2[NQ];
    core.finish(lse2, h2, p.sc2);
    const AxisMap am = p.map.template col_axis<PAD>(cur.i);
    const int l0 = cur.t * p.rt + row_of(cur.qg, 0) - lane % 16, lend = cur.t * p.rt + p.rt;
    if constexpr (WITH_PV) {
      T* Y = static_cast<T*>(p.y) + (size_t)cur.sl * p.N * D;
#pragma unroll
      for (int n = 0; n < NQ; ++n) {
        bf16x4 y[D / 16];
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) y[dt] = __builtin_convertvector(core.o[n][dt], bf16x4);
        if constexpr (DIRECT_Y) {
          // lane (q, g) holds columns 16 dt + 4 g .. + 3 of row q
          const int l = l0 + n * 16 + lane % 16;
          T* dst = nullptr;
          if constexpr (PAD) dst = l < lend && am.valid(l) ? Y + am.at(l) * D : nullptr;
          else dst = l < lend ? Y + am.raw(l) * D : nullptr;
          if (dst) {
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt) *reinterpret_cast<bf16x4*>(dst + 16 * dt + 4 * g) = y[dt];
          }
        } else {
          WaveRows<D>::put(stg, y);
          WaveRows<D>::drain(stg, [&](int r) -> T* {
            const int l = l0 + n * 16 + r;
            if constexpr (PAD) return l < lend && am.valid(l) ? Y + am.at(l) * D : nullptr;
            else return l < lend ? Y + am.raw(l) * D : nullptr;
          });
        }
      }
    }
#pragma unroll
    for (int n = 0; n < NQ; ++n) {
      const int ll = row_of(cur.qg, n);
      if (ll >= p.rt || g != 0) continue;
      const int l = cur.t * p.rt + ll;
      p.lse2[((size_t)cur.sl * p.b2 + cur.i) * p.b1 + l] = lse2[n];
      if (p.lse_out) {
        if constexpr (PAD) {
          if (am.valid(l)) p.lse_out[(size_t)cur.sl * p.N + am.at(l)] = lse2[n] * LN2;
        } else {
          p.lse_out[(size_t)cur.sl * p.N + am.raw(l)] = lse2[n] * LN2;
        }
      }
    }
  };
  auto unit = [&](const char* cb, float* bias, char* nxt) -> bool {
    const int nvalid = min(KC, p.nkeys - ch * KC);
    wait_vmem();
    if (wave == NW - 1) {
      // keys past the end of the column get a bias that zeroes their
      // probabilities, so a partial chunk takes the full-chunk path
#pragma unroll
      for (int j = 0; j < (KC + WAVE - 1) / WAVE; ++j)
        if (lane + WAVE * j < KC) bias[lane + WAVE * j] = lane + WAVE * j < nvalid ? hn[j] : -1e30f;
    }
    __syncthreads();              // cb landed everywhere; nobody reads nxt any more
    if (ch == 0) {
      core.init();
      if constexpr (QLDS) {
#pragma unroll
        for (int n = 0; n < NQ; ++n)
#pragma unroll
          for (int ks_ = 0; ks_ < Core::NKS; ++ks_)
            core.qf[n][ks_] = *reinterpret_cast<const frag*>(qw + SwzTile<D>::offset(n * 16 + lane % 16, 4 * ks_ + g));
        // the rows are in registers before the next item's copy may refill qw
        __builtin_amdgcn_s_waitcnt(0xC07F);
      } else if constexpr (!QLATE) {
        core.set_queries(qn, qnl);
      }
    }
    int nchk = ch + 1;
    bool more = true;
    if (nchk == cur.nch) {
      nchk = 0;
      more = cur.item + (int)gridDim.x < nitems;
      if (more) nx = decode(cur.item + gridDim.x);
    }
    if (more) issue(nchk == 0 ? nx : cur, nchk, nxt);

    int how = CH_WHOLE;
    if constexpr (!CAUSAL) {
      core.scores_v(SwzKeys<D>(cb + SM::HI, cb + SM::LO), 0, Core::MT);
      if constexpr (QLATE) {
        if (nchk == 0 && more) load_queries(core, nx);
      }
      core.template softmax_step<true, false>(bias, p.sc2, 0, KC);
      if constexpr (WITH_PV) core.template pv<false>(SwzValuesT<D>(cb + SM::U, cb + SM::U), 0, KC);
      how = CH_SKIP;
    } else if (p.causal) {
      how = causal_chunk<NQ>(core, p, cur.t, row_of(cur.qg, 0) - lane % 16,
                             [&](int n) { return row_of(cur.qg, n); }, ch * KC, nvalid);
    }
    const bool rowmask = how == CH_ROWMASK;
    if (how != CH_SKIP) {
      core.scores_v(SwzKeys<D>(cb + SM::HI, cb + SM::LO), 0, Core::MT);
      if (rowmask) core.template softmax_step<true, true, 0, true>(bias, p.sc2, 0, nvalid);
      else if (nvalid == KC) core.template softmax_step<true, false>(bias, p.sc2, 0, nvalid);
      else core.template softmax_step<true, true>(bias, p.sc2, 0, nvalid);
      if constexpr (WITH_PV) {
        const SwzValuesT<D> vv(cb + SM::U, cb + SM::U);
        if (nvalid == KC && !rowmask) core.template pv<false>(vv, 0, nvalid);
        else core.template pv<true>(vv, 0, nvalid);
      }
    }
    if (ch == cur.nch - 1) store();
    if (!more) return false;
    if (nchk == 0) cur = nx;
    ch = nchk;
    return true;
  };
  while (unit(buf_a, bias_a, buf_b) && unit(buf_b, bias_b, buf_a)) {
  }
  }
};

template <int D, int NW, int NQ, bool WITH_PV, bool PRECISE, int KC = KT, bool PAD = false, bool CAUSAL = true,
          int WPC = (NQ > 1 ? 2 : 1)>
__global__ __launch_bounds__(NW * WAVE, WPC) void stage2_async_kernel(Stage2Params p) {
  typedef Stage2Async<D, NW, NQ, WITH_PV, PRECISE, KC, PAD, CAUSAL> S;
  __shared__ __attribute__((aligned(1024))) char lds[S::LDS_BYTES];
  S::run(p, lds);
}

// ---------------------------------------------------------------------------
// Stage 2 of the last step for columns of 65-128 keys at head_dim 64 (the
// 128 x 128 grid of a 16K sequence), bidirectional, unpadded, one row tile:
// an item is one column's query group of 128 rows, and its keys are one
// 128-key chunk.  The same arithmetic as the general stage 2 on such a
// column (one online-softmax update from a fresh state, then O += P U), with
// a leaner data path: each wave reads its query rows of the next item into
// registers, the bias row is staged by one wave, and y leaves through an
// 8-row staging tile per wave.  73 KB of LDS and at most 128 registers a
// lane, so two workgroups share a CU at four waves a SIMD.
// ---------------------------------------------------------------------------
// PAD: a padded flat sequence (query rows clamped on load, no output at
// padding positions).
template <int D, bool PAD = false>
struct Stage2Col {
  static constexpr int NW = 8, QG = NW * 16, KC = 2 * KT;
  static constexpr int TILE = KC * SwzTile<D>::RB;
  static constexpr int BUF = 2 * TILE;                     // c tile, u tile
  static constexpr int STG = 8 * SwzTile<D>::RB;           // a wave's y staging: 8 rows
  static constexpr int LDS_BYTES = 2 * BUF + 2 * KC * 4 + NW * STG;

  __host__ __device__ static bool serves(int b2, int c1, int nkeys, int causal, bool padded) {
    return b2 > KT && c1 == 1 && nkeys > KT && nkeys <= KC && !causal && padded == PAD;
  }

  __device__ static void run(const Stage2Params& p, char* lds) {
    typedef bf16 T;
    typedef FlashCore<T, D, D, 1, KC, false, true, false, 0> Core;
    typedef typename Core::frag frag;
    char* const buf_a = lds;
    char* const buf_b = lds + BUF;
    float* const bias_a = reinterpret_cast<float*>(lds + 2 * BUF);
    float* const bias_b = bias_a + KC;
    const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE, g = lane / 16;
    char* const stg = lds + 2 * BUF + 2 * KC * 4 + wave * STG;
    const int nitems = p.S * p.b2 * p.nqg;
    const size_t xs = x_stride(p.b2, p.c1);
    struct It {
      int item, sl, i, qg;
    };
    auto decode = [&](int item) {
      It it;
      it.item = item;
      it.qg = item % p.nqg; item /= p.nqg;
      it.i = item % p.b2;
      it.sl = item / p.b2;
      return it;
    };
    auto row_of = [&](int qg) { return qg * QG + wave * 16 + lane % 16; };
    frag qn[1][Core::NKS];
    typename Core::QLo qnl;
    float hn[KC / WAVE];            // bias of the item in flight (last wave)
    auto issue = [&](const It& it, char* b) {
      const size_t base = x_base(p.b1, p.b2, p.c1, p.c2, it.sl, 0, it.i);
      const T* C = static_cast<const T*>(p.cx) + base * D;
      const T* U = static_cast<const T*>(p.ux) + base * D;
      SwzTile<D>::template load<KC, NW>(b, [&](int r) { return C + (size_t)r * xs * D; }, p.nkeys);
      SwzTile<D>::template load<KC, NW>(b + TILE, [&](int r) { return U + (size_t)r * xs * D; }, p.nkeys);
      if (wave == NW - 1) {
#pragma unroll
        for (int j = 0; j < KC / WAVE; ++j) hn[j] = p.h2x[base + (size_t)min(lane + WAVE * j, p.nkeys - 1) * xs];
      }
      Core::fetch_queries([&](int) { return stage2_qsrc<T, D, PAD>(p, it.sl, it.i, 0, row_of(it.qg)); },
                          Q_INPUT, qn, qnl);
    };
    Core core;
    auto step = [&](const It& it, const char* cur, float* bias, char* nxt, It& next) {
      wait_vmem();
      if (wave == NW - 1) {
        // keys past the end of the column: a bias that zeroes their probabilities
#pragma unroll
        for (int j = 0; j < KC / WAVE; ++j) bias[lane + WAVE * j] = lane + WAVE * j < p.nkeys ? hn[j] : -1e30f;
      }
      __syncthreads();              // cur and its bias landed everywhere; nobody reads nxt any more
      core.init();
      core.set_queries(qn, qnl);
      next.item = it.item + (int)gridDim.x;
      if (next.item < nitems) {
        next = decode(next.item);
        issue(next, nxt);
      }
      core.scores_v(SwzKeys<D>(cur, nullptr), 0, Core::MT);
      core.template softmax_step<true, false>(bias, p.sc2, 0, KC);
      core.template pv<false>(SwzValuesT<D>(cur + TILE, cur + TILE), 0, KC);
      float lse2[1], h2[1];
      core.finish(lse2, h2, p.sc2);
      // y rows: lane (q, g) holds columns 16 dt + 4 g .. + 3 of row q.  They
      // leave through the wave's 8-row staging tile, half the rows at a
      // time, so that every store instruction writes whole rows (whole
      // lines) instead of a quarter of each of 16 rows.
      const AxisMap am = p.map.template col_axis<PAD>(it.i);
      auto real_row = [&](int l, int64_t& tk) -> bool {
        if constexpr (PAD) {
          tk = am.at(l);
          return l < p.rt && am.valid(l);
        } else {
          tk = am.raw(l);
          return l < p.rt;
        }
      };
      {
        bf16x4 v[D / 16];
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) v[dt] = __builtin_convertvector(core.o[0][dt], bf16x4);
        T* const Y = static_cast<T*>(p.y) + (size_t)it.sl * p.N * D;
        const int l0 = it.qg * QG + wave * 16, q = lane % 16;
        constexpr int CPR = D / 8, RPI = WAVE / CPR;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          wave_sync();        // the previous reads of the tile are done
          if ((q >> 3) == h) {
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt)
              *reinterpret_cast<bf16x4*>(stg + SwzTile<D>::offset(q - 8 * h, 2 * dt + g / 2) + 8 * (g % 2)) = v[dt];
          }
          wave_sync();        // every lane's half of the rows is in the tile
#pragma unroll
          for (int r0 = 0; r0 < 8; r0 += RPI) {
            const int r = r0 + lane / CPR, c = lane % CPR;
            const bf16x8 val = *reinterpret_cast<const bf16x8*>(stg + SwzTile<D>::offset(r, c));
            int64_t tk;
            if (real_row(l0 + 8 * h + r, tk)) *reinterpret_cast<bf16x8*>(Y + tk * D + c * 8) = val;
          }
        }
      }
      const int l = row_of(it.qg);
      int64_t tk;
      const bool real = real_row(l, tk);
      if (l < p.rt && g == 0) {
        p.lse2[((size_t)it.sl * p.b2 + it.i) * p.b1 + l] = lse2[0];
        if (p.lse_out && real) p.lse_out[(size_t)it.sl * p.N + tk] = lse2[0] * LN2;
      }
    };
    const int item0 = (int)xcd_swizzle(blockIdx.x, gridDim.x);
    if (item0 >= nitems) return;
    It ia = decode(item0), ib;
    issue(ia, buf_a);
    for (;;) {
      step(ia, buf_a, bias_a, buf_b, ib);
      if (ib.item >= nitems) break;
      step(ib, buf_b, bias_b, buf_a, ia);
      if (ia.item >= nitems) break;
    }
  }
};

template <int D, bool PAD>
__global__ __launch_bounds__(8 * WAVE, 4) void stage2_col_kernel(Stage2Params p) {
  __shared__ __attribute__((aligned(1024))) char lds[Stage2Col<D, PAD>::LDS_BYTES];
  Stage2Col<D, PAD>::run(p, lds);
}

// ---------------------------------------------------------------------------
// A step before the last of an untiled, unpadded run whose columns hold at
// most 64 rows and 64 keys: the L-update and the next step's queries in one
// launch.  One workgroup of 4 waves per (slice, column i) copies the
// column's keys c (hi + lo planes on the split path) and its query rows into
// LDS.  Each wave scores its 16 rows against every key (MFMA), takes the row
// softmax over the keys (L; the row normaliser is stored as stage 2 stores
// it) and writes its rows of L, transposed, into LDS.  Then wave w forms, for
// the keys of its 16-key tile, alpha = sum_l L[l,k] q[l] (MFMA; L enters as
// bf16 hi + lo on the split path) and beta = sum_l L[l,k], and stores
// qt = alpha / beta, or the column mean of q where beta is zero (the
// zero-weight fallback).  This replaces a stage-2 statistics launch plus
// the alpha launch, which read c and Q again and recomputed the scores.
// ---------------------------------------------------------------------------
template <int D>
struct Stage2AlphaSmem {
  static constexpr int TILE = 64 * SwzTile<D>::RB;            // 64 rows of D bf16
  static constexpr int CHI = 0, CLO = TILE, QT = 2 * TILE;    // keys (hi, lo), query rows
  static constexpr int LDL = 64 + 4;                           // fp32 stride of a row of L^T
  static constexpr int LT = 3 * TILE;                          // L^T: [64 keys][LDL]
  static constexpr int BIAS = LT + 64 * LDL * 4;
  static constexpr int BYTES = BIAS + 64 * 4;
};

template <int D, bool PRECISE>
__global__ __launch_bounds__(256) void stage2_alpha_kernel(Stage2Params p, float* qt_out) {
  typedef bf16 T;
  constexpr bool KLO = split_x<T, PRECISE>();
  typedef FlashCore<T, D, D, 1, 64, false, false, KLO, 0> Core;
  typedef typename Core::frag frag;
  typedef Stage2AlphaSmem<D> SM;
  __shared__ __attribute__((aligned(1024))) char lds[SM::BYTES];
  const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE, g = lane / 16;
  const int i = blockIdx.x % p.b2, sl = blockIdx.x / p.b2;
  const int nk = p.nkeys, rt = p.rt;           // both at most 64 (host-checked)
  const size_t xs = x_stride(p.b2, 1), base = x_base(p.b1, p.b2, 1, 1, sl, 0, i);
  const T* C = static_cast<const T*>(p.cx) + base * D;
  const T* Q = static_cast<const T*>(p.q) + (size_t)sl * p.N * D;
  const AxisMap am = p.map.template col_axis<false>(i);
  // rows past nk / rt repeat the last one (their scores are masked, their L is 0)
  SwzTile<D>::template load<64, 4>(lds + SM::CHI, [&](int r) { return C + (size_t)r * xs * D; }, nk);
  if constexpr (KLO)
    SwzTile<D>::template load<64, 4>(lds + SM::CLO, [&](int r) { return C + p.xlo + (size_t)r * xs * D; }, nk);
  SwzTile<D>::template load<64, 4>(lds + SM::QT, [&](int r) { return Q + am.raw(r) * D; }, rt);
  float* bias = reinterpret_cast<float*>(lds + SM::BIAS);
  if (threadIdx.x < 64) bias[threadIdx.x] = p.h2x[base + (size_t)min((int)threadIdx.x, nk - 1) * xs];
  wait_vmem();
  __syncthreads();

  // L-update of this wave's 16 rows
  Core core;
  core.init();
  const int row = 16 * wave + lane % 16;
  const int rowc = min(row, rt - 1);
#pragma unroll
  for (int ks = 0; ks < Core::NKS; ++ks)
    core.qf[0][ks] = *reinterpret_cast<const frag*>(lds + SM::QT + SwzTile<D>::offset(rowc, 4 * ks + g));
  core.scores_v(SwzKeys<D>(lds + SM::CHI, lds + SM::CLO), 0, Core::MT);
  if (nk == 64) core.template softmax_step<true, false>(bias, p.sc2, 0, 64);
  else core.template softmax_step<true, true>(bias, p.sc2, 0, nk);
  const float lt = wave_sum_x16x32(core.l[0]);
  float lse2[1], h2[1];
  core.finish(lse2, h2, p.sc2);
  if (g == 0 && row < rt) p.lse2[((size_t)sl * p.b2 + i) * p.b1 + row] = lse2[0];
  float* Lt = reinterpret_cast<float*>(lds + SM::LT);
  const float inv = row < rt ? 1.f / lt : 0.f;        // rows past the column carry no L
#pragma unroll
  for (int mt = 0; mt < Core::MT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) Lt[(mt * 16 + 4 * g + r) * SM::LDL + row] = core.s[0][mt][r] * inv;
  __syncthreads();

  // alpha and beta of this wave's keys, over all rows
  if (16 * wave >= nk) return;
  const int key = 16 * wave + lane % 16;
  const SwzValuesT<D> qv(lds + SM::QT, lds + SM::QT);
  f32x4 acc[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float beta = 0.f;
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    // rows {32kk + 4g + r} and {32kk + 16 + 4g + r}: the k order of qv.at
    const f32x4 a0 = *reinterpret_cast<const f32x4*>(Lt + key * SM::LDL + 32 * kk + 4 * g);
    const f32x4 a1 = *reinterpret_cast<const f32x4*>(Lt + key * SM::LDL + 32 * kk + 16 + 4 * g);
    const bf16x4 h0 = __builtin_convertvector(a0, bf16x4), h1 = __builtin_convertvector(a1, bf16x4);
    const frag b = __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7);
    frag bl = {};
    if constexpr (PRECISE) {
      bl = __builtin_shufflevector(__builtin_convertvector(a0 - __builtin_convertvector(h0, f32x4), bf16x4),
                                   __builtin_convertvector(a1 - __builtin_convertvector(h1, f32x4), bf16x4),
                                   0, 1, 2, 3, 4, 5, 6, 7);
      beta += (a0[0] + a0[1]) + (a0[2] + a0[3]) + (a1[0] + a1[1]) + (a1[2] + a1[3]);
    } else {
      // the values the MFMA consumes
      const f32x4 r0 = __builtin_convertvector(h0, f32x4), r1 = __builtin_convertvector(h1, f32x4);
      beta += (r0[0] + r0[1]) + (r0[2] + r0[3]) + (r1[0] + r1[1]) + (r1[2] + r1[3]);
    }
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      const frag a = qv.at(dt, kk);
      acc[dt] = Mfma<T>::mma(a, b, acc[dt]);
      if constexpr (PRECISE) acc[dt] = Mfma<T>::mma(a, bl, acc[dt]);
    }
  }
  beta = wave_sum_x16x32(beta);
  // lane (g, key) holds alpha[key][16 dt + 4 g + r]
  float* out = qt_out + (((size_t)sl * p.b1 + min(key, nk - 1)) * p.b2 + i) * D;
  if (__any(beta <= 0.f)) {
    // zero weight somewhere in this wave: the column mean of q over its rows
    f32x4 mean[D / 16];
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      mean[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int d0 = 16 * dt + 4 * g;
      for (int r = 0; r < rt; ++r) {
        const bf16x4 v = *reinterpret_cast<const bf16x4*>(lds + SM::QT + SwzTile<D>::offset(r, d0 / 8) +
                                                          2 * (d0 % 8));
        mean[dt] += __builtin_convertvector(v, f32x4);
      }
      mean[dt] *= 1.f / (float)rt;
    }
    if (beta <= 0.f) {
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) acc[dt] = mean[dt];
      beta = 1.f;
    }
  }
  if (key >= nk) return;
  const float ib = 1.f / beta;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) store4(out + dt * 16 + 4 * g, acc[dt] * ib);
}

// ---------------------------------------------------------------------------
// Fused single launch for T = 1 (untiled): stage 1 over every block, a
// grid-wide barrier, stage 2 over every column, in one cooperative launch of
// resident persistent workgroups.  Removes the launch gap between the stages;
// the exchange written by phase 1 is read by phase 2 while it is still warm
// in the Infinity Cache.  Both phases use NW waves per workgroup.
// ---------------------------------------------------------------------------
template <int D, int NW, int KTB, bool PRECISE, int KC2 = KT>
__global__ __launch_bounds__(NW * WAVE) void fused_async_kernel(Stage1Params p1, Stage2Params p2) {
  typedef Stage1Async<D, NW, KTB, true, PRECISE> S1;
  // head_dim 128 (fast path): the staged launch's stage 2 of 32 rows a wave
  // and KC_R32-key chunks, so that both give the same result
  constexpr bool R32 = D == 128 && !PRECISE;
  typedef Stage2Async<D, NW, R32 ? 2 : 1, true, PRECISE, R32 ? KC_R32 : KC2> S2;
  // head_dim 64, 8 waves, blocks of 65-128 keys in one segment: the staged
  // launch's whole-block stage 1, so that both give the same result
  constexpr bool PAIR = D == 64 && NW == 8 && KTB == 2 * KT && !PRECISE;
  constexpr int B12 = S1::LDS_BYTES > S2::LDS_BYTES ? S1::LDS_BYTES : S2::LDS_BYTES;
  constexpr int BYTES = PAIR && Stage1Pair<D>::LDS_BYTES > B12 ? Stage1Pair<D>::LDS_BYTES : B12;
  __shared__ __attribute__((aligned(1024))) char lds[BYTES];
  if constexpr (PAIR) {
    if (Stage1Pair<D>::serves(p1.b2, p1.c1, p1.c2, false)) Stage1Pair<D>::run(p1, lds);
    else S1::run(p1, lds);
  } else {
    S1::run(p1, lds);
  }
  __syncthreads();
  cooperative_groups::this_grid().sync();
  S2::run(p2, lds);
}

}  // namespace ma
