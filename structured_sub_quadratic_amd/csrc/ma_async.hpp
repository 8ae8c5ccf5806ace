// Stage kernels for bf16 whose LDS tiles are filled by direct global->LDS
// copies (global_load_lds, 16 bytes a lane) instead of register staging.
//
// Each persistent workgroup keeps two LDS buffers: while it computes on one,
// the copies of its next unit of work stream into the other, so the loads of
// a whole tile are in flight behind the arithmetic without holding any
// registers.  Tiles stay row-major (as they are in HBM); the 16-byte chunks
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

#include "ma_stage_kernels.hpp"

namespace ma {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;

// Wait until every vector-memory operation of this wave has completed
// (direct-to-LDS copies included): vmcnt(0), other counters untouched.
__device__ inline void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Copy 16 bytes at g into LDS at wave_base + 16 * lane (wave_base uniform).
__device__ inline void copy16_to_lds(const void* g, void* wave_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_void_t*)wave_base, 16, 0, 0);
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
#pragma unroll
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
// Stage 1, whole block in one tile (b2 <= KTB).  Item = (slice, block k,
// query group of NW*NQ*16 slots); NW waves of NQ sub-tiles of 16 queries.
// ---------------------------------------------------------------------------
template <int D, int NW, int NQ, int KTB, bool WITH_U>
struct Stage1AsyncSmem {
  static constexpr int TILE = KTB * SwzTile<D>::RB;            // one K or V tile
  static constexpr int BUF = (WITH_U ? 2 : 1) * TILE;
  static constexpr int BYTES = 2 * BUF;
};

template <int D, int NW, int NQ, int KTB, bool WITH_U, bool PRECISE, bool QSPLIT>
__global__ __launch_bounds__(NW * WAVE) void stage1_async_kernel(Stage1Params p) {
  typedef bf16 T;
  constexpr bool SPLITX = split_x<T, PRECISE>();
  constexpr int DV = WITH_U ? 2 * D : D;
  constexpr int QG = NW * NQ * 16;
  constexpr int NSPLIT = PRECISE ? D / 16 : 0;
  typedef FlashCore<T, D, DV, NQ, KT, true, true, false, NSPLIT, QSPLIT> Core;
  typedef typename Core::frag frag;
  typedef Stage1AsyncSmem<D, NW, NQ, KTB, WITH_U> SM;
  __shared__ __attribute__((aligned(1024))) char smem[SM::BYTES];

  const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE, g = lane / 16;
  const int nitems = p.S * p.b1 * p.nqg;
  const int mode = stage1_qmode(p);
  const bool split = PRECISE && mode != Q_INPUT;
  auto slot_of = [&](int qg, int n) { return qg * QG + wave * NQ * 16 + n * 16 + lane % 16; };

  frag qn[NQ][Core::NKS];
  typename Core::QLo qnl;
  auto issue = [&](int item, int buf) {
    const int qg = item % p.nqg, k = (item / p.nqg) % p.b1, sl = item / (p.nqg * p.b1);
    const T* K = static_cast<const T*>(p.k) + (size_t)sl * p.N * D;
    char* b = smem + buf * SM::BUF;
    SwzTile<D>::template load<KTB, NW>(b, [&](int r) { return K + (size_t)p.map.token(k, r) * D; }, p.b2);
    if constexpr (WITH_U) {
      const T* V = static_cast<const T*>(p.v) + (size_t)sl * p.N * D;
      SwzTile<D>::template load<KTB, NW>(b + SM::TILE, [&](int r) { return V + (size_t)p.map.token(k, r) * D; }, p.b2);
    }
    Core::fetch_queries([&](int n) { return stage1_qsrc<T, D>(p, sl, k, slot_of(qg, n), 0); }, mode, qn, qnl);
  };

  int item = blockIdx.x;
  if (item >= nitems) return;
  issue(item, 0);
  Core core;
  core.qsplit = QSPLIT && split;
  for (int j = 0; item < nitems; ++j, item += gridDim.x) {
    const int qg = item % p.nqg, k = (item / p.nqg) % p.b1, sl = item / (p.nqg * p.b1);
    wait_vmem();
    __syncthreads();              // tile j landed everywhere; buffer j+1 is free
    core.set_queries(qn, qnl);
    if (item + (int)gridDim.x < nitems) issue(item + gridDim.x, (j + 1) & 1);
    const char* kt = smem + (j & 1) * SM::BUF;
    const char* vt = WITH_U ? kt + SM::TILE : kt;
    for (int s = 0; s < p.c2; ++s) {
      if (s > 0 && !p.first_step)
        core.load_queries([&](int n) { return stage1_qsrc<T, D>(p, sl, k, slot_of(qg, n), s); }, mode, split);
      const int klo = s * p.sw, khi = klo + p.sw;
      core.init();
#pragma unroll
      for (int c0 = 0; c0 < KTB; c0 += KT) {
        if (c0 >= khi || c0 + KT <= klo) continue;
        const int lo = max(klo - c0, 0), hi = min(khi - c0, KT);
        const int off = c0 * SwzTile<D>::RB;
        core.scores_v(SwzKeys<D>(kt + off, nullptr), lo / 16, (hi + 15) / 16);
        const SwzValuesT<D> vv(kt + off, vt + off);
        if (lo == 0 && hi == KT) {
          core.template softmax_step<false, false>(nullptr, p.sc2, lo, hi);
          core.template pv<false>(vv, lo, hi);
        } else {
          core.template softmax_step<false, true>(nullptr, p.sc2, lo, hi);
          core.template pv<true>(vv, lo, hi);
        }
      }
      float lse2[NQ], h2[NQ];
      core.finish(lse2, h2, p.sc2);
#pragma unroll
      for (int n = 0; n < NQ; ++n) {
        const int slot = slot_of(qg, n);
        if (slot >= p.nqs) continue;
        const int t = slot / p.b2, i = slot % p.b2;
        const size_t row = ((((size_t)sl * p.b2 + i) * p.c1 + t) * p.b1 + k) * p.c2 + s;
        T* C = static_cast<T*>(p.cx) + row * D;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
          const f32x4 v = core.o[n][dt];
          const bf16x4 h = __builtin_convertvector(v, bf16x4);
          *reinterpret_cast<bf16x4*>(C + dt * 16 + 4 * g) = h;
          if constexpr (SPLITX) {
            const bf16x4 l = __builtin_convertvector(v - __builtin_convertvector(h, f32x4), bf16x4);
            *reinterpret_cast<bf16x4*>(C + p.xlo + dt * 16 + 4 * g) = l;
          }
        }
        if (WITH_U) {
          T* U = static_cast<T*>(p.ux) + row * D;
#pragma unroll
          for (int dt = 0; dt < D / 16; ++dt) store4(U + dt * 16 + 4 * g, core.o[n][D / 16 + dt]);
        }
        if (g == 0) {
          p.h2x[row] = h2[n];
          p.lser[row] = lse2[n];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Stage 2.  Item = (slice, column i, row tile t, query group of NW*NQ*16
// rows); its b1*c2 keys are streamed in chunks of KT.  A workgroup walks the
// flat sequence of (item, chunk) units of its items, copying unit u+1 into
// the other buffer while unit u computes.
// ---------------------------------------------------------------------------
template <int D, bool KLO, bool WITH_PV>
struct Stage2AsyncSmem {
  static constexpr int TILE = KT * SwzTile<D>::RB;
  static constexpr int HI = 0;
  static constexpr int LO = TILE;
  static constexpr int U = (KLO ? 2 : 1) * TILE;
  static constexpr int BUF = U + (WITH_PV ? TILE : 0);
  static constexpr int BYTES = 2 * BUF;
};

template <int D, int NW, int NQ, bool WITH_PV, bool PRECISE>
__global__ __launch_bounds__(NW * WAVE) void stage2_async_kernel(Stage2Params p) {
  typedef bf16 T;
  constexpr bool KLO = split_x<T, PRECISE>();
  constexpr int QG = NW * NQ * 16;
  typedef FlashCore<T, D, D, NQ, KT, false, WITH_PV, KLO, 0> Core;
  typedef typename Core::frag frag;
  typedef Stage2AsyncSmem<D, KLO, WITH_PV> SM;
  __shared__ __attribute__((aligned(1024))) char smem[SM::BYTES];
  __shared__ float bias_buf[2][KT];

  const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE, g = lane / 16;
  const int nitems = p.S * p.b2 * p.c1 * p.nqg;
  const int nch = (p.nkeys + KT - 1) / KT;
  auto decode = [&](int item, int& sl, int& i, int& t, int& qg) {
    qg = item % p.nqg; item /= p.nqg;
    t = item % p.c1; item /= p.c1;
    i = item % p.b2;
    sl = item / p.b2;
  };
  auto row_of = [&](int qg, int n) { return qg * QG + wave * NQ * 16 + n * 16 + lane % 16; };

  frag qn[NQ][Core::NKS];
  typename Core::QLo qnl;
  float hn = 0.f;               // bias of the unit in flight (last wave, one key a lane)
  auto issue = [&](int item, int ch, int buf) {
    int sl, i, t, qg;
    decode(item, sl, i, t, qg);
    const size_t base = (((size_t)sl * p.b2 + i) * p.c1 + t) * (size_t)p.b1 * p.c2 + (size_t)ch * KT;
    const int nvalid = min(KT, p.nkeys - ch * KT);
    char* b = smem + buf * SM::BUF;
    const T* C = static_cast<const T*>(p.cx) + base * D;
    SwzTile<D>::template load<KT, NW>(b + SM::HI, [&](int r) { return C + (size_t)r * D; }, nvalid);
    if constexpr (KLO)
      SwzTile<D>::template load<KT, NW>(b + SM::LO, [&](int r) { return C + p.xlo + (size_t)r * D; }, nvalid);
    if constexpr (WITH_PV) {
      const T* U = static_cast<const T*>(p.ux) + base * D;
      SwzTile<D>::template load<KT, NW>(b + SM::U, [&](int r) { return U + (size_t)r * D; }, nvalid);
    }
    if (wave == NW - 1) hn = p.h2x[base + min(lane, nvalid - 1)];
    if (ch == 0)
      Core::fetch_queries([&](int n) { return stage2_qsrc<T, D>(p, sl, i, t, row_of(qg, n)); },
                          Q_INPUT, qn, qnl);
  };

  int item = blockIdx.x;
  if (item >= nitems) return;
  int ch = 0;
  issue(item, 0, 0);
  Core core;
  for (int j = 0;; ++j) {
    wait_vmem();
    if (wave == NW - 1) bias_buf[j & 1][lane] = hn;
    __syncthreads();              // unit j landed everywhere; buffer j+1 is free
    if (ch == 0) {
      core.init();
      core.set_queries(qn, qnl);
    }
    int nitem = item, nchk = ch + 1;
    if (nchk == nch) { nitem = item + gridDim.x; nchk = 0; }
    if (nitem < nitems) issue(nitem, nchk, (j + 1) & 1);

    const char* b = smem + (j & 1) * SM::BUF;
    const float* bias = bias_buf[j & 1];
    const int nvalid = min(KT, p.nkeys - ch * KT);
    core.scores_v(SwzKeys<D>(b + SM::HI, b + SM::LO), 0, Core::MT);
    if (nvalid == KT) core.template softmax_step<true, false>(bias, p.sc2, 0, nvalid);
    else core.template softmax_step<true, true>(bias, p.sc2, 0, nvalid);
    if constexpr (WITH_PV) {
      const SwzValuesT<D> vv(b + SM::U, b + SM::U);
      if (nvalid == KT) core.template pv<false>(vv, 0, nvalid);
      else core.template pv<true>(vv, 0, nvalid);
    }
    if (ch == nch - 1) {
      int sl, i, t, qg;
      decode(item, sl, i, t, qg);
      float lse2[NQ], h2[NQ];
      core.finish(lse2, h2, p.sc2);
      T* Y = static_cast<T*>(p.y) + (size_t)sl * p.N * D;
#pragma unroll
      for (int n = 0; n < NQ; ++n) {
        const int ll = row_of(qg, n);
        if (ll >= p.rt) continue;
        const int l = t * p.rt + ll;
        const int64_t tok = p.map.token(l, i);
        if (WITH_PV) {
#pragma unroll
          for (int dt = 0; dt < D / 16; ++dt) store4(Y + (size_t)tok * D + dt * 16 + 4 * g, core.o[n][dt]);
        }
        if (g == 0) {
          p.lse2[((size_t)sl * p.b2 + i) * p.b1 + l] = lse2[n];
          if (p.lse_out) p.lse_out[(size_t)sl * p.N + tok] = lse2[n] * LN2;
        }
      }
    }
    if (nitem >= nitems) break;
    item = nitem;
    ch = nchk;
  }
}

}  // namespace ma
