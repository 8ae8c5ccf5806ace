// MonarchAttention forward kernels for gfx950.
//
// Per (batch, head) slice the method runs, for each of its T steps,
//   stage 1 (R-update + aggregation), one problem per key block k (and per
//     sub-tile (t, s) when tiled): the b2 query rows qt[k, i, t, s] attend to
//     the keys of segment s of block k; the softmax rows are R, and the
//     kernel emits c = R K, u = R V (last step), the row entropy H_R, and the
//     row log-normaliser;
//   stage 2 (L-update + application), one problem per column i (and row
//     tile t): the queries q[l, i], l in tile t, attend to the b1*c2 "keys"
//     c[k, i, t, s] with additive per-key bias H_R; the softmax rows are L
//     and y = L u (last step), or only the row log-normalisers (earlier
//     steps, which feed the next query qt = L^T q / L^T 1).
// Both stages are block-local attention with at most one extra bias term, so
// they share one streamed design: keys in tiles of 64 through LDS, scores by
// MFMA with keys on the M dimension, online softmax in registers, and the
// weighted sums again by MFMA against the transposed value tile.
//
// Precision (bf16 inputs).  Scores of a peaked row are large, and the
// aggregate c = R K enters the next scores multiplied by |q|, so rounding R
// or c to bf16 moves L by about 1e-2.  With PRECISE, the c path carries
// about 16 significant bits: R is split into bf16 hi + lo parts for the R K
// product (two MFMAs), c travels in fp32 and is split again into hi + lo keys
// for the stage-2 scores, and the next-step queries qt stay in fp32 (split on
// load).  u = R V and y = L u use plain bf16 operands.
//
// Sources: MonarchAttention (scime summary "Approach": batched matmuls and
// FlashAttention-like fused kernels; OpenReview author response on GQA/MLA:
// every intermediate step is a FlashAttention-like call on square-root-size
// blocks) and MonarchRT ("Method" part (2): tiled Monarch).
#pragma once

#include <type_traits>

#include "ma_device.hpp"

namespace ma {

template <typename T> constexpr bool is_bf16() { return std::is_same<T, bf16>::value; }

// Element type of the exchanged aggregate c.
template <typename T, bool PRECISE>
using XcT = typename std::conditional<(PRECISE || !is_bf16<T>()), float, T>::type;

__device__ inline void split_bf16(float x, bf16& hi, bf16& lo) {
  hi = (bf16)x;
  lo = (bf16)(x - (float)hi);
}

// ---------------------------------------------------------------------------
// LDS staging
// ---------------------------------------------------------------------------
template <typename T, int D, int DV, bool KLO>
struct alignas(16) TileSmem {
  static constexpr int LDK = D + 16 / (int)sizeof(T);   // +16 bytes per row
  static constexpr int LDV = KT + 4;                     // +4 elements per row
  T ks[KT][LDK];                 // key tile, row major: ks[key][dim]
  T ks_lo[KLO ? KT : 1][LDK];    // low parts of split keys
  T vt[DV][LDV];                 // value tile, transposed: vt[dim][key]
  float bias[KT];                // per-key additive score (base-2 units)
};

// dst[j][.] = row(j)[0 .. D) for j < nvalid, zero for nvalid <= j < KT.
template <typename T, int D, int LD, class RowFn>
__device__ inline void load_rows(T (*dst)[LD], int nvalid, RowFn row) {
  typedef typename Vec16<T>::type V;
  constexpr int VN = Vec16<T>::N;
  constexpr int CH = D / VN;
  for (int task = threadIdx.x; task < KT * CH; task += THREADS) {
    const int j = task / CH, c = task % CH;
    V v = {};
    if (j < nvalid) v = *reinterpret_cast<const V*>(row(j) + c * VN);
    *reinterpret_cast<V*>(&dst[j][c * VN]) = v;
  }
}

// fp32 rows split into bf16 hi / lo tiles.
template <int D, int LD, class RowFn>
__device__ inline void load_rows_split(bf16 (*hi)[LD], bf16 (*lo)[LD], int nvalid, RowFn row) {
  constexpr int CH = D / 4;
  for (int task = threadIdx.x; task < KT * CH; task += THREADS) {
    const int j = task / CH, c = task % CH;
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (j < nvalid) v = *reinterpret_cast<const f32x4*>(row(j) + c * 4);
    bf16x4 h, l;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      bf16 a, b;
      split_bf16(v[e], a, b);
      h[e] = a;
      l[e] = b;
    }
    *reinterpret_cast<bf16x4*>(&hi[j][c * 4]) = h;
    *reinterpret_cast<bf16x4*>(&lo[j][c * 4]) = l;
  }
}

// dst[off + e][j] = row(j)[e] for e < D, j < nvalid (zero for j >= nvalid).
template <typename T, int D, int LD, class RowFn>
__device__ inline void load_rows_transposed(T (*dst)[LD], int off, int nvalid, RowFn row) {
  typedef typename Vec16<T>::type V;
  constexpr int VN = Vec16<T>::N;
  constexpr int CH = D / VN;
  for (int task = threadIdx.x; task < (KT / 4) * CH; task += THREADS) {
    const int jq = task / CH, c = task % CH;
    V v[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = 4 * jq + r;
      v[r] = V{};
      if (j < nvalid) v[r] = *reinterpret_cast<const V*>(row(j) + c * VN);
    }
#pragma unroll
    for (int e = 0; e < VN; ++e) {
      typedef T T4 __attribute__((ext_vector_type(4)));
      T4 w;
      w[0] = v[0][e]; w[1] = v[1][e]; w[2] = v[2][e]; w[3] = v[3][e];
      *reinterpret_cast<T4*>(&dst[off + c * VN + e][4 * jq]) = w;
    }
  }
}

// A query row for the score MFMA: either exact input values (T) or an fp32
// row (next-step queries, tile means) that is split into hi + lo for bf16.
template <typename T> struct QSrc {
  const T* t;
  const float* f;
};

// ---------------------------------------------------------------------------
// Streamed attention core: one wave owns NQ sub-tiles of 16 queries.
//   KLO    keys carry a low part (extra MFMA per score step)
//   NSPLIT the first NSPLIT value sub-tiles use hi + lo probabilities
// ---------------------------------------------------------------------------
template <typename T, int D, int DV, int NQ, bool ENTROPY, bool WITH_PV, bool KLO, int NSPLIT>
struct FlashCore {
  typedef Mfma<T> MM;
  typedef typename MM::frag frag;
  static constexpr int KPL = MM::KPL;
  static constexpr int KSTEP = 4 * KPL;
  static constexpr int NKS = D / KSTEP;     // MFMA steps over the head dim
  static constexpr int MT = KT / 16;        // key sub-tiles per tile
  static constexpr int DT = DV / 16;        // value sub-tiles
  static_assert(KPL == 8 || (!KLO && NSPLIT == 0), "split precision is for bf16 only");

  frag qf[NQ][NKS];       // query fragments (B operand of S^T = K Q^T)
  frag qlo[NQ][NKS];      // low parts (when qsplit)
  bool qsplit;
  f32x4 o[NQ][DT];        // O^T accumulators: lane holds O[q][16dt + 4g + r]
  float m[NQ], l[NQ], e[NQ];

  __device__ inline void init() {
#pragma unroll
    for (int n = 0; n < NQ; ++n) {
      m[n] = -INFINITY; l[n] = 0.f; e[n] = 0.f;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[n][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }

  // qrow(n) -> QSrc of this lane's query in sub-tile n ({nullptr, nullptr}
  // for a padding query: zeros).  split: the sources are fp32 rows
  // (uniform over the workgroup).
  template <class QRow>
  __device__ inline void load_queries(QRow qrow, bool split) {
    const int g = (threadIdx.x % WAVE) / 16;
    qsplit = split && KPL == 8;
#pragma unroll
    for (int n = 0; n < NQ; ++n) {
      const QSrc<T> src = qrow(n);
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
        frag f = {}, fl = {};
        const int off = s * KSTEP + g * KPL;
        if (src.t) {
          f = *reinterpret_cast<const frag*>(src.t + off);
        } else if (src.f) {
          if constexpr (KPL == 8) {
            const f32x4 a = *reinterpret_cast<const f32x4*>(src.f + off);
            const f32x4 b = *reinterpret_cast<const f32x4*>(src.f + off + 4);
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
              bf16 h, lo;
              split_bf16(a[e2], h, lo); f[e2] = h; fl[e2] = lo;
              split_bf16(b[e2], h, lo); f[4 + e2] = h; fl[4 + e2] = lo;
            }
          } else {
            f = from_f32<T>(src.f[off]);
          }
        }
        qf[n][s] = f;
        qlo[n][s] = fl;
      }
    }
  }

  // One key tile (already in LDS).  sc2 = score scale in base-2 units;
  // nvalid = valid keys in this tile; bias from LDS if HAS_BIAS.
  template <int LDK, int LDV, bool HAS_BIAS>
  __device__ inline void tile(const T (*ks)[LDK], const T (*ks_lo)[LDK], const T (*vt)[LDV],
                              const float* bias, float sc2, int nvalid) {
    const int lane = threadIdx.x % WAVE, mrow = lane % 16, g = lane / 16;
    f32x4 s[NQ][MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int n = 0; n < NQ; ++n) s[n][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks_ = 0; ks_ < NKS; ++ks_) {
        const frag a = *reinterpret_cast<const frag*>(&ks[mt * 16 + mrow][ks_ * KSTEP + g * KPL]);
#pragma unroll
        for (int n = 0; n < NQ; ++n) {
          s[n][mt] = MM::mma(a, qf[n][ks_], s[n][mt]);
          if (qsplit) s[n][mt] = MM::mma(a, qlo[n][ks_], s[n][mt]);
        }
        if constexpr (KLO) {
          const frag al = *reinterpret_cast<const frag*>(&ks_lo[mt * 16 + mrow][ks_ * KSTEP + g * KPL]);
#pragma unroll
          for (int n = 0; n < NQ; ++n) s[n][mt] = MM::mma(al, qf[n][ks_], s[n][mt]);
        }
      }
    }
#pragma unroll
    for (int n = 0; n < NQ; ++n) {
      float tmax = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = mt * 16 + 4 * g + r;
          float z = s[n][mt][r] * sc2;
          if constexpr (HAS_BIAS) z += bias[key];
          if (key >= nvalid) z = -INFINITY;
          s[n][mt][r] = z;
          tmax = fmaxf(tmax, z);
        }
      }
      tmax = wave_max_x16x32(tmax);
      const float mnew = fmaxf(m[n], tmax);
      const float resc = __builtin_amdgcn_exp2f(m[n] - mnew);
      if (ENTROPY) e[n] = resc * (e[n] + (l[n] > 0.f ? (m[n] - mnew) * l[n] : 0.f));
      l[n] *= resc;
      if (WITH_PV) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[n][dt] *= resc;
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float z = s[n][mt][r];
          const float p = __builtin_amdgcn_exp2f(z - mnew);
          l[n] += p;
          if (ENTROPY && z > -INFINITY) e[n] += p * (z - mnew);
          s[n][mt][r] = p;
        }
      }
      m[n] = mnew;
    }
    if (!WITH_PV) return;
    if constexpr (KPL == 8) {
      // 32 keys per MFMA: lane group g supplies keys {32kk+4g+r, 32kk+16+4g+r}
#pragma unroll
      for (int kk = 0; kk < KT / 32; ++kk) {
        frag b[NQ], bl[NQ];
#pragma unroll
        for (int n = 0; n < NQ; ++n) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            if constexpr (NSPLIT > 0) {
              bf16 h, lo;
              split_bf16(s[n][2 * kk][r], h, lo); b[n][r] = h; bl[n][r] = lo;
              split_bf16(s[n][2 * kk + 1][r], h, lo); b[n][4 + r] = h; bl[n][4 + r] = lo;
            } else {
              b[n][r] = (bf16)s[n][2 * kk][r];
              b[n][4 + r] = (bf16)s[n][2 * kk + 1][r];
            }
          }
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const bf16x4 lo4 = *reinterpret_cast<const bf16x4*>(&vt[dt * 16 + mrow][32 * kk + 4 * g]);
          const bf16x4 hi4 = *reinterpret_cast<const bf16x4*>(&vt[dt * 16 + mrow][32 * kk + 16 + 4 * g]);
          frag a;
#pragma unroll
          for (int r = 0; r < 4; ++r) { a[r] = lo4[r]; a[4 + r] = hi4[r]; }
#pragma unroll
          for (int n = 0; n < NQ; ++n) {
            o[n][dt] = MM::mma(a, b[n], o[n][dt]);
            if (dt < NSPLIT) o[n][dt] = MM::mma(a, bl[n], o[n][dt]);
          }
        }
      }
    } else {
      // fp32: 4 keys per MFMA: lane group g supplies key 16mt + 4g + r
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            const float a = to_f32(vt[dt * 16 + mrow][mt * 16 + 4 * g + r]);
#pragma unroll
            for (int n = 0; n < NQ; ++n) o[n][dt] = MM::mma(a, s[n][mt][r], o[n][dt]);
          }
        }
      }
    }
  }

  // Totals over the four lanes of each query; normalise O.
  // lse2 = log2 sum 2^z (base-2 normaliser), h2 = entropy in bits.
  __device__ inline void finish(float (&lse2)[NQ], float (&h2)[NQ]) {
#pragma unroll
    for (int n = 0; n < NQ; ++n) {
      const float lt = wave_sum_x16x32(l[n]);
      const float et = ENTROPY ? wave_sum_x16x32(e[n]) : 0.f;
      const float inv = 1.f / lt;
      const float lg = __builtin_amdgcn_logf(lt);
      lse2[n] = m[n] + lg;
      h2[n] = lg - et * inv;
      if (WITH_PV) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[n][dt] *= inv;
      }
    }
  }
};

// ---------------------------------------------------------------------------
// Stage 1: R-update and aggregation
// ---------------------------------------------------------------------------
struct Stage1Params {
  const void* q; const void* k; const void* v;   // [S, N, D]
  const float* qtil;     // qt buffer [S, b1, c1, c2, b2, D] fp32 (steps after the first)
  const float* qbar;     // tile means [S, c1, b2, D] fp32 (first step, c1 > 1)
  void* cx; void* ux;    // exchange c (XcT), u (T): [S, b2, c1, b1, c2, D]
  float* h2x;            // entropy (bits): [S, b2, c1, b1, c2]
  float* lser;           // stage-1 row normaliser (base 2), same layout
  GridMap map;
  int S, N, b1, b2, c1, c2, sw, rt, nqg;
  float sc2;
  int first_step;
};

template <typename T, int D, int NQ, bool WITH_U, bool PRECISE>
__global__ __launch_bounds__(THREADS) void stage1_kernel(Stage1Params p) {
  typedef XcT<T, PRECISE> XC;
  constexpr int DV = WITH_U ? 2 * D : D;
  constexpr int QG = WAVES * NQ * 16;
  constexpr int NSPLIT = (PRECISE && is_bf16<T>()) ? D / 16 : 0;
  typedef FlashCore<T, D, DV, NQ, true, true, false, NSPLIT> Core;
  typedef TileSmem<T, D, DV, false> Smem;
  __shared__ Smem sm;

  const uint32_t nwg = gridDim.x;
  uint32_t id = xcd_swizzle(blockIdx.x, nwg);
  const int qg = id % p.nqg; id /= p.nqg;
  const int s = id % p.c2; id /= p.c2;
  const int t = id % p.c1; id /= p.c1;
  const int k = id % p.b1; id /= p.b1;
  const int sl = id;

  const T* Q = static_cast<const T*>(p.q) + (size_t)sl * p.N * D;
  const T* K = static_cast<const T*>(p.k) + (size_t)sl * p.N * D;
  const T* V = static_cast<const T*>(p.v) + (size_t)sl * p.N * D;
  const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE, g = lane / 16;

  Core core;
  core.init();
  const int own_tile = k / p.rt;
  const bool from_input = p.first_step && t == own_tile;
  core.load_queries([&](int n) -> QSrc<T> {
    const int i = qg * QG + wave * NQ * 16 + n * 16 + lane % 16;
    if (i >= p.b2) return QSrc<T>{nullptr, nullptr};
    if (!p.first_step)
      return QSrc<T>{nullptr, p.qtil + (((((size_t)sl * p.b1 + k) * p.c1 + t) * p.c2 + s) * p.b2 + i) * D};
    if (from_input) return QSrc<T>{Q + (size_t)p.map.token(k, i) * D, nullptr};
    return QSrc<T>{nullptr, p.qbar + (((size_t)sl * p.c1 + t) * p.b2 + i) * D};
  }, PRECISE && !from_input);

  const int j0 = s * p.sw;
  for (int kt0 = 0; kt0 < p.sw; kt0 += KT) {
    const int nvalid = min(KT, p.sw - kt0);
    __syncthreads();
    load_rows<T, D>(sm.ks, nvalid, [&](int j) { return K + (size_t)p.map.token(k, j0 + kt0 + j) * D; });
    load_rows_transposed<T, D>(sm.vt, 0, nvalid,
                               [&](int j) { return K + (size_t)p.map.token(k, j0 + kt0 + j) * D; });
    if (WITH_U)
      load_rows_transposed<T, D>(sm.vt, D, nvalid,
                                 [&](int j) { return V + (size_t)p.map.token(k, j0 + kt0 + j) * D; });
    __syncthreads();
    core.template tile<Smem::LDK, Smem::LDV, false>(sm.ks, sm.ks_lo, sm.vt, nullptr, p.sc2, nvalid);
  }

  float lse2[NQ], h2[NQ];
  core.finish(lse2, h2);
#pragma unroll
  for (int n = 0; n < NQ; ++n) {
    const int i = qg * QG + wave * NQ * 16 + n * 16 + lane % 16;
    if (i >= p.b2) continue;
    const size_t row = ((((size_t)sl * p.b2 + i) * p.c1 + t) * p.b1 + k) * p.c2 + s;
    XC* C = static_cast<XC*>(p.cx) + row * D;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) store4(C + dt * 16 + 4 * g, core.o[n][dt]);
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

// ---------------------------------------------------------------------------
// Stage 2: L-update and application
// ---------------------------------------------------------------------------
struct Stage2Params {
  const void* q; void* y;            // [S, N, D]
  const void* cx; const void* ux;    // exchange [S, b2, c1, b1, c2, D]
  const float* h2x;                  // [S, b2, c1, b1, c2]
  float* lse2;                       // [S, b2, b1] row normaliser (base 2)
  float* lse_out;                    // optional [S, N] natural log, token order
  GridMap map;
  int S, N, b1, b2, c1, c2, rt, nkeys, nqg;
  float sc2;
};

template <typename T, int D, int NQ, bool WITH_PV, bool PRECISE>
__global__ __launch_bounds__(THREADS) void stage2_kernel(Stage2Params p) {
  typedef XcT<T, PRECISE> XC;
  constexpr bool KLO = PRECISE && is_bf16<T>();
  constexpr int DV = D;
  constexpr int QG = WAVES * NQ * 16;
  typedef FlashCore<T, D, DV, NQ, false, WITH_PV, KLO, 0> Core;
  typedef TileSmem<T, D, DV, KLO> Smem;
  __shared__ Smem sm;

  const uint32_t nwg = gridDim.x;
  uint32_t id = xcd_swizzle(blockIdx.x, nwg);
  const int qg = id % p.nqg; id /= p.nqg;
  const int t = id % p.c1; id /= p.c1;
  const int i = id % p.b2; id /= p.b2;
  const int sl = id;

  const T* Q = static_cast<const T*>(p.q) + (size_t)sl * p.N * D;
  const size_t base = (((size_t)sl * p.b2 + i) * p.c1 + t) * (size_t)p.b1 * p.c2;
  const XC* C = static_cast<const XC*>(p.cx) + base * D;
  const T* U = static_cast<const T*>(p.ux) + base * D;
  const float* H = p.h2x + base;
  const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE, g = lane / 16;

  Core core;
  core.init();
  core.load_queries([&](int n) -> QSrc<T> {
    const int ll = qg * QG + wave * NQ * 16 + n * 16 + lane % 16;
    if (ll >= p.rt) return QSrc<T>{nullptr, nullptr};
    return QSrc<T>{Q + (size_t)p.map.token(t * p.rt + ll, i) * D, nullptr};
  }, false);

  for (int kt0 = 0; kt0 < p.nkeys; kt0 += KT) {
    const int nvalid = min(KT, p.nkeys - kt0);
    __syncthreads();
    if constexpr (KLO)
      load_rows_split<D>(sm.ks, sm.ks_lo, nvalid, [&](int j) { return C + (size_t)(kt0 + j) * D; });
    else
      load_rows<T, D>(sm.ks, nvalid, [&](int j) { return C + (size_t)(kt0 + j) * D; });
    if (WITH_PV)
      load_rows_transposed<T, D>(sm.vt, 0, nvalid, [&](int j) { return U + (size_t)(kt0 + j) * D; });
    if (threadIdx.x < KT) sm.bias[threadIdx.x] = threadIdx.x < nvalid ? H[kt0 + threadIdx.x] : 0.f;
    __syncthreads();
    core.template tile<Smem::LDK, Smem::LDV, true>(sm.ks, sm.ks_lo, sm.vt, sm.bias, p.sc2, nvalid);
  }

  float lse2[NQ], h2[NQ];
  core.finish(lse2, h2);
  T* Y = static_cast<T*>(p.y) + (size_t)sl * p.N * D;
#pragma unroll
  for (int n = 0; n < NQ; ++n) {
    const int ll = qg * QG + wave * NQ * 16 + n * 16 + lane % 16;
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

// ---------------------------------------------------------------------------
// Column reduction for the next step's queries, and the L export:
//   L[i,l,(k,s)] = 2^(w2 - lse2[l]),  w2 = sc2 * q[l,i].c[k,i,t,s] + h2[k,i,t,s]
//   qt[k,i,t,s]  = sum_{l in t} L q[l,i] / sum_{l in t} L
// One workgroup per (slice, column i, tile t, 64 keys); each wave owns 16
// keys and streams the query rows of tile t in chunks of 32.
// ---------------------------------------------------------------------------
struct AlphaParams {
  const void* q; const void* cx; const float* h2x; const float* lse2;
  const float* qbar;    // [S, c1, b2, D] fallback for zero weight
  float* qt_out;        // [S, b1, c1, c2, b2, D] or null
  float* L_out;         // [S, b2, b1, b1*c2] or null
  GridMap map;
  int S, N, b1, b2, c1, c2, rt, nkeys, nkt;
  float sc2;
};

template <typename T, int D, bool PRECISE>
__global__ __launch_bounds__(THREADS) void alpha_kernel(AlphaParams p) {
  typedef Mfma<T> MM;
  typedef typename MM::frag frag;
  typedef XcT<T, PRECISE> XC;
  constexpr bool SPLIT = PRECISE && is_bf16<T>();
  constexpr int KPL = MM::KPL, KSTEP = 4 * KPL, NKS = D / KSTEP;
  constexpr int QT = 32;
  constexpr int LDQ = D + 16 / (int)sizeof(T);
  constexpr int LDT = QT + 4;
  __shared__ __attribute__((aligned(16))) T qs[QT][LDQ];    // query chunk, row major
  __shared__ __attribute__((aligned(16))) T qtr[D][LDT];    // query chunk, transposed
  __shared__ float lq[QT];

  const uint32_t nwg = gridDim.x;
  uint32_t id = xcd_swizzle(blockIdx.x, nwg);
  const int kt = id % p.nkt; id /= p.nkt;
  const int t = id % p.c1; id /= p.c1;
  const int i = id % p.b2; id /= p.b2;
  const int sl = id;

  const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE, mrow = lane % 16, g = lane / 16;
  const int key = kt * KT + wave * 16 + mrow;
  const bool kvalid = key < p.nkeys;
  const size_t base = (((size_t)sl * p.b2 + i) * p.c1 + t) * (size_t)p.b1 * p.c2;
  const T* Q = static_cast<const T*>(p.q) + (size_t)sl * p.N * D;
  const XC* Crow = static_cast<const XC*>(p.cx) + (base + (kvalid ? key : 0)) * D;

  frag cf[NKS], cl[NKS];
#pragma unroll
  for (int s_ = 0; s_ < NKS; ++s_) {
    cf[s_] = frag{};
    cl[s_] = frag{};
    if (!kvalid) continue;
    const int off = s_ * KSTEP + g * KPL;
    if constexpr (SPLIT) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(Crow + off);
      const f32x4 b = *reinterpret_cast<const f32x4*>(Crow + off + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        bf16 h, lo;
        split_bf16(a[e], h, lo); cf[s_][e] = h; cl[s_][e] = lo;
        split_bf16(b[e], h, lo); cf[s_][4 + e] = h; cl[s_][4 + e] = lo;
      }
    } else if constexpr (KPL == 8) {
      cf[s_] = *reinterpret_cast<const frag*>(Crow + off);
    } else {
      cf[s_] = from_f32<T>(to_f32(Crow[off]));
    }
  }
  const float hk = kvalid ? p.h2x[base + key] : 0.f;
  f32x4 acc[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float beta = 0.f;

  for (int q0 = 0; q0 < p.rt; q0 += QT) {
    const int nq = min(QT, p.rt - q0);
    __syncthreads();
    auto qrow = [&](int j) { return Q + (size_t)p.map.token(t * p.rt + q0 + j, i) * D; };
    {
      typedef typename Vec16<T>::type V;
      constexpr int VN = Vec16<T>::N, CH = D / VN;
      for (int task = threadIdx.x; task < QT * CH; task += THREADS) {
        const int j = task / CH, c = task % CH;
        V v = {};
        if (j < nq) v = *reinterpret_cast<const V*>(qrow(j) + c * VN);
        *reinterpret_cast<V*>(&qs[j][c * VN]) = v;
#pragma unroll
        for (int e = 0; e < VN; ++e) qtr[c * VN + e][j] = v[e];
      }
    }
    if (threadIdx.x < QT)
      lq[threadIdx.x] = threadIdx.x < nq
          ? p.lse2[((size_t)sl * p.b2 + i) * p.b1 + t * p.rt + q0 + threadIdx.x] : INFINITY;
    __syncthreads();

    float Lv[2][4];
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s_ = 0; s_ < NKS; ++s_) {
        const frag a = *reinterpret_cast<const frag*>(&qs[n * 16 + mrow][s_ * KSTEP + g * KPL]);
        sacc = MM::mma(a, cf[s_], sacc);
        if constexpr (SPLIT) sacc = MM::mma(a, cl[s_], sacc);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int qq = n * 16 + 4 * g + r;
        float lv = __builtin_amdgcn_exp2f(sacc[r] * p.sc2 + hk - lq[qq]);
        if (!kvalid || qq >= nq) lv = 0.f;
        if (p.L_out && kvalid && qq < nq)
          p.L_out[(((size_t)sl * p.b2 + i) * p.b1 + t * p.rt + q0 + qq) * p.nkeys + key] = lv;
        if (KPL == 8 && !SPLIT) lv = (float)(bf16)lv;   // the value the MFMA consumes
        Lv[n][r] = lv;
        beta += lv;
      }
    }
    if (!p.qt_out) continue;
    if constexpr (KPL == 8) {
      frag b, bl;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if constexpr (SPLIT) {
          bf16 h, lo;
          split_bf16(Lv[0][r], h, lo); b[r] = h; bl[r] = lo;
          split_bf16(Lv[1][r], h, lo); b[4 + r] = h; bl[4 + r] = lo;
        } else {
          b[r] = (bf16)Lv[0][r];
          b[4 + r] = (bf16)Lv[1][r];
        }
      }
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        frag a;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          a[r] = qtr[dt * 16 + mrow][4 * g + r];
          a[4 + r] = qtr[dt * 16 + mrow][16 + 4 * g + r];
        }
        acc[dt] = MM::mma(a, b, acc[dt]);
        if constexpr (SPLIT) acc[dt] = MM::mma(a, bl, acc[dt]);
      }
    } else {
#pragma unroll
      for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int dt = 0; dt < D / 16; ++dt)
            acc[dt] = MM::mma(to_f32(qtr[dt * 16 + mrow][n * 16 + 4 * g + r]), Lv[n][r], acc[dt]);
    }
  }
  if (!p.qt_out || !kvalid) return;
  beta = wave_sum_x16x32(beta);
  const int k = key / p.c2, s = key % p.c2;
  float* out = p.qt_out + (((((size_t)sl * p.b1 + k) * p.c1 + t) * p.c2 + s) * p.b2 + i) * D;
  if (beta > 0.f) {
    const float inv = 1.f / beta;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) store4(out + dt * 16 + 4 * g, acc[dt] * inv);
  } else {
    const float* qb = p.qbar + (((size_t)sl * p.c1 + t) * p.b2 + i) * D;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
      store4(out + dt * 16 + 4 * g, *reinterpret_cast<const f32x4*>(qb + dt * 16 + 4 * g));
  }
}

// ---------------------------------------------------------------------------
// Small kernels: tile means of the queries, R export, objective.
// ---------------------------------------------------------------------------
struct QbarParams {
  const void* q; float* qbar;   // qbar [S, c1, b2, D] fp32
  GridMap map;
  int S, N, b2, c1, rt, D;
};

template <typename T>
__global__ __launch_bounds__(256) void qbar_kernel(QbarParams p) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t total = (size_t)p.S * p.c1 * p.b2 * p.D;
  if (idx >= total) return;
  const int d = idx % p.D;
  size_t r = idx / p.D;
  const int i = r % p.b2; r /= p.b2;
  const int t = r % p.c1;
  const int sl = r / p.c1;
  const T* Q = static_cast<const T*>(p.q) + (size_t)sl * p.N * p.D;
  float acc = 0.f;
  for (int ll = 0; ll < p.rt; ++ll) acc += to_f32(Q[(size_t)p.map.token(t * p.rt + ll, i) * p.D + d]);
  p.qbar[idx] = acc / (float)p.rt;
}

struct RExportParams {
  const void* q; const void* k; const float* qtil; const float* qbar;
  const float* lser;    // [S, b2, c1, b1, c2]
  float* R_out;         // [S, b1, b2, c1, b2]
  GridMap map;
  int S, N, b1, b2, c1, c2, sw, rt, D;
  float sc2;
  int first_step;
};

template <typename T>
__global__ __launch_bounds__(256) void r_export_kernel(RExportParams p) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t total = (size_t)p.S * p.b1 * p.b2 * p.c1 * p.b2;
  if (idx >= total) return;
  size_t r = idx;
  const int j = r % p.b2; r /= p.b2;
  const int t = r % p.c1; r /= p.c1;
  const int i = r % p.b2; r /= p.b2;
  const int k = r % p.b1;
  const int sl = r / p.b1;
  const int s = j / p.sw;
  const T* Q = static_cast<const T*>(p.q) + (size_t)sl * p.N * p.D;
  const T* K = static_cast<const T*>(p.k) + (size_t)sl * p.N * p.D;
  const T* krow = K + (size_t)p.map.token(k, j) * p.D;
  float dot = 0.f;
  if (p.first_step && t == k / p.rt) {
    const T* qrow = Q + (size_t)p.map.token(k, i) * p.D;
    for (int d = 0; d < p.D; ++d) dot += to_f32(qrow[d]) * to_f32(krow[d]);
  } else {
    const float* qrow = !p.first_step
        ? p.qtil + (((((size_t)sl * p.b1 + k) * p.c1 + t) * p.c2 + s) * p.b2 + i) * p.D
        : p.qbar + (((size_t)sl * p.c1 + t) * p.b2 + i) * p.D;
    for (int d = 0; d < p.D; ++d) dot += qrow[d] * to_f32(krow[d]);
  }
  const float ln = p.lser[((((size_t)sl * p.b2 + i) * p.c1 + t) * p.b1 + k) * p.c2 + s];
  p.R_out[idx] = __builtin_amdgcn_exp2f(dot * p.sc2 - ln);
}

struct ObjectiveParams {
  const float* lse2;    // [S, b2, b1]
  double* out;          // [S]
  int N;
};

__global__ __launch_bounds__(256) void objective_kernel(ObjectiveParams p) {
  __shared__ double part[256];
  const float* src = p.lse2 + (size_t)blockIdx.x * p.N;
  double acc = 0.0;
  for (int n = threadIdx.x; n < p.N; n += 256) acc += (double)src[n];
  part[threadIdx.x] = acc;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) p.out[blockIdx.x] = part[0] * 0.6931471805599453;
}

}  // namespace ma
