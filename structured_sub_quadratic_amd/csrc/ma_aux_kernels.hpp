// Auxiliary MonarchAttention kernels for gfx950: the column reduction that
// forms the next step's queries (and the L export), the tile means of the
// queries, the R export and the objective.
#pragma once

#include "ma_common.hpp"

namespace ma {

// ---------------------------------------------------------------------------
// Column reduction for the next step's queries, and the L export:
//   L[i,l,(k,s)] = 2^(w2 - lse2[l]),  w2 = sc2 * q[l,i].c[k,i,t,s] + h2[k,i,t,s]
//   qt[k,i,t,s]  = sum_{l in t} L q[l,i] / sum_{l in t} L
// (sums over real rows: padding rows have no L row and export zeros).
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
  size_t xlo;           // lo plane of split c (elements after cx)
  float* beta_out;      // [rows] column sums of L (exchange rows), or null
  int causal;           // 0, or grid blocks per causal unit (L is zero past causal_key_end)
};

template <typename T, int D, bool PRECISE>
__global__ __launch_bounds__(THREADS) void alpha_kernel(AlphaParams p) {
  typedef Mfma<T> MM;
  typedef typename MM::frag frag;
  constexpr bool SPLIT = split_x<T, PRECISE>();
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
  const size_t xrow = x_base(p.b1, p.b2, p.c1, p.c2, sl, t, i) + (size_t)(kvalid ? key : 0) * x_stride(p.b2, p.c1);
  const T* Q = static_cast<const T*>(p.q) + (size_t)sl * p.N * D;
  const T* Crow = static_cast<const T*>(p.cx) + xrow * D;

  frag cf[NKS], cl[NKS];
#pragma unroll
  for (int s_ = 0; s_ < NKS; ++s_) {
    cf[s_] = frag{};
    cl[s_] = frag{};
    if (!kvalid) continue;
    const int off = s_ * KSTEP + g * KPL;
    if constexpr (SPLIT) {
      cf[s_] = *reinterpret_cast<const frag*>(Crow + off);
      cl[s_] = *reinterpret_cast<const frag*>(Crow + p.xlo + off);
    } else if constexpr (KPL == 8) {
      cf[s_] = *reinterpret_cast<const frag*>(Crow + off);
    } else {
      cf[s_] = from_f32<T>(to_f32(Crow[off]));
    }
  }
  const float hk = kvalid ? p.h2x[xrow] : 0.f;
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
    // an infinite normaliser gives L = 0: rows past the tile and padding rows
    if (threadIdx.x < QT)
      lq[threadIdx.x] = threadIdx.x < nq && p.map.valid(t * p.rt + q0 + threadIdx.x, i)
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
        if (p.causal && key >= causal_key_end(t * p.rt + q0 + qq, p.causal, p.b1, p.c2)) lv = 0.f;
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
  if (p.beta_out && g == 0) p.beta_out[xrow] = beta;
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
// Tile means of the queries, qbar[t, i] = mean over the real rows l of tile t
// of q[l, i] (fp32; zero if the tile has none): one workgroup per (slice, t,
// i); 16 row lanes x D/VN column chunks, reduced through LDS.
// ---------------------------------------------------------------------------
struct QbarParams {
  const void* q; float* qbar;   // qbar [S, c1, b2, D] fp32
  GridMap map;
  int S, N, b2, c1, rt;
  void* qbar_lp;                // optional copy in the input type, same layout
};

template <typename T, int D>
struct QbarItem {
  typedef typename Vec16<T>::type V;
  static constexpr int VN = Vec16<T>::N, CH = D / VN, RL = 256 / CH;
  typedef float Smem[RL][D + 1];

  __device__ static inline int items(const QbarParams& p) { return p.S * p.c1 * p.b2; }

  __device__ static inline void run(const QbarParams& p, Smem& part, uint32_t id) {
    const int i = id % p.b2; id /= p.b2;
    const int t = id % p.c1;
    const int sl = id / p.c1;
    const T* Q = static_cast<const T*>(p.q) + (size_t)sl * p.N * D;
    const int c = threadIdx.x % CH, rl = threadIdx.x / CH;
    float acc[VN];
#pragma unroll
    for (int e = 0; e < VN; ++e) acc[e] = 0.f;
    const bool padded = p.map.padded();
    const int nreal = padded ? p.map.real_rows(i, t * p.rt, t * p.rt + p.rt) : p.rt;
    const AxisMap am = p.map.col_axis(i);
    for (int ll = rl; ll < p.rt; ll += RL) {
      const int l = t * p.rt + ll;
      if (padded && !am.valid(l)) continue;
      const V v = *reinterpret_cast<const V*>(Q + (size_t)am.at(l) * D + c * VN);
#pragma unroll
      for (int e = 0; e < VN; ++e) acc[e] += to_f32(v[e]);
    }
    const float inv = nreal > 0 ? 1.f / (float)nreal : 0.f;
#pragma unroll
    for (int e = 0; e < VN; ++e) part[rl][c * VN + e] = acc[e];
    __syncthreads();
    if (threadIdx.x < D) {
      float s = 0.f;
      for (int r = 0; r < RL; ++r) s += part[r][threadIdx.x];
      const size_t at = (((size_t)sl * p.c1 + t) * p.b2 + i) * D + threadIdx.x;
      p.qbar[at] = s * inv;
      if (p.qbar_lp) static_cast<T*>(p.qbar_lp)[at] = from_f32<T>(s * inv);
    }
    __syncthreads();
  }
};

template <typename T, int D>
__global__ __launch_bounds__(256) void qbar_kernel(QbarParams p) {
  __shared__ typename QbarItem<T, D>::Smem part;
  QbarItem<T, D>::run(p, part, blockIdx.x);
}

struct RExportParams {
  const void* q; const void* k; const float* qtil; const float* qbar;
  const float* lser;    // exchange rows (x_row)
  float* R_out;         // [S, b1, b2, c1, b2]
  GridMap map;
  int S, N, b1, b2, c1, c2, sw, rt, D;
  float sc2;
  int first_step;
  int heads, group;     // K slice of query slice sl: kv_slice(sl, heads, group)
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
  const T* K = static_cast<const T*>(p.k) + (size_t)kv_slice(sl, p.heads, p.group) * p.N * p.D;
  if (j < p.map.key_lo(k) || j >= p.map.key_hi(k)) {   // padding key: no weight
    p.R_out[idx] = 0.f;
    return;
  }
  const T* krow = K + (size_t)p.map.token(k, j) * p.D;
  float dot = 0.f;
  if (p.first_step && t == k / p.rt && p.map.valid(k, i)) {
    const T* qrow = Q + (size_t)p.map.token(k, i) * p.D;
    for (int d = 0; d < p.D; ++d) dot += to_f32(qrow[d]) * to_f32(krow[d]);
  } else {
    const float* qrow = !p.first_step
        ? p.qtil + (((((size_t)sl * p.b1 + k) * p.c1 + t) * p.c2 + s) * p.b2 + i) * p.D
        : p.qbar + (((size_t)sl * p.c1 + t) * p.b2 + i) * p.D;
    for (int d = 0; d < p.D; ++d) dot += qrow[d] * to_f32(krow[d]);
  }
  const float ln = p.lser[x_row(p.b1, p.b2, p.c1, p.c2, sl, k, s, t, i)];
  p.R_out[idx] = __builtin_amdgcn_exp2f(dot * p.sc2 - ln);
}

struct ObjectiveParams {
  const float* lse2;    // [S, b2, b1]
  double* out;          // [S]
  GridMap map;          // real rows only
};

static __global__ __launch_bounds__(256) void objective_kernel(ObjectiveParams p) {
  __shared__ double part[256];
  const int b1 = p.map.b1, G = p.map.b1 * p.map.b2;
  const float* src = p.lse2 + (size_t)blockIdx.x * G;
  double acc = 0.0;
  for (int n = threadIdx.x; n < G; n += 256)
    if (p.map.valid(n % b1, n / b1)) acc += (double)src[n];
  part[threadIdx.x] = acc;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) p.out[blockIdx.x] = part[0] * 0.6931471805599453;
}

}  // namespace ma
