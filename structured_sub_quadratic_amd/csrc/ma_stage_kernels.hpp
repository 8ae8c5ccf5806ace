// MonarchAttention forward: the two stages of every step, for gfx950.
//
// Per (batch, head) slice the method runs, for each of its T steps,
//   stage 1 (R-update + aggregation), one workgroup per key block k: the
//     query rows qt[k, i, t, s] (all i, all row tiles t) attend to the keys
//     of block k, one segment s at a time; the softmax rows are R, and the
//     kernel emits c = R K, u = R V (last step), the row entropy H_R, and the
//     row log-normaliser;
//   stage 2 (L-update + application), one workgroup per column i, row tile t
//     and 128 query rows: the queries q[l, i] attend to the b1*c2 "keys"
//     c[k, i, t, s] with additive per-key bias H_R, streamed in tiles of 64
//     with the next tile prefetched into registers; the softmax rows are L
//     and y = L u (last step), or only the row log-normalisers (earlier
//     steps, which feed the next query qt = L^T q / L^T 1).
// Scores are computed transposed by MFMA (keys on M, queries on N), so a lane
// owns one query and the four lanes l, l^16, l^32, l^48 share it: row
// reductions over keys are register-local plus two cross-lane steps.  The
// weighted sums are MFMAs against a transposed value tile in LDS.
//
// Sources: MonarchAttention (scime summary "Approach": batched matmuls and
// FlashAttention-like fused kernels; OpenReview author response on GQA/MLA:
// every intermediate step is a FlashAttention-like call on square-root-size
// blocks) and MonarchRT ("Method" part (2): tiled Monarch).
#pragma once

#include "ma_common.hpp"

namespace ma {

// ---------------------------------------------------------------------------
// Attention core: one wave owns NQ sub-tiles of 16 queries; KTL keys per
// LDS tile.
//   KLO    keys carry a low part (extra MFMA per score step)
//   NSPLIT the first NSPLIT value sub-tiles use hi + lo probabilities
// ---------------------------------------------------------------------------
template <typename T, int D, int DV, int NQ, int KTL, bool ENTROPY, bool WITH_PV, bool KLO,
          int NSPLIT, bool QSPLIT = false>
struct FlashCore {
  typedef Mfma<T> MM;
  typedef typename MM::frag frag;
  static constexpr int KPL = MM::KPL;
  static constexpr int KSTEP = 4 * KPL;
  static constexpr int NKS = D / KSTEP;     // MFMA steps over the head dim
  static constexpr int MT = KTL / 16;       // key sub-tiles per tile
  static constexpr int DT = DV / 16;        // value sub-tiles
  static_assert(KPL == 8 || (!KLO && NSPLIT == 0), "split precision is for bf16 only");
  static_assert(KTL % 32 == 0, "tile must hold whole 32-key MFMA steps");

  frag qf[NQ][NKS];       // query fragments (B operand of S^T = K Q^T)
  frag qlo[QSPLIT ? NQ : 1][QSPLIT ? NKS : 1];   // low parts (QSPLIT builds only)
  bool qsplit = false;
  f32x4 o[NQ][DT];        // O^T accumulators: lane holds O[q][16dt + 4g + r]
  f32x4 s[NQ][MT];        // score / probability tile
  f32x4 s2[NQ][MT];       // a second one (two tiles in flight; unused registers otherwise)
  template <int B> __device__ inline f32x4 (&buf())[NQ][MT] {
    if constexpr (B == 0) return s;
    else return s2;
  }
  float m[NQ], l[NQ], e[NQ];
  int qlim[NQ];           // QLIM steps: keys at or past qlim[n] (tile-local) are masked for query n
  bool fresh;             // no key seen since init()

  __device__ inline void init() {
    fresh = true;
#pragma unroll
    for (int n = 0; n < NQ; ++n) {
      m[n] = -INFINITY; l[n] = 0.f; e[n] = 0.f;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[n][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }

  typedef frag QLo[QSPLIT ? NQ : 1][QSPLIT ? NKS : 1];

  // Query fragments of this lane: qrow(n) -> QSrc of its query in sub-tile
  // n.  mode (uniform) decides which of the two rows every lane reads, so
  // all loads are issued back to back without branches.  fp32 rows are split
  // into hi + lo (lo kept only in QSPLIT builds).
  template <class QRow>
  __device__ static inline void fetch_queries(QRow qrow, int mode, frag (&f)[NQ][NKS], QLo& fl) {
    const int g = (threadIdx.x % WAVE) / 16;
    QSrc<T> src[NQ];
#pragma unroll
    for (int n = 0; n < NQ; ++n) src[n] = qrow(n);
    if (mode == Q_INPUT) {
#pragma unroll
      for (int n = 0; n < NQ; ++n)
#pragma unroll
        for (int s_ = 0; s_ < NKS; ++s_) {
          f[n][s_] = *reinterpret_cast<const frag*>(src[n].t + s_ * KSTEP + g * KPL);
          if constexpr (QSPLIT) fl[n][s_] = frag{};
        }
      return;
    }
    // fp32 rows (and, when mixed, input rows as well)
#pragma unroll
    for (int n = 0; n < NQ; ++n)
#pragma unroll
      for (int s_ = 0; s_ < NKS; ++s_) {
        const int off = s_ * KSTEP + g * KPL;
        frag h, lo;
        if constexpr (KPL == 8) {
          const f32x4 a = *reinterpret_cast<const f32x4*>(src[n].f + off);
          const f32x4 b = *reinterpret_cast<const f32x4*>(src[n].f + off + 4);
          const bf16x4 ha = __builtin_convertvector(a, bf16x4), hb = __builtin_convertvector(b, bf16x4);
          h = __builtin_shufflevector(ha, hb, 0, 1, 2, 3, 4, 5, 6, 7);
          lo = __builtin_shufflevector(__builtin_convertvector(a - __builtin_convertvector(ha, f32x4), bf16x4),
                                       __builtin_convertvector(b - __builtin_convertvector(hb, f32x4), bf16x4),
                                       0, 1, 2, 3, 4, 5, 6, 7);
        } else {
          h = from_f32<T>(src[n].f[off]);
          lo = frag{};
        }
        if (mode == Q_MIXED) {
          const frag hi_in = *reinterpret_cast<const frag*>(src[n].t + off);
          if (!src[n].use_f) { h = hi_in; lo = frag{}; }
        }
        f[n][s_] = h;
        if constexpr (QSPLIT) fl[n][s_] = lo;
      }
  }

  // split (uniform): the low parts of fp32 sources are used.
  template <class QRow>
  __device__ inline void load_queries(QRow qrow, int mode, bool split) {
    qsplit = QSPLIT && split && KPL == 8;
    fetch_queries(qrow, mode, qf, qlo);
  }

  __device__ inline void set_queries(const frag (&f)[NQ][NKS], const QLo& fl) {
#pragma unroll
    for (int n = 0; n < NQ; ++n)
#pragma unroll
      for (int s_ = 0; s_ < NKS; ++s_) {
        qf[n][s_] = f[n][s_];
        if constexpr (QSPLIT) qlo[n][s_] = fl[n][s_];
      }
  }

  // Raw scores S^T for the key sub-tiles [mt0, mt1) of a key tile; kv.a(mt,
  // ks) is this lane's A fragment of key sub-tile mt at head-dim step ks
  // (kv.alo the low part when KLO).
  // The head-dim steps are the outer loop, so the MFMAs of one step go to
  // independent accumulators (one per key sub-tile) and the operand reads of
  // a step are issued together; each accumulator still sums its steps in
  // order.
  template <int B = 0, class KV>
  __device__ inline void scores_v(const KV& kv, int mt0, int mt1) {
    f32x4 (&s)[NQ][MT] = buf<B>();
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if (mt < mt0 || mt >= mt1) continue;
#pragma unroll
      for (int n = 0; n < NQ; ++n) s[n][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int ks_ = 0; ks_ < NKS; ++ks_) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        if (mt < mt0 || mt >= mt1) continue;
        const frag a = kv.a(mt, ks_);
#pragma unroll
        for (int n = 0; n < NQ; ++n) {
          s[n][mt] = MM::mma(a, qf[n][ks_], s[n][mt]);
          if constexpr (QSPLIT) {
            if (qsplit) s[n][mt] = MM::mma(a, qlo[n][ks_], s[n][mt]);
          }
        }
        if constexpr (KLO) {
          const frag al = kv.alo(mt, ks_);
#pragma unroll
          for (int n = 0; n < NQ; ++n) s[n][mt] = MM::mma(al, qf[n][ks_], s[n][mt]);
        }
      }
    }
  }

  // Padded row-major key tiles in LDS (register-staged kernels).
  template <int LDK> struct PaddedKeys {
    const T (*ks)[LDK];
    const T (*ks_lo)[LDK];
    __device__ inline frag a(int mt, int ks_) const {
      const int lane = threadIdx.x % WAVE;
      return *reinterpret_cast<const frag*>(&ks[mt * 16 + lane % 16][ks_ * KSTEP + (lane / 16) * KPL]);
    }
    __device__ inline frag alo(int mt, int ks_) const {
      const int lane = threadIdx.x % WAVE;
      return *reinterpret_cast<const frag*>(&ks_lo[mt * 16 + lane % 16][ks_ * KSTEP + (lane / 16) * KPL]);
    }
  };

  template <int LDK>
  __device__ inline void scores(const T (*ks)[LDK], const T (*ks_lo)[LDK], int mt0, int mt1) {
    scores_v(PaddedKeys<LDK>{ks, ks_lo}, mt0, mt1);
  }

  // Online-softmax update with the LDS keys [klo, khi) of the tile (scores
  // already in s for every sub-tile overlapping that range); sc2 = score
  // scale in base-2 units; bias (base-2) from LDS if HAS_BIAS; MASK: the
  // range does not cover the whole tile.
  //
  // The running maximum m is only raised when a new score exceeds it by more
  // than 8 (base 2), so most tiles skip the rescale of l, e and O; the
  // probabilities are then at most 2^8 (exact in fp32, same relative
  // precision in bf16) and the final normalisation divides them out.
  // Entropy: e = sum p z in raw score units; finish() turns it into
  // H = lse - sc2 * e / l (fp32 keeps its absolute error near 1e-6 bits for
  // scores of a few tens of bits).
  // Maxima and sums over the lane's 4*MT keys are pairwise trees, so the
  // dependent chains are short.
  // three-input maxima (one v_max3_f32 each) where a level has three left
  template <int K> __device__ static inline float tree_max(const float (&v)[K]) {
    if constexpr (K == 1) return v[0];
    else if constexpr (K == 2) return fmaxf(v[0], v[1]);
    else {
      constexpr int H = (K + 2) / 3;
      float h[H];
#pragma unroll
      for (int j = 0; j < H; ++j) {
        if (3 * j + 2 < K) h[j] = fmaxf(fmaxf(v[3 * j], v[3 * j + 1]), v[3 * j + 2]);
        else if (3 * j + 1 < K) h[j] = fmaxf(v[3 * j], v[3 * j + 1]);
        else h[j] = v[3 * j];
      }
      return tree_max(h);
    }
  }
  template <int K> __device__ static inline float tree_sum(const float (&v)[K]) {
    if constexpr (K == 1) return v[0];
    else {
      float h[K / 2];
#pragma unroll
      for (int j = 0; j < K / 2; ++j) h[j] = v[2 * j] + v[2 * j + 1];
      return tree_sum(h);
    }
  }

  // QLIM (with MASK): each query n also masks the keys at or past qlim[n]
  // (block-causal use: the keys a query row may attend to end at a bound of
  // its own); the first tile of every row must keep at least one key.
  template <bool HAS_BIAS, bool MASK, int B = 0, bool QLIM = false>
  __device__ inline void softmax_step(const float* bias, float sc2, int klo, int khi) {
    f32x4 (&s)[NQ][MT] = buf<B>();
    constexpr float TAU = 8.f;
    constexpr float MASKED = -1e30f;
    const int lane = threadIdx.x % WAVE, g = lane / 16;
#pragma unroll
    for (int n = 0; n < NQ; ++n) {
      float zs[4 * MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float z = s[n][mt][r];
          if constexpr (HAS_BIAS) z = fmaf(z, sc2, bias[mt * 16 + 4 * g + r]);
          if constexpr (MASK) {
            const int key = mt * 16 + 4 * g + r;
            if (key < klo || key >= khi || (QLIM && key >= qlim[n])) z = MASKED;
          }
          s[n][mt][r] = z;
          zs[4 * mt + r] = z;
        }
      }
      float tmax = wave_max_x16x32(tree_max(zs));
      const float tm = HAS_BIAS ? tmax : tmax * sc2;          // base-2 units
      const bool raise = tm > m[n] + TAU;                       // true on the first tile
      const float mnew = raise ? tm : m[n];
      if (!fresh && __any(raise)) {
        const float resc = __builtin_amdgcn_exp2f(m[n] - mnew);
        l[n] *= resc;
        if (ENTROPY) e[n] *= resc;
        if (WITH_PV) {
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) o[n][dt] *= resc;
        }
      }
      m[n] = mnew;
      float ps[4 * MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float z = s[n][mt][r];
          const float p = HAS_BIAS ? __builtin_amdgcn_exp2f(z - mnew)
                                   : __builtin_amdgcn_exp2f(fmaf(z, sc2, -mnew));
          ps[4 * mt + r] = p;
          s[n][mt][r] = p;
        }
      }
      l[n] += tree_sum(ps);
      if (ENTROPY) {
        // sum p z over the tile: pairs as one multiply and one fma
        float pz[2 * MT];
#pragma unroll
        for (int j = 0; j < 2 * MT; ++j) pz[j] = fmaf(ps[2 * j], zs[2 * j], ps[2 * j + 1] * zs[2 * j + 1]);
        e[n] += tree_sum(pz);
      }
    }
    fresh = false;
  }

  // Value tile transposed in padded LDS rows (register-staged kernels).
  template <int LDV> struct PaddedVT {
    const T (*vt)[LDV];
    // A fragment of V^T for value sub-tile dt and keys {32kk+4g+r, 32kk+16+4g+r}
    __device__ inline frag at(int dt, int kk) const {
      const int lane = threadIdx.x % WAVE, mrow = lane % 16, g = lane / 16;
      const bf16x4 lo4 = *reinterpret_cast<const bf16x4*>(&vt[dt * 16 + mrow][32 * kk + 4 * g]);
      const bf16x4 hi4 = *reinterpret_cast<const bf16x4*>(&vt[dt * 16 + mrow][32 * kk + 16 + 4 * g]);
      return __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    __device__ inline float scalar(int dt, int key) const {
      return to_f32(vt[dt * 16 + (threadIdx.x % WAVE) % 16][key]);
    }
  };

  template <int LDV, bool HAS_BIAS, bool MASK>
  __device__ inline void update(const T (*vt)[LDV], const float* bias, float sc2, int klo, int khi) {
    softmax_step<HAS_BIAS, MASK>(bias, sc2, klo, khi);
    if constexpr (WITH_PV) pv<MASK>(PaddedVT<LDV>{vt}, klo, khi);
  }

  // O^T += V^T P^T over the keys [klo, khi) of the tile (probabilities in s).
  template <bool MASK, int B = 0, class VV>
  __device__ inline void pv(const VV& vv, int klo, int khi) {
    f32x4 (&s)[NQ][MT] = buf<B>();
    const int lane = threadIdx.x % WAVE, g = lane / 16;
    if constexpr (KPL == 8) {
      // 32 keys per MFMA: lane group g supplies keys {32kk+4g+r, 32kk+16+4g+r}
#pragma unroll
      for (int kk = 0; kk < KTL / 32; ++kk) {
        if (MASK && (32 * kk >= khi || 32 * kk + 32 <= klo)) continue;
        frag b[NQ], bl[NQ];
#pragma unroll
        for (int n = 0; n < NQ; ++n) {
          const bf16x4 h0 = __builtin_convertvector(s[n][2 * kk], bf16x4);
          const bf16x4 h1 = __builtin_convertvector(s[n][2 * kk + 1], bf16x4);
          b[n] = __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7);
          if constexpr (NSPLIT > 0) {
            const f32x4 r0 = s[n][2 * kk] - __builtin_convertvector(h0, f32x4);
            const f32x4 r1 = s[n][2 * kk + 1] - __builtin_convertvector(h1, f32x4);
            bl[n] = __builtin_shufflevector(__builtin_convertvector(r0, bf16x4),
                                            __builtin_convertvector(r1, bf16x4), 0, 1, 2, 3, 4, 5, 6, 7);
          }
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const frag a = vv.at(dt, kk);
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
        if (MASK && (16 * mt >= khi || 16 * mt + 16 <= klo)) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            const float a = vv.scalar(dt, mt * 16 + 4 * g + r);
#pragma unroll
            for (int n = 0; n < NQ; ++n) o[n][dt] = MM::mma(a, s[n][mt][r], o[n][dt]);
          }
        }
      }
    }
  }

  // Totals over the four lanes of each query; normalise O.
  // lse2 = log2 sum 2^z (base-2 normaliser), h2 = entropy in bits.
  __device__ inline void finish(float (&lse2)[NQ], float (&h2)[NQ], float sc2) {
#pragma unroll
    for (int n = 0; n < NQ; ++n) {
      const float lt = wave_sum_x16x32(l[n]);
      const float inv = 1.f / lt;
      const float lg = __builtin_amdgcn_logf(lt);
      lse2[n] = m[n] + lg;
      if (ENTROPY) {
        // H = lse2 - sc2 * (sum p z) / lt
        const float et = wave_sum_x16x32(e[n]);
        h2[n] = lse2[n] - sc2 * et * inv;
      } else {
        h2[n] = 0.f;
      }
      if (WITH_PV) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[n][dt] *= inv;
      }
    }
  }
};

// ---------------------------------------------------------------------------
// Stage 1: R-update and aggregation, one workgroup per (slice, block k,
// group of query slots).  Slot = t*b2 + i.  When the whole block fits one
// LDS tile (b2 <= KTB) its keys are loaded once and every segment s is a key
// range of that tile; otherwise each segment is loaded on its own.
// ---------------------------------------------------------------------------
struct Stage1Params {
  const void* q; const void* k; const void* v;   // [S, N, D]
  const float* qtil;     // qt buffer [S, b1, c1, c2, b2, D] fp32 (steps after the first)
  const float* qbar;     // tile means [S, c1, b2, D] fp32 (first step, c1 > 1)
  void* cx; void* ux;    // exchange c, u (T): x_row rows of D; the lo plane
                         // of split c starts xlo elements after cx
  float* h2x;            // entropy (bits), one per exchange row
  float* lser;           // stage-1 row normaliser (base 2), same layout
  GridMap map;
  int S, N, b1, b2, c1, c2, sw, rt, nqs, nqg;
  float sc2;
  int first_step;
  size_t xlo;
  const void* qbar_lp;   // tile means in the input type (first tiled step, plain c path)
  int heads, group;      // K/V slice of query slice sl: kv_slice(sl, heads, group)
};

template <typename T, int D, int DV, int KTB>
struct alignas(16) Stage1Smem {
  static constexpr int LDK = D + pad16<T>();
  static constexpr int LDV = KTB + 4;
  T ks[KTB][LDK];       // keys, row major
  T vt[DV][LDV];        // [K | V] transposed
};

// Query source of one stage-1 slot (every pointer valid; slots past the last
// read the last).  mode: Q_INPUT at the first step of untiled Monarch, Q_MIXED
// at the first tiled or padded step (own row tile from Q, other tiles and
// padding positions from the tile means), Q_F32 at later steps.  PAD: a
// padded flat sequence (padding positions clamped on load).
template <typename T, int D, bool PAD = false>
__device__ inline QSrc<T> stage1_qsrc(const Stage1Params& p, int sl, int k, int slot, int s) {
  slot = min(slot, p.nqs - 1);
  const int t = slot / p.b2, i = slot % p.b2;
  QSrc<T> r;
  const int64_t tok = PAD ? p.map.token(k, i) : p.map.template raw_token<false>(k, i);
  r.t = static_cast<const T*>(p.q) + ((size_t)sl * p.N + tok) * D;
  if (!p.first_step) {
    r.f = p.qtil + (((((size_t)sl * p.b1 + k) * p.c1 + t) * p.c2 + s) * p.b2 + i) * D;
    r.use_f = true;
  } else if (p.c1 > 1 || PAD) {
    r.f = p.qbar + (((size_t)sl * p.c1 + t) * p.b2 + i) * D;
    r.use_f = t != k / p.rt || (PAD && !p.map.valid(k, i));
  } else {
    r.f = nullptr;
    r.use_f = false;
  }
  return r;
}
template <bool PAD = false>
__device__ inline int stage1_qmode(const Stage1Params& p) {
  return !p.first_step ? Q_F32 : (p.c1 > 1 || PAD ? Q_MIXED : Q_INPUT);
}

// Keys (and values) j0 .. j0+nk of block k held by this thread: NT tasks of
// four rows x one 16-byte chunk.  Rows past nk repeat row j0 (their scores are
// masked); tasks past the tile are not stored.
template <typename T, int D, int KTB, bool WITH_U, bool PAD = false>
struct Stage1Keys {
  typedef typename Vec16<T>::type V;
  static constexpr int VN = Vec16<T>::N, CH = D / VN;
  static constexpr int NTASK = (KTB / 4) * CH;
  static constexpr int NT = (NTASK + THREADS - 1) / THREADS;
  V kv[NT][4], vv[WITH_U ? NT : 1][4];

  __device__ inline void load(const Stage1Params& p, const T* K, const T* Vv, int k, int j0, int nk) {
    size_t off[NT][4];
#pragma unroll
    for (int a = 0; a < NT; ++a) {
      const int task = min((int)threadIdx.x + a * THREADS, NTASK - 1);
      const int jq = task / CH, c = task % CH;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = min(4 * jq + r, nk - 1);
        const int64_t tok = PAD ? p.map.token(k, j0 + j) : p.map.template raw_token<false>(k, j0 + j);
        off[a][r] = (size_t)tok * D + c * VN;
      }
    }
#pragma unroll
    for (int a = 0; a < NT; ++a)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        kv[a][r] = *reinterpret_cast<const V*>(K + off[a][r]);
        if (WITH_U) vv[a][r] = *reinterpret_cast<const V*>(Vv + off[a][r]);
      }
  }

  template <class Smem>
  __device__ inline void store(Smem& sm) const {
#pragma unroll
    for (int a = 0; a < NT; ++a) {
      const int task = threadIdx.x + a * THREADS;
      if (task >= NTASK) continue;
      const int jq = task / CH, c = task % CH;
#pragma unroll
      for (int r = 0; r < 4; ++r) *reinterpret_cast<V*>(&sm.ks[4 * jq + r][c * VN]) = kv[a][r];
      store_transposed4<T, Smem::LDV>(sm.vt, 0, c, 4 * jq, kv[a]);
      if (WITH_U) store_transposed4<T, Smem::LDV>(sm.vt, D, c, 4 * jq, vv[a]);
    }
  }
};

// One segment of a stage-1 item: walk the LDS tile in chunks of KT keys over
// [klo, khi), then write c, u, H_R and the normaliser of every valid slot.
template <typename T, bool SPLITX, int D, int NQ, int KTB, bool WITH_U, class Core, class Smem>
__device__ inline void stage1_segment(Core& core, const Smem& sm, const Stage1Params& p, int sl,
                                      int k, int qg, int s, int klo, int khi) {
  const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE, g = lane / 16;
  constexpr int QG = WAVES * NQ * 16;
  core.init();
#pragma unroll
  for (int c0 = 0; c0 < KTB; c0 += KT) {
    if (c0 >= khi || c0 + KT <= klo) continue;
    const int lo = max(klo - c0, 0), hi = min(khi - c0, KT);
    core.template scores<Smem::LDK>(reinterpret_cast<const T (*)[Smem::LDK]>(&sm.ks[c0][0]), nullptr,
                                    lo / 16, (hi + 15) / 16);
    const T (*vtc)[Smem::LDV] = reinterpret_cast<const T (*)[Smem::LDV]>(&sm.vt[0][c0]);
    if (lo == 0 && hi == KT) core.template update<Smem::LDV, false, false>(vtc, nullptr, p.sc2, lo, hi);
    else core.template update<Smem::LDV, false, true>(vtc, nullptr, p.sc2, lo, hi);
  }
  float lse2[NQ], h2[NQ];
  core.finish(lse2, h2, p.sc2);
#pragma unroll
  for (int n = 0; n < NQ; ++n) {
    const int slot = qg * QG + wave * NQ * 16 + n * 16 + lane % 16;
    if (slot >= p.nqs) continue;
    const int t = slot / p.b2, i = slot % p.b2;
    const size_t row = x_row(p.b1, p.b2, p.c1, p.c2, sl, k, s, t, i);
    T* C = static_cast<T*>(p.cx) + row * D;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      if constexpr (SPLITX) {
        const f32x4 v = core.o[n][dt];
        const bf16x4 hi = __builtin_convertvector(v, bf16x4);
        const bf16x4 lo = __builtin_convertvector(v - __builtin_convertvector(hi, f32x4), bf16x4);
        *reinterpret_cast<bf16x4*>(C + dt * 16 + 4 * g) = hi;
        *reinterpret_cast<bf16x4*>(C + p.xlo + dt * 16 + 4 * g) = lo;
      } else {
        store4(C + dt * 16 + 4 * g, core.o[n][dt]);
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

template <typename T, int D, int NQ, int KTB, bool WITH_U, bool PRECISE, bool QSPLIT, bool PAD = false>
struct Stage1Item {
  static constexpr bool SPLITX = split_x<T, PRECISE>();
  static constexpr int DV = WITH_U ? 2 * D : D;
  static constexpr int QG = WAVES * NQ * 16;
  static constexpr int NSPLIT = (PRECISE && is_bf16<T>()) ? D / 16 : 0;
  // the LDS tile holds KTB keys; the core walks it in chunks of KT keys
  typedef FlashCore<T, D, DV, NQ, KT, true, true, false, NSPLIT, QSPLIT> Core;
  typedef Stage1Smem<T, D, DV, KTB> Smem;

  __device__ static inline int items(const Stage1Params& p) { return p.S * p.b1 * p.nqg; }

  // One item (slice, block k, query group); leaves LDS free on return.
  __device__ static inline void run(const Stage1Params& p, Smem& sm, uint32_t id) {
    const int qg = id % p.nqg; id /= p.nqg;
    const int k = id % p.b1; id /= p.b1;
    const int sl = id;
    const int kvs = kv_slice(sl, p.heads, p.group);
    const T* K = static_cast<const T*>(p.k) + (size_t)kvs * p.N * D;
    const T* Vv = static_cast<const T*>(p.v) + (size_t)kvs * p.N * D;
    const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE;
    const bool whole = p.b2 <= KTB;
    const int mode = stage1_qmode<PAD>(p);
    const bool split = PRECISE && mode != Q_INPUT;
    auto qrow = [&](int n, int s) {
      return stage1_qsrc<T, D, PAD>(p, sl, k, qg * QG + wave * NQ * 16 + n * 16 + lane % 16, s);
    };

    Stage1Keys<T, D, KTB, WITH_U, PAD> keys;
    Core core;
    core.load_queries([&](int n) { return qrow(n, 0); }, mode, split);
    if (whole) {
      keys.load(p, K, Vv, k, 0, p.b2);
      keys.store(sm);
    }
    for (int s = 0; s < p.c2; ++s) {
      // key range of segment s within the LDS tile
      int klo = 0, khi = p.sw;
      if constexpr (PAD) {     // real keys of block k
        klo = max(p.map.key_lo(k) - s * p.sw, 0);
        khi = min(p.map.key_hi(k) - s * p.sw, p.sw);
      }
      if (whole) {
        klo += s * p.sw;
        khi += s * p.sw;
      } else {
        __syncthreads();
        keys.load(p, K, Vv, k, s * p.sw, p.sw);
        keys.store(sm);
      }
      if (s > 0 && !p.first_step) core.load_queries([&](int n) { return qrow(n, s); }, mode, split);
      __syncthreads();
      stage1_segment<T, SPLITX, D, NQ, KTB, WITH_U>(core, sm, p, sl, k, qg, s, klo, khi);
    }
    __syncthreads();
  }
};

template <typename T, int D, int NQ, int KTB, bool WITH_U, bool PRECISE, bool QSPLIT, bool PAD = false>
__global__ __launch_bounds__(THREADS) void stage1_kernel(Stage1Params p) {
  typedef Stage1Item<T, D, NQ, KTB, WITH_U, PRECISE, QSPLIT, PAD> Item;
  __shared__ typename Item::Smem sm;
  Item::run(p, sm, xcd_swizzle(blockIdx.x, gridDim.x));
}

// ---------------------------------------------------------------------------
// Stage 2: L-update and application.  One workgroup per (slice, column i,
// row tile t, group of 64*NQ query rows); keys streamed in tiles of 64, the
// next tile's global loads in flight while the current tile computes.
// ---------------------------------------------------------------------------
struct Stage2Params {
  const void* q; void* y;            // [S, N, D]
  const void* cx; const void* ux;    // exchange, x_row rows of D
  const float* h2x;                  // entropy, one per exchange row
  float* lse2;                       // [S, b2, b1] row normaliser (base 2)
  float* lse_out;                    // optional [S, N] natural log, token order
  GridMap map;
  int S, N, b1, b2, c1, c2, rt, nkeys, nqg;
  float sc2;
  size_t xlo;                        // lo plane of split c (elements after cx)
  int causal;                        // 0, or grid blocks per causal unit (causal_key_end)
};

// Block-causal use: how one wave treats the stage-2 key chunk [base, base +
// nvalid) of row tile t.  Its query rows (within the tile) start at r0 and
// row(n) is the row of this lane in sub-tile n.  Returns CH_SKIP when every
// row of the wave ends before the chunk (nothing to compute), CH_ROWMASK
// (core.qlim set to each row's bound relative to base) when the chunk
// crosses the bound of one of them, CH_WHOLE otherwise.
enum { CH_WHOLE = 0, CH_ROWMASK = 1, CH_SKIP = 2 };
template <int NQ, class Core, class RowFn>
__device__ inline int causal_chunk(Core& core, const Stage2Params& p, int t, int r0, RowFn row, int base,
                                   int nvalid) {
  if (!p.causal) return CH_WHOLE;
  if (r0 >= p.rt) return CH_SKIP;      // no real row in this wave (results unused)
  const int lo = causal_key_end(t * p.rt + r0, p.causal, p.b1, p.c2);
  const int hi = causal_key_end(t * p.rt + min(r0 + NQ * 16, p.rt) - 1, p.causal, p.b1, p.c2);
  if (base >= hi) return CH_SKIP;
  if (base + nvalid <= lo) return CH_WHOLE;
#pragma unroll
  for (int n = 0; n < NQ; ++n)
    core.qlim[n] = causal_key_end(t * p.rt + min(row(n), p.rt - 1), p.causal, p.b1, p.c2) - base;
  return CH_ROWMASK;
}

// Keys the rows [r0, r1) of row tile t read: all, or (block-causal) those
// below the bound of the last of them.
__device__ inline int stage2_keys(const Stage2Params& p, int t, int r1) {
  return p.causal ? causal_key_end(t * p.rt + min(r1, p.rt) - 1, p.causal, p.b1, p.c2) : p.nkeys;
}

template <typename T, int D, bool KLO, int KR = KT>
struct alignas(16) Stage2Smem {
  static constexpr int LDK = D + pad16<T>();
  static constexpr int LDV = KR + 4;
  T ks[KR][LDK];                 // key tile (hi parts when split)
  T ks_lo[KLO ? KR : 1][LDK];    // low parts of split keys
  T vt[D][LDV];                  // value tile, transposed
  float bias[KR];
};

// Register staging of one key tile of stage 2: c rows (hi and, when KLO, lo
// planes), u rows (four rows per task for the transposed store) and the
// bias.  Rows past nvalid repeat the last valid row (their scores are
// masked).
template <typename T, int D, bool WITH_PV, bool KLO, int KR = KT>
struct Stage2Prefetch {
  typedef typename Vec16<T>::type VT;
  static constexpr int VNT = Vec16<T>::N;
  static constexpr int TC = KR * (D / VNT);              // c chunks per tile
  static constexpr int NC = (TC + THREADS - 1) / THREADS;
  static constexpr int TU = (KR / 4) * (D / VNT);        // u tasks per tile
  static constexpr int NU = WITH_PV ? (TU + THREADS - 1) / THREADS : 0;
  VT c[NC], cl[KLO ? NC : 1];
  VT u[NU > 0 ? NU : 1][4];
  float h;

  // C, U, H address the tile's first key row; keys are xs rows apart.
  __device__ inline void load(const T* C, size_t xlo, const T* U, const float* H, int nvalid, size_t xs) {
#pragma unroll
    for (int a = 0; a < NC; ++a) {
      const int task = min((int)threadIdx.x + a * THREADS, TC - 1);
      const int j = min(task / (D / VNT), nvalid - 1), cc = task % (D / VNT);
      c[a] = *reinterpret_cast<const VT*>(C + (size_t)j * xs * D + cc * VNT);
      if constexpr (KLO) cl[a] = *reinterpret_cast<const VT*>(C + xlo + (size_t)j * xs * D + cc * VNT);
    }
#pragma unroll
    for (int a = 0; a < NU; ++a) {
      const int task = min((int)threadIdx.x + a * THREADS, TU - 1);
      const int jq = task / (D / VNT), cc = task % (D / VNT);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = min(4 * jq + r, nvalid - 1);
        u[a][r] = *reinterpret_cast<const VT*>(U + (size_t)j * xs * D + cc * VNT);
      }
    }
    h = H[(size_t)min((int)threadIdx.x, nvalid - 1) * xs];
  }

  template <class Smem>
  __device__ inline void store(Smem& sm) const {
#pragma unroll
    for (int a = 0; a < NC; ++a) {
      const int task = threadIdx.x + a * THREADS;
      if (task >= TC) continue;
      const int j = task / (D / VNT), cc = task % (D / VNT);
      *reinterpret_cast<VT*>(&sm.ks[j][cc * VNT]) = c[a];
      if constexpr (KLO) *reinterpret_cast<VT*>(&sm.ks_lo[j][cc * VNT]) = cl[a];
    }
#pragma unroll
    for (int a = 0; a < NU; ++a) {
      const int task = threadIdx.x + a * THREADS;
      if (task >= TU) continue;
      const int jq = task / (D / VNT), cc = task % (D / VNT);
      store_transposed4<T, Smem::LDV>(sm.vt, 0, cc, 4 * jq, u[a]);
    }
    if (threadIdx.x < KR) sm.bias[threadIdx.x] = h;
  }
};

// CLAMP: padding positions read a real row (their results are not stored)
template <typename T, int D, bool CLAMP>
__device__ inline QSrc<T> stage2_qsrc(const Stage2Params& p, int sl, int i, int t, int ll) {
  ll = min(ll, p.rt - 1);
  const int64_t tok = CLAMP ? p.map.token(t * p.rt + ll, i) : p.map.template raw_token<false>(t * p.rt + ll, i);
  return QSrc<T>{static_cast<const T*>(p.q) + ((size_t)sl * p.N + tok) * D, nullptr, false};
}

// Output of a stage-2 item: y rows (last step) and the row normalisers (PAD:
// no output at padding positions).
template <typename T, int D, int NQ, bool WITH_PV, bool PAD, class Core>
__device__ inline void stage2_store(const Core& core, const Stage2Params& p, const float (&lse2)[NQ],
                                    int sl, int i, int t, int qg) {
  const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE, g = lane / 16;
  constexpr int QG = WAVES * NQ * 16;
  T* Y = static_cast<T*>(p.y) + (size_t)sl * p.N * D;
#pragma unroll
  for (int n = 0; n < NQ; ++n) {
    const int ll = qg * QG + wave * NQ * 16 + n * 16 + lane % 16;
    if (ll >= p.rt) continue;
    const int l = t * p.rt + ll;
    const int64_t tok = PAD ? p.map.token(l, i) : p.map.template raw_token<false>(l, i);
    const bool real = !PAD || p.map.valid(l, i);
    if (WITH_PV && real) {
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) store4(Y + (size_t)tok * D + dt * 16 + 4 * g, core.o[n][dt]);
    }
    if (g == 0) {
      p.lse2[((size_t)sl * p.b2 + i) * p.b1 + l] = lse2[n];
      if (p.lse_out && real) p.lse_out[(size_t)sl * p.N + tok] = lse2[n] * LN2;
    }
  }
}

template <typename T, int D, int NQ, bool WITH_PV, bool PRECISE, bool PAD = false>
struct Stage2Item {
  static constexpr bool KLO = split_x<T, PRECISE>();
  static constexpr int QG = WAVES * NQ * 16;
  typedef FlashCore<T, D, D, NQ, KT, false, WITH_PV, KLO, 0> Core;
  typedef Stage2Smem<T, D, KLO> Smem;

  __device__ static inline int items(const Stage2Params& p) { return p.S * p.b2 * p.c1 * p.nqg; }

  // One item (slice, column i, row tile t, query group); leaves LDS free.
  __device__ static inline void run(const Stage2Params& p, Smem& sm, uint32_t id) {
    const int qg = id % p.nqg; id /= p.nqg;
    const int t = id % p.c1; id /= p.c1;
    const int i = id % p.b2; id /= p.b2;
    const int sl = id;

    const size_t base = x_base(p.b1, p.b2, p.c1, p.c2, sl, t, i), xs = x_stride(p.b2, p.c1);
    const T* C = static_cast<const T*>(p.cx) + base * D;
    const T* U = static_cast<const T*>(p.ux) + base * D;
    const float* H = p.h2x + base;
    const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE;

    Stage2Prefetch<T, D, WITH_PV, KLO> pf;
    pf.load(C, p.xlo, U, H, min(KT, p.nkeys), xs);

    Core core;
    core.init();
    auto row = [&](int n) { return qg * QG + wave * NQ * 16 + n * 16 + lane % 16; };
    core.load_queries([&](int n) { return stage2_qsrc<T, D, PAD>(p, sl, i, t, row(n)); }, Q_INPUT, false);

    const int kmax = stage2_keys(p, t, qg * QG + QG);
    for (int kt0 = 0; kt0 < kmax; kt0 += KT) {
      const int nvalid = min(KT, p.nkeys - kt0);
      __syncthreads();
      pf.store(sm);
      __syncthreads();
      if (kt0 + KT < kmax)
        pf.load(C + (size_t)(kt0 + KT) * xs * D, p.xlo, U + (size_t)(kt0 + KT) * xs * D,
                H + (size_t)(kt0 + KT) * xs, min(KT, p.nkeys - kt0 - KT), xs);
      const int how = causal_chunk<NQ>(core, p, t, row(0) - lane % 16, row, kt0, nvalid);
      if (how == CH_SKIP) continue;
      core.template scores<Smem::LDK>(sm.ks, sm.ks_lo, 0, Core::MT);
      if (how == CH_ROWMASK) {
        core.template softmax_step<true, true, 0, true>(sm.bias, p.sc2, 0, nvalid);
        if constexpr (WITH_PV) core.template pv<true>(typename Core::template PaddedVT<Smem::LDV>{sm.vt}, 0, nvalid);
      } else if (nvalid == KT) {
        core.template update<Smem::LDV, true, false>(sm.vt, sm.bias, p.sc2, 0, nvalid);
      } else {
        core.template update<Smem::LDV, true, true>(sm.vt, sm.bias, p.sc2, 0, nvalid);
      }
    }

    float lse2[NQ], h2[NQ];
    core.finish(lse2, h2, p.sc2);
    stage2_store<T, D, NQ, WITH_PV, PAD>(core, p, lse2, sl, i, t, qg);
    __syncthreads();
  }
};

template <typename T, int D, int NQ, bool WITH_PV, bool PRECISE, bool PAD = false>
__global__ __launch_bounds__(THREADS) void stage2_kernel(Stage2Params p) {
  typedef Stage2Item<T, D, NQ, WITH_PV, PRECISE, PAD> Item;
  __shared__ typename Item::Smem sm;
  Item::run(p, sm, xcd_swizzle(blockIdx.x, gridDim.x));
}

// ---------------------------------------------------------------------------
// Persistent variants for problems whose keys fit one LDS tile (stage 1:
// b2 <= KTB; stage 2: b1*c2 <= KTB).  Each workgroup walks its items with
// stride gridDim.x and keeps the next item's operands in flight (registers)
// while the current item computes, so global loads are outstanding most of
// the time even at low occupancy.
// ---------------------------------------------------------------------------
// Occupancy hint of the persistent kernels: two resident workgroups per CU
// when one wave holds 16 queries of bf16 head_dim 64; otherwise one, so that
// the accumulation registers are available and nothing spills.
template <typename T, int NQ, int D> constexpr int persistent_waves() {
  return (NQ == 1 && D == 64 && sizeof(T) == 2) ? 2 : 1;
}

template <typename T, int D, int NQ, int KTB, bool WITH_U, bool PRECISE, bool QSPLIT>
__global__ __launch_bounds__(THREADS, (persistent_waves<T, NQ, D>())) void stage1_persistent_kernel(Stage1Params p) {
  constexpr bool SPLITX = split_x<T, PRECISE>();
  constexpr int DV = WITH_U ? 2 * D : D;
  constexpr int QG = WAVES * NQ * 16;
  constexpr int NSPLIT = (PRECISE && is_bf16<T>()) ? D / 16 : 0;
  typedef FlashCore<T, D, DV, NQ, KT, true, true, false, NSPLIT, QSPLIT> Core;
  typedef typename Core::frag frag;
  typedef Stage1Smem<T, D, DV, KTB> Smem;
  __shared__ Smem sm;

  const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE;
  const int nitems = p.S * p.b1 * p.nqg;
  const int mode = stage1_qmode(p);
  const bool split = PRECISE && mode != Q_INPUT;

  Stage1Keys<T, D, KTB, WITH_U> keys;     // unpadded sequences only
  frag qn[NQ][Core::NKS];
  typename Core::QLo qnl;
  auto fetch = [&](int item) {
    const int qg = item % p.nqg, k = (item / p.nqg) % p.b1, sl = item / (p.nqg * p.b1);
    const int kvs = kv_slice(sl, p.heads, p.group);
    keys.load(p, static_cast<const T*>(p.k) + (size_t)kvs * p.N * D,
              static_cast<const T*>(p.v) + (size_t)kvs * p.N * D, k, 0, p.b2);
    Core::fetch_queries([&](int n) {
      return stage1_qsrc<T, D>(p, sl, k, qg * QG + wave * NQ * 16 + n * 16 + lane % 16, 0);
    }, mode, qn, qnl);
  };

  int item = blockIdx.x;
  if (item >= nitems) return;
  fetch(item);
  Core core;
  core.qsplit = QSPLIT && split && Core::KPL == 8;
  for (; item < nitems; item += gridDim.x) {
    const int qg = item % p.nqg, k = (item / p.nqg) % p.b1, sl = item / (p.nqg * p.b1);
    __syncthreads();
    keys.store(sm);
    core.set_queries(qn, qnl);
    __syncthreads();
    if (item + (int)gridDim.x < nitems) fetch(item + gridDim.x);
    for (int s = 0; s < p.c2; ++s) {
      if (s > 0 && !p.first_step)
        core.load_queries([&](int n) {
          return stage1_qsrc<T, D>(p, sl, k, qg * QG + wave * NQ * 16 + n * 16 + lane % 16, s);
        }, mode, split);
      stage1_segment<T, SPLITX, D, NQ, KTB, WITH_U>(core, sm, p, sl, k, qg, s, s * p.sw, s * p.sw + p.sw);
    }
  }
}

template <typename T, int D, int NQ, int KTB, bool WITH_PV, bool PRECISE>
__global__ __launch_bounds__(THREADS, (persistent_waves<T, NQ, D>())) void stage2_persistent_kernel(Stage2Params p) {
  constexpr bool KLO = split_x<T, PRECISE>();
  constexpr int QG = WAVES * NQ * 16;
  typedef FlashCore<T, D, D, NQ, KT, false, WITH_PV, KLO, 0> Core;
  typedef typename Core::frag frag;
  typedef Stage2Smem<T, D, KLO, KTB> Smem;
  __shared__ Smem sm;

  const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE;
  const int nitems = p.S * p.b2 * p.c1 * p.nqg;
  auto decode = [&](int item, int& sl, int& i, int& t, int& qg) {
    qg = item % p.nqg; item /= p.nqg;
    t = item % p.c1; item /= p.c1;
    i = item % p.b2;
    sl = item / p.b2;
  };

  Stage2Prefetch<T, D, WITH_PV, KLO, KTB> pf;
  frag qn[NQ][Core::NKS];
  typename Core::QLo qnl;
  auto fetch = [&](int item) {
    int sl, i, t, qg;
    decode(item, sl, i, t, qg);
    const size_t base = x_base(p.b1, p.b2, p.c1, p.c2, sl, t, i);
    pf.load(static_cast<const T*>(p.cx) + base * D, p.xlo, static_cast<const T*>(p.ux) + base * D,
            p.h2x + base, p.nkeys, x_stride(p.b2, p.c1));
    Core::fetch_queries([&](int n) {
      return stage2_qsrc<T, D, false>(p, sl, i, t, qg * QG + wave * NQ * 16 + n * 16 + lane % 16);
    }, Q_INPUT, qn, qnl);
  };

  int item = blockIdx.x;
  if (item >= nitems) return;
  fetch(item);
  Core core;
  for (; item < nitems; item += gridDim.x) {
    int sl, i, t, qg;
    decode(item, sl, i, t, qg);
    __syncthreads();
    pf.store(sm);
    core.set_queries(qn, qnl);
    __syncthreads();
    if (item + (int)gridDim.x < nitems) fetch(item + gridDim.x);
    core.init();
    auto row = [&](int n) { return qg * QG + wave * NQ * 16 + n * 16 + lane % 16; };
#pragma unroll
    for (int c0 = 0; c0 < KTB; c0 += KT) {
      if (c0 >= p.nkeys) continue;
      const int nv = min(KT, p.nkeys - c0);
      const int how = causal_chunk<NQ>(core, p, t, row(0) - lane % 16, row, c0, nv);
      if (how == CH_SKIP) continue;
      const T (*vtc)[Smem::LDV] = reinterpret_cast<const T (*)[Smem::LDV]>(&sm.vt[0][c0]);
      core.template scores<Smem::LDK>(reinterpret_cast<const T (*)[Smem::LDK]>(&sm.ks[c0][0]),
                                      reinterpret_cast<const T (*)[Smem::LDK]>(&sm.ks_lo[KLO ? c0 : 0][0]),
                                      0, Core::MT);
      if (how == CH_ROWMASK) {
        core.template softmax_step<true, true, 0, true>(sm.bias + c0, p.sc2, 0, nv);
        if constexpr (WITH_PV) core.template pv<true>(typename Core::template PaddedVT<Smem::LDV>{vtc}, 0, nv);
      } else if (nv == KT) {
        core.template update<Smem::LDV, true, false>(vtc, sm.bias + c0, p.sc2, 0, nv);
      } else {
        core.template update<Smem::LDV, true, true>(vtc, sm.bias + c0, p.sc2, 0, nv);
      }
    }
    float lse2[NQ], h2[NQ];
    core.finish(lse2, h2, p.sc2);
    stage2_store<T, D, NQ, WITH_PV, false>(core, p, lse2, sl, i, t, qg);
  }
}

}  // namespace ma
