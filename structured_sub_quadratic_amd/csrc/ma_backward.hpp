// Backward pass of MonarchAttention for gfx950.
//
// The forward of one slice is two block-local attentions (MonarchAttention,
// OpenReview author response on GQA/MLA: every intermediate step is a
// FlashAttention-like call), so the gradient of one step is two block-local
// attention backward passes in reverse order, each recomputing its softmax
// from the normalisers the forward stored (T = 1, untiled, below; row tiles
// and key segments, and the steps before the last of T > 1, are variants
// described at their kernels):
//
//   stage 2, one workgroup per column i (queries q_l = Q(l, i), keys c_k,
//   values u_k, bias H_k):
//     P = exp(sigma q.c + H - lse),  dP = dY u^T,  D_l = sum_k P dP,
//     dW = P (dP - D),  dQ += sigma dW c,  dc = sigma dW^T q,  dH = 1^T dW,
//     du = P^T dY
//   stage 1, one workgroup per block k (queries q_i = Q(k, i), keys and
//   values K(k, j), V(k, j)):
//     R = exp(sigma q.k - lse),  dR = du V^T + dc K^T,  G_i = sum_j R dR,
//     dz = R (dR - G) - dH R (log R + H)        (H = -sum R log R),
//     dQ += sigma dz K,  dK = sigma dz^T q + R^T dc,  dV = R^T du.
//
// The entropy term is the derivative of H_R = -sum_j R log R with respect to
// the scores: -R (log R + H).  Every product runs on MFMA from LDS tiles; bf16
// inputs stay exact bf16 operands, and the fp32 matrices computed in the
// kernel (P, dW, R, dz, du, dc) enter as bf16 hi + lo pairs (16 significant
// bits).  Query rows stream in chunks of RB; the per-key sums (dc, du, dK,
// dV) stay in registers across the chunks, so no global atomics are needed.
// Each wave computes strips of output tiles that share one A fragment per
// k-step, and the chunk's q, dY and the gradients of c, u are also stored
// transposed so that most operands are contiguous 16-byte LDS reads.
#pragma once

#include <type_traits>

#include "ma_launch.hpp"

namespace ma {

struct BwdParams {
  const void* q; const void* k; const void* v; const void* dy;   // [S, N, D]
  void* dq; void* dk; void* dv;                                  // [S, N, D]
  const void* cx; const void* ux;   // forward exchange c, u (input type), rows x_row
  const float* lser;                // stage-1 row normaliser (base 2), one per exchange row
  const float* h2x;                 // entropy (bits), one per exchange row
  const float* lse2;                // stage-2 row normaliser (base 2), [S, b2, b1]
  float* dq2;                       // [S, N, D] stage-2 part of dQ, token order
  float* dq2p;                      // columns of several key chunks: one [S, N, D] part per
                                    // chunk (summed into dq2 in chunk order), else null
  float* dcx; float* dux;           // [rows, D] gradients of c and u
  float* dhx;                       // [rows] gradient of H_R (nats)
  float* dkp; float* dvp;           // [S, N, D] per-query-head dK, dV (grouped K/V), or null
  float* dlx;                       // [S, b2, b1] D = rowsum(P dP) (columns of several key chunks)
  const void* qbt;                  // padded: tile means [S, b2, D] in the input type (first-step
                                    // queries of padding positions), else null
  float* dqbar;                     // padded: [S, b2, D] gradient of those tile means
  // several steps: the step's queries q~ ([rows, D] fp32, exchange rows), the
  // gradient of the next step's queries (in: dq~, rewritten as dalpha =
  // dq~ / beta) and dbeta = -dq~ . q~ / beta, and the lo plane of split c
  const float* qtil; float* dqt; const float* dbt;
  size_t xlo;
  GridMap map;
  int S, N, b1, b2, c1, c2;         // c1 row tiles, c2 key segments
  float sc, sc2;                    // scale, scale * log2(e)
  int heads, group;                 // K/V slice of query slice sl: kv_slice(sl, heads, group)
  int causal;                       // 0, or grid blocks per causal unit (keys past causal_key_end get no L)
};

// NBK: keys held in LDS (0: the largest that fits, 128; 64 for fp32 with
// head_dim 128).  A 64-key build serves blocks and columns of at most 64
// keys with about half the LDS, so two workgroups share a CU.
template <typename T, int D, int NBK = 0> struct BwdShape {
  static constexpr bool F32 = std::is_same<T, float>::value;
  static constexpr int NB = NBK ? NBK : ((F32 && D == 128) ? 64 : 128);   // keys held in LDS
  static constexpr int RB = 32;                             // query rows per chunk
  static constexpr int LDI = D + 16 / (int)sizeof(T);       // row stride over d (input type)
  static constexpr int LDN = NB + 16 / (int)sizeof(T);      // row stride over keys (input type)
  static constexpr int LDR = RB + 16 / (int)sizeof(T);      // row stride over chunk rows
  static constexpr int LDP = NB + 4;                        // fp32 row stride over keys
  static constexpr int KQ = F32 ? 16 : 32;                  // key count granularity
  // transposed copies of the keys (K^T, c^T) for the dQ product when LDS
  // allows (not in 64-key builds, which are there to halve the LDS)
  static constexpr bool KT_COPY = D == 64 && !F32 && NB == 128;
  // waves per workgroup: 8 (at head_dim 128 this halves the per-wave dK, dV
  // accumulators against 4 waves, so nothing spills and two waves share a
  // SIMD)
  static constexpr int NW = 8;
  static constexpr int NG = NW == 8 ? 2 : 4;                // key tiles per score strip
  static constexpr int DQ = NW == 8 ? 1 : (D / 16 < 4 ? D / 16 : 4);   // d tiles per dQ strip
  static constexpr int NTH = NW * WAVE;
  static constexpr int SK = (NB / 16 + NW - 1) / NW;        // key-tile strips per wave
  // the next row chunk's global inputs are held in registers while the
  // current chunk computes (head_dim 64: a few registers a thread), and the
  // stage-2 part of dQ is staged in LDS with them
  static constexpr bool PREFETCH = D == 64;
  // stage 2 (fewer live registers than stage 1) runs 8 waves at every
  // head_dim, with the prefetch
  static constexpr int NW2 = 8, NTH2 = NW2 * WAVE, NG2 = 2, DQ2 = 1;
  static constexpr int SK2 = (NB / 16 + NW2 - 1) / NW2;
  static constexpr int RG = (F32 && D == 128) ? 2 : 4;     // row chunks of a D-only workgroup
};

// Transposed bf16 tiles X^T[d][j] hold element (d, j) at column j ^ tsw(d):
// the 16-byte column chunks of row d are permuted by the row's 16-row group,
// so that the 16 lanes that write one column j with consecutive d (the
// transposing stores) fall in distinct LDS banks.  Readers of a whole chunk
// apply the same permutation to its start.
__device__ inline int tsw(int d) { return ((d >> 4) & 3) << 3; }
template <typename T> __device__ inline int tcol(int d, int j) {
  if constexpr (std::is_same<T, float>::value) return j;
  else return j ^ tsw(d);
}

// Register staging of up to RB rows of a matrix: the loads of the next row
// chunk are issued before the current chunk computes and land in LDS at the
// start of the next one.  Input-type rows (store: row major, optionally also
// transposed) or fp32 rows (store: transposed hi/lo planes, or fp32 rows).
template <typename T, int D, int RB, int NTH>
struct RowsIn {
  typedef typename Vec16<T>::type V;
  static constexpr int VN = Vec16<T>::N, CH = D / VN, NT = (RB * CH + NTH - 1) / NTH;
  V v[NT];
  template <class Src> __device__ inline void load(int n, Src src) {
#pragma unroll
    for (int a = 0; a < NT; ++a) {
      const int task = threadIdx.x + a * NTH, j = task / CH, c = task % CH;
      v[a] = V{};
      if (task < RB * CH && j < n) {
        const T* row = src(j);             // null: a padding row, zeros
        if (row) v[a] = *reinterpret_cast<const V*>(row + c * VN);
      }
    }
  }
  template <int LD, bool TR, int LDT> __device__ inline void store(T* dst, T* dt) const {
#pragma unroll
    for (int a = 0; a < NT; ++a) {
      const int task = threadIdx.x + a * NTH, j = task / CH, c = task % CH;
      if (task >= RB * CH) continue;
      *reinterpret_cast<V*>(dst + (size_t)j * LD + c * VN) = v[a];
      if constexpr (TR) {
#pragma unroll
        for (int e = 0; e < VN; ++e) dt[(size_t)(c * VN + e) * LDT + tcol<T>(c * VN + e, j)] = v[a][e];
      }
    }
  }
};
template <typename T, int D, int RB, int NTH>
struct RowsF32 {
  static constexpr int CH = D / 4, NT = (RB * CH + NTH - 1) / NTH;
  f32x4 v[NT];
  template <class Src> __device__ inline void load(int n, Src src) {
#pragma unroll
    for (int a = 0; a < NT; ++a) {
      const int task = threadIdx.x + a * NTH, j = task / CH, c = task % CH;
      v[a] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (task < RB * CH && j < n) v[a] = *reinterpret_cast<const f32x4*>(src(j) + c * 4);
    }
  }
  // rows of the input type (st(j) not null) or fp32 rows (sf(j))
  template <class SrcT, class SrcF> __device__ inline void load_mixed(int n, SrcT st, SrcF sf) {
#pragma unroll
    for (int a = 0; a < NT; ++a) {
      const int task = threadIdx.x + a * NTH, j = task / CH, c = task % CH;
      v[a] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (task >= RB * CH || j >= n) continue;
      const T* t = st(j);
      if (!t) {
        v[a] = *reinterpret_cast<const f32x4*>(sf(j) + c * 4);
      } else if constexpr (std::is_same<T, float>::value) {
        v[a] = *reinterpret_cast<const f32x4*>(t + c * 4);
      } else {
        const bf16x4 h = *reinterpret_cast<const bf16x4*>(t + c * 4);
        v[a] = f32x4{(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
      }
    }
  }
  template <int LDT> __device__ inline void store_tplanes(T* hi, size_t plane) const {
#pragma unroll
    for (int a = 0; a < NT; ++a) {
      const int task = threadIdx.x + a * NTH, j = task / CH, c = task % CH;
      if (task >= RB * CH) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        T* at = hi + (size_t)(c * 4 + e) * LDT + tcol<T>(c * 4 + e, j);
        if constexpr (std::is_same<T, float>::value) {
          *at = v[a][e];
        } else {
          const bf16 h = (bf16)v[a][e];
          at[0] = h;
          at[plane] = (bf16)(v[a][e] - (float)h);
        }
      }
    }
  }
  // rows as planes of the element type: hi[j][.] (and lo for bf16); rows of
  // LD elements, 8-byte aligned
  template <int LD> __device__ inline void store_planes(T* hi, size_t plane) const {
#pragma unroll
    for (int a = 0; a < NT; ++a) {
      const int task = threadIdx.x + a * NTH, j = task / CH, c = task % CH;
      if (task >= RB * CH) continue;
      T* at = hi + (size_t)j * LD + c * 4;
      if constexpr (std::is_same<T, float>::value) {
        *reinterpret_cast<f32x4*>(at) = v[a];
      } else {
        bf16x4 h, l;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          h[e] = (bf16)v[a][e];
          l[e] = (bf16)(v[a][e] - (float)h[e]);
        }
        *reinterpret_cast<bf16x4*>(at) = h;
        *reinterpret_cast<bf16x4*>(at + plane) = l;
      }
    }
  }
  template <int LD> __device__ inline void store_rows(float* dst) const {
#pragma unroll
    for (int a = 0; a < NT; ++a) {
      const int task = threadIdx.x + a * NTH, j = task / CH, c = task % CH;
      if (task < RB * CH) *reinterpret_cast<f32x4*>(dst + (size_t)j * LD + c * 4) = v[a];
    }
  }
};

// Operand access for one MFMA step: ROW reads X[idx][k] (k contiguous), COL
// reads X[k][idx].  Operand kinds: IN, an exact matrix of the element type;
// F32, an fp32 matrix split into hi + lo on the fly (bf16 only); PL, two
// planes hi, lo of the element type (lo `plane` elements after hi; for fp32
// only hi is read); INS, PLS: IN, PL of a transposed tile stored with the
// tcol permutation (bf16; for fp32 the same as IN, PL).
enum { ROW = 0, COL = 1 };
enum { IN = 0, F32 = 1, PL = 2, INS = 3, PLS = 4 };
constexpr bool has_lo(int kind) { return kind == F32 || kind == PL || kind == PLS; }

template <int KIND, bool SW = false>
__device__ inline bf16x8 frag_in(const bf16* X, int ld, int idx, int k) {
  if constexpr (KIND == ROW) return *reinterpret_cast<const bf16x8*>(X + (size_t)idx * ld + (SW ? k ^ tsw(idx) : k));
  bf16x8 f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = X[(size_t)(k + e) * ld + (SW ? idx ^ tsw(k + e) : idx)];
  return f;
}
template <int KIND>
__device__ inline void frag_f32(const float* X, int ld, int idx, int k, bf16x8& hi, bf16x8& lo) {
  float x[8];
  if constexpr (KIND == ROW) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(X + (size_t)idx * ld + k);
    const f32x4 b = *reinterpret_cast<const f32x4*>(X + (size_t)idx * ld + k + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) { x[e] = a[e]; x[4 + e] = b[e]; }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = X[(size_t)(k + e) * ld + idx];
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const bf16 h = (bf16)x[e];
    hi[e] = h;
    lo[e] = (bf16)(x[e] - (float)h);
  }
}

// One lane's operand fragment of kind OK in layout L (bf16): hi, and lo when
// the kind carries one.
template <int OK, int L>
__device__ inline void frag(const void* X, int ld, size_t plane, int idx, int k, bf16x8& hi, bf16x8& lo) {
  if constexpr (OK == F32) {
    frag_f32<L>(static_cast<const float*>(X), ld, idx, k, hi, lo);
  } else {
    constexpr bool SW = OK == INS || OK == PLS;
    hi = frag_in<L, SW>(static_cast<const bf16*>(X), ld, idx, k);
    if constexpr (OK == PL || OK == PLS) lo = frag_in<L, SW>(static_cast<const bf16*>(X) + plane, ld, idx, k);
  }
}

// acc[t] += A B for the NT tiles (m0, n0 + 16 t): the A fragment of each
// k-step is built once and shared by the NT tiles.  A(m, k) has kind AK in
// layout AL, B(k, n) kind BK in layout BL; K is a multiple of 4 * KPL.  For
// bf16, a split operand adds the products of its low part (lo x lo is below
// the result's precision and skipped).
template <typename T, int NT, int AK, int AL, int BK, int BL>
__device__ inline void strip_mma(f32x4 (&acc)[NT], const void* A, int lda, size_t aplane, const void* B,
                                 int ldb, size_t bplane, int m0, int n0, int K) {
  const int lane = threadIdx.x % WAVE, r = lane % 16, g = lane / 16;
  if constexpr (std::is_same<T, float>::value) {
    const float* a = static_cast<const float*>(A);
    const float* b = static_cast<const float*>(B);
    for (int k0 = 0; k0 < K; k0 += 4) {
      const int k = k0 + g;
      const float av = AL == ROW ? a[(size_t)(m0 + r) * lda + k] : a[(size_t)k * lda + m0 + r];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int n = n0 + 16 * t + r;
        const float bv = BL == ROW ? b[(size_t)n * ldb + k] : b[(size_t)k * ldb + n];
        acc[t] = Mfma<float>::mma(av, bv, acc[t]);
      }
    }
  } else {
    for (int k0 = 0; k0 < K; k0 += 32) {
      const int k = k0 + 8 * g;
      bf16x8 ah, al;
      frag<AK, AL>(A, lda, aplane, m0 + r, k, ah, al);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        bf16x8 bh, bl;
        frag<BK, BL>(B, ldb, bplane, n0 + 16 * t + r, k, bh, bl);
        acc[t] = Mfma<bf16>::mma(ah, bh, acc[t]);
        if constexpr (has_lo(AK)) acc[t] = Mfma<bf16>::mma(al, bh, acc[t]);
        if constexpr (has_lo(BK)) acc[t] = Mfma<bf16>::mma(ah, bl, acc[t]);
      }
    }
  }
}

// Sum over the 16 lanes that share lane / 16 (one output row group of a tile).
__device__ inline float sum16(float v) {
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) v += __shfl_xor(v, o);
  return v;
}

// Rows of an input-type matrix into LDS: dst[j][0..D) = src(j) for j < n,
// zero for n <= j < NR; with TR, also the transpose dt[c][j] (stride LDT).
template <typename T, int D, int LD, int NTH, bool TR = false, int LDT = 0, class Src>
__device__ inline void bwd_load_rows(T* dst, T* dt, int NR, int n, Src src) {
  typedef typename Vec16<T>::type V;
  constexpr int VN = Vec16<T>::N, CH = D / VN;
  for (int task = threadIdx.x; task < NR * CH; task += NTH) {
    const int j = task / CH, c = task % CH;
    V v = {};
    if (j < n) v = *reinterpret_cast<const V*>(src(j) + c * VN);
    *reinterpret_cast<V*>(dst + (size_t)j * LD + c * VN) = v;
    if constexpr (TR) {
#pragma unroll
      for (int e = 0; e < VN; ++e) dt[(size_t)(c * VN + e) * LDT + tcol<T>(c * VN + e, j)] = v[e];
    }
  }
}
// ---------------------------------------------------------------------------
// Stage 2 backward.  MODE S2_COLUMN: one workgroup per (slice, column i)
// whose b1 keys fit one chunk, D computed on the way.  Columns of more keys
// take two launches: S2_ROWSUM, one workgroup per (slice, column, chunk of
// RB rows), computes D = rowsum(P dP) over all key chunks into dlx; then
// S2_KEYS, one workgroup per (slice, column, chunk of NB keys), the
// gradients of that key chunk, adding its part of dQ with fp32 atomics.
// S2_ALPHA, a step before the last one of T > 1 (columns of one key chunk):
// that step's L fed the next queries q~ = alpha / beta (alpha = L^T q, beta =
// column sums of L), so dP = q dalpha^T + dbeta, dQ gains the direct term
// P dalpha on top of the softmax part, and there is no u.  S2_ROWSUM_A and
// S2_KEYS_A are the two launches of such a step for columns of several key
// chunks.  SPLITC: c is read as its two bf16 planes (the split path of bf16
// with T > 1).
// ---------------------------------------------------------------------------
enum { S2_COLUMN = 0, S2_ROWSUM = 1, S2_KEYS = 2, S2_ALPHA = 3, S2_ROWSUM_A = 4, S2_KEYS_A = 5 };

template <typename T, int D, int MODE, bool SPLITC = false, int NBK = 0>
__global__ __launch_bounds__((BwdShape<T, D, NBK>::NTH2)) void stage2_bwd_kernel(BwdParams p) {
  typedef BwdShape<T, D, NBK> SH;
  constexpr int NW = SH::NW2, NTH = SH::NTH2, RG = SH::RG;
  constexpr int NB = SH::NB, RB = SH::RB, LDI = SH::LDI, LDN = SH::LDN, LDR = SH::LDR, LDP = SH::LDP;
  constexpr int DT = D / 16, NG = SH::NG2;                   // d tiles; key tiles per score strip
  constexpr int DS = DT < 4 ? DT : 4;                        // d tiles per dc, du strip
  constexpr int DQ = SH::DQ2;                                // d tiles per dQ strip
  constexpr int SK = SH::SK2;                                // key-tile strips of dc, du per wave
  constexpr bool AL = MODE == S2_ALPHA || MODE == S2_ROWSUM_A || MODE == S2_KEYS_A;
  constexpr bool RS = MODE == S2_ROWSUM || MODE == S2_ROWSUM_A;   // D-only workgroup: RG row chunks stay in LDS
  constexpr bool KEYS = MODE == S2_KEYS || MODE == S2_KEYS_A;      // one key chunk of a long column
  constexpr int CK = SPLITC ? PL : IN;                       // operand kind of c
  constexpr int CKT = SPLITC ? PLS : INS;                    // and of its transposed copy
  constexpr size_t CPL = (size_t)NB * LDI, CTPL = (size_t)D * LDN;   // lo planes of c, c^T
  constexpr bool SPLIT = !std::is_same<T, float>::value;
  constexpr int DAK = SPLIT ? PL : IN;                       // dalpha: hi, lo planes for bf16
  constexpr size_t DPL = (size_t)NB * LDI;
  __shared__ __attribute__((aligned(16))) T cs[(SPLITC ? 2 : 1) * NB * LDI];
  __shared__ __attribute__((aligned(16))) T us[AL ? 1 : NB * LDI];
  __shared__ __attribute__((aligned(16))) T ct[SH::KT_COPY ? (SPLITC ? 2 : 1) * D * LDN : 1];   // c^T
  __shared__ __attribute__((aligned(16))) T qs[RB * LDI];
  __shared__ __attribute__((aligned(16))) T dys[AL ? 1 : RB * LDI];
  __shared__ __attribute__((aligned(16))) T qt[D * LDR];    // q^T of the chunk
  __shared__ __attribute__((aligned(16))) T dyt[AL ? 1 : D * LDR];   // dY^T of the chunk
  __shared__ __attribute__((aligned(16))) T das[AL ? (SPLIT ? 2 : 1) * NB * LDI : 1];   // dalpha of the keys
  __shared__ float dbk[AL ? NB : 1];                                      // dbeta of the keys
  __shared__ __attribute__((aligned(16))) float ps[RB * LDP];
  __shared__ __attribute__((aligned(16))) float dws[RB * LDP];
  __shared__ float h2k[NB], dhk[NB], lsel[RB], dl[RB];
  // row sums of P dP per score strip (key strips of a row tile) go to the
  // padding columns NB .. NB + 3 of ps (which nothing else reads) and are
  // added up in strip order afterwards, so the sums do not depend on wave
  // timing
  static_assert(NB / (16 * NG) <= LDP - NB, "one padding column per key strip");
  __shared__ __attribute__((aligned(16))) T qsb[RS ? RG * RB * LDI : 1];
  __shared__ __attribute__((aligned(16))) T dysb[RS && !AL ? RG * RB * LDI : 1];
  __shared__ float lsb[RS ? RG * RB : 1], dlb[RS ? RG * RB : 1];

  const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE, g = lane / 16;
  // the column's queries: rows r0 .. r0 + rt of row tile t; its keys: the
  // b1 * c2 exchange rows (k, s) of (t, i)
  const int rt = p.b1 / p.c1, nkeys = p.b1 * p.c2;
  const int nkc = (nkeys + NB - 1) / NB;                     // key chunks of NB keys
  const int nsub = !RS && !KEYS ? 1 : (RS ? (rt + RG * RB - 1) / (RG * RB) : nkc);
  const int sub = blockIdx.x % nsub;                         // row chunk (ROWSUM) or key chunk (KEYS)
  const int cid = blockIdx.x / nsub;
  const int i = cid % p.b2, t = (cid / p.b2) % p.c1, sl = cid / p.b2 / p.c1, r0 = t * rt;
  float* const dlx = p.dlx + ((size_t)sl * p.b2 + i) * p.b1 + r0;   // D of the column's rows
  const size_t xs = (size_t)p.c1 * p.b2;                     // exchange stride between keys
  const size_t xb = ((size_t)sl * p.b1 * p.c2 * p.c1 + t) * p.b2 + i;   // exchange row of key 0
  const T* C = static_cast<const T*>(p.cx);
  const T* U = static_cast<const T*>(p.ux);
  const T* Q = static_cast<const T*>(p.q) + (size_t)sl * p.N * D;
  const T* dY = static_cast<const T*>(p.dy) + (size_t)sl * p.N * D;
  const AxisMap col = p.map.col_axis(i);
  const bool padded = p.map.padded();
  int k0 = 0, nb = 0, nbp = 0;                               // current key chunk
  auto load_keys = [&](int kc) {
    k0 = kc * NB;
    nb = min(NB, nkeys - k0);
    nbp = (nb + SH::KQ - 1) / SH::KQ * SH::KQ;
    bwd_load_rows<T, D, LDI, NTH, SH::KT_COPY, LDN>(cs, ct, NB, nb, [&](int k) { return C + (xb + (k0 + k) * xs) * D; });
    if constexpr (SPLITC)
      bwd_load_rows<T, D, LDI, NTH, SH::KT_COPY, LDN>(cs + CPL, SH::KT_COPY ? ct + CTPL : nullptr, NB, nb,
                                                      [&](int k) { return C + p.xlo + (xb + (k0 + k) * xs) * D; });
    if constexpr (AL) {
      for (int task = threadIdx.x; task < NB * (D / 4); task += NTH) {
        const int k = task / (D / 4), c = task % (D / 4);
        f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
        if (k < nb) v = *reinterpret_cast<const f32x4*>(p.dqt + (xb + (k0 + k) * xs) * D + c * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          T* at = das + k * LDI + c * 4 + e;
          if constexpr (SPLIT) {
            const bf16 h = (bf16)v[e];
            at[0] = h;
            at[DPL] = (bf16)(v[e] - (float)h);
          } else {
            *at = v[e];
          }
        }
      }
    } else {
      bwd_load_rows<T, D, LDI, NTH>(us, nullptr, NB, nb, [&](int k) { return U + (xb + (k0 + k) * xs) * D; });
    }
    for (int k = threadIdx.x; k < NB; k += NTH) {
      h2k[k] = k < nb ? p.h2x[xb + (k0 + k) * xs] : 0.f;
      dhk[k] = 0.f;
      if constexpr (AL) dbk[k] = k < nb ? p.dbt[xb + (k0 + k) * xs] : 0.f;
    }
  };
  RowsIn<T, D, RB, NTH> pq, pdy;
  float pls = 0.f, pdl = 0.f;
  auto fetch = [&](int l0) {
    const int n = min(RB, rt - l0);
    pq.load(n, [&](int r) { return Q + col.at(r0 + l0 + r) * D; });
    if constexpr (!AL)
      pdy.load(n, [&](int r) -> const T* {     // no upstream gradient at padding rows
        return !padded || col.valid(r0 + l0 + r) ? dY + col.at(r0 + l0 + r) * D : nullptr;
      });
    if (threadIdx.x < RB) {
      pls = (int)threadIdx.x < n ? p.lse2[((size_t)sl * p.b2 + i) * p.b1 + r0 + l0 + threadIdx.x] : 0.f;
      if (KEYS) pdl = (int)threadIdx.x < n ? dlx[l0 + threadIdx.x] : 0.f;
    }
  };
  // P = exp2(sc2 q.c + h2 - lse2) and dP = dY u^T (S2_ALPHA: q dalpha^T +
  // dbeta) of a row chunk against the current key chunk, in strips of one row
  // tile x NG key tiles; STORE keeps them in LDS, and the row sums of P dP go
  // to dsum[row] (if not null); l0s is the chunk's first row in the tile
  auto scores = [&](int l0s, int nr, bool store, float* dsum, const T* qs, const T* dys, const float* lsel) {
    const int ng = (nbp / 16 + NG - 1) / NG;
    for (int st = wave; st < (RB / 16) * ng; st += NW) {
      const int m0 = (st / ng) * 16, n0 = (st % ng) * 16 * NG;
      const int nt = min(NG, nbp / 16 - n0 / 16);
      f32x4 s[NG], dp[NG];
#pragma unroll
      for (int t = 0; t < NG; ++t) s[t] = dp[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (nt == NG) {
        strip_mma<T, NG, IN, ROW, CK, ROW>(s, qs, LDI, 0, cs, LDI, CPL, m0, n0, D);
        if constexpr (AL) strip_mma<T, NG, IN, ROW, DAK, ROW>(dp, qs, LDI, 0, das, LDI, DPL, m0, n0, D);
        else strip_mma<T, NG, IN, ROW, IN, ROW>(dp, dys, LDI, 0, us, LDI, 0, m0, n0, D);
      } else {
        for (int t = 0; t < nt; ++t) {
          f32x4 a1[1] = {s[t]}, a2[1] = {dp[t]};
          strip_mma<T, 1, IN, ROW, CK, ROW>(a1, qs, LDI, 0, cs, LDI, CPL, m0, n0 + 16 * t, D);
          if constexpr (AL) strip_mma<T, 1, IN, ROW, DAK, ROW>(a2, qs, LDI, 0, das, LDI, DPL, m0, n0 + 16 * t, D);
          else strip_mma<T, 1, IN, ROW, IN, ROW>(a2, dys, LDI, 0, us, LDI, 0, m0, n0 + 16 * t, D);
          s[t] = a1[0];
          dp[t] = a2[0];
        }
      }
      float part[4] = {0.f, 0.f, 0.f, 0.f};
      // block-causal use: keys at or past kend[e] (chunk-local) carry no L
      // entry of this lane's row e (computed once per strip)
      int kend[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) kend[e] = nb;
      if (p.causal) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          kend[e] = min(nb, causal_key_end(r0 + l0s + m0 + 4 * g + e, p.causal, p.b1, p.c2) - k0);
      }
#pragma unroll
      for (int t = 0; t < NG; ++t) {
        if (t >= nt) continue;
        const int key = n0 + 16 * t + lane % 16;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = m0 + 4 * g + e;
          // padding rows carry no L row (no upstream gradient, no next-query weight)
          const bool ok = row < nr && key < kend[e] && (!padded || col.valid(r0 + l0s + row));
          const float pv = ok ? __builtin_amdgcn_exp2f(s[t][e] * p.sc2 + h2k[key] - lsel[row]) : 0.f;
          const float dv = ok ? dp[t][e] + (AL ? dbk[key] : 0.f) : 0.f;
          if (store) {
            ps[row * LDP + key] = pv;
            dws[row * LDP + key] = dv;
          }
          part[e] += pv * dv;
        }
      }
      if (dsum) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float v = sum16(part[e]);
          if (lane % 16 == 0) ps[(m0 + 4 * g + e) * LDP + NB + st % ng] = v;
        }
      }
    }
  };
  // dsum[r] += the strips' row sums of the last scores() call, in strip
  // order (between two barriers)
  auto add_rowsums = [&](float* dsum, int nbpk) {
    const int ng = (nbpk / 16 + NG - 1) / NG;
    for (int r = threadIdx.x; r < RB; r += NTH) {
      float v = 0.f;
      for (int j = 0; j < ng; ++j) v += ps[r * LDP + NB + j];
      dsum[r] += v;
    }
  };

  if constexpr (RS) {
    // D = rowsum(P dP) of RG row chunks over all key chunks
    const int g0 = sub * RG * RB;
    for (int c = 0; c < RG; ++c) {
      const int l0 = g0 + c * RB;
      fetch(l0);
      pq.template store<LDI, false, LDR>(qsb + c * RB * LDI, nullptr);
      if constexpr (!AL) pdy.template store<LDI, false, LDR>(dysb + c * RB * LDI, nullptr);
      if (threadIdx.x < RB) {
        lsb[c * RB + threadIdx.x] = pls;
        dlb[c * RB + threadIdx.x] = 0.f;
      }
    }
    for (int kc = 0; kc < nkc; ++kc) {
      __syncthreads();
      load_keys(kc);
      __syncthreads();
      for (int c = 0; c < RG; ++c) {
        const int l0 = g0 + c * RB;
        if (l0 >= rt) break;
        scores(l0, min(RB, rt - l0), false, dlb + c * RB, qsb + c * RB * LDI, AL ? nullptr : dysb + c * RB * LDI,
               lsb + c * RB);
        __syncthreads();
        add_rowsums(dlb + c * RB, nbp);
        __syncthreads();
      }
    }
    __syncthreads();
    for (int r = threadIdx.x; r < RG * RB; r += NTH)
      if (g0 + r < rt) dlx[g0 + r] = dlb[r];
    return;
  }

  {
  const int kc = KEYS ? sub : 0;
  load_keys(kc);
  f32x4 adc[SK][DT], adu[SK][DT];
#pragma unroll
  for (int s = 0; s < SK; ++s)
#pragma unroll
    for (int t = 0; t < DT; ++t) adc[s][t] = adu[s][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  fetch(0);
  for (int l0 = 0; l0 < rt; l0 += RB) {
    const int nr = min(RB, rt - l0);
    __syncthreads();
    pq.template store<LDI, true, LDR>(qs, qt);
    if constexpr (!AL) pdy.template store<LDI, true, LDR>(dys, dyt);
    if (threadIdx.x < RB) {
      lsel[threadIdx.x] = pls;
      dl[threadIdx.x] = KEYS ? pdl : 0.f;
    }
    if (l0 + RB < rt) fetch(l0 + RB);       // in flight while this chunk computes
    __syncthreads();
    scores(l0, nr, true, KEYS ? nullptr : dl, qs, dys, lsel);
    __syncthreads();
    if (!KEYS) {
      add_rowsums(dl, nbp);
      __syncthreads();
    }
    // dW = P (dP - D)
    for (int idx = threadIdx.x; idx < RB * nbp; idx += NTH) {
      const int r = idx / nbp, k = idx % nbp;
      dws[r * LDP + k] = ps[r * LDP + k] * (dws[r * LDP + k] - dl[r]);
    }
    __syncthreads();
    // dQ (stage-2 part) = sc dW c: strips of one row tile x DQ d tiles
    for (int st = wave; st < (RB / 16) * (DT / DQ); st += NW) {
      const int m0 = (st / (DT / DQ)) * 16, h = st % (DT / DQ);
      {
      f32x4 a[DQ], a2[DQ];
#pragma unroll
      for (int t = 0; t < DQ; ++t) a[t] = a2[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (SH::KT_COPY) strip_mma<T, DQ, F32, ROW, CKT, ROW>(a, dws, LDP, 0, ct, LDN, CTPL, m0, 16 * DQ * h, nbp);
      else strip_mma<T, DQ, F32, ROW, CK, COL>(a, dws, LDP, 0, cs, LDI, CPL, m0, 16 * DQ * h, nbp);
      // the direct term of the next queries: P dalpha
      if constexpr (AL) strip_mma<T, DQ, F32, ROW, DAK, COL>(a2, ps, LDP, 0, das, LDI, DPL, m0, 16 * DQ * h, nbp);
#pragma unroll
      for (int t = 0; t < DQ; ++t) {
        const int d = 16 * (DQ * h + t) + lane % 16;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = m0 + 4 * g + e;
          if (row >= nr || (padded && !col.valid(r0 + l0 + row))) continue;
          const size_t o = ((size_t)sl * p.N + col.at(r0 + l0 + row)) * D + d;
          // a key chunk's part of dQ goes to its own buffer (summed in
          // chunk order later); later steps' parts are in dq2 already
          if (KEYS) p.dq2p[(size_t)kc * p.S * p.N * D + o] = a[t][e] * p.sc + (AL ? a2[t][e] : 0.f);
          else if (AL) p.dq2[o] += a[t][e] * p.sc + a2[t][e];
          else p.dq2[o] = a[t][e] * p.sc;
        }
      }
      }
    }
    // dc += dW^T q, du += P^T dY: strips of one key tile over all d tiles;
    // the strip's wave also adds the key tile's column sums of dW to dH
#pragma unroll
    for (int s = 0; s < SK; ++s) {
      const int m0 = (wave + NW * s) * 16;
      if (m0 >= nbp) continue;
      {
        float cs8 = 0.f;                      // rows 8g .. 8g + 7 of key m0 + lane % 16
#pragma unroll
        for (int e = 0; e < RB / 4; ++e) cs8 += dws[(g * (RB / 4) + e) * LDP + m0 + lane % 16];
        cs8 += __shfl_xor(cs8, 16);
        cs8 += __shfl_xor(cs8, 32);
        if (g == 0) dhk[m0 + lane % 16] += cs8;
      }
#pragma unroll
      for (int h = 0; h < DT / DS; ++h) {
        f32x4 (&c)[DS] = *reinterpret_cast<f32x4(*)[DS]>(&adc[s][DS * h]);
        f32x4 (&u)[DS] = *reinterpret_cast<f32x4(*)[DS]>(&adu[s][DS * h]);
        strip_mma<T, DS, F32, COL, INS, ROW>(c, dws, LDP, 0, qt, LDR, 0, m0, 16 * DS * h, RB);
        if constexpr (!AL) strip_mma<T, DS, F32, COL, INS, ROW>(u, ps, LDP, 0, dyt, LDR, 0, m0, 16 * DS * h, RB);
      }
    }
  }
  // per-key results of the key chunk
#pragma unroll
  for (int s = 0; s < SK; ++s) {
    const int m0 = (wave + NW * s) * 16;
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      const int d = 16 * t + lane % 16;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int key = m0 + 4 * g + e;
        if (key >= nb) continue;
        const size_t row = xb + (k0 + key) * xs;
        p.dcx[row * D + d] = adc[s][t][e] * p.sc;
        if constexpr (!AL) p.dux[row * D + d] = adu[s][t][e];
      }
    }
  }
  __syncthreads();
  for (int k = threadIdx.x; k < nb; k += NTH) p.dhx[xb + (k0 + k) * xs] = dhk[k];
  }
}

// dq2 = sum of the nkc per-key-chunk parts, in chunk order (the stage-2 part
// of dQ of columns of several key chunks; n floats per part), four floats a
// thread; with acc, added to what dq2 holds (the parts of later steps).
static __global__ __launch_bounds__(256) void dq2_sum_kernel(const float* parts, float* dq2, size_t n, int nkc,
                                                             int add) {
  const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  f32x4 acc = *reinterpret_cast<const f32x4*>(parts + i);
  for (int c = 1; c < nkc; ++c) acc += *reinterpret_cast<const f32x4*>(parts + (size_t)c * n + i);
  if (add) acc += *reinterpret_cast<const f32x4*>(dq2 + i);
  *reinterpret_cast<f32x4*>(dq2 + i) = acc;
}

// ---------------------------------------------------------------------------
// Stage 1 backward: one workgroup per (slice, block k).  SM (step mode):
// S1_ONLY, the single step of T = 1 (queries q, dQ = stage-2 part + own);
// with several steps, S1_LAST (queries q~ in fp32, u and V path, dq~ out,
// dK into its fp32 sum, dV out), S1_MID (q~, no V path, dq~ out, dK added)
// and S1_FIRST (queries q, no V path, dQ = the other parts + own, dK
// finished).  With grouped K/V every step keeps dK, dV as fp32 shares.
// S1_TILED (T = 1 with row tiles and key segments): one workgroup per
// (slice, block k, segment s) with the segment's keys and the c1 * b2
// queries (t, i) -- q(k, i) for k's own row tile, the tile mean of (t, i)
// otherwise; each query's gradient goes to its exchange row (dq~).
// S1_FIRSTP: S1_FIRST of a padded sequence, whose padding positions took the
// fp32 tile means as queries (held as fp32 planes like q~; their gradient
// goes to dqbar).  S1_LAST_T, S1_MID_T and S1_FIRST_T: the three step modes
// of several steps with row tiles and key segments, in the S1_TILED
// geometry; every query gradient goes to its exchange row (step 0's queries
// are q(k, i) and the fp32 tile means; tiled_dq_kernel finishes dQ).
// ---------------------------------------------------------------------------
enum { S1_ONLY = 0, S1_LAST = 1, S1_MID = 2, S1_FIRST = 3, S1_TILED = 4, S1_FIRSTP = 5, S1_LAST_T = 6,
       S1_MID_T = 7, S1_FIRST_T = 8 };

template <typename T, int D, int SM = S1_ONLY, int NBK = 0>
__global__ __launch_bounds__((BwdShape<T, D, NBK>::NTH)) void stage1_bwd_kernel(BwdParams p) {
  typedef BwdShape<T, D, NBK> SH;
  constexpr int NW = SH::NW, NTH = SH::NTH;
  constexpr int NB = SH::NB, RB = SH::RB, LDI = SH::LDI, LDN = SH::LDN, LDR = SH::LDR, LDP = SH::LDP;
  constexpr int DT = D / 16, NG = SH::NG;
  constexpr int DS = DT < 4 ? DT : 4;                        // d tiles per dK, dV strip
  constexpr int DQ = SH::DQ;                                 // d tiles per dQ strip
  constexpr int SK = SH::SK;                                 // key-tile strips of dK, dV per wave
  constexpr bool SPLIT = !std::is_same<T, float>::value;
  constexpr bool FP = SM == S1_FIRSTP;
  constexpr bool FT = SM == S1_FIRST_T;                      // tiled step 0 of several
  constexpr bool LASTS = SM == S1_LAST || SM == S1_LAST_T;   // the last of several steps
  constexpr bool MIDS = SM == S1_MID || SM == S1_MID_T;
  constexpr bool FIRST = SM == S1_FIRST || FP || FT;         // step 0 of several
  constexpr bool QF = LASTS || MIDS || FP || FT;             // queries as fp32 planes
  constexpr bool TL = SM == S1_TILED || SM == S1_LAST_T || SM == S1_MID_T || FT;
  constexpr bool XQ = LASTS || MIDS || TL;                   // query gradients to exchange rows
  constexpr bool WV = SM == S1_ONLY || LASTS || SM == S1_TILED;   // u = R V path
  constexpr bool QP = QF && SPLIT;                           // queries carry a lo plane
  constexpr bool DQO = SM == S1_ONLY || SM == S1_FIRST || FP;     // dQ finished here
  constexpr size_t TPL = (size_t)D * LDR;                    // plane offset of the transposed grads
  constexpr size_t QPL = (size_t)RB * LDI;                   // plane offset of the query rows
  __shared__ __attribute__((aligned(16))) T ks[NB * LDI];
  __shared__ __attribute__((aligned(16))) T vs[WV ? NB * LDI : 1];
  __shared__ __attribute__((aligned(16))) T kt[SH::KT_COPY ? D * LDN : 1];   // K^T
  __shared__ __attribute__((aligned(16))) T qs[(QP ? 2 : 1) * RB * LDI];
  __shared__ __attribute__((aligned(16))) T qt[(QP ? 2 : 1) * D * LDR];    // q^T of the chunk
  __shared__ __attribute__((aligned(16))) T dut[WV ? (SPLIT ? 2 : 1) * D * LDR : 1]; // du^T (hi, lo)
  __shared__ __attribute__((aligned(16))) T dct[(SPLIT ? 2 : 1) * D * LDR]; // dc^T (hi, lo)
  // bf16 at head_dim 64: du and dc also row major (hi, lo), so that dR reads
  // its A operand as 16-byte rows instead of gathering the transposed copy
  constexpr bool RC = SPLIT && D == 64;
  constexpr size_t RPL = (size_t)RB * LDI;
  __shared__ __attribute__((aligned(16))) T dur[RC && WV ? 2 * RB * LDI : 1];
  __shared__ __attribute__((aligned(16))) T dcr[RC ? 2 * RB * LDI : 1];
  __shared__ __attribute__((aligned(16))) float rs[RB * LDP];
  __shared__ __attribute__((aligned(16))) float dzs[RB * LDP];
  __shared__ float lser[RB], dhr[RB], gr[RB], hr[RB];
  // per-strip row sums of R dR and R log R go to the padding columns NB ..
  // NB + 3 of rs and dzs (one per key strip of a row tile), which nothing
  // else reads
  static_assert(NB / (16 * NG) <= LDP - NB, "one padding column per key strip");
  __shared__ __attribute__((aligned(16))) float dq2s[SH::PREFETCH && DQO ? RB * (D + 4) : 1];   // dQ (stage 2)

  const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE, g = lane / 16;
  const int nseg = TL ? p.c2 : 1, sg = blockIdx.x % nseg;
  const int k = (blockIdx.x / nseg) % p.b1, sl = blockIdx.x / nseg / p.b1;
  const int nb = p.b2 / nseg, nbp = (nb + SH::KQ - 1) / SH::KQ * SH::KQ;
  const int j0 = sg * nb;                                    // first key of the segment
  const int nq = TL ? p.c1 * p.b2 : p.b2;                    // query rows (t, i)
  const int own = k / (p.b1 / p.c1);                         // row tile of block k
  // exchange row of query row 0 (rows (t, i) of one (k, s) are contiguous)
  const size_t xb = ((size_t)sl * p.b1 + k) * (TL ? (size_t)p.c2 * p.c1 * p.b2 : (size_t)p.b2) +
                    (TL ? (size_t)sg * p.c1 * p.b2 : 0);
  const T* Q = static_cast<const T*>(p.q) + (size_t)sl * p.N * D;
  const int kvs = kv_slice(sl, p.heads, p.group);
  const T* K = static_cast<const T*>(p.k) + (size_t)kvs * p.N * D;
  const T* V = static_cast<const T*>(p.v) + (size_t)kvs * p.N * D;
  const AxisMap row = p.map.row_axis(k);

  bwd_load_rows<T, D, LDI, NTH, SH::KT_COPY, LDN>(ks, kt, NB, nb, [&](int j) { return K + row.at(j0 + j) * D; });
  if constexpr (WV) bwd_load_rows<T, D, LDI, NTH>(vs, nullptr, NB, nb, [&](int j) { return V + row.at(j0 + j) * D; });
  f32x4 adk[SK][DT], adv[SK][DT];
#pragma unroll
  for (int s = 0; s < SK; ++s)
#pragma unroll
    for (int t = 0; t < DT; ++t) adk[s][t] = adv[s][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  RowsIn<T, D, RB, NTH> pq;
  RowsF32<T, D, RB, NTH> pdu, pdc, pdq, pqf;
  float pls = 0.f, pdh = 0.f;
  // a padding position (k, i) took the tile mean of column i as its query
  const bool padded = p.map.padded();
  const T* QB = static_cast<const T*>(p.qbt) + (size_t)sl * (TL ? p.c1 : 1) * p.b2 * D;
  const int jlo = p.map.key_lo(k), jhi = p.map.key_hi(k);   // real keys of block k
  auto fetch = [&](int i0) {
    const int n = min(RB, nq - i0);
    if constexpr (FP) {
      pqf.load_mixed(n, [&](int r) -> const T* { return row.valid(i0 + r) ? Q + row.at(i0 + r) * D : nullptr; },
                     [&](int r) { return static_cast<const float*>(p.qbt) + ((size_t)sl * p.b2 + i0 + r) * D; });
    } else if constexpr (FT) {      // own row tile: q(k, i); the others and padding: the fp32 tile means
      pqf.load_mixed(n, [&](int r) -> const T* {
        const int q = i0 + r, t = q / p.b2, i = q - t * p.b2;
        return t == own && (!padded || row.valid(i)) ? Q + row.at(i) * D : nullptr;
      }, [&](int r) { return static_cast<const float*>(p.qbt) + ((size_t)sl * p.c1 * p.b2 + i0 + r) * D; });
    } else if constexpr (QF) {      // q~ rows are ordered (k, t, s, i)
      pqf.load(n, [&](int r) {
        if constexpr (TL) {
          const int q = i0 + r, t = q / p.b2;
          return p.qtil + (((((size_t)sl * p.b1 + k) * p.c1 + t) * p.c2 + sg) * p.b2 + q - t * p.b2) * D;
        } else {
          return p.qtil + (xb + i0 + r) * D;
        }
      });
    } else if constexpr (TL) {
      // a padding position of the own tile took the tile mean, as the other tiles
      pq.load(n, [&](int r) {
        const int q = i0 + r, t = q / p.b2, i = q % p.b2;
        return t == own && (!padded || row.valid(i)) ? Q + row.at(i) * D : QB + (size_t)q * D;
      });
    } else {
      pq.load(n, [&](int r) {
        return !padded || row.valid(i0 + r) ? Q + row.at(i0 + r) * D : QB + (size_t)(i0 + r) * D;
      });
    }
    if constexpr (WV) pdu.load(n, [&](int r) { return p.dux + (xb + i0 + r) * D; });
    pdc.load(n, [&](int r) { return p.dcx + (xb + i0 + r) * D; });
    if constexpr (SH::PREFETCH && DQO)
      pdq.load(n, [&](int r) { return p.dq2 + ((size_t)sl * p.N + row.at(i0 + r)) * D; });
    if (threadIdx.x < RB) {
      pls = (int)threadIdx.x < n ? p.lser[xb + i0 + threadIdx.x] : 0.f;
      pdh = (int)threadIdx.x < n ? p.dhx[xb + i0 + threadIdx.x] : 0.f;
    }
  };
  if constexpr (SH::PREFETCH) fetch(0);
  for (int i0 = 0; i0 < nq; i0 += RB) {
    const int nr = min(RB, nq - i0);
    __syncthreads();
    if constexpr (!SH::PREFETCH) fetch(i0);
    if constexpr (QF) {
      pqf.template store_planes<LDI>(qs, QPL);
      pqf.template store_tplanes<LDR>(qt, TPL);
    } else {
      pq.template store<LDI, true, LDR>(qs, qt);
    }
    if constexpr (WV) pdu.template store_tplanes<LDR>(dut, TPL);
    pdc.template store_tplanes<LDR>(dct, TPL);
    if constexpr (RC) {
      if constexpr (WV) pdu.template store_planes<LDI>(dur, RPL);
      pdc.template store_planes<LDI>(dcr, RPL);
    }
    if constexpr (SH::PREFETCH && DQO) pdq.template store_rows<D + 4>(dq2s);
    if (threadIdx.x < RB) {
      lser[threadIdx.x] = pls;
      dhr[threadIdx.x] = pdh;
      gr[threadIdx.x] = 0.f;
      hr[threadIdx.x] = 0.f;
    }
    if constexpr (SH::PREFETCH) {
      if (i0 + RB < nq) fetch(i0 + RB);     // in flight while this chunk computes
    }
    __syncthreads();
    // R = exp2(sc2 q.k - lse2), dR = du V^T + dc K^T, G = rowsum(R dR) and
    // H = -rowsum(R log R), in strips of one row tile x NG key tiles
    const int ng = (nbp / 16 + NG - 1) / NG;
    for (int st = wave; st < (RB / 16) * ng; st += NW) {
      const int m0 = (st / ng) * 16, n0 = (st % ng) * 16 * NG;
      const int nt = min(NG, nbp / 16 - n0 / 16);
      f32x4 z[NG], dr[NG];
#pragma unroll
      for (int t = 0; t < NG; ++t) z[t] = dr[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (nt == NG) {
        strip_mma<T, NG, QP ? PL : IN, ROW, IN, ROW>(z, qs, LDI, QPL, ks, LDI, 0, m0, n0, D);
        if constexpr (RC) {
          if constexpr (WV) strip_mma<T, NG, PL, ROW, IN, ROW>(dr, dur, LDI, RPL, vs, LDI, 0, m0, n0, D);
          strip_mma<T, NG, PL, ROW, IN, ROW>(dr, dcr, LDI, RPL, ks, LDI, 0, m0, n0, D);
        } else {
          if constexpr (WV) strip_mma<T, NG, PLS, COL, IN, ROW>(dr, dut, LDR, TPL, vs, LDI, 0, m0, n0, D);
          strip_mma<T, NG, PLS, COL, IN, ROW>(dr, dct, LDR, TPL, ks, LDI, 0, m0, n0, D);
        }
      } else {
        for (int t = 0; t < nt; ++t) {
          f32x4 a1[1] = {z[t]}, a2[1] = {dr[t]};
          strip_mma<T, 1, QP ? PL : IN, ROW, IN, ROW>(a1, qs, LDI, QPL, ks, LDI, 0, m0, n0 + 16 * t, D);
          if constexpr (RC) {
            if constexpr (WV) strip_mma<T, 1, PL, ROW, IN, ROW>(a2, dur, LDI, RPL, vs, LDI, 0, m0, n0 + 16 * t, D);
            strip_mma<T, 1, PL, ROW, IN, ROW>(a2, dcr, LDI, RPL, ks, LDI, 0, m0, n0 + 16 * t, D);
          } else {
            if constexpr (WV) strip_mma<T, 1, PLS, COL, IN, ROW>(a2, dut, LDR, TPL, vs, LDI, 0, m0, n0 + 16 * t, D);
            strip_mma<T, 1, PLS, COL, IN, ROW>(a2, dct, LDR, TPL, ks, LDI, 0, m0, n0 + 16 * t, D);
          }
          z[t] = a1[0];
          dr[t] = a2[0];
        }
      }
      float pg[4] = {0.f, 0.f, 0.f, 0.f}, ph[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < NG; ++t) {
        if (t >= nt) continue;
        const int key = n0 + 16 * t + lane % 16;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = m0 + 4 * g + e;
          // (the tile holds the keys j0 .. j0 + nb of the block)
          const bool ok = r < nr && key < nb && (!padded || (j0 + key >= jlo && j0 + key < jhi));
          const float lg2 = z[t][e] * p.sc2 - lser[r];        // log2 R
          const float rv = ok ? __builtin_amdgcn_exp2f(lg2) : 0.f;
          const float dv = ok ? dr[t][e] : 0.f;
          rs[r * LDP + key] = rv;
          dzs[r * LDP + key] = dv;
          pg[e] += rv * dv;
          ph[e] -= rv > 0.f ? rv * lg2 * LN2 : 0.f;
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float vg = sum16(pg[e]), vh = sum16(ph[e]);
        if (lane % 16 == 0) {
          rs[(m0 + 4 * g + e) * LDP + NB + st % ng] = vg;
          dzs[(m0 + 4 * g + e) * LDP + NB + st % ng] = vh;
        }
      }
    }
    __syncthreads();
    // G and H of each row: the strips' sums added in strip order, so they do
    // not depend on wave timing
    for (int r = threadIdx.x; r < RB; r += NTH) {
      float vg = gr[r], vh = hr[r];
      for (int j = 0; j < ng; ++j) {
        vg += rs[r * LDP + NB + j];
        vh += dzs[r * LDP + NB + j];
      }
      gr[r] = vg;
      hr[r] = vh;
    }
    __syncthreads();
    // sc * dz = sc * (R (dR - G) - dH R (log R + H))
    for (int idx = threadIdx.x; idx < RB * nbp; idx += NTH) {
      const int r = idx / nbp, j = idx % nbp;
      const float rv = rs[r * LDP + j];
      const float lg = rv > 0.f ? __logf(rv) : 0.f;
      dzs[r * LDP + j] = p.sc * rv * ((dzs[r * LDP + j] - gr[r]) - dhr[r] * (lg + hr[r]));
    }
    __syncthreads();
    // dQ = dQ (stage 2) + sc dz K: strips of one row tile x DQ d tiles
    T* dQ = static_cast<T*>(p.dq) + (size_t)sl * p.N * D;
    for (int st = wave; st < (RB / 16) * (DT / DQ); st += NW) {
      const int m0 = (st / (DT / DQ)) * 16, h = st % (DT / DQ);
      {
      f32x4 a[DQ];
#pragma unroll
      for (int t = 0; t < DQ; ++t) a[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (SH::KT_COPY) strip_mma<T, DQ, F32, ROW, INS, ROW>(a, dzs, LDP, 0, kt, LDN, 0, m0, 16 * DQ * h, nbp);
      else strip_mma<T, DQ, F32, ROW, IN, COL>(a, dzs, LDP, 0, ks, LDI, 0, m0, 16 * DQ * h, nbp);
#pragma unroll
      for (int t = 0; t < DQ; ++t) {
        const int d = 16 * (DQ * h + t) + lane % 16;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = m0 + 4 * g + e;
          if (r >= nr) continue;
          if constexpr (XQ) {                       // gradient of this query row (q~, or own / tile mean)
            p.dqt[(xb + i0 + r) * D + d] = a[t][e];
            continue;
          }
          if (padded && !row.valid(i0 + r)) {     // gradient of the tile mean it used
            p.dqbar[((size_t)sl * p.b2 + i0 + r) * D + d] = a[t][e];
            continue;
          }
          const int64_t tok = row.at(i0 + r);
          const float q2 = SH::PREFETCH ? dq2s[r * (D + 4) + d] : p.dq2[((size_t)sl * p.N + tok) * D + d];
          dQ[tok * D + d] = from_f32<T>(a[t][e] + q2);
        }
      }
      }
    }
    // dK += sc dz^T q + R^T dc, dV += R^T du: strips of one key tile over all d tiles
#pragma unroll
    for (int s = 0; s < SK; ++s) {
      const int m0 = (wave + NW * s) * 16;
      if (m0 >= nbp) continue;
#pragma unroll
      for (int h = 0; h < DT / DS; ++h) {
        f32x4 (&a)[DS] = *reinterpret_cast<f32x4(*)[DS]>(&adk[s][DS * h]);
        f32x4 (&v)[DS] = *reinterpret_cast<f32x4(*)[DS]>(&adv[s][DS * h]);
        strip_mma<T, DS, F32, COL, QP ? PLS : INS, ROW>(a, dzs, LDP, 0, qt, LDR, TPL, m0, 16 * DS * h, RB);
        strip_mma<T, DS, F32, COL, PLS, ROW>(a, rs, LDP, 0, dct, LDR, TPL, m0, 16 * DS * h, RB);
        if constexpr (WV) strip_mma<T, DS, F32, COL, PLS, ROW>(v, rs, LDP, 0, dut, LDR, TPL, m0, 16 * DS * h, RB);
      }
    }
  }
  T* dK = static_cast<T*>(p.dk) + (size_t)sl * p.N * D;
  T* dV = static_cast<T*>(p.dv) + (size_t)sl * p.N * D;
  // several steps: the fp32 sum of dK over the later steps, all loads issued
  // before the first store
  constexpr bool ADD = MIDS || FIRST;
  float old[ADD ? SK : 1][ADD ? DT : 1][4];
  if constexpr (ADD) {
#pragma unroll
    for (int s = 0; s < SK; ++s)
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = (wave + NW * s) * 16 + 4 * g + e;
          old[s][t][e] = key < nb ? p.dkp[((size_t)sl * p.N + row.at(j0 + key)) * D + 16 * t + lane % 16] : 0.f;
        }
  }
#pragma unroll
  for (int s = 0; s < SK; ++s) {
    const int m0 = (wave + NW * s) * 16;
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      const int d = 16 * t + lane % 16;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int key = m0 + 4 * g + e;
        if (key >= nb || (padded && (j0 + key < jlo || j0 + key >= jhi))) continue;
        const int64_t tok = row.at(j0 + key);
        if constexpr (LASTS || MIDS || FIRST) {   // several steps
          const size_t at = ((size_t)sl * p.N + tok) * D + d;
          if constexpr (LASTS) {
            p.dkp[at] = adk[s][t][e];
            if (p.group > 1) p.dvp[at] = adv[s][t][e];
            else dV[tok * D + d] = from_f32<T>(adv[s][t][e]);
          } else if (FIRST && p.group == 1) {
            dK[tok * D + d] = from_f32<T>(old[s][t][e] + adk[s][t][e]);
          } else {
            p.dkp[at] = old[s][t][e] + adk[s][t][e];
          }
          continue;
        }
        if (p.dkp) {     // grouped K/V: this query head's share, summed by kv_reduce_kernel
          p.dkp[((size_t)sl * p.N + tok) * D + d] = adk[s][t][e];
          p.dvp[((size_t)sl * p.N + tok) * D + d] = adv[s][t][e];
        } else {
          dK[tok * D + d] = from_f32<T>(adk[s][t][e]);
          dV[tok * D + d] = from_f32<T>(adv[s][t][e]);
        }
      }
    }
  }
}

// Padded sequences: a padding position (k, i) used the mean of the real rows
// of column i as its first-step query, so its query gradient dqbar(i) goes
// to each of those rows divided by their number.  One workgroup per (slice,
// column), one thread per d.
template <typename T>
__global__ __launch_bounds__(128) void qbar_grad_kernel(const float* dqbar, T* dq, GridMap map, int N, int D) {
  const int i = blockIdx.x % map.b2, sl = blockIdx.x / map.b2, d = threadIdx.x;
  const int nreal = map.real_rows(i, 0, map.b1);
  if (nreal == map.b1 || nreal == 0 || d >= D) return;       // no padding row in this column
  const float gv = dqbar[((size_t)sl * map.b2 + i) * D + d] / (float)nreal;
  T* Y = dq + (size_t)sl * N * D;
  for (int l = 0; l < map.b1; ++l) {
    if (!map.valid(l, i)) continue;
    T* at = Y + map.token(l, i) * D + d;
    *at = from_f32<T>(to_f32(*at) + gv);
  }
}

// D = rowsum(P dP) of every stage-2 row from the forward's output: P dP
// summed over the keys is dY . y (y = P u).  One 16-lane group per (slice,
// column, row) of dlx; padding rows get 0.
template <typename T, int D>
__global__ __launch_bounds__(256) void dy_dot_y_kernel(const T* dy, const T* y, float* dlx, GridMap map,
                                                       int N, size_t rows) {
  constexpr int PER = D / 16;
  const size_t r = ((size_t)blockIdx.x * 256 + threadIdx.x) / 16;
  const int lane = threadIdx.x % 16;
  if (r >= rows) return;                      // whole groups of 16 lanes leave together
  const int l = r % map.b1, i = (r / map.b1) % map.b2;
  const size_t sl = r / map.b1 / map.b2;
  float acc = 0.f;
  if (map.valid(l, i)) {
    const size_t o = ((size_t)sl * N + map.token(l, i)) * D + lane * PER;
#pragma unroll
    for (int e = 0; e < PER; ++e) acc += to_f32(dy[o + e]) * to_f32(y[o + e]);
  }
  acc = sum16(acc);
  if (lane == 0) dlx[r] = acc;
}

// Row tiles / key segments (T = 1): the query gradient of exchange row
// (k, s, t, i) belongs to q(k, i) when t is k's own row tile and (k, i) a
// real position, and to the tile mean qbar(t, i) otherwise; qbar(t, i) is the
// mean of the real rows of tile t in column i (all rt of them unless the
// sequence is padded), so each of them gets an equal share of its gradient,
// and padding rows, which are not tokens, get none.  One workgroup per (slice, t,
// i): 512 / D groups of D threads split the blocks k (the sum for qbar, then
// the rows of tile t): dQ(l, i) = stage-2 part + own rows + dqbar / rt.
template <typename T, int D>
__global__ __launch_bounds__(512) void tiled_dq_kernel(const float* dqx, const float* dq2, T* dq, GridMap map,
                                                       int N, int b1, int b2, int c1, int c2) {
  constexpr int NG = 512 / D;
  __shared__ float part[NG][D];
  const int i = blockIdx.x % b2, t = (blockIdx.x / b2) % c1, sl = blockIdx.x / b2 / c1;
  const int d = threadIdx.x % D, grp = threadIdx.x / D;
  const int rt = b1 / c1;
  // exchange row (k, s, t, i) = (((sl b1 + k) c2 + s) c1 + t) b2 + i
  auto at = [&](int k, int s) { return dqx[(((((size_t)sl * b1 + k) * c2 + s) * c1 + t) * b2 + i) * D + d]; };
  float bar = 0.f;
  for (int k = grp; k < b1; k += NG) {
    if (k / rt == t && map.valid(k, i)) continue;
    for (int s = 0; s < c2; ++s) bar += at(k, s);
  }
  part[grp][d] = bar;
  __syncthreads();
  bar = 0.f;
#pragma unroll
  for (int g2 = 0; g2 < NG; ++g2) bar += part[g2][d];
  bar /= (float)max(1, map.real_rows(i, t * rt, t * rt + rt));
  for (int r = grp; r < rt; r += NG) {
    const int l = t * rt + r;
    if (!map.valid(l, i)) continue;       // a padding row: no token
    float own = 0.f;
    for (int s = 0; s < c2; ++s) own += at(l, s);
    const size_t o = ((size_t)sl * N + map.token(l, i)) * D + d;
    dq[o] = from_f32<T>(dq2[o] + own + bar);
  }
}

// Grouped K/V: dK, dV of K/V slice kv = the sums of the per-query-head
// shares of its `group` query heads (consecutive heads of one batch).
template <typename T>
__global__ __launch_bounds__(256) void kv_reduce_kernel(const float* dkp, const float* dvp, T* dk, T* dv,
                                                        int heads, int group, size_t per_slice,
                                                        size_t total) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= total) return;
  const size_t kv = idx / per_slice, off = idx % per_slice;
  const int hkv = heads / group;
  const size_t b = kv / hkv, h0 = (kv % hkv) * group;
  float sk = 0.f, sv = 0.f;
  for (int j = 0; j < group; ++j) {
    const size_t src = (b * heads + h0 + j) * per_slice + off;
    sk += dkp[src];
    sv += dvp[src];
  }
  dk[idx] = from_f32<T>(sk);
  dv[idx] = from_f32<T>(sv);
}

// T > 1: the gradient of the next step's queries q~ = alpha / beta, per
// exchange row (16 lanes a row): dalpha = dq~ / beta, written over dq~, and
// dbeta = -dq~ . q~ / beta.  A row whose L weights all underflowed (beta =
// 0) took the tile mean in the forward; no gradient is passed back there.
// dq~ and beta are in exchange-row order (k, s, t, i), q~ in (k, t, s, i).
template <int D>
__global__ __launch_bounds__(256) void alpha_grad_kernel(float* dqt, const float* beta, const float* qnext,
                                                          float* dbt, size_t rows, int b2, int c1, int c2) {
  constexpr int PER = D / 16;                   // floats a lane
  const size_t row = ((size_t)blockIdx.x * 256 + threadIdx.x) / 16;
  const int l = threadIdx.x % 16;
  if (row >= rows) return;                      // whole groups of 16 lanes leave together
  size_t qrow = row;
  if (c1 * c2 > 1) {
    const int i = (int)(row % b2), t = (int)(row / b2 % c1), s = (int)(row / b2 / c1 % c2);
    const size_t ks = row / b2 / c1 / c2;       // (slice, block)
    qrow = ((ks * c1 + t) * c2 + s) * b2 + i;
  }
  float* gq = dqt + row * D + l * PER;
  const float* qn = qnext + qrow * D + l * PER;
  f32x4 v[PER / 4];
  float dot = 0.f;
#pragma unroll
  for (int c = 0; c < PER / 4; ++c) {
    v[c] = *reinterpret_cast<const f32x4*>(gq + 4 * c);
    const f32x4 q = *reinterpret_cast<const f32x4*>(qn + 4 * c);
#pragma unroll
    for (int e = 0; e < 4; ++e) dot += v[c][e] * q[e];
  }
  dot = sum16(dot);
  const float b = beta[row];
  const float inv = b > 0.f ? 1.f / b : 0.f;
#pragma unroll
  for (int c = 0; c < PER / 4; ++c) *reinterpret_cast<f32x4*>(gq + 4 * c) = v[c] * inv;
  if (l == 0) dbt[row] = -dot * inv;
}

template <typename T, int D>
BwdParams bwd_params(const Plan& pl, const BwdBufs& b) {
  char* ws = b.ws;
  const bool kvp = pl.group > 1 || pl.T > 1;     // fp32 dK, dV shares
  return BwdParams{b.q, b.k, b.v, b.dy, b.dq, b.dk, b.dv,
              ws + pl.off_cx, ws + pl.off_ux,
              reinterpret_cast<const float*>(ws + pl.off_lser),
              reinterpret_cast<const float*>(ws + pl.off_h2),
              reinterpret_cast<const float*>(ws + pl.off_lse2),
              reinterpret_cast<float*>(ws + pl.off_dq2),
              pl.dq2_parts > 1 ? reinterpret_cast<float*>(ws + pl.off_dq2p) : nullptr,
              reinterpret_cast<float*>(ws + pl.off_dcx), reinterpret_cast<float*>(ws + pl.off_dux),
              reinterpret_cast<float*>(ws + pl.off_dhx),
              kvp ? reinterpret_cast<float*>(ws + pl.off_dkp) : nullptr,
              kvp ? reinterpret_cast<float*>(ws + pl.off_dvp) : nullptr,
              reinterpret_cast<float*>(ws + pl.off_dlx),
              pl.need_qbar
                  ? (pl.precise ? (const void*)(ws + pl.off_qbar) : (const void*)(ws + pl.off_qbar_lp))
                  : nullptr,
              pl.padded ? reinterpret_cast<float*>(ws + pl.off_dqbar) : nullptr,
              pl.T > 1 ? reinterpret_cast<const float*>(ws + pl.off_qtil) : nullptr,
              pl.T > 1 || pl.c1 > 1 || pl.c2 > 1 ? reinterpret_cast<float*>(ws + pl.off_dqt) : nullptr,
              pl.T > 1 ? reinterpret_cast<const float*>(ws + pl.off_dbt) : nullptr,
              pl.xlo,
              pl.map, (int)pl.S, (int)pl.N, pl.b1, pl.b2, pl.c1, pl.c2, pl.scale, pl.sc2, pl.heads,
              pl.group, pl.causal};
}

// dK, dV from their fp32 shares (grouped K/V: summed over the group).
template <typename T, int D>
void bwd_kv_out(const Plan& pl, const BwdParams& p, const BwdBufs& b, hipStream_t st) {
  const size_t per = (size_t)pl.N * D, total = (size_t)pl.S / pl.group * per;
  hipLaunchKernelGGL((kv_reduce_kernel<T>), dim3(grid1((total + 255) / 256)), dim3(256), 0, st, p.dkp,
                     p.dvp, static_cast<T*>(b.dk), static_cast<T*>(b.dv), pl.heads, pl.group, per, total);
}

// Launch of a stage-2 backward build: the 64-key build (two workgroups a CU
// where the registers allow) when the default holds more and `small` says
// the keys fit 64; ONLY64 launches nothing else (bf16 head_dim 128 with
// split c, whose 128-key tiles exceed LDS).
#define MA_BWD2(MODE, SC, small, grid)                                                               \
  do {                                                                                             \
    if constexpr (BwdShape<T, D>::NB > 64) {                                                       \
      if (ONLY64 || (small)) {                                                                     \
        hipLaunchKernelGGL((stage2_bwd_kernel<T, D, MODE, SC, 64>), grid, dim3(NTH2), 0, st, p);   \
        break;                                                                                     \
      }                                                                                            \
    }                                                                                              \
    if constexpr (!ONLY64) hipLaunchKernelGGL((stage2_bwd_kernel<T, D, MODE, SC>), grid, dim3(NTH2), 0, st, p); \
  } while (0)
// Stage 1: the 64-key build only where the default does not fit (ONLY64);
// its registers allow one workgroup a CU either way, and the default keeps
// the transposed key copy.
#define MA_BWD1(SM, grid)                                                                            \
  do {                                                                                             \
    if constexpr (ONLY64) hipLaunchKernelGGL((stage1_bwd_kernel<T, D, SM, 64>), grid, dim3(NTH), 0, st, p); \
    else hipLaunchKernelGGL((stage1_bwd_kernel<T, D, SM>), grid, dim3(NTH), 0, st, p);             \
  } while (0)

// T > 1.  The forward
// is recomputed step by step into per-step state (c, entropy, both
// normalisers, the step's queries q~ and the column sums beta of L); then
// the steps are differentiated in reverse.  The last step as for T = 1 but
// with q~ as its stage-1 queries (giving dq~); every earlier step t takes
// dq~ of step t + 1 through q~ = alpha / beta into its stage 2 (dQ direct
// and softmax parts, dc, dH) and its stage 1 (dq~ of step t, or at t = 0
// the rest of dQ; dK).  dQ and dK accumulate in fp32 over the steps; the
// step-0 stage 1, which runs last, writes them out.  A column of more keys
// than one chunk takes, at every step, a D pass and one workgroup per key
// chunk, whose parts of dQ are added in chunk order.
template <typename T, int D, bool PRECISE>
ma_status run_bwd_steps_t(const Plan& pl, const BwdBufs& b, hipStream_t st) {
  Bufs fb{b.q, b.k, b.v, nullptr, b.ws, nullptr, nullptr, nullptr, nullptr};
  if (pl.need_qbar && launch_one<T, D, PRECISE>(pl, fb, L_QBAR, 0, st) != hipSuccess) return MA_ERR_DEVICE;
  for (int t = 0; t < pl.T; ++t) {
    const Plan sp = step_plan(pl, t);
    const bool last = t == pl.T - 1;
    if (launch_one<T, D, PRECISE>(sp, fb, last ? L_STAGE1_LAST : L_STAGE1, t, st) != hipSuccess)
      return MA_ERR_DEVICE;
    if (launch_one<T, D, PRECISE>(sp, fb, L_STAGE2_STATS, t, st) != hipSuccess) return MA_ERR_DEVICE;
    if (!last) {       // next queries into step t + 1's region, beta into step t's
      Plan ap = sp;
      ap.off_qtil = step_plan(pl, t + 1).off_qtil;
      ap.beta_out = true;
      if (launch_one<T, D, PRECISE>(ap, fb, L_ALPHA, t, st) != hipSuccess) return MA_ERR_DEVICE;
    }
  }
  constexpr int NTH = BwdShape<T, D>::NTH, NTH2 = BwdShape<T, D>::NTH2;
  constexpr bool SPLITC = !std::is_same<T, float>::value && PRECISE;
  constexpr bool ONLY64 = SPLITC && D == 128;              // blocks and columns of <= 64 keys
  // row tiles and key segments: stage 2 per (row tile, column), stage 1 per
  // (block, segment)
  const bool tiled = pl.c1 > 1 || pl.c2 > 1;
  const size_t cols = (size_t)pl.S * pl.c1 * pl.b2, nq = (size_t)pl.S * pl.N * D;
  const dim3 g2(grid1(cols)), g1(grid1((size_t)pl.S * pl.b1 * pl.c2));
  const size_t rows = (size_t)pl.S * pl.G;                 // stage-2 rows
  const size_t xrows = rows * pl.c1 * pl.c2;               // exchange rows
  BwdParams p = bwd_params<T, D>(pl, b);
  const int nkeys = pl.b1 * pl.c2;                         // keys of a stage-2 column
  const bool k2 = nkeys <= 64;                             // 64-key stage-2 build
  // columns of several key chunks
  constexpr int NBK = ONLY64 ? 64 : 0;                    // the chunked build
  constexpr int NBC = BwdShape<T, D, NBK>::NB, RGC = BwdShape<T, D, NBK>::RG, RBC = BwdShape<T, D, NBK>::RB;
  const bool chunked = nkeys > NBC;
  const int nkc = (nkeys + NBC - 1) / NBC;
  const dim3 grs(grid1(cols * ((pl.rt + RGC * RBC - 1) / (RGC * RBC)))), gks(grid1(cols * nkc));
  const dim3 gsum(grid1((nq / 4 + 255) / 256));
  if (chunked) {                         // D = dY . y, or a D pass; then the key chunks
    if (b.y)
      hipLaunchKernelGGL((dy_dot_y_kernel<T, D>), dim3(grid1((rows * 16 + 255) / 256)), dim3(256), 0, st,
                         static_cast<const T*>(b.dy), static_cast<const T*>(b.y), p.dlx, pl.map, (int)pl.N, rows);
    else
      hipLaunchKernelGGL((stage2_bwd_kernel<T, D, S2_ROWSUM, SPLITC, NBK>), grs, dim3(NTH2), 0, st, p);
    hipLaunchKernelGGL((stage2_bwd_kernel<T, D, S2_KEYS, SPLITC, NBK>), gks, dim3(NTH2), 0, st, p);
    hipLaunchKernelGGL(dq2_sum_kernel, gsum, dim3(256), 0, st, p.dq2p, p.dq2, nq, nkc, 0);
  } else {
    MA_BWD2(S2_COLUMN, SPLITC, k2, g2);
  }
  if (tiled) MA_BWD1(S1_LAST_T, g1);
  else MA_BWD1(S1_LAST, g1);
  for (int t = pl.T - 2; t >= 0; --t) {
    const Plan sp = step_plan(pl, t);
    char* ws = b.ws;
    p.cx = ws + sp.off_cx;
    p.lser = reinterpret_cast<const float*>(ws + sp.off_lser);
    p.h2x = reinterpret_cast<const float*>(ws + sp.off_h2);
    p.lse2 = reinterpret_cast<const float*>(ws + sp.off_lse2);
    p.qtil = reinterpret_cast<const float*>(ws + sp.off_qtil);
    hipLaunchKernelGGL((alpha_grad_kernel<D>), dim3(grid1((xrows * 16 + 255) / 256)), dim3(256), 0, st, p.dqt,
                       reinterpret_cast<const float*>(ws + sp.off_beta),
                       reinterpret_cast<const float*>(ws + step_plan(pl, t + 1).off_qtil),
                       reinterpret_cast<float*>(ws + pl.off_dbt), xrows, pl.b2, pl.c1, pl.c2);
    if (chunked) {                       // the parts of dQ add to those of later steps
      hipLaunchKernelGGL((stage2_bwd_kernel<T, D, S2_ROWSUM_A, SPLITC, NBK>), grs, dim3(NTH2), 0, st, p);
      hipLaunchKernelGGL((stage2_bwd_kernel<T, D, S2_KEYS_A, SPLITC, NBK>), gks, dim3(NTH2), 0, st, p);
      hipLaunchKernelGGL(dq2_sum_kernel, gsum, dim3(256), 0, st, p.dq2p, p.dq2, nq, nkc, 1);
    } else {
      MA_BWD2(S2_ALPHA, SPLITC, k2, g2);
    }
    if (tiled) {
      if (t > 0) MA_BWD1(S1_MID_T, g1);
      else MA_BWD1(S1_FIRST_T, g1);
    } else {
      if (t > 0) MA_BWD1(S1_MID, g1);
      else if (pl.padded) MA_BWD1(S1_FIRSTP, g1);
      else MA_BWD1(S1_FIRST, g1);
    }
  }
  if (tiled)                            // dQ from the step-0 query gradients and the stage-2 parts
    hipLaunchKernelGGL((tiled_dq_kernel<T, D>), g2, dim3(512), 0, st, p.dqt, p.dq2, static_cast<T*>(b.dq),
                       pl.map, (int)pl.N, pl.b1, pl.b2, pl.c1, pl.c2);
  else if (pl.padded)
    hipLaunchKernelGGL((qbar_grad_kernel<T>), dim3(grid1((size_t)pl.S * pl.b2)), dim3(128), 0, st, p.dqbar,
                       static_cast<T*>(b.dq), pl.map, (int)pl.N, D);
  if (pl.group > 1) bwd_kv_out<T, D>(pl, p, b, st);
  return hipGetLastError() == hipSuccess ? MA_OK : MA_ERR_DEVICE;
}

// The whole backward call on stream st: the forward's stage 1 (last-step
// kind: c, u, entropy, normaliser) and stage 2 statistics (row normalisers,
// no output) refill the workspace (unless a forward call left them there),
// then the two backward kernels run.
template <typename T, int D, bool PRECISE>
ma_status run_bwd_t(const Plan& pl, const BwdBufs& b, hipStream_t st) {
  if constexpr (std::is_same<T, float>::value) {
    if (pl.T > 1) return run_bwd_steps_t<T, D, PRECISE>(pl, b, st);
  } else if (pl.T > 1) {
    return MA_ERR_UNSUPPORTED;      // bf16 T > 1 runs the split-c entry
  }
  Bufs fb{b.q, b.k, b.v, nullptr, b.ws, nullptr, nullptr, nullptr, nullptr};
  if (!pl.reuse_state) {
    if (pl.need_qbar && launch_one<T, D, PRECISE>(pl, fb, L_QBAR, 0, st) != hipSuccess) return MA_ERR_DEVICE;
    if (launch_one<T, D, PRECISE>(pl, fb, L_STAGE1_LAST, 0, st) != hipSuccess) return MA_ERR_DEVICE;
    if (launch_one<T, D, PRECISE>(pl, fb, L_STAGE2_STATS, 0, st) != hipSuccess) return MA_ERR_DEVICE;
  }
  const BwdParams p = bwd_params<T, D>(pl, b);
  constexpr int NTH = BwdShape<T, D>::NTH, NTH2 = BwdShape<T, D>::NTH2;
  constexpr int NB = BwdShape<T, D>::NB, RB = BwdShape<T, D>::RB, RG = BwdShape<T, D>::RG;
  constexpr bool ONLY64 = false;
  // stage-2 columns: (slice, row tile t, column i), rt queries over b1 * c2 keys
  const size_t cols = (size_t)pl.S * pl.c1 * pl.b2;
  const int nkeys = pl.b1 * pl.c2;
  if (nkeys <= NB) {
    MA_BWD2(S2_COLUMN, false, nkeys <= 64, dim3(grid1(cols)));
  } else {                                 // D first, then one workgroup per key chunk
    if (b.y) {                             // D = dY . y
      const size_t rows = (size_t)pl.S * pl.G;
      hipLaunchKernelGGL((dy_dot_y_kernel<T, D>), dim3(grid1((rows * 16 + 255) / 256)), dim3(256), 0, st,
                         static_cast<const T*>(b.dy), static_cast<const T*>(b.y), p.dlx, pl.map, (int)pl.N,
                         rows);
    } else {
      hipLaunchKernelGGL((stage2_bwd_kernel<T, D, S2_ROWSUM>),
                         dim3(grid1(cols * ((pl.rt + RG * RB - 1) / (RG * RB)))), dim3(NTH2), 0, st, p);
    }
    const int nkc = (nkeys + NB - 1) / NB;
    hipLaunchKernelGGL((stage2_bwd_kernel<T, D, S2_KEYS>), dim3(grid1(cols * nkc)), dim3(NTH2), 0, st, p);
    // the key chunks' parts of dQ, added in chunk order
    const size_t n = (size_t)pl.S * pl.N * D;
    hipLaunchKernelGGL(dq2_sum_kernel, dim3(grid1((n / 4 + 255) / 256)), dim3(256), 0, st, p.dq2p, p.dq2, n,
                       nkc, 0);
  }
  if (pl.c1 > 1 || pl.c2 > 1) {            // per (block, segment), then the query gradients
    MA_BWD1(S1_TILED, dim3(grid1((size_t)pl.S * pl.b1 * pl.c2)));
    hipLaunchKernelGGL((tiled_dq_kernel<T, D>), dim3(grid1(cols)), dim3(512), 0, st, p.dqt, p.dq2,
                       static_cast<T*>(b.dq), pl.map, (int)pl.N, pl.b1, pl.b2, pl.c1, pl.c2);
  } else {
    MA_BWD1(S1_ONLY, dim3(grid1((size_t)pl.S * pl.b1)));
  }
  if (pl.padded && pl.c1 == 1 && pl.c2 == 1)     // (tiled: tiled_dq_kernel routes the tile means)
    hipLaunchKernelGGL((qbar_grad_kernel<T>), dim3(grid1((size_t)pl.S * pl.b2)), dim3(128), 0, st, p.dqbar,
                       static_cast<T*>(b.dq), pl.map, (int)pl.N, D);
  if (pl.group > 1) bwd_kv_out<T, D>(pl, p, b, st);
  return hipGetLastError() == hipSuccess ? MA_OK : MA_ERR_DEVICE;
}

#undef MA_BWD1
#undef MA_BWD2

}  // namespace ma
