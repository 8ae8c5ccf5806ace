// Shared pieces of the MonarchAttention kernels for gfx950: element types,
// the split-bf16 helper, query sources and the LDS tile loaders.
//
// Precision (bf16 inputs).  Scores of a peaked row are large, and the
// aggregate c = R K enters the next scores multiplied by |q|, so rounding R
// or c to bf16 moves L by about 1e-2.  With PRECISE, the c path carries
// about 16 significant bits: R is split into bf16 hi + lo parts for the R K
// product (two MFMAs), c is written as two bf16 planes hi = bf16(c),
// lo = bf16(c - hi) (the bytes of fp32, but ready to be copied into LDS as
// MFMA operands), and the next-step queries qt stay in fp32 (split on load).
// u = R V and y = L u use plain bf16 operands.
#pragma once

#include <type_traits>

#include "ma_device.hpp"

namespace ma {

template <typename T> constexpr bool is_bf16() { return std::is_same<T, bf16>::value; }

// The exchanged aggregate c is stored as two planes (hi, lo) of T.
template <typename T, bool PRECISE> constexpr bool split_x() { return PRECISE && is_bf16<T>(); }

// Rows of the stage-1 -> stage-2 exchange (c, u, entropy, row normaliser),
// block-major: row(sl, k, s, t, i) = (((sl*b1 + k)*c2 + s)*c1 + t)*b2 + i.
// Stage 1 (block k) writes contiguous rows; stage 2 (column i, row tile t)
// reads its keys kk = k*c2 + s at x_base(sl, t, i) + kk * x_stride.
__device__ inline size_t x_row(int b1, int b2, int c1, int c2, int sl, int k, int s, int t, int i) {
  return ((((size_t)sl * b1 + k) * c2 + s) * c1 + t) * b2 + i;
}
__device__ inline size_t x_base(int b1, int b2, int c1, int c2, int sl, int t, int i) {
  return (((size_t)sl * b1 * c2) * c1 + t) * b2 + i;
}
__device__ inline size_t x_stride(int b2, int c1) { return (size_t)c1 * b2; }

// Block-causal use: query row l (grid row) attends to key block k iff
// floor(k / causal) <= floor(l / causal), i.e. to the stage-2 keys
// kk = k*c2 + s below causal_key_end(l); causal = 0 allows every key.
// (MonarchAttention scime summary "Limitations": causal masking does not fit
// the method at token level; MonarchRT summary: autoregressive video, causal
// across chunks of frames.  A mask over whole blocks keeps every block rank
// one.)
__device__ inline int causal_key_end(int l, int causal, int b1, int c2) {
  return (causal ? min(b1, (l / causal + 1) * causal) : b1) * c2;
}

// K/V slice of query slice sl (= batch * heads + head) when groups of `group`
// consecutive query heads share one K/V head.
__device__ inline int kv_slice(int sl, int heads, int group) {
  return group == 1 ? sl : (sl / heads) * (heads / group) + (sl % heads) / group;
}

__device__ inline void split_bf16(float x, bf16& hi, bf16& lo) {
  hi = (bf16)x;
  lo = (bf16)(x - (float)hi);
}

// A query row for the score MFMA: exact input values (T) or an fp32 row
// (next-step queries, tile means) that is split into hi + lo for bf16.  Both
// pointers always address valid rows (padding queries point at a real row
// and are simply not stored), so the loads need no branches; use_f selects
// per lane in the mixed mode.
template <typename T> struct QSrc {
  const T* t;
  const float* f;
  bool use_f;
};

// Where the queries of a workgroup come from (uniform over the workgroup).
enum QMode { Q_INPUT = 0, Q_F32 = 1, Q_MIXED = 2 };

template <typename T> constexpr int pad16() { return 16 / (int)sizeof(T); }

// dst[j][.] = row(j)[0 .. D) for j < nvalid, zero for nvalid <= j < NR.
template <typename T, int D, int NR, int LD, class RowFn>
__device__ inline void load_rows(T (*dst)[LD], int nvalid, RowFn row) {
  typedef typename Vec16<T>::type V;
  constexpr int VN = Vec16<T>::N;
  constexpr int CH = D / VN;
  for (int task = threadIdx.x; task < NR * CH; task += THREADS) {
    const int j = task / CH, c = task % CH;
    V v = {};
    if (j < nvalid) v = *reinterpret_cast<const V*>(row(j) + c * VN);
    *reinterpret_cast<V*>(&dst[j][c * VN]) = v;
  }
}

// Four rows x one 16-byte column chunk, written transposed:
// dst[off + c*VN + e][j0 .. j0+4) = rows[0..4)[e].
template <typename T, int LD>
__device__ inline void store_transposed4(T (*dst)[LD], int off, int c, int j0,
                                         const typename Vec16<T>::type (&v)[4]) {
  constexpr int VN = Vec16<T>::N;
  typedef T T4 __attribute__((ext_vector_type(4)));
#pragma unroll
  for (int e = 0; e < VN; ++e) {
    T4 w;
    w[0] = v[0][e]; w[1] = v[1][e]; w[2] = v[2][e]; w[3] = v[3][e];
    *reinterpret_cast<T4*>(&dst[off + c * VN + e][j0]) = w;
  }
}

}  // namespace ma
