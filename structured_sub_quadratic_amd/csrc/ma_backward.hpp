// Backward pass of MonarchAttention (T = 1, untiled) for gfx950.
//
// The forward of one slice is two block-local attentions (MonarchAttention,
// OpenReview author response on GQA/MLA: every intermediate step is a
// FlashAttention-like call), so its gradient is two block-local attention
// backward passes in reverse order, each recomputing its softmax from the
// normalisers the forward stored:
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
// dV) stay in registers across the chunks, so no atomics are needed.
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
  float* dcx; float* dux;           // [rows, D] gradients of c and u
  float* dhx;                       // [rows] gradient of H_R (nats)
  GridMap map;
  int S, N, b1, b2;
  float sc, sc2;                    // scale, scale * log2(e)
};

template <typename T, int D> struct BwdShape {
  static constexpr bool F32 = std::is_same<T, float>::value;
  static constexpr int NB = (F32 && D == 128) ? 64 : 128;   // keys held in LDS
  static constexpr int RB = (D == 64 && !F32) ? 64 : 32;    // query rows per chunk
  static constexpr int LDI = D + 16 / (int)sizeof(T);       // input-type row stride
  static constexpr int LDF = D + 4;                         // fp32 row stride over d
  static constexpr int LDP = NB + 4;                        // fp32 row stride over keys
  static constexpr int KQ = F32 ? 16 : 32;                  // key count granularity
  static constexpr int KPL = Mfma<T>::KPL;
};

// Operand access for one MFMA step: ROW reads X[idx][k] (k contiguous), COL
// reads X[k][idx].  Input-type matrices are exact operands; fp32 matrices are
// split into hi + lo for bf16.
enum { ROW = 0, COL = 1 };

template <int KIND>
__device__ inline bf16x8 frag_in(const bf16* X, int ld, int idx, int k) {
  if constexpr (KIND == ROW) return *reinterpret_cast<const bf16x8*>(X + (size_t)idx * ld + k);
  bf16x8 f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = X[(size_t)(k + e) * ld + idx];
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

// acc += A B over k in [0, K) for the 16 x 16 tile (m0, n0): A(m, k) from
// matrix A (input type when FA is false, fp32 otherwise) in layout KA, B(k, n)
// likewise.  K is a multiple of 4 * KPL.
template <typename T, int KA, bool FA, int KB, bool FB>
__device__ inline f32x4 tile_mma(const void* A, int lda, const void* B, int ldb, int m0, int n0,
                                 int K, f32x4 acc) {
  const int lane = threadIdx.x % WAVE, r = lane % 16, g = lane / 16;
  if constexpr (std::is_same<T, float>::value) {
    const float* a = static_cast<const float*>(A);
    const float* b = static_cast<const float*>(B);
    for (int k0 = 0; k0 < K; k0 += 4) {
      const int k = k0 + g;
      const float av = KA == ROW ? a[(size_t)(m0 + r) * lda + k] : a[(size_t)k * lda + m0 + r];
      const float bv = KB == ROW ? b[(size_t)(n0 + r) * ldb + k] : b[(size_t)k * ldb + n0 + r];
      acc = Mfma<float>::mma(av, bv, acc);
    }
  } else {
    for (int k0 = 0; k0 < K; k0 += 32) {
      const int k = k0 + 8 * g;
      bf16x8 ah, al, bh, bl;
      if constexpr (FA) frag_f32<KA>(static_cast<const float*>(A), lda, m0 + r, k, ah, al);
      else ah = frag_in<KA>(static_cast<const bf16*>(A), lda, m0 + r, k);
      if constexpr (FB) frag_f32<KB>(static_cast<const float*>(B), ldb, n0 + r, k, bh, bl);
      else bh = frag_in<KB>(static_cast<const bf16*>(B), ldb, n0 + r, k);
      acc = Mfma<bf16>::mma(ah, bh, acc);
      if constexpr (FA) acc = Mfma<bf16>::mma(al, bh, acc);
      if constexpr (FB) acc = Mfma<bf16>::mma(ah, bl, acc);
    }
  }
  return acc;
}

// Rows of an input-type matrix into LDS: dst[j][0..D) = src(j) for j < n,
// zero for n <= j < NR.
template <typename T, int D, int LD, class Src>
__device__ inline void bwd_load_rows(T* dst, int NR, int n, Src src) {
  typedef typename Vec16<T>::type V;
  constexpr int VN = Vec16<T>::N, CH = D / VN;
  for (int task = threadIdx.x; task < NR * CH; task += THREADS) {
    const int j = task / CH, c = task % CH;
    V v = {};
    if (j < n) v = *reinterpret_cast<const V*>(src(j) + c * VN);
    *reinterpret_cast<V*>(dst + (size_t)j * LD + c * VN) = v;
  }
}
template <int D, int LD, class Src>
__device__ inline void bwd_load_rows_f32(float* dst, int NR, int n, Src src) {
  constexpr int CH = D / 4;
  for (int task = threadIdx.x; task < NR * CH; task += THREADS) {
    const int j = task / CH, c = task % CH;
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (j < n) v = *reinterpret_cast<const f32x4*>(src(j) + c * 4);
    *reinterpret_cast<f32x4*>(dst + (size_t)j * LD + c * 4) = v;
  }
}

// ---------------------------------------------------------------------------
// Stage 2 backward: one workgroup per (slice, column i).
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(THREADS) void stage2_bwd_kernel(BwdParams p) {
  typedef BwdShape<T, D> SH;
  constexpr int NB = SH::NB, RB = SH::RB, LDI = SH::LDI, LDP = SH::LDP;
  constexpr int MJ = (NB / 16) * (D / 16) / WAVES;          // dc, du tiles per wave
  __shared__ __attribute__((aligned(16))) T cs[NB * LDI];
  __shared__ __attribute__((aligned(16))) T us[NB * LDI];
  __shared__ __attribute__((aligned(16))) T qs[RB * LDI];
  __shared__ __attribute__((aligned(16))) T dys[RB * LDI];
  __shared__ __attribute__((aligned(16))) float ps[RB * LDP];
  __shared__ __attribute__((aligned(16))) float dws[RB * LDP];
  __shared__ float h2k[NB], dhk[NB], lsel[RB], dl[RB];

  const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE, g = lane / 16;
  const int i = blockIdx.x % p.b2, sl = blockIdx.x / p.b2;
  const int nb = p.b1, nbp = (nb + SH::KQ - 1) / SH::KQ * SH::KQ;
  const size_t xs = (size_t)p.b2;                            // exchange stride between keys
  const size_t xb = (size_t)sl * p.b1 * p.b2 + i;            // exchange row of key 0
  const T* C = static_cast<const T*>(p.cx);
  const T* U = static_cast<const T*>(p.ux);
  const T* Q = static_cast<const T*>(p.q) + (size_t)sl * p.N * D;
  const T* dY = static_cast<const T*>(p.dy) + (size_t)sl * p.N * D;
  const AxisMap col = p.map.col_axis(i);

  bwd_load_rows<T, D, LDI>(cs, NB, nb, [&](int k) { return C + (xb + k * xs) * D; });
  bwd_load_rows<T, D, LDI>(us, NB, nb, [&](int k) { return U + (xb + k * xs) * D; });
  for (int k = threadIdx.x; k < NB; k += THREADS) {
    h2k[k] = k < nb ? p.h2x[xb + k * xs] : 0.f;
    dhk[k] = 0.f;
  }
  f32x4 adc[MJ], adu[MJ];
#pragma unroll
  for (int j = 0; j < MJ; ++j) adc[j] = adu[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int l0 = 0; l0 < p.b1; l0 += RB) {
    const int nr = min(RB, p.b1 - l0);
    __syncthreads();
    bwd_load_rows<T, D, LDI>(qs, RB, nr, [&](int r) { return Q + col.at(l0 + r) * D; });
    bwd_load_rows<T, D, LDI>(dys, RB, nr, [&](int r) { return dY + col.at(l0 + r) * D; });
    for (int r = threadIdx.x; r < RB; r += THREADS)
      lsel[r] = r < nr ? p.lse2[((size_t)sl * p.b2 + i) * p.b1 + l0 + r] : 0.f;
    __syncthreads();
    // P = exp2(sc2 q.c + h2 - lse2) and dP = dY u^T, RB x nbp
    for (int t = wave; t < (RB / 16) * (nbp / 16); t += WAVES) {
      const int m0 = (t / (nbp / 16)) * 16, n0 = (t % (nbp / 16)) * 16;
      f32x4 s = tile_mma<T, ROW, false, ROW, false>(qs, LDI, cs, LDI, m0, n0, D, f32x4{0.f, 0.f, 0.f, 0.f});
      f32x4 dp = tile_mma<T, ROW, false, ROW, false>(dys, LDI, us, LDI, m0, n0, D, f32x4{0.f, 0.f, 0.f, 0.f});
      const int key = n0 + lane % 16;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = m0 + 4 * g + e;
        const bool ok = row < nr && key < nb;
        ps[row * LDP + key] = ok ? __builtin_amdgcn_exp2f(s[e] * p.sc2 + h2k[key] - lsel[row]) : 0.f;
        dws[row * LDP + key] = ok ? dp[e] : 0.f;
      }
    }
    __syncthreads();
    // D_l = sum_k P dP
    for (int r = threadIdx.x; r < RB; r += THREADS) {
      float acc = 0.f;
      for (int k = 0; k < nbp; ++k) acc += ps[r * LDP + k] * dws[r * LDP + k];
      dl[r] = acc;
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < RB * nbp; idx += THREADS) {
      const int r = idx / nbp, k = idx % nbp;
      dws[r * LDP + k] = ps[r * LDP + k] * (dws[r * LDP + k] - dl[r]);
    }
    __syncthreads();
    // dQ (stage-2 part) = sc dW c, RB x D
    for (int t = wave; t < (RB / 16) * (D / 16); t += WAVES) {
      const int m0 = (t / (D / 16)) * 16, n0 = (t % (D / 16)) * 16;
      const f32x4 a = tile_mma<T, ROW, true, COL, false>(dws, LDP, cs, LDI, m0, n0, nbp,
                                                          f32x4{0.f, 0.f, 0.f, 0.f});
      const int d = n0 + lane % 16;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = m0 + 4 * g + e;
        if (row < nr) p.dq2[((size_t)sl * p.N + col.at(l0 + row)) * D + d] = a[e] * p.sc;
      }
    }
    // dc += dW^T q, du += P^T dY (NB x D, over the chunk's rows)
#pragma unroll
    for (int j = 0; j < MJ; ++j) {
      const int t = wave + WAVES * j;
      const int m0 = (t / (D / 16)) * 16, n0 = (t % (D / 16)) * 16;
      if (m0 >= nbp) continue;
      adc[j] = tile_mma<T, COL, true, COL, false>(dws, LDP, qs, LDI, m0, n0, RB, adc[j]);
      adu[j] = tile_mma<T, COL, true, COL, false>(ps, LDP, dys, LDI, m0, n0, RB, adu[j]);
    }
    for (int k = threadIdx.x; k < nbp; k += THREADS) {
      float acc = 0.f;
      for (int r = 0; r < RB; ++r) acc += dws[r * LDP + k];
      dhk[k] += acc;
    }
  }
  // per-key results
#pragma unroll
  for (int j = 0; j < MJ; ++j) {
    const int t = wave + WAVES * j;
    const int m0 = (t / (D / 16)) * 16, n0 = (t % (D / 16)) * 16;
    const int d = n0 + lane % 16;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int key = m0 + 4 * g + e;
      if (key >= nb) continue;
      const size_t row = xb + key * xs;
      p.dcx[row * D + d] = adc[j][e] * p.sc;
      p.dux[row * D + d] = adu[j][e];
    }
  }
  __syncthreads();
  for (int k = threadIdx.x; k < nb; k += THREADS) p.dhx[xb + k * xs] = dhk[k];
}

// ---------------------------------------------------------------------------
// Stage 1 backward: one workgroup per (slice, block k).
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(THREADS) void stage1_bwd_kernel(BwdParams p) {
  typedef BwdShape<T, D> SH;
  constexpr int NB = SH::NB, RB = SH::RB, LDI = SH::LDI, LDF = SH::LDF, LDP = SH::LDP;
  constexpr int MJ = (NB / 16) * (D / 16) / WAVES;          // dK, dV tiles per wave
  __shared__ __attribute__((aligned(16))) T ks[NB * LDI];
  __shared__ __attribute__((aligned(16))) T vs[NB * LDI];
  __shared__ __attribute__((aligned(16))) T qs[RB * LDI];
  __shared__ __attribute__((aligned(16))) float dus[RB * LDF];
  __shared__ __attribute__((aligned(16))) float dcs[RB * LDF];
  __shared__ __attribute__((aligned(16))) float rs[RB * LDP];
  __shared__ __attribute__((aligned(16))) float dzs[RB * LDP];
  __shared__ float lser[RB], dhr[RB], gr[RB], hr[RB];

  const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE, g = lane / 16;
  const int k = blockIdx.x % p.b1, sl = blockIdx.x / p.b1;
  const int nb = p.b2, nbp = (nb + SH::KQ - 1) / SH::KQ * SH::KQ;
  const size_t xb = ((size_t)sl * p.b1 + k) * p.b2;          // exchange row of (k, i = 0)
  const T* Q = static_cast<const T*>(p.q) + (size_t)sl * p.N * D;
  const T* K = static_cast<const T*>(p.k) + (size_t)sl * p.N * D;
  const T* V = static_cast<const T*>(p.v) + (size_t)sl * p.N * D;
  const AxisMap row = p.map.row_axis(k);

  bwd_load_rows<T, D, LDI>(ks, NB, nb, [&](int j) { return K + row.at(j) * D; });
  bwd_load_rows<T, D, LDI>(vs, NB, nb, [&](int j) { return V + row.at(j) * D; });
  f32x4 adk[MJ], adv[MJ];
#pragma unroll
  for (int j = 0; j < MJ; ++j) adk[j] = adv[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int i0 = 0; i0 < p.b2; i0 += RB) {
    const int nr = min(RB, p.b2 - i0);
    __syncthreads();
    bwd_load_rows<T, D, LDI>(qs, RB, nr, [&](int r) { return Q + row.at(i0 + r) * D; });
    bwd_load_rows_f32<D, LDF>(dus, RB, nr, [&](int r) { return p.dux + (xb + i0 + r) * D; });
    bwd_load_rows_f32<D, LDF>(dcs, RB, nr, [&](int r) { return p.dcx + (xb + i0 + r) * D; });
    for (int r = threadIdx.x; r < RB; r += THREADS) {
      lser[r] = r < nr ? p.lser[xb + i0 + r] : 0.f;
      dhr[r] = r < nr ? p.dhx[xb + i0 + r] : 0.f;
    }
    __syncthreads();
    // R = exp2(sc2 q.k - lse2) and dR = du V^T + dc K^T, RB x nbp
    for (int t = wave; t < (RB / 16) * (nbp / 16); t += WAVES) {
      const int m0 = (t / (nbp / 16)) * 16, n0 = (t % (nbp / 16)) * 16;
      const f32x4 z = tile_mma<T, ROW, false, ROW, false>(qs, LDI, ks, LDI, m0, n0, D,
                                                          f32x4{0.f, 0.f, 0.f, 0.f});
      f32x4 dr = tile_mma<T, ROW, true, ROW, false>(dus, LDF, vs, LDI, m0, n0, D, f32x4{0.f, 0.f, 0.f, 0.f});
      dr = tile_mma<T, ROW, true, ROW, false>(dcs, LDF, ks, LDI, m0, n0, D, dr);
      const int key = n0 + lane % 16;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = m0 + 4 * g + e;
        const bool ok = r < nr && key < nb;
        rs[r * LDP + key] = ok ? __builtin_amdgcn_exp2f(z[e] * p.sc2 - lser[r]) : 0.f;
        dzs[r * LDP + key] = ok ? dr[e] : 0.f;
      }
    }
    __syncthreads();
    // G_i = sum_j R dR and H_i = -sum_j R log R
    for (int r = threadIdx.x; r < RB; r += THREADS) {
      float ga = 0.f, ha = 0.f;
      for (int j = 0; j < nbp; ++j) {
        const float rv = rs[r * LDP + j];
        ga += rv * dzs[r * LDP + j];
        ha -= rv > 0.f ? rv * __logf(rv) : 0.f;
      }
      gr[r] = ga;
      hr[r] = ha;
    }
    __syncthreads();
    // sc * dz = sc * (R (dR - G) - dH R (log R + H))
    for (int idx = threadIdx.x; idx < RB * nbp; idx += THREADS) {
      const int r = idx / nbp, j = idx % nbp;
      const float rv = rs[r * LDP + j];
      const float lg = rv > 0.f ? __logf(rv) : 0.f;
      dzs[r * LDP + j] = p.sc * rv * ((dzs[r * LDP + j] - gr[r]) - dhr[r] * (lg + hr[r]));
    }
    __syncthreads();
    // dQ = dQ (stage 2) + sc dz K, RB x D
    T* dQ = static_cast<T*>(p.dq) + (size_t)sl * p.N * D;
    for (int t = wave; t < (RB / 16) * (D / 16); t += WAVES) {
      const int m0 = (t / (D / 16)) * 16, n0 = (t % (D / 16)) * 16;
      const f32x4 a = tile_mma<T, ROW, true, COL, false>(dzs, LDP, ks, LDI, m0, n0, nbp,
                                                          f32x4{0.f, 0.f, 0.f, 0.f});
      const int d = n0 + lane % 16;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = m0 + 4 * g + e;
        if (r >= nr) continue;
        const int64_t tok = row.at(i0 + r);
        dQ[tok * D + d] = from_f32<T>(a[e] + p.dq2[((size_t)sl * p.N + tok) * D + d]);
      }
    }
    // dK += sc dz^T q + R^T dc, dV += R^T du (NB x D, over the chunk's rows)
#pragma unroll
    for (int j = 0; j < MJ; ++j) {
      const int t = wave + WAVES * j;
      const int m0 = (t / (D / 16)) * 16, n0 = (t % (D / 16)) * 16;
      if (m0 >= nbp) continue;
      adk[j] = tile_mma<T, COL, true, COL, false>(dzs, LDP, qs, LDI, m0, n0, RB, adk[j]);
      adk[j] = tile_mma<T, COL, true, COL, true>(rs, LDP, dcs, LDF, m0, n0, RB, adk[j]);
      adv[j] = tile_mma<T, COL, true, COL, true>(rs, LDP, dus, LDF, m0, n0, RB, adv[j]);
    }
  }
  T* dK = static_cast<T*>(p.dk) + (size_t)sl * p.N * D;
  T* dV = static_cast<T*>(p.dv) + (size_t)sl * p.N * D;
#pragma unroll
  for (int j = 0; j < MJ; ++j) {
    const int t = wave + WAVES * j;
    const int m0 = (t / (D / 16)) * 16, n0 = (t % (D / 16)) * 16;
    const int d = n0 + lane % 16;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int key = m0 + 4 * g + e;
      if (key >= nb) continue;
      const int64_t tok = row.at(key);
      dK[tok * D + d] = from_f32<T>(adk[j][e]);
      dV[tok * D + d] = from_f32<T>(adv[j][e]);
    }
  }
}

// The whole backward call on stream st: the forward's stage 1 (last-step
// kind: c, u, entropy, normaliser) and stage 2 statistics (row normalisers,
// no output) refill the workspace, then the two backward kernels run.
template <typename T, int D, bool PRECISE>
ma_status run_bwd_t(const Plan& pl, const BwdBufs& b, hipStream_t st) {
  Bufs fb{b.q, b.k, b.v, nullptr, b.ws, nullptr, nullptr, nullptr, nullptr};
  if (launch_one<T, D, PRECISE>(pl, fb, L_STAGE1_LAST, 0, st) != hipSuccess) return MA_ERR_DEVICE;
  if (launch_one<T, D, PRECISE>(pl, fb, L_STAGE2_STATS, 0, st) != hipSuccess) return MA_ERR_DEVICE;
  char* ws = b.ws;
  BwdParams p{b.q, b.k, b.v, b.dy, b.dq, b.dk, b.dv,
              ws + pl.off_cx, ws + pl.off_ux,
              reinterpret_cast<const float*>(ws + pl.off_lser),
              reinterpret_cast<const float*>(ws + pl.off_h2),
              reinterpret_cast<const float*>(ws + pl.off_lse2),
              reinterpret_cast<float*>(ws + pl.off_dq2),
              reinterpret_cast<float*>(ws + pl.off_dcx), reinterpret_cast<float*>(ws + pl.off_dux),
              reinterpret_cast<float*>(ws + pl.off_dhx),
              pl.map, (int)pl.S, (int)pl.N, pl.b1, pl.b2, pl.scale, pl.sc2};
  hipLaunchKernelGGL((stage2_bwd_kernel<T, D>), dim3(grid1((size_t)pl.S * pl.b2)), dim3(THREADS), 0, st, p);
  hipLaunchKernelGGL((stage1_bwd_kernel<T, D>), dim3(grid1((size_t)pl.S * pl.b1)), dim3(THREADS), 0, st, p);
  return hipGetLastError() == hipSuccess ? MA_OK : MA_ERR_DEVICE;
}

}  // namespace ma
