// Weight-streaming MFMA tile for skinny products (few tokens per weight row).
//
//   Y[tok][n] = sum_k W[n][k] * X[tok][k]      (one matrix), or
//   h[tok][n] = silu(G) * U with G, U the same product for two matrices.
//
// Work split: one 256-thread workgroup owns 16 weight rows (per matrix) and up
// to 64 tokens; its four waves take interleaved k-blocks of the contraction
// axis and their partial tiles are summed in LDS.  Weights stream straight
// from HBM into MFMA A-operand registers; each lane reads one contiguous run
// of its row per k-block (64 bytes: 32 bf16 or 128 FP4 codes plus their four
// E8M0 scales), four lanes cover 256 contiguous bytes of a row.  The
// contraction index is permuted identically on the A (weights) and B
// (activations) side: in MFMA step d a lane supplies elements [8d, 8d+8) of
// its own run, so the A and B lanes that meet in one k-slot always hold the
// same k.  Activations are bf16, read from L2 (they are small and shared by
// every weight tile).
//
// MFMA v_mfma_f32_16x16x32_bf16 operand layout (CDNA3/CDNA4 ISA):
//   A: lane l holds A[l%16][8*(l/16) .. +7], B: lane l holds B[8*(l/16) .. +7][l%16],
//   D: lane l holds D[4*(l/16) + v][l%16], v = 0..3.
#pragma once

#include "ft_internal.hpp"

namespace ft {

enum { WF_BF16 = 0, WF_FP4 = 1 };

constexpr int kStreamThreads = 256;
constexpr int kStreamMaxTok = 64;   // tokens per pass (4 MFMA column tiles)

// LDS floats needed by stream_tile<.., GLU, NT>.
template <bool GLU, int NT>
constexpr int stream_red_floats() { return 4 * (GLU ? 2 : 1) * NT * 256; }

// One 16-row x (16*NT)-token tile.  All 256 threads must call it.
//  w0/s0, w1/s1 : weight (codes) and scale bases of matrix 0 and 1 (row 0).
//  K            : contraction length (multiple of the k-block).
//  row0, N      : first weight row of the tile and the number of rows.
//  X, ldx       : bf16 activations; token j of the tile is row s_tok[j].
//  m            : valid tokens (1..16*NT).
//  out, ldo     : GLU -> bf16 h, else fp32; token j goes to row s_orow[j].
template <int WF, bool GLU, int NT>
__device__ __forceinline__ void stream_tile(const uint8_t *__restrict__ w0,
                                            const uint8_t *__restrict__ s0,
                                            const uint8_t *__restrict__ w1,
                                            const uint8_t *__restrict__ s1, int K, int row0, int N,
                                            const uint16_t *__restrict__ X, int64_t ldx,
                                            const int *__restrict__ s_tok, int m,
                                            float *__restrict__ s_red, void *__restrict__ out,
                                            int64_t ldo, const int *__restrict__ s_orow) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = lane & 15, q = lane >> 4;
  constexpr int MATS = GLU ? 2 : 1;
  constexpr int KB = (WF == WF_BF16) ? 128 : 512;  // elements per k-block
  constexpr int RUN = KB / 4;                      // elements per lane per k-block
  constexpr int DSTEPS = RUN / 8;                  // MFMA steps per k-block
  const int nkb = K / KB;

  f32x4 acc[MATS][NT];
#pragma unroll
  for (int mt = 0; mt < MATS; ++mt)
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) acc[mt][tt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const uint16_t *xrow[NT];
  bool xok[NT];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
    const int j = tt * 16 + r;
    xok[tt] = j < m;
    xrow[tt] = X + int64_t(s_tok[xok[tt] ? j : 0]) * ldx;
  }

  const int wrow = row0 + r;
  const bool rok = wrow < N;
  const int64_t crow = rok ? wrow : 0;
  const u32x4 zero4 = {0u, 0u, 0u, 0u};

  if constexpr (WF == WF_BF16) {
    const uint8_t *wr0 = w0 + crow * int64_t(K) * 2;
    const uint8_t *wr1 = GLU ? (w1 + crow * int64_t(K) * 2) : nullptr;
    for (int kb = wave; kb < nkb; kb += 4) {
      const int kofs = kb * KB + q * RUN;
      u32x4 a0[4], a1[4];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        a0[d] = rok ? ld16(wr0 + int64_t(kofs + 8 * d) * 2) : zero4;
        if constexpr (GLU) a1[d] = rok ? ld16(wr1 + int64_t(kofs + 8 * d) * 2) : zero4;
      }
#pragma unroll
      for (int d = 0; d < 4; ++d) {
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
          const u32x4 xb = xok[tt] ? ld16(xrow[tt] + kofs + 8 * d) : zero4;
          acc[0][tt] = mfma16(as_bf16x8(a0[d]), as_bf16x8(xb), acc[0][tt]);
          if constexpr (GLU) acc[MATS - 1][tt] = mfma16(as_bf16x8(a1[d]), as_bf16x8(xb), acc[MATS - 1][tt]);
        }
      }
    }
  } else {
    const uint8_t *cr0 = w0 + crow * int64_t(K / 2);
    const uint8_t *sr0 = s0 + crow * int64_t(K / 32);
    const uint8_t *cr1 = GLU ? (w1 + crow * int64_t(K / 2)) : nullptr;
    const uint8_t *sr1 = GLU ? (s1 + crow * int64_t(K / 32)) : nullptr;
    for (int kb = wave; kb < nkb; kb += 4) {
      const int kofs = kb * KB + q * RUN;
      u32x4 c0[4], c1[4];
      uint32_t sc0 = 0, sc1 = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        c0[i] = rok ? ld16(cr0 + kofs / 2 + 16 * i) : zero4;
        if constexpr (GLU) c1[i] = rok ? ld16(cr1 + kofs / 2 + 16 * i) : zero4;
      }
      sc0 = rok ? *reinterpret_cast<const uint32_t *>(sr0 + kofs / 32) : 0u;
      if constexpr (GLU) sc1 = rok ? *reinterpret_cast<const uint32_t *>(sr1 + kofs / 32) : 0u;
#pragma unroll
      for (int d = 0; d < DSTEPS; ++d) {
        const float f0 = e8m0_to_f32((sc0 >> (8 * (d / 4))) & 0xffu);
        const bf16x8 a0 = fp4x8_to_bf16x8(c0[d / 4][d % 4], f0);
        bf16x8 a1;
        if constexpr (GLU) {
          const float f1 = e8m0_to_f32((sc1 >> (8 * (d / 4))) & 0xffu);
          a1 = fp4x8_to_bf16x8(c1[d / 4][d % 4], f1);
        }
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
          const u32x4 xb = xok[tt] ? ld16(xrow[tt] + kofs + 8 * d) : zero4;
          acc[0][tt] = mfma16(a0, as_bf16x8(xb), acc[0][tt]);
          if constexpr (GLU) acc[MATS - 1][tt] = mfma16(a1, as_bf16x8(xb), acc[MATS - 1][tt]);
        }
      }
    }
  }

  // Sum the four waves' partial tiles.
#pragma unroll
  for (int mt = 0; mt < MATS; ++mt)
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
      *reinterpret_cast<f32x4 *>(&s_red[(((wave * MATS + mt) * NT + tt) * 64 + lane) * 4]) = acc[mt][tt];
  __syncthreads();
  for (int u = tid; u < NT * 64; u += kStreamThreads) {
    const int tt = u >> 6, ln = u & 63;
    const int j = tt * 16 + (ln & 15);
    const int n = row0 + 4 * (ln >> 4);
    if (j >= m || n >= N) continue;
    f32x4 g = {0.f, 0.f, 0.f, 0.f};
    f32x4 uu = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      g += *reinterpret_cast<const f32x4 *>(&s_red[(((w * MATS + 0) * NT + tt) * 64 + ln) * 4]);
      if constexpr (GLU)
        uu += *reinterpret_cast<const f32x4 *>(&s_red[(((w * MATS + 1) * NT + tt) * 64 + ln) * 4]);
    }
    const int64_t o = int64_t(s_orow[j]) * ldo + n;
    if constexpr (GLU) {
      uint16_t hv[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) hv[v] = f32_to_bf16_rne(silu(g[v]) * uu[v]);
      uint16_t *hp = reinterpret_cast<uint16_t *>(out) + o;
      if (n + 3 < N && (o & 3) == 0) {
        u32x2 pk = {uint32_t(hv[0]) | (uint32_t(hv[1]) << 16), uint32_t(hv[2]) | (uint32_t(hv[3]) << 16)};
        *reinterpret_cast<u32x2 *>(hp) = pk;
      } else {
        for (int v = 0; v < 4 && n + v < N; ++v) hp[v] = hv[v];
      }
    } else {
      float *yp = reinterpret_cast<float *>(out) + o;
      if (n + 3 < N && (o & 3) == 0) {
        *reinterpret_cast<f32x4 *>(yp) = g;
      } else {
        for (int v = 0; v < 4 && n + v < N; ++v) yp[v] = g[v];
      }
    }
  }
  __syncthreads();
}

// Dispatch on the number of 16-token column tiles (1..4).
template <int WF, bool GLU>
__device__ __forceinline__ void stream_tile_any(const uint8_t *w0, const uint8_t *s0, const uint8_t *w1,
                                                const uint8_t *s1, int K, int row0, int N,
                                                const uint16_t *X, int64_t ldx, const int *s_tok, int m,
                                                float *s_red, void *out, int64_t ldo, const int *s_orow) {
  switch ((m + 15) >> 4) {
    case 1: stream_tile<WF, GLU, 1>(w0, s0, w1, s1, K, row0, N, X, ldx, s_tok, m, s_red, out, ldo, s_orow); break;
    case 2: stream_tile<WF, GLU, 2>(w0, s0, w1, s1, K, row0, N, X, ldx, s_tok, m, s_red, out, ldo, s_orow); break;
    case 3: stream_tile<WF, GLU, 3>(w0, s0, w1, s1, K, row0, N, X, ldx, s_tok, m, s_red, out, ldo, s_orow); break;
    default: stream_tile<WF, GLU, 4>(w0, s0, w1, s1, K, row0, N, X, ldx, s_tok, m, s_red, out, ldo, s_orow); break;
  }
}

}  // namespace ft
