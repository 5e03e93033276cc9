// Weight-streaming MFMA tile for skinny products (few tokens per weight row).
//
//   Y[tok][n] = sum_k W[n][k] * X[tok][k]      (one matrix), or
//   h[tok][n] = silu(G) * U with G, U the same product for two matrices.
//
// Work split: one workgroup of WAVES waves owns 16 weight rows (per matrix)
// and up to 16*NT tokens; the waves take interleaved k-blocks of the
// contraction axis and their partial tiles are summed in LDS.  Weights stream
// from HBM straight into MFMA A-operand registers (bf16 and MXFP4: read as
// whole 128-byte lines and moved into the operand layout in registers, see
// wfrag_fix).
// Activations are bf16 and are read from L2 (small, shared by every weight
// tile).
//
// All loads are raw buffer loads with 32-bit offsets.  Rows past N and token
// columns past m get an out-of-range offset, so they load zeros without a
// branch and without memory traffic.  All loads of a k-block are issued
// before its first MFMA; with two k-blocks in flight, the activation loads of
// this k-block go out before the next k-block's weights, so the in-order
// vector-memory counter lets this k-block's MFMAs start while the next
// weights are still in flight.
//
// v_mfma_f32_16x16x32_bf16 operand layout (CDNA3/CDNA4 ISA):
//   A: lane l holds A[l%16][8*(l/16) .. +7], B: lane l holds B[8*(l/16) .. +7][l%16],
//   D: lane l holds D[4*(l/16) + v][l%16], v = 0..3.
//
// k-block = DL 16-byte loads per lane:
//   bf16: 256 bytes of a row = 128 elements (two lines, four loads);
//   FP4 : 128 bytes of a row = 256 elements (one line, two loads); after
//         wfrag_fix register a of lane (r, q) holds E8M0 block 2q + a, and
//         MFMA (a, m), m = 0..3, takes its elements 8m .. 8m+7.  The 8 scale
//         bytes of the k-block come in one 8-byte load per row;
//   NVFP4: 64 bytes of a row = 128 elements (one load in the operand layout).
// The activations are read with the same element map (wl_xk), so each MFMA
// pairs equal k.
#pragma once

#include "ft_internal.hpp"

namespace ft {

// weight formats of the streaming kernels: bf16, MXFP4, NVFP4
enum { WF_BF16 = 0, WF_FP4 = 1, WF_NV4 = 2 };

constexpr int kStreamMaxTok = 64;  // tokens per pass (4 MFMA column tiles)

// Elements of the contraction axis per k-block.
template <int WF>
constexpr int stream_kblock() { return WF == WF_FP4 ? 256 : 128; }

// LDS floats needed by stream_tile<.., GLU, NT, WAVES>.
template <bool GLU, int NT, int WAVES>
constexpr int stream_red_floats() { return WAVES * (GLU ? 2 : 1) * NT * 256; }

template <int WF, int MATS>
struct WFrag {
  static constexpr int DL = WF == WF_BF16 ? 4 : (WF == WF_FP4 ? 2 : 1);  // 16-byte weight loads per lane per k-block
  u32x4 w[MATS][DL];
  u32x2 s[MATS];
};

// ---- weight loads by whole 128-byte lines (bf16 and MXFP4)
//
// In the A-operand layout one load reads 64 bytes of each of 16 rows, half of every line it
// touches.  Instead load d of a k-block reads tile row 8 (d & 1) + (lane & 7), bytes
// 128 (d >> 1) + 16 (lane >> 3) .. +15 of the k-block, and wfrag_fix moves the data into the operand
// layout (for each pair of loads a lane whose bit 3 is set swaps in the partner half through a DPP
// rotation by 8 lanes).  Afterwards register d + a (a = 0, 1) holds at lane (r, q) row r, bytes
// 128 (d >> 1) + 32 q + 16 a .. +15 of the k-block: bf16 elements 64 (d >> 1) + 16 q + 8 a .. +7
// (MFMA d + a); FP4 elements 64 q + 32 a .. +31 = E8M0 block 2q + a.  wl_xk gives the activations
// the matching element map.  The decode kernels' weight loads (wl_load) also carry the
// non-temporal bit: each weight byte is read once per call.  Measured on MI355X (decode layer
// steps): whole lines with the bit 231 -> 216 us (bf16, 64 tokens), 158 -> 148 us (16 tokens),
// 367 -> 342 us (MXFP4, 32 tokens); whole lines alone or the bit alone gained nothing or lost (with
// half-line loads the bit made the line's second half come from HBM again).  A 1 GiB read probe
// gave 5.96 TB/s in the operand pattern, 6.85 TB/s in whole lines.  NVFP4 k-blocks are half a line
// and keep the operand layout and plain loads.
template <int WF>
constexpr bool wl_lines() { return WF != WF_NV4; }
template <int WF>
constexpr int wl_halves() { return wl_lines<WF>() ? 2 : 1; }
// Tile row (0..15) that this lane reads in load d of a k-block, and the byte offset inside the k-block.
template <int WF>
__device__ __forceinline__ int wl_row(int lane, int d) { return wl_lines<WF>() ? 8 * (d & 1) + (lane & 7) : (lane & 15); }
template <int WF>
__device__ __forceinline__ uint32_t wl_byte(int lane, int d) {
  return wl_lines<WF>() ? uint32_t(128 * (d >> 1) + 16 * (lane >> 3)) : uint32_t(64 * d + 16 * (lane >> 4));
}
// Offset of load d relative to load d % halves of the same rows.
template <int WF>
__device__ __forceinline__ uint32_t wl_dcol(int d) { return wl_lines<WF>() ? uint32_t(d >> 1) * 128u : uint32_t(d) * 64u; }
template <int WF>
constexpr uint32_t wl_kbytes() { return WFrag<WF, 1>::DL * 64; }
__device__ __forceinline__ uint32_t dpp_ror8(uint32_t v) {
  return uint32_t(__builtin_amdgcn_mov_dpp(int(v), 0x128, 0xf, 0xf, true));  // row_ror:8
}
__device__ __forceinline__ void wl_swap(u32x4 &x0, u32x4 &x1) {
  const bool up = (threadIdx.x & 8) != 0;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const uint32_t a = x0[c], b = x1[c];
    const uint32_t ra = dpp_ror8(a), rb = dpp_ror8(b);
    x0[c] = up ? rb : a;
    x1[c] = up ? b : ra;
  }
}
template <int WF, int MATS>
__device__ __forceinline__ void wfrag_fix(WFrag<WF, MATS> &f) {
  if constexpr (wl_lines<WF>()) {
#pragma unroll
    for (int mt = 0; mt < MATS; ++mt)
#pragma unroll
      for (int d = 0; d < WFrag<WF, MATS>::DL; d += 2) wl_swap(f.w[mt][d], f.w[mt][d + 1]);
  }
}
// Element offset inside the k-block of activation load dx of lane group q (bf16: MFMA dx; FP4:
// MFMA dx = 4 a + mm; NVFP4: word dx of lane q's 32 elements).
template <int WF>
__device__ __forceinline__ int wl_xk(int dx, int q) {
  return WF == WF_BF16 ? 64 * (dx >> 1) + 16 * q + 8 * (dx & 1)
         : WF == WF_FP4 ? 32 * (dx >> 2) + 64 * q + 8 * (dx & 3)
                        : 32 * q + 8 * dx;
}
// MXFP4: the E8M0 scale of the block in register a of lane group q (block 2q + a of the row's eight).
template <int WF>
__device__ __forceinline__ uint32_t wl_mx_scale(const u32x2 &s, int a, int q) {
  return ((q >> 1) ? s[1] : s[0]) >> (8 * (2 * (q & 1) + a)) & 0xffu;
}
// A decode kernel's weight load: whole lines with the non-temporal bit, NVFP4 half lines without.
template <int WF>
__device__ __forceinline__ u32x4 wl_load(rsrc_t r, uint32_t off) {
  if constexpr (wl_lines<WF>()) return bld16nt(r, off);
  else return bld16(r, off);
}

// One 16-row x (16*NT)-token tile.  All WAVES*64 threads must call it.
//  w0/s0, w1/s1 : weight (codes) and scale bases of matrix 0 and 1 (row 0).
//  K            : contraction length (multiple of the k-block).
//  row0, N      : first weight row of the tile and the number of rows.
//  X, ldx       : bf16 activations; token j of the tile is row s_tok[j];
//  x_bytes      : bytes of the whole activation buffer (bounds the offsets).
//  m            : valid tokens (1..16*NT).
//  out, ldo     : GLU -> bf16 h, else fp32; token j goes to row s_orow[j].
template <int WF, bool GLU, int NT, int WAVES, bool PIPE>
__device__ __forceinline__ void stream_tile(const uint8_t *__restrict__ w0,
                                            const uint8_t *__restrict__ s0,
                                            const uint8_t *__restrict__ w1,
                                            const uint8_t *__restrict__ s1, int K, int row0, int N,
                                            const uint16_t *__restrict__ X, int64_t ldx, uint32_t x_bytes,
                                            const int *__restrict__ s_tok, int m,
                                            float *__restrict__ s_red, void *__restrict__ out,
                                            int64_t ldo, const int *__restrict__ s_orow) {
  constexpr int THREADS = WAVES * 64;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = lane & 15, q = lane >> 4;
  constexpr int MATS = GLU ? 2 : 1;
  constexpr int KB = stream_kblock<WF>();
  constexpr int DL = WFrag<WF, MATS>::DL;
  constexpr int DX = WF == WF_BF16 ? 4 : 8;  // 16-byte activation loads per lane per k-block per column tile
  const int nkb = K / KB;

  f32x4 acc[MATS][NT];
#pragma unroll
  for (int mt = 0; mt < MATS; ++mt)
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) acc[mt][tt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // byte offset of token column r of tile tt (out of range past m)
  const rsrc_t xres = make_rsrc(X, x_bytes);
  uint32_t xo[NT];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
    const int j = tt * 16 + r;
    xo[tt] = j < m ? uint32_t(s_tok[j]) * uint32_t(ldx) * 2u : kOOB;
  }

  // byte pitch of one weight row and of its scale row
  const uint32_t wpitch = (WF == WF_BF16) ? uint32_t(K) * 2 : uint32_t(K) / 2;
  const uint32_t spitch = uint32_t(K) / 32;
  rsrc_t wres[MATS], sres[MATS];
  wres[0] = make_rsrc(w0, uint32_t(N) * wpitch);
  sres[0] = make_rsrc(s0, uint32_t(N) * spitch);
  if constexpr (GLU) {
    wres[MATS - 1] = make_rsrc(w1, uint32_t(N) * wpitch);
    sres[MATS - 1] = make_rsrc(s1, uint32_t(N) * spitch);
  }
  // rows past N fall outside the buffer; the scales are those of the lane's own operand row r
  const uint32_t so = uint32_t(row0 + r) * spitch;

  auto load_w = [&](int kb, WFrag<WF, MATS> &f) {
#pragma unroll
    for (int mt = 0; mt < MATS; ++mt) {
#pragma unroll
      for (int d = 0; d < DL; ++d)
        f.w[mt][d] = bld16(wres[mt], uint32_t(row0 + wl_row<WF>(lane, d)) * wpitch + uint32_t(kb) * wl_kbytes<WF>() +
                                         wl_byte<WF>(lane, d));  // plain: a router's rows serve every token tile
      if constexpr (WF == WF_FP4) f.s[mt] = bld8(sres[mt], so + uint32_t(kb) * 8);
    }
  };
  // activation element offset of this lane's load dx of k-block kb
  auto xoff = [&](int kb, int dx) { return kb * KB + wl_xk<WF>(dx, q); };
  auto load_x = [&](int kb, u32x4 (&xb)[NT][DX]) {
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
      for (int dx = 0; dx < DX; ++dx) xb[tt][dx] = bld16(xres, xo[tt] + uint32_t(xoff(kb, dx)) * 2u);
  };
  auto compute = [&](WFrag<WF, MATS> f, const u32x4 (&xb)[NT][DX]) {
    wfrag_fix(f);
    if constexpr (WF == WF_BF16) {
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
          for (int mt = 0; mt < MATS; ++mt)
            acc[mt][tt] = mfma16(as_bf16x8(f.w[mt][d]), as_bf16x8(xb[tt][d]), acc[mt][tt]);
    } else {
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        float sc[MATS];
#pragma unroll
        for (int mt = 0; mt < MATS; ++mt) sc[mt] = e8m0_to_f32(wl_mx_scale<WF>(f.s[mt], d, q));
#pragma unroll
        for (int mm = 0; mm < 4; ++mm) {
          bf16x8 a[MATS];
#pragma unroll
          for (int mt = 0; mt < MATS; ++mt) a[mt] = fp4x8_to_bf16x8(f.w[mt][d][mm], sc[mt]);
#pragma unroll
          for (int tt = 0; tt < NT; ++tt)
#pragma unroll
            for (int mt = 0; mt < MATS; ++mt)
              acc[mt][tt] = mfma16(a[mt], as_bf16x8(xb[tt][4 * d + mm]), acc[mt][tt]);
        }
      }
    }
  };

  if constexpr (PIPE) {
    // The next k-block's weights are in flight while this one is multiplied.
    WFrag<WF, MATS> fa, fb;
    u32x4 xb[NT][DX];
    int kb = wave;
    if (kb < nkb) load_w(kb, fa);
    while (kb < nkb) {
      const int k1 = kb + WAVES;
      load_x(kb, xb);
      __builtin_amdgcn_sched_barrier(0);
      if (k1 < nkb) load_w(k1, fb);
      __builtin_amdgcn_sched_barrier(0);
      compute(fa, xb);
      if (k1 >= nkb) break;
      const int k2 = k1 + WAVES;
      load_x(k1, xb);
      __builtin_amdgcn_sched_barrier(0);
      if (k2 < nkb) load_w(k2, fa);
      __builtin_amdgcn_sched_barrier(0);
      compute(fb, xb);
      kb = k2;
    }
  } else {
    for (int kb = wave; kb < nkb; kb += WAVES) {
      WFrag<WF, MATS> fa;
      u32x4 xb[NT][DX];
      load_w(kb, fa);
      load_x(kb, xb);
      __builtin_amdgcn_sched_barrier(0);
      compute(fa, xb);
    }
  }

  // Sum the waves' partial tiles.
#pragma unroll
  for (int mt = 0; mt < MATS; ++mt)
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
      *reinterpret_cast<f32x4 *>(&s_red[(((wave * MATS + mt) * NT + tt) * 64 + lane) * 4]) = acc[mt][tt];
  __syncthreads();
  for (int u = tid; u < NT * 64; u += THREADS) {
    const int tt = u >> 6, ln = u & 63;
    const int j = tt * 16 + (ln & 15);
    const int n = row0 + 4 * (ln >> 4);
    if (j >= m || n >= N) continue;
    f32x4 g = {0.f, 0.f, 0.f, 0.f};
    f32x4 uu = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
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

// Dispatch on the number of 16-token column tiles (1..NTMAX).
template <int WF, bool GLU, int NTMAX, int WAVES, bool PIPE>
__device__ __forceinline__ void stream_tile_any(const uint8_t *w0, const uint8_t *s0, const uint8_t *w1,
                                                const uint8_t *s1, int K, int row0, int N,
                                                const uint16_t *X, int64_t ldx, uint32_t x_bytes, const int *s_tok,
                                                int m, float *s_red, void *out, int64_t ldo, const int *s_orow) {
  const int nt = (m + 15) >> 4;
  if (NTMAX == 1 || nt <= 1) {
    stream_tile<WF, GLU, 1, WAVES, PIPE>(w0, s0, w1, s1, K, row0, N, X, ldx, x_bytes, s_tok, m, s_red, out, ldo, s_orow);
  } else if (NTMAX == 2 || nt == 2) {
    stream_tile<WF, GLU, (NTMAX >= 2 ? 2 : 1), WAVES, PIPE>(w0, s0, w1, s1, K, row0, N, X, ldx, x_bytes, s_tok, m,
                                                            s_red, out, ldo, s_orow);
  } else if (nt == 3) {
    stream_tile<WF, GLU, (NTMAX >= 3 ? 3 : 1), WAVES, PIPE>(w0, s0, w1, s1, K, row0, N, X, ldx, x_bytes, s_tok, m,
                                                            s_red, out, ldo, s_orow);
  } else {
    stream_tile<WF, GLU, NTMAX, WAVES, PIPE>(w0, s0, w1, s1, K, row0, N, X, ldx, x_bytes, s_tok, m, s_red, out,
                                             ldo, s_orow);
  }
}

// Launch shape of a streaming tile: tokens per pass (16*NTMAX), waves per
// workgroup, and whether each wave keeps two k-blocks in flight.
struct StreamShape {
  int ntmax, waves;
  bool pipe;
};

// T bounds the tokens of any segment; nkb = k-blocks of the contraction axis.
// Decode batches (T <= 64) use one 16-token column tile per pass (longer
// segments take several passes); each wave gets one k-block when the
// contraction axis has at most 16 of them, else two or more in flight.
inline StreamShape stream_shape(int T, int nkb) {
  const int ntmax = T <= 64 ? 1 : 2;
  for (int w : {16, 8, 6, 4})
    if (nkb % w == 0) return {ntmax, w, nkb > w};
  return {ntmax, 4, nkb > 4};
}

}  // namespace ft
