// Grouped block-scaled MFMA GEMM: the native MXFP4 expert mode.
//
//   stage 1: h[p][i] = silu(sum_k X[p][k] Wg[i][k]) * (sum_k X[p][k] Wu[i][k])
//   stage 2: y[p][n] = sum_k h[p][k] Wd[n][k]
//
// with X (and h) as MXFP8 E4M3 rows and the weights as stored, MXFP4 E2M1 with
// their E8M0 block scales, both fed straight to
// v_mfma_scale_f32_16x16x128_f8f6f4 (A = tokens, B = weights); nothing is
// decoded in registers.
//
// Workgroup = 4 waves; tile = 128 segment rows (tokens) x 256 weight rows, the
// same split as the exact-mode GEMM: stage 1 gives each wave 32 gate rows and
// the same 32 up rows, stage 2 64 weight rows; per wave 8 token tiles x 4
// weight tiles of 16x16 accumulators.  A chunk is 256 contraction elements,
// two MFMA steps, so the workgroup meets at a barrier once per 256 elements.
// Token codes of a chunk (128 rows x 256 bytes) and their scales (128 rows x
// 8 bytes) are gathered into LDS by direct buffer-to-LDS loads.  Weights go
// from global memory straight to registers (each weight row is used by one
// wave).  Two chunks are in flight while one is multiplied (three LDS buffers,
// three weight register sets); one workgroup per CU, the accumulators in
// AGPRs.
//
// Index maps per chunk c (MFMA steps s = 0, 1), lane (r, g):
//   token operand: row r of the 16-row tile, row bytes 128 s + 16 g .. +15 and
//                  128 s + 64 + 16 g .. +15; 16-byte piece j of a row is stored
//                  in slot j ^ (row % 16), so the 16 rows an MFMA operand reads
//                  hit distinct banks; scale = byte 4 s + g of the row's 8
//                  scale bytes of the chunk.
//   weight operand: row r of the tile, code bytes 128 c + 64 s + 16 g .. +15
//                   (elements 256 c + 128 s + 32 g .. +31); scale byte
//                   8 c + 4 s + g of the row.
// A segment's last tile runs with 4 or 2 of its 8 token sub-tiles when it
// holds <= 64 or <= 32 rows (the others would only multiply padding).
#pragma once

#include <type_traits>

#include "ft_internal.hpp"
#include "gemm_prefill.hpp"

namespace ft {

constexpr int kMxBK = 256;                               // contraction elements per chunk (two MFMA steps)
constexpr int kMxPitch = 256;                            // LDS bytes per token row (codes of one chunk)
constexpr int kMxCodeBytes = kGemmBM * kMxPitch;         // 32 KiB per buffer
constexpr int kMxScaleBytes = 4 * 256;                   // per wave: 32 rows x 8 B
constexpr int kMxBufBytes = kMxCodeBytes + kMxScaleBytes;
constexpr int kMxStages = 3;                             // LDS buffers (chunks in flight + 1)

struct MxGemmArgs {
  GemmArgs g;          // shapes, weights, segments and outputs (g.X, g.ldx, g.x_bytes unused)
  const uint8_t *Xq;   // E4M3 codes [rows, K]
  const uint8_t *Xs;   // E8M0 scales [rows, K / 32]
  uint32_t xq_bytes, xs_bytes;
};


template <bool GLU, int MT>
__device__ __forceinline__ void gemm_mx_body(const MxGemmArgs &ma, LdsRing<kMxStages> L, int nt_idx, int row0, int m,
                                             bool shared, const uint8_t *blob);

template <bool GLU>
__device__ __forceinline__ void gemm_mx_tile(const MxGemmArgs &ma, LdsRing<kMxStages> L) {
  int nt_idx, row0, m;
  bool shared;
  const uint8_t *blob;
  if (!gemm_setup<GLU>(ma.g, nt_idx, row0, m, shared, blob)) return;
  if (m > 64)
    gemm_mx_body<GLU, 8>(ma, L, nt_idx, row0, m, shared, blob);
  else if (m > 32)
    gemm_mx_body<GLU, 4>(ma, L, nt_idx, row0, m, shared, blob);
  else
    gemm_mx_body<GLU, 2>(ma, L, nt_idx, row0, m, shared, blob);
}

template <bool GLU, int MT>
__device__ __forceinline__ void gemm_mx_body(const MxGemmArgs &ma, LdsRing<kMxStages> L, int nt_idx, int row0, int m,
                                             bool shared, const uint8_t *blob) {
  const GemmArgs &a = ma.g;
  constexpr int NT = 4;  // weight tiles (16 rows) per wave
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = lane & 15, q = lane >> 4;
  (void)tid;
  auto src_row = [&](int rr) -> int {
    if (rr >= m) return -1;
    if (a.sorted_rows == nullptr) return (shared ? a.T * a.k : 0) + row0 + rr;  // hidden row
    if (shared) return row0 + rr;                                             // token
    return a.sorted_rows[row0 + rr] / a.k;                                    // gathered token
  };

  // ---- token codes: wave w fills rows 32w..32w+31 with 8 direct loads of 4
  // rows each (lane i: row 4t + i/16, slot i%16); scales: one 4-byte direct
  // load per wave into its own 256-byte area (lane i: row 32w + i/2, bytes
  // 4 (i%2) .. +3 of the row's 8 scale bytes of the chunk)
  const uint32_t kq = uint32_t(a.K), ks32 = uint32_t(a.K) / 32;
  const rsrc_t qres = make_rsrc(ma.Xq, ma.xq_bytes);
  const rsrc_t sres_x = make_rsrc(ma.Xs, ma.xs_bytes);
  uint32_t qsrc[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int rr = wave * 32 + t * 4 + (lane >> 4);
    const int src = src_row(rr);
    const int j = (lane & 15) ^ (rr & 15);
    qsrc[t] = src >= 0 ? uint32_t(src) * kq + uint32_t(j) * 16u : kOOB;
  }
  uint32_t ssrc = kOOB;
  {
    const int src = src_row(wave * 32 + (lane >> 1));
    ssrc = src >= 0 ? uint32_t(src) * ks32 + uint32_t(lane & 1) * 4u : kOOB;
  }

  // ---- weights of this wave
  const uint32_t wpitch = uint32_t(a.K) / 2, spitch = uint32_t(a.K) / 32;
  const uint32_t wbytes = uint32_t(a.N) * wpitch, sbytes = uint32_t(a.N) * spitch;
  rsrc_t wres[NT], sres[NT];
  uint32_t wrow[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    int row;
    const uint8_t *wb, *sb;
    if (GLU) {
      row = nt_idx * (kGemmBN / 2) + wave * 32 + (t & 1) * 16 + r;
      wb = blob + (t < 2 ? a.off_w0 : a.off_w1);
      sb = blob + (t < 2 ? a.off_s0 : a.off_s1);
    } else {
      row = nt_idx * kGemmBN + wave * 64 + t * 16 + r;
      wb = blob + a.off_w0;
      sb = blob + a.off_s0;
    }
    wres[t] = make_rsrc(wb, wbytes);
    sres[t] = make_rsrc(sb, sbytes);
    wrow[t] = uint32_t(row);
  }
  struct BFrag {
    u32x4 w[NT][2];  // MFMA steps 0, 1 of the chunk
    u32x2 s[NT];     // 8 scale bytes: step s, block g at byte 4 s + g
  };
  const int nch = a.K / kMxBK;
  // A chunk past the end is still issued, with out-of-range offsets (no memory
  // traffic, zeros): every step then has the same loads in flight, and the
  // vmcnt arithmetic below holds on every path.
  auto load_b = [&](int c, BFrag &f) {
    const bool live = c < nch;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      f.w[t][0] = bld16(wres[t], live ? wrow[t] * wpitch + uint32_t(c) * 128u + q * 16 : kOOB);
      f.w[t][1] = bld16(wres[t], live ? wrow[t] * wpitch + uint32_t(c) * 128u + 64u + q * 16 : kOOB);
      f.s[t] = bld8(sres[t], live ? wrow[t] * spitch + uint32_t(c) * 8u : kOOB);
    }
  };
  auto load_a = [&](int c, uint8_t *base) {
    const bool live = c < nch;
    uint8_t *cb = base + wave * 32 * kMxPitch;
#pragma unroll
    for (int t = 0; t < 8; ++t)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          qres, (__attribute__((address_space(3))) void *)(cb + t * 4 * kMxPitch), 16,
          (qsrc[t] == kOOB || !live) ? kOOB : qsrc[t] + uint32_t(c) * 256u, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        sres_x, (__attribute__((address_space(3))) void *)(base + kMxCodeBytes + wave * 256), 4,
        (ssrc == kOOB || !live) ? kOOB : ssrc + uint32_t(c) * 8u, 0, 0, 0);
  };

  f32x4 acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // this lane's LDS read addresses in buffer 0, tile 0: the two 16-byte pieces
  // of its row for each MFMA step and the row's scale bytes; tile i adds i * 16
  // rows (the slot map depends on row % 16 only)
  int oa_lo[2], oa_hi[2];
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    oa_lo[st] = r * kMxPitch + (((8 * st + q) ^ r) << 4);
    oa_hi[st] = r * kMxPitch + (((8 * st + 4 + q) ^ r) << 4);
  }
  const int oa_s = kMxCodeBytes + r * 8;
  // ---- pipeline: P chunks in flight ahead of the one being multiplied, in
  // P + 1 LDS buffers and P + 1 weight register sets (a ring, unrolled so the
  // register set of every step is fixed at compile time)
  constexpr int NBUF = kMxStages;
  constexpr int P = NBUF - 1;
  constexpr int LOADS = 8 + 1 + 3 * NT;  // vector-memory instructions per chunk and wave
  BFrag fr[NBUF];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    load_a(p, L.b[p]);
    load_b(p, fr[p]);
  }
  wait_vmcnt<(P - 1) * LOADS>();  // chunk 0 has landed
  lds_barrier();

  auto body = [&](auto jc, int c) {
    constexpr int J = decltype(jc)::value;
    load_a(c + P, L.b[(J + P) % NBUF]);  // the buffer and registers the previous chunk used
    load_b(c + P, fr[(J + P) % NBUF]);
    if (c < nch) {
      const BFrag &f = fr[J];
      const uint8_t *buf = L.b[J];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        i32x8 bw[NT];
        int bs[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          // FP4 operands use the low four dwords only
          bw[t] = __builtin_bit_cast(i32x8,
                                     __builtin_shufflevector(f.w[t][st], f.w[t][st], 0, 1, 2, 3, -1, -1, -1, -1));
          bs[t] = int(f.s[t][st] >> (8 * q));
        }
#pragma unroll
        for (int i = 0; i < MT; ++i) {
          const u32x4 lo = *reinterpret_cast<const u32x4 *>(buf + oa_lo[st] + i * 16 * kMxPitch);
          const u32x4 hi = *reinterpret_cast<const u32x4 *>(buf + oa_hi[st] + i * 16 * kMxPitch);
          // scales: wave area (row / 32) * 256, row (row % 32) * 8, step st
          const int as = int(*reinterpret_cast<const uint32_t *>(buf + oa_s + (i >> 1) * 256 + (i & 1) * 128 + 4 * st) >>
                             (8 * q));
          const i32x8 av = __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
          for (int t = 0; t < NT; ++t) acc[i][t] = mfma_mx(av, bw[t], acc[i][t], as, bs[t]);
        }
      }
    }
    wait_vmcnt<(P - 1) * LOADS>();  // chunk c + 1 has landed; c + 2 .. c + P may still fly
    lds_barrier();
  };
  static_assert((P - 1) * LOADS < 64, "vmcnt is six bits");
  for (int c = 0; c < nch; c += NBUF)
    unroll_ring([&](auto jc) { body(jc, c + decltype(jc)::value); }, std::make_integer_sequence<int, NBUF>{});
  wait_vmcnt<0>();

  // ---- epilogue: lane holds D[token 4q+v][weight row r] of each tile
#pragma unroll
  for (int i = 0; i < MT; ++i) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int rr = i * 16 + 4 * q + v;
      if (rr >= m) continue;
      if constexpr (GLU) {
        const int hrow = shared ? a.T * a.k + row0 + rr : row0 + rr;
        uint16_t *hp = reinterpret_cast<uint16_t *>(a.out) + int64_t(hrow) * a.ldo;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int col = nt_idx * (kGemmBN / 2) + wave * 32 + t * 16 + r;
          if (col < a.N) hp[col] = f32_to_bf16_rne(silu(acc[i][t][v]) * acc[i][t + 2][v]);
        }
      } else {
        float *yp = shared ? a.out_shared + int64_t(row0 + rr) * a.ldo
                           : reinterpret_cast<float *>(a.out) + int64_t(row0 + rr) * a.ldo;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const int col = nt_idx * kGemmBN + wave * 64 + t * 16 + r;
          if (col < a.N) yp[col] = acc[i][t][v];
        }
      }
    }
  }
}

}  // namespace ft
