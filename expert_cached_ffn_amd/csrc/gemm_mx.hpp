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
// Token codes of a chunk (128 rows x 256 bytes) are gathered into LDS by
// direct buffer-to-LDS loads.  Weights go from global memory straight to
// registers (each weight row is used by one wave).  Two chunks are in flight
// while one is multiplied (three LDS buffers, three weight register sets); one
// workgroup per CU, the accumulators in AGPRs.
//
// Block scales are not fetched per chunk: a chunk needs 8 bytes of each row,
// and fetching them one chunk at a time costs the L1 a request per row for 8
// bytes.  Instead each row's scales of a window of 16 chunks (128 bytes, one
// cache line) are copied into LDS once -- for the 256 weight rows and the 128
// token rows of the tile -- and every chunk reads its 8 bytes per row from
// there.  A window covers K <= 4096 whole; longer rows load the next window
// at its first chunk, with the pipeline drained around that load.
//
// Index maps per chunk c (MFMA steps s = 0, 1), lane (r, g):
//   token operand: row r of the 16-row tile, row bytes 128 s + 16 g .. +15 and
//                  128 s + 64 + 16 g .. +15; 16-byte piece j of a row is stored
//                  in slot j ^ (row % 16), so the 16 rows an MFMA operand reads
//                  hit distinct banks.
//   weight operand: row r of the tile, code bytes 128 c + 64 s + 16 g .. +15
//                   (elements 256 c + 128 s + 32 g .. +31).
//   scales (either operand): byte 8 c + 4 s + g of the row's scales.  In the
//                  LDS copy a row takes P bytes (128, or the row's scale bytes
//                  rounded up to a power of two >= 16 when they are fewer), and
//                  its 16-byte piece j is stored in slot j ^ f(row % 16) with
//                  f(R) = (R / (16 / (P/16))) mod (P/16), so that the 16 rows
//                  one read touches sit in distinct banks.
// A segment's last tile runs with 4 or 2 of its 8 token sub-tiles when it
// holds <= 64 or <= 32 rows (the others would only multiply padding).
#pragma once

#include <type_traits>

#include "ft_internal.hpp"
#include "gemm_prefill.hpp"

namespace ft {

constexpr int kMxBK = 256;                        // contraction elements per chunk (two MFMA steps)
constexpr int kMxPitch = 256;                     // LDS bytes per token row (codes of one chunk)
constexpr int kMxCodeBytes = kGemmBM * kMxPitch;  // 32 KiB per buffer
constexpr int kMxStages = 3;                      // LDS code buffers (chunks in flight + 1)
constexpr int kMxSWin = 128;                      // scale bytes per row in one window (16 chunks)
constexpr int kMxWScaleBytes = kGemmBN * kMxSWin; // weight scales of a window: 32 KiB
constexpr int kMxXScaleBytes = kGemmBM * kMxSWin; // token scales of a window: 16 KiB

struct MxGemmArgs {
  GemmArgs g;          // shapes, weights, segments and outputs (g.X, g.ldx, g.x_bytes unused)
  const uint8_t *Xq;   // E4M3 codes [rows, K]
  const uint8_t *Xs;   // E8M0 scales [rows, K / 32]
  uint32_t xq_bytes, xs_bytes;
};

// LDS of one workgroup: the code ring and the two scale windows.
struct MxLds {
  LdsRing<kMxStages> code;
  uint8_t *wsc;  // [4 waves][64 rows][P], 8 KiB per wave
  uint8_t *xsc;  // [4 waves][32 rows][P], 4 KiB per wave
};

template <bool GLU, int MT>
__device__ __forceinline__ void gemm_mx_body(const MxGemmArgs &ma, const MxLds &L, int nt_idx, int row0, int m,
                                             bool shared, const uint8_t *blob);

template <bool GLU>
__device__ __forceinline__ void gemm_mx_tile(const MxGemmArgs &ma, const MxLds &L) {
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
__device__ __forceinline__ void gemm_mx_body(const MxGemmArgs &ma, const MxLds &L, int nt_idx, int row0, int m,
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
  // rows each (lane i: row 4t + i/16, slot i%16)
  const uint32_t kq = uint32_t(a.K);
  const rsrc_t qres = make_rsrc(ma.Xq, ma.xq_bytes);
  uint32_t qsrc[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int rr = wave * 32 + t * 4 + (lane >> 4);
    const int src = src_row(rr);
    const int j = (lane & 15) ^ (rr & 15);
    qsrc[t] = src >= 0 ? uint32_t(src) * kq + uint32_t(j) * 16u : kOOB;
  }

  // ---- weight codes of this wave
  const uint32_t wpitch = uint32_t(a.K) / 2;
  const uint32_t wbytes = uint32_t(a.N) * wpitch;
  rsrc_t wres[NT];
  uint32_t wbase[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    int row;
    const uint8_t *wb;
    if (GLU) {
      row = nt_idx * (kGemmBN / 2) + wave * 32 + (t & 1) * 16 + r;
      wb = blob + (t < 2 ? a.off_w0 : a.off_w1);
    } else {
      row = nt_idx * kGemmBN + wave * 64 + t * 16 + r;
      wb = blob + a.off_w0;
    }
    wres[t] = make_rsrc(wb, wbytes);
    wbase[t] = uint32_t(row) * wpitch + q * 16;  // rows past N fall outside the buffer
  }

  // ---- scale windows: P bytes per row in LDS, 16-byte pieces swizzled by f
  const int srow = a.K / 32;  // scale bytes per row
  int P = kMxSWin;
  if (srow < kMxSWin) {
    P = 16;
    while (P < srow) P <<= 1;
  }
  const int ppr = P / 16;  // pieces per row: 1, 2, 4 or 8
  auto fsw = [&](int R) { return (R / (16 / ppr)) & (ppr - 1); };
  const rsrc_t bres = make_rsrc(blob, uint32_t(a.expert_bytes));
  const rsrc_t xsres = make_rsrc(ma.Xs, ma.xs_bytes);
  uint8_t *const wsc_w = L.wsc + wave * (64 * kMxSWin);
  uint8_t *const xsc_w = L.xsc + wave * (32 * kMxSWin);
  // window win of this wave's 64 weight rows (ppr loads of 1 KiB) and 32 token
  // rows (max(1, ppr / 2) loads); lane i of load n covers row (64 n + i) / ppr,
  // slot (64 n + i) % ppr
  auto load_scales = [&](int win) {
    const uint32_t woff = uint32_t(win) * kMxSWin;
    for (int n = 0; n < ppr; ++n) {
      const int u = n * 64 + lane, rho = u / ppr, j = u % ppr;
      const int piece = j ^ fsw(rho & 15);
      int row;
      uint64_t moff;
      if (GLU) {
        row = nt_idx * (kGemmBN / 2) + wave * 32 + (rho & 31);
        moff = rho < 32 ? a.off_s0 : a.off_s1;
      } else {
        row = nt_idx * kGemmBN + wave * 64 + rho;
        moff = a.off_s0;
      }
      const uint32_t off = row < a.N ? uint32_t(moff) + uint32_t(row) * uint32_t(srow) + woff + uint32_t(piece) * 16u
                                     : kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(bres, (__attribute__((address_space(3))) void *)(wsc_w + n * 1024), 16,
                                               off, 0, 0, 0);
    }
    const int nx = ppr > 2 ? ppr / 2 : 1;
    for (int n = 0; n < nx; ++n) {
      const int u = n * 64 + lane, rho = u / ppr, j = u % ppr;
      const int piece = j ^ fsw(rho & 15);
      const int src = rho < 32 ? src_row(wave * 32 + rho) : -1;
      const uint32_t off = src >= 0 ? uint32_t(src) * uint32_t(srow) + woff + uint32_t(piece) * 16u : kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xsres, (__attribute__((address_space(3))) void *)(xsc_w + n * 1024),
                                               16, off, 0, 0, 0);
    }
  };
  // this lane's scale rows in LDS: weight tile t adds 16 t P; token tile i
  // adds (i / 2) 4096 (the wave area of its rows) + (i % 2) 16 P
  const int f_r = fsw(r);
  const uint8_t *const wsc_t = L.wsc + wave * (64 * kMxSWin) + r * P;
  const uint8_t *const xsc_t = L.xsc + r * P;

  struct BFrag {
    u32x4 w[NT][2];  // MFMA steps 0, 1 of the chunk
  };
  const int nch = a.K / kMxBK;
  // A chunk past the end is still issued, with out-of-range offsets (no memory
  // traffic, zeros): every step then has the same loads in flight, and the
  // vmcnt arithmetic below holds on every path.  Offsets of such a chunk get
  // bit 31 set (kOOB) by an OR with a wave-uniform word rather than a select:
  // every offset below stays under 2^31, and an offset that is already kOOB
  // stays past the buffer.
  auto dead_bit = [&](int c) -> uint32_t { return c < nch ? 0u : kOOB; };
  auto load_b = [&](int c, BFrag &f) {
    const uint32_t dead = dead_bit(c);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      f.w[t][0] = bld16(wres[t], (wbase[t] + uint32_t(c) * 128u) | dead);
      f.w[t][1] = bld16(wres[t], (wbase[t] + uint32_t(c) * 128u + 64u) | dead);
    }
  };
  auto load_a = [&](int c, uint8_t *base) {
    const uint32_t dead = dead_bit(c);
    uint8_t *cb = base + wave * 32 * kMxPitch;
#pragma unroll
    for (int t = 0; t < 8; ++t)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(qres, (__attribute__((address_space(3))) void *)(cb + t * 4 * kMxPitch),
                                               16, (qsrc[t] + uint32_t(c) * 256u) | dead, 0, 0, 0);
  };

  f32x4 acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // this lane's LDS read addresses of token codes in buffer 0, tile 0: the two
  // 16-byte pieces of its row for each MFMA step; tile i adds i * 16 rows (the
  // slot map depends on row % 16 only)
  int oa_lo[2], oa_hi[2];
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    oa_lo[st] = r * kMxPitch + (((8 * st + q) ^ r) << 4);
    oa_hi[st] = r * kMxPitch + (((8 * st + 4 + q) ^ r) << 4);
  }
  // ---- pipeline: PF chunks in flight ahead of the one being multiplied, in
  // PF + 1 LDS buffers and PF + 1 weight register sets (a ring, unrolled so the
  // register set of every step is fixed at compile time)
  constexpr int NBUF = kMxStages;
  constexpr int PF = NBUF - 1;
  constexpr int LOADS = 8 + 2 * NT;  // vector-memory instructions per chunk and wave
  BFrag fr[NBUF];
  // The vmcnt arithmetic needs the loads issued window first, then chunk by
  // chunk: keep the scheduler from interleaving them (it would, and the waits
  // inserted for the registers of chunk 0 would then also stall every pass of
  // the loop below on loads just issued).
  load_scales(0);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int p = 0; p < PF; ++p) {
    load_a(p, L.code.b[p]);
    load_b(p, fr[p]);
    __builtin_amdgcn_sched_barrier(0);
  }
  wait_vmcnt<(PF - 1) * LOADS>();  // the window and chunk 0 have landed
  lds_barrier();

  constexpr int kChunksPerWin = kMxSWin / 8;
  auto body = [&](auto jc, int c) {
    constexpr int J = decltype(jc)::value;
    if (c > 0 && c < nch && c % kChunksPerWin == 0) {
      // next scale window (rows longer than 4096): every wave is past the
      // previous chunk's reads; drain, load, and meet again
      lds_barrier();
      load_scales(c / kChunksPerWin);
      wait_vmcnt<0>();
      lds_barrier();
    }
    load_a(c + PF, L.code.b[(J + PF) % NBUF]);  // the buffer and registers the previous chunk used
    load_b(c + PF, fr[(J + PF) % NBUF]);
    __builtin_amdgcn_sched_barrier(0);
    if (c < nch) {
      const BFrag &f = fr[J];
      const uint8_t *buf = L.code.b[J];
      // this chunk's 8 scale bytes of a row: piece (c mod 16) / 2, half c mod 2
      const int cw = c % kChunksPerWin;
      const int soff = (((cw >> 1) ^ f_r) << 4) + ((cw & 1) << 3);
      u32x2 ws[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) ws[t] = *reinterpret_cast<const u32x2 *>(wsc_t + t * 16 * P + soff);
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        i32x8 bw[NT];
        int bs[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          // FP4 operands use the low four dwords only
          bw[t] = __builtin_bit_cast(i32x8,
                                     __builtin_shufflevector(f.w[t][st], f.w[t][st], 0, 1, 2, 3, -1, -1, -1, -1));
          bs[t] = int(ws[t][st] >> (8 * q));
        }
#pragma unroll
        for (int i = 0; i < MT; ++i) {
          const u32x4 lo = *reinterpret_cast<const u32x4 *>(buf + oa_lo[st] + i * 16 * kMxPitch);
          const u32x4 hi = *reinterpret_cast<const u32x4 *>(buf + oa_hi[st] + i * 16 * kMxPitch);
          const int as = int(*reinterpret_cast<const uint32_t *>(xsc_t + (i >> 1) * (32 * kMxSWin) +
                                                                 (i & 1) * 16 * P + soff + 4 * st) >>
                             (8 * q));
          const i32x8 av = __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
          for (int t = 0; t < NT; ++t) acc[i][t] = mfma_mx(av, bw[t], acc[i][t], as, bs[t]);
        }
      }
    }
    wait_vmcnt<(PF - 1) * LOADS>();  // chunk c + 1 has landed; c + 2 .. c + PF may still fly
    lds_barrier();
  };
  static_assert(8 + 4 + PF * LOADS < 64, "vmcnt is six bits");
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
