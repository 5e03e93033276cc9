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
// Workgroup = 4 waves; tile = 128 segment rows (tokens) x 256 weight rows:
// stage 1 gives each wave 32 gate rows and the same 32 up rows, stage 2 64
// weight rows; per wave 8 token tiles x 4 weight tiles of 16x16 accumulators.
// Two workgroups share a CU (two waves per SIMD): with one wave per SIMD the
// MFMA pipe idled through every wait of that wave -- measured, the kernel then
// ran at a quarter of the MFMA rate whether or not its loads hit in cache --
// and that is what sizes everything else: 128 accumulators, two weight
// register sets and 56 KiB of LDS per workgroup.  A chunk is 128 contraction
// elements (one MFMA step); the token codes of a chunk (128 rows x 128 bytes)
// are gathered into LDS by direct buffer-to-LDS loads, the weights go from
// global memory straight to registers (each weight row is used by one wave).
// One chunk is in flight while one is multiplied (two LDS buffers, two weight
// register sets).
//
// Block scales are not fetched per chunk: a chunk needs 4 bytes of each row,
// and fetching them one chunk at a time costs the L1 a request per row for 4
// bytes.  Instead each row's scales of a window of 16 chunks (64 bytes) are
// copied into LDS once -- for the 256 weight rows and the 128 token rows of the
// tile -- and every chunk reads its 4 bytes per row from there.  A window
// covers K <= 2048 whole; longer rows load the next window at its first chunk,
// with the pipeline drained around that load.
//
// Index maps per chunk c, lane (r, g):
//   token operand: row r of the 16-row tile, row bytes 16 g .. +15 and
//                  64 + 16 g .. +15 of the chunk; 16-byte piece j of a row is
//                  stored in slot j ^ ((row / 2) % 8), so the 16 rows an MFMA
//                  operand reads hit distinct banks.
//   weight operand: row r of the tile, code bytes 64 c + 16 g .. +15
//                   (elements 128 c + 32 g .. +31).
//   scales (either operand): byte 4 c + g of the row's scales.  In the LDS
//                  copy a row takes P bytes (64, or the row's scale bytes
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

constexpr int kMxBM = 128;                        // token rows per tile
constexpr int kMxRW = kMxBM / 4;                  // token rows each wave loads
constexpr int kMxBK = 128;                        // contraction elements per chunk (one MFMA step)
constexpr int kMxPitch = 128;                     // LDS bytes per token row (codes of one chunk)
constexpr int kMxCodeBytes = kMxBM * kMxPitch;    // 16 KiB per buffer
constexpr int kMxStages = 2;                      // LDS code buffers (chunks in flight + 1)
constexpr int kMxSWin = 64;                       // scale bytes per row in one window (16 chunks)
constexpr int kMxWScaleBytes = kGemmBN * kMxSWin; // weight scales of a window: 16 KiB
constexpr int kMxXScaleBytes = kMxBM * kMxSWin;   // token scales of a window: 8 KiB

struct MxGemmArgs {
  GemmArgs g;          // shapes, weights, segments and outputs (g.X, g.ldx, g.x_bytes unused)
  const uint8_t *Xq;   // E4M3 codes [rows, K]
  const uint8_t *Xs;   // E8M0 scales [rows, K / 32]
  uint32_t xq_bytes, xs_bytes;
};

// LDS of one workgroup: the code ring and the two scale windows.
struct MxLds {
  LdsRing<kMxStages> code;
  uint8_t *wsc;  // [4 waves][64 rows][P], 4 KiB per wave
  uint8_t *xsc;  // [4 waves][32 rows][P], 2 KiB per wave
};

template <bool GLU, int MT>
__device__ __forceinline__ void gemm_mx_body(const MxGemmArgs &ma, const MxLds &L, int nt_idx, int row0, int m,
                                             bool shared, const uint8_t *blob);

template <bool GLU>
__device__ __forceinline__ void gemm_mx_tile(const MxGemmArgs &ma, const MxLds &L) {
  int nt_idx, row0, m;
  bool shared;
  const uint8_t *blob;
  if (!gemm_setup<GLU, kMxBM>(ma.g, nt_idx, row0, m, shared, blob)) return;
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

  // ---- token codes: wave w fills rows 64w..64w+63 with 8 direct loads of 8
  // rows each (lane i: row 8t + i/8, slot i%8)
  const uint32_t kq = uint32_t(a.K);
  const rsrc_t qres = make_rsrc(ma.Xq, ma.xq_bytes);
  constexpr int TL = kMxRW / 8;  // token-code loads per wave and chunk
  uint32_t qsrc[TL];
#pragma unroll
  for (int t = 0; t < TL; ++t) {
    const int rr = wave * kMxRW + t * 8 + (lane >> 3);
    const int src = src_row(rr);
    const int j = (lane & 7) ^ ((rr >> 1) & 7);
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
  const int ppr = P / 16;  // pieces per row: 1, 2 or 4
  auto fsw = [&](int R) { return (R / (16 / ppr)) & (ppr - 1); };
  const rsrc_t bres = make_rsrc(blob, uint32_t(a.expert_bytes));
  const rsrc_t xsres = make_rsrc(ma.Xs, ma.xs_bytes);
  uint8_t *const wsc_w = L.wsc + wave * (64 * kMxSWin);
  uint8_t *const xsc_w = L.xsc + wave * (kMxRW * kMxSWin);
  // window win of this wave's 64 weight rows and 64 token rows (ppr loads of
  // 1 KiB each); lane i of load n covers row (64 n + i) / ppr, slot
  // (64 n + i) % ppr
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
    const int nx = (kMxRW * ppr + 63) / 64;
    for (int n = 0; n < nx; ++n) {
      const int u = n * 64 + lane, rho = u / ppr, j = u % ppr;
      const int piece = j ^ fsw(rho & 15);
      const int src = rho < kMxRW ? src_row(wave * kMxRW + rho) : -1;
      const uint32_t off = src >= 0 ? uint32_t(src) * uint32_t(srow) + woff + uint32_t(piece) * 16u : kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xsres, (__attribute__((address_space(3))) void *)(xsc_w + n * 1024),
                                               16, off, 0, 0, 0);
    }
  };
  // this lane's scale rows in LDS: weight tile t adds 16 t P; token tile i
  // adds (i / 4) 4096 (the wave area of its rows) + (i % 4) 16 P
  const int f_r = fsw(r);
  const uint8_t *const wsc_t = L.wsc + wave * (64 * kMxSWin) + r * P;
  const uint8_t *const xsc_t = L.xsc + r * P;

  struct BFrag {
    u32x4 w[NT];
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
    for (int t = 0; t < NT; ++t) f.w[t] = bld16(wres[t], (wbase[t] + uint32_t(c) * 64u) | dead);
  };
  auto load_a = [&](int c, uint8_t *base) {
    const uint32_t dead = dead_bit(c);
    uint8_t *cb = base + wave * kMxRW * kMxPitch;
#pragma unroll
    for (int t = 0; t < TL; ++t)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(qres, (__attribute__((address_space(3))) void *)(cb + t * 8 * kMxPitch),
                                               16, (qsrc[t] + uint32_t(c) * 128u) | dead, 0, 0, 0);
  };

  f32x4 acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // this lane's LDS read addresses of token codes in buffer 0, tile 0: the two
  // 16-byte pieces of its row; tile i adds i * 16 rows (the slot map depends on
  // row % 16 only)
  const int sw = (r >> 1) & 7;
  const int oa_lo = r * kMxPitch + ((q ^ sw) << 4);
  const int oa_hi = r * kMxPitch + (((4 + q) ^ sw) << 4);
  // ---- pipeline: PF chunks in flight ahead of the one being multiplied, in
  // PF + 1 LDS buffers and PF + 1 weight register sets (a ring, unrolled so the
  // register set of every step is fixed at compile time)
  constexpr int NBUF = kMxStages;
  constexpr int PF = NBUF - 1;
  constexpr int LOADS = TL + NT;  // vector-memory instructions per chunk and wave
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

  constexpr int kChunksPerWin = kMxSWin / 4;
  auto body = [&](auto jc, int c) {
    constexpr int J = decltype(jc)::value;
    if (c > 0 && c < nch && c % kChunksPerWin == 0) {
      // next scale window (rows longer than 2048): every wave is past the
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
      // this chunk's scale byte of a row for lane group g: piece (c mod 16) / 4,
      // byte 4 (c mod 4) + g; each lane reads its own byte, so it needs no shift
      const int cw = c % kChunksPerWin;
      const int soff = (((cw >> 2) ^ f_r) << 4) + ((cw & 3) << 2) + q;
      i32x8 bw[NT];
      int bs[NT], as[MT];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        // FP4 operands use the low four dwords only
        bw[t] = __builtin_bit_cast(i32x8, __builtin_shufflevector(f.w[t], f.w[t], 0, 1, 2, 3, -1, -1, -1, -1));
        bs[t] = wsc_t[t * 16 * P + soff];
      }
#pragma unroll
      for (int i = 0; i < MT; ++i)
        as[i] = xsc_t[(i / (kMxRW / 16)) * (kMxRW * kMxSWin) + (i % (kMxRW / 16)) * 16 * P + soff];
      // token operands read from LDS one sub-tile ahead of their MFMAs
      constexpr int D = 1;
      u32x4 alo[MT], ahi[MT];
      auto read_a = [&](int i) {
        alo[i] = *reinterpret_cast<const u32x4 *>(buf + oa_lo + i * 16 * kMxPitch);
        ahi[i] = *reinterpret_cast<const u32x4 *>(buf + oa_hi + i * 16 * kMxPitch);
      };
#pragma unroll
      for (int i = 0; i < D; ++i) read_a(i);
      __builtin_amdgcn_sched_group_barrier(0x100, NT + MT + 2 * D, 0);  // scale bytes, sub-tiles 0 .. D-1
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        if (i + D < MT) read_a(i + D);
        const i32x8 av = __builtin_bit_cast(i32x8, __builtin_shufflevector(alo[i], ahi[i], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[i][t] = mfma_mx(av, bw[t], acc[i][t], as[i], bs[t]);
        if (i + D < MT) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // operand of sub-tile i + D
        __builtin_amdgcn_sched_group_barrier(0x008, NT, 0);                 // MFMAs of sub-tile i
      }
    }
    wait_vmcnt<(PF - 1) * LOADS>();  // chunk c + 1 has landed; c + 2 .. c + PF may still fly
    lds_barrier();
  };
  static_assert(2 * 4 + PF * LOADS < 64, "vmcnt is six bits");
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
