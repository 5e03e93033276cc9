// Grouped MFMA GEMM for the prefill regime (segments of hundreds to thousands
// of tokens per expert).
//
//   stage 1: h[p][i] = silu(sum_k X[p][k] Wg[i][k]) * (sum_k X[p][k] Wu[i][k])
//   stage 2: y[p][n] = sum_k h[p][k] Wd[n][k]
//
// Workgroup = 4 waves; tile = 128 segment rows (tokens) x 256 weight rows.
// Stage 1 gives each wave 32 gate rows and the same 32 up rows, so every
// thread holds G and U of the same outputs for the SwiGLU epilogue.  Per wave
// the MFMA register block is 8 token tiles x 4 weight tiles of
// v_mfma_f32_16x16x32_bf16 (A = tokens, B = weights).
//
// The token rows of the tile are gathered through the segment's row list into
// LDS, 128 contraction elements at a time, double buffered, by direct
// buffer-to-LDS loads (lane i of a load writes 16 bytes at base + 16 i); every
// wave reads them from LDS.  Within a row, 16-byte chunk j is stored in slot
// j ^ (row % 16), so the 16 rows an MFMA operand reads hit distinct banks.  Weights are read by each wave straight from global memory
// (each weight row is used by exactly one wave) and, for FP4, decoded in
// registers; the next chunk's weights and tokens are in flight while the
// current chunk is multiplied.
//
// Index maps per 128-element chunk c (bf16 weights and FP4 weights differ):
//   FP4 : lane (n, q) of a weight tile loads 16 bytes = elements 32q..32q+31 of
//         row n (one E8M0 block); MFMA mm (0..3) uses elements 32q + 8mm .. +7.
//   bf16: lane (n, q) loads 16 bytes at elements 32d + 8q .. +7 for MFMA d.
//   Token lane (m, q) supplies the same element indices of row m from LDS.
//
// Work items: (weight tile, token tile) pairs, token tiles counted per expert
// segment (ragged: the last tile of a segment is partial, rows past it load
// zeros and are not written).  Items are ordered expert by expert and block
// ids are remapped so that consecutive items run on the same XCD and share its
// L2 (the order is described at gemm_find_item).
#pragma once

#include <type_traits>
#include <utility>

#include "ft_internal.hpp"

namespace ft {

constexpr int kGemmBM = 128;      // token rows per tile
constexpr int kGemmBN = 256;      // weight rows per tile (stage 1: 128 gate + 128 up)
constexpr int kGemmBK = 128;      // contraction elements per chunk
constexpr int kGemmPitch = 256;   // LDS bytes per token row (one chunk, XOR-swizzled)
constexpr int kGemmThreads = 256;

struct GemmArgs {
  const uint8_t *pool;
  const int32_t *slot_of_expert;  // NULL: slot e
  int32_t n_slots;                // slots in the pool (a larger table value reads as not resident)
  uint64_t expert_bytes;
  const uint8_t *shared_blob;     // NULL: none
  uint64_t off_w0, off_w1, off_s0, off_s1;
  uint64_t off_t0, off_t1;        // NVFP4: byte offsets of the fp32 tensor scales of matrix 0 / 1
  int K, N;                       // contraction length, weight rows of one matrix
  const int32_t *offsets;         // [E+1]
  int E, T, k;
  const int32_t *sorted_rows;     // stage 1: token of permuted row p = sorted_rows[p] / k; NULL: row p
  const uint16_t *X;
  int64_t ldx;
  uint32_t x_bytes;
  void *out;                      // stage 1: bf16 hidden rows; stage 2: fp32 rows
  int64_t ldo;
  float *out_shared;              // stage 2: shared-expert rows by token
  int n_ntiles;                   // weight tiles
  int n_mtiles;                   // token tiles (upper bound over the segments)
  int n_items;                    // work items
};

// Work items are expert-major: the items of expert e (its token tiles x the
// weight tiles) are consecutive, ascending expert, the shared expert last;
// within an expert they are weight-tile major (the token tiles of one weight
// tile are consecutive).  Each XCD takes a contiguous range of the items
// actually present, so a small expert -- a few token tiles -- runs whole on
// one XCD: its token rows are fetched into that XCD's L2 once and shared by
// all its weight tiles, and each weight tile is shared by the expert's token
// tiles.  (Weight-tile major over all experts fetched every token row once per
// weight tile: about 2.5x the bytes past L2 at the 8192-token prefill.)
__host__ __device__ inline int gemm_item_count(int n_mtiles, int n_ntiles) { return n_mtiles * n_ntiles; }

// Block-wide: this block's work item -- weight tile, expert, first row of the
// token tile (BM rows) and its row count.  False if the block has none.
template <int THREADS, int BM = kGemmBM>
__device__ bool gemm_find_item(const GemmArgs &a, int *nt_out, int *e_out, int *row0_out, int *m_out) {
  constexpr int NW = THREADS / 64;
  __shared__ int s_cnt[NW];
  __shared__ int s_e, s_first, s_lo, s_rows;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int NT = a.n_ntiles;
  auto rows_of = [&](int e, int *lo) -> int {
    if (e >= a.E) return 0;
    *lo = a.offsets[e];
    return a.offsets[e + 1] - *lo;
  };
  // pass 1: the number of items present (the first THREADS experts' rows are
  // kept for pass 2)
  int total = 0, lo_c0 = 0, rows_c0 = 0;
  for (int c0 = 0; c0 < a.E; c0 += THREADS) {
    int lo = 0;
    const int rows = rows_of(c0 + tid, &lo);
    if (c0 == 0) {
      lo_c0 = lo;
      rows_c0 = rows;
    }
    const int v = wave_sum_i32((rows + BM - 1) / BM);
    if (lane == 0) s_cnt[wave] = v;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < NW; ++w) total += s_cnt[w];
    __syncthreads();
  }
  const int routed_items = total * NT;
  const int shared_tiles = a.shared_blob != nullptr ? (a.T + BM - 1) / BM : 0;
  const int n_items = routed_items + shared_tiles * NT;
  // this block's item: block ids go round-robin over the 8 XCDs; XCD x takes
  // items [x per, (x + 1) per)
  const int b = int(blockIdx.x);
  const int per = (n_items + 7) / 8;
  const int logical = (b % 8) * per + b / 8;
  if (b / 8 >= per || logical >= n_items) return false;
  if (logical >= routed_items) {
    const int local = logical - routed_items;
    const int ms = local % shared_tiles;
    *nt_out = local / shared_tiles;
    *e_out = a.E;
    *row0_out = ms * BM;  // token index of the first row
    *m_out = min(BM, a.T - ms * BM);
    return true;
  }
  // pass 2: the expert whose items hold it (inclusive scan of items)
  if (tid == 0) s_e = -1;
  int base = 0;
  for (int c0 = 0; c0 < a.E; c0 += THREADS) {
    const int e = c0 + tid;
    int lo = lo_c0;
    const int rows = c0 == 0 ? rows_c0 : rows_of(e, &lo);
    const int items = (rows + BM - 1) / BM * NT;
    const int v = wave_incl_scan_i32(items);
    if (lane == 63) s_cnt[wave] = v;
    __syncthreads();
    int before = base, sum = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      if (w < wave) before += s_cnt[w];
      sum += s_cnt[w];
    }
    const int first = before + v - items;  // exclusive
    if (items > 0 && logical >= first && logical < first + items) {
      s_e = e;
      s_first = first;
      s_lo = lo;
      s_rows = rows;
    }
    base += sum;
    __syncthreads();
    if (s_e >= 0) break;
  }
  const int e = s_e;
  if (e < 0) return false;
  const int lo = s_lo, cnt = s_rows;
  const int tiles = (cnt + BM - 1) / BM;
  const int local = logical - s_first;
  const int mi = local % tiles;
  *nt_out = local / tiles;
  *e_out = e;
  *row0_out = lo + mi * BM;
  *m_out = min(BM, cnt - mi * BM);
  return true;
}

// LDS buffers of a pipelined GEMM: one distinct array per stage, so that the
// compiler can tell a direct load into one buffer from reads of another.
template <int N>
struct LdsRing {
  uint8_t *b[N];
};

// Calls f(std::integral_constant<int, J>) for J = 0 .. N-1.
template <typename F, int... J>
__device__ __forceinline__ void unroll_ring(F &&f, std::integer_sequence<int, J...>) {
  (f(std::integral_constant<int, J>{}), ...);
}

// The multiply of one work item, with MT 16-row token sub-tiles per wave: a
// segment's last tile often holds a few dozen rows, and running it with
// MT = 4 or 2 skips the MFMAs of the sub-tiles that would only hold padding
// (the loads of those rows are out of range anyway: no traffic).
template <int WF, bool GLU, int NBUF, int MT>
__device__ __forceinline__ void gemm_body(const GemmArgs &a, LdsRing<NBUF> L, int nt_idx, int row0, int m,
                                          bool shared, const uint8_t *blob);

// This workgroup's work item: the weight tile, the token tile's first row
// and row count, the expert's blob.  False if there is none, or if the expert
// is not resident (its outputs of this tile were then marked NaN).
template <bool GLU, int BM = kGemmBM>
__device__ __forceinline__ bool gemm_setup(const GemmArgs &a, int &nt_idx, int &row0, int &m, bool &shared,
                                           const uint8_t *&blob) {
  const int tid = threadIdx.x;
  int e;
  if (!gemm_find_item<kGemmThreads, BM>(a, &nt_idx, &e, &row0, &m)) return false;
  shared = e == a.E;
  if (shared) {
    blob = a.shared_blob;
  } else {
    const int slot = table_slot(a.slot_of_expert, e, a.n_slots);
    if (slot == FT_SLOT_SKIP) return false;  // another call computes these rows
    if (slot < 0) {
      // not resident: mark this tile's outputs NaN
      const int cols = GLU ? kGemmBN / 2 : kGemmBN;
      const int c0 = nt_idx * cols;
      for (int u = tid; u < m * cols; u += kGemmThreads) {
        const int rr = u / cols, cc = c0 + u % cols;
        if (cc >= a.N) continue;
        if (GLU) reinterpret_cast<uint16_t *>(a.out)[int64_t(row0 + rr) * a.ldo + cc] = 0x7fc0;
        else reinterpret_cast<float *>(a.out)[int64_t(row0 + rr) * a.ldo + cc] = __builtin_nanf("");
      }
      return false;
    }
    blob = a.pool + uint64_t(slot) * a.expert_bytes;
  }
  return true;
}

template <int WF, bool GLU, int NBUF>
__device__ __forceinline__ void gemm_tile(const GemmArgs &a, LdsRing<NBUF> L) {
  int nt_idx, row0, m;
  bool shared;
  const uint8_t *blob;
  if (!gemm_setup<GLU>(a, nt_idx, row0, m, shared, blob)) return;
  if (m > 64)
    gemm_body<WF, GLU, NBUF, 8>(a, L, nt_idx, row0, m, shared, blob);
  else if (m > 32)
    gemm_body<WF, GLU, NBUF, 4>(a, L, nt_idx, row0, m, shared, blob);
  else
    gemm_body<WF, GLU, NBUF, 2>(a, L, nt_idx, row0, m, shared, blob);
}

template <int WF, bool GLU, int NBUF, int MT>
__device__ __forceinline__ void gemm_body(const GemmArgs &a, LdsRing<NBUF> L, int nt_idx, int row0, int m,
                                          bool shared, const uint8_t *blob) {
  constexpr int NT = 4;   // weight tiles (16 rows) per wave
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = lane & 15, q = lane >> 4;
  // ---- token rows: wave w fills rows 32w..32w+31 of a chunk buffer with 8
  // direct loads of 4 rows each; lane i covers row 4t + i/16, slot i%16
  const rsrc_t xres = make_rsrc(a.X, a.x_bytes);
  uint32_t xsrc[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int rr = wave * 32 + t * 4 + (lane >> 4);
    int src = -1;
    if (rr < m) {
      if (a.sorted_rows == nullptr) src = (shared ? a.T * a.k : 0) + row0 + rr;  // hidden row
      else if (shared) src = row0 + rr;                                        // token
      else src = a.sorted_rows[row0 + rr] / a.k;                               // gathered token
    }
    const int j = (lane & 15) ^ (rr & 15);  // global chunk stored in this lane's slot
    xsrc[t] = src >= 0 ? uint32_t(src) * uint32_t(a.ldx) * 2u + uint32_t(j) * 16u : kOOB;
  }

  // ---- weights of this wave
  const uint32_t wpitch = (WF == WF_BF16) ? uint32_t(a.K) * 2 : uint32_t(a.K) / 2;
  const uint32_t spitch = uint32_t(a.K) / (WF == WF_NV4 ? 16 : 32);
  const uint32_t wbytes = uint32_t(a.N) * wpitch, sbytes = uint32_t(a.N) * spitch;
  rsrc_t wres[NT], sres[NT];
  uint32_t wrow[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    int row;
    const uint8_t *wb, *sb;
    if (GLU) {
      // tiles 0,1: gate rows; tiles 2,3: the same up rows
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
    wrow[t] = uint32_t(row);  // rows past N fall outside the buffer
  }
  constexpr int DLW = WF == WF_BF16 ? 4 : 1;  // 16-byte weight loads per tile per chunk
  struct BFrag {
    u32x4 w[NT][DLW];
  };
  // Block scales (4 E8M0 or 8 E4M3 bytes per row and chunk) come four chunks
  // at a time: lane group g loads the scales of chunk c0 + g, so the four
  // lanes of a row fetch 16 or 32 contiguous bytes in one request (one load
  // per chunk and row cost a request for 4 or 8 bytes), and a chunk's step
  // takes its row's scales from lane group c mod 4.
  using SWord = std::conditional_t<WF == WF_NV4, u32x2, uint32_t>;
  constexpr int SB = WF == WF_NV4 ? 8 : 4;  // scale bytes per row and chunk
  const int nch = a.K / kGemmBK;
  // A chunk past the end is still issued, with out-of-range offsets (no memory
  // traffic, zeros): every step then has the same loads in flight, and the
  // vmcnt arithmetic below holds on every path.
  auto load_b = [&](int c, BFrag &f) {
    const bool live = c < nch;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if constexpr (WF == WF_BF16) {
#pragma unroll
        for (int d = 0; d < 4; ++d)
          f.w[t][d] = bld16(wres[t], live ? wrow[t] * wpitch + uint32_t(c) * 256u + d * 64 + q * 16 : kOOB);
      } else {
        f.w[t][0] = bld16(wres[t], live ? wrow[t] * wpitch + uint32_t(c) * 64u + q * 16 : kOOB);
      }
    }
  };
  auto load_a = [&](int c, uint8_t *buf) {
    const bool live = c < nch;
    uint8_t *base = buf + wave * 32 * kGemmPitch;
#pragma unroll
    for (int t = 0; t < 8; ++t)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          xres, (__attribute__((address_space(3))) void *)(base + t * 4 * kGemmPitch), 16,
          (xsrc[t] == kOOB || !live) ? kOOB : xsrc[t] + uint32_t(c) * 256u, 0, 0, 0);
  };

  auto load_s = [&](int c0, SWord *g) {
    const bool live = c0 + q < nch;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const uint32_t off = live ? wrow[t] * spitch + uint32_t(c0 + q) * SB : kOOB;
      if constexpr (WF == WF_NV4)
        g[t] = bld8(sres[t], off);
      else
        g[t] = bld4(sres[t], off);
    }
  };

  f32x4 acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- pipeline: P = NBUF - 1 chunks in flight ahead of the one being
  // multiplied, in NBUF LDS buffers and NBUF weight register sets (a ring,
  // unrolled so the register set of every step is fixed at compile time).
  // Step c issues chunk c + P into the buffer and registers step c - 1 used
  // (every wave passed the barrier that ended step c - 1), multiplies chunk c,
  // then waits until chunk c + 1 has landed and meets the other waves.
  constexpr int P = NBUF - 1;
  static_assert(P == 1, "every step waits for all of its loads");
  constexpr int UNR = WF == WF_BF16 ? NBUF : 4;  // steps per loop pass: a multiple of NBUF and of 4
  static_assert(UNR % NBUF == 0, "ring");
  BFrag fr[NBUF];
  SWord sg[NT], sgn[NT];  // scales of chunks c0 .. c0+3 (lane group g: c0 + g), and of the next four
  if constexpr (WF != WF_BF16) {
    load_s(0, sg);
#pragma unroll
    for (int t = 0; t < NT; ++t) sgn[t] = sg[t];
  }
  load_a(0, L.b[0]);
  load_b(0, fr[0]);
  wait_vmcnt<0>();  // chunk 0 has landed
  lds_barrier();
  auto step = [&](auto jc, int c) {
    constexpr int JU = decltype(jc)::value;
    constexpr int J = JU % NBUF;
    if (c + P < nch) {
      load_a(c + P, L.b[(J + P) % NBUF]);
      load_b(c + P, fr[(J + P) % NBUF]);
      if constexpr (WF != WF_BF16 && JU % 4 == 3) load_s(c + 1, sgn);
    }
    if (c < nch) {
      const BFrag &f = fr[J];
      const uint8_t *abuf = L.b[J];
      // this chunk's scales of the lane's row, from lane group c mod 4
      SWord cs[NT];
      if constexpr (WF != WF_BF16) {
        const int src = (r + 16 * (JU % 4)) * 4;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          if constexpr (WF == WF_NV4) {
            cs[t][0] = uint32_t(__builtin_amdgcn_ds_bpermute(src, int(sg[t][0])));
            cs[t][1] = uint32_t(__builtin_amdgcn_ds_bpermute(src, int(sg[t][1])));
          } else {
            cs[t] = uint32_t(__builtin_amdgcn_ds_bpermute(src, int(sg[t])));
          }
        }
      }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        bf16x8 bw[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          if constexpr (WF == WF_BF16) {
            bw[t] = as_bf16x8(f.w[t][ks]);
          } else if constexpr (WF == WF_FP4) {
            bw[t] = fp4x8_to_bf16x8(f.w[t][0][ks], e8m0_to_f32((cs[t] >> (8 * q)) & 0xffu));
          } else {  // NVFP4: elements 32q + 8ks .. +7 lie in 16-element block 2q + ks/2
            const uint32_t sw = (q >> 1) ? cs[t][1] : cs[t][0];
            bw[t] = nvfp4x8_to_bf16x8(f.w[t][0][ks], e4m3_to_f32(sw >> (8 * ((2 * q + (ks >> 1)) & 3))));
          }
        }
        const int j = WF == WF_BF16 ? 4 * ks + q : 4 * q + ks;  // 16-byte chunk of the row
#pragma unroll
        for (int i = 0; i < MT; ++i) {
          const u32x4 af = *reinterpret_cast<const u32x4 *>(abuf + (i * 16 + r) * kGemmPitch + ((j ^ r) << 4));
#pragma unroll
          for (int t = 0; t < NT; ++t) acc[i][t] = mfma16(as_bf16x8(af), bw[t], acc[i][t]);
        }
      }
    }
    wait_vmcnt<0>();  // chunk c + 1 (and the next scales) have landed
    lds_barrier();
    if constexpr (WF != WF_BF16 && JU % 4 == 3) {
#pragma unroll
      for (int t = 0; t < NT; ++t) sg[t] = sgn[t];
    }
  };
  for (int c = 0; c < nch; c += UNR)
    unroll_ring([&](auto jc) { step(jc, c + decltype(jc)::value); }, std::make_integer_sequence<int, UNR>{});
  wait_vmcnt<0>();

  // ---- epilogue: lane holds D[token 4q+v][weight row r] of each tile
  float ts0 = 1.f, ts1 = 1.f;  // NVFP4: the per-tensor scales, on the fp32 sums
  if constexpr (WF == WF_NV4) {
    ts0 = *reinterpret_cast<const float *>(blob + a.off_t0);
    ts1 = *reinterpret_cast<const float *>(blob + a.off_t1);
  }
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
          if (col < a.N) hp[col] = f32_to_bf16_rne(silu(acc[i][t][v] * ts0) * (acc[i][t + 2][v] * ts1));
        }
      } else {
        float *yp = shared ? a.out_shared + int64_t(row0 + rr) * a.ldo
                           : reinterpret_cast<float *>(a.out) + int64_t(row0 + rr) * a.ldo;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const int col = nt_idx * kGemmBN + wave * 64 + t * 16 + r;
          if (col < a.N) yp[col] = acc[i][t][v] * ts0;
        }
      }
    }
  }
}

}  // namespace ft
