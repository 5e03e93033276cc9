// Persistent weight-streaming kernel body for the decode regime (segments of at
// most a few dozen tokens).
//
// One workgroup of WAVES waves stays resident and walks a strided list of
// units.  A unit is (active expert, 16-row weight tile, group of <= 16 tokens
// of that expert's segment).  The waves split the contraction axis (KPW
// k-blocks each, interleaved) and meet in LDS to sum their partial 16x16
// tiles.  While a unit is multiplied, the weights and token indices of the
// workgroup's next unit are already in flight, so HBM latency is overlapped
// with MFMA work and the epilogue instead of being paid per workgroup.
//
// The active-expert table (experts with a non-empty segment, ascending, then
// the shared expert) is built once per workgroup in LDS from the segment
// offsets.  Loads, index maps and masking are those of stream_gemm.hpp (raw
// buffer loads; out-of-range offsets return zero without memory traffic).
#pragma once

#include "permute_util.hpp"
#include "stream_gemm.hpp"
#include "topk_util.hpp"

namespace ft {

constexpr int kPersistMaxE = 1024;     // experts the LDS table holds (larger E uses the plain kernel)
constexpr int kPersistMaxRows = 4096;  // routed rows whose token indices fit the LDS copy

// Small decode batches routed inside the FFN (the layer call's fused path).
constexpr int kRouteMaxT = 4;          // tokens (one wave each in the routing prologue)
constexpr int kRouteMaxE = 256;        // experts (four logits per lane)
constexpr int kRouteMaxRows = 64;      // routed rows (one wave sorts them)
constexpr int kFusedMaxK = 16;       // picks per token of the fused combine
constexpr int kStageCols = 256;      // down stage: output columns staged in LDS before they are written

struct PersistArgs {
  const uint8_t *pool;
  const int32_t *slot_of_expert;  // NULL: slot e
  int32_t n_slots;                // slots in the pool (a larger table value reads as not resident)
  uint64_t expert_bytes;
  const uint8_t *shared_blob;     // NULL: none
  uint64_t off_w0, off_w1, off_s0, off_s1;
  uint64_t off_t0, off_t1;        // NVFP4: byte offsets of the fp32 tensor scales of matrix 0 / 1
  int K, N;                       // contraction length, weight rows
  const int32_t *offsets;         // [E+1]
  int E, T, k;
  const int32_t *sorted_rows;     // gather: token of permuted row p = sorted_rows[p] / k (NULL: row p itself)
  const uint16_t *X;              // bf16 activations (x or hidden rows)
  int64_t ldx;
  uint32_t x_bytes;
  void *out;                      // GLU: bf16 hidden rows; else fp32 rows
  int64_t ldo;
  float *out_shared;              // non-GLU: rows of the shared expert go here (by token)
  int n_tiles;                    // ceil(N / tile rows)
  int tile_rows;                  // fused layer call: weight rows per tile, 16 or 8 (other kernels: 16)
  // routing prologue (gate/up of the fused layer call): every workgroup takes top-k, gating and the
  // permutation of the T tokens from the logits; workgroup 0 also writes them out
  const float *logits;            // [T, E]
  int gating, renorm;
  int32_t *ids_out, *off_out, *rows_out, *pos_out;
  float *w_out;
  // combine folded into the down stage (fused layer call): out[t] = sum_j w[t, j] y_j (+ shared)
  const int32_t *ids;             // [T, k]
  const float *topk_w;            // [T, k]
  const int32_t *row_pos;         // [T*k]: hidden row of pick (t, j)
  void *comb_out;                 // [T, ldo] bf16 or fp32
  int comb_bf16;
};

// Top-k, gating and the permutation of the batch's T <= kRouteMaxT tokens by
// one workgroup (wave t takes token t; wave 0 then sorts the T*k <= 64 rows),
// into LDS; workgroup 0 also writes ids, weights, offsets, sorted rows and
// row positions out for the down stage, the combine and the caller.
template <int THREADS>
__device__ __forceinline__ void route_prologue(const PersistArgs &a, int32_t *s_ids, int32_t *s_off,
                                               int32_t *s_rows, int32_t *s_pos, int32_t *s_sorted) {
  const int tid = threadIdx.x, wave = tid >> 6;
  const bool pub = blockIdx.x == 0;
  if (wave < a.T)
    topk_token<kRouteMaxE / 64>(a.logits, wave, a.E, a.k, a.gating, a.renorm, pub ? a.ids_out : nullptr,
                                pub ? a.w_out : nullptr, s_ids);
  __syncthreads();
  const int R = a.T * a.k;
  if (wave == 0) permute_wave64(s_ids, R, a.E, s_sorted, s_off, s_rows, s_pos);
  __syncthreads();
  if (pub) {
    for (int e = tid; e <= a.E; e += THREADS) a.off_out[e] = s_off[e];
    for (int p = tid; p < R; p += THREADS) {
      a.rows_out[p] = s_rows[p];
      a.pos_out[p] = s_pos[p];
    }
  }
}

// A value every lane of the wave holds (an LDS table entry read at a uniform
// index) moved to a scalar register, so descriptors built from it stay scalar.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// NB: units in flight per wave (a ring of NB register sets; the loads of unit
// i+NB-1 are issued before unit i is multiplied).  NB = 1 issues a unit's
// activations at its own start, still ahead of the next unit's weights,
// which saves registers.
template <int WF, bool GLU, int WAVES, int KPW, int NB>
__device__ __forceinline__ void stream_persist(const PersistArgs &a, float *s_red) {
  constexpr int THREADS = WAVES * 64;
  constexpr int NW = WAVES;
  constexpr int MATS = GLU ? 2 : 1;
  constexpr int KB = stream_kblock<WF>();
  constexpr int DL = WFrag<WF, MATS>::DL;
  constexpr int DX = WF == WF_BF16 ? 4 : 8;
  __shared__ int s_e[kPersistMaxE + 1];    // expert id (E = shared expert)
  __shared__ int s_pos[kPersistMaxE + 1];  // first permuted row of its segment
  __shared__ int s_m[kPersistMaxE + 1];    // rows of its segment
  __shared__ int s_slot[kPersistMaxE + 1];
  __shared__ int s_cnt[NW];
  __shared__ int s_tok[kPersistMaxRows];  // token of every routed row (gather mode)
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  if (a.sorted_rows != nullptr)
    for (int p = tid; p < a.T * a.k; p += THREADS) s_tok[p] = a.sorted_rows[p] / a.k;
  const int r = lane & 15, q = lane >> 4;

  // ---- active-expert table
  int base = 0;
  for (int c0 = 0; c0 < a.E; c0 += THREADS) {
    const int e = c0 + tid;
    int lo = 0, cnt = 0;
    if (e < a.E) {
      lo = a.offsets[e];
      cnt = a.offsets[e + 1] - lo;
      if (cnt > 0 && a.slot_of_expert != nullptr && a.slot_of_expert[e] == FT_SLOT_SKIP) cnt = 0;  // another call's
    }
    const bool f = cnt > 0;
    const uint64_t mask = __ballot(f);
    if (lane == 0) s_cnt[wave] = __popcll(mask);
    __syncthreads();
    int before = base, total = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      if (w < wave) before += s_cnt[w];
      total += s_cnt[w];
    }
    if (f) {
      const int i = before + __popcll(mask & ((uint64_t(1) << lane) - 1));
      s_e[i] = e;
      s_pos[i] = lo;
      s_m[i] = cnt;
      s_slot[i] = table_slot(a.slot_of_expert, e, a.n_slots);
    }
    base += total;
    __syncthreads();
  }
  int n_act = base;
  if (a.shared_blob != nullptr) {
    if (tid == 0) {
      s_e[n_act] = a.E;
      s_pos[n_act] = a.T * a.k;
      s_m[n_act] = a.T;
      s_slot[n_act] = 0;
    }
    ++n_act;
    __syncthreads();
  }
  const int n_items = n_act * a.n_tiles;

  // ---- per-unit state
  struct Unit {
    int item, g0;  // item = active index * n_tiles + tile; g0 = first token of the group
  };
  auto valid = [&](const Unit &u) { return u.item < n_items; };
  auto first_unit = [&]() { return Unit{int(blockIdx.x), 0}; };
  auto next_unit = [&](const Unit &u) {
    const int ai = u.item / a.n_tiles;
    if (u.g0 + 16 < uniform(s_m[ai])) return Unit{u.item, u.g0 + 16};
    return Unit{u.item + int(gridDim.x), 0};
  };

  const uint32_t wpitch = (WF == WF_BF16) ? uint32_t(a.K) * 2 : uint32_t(a.K) / 2;
  const uint32_t spitch = uint32_t(a.K) / 32;
  const uint32_t wbytes = uint32_t(a.N) * wpitch, sbytes = uint32_t(a.N) * spitch;
  const rsrc_t xres = make_rsrc(a.X, a.x_bytes);

  // Register set of one unit: its weights and activations.
  struct UnitRegs {
    WFrag<WF, MATS> f[KPW];
    u32x4 xb[KPW][DX];
  };

  auto issue_w = [&](const Unit &u, UnitRegs &R) {
    if (!valid(u)) return;
    const int ai = u.item / a.n_tiles, tile = u.item % a.n_tiles;
    const int e = uniform(s_e[ai]), slot = uniform(s_slot[ai]);
    const uint8_t *blob = e == a.E ? a.shared_blob : a.pool + uint64_t(max(slot, 0)) * a.expert_bytes;
    rsrc_t wres[MATS], sres[MATS];
    wres[0] = make_rsrc(blob + a.off_w0, wbytes);
    sres[0] = make_rsrc(blob + a.off_s0, sbytes);
    if constexpr (GLU) {
      wres[MATS - 1] = make_rsrc(blob + a.off_w1, wbytes);
      sres[MATS - 1] = make_rsrc(blob + a.off_s1, sbytes);
    }
    constexpr int NH = wl_halves<WF>();
    uint32_t wo[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) wo[h] = uint32_t(tile * 16 + wl_row<WF>(lane, h)) * wpitch + wl_byte<WF>(lane, h);
    const uint32_t so = uint32_t(tile * 16 + r) * spitch;
#pragma unroll
    for (int c = 0; c < KPW; ++c) {
      const int kb = wave + c * WAVES;
#pragma unroll
      for (int mt = 0; mt < MATS; ++mt) {
#pragma unroll
        for (int d = 0; d < DL; ++d)
          R.f[c].w[mt][d] = wl_load<WF>(wres[mt], wo[d % NH] + uint32_t(kb) * wl_kbytes<WF>() + wl_dcol<WF>(d));
        if constexpr (WF == WF_FP4) R.f[c].s[mt] = bld8(sres[mt], so + uint32_t(kb) * 8);
      }
    }
  };
  // Activations of unit u (this lane's token row from the LDS copy).
  auto issue_x = [&](const Unit &u, u32x4 (&xb)[KPW][DX]) {
    if (!valid(u)) return;
    const int ai = u.item / a.n_tiles;
    const int e = uniform(s_e[ai]), pos = uniform(s_pos[ai]), m = uniform(s_m[ai]);
    const int j = u.g0 + r;
    int row = -1;
    if (j < m) {
      if (a.sorted_rows == nullptr) row = pos + j;      // hidden row p
      else row = e == a.E ? j : s_tok[pos + j];         // token of the shared / routed expert
    }
    const uint32_t xo = row >= 0 ? uint32_t(row) * uint32_t(a.ldx) * 2u : kOOB;
#pragma unroll
    for (int c = 0; c < KPW; ++c) {
      const int kb = wave + c * WAVES;
#pragma unroll
      for (int dx = 0; dx < DX; ++dx) {
        xb[c][dx] = bld16(xres, xo + uint32_t(kb * KB + wl_xk<WF>(dx, q)) * 2u);
      }
    }
  };

  // Multiply unit u (weights in cur, activations in xcur), sum the wave
  // partials in LDS and write its 16x16 output tile.
  auto finish = [&](const Unit &u, const UnitRegs &cur, const u32x4 (&xcur)[KPW][DX]) {
    const int ai = u.item / a.n_tiles, tile = u.item % a.n_tiles;
    const int e = uniform(s_e[ai]), slot = uniform(s_slot[ai]), pos = uniform(s_pos[ai]), m = uniform(s_m[ai]);
    const bool shared = e == a.E;
    const bool missing = !shared && slot < 0;
    f32x4 acc[MATS];
#pragma unroll
    for (int mt = 0; mt < MATS; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < KPW; ++c) {
      WFrag<WF, MATS> f = cur.f[c];
      wfrag_fix(f);
      if constexpr (WF == WF_BF16) {
#pragma unroll
        for (int d = 0; d < 4; ++d)
#pragma unroll
          for (int mt = 0; mt < MATS; ++mt) acc[mt] = mfma16(as_bf16x8(f.w[mt][d]), as_bf16x8(xcur[c][d]), acc[mt]);
      } else {
#pragma unroll
        for (int d = 0; d < 2; ++d) {
          float sc[MATS];
#pragma unroll
          for (int mt = 0; mt < MATS; ++mt) sc[mt] = e8m0_to_f32(wl_mx_scale<WF>(f.s[mt], d, q));
#pragma unroll
          for (int mm = 0; mm < 4; ++mm)
#pragma unroll
            for (int mt = 0; mt < MATS; ++mt)
              acc[mt] = mfma16(fp4x8_to_bf16x8(f.w[mt][d][mm], sc[mt]), as_bf16x8(xcur[c][4 * d + mm]), acc[mt]);
        }
      }
    }
    // Sum the waves' partial tiles: thread t < 256 owns element (lane t/4, value t%4).
#pragma unroll
    for (int mt = 0; mt < MATS; ++mt)
      *reinterpret_cast<f32x4 *>(&s_red[((wave * MATS + mt) * 64 + lane) * 4]) = acc[mt];
    __syncthreads();
    if (tid < 256) {
      const int ln = tid >> 2, v = tid & 3;
      const int jj = u.g0 + (ln & 15);
      const int n = tile * 16 + 4 * (ln >> 4) + v;
      float g = 0.f, uu = 0.f;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) {
        g += s_red[((w * MATS + 0) * 64 + ln) * 4 + v];
        if constexpr (GLU) uu += s_red[((w * MATS + 1) * 64 + ln) * 4 + v];
      }
      if (jj < m && n < a.N) {
        const int p = pos + jj;  // permuted row; hidden rows of the shared expert follow the routed ones
        if constexpr (GLU) {
          reinterpret_cast<uint16_t *>(a.out)[int64_t(p) * a.ldo + n] =
              missing ? uint16_t(0x7fc0) : f32_to_bf16_rne(silu(g) * uu);
        } else {
          float *yp = shared ? a.out_shared + int64_t(jj) * a.ldo : reinterpret_cast<float *>(a.out) + int64_t(p) * a.ldo;
          yp[n] = missing ? __builtin_nanf("") : g;
        }
      }
    }
    __syncthreads();
  };

  Unit u = first_unit();
  if constexpr (NB == 1) {
    // This unit's activations, then the next unit's weights, then the multiply
    // (which waits for the activations only).
    UnitRegs ra, rb;
    u32x4 xcur[KPW][DX];
    auto step = [&](const Unit &uc, UnitRegs &cur, UnitRegs &nxt) {
      issue_x(uc, xcur);
      __builtin_amdgcn_sched_barrier(0);
      issue_w(next_unit(uc), nxt);
      __builtin_amdgcn_sched_barrier(0);
      finish(uc, cur, xcur);
    };
    issue_w(u, ra);
    while (valid(u)) {
      step(u, ra, rb);
      u = next_unit(u);
      if (!valid(u)) break;
      step(u, rb, ra);
      u = next_unit(u);
    }
  } else {
    // Ring of NB register sets: unit i+NB-1 is issued before unit i is multiplied.
    UnitRegs ring[NB];
    Unit ahead = u;
#pragma unroll
    for (int s = 0; s < NB - 1; ++s) {
      issue_w(ahead, ring[s]);
      issue_x(ahead, ring[s].xb);
      ahead = next_unit(ahead);
    }
    while (valid(u)) {
#pragma unroll
      for (int s = 0; s < NB; ++s) {
        if (valid(u)) {
          issue_w(ahead, ring[(s + NB - 1) % NB]);
          issue_x(ahead, ring[(s + NB - 1) % NB].xb);
          ahead = next_unit(ahead);
          __builtin_amdgcn_sched_barrier(0);
          finish(u, ring[s], ring[s].xb);
          u = next_unit(u);
        }
      }
    }
  }
}

// X-stationary variant.  A workgroup owns a contiguous run of units ordered
// (active expert, group of <= 16 tokens, 16-row weight tile), so the group's
// activations are loaded once and stay in registers while its tiles stream
// through a ring of NB weight register sets: the registers a per-unit
// activation copy would take hold more weights in flight instead.  A group
// change drains the ring once (one HBM round trip per group and workgroup).
constexpr int kPersistMaxGroups = kPersistMaxE + 1 + kPersistMaxRows / 16;

//
// RT = 2 (down stage only): a unit is two adjacent 16-row tiles, multiplied
// with the same activation registers and summed in one LDS round, which
// halves the barriers per weight byte where a tile is small (NVFP4 tiles of a
// short contraction).
//
// ROUTE: the gate/up stage of the fused layer call -- the segments come from
// route_prologue instead of offsets / sorted rows in memory.
// With ROUTE the weight rows per tile are a.tile_rows, 16 or 8 (8: rows 8..15
// of the MFMA operand load nothing; twice the units, for batches whose 16-row
// units would not spread evenly over the compute units).
template <int WF, bool GLU, int WAVES, int KPW, int NB, int RT = 1, bool ROUTE = false>
__device__ __forceinline__ void stream_persist_xs(const PersistArgs &a, float *s_red) {
  static_assert(NB >= 2, "the ring needs two register sets");
  static_assert(RT == 1 || (RT == 2 && !GLU), "two row tiles per unit: down stage only");
  static_assert(!ROUTE || GLU, "the routing prologue feeds the gate/up stage");
  const int TR = ROUTE ? a.tile_rows : 16;
  constexpr int THREADS = WAVES * 64;
  constexpr int NW = WAVES;
  constexpr int MATS = GLU ? 2 : RT;
  constexpr int KB = stream_kblock<WF>();
  constexpr int DL = WFrag<WF, MATS>::DL;
  constexpr int DX = WF == WF_FP4 ? 8 : 4;
  __shared__ int s_e[kPersistMaxE + 1];      // expert id (E = shared expert)
  __shared__ int s_pos[kPersistMaxE + 1];    // first permuted row of its segment
  __shared__ int s_m[kPersistMaxE + 1];      // rows of its segment
  __shared__ int s_slot[kPersistMaxE + 1];
  __shared__ int s_gbase[kPersistMaxE + 1];  // first token group of active expert i
  __shared__ int s_gexp[kPersistMaxGroups];  // active expert of token group g
  __shared__ int s_cnt[NW];
  __shared__ int s_tok[GLU ? kPersistMaxRows : 1];  // token of every routed row (gather mode: gate/up only)
  constexpr int RE = ROUTE ? kRouteMaxE + 1 : 1, RR = ROUTE ? kRouteMaxRows : 1;
  __shared__ int32_t s_roff[RE], s_rids[RR], s_rrows[RR], s_rpos[RR], s_rsorted[RR];
  // Down stage: the units' fp32 outputs are staged here and written out kStageCols columns at a
  // time, as whole row segments, rather than a few floats per row per unit in the middle of the
  // weight stream (measured at 64 tokens, bf16 weights: 78.9 -> 74.3 us; the output rows' write
  // traffic slowed the weight reads, and writing it in fewer, later bursts interferes less)
  constexpr int UC = 16 * RT;                    // output columns of a unit
  constexpr int BU = GLU ? 1 : kStageCols / UC;  // units per staged window
  constexpr int SP = kStageCols + 4;             // row pitch (floats)
  __shared__ float s_y[GLU ? 1 : 16 * SP];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int32_t *offs = a.offsets, *srows = a.sorted_rows;
  if constexpr (ROUTE) {
    route_prologue<THREADS>(a, s_rids, s_roff, s_rrows, s_rpos, s_rsorted);
    offs = s_roff;
    srows = s_rrows;
  }
  const bool gather = GLU && srows != nullptr;  // the down stage reads hidden rows in order
  if (gather)
    for (int p = tid; p < a.T * a.k; p += THREADS) s_tok[p] = srows[p] / a.k;
  const int r = lane & 15, q = lane >> 4;

  // ---- active-expert table (ascending expert id, then the shared expert)
  int base = 0;
  for (int c0 = 0; c0 < a.E; c0 += THREADS) {
    const int e = c0 + tid;
    int lo = 0, cnt = 0;
    if (e < a.E) {
      lo = offs[e];
      cnt = offs[e + 1] - lo;
      if (cnt > 0 && a.slot_of_expert != nullptr && a.slot_of_expert[e] == FT_SLOT_SKIP) cnt = 0;  // another call's
    }
    const bool f = cnt > 0;
    const uint64_t mask = __ballot(f);
    if (lane == 0) s_cnt[wave] = __popcll(mask);
    __syncthreads();
    int before = base, total = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      if (w < wave) before += s_cnt[w];
      total += s_cnt[w];
    }
    if (f) {
      const int i = before + __popcll(mask & ((uint64_t(1) << lane) - 1));
      s_e[i] = e;
      s_pos[i] = lo;
      s_m[i] = cnt;
      s_slot[i] = table_slot(a.slot_of_expert, e, a.n_slots);
    }
    base += total;
    __syncthreads();
  }
  int n_act = base;
  if (a.shared_blob != nullptr) {
    if (tid == 0) {
      s_e[n_act] = a.E;
      s_pos[n_act] = a.T * a.k;
      s_m[n_act] = a.T;
      s_slot[n_act] = 0;
    }
    ++n_act;
    __syncthreads();
  }
  // ---- token groups: ceil(m / 16) per active expert, prefix-summed
  int n_groups = 0;
  for (int c0 = 0; c0 < n_act; c0 += THREADS) {
    const int i = c0 + tid;
    const int g = i < n_act ? (s_m[i] + 15) >> 4 : 0;
    const int v = wave_incl_scan_i32(g);
    if (lane == 63) s_cnt[wave] = v;
    __syncthreads();
    int before = n_groups, total = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      if (w < wave) before += s_cnt[w];
      total += s_cnt[w];
    }
    if (i < n_act) {
      const int gb = before + v - g;
      s_gbase[i] = gb;
      for (int j = 0; j < g && gb + j < kPersistMaxGroups; ++j) s_gexp[gb + j] = i;  // <= 1220 groups for T <= 64
    }
    n_groups += total;
    __syncthreads();
  }

  // ---- this workgroup's run of units
  const int n_tiles = RT == 1 ? a.n_tiles : (a.N + 16 * RT - 1) / (16 * RT);  // units per token group
  const int n_units = n_groups * n_tiles;
  const int u_begin = int(int64_t(n_units) * blockIdx.x / gridDim.x);
  const int u_end = int(int64_t(n_units) * (blockIdx.x + 1) / gridDim.x);

  const uint32_t wpitch = (WF == WF_BF16) ? uint32_t(a.K) * 2 : uint32_t(a.K) / 2;
  const uint32_t spitch = uint32_t(a.K) / (WF == WF_NV4 ? 16 : 32);
  const uint32_t wbytes = uint32_t(a.N) * wpitch, sbytes = uint32_t(a.N) * spitch;
  const rsrc_t xres = make_rsrc(a.X, a.x_bytes);

  // Weights of tile `tile` of active expert ai (tile < 0: past the run; the
  // loads still issue, at an offset past the buffer, so every ring step
  // issues the same number of loads).
  auto issue_w = [&](int ai, int tile, WFrag<WF, MATS> (&f)[KPW]) {
    const int e = uniform(s_e[ai]), slot = uniform(s_slot[ai]);
    const uint8_t *blob = e == a.E ? a.shared_blob : a.pool + uint64_t(max(slot, 0)) * a.expert_bytes;
    rsrc_t wres[MATS], sres[MATS];
    wres[0] = make_rsrc(blob + a.off_w0, wbytes);
    sres[0] = make_rsrc(blob + a.off_s0, sbytes);
    if constexpr (GLU) {
      wres[MATS - 1] = make_rsrc(blob + a.off_w1, wbytes);
      sres[MATS - 1] = make_rsrc(blob + a.off_s1, sbytes);
    } else if constexpr (RT == 2) {
      wres[1] = wres[0];
      sres[1] = sres[0];
    }
    // rows past N fall outside the buffer (zeros, no traffic); so do operand rows past TR
    constexpr int NH = wl_halves<WF>();  // row halves of the whole-line loads (d & 1)
    uint32_t wo[MATS][NH], so[MATS];
#pragma unroll
    for (int mt = 0; mt < MATS; ++mt) {
      const int row0 = tile * TR * RT + (GLU ? 0 : 16 * mt);
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        const int rr = wl_row<WF>(lane, h);
        wo[mt][h] = tile >= 0 && rr < TR ? uint32_t(row0 + rr) * wpitch + wl_byte<WF>(lane, h) : kOOB;
      }
      so[mt] = tile >= 0 && r < TR ? uint32_t(row0 + r) * spitch : kOOB;
    }
#pragma unroll
    for (int c = 0; c < KPW; ++c) {
      const int kb = wave + c * WAVES;
#pragma unroll
      for (int mt = 0; mt < MATS; ++mt) {
#pragma unroll
        for (int d = 0; d < DL; ++d)
          f[c].w[mt][d] = wl_load<WF>(wres[mt], wo[mt][d % NH] + uint32_t(kb) * wl_kbytes<WF>() + wl_dcol<WF>(d));
        if constexpr (WF != WF_BF16) f[c].s[mt] = bld8(sres[mt], so[mt] + uint32_t(kb) * 8);  // 8 blocks
      }
    }
  };
  // Activations of token group (ai, g0): this lane's token row.
  auto issue_x = [&](int ai, int g0, u32x4 (&xb)[KPW][DX]) {
    const int e = uniform(s_e[ai]), pos = uniform(s_pos[ai]), m = uniform(s_m[ai]);
    const int j = g0 + r;
    int row = -1;
    if (j < m) {
      if (!gather) row = pos + j;                        // hidden row p
      else row = e == a.E ? j : s_tok[pos + j];         // token of the shared / routed expert
    }
    const uint32_t xo = row >= 0 ? uint32_t(row) * uint32_t(a.ldx) * 2u : kOOB;
#pragma unroll
    for (int c = 0; c < KPW; ++c) {
      const int kb = wave + c * WAVES;
#pragma unroll
      for (int dx = 0; dx < DX; ++dx) {
        xb[c][dx] = bld16(xres, xo + uint32_t(kb * KB + wl_xk<WF>(dx, q)) * 2u);
      }
    }
  };
  // Multiply one tile of group (ai, g0), sum the wave partials in LDS, write
  // its 16x16 output tile (down stage: into the staging buffer).
  int wb = 0;  // down stage: the first unit of the staged window
  auto finish = [&](int ai, int g0, int tile, const WFrag<WF, MATS> (&f)[KPW], const u32x4 (&xcur)[KPW][DX],
                    float ts0, float ts1) {
    const int e = uniform(s_e[ai]), slot = uniform(s_slot[ai]), pos = uniform(s_pos[ai]), m = uniform(s_m[ai]);
    const bool shared = e == a.E;
    const bool missing = !shared && slot < 0;
    f32x4 acc[MATS];
#pragma unroll
    for (int mt = 0; mt < MATS; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < KPW; ++c) {
      WFrag<WF, MATS> fc = f[c];
      wfrag_fix(fc);
      if constexpr (WF == WF_BF16) {
#pragma unroll
        for (int d = 0; d < 4; ++d)
#pragma unroll
          for (int mt = 0; mt < MATS; ++mt) acc[mt] = mfma16(as_bf16x8(fc.w[mt][d]), as_bf16x8(xcur[c][d]), acc[mt]);
      } else if constexpr (WF == WF_FP4) {
#pragma unroll
        for (int d = 0; d < 2; ++d) {
          float sc[MATS];
#pragma unroll
          for (int mt = 0; mt < MATS; ++mt) sc[mt] = e8m0_to_f32(wl_mx_scale<WF>(fc.s[mt], d, q));
#pragma unroll
          for (int mm = 0; mm < 4; ++mm)
#pragma unroll
            for (int mt = 0; mt < MATS; ++mt)
              acc[mt] = mfma16(fp4x8_to_bf16x8(fc.w[mt][d][mm], sc[mt]), as_bf16x8(xcur[c][4 * d + mm]), acc[mt]);
        }
      } else {
        // NVFP4: lane (r, q) holds elements 32q .. 32q+31 of the k-block (16-element
        // blocks 2q and 2q+1); word mm covers 32q + 8mm .. +7, block 2q + mm/2.
#pragma unroll
        for (int mm = 0; mm < 4; ++mm)
#pragma unroll
          for (int mt = 0; mt < MATS; ++mt) {
            const uint32_t sw = (q >> 1) ? f[c].s[mt][1] : f[c].s[mt][0];
            const float sc = e4m3_to_f32(sw >> (8 * ((2 * q + (mm >> 1)) & 3)));
            acc[mt] = mfma16(nvfp4x8_to_bf16x8(f[c].w[mt][0][mm], sc), as_bf16x8(xcur[c][mm]), acc[mt]);
          }
      }
    }
#pragma unroll
    for (int mt = 0; mt < MATS; ++mt)
      *reinterpret_cast<f32x4 *>(&s_red[((wave * MATS + mt) * 64 + lane) * 4]) = acc[mt];
    __syncthreads();
    if (tid < 256) {
      const int ln = tid >> 2, v = tid & 3;
      const int jj = g0 + (ln & 15);
      const int nr = 4 * (ln >> 4) + v;                 // row inside the tile
      const int n = tile * TR * RT + nr;                 // RT = 2: uu is row n + 16
      float g = 0.f, uu = 0.f;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) {
        g += s_red[((w * MATS + 0) * 64 + ln) * 4 + v];
        if constexpr (MATS == 2) uu += s_red[((w * MATS + 1) * 64 + ln) * 4 + v];
      }
      if constexpr (WF == WF_NV4) {  // the per-tensor scales, on the fp32 sums
        g *= ts0;
        if constexpr (GLU) uu *= ts1;
        else if constexpr (RT == 2) uu *= ts0;
      }
      if (jj < m && n < a.N && nr < TR) {
        const int p = pos + jj;  // permuted row; hidden rows of the shared expert follow the routed ones
        if constexpr (GLU) {
          reinterpret_cast<uint16_t *>(a.out)[int64_t(p) * a.ldo + n] =
              missing ? uint16_t(0x7fc0) : f32_to_bf16_rne(silu(g) * uu);
        } else {
          float *sy = &s_y[(ln & 15) * SP + (tile - wb) * UC + nr];
          sy[0] = missing ? __builtin_nanf("") : g;
          if constexpr (RT == 2) sy[16] = missing ? __builtin_nanf("") : uu;
        }
      }
    }
    __syncthreads();
  };
  // Down stage: write out the staged outputs of units [wb, wb + nu) of token group (ai, g0): rows
  // of up to kStageCols consecutive floats, four per lane where the rows allow.  (Called after
  // finish's last barrier; the next finish writes the buffer only after its own first barrier.)
  const bool y16 = ((reinterpret_cast<uintptr_t>(a.out) | reinterpret_cast<uintptr_t>(a.out_shared) |
                     uintptr_t(a.ldo) * 4u) & 15u) == 0;
  auto flush = [&](int ai, int g0, int nu) {
    if constexpr (!GLU) {
      const int e = uniform(s_e[ai]), pos = uniform(s_pos[ai]), m = uniform(s_m[ai]);
      const int rows = min(16, m - g0);
      const int c0 = wb * UC, cols = min(nu * UC, a.N - c0);  // columns past N were never computed
      if (rows <= 0 || cols <= 0) return;
      auto row_ptr = [&](int i) {
        const int jj = g0 + i;  // hidden rows of the shared expert follow the routed ones
        return e == a.E ? a.out_shared + int64_t(jj) * a.ldo : reinterpret_cast<float *>(a.out) + int64_t(pos + jj) * a.ldo;
      };
      if (y16 && (cols & 3) == 0) {
        const int q4 = cols >> 2;
        for (int idx = tid; idx < rows * q4; idx += THREADS) {
          const int i = idx / q4, c = (idx - i * q4) * 4;
          *reinterpret_cast<f32x4 *>(row_ptr(i) + c0 + c) = *reinterpret_cast<const f32x4 *>(&s_y[i * SP + c]);
        }
      } else {
        for (int idx = tid; idx < rows * cols; idx += THREADS) {
          const int i = idx / cols, c = idx - i * cols;
          row_ptr(i)[c0 + c] = s_y[i * SP + c];
        }
      }
    }
  };

  WFrag<WF, MATS> ring[NB][KPW];
  u32x4 xcur[KPW][DX];
  int u = u_begin;
  while (u < u_end) {
    const int gi = u / n_tiles;
    const int t_begin = u - gi * n_tiles;
    const int t_end = min(n_tiles, u_end - gi * n_tiles);
    const int ai = uniform(s_gexp[gi]);
    const int g0 = (gi - uniform(s_gbase[ai])) * 16;
    float ts0 = 1.f, ts1 = 1.f;  // NVFP4 tensor scales of this expert, loaded once per group
    if constexpr (WF == WF_NV4) {
      const int e = uniform(s_e[ai]), slot = uniform(s_slot[ai]);
      const uint8_t *blob = e == a.E ? a.shared_blob : a.pool + uint64_t(max(slot, 0)) * a.expert_bytes;
      ts0 = *reinterpret_cast<const float *>(blob + a.off_t0);
      if constexpr (GLU) ts1 = *reinterpret_cast<const float *>(blob + a.off_t1);
    }
    issue_x(ai, g0, xcur);
#pragma unroll
    for (int s = 0; s < NB - 1; ++s) issue_w(ai, t_begin + s < t_end ? t_begin + s : -1, ring[s]);
    wb = t_begin;
    for (int t = t_begin; t < t_end; t += NB) {
#pragma unroll
      for (int s = 0; s < NB; ++s) {
        const int ta = t + s + NB - 1;  // the tile issued at this step
        issue_w(ai, ta < t_end ? ta : -1, ring[(s + NB - 1) % NB]);
        __builtin_amdgcn_sched_barrier(0);
        if (t + s < t_end) {
          finish(ai, g0, t + s, ring[s], xcur, ts0, ts1);
          if constexpr (!GLU) {
            // the window is full or the run ends: write it out
            if (t + s + 1 - wb == BU || t + s + 1 == t_end) {
              flush(ai, g0, t + s + 1 - wb);
              wb = t + s + 1;
            }
          }
        }
      }
    }
    u = gi * n_tiles + t_end;
  }
}

}  // namespace ft
