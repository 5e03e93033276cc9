// One-token decode as matrix-vector products (the fused layer call at T = 1).
//
// With one token every expert matrix is read once and multiplied by one
// vector: HBM-bound work with no reuse, so no MFMA tile.  A workgroup owns a
// fixed block of weight rows, issues all of their 16-byte loads at once (the
// whole block in flight, one HBM round trip), and each wave reduces its rows'
// dot products with DPP lane moves.  Many small workgroups rather than a
// persistent grid: at one token a persistent unit (expert table, LDS
// reduction, barriers per 16-row tile) costs more than its weight stream.
//
// The kernels that wrap these bodies ask for at least two waves per SIMD
// (up to 256 registers), so a wave's whole block of loads stays in registers;
// with the default budget the compiler waited for early loads before issuing
// the rest.
//
// Row layout: 64 lanes cover 1 KiB of a row's codes per "chunk" (lane l holds
// bytes 16 l .. 16 l + 15 of chunk c, i.e. byte 1024 c + 16 l); a row of B
// code bytes has ceil(B / 1024) chunks, the last possibly partial.
//   bf16  : 16 bytes = 8 elements
//   MXFP4 : 16 bytes = 32 elements = one E8M0 block (scale byte 64 c + l)
//   NVFP4 : 16 bytes = 32 elements = two E4M3 blocks (scale bytes 2 (64 c + l), +1)
#pragma once

#include "stream_persist.hpp"

namespace ft {

// Weight rows are read here 1 KiB per load (whole lines) and once per call: bf16 and MXFP4 rows with
// the non-temporal bit (one-token layer call measured 20.8 -> 20.5 us bf16, 27.1 -> 26.5 us MXFP4);
// NVFP4 rows without it (measured 0.2 us slower with it).
template <int WF>
__device__ __forceinline__ u32x4 wload(rsrc_t r, uint32_t off) {
  if constexpr (WF == WF_NV4) return bld16(r, off);
  else return bld16nt(r, off);
}

constexpr int kGemvThreads = 256;   // down + combine: 4 waves
constexpr int kGemvGuThreads = 512; // gate/up: 8 waves
constexpr int kGemvMaxChunks = 4;   // rows of at most 4 KiB of codes

template <int WF>
struct GemvFmt {
  static constexpr int EPC = WF == WF_BF16 ? 8 : 32;    // elements per 16-byte chunk piece
  static constexpr int XV = EPC / 8;                    // u32x4 of bf16 activations per piece
};

// fp32 dot of one 16-byte weight piece with its activations (bf16 pairs, element order).  The
// products run on v_dot2 (two bf16 products added to an fp32 accumulator); FP4 codes are widened
// to bf16 pairs first, which is exact: an E2M1 value has 2 significant bits, times a power of two
// (MXFP4, applied in the conversion) or later times an E4M3 scale of 4 significant bits (NVFP4,
// applied to each 16-element block's sum, since the scaled conversions use only the exponent of
// their scale).
// Four partial sums per dot product, one per dword of the piece, so that consecutive v_dot2 do not
// wait on each other (a single accumulator chained 16 of them per MXFP4 piece: measured 3 us of a
// 27 us one-token layer in the products).
struct Acc4 {
  float a[4];
  __device__ __forceinline__ Acc4() : a{0.f, 0.f, 0.f, 0.f} {}
  __device__ __forceinline__ float sum() const { return (a[0] + a[1]) + (a[2] + a[3]); }
};

template <int WF>
__device__ __forceinline__ void piece_dot(const u32x4 w, const uint32_t scw, const u32x4 *x, Acc4 &acc) {
  // the lane's scale bits in the dword piece_scale loaded (piece 64 c + lane: byte lane % 4 for
  // MXFP4, bytes 2 (lane % 2) and up for NVFP4)
  const uint32_t sc = WF == WF_FP4 ? scw >> (8 * (threadIdx.x & 3)) : scw >> (16 * (threadIdx.x & 1));
  if constexpr (WF == WF_BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc.a[i] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w[i]), as_bf16x2(x[0][i]), acc.a[i], false);
  } else if constexpr (WF == WF_FP4) {
    // dword d holds elements 8d .. 8d+7, byte b of it elements 8d+2b, 8d+2b+1 (low nibble first);
    // activations dword x[d][b] holds the same two elements (the selector operand must be a literal)
    const float s = e8m0_to_f32(sc & 0xffu);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      float t = acc.a[d];
      t = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[d], s, 0), as_bf16x2(x[d][0]), t, false);
      t = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[d], s, 1), as_bf16x2(x[d][1]), t, false);
      t = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[d], s, 2), as_bf16x2(x[d][2]), t, false);
      t = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[d], s, 3), as_bf16x2(x[d][3]), t, false);
      acc.a[d] = t;
    }
  } else {
    // two 16-element blocks (dwords 0-1: scale byte 0, dwords 2-3: byte 1), each summed unscaled
    float blk[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      float b = 0.f;
      b = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[d], 1.0f, 0), as_bf16x2(x[d][0]), b, false);
      b = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[d], 1.0f, 1), as_bf16x2(x[d][1]), b, false);
      b = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[d], 1.0f, 2), as_bf16x2(x[d][2]), b, false);
      b = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[d], 1.0f, 3), as_bf16x2(x[d][3]), b, false);
      blk[d] = b;
    }
    const float s0 = e4m3_to_f32(sc & 0xffu), s1 = e4m3_to_f32((sc >> 8) & 0xffu);
    acc.a[0] = fmaf(s0, blk[0], acc.a[0]);
    acc.a[1] = fmaf(s0, blk[1], acc.a[1]);
    acc.a[2] = fmaf(s1, blk[2], acc.a[2]);
    acc.a[3] = fmaf(s1, blk[3], acc.a[3]);
  }
}

// The aligned dword holding the scale bits of piece `piece` (= 64 c + lane) of the row whose scales
// start at byte `so` of `sres` (the 4-bit formats; no per-lane byte loads; an offset at or past the
// buffer gives 0).  MXFP4: one byte; NVFP4: two bytes, elements 0..15 then 16..31.  The word is
// returned as loaded: piece_dot shifts the lane's bits out where it uses them, so that issuing a
// job's loads never waits for one of them.
template <int WF>
__device__ __forceinline__ uint32_t piece_scale(rsrc_t sres, uint32_t so, int piece, bool ok) {
  if constexpr (WF == WF_BF16) {
    return 0u;
  } else {
    const uint32_t b = WF == WF_FP4 ? uint32_t(piece) : 2u * uint32_t(piece);
    return bld4(sres, ok ? so + (b & ~3u) : kOOB);
  }
}

// ---------------------------------------------------------------- routing of the one token

// Top-k, gating and permutation of one token by one wave (all 64 lanes call
// it); lane j < k ends with pick j.  The order is topk_token's: descending
// logit, the lower expert index first among equal logits, softmax over all E
// or element-wise sigmoid, optionally renormalised over the picks.  A round
// is a 32-bit wave max of the logits' order keys and one ballot per logit
// slot for the lowest index holding it (topk_token carries the index in a
// 64-bit key instead, which doubles every butterfly step).  The picks are
// distinct experts, so the token's permuted rows are the picks in ascending
// id and a pick's row is its rank among them.
struct TokenPick {
  int id;     // expert (lanes >= k: -1)
  float w;    // gating weight
  int rank;   // position of the pick among the picks in ascending expert id = its permuted row
};

// The token's logits, lane l holding experts l, l + 64, ... (separate from the routing so that loads
// which do not depend on it can be issued between the two).
struct TokenLogits {
  float v[kRouteMaxE / 64];
};

__device__ __forceinline__ TokenLogits one_token_logits(const float *__restrict__ lr, int E) {
  const int lane = threadIdx.x & 63;
  const rsrc_t res = make_rsrc(lr, uint32_t(E) * 4u);  // past E: 0 (masked by the routing)
  TokenLogits t;
#pragma unroll
  for (int i = 0; i < kRouteMaxE / 64; ++i) t.v[i] = __uint_as_float(bld4(res, uint32_t(lane + 64 * i) * 4u));
  return t;
}

// s_pick / s_npicks (LDS, nullable): pick j's expert is stored as soon as it is found, then the count
// of picks found, so that other waves can start on pick j's weights while later picks are searched.
__device__ __forceinline__ TokenPick one_token_route(const TokenLogits &lg, int E, int k, int gating,
                                                     int renorm, int *s_pick = nullptr,
                                                     int *s_npicks = nullptr) {
  constexpr int VPL = kRouteMaxE / 64;
  const int lane = threadIdx.x & 63;
  const float *v = lg.v;
  uint32_t key[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    // 0 marks "absent or already picked": real keys start at 1 (only the all-ones NaN maps to 0)
    const uint32_t kk = order_key(v[i]);
    key[i] = lane + 64 * i < E ? (kk == 0u ? 1u : kk) : 0u;
  }
  int pid = -1;
  float pval = 0.f, mx = 0.f;
  for (int j = 0; j < k; ++j) {
    uint32_t m = key[0];
#pragma unroll
    for (int i = 1; i < VPL; ++i) m = max(m, key[i]);
    m = wave_max_u32(m);
    int e = 1 << 30;  // the lowest expert index whose key is m (scalar); lower slots hold lower indices
#pragma unroll
    for (int i = VPL - 1; i >= 0; --i) {
      const uint64_t b = __ballot(key[i] == m);
      e = b != 0 ? 64 * i + int(__builtin_ctzll(b)) : e;
    }
#pragma unroll
    for (int i = 0; i < VPL; ++i) key[i] = lane + 64 * i == e ? 0u : key[i];
    if (s_pick != nullptr && lane == 0) {
      s_pick[j] = e;
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0): the pick lands first
      __hip_atomic_store(s_npicks, j + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    if (j == 0) mx = key_value(m);  // the largest logit
    if (lane == j) {
      pid = e;
      pval = key_value(m);
    }
  }
  float denom = 1.0f;
  if (gating == FT_SOFTMAX) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      if (lane + 64 * i < E) s += expf(v[i] - mx);
    denom = wave_sum_f32(s);
  }
  float p = 0.f;
  if (lane < k) p = gating == FT_SOFTMAX ? expf(pval - mx) / denom : 1.0f / (1.0f + expf(-pval));
  const float wsum = renorm ? wave_sum_f32(p) : 1.0f;
  int rank = 0;
  for (int i = 0; i < k; ++i) rank += __builtin_amdgcn_readlane(pid, i) < pid ? 1 : 0;
  return TokenPick{pid, renorm ? p / wsum : p, rank};
}

// ---------------------------------------------------------------- one-token layer kernel: the wait

// The one-token layer kernel runs gate/up and then down + combine in one
// launch; the down stage needs every hidden value, so the workgroups meet at a
// grid-wide wait in between.  The grid never exceeds the workgroups that fit
// on the device at once, so every workgroup is resident and the wait ends.
//
// The wait is two-level, so that no memory word takes more than a few dozen
// atomic adds (one word for all workgroups measured about 20 us): workgroup b
// counts itself in group b % 16; the last of a group counts the group in the
// top counter; the last group bumps the 16 copies of the round number, each
// group polling its own copy.  Counters and copies sit on separate 128-byte
// lines.  The last arrival at each counter clears it, so all counters are zero
// again for the next launch.
//
// The hidden values cross the compute dies' separate L2 caches: they are
// stored and loaded with agent-scope coherence (the sc1 cache policy), and a
// wave waits for its stores to complete before its workgroup arrives.  (An
// agent-scope release / acquire fence would write back and invalidate the
// whole L2 instead, thousands of times per launch: measured about 150 us.)
// The wait is bounded: after kBarrierPolls polls of the round copy it gives
// up and reports false (the caller then writes NaN).
constexpr int kBarrierPolls = 1 << 16;
constexpr int kCoherentAgent = 16;  // buffer cache policy: sc1 (agent scope)
constexpr int kWaitGroups = 16;
constexpr int kWaitStride = 32;     // words between counters: one 128-byte line each
static_assert(kWaitStride * 4 * (2 * kWaitGroups + 1) <= int(kLayerWaitBytes), "wait words fit their area");

// PENDING: vector memory operations this wave issued after its last hidden store (they may stay in
// flight; everything before them, the stores included, has completed when the wave arrives).
template <int PENDING>
__device__ __forceinline__ bool grid_wait(uint32_t *bar) {
  __shared__ int s_ok;
  wait_vmcnt<PENDING>();
  lds_barrier();  // orders LDS only: the loads left in flight stay in flight
  if (threadIdx.x == 0) {
    const int G = int(gridDim.x), b = int(blockIdx.x);
    const int ng = G < kWaitGroups ? G : kWaitGroups;
    const int grp = b % ng;
    const uint32_t gs = uint32_t((G - grp + ng - 1) / ng);  // workgroups in this group
    uint32_t *cnt = bar + kWaitStride * grp, *top = bar + kWaitStride * kWaitGroups;
    uint32_t *rnd = bar + kWaitStride * (kWaitGroups + 1 + grp);
    const uint32_t round = __hip_atomic_load(rnd, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (__hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == gs - 1) {
      __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (__hip_atomic_fetch_add(top, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == uint32_t(ng - 1)) {
        __hip_atomic_store(top, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        for (int g = 0; g < ng; ++g)
          __hip_atomic_fetch_add(bar + kWaitStride * (kWaitGroups + 1 + g), 1u, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    int ok = 1, n = 0;
    while (__hip_atomic_load(rnd, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == round) {
      if (++n >= kBarrierPolls) {
        ok = 0;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    s_ok = ok;
  }
  lds_barrier();
  return s_ok != 0;
}

// Down + combine of the one token after the wait.  Wave w takes step w -- the
// pick of rank w (hidden row w) or, at w = k, the shared expert -- for the
// workgroup's blocks of RB output rows; the step weights of the first block
// are loaded before the wait (they depend only on the routing, which every
// workgroup holds in LDS), the hidden row after it.  Per row the waves'
// weighted dots meet in LDS and are added in wave order.
template <int WF, int NCHD, int RB>
__device__ __forceinline__ void token_down_after_wait(const PersistArgs &d, uint32_t *bar, const int *s_act,
                                                      const float *s_w, const int *s_slot, int S) {
  constexpr int WAVES = kGemvGuThreads / 64;
  using F = GemvFmt<WF>;
  __shared__ float s_part[WAVES][RB];
  const int tid = threadIdx.x, wave = uniform(tid >> 6), lane = tid & 63;
  const uint32_t rbytes = WF == WF_BF16 ? uint32_t(d.K) * 2 : uint32_t(d.K) / 2;
  const uint32_t sbytes = WF == WF_FP4 ? uint32_t(d.K) / 32 : (WF == WF_NV4 ? uint32_t(d.K) / 16 : 0u);
  const bool live = wave < S;
  const int e = live ? uniform(s_act[wave]) : -1;
  const bool shared = e == d.E;
  const int slot = (e < 0 || shared) ? 0 : uniform(s_slot[e]);
  const bool missing = live && !shared && slot < 0;
  const uint8_t *blob = shared ? d.shared_blob : d.pool + uint64_t(slot < 0 ? 0 : slot) * d.expert_bytes;
  const float wgt = !live ? 0.f : (shared ? 1.f : s_w[wave]);
  const rsrc_t wres = make_rsrc(blob + d.off_w0, uint32_t(d.N) * rbytes);
  const rsrc_t sres = make_rsrc(blob + d.off_s0, uint32_t(d.N) * sbytes);
  float ts = 1.f;
  if constexpr (WF == WF_NV4)
    if (live) ts = *reinterpret_cast<const float *>(blob + d.off_t0);
  const int blocks = (d.N + RB - 1) / RB;
  u32x4 w[RB][NCHD];
  uint32_t sc[RB][NCHD];
  auto issue = [&](int rb) {
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
      for (int c = 0; c < NCHD; ++c) {
        const int row = rb * RB + r;
        const uint32_t cb = 1024u * c + 16u * lane;
        const bool ok = live && row < d.N && cb < rbytes;
        w[r][c] = wload<WF>(wres, ok ? uint32_t(row) * rbytes + cb : kOOB);
        sc[r][c] = piece_scale<WF>(sres, uint32_t(row) * sbytes, int(cb >> 4), ok);
      }
  };
  // the first block's loads always issue (past the rows: offsets past the buffers), so the wait
  // knows how many of this wave's memory operations follow its hidden stores
  int rb = int(blockIdx.x);
  __builtin_amdgcn_sched_barrier(0);
  issue(rb);
  __builtin_amdgcn_sched_barrier(0);
  const bool ok = grid_wait<RB * NCHD * (WF == WF_BF16 ? 1 : 2)>(bar);
  const rsrc_t hres = make_rsrc(d.X, d.x_bytes);
  u32x4 hv[NCHD][F::XV];
#pragma unroll
  for (int c = 0; c < NCHD; ++c)
#pragma unroll
    for (int v = 0; v < F::XV; ++v) {
      const uint32_t el = uint32_t(64 * c + lane) * F::EPC + 8u * v;
      hv[c][v] = __builtin_amdgcn_raw_buffer_load_b128(
          hres, (live && el < uint32_t(d.K)) ? (uint32_t(wave) * uint32_t(d.ldx) + el) * 2u : kOOB, 0, kCoherentAgent);
    }
  for (; rb < blocks; rb += int(gridDim.x)) {
    if (rb != int(blockIdx.x)) issue(rb);
    float dv[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      Acc4 dd;
#pragma unroll
      for (int c = 0; c < NCHD; ++c) piece_dot<WF>(w[r][c], sc[r][c], hv[c], dd);
      dv[r] = dd.sum();
    }
    const float tot = wave_sums<RB>(dv);
    if ((lane & (RB == 8 ? 7 : 15)) == 0)  // the first lane of each group holds one row's total
      s_part[wave][wave_sums_index<RB>(lane)] = missing ? __builtin_nanf("") : wgt * (ts * tot);
    __syncthreads();
    if (tid < RB) {
      const int row = rb * RB + tid;
      float v = 0.f;
#pragma unroll
      for (int w2 = 0; w2 < WAVES; ++w2) v += s_part[w2][tid];
      if (!ok) v = __builtin_nanf("");
      if (row < d.N) {
        if (d.comb_bf16) reinterpret_cast<uint16_t *>(d.comb_out)[row] = f32_to_bf16_rne(v);
        else reinterpret_cast<float *>(d.comb_out)[row] = v;
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- gate/up + SwiGLU, one token

// Work is a list of wave jobs: RPW consecutive (gate row, up row) pairs of one
// expert, the shared expert's first (when there is one), then the routed
// experts' in pick order.  Every workgroup routes the token itself
// (one_token_route in wave 0; workgroup 0 publishes the result); each wave
// takes a contiguous run of the job list, the next job's loads issued before
// the current job is multiplied.  The grid is sized to the workgroups that
// fit on the device at once, so no workgroup pays the prologue in a second
// round.
//
// The routing overlaps the weight stream: wave 0 stores each pick in LDS as
// soon as its top-k round finds it, and a wave issues a job as soon as the
// job's expert is known (a shared-expert job at once).  Wave 0's loads of
// the activations, slot table entries and logits go out first, in one round
// trip.  Data every wave reads is fetched once
// per workgroup: the activations go through LDS (per wave they would be the
// same few KiB read by thousands of waves from the few L2 channels that hold
// them), and large (8-wave) workgroups keep that shared traffic small.
template <int WF, int NCH, int RPW, int NCHD = 0, int RB = 0>
__device__ __forceinline__ void gemv_gate_up(const PersistArgs &a, const PersistArgs *d = nullptr,
                                             uint32_t *bar = nullptr) {
  constexpr int THREADS = kGemvGuThreads, WAVES = THREADS / 64;
  using F = GemvFmt<WF>;
  constexpr int XN = NCH * 64 * F::XV;            // u32x4 of activations the lanes' pieces cover
  constexpr int XPL = (XN + 63) / 64;             // of them per lane of wave 0
  __shared__ int s_act[kFusedMaxK + 1];     // the picks in pick order (= their hidden rows), then the shared expert
  __shared__ float s_w[kFusedMaxK + 1];     // their gating weights
  __shared__ int s_slot[kRouteMaxE];        // slot of every expert (-1: not resident)
  __shared__ int s_npicks;                  // picks stored in s_act so far
  __shared__ int s_xready;                  // s_x and s_slot written
  __shared__ u32x4 s_x[XN];                 // the token's activations, u32x4 i = elements 8i .. 8i+7
  const int tid = threadIdx.x, wave = uniform(tid >> 6), lane = tid & 63;
  if (tid == 0) {
    s_npicks = 0;
    s_xready = 0;
  }
  lds_barrier();
  const uint32_t rbytes = WF == WF_BF16 ? uint32_t(a.K) * 2 : uint32_t(a.K) / 2;  // code bytes of a row
  const uint32_t sbytes = WF == WF_FP4 ? uint32_t(a.K) / 32 : (WF == WF_NV4 ? uint32_t(a.K) / 16 : 0u);
  // Raw buffer loads throughout: an offset past the buffer reads zero without a branch, so a job's
  // loads are all issued before the first wait.
  // Wave 0 loads what the workgroup shares -- activations, slot table, logits -- and routes; the
  // other waves meanwhile issue their first job when it is a shared-expert job.
  const rsrc_t xres = make_rsrc(a.X, uint32_t(a.K) * 2u);
  constexpr int SPL = kRouteMaxE / 64;
  u32x4 xg[XPL];
  int sl[SPL];
  TokenLogits lg;
  if (wave == 0) {
#pragma unroll
    for (int i = 0; i < XPL; ++i) {
      const uint32_t u = uint32_t(lane + 64 * i);
      xg[i] = bld16(xres, u < uint32_t(XN) ? u * 16u : kOOB);
    }
    // the slot table as raw words (a buffer of no bytes when there is none): no wait before the
    // logits' loads are issued
    const rsrc_t stres = make_rsrc(a.slot_of_expert, a.slot_of_expert != nullptr ? uint32_t(a.E) * 4u : 0u);
#pragma unroll
    for (int i = 0; i < SPL; ++i) sl[i] = int(bld4(stres, uint32_t(lane + 64 * i) * 4u));
    lg = one_token_logits(a.logits, a.E);
  }

  const int has_shared = a.shared_blob != nullptr ? 1 : 0;
  const int jobs_per_expert = (a.N + RPW - 1) / RPW;
  const int n_act = a.k + has_shared;
  const int n_jobs = n_act * jobs_per_expert;
  // waits on wave 0's progress (LDS polls; wave 0 depends on no other wave, so they end)
  // (LDS atomic loads of the flags themselves: through a pointer they became flat loads, whose wait
  // also waited for every weight load in flight)
  auto npicks = [&] { return __hip_atomic_load(&s_npicks, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP); };
  auto xready = [&] { return __hip_atomic_load(&s_xready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP); };
  struct Job {
    u32x4 wg[RPW][NCH], wu[RPW][NCH];
    uint32_t sg[RPW][NCH], su[RPW][NCH];
    float ts0, ts1;  // NVFP4 tensor scales
  };
  // job list entry ai: the shared expert at 0 (reads no LDS), then the picks in pick order (= hidden row)
  auto job_expert = [&](int ai) { return has_shared && ai == 0 ? a.E : uniform(s_act[ai - has_shared]); };
  auto job_row = [&](int ai) { return has_shared && ai == 0 ? a.k : ai - has_shared; };
  // Job j's expert is known once its pick has been found (a shared-expert job needs no routing).
  // `known` keeps the last count seen, so consecutive jobs of one expert read no LDS (a read here
  // also waits for this wave's own weight loads: its register may have been theirs).
  int known = 0;
  auto wait_job = [&](int j, int je) {
    if (j >= je) return;
    const int need = j / jobs_per_expert - has_shared + 1;
    if (need <= known) return;
    int n;
    while ((n = __builtin_amdgcn_readfirstlane(npicks())) < need) __builtin_amdgcn_s_sleep(1);
    known = n;
    asm volatile("" ::: "memory");  // the pick is read after its count
  };
  // the loads of job j (live false: offsets past the buffers, nothing read)
  auto issue = [&](int j, bool live, Job &J) {
    const int jj = live ? j : 0;
    const int ai = jj / jobs_per_expert, row0 = (jj - ai * jobs_per_expert) * RPW;
    const int e = live ? job_expert(ai) : -1;  // -1: no job, the loads stay past the pool's first blob
    const int slot = e < 0 || e == a.E ? 0 : uniform(s_slot[e]);
    const uint8_t *blob = e == a.E ? a.shared_blob : a.pool + uint64_t(slot < 0 ? 0 : slot) * a.expert_bytes;
    const rsrc_t gres = make_rsrc(blob + a.off_w0, uint32_t(a.N) * rbytes);
    const rsrc_t ures = make_rsrc(blob + a.off_w1, uint32_t(a.N) * rbytes);
    const rsrc_t gsres = make_rsrc(blob + a.off_s0, uint32_t(a.N) * sbytes);
    const rsrc_t usres = make_rsrc(blob + a.off_s1, uint32_t(a.N) * sbytes);
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const int row = row0 + r;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const uint32_t cb = 1024u * c + 16u * lane;
        const bool ok = live && row < a.N && cb < rbytes;
        const uint32_t wo = ok ? uint32_t(row) * rbytes + cb : kOOB;
        J.wg[r][c] = wload<WF>(gres, wo);
        J.wu[r][c] = wload<WF>(ures, wo);
        J.sg[r][c] = piece_scale<WF>(gsres, uint32_t(row) * sbytes, int(cb >> 4), ok);
        J.su[r][c] = piece_scale<WF>(usres, uint32_t(row) * sbytes, int(cb >> 4), ok);
      }
    }
    J.ts0 = J.ts1 = 1.f;
    if constexpr (WF == WF_NV4)
      if (live) {
        J.ts0 = *reinterpret_cast<const float *>(blob + a.off_t0);
        J.ts1 = *reinterpret_cast<const float *>(blob + a.off_t1);
      }
  };
  // This wave's jobs: a contiguous run of the list (consecutive rows, mostly of one expert).
  Job ring[2];
  const int gw = int(blockIdx.x) * WAVES + wave, nw = int(gridDim.x) * WAVES;
  int j = int(int64_t(n_jobs) * gw / nw);
  const int je = int(int64_t(n_jobs) * (gw + 1) / nw);
  // The other waves issue their first job as soon as its expert is known: at once for the shared
  // expert, else once wave 0's top-k has found that pick (picks are stored as they are found).
  if (wave != 0) {
    wait_job(j, je);
    issue(j, j < je, ring[0]);
  }

  if (wave == 0) {  // the routing; workgroup 0 publishes it (ids, weights, offsets, rows) for the down stage
#pragma unroll
    for (int i = 0; i < XPL; ++i)
      if (lane + 64 * i < XN) s_x[lane + 64 * i] = xg[i];
#pragma unroll
    for (int i = 0; i < SPL; ++i) {  // table_slot's reading of the words
      const int e = lane + 64 * i;
      const int sv = a.slot_of_expert != nullptr ? sl[i] : e;
      s_slot[e] = e < a.E && sv < a.n_slots ? sv : -1;
    }
    if (lane == 0) {
      if (has_shared) s_act[a.k] = a.E;
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0): s_x, s_slot landed
      __hip_atomic_store(&s_xready, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    const TokenPick pk = one_token_route(lg, a.E, a.k, a.gating, a.renorm, s_act, &s_npicks);
    if (lane < a.k) s_w[lane] = pk.w;
    if (lane == 0) {  // the routing is complete: every pick and its weight (count k + 1)
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0): s_w landed
      __hip_atomic_store(&s_npicks, a.k + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    if (blockIdx.x == 0) {
      if (lane < a.k) {
        a.ids_out[lane] = pk.id;
        a.w_out[lane] = pk.w;
        a.rows_out[pk.rank] = lane;
        a.pos_out[lane] = pk.rank;
      }
      for (int e = lane; e <= a.E; e += 64) {  // expert e's segment starts after the picks below e
        int c = 0;
        for (int i = 0; i < a.k; ++i) c += __builtin_amdgcn_readlane(pk.id, i) < e ? 1 : 0;
        a.off_out[e] = c;
      }
    }
  }
  if (wave == 0) issue(j, j < je, ring[0]);
  // this lane's activations: piece (c, v) = elements (64 c + lane) * EPC + 8 v ..
  while (__builtin_amdgcn_readfirstlane(xready()) < 1) __builtin_amdgcn_s_sleep(1);
  asm volatile("" ::: "memory");  // s_x is read after the flag
  u32x4 xv[NCH][F::XV];
#pragma unroll
  for (int c = 0; c < NCH; ++c)
#pragma unroll
    for (int v = 0; v < F::XV; ++v) xv[c][v] = s_x[(64 * c + lane) * F::XV + v];
  const rsrc_t hres_out = make_rsrc(a.out, uint32_t(n_act * a.ldo) * 2u);  // the hidden rows

  // multiply job j and write its hidden values
  auto finish = [&](int j, const Job &J) {
    const int ai = j / jobs_per_expert, row0 = (j - ai * jobs_per_expert) * RPW;
    const int e = job_expert(ai);
    const bool shared = e == a.E;
    const bool missing = !shared && uniform(s_slot[e]) < 0;
    const int p = job_row(ai);  // the token's permuted row of this expert: its rank among the picks
    // the job's 2 RPW dot products: gate rows first, then up rows, summed over the wave at once
    float v[2 * RPW];
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      Acc4 g, u;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        piece_dot<WF>(J.wg[r][c], J.sg[r][c], xv[c], g);
        piece_dot<WF>(J.wu[r][c], J.su[r][c], xv[c], u);
      }
      v[r] = g.sum();
      v[RPW + r] = u.sum();
    }
    const float tot = wave_sums<2 * RPW>(v);
    // gate total of row r sits in lanes holding value r; its up total (value RPW + r) in lane
    // l + 32 (RPW 1), l + 16 (RPW 2) or l ^ 8 (RPW 4)
    float other;
    if constexpr (RPW == 4) {
      other = dpp_f32<0x128>(tot, tot);
    } else {
      const auto sw = RPW == 2 ? __builtin_amdgcn_permlane16_swap(__float_as_uint(tot), __float_as_uint(tot), false, false)
                               : __builtin_amdgcn_permlane32_swap(__float_as_uint(tot), __float_as_uint(tot), false, false);
      other = __uint_as_float(sw[1]);
    }
    const int r = wave_sums_index<2 * RPW>(lane);
    const int row = row0 + r;
    const uint16_t hval = missing ? uint16_t(0x7fc0) : f32_to_bf16_rne(silu(tot * J.ts0) * (other * J.ts1));
    // one writer per row: the first lane of each group holding a gate total
    const bool writer = (lane & (RPW == 4 ? 15 : (RPW == 2 ? 31 : 63))) == 0 && r < RPW;
    if (writer && row < a.N) {
      if constexpr (NCHD > 0)  // read by other workgroups in this launch: stored coherent at agent scope
        __builtin_amdgcn_raw_buffer_store_b16(hval, hres_out, uint32_t(p * a.ldo + row) * 2u, 0, kCoherentAgent);
      else
        reinterpret_cast<uint16_t *>(a.out)[int64_t(p) * a.ldo + row] = hval;
    }
  };
  while (j < je) {
    wait_job(j + 1, je);
    issue(j + 1, j + 1 < je, ring[1]);
    __builtin_amdgcn_sched_barrier(0);
    finish(j, ring[0]);
    if (++j >= je) break;
    wait_job(j + 1, je);
    issue(j + 1, j + 1 < je, ring[0]);
    __builtin_amdgcn_sched_barrier(0);
    finish(j, ring[1]);
    ++j;
  }
  if constexpr (NCHD > 0) {
    // a wave may get here while wave 0 still routes (its own jobs all had early picks): the down
    // stage reads every pick and weight
    while (__builtin_amdgcn_readfirstlane(npicks()) < a.k + 1) __builtin_amdgcn_s_sleep(1);
    asm volatile("" ::: "memory");
    token_down_after_wait<WF, NCHD, RB>(*d, bar, s_act, s_w, s_slot, n_act);
  }
}

// ---------------------------------------------------------------- down + combine, one token

// Workgroup = block of RPW output rows; its 4 waves split the token's S = k
// (+1 shared) steps (wave w takes steps w, w + 4, ...; at most SPW each).  A
// wave issues every load of its steps at once -- the hidden row pieces and the
// weight pieces of its rows -- so one HBM round trip covers them; the lane sums
// w_s * (piece dot) over its steps, each row gets one wave sum, and the four
// waves' sums meet in LDS (wave 0 adds them in wave order and writes out).
template <int WF, int NCH, int RPW, int SPW>
__device__ __forceinline__ void gemv_down_combine(const PersistArgs &a) {
  using F = GemvFmt<WF>;
  __shared__ float s_part[4][RPW];
  // the wave index as a scalar: the steps, their expert blobs and buffer descriptors stay scalar
  const int tid = threadIdx.x, wave = uniform(tid >> 6), lane = tid & 63;
  const bool has_shared = a.shared_blob != nullptr;
  const int S = a.k + (has_shared ? 1 : 0);
  const int K = a.K;  // the hidden (contraction) length
  const uint32_t rbytes = WF == WF_BF16 ? uint32_t(K) * 2 : uint32_t(K) / 2;
  const uint32_t sbytes = WF == WF_FP4 ? uint32_t(K) / 32 : (WF == WF_NV4 ? uint32_t(K) / 16 : 0u);
  const rsrc_t hres = make_rsrc(a.X, uint32_t(a.x_bytes));
  const int row0 = int(blockIdx.x) * RPW;
  // the slot table, loaded with the routing below in one round trip (lane l holds experts l, l+64, ...)
  constexpr int VPL = kRouteMaxE / 64;
  int st[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = lane + 64 * i;
    st[i] = e < a.E ? table_slot(a.slot_of_expert, e, a.n_slots) : -1;
  }
  // this wave's steps: expert blob, hidden row, combine weight (scalar loads: uniform per wave)
  const uint8_t *blob[SPW];
  int kind[SPW], hrow[SPW];
  float wgt[SPW];
#pragma unroll
  for (int j = 0; j < SPW; ++j) {
    const int s = wave + 4 * j;
    kind[j] = 3;  // past the steps: no loads, no contribution
    blob[j] = a.pool;
    hrow[j] = 0;
    wgt[j] = 0.f;
    if (s < a.k) {
      const int e = a.ids[s];
      int slot = -1;
      if (e >= 0 && e < a.E) {  // expert e's entry: lane e % 64 of st[e / 64]
        int v = st[0];
#pragma unroll
        for (int i = 1; i < VPL; ++i) v = (e >> 6) == i ? st[i] : v;
        slot = __builtin_amdgcn_readlane(v, e & 63);
      }
      kind[j] = slot >= 0 ? 0 : 2;
      blob[j] = a.pool + uint64_t(slot >= 0 ? slot : 0) * a.expert_bytes;
      hrow[j] = s;  // the one-token gate/up writes hidden rows in pick order
      wgt[j] = a.topk_w[s];
    } else if (s < S) {
      kind[j] = 1;
      blob[j] = a.shared_blob;
      hrow[j] = a.T * a.k;
      wgt[j] = 1.f;
    }
  }
  // every load of this wave's steps in flight at once
  u32x4 hv[SPW][NCH][F::XV];
  u32x4 w[SPW][RPW][NCH];
  uint32_t sc[SPW][RPW][NCH];
#pragma unroll
  for (int j = 0; j < SPW; ++j) {
    const bool live = kind[j] != 3;
    const rsrc_t wres = make_rsrc(blob[j] + a.off_w0, uint32_t(a.N) * rbytes);
    const rsrc_t sres = make_rsrc(blob[j] + a.off_s0, uint32_t(a.N) * sbytes);
#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
      for (int v = 0; v < F::XV; ++v) {
        const uint32_t el = uint32_t(64 * c + lane) * F::EPC + 8u * v;
        hv[j][c][v] = bld16(hres, (live && el < uint32_t(K)) ? (uint32_t(hrow[j]) * uint32_t(a.ldx) + el) * 2u : kOOB);
      }
#pragma unroll
    for (int r = 0; r < RPW; ++r)
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const int row = row0 + r;
        const uint32_t cb = 1024u * c + 16u * lane;
        const bool ok = live && row < a.N && cb < rbytes;
        w[j][r][c] = wload<WF>(wres, ok ? uint32_t(row) * rbytes + cb : kOOB);
        sc[j][r][c] = piece_scale<WF>(sres, uint32_t(row) * sbytes, int(cb >> 4), ok);
      }
  }
  float ts[SPW];
#pragma unroll
  for (int j = 0; j < SPW; ++j) {
    ts[j] = 1.f;
    if constexpr (WF == WF_NV4)
      if (kind[j] == 0 || kind[j] == 1) ts[j] = *reinterpret_cast<const float *>(blob[j] + a.off_t0);
  }
  float acc[RPW];
#pragma unroll
  for (int r = 0; r < RPW; ++r) acc[r] = 0.f;
#pragma unroll
  for (int j = 0; j < SPW; ++j) {
    if (kind[j] == 3) continue;  // uniform per wave
    const float ws = wgt[j] * ts[j];
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      Acc4 pd;
#pragma unroll
      for (int c = 0; c < NCH; ++c) piece_dot<WF>(w[j][r][c], sc[j][r][c], hv[j][c], pd);
      acc[r] = fmaf(ws, kind[j] == 2 ? __builtin_nanf("") : pd.sum(), acc[r]);
    }
  }
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const float v = wave_sum_f32(acc[r]);
    if (lane == 0) s_part[wave][r] = v;
  }
  __syncthreads();
  if (tid < RPW) {
    const int row = row0 + tid;
    const float v = ((s_part[0][tid] + s_part[1][tid]) + s_part[2][tid]) + s_part[3][tid];
    if (row < a.N) {
      if (a.comb_bf16) reinterpret_cast<uint16_t *>(a.comb_out)[row] = f32_to_bf16_rne(v);
      else reinterpret_cast<float *>(a.comb_out)[row] = v;
    }
  }
}

}  // namespace ft
