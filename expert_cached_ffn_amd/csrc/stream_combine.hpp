// Down projection with the weighted combine folded in, for the few tokens of
// the fused layer call (at most kRouteMaxT).
//
// The combine out[t] = sum_j w[t, j] y_j + y_shared needs every expert output
// of one token; across workgroups that would take device-scope publication of
// the expert rows.  Here one unit is (token t, TR-row tile of the output) and
// walks the token's k routed experts in pick order and then the shared
// expert: each step multiplies the expert's weight tile (a.tile_rows rows,
// 16 or 8) by the token's hidden
// row, the waves' partial sums meet in LDS, and the weighted sum stays in a
// register of the thread that owns the output element; the last step writes
// it.  Steps stream through a ring of NB register sets (weights and hidden
// row of one step each), so a step's loads are in flight NB-1 steps early.
// At one token the y rows never reach memory and no combine launch follows.
#pragma once

#include "stream_persist.hpp"

namespace ft {

template <int WF, int WAVES, int KPW, int NB>
__device__ __forceinline__ void stream_combine_xs(const PersistArgs &a, float *s_red) {
  static_assert(NB >= 2, "the ring needs two register sets");
  const int TR = a.tile_rows;  // 16 or 8
  constexpr int THREADS = WAVES * 64;
  constexpr int KB = stream_kblock<WF>();
  constexpr int DX = WF == WF_FP4 ? 8 : 4;
  constexpr int MS = kRouteMaxT * (kFusedMaxK + 1);
  __shared__ uint64_t s_off[MS];  // byte offset of the step's blob in the pool (shared expert: unused)
  __shared__ int s_row[MS];       // the token's hidden row for this expert
  __shared__ int s_kind[MS];      // 0 routed and resident, 1 shared expert, 2 not resident
  __shared__ float s_w[MS];       // combine weight
  __shared__ float s_ts[MS];      // NVFP4: the down matrix's tensor scale
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = lane & 15, q = lane >> 4;
  const bool has_shared = a.shared_blob != nullptr;
  const int S = a.k + (has_shared ? 1 : 0);

  // ---- the steps of every token: expert blob, hidden row, weight
  for (int i = tid; i < a.T * S; i += THREADS) {
    const int t = i / S, s = i - t * S;
    int kind = 1, row = a.T * a.k + t;
    float w = 1.f, ts = 1.f;
    uint64_t off = 0;
    if (s < a.k) {
      const int e = a.ids[t * a.k + s];
      const int slot = (e >= 0 && e < a.E) ? table_slot(a.slot_of_expert, e, a.n_slots) : -1;
      kind = slot >= 0 ? 0 : 2;
      off = slot >= 0 ? uint64_t(slot) * a.expert_bytes : 0;
      row = a.row_pos[t * a.k + s];
      w = a.topk_w[t * a.k + s];
    }
    if constexpr (WF == WF_NV4)
      if (kind != 2) ts = *reinterpret_cast<const float *>((kind == 1 ? a.shared_blob : a.pool + off) + a.off_t0);
    s_off[i] = off;
    s_row[i] = row;
    s_kind[i] = kind;
    s_w[i] = w;
    s_ts[i] = ts;
  }
  __syncthreads();

  // ---- this workgroup's run of units (token-major), S steps each
  const int n_units = a.T * a.n_tiles;
  const int u_begin = int(int64_t(n_units) * blockIdx.x / gridDim.x);
  const int u_end = int(int64_t(n_units) * (blockIdx.x + 1) / gridDim.x);
  const int i_begin = u_begin * S, i_end = u_end * S;

  const uint32_t wpitch = (WF == WF_BF16) ? uint32_t(a.K) * 2 : uint32_t(a.K) / 2;
  const uint32_t spitch = uint32_t(a.K) / (WF == WF_NV4 ? 16 : 32);
  const uint32_t wbytes = uint32_t(a.N) * wpitch, sbytes = uint32_t(a.N) * spitch;
  const rsrc_t xres = make_rsrc(a.X, a.x_bytes);

  struct StepRegs {
    WFrag<WF, 1> f[KPW];
    u32x4 xb[KPW][DX];
  };

  // Loads of step i (i >= i_end: offsets past every buffer, so each ring step
  // issues the same number of loads).
  auto issue = [&](int i, StepRegs &R) {
    const bool live = i < i_end;
    const int ic = live ? i : i_begin;
    const int u = ic / S, s = ic - u * S;
    const int t = u / a.n_tiles, tile = u - t * a.n_tiles;
    const int m = uniform(t * S + s);
    const int kind = uniform(s_kind[m]);
    // the blob offset as two scalar words; readfirstlane returns int, so each word goes back to
    // unsigned before the 64-bit sum (a signed low word would point below the pool past 2 GiB)
    const uint64_t off = s_off[m];
    const uint32_t lo = uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(off))));
    const uint32_t hi = uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(off >> 32))));
    const uint8_t *blob = kind == 1 ? a.shared_blob : a.pool + ((uint64_t(hi) << 32) | uint64_t(lo));
    const rsrc_t wres = make_rsrc(blob + a.off_w0, wbytes);
    const rsrc_t sres = make_rsrc(blob + a.off_s0, sbytes);
    // rows past N fall outside the buffer; so do operand rows past TR
    constexpr int NH = wl_halves<WF>();
    uint32_t wo[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      const int rr = wl_row<WF>(lane, h);
      wo[h] = live && rr < TR ? uint32_t(tile * TR + rr) * wpitch + wl_byte<WF>(lane, h) : kOOB;
    }
    const uint32_t so = live && r < TR ? uint32_t(tile * TR + r) * spitch : kOOB;
    const int hrow = uniform(s_row[m]);
    const uint32_t xo = (live && r == 0) ? uint32_t(hrow) * uint32_t(a.ldx) * 2u : kOOB;  // one token column
#pragma unroll
    for (int c = 0; c < KPW; ++c) {
      const int kb = wave + c * WAVES;
#pragma unroll
      for (int d = 0; d < WFrag<WF, 1>::DL; ++d)
        R.f[c].w[0][d] = wl_load<WF>(wres, wo[d % NH] + uint32_t(kb) * wl_kbytes<WF>() + wl_dcol<WF>(d));
      if constexpr (WF != WF_BF16) R.f[c].s[0] = bld8(sres, so + uint32_t(kb) * 8);
#pragma unroll
      for (int dx = 0; dx < DX; ++dx) {
        R.xb[c][dx] = bld16(xres, xo + uint32_t(kb * KB + wl_xk<WF>(dx, q)) * 2u);
      }
    }
  };

  float oacc = 0.f;  // the weighted sum of the element this thread owns (tid < 256, token column 0)
  // Multiply step i, sum the wave partials, fold w * y into the running sum; the last step of a unit
  // writes the unit's output rows.
  auto finish = [&](int i, const StepRegs &R) {
    const int u = i / S, s = i - u * S;
    const int t = u / a.n_tiles, tile = u - t * a.n_tiles;
    const int m = t * S + s;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < KPW; ++c) {
      WFrag<WF, 1> fc = R.f[c];
      wfrag_fix(fc);
      if constexpr (WF == WF_BF16) {
#pragma unroll
        for (int d = 0; d < 4; ++d) acc = mfma16(as_bf16x8(fc.w[0][d]), as_bf16x8(R.xb[c][d]), acc);
      } else if constexpr (WF == WF_FP4) {
#pragma unroll
        for (int d = 0; d < 2; ++d) {
          const float sc = e8m0_to_f32(wl_mx_scale<WF>(fc.s[0], d, q));
#pragma unroll
          for (int mm = 0; mm < 4; ++mm) acc = mfma16(fp4x8_to_bf16x8(fc.w[0][d][mm], sc), as_bf16x8(R.xb[c][4 * d + mm]), acc);
        }
      } else {
#pragma unroll
        for (int mm = 0; mm < 4; ++mm) {
          const uint32_t sw = (q >> 1) ? R.f[c].s[0][1] : R.f[c].s[0][0];
          const float sc = e4m3_to_f32(sw >> (8 * ((2 * q + (mm >> 1)) & 3)));
          acc = mfma16(nvfp4x8_to_bf16x8(R.f[c].w[0][0][mm], sc), as_bf16x8(R.xb[c][mm]), acc);
        }
      }
    }
    *reinterpret_cast<f32x4 *>(&s_red[(wave * 64 + lane) * 4]) = acc;
    __syncthreads();
    if (tid < 256) {
      const int ln = tid >> 2, v = tid & 3;
      if ((ln & 15) == 0) {  // token column 0
        float y = 0.f;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) y += s_red[(w * 64 + ln) * 4 + v];
        const int kind = s_kind[m];
        if constexpr (WF == WF_NV4) y *= s_ts[m];
        if (kind == 2) y = __builtin_nanf("");
        oacc = s == 0 ? s_w[m] * y : oacc + s_w[m] * y;
        const int nr = 4 * (ln >> 4) + v, n = tile * TR + nr;
        if (s == S - 1 && nr < TR && n < a.N) {
          if (a.comb_bf16)
            reinterpret_cast<uint16_t *>(a.comb_out)[int64_t(t) * a.ldo + n] = f32_to_bf16_rne(oacc);
          else
            reinterpret_cast<float *>(a.comb_out)[int64_t(t) * a.ldo + n] = oacc;
        }
      }
    }
    __syncthreads();
  };

  StepRegs ring[NB];
#pragma unroll
  for (int s = 0; s < NB - 1; ++s) issue(i_begin + s, ring[s]);
  for (int i = i_begin; i < i_end; i += NB) {
#pragma unroll
    for (int s = 0; s < NB; ++s) {
      issue(i + s + NB - 1, ring[(s + NB - 1) % NB]);
      __builtin_amdgcn_sched_barrier(0);
      if (i + s < i_end) finish(i + s, ring[s]);
    }
  }
}

}  // namespace ft
