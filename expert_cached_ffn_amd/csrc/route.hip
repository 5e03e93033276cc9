// ft_moe_route: router logits (optional), top-k selection and gating weights.
//
// A router activates a small subset of the experts for each token (FreeToken
// linux page, "Cómo gestiona FreeToken la memoria MoE": 6 of 256 routed
// experts per layer in the pages' example).  Selection order and gating are
// the textbook forms: descending logit with the lower expert index first on
// ties; softmax over all E or element-wise sigmoid, optionally renormalised
// over the k picked.
#include <math.h>

#include "ft_internal.hpp"
#include "permute_util.hpp"
#include "topk_util.hpp"
#include "stream_gemm.hpp"

namespace ft {

// ------------------------------------------------------------------ logits

// bf16: logits[t, e] = sum_h x[t, h] W_r[e, h] on MFMA; one workgroup per
// (16 experts, 16*NTMAX tokens), its waves splitting the hidden axis.
template <int NTMAX, int WAVES, bool PIPE>
__global__ __launch_bounds__(WAVES * 64) void router_logits_bf16(const uint16_t *__restrict__ x,
                                                                 const uint8_t *__restrict__ wr,
                                                                 float *__restrict__ logits, int T, int H, int E) {
  constexpr int GROUP = 16 * NTMAX;
  __shared__ int s_tok[GROUP];
  __shared__ float s_red[stream_red_floats<false, NTMAX, WAVES>()];
  const int tile = blockIdx.x, g0 = blockIdx.y * GROUP;
  const int mm = min(GROUP, T - g0);
  if (threadIdx.x < mm) s_tok[threadIdx.x] = g0 + threadIdx.x;
  __syncthreads();
  stream_tile_any<WF_BF16, false, NTMAX, WAVES, PIPE>(wr, wr, wr, wr, H, tile * 16, E, x, H,
                                                      uint32_t(uint64_t(T) * H * 2), s_tok, mm, s_red, logits, E,
                                                      s_tok);
}

// bf16, a few tokens (T <= TT <= 4): one single-wave workgroup per expert,
// so the router weights stream through E compute units instead of the E/16
// workgroups of the MFMA tile.  Lane l dots the 8-element pieces l, l+64, ...
// of the expert's row with the tokens' rows (v_dot2: pairs of bf16 products
// added into an fp32 sum), every piece of a 4096-element pass loaded before
// the first product, then one wave sum per token.
template <int TT>
__global__ __launch_bounds__(64) void router_logits_gemv_bf16(const uint16_t *__restrict__ x,
                                                             const uint16_t *__restrict__ wr,
                                                             float *__restrict__ logits, int T, int H, int E) {
  constexpr int NP = 8;  // 16-byte pieces per lane per pass: 4096 elements of the row, all loads in flight
  const int e = blockIdx.x, lane = threadIdx.x;
  // raw buffer loads: a piece past the row (or a token past T) reads zero without a branch
  const rsrc_t wres = make_rsrc(wr + int64_t(e) * H, uint32_t(H) * 2u);
  const rsrc_t xres = make_rsrc(x, uint32_t(T) * uint32_t(H) * 2u);
  float acc[TT];
#pragma unroll
  for (int t = 0; t < TT; ++t) acc[t] = 0.f;
  for (int h0 = 0; h0 < H; h0 += NP * 512) {
    u32x4 wv[NP], xv[TT][NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const uint32_t h = uint32_t(h0 + 512 * p + 8 * lane);
      wv[p] = bld16(wres, h < uint32_t(H) ? h * 2u : kOOB);
#pragma unroll
      for (int t = 0; t < TT; ++t)
        xv[t][p] = bld16(xres, (t < T && h < uint32_t(H)) ? (uint32_t(t) * uint32_t(H) + h) * 2u : kOOB);
    }
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int t = 0; t < TT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc[t] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(wv[p][i]), as_bf16x2(xv[t][p][i]), acc[t], false);
  }
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    const float v = wave_sum_f32(acc[t]);
    if (t < T && lane == 0) logits[int64_t(t) * E + e] = v;
  }
}

// bf16, split over the hidden axis (decode batches of 5+ tokens in the layer call): workgroup
// (expert tile, token tile, part p) multiplies k-blocks p*kpp .. p*kpp + kpp - 1 of its 16 experts x
// 16 tokens, its waves taking the k-blocks in turn, and writes the partial tile to part[p][t][e];
// the routing tail adds the parts in p order (no atomics, a fixed order).  The unsplit tile kernel
// streams its 16 experts' whole rows through one compute unit per tile: 32 workgroups at 64 tokens
// and 128 experts (a 128 KiB share each), 8 at 16 tokens.
constexpr int kSplitWaves = 4;

__global__ __launch_bounds__(kSplitWaves * 64) void router_logits_split_bf16(const uint16_t *__restrict__ x,
                                                                            const uint16_t *__restrict__ wr,
                                                                            float *__restrict__ part, int T,
                                                                            int H, int E, int kpp) {
  __shared__ f32x4 s_red[kSplitWaves][64];
  const int et = blockIdx.x, tt = blockIdx.y, p = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, r = lane & 15, q = lane >> 4;
  // rows past E and tokens past T get an out-of-range offset: zeros, no traffic
  const rsrc_t wres = make_rsrc(wr, uint32_t(E) * uint32_t(H) * 2u);
  const rsrc_t xres = make_rsrc(x, uint32_t(T) * uint32_t(H) * 2u);
  const int e = et * 16 + r, t = tt * 16 + r;
  const uint32_t wo = e < E ? uint32_t(e) * uint32_t(H) * 2u : kOOB;
  const uint32_t xo = t < T ? uint32_t(t) * uint32_t(H) * 2u : kOOB;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int kb = p * kpp + wave; kb < (p + 1) * kpp; kb += kSplitWaves) {
    // lane (r, q) holds elements 32d + 8q .. +7 of the k-block for MFMA d (A: expert rows, B: tokens)
    u32x4 wa[4], xb[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t off = uint32_t(kb * 128 + 32 * d + 8 * q) * 2u;
      wa[d] = bld16(wres, wo + off);
      xb[d] = bld16(xres, xo + off);
    }
#pragma unroll
    for (int d = 0; d < 4; ++d) acc = mfma16(as_bf16x8(wa[d]), as_bf16x8(xb[d]), acc);
  }
  s_red[wave][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    f32x4 sum = s_red[0][lane];
#pragma unroll
    for (int w = 1; w < kSplitWaves; ++w) sum += s_red[w][lane];  // wave order
    // lane holds D[4q + v][r]: expert et*16 + 4q + v, token tt*16 + r
    const int tok = tt * 16 + r;
    if (tok < T) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int ee = et * 16 + 4 * q + v;
        if (ee < E) part[(int64_t(p) * T + tok) * E + ee] = sum[v];
      }
    }
  }
}

// fp32: one thread per (token, expert).
__global__ __launch_bounds__(256) void router_logits_f32(const float *__restrict__ x,
                                                         const float *__restrict__ wr,
                                                         float *__restrict__ logits, int T, int H, int E) {
  const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= int64_t(T) * E) return;
  const int t = int(idx / E), e = int(idx % E);
  const float *xr = x + int64_t(t) * H, *w = wr + int64_t(e) * H;
  float s = 0.f;
  for (int c = 0; c < H; ++c) s = fmaf(xr[c], w[c], s);
  logits[idx] = s;
}

// ------------------------------------------------------------------ top-k

constexpr int kTopkWaves = 4;

template <int VPL>
__global__ __launch_bounds__(64 * kTopkWaves) void topk_gating_kernel(const float *__restrict__ logits,
                                                                       int T, int E, int k, int gating,
                                                                       int renorm, int32_t *__restrict__ ids,
                                                                       float *__restrict__ w) {
  const int t = blockIdx.x * kTopkWaves + (threadIdx.x >> 6);
  if (t < T) topk_token<VPL>(logits, t, E, k, gating, renorm, ids, w, nullptr);
}

// ------------------------------------------------------------------ fused decode routing

constexpr int kFusedMaxT = 16;      // tokens of the fused path (one workgroup: at 64 tokens its top-k,
                                     // VALU-bound on one CU, took 16 us against 4.7 us over 16 CUs)
constexpr int kFusedMaxRows = 2048; // routed rows (T * k) of the fused path

struct FusedRouteArgs {
  const float *logits;       // [T, E]
  int T, E, k, gating, renorm;
  int32_t *ids;
  float *w;
  int32_t *offsets, *sorted_rows, *row_pos;
  // non-NULL: the logits are the sum of nparts (2, 4, 8 or 16) partial planes parts[p][T][E], added in
  // p order by the token's wave, which also writes the sums to logits_out
  const float *parts;
  int nparts;
  float *logits_out;
};

// Token t's logits as the sum of NP partial planes: every load in flight before the first add.
template <int VPL, int NP>
__device__ __forceinline__ void sum_parts(const FusedRouteArgs &a, int t, float (&v)[VPL]) {
  const int lane = threadIdx.x & 63;
  float pv[NP][VPL];
#pragma unroll
  for (int p = 0; p < NP; ++p)
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int e = lane + 64 * i;
      pv[p][i] = a.parts[(int64_t(p) * a.T + t) * a.E + (e < a.E ? e : 0)];
    }
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    float sum = pv[0][i];
#pragma unroll
    for (int p = 1; p < NP; ++p) sum += pv[p][i];
    const int e = lane + 64 * i;
    if (e < a.E) a.logits_out[int64_t(t) * a.E + e] = sum;
    v[i] = sum;
  }
}

// Top-k and gating of token t (one wave), from the logits or from their partial sums.
template <int VPL>
__device__ __forceinline__ void route_token(const FusedRouteArgs &a, int t, int32_t *ids, float *w, int32_t *ids_lds) {
  // (the split router covers E <= 256: four logits per lane at most)
  if (VPL > 4 || a.parts == nullptr) {
    topk_token<VPL>(a.logits, t, a.E, a.k, a.gating, a.renorm, ids, w, ids_lds);
    return;
  }
  float v[1][VPL];
  if constexpr (VPL <= 4) {
    switch (a.nparts) {
      case 2: sum_parts<VPL, 2>(a, t, v[0]); break;
      case 4: sum_parts<VPL, 4>(a, t, v[0]); break;
      case 8: sum_parts<VPL, 8>(a, t, v[0]); break;
      default: sum_parts<VPL, 16>(a, t, v[0]); break;
    }
  }
  const int tt[1] = {t};
  topk_values<VPL, 1>(v, tt, 1, a.E, a.k, a.gating, a.renorm, ids, w, ids_lds);
}

// Top-k, gating and the permutation of all T tokens by one workgroup.
template <int VPL>
__device__ __forceinline__ void route_tail(const FusedRouteArgs &a, int32_t *s_ids, int *s_cnt, int *s_cc,
                                           int *s_tmp) {
  const int wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  for (int t = wave; t < a.T; t += nw) route_token<VPL>(a, t, a.ids, a.w, s_ids);
  __syncthreads();
  const int R = a.T * a.k;
  if (R <= 64) {
    if (wave == 0) permute_wave64(s_ids, R, a.E, s_cnt, a.offsets, a.sorted_rows, a.row_pos);
  } else if (R <= kChunkPermMaxRows && a.E <= kChunkPermMaxE && R <= 64 * nw) {
    permute_chunks(s_ids, R, a.E, s_cc, s_cnt, s_tmp, a.offsets, a.sorted_rows, a.row_pos);
  } else {
    permute_block(s_ids, R, a.E, s_cnt, s_tmp, a.offsets, a.sorted_rows, a.row_pos);
  }
}

// Top-k, gating and permutation of all T tokens in one workgroup (small
// decode batches, T <= 16): one launch after the router instead of two.  Up to
// 64 routed rows the workgroup is one wave per token and wave 0 sorts the rows
// alone (no block-wide histogram, scan and barriers); above that the rows are
// sorted chunk-parallel.  (A single
// launch with the router, its last workgroup doing this, was measured
// slower: the device-scope fences that publish the logits write back and
// invalidate the L2 of every XCD.)
template <int VPL>
__global__ __launch_bounds__(1024) void route_tail_kernel(FusedRouteArgs a) {
  __shared__ int32_t s_ids[kFusedMaxRows];
  __shared__ int s_cnt[kMaxE];
  __shared__ int s_cc[kChunkPermMaxRows / 64 * kChunkPermMaxE];
  __shared__ int s_tmp[32];
  route_tail<VPL>(a, s_ids, s_cnt, s_cc, s_tmp);
}

// Top-k and gating over the grid, one token per wave, then the permutation by the workgroup that
// finishes last (decode batches past the one-workgroup tail: that tail's top-k is VALU-bound on one
// CU).  Each workgroup writes its tokens' ids through to the device-coherent level (sc1: the dies'
// L2s are not coherent with each other), waits for those stores, and counts itself done on a zeroed
// counter; the workgroup whose count is the last reads every id back the same way, sorts the rows
// chunk-parallel (R <= 64 * NW) and clears the counter.  One launch instead of two.
constexpr int kCoherent = 16;  // buffer cache policy: sc1 (agent scope)

template <int VPL, int NW>
__global__ __launch_bounds__(64 * NW) void topk_permute_kernel(FusedRouteArgs a, uint32_t *done) {
  __shared__ int32_t s_ids[64 * NW];  // the rows' ids at their flat index t * k + j (R <= 64 * NW)
  __shared__ int s_cc[NW * kChunkPermMaxE];
  __shared__ int s_seg[kChunkPermMaxE];
  __shared__ int s_tmp[32];
  __shared__ int s_last;
  const int tid = threadIdx.x, wave = tid >> 6;
  const int t0 = int(blockIdx.x) * NW, nt = min(NW, a.T - t0);
  const int R = a.T * a.k;
  if (wave < nt) route_token<VPL>(a, t0 + wave, nullptr, a.w, s_ids);
  __syncthreads();
  const rsrc_t ids = make_rsrc(a.ids, uint32_t(R) * 4u);
  for (int p = t0 * a.k + tid; p < (t0 + nt) * a.k; p += 64 * NW)
    __builtin_amdgcn_raw_buffer_store_b32(s_ids[p], ids, uint32_t(p) * 4u, 0, kCoherent);
  wait_vmcnt<0>();
  __syncthreads();
  if (tid == 0)
    s_last = __hip_atomic_fetch_add(done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == gridDim.x - 1;
  __syncthreads();
  if (!s_last) return;
  for (int p = tid; p < R; p += 64 * NW) s_ids[p] = int32_t(__builtin_amdgcn_raw_buffer_load_b32(ids, uint32_t(p) * 4u, 0, kCoherent));
  __syncthreads();
  permute_chunks(s_ids, R, a.E, s_cc, s_seg, s_tmp, a.offsets, a.sorted_rows, a.row_pos);
  if (tid == 0) __hip_atomic_store(done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Parts of the split router for a layer call (0: not split).  Up to 4 tokens the one-wave-per-expert
// router serves; the split needs bf16 tokens, H a multiple of 128, a routing tail that covers the
// batch and room for the partial planes in the workspace.
int router_split_parts(const void *x, int32_t x_dtype, const void *w_router, int T, int H, int E, int k,
                       size_t ws_bytes) {
  if (w_router == nullptr || x == nullptr || x_dtype != FT_BF16 || T <= 4 || H % 128 != 0 || E > kMaxE || k > E ||
      int64_t(T) * k > kChunkPermMaxRows || E > kChunkPermMaxE)
    return 0;
  if (!(T <= kFusedMaxT && int64_t(T) * k <= kFusedMaxRows) && !route_permute_counted_covers(T, k, E)) return 0;
  // parts: the fewest that give 128 workgroups (one per 2 CUs), a power of two dividing the k-blocks
  const int nkb = H / 128, base = cdiv(E, 16) * cdiv(T, 16);
  int P = 1;
  while (P < 16 && P < nkb && base * P < 128 && nkb % (2 * P) == 0) P *= 2;
  if (P == 1 || size_t(P) * size_t(T) * size_t(E) * 4u > ws_bytes) return 0;
  return P;
}

// The split router (partial planes in ws), then top-k, gating and the permutation in one launch: the
// one-workgroup tail up to 16 tokens, the grid-wide top-k with the counted sort past that.
ft_status route_permute_split(const void *x, const void *w_router, float *logits, int32_t T, int32_t H, int32_t E,
                              int32_t k, int32_t gating, int32_t renormalize, int32_t *topk_ids, float *topk_w,
                              int32_t *expert_offsets, int32_t *sorted_rows, int32_t *row_pos, int parts, void *ws,
                              uint32_t *done, hipStream_t stream) {
  const ft_status st = route_logits(x, FT_BF16, w_router, logits, T, H, E, k, gating, topk_ids, topk_w, stream, false);
  if (st != FT_OK) return st;
  float *part = static_cast<float *>(ws);
  const int nkb = H / 128;
  hipLaunchKernelGGL(router_logits_split_bf16, dim3(unsigned(cdiv(E, 16)), unsigned(cdiv(T, 16)), unsigned(parts)),
                     dim3(kSplitWaves * 64), 0, stream, static_cast<const uint16_t *>(x),
                     static_cast<const uint16_t *>(w_router), part, T, H, E, nkb / parts);
  FT_LAUNCHED("router_logits_split_bf16");
  FusedRouteArgs a{};
  a.logits = logits;
  a.T = T;
  a.E = E;
  a.k = k;
  a.gating = gating;
  a.renorm = renormalize ? 1 : 0;
  a.ids = topk_ids;
  a.w = topk_w;
  a.offsets = expert_offsets;
  a.sorted_rows = sorted_rows;
  a.row_pos = row_pos;
  a.parts = part;
  a.nparts = parts;
  a.logits_out = logits;
  const int R = T * k, vpl = cdiv(E, 64);
  if (T <= kFusedMaxT && R <= kFusedMaxRows) {
    const dim3 blk(R <= 64 ? 64 * T : 1024);
    if (vpl <= 2) hipLaunchKernelGGL(route_tail_kernel<2>, dim3(1), blk, 0, stream, a);
    else if (vpl <= 4) hipLaunchKernelGGL(route_tail_kernel<4>, dim3(1), blk, 0, stream, a);
    else hipLaunchKernelGGL(route_tail_kernel<16>, dim3(1), blk, 0, stream, a);
    FT_LAUNCHED("route_tail_kernel");
  } else {
#define FT_TOPK_PERM(V, NW) \
  hipLaunchKernelGGL((topk_permute_kernel<V, NW>), dim3(unsigned(cdiv(T, NW))), dim3(64 * NW), 0, stream, a, done)
    if (R <= 512) {
      if (vpl <= 2) FT_TOPK_PERM(2, 8);
      else FT_TOPK_PERM(4, 8);
    } else {
      if (vpl <= 2) FT_TOPK_PERM(2, 16);
      else FT_TOPK_PERM(4, 16);
    }
#undef FT_TOPK_PERM
    FT_LAUNCHED("topk_permute_kernel");
  }
  clear_error();
  return FT_OK;
}

bool route_permute_counted_covers(int T, int k, int E) {
  return T > kFusedMaxT && int64_t(T) * k <= kChunkPermMaxRows && E <= kChunkPermMaxE && k <= E;
}

ft_status route_permute_counted(const void *x, int32_t x_dtype, const void *w_router, float *logits, int32_t T,
                                int32_t H, int32_t E, int32_t k, int32_t gating, int32_t renormalize,
                                int32_t *topk_ids, float *topk_w, int32_t *expert_offsets, int32_t *sorted_rows,
                                int32_t *row_pos, uint32_t *done, hipStream_t stream) {
  const ft_status st = route_logits(x, x_dtype, w_router, logits, T, H, E, k, gating, topk_ids, topk_w, stream);
  if (st != FT_OK) return st;
  FusedRouteArgs a{};
  a.logits = logits;
  a.T = T;
  a.E = E;
  a.k = k;
  a.gating = gating;
  a.renorm = renormalize ? 1 : 0;
  a.ids = topk_ids;
  a.w = topk_w;
  a.offsets = expert_offsets;
  a.sorted_rows = sorted_rows;
  a.row_pos = row_pos;
  const int R = T * k, vpl = cdiv(E, 64);
#define FT_TOPK_PERM(V, NW) \
  hipLaunchKernelGGL((topk_permute_kernel<V, NW>), dim3(unsigned(cdiv(T, NW))), dim3(64 * NW), 0, stream, a, done)
  if (R <= 512) {
    if (vpl <= 2) FT_TOPK_PERM(2, 8);
    else FT_TOPK_PERM(4, 8);
  } else {
    if (vpl <= 2) FT_TOPK_PERM(2, 16);
    else FT_TOPK_PERM(4, 16);
  }
#undef FT_TOPK_PERM
  FT_LAUNCHED("topk_permute_kernel");
  clear_error();
  return FT_OK;
}

}  // namespace ft

using namespace ft;

// Checks the arguments of a routing call and launches the router logits
// kernel when there is a router (FT_OK with nothing launched when T == 0).
ft_status ft::route_logits(const void *x, int32_t x_dtype, const void *w_router, float *logits, int32_t T,
                              int32_t H, int32_t E, int32_t k, int32_t gating, int32_t *topk_ids, float *topk_w,
                              hipStream_t stream, bool launch) {
  FT_REQUIRE(T >= 0 && E >= 1 && k >= 1, "ft_moe_route: need T >= 0, E >= 1, k >= 1");
  FT_SUPPORTED(k <= E, "ft_moe_route: k > E");
  FT_SUPPORTED(E <= kMaxE, "ft_moe_route: E > 1024");
  FT_SUPPORTED(k <= kMaxK, "ft_moe_route: k > 256");
  FT_REQUIRE(gating == FT_SOFTMAX || gating == FT_SIGMOID, "ft_moe_route: unknown gating");
  FT_REQUIRE(int64_t(T) * E < (int64_t(1) << 31), "ft_moe_route: T*E too large");
  if (w_router != nullptr) {
    FT_REQUIRE(H >= 1, "ft_moe_route: H must be positive");
    FT_REQUIRE(x_dtype == FT_F32 || x_dtype == FT_BF16, "ft_moe_route: x_dtype must be FT_F32 or FT_BF16");
    if (x_dtype == FT_BF16) {
      FT_SUPPORTED(H % 128 == 0, "ft_moe_route: bf16 router needs H multiple of 128");
      FT_SUPPORTED(int64_t(T) * H * 2 < (int64_t(1) << 31) && int64_t(E) * H * 2 < (int64_t(1) << 31),
                   "ft_moe_route: x or w_router above 2 GiB");
    }
  }
  if (T == 0) {
    clear_error();
    return FT_OK;
  }
  FT_REQUIRE(logits && topk_ids && topk_w, "ft_moe_route: NULL logits / topk_ids / topk_w");
  FT_REQUIRE(aligned(logits, 16) && aligned(topk_ids, 4) && aligned(topk_w, 4),
             "ft_moe_route: misaligned output buffer");
  if (w_router != nullptr) {
    FT_REQUIRE(x != nullptr, "ft_moe_route: x is NULL");
    FT_REQUIRE(aligned(x, 16) && aligned(w_router, 16), "ft_moe_route: x / w_router must be 16-byte aligned");
    if (!launch) return FT_OK;
    if (x_dtype == FT_BF16) {
      const uint16_t *xb = static_cast<const uint16_t *>(x);
      const uint8_t *wb = static_cast<const uint8_t *>(w_router);
      // One wave per expert for a few tokens (one-token decode, 256 x 4096 router: 3.2 us against
      // 5.1 us for the MFMA tile).
      if (T <= 4) {
        const uint16_t *wh = static_cast<const uint16_t *>(w_router);
        if (T == 1)
          hipLaunchKernelGGL(router_logits_gemv_bf16<1>, dim3(unsigned(E)), dim3(64), 0, stream, xb, wh, logits, T, H, E);
        else if (T == 2)
          hipLaunchKernelGGL(router_logits_gemv_bf16<2>, dim3(unsigned(E)), dim3(64), 0, stream, xb, wh, logits, T, H, E);
        else
          hipLaunchKernelGGL(router_logits_gemv_bf16<4>, dim3(unsigned(E)), dim3(64), 0, stream, xb, wh, logits, T, H, E);
        FT_LAUNCHED("router_logits_gemv_bf16");
        return FT_OK;
      }
      // all the waves of a workgroup split the hidden axis; 16 tokens per workgroup
      const dim3 g1(unsigned(cdiv(E, 16)), unsigned(cdiv(T, 16)));
      const StreamShape sh = stream_shape(1, H / stream_kblock<WF_BF16>());
#define FT_ROUTER(W, P)                                                                                  \
  if (sh.waves == W && sh.pipe == P)                                                                     \
    hipLaunchKernelGGL((router_logits_bf16<1, W, P>), g1, dim3(W * 64), 0, stream, xb, wb, logits, T, H, E);
      FT_ROUTER(16, false)
      FT_ROUTER(16, true)
      FT_ROUTER(8, false)
      FT_ROUTER(8, true)
      FT_ROUTER(6, false)
      FT_ROUTER(6, true)
      FT_ROUTER(4, false)
      FT_ROUTER(4, true)
#undef FT_ROUTER
      FT_LAUNCHED("router_logits_bf16");
    } else {
      const int64_t n = int64_t(T) * E;
      hipLaunchKernelGGL(router_logits_f32, dim3(unsigned(cdiv<int64_t>(n, 256))), dim3(256), 0, stream,
                         static_cast<const float *>(x), static_cast<const float *>(w_router), logits, T, H,
                         E);
      FT_LAUNCHED("router_logits_f32");
    }
  }
  return FT_OK;
}

extern "C" ft_status ft_moe_route(const void *x, int32_t x_dtype, const void *w_router, float *logits,
                                  int32_t T, int32_t H, int32_t E, int32_t k, int32_t gating,
                                  int32_t renormalize, int32_t *topk_ids, float *topk_w,
                                  hipStream_t stream) {
  const ft_status st = route_logits(x, x_dtype, w_router, logits, T, H, E, k, gating, topk_ids, topk_w, stream);
  if (st != FT_OK) return st;
  if (T == 0) {
    clear_error();
    return FT_OK;
  }
  const dim3 grid(unsigned(cdiv(T, kTopkWaves))), blk(64 * kTopkWaves);
  const int vpl = cdiv(E, 64);
#define FT_TOPK(V)                                                                                     \
  hipLaunchKernelGGL(topk_gating_kernel<V>, grid, blk, 0, stream, logits, T, E, k, gating, renormalize, \
                     topk_ids, topk_w)
  if (vpl <= 1) FT_TOPK(1);
  else if (vpl <= 2) FT_TOPK(2);
  else if (vpl <= 4) FT_TOPK(4);
  else if (vpl <= 8) FT_TOPK(8);
  else FT_TOPK(16);
#undef FT_TOPK
  FT_LAUNCHED("topk_gating_kernel");
  clear_error();
  return FT_OK;
}

extern "C" ft_status ft_moe_route_permute(const void *x, int32_t x_dtype, const void *w_router, float *logits,
                                          int32_t T, int32_t H, int32_t E, int32_t k, int32_t gating,
                                          int32_t renormalize, int32_t *topk_ids, float *topk_w,
                                          int32_t *expert_offsets, int32_t *sorted_rows, int32_t *row_pos,
                                          void *workspace, size_t workspace_bytes, hipStream_t stream) {
  const bool fused = T >= 1 && T <= kFusedMaxT && int64_t(T) * k <= kFusedMaxRows && k >= 1 && k <= E &&
                     E <= kMaxE && (gating == FT_SOFTMAX || gating == FT_SIGMOID);
  if (!fused) {
    // the two calls, one after the other (they validate their own arguments)
    const ft_status st = ft_moe_route(x, x_dtype, w_router, logits, T, H, E, k, gating, renormalize, topk_ids,
                                      topk_w, stream);
    if (st != FT_OK) return st;
    return ft_moe_permute(topk_ids, T, k, E, expert_offsets, sorted_rows, row_pos, workspace, workspace_bytes,
                          stream);
  }
  FT_REQUIRE(expert_offsets && sorted_rows && row_pos && aligned(expert_offsets, 4) && aligned(sorted_rows, 4) &&
                 aligned(row_pos, 4),
             "ft_moe_route_permute: NULL or misaligned permutation output");
  // validation of the routing arguments and the router logits (if any); the tail replaces the top-k kernel
  const ft_status st = route_logits(x, x_dtype, w_router, logits, T, H, E, k, gating, topk_ids, topk_w, stream);
  if (st != FT_OK) return st;
  FusedRouteArgs a{};
  a.logits = logits;
  a.T = T;
  a.E = E;
  a.k = k;
  a.gating = gating;
  a.renorm = renormalize ? 1 : 0;
  a.ids = topk_ids;
  a.w = topk_w;
  a.offsets = expert_offsets;
  a.sorted_rows = sorted_rows;
  a.row_pos = row_pos;
  const int vpl = cdiv(E, 64);
  // up to 64 routed rows one wave sorts them: one wave per token is enough; above that 16 waves
  const dim3 blk(T * k <= 64 ? 64 * T : 1024);
  if (vpl <= 2) hipLaunchKernelGGL(route_tail_kernel<2>, dim3(1), blk, 0, stream, a);
  else if (vpl <= 4) hipLaunchKernelGGL(route_tail_kernel<4>, dim3(1), blk, 0, stream, a);
  else hipLaunchKernelGGL(route_tail_kernel<16>, dim3(1), blk, 0, stream, a);
  FT_LAUNCHED("route_tail_kernel");
  clear_error();
  return FT_OK;
}
