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
// of the expert's row with the tokens' rows (fp32 fused multiply-adds), then
// one wave sum per token.
template <int TT>
__global__ __launch_bounds__(64) void router_logits_gemv_bf16(const uint16_t *__restrict__ x,
                                                             const uint16_t *__restrict__ wr,
                                                             float *__restrict__ logits, int T, int H, int E) {
  const int e = blockIdx.x, lane = threadIdx.x;
  const uint16_t *w = wr + int64_t(e) * H;
  float acc[TT];
#pragma unroll
  for (int t = 0; t < TT; ++t) acc[t] = 0.f;
#pragma unroll 4
  for (int h = lane * 8; h < H; h += 512) {
    const u32x4 wv = *reinterpret_cast<const u32x4 *>(w + h);
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      if (t < T) {
        const u32x4 xv = *reinterpret_cast<const u32x4 *>(x + int64_t(t) * H + h);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[t] = fmaf(__uint_as_float(wv[i] << 16), __uint_as_float(xv[i] << 16), acc[t]);
          acc[t] = fmaf(__uint_as_float(wv[i] & 0xffff0000u), __uint_as_float(xv[i] & 0xffff0000u), acc[t]);
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    const float v = wave_sum_f32(acc[t]);
    if (t < T && lane == 0) logits[int64_t(t) * E + e] = v;
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
constexpr int kMaxE = 1024;  // 16 logits per lane
constexpr int kMaxK = 256;

__device__ __forceinline__ bool better(float a, int ia, float b, int ib) {
  return a > b || (a == b && ia < ib);
}

__device__ __forceinline__ float wave_sum(float v) { return wave_sum_f32(v); }

// One wave per token.  Lane l holds the token's logits l, l+64, ... as 64-bit
// keys: the logit mapped to an unsigned integer of the same order (-0.0 taken
// as +0.0) in the high half, the complement of the expert index in the low
// half, so that the largest key is the largest logit and, among equal logits,
// the lowest index; all keys differ.  Pick j is found by one wave-wide max
// (a lane-local max, then six butterfly steps) and its owner then drops it:
// k rounds.  Then the gating weights of the picked experts.
__device__ __forceinline__ uint32_t order_key(float x) {
  if (x == 0.0f) x = 0.0f;  // -0.0 and +0.0 are the same key
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// The logit an order key was made from (-0.0 comes back as +0.0).
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Top-k and gating of token t by one wave (all 64 lanes call it).  ids / w
// receive the picks at [t * k + j]; ids_lds (nullable) gets the same ids.
template <int VPL>
__device__ __forceinline__ void topk_token(const float *__restrict__ logits, int t, int E, int k, int gating,
                                           int renorm, int32_t *__restrict__ ids, float *__restrict__ w,
                                           int32_t *ids_lds) {
  const int lane = threadIdx.x & 63;
  const float *lr = logits + int64_t(t) * E;
  float v[VPL];
  uint64_t key[VPL];
  static_assert(kMaxK % 64 == 0, "picks are held 64 per slot");
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = lane + 64 * i;
    v[i] = e < E ? lr[e] : -INFINITY;
    key[i] = e < E ? (uint64_t(order_key(v[i])) << 32) | uint32_t(~e) : 0;  // 0: below every real key
  }
  // k rounds of wave arg-max; pick j ends up in lane j % 64, slot j / 64
  constexpr int KS = kMaxK / 64;
  int pid[KS];
  float pval[KS];  // the picks' logits, recovered from their keys (no second read of the logits)
#pragma unroll
  for (int s2 = 0; s2 < KS; ++s2) {
    pid[s2] = -1;
    pval[s2] = 0.f;
  }
  for (int j = 0; j < k; ++j) {
    uint64_t best = key[0];
#pragma unroll
    for (int i = 1; i < VPL; ++i) best = key[i] > best ? key[i] : best;
    best = wave_max_u64(best);
    const int e = int(~uint32_t(best));
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      if (key[i] == best) key[i] = 0;  // the owner drops its pick
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2)
      if ((j >> 6) == s2 && lane == (j & 63)) {
        pid[s2] = e;
        pval[s2] = key_value(uint32_t(best >> 32));
      }
  }
  // Gating.  softmax: p_e = exp(l_e - max) / sum_E exp(l - max); sigmoid: 1/(1+exp(-l)).
  float mx = v[0];
#pragma unroll
  for (int i = 1; i < VPL; ++i) mx = fmaxf(mx, v[i]);
  mx = wave_max_f32(mx);
  float denom = 1.0f;
  if (gating == FT_SOFTMAX) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      if (lane + 64 * i < E) s += expf(v[i] - mx);
    denom = wave_sum(s);
  }
  float p[KS];
  float local = 0.f;
#pragma unroll
  for (int s2 = 0; s2 < KS; ++s2) {
    p[s2] = 0.f;
    if (pid[s2] >= 0) {
      const float x = pval[s2];
      p[s2] = gating == FT_SOFTMAX ? expf(x - mx) / denom : 1.0f / (1.0f + expf(-x));
      local += p[s2];
    }
  }
  const float wsum = renorm ? wave_sum(local) : 1.0f;
#pragma unroll
  for (int s2 = 0; s2 < KS; ++s2) {
    if (pid[s2] >= 0) {
      const int jj = lane + 64 * s2;
      ids[int64_t(t) * k + jj] = pid[s2];
      w[int64_t(t) * k + jj] = renorm ? p[s2] / wsum : p[s2];
      if (ids_lds) ids_lds[t * k + jj] = pid[s2];
    }
  }
}

template <int VPL>
__global__ __launch_bounds__(64 * kTopkWaves) void topk_gating_kernel(const float *__restrict__ logits,
                                                                       int T, int E, int k, int gating,
                                                                       int renorm, int32_t *__restrict__ ids,
                                                                       float *__restrict__ w) {
  const int t = blockIdx.x * kTopkWaves + (threadIdx.x >> 6);
  if (t < T) topk_token<VPL>(logits, t, E, k, gating, renorm, ids, w, nullptr);
}

// ------------------------------------------------------------------ fused decode routing

constexpr int kFusedMaxT = 16;      // tokens of the fused path (one per wave; more is slower than two launches)
constexpr int kFusedMaxRows = 2048; // routed rows (T * k) of the fused path

struct FusedRouteArgs {
  const float *logits;       // [T, E]
  int T, E, k, gating, renorm;
  int32_t *ids;
  float *w;
  int32_t *offsets, *sorted_rows, *row_pos;
};

// Top-k, gating and the permutation of all T tokens by one workgroup.
template <int VPL>
__device__ __forceinline__ void route_tail(const FusedRouteArgs &a, int32_t *s_ids, int *s_cnt, int *s_tmp) {
  const int wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  for (int t = wave; t < a.T; t += nw) topk_token<VPL>(a.logits, t, a.E, a.k, a.gating, a.renorm, a.ids, a.w, s_ids);
  __syncthreads();
  if (a.T * a.k <= 64) {
    if (wave == 0) permute_wave64(s_ids, a.T * a.k, a.E, s_cnt, a.offsets, a.sorted_rows, a.row_pos);
  } else {
    permute_block(s_ids, a.T * a.k, a.E, s_cnt, s_tmp, a.offsets, a.sorted_rows, a.row_pos);
  }
}

// Top-k, gating and permutation of all T tokens in one workgroup (small decode
// batches, T <= 16): one launch after the router instead of two.  Up to 64
// routed rows the workgroup is one wave per token and wave 0 sorts the rows
// alone (no block-wide histogram, scan and barriers).  (A single
// launch with the router, its last workgroup doing this, was measured
// slower: the device-scope fences that publish the logits write back and
// invalidate the L2 of every XCD.)
template <int VPL>
__global__ __launch_bounds__(1024) void route_tail_kernel(FusedRouteArgs a) {
  __shared__ int32_t s_ids[kFusedMaxRows];
  __shared__ int s_cnt[kMaxE];
  __shared__ int s_tmp[32];
  route_tail<VPL>(a, s_ids, s_cnt, s_tmp);
}

}  // namespace ft

using namespace ft;

// Checks the arguments of a routing call and launches the router logits
// kernel when there is a router (FT_OK with nothing launched when T == 0).
static ft_status route_logits(const void *x, int32_t x_dtype, const void *w_router, float *logits, int32_t T,
                              int32_t H, int32_t E, int32_t k, int32_t gating, int32_t *topk_ids, float *topk_w,
                              hipStream_t stream) {
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
    if (x_dtype == FT_BF16) {
      const uint16_t *xb = static_cast<const uint16_t *>(x);
      const uint8_t *wb = static_cast<const uint8_t *>(w_router);
      // One wave per expert for a few tokens and a large router (1-token decode,
      // 256 x 4096 router: 54.7 against 56.4 us per step); at 128 x 2048 the
      // MFMA tile measured 0.4 us faster, so it keeps those.
      if (T <= 4 && int64_t(E) * H >= (int64_t(1) << 20)) {
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
  // up to 64 routed rows one wave sorts them: one wave per token is enough
  const dim3 blk(T * k <= 64 ? 64 * T : 1024);
  if (vpl <= 2) hipLaunchKernelGGL(route_tail_kernel<2>, dim3(1), blk, 0, stream, a);
  else if (vpl <= 4) hipLaunchKernelGGL(route_tail_kernel<4>, dim3(1), blk, 0, stream, a);
  else hipLaunchKernelGGL(route_tail_kernel<16>, dim3(1), blk, 0, stream, a);
  FT_LAUNCHED("route_tail_kernel");
  clear_error();
  return FT_OK;
}
