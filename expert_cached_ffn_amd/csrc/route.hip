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
#include "stream_gemm.hpp"

namespace ft {

// ------------------------------------------------------------------ logits

// bf16: logits[t, e] = sum_h x[t, h] W_r[e, h] on MFMA; one workgroup per
// (16 experts, 64 tokens).
__global__ __launch_bounds__(kStreamThreads) void router_logits_bf16(const uint16_t *__restrict__ x,
                                                                     const uint8_t *__restrict__ wr,
                                                                     float *__restrict__ logits, int T,
                                                                     int H, int E) {
  __shared__ int s_tok[kStreamMaxTok];
  __shared__ float s_red[stream_red_floats<false, 4>()];
  const int tile = blockIdx.x, g0 = blockIdx.y * kStreamMaxTok;
  const int mm = min(kStreamMaxTok, T - g0);
  if (threadIdx.x < mm) s_tok[threadIdx.x] = g0 + threadIdx.x;
  __syncthreads();
  stream_tile_any<WF_BF16, false>(wr, wr, wr, wr, H, tile * 16, E, x, H, s_tok, mm, s_red, logits, E, s_tok);
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

// One wave per token: k rounds of a wave-wide arg-max over the lanes'
// remaining logits, then the gating weights of the picked experts.  Pick j is
// kept by lane j % 64 (slot j / 64); no LDS and no barrier.
template <int VPL>
__global__ __launch_bounds__(64 * kTopkWaves) void topk_gating_kernel(const float *__restrict__ logits,
                                                                       int T, int E, int k, int gating,
                                                                       int renorm, int32_t *__restrict__ ids,
                                                                       float *__restrict__ w) {
  constexpr int KPL = kMaxK / 64;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * kTopkWaves + wave;
  if (t >= T) return;  // whole wave leaves together
  const float *lr = logits + int64_t(t) * E;
  float v[VPL];
  bool live[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = lane + 64 * i;
    live[i] = e < E;
    float x = live[i] ? lr[e] : -INFINITY;
    if (x == 0.0f) x = 0.0f;  // -0.0 and +0.0 are the same key
    v[i] = x;
  }
  float kv[KPL];
  int ki[KPL];
#pragma unroll
  for (int s = 0; s < KPL; ++s) {
    kv[s] = 0.f;
    ki[s] = 0;
  }
  float mx = 0.f;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      if (live[i] && better(v[i], lane + 64 * i, bv, bi)) {
        bv = v[i];
        bi = lane + 64 * i;
      }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      if (better(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if (j == 0) mx = bv;  // the largest logit of the token
    if ((bi & 63) == lane) {
#pragma unroll
      for (int i = 0; i < VPL; ++i)
        if (bi == lane + 64 * i) live[i] = false;
    }
    if ((j & 63) == lane) {
#pragma unroll
      for (int s = 0; s < KPL; ++s)
        if ((j >> 6) == s) {
          kv[s] = bv;
          ki[s] = bi;
        }
    }
  }
  // Gating.  softmax: p_e = exp(l_e - max) / sum_E exp(l - max); sigmoid: 1/(1+exp(-l)).
  float denom = 1.0f;
  if (gating == FT_SOFTMAX) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      if (lane + 64 * i < E) s += expf(v[i] - mx);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
    denom = s;
  }
  float p[KPL];
  float local = 0.f;
#pragma unroll
  for (int s = 0; s < KPL; ++s) {
    const int j = s * 64 + lane;
    p[s] = 0.f;
    if (j < k) {
      p[s] = gating == FT_SOFTMAX ? expf(kv[s] - mx) / denom : 1.0f / (1.0f + expf(-kv[s]));
      local += p[s];
    }
  }
  float wsum = local;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) wsum += __shfl_xor(wsum, off);
#pragma unroll
  for (int s = 0; s < KPL; ++s) {
    const int j = s * 64 + lane;
    if (j < k) {
      ids[int64_t(t) * k + j] = ki[s];
      w[int64_t(t) * k + j] = renorm ? p[s] / wsum : p[s];
    }
  }
}

}  // namespace ft

using namespace ft;

extern "C" ft_status ft_moe_route(const void *x, int32_t x_dtype, const void *w_router, float *logits,
                                  int32_t T, int32_t H, int32_t E, int32_t k, int32_t gating,
                                  int32_t renormalize, int32_t *topk_ids, float *topk_w,
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
    if (x_dtype == FT_BF16) FT_SUPPORTED(H % 128 == 0, "ft_moe_route: bf16 router needs H multiple of 128");
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
      dim3 grid(unsigned(cdiv(E, 16)), unsigned(cdiv(T, kStreamMaxTok)));
      hipLaunchKernelGGL(router_logits_bf16, grid, dim3(kStreamThreads), 0, stream,
                         static_cast<const uint16_t *>(x), static_cast<const uint8_t *>(w_router), logits,
                         T, H, E);
      FT_LAUNCHED("router_logits_bf16");
    } else {
      const int64_t n = int64_t(T) * E;
      hipLaunchKernelGGL(router_logits_f32, dim3(unsigned(cdiv<int64_t>(n, 256))), dim3(256), 0, stream,
                         static_cast<const float *>(x), static_cast<const float *>(w_router), logits, T, H,
                         E);
      FT_LAUNCHED("router_logits_f32");
    }
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
