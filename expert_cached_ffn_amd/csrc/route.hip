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

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// One wave per token.  The token's logits go to LDS; every lane ranks its own
// logits against all E (rank = number of logits that come before it in the
// order (-logit, index)), so pick j is the logit of rank j -- no serial
// arg-max rounds.  Then the gating weights of the picked experts.
template <int VPL>
__global__ __launch_bounds__(64 * kTopkWaves) void topk_gating_kernel(const float *__restrict__ logits,
                                                                       int T, int E, int k, int gating,
                                                                       int renorm, int32_t *__restrict__ ids,
                                                                       float *__restrict__ w) {
  __shared__ float s_l[kTopkWaves][kMaxE];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * kTopkWaves + wave;
  const bool active = t < T;
  const float *lr = logits + int64_t(active ? t : 0) * E;
  float v[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = lane + 64 * i;
    float x = (active && e < E) ? lr[e] : -INFINITY;
    if (x == 0.0f) x = 0.0f;  // -0.0 and +0.0 are the same key
    v[i] = x;
    if (e < E) s_l[wave][e] = x;
  }
  __syncthreads();
  if (!active) return;
  int rank[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) rank[i] = 0;
  const int E4 = E & ~3;
  for (int e = 0; e < E4; e += 4) {
    const f32x4 o = *reinterpret_cast<const f32x4 *>(&s_l[wave][e]);
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int me = lane + 64 * i;
#pragma unroll
      for (int c = 0; c < 4; ++c) rank[i] += int(o[c] > v[i]) + (int(o[c] == v[i]) & int(e + c < me));
    }
  }
  for (int e = E4; e < E; ++e) {
    const float o = s_l[wave][e];
#pragma unroll
    for (int i = 0; i < VPL; ++i) rank[i] += int(o > v[i]) + (int(o == v[i]) & int(e < lane + 64 * i));
  }
  // Gating.  softmax: p_e = exp(l_e - max) / sum_E exp(l - max); sigmoid: 1/(1+exp(-l)).
  float mx = v[0];
#pragma unroll
  for (int i = 1; i < VPL; ++i) mx = fmaxf(mx, v[i]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  float denom = 1.0f;
  if (gating == FT_SOFTMAX) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      if (lane + 64 * i < E) s += expf(v[i] - mx);
    denom = wave_sum(s);
  }
  float p[VPL];
  float local = 0.f;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    p[i] = 0.f;
    if (lane + 64 * i < E && rank[i] < k) {
      p[i] = gating == FT_SOFTMAX ? expf(v[i] - mx) / denom : 1.0f / (1.0f + expf(-v[i]));
      local += p[i];
    }
  }
  const float wsum = renorm ? wave_sum(local) : 1.0f;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    if (lane + 64 * i < E && rank[i] < k) {
      ids[int64_t(t) * k + rank[i]] = lane + 64 * i;
      w[int64_t(t) * k + rank[i]] = renorm ? p[i] / wsum : p[i];
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
