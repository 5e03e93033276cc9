// Per-token top-k and gating by one wave, shared by the routing kernels and
// the decode FFN's routing prologue.
//
// A router activates a small subset of the experts for each token (FreeToken
// linux page, "Cómo gestiona FreeToken la memoria MoE").  Selection order and
// gating are the textbook forms: descending logit with the lower expert index
// first on ties; softmax over all E or element-wise sigmoid, optionally
// renormalised over the k picked.
#pragma once

#include <math.h>

#include "ft_internal.hpp"

namespace ft {

constexpr int kMaxE = 1024;  // 16 logits per lane
constexpr int kMaxK = 256;

__device__ __forceinline__ float wave_sum(float v) { return wave_sum_f32(v); }

// One wave per token.  Lane l holds the token's logits l, l+64, ... as 32-bit
// order keys: the logit mapped to an unsigned integer of the same order (-0.0
// taken as +0.0), so the largest key is the largest logit.  Pick j is found by
// one wave-wide maximum (a lane-local max, then six butterfly steps) and one
// ballot per logit slot, which names the lowest expert index holding that key
// (ties go to the lower index); its owner then drops it: k rounds.  Key 0
// marks an absent or already picked logit, so real keys start at 1 (the one
// logit bit pattern whose key would be 0, the all-ones NaN, ranks with the
// next-lowest NaN).  Then the gating weights of the picked experts.
__device__ __forceinline__ uint32_t order_key(float x) {
  if (x == 0.0f) x = 0.0f;  // -0.0 and +0.0 are the same key
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// The logit an order key was made from (-0.0 comes back as +0.0).
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Token t's logits into v (lane l: logits l, l + 64, ...): all VPL loads in flight together, each
// at an in-range address (lanes past E are masked by topk_values).
template <int VPL>
__device__ __forceinline__ void topk_load(const float *__restrict__ logits, int t, int E, float (&v)[VPL]) {
  const int lane = threadIdx.x & 63;
  const float *lr = logits + int64_t(t) * E;
#pragma unroll
  for (int i = 0; i < VPL; ++i) v[i] = lr[lane + 64 * i < E ? lane + 64 * i : 0];
}

// Top-k and gating of TPW tokens t[0..TPW) from their loaded logits (see topk_token); only the
// first `live` tokens are written.  The tokens' rounds interleave (the pick's index comes from
// scalar selects, not branches), so one token's dependent max / ballot chain overlaps the others'.
template <int VPL, int TPW>
__device__ __forceinline__ void topk_values(float (&v)[TPW][VPL], const int (&t)[TPW], int live, int E, int k,
                                            int gating, int renorm, int32_t *__restrict__ ids,
                                            float *__restrict__ w, int32_t *ids_lds) {
  const int lane = threadIdx.x & 63;
  uint32_t key[TPW][VPL];
  static_assert(kMaxK % 64 == 0, "picks are held 64 per slot");
#pragma unroll
  for (int u = 0; u < TPW; ++u)
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int e = lane + 64 * i;
      v[u][i] = e < E ? v[u][i] : -INFINITY;
      const uint32_t kk = order_key(v[u][i]);
      key[u][i] = e < E ? (kk == 0u ? 1u : kk) : 0u;  // 0: below every real key
    }
  // k rounds of wave arg-max; pick j ends up in lane j % 64, slot j / 64
  constexpr int KS = kMaxK / 64;
  int pid[TPW][KS];
  float pval[TPW][KS];  // the picks' logits, recovered from their keys (no second read of the logits)
#pragma unroll
  for (int u = 0; u < TPW; ++u)
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) {
      pid[u][s2] = -1;
      pval[u][s2] = 0.f;
    }
  for (int j = 0; j < k; ++j) {
    uint32_t m[TPW];
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      m[u] = key[u][0];
#pragma unroll
      for (int i = 1; i < VPL; ++i) m[u] = max(m[u], key[u][i]);
      m[u] = wave_max_u32(m[u]);
    }
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      int e = 1 << 30;  // the lowest expert index holding key m (scalar); lower slots hold lower indices
#pragma unroll
      for (int i = VPL - 1; i >= 0; --i) {
        const uint64_t b = __ballot(key[u][i] == m[u]);
        e = b != 0 ? 64 * i + int(__builtin_ctzll(b)) : e;
      }
#pragma unroll
      for (int i = 0; i < VPL; ++i) key[u][i] = lane + 64 * i == e ? 0u : key[u][i];  // the owner drops it
#pragma unroll
      for (int s2 = 0; s2 < KS; ++s2)
        if ((j >> 6) == s2 && lane == (j & 63)) {
          pid[u][s2] = e;
          pval[u][s2] = key_value(m[u]);
        }
    }
  }
  // Gating.  softmax: p_e = exp(l_e - max) / sum_E exp(l - max); sigmoid: 1/(1+exp(-l)).
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    float mx = v[u][0];
#pragma unroll
    for (int i = 1; i < VPL; ++i) mx = fmaxf(mx, v[u][i]);
    mx = wave_max_f32(mx);
    float denom = 1.0f;
    if (gating == FT_SOFTMAX) {
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < VPL; ++i)
        if (lane + 64 * i < E) s += expf(v[u][i] - mx);
      denom = wave_sum(s);
    }
    float p[KS];
    float local = 0.f;
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) {
      p[s2] = 0.f;
      if (pid[u][s2] >= 0) {
        const float x = pval[u][s2];
        p[s2] = gating == FT_SOFTMAX ? expf(x - mx) / denom : 1.0f / (1.0f + expf(-x));
        local += p[s2];
      }
    }
    const float wsum = renorm ? wave_sum(local) : 1.0f;
    if (u < live) {
#pragma unroll
      for (int s2 = 0; s2 < KS; ++s2) {
        if (pid[u][s2] >= 0) {
          const int jj = lane + 64 * s2;
          if (ids) ids[int64_t(t[u]) * k + jj] = pid[u][s2];
          if (w) w[int64_t(t[u]) * k + jj] = renorm ? p[s2] / wsum : p[s2];
          if (ids_lds) ids_lds[t[u] * k + jj] = pid[u][s2];
        }
      }
    }
  }
}

// Top-k and gating of token t by one wave (all 64 lanes call it).  ids / w
// receive the picks at [t * k + j]; ids_lds (nullable) gets the same ids.
template <int VPL>
__device__ __forceinline__ void topk_token(const float *__restrict__ logits, int t, int E, int k, int gating,
                                           int renorm, int32_t *__restrict__ ids, float *__restrict__ w,
                                           int32_t *ids_lds) {
  float v[1][VPL];
  topk_load<VPL>(logits, t, E, v[0]);
  const int tt[1] = {t};
  topk_values<VPL, 1>(v, tt, 1, E, k, gating, renorm, ids, w, ids_lds);
}

}  // namespace ft
