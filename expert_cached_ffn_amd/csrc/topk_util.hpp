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

// Top-k and gating of token t by one wave (all 64 lanes call it).  ids / w
// receive the picks at [t * k + j]; ids_lds (nullable) gets the same ids.
template <int VPL>
__device__ __forceinline__ void topk_token(const float *__restrict__ logits, int t, int E, int k, int gating,
                                           int renorm, int32_t *__restrict__ ids, float *__restrict__ w,
                                           int32_t *ids_lds) {
  const int lane = threadIdx.x & 63;
  const float *lr = logits + int64_t(t) * E;
  float v[VPL];
  uint32_t key[VPL];
  static_assert(kMaxK % 64 == 0, "picks are held 64 per slot");
#pragma unroll
  for (int i = 0; i < VPL; ++i) v[i] = lr[lane + 64 * i < E ? lane + 64 * i : 0];
  // all VPL loads above are in flight together (each lane loads an in-range address; lanes past E
  // take -inf below), rather than one round trip per logit
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = lane + 64 * i;
    v[i] = e < E ? v[i] : -INFINITY;
    const uint32_t kk = order_key(v[i]);
    key[i] = e < E ? (kk == 0u ? 1u : kk) : 0u;  // 0: below every real key
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
    uint32_t m = key[0];
#pragma unroll
    for (int i = 1; i < VPL; ++i) m = max(m, key[i]);
    m = wave_max_u32(m);
    int e = -1;  // the lowest expert index holding key m (scalar)
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const uint64_t b = __ballot(key[i] == m);
      if (e < 0 && b != 0) e = 64 * i + int(__builtin_ctzll(b));
    }
#pragma unroll
    for (int i = 0; i < VPL; ++i) key[i] = lane + 64 * i == e ? 0u : key[i];  // the owner drops its pick
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2)
      if ((j >> 6) == s2 && lane == (j & 63)) {
        pid[s2] = e;
        pval[s2] = key_value(m);
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
      if (ids) ids[int64_t(t) * k + jj] = pid[s2];
      if (w) w[int64_t(t) * k + jj] = renorm ? p[s2] / wsum : p[s2];
      if (ids_lds) ids_lds[t * k + jj] = pid[s2];
    }
  }
}

}  // namespace ft
