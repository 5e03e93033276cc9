// ft_moe_grouped_ffn: the SwiGLU expert FFN over per-expert segments, with the
// weights of every expert read through the resident-expert slot table.
//
// Hits run on the GPU straight from the cached copy (FreeToken quantization
// page, "Cómo se desplazan los pesos MoE cuantizados por la memoria"); the
// expert network itself is the textbook SwiGLU FFN (Shazeer 2020), since the
// pages call it an "expert network" and no more.
//
// Two launches per call on one stream:
//   stage 1  h = silu(x Wg^T) * (x Wu^T)   -> bf16 (fp32 for fp32 weights) workspace rows
//   stage 2  y = h Wd^T                    -> fp32 y_rows / y_shared
// bf16 / MXFP4 weights use the weight-streaming MFMA tile (stream_gemm.hpp);
// fp32 weights use a plain FMA kernel.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <unordered_map>

#include "ft_internal.hpp"
#include "stream_gemm.hpp"
#include "stream_persist.hpp"
#include "stream_combine.hpp"
#include "gemv_token.hpp"
#include "gemm_prefill.hpp"
#include "gemm_mx.hpp"

namespace ft {

ft_status mx_quantize_launch(const uint16_t *x, int64_t ldx, int n, int K, uint8_t *q, uint8_t *s,
                             hipStream_t stream);

// Workspace of the native MXFP4 mode: bf16 hidden rows, their MXFP8 codes and
// scales, and the MXFP8 codes and scales of the input tokens (256-B aligned parts).
struct MxWorkspace {
  uint64_t h, hq, hs, xq, xs, total;
};
static MxWorkspace mx_workspace_layout(int64_t T, int64_t k, int64_t H, int64_t I) {
  auto al = [](uint64_t b) { return (b + 255) / 256 * 256; };
  const uint64_t rows = uint64_t(T * k + T);
  MxWorkspace w;
  w.h = 0;
  w.hq = al(rows * I * 2);
  w.hs = w.hq + al(rows * I);
  w.xq = w.hs + al(rows * I / 32);
  w.xs = w.xq + al(uint64_t(T * H));
  w.total = w.xs + al(uint64_t(T * H / 32));
  return w;
}

size_t ffn_workspace_bytes(int32_t T, int32_t k, int32_t E, int32_t H, int32_t I) {
  (void)E;
  const uint64_t rows = uint64_t(T) * uint64_t(k) + uint64_t(T);
  const uint64_t b = (rows * uint64_t(I) * 4 + 255) / 256 * 256;  // fp32 hidden rows (bf16 paths use half)
  const uint64_t mx = mx_workspace_layout(T, k, H, I).total;
  return size_t(b > mx ? b : mx);
}

// Block-wide: index of the aidx-th expert with a non-empty segment (ascending
// expert id), or -1; *n_active = number of non-empty segments.
template <int THREADS>
__device__ int find_active_expert(const int32_t *__restrict__ off, int E, int aidx, int *n_active) {
  constexpr int NW = THREADS / 64;
  __shared__ int s_cnt[NW];
  __shared__ int s_found;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  if (tid == 0) s_found = -1;
  int base = 0;
  for (int c0 = 0; c0 < E; c0 += THREADS) {
    const int e = c0 + tid;
    const bool f = e < E && off[e + 1] > off[e];
    const uint64_t mask = __ballot(f);
    const int lp = __popcll(mask & ((uint64_t(1) << lane) - 1));
    if (lane == 0) s_cnt[wave] = __popcll(mask);
    __syncthreads();
    int before = base, total = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      if (w < wave) before += s_cnt[w];
      total += s_cnt[w];
    }
    if (f && before + lp == aidx) s_found = e;
    base += total;
    __syncthreads();
  }
  *n_active = base;
  return s_found;
}

struct FfnArgs {
  const uint8_t *pool;
  const int32_t *slot_of_expert;
  int32_t n_slots;
  uint64_t expert_bytes;
  const uint8_t *shared_blob;
  uint64_t off_w0, off_w1, off_s0, off_s1;
  int K, N;
  const int32_t *offsets;
  int E, T, k;
  const int32_t *sorted_rows;  // stage 1: token of permuted row p is sorted_rows[p] / k
  const uint16_t *X;           // stage 1: x; stage 2: h rows
  int64_t ldx;
  uint32_t x_bytes;            // bytes of X
  void *out;                   // stage 1: h rows (bf16); stage 2: y_rows (fp32)
  int64_t ldo;
  float *out_shared;           // stage 2: y_shared
  int n_tiles;
  int has_shared;
};

// Grid: (upper bound of active experts incl. shared) x n_tiles workgroups of
// WAVES waves; tokens of a segment are processed 16*NTMAX at a time.
template <int WF, bool STAGE1, int NTMAX, int WAVES, bool PIPE>
__global__ __launch_bounds__(WAVES * 64) void ffn_stream_kernel(FfnArgs a) {
  constexpr int THREADS = WAVES * 64, GROUP = 16 * NTMAX;
  __shared__ int s_tok[GROUP], s_orow[GROUP];
  __shared__ float s_red[stream_red_floats<STAGE1, NTMAX, WAVES>()];
  const int tid = threadIdx.x;
  const int aidx = blockIdx.x / a.n_tiles, tile = blockIdx.x % a.n_tiles;
  int n_act;
  const int e = find_active_expert<THREADS>(a.offsets, a.E, aidx, &n_act);
  const bool is_shared = e < 0 && a.has_shared && aidx == n_act;
  if (e < 0 && !is_shared) return;

  const uint8_t *blob;
  int pos0, m;
  if (is_shared) {
    blob = a.shared_blob;
    pos0 = a.T * a.k;
    m = a.T;
  } else {
    const int slot = table_slot(a.slot_of_expert, e, a.n_slots);
    pos0 = a.offsets[e];
    m = a.offsets[e + 1] - pos0;
    if (slot == FT_SLOT_SKIP) return;  // another call computes these rows
    if (slot < 0) {
      // Caller error: the expert is not resident.  Mark its rows NaN.
      const int row0 = tile * 16;
      for (int u = tid; u < m * 16; u += THREADS) {
        const int j = u / 16, n = row0 + (u % 16);
        if (n >= a.N) continue;
        if (STAGE1)
          reinterpret_cast<uint16_t *>(a.out)[int64_t(pos0 + j) * a.ldo + n] = 0x7fc0;
        else
          reinterpret_cast<float *>(a.out)[int64_t(pos0 + j) * a.ldo + n] = __builtin_nanf("");
      }
      return;
    }
    blob = a.pool + uint64_t(slot) * a.expert_bytes;
  }
  const uint8_t *w0 = blob + a.off_w0, *s0 = blob + a.off_s0;
  const uint8_t *w1 = blob + a.off_w1, *s1 = blob + a.off_s1;
  void *out = a.out;
  if (!STAGE1 && is_shared) out = a.out_shared;

  for (int g0 = 0; g0 < m; g0 += GROUP) {
    const int mm = min(GROUP, m - g0);
    if (tid < mm) {
      const int p = pos0 + g0 + tid;
      if (STAGE1) {
        s_tok[tid] = is_shared ? (g0 + tid) : (a.sorted_rows[p] / a.k);
        s_orow[tid] = p;
      } else {
        s_tok[tid] = p;
        s_orow[tid] = is_shared ? (g0 + tid) : p;
      }
    }
    __syncthreads();
    stream_tile_any<WF, STAGE1, NTMAX, WAVES, PIPE>(w0, s0, w1, s1, a.K, tile * 16, a.N, a.X, a.ldx, a.x_bytes,
                                                    s_tok, mm, s_red, out, a.ldo, s_orow);
  }
}

// Launch one stage with the wave count / token grouping suited to T and K.
template <int WF, bool STAGE1>
static ft_status launch_stream(const FfnArgs &a, int a_max, int T, hipStream_t stream, const char *name) {
  const dim3 grid(unsigned(a_max * a.n_tiles));
  const StreamShape sh = stream_shape(T, a.K / stream_kblock<WF>());
#define FT_STREAM(NT, W, P)                                                                                   \
  if (sh.ntmax == NT && sh.waves == W && sh.pipe == P)                                                        \
    hipLaunchKernelGGL((ffn_stream_kernel<WF, STAGE1, NT, W, P>), grid, dim3(W * 64), 0, stream, a);
  FT_STREAM(1, 16, false)
  FT_STREAM(1, 16, true)
  FT_STREAM(1, 8, false)
  FT_STREAM(1, 8, true)
  FT_STREAM(1, 6, false)
  FT_STREAM(1, 6, true)
  FT_STREAM(1, 4, false)
  FT_STREAM(1, 4, true)
  FT_STREAM(2, 16, false)
  FT_STREAM(2, 16, true)
  FT_STREAM(2, 8, false)
  FT_STREAM(2, 8, true)
  FT_STREAM(2, 6, false)
  FT_STREAM(2, 6, true)
  FT_STREAM(2, 4, false)
  FT_STREAM(2, 4, true)
#undef FT_STREAM
  FT_LAUNCHED(name);
  return FT_OK;
}

// ------------------------------------------------------------------ persistent decode path

// Weight register sets in flight for the x-stationary kernel, per shape.
#ifndef FT_XS_NB
// (NVFP4 tiles hold half the MXFP4 weight registers: deeper rings.  bf16 down
// tiles: 4, not 6, keeps 99 VGPRs and four waves per SIMD; measured 244 vs 247
// us per 64-token step, and 2 or 3 sets were slower)
#define FT_XS_NB(WF, GLU, WAVES, KPW)                                                     \
  ((WF) == WF_NV4 ? ((GLU) ? ((WAVES) >= 16 ? 2 : 4) : 6)                                  \
                  : ((GLU) ? ((WAVES) >= 16 || (KPW) == 2 ? 2 : 4) : ((KPW) == 2 || (WF) == WF_BF16 ? 4 : 6)))
#endif

// Register sets for two-row-tile units (RT = 2, NVFP4 down stage): 3 sets
// measured 118.3 us per 64-token step against 121.0 / 120.3 / 133.8 us with
// 2 / 4 / 6 sets (111 VGPRs at 4 sets).
#ifndef FT_XS_NB_RT2
#define FT_XS_NB_RT2 3
#endif

template <int WF, bool GLU, int WAVES, int KPW, int RT = 1>
__global__ __launch_bounds__(WAVES * 64) void ffn_persist_xs_kernel(PersistArgs a) {
  __shared__ float s_red[WAVES * (GLU ? 2 : RT) * 256];
  constexpr int NB = RT == 2 ? FT_XS_NB_RT2 : FT_XS_NB(WF, GLU, WAVES, KPW);
  stream_persist_xs<WF, GLU, WAVES, KPW, NB, RT>(a, s_red);
}

template <int WF, bool GLU, int WAVES, int KPW>
__global__ __launch_bounds__(WAVES * 64) void ffn_persist_kernel(PersistArgs a) {
  __shared__ float s_red[WAVES * (GLU ? 2 : 1) * 256];
  // Units in flight: a 16-wave gate/up tile leaves no registers for a second
  // activation set (128 per lane in a 1024-thread workgroup); 8-wave bf16
  // gate/up tiles take two (measured faster; MXFP4 tiles were slower with two);
  // the smaller down-projection tiles need a deeper ring to cover HBM latency.
  constexpr int NB = GLU ? (WAVES * KPW >= 16 ? (WAVES <= 8 && WF == WF_BF16 ? 2 : 1) : 2)
                         : (WAVES * KPW >= 16 ? 2 : 3);
  stream_persist<WF, GLU, WAVES, KPW, NB>(a, s_red);
}

// Resident workgroups per CU of a kernel (cached) times the CU count.
static int resident_grid(const void *kernel, int threads) {
  static std::mutex mu;
  static std::unordered_map<const void *, int> cache;
  static int cus = 0;
  std::lock_guard<std::mutex> lock(mu);
  if (cus == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
  }
  auto it = cache.find(kernel);
  if (it != cache.end()) return it->second;
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess || per_cu <= 0) {
    (void)hipGetLastError();
    per_cu = 1;
  }
  const int g = per_cu * cus;
  cache[kernel] = g;
  return g;
}

// Waves per workgroup x k-blocks per wave covering nkb exactly, or {0, 0}.
static void persist_shape(int nkb, int *waves, int *kpw) {
  *waves = 0;
  *kpw = 0;
  if (nkb == 16) {  // 8 waves x 2 k-blocks: measured faster than 16 x 1 for bf16 and MXFP4 weights
    *waves = 8;
    *kpw = 2;
    return;
  }
  for (int c : {1, 2})
    for (int w : {16, 12, 8, 6, 4})
      if (w * c == nkb && (c == 1 || w <= 8)) {  // wider 2-block shapes exceed the register budget
        *waves = w;
        *kpw = c;
        return;
      }
}

// Shape override for tuning: FTMOE_PERSIST_GU / FTMOE_PERSIST_DN = "waves,kpw"
// (used only when waves * kpw equals the stage's k-block count).
static void persist_override(bool glu, int nkb, int *waves, int *kpw) {
  const char *v = getenv(glu ? "FTMOE_PERSIST_GU" : "FTMOE_PERSIST_DN");
  int w = 0, c = 0;
  if (v && sscanf(v, "%d,%d", &w, &c) == 2 && w * c == nkb) {
    *waves = w;
    *kpw = c;
  }
}

// A persistent shape covers a contraction length K of weight format WF.
template <int WF>
static bool persist_covers(int K) {
  if (K % stream_kblock<WF>() != 0) return false;
  int waves, kpw;
  persist_shape(K / stream_kblock<WF>(), &waves, &kpw);
  return waves > 0;
}

template <int WF, bool GLU>
static bool launch_persist(const PersistArgs &a, int max_units, hipStream_t stream) {
  int waves, kpw;
  persist_shape(a.K / stream_kblock<WF>(), &waves, &kpw);
  // FP4 down stage over 8 k-blocks: 4 waves x 2 blocks (measured ~2 us faster than 8 x 1 at 1-32 tokens:
  // half the waves meet at each unit's reduction)
  if (!GLU && WF != WF_BF16 && waves == 8 && kpw == 1) {
    waves = 4;
    kpw = 2;
  }
  // NVFP4 over 16 k-blocks: 16 waves x 1 block (90 VGPRs, four waves per SIMD)
  // instead of 8 x 2 (172 VGPRs, two): its decode's dependent VALU chains
  // need the waves; measured 70.6 -> 61.1 us for the gate/up stage at 64
  // tokens.  (MXFP4 and bf16 measured no gain.)
  if (WF == WF_NV4 && waves == 8 && kpw == 2) {
    waves = 16;
    kpw = 1;
  }
  persist_override(GLU, a.K / stream_kblock<WF>(), &waves, &kpw);
  // x-stationary runs for MXFP4 weights (measured 1.65x at 32 tokens: a 16-row
  // FP4 tile is half the bytes of a bf16 one, so the freed activation
  // registers matter).  bf16 gate/up tiles keep the strided order (measured
  // faster); the bf16 down stage goes x-stationary once there are as many
  // routed rows as experts (128 experts, top-8: 167.7 -> 164.8 us per step at
  // 16 tokens, 253.0 -> 244.1 at 64; at 1 token it measured 2 us slower).
  // FTMOE_PERSIST_XS = "<gate/up><down>", each 0 or 1 (e.g. "01").
  static const char *xs_env = getenv("FTMOE_PERSIST_XS");
  const int xs_req = (xs_env && strlen(xs_env) == 2) ? xs_env[GLU ? 0 : 1] - '0' : -1;
  const bool xs_auto = WF == WF_FP4 || (!GLU && int64_t(a.T) * a.k >= int64_t(a.E));
  const bool xs = WF == WF_NV4 || (xs_req < 0 ? xs_auto : xs_req != 0);  // NVFP4: x-stationary only
  // NVFP4 down stage: two 16-row tiles per unit (a 16-row tile of a 768-long
  // contraction is 6.75 KB, so the per-unit LDS round and barriers dominated:
  // 46.4 -> 35.7 us per launch at 64 tokens, 129.4 -> 118.3 us per step).  bf16
  // down tiles measured equal with two, so they keep one.  FTMOE_PERSIST_RT =
  // "1" keeps one tile for NVFP4 too.
  static const char *rt_env = getenv("FTMOE_PERSIST_RT");
  const bool rt2 = WF == WF_NV4 && !GLU && !(rt_env && rt_env[0] == '1');
#define FT_PERSIST(W, C)                                                                          \
  if (waves == W && kpw == C) {                                                                   \
    if constexpr (WF == WF_NV4 && !GLU) {                                                         \
      if (rt2) {                                                                                  \
        const void *kern = reinterpret_cast<const void *>(&ffn_persist_xs_kernel<WF, GLU, W, C, 2>); \
        const int g = std::max(1, std::min(max_units, resident_grid(kern, W * 64)));               \
        hipLaunchKernelGGL((ffn_persist_xs_kernel<WF, GLU, W, C, 2>), dim3(g), dim3(W * 64), 0, stream, a); \
        return true;                                                                              \
      }                                                                                           \
    }                                                                                             \
    if (xs) {                                                                                     \
      const void *kern = reinterpret_cast<const void *>(&ffn_persist_xs_kernel<WF, GLU, W, C>); \
      const int g = std::max(1, std::min(max_units, resident_grid(kern, W * 64)));                 \
      hipLaunchKernelGGL((ffn_persist_xs_kernel<WF, GLU, W, C>), dim3(g), dim3(W * 64), 0, stream, a); \
    } else if constexpr (WF != WF_NV4) {                                                          \
      const void *kern = reinterpret_cast<const void *>(&ffn_persist_kernel<WF, GLU, W, C>);      \
      const int g = std::max(1, std::min(max_units, resident_grid(kern, W * 64)));                 \
      hipLaunchKernelGGL((ffn_persist_kernel<WF, GLU, W, C>), dim3(g), dim3(W * 64), 0, stream, a); \
    }                                                                                             \
    return true;                                                                                  \
  }
  FT_PERSIST(16, 1)
  FT_PERSIST(12, 1)
  FT_PERSIST(8, 1)
  FT_PERSIST(6, 1)
  FT_PERSIST(4, 1)
  FT_PERSIST(8, 2)
  FT_PERSIST(6, 2)
  FT_PERSIST(4, 2)
#undef FT_PERSIST
  return false;
}

// ------------------------------------------------------------------ fused layer call (a few tokens)

// Gate/up of the fused layer call: routing prologue, then the x-stationary
// weight stream (rows per tile in a.tile_rows).
template <int WF, int WAVES, int KPW>
__global__ __launch_bounds__(WAVES * 64) void ffn_route_gate_up_kernel(PersistArgs a) {
  __shared__ float s_red[WAVES * 2 * 256];
  constexpr int NB = FT_XS_NB(WF, true, WAVES, KPW);
  stream_persist_xs<WF, true, WAVES, KPW, NB, 1, true>(a, s_red);
}

// Down projection with the combine folded in.  Register sets per step: bf16
// 32 VGPRs (weights + hidden row), MXFP4 42, NVFP4 22 at one k-block per wave.
template <int WF, int WAVES, int KPW>
__global__ __launch_bounds__(WAVES * 64) void ffn_down_combine_kernel(PersistArgs a) {
  __shared__ float s_red[WAVES * 256];
  constexpr int NB = KPW == 2 ? 2 : (WF == WF_FP4 ? 3 : 4);
  stream_combine_xs<WF, WAVES, KPW, NB>(a, s_red);
}

// The persistent shape of the fused kernels for a contraction of nkb k-blocks
// (the decode path's choice; NVFP4 gate/up as 16 waves x 1), or false.
template <int WF>
static bool fused_shape(bool glu, int nkb, int *waves, int *kpw) {
  persist_shape(nkb, waves, kpw);
  if (WF == WF_NV4 && glu && *waves == 8 && *kpw == 2) {
    *waves = 16;
    *kpw = 1;
  }
  return *waves > 0 && !(*waves == 16 && !glu);
}

// Rows per tile (16 or 8) that finish `units16` 16-row units soonest on `grid`
// workgroups: ceil(units / grid) * rows, ties to 16.
// FTMOE_FUSED_TR = "8" or "16" forces the choice (tuning measurements).
static int tile_rows_for(int units16, int grid) {
  static const char *env = getenv("FTMOE_FUSED_TR");
  if (env && (env[0] == '8' || (env[0] == '1' && env[1] == '6'))) return env[0] == '8' ? 8 : 16;
  // 8-row tiles only when they at least halve the time in rows streamed (measured: at equal cost the
  // extra per-tile reductions made them slower)
  const int t16 = cdiv(units16, grid) * 16, t8 = cdiv(2 * units16, grid) * 8;
  return 2 * t8 <= t16 ? 8 : 16;
}

template <int WF, bool GLU>
static ft_status launch_fused(PersistArgs a, int units16, int groups, hipStream_t stream) {
  int waves = 0, kpw = 0;
  if (!fused_shape<WF>(GLU, a.K / stream_kblock<WF>(), &waves, &kpw))
    return fail(FT_ENOTSUP, "ft_moe_layer: no fused kernel for this contraction length");
#define FT_FUSED(W, C)                                                                                     \
  if (waves == W && kpw == C) {                                                                           \
    const void *kern = nullptr;                                                                           \
    if constexpr (GLU)                                                                                    \
      kern = reinterpret_cast<const void *>(&ffn_route_gate_up_kernel<WF, W, C>);                         \
    else                                                                                                  \
      kern = reinterpret_cast<const void *>(&ffn_down_combine_kernel<WF, W, C>);                          \
    const int rg = resident_grid(kern, W * 64);                                                           \
    a.tile_rows = tile_rows_for(units16, rg);                                                             \
    a.n_tiles = cdiv(a.N, a.tile_rows);                                                                   \
    const int g = std::max(1, std::min(units16 * (16 / a.tile_rows) * groups, rg));                        \
    if constexpr (GLU)                                                                                    \
      hipLaunchKernelGGL((ffn_route_gate_up_kernel<WF, W, C>), dim3(g), dim3(W * 64), 0, stream, a);      \
    else                                                                                                  \
      hipLaunchKernelGGL((ffn_down_combine_kernel<WF, W, C>), dim3(g), dim3(W * 64), 0, stream, a);       \
    FT_LAUNCHED((GLU ? "ffn_route_gate_up_kernel" : "ffn_down_combine_kernel"));                           \
    return FT_OK;                                                                                         \
  }
  if constexpr (WF == WF_NV4 && GLU) FT_FUSED(16, 1)
  FT_FUSED(8, 2)
  FT_FUSED(12, 1)
  FT_FUSED(8, 1)
  FT_FUSED(6, 1)
  FT_FUSED(4, 1)
#undef FT_FUSED
  return fail(FT_ENOTSUP, "ft_moe_layer: no fused kernel for this persistent shape");
}

// ------------------------------------------------------------------ one-token layer call (GEMV)

template <int WF, int NCH, int RPW>
__global__ __launch_bounds__(kGemvGuThreads) __attribute__((amdgpu_waves_per_eu(2))) void ffn_token_gate_up_kernel(
    PersistArgs a) {
  gemv_gate_up<WF, NCH, RPW>(a);
}

template <int WF, int NCH, int RPW, int NCHD, int RB>
__global__ __launch_bounds__(kGemvGuThreads) __attribute__((amdgpu_waves_per_eu(2))) void ffn_token_layer_kernel(
    PersistArgs a, PersistArgs d, uint32_t *wait_words) {
  gemv_gate_up<WF, NCH, RPW, NCHD, RB>(a, &d, wait_words);
}

template <int WF, int NCH, int RPW, int SPW>
__global__ __launch_bounds__(kGemvThreads) __attribute__((amdgpu_waves_per_eu(2))) void ffn_token_down_combine_kernel(
    PersistArgs a) {
  gemv_down_combine<WF, NCH, RPW, SPW>(a);
}

// Code bytes of one weight row of K elements.
template <int WF>
static int row_code_bytes(int K) { return WF == WF_BF16 ? 2 * K : K / 2; }

// 1 KiB chunks per row rounded up to 1, 2 or 4 (0: rows longer than 4 KiB).
static int gemv_chunks(int row_bytes) {
  const int c = cdiv(row_bytes, 1024);
  return c <= 1 ? 1 : (c <= 2 ? 2 : (c <= 4 ? 4 : 0));
}

// The one-token kernels cover this layer: routing limits of the prologue, rows of at most
// 4 KiB of codes, at most 12 down steps (k routed + shared; 3 per wave).
template <int WF>
static bool token_gemv_covers(int H, int I, int E, int k, bool shared) {
  return E <= kRouteMaxE && k <= kFusedMaxK && k + (shared ? 1 : 0) <= 12 && gemv_chunks(row_code_bytes<WF>(H)) > 0 &&
         gemv_chunks(row_code_bytes<WF>(I)) > 0;
}

// The one-launch layer kernel for gate/up chunks C, down chunks CD: rows per down block 4, or 8
// where 4-row blocks would outnumber the workgroups that fit (not with 4-chunk down rows, whose
// 8-row blocks do not fit in registers; there workgroups take several blocks); the grid is at most
// the workgroups that fit at once (the grid-wide wait needs them all resident).
template <int WF, int C, int R, int CD, int RB>
static void launch_token_layer_rb(const PersistArgs &p1, const PersistArgs &p2, uint32_t *wait_words, int grid,
                                  hipStream_t stream) {
  hipLaunchKernelGGL((ffn_token_layer_kernel<WF, C, R, CD, RB>), dim3(grid), dim3(kGemvGuThreads), 0, stream, p1, p2,
                     wait_words);
}

template <int WF, int C, int R, int CD>
static void launch_token_layer(const PersistArgs &p1, const PersistArgs &p2, uint32_t *wait_words, int jobs,
                               hipStream_t stream) {
  const int r4 = resident_grid(reinterpret_cast<const void *>(&ffn_token_layer_kernel<WF, C, R, CD, 4>),
                               kGemvGuThreads);
  const int want = cdiv(jobs, kGemvGuThreads / 64);
  if constexpr (CD < 4) {
    if (cdiv(p2.N, 4) > r4) {
      const int r8 = resident_grid(reinterpret_cast<const void *>(&ffn_token_layer_kernel<WF, C, R, CD, 8>),
                                   kGemvGuThreads);
      launch_token_layer_rb<WF, C, R, CD, 8>(p1, p2, wait_words, std::max(1, std::min(r8, std::max(want, cdiv(p2.N, 8)))),
                                             stream);
      return;
    }
  }
  launch_token_layer_rb<WF, C, R, CD, 4>(p1, p2, wait_words, std::max(1, std::min(r4, std::max(want, cdiv(p2.N, 4)))),
                                         stream);
}

template <int WF>
static ft_status launch_token_gemv(const PersistArgs &p1, const PersistArgs &p2, uint32_t *wait_words,
                                   hipStream_t stream) {
  // gate/up: 4 / NCH row pairs per wave job (8 loads of 16 bytes per lane, two jobs in flight);
  // the grid: the workgroups that fit at once, or fewer if there are fewer jobs
  const int c1 = gemv_chunks(row_code_bytes<WF>(p1.K));
  const int acts = std::min(p1.E, p1.k) + (p1.shared_blob != nullptr ? 1 : 0);
  const int c2 = gemv_chunks(row_code_bytes<WF>(p2.K));
  if (acts <= kGemvGuThreads / 64) {
    // every down step has a wave of its own: gate/up and down + combine in one launch
    const int jobs = acts * cdiv(p1.N, 4 / c1);
#define FT_TLY(C, R, CD) \
  if (c1 == C && c2 == CD) launch_token_layer<WF, C, R, CD>(p1, p2, wait_words, jobs, stream);
    FT_TLY(1, 4, 1)
    FT_TLY(1, 4, 2)
    FT_TLY(1, 4, 4)
    FT_TLY(2, 2, 1)
    FT_TLY(2, 2, 2)
    FT_TLY(2, 2, 4)
    FT_TLY(4, 1, 1)
    FT_TLY(4, 1, 2)
    FT_TLY(4, 1, 4)
#undef FT_TLY
    FT_LAUNCHED("ffn_token_layer_kernel");
    return FT_OK;
  }
#define FT_TGU(C, R)                                                                                     \
  if (c1 == C) {                                                                                         \
    const void *kern = reinterpret_cast<const void *>(&ffn_token_gate_up_kernel<WF, C, R>);             \
    const int grid = std::max(1, std::min(resident_grid(kern, kGemvGuThreads),                          \
                                          cdiv(acts * cdiv(p1.N, R), kGemvGuThreads / 64)));              \
    hipLaunchKernelGGL((ffn_token_gate_up_kernel<WF, C, R>), dim3(grid), dim3(kGemvGuThreads), 0, stream, p1); \
  }
  FT_TGU(1, 4)
  FT_TGU(2, 2)
  FT_TGU(4, 1)
#undef FT_TGU
  FT_LAUNCHED("ffn_token_gate_up_kernel");
  // down + combine: the waves split the steps (2 or 3 each); rows per workgroup so that about
  // 16 weight pieces per lane are in flight
  const int spw = (p2.k + (p2.shared_blob != nullptr ? 1 : 0)) <= 8 ? 2 : 3;
#define FT_TDN(C, R, SP)                                                                                 \
  if (c2 == C && spw == SP) {                                                                            \
    const int grid = cdiv(p2.N, R);                                                                      \
    hipLaunchKernelGGL((ffn_token_down_combine_kernel<WF, C, R, SP>), dim3(grid), dim3(kGemvThreads), 0, stream, p2); \
  }
  FT_TDN(1, 8, 2)
  FT_TDN(1, 4, 3)
  FT_TDN(2, 4, 2)
  FT_TDN(2, 2, 3)
  FT_TDN(4, 2, 2)
  FT_TDN(4, 1, 3)
#undef FT_TDN
  FT_LAUNCHED("ffn_token_down_combine_kernel");
  return FT_OK;
}

// ------------------------------------------------------------------ prefill grouped GEMM

// Two pipeline stages.  MXFP4 and NVFP4 weights: two workgroups per CU
// (measured faster than four stages at one workgroup per CU: the second wave
// on each SIMD hides the 4-bit decode and the MFMA dependency chains; NVFP4
// went from 1.57 to 1.12 ms per 8192-token layer when its scales stopped
// taking a register set per stage).  bf16 weights need four times the weight
// registers: one workgroup per CU, so that nothing spills.
template <int WF, bool GLU>
__global__ __launch_bounds__(kGemmThreads, WF == WF_BF16 ? 1 : 2) void ffn_gemm_kernel(GemmArgs a) {
  constexpr int B = kGemmBM * kGemmPitch;
  __shared__ __attribute__((aligned(16))) uint8_t l0[B];
  __shared__ __attribute__((aligned(16))) uint8_t l1[B];
  gemm_tile<WF, GLU, 2>(a, LdsRing<2>{{l0, l1}});
}

// Upper bound of token tiles of BM rows over all segments (+ the shared expert).
static int gemm_mtiles_bound(int T, int k, int E, bool shared, int BM = kGemmBM) {
  const int64_t routed = int64_t(T) * k;
  return int(routed / BM + std::min<int64_t>(E, routed) + (shared ? cdiv(T, BM) : 0));
}

template <int WF, bool GLU>
static ft_status launch_gemm(GemmArgs a, hipStream_t stream, const char *name) {
  const int nt = GLU ? cdiv(a.N, kGemmBN / 2) : cdiv(a.N, kGemmBN);
  const int mb = gemm_mtiles_bound(a.T, a.k, a.E, a.shared_blob != nullptr);
  a.n_ntiles = nt;
  a.n_mtiles = mb;
  a.n_items = gemm_item_count(mb, nt);
  const int grid = cdiv(a.n_items, 8) * 8;
  hipLaunchKernelGGL((ffn_gemm_kernel<WF, GLU>), dim3(unsigned(grid)), dim3(kGemmThreads), 0, stream, a);
  FT_LAUNCHED(name);
  return FT_OK;
}

// ------------------------------------------------------------------ native MXFP4 mode GEMM

// Three pipeline stages of 128-element chunks of 128 token rows and the two
// scale windows: 72 KiB of LDS, two workgroups per CU.
template <bool GLU>
__global__ __launch_bounds__(kGemmThreads, 2) void ffn_mx_gemm_kernel(MxGemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds0[kMxCodeBytes];
  __shared__ __attribute__((aligned(16))) uint8_t lds1[kMxCodeBytes];
  __shared__ __attribute__((aligned(16))) uint8_t wsc[kMxWScaleBytes];
  __shared__ __attribute__((aligned(16))) uint8_t xsc[kMxXScaleBytes];
  static_assert(kMxStages == 2, "one array per stage");
  gemm_mx_tile<GLU>(a, MxLds{LdsRing<kMxStages>{{lds0, lds1}}, wsc, xsc});
}

template <bool GLU>
static ft_status launch_mx_gemm(MxGemmArgs a, hipStream_t stream, const char *name) {
  const int nt = GLU ? cdiv(a.g.N, kGemmBN / 2) : cdiv(a.g.N, kGemmBN);
  const int mb = gemm_mtiles_bound(a.g.T, a.g.k, a.g.E, a.g.shared_blob != nullptr, kMxBM);
  a.g.n_ntiles = nt;
  a.g.n_mtiles = mb;
  a.g.n_items = gemm_item_count(mb, nt);
  const int grid = cdiv(a.g.n_items, 8) * 8;
  hipLaunchKernelGGL((ffn_mx_gemm_kernel<GLU>), dim3(unsigned(grid)), dim3(kGemmThreads), 0, stream, a);
  FT_LAUNCHED(name);
  return FT_OK;
}

// ------------------------------------------------------------------ fp32 path

struct FfnF32Args {
  const uint8_t *pool;
  const int32_t *slot_of_expert;
  int32_t n_slots;
  uint64_t expert_bytes;
  const uint8_t *shared_blob;
  uint64_t off_gate, off_up, off_down;
  int H, I;
  const int32_t *offsets;
  int E, T, k;
  const int32_t *sorted_rows;
  const float *x;
  float *h;  // [T*k (+T), I]
  float *y_rows;
  float *y_shared;
  int rows;  // T*k (+T)
};

// Expert of permuted row p (p < T*k): offsets[e] <= p < offsets[e+1].
__device__ __forceinline__ int expert_of_row(const int32_t *off, int E, int p) {
  int lo = 0, hi = E;  // answer in [lo, hi)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (off[mid] <= p) lo = mid; else hi = mid;
  }
  return lo;
}

// The blob of permuted row p; *ok false: not resident (NaN rows); *skip: FT_SLOT_SKIP (row left untouched).
__device__ __forceinline__ const float *f32_blob(const FfnF32Args &a, int p, int *tok, bool *ok, bool *skip) {
  const int routed = a.T * a.k;
  *ok = true;
  *skip = false;
  if (p >= routed) {
    *tok = p - routed;
    return reinterpret_cast<const float *>(a.shared_blob);
  }
  const int e = expert_of_row(a.offsets, a.E, p);
  *tok = a.sorted_rows[p] / a.k;
  const int slot = table_slot(a.slot_of_expert, e, a.n_slots);
  if (slot < 0) {
    *ok = false;
    *skip = slot == FT_SLOT_SKIP;
    return nullptr;
  }
  return reinterpret_cast<const float *>(a.pool + uint64_t(slot) * a.expert_bytes);
}

__global__ __launch_bounds__(256) void ffn_f32_stage1(FfnF32Args a) {
  const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= int64_t(a.rows) * a.I) return;
  const int p = int(idx / a.I), i = int(idx % a.I);
  int tok;
  bool ok, skip;
  const float *b = f32_blob(a, p, &tok, &ok, &skip);
  if (!ok) {
    if (!skip) a.h[idx] = __builtin_nanf("");
    return;
  }
  const float *wg = reinterpret_cast<const float *>(reinterpret_cast<const uint8_t *>(b) + a.off_gate) + int64_t(i) * a.H;
  const float *wu = reinterpret_cast<const float *>(reinterpret_cast<const uint8_t *>(b) + a.off_up) + int64_t(i) * a.H;
  const float *xr = a.x + int64_t(tok) * a.H;
  float g = 0.f, u = 0.f;
  for (int c = 0; c < a.H; ++c) {
    g = fmaf(xr[c], wg[c], g);
    u = fmaf(xr[c], wu[c], u);
  }
  a.h[idx] = g / (1.0f + expf(-g)) * u;
}

__global__ __launch_bounds__(256) void ffn_f32_stage2(FfnF32Args a) {
  const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= int64_t(a.rows) * a.H) return;
  const int p = int(idx / a.H), n = int(idx % a.H);
  int tok;
  bool ok, skip;
  const float *b = f32_blob(a, p, &tok, &ok, &skip);
  const int routed = a.T * a.k;
  float *dst = p >= routed ? (a.y_shared + int64_t(tok) * a.H + n) : (a.y_rows + int64_t(p) * a.H + n);
  if (!ok) {
    if (!skip) *dst = __builtin_nanf("");
    return;
  }
  const float *wd = reinterpret_cast<const float *>(reinterpret_cast<const uint8_t *>(b) + a.off_down) + int64_t(n) * a.I;
  const float *hr = a.h + int64_t(p) * a.I;
  float y = 0.f;
  for (int c = 0; c < a.I; ++c) y = fmaf(hr[c], wd[c], y);
  *dst = y;
}

}  // namespace ft

using namespace ft;

// The argument checks of ft_moe_grouped_ffn (FT_OK for a valid call, T = 0 included).
static ft_status ffn_check(const ft_expert_layout *L, const void *slot_pool, int32_t n_slots,
                           const int32_t *slot_of_expert, const void *shared_blob, const void *x, int32_t x_dtype,
                           int32_t T, int32_t k, int32_t E, const int32_t *expert_offsets,
                           const int32_t *sorted_rows, const float *y_rows, const float *y_shared, int32_t mode,
                           const void *workspace, size_t workspace_bytes) {
  FT_REQUIRE(L != nullptr, "ft_moe_grouped_ffn: layout is NULL");
  FT_REQUIRE(T >= 0 && k >= 1 && E >= 1, "ft_moe_grouped_ffn: need T >= 0, k >= 1, E >= 1");
  FT_REQUIRE(int64_t(T) * (k + 1) < (int64_t(1) << 31), "ft_moe_grouped_ffn: T*k too large");
  FT_SUPPORTED((int64_t(T) * (k + 1)) * L->I * 2 < (int64_t(1) << 31) && int64_t(T) * L->H * 2 < (int64_t(1) << 31) &&
                   int64_t(L->H) * L->I * 2 < (int64_t(1) << 31),
               "ft_moe_grouped_ffn: activation, hidden or weight matrix above 2 GiB");
  FT_SUPPORTED(k <= E, "ft_moe_grouped_ffn: k > E");
  FT_SUPPORTED(E <= 4096, "ft_moe_grouped_ffn: E > 4096");
  const int stages = mode & (FT_FFN_GATE_UP_ONLY | FT_FFN_DOWN_ONLY);
  FT_REQUIRE(stages != (FT_FFN_GATE_UP_ONLY | FT_FFN_DOWN_ONLY),
             "ft_moe_grouped_ffn: FT_FFN_GATE_UP_ONLY and FT_FFN_DOWN_ONLY together");
  FT_REQUIRE((mode & ~0x3ff) == 0, "ft_moe_grouped_ffn: unknown mode bits");
  const int variant = mode & 0xff;
  FT_SUPPORTED(variant == FT_FFN_EXACT || variant == FT_FFN_NATIVE_MX, "ft_moe_grouped_ffn: unknown mode");
  const int H = L->H, I = L->I;
  FT_REQUIRE(H >= 1 && I >= 1 && L->expert_bytes > 0, "ft_moe_grouped_ffn: layout not initialised");
  const int wd = L->wdtype;
  if (wd == FT_F32) {
    FT_REQUIRE(x_dtype == FT_F32, "ft_moe_grouped_ffn: fp32 weights need fp32 activations");
  } else if (wd == FT_BF16) {
    FT_REQUIRE(x_dtype == FT_BF16, "ft_moe_grouped_ffn: bf16 weights need bf16 activations");
    FT_SUPPORTED(H % 128 == 0 && I % 128 == 0, "ft_moe_grouped_ffn: bf16 weights need H, I multiples of 128");
  } else if (wd == FT_MXFP4) {
    FT_REQUIRE(x_dtype == FT_BF16, "ft_moe_grouped_ffn: MXFP4 weights need bf16 activations");
    FT_SUPPORTED(H % 256 == 0 && I % 256 == 0, "ft_moe_grouped_ffn: MXFP4 weights need H, I multiples of 256");
  } else if (wd == FT_NVFP4) {
    FT_REQUIRE(x_dtype == FT_BF16, "ft_moe_grouped_ffn: NVFP4 weights need bf16 activations");
    FT_SUPPORTED(H % 128 == 0 && I % 128 == 0, "ft_moe_grouped_ffn: NVFP4 weights need H, I multiples of 128");
  } else {
    return fail(FT_EINVAL, "ft_moe_grouped_ffn: unknown weight dtype in layout");
  }
  FT_SUPPORTED(variant == FT_FFN_EXACT || wd == FT_MXFP4,
               "ft_moe_grouped_ffn: the native scaled-MFMA mode needs MXFP4 weights");
  if (T == 0) return FT_OK;
  FT_REQUIRE(slot_pool && x && expert_offsets && sorted_rows && y_rows,
             "ft_moe_grouped_ffn: NULL pointer argument");
  FT_REQUIRE(n_slots >= 1 && (slot_of_expert != nullptr || n_slots >= E),
             "ft_moe_grouped_ffn: n_slots must be >= 1, and >= E when slot_of_expert is NULL");
  FT_REQUIRE((shared_blob == nullptr) == (y_shared == nullptr),
             "ft_moe_grouped_ffn: shared_blob and y_shared must both be given or both be NULL");
  FT_REQUIRE(aligned(slot_pool, 256) && (!shared_blob || aligned(shared_blob, 256)) &&
                 L->expert_bytes % 256 == 0,
             "ft_moe_grouped_ffn: slot_pool / shared_blob must be 256-byte aligned");
  FT_REQUIRE(aligned(x, 16) && aligned(y_rows, 16) && (!y_shared || aligned(y_shared, 16)) &&
                 aligned(workspace, 16),
             "ft_moe_grouped_ffn: x, y_rows, y_shared, workspace must be 16-byte aligned");
  const size_t need = ffn_workspace_bytes(T, k, E, H, I);
  FT_REQUIRE(workspace != nullptr && workspace_bytes >= need,
             "ft_moe_grouped_ffn: workspace too small (see ft_workspace_bytes)");
  return FT_OK;
}

extern "C" ft_status ft_moe_grouped_ffn(const ft_expert_layout *L, const void *slot_pool, int32_t n_slots,
                                        const int32_t *slot_of_expert, const void *shared_blob,
                                        const void *x, int32_t x_dtype, int32_t T, int32_t k,
                                        int32_t E, const int32_t *expert_offsets,
                                        const int32_t *sorted_rows, float *y_rows, float *y_shared,
                                        int32_t mode, void *workspace, size_t workspace_bytes,
                                        hipStream_t stream) {
  const ft_status cst = ffn_check(L, slot_pool, n_slots, slot_of_expert, shared_blob, x, x_dtype, T, k, E,
                                  expert_offsets, sorted_rows, y_rows, y_shared, mode, workspace, workspace_bytes);
  if (cst != FT_OK) return cst;
  if (T == 0) {
    clear_error();
    return FT_OK;
  }
  const int stages = mode & (FT_FFN_GATE_UP_ONLY | FT_FFN_DOWN_ONLY);
  const int variant = mode & 0xff;
  const bool run1 = stages != FT_FFN_DOWN_ONLY, run2 = stages != FT_FFN_GATE_UP_ONLY;
  const int H = L->H, I = L->I;
  const int wd = L->wdtype;

  const bool has_shared = shared_blob != nullptr;
  const int routed = T * k;
  const int rows = routed + (has_shared ? T : 0);

  if (variant == FT_FFN_NATIVE_MX) {
    const MxWorkspace W = mx_workspace_layout(T, k, H, I);
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    GemmArgs g1{};
    g1.pool = static_cast<const uint8_t *>(slot_pool);
    g1.slot_of_expert = slot_of_expert;
    g1.n_slots = n_slots;
    g1.expert_bytes = L->expert_bytes;
    g1.shared_blob = static_cast<const uint8_t *>(shared_blob);
    g1.offsets = expert_offsets;
    g1.E = E;
    g1.T = T;
    g1.k = k;
    GemmArgs g2 = g1;
    g1.off_w0 = L->off_gate;
    g1.off_w1 = L->off_up;
    g1.off_s0 = L->off_sgate;
    g1.off_s1 = L->off_sup;
    g1.K = H;
    g1.N = I;
    g1.sorted_rows = sorted_rows;
    g1.out = ws + W.h;
    g1.ldo = I;
    g2.off_w0 = g2.off_w1 = L->off_down;
    g2.off_s0 = g2.off_s1 = L->off_sdown;
    g2.K = I;
    g2.N = H;
    g2.sorted_rows = nullptr;
    g2.out = y_rows;
    g2.ldo = H;
    g2.out_shared = y_shared;
    MxGemmArgs m1{g1, ws + W.xq, ws + W.xs, uint32_t(uint64_t(T) * H), uint32_t(uint64_t(T) * H / 32)};
    MxGemmArgs m2{g2, ws + W.hq, ws + W.hs, uint32_t(uint64_t(rows) * I), uint32_t(uint64_t(rows) * I / 32)};
    ft_status st = FT_OK;
    if (run1) {
      if ((st = mx_quantize_launch(static_cast<const uint16_t *>(x), H, T, H, ws + W.xq, ws + W.xs, stream)) != FT_OK)
        return st;
      if ((st = launch_mx_gemm<true>(m1, stream, "ffn_mx_gemm_kernel<gate_up>")) != FT_OK) return st;
    }
    if (run2) {
      if ((st = mx_quantize_launch(reinterpret_cast<const uint16_t *>(ws + W.h), I, rows, I, ws + W.hq, ws + W.hs,
                                   stream)) != FT_OK)
        return st;
      if ((st = launch_mx_gemm<false>(m2, stream, "ffn_mx_gemm_kernel<down>")) != FT_OK) return st;
    }
    clear_error();
    return FT_OK;
  }

  if (wd == FT_F32) {
    FfnF32Args a{};
    a.pool = static_cast<const uint8_t *>(slot_pool);
    a.slot_of_expert = slot_of_expert;
    a.n_slots = n_slots;
    a.expert_bytes = L->expert_bytes;
    a.shared_blob = static_cast<const uint8_t *>(shared_blob);
    a.off_gate = L->off_gate;
    a.off_up = L->off_up;
    a.off_down = L->off_down;
    a.H = H;
    a.I = I;
    a.offsets = expert_offsets;
    a.E = E;
    a.T = T;
    a.k = k;
    a.sorted_rows = sorted_rows;
    a.x = static_cast<const float *>(x);
    a.h = static_cast<float *>(workspace);
    a.y_rows = y_rows;
    a.y_shared = y_shared;
    a.rows = rows;
    const int64_t n1 = int64_t(rows) * I, n2 = int64_t(rows) * H;
    if (run1) {
      hipLaunchKernelGGL(ffn_f32_stage1, dim3(unsigned(cdiv<int64_t>(n1, 256))), dim3(256), 0, stream, a);
      FT_LAUNCHED("ffn_f32_stage1");
    }
    if (run2) {
      hipLaunchKernelGGL(ffn_f32_stage2, dim3(unsigned(cdiv<int64_t>(n2, 256))), dim3(256), 0, stream, a);
      FT_LAUNCHED("ffn_f32_stage2");
    }
    clear_error();
    return FT_OK;
  }

  const int a_max = std::min(E, routed) + (has_shared ? 1 : 0);
  FfnArgs a{};
  a.pool = static_cast<const uint8_t *>(slot_pool);
  a.slot_of_expert = slot_of_expert;
  a.n_slots = n_slots;
  a.expert_bytes = L->expert_bytes;
  a.shared_blob = static_cast<const uint8_t *>(shared_blob);
  a.offsets = expert_offsets;
  a.E = E;
  a.T = T;
  a.k = k;
  a.sorted_rows = sorted_rows;
  a.has_shared = has_shared ? 1 : 0;
  uint16_t *hbuf = static_cast<uint16_t *>(workspace);

  // stage 1: gate/up + SwiGLU -> h [rows, I] bf16
  FfnArgs s1 = a;
  s1.off_w0 = L->off_gate;
  s1.off_w1 = L->off_up;
  s1.off_s0 = L->off_sgate;
  s1.off_s1 = L->off_sup;
  s1.K = H;
  s1.N = I;
  s1.X = static_cast<const uint16_t *>(x);
  s1.ldx = H;
  s1.x_bytes = uint32_t(uint64_t(T) * H * 2);
  s1.out = hbuf;
  s1.ldo = I;
  s1.n_tiles = cdiv(I, 16);
  // stage 2: down -> y_rows / y_shared fp32
  FfnArgs s2 = a;
  s2.off_w0 = L->off_down;
  s2.off_w1 = L->off_down;
  s2.off_s0 = L->off_sdown;
  s2.off_s1 = L->off_sdown;
  s2.K = I;
  s2.N = H;
  s2.X = hbuf;
  s2.ldx = I;
  s2.x_bytes = uint32_t(uint64_t(rows) * I * 2);
  s2.out = y_rows;
  s2.ldo = H;
  s2.out_shared = y_shared;
  s2.n_tiles = cdiv(H, 16);

  // Decode batches: persistent weight-streaming kernels.
  if (T <= 64 && E <= kPersistMaxE && T * k <= kPersistMaxRows) {
    PersistArgs p1{};
    p1.pool = a.pool;
    p1.slot_of_expert = slot_of_expert;
    p1.n_slots = n_slots;
    p1.expert_bytes = L->expert_bytes;
    p1.shared_blob = a.shared_blob;
    p1.offsets = expert_offsets;
    p1.E = E;
    p1.T = T;
    p1.k = k;
    PersistArgs p2 = p1;
    p1.off_w0 = L->off_gate;
    p1.off_w1 = L->off_up;
    p1.off_s0 = L->off_sgate;
    p1.off_s1 = L->off_sup;
    p1.off_t0 = L->off_tscale;
    p1.off_t1 = L->off_tscale + 4;
    p1.K = H;
    p1.N = I;
    p1.sorted_rows = sorted_rows;
    p1.X = static_cast<const uint16_t *>(x);
    p1.ldx = H;
    p1.x_bytes = uint32_t(uint64_t(T) * H * 2);
    p1.out = hbuf;
    p1.ldo = I;
    p1.n_tiles = cdiv(I, 16);
    p2.off_w0 = p2.off_w1 = L->off_down;
    p2.off_s0 = p2.off_s1 = L->off_sdown;
    p2.off_t0 = p2.off_t1 = L->off_tscale + 8;
    p2.K = I;
    p2.N = H;
    p2.sorted_rows = nullptr;
    p2.X = hbuf;
    p2.ldx = I;
    p2.x_bytes = uint32_t(uint64_t(rows) * I * 2);
    p2.out = y_rows;
    p2.ldo = H;
    p2.out_shared = y_shared;
    p2.n_tiles = cdiv(H, 16);
    const int groups = cdiv(T, 16);
    // stage by stage; a contraction length no persistent shape covers uses the general kernel
    // (NVFP4 has none: such shapes are not supported)
    if (wd == FT_NVFP4) {
      FT_SUPPORTED((!run1 || persist_covers<WF_NV4>(p1.K)) && (!run2 || persist_covers<WF_NV4>(p2.K)),
                   "ft_moe_grouped_ffn: NVFP4 decode needs H/128 and I/128 in {4, 6, 8, 12, 16}");
      // a tuning override naming a shape with no kernel instance launches nothing: refuse rather
      // than leave the stage's outputs unwritten
      if (run1 && !launch_persist<WF_NV4, true>(p1, a_max * p1.n_tiles * groups, stream))
        return fail(FT_ENOTSUP, "ft_moe_grouped_ffn: no NVFP4 gate/up kernel for this persistent shape");
      if (run2 && !launch_persist<WF_NV4, false>(p2, a_max * p2.n_tiles * groups, stream))
        return fail(FT_ENOTSUP, "ft_moe_grouped_ffn: no NVFP4 down kernel for this persistent shape");
    } else if (wd == FT_BF16) {
      if (run1 && !launch_persist<WF_BF16, true>(p1, a_max * p1.n_tiles * groups, stream)) {
        const ft_status st = launch_stream<WF_BF16, true>(s1, a_max, T, stream, "ffn_stream_kernel<bf16, gate_up>");
        if (st != FT_OK) return st;
      }
      if (run2 && !launch_persist<WF_BF16, false>(p2, a_max * p2.n_tiles * groups, stream)) {
        const ft_status st = launch_stream<WF_BF16, false>(s2, a_max, T, stream, "ffn_stream_kernel<bf16, down>");
        if (st != FT_OK) return st;
      }
    } else {
      if (run1 && !launch_persist<WF_FP4, true>(p1, a_max * p1.n_tiles * groups, stream)) {
        const ft_status st = launch_stream<WF_FP4, true>(s1, a_max, T, stream, "ffn_stream_kernel<mxfp4, gate_up>");
        if (st != FT_OK) return st;
      }
      if (run2 && !launch_persist<WF_FP4, false>(p2, a_max * p2.n_tiles * groups, stream)) {
        const ft_status st = launch_stream<WF_FP4, false>(s2, a_max, T, stream, "ffn_stream_kernel<mxfp4, down>");
        if (st != FT_OK) return st;
      }
    }
    FT_LAUNCHED("ffn_persist_kernel");
    clear_error();
    return FT_OK;
  }
  // Prefill: grouped MFMA GEMM tiles (K a multiple of the 128-element chunk).
  if (H % kGemmBK == 0 && I % kGemmBK == 0) {
    GemmArgs g1{};
    g1.pool = a.pool;
    g1.slot_of_expert = slot_of_expert;
    g1.n_slots = n_slots;
    g1.expert_bytes = L->expert_bytes;
    g1.shared_blob = a.shared_blob;
    g1.offsets = expert_offsets;
    g1.E = E;
    g1.T = T;
    g1.k = k;
    GemmArgs g2 = g1;
    g1.off_w0 = L->off_gate;
    g1.off_w1 = L->off_up;
    g1.off_s0 = L->off_sgate;
    g1.off_s1 = L->off_sup;
    g1.off_t0 = L->off_tscale;
    g1.off_t1 = L->off_tscale + 4;
    g1.K = H;
    g1.N = I;
    g1.sorted_rows = sorted_rows;
    g1.X = static_cast<const uint16_t *>(x);
    g1.ldx = H;
    g1.x_bytes = s1.x_bytes;
    g1.out = hbuf;
    g1.ldo = I;
    g2.off_w0 = g2.off_w1 = L->off_down;
    g2.off_s0 = g2.off_s1 = L->off_sdown;
    g2.off_t0 = g2.off_t1 = L->off_tscale + 8;
    g2.K = I;
    g2.N = H;
    g2.sorted_rows = nullptr;
    g2.X = hbuf;
    g2.ldx = I;
    g2.x_bytes = s2.x_bytes;
    g2.out = y_rows;
    g2.ldo = H;
    g2.out_shared = y_shared;
    ft_status st = FT_OK;
    if (wd == FT_BF16) {
      if (run1 && (st = launch_gemm<WF_BF16, true>(g1, stream, "ffn_gemm_kernel<bf16, gate_up>")) != FT_OK) return st;
      if (run2 && (st = launch_gemm<WF_BF16, false>(g2, stream, "ffn_gemm_kernel<bf16, down>")) != FT_OK) return st;
    } else if (wd == FT_NVFP4) {
      if (run1 && (st = launch_gemm<WF_NV4, true>(g1, stream, "ffn_gemm_kernel<nvfp4, gate_up>")) != FT_OK) return st;
      if (run2 && (st = launch_gemm<WF_NV4, false>(g2, stream, "ffn_gemm_kernel<nvfp4, down>")) != FT_OK) return st;
    } else {
      if (run1 && (st = launch_gemm<WF_FP4, true>(g1, stream, "ffn_gemm_kernel<mxfp4, gate_up>")) != FT_OK) return st;
      if (run2 && (st = launch_gemm<WF_FP4, false>(g2, stream, "ffn_gemm_kernel<mxfp4, down>")) != FT_OK) return st;
    }
    clear_error();
    return FT_OK;
  }
  ft_status st = FT_OK;
  if (wd == FT_BF16) {
    if (run1 && (st = launch_stream<WF_BF16, true>(s1, a_max, T, stream, "ffn_stream_kernel<bf16, gate_up>")) != FT_OK)
      return st;
    if (run2 && (st = launch_stream<WF_BF16, false>(s2, a_max, T, stream, "ffn_stream_kernel<bf16, down>")) != FT_OK)
      return st;
  } else {
    if (run1 && (st = launch_stream<WF_FP4, true>(s1, a_max, T, stream, "ffn_stream_kernel<mxfp4, gate_up>")) != FT_OK)
      return st;
    if (run2 && (st = launch_stream<WF_FP4, false>(s2, a_max, T, stream, "ffn_stream_kernel<mxfp4, down>")) != FT_OK)
      return st;
  }
  clear_error();
  return FT_OK;
}

// ------------------------------------------------------------------ the whole layer in one call

// The routing's completion counter (route_permute_counted) in the layer call's zeroed wait area: the
// line after the one-token kernel's grid-wide wait words.
constexpr int kLayerRouteWord = kWaitStride * (2 * kWaitGroups + 1);
static_assert((kLayerRouteWord + 1) * 4 <= int(kLayerWaitBytes), "the routing counter fits the wait area");

extern "C" ft_status ft_moe_layer(const ft_expert_layout *L, const void *slot_pool, int32_t n_slots,
                                  const int32_t *slot_of_expert, const void *shared_blob, const void *x,
                                  int32_t x_dtype, const void *w_router, float *logits, int32_t T, int32_t E,
                                  int32_t k, int32_t gating, int32_t renormalize, int32_t *topk_ids, float *topk_w,
                                  int32_t *expert_offsets, int32_t *sorted_rows, int32_t *row_pos, float *y_rows,
                                  float *y_shared, int32_t mode, int32_t out_dtype, void *out, void *workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
  // every step's checks before anything is enqueued
  FT_REQUIRE(L != nullptr, "ft_moe_layer: layout is NULL");
  FT_REQUIRE((mode & ~0xff) == 0, "ft_moe_layer: stage bits are not taken (the call runs the whole layer)");
  FT_REQUIRE(out_dtype == FT_F32 || out_dtype == FT_BF16, "ft_moe_layer: out_dtype must be FT_F32 or FT_BF16");
  ft_status st = route_logits(x, x_dtype, w_router, logits, T, L->H, E, k, gating, topk_ids, topk_w, stream, false);
  if (st != FT_OK) return st;
  FT_SUPPORTED(k <= 64, "ft_moe_layer: k > 64");
  FT_SUPPORTED(L->H % 4 == 0, "ft_moe_layer: H must be a multiple of 4");
  FT_REQUIRE(T <= 65535, "ft_moe_layer: T > 65535");
  if (T > 0) {
    FT_REQUIRE(expert_offsets && sorted_rows && row_pos && out && aligned(out, 16),
               "ft_moe_layer: NULL or misaligned permutation or output buffer");
    FT_REQUIRE(workspace != nullptr && aligned(workspace, 256) &&
                   workspace_bytes >= kLayerWaitBytes + permute_workspace_bytes(T, k, E),
               "ft_moe_layer: workspace NULL, not 256-byte aligned or too small "
               "(see ft_workspace_bytes(FT_WS_LAYER, ...))");
  }
  // the wait words first, then the workspace of the steps
  uint32_t *wait_words = static_cast<uint32_t *>(workspace);
  void *ws = T > 0 ? static_cast<uint8_t *>(workspace) + kLayerWaitBytes : workspace;
  const size_t ws_bytes = T > 0 ? workspace_bytes - kLayerWaitBytes : workspace_bytes;
  st = ffn_check(L, slot_pool, n_slots, slot_of_expert, shared_blob, x, x_dtype, T, k, E, expert_offsets,
                 sorted_rows, y_rows, y_shared, mode, ws, ws_bytes);
  if (st != FT_OK) return st;
  if (T == 0) {
    clear_error();
    return FT_OK;
  }
  const int H = L->H, I = L->I, wd = L->wdtype;
  const bool has_shared = shared_blob != nullptr;
  int w1 = 0, c1 = 0, w2 = 0, c2 = 0;
  const bool shapes = wd == FT_BF16   ? fused_shape<WF_BF16>(true, H / stream_kblock<WF_BF16>(), &w1, &c1) &&
                                          fused_shape<WF_BF16>(false, I / stream_kblock<WF_BF16>(), &w2, &c2)
                      : wd == FT_MXFP4 ? fused_shape<WF_FP4>(true, H / stream_kblock<WF_FP4>(), &w1, &c1) &&
                                          fused_shape<WF_FP4>(false, I / stream_kblock<WF_FP4>(), &w2, &c2)
                      : wd == FT_NVFP4 ? fused_shape<WF_NV4>(true, H / stream_kblock<WF_NV4>(), &w1, &c1) &&
                                          fused_shape<WF_NV4>(false, I / stream_kblock<WF_NV4>(), &w2, &c2)
                                       : false;
  const bool exact = (mode & 0xff) == FT_FFN_EXACT;
  const bool gemv = T == 1 && exact &&
                    (wd == FT_BF16    ? token_gemv_covers<WF_BF16>(H, I, E, k, has_shared)
                     : wd == FT_MXFP4 ? token_gemv_covers<WF_FP4>(H, I, E, k, has_shared)
                     : wd == FT_NVFP4 ? token_gemv_covers<WF_NV4>(H, I, E, k, has_shared)
                                      : false);
  const bool fused = gemv || (T <= kRouteMaxT && exact && shapes && E <= kRouteMaxE && k <= kFusedMaxK &&
                              T * k <= kRouteMaxRows && w1 >= T);
  if (!fused) {
    // route + permute, the grouped FFN and the combine, one call after the other (the router split
    // over the hidden axis when it covers the batch: its partial planes use the FFN's workspace, free
    // until the gate/up stage; FTMOE_ROUTER_SPLIT = "0" keeps the one-pass router)
    static const char *split_env = getenv("FTMOE_ROUTER_SPLIT");
    const int parts = (split_env && split_env[0] == '0') ? 0 : router_split_parts(x, x_dtype, w_router, T, H, E, k, ws_bytes);
    st = parts > 0 ? route_permute_split(x, w_router, logits, T, H, E, k, gating, renormalize, topk_ids, topk_w,
                                         expert_offsets, sorted_rows, row_pos, parts, ws, wait_words + kLayerRouteWord,
                                         stream)
         : route_permute_counted_covers(T, k, E)
             ? route_permute_counted(x, x_dtype, w_router, logits, T, H, E, k, gating, renormalize, topk_ids, topk_w,
                                     expert_offsets, sorted_rows, row_pos, wait_words + kLayerRouteWord, stream)
             : ft_moe_route_permute(x, x_dtype, w_router, logits, T, H, E, k, gating, renormalize, topk_ids, topk_w,
                                    expert_offsets, sorted_rows, row_pos, ws, ws_bytes, stream);
    if (st != FT_OK) return st;
    st = ft_moe_grouped_ffn(L, slot_pool, n_slots, slot_of_expert, shared_blob, x, x_dtype, T, k, E,
                            expert_offsets, sorted_rows, y_rows, y_shared, mode, ws, ws_bytes, stream);
    if (st != FT_OK) return st;
    return ft_moe_combine(y_rows, topk_w, row_pos, y_shared, T, k, H, out_dtype, out, stream);
  }
  // A few tokens: the router, then gate/up with top-k, gating and the permutation done in every
  // workgroup (the routing kernel's launch saved), then the down projection with the combine folded
  // in (the combine's launch and the y rows' round trip saved).  y_rows / y_shared are not written.
  st = route_logits(x, x_dtype, w_router, logits, T, H, E, k, gating, topk_ids, topk_w, stream, true);
  if (st != FT_OK) return st;
  const int rows = T * k + (has_shared ? T : 0);
  uint16_t *hbuf = static_cast<uint16_t *>(ws);
  PersistArgs p1{};
  p1.pool = static_cast<const uint8_t *>(slot_pool);
  p1.slot_of_expert = slot_of_expert;
  p1.n_slots = n_slots;
  p1.expert_bytes = L->expert_bytes;
  p1.shared_blob = static_cast<const uint8_t *>(shared_blob);
  p1.E = E;
  p1.T = T;
  p1.k = k;
  PersistArgs p2 = p1;
  p1.off_w0 = L->off_gate;
  p1.off_w1 = L->off_up;
  p1.off_s0 = L->off_sgate;
  p1.off_s1 = L->off_sup;
  p1.off_t0 = L->off_tscale;
  p1.off_t1 = L->off_tscale + 4;
  p1.K = H;
  p1.N = I;
  p1.X = static_cast<const uint16_t *>(x);
  p1.ldx = H;
  p1.x_bytes = uint32_t(uint64_t(T) * H * 2);
  p1.out = hbuf;
  p1.ldo = I;
  p1.logits = logits;
  p1.gating = gating;
  p1.renorm = renormalize ? 1 : 0;
  p1.ids_out = topk_ids;
  p1.w_out = topk_w;
  p1.off_out = expert_offsets;
  p1.rows_out = sorted_rows;
  p1.pos_out = row_pos;
  p2.off_w0 = p2.off_w1 = L->off_down;
  p2.off_s0 = p2.off_s1 = L->off_sdown;
  p2.off_t0 = p2.off_t1 = L->off_tscale + 8;
  p2.K = I;
  p2.N = H;
  p2.X = hbuf;
  p2.ldx = I;
  p2.x_bytes = uint32_t(uint64_t(rows) * I * 2);
  p2.ids = topk_ids;
  p2.topk_w = topk_w;
  p2.row_pos = row_pos;
  p2.comb_out = out;
  p2.comb_bf16 = out_dtype == FT_BF16 ? 1 : 0;
  p2.ldo = H;
  if (gemv) {  // one token: the matrix-vector kernels
    st = wd == FT_BF16    ? launch_token_gemv<WF_BF16>(p1, p2, wait_words, stream)
         : wd == FT_MXFP4 ? launch_token_gemv<WF_FP4>(p1, p2, wait_words, stream)
                          : launch_token_gemv<WF_NV4>(p1, p2, wait_words, stream);
    if (st != FT_OK) return st;
    clear_error();
    return FT_OK;
  }
  const int units1 = (std::min(E, T * k) + (has_shared ? 1 : 0)) * cdiv(I, 16);  // 16-row gate/up units, at most
  const int units2 = T * cdiv(H, 16);
  if (wd == FT_BF16) {
    if ((st = launch_fused<WF_BF16, true>(p1, units1, 1, stream)) != FT_OK) return st;
    st = launch_fused<WF_BF16, false>(p2, units2, 1, stream);
  } else if (wd == FT_MXFP4) {
    if ((st = launch_fused<WF_FP4, true>(p1, units1, 1, stream)) != FT_OK) return st;
    st = launch_fused<WF_FP4, false>(p2, units2, 1, stream);
  } else {
    if ((st = launch_fused<WF_NV4, true>(p1, units1, 1, stream)) != FT_OK) return st;
    st = launch_fused<WF_NV4, false>(p2, units2, 1, stream);
  }
  if (st != FT_OK) return st;
  clear_error();
  return FT_OK;
}

// ------------------------------------------------------------------ no-allocation variant
//
// ft_moe_grouped_ffn_noalloc: the same call with its workspace in a static
// device array, for callers that cannot allocate (code under graph capture,
// tight serving loops, harnesses that forbid hipMalloc).  The array is
// `scratch`; in host code its name is only a stand-in, so its device address
// on each GPU is resolved once with hipGetSymbolAddress (with that GPU
// current) and only that address is passed to kernels.  Nothing in it must
// start at zero: the FFN's kernels write every hidden row (and quantized
// operand) before they read it.
namespace ft {
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;  // per GPU
constexpr int kMaxScratchDevices = 64;
}  // namespace ft

static __device__ __align__(256) uint8_t scratch[ft::kNoAllocScratchBytes];

namespace {
std::mutex g_scratch_mu;
void *g_scratch_dev[ft::kMaxScratchDevices];  // device address of `scratch` on GPU d
}  // namespace

static ft_status scratch_address(void **out) {
  int dev = 0;
  FT_HIP(hipGetDevice(&dev));
  FT_SUPPORTED(dev >= 0 && dev < kMaxScratchDevices, "ft_moe_grouped_ffn_noalloc: device index above 63");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    void *p = nullptr;
    FT_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    FT_REQUIRE(p != nullptr && aligned(p, 256), "ft_moe_grouped_ffn_noalloc: scratch address not resolved");
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return FT_OK;
}

extern "C" size_t ft_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

extern "C" ft_status ft_moe_grouped_ffn_noalloc(const ft_expert_layout *L, const void *slot_pool, int32_t n_slots,
                                                const int32_t *slot_of_expert, const void *shared_blob,
                                                const void *x, int32_t x_dtype, int32_t T, int32_t k, int32_t E,
                                                const int32_t *expert_offsets, const int32_t *sorted_rows,
                                                float *y_rows, float *y_shared, int32_t mode, hipStream_t stream) {
  FT_REQUIRE(L != nullptr, "ft_moe_grouped_ffn_noalloc: layout is NULL");
  FT_REQUIRE(T >= 0 && k >= 1 && E >= 1 && L->H >= 1 && L->I >= 1,
             "ft_moe_grouped_ffn_noalloc: need T >= 0, k >= 1, E >= 1 and an initialised layout");
  FT_REQUIRE(int64_t(T) * (k + 1) < (int64_t(1) << 31), "ft_moe_grouped_ffn_noalloc: T*k too large");
  const size_t need = ffn_workspace_bytes(T, k, E, L->H, L->I);
  if (need > kNoAllocScratchBytes)
    return fail(FT_ECAPACITY, "ft_moe_grouped_ffn_noalloc: this call needs " + std::to_string(need) +
                                  " bytes of scratch, above the static " + std::to_string(kNoAllocScratchBytes) +
                                  " (use ft_moe_grouped_ffn with a workspace)");
  void *ws = nullptr;
  const ft_status st = scratch_address(&ws);
  if (st != FT_OK) return st;
  return ft_moe_grouped_ffn(L, slot_pool, n_slots, slot_of_expert, shared_blob, x, x_dtype, T, k, E, expert_offsets,
                            sorted_rows, y_rows, y_shared, mode, ws, kNoAllocScratchBytes, stream);
}
