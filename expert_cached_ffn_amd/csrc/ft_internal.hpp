// Internal helpers shared by the gfx950 kernels and the C-ABI entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>
#include <string>

#include "../../include/ft_moe.h"

// ---------------------------------------------------------------------------
// host-side status handling
// ---------------------------------------------------------------------------
namespace ft {

// Bytes at the start of the layer call's workspace reserved for the one-token
// kernel's grid-wide wait (counters on separate 128-byte lines); the rest of
// the workspace follows.
constexpr size_t kLayerWaitBytes = 8192;

void set_error(const std::string &msg);
void clear_error();

inline ft_status fail(ft_status st, const std::string &msg) {
  set_error(msg);
  return st;
}

inline bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Workspace sizes (bytes) of the calls that take one.
size_t permute_workspace_bytes(int32_t T, int32_t k, int32_t E);
size_t ffn_workspace_bytes(int32_t T, int32_t k, int32_t E, int32_t H, int32_t I);

// Validates the routing arguments of ft_moe_route and (launch) enqueues the
// router logits when w_router != NULL; nothing else.
ft_status route_logits(const void *x, int32_t x_dtype, const void *w_router, float *logits, int32_t T, int32_t H,
                       int32_t E, int32_t k, int32_t gating, int32_t *topk_ids, float *topk_w, hipStream_t stream,
                       bool launch = true);

// The routing of ft_moe_route_permute as two launches after the router instead of three (top-k over
// the grid, the permutation by its last workgroup) for decode batches of more than 16 tokens with at
// most 1024 routed rows over at most 256 experts; `done` is a zeroed counter, left zero.  Arguments
// are those of ft_moe_route_permute, checked by the caller.
bool route_permute_counted_covers(int T, int k, int E);
int router_split_parts(const void *x, int32_t x_dtype, const void *w_router, int T, int H, int E, int k,
                       size_t ws_bytes);
ft_status route_permute_split(const void *x, const void *w_router, float *logits, int32_t T, int32_t H, int32_t E,
                              int32_t k, int32_t gating, int32_t renormalize, int32_t *topk_ids, float *topk_w,
                              int32_t *expert_offsets, int32_t *sorted_rows, int32_t *row_pos, int parts, void *ws,
                              uint32_t *done, hipStream_t stream);
ft_status route_permute_counted(const void *x, int32_t x_dtype, const void *w_router, float *logits, int32_t T,
                                int32_t H, int32_t E, int32_t k, int32_t gating, int32_t renormalize,
                                int32_t *topk_ids, float *topk_w, int32_t *expert_offsets, int32_t *sorted_rows,
                                int32_t *row_pos, uint32_t *done, hipStream_t stream);

}  // namespace ft

#define FT_REQUIRE(cond, msg)                                   \
  do {                                                          \
    if (!(cond)) return ft::fail(FT_EINVAL, std::string(msg));  \
  } while (0)

#define FT_SUPPORTED(cond, msg)                                  \
  do {                                                           \
    if (!(cond)) return ft::fail(FT_ENOTSUP, std::string(msg));  \
  } while (0)

#define FT_HIP(expr)                                                                    \
  do {                                                                                  \
    hipError_t e_ = (expr);                                                             \
    if (e_ != hipSuccess)                                                               \
      return ft::fail(FT_EHIP, std::string(#expr) + ": " + hipGetErrorString(e_));      \
  } while (0)

// Check the launch that was just enqueued.
#define FT_LAUNCHED(name)                                                               \
  do {                                                                                  \
    hipError_t e_ = hipGetLastError();                                                  \
    if (e_ != hipSuccess)                                                               \
      return ft::fail(FT_EHIP, std::string("launch of ") + name + ": " + hipGetErrorString(e_)); \
  } while (0)

// ---------------------------------------------------------------------------
// device-side types and helpers
// ---------------------------------------------------------------------------
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((ext_vector_type(8))) int32_t i32x8;

namespace ft {

// fp32 -> bf16 bits, round to nearest even (NaN -> quiet NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t b = __float_as_uint(f);
  if ((b & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  b += 0x7fffu + ((b >> 16) & 1u);
  return static_cast<uint16_t>(b >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// E8M0 scale byte -> fp32 2^(s-127) for s in 1..254 (the exponent field itself).
__device__ __forceinline__ float e8m0_to_f32(uint32_t s) { return __uint_as_float(s << 23); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
// One dword as a bf16 pair.  Takes the dword by value: __builtin_bit_cast applied directly to an
// element of a u32x4 (v[i]) compiles to a read of element 0 whatever i is.
__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t v) { return __builtin_bit_cast(bf16x2, v); }

// Eight FP4 E2M1 codes (one dword, element 2i in the low nibble of byte i)
// times a power-of-two scale -> eight bf16, in element order.
__device__ __forceinline__ bf16x8 fp4x8_to_bf16x8(uint32_t codes, float scale) {
  bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 0);
  bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 1);
  bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 2);
  bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 3);
  bf16x8 r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// FP8 E4M3 code (OCP, the low byte of `b`) -> fp32: v_cvt_f32_fp8 on gfx950
// decodes OCP E4M3 (checked against the bit-field definition on all 256 codes).
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) { return __builtin_amdgcn_cvt_f32_fp8(int(b), 0); }

// Eight NVFP4 codes (one dword) times an E4M3 block scale -> eight bf16.  The
// scaled conversion instructions take only the exponent of their scale, so
// the codes are converted to fp32 unscaled and multiplied by the full scale;
// every E2M1 x E4M3 product has at most 6 significant bits, so the multiply
// and the bf16 packing are exact.
__device__ __forceinline__ bf16x8 nvfp4x8_to_bf16x8(uint32_t codes, float scale) {
  const auto p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 0);
  const auto p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 1);
  const auto p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 2);
  const auto p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 3);
  bf16x8 r;
  r[0] = static_cast<__bf16>(p0[0] * scale);
  r[1] = static_cast<__bf16>(p0[1] * scale);
  r[2] = static_cast<__bf16>(p1[0] * scale);
  r[3] = static_cast<__bf16>(p1[1] * scale);
  r[4] = static_cast<__bf16>(p2[0] * scale);
  r[5] = static_cast<__bf16>(p2[1] * scale);
  r[6] = static_cast<__bf16>(p3[0] * scale);
  r[7] = static_cast<__bf16>(p3[1] * scale);
  return r;
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Block-scaled MFMA (OCP MX): D += (A * 2^(sa-127)) (B * 2^(sb-127)) over 128
// contraction elements, A = 16 rows of FP8 E4M3, B = 16 columns of FP4 E2M1.
// Operand lanes (l = 16 g + r): A lane holds row r at elements 16g..16g+15
// (bytes 0..15) and 64+16g..64+16g+15 (bytes 16..31); B lane holds column r at
// elements 32g..32g+31 (16 bytes, element 2i in the low nibble of byte i; the
// upper four dwords are unused); the scale byte OPA of `sa` / OPB of `sb` in
// lane (r, g) is the E8M0 scale of row / column r, elements 32g..32g+31.
// Output lane (r, g) holds D[4g + v][r], v = 0..3.
template <int OPA = 0, int OPB = 0>
__device__ __forceinline__ f32x4 mfma_mx(i32x8 a, i32x8 b, f32x4 c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 4, OPA, sa, OPB, sb);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// Slot of expert e in a slot table (NULL: slot e).  A value at or past the
// pool's n_slots reads as -1, like any slot of an expert that is not
// resident, so a bad table never addresses memory outside the pool.
__device__ __forceinline__ int table_slot(const int32_t *slot_of_expert, int e, int n_slots) {
  const int s = slot_of_expert ? slot_of_expert[e] : e;
  return s >= n_slots ? -1 : s;
}

// Raw buffer loads (gfx9 descriptor: 32-bit data format word 0x00020000).  An
// offset at or past `bytes` returns zero and touches no memory, which is how
// padding rows and token columns are masked without branches.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 bld16(rsrc_t r, uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0); }
__device__ __forceinline__ u32x2 bld8(rsrc_t r, uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0); }
// A 16-byte load of bytes read once per call, with the non-temporal bit: for loads that take whole
// 128-byte lines (a plain 1 GiB read: 6.4 against 5.9 TB/s).  Loads that take half a line must not
// use it: the line's other half, read by the next load, then came from HBM again (measured: the
// multi-token decode kernels' gate/up fell from 5.6 to 4.8 TB/s).
__device__ __forceinline__ u32x4 bld16nt(rsrc_t r, uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2); }

__device__ __forceinline__ uint32_t bld4(rsrc_t r, uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0); }
constexpr uint32_t kOOB = 0x80000000u;  // an offset past every buffer used here

// s_waitcnt for vector-memory operations only: at most N still outstanding
// (gfx9 encoding: vmcnt bits 3:0 and 15:14; expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier without the vector-memory part of __syncthreads()'s fence:
// that would wait for every direct-to-LDS load in flight, including those
// meant to stay in flight across the barrier.  Callers wait (vmcnt) for the
// loads the other waves must see before calling it.  This wave's own LDS
// reads do complete first (lgkmcnt 0): another wave may overwrite the buffer
// as soon as it passes.  The empty asm statements keep the compiler from
// moving memory accesses across.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0), vmcnt/expcnt untouched
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// 16-byte global load/store helpers.
__device__ __forceinline__ u32x4 ld16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }
__device__ __forceinline__ void st16(void *p, u32x4 v) { *reinterpret_cast<u32x4 *>(p) = v; }

template <typename T>
__host__ __device__ __forceinline__ T cdiv(T a, T b) { return (a + b - 1) / b; }

// ---- wave-wide reductions and scans on DPP lane moves.  A shuffle through
// ds_bpermute is an LDS round trip; the reductions below stay in the VALU.
// Every lane of the wave must be active.  DPP controls used: quad_perm
// [1,0,3,2] (0xB1) and [2,3,0,1] (0x4E), row_shr:n (0x110 + n), row_ror:n
// (0x120 + n), row_mirror (0x140), row_half_mirror (0x141), row_bcast:15
// (0x142, written to rows 1 and 3) and row_bcast:31 (0x143, rows 2 and 3).
// A lane whose source is outside its row, or whose row is masked off, gets
// `old`.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t old, uint32_t src) {
  return uint32_t(__builtin_amdgcn_update_dpp(int(old), int(src), CTRL, ROW_MASK, 0xf, false));
}

template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ uint64_t dpp_max_u64_step(uint64_t x) {
  const uint32_t lo = uint32_t(x), hi = uint32_t(x >> 32);
  const uint64_t o = (uint64_t(dpp_u32<CTRL, ROW_MASK>(hi, hi)) << 32) | dpp_u32<CTRL, ROW_MASK>(lo, lo);
  return o > x ? o : x;
}

// Maximum over the wave, in every lane: quads, half rows and rows by
// butterflies (max is idempotent, so mirrors serve), then rows 0+1 and 2+3 by
// broadcasts, the total landing in lane 63.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x) {
  x = dpp_max_u64_step<0xB1>(x);
  x = dpp_max_u64_step<0x4E>(x);
  x = dpp_max_u64_step<0x141>(x);
  x = dpp_max_u64_step<0x140>(x);
  x = dpp_max_u64_step<0x142, 0xA>(x);
  x = dpp_max_u64_step<0x143, 0xC>(x);
  const uint32_t lo = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(x)), 63));
  const uint32_t hi = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(x >> 32)), 63));
  return (uint64_t(hi) << 32) | lo;
}

template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp_f32(float old, float src) {
  return __builtin_bit_cast(float, dpp_u32<CTRL, ROW_MASK>(__builtin_bit_cast(uint32_t, old),
                                                           __builtin_bit_cast(uint32_t, src)));
}

__device__ __forceinline__ float wave_max_f32(float x) {
  x = fmaxf(x, dpp_f32<0xB1>(x, x));
  x = fmaxf(x, dpp_f32<0x4E>(x, x));
  x = fmaxf(x, dpp_f32<0x141>(x, x));
  x = fmaxf(x, dpp_f32<0x140>(x, x));
  x = fmaxf(x, dpp_f32<0x142, 0xA>(x, x));
  x = fmaxf(x, dpp_f32<0x143, 0xC>(x, x));
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = max(x, dpp_u32<0xB1>(x, x));
  x = max(x, dpp_u32<0x4E>(x, x));
  x = max(x, dpp_u32<0x141>(x, x));
  x = max(x, dpp_u32<0x140>(x, x));
  x = max(x, dpp_u32<0x142, 0xA>(x, x));
  x = max(x, dpp_u32<0x143, 0xC>(x, x));
  return uint32_t(__builtin_amdgcn_readlane(int(x), 63));
}

// Sum over the wave, in every lane: quad butterflies, then each lane adds the
// quad 4 and the pair of quads 8 lanes around its row (row sums), then the
// row broadcasts as above.
__device__ __forceinline__ float wave_sum_f32(float x) {
  x += dpp_f32<0xB1>(x, x);
  x += dpp_f32<0x4E>(x, x);
  x += dpp_f32<0x124>(x, x);
  x += dpp_f32<0x128>(x, x);
  x += dpp_f32<0x142, 0xA>(0.f, x);
  x += dpp_f32<0x143, 0xC>(0.f, x);
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}

// Wave sums of N = 2, 4 or 8 values per lane at once (a transposing
// reduction): each permlane swap stage pairs two values and halves what a
// lane holds -- v_permlane32_swap exchanges half-waves, v_permlane16_swap the
// second and fourth 16-lane rows -- and a row-rotate stage does the same for
// N = 8; DPP lane moves then sum inside the 8-, 16- or 32-lane groups that
// share a value.  About 20 instructions for 8 values against 8 x 14 for eight
// separate sums.  Lane l ends with the total of value wave_sums_index<N>(l).
__device__ __forceinline__ void permlane_pair_add(float &a, float b, bool sixteen) {
  const auto r = sixteen ? __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false)
                         : __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  a = __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int N>
__device__ __forceinline__ float wave_sums(const float (&v)[N]) {
  static_assert(N == 2 || N == 4 || N == 8, "2, 4 or 8 values");
  float t[N];
#pragma unroll
  for (int i = 0; i < N; ++i) t[i] = v[i];
  // half-waves: lanes 0-31 keep value 2i of the pair, lanes 32-63 value 2i+1
#pragma unroll
  for (int i = 0; i < N / 2; ++i) {
    t[i] = t[2 * i];
    permlane_pair_add(t[i], t[2 * i + 1], false);
  }
  if constexpr (N >= 4) {  // 16-lane rows: rows 0 / 2 keep the first of the pair, rows 1 / 3 the second
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      t[i] = t[2 * i];
      permlane_pair_add(t[i], t[2 * i + 1], true);
    }
  }
  if constexpr (N == 8) {  // lanes 8-15 of each row keep the second value, taking lane l ^ 8's copy
    const bool hi = (threadIdx.x & 8) != 0;
    const float keep = hi ? t[1] : t[0], send = hi ? t[0] : t[1];
    t[0] = keep + dpp_f32<0x128>(send, send);  // row_ror:8
  }
  float x = t[0];
  x += dpp_f32<0xB1>(x, x);   // lane l ^ 1
  x += dpp_f32<0x4E>(x, x);   // lane l ^ 2
  x += dpp_f32<0x141>(x, x);  // row_half_mirror: the other quad of the 8
  if constexpr (N <= 4) x += dpp_f32<0x128>(x, x);  // row_ror:8: the other 8 of the row
  if constexpr (N == 2) {     // the other row of the half-wave
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  return x;
}

// The value whose total lane `lane` holds after wave_sums<N>.
template <int N>
__device__ __forceinline__ int wave_sums_index(int lane) {
  if constexpr (N == 2) {
    return lane >> 5;
  } else {
    const int g = (lane >> 4) & 3;
    const int m = g == 1 ? 2 : (g == 2 ? 1 : g);  // rows 0, 1, 2, 3 hold values 0, 2, 1, 3 (+ 4j)
    return N == 4 ? m : 4 * ((lane >> 3) & 1) + m;
  }
}

__device__ __forceinline__ int wave_sum_i32(int x) {
  x += int(dpp_u32<0xB1>(uint32_t(x), uint32_t(x)));
  x += int(dpp_u32<0x4E>(uint32_t(x), uint32_t(x)));
  x += int(dpp_u32<0x124>(uint32_t(x), uint32_t(x)));
  x += int(dpp_u32<0x128>(uint32_t(x), uint32_t(x)));
  x += int(dpp_u32<0x142, 0xA>(0u, uint32_t(x)));
  x += int(dpp_u32<0x143, 0xC>(0u, uint32_t(x)));
  return __builtin_amdgcn_readlane(x, 63);
}

// Inclusive prefix sum over the lanes: a shift-and-add scan within each row of
// 16 lanes, then the rows' totals carried by the row broadcasts.
__device__ __forceinline__ int wave_incl_scan_i32(int x) {
  x += int(dpp_u32<0x111>(0u, uint32_t(x)));
  x += int(dpp_u32<0x112>(0u, uint32_t(x)));
  x += int(dpp_u32<0x114>(0u, uint32_t(x)));
  x += int(dpp_u32<0x118>(0u, uint32_t(x)));
  x += int(dpp_u32<0x142, 0xA>(0u, uint32_t(x)));
  x += int(dpp_u32<0x143, 0xC>(0u, uint32_t(x)));
  return x;
}

}  // namespace ft
