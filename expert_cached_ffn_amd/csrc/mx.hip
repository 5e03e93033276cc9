// ft_mxfp8_quantize: bf16 activation rows -> MXFP8 (E4M3 codes + E8M0 scales),
// the activation side of the native MXFP4 expert mode.
//
// The pages name natively MXFP4-quantized routed experts (FreeToken
// quantization page, "Formatos compatibles, hardware y perfil de rendimiento");
// a matrix unit that consumes MXFP4 weights directly needs its other operand in
// an MX format too.  The conversion follows OCP Microscaling Formats v1.0: each
// block of 32 consecutive elements shares the scale X = 2^(floor(log2 amax) - 8)
// (8 = exponent of E4M3's largest normal), stored as an E8M0 byte, and every
// element becomes the E4M3 value nearest v / X, ties to even, saturating at
// +-448.  An all-zero block gets scale byte 0; an exponent below -127 clamps
// to byte 0.
//
// One thread per block: 64 bytes in, 32 code bytes and one scale byte out.
// The block maximum is taken on the bf16 magnitude bits (monotone in the
// value), floor(log2 amax) read from its exponent field.  v / X is a power-of
// two multiply, exact in fp32; clamping to +-448 first makes the hardware
// conversion (round to nearest even, NaN beyond the format) saturate.
#include "ft_internal.hpp"

namespace ft {

// E8M0 scale byte of a block whose largest |bf16| has magnitude bits `amax`.
__device__ __forceinline__ uint32_t mx_scale_byte(uint32_t amax) {
  if (amax == 0) return 0;
  const int ef = int(amax >> 7);
  // floor(log2 |v|): normal -> exponent field - 127; subnormal (m * 2^-133) -> log2 m - 133
  const int e = ef > 0 ? ef - 127 : (31 - __builtin_clz(amax)) - 133;
  const int b = e - 8 + 127;
  return uint32_t(b < 0 ? 0 : (b > 254 ? 254 : b));
}

// Two bf16 (one dword) times 2^(127-byte) -> two E4M3 codes in the low 16 bits.
__device__ __forceinline__ uint32_t mx_e4m3x2(uint32_t d, float inv) {
  float a = __uint_as_float(d << 16) * inv;
  float b = __uint_as_float(d & 0xffff0000u) * inv;
  a = fminf(fmaxf(a, -448.f), 448.f);
  b = fminf(fmaxf(b, -448.f), 448.f);
  return uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false)) & 0xffffu;
}

__global__ __launch_bounds__(256) void mx_quantize_kernel(const uint16_t *__restrict__ x, int64_t ldx, int n,
                                                          int K, uint8_t *__restrict__ q,
                                                          uint8_t *__restrict__ s) {
  const int nb = K / 32;
  const int64_t b = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (b >= int64_t(n) * nb) return;
  const int64_t row = b / nb;
  const int blk = int(b % nb);
  const uint16_t *src = x + row * ldx + int64_t(blk) * 32;
  u32x4 v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = ld16(src + 8 * i);
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t d = v[i][j];
      amax = max(amax, max(d & 0x7fffu, (d >> 16) & 0x7fffu));
    }
  const uint32_t sb = mx_scale_byte(amax);
  const float inv = __uint_as_float((254u - sb) << 23);  // 2^(127 - sb); sb <= 246 for bf16 input
  u32x4 out[2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; j += 2) {
      const uint32_t lo = mx_e4m3x2(v[i][j], inv), hi = mx_e4m3x2(v[i][j + 1], inv);
      out[i / 2][(i % 2) * 2 + j / 2] = lo | (hi << 16);
    }
  uint8_t *dst = q + row * K + int64_t(blk) * 32;
  st16(dst, out[0]);
  st16(dst + 16, out[1]);
  s[row * nb + blk] = uint8_t(sb);
}

ft_status mx_quantize_launch(const uint16_t *x, int64_t ldx, int n, int K, uint8_t *q, uint8_t *s,
                             hipStream_t stream) {
  const int64_t blocks = int64_t(n) * (K / 32);
  if (blocks == 0) return FT_OK;
  hipLaunchKernelGGL(mx_quantize_kernel, dim3(unsigned(cdiv<int64_t>(blocks, 256))), dim3(256), 0, stream, x, ldx, n,
                     K, q, s);
  FT_LAUNCHED("mx_quantize_kernel");
  return FT_OK;
}

}  // namespace ft

using namespace ft;

extern "C" ft_status ft_mxfp8_quantize(const void *x, int64_t ldx, int32_t n, int32_t K, uint8_t *codes,
                                       uint8_t *scales, hipStream_t stream) {
  FT_REQUIRE(n >= 0 && K >= 0, "ft_mxfp8_quantize: need n >= 0, K >= 0");
  FT_REQUIRE(K % 32 == 0, "ft_mxfp8_quantize: K must be a multiple of 32");
  FT_REQUIRE(ldx >= K, "ft_mxfp8_quantize: row pitch below K");
  if (n == 0 || K == 0) {
    clear_error();
    return FT_OK;
  }
  FT_REQUIRE(x && codes && scales, "ft_mxfp8_quantize: NULL pointer argument");
  FT_REQUIRE(ldx % 8 == 0 && aligned(x, 16) && aligned(codes, 16),
             "ft_mxfp8_quantize: x and codes must be 16-byte aligned, row pitch a multiple of 8");
  const ft_status st = mx_quantize_launch(static_cast<const uint16_t *>(x), ldx, n, K, codes, scales, stream);
  if (st != FT_OK) return st;
  clear_error();
  return FT_OK;
}
