// ft_moe_combine: weighted sum of each token's expert rows ("scatter-add"
// of the permuted rows back to token order), plus the shared expert.
//
// out[t] = sum_{j<k} w[t, j] * y_rows[row_pos[t*k + j]]  (+ y_shared[t]),
// summed in j order, then the shared row, in fp32.  The gating weight of each
// routed expert scales its output (the pages' router activates a small subset
// of experts per token; FreeToken linux page, "Cómo gestiona FreeToken la
// memoria MoE"); the weighted sum is the textbook MoE combine.
//
// Gather form of the scatter-add: each thread owns 4 consecutive hidden
// elements of one token and reads its k rows with 16-byte loads, so no
// atomics are needed and the sum order is fixed.
#include "ft_internal.hpp"

namespace ft {

constexpr int kCombineThreads = 256;
constexpr int kCombineMaxK = 64;

template <bool BF16OUT>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(const float *__restrict__ y_rows,
                                                                  const float *__restrict__ w,
                                                                  const int32_t *__restrict__ row_pos,
                                                                  const float *__restrict__ y_shared, int T,
                                                                  int k, int H, void *__restrict__ out) {
  __shared__ int s_pos[kCombineMaxK];
  __shared__ float s_w[kCombineMaxK];
  const int t = blockIdx.y;
  const int h4 = (blockIdx.x * kCombineThreads + threadIdx.x) * 4;
  if (threadIdx.x < k) {
    s_pos[threadIdx.x] = row_pos[int64_t(t) * k + threadIdx.x];
    s_w[threadIdx.x] = w[int64_t(t) * k + threadIdx.x];
  }
  __syncthreads();
  if (h4 >= H) return;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < k; ++j) {
    const f32x4 y = *reinterpret_cast<const f32x4 *>(y_rows + int64_t(s_pos[j]) * H + h4);
    const float wj = s_w[j];
    acc[0] = fmaf(wj, y[0], acc[0]);
    acc[1] = fmaf(wj, y[1], acc[1]);
    acc[2] = fmaf(wj, y[2], acc[2]);
    acc[3] = fmaf(wj, y[3], acc[3]);
  }
  if (y_shared != nullptr) acc += *reinterpret_cast<const f32x4 *>(y_shared + int64_t(t) * H + h4);
  if constexpr (BF16OUT) {
    u32x2 pk = {uint32_t(f32_to_bf16_rne(acc[0])) | (uint32_t(f32_to_bf16_rne(acc[1])) << 16),
                uint32_t(f32_to_bf16_rne(acc[2])) | (uint32_t(f32_to_bf16_rne(acc[3])) << 16)};
    *reinterpret_cast<u32x2 *>(reinterpret_cast<uint16_t *>(out) + int64_t(t) * H + h4) = pk;
  } else {
    *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(out) + int64_t(t) * H + h4) = acc;
  }
}

}  // namespace ft

using namespace ft;

extern "C" ft_status ft_moe_combine(const float *y_rows, const float *topk_w, const int32_t *row_pos,
                                    const float *y_shared, int32_t T, int32_t k, int32_t H,
                                    int32_t out_dtype, void *out, hipStream_t stream) {
  FT_REQUIRE(T >= 0 && k >= 1 && H >= 1, "ft_moe_combine: need T >= 0, k >= 1, H >= 1");
  FT_SUPPORTED(k <= kCombineMaxK, "ft_moe_combine: k > 64");
  FT_SUPPORTED(H % 4 == 0, "ft_moe_combine: H must be a multiple of 4");
  FT_REQUIRE(out_dtype == FT_F32 || out_dtype == FT_BF16, "ft_moe_combine: out_dtype must be FT_F32 or FT_BF16");
  FT_REQUIRE(T <= 65535, "ft_moe_combine: T > 65535");
  if (T == 0) {
    clear_error();
    return FT_OK;
  }
  FT_REQUIRE(y_rows && topk_w && row_pos && out, "ft_moe_combine: NULL pointer argument");
  FT_REQUIRE(aligned(y_rows, 16) && aligned(out, 16) && (!y_shared || aligned(y_shared, 16)),
             "ft_moe_combine: y_rows, y_shared, out must be 16-byte aligned");
  const dim3 grid(unsigned(cdiv(H / 4, kCombineThreads)), unsigned(T));
  if (out_dtype == FT_BF16)
    hipLaunchKernelGGL(combine_kernel<true>, grid, dim3(kCombineThreads), 0, stream, y_rows, topk_w, row_pos,
                       y_shared, T, k, H, out);
  else
    hipLaunchKernelGGL(combine_kernel<false>, grid, dim3(kCombineThreads), 0, stream, y_rows, topk_w, row_pos,
                       y_shared, T, k, H, out);
  FT_LAUNCHED("combine_kernel");
  clear_error();
  return FT_OK;
}
