// ft_moe_permute: group the routed rows by expert (counting sort, stable).
//
// Each flat row r = t*k + j (token t's j-th pick) goes to segment ids[r];
// segments are laid out in expert order and keep rows ascending inside a
// segment.  The per-expert segments are what the grouped expert FFN walks:
// one contiguous block of rows per cached (layer, expert) entry (FreeToken
// rtx 4090 page, "Cómo funciona la jerarquía de memoria MoE": the runtime
// executes whole experts).
//
// Small inputs: one workgroup -- LDS histogram, exclusive scan, then one wave
// scatters 64 rows at a time, ranking equal keys with per-bit ballots.
// Large inputs: count per 1024-row block -> one-workgroup scan over blocks ->
// per-block scatter from the block's own bases.
#include "ft_internal.hpp"
#include "permute_util.hpp"

namespace ft {

constexpr int kPermSmallRows = 2048;  // one workgroup up to this many rows
constexpr int kPermChunk = 1024;      // rows per block of the multi-block path
constexpr int kPermMaxE = 4096;

size_t permute_workspace_bytes(int32_t T, int32_t k, int32_t E) {
  const int64_t R = int64_t(T) * k;
  if (R <= kPermSmallRows) return 0;
  const int64_t B = (R + kPermChunk - 1) / kPermChunk;
  return size_t(((B * E * 4) + 255) / 256 * 256);
}

// One workgroup (256 threads) does everything.
__global__ __launch_bounds__(256) void permute_small_kernel(const int32_t *__restrict__ ids, int R, int E,
                                                            int32_t *__restrict__ offsets,
                                                            int32_t *__restrict__ sorted_rows,
                                                            int32_t *__restrict__ row_pos) {
  __shared__ int s_cnt[kPermMaxE];
  __shared__ int s_tmp[32];
  permute_block(ids, R, E, s_cnt, s_tmp, offsets, sorted_rows, row_pos);
}

// One workgroup of 16 waves, up to 1024 rows over at most 256 experts: the
// ids into LDS, then the chunk-parallel sort (the 256-thread kernel above
// scatters 64 rows at a time with one wave: 6.5 us for 512 rows).
__global__ __launch_bounds__(1024) void permute_chunk_kernel(const int32_t *__restrict__ ids, int R, int E,
                                                             int32_t *__restrict__ offsets,
                                                             int32_t *__restrict__ sorted_rows,
                                                             int32_t *__restrict__ row_pos) {
  __shared__ int32_t s_ids[kChunkPermMaxRows];
  __shared__ int s_cc[kChunkPermMaxRows / 64 * kChunkPermMaxE];
  __shared__ int s_seg[kChunkPermMaxE];
  __shared__ int s_tmp[32];
  for (int r = threadIdx.x; r < R; r += blockDim.x) s_ids[r] = ids[r];
  __syncthreads();
  permute_chunks(s_ids, R, E, s_cc, s_seg, s_tmp, offsets, sorted_rows, row_pos);
}

// Multi-block pass 1: per-block histogram -> counts[b][e].
__global__ __launch_bounds__(256) void permute_count_kernel(const int32_t *__restrict__ ids, int R, int E,
                                                            int32_t *__restrict__ counts) {
  __shared__ int s_cnt[kPermMaxE];
  const int tid = threadIdx.x, b = blockIdx.x;
  for (int e = tid; e < E; e += 256) s_cnt[e] = 0;
  __syncthreads();
  const int r0 = b * kPermChunk, r1 = min(R, r0 + kPermChunk);
  for (int r = r0 + tid; r < r1; r += 256) {
    const int key = ids[r];
    if (key >= 0 && key < E) atomicAdd(&s_cnt[key], 1);
  }
  __syncthreads();
  for (int e = tid; e < E; e += 256) counts[int64_t(b) * E + e] = s_cnt[e];
}

// Multi-block pass 2 (one workgroup): counts[b][e] := sum_{b'<b} counts[b'][e];
// offsets = exclusive scan of the per-expert totals.
__global__ __launch_bounds__(1024) void permute_scan_kernel(int32_t *__restrict__ counts, int B, int E,
                                                            int32_t *__restrict__ offsets) {
  __shared__ int s_tot[kPermMaxE];
  __shared__ int s_tmp[32];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += 1024) {
    int run = 0;
    for (int b = 0; b < B; ++b) {
      const int c = counts[int64_t(b) * E + e];
      counts[int64_t(b) * E + e] = run;
      run += c;
    }
    s_tot[e] = run;
  }
  __syncthreads();
  const int total = block_exclusive_scan(s_tot, E, s_tmp);
  for (int e = tid; e < E; e += 1024) offsets[e] = s_tot[e];
  if (tid == 0) offsets[E] = total;
}

// Multi-block pass 3: block b scatters its rows from offsets[e] + counts[b][e].
__global__ __launch_bounds__(64) void permute_scatter_kernel(const int32_t *__restrict__ ids, int R, int E,
                                                             const int32_t *__restrict__ counts,
                                                             const int32_t *__restrict__ offsets,
                                                             int32_t *__restrict__ sorted_rows,
                                                             int32_t *__restrict__ row_pos) {
  __shared__ int s_base[kPermMaxE];
  const int b = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += 64) s_base[e] = offsets[e] + counts[int64_t(b) * E + e];
  __syncthreads();
  const int r0 = b * kPermChunk, r1 = min(R, r0 + kPermChunk);
  wave_scatter(ids, r0, r1, E, s_base, sorted_rows, row_pos);
}

}  // namespace ft

using namespace ft;

extern "C" ft_status ft_moe_permute(const int32_t *topk_ids, int32_t T, int32_t k, int32_t E,
                                    int32_t *expert_offsets, int32_t *sorted_rows, int32_t *row_pos,
                                    void *workspace, size_t workspace_bytes, hipStream_t stream) {
  FT_REQUIRE(T >= 0 && k >= 1 && E >= 1, "ft_moe_permute: need T >= 0, k >= 1, E >= 1");
  FT_SUPPORTED(E <= kPermMaxE, "ft_moe_permute: E > 4096");
  FT_REQUIRE(int64_t(T) * k < (int64_t(1) << 31), "ft_moe_permute: T*k too large");
  FT_REQUIRE(expert_offsets != nullptr, "ft_moe_permute: expert_offsets is NULL");
  const int R = T * k;
  if (R > 0) FT_REQUIRE(topk_ids && sorted_rows && row_pos, "ft_moe_permute: NULL pointer argument");
  const size_t need = permute_workspace_bytes(T, k, E);
  FT_REQUIRE(need == 0 || (workspace != nullptr && workspace_bytes >= need && aligned(workspace, 4)),
             "ft_moe_permute: workspace too small (see ft_workspace_bytes)");
  if (R > 64 && R <= kChunkPermMaxRows && E <= kChunkPermMaxE) {
    hipLaunchKernelGGL(permute_chunk_kernel, dim3(1), dim3(1024), 0, stream, topk_ids, R, E, expert_offsets,
                       sorted_rows, row_pos);
    FT_LAUNCHED("permute_chunk_kernel");
  } else if (R <= kPermSmallRows) {
    hipLaunchKernelGGL(permute_small_kernel, dim3(1), dim3(256), 0, stream, topk_ids, R, E, expert_offsets,
                       sorted_rows, row_pos);
    FT_LAUNCHED("permute_small_kernel");
  } else {
    const int B = cdiv(R, kPermChunk);
    int32_t *counts = static_cast<int32_t *>(workspace);
    hipLaunchKernelGGL(permute_count_kernel, dim3(B), dim3(256), 0, stream, topk_ids, R, E, counts);
    FT_LAUNCHED("permute_count_kernel");
    hipLaunchKernelGGL(permute_scan_kernel, dim3(1), dim3(1024), 0, stream, counts, B, E, expert_offsets);
    FT_LAUNCHED("permute_scan_kernel");
    hipLaunchKernelGGL(permute_scatter_kernel, dim3(B), dim3(64), 0, stream, topk_ids, R, E, counts,
                       expert_offsets, sorted_rows, row_pos);
    FT_LAUNCHED("permute_scatter_kernel");
  }
  clear_error();
  return FT_OK;
}
