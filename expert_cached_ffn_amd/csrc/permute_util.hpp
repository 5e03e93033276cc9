// Block-level pieces of the stable counting sort of routed rows by expert,
// shared by ft_moe_permute and the fused decode routing call.
#pragma once

#include "ft_internal.hpp"

namespace ft {

__device__ __forceinline__ int bits_for(int E) {
  int b = 1;
  while ((1 << b) < E) ++b;
  return b;
}

// Stable scatter of rows [r0, r1) by one wave.  s_base[e] holds the next
// free position of expert e and is advanced as rows are placed.
__device__ __forceinline__ void wave_scatter(const int32_t *__restrict__ ids, int r0, int r1, int E,
                                             int *s_base, int32_t *__restrict__ sorted_rows,
                                             int32_t *__restrict__ row_pos) {
  const int lane = threadIdx.x & 63;
  const int nb = bits_for(E);
  const uint64_t lt = (uint64_t(1) << lane) - 1;
  for (int c = r0; c < r1; c += 64) {
    const int r = c + lane;
    const bool act = r < r1;
    int key = act ? ids[r] : 0;
    const bool ok = act && key >= 0 && key < E;
    const uint64_t active = __ballot(ok);
    uint64_t same = active;
    for (int b = 0; b < nb; ++b) {
      const uint64_t ones = __ballot((key >> b) & 1);
      same &= ((key >> b) & 1) ? ones : ~ones;
    }
    if (ok) {
      const int rank = __popcll(same & lt);
      const int pos = s_base[key] + rank;
      sorted_rows[pos] = r;
      row_pos[r] = pos;
    }
    __builtin_amdgcn_wave_barrier();
    if (ok && (same >> lane) == 1) s_base[key] += __popcll(same);  // last lane of its key
    __builtin_amdgcn_wave_barrier();
  }
}

// Block-wide exclusive scan of s[0..n) in place (n <= 4096); returns the total.
__device__ inline int block_exclusive_scan(int *s, int n, int *s_tmp /* >= 32 ints */) {
  const int tid = threadIdx.x, nt = blockDim.x;
  const int per = (n + nt - 1) / nt;
  const int a = min(n, tid * per), b = min(n, a + per);
  int local = 0;
  for (int i = a; i < b; ++i) local += s[i];
  // inclusive scan of `local` across the block
  const int lane = tid & 63, wave = tid >> 6, nw = nt >> 6;
  const int v = wave_incl_scan_i32(local);
  if (lane == 63) s_tmp[wave] = v;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int w = 0; w < nw; ++w) {
      const int t = s_tmp[w];
      s_tmp[w] = run;
      run += t;
    }
    s_tmp[nw] = run;
  }
  __syncthreads();
  int excl = s_tmp[wave] + v - local;
  for (int i = a; i < b; ++i) {
    const int t = s[i];
    s[i] = excl;
    excl += t;
  }
  const int total = s_tmp[nw];
  __syncthreads();
  return total;
}

// The whole permutation of R routed rows by one workgroup: LDS histogram,
// exclusive scan, then one wave scatters 64 rows at a time, ranking equal keys
// with per-bit ballots (so rows stay ascending inside a segment).  s_cnt holds
// E ints; ids may be global or LDS.
__device__ inline void permute_block(const int32_t *ids, int R, int E, int *s_cnt, int *s_tmp,
                                     int32_t *__restrict__ offsets, int32_t *__restrict__ sorted_rows,
                                     int32_t *__restrict__ row_pos) {
  const int tid = threadIdx.x, nt = blockDim.x;
  for (int e = tid; e < E; e += nt) s_cnt[e] = 0;
  __syncthreads();
  for (int r = tid; r < R; r += nt) {
    const int key = ids[r];
    if (key >= 0 && key < E) atomicAdd(&s_cnt[key], 1);
  }
  __syncthreads();
  const int total = block_exclusive_scan(s_cnt, E, s_tmp);
  for (int e = tid; e < E; e += nt) offsets[e] = s_cnt[e];
  if (tid == 0) offsets[E] = total;
  __syncthreads();
  if (tid < 64) wave_scatter(ids, 0, R, E, s_cnt, sorted_rows, row_pos);
}

// Stable counting sort of 64 < R <= kChunkPermMaxRows routed rows over E <=
// kChunkPermMaxE experts by one workgroup of at least R / 64 waves: wave c
// ranks the 64 rows of chunk c among themselves by per-bit ballots, the
// first row of each (chunk, expert) group records the group's size, a prefix
// over the chunks turns each expert's counts into chunk bases, a block scan
// turns the experts' totals into segment starts, and a row's place is its
// segment start + its chunk base + its rank in the chunk (rows stay
// ascending inside a segment).  ids in LDS; a row whose id lies outside
// [0, E) is left out (it gets no place).  s_cc: kChunkPermMaxRows / 64 *
// kChunkPermMaxE ints; s_seg: E ints.
constexpr int kChunkPermMaxRows = 1024, kChunkPermMaxE = 256;

__device__ inline void permute_chunks(const int32_t *s_ids, int R, int E, int *s_cc, int *s_seg, int *s_tmp,
                                      int32_t *__restrict__ offsets, int32_t *__restrict__ sorted_rows,
                                      int32_t *__restrict__ row_pos) {
  const int tid = threadIdx.x, nt = blockDim.x, wave = tid >> 6, lane = tid & 63;
  const int nch = (R + 63) / 64;
  for (int i = tid; i < nch * kChunkPermMaxE; i += nt) s_cc[i] = 0;
  __syncthreads();
  const int r = 64 * wave + lane;
  const int id = wave < nch && r < R ? s_ids[r] : -1;
  const bool act = id >= 0 && id < E;
  const int key = act ? id : 0;
  int rank = 0;
  if (wave < nch) {
    uint64_t same = __ballot(act);
    for (int b = bits_for(E) - 1; b >= 0; --b) {
      const int bit = (key >> b) & 1;
      const uint64_t ones = __ballot(bit);
      same &= bit ? ones : ~ones;
    }
    rank = __popcll(same & ((uint64_t(1) << lane) - 1));
    if (act && rank == 0) s_cc[wave * kChunkPermMaxE + key] = __popcll(same);
  }
  __syncthreads();
  for (int e = tid; e < E; e += nt) {
    int run = 0;
    for (int c = 0; c < nch; ++c) {
      const int v = s_cc[c * kChunkPermMaxE + e];
      s_cc[c * kChunkPermMaxE + e] = run;
      run += v;
    }
    s_seg[e] = run;
  }
  __syncthreads();
  const int total = block_exclusive_scan(s_seg, E, s_tmp);  // ends with a barrier
  for (int e = tid; e < E; e += nt) offsets[e] = s_seg[e];
  if (tid == 0) offsets[E] = total;
  if (act) {
    const int pos = s_seg[key] + s_cc[wave * kChunkPermMaxE + key] + rank;
    sorted_rows[pos] = r;
    row_pos[r] = pos;
  }
}

// Stable counting sort of R <= 64 routed rows by one wave, without a block
// barrier: lane i ranks row i by per-bit ballots -- the rows with a smaller
// expert id (counted among the lanes that agree with it on the higher bits and
// hold a 0 where it holds a 1) plus the rows of its own expert in lower lanes
// -- and writes its place; each expert's segment start is then the lower
// bound of its id in the sorted ids (s_sorted, 64 ints of LDS).  ids may be
// global or LDS; every id must lie in [0, E).
__device__ inline void permute_wave64(const int32_t *ids, int R, int E, int32_t *s_sorted,
                                      int32_t *__restrict__ offsets, int32_t *__restrict__ sorted_rows,
                                      int32_t *__restrict__ row_pos) {
  const int lane = threadIdx.x & 63;
  const bool act = lane < R;
  const int key = act ? ids[lane] : 0;
  uint64_t eq = __ballot(act);
  int less = 0;
  for (int b = bits_for(E) - 1; b >= 0; --b) {
    const int bit = (key >> b) & 1;
    const uint64_t ones = __ballot(bit);
    if (bit) less += __popcll(eq & ~ones);
    eq &= bit ? ones : ~ones;
  }
  const int pos = less + __popcll(eq & ((uint64_t(1) << lane) - 1));
  if (act) {
    sorted_rows[pos] = lane;
    row_pos[lane] = pos;
    s_sorted[pos] = key;
  }
  __builtin_amdgcn_wave_barrier();
  for (int e = lane; e <= E; e += 64) {
    int lo = 0, hi = R;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (s_sorted[mid] < e)
        lo = mid + 1;
      else
        hi = mid;
    }
    offsets[e] = lo;
  }
}

}  // namespace ft
