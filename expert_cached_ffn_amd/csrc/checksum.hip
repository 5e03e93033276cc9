// ft_read_checksum: the XOR of a device buffer's 32-bit words, the buffer read once.
//
// A weight stream's ceiling on this part is a plain read: the decode kernels are measured against
// it, and the same call checks that a copied expert blob arrived whole.  Wave w of the grid takes
// the 16 KiB pieces w, w + W, ... (W waves); a piece is 16 loads of 1 KiB of consecutive bytes (lane
// l: bytes 16 l .. 16 l + 15 of each), all in flight before the first XOR, so every load reads whole
// 128-byte lines.  Bytes past the end load as zero through the buffer descriptor, which leaves the
// XOR unchanged.  XOR needs no order: the result does not depend on the grid.
#include <algorithm>

#include "ft_internal.hpp"

namespace ft {

constexpr int kSumThreads = 512;  // 8 waves; two workgroups per compute unit
constexpr uint32_t kSumPiece = 16384;

__global__ __launch_bounds__(kSumThreads) void read_checksum_kernel(const uint8_t *__restrict__ buf, uint32_t bytes,
                                                                    uint32_t *__restrict__ sink) {
  const rsrc_t res = make_rsrc(buf, bytes);
  const int lane = threadIdx.x & 63;
  const uint32_t gw = blockIdx.x * (kSumThreads / 64) + (threadIdx.x >> 6), W = gridDim.x * (kSumThreads / 64);
  const uint32_t pieces = (bytes + kSumPiece - 1) / kSumPiece;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (uint32_t p = gw; p < pieces; p += W) {
    u32x4 v[16];
#pragma unroll
    for (int d = 0; d < 16; ++d) v[d] = bld16nt(res, p * kSumPiece + uint32_t(d) * 1024u + uint32_t(lane) * 16u);
#pragma unroll
    for (int d = 0; d < 16; ++d) acc ^= v[d];
  }
  uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x ^= uint32_t(__shfl_xor(int(x), o));
  if (lane == 0) atomicXor(sink, x);
}

}  // namespace ft

using namespace ft;

extern "C" ft_status ft_read_checksum(const void *buf, uint64_t bytes, uint32_t *sink, hipStream_t stream) {
  FT_REQUIRE(sink != nullptr && aligned(sink, 4), "ft_read_checksum: sink NULL or not 4-byte aligned");
  FT_REQUIRE(bytes % 16 == 0, "ft_read_checksum: bytes must be a multiple of 16");
  FT_SUPPORTED(bytes <= (uint64_t(1) << 31), "ft_read_checksum: above 2 GiB (checksum slices and XOR them)");
  if (bytes == 0) {
    clear_error();
    return FT_OK;
  }
  FT_REQUIRE(buf != nullptr && aligned(buf, 16), "ft_read_checksum: buf NULL or not 16-byte aligned");
  const uint32_t pieces = uint32_t((bytes + kSumPiece - 1) / kSumPiece);
  const unsigned grid = unsigned(std::min<uint32_t>(512u, (pieces + kSumThreads / 64 - 1) / (kSumThreads / 64)));
  hipLaunchKernelGGL(read_checksum_kernel, dim3(grid), dim3(kSumThreads), 0, stream, static_cast<const uint8_t *>(buf),
                     uint32_t(bytes), sink);
  FT_LAUNCHED("read_checksum_kernel");
  clear_error();
  return FT_OK;
}
