// Plain HBM read stream: the practical ceiling against which the split-KV decode kernel's
// bandwidth is reported. Each workgroup reads one contiguous chunk of 16-byte words (eight
// loads in flight per lane), folds them with XOR so the loads cannot be dropped, and
// writes one word per workgroup. No page defines this; it is a measurement aid.
#include "common.hpp"

namespace mi_attn {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 8;

template <bool NT>
__global__ __launch_bounds__(kStreamThreads) void read_stream_kernel(const u32x4_t* __restrict__ src, size_t words,
                                                                      size_t words_per_block,
                                                                      uint32_t* __restrict__ sink) {
  const size_t w0 = static_cast<size_t>(blockIdx.x) * words_per_block;
  const size_t w1 = w0 + words_per_block < words ? w0 + words_per_block : words;
  u32x4_t acc = {0u, 0u, 0u, 0u};
  size_t w = w0 + threadIdx.x;
  constexpr size_t step = static_cast<size_t>(kStreamThreads) * kStreamUnroll;
  for (; w + (kStreamUnroll - 1) * kStreamThreads < w1; w += step) {
    u32x4_t x[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) {
      if constexpr (NT) x[u] = __builtin_nontemporal_load(src + w + u * kStreamThreads);
      else x[u] = src[w + u * kStreamThreads];
    }
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) acc ^= x[u];
  }
  for (; w < w1; w += kStreamThreads) acc ^= src[w];
  uint32_t r = acc.x ^ acc.y ^ acc.z ^ acc.w;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) r ^= static_cast<uint32_t>(__shfl_xor(static_cast<int>(r), o, kWave));
  __shared__ uint32_t part[kStreamThreads / kWave];
  if (threadIdx.x % kWave == 0) part[threadIdx.x / kWave] = r;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0;
    for (int i = 0; i < kStreamThreads / kWave; ++i) t ^= part[i];
    sink[blockIdx.x] = t;
  }
}

}  // namespace
}  // namespace mi_attn

extern "C" int attn_read_stream(const void* src, size_t bytes, int nontemporal, uint32_t* sink, void* stream) {
  using namespace mi_attn;
  if (src == nullptr || sink == nullptr || bytes == 0 || bytes % 16 != 0 ||
      (reinterpret_cast<uintptr_t>(src) & 15u) != 0)
    return MI_ATTN_EINVAL;
  const size_t words = bytes / 16;
  const size_t per_block = MI_ATTN_READ_STREAM_CHUNK / 16;
  const size_t blocks = (words + per_block - 1) / per_block;
  if (blocks > 0x7fffffffu) return MI_ATTN_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const u32x4_t* p = static_cast<const u32x4_t*>(src);
  if (nontemporal)
    hipLaunchKernelGGL(read_stream_kernel<true>, dim3(static_cast<unsigned>(blocks)), dim3(kStreamThreads), 0, s, p,
                       words, per_block, sink);
  else
    hipLaunchKernelGGL(read_stream_kernel<false>, dim3(static_cast<unsigned>(blocks)), dim3(kStreamThreads), 0, s, p,
                       words, per_block, sink);
  return hipGetLastError() == hipSuccess ? MI_ATTN_OK : MI_ATTN_EHIP;
}
