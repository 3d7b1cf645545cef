// Dynamic top-k mask (flash-sparse-attention issue #11 page, "Overview": zero_hold values
// computed ahead of the kernel select, per query row, the keys that stay visible; causal
// masking and top-k selection combined, sized by keep_window_size).
//
// Per (batch, KV head):
//   1. rank: each key's place in the total order (value descending, index ascending).
//      Keys are packed into 64-bit words (order-preserving value bits << 32 | index) and
//      sorted in LDS with a bitonic network; an O(Lk^2) counting kernel covers long caches.
//   2. tau: per query row, the keep_k-th smallest rank among the row's allowed keys. One
//      wavefront sweeps a run of consecutive rows holding a bitmap of the ranks seen so
//      far in registers; the keep_k-th set bit is found with a wavefront prefix count.
//   3. optional keep bitmask and per-tile minimum rank (tile skipping in attention).
#include "common.hpp"

namespace mi_attn {

namespace {

constexpr int kSortMax = 8192;       // keys per (b,h) sorted in LDS (64 KiB of u64)
constexpr int kSortThreads = 1024;

// Ascending order of the returned word == descending order of x; -0.0 ties +0.0.
__device__ __forceinline__ uint32_t desc_bits(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) == 0) u = 0;
  const uint32_t asc = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ~asc;
}

__global__ __launch_bounds__(kSortThreads) void rank_sort_kernel(const float* zh, int Lk, int N,
                                                                   int32_t* rank, int32_t* order) {
  extern __shared__ unsigned long long skey[];
  const int bh = blockIdx.x;
  const float* z = zh + static_cast<long>(bh) * Lk;
  for (int t = threadIdx.x; t < N; t += blockDim.x)
    skey[t] = (t < Lk) ? ((static_cast<unsigned long long>(desc_bits(z[t])) << 32) | static_cast<unsigned>(t))
                       : ~0ull;
  __syncthreads();
  for (int kk = 2; kk <= N; kk <<= 1) {
    for (int j = kk >> 1; j > 0; j >>= 1) {
      for (int t = threadIdx.x; t < N; t += blockDim.x) {
        const int u = t ^ j;
        if (u > t) {
          const unsigned long long a = skey[t], b = skey[u];
          const bool up = (t & kk) == 0;
          if ((a > b) == up) { skey[t] = b; skey[u] = a; }
        }
      }
      __syncthreads();
    }
  }
  for (int t = threadIdx.x; t < Lk; t += blockDim.x) {
    const int idx = static_cast<int>(skey[t] & 0xffffffffu);
    rank[static_cast<long>(bh) * Lk + idx] = t;
    order[static_cast<long>(bh) * Lk + t] = idx;
  }
}

// O(Lk^2) rank for caches longer than the LDS sort: rank_j = #keys ordered before j.
__global__ __launch_bounds__(256) void rank_count_kernel(const float* zh, int Lk, int32_t* rank,
                                                           int32_t* order) {
  __shared__ unsigned long long tile[256];
  const int bh = blockIdx.x;
  const float* z = zh + static_cast<long>(bh) * Lk;
  const int j = blockIdx.y * 256 + threadIdx.x;
  const unsigned long long mine =
      (j < Lk) ? ((static_cast<unsigned long long>(desc_bits(z[j])) << 32) | static_cast<unsigned>(j)) : ~0ull;
  int cnt = 0;
  for (int m0 = 0; m0 < Lk; m0 += 256) {
    const int m = m0 + threadIdx.x;
    tile[threadIdx.x] =
        (m < Lk) ? ((static_cast<unsigned long long>(desc_bits(z[m])) << 32) | static_cast<unsigned>(m)) : ~0ull;
    __syncthreads();
    const int n = (Lk - m0) < 256 ? (Lk - m0) : 256;
    for (int t = 0; t < n; ++t) cnt += (tile[t] < mine) ? 1 : 0;
    __syncthreads();
  }
  if (j < Lk) {
    rank[static_cast<long>(bh) * Lk + j] = cnt;
    order[static_cast<long>(bh) * Lk + cnt] = j;
  }
}

constexpr int kTauRowsPerWave = 64;

// WPL = 32-bit bitmap words per lane; one wavefront covers 64 * 32 * WPL ranks.
template <int WPL>
__global__ __launch_bounds__(256) void tau_kernel(const int32_t* rank, const int32_t* order, int Lq,
                                                    int Lk, int keep_k, int32_t* tau) {
  const int bh = blockIdx.x;
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int r0 = (blockIdx.y * 4 + wave) * kTauRowsPerWave;
  if (r0 >= Lq) return;
  const int r1 = (r0 + kTauRowsPerWave) < Lq ? (r0 + kTauRowsPerWave) : Lq;
  const int32_t* rk = rank + static_cast<long>(bh) * Lk;
  const int32_t* od = order + static_cast<long>(bh) * Lk;
  const int base = lane * 32 * WPL;  // first rank owned by this lane

  // bitmap of the ranks of keys 0 .. pos(r0) - 1
  const int pos0 = Lk - Lq + r0;
  uint32_t words[WPL];
#pragma unroll
  for (int w = 0; w < WPL; ++w) {
    uint32_t x = 0;
    for (int bit = 0; bit < 32; ++bit) {
      const int r = base + w * 32 + bit;
      if (r < Lk && od[r] < pos0) x |= 1u << bit;
    }
    words[w] = x;
  }

  for (int i = r0; i < r1; ++i) {
    const int pos = Lk - Lq + i;
    if (pos >= 0) {
      const int r = rk[pos];
      if (r >= base && r < base + 32 * WPL) {
        const int w = (r - base) >> 5;
#pragma unroll
        for (int t = 0; t < WPL; ++t)
          if (t == w) words[t] |= 1u << (r & 31);
      }
    }
    const int n_allowed = pos + 1;  // pos <= Lk - 1 always
    if (n_allowed <= keep_k) {
      if (lane == 0) tau[static_cast<long>(bh) * Lq + i] = 0x7fffffff;
      continue;
    }
    int c = 0;
#pragma unroll
    for (int w = 0; w < WPL; ++w) c += __popc(words[w]);
    int incl = c;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int y = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += y;
    }
    const int excl = incl - c;
    if (excl < keep_k && keep_k <= incl) {
      int need = keep_k - excl;
      int found = -1;
#pragma unroll
      for (int w = 0; w < WPL; ++w) {
        const int pc = __popc(words[w]);
        if (found < 0) {
          if (need <= pc) {
            uint32_t x = words[w];
            for (int t = 1; t < need; ++t) x &= x - 1;
            found = base + w * 32 + (__ffs(x) - 1);
          } else {
            need -= pc;
          }
        }
      }
      tau[static_cast<long>(bh) * Lq + i] = found;
    }
  }
}

__global__ void tau_const_kernel(int n, int32_t value, int32_t* tau) {
  const long t = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t < n) tau[t] = value;
}

// One thread per 32-key word of one row.
__global__ void keep_bits_kernel(const int32_t* rank, const int32_t* tau, int BH, int Lq, int Lk,
                                 int causal, uint32_t* bits) {
  const int nw = (Lk + 31) / 32;
  const long t = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
  const long total = static_cast<long>(BH) * Lq * nw;
  if (t >= total) return;
  const int w = static_cast<int>(t % nw);
  const long row = t / nw;  // bh * Lq + i
  const int i = static_cast<int>(row % Lq);
  const long bh = row / Lq;
  const int pos = Lk - Lq + i;
  const int32_t th = tau[row];
  uint32_t x = 0;
  for (int bit = 0; bit < 32; ++bit) {
    const int j = w * 32 + bit;
    if (j < Lk && (!causal || j <= pos) && rank[bh * Lk + j] <= th) x |= 1u << bit;
  }
  bits[t] = x;
}

__global__ void tile_min_rank_kernel(const int32_t* rank, int BH, int Lk, int block_n, int32_t* out) {
  const int nt = (Lk + block_n - 1) / block_n;
  const long t = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t >= static_cast<long>(BH) * nt) return;
  const long bh = t / nt;
  const int j0 = static_cast<int>(t % nt) * block_n;
  const int j1 = (j0 + block_n) < Lk ? (j0 + block_n) : Lk;
  int32_t mn = 0x7fffffff;
  for (int j = j0; j < j1; ++j) {
    const int32_t r = rank[bh * Lk + j];
    mn = r < mn ? r : mn;
  }
  out[t] = mn;
}

// One wavefront per (query block, key tile): flag = 1 iff some entry is above -inf.
__global__ __launch_bounds__(256) void mask_summary_kernel(const float* mask, int Lq, int Lk,
                                                             int q_per_block, int block_n, int ntiles,
                                                             long nflags, uint8_t* flags) {
  const long f = static_cast<long>(blockIdx.x) * 4 + threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  if (f >= nflags) return;
  const int qb = static_cast<int>(f / ntiles);
  const int t = static_cast<int>(f % ntiles);
  const int i0 = qb * q_per_block;
  const int i1 = (i0 + q_per_block) < Lq ? (i0 + q_per_block) : Lq;
  const int j0 = t * block_n;
  const int j1 = (j0 + block_n) < Lk ? (j0 + block_n) : Lk;
  const int w = j1 - j0;
  bool live = false;
  for (long e = lane; e < static_cast<long>(i1 - i0) * w; e += kWave) {
    const int i = i0 + static_cast<int>(e / w);
    const int j = j0 + static_cast<int>(e % w);
    live |= mask[static_cast<long>(i) * Lk + j] > kNegInf;
  }
  const bool any = __any(live);
  if (lane == 0) flags[f] = any ? 1 : 0;
}

}  // namespace

hipError_t launch_topk(const float* zh, int BH, int Lq, int Lk, int keep_k, int causal, int32_t* rank,
                       int32_t* tau, uint32_t* keep_bits, hipStream_t s) {
  // `order` (the inverse permutation) lives in a stream-ordered scratch buffer.
  int32_t* order = nullptr;
  hipError_t e = hipMallocAsync(reinterpret_cast<void**>(&order), sizeof(int32_t) * static_cast<size_t>(BH) * Lk, s);
  if (e != hipSuccess) return e;
  if (Lk <= kSortMax) {
    int N = 1;
    while (N < Lk) N <<= 1;
    const int threads = N < kSortThreads ? (N < 64 ? 64 : N) : kSortThreads;
    hipLaunchKernelGGL(rank_sort_kernel, dim3(BH), dim3(threads), sizeof(unsigned long long) * N, s, zh, Lk, N,
                       rank, order);
  } else {
    hipLaunchKernelGGL(rank_count_kernel, dim3(BH, (Lk + 255) / 256), dim3(256), 0, s, zh, Lk, rank, order);
  }
  e = hipGetLastError();
  if (e == hipSuccess) {
    if (!causal) {
      const int32_t v = (Lk > keep_k) ? keep_k - 1 : 0x7fffffff;
      const long n = static_cast<long>(BH) * Lq;
      hipLaunchKernelGGL(tau_const_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s,
                         static_cast<int>(n), v, tau);
    } else {
      dim3 grid(BH, (Lq + 4 * kTauRowsPerWave - 1) / (4 * kTauRowsPerWave));
      const int wpl = (Lk + 64 * 32 - 1) / (64 * 32);
      if (wpl <= 1) hipLaunchKernelGGL(tau_kernel<1>, grid, dim3(256), 0, s, rank, order, Lq, Lk, keep_k, tau);
      else if (wpl <= 2) hipLaunchKernelGGL(tau_kernel<2>, grid, dim3(256), 0, s, rank, order, Lq, Lk, keep_k, tau);
      else if (wpl <= 4) hipLaunchKernelGGL(tau_kernel<4>, grid, dim3(256), 0, s, rank, order, Lq, Lk, keep_k, tau);
      else if (wpl <= 8) hipLaunchKernelGGL(tau_kernel<8>, grid, dim3(256), 0, s, rank, order, Lq, Lk, keep_k, tau);
      else if (wpl <= 16) hipLaunchKernelGGL(tau_kernel<16>, grid, dim3(256), 0, s, rank, order, Lq, Lk, keep_k, tau);
      else hipLaunchKernelGGL(tau_kernel<32>, grid, dim3(256), 0, s, rank, order, Lq, Lk, keep_k, tau);
    }
    e = hipGetLastError();
  }
  if (e == hipSuccess && keep_bits != nullptr) {
    const long total = static_cast<long>(BH) * Lq * ((Lk + 31) / 32);
    hipLaunchKernelGGL(keep_bits_kernel, dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256), 0, s, rank,
                       tau, BH, Lq, Lk, causal, keep_bits);
    e = hipGetLastError();
  }
  const hipError_t ef = hipFreeAsync(order, s);
  return e != hipSuccess ? e : ef;
}

hipError_t launch_tile_min_rank(const int32_t* rank, int BH, int Lk, int block_n, int32_t* out, hipStream_t s) {
  const long n = static_cast<long>(BH) * ((Lk + block_n - 1) / block_n);
  hipLaunchKernelGGL(tile_min_rank_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s, rank, BH,
                     Lk, block_n, out);
  return hipGetLastError();
}

hipError_t launch_mask_summary(const float* mask, int Lq, int Lk, int q_per_block, int block_n, uint8_t* flags,
                               hipStream_t s) {
  const int nqb = (Lq + q_per_block - 1) / q_per_block;
  const int nt = (Lk + block_n - 1) / block_n;
  const long nflags = static_cast<long>(nqb) * nt;
  hipLaunchKernelGGL(mask_summary_kernel, dim3(static_cast<unsigned>((nflags + 3) / 4)), dim3(256), 0, s, mask, Lq,
                     Lk, q_per_block, block_n, nt, nflags, flags);
  return hipGetLastError();
}

}  // namespace mi_attn
