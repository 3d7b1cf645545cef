// Dynamic top-k mask (flash-sparse-attention issue #11 page, "Overview": zero_hold values
// computed ahead of the kernel select, per query row, the keys that stay visible; causal
// masking and top-k selection combined, sized by keep_window_size).
//
// Per (batch, KV head):
//   1. rank: each key's place in the total order (value descending, index ascending).
//      Keys are packed into 64-bit words (order-preserving value bits << 32 | index).
//      Caches of up to 8192 keys: every 512-key chunk is bitonic-sorted by one workgroup
//      (in registers and wavefront shuffles, LDS only for the cross-wavefront stages),
//      then each key's rank is the sum over chunks of the number of smaller words, found
//      by a binary search in the sorted chunks staged in LDS. Longer caches first merge
//      the chunks into sorted runs of 8192 keys the same way, then search the runs.
//   2. tau: per query row, the keep_k-th smallest rank among the row's allowed keys. One
//      wavefront sweeps 32 consecutive rows, holding a bitmap of the ranks seen so far in
//      registers. Under the causal mask a row allows one key more than the row before,
//      so tau can only fall: it is found once by a wavefront prefix count and afterwards
//      moves, when the new key ranks below it, to the largest set rank below the old tau.
//   3. optional keep bitmask and per-tile minimum rank (tile skipping in attention).
#include <type_traits>

#include "common.hpp"

namespace mi_attn {

namespace {

using u64 = unsigned long long;

constexpr int kChunk = 512;               // keys bitonic-sorted per workgroup
constexpr int kChunkThreads = kChunk / 2; // two keys per thread
constexpr int kMergeMaxKeys = 8192;       // sorted chunks of one (b,h) staged in 68 KiB of LDS (padded)
constexpr int kRankThreads = 256;
constexpr u64 kPadKey = ~0ull;            // above every real key
constexpr int32_t kAllKept = 0x7fffffff;  // "no threshold" and the rank past the last key

// Ascending order of the returned word == descending order of x; -0.0 ties +0.0.
__device__ __forceinline__ uint32_t desc_bits(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) == 0) u = 0;
  const uint32_t asc = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ~asc;
}

// Strictly increasing in the total order; never equal to kPadKey (NaN is excluded).
__device__ __forceinline__ u64 order_key(const float* z, int j) {
  return (static_cast<u64>(desc_bits(z[j])) << 32) | static_cast<unsigned>(j);
}

__device__ __forceinline__ u64 shfl_xor_u64(u64 x, int m) {
  const int lo = __shfl_xor(static_cast<int>(static_cast<uint32_t>(x)), m, kWave);
  const int hi = __shfl_xor(static_cast<int>(static_cast<uint32_t>(x >> 32)), m, kWave);
  return (static_cast<u64>(static_cast<uint32_t>(hi)) << 32) | static_cast<uint32_t>(lo);
}

__device__ __forceinline__ u64 min_u64(u64 a, u64 b) { return a < b ? a : b; }
__device__ __forceinline__ u64 max_u64(u64 a, u64 b) { return a < b ? b : a; }

// Sorts chunk blockIdx.y of (b,h) = blockIdx.x ascending into sorted[bh][chunk][0..511].
// Thread t holds elements 2t and 2t+1. In the stage comparing elements i and i^j, pairs
// with j <= 64 sit in one wavefront (thread distance j/2 <= 32): shuffles. Larger j go
// through LDS.
__global__ __launch_bounds__(kChunkThreads) void chunk_sort_kernel(const float* zh, int Lk, int nchunks,
                                                                     u64* sorted) {
  __shared__ u64 xch[kChunk];
  const int bh = blockIdx.x;
  const int c0 = blockIdx.y * kChunk;
  const float* z = zh + static_cast<long>(bh) * Lk;
  const int e0 = 2 * static_cast<int>(threadIdx.x);
  u64 a = (c0 + e0 < Lk) ? order_key(z, c0 + e0) : kPadKey;
  u64 b = (c0 + e0 + 1 < Lk) ? order_key(z, c0 + e0 + 1) : kPadKey;
#pragma unroll
  for (int k = 2; k <= kChunk; k <<= 1) {
    const bool up = (e0 & k) == 0;  // this run of k elements sorts ascending
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      if (j == 1) {
        const u64 lo = min_u64(a, b), hi = max_u64(a, b);
        a = up ? lo : hi;
        b = up ? hi : lo;
      } else {
        u64 pa, pb;
        if (j <= 64) {
          pa = shfl_xor_u64(a, j >> 1);
          pb = shfl_xor_u64(b, j >> 1);
        } else {
          __syncthreads();
          xch[e0] = a;
          xch[e0 + 1] = b;
          __syncthreads();
          pa = xch[e0 ^ j];
          pb = xch[(e0 + 1) ^ j];
        }
        const bool keep_min = ((e0 & j) == 0) == up;
        a = keep_min ? min_u64(a, pa) : max_u64(a, pa);
        b = keep_min ? min_u64(b, pb) : max_u64(b, pb);
      }
    }
  }
  u64* dst = sorted + (static_cast<long>(bh) * nchunks + blockIdx.y) * kChunk;
  dst[e0] = a;
  dst[e0 + 1] = b;
}

// LDS slot of staged sorted word g: 16 bytes of padding after every 32 words. The probes of
// one binary-search level are words s - 1 (mod s) for a step s, so without padding those of
// the small steps fall on a few banks.
__host__ __device__ constexpr int pad_slot(int g) { return g + 2 * (g >> 5); }

// rank_j = number of keys before j in the total order = sum over the sorted chunks of the
// count of words below key_j (branch-free lower bound over 512 entries). When tile_min is
// given, also the smallest rank of each block_n-key tile (block_n divides kRankThreads).
__global__ __launch_bounds__(kRankThreads) void rank_merge_kernel(const float* zh, const u64* sorted, int Lk,
                                                                    int nchunks, int32_t* rank, int32_t* tile_min,
                                                                    int block_n) {
  extern __shared__ u64 srt[];
  __shared__ int32_t rk_s[kRankThreads];
  const int bh = blockIdx.x;
  const int n = nchunks * kChunk;
  const uint4* src = reinterpret_cast<const uint4*>(sorted + static_cast<long>(bh) * n);
  // words 2t, 2t + 1 stay side by side (16-byte aligned) in the padded layout
  for (int t = threadIdx.x; t < n / 2; t += kRankThreads) *reinterpret_cast<uint4*>(srt + pad_slot(2 * t)) = src[t];
  __syncthreads();
  const int j = blockIdx.y * kRankThreads + threadIdx.x;
  int cnt = kAllKept;
  if (j < Lk) {
    const u64 key = order_key(zh + static_cast<long>(bh) * Lk, j);
    cnt = 0;
    // four independent searches at a time, so their LDS latencies overlap; chunks past
    // nchunks are searched in chunk 0 and not counted. A chunk starts on a multiple of 32
    // words, so its word i sits at its own start plus pad_slot(i).
    for (int c = 0; c < nchunks; c += 4) {
      const u64* s[4];
      int pos[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        s[u] = srt + pad_slot((c + u < nchunks ? c + u : 0) * kChunk);
        pos[u] = 0;
      }
#pragma unroll
      for (int step = kChunk / 2; step > 0; step >>= 1)
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (s[u][pad_slot(pos[u] + step - 1)] < key) pos[u] += step;
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (c + u < nchunks) cnt += pos[u] + (s[u][pad_slot(pos[u])] < key ? 1 : 0);
    }
    rank[static_cast<long>(bh) * Lk + j] = cnt;
  }
  if (tile_min == nullptr) return;
  rk_s[threadIdx.x] = cnt;
  __syncthreads();
  const int ntiles = (Lk + block_n - 1) / block_n;
  const int tile = blockIdx.y * (kRankThreads / block_n) + static_cast<int>(threadIdx.x);
  if (static_cast<int>(threadIdx.x) < kRankThreads / block_n && tile < ntiles) {
    int32_t mn = kAllKept;
    for (int e = 0; e < block_n; ++e) {
      const int32_t r = rk_s[threadIdx.x * block_n + e];
      mn = r < mn ? r : mn;
    }
    tile_min[static_cast<long>(bh) * ntiles + tile] = mn;
  }
}

// Caches longer than kMergeMaxKeys: the sorted 512-key chunks are first merged into
// sorted runs of kRunChunks chunks (8192 keys, staged in LDS like the merge above), then
// each key's rank is the sum over the runs of a binary search in global memory
// (log2(8192) + 1 probes per run, the runs of one (b,h) read from L2).
constexpr int kRunChunks = kMergeMaxKeys / kChunk;  // chunks per run
constexpr int kRunKeys = kMergeMaxKeys;

// Run blockIdx.y of (b,h) = blockIdx.x: each key of the run moves to its place among the
// run's keys (the count of smaller words over the run's sorted chunks). Slots at or past
// the run's real keys (the padding of the last chunk) receive kPadKey.
__global__ __launch_bounds__(kRankThreads) void run_merge_kernel(const u64* sorted, int Lk, int nchunks,
                                                                   u64* runs) {
  extern __shared__ u64 srt[];
  const int bh = blockIdx.x;
  const int run = blockIdx.y;
  const int c0 = run * kRunChunks;
  const int rc = (nchunks - c0) < kRunChunks ? (nchunks - c0) : kRunChunks;  // chunks in this run
  const int n = rc * kChunk;
  const u64* base = sorted + (static_cast<long>(bh) * nchunks + c0) * kChunk;
  const uint4* src = reinterpret_cast<const uint4*>(base);
  uint4* dst = reinterpret_cast<uint4*>(srt);
  for (int t = threadIdx.x; t < n / 2; t += kRankThreads) dst[t] = src[t];
  __syncthreads();
  const int local = blockIdx.z * kRankThreads + threadIdx.x;  // slot in the run
  if (local >= n) return;
  u64* out = runs + (static_cast<long>(bh) * nchunks + c0) * kChunk;
  const long real = static_cast<long>(Lk) - static_cast<long>(c0) * kChunk;  // real keys from the run start
  if (local >= real) {
    out[local] = kPadKey;
    return;
  }
  // the run's keys are those of its chunks; a real key's place is the number of words
  // below it over all of them (its own chunk included)
  const u64 key = srt[local];
  int cnt = 0;
  for (int c = 0; c < rc; c += 4) {
    const u64* sp[4];
    int pos[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      sp[u] = srt + (c + u < rc ? c + u : 0) * kChunk;
      pos[u] = 0;
    }
#pragma unroll
    for (int step = kChunk / 2; step > 0; step >>= 1)
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (sp[u][pos[u] + step - 1] < key) pos[u] += step;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (c + u < rc) cnt += pos[u] + (sp[u][pos[u]] < key ? 1 : 0);
  }
  out[cnt] = key;
}

// rank_j = sum over the sorted runs of the number of words below key_j (lower bound by
// binary search over each run's kRunKeys or fewer slots), plus the per-tile minimum rank
// when tile_min is given (as in rank_merge_kernel).
__global__ __launch_bounds__(kRankThreads) void rank_runs_kernel(const float* zh, const u64* runs, int Lk,
                                                                   int nchunks, int32_t* rank, int32_t* tile_min,
                                                                   int block_n) {
  __shared__ int32_t rk_s[kRankThreads];
  const int bh = blockIdx.x;
  const int nruns = (nchunks + kRunChunks - 1) / kRunChunks;
  const u64* rb = runs + static_cast<long>(bh) * nchunks * kChunk;
  const int j = blockIdx.y * kRankThreads + threadIdx.x;
  int cnt = kAllKept;
  if (j < Lk) {
    const u64 key = order_key(zh + static_cast<long>(bh) * Lk, j);
    cnt = 0;
    for (int r = 0; r < nruns; r += 4) {
      const u64* sp[4];
      int len[4], pos[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int rr = r + u < nruns ? r + u : 0;
        sp[u] = rb + static_cast<long>(rr) * kRunKeys;
        const int rcn = (nchunks - rr * kRunChunks) < kRunChunks ? (nchunks - rr * kRunChunks) : kRunChunks;
        len[u] = rcn * kChunk;
        pos[u] = 0;
      }
#pragma unroll
      for (int step = kRunKeys / 2; step > 0; step >>= 1)
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (pos[u] + step <= len[u] && sp[u][pos[u] + step - 1] < key) pos[u] += step;
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (r + u < nruns) cnt += pos[u] + (pos[u] < len[u] && sp[u][pos[u]] < key ? 1 : 0);
    }
    rank[static_cast<long>(bh) * Lk + j] = cnt;
  }
  if (tile_min == nullptr) return;
  rk_s[threadIdx.x] = cnt;
  __syncthreads();
  const int ntiles = (Lk + block_n - 1) / block_n;
  const int tile = blockIdx.y * (kRankThreads / block_n) + static_cast<int>(threadIdx.x);
  if (static_cast<int>(threadIdx.x) < kRankThreads / block_n && tile < ntiles) {
    int32_t mn = kAllKept;
    for (int e = 0; e < block_n; ++e) {
      const int32_t rv = rk_s[threadIdx.x * block_n + e];
      mn = rv < mn ? rv : mn;
    }
    tile_min[static_cast<long>(bh) * ntiles + tile] = mn;
  }
}

// Kept-key list of one (b, KV head, query block): the keys j < n (n: keys 0 .. p of the
// block's last row, or every key when rows may keep any) whose rank is at most the
// threshold tf of the block's first row (thresholds do not grow with the row position, so
// every row of the block keeps a subset), ascending, padded to a whole number of 64-key
// tiles with key Lk. Exactly keep_k keys up to the first row's position pass the test when
// its threshold is finite, and every key when it is not (then that position is below
// keep_k), so a list never holds more than keep_k + q_per_block - 1 keys. Run by all
// kListThreads threads of a workgroup.
constexpr int kListThreads = 256;
constexpr int kListWaves = kListThreads / kWave;
constexpr int kListSub = 16;  // 256-key sub-passes per pass (4096 keys per pass)
__device__ __forceinline__ void build_topk_list(const int32_t* rk, const float* z, int32_t tf, int n, int Lk,
                                                long base, int cap, int32_t* lidx, int32_t* lrank, float* lzh,
                                                int32_t* lcount) {
  __shared__ int sub_cnt[kListSub][kListWaves];
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  int cnt = 0;
  // a pass covers 4096 keys: sub-pass u holds keys j0 + 256 u + (0..255), so the loads are
  // coalesced and all 16 are in flight together; per-wavefront ballot counts of every
  // sub-pass go to LDS and one barrier later each lane knows where its keys go
  for (int j0 = 0; j0 < n; j0 += kListThreads * kListSub) {
    int32_t r[kListSub];
#pragma unroll
    for (int u = 0; u < kListSub; ++u) {
      const int j = j0 + u * kListThreads + tid;
      r[u] = j < n ? rk[j] : kAllKept;
    }
    unsigned long long ball[kListSub];
#pragma unroll
    for (int u = 0; u < kListSub; ++u) {
      const int j = j0 + u * kListThreads + tid;
      ball[u] = __ballot(j < n && r[u] <= tf);
      if (lane == 0) sub_cnt[u][wave] = __popcll(ball[u]);
    }
    __syncthreads();
    int run = cnt;  // kept keys before sub-pass u
#pragma unroll
    for (int u = 0; u < kListSub; ++u) {
      int before = run;
#pragma unroll
      for (int w = 0; w < kListWaves; ++w) {
        const int c = sub_cnt[u][w];
        before += w < wave ? c : 0;
        run += c;
      }
      const unsigned long long b_u = ball[u];
      if ((b_u >> lane) & 1ull) {
        const int e = before + __builtin_amdgcn_mbcnt_hi(static_cast<unsigned>(b_u >> 32),
                                                        __builtin_amdgcn_mbcnt_lo(static_cast<unsigned>(b_u), 0));
        const int j = j0 + u * kListThreads + tid;
        if (e < cap) {
          lidx[base + e] = j;
          lrank[base + e] = r[u];
          lzh[base + e] = z[j] * kLog2e;
        }
      }
    }
    cnt = run;
    __syncthreads();  // sub_cnt is rewritten by the next pass
  }
  cnt = cnt < cap ? cnt : cap;  // the bound above makes this a no-op
  const int padded = ((cnt + 63) / 64) * 64;
  for (int e = cnt + tid; e < padded; e += kListThreads) {
    lidx[base + e] = Lk;
    lrank[base + e] = kAllKept;
    lzh[base + e] = 0.f;
  }
  if (tid == 0) *lcount = cnt;
}

// One workgroup per (b, KV head, query block).
__global__ __launch_bounds__(kListThreads) void topk_list_kernel(const int32_t* rank, const int32_t* tau,
                                                                   const float* zh, int Lq, int Lk, int q_per_block,
                                                                   int nqb, int cap, int causal, int32_t* lidx,
                                                                   int32_t* lrank, float* lzh, int32_t* lcount) {
  const int qb = blockIdx.x;
  const int bh = blockIdx.y;
  const int i_first = qb * q_per_block;
  const int i_last = min(Lq, i_first + q_per_block) - 1;
  const int n = causal ? Lk - Lq + i_last + 1 : Lk;
  build_topk_list(rank + static_cast<long>(bh) * Lk, zh + static_cast<long>(bh) * Lk,
                  tau[static_cast<long>(bh) * Lq + i_first], n, Lk, (static_cast<long>(bh) * nqb + qb) * cap, cap,
                  lidx, lrank, lzh, lcount + static_cast<long>(bh) * nqb + qb);
}

constexpr int kTauRowsPerWave = 32;
constexpr int kTauWaves = 4;

// keep_k-th smallest set rank of the wavefront's bitmap (lane l owns ranks
// [32 * WPL * l, 32 * WPL * (l + 1)) in words[]); the bitmap holds at least keep_k bits.
template <int WPL>
__device__ __forceinline__ int kth_set_rank(const uint32_t (&words)[WPL], int keep_k, int lane) {
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
  const bool here = excl < keep_k && keep_k <= incl;
  int found = 0;
  if (here) {
    int need = keep_k - excl;
#pragma unroll
    for (int w = 0; w < WPL; ++w) {
      const int pc = __popc(words[w]);
      if (need > 0 && need <= pc) {
        uint32_t x = words[w];
        for (int t = 1; t < need; ++t) x &= x - 1;
        found = (lane * WPL + w) * 32 + (__ffs(x) - 1);
      }
      need -= pc;
    }
  }
  const int src = __ffsll(static_cast<unsigned long long>(__ballot(here))) - 1;
  return __builtin_amdgcn_readlane(found, src);
}

// Largest set rank below t; the bitmap holds at least one.
template <int WPL>
__device__ __forceinline__ int set_rank_below(const uint32_t (&words)[WPL], int t, int lane) {
  int cand = -1;
#pragma unroll
  for (int w = 0; w < WPL; ++w) {
    const int base = (lane * WPL + w) * 32;
    const int lim = t - base;
    const uint32_t keep = lim >= 32 ? ~0u : (lim <= 0 ? 0u : ((1u << lim) - 1u));
    const uint32_t x = words[w] & keep;
    if (x != 0) cand = base + 31 - __clz(x);
  }
  const unsigned long long b = __ballot(cand >= 0);
  const int src = 63 - __clzll(b);
  return __builtin_amdgcn_readlane(cand, src);
}

// Causal tau. WPL = 32-bit bitmap words per lane; one wavefront covers 64 * 32 * WPL ranks.
// Workgroup = 4 wavefronts = 128 consecutive rows of one (b,h). Every global load of the
// kernel is issued before the first barrier, so their latencies overlap. LISTS: the
// workgroup then builds the kept-key lists of the query blocks its rows start (their
// first rows' thresholds are in LDS by then).
template <int WPL, bool LISTS>
__global__ __launch_bounds__(kTauWaves * kWave) void tau_kernel(const int32_t* rank, int Lq, int Lk, int keep_k,
                                                                  int32_t* tau, TopkListArgs la) {
  constexpr int NW = kWave * WPL;
  constexpr int kThreads = kTauWaves * kWave;
  constexpr int kBuild = (8 * WPL) < 16 ? (8 * WPL) : 16;  // keys per thread per pass of the shared bitmap
  __shared__ uint32_t block_bm[NW];
  __shared__ uint32_t wave_bm[kTauWaves][NW];
  const int bh = blockIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // uniform: scalar branches below
  const int lane = threadIdx.x % kWave;
  const int32_t* rk = rank + static_cast<long>(bh) * Lk;
  const int rb = blockIdx.y * kTauWaves * kTauRowsPerWave;  // first row of the workgroup (< Lq)
  const int pos_b = Lk - Lq + rb;                            // keys [0, pos_b) precede it (pos_b < Lk)
  const int r0 = rb + wave * kTauRowsPerWave;
  const int pos_w = pos_b + wave * kTauRowsPerWave;          // keys [0, pos_w) precede row r0
  const int n = r0 < Lq ? ((Lq - r0) < kTauRowsPerWave ? (Lq - r0) : kTauRowsPerWave) : 0;

  for (int w = threadIdx.x; w < NW; w += kThreads) block_bm[w] = 0;
  // shared part: keys [0, pos_b), kBuild * kThreads of them per pass
  int br[kBuild];
#pragma unroll
  for (int u = 0; u < kBuild; ++u) {
    const int t = u * kThreads + static_cast<int>(threadIdx.x);
    br[u] = t < pos_b ? rk[t] : -1;
  }
  // this wavefront's part: keys [max(pos_b, 0), pos_w), at most (kTauWaves - 1) * kTauRowsPerWave
  constexpr int kExtra = ((kTauWaves - 1) * kTauRowsPerWave + kWave - 1) / kWave;
  int xr[kExtra];
  const int x0 = pos_b > 0 ? pos_b : 0;
  const int x_end = n > 0 ? pos_w : 0;
#pragma unroll
  for (int u = 0; u < kExtra; ++u) {
    const int t = x0 + u * kWave + lane;
    xr[u] = t < x_end ? rk[t] : -1;
  }
  // the key each row adds: lane i holds the rank of key p_{r0 + i}
  const int my_pos = pos_w + lane;
  const int my_rank = (lane < n && my_pos >= 0) ? rk[my_pos] : -1;
  __syncthreads();
  for (int t0 = 0;;) {
#pragma unroll
    for (int u = 0; u < kBuild; ++u)
      if (br[u] >= 0) atomicOr(&block_bm[br[u] >> 5], 1u << (br[u] & 31));
    t0 += kBuild * kThreads;
    if (t0 >= pos_b) break;
#pragma unroll
    for (int u = 0; u < kBuild; ++u) {
      const int t = t0 + u * kThreads + static_cast<int>(threadIdx.x);
      br[u] = t < pos_b ? rk[t] : -1;
    }
  }
  __syncthreads();
  for (int w = lane; w < NW; w += kWave) wave_bm[wave][w] = block_bm[w];
#pragma unroll
  for (int u = 0; u < kExtra; ++u)
    if (xr[u] >= 0) atomicOr(&wave_bm[wave][xr[u] >> 5], 1u << (xr[u] & 31));
  __syncthreads();
  __shared__ int32_t tau_s[LISTS ? kTauWaves * kTauRowsPerWave : 1];
  if (!LISTS && n == 0) return;

  uint32_t words[WPL];
#pragma unroll
  for (int w = 0; w < WPL; ++w) words[w] = wave_bm[wave][lane * WPL + w];
  int my_tau = kAllKept;
  int cur = kAllKept;  // kAllKept until the rows allow more than keep_k keys
  for (int i = 0; i < n; ++i) {
    const int r = __builtin_amdgcn_readlane(my_rank, i);
    if (r >= 0) {
      const int owner = r / (32 * WPL);
      const int wi = (r >> 5) - owner * WPL;
      if (lane == owner) {
#pragma unroll
        for (int w = 0; w < WPL; ++w)
          if (w == wi) words[w] |= 1u << (r & 31);
      }
    }
    const int allowed = pos_w + i + 1;  // keys 0 .. p_i
    if (allowed <= keep_k) cur = kAllKept;
    else if (cur == kAllKept) cur = kth_set_rank<WPL>(words, keep_k, lane);
    else if (r < cur) cur = set_rank_below<WPL>(words, cur, lane);
    if (lane == i) my_tau = cur;
  }
  if (lane < n) tau[static_cast<long>(bh) * Lq + r0 + lane] = my_tau;
  if constexpr (LISTS) {
    if (lane < kTauRowsPerWave) tau_s[wave * kTauRowsPerWave + lane] = my_tau;
    __syncthreads();
    // query blocks whose first row lies in this workgroup's rows
    const int qb0 = (rb + la.q_per_block - 1) / la.q_per_block;
    const int qb1 = min(la.nqb, (rb + kTauWaves * kTauRowsPerWave + la.q_per_block - 1) / la.q_per_block);
    for (int qb = qb0; qb < qb1; ++qb) {
      const int i_first = qb * la.q_per_block;
      const int i_last = min(Lq, i_first + la.q_per_block) - 1;
      build_topk_list(rk, la.zh + static_cast<long>(bh) * Lk, tau_s[i_first - rb], Lk - Lq + i_last + 1, Lk,
                      (static_cast<long>(bh) * la.nqb + qb) * la.cap, la.cap, la.lidx, la.lrank, la.lzh,
                      la.lcount + static_cast<long>(bh) * la.nqb + qb);
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

// One wavefront per flag (batch, KV head, query block, key tile) of a dense mask that may
// differ per batch and head (see AttnParams::flag_b): 1 iff some entry is above -inf for
// some row of the block and some query head of the KV head. A mask shared over a
// dimension has one flag row for it.
__global__ __launch_bounds__(256) void mask_summary_kernel(AttnParams p, int block_n, int nqb, int ntiles,
                                                             long nflags, uint8_t* flags) {
  const long f = static_cast<long>(blockIdx.x) * 4 + threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  if (f >= nflags) return;
  const int t = static_cast<int>(f % ntiles);
  const int qb = static_cast<int>((f / ntiles) % nqb);
  const int fg = static_cast<int>((f / (static_cast<long>(ntiles) * nqb)) % p.flag_g);
  const int fb = static_cast<int>(f / (static_cast<long>(ntiles) * nqb * p.flag_g));
  const int i0 = qb * p.q_per_block;
  const int i1 = (i0 + p.q_per_block) < p.Lq ? (i0 + p.q_per_block) : p.Lq;
  const int j0 = t * block_n;
  const int j1 = (j0 + block_n) < p.Lk ? (j0 + block_n) : p.Lk;
  const int w = j1 - j0;
  // query heads of the KV head whose mask rows differ (one when the mask is shared over
  // heads); with a single KV head flag_g is 1 even when the rows differ per query head
  const int nh = (p.Hq > 1 && p.ms[1] != 0) ? p.G : 1;
  const float* mb = p.mask + fb * p.ms[0] + static_cast<long>(fg) * p.G * p.ms[1];
  // lanes take consecutive keys, the wavefront walks the rows (query position, head) and
  // stops at the first row with a visible key
  bool any = false;
  for (int i = i0; i < i1 && !any; ++i) {
    for (int hh = 0; hh < nh && !any; ++hh) {
      const float* row = mb + hh * p.ms[1] + i * p.ms[2];
      bool live = false;
      for (int jj = lane; jj < w; jj += kWave) live |= row[(j0 + jj) * p.ms[3]] > kNegInf;
      any = __any(live);
    }
  }
  if (lane == 0) flags[f] = any ? 1 : 0;
}

}  // namespace

size_t topk_sort_ws_bytes(int BH, int Lk) {
  const int nchunks = (Lk + kChunk - 1) / kChunk;
  const size_t one = sizeof(u64) * static_cast<size_t>(BH) * nchunks * kChunk;
  return Lk > kMergeMaxKeys ? 2 * one : one;  // sorted chunks (and the merged runs)
}

hipError_t launch_topk(const float* zh, int BH, int Lq, int Lk, int keep_k, int causal, int32_t* rank,
                       int32_t* tau, uint32_t* keep_bits, int32_t* tile_min, int block_n, hipStream_t s,
                       void* sort_ws, const TopkListArgs* lists) {
  if (lists != nullptr && (!causal || lists->cap % 64 != 0 || lists->q_per_block <= 0)) return hipErrorInvalidValue;
  if (tile_min != nullptr && (block_n <= 0 || block_n > kWave || kRankThreads % block_n != 0))
    return hipErrorInvalidValue;
  hipError_t e = hipSuccess;
  // sorted chunks (and, past kMergeMaxKeys, the merged runs): the caller's workspace
  const int nchunks = (Lk + kChunk - 1) / kChunk;
  const size_t chunk_words = static_cast<size_t>(BH) * nchunks * kChunk;
  u64* sorted = static_cast<u64*>(sort_ws);
  if (sorted == nullptr && topk_sort_ws_bytes(BH, Lk) > 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(chunk_sort_kernel, dim3(BH, nchunks), dim3(kChunkThreads), 0, s, zh, Lk, nchunks, sorted);
  if (Lk <= kMergeMaxKeys) {
    hipLaunchKernelGGL(rank_merge_kernel, dim3(BH, (Lk + kRankThreads - 1) / kRankThreads), dim3(kRankThreads),
                       sizeof(u64) * pad_slot(nchunks * kChunk), s, zh, sorted, Lk, nchunks, rank, tile_min, block_n);
  } else {
    u64* runs = sorted + chunk_words;
    const int nruns = (nchunks + kRunChunks - 1) / kRunChunks;
    hipLaunchKernelGGL(run_merge_kernel, dim3(BH, nruns, kRunKeys / kRankThreads), dim3(kRankThreads),
                       sizeof(u64) * kRunKeys, s, sorted, Lk, nchunks, runs);
    hipLaunchKernelGGL(rank_runs_kernel, dim3(BH, (Lk + kRankThreads - 1) / kRankThreads), dim3(kRankThreads), 0, s,
                       zh, runs, Lk, nchunks, rank, tile_min, block_n);
  }
  e = hipGetLastError();
  if (e == hipSuccess) {
    if (!causal) {
      const int32_t v = (Lk > keep_k) ? keep_k - 1 : kAllKept;
      const long n = static_cast<long>(BH) * Lq;
      hipLaunchKernelGGL(tau_const_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s,
                         static_cast<int>(n), v, tau);
    } else {
      const dim3 grid(BH, (Lq + kTauWaves * kTauRowsPerWave - 1) / (kTauWaves * kTauRowsPerWave));
      const dim3 block(kTauWaves * kWave);
      const int wpl = (Lk + 64 * 32 - 1) / (64 * 32);
      const TopkListArgs la = lists != nullptr ? *lists : TopkListArgs{};
      auto go = [&](auto wpl_tag) {
        constexpr int W = decltype(wpl_tag)::value;
        if (lists != nullptr) hipLaunchKernelGGL((tau_kernel<W, true>), grid, block, 0, s, rank, Lq, Lk, keep_k, tau, la);
        else hipLaunchKernelGGL((tau_kernel<W, false>), grid, block, 0, s, rank, Lq, Lk, keep_k, tau, la);
      };
      if (wpl <= 1) go(std::integral_constant<int, 1>{});
      else if (wpl <= 2) go(std::integral_constant<int, 2>{});
      else if (wpl <= 4) go(std::integral_constant<int, 4>{});
      else if (wpl <= 8) go(std::integral_constant<int, 8>{});
      else if (wpl <= 16) go(std::integral_constant<int, 16>{});
      else go(std::integral_constant<int, 32>{});
    }
    e = hipGetLastError();
  }
  if (e == hipSuccess && keep_bits != nullptr) {
    const long total = static_cast<long>(BH) * Lq * ((Lk + 31) / 32);
    hipLaunchKernelGGL(keep_bits_kernel, dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256), 0, s, rank,
                       tau, BH, Lq, Lk, causal, keep_bits);
    e = hipGetLastError();
  }
  return e;
}

hipError_t launch_topk_lists(const int32_t* rank, const int32_t* tau, const float* zh, int BH, int Lq, int Lk,
                             int q_per_block, int cap, int causal, int32_t* list_idx, int32_t* list_rank,
                             float* list_zh, int32_t* list_count, hipStream_t s) {
  const int nqb = (Lq + q_per_block - 1) / q_per_block;
  if (cap % 64 != 0 || BH > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(topk_list_kernel, dim3(nqb, BH), dim3(kListThreads), 0, s, rank, tau, zh, Lq, Lk, q_per_block,
                     nqb, cap, causal, list_idx, list_rank, list_zh, list_count);
  return hipGetLastError();
}

hipError_t launch_mask_summary(const AttnParams& p, int block_n, uint8_t* flags, hipStream_t s) {
  const int nqb = (p.Lq + p.q_per_block - 1) / p.q_per_block;
  const int nt = (p.Lk + block_n - 1) / block_n;
  const long nflags = static_cast<long>(p.flag_b) * p.flag_g * nqb * nt;
  if ((nflags + 3) / 4 > 0x7fffffffL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(mask_summary_kernel, dim3(static_cast<unsigned>((nflags + 3) / 4)), dim3(256), 0, s, p, block_n,
                     nqb, nt, nflags, flags);
  return hipGetLastError();
}

}  // namespace mi_attn
