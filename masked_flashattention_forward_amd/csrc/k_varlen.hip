// Work lists and the LSE merge of the varlen forward (attn_fwd_varlen).
//
// A batch of sequences of different lengths (vLLM pull request #11277 page, the varlen
// call with cu_seqlens and a block table) is planned on the device, since the lengths
// live there:
//   unit  one sequence with at most 32 query rows per KV head (decode type: a decode
//         step or a short chunk), or q_per_block queries of a longer one (prefill type);
//   item  a run of whole 64-key tiles of a unit's visible key range; one workgroup per
//         (item, KV head). Each type gets about `target_items` items of near-equal
//         length, so a long sequence is spread over many workgroups and a short one
//         is not split at all.
// Prefill-type items run on the MFMA prefill kernel, decode-type items on the split-KV
// decode kernel. A unit with one item writes the output directly; the partial results
// of a unit with several are combined here by log-sum-exp (ExecuTorch pull request
// #10466 page, "Summary": chunks along the key dimension, merged through their running
// max and sum).
#include "common.hpp"
#include "kernels.hpp"
#include "mfma_common.hpp"

namespace mi_attn {

hipError_t launch_prefill_varlen(const AttnParams& p, int dtype, hipStream_t s);
hipError_t launch_decode_varlen(const AttnParams& p, int dtype, hipStream_t s);

namespace {

constexpr int kPlanThreads = 256;
constexpr int kPlanWaves = kPlanThreads / kWave;
constexpr int kItemTile = 64;     // item boundaries fall on 64-key tiles
constexpr int kMinItemTiles = 8;  // an item has at least 512 keys, unless its unit is shorter
constexpr int kDecodeRows = 32;   // decode type: query rows per KV head (G * Lq) at most
constexpr int kDecodeFlag = 1 << 30;
constexpr int kResidentBlocks = 512;  // prefill workgroups resident at once: 256 CUs x 2

using mfma::VarlenSeq;
using mfma::varlen_seq;

__device__ bool decode_type(const AttnParams& p, const VarlenSeq& v) { return v.Lq * p.G <= kDecodeRows; }

// query blocks of a sequence (units)
__device__ int units_of(const AttnParams& p, const VarlenSeq& v) {
  if (v.Lq == 0) return 0;
  return decode_type(p, v) ? 1 : (v.Lq + p.q_per_block - 1) / p.q_per_block;
}

// visible key range [lo, hi) of unit qb: bottom-right positions and the mask's bounds;
// empty for a two-source sequence with fewer keys than queries
__device__ void unit_keys(const AttnParams& p, const VarlenSeq& v, int qb, int* lo, int* hi) {
  const bool dec = decode_type(p, v);
  const int i_first = dec ? 0 : qb * p.q_per_block;
  const int i_last = dec ? v.Lq - 1 : min(v.Lq, i_first + p.q_per_block) - 1;
  key_range(p.mask_kind, p.window_left, v.Lk, v.Lk - v.Lq + i_first, v.Lk - v.Lq + i_last, lo, hi);
  if (p.no_skip) {
    *lo = 0;
    *hi = v.Lk;
  }
  if (v.ctx < 0) *hi = *lo;
}

__device__ int tiles_of(int lo, int hi) { return hi > lo ? (hi - 1) / kItemTile + 1 - lo / kItemTile : 0; }

// items of a unit with `tiles` tiles at about `per` tiles each (forced: `force` items):
// n items of per_u tiles, the last one shorter; a unit with no visible key still gets
// one (empty) item, which writes its fully masked rows
__device__ void split_unit(int tiles, int per, int force, int* n, int* per_u) {
  if (tiles == 0) {
    *n = 1;
    *per_u = 0;
    return;
  }
  int k = force > 0 ? force : tiles / per + (tiles % per != 0);
  if (k > tiles) k = tiles;
  *per_u = tiles / k + (tiles % k != 0);
  *n = tiles / *per_u + (tiles % *per_u != 0);
}

// block-wide exclusive scan and total of NV int64 values (every thread calls it)
template <int NV>
__device__ void block_scan(const long long (&v)[NV], long long (&excl)[NV], long long (&tot)[NV],
                           long long (*wsum)[kPlanWaves]) {
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  long long inc[NV];
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    inc[k] = v[k];
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const long long y = __shfl_up(inc[k], o, kWave);
      if (lane >= o) inc[k] += y;
    }
    if (lane == kWave - 1) wsum[k][wave] = inc[k];
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    long long before = 0, all = 0;
    for (int w = 0; w < kPlanWaves; ++w) {
      if (w < wave) before += wsum[k][w];
      all += wsum[k][w];
    }
    excl[k] = before + inc[k] - v[k];
    tot[k] = all;
  }
  __syncthreads();  // wsum is reused by the next call
}

// One workgroup. Sequences are taken in rounds of 256: their lengths and unit offsets go
// to LDS, and each thread then takes units of the round (not whole sequences, so a long
// prefill sequence's units do not run one after another on a single lane). Pass 1 sums
// the tiles of each type and fixes the item length per type; pass 2 numbers units and
// items in sequence order and writes them. Units of a sequence are written longest key
// range first. Writes stop at the caps, which consistent lengths never reach.
__global__ __launch_bounds__(kPlanThreads) void varlen_plan_kernel(AttnParams p, int4* units, int4* items_p,
                                                                   int4* items_d, int32_t* counts, int units_cap,
                                                                   int items_cap, int target_items, int force) {
  __shared__ long long wsum[3][kPlanWaves];
  __shared__ int s_lq[kPlanThreads], s_lk[kPlanThreads], s_ctx[kPlanThreads], s_off[kPlanThreads + 1];
  const int tid = threadIdx.x;

  // the round of sequences [base, base + kPlanThreads): lengths and the offsets of their
  // units within the round; returns the round's unit count
  auto load_round = [&](int base) {
    const int s = base + tid;
    long long nu[1] = {0}, ex[1], tot[1];
    s_lq[tid] = s_lk[tid] = s_ctx[tid] = 0;
    if (s < p.num_seqs) {
      const VarlenSeq v = varlen_seq(p, s);
      s_lq[tid] = v.Lq;
      s_lk[tid] = v.Lk;
      s_ctx[tid] = v.ctx;
      nu[0] = units_of(p, v);
    }
    block_scan<1>(nu, ex, tot, wsum);
    s_off[tid] = static_cast<int>(ex[0]);
    if (tid == 0) s_off[kPlanThreads] = static_cast<int>(tot[0]);
    __syncthreads();
    return static_cast<int>(tot[0]);
  };
  // unit j of the round: its sequence's slot in the round, lengths and query block
  auto unit_at = [&](int j, int* ls, int* qb, VarlenSeq* v) {
    int lo = 0, hi = kPlanThreads;  // the last slot whose offset is <= j (a non-empty one)
    while (hi - lo > 1) {
      const int mid = (lo + hi) / 2;
      if (s_off[mid] <= j) lo = mid;
      else hi = mid;
    }
    *ls = lo;
    *qb = s_off[lo + 1] - 1 - j;  // the round's units run longest key range first
    *v = VarlenSeq{};
    v->Lq = s_lq[lo];
    v->Lk = s_lk[lo];
    v->ctx = s_ctx[lo];
  };

  // tiles of prefill-type and decode-type units, and the prefill-type unit count
  long long t3[3] = {0, 0, 0};
  for (int base = 0; base < p.num_seqs; base += kPlanThreads) {
    const int nunits = load_round(base);
    for (int j = tid; j < nunits; j += kPlanThreads) {
      int ls, qb, lo, hi;
      VarlenSeq v;
      unit_at(j, &ls, &qb, &v);
      const bool dec = decode_type(p, v);
      if (!dec) t3[2] += 1;
      unit_keys(p, v, qb, &lo, &hi);
      t3[dec ? 1 : 0] += tiles_of(lo, hi);
    }
    __syncthreads();  // the next round rewrites the LDS arrays
  }
  long long ex3[3], tot3[3];
  block_scan<3>(t3, ex3, tot3, wsum);
  // prefill-type units are split only when they cannot fill the GPU's resident
  // workgroup slots on their own; decode-type units always aim at target_items items
  const bool split_p = tot3[2] * p.Hkv < kResidentBlocks;
  const long long kNever = 0x3fffffff;
  const int per_p = static_cast<int>(
      split_p ? min(kNever, max(static_cast<long long>(kMinItemTiles), (tot3[0] + target_items - 1) / target_items))
              : kNever);
  const int per_d = static_cast<int>(
      min(kNever, max(static_cast<long long>(kMinItemTiles), (tot3[1] + target_items - 1) / target_items)));

  long long carry[3] = {0, 0, 0};  // units, prefill-type items, decode-type items so far
  for (int base = 0; base < p.num_seqs; base += kPlanThreads) {
    const int nunits = load_round(base);
    for (int j0 = 0; j0 < nunits; j0 += kPlanThreads) {
      const int j = j0 + tid;
      int ls = 0, qb = 0, lo = 0, hi = 0, n = 0, per_u = 0;
      bool dec = false;
      long long cnt[3] = {0, 0, 0};
      if (j < nunits) {
        VarlenSeq v;
        unit_at(j, &ls, &qb, &v);
        dec = decode_type(p, v);
        unit_keys(p, v, qb, &lo, &hi);
        split_unit(tiles_of(lo, hi), dec ? per_d : per_p, force, &n, &per_u);
        cnt[0] = 1;
        cnt[dec ? 2 : 1] = n;
      }
      long long ex[3], tot[3];
      block_scan<3>(cnt, ex, tot, wsum);
      if (j < nunits) {
        const long long u = carry[0] + ex[0];
        long long it = carry[dec ? 2 : 1] + ex[dec ? 2 : 1];
        int4* items = dec ? items_d : items_p;
        if (u < units_cap)
          units[u] = make_int4(base + ls, qb, static_cast<int>(it < items_cap ? it : items_cap), n | (dec ? kDecodeFlag : 0));
        const long long t0 = lo / kItemTile;
        for (int k = 0; k < n; ++k, ++it) {
          const long long a = k == 0 ? lo : max(static_cast<long long>(lo), (t0 + k * per_u) * kItemTile);
          const long long b = min(static_cast<long long>(hi), (t0 + (k + 1) * static_cast<long long>(per_u)) * kItemTile);
          if (it < items_cap && u < units_cap)
            items[it] = make_int4(static_cast<int>(u), static_cast<int>(a), static_cast<int>(max(a, b)), 0);
        }
      }
      for (int k = 0; k < 3; ++k) carry[k] += tot[k];
    }
    __syncthreads();  // the next round rewrites the LDS arrays
  }
  if (tid == 0) {
    counts[0] = static_cast<int32_t>(min(carry[0], static_cast<long long>(units_cap)));
    counts[1] = static_cast<int32_t>(min(carry[1], static_cast<long long>(items_cap)));
    counts[2] = static_cast<int32_t>(min(carry[2], static_cast<long long>(items_cap)));
  }
}

// LSE merge of the units with several items: one workgroup per (unit, KV head), one
// thread per (row, 4 dims) at a time. lse = log sum_i exp(lse_i) (all -inf gives -inf
// and output 0); out = sum_i exp(lse_i - lse) o_i.
template <typename T, int D>
__global__ __launch_bounds__(256) void varlen_merge_kernel(AttnParams p, const int4* units, const int32_t* counts,
                                                           int items_cap, const float* pp_out, const float* pp_lse,
                                                           const float* pd_out, const float* pd_lse) {
  const int u = blockIdx.x;
  const int g = blockIdx.y;
  if (u >= counts[0]) return;
  const int4 un = units[u];
  const int n = un.w & (kDecodeFlag - 1);
  if (n <= 1 || un.z > items_cap - n) return;  // (the second only for inconsistent lengths)
  const bool dec = (un.w & kDecodeFlag) != 0;
  const VarlenSeq v = varlen_seq(p, un.x);
  const int i_first = dec ? 0 : un.y * p.q_per_block;
  const int i_last = dec ? v.Lq - 1 : min(v.Lq, i_first + p.q_per_block) - 1;
  const int rows = (i_last - i_first + 1) * p.G;
  const int rpb = dec ? kDecodeRows : kVarlenPrefillRows;  // partial rows per (item, KV head)
  const float* po = dec ? pd_out : pp_out;
  const float* pl = dec ? pd_lse : pp_lse;
  constexpr int kPerRow = D / 4;
  constexpr int kBatch = 8;  // items whose partials are loaded together (their latencies overlap)
  for (int idx = threadIdx.x; idx < rows * kPerRow; idx += blockDim.x) {
    const int r = idx / kPerRow;
    const int d0 = (idx % kPerRow) * 4;
    auto slot_of = [&](int k) { return (static_cast<long>(un.z + k) * p.Hkv + g) * rpb + r; };
    float mx = kNegInf;
    for (int k0 = 0; k0 < n; k0 += kBatch) {
      float ls[kBatch];
#pragma unroll
      for (int k = 0; k < kBatch; ++k) ls[k] = k0 + k < n ? pl[slot_of(k0 + k)] : kNegInf;
#pragma unroll
      for (int k = 0; k < kBatch; ++k) mx = fmaxf(mx, ls[k]);
    }
    float4 acc = {0.f, 0.f, 0.f, 0.f};
    float tot = 0.f;
    if (mx != kNegInf) {
      for (int k0 = 0; k0 < n; k0 += kBatch) {
        float ls[kBatch];
        float4 os[kBatch];
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
          ls[k] = kNegInf;
          os[k] = float4{0.f, 0.f, 0.f, 0.f};
          if (k0 + k < n) {
            const long slot = slot_of(k0 + k);
            ls[k] = pl[slot];
            os[k] = *reinterpret_cast<const float4*>(po + slot * D + d0);
          }
        }
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
          const float w = __expf(ls[k] - mx);  // 0 for the items past n
          acc.x += w * os[k].x; acc.y += w * os[k].y; acc.z += w * os[k].z; acc.w += w * os[k].w;
          tot += w;
        }
      }
    }
    const bool dead = !(tot > 0.f);
    const float inv = dead ? 0.f : 1.f / tot;
    const long row = static_cast<long>(v.q_start + i_first + r / p.G) * p.Hq + g * p.G + r % p.G;
    T* O = static_cast<T*>(p.out) + row * D + d0;
    O[0] = from_f32<T>(acc.x * inv);
    O[1] = from_f32<T>(acc.y * inv);
    O[2] = from_f32<T>(acc.z * inv);
    O[3] = from_f32<T>(acc.w * inv);
    if (d0 == 0 && p.lse != nullptr) p.lse[row] = dead ? kNegInf : mx + logf(tot);
  }
}

template <typename T>
hipError_t launch_merge_t(const AttnParams& p, const VarlenBuffers& b, hipStream_t s) {
  dim3 grid(static_cast<unsigned>(b.units_cap), static_cast<unsigned>(p.Hkv)), block(256);
  if (p.d == 128)
    hipLaunchKernelGGL((varlen_merge_kernel<T, 128>), grid, block, 0, s, p, b.units, b.counts, b.items_cap,
                       b.pp_out, b.pp_lse, b.pd_out, b.pd_lse);
  else
    hipLaunchKernelGGL((varlen_merge_kernel<T, 64>), grid, block, 0, s, p, b.units, b.counts, b.items_cap,
                       b.pp_out, b.pp_lse, b.pd_out, b.pd_lse);
  return hipGetLastError();
}

}  // namespace

int varlen_items_cap(int units_cap, int target_items, int force) {
  const long a = static_cast<long>(target_items) + units_cap;
  const long f = static_cast<long>(units_cap) * (force > 0 ? force : 1);
  const long c = a > f ? a : f;
  return c > 0x3fffffffL ? 0x3fffffff : static_cast<int>(c);
}

hipError_t launch_varlen(const AttnParams& p, int dtype, const VarlenBuffers& b, hipStream_t s) {
  if (dtype != MI_ATTN_BF16 && dtype != MI_ATTN_F16) return hipErrorInvalidValue;
  if (static_cast<long>(b.units_cap) > 0x7fffffffL || p.Hkv > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(varlen_plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, p, b.units, b.items_p, b.items_d,
                     b.counts, b.units_cap, b.items_cap, b.target_items, b.force_items);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  AttnParams q = p;
  q.vl_units = b.units;
  q.vl_counts = b.counts;
  q.vl_items_cap = b.items_cap;
  q.vl_items = b.items_p;
  q.part_out = b.pp_out;
  q.part_lse = b.pp_lse;
  e = launch_prefill_varlen(q, dtype, s);
  if (e != hipSuccess) return e;
  q.vl_items = b.items_d;
  q.part_out = b.pd_out;
  q.part_lse = b.pd_lse;
  e = launch_decode_varlen(q, dtype, s);
  if (e != hipSuccess) return e;
  return dtype == MI_ATTN_BF16 ? launch_merge_t<bf16_t>(p, b, s) : launch_merge_t<f16_t>(p, b, s);
}

}  // namespace mi_attn
