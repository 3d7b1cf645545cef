// Shared device helpers and launch declarations of the masked attention library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mi_attn.h"

namespace mi_attn {

// ------------------------------------------------------------------ element types
// Storage types are raw 16-bit patterns for fp16/bf16; conversions below are exact
// (upcast) or round-to-nearest-even (downcast).
struct bf16_t { uint16_t bits; };
struct f16_t { uint16_t bits; };

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) {
  return __uint_as_float(static_cast<uint32_t>(x.bits) << 16);
}
__device__ __forceinline__ float to_f32(f16_t x) {
  _Float16 h;
  __builtin_memcpy(&h, &x.bits, 2);
  return static_cast<float>(h);
}

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) {
  uint32_t u = __float_as_uint(x);
  bf16_t r;
  if ((u & 0x7fffffffu) > 0x7f800000u) {
    r.bits = 0x7fc0;  // NaN stays NaN
  } else {
    u += 0x7fffu + ((u >> 16) & 1u);
    r.bits = static_cast<uint16_t>(u >> 16);
  }
  return r;
}
template <> __device__ __forceinline__ f16_t from_f32<f16_t>(float x) {
  _Float16 h = static_cast<_Float16>(x);  // v_cvt_f16_f32: round to nearest even
  f16_t r;
  __builtin_memcpy(&r.bits, &h, 2);
  return r;
}

// ------------------------------------------------------------------ wave helpers
constexpr int kWave = 64;

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, kWave));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, kWave);
  return x;
}

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ------------------------------------------------------------------ problem description
// Everything a kernel needs to know about one attn_fwd call.
struct AttnParams {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;
  const float* mask;       // dense [Lq, Lk]
  const float* zero_hold;  // [B, Hkv, Lk]
  const int32_t* rank;     // top-k: [B, Hkv, Lk]
  const int32_t* tau;      // top-k: [B, Hkv, Lq]
  const int32_t* tile_min_rank;  // top-k: [B, Hkv, ceil(Lk / block_n)]
  const uint8_t* tile_live;      // dense: [ceil(Lq / q_per_block), ceil(Lk / block_n)]
  // top-k, gathered form (prefill): per (b, KV head, query block) the keys any row of the
  // block keeps, ascending, padded to whole 64-key tiles; list_idx == nullptr when unused
  const int32_t* list_idx;       // [B * Hkv, nqb, list_cap] key index (Lk in the padding)
  const int32_t* list_rank;      // same layout, the key's rank (INT32_MAX in the padding)
  const float* list_zh;          // same layout, zero_hold * log2(e) (0 in the padding)
  const int32_t* list_count;     // [B * Hkv, nqb] keys listed
  int list_cap;                  // entries per list (a multiple of 64)
  // varlen (attn_fwd_varlen): q/out token-major [total_q, Hq, d], lse [total_q, Hq];
  // K/V paged [kv_rows pages, 1 << page_shift, Hkv, d] through block_table, or packed
  // [kv_rows, Hkv, d] at the cu_k offsets when block_table == nullptr
  const int32_t* cu_q;          // [num_seqs + 1]
  const int32_t* cu_k;          // [num_seqs + 1]
  const int32_t* block_table;   // [num_seqs, max_pages]
  const void* k_new;            // two-source form: [total_q, Hkv, d], the last Lq keys
  const void* v_new;
  // work lists built on the device (varlen_plan_kernel): a unit is (sequence, query
  // block), split into items, each a key range [k0, k1) handled by one workgroup per KV
  // head. Units with one item write the output; the others write partials that
  // varlen_merge_kernel combines.
  const int4* vl_units;         // {sequence, query block, first item, items | decode-type << 30}
  const int4* vl_items;         // the launching kernel's list: {unit, k0, k1, 0}
  const int32_t* vl_counts;     // {units, prefill-type items, decode-type items}
  int vl_items_cap;             // entries of each item list (grid x = vl_items_cap * Hkv)
  int num_seqs, total_q, max_pages, page_shift, kv_rows;
  float* part_out;         // split-KV partials [splits, B*Hq*Lq, d] fp32, or per varlen item
                           // [items_cap, Hkv, rows per workgroup, d]
  float* part_lse;         // the matching LSE partials (natural log)
  int B, Hq, Hkv, Lq, Lk, d;
  int G;                   // Hq / Hkv
  float scale;
  int mask_kind;
  int window_left;
  int keep_k;
  int no_skip;
  int splits;
  int keys_per_split;
  int block_n;
  int q_per_block;         // query positions per workgroup (summary granularity)
  // Element strides of q, k, v and out: {batch, head, row}; the head dimension is
  // contiguous. attn_fwd passes the contiguous ones. (Not used by the varlen kernels.)
  long qs[3], ks[3], vs[3], os[3];
  // dense mask element (b, h, i, j) at mask[b*ms[0] + h*ms[1] + i*ms[2] + j*ms[3]]; a
  // zero stride shares the mask over that dimension
  long ms[4];
  // dense-mask summary flags: [flag_b][flag_g][query blocks][tiles], flag_b = B when
  // the mask varies with the batch (else 1), flag_g = Hkv when it varies with the head
  int flag_b, flag_g;
  const float* alibi;      // [Hq] slopes or nullptr: logit -= slope_h * |p_i - j|
  float softcap;           // > 0: logit -> softcap * tanh(logit / softcap) before the bias
  int topk_causal;         // top-k among causally allowed keys (1) or among all keys (0)
  // backward (attn_bwd): the output gradient and the gradients, laid out like out, q, k, v.
  // bwd_side: three arrays of B*Hq*Lq 4-byte values, each [B, Hkv, Lq * G] with the rows
  // of one KV head query-major (row r = i * G + (h - g * G)): -lse * log2(e) (-inf for a
  // row that sees no key), rowsum(dout * out), and the row's top-k threshold (top-k) or
  // query index i (dense mask). The dQ kernel writes them; the dK/dV kernel reads them.
  // one-tile dump (attn_fwd_dump): when dump != nullptr, the workgroup of (batch * Hkv +
  // KV head) = dump_bg and query block dump_qb writes the intermediates of key tile
  // dump_tile (see MI_ATTN_DUMP_FLOATS); nullptr otherwise
  float* dump;
  int dump_bg, dump_qb, dump_tile;
  // query blocks of the prefill grid. For the key-position masks with one split, when it
  // exceeds gridDim.x the grid holds only the workgroups the device runs at once and each
  // takes several blocks (see prefill_kernel); otherwise it equals gridDim.x.
  unsigned n_blocks;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* bwd_side;
};

// Whether a call carries a per-element score modifier (every tile is then modified).
__host__ __device__ inline bool has_mods(const AttnParams& p) { return p.softcap > 0.f || p.alibi != nullptr; }

// The mask kind whose bounds limit the visited key range: top-k over all keys visits
// every key, like no mask.
__host__ __device__ inline int range_kind(const AttnParams& p) {
  return (p.mask_kind == MI_ATTN_MASK_TOPK && !p.topk_causal) ? MI_ATTN_MASK_NONE : p.mask_kind;
}

// Visible key range [lo, hi) for a contiguous span of query positions [p0, p1]
// (positions are bottom-right aligned). Keys outside the range are hidden for every
// row of the span; keys inside may still be hidden per element.
__host__ __device__ inline void key_range(int mask_kind, int window_left, int Lk, int p0, int p1,
                                          int* lo, int* hi) {
  int a = 0, b = Lk;
  if (mask_kind == MI_ATTN_MASK_CAUSAL || mask_kind == MI_ATTN_MASK_TOPK ||
      mask_kind == MI_ATTN_MASK_WINDOW) {
    b = p1 + 1 < Lk ? p1 + 1 : Lk;
    if (b < 0) b = 0;
  }
  if (mask_kind == MI_ATTN_MASK_WINDOW) {
    a = p0 - window_left;
    if (a < 0) a = 0;
  }
  if (a > b) a = b;
  *lo = a;
  *hi = b;
}

// ------------------------------------------------------------------ launchers
hipError_t launch_row_kernel(const AttnParams& p, int dtype, hipStream_t s);
// backward: the dQ kernel (which also writes the row side arrays), then the dK/dV
// kernel (contiguous layouts, fp16/bf16, d 64 or 128)
hipError_t launch_backward(const AttnParams& p, int dtype, hipStream_t s);
// tile_min (optional, [BH, ceil(Lk / block_n)]) receives the smallest rank of each
// block_n-key tile; block_n must divide 256 and be at most 64.
// sort_ws: topk_sort_ws_bytes(BH, Lk) bytes of device memory for the sorted key chunks.
// lists (optional, causal only): the kept-key lists of the gathered attention, written by
// the threshold kernel itself (see launch_topk_lists for their layout).
struct TopkListArgs {
  const float* zh;
  int q_per_block, nqb, cap;
  int32_t *lidx, *lrank, *lcount;
  float* lzh;
};
hipError_t launch_topk(const float* zh, int BH, int Lq, int Lk, int keep_k, int causal,
                       int32_t* rank, int32_t* tau, uint32_t* keep_bits, int32_t* tile_min, int block_n,
                       hipStream_t s, void* sort_ws, const TopkListArgs* lists = nullptr);
size_t topk_sort_ws_bytes(int BH, int Lk);
// Kept-key lists of the gathered top-k attention (see AttnParams::list_*).
// causal == 0: every row may keep any key (the lists hold the keys of rank <= tau).
hipError_t launch_topk_lists(const int32_t* rank, const int32_t* tau, const float* zh, int BH, int Lq, int Lk,
                             int q_per_block, int cap, int causal, int32_t* list_idx, int32_t* list_rank,
                             float* list_zh, int32_t* list_count, hipStream_t s);
// Dense-mask summary flags (see AttnParams::flag_b): 1 iff some entry of the tile is
// above -inf for some row of the query block and some query head of the KV head.
hipError_t launch_mask_summary(const AttnParams& p, int block_n, uint8_t* flags, hipStream_t s);

}  // namespace mi_attn
