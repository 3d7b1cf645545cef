// Planning and launch interface of the fp16/bf16 kernels (MFMA prefill, split-KV decode).
#pragma once

#include "common.hpp"

namespace mi_attn {

struct HalfPlan {
  int block_m;      // query rows per workgroup
  int block_n;      // keys per KV tile
  int q_per_block;  // query positions per workgroup
  int grid;         // workgroups of the main kernel
  int splits;       // key-range splits (decode path)
};

// Path the planner picks for fp16/bf16 inputs: 0 row kernel, 1 MFMA prefill, 2 split-KV decode.
int choose_half_path(int B, int Hkv, int G, int Lq, int Lk, int d, int mask_kind);
// Whether `path` can run this head dim and rows-per-KV-head count.
bool half_path_available(int path, int d, int G, int Lq);
HalfPlan plan_half_path(int path, int B, int Hkv, int G, int Lq, int Lk, int d, int mask_kind, int window_left,
                        int force_splits);
hipError_t launch_half_path(int path, const AttnParams& p, int dtype, hipStream_t s);

// MFMA prefill tile shape: query rows and keys per workgroup tile.
int prefill_block_m();
// keys per tile of the MFMA prefill kernel for head dim d and a mask kind
int prefill_block_n(int d, int mask_kind);

// Varlen / paged forward (attn_fwd_varlen): device-built work lists (units and items, see
// k_varlen.hip), the MFMA prefill and split-KV decode kernels over them, and the LSE
// merge of units split into several items. Buffers are sized by the host:
//   units    int4 [units_cap]        items_p, items_d  int4 [items_cap]     counts int32 [3]
//   pp_out   fp32 [items_cap, Hkv, 128, d]   pp_lse  [items_cap, Hkv, 128]
//   pd_out   fp32 [items_cap, Hkv, 32, d]    pd_lse  [items_cap, Hkv, 32]
constexpr int kVarlenPrefillRows = 128;  // = prefill_block_m(): partial rows per prefill-type item
struct VarlenBuffers {
  int4* units;
  int4* items_p;
  int4* items_d;
  int32_t* counts;
  float* pp_out;
  float* pp_lse;
  float* pd_out;
  float* pd_lse;
  int units_cap;     // >= the number of (sequence, query block) units
  int items_cap;     // varlen_items_cap(units_cap, target_items, force_items)
  int target_items;  // items per type the plan aims for
  int force_items;   // > 0: exactly this many items per unit (fewer for short units)
};
int varlen_q_per_block(int G);
int varlen_target_items(int Hkv);
int varlen_items_cap(int units_cap, int target_items, int force);
hipError_t launch_varlen(const AttnParams& p, int dtype, const VarlenBuffers& b, hipStream_t s);

}  // namespace mi_attn
