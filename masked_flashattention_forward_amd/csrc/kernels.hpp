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

}  // namespace mi_attn
