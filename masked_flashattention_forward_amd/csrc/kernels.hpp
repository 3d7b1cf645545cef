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
int prefill_block_n(int d);

// Varlen / paged forward (attn_fwd_varlen): query positions per workgroup for G heads
// per KV head, the key-range split count, and the launch (schedule kernel, MFMA kernel,
// and the LSE merge when split). sched must hold p.sched_cap entries.
int varlen_q_per_block(int G);
int varlen_splits(long blocks, int max_seqlen_k, int force_splits);
hipError_t launch_prefill_varlen(const AttnParams& p, int dtype, int2* sched, int32_t* sched_count, hipStream_t s);

}  // namespace mi_attn
