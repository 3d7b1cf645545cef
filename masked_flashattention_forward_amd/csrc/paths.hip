// Path choice for fp16/bf16 inputs: the MFMA kernel over the whole key range (path 1) or
// split into key ranges whose partial results are merged by log-sum-exp (path 2).
#include "kernels.hpp"

namespace mi_attn {

int prefill_block_n(int d);
int prefill_block_m();
hipError_t launch_prefill(const AttnParams& p, int dtype, hipStream_t s);

namespace {

constexpr int kTargetBlocks = 2048;   // ~8 workgroups per CU over 256 CUs
constexpr int kMinTilesPerSplit = 8;

int q_per_block_for(int G) { return prefill_block_m() / G; }

int auto_splits(int blocks, int Lk, int bn) {
  if (blocks >= kTargetBlocks / 2) return 1;
  const int max_by_len = (Lk + bn * kMinTilesPerSplit - 1) / (bn * kMinTilesPerSplit);
  int s = (kTargetBlocks + blocks - 1) / blocks;
  if (s > max_by_len) s = max_by_len;
  return s < 1 ? 1 : s;
}

}  // namespace

bool half_path_available(int path, int d, int G, int /*Lq*/) {
  if (path != 1 && path != 2) return false;
  return (d == 64 || d == 128) && G <= prefill_block_m();
}

int choose_half_path(int B, int Hkv, int G, int Lq, int Lk, int d, int /*mask_kind*/) {
  if (!half_path_available(1, d, G, Lq)) return 0;
  const int qpb = q_per_block_for(G);
  const long blocks = static_cast<long>(B) * Hkv * ((Lq + qpb - 1) / qpb);
  return auto_splits(static_cast<int>(blocks < 0x7fffffff ? blocks : 0x7fffffff), Lk, prefill_block_n(d)) > 1 ? 2 : 1;
}

HalfPlan plan_half_path(int path, int B, int Hkv, int G, int Lq, int Lk, int d, int /*mask_kind*/,
                        int /*window_left*/, int force_splits) {
  HalfPlan h{};
  h.block_m = prefill_block_m();
  h.block_n = prefill_block_n(d);
  h.q_per_block = q_per_block_for(G);
  const long blocks = static_cast<long>(B) * Hkv * ((Lq + h.q_per_block - 1) / h.q_per_block);
  h.grid = static_cast<int>(blocks < 0x7fffffff ? blocks : 0x7fffffff);
  int splits = 1;
  if (path == 2) {
    splits = force_splits > 0 ? force_splits : auto_splits(h.grid, Lk, h.block_n);
    if (splits < 2) splits = 2;
  }
  // split boundaries fall on tile boundaries
  const int tiles = (Lk + h.block_n - 1) / h.block_n;
  if (splits > tiles) splits = tiles;
  if (splits < 1) splits = 1;
  const int tiles_per_split = (tiles + splits - 1) / splits;
  h.splits = (tiles + tiles_per_split - 1) / tiles_per_split;
  return h;
}

hipError_t launch_half_path(int /*path*/, const AttnParams& p, int dtype, hipStream_t s) {
  return launch_prefill(p, dtype, s);
}

}  // namespace mi_attn
