// Path choice for fp16/bf16 inputs:
//   1  MFMA prefill kernel over the whole key range, or split into key ranges whose
//      partial results are merged by log-sum-exp when there are too few workgroups;
//   2  split-KV decode kernel, for at most 32 query rows per KV head (G * Lq).
#include "kernels.hpp"

namespace mi_attn {

int decode_block_n();
int decode_max_rows();
hipError_t launch_prefill(const AttnParams& p, int dtype, hipStream_t s);
hipError_t launch_decode(const AttnParams& p, int dtype, hipStream_t s);

namespace {

constexpr int kTargetBlocks = 2048;      // prefill: ~8 workgroups per CU over 256 CUs
constexpr int kMinTilesPerSplit = 8;
constexpr int kDecodeTargetBlocks = 512;  // decode: 2 resident workgroups per CU
constexpr int kDecodeMinKeysPerSplit = 512;  // 4 tiles of 32 keys per wavefront

int q_per_block_for(int G) { return prefill_block_m() / G; }

int auto_splits(int blocks, int Lk, int bn) {
  if (blocks >= kTargetBlocks / 2) return 1;
  // every split keeps at least kMinTilesPerSplit tiles (a shorter one does not repay the
  // merge kernel)
  const int max_by_len = ((Lk + bn - 1) / bn) / kMinTilesPerSplit;
  int s = (kTargetBlocks + blocks - 1) / blocks;
  if (s > max_by_len) s = max_by_len;
  return s < 1 ? 1 : s;
}

int decode_splits(int groups, int Lk) {
  int s = (kDecodeTargetBlocks + groups - 1) / groups;
  const int max_by_len = (Lk + kDecodeMinKeysPerSplit - 1) / kDecodeMinKeysPerSplit;
  if (s > max_by_len) s = max_by_len;
  return s < 1 ? 1 : s;
}

long prefill_blocks(int B, int Hkv, int G, int Lq) {
  const int qpb = q_per_block_for(G);
  return static_cast<long>(B) * Hkv * ((Lq + qpb - 1) / qpb);
}

}  // namespace

bool half_path_available(int path, int d, int G, int Lq) {
  if (d != 64 && d != 128) return false;
  if (path == 1) return G <= prefill_block_m();
  if (path == 2) return static_cast<long>(G) * Lq <= decode_max_rows();
  return false;
}

int choose_half_path(int B, int Hkv, int G, int Lq, int Lk, int d, int /*mask_kind*/) {
  if (!half_path_available(1, d, G, Lq)) return half_path_available(2, d, G, Lq) ? 2 : 0;
  const long blocks = prefill_blocks(B, Hkv, G, Lq);
  // few query rows per KV head and a long key range: stream it with the decode kernel
  if (half_path_available(2, d, G, Lq) && blocks < kTargetBlocks / 2 && Lk >= 2 * kDecodeMinKeysPerSplit) return 2;
  return 1;
}

HalfPlan plan_half_path(int path, int B, int Hkv, int G, int Lq, int Lk, int d, int mask_kind,
                        int /*window_left*/, int force_splits) {
  HalfPlan h{};
  int splits = 1;
  if (path == 2) {
    h.block_m = decode_max_rows();
    h.block_n = decode_block_n();
    h.q_per_block = Lq;  // all query rows of a KV head in one workgroup
    h.grid = B * Hkv;
    splits = force_splits > 0 ? force_splits : decode_splits(h.grid, Lk);
  } else {
    h.block_m = prefill_block_m();
    h.block_n = prefill_block_n(d, mask_kind);
    h.q_per_block = q_per_block_for(G);
    const long blocks = prefill_blocks(B, Hkv, G, Lq);
    h.grid = static_cast<int>(blocks < 0x7fffffff ? blocks : 0x7fffffff);
    splits = force_splits > 0 ? force_splits : auto_splits(h.grid, Lk, h.block_n);
  }
  // split boundaries fall on tile boundaries
  const int tiles = (Lk + h.block_n - 1) / h.block_n;
  if (splits > tiles) splits = tiles;
  if (splits < 1) splits = 1;
  const int tiles_per_split = (tiles + splits - 1) / splits;
  h.splits = (tiles + tiles_per_split - 1) / tiles_per_split;
  return h;
}

int varlen_q_per_block(int G) { return q_per_block_for(G); }

int varlen_target_items(int Hkv) {
  const int t = kTargetBlocks / (Hkv > 0 ? Hkv : 1);
  return t < 1 ? 1 : t;
}

hipError_t launch_half_path(int path, const AttnParams& p, int dtype, hipStream_t s) {
  return path == 2 ? launch_decode(p, dtype, s) : launch_prefill(p, dtype, s);
}

}  // namespace mi_attn
