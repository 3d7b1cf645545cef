// MFMA prefill kernel for fp16/bf16 inputs, head dim 64 or 128, every mask kind.
//
// Work unit: one workgroup = 4 wavefronts = up to 128 query rows of ONE (batch, KV head)
// group. Rows are the query heads sharing that KV head, packed query-major
// (row r -> query i = r / G, head g*G + r % G), so a K/V tile staged once in LDS serves
// all G heads (InfiniTrain page, "Transformer integration": the flash path keeps the
// original KV heads instead of expanding them).
//
// Per KV tile of BN keys (64; 128 for the position masks at d = 64) (ExecuTorch page,
// "Summary": chunks along the key dimension, online softmax finalised at the end):
//   S^T = K Q^T      v_mfma_f32_32x32x16 (K from LDS as the A operand, Q^T from registers).
//                    Each lane then holds one query column and 16 keys per 32-key block,
//                    so the row max/sum is in-lane plus one exchange with lane ^ 32.
//   mask             only on tiles the mask does not cover entirely (boundary tiles).
//   online softmax   running max m and sum l per row in the log2 domain, guarded so an
//                    all -inf tile (or row) never produces exp(-inf - -inf); where the
//                    registers allow, the exponentials are taken against the running max
//                    as it stands and the max is reduced only on the rare tile that moves
//                    it (see kRunningMaxExps).
//   O^T += V^T P^T   P^T straight from the S^T registers (packed to 16 bit) as the B
//                    operand; V stays in LDS row-major and its A operand comes from
//                    transposed reads (ds_read_b64_tr_b16) whose lane-to-key map matches
//                    the keys each lane's P registers hold.
// Tiles that the mask hides entirely are never loaded: their range comes from the causal
// / window bounds, the dense-mask summary flags or in-kernel scan, or the top-k kept-key
// lists and minimum rank per tile.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "mfma_common.hpp"

namespace mi_attn {

namespace {

using namespace mfma;

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kBlockM = 32 * kWaves;  // query rows per workgroup
constexpr int kDumpRows = kBlockM;      // rows of a one-tile dump
static_assert(kBlockM == kVarlenPrefillRows, "varlen partial slots hold one workgroup's rows");

template <int D, int BN>
struct Tile {
  static constexpr int rowBytes = D * 2;
  static constexpr int kBytes = BN * rowBytes;          // K tile, [key][d], no padding
  static constexpr int vBytes = BN * rowBytes;          // V tile, [key][d], no padding
  // top-k side data: BN int32 ranks, BN fp32 values (zero_hold * log2 e), BN int32 key
  // indices (gathered form), padded to keep the stage a multiple of 512 bytes
  static constexpr int xBytes = 16 * BN;
  static constexpr int stage = kBytes + vBytes + xBytes;
  static constexpr int rowsPerWaveLoad = 1024 / rowBytes;  // one wave's 64 x 16 B direct load
  static constexpr int loadRounds = kBytes / (kThreads * 16);
  static_assert(loadRounds * kThreads * 16 == kBytes, "tile split evenly across direct loads");
  static_assert(BN <= kThreads, "one top-k side entry per thread");
};

// log2 of the keys one round of direct loads covers (4 waves x 1 KB of 2*D-byte rows)
template <int D>
constexpr int kLog2RoundKeys = (D == 128) ? 4 : 5;
constexpr int kLog2BN = 6;  // 64-key tiles

// resident workgroups per CU: LDS allows 2 for d = 128 and for 128-key tiles at d = 64,
// and 4 for 64-key tiles at d = 64. There the top-k variant's extra state and the score
// modifiers (EXT) keep it at 2, and the varlen variant's per-row addressing and the dense
// mask's liveness scan at 3 (4 would cap them at 128 VGPRs and spill).
template <int D, int MK, bool VARLEN, bool EXT, int BN>
constexpr int kMinBlocks = (D == 128 || BN == 128) ? 2
                           : (MK == MI_ATTN_MASK_TOPK || EXT) ? 2
                           : (VARLEN || MK == MI_ATTN_MASK_DENSE) ? 3
                                                                   : 4;

// Keys per tile of the position-mask (none / causal / window) instances: 128 at d = 64,
// where the tile's fixed costs (barrier, loads, bookkeeping) would otherwise be spread
// over half the MFMA work of d = 128 (c4 d64: 654 -> 609 us with the max still reduced
// first); 64 at d = 128 (two 64 KB stages per workgroup leave room for two per CU). The
// dense, top-k and varlen instances take 64-key tiles.
template <int D>
constexpr int kPosBN = D == 64 ? 128 : 64;
// Instances whose grid may run as resident workgroups that take several query blocks:
// the key-position masks, whose block costs fall off steadily with the heavy-first block
// order (the dense and top-k kinds keep one workgroup per block, which the dispatcher
// balances by itself when block costs vary with the mask)
template <int MK, bool VARLEN>
constexpr bool kResident = !VARLEN && MK <= MI_ATTN_MASK_WINDOW;

// Softmax against the running max without a per-tile max reduction (see the tile loop).
// Its second code path does not fit the registers with 64-key tiles at d = 64 (4
// workgroups per CU, 128 VGPRs) nor beside the score modifiers' state, and for a dense
// mask it would read the mask entries of a tile twice; those reduce the max first.
template <int D, int BN, int MK, bool EXT>
constexpr bool kRunningMaxExps = (D == 128 || BN == 128) && !EXT && MK != MI_ATTN_MASK_DENSE;

// GATHER (top-k only): tiles are consecutive 64-key runs of the block's kept-key list
// (AttnParams::list_*) instead of consecutive keys, so only keys some row of the block
// keeps are loaded and multiplied.
// VARLEN: a batch of sequences of different lengths (vLLM pull request #11277 page, the
// varlen call with cu_seqlens and a block table): queries token-major, a workgroup takes
// one item of the device-built work list (a key range of one (sequence, query block)),
// and each K/V row is fetched from its own cache page (or packed row, or the new-token
// array of the two-source form) with a per-lane 64-bit address.
// DUMP: the instance attn_fwd_dump runs (AttnParams::dump set): one workgroup writes the
// intermediates of one tile. The checks live only in these instances, so the others
// carry no per-tile test for it (it cost 1.5% at c4 d128).
template <typename T, int D, int BN, int MK, bool GATHER = false, bool VARLEN = false, bool EXT = false,
          bool DUMP = false>
__global__ __launch_bounds__(kThreads, (kMinBlocks<D, MK, VARLEN, EXT, BN>)) void prefill_kernel(AttnParams p) {
  static_assert(!GATHER || (MK == MI_ATTN_MASK_TOPK && BN == 64), "gathered tiles are top-k lists of 64 keys");
  static_assert(!VARLEN || (!GATHER && MK <= MI_ATTN_MASK_WINDOW), "varlen takes the key-position masks");
  static_assert(!DUMP || (BN == 64 && !VARLEN && !EXT), "the dump covers 64-key tiles without score modifiers");
  using TL = Tile<D, BN>;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * TL::stage];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // uniform, so wave-derived values stay scalar
  const int lane = tid % kWave;
  const int l32 = lane & 31;
  const int hf = lane >> 5;  // lane half

  // ---- work unit: (b, g, query block, split), or a varlen item and g
  const int split = blockIdx.y;
  // One query block (VARLEN: one work item). Workgroup-wide returns inside end this block
  // only; a lane's early return skips its own output and nothing else.
  auto run_block = [&](const unsigned lb) {
    int nqb = 1, qb, bg, b, g, Lq, Lk;
    VarlenSeq sq{};
    int item = 0, k0 = 0, k1 = 0;  // VARLEN: item, its key range
    bool item_partial = false;     // VARLEN: the unit has several items (partials + merge)
    if constexpr (VARLEN) {
      // The grid is sized for the most items possible; the valid (item, KV head) pairs
      // are spread evenly over the 8 XCDs (workgroups go to XCDs round-robin), each XCD
      // taking a contiguous run of items of one KV head, so the query blocks of a
      // sequence, which share its K/V, run together on one XCD and its L2.
      (void)lb;
      const int n_items = p.vl_counts[1];
      const int n_work = n_items * p.Hkv;
      const int per_xcd = (n_work + 7) / 8;
      const int k_in_xcd = static_cast<int>(blockIdx.x / 8u);
      const int w = static_cast<int>(blockIdx.x % 8u) * per_xcd + k_in_xcd;
      if (k_in_xcd >= per_xcd || w >= n_work) return;  // the whole workgroup, before any barrier
      g = w / n_items;
      item = w % n_items;
      const int4 it = p.vl_items[item];
      const int4 un = p.vl_units[it.x];
      sq = varlen_seq(p, un.x);
      sq.q_start = __builtin_amdgcn_readfirstlane(sq.q_start);  // uniform: keep them scalar
      sq.Lq = __builtin_amdgcn_readfirstlane(sq.Lq);
      sq.Lk = __builtin_amdgcn_readfirstlane(sq.Lk);
      sq.ctx = __builtin_amdgcn_readfirstlane(sq.ctx);
      sq.k_start = __builtin_amdgcn_readfirstlane(sq.k_start);
      qb = un.y;
      item_partial = (un.w & 0x3fffffff) > 1;
      k0 = it.y;
      k1 = it.z;
      Lq = sq.Lq;
      Lk = sq.Lk;
      b = 0;
      bg = 0;
    } else {
      Lq = p.Lq;
      Lk = p.Lk;
      nqb = (Lq + p.q_per_block - 1) / p.q_per_block;
      qb = nqb - 1 - static_cast<int>(lb % nqb);
      bg = static_cast<int>(lb / nqb);
      b = bg / p.Hkv;
      g = bg % p.Hkv;
    }
    const int i_first = qb * p.q_per_block;
    const int i_last = min(Lq, i_first + p.q_per_block) - 1;
    const int rows_blk = (i_last - i_first + 1) * p.G;
    const int P0 = Lk - Lq + i_first;
    const int P1 = Lk - Lq + i_last;

    // ---- this lane's query row (the S^T column it owns)
    const int rloc = wave * 32 + l32;
    const bool row_ok = rloc < rows_blk;
    const int i_row = i_first + (row_ok ? rloc / p.G : 0);
    const int h_row = g * p.G + (row_ok ? rloc % p.G : 0);
    const int pos = Lk - Lq + i_row;
    // output row: [B, Hq, Lq] order, or token-major [total_q, Hq] for VARLEN
    const long row_index = VARLEN ? static_cast<long>(sq.q_start + i_row) * p.Hq + h_row
                                  : (static_cast<long>(b) * p.Hq + h_row) * Lq + i_row;
    const long rows_all = VARLEN ? static_cast<long>(p.total_q) * p.Hq : static_cast<long>(p.B) * p.Hq * Lq;

    // element offsets of this lane's q and out rows (strided for the single-batch call)
    const long q_off = VARLEN ? row_index * D : b * p.qs[0] + h_row * p.qs[1] + i_row * p.qs[2];
    const long o_off = VARLEN ? row_index * D : b * p.os[0] + h_row * p.os[1] + i_row * p.os[2];

    // ---- Q^T operand in registers: lane holds 8 dims (dc*16 + hf*8 ..) of its row
    const T* Q = static_cast<const T*>(p.q);
    const bool negate = p.scale < 0.f;  // fold the sign into Q so the log2-domain scale is > 0
    const float cexp = fabsf(p.scale) * kLog2e;
    // score modifiers and the dense mask row of this lane (rows past the block read row i_first)
    const Mods md = make_mods<EXT>(p, cexp, b, h_row, i_row, pos, MK == MI_ATTN_MASK_DENSE || MK == MI_ATTN_MASK_TOPK);
    // dense: every lane's mask row is contiguous and 16-byte aligned (the strides of the
    // dimensions in use and the base are multiples of 4 floats)
    const bool dense_vec = MK == MI_ATTN_MASK_DENSE && p.mask != nullptr && p.ms[3] == 1 && (p.ms[2] & 3) == 0 &&
                           (p.ms[1] & 3) == 0 && (p.ms[0] & 3) == 0 && (reinterpret_cast<uintptr_t>(p.mask) & 15) == 0;
    u32x4_t qreg[D / 16];
#pragma unroll
    for (int dc = 0; dc < D / 16; ++dc) {
      u32x4_t x = {0u, 0u, 0u, 0u};
      if (row_ok) x = *reinterpret_cast<const u32x4_t*>(Q + q_off + dc * 16 + hf * 8);
      if (negate) x ^= 0x80008000u;
      qreg[dc] = x;
    }

    // ---- key range of this block (and split)
    int lo, hi;
    key_range(range_kind(p), p.window_left, Lk, P0, P1, &lo, &hi);
    if (p.no_skip) { lo = 0; hi = Lk; }
    if (VARLEN) {
      // the item's range: part of [lo, hi) cut on tile boundaries by the work-list kernel
      // (empty for a two-source sequence with fewer keys than queries)
      lo = k0;
      hi = k1;
    } else if (p.splits > 1) {
      const int s0 = split * p.keys_per_split;
      const int s1 = min(Lk, s0 + p.keys_per_split);
      lo = max(lo, s0);
      hi = min(hi, s1);
      if (hi < lo) hi = lo;
    }
    const int ntiles_all = (Lk + BN - 1) / BN;
    int t_lo = lo / BN;
    // an empty range visits no tile (a rounded-up end would reach into the next split)
    int t_hi = (hi > lo) ? (hi + BN - 1) / BN : t_lo;
    long list_base = 0;  // GATHER: this block's kept-key list; tile t = entries [t*BN, t*BN + BN)
    if constexpr (GATHER) {
      const long li = static_cast<long>(bg) * nqb + qb;
      list_base = li * p.list_cap;
      const int ntl = (p.list_count[li] + BN - 1) / BN;
      const int per = p.keys_per_split / BN;  // list tiles per split
      t_lo = split * per;
      t_hi = min(ntl, t_lo + per);
      if (t_hi < t_lo) t_hi = t_lo;
    }

    // VARLEN base pointers, held in registers so that the per-lane choice between the cache
    // and the new-token arrays selects values, not kernel-argument addresses
    const T* const k_cache = static_cast<const T*>(p.k);
    const T* const v_cache = static_cast<const T*>(p.v);
    const T* const k_fresh = static_cast<const T*>(p.k_new);
    const T* const v_fresh = static_cast<const T*>(p.v_new);
    // K / V of this (batch, KV head): rows ks / vs elements apart (D for contiguous K/V)
    const long ksr = VARLEN ? D : p.ks[2];
    const long vsr = VARLEN ? D : p.vs[2];
    const T* K = static_cast<const T*>(p.k) + (VARLEN ? 0 : b * p.ks[0] + g * p.ks[1]);
    const T* V = static_cast<const T*>(p.v) + (VARLEN ? 0 : b * p.vs[0] + g * p.vs[1]);
    const long bgk = static_cast<long>(bg) * Lk;

    // top-k: the block's largest threshold (thresholds do not grow with the row position)
    int32_t tau_row = 0, tau_blk = 0;
    if constexpr (MK == MI_ATTN_MASK_TOPK) {
      // ranks of real keys are below Lk: the clamp keeps every allowed key when tau says
      // "all kept" (INT32_MAX) and never keeps padding keys (rank INT32_MAX)
      tau_row = min(p.tau[static_cast<long>(bg) * p.Lq + i_row], Lk - 1);
      tau_blk = min(p.tau[static_cast<long>(bg) * p.Lq + i_first], Lk - 1);
    }
    // dense-mask summary flags of this (batch, KV head), query block
    const long flag_base = ((static_cast<long>(p.flag_b > 1 ? b : 0) * p.flag_g + (p.flag_g > 1 ? g : 0)) * nqb + qb) *
                           ntiles_all;
    // Dense masks over short key ranges come without summary flags (no separate pass):
    // the workgroup reads its own rows' mask entries over its tiles (at most 32 of them)
    // once, up front, and keeps one live bit per tile.
    uint32_t live_bits = 0xffffffffu;
    if constexpr (MK == MI_ATTN_MASK_DENSE) {
      if (p.tile_live == nullptr && !p.no_skip && t_hi > t_lo && t_hi - t_lo <= 32) {
        __shared__ uint32_t live_shared;
        if (tid == 0) live_shared = 0u;
        // rows whose entries differ: the block's positions, times its query heads when the
        // mask varies with the head
        const int nh = (p.Hq > 1 && p.ms[1] != 0) ? p.G : 1;
        const int j_lo = t_lo * BN;
        const int nk = min(t_hi * BN, Lk) - j_lo;
        const int nrows = (i_last - i_first + 1) * nh;
        const float* mb = p.mask + b * p.ms[0] + static_cast<long>(g) * p.G * p.ms[1];
        uint32_t bits = 0u;
        // A thread takes a group of keys (4 consecutive ones when rows are contiguous and
        // aligned, else 1) of every row, consecutive threads consecutive groups. Rows advance
        // as (position, head) pairs with wave-uniform offsets, sixteen independent loads per
        // pass so their latencies overlap. A group never straddles a tile.
        constexpr int kUnroll = 16;
        const int gk = dense_vec ? 4 : 1;
        for (int kk = tid * gk; kk < nk; kk += kThreads * gk) {
          const float* col = mb + static_cast<long>(j_lo + kk) * p.ms[3];
          const bool whole = dense_vec && kk + 3 < nk;  // a 16-byte load covers the group
          int h = 0;
          long roff = static_cast<long>(i_first) * p.ms[2];  // offset of row (i_first, head 0)
          bool live = false;
          for (int r0 = 0; r0 < nrows; r0 += kUnroll) {
            float mv[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
              const float* a = col + roff + h * p.ms[1];
              float m = kNegInf;
              if (r0 + u < nrows) {
                if (whole) {
                  const float4 q4 = *reinterpret_cast<const float4*>(a);
                  m = fmaxf(fmaxf(q4.x, q4.y), fmaxf(q4.z, q4.w));
                } else {
                  for (int e = 0; e < gk && kk + e < nk; ++e) m = fmaxf(m, a[e * p.ms[3]]);
                }
              }
              mv[u] = m;
              if (++h == nh) {
                h = 0;
                roff += p.ms[2];
              }
            }
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) live = live || mv[u] > kNegInf;
          }
          if (live) bits |= 1u << (kk / BN);
        }
        __syncthreads();
        if (bits != 0u) atomicOr(&live_shared, bits);
        __syncthreads();
        live_bits = live_shared;
      }
    }
    auto tile_live = [&](int t) -> bool {
      if (GATHER || p.no_skip) return true;
      if constexpr (MK == MI_ATTN_MASK_DENSE)
        return p.tile_live == nullptr ? ((live_bits >> (t - t_lo)) & 1u) != 0 : p.tile_live[flag_base + t] != 0;
      if constexpr (MK == MI_ATTN_MASK_TOPK)
        return p.tile_min_rank[static_cast<long>(bg) * ntiles_all + t] <= tau_blk;
      return true;
    };
    auto next_live = [&](int t) -> int {
      while (t < t_hi && !tile_live(t)) ++t;
      return t;
    };

    // ---- tile loads straight into LDS (buffer_load ... lds): each wave instruction fills
    // 1 KB of the tile; lane i of it takes the global 16-byte chunk that belongs in slot i
    // of the swizzled layout. Rows at or past Lk read as zeros (buffer range check). A
    // lane's swizzle does not depend on the load round, so its global offset is one
    // loop-invariant register plus a wave-uniform (scalar) offset for the tile and round.
    // the range covers rows 0 .. Lk-1 (the host keeps it below 2^31 bytes)
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(K, VARLEN ? 0 : static_cast<int>(((Lk - 1) * ksr + D) * 2));
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc(V, VARLEN ? 0 : static_cast<int>(((Lk - 1) * vsr + D) * 2));
    int dma_lane_k, dma_lane_v;
    {
      const int r = wave * TL::rowsPerWaveLoad + lane / (D / 8);
      const int ps = lane % (D / 8);                   // physical slot this lane fills
      dma_lane_k = static_cast<int>((r * ksr + ((ps ^ swz<D>(r)) << 3)) * 2);
      dma_lane_v = static_cast<int>((r * vsr + ((ps ^ swz<D>(r)) << 3)) * 2);
    }
    const unsigned smem_addr = __builtin_amdgcn_readfirstlane(lds_address(smem));
    // GATHER: row r of a tile comes from key list[t*BN + r]; a lane's rows in load round c
    // are r_c = (c * kWaves + wave) * rowsPerWaveLoad + lane / (D / 8), whose swizzle does not
    // depend on c. Their key indices are loaded one tile ahead into gidx[], so the waits for
    // them fall on loads that have long completed.
    int dma_slot = 0;
    int gidx[TL::loadRounds];
    if constexpr (GATHER || VARLEN) {
      const int r = wave * TL::rowsPerWaveLoad + lane / (D / 8);
      dma_slot = ((lane % (D / 8)) ^ swz<D>(r)) << 4;
    }
    // VARLEN addressing. A load round covers kRoundKeys consecutive keys; the lane fills row
    // rl of the round at 16-byte slot dma_slot. A tile inside one source whose rounds each
    // lie in one page (or are consecutive packed or new-token rows) is loaded from per-lane
    // 64-bit addresses lane_base + row * row_bytes, one multiply-add per round, with the
    // pages of the tile's rounds read from one block-table entry per lane loaded a tile
    // ahead (lane i & 3 holds the tile's (i & 3)-th page). Other tiles (the last one, one
    // across the cached / new boundary, pages shorter than a round) address every row on
    // its own.
    constexpr int kRoundKeys = kWaves * TL::rowsPerWaveLoad;
    static_assert((1 << kLog2RoundKeys<D>) == kRoundKeys, "round keys");
    static_assert(!VARLEN || (1 << kLog2BN) == BN, "varlen tiles of 64 keys");
    static_assert(BN / kRoundKeys <= 4, "a tile of direct rounds spans at most 4 pages");
    const int page_mask = VARLEN ? (1 << p.page_shift) - 1 : 0;
    const unsigned row_bytes = static_cast<unsigned>(p.Hkv) * D * 2;  // one key's row of all KV heads
    const uint64_t lane_part = VARLEN ? static_cast<uint64_t>(g) * D * 2 +
                                            static_cast<uint64_t>(wave * TL::rowsPerWaveLoad + lane / (D / 8)) * row_bytes +
                                            dma_slot
                                      : 0;
    const uint64_t kc_lane = reinterpret_cast<uint64_t>(p.k) + lane_part;
    const uint64_t vc_lane = reinterpret_cast<uint64_t>(p.v) + lane_part;
    const uint64_t kf_lane = reinterpret_cast<uint64_t>(p.k_new) + lane_part;
    const uint64_t vf_lane = reinterpret_cast<uint64_t>(p.v_new) + lane_part;
    int pg_lane = 0;
    auto load_pages = [&](int t) {
      if (VARLEN && p.block_table != nullptr) {
        const int last = (max(sq.Lk, 1) - 1) >> p.page_shift;
        const int idx = min(min(((t * BN) >> p.page_shift) + (lane & 3), last), p.max_pages - 1);
        pg_lane = p.block_table[static_cast<long>(sq.seq) * p.max_pages + idx];
      }
    };
    // The fast form needs every row it forms to lie in its array: new-token rows always do
    // (q_start and Lq are clamped to total_q), paged rows sit in a clamped page, and packed
    // rows only when the sequence's slice [k_start + j0, k_start + j0 + BN) lies inside the
    // kv_rows rows of the cache (the lengths are caller data; anything else takes the
    // clamped per-row form).
    auto tile_direct = [&](int j0) -> bool {
      if (j0 + BN > sq.Lk) return false;
      if (j0 >= sq.ctx) return true;  // new-token rows (two-source form)
      if (j0 + BN > sq.ctx) return false;
      if (p.block_table != nullptr) return p.page_shift >= kLog2RoundKeys<D>;
      return sq.k_start >= 0 && sq.k_start <= p.kv_rows - (j0 + BN);
    };
    auto load_gidx = [&](int t) {
      if constexpr (GATHER) {
#pragma unroll
        for (int c = 0; c < TL::loadRounds; ++c) {
          const int r = (c * kWaves + wave) * TL::rowsPerWaveLoad + lane / (D / 8);
          gidx[c] = p.list_idx[list_base + t * BN + r];
        }
      }
    };
    int32_t xrank = 0, xidx = 0;
    float xzh = 0.f;
    auto issue_tile = [&](int t, int stg) {
      const int j0 = t * BN;
      const unsigned kst = smem_addr + stg * TL::stage;
      if constexpr (VARLEN) {
        if (tile_direct(j0)) {
          const bool fresh = j0 >= sq.ctx;
          const uint64_t kl = fresh ? kf_lane : kc_lane;
          const uint64_t vl = fresh ? vf_lane : vc_lane;
          // first row of each round (every index below 2^31), all formed before the first
          // load is issued: reading the page register waits for outstanding vector memory
          // operations, which must not include this tile's own loads
          unsigned row[TL::loadRounds];
#pragma unroll
          for (int c = 0; c < TL::loadRounds; ++c) {
            const int jc = j0 + c * kRoundKeys;
            if (fresh) {
              row[c] = static_cast<unsigned>(sq.q_start + (jc - sq.ctx));
            } else if (p.block_table != nullptr) {
              const int pg = min(max(__builtin_amdgcn_readlane(pg_lane, (c * kRoundKeys) >> p.page_shift), 0),
                                 p.kv_rows - 1);
              row[c] = (static_cast<unsigned>(pg) << p.page_shift) | static_cast<unsigned>(jc & page_mask);
            } else {
              row[c] = static_cast<unsigned>(sq.k_start + jc);
            }
          }
#pragma unroll
          for (int c = 0; c < TL::loadRounds; ++c) {
            const unsigned blk = (c * kWaves + wave) * 1024;
            const uint64_t off = static_cast<uint64_t>(row[c]) * row_bytes;
            lds_dma16_global(kst + blk, reinterpret_cast<const void*>(kl + off));
            lds_dma16_global(kst + TL::kBytes + blk, reinterpret_cast<const void*>(vl + off));
          }
        } else {
          // every row on its own (clamped to the last key), its page read here
          int page[TL::loadRounds];
#pragma unroll
          for (int c = 0; c < TL::loadRounds; ++c) {
            const int j = j0 + (c * kWaves + wave) * TL::rowsPerWaveLoad + lane / (D / 8);
            page[c] = p.block_table != nullptr ? varlen_page(p, sq, j) : 0;
          }
#pragma unroll
          for (int c = 0; c < TL::loadRounds; ++c) {
            const unsigned blk = (c * kWaves + wave) * 1024;
            const int j = j0 + (c * kWaves + wave) * TL::rowsPerWaveLoad + lane / (D / 8);
            bool is_new;
            const long e = varlen_row<D>(p, sq, g, j, page[c], dma_slot >> 1, &is_new);
            lds_dma16_global(kst + blk, pick(is_new, k_fresh, k_cache) + e);
            lds_dma16_global(kst + TL::kBytes + blk, pick(is_new, v_fresh, v_cache) + e);
          }
        }
      }
#pragma unroll
      for (int c = 0; c < TL::loadRounds && !VARLEN; ++c) {
        const unsigned blk = (c * kWaves + wave) * 1024;  // 1 KB block of the tile
        if constexpr (GATHER) {
          // padding entries (key Lk) lie past the buffer range and read as zeros
          lds_dma16_at(krs, kst + blk, static_cast<int>(gidx[c] * ksr * 2) + dma_slot, 0);
          lds_dma16_at(vrs, kst + TL::kBytes + blk, static_cast<int>(gidx[c] * vsr * 2) + dma_slot, 0);
        } else {
          const int row0 = j0 + c * kWaves * TL::rowsPerWaveLoad;
          lds_dma16_at(krs, kst + blk, dma_lane_k, static_cast<int>(row0 * ksr * 2));
          lds_dma16_at(vrs, kst + TL::kBytes + blk, dma_lane_v, static_cast<int>(row0 * vsr * 2));
        }
      }
      if constexpr (GATHER) {
        if (tid < BN) {
          const long e = list_base + j0 + tid;
          xrank = p.list_rank[e];
          xzh = p.list_zh[e];
          xidx = p.list_idx[e];
        }
        if (t + 1 < t_hi) load_gidx(t + 1);
      } else if constexpr (VARLEN) {
        load_pages(t + 1);  // clamped, so past the last tile it reads a valid entry
      } else if constexpr (MK == MI_ATTN_MASK_TOPK) {
        if (tid < BN) {
          const int key = j0 + tid;
          xrank = key < Lk ? p.rank[bgk + key] : 0x7fffffff;
          xzh = key < Lk ? p.zero_hold[bgk + key] * kLog2e : 0.f;
        }
      }
    };
    auto finish_tile = [&](int stg) {
      if constexpr (MK == MI_ATTN_MASK_TOPK) {
        if (tid < BN) {
          int32_t* xr = reinterpret_cast<int32_t*>(smem + stg * TL::stage + TL::kBytes + TL::vBytes);
          xr[tid] = xrank;
          reinterpret_cast<float*>(xr + BN)[tid] = xzh;
          if constexpr (GATHER) xr[2 * BN + tid] = xidx;
        }
      }
      __builtin_amdgcn_s_waitcnt(0);  // this wave's direct loads have landed
    };

    // ---- LDS operand addresses. Slot s of row r sits at ((s ^ swz(r)) << 4) in the row;
    // the swizzle bits of the rows a lane reads do not change with the 32-key block (K) or
    // the 16-key chunk (V), and the dim chunk enters as a plain XOR: a K fragment is at
    // kb * 32 * rowBytes + (k_base ^ (dc << 5)), a V^T fragment at
    // kc * 16 * rowBytes + (v_base[h] ^ (db << 6)). Stage offsets are multiples of 512
    // bytes and leave the XOR-ed address bits alone.
    int k_base, v_base0, v_base1;
    {
      k_base = l32 * TL::rowBytes | ((hf ^ swz<D>(l32)) << 4);
      const int tr_row = 4 * hf + (lane & 15) / 4;
      const int sl = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
      v_base0 = tr_row * TL::rowBytes | ((sl ^ swz<D>(tr_row)) << 4) | (8 * (lane & 1));
      v_base1 = (tr_row + 8) * TL::rowBytes | ((sl ^ swz<D>(tr_row + 8)) << 4) | (8 * (lane & 1));
    }
    static_assert(TL::stage % 512 == 0 && TL::kBytes % 512 == 0, "stage offsets keep the XOR-ed address bits");
    // The tile loop runs unrolled by two (kUnroll2) for the position masks at d = 128 and
    // with 128-key tiles at d = 64: the
    // stage is then a constant in each copy. Byte offsets in smem of a lane's K fragment (dim
    // chunk dc) and V^T fragment (dim block db) in the stage at byte offset ofs: adding a
    // multiple of 512 commutes with the XOR, so unrolled, the XOR-ed base is loop-invariant
    // and the stage offset an immediate. The other instances (d = 64 at 128 VGPRs; dense,
    // top-k and score modifiers, whose extra state leaves no room for the 16 invariant
    // addresses) keep the form that needs no extra live registers.
    constexpr bool kUnroll2 = (D == 128 || BN == 128) && MK <= MI_ATTN_MASK_WINDOW && !EXT;
    auto k_addr = [&](int dc, int ofs) -> int {
      return kUnroll2 ? (k_base ^ (dc << 5)) + ofs : ((k_base + ofs) ^ (dc << 5));
    };
    auto v_addr = [&](int vbase, int db, int ofs) -> int {
      return kUnroll2 ? (vbase ^ (db << 6)) + ofs : ((vbase + ofs) ^ (db << 6));
    };

    // ---- running state
    constexpr int NKB = BN / 32;  // 32-key blocks per tile
    constexpr int NDB = D / 32;   // 32-dim blocks of O^T
    f32x16_t oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[db] = f32x16_t{};
    float m_run = kNegInf;  // running max, log2 domain (may lag the true max by < 2^8)
    float l_run = 0.f;      // this lane's partial running sum

    int t = next_live(t_lo);
    if (t < t_hi) {
      load_gidx(t);
      load_pages(t);
      issue_tile(t, 0);
      finish_tile(0);
    }
    __syncthreads();

    // One key tile; `stage_c` is the LDS stage it sits in (an integral_constant when the loop
    // is unrolled by two, see kUnroll2; otherwise an int).
    // first_c: the block's first tile (every row's running max still -inf), peeled off the
    // unrolled loop so that it can take the exact softmax path directly
    auto tile_step = [&](auto stage_c, auto first_c) {
      const int stage = stage_c;
      const int tn = next_live(t + 1);
      if (tn < t_hi) issue_tile(tn, stage ^ 1);  // lands in the other stage while this tile computes

      const int ks_ofs = stage * TL::stage;
      const int vs_ofs = ks_ofs + TL::kBytes;
      const unsigned char* vs = smem + vs_ofs;
      const int j0 = t * BN;

      // dense, d = 128: this tile's mask entries of the lane's row, requested before the S
      // MFMAs so their latency overlaps them (at d = 64 the 32 extra registers do not fit the
      // 128 of four workgroups per CU; mask_tile reads them itself there)
      constexpr bool kDensePre = MK == MI_ATTN_MASK_DENSE && D == 128;
      float4 dmask[kDensePre ? NKB * 4 : 1];
      if constexpr (kDensePre) load_dense_tile<NKB>(dmask, md, Lk, j0, hf, dense_vec);

      // S^T = K Q^T. The first 32-key block's K fragments are read before its first MFMA;
      // afterwards each MFMA overlaps the read of one fragment of the next block. (A lambda,
      // as are the mask below: the rare tile that moves the running max computes its logits
      // a second time, K still being in LDS, rather than keeping them live.)
      f32x16_t sacc[NKB];
      auto qk = [&]() {
        constexpr int NDC = D / 16;
        u32x4_t kf[NKB][NDC];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int dc = 0; dc < NDC; ++dc)
            kf[kb][dc] = *reinterpret_cast<const u32x4_t*>(smem + kb * 32 * TL::rowBytes + k_addr(dc, ks_ofs));
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          f32x16_t acc = f32x16_t{};
#pragma unroll
          for (int dc = 0; dc < NDC; ++dc) acc = mfma32(T{}, kf[kb][dc], qreg[dc], acc);
          sacc[kb] = acc;
        }
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, NDC, 0);
#pragma unroll
        for (int i = 0; i < (NKB - 1) * NDC; ++i) {
          __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
          __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, NDC, 0);
      };
      qk();

      // mask (tiles the mask does not cover entirely); masked tiles move to the log2
      // domain here (cm = 1), unmasked ones are scaled inside the exponent (cm = cexp)
      float cm = cexp;
      auto apply_mask = [&]() {
      if constexpr (GATHER) {
        const int32_t* xr = reinterpret_cast<const int32_t*>(vs + TL::vBytes);
        const float* xzl = reinterpret_cast<const float*>(xr + BN);
        const int32_t* xi = xr + 2 * BN;
        // the list ascends: its last key decides whether positions matter (causal selection)
        if (p.topk_causal && xi[BN - 1] > P0)
          mask_tile_topk_list<NKB, true, EXT>(sacc, hf, pos, tau_row, md, xr, xzl, xi);
        else
          mask_tile_topk_list<NKB, false, EXT>(sacc, hf, pos, tau_row, md, xr, xzl, xi);
        cm = 1.f;
      } else if constexpr (MK == MI_ATTN_MASK_TOPK) {
        const int32_t* xr = reinterpret_cast<const int32_t*>(vs + TL::vBytes);
        const float* xzl = reinterpret_cast<const float*>(xr + BN);
        if (p.topk_causal && j0 + BN - 1 > P0)
          mask_tile_topk<NKB, true, EXT>(sacc, j0, hf, pos, tau_row, md, xr, xzl);
        else
          mask_tile_topk<NKB, false, EXT>(sacc, j0, hf, pos, tau_row, md, xr, xzl);
        cm = 1.f;
      } else if (tile_needs_mask<MK, BN>(p, Lk, j0, P0, P1)) {
        mask_tile<MK, NKB, EXT>(sacc, p, Lk, j0, hf, pos, tau_row, md, nullptr, nullptr,
                                kDensePre ? dmask : nullptr);
        cm = 1.f;
      } else if constexpr (EXT) {
        mods_tile<NKB>(sacc, j0, hf, md);  // a tile every row sees: the score modifiers alone
        cm = 1.f;
      }
      };
      apply_mask();

      // one-tile dump (a debug call): the scaled, masked logits in natural-log units
      const bool dump_here = DUMP && bg == p.dump_bg && qb == p.dump_qb && t == p.dump_tile;
      if (dump_here && row_ok) {
        float* ds = p.dump + static_cast<long>(rloc) * BN;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int e = 0; e < 16; ++e) ds[kb * 32 + (e / 4) * 8 + hf * 4 + e % 4] = sacc[kb][e] * cm * kLn2;
      }

      u32x4_t preg[BN / 16];
      if constexpr (kRunningMaxExps<D, BN, MK, EXT>) {
        // Online softmax (log2 domain) against the running max m_run as it stands, with no
        // per-tile max reduction. That is exact online softmax as long as no exponential
        // exceeds 2^kRescaleThreshold, which holds whenever this lane's sum of them does
        // (the sum also fails for inf / NaN, i.e. a row with no visible key so far). Only
        // when some lane's sum fails does the wave compute the tile's logits again, reduce
        // their row maxima, move m to the exact running max, rescale l and O and take the
        // exponentials again; a dump takes that exact path too.
        auto exps = [&](float m_ref) -> float {  // P packed for the PV operand; the lane's sum
          float ps4[4] = {-0.f, -0.f, -0.f, -0.f};  // four independent chains (-0 + x is x: no add)
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
            for (int half = 0; half < 2; ++half) {
              float pv[8];
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                pv[e] = fast_exp2(fmaf(sacc[kb][half * 8 + e], cm, -m_ref));
                ps4[e & 3] += pv[e];
              }
              u32x4_t pk;
              pk.x = pack2(T{}, pv[0], pv[1]);
              pk.y = pack2(T{}, pv[2], pv[3]);
              pk.z = pack2(T{}, pv[4], pv[5]);
              pk.w = pack2(T{}, pv[6], pv[7]);
              preg[kb * 2 + half] = pk;
            }
          }
          return (ps4[0] + ps4[1]) + (ps4[2] + ps4[3]);
        };
        float m_ref = m_run;
        // a row with no running max yet (its first live tile) fails the check for sure: with
        // 128-key tiles go straight to the exact path, with the logits still in the
        // registers (d = 64: 1.2% faster; at d = 128 the registers that keeps live cost more)
        const bool fresh = decltype(first_c)::value || (BN == 128 && !__all(m_run != kNegInf));
        float lsum = fresh ? 0.f : exps(m_ref);
        if (fresh || !__all(lsum <= kFastSumLimit) || dump_here) {
          if (!fresh) {
            // a compiler-only memory barrier: K is read from LDS again, not kept in registers
            asm volatile("" ::: "memory");
            qk();
            cm = cexp;
            apply_mask();
          }
          float mx4[4] = {kNegInf, kNegInf, kNegInf, kNegInf};  // four independent chains
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int e = 0; e < 16; ++e) mx4[e & 3] = fmaxf(mx4[e & 3], sacc[kb][e]);
          const float mx = max_halves(fmaxf(fmaxf(mx4[0], mx4[1]), fmaxf(mx4[2], mx4[3]))) * cm;
          const float m_next = fmaxf(m_run, mx);
          m_ref = (m_next == kNegInf) ? 0.f : m_next;
          const float alpha = fast_exp2(m_run - m_ref);  // 0 from -inf
          if (dump_here) {
            // P (fp32, before rounding to 16 bits) against the reference max m
            float* dp = p.dump + kDumpRows * BN + static_cast<long>(rloc) * BN;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
              for (int e = 0; e < 16; ++e)
                if (row_ok) dp[kb * 32 + (e / 4) * 8 + hf * 4 + e % 4] = fast_exp2(fmaf(sacc[kb][e], cm, -m_ref));
          }
          lsum = exps(m_ref);
          l_run *= alpha;
          if (!__all(alpha == 1.f)) {
#pragma unroll
            for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
          }
          m_run = m_next;
        }
        l_run += lsum;
        if (dump_here) {
          // that max and the running sum after this tile, in natural-log units
          const float l_all = sum_halves(l_run);  // every lane: a cross-lane exchange
          if (hf == 0 && row_ok) {
            p.dump[2 * kDumpRows * BN + rloc] = m_ref * kLn2;
            p.dump[2 * kDumpRows * BN + kDumpRows + rloc] = l_all;
          }
        }
      } else {
        // online softmax (log2 domain), guarded against all -inf tiles and rows
        float mx4[4] = {kNegInf, kNegInf, kNegInf, kNegInf};  // four independent chains
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int e = 0; e < 16; ++e) mx4[e & 3] = fmaxf(mx4[e & 3], sacc[kb][e]);
        float mx = fmaxf(fmaxf(mx4[0], mx4[1]), fmaxf(mx4[2], mx4[3]));
        mx = max_halves(mx) * cm;
        const float m_next = (mx > m_run + kRescaleThreshold) ? mx : m_run;
        const float m_use = (m_next == kNegInf) ? 0.f : m_next;
        const float alpha = fast_exp2(m_run - m_use);  // 1 when the max did not move, 0 from -inf
        float ps4[4] = {-0.f, -0.f, -0.f, -0.f};  // four independent chains (-0 + x is x: no add)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            float pv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              pv[e] = fast_exp2(fmaf(sacc[kb][half * 8 + e], cm, -m_use));
              ps4[e & 3] += pv[e];
            }
            u32x4_t pk;
            pk.x = pack2(T{}, pv[0], pv[1]);
            pk.y = pack2(T{}, pv[2], pv[3]);
            pk.z = pack2(T{}, pv[4], pv[5]);
            pk.w = pack2(T{}, pv[6], pv[7]);
            preg[kb * 2 + half] = pk;
          }
        }
        l_run = fmaf(l_run, alpha, (ps4[0] + ps4[1]) + (ps4[2] + ps4[3]));
        m_run = m_next;
        if (dump_here) {
          // P (fp32, before rounding to 16 bits) against the reference max m, that max and
          // the running sum after this tile, both in natural-log units (rows of the block only)
          const float l_all = sum_halves(l_run);  // every lane: a cross-lane exchange
          float* dp = p.dump + kDumpRows * BN + static_cast<long>(rloc) * BN;
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int e = 0; e < 16; ++e)
              if (row_ok) dp[kb * 32 + (e / 4) * 8 + hf * 4 + e % 4] = fast_exp2(fmaf(sacc[kb][e], cm, -m_use));
          if (hf == 0 && row_ok) {
            p.dump[2 * kDumpRows * BN + rloc] = m_use * kLn2;
            p.dump[2 * kDumpRows * BN + kDumpRows + rloc] = l_all;
          }
        }
        if (!__all(alpha == 1.f)) {
#pragma unroll
          for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
        }
      }

      // O^T += V^T P^T. The V^T operand comes from two transposed reads: lane (16 * g + i)
      // reads 8 bytes of key row R0 + i / 4 at dims D0 + 4 * (i % 4) and receives keys
      // R0..R0+3 of dim D0 + i. Keys 4*hf+0..3 and 8+4*hf+0..3 of the 16-key chunk are what
      // its P registers hold. Key chunks run outermost, so the NDB accumulators are
      // independent chains, and the next chunk's V fragments are read during this chunk's
      // MFMAs.
      // The PV MFMAs issue at raised wavefront priority: when the other wavefront on the SIMD
      // has vector work ready at the same time, the matrix core is kept fed first (measured
      // +4% on c3 prefill; raising it for the QK MFMAs as well gains nothing).
      __builtin_amdgcn_s_setprio(1);
      {
        constexpr int NKC = BN / 16;

        u32x4_t vf[NKC][NDB];
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const unsigned char* row = smem + kc * 16 * TL::rowBytes;
            const u32x2_t lo = lds_read_tr16(row + v_addr(v_base0, db, vs_ofs));
            const u32x2_t hi2 = lds_read_tr16(row + v_addr(v_base1, db, vs_ofs));
            vf[kc][db] = u32x4_t{lo.x, lo.y, hi2.x, hi2.y};
          }
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
          for (int db = 0; db < NDB; ++db) oacc[db] = mfma32(T{}, vf[kc][db], preg[kc], oacc[db]);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * NDB, 0);
#pragma unroll
        for (int i = 0; i < (NKC - 1) * NDB; ++i) {
          __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
          __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, NDB, 0);
      }
      __builtin_amdgcn_s_setprio(0);

      if (tn < t_hi) finish_tile(stage ^ 1);
      __syncthreads();
      t = tn;
    };
    if constexpr (kUnroll2) {
      using F = std::false_type;
      if (t < t_hi) tile_step(std::integral_constant<int, 0>{}, std::true_type{});
      while (t < t_hi) {
        tile_step(std::integral_constant<int, 1>{}, F{});
        if (t >= t_hi) break;
        tile_step(std::integral_constant<int, 0>{}, F{});
      }
    } else if constexpr (kRunningMaxExps<D, BN, MK, EXT>) {
      int stage = 0;
      if (t < t_hi) {
        tile_step(0, std::true_type{});
        stage = 1;
      }
      for (; t < t_hi; stage ^= 1) tile_step(stage, std::false_type{});
    } else {
      for (int stage = 0; t < t_hi; stage ^= 1) tile_step(stage, std::false_type{});
    }

    // ---- epilogue: combine the two lane halves' partial sums, normalise, store
    const float l_tot = sum_halves(l_run);
    if (!row_ok) return;
    const bool dead = !(l_tot > 0.f);
    const float inv = dead ? 0.f : 1.f / l_tot;
    const float lse = dead ? kNegInf : (m_run + fast_log2(l_tot)) * kLn2;
    if (VARLEN ? item_partial : p.splits > 1) {
      // partial slot: split-major rows, or the item's own [Hkv, kBlockM] rows
      const long slot = VARLEN ? (static_cast<long>(item) * p.Hkv + g) * kBlockM + rloc
                               : static_cast<long>(split) * rows_all + row_index;
      float* po = p.part_out + slot * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int d0 = db * 32 + r4 * 8 + hf * 4;
          float4 v = {oacc[db][r4 * 4] * inv, oacc[db][r4 * 4 + 1] * inv, oacc[db][r4 * 4 + 2] * inv,
                      oacc[db][r4 * 4 + 3] * inv};
          *reinterpret_cast<float4*>(po + d0) = v;
        }
      if (hf == 0) p.part_lse[slot] = lse;
      return;
    }
    T* O = static_cast<T*>(p.out) + o_off;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = db * 32 + r4 * 8 + hf * 4;
        u32x2_t w;
        w.x = pack2(T{}, oacc[db][r4 * 4] * inv, oacc[db][r4 * 4 + 1] * inv);
        w.y = pack2(T{}, oacc[db][r4 * 4 + 2] * inv, oacc[db][r4 * 4 + 3] * inv);
        *reinterpret_cast<u32x2_t*>(O + d0) = w;
      }
    if (hf == 0 && p.lse != nullptr) p.lse[row_index] = lse;
  };

  // Resident workgroups (key-position masks, n_blocks > gridDim.x): the grid holds only
  // what the device runs at once, S workgroups per XCD, and workgroup w takes the query
  // blocks w % 8 + 8 i that the hardware would have placed on its XCD (whose K/V share
  // that XCD's L2), i running over that XCD's list in rounds of S: w / 8 in even rounds,
  // S - 1 - w / 8 in odd ones. The list is heavy-first per (batch, KV head), so the zigzag
  // pairs heavy blocks with light ones and every workgroup gets about the same work; and
  // a workgroup goes straight on to its next block instead of being relaunched by the
  // dispatcher, which feeds the shader engines of an XCD in a fixed rotation and leaves
  // slots idle behind a busy one.
  const unsigned nb = kResident<MK, VARLEN> ? p.n_blocks : gridDim.x;
  const bool resident = kResident<MK, VARLEN> && nb > gridDim.x;
  const unsigned xq = blockIdx.x % 8u, slots = gridDim.x / 8u, slot = blockIdx.x / 8u;
  for (unsigned r = 0;; ++r) {
    unsigned bid = blockIdx.x;
    if (resident) {
      if (xq + 8u * r * slots >= nb) break;  // no block of this XCD in round r
      bid = xq + 8u * (r * slots + ((r & 1u) ? slots - 1u - slot : slot));
      if (bid >= nb) continue;  // the last round is partial
      if (r > 0) __syncthreads();  // every wave is done with the previous block's LDS
    } else if (r > 0) {
      break;
    }
    run_block(VARLEN ? 0u : logical_block(bid, nb));
  }
}

// Split-KV combine: one thread per (row, 4 dims). lse = log sum_s exp(lse_s) (all -inf
// gives -inf and output 0); out = sum_s exp(lse_s - lse) o_s.
template <typename T>
__global__ __launch_bounds__(256) void lse_merge_kernel(AttnParams p) {
  const int D = p.d;
  const long rows_all = static_cast<long>(p.B) * p.Hq * p.Lq;
  const long t = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int per_row = D / 4;
  if (t >= rows_all * per_row) return;
  const long row = t / per_row;
  const int d0 = static_cast<int>(t % per_row) * 4;
  constexpr int kBatch = 8;  // splits whose partials are loaded together (their latencies overlap)
  float mx = kNegInf;
  for (int s0 = 0; s0 < p.splits; s0 += kBatch) {
    float ls[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) ls[k] = s0 + k < p.splits ? p.part_lse[(s0 + k) * rows_all + row] : kNegInf;
#pragma unroll
    for (int k = 0; k < kBatch; ++k) mx = fmaxf(mx, ls[k]);
  }
  float4 acc = {0.f, 0.f, 0.f, 0.f};
  float tot = 0.f;
  if (mx != kNegInf) {
    for (int s0 = 0; s0 < p.splits; s0 += kBatch) {
      float ls[kBatch];
      float4 os[kBatch];
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        ls[k] = kNegInf;
        os[k] = float4{0.f, 0.f, 0.f, 0.f};
        if (s0 + k < p.splits) {
          const long slot = (s0 + k) * rows_all + row;
          ls[k] = p.part_lse[slot];
          os[k] = *reinterpret_cast<const float4*>(p.part_out + slot * D + d0);
        }
      }
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        const float w = __expf(ls[k] - mx);  // 0 for the splits past the last
        acc.x += w * os[k].x; acc.y += w * os[k].y; acc.z += w * os[k].z; acc.w += w * os[k].w;
        tot += w;
      }
    }
  }
  const bool dead = !(tot > 0.f);
  const float inv = dead ? 0.f : 1.f / tot;
  const long i = row % p.Lq, h = (row / p.Lq) % p.Hq, bb = row / (static_cast<long>(p.Lq) * p.Hq);
  T* O = static_cast<T*>(p.out) + bb * p.os[0] + h * p.os[1] + i * p.os[2] + d0;
  O[0] = from_f32<T>(acc.x * inv);
  O[1] = from_f32<T>(acc.y * inv);
  O[2] = from_f32<T>(acc.z * inv);
  O[3] = from_f32<T>(acc.w * inv);
  if (d0 == 0 && p.lse != nullptr) p.lse[row] = dead ? kNegInf : mx + logf(tot);
}

template <typename T>
hipError_t launch_lse_merge_t(const AttnParams& p, hipStream_t s) {
  const long n = static_cast<long>(p.B) * p.Hq * p.Lq * (p.d / 4);
  hipLaunchKernelGGL(lse_merge_kernel<T>, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s, p);
  return hipGetLastError();
}

// Workgroups of one prefill kernel instance that the stream's device holds at once.
template <void (*K)(AttnParams)>
unsigned resident_workgroups(hipStream_t s) {
  static const int per_cu = [] {
    int n = 0;
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, K, kThreads, 0) == hipSuccess ? n : 0;
  }();
  int dev = 0, cus = 0;
  if ((s == nullptr ? hipGetDevice(&dev) : hipStreamGetDevice(s, &dev)) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return static_cast<unsigned>(per_cu > 0 && cus > 0 ? per_cu * cus : 0);
}

// Launches one instance: an unsplit grid of more query blocks than the device holds at
// once runs as that many resident workgroups (a multiple of 8, the same number per XCD),
// each taking several blocks; otherwise one workgroup per block.
template <void (*K)(AttnParams), bool RESIDENT>
void launch_prefill_instance(dim3 grid, const AttnParams& p, hipStream_t s) {
  AttnParams a = p;
  a.n_blocks = grid.x;
  if (RESIDENT && grid.y == 1) {
    const unsigned resident = resident_workgroups<K>(s) / 8u * 8u;
    if (resident >= 8u && grid.x > resident) grid.x = resident;
  }
  hipLaunchKernelGGL(K, grid, dim3(kThreads), 0, s, a);
}

template <typename T, int D, bool EXT>
void launch_prefill_d(dim3 grid, const AttnParams& p, hipStream_t s) {
  switch (p.mask_kind) {
    case MI_ATTN_MASK_NONE: launch_prefill_instance<prefill_kernel<T, D, kPosBN<D>, 0, false, false, EXT>, true>(grid, p, s); break;
    case MI_ATTN_MASK_CAUSAL: launch_prefill_instance<prefill_kernel<T, D, kPosBN<D>, 1, false, false, EXT>, true>(grid, p, s); break;
    case MI_ATTN_MASK_WINDOW: launch_prefill_instance<prefill_kernel<T, D, kPosBN<D>, 2, false, false, EXT>, true>(grid, p, s); break;
    case MI_ATTN_MASK_DENSE: launch_prefill_instance<prefill_kernel<T, D, 64, 3, false, false, EXT>, false>(grid, p, s); break;
    default:
      if (p.list_idx != nullptr)
        launch_prefill_instance<prefill_kernel<T, D, 64, 4, true, false, EXT>, false>(grid, p, s);
      else
        launch_prefill_instance<prefill_kernel<T, D, 64, 4, false, false, EXT>, false>(grid, p, s);
      break;
  }
}

// The dump instances (64-key tiles, no score modifiers), one workgroup per block.
template <typename T, int D>
hipError_t launch_prefill_dump(dim3 grid, const AttnParams& p, hipStream_t s) {
  AttnParams a = p;
  a.n_blocks = grid.x;
  const dim3 block(kThreads);
  switch (p.mask_kind) {
    case MI_ATTN_MASK_NONE:
    case MI_ATTN_MASK_CAUSAL:
    case MI_ATTN_MASK_WINDOW:
      if constexpr (kPosBN<D> == 64) {
        if (p.mask_kind == MI_ATTN_MASK_NONE)
          hipLaunchKernelGGL((prefill_kernel<T, D, 64, 0, false, false, false, true>), grid, block, 0, s, a);
        else if (p.mask_kind == MI_ATTN_MASK_CAUSAL)
          hipLaunchKernelGGL((prefill_kernel<T, D, 64, 1, false, false, false, true>), grid, block, 0, s, a);
        else
          hipLaunchKernelGGL((prefill_kernel<T, D, 64, 2, false, false, false, true>), grid, block, 0, s, a);
        break;
      } else {
        return hipErrorInvalidValue;  // these kinds take 128-key tiles at this head dim
      }
    case MI_ATTN_MASK_DENSE: hipLaunchKernelGGL((prefill_kernel<T, D, 64, 3, false, false, false, true>), grid, block, 0, s, a); break;
    default:
      if (p.list_idx != nullptr)
        hipLaunchKernelGGL((prefill_kernel<T, D, 64, 4, true, false, false, true>), grid, block, 0, s, a);
      else
        hipLaunchKernelGGL((prefill_kernel<T, D, 64, 4, false, false, false, true>), grid, block, 0, s, a);
      break;
  }
  return hipSuccess;
}

template <typename T>
hipError_t launch_prefill_t(const AttnParams& p, hipStream_t s) {
  const int nqb = (p.Lq + p.q_per_block - 1) / p.q_per_block;
  const long blocks = static_cast<long>(p.B) * p.Hkv * nqb;
  if (blocks > 0x7fffffffL || p.splits > 65535) return hipErrorInvalidValue;
  dim3 grid(static_cast<unsigned>(blocks), p.splits);
  const bool ext = needs_ext(p);
  if (p.dump != nullptr) {
    if (ext) return hipErrorInvalidValue;
    const hipError_t e = p.d == 128 ? launch_prefill_dump<T, 128>(grid, p, s) : launch_prefill_dump<T, 64>(grid, p, s);
    if (e != hipSuccess) return e;
  } else if (p.d == 128) {
    if (ext) launch_prefill_d<T, 128, true>(grid, p, s);
    else launch_prefill_d<T, 128, false>(grid, p, s);
  } else {
    if (ext) launch_prefill_d<T, 64, true>(grid, p, s);
    else launch_prefill_d<T, 64, false>(grid, p, s);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits <= 1) return e;
  return launch_lse_merge_t<T>(p, s);
}

// Varlen items of prefill type (query runs longer than 32 rows per KV head); the LSE
// merge of split units runs separately.
template <typename T, bool EXT>
hipError_t launch_prefill_varlen_t(const AttnParams& p, hipStream_t s) {
  const long blocks = (static_cast<long>(p.vl_items_cap) * p.Hkv + 7) / 8 * 8;  // whole rounds of 8 XCDs
  if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
  dim3 grid(static_cast<unsigned>(blocks)), block(kThreads);
  if (p.d == 128) {
    switch (p.mask_kind) {
      case MI_ATTN_MASK_NONE:
        hipLaunchKernelGGL((prefill_kernel<T, 128, 64, 0, false, true, EXT>), grid, block, 0, s, p);
        break;
      case MI_ATTN_MASK_CAUSAL:
        hipLaunchKernelGGL((prefill_kernel<T, 128, 64, 1, false, true, EXT>), grid, block, 0, s, p);
        break;
      default: hipLaunchKernelGGL((prefill_kernel<T, 128, 64, 2, false, true, EXT>), grid, block, 0, s, p); break;
    }
  } else {
    switch (p.mask_kind) {
      case MI_ATTN_MASK_NONE:
        hipLaunchKernelGGL((prefill_kernel<T, 64, 64, 0, false, true, EXT>), grid, block, 0, s, p);
        break;
      case MI_ATTN_MASK_CAUSAL:
        hipLaunchKernelGGL((prefill_kernel<T, 64, 64, 1, false, true, EXT>), grid, block, 0, s, p);
        break;
      default: hipLaunchKernelGGL((prefill_kernel<T, 64, 64, 2, false, true, EXT>), grid, block, 0, s, p); break;
    }
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_varlen(const AttnParams& p, int dtype, hipStream_t s) {
  // score modifiers (ALiBi, softcap) run the EXT instances
  const bool ext = has_mods(p);
  if (dtype == MI_ATTN_BF16) return ext ? launch_prefill_varlen_t<bf16_t, true>(p, s) : launch_prefill_varlen_t<bf16_t, false>(p, s);
  if (dtype == MI_ATTN_F16) return ext ? launch_prefill_varlen_t<f16_t, true>(p, s) : launch_prefill_varlen_t<f16_t, false>(p, s);
  return hipErrorInvalidValue;
}

int prefill_block_n(int d, int mask_kind) {
  return mask_kind <= MI_ATTN_MASK_WINDOW ? (d == 64 ? kPosBN<64> : kPosBN<128>) : 64;
}
int prefill_block_m() { return kBlockM; }

hipError_t launch_lse_merge(const AttnParams& p, int dtype, hipStream_t s) {
  if (dtype == MI_ATTN_BF16) return launch_lse_merge_t<bf16_t>(p, s);
  if (dtype == MI_ATTN_F16) return launch_lse_merge_t<f16_t>(p, s);
  return hipErrorInvalidValue;
}

hipError_t launch_prefill(const AttnParams& p, int dtype, hipStream_t s) {
  if (dtype == MI_ATTN_BF16) return launch_prefill_t<bf16_t>(p, s);
  if (dtype == MI_ATTN_F16) return launch_prefill_t<f16_t>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace mi_attn
