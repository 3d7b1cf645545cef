// Backward of the masked attention forward: dq, dk, dv from the saved LSE.
//
// The InfiniTrain pull request #193 page integrates forward and backward kernels for the
// same attention ("main changes": fwd/bwd for FP16 and BF16, head dims 64 and 128; the
// autograd function saves what the backward needs). With P recomputed from q, k and the
// saved LSE, the chain rule of the forward gives, per (row i, key j):
//   dv_j += P_ij dO_i                   dP_ij = dO_i . v_j
//   dS_ij = P_ij (dP_ij - D_i),         D_i  = rowsum(dO_i * O_i)
//   dq_i += scale dS_ij k_j             dk_j += scale dS_ij q_i
// (the softmax Jacobian; a fully masked row has P = 0 and contributes nothing).
//
// Two kernels, no atomics:
//   dq_kernel    the forward's structure: one workgroup per (batch, KV head, 128 rows of
//                the G heads, query-major), 64-key K/V tiles in LDS:
//                S^T = K Q^T, dP^T = V dO^T, dQ^T += K^T dS^T. It computes D itself from
//                the rows it holds and writes the per-row side arrays (-LSE in log2 units,
//                D, and the top-k threshold or query index) in the row order below.
//   dkdv_kernel  one workgroup per (batch, KV head, 128 keys); each wavefront owns 32 keys
//                (K and V as B operands in registers) and loops over 32-row tiles of the
//                query rows of all G heads that read the KV head (query-major), staged in
//                LDS by direct loads three tiles deep: S = Q K^T, dP = dO V^T, then
//                dV^T += dO^T P and dK^T += Q^T dS with dO^T / Q^T from transposed LDS
//                reads and P / dS straight from the registers (the C layout of S is the B
//                layout these products need).
#include <type_traits>

#include "common.hpp"
#include "mfma_common.hpp"

namespace mi_attn {

namespace {

using namespace mfma;

constexpr int kBW = 4;             // wavefronts per workgroup
constexpr int kBT = kBW * kWave;

// A tile of `ROWS` rows of D 16-bit values in LDS: [row][d], unpadded, 16-byte slots
// swizzled by swz<D> (the forward's layout, conflict-free for both operand reads).
template <int D, int ROWS>
struct BTile {
  static constexpr int rowBytes = D * 2;
  static constexpr int bytes = ROWS * rowBytes;
  static constexpr int rowsPerWaveLoad = 1024 / rowBytes;  // rows one wave's direct load fills
  static constexpr int rounds = bytes / (kBT * 16);        // direct loads per wave
  static_assert(rounds * kBT * 16 == bytes, "tile split evenly over the direct loads");
};

// LDS operand addresses shared by both kernels (see the forward kernel): a row fragment
// (A operand: lane = row l32, 8 values dc*16 + hf*8) at blk * 32 * rowBytes +
// (row_base ^ (dc << 5)); a transposed fragment (A operand: lane = column D0 + l32, the 8
// rows whose values its P / dS registers hold) from two 64-bit transposed reads at
// chunk * 16 * rowBytes + (tr_base[0|1] ^ (db << 6)).
template <int D>
struct Bases {
  int row_base, tr0, tr1;
  __device__ Bases(int lane) {
    const int l32 = lane & 31, hf = lane >> 5;
    constexpr int rb = D * 2;
    row_base = l32 * rb | ((hf ^ swz<D>(l32)) << 4);
    const int tr_row = 4 * hf + (lane & 15) / 4;
    const int sl = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    tr0 = tr_row * rb | ((sl ^ swz<D>(tr_row)) << 4) | (8 * (lane & 1));
    tr1 = (tr_row + 8) * rb | ((sl ^ swz<D>(tr_row + 8)) << 4) | (8 * (lane & 1));
  }
};

__device__ __forceinline__ u32x4_t row_frag(const unsigned char* tile, int row_base, int blk, int dc, int rowBytes) {
  return *reinterpret_cast<const u32x4_t*>(tile + blk * 32 * rowBytes + (row_base ^ (dc << 5)));
}
__device__ __forceinline__ u32x4_t tr_frag(const unsigned char* tile, int tr0, int tr1, int chunk, int db,
                                           int rowBytes) {
  const unsigned char* r = tile + chunk * 16 * rowBytes;
  const u32x2_t lo = lds_read_tr16(r + (tr0 ^ (db << 6)));
  const u32x2_t hi = lds_read_tr16(r + (tr1 ^ (db << 6)));
  return u32x4_t{lo.x, lo.y, hi.x, hi.y};
}

// P (or dS) registers of one 32-column C tile packed to 16 bit: chunk c holds rows
// 16 c + {4 hf .. 4 hf + 3, 8 + 4 hf .. 8 + 4 hf + 3}, the rows the transposed reads pair
// them with.
template <typename T>
__device__ __forceinline__ u32x4_t pack_half(const f32x16_t& x, int half) {
  return u32x4_t{pack2(T{}, x[half * 8 + 0], x[half * 8 + 1]), pack2(T{}, x[half * 8 + 2], x[half * 8 + 3]),
                 pack2(T{}, x[half * 8 + 4], x[half * 8 + 5]), pack2(T{}, x[half * 8 + 6], x[half * 8 + 7])};
}

// 16 fp32 values of a 32x32 C tile column as 4 groups of 4 consecutive rows, scaled and
// rounded into a T row at `dst` (dims db * 32 + 8 * r4 + 4 * hf .. + 3).
template <typename T>
__device__ __forceinline__ void store_col(T* dst, const f32x16_t& x, int db, int hf, float mul) {
#pragma unroll
  for (int r4 = 0; r4 < 4; ++r4) {
    const int d0 = db * 32 + r4 * 8 + hf * 4;
    *reinterpret_cast<u32x2_t*>(dst + d0) = u32x2_t{pack2(T{}, x[r4 * 4] * mul, x[r4 * 4 + 1] * mul),
                                                    pack2(T{}, x[r4 * 4 + 2] * mul, x[r4 * 4 + 3] * mul)};
  }
}

// s_waitcnt: at most n vector-memory operations outstanding and no LDS operation
constexpr int vm_lgkm0_imm(int n) { return (n & 0xf) | ((n >> 4) << 14) | (0x7 << 4); }

// ------------------------------------------------------------------ dQ (+ row side arrays)
template <typename T, int D, int MK>
__global__ __launch_bounds__(kBT, 2) void dq_kernel(AttnParams p) {
  constexpr int BN = 64;
  using KT = BTile<D, BN>;
  constexpr int NDC = D / 16;
  constexpr int NDB = D / 32;
  constexpr int kStage = 2 * KT::bytes;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * kStage];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int l32 = lane & 31;
  const int hf = lane >> 5;
  const int Lq = p.Lq, Lk = p.Lk, G = p.G;

  const int nqb = (Lq + p.q_per_block - 1) / p.q_per_block;
  const unsigned lb = logical_block(blockIdx.x, gridDim.x);
  const int qb = nqb - 1 - static_cast<int>(lb % nqb);
  const int bg = static_cast<int>(lb / nqb);
  const int b = bg / p.Hkv, g = bg % p.Hkv;
  const int i_first = qb * p.q_per_block;
  const int i_last = min(Lq, i_first + p.q_per_block) - 1;
  const int rows_blk = (i_last - i_first + 1) * G;
  const int P0 = Lk - Lq + i_first, P1 = Lk - Lq + i_last;

  // this lane's row (the S^T column it owns), query-major over the G heads
  const int rloc = wave * 32 + l32;
  const bool row_ok = rloc < rows_blk;
  const int i_row = i_first + (row_ok ? rloc / G : 0);
  const int h_row = g * G + (row_ok ? rloc % G : 0);
  const int pos = Lk - Lq + i_row;
  const long row_index = (static_cast<long>(b) * p.Hq + h_row) * Lq + i_row;

  u32x4_t qreg[NDC], oreg[NDC];  // Q^T and dO^T B operands of the lane's row
  float dpart = 0.f;             // this lane half's part of D = rowsum(dO * O)
#pragma unroll
  for (int dc = 0; dc < NDC; ++dc) {
    u32x4_t x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u}, z = {0u, 0u, 0u, 0u};
    if (row_ok) {
      const long e = row_index * D + dc * 16 + hf * 8;
      x = *reinterpret_cast<const u32x4_t*>(static_cast<const T*>(p.q) + e);
      y = *reinterpret_cast<const u32x4_t*>(static_cast<const T*>(p.dout) + e);
      z = *reinterpret_cast<const u32x4_t*>(static_cast<const T*>(p.out) + e);
    }
    qreg[dc] = x;
    oreg[dc] = y;
    const T* yt = reinterpret_cast<const T*>(&y);
    const T* zt = reinterpret_cast<const T*>(&z);
#pragma unroll
    for (int c = 0; c < 8; ++c) dpart = fmaf(to_f32(yt[c]), to_f32(zt[c]), dpart);
  }
  const float dsum = sum_halves(dpart);
  const float cexp = p.scale * kLog2e;  // signed: no sign folded into an operand here
  const float lse = row_ok ? p.lse[row_index] : kNegInf;
  const float lse2 = lse == kNegInf ? __builtin_inff() : lse * kLog2e;  // dead rows: P = 0
  const Mods md = make_mods<false>(p, cexp, b, h_row, i_row, pos, MK == MI_ATTN_MASK_DENSE);
  int32_t tau_row = 0;
  if constexpr (MK == MI_ATTN_MASK_TOPK) tau_row = min(p.tau[static_cast<long>(bg) * Lq + i_row], Lk - 1);
  const long bgk = static_cast<long>(bg) * Lk;

  // side arrays of the dK/dV kernel, at row r = i * G + hh of this KV head
  if (row_ok && hf == 0) {
    const long nr = static_cast<long>(p.B) * p.Hq * Lq;
    const long si = static_cast<long>(bg) * G * Lq + static_cast<long>(i_first) * G + rloc;
    p.bwd_side[si] = -lse2;
    p.bwd_side[nr + si] = dsum;
    if constexpr (MK == MI_ATTN_MASK_TOPK) reinterpret_cast<int32_t*>(p.bwd_side)[2 * nr + si] = tau_row;
    if constexpr (MK == MI_ATTN_MASK_DENSE) reinterpret_cast<int32_t*>(p.bwd_side)[2 * nr + si] = i_row;
  }

  int lo, hi;
  key_range(MK, p.window_left, Lk, P0, P1, &lo, &hi);
  if (p.no_skip) { lo = 0; hi = Lk; }
  const int t_lo = lo / BN;
  const int t_hi = hi > lo ? (hi + BN - 1) / BN : t_lo;

  const T* K = static_cast<const T*>(p.k) + bgk * D;
  const T* V = static_cast<const T*>(p.v) + bgk * D;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(K, Lk * D * 2);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(V, Lk * D * 2);
  const unsigned smem_addr = __builtin_amdgcn_readfirstlane(lds_address(smem));
  int dma_lane;
  {
    const int r = wave * KT::rowsPerWaveLoad + lane / (D / 8);
    dma_lane = (r * D + (((lane % (D / 8)) ^ swz<D>(r)) << 3)) * 2;
  }
  auto issue = [&](int t, int stg) {
#pragma unroll
    for (int c = 0; c < KT::rounds; ++c) {
      const int so = (t * BN + c * kBW * KT::rowsPerWaveLoad) * D * 2;
      const unsigned dst = smem_addr + stg * kStage + (c * kBW + wave) * 1024;
      lds_dma16_at(krs, dst, dma_lane, so);
      lds_dma16_at(vrs, dst + KT::bytes, dma_lane, so);
    }
  };

  const Bases<D> bs(lane);
  f32x16_t dqacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dqacc[db] = f32x16_t{};

  int t = t_lo, stg = 0;
  if (t < t_hi) {
    issue(t, 0);
    __builtin_amdgcn_s_waitcnt(0);
  }
  __syncthreads();
  while (t < t_hi) {
    if (t + 1 < t_hi) issue(t + 1, stg ^ 1);
    const unsigned char* kt = smem + stg * kStage;
    const unsigned char* vt = kt + KT::bytes;
    const int j0 = t * BN;

    // S^T = K Q^T and dP^T = V dO^T (64 keys x 32 rows; lane = row, registers = keys)
    f32x16_t s[2], dp[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16_t a = f32x16_t{}, c = f32x16_t{};
#pragma unroll
      for (int dc = 0; dc < NDC; ++dc) a = mfma32(T{}, row_frag(kt, bs.row_base, kb, dc, KT::rowBytes), qreg[dc], a);
#pragma unroll
      for (int dc = 0; dc < NDC; ++dc) c = mfma32(T{}, row_frag(vt, bs.row_base, kb, dc, KT::rowBytes), oreg[dc], c);
      s[kb] = a;
      dp[kb] = c;
    }
    // logits in log2 units (masked where the tile needs it), P, dS = P (dP - D)
    if (tile_needs_mask<MK, BN>(p, Lk, j0, P0, P1)) {
      mask_tile<MK, 2, false>(s, p, Lk, j0, hf, pos, tau_row, md,
                              MK == MI_ATTN_MASK_TOPK ? p.rank + bgk + j0 : nullptr,
                              MK == MI_ATTN_MASK_TOPK ? p.zero_hold + bgk + j0 : nullptr);
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) s[kb] *= cexp;
    }
    u32x4_t dsreg[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float pv = fast_exp2(s[kb][e] - lse2);
        dp[kb][e] = pv * (dp[kb][e] - dsum);
      }
      dsreg[kb * 2] = pack_half<T>(dp[kb], 0);
      dsreg[kb * 2 + 1] = pack_half<T>(dp[kb], 1);
    }
    // dQ^T += K^T dS^T (d x 32 rows; contraction over the 64 keys)
#pragma unroll
    for (int kc = 0; kc < 4; ++kc)
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        dqacc[db] = mfma32(T{}, tr_frag(kt, bs.tr0, bs.tr1, kc, db, KT::rowBytes), dsreg[kc], dqacc[db]);

    if (t + 1 < t_hi) __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    ++t;
    stg ^= 1;
  }

  if (!row_ok) return;
  T* dq = static_cast<T*>(p.dq) + row_index * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db) store_col<T>(dq, dqacc[db], db, hf, p.scale);
}

// ------------------------------------------------------------------ dK, dV
template <typename T, int D, int MK>
__global__ __launch_bounds__(kBT, 2) void dkdv_kernel(AttnParams p) {
  using QT = BTile<D, 32>;
  using KT = BTile<D, 128>;
  constexpr int NDC = D / 16;
  constexpr int NDB = D / 32;
  constexpr bool kAux = MK == MI_ATTN_MASK_DENSE || MK == MI_ATTN_MASK_TOPK;
  constexpr bool kCausal = MK == MI_ATTN_MASK_CAUSAL || MK == MI_ATTN_MASK_WINDOW || MK == MI_ATTN_MASK_TOPK;
  // d = 128: the block's K tile lives in LDS (read like Q each tile) instead of 64
  // registers, so two workgroups fit per CU (two wavefronts per SIMD); LDS then holds a
  // two-stage ring. d = 64 keeps K in registers and a three-stage ring.
  constexpr bool kKLds = D == 128;
  constexpr int kStages = kKLds ? 2 : 3;
  constexpr int kDist = kStages - 1;  // tiles loaded ahead
  // stage: Q tile, dO tile, then the side values of its 32 rows: -LSE2 [32], D [32],
  // threshold or query index [32], 128 bytes unused
  constexpr int kSide = 512;
  constexpr int kStage = 2 * QT::bytes + kSide;
  static_assert(kStage % 512 == 0, "stage offsets keep the XOR-ed address bits");
  constexpr int kKBytes = kKLds ? KT::bytes : 0;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kStages * kStage + kKBytes];
  unsigned char* const ktile = smem + kStages * kStage;  // d = 128: keys kblk * 128 + r

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int l32 = lane & 31;
  const int hf = lane >> 5;
  const int Lq = p.Lq, Lk = p.Lk, G = p.G;
  const int R = G * Lq;  // query rows of the KV head

  const int nkb = (Lk + 127) / 128;
  const unsigned lb = logical_block(blockIdx.x, gridDim.x);
  const int kblk = static_cast<int>(lb % nkb);
  const int bg = static_cast<int>(lb / nkb);
  const int b = bg / p.Hkv, g = bg % p.Hkv;
  const int j_lane = kblk * 128 + wave * 32 + l32;  // this lane's key (the column it owns)
  const bool key_ok = j_lane < Lk;
  const long kv_row = (static_cast<long>(bg) * Lk + (key_ok ? j_lane : 0)) * D;

  // K^T and V^T B operands of the lane's key (K from LDS at d = 128)
  u32x4_t kreg[kKLds ? 1 : NDC], vreg[NDC];
#pragma unroll
  for (int dc = 0; dc < NDC; ++dc) {
    u32x4_t x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u};
    if (key_ok) {
      if (!kKLds) x = *reinterpret_cast<const u32x4_t*>(static_cast<const T*>(p.k) + kv_row + dc * 16 + hf * 8);
      y = *reinterpret_cast<const u32x4_t*>(static_cast<const T*>(p.v) + kv_row + dc * 16 + hf * 8);
    }
    if (!kKLds) kreg[dc] = x;
    vreg[dc] = y;
  }
  int32_t rank_lane = 0x7fffffff;
  float zh_lane = 0.f;
  if constexpr (MK == MI_ATTN_MASK_TOPK) {
    if (key_ok) {
      rank_lane = p.rank[static_cast<long>(bg) * Lk + j_lane];
      zh_lane = p.zero_hold[static_cast<long>(bg) * Lk + j_lane] * kLog2e;
    }
  }

  // Rows that see the lane's key: r in [r_lo, r_hi). Row r = i * G + hh sits at position
  // Lk - Lq + i, so "i >= j - (Lk - Lq)" is "r >= (j - (Lk - Lq)) * G".
  const long off = static_cast<long>(Lk) - Lq;
  auto row_at = [&](long i) { return static_cast<int>(min(static_cast<long>(R), max(0L, i * G))); };
  int r_lo = key_ok ? 0 : R, r_hi = key_ok ? R : 0;
  if (kCausal && key_ok) r_lo = row_at(j_lane - off);
  if (MK == MI_ATTN_MASK_WINDOW && key_ok) r_hi = row_at(j_lane + static_cast<long>(p.window_left) - off + 1);
  // the same for the block's keys together (row tiles to visit) and for all of them
  // (tiles that need no per-element mask)
  const int k_first = kblk * 128, k_last = min(Lk, k_first + 128) - 1;
  int blk_lo = 0, blk_hi = R, all_lo = 0, all_hi = R;
  if (kCausal) {
    blk_lo = row_at(k_first - off);
    all_lo = row_at(k_last - off);
  }
  if (MK == MI_ATTN_MASK_WINDOW) {
    blk_hi = row_at(k_last + static_cast<long>(p.window_left) - off + 1);
    all_hi = row_at(k_first + static_cast<long>(p.window_left) - off + 1);
  }
  const bool full_block = k_first + 128 <= Lk;
  if (p.no_skip) { blk_lo = 0; blk_hi = R; }
  const int t_lo = blk_lo / 32;
  const int t_hi = blk_hi > blk_lo ? (blk_hi + 31) / 32 : t_lo;

  // direct loads: lane fills 16-byte slot ps of row rr of its load rounds; rows of the
  // batch are addressed through a buffer over all its query heads (past the end: zeros)
  const T* qb_ptr = static_cast<const T*>(p.q) + static_cast<long>(b) * p.Hq * Lq * D;
  const T* ob_ptr = static_cast<const T*>(p.dout) + static_cast<long>(b) * p.Hq * Lq * D;
  const int batch_bytes = p.Hq * Lq * D * 2;  // < 2^31 (checked on the host)
  const __amdgpu_buffer_rsrc_t qrs = make_rsrc(qb_ptr, batch_bytes);
  const __amdgpu_buffer_rsrc_t ors = make_rsrc(ob_ptr, batch_bytes);
  const long nr = static_cast<long>(p.B) * p.Hq * Lq;
  const __amdgpu_buffer_rsrc_t srs = make_rsrc(p.bwd_side, static_cast<int>(nr * (kAux ? 12 : 8)));
  const int side_base = static_cast<int>(static_cast<long>(bg) * R * 4);
  // wave 0: lanes 0-31 load -LSE2 and lanes 32-63 D of the tile's rows; wave 1 (lanes
  // 0-31): the thresholds or query indices
  const int side_lane = wave == 0 ? (hf ? static_cast<int>(nr * 4) : 0) + side_base + l32 * 4
                                  : static_cast<int>(nr * 8) + side_base + l32 * 4;
  const unsigned smem_addr = __builtin_amdgcn_readfirstlane(lds_address(smem));
  const int ps = lane % (D / 8);
  // The lane's row in load round c of the next tile to load, r = i * G + hh, kept as (i,
  // hh, byte offset of the row in the batch) and advanced by 32 rows per tile without a
  // division. Tiles are loaded in order from t_lo.
  int st_i[QT::rounds], st_h[QT::rounds];
  unsigned st_o[QT::rounds];
  int sw[QT::rounds];
#pragma unroll
  for (int c = 0; c < QT::rounds; ++c) {
    const int rr = (c * kBW + wave) * QT::rowsPerWaveLoad + lane / (D / 8);
    const int r = t_lo * 32 + rr;
    st_i[c] = r / G;
    st_h[c] = r - st_i[c] * G;
    st_o[c] = static_cast<unsigned>(((static_cast<long>(g) * G + st_h[c]) * Lq + st_i[c]) * D * 2);
    sw[c] = (ps ^ swz<D>(rr)) << 4;
  }
  const int adv_i = 32 / G, adv_h = 32 % G;
  const unsigned adv_o = static_cast<unsigned>((adv_i + static_cast<long>(adv_h) * Lq) * D * 2);
  const unsigned wrap_o = static_cast<unsigned>((1 - static_cast<long>(G) * Lq) * D * 2);
  auto issue = [&](int t, int stg) {
    const int r0 = t * 32;
    const unsigned sb = smem_addr + stg * kStage;
#pragma unroll
    for (int c = 0; c < QT::rounds; ++c) {
      // rows past the last one (i >= Lq) read zeros (the offset is past the buffer)
      const int o = st_i[c] < Lq ? static_cast<int>(st_o[c]) + sw[c] : batch_bytes;
      const unsigned dst = sb + (c * kBW + wave) * 1024;
      lds_dma16_at(qrs, dst, o, 0);
      lds_dma16_at(ors, dst + QT::bytes, o, 0);
      st_h[c] += adv_h;
      st_i[c] += adv_i;
      st_o[c] += adv_o;
      if (st_h[c] >= G) {
        st_h[c] -= G;
        st_i[c] += 1;
        st_o[c] += wrap_o;
      }
    }
    if (wave == 0) lds_dma4_at(srs, sb + 2 * QT::bytes, side_lane, r0 * 4);
    if (kAux && wave == 1 && lane < 32) lds_dma4_at(srs, sb + 2 * QT::bytes + 256, side_lane, r0 * 4);
  };
  // direct loads one tile issues in this wave; "the tile after next may still be in
  // flight" (three stages) or "nothing may" (two stages)
  const bool one_more = wave == 0 || (kAux && wave == 1);
  auto wait_next_tile = [&]() {
    if constexpr (kDist == 1) {
      __builtin_amdgcn_s_waitcnt(vm_lgkm0_imm(0));
    } else {
      if (one_more) __builtin_amdgcn_s_waitcnt(vm_lgkm0_imm(2 * QT::rounds + 1));
      else __builtin_amdgcn_s_waitcnt(vm_lgkm0_imm(2 * QT::rounds));
    }
  };

  const Bases<D> bs(lane);
  const float cexp = p.scale * kLog2e;  // signed: no sign folded into an operand here
  f32x16_t dkacc[NDB], dvacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    dkacc[db] = f32x16_t{};
    dvacc[db] = f32x16_t{};
  }

  // d = 128: the block's K tile (keys past Lk read as zeros), before the first ring tile
  if constexpr (kKLds) {
    const T* Kb = static_cast<const T*>(p.k) + static_cast<long>(bg) * Lk * D;
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(Kb, Lk * D * 2);  // < 2^31 (host check)
#pragma unroll
    for (int c = 0; c < KT::rounds; ++c) {
      const int rr = (c * kBW + wave) * KT::rowsPerWaveLoad + lane / (D / 8);
      const int o = (kblk * 128 + rr) * D * 2 + ((ps ^ swz<D>(rr)) << 4);
      lds_dma16_at(krs, smem_addr + kStages * kStage + (c * kBW + wave) * 1024, o, 0);
    }
  }

  // ring: tiles t + 1 .. t + kDist load while tile t is computed
  if (t_lo < t_hi) issue(t_lo, 0);
  if (kDist == 2 && t_lo + 1 < t_hi) {
    issue(t_lo + 1, 1);
    wait_next_tile();
  } else {
    __builtin_amdgcn_s_waitcnt(0);
  }
  __syncthreads();
  int stg = 0;
  for (int t = t_lo; t < t_hi; ++t) {
    if (t + kDist < t_hi) issue(t + kDist, stg + kDist < kStages ? stg + kDist : stg + kDist - kStages);
    const unsigned char* qt = smem + stg * kStage;
    const unsigned char* ot = qt + QT::bytes;
    const float* side_m = reinterpret_cast<const float*>(qt + 2 * QT::bytes);
    const float* side_d = side_m + 32;
    const int32_t* side_a = reinterpret_cast<const int32_t*>(side_m + 64);
    const int r0 = t * 32;

    // S = Q K^T and dP = dO V^T (32 rows x 32 keys; lane = key, registers = rows)
    f32x16_t s = f32x16_t{}, dp = f32x16_t{};
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) {
      const u32x4_t kf = kKLds ? row_frag(ktile, bs.row_base, wave, dc, QT::rowBytes) : kreg[kKLds ? 0 : dc];
      s = mfma32(T{}, row_frag(qt, bs.row_base, 0, dc, QT::rowBytes), kf, s);
      dp = mfma32(T{}, row_frag(ot, bs.row_base, 0, dc, QT::rowBytes), vreg[dc], dp);
    }
    // each MFMA overlaps the LDS read of the operand(s) two MFMAs ahead
    constexpr int kRd = kKLds ? 3 : 2;  // reads per S/dP MFMA pair
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, kRd, 0);
#pragma unroll
    for (int i = 0; i < NDC - 1; ++i) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, kRd, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2, 0);
    __builtin_amdgcn_sched_barrier(0);

    // P = exp2(logit - LSE2) where the pair is visible; dS = P (dP - D). Tiles whose rows
    // all see every key of the block skip the per-element mask (a uniform branch).
    const bool interior = !kAux && full_block && r0 >= all_lo && r0 + 32 <= all_hi && !p.no_skip;
    const int lo = r_lo - r0, hi = r_hi - r0;  // visible rows of the lane's key, tile-relative
    const bool uniform_interior = __builtin_amdgcn_readfirstlane(static_cast<int>(interior));
    // P and dS of the 4 consecutive rows rb .. rb + 3 held in registers r4 * 4 .. + 3, with
    // their side values read from LDS just before (short live ranges)
    auto rows4 = [&](int r4, auto masked_c) {
      constexpr bool MASKED = decltype(masked_c)::value;
      const int rb = r4 * 8 + hf * 4;  // first of the 4 consecutive rows of these registers
      const float4 ml = *reinterpret_cast<const float4*>(side_m + rb);
      const float4 dd = *reinterpret_cast<const float4*>(side_d + rb);
      const float mls[4] = {ml.x, ml.y, ml.z, ml.w};
      const float dds[4] = {dd.x, dd.y, dd.z, dd.w};
      int4 ax = {0, 0, 0, 0};
      if constexpr (kAux) ax = *reinterpret_cast<const int4*>(side_a + rb);
      const int axs[4] = {ax.x, ax.y, ax.z, ax.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float x = fmaf(s[r4 * 4 + e], cexp, mls[e]);
        if constexpr (!MASKED) {
          const float pv = fast_exp2(x);
          dp[r4 * 4 + e] = pv * (dp[r4 * 4 + e] - dds[e]);
          s[r4 * 4 + e] = pv;
        } else {
          bool vis = rb + e >= lo && rb + e < hi;
          if constexpr (MK == MI_ATTN_MASK_DENSE) {
            const float mv = vis ? p.mask[static_cast<long>(axs[e]) * Lk + j_lane] : 0.f;
            x = fmaf(mv, kLog2e, x);
          }
          if constexpr (MK == MI_ATTN_MASK_TOPK) {
            vis = vis && rank_lane <= axs[e];
            x += zh_lane;
          }
          // selects, not branches; hidden rows past the last one read other rows' side
          // values, and nothing of them may reach dS
          const float pv = fast_exp2(vis ? x : kNegInf);
          dp[r4 * 4 + e] = vis ? pv * (dp[r4 * 4 + e] - dds[e]) : 0.f;
          s[r4 * 4 + e] = pv;
        }
      }
    };
    if (uniform_interior) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) rows4(r4, std::false_type{});
    } else {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) rows4(r4, std::true_type{});
    }

    // dV^T += dO^T P and dK^T += Q^T dS (d x 32 keys; contraction over the 32 rows)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const u32x4_t pb = pack_half<T>(s, half);
      const u32x4_t sb = pack_half<T>(dp, half);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        dvacc[db] = mfma32(T{}, tr_frag(ot, bs.tr0, bs.tr1, half, db, QT::rowBytes), pb, dvacc[db]);
        dkacc[db] = mfma32(T{}, tr_frag(qt, bs.tr0, bs.tr1, half, db, QT::rowBytes), sb, dkacc[db]);
      }
    }
    // the transposed reads (two per MFMA) run two MFMAs ahead
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4, 0);
#pragma unroll
    for (int i = 0; i < 4 * NDB - 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2, 0);
    __builtin_amdgcn_sched_barrier(0);

    // tile t + 1 has landed (this wave's part); every wave is done with this stage
    if (t + kDist < t_hi) wait_next_tile();
    else __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    stg = stg + 1 == kStages ? 0 : stg + 1;
  }

  if (!key_ok) return;
  T* dk = static_cast<T*>(p.dk) + kv_row;
  T* dv = static_cast<T*>(p.dv) + kv_row;
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    store_col<T>(dk, dkacc[db], db, hf, p.scale);
    store_col<T>(dv, dvacc[db], db, hf, 1.f);
  }
}

template <typename T, int D>
hipError_t launch_bwd_t(const AttnParams& p, hipStream_t s) {
  const long nqb = (p.Lq + p.q_per_block - 1) / p.q_per_block;
  const dim3 gq(static_cast<unsigned>(static_cast<long>(p.B) * p.Hkv * nqb));
  const long nkb = (p.Lk + 127) / 128;
  const dim3 gk(static_cast<unsigned>(static_cast<long>(p.B) * p.Hkv * nkb));
  switch (p.mask_kind) {
#define MI_BWD_CASE(KIND)                                                              \
  case KIND:                                                                           \
    hipLaunchKernelGGL((dq_kernel<T, D, KIND>), gq, dim3(kBT), 0, s, p);               \
    hipLaunchKernelGGL((dkdv_kernel<T, D, KIND>), gk, dim3(kBT), 0, s, p);             \
    break;
    MI_BWD_CASE(MI_ATTN_MASK_NONE)
    MI_BWD_CASE(MI_ATTN_MASK_CAUSAL)
    MI_BWD_CASE(MI_ATTN_MASK_WINDOW)
    MI_BWD_CASE(MI_ATTN_MASK_DENSE)
    MI_BWD_CASE(MI_ATTN_MASK_TOPK)
#undef MI_BWD_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_backward(const AttnParams& p, int dtype, hipStream_t s) {
  if (dtype == MI_ATTN_BF16) return p.d == 128 ? launch_bwd_t<bf16_t, 128>(p, s) : launch_bwd_t<bf16_t, 64>(p, s);
  if (dtype == MI_ATTN_F16) return p.d == 128 ? launch_bwd_t<f16_t, 128>(p, s) : launch_bwd_t<f16_t, 64>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace mi_attn
