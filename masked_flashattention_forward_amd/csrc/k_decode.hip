// Split-KV decode kernel: few query rows per KV head (G * Lq <= 32), long key range.
//
// This is the decode step of the chunked forward (ExecuTorch pull request #10466 page,
// "Summary") with past keys and Lq << Lk (FastChat pull request #2315 page): the cost is
// streaming K and V once from HBM. A workgroup takes one (batch, KV head) and one key
// range ("split"); its 4 wavefronts stream disjoint 32-key tiles of that range
// independently, each with its own online-softmax state for all G * Lq rows:
//   K tile   loaded straight into registers in the 32x32x16 MFMA A-operand layout;
//   V tile   loaded straight into a private 2-stage LDS ring (buffer_load ... lds, with the
//            non-temporal hint) and read back transposed (ds_read_b64_tr_b16) as the V^T
//            operand;
//   S^T = K Q^T and O^T += V^T P^T on MFMA, softmax guarded as in the prefill kernel.
// No workgroup barrier is needed while streaming; at the end the four states are merged
// through LDS by log-sum-exp, giving the split's partial (o, lse) or, with one split, the
// output itself.
#include "common.hpp"
#include "kernels.hpp"
#include "mfma_common.hpp"

namespace mi_attn {

hipError_t launch_lse_merge(const AttnParams& p, int dtype, hipStream_t s);

namespace {

using namespace mfma;

constexpr int kDecWaves = 4;
constexpr int kDecThreads = kDecWaves * kWave;
constexpr int kDecBN = 32;  // keys per wavefront tile


template <int D>
struct DecTile {
  static constexpr int vBytes = kDecBN * D * 2;     // one V tile in LDS
  static constexpr int vLoads = vBytes / 1024;      // 1 KB direct loads per V tile
  static constexpr int kLoads = D / 16;             // 16-byte K loads per lane per tile
  static constexpr int waveBytes = 2 * vBytes;      // 2-stage ring per wavefront
  static constexpr int lds = kDecWaves * waveBytes;
  static constexpr int NDB = D / 32;
  // merge area (reuses the rings): per non-zero wave, O^T registers + m + l per lane
  static constexpr int mergeFloats = (NDB * 16 + 2) * kWave;
  static_assert((kDecWaves - 1) * mergeFloats * 4 <= lds, "merge area fits in the rings");
};

// VARLEN: one item of the varlen work list (a key range of a sequence with at most 32
// query rows per KV head); K/V rows come from cache pages, packed rows or the new-token
// arrays through per-lane 64-bit addresses, and the output is token-major.
template <typename T, int D, int MK, bool VARLEN = false, bool EXT = false>
__global__ __launch_bounds__(kDecThreads, 2) void decode_kernel(AttnParams p) {
  static_assert(!VARLEN || MK <= MI_ATTN_MASK_WINDOW, "varlen takes the key-position masks");
  using TL = DecTile<D>;
  constexpr int NDB = TL::NDB;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[TL::lds];

  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  const int l32 = lane & 31;
  const int hf = lane >> 5;

  int bg, b, g, Lq, Lk;
  const int split = blockIdx.y;
  VarlenSeq vs{};
  int item = 0;
  bool item_partial = false;
  int lo, hi;
  if constexpr (VARLEN) {
    // the KV heads of one item are consecutive workgroups (they read the same cache rows)
    g = static_cast<int>(blockIdx.x % static_cast<unsigned>(p.Hkv));
    item = static_cast<int>(blockIdx.x / static_cast<unsigned>(p.Hkv));
    if (item >= p.vl_counts[2]) return;  // the whole workgroup, before any barrier
    const int4 it = p.vl_items[item];
    const int4 un = p.vl_units[it.x];
    vs = varlen_seq(p, un.x);
    item_partial = (un.w & 0x3fffffff) > 1;
    lo = it.y;  // the item's key range, cut on 64-key boundaries by the work-list kernel
    hi = it.z;
    Lq = vs.Lq;
    Lk = vs.Lk;
    bg = 0;
    b = 0;
  } else {
    bg = blockIdx.x;
    b = bg / p.Hkv;
    g = bg % p.Hkv;
    Lq = p.Lq;
    Lk = p.Lk;
  }
  const int rows = p.G * Lq;
  const int P0 = Lk - Lq;      // position of the first query row
  const int P1 = Lk - 1;       // position of the last

  // this lane's row (query-major: row r -> query r / G, head g*G + r % G)
  const bool row_ok = l32 < rows;
  const int i_row = row_ok ? l32 / p.G : 0;
  const int h_row = g * p.G + (row_ok ? l32 % p.G : 0);
  const int pos = Lk - Lq + i_row;
  const long row_index = VARLEN ? static_cast<long>(vs.q_start + i_row) * p.Hq + h_row
                                : (static_cast<long>(b) * p.Hq + h_row) * Lq + i_row;

  // element offsets of this lane's q and out rows (strided for the single-batch call)
  const long q_off = VARLEN ? row_index * D : b * p.qs[0] + h_row * p.qs[1] + i_row * p.qs[2];
  const long o_off = VARLEN ? row_index * D : b * p.os[0] + h_row * p.os[1] + i_row * p.os[2];
  const T* Q = static_cast<const T*>(p.q);
  const bool negate = p.scale < 0.f;
  const float cexp = fabsf(p.scale) * kLog2e;
  const Mods md = make_mods<EXT>(p, cexp, b, h_row, i_row, pos, MK == MI_ATTN_MASK_DENSE || MK == MI_ATTN_MASK_TOPK);
  u32x4_t qreg[D / 16];
#pragma unroll
  for (int dc = 0; dc < D / 16; ++dc) {
    u32x4_t x = {0u, 0u, 0u, 0u};
    if (row_ok) x = *reinterpret_cast<const u32x4_t*>(Q + q_off + dc * 16 + hf * 8);
    if (negate) x ^= 0x80008000u;
    qreg[dc] = x;
  }

  // key range of this split
  if constexpr (!VARLEN) {
    key_range(range_kind(p), p.window_left, Lk, P0, P1, &lo, &hi);
    if (p.no_skip) { lo = 0; hi = Lk; }
    const int s0 = split * p.keys_per_split;
    const int s1 = min(Lk, s0 + p.keys_per_split);
    lo = max(lo, s0);
    hi = min(hi, s1);
  }
  const int t_lo = lo / kDecBN;
  const int t_hi = (hi > lo) ? (hi + kDecBN - 1) / kDecBN : t_lo;
  const int ntiles_all = (Lk + kDecBN - 1) / kDecBN;

  // K / V of this (batch, KV head): rows ks / vs elements apart (D for contiguous K/V);
  // the ranges cover rows 0 .. Lk-1 (the host keeps them below 2^31 bytes)
  const long ksr = VARLEN ? D : p.ks[2];
  const long vsr = VARLEN ? D : p.vs[2];
  const long bgk = static_cast<long>(bg) * Lk;
  const __amdgpu_buffer_rsrc_t krs =
      make_rsrc(static_cast<const T*>(p.k) + (VARLEN ? 0 : b * p.ks[0] + g * p.ks[1]),
                VARLEN ? 0 : static_cast<int>(((Lk - 1) * ksr + D) * 2));
  const __amdgpu_buffer_rsrc_t vrs =
      make_rsrc(static_cast<const T*>(p.v) + (VARLEN ? 0 : b * p.vs[0] + g * p.vs[1]),
                VARLEN ? 0 : static_cast<int>(((Lk - 1) * vsr + D) * 2));

  int32_t tau_row = 0, tau_blk = 0;
  if constexpr (MK == MI_ATTN_MASK_TOPK) {
    // clamped below Lk: every allowed key when tau says "all kept", never a padding key
    tau_row = min(p.tau[static_cast<long>(bg) * p.Lq + i_row], Lk - 1);
    tau_blk = min(p.tau[static_cast<long>(bg) * p.Lq], Lk - 1);
  }
  // dense-mask summary flags of this (batch, KV head) (one query block)
  const long flag_base =
      (static_cast<long>(p.flag_b > 1 ? b : 0) * p.flag_g + (p.flag_g > 1 ? g : 0)) * ntiles_all;
  auto tile_live = [&](int t) -> bool {
    if (p.no_skip) return true;
    if constexpr (MK == MI_ATTN_MASK_DENSE) return p.tile_live == nullptr || p.tile_live[flag_base + t] != 0;
    if constexpr (MK == MI_ATTN_MASK_TOPK) return p.tile_min_rank[static_cast<long>(bg) * ntiles_all + t] <= tau_blk;
    return true;
  };
  // this wavefront's tiles: t_lo + wave, then every 4th, skipping dead ones
  auto next_tile = [&](int t) -> int {
    while (t < t_hi && !tile_live(t)) t += kDecWaves;
    return t;
  };

  unsigned char* const ring = smem + wave * TL::waveBytes;
  // VARLEN base pointers in registers (the per-lane cache / new-token choice selects values)
  const T* const k_cache = static_cast<const T*>(p.k);
  const T* const v_cache = static_cast<const T*>(p.v);
  const T* const k_fresh = static_cast<const T*>(p.k_new);
  const T* const v_fresh = static_cast<const T*>(p.v_new);
  // VARLEN (paged form): block-table entry of key j0 + l32 of the next tile to issue,
  // loaded one tile ahead; the V rows' entries come from the lanes holding those keys.
  int page_next = 0;
  auto issue = [&](int t, u32x4_t* kr, int stg) {
    const int j0 = t * kDecBN;
    unsigned char* dst = ring + stg * TL::vBytes;
    if constexpr (VARLEN) {
      const int page = page_next;
      bool nk;
      const long ek = varlen_row<D>(p, vs, g, j0 + l32, page, hf * 8, &nk);
      const T* kb = pick(nk, k_fresh, k_cache) + ek;
#pragma unroll
      for (int dc = 0; dc < TL::kLoads; ++dc) kr[dc] = *reinterpret_cast<const u32x4_t*>(kb + dc * 16);
#pragma unroll
      for (int c = 0; c < TL::vLoads; ++c) {
        const int r = c * (1024 / (D * 2)) + lane / (D / 8);
        const int ps = lane % (D / 8);
        bool nv;
        const long ev = varlen_row<D>(p, vs, g, j0 + r, __shfl(page, r, kWave), (ps ^ swz<D>(r)) << 3, &nv);
        lds_dma16_global_nt(lds_address(dst + c * 1024), pick(nv, v_fresh, v_cache) + ev);
      }
      if (p.block_table != nullptr) page_next = varlen_page(p, vs, j0 + kDecWaves * kDecBN + l32);
      return;
    }
    // K: lane holds key j0 + l32, dims dc*16 + hf*8 .. +8 (the A operand of S^T = K Q^T)
#pragma unroll
    for (int dc = 0; dc < TL::kLoads; ++dc)
      kr[dc] = buffer_load16(krs, static_cast<int>(((j0 + l32) * ksr + dc * 16 + hf * 8) * 2));
    // V: 1 KB direct loads into the swizzled [key][d] tile, non-temporal (read once, whole rows)
#pragma unroll
    for (int c = 0; c < TL::vLoads; ++c) {
      const int r = c * (1024 / (D * 2)) + lane / (D / 8);
      const int ps = lane % (D / 8);
      const int gofs = static_cast<int>(((j0 + r) * vsr + ((ps ^ swz<D>(r)) << 3)) * 2);
      lds_dma16_nt(vrs, dst + c * 1024, gofs);
    }
  };
  constexpr int kLoadsPerTile = TL::kLoads + TL::vLoads;

  f32x16_t oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16_t{};
  float m_run = kNegInf;
  float l_run = 0.f;

  u32x4_t kcur[TL::kLoads], knext[TL::kLoads];
  int t = next_tile(t_lo + wave);
  int stg = 0;
  if (VARLEN && t < t_hi && p.block_table != nullptr) page_next = varlen_page(p, vs, t * kDecBN + l32);
  if (t < t_hi) issue(t, kcur, 0);
  const int tr_row = 4 * hf + (lane & 15) / 4;
  const int tr_dim = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  while (t < t_hi) {
    const int tn = next_tile(t + kDecWaves);
    if (tn < t_hi) {
      issue(tn, knext, stg ^ 1);
      // tile t has landed (tn's loads, and the varlen block-table load behind them, may not)
      if (VARLEN && p.block_table != nullptr)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(kLoadsPerTile + 1));
      else
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(kLoadsPerTile));
    } else {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    }
    const int j0 = t * kDecBN;

    // S^T = K Q^T (32 keys x 32 rows)
    f32x16_t sacc[1];
    {
      f32x16_t acc = f32x16_t{};
#pragma unroll
      for (int dc = 0; dc < D / 16; ++dc) acc = mfma32(T{}, kcur[dc], qreg[dc], acc);
      sacc[0] = acc;
    }
    float cm = cexp;
    if (tile_needs_mask<MK, kDecBN>(p, Lk, j0, P0, P1)) {
      const int32_t* xr = nullptr;
      const float* xz = nullptr;
      if constexpr (MK == MI_ATTN_MASK_TOPK) {
        xr = p.rank + bgk + j0;
        xz = p.zero_hold + bgk + j0;
      }
      mask_tile<MK, 1, EXT>(sacc, p, Lk, j0, hf, pos, tau_row, md, xr, xz);
      cm = 1.f;
    } else if constexpr (EXT) {
      mods_tile<1>(sacc, j0, hf, md);  // a tile every row sees: the score modifiers alone
      cm = 1.f;
    }

    float mx4[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
#pragma unroll
    for (int e = 0; e < 16; ++e) mx4[e & 3] = fmaxf(mx4[e & 3], sacc[0][e]);
    float mx = fmaxf(fmaxf(mx4[0], mx4[1]), fmaxf(mx4[2], mx4[3]));
    mx = max_halves(mx) * cm;
    const float m_next = (mx > m_run + kRescaleThreshold) ? mx : m_run;
    const float m_use = (m_next == kNegInf) ? 0.f : m_next;
    const float alpha = fast_exp2(m_run - m_use);
    m_run = m_next;
    if (!__all(alpha == 1.f)) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
    }
    float ps4[4] = {-0.f, -0.f, -0.f, -0.f};  // (-0 + x is x: the first adds fold away)
    u32x4_t preg[2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      float pv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pv[e] = fast_exp2(fmaf(sacc[0][half * 8 + e], cm, -m_use));
        ps4[e & 3] += pv[e];
      }
      preg[half] = u32x4_t{pack2(T{}, pv[0], pv[1]), pack2(T{}, pv[2], pv[3]), pack2(T{}, pv[4], pv[5]),
                           pack2(T{}, pv[6], pv[7])};
    }
    l_run = fmaf(l_run, alpha, (ps4[0] + ps4[1]) + (ps4[2] + ps4[3]));

    // O^T += V^T P^T (transposed V reads; see the prefill kernel for the lane mapping)
    const unsigned char* vs = ring + stg * TL::vBytes;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        const int d0 = db * 32 + tr_dim;
        const int r0 = kc * 16 + tr_row;
        const u32x2_t lo2 = lds_read_tr16(vs + tile_off<D>(r0, d0 >> 3) + ((d0 & 7) << 1));
        const u32x2_t hi2 = lds_read_tr16(vs + tile_off<D>(r0 + 8, d0 >> 3) + ((d0 & 7) << 1));
        oacc[db] = mfma32(T{}, u32x4_t{lo2.x, lo2.y, hi2.x, hi2.y}, preg[kc], oacc[db]);
      }
    }
#pragma unroll
    for (int dc = 0; dc < TL::kLoads; ++dc) kcur[dc] = knext[dc];
    t = tn;
    stg ^= 1;
  }

  // ---- merge the four wavefronts' states (log-sum-exp), then store
  __syncthreads();  // every wavefront is done with its ring
  float* mf = reinterpret_cast<float*>(smem);
  if (wave > 0) {
    float* dst = mf + (wave - 1) * TL::mergeFloats;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) dst[(db * 16 + i) * kWave + lane] = oacc[db][i];
    dst[(NDB * 16) * kWave + lane] = m_run;
    dst[(NDB * 16 + 1) * kWave + lane] = l_run;
  }
  __syncthreads();
  if (wave != 0) return;
  float m_all = m_run;
#pragma unroll
  for (int w = 1; w < kDecWaves; ++w) m_all = fmaxf(m_all, mf[(w - 1) * TL::mergeFloats + (NDB * 16) * kWave + lane]);
  const float m_ref = (m_all == kNegInf) ? 0.f : m_all;
  const float s0 = fast_exp2(m_run - m_ref);
  float l_all = l_run * s0;
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] *= s0;
#pragma unroll
  for (int w = 1; w < kDecWaves; ++w) {
    const float* src = mf + (w - 1) * TL::mergeFloats;
    const float sw = fast_exp2(src[(NDB * 16) * kWave + lane] - m_ref);
    l_all = fmaf(src[(NDB * 16 + 1) * kWave + lane], sw, l_all);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[db][i] = fmaf(src[(db * 16 + i) * kWave + lane], sw, oacc[db][i]);
  }
  const float l_tot = sum_halves(l_all);
  if (!row_ok) return;
  const bool dead = !(l_tot > 0.f);
  const float inv = dead ? 0.f : 1.f / l_tot;
  const float lse = dead ? kNegInf : (m_all + fast_log2(l_tot)) * kLn2;
  if (VARLEN ? item_partial : p.splits > 1) {
    // partial slot: split-major rows, or the item's own [Hkv, 32] rows
    const long slot = VARLEN ? (static_cast<long>(item) * p.Hkv + g) * 32 + l32
                             : static_cast<long>(split) * p.B * p.Hq * Lq + row_index;
    float* po = p.part_out + slot * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = db * 32 + r4 * 8 + hf * 4;
        *reinterpret_cast<float4*>(po + d0) = float4{oacc[db][r4 * 4] * inv, oacc[db][r4 * 4 + 1] * inv,
                                                     oacc[db][r4 * 4 + 2] * inv, oacc[db][r4 * 4 + 3] * inv};
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
      *reinterpret_cast<u32x2_t*>(O + d0) =
          u32x2_t{pack2(T{}, oacc[db][r4 * 4] * inv, oacc[db][r4 * 4 + 1] * inv),
                  pack2(T{}, oacc[db][r4 * 4 + 2] * inv, oacc[db][r4 * 4 + 3] * inv)};
    }
  if (hf == 0 && p.lse != nullptr) p.lse[row_index] = lse;
}

template <typename T, int D, bool EXT>
void launch_decode_e(const AttnParams& p, hipStream_t s) {
  dim3 grid(p.B * p.Hkv, p.splits), block(kDecThreads);
  switch (p.mask_kind) {
    case MI_ATTN_MASK_NONE: hipLaunchKernelGGL((decode_kernel<T, D, 0, false, EXT>), grid, block, 0, s, p); break;
    case MI_ATTN_MASK_CAUSAL: hipLaunchKernelGGL((decode_kernel<T, D, 1, false, EXT>), grid, block, 0, s, p); break;
    case MI_ATTN_MASK_WINDOW: hipLaunchKernelGGL((decode_kernel<T, D, 2, false, EXT>), grid, block, 0, s, p); break;
    case MI_ATTN_MASK_DENSE: hipLaunchKernelGGL((decode_kernel<T, D, 3, false, EXT>), grid, block, 0, s, p); break;
    default: hipLaunchKernelGGL((decode_kernel<T, D, 4, false, EXT>), grid, block, 0, s, p); break;
  }
}

template <typename T, int D>
void launch_decode_d(const AttnParams& p, hipStream_t s) {
  if (needs_ext(p)) launch_decode_e<T, D, true>(p, s);
  else launch_decode_e<T, D, false>(p, s);
}

// varlen items of decode type: grid = items x KV heads, no split dimension
template <typename T, int D, bool EXT>
void launch_decode_varlen_e(const AttnParams& p, hipStream_t s) {
  dim3 grid(static_cast<unsigned>(static_cast<long>(p.vl_items_cap) * p.Hkv)), block(kDecThreads);
  switch (p.mask_kind) {
    case MI_ATTN_MASK_NONE: hipLaunchKernelGGL((decode_kernel<T, D, 0, true, EXT>), grid, block, 0, s, p); break;
    case MI_ATTN_MASK_CAUSAL: hipLaunchKernelGGL((decode_kernel<T, D, 1, true, EXT>), grid, block, 0, s, p); break;
    default: hipLaunchKernelGGL((decode_kernel<T, D, 2, true, EXT>), grid, block, 0, s, p); break;
  }
}
template <typename T, int D>
void launch_decode_varlen_d(const AttnParams& p, hipStream_t s) {
  // score modifiers (ALiBi, softcap) run the EXT instances
  if (has_mods(p)) launch_decode_varlen_e<T, D, true>(p, s);
  else launch_decode_varlen_e<T, D, false>(p, s);
}

}  // namespace

int decode_block_n() { return kDecBN; }

hipError_t launch_decode_varlen(const AttnParams& p, int dtype, hipStream_t s) {
  if (static_cast<long>(p.vl_items_cap) * p.Hkv > 0x7fffffffL) return hipErrorInvalidValue;
  if (dtype == MI_ATTN_BF16) {
    if (p.d == 128) launch_decode_varlen_d<bf16_t, 128>(p, s); else launch_decode_varlen_d<bf16_t, 64>(p, s);
  } else if (dtype == MI_ATTN_F16) {
    if (p.d == 128) launch_decode_varlen_d<f16_t, 128>(p, s); else launch_decode_varlen_d<f16_t, 64>(p, s);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

int decode_max_rows() { return 32; }

hipError_t launch_decode(const AttnParams& p, int dtype, hipStream_t s) {
  if (static_cast<long>(p.B) * p.Hkv > 0x7fffffffL || p.splits > 65535) return hipErrorInvalidValue;
  if (dtype == MI_ATTN_BF16) {
    if (p.d == 128) launch_decode_d<bf16_t, 128>(p, s); else launch_decode_d<bf16_t, 64>(p, s);
  } else if (dtype == MI_ATTN_F16) {
    if (p.d == 128) launch_decode_d<f16_t, 128>(p, s); else launch_decode_d<f16_t, 64>(p, s);
  } else {
    return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits <= 1) return e;
  return launch_lse_merge(p, dtype, s);
}

}  // namespace mi_attn
