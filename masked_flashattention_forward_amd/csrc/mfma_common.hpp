// Device helpers shared by the MFMA attention kernels (prefill and split-KV decode).
#pragma once

#include "common.hpp"

namespace mi_attn {
namespace mfma {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x16_t mfma32(bf16_t, const u32x4_t& a, const u32x4_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}
__device__ __forceinline__ f32x16_t mfma32(f16_t, const u32x4_t& a, const u32x4_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c, 0,
                                                0, 0);
}

__device__ __forceinline__ uint32_t pack2(bf16_t, float a, float b) {
  f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
__device__ __forceinline__ uint32_t pack2(f16_t, float a, float b) {
  f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
}

// max over lanes l and l ^ 32 (v_permlane32_swap, no LDS round trip)
__device__ __forceinline__ float max_halves(float x) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// Buffer resource over `bytes` bytes at `base`: loads past the end return zeros.
// Every caller's base and size are wave-uniform. They are passed through readfirstlane so
// the descriptor is built in SGPRs whatever the compiler's uniformity analysis concludes:
// the inline-asm direct loads take it with an "s" constraint, which a VGPR copy would not
// satisfy.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
  void* ub = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ub, static_cast<short>(0), __builtin_amdgcn_readfirstlane(bytes),
                                           0x00020000);
}
__device__ __forceinline__ u32x4_t buffer_load16(__amdgpu_buffer_rsrc_t r, int byte_offset) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, byte_offset, 0, 0));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// 16-byte slot swizzle of a tile row. Rows are stored unpadded; slot s of row r lives at
// slot s ^ swz(r). With 64 banks (16 lanes per cycle for 128-bit reads, 32 lanes for
// 64-bit reads) it makes both operand reads conflict-free: the K read (16 consecutive
// rows, one slot each) and the transposed V read (4 consecutive rows x 4 aligned slots).
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}
template <int D>
__device__ __forceinline__ int tile_off(int r, int slot) {
  return r * (D * 2) + ((slot ^ swz<D>(r)) << 4);
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));

// Transposed 64-bit LDS read: within each 16-lane group, lane j receives element j % 4 of
// the 8-byte rows read by lanes j / 4, 4 + j / 4, 8 + j / 4 and 12 + j / 4.
__device__ __forceinline__ u32x2_t lds_read_tr16(const unsigned char* p) {
  const bf16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4_t*)(p));
  return __builtin_bit_cast(u32x2_t, v);
}

// instruction classes of __builtin_amdgcn_sched_group_barrier
constexpr int kSchedValu = 0x002;
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;

// The running max only moves when a row's maximum grows by more than 2^8 (log2 units).
// Between moves, p = exp2(s - m) stays below 2^8, which fp32 sums and 16-bit P hold
// without loss of relative precision; l and the output use the same m, so the result is
// unchanged up to rounding, and most tiles skip rescaling the output accumulator.
constexpr float kRescaleThreshold = 8.0f;
// A lane's sum of exponentials up to this bound (2^kRescaleThreshold) proves that none of
// them exceeds it: the prefill kernel's test for keeping the running max of a tile.
constexpr float kFastSumLimit = 256.0f;

// Workgroup -> (KV group, query block). Workgroups are handed to the 8 XCDs round-robin;
// the remap gives each XCD a contiguous run of KV groups (their K/V stays in that XCD's
// L2), and inside a KV group the query blocks with the most tiles start first.
__device__ __forceinline__ unsigned logical_block(unsigned bid, unsigned nblk) {
  const unsigned per = nblk / 8u;
  if (bid < per * 8u) return (bid % 8u) * per + bid / 8u;
  return bid;
}

// 32-bit LDS address of a pointer into __shared__ memory
__device__ __forceinline__ unsigned lds_address(const void* p) {
  return static_cast<unsigned>(reinterpret_cast<size_t>((__attribute__((address_space(3))) const void*)p));
}

// 16-byte (or 4-byte) buffer load of each lane written straight to LDS at lds_base +
// lane * size (buffer_load ... lds, base in M0). Issued through inline assembly so that
// the compiler does not tie later LDS reads of OTHER ring stages to these loads with a
// conservative vmcnt(0) wait; the kernels order them with explicit vmcnt waits and
// workgroup barriers instead.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rs, const void* lds_base, int voffset) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane(lds_address(lds_base));  // wave-uniform
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(m0), "v"(voffset), "s"(rs)
               : "memory", "m0");
}
// The same with the non-temporal hint (cache policy nt), for rows read once and whole, such
// as the V stream of decode: a 2 GiB read stream of such loads measured 6.6-7.0 TB/s against
// 5.9-6.1 TB/s without the hint. (Not for K in decode: its loads take 32 bytes of a row at a
// time and rely on the cache for the rest of the line; with the hint the kernel got slower.)
__device__ __forceinline__ void lds_dma16_nt(__amdgpu_buffer_rsrc_t rs, const void* lds_base, int voffset) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane(lds_address(lds_base));
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
               :
               : "s"(m0), "v"(voffset), "s"(rs)
               : "memory", "m0");
}
// The same with the LDS destination given as a 32-bit LDS byte address and a
// wave-uniform byte offset added to every lane's voffset (soffset).
__device__ __forceinline__ void lds_dma16_at(__amdgpu_buffer_rsrc_t rs, unsigned lds_addr, int voffset,
                                             int soffset) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane(lds_addr);
  const int so = __builtin_amdgcn_readfirstlane(soffset);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(m0), "v"(voffset), "s"(rs), "s"(so)
               : "memory", "m0");
}

// 4-byte form (buffer_load_dword ... lds): lane i's dword lands at lds_addr + 4 * i.
__device__ __forceinline__ void lds_dma4_at(__amdgpu_buffer_rsrc_t rs, unsigned lds_addr, int voffset, int soffset) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane(lds_addr);
  const int so = __builtin_amdgcn_readfirstlane(soffset);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :
               : "s"(m0), "v"(voffset), "s"(rs), "s"(so)
               : "memory", "m0");
}

// The same from a per-lane 64-bit global address (global_load_lds_dwordx4): lane i's 16
// bytes from src land at lds_addr + 16 * i. Used where the rows of one tile come from
// unrelated places (cache pages), which a 32-bit buffer offset cannot always reach.
__device__ __forceinline__ void lds_dma16_global(unsigned lds_addr, const void* src) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane(lds_addr);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(m0), "v"(src)
               : "memory", "m0");
}
// The same with the non-temporal hint (see lds_dma16_nt).
__device__ __forceinline__ void lds_dma16_global_nt(unsigned lds_addr, const void* src) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane(lds_addr);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off nt"
               :
               : "s"(m0), "v"(src)
               : "memory", "m0");
}

// Varlen K/V addressing. A sequence's keys 0 .. Lk-1: the first ctx come from the cache
// (paged through the block table, or packed at cu_k[seq]), the rest (two-source form)
// from the new-token arrays at row q_start + j - ctx. Every index is clamped into its
// array, so no value of the caller's int32 arrays can move an access out of bounds.
struct VarlenSeq {
  int seq, q_start, Lq, Lk, ctx, k_start;
};

__device__ __forceinline__ VarlenSeq varlen_seq(const AttnParams& p, int seq) {
  VarlenSeq v;
  v.seq = seq;
  v.q_start = min(max(p.cu_q[seq], 0), p.total_q);
  v.Lq = min(max(p.cu_q[seq + 1], v.q_start), p.total_q) - v.q_start;
  // at most the keys the cache can hold for one sequence (plus its new ones), so loop
  // bounds stay small whatever the lengths say
  const int cache_keys = p.block_table != nullptr ? (p.max_pages << p.page_shift) : p.kv_rows;
  v.k_start = p.cu_k[seq];
  v.Lk = min(max(p.cu_k[seq + 1] - v.k_start, 0), cache_keys + (p.k_new != nullptr ? v.Lq : 0));
  v.ctx = p.k_new != nullptr ? v.Lk - v.Lq : v.Lk;
  return v;
}

// Block-table entry for key j (clamped to the last key, which the mask hides when j is
// past it); only meaningful for the paged form.
__device__ __forceinline__ int varlen_page(const AttnParams& p, const VarlenSeq& v, int j) {
  j = min(j, v.Lk - 1);
  return p.block_table[static_cast<long>(v.seq) * p.max_pages + min(max(j, 0) >> p.page_shift, p.max_pages - 1)];
}

// Element offset of key j's row of KV head g (plus `col` elements), and whether it lies
// in the new-token arrays; `page` is varlen_page(p, v, j) for the paged form. Branch
// free: both candidate rows are formed and one is selected per lane (callers select the
// base pointer the same way, from values held in registers).
template <int D>
__device__ __forceinline__ long varlen_row(const AttnParams& p, const VarlenSeq& v, int g, int j, int page, int col,
                                           bool* is_new) {
  j = min(j, v.Lk - 1);
  const bool nw = j >= v.ctx;
  const int pg = min(max(page, 0), p.kv_rows - 1);
  const long paged_row = (static_cast<long>(pg) << p.page_shift) | (j & ((1 << p.page_shift) - 1));
  const long packed_row = min(max(static_cast<long>(v.k_start) + j, 0L), static_cast<long>(p.kv_rows) - 1);
  const long cache_row = p.block_table != nullptr ? paged_row : packed_row;
  const long row = nw ? static_cast<long>(v.q_start) + (j - v.ctx) : cache_row;
  *is_new = nw;
  return (row * p.Hkv + g) * D + col;
}

// c ? a : b on pointer values (by-value parameters: a select of two variables would
// otherwise become a select of their addresses and a load)
template <typename T>
__device__ __forceinline__ const T* pick(bool c, const T* a, const T* b) {
  return c ? a : b;
}

// s_waitcnt immediate for "at most n vector-memory operations outstanding" (gfx9
// encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt left at their maximum).
constexpr int vmcnt_imm(int n) { return (n & 0xf) | ((n >> 4) << 14) | (0x7 << 4) | (0xf << 8); }

// Per-lane state of the score modifiers and the dense mask (built once per kernel).
// The MFMA gives s = q.k (the sign of the scale folded into Q); the logit in log2 units
// is s * cexp with cexp = |scale| * log2(e).
struct Mods {
  float cexp;     // |scale| * log2(e)
  float cap;      // softcap (0: off)
  float ct;       // softcap: 2 * |scale| / cap * log2(e), the exponent factor of tanh
  float k1, k2;   // softcap: cap * log2(e) and -2 * cap * log2(e)
  float slope2;   // ALiBi slope of the lane's query head times log2(e) (0: off)
  int pos;        // the lane's absolute query position
  const float* mrow;  // dense mask row of the lane's (b, h, i), or nullptr
  long msj;           // its key stride
};

// (EXT: the modifier fields; the dense mask row is used by the dense kind, and by EXT
// instances of the top-k kind)
template <bool EXT>
__device__ __forceinline__ Mods make_mods(const AttnParams& p, float cexp, int b, int h_row, int i_row, int pos,
                                          bool with_mask) {
  Mods m{};
  m.cexp = cexp;
  if constexpr (EXT) {
    m.cap = p.softcap;
    if (m.cap > 0.f) {
      m.ct = 2.f * fabsf(p.scale) / m.cap * kLog2e;
      m.k1 = m.cap * kLog2e;
      m.k2 = -2.f * m.cap * kLog2e;
    }
    m.slope2 = p.alibi != nullptr ? p.alibi[h_row] * kLog2e : 0.f;
    m.pos = pos;
  }
  m.mrow = with_mask && p.mask != nullptr ? p.mask + b * p.ms[0] + h_row * p.ms[1] + i_row * p.ms[2] : nullptr;
  m.msj = p.ms[3];
  return m;
}

// Whether a call needs the EXT kernel instances.
__host__ __device__ inline bool needs_ext(const AttnParams& p) {
  return has_mods(p) || (p.mask_kind == MI_ATTN_MASK_TOPK && p.mask != nullptr);
}

// Logit in log2 units from the raw score s of a key at signed distance dist = j - p_i
// (a float: exact below 2^24). EXT instances apply softcap, cap * tanh(t / cap) of the
// scaled score t with tanh(x) = 1 - 2 / (e^{2x} + 1) (saturates to +-1, no overflow),
// then the ALiBi bias -slope * |dist| (the abs is an operand modifier); the others
// only scale.
template <bool EXT>
__device__ __forceinline__ float modified_logit(float s, float dist, const Mods& m) {
  if constexpr (!EXT) {
    return s * m.cexp;
  } else {
    float x;
    if (m.cap > 0.f) {
      const float r = __builtin_amdgcn_rcpf(__builtin_amdgcn_exp2f(s * m.ct) + 1.f);
      x = fmaf(m.k2, r, m.k1);
    } else {
      x = s * m.cexp;
    }
    if (m.slope2 != 0.f) x = fmaf(-m.slope2, fabsf(dist), x);
    return x;
  }
}

// EXT tile that needs no mask (every key visible to every row of the block): the score
// modifiers only, in the log2 domain.
template <int NKB>
__device__ __forceinline__ void mods_tile(f32x16_t* sacc, int j0, int hf, const Mods& md) {
  const float base = static_cast<float>(j0 + hf * 4 - md.pos);  // distance of the lane's first key
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i)
      sacc[kb][i] = modified_logit<true>(sacc[kb][i], base + static_cast<float>(kb * 32 + (i / 4) * 8 + i % 4), md);
}

// Per-element mask of one tile's S^T registers (32x32 MFMA layout: lane holds query column
// l % 32 and, per 32-key block kb, keys kb*32 + 8*(i/4) + 4*hf + i%4 in register i).
// Visible logits move to the log2 domain (modified_logit, plus the dense mask or the top-k
// bias, times log2 e); hidden ones become -inf. `xr`/`xz` are the tile's top-k ranks and
// zero_hold values (index = key - j0); a dense mask given with the top-k kind is added to
// the kept keys. Lk is the key count of the (batch or sequence) the tile belongs to; tau_row
// is clamped to Lk - 1 by the caller, so keys past Lk (rank INT32_MAX) are never kept.
// (dense kind: pre, when given, holds the lane's 4 NKB groups of 4 entries, loaded ahead by
// load_dense_tile; otherwise the entries are read here)
template <int MK, int NKB, bool EXT>
__device__ __forceinline__ void mask_tile(f32x16_t* sacc, const AttnParams& p, int Lk, int j0, int hf, int pos,
                                          int32_t tau_row, const Mods& md, const int32_t* xr, const float* xz,
                                          const float4* pre = nullptr) {
  const float base = EXT ? static_cast<float>(j0 + hf * 4 - pos) : 0.f;  // distance of the lane's first key
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int kk = kb * 32 + r4 * 8 + hf * 4;  // first of 4 consecutive keys in the tile
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = j0 + kk + e;
        float s = modified_logit<EXT>(sacc[kb][r4 * 4 + e], base + static_cast<float>(kk - hf * 4 + e), md);
        bool vis = j < Lk;
        if constexpr (MK == MI_ATTN_MASK_CAUSAL) vis = vis && j <= pos;
        if constexpr (MK == MI_ATTN_MASK_WINDOW) vis = vis && j <= pos && j >= pos - p.window_left;
        // side reads use key j0 (always < Lk in a visited tile) in place of keys past Lk
        if constexpr (MK == MI_ATTN_MASK_DENSE) {
          float mv;
          if (pre != nullptr) {
            const float4 q4 = pre[kb * 4 + r4];
            mv = e == 0 ? q4.x : e == 1 ? q4.y : e == 2 ? q4.z : q4.w;
          } else {
            mv = md.mrow[(vis ? j : j0) * md.msj];
          }
          s = fmaf(vis ? mv : 0.f, kLog2e, s);
        }
        if constexpr (MK == MI_ATTN_MASK_TOPK) {
          const int idx = vis ? kk + e : 0;
          vis = vis && (!p.topk_causal || j <= pos) && xr[idx] <= tau_row;
          float bias = xz[idx];
          if (EXT && md.mrow != nullptr) bias += md.mrow[(vis ? j : j0) * md.msj];
          s = fmaf(bias, kLog2e, s);
        }
        sacc[kb][r4 * 4 + e] = vis ? s : kNegInf;
      }
    }
  }
}

// The dense-mask entries a lane's mask_tile needs for the tile at key j0: group kb * 4 + r4
// holds keys j0 + kb * 32 + r4 * 8 + hf * 4 + 0..3 of its row. One 16-byte load per group
// when vec (the caller's test that the row is contiguous and 16-byte aligned) and the group
// lies below Lk; otherwise four loads with keys clamped to the tile's first key.
template <int NKB>
__device__ __forceinline__ void load_dense_tile(float4* out, const Mods& md, int Lk, int j0, int hf, bool vec) {
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int j = j0 + kb * 32 + r4 * 8 + hf * 4;
      if (vec && j + 3 < Lk) {
        out[kb * 4 + r4] = *reinterpret_cast<const float4*>(md.mrow + j);
      } else {
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = md.mrow[(j + e < Lk ? j + e : j0) * md.msj];
        out[kb * 4 + r4] = float4{v[0], v[1], v[2], v[3]};
      }
    }
}

// Top-k mask of one tile whose side data sits in LDS, padded to the full tile:
// xr[k] = rank of key j0 + k (INT32_MAX past Lk) and xzl[k] = its zero_hold times log2(e)
// (0 past Lk). A key stays when its rank is at most the row's threshold (clamped below
// Lk, so keys past Lk never stay); kDiag tiles (reaching past the block's first query
// position, causal selection only) also hide keys after the row's own position. Results
// are in the log2 domain.
template <int NKB, bool kDiag, bool EXT>
__device__ __forceinline__ void mask_tile_topk(f32x16_t* sacc, int j0, int hf, int pos, int32_t tau_row,
                                               const Mods& md, const int32_t* xr, const float* xzl) {
  const int lim = pos - j0;  // keys kk <= lim are at or before the row's position
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int kk = kb * 32 + r4 * 8 + hf * 4;  // first of 4 consecutive keys in the tile
      const int4 rk = *reinterpret_cast<const int4*>(xr + kk);
      const float4 zl = *reinterpret_cast<const float4*>(xzl + kk);
      const int rks[4] = {rk.x, rk.y, rk.z, rk.w};
      const float zs[4] = {zl.x, zl.y, zl.z, zl.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        bool vis = rks[e] <= tau_row;
        if constexpr (kDiag) vis = vis && kk + e <= lim;
        float bias = zs[e];
        if (EXT && md.mrow != nullptr) bias = fmaf(md.mrow[(vis ? j0 + kk + e : j0) * md.msj], kLog2e, bias);
        const float s = modified_logit<EXT>(sacc[kb][r4 * 4 + e], static_cast<float>(j0 + kk + e - pos), md) + bias;
        sacc[kb][r4 * 4 + e] = vis ? s : kNegInf;
      }
    }
  }
}

// The same for a gathered tile: key k of the tile is key xi[k] of the cache (ascending;
// padding entries carry key Lk, rank INT32_MAX and value 0, and the clamped threshold
// hides them).
template <int NKB, bool kDiag, bool EXT>
__device__ __forceinline__ void mask_tile_topk_list(f32x16_t* sacc, int hf, int pos, int32_t tau_row,
                                                    const Mods& md, const int32_t* xr, const float* xzl,
                                                    const int32_t* xi) {
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int kk = kb * 32 + r4 * 8 + hf * 4;  // first of 4 consecutive keys in the tile
      const int4 rk = *reinterpret_cast<const int4*>(xr + kk);
      const float4 zl = *reinterpret_cast<const float4*>(xzl + kk);
      const int4 ji = *reinterpret_cast<const int4*>(xi + kk);
      const int rks[4] = {rk.x, rk.y, rk.z, rk.w};
      const float zs[4] = {zl.x, zl.y, zl.z, zl.w};
      const int js[4] = {ji.x, ji.y, ji.z, ji.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        bool vis = rks[e] <= tau_row;
        if constexpr (kDiag) vis = vis && js[e] <= pos;
        float bias = zs[e];
        if (EXT && md.mrow != nullptr) bias = fmaf(md.mrow[(vis ? js[e] : 0) * md.msj], kLog2e, bias);
        const float s = modified_logit<EXT>(sacc[kb][r4 * 4 + e], static_cast<float>(js[e] - pos), md) + bias;
        sacc[kb][r4 * 4 + e] = vis ? s : kNegInf;
      }
    }
  }
}

// Whether a tile [j0, j0 + BN) needs per-element masking for a block whose query rows sit
// at positions P0..P1: tiles every row sees entirely (and inside Lk) skip it (EXT
// instances then apply the score modifiers alone, mods_tile).
template <int MK, int BN>
__device__ __forceinline__ bool tile_needs_mask(const AttnParams& p, int Lk, int j0, int P0, int P1) {
  const int j_end = j0 + BN - 1;
  bool need = p.no_skip || j_end >= Lk || MK == MI_ATTN_MASK_DENSE || MK == MI_ATTN_MASK_TOPK;
  if constexpr (MK == MI_ATTN_MASK_CAUSAL || MK == MI_ATTN_MASK_WINDOW) need = need || j_end > P0;
  if constexpr (MK == MI_ATTN_MASK_WINDOW) need = need || j0 < P1 - p.window_left;
  return need;
}

}  // namespace mfma
}  // namespace mi_attn
