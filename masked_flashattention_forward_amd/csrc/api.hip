// Host side of the C ABI: argument validation, path planning, temporary device memory
// and kernel launches on the caller's stream.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "common.hpp"
#include "kernels.hpp"

using namespace mi_attn;

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(MI_ATTN_EHIP, "%s: %s", what, hipGetErrorString(e));
}

// debug switches (attn_set_debug)
int g_no_skip = 0;
int g_force_path = -1;
int g_force_splits = 0;

struct Shape {
  int B, Hq, Hkv, Lq, Lk, d, mask_kind, window_left, keep_k, dtype;
  int flag_b = 1, flag_g = 1;  // dense-mask summary rows per batch / KV head (1: shared)
};

int validate(const Shape& s) {
  if (s.B <= 0 || s.Hq <= 0 || s.Hkv <= 0 || s.Lq <= 0 || s.Lk <= 0 || s.d <= 0)
    return fail(MI_ATTN_EINVAL, "sizes must be positive (B=%d Hq=%d Hkv=%d Lq=%d Lk=%d d=%d)", s.B, s.Hq, s.Hkv,
                s.Lq, s.Lk, s.d);
  if (s.Hq % s.Hkv != 0)
    return fail(MI_ATTN_EINVAL, "Hq (%d) must be a multiple of Hkv (%d)", s.Hq, s.Hkv);
  if (s.mask_kind < MI_ATTN_MASK_NONE || s.mask_kind > MI_ATTN_MASK_TOPK)
    return fail(MI_ATTN_EINVAL, "unknown mask_kind %d", s.mask_kind);
  if (s.dtype < MI_ATTN_F32 || s.dtype > MI_ATTN_BF16) return fail(MI_ATTN_EINVAL, "unknown dtype %d", s.dtype);
  if (s.mask_kind == MI_ATTN_MASK_WINDOW && s.window_left < 0)
    return fail(MI_ATTN_EINVAL, "window_left must be >= 0 (got %d)", s.window_left);
  if (s.mask_kind == MI_ATTN_MASK_TOPK && s.keep_k < 1)
    return fail(MI_ATTN_EINVAL, "keep_k must be >= 1 (got %d)", s.keep_k);
  const double elems_q = static_cast<double>(s.B) * s.Hq * s.Lq * s.d;
  const double elems_kv = static_cast<double>(s.B) * s.Hkv * s.Lk * s.d;
  if (elems_q > 9.0e15 || elems_kv > 9.0e15) return fail(MI_ATTN_EINVAL, "tensor too large");
  if (s.dtype == MI_ATTN_F32) {
    if (s.d % 4 != 0 || s.d > 256)
      return fail(MI_ATTN_EUNSUPPORTED, "fp32 head dim must be a multiple of 4 up to 256 (got %d)", s.d);
  } else if (s.d != 64 && s.d != 128) {
    return fail(MI_ATTN_EUNSUPPORTED, "fp16/bf16 head dim must be 64 or 128 (got %d)", s.d);
  } else if (static_cast<double>(s.Lk) * s.d * 2 > 2147483647.0) {
    // one (batch, KV head) slice of K or V is addressed with 32-bit byte offsets
    return fail(MI_ATTN_EUNSUPPORTED, "Lk * d * 2 must stay below 2^31 bytes (Lk=%d d=%d)", s.Lk, s.d);
  }
  if (s.mask_kind == MI_ATTN_MASK_TOPK && s.Lk > 65536)
    return fail(MI_ATTN_EUNSUPPORTED, "top-k mask supports Lk <= 65536 (got %d)", s.Lk);
  return MI_ATTN_OK;
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

constexpr int kSummaryMinTiles = 32;  // dense-mask summary from this many key tiles up

struct Plan {
  attn_plan_t pub;
  int q_per_block;     // query positions per workgroup (dense-mask summary granularity)
  size_t off_rank, off_tau, off_tmin, off_sort, off_flags, off_pout, off_plse;
  int list_cap;        // top-k gathered form: entries per kept-key list (0 when not used)
  size_t off_lidx, off_lrank, off_lzh, off_lcnt;
};

// Top-k on the prefill path: attend over per-block kept-key lists (at most keep_k +
// q_per_block - 1 keys each) instead of every causal tile, when the lists are clearly
// shorter than the key range.
int topk_list_cap(int keep_k, int q_per_block, int Lk) {
  const long cap = ((static_cast<long>(keep_k) + q_per_block + 63) / 64) * 64;
  return (cap * 4 <= static_cast<long>(Lk) * 3) ? static_cast<int>(cap) : 0;
}

int make_plan(const Shape& s, Plan* pl) {
  *pl = Plan{};
  attn_plan_t& p = pl->pub;
  const int G = s.Hq / s.Hkv;
  int path = 0;
  if (s.dtype != MI_ATTN_F32) path = choose_half_path(s.B, s.Hkv, G, s.Lq, s.Lk, s.d, s.mask_kind);
  if (g_force_path >= 0) {
    if (g_force_path == 0) {
      path = 0;
    } else if (s.dtype == MI_ATTN_F32) {
      return fail(MI_ATTN_EUNSUPPORTED, "forced path %d needs fp16/bf16 inputs", g_force_path);
    } else if (!half_path_available(g_force_path, s.d, G, s.Lq)) {
      return fail(MI_ATTN_EUNSUPPORTED, "forced path %d cannot run d=%d G*Lq=%d", g_force_path, s.d, G * s.Lq);
    } else {
      path = g_force_path;
    }
  }
  p.path = path;
  p.splits = 1;
  HalfPlan hp{};
  if (path == 0) {
    p.block_m = 4;
    p.block_n = 64;
    p.grid = static_cast<int>((static_cast<long>(s.B) * s.Hq * s.Lq + 3) / 4);
    pl->q_per_block = 1;
  } else {
    hp = plan_half_path(path, s.B, s.Hkv, G, s.Lq, s.Lk, s.d, s.mask_kind, s.window_left, g_force_splits);
    p.block_m = hp.block_m;
    p.block_n = hp.block_n;
    p.grid = hp.grid;
    p.splits = hp.splits;
    pl->q_per_block = hp.q_per_block;
  }
  // workspace layout
  size_t off = 0;
  const long bh = static_cast<long>(s.B) * s.Hkv;
  if (s.mask_kind == MI_ATTN_MASK_TOPK) {
    pl->off_rank = off; off = align256(off + sizeof(int32_t) * bh * s.Lk);
    pl->off_tau = off;  off = align256(off + sizeof(int32_t) * bh * s.Lq);
    pl->off_tmin = off; off = align256(off + sizeof(int32_t) * bh * ((s.Lk + p.block_n - 1) / p.block_n));
    pl->off_sort = off; off = align256(off + topk_sort_ws_bytes(static_cast<int>(bh), s.Lk));
    if (path == 1 && !g_no_skip) pl->list_cap = topk_list_cap(s.keep_k, pl->q_per_block, s.Lk);
    if (pl->list_cap > 0) {
      const size_t nl = static_cast<size_t>(bh) * ((s.Lq + pl->q_per_block - 1) / pl->q_per_block);
      pl->off_lidx = off;  off = align256(off + sizeof(int32_t) * nl * pl->list_cap);
      pl->off_lrank = off; off = align256(off + sizeof(int32_t) * nl * pl->list_cap);
      pl->off_lzh = off;   off = align256(off + sizeof(float) * nl * pl->list_cap);
      pl->off_lcnt = off;  off = align256(off + sizeof(int32_t) * nl);
    }
  }
  // Dense masks: per-tile summary flags let the kernels skip tiles the mask hides
  // entirely. For short key ranges the separate summary pass and its buffer cost more than
  // visiting every tile (each visited tile reads its mask entries anyway), so the flags
  // are only built from kSummaryMinTiles key tiles up.
  const int key_tiles = (s.Lk + p.block_n - 1) / p.block_n;
  if (s.mask_kind == MI_ATTN_MASK_DENSE && path != 0 && key_tiles >= kSummaryMinTiles) {
    p.mask_summary = 1;
    pl->off_flags = off;
    off = align256(off + static_cast<size_t>(s.flag_b) * s.flag_g *
                             ((s.Lq + pl->q_per_block - 1) / pl->q_per_block) * ((s.Lk + p.block_n - 1) / p.block_n));
  }
  if (p.splits > 1) {
    const size_t rows = static_cast<size_t>(s.B) * s.Hq * s.Lq;
    pl->off_pout = off; off = align256(off + sizeof(float) * p.splits * rows * s.d);
    pl->off_plse = off; off = align256(off + sizeof(float) * p.splits * rows);
  }
  p.workspace_bytes = off;
  p.topk_list_cap = pl->list_cap;
  return MI_ATTN_OK;
}

}  // namespace

extern "C" {

int attn_abi_version(void) { return MI_ATTN_ABI_VERSION; }

const char* attn_last_error(void) { return g_err.c_str(); }

void attn_set_debug(int no_skip, int force_path, int force_splits) {
  g_no_skip = no_skip ? 1 : 0;
  g_force_path = (force_path >= 0 && force_path <= 2) ? force_path : -1;
  g_force_splits = force_splits > 0 ? force_splits : 0;
}

int attn_fwd_plan(int B, int Hq, int Hkv, int Lq, int Lk, int d, int mask_kind, int window_left, int keep_k,
                  int dtype, attn_plan_t* plan) {
  g_err.clear();
  if (plan == nullptr) return fail(MI_ATTN_EINVAL, "plan must not be NULL");
  const Shape s{B, Hq, Hkv, Lq, Lk, d, mask_kind, window_left, keep_k, dtype};
  int rc = validate(s);
  if (rc != MI_ATTN_OK) return rc;
  Plan pl;
  rc = make_plan(s, &pl);
  if (rc != MI_ATTN_OK) return rc;
  *plan = pl.pub;
  return MI_ATTN_OK;
}

}  // extern "C"

namespace mi_attn {

// ---- per-device workspace arena. A call's temporary memory is one block per device, kept
// and reused by later calls (grown when a call needs more) instead of a stream-ordered
// allocation per call: on this runtime hipMallocAsync / hipFreeAsync wait for the device,
// which left the device idle ~16 us between back-to-back c5 calls. Calls on one stream use
// the block in stream order; a call on another stream first makes its stream wait (on the
// device) for the event recorded after the previous call's work. A host thread holds the
// arena's mutex while its call enqueues, so concurrent callers take turns. The block is
// held until the process ends.
constexpr int kArenaDevices = 64;
struct Arena {
  std::mutex mu;
  char* ptr = nullptr;
  size_t cap = 0;
  hipStream_t last = nullptr;  // stream of the previous call that used the block
  hipEvent_t done = nullptr;   // recorded on `last` after that call's work
  bool recorded = false;
};
Arena g_arena[kArenaDevices];

// RAII: acquire() locks the device's arena and returns a block of at least `bytes` that
// no earlier call's work still uses on another stream; the destructor records the event
// after this call's work and unlocks.
class ArenaLease {
 public:
  ~ArenaLease() {
    if (a_ == nullptr) return;
    if (hipEventRecord(a_->done, s_) == hipSuccess) {
      a_->last = s_;
      a_->recorded = true;
    } else {
      // nothing to wait for later: make sure the work enqueued so far has finished
      (void)hipStreamSynchronize(s_);
      a_->recorded = false;
    }
    a_->mu.unlock();
  }
  hipError_t acquire(size_t bytes, hipStream_t s, char** out) {
    *out = nullptr;
    if (bytes == 0) return hipSuccess;
    int cur = 0, dev = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    dev = cur;
    if (s != nullptr && (e = hipStreamGetDevice(s, &dev)) != hipSuccess) return e;
    if (dev < 0 || dev >= kArenaDevices) return hipErrorInvalidDevice;
    Arena& a = g_arena[dev];
    a.mu.lock();
    const bool switch_dev = dev != cur;
    if (switch_dev && (e = hipSetDevice(dev)) != hipSuccess) {
      a.mu.unlock();
      return e;
    }
    if (a.done == nullptr) e = hipEventCreateWithFlags(&a.done, hipEventDisableTiming);
    if (e == hipSuccess && a.cap < bytes) {
      // grow: the old block may still be in use by queued work
      if (a.ptr != nullptr) {
        if (a.recorded) e = hipEventSynchronize(a.done);
        if (e == hipSuccess) e = hipFree(a.ptr);
        a.ptr = nullptr;
        a.cap = 0;
        a.recorded = false;
      }
      size_t want = size_t{1} << 20;
      while (want < bytes) want <<= 1;
      if (e == hipSuccess) e = hipMalloc(reinterpret_cast<void**>(&a.ptr), want);
      if (e == hipSuccess) a.cap = want;
      else a.ptr = nullptr;
    }
    if (e == hipSuccess && a.recorded && a.last != s) e = hipStreamWaitEvent(s, a.done, 0);
    if (switch_dev) (void)hipSetDevice(cur);
    if (e != hipSuccess) {
      a.mu.unlock();
      return e;
    }
    a_ = &a;
    s_ = s;
    *out = a.ptr;
    return hipSuccess;
  }

 private:
  Arena* a_ = nullptr;
  hipStream_t s_ = nullptr;
};

}  // namespace mi_attn

// Fixed scratch of attn_fwd_noalloc (see scratch_for below).
static __device__ __align__(256) unsigned char scratch[MI_ATTN_NOALLOC_MAX_WORKSPACE];

namespace {

// The forward call behind attn_fwd_ex / attn_fwd / attn_fwd_noalloc. Temporary device
// memory comes from a stream-ordered allocation when fixed_ws is null, else from fixed_ws
// (fixed_cap bytes), and the call is refused when its plan needs more.
struct DumpReq {
  float* buf;
  int b, kv_head, query_block, tile;
};

int fwd_impl(const attn_fwd_args_t* a, void* stream, char* fixed_ws, size_t fixed_cap,
             const DumpReq* dump = nullptr) {
  if (a == nullptr) return fail(MI_ATTN_EINVAL, "args must not be NULL");
  Shape s{a->B, a->Hq, a->Hkv, a->Lq, a->Lk, a->d, a->mask_kind, a->window_left, a->keep_k, a->dtype};
  int rc = validate(s);
  if (rc != MI_ATTN_OK) return rc;
  if (a->q == nullptr || a->k == nullptr || a->v == nullptr || a->out == nullptr)
    return fail(MI_ATTN_EINVAL, "q, k, v and out must not be NULL");
  if (!std::isfinite(a->scale)) return fail(MI_ATTN_EINVAL, "scale must be finite");
  if (a->mask_kind == MI_ATTN_MASK_DENSE && a->mask == nullptr)
    return fail(MI_ATTN_EINVAL, "mask_kind DENSE needs a mask pointer");
  if (a->mask_kind == MI_ATTN_MASK_TOPK && a->zero_hold == nullptr)
    return fail(MI_ATTN_EINVAL, "mask_kind TOPK needs a zero_hold pointer");
  if (a->topk_causal != 0 && a->topk_causal != 1) return fail(MI_ATTN_EINVAL, "topk_causal must be 0 or 1");
  if (!std::isfinite(a->softcap) || a->softcap < 0.f) return fail(MI_ATTN_EINVAL, "softcap must be finite and >= 0");
  // strides: non-negative; out never written twice; 16-byte rows for the vector loads
  const int64_t* st[4] = {a->q_stride, a->k_stride, a->v_stride, a->out_stride};
  const char* nm[4] = {"q", "k", "v", "out"};
  const int hs[4] = {a->Hq, a->Hkv, a->Hkv, a->Hq};
  const int ls[4] = {a->Lq, a->Lk, a->Lk, a->Lq};
  const void* ptr[4] = {a->q, a->k, a->v, a->out};
  const int es = a->dtype == MI_ATTN_F32 ? 4 : 2;
  for (int t = 0; t < 4; ++t) {
    for (int x = 0; x < 3; ++x)
      if (st[t][x] < 0) return fail(MI_ATTN_EINVAL, "%s stride %d is negative", nm[t], x);
    if (t == 3 && ((a->B > 1 && st[t][0] == 0) || (a->Hq > 1 && st[t][1] == 0) || (a->Lq > 1 && st[t][2] == 0)))
      return fail(MI_ATTN_EINVAL, "out strides must be positive over dimensions longer than 1");
    if (a->dtype != MI_ATTN_F32) {
      if (reinterpret_cast<uintptr_t>(ptr[t]) % 16 != 0 || st[t][0] % 8 || st[t][1] % 8 || st[t][2] % 8)
        return fail(MI_ATTN_EINVAL, "%s must be 16-byte aligned with strides in multiples of 8 elements", nm[t]);
      if (t == 1 || t == 2) {
        // one (batch, KV head) slice is addressed with 32-bit byte offsets
        const double span = (static_cast<double>(ls[t]) * st[t][2] + a->d) * es;
        if (span > 2147483647.0)
          return fail(MI_ATTN_EUNSUPPORTED, "%s rows too far apart for 32-bit offsets (Lk * row stride)", nm[t]);
      }
    }
    (void)hs;
  }
  for (int x = 0; x < 4; ++x)
    if (a->mask_stride[x] < 0) return fail(MI_ATTN_EINVAL, "mask stride %d is negative", x);
  const bool use_mask = a->mask_kind == MI_ATTN_MASK_DENSE || (a->mask_kind == MI_ATTN_MASK_TOPK && a->mask != nullptr);
  if (a->mask_kind == MI_ATTN_MASK_DENSE) {
    s.flag_b = (a->B > 1 && a->mask_stride[0] != 0) ? a->B : 1;
    s.flag_g = (a->Hq > 1 && a->mask_stride[1] != 0) ? a->Hkv : 1;
  }
  Plan pl;
  rc = make_plan(s, &pl);
  if (rc != MI_ATTN_OK) return rc;
  if (dump != nullptr) {
    if (pl.pub.path != 1)
      return fail(MI_ATTN_EUNSUPPORTED, "the one-tile dump runs on the MFMA prefill path only (this call takes path %d)",
                  pl.pub.path);
    if (pl.pub.block_n != 64)
      return fail(MI_ATTN_EUNSUPPORTED, "the one-tile dump covers 64-key tiles (this call takes %d-key tiles)",
                  pl.pub.block_n);
    if (a->alibi_slopes != nullptr || a->softcap > 0.f ||
        (a->mask_kind == MI_ATTN_MASK_TOPK && a->mask != nullptr))
      return fail(MI_ATTN_EUNSUPPORTED,
                  "the one-tile dump covers calls without score modifiers (ALiBi, softcap, a mask added to top-k)");
    const int nqb = (a->Lq + pl.q_per_block - 1) / pl.q_per_block;
    const int ntiles = pl.list_cap > 0 ? pl.list_cap / 64 : (a->Lk + pl.pub.block_n - 1) / pl.pub.block_n;
    if (dump->buf == nullptr || dump->b < 0 || dump->b >= a->B || dump->kv_head < 0 || dump->kv_head >= a->Hkv ||
        dump->query_block < 0 || dump->query_block >= nqb || dump->tile < 0 || dump->tile >= ntiles)
      return fail(MI_ATTN_EINVAL, "dump: need a buffer, b < %d, kv_head < %d, query_block < %d and tile < %d", a->B,
                  a->Hkv, nqb, ntiles);
  }

  hipStream_t st_ = static_cast<hipStream_t>(stream);
  char* ws = nullptr;
  ArenaLease lease;
  if (fixed_ws != nullptr) {
    if (pl.pub.workspace_bytes > fixed_cap)
      return fail(MI_ATTN_EUNSUPPORTED, "the call needs %zu bytes of temporary memory, above the %zu-byte fixed scratch",
                  pl.pub.workspace_bytes, fixed_cap);
    ws = fixed_ws;
  } else if (pl.pub.workspace_bytes > 0) {
    const hipError_t e = lease.acquire(pl.pub.workspace_bytes, st_, &ws);
    if (e != hipSuccess) return hip_fail(e, "workspace");
  }

  const int B = a->B, Hq = a->Hq, Hkv = a->Hkv, Lq = a->Lq, Lk = a->Lk;
  AttnParams p{};
  p.q = a->q; p.k = a->k; p.v = a->v; p.out = a->out; p.lse = a->lse;
  p.mask = use_mask ? a->mask : nullptr;
  p.zero_hold = a->zero_hold;
  p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.Lq = Lq; p.Lk = Lk; p.d = a->d; p.G = Hq / Hkv;
  p.scale = a->scale; p.mask_kind = a->mask_kind; p.window_left = a->window_left; p.keep_k = a->keep_k;
  for (int x = 0; x < 3; ++x) {
    p.qs[x] = a->q_stride[x]; p.ks[x] = a->k_stride[x]; p.vs[x] = a->v_stride[x]; p.os[x] = a->out_stride[x];
  }
  for (int x = 0; x < 4; ++x) p.ms[x] = a->mask_stride[x];
  p.flag_b = s.flag_b;
  p.flag_g = s.flag_g;
  p.alibi = a->alibi_slopes;
  p.softcap = a->softcap;
  p.topk_causal = a->mask_kind == MI_ATTN_MASK_TOPK ? a->topk_causal : 1;
  p.no_skip = g_no_skip;
  p.splits = pl.pub.splits;
  {
    // split boundaries fall on tiles of the key range (or of the kept-key list)
    const int tiles = pl.list_cap > 0 ? pl.list_cap / 64 : (Lk + pl.pub.block_n - 1) / pl.pub.block_n;
    const int unit = pl.list_cap > 0 ? 64 : pl.pub.block_n;
    p.keys_per_split = ((tiles + pl.pub.splits - 1) / pl.pub.splits) * unit;
  }
  p.block_n = pl.pub.block_n;
  p.q_per_block = pl.q_per_block;
  if (dump != nullptr) {
    p.dump = dump->buf;
    p.dump_bg = dump->b * Hkv + dump->kv_head;
    p.dump_qb = dump->query_block;
    p.dump_tile = dump->tile;
  }

  hipError_t e = hipSuccess;
  const char* what = "";
  if (a->mask_kind == MI_ATTN_MASK_TOPK) {
    int32_t* rank = reinterpret_cast<int32_t*>(ws + pl.off_rank);
    int32_t* tau = reinterpret_cast<int32_t*>(ws + pl.off_tau);
    int32_t* tmin = reinterpret_cast<int32_t*>(ws + pl.off_tmin);
    what = "top-k selection";
    // gathered tiles: the kept-key lists, written by the causal threshold kernel itself
    // or by a list kernel after the constant thresholds of the non-causal selection
    TopkListArgs la{};
    if (pl.list_cap > 0) {
      la.zh = a->zero_hold;
      la.q_per_block = pl.q_per_block;
      la.nqb = (Lq + pl.q_per_block - 1) / pl.q_per_block;
      la.cap = pl.list_cap;
      la.lidx = reinterpret_cast<int32_t*>(ws + pl.off_lidx);
      la.lrank = reinterpret_cast<int32_t*>(ws + pl.off_lrank);
      la.lzh = reinterpret_cast<float*>(ws + pl.off_lzh);
      la.lcount = reinterpret_cast<int32_t*>(ws + pl.off_lcnt);
    }
    const bool fused_lists = pl.list_cap > 0 && p.topk_causal;
    e = launch_topk(a->zero_hold, B * Hkv, Lq, Lk, a->keep_k, p.topk_causal, rank, tau, nullptr, tmin, pl.pub.block_n,
                    st_, topk_sort_ws_bytes(B * Hkv, Lk) > 0 ? ws + pl.off_sort : nullptr, fused_lists ? &la : nullptr);
    p.rank = rank; p.tau = tau; p.tile_min_rank = tmin;
    if (e == hipSuccess && pl.list_cap > 0) {
      if (!fused_lists) {
        what = "top-k kept-key lists";
        e = launch_topk_lists(rank, tau, a->zero_hold, B * Hkv, Lq, Lk, pl.q_per_block, pl.list_cap, p.topk_causal,
                              la.lidx, la.lrank, la.lzh, la.lcount, st_);
      }
      p.list_idx = la.lidx; p.list_rank = la.lrank; p.list_zh = la.lzh; p.list_count = la.lcount;
      p.list_cap = pl.list_cap;
    }
  }
  if (e == hipSuccess && pl.pub.mask_summary) {
    uint8_t* flags = reinterpret_cast<uint8_t*>(ws + pl.off_flags);
    what = "dense-mask summary";
    e = launch_mask_summary(p, pl.pub.block_n, flags, st_);
    p.tile_live = flags;
  }
  if (e == hipSuccess) {
    if (pl.pub.splits > 1) {
      p.part_out = reinterpret_cast<float*>(ws + pl.off_pout);
      p.part_lse = reinterpret_cast<float*>(ws + pl.off_plse);
    }
    what = "attention kernel";
    e = (pl.pub.path == 0) ? launch_row_kernel(p, a->dtype, st_) : launch_half_path(pl.pub.path, p, a->dtype, st_);
  }
  if (e != hipSuccess) return hip_fail(e, what);
  return MI_ATTN_OK;
}

// attn_fwd's argument list as an argument block (contiguous layouts, the single [Lq, Lk]
// mask for the dense kind, causal top-k)
attn_fwd_args_t contiguous_args(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Hq,
                                int Hkv, int Lq, int Lk, int d, float scale, int mask_kind, int window_left,
                                const float* mask, const float* zero_hold, int keep_k, int dtype) {
  attn_fwd_args_t a{};
  a.q = q; a.k = k; a.v = v; a.out = out; a.lse = lse;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Lq = Lq; a.Lk = Lk; a.d = d;
  const int64_t qh = static_cast<int64_t>(Lq) * d, kh = static_cast<int64_t>(Lk) * d;
  a.q_stride[0] = a.out_stride[0] = qh * Hq;
  a.q_stride[1] = a.out_stride[1] = qh;
  a.q_stride[2] = a.out_stride[2] = d;
  a.k_stride[0] = a.v_stride[0] = kh * Hkv;
  a.k_stride[1] = a.v_stride[1] = kh;
  a.k_stride[2] = a.v_stride[2] = d;
  a.scale = scale; a.mask_kind = mask_kind; a.window_left = window_left;
  a.mask = mask_kind == MI_ATTN_MASK_DENSE ? mask : nullptr;
  a.mask_stride[2] = Lk;
  a.mask_stride[3] = 1;
  a.zero_hold = zero_hold; a.keep_k = keep_k; a.topk_causal = 1;
  a.dtype = dtype;
  return a;
}

// ---- fixed scratch for attn_fwd_noalloc: one copy of this array per GPU, for the life of
// the process. Host code never passes the array's name to a kernel (on the host it is only
// a stand-in for the symbol); it uses the device address hipGetSymbolAddress returns, looked
// up once per device with that device current and kept here.
constexpr size_t kScratchBytes = MI_ATTN_NOALLOC_MAX_WORKSPACE;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// device address of `scratch` on the device `stream` belongs to (the current device for
// the null stream)
int scratch_for(hipStream_t stream, char** out) {
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  int dev = cur;
  if (stream != nullptr) {
    e = hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess) return hip_fail(e, "hipStreamGetDevice");
  }
  if (dev < 0 || dev >= kMaxDevices) return fail(MI_ATTN_EUNSUPPORTED, "device %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return hip_fail(e, "hipSetDevice");
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (dev != cur) (void)hipSetDevice(cur);
    if (e != hipSuccess || ptr == nullptr) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = ptr;
  }
  *out = static_cast<char*>(g_scratch_ptr[dev]);
  return MI_ATTN_OK;
}

}  // namespace

extern "C" {

int attn_fwd_ex(const attn_fwd_args_t* a, void* stream) {
  g_err.clear();
  return fwd_impl(a, stream, nullptr, 0);
}

int attn_fwd_dump(const attn_fwd_args_t* a, int b, int kv_head, int query_block, int tile, float* dump,
                  void* stream) {
  g_err.clear();
  const DumpReq req{dump, b, kv_head, query_block, tile};
  return fwd_impl(a, stream, nullptr, 0, &req);
}

int attn_fwd_noalloc(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Hq, int Hkv,
                     int Lq, int Lk, int d, float scale, int mask_kind, int window_left, const float* mask,
                     const float* zero_hold, int keep_k, int dtype, void* stream) {
  g_err.clear();
  const attn_fwd_args_t a = contiguous_args(q, k, v, out, lse, B, Hq, Hkv, Lq, Lk, d, scale, mask_kind, window_left,
                                            mask, zero_hold, keep_k, dtype);
  // validate and plan first, so that a refused call touches no device state
  {
    Shape sh{B, Hq, Hkv, Lq, Lk, d, mask_kind, window_left, keep_k, dtype};
    int rc = validate(sh);
    if (rc != MI_ATTN_OK) return rc;
  }
  char* ws = nullptr;
  const int rc = scratch_for(static_cast<hipStream_t>(stream), &ws);
  if (rc != MI_ATTN_OK) return rc;
  return fwd_impl(&a, stream, ws, kScratchBytes);
}

int attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Hq, int Hkv, int Lq,
             int Lk, int d, float scale, int mask_kind, int window_left, const float* mask, const float* zero_hold,
             int keep_k, int dtype, void* stream) {
  g_err.clear();
  const attn_fwd_args_t a = contiguous_args(q, k, v, out, lse, B, Hq, Hkv, Lq, Lk, d, scale, mask_kind, window_left,
                                            mask, zero_hold, keep_k, dtype);
  return fwd_impl(&a, stream, nullptr, 0);
}

int attn_bwd(const void* q, const void* k, const void* v, const void* out, const float* lse, const void* dout,
             void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Lq, int Lk, int d, float scale,
             int mask_kind, int window_left, const float* mask, const float* zero_hold, int keep_k, int dtype,
             void* stream) {
  g_err.clear();
  const Shape s{B, Hq, Hkv, Lq, Lk, d, mask_kind, window_left, keep_k, dtype};
  int rc = validate(s);
  if (rc != MI_ATTN_OK) return rc;
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr || lse == nullptr || dout == nullptr ||
      dq == nullptr || dk == nullptr || dv == nullptr)
    return fail(MI_ATTN_EINVAL, "q, k, v, out, lse, dout, dq, dk and dv must not be NULL");
  if (!std::isfinite(scale)) return fail(MI_ATTN_EINVAL, "scale must be finite");
  if (mask_kind == MI_ATTN_MASK_DENSE && mask == nullptr)
    return fail(MI_ATTN_EINVAL, "mask_kind DENSE needs a mask pointer");
  if (mask_kind == MI_ATTN_MASK_TOPK && zero_hold == nullptr)
    return fail(MI_ATTN_EINVAL, "mask_kind TOPK needs a zero_hold pointer");
  if (dtype == MI_ATTN_F32) return fail(MI_ATTN_EUNSUPPORTED, "attn_bwd takes fp16/bf16 inputs");
  const int G = Hq / Hkv;
  if (G > 128) return fail(MI_ATTN_EUNSUPPORTED, "attn_bwd supports at most 128 query heads per KV head");
  if (static_cast<double>(Hq) * Lq * d * 2 > 2147483647.0)
    return fail(MI_ATTN_EUNSUPPORTED, "Hq * Lq * d * 2 must stay below 2^31 bytes");
  if (static_cast<double>(B) * Hq * Lq * 12 > 2147483647.0)
    return fail(MI_ATTN_EUNSUPPORTED, "B * Hq * Lq must stay below 2^31 / 12 query rows");
  // the kernels move 16-byte vectors of the tensors and 4-byte values of lse
  const void* vec[8] = {q, k, v, out, dout, dq, dk, dv};
  for (const void* x : vec)
    if (reinterpret_cast<uintptr_t>(x) % 16 != 0)
      return fail(MI_ATTN_EINVAL, "q, k, v, out, dout, dq, dk and dv must be 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(lse) % 4 != 0) return fail(MI_ATTN_EINVAL, "lse must be 4-byte aligned");

  const long rows = static_cast<long>(B) * Hq * Lq;
  const long bh = static_cast<long>(B) * Hkv;
  size_t off = 0;
  const size_t off_side = off; off = align256(off + 3 * sizeof(float) * rows);
  size_t off_rank = 0, off_tau = 0;
  size_t off_sort = 0;
  if (mask_kind == MI_ATTN_MASK_TOPK) {
    off_rank = off; off = align256(off + sizeof(int32_t) * bh * Lk);
    off_tau = off;  off = align256(off + sizeof(int32_t) * bh * Lq);
    off_sort = off; off = align256(off + topk_sort_ws_bytes(static_cast<int>(bh), Lk));
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = nullptr;
  ArenaLease lease;
  hipError_t e = lease.acquire(off, st, &ws);
  if (e != hipSuccess) return hip_fail(e, "workspace");

  AttnParams p{};
  p.q = q; p.k = k; p.v = v; p.out = const_cast<void*>(out); p.lse = const_cast<float*>(lse);
  p.dout = dout; p.dq = dq; p.dk = dk; p.dv = dv;
  p.bwd_side = reinterpret_cast<float*>(ws + off_side);
  p.mask = mask_kind == MI_ATTN_MASK_DENSE ? mask : nullptr;
  p.ms[2] = Lk;
  p.ms[3] = 1;
  p.zero_hold = zero_hold;
  p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.Lq = Lq; p.Lk = Lk; p.d = d; p.G = G;
  p.scale = scale; p.mask_kind = mask_kind; p.window_left = window_left; p.keep_k = keep_k;
  p.topk_causal = 1;
  p.no_skip = g_no_skip;
  p.splits = 1;
  p.q_per_block = 128 / G;
  const char* what = "attention backward kernels";
  if (mask_kind == MI_ATTN_MASK_TOPK) {
    int32_t* rank = reinterpret_cast<int32_t*>(ws + off_rank);
    int32_t* tau = reinterpret_cast<int32_t*>(ws + off_tau);
    what = "top-k selection";
    e = launch_topk(zero_hold, B * Hkv, Lq, Lk, keep_k, 1, rank, tau, nullptr, nullptr, 0, st, ws + off_sort);
    p.rank = rank;
    p.tau = tau;
    if (e == hipSuccess) what = "attention backward kernels";
  }
  if (e == hipSuccess) e = launch_backward(p, dtype, st);
  if (e != hipSuccess) return hip_fail(e, what);
  return MI_ATTN_OK;
}

int attn_fwd_varlen(const void* q, const void* k, const void* v, void* out, float* lse,
                    const int32_t* cu_seqlens_q, int max_seqlen_q, const int32_t* cu_seqlens_k, int max_seqlen_k,
                    int num_seqs, int total_q, int Hq, int Hkv, int d, float scale, int mask_kind, int window_left,
                    const int32_t* block_table, int max_pages, int page_size, int kv_rows, const void* k_new,
                    const void* v_new, const float* alibi_slopes, float softcap, int dtype, void* stream) {
  g_err.clear();
  if (num_seqs < 0 || total_q < 0 || max_seqlen_q < 0 || max_seqlen_k < 0)
    return fail(MI_ATTN_EINVAL, "num_seqs, total_q and max_seqlen_q/k must be >= 0");
  if (Hq <= 0 || Hkv <= 0 || d <= 0) return fail(MI_ATTN_EINVAL, "Hq, Hkv and d must be positive");
  if (Hq % Hkv != 0) return fail(MI_ATTN_EINVAL, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
  if (mask_kind < MI_ATTN_MASK_NONE || mask_kind > MI_ATTN_MASK_TOPK)
    return fail(MI_ATTN_EINVAL, "unknown mask_kind %d", mask_kind);
  if (dtype < MI_ATTN_F32 || dtype > MI_ATTN_BF16) return fail(MI_ATTN_EINVAL, "unknown dtype %d", dtype);
  if (mask_kind == MI_ATTN_MASK_WINDOW && window_left < 0)
    return fail(MI_ATTN_EINVAL, "window_left must be >= 0 (got %d)", window_left);
  if (!std::isfinite(scale)) return fail(MI_ATTN_EINVAL, "scale must be finite");
  if ((k_new == nullptr) != (v_new == nullptr)) return fail(MI_ATTN_EINVAL, "give both k_new and v_new, or neither");
  if (!std::isfinite(softcap) || softcap < 0.f) return fail(MI_ATTN_EINVAL, "softcap must be finite and >= 0");
  if (kv_rows < 1) return fail(MI_ATTN_EINVAL, "kv_rows must be >= 1 (got %d)", kv_rows);
  int page_shift = 0;
  if (block_table != nullptr) {
    if (page_size < 1 || (page_size & (page_size - 1)) != 0)
      return fail(MI_ATTN_EINVAL, "page_size must be a power of two (got %d)", page_size);
    if (max_pages < 1) return fail(MI_ATTN_EINVAL, "max_pages must be >= 1 (got %d)", max_pages);
    while ((1 << page_shift) < page_size) ++page_shift;
    if (static_cast<double>(kv_rows) * page_size > 2147483647.0)
      return fail(MI_ATTN_EUNSUPPORTED, "kv_rows * page_size must stay below 2^31 keys");
    if (static_cast<double>(max_pages) * page_size > 1073741824.0)
      return fail(MI_ATTN_EUNSUPPORTED, "max_pages * page_size must stay at or below 2^30 keys");
  } else if (kv_rows > (1 << 30)) {
    return fail(MI_ATTN_EUNSUPPORTED, "packed K/V must have at most 2^30 rows");
  }
  if (total_q > (1 << 30)) return fail(MI_ATTN_EUNSUPPORTED, "total_q must be at most 2^30");
  if (dtype == MI_ATTN_F32) return fail(MI_ATTN_EUNSUPPORTED, "varlen attention takes fp16/bf16 inputs");
  if (d != 64 && d != 128) return fail(MI_ATTN_EUNSUPPORTED, "head dim must be 64 or 128 (got %d)", d);
  if (mask_kind == MI_ATTN_MASK_DENSE || mask_kind == MI_ATTN_MASK_TOPK)
    return fail(MI_ATTN_EUNSUPPORTED, "varlen attention takes the none, causal and window masks");
  const int G = Hq / Hkv;
  if (G > prefill_block_m())
    return fail(MI_ATTN_EUNSUPPORTED, "at most %d query heads per KV head", prefill_block_m());
  if (static_cast<double>(total_q) * Hq * d > 9.0e15) return fail(MI_ATTN_EINVAL, "tensor too large");
  if (total_q == 0 || num_seqs == 0) return MI_ATTN_OK;
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr || cu_seqlens_q == nullptr ||
      cu_seqlens_k == nullptr)
    return fail(MI_ATTN_EINVAL, "q, k, v, out, cu_seqlens_q and cu_seqlens_k must not be NULL");

  // work units: sum over sequences of ceil(Lq_s / qpb) <= (total_q + num_seqs * (qpb - 1)) / qpb
  // (a decode-type sequence is one unit, which that bound also covers)
  const int qpb = varlen_q_per_block(G);
  const long units_cap = (static_cast<long>(total_q) + static_cast<long>(num_seqs) * (qpb - 1)) / qpb;
  if (units_cap > 0x3fffffffL) return fail(MI_ATTN_EUNSUPPORTED, "too many work units (%ld)", units_cap);
  VarlenBuffers b{};
  b.units_cap = static_cast<int>(units_cap);
  b.target_items = varlen_target_items(Hkv);
  b.force_items = g_force_splits;
  b.items_cap = varlen_items_cap(b.units_cap, b.target_items, b.force_items);
  if (static_cast<long>(b.items_cap) * Hkv > 0x7fffffffL)
    return fail(MI_ATTN_EUNSUPPORTED, "too many workgroups (%ld items x %d KV heads)", static_cast<long>(b.items_cap),
                Hkv);
  const size_t ic = static_cast<size_t>(b.items_cap) * Hkv;
  size_t off = 0;
  const size_t off_units = off; off = align256(off + sizeof(int4) * b.units_cap);
  const size_t off_ip = off;    off = align256(off + sizeof(int4) * b.items_cap);
  const size_t off_id = off;    off = align256(off + sizeof(int4) * b.items_cap);
  const size_t off_cnt = off;   off = align256(off + sizeof(int32_t) * 3);
  const size_t off_ppo = off;   off = align256(off + sizeof(float) * ic * kVarlenPrefillRows * d);
  const size_t off_ppl = off;   off = align256(off + sizeof(float) * ic * kVarlenPrefillRows);
  const size_t off_pdo = off;   off = align256(off + sizeof(float) * ic * 32 * d);
  const size_t off_pdl = off;   off = align256(off + sizeof(float) * ic * 32);
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = nullptr;
  ArenaLease lease;
  hipError_t e = lease.acquire(off, st, &ws);
  if (e != hipSuccess) return hip_fail(e, "workspace");
  b.units = reinterpret_cast<int4*>(ws + off_units);
  b.items_p = reinterpret_cast<int4*>(ws + off_ip);
  b.items_d = reinterpret_cast<int4*>(ws + off_id);
  b.counts = reinterpret_cast<int32_t*>(ws + off_cnt);
  b.pp_out = reinterpret_cast<float*>(ws + off_ppo);
  b.pp_lse = reinterpret_cast<float*>(ws + off_ppl);
  b.pd_out = reinterpret_cast<float*>(ws + off_pdo);
  b.pd_lse = reinterpret_cast<float*>(ws + off_pdl);

  AttnParams p{};
  p.q = q; p.k = k; p.v = v; p.out = out; p.lse = lse;
  p.B = 1; p.Hq = Hq; p.Hkv = Hkv; p.Lq = 0; p.Lk = 0; p.d = d; p.G = G;
  p.scale = scale; p.mask_kind = mask_kind; p.window_left = window_left;
  p.alibi = alibi_slopes;
  p.softcap = softcap;
  p.no_skip = g_no_skip;
  p.splits = 1;
  p.block_n = 64;  // varlen instances take 64-key tiles
  p.q_per_block = qpb;
  p.cu_q = cu_seqlens_q; p.cu_k = cu_seqlens_k;
  p.block_table = block_table; p.k_new = k_new; p.v_new = v_new;
  p.num_seqs = num_seqs; p.total_q = total_q;
  p.max_pages = block_table != nullptr ? max_pages : 1;
  p.page_shift = page_shift;
  p.kv_rows = kv_rows;
  (void)max_seqlen_q;
  (void)max_seqlen_k;
  e = launch_varlen(p, dtype, b, st);
  if (e != hipSuccess) return hip_fail(e, "varlen attention kernels");
  return MI_ATTN_OK;
}

int dynamic_mask_topk(const float* zero_hold, int B, int H, int Lq, int Lk, int keep_k, int causal, int32_t* rank,
                      int32_t* tau, uint32_t* keep_bits, void* stream) {
  g_err.clear();
  if (B <= 0 || H <= 0 || Lq <= 0 || Lk <= 0)
    return fail(MI_ATTN_EINVAL, "sizes must be positive (B=%d H=%d Lq=%d Lk=%d)", B, H, Lq, Lk);
  if (keep_k < 1) return fail(MI_ATTN_EINVAL, "keep_k must be >= 1 (got %d)", keep_k);
  if (zero_hold == nullptr || rank == nullptr || tau == nullptr)
    return fail(MI_ATTN_EINVAL, "zero_hold, rank and tau must not be NULL");
  if (Lk > 65536) return fail(MI_ATTN_EUNSUPPORTED, "Lk must be <= 65536 (got %d)", Lk);
  if (static_cast<double>(B) * H * Lq * ((Lk + 31) / 32) > 2.0e9) return fail(MI_ATTN_EINVAL, "tensor too large");
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = nullptr;
  ArenaLease lease;
  hipError_t e = lease.acquire(topk_sort_ws_bytes(B * H, Lk), st, &ws);
  if (e != hipSuccess) return hip_fail(e, "workspace");
  e = launch_topk(zero_hold, B * H, Lq, Lk, keep_k, causal ? 1 : 0, rank, tau, keep_bits, nullptr, 0, st, ws);
  if (e != hipSuccess) return hip_fail(e, "dynamic_mask_topk");
  return MI_ATTN_OK;
}

}  // extern "C"
