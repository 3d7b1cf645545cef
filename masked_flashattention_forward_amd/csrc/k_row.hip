// Row kernel: one wavefront per query row, online softmax over 64-key chunks.
//
// This is the plain GPU form of the chunked forward (ExecuTorch pull request #10466 page,
// "Summary"): keys arrive in chunks, the row keeps a running max m and running sum l,
// and the unnormalised output is rescaled whenever m grows. It serves the fp32 inputs
// (computed in fp32 end to end) and, through the debug switch, cross-checks the MFMA
// kernels for fp16/bf16. Every mask kind is applied per element.
#include "common.hpp"

namespace mi_attn {

namespace {

constexpr int kRowsPerBlock = 4;  // one row per wavefront
constexpr int kMaxD = 256;

template <typename T>
__global__ __launch_bounds__(kRowsPerBlock * kWave) void row_kernel(AttnParams p) {
  __shared__ float sq[kRowsPerBlock][kMaxD];
  __shared__ float sp[kRowsPerBlock][kWave];
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const long row = static_cast<long>(blockIdx.x) * kRowsPerBlock + wave;
  const long nrows = static_cast<long>(p.B) * p.Hq * p.Lq;
  if (row >= nrows) return;  // whole wavefront leaves together; no block barrier below

  const int i = static_cast<int>(row % p.Lq);
  const int h = static_cast<int>((row / p.Lq) % p.Hq);
  const int b = static_cast<int>(row / (static_cast<long>(p.Lq) * p.Hq));
  const int g = h / p.G;
  const int d = p.d;
  const int pos = p.Lk - p.Lq + i;  // bottom-right aligned absolute position

  // strided rows (element strides {batch, head, row}; the head dimension is contiguous)
  const T* qrow = static_cast<const T*>(p.q) + b * p.qs[0] + h * p.qs[1] + i * p.qs[2];
  const T* kb = static_cast<const T*>(p.k) + b * p.ks[0] + g * p.ks[1];
  const T* vb = static_cast<const T*>(p.v) + b * p.vs[0] + g * p.vs[1];
  const long ksr = p.ks[2], vsr = p.vs[2];
  // dense mask row of (b, h, i) (also added to the kept keys of the top-k kind)
  const float* mrow = p.mask != nullptr ? p.mask + b * p.ms[0] + h * p.ms[1] + i * p.ms[2] : nullptr;
  const float slope = p.alibi != nullptr ? p.alibi[h] : 0.f;

  for (int c = lane; c < d; c += kWave) sq[wave][c] = to_f32(qrow[c]);
  __builtin_amdgcn_wave_barrier();

  int lo, hi;
  key_range(range_kind(p), p.window_left, p.Lk, pos, pos, &lo, &hi);
  if (p.no_skip) { lo = 0; hi = p.Lk; }

  const long bg = static_cast<long>(b) * p.Hkv + g;
  // clamped below Lk: ranks of real keys are 0 .. Lk-1
  const int32_t tau = (p.mask_kind == MI_ATTN_MASK_TOPK) ? min(p.tau[bg * p.Lq + i], p.Lk - 1) : 0;

  float m = kNegInf, l = 0.f;
  float acc[kMaxD / kWave];
#pragma unroll
  for (int t = 0; t < kMaxD / kWave; ++t) acc[t] = 0.f;

  for (int j0 = lo; j0 < hi; j0 += kWave) {
    const int j = j0 + lane;
    float s = kNegInf;
    if (j < hi) {
      const T* kr = kb + static_cast<long>(j) * ksr;
      float dot = 0.f;
      for (int c = 0; c < d; ++c) dot = fmaf(sq[wave][c], to_f32(kr[c]), dot);
      s = dot * p.scale;
      // score modifiers: softcap of the scaled score, then the ALiBi distance bias
      if (p.softcap > 0.f) s = p.softcap * tanhf(s / p.softcap);
      if (slope != 0.f) s -= slope * static_cast<float>(abs(pos - j));
      switch (p.mask_kind) {
        case MI_ATTN_MASK_CAUSAL:
          if (j > pos) s = kNegInf;
          break;
        case MI_ATTN_MASK_WINDOW:
          if (j > pos || j < pos - p.window_left) s = kNegInf;
          break;
        case MI_ATTN_MASK_DENSE:
          s += mrow[j * p.ms[3]];
          break;
        case MI_ATTN_MASK_TOPK:
          if ((!p.topk_causal || j <= pos) && p.rank[bg * p.Lk + j] <= tau)
            s += p.zero_hold[bg * p.Lk + j] + (mrow != nullptr ? mrow[j * p.ms[3]] : 0.f);
          else
            s = kNegInf;
          break;
        default:
          break;
      }
    }
    const float m_new = fmaxf(m, wave_max(s));
    // Guard: a chunk whose logits are all -inf leaves m_new = -inf. Subtracting a
    // finite stand-in keeps exp(-inf - ref) = 0 instead of exp(-inf + inf) = NaN.
    const float ref = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = expf(m - ref);
    const float pj = expf(s - ref);
    l = alpha * l + wave_sum(pj);
    m = m_new;
    sp[wave][lane] = pj;
    __builtin_amdgcn_wave_barrier();
    const int nk = (hi - j0) < kWave ? (hi - j0) : kWave;
#pragma unroll
    for (int t = 0; t < kMaxD / kWave; ++t) {
      const int c = lane + t * kWave;
      if (c < d) {
        float a = acc[t] * alpha;
        for (int jj = 0; jj < nk; ++jj)
          a = fmaf(sp[wave][jj], to_f32(vb[static_cast<long>(j0 + jj) * vsr + c]), a);
        acc[t] = a;
      }
    }
    __builtin_amdgcn_wave_barrier();
  }

  T* orow = static_cast<T*>(p.out) + b * p.os[0] + h * p.os[1] + i * p.os[2];
  const bool dead = (l == 0.f);
  const float inv = dead ? 0.f : 1.f / l;
#pragma unroll
  for (int t = 0; t < kMaxD / kWave; ++t) {
    const int c = lane + t * kWave;
    if (c < d) orow[c] = from_f32<T>(dead ? 0.f : acc[t] * inv);
  }
  if (p.lse != nullptr && lane == 0) p.lse[row] = dead ? kNegInf : (m + logf(l));
}

}  // namespace

hipError_t launch_row_kernel(const AttnParams& p, int dtype, hipStream_t s) {
  const long nrows = static_cast<long>(p.B) * p.Hq * p.Lq;
  const long blocks = (nrows + kRowsPerBlock - 1) / kRowsPerBlock;
  if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
  dim3 grid(static_cast<unsigned>(blocks)), block(kRowsPerBlock * kWave);
  switch (dtype) {
    case MI_ATTN_F32: hipLaunchKernelGGL(row_kernel<float>, grid, block, 0, s, p); break;
    case MI_ATTN_F16: hipLaunchKernelGGL(row_kernel<f16_t>, grid, block, 0, s, p); break;
    case MI_ATTN_BF16: hipLaunchKernelGGL(row_kernel<bf16_t>, grid, block, 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mi_attn
