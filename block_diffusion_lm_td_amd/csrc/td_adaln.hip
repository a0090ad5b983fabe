// adaLN-single time conditioning between two denoiser layers, on gfx950
// (news.chathome.org, "NVIDIA releases Nemotron-Labs-TwoTower ...", inference
// paragraph: the diffusion timestep modulates every layer through
// adaLN-single).  Read as PixArt-alpha's adaLN-single: each sequence's shared
// timestep vectors t_mod (shift, scale, gate) plus each layer's own table.
// For every token:
//   r = x + (t_mod_gate + tab_gate) * f           (layer l's gated residual)
//   h = r * rsqrt(mean(r^2) + eps) * w_norm * (1 + t_mod_scale + tab_scale)
//         + (t_mod_shift + tab_shift)             (layer l+1's modulated norm)
// r is stored in bf16 and h is taken from the stored r.
//
// adaln_rows: one 512-thread workgroup per sequence and run of R tokens.  Each
// thread owns 8 consecutive hidden units per pass of 4096 (one 16-byte bf16
// vector), and loads the modulation of its units (gate, w_norm * (1 + scale),
// shift) to registers once for the R tokens.  Per token: the next token's x
// and f are requested first (they stay in flight across the barrier, which
// waits on LDS only), then the gated sum, its bf16 rounding and store, the
// row's sum of squares reduced across the workgroup (one barrier,
// double-buffered slot), then h.  Bound by HBM: x, f, r and h are 8 bytes per
// element, the modulation rows are shared by a sequence's tokens.
#include <hip/hip_runtime.h>

#include "td_internal.h"

namespace td {
namespace {

typedef __bf16 bf16;

constexpr int kThreadsA = 512;                  // 8 waves
constexpr int kColsPerPass = kThreadsA * 8;

__device__ inline void unpack8(const uint4 v, float o[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    o[2 * q] = __uint_as_float(w[q] << 16);
    o[2 * q + 1] = __uint_as_float(w[q] & 0xffff0000u);
  }
}
__device__ inline uint32_t pack2(float a, float b) {
  const bf16 x = bf16(a), y = bf16(b);
  return uint32_t(__builtin_bit_cast(uint16_t, x)) | (uint32_t(__builtin_bit_cast(uint16_t, y)) << 16);
}
__device__ inline uint4 pack8(const float v[8]) {
  return make_uint4(pack2(v[0], v[1]), pack2(v[2], v[3]), pack2(v[4], v[5]), pack2(v[6], v[7]));
}
// 8 floats at p (32-byte aligned), or `fill` when p is null
__device__ inline void ld8f(const float *p, float o[8], float fill) {
  if (!p) {
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = fill;
    return;
  }
  const float4 a = *reinterpret_cast<const float4 *>(p), b = *reinterpret_cast<const float4 *>(p + 4);
  o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
  o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}

template <int PASSES>
__global__ __launch_bounds__(kThreadsA) void adaln_rows(
    const bf16 *x, const bf16 *f, const float *__restrict__ t_mod,   // x, f may be r_out or h
    const float *__restrict__ tab_gate, const float *__restrict__ tab_shift,
    const float *__restrict__ tab_scale, const float *__restrict__ w_norm, bf16 *r_out, bf16 *h,
    int S, int H, int R, float eps) {
  __shared__ float s_red[2][kThreadsA / 64];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int runs = (S + R - 1) / R;
  // workgroups are dealt to the 8 XCDs in turn: within each window of 8
  // sequences, XCD x takes all runs of the window's sequence x, so that the
  // sequence's timestep rows are fetched into one L2 only
  const unsigned win = 8u * unsigned(runs), bid = blockIdx.x;
  const unsigned lwg = bid >= gridDim.x / win * win
                           ? bid
                           : bid / win * win + unsigned(runs) * (bid & 7u) + (bid >> 3) % unsigned(runs);
  const int b = int(lwg / unsigned(runs));
  const int s0 = (int(lwg) - b * runs) * R, s1 = min(S, s0 + R);
  const float *tm = t_mod + int64_t(b) * 3 * H;

  // this thread's units: 8 * (tid + 256 k), k < PASSES (past H: unused)
  float gt[PASSES][8], sc[PASSES][8], sh[PASSES][8];
#pragma unroll
  for (int k = 0; k < PASSES; ++k) {
    const int col = 8 * (tid + kThreadsA * k);
    if (col >= H) continue;
    float t[8], u[8];
    ld8f(tm + col, sh[k], 0.f);                    // t_mod row 0: shift
    ld8f(tab_shift ? tab_shift + col : nullptr, t, 0.f);
    ld8f(tm + H + col, sc[k], 0.f);                // row 1: scale
    ld8f(tab_scale ? tab_scale + col : nullptr, u, 0.f);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      sh[k][i] += t[i];
      sc[k][i] = 1.f + (sc[k][i] + u[i]);
    }
    ld8f(w_norm ? w_norm + col : nullptr, t, 1.f);
#pragma unroll
    for (int i = 0; i < 8; ++i) sc[k][i] *= t[i];   // w_norm * (1 + scale)
    if (f) {
      ld8f(tm + 2 * H + col, gt[k], 0.f);          // row 2: gate
      ld8f(tab_gate ? tab_gate + col : nullptr, t, 0.f);
#pragma unroll
      for (int i = 0; i < 8; ++i) gt[k][i] += t[i];
    }
  }

  const float inv_h = 1.f / float(H);
  uint4 xq[PASSES], fq[PASSES];
  {
    const int64_t row = (int64_t(b) * S + s0) * H;
#pragma unroll
    for (int k = 0; k < PASSES; ++k) {
      const int col = 8 * (tid + kThreadsA * k);
      if (col >= H) continue;
      xq[k] = *reinterpret_cast<const uint4 *>(x + row + col);
      if (f) fq[k] = *reinterpret_cast<const uint4 *>(f + row + col);
    }
  }
  for (int s = s0; s < s1; ++s) {
    const int64_t row = (int64_t(b) * S + s) * H;
    uint4 rv[PASSES], fc[PASSES];
#pragma unroll
    for (int k = 0; k < PASSES; ++k) { rv[k] = xq[k]; fc[k] = fq[k]; }
    if (s + 1 < s1) {
#pragma unroll
      for (int k = 0; k < PASSES; ++k) {
        const int col = 8 * (tid + kThreadsA * k);
        if (col >= H) continue;
        xq[k] = *reinterpret_cast<const uint4 *>(x + row + H + col);
        if (f) fq[k] = *reinterpret_cast<const uint4 *>(f + row + H + col);
      }
    }
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < PASSES; ++k) {
      const int col = 8 * (tid + kThreadsA * k);
      if (col >= H) continue;
      if (f) {
        float xv[8], fv[8];
        unpack8(rv[k], xv);
        unpack8(fc[k], fv);
#pragma unroll
        for (int i = 0; i < 8; ++i) xv[i] = __builtin_fmaf(gt[k][i], fv[i], xv[i]);
        rv[k] = pack8(xv);
        *reinterpret_cast<uint4 *>(r_out + row + col) = rv[k];
      }
      float rr[8];
      unpack8(rv[k], rr);                          // the stored (rounded) r
#pragma unroll
      for (int i = 0; i < 8; ++i) ss = __builtin_fmaf(rr[i], rr[i], ss);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
    if (lane == 0) s_red[s & 1][wv] = ss;
    __syncthreads();                               // slot s&1 is next written two tokens on
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < kThreadsA / 64; ++w) tot += s_red[s & 1][w];
    const float rinv = rsqrtf(tot * inv_h + eps);
#pragma unroll
    for (int k = 0; k < PASSES; ++k) {
      const int col = 8 * (tid + kThreadsA * k);
      if (col >= H) continue;
      float rr[8];
      unpack8(rv[k], rr);
#pragma unroll
      for (int i = 0; i < 8; ++i) rr[i] = __builtin_fmaf(rr[i] * rinv, sc[k][i], sh[k][i]);
      *reinterpret_cast<uint4 *>(h + row + col) = pack8(rr);
    }
  }
}

}  // namespace

int launch_adaln(const td_adaln_args *a, void *stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  // tokens per workgroup: the most that still leaves a workgroup per CU (more
  // tokens amortise the modulation loads and pipeline the rows; at 64 x 16 x
  // 4096, 4 tokens take 11.4 us against 12.4 us for 2 and 14.0 us for 8)
  int R = 1;
  for (int r : {8, 4, 2})
    if (int64_t(a->B) * ((a->S + r - 1) / r) >= 256) {
      R = r;
      break;
    }
  const dim3 grid(unsigned(int64_t(a->B) * ((a->S + R - 1) / R))), block(kThreadsA);
  const int passes = (a->H + kColsPerPass - 1) / kColsPerPass;
#define TD_ADALN(PS)                                                                                \
  hipLaunchKernelGGL((adaln_rows<PS>), grid, block, 0, st, static_cast<const bf16 *>(a->x),        \
                     static_cast<const bf16 *>(a->f), a->t_mod, a->tab_gate, a->tab_shift,          \
                     a->tab_scale, a->w_norm, static_cast<bf16 *>(a->r_out), static_cast<bf16 *>(a->h), \
                     a->S, a->H, R, a->eps)
  if (passes <= 1) TD_ADALN(1);
  else if (passes <= 2) TD_ADALN(2);                // H <= 8192
  else return TD_ERR_UNSUPPORTED;
#undef TD_ADALN
  return hipGetLastError() == hipSuccess ? TD_OK : TD_ERR_HIP;
}

}  // namespace td
