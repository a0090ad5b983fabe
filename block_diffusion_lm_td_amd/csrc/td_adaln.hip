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
// vector).  At the start it requests, in the order they are needed, the
// first token's x and f, the modulation of its units (gate, w_norm, scale,
// shift: once for the R tokens), then the other tokens' x and f, so the whole
// run is in flight at once and each token waits on its own rows only.  Per
// token: the gated sum, its bf16 rounding and store, the row's sum of squares
// reduced across the workgroup (one barrier, double-buffered slot), then h.
// Bound by HBM: x, f, r and h are 8 bytes per element, streamed with the
// non-temporal hint; the modulation rows are shared by a sequence's tokens.
#include <hip/hip_runtime.h>

#include "td_internal.h"

namespace td {
namespace {

typedef __bf16 bf16;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// x, f, r and h are each touched once per call: their rows are streamed with
// the non-temporal hint, so they do not displace the modulation rows that a
// sequence's workgroups share in L2
__device__ inline uint4 ld_stream(const void *p) {
  const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
  return make_uint4(w.x, w.y, w.z, w.w);
}
__device__ inline void st_stream(void *p, uint4 v) {
  const u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4 *>(p));
}

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
// stands in for an absent [H] table row (zero-initialised device memory), so
// that every load is unconditional and the waits on them can be counted
__device__ float kZeroRow[8192];

// 8 floats at p (32-byte aligned)
__device__ inline void ld8f(const float *p, float o[8]) {
  const float4 a = *reinterpret_cast<const float4 *>(p), b = *reinterpret_cast<const float4 *>(p + 4);
  o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
  o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}

template <int PASSES, int RT, bool GATED>
__global__ __launch_bounds__(kThreadsA) void adaln_rows(
    const bf16 *x, const bf16 *f, const float *t_mod,   // x, f may be r_out or h
    const float *tab_gate, const float *tab_shift, const float *tab_scale, const float *w_norm,
    bf16 *r_out, bf16 *h,
    int S, int H, float eps) {
  __shared__ float s_red[2][kThreadsA / 64];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int runs = (S + RT - 1) / RT;
  // workgroups are dealt to the 8 XCDs in turn: within each window of 8
  // sequences, XCD x takes all runs of the window's sequence x, so that the
  // sequence's timestep rows are fetched into one L2 only
  const unsigned win = 8u * unsigned(runs), bid = blockIdx.x;
  const unsigned lwg = bid >= gridDim.x / win * win
                           ? bid
                           : bid / win * win + unsigned(runs) * (bid & 7u) + (bid >> 3) % unsigned(runs);
  const int b = int(lwg / unsigned(runs));
  const int s0 = (int(lwg) - b * runs) * RT, s1 = min(S, s0 + RT);
  const float *tm = t_mod + int64_t(b) * 3 * H;
  const float *tg = tab_gate ? tab_gate : kZeroRow, *ts = tab_shift ? tab_shift : kZeroRow;
  const float *tc = tab_scale ? tab_scale : kZeroRow, *wn = w_norm ? w_norm : kZeroRow;
  const float w_add = w_norm ? 0.f : 1.f;          // an absent weight is all ones

  // this thread's units: 8 * (tid + 512 k), k < PASSES.  Past H a lane loads
  // the last 8 units (in bounds) and stores nothing.
  int col[PASSES];
  bool live[PASSES];
#pragma unroll
  for (int k = 0; k < PASSES; ++k) {
    const int c = 8 * (tid + kThreadsA * k);
    live[k] = c < H;
    col[k] = min(c, H - 8);
  }
  // requested in the order they are needed: the first token's x and f, the
  // modulation rows, then the other tokens of the run (a run shorter than RT
  // re-reads its last row), so the whole run is in flight at the start and
  // each token waits only on its own rows
  uint4 xq[RT][PASSES], fq[RT][PASSES];
  auto load_token = [&](int t) {
    const int64_t row = (int64_t(b) * S + min(s0 + t, s1 - 1)) * H;
#pragma unroll
    for (int k = 0; k < PASSES; ++k) {
      xq[t][k] = ld_stream(x + row + col[k]);
      if (GATED) fq[t][k] = ld_stream(f + row + col[k]);
    }
  };
  load_token(0);
  float gt[PASSES][8], sc[PASSES][8], sh[PASSES][8], t0[PASSES][8], t1[PASSES][8], t2[PASSES][8],
      t3[PASSES][8];
#pragma unroll
  for (int k = 0; k < PASSES; ++k) {
    ld8f(tm + col[k], sh[k]);                      // t_mod row 0: shift
    ld8f(ts + col[k], t0[k]);
    ld8f(tm + H + col[k], sc[k]);                  // row 1: scale
    ld8f(tc + col[k], t1[k]);
    ld8f(wn + col[k], t2[k]);
    if (GATED) {
      ld8f(tm + 2 * H + col[k], gt[k]);            // row 2: gate
      ld8f(tg + col[k], t3[k]);
    }
  }
#pragma unroll
  for (int t = 1; t < RT; ++t) load_token(t);
  // keep every load ahead of the first use: the empty asm stops the loads
  // from being sunk to their uses, the barrier stops the scheduler
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int k = 0; k < PASSES; ++k)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      sh[k][i] += t0[k][i];
      sc[k][i] = (1.f + (sc[k][i] + t1[k][i])) * (t2[k][i] + w_add);   // w_norm * (1 + scale)
      if (GATED) gt[k][i] += t3[k][i];
    }

  const float inv_h = 1.f / float(H);
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    const int s = s0 + t;
    if (s >= s1) break;
    const int64_t row = (int64_t(b) * S + s) * H;
    uint4 rv[PASSES];
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < PASSES; ++k) {
      rv[k] = xq[t][k];
      if (GATED) {
        float xv[8], fv[8];
        unpack8(rv[k], xv);
        unpack8(fq[t][k], fv);
#pragma unroll
        for (int i = 0; i < 8; ++i) xv[i] = __builtin_fmaf(gt[k][i], fv[i], xv[i]);
        rv[k] = pack8(xv);
        if (live[k]) st_stream(r_out + row + col[k], rv[k]);
      }
      float rr[8], q = 0.f;
      unpack8(rv[k], rr);                          // the stored (rounded) r
#pragma unroll
      for (int i = 0; i < 8; ++i) q = __builtin_fmaf(rr[i], rr[i], q);
      ss += live[k] ? q : 0.f;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
    if (lane == 0) s_red[t & 1][wv] = ss;
    __syncthreads();                               // slot t&1 is next written two tokens on
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < kThreadsA / 64; ++w) tot += s_red[t & 1][w];
    const float rinv = rsqrtf(tot * inv_h + eps);
#pragma unroll
    for (int k = 0; k < PASSES; ++k) {
      float rr[8];
      unpack8(rv[k], rr);
#pragma unroll
      for (int i = 0; i < 8; ++i) rr[i] = __builtin_fmaf(rr[i] * rinv, sc[k][i], sh[k][i]);
      if (live[k]) st_stream(h + row + col[k], pack8(rr));
    }
  }
}

}  // namespace

int launch_adaln(const td_adaln_args *a, void *stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  // tokens per workgroup: the most that still leaves a workgroup per CU (more
  // tokens amortise the modulation loads and put more rows in flight; at
  // 64 x 16 x 4096, 4 tokens take 10.0 us against 12.0 us for 2)
  int R = 1;
  for (int r : {8, 4, 2})
    if (int64_t(a->B) * ((a->S + r - 1) / r) >= 256) {
      R = r;
      break;
    }
  const dim3 grid(unsigned(int64_t(a->B) * ((a->S + R - 1) / R))), block(kThreadsA);
  const int passes = (a->H + kColsPerPass - 1) / kColsPerPass;
#define TD_ADALN(PS, RR)                                                                            \
  hipLaunchKernelGGL((a->f ? adaln_rows<PS, RR, true> : adaln_rows<PS, RR, false>), grid, block, 0, st, static_cast<const bf16 *>(a->x),    \
                     static_cast<const bf16 *>(a->f), a->t_mod, a->tab_gate, a->tab_shift,          \
                     a->tab_scale, a->w_norm, static_cast<bf16 *>(a->r_out), static_cast<bf16 *>(a->h), \
                     a->S, a->H, a->eps)
#define TD_ADALN_R(PS)                                                                              \
  switch (R) {                                                                                      \
    case 8: TD_ADALN(PS, 8); break;                                                                 \
    case 4: TD_ADALN(PS, 4); break;                                                                 \
    case 2: TD_ADALN(PS, 2); break;                                                                 \
    default: TD_ADALN(PS, 1); break;                                                                \
  }
  if (passes <= 1) TD_ADALN_R(1)
  else if (passes <= 2) TD_ADALN_R(2)               // H <= 8192
  else return TD_ERR_UNSUPPORTED;
#undef TD_ADALN_R
#undef TD_ADALN
  return hipGetLastError() == hipSuccess ? TD_OK : TD_ERR_HIP;
}

}  // namespace td
