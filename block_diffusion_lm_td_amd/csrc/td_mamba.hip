// State-space core of a denoiser Mamba-2 layer over the block, seeded from the
// context tower's state, on gfx950 (news.chathome.org, "NVIDIA releases
// Nemotron-Labs-TwoTower ...", inference paragraph: the denoiser's Mamba-2
// layers start from the context tower's state).  The recurrence is Mamba-2's
// selective scan with one decay rate per head:
//   h_t = exp(dt_t A) h_{t-1} + dt_t x_t (outer) B_t,  y_t = h_t C_t + D x_t,
// h_0 the seed.  Over a block of S <= 16 tokens it is computed as one sum,
// with c_t = sum_{r<=t} dt_r A:
//   y_t = e^{c_t} (h_0 C_t) + sum_{s<=t} e^{c_t - c_s} dt_s (C_t . B_s) x_s + D x_t
// so the seed state is read once and no state is carried token to token.
//
// mamba_block: one wave per (sequence, head), fp32 arithmetic throughout.
//   - Inter term h_0 C^T: [P x N] . [N x S] on v_mfma_f32_16x16x4_f32, the 16
//     tokens as the 16 columns.  h_0 streams from HBM in 32-wide slices: per
//     load instruction the four lanes of a row read one contiguous 64-byte
//     half of its 128-byte line (a half spread over the whole line costs about
//     1.4 line fetches per line, L2 serving the second half late); the K order
//     inside each slice is permuted the same way on both operands.
//   - Intra term: C B^T [S x S] on the same MFMA (the C loads are shared
//     with the inter term), decayed and masked to s <= t, transposed through
//     the wave's LDS slot, then times x [S x P].
//   - y = e^{c_t} (inter) + (intra) + D x in bf16.
// The work is bound by reading h_0 (P*N*4 bytes per sequence and head).
#include <hip/hip_runtime.h>

#include "td_internal.h"

namespace td {
namespace {

typedef __bf16 bf16;
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWavesM = 4;

__device__ inline f32x4 ld_bf16x4(const bf16 *p) {
  const uint2 v = *reinterpret_cast<const uint2 *>(p);
  return f32x4{__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u),
               __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xffff0000u)};
}
// Orders this wave's LDS writes before its later LDS reads of other lanes'
// entries (the slot is the wave's own: no workgroup barrier).
__device__ inline void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}
__device__ inline uint32_t pack_bf16(float a, float b) {
  const bf16 x = bf16(a), y = bf16(b);
  return uint32_t(__builtin_bit_cast(uint16_t, x)) | (uint32_t(__builtin_bit_cast(uint16_t, y)) << 16);
}

template <int PT>
__global__ __launch_bounds__(kWavesM * 64) void mamba_block(
    const bf16 *__restrict__ x, const float *__restrict__ dt, const float *__restrict__ A,
    const bf16 *__restrict__ Bm, const bf16 *__restrict__ Cm, const float *__restrict__ Dv,
    const float *__restrict__ h0, bf16 *__restrict__ y, int nseq, int S, int H, int N, int G) {
  constexpr int P = 16 * PT;
  __shared__ float s_x[kWavesM][16][P + 1];      // x[s][p] (fp32; +1: no bank conflicts on columns)
  __shared__ float s_m[kWavesM][16][17];         // M[t][s]
  __shared__ float s_c[kWavesM][16], s_dt[kWavesM][16];
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r16 = lane & 15, g4 = lane >> 4;
  // workgroups are dealt to the 8 XCDs in turn: within each run of 32, XCD x
  // takes the four consecutive ones 4x..4x+3 (heads of one group when H/G is
  // a multiple of 16, sharing B and C in that XCD's L2), and the runs keep
  // launch order, so the workgroups in flight read neighbouring seed states
  const unsigned nwg = gridDim.x, bid = blockIdx.x;
  const unsigned lwg = bid >= (nwg & ~31u) ? bid : (bid & ~31u) + 4 * (bid & 7u) + ((bid >> 3) & 3u);
  const int64_t unit = int64_t(lwg) * kWavesM + wv;
  if (unit >= int64_t(nseq) * H) return;          // no barriers below: every wave is on its own
  const int b = int(unit / H), h = int(unit - int64_t(b) * H);
  const int grp = h / (H / G);
  const float a_h = A[h], d_h = Dv[h];

  // dt and the running decay exponent c_t (tokens past S: dt = 0)
  if (lane < 16) {
    const float d = lane < S ? dt[(int64_t(b) * S + lane) * H + h] : 0.f;
    float c = d * a_h;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const float v = __shfl_up(c, o, 16);
      if (lane >= o) c += v;
    }
    s_dt[wv][lane] = d;
    s_c[wv][lane] = c;
  }
  // x [S x P], 8 values per lane and load (rows past S: zero); loaded now,
  // written to the slot after the state loop so that its latency overlaps
  // the stream of h_0
  constexpr int kXL = (2 * P + 63) / 64;
  uint4 xv[kXL];
#pragma unroll
  for (int k = 0; k < kXL; ++k) {
    const int i = lane + 64 * k;
    const int s = i / (P / 8), p = (i - s * (P / 8)) * 8;
    xv[k] = make_uint4(0, 0, 0, 0);
    if (i < 2 * P && s < S) xv[k] = *reinterpret_cast<const uint4 *>(x + ((int64_t(b) * S + s) * H + h) * P + p);
  }

  // token row of B / C for lane r16 (rows past S read row S-1; masked later)
  const int tr = r16 < S ? r16 : S - 1;
  const bf16 *crow = Cm + ((int64_t(b) * S + tr) * G + grp) * N + 4 * g4;
  const bf16 *brow = Bm + ((int64_t(b) * S + tr) * G + grp) * N + 4 * g4;
  const float *hrow = h0 + ((int64_t(b) * H + h) * P + r16) * N + 4 * g4;

  f32x4 acc[PT];                                   // Y^T tiles: lane -> token r16, p = 16*pt + 4*g4 + i
#pragma unroll
  for (int pt = 0; pt < PT; ++pt) acc[pt] = f32x4{};
  f32x4 cb = f32x4{};                              // (C B^T)^T: lane -> s = r16, t = 4*g4 + i
  // 32-wide slices of the state: per half u the four lanes of a row read 16
  // consecutive entries of h_0 (and of C / B).  MFMA k = 4*g4 + i of half u
  // stands for state entry j + 16*u + 4*g4 + i on every operand.
  for (int j = 0; j < N; j += 32) {
    f32x4 cv[2], bv[2], hv[PT][2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      cv[u] = ld_bf16x4(crow + j + 16 * u);
      bv[u] = ld_bf16x4(brow + j + 16 * u);
#pragma unroll
      for (int pt = 0; pt < PT; ++pt)
        hv[pt][u] = *reinterpret_cast<const f32x4 *>(hrow + int64_t(16 * pt) * N + j + 16 * u);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int pt = 0; pt < PT; ++pt)
          acc[pt] = __builtin_amdgcn_mfma_f32_16x16x4f32(hv[pt][u][i], cv[u][i], acc[pt], 0, 0, 0);
        cb = __builtin_amdgcn_mfma_f32_16x16x4f32(cv[u][i], bv[u][i], cb, 0, 0, 0);
      }
  }
#pragma unroll
  for (int k = 0; k < kXL; ++k) {
    const int i = lane + 64 * k;
    if (i >= 2 * P) break;
    const int s = i / (P / 8), p = (i - s * (P / 8)) * 8;
    const uint32_t w4[4] = {xv[k].x, xv[k].y, xv[k].z, xv[k].w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      s_x[wv][s][p + 2 * q] = __uint_as_float(w4[q] << 16);
      s_x[wv][s][p + 2 * q + 1] = __uint_as_float(w4[q] & 0xffff0000u);
    }
  }
  wave_sync();                                     // s_c, s_dt and s_x visible to the wave
  // inter term: column t = r16 scaled by e^{c_t}
  const float et = __expf(s_c[wv][r16]);
#pragma unroll
  for (int pt = 0; pt < PT; ++pt) acc[pt] *= et;
  // M[t][s] = (C_t . B_s) e^{c_t - c_s} dt_s for s <= t < S, else 0; cb holds
  // t = 4*g4 + i, s = r16
  {
    const int s = r16;
    const float cs = s_c[wv][s], ds = s_dt[wv][s];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 4 * g4 + i;
      s_m[wv][t][s] = (s <= t && t < S) ? cb[i] * __expf(s_c[wv][t] - cs) * ds : 0.f;
    }
  }
  wave_sync();
  // intra term: Y^T[p][t] += sum_s x[s][p] M[t][s]  (A = x^T, B = M^T; k = s)
#pragma unroll
  for (int k0 = 0; k0 < 16; k0 += 4) {
    const int s = k0 + g4;
    const float mv = s_m[wv][r16][s];
#pragma unroll
    for (int pt = 0; pt < PT; ++pt)
      acc[pt] = __builtin_amdgcn_mfma_f32_16x16x4f32(s_x[wv][s][16 * pt + r16], mv, acc[pt], 0, 0, 0);
  }
  // y = inter + intra + D x, bf16; lane -> token r16, p = 16*pt + 4*g4 + i
  if (r16 < S) {
    bf16 *yr = y + ((int64_t(b) * S + r16) * H + h) * P;
#pragma unroll
    for (int pt = 0; pt < PT; ++pt) {
      const int p = 16 * pt + 4 * g4;
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = acc[pt][i] + d_h * s_x[wv][r16][p + i];
      *reinterpret_cast<uint2 *>(yr + p) = make_uint2(pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]));
    }
  }
}

}  // namespace

int launch_mamba(const td_mamba_args *a, void *stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int64_t units = int64_t(a->B) * a->H;
  const dim3 grid(unsigned((units + kWavesM - 1) / kWavesM)), block(kWavesM * 64);
#define TD_MAMBA(PT)                                                                              \
  hipLaunchKernelGGL((mamba_block<PT>), grid, block, 0, st, static_cast<const bf16 *>(a->x),     \
                     a->dt, a->A, static_cast<const bf16 *>(a->Bm), static_cast<const bf16 *>(a->Cm), \
                     a->D, a->h0, static_cast<bf16 *>(a->y), a->B, a->S, a->H, a->N, a->G)
  switch (a->P / 16) {
    case 1: TD_MAMBA(1); break;
    case 2: TD_MAMBA(2); break;
    case 4: TD_MAMBA(4); break;
    case 8: TD_MAMBA(8); break;
    default: return TD_ERR_UNSUPPORTED;
  }
#undef TD_MAMBA
  return hipGetLastError() == hipSuccess ? TD_OK : TD_ERR_HIP;
}

}  // namespace td
