// Confidence-masked commit of one denoise step on gfx950 (news.chathome.org,
// "NVIDIA releases Nemotron-Labs-TwoTower ...", evaluation paragraph:
// confidence masking with threshold gamma; block-generation paragraph:
// several positions may commit in one step, and every block finishes).
//
// commit_rows: one streaming pass over each row of logits (R workgroups per
//   row, 16-byte loads).  Every lane keeps a running max m, the index of the
//   first 8-element vector where it reached m, and Z = sum exp(x - m) with
//   the usual rescale when m grows.  The argmax inside the winning vector is
//   resolved once at the end by re-reading that vector, so the per-element
//   work is a convert, a max, an fma, an exp2 and an add.  Lanes, waves and
//   row parts are merged as (max, lowest index) pairs and Z rescaled to the
//   common max, in a fixed order (deterministic).
// commit_finalize: one wave per sequence; merges the row parts, p = 1/Z,
//   applies p >= gamma to the eligible positions and the force-one rule
//   (largest p among eligible, lowest position on ties), writes the outputs
//   and counts the positions still masked.
#include <hip/hip_runtime.h>

#include "td_internal.h"

namespace td {
namespace {

typedef __bf16 bf16;
constexpr float kNegInf = -__builtin_inff();
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kNoIndex = 0x7fffffff;
// The logits are read exactly once: non-temporal loads keep the stream from
// being allocated in the caches (measured 54.3 -> 48.1 us per td_commit at
// 64 x 16 rows of 131072 bf16 logits).
typedef unsigned int u32x4n __attribute__((ext_vector_type(4)));
typedef float f32x4n __attribute__((ext_vector_type(4)));
__device__ inline uint4 ldv(const uint4 *p) {
  const u32x4n v = __builtin_nontemporal_load(reinterpret_cast<const u32x4n *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ inline float4 ldv(const float4 *p) {
  const f32x4n v = __builtin_nontemporal_load(reinterpret_cast<const f32x4n *>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ inline void unpack(const uint4 &v, float (&f)[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ inline void unpack(const float4 &v, float (&f)[4]) {
  f[0] = v.x; f[1] = v.y; f[2] = v.z; f[3] = v.w;
}

template <typename T> struct Vec;
template <> struct Vec<bf16> { typedef uint4 type; static constexpr int n = 8; };
template <> struct Vec<float> { typedef float4 type; static constexpr int n = 4; };

__device__ inline float to_f(bf16 x) { return float(x); }
__device__ inline float to_f(float x) { return x; }

// Lane state update with the NV values of one vector starting at element e0.
template <int NV>
__device__ inline void absorb(const float (&f)[NV], int vi, float &m, float &z, int &bv) {
  float vmax = f[0];
#pragma unroll
  for (int k = 1; k < NV; ++k) vmax = fmaxf(vmax, f[k]);
  if (vmax > m) {
    z *= fast_exp2((m - vmax) * kLog2e);     // m = -inf: z is 0 and stays 0
    m = vmax;
    bv = vi;
  }
  const float mc = (m == kNegInf) ? 0.f : m * kLog2e;
#pragma unroll
  for (int k = 0; k < NV; ++k) z += fast_exp2(__builtin_fmaf(f[k], kLog2e, -mc));
}

template <typename T, bool VEC>
__global__ __launch_bounds__(256) void commit_rows(const T *__restrict__ logits, int V, int span,
                                                   int R, Part *__restrict__ parts,
                                                   int32_t *__restrict__ n_masked_left,
                                                   const int32_t *__restrict__ gate) {
  typedef typename Vec<T>::type VT;
  constexpr int NV = Vec<T>::n;
  const int64_t row = blockIdx.x / R;
  const int r = blockIdx.x - int(row) * R;
  const int tid = threadIdx.x;
  // cleared even in a gated-off step, so that a chain of gated steps stays off
  if (blockIdx.x == 0 && tid == 0 && n_masked_left) *n_masked_left = 0;
  if (gate && *gate == 0) return;
  const int e_lo = r * span;
  const int e_hi = min(V, e_lo + span);
  const T *x = logits + row * V;

  float m = kNegInf, z = 0.f;
  int bv = -1;    // vector index (VEC) or element index (scalar) of the lane's max
  if (VEC) {
    const VT *src = reinterpret_cast<const VT *>(x);
    const int v_lo = e_lo / NV, v_hi = e_hi / NV;
    int vi = v_lo + tid;
    for (; vi + 3 * 256 < v_hi; vi += 4 * 256) {
      const VT a0 = ldv(src + vi), a1 = ldv(src + vi + 256), a2 = ldv(src + vi + 512), a3 = ldv(src + vi + 768);
      float f[NV];
      unpack(a0, f); absorb<NV>(f, vi, m, z, bv);
      unpack(a1, f); absorb<NV>(f, vi + 256, m, z, bv);
      unpack(a2, f); absorb<NV>(f, vi + 512, m, z, bv);
      unpack(a3, f); absorb<NV>(f, vi + 768, m, z, bv);
    }
    for (; vi < v_hi; vi += 256) {
      float f[NV];
      unpack(ldv(src + vi), f);
      absorb<NV>(f, vi, m, z, bv);
    }
  } else {
    for (int e = e_lo + tid; e < e_hi; e += 256) {
      float f[1] = {to_f(x[e])};
      absorb<1>(f, e, m, z, bv);
    }
  }
  // lowest index of the lane's max; only lanes holding their wave's max can
  // hold the row's argmax, so only they re-read their best vector
  int idx = kNoIndex;
  float wmx = m;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) wmx = fmaxf(wmx, __shfl_xor(wmx, o));
  if (m < wmx) bv = -1;
  if (bv >= 0) {
    if (VEC) {
      float f[NV];
      unpack(reinterpret_cast<const VT *>(x)[bv], f);
      int k = NV - 1;
#pragma unroll
      for (int kk = NV - 1; kk >= 0; --kk)
        if (f[kk] == m) k = kk;
      idx = bv * NV + k;
    } else {
      idx = bv;
    }
  }
  // wave merge of (m, idx): larger m, then lower idx
  float wm = m;
  int wi = idx;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float om = __shfl_xor(wm, o);
    const int oi = __shfl_xor(wi, o);
    if (om > wm || (om == wm && oi < wi)) { wm = om; wi = oi; }
  }
  float zs = (m == kNegInf) ? 0.f : z * fast_exp2((m - wm) * kLog2e);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) zs += __shfl_xor(zs, o);

  __shared__ float sm[4], sz[4];
  __shared__ int si[4];
  const int wv = tid >> 6;
  if ((tid & 63) == 0) { sm[wv] = wm; sz[wv] = zs; si[wv] = wi; }
  __syncthreads();
  if (tid == 0) {
    float M = sm[0];
    int I = si[0];
#pragma unroll
    for (int k = 1; k < 4; ++k)
      if (sm[k] > M || (sm[k] == M && si[k] < I)) { M = sm[k]; I = si[k]; }
    float Z = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) Z += (sm[k] == kNegInf) ? 0.f : sz[k] * fast_exp2((sm[k] - M) * kLog2e);
    Part p;
    p.m = M; p.z = Z; p.idx = I; p.pad = 0;
    parts[row * R + r] = p;
  }
}

__global__ __launch_bounds__(64) void commit_finalize(
    const Part *__restrict__ parts, int S, int R, float gamma, const uint8_t *masked_in,
    uint8_t *__restrict__ commit, int32_t *__restrict__ token, float *__restrict__ maxprob,
    int32_t *__restrict__ n_commit, uint8_t *masked_out, int32_t *__restrict__ tokens,
    int32_t *__restrict__ n_masked_left, const int32_t *__restrict__ gate, bool skip_inelig) {
  if (gate && *gate == 0) return;
  const int b = blockIdx.x;
  const int i = threadIdx.x;
  const bool act = i < S;
  const int64_t row = int64_t(b) * S + i;
  float p = 0.f;
  int idx = 0;
  bool elig = false;
  if (act) elig = masked_in ? masked_in[row] != 0 : true;
  if (act && skip_inelig && !elig) {
    idx = -1;                        // not scored: no parts were made for it
  } else if (act) {
    float M = kNegInf;
    for (int r = 0; r < R; ++r) M = fmaxf(M, parts[row * R + r].m);
    float Z = 0.f;
    idx = kNoIndex;
    for (int r = 0; r < R; ++r) {
      const Part q = parts[row * R + r];
      if (q.m == M && q.idx < idx) idx = q.idx;
      Z += (q.m == kNegInf) ? 0.f : q.z * fast_exp2((q.m - M) * kLog2e);
    }
    p = 1.0f / Z;
  }
  const bool pass = act && elig && p >= gamma;
  const unsigned long long pm = __ballot(pass);
  const unsigned long long em = __ballot(act && elig);
  bool cm = pass;
  if (pm == 0ull && em != 0ull) {
    float bp = (act && elig) ? p : -1.0f;
    int bi = (act && elig) ? i : 1 << 30;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float op = __shfl_xor(bp, o);
      const int oi = __shfl_xor(bi, o);
      if (op > bp || (op == bp && oi < bi)) { bp = op; bi = oi; }
    }
    cm = act && (i == bi);
  }
  const unsigned long long cmask = __ballot(cm);
  const bool still = act && elig && !cm;
  const unsigned long long lmask = __ballot(still);
  if (act) {
    commit[row] = cm ? 1 : 0;
    token[row] = idx;
    if (maxprob) maxprob[row] = p;
    if (masked_out) masked_out[row] = still ? 1 : 0;
    if (tokens && cm) tokens[row] = idx;
  }
  if (i == 0) {
    if (n_commit) n_commit[b] = __popcll(cmask);
    if (n_masked_left) atomicAdd(n_masked_left, int(__popcll(lmask)));
  }
}

}  // namespace

int launch_commit_finalize(const Part *parts, int R, int B, int S, float gamma,
                           const uint8_t *masked_in, uint8_t *commit, int32_t *token,
                           float *maxprob, int32_t *n_commit, uint8_t *masked_out,
                           int32_t *tokens, int32_t *n_masked_left, void *stream,
                           const int32_t *gate, bool skip_ineligible) {
  hipLaunchKernelGGL(commit_finalize, dim3(B), dim3(64), 0, reinterpret_cast<hipStream_t>(stream),
                     parts, S, R, gamma, masked_in, commit, token, maxprob, n_commit, masked_out,
                     tokens, n_masked_left, gate, skip_ineligible);
  return hipGetLastError() == hipSuccess ? TD_OK : TD_ERR_HIP;
}

int launch_commit(const td_commit_args *c, const CommitPlan &p, void *ws, void *stream,
                  const int32_t *gate) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  Part *parts = reinterpret_cast<Part *>(ws);
  const unsigned nblk = unsigned(p.rows * p.R);
  if (c->dtype == TD_BF16) {
    if (p.vec)
      hipLaunchKernelGGL((commit_rows<bf16, true>), dim3(nblk), dim3(256), 0, st,
                         static_cast<const bf16 *>(c->logits), c->V, p.span, p.R, parts, c->n_masked_left, gate);
    else
      hipLaunchKernelGGL((commit_rows<bf16, false>), dim3(nblk), dim3(256), 0, st,
                         static_cast<const bf16 *>(c->logits), c->V, p.span, p.R, parts, c->n_masked_left, gate);
  } else {
    if (p.vec)
      hipLaunchKernelGGL((commit_rows<float, true>), dim3(nblk), dim3(256), 0, st,
                         static_cast<const float *>(c->logits), c->V, p.span, p.R, parts, c->n_masked_left, gate);
    else
      hipLaunchKernelGGL((commit_rows<float, false>), dim3(nblk), dim3(256), 0, st,
                         static_cast<const float *>(c->logits), c->V, p.span, p.R, parts, c->n_masked_left, gate);
  }
  if (hipGetLastError() != hipSuccess) return TD_ERR_HIP;
  return launch_commit_finalize(parts, p.R, c->B, c->S, c->gamma, c->masked_in, c->commit, c->token,
                                c->maxprob, c->n_commit, c->masked_out, c->tokens,
                                c->n_masked_left, stream, gate);
}

}  // namespace td
