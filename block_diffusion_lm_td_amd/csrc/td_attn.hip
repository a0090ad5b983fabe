// Block attention of one denoiser layer on gfx950: the S block queries of
// every query head attend, in ONE softmax, to the context tower's cached
// keys of the sequence and to the block's own keys (news.chathome.org,
// "NVIDIA releases Nemotron-Labs-TwoTower ...", inference paragraph:
// bidirectional inside the block, layer-aligned cross-attention to the
// per-layer KV cache; aiboss88.com, technical-principle section).
//
// bf16, D = 128: attn_bf16_mfma.  One workgroup owns up to 256 query rows
// (the G heads x S positions that share one KV head, the GQA group) and one
// chunk of the [context ; block] key sequence.  Four waves of 64 rows each.
// K tiles are staged row-major in LDS, V tiles transposed (keys innermost),
// and both products run on v_mfma_f32_32x32x16_bf16 in the transposed
// orientation S^T = K Q^T, O^T = V^T P^T: the score matrix then lands with
// one query per lane column, so the softmax max/sum over keys is 15 in-lane
// ops plus one cross-half swap, and P^T feeds the PV product straight from
// the accumulator registers (the key order inside a 16-key group is
// permuted identically on both operands).  Softmax runs in the exp2 domain
// with a lazy rescale: the running max only moves when a tile's max exceeds
// it by more than 2^8, which is exact in real arithmetic and keeps P <= 256.
// A chunk that is not the whole sequence writes fp32 partials (O, m, l);
// attn_combine merges them by log-sum-exp in chunk order (deterministic).
//
// Any other dtype / head dim: attn_valu, one thread per query row (a plain
// correctness path for small fp32 problems).
#include <hip/hip_runtime.h>

#include "td_internal.h"

namespace td {
namespace {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int HD = 128;                 // head dim of the MFMA path
constexpr int KSTR = HD + 8;            // LDS row stride of the K tile (elements)
constexpr int VSTR = kKeyTile + 8;      // LDS row stride of the V^T tile (elements)
constexpr float kNegInf = -__builtin_inff();
constexpr float kLazy = 8.0f;           // rescale only when the max grows by > 2^8

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Clamped sequence range: never reads outside [0, total_ctx) whatever the
// device offsets hold; L is also capped at max_ctx (the grid's assumption).
__device__ inline void seq_range(const int64_t *off, int b, int64_t total, int max_ctx,
                                 int64_t &lo, int &L) {
  int64_t a = off[b], e = off[b + 1];
  a = a < 0 ? 0 : (a > total ? total : a);
  e = e < a ? a : (e > total ? total : e);
  int64_t len = e - a;
  lo = a;
  L = int(len > max_ctx ? max_ctx : len);
}

__global__ __launch_bounds__(256, 1) void attn_bf16_mfma(
    const bf16 *__restrict__ q, const bf16 *__restrict__ kb, const bf16 *__restrict__ vb,
    const bf16 *__restrict__ kc, const bf16 *__restrict__ vc, const int64_t *__restrict__ off,
    int64_t total_ctx, int max_ctx, int S, int Hq, int Hkv, int G, int M, int row_groups,
    int chunk, int nchunks, float sl2, float *__restrict__ ws_o, float2 *__restrict__ ws_ml,
    bf16 *__restrict__ out) {
  __shared__ __attribute__((aligned(16))) bf16 Ks[kKeyTile * KSTR];
  __shared__ __attribute__((aligned(16))) bf16 Vt[HD * VSTR];

  const int c = blockIdx.x;
  const int g = blockIdx.y % Hkv;
  const int rg = blockIdx.y / Hkv;
  const int b = blockIdx.z;
  int64_t lo;
  int L;
  seq_range(off, b, total_ctx, max_ctx, lo, L);
  const int N = L + S;
  const int k0 = c * chunk;
  if (k0 >= N) return;
  const int k1 = min(k0 + chunk, N);
  const int nc_b = (N + chunk - 1) / chunk;

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, lq = lane & 31, lh = lane >> 5;
  const int64_t kvstride = int64_t(Hkv) * HD;

  // ---- Q fragments (B operand of S^T = K Q^T): lane (query lq, half lh)
  // holds Q[row][ks*16 + lh*8 .. +8] for the 8 k-steps of D = 128.
  bf16x8 qf[2][8];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int row = rg * kRowsPerWG + w * 64 + qb * 32 + lq;
    if (row < M) {
      const int s = row / G, j = row - s * G;
      const bf16 *p = q + ((int64_t(b) * S + s) * Hq + int64_t(g) * G + j) * HD + lh * 8;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) qf[qb][ks] = *reinterpret_cast<const bf16x8 *>(p + ks * 16);
    } else {
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) qf[qb][ks] = bf16x8{};
    }
  }

  f32x16 o[2][4];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int db = 0; db < 4; ++db) o[qb][db] = f32x16{};
  float m[2] = {kNegInf, kNegInf};
  float l[2] = {0.f, 0.f};

  // ---- tile loaders (global -> registers), keys n in [k0, k1)
  const bf16 *kc_g = kc + lo * kvstride + int64_t(g) * HD;
  const bf16 *vc_g = vc + lo * kvstride + int64_t(g) * HD;
  const bf16 *kb_g = kb + int64_t(b) * S * kvstride + int64_t(g) * HD;
  const bf16 *vb_g = vb + int64_t(b) * S * kvstride + int64_t(g) * HD;
  const int kr = tid >> 4, kc8 = (tid & 15) * 8;         // K: 2 x 16 B per thread
  const int vk4 = tid >> 5, vd4 = (tid & 31) * 4;        // V: 4 keys x 4 dims per thread
  uint4 kreg[2];
  uint2 vreg[4];
  auto load_tile = [&](int t) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int n = t + kr + r * 16;
      uint4 x = make_uint4(0, 0, 0, 0);
      if (n < k1) {
        const bf16 *src = n < L ? kc_g + int64_t(n) * kvstride : kb_g + int64_t(n - L) * kvstride;
        x = *reinterpret_cast<const uint4 *>(src + kc8);
      }
      kreg[r] = x;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int n = t + vk4 * 4 + i;
      uint2 x = make_uint2(0, 0);
      if (n < k1) {
        const bf16 *src = n < L ? vc_g + int64_t(n) * kvstride : vb_g + int64_t(n - L) * kvstride;
        x = *reinterpret_cast<const uint2 *>(src + vd4);
      }
      vreg[i] = x;
    }
  };
  // V^T tile position of key k (0..31): within each 16-key group, key
  // j*8 + h*4 + i (the accumulator's row order) goes to h*8 + j*4 + i, so a
  // lane's 8 PV operand keys are contiguous.
  const int vpos = (vk4 >> 2) * 16 + (vk4 & 1) * 8 + ((vk4 >> 1) & 1) * 4;
  auto store_tile = [&]() {
#pragma unroll
    for (int r = 0; r < 2; ++r)
      *reinterpret_cast<uint4 *>(&Ks[(kr + r * 16) * KSTR + kc8]) = kreg[r];
    const uint32_t a0 = vreg[0].x, a1 = vreg[1].x, a2 = vreg[2].x, a3 = vreg[3].x;
    const uint32_t b0 = vreg[0].y, b1 = vreg[1].y, b2 = vreg[2].y, b3 = vreg[3].y;
    uint2 t0, t1, t2, t3;
    t0.x = (a0 & 0xffffu) | (a1 << 16);          t0.y = (a2 & 0xffffu) | (a3 << 16);
    t1.x = (a0 >> 16) | (a1 & 0xffff0000u);      t1.y = (a2 >> 16) | (a3 & 0xffff0000u);
    t2.x = (b0 & 0xffffu) | (b1 << 16);          t2.y = (b2 & 0xffffu) | (b3 << 16);
    t3.x = (b0 >> 16) | (b1 & 0xffff0000u);      t3.y = (b2 >> 16) | (b3 & 0xffff0000u);
    *reinterpret_cast<uint2 *>(&Vt[(vd4 + 0) * VSTR + vpos]) = t0;
    *reinterpret_cast<uint2 *>(&Vt[(vd4 + 1) * VSTR + vpos]) = t1;
    *reinterpret_cast<uint2 *>(&Vt[(vd4 + 2) * VSTR + vpos]) = t2;
    *reinterpret_cast<uint2 *>(&Vt[(vd4 + 3) * VSTR + vpos]) = t3;
  };

  load_tile(k0);
  for (int t = k0; t < k1; t += kKeyTile) {
    __syncthreads();                      // previous tile fully consumed
    store_tile();
    __syncthreads();
    if (t + kKeyTile < k1) load_tile(t + kKeyTile);   // in flight during compute
    const int nvalid = k1 - t;

    // ---- S^T = K Q^T : 32 keys x 64 queries per wave (two 32x32 blocks)
    f32x16 sc[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const bf16x8 ka = *reinterpret_cast<const bf16x8 *>(&Ks[lq * KSTR + ks * 16 + lh * 8]);
      sc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[0][ks], sc[0], 0, 0, 0);
      sc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[1][ks], sc[1], 0, 0, 0);
    }
    if (nvalid < kKeyTile) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = (r >> 2) * 8 + lh * 4 + (r & 3);
        if (key >= nvalid) { sc[0][r] = kNegInf; sc[1][r] = kNegInf; }
      }
    }

    // ---- online softmax (exp2 domain, lazy rescale) and P^T as bf16
    bf16x8 pb[2][2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float mx = sc[qb][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sc[qb][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mxs = mx * sl2;
      const bool need = mxs > m[qb] + kLazy;
      if (__any(need)) {
        const float mn = need ? mxs : m[qb];
        const float alpha = fast_exp2(m[qb] - mn);
#pragma unroll
        for (int db = 0; db < 4; ++db) o[qb][db] *= alpha;
        l[qb] *= alpha;
        m[qb] = mn;
      }
      float ls = 0.f;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float p = fast_exp2(__builtin_fmaf(sc[qb][kk * 8 + i], sl2, -m[qb]));
          ls += p;
          pb[qb][kk][i] = bf16(p);
        }
      }
      l[qb] += ls;
    }

    // ---- O^T += V^T P^T : 128 dims x 64 queries per wave
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const bf16x8 va =
            *reinterpret_cast<const bf16x8 *>(&Vt[(db * 32 + lq) * VSTR + kk * 16 + lh * 8]);
        o[0][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[0][kk], o[0][db], 0, 0, 0);
        o[1][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[1][kk], o[1][db], 0, 0, 0);
      }
    }
  }

#pragma unroll
  for (int qb = 0; qb < 2; ++qb) l[qb] += __shfl_xor(l[qb], 32);

  if (nc_b == 1) {
    // The whole sequence is in this chunk: normalise and store bf16 (RNE).
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int row = rg * kRowsPerWG + w * 64 + qb * 32 + lq;
      if (row >= M) continue;
      const int s = row / G, j = row - s * G;
      bf16 *dst = out + ((int64_t(b) * S + s) * Hq + int64_t(g) * G + j) * HD;
      const float inv = 1.0f / l[qb];
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) {
          bf16x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = bf16(o[qb][db][gi * 4 + e] * inv);
          *reinterpret_cast<bf16x4 *>(dst + db * 32 + gi * 8 + lh * 4) = v;
        }
    }
  } else {
    // Partials in accumulator-fragment order: float4 [frag][lane] per slot.
    const size_t slot = (size_t(blockIdx.z * Hkv + g) * row_groups + rg) * nchunks + c;
    float4 *wo = reinterpret_cast<float4 *>(ws_o + slot * (size_t(kRowsPerWG) * HD));
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) {
          const int frag = ((w * 2 + qb) * 4 + db) * 4 + gi;
          wo[frag * 64 + lane] = make_float4(o[qb][db][gi * 4 + 0], o[qb][db][gi * 4 + 1],
                                             o[qb][db][gi * 4 + 2], o[qb][db][gi * 4 + 3]);
        }
    if (lh == 0) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
        ws_ml[slot * kRowsPerWG + w * 64 + qb * 32 + lq] = make_float2(m[qb], l[qb]);
    }
  }
}

// Log-sum-exp merge of the chunk partials of every (b, kv head, row group)
// whose sequence spans more than one chunk.  One thread per float4 of the
// fragment layout; chunks merged in increasing order.
__global__ __launch_bounds__(256) void attn_combine(
    const float *__restrict__ ws_o, const float2 *__restrict__ ws_ml, const int64_t *__restrict__ off,
    int64_t total_ctx, int max_ctx, int S, int Hq, int Hkv, int G, int M, int row_groups,
    int chunk, int nchunks, bf16 *__restrict__ out) {
  const int unit = blockIdx.y;
  const int rg = unit % row_groups;
  const int g = (unit / row_groups) % Hkv;
  const int b = unit / (row_groups * Hkv);
  int64_t lo;
  int L;
  seq_range(off, b, total_ctx, max_ctx, lo, L);
  const int N = L + S;
  const int nc_b = (N + chunk - 1) / chunk;
  if (nc_b <= 1) return;
  const int f = blockIdx.x * 256 + threadIdx.x;      // 0 .. 8191
  const int lane = f & 63, frag = f >> 6;
  const int gi = frag & 3, db = (frag >> 2) & 3, qb = (frag >> 4) & 1, w = frag >> 5;
  const int rloc = w * 64 + qb * 32 + (lane & 31);
  const int row = rg * kRowsPerWG + rloc;
  if (row >= M) return;
  const size_t slot0 = size_t(unit) * nchunks;
  float mmax = kNegInf;
  for (int cc = 0; cc < nc_b; ++cc) mmax = fmaxf(mmax, ws_ml[(slot0 + cc) * kRowsPerWG + rloc].x);
  float lsum = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  const float4 *wo = reinterpret_cast<const float4 *>(ws_o);
  for (int cc = 0; cc < nc_b; ++cc) {
    const float2 ml = ws_ml[(slot0 + cc) * kRowsPerWG + rloc];
    const float wgt = fast_exp2(ml.x - mmax);
    lsum += wgt * ml.y;
    const float4 v = wo[(slot0 + cc) * (kRowsPerWG * HD / 4) + f];
    acc.x += wgt * v.x; acc.y += wgt * v.y; acc.z += wgt * v.z; acc.w += wgt * v.w;
  }
  const float inv = 1.0f / lsum;
  const int s = row / G, j = row - s * G;
  const int d = db * 32 + gi * 8 + (lane >> 5) * 4;
  bf16x4 v;
  v[0] = bf16(acc.x * inv); v[1] = bf16(acc.y * inv); v[2] = bf16(acc.z * inv); v[3] = bf16(acc.w * inv);
  *reinterpret_cast<bf16x4 *>(out + ((int64_t(b) * S + s) * Hq + int64_t(g) * G + j) * HD + d) = v;
}

// ---------------------------------------------------------------------------
// VALU path: one thread per query row, keys staged 32 at a time in LDS.
// ---------------------------------------------------------------------------
template <typename T>
__device__ inline float ld(const T *p);
template <>
__device__ inline float ld<float>(const float *p) { return *p; }
template <>
__device__ inline float ld<bf16>(const bf16 *p) { return float(*p); }
template <typename T>
__device__ inline void st(T *p, float v);
template <>
__device__ inline void st<float>(float *p, float v) { *p = v; }
template <>
__device__ inline void st<bf16>(bf16 *p, float v) { *p = bf16(v); }

template <typename T, int DD>
__global__ __launch_bounds__(64) void attn_valu(
    const T *__restrict__ q, const T *__restrict__ kb, const T *__restrict__ vb,
    const T *__restrict__ kc, const T *__restrict__ vc, const int64_t *__restrict__ off,
    int64_t total_ctx, int max_ctx, int S, int Hq, int Hkv, int G, int M, float sl2,
    T *__restrict__ out) {
  __shared__ float Kt[32][DD];
  __shared__ float Vt2[32][DD];
  const int g = blockIdx.y, b = blockIdx.z;
  const int row = blockIdx.x * 64 + threadIdx.x;
  const bool valid = row < M;
  int64_t lo;
  int L;
  seq_range(off, b, total_ctx, max_ctx, lo, L);
  const int N = L + S;
  const int64_t kvstride = int64_t(Hkv) * DD;
  const int s = valid ? row / G : 0, j = valid ? row - (row / G) * G : 0;
  const T *qp = q + ((int64_t(b) * S + s) * Hq + int64_t(g) * G + j) * DD;
  float qv[DD], o[DD];
#pragma unroll
  for (int d = 0; d < DD; ++d) {
    qv[d] = valid ? ld(qp + d) * sl2 : 0.f;
    o[d] = 0.f;
  }
  float m = kNegInf, l = 0.f;
  for (int t = 0; t < N; t += 32) {
    __syncthreads();
    for (int e = threadIdx.x; e < 32 * DD; e += 64) {
      const int k = e / DD, d = e - k * DD, n = t + k;
      float kv = 0.f, vv = 0.f;
      if (n < N) {
        const int64_t r = n < L ? (lo + n) * kvstride : (int64_t(b) * S + (n - L)) * kvstride;
        const T *kbase = n < L ? kc : kb;
        const T *vbase = n < L ? vc : vb;
        kv = ld(kbase + r + int64_t(g) * DD + d);
        vv = ld(vbase + r + int64_t(g) * DD + d);
      }
      Kt[k][d] = kv;
      Vt2[k][d] = vv;
    }
    __syncthreads();
    const int nk = min(32, N - t);
    for (int k = 0; k < nk; ++k) {
      float dot = 0.f;
#pragma unroll
      for (int d = 0; d < DD; ++d) dot = __builtin_fmaf(qv[d], Kt[k][d], dot);
      const float mn = fmaxf(m, dot);
      const float alpha = fast_exp2(m - mn);
      const float p = fast_exp2(dot - mn);
      l = l * alpha + p;
#pragma unroll
      for (int d = 0; d < DD; ++d) o[d] = __builtin_fmaf(p, Vt2[k][d], o[d] * alpha);
      m = mn;
    }
  }
  if (!valid) return;
  T *op = out + ((int64_t(b) * S + s) * Hq + int64_t(g) * G + j) * DD;
  const float inv = 1.0f / l;
#pragma unroll
  for (int d = 0; d < DD; ++d) st(op + d, o[d] * inv);
}

}  // namespace

int launch_attn(const td_attn_args *a, const AttnPlan &p, void *ws, void *stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int max_ctx = int(a->max_ctx);
  if (p.mfma) {
    float *ws_o = reinterpret_cast<float *>(ws);
    float2 *ws_ml = reinterpret_cast<float2 *>(reinterpret_cast<char *>(ws) + p.ws_o_bytes);
    dim3 grid(p.nchunks, a->Hkv * p.row_groups, a->B);
    hipLaunchKernelGGL(attn_bf16_mfma, grid, dim3(kWGThreads), 0, st,
                       static_cast<const bf16 *>(a->q), static_cast<const bf16 *>(a->k_blk),
                       static_cast<const bf16 *>(a->v_blk), static_cast<const bf16 *>(a->k_ctx),
                       static_cast<const bf16 *>(a->v_ctx), a->ctx_offsets, a->total_ctx, max_ctx,
                       a->S, a->Hq, a->Hkv, p.G, p.M, p.row_groups, p.chunk, p.nchunks,
                       p.scale_log2, ws_o, ws_ml, static_cast<bf16 *>(a->out));
    if (p.nchunks > 1) {
      dim3 g2(kRowsPerWG * HD / 4 / 256, unsigned(p.units));
      hipLaunchKernelGGL(attn_combine, g2, dim3(256), 0, st, ws_o, ws_ml, a->ctx_offsets,
                         a->total_ctx, max_ctx, a->S, a->Hq, a->Hkv, p.G, p.M, p.row_groups,
                         p.chunk, p.nchunks, static_cast<bf16 *>(a->out));
    }
  } else {
    dim3 grid(p.row_groups, a->Hkv, a->B);
#define TD_VALU(T, DD)                                                                         \
  hipLaunchKernelGGL((attn_valu<T, DD>), grid, dim3(64), 0, st,                              \
                     static_cast<const T *>(a->q), static_cast<const T *>(a->k_blk),         \
                     static_cast<const T *>(a->v_blk), static_cast<const T *>(a->k_ctx),     \
                     static_cast<const T *>(a->v_ctx), a->ctx_offsets, a->total_ctx, max_ctx, \
                     a->S, a->Hq, a->Hkv, p.G, p.M, p.scale_log2, static_cast<T *>(a->out))
    if (a->dtype == TD_F32) {
      if (a->D == 64) TD_VALU(float, 64); else TD_VALU(float, 128);
    } else {
      if (a->D == 64) TD_VALU(bf16, 64); else TD_VALU(bf16, 128);
    }
#undef TD_VALU
  }
  return hipGetLastError() == hipSuccess ? TD_OK : TD_ERR_HIP;
}

}  // namespace td
