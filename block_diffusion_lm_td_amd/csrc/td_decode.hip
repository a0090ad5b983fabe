// Attention for decode-shaped blocks on gfx950: at most 16 query rows per KV
// head (G heads x S positions, G*S <= 16), as in the one-token AR and mock-AR
// decoding of the TwoTower model (news.chathome.org, "NVIDIA releases
// Nemotron-Labs-TwoTower ...", modes paragraph; inference paragraph for the
// attention itself: one softmax over [context cache ; block]).
//
// With so few rows per KV head the 256-row MFMA tiles of the block kernel
// are mostly empty, and the work is one pass over the context cache: a
// stream, bound by HBM.  Here v_mfma_f32_16x16x32_bf16 is filled exactly by
// the 16 query rows, and the key range of every (sequence, KV head) is cut
// into pieces of kDecodePieceKeys keys, one per wave:
//   - Each 32-key block comes from HBM into registers with ordinary 16-byte
//     loads: K already in the MFMA operand layout (each lane 16 bytes of one
//     key row per MFMA), V in 16-byte chunks.  Two register sets alternate,
//     so every wave keeps the next block in flight while it works on the
//     current one (a stream needs many bytes in flight; the register file
//     holds them, the LDS only the one block being transposed).
//   - S^T = K Q^T in 16-key tiles.
//   - O^T += V^T P^T: the V block goes into the wave's own LDS slot (no
//     barriers), row-major with 16-byte chunks XOR-swizzled by 2*(row % 8),
//     and comes back transposed through gfx950's 8-byte transposing LDS
//     reads.  P^T needs no data movement: the lane that holds a query's
//     scores for keys 4g..4g+3 of both 16-key tiles is the lane whose PV
//     operand takes those 8 keys.
//   - Online softmax in fp32 (exp2 domain); each piece writes (m, l) in fp32
//     and O / l in bf16 to the workspace.
// decode_merge: one workgroup per (sequence, KV head, query row) merges the
//   pieces (deterministic order) and writes out in the input dtype.
#include <hip/hip_runtime.h>

#include "td_internal.h"

namespace td {
namespace {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

constexpr int HD = 128;
constexpr int kPiece = kDecodePieceKeys;   // keys per wave-piece
constexpr int kBlk = 32;                   // keys per step
constexpr int kDecWaves = 4;
constexpr float kNegInf = -__builtin_inff();

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
// two floats -> two bf16 (round to nearest even), low half first
__device__ inline uint32_t pack_bf16(float a, float b) {
  const bf16 x = bf16(a), y = bf16(b);
  return uint32_t(__builtin_bit_cast(uint16_t, x)) | (uint32_t(__builtin_bit_cast(uint16_t, y)) << 16);
}

__device__ inline int64_t clamp64(int64_t x, int64_t lo, int64_t hi) {
  return x < lo ? lo : (x > hi ? hi : x);
}
// clamped range of sequence b, as the block kernel reads it
__device__ inline void seq_lo_len(const int64_t *off, int b, int64_t total, int max_ctx,
                                  int64_t &lo, int &L) {
  lo = clamp64(off[b], 0, total);
  const int64_t hi = clamp64(off[b + 1], lo, total);
  L = int(hi - lo < max_ctx ? hi - lo : max_ctx);
}
__device__ inline int pieces_of(int L, int S) { return (L + S + kPiece - 1) / kPiece; }

// One wave per piece: pieces are numbered g * T1 + (pre[b] + u) for KV head
// g, sequence b and piece u of that sequence, with pre[b] the pieces of
// sequences 0 .. b-1 and T1 = pre[B].  Every workgroup scans the table into
// LDS (B <= kDecodeMaxB); workgroup 0 also leaves it in the workspace for
// the merge.
__global__ __launch_bounds__(kDecWaves * 64, 2) void attn_decode(
    const bf16 *__restrict__ q, const bf16 *__restrict__ kb, const bf16 *__restrict__ vb,
    const bf16 *__restrict__ kc, const bf16 *__restrict__ vc, const int64_t *__restrict__ off,
    int64_t total, int max_ctx, int B, int S, int Hq, int Hkv, int G, float sl2,
    int64_t *__restrict__ pre, int64_t P_max, bf16 *__restrict__ ws_o,
    float2 *__restrict__ ws_ml, const int32_t *__restrict__ gate) {
  if (gate && *gate == 0) return;
  __shared__ __attribute__((aligned(1024))) bf16 vbuf[kDecWaves * kBlk * HD];
  __shared__ int s_pre[kDecodeMaxB + 1];
  __shared__ int s_wsum[kDecWaves];
  const int tid = threadIdx.x;
  const int wv = tid >> 6, lane = tid & 63;
  const int n16 = lane & 15, g4 = lane >> 4;
  {
    int base = 0;
    for (int c0 = 0; c0 < B; c0 += kDecWaves * 64) {
      const int bb = c0 + tid;
      int n = 0;
      if (bb < B) {
        int64_t lo_;
        int L_;
        seq_lo_len(off, bb, total, max_ctx, lo_, L_);
        n = pieces_of(L_, S);
      }
      int x = n;                                // inclusive scan in the wave
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o);
        if (lane >= o) x += y;
      }
      if (lane == 63) s_wsum[wv] = x;
      __syncthreads();
      int before = 0, all = 0;
#pragma unroll
      for (int k = 0; k < kDecWaves; ++k) {
        before += k < wv ? s_wsum[k] : 0;
        all += s_wsum[k];
      }
      if (bb < B) s_pre[bb] = base + before + x - n;
      __syncthreads();
      base += all;
    }
    if (tid == 0) s_pre[B] = base;
    __syncthreads();
    if (blockIdx.x == 0)
      for (int i = tid; i <= B; i += kDecWaves * 64) pre[i] = s_pre[i];
  }
  const int64_t T1 = s_pre[B];
  const int64_t pi = int64_t(blockIdx.x) * kDecWaves + wv;
  // past the last piece; P_max (the workspace's capacity) only binds for
  // inconsistent offsets.  No barriers below.
  if (pi >= (T1 * Hkv < P_max ? T1 * Hkv : P_max)) return;
  const int g = int(pi / T1);
  const int64_t j = pi - int64_t(g) * T1;
  int lo_b = 0, hi_b = B;                       // sequence: last b with pre[b] <= j
  while (hi_b - lo_b > 1) {
    const int mid = (lo_b + hi_b) >> 1;
    if (s_pre[mid] <= j) lo_b = mid;
    else hi_b = mid;
  }
  const int b = lo_b;
  const int u = int(j - s_pre[b]);
  int64_t lo;
  int L;
  seq_lo_len(off, b, total, max_ctx, lo, L);
  const int nkeys = L + S;
  const int k0 = u * kPiece;
  const int k1 = min(k0 + kPiece, nkeys);

  // Q^T operand (B of S^T = K Q^T): lane -> query row n16 (s = n16 / G,
  // h = n16 % G), dims 8*g4 + 32*kk .. +7; rows past G*S are zero
  bf16x8 qt[4];
  {
    const int M = G * S;
    const bool ok = n16 < M;
    const int s = ok ? n16 / G : 0, h = ok ? n16 - (n16 / G) * G : 0;
    const bf16 *qr = q + ((int64_t(b) * S + s) * Hq + int64_t(g) * G + h) * HD + 8 * g4;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      qt[kk] = ok ? *reinterpret_cast<const bf16x8 *>(qr + 32 * kk) : bf16x8{};
  }
  // row pointer of key k of this (b, g): cache rows first, then the block
  auto krow = [&](const bf16 *ctx, const bf16 *blk, int k) -> const bf16 * {
    return k < L ? ctx + ((lo + k) * Hkv + g) * HD
                 : blk + ((int64_t(b) * S + (k - L)) * Hkv + g) * HD;
  };
  // One 32-key block in registers: the K operand (tiles t = 0, 1; dims
  // 32*kk + 8*g4; lane key kbase + 16t + n16) and 16-byte chunks of V (chunk
  // n16 of row 4i + g4), keys clamped to the piece (masked below)
  struct Blk {
    bf16x8 k[2][4];
    bf16x8 v[8];
  };
  auto load_blk = [&](int kbase, Blk &x) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const bf16 *r = krow(kc, kb, min(kbase + 16 * t + n16, k1 - 1)) + 8 * g4;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) x.k[t][kk] = *reinterpret_cast<const bf16x8 *>(r + 32 * kk);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = 4 * i + g4;
      x.v[i] = *reinterpret_cast<const bf16x8 *>(krow(vc, vb, min(kbase + row, k1 - 1)) + n16 * 8);
    }
  };
  bf16 *vl = vbuf + wv * kBlk * HD;             // this wave's V block, row-major, swizzled

  f32x4 o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) o[dt] = f32x4{};
  float m = kNegInf, l = 0.f;
  const int nblk = (k1 - k0 + kBlk - 1) / kBlk;

  // block jb from registers x: V into LDS, scores, softmax, PV
  auto step = [&](int jb, const Blk &x) {
    const int kbase = k0 + jb * kBlk;
    // V rows into the wave's slot: logical chunk n16 of row r at n16 ^ 2*(r % 8)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = 4 * i + g4;
      *reinterpret_cast<bf16x8 *>(vl + row * HD + ((n16 ^ (2 * (row & 7))) * 8)) = x.v[i];
    }
    // scores of the two 16-key tiles: lane -> query n16, keys 4*g4 + i
    f32x4 s[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      s[t] = f32x4{};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        s[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x.k[t][kk], qt[kk], s[t], 0, 0, 0);
    }
    float mx = kNegInf;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int k = kbase + 16 * t + 4 * g4 + i;
        s[t][i] = k < k1 ? s[t][i] * sl2 : kNegInf;
        mx = fmaxf(mx, s[t][i]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mn = fmaxf(m, mx);              // finite: every block holds a key
    const float alpha = fast_exp2(m - mn);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[dt] *= alpha;
    l *= alpha;
    m = mn;
    // P^T operand: keys 8*g4 + i are tile 0 rows 4*g4 + i (i < 4) and tile 1
    // rows 4*g4 + i - 4 (i >= 4), both already in this lane
    bf16x8 pt;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p0 = fast_exp2(s[0][i] - mn), p1 = fast_exp2(s[1][i] - mn);
      l += p0 + p1;
      pt[i] = bf16(p0);
      pt[4 + i] = bf16(p1);
    }
    // V^T operand of D tile dt: keys 8*g4 + i (rows 4*g4 + e, then 16 + 4*g4
    // + e), dims 16*dt + n16; source lane 4e + a of a 16-lane group addresses
    // row (.. + e), dims 16*dt + 4a .. +3
    const int e = n16 >> 2, a = n16 & 3;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const int r0 = 4 * g4 + e, r1 = 16 + 4 * g4 + e;
      const int cidx = 2 * dt + (a >> 1), half = (a & 1) * 4;
      const bf16 *p0 = vl + r0 * HD + ((cidx ^ (2 * (r0 & 7))) * 8) + half;
      const bf16 *p1 = vl + r1 * HD + ((cidx ^ (2 * (r1 & 7))) * 8) + half;
      const s16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)p0);
      const s16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)p1);
      const u32x2 a0 = __builtin_bit_cast(u32x2, x0), a1 = __builtin_bit_cast(u32x2, x1);
      const u32x4 a01 = {a0.x, a0.y, a1.x, a1.y};
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a01), pt, o[dt], 0, 0, 0);
    }
  };
  // two register sets: block jb + 1 loads while block jb is processed
  Blk b0, b1;
  load_blk(k0, b0);
  for (int jb = 0; jb < nblk; jb += 2) {
    if (jb + 1 < nblk) load_blk(k0 + (jb + 1) * kBlk, b1);
    step(jb, b0);
    if (jb + 1 >= nblk) break;
    if (jb + 2 < nblk) load_blk(k0 + (jb + 2) * kBlk, b0);
    step(jb + 1, b1);
  }
  // l: the four lanes of a query hold disjoint keys
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  // partial: O^T / l in bf16 (lane -> query n16, dims 16*dt + 4*g4 + i) and
  // (m, l) in fp32
  const float inv = 1.0f / l;
  bf16 *po = ws_o + pi * (16 * HD) + n16 * HD + 4 * g4;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    const f32x4 v = o[dt] * inv;
    *reinterpret_cast<uint2 *>(po + 16 * dt) =
        make_uint2(pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]));
  }
  if (g4 == 0) ws_ml[pi * 16 + n16] = make_float2(m, l);
}

// One workgroup per (sequence, KV head, query row): 8 groups of 32 threads
// (each thread 4 dims) take every eighth piece, merge their share online
// with all its loads in flight at once, and the 8 group results are merged
// in group order through LDS (deterministic).
__global__ __launch_bounds__(256) void decode_merge(
    int B, int S, int Hq, int Hkv, int G, const int64_t *__restrict__ pre, int64_t P_max,
    const bf16 *__restrict__ ws_o, const float2 *__restrict__ ws_ml, bf16 *__restrict__ out,
    const int32_t *__restrict__ gate) {
  if (gate && *gate == 0) return;
  const int n = blockIdx.x & 15, unit = blockIdx.x >> 4;
  const int M = G * S;
  if (n >= M) return;                           // uniform per workgroup: no barrier is skipped
  const int b = unit / Hkv, g = unit - (unit / Hkv) * Hkv;
  const int64_t T1 = pre[B];
  int64_t p0 = int64_t(g) * T1 + pre[b], p1 = int64_t(g) * T1 + pre[b + 1];
  p0 = p0 < P_max ? p0 : P_max;                 // binds only for inconsistent offsets
  p1 = p1 < P_max ? p1 : P_max;
  const int tid = threadIdx.x, d = (tid & 31) * 4, grp = tid >> 5;
  constexpr int kBatch = 8;
  float mm = kNegInf, ls = 0.f;
  f32x4 acc = f32x4{};
  for (int64_t pb = p0 + grp; pb < p1; pb += 8 * kBatch) {
    float2 ml[kBatch];
    uint2 ov[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int64_t p = pb + 8 * i < p1 ? pb + 8 * i : pb;
      ml[i] = ws_ml[p * 16 + n];
      ov[i] = *reinterpret_cast<const uint2 *>(ws_o + p * (16 * HD) + n * HD + d);
    }
    float bm = mm;
#pragma unroll
    for (int i = 0; i < kBatch; ++i)
      if (pb + 8 * i < p1) bm = fmaxf(bm, ml[i].x);
    const float r = fast_exp2(mm - bm);         // 0 while mm is -inf
    acc *= r;
    ls *= r;
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      if (pb + 8 * i >= p1) continue;
      const float wl = fast_exp2(ml[i].x - bm) * ml[i].y;
      const f32x4 v = {__uint_as_float(ov[i].x << 16), __uint_as_float(ov[i].x & 0xffff0000u),
                       __uint_as_float(ov[i].y << 16), __uint_as_float(ov[i].y & 0xffff0000u)};
      acc += wl * v;
      ls += wl;
    }
    mm = bm;
  }
  __shared__ float s_m[8][32], s_l[8][32];
  __shared__ f32x4 s_a[8][32];
  s_m[grp][tid & 31] = mm;
  s_l[grp][tid & 31] = ls;
  s_a[grp][tid & 31] = acc;
  __syncthreads();
  if (grp != 0) return;
  float M_ = kNegInf;
#pragma unroll
  for (int k = 0; k < 8; ++k) M_ = fmaxf(M_, s_m[k][tid]);
  float L_ = 0.f;
  f32x4 A = f32x4{};
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    if (s_m[k][tid] == kNegInf) continue;       // a group without pieces
    const float w = fast_exp2(s_m[k][tid] - M_);
    L_ += w * s_l[k][tid];
    A += w * s_a[k][tid];
  }
  const float inv = 1.0f / L_;
  const int s = n / G, h = n - (n / G) * G;
  bf16 *dst = out + ((int64_t(b) * S + s) * Hq + int64_t(g) * G + h) * HD + d;
  *reinterpret_cast<uint2 *>(dst) =
      make_uint2(pack_bf16(A[0] * inv, A[1] * inv), pack_bf16(A[2] * inv, A[3] * inv));
}

}  // namespace

int launch_attn_decode(const td_attn_args *a, const AttnPlan &p, void *ws, void *stream,
                       const int32_t *gate) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char *w = static_cast<char *>(ws);
  int64_t *pre = reinterpret_cast<int64_t *>(w + p.off_prefix);
  float2 *ml = reinterpret_cast<float2 *>(w + p.off_ml);
  bf16 *o = reinterpret_cast<bf16 *>(w + p.off_o);
  const int max_ctx = int(a->max_ctx);
  const int64_t waves = p.units;                // upper bound of pieces (all KV heads)
  hipLaunchKernelGGL(attn_decode, dim3(unsigned((waves + kDecWaves - 1) / kDecWaves)),
                     dim3(kDecWaves * 64), 0, st, static_cast<const bf16 *>(a->q),
                     static_cast<const bf16 *>(a->k_blk), static_cast<const bf16 *>(a->v_blk),
                     static_cast<const bf16 *>(a->k_ctx), static_cast<const bf16 *>(a->v_ctx),
                     a->ctx_offsets, a->total_ctx, max_ctx, a->B, a->S, a->Hq, a->Hkv, p.G,
                     p.scale_log2, pre, waves, o, ml, gate);
  hipLaunchKernelGGL(decode_merge, dim3(unsigned(a->B * a->Hkv * 16)), dim3(256), 0, st, a->B,
                     a->S, a->Hq, a->Hkv, p.G, pre, waves, o, ml, static_cast<bf16 *>(a->out),
                     gate);
  return hipGetLastError() == hipSuccess ? TD_OK : TD_ERR_HIP;
}

}  // namespace td
