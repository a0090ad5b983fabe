// LM head of the block positions fused with the commit's vocabulary pass, on
// gfx950 (news.chathome.org, "NVIDIA releases Nemotron-Labs-TwoTower ...",
// block-generation and evaluation paragraphs: every denoising step scores the
// vocabulary at each block position, then commits by confidence).
//
// lmhead_tiles: logits^T = W_head . hidden^T on v_mfma_f32_32x32x16_bf16, one
//   256 (vocabulary rows) x 256 (positions) tile per workgroup, fp32
//   accumulation.  The logits never leave the registers: the epilogue reduces
//   each position's 256 logits of the tile to (max, lowest argmax, sum of
//   exp(x - max)), the same partial the commit's vocabulary pass produces,
//   and writes 16 bytes per (position, tile) instead of 512.
//   - Operands stream through a 4-stage LDS ring of 32-wide hidden slices
//     (16 KiB of head rows + 16 KiB of hidden rows per stage) by 16-byte
//     global->LDS DMA; 16-byte chunks are XOR-swizzled per row so that the
//     MFMA operand reads are free of bank conflicts.
//   - 8 waves: wave w covers head rows (w % 4)*64 .. +63 and positions
//     (w / 4)*128 .. +127 of the tile, 2 x 4 blocks of 32 x 32.  In the
//     transposed orientation a lane holds 16 logits of one position per
//     block, so the reduction over the vocabulary is mostly in-lane.
//   - Tiles are numbered with the position tile fastest and dealt to the
//     XCDs in contiguous ranges, so the position tiles that share a slice of
//     the head run together on one XCD and read it from its L2.
// lmhead_merge: one workgroup per position merges the tiles' partials in
//   tile order (deterministic) into one partial, which the commit's
//   per-sequence decision kernel then takes as a single vocabulary part.
#include <hip/hip_runtime.h>

#include "td_internal.h"

namespace td {
namespace {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kTM = 256;          // positions per tile
constexpr int kTN = 256;          // head rows (token ids) per tile
constexpr int kTK = 32;           // hidden units per pipeline stage
constexpr int kStages = 4;
constexpr int kThreads = 512;
constexpr int kRowBytes = kTK * 2;                     // 64 bytes of one row per stage
constexpr int kStageBytes = (kTN + kTM) * kRowBytes;   // 32 KiB
constexpr float kNegInf = -__builtin_inff();
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kNoIndex = 0x7fffffff;

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 16-byte global->LDS DMA of one wave: lane i's 16 bytes from base + voff
// land at LDS byte address lds_base + 16*i.  Written in asm (no outputs) so
// that the compiler neither waits for it nor orders LDS reads behind it;
// completion is checked with explicit vmcnt waits before the barrier that
// publishes a stage.  It sets M0 itself, which is safe while the compiler
// keeps nothing of its own in M0 (checked on the generated assembly by
// tests/test_kernel_asm.py).
__device__ inline void dma16(const void *base, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 sc1 nt\n\ts_nop 1"
               :
               : "s"(lds_base), "v"(voff), "s"(base)
               : "memory", "m0");
}
__device__ inline uint32_t lds_addr(const void *p) {
  return uint32_t(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void *)p));
}
__device__ inline void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}
// Wait until at most n of this wave's DMA instructions are outstanding.
__device__ inline void wait_dma(int n) {
  if (n >= 8) __builtin_amdgcn_s_waitcnt(0xF70 | 8);
  else if (n >= 4) __builtin_amdgcn_s_waitcnt(0xF70 | 4);
  else __builtin_amdgcn_s_waitcnt(0xF70);
}
// chunk swizzle of a 64-byte row: logical 16-byte chunk c of row r sits at
// c ^ ((r >> 2) & 3), so 16 consecutive rows read at one logical chunk hit
// 16 distinct 16-byte bank groups
__device__ inline int swz(int r) { return (r >> 2) & 3; }

// merge (m, z, idx) partials: larger max, then lower index; z rescaled
__device__ inline void merge_part(float &m, float &z, int &idx, float om, float oz, int oi) {
  const float M = fmaxf(m, om);
  if (M == kNegInf) return;                 // both empty
  const float za = (m == kNegInf) ? 0.f : z * fast_exp2((m - M) * kLog2e);
  const float zb = (om == kNegInf) ? 0.f : oz * fast_exp2((om - M) * kLog2e);
  int I = kNoIndex;
  if (m == M) I = idx;
  if (om == M && oi < I) I = oi;
  m = M;
  z = za + zb;
  idx = I;
}

__global__ __launch_bounds__(kThreads, 1) void lmhead_tiles(
    const bf16 *__restrict__ hidden, const bf16 *__restrict__ whead, int M, int V, int H,
    int m_tiles, int n_tiles, Part *__restrict__ parts) {
  __shared__ __attribute__((aligned(1024))) unsigned char ring[kStages * kStageBytes];
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, lq = lane & 31, lh = lane >> 5;
  const int wn = w & 3, wm = w >> 2;

  // XCD-aware tile number: workgroup b runs on XCD b % 8; XCD x takes the
  // contiguous tile range [x*q + min(x, r), ...) of its q or q+1 tiles
  const int nwg = m_tiles * n_tiles;
  const int b = blockIdx.x, x = b & 7, k = b >> 3;
  const int q = nwg >> 3, r8 = nwg & 7;
  const int t = x * q + (x < r8 ? x : r8) + k;
  const int tn = t / m_tiles, tm = t - tn * m_tiles;
  const int n0 = tn * kTN, m0 = tm * kTM;

  // DMA plan: per stage, 16 KiB of head rows (16 wave-instructions of 1 KiB)
  // then 16 KiB of hidden rows; wave w issues head instructions w and w + 8
  // and hidden instructions w and w + 8.  Instruction i fills rows
  // 16i .. 16i+15: lane l writes physical chunk l % 4 of row 16i + l / 4,
  // which holds logical chunk (l % 4) ^ swz(row).  Rows past V or M re-read
  // the last valid row (finite data; those logits are masked or dropped).
  uint32_t voff_w[2], voff_h[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int i = w + 8 * u;
    const int row = 16 * i + (lane >> 2);
    const int c = (lane & 3) ^ swz(row);
    const int rw = min(n0 + row, V - 1) - n0;
    const int rh = min(m0 + row, M - 1) - m0;
    voff_w[u] = uint32_t(rw) * uint32_t(H) * 2u + uint32_t(c) * 16u;
    voff_h[u] = uint32_t(rh) * uint32_t(H) * 2u + uint32_t(c) * 16u;
  }
  const bf16 *wbase = whead + int64_t(n0) * H;
  const bf16 *hbase = hidden + int64_t(m0) * H;
  const uint32_t lds0 = lds_addr(ring);
  const int nk = H / kTK;

  auto issue = [&](int kt) {
    const uint32_t st = lds0 + uint32_t((kt % kStages) * kStageBytes);
    const bf16 *wb = wbase + kt * kTK, *hb = hbase + kt * kTK;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const uint32_t i = uint32_t(w + 8 * u);
      dma16(wb, voff_w[u], __builtin_amdgcn_readfirstlane(st + i * 1024u));
      dma16(hb, voff_h[u], __builtin_amdgcn_readfirstlane(st + uint32_t(kTN * kRowBytes) + i * 1024u));
    }
  };

  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  for (int s = 0; s < kStages - 1 && s < nk; ++s) issue(s);

  for (int kt = 0; kt < nk; ++kt) {
    // stages issued so far: up to min(kt + kStages - 2, nk - 1); this wave
    // has 4 DMA instructions per stage, and stage kt must have landed
    const int ahead = min(kStages - 2, nk - 1 - kt);
    wait_dma(4 * ahead);
    lds_barrier();                 // stage kt visible; stage kt-1 free for reuse
    if (kt + kStages - 1 < nk) issue(kt + kStages - 1);
    const unsigned char *st = ring + (kt % kStages) * kStageBytes;
    const unsigned char *wl = st, *hl = st + kTN * kRowBytes;
#pragma unroll
    for (int ks = 0; ks < kTK / 16; ++ks) {
      const int c = ks * 2 + lh;
      bf16x8 a[2], bb[4];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = wn * 64 + i * 32 + lq;
        a[i] = *reinterpret_cast<const bf16x8 *>(wl + row * kRowBytes + ((c ^ swz(row)) * 16));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = wm * 128 + j * 32 + lq;
        bb[j] = *reinterpret_cast<const bf16x8 *>(hl + row * kRowBytes + ((c ^ swz(row)) * 16));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], bb[j], acc[i][j], 0, 0, 0);
    }
  }

  // ---- epilogue: per position, (max, lowest argmax, sum exp) over the tile
  // acc[i][j] element e of lane (lq, lh): head row n0 + wn*64 + i*32 +
  // (e >> 2)*8 + lh*4 + (e & 3), position m0 + wm*128 + j*32 + lq
  float pm[4], pz[4];
  int pi[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float mx = kNegInf;
    int id = kNoIndex;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int n = n0 + wn * 64 + i * 32 + (e >> 2) * 8 + lh * 4 + (e & 3);
        const float v = n < V ? acc[i][j][e] : kNegInf;
        acc[i][j][e] = v;
        if (v > mx) { mx = v; id = n; }     // n increases along (i, e): first max wins
      }
    float z = 0.f;
    if (mx != kNegInf) {
      const float mc = mx * kLog2e;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) z += fast_exp2(__builtin_fmaf(acc[i][j][e], kLog2e, -mc));
    }
    // the other lane half holds the other head rows of the same position
    merge_part(mx, z, id, __shfl_xor(mx, 32), __shfl_xor(z, 32), __shfl_xor(id, 32));
    pm[j] = mx; pz[j] = z; pi[j] = id;
  }
  lds_barrier();                   // every wave is done with the ring
  float *red_m = reinterpret_cast<float *>(ring);                 // [4][kTM]
  float *red_z = red_m + 4 * kTM;
  int *red_i = reinterpret_cast<int *>(red_z + 4 * kTM);
  if (lh == 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int p = wm * 128 + j * 32 + lq;
      red_m[wn * kTM + p] = pm[j];
      red_z[wn * kTM + p] = pz[j];
      red_i[wn * kTM + p] = pi[j];
    }
  }
  lds_barrier();
  if (tid < kTM && m0 + tid < M) {
    float mx = red_m[tid], z = red_z[tid];
    int id = red_i[tid];
#pragma unroll
    for (int g = 1; g < 4; ++g) merge_part(mx, z, id, red_m[g * kTM + tid], red_z[g * kTM + tid], red_i[g * kTM + tid]);
    Part pt;
    pt.m = mx; pt.z = z; pt.idx = id; pt.pad = 0;
    parts[int64_t(m0 + tid) * n_tiles + tn] = pt;
  }
}

// One workgroup per position: the n_tiles partials, merged in tile order.
__global__ __launch_bounds__(256) void lmhead_merge(const Part *__restrict__ parts, int n_tiles,
                                                   Part *__restrict__ merged,
                                                   int32_t *__restrict__ n_masked_left) {
  const int row = blockIdx.x, tid = threadIdx.x;
  if (row == 0 && tid == 0 && n_masked_left) *n_masked_left = 0;
  float m = kNegInf, z = 0.f;
  int idx = kNoIndex;
  for (int t = tid; t < n_tiles; t += 256) {
    const Part p = parts[int64_t(row) * n_tiles + t];
    merge_part(m, z, idx, p.m, p.z, p.idx);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1)
    merge_part(m, z, idx, __shfl_xor(m, o), __shfl_xor(z, o), __shfl_xor(idx, o));
  __shared__ float sm[4], sz[4];
  __shared__ int si[4];
  if ((tid & 63) == 0) { sm[tid >> 6] = m; sz[tid >> 6] = z; si[tid >> 6] = idx; }
  __syncthreads();
  if (tid == 0) {
    float M = sm[0], Z = sz[0];
    int I = si[0];
    for (int g = 1; g < 4; ++g) merge_part(M, Z, I, sm[g], sz[g], si[g]);
    Part p;
    p.m = M; p.z = Z; p.idx = I; p.pad = 0;
    merged[row] = p;
  }
}

}  // namespace

size_t lmhead_parts_bytes(const td_lmhead_args *a) {
  const int64_t M = int64_t(a->B) * a->S;
  const int64_t n_tiles = (int64_t(a->V) + kTN - 1) / kTN;
  return size_t(M * n_tiles) * sizeof(Part);
}

int launch_lmhead(const td_lmhead_args *a, void *ws, void *stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int M = a->B * a->S;
  const int m_tiles = (M + kTM - 1) / kTM;
  const int n_tiles = (a->V + kTN - 1) / kTN;
  Part *parts = reinterpret_cast<Part *>(ws);
  Part *merged = reinterpret_cast<Part *>(static_cast<char *>(ws) + align256(lmhead_parts_bytes(a)));
  hipLaunchKernelGGL(lmhead_tiles, dim3(unsigned(m_tiles * n_tiles)), dim3(kThreads), 0, st,
                     static_cast<const bf16 *>(a->hidden), static_cast<const bf16 *>(a->w_head), M,
                     a->V, a->H, m_tiles, n_tiles, parts);
  hipLaunchKernelGGL(lmhead_merge, dim3(unsigned(M)), dim3(256), 0, st, parts, n_tiles, merged,
                     a->n_masked_left);
  if (hipGetLastError() != hipSuccess) return TD_ERR_HIP;
  return launch_commit_finalize(merged, 1, a->B, a->S, a->gamma, a->masked_in, a->commit, a->token,
                                a->maxprob, a->n_commit, a->masked_out, a->tokens,
                                a->n_masked_left, stream);
}

}  // namespace td
