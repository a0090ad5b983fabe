// LM head of the block positions fused with the commit's vocabulary pass, on
// gfx950 (news.chathome.org, "NVIDIA releases Nemotron-Labs-TwoTower ...",
// block-generation and evaluation paragraphs: every denoising step scores the
// vocabulary at each block position, then commits by confidence).
//
// lmhead_tiles: logits^T = W_head . hidden^T on v_mfma_f32_16x16x32_bf16, one
//   256 (vocabulary rows) x 256 (positions) tile per workgroup, fp32
//   accumulation.  The logits never leave the registers: the epilogue reduces
//   each position's 256 logits of the tile to (max, lowest argmax, sum of
//   exp(x - max)), the same partial the commit's vocabulary pass produces,
//   and writes 16 bytes per (position, tile) instead of 512.
//   - Operands stream through a 2-stage LDS ring of 64-wide hidden slices
//     (32 KiB of head rows + 32 KiB of hidden rows per stage, one 128-byte
//     line per row) by 16-byte global->LDS DMA; 16-byte chunks are
//     XOR-swizzled per row so that the MFMA operand reads are free of bank
//     conflicts.
//   - 16 waves, four per SIMD: wave w covers head rows (w % 4)*64 .. +63 and
//     positions (w / 4)*64 .. +63 of the tile, 4 x 4 blocks of 16 x 16.  In
//     the transposed orientation a lane holds 4 logits of one position per
//     block, 16 per position over the wave's head rows, so the reduction
//     over the vocabulary is mostly in-lane.
//   - The 16x16x32 shape reads the same LDS bytes per flop as 32x32x16 with
//     this 64 x 64 wave tile and the same accumulator registers, and at this
//     chip's power limit it sustains more flops (a bare loop on random
//     operands: 1.92 against 1.77 PF/s, at lower energy per flop).
//   - Tiles are numbered with the position tile fastest and dealt to the
//     XCDs in contiguous ranges, so the position tiles that share a slice of
//     the head run together on one XCD and read it from its L2.
//   - When 128-position tiles pad the positions less (at most 128 left, a
//     block's late steps, or 257 .. 384) the tiles are 256 x 128 with a
//     3-stage ring of 48 KiB stages: two head stages stay in flight instead
//     of one, and no half-empty position tile is computed.  At 103 positions
//     a call goes from about 258 to 192 us, at 266 from 457 to 421 us.
//   Measured at 64 x 16 positions, H = 4096, V = 131072, every position
//   scored (median of 7 x 20 launches of td_lmhead_commit): 879 us, against
//   927 us for the same tiles on 32x32x16 blocks.  Earlier 32x32x16 layouts:
//   32-wide slices in a 4-stage ring, 8 waves of 64 x 128: 1154 us; 4 waves
//   of 128 x 128: 1246 us.
// lmhead_merge: one workgroup per position merges the tiles' partials in
//   tile order (deterministic) into one partial, which the commit's
//   per-sequence decision kernel then takes as a single vocabulary part.
#include <hip/hip_runtime.h>

#include "td_internal.h"

namespace td {
namespace {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kTM = 256;
constexpr int kTN = 256;
constexpr int kTK = 64;           // hidden units per pipeline stage: 128-byte rows
constexpr int kStages = 2;        // double buffer: 2 x 64 KiB of LDS
constexpr int kWaves = 16;        // 4 per SIMD; wave tile 64 head rows x 64 positions
constexpr int kThreads = 64 * kWaves;
constexpr int kGrid = 256;        // persistent: one workgroup per CU of MI355X
constexpr int kRowBytes = kTK * 2;
constexpr int kStageBytes = (kTN + kTM) * kRowBytes;
constexpr int kTMSmall = 128;     // positions per tile of the smaller (3-stage) tiles
constexpr int kRingBytes = kStages * kStageBytes > 3 * (kTN + kTMSmall) * kRowBytes
                               ? kStages * kStageBytes
                               : 3 * (kTN + kTMSmall) * kRowBytes;
constexpr int kRPB = 256 / kRowBytes;          // rows per 256 bytes
constexpr int kCPR = kRowBytes / 16;           // 16-byte chunks per row
constexpr int kRPI = 1024 / kRowBytes;         // rows per 1 KiB DMA instruction
constexpr int kInstr = kTN * kRowBytes / 1024; // DMA instructions per operand per stage
constexpr int kIPW = kInstr / kWaves;          // head DMA instructions per wave and stage
constexpr int WN = 4, WM = kWaves / 4;
constexpr int TNW = kTN / WN;                  // head rows per wave
constexpr int kMB = 16;                        // v_mfma_f32_16x16x32_bf16 blocks
constexpr int NI = TNW / kMB;
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
// tests/test_kernel_asm.py).  The head slice is re-read by the other
// position tiles and the hidden rows by every head tile, through L2: no
// non-temporal hint (sc1 only: 932 us against 951 us with nt at the batched
// step's shape).
__device__ inline void dma16(const void *base, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 sc1\n\ts_nop 1"
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
template <int PER>
__device__ inline void wait_dma(int ahead) {
  // at most PER * ahead of this wave's DMA instructions outstanding (ahead <= 2)
  if (ahead >= 2) {
    if constexpr (2 * PER >= 16) __builtin_amdgcn_s_waitcnt((0xF70 | ((2 * PER) & 15)) | (((2 * PER) >> 4) << 14));
    else __builtin_amdgcn_s_waitcnt(0xF70 | (2 * PER));
  } else if (ahead == 1) {
    if constexpr (PER >= 16) __builtin_amdgcn_s_waitcnt((0xF70 | (PER & 15)) | ((PER >> 4) << 14));
    else __builtin_amdgcn_s_waitcnt(0xF70 | PER);
  } else {
    __builtin_amdgcn_s_waitcnt(0xF70);
  }
}
__device__ inline int swz(int r) { return (r / kRPB) % kCPR; }
__device__ inline void merge_part(float &m, float &z, int &idx, float om, float oz, int oi) {
  const float M = fmaxf(m, om);
  if (M == kNegInf) return;
  const float za = (m == kNegInf) ? 0.f : z * fast_exp2((m - M) * kLog2e);
  const float zb = (om == kNegInf) ? 0.f : oz * fast_exp2((om - M) * kLog2e);
  int I = kNoIndex;
  if (m == M) I = idx;
  if (om == M && oi < I) I = oi;
  m = M;
  z = za + zb;
  idx = I;
}

// Positions still to score, in order: rows[0 .. *count) lists every i with
// masked[i] != 0 (one workgroup, a ballot scan per 1024 positions).
__global__ __launch_bounds__(1024) void lmhead_compact(const uint8_t *__restrict__ masked, int M,
                                                      int32_t *__restrict__ rows,
                                                      int32_t *__restrict__ count) {
  __shared__ int wsum[16];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  int base = 0;
  for (int c0 = 0; c0 < M; c0 += 1024) {
    const int i = c0 + tid;
    const bool f = i < M && masked[i] != 0;
    const unsigned long long bal = __ballot(f);
    const int pre = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) wsum[w] = __popcll(bal);
    __syncthreads();
    int off = 0, tot = 0;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      off += k < w ? wsum[k] : 0;
      tot += wsum[k];
    }
    if (f) rows[base + off + pre] = i;
    __syncthreads();
    base += tot;
  }
  if (tid == 0) *count = base;
}

// Persistent: one workgroup per CU (kGrid, a multiple of 8) loops over the
// tiles.  rows / count: the compacted positions (NULL: all M positions in
// order); only the ceil(count / TM) position tiles that hold positions are
// visited.  Tiles are numbered with the position tile fastest; XCD x (the
// workgroups b with b % 8 == x) takes a contiguous range of them, its
// workgroups in turn, so the position tiles of one head slice run at the
// same time on one XCD and share the slice through its L2.
//
// TM positions per tile: 256 with a 2-stage ring of 64 KiB stages, or 128
// with a 3-stage ring of 48 KiB stages (each wave 64 head rows x 32
// positions), which keeps two stages of the head in flight instead of one.
template <bool kPacked, int TM>
__device__ __forceinline__ void tiles_body(unsigned char *ring, const bf16 *__restrict__ hidden,
                                           const bf16 *__restrict__ whead, int Mc, int V, int H,
                                           int n_tiles, const int32_t *__restrict__ rows,
                                           Part *__restrict__ parts) {
  constexpr int NST = TM == kTM ? kStages : 3;           // ring stages
  constexpr int SB = (kTN + TM) * kRowBytes;             // bytes per stage
  constexpr int IPWH = TM * kRowBytes / 1024 / kWaves;   // hidden DMA instructions per wave
  constexpr int TMWv = TM / WM, NJv = TMWv / kMB;
  static_assert(NST * SB <= kRingBytes && IPWH >= 1 && NJv >= 1, "tile shape");
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, l16 = lane & 15, l4 = lane >> 4;
  const int wn = w % WN, wm = w / WN;
  const int m_act = (Mc + TM - 1) / TM;
  const int n_act = m_act * n_tiles;
  const int x = blockIdx.x & 7, px = blockIdx.x >> 3, PX = gridDim.x >> 3;
  const int q = n_act >> 3, r8 = n_act & 7;
  const int x_lo = x * q + (x < r8 ? x : r8), x_n = q + (x < r8 ? 1 : 0);
  for (int j = px; j < x_n; j += PX) {
    const int t = x_lo + j;
    const int tn = t / m_act, tm = t - tn * m_act;
    const int n0 = tn * kTN, m0 = tm * TM;
    uint32_t voff_w[kIPW], voff_h[IPWH];
#pragma unroll
    for (int u = 0; u < kIPW; ++u) {
      const int i = w + kWaves * u;
      const int row = kRPI * i + lane / kCPR;
      const int c = (lane % kCPR) ^ swz(row);
      const int rw = min(n0 + row, V - 1) - n0;     // row-major: rows past V re-read row V-1
      // packed: the stage's 256 x 64 block is contiguous, rows past V are zeros
      voff_w[u] = kPacked ? uint32_t(row) * uint32_t(kRowBytes) + uint32_t(c) * 16u
                          : uint32_t(rw) * uint32_t(H) * 2u + uint32_t(c) * 16u;
    }
#pragma unroll
    for (int u = 0; u < IPWH; ++u) {
      const int i = w + kWaves * u;
      const int row = kRPI * i + lane / kCPR;
      const int c = (lane % kCPR) ^ swz(row);
      const int cm = min(m0 + row, Mc - 1);
      const int rh = rows ? rows[cm] : cm;        // hidden row of this position
      voff_h[u] = uint32_t(rh) * uint32_t(H) * 2u + uint32_t(c) * 16u;
    }
    const bf16 *wbase = whead + int64_t(n0) * H;
    const bf16 *hbase = hidden;
    const uint32_t lds0 = lds_addr(ring);
    const int nk = H / kTK;
    auto issue = [&](int kt) {
      const uint32_t st = lds0 + uint32_t((kt % NST) * SB);
      const bf16 *wb = kPacked ? whead + (int64_t(tn) * nk + kt) * (kTN * kTK) : wbase + kt * kTK;
      const bf16 *hb = hbase + kt * kTK;
#pragma unroll
      for (int u = 0; u < kIPW; ++u) {
        const uint32_t i = uint32_t(w + kWaves * u);
        dma16(wb, voff_w[u], __builtin_amdgcn_readfirstlane(st + i * 1024u));
      }
#pragma unroll
      for (int u = 0; u < IPWH; ++u) {
        const uint32_t i = uint32_t(w + kWaves * u);
        dma16(hb, voff_h[u], __builtin_amdgcn_readfirstlane(st + uint32_t(kTN * kRowBytes) + i * 1024u));
      }
    };
    f32x4 acc[NI][NJv];
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int j = 0; j < NJv; ++j) acc[i][j] = f32x4{};
    for (int s = 0; s < NST - 1 && s < nk; ++s) issue(s);
    for (int kt = 0; kt < nk; ++kt) {
      const int ahead = min(NST - 2, nk - 1 - kt);
      wait_dma<kIPW + IPWH>(ahead);  // this wave's part of stage kt has landed
      lds_barrier();                 // all of stage kt visible; stage kt-1 free for reuse
      if (kt + NST - 1 < nk) issue(kt + NST - 1);
      const unsigned char *st = ring + (kt % NST) * SB;
      const unsigned char *wl = st, *hl = st + kTN * kRowBytes;
      // lane: row l16 of each 16-row block, hidden units ks*32 + 8*l4 .. +7
#pragma unroll
      for (int ks = 0; ks < kTK / 32; ++ks) {
        const int c = ks * 4 + l4;
        bf16x8 a[NI], bb[NJv];
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          const int row = wn * TNW + i * kMB + l16;
          a[i] = *reinterpret_cast<const bf16x8 *>(wl + row * kRowBytes + ((c ^ swz(row)) * 16));
        }
#pragma unroll
        for (int j = 0; j < NJv; ++j) {
          const int row = wm * TMWv + j * kMB + l16;
          bb[j] = *reinterpret_cast<const bf16x8 *>(hl + row * kRowBytes + ((c ^ swz(row)) * 16));
        }
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
          for (int j = 0; j < NJv; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], bb[j], acc[i][j], 0, 0, 0);
      }
    }
    // lane: position l16 of each 16-position block, head rows 4*l4 .. +3 of
    // each 16-row block
    float pm[NJv], pz[NJv];
    int pi[NJv];
#pragma unroll
    for (int j = 0; j < NJv; ++j) {
      float mx = kNegInf;
      int id = kNoIndex;
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int n = n0 + wn * TNW + i * kMB + l4 * 4 + e;
          const float v = n < V ? acc[i][j][e] : kNegInf;
          acc[i][j][e] = v;
          if (v > mx) { mx = v; id = n; }
        }
      float z = 0.f;
      if (mx != kNegInf) {
        const float mc = mx * kLog2e;
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e) z += fast_exp2(__builtin_fmaf(acc[i][j][e], kLog2e, -mc));
      }
      merge_part(mx, z, id, __shfl_xor(mx, 16), __shfl_xor(z, 16), __shfl_xor(id, 16));
      merge_part(mx, z, id, __shfl_xor(mx, 32), __shfl_xor(z, 32), __shfl_xor(id, 32));
      pm[j] = mx; pz[j] = z; pi[j] = id;
    }
    lds_barrier();
    float *red_m = reinterpret_cast<float *>(ring);
    float *red_z = red_m + WN * TM;
    int *red_i = reinterpret_cast<int *>(red_z + WN * TM);
    if (l4 == 0) {
#pragma unroll
      for (int j = 0; j < NJv; ++j) {
        const int p = wm * TMWv + j * kMB + l16;
        red_m[wn * TM + p] = pm[j];
        red_z[wn * TM + p] = pz[j];
        red_i[wn * TM + p] = pi[j];
      }
    }
    lds_barrier();
    for (int p = tid; p < TM; p += kThreads) {
      if (m0 + p >= Mc) break;
      float mx = red_m[p], z = red_z[p];
      int id = red_i[p];
#pragma unroll
      for (int g = 1; g < WN; ++g) merge_part(mx, z, id, red_m[g * TM + p], red_z[g * TM + p], red_i[g * TM + p]);
      Part pt;
      pt.m = mx; pt.z = z; pt.idx = id; pt.pad = 0;
      parts[int64_t(m0 + p) * n_tiles + tn] = pt;
    }
    lds_barrier();                   // the next tile's DMA reuses the ring
  }
}

template <bool kPacked>
__global__ __launch_bounds__(kThreads, 1) void lmhead_tiles(
    const bf16 *__restrict__ hidden, const bf16 *__restrict__ whead, int M, int V, int H,
    int n_tiles, const int32_t *__restrict__ rows, const int32_t *__restrict__ count,
    Part *__restrict__ parts) {
  __shared__ __attribute__((aligned(1024))) unsigned char ring[kRingBytes];
  const int Mc = count ? *count : M;
  // 128-position tiles when they pad the positions to at most 5/6 of the
  // rows that 256-position tiles would: per flop they run at about 0.83 of
  // the larger tiles' rate, so they pay when they skip a padded half tile
  // (at most 128 positions left, or 257 .. 384)
  const int rows_s = (Mc + kTMSmall - 1) / kTMSmall * kTMSmall, rows_b = (Mc + kTM - 1) / kTM * kTM;
  if (rows_s * 6 < rows_b * 5)
    tiles_body<kPacked, kTMSmall>(ring, hidden, whead, Mc, V, H, n_tiles, rows, parts);
  else
    tiles_body<kPacked, kTM>(ring, hidden, whead, Mc, V, H, n_tiles, rows, parts);
}

// One workgroup per position: the n_tiles partials, merged in tile order.
__global__ __launch_bounds__(256) void lmhead_merge(const Part *__restrict__ parts, int n_tiles,
                                                   const int32_t *__restrict__ rows,
                                                   const int32_t *__restrict__ count,
                                                   Part *__restrict__ merged,
                                                   int32_t *__restrict__ n_masked_left) {
  const int row = blockIdx.x, tid = threadIdx.x;
  if (row == 0 && tid == 0 && n_masked_left) *n_masked_left = 0;
  if (count && row >= *count) return;
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
    merged[rows ? rows[row] : row] = p;
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
  const int n_tiles = (a->V + kTN - 1) / kTN;
  char *w = static_cast<char *>(ws);
  Part *parts = reinterpret_cast<Part *>(w);
  w += align256(lmhead_parts_bytes(a));
  Part *merged = reinterpret_cast<Part *>(w);
  w += align256(size_t(M) * sizeof(Part));
  int32_t *rows = nullptr, *count = nullptr;
  if (a->masked_in) {
    rows = reinterpret_cast<int32_t *>(w);
    count = rows + M;
    hipLaunchKernelGGL(lmhead_compact, dim3(1), dim3(1024), 0, st, a->masked_in, M, rows, count);
  }
  if (a->w_head_packed)
    hipLaunchKernelGGL(lmhead_tiles<true>, dim3(kGrid), dim3(kThreads), 0, st,
                       static_cast<const bf16 *>(a->hidden), static_cast<const bf16 *>(a->w_head), M,
                       a->V, a->H, n_tiles, rows, count, parts);
  else
    hipLaunchKernelGGL(lmhead_tiles<false>, dim3(kGrid), dim3(kThreads), 0, st,
                       static_cast<const bf16 *>(a->hidden), static_cast<const bf16 *>(a->w_head), M,
                       a->V, a->H, n_tiles, rows, count, parts);
  hipLaunchKernelGGL(lmhead_merge, dim3(unsigned(M)), dim3(256), 0, st, parts, n_tiles, rows, count,
                     merged, a->n_masked_left);
  if (hipGetLastError() != hipSuccess) return TD_ERR_HIP;
  return launch_commit_finalize(merged, 1, a->B, a->S, a->gamma, a->masked_in, a->commit, a->token,
                                a->maxprob, a->n_commit, a->masked_out, a->tokens,
                                a->n_masked_left, stream, nullptr, a->masked_in != nullptr);
}

namespace {
// One 16-byte chunk per thread, in the packed order: chunk d is chunk (d & 7)
// of row (d >> 3) & 255 of block (tn, kt) = divmod(d >> 11, H / 64).  Writes
// are contiguous; each 8 lanes read one 128-byte row segment.
__global__ __launch_bounds__(256) void lmhead_pack(const bf16 *__restrict__ w, int V, int H,
                                                   uint4 *__restrict__ out, int64_t chunks) {
  const int nk = H / kTK;
  for (int64_t d = int64_t(blockIdx.x) * 256 + threadIdx.x; d < chunks; d += int64_t(gridDim.x) * 256) {
    const int c = int(d & 7), row = int((d >> 3) & 255);
    const int64_t blk = d >> 11;
    const int64_t tn = blk / nk;
    const int kt = int(blk - tn * nk);
    const int64_t n = tn * kTN + row;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (n < V) v = *reinterpret_cast<const uint4 *>(w + n * H + kt * kTK + c * 8);
    out[d] = v;
  }
}
}  // namespace

int launch_lmhead_pack(const void *w_head, int32_t V, int32_t H, void *w_packed, void *stream) {
  const int64_t chunks = int64_t(lmhead_packed_bytes(V, H)) / 16;
  const int64_t blocks = std::min<int64_t>((chunks + 255) / 256, int64_t(1) << 20);
  hipLaunchKernelGGL(lmhead_pack, dim3(unsigned(blocks)), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), static_cast<const bf16 *>(w_head), V, H,
                     static_cast<uint4 *>(w_packed), chunks);
  return hipGetLastError() == hipSuccess ? TD_OK : TD_ERR_HIP;
}

}  // namespace td
