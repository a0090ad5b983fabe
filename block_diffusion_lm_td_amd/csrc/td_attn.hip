// Block attention of one denoiser layer on gfx950: the S block queries of
// every query head attend, in ONE softmax, to the context tower's cached
// keys of the sequence and to the block's own keys (news.chathome.org,
// "NVIDIA releases Nemotron-Labs-TwoTower ...", inference paragraph:
// bidirectional inside the block, layer-aligned cross-attention to the
// per-layer KV cache; aiboss88.com, technical-principle section).
//
// bf16, D = 128: attn_bf16_mfma + attn_merge.  A workgroup of 8 waves owns
// up to 256 query rows (the G heads x S positions that share one KV head,
// the GQA group), 32 rows per wave, two waves per SIMD; inside each wave the
// softmax of one 32-key half is interleaved instruction by instruction with
// the matrix products of the others (step16).  K and V tiles of 64 keys
// stream from HBM straight into a 4-stage LDS ring (16-byte global->LDS
// DMA, two tiles in flight while one is consumed), stored row-major with
// XOR-swizzled 16-byte chunks so every LDS read is bank-conflict free.  Both
// products run on v_mfma_f32_32x32x16_bf16 in the transposed orientation
// S^T = K Q^T, O^T = V^T P^T: the scores land with one query per lane, so the
// softmax max/sum over keys is in-lane plus one cross-half swap, and P^T
// feeds the PV product straight from the accumulator registers; the V^T
// operand comes from row-major V through gfx950's transposing 8-byte LDS
// reads.  The key order inside each 16-key step is permuted identically on
// both operands.  Softmax runs in the exp2 domain with a lazy rescale: the
// running max only moves when a tile's max exceeds it by more than 2^8,
// which is exact in real arithmetic and keeps P <= 256.  Full tiles skip the
// max altogether: P is computed against the running max and the max is only
// taken (and O rescaled) when a lane's sum of P exceeds 256.
//
// fp32 (D = 64 or 128): attn_valu, one thread per query row (a plain
// correctness path for small problems).  bf16 with another head dim is
// rejected on the host.
#include <hip/hip_runtime.h>

#include "td_finalize.h"
#include "td_internal.h"

namespace td {
namespace {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int HD = 128;                 // head dim of the MFMA path
constexpr float kNegInf = -__builtin_inff();
constexpr float kLazy = 8.0f;           // rescale only when the max grows by > 2^8

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Workgroup barrier ordering LDS only.  Tiles arrive by global->LDS DMA whose
// completion each wave checks with an explicit vmcnt wait before this
// barrier; a full __syncthreads() would also drain the DMA still in flight
// for the next tiles.
__device__ inline void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

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

// ---------------------------------------------------------------------------
// bf16 MFMA path: persistent, stream-K over 64-key tiles
// ---------------------------------------------------------------------------
// Work units are (sequence b, KV head g, row group rg); unit u owns the
// ceil((L_b + S) / 64) key tiles of its sequence, and all units' tiles form
// one global sequence of W tiles.  Each of the Pe = min(P, W) persistent
// workgroups scans the ragged lengths itself (no separate planning launch)
// and walks a contiguous range of that sequence, the ranges being
// equal in cost (tiles plus a fixed charge per unit started).  Units a
// workgroup covers whole are normalised and written directly; where a range
// cuts a unit, the workgroup writes a partial (O / l in bf16, m, l) into one of its
// two slots, and attn_merge combines the partials of every cut unit after
// the kernel (in workgroup order, so the result is deterministic).  Merging
// in a second launch keeps the main kernel free of device-scope fences,
// which on this part write back and invalidate a whole XCD's L2.
constexpr int T = kKeyTile;       // keys per tile
constexpr int NST = 4;            // LDS stages: tile t-1 (its V), tile t, and t+1, t+2 landing
constexpr int TE = T * HD;        // elements of one K (or V) tile: 16 KB
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

// 16-byte global->LDS DMA of one wave: lane i's 16 bytes from `src` land at
// LDS byte address lds_base + 16*i.  Issued through asm so that the compiler
// does not order later LDS reads behind it (completion is checked with
// explicit vmcnt waits before the barrier that publishes a tile).  The asm
// has no outputs.  It loads M0 itself; that is safe only while the compiler
// keeps nothing of its own in M0, which tests/test_kernel_asm.py checks on
// the generated assembly.
__device__ inline void dma16(const void *src, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off sc1 nt\n\ts_nop 1"
               :
               : "s"(lds_base), "v"(src)
               : "memory", "m0");
}
// The same with a wave-uniform 64-bit base and a per-lane 32-bit byte offset:
// no per-lane address arithmetic.
__device__ inline void dma16s(const void *base, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 sc1 nt\n\ts_nop 1"
               :
               : "s"(lds_base), "v"(voff), "s"(base)
               : "memory", "m0");
}
// The same without the non-temporal hint, for a context read by several row
// groups: the tiles stay in L2 for the sibling workgroups (consecutive
// logical workgroups, on one XCD) that stream the same keys at the same time.
__device__ inline void dma16s_keep(const void *base, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 sc1\n\ts_nop 1"
               :
               : "s"(lds_base), "v"(voff), "s"(base)
               : "memory", "m0");
}
__device__ inline uint32_t lds_addr(const void *p) {
  return uint32_t(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void *)p));
}

// two floats -> two bf16 (round to nearest even), low half first
__device__ inline uint32_t pack_bf16(float a, float b) {
  const bf16 x = bf16(a), y = bf16(b);
  return uint32_t(__builtin_bit_cast(uint16_t, x)) | (uint32_t(__builtin_bit_cast(uint16_t, y)) << 16);
}

// Work split.  Starting a unit inside a workgroup's range costs about as much
// as kSegCost key tiles (the new Q, the pipeline fill and drain, the output),
// so the split is even in cost, not in tiles: unit (b, g) occupies the cost
// slots [Cu, Cu + kSegCost + n_b) of a global cost axis, its n_b tiles being
// the last n_b of them, with Cu = UPS*(prefix_b + kSegCost*b) + u*(n_b + kSegCost)
// for the sequence's u-th unit (prefix_b = tiles of the sequences before b,
// UPS units per sequence).
// Logical workgroup p owns the slots [X_p, X_{p+1}), X_p = p*C/P, and with them
// a contiguous (possibly empty) range of the global tile sequence.
constexpr int kSegCost = 4;
__device__ inline int64_t cost_begin(int64_t p, int64_t C, int P) { return p * C / P; }
// logical workgroup whose cost range holds slot y
__device__ inline int64_t slot_owner(int64_t y, int64_t C, int P) { return ((y + 1) * P - 1) / C; }
// partial slot of workgroup pq holding its piece of the unit whose cost range
// starts at Cu: pq's second slot when pq's range also holds the previous unit
__device__ inline int64_t piece_slot(int64_t pq, int64_t p_first, int64_t Cu, int64_t C, int P) {
  return 2 * pq + ((pq == p_first && cost_begin(pq, C, P) < Cu) ? 1 : 0);
}

struct Cur {
  int b, uis, j, n, L;
  int64_t lo;
};

__device__ inline void cur_load(Cur &c, const int64_t *off, int64_t total, int max_ctx, int S) {
  seq_range(off, c.b, total, max_ctx, c.lo, c.L);
  c.n = (c.L + S + T - 1) / T;
}
__device__ inline void cur_next(Cur &c, int UPS, int B, const int64_t *off, int64_t total,
                                int max_ctx, int S) {
  if (++c.j < c.n) return;
  c.j = 0;
  if (++c.uis < UPS) return;
  c.uis = 0;
  if (++c.b < B) cur_load(c, off, total, max_ctx, S);
}

// ---- half-tile pieces (32 keys) of the per-tile pipeline
// QK for keys h*32 .. h*32+31 of the tile: S^T half = K Q^T (one 32x32 block)
__device__ __forceinline__ void qk_half(const bf16 *__restrict__ Kt, int h, int lq, int lh,
                                        const bf16x8 (&qf)[8], f32x16 &s) {
  s = f32x16{};
  const int row = h * 32 + lq;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    const bf16x8 ka = *reinterpret_cast<const bf16x8 *>(Kt + row * HD + (((ks * 2 + lh) ^ (row & 15)) * 8));
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[ks], s, 0, 0, 0);
  }
}
// Two P values rounded to bf16 (one v_cvt_pk_bf16_f32), stored at positions
// i, i+1 of p, and added to the lane's row sum with one v_dot2 against
// (1, 1): the sum is over the same rounded P the PV product uses.
__device__ __forceinline__ float p_pair(float a, float b, bf16x8 &p, int i, float acc) {
  const bf16x2 pr = {bf16(a), bf16(b)};
  p[i] = pr.x;
  p[i + 1] = pr.y;
  const bf16x2 one = {bf16(1.0f), bf16(1.0f)};
  return __builtin_amdgcn_fdot2_f32_bf16(pr, one, acc, false);
}
// softmax of a half: P^T as bf16 (k-steps kk = 0, 1 of the half) and its lane sum
__device__ __forceinline__ float sm_half(const f32x16 &s, float m, float sl2, bf16x8 (&p)[2]) {
  float acc = 0.f;
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      const float p0 = fast_exp2(__builtin_fmaf(s[kk * 8 + i], sl2, -m));
      const float p1 = fast_exp2(__builtin_fmaf(s[kk * 8 + i + 1], sl2, -m));
      acc = p_pair(p0, p1, p[kk], i, acc);
    }
  return acc;
}
// O^T += V^T P^T for keys h*32 .. h*32+31; the V^T operand comes from two
// transposing 8-byte LDS reads (16-lane group g: source lane 4e+a addresses
// key (k-step*16 + rd*8 + (g/2)*4 + e), dims db*32 + (g%2)*16 + 4a..+3; lane t
// of the group then holds dim db*32 + (g%2)*16 + t of those 4 keys)
__device__ __forceinline__ void pv_half(const bf16 *__restrict__ Vt, int h, int e4, int v_lane_off,
                                        const bf16x8 (&p)[2], f32x16 (&o)[4]) {
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int sw = (db ^ e4) * 32;
      const bf16 *base = Vt + (h * 2 + kk) * 16 * HD + v_lane_off + sw;
      const s16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)(base));
      const s16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)(base + 8 * HD));
      // whole-vector bit casts: building the operand element by element
      // from the 16-bit lanes of the two reads does not compile correctly
      const u32x2 a0 = __builtin_bit_cast(u32x2, r0), a1 = __builtin_bit_cast(u32x2, r1);
      const u32x4 a01 = {a0.x, a0.y, a1.x, a1.y};
      const bf16x8 va = __builtin_bit_cast(bf16x8, a01);
      o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, p[kk], o[db], 0, 0, 0);
    }
}
// row max of a half (both lane halves hold the same query), in the exp2 domain
__device__ __forceinline__ float max_half(const f32x16 &s, float sl2) {
  float a = fmaxf(fmaxf(s[0], s[1]), s[2]), b = fmaxf(fmaxf(s[3], s[4]), s[5]);
  float c = fmaxf(fmaxf(s[6], s[7]), s[8]), d = fmaxf(fmaxf(s[9], s[10]), s[11]);
  float e = fmaxf(fmaxf(s[12], s[13]), s[14]);
  a = fmaxf(fmaxf(a, b), c);
  d = fmaxf(fmaxf(d, e), s[15]);
  const float mx = fmaxf(a, d);
  return fmaxf(mx, __shfl_xor(mx, 32)) * sl2;
}
// One pipeline step in a fixed instruction order: QK for keys hq*32.. of the
// K tile Kq into sq (8 MFMAs, one dependent chain), PV for keys hv*32.. of
// the V tile Vv with P = pv (8 MFMAs, four chains), and the softmax of the
// scores ss into ps.  Slot i issues one MFMA (QK and PV alternating, so the
// QK chain never stalls on itself), the softmax of score i, and the LDS reads
// of the operands for slot i + kAhead; the scheduling fences keep that order,
// so each wave keeps the matrix core and the VALU busy at once.  Returns the
// lane's sum of its 16 P values.
constexpr int kAhead = 2;
__device__ __forceinline__ float step16(const bf16 *__restrict__ Kq, int hq, const bf16 *__restrict__ Vv,
                                        int hv, int lq, int lh, int e4, int v_lane_off,
                                        const bf16x8 (&qf)[8], f32x16 &sq, const bf16x8 (&pv)[2],
                                        f32x16 (&o)[4], const f32x16 &ss, float m, float sl2,
                                        bf16x8 (&ps)[2]) {
  const int row = hq * 32 + lq;
  bf16x8 opnd[16];
  auto load = [&](int i) {
    if ((i & 1) == 0) {
      const int ks = i >> 1;
      opnd[i] = *reinterpret_cast<const bf16x8 *>(Kq + row * HD + (((ks * 2 + lh) ^ (row & 15)) * 8));
    } else {
      const int kk = (i >> 1) >> 2, db = (i >> 1) & 3;
      const bf16 *base = Vv + (hv * 2 + kk) * 16 * HD + v_lane_off + ((db ^ e4) * 32);
      const s16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)(base));
      const s16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)(base + 8 * HD));
      const u32x2 a0 = __builtin_bit_cast(u32x2, r0), a1 = __builtin_bit_cast(u32x2, r1);
      const u32x4 a01 = {a0.x, a0.y, a1.x, a1.y};
      opnd[i] = __builtin_bit_cast(bf16x8, a01);
    }
  };
#pragma unroll
  for (int i = 0; i < kAhead; ++i) load(i);
  float acc = 0.f, pe_prev = 0.f;
  sq = f32x16{};
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    __builtin_amdgcn_sched_barrier(0);
    if ((i & 1) == 0) {
      sq = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opnd[i], qf[i >> 1], sq, 0, 0, 0);
    } else {
      const int kk = (i >> 1) >> 2, db = (i >> 1) & 3;
      o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opnd[i], pv[kk], o[db], 0, 0, 0);
    }
    const float pe = fast_exp2(__builtin_fmaf(ss[i], sl2, -m));
    if (i & 1)
      acc = p_pair(pe_prev, pe, ps[i >> 3], (i & 7) - 1, acc);
    else
      pe_prev = pe;
    if (i + kAhead < 16) load(i + kAhead);
  }
  __builtin_amdgcn_sched_barrier(0);
  return acc;
}
// keys h*32 + key >= nvalid get a score of -inf
__device__ __forceinline__ void mask_half(f32x16 &s, int h, int lh, int nvalid) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int key = h * 32 + (r >> 2) * 8 + lh * 4 + (r & 3);
    if (key >= nvalid) s[r] = kNegInf;
  }
}

// KEEP: units of several row groups (RG > 1) read each context tile once per
// row group; the DMA then keeps the tiles in L2 for the siblings.
template <bool KEEP>
__global__ __launch_bounds__(kWGThreads, 1) void attn_bf16_mfma(
    const bf16 *__restrict__ q, const bf16 *__restrict__ kb, const bf16 *__restrict__ vb,
    const bf16 *__restrict__ kc, const bf16 *__restrict__ vc, const int64_t *__restrict__ off,
    int64_t total_ctx, int max_ctx, int B, int S, int Hq, int Hkv, int G, int M, int RG, int P,
    float sl2, int64_t *__restrict__ prefix_out, float2 *__restrict__ ws_ml,
    bf16 *__restrict__ ws_o, bf16 *__restrict__ out, const int32_t *__restrict__ gate) {
  if (gate && *gate == 0) return;           // a gated step whose block has finished
  // K and V tiles, row-major [key][d] with 16-byte chunks XOR-swizzled per row:
  // K chunk c of key r sits at c ^ (r % 16), V chunk c at c ^ 4*(r % 4).
  __shared__ __attribute__((aligned(1024))) bf16 Ks[NST * TE];
  __shared__ __attribute__((aligned(1024))) bf16 Vs[NST * TE];
  __shared__ int64_t s_wsum[kWaves];
  __shared__ int64_t s_t[2];
  __shared__ int s_loc[3];

  const int UPS = Hkv * RG;
  const int tid = threadIdx.x;
  // consecutive logical ranges land on one XCD (dispatch is round-robin over 8)
  const int pid = (P % 8 == 0) ? int(blockIdx.x % 8) * (P / 8) + int(blockIdx.x / 8) : int(blockIdx.x);

  // ---- ragged plan: tiles per sequence, their prefix, this workgroup's range
  auto ntiles = [&](int b) -> int64_t {
    int64_t lo;
    int L;
    seq_range(off, b, total_ctx, max_ctx, lo, L);
    return (int64_t(L) + S + T - 1) / T;
  };
  // inclusive scan of v over the workgroup's threads: shuffles inside each
  // wave, then the wave totals through LDS; also returns the grand total
  // (a sequence's tile count is below 2^25 and a sum of 64 of them below
  // 2^31, as the host bounds max_ctx, so the wave part runs in 32 bits)
  auto wg_scan = [&](int64_t v64, int64_t &total) -> int64_t {
    const int ln = tid & 63, wv = tid >> 6;
    uint32_t v = uint32_t(v64);
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const uint32_t y = __shfl_up(v, d);
      if (ln >= d) v += y;
    }
    if (ln == 63) s_wsum[wv] = v;
    __syncthreads();
    int64_t before = 0;
    total = 0;
#pragma unroll
    for (int k = 0; k < kWaves; ++k) {
      const int64_t x = s_wsum[k];
      if (k < wv) before += x;
      total += x;
    }
    __syncthreads();                           // s_wsum is reused by the next call
    return int64_t(v) + before;
  };
  // a workgroup-uniform 64-bit value held in vector registers, moved to scalar ones
  auto uniform64 = [](int64_t x) -> int64_t {
    const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(x));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(uint64_t(x) >> 32));
    return int64_t((uint64_t(hi) << 32) | lo);
  };
  const bool one_pass = B <= kWGThreads;
  int64_t n_mine = 0, incl_mine = 0, wseq = 0;
  if (one_pass) {
    n_mine = tid < B ? ntiles(tid) : 0;
    incl_mine = wg_scan(n_mine, wseq);
  } else {
    for (int base = 0; base < B; base += kWGThreads) {
      int64_t tot;
      wg_scan(base + tid < B ? ntiles(base + tid) : 0, tot);
      wseq += tot;
    }
  }
  wseq = uniform64(wseq);
  const int64_t W = wseq * UPS;
  const int Pe = int(W < P ? W : P);          // logical workgroups with work
  if (pid >= Pe) return;
  const int64_t C = UPS * (wseq + int64_t(kSegCost) * B);
  const int64_t X0 = cost_begin(pid, C, Pe), X1 = cost_begin(pid + 1, C, Pe);
  // the first tile at or after cost slot X of sequence b (excl tiles before it,
  // n per unit); the sequences' cost ranges tile [0, C), so for X < C exactly
  // one thread finds it
  auto locate = [&](int64_t X, int b, int64_t excl, int64_t n, int k) {
    const int64_t ce = UPS * (excl + int64_t(kSegCost) * b);
    const int64_t ci = ce + UPS * (n + kSegCost);
    if (ce <= X && X < ci) {
      const int64_t r = X - ce, uc = n + kSegCost;
      const int64_t u = r / uc, rr = r - u * uc;
      const int64_t j = rr > kSegCost ? rr - kSegCost : 0;
      s_t[k] = excl * UPS + u * n + j;
      if (k == 0) { s_loc[0] = b; s_loc[1] = int(u); s_loc[2] = int(j); }
    }
  };
  if (pid == 0 && tid == 0) prefix_out[0] = 0;
  if (one_pass) {
    if (tid < B) {
      const int64_t excl = incl_mine - n_mine;
      if (pid == 0) prefix_out[tid + 1] = incl_mine;
      locate(X0, tid, excl, n_mine, 0);
      locate(X1, tid, excl, n_mine, 1);
    }
  } else {
    int64_t running = 0;
    for (int base = 0; base < B; base += kWGThreads) {
      const int b = base + tid;
      const int64_t n = b < B ? ntiles(b) : 0;
      int64_t tot;
      const int64_t incl = running + wg_scan(n, tot), excl = incl - n;
      if (b < B) {
        if (pid == 0) prefix_out[b + 1] = incl;
        locate(X0, b, excl, n, 0);
        locate(X1, b, excl, n, 1);
      }
      running += tot;
    }
  }
  __syncthreads();
  const int64_t t_begin = uniform64(s_t[0]), t_end = uniform64(X1 >= C ? W : s_t[1]);
  if (t_begin >= t_end) return;                // a range of overhead slots only

  const int w = tid >> 6, lane = tid & 63, lq = lane & 31, lh = lane >> 5;
  const int64_t kvs = int64_t(Hkv) * HD;

  // ---- DMA issue of one tile: K and V rows w*8 .. w*8+7, two 4-row (1 KB)
  // pieces each; lane i fills LDS slot i%16 of row w*8 + r*4 + i/16
  uint32_t dko[2], dvo[2];       // lane byte offsets inside a tile of the context cache
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int R = w * 8 + r * 4 + (lane >> 4), cs = lane & 15;
    dko[r] = uint32_t(R) * uint32_t(kvs) * 2u + uint32_t(cs ^ (R & 15)) * 16u;
    dvo[r] = uint32_t(R) * uint32_t(kvs) * 2u + uint32_t(cs ^ ((R & 3) << 2)) * 16u;
  }
  const uint32_t lds_k = __builtin_amdgcn_readfirstlane(lds_addr(Ks + (w * 8) * HD));
  const uint32_t lds_v = __builtin_amdgcn_readfirstlane(lds_addr(Vs + (w * 8) * HD));
  auto issue = [&](const Cur &c, int stage) {
    const int g = c.uis / RG;
    const int k0 = c.j * T;
    const uint32_t lk = lds_k + uint32_t(stage) * (TE * 2), lv = lds_v + uint32_t(stage) * (TE * 2);
    if (k0 + T <= c.L) {                       // whole tile in the context cache
      const int64_t e0 = (c.lo + k0) * kvs + int64_t(g) * HD;
      if (KEEP) {
        dma16s_keep(kc + e0, dko[0], lk);
        dma16s_keep(vc + e0, dvo[0], lv);
        dma16s_keep(kc + e0, dko[1], lk + 4 * HD * 2);
        dma16s_keep(vc + e0, dvo[1], lv + 4 * HD * 2);
      } else {
        dma16s(kc + e0, dko[0], lk);
        dma16s(vc + e0, dvo[0], lv);
        dma16s(kc + e0, dko[1], lk + 4 * HD * 2);
        dma16s(vc + e0, dvo[1], lv + 4 * HD * 2);
      }
      return;
    }
    // the tile reaches into the block's own keys (or past their end)
    const int nvalid = min(T, c.L + S - k0);
    const bf16 *kcg = kc + c.lo * kvs + int64_t(g) * HD;
    const bf16 *vcg = vc + c.lo * kvs + int64_t(g) * HD;
    const bf16 *kbg = kb + int64_t(c.b) * S * kvs + int64_t(g) * HD;
    const bf16 *vbg = vb + int64_t(c.b) * S * kvs + int64_t(g) * HD;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int R = w * 8 + r * 4 + (lane >> 4);
      const int cs = lane & 15;
      const int key = k0 + (R < nvalid ? R : 0);           // rows past the end re-read a valid key
      const int64_t roff = int64_t(key < c.L ? key : key - c.L) * kvs;
      dma16((key < c.L ? kcg : kbg) + roff + (cs ^ (R & 15)) * 8, lk + r * 4 * HD * 2);
      dma16((key < c.L ? vcg : vbg) + roff + (cs ^ ((R & 3) << 2)) * 8, lv + r * 4 * HD * 2);
    }
  };

  Cur ld, cc;
  ld.b = __builtin_amdgcn_readfirstlane(s_loc[0]);
  ld.uis = __builtin_amdgcn_readfirstlane(s_loc[1]);
  ld.j = __builtin_amdgcn_readfirstlane(s_loc[2]);
  cur_load(ld, off, total_ctx, max_ctx, S);
  cc = ld;
  // Q fragments of unit c's rows held by this wave (zeros past M).  A
  // segment's Q is loaded ahead of use: the first segment's before the first
  // tiles' DMA, so compute starts once Q and tile 0 have landed; each later
  // segment's right after the previous segment's last QK, while its last
  // tile drains.  The compiler waits for these loads before Q's first use;
  // the tile DMA it does not see only ever makes that wait stricter, as
  // vector memory operations retire in issue order.
  bf16x8 qf[8];
  auto load_q = [&](const Cur &c) {
    const int g = c.uis / RG, rg = c.uis - (c.uis / RG) * RG;
    const int row = rg * kRowsPerWG + w * 32 + lq;
    if (row < M) {
      const int s = row / G, jh = row - (row / G) * G;
      const bf16 *p = q + ((int64_t(c.b) * S + s) * Hq + int64_t(g) * G + jh) * HD + lh * 8;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) qf[ks] = *reinterpret_cast<const bf16x8 *>(p + ks * 16);
    } else {
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) qf[ks] = bf16x8{};
    }
  };
  load_q(ld);
  for (int x = 0; x < 2 && t_begin + x < t_end; ++x) {
    issue(ld, x);
    cur_next(ld, UPS, B, off, total_ctx, max_ctx, S);
  }

  // per-lane LDS offsets (elements) of the MFMA operands
  // K (A operand of S^T = K Q^T): key kb*32 + lq, chunk ks*2 + lh
  // V (A operand of O^T = V^T P^T, via transposing reads): see below
  const int e4 = (lane & 15) >> 2, a4 = lane & 3, gh = (lane >> 4) & 1;
  const int v_lane_off = (lh * 4 + e4) * HD + gh * 16 + a4 * 4;

  f32x16 o[4];
  f32x16 sA, sB;                 // scores of the two 32-key halves of a tile
  bf16x8 pA[2], pB[2];
  float m = kNegInf, l = 0.f;

  // Moves the running max when the half's max exceeds it by more than 2^8
  // (lazy rescale: exact in real arithmetic, keeps P <= 256).  O must hold
  // exactly the products made with the old max when this runs.
  // The rescale is rare after a sequence's first tiles; the empty volatile
  // asm keeps it behind a real branch (the compiler would otherwise
  // if-convert it and pay the 64 multiplies on every tile).
  auto lazy = [&](float mxs) {
    const bool need = mxs > m + kLazy;
    if (__any(need)) {
      asm volatile("");
      const float mn = need ? mxs : m;
      const float alpha = fast_exp2(m - mn);
#pragma unroll
      for (int db = 0; db < 4; ++db) o[db] *= alpha;
      l *= alpha;
      m = mn;
    }
  };

  // Softmax of a half of a full tile against the running max, without first
  // taking the half's max: every P <= 256 as long as no lane's sum exceeds
  // 256; if one does, the half's scores are recomputed from the K tile
  // (still in LDS) and masked as before, the half's max is taken, O and l
  // are rescaled (lazy: only if the max grew by more than 2^8) and P is
  // recomputed.  Recomputing the scores on that rare path, rather than
  // keeping them, frees their registers once P is formed.
  auto guard = [&](float sum, bf16x8 (&pX)[2], const bf16 *Kx, int hx, int nv) -> float {
    if (__any(!(sum <= 256.f))) {
      asm volatile("");
      f32x16 sR;
      qk_half(Kx, hx, lq, lh, qf, sR);
      if (nv < 32 * (hx + 1)) mask_half(sR, hx, lh, nv);
      lazy(max_half(sR, sl2));
      sum = sm_half(sR, m, sl2, pX);
    }
    return sum;
  };

  // Per tile t (halves A = keys 0-31, B = keys 32-63), two steps of 16
  // MFMAs each, whose matrix work and softmax work are independent:
  //   1: QK_A(t) + PV_A(t-1)     || softmax B(t-1)
  //   2: QK_B(t) + PV_B(t-1)     || softmax A(t)
  // so a half's scores wait one step for their softmax and its P one more
  // for the PV product.  A segment's first tile only fills the pipeline
  // (QK of both halves, softmax A); its last tile is finished after the loop.
  // Each step is one basic block up to the softmax guard.
  int64_t t = t_begin;
  int st = 0;
  // wait for tile t (only tile t+1 may still be in flight), publish it, and
  // refill the stage of tile t-2 with tile t+2
  auto next_tile = [&]() {
    if (t + 1 < t_end) {
      __builtin_amdgcn_s_waitcnt(0xF70 | 4);
    } else {
      __builtin_amdgcn_s_waitcnt(0xF70);
    }
    lds_barrier();
    if (t + 2 < t_end) {
      issue(ld, (st + 2) & (NST - 1));
      cur_next(ld, UPS, B, off, total_ctx, max_ctx, S);
    }
  };
  while (t < t_end) {
    // ---- segment: this WG's tiles of one unit
    const int g = cc.uis / RG, rg = cc.uis - (cc.uis / RG) * RG;
    const int64_t seg_t0 = t;
    const int seg_j0 = cc.j;
    const int64_t seg_t1 = min(t_end, t + (cc.n - cc.j));     // one past the segment's last tile
    const Cur cu = cc;                                         // the segment's unit
#pragma unroll
    for (int db = 0; db < 4; ++db) o[db] = f32x16{};
    m = kNegInf;
    l = 0.f;

    // first tile of the segment
    next_tile();
    int nvalid = min(T, cc.L + S - cc.j * T);
    {
      const bf16 *Kt = Ks + st * TE;
      qk_half(Kt, 0, lq, lh, qf, sA);
      if (nvalid < 32) mask_half(sA, 0, lh, nvalid);
      lazy(max_half(sA, sl2));
      qk_half(Kt, 1, lq, lh, qf, sB);
      l += sm_half(sA, m, sl2, pA);
    }
    // steady tiles: all full (only a segment's last tile can be partial)
    auto steady = [&](bool may_mask) {
      next_tile();
      nvalid = min(T, cc.L + S - cc.j * T);
      const bf16 *Kt = Ks + st * TE;
      const bf16 *Kp = Ks + ((st + NST - 1) & (NST - 1)) * TE;
      const bf16 *Vp = Vs + ((st + NST - 1) & (NST - 1)) * TE;
      // step 1 (PV_A(t-1) comes before B(t-1)'s guard in program order, so a
      // rescale there finds O complete up to A(t-1) and no P pending)
      l += guard(step16(Kt, 0, Vp, 0, lq, lh, e4, v_lane_off, qf, sA, pA, o, sB, m, sl2, pB),
                 pB, Kp, 1, T);
      if (may_mask && nvalid < 32) mask_half(sA, 0, lh, nvalid);
      // step 2
      l += guard(step16(Kt, 1, Vp, 1, lq, lh, e4, v_lane_off, qf, sB, pB, o, sA, m, sl2, pA),
                 pA, Kt, 0, may_mask ? nvalid : T);
    };
    auto advance = [&]() {
      ++t;
      st = (st + 1) & (NST - 1);
      cur_next(cc, UPS, B, off, total_ctx, max_ctx, S);
    };
    advance();
    for (; t + 1 < seg_t1; advance()) steady(false);
    if (t < seg_t1) {
      steady(true);
      advance();
    }
    // the next segment's Q (this segment's QK is complete)
    if (t < t_end) load_q(cc);
    // PV_A and the B half of the segment's last tile (stage st - 1), then the output
    {
      const int stl = (st + NST - 1) & (NST - 1);
      const bf16 *Vl = Vs + stl * TE;
      pv_half(Vl, 0, e4, v_lane_off, pA, o);
      if (nvalid < T) mask_half(sB, 1, lh, nvalid);
      lazy(max_half(sB, sl2));
      l += sm_half(sB, m, sl2, pB);
      pv_half(Vl, 1, e4, v_lane_off, pB, o);
    }
    l += __shfl_xor(l, 32);
    const int row = rg * kRowsPerWG + w * 32 + lq;
    const int last_j = seg_j0 + int(seg_t1 - seg_t0) - 1;
    if (seg_j0 == 0 && last_j == cu.n - 1) {               // the whole unit: output
      if (row < M) {
        const int s = row / G, jh = row - (row / G) * G;
        bf16 *dst = out + ((int64_t(cu.b) * S + s) * Hq + int64_t(g) * G + jh) * HD;
        const float inv = 1.0f / l;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int gi = 0; gi < 4; ++gi) {
            bf16x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = bf16(o[db][gi * 4 + e] * inv);
            *reinterpret_cast<bf16x4 *>(dst + db * 32 + gi * 8 + lh * 4) = v;
          }
      }
    } else {                                                   // a piece: partial slot
      // O / l in bf16 (the merge weighs pieces by l * 2^(m - max m)); lane's
      // 16 values of fragment db are 32 contiguous bytes
      const int64_t slot = 2 * int64_t(pid) + (seg_t0 == t_begin ? 0 : 1);
      uint4 *wo = reinterpret_cast<uint4 *>(ws_o + slot * (kRowsPerWG * HD));
      const float inv = 1.0f / l;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        uint32_t h[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) h[i] = pack_bf16(o[db][2 * i] * inv, o[db][2 * i + 1] * inv);
        wo[((w * 4 + db) * 64 + lane) * 2 + 0] = make_uint4(h[0], h[1], h[2], h[3]);
        wo[((w * 4 + db) * 64 + lane) * 2 + 1] = make_uint4(h[4], h[5], h[6], h[7]);
      }
      if (lh == 0) ws_ml[slot * kRowsPerWG + w * 32 + lq] = make_float2(m, l);
    }
  }
}

// Merge of the partials of every unit cut between workgroups.  A 32-row block
// of one wave's rows is merged by PG workgroups of 256 threads, each taking
// 32/PG of its rows; inside a workgroup PG thread groups split the unit's
// pieces round-robin (group q takes pieces q, q + PG, ...).  A thread (db, lh,
// row) combines the 16 values of fragment db that lane (lh, row) held, over
// its group's pieces in workgroup order with a running max; the groups'
// states are then combined in group order through LDS (deterministic).  PRE
// pieces are fetched per memory round trip.  PG = 1, PRE = 4 serves the
// common case of a few pieces per unit; long contexts over few sequences cut
// each unit into dozens of pieces, and PG = 4, PRE = 8 spreads them over four
// times the workgroups and threads.
template <int PRE, int PG>
__device__ __forceinline__ void merge_block(
    int64_t blk, const int64_t *__restrict__ prefix, int B, int S, int Hq, int Hkv, int G, int M,
    int RG, int P, const float2 *__restrict__ ws_ml, const bf16 *__restrict__ ws_o,
    bf16 *__restrict__ out) {
  constexpr int RW = 32 / PG;                      // rows of this workgroup
  constexpr int TG = 256 / PG;                     // threads per piece group
  static_assert(PG == 1 || PG == 2 || PG == 4 || PG == 8, "piece groups");
  const int UPS = Hkv * RG;
  const int64_t u = blk / (8 * PG);
  const int w = int((blk / PG) & 7);
  const int sb = int(blk % PG);
  const int b = int(u / UPS), uis = int(u - (u / UPS) * UPS);
  const int g = uis / RG, rg = uis - (uis / RG) * RG;
  const int64_t W = prefix[B] * UPS;
  const int Pe = int(W < P ? W : P);
  const int64_t C = UPS * (prefix[B] + int64_t(kSegCost) * B);
  const int64_t n = prefix[b + 1] - prefix[b];
  const int64_t Cu = UPS * (prefix[b] + int64_t(kSegCost) * b) + int64_t(uis) * (n + kSegCost);
  const int64_t y0 = Cu + kSegCost;               // cost slots of the unit's first and last tiles
  const int64_t p_first = slot_owner(y0, C, Pe), p_last = slot_owner(y0 + n - 1, C, Pe);
  if (p_first == p_last) return;                 // written whole by its workgroup (uniform)
  const int pg = threadIdx.x / TG, t = threadIdx.x - pg * TG;
  const int db = t / (2 * RW), r2 = t - db * (2 * RW);
  const int lh = r2 / RW, lq = sb * RW + (r2 - lh * RW);
  const int lane = lh * 32 + lq;
  const int row = rg * kRowsPerWG + w * 32 + lq;
  const bool live = row < M;
  if (PG == 1 && !live) return;                  // no barrier below with one group
  const uint4 *wo = reinterpret_cast<const uint4 *>(ws_o);
  float mx = kNegInf, lsum = 0.f;
  float acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
  // piece pq's (m, l) and this thread's 16 values of O / l (just written by the
  // main kernel and usually still cached, so ordinary loads)
  auto fetch = [&](int64_t pq, float2 &ml, uint4 &x0, uint4 &x1) {
    const int64_t sq = piece_slot(pq, p_first, Cu, C, Pe);
    const int64_t f = (sq * (kRowsPerWG * HD / 8)) + ((w * 4 + db) * 64 + lane) * 2;
    ml = ws_ml[sq * kRowsPerWG + w * 32 + lq];
    x0 = wo[f];
    x1 = wo[f + 1];
  };
  auto absorb = [&](const float2 &ml, const uint4 &x0, const uint4 &x1) {
    if (ml.x > mx) {
      const float c = fast_exp2(mx - ml.x);
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] *= c;
      lsum *= c;
      mx = ml.x;
    }
    const float wgt = ml.y * fast_exp2(ml.x - mx);
    lsum += wgt;
    const uint32_t h[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      acc[2 * i] += wgt * __uint_as_float(h[i] << 16);
      acc[2 * i + 1] += wgt * __uint_as_float(h[i] & 0xffff0000u);
    }
  };
  // this group's pieces, PRE at a time (one memory round trip per batch),
  // combined in workgroup order
  if (live) {
    for (int64_t base = p_first + pg; base <= p_last; base += int64_t(PRE) * PG) {
      float2 mlv[PRE];
      uint4 xa[PRE], xb[PRE];
#pragma unroll
      for (int k = 0; k < PRE; ++k)
        if (base + int64_t(k) * PG <= p_last) fetch(base + int64_t(k) * PG, mlv[k], xa[k], xb[k]);
#pragma unroll
      for (int k = 0; k < PRE; ++k)
        if (base + int64_t(k) * PG <= p_last) absorb(mlv[k], xa[k], xb[k]);
    }
  }
  if constexpr (PG > 1) {
    // the groups' states meet in LDS; group 0 folds groups 1.. in order
    __shared__ float s_st[PG - 1][18][TG];
    if (pg > 0) {
      s_st[pg - 1][0][t] = mx;
      s_st[pg - 1][1][t] = lsum;
#pragma unroll
      for (int i = 0; i < 16; ++i) s_st[pg - 1][2 + i][t] = acc[i];
    }
    __syncthreads();
    if (pg > 0 || !live) return;
#pragma unroll
    for (int q = 0; q < PG - 1; ++q) {
      const float qm = s_st[q][0][t], ql = s_st[q][1][t];
      if (ql == 0.f) continue;                     // a group with no pieces
      if (qm > mx) {
        const float c = fast_exp2(mx - qm);
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[i] *= c;
        lsum *= c;
        mx = qm;
      }
      const float c = fast_exp2(qm - mx);
      lsum += ql * c;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] += s_st[q][2 + i][t] * c;
    }
  }
  if (!live) return;
  const float inv = 1.0f / lsum;
  const int s = row / G, jh = row - (row / G) * G;
  bf16 *dst = out + ((int64_t(b) * S + s) * Hq + int64_t(g) * G + jh) * HD + db * 32 + lh * 4;
#pragma unroll
  for (int gi = 0; gi < 4; ++gi)
    *reinterpret_cast<uint2 *>(dst + gi * 8) =
        make_uint2(pack_bf16(acc[gi * 4] * inv, acc[gi * 4 + 1] * inv),
                   pack_bf16(acc[gi * 4 + 2] * inv, acc[gi * 4 + 3] * inv));
}

template <int PRE, int PG>
__global__ __launch_bounds__(256) void attn_merge(
    const int64_t *__restrict__ prefix, int B, int S, int Hq, int Hkv, int G, int M, int RG, int P,
    const float2 *__restrict__ ws_ml, const bf16 *__restrict__ ws_o, bf16 *__restrict__ out,
    const int32_t *__restrict__ gate) {
  if (gate && *gate == 0) return;
  merge_block<PRE, PG>(blockIdx.x, prefix, B, S, Hq, Hkv, G, M, RG, P, ws_ml, ws_o, out);
}

// The tail of a denoise step in one launch: the attention merge (blocks
// [0, merge_blocks), as attn_merge) and, beside it, the commit's block
// decision (the remaining blocks, one wave per sequence, as
// commit_finalize).  The two share no data; running them in one grid saves
// a launch and its drain on the step's critical path.
template <int PRE, int PG>
__global__ __launch_bounds__(256) void step_tail(
    const int64_t *__restrict__ prefix, int B, int S, int Hq, int Hkv, int G, int M, int RG, int P,
    const float2 *__restrict__ ws_ml, const bf16 *__restrict__ ws_o, bf16 *__restrict__ out,
    int64_t merge_blocks, const Part *__restrict__ parts, int R, float gamma,
    const uint8_t *masked_in, uint8_t *__restrict__ commit, int32_t *__restrict__ token,
    float *__restrict__ maxprob, int32_t *__restrict__ n_commit, uint8_t *masked_out,
    int32_t *__restrict__ tokens, int32_t *__restrict__ n_masked_left,
    const int32_t *__restrict__ gate) {
  if (gate && *gate == 0) return;
  if (int64_t(blockIdx.x) < merge_blocks) {
    merge_block<PRE, PG>(blockIdx.x, prefix, B, S, Hq, Hkv, G, M, RG, P, ws_ml, ws_o, out);
    return;
  }
  const int b = int(int64_t(blockIdx.x) - merge_blocks) * 4 + int(threadIdx.x >> 6);
  if (b < B)
    fin::finalize_seq(b, threadIdx.x & 63, parts, S, R, gamma, masked_in, commit, token, maxprob,
                      n_commit, masked_out, tokens, n_masked_left, false);
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
    T *__restrict__ out, const int32_t *__restrict__ gate) {
  if (gate && *gate == 0) return;
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

// More than about four pieces per cut unit on average (launch workgroups
// against units): long contexts over few sequences.
inline bool many_pieces(const AttnPlan &p) { return int64_t(p.launch) > 4 * p.units; }

}  // namespace

int launch_attn(const td_attn_args *a, const AttnPlan &p, void *ws, void *stream,
                const int32_t *gate, bool merge) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int max_ctx = int(a->max_ctx);
  if (p.mfma) {
    char *wsb = static_cast<char *>(ws);
    int64_t *prefix = reinterpret_cast<int64_t *>(wsb + p.off_prefix);
    float2 *ws_ml = reinterpret_cast<float2 *>(wsb + p.off_ml);
    bf16 *ws_o = reinterpret_cast<bf16 *>(wsb + p.off_o);
    auto k = p.row_groups > 1 ? attn_bf16_mfma<true> : attn_bf16_mfma<false>;
    hipLaunchKernelGGL(k, dim3(p.launch), dim3(kWGThreads), 0, st,
                       static_cast<const bf16 *>(a->q), static_cast<const bf16 *>(a->k_blk),
                       static_cast<const bf16 *>(a->v_blk), static_cast<const bf16 *>(a->k_ctx),
                       static_cast<const bf16 *>(a->v_ctx), a->ctx_offsets, a->total_ctx, max_ctx,
                       a->B, a->S, a->Hq, a->Hkv, p.G, p.M, p.row_groups, p.launch, p.scale_log2,
                       prefix, ws_ml, ws_o, static_cast<bf16 *>(a->out), gate);
    if (merge) {
      const bool many = many_pieces(p);
      auto k = many ? attn_merge<8, 4> : attn_merge<4, 1>;
      hipLaunchKernelGGL(k, dim3(unsigned(p.units * 8 * (many ? 4 : 1))), dim3(256), 0, st, prefix, a->B,
                         a->S, a->Hq, a->Hkv, p.G, p.M, p.row_groups, p.launch, ws_ml, ws_o,
                         static_cast<bf16 *>(a->out), gate);
    }
  } else {
    dim3 grid(p.row_groups, a->Hkv, a->B);
#define TD_VALU(T, DD)                                                                         \
  hipLaunchKernelGGL((attn_valu<T, DD>), grid, dim3(64), 0, st,                              \
                     static_cast<const T *>(a->q), static_cast<const T *>(a->k_blk),         \
                     static_cast<const T *>(a->v_blk), static_cast<const T *>(a->k_ctx),     \
                     static_cast<const T *>(a->v_ctx), a->ctx_offsets, a->total_ctx, max_ctx, \
                     a->S, a->Hq, a->Hkv, p.G, p.M, p.scale_log2, static_cast<T *>(a->out), gate)
    if (a->D == 64) TD_VALU(float, 64); else TD_VALU(float, 128);
#undef TD_VALU
  }
  return hipGetLastError() == hipSuccess ? TD_OK : TD_ERR_HIP;
}

int launch_step_tail(const td_attn_args *a, const AttnPlan &p, void *ws, const td_commit_args *c,
                     const CommitPlan &pc, void *ws_commit, void *stream, const int32_t *gate) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char *wsb = static_cast<char *>(ws);
  const bool many = many_pieces(p);
  const int64_t merge_blocks = p.units * 8 * (many ? 4 : 1);
  const int64_t fin_blocks = (int64_t(c->B) + 3) / 4;
  auto k = many ? step_tail<8, 4> : step_tail<4, 1>;
  hipLaunchKernelGGL(k, dim3(unsigned(merge_blocks + fin_blocks)), dim3(256), 0, st,
                     reinterpret_cast<int64_t *>(wsb + p.off_prefix), a->B, a->S, a->Hq, a->Hkv, p.G,
                     p.M, p.row_groups, p.launch, reinterpret_cast<float2 *>(wsb + p.off_ml),
                     reinterpret_cast<bf16 *>(wsb + p.off_o), static_cast<bf16 *>(a->out),
                     merge_blocks, static_cast<const Part *>(ws_commit), pc.R, c->gamma, c->masked_in,
                     c->commit, c->token, c->maxprob, c->n_commit, c->masked_out, c->tokens,
                     c->n_masked_left, gate);
  return hipGetLastError() == hipSuccess ? TD_OK : TD_ERR_HIP;
}

}  // namespace td
