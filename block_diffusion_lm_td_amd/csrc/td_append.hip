// Context-cache append on gfx950 (news.chathome.org, "NVIDIA releases
// Nemotron-Labs-TwoTower ...", block-generation paragraph: after a block has
// committed, the context tower takes in its tokens and the per-layer KV cache
// grows by them).
//
// The packed cache moves sequence b down by b*S rows and follows its L_b old
// rows with the block's S new rows.  The copy is laid out over OUTPUT rows:
// workgroup i owns rows [i*kRows, (i+1)*kRows) of k_out and of v_out, a
// contiguous byte range of each, so every output row is written exactly once
// and the stores stream linearly.  Before copying, kRows lanes find each of
// those rows' source (a context row or a new row) by a binary search over the
// shifted offsets off[b] + b*S and leave it in LDS; then all four waves copy
// K and V in 16-byte vectors, every load of a workgroup in flight before the
// first store.  The work is pure HBM streaming: 2 * row bytes read and
// written per output row, no arithmetic.
#include <hip/hip_runtime.h>

#include "td_internal.h"

namespace td {
namespace {

// Small workgroups: at 2 x 128 bf16 per row a workgroup moves 16 KiB of K and
// 16 KiB of V (two 16-byte vectors per thread and tensor), and the ~18.6K
// workgroups of a 64 x 1K..8K cache keep every CU's queue full to the end.
// Measured on that cache (297K output rows): 16 rows 102.5 us, 32 rows 108.0,
// 64 rows 114.7, 128 rows 117.7 (all with non-temporal loads and stores);
// torch's device copy of the same bytes takes 113.7 us.
constexpr int kThreads = 256;
constexpr int kRows = 16;         // output rows per workgroup
constexpr int kMaxVecsPerThread = 8;   // 16-byte vectors in flight per thread and tensor

// Every source row is read once and every output row written once, and the
// cache is larger than the last-level cache: non-temporal loads and stores
// keep the stream out of the caches (64-row workgroups: 119.3 us with plain
// stores, 114.6 with non-temporal ones; plain loads cost another 3.6 us).
typedef unsigned int u32x4n __attribute__((ext_vector_type(4)));
__device__ inline u32x4n ldnt(const u32x4n *p) { return __builtin_nontemporal_load(p); }
__device__ inline void stnt(u32x4n v, u32x4n *p) { __builtin_nontemporal_store(v, p); }

__device__ inline int64_t clamp64(int64_t x, int64_t lo, int64_t hi) {
  return x < lo ? lo : (x > hi ? hi : x);
}

// row_vecs: 16-byte vectors per row (Hkv*D*element size / 16, at most 4096);
// N: output rows (total_ctx + B*S).
__global__ __launch_bounds__(kThreads) void cache_append_rows(
    const u32x4n *__restrict__ k_ctx, const u32x4n *__restrict__ v_ctx,
    const int64_t *__restrict__ off, int64_t T, const u32x4n *__restrict__ k_new,
    const u32x4n *__restrict__ v_new, int B, int S, int row_vecs, u32x4n *__restrict__ k_out,
    u32x4n *__restrict__ v_out, int64_t *__restrict__ off_out, int64_t N) {
  __shared__ int64_t src[kRows];   // >= 0: context row; < 0: -(1 + b*S + s), new row s of b
  const int tid = threadIdx.x;
  const int64_t r0 = int64_t(blockIdx.x) * kRows;
  if (blockIdx.x == 0) {
    for (int b = tid; b <= B; b += kThreads) off_out[b] = clamp64(off[b], 0, T) + int64_t(b) * S;
  }
  // shifted start of sequence b in the output, off[b] clamped into [0, T]
  auto out_start = [&](int b) { return clamp64(off[b], 0, T) + int64_t(b) * S; };
  if (tid < kRows && r0 + tid < N) {
    const int64_t r = r0 + tid;
    int lo = 0, hi = B;            // the last b in [0, B) with out_start(b) <= r
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (out_start(mid) <= r) lo = mid;
      else hi = mid;
    }
    const int64_t st = clamp64(off[lo], 0, T);
    const int64_t en = clamp64(off[lo + 1], st, T);
    const int64_t j = r - (st + int64_t(lo) * S) > 0 ? r - (st + int64_t(lo) * S) : 0;
    const int64_t L = en - st;
    // S == 0 only with inconsistent offsets can reach j >= L: any in-bounds
    // context row will do then (T >= 1 since N >= 1)
    src[tid] = (j < L || S == 0) ? clamp64(st + j, 0, T - 1)
                                 : -(1 + int64_t(lo) * S + (j - L < S ? j - L : S - 1));
  }
  __syncthreads();

  const int64_t rows = N - r0 < kRows ? N - r0 : kRows;
  const int total = int(rows) * row_vecs;
  const int64_t out0 = r0 * row_vecs;
  for (int base = 0; base < total; base += kThreads * kMaxVecsPerThread) {
    u32x4n kv[kMaxVecsPerThread], vv[kMaxVecsPerThread];
#pragma unroll
    for (int u = 0; u < kMaxVecsPerThread; ++u) {
      const int e = base + u * kThreads + tid;
      if (e < total) {
        const int row = e / row_vecs;
        const int vec = e - row * row_vecs;
        const int64_t s = src[row];
        const int64_t idx = (s >= 0 ? s : -1 - s) * row_vecs + vec;
        kv[u] = ldnt((s >= 0 ? k_ctx : k_new) + idx);
        vv[u] = ldnt((s >= 0 ? v_ctx : v_new) + idx);
      }
    }
#pragma unroll
    for (int u = 0; u < kMaxVecsPerThread; ++u) {
      const int e = base + u * kThreads + tid;
      if (e < total) {
        stnt(kv[u], k_out + out0 + e);
        stnt(vv[u], v_out + out0 + e);
      }
    }
  }
}

}  // namespace

int launch_append(const td_append_args *p, void *stream) {
  const int64_t esize = p->dtype == TD_BF16 ? 2 : 4;
  const int row_vecs = int(int64_t(p->Hkv) * p->D * esize / 16);
  const int64_t N = p->total_ctx + int64_t(p->B) * p->S;
  const int64_t blocks = N > 0 ? (N + kRows - 1) / kRows : 1;
  hipLaunchKernelGGL(cache_append_rows, dim3(unsigned(blocks)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream),
                     static_cast<const u32x4n *>(p->k_ctx), static_cast<const u32x4n *>(p->v_ctx),
                     p->ctx_offsets, p->total_ctx, static_cast<const u32x4n *>(p->k_new),
                     static_cast<const u32x4n *>(p->v_new), p->B, p->S, row_vecs,
                     static_cast<u32x4n *>(p->k_out), static_cast<u32x4n *>(p->v_out),
                     p->offsets_out, N);
  return hipGetLastError() == hipSuccess ? TD_OK : TD_ERR_HIP;
}

}  // namespace td
