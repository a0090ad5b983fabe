// The commit's block decision for one sequence, done by one wave (news.
// chathome.org, "NVIDIA releases Nemotron-Labs-TwoTower ...", evaluation
// paragraph: confidence masking with threshold gamma; block-generation
// paragraph: several positions may commit per step and every block
// finishes).  Shared by commit_finalize (td_commit.hip) and the step's tail
// kernel, which runs it beside the attention merge (td_attn.hip).
//
// Lane i < S handles position i: it merges the R parts of its row in slice
// order (max, lowest index attaining it, sum of exp rescaled to the common
// max), sets p = 1/Z, and the wave then applies p >= gamma to the eligible
// positions and the force-one rule (largest p among the eligible, lowest
// position on ties), writes the outputs and adds the positions still masked
// to n_masked_left.
#pragma once

#include <hip/hip_runtime.h>

#include "td_internal.h"

namespace td {
namespace fin {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kNoIndex = 0x7fffffff;

__device__ __forceinline__ void finalize_seq(
    int b, int i, const Part *__restrict__ parts, int S, int R, float gamma,
    const uint8_t *masked_in, uint8_t *__restrict__ commit, int32_t *__restrict__ token,
    float *__restrict__ maxprob, int32_t *__restrict__ n_commit, uint8_t *masked_out,
    int32_t *__restrict__ tokens, int32_t *__restrict__ n_masked_left, bool skip_inelig) {
  const bool act = i < S;
  const int64_t row = int64_t(b) * S + i;
  float p = 0.f;
  int idx = 0;
  bool elig = false;
  if (act) elig = masked_in ? masked_in[row] != 0 : true;
  if (act && skip_inelig && !elig) {
    idx = -1;                        // not scored: no parts were made for it
  } else if (act) {
    float M = -__builtin_inff();
    for (int r = 0; r < R; ++r) M = fmaxf(M, parts[row * R + r].m);
    float Z = 0.f;
    idx = kNoIndex;
    for (int r = 0; r < R; ++r) {
      const Part q = parts[row * R + r];
      if (q.m == M && q.idx < idx) idx = q.idx;
      Z += (q.m == -__builtin_inff()) ? 0.f : q.z * __builtin_amdgcn_exp2f((q.m - M) * kLog2e);
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

}  // namespace fin
}  // namespace td
