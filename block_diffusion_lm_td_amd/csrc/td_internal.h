// Internal declarations shared by the host library's translation units.
// Not part of the public ABI (include/td.h is).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "td.h"

namespace td {

// Tiling constants of the bf16 MFMA attention kernel.
constexpr int kRowsPerWG = 256;   // query rows (G*S rows of one KV head) per workgroup
constexpr int kKeyTile = 64;      // keys per LDS tile
constexpr int kWaves = 8;         // 8 waves x 32 rows; two waves share each SIMD
constexpr int kWGThreads = 64 * kWaves;
constexpr int kGridWGs = 256;     // persistent grid: one workgroup per CU of MI355X
constexpr int kDecodeBlockKeys = 32;    // keys per block of the decode path
constexpr int kDecodeWaves = 4;         // waves per decode workgroup
constexpr int kDecodeGridWGs = 256;     // one resident generation: one workgroup per CU
constexpr int kDecodeMinBlocks = 8;     // fewer waves below about 8 blocks each
constexpr int kDecodeMaxB = 4096;       // sequences whose piece table fits the decode kernel's LDS

// Partial of the commit's vocabulary pass over one part of a row (16 bytes).
struct Part {
  float m;    // max of the part
  float z;    // sum exp(x - m) over the part
  int idx;    // lowest index attaining m
  int pad;
};

// Launch plan of one td_block_attn call, derived on the host from sizes only.
struct AttnPlan {
  bool mfma;            // bf16, D == 128: MFMA kernel; otherwise the VALU kernel
  bool decode;          // bf16, D == 128, M <= 16: the decode kernels (units = partial slots)
  int G;                // Hq / Hkv
  int M;                // G * S query rows per (b, kv head)
  int row_groups;       // ceil(M / kRowsPerWG) (MFMA) or ceil(M / 64) (VALU)
  int grid;             // persistent workgroups the workspace holds slots for (MFMA path)
  int launch;           // workgroups launched (<= grid): fewer when the key tiles are few
  int64_t units;        // B * Hkv * row_groups
  // workspace pieces (byte offsets), MFMA path
  size_t off_prefix;    // int64 [B+1]: tile prefix over sequences (for the merge)
  size_t off_ml;        // float2 [2*grid][256]: partial (m, l)
  size_t off_o;         // bf16 [2*grid][256*128]: partial O / l
  size_t ws_bytes;      // total
  float scale_log2;     // scale * log2(e)
};

struct CommitPlan {
  int R;                // workgroups per row
  int span;             // elements per workgroup (multiple of the vector width)
  bool vec;             // 16-byte vector loads usable
  int64_t rows;         // B * S
  size_t ws_bytes;
};

// Host-side validation and planning (td_plan.cpp): pure functions.
int validate_attn(const td_attn_args *a, bool check_ptrs);
int validate_commit(const td_commit_args *c, bool check_ptrs);
int validate_append(const td_append_args *p);
int validate_lmhead(const td_lmhead_args *a, bool check_ptrs);
int validate_mamba(const td_mamba_args *a);
int validate_adaln(const td_adaln_args *a);
AttnPlan plan_attn(const td_attn_args *a);
CommitPlan plan_commit(const td_commit_args *c);

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Launchers (td_attn.hip / td_commit.hip); return a td_status.
// gate: NULL, or a device int32 that every kernel reads first; 0 = do nothing
// (the commit still clears n_masked_left)
// merge = false (MFMA path only): the main kernel alone; the merge then runs in
// launch_step_tail
int launch_attn(const td_attn_args *a, const AttnPlan &p, void *ws, void *stream,
                const int32_t *gate = nullptr, bool merge = true);
// merge = false: the streaming kernel alone; the merge then runs in
// launch_decode_step_tail
int launch_attn_decode(const td_attn_args *a, const AttnPlan &p, void *ws, void *stream,
                       const int32_t *gate = nullptr, bool merge = true);
// finalize = false: the row pass alone; the decision then runs in launch_step_tail
int launch_commit(const td_commit_args *c, const CommitPlan &p, void *ws, void *stream,
                  const int32_t *gate = nullptr, bool finalize = true);
// the tail of a denoise step on the MFMA attention path, in one launch: the
// attention merge and the commit's decision (td_attn.hip); ws is the
// attention's workspace, ws_commit the commit's
int launch_step_tail(const td_attn_args *a, const AttnPlan &p, void *ws, const td_commit_args *c,
                     const CommitPlan &pc, void *ws_commit, void *stream, const int32_t *gate);
// the same on the decode attention path: the decode merge and the commit's
// decision in one launch (td_decode.hip)
int launch_decode_step_tail(const td_attn_args *a, const AttnPlan &p, void *ws,
                            const td_commit_args *c, const CommitPlan &pc, void *ws_commit,
                            void *stream, const int32_t *gate);
int launch_append(const td_append_args *p, void *stream);
// the commit's per-sequence decision over R parts per position (td_commit.hip)
int launch_commit_finalize(const Part *parts, int R, int B, int S, float gamma,
                           const uint8_t *masked_in, uint8_t *commit, int32_t *token,
                           float *maxprob, int32_t *n_commit, uint8_t *masked_out,
                           int32_t *tokens, int32_t *n_masked_left, void *stream,
                           const int32_t *gate = nullptr, bool skip_ineligible = false);
// fused LM head + commit (td_lmhead.hip): workspace = parts, one merged part
// per position, then the compacted position list and its count
size_t lmhead_parts_bytes(const td_lmhead_args *a);
inline size_t lmhead_ws_bytes(const td_lmhead_args *a) {
  const size_t M = size_t(a->B) * a->S;
  return align256(lmhead_parts_bytes(a)) + align256(M * sizeof(Part)) + (M + 1) * sizeof(int32_t);
}
int launch_lmhead(const td_lmhead_args *a, void *ws, void *stream);
size_t lmhead_packed_bytes(int32_t V, int32_t H);
int validate_lmhead_pack(const void *w_head, int32_t V, int32_t H, const void *w_packed);
int launch_lmhead_pack(const void *w_head, int32_t V, int32_t H, void *w_packed, void *stream);
int launch_mamba(const td_mamba_args *a, void *stream);
int launch_adaln(const td_adaln_args *a, void *stream);
// device address of the library-held scratch array on the current device
// (td_noalloc.hip); looked up once per device, TD_ERR_HIP if that fails
int noalloc_scratch(void **ptr);

}  // namespace td
