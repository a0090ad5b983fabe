// extern "C" entry points of libtd.so (declared and documented in td.h).
// Validation and planning happen here, on the host, before anything is
// enqueued; the launchers live in td_attn.hip / td_commit.hip / td_lmhead.hip /
// td_mamba.hip / td_adaln.hip / td_append.hip, the library-held scratch of
// td_denoise_step_noalloc in td_noalloc.hip.
#include <stdint.h>

#include "td_internal.h"

using namespace td;

namespace {

int check_ws(size_t need, void *ws, size_t ws_bytes) {
  if (need == 0) return TD_OK;
  if (!ws || ws_bytes < need || (reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return TD_ERR_WORKSPACE;
  return TD_OK;
}

int attn_launch(const td_attn_args *a, const AttnPlan &p, void *ws, td_stream_t stream,
                const int32_t *gate) {
  return p.decode ? launch_attn_decode(a, p, ws, stream, gate) : launch_attn(a, p, ws, stream, gate);
}

int denoise(const td_attn_args *a, const td_commit_args *c, const int32_t *gate, void *ws,
            size_t ws_bytes, td_stream_t stream) {
  int rc = validate_attn(a, true);
  if (rc != TD_OK) return rc;
  rc = validate_commit(c, true);
  if (rc != TD_OK) return rc;
  if (a->B != c->B || a->S != c->S) return TD_ERR_INVALID;
  const AttnPlan pa = plan_attn(a);
  const CommitPlan pc = plan_commit(c);
  const size_t wa = align256(pa.ws_bytes), wc = align256(pc.ws_bytes);
  rc = check_ws(wa + wc, ws, ws_bytes);
  if (rc != TD_OK) return rc;
  char *wsc = static_cast<char *>(ws) + wa;
  if (!pa.mfma) {
    rc = attn_launch(a, pa, ws, stream, gate);
    if (rc != TD_OK) return rc;
    return launch_commit(c, pc, wsc, stream, gate);
  }
  if (pa.decode) {
    // decode path: the streaming kernel, the commit's row pass, then one
    // launch for the decode merge and the commit decision
    rc = launch_attn_decode(a, pa, ws, stream, gate, false);
    if (rc != TD_OK) return rc;
    rc = launch_commit(c, pc, wsc, stream, gate, false);
    if (rc != TD_OK) return rc;
    return launch_decode_step_tail(a, pa, ws, c, pc, wsc, stream, gate);
  }
  // MFMA path: attention main kernel, the commit's row pass, then one launch
  // for both small tails (attention merge + commit decision)
  rc = launch_attn(a, pa, ws, stream, gate, false);
  if (rc != TD_OK) return rc;
  rc = launch_commit(c, pc, wsc, stream, gate, false);
  if (rc != TD_OK) return rc;
  return launch_step_tail(a, pa, ws, c, pc, wsc, stream, gate);
}

}  // namespace

extern "C" {

uint32_t td_abi_version(void) { return TD_ABI_VERSION; }
size_t td_sizeof_attn_args(void) { return sizeof(td_attn_args); }
size_t td_sizeof_commit_args(void) { return sizeof(td_commit_args); }
size_t td_sizeof_append_args(void) { return sizeof(td_append_args); }
size_t td_sizeof_lmhead_args(void) { return sizeof(td_lmhead_args); }
size_t td_sizeof_mamba_args(void) { return sizeof(td_mamba_args); }
size_t td_sizeof_adaln_args(void) { return sizeof(td_adaln_args); }

const char *td_status_str(int status) {
  switch (status) {
    case TD_OK: return "TD_OK";
    case TD_ERR_INVALID: return "TD_ERR_INVALID: invalid argument";
    case TD_ERR_UNSUPPORTED: return "TD_ERR_UNSUPPORTED: valid but unsupported configuration";
    case TD_ERR_WORKSPACE: return "TD_ERR_WORKSPACE: workspace missing, too small or not 256-byte aligned";
    case TD_ERR_HIP: return "TD_ERR_HIP: HIP runtime error at launch";
    default: return "unknown td_status";
  }
}

size_t td_attn_workspace_bytes(const td_attn_args *a) {
  if (validate_attn(a, false) != TD_OK) return 0;
  return plan_attn(a).ws_bytes;
}

size_t td_commit_workspace_bytes(const td_commit_args *c) {
  if (validate_commit(c, false) != TD_OK) return 0;
  return plan_commit(c).ws_bytes;
}

size_t td_denoise_workspace_bytes(const td_attn_args *a, const td_commit_args *c) {
  if (validate_attn(a, false) != TD_OK || validate_commit(c, false) != TD_OK) return 0;
  return align256(plan_attn(a).ws_bytes) + align256(plan_commit(c).ws_bytes);
}

size_t td_lmhead_commit_workspace_bytes(const td_lmhead_args *a) {
  if (validate_lmhead(a, false) != TD_OK) return 0;
  return lmhead_ws_bytes(a);
}

int td_block_attn(const td_attn_args *a, void *ws, size_t ws_bytes, td_stream_t stream) {
  int rc = validate_attn(a, true);
  if (rc != TD_OK) return rc;
  const AttnPlan p = plan_attn(a);
  rc = check_ws(p.ws_bytes, ws, ws_bytes);
  if (rc != TD_OK) return rc;
  return attn_launch(a, p, ws, stream, nullptr);
}

int td_commit(const td_commit_args *c, void *ws, size_t ws_bytes, td_stream_t stream) {
  int rc = validate_commit(c, true);
  if (rc != TD_OK) return rc;
  const CommitPlan p = plan_commit(c);
  rc = check_ws(p.ws_bytes, ws, ws_bytes);
  if (rc != TD_OK) return rc;
  return launch_commit(c, p, ws, stream);
}

int td_denoise_step(const td_attn_args *a, const td_commit_args *c, void *ws, size_t ws_bytes,
                    td_stream_t stream) {
  return denoise(a, c, nullptr, ws, ws_bytes, stream);
}

int td_denoise_step_noalloc(const td_attn_args *a, const td_commit_args *c, td_stream_t stream) {
  // validate and size first: a bad or oversized call is rejected before the
  // scratch array is looked up
  int rc = validate_attn(a, true);
  if (rc != TD_OK) return rc;
  rc = validate_commit(c, true);
  if (rc != TD_OK) return rc;
  if (a->B != c->B || a->S != c->S) return TD_ERR_INVALID;
  if (td_denoise_workspace_bytes(a, c) > TD_NOALLOC_SCRATCH_BYTES) return TD_ERR_WORKSPACE;
  void *ws = nullptr;
  rc = noalloc_scratch(&ws);
  if (rc != TD_OK) return rc;
  return denoise(a, c, nullptr, ws, TD_NOALLOC_SCRATCH_BYTES, stream);
}

int td_denoise_step_if(const td_attn_args *a, const td_commit_args *c, const int32_t *gate,
                       void *ws, size_t ws_bytes, td_stream_t stream) {
  if (!gate || !c || gate == c->n_masked_left) return TD_ERR_INVALID;
  return denoise(a, c, gate, ws, ws_bytes, stream);
}

int td_lmhead_commit(const td_lmhead_args *a, void *ws, size_t ws_bytes, td_stream_t stream) {
  int rc = validate_lmhead(a, true);
  if (rc != TD_OK) return rc;
  rc = check_ws(lmhead_ws_bytes(a), ws, ws_bytes);
  if (rc != TD_OK) return rc;
  return launch_lmhead(a, ws, stream);
}

size_t td_lmhead_packed_bytes(int32_t V, int32_t H) { return lmhead_packed_bytes(V, H); }

int td_lmhead_pack_head(const void *w_head, int32_t V, int32_t H, void *w_packed, td_stream_t stream) {
  const int rc = validate_lmhead_pack(w_head, V, H, w_packed);
  if (rc != TD_OK) return rc;
  return launch_lmhead_pack(w_head, V, H, w_packed, stream);
}

int td_mamba_block_scan(const td_mamba_args *a, td_stream_t stream) {
  const int rc = validate_mamba(a);
  if (rc != TD_OK) return rc;
  return launch_mamba(a, stream);
}

int td_adaln_modulate(const td_adaln_args *a, td_stream_t stream) {
  const int rc = validate_adaln(a);
  if (rc != TD_OK) return rc;
  if (int64_t(a->B) * a->S == 0) return TD_OK;
  return launch_adaln(a, stream);
}

int td_cache_append(const td_append_args *p, td_stream_t stream) {
  const int rc = validate_append(p);
  if (rc != TD_OK) return rc;
  return launch_append(p, stream);
}

}  // extern "C"
