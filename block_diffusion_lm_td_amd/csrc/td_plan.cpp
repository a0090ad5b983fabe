// Host-side argument validation, launch planning and workspace sizing of the
// td_* entry points.  No HIP calls: everything here is plain C++ on sizes.
#include <math.h>
#include <stdlib.h>

#include <algorithm>

#include "td_internal.h"

namespace td {

static bool finite_f(float x) { return isfinite(x) != 0; }

int validate_attn(const td_attn_args *a, bool check_ptrs) {
  if (!a) return TD_ERR_INVALID;
  if (a->B < 1 || a->S < 1 || a->S > 64 || a->Hq < 1 || a->Hkv < 1) return TD_ERR_INVALID;
  if (a->B > 65535 || a->Hkv > 4096) return TD_ERR_UNSUPPORTED;   // launch-grid limits
  if (int64_t(a->B) * a->Hkv * ((int64_t(a->Hq / a->Hkv) * a->S + 255) / 256) > (int64_t(1) << 30))
    return TD_ERR_UNSUPPORTED;
  if (a->Hq % a->Hkv != 0) return TD_ERR_INVALID;
  if (a->Hq / a->Hkv > 64) return TD_ERR_UNSUPPORTED;
  if (a->dtype != TD_F32 && a->dtype != TD_BF16) return TD_ERR_INVALID;
  if (a->D != 64 && a->D != 128) return TD_ERR_UNSUPPORTED;
  if (!(a->scale == a->scale) || isinf(a->scale)) return TD_ERR_INVALID;
  if (a->total_ctx < 0 || a->max_ctx < 0 || a->max_ctx > a->total_ctx) return TD_ERR_INVALID;
  if (a->max_ctx > (int64_t(1) << 30)) return TD_ERR_UNSUPPORTED;
  if (a->total_ctx > (int64_t(1) << 40) / (int64_t(a->Hkv) * a->D)) return TD_ERR_UNSUPPORTED;
  // every sequence is at most max_ctx long, so total <= B * max
  if (a->total_ctx > int64_t(a->B) * a->max_ctx) return TD_ERR_INVALID;
  if (int64_t(a->B) * a->S * a->Hq * a->D > (int64_t(1) << 40)) return TD_ERR_UNSUPPORTED;
  if (check_ptrs) {
    if (!a->q || !a->k_blk || !a->v_blk || !a->out || !a->ctx_offsets) return TD_ERR_INVALID;
    if (a->total_ctx > 0 && (!a->k_ctx || !a->v_ctx)) return TD_ERR_INVALID;
  }
  return TD_OK;
}

int validate_commit(const td_commit_args *c, bool check_ptrs) {
  if (!c) return TD_ERR_INVALID;
  if (c->B < 1 || c->S < 1 || c->S > 64 || c->V < 1) return TD_ERR_INVALID;
  if (c->dtype != TD_F32 && c->dtype != TD_BF16) return TD_ERR_INVALID;
  if (!finite_f(c->gamma)) return TD_ERR_INVALID;
  if (int64_t(c->B) * c->S * int64_t(c->V) > (int64_t(1) << 40)) return TD_ERR_UNSUPPORTED;
  if (int64_t(c->B) * c->S > (int64_t(1) << 24)) return TD_ERR_UNSUPPORTED;
  if (check_ptrs) {
    if (!c->logits || !c->commit || !c->token) return TD_ERR_INVALID;
  }
  return TD_OK;
}

static int grid_override() {
  const char *env = getenv("TD_ATTN_GRID");
  if (env && atoi(env) >= 1 && atoi(env) <= 4096) return atoi(env);
  return 0;
}

// Workgroups to launch for an estimated W key tiles: one per CU while every
// workgroup gets at least kMinTilesPerWG tiles, fewer below that, where the
// per-segment start and the partials would outweigh the extra bandwidth
// (B = 8 x 4K context: 29.6 us on 160 workgroups against 32.1 us on 256).
// A multiple of 8 keeps the XCD-aware workgroup mapping.  The choice only
// affects speed: any grid computes the same result.
static constexpr int64_t kMinTilesPerWG = 6;
static int launch_wgs(int64_t tiles_est, int grid) {
  int64_t n = (tiles_est + kMinTilesPerWG - 1) / kMinTilesPerWG;
  n = (n + 7) / 8 * 8;
  return int(std::max<int64_t>(8, std::min<int64_t>(n, grid)));
}

AttnPlan plan_attn(const td_attn_args *a) {
  AttnPlan p{};
  p.G = a->Hq / a->Hkv;
  p.M = p.G * a->S;
  p.mfma = (a->dtype == TD_BF16 && a->D == 128);
  float scale = a->scale > 0.f ? a->scale : 1.0f / sqrtf(float(a->D));
  p.scale_log2 = scale * 1.4426950408889634f;
  if (p.mfma) {
    p.row_groups = (p.M + kRowsPerWG - 1) / kRowsPerWG;
    p.units = int64_t(a->B) * a->Hkv * p.row_groups;
    const int forced = grid_override();
    p.grid = forced ? forced : kGridWGs;
    // key tiles: sum over sequences of ceil((L_b + S) / 64), estimated from
    // the total context (the lengths themselves are on the device)
    const int64_t seq_tiles = (a->total_ctx + int64_t(a->B) * a->S) / kKeyTile + (a->B + 1) / 2;
    p.launch = forced ? forced : launch_wgs(int64_t(a->Hkv) * p.row_groups * seq_tiles, p.grid);
    size_t o = 0;
    p.off_prefix = o; o += align256(size_t(a->B + 1) * 8);
    p.off_ml = o;     o += align256(size_t(2) * p.grid * kRowsPerWG * 8);
    p.off_o = o;      o += align256(size_t(2) * p.grid * kRowsPerWG * 128 * 2);
    p.ws_bytes = o;
  } else {
    p.row_groups = (p.M + 63) / 64;
    p.units = int64_t(a->B) * a->Hkv * p.row_groups;
    p.ws_bytes = 0;
  }
  return p;
}

CommitPlan plan_commit(const td_commit_args *c) {
  CommitPlan p{};
  p.rows = int64_t(c->B) * c->S;
  int esz = c->dtype == TD_BF16 ? 2 : 4;
  int vw = 16 / esz;
  p.vec = (int64_t(c->V) * esz) % 16 == 0 &&
          (reinterpret_cast<uintptr_t>(c->logits) % 16) == 0;
  // Enough workgroups to cover the chip several times over, but each one
  // streams at least 16K elements so the per-row partials stay negligible.
  int64_t target = 2048;
  int R = int((target + p.rows - 1) / p.rows);
  int64_t maxR = std::max<int64_t>(1, c->V / 16384);
  R = int(std::max<int64_t>(1, std::min<int64_t>(R, maxR)));
  const char *env = getenv("TD_COMMIT_SPLIT");
  if (env && atoi(env) >= 1) R = std::min(atoi(env), std::max(1, c->V / vw));
  int64_t span = (int64_t(c->V) + R - 1) / R;
  span = (span + vw - 1) / vw * vw;
  R = int((int64_t(c->V) + span - 1) / span);
  p.R = R;
  p.span = int(span);
  p.ws_bytes = align256(size_t(p.rows) * R * 16);
  return p;
}

}  // namespace td
