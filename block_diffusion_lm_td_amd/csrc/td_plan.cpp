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
  // bf16 runs on the MFMA kernels, which are built for D = 128 only
  if (a->dtype == TD_BF16 && a->D != 128) return TD_ERR_UNSUPPORTED;
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

namespace {
struct Range {
  uintptr_t lo, hi;   // [lo, hi), empty when lo == hi
};
bool overlap(Range a, Range b) { return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi; }
Range range(const void *p, int64_t bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return {lo, p ? lo + uintptr_t(bytes) : lo};
}
bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
}  // namespace

int validate_append(const td_append_args *p) {
  if (!p) return TD_ERR_INVALID;
  if (p->B < 1 || p->S < 0 || p->S > 65536 || p->Hkv < 1 || p->D < 1) return TD_ERR_INVALID;
  if (p->dtype != TD_F32 && p->dtype != TD_BF16) return TD_ERR_INVALID;
  if (p->total_ctx < 0) return TD_ERR_INVALID;
  const int64_t esize = p->dtype == TD_BF16 ? 2 : 4;
  const int64_t row = int64_t(p->Hkv) * p->D * esize;
  if (row % 16 != 0 || row > 65536) return TD_ERR_UNSUPPORTED;
  if (p->B > (1 << 24)) return TD_ERR_UNSUPPORTED;
  const int64_t n_new = int64_t(p->B) * p->S;
  const int64_t N = p->total_ctx + n_new;
  // one workgroup per 16 output rows: the grid stays below 2^31 workgroups
  if (N > (int64_t(1) << 34) || N * row > (int64_t(1) << 42)) return TD_ERR_UNSUPPORTED;
  if (!p->ctx_offsets || !p->offsets_out) return TD_ERR_INVALID;
  if (p->total_ctx > 0 && (!p->k_ctx || !p->v_ctx)) return TD_ERR_INVALID;
  if (n_new > 0 && (!p->k_new || !p->v_new)) return TD_ERR_INVALID;
  if (N > 0 && (!p->k_out || !p->v_out)) return TD_ERR_INVALID;
  for (const void *q : {p->k_ctx, p->v_ctx, p->k_new, p->v_new, (const void *)p->k_out,
                        (const void *)p->v_out})
    if (!aligned16(q)) return TD_ERR_INVALID;
  if ((reinterpret_cast<uintptr_t>(p->ctx_offsets) & 7u) != 0 ||
      (reinterpret_cast<uintptr_t>(p->offsets_out) & 7u) != 0)
    return TD_ERR_INVALID;
  const Range ins[] = {range(p->k_ctx, p->total_ctx * row), range(p->v_ctx, p->total_ctx * row),
                       range(p->k_new, n_new * row), range(p->v_new, n_new * row),
                       range(p->ctx_offsets, (int64_t(p->B) + 1) * 8)};
  const Range outs[] = {range(p->k_out, N * row), range(p->v_out, N * row),
                        range(p->offsets_out, (int64_t(p->B) + 1) * 8)};
  for (const Range &o : outs)
    for (const Range &i : ins)
      if (overlap(o, i)) return TD_ERR_INVALID;
  for (int x = 0; x < 3; ++x)
    for (int y = x + 1; y < 3; ++y)
      if (overlap(outs[x], outs[y])) return TD_ERR_INVALID;
  return TD_OK;
}

int validate_adaln(const td_adaln_args *a) {
  if (!a) return TD_ERR_INVALID;
  if (a->B < 0 || a->S < 0 || a->H < 1) return TD_ERR_INVALID;
  if (!finite_f(a->eps) || a->eps < 0.f) return TD_ERR_INVALID;
  if (a->H % 8 != 0 || a->H > 8192) return TD_ERR_UNSUPPORTED;
  const int64_t M = int64_t(a->B) * a->S;
  if (M > (int64_t(1) << 30)) return TD_ERR_UNSUPPORTED;
  if (M == 0) return TD_OK;
  if (!a->x || !a->t_mod || !a->h || (a->f && !a->r_out)) return TD_ERR_INVALID;
  const void *r_out = a->f ? a->r_out : nullptr;     // unused without f
  for (const void *q : {a->x, a->f, (const void *)a->t_mod, (const void *)a->tab_gate,
                        (const void *)a->tab_shift, (const void *)a->tab_scale,
                        (const void *)a->w_norm, r_out, (const void *)a->h})
    if (!aligned16(q)) return TD_ERR_INVALID;
  const int64_t act = M * a->H * 2, row = int64_t(a->H) * 4;
  const Range ins[] = {range(a->x, act), range(a->f, act), range(a->t_mod, int64_t(a->B) * 3 * row),
                       range(a->tab_gate, row), range(a->tab_shift, row), range(a->tab_scale, row),
                       range(a->w_norm, row)};
  const Range outs[] = {range(r_out, act), range(a->h, act)};
  // r_out may be x itself, h may be x or f itself (each row is read whole
  // before any of it is written); any other overlap with an input is refused
  for (int i = 0; i < 7; ++i) {
    if (overlap(outs[0], ins[i]) && !(i == 0 && r_out == a->x)) return TD_ERR_INVALID;
    if (overlap(outs[1], ins[i]) && !((i == 0 && a->h == a->x) || (i == 1 && a->h == a->f)))
      return TD_ERR_INVALID;
  }
  if (overlap(outs[0], outs[1])) return TD_ERR_INVALID;
  return TD_OK;
}

int validate_lmhead(const td_lmhead_args *a, bool check_ptrs) {
  if (!a) return TD_ERR_INVALID;
  if (a->B < 1 || a->S < 1 || a->S > 64 || a->V < 1 || a->H < 1) return TD_ERR_INVALID;
  if (a->dtype != TD_F32 && a->dtype != TD_BF16) return TD_ERR_INVALID;
  if (!finite_f(a->gamma)) return TD_ERR_INVALID;
  if (a->dtype != TD_BF16) return TD_ERR_UNSUPPORTED;
  if (a->H % 64 != 0 || a->H > 65536 || a->V > (1 << 30)) return TD_ERR_UNSUPPORTED;
  const int64_t M = int64_t(a->B) * a->S;
  const int64_t m_tiles = (M + 255) / 256, n_tiles = (int64_t(a->V) + 255) / 256;
  if (M > (1 << 24) || m_tiles * n_tiles > (int64_t(1) << 31) - 1) return TD_ERR_UNSUPPORTED;
  if (M * a->H * 2 >= (int64_t(1) << 32)) return TD_ERR_UNSUPPORTED;   // 32-bit row offsets
  if (a->w_head_packed != 0 && a->w_head_packed != 1) return TD_ERR_INVALID;
  if (check_ptrs) {
    if (!a->hidden || !a->w_head || !a->commit || !a->token) return TD_ERR_INVALID;
    if (!aligned16(a->hidden) || !aligned16(a->w_head)) return TD_ERR_INVALID;
  }
  return TD_OK;
}

size_t lmhead_packed_bytes(int32_t V, int32_t H) {
  if (V < 1 || V > (1 << 30) || H < 64 || H > 65536 || H % 64 != 0) return 0;
  return size_t((int64_t(V) + 255) / 256) * 256 * size_t(H) * 2;
}

int validate_lmhead_pack(const void *w_head, int32_t V, int32_t H, const void *w_packed) {
  if (V < 1 || H < 1) return TD_ERR_INVALID;
  if (lmhead_packed_bytes(V, H) == 0) return TD_ERR_UNSUPPORTED;
  if (!w_head || !w_packed || !aligned16(w_head) || !aligned16(w_packed)) return TD_ERR_INVALID;
  if (overlap(range(w_head, int64_t(V) * H * 2), range(w_packed, int64_t(lmhead_packed_bytes(V, H)))))
    return TD_ERR_INVALID;
  return TD_OK;
}

int validate_mamba(const td_mamba_args *a) {
  if (!a) return TD_ERR_INVALID;
  if (a->B < 1 || a->S < 1 || a->H < 1 || a->P < 1 || a->N < 1 || a->G < 1) return TD_ERR_INVALID;
  if (a->H % a->G != 0) return TD_ERR_INVALID;
  if (a->S > 16) return TD_ERR_UNSUPPORTED;
  if (a->P != 16 && a->P != 32 && a->P != 64 && a->P != 128) return TD_ERR_UNSUPPORTED;
  if (a->N % 32 != 0 || a->N > 1024) return TD_ERR_UNSUPPORTED;
  if (int64_t(a->B) * a->H > (int64_t(1) << 31) - 4) return TD_ERR_UNSUPPORTED;
  if (!a->x || !a->dt || !a->A || !a->Bm || !a->Cm || !a->D || !a->h0 || !a->y) return TD_ERR_INVALID;
  if (!aligned16(a->x) || !aligned16(a->Bm) || !aligned16(a->Cm) || !aligned16(a->h0)) return TD_ERR_INVALID;
  if (reinterpret_cast<uintptr_t>(a->y) & 7u) return TD_ERR_INVALID;
  return TD_OK;
}

static int decode_grid_override() {
  const char *env = getenv("TD_DECODE_GRID");
  if (env && atoi(env) >= 1 && atoi(env) <= 4096) return atoi(env);
  return 0;
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
  p.decode = p.mfma && p.M <= 16 && a->B <= kDecodeMaxB;
  if (p.decode) {
    // blocks of kDecodeBlockKeys keys: sum over sequences of
    // ceil((L_b + S) / 32) <= (total + B*S) / 32 + B, per KV head; one
    // resident generation of waves, fewer when they would get under
    // kDecodeMinBlocks blocks each.  Two partial slots per wave.  The choice
    // only affects speed: any grid computes the same function.
    p.row_groups = 1;
    const int64_t blocks = int64_t(a->Hkv) * ((a->total_ctx + int64_t(a->B) * a->S) / kDecodeBlockKeys + a->B);
    int64_t wgs = (blocks + int64_t(kDecodeWaves) * kDecodeMinBlocks - 1) / (int64_t(kDecodeWaves) * kDecodeMinBlocks);
    wgs = std::max<int64_t>(1, std::min<int64_t>(wgs, kDecodeGridWGs));
    const int forced = decode_grid_override();
    p.launch = forced ? forced : int(wgs);
    p.units = int64_t(2) * p.launch * kDecodeWaves;
    size_t o = 0;
    p.off_prefix = o; o += align256(size_t(a->B + 1) * 8);
    p.off_ml = o;     o += align256(size_t(p.units) * 16 * 8);
    p.off_o = o;      o += align256(size_t(p.units) * 16 * 128 * 2);
    p.ws_bytes = o;
  } else if (p.mfma) {
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
