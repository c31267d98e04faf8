// C ABI of the fused linear cross-entropy library: argument validation,
// planning (tile counts, vocabulary splits and chunks, workspace layout) and
// the entry points.  Validation runs on the host before any HIP call.
#include <math.h>
#include <string.h>

#include "flce_internal.h"

namespace flce {

static size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Scratch budget for the dlogits chunk (N_pad x Vc elements).
static constexpr size_t kDlogitsBudget = size_t(512) << 20;
static constexpr int64_t kMaxChunkTiles = 128;
// grad_hidden K splits: at least this many 64-row stages each, partials within this budget
static constexpr int64_t kMinStagesPerPart = 8;
static constexpr size_t kGhPartBudget = size_t(256) << 20;
// Number of compute units the forward split count is sized for (MI355X).
static constexpr int64_t kTargetWorkgroups = 256;

void plan_gh_split(int64_t tiles, int64_t cvn, int esize, int64_t N, int64_t H, int* parts_out, int* kt_out) {
  const int64_t stages = cvn * esize / 128;   // K stages of 128 bytes per row
  int64_t parts = tiles > 0 ? (kTargetWorkgroups + tiles - 1) / tiles : 1;
  if (parts > stages / kMinStagesPerPart) parts = stages / kMinStagesPerPart;
  const int64_t per_part_bytes = N * H * 4;
  if (per_part_bytes > 0 && parts > (int64_t)(kGhPartBudget / per_part_bytes))
    parts = (int64_t)(kGhPartBudget / per_part_bytes);
  if (parts < 2 || tiles >= kTargetWorkgroups / 2) parts = 1;
  const int64_t kt = (stages + parts - 1) / parts;
  *kt_out = (int)kt;
  *parts_out = (int)((stages + kt - 1) / kt);
}

int forward_splits(int64_t n_tt, int64_t n_vt) {
  int64_t S = n_tt > 0 ? (kTargetWorkgroups + n_tt / 2) / n_tt : 1;
  if (S < 1) S = 1;
  if (S > n_vt) S = n_vt;
  return (int)S;
}

int make_plan(const flce_params* p, Plan* pl) {
  if (!p || !pl) return FLCE_ERR_INVALID_ARG;
  if (p->n_tokens < 0 || p->hidden <= 0 || p->vocab <= 0) return FLCE_ERR_INVALID_ARG;
  if (p->dtype != FLCE_F32 && p->dtype != FLCE_BF16 && p->dtype != FLCE_F16) return FLCE_ERR_INVALID_ARG;
  if (p->grad_weight_dtype != FLCE_F32 && p->grad_weight_dtype != FLCE_BF16 && p->grad_weight_dtype != FLCE_F16)
    return FLCE_ERR_INVALID_ARG;
  if (p->reduction != FLCE_REDUCTION_NONE && p->reduction != FLCE_REDUCTION_SUM &&
      p->reduction != FLCE_REDUCTION_MEAN)
    return FLCE_ERR_INVALID_ARG;
  if ((p->flags & ~(FLCE_ACCUMULATE_GRAD_WEIGHT | FLCE_ACCUMULATE_GRAD_BIAS | FLCE_TARGETS_INT32 |
                    FLCE_GRAD_WEIGHT_ACCUM_IN_OUTPUT)) != 0 ||
      p->reserved_f != 0.0f)
    return FLCE_ERR_INVALID_ARG;
  if (!isfinite(p->logit_scale) || !isfinite(p->softcap) || !isfinite(p->z_loss) || p->z_loss < 0.0f)
    return FLCE_ERR_INVALID_ARG;
  if (p->vocab_chunk < 0) return FLCE_ERR_INVALID_ARG;
  if (p->vocab_chunk % 256 != 0) return FLCE_ERR_UNSUPPORTED;
  if (p->hidden % 8 != 0) return FLCE_ERR_UNSUPPORTED;
  const int esize = p->dtype == FLCE_F32 ? 4 : 2;
  // 32-bit buffer offsets and int indices inside the kernels
  if (p->n_tokens > (int64_t(1) << 30) || p->vocab > (int64_t(1) << 30) || p->hidden > (int64_t(1) << 20))
    return FLCE_ERR_UNSUPPORTED;
  if (p->n_tokens * p->hidden * esize >= (int64_t(1) << 31)) return FLCE_ERR_UNSUPPORTED;

  Plan& P = *pl;
  memset(&P, 0, sizeof(P));
  P.N = p->n_tokens;
  P.H = p->hidden;
  P.V = p->vocab;
  P.ignore_index = p->ignore_index;
  P.dtype = p->dtype;
  P.gw_dtype = p->grad_weight_dtype;
  P.reduction = p->reduction;
  P.accum_gw = (p->flags & FLCE_ACCUMULATE_GRAD_WEIGHT) != 0;
  P.accum_gb = (p->flags & FLCE_ACCUMULATE_GRAD_BIAS) != 0;
  P.tgt_i32 = (p->flags & FLCE_TARGETS_INT32) != 0;
  P.gw_accum_out = (p->flags & FLCE_GRAD_WEIGHT_ACCUM_IN_OUTPUT) != 0;
  P.scale = p->logit_scale;
  P.cap = p->softcap > 0.0f ? p->softcap : 0.0f;
  P.z_loss = p->z_loss;
  P.esize = esize;
  P.n_tt = (P.N + 255) / 256;
  P.n_vt = (P.V + 255) / 256;
  P.n_ht = (P.H + 255) / 256;
  P.N_pad = P.n_tt * 256;
  P.V_pad = P.n_vt * 256;

  // forward: split the vocabulary so that about one workgroup runs per CU
  const int64_t S = forward_splits(P.n_tt, P.n_vt);
  P.S = (int)S;
  P.f_part = kStatusBytes;
  const size_t part_bytes = size_t(5) * S * P.N_pad * 4;
  P.f_blk = align_up(P.f_part + part_bytes, 256);
  const int64_t nblk = P.N > 0 ? (P.N + 255) / 256 : 1;
  P.f_bytes = align_up(P.f_blk + size_t(nblk) * sizeof(BlockPart), 256);

  // backward: vocabulary chunks of the caller's width, or the widest whose
  // dlogits scratch fits the budget
  int64_t max_tiles = kMaxChunkTiles;
  if (p->vocab_chunk > 0) {
    max_tiles = p->vocab_chunk / 256;
  } else if (P.N_pad > 0) {
    const int64_t fit = (int64_t)(kDlogitsBudget / (size_t(P.N_pad) * esize * 256));
    if (fit < max_tiles) max_tiles = fit;
  }
  if (max_tiles < 1) max_tiles = 1;
  P.n_chunks = (int)((P.n_vt + max_tiles - 1) / max_tiles);
  const int64_t tiles_per_chunk = (P.n_vt + P.n_chunks - 1) / P.n_chunks;
  P.Vc = tiles_per_chunk * 256;
  if (P.Vc * P.H * esize >= (int64_t(1) << 31)) return FLCE_ERR_UNSUPPORTED;
  if (P.N_pad * P.Vc * esize >= (int64_t(1) << 31)) return FLCE_ERR_UNSUPPORTED;
  // grad_hidden has only n_ht x n_tt output tiles; when that is well under one
  // workgroup per CU, split each chunk's contraction (K = vocabulary rows) and
  // add the fp32 partials in a fixed order afterwards
  plan_gh_split(P.n_ht * P.n_tt, P.Vc, esize, P.N, P.H, &P.gh_parts, &P.gh_kt_per_part);
  size_t o = kStatusBytes;
  P.b_coefA = o;
  o = align_up(o + size_t(P.N_pad) * 4, 256);
  P.b_coefB = o;
  o = align_up(o + size_t(P.N_pad) * 4, 256);
  P.b_lseL = o;
  o = align_up(o + size_t(P.N_pad) * 4, 256);
  P.b_tgt = o;
  o = align_up(o + size_t(P.N_pad) * 4, 256);
  P.b_D = o;
  o = align_up(o + size_t(P.N_pad) * P.Vc * esize, 256);
  P.b_xt = o;
  o = align_up(o + size_t(P.N_pad) * P.H * esize, 256);
  P.b_ghacc = o;
  if (P.dtype != FLCE_F32 && P.n_chunks > 1) o = align_up(o + size_t(P.N) * P.H * 4, 256);
  P.b_ghpart = o;
  if (P.gh_parts > 1) o = align_up(o + size_t(P.gh_parts) * P.N * P.H * 4, 256);
  P.b_gbpart = o;
  o = align_up(o + size_t(P.n_tt) * P.V_pad * 4, 256);
  P.b_bytes = o;
  return FLCE_OK;
}

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Logits block budget of the generic chunked loss: rows per block so that
// rows x V_pad elements stay within it (and within 32-bit offsets).
static constexpr size_t kLogitsBlockBudget = size_t(1) << 30;

static bool valid_dtype(int d) { return d == FLCE_F32 || d == FLCE_BF16 || d == FLCE_F16; }

int make_chunk_plan(const flce_chunked_params* p, ChunkPlan* pl) {
  if (!p || !pl) return FLCE_ERR_INVALID_ARG;
  if (p->n_tokens < 0 || p->hidden <= 0 || p->vocab <= 0 || p->chunk_rows < 0) return FLCE_ERR_INVALID_ARG;
  if (!valid_dtype(p->dtype) || !valid_dtype(p->grad_weight_dtype)) return FLCE_ERR_INVALID_ARG;
  if (p->accum_dtype != FLCE_F32 && p->accum_dtype != p->grad_weight_dtype) return FLCE_ERR_INVALID_ARG;
  if ((p->flags & ~FLCE_ACCUMULATE_GRAD_WEIGHT) != 0) return FLCE_ERR_INVALID_ARG;
  if (p->hidden % 8 != 0 || p->chunk_rows % 256 != 0) return FLCE_ERR_UNSUPPORTED;
  if (p->n_tokens > (int64_t(1) << 30) || p->vocab > (int64_t(1) << 30) || p->hidden > (int64_t(1) << 20))
    return FLCE_ERR_UNSUPPORTED;
  const int esize = p->dtype == FLCE_F32 ? 4 : 2;
  if (p->n_tokens * p->hidden * 4 >= (int64_t(1) << 31)) return FLCE_ERR_UNSUPPORTED;

  ChunkPlan& P = *pl;
  memset(&P, 0, sizeof(P));
  P.N = p->n_tokens;
  P.H = p->hidden;
  P.V = p->vocab;
  P.dtype = p->dtype;
  P.gw_dtype = p->grad_weight_dtype;
  P.esize = esize;
  P.accum_gw = (p->flags & FLCE_ACCUMULATE_GRAD_WEIGHT) != 0;
  P.n_ht = (P.H + 255) / 256;
  P.n_vt = (P.V + 255) / 256;
  P.V_pad = P.n_vt * 256;
  const int64_t row_bytes = P.V_pad * esize;
  int64_t rows = p->chunk_rows;
  if (rows == 0) {
    rows = (int64_t)(kLogitsBlockBudget / (size_t)row_bytes) / 256 * 256;
    const int64_t n_pad = (P.N + 255) / 256 * 256;
    if (rows > n_pad) rows = n_pad;
    if (rows < 256) rows = 256;
  }
  if (rows * row_bytes >= (int64_t(1) << 31)) return FLCE_ERR_UNSUPPORTED;
  P.rows_c = rows;
  P.n_chunks = P.N > 0 ? (int)((P.N + rows - 1) / rows) : 0;
  // vocabulary chunks of the grad_inputs contraction: weight rows x H within 32-bit offsets
  int64_t vc = ((int64_t(1) << 31) - 1) / (P.H * esize) / 256 * 256;
  if (vc < 256) return FLCE_ERR_UNSUPPORTED;
  if (vc > P.V_pad) vc = P.V_pad;
  P.Vc = vc;
  P.n_vchunks = (int)((P.V_pad + vc - 1) / vc);
  P.gw_acc32 = p->accum_dtype == FLCE_F32 && P.gw_dtype != FLCE_F32 && P.n_chunks > 1;

  size_t o = kStatusBytes;
  P.b_L = o;
  o = align_up(o + size_t(rows) * row_bytes, 256);
  P.b_xt = o;
  o = align_up(o + size_t(P.H) * rows * esize, 256);
  P.b_giacc = o;
  if (P.dtype != FLCE_F32 && P.n_vchunks > 1) o = align_up(o + size_t(rows) * P.H * 4, 256);
  P.b_gwacc = o;
  if (P.gw_acc32) o = align_up(o + size_t(P.V) * P.H * 4, 256);
  P.b_ghpart = o;
  {
    // the largest K split any block asks for (blocks differ only in the last one's rows)
    int parts = 1, kt = 0, parts2 = 1;
    plan_gh_split(P.n_ht * (rows / 256), P.Vc, esize, rows, P.H, &parts, &kt);
    const int64_t last = P.N > 0 ? P.N - (int64_t)(P.n_chunks - 1) * rows : 0;
    const int64_t last_tt = (last + 255) / 256;
    plan_gh_split(P.n_ht * last_tt, P.Vc, esize, last, P.H, &parts2, &kt);
    size_t part_bytes = 0;
    if (parts > 1) part_bytes = size_t(parts) * rows * P.H * 4;
    if (parts2 > 1 && size_t(parts2) * last * P.H * 4 > part_bytes) part_bytes = size_t(parts2) * last * P.H * 4;
    o = align_up(o + part_bytes, 256);
  }
  P.b_bytes = o;
  return FLCE_OK;
}

// One-pass forward + backward: blocks of rows whose logits (rows x V_pad in the
// input dtype) fit the logits budget.
int plan_forward_backward(Plan* pl, int64_t block_rows) {
  Plan& P = *pl;
  if (block_rows < 0 || block_rows % 256 != 0) return FLCE_ERR_UNSUPPORTED;
  const int64_t row_bytes = P.V_pad * P.esize;
  int64_t rows = block_rows;
  if (rows == 0) {
    rows = (int64_t)(kLogitsBlockBudget / (size_t)row_bytes) / 256 * 256;
    if (rows > P.N_pad) rows = P.N_pad;
    if (rows < 256) rows = 256;
  }
  if (rows * row_bytes >= (int64_t(1) << 31) || rows * P.H * P.esize >= (int64_t(1) << 31))
    return FLCE_ERR_UNSUPPORTED;
  P.fb_rows = rows;
  P.fb_blocks = P.N > 0 ? (int)((P.N + rows - 1) / rows) : 0;
  int64_t vc = ((int64_t(1) << 31) - 1) / (P.H * P.esize) / 256 * 256;
  if (vc < 256) return FLCE_ERR_UNSUPPORTED;
  if (vc > P.V_pad) vc = P.V_pad;
  P.fb_Vc = vc;
  P.fb_vchunks = (int)((P.V_pad + vc - 1) / vc);
  P.fb_gw_acc32 = P.gw_dtype != FLCE_F32 && P.fb_blocks > 1 && !P.gw_accum_out;
  const int64_t last = P.N > 0 ? P.N - (int64_t)(P.fb_blocks - 1) * rows : 0;
  const int64_t full_tt = rows / 256, last_tt = (last + 255) / 256;

  size_t o = kStatusBytes;
  P.fb_part = o;
  {
    const size_t a = size_t(forward_splits(full_tt, P.n_vt)) * rows;
    const size_t b = size_t(forward_splits(last_tt, P.n_vt)) * last_tt * 256;
    o = align_up(o + 5 * 4 * (a > b ? a : b), 256);
  }
  P.fb_blk = o;
  o = align_up(o + size_t(P.n_tt > 0 ? P.n_tt : 1) * sizeof(BlockPart), 256);
  P.fb_coefA = o;
  o = align_up(o + size_t(P.N_pad) * 4, 256);
  P.fb_coefB = o;
  o = align_up(o + size_t(P.N_pad) * 4, 256);
  P.fb_lseL = o;
  o = align_up(o + size_t(P.N_pad) * 4, 256);
  P.fb_tgt = o;
  o = align_up(o + size_t(P.N_pad) * 4, 256);
  P.fb_Z = o;
  o = align_up(o + size_t(rows) * row_bytes, 256);
  P.fb_xt = o;
  o = align_up(o + size_t(P.H) * rows * P.esize, 256);
  P.fb_ghacc = o;
  if (P.dtype != FLCE_F32 && P.fb_vchunks > 1) o = align_up(o + size_t(rows) * P.H * 4, 256);
  P.fb_gwacc = o;
  if (P.fb_gw_acc32) o = align_up(o + size_t(P.V) * P.H * 4, 256);
  P.fb_ghpart = o;
  {
    int parts = 1, kt = 0, parts2 = 1;
    plan_gh_split(P.n_ht * full_tt, vc, P.esize, rows, P.H, &parts, &kt);
    plan_gh_split(P.n_ht * last_tt, vc, P.esize, last, P.H, &parts2, &kt);
    size_t part_bytes = 0;
    if (parts > 1) part_bytes = size_t(parts) * rows * P.H * 4;
    if (parts2 > 1 && size_t(parts2) * last * P.H * 4 > part_bytes) part_bytes = size_t(parts2) * last * P.H * 4;
    o = align_up(o + part_bytes, 256);
  }
  P.fb_gbpart = o;
  o = align_up(o + size_t(P.N_pad) / 256 * P.V_pad * 4, 256);
  P.fb_bytes = o;
  return FLCE_OK;
}

}  // namespace flce

using namespace flce;

extern "C" {

int flce_version(void) { return 100; }

const char* flce_status_string(int s) {
  switch (s) {
    case FLCE_OK: return "ok";
    case FLCE_ERR_INVALID_ARG: return "invalid argument";
    case FLCE_ERR_UNSUPPORTED: return "unsupported shape, alignment or size";
    case FLCE_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case FLCE_ERR_HIP: return "HIP runtime error";
    case FLCE_ERR_TARGET_OUT_OF_RANGE: return "a target is outside [0, vocab) and not ignore_index";
    case FLCE_ERR_CALLBACK: return "the chunk loss function reported an error";
    default: return "unknown status";
  }
}

int flce_workspace_size(const flce_params* p, int pass, size_t* bytes) {
  if (!bytes) return FLCE_ERR_INVALID_ARG;
  Plan pl;
  const int rc = make_plan(p, &pl);
  if (rc != FLCE_OK) return rc;
  if (pass == FLCE_PASS_FORWARD) *bytes = pl.f_bytes;
  else if (pass == FLCE_PASS_BACKWARD) *bytes = pl.b_bytes;
  else return FLCE_ERR_INVALID_ARG;
  return FLCE_OK;
}

static bool timer_ok(const flce_launch_timer* t) {
  return !t || (t->events && t->kernel && t->capacity >= 0 && t->count >= 0 && t->count <= t->capacity);
}

int flce_forward_timed(const flce_params* p, const void* hidden, const void* weight, const void* bias,
                       const void* targets, float* loss, float* lse, int64_t* num_correct, float* entropy_sum,
                       void* workspace, size_t workspace_bytes, void* stream, flce_launch_timer* timer) {
  Plan pl;
  int rc = make_plan(p, &pl);
  if (rc != FLCE_OK) return rc;
  pl.has_bias = bias != nullptr;
  if (!workspace || !timer_ok(timer)) return FLCE_ERR_INVALID_ARG;
  if (!loss && (pl.reduction != FLCE_REDUCTION_NONE || pl.N > 0)) return FLCE_ERR_INVALID_ARG;
  if (pl.N > 0 && (!hidden || !targets || !lse)) return FLCE_ERR_INVALID_ARG;
  if (!weight) return FLCE_ERR_INVALID_ARG;
  if (!aligned16(hidden) || !aligned16(weight) || !aligned16(bias) || !aligned16(workspace) ||
      !aligned16(targets))
    return FLCE_ERR_UNSUPPORTED;
  if (workspace_bytes < pl.f_bytes) return FLCE_ERR_WORKSPACE_TOO_SMALL;
  pl.timer = timer;
  hipError_t e = launch_forward(pl, hidden, weight, bias, targets, loss, lse, num_correct, entropy_sum,
                                static_cast<char*>(workspace), static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FLCE_OK : FLCE_ERR_HIP;
}

int flce_forward(const flce_params* p, const void* hidden, const void* weight, const void* bias,
                 const void* targets, float* loss, float* lse, int64_t* num_correct,
                 float* entropy_sum, void* workspace, size_t workspace_bytes, void* stream) {
  return flce_forward_timed(p, hidden, weight, bias, targets, loss, lse, num_correct, entropy_sum, workspace,
                            workspace_bytes, stream, nullptr);
}

int flce_backward_timed(const flce_params* p, const void* hidden, const void* weight, const void* bias,
                        const void* targets, const float* lse, const float* grad_loss, void* grad_hidden,
                        void* grad_weight, void* grad_bias, void* workspace, size_t workspace_bytes, void* stream,
                        flce_launch_timer* timer) {
  Plan pl;
  int rc = make_plan(p, &pl);
  if (rc != FLCE_OK) return rc;
  pl.has_bias = bias != nullptr;
  if (!weight || !grad_weight || !workspace || !timer_ok(timer)) return FLCE_ERR_INVALID_ARG;
  if (!grad_loss && (pl.reduction != FLCE_REDUCTION_NONE || pl.N > 0)) return FLCE_ERR_INVALID_ARG;
  if (pl.N > 0 && (!hidden || !targets || !lse || !grad_hidden)) return FLCE_ERR_INVALID_ARG;
  if (grad_bias && !bias) return FLCE_ERR_INVALID_ARG;
  if (!aligned16(hidden) || !aligned16(weight) || !aligned16(bias) || !aligned16(workspace) ||
      !aligned16(targets) || !aligned16(grad_hidden) || !aligned16(grad_weight) || !aligned16(grad_bias))
    return FLCE_ERR_UNSUPPORTED;
  if (workspace_bytes < pl.b_bytes) return FLCE_ERR_WORKSPACE_TOO_SMALL;
  pl.timer = timer;
  hipError_t e = launch_backward(pl, hidden, weight, bias, targets, lse, grad_loss, grad_hidden,
                                 grad_weight, grad_bias, static_cast<char*>(workspace),
                                 static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FLCE_OK : FLCE_ERR_HIP;
}

int flce_backward(const flce_params* p, const void* hidden, const void* weight, const void* bias,
                  const void* targets, const float* lse, const float* grad_loss, void* grad_hidden,
                  void* grad_weight, void* grad_bias, void* workspace, size_t workspace_bytes,
                  void* stream) {
  return flce_backward_timed(p, hidden, weight, bias, targets, lse, grad_loss, grad_hidden, grad_weight, grad_bias,
                             workspace, workspace_bytes, stream, nullptr);
}

int flce_forward_backward_workspace_size(const flce_params* p, int64_t block_rows, size_t* bytes) {
  if (!bytes) return FLCE_ERR_INVALID_ARG;
  Plan pl;
  int rc = make_plan(p, &pl);
  if (rc != FLCE_OK) return rc;
  rc = plan_forward_backward(&pl, block_rows);
  if (rc != FLCE_OK) return rc;
  *bytes = pl.fb_bytes;
  return FLCE_OK;
}

int flce_forward_backward(const flce_params* p, int64_t block_rows, const void* hidden, const void* weight,
                          const void* bias, const void* targets, const float* grad_loss, float* loss, float* lse,
                          int64_t* num_correct, float* entropy_sum, void* grad_hidden, void* grad_weight,
                          void* grad_bias, void* workspace, size_t workspace_bytes, void* stream) {
  Plan pl;
  int rc = make_plan(p, &pl);
  if (rc != FLCE_OK) return rc;
  rc = plan_forward_backward(&pl, block_rows);
  if (rc != FLCE_OK) return rc;
  pl.has_bias = bias != nullptr;
  if (!weight || !grad_weight || !workspace) return FLCE_ERR_INVALID_ARG;
  if (!loss && (pl.reduction != FLCE_REDUCTION_NONE || pl.N > 0)) return FLCE_ERR_INVALID_ARG;
  if (!grad_loss && (pl.reduction != FLCE_REDUCTION_NONE || pl.N > 0)) return FLCE_ERR_INVALID_ARG;
  if (pl.N > 0 && (!hidden || !targets || !lse || !grad_hidden)) return FLCE_ERR_INVALID_ARG;
  if (grad_bias && !bias) return FLCE_ERR_INVALID_ARG;
  if (!aligned16(hidden) || !aligned16(weight) || !aligned16(bias) || !aligned16(workspace) ||
      !aligned16(targets) || !aligned16(grad_hidden) || !aligned16(grad_weight) || !aligned16(grad_bias))
    return FLCE_ERR_UNSUPPORTED;
  if (workspace_bytes < pl.fb_bytes) return FLCE_ERR_WORKSPACE_TOO_SMALL;
  hipError_t e = launch_forward_backward(pl, hidden, weight, bias, targets, grad_loss, loss, lse, num_correct,
                                         entropy_sum, grad_hidden, grad_weight, grad_bias,
                                         static_cast<char*>(workspace), static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FLCE_OK : FLCE_ERR_HIP;
}

int flce_scale_gradients(const flce_params* p, const float* g, void* grad_hidden, void* grad_weight,
                         void* grad_bias, void* stream) {
  Plan pl;
  const int rc = make_plan(p, &pl);
  if (rc != FLCE_OK) return rc;
  if (pl.reduction == FLCE_REDUCTION_NONE || !g || !grad_weight) return FLCE_ERR_INVALID_ARG;
  if (pl.N > 0 && !grad_hidden) return FLCE_ERR_INVALID_ARG;
  if (!aligned16(grad_hidden) || !aligned16(grad_weight) || !aligned16(grad_bias)) return FLCE_ERR_UNSUPPORTED;
  const hipError_t e = launch_scale_gradients(pl, g, grad_hidden, grad_weight, grad_bias,
                                              static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FLCE_OK : FLCE_ERR_HIP;
}

int flce_chunked_workspace_size(const flce_chunked_params* p, size_t* bytes) {
  if (!bytes) return FLCE_ERR_INVALID_ARG;
  ChunkPlan pl;
  const int rc = make_chunk_plan(p, &pl);
  if (rc != FLCE_OK) return rc;
  *bytes = pl.b_bytes;
  return FLCE_OK;
}

int flce_chunked_linear_loss(const flce_chunked_params* p, const void* inputs, const void* weight,
                             flce_chunk_loss_fn fn, void* user, float* loss, void* grad_inputs,
                             void* grad_weight, void* workspace, size_t workspace_bytes, void* stream) {
  ChunkPlan pl;
  const int rc = make_chunk_plan(p, &pl);
  if (rc != FLCE_OK) return rc;
  if (!fn || !loss || !weight || !grad_weight || !workspace) return FLCE_ERR_INVALID_ARG;
  if (pl.N > 0 && (!inputs || !grad_inputs)) return FLCE_ERR_INVALID_ARG;
  if (!aligned16(inputs) || !aligned16(weight) || !aligned16(grad_inputs) || !aligned16(grad_weight) ||
      !aligned16(workspace))
    return FLCE_ERR_UNSUPPORTED;
  if (workspace_bytes < pl.b_bytes) return FLCE_ERR_WORKSPACE_TOO_SMALL;
  return launch_chunked(pl, inputs, weight, fn, user, loss, grad_inputs, grad_weight,
                        static_cast<char*>(workspace), static_cast<hipStream_t>(stream));
}

int flce_weighted_mse_chunk(void* user, int64_t row0, int64_t rows, int64_t vocab, void* logits, int64_t ld,
                            int32_t dtype, float* loss, void* stream) {
  const flce_wmse_args* a = static_cast<const flce_wmse_args*>(user);
  if (!a || !a->target || !a->row_weight || !a->feature_weight || !a->row_loss || !logits || !loss)
    return FLCE_ERR_INVALID_ARG;
  if (!valid_dtype(dtype) || row0 < 0 || rows < 0 || vocab <= 0 || ld < vocab || a->ld_target < vocab)
    return FLCE_ERR_INVALID_ARG;
  const uintptr_t fa = reinterpret_cast<uintptr_t>(a->target) | reinterpret_cast<uintptr_t>(a->row_weight) |
                       reinterpret_cast<uintptr_t>(a->feature_weight) | reinterpret_cast<uintptr_t>(a->row_loss);
  if ((fa & 3) != 0 || ld % 4 != 0 || !aligned16(logits) || rows > (int64_t(1) << 30) ||
      vocab > (int64_t(1) << 30))
    return FLCE_ERR_UNSUPPORTED;
  if (rows == 0) return FLCE_OK;
  return launch_wmse(*a, row0, (int)rows, (int)vocab, logits, (int)ld, dtype, loss, static_cast<hipStream_t>(stream));
}

int flce_get_status(const void* workspace, void* stream) {
  if (!workspace) return FLCE_ERR_INVALID_ARG;
  if (hipStreamSynchronize(static_cast<hipStream_t>(stream)) != hipSuccess) return FLCE_ERR_HIP;
  int v = 0;
  if (hipMemcpy(&v, workspace, sizeof(int), hipMemcpyDeviceToHost) != hipSuccess) return FLCE_ERR_HIP;
  return v;
}

}  // extern "C"
