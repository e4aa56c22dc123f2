// lmtopk_api.cpp - the C ABI of liblmtopk: argument checks, chunk geometry,
// merge plan, and dispatch to the HIP launchers.  Plain host C++: every check
// here runs before anything is enqueued (the only HIP calls before that query
// the device's LDS limit), so an invalid call launches nothing and writes
// nothing.

#include <stdint.h>
#include <string.h>

#include "lmtopk.h"
#include "lmtopk_internal.hpp"

namespace lmtopk {
namespace {

constexpr int64_t kMaxV = INT32_MAX;  // indices are carried as int32 inside the library

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int check_options(const lmtopk_options* opt) {
  if (!opt) return LMTOPK_OK;
  if (opt->reserved != 0) return LMTOPK_ERR_OPTIONS;
  const int c = opt->chunk_rows;
  if (c == 0) return LMTOPK_OK;
  if (c == 2048) return LMTOPK_OK;
  if (c >= 64 && c <= 1024 && c % 64 == 0) return LMTOPK_OK;
  return LMTOPK_ERR_OPTIONS;
}

int check_mvk(int64_t M, int64_t V, int32_t k) {
  if (M < 1 || M > LMTOPK_MAX_ROWS) return LMTOPK_ERR_SHAPE;
  if (V < 1 || V > kMaxV) return LMTOPK_ERR_SHAPE;
  if (k < 1 || k > LMTOPK_MAX_K || (int64_t)k > V) return LMTOPK_ERR_K;
  return LMTOPK_OK;
}

lmtopk_status hip_status(int e) { return e == 0 ? LMTOPK_OK : LMTOPK_ERR_HIP; }

}  // namespace

int make_geometry(int64_t M, int64_t V, int32_t k, int32_t chunk_rows_opt, int split_ok,
                  Geometry* g) {
  int st = check_mvk(M, V, k);
  if (st) return st;
  memset(g, 0, sizeof(*g));
  g->M = M;
  g->V = V;
  g->k = k;
  g->n_tiles = (V + 63) / 64;
  int C = chunk_rows_opt;
  if (C == 0) {
    // one 1024-row chunk per workgroup; small vocabularies use one chunk.
    // Up to 128 such chunks leave at least half of the 256 CUs idle: with
    // two waves per tile a 512-row chunk still has 16 waves, so twice the
    // workgroups stream the head (if the fused merge still holds their
    // candidates).
    C = V >= 1024 ? 1024 : (int)(g->n_tiles * 64);
    const int64_t n512 = (V + 511) / 512;
    if (split_ok && V >= 1024 && (V + 1023) / 1024 <= 128 && k <= kFusedMaxK &&
        n512 * (k < 512 ? k : 512) <= 1024 * kFusedSlots)
      C = 512;
  }
  g->chunk_rows = C;
  // rows per lane: 1 for chunks of up to 1024 rows (up to 16 waves); a
  // 2048-row chunk is 8 waves of 4 rows per lane.  Chunks of up to 512 rows
  // take two waves per tile where the caller can.
  g->rpl = C <= 1024 ? 1 : 4;
  g->ks = split_ok && C <= 512 ? 2 : 1;
  g->nw = g->ks * C / (64 * g->rpl);
  g->n_chunks = (int)((V + C - 1) / C);
  g->kc = k < C ? k : C;
  const int64_t n0 = (int64_t)g->n_chunks * g->kc;
  g->sync_bytes = kCounterBytes + kHistBytes;
  static_assert(LMTOPK_MAX_ROWS * kHistBins * 4 == kHistBytes, "one histogram per row");
  g->heads_bytes = round_up((size_t)(M * g->n_chunks * 4 * 8), 256);
  g->region0_bytes = round_up((size_t)(M * n0 * 8), 256);

  // merge plan: a level either fits one workgroup (final) or splits the
  // candidates into segments of kSegMax and keeps k per segment
  int64_t n = n0;
  int lv = 0;
  while (true) {
    if (lv >= kMaxMergeLevels) return LMTOPK_ERR_SHAPE;
    MergeLevel& L = g->level[lv];
    L.n_in = n;
    if (n <= kSegMax) {
      static const int rms[] = {1, 2, 4, 8, 12, 16};
      int rm = 16;
      for (int r : rms) {
        if (n <= (int64_t)1024 * r) {
          rm = r;
          break;
        }
      }
      L.rm = rm;
      L.nw = (int)((n + 64 * rm - 1) / (64 * rm));
      L.n_seg = 1;
      ++lv;
      break;
    }
    L.rm = 16;
    L.nw = 16;
    L.n_seg = (int)((n + kSegMax - 1) / kSegMax);
    n = (int64_t)L.n_seg * k;
    if (lv == 0) g->region1_bytes = round_up((size_t)(M * n * 8), 256);
    ++lv;
  }
  g->n_levels = lv;
  // one merge level whose candidates fit the chunk workgroup, and k up to
  // kFusedMaxK: its last workgroup merges instead of a second launch
  const int64_t chunk_threads = (int64_t)64 * g->nw;
  if (lv == 1 && n0 <= chunk_threads * kFusedSlots && k <= kFusedMaxK) {
    g->fused = 1;
    g->n_levels = 0;
  }
  g->lse_bytes = round_up((size_t)(M * g->n_chunks * 8), 256);
  g->counts_bytes = g->n_levels == 2 && g->level[0].n_seg <= kGatherSegs
                        ? round_up((size_t)(M * g->level[0].n_seg * 4), 256)
                        : 0;
  g->workspace_bytes = g->sync_bytes + g->heads_bytes + g->region0_bytes + g->region1_bytes +
                       g->lse_bytes + g->counts_bytes;
  return LMTOPK_OK;
}

}  // namespace lmtopk

using lmtopk::Geometry;

extern "C" {

int32_t lmtopk_layout_version(void) { return LMTOPK_LAYOUT_VERSION; }

const char* lmtopk_status_string(lmtopk_status s) {
  switch (s) {
    case LMTOPK_OK: return "ok";
    case LMTOPK_ERR_NULL: return "a required pointer is NULL";
    case LMTOPK_ERR_SHAPE: return "invalid shape (M, V, H, ld or a size limit)";
    case LMTOPK_ERR_K: return "k must satisfy 1 <= k <= min(V, 2048)";
    case LMTOPK_ERR_GROUP: return "group_size must be 128 and H a multiple of 128";
    case LMTOPK_ERR_DTYPE: return "unknown dtype";
    case LMTOPK_ERR_ALIGN: return "pointer or row not 16-byte aligned";
    case LMTOPK_ERR_WORKSPACE: return "workspace missing or too small";
    case LMTOPK_ERR_OPTIONS: return "invalid lmtopk_options";
    case LMTOPK_ERR_HIP: return "the HIP runtime refused a launch";
  }
  return "unknown status";
}

lmtopk_status lmtopk_packed_bytes(int64_t V, int64_t H, int32_t group_size, size_t* wq_bytes,
                                  size_t* wscale_bytes) {
  if (!wq_bytes || !wscale_bytes) return LMTOPK_ERR_NULL;
  if (V < 1 || V > INT32_MAX || H < 1) return LMTOPK_ERR_SHAPE;
  if (group_size != LMTOPK_GROUP_SIZE || H % LMTOPK_GROUP_SIZE != 0) return LMTOPK_ERR_GROUP;
  const int64_t V64 = (V + 63) / 64 * 64;
  const int64_t G = H / LMTOPK_GROUP_SIZE;
  const int64_t G4 = (G + 3) / 4 * 4;
  *wq_bytes = (size_t)(V64 * H / 8);
  *wscale_bytes = (size_t)(V64 * G4 * 4);
  return LMTOPK_OK;
}

lmtopk_status lmtopk_workspace_bytes(int64_t M, int64_t V, int32_t k, const lmtopk_options* opt,
                                     size_t* bytes) {
  if (!bytes) return LMTOPK_ERR_NULL;
  int st = lmtopk::check_options(opt);
  if (st) return (lmtopk_status)st;
  // every path's plan: with and without two waves per tile
  size_t need = 0;
  for (int split_ok = 0; split_ok < 2; ++split_ok) {
    Geometry g;
    st = lmtopk::make_geometry(M, V, k, opt ? opt->chunk_rows : 0, split_ok, &g);
    if (st) return (lmtopk_status)st;
    if (g.workspace_bytes > need) need = g.workspace_bytes;
  }
  *bytes = need;
  return LMTOPK_OK;
}

lmtopk_status lmtopk_workspace_init(void* workspace, size_t bytes, void* stream) {
  if (!workspace) return LMTOPK_ERR_NULL;
  if (!lmtopk::aligned16(workspace)) return LMTOPK_ERR_ALIGN;
  if (bytes == 0) return LMTOPK_OK;
  return lmtopk::hip_status(lmtopk::launch_zero(workspace, bytes, stream));
}

lmtopk_status lmtopk_pack_binary(const void* w, lmtopk_dtype w_dtype, int64_t V, int64_t H,
                                 int32_t group_size, void* wq, float* wscale, void* stream) {
  if (!w || !wq || !wscale) return LMTOPK_ERR_NULL;
  if (V < 1 || V > INT32_MAX || H < 1) return LMTOPK_ERR_SHAPE;
  if (group_size != LMTOPK_GROUP_SIZE || H % LMTOPK_GROUP_SIZE != 0) return LMTOPK_ERR_GROUP;
  if (w_dtype != LMTOPK_F32 && w_dtype != LMTOPK_BF16) return LMTOPK_ERR_DTYPE;
  if (!lmtopk::aligned16(w) || !lmtopk::aligned16(wq) || !lmtopk::aligned16(wscale))
    return LMTOPK_ERR_ALIGN;
  return lmtopk::hip_status(
      lmtopk::launch_pack(w, w_dtype == LMTOPK_BF16, V, H, wq, wscale, stream));
}

// The call's token draw (lmtopk_sampling) into g->smp; OPTIONS for a scalar
// top_k above k, NULL / ALIGN for the arrays.
static lmtopk_status sampling_checks(const lmtopk_sampling* sp, int32_t k, Geometry* g) {
  memset(&g->smp, 0, sizeof(g->smp));
  if (!sp) return LMTOPK_OK;
  if (!sp->tokens) return LMTOPK_ERR_NULL;
  if (sp->top_k > k) return LMTOPK_ERR_OPTIONS;
  const void* arrays[] = {sp->tokens, sp->kept, sp->temperature_rows, sp->top_k_rows,
                          sp->top_p_rows, sp->min_p_rows, sp->offset_device};
  for (const void* p : arrays)
    if (p && !lmtopk::aligned16(p)) return LMTOPK_ERR_ALIGN;
  lmtopk::SampleParams& s = g->smp;
  s.on = 1;
  s.need_norm = (sp->top_p_rows != nullptr || sp->top_p < 1.f) ? 1 : 0;
  s.temperature = sp->temperature;
  s.top_k = sp->top_k;
  s.top_p = sp->top_p;
  s.min_p = sp->min_p;
  s.temperature_rows = sp->temperature_rows;
  s.top_k_rows = sp->top_k_rows;
  s.top_p_rows = sp->top_p_rows;
  s.min_p_rows = sp->min_p_rows;
  s.seed = sp->seed;
  s.offset = sp->offset;
  s.offset_device = sp->offset_device;
  s.tokens = sp->tokens;
  s.kept = sp->kept;
  return LMTOPK_OK;
}

static lmtopk_status common_checks(const void* workspace, size_t workspace_bytes, float* values,
                                   int64_t* indices, const lmtopk_options* opt, int64_t M,
                                   int64_t V, int32_t k, int split_ok, Geometry* g) {
  if (!values || !indices) return LMTOPK_ERR_NULL;
  int st = lmtopk::check_options(opt);
  if (st) return (lmtopk_status)st;
  st = lmtopk::make_geometry(M, V, k, opt ? opt->chunk_rows : 0, split_ok, g);
  if (st) return (lmtopk_status)st;
  if (!lmtopk::aligned16(values) || !lmtopk::aligned16(indices)) return LMTOPK_ERR_ALIGN;
  g->lse = opt ? opt->lse : nullptr;
  if (g->lse && !lmtopk::aligned16(g->lse)) return LMTOPK_ERR_ALIGN;
  g->allowed = opt ? opt->allowed : nullptr;
  if (g->allowed && !lmtopk::aligned16(g->allowed)) return LMTOPK_ERR_ALIGN;
  st = sampling_checks(opt ? opt->sampling : nullptr, k, g);
  if (st) return (lmtopk_status)st;
  if (!workspace || workspace_bytes < g->workspace_bytes) return LMTOPK_ERR_WORKSPACE;
  if (!lmtopk::aligned16(workspace)) return LMTOPK_ERR_ALIGN;
  return LMTOPK_OK;
}

static lmtopk_status finish(const Geometry& g, int e, void* workspace, float* values,
                            int64_t* indices, void* stream) {
  if (e) return LMTOPK_ERR_HIP;
  return lmtopk::hip_status(lmtopk::launch_merges(g, workspace, values, indices, stream));
}

static void* const* score_events(const lmtopk_options* opt) {
  return opt ? static_cast<void* const*>(opt->score_events) : nullptr;
}

// Two waves per tile for the binary path where their exchange area fits
// gfx950's LDS (M and H are checked elsewhere; any value here is safe).
static int binary_split_ok(int64_t M, int64_t H) {
  return H >= 1 && M >= 1 && M <= LMTOPK_MAX_ROWS && H <= LMTOPK_MAX_BINARY_MH &&
         lmtopk::binary_lds_bytes(M, H, 2, 1) + lmtopk::kChunkStaticLds <= lmtopk::kLdsPerBlock;
}

lmtopk_status lmtopk_binary_plan(int64_t M, int64_t V, int64_t H, int32_t k,
                                 const lmtopk_options* opt, int32_t* chunk_rows,
                                 int32_t* n_chunks, int32_t* waves) {
  if (!chunk_rows || !n_chunks || !waves) return LMTOPK_ERR_NULL;
  int st = lmtopk::check_options(opt);
  if (st) return (lmtopk_status)st;
  if (H < 1) return LMTOPK_ERR_SHAPE;
  if (H % LMTOPK_GROUP_SIZE != 0) return LMTOPK_ERR_GROUP;
  Geometry g;
  st = lmtopk::make_geometry(M, V, k, opt ? opt->chunk_rows : 0, binary_split_ok(M, H), &g);
  if (st) return (lmtopk_status)st;
  *chunk_rows = g.chunk_rows;
  *n_chunks = g.n_chunks;
  *waves = g.nw;
  return LMTOPK_OK;
}

// The binary call in two phases: every argument check (the workspace only
// as a size and an alignment), then the launches.  lmtopk_binary and
// lmtopk_binary_noalloc share both.
static lmtopk_status binary_checks(const int8_t* act_q, const float* act_scale, const void* wq,
                                   const float* wscale, const float* bias, int64_t M, int64_t V,
                                   int64_t H, int32_t group_size, int32_t k, float* values,
                                   int64_t* indices, const void* workspace,
                                   size_t workspace_bytes, const lmtopk_options* opt, Geometry* g) {
  if (!act_q || !act_scale || !wq || !wscale) return LMTOPK_ERR_NULL;
  lmtopk_status st = common_checks(workspace, workspace_bytes, values, indices, opt, M, V, k,
                                   binary_split_ok(M, H), g);
  if (st) return st;
  if (H < 1) return LMTOPK_ERR_SHAPE;
  if (group_size != LMTOPK_GROUP_SIZE || H % LMTOPK_GROUP_SIZE != 0) return LMTOPK_ERR_GROUP;
  if (M * H > LMTOPK_MAX_BINARY_MH) return LMTOPK_ERR_SHAPE;
  if (g->rpl > 1 && M > lmtopk::kMaxRowsWide) return LMTOPK_ERR_OPTIONS;
  if (!lmtopk::aligned16(act_q) || !lmtopk::aligned16(act_scale) || !lmtopk::aligned16(wq) ||
      !lmtopk::aligned16(wscale) || (bias && !lmtopk::aligned16(bias)))
    return LMTOPK_ERR_ALIGN;
  size_t lds_max = 0;
  if (lmtopk::max_lds_per_block(&lds_max)) return LMTOPK_ERR_HIP;
  if (lmtopk::binary_lds_bytes(M, H, g->ks, g->rpl) + lmtopk::kChunkStaticLds > lds_max)
    return LMTOPK_ERR_SHAPE;
  return LMTOPK_OK;
}

static lmtopk_status binary_launch(const Geometry& g, const int8_t* act_q, const float* act_scale,
                                   const void* wq, const float* wscale, const float* bias, int64_t H,
                                   float* values, int64_t* indices, void* workspace,
                                   const lmtopk_options* opt, void* stream) {
  const int e =
      lmtopk::launch_binary_chunks(g, act_q, act_scale, wq, wscale, bias, H, workspace, values,
                                   indices, stream, score_events(opt));
  return finish(g, e, workspace, values, indices, stream);
}

lmtopk_status lmtopk_binary(const int8_t* act_q, const float* act_scale, const void* wq,
                            const float* wscale, const float* bias, int64_t M, int64_t V,
                            int64_t H, int32_t group_size, int32_t k, float* values,
                            int64_t* indices, void* workspace, size_t workspace_bytes,
                            const lmtopk_options* opt, void* stream) {
  Geometry g;
  const lmtopk_status st = binary_checks(act_q, act_scale, wq, wscale, bias, M, V, H, group_size,
                                         k, values, indices, workspace, workspace_bytes, opt, &g);
  if (st) return st;
  return binary_launch(g, act_q, act_scale, wq, wscale, bias, H, values, indices, workspace, opt,
                       stream);
}

lmtopk_status lmtopk_binary_noalloc(const int8_t* act_q, const float* act_scale, const void* wq,
                                    const float* wscale, const float* bias, int64_t M, int64_t V,
                                    int64_t H, int32_t group_size, int32_t k, float* values,
                                    int64_t* indices, const lmtopk_options* opt, void* stream) {
  Geometry g;
  // the scratch array stands in for the workspace: checked as one of
  // LMTOPK_NOALLOC_SCRATCH_BYTES bytes at a 256-byte aligned address
  const lmtopk_status st =
      binary_checks(act_q, act_scale, wq, wscale, bias, M, V, H, group_size, k, values, indices,
                    reinterpret_cast<const void*>(static_cast<uintptr_t>(256)),
                    (size_t)LMTOPK_NOALLOC_SCRATCH_BYTES, opt, &g);
  if (st) return st;
  void* scratch = nullptr;
  if (lmtopk::noalloc_scratch(&scratch, stream)) return LMTOPK_ERR_HIP;
  return binary_launch(g, act_q, act_scale, wq, wscale, bias, H, values, indices, scratch, opt,
                       stream);
}

lmtopk_status lmtopk_dense(const void* hidden, const void* weight, lmtopk_dtype dtype,
                           const float* bias, int64_t M, int64_t V, int64_t H, int32_t k,
                           float* values, int64_t* indices, void* workspace,
                           size_t workspace_bytes, const lmtopk_options* opt, void* stream) {
  if (!hidden || !weight) return LMTOPK_ERR_NULL;
  Geometry g;
  lmtopk_status st =
      common_checks(workspace, workspace_bytes, values, indices, opt, M, V, k, 0, &g);
  if (st) return st;
  if (H < 1) return LMTOPK_ERR_SHAPE;
  if (dtype != LMTOPK_F32 && dtype != LMTOPK_BF16) return LMTOPK_ERR_DTYPE;
  const int64_t esz = dtype == LMTOPK_BF16 ? 2 : 4;
  if ((H * esz) % 16 != 0) return LMTOPK_ERR_ALIGN;
  if (!lmtopk::aligned16(hidden) || !lmtopk::aligned16(weight) || (bias && !lmtopk::aligned16(bias)))
    return LMTOPK_ERR_ALIGN;
  size_t lds_max = 0;
  if (lmtopk::max_lds_per_block(&lds_max)) return LMTOPK_ERR_HIP;
  if (lmtopk::dense_lds_bytes(M, g.chunk_rows) + lmtopk::kChunkStaticLds > lds_max)
    return LMTOPK_ERR_SHAPE;
  const int e = lmtopk::launch_dense_chunks(g, hidden, weight, dtype == LMTOPK_BF16, bias, H,
                                            workspace, values, indices, stream, score_events(opt));
  return finish(g, e, workspace, values, indices, stream);
}

lmtopk_status lmtopk_select(const float* logits, int64_t M, int64_t V, int64_t ld, int32_t k,
                            float* values, int64_t* indices, void* workspace,
                            size_t workspace_bytes, const lmtopk_options* opt, void* stream) {
  if (!logits) return LMTOPK_ERR_NULL;
  Geometry g;
  lmtopk_status st =
      common_checks(workspace, workspace_bytes, values, indices, opt, M, V, k, 0, &g);
  if (st) return st;
  if (ld < V) return LMTOPK_ERR_SHAPE;
  if (!lmtopk::aligned16(logits)) return LMTOPK_ERR_ALIGN;
  const int e = lmtopk::launch_select_chunks(g, logits, ld, workspace, values, indices, stream,
                                             score_events(opt));
  return finish(g, e, workspace, values, indices, stream);
}

}  // extern "C"
