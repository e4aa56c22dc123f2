// lmtopk_internal.hpp - interface between the C ABI (host validation and
// geometry, plain C++) and the HIP translation unit (kernels and launchers).
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace lmtopk {

constexpr int kMaxMergeLevels = 8;
constexpr int64_t kSegMax = 16384;  // candidates one merge workgroup can hold (1024 x 16)
constexpr int64_t kFusedSlots = 16; // candidate slots per thread of the fused final merge
// Largest k the chunk launch merges itself: its last workgroup orders the
// result by rank counting, which is quadratic in k; larger k go to a merge
// launch, which sorts them (a radix sort kept out of the chunk kernels,
// whose tail code it would lengthen).
constexpr int kFusedMaxK = 256;
// The workspace starts with the fused merge's completion counter, then one
// key histogram per row (kHistBins counts of the top 11 bits of the
// order-preserving key), at offsets that do not depend on the call, so that
// both stay zero between calls whatever calls share the workspace.  A merge
// with intermediate levels counts the candidates' keys there first; its
// first level then keeps only keys in or above the bin of the k-th largest,
// and its last level sets the row's counts back to zero.
constexpr size_t kCounterBytes = 256;
constexpr int kHistBins = 2048;
constexpr size_t kHistBytes = (size_t)8 * kHistBins * 4;  // LMTOPK_MAX_ROWS rows
// With two merge levels of at most kGatherSegs segments, the first level
// writes only its selected candidates and their count per segment, and the
// last gathers them.
constexpr int kGatherSegs = 64;

struct MergeLevel {
  int64_t n_in;  // candidates per row read by this level
  int n_seg;     // segments per row (workgroups per row); 1 = final level
  int rm;        // candidate slots per thread
  int nw;        // waves per workgroup
};

// The call's token draw (lmtopk_sampling), as the kernels read it.  on == 0:
// no draw.  need_norm: the chunk kernels form the normaliser partials of the
// scaled logits (top-p needs lse_T).
struct SampleParams {
  int on;
  int need_norm;
  float temperature;
  int top_k;
  float top_p;
  float min_p;
  const float* temperature_rows;
  const int32_t* top_k_rows;
  const float* top_p_rows;
  const float* min_p_rows;
  uint64_t seed;
  uint64_t offset;
  const uint64_t* offset_device;
  int64_t* tokens;
  int32_t* kept;
};

// Chunking and merge plan of one call; identical for every path given
// (M, V, k, chunk_rows).
struct Geometry {
  int64_t M, V;
  int k;
  int chunk_rows;  // C: vocabulary rows per chunk (workgroup)
  int rpl;         // rows per lane
  int ks;          // waves per 64-row tile: 1, or 2 (binary path: each wave
                   // scores half of the groups); C * ks = 64 * nw * rpl
  int nw;          // waves per chunk workgroup
  int n_chunks;
  int kc;          // candidate slots per chunk per row = min(k, C)
  int64_t n_tiles; // 64-row tiles covering V
  int n_levels;    // merge kernel launches (0 when fused)
  int fused;       // the chunk launch's last workgroup does the final merge
  MergeLevel level[kMaxMergeLevels];
  size_t sync_bytes;     // completion counter and key histograms (zero between calls)
  size_t heads_bytes;    // best candidates of each chunk [M][n_chunks][4] x 8 B
  size_t region0_bytes;  // chunk candidates [M][n_chunks * kc] x 8 B
  size_t region1_bytes;  // first intermediate merge output, or 0
  size_t lse_bytes;      // log-sum-exp pairs [M][n_chunks] x (max, sum)
  size_t counts_bytes;   // two merge levels: the first level's output count
                         // per row and segment [M][n_seg] x 4 B, or 0
  size_t workspace_bytes;
  float* lse;            // this call's log-sum-exp output [M], or null (not part of the plan)
  const int32_t* allowed;  // this call's bitmask [M][ceil(V/32)], or null (not part of the plan)
  SampleParams smp;        // this call's draw (not part of the plan)
};

// Returns 0 or an lmtopk_status code (SHAPE, K, OPTIONS).  split_ok: the
// caller's chunk kernel can score a tile with two waves (the binary path,
// when its LDS allows); the automatic chunk size and the waves per chunk
// then take it into account.
int make_geometry(int64_t M, int64_t V, int32_t k, int32_t chunk_rows_opt, int split_ok,
                  Geometry* g);

// Launchers; each returns a hipError_t value (0 = success).  `events` of the
// chunk launchers: null, or two hipEvent_t recording the kernel's start and end.
int launch_pack(const void* w, int w_is_bf16, int64_t V, int64_t H, void* wq, float* wscale,
                void* stream);
int launch_binary_chunks(const Geometry& g, const int8_t* act_q, const float* act_scale,
                         const void* wq, const float* wscale, const float* bias, int64_t H,
                         void* workspace, float* values, int64_t* indices, void* stream,
                         void* const* events);
int launch_dense_chunks(const Geometry& g, const void* hidden, const void* weight, int is_bf16,
                        const float* bias, int64_t H, void* workspace, float* values,
                        int64_t* indices, void* stream, void* const* events);
int launch_select_chunks(const Geometry& g, const float* logits, int64_t ld, void* workspace,
                         float* values, int64_t* indices, void* stream, void* const* events);
int launch_merges(const Geometry& g, void* workspace, float* values, int64_t* indices,
                  void* stream);
// Zero fill of n bytes (n % 16 == 0 handled by the caller's rounding rules:
// any n; p 16-byte aligned).
int launch_zero(void* p, size_t n, void* stream);
// The binary path's 2048-row chunks (four rows per lane) serve at most this
// many activation rows.
constexpr int kMaxRowsWide = 2;

// The device address of the current device's scratch array (the workspace of
// lmtopk_binary_noalloc, LMTOPK_NOALLOC_SCRATCH_BYTES bytes), found on its
// first use on that device, when its completion counter is also cleared by a
// kernel on `stream`.  Returns a hipError_t value.
int noalloc_scratch(void** ptr, void* stream);

// Largest LDS (bytes) one workgroup may use on the current device.
int max_lds_per_block(size_t* bytes);

// Upper bound of the static LDS of the chunk kernels (selection histograms
// and the head staging); the dynamic LDS comes on top.
constexpr size_t kChunkStaticLds = 57344;

// LDS per workgroup of gfx950 (the split decision is made from it, so that
// it does not need a device; the launch checks the device's own limit).
constexpr size_t kLdsPerBlock = 163840;

// LDS bytes the scoring kernels need; ks = waves per tile, rpl: rows per lane.
size_t binary_lds_bytes(int64_t M, int64_t H, int ks, int rpl);
size_t dense_lds_bytes(int64_t M, int chunk_rows);

}  // namespace lmtopk
