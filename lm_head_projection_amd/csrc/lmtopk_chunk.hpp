// lmtopk_chunk.hpp - pieces shared by the chunk kernels (binary, dense and
// selection-only): the candidate output of a chunk, its exact per-chunk
// top-k (lm-head-topk page, section "Method": every chunk offers k
// candidates), streaming loads, and the launch helper.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

#include "lmtopk_device.hpp"
#include "lmtopk_internal.hpp"
#include "lmtopk_sample.hpp"

namespace lmtopk {

// LDS of a chunk kernel: the chunk selection's staging, and, after it, the
// final merge of the fused path.
union ChunkSmem {
  HeadStage hs;
  FinalSmem fs;
};

// What the fused final merge needs: the launch's candidate lists and heads,
// the outputs, and a workspace counter that is zero between calls.
struct FusedMerge {
  uint32_t* counter;
  const uint2* cand;   // [M][n_chunks][kc]
  const uint2* heads;  // [M][n_chunks][kHeads]
  float* values;       // [M][k]
  int64_t* indices;    // [M][k]
  int M;
  int n_chunks;
  int kc;
  int k;
  const uint2* lse_part;  // [M][n_chunks] log-sum-exp pairs, or null
  float* lse;             // [M] or null
  SampleParams smp;       // the token draw (smp.on == 0: none)
};

// Fused second pass (lm-head-topk page, section "Method": the chunk
// candidates are merged into the final top-k).  Called by every workgroup
// of a chunk launch (one workgroup per chunk) after it has stored its
// candidates and heads with st_cand.  Each workgroup waits until those
// stores are complete at device scope, then counts itself done on the
// counter; the workgroup that counts last sees every chunk's candidates and
// merges all M rows, then sets the counter back to zero for the next call.
// n_chunks * kc <= blockDim.x * RM.  With a token draw, each row's token is
// drawn right after its merge (sample_row).
// kExtras false: the launch has no log-sum-exp output or bitmask; kSample
// false: no draw; that code is left out.
// kRows (compile-time rows, 2 or more, and no draw): the rows' bounded
// merges run side by side, each by its own group of waves
// (merge_rows_grouped), and then each row's log-sum-exp by the first wave of
// its group; rows it leaves, and every row where the sizes do not allow it,
// are merged one after another as for one row.
template <int RM, bool kExtras = true, bool kSample = true, int kRows = 0>
__device__ __forceinline__ void fused_merge_tail(const FusedMerge& f, SelectSmem& sm, FinalSmem& fs,
                                 uint32_t& last) {
  // every store of this thread has been acknowledged (gfx9 counts stores in vmcnt)
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  lds_barrier();
  if (threadIdx.x == 0) {
    const uint32_t done =
        __hip_atomic_fetch_add(f.counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last = done == (uint32_t)f.n_chunks - 1u ? 1u : 0u;
  }
  lds_barrier();
  if (uniform(last) == 0u) return;
  const int64_t n_in = (int64_t)f.n_chunks * f.kc;
  const int n_part = f.n_chunks;  // one log-sum-exp pair per chunk and row
  if constexpr (kRows >= 2 && !kSample) {
    constexpr int G = kMaxWaves / kRows;  // waves per row
    if ((int)(blockDim.x >> 6) >= kRows * G &&
        merge_bounded(f.heads, f.n_chunks, (uint32_t)f.k, kMaxWaves * 64)) {
      // the first wave of each group requests its row's log-sum-exp pairs
      // (n_chunks <= 64 * kLsePairs here) before the merge
      const int wave = wave_id();
      const int row = wave / G;
      const bool lse_lead = kExtras && f.lse_part != nullptr && row < kRows && wave == row * G;
      uint2 pre[kLsePairs];
      const uint2* lse_row = lse_lead ? f.lse_part + (size_t)row * n_part : f.lse_part;
      if (kExtras) load_lse_pairs_wave(lse_row, n_part, lse_lead, pre);
      if (threadIdx.x < (unsigned)kMaxRows) {
        fs.g_sync[threadIdx.x] = 0u;
        fs.g_done[threadIdx.x] = 0u;
      }
      lds_barrier();
      merge_rows_grouped<kRows, G>(f.cand, n_in, f.heads, f.n_chunks, f.kc, (uint32_t)f.k, f.values,
                                   f.indices, fs);
      if (kExtras && lse_lead) lse_wave(pre, f.lse ? f.lse + row : nullptr);
      lds_barrier();
      for (int m = 0; m < kRows; ++m) {
        if (uniform(fs.g_done[m])) continue;
        merge_final<RM, false>(f.cand + (size_t)m * n_in, n_in, f.heads + (size_t)m * f.n_chunks * kHeads,
                               f.n_chunks, f.kc, (uint32_t)f.k, f.values + (size_t)m * f.k,
                               f.indices + (size_t)m * f.k, (int)blockDim.x, sm, fs);
        lds_barrier();  // fs is reused by the next row
      }
      if (threadIdx.x == 0) __hip_atomic_store(f.counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
  }
  for (int m = 0; m < f.M; ++m) {
    // the row's log-sum-exp partials and draw parameters are requested
    // before the merge, which waits for its own loads meanwhile
    uint2 pre[kLsePairs];
    int have = 0;
    if (kExtras && f.lse_part != nullptr) have = load_lse_pairs(f.lse_part + (size_t)m * n_part, n_part, pre);
    RowSample rs;
    if (kSample && f.smp.on) rs = load_row_sample(f.smp, m);
    merge_final<RM, false>(f.cand + (size_t)m * n_in, n_in, f.heads + (size_t)m * f.n_chunks * kHeads,
                    f.n_chunks, f.kc, (uint32_t)f.k, f.values + (size_t)m * f.k,
                    f.indices + (size_t)m * f.k, (int)blockDim.x, sm, fs);
    lds_barrier();  // fs.out_* are complete; fs is reused by the next row
    // the log-sum-exp (wave 0, or the workgroup for many chunks) and the
    // draw's noise (another wave) at the same time, then the draw
    float lse = 0.f;
    if (kExtras && f.lse_part != nullptr)
      lse = merge_lse(f.lse_part + (size_t)m * n_part, n_part, f.lse ? f.lse + m : nullptr, fs, have,
                      pre, kSample && f.smp.on);
    if (kSample && f.smp.on) {
      float* noise = reinterpret_cast<float*>(fs.key);  // free after the merge
      draw_noise(fs.out_idx, f.k, rs, m, f.smp, noise);
      lds_barrier();
      sample_row(fs.out_bits, fs.out_idx, noise, f.k, lse, rs, m, f.smp);
      lds_barrier();  // fs is reused by the next row
    }
  }
  if (threadIdx.x == 0) __hip_atomic_store(f.counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}


struct ChunkOut {
  uint2* cand;        // [M][n_chunks][kc]
  uint2* heads;       // [M][n_chunks][kHeads]
  uint32_t* counter;  // completion counter of the fused merge
  float* values;      // [M][k] final outputs (fused merge)
  int64_t* indices;   // [M][k]
  int n_chunks;
  int kc;
  int k;
  int M;
  int fused;          // the launch's last workgroup merges (fused_merge_tail)
  uint2* lse_part;    // log-sum-exp pairs [M][n_chunks], or null
  float* lse;         // [M] or null
  const int32_t* allowed;  // bitmask [M][allowed_words] (bit 1 = allowed), or null
  int allowed_words;       // ceil(V / 32)
  SampleParams smp;        // the token draw (smp.on == 0: none)
  // select_top_small's providers (small_select_plan): P and h for a full
  // chunk and for the last one
  int sel_p[2], sel_h[2];
};

// The fused merge's view of a chunk launch's outputs.
__device__ __forceinline__ FusedMerge fused_merge_of(const ChunkOut& o) {
  FusedMerge f;
  f.counter = o.counter;
  f.cand = o.cand;
  f.heads = o.heads;
  f.values = o.values;
  f.indices = o.indices;
  f.M = o.M;
  f.n_chunks = o.n_chunks;
  f.kc = o.kc;
  f.k = o.k;
  f.lse_part = o.lse_part;
  f.lse = o.lse;
  f.smp = o.smp;
  return f;
}

// Candidate slots per thread of the fused final merge (n_chunks * kc <=
// 16 * threads per chunk workgroup; the host checks it).
constexpr int kFusedRM = 16;

// Selects the chunk's top-k of row m from RPL slots per lane and writes them
// followed by padding up to kc entries, then the chunk's heads.  Small k:
// select_top_small, candidates in output order.  Otherwise (or when it gives
// up): radix select, candidates in ascending index order.  Either order keeps
// equal values in ascending index, which is all the merge relies on.  `last`
// = no further row follows in this workgroup.
// Bit r: vocabulary row v = rows[r] of activation row m is allowed by the
// call's bitmask (always, without one).  rows[r] must be < V; the loads are
// unconditional (from a valid dummy address without a mask), so a caller
// may issue them among loads whose count must not vary.
template <int RPL>
__device__ __forceinline__ uint32_t allowed_bits(const ChunkOut& o, int m, const int64_t (&rows)[RPL],
                                                 const void* dummy) {
  uint32_t w[RPL];
#pragma unroll
  for (int r = 0; r < RPL; ++r) {
    const int32_t* p = o.allowed != nullptr
                           ? o.allowed + (size_t)m * o.allowed_words + (rows[r] >> 5)
                           : static_cast<const int32_t*>(dummy);
    w[r] = (uint32_t)*p;
  }
  uint32_t bits = 0u;
#pragma unroll
  for (int r = 0; r < RPL; ++r)
    bits |= (o.allowed == nullptr ? 1u : (w[r] >> (rows[r] & 31)) & 1u) << r;
  return bits;
}

// This wave's log-sum-exp pair (max, sum of exp(z - max)) of row m over its
// valid rows, z = zs * logit; the wave that posts its pair last combines the
// chunk's pairs (lane w holds wave w's pair) and stores the chunk's pair.  No
// barrier.
template <int RPL>
__device__ __forceinline__ void chunk_lse_pair(const float (&val)[RPL], uint32_t valid, int m,
                                               const ChunkOut& o, HeadStage& st, float zs) {
  const size_t row_chunk = (size_t)m * o.n_chunks + blockIdx.x;
  const int wave = wave_id();
  const int lane = lane_id();
  float z[RPL];
#pragma unroll
  for (int r = 0; r < RPL; ++r) z[r] = val[r] * zs;
  float mx = -INFINITY;
#pragma unroll
  for (int r = 0; r < RPL; ++r)
    if ((valid >> r) & 1u) mx = fmaxf(mx, z[r]);
  mx = wave_max_f32(mx);
  float sum = mx == INFINITY ? 1.f : 0.f;
  if (mx != INFINITY && mx != -INFINITY) {
#pragma unroll
    for (int r = 0; r < RPL; ++r)
      if ((valid >> r) & 1u) sum += expf(z[r] - mx);
  }
  sum = wave_sum_f32(sum);
  if (lane == 0) st.lse_w[m][wave] = make_uint2(__float_as_uint(mx), __float_as_uint(sum));
  // the pair is written before the count (LDS operations of a wave
  // complete in order; the fence keeps the compiler from reordering)
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  uint32_t done = 0u;
  if (lane == 0) done = atomicAdd(&st.lse_done[m], 1u);
  done = readlane_u32(done, 0);
  if (done == (blockDim.x >> 6) - 1u) {
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    float cm = -INFINITY, cs = 0.f;
    if (lane < (int)(blockDim.x >> 6)) {
      const uint2 p = st.lse_w[m][lane];
      cm = __uint_as_float(p.x);
      cs = __uint_as_float(p.y);
    }
    lse_combine_wave(cm, cs);
    if (lane == 0) st_cand(&o.lse_part[row_chunk], make_uint2(__float_as_uint(cm), __float_as_uint(cs)));
  }
}

// `allow` bit r clear: row r's logit counts as -inf (a disallowed entry).
// zs: the row's logits are scaled by zs before the normaliser partials (1 /
// T of a sampled row, else 1); the candidates keep the logits themselves.
// kExtras false: the call has no log-sum-exp output, bitmask or draw, and
// that code is left out.
template <int RPL, bool kExtras = true>
__device__ __forceinline__ void chunk_select_write(const float (&val_in)[RPL], const int32_t (&idx)[RPL],
                                                   uint32_t valid, int m, const ChunkOut& o,
                                                   SelectSmem& sm, HeadStage& st, bool last,
                                                   uint32_t allow = 0xFFFFFFFFu, float zs = 1.f) {
  float val[RPL];
  uint32_t key[RPL], vb[RPL];
#pragma unroll
  for (int r = 0; r < RPL; ++r) {
    val[r] = (!kExtras || ((allow >> r) & 1u)) ? val_in[r] : -INFINITY;
    vb[r] = __float_as_uint(val[r]);
    key[r] = float_key(val[r]);
  }
  const size_t row_chunk = (size_t)m * o.n_chunks + blockIdx.x;
  if (kExtras && o.lse_part != nullptr) chunk_lse_pair<RPL>(val, valid, m, o, st, zs);
  uint2* out = o.cand + row_chunk * o.kc;
  uint2* heads = o.heads + row_chunk * kHeads;
  const int plan = blockIdx.x == (unsigned)o.n_chunks - 1u ? 1 : 0;  // the last chunk may be partial
  if (o.sel_p[plan] >= 0) {  // small k: the plan's P * h <= 64 tops cover it
    const uint32_t n = select_top_small<RPL>(key, valid, vb, idx, (uint32_t)o.k, o.sel_p[plan],
                                             o.sel_h[plan], st,
                                             [&](uint32_t pos, uint32_t bits, int32_t ix) {
                                               const uint2 e = make_uint2(bits, (uint32_t)ix);
                                               st_cand(&out[pos], e);
                                               if (pos < (uint32_t)kHeads) st_cand(&heads[pos], e);
                                             });
    if (n != 0xFFFFFFFFu) {
      for (int i = (int)n + (int)threadIdx.x; i < o.kc; i += blockDim.x)
        st_cand(&out[i], make_uint2(0u, 0xFFFFFFFFu));
      for (int i = (int)n + (int)threadIdx.x; i < kHeads; i += blockDim.x)
        st_cand(&heads[i], make_uint2(0u, 0xFFFFFFFFu));
      if (!last) lds_barrier();  // the staging is refilled by the next row
      return;
    }
  }
  const SelectRange s = block_select<RPL>(key, valid, (uint32_t)o.k, sm);
  const uint32_t n = block_compact<RPL>(key, valid, s, vb, idx, sm,
                                        [&](uint32_t pos, uint32_t bits, int32_t ix) {
                                          st_cand(&out[pos], make_uint2(bits, (uint32_t)ix));
                                        });
  for (int i = (int)n + (int)threadIdx.x; i < o.kc; i += blockDim.x)
    st_cand(&out[i], make_uint2(0u, 0xFFFFFFFFu));
  // the chunk's best entries are the best of its candidates (a head beyond
  // a k < 4 is still a real logit of the row, which the merge may consider)
  block_heads<RPL>(key, valid, vb, idx, st, heads);
  if (!last) lds_barrier();  // the staging is refilled by the next row
}

// chunk_select_write for rows 0 .. M-1 at once (M >= 2; the binary path):
// each row's candidates and heads as chunk_select_write writes them, with
// the small-k selection of all rows between the same two barriers
// (select_top_rows); rows it leaves (too many staged rows), and every row
// when k is above the small-k range, take the radix select in turn.
template <int RPL, int M, bool kExtras = true>
__device__ __forceinline__ void chunk_select_rows(const float (&val_in)[M][RPL], const int32_t (&idx)[RPL],
                                                  uint32_t valid, const ChunkOut& o, SelectSmem& sm,
                                                  HeadStage& st, const uint32_t (&allow)[M],
                                                  const float (&zs)[M]) {
  uint32_t key[M][RPL], vb[M][RPL];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    float val[RPL];
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
      val[r] = (!kExtras || ((allow[m] >> r) & 1u)) ? val_in[m][r] : -INFINITY;
      vb[m][r] = __float_as_uint(val[r]);
      key[m][r] = float_key(val[r]);
    }
    if (kExtras && o.lse_part != nullptr) chunk_lse_pair<RPL>(val, valid, m, o, st, zs[m]);
  }
  const int plan = blockIdx.x == (unsigned)o.n_chunks - 1u ? 1 : 0;  // the last chunk may be partial
  uint32_t n_out[M];
  const bool small = o.sel_p[plan] >= 0;
  if (small) {
    select_top_rows<M, RPL>(key, valid, vb, idx, (uint32_t)o.k, o.sel_p[plan], o.sel_h[plan], st, n_out,
                            [&](int m, uint32_t pos, uint32_t bits, int32_t ix) {
                              const size_t rc = (size_t)m * o.n_chunks + blockIdx.x;
                              const uint2 e = make_uint2(bits, (uint32_t)ix);
                              st_cand(&o.cand[rc * o.kc + pos], e);
                              if (pos < (uint32_t)kHeads) st_cand(&o.heads[rc * kHeads + pos], e);
                            });
#pragma unroll
    for (int m = 0; m < M; ++m) {
      if (n_out[m] == 0xFFFFFFFFu) continue;
      const size_t rc = (size_t)m * o.n_chunks + blockIdx.x;
      for (int i = (int)n_out[m] + (int)threadIdx.x; i < o.kc; i += blockDim.x)
        st_cand(&o.cand[rc * o.kc + i], make_uint2(0u, 0xFFFFFFFFu));
      for (int i = (int)n_out[m] + (int)threadIdx.x; i < kHeads; i += blockDim.x)
        st_cand(&o.heads[rc * kHeads + i], make_uint2(0u, 0xFFFFFFFFu));
    }
  }
  bool after = false;  // a radix row has run: the next one reuses its LDS
#pragma unroll
  for (int m = 0; m < M; ++m) {
    if (small && n_out[m] != 0xFFFFFFFFu) continue;
    if (after) lds_barrier();
    const size_t rc = (size_t)m * o.n_chunks + blockIdx.x;
    uint2* out = o.cand + rc * o.kc;
    const SelectRange s = block_select<RPL>(key[m], valid, (uint32_t)o.k, sm);
    const uint32_t n = block_compact<RPL>(key[m], valid, s, vb[m], idx, sm,
                                          [&](uint32_t pos, uint32_t bits, int32_t ix) {
                                            st_cand(&out[pos], make_uint2(bits, (uint32_t)ix));
                                          });
    for (int i = (int)n + (int)threadIdx.x; i < o.kc; i += blockDim.x)
      st_cand(&out[i], make_uint2(0u, 0xFFFFFFFFu));
    block_heads<RPL>(key[m], valid, vb[m], idx, st, o.heads + rc * kHeads);
    after = true;
  }
}

// Row m's temperature (1 without a draw; its z_scale is what the normaliser
// partials scale the logits by).  The load is unconditional, from `dummy`
// (any valid address) when the temperatures do not come per row, so a
// caller may issue it among loads whose count must not vary; the value is
// read after the caller's main loop.
__device__ __forceinline__ float row_temperature(const ChunkOut& o, int m, const float* dummy) {
  const bool rows = o.smp.on && o.smp.temperature_rows != nullptr;
  const float x = rows ? o.smp.temperature_rows[m] : *dummy;
  return !o.smp.on ? 1.f : rows ? x : o.smp.temperature;
}

// Streaming loads of the head (and of logits on the selection-only path):
// every byte is used once per call, so they are issued non-temporal (nt),
// which keeps them from displacing other data in the caches and streams
// faster from HBM than plain loads.
__device__ __forceinline__ uint4 ld_stream(const uint4* p) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float ld_stream(const float* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ float4 ld_stream(const float4* p) {
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}

// events: null, or two hipEvent_t that record the kernel's own start and end
template <typename Arg>
inline hipError_t launch1(void (*kern)(Arg), dim3 grid, dim3 block, size_t lds, void* stream, Arg arg,
                   void* const* events = nullptr) {
  if (lds + kChunkStaticLds > 65536) {  // with the static LDS the total may pass 64 KiB
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  void* args[] = {&arg};
  if (events)
    return hipExtLaunchKernel(reinterpret_cast<const void*>(kern), grid, block, args, lds,
                              static_cast<hipStream_t>(stream),
                              static_cast<hipEvent_t>(events[0]),
                              static_cast<hipEvent_t>(events[1]), 0);
  return hipLaunchKernel(reinterpret_cast<const void*>(kern), grid, block, args, lds,
                         static_cast<hipStream_t>(stream));
}
inline ChunkOut chunk_out(const Geometry& g, void* workspace, float* values, int64_t* indices) {
  ChunkOut o;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  o.heads = reinterpret_cast<uint2*>(ws + g.sync_bytes);
  o.cand = reinterpret_cast<uint2*>(ws + g.sync_bytes + g.heads_bytes);
  o.n_chunks = g.n_chunks;
  o.kc = g.kc;
  o.k = g.k;
  o.fused = g.fused;
  o.counter = reinterpret_cast<uint32_t*>(ws);
  o.values = values;
  o.indices = indices;
  o.M = (int)g.M;
  o.lse = g.lse;
  o.allowed = g.allowed;
  o.allowed_words = (int)((g.V + 31) / 32);
  {
    const int nw = g.nw;
    const int cap = g.chunk_rows / nw;  // rows per wave, in row order
    const int kk = g.k < g.chunk_rows ? g.k : g.chunk_rows;
    o.sel_p[0] = small_select_plan(kk, nw, cap, g.chunk_rows, &o.sel_h[0]);
    o.sel_p[1] = small_select_plan(kk, nw, cap, g.V - (int64_t)(g.n_chunks - 1) * g.chunk_rows,
                                   &o.sel_h[1]);
  }
  o.lse_part = (g.lse || g.smp.need_norm)
                   ? reinterpret_cast<uint2*>(ws + g.sync_bytes + g.heads_bytes + g.region0_bytes +
                                              g.region1_bytes)
                   : nullptr;
  o.smp = g.smp;
  return o;
}
}  // namespace lmtopk
