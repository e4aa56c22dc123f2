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

namespace lmtopk {

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
  uint2* lse_part;    // log-sum-exp partials [M][n_chunks][waves], or null
  float* lse;         // [M] or null
  const int32_t* allowed;  // bitmask [M][allowed_words] (bit 1 = allowed), or null
  int allowed_words;       // ceil(V / 32)
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

// `allow` bit r clear: row r's logit counts as -inf (a disallowed entry).
// kExtras false: the call has neither a log-sum-exp output nor a bitmask,
// and that code is left out.
template <int RPL, bool kExtras = true>
__device__ __forceinline__ void chunk_select_write(const float (&val_in)[RPL], const int32_t (&idx)[RPL],
                                                   uint32_t valid, int m, const ChunkOut& o,
                                                   SelectSmem& sm, HeadStage& st, bool last,
                                                   uint32_t allow = 0xFFFFFFFFu) {
  float val[RPL];
  uint32_t key[RPL], vb[RPL];
#pragma unroll
  for (int r = 0; r < RPL; ++r) {
    val[r] = (!kExtras || ((allow >> r) & 1u)) ? val_in[r] : -INFINITY;
    vb[r] = __float_as_uint(val[r]);
    key[r] = float_key(val[r]);
  }
  const size_t row_chunk = (size_t)m * o.n_chunks + blockIdx.x;
  if (kExtras && o.lse_part != nullptr) {
    // this wave's (max, sum of exp(logit - max)) over its valid rows
    const int wave = wave_id();
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < RPL; ++r)
      if ((valid >> r) & 1u) mx = fmaxf(mx, val[r]);
    mx = wave_max_f32(mx);
    float sum = mx == INFINITY ? 1.f : 0.f;
    if (mx != INFINITY && mx != -INFINITY) {
#pragma unroll
      for (int r = 0; r < RPL; ++r)
        if ((valid >> r) & 1u) sum += expf(val[r] - mx);
    }
    sum = wave_sum_f32(sum);
    if (lane_id() == 0)
      st_cand(&o.lse_part[row_chunk * (blockDim.x >> 6) + wave],
              make_uint2(__float_as_uint(mx), __float_as_uint(sum)));
  }
  uint2* out = o.cand + row_chunk * o.kc;
  uint2* heads = o.heads + row_chunk * kHeads;
  if (o.k <= kWaveTops * (int)(blockDim.x >> 6)) {
    const uint32_t n = select_top_small<RPL>(key, valid, vb, idx, (uint32_t)o.k, st,
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
  o.lse_part = g.lse ? reinterpret_cast<uint2*>(ws + g.sync_bytes + g.heads_bytes + g.region0_bytes +
                                                g.region1_bytes)
                     : nullptr;
  return o;
}
}  // namespace lmtopk
