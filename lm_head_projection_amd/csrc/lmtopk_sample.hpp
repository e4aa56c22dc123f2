// lmtopk_sample.hpp - one token per row drawn from the exact top-k survivors
// (logits-processor page, section "API": temperature, top-k, top-p, min-p,
// a draw keyed by (seed, row, offset); section "Method": the filters meet in
// one keep set, the token is drawn by Gumbel-max over it).
//
// Runs in the workgroup that finishes a row's merge, after the merge has
// left the row's k survivors in LDS in output order (value descending, lower
// index first) and, when top-p is on, after the normaliser lse_T of the
// scaled logits z = L / T over the whole vocabulary.  One wave does the
// work: lane l owns the J = ceil(k / 64) consecutive positions
// [l J, l J + J), so a per-lane running sum plus one wave scan gives every
// position the probability mass of the positions before it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lmtopk_device.hpp"
#include "lmtopk_internal.hpp"

namespace lmtopk {

// Philox4x32 with 10 rounds (Salmon, Moraes, Dror and Shaw, "Parallel random
// numbers: as easy as 1, 2, 3", SC 2011): per round, counter words 0 and 2
// are multiplied by the two round constants into 64-bit products; the new
// words are (hi2 ^ c1 ^ k0, lo2, hi0 ^ c3 ^ k1, lo0); the key advances by the
// two Weyl increments before every round after the first.  Only the first
// output word is used.
__device__ __forceinline__ uint32_t philox_word0(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                                 uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint32_t lo0 = 0xD2511F53u * c0, hi0 = __umulhi(0xD2511F53u, c0);
    const uint32_t lo1 = 0xCD9E8D57u * c2, hi1 = __umulhi(0xCD9E8D57u, c2);
    c0 = hi1 ^ c1 ^ k0;
    c1 = lo1;
    c2 = hi0 ^ c3 ^ k1;
    c3 = lo0;
  }
  return c0;
}

// (x >> 9 + 1/2) * 2^-23: a uniform in (0, 1) with 24 significant bits,
// exact in fp32.
__device__ __forceinline__ float uniform_of(uint32_t x) {
  return fmaf((float)(x >> 9), 0x1p-23f, 0x1p-24f);
}

// One row's parameters, loaded once per row (scalars, or the row's entry of
// a per-row array).
struct RowSample {
  float temperature;
  int top_k;
  float top_p;
  float min_p;
  uint64_t offset;
};

__device__ __forceinline__ RowSample load_row_sample(const SampleParams& s, int m) {
  RowSample r;
  r.temperature = s.temperature_rows ? s.temperature_rows[m] : s.temperature;
  r.top_k = s.top_k_rows ? s.top_k_rows[m] : s.top_k;
  r.top_p = s.top_p_rows ? s.top_p_rows[m] : s.top_p;
  r.min_p = s.min_p_rows ? s.min_p_rows[m] : s.min_p;
  r.offset = s.offset_device ? *s.offset_device : s.offset;
  return r;
}

// Scale applied to a row's logits before the normaliser partials: 1 / T for
// a sampled row, 1 for a greedy row or a call without sampling.
__device__ __forceinline__ float z_scale(float temperature) {
  return temperature > 0.f ? 1.f / temperature : 1.f;
}

// Inclusive prefix sum over the 64 lanes, fp32, fixed order.
__device__ __forceinline__ float wave_scan_inclusive_f32(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kRowShr1, 0xF, 0xF, true));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kRowShr2, 0xF, 0xF, true));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kRowShr4, 0xF, 0xF, true));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kRowShr8, 0xF, 0xF, true));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kRowBcast15, 0xA, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kRowBcast31, 0xC, 0xF, false));
  return v;
}

// The positions a row's draw can keep: the top-k limit.
__device__ __forceinline__ int draw_limit(const RowSample& rs, int k) {
  return (rs.top_k <= 0 || rs.top_k >= k) ? k : rs.top_k;
}

// Gumbel noise g_i = -log(-log(u_i)) of positions i < limit of row m's
// survivors (idx [0, k) in LDS, output order), u_i from the Philox stream
// of (vocabulary index, row, offset) under (seed), into g[i].  One wave
// does it (wave 1 when there is one, so that it overlaps wave 0's
// log-sum-exp); the caller orders g with a barrier before sample_row.
__device__ __forceinline__ void draw_noise(const int32_t* idx, int k, const RowSample& rs, int m,
                                           const SampleParams& s, float* g) {
  const int noise_wave = (blockDim.x >> 6) > 1 ? 1 : 0;
  if (wave_id() != noise_wave) return;
  const int limit = draw_limit(rs, k);
  const uint64_t off = rs.offset;
  for (int i = lane_id(); i < limit; i += 64) {
    const uint32_t x = philox_word0((uint32_t)idx[i], (uint32_t)m, (uint32_t)off,
                                    (uint32_t)(off >> 32), (uint32_t)s.seed,
                                    (uint32_t)(s.seed >> 32));
    g[i] = -logf(-logf(uniform_of(x)));
  }
}

// Draws row m's token from its k survivors (bits / idx [0, k) in LDS, output
// order; g [0, limit) their Gumbel noise from draw_noise) and writes
// tokens[m] (and kept[m]).  lse: the normaliser of the scaled logits (read
// only when top-p is on).  Called by every thread of the workgroup; wave 0
// does the work; no barrier inside.
__device__ __forceinline__ void sample_row(const uint32_t* bits, const int32_t* idx, const float* g,
                                           int k, float lse, const RowSample& rs, int m,
                                           const SampleParams& s) {
  if (wave_id() != 0) return;
  const int lane = lane_id();
  const float L0 = __uint_as_float(bits[0]);
  const bool greedy = !(rs.temperature > 0.f) || L0 == INFINITY || L0 == -INFINITY;
  uint32_t n_keep = 1u, pick = 0u;
  if (!greedy) {
    const float zs = 1.f / rs.temperature;
    const float z0 = L0 * zs;
    const int limit = draw_limit(rs, k);
    const bool use_p = rs.top_p < 1.f;
    const bool use_m = rs.min_p > 0.f;
    const int J = (k + 63) >> 6;
    const int i0 = lane * J;
    // probability mass of this lane's positions below the limit
    float mine = 0.f;
    if (use_p) {
      for (int j = 0; j < J; ++j) {
        const int i = i0 + j;
        if (i >= limit) break;
        mine += expf(__uint_as_float(bits[i]) * zs - lse);
      }
    }
    float below = wave_scan_inclusive_f32(mine) - mine;  // mass before this lane's first position
    // first position that leaves the prefix (limit if none)
    uint32_t stop = (uint32_t)limit;
    for (int j = 0; j < J; ++j) {
      const int i = i0 + j;
      if (i >= limit) break;
      const float z = __uint_as_float(bits[i]) * zs;
      if (i > 0 && (z == -INFINITY || (use_p && below >= rs.top_p) ||
                    (use_m && expf(z - z0) < rs.min_p))) {
        stop = (uint32_t)i;
        break;
      }
      if (use_p) below += expf(z - lse);
    }
    n_keep = wave_min_u32(stop);
    // Gumbel-max over the kept prefix; a lane's positions ascend, so its
    // first maximum is its lowest position
    float best = -INFINITY;
    uint32_t best_i = 0xFFFFFFFFu;
    for (int j = 0; j < J; ++j) {
      const int i = i0 + j;
      if (i >= (int)n_keep) break;
      const float v = __uint_as_float(bits[i]) * zs + g[i];
      if (v > best) {
        best = v;
        best_i = (uint32_t)i;
      }
    }
    const float top = wave_max_f32(best);
    pick = wave_min_u32(best == top ? best_i : 0xFFFFFFFFu);
  }
  if (lane == 0) {
    s.tokens[m] = (int64_t)idx[pick];
    if (s.kept) s.kept[m] = (int32_t)n_keep;
  }
}

}  // namespace lmtopk
