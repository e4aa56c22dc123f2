// lmtopk_device.hpp - device-side selection building blocks for gfx950 (wave64).
//
// Exact top-k of a set of fp32 scores spread over the registers of one
// workgroup.  Used by every chunk kernel (the per-chunk selection of the
// lm-head-topk page, section "Method": each chunk offers its own k
// candidates) and by the merge kernel (the page's second pass).
//
// Order: value descending, equal values by lower index first, +0.0 == -0.0
// (lm-head-topk page, sections "API" and "Method").  Scores are mapped to
// order-preserving unsigned keys; positions in the workgroup's slot order are
// always arranged so that slot order == vocabulary index order, so "lower
// index first" becomes "earlier slot first".
//
// Selection is an MSB-first radix select on the keys:
//   1. block min / max / count of the valid keys; the bits the min and max
//      share are common to every key, so the search starts below them;
//   2. 8-bit digits: per-digit counts in an LDS histogram (integer atomics,
//      so the result does not depend on their order), a wave-wide suffix scan
//      finds the digit that holds the k-th key, and the search stops as soon
//      as the keys that share the prefix found so far are exactly the ones
//      still needed;
//   3. ordered compaction: keys above the prefix range are all taken, keys in
//      the range are taken in slot order until k are taken.
// Every wave repeats the (cheap) decision of step 2 itself, so each digit
// costs one barrier; three histogram buffers rotate so that clearing the next
// one never races with a wave still reading the current one.

#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lmtopk {

constexpr int kWave = 64;
constexpr int kMaxWaves = 16;
constexpr int kMaxK = 2048;

// Order-preserving map fp32 -> uint32 (larger float => larger key).  -0.0 is
// first turned into +0.0 so the two tie.
__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u << 1) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int lane_id() {
  return (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

// Number of set bits of `mask` below this lane.
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

__device__ __forceinline__ uint32_t readlane_u32(uint32_t v, int lane) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, lane);
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, o));
  return v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o));
  return v;
}

// Inclusive prefix sum over lanes 0..15 (lanes >= 16 get garbage).
__device__ __forceinline__ uint32_t scan16_inclusive(uint32_t x, int lane) {
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) {
    uint32_t t = (uint32_t)__shfl_up((int)x, o);
    if (lane >= o) x += t;
  }
  return x;
}

// LDS used by one selection (any number of sequential selections may reuse it).
struct alignas(16) SelectSmem {
  uint32_t hist[3][256];
  uint32_t wmin[kMaxWaves];
  uint32_t wmax[kMaxWaves];
  uint32_t wcnt[kMaxWaves];
  uint32_t cgt[kMaxWaves];
  uint32_t ceq[kMaxWaves];
};

// Outcome of the search: keys k with (k & mask) > prefix are all selected;
// keys with (k & mask) == prefix are selected in slot order, the first
// `need` of them.  total = number of valid keys.
struct SelectRange {
  uint32_t prefix;
  uint32_t mask;
  uint32_t need;
  uint32_t total;
};

// Block-wide search.  Every thread of the block must call it with its R
// slots; slot r of lane l in wave w has position (w * R + r) * 64 + l.
// valid bit r of `valid` marks slot r as a real entry.  k >= 1.
template <int R>
__device__ SelectRange block_select(const uint32_t (&key)[R], uint32_t valid, uint32_t k,
                                    SelectSmem& sm) {
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid >> 6;
  const int nw = blockDim.x >> 6;

  // histogram buffers 0 and 1 start clean; buffer 2 is cleared in pass 0
  for (int i = tid; i < 512; i += blockDim.x) (&sm.hist[0][0])[i] = 0u;

  uint32_t lmin = 0xFFFFFFFFu, lmax = 0u, cnt = 0u;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const bool v = (valid >> r) & 1u;
    if (v) {
      lmin = min(lmin, key[r]);
      lmax = max(lmax, key[r]);
    }
    cnt += (uint32_t)__popcll(ballot(v));
  }
  lmin = wave_min_u32(lmin);
  lmax = wave_max_u32(lmax);
  if (lane == 0) {
    sm.wmin[wave] = lmin;
    sm.wmax[wave] = lmax;
    sm.wcnt[wave] = cnt;
  }
  __syncthreads();
  uint32_t a = 0xFFFFFFFFu, b = 0u, c = 0u;
  if (lane < nw) {
    a = sm.wmin[lane];
    b = sm.wmax[lane];
    c = sm.wcnt[lane];
  }
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) {
    a = min(a, (uint32_t)__shfl_xor((int)a, o));
    b = max(b, (uint32_t)__shfl_xor((int)b, o));
    c += (uint32_t)__shfl_xor((int)c, o);
  }
  const uint32_t gmin = readlane_u32(a, 0);
  const uint32_t gmax = readlane_u32(b, 0);
  const uint32_t total = readlane_u32(c, 0);

  SelectRange res;
  res.total = total;
  if (total <= k) {  // every valid entry is selected
    res.prefix = 0u;
    res.mask = 0u;
    res.need = total;
    return res;
  }
  if (gmin == gmax) {  // all valid keys equal: first k in slot order
    res.prefix = gmin;
    res.mask = 0xFFFFFFFFu;
    res.need = k;
    return res;
  }
  const int common = __clz(gmin ^ gmax);  // leading bits shared by every key
  uint32_t mask = common ? (0xFFFFFFFFu << (32 - common)) : 0u;
  uint32_t prefix = gmin & mask;
  uint32_t need = k;
  int hi = 31 - common;  // highest bit not yet decided
  int pass = 0;
  while (true) {
    const int shift = hi >= 7 ? hi - 7 : 0;
    const uint32_t dmask = (2u << (hi - shift)) - 1u;
    uint32_t* hist = sm.hist[pass % 3];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (((valid >> r) & 1u) && ((key[r] & mask) == prefix))
        atomicAdd(&hist[(key[r] >> shift) & dmask], 1u);
    }
    __syncthreads();
    // every wave finds the digit of the k-th key on its own
    const uint4 h = *reinterpret_cast<const uint4*>(&hist[4 * lane]);
    const uint32_t s3 = h.w, s2 = h.z + s3, s1 = h.y + s2, s0 = h.x + s1;
    uint32_t x = s0;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t t = (uint32_t)__shfl_down((int)x, o);
      if (lane + o < 64) x += t;
    }
    const uint32_t after = x - s0;  // keys in lanes above this one
    const uint64_t have = ballot(s0 + after >= need);
    const int L = 63 - __clzll(have);
    uint32_t ge_i, h_i;
    int i_star;
    if (s3 + after >= need) { i_star = 3; ge_i = s3 + after; h_i = h.w; }
    else if (s2 + after >= need) { i_star = 2; ge_i = s2 + after; h_i = h.z; }
    else if (s1 + after >= need) { i_star = 1; ge_i = s1 + after; h_i = h.y; }
    else { i_star = 0; ge_i = s0 + after; h_i = h.x; }
    const uint32_t digit = 4u * (uint32_t)L + readlane_u32((uint32_t)i_star, L);
    const uint32_t ge = readlane_u32(ge_i, L);
    const uint32_t cnt_eq = readlane_u32(h_i, L);
    const uint32_t above = ge - cnt_eq;
    // clear the buffer two passes ahead (its readers finished before this barrier)
    uint32_t* nxt = sm.hist[(pass + 2) % 3];
    for (int i = tid; i < 256; i += blockDim.x) nxt[i] = 0u;
    need -= above;
    prefix |= digit << shift;
    mask |= dmask << shift;
    if (cnt_eq == need || shift == 0) break;
    hi = shift - 1;
    ++pass;
  }
  res.prefix = prefix;
  res.mask = mask;
  res.need = need;
  return res;
}

// Ordered compaction after block_select.  Calls sink(pos, value_bits, index)
// for each selected slot, pos in [0, selected) following slot order.
// Returns the number selected (uniform).  vbits[r], index[r] are the payload
// of slot r.
template <int R, typename Sink>
__device__ uint32_t block_compact(const uint32_t (&key)[R], uint32_t valid, const SelectRange& s,
                                  const uint32_t (&vbits)[R], const int32_t (&index)[R],
                                  SelectSmem& sm, Sink&& sink) {
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid >> 6;
  const int nw = blockDim.x >> 6;
  bool gt[R], eq[R];
  uint32_t ngt = 0, neq = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const bool v = (valid >> r) & 1u;
    const uint32_t km = key[r] & s.mask;
    gt[r] = v && km > s.prefix;
    eq[r] = v && km == s.prefix;
    ngt += (uint32_t)__popcll(ballot(gt[r]));
    neq += (uint32_t)__popcll(ballot(eq[r]));
  }
  if (lane == 0) {
    sm.cgt[wave] = ngt;
    sm.ceq[wave] = neq;
  }
  __syncthreads();
  uint32_t cg = 0, ce = 0;
  if (lane < nw) {
    cg = sm.cgt[lane];
    ce = sm.ceq[lane];
  }
  const uint32_t ce_incl = scan16_inclusive(ce, lane);
  const uint32_t ce_excl = ce_incl - ce;
  const uint32_t left = s.need > ce_excl ? s.need - ce_excl : 0u;
  const uint32_t take = lane < nw ? min(ce, left) : 0u;
  const uint32_t sel = cg + take;
  const uint32_t sel_incl = scan16_inclusive(sel, lane);
  uint32_t eq_before = readlane_u32(ce_excl, wave);
  uint32_t sel_before = readlane_u32(sel_incl - sel, wave);
  const uint32_t selected = readlane_u32(sel_incl, nw - 1);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint64_t beq = ballot(eq[r]);
    const bool tk = eq[r] && (eq_before + lanes_below(beq) < s.need);
    const bool pick = gt[r] || tk;
    const uint64_t bsel = ballot(pick);
    if (pick) sink(sel_before + lanes_below(bsel), vbits[r], index[r]);
    eq_before += (uint32_t)__popcll(beq);
    sel_before += (uint32_t)__popcll(bsel);
  }
  return selected;
}

}  // namespace lmtopk
