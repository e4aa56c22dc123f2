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
constexpr int kMaxRows = 8;  // activation rows per call
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

// A value the whole wave shares, marked as such for the compiler (scalar
// register), e.g. the wave index or a count read from LDS: loops and
// branches on it stay uniform instead of becoming per-lane.
__device__ __forceinline__ uint32_t uniform(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int wave_id() { return (int)uniform(threadIdx.x >> 6); }

__device__ __forceinline__ uint32_t readlane_u32(uint32_t v, int lane) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, lane);
}

// Cross-lane steps with DPP (gfx9 row and broadcast controls).  A DPP read of
// a lane that is out of range, or of a row masked off, yields `old`.
template <int kCtrl, int kRowMask = 0xF, bool kBoundZero = false>
__device__ __forceinline__ uint32_t dpp(uint32_t old, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, kCtrl, kRowMask, 0xF, kBoundZero);
}
constexpr int kQuadBcast0 = 0x00;    // quad_perm [0,0,0,0]
constexpr int kQuadBcast3 = 0xFF;    // quad_perm [3,3,3,3]
constexpr int kQuadSwap1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;
constexpr int kRowBcast15 = 0x142;   // lane 15 of a row -> the next row
constexpr int kRowBcast31 = 0x143;   // lane 31 -> rows 2 and 3
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;

// Wave-wide min / max / sum; the result is returned to every lane.
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, dpp<kQuadSwap1>(0xFFFFFFFFu, v));
  v = min(v, dpp<kQuadSwap2>(0xFFFFFFFFu, v));
  v = min(v, dpp<kRowHalfMirror>(0xFFFFFFFFu, v));
  v = min(v, dpp<kRowMirror>(0xFFFFFFFFu, v));
  v = min(v, dpp<kRowBcast15, 0xA>(0xFFFFFFFFu, v));
  v = min(v, dpp<kRowBcast31, 0xC>(0xFFFFFFFFu, v));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp<kQuadSwap1>(0u, v));
  v = max(v, dpp<kQuadSwap2>(0u, v));
  v = max(v, dpp<kRowHalfMirror>(0u, v));
  v = max(v, dpp<kRowMirror>(0u, v));
  v = max(v, dpp<kRowBcast15, 0xA>(0u, v));
  v = max(v, dpp<kRowBcast31, 0xC>(0u, v));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// The same steps on fp32 values: max (identity -inf) and sum (identity 0) in
// a fixed order, so a result does not depend on timing.
template <int kCtrl, int kRowMask = 0xF>
__device__ __forceinline__ float dpp_f32(float old, float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), kCtrl,
                                                    kRowMask, 0xF, false));
}
__device__ __forceinline__ float wave_max_f32(float v) {
  v = fmaxf(v, dpp_f32<kQuadSwap1>(-INFINITY, v));
  v = fmaxf(v, dpp_f32<kQuadSwap2>(-INFINITY, v));
  v = fmaxf(v, dpp_f32<kRowHalfMirror>(-INFINITY, v));
  v = fmaxf(v, dpp_f32<kRowMirror>(-INFINITY, v));
  v = fmaxf(v, dpp_f32<kRowBcast15, 0xA>(-INFINITY, v));
  v = fmaxf(v, dpp_f32<kRowBcast31, 0xC>(-INFINITY, v));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ __forceinline__ float wave_sum_f32(float v) {
  v += dpp_f32<kQuadSwap1>(0.f, v);
  v += dpp_f32<kQuadSwap2>(0.f, v);
  v += dpp_f32<kRowHalfMirror>(0.f, v);
  v += dpp_f32<kRowMirror>(0.f, v);
  v += dpp_f32<kRowBcast15, 0xA>(0.f, v);
  v += dpp_f32<kRowBcast31, 0xC>(0.f, v);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Inclusive prefix sum over the 16 lanes of each row (Kogge-Stone, zero fill).
__device__ __forceinline__ uint32_t row_scan_inclusive(uint32_t v) {
  v += dpp<kRowShr1, 0xF, true>(0u, v);
  v += dpp<kRowShr2, 0xF, true>(0u, v);
  v += dpp<kRowShr4, 0xF, true>(0u, v);
  v += dpp<kRowShr8, 0xF, true>(0u, v);
  return v;
}

// Inclusive prefix sum over all 64 lanes.
__device__ __forceinline__ uint32_t wave_scan_inclusive(uint32_t v) {
  v = row_scan_inclusive(v);
  v += dpp<kRowBcast15, 0xA>(0u, v);
  v += dpp<kRowBcast31, 0xC>(0u, v);
  return v;
}

// Workgroup barrier that orders LDS only: LDS writes before it are visible to
// every wave after it, while global loads in flight stay in flight (a full
// __syncthreads() would also wait for them).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Candidate lists and chunk heads are written by every chunk workgroup and,
// on the fused path, read back by the last workgroup of the same launch,
// which may sit on another XCD with its own L2.  They are therefore accessed
// with device-scope (agent) atomic loads and stores: on gfx950 these are
// plain 8-byte vector loads and stores whose scope bits make the store write
// through the XCD's L2 and the load fetch past it, so no cache write-back
// fence is needed.
__device__ __forceinline__ void st_cand(uint2* p, uint2 v) {
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), ((uint64_t)v.y << 32) | (uint64_t)v.x,
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint2 ld_cand(const uint2* p) {
  const uint64_t x = __hip_atomic_load(const_cast<uint64_t*>(reinterpret_cast<const uint64_t*>(p)),
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return make_uint2((uint32_t)x, (uint32_t)(x >> 32));
}

// LDS used by one selection (any number of sequential selections may reuse
// it).  NC copies of each 256-bin histogram: bin d of copy c is word
// d * NC + c, and lane l adds into copy l % NC, so that up to NC lanes of a
// wave with the same digit hit different words (fewer same-word atomics
// where the digits are skewed); the chunk kernels use one copy (their LDS is
// mostly the activations), the merge launches four.
template <int NC>
struct alignas(16) SelectSmemT {
  static_assert(NC == 1 || NC == 4, "one or four histogram copies");
  uint32_t hist[3][256 * NC];
  uint32_t wmin[kMaxWaves];
  uint32_t wmax[kMaxWaves];
  uint32_t wcnt[kMaxWaves];
  uint32_t cgt[kMaxWaves];
  uint32_t ceq[kMaxWaves];
};
using SelectSmem = SelectSmemT<1>;
using MergeSelectSmem = SelectSmemT<4>;

// Outcome of the search: keys k with (k & mask) > prefix are all selected;
// keys with (k & mask) == prefix are selected in slot order, the first
// `need` of them.  total = number of valid keys.
struct SelectRange {
  uint32_t prefix;
  uint32_t mask;
  uint32_t need;
  uint32_t total;
  uint32_t kmax;  // largest valid key (0 if none)
};

// Block-wide search.  Every thread of the block must call it with its R
// slots; slot r of lane l in wave w has position (w * R + r) * 64 + l.
// valid bit r of `valid` marks slot r as a real entry.  k >= 1.
template <int R, int NC>
__device__ SelectRange block_select(const uint32_t (&key)[R], uint32_t valid, uint32_t k,
                                    SelectSmemT<NC>& sm) {
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = wave_id();
  const int nw = blockDim.x >> 6;

  // histogram buffers 0 and 1 start clean; buffer 2 is cleared in pass 0
  for (int i = tid; i < 512 * NC; i += blockDim.x) (&sm.hist[0][0])[i] = 0u;

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
  lds_barrier();
  uint32_t a = 0xFFFFFFFFu, b = 0u, c = 0u;
  if (lane < nw) {
    a = sm.wmin[lane];
    b = sm.wmax[lane];
    c = sm.wcnt[lane];
  }
  const uint32_t gmin = wave_min_u32(a);
  const uint32_t gmax = wave_max_u32(b);
  const uint32_t total = readlane_u32(row_scan_inclusive(c), 15);

  SelectRange res;
  res.total = total;
  res.kmax = total ? gmax : 0u;
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
      if (((valid >> r) & 1u) && ((key[r] & mask) == prefix)) {
        const uint32_t d = (key[r] >> shift) & dmask;
        atomicAdd(&hist[NC == 1 ? d : d * NC + (uint32_t)(lane & (NC - 1))], 1u);
      }
    }
    lds_barrier();
    // every wave finds the digit of the k-th key on its own (lane l: digits
    // 4l .. 4l + 3)
    uint4 h;
    if (NC == 1) {
      h = *reinterpret_cast<const uint4*>(&hist[4 * lane]);
    } else {
      uint32_t c[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 q = *reinterpret_cast<const uint4*>(&hist[(4 * lane + i) * NC]);
        c[i] = q.x + q.y + q.z + q.w;
      }
      h = make_uint4(c[0], c[1], c[2], c[3]);
    }
    const uint32_t s3 = h.w, s2 = h.z + s3, s1 = h.y + s2, s0 = h.x + s1;
    const uint32_t incl = wave_scan_inclusive(s0);
    const uint32_t after = readlane_u32(incl, 63) - incl;  // keys in lanes above this one
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
    for (int i = tid; i < 256 * NC; i += blockDim.x) nxt[i] = 0u;
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
template <int R, int NC, typename Sink>
__device__ uint32_t block_compact(const uint32_t (&key)[R], uint32_t valid, const SelectRange& s,
                                  const uint32_t (&vbits)[R], const int32_t (&index)[R],
                                  SelectSmemT<NC>& sm, Sink&& sink) {
  const int lane = lane_id();
  const int wave = wave_id();
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
  lds_barrier();
  uint32_t cg = 0, ce = 0;
  if (lane < nw) {
    cg = sm.cgt[lane];
    ce = sm.ceq[lane];
  }
  const uint32_t ce_incl = row_scan_inclusive(ce);
  const uint32_t ce_excl = ce_incl - ce;
  const uint32_t left = s.need > ce_excl ? s.need - ce_excl : 0u;
  const uint32_t take = lane < nw ? min(ce, left) : 0u;
  const uint32_t sel = cg + take;
  const uint32_t sel_incl = row_scan_inclusive(sel);
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

// Chunk heads: besides its candidates, every chunk writes its kHeads best
// candidates in output order (value desc, index asc), padded with index -1.
// The merge reads only these heads unless a chunk may hold more winners than
// its heads.
constexpr int kHeads = 4;

// Small-k chunk selection (select_top_small): its providers' tops number at
// most kMaxWaves * kWaveTops = 64 (so k <= 64).
constexpr int kWaveTops = 4;
// ... and gives up (the radix select runs) above this many survivors.
constexpr uint32_t kSmallSurvivorsMax = 256;

// Providers of select_top_small for a chunk of n_valid valid rows (its
// first rows), wave w holding rows [w cap, (w + 1) cap): the first P waves,
// all of whose rows are valid (3/4 of the waves, fewer in a partial last
// chunk), each take h = ceil(k / P) tops, with P * h <= 64 and h <= cap (P
// shrinks until both hold).  Returns P (and h); 0 when no such P exists and
// at most kSmallSurvivorsMax rows are valid (every valid row is staged), -1
// otherwise (the radix select runs).  Host and device.
__host__ __device__ inline int small_select_plan(int k, int nw, int cap, int64_t n_valid, int* h_out) {
  const int full = (int)(n_valid / cap);
  int P = (3 * nw) / 4;
  P = P < 1 ? 1 : P;
  P = P < full ? P : full;
  int h = P > 0 ? (k + P - 1) / P : 0;
  if (P * h > kMaxWaves * kWaveTops) {
    P = nw < full ? nw : full;
    h = (k + P - 1) / P;
  }
  while (P > 1 && (P * h > kMaxWaves * kWaveTops || h > cap)) {
    --P;
    h = (k + P - 1) / P;
  }
  *h_out = h;
  if (P >= 1 && P * h <= kMaxWaves * kWaveTops && h <= cap) return P;
  *h_out = 0;
  return n_valid <= (int64_t)kSmallSurvivorsMax ? 0 : -1;
}

// LDS of the chunk selection's second stage: staged entries, their ranks and
// the small-k path's per-wave tops.
struct alignas(16) HeadStage {
  uint32_t tops[kMaxWaves * kWaveTops];  // select_top_small: the providers' tops
  uint32_t hkey[kMaxWaves * kHeads];     // block_heads: each wave's best entries
  int32_t hidx[kMaxWaves * kHeads];
  uint32_t hbits[kMaxWaves * kHeads];
  uint32_t key[kMaxK];
  uint32_t bits[kMaxK];
  int32_t idx[kMaxK];
  uint32_t rank[kMaxK];  // zero between uses
  // select_top_small's scalars, zero between uses
  uint32_t count;      // staged rows
  uint32_t tops_done;  // provider waves that have published their tops
  uint32_t thr_ready;  // thr is valid
  uint32_t thr;        // T
  // the chunk's log-sum-exp pairs: one per wave and row, and per row the
  // waves that have posted theirs (zero from head_stage_init on)
  uint2 lse_w[kMaxRows][kMaxWaves];
  uint32_t lse_done[kMaxRows];
  // select_top_rows (several rows at once): per row the providers' tops and
  // the scalars above, zero between uses; row m stages into entries
  // [m * kSmallSurvivorsMax, (m + 1) * kSmallSurvivorsMax) of key .. rank
  uint32_t rtops[kMaxRows][kMaxWaves * kWaveTops];
  uint32_t rcount[kMaxRows];
  uint32_t rtops_done[kMaxRows];
  uint32_t rthr_ready[kMaxRows];
  uint32_t rthr[kMaxRows];
};
static_assert(kMaxRows * kSmallSurvivorsMax <= kMaxK, "every row's staging fits");

// Puts st in the state select_top_small, select_top_rows (kRows) and
// block_heads expect on entry; the caller orders it before their first use
// with a barrier.
template <bool kRows = false>
__device__ __forceinline__ void head_stage_init(HeadStage& st) {
  for (int i = threadIdx.x; i < kMaxK; i += blockDim.x) st.rank[i] = 0u;
  if (threadIdx.x == 0) {
    st.count = 0u;
    st.tops_done = 0u;
    st.thr_ready = 0u;
  }
  if (threadIdx.x < kMaxRows) st.lse_done[threadIdx.x] = 0u;
  if (kRows && threadIdx.x < kMaxRows) {
    st.rcount[threadIdx.x] = 0u;
    st.rtops_done[threadIdx.x] = 0u;
    st.rthr_ready[threadIdx.x] = 0u;
  }
}

// Counting over n entries in LDS, for each entry i < n:
//   kAhead: rank[i] += #{j : key[j] > key[i], or key[j] == key[i] and
//           idx[j] < idx[i]} (idx == nullptr: positions instead of idx), the
//           entry's position in (key desc, idx asc) order; idx >= 0, so
//           (key, idx) compares as one unsigned 64-bit word, the key high
//           and the complemented index low;
//   else:   rank[i] += #{j : key[j] >= key[i]} (idx unused; the entry itself
//           counts).
// The jobs (slice of 16 entries j, read as four LDS broadcasts per array;
// block of 64 entries i) are spread over every wave, and each adds its
// counts with one LDS atomic per entry (integer adds: the result does not
// depend on their order).  Wide slices keep the per-job overhead small; the
// whole workgroup's VALU is one shared pool.
// key and idx must be readable up to index 16 * ceil(n / 16) (entries past
// n are not counted); rank[0, n) must be zero on entry; the caller orders
// the result with a barrier.
// (wave, nw: this wave's place among the waves sharing the jobs, by default
// the whole workgroup.)
template <bool kAhead = true>
__device__ __forceinline__ void rank_count(const uint32_t* key, const int32_t* idx, uint32_t n,
                                           uint32_t* rank, uint32_t wave = (uint32_t)wave_id(),
                                           uint32_t nw = blockDim.x >> 6) {
  n = uniform(n);
  if (n == 0u) return;
  const int lane = lane_id();
  const uint32_t nb = (n + 63u) >> 6;
  const uint32_t ns = (n + 15u) >> 4;
  // job = (slice, block), spread over every wave
  for (uint32_t job = wave; job < ns * nb; job += nw) {
    const uint32_t sl = job % ns, b = job / ns;
    const uint32_t j0 = sl * 16u;
    uint32_t kj[16];
    int32_t ij[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 kq = *reinterpret_cast<const uint4*>(&key[j0 + 4 * q]);
      kj[4 * q] = kq.x;
      kj[4 * q + 1] = kq.y;
      kj[4 * q + 2] = kq.z;
      kj[4 * q + 3] = kq.w;
      if (kAhead) {
        const int4 iq = idx ? *reinterpret_cast<const int4*>(&idx[j0 + 4 * q])
                            : make_int4((int)j0 + 4 * q, (int)j0 + 4 * q + 1, (int)j0 + 4 * q + 2,
                                        (int)j0 + 4 * q + 3);
        ij[4 * q] = iq.x;
        ij[4 * q + 1] = iq.y;
        ij[4 * q + 2] = iq.z;
        ij[4 * q + 3] = iq.w;
      }
    }
    const uint32_t m = min(16u, n - j0);  // real entries in this slice
    const uint32_t i = b * 64u + (uint32_t)lane;
    const bool vi = i < n;
    const uint32_t ki = vi ? key[i] : 0u;
    const int32_t ii = (kAhead && vi) ? (idx ? idx[i] : (int32_t)i) : 0;
    uint32_t c = 0u;
    const uint64_t ki64 = ((uint64_t)ki << 32) | (uint64_t)(~(uint32_t)ii);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const uint64_t kj64 = ((uint64_t)kj[e] << 32) | (uint64_t)(~(uint32_t)ij[e]);
      const bool hit = kAhead ? kj64 > ki64 : kj[e] >= ki;
      c += ((uint32_t)e < m && hit) ? 1u : 0u;
    }
    if (vi && c) atomicAdd(&rank[i], c);
  }
}

// The kHeads best valid entries of a chunk row in output order -> heads[0,
// kHeads), padded with index -1, straight from the registers (slot layout as
// in block_select).  Each wave takes its kHeads best (largest key, lowest
// position among equal keys); wave 0 ranks the waves' entries by (key desc,
// index asc).  Called by the whole workgroup; ends without a barrier.
template <int R>
__device__ void block_heads(const uint32_t (&key)[R], uint32_t valid, const uint32_t (&vbits)[R],
                            const int32_t (&index)[R], HeadStage& st, uint2* heads) {
  const int lane = lane_id();
  const int wave = wave_id();
  const int nw = blockDim.x >> 6;
  uint32_t left = valid;
#pragma unroll
  for (int h = 0; h < kHeads; ++h) {
    uint32_t best = 0u;
    int br = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (((left >> r) & 1u) && key[r] > best) {
        best = key[r];
        br = r;
      }
    }
    const uint32_t wm = wave_max_u32(best);
    const int slot = wave * kHeads + h;
    if (wm == 0u) {  // fewer than h + 1 valid entries in this wave
      if (lane == 0) {
        st.hkey[slot] = 0u;
        st.hidx[slot] = 0x7FFFFFFF;
        st.hbits[slot] = 0u;
      }
      continue;
    }
    // among equal keys the lowest position (r * 64 + lane) is the lowest index
    const uint32_t pmin = wave_min_u32(best == wm ? (uint32_t)(br * 64 + lane) : 0xFFFFFFFFu);
    if ((uint32_t)(br * 64 + lane) == pmin && best == wm) {
      st.hkey[slot] = wm;
      st.hidx[slot] = index[br];
      st.hbits[slot] = vbits[br];
      left &= ~(1u << br);
    }
  }
  lds_barrier();
  if (wave == 0) {
    const int E = nw * kHeads;
    uint32_t e = 0u;
    int32_t ei = 0x7FFFFFFF;
    if (lane < E) {
      e = st.hkey[lane];
      ei = st.hidx[lane];
    }
    uint32_t rank = 0;
    for (int q = 0; q < E; q += 4) {
      const uint4 kq = *reinterpret_cast<const uint4*>(&st.hkey[q]);
      const int4 iq = *reinterpret_cast<const int4*>(&st.hidx[q]);
      rank += (kq.x > e || (kq.x == e && iq.x < ei)) ? 1u : 0u;
      rank += (kq.y > e || (kq.y == e && iq.y < ei)) ? 1u : 0u;
      rank += (kq.z > e || (kq.z == e && iq.z < ei)) ? 1u : 0u;
      rank += (kq.w > e || (kq.w == e && iq.w < ei)) ? 1u : 0u;
    }
    // absent entries (key 0, index INT_MAX) rank after every real one
    if (lane < E && rank < (uint32_t)kHeads)
      st_cand(&heads[rank], e != 0u ? make_uint2(st.hbits[lane], (uint32_t)ei) : make_uint2(0u, 0xFFFFFFFFu));
  }
}

// T in the LDS address space: volatile accesses through a generic pointer
// would become flat accesses, which wait for every outstanding global load.
template <typename T>
using lds_t = __attribute__((address_space(3))) T;

// Bound of a wave's wait for the selection threshold (polls with a short
// sleep each; the wave that publishes it never waits for anything).
constexpr int kThresholdSpinMax = 1 << 22;

// Exact top-k of one chunk row for small k (a plan of P * h <= 64 tops), without
// radix passes.  The first P waves (the "providers", all of whose rows are
// valid; `small_select_plan`) each take their h largest keys; the provider
// that completes this set finds T, the k-th largest of the P h tops, alone
// and publishes it.  P = 0: every valid row is staged (a last chunk of at
// most kSmallSurvivorsMax rows).  T is at most the chunk's k-th largest key
// (the tops are real entries of the chunk), so every winner has key >= T.
// Every wave stages its rows with key >= T as soon as T is published: the
// waves a CU serves first have finished streaming long before the last
// ones, so T and most of the staging are ready when the last wave arrives,
// and no barrier precedes the staging.  The staged rows (typically a few
// more than k) are ranked after one barrier, and out(pos, value_bits,
// index) is called for output positions pos < min(k, valid rows), in no
// particular order of calls.  Returns that count, or 0xFFFFFFFF (after
// writing nothing) when more than kSmallSurvivorsMax rows pass T, e.g. with
// many equal keys.  Slot r of lane l in wave w is position (w * R + r) * 64
// + l as in block_select.  st must be as head_stage_init leaves it and is so
// again on return.  Two barriers: after the staging, after the ranks.
template <int R, typename Out>
__device__ uint32_t select_top_small(const uint32_t (&key)[R], uint32_t valid,
                                     const uint32_t (&vbits)[R], const int32_t (&index)[R],
                                     uint32_t k, int P, int h, HeadStage& st, Out&& out) {
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = wave_id();
  P = uniform(P);
  h = uniform(h);
  const bool stage_all = P == 0;

  // 1. providers: this wave's h largest keys (repeats count), 0 where absent
  if (!stage_all && wave < P) {
    uint32_t left = valid, top = 0u;
    for (int j = 0; j < h; ++j) {
      uint32_t best = 0u;
      int br = 0;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if (((left >> r) & 1u) && key[r] > best) {
          best = key[r];
          br = r;
        }
      }
      const uint32_t wm = wave_max_u32(best);
      if (lane == j) top = wm;
      if (wm == 0u) break;
      const uint64_t holders = ballot(best == wm);
      if (lane == __ffsll((long long)holders) - 1) left &= ~(1u << br);
    }
    if (lane < h) st.tops[wave * h + lane] = top;
    // the tops are written before the count (LDS operations of a wave
    // complete in order; the fence keeps the compiler from reordering)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    uint32_t done = 0u;
    if (lane == 0) done = atomicAdd(&st.tops_done, 1u);
    done = readlane_u32(done, 0);
    if (done == (uint32_t)P - 1u) {
      // the last provider: T = the largest top with at least k tops >= it
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
      const int E = P * h;  // <= 64
      const uint32_t mine = lane < E ? st.tops[lane] : 0u;
      uint32_t cnt = 0u;
      for (int j0 = 0; j0 < E; j0 += 4) {
        const uint4 q = *reinterpret_cast<const uint4*>(&st.tops[j0]);
        cnt += (q.x >= mine ? 1u : 0u) + (j0 + 1 < E && q.y >= mine ? 1u : 0u) +
               (j0 + 2 < E && q.z >= mine ? 1u : 0u) + (j0 + 3 < E && q.w >= mine ? 1u : 0u);
      }
      const uint32_t T = wave_max_u32(lane < E && cnt >= k ? mine : 0u);
      if (lane == 0) st.thr = T;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
      if (lane == 0) *(volatile lds_t<uint32_t>*)&st.thr_ready = 1u;
    }
  }

  // 2. wait for T (bounded; on a time-out every valid row is staged, a
  //    superset of the winners), then stage the rows with key >= T (one
  //    atomic per wave reserves its slots)
  uint32_t ready = 0u;
  for (int spin = 0; !stage_all && spin < kThresholdSpinMax; ++spin) {
    ready = uniform(*(volatile lds_t<uint32_t>*)&st.thr_ready);
    if (ready) break;
    __builtin_amdgcn_s_sleep(2);
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  uint32_t t = 1u;  // keeps every valid row (real keys are never 0)
  if (ready) {
    const uint32_t b = uniform(*(volatile lds_t<uint32_t>*)&st.thr);
    if (b != 0u) t = b;  // else fewer than k real tops: keep every valid row
  }
  uint64_t sv[R];
  uint32_t nsv = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    sv[r] = ballot(((valid >> r) & 1u) && key[r] >= t);
    nsv += (uint32_t)__popcll(sv[r]);
  }
  if (nsv) {
    uint32_t base = 0;
    if (lane == 0) base = atomicAdd(&st.count, nsv);
    base = readlane_u32(base, 0);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint32_t p = base + lanes_below(sv[r]);
      if (((sv[r] >> lane) & 1u) && p < kSmallSurvivorsMax) {
        st.key[p] = key[r];
        st.bits[p] = vbits[r];
        st.idx[p] = index[r];
      }
      base += (uint32_t)__popcll(sv[r]);
    }
  }
  lds_barrier();
  const uint32_t n = uniform(st.count);
  if (n > kSmallSurvivorsMax) {
    lds_barrier();  // every wave has read the count
    if (tid == 0) {
      st.count = 0u;
      st.tops_done = 0u;
      st.thr_ready = 0u;
    }
    return 0xFFFFFFFFu;
  }

  // 3. rank the staged rows and emit the first k
  rank_count(st.key, st.idx, n, st.rank);
  lds_barrier();
  for (uint32_t i = tid; i < n; i += blockDim.x) {
    const uint32_t r = st.rank[i];
    if (r < k) out(r, st.bits[i], st.idx[i]);
    st.rank[i] = 0u;
  }
  if (tid == 0) {  // every wave has read them before the barrier above
    st.count = 0u;
    st.tops_done = 0u;
    st.thr_ready = 0u;
  }
  return n < k ? n : k;
}

// select_top_small for rows 0 .. M-1 of a chunk at once (the same P and h
// for every row; from six rows on at most eight providers, with h raised to
// keep P * h >= k): the providers take their tops of every row in turn, the
// last provider of a row publishes its T, and every wave then stages each
// row's keys >= T into that row's own part of the staging, so no row waits
// for another row's barriers; the staged rows of all rows are ranked
// between the same two barriers.  The result of each row is the one
// select_top_small gives.  out(m, pos, value_bits, index) is called for
// pos < n_out[m] = min(k, valid rows); a row with more than
// kSmallSurvivorsMax staged rows writes nothing, gets n_out[m] =
// 0xFFFFFFFF and is left to the caller.  st must be as head_stage_init<true>
// leaves it and is so again on return.
template <int M, int R, typename Out>
__device__ void select_top_rows(const uint32_t (&key)[M][R], uint32_t valid,
                                const uint32_t (&vbits)[M][R], const int32_t (&index)[R],
                                uint32_t k, int P, int h, HeadStage& st, uint32_t (&n_out)[M],
                                Out&& out) {
  static_assert(M <= kMaxRows, "rows per call");
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = wave_id();
  P = uniform(P);
  h = uniform(h);
  // From six rows on the later providers' tops of every row come after the
  // youngest waves have streamed; the first eight waves alone (still
  // P * h >= k tops, at most 64) have theirs ready by then
  if (M >= 6 && P > 8) {
    P = 8;
    h = ((int)k + 7) / 8;
  }
  const bool stage_all = P == 0;

  // 1. providers: this wave's h largest keys of each row
  if (!stage_all && wave < P) {
#pragma unroll
    for (int m = 0; m < M; ++m) {
      uint32_t left = valid, top = 0u;
      for (int j = 0; j < h; ++j) {
        uint32_t best = 0u;
        int br = 0;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          if (((left >> r) & 1u) && key[m][r] > best) {
            best = key[m][r];
            br = r;
          }
        }
        const uint32_t wm = wave_max_u32(best);
        if (lane == j) top = wm;
        if (wm == 0u) break;
        const uint64_t holders = ballot(best == wm);
        if (lane == __ffsll((long long)holders) - 1) left &= ~(1u << br);
      }
      if (lane < h) st.rtops[m][wave * h + lane] = top;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
      uint32_t done = 0u;
      if (lane == 0) done = atomicAdd(&st.rtops_done[m], 1u);
      done = readlane_u32(done, 0);
      if (done == (uint32_t)P - 1u) {
        // the last provider of row m: T = the largest top with at least k
        // tops >= it
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
        const int E = P * h;  // <= 64
        const uint32_t mine = lane < E ? st.rtops[m][lane] : 0u;
        uint32_t cnt = 0u;
        for (int j0 = 0; j0 < E; j0 += 4) {
          const uint4 q = *reinterpret_cast<const uint4*>(&st.rtops[m][j0]);
          cnt += (q.x >= mine ? 1u : 0u) + (j0 + 1 < E && q.y >= mine ? 1u : 0u) +
                 (j0 + 2 < E && q.z >= mine ? 1u : 0u) + (j0 + 3 < E && q.w >= mine ? 1u : 0u);
        }
        const uint32_t T = wave_max_u32(lane < E && cnt >= k ? mine : 0u);
        if (lane == 0) st.rthr[m] = T;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
        if (lane == 0) *(volatile lds_t<uint32_t>*)&st.rthr_ready[m] = 1u;
      }
    }
  }

  // 2. each row: wait for its T (bounded, as in select_top_small), stage
  //    its keys >= T
#pragma unroll
  for (int m = 0; m < M; ++m) {
    uint32_t ready = 0u;
    for (int spin = 0; !stage_all && spin < kThresholdSpinMax; ++spin) {
      ready = uniform(*(volatile lds_t<uint32_t>*)&st.rthr_ready[m]);
      if (ready) break;
      __builtin_amdgcn_s_sleep(2);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    uint32_t t = 1u;  // keeps every valid row (real keys are never 0)
    if (ready) {
      const uint32_t b = uniform(*(volatile lds_t<uint32_t>*)&st.rthr[m]);
      if (b != 0u) t = b;
    }
    uint64_t sv[R];
    uint32_t nsv = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      sv[r] = ballot(((valid >> r) & 1u) && key[m][r] >= t);
      nsv += (uint32_t)__popcll(sv[r]);
    }
    if (nsv) {
      uint32_t base = 0;
      if (lane == 0) base = atomicAdd(&st.rcount[m], nsv);
      base = readlane_u32(base, 0);
      const uint32_t o = (uint32_t)m * kSmallSurvivorsMax;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const uint32_t p = base + lanes_below(sv[r]);
        if (((sv[r] >> lane) & 1u) && p < kSmallSurvivorsMax) {
          st.key[o + p] = key[m][r];
          st.bits[o + p] = vbits[m][r];
          st.idx[o + p] = index[r];
        }
        base += (uint32_t)__popcll(sv[r]);
      }
    }
  }
  lds_barrier();

  // 3. rank every row's staged rows, then emit each row's first k; the
  //    rows' ranking jobs, and then their entries, are dealt out to the
  //    waves (threads) as one sequence, so no wave idles while others take
  //    a job of every row
  const uint32_t nw = blockDim.x >> 6;
  uint32_t n[M];
  uint32_t jobs = 0u;  // ranking jobs of the rows before
#pragma unroll
  for (int m = 0; m < M; ++m) {
    n[m] = uniform(st.rcount[m]);
    const uint32_t o = (uint32_t)m * kSmallSurvivorsMax;
    if (n[m] <= kSmallSurvivorsMax && n[m] != 0u) {
      rank_count(st.key + o, st.idx + o, n[m], st.rank + o, ((uint32_t)wave + nw - jobs % nw) % nw, nw);
      jobs += ((n[m] + 15u) >> 4) * ((n[m] + 63u) >> 6);
    }
  }
  lds_barrier();
  uint32_t items = 0u;  // entries of the rows before
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const uint32_t o = (uint32_t)m * kSmallSurvivorsMax;
    if (n[m] <= kSmallSurvivorsMax) {
      for (uint32_t i = ((uint32_t)tid + blockDim.x - items % blockDim.x) % blockDim.x; i < n[m];
           i += blockDim.x) {
        const uint32_t r = st.rank[o + i];
        if (r < k) out(m, r, st.bits[o + i], st.idx[o + i]);
        st.rank[o + i] = 0u;
      }
      items += n[m];
      n_out[m] = n[m] < k ? n[m] : k;
    } else {
      n_out[m] = 0xFFFFFFFFu;
    }
  }
  if (tid < M) {  // every wave has read them before the barrier above
    st.rcount[tid] = 0u;
    st.rtops_done[tid] = 0u;
    st.rthr_ready[tid] = 0u;
  }
}

// LDS of the final merge: up to kMaxK entries to sort (4 slack entries so the
// rank loop can read whole uint4 words), their ranks, and two scalars.
struct alignas(16) FinalSmem {
  uint32_t key[kMaxK + 4];
  uint32_t bits[kMaxK + 4];
  int32_t idx[kMaxK + 4];
  uint32_t rank[kMaxK + 4];
  uint32_t count;   // survivors placed so far
  uint32_t bound;   // survivor threshold (a key)
  uint32_t n_over;  // chunks whose heads may not hold all their survivors
  int32_t over[256];
  uint32_t wmin[kMaxWaves];
  uint32_t wmax[kMaxWaves];
  uint32_t hist[256];  // chunk maxima per 8-bit digit
  // the row's result in output order, kept for the token draw
  // (16-byte aligned: merge_rows_grouped keeps histograms there)
  alignas(16) uint32_t out_bits[kMaxK];
  alignas(16) int32_t out_idx[kMaxK];
  uint2 lse_w[kMaxWaves];  // merge_lse: each wave's log-sum-exp pair
  // merge_rows_grouped: per group (row) its barrier counter, survivor and
  // over-chunk counts and outcome
  uint32_t g_sync[kMaxRows];
  uint32_t g_count[kMaxRows];
  uint32_t g_over[kMaxRows];
  uint32_t g_done[kMaxRows];
};

// Entries [0, n) of fs are filled, [n, 4 * ceil(n / 4)) hold padding that is
// never ahead of anything, and rank[0, n) is zero.  Each entry's output
// position is the number of entries ahead of it (greater key, or equal key
// and lower index).  The count for entry i is split over up to
// blockDim / n threads, each scanning one segment of the entries, and summed
// with LDS atomics (integer adds: the result does not depend on their order).
__device__ __forceinline__ void rank_and_write(FinalSmem& fs, uint32_t n, uint32_t k, float* values,
                               int64_t* indices) {
  if (n == 0) return;
  const uint32_t nq = (n + 3u) >> 2;
  uint32_t segs = blockDim.x / n;
  segs = segs < 1u ? 1u : (segs > nq ? nq : segs);
  const uint32_t per = (nq + segs - 1u) / segs;
  for (uint32_t t = threadIdx.x; t < n * segs; t += blockDim.x) {
    const uint32_t i = t % n;
    const uint32_t q0 = (t / n) * per;
    const uint32_t q1 = min(nq, q0 + per);
    const uint32_t ki = fs.key[i];
    const int32_t ii = fs.idx[i];
    uint32_t rank = 0;
    for (uint32_t q = q0; q < q1; ++q) {
      const uint4 kj = *reinterpret_cast<const uint4*>(&fs.key[4 * q]);
      const int4 ij = *reinterpret_cast<const int4*>(&fs.idx[4 * q]);
      rank += (kj.x > ki || (kj.x == ki && ij.x < ii)) ? 1u : 0u;
      rank += (kj.y > ki || (kj.y == ki && ij.y < ii)) ? 1u : 0u;
      rank += (kj.z > ki || (kj.z == ki && ij.z < ii)) ? 1u : 0u;
      rank += (kj.w > ki || (kj.w == ki && ij.w < ii)) ? 1u : 0u;
    }
    if (rank) atomicAdd(&fs.rank[i], rank);
  }
  lds_barrier();
  for (uint32_t i = threadIdx.x; i < n; i += blockDim.x) {
    const uint32_t rank = fs.rank[i];
    if (rank < k) {
      values[rank] = __uint_as_float(fs.bits[i]);
      indices[rank] = (int64_t)fs.idx[i];
      fs.out_bits[rank] = fs.bits[i];
      fs.out_idx[rank] = fs.idx[i];
    }
  }
}

// Digit (4 bits at `shift`, inverted so that larger keys come first) of the
// key at position p of a radix-sort pass, and the ballots that group the
// 64 positions of p's group by digit.
struct SortDigits {
  uint32_t d;       // this lane's digit
  uint64_t valid;   // lanes of the group holding an entry
  uint64_t b[4];    // lanes whose digit has bit i set
};
__device__ __forceinline__ SortDigits sort_digits(uint32_t key, bool ok, int shift) {
  SortDigits g;
  g.d = 15u - ((key >> shift) & 15u);
  g.valid = ballot(ok);
#pragma unroll
  for (int i = 0; i < 4; ++i) g.b[i] = ballot(((g.d >> i) & 1u) != 0u);
  return g;
}
// Lanes of the group whose digit is d.
__device__ __forceinline__ uint64_t sort_peers(const SortDigits& g, uint32_t d) {
  uint64_t m = g.valid;
#pragma unroll
  for (int i = 0; i < 4; ++i) m &= ((d >> i) & 1u) ? g.b[i] : ~g.b[i];
  return m;
}

// Output order of fs's n entries (1 <= n <= kMaxK, in index order) by a
// stable least-significant-digit radix sort of their keys, largest first, 4
// bits per pass over bits [0, hi_bit] (the keys agree above hi_bit; hi_bit <
// 0: all equal).  Stability keeps equal keys in index order, so the result
// is (value desc, index asc); then the first min(n, k) are written as
// rank_and_write does.  Each pass: every group of 64 positions counts its
// digits with four ballots (lanes 0-15 store the 16 counts), wave 0 turns
// the [digit][group] counts into exclusive offsets, and every entry moves to
// its digit's offset plus the number of equal digits before it in its
// group.  Linear in n, where rank_and_write's counting is quadratic.
// Scratch inside fs: out_bits is the second key buffer, out_idx the
// [16][32] count table, rank two 16-bit position buffers; fs.key is
// overwritten, fs.bits and fs.idx are kept.
__device__ void sort_and_write(FinalSmem& fs, uint32_t n, uint32_t k, int hi_bit, float* values,
                               int64_t* indices) {
  const int lane = lane_id();
  const uint32_t wave = (uint32_t)wave_id(), nw = blockDim.x >> 6;
  const uint32_t ng = (n + 63u) >> 6;  // groups of 64 positions, <= 32
  uint32_t* key_a = fs.key;
  uint32_t* key_b = fs.out_bits;
  uint16_t* pos_a = reinterpret_cast<uint16_t*>(fs.rank);
  uint16_t* pos_b = pos_a + kMaxK;
  uint32_t* tab = reinterpret_cast<uint32_t*>(fs.out_idx);
  bool first = true;  // positions are still the identity
  for (int shift = 0; shift <= hi_bit; shift += 4) {
    for (uint32_t g = wave; g < ng; g += nw) {
      const uint32_t p = g * 64u + (uint32_t)lane;
      const bool ok = p < n;
      const SortDigits sd = sort_digits(ok ? key_a[p] : 0u, ok, shift);
      if (lane < 16) tab[lane * 32 + g] = (uint32_t)__popcll(sort_peers(sd, (uint32_t)lane));
    }
    lds_barrier();
    if (wave == 0) {
      // lane L: table entries [8L, 8L + 8), i.e. digit L / 4, groups 8 (L % 4) + i
      uint32_t c[8], sum = 0u;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t g = (uint32_t)(8 * (lane & 3) + i);
        c[i] = g < ng ? tab[8 * lane + i] : 0u;
        sum += c[i];
      }
      uint32_t off = wave_scan_inclusive(sum) - sum;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        tab[8 * lane + i] = off;
        off += c[i];
      }
    }
    lds_barrier();
    for (uint32_t g = wave; g < ng; g += nw) {
      const uint32_t p = g * 64u + (uint32_t)lane;
      const bool ok = p < n;
      const uint32_t key = ok ? key_a[p] : 0u;
      const uint32_t pos = first ? p : (ok ? (uint32_t)pos_a[p] : 0u);
      const SortDigits sd = sort_digits(key, ok, shift);
      if (ok) {
        const uint32_t dst = tab[sd.d * 32u + g] + lanes_below(sort_peers(sd, sd.d));
        key_b[dst] = key;
        pos_b[dst] = (uint16_t)pos;
      }
    }
    lds_barrier();
    uint32_t* kt = key_a;
    key_a = key_b;
    key_b = kt;
    uint16_t* pt = pos_a;
    pos_a = pos_b;
    pos_b = pt;
    first = false;
  }
  const uint32_t n_out = n < k ? n : k;
  for (uint32_t r = threadIdx.x; r < n_out; r += blockDim.x) {
    const uint32_t p = first ? r : (uint32_t)pos_a[r];
    const uint32_t b = fs.bits[p];
    const int32_t ix = fs.idx[p];
    values[r] = __uint_as_float(b);
    indices[r] = (int64_t)ix;
    fs.out_bits[r] = b;  // key_a / key_b are no longer read
    fs.out_idx[r] = ix;
  }
}

// Puts this lane's entry into the survivor list if `take`: one LDS atomic per
// wave reserves the wave's slots; entries past kSurvivorsMax are counted but
// not stored (the caller then falls back).
constexpr uint32_t kSurvivorsMax = 512;

__device__ __forceinline__ void place_survivor(FinalSmem& fs, bool take, uint32_t key,
                                               uint32_t bits, int32_t ix) {
  const uint64_t b = ballot(take);
  if (b == 0u) return;
  uint32_t base = 0;
  if (lane_id() == 0) base = atomicAdd(&fs.count, (uint32_t)__popcll(b));
  base = readlane_u32(base, 0);
  const uint32_t p = base + lanes_below(b);
  if (take && p < kSurvivorsMax) {
    fs.key[p] = key;
    fs.bits[p] = bits;
    fs.idx[p] = ix;
  }
}

// Above this many selected entries the full path of a merge launch orders
// them by radix sort (linear) instead of rank counting (quadratic); the
// chunk kernels' fused merge handles k <= this and never sorts.
constexpr uint32_t kSortAbove = 256;

// Candidate p of a merge's input: in[p] (p clamped into [0, n)).
struct CandAt {
  const uint2* in;
  __device__ __forceinline__ uint2 operator()(int64_t p, int64_t n) const {
    return ld_cand(&in[p < n ? p : n - 1]);
  }
};

// merge_final's full path with R slots per thread (n_in <= R * nthreads):
// radix select over every candidate (slot order = index order), ordered
// compaction, rank and write.  at(p, n_in) gives candidate p.
template <int R, bool kSort, int NC, typename At = CandAt>
__device__ __forceinline__ void merge_full(At at, int64_t n_in, uint32_t k, float* values,
                                           int64_t* indices, int nthreads, SelectSmemT<NC>& sm,
                                           FinalSmem& fs) {
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = wave_id();
  uint32_t key[R], vb[R];
  int32_t idx[R];
  uint32_t valid = 0u;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t pos = (int64_t)(wave * R + r) * 64 + lane;
    // unconditional (clamped) loads: all R are in flight before the first
    // wait; slots past n_in are marked invalid below
    const uint2 x = at(pos, n_in);
    vb[r] = x.x;
    idx[r] = (int32_t)x.y;
    key[r] = float_key(__uint_as_float(x.x));
    valid |= (pos < n_in && idx[r] >= 0 ? 1u : 0u) << r;
  }
  const SelectRange s = block_select<R>(key, valid, k, sm);
  const uint32_t n = block_compact<R>(key, valid, s, vb, idx, sm,
                                       [&](uint32_t pos, uint32_t bits, int32_t ix) {
                                         fs.key[pos] = float_key(__uint_as_float(bits));
                                         fs.bits[pos] = bits;
                                         fs.idx[pos] = ix;
                                       });
  if (kSort && n > kSortAbove) {
    // the selected keys lie in [s.prefix, s.kmax], so they agree above the
    // highest bit in which those two differ
    const uint32_t span = s.prefix ^ s.kmax;
    lds_barrier();
    sort_and_write(fs, n, k, span ? 31 - __clz(span) : -1, values, indices);
    return;
  }
  for (uint32_t i = n + tid; i < ((n + 3u) & ~3u); i += nthreads) {
    fs.key[i] = 0u;
    fs.idx[i] = 0x7FFFFFFF;
  }
  lds_barrier();
  rank_and_write(fs, n, k, values, indices);
}

// Whether merge_final takes its bounded path for these sizes (with nthreads
// threads, one head each).
__device__ __forceinline__ bool merge_bounded(const uint2* heads, int n_max, uint32_t k, int nthreads) {
  return heads != nullptr && n_max >= (int)k && n_max <= 256 && n_max * kHeads <= nthreads;
}

// Barrier of the `waves` waves of one group (not the whole workgroup): each
// wave counts itself on the group's LDS counter and waits until the count
// reaches target + waves (bounded, as every wait here; the waves of a
// workgroup are all resident, so the count always gets there).
__device__ __forceinline__ void group_sync(uint32_t* ctr, uint32_t waves, uint32_t& target) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  target += waves;
  if (lane_id() == 0) atomicAdd(ctr, 1u);
  for (int spin = 0; spin < kThresholdSpinMax; ++spin) {
    if (uniform(*(volatile lds_t<uint32_t>*)ctr) >= target) break;
    __builtin_amdgcn_s_sleep(1);
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// merge_final's bounded path for rows 0 .. M-1 at once: row g is merged by
// waves [g G, (g + 1) G) with barriers of their own (group_sync), so the
// rows' merges overlap instead of following one another.  Same T,
// survivors, ranks and outputs as merge_final; a group's LDS is the part g
// of fs's arrays (survivors: 256 entries of key .. rank, maxima histogram:
// out_bits, over-chunk list: out_idx).  Requires merge_bounded() for the
// sizes and M * G <= waves.  Row g's outcome is fs.g_done[g] = 1 when
// written, 0 when it has more than 256 survivors (the caller then merges it
// with merge_final); ordered by the caller's next workgroup barrier.
constexpr uint32_t kGroupSurvivors = 256;
template <int M, int G>
__device__ void merge_rows_grouped(const uint2* cand, int64_t n_in, const uint2* heads, int n_max, int kc,
                                   uint32_t k, float* values, int64_t* indices, FinalSmem& fs) {
  static_assert(M * G <= kMaxWaves && G >= 2 && M * kGroupSurvivors <= kMaxK, "groups");
  constexpr int S = 64 * G;  // threads per group
  constexpr int J = (kMaxWaves * kHeads * 16 + S - 1) / S;  // heads per thread (n_heads <= 1024)
  const int wave = wave_id();
  const int lane = lane_id();
  const int g = wave / G;
  if (g >= M) return;
  const int gw = wave - g * G;
  const int t = gw * 64 + lane;
  const int n_heads = n_max * kHeads;
  const uint2* hrow = heads + (size_t)g * n_heads;
  const uint2* crow = cand + (size_t)g * n_in;
  uint32_t* skey = fs.key + g * kGroupSurvivors;
  uint32_t* sbits = fs.bits + g * kGroupSurvivors;
  int32_t* sidx = fs.idx + g * kGroupSurvivors;
  uint32_t* srank = fs.rank + g * kGroupSurvivors;
  uint32_t* hist = fs.out_bits + g * 256;
  int32_t* over_list = fs.out_idx + g * 256;
  uint32_t* ctr = &fs.g_sync[g];
  uint32_t target = 0u;

  // every head of the row, J per thread (head e = t + j S; the four heads of
  // a chunk sit in one quad of lanes), all loads in flight at once
  uint32_t hb[J];
  int32_t hx[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int e = t + j * S;
    const uint2 x = ld_cand(&hrow[e < n_heads ? e : n_heads - 1]);
    hb[j] = x.x;
    hx[j] = e < n_heads ? (int32_t)x.y : -1;
  }
  for (int i = t; i < 256; i += S) hist[i] = 0u;
  for (int i = t; i < (int)kGroupSurvivors; i += S) srank[i] = 0u;
  if (t == 0) {
    fs.g_count[g] = 0u;
    fs.g_over[g] = 0u;
  }
  // the chunk maxima (first lane of each quad): shared high bits
  const bool q0 = (lane & 3) == 0;
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    if (q0 && hx[j] >= 0) {
      const uint32_t kj = float_key(__uint_as_float(hb[j]));
      lo = min(lo, kj);
      hi = max(hi, kj);
    }
  }
  lo = wave_min_u32(lo);
  hi = wave_max_u32(hi);
  if (lane == 0) {
    fs.wmin[wave] = lo;
    fs.wmax[wave] = hi;
  }
  group_sync(ctr, G, target);
  const uint32_t gmin = wave_min_u32(lane < G ? fs.wmin[g * G + lane] : 0xFFFFFFFFu);
  const uint32_t gmax = wave_max_u32(lane < G ? fs.wmax[g * G + lane] : 0u);
  // T as merge_final finds it: one histogram of the maxima's next 8 bits
  uint32_t t_key = gmin;
  if (gmin != gmax) {
    const int top = 31 - __clz(gmin ^ gmax);
    const int shift = top >= 7 ? top - 7 : 0;
#pragma unroll
    for (int j = 0; j < J; ++j)
      if (q0 && hx[j] >= 0) atomicAdd(&hist[(float_key(__uint_as_float(hb[j])) >> shift) & 0xFFu], 1u);
    group_sync(ctr, G, target);
    const uint4 h = *reinterpret_cast<const uint4*>(&hist[4 * lane]);
    const uint32_t s3 = h.w, s2 = h.z + s3, s1 = h.y + s2, s0 = h.x + s1;
    const uint32_t incl = wave_scan_inclusive(s0);
    const uint32_t after = readlane_u32(incl, 63) - incl;
    const uint64_t have = ballot(s0 + after >= k);
    const int L = 63 - __clzll(have);
    const uint32_t i_star = s3 + after >= k ? 3u : s2 + after >= k ? 2u : s1 + after >= k ? 1u : 0u;
    const uint32_t digit = 4u * (uint32_t)L + readlane_u32(i_star, L);
    const uint32_t low = shift + 8 >= 32 ? 0xFFFFFFFFu : (1u << (shift + 8)) - 1u;
    t_key = (gmax & ~low) | (digit << shift);
  }
  // survivors: heads >= T of chunks whose last head is below T; the other
  // chunks ("over") may hold survivors beyond their heads
  auto place = [&](bool take, uint32_t kx, uint32_t bits, int32_t ix) {
    const uint64_t b = ballot(take);
    if (b == 0u) return;
    uint32_t base = 0;
    if (lane == 0) base = atomicAdd(&fs.g_count[g], (uint32_t)__popcll(b));
    base = readlane_u32(base, 0);
    const uint32_t p = base + lanes_below(b);
    if (take && p < kGroupSurvivors) {
      skey[p] = kx;
      sbits[p] = bits;
      sidx[p] = ix;
    }
  };
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const uint32_t kj = float_key(__uint_as_float(hb[j]));
    const uint32_t last_in = (lane & 3) == 3 && kc > kHeads && hx[j] >= 0 && kj >= t_key ? 1u : 0u;
    const bool over = dpp<kQuadBcast3>(0u, last_in) != 0u;
    place(hx[j] >= 0 && !over && kj >= t_key, kj, hb[j], hx[j]);
    const uint64_t bo = ballot(q0 && over);
    if (bo != 0u) {
      uint32_t base = 0;
      if (lane == 0) base = atomicAdd(&fs.g_over[g], (uint32_t)__popcll(bo));
      base = readlane_u32(base, 0);
      if (q0 && over) over_list[base + lanes_below(bo)] = (t + j * S) >> 2;
    }
  }
  group_sync(ctr, G, target);
  const uint32_t n_over = uniform(fs.g_over[g]);
  if (n_over) {  // rare: those chunks' candidate lists in full
    const uint32_t total = n_over * (uint32_t)kc;
    for (uint32_t base = 0; base < total; base += S) {
      const uint32_t i = base + (uint32_t)t;
      bool take = false;
      uint2 x = make_uint2(0u, 0xFFFFFFFFu);
      uint32_t kx = 0u;
      if (i < total) {
        x = ld_cand(&crow[(int64_t)over_list[i / (uint32_t)kc] * kc + i % (uint32_t)kc]);
        kx = float_key(__uint_as_float(x.x));
        take = (int32_t)x.y >= 0 && kx >= t_key;
      }
      place(take, kx, x.x, (int32_t)x.y);
    }
    group_sync(ctr, G, target);
  }
  const uint32_t n = uniform(fs.g_count[g]);
  if (n > kGroupSurvivors) {
    if (t == 0) fs.g_done[g] = 0u;
    return;
  }
  rank_count(skey, sidx, n, srank, (uint32_t)gw, (uint32_t)G);
  group_sync(ctr, G, target);
  float* vo = values + (size_t)g * k;
  int64_t* io = indices + (size_t)g * k;
  for (uint32_t i = t; i < n; i += S) {
    const uint32_t r = srank[i];
    if (r < k) {
      vo[r] = __uint_as_float(sbits[i]);
      io[r] = (int64_t)sidx[i];
    }
  }
  if (t == 0) fs.g_done[g] = 1u;
}

// Final merge of one row.  `in` holds the n_in candidates of the n_max chunks
// (kc per chunk, fp32 value bits and int32 index, index -1 = padding) in
// ascending index order; RM slots per thread cover them (n_in <=
// blockDim.x * RM).  `heads` (optional) holds each chunk's kHeads best
// candidates in output order.  Writes the exact top-k sorted by (value desc,
// index asc) to values / indices, and keeps it in fs.out_bits / fs.out_idx
// for the token draw (ordered by the caller's next barrier).  kSort (merge
// launches): the full path orders more than kSortAbove selected entries by
// radix sort; without it (the chunk kernels' fused merge, k <= kSortAbove)
// always by rank counting.
//
// Bounded path: a threshold T with at least k chunk maxima >= T is at most
// the row's k-th largest value (those maxima are k distinct logits), so only
// candidates with key >= T can be in the result.  Wave 0 finds T from the
// heads' first entries.  A chunk whose last head is below T has all its
// survivors among its heads; the few other chunks (typically none) are read
// in full.  The survivors (typically a few dozen) go to LDS in any order and
// are ranked there.  With too many chunks or survivors, the radix select of
// all candidates runs instead.
template <int RM, bool kSort, int NC>
__device__ __forceinline__ void merge_final(const uint2* in, int64_t n_in, const uint2* heads, int n_max, int kc,
                            uint32_t k, float* values, int64_t* indices, int nthreads,
                            SelectSmemT<NC>& sm, FinalSmem& fs) {
  // nthreads == blockDim.x, passed in so that no load of it queues behind
  // the data loads
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = wave_id();
  const int n_heads = n_max * kHeads;

  for (int i = tid; i < kMaxK + 4; i += nthreads) fs.rank[i] = 0u;

  if (heads != nullptr && n_max >= (int)k && n_max <= 256 && n_heads <= nthreads) {
    // Every thread below n_heads loads one head and, for the first head of a
    // chunk, that chunk's last head, so all loads are in flight at once;
    // thread 4c holds chunk c's maximum.
    const int e = min(tid, n_heads - 1);
    const int c = e / kHeads;
    const uint2 absent = make_uint2(0u, 0xFFFFFFFFu);
    const uint2 he = tid < n_heads ? ld_cand(&heads[e]) : absent;
    const uint2 hl = tid < n_heads && e == c * kHeads ? ld_cand(&heads[(size_t)c * kHeads + (kHeads - 1)])
                                                        : absent;
    for (int i = tid; i < (int)kSurvivorsMax + 4; i += nthreads) {
      fs.key[i] = 0u;  // padding: below every real key
      fs.idx[i] = 0x7FFFFFFF;
    }
    for (int i = tid; i < 256; i += nthreads) fs.hist[i] = 0u;
    if (tid == 0) {
      fs.count = 0u;
      fs.n_over = 0u;
    }
    const uint32_t key = float_key(__uint_as_float(he.x));
    const bool is_max = tid < n_heads && (tid % kHeads) == 0 && (int32_t)he.y >= 0;
    {
      const uint32_t lo = wave_min_u32(is_max ? key : 0xFFFFFFFFu);
      const uint32_t hi = wave_max_u32(is_max ? key : 0u);
      if (lane == 0) {
        fs.wmin[wave] = lo;
        fs.wmax[wave] = hi;
      }
    }
    lds_barrier();
    // T: the maxima share the bits above their highest differing bit; one
    // histogram over the next 8 bits finds the digit d such that at least k
    // maxima have digit >= d, and T = (shared bits, d, zeros) is at most the
    // k-th largest maximum, hence at most the row's k-th largest value
    // (those maxima are k distinct logits).
    const int nw = nthreads >> 6;
    const uint32_t gmin = wave_min_u32(lane < nw ? fs.wmin[lane] : 0xFFFFFFFFu);
    const uint32_t gmax = wave_max_u32(lane < nw ? fs.wmax[lane] : 0u);
    int shift = 0;
    if (gmin != gmax) {
      const int top = 31 - __clz(gmin ^ gmax);
      shift = top >= 7 ? top - 7 : 0;
      if (is_max) atomicAdd(&fs.hist[(key >> shift) & 0xFFu], 1u);
    }
    lds_barrier();
    uint32_t t = gmin;  // all maxima equal: every one is >= T
    if (gmin != gmax) {
      const uint4 h = *reinterpret_cast<const uint4*>(&fs.hist[4 * lane]);
      const uint32_t s3 = h.w, s2 = h.z + s3, s1 = h.y + s2, s0 = h.x + s1;
      const uint32_t incl = wave_scan_inclusive(s0);
      const uint32_t after = readlane_u32(incl, 63) - incl;  // maxima in the digits of higher lanes
      const uint64_t have = ballot(s0 + after >= k);
      const int L = 63 - __clzll(have);
      const uint32_t i_star = s3 + after >= k ? 3u : s2 + after >= k ? 2u : s1 + after >= k ? 1u : 0u;
      const uint32_t digit = 4u * (uint32_t)L + readlane_u32(i_star, L);
      const uint32_t low = shift + 8 >= 32 ? 0xFFFFFFFFu : (1u << (shift + 8)) - 1u;
      t = (gmax & ~low) | (digit << shift);
    }
    const bool mine = tid < n_heads && (int32_t)he.y >= 0;
    // a chunk with more candidates than heads may hold survivors beyond them
    // (decided by the chunk's first head thread, which holds the last head,
    // and passed to the other three threads of the chunk: one quad of lanes)
    const uint32_t over0 =
        kc > kHeads && (int32_t)hl.y >= 0 && float_key(__uint_as_float(hl.x)) >= t ? 1u : 0u;
    static_assert(kHeads == 4, "one chunk's heads are one quad of lanes");
    const bool over = dpp<kQuadBcast0>(0u, over0) != 0u;
    place_survivor(fs, mine && !over && key >= t, key, he.x, (int32_t)he.y);
    if (tid < n_heads && over && e == c * kHeads) fs.over[atomicAdd(&fs.n_over, 1u)] = c;
    lds_barrier();
    const uint32_t n_over = uniform(fs.n_over);
    if (n_over) {  // rare: read those chunks' candidate lists in full
      const int64_t total = (int64_t)n_over * kc;
      for (int64_t base = 0; base < total; base += nthreads) {
        const int64_t j = base + tid;
        bool take = false;
        uint2 x = make_uint2(0u, 0xFFFFFFFFu);
        uint32_t kx = 0u;
        if (j < total) {
          x = ld_cand(&in[(int64_t)fs.over[j / kc] * kc + j % kc]);
          kx = float_key(__uint_as_float(x.x));
          take = (int32_t)x.y >= 0 && kx >= t;
        }
        place_survivor(fs, take, kx, x.x, (int32_t)x.y);
      }
      lds_barrier();
    }
    const uint32_t n = uniform(fs.count);
    if (n <= kSurvivorsMax) {
      rank_count(fs.key, fs.idx, n, fs.rank);
      lds_barrier();
      for (uint32_t i = tid; i < n; i += nthreads) {
        const uint32_t r = fs.rank[i];
        if (r < k) {
          values[r] = __uint_as_float(fs.bits[i]);
          indices[r] = (int64_t)fs.idx[i];
          fs.out_bits[r] = fs.bits[i];
          fs.out_idx[r] = fs.idx[i];
        }
      }
      return;
    }
  }

  // Full path: radix select over every candidate (slot order = index order),
  // ordered compaction, rank; with R slots per thread, the fewest that hold
  // the candidates (slot order is position order, so with too many slots per
  // thread a few candidates would all fall to the first wave).  The smaller
  // forms are marked unlikely so that the compiler places them out of line.
  if (__builtin_expect(RM > 1 && n_in <= (int64_t)nthreads, 0)) {
    merge_full<1, kSort>(CandAt{in}, n_in, k, values, indices, nthreads, sm, fs);
  } else if (__builtin_expect(RM > 4 && n_in <= (int64_t)4 * nthreads, 0)) {
    merge_full<4, kSort>(CandAt{in}, n_in, k, values, indices, nthreads, sm, fs);
  } else {
    merge_full<RM, kSort>(CandAt{in}, n_in, k, values, indices, nthreads, sm, fs);
  }
}

// Log-sum-exp pairs (Selective Log Softmax page, section "Kernel design":
// per-slice maxima and sums of exponentials, combined).  A pair (m, s)
// stands for m + log(s): m the largest logit of a slice and s the sum of
// exp(logit - m) over it; (-inf, 0) is an empty slice (or one of -inf
// logits only) and (+inf, 1) a slice with an +inf logit.  Pairs combine as
// (M, sum of s_i exp(m_i - M)), M the largest m_i: M is +inf or -inf for
// the whole set when it is for the result.
//
// Combines the pairs held by the lanes of one wave (absent lanes hold
// (-inf, 0)) into the pair every lane returns: the wave's maximum, then
// the wave's sum of the rescaled s (fixed reduction orders).
__device__ __forceinline__ void lse_combine_wave(float& m, float& s) {
  const float M = wave_max_f32(m);
  float t = 0.f;
  if (M == INFINITY) t = m == INFINITY ? 1.f : 0.f;  // one +inf slice counts once
  else if (M != -INFINITY && m != -INFINITY) t = s * expf(m - M);
  s = wave_sum_f32(t);
  if (M == INFINITY) s = 1.f;
  m = M;
}

// Log-sum-exp of one row from part[0, n), one pair per chunk of the row,
// written to *out (unless out is null) and returned to the threads named
// below when `want` (else 0).  The maximum M over the pairs, then the sum of
// s * exp(m - M), each in a fixed order.
//   mode 1 (n <= 64 * kLsePairs): wave 0 alone, from the pairs it preloaded
//     (lane l: pairs l + 64 j); no barrier; the result goes to wave 0.
//   mode 2 (n <= kLsePairs * threads): every thread from its preloaded pairs
//     (i = thread + j * threads), each wave, then every wave over the
//     waves' values in fs.lse_w; two barriers; the result goes to all.
//   mode 0: as mode 2, with the pairs read here.
// Called by the whole workgroup; fs.lse_w is not written again before the
// caller's next barrier.  Preloading (load_lse_pairs) lets the pairs' round
// trip overlap the merge.
constexpr int kLsePairs = 4;
__device__ __forceinline__ int load_lse_pairs(const uint2* part, int n, uint2 (&p)[kLsePairs]) {
  const int mode = n <= 64 * kLsePairs ? 1 : n <= kLsePairs * (int)blockDim.x ? 2 : 0;
  const bool mine = mode == 2 || (mode == 1 && wave_id() == 0);
  const int step = mode == 1 ? 64 : (int)blockDim.x;
#pragma unroll
  for (int j = 0; j < kLsePairs; ++j) {
    const int i = (int)threadIdx.x + j * step;
    p[j] = mine && i < n ? ld_cand(&part[i]) : make_uint2(__float_as_uint(-INFINITY), 0u);
  }
  return mode;
}

// Mode 1 by any one wave: lane l holds the pairs l + 64 j of the row (absent
// ones (-inf, 0)); every lane of the wave returns the result and lane 0
// stores it to *out (unless out is null).
__device__ __forceinline__ float lse_wave(const uint2 (&pre)[kLsePairs], float* out) {
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < kLsePairs; ++j) mx = fmaxf(mx, __uint_as_float(pre[j].x));
  const float M = wave_max_f32(mx);
  float sum = 0.f;
  if (M != INFINITY && M != -INFINITY) {
#pragma unroll
    for (int j = 0; j < kLsePairs; ++j) {
      const float pm = __uint_as_float(pre[j].x);
      if (pm != -INFINITY) sum += __uint_as_float(pre[j].y) * expf(pm - M);
    }
  }
  const float S = wave_sum_f32(sum);
  const float r = M == INFINITY ? INFINITY : M == -INFINITY ? -INFINITY : M + logf(S);
  if (lane_id() == 0 && out != nullptr) *out = r;
  return r;
}
// The row's pairs for lse_wave, requested by the waves with `mine` set
// (n <= 64 * kLsePairs).
__device__ __forceinline__ void load_lse_pairs_wave(const uint2* part, int n, bool mine,
                                                    uint2 (&p)[kLsePairs]) {
#pragma unroll
  for (int j = 0; j < kLsePairs; ++j) {
    const int i = lane_id() + j * 64;
    p[j] = mine && i < n ? ld_cand(&part[i]) : make_uint2(__float_as_uint(-INFINITY), 0u);
  }
}

__device__ __forceinline__ float merge_lse(const uint2* part, int n, float* out, FinalSmem& fs,
                                          int mode, const uint2 (&pre)[kLsePairs],
                                          bool want = true) {
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = wave_id();
  const int nw = blockDim.x >> 6;
  if (mode == 1) {
    if (wave != 0) return 0.f;
    const float r = lse_wave(pre, out);
    return want ? r : 0.f;
  }
  const bool have = mode != 0;
  // 1. the row's maximum M
  float mx = -INFINITY;
  if (have) {
#pragma unroll
    for (int j = 0; j < kLsePairs; ++j) mx = fmaxf(mx, __uint_as_float(pre[j].x));
  } else {
    for (int i = tid; i < n; i += (int)blockDim.x) mx = fmaxf(mx, __uint_as_float(ld_cand(&part[i]).x));
  }
  mx = wave_max_f32(mx);
  if (lane == 0) fs.lse_w[wave].x = __float_as_uint(mx);
  lds_barrier();
  const float M = wave_max_f32(lane < nw ? __uint_as_float(fs.lse_w[lane].x) : -INFINITY);
  // 2. the sum of s * exp(m - M)
  float sum = 0.f;
  if (M != INFINITY && M != -INFINITY) {
    auto add = [&](const uint2& p) {
      const float pm = __uint_as_float(p.x);
      if (pm != -INFINITY) sum += __uint_as_float(p.y) * expf(pm - M);
    };
    if (have) {
#pragma unroll
      for (int j = 0; j < kLsePairs; ++j) add(pre[j]);
    } else {
      for (int i = tid; i < n; i += (int)blockDim.x) add(ld_cand(&part[i]));
    }
  }
  sum = wave_sum_f32(sum);
  if (lane == 0) fs.lse_w[wave].y = __float_as_uint(sum);
  lds_barrier();
  const float S = wave_sum_f32(lane < nw ? __uint_as_float(fs.lse_w[lane].y) : 0.f);
  const float r = M == INFINITY ? INFINITY : M == -INFINITY ? -INFINITY : M + logf(S);
  if (tid == 0 && out != nullptr) *out = r;
  return want ? r : 0.f;
}

}  // namespace lmtopk
