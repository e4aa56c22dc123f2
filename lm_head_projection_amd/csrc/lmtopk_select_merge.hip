// lmtopk_select_merge.hip - pack, selection-only and merge kernels (gfx950).
//
//   k_pack          pack a dense fp32/bf16 head into signs + group scales
//                   (lm-head-topk page, sections "Usage" and "Requirements and
//                   limits": binary weights are packed offline)
//   k_select_chunk  the chunk selection fed from fp32 logits in memory
//   k_merge         merges chunk candidates into the final sorted top-k
//                   (section "Method", second pass), or into a smaller
//                   candidate set when one workgroup cannot hold them all;
//                   used when the chunk launch cannot merge in its last
//                   workgroup
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

#include "lmtopk_chunk.hpp"

namespace lmtopk {

constexpr int kGroup = 128;

// One wave per (64-row tile, quad of groups): lane r owns row 64 t + r and
// reads its 4 x 128 weights itself (each lane a contiguous 512 B or 256 B),
// so signs and the fp64 |w| sums need no cross-lane traffic.  Writes are one
// uint4 of sign words per group and one float4 of scales per lane, coalesced
// across the wave.
template <bool BF16>
__global__ __launch_bounds__(256) void k_pack(const void* __restrict__ w, int64_t V, int64_t H,
                                              int64_t n_tiles, uint4* __restrict__ wq,
                                              float4* __restrict__ wscale) {
  const int lane = lane_id();
  const int64_t wave_id = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const int G = (int)(H / kGroup);
  const int Q = (G + 3) / 4;
  if (wave_id >= n_tiles * Q) return;
  const int64_t t = wave_id / Q;
  const int q = (int)(wave_id - t * Q);
  const int64_t v = t * 64 + lane;
  const bool row_ok = v < V;
  float sc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int g = 4 * q + i;
    if (g >= G) break;
    uint32_t word[4] = {0u, 0u, 0u, 0u};
    double s = 0.0;
    if (row_ok) {
      if (BF16) {
        const uint4* src = reinterpret_cast<const uint4*>(
            static_cast<const uint16_t*>(w) + v * H + (int64_t)g * kGroup);
#pragma unroll
        for (int c = 0; c < 16; ++c) {  // 16 x 8 bf16
          const uint4 x = src[c];
          const uint32_t part[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t hbits = (part[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu;
            const float f = __uint_as_float(hbits << 16);
            const int j = c * 8 + e;
            word[j >> 5] |= (f >= 0.f ? 1u : 0u) << (j & 31);
            s += (double)fabsf(f);
          }
        }
      } else {
        const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(w) + v * H +
                                                            (int64_t)g * kGroup);
#pragma unroll
        for (int c = 0; c < 32; ++c) {  // 32 x 4 fp32
          const float4 x = src[c];
          const float f4[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int j = c * 4 + e;
            word[j >> 5] |= (f4[e] >= 0.f ? 1u : 0u) << (j & 31);
            s += (double)fabsf(f4[e]);
          }
        }
      }
      sc[i] = (float)(s / 128.0);
    }
    wq[((size_t)t * G + g) * 64 + lane] = make_uint4(word[0], word[1], word[2], word[3]);
  }
  wscale[((size_t)t * Q + q) * 64 + lane] = make_float4(sc[0], sc[1], sc[2], sc[3]);
}
// ---------------------------------------------------------------------------
// selection-only chunk kernel (scores read from fp32 logits)
// ---------------------------------------------------------------------------
struct SelectArgs {
  const float* logits;  // [M][ld]
  int64_t M, V, ld;
  int chunk_rows;
  ChunkOut out;
};

template <int RPL>
__global__ __launch_bounds__(1024) void k_select_chunk(SelectArgs a) {
  __shared__ SelectSmem ssm;
  __shared__ ChunkSmem csm;
  __shared__ uint32_t last_wg;
  HeadStage& hst = csm.hs;
  head_stage_init(hst);
  lds_barrier();  // the selection writes LDS before its first barrier
  const int wave = wave_id();
  const int lane = lane_id();
  const int64_t base = (int64_t)blockIdx.x * a.chunk_rows;
  // lane m: row m's temperature (the draw's logit scale for the normaliser)
  const float temp_v = row_temperature(a.out, lane < (int)a.M ? lane : (int)a.M - 1, a.logits);
  int32_t idx[RPL];
  uint32_t valid = 0u;
#pragma unroll
  for (int r = 0; r < RPL; ++r) {
    const int64_t v = base + (wave * RPL + r) * 64 + lane;
    idx[r] = (int32_t)v;
    valid |= (v < a.V ? 1u : 0u) << r;
  }
  for (int m = 0; m < (int)a.M; ++m) {
    const float* row = a.logits + (size_t)m * a.ld;
    float val[RPL];
#pragma unroll
    for (int r = 0; r < RPL; ++r) val[r] = ((valid >> r) & 1u) ? ld_stream(&row[idx[r]]) : 0.f;
    int64_t rows[RPL];
#pragma unroll
    for (int r = 0; r < RPL; ++r) rows[r] = ((valid >> r) & 1u) ? (int64_t)idx[r] : 0;
    const uint32_t allow = allowed_bits<RPL>(a.out, m, rows, a.logits);
    const float zs = z_scale(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(temp_v), m)));
    chunk_select_write<RPL>(val, idx, valid, m, a.out, ssm, hst, m == (int)a.M - 1, allow, zs);
  }
  if (a.out.fused) fused_merge_tail<kFusedRM>(fused_merge_of(a.out), ssm, csm.fs, last_wg);
}
// ---------------------------------------------------------------------------
// merge
// ---------------------------------------------------------------------------
struct MergeArgs {
  const uint2* in;  // [M][n_in] candidates, ascending index within each row
  const uint2* heads;  // [M][n_max][kHeads] chunk heads, or null
  int n_max;           // chunks
  int kc;              // candidates per chunk
  int64_t n_in;
  int k;
  int threads;      // blockDim.x
  int n_seg;        // segments per row; blockIdx.x = segment, blockIdx.y = row
  int64_t seg;      // candidates per segment
  uint2* out;       // intermediate: [M][n_seg][k]
  float* values;    // final: [M][k]
  int64_t* indices; // final: [M][k]
  const uint2* lse_part;  // final: log-sum-exp pairs [M][n_part] (one per chunk), or null
  int n_part;
  float* lse;             // final: [M] or null
  SampleParams smp;       // final: the token draw (smp.on == 0: none)
  const uint32_t* hist;   // first of several levels: the rows' key histograms
                          // [M][kHistBins] (k_hist), or null
  uint32_t* hist_clear;   // last of several levels: the same, set back to zero
  uint32_t* counts;       // first of two levels: its output count per row and
                          // segment [M][n_seg] (then it writes no padding), or null
  const uint32_t* in_counts;  // last of two levels: those counts, or null
  int in_seg;                 // ... and the first level's segments (<= kGatherSegs)
};

// Candidate p of the concatenation of the first level's outputs, segment s
// holding its count[s] selected candidates at in[s * k]: seg_off (in LDS)
// holds the exclusive prefix of the counts, n_seg + 1 entries.
struct GatherAt {
  const uint2* in;
  const lds_t<uint32_t>* seg_off;
  int n_seg;
  int k;
  __device__ __forceinline__ uint2 operator()(int64_t p, int64_t n) const {
    const uint32_t q = (uint32_t)(p < n ? p : n - 1);
    int lo = 0, hi = n_seg - 1;  // the last segment starting at or before q
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (seg_off[mid] <= q) lo = mid;
      else hi = mid - 1;
    }
    return ld_cand(&in[(size_t)lo * k + (q - seg_off[lo])]);
  }
};

// Counts of the top 11 bits of the candidates' keys, per row (grid: x = a
// span of kHistSpan candidates, y = row), added into hist [M][kHistBins],
// which is zero on entry.  Padding (index -1) is not counted.
constexpr int kHistSpan = 4096;
__global__ __launch_bounds__(1024) void k_hist(const uint2* __restrict__ in, int64_t n_in,
                                               uint32_t* __restrict__ hist) {
  __shared__ uint32_t h[kHistBins];
  const int tid = threadIdx.x;
  for (int i = tid; i < kHistBins; i += blockDim.x) h[i] = 0u;
  lds_barrier();
  const uint2* row = in + (size_t)blockIdx.y * n_in;
  const int64_t base = (int64_t)blockIdx.x * kHistSpan;
  for (int i = tid; i < kHistSpan; i += blockDim.x) {
    const int64_t pos = base + i;
    if (pos < n_in) {
      const uint2 x = row[pos];
      if ((int32_t)x.y >= 0) atomicAdd(&h[float_key(__uint_as_float(x.x)) >> 21], 1u);
    }
  }
  lds_barrier();
  uint32_t* out = hist + (size_t)blockIdx.y * kHistBins;
  for (int i = tid; i < kHistBins; i += blockDim.x)
    if (h[i] != 0u) atomicAdd(&out[i], h[i]);
}

// The bin of a row's k-th largest key from its histogram: the largest bin b
// with at least k counted keys in bins >= b (every key of the top k has bin
// >= b).  Wave 0 finds it from q, its lane l's bins 32 l .. 32 l + 31 (as
// kth_bin_load reads them), and posts it in *bin; the caller orders it with
// a barrier.
struct HistSlice {
  uint4 q[8];
};
__device__ __forceinline__ HistSlice kth_bin_load(const uint32_t* hist) {
  HistSlice h;
  const uint4* p = reinterpret_cast<const uint4*>(hist + 32 * lane_id());
#pragma unroll
  for (int j = 0; j < 8; ++j) h.q[j] = p[j];
  return h;
}
__device__ __forceinline__ void kth_bin(const HistSlice& h, uint32_t k, uint32_t* bin) {
  const int lane = lane_id();
  uint32_t c[32];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    c[4 * j] = h.q[j].x;
    c[4 * j + 1] = h.q[j].y;
    c[4 * j + 2] = h.q[j].z;
    c[4 * j + 3] = h.q[j].w;
  }
  uint32_t sum = 0u;
#pragma unroll
  for (int j = 0; j < 32; ++j) sum += c[j];
  const uint32_t incl = wave_scan_inclusive(sum);
  const uint32_t above = readlane_u32(incl, 63) - incl;  // keys in the lanes above
  // the lane whose bins hold the k-th largest: the highest lane with
  // above + sum >= k (at least k keys in total, or bin 0)
  const uint64_t have = ballot(above + sum >= k);
  const int L = have ? 63 - __clzll(have) : 0;
  if (lane == L) {
    uint32_t acc = above;
    uint32_t b = 32u * (uint32_t)lane;
#pragma unroll
    for (int j = 31; j >= 0; --j) {
      acc += c[j];
      if (acc >= k) {
        b = 32u * (uint32_t)lane + (uint32_t)j;
        break;
      }
    }
    *bin = b;
  }
}

// Workgroup (segment s, row m) takes candidates [s*seg, (s+1)*seg) of row m,
// RM slots per thread (slot order = candidate order = index order), selects
// their exact top-k and either writes them in index order (intermediate
// level) or sorts them by (value desc, index asc) -- by rank counting (each
// entry's output position is the number of entries ahead of it) for up to
// 256 of them, else by a stable radix sort -- and writes values / indices
// (final level).  Its selection uses four copies of each histogram.
template <int RM>
__global__ __launch_bounds__(1024) void k_merge(MergeArgs a) {
  __shared__ MergeSelectSmem ssm;
  const int m = blockIdx.y;
  const uint2* in = a.in + (size_t)m * a.n_in;
  if (a.n_seg == 1) {
    __shared__ FinalSmem fs;
    if (a.hist_clear != nullptr) {  // the first level has read the counts
      uint4* h = reinterpret_cast<uint4*>(a.hist_clear + (size_t)m * kHistBins);
      for (int i = threadIdx.x; i < kHistBins / 4; i += blockDim.x) h[i] = make_uint4(0u, 0u, 0u, 0u);
    }
    uint2 pre[kLsePairs];
    int have = 0;
    if (a.lse_part != nullptr) have = load_lse_pairs(a.lse_part + (size_t)m * a.n_part, a.n_part, pre);
    RowSample rs;
    if (a.smp.on) rs = load_row_sample(a.smp, m);
    // after two levels, the first level's selected candidates alone,
    // gathered in segment order (index order), when they fit 4 slots per
    // thread; else the padded segments
    __shared__ uint32_t seg_off[kGatherSegs + 1];
    int64_t total = -1;
    if (a.in_counts != nullptr) {
      if (wave_id() == 0) {
        const int lane = lane_id();
        const uint32_t c = lane < a.in_seg ? a.in_counts[(size_t)m * a.in_seg + lane] : 0u;
        const uint32_t incl = wave_scan_inclusive(c);
        seg_off[lane + 1] = incl;
        if (lane == 0) seg_off[0] = 0u;
      }
      lds_barrier();
      total = (int64_t)uniform(seg_off[a.in_seg]);
    }
    if (total >= 0 && total <= (int64_t)4 * a.threads) {
      const GatherAt at{in, (const lds_t<uint32_t>*)seg_off, a.in_seg, a.k};
      float* vo = a.values + (size_t)m * a.k;
      int64_t* io = a.indices + (size_t)m * a.k;
      for (int i = threadIdx.x; i < kMaxK + 4; i += blockDim.x) fs.rank[i] = 0u;
      if (RM == 1 || total <= (int64_t)a.threads)
        merge_full<1, true>(at, total, (uint32_t)a.k, vo, io, a.threads, ssm, fs);
      else
        merge_full<(RM < 4 ? RM : 4), true>(at, total, (uint32_t)a.k, vo, io, a.threads, ssm, fs);
    } else {
      merge_final<RM, true>(in, a.n_in, a.heads ? a.heads + (size_t)m * a.n_max * kHeads : nullptr,
                            a.n_max, a.kc, (uint32_t)a.k, a.values + (size_t)m * a.k,
                            a.indices + (size_t)m * a.k, a.threads, ssm, fs);
    }
    lds_barrier();  // ssm is reused; fs.out_* are complete
    float lse = 0.f;
    if (a.lse_part != nullptr)
      lse = merge_lse(a.lse_part + (size_t)m * a.n_part, a.n_part, a.lse ? a.lse + m : nullptr, fs, have, pre);
    if (a.smp.on) {
      float* noise = reinterpret_cast<float*>(fs.key);  // free after the merge
      draw_noise(fs.out_idx, a.k, rs, m, a.smp, noise);
      lds_barrier();
      sample_row(fs.out_bits, fs.out_idx, noise, a.k, lse, rs, m, a.smp);
    }
    return;
  }
  const int wave = wave_id();
  const int lane = lane_id();
  const int64_t s0 = (int64_t)blockIdx.x * a.seg;
  __shared__ uint32_t kbin;
  // with the row's key histogram: only keys in or above the bin of the
  // row's k-th largest can be in its top k (wave 0 reads the counts before
  // its candidates, so both are in flight together)
  const bool counted = a.hist != nullptr;
  HistSlice hs;
  if (counted && wave == 0) hs = kth_bin_load(a.hist + (size_t)m * kHistBins);
  uint32_t key[RM], vb[RM];
  int32_t idx[RM];
  uint32_t valid = 0u;
#pragma unroll
  for (int r = 0; r < RM; ++r) {
    const int64_t local = (int64_t)(wave * RM + r) * 64 + lane;
    const int64_t pos = s0 + local;
    uint2 e = make_uint2(0u, 0xFFFFFFFFu);
    if (local < a.seg && pos < a.n_in) e = in[pos];
    vb[r] = e.x;
    idx[r] = (int32_t)e.y;
    key[r] = float_key(__uint_as_float(e.x));
    valid |= (idx[r] >= 0 ? 1u : 0u) << r;
  }
  if (counted) {
    if (wave == 0) kth_bin(hs, (uint32_t)a.k, &kbin);
    lds_barrier();
    const uint32_t b = uniform(kbin);
#pragma unroll
    for (int r = 0; r < RM; ++r)
      if ((key[r] >> 21) < b) valid &= ~(1u << r);
  }
  const SelectRange s = block_select<RM>(key, valid, (uint32_t)a.k, ssm);
  uint2* out = a.out + ((size_t)m * a.n_seg + blockIdx.x) * a.k;
  const uint32_t n = block_compact<RM>(key, valid, s, vb, idx, ssm,
                                       [&](uint32_t pos, uint32_t bits, int32_t ix) {
                                         out[pos] = make_uint2(bits, (uint32_t)ix);
                                       });
  // the count lets the last level gather the selected candidates alone;
  // the padding serves it when there are too many of them for that
  if (a.counts != nullptr && threadIdx.x == 0) a.counts[(size_t)m * a.n_seg + blockIdx.x] = n;
  for (int i = (int)n + (int)threadIdx.x; i < a.k; i += blockDim.x)
    out[i] = make_uint2(0u, 0xFFFFFFFFu);
}
// Zero fill of a workspace (a kernel, not a memset, so that graph capture
// records a kernel node).  n16 whole 16-byte vectors, then tail bytes.
__global__ __launch_bounds__(256) void k_zero(uint4* __restrict__ p, int64_t n16, uint8_t* tail,
                                              int n_tail) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
  if (blockIdx.x == 0 && (int)threadIdx.x < n_tail) tail[threadIdx.x] = 0;
}

namespace {

void (*select_kernel(int rpl))(SelectArgs) {
  switch (rpl) {
    case 1: return k_select_chunk<1>;
    case 4: return k_select_chunk<4>;
  }
  return nullptr;
}
void (*merge_kernel(int rm))(MergeArgs) {
  switch (rm) {
    case 1: return k_merge<1>;
    case 2: return k_merge<2>;
    case 4: return k_merge<4>;
    case 8: return k_merge<8>;
    case 12: return k_merge<12>;
    case 16: return k_merge<16>;
  }
  return nullptr;
}
}  // namespace

int max_lds_per_block(size_t* bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  int v = 0;
  e = hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
  if (e != hipSuccess) return (int)e;
  *bytes = (size_t)v;
  return 0;
}
int launch_pack(const void* w, int w_is_bf16, int64_t V, int64_t H, void* wq, float* wscale,
                void* stream) {
  const int64_t n_tiles = (V + 63) / 64;
  const int64_t G = H / kGroup;
  const int64_t waves = n_tiles * ((G + 3) / 4);
  const dim3 grid((unsigned)((waves + 3) / 4));
  const dim3 block(256);
  const void* a_w = w;
  int64_t a_V = V, a_H = H, a_tiles = n_tiles;
  uint4* a_wq = static_cast<uint4*>(wq);
  float4* a_ws = reinterpret_cast<float4*>(wscale);
  void* args[] = {&a_w, &a_V, &a_H, &a_tiles, &a_wq, &a_ws};
  const void* kern = w_is_bf16 ? reinterpret_cast<const void*>(k_pack<true>)
                               : reinterpret_cast<const void*>(k_pack<false>);
  return (int)hipLaunchKernel(kern, grid, block, args, 0, static_cast<hipStream_t>(stream));
}
int launch_zero(void* p, size_t n, void* stream) {
  const int64_t n16 = (int64_t)(n / 16);
  uint8_t* tail = static_cast<uint8_t*>(p) + n16 * 16;
  const int n_tail = (int)(n % 16);
  int64_t blocks = (n16 + 255) / 256;
  blocks = blocks < 1 ? 1 : (blocks > 1024 ? 1024 : blocks);
  uint4* a_p = static_cast<uint4*>(p);
  int64_t a_n16 = n16;
  uint8_t* a_tail = tail;
  int a_nt = n_tail;
  void* args[] = {&a_p, &a_n16, &a_tail, &a_nt};
  return (int)hipLaunchKernel(reinterpret_cast<const void*>(k_zero), dim3((unsigned)blocks), dim3(256),
                              args, 0, static_cast<hipStream_t>(stream));
}
int launch_select_chunks(const Geometry& g, const float* logits, int64_t ld, void* workspace,
                         float* values, int64_t* indices, void* stream, void* const* events) {
  SelectArgs a;
  a.logits = logits;
  a.M = g.M;
  a.V = g.V;
  a.ld = ld;
  a.chunk_rows = g.chunk_rows;
  a.out = chunk_out(g, workspace, values, indices);
  auto kern = select_kernel(g.rpl);
  if (!kern) return (int)hipErrorInvalidValue;
  return (int)launch1(kern, dim3(g.n_chunks), dim3(64 * g.nw), 0, stream, a, events);
}
int launch_merges(const Geometry& g, void* workspace, float* values, int64_t* indices,
                  void* stream) {
  if (g.fused) return 0;  // the chunk launch merged already
  uint32_t* hist = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(workspace) + kCounterBytes);
  uint8_t* ws = static_cast<uint8_t*>(workspace) + g.sync_bytes;
  const uint2* heads = reinterpret_cast<const uint2*>(ws);
  ws += g.heads_bytes;
  uint2* regions[2] = {reinterpret_cast<uint2*>(ws), reinterpret_cast<uint2*>(ws + g.region0_bytes)};
  const bool counted = g.n_levels >= 2;  // intermediate levels: count the keys first
  if (counted) {
    const int64_t n0 = g.level[0].n_in;
    const dim3 grid((unsigned)((n0 + kHistSpan - 1) / kHistSpan), (unsigned)g.M);
    const uint2* a_in = regions[0];
    int64_t a_n = n0;
    uint32_t* a_h = hist;
    void* args[] = {&a_in, &a_n, &a_h};
    const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(k_hist), grid, dim3(1024), args, 0,
                                         static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return (int)e;
  }
  for (int l = 0; l < g.n_levels; ++l) {
    const MergeLevel& L = g.level[l];
    MergeArgs a;
    a.in = regions[l & 1];
    a.heads = l == 0 ? heads : nullptr;  // heads describe the chunk candidates only
    a.n_max = g.n_chunks;
    a.kc = g.kc;
    a.n_in = L.n_in;
    a.k = g.k;
    a.n_seg = L.n_seg;
    a.threads = 64 * L.nw;
    a.seg = (int64_t)L.nw * 64 * L.rm;
    a.out = regions[(l + 1) & 1];
    a.values = values;
    a.indices = indices;
    a.lse = g.lse;
    a.n_part = g.n_chunks;
    a.lse_part = (g.lse || g.smp.need_norm)
                     ? reinterpret_cast<const uint2*>(ws + g.region0_bytes + g.region1_bytes)
                     : nullptr;
    a.smp = g.smp;
    a.hist = counted && l == 0 ? hist : nullptr;
    a.hist_clear = counted && l == g.n_levels - 1 ? hist : nullptr;
    // two levels: the first writes counts, the last gathers
    uint32_t* counts = g.counts_bytes ? reinterpret_cast<uint32_t*>(ws + g.region0_bytes + g.region1_bytes +
                                                                    g.lse_bytes)
                                      : nullptr;
    a.counts = l == 0 ? counts : nullptr;
    a.in_counts = l == 1 ? counts : nullptr;
    a.in_seg = g.level[0].n_seg;
    auto kern = merge_kernel(L.rm);
    if (!kern) return (int)hipErrorInvalidValue;
    const hipError_t e = launch1(kern, dim3(L.n_seg, (unsigned)g.M), dim3(64 * L.nw), 0, stream, a);
    if (e != hipSuccess) return (int)e;
  }
  return 0;
}

}  // namespace lmtopk
