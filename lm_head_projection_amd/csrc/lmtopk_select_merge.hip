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
};

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
    uint2 pre[kLsePairs];
    int have = 0;
    if (a.lse_part != nullptr) have = load_lse_pairs(a.lse_part + (size_t)m * a.n_part, a.n_part, pre);
    RowSample rs;
    if (a.smp.on) rs = load_row_sample(a.smp, m);
    merge_final<RM, true>(in, a.n_in, a.heads ? a.heads + (size_t)m * a.n_max * kHeads : nullptr,
                    a.n_max, a.kc, (uint32_t)a.k, a.values + (size_t)m * a.k, a.indices + (size_t)m * a.k,
                    a.threads, ssm, fs);
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
  const SelectRange s = block_select<RM>(key, valid, (uint32_t)a.k, ssm);
  uint2* out = a.out + ((size_t)m * a.n_seg + blockIdx.x) * a.k;
  const uint32_t n = block_compact<RM>(key, valid, s, vb, idx, ssm,
                                       [&](uint32_t pos, uint32_t bits, int32_t ix) {
                                         out[pos] = make_uint2(bits, (uint32_t)ix);
                                       });
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
  uint8_t* ws = static_cast<uint8_t*>(workspace) + g.sync_bytes;
  const uint2* heads = reinterpret_cast<const uint2*>(ws);
  ws += g.heads_bytes;
  uint2* regions[2] = {reinterpret_cast<uint2*>(ws), reinterpret_cast<uint2*>(ws + g.region0_bytes)};
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
    auto kern = merge_kernel(L.rm);
    if (!kern) return (int)hipErrorInvalidValue;
    const hipError_t e = launch1(kern, dim3(L.n_seg, (unsigned)g.M), dim3(64 * L.nw), 0, stream, a);
    if (e != hipSuccess) return (int)e;
  }
  return 0;
}

}  // namespace lmtopk
