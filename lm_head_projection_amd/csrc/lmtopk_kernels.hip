// lmtopk_kernels.hip - HIP kernels for gfx950 (CDNA4, wave64) and their launchers.
//
// Kernels
//   k_pack          pack a dense fp32/bf16 head into signs + group scales
//                   (lm-head-topk page, sections "Usage" and "Requirements and
//                   limits": binary weights are packed offline)
//   k_binary_chunk  binary head: one workgroup scores one vocabulary chunk for
//                   all M rows, streaming every packed weight byte once, and
//                   selects that chunk's exact top-k (section "Method")
//   k_dense_chunk   dense fp32/bf16 head, same structure (section "Usage",
//                   dense entry point)
//   k_select_chunk  the chunk selection fed from fp32 logits in memory
//   k_merge         merges chunk candidates into the final sorted top-k
//                   (section "Method", second pass), or into a smaller
//                   candidate set when one workgroup cannot hold them all
//
// Candidates are (fp32 value bits, int32 index) pairs, index -1 = padding.
// Every list of candidates is kept in ascending vocabulary index order, so
// "lower index first" on ties reduces to "earlier position first".

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

#include "lmtopk_device.hpp"
#include "lmtopk_internal.hpp"

namespace lmtopk {

constexpr int kGroup = 128;

// ---------------------------------------------------------------------------
// pack
// ---------------------------------------------------------------------------
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
// shared pieces of the chunk kernels
// ---------------------------------------------------------------------------
struct ChunkOut {
  uint2* cand;   // [M][n_chunks][kc]
  uint2* heads;  // [M][n_chunks][kHeads]
  int n_chunks;
  int kc;
  int k;
};

// Selects the chunk's top-k of row m from RPL slots per lane and writes them
// followed by padding up to kc entries, then the chunk's heads.  Small k:
// select_top_small, candidates in output order.  Otherwise (or when it gives
// up): radix select, candidates in ascending index order.  Either order keeps
// equal values in ascending index, which is all the merge relies on.  `last`
// = no further row follows in this workgroup.
template <int RPL>
__device__ __forceinline__ void chunk_select_write(const float (&val)[RPL], const int32_t (&idx)[RPL],
                                                   uint32_t valid, int m, const ChunkOut& o,
                                                   SelectSmem& sm, HeadStage& st, bool last) {
  uint32_t key[RPL], vb[RPL];
#pragma unroll
  for (int r = 0; r < RPL; ++r) {
    vb[r] = __float_as_uint(val[r]);
    key[r] = float_key(val[r]);
  }
  const size_t row_chunk = (size_t)m * o.n_chunks + blockIdx.x;
  uint2* out = o.cand + row_chunk * o.kc;
  uint2* heads = o.heads + row_chunk * kHeads;
  if (o.k <= kWaveTops * (int)(blockDim.x >> 6)) {
    const uint32_t n = select_top_small<RPL>(key, valid, vb, idx, (uint32_t)o.k, st,
                                             [&](uint32_t pos, uint32_t bits, int32_t ix) {
                                               const uint2 e = make_uint2(bits, (uint32_t)ix);
                                               out[pos] = e;
                                               if (pos < (uint32_t)kHeads) heads[pos] = e;
                                             });
    if (n != 0xFFFFFFFFu) {
      for (int i = (int)n + (int)threadIdx.x; i < o.kc; i += blockDim.x)
        out[i] = make_uint2(0u, 0xFFFFFFFFu);
      for (int i = (int)n + (int)threadIdx.x; i < kHeads; i += blockDim.x)
        heads[i] = make_uint2(0u, 0xFFFFFFFFu);
      if (!last) lds_barrier();  // the staging is refilled by the next row
      return;
    }
  }
  const SelectRange s = block_select<RPL>(key, valid, (uint32_t)o.k, sm);
  const uint32_t n = block_compact<RPL>(key, valid, s, vb, idx, sm,
                                        [&](uint32_t pos, uint32_t bits, int32_t ix) {
                                          out[pos] = make_uint2(bits, (uint32_t)ix);
                                        });
  for (int i = (int)n + (int)threadIdx.x; i < o.kc; i += blockDim.x)
    out[i] = make_uint2(0u, 0xFFFFFFFFu);
  // the chunk's best entries are the best of its candidates (a head beyond
  // a k < 4 is still a real logit of the row, which the merge may consider)
  block_heads<RPL>(key, valid, vb, idx, st, heads);
  if (!last) lds_barrier();  // the staging is refilled by the next row
}

// ---------------------------------------------------------------------------
// binary chunk kernel
// ---------------------------------------------------------------------------
// Activations in balanced ternary.  Every int8 activation a is written as
// a = sum_{p<6} 3^p d_p with digits d_p in {-1, 0, +1} (six trits reach
// +-364).  For one group of 128 activations and trit p, two bit masks are
// kept: NZ_p (d_p != 0) and POS_p (d_p == +1).  With the sign bits b of one
// weight row (bit 1 = +1) the group's trit-p dot is
//   sum_j sign_j d_pj = 2 popcount(XNOR(b, POS_p) AND NZ_p) - popcount(NZ_p),
// so the exact integer group dot is
//   D = sum_j a_j sign_j = 2 S - C,   S = sum_p 3^p popcount(XNOR(b, POS_p) AND NZ_p),
//   C = sum_p 3^p popcount(NZ_p)  (the same for every weight row).
// Per 32 weights and trit that is one 3-input bit operation (v_bitop3) and
// one accumulating popcount (v_bcnt), 48 + 5 Horner steps per group of 128.
struct TritGroup {
  uint4 pos_nz[12];  // [trit p] -> {POS_p, NZ_p}, 4 words = 128 activations each
};

struct BinaryArgs {
  const int8_t* act_q;     // [M][H]
  const float* act_scale;  // [M]
  const uint4* wq;         // packed signs, layout v1
  const float4* wscale;    // packed scales, layout v1
  const float* bias;       // [V] or null
  int64_t V, H, n_tiles;
  int G, Q;
  int tiles_per_chunk;
  ChunkOut out;
};

__device__ __forceinline__ uint32_t bcnt_acc(uint32_t x, uint32_t acc) {
  uint32_t r;
  asm("v_bcnt_u32_b32 %0, %1, %2" : "=v"(r) : "v"(x), "v"(acc));
  return r;
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

__device__ __forceinline__ float comp4(const float4& f, int i) {
  return i == 0 ? f.x : i == 1 ? f.y : i == 2 ? f.z : f.w;
}

// S of one group for R weight rows at once: the trit masks are read once and
// serve all R rows.
template <int R>
__device__ __forceinline__ void trit_dot(const uint4 (&w)[R], const uint4* tg, uint32_t (&u)[R]) {
#pragma unroll
  for (int r = 0; r < R; ++r) u[r] = 0u;
#pragma unroll
  for (int p = 5; p >= 0; --p) {
    const uint4 pos = tg[2 * p];
    const uint4 nz = tg[2 * p + 1];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      uint32_t x = (u[r] << 1) + u[r];
      x = bcnt_acc(~(w[r].x ^ pos.x) & nz.x, x);
      x = bcnt_acc(~(w[r].y ^ pos.y) & nz.y, x);
      x = bcnt_acc(~(w[r].z ^ pos.z) & nz.z, x);
      x = bcnt_acc(~(w[r].w ^ pos.w) & nz.w, x);
      u[r] = x;
    }
  }
}

// Lane l of wave w owns the R rows ((chunk * tiles_per_chunk + w * R + r) * 64 + l),
// r < R, and scores them together.  Each group's 128 sign bits of a row are
// one 16-byte load; the four scales of a quad of groups are one more.  The
// fp32 logit accumulates fmaf((float)D_g, scale_g, acc) in ascending g, so
// every row takes the same operation sequence wherever it sits.
//
// Latency: the activation bytes are requested first and the first two quads
// of weights right after them; the trit masks are built while those weights
// are in flight (the barriers here only order LDS, so they do not wait for
// the weight loads).  In the steady state two quads are in flight while one
// is computed; the loads are issued unconditionally and pinned in place so
// that each wait covers only the buffer about to be used.
static_assert(sizeof(SelectSmem) + sizeof(HeadStage) <= kChunkStaticLds,
              "static LDS of the chunk kernels exceeds the bound the host checks");

// Quads of weight loads in flight per wave.
constexpr int kQuadBuffers = 2;

template <int M, int R>
__global__ __launch_bounds__(R == 1 ? 1024 : 512) void k_binary_chunk(BinaryArgs a) {
  extern __shared__ __align__(16) uint8_t dyn_lds[];
  __shared__ SelectSmem ssm;
  __shared__ HeadStage hst;
  for (int i = threadIdx.x; i < kMaxK; i += blockDim.x) hst.rank[i] = 0u;  // ordered by the barriers below
  const int G = a.G;
  uint16_t* table = reinterpret_cast<uint16_t*>(dyn_lds);             // [256] trit codes
  TritGroup* tgs = reinterpret_cast<TritGroup*>(dyn_lds + 512);       // [M][G]
  int* cg = reinterpret_cast<int*>(tgs + (size_t)M * G);              // [M][G] C of the group
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid >> 6;
  const int nw = blockDim.x >> 6;
  const int Qf = G >> 2;  // full quads
  const int64_t tile0 = (int64_t)blockIdx.x * a.tiles_per_chunk + (int64_t)wave * R;
  const bool active = tile0 < a.n_tiles;

  // a tile past the last one reads the last tile; its rows are never offered
  const uint4* wp[R];
  const float4* sp[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t t = tile0 + r < a.n_tiles ? tile0 + r : a.n_tiles - 1;
    wp[r] = a.wq + (size_t)t * G * 64 + lane;
    sp[r] = a.wscale + (size_t)t * a.Q * 64 + lane;
  }

  // Prologue.  Everything whose load count depends on the shapes happens
  // before the weight prefetch, and the prefetch is followed only by
  // straight-line code, so the waits after it cover exactly what they need.
  // 1. trit code of every int8 value: bits 0..5 NZ_p, bits 8..13 POS_p
  for (int e = tid; e < 256; e += blockDim.x) {
    int v = e < 128 ? e : e - 256;
    uint32_t c = 0u;
#pragma unroll
    for (int p = 0; p < 6; ++p) {
      int r = v % 3;  // in {-2, ..., 2}
      if (r == 2) r = -1;
      if (r == -2) r = 1;
      if (r != 0) c |= 1u << p;
      if (r == 1) c |= 1u << (8 + p);
      v = (v - r) / 3;
    }
    table[e] = (uint16_t)c;
  }
  lds_barrier();

  // 2. trit masks of a batch of groups: each mask word is one ballot over 64
  //    activations (groups b0, b0 + nw, ..., this wave's share)
  constexpr int kBatch = 4;
  const int n_mg = M * G;
  auto load_acts = [&](int b0, int8_t (&y0)[kBatch], int8_t (&y1)[kBatch]) {
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      int mg = b0 + i * nw;
      mg = mg < n_mg ? mg : n_mg - 1;  // clamped; the extra groups are not used
      const int m = mg / G;
      const int8_t* src = a.act_q + (size_t)m * a.H + (size_t)(mg - m * G) * kGroup;
      y0[i] = src[lane];
      y1[i] = src[64 + lane];
    }
  };
  auto build_masks = [&](int b0, const int8_t (&y0)[kBatch], const int8_t (&y1)[kBatch]) {
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int mg = b0 + i * nw;
      if (mg >= n_mg) break;
      const uint32_t c0 = table[(uint8_t)y0[i]];
      const uint32_t c1 = table[(uint8_t)y1[i]];
      uint4 mine = make_uint4(0u, 0u, 0u, 0u);
      int cgroup = 0, w3 = 1;
#pragma unroll
      for (int p = 0; p < 6; ++p) {
        const uint64_t p0 = ballot((c0 >> (8 + p)) & 1u), p1 = ballot((c1 >> (8 + p)) & 1u);
        const uint64_t n0 = ballot((c0 >> p) & 1u), n1 = ballot((c1 >> p) & 1u);
        if (lane == 2 * p)
          mine = make_uint4((uint32_t)p0, (uint32_t)(p0 >> 32), (uint32_t)p1, (uint32_t)(p1 >> 32));
        if (lane == 2 * p + 1)
          mine = make_uint4((uint32_t)n0, (uint32_t)(n0 >> 32), (uint32_t)n1, (uint32_t)(n1 >> 32));
        cgroup += w3 * (__popcll(n0) + __popcll(n1));
        w3 *= 3;
      }
      if (lane < 12) tgs[mg].pos_nz[lane] = mine;
      if (lane == 0) cg[mg] = cgroup;
    }
  };
  //    batches after the first (large M * H only)
  for (int b0 = wave + nw * kBatch; b0 < n_mg; b0 += nw * kBatch) {
    int8_t y0[kBatch], y1[kBatch];
    load_acts(b0, y0, y1);
    build_masks(b0, y0, y1);
  }
  // 3. the first batch's activation bytes, this lane's bias and the row
  //    scales (loaded now: after the main loop a load would cost a full
  //    memory round trip in the tail)
  int8_t x0[kBatch], x1[kBatch];
  load_acts(wave, x0, x1);
  float bias_v[R];
  {
    // unconditional loads from valid addresses; the values are used only
    // for real rows of a real bias
    const float* bp = a.bias != nullptr ? a.bias : a.act_scale;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      int64_t v = (tile0 + r) * 64 + lane;
      v = a.bias != nullptr ? (v < a.V ? v : a.V - 1) : 0;
      bias_v[r] = bp[v];
    }
  }
  float act_s[M];
#pragma unroll
  for (int m = 0; m < M; ++m) act_s[m] = a.act_scale[m];
  __builtin_amdgcn_sched_barrier(0);
  // every wave's activation requests go out before any wave's weight
  // requests: the CU serves its requests in order, so otherwise the last
  // waves would wait for most of the weight prefetch before they could build
  // their masks
  lds_barrier();

  // 4. first quads of weights (group and quad indices clamped into the head),
  //    issued in the same order as the main loop's refills
  uint4 buf[kQuadBuffers][R][4];
  float4 sbuf[kQuadBuffers][R];
#pragma unroll
  for (int b = 0; b < kQuadBuffers; ++b) {
    const int qc = b < a.Q ? b : a.Q - 1;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      sbuf[b][r] = ld_stream(&sp[r][qc * 64]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int g = 4 * b + i;
        buf[b][r][i] = ld_stream(&wp[r][(g < G ? g : G - 1) * 64]);
      }
    }
  }

  __builtin_amdgcn_sched_barrier(0);
  // 5. the first batch's masks, built while the weights are in flight
  build_masks(wave, x0, x1);
  lds_barrier();

  float acc[R][M];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[r][m] = 0.f;

  auto compute_group = [&](int g, const uint4 (&w)[R], const float (&s)[R]) {
#pragma unroll
    for (int m = 0; m < M; ++m) {
      uint32_t u[R];
      trit_dot<R>(w, tgs[(size_t)m * G + g].pos_nz, u);
      const int c = cg[m * G + g];
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r][m] = fmaf((float)(2 * (int)u[r] - c), s[r], acc[r][m]);
    }
  };
  auto compute_quad = [&](int q, const uint4 (&buf)[R][4], const float4 (&s)[R]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint4 w[R];
      float sc[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        w[r] = buf[r][i];
        sc[r] = comp4(s[r], i);
      }
      compute_group(4 * q + i, w, sc);
    }
  };
  auto load_quad = [&](int q, uint4 (&w)[R][4], float4 (&s)[R]) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      s[r] = ld_stream(&sp[r][q * 64]);
#pragma unroll
      for (int i = 0; i < 4; ++i) w[r][i] = ld_stream(&wp[r][(4 * q + i) * 64]);
    }
  };

  if (active) {
    // quads q .. q + kQuadBuffers - 1 are in flight at the top; each buffer is
    // refilled right after its last use
    constexpr int NB = kQuadBuffers;
    int q = 0;
    for (; q + 2 * NB - 1 < Qf; q += NB) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        compute_quad(q + b, buf[b], sbuf[b]);
        __builtin_amdgcn_sched_barrier(0);
        load_quad(q + b + NB, buf[b], sbuf[b]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // drain: fewer than 2 * NB quads remain
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (q + b < Qf) {
        compute_quad(q + b, buf[b], sbuf[b]);
        if (q + b + NB < Qf) load_quad(q + b + NB, buf[b], sbuf[b]);
      }
    }
#pragma unroll
    for (int b = 0; b < NB; ++b)
      if (q + NB + b < Qf) compute_quad(q + NB + b, buf[b], sbuf[b]);
    if (4 * Qf < G) {  // last, partial quad
      float4 st[R];
#pragma unroll
      for (int r = 0; r < R; ++r) st[r] = ld_stream(&sp[r][Qf * 64]);
      for (int g = 4 * Qf; g < G; ++g) {
        uint4 w[R];
        float sc[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          w[r] = ld_stream(&wp[r][g * 64]);
          sc[r] = comp4(st[r], g - 4 * Qf);
        }
        compute_group(g, w, sc);
      }
    }
  }

  int32_t idx[R];
  uint32_t valid = 0u;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t v = (tile0 + r) * 64 + lane;
    idx[r] = (int32_t)v;
    const bool vv = (tile0 + r) < a.n_tiles && v < a.V;
    valid |= (vv ? 1u : 0u) << r;
    if (a.bias == nullptr || !vv) bias_v[r] = 0.f;
  }
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const float s = act_s[m];
    float val[R];
#pragma unroll
    for (int r = 0; r < R; ++r) val[r] = fmaf(acc[r][m], s, bias_v[r]);
    chunk_select_write<R>(val, idx, valid, m, a.out, ssm, hst, m == M - 1);
  }
}

// ---------------------------------------------------------------------------
// dense chunk kernel
// ---------------------------------------------------------------------------
struct DenseArgs {
  const uint8_t* hidden;  // [M][H] fp32 or bf16
  const uint8_t* weight;  // [V][H] fp32 or bf16
  const float* bias;
  int64_t V, H;
  int chunk_rows;
  ChunkOut out;
};

template <bool BF16>
__device__ __forceinline__ float dot16(const uint4& h, const uint4& w, float acc) {
  if (BF16) {
    const uint32_t hp[4] = {h.x, h.y, h.z, h.w};
    const uint32_t wp[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc = fmaf(__uint_as_float(hp[e] << 16), __uint_as_float(wp[e] << 16), acc);
      acc = fmaf(__uint_as_float(hp[e] & 0xFFFF0000u), __uint_as_float(wp[e] & 0xFFFF0000u), acc);
    }
  } else {
    acc = fmaf(__uint_as_float(h.x), __uint_as_float(w.x), acc);
    acc = fmaf(__uint_as_float(h.y), __uint_as_float(w.y), acc);
    acc = fmaf(__uint_as_float(h.z), __uint_as_float(w.z), acc);
    acc = fmaf(__uint_as_float(h.w), __uint_as_float(w.w), acc);
  }
  return acc;
}

// One wave computes one vocabulary row at a time (two rows interleaved):
// lane l takes the 16-byte vectors l, l+64, ... of the row, accumulates in
// fp32 in that order, then an xor-butterfly over the 64 lanes gives the row
// sum (the same tree for every row).  Scores go to LDS; the chunk selection
// reads them back one row per lane slot.
template <int M, bool BF16, int RPL>
__global__ __launch_bounds__(1024) void k_dense_chunk(DenseArgs a) {
  extern __shared__ __align__(16) uint8_t dyn_lds[];
  __shared__ SelectSmem ssm;
  __shared__ HeadStage hst;
  for (int i = threadIdx.x; i < kMaxK; i += blockDim.x) hst.rank[i] = 0u;  // ordered by the barriers below
  float* scores = reinterpret_cast<float*>(dyn_lds);  // [M][C]
  const int C = a.chunk_rows;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid >> 6;
  const int esz = BF16 ? 2 : 4;
  const int64_t nvec = a.H * esz / 16;
  const int64_t row_bytes = a.H * esz;
  const int64_t base = (int64_t)blockIdx.x * C;
  const int rows_per_wave = 64 * RPL;

  for (int rr = 0; rr < rows_per_wave; rr += 2) {
    const int lr0 = wave * rows_per_wave + rr;
    const int64_t v0 = base + lr0, v1 = v0 + 1;
    const bool ok0 = v0 < a.V, ok1 = v1 < a.V;
    if (!ok0) break;  // rows are in increasing order
    float acc0[M], acc1[M];
#pragma unroll
    for (int m = 0; m < M; ++m) acc0[m] = acc1[m] = 0.f;
    const uint4* w0 = reinterpret_cast<const uint4*>(a.weight + v0 * row_bytes);
    const uint4* w1 = reinterpret_cast<const uint4*>(a.weight + (ok1 ? v1 : v0) * row_bytes);
#pragma unroll 2
    for (int64_t i = lane; i < nvec; i += 64) {
      const uint4 x0 = ld_stream(&w0[i]);
      const uint4 x1 = ld_stream(&w1[i]);
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const uint4 h = reinterpret_cast<const uint4*>(a.hidden + (int64_t)m * row_bytes)[i];
        acc0[m] = dot16<BF16>(h, x0, acc0[m]);
        acc1[m] = dot16<BF16>(h, x1, acc1[m]);
      }
    }
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float s0 = acc0[m], s1 = acc1[m];
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        s0 += __shfl_xor(s0, o);
        s1 += __shfl_xor(s1, o);
      }
      if (lane == 0) {
        scores[m * C + lr0] = s0 + (a.bias ? a.bias[v0] : 0.f);
        if (ok1) scores[m * C + lr0 + 1] = s1 + (a.bias ? a.bias[v1] : 0.f);
      }
    }
  }
  __syncthreads();

  int32_t idx[RPL];
  uint32_t valid = 0u;
  int lr[RPL];
#pragma unroll
  for (int r = 0; r < RPL; ++r) {
    lr[r] = (wave * RPL + r) * 64 + lane;
    const int64_t v = base + lr[r];
    idx[r] = (int32_t)v;
    valid |= (v < a.V ? 1u : 0u) << r;
  }
#pragma unroll
  for (int m = 0; m < M; ++m) {
    float val[RPL];
#pragma unroll
    for (int r = 0; r < RPL; ++r) val[r] = ((valid >> r) & 1u) ? scores[m * C + lr[r]] : 0.f;
    chunk_select_write<RPL>(val, idx, valid, m, a.out, ssm, hst, m == M - 1);
  }
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
  __shared__ HeadStage hst;
  for (int i = threadIdx.x; i < kMaxK; i += blockDim.x) hst.rank[i] = 0u;  // ordered by the selection's barriers
  const int wave = threadIdx.x >> 6;
  const int lane = lane_id();
  const int64_t base = (int64_t)blockIdx.x * a.chunk_rows;
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
    chunk_select_write<RPL>(val, idx, valid, m, a.out, ssm, hst, m == (int)a.M - 1);
  }
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
};

// Workgroup (segment s, row m) takes candidates [s*seg, (s+1)*seg) of row m,
// RM slots per thread (slot order = candidate order = index order), selects
// their exact top-k and either writes them in index order (intermediate
// level) or sorts them by (value desc, index asc) through rank counting --
// each entry's output position is the number of entries ahead of it -- and
// writes values / indices (final level).
template <int RM>
__global__ __launch_bounds__(1024) void k_merge(MergeArgs a) {
  __shared__ SelectSmem ssm;
  const int m = blockIdx.y;
  const uint2* in = a.in + (size_t)m * a.n_in;
  if (a.n_seg == 1) {
    __shared__ FinalSmem fs;
    merge_final<RM>(in, a.n_in, a.heads ? a.heads + (size_t)m * a.n_max * kHeads : nullptr,
                    a.n_max, a.kc, (uint32_t)a.k, a.values + (size_t)m * a.k, a.indices + (size_t)m * a.k,
                    a.threads, ssm, fs);
    return;
  }
  const int wave = threadIdx.x >> 6;
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

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
namespace {

// events: null, or two hipEvent_t that record the kernel's own start and end
template <typename Arg>
hipError_t launch1(void (*kern)(Arg), dim3 grid, dim3 block, size_t lds, void* stream, Arg arg,
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

template <int M>
void (*binary_kernel_m(int rpl))(BinaryArgs) {
  switch (rpl) {
    case 1: return k_binary_chunk<M, 1>;
    case 2: return k_binary_chunk<M, 2>;
    case 4: return k_binary_chunk<M, 4>;
  }
  return nullptr;
}

void (*binary_kernel(int M, int rpl))(BinaryArgs) {
  switch (M) {
    case 1: return binary_kernel_m<1>(rpl);
    case 2: return binary_kernel_m<2>(rpl);
    case 3: return binary_kernel_m<3>(rpl);
    case 4: return binary_kernel_m<4>(rpl);
    case 5: return binary_kernel_m<5>(rpl);
    case 6: return binary_kernel_m<6>(rpl);
    case 7: return binary_kernel_m<7>(rpl);
    case 8: return binary_kernel_m<8>(rpl);
  }
  return nullptr;
}

template <int M, bool BF16>
void (*dense_kernel_mb(int rpl))(DenseArgs) {
  switch (rpl) {
    case 1: return k_dense_chunk<M, BF16, 1>;
    case 2: return k_dense_chunk<M, BF16, 2>;
    case 4: return k_dense_chunk<M, BF16, 4>;
  }
  return nullptr;
}

template <bool BF16>
void (*dense_kernel_b(int M, int rpl))(DenseArgs) {
  switch (M) {
    case 1: return dense_kernel_mb<1, BF16>(rpl);
    case 2: return dense_kernel_mb<2, BF16>(rpl);
    case 3: return dense_kernel_mb<3, BF16>(rpl);
    case 4: return dense_kernel_mb<4, BF16>(rpl);
    case 5: return dense_kernel_mb<5, BF16>(rpl);
    case 6: return dense_kernel_mb<6, BF16>(rpl);
    case 7: return dense_kernel_mb<7, BF16>(rpl);
    case 8: return dense_kernel_mb<8, BF16>(rpl);
  }
  return nullptr;
}

void (*select_kernel(int rpl))(SelectArgs) {
  switch (rpl) {
    case 1: return k_select_chunk<1>;
    case 2: return k_select_chunk<2>;
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

ChunkOut chunk_out(const Geometry& g, void* workspace) {
  ChunkOut o;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  o.heads = reinterpret_cast<uint2*>(ws);
  o.cand = reinterpret_cast<uint2*>(ws + g.heads_bytes);
  o.n_chunks = g.n_chunks;
  o.kc = g.kc;
  o.k = g.k;
  return o;
}

}  // namespace

size_t binary_lds_bytes(int64_t M, int64_t H) {
  const int64_t G = H / kGroup;
  return (size_t)(512 + M * G * sizeof(TritGroup) + M * G * 4);
}

size_t dense_lds_bytes(int64_t M, int chunk_rows) { return (size_t)(M * chunk_rows * 4); }

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

int launch_binary_chunks(const Geometry& g, const int8_t* act_q, const float* act_scale,
                         const void* wq, const float* wscale, const float* bias, int64_t H,
                         void* workspace, void* stream, void* const* events) {
  BinaryArgs a;
  a.act_q = act_q;
  a.act_scale = act_scale;
  a.wq = static_cast<const uint4*>(wq);
  a.wscale = reinterpret_cast<const float4*>(wscale);
  a.bias = bias;
  a.V = g.V;
  a.H = H;
  a.n_tiles = g.n_tiles;
  a.G = (int)(H / kGroup);
  a.Q = (a.G + 3) / 4;
  a.tiles_per_chunk = g.chunk_rows / 64;
  a.out = chunk_out(g, workspace);
  auto kern = binary_kernel((int)g.M, g.rpl);
  if (!kern) return (int)hipErrorInvalidValue;
  return (int)launch1(kern, dim3(g.n_chunks), dim3(64 * g.nw), binary_lds_bytes(g.M, H), stream, a,
                      events);
}

int launch_dense_chunks(const Geometry& g, const void* hidden, const void* weight, int is_bf16,
                        const float* bias, int64_t H, void* workspace, void* stream,
                        void* const* events) {
  DenseArgs a;
  a.hidden = static_cast<const uint8_t*>(hidden);
  a.weight = static_cast<const uint8_t*>(weight);
  a.bias = bias;
  a.V = g.V;
  a.H = H;
  a.chunk_rows = g.chunk_rows;
  a.out = chunk_out(g, workspace);
  auto kern = is_bf16 ? dense_kernel_b<true>((int)g.M, g.rpl) : dense_kernel_b<false>((int)g.M, g.rpl);
  if (!kern) return (int)hipErrorInvalidValue;
  return (int)launch1(kern, dim3(g.n_chunks), dim3(64 * g.nw), dense_lds_bytes(g.M, g.chunk_rows),
                      stream, a, events);
}

int launch_select_chunks(const Geometry& g, const float* logits, int64_t ld, void* workspace,
                         void* stream, void* const* events) {
  SelectArgs a;
  a.logits = logits;
  a.M = g.M;
  a.V = g.V;
  a.ld = ld;
  a.chunk_rows = g.chunk_rows;
  a.out = chunk_out(g, workspace);
  auto kern = select_kernel(g.rpl);
  if (!kern) return (int)hipErrorInvalidValue;
  return (int)launch1(kern, dim3(g.n_chunks), dim3(64 * g.nw), 0, stream, a, events);
}

int launch_merges(const Geometry& g, void* workspace, float* values, int64_t* indices,
                  void* stream) {
  uint8_t* ws = static_cast<uint8_t*>(workspace);
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
    auto kern = merge_kernel(L.rm);
    if (!kern) return (int)hipErrorInvalidValue;
    const hipError_t e = launch1(kern, dim3(L.n_seg, (unsigned)g.M), dim3(64 * L.nw), 0, stream, a);
    if (e != hipSuccess) return (int)e;
  }
  return 0;
}


}  // namespace lmtopk
