// lmtopk_binary.hip - binary-head chunk kernel (gfx950) and its launcher.
//
// k_binary_chunk: one workgroup scores one vocabulary chunk of a packed
// binary head for all M rows, streaming every packed weight byte once, and
// selects that chunk's exact top-k (lm-head-topk page, section "Method").
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

#include "lmtopk_chunk.hpp"

namespace lmtopk {

constexpr int kGroup = 128;

// Activations as two's-complement bit planes.  Every int8 activation is
// a = sum_{p<8} c_p a_p with bits a_p and weights c_p = 2^p (p < 7),
// c_7 = -128.  For one group of 128 activations and bit p the plane P_p
// holds a_p of each activation (4 words, bit b of word w = activation
// 32 w + b).  With the sign bits b of one weight row (bit 1 = +1, so
// sign_j = 2 b_j - 1) the exact integer group dot is
//   D = sum_j a_j sign_j = 2 S - C,
//   S = sum_j a_j b_j = sum_p c_p sum_{w<4} popcount(b_w AND P_pw),
//   C = sum_j a_j  (the same for every weight row).
// S is accumulated by Horner's rule over the planes, top plane first.  Per
// 32 weights and plane that is one AND and one accumulating popcount
// (v_bcnt): 64 operations and 8 mask reads of 16 bytes per group of 128.
struct PlaneGroup {
  uint4 plane[8];  // [bit p] -> P_p, 4 words = 128 activations
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
  int ks;  // waves per tile: 1, or 2 (a pair of waves splits the groups)
  ChunkOut out;
};

__device__ __forceinline__ uint32_t bcnt_acc(uint32_t x, uint32_t acc) {
  uint32_t r;
  asm("v_bcnt_u32_b32 %0, %1, %2" : "=v"(r) : "v"(x), "v"(acc));
  return r;
}

__device__ __forceinline__ float comp4(const float4& f, int i) {
  return i == 0 ? f.x : i == 1 ? f.y : i == 2 ? f.z : f.w;
}

// S of one group for R weight rows at once: each plane is read once and
// serves all R rows.
template <int R>
__device__ __forceinline__ void plane_dot(const uint4 (&w)[R], const uint4* pg, uint32_t (&u)[R]) {
#pragma unroll
  for (int r = 0; r < R; ++r) u[r] = 0u;
#pragma unroll
  for (int p = 7; p >= 0; --p) {
    const uint4 pl = pg[p];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      uint32_t x = bcnt_acc(w[r].x & pl.x, 0u);
      x = bcnt_acc(w[r].y & pl.y, x);
      x = bcnt_acc(w[r].z & pl.z, x);
      x = bcnt_acc(w[r].w & pl.w, x);
      // S = (...((-S_7) * 2 + S_6) * 2 + ...) + S_0, in two's complement
      u[r] = p == 7 ? 0u - x : (u[r] << 1) + x;
    }
  }
}

// From two rows on (one row per lane) a group's integer sums come from the
// matrix cores.  For each block of 16 rows of the tile, two
// v_mfma_i32_16x16x64_i8 (64 elements each) multiply the activation bytes
// (A, 16 x 64: activation row m in lanes m, 16 + m, 32 + m, 48 + m; rows M
// to 15 repeat row 0 and are not used) by the sign bits as 0/1 bytes (B,
// 64 x 16: the block's rows) into 16 x 16 integer sums.  Lane layouts on
// gfx950: lane 16 q + j holds elements [16 q, 16 q + 16) of A's row j and of
// B's column j, and rows 4 q .. 4 q + 3 of column j of the sums.
//   The sign bits arrive one row per lane (four words); transpose4 over the
// four lane groups gives lane 16 q + p word q of the rows 16 b + p, b = 0..3,
// and (y >> j) & 0x01010101, j = 0..7, spreads a word into bytes: byte i of
// spread j is bit 8 i + j.  The activation bytes are kept in LDS in the
// matching order (element 32 q + 8 i + j of a group at byte 32 q + 4 j + i,
// act_byte_slot).  The same transpose brings each row's sums back to the
// row's own lane.  The sums are the same exact integers as the bit-plane
// sums: 4 + 60 + 12 + 3 M vector instructions and 8 matrix instructions
// per group, against 96 + 32 M with 8-bit dot products.
typedef int v4i32_t __attribute__((ext_vector_type(4)));
constexpr uint32_t kByteBits = 0x01010101u;
__device__ __forceinline__ uint32_t act_byte_slot(uint32_t e) {
  return (e & ~31u) | ((e & 7u) << 2) | ((e >> 3) & 3u);
}
// Register j of lane 16 q + p receives register q of lane 16 j + p (a 4 x 4
// transpose of lane groups and registers): first the upper lane half of
// r0 / r1 with the lower half of r2 / r3, then the odd lane groups of r0 /
// r2 with the even ones of r1 / r3.
__device__ __forceinline__ void transpose4(uint32_t& r0, uint32_t& r1, uint32_t& r2, uint32_t& r3) {
  const auto s02 = __builtin_amdgcn_permlane32_swap(r0, r2, false, false);
  const auto s13 = __builtin_amdgcn_permlane32_swap(r1, r3, false, false);
  const auto s01 = __builtin_amdgcn_permlane16_swap(s02[0], s13[0], false, false);
  const auto s23 = __builtin_amdgcn_permlane16_swap(s02[1], s13[1], false, false);
  r0 = s01[0];
  r1 = s01[1];
  r2 = s23[0];
  r3 = s23[1];
}

// Lane l of wave w owns the R rows ((chunk * tiles_per_chunk + w * R + r) * 64 + l),
// r < R, and scores them together.  Each group's 128 sign bits of a row are
// one 16-byte load; the four scales of a quad of groups are one more.
//
// Accumulation order (the same on every path, so a row's logit does not
// depend on the chunk size or on M): with Q = ceil(G / 4) quads and
// Qh = floor(Q / 2), the quads [0, Qh) and [Qh, Q) are two chains, each
// accumulating fmaf((float)D_g, scale_g, acc) from 0 in ascending g, and the
// logit's dot part is lo + hi.
//
// Two waves per tile (ks = 2, chunks of up to 512 rows, one row per lane):
// waves 2t and 2t + 1 share tile t, the first running the chain of [0, Qh)
// and the second that of [Qh, Q) for all 64 rows, so a workgroup of 16
// waves streams a 512-row chunk.  The first then keeps rows 0-31 of the
// tile and the second rows 32-63; each leaves the partial sums of the rows
// it gives up in LDS for the other.  Without a split (ks = 1) one wave runs
// both chains.
//
// Latency: the activation bytes are requested first and the first two quads
// of weights right after them; the bit planes are built while those weights
// are in flight (the barriers here only order LDS, so they do not wait for
// the weight loads).  In the steady state two quads are in flight while one
// is computed; the loads are issued unconditionally and pinned in place so
// that each wait covers only the buffer about to be used.
static_assert(sizeof(SelectSmem) + sizeof(ChunkSmem) + 16 <= kChunkStaticLds,
              "static LDS of the chunk kernels exceeds the bound the host checks");

// Quads of weight loads in flight per wave.
constexpr int kQuadBuffers = 2;
// Waves of a chunk workgroup with two waves per tile (512-row chunks).
constexpr int kPairWaves = 16;
// Buffer resource word 3 for raw (untyped) buffer loads on gfx9, and the
// cache-policy operand that marks a buffer load non-temporal.
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kBufNt = 2;

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 as_uint4(u32x4_t v) { return make_uint4(v.x, v.y, v.z, v.w); }
__device__ __forceinline__ float4 as_float4(u32x4_t v) {
  return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z),
                     __uint_as_float(v.w));
}

// kExtras: a log-sum-exp output or a bitmask; kSample (implies kExtras): a
// token draw.  Calls without them run instances with that code left out.
//
template <int M, int R, bool kExtras, bool kSample = false>
__global__ __launch_bounds__(R == 1 ? 1024 : 512) void k_binary_chunk(BinaryArgs a) {
  extern __shared__ __align__(16) uint8_t dyn_lds[];
  __shared__ SelectSmem ssm;
  __shared__ ChunkSmem csm;
  __shared__ uint32_t last_wg;
  HeadStage& hst = csm.hs;
  head_stage_init<(M >= 2)>(hst);  // ordered by the barriers below
  // from two rows on (one row per lane), the activation bytes and the
  // matrix cores (see transpose4) take fewer instructions than the bit planes
  constexpr bool kBytes = M >= 2 && R == 1;
  const int G = a.G;
  PlaneGroup* pgs = reinterpret_cast<PlaneGroup*>(dyn_lds);          // [M][G]
  int* cg = reinterpret_cast<int*>(pgs + (size_t)M * G);              // [M][G] C of the group
  float* xch = reinterpret_cast<float*>(cg + (size_t)M * G);          // ks = 2: [waves][32][M]
  uint32_t* xflag = reinterpret_cast<uint32_t*>(xch + (size_t)kPairWaves * 32 * M);  // [waves]
  const int lane = lane_id();
  const int wave = wave_id();
  const int nw = blockDim.x >> 6;
  const int a_row = (lane & 15) < M ? (lane & 15) : 0;  // kBytes: this lane's activation row of A
  const int Qf = G >> 2;  // full quads
  const bool pair = R == 1 && a.ks == 2;
  const bool second = pair && (wave & 1);  // runs the second chain of a pair
  const int64_t tile0 =
      (int64_t)blockIdx.x * a.tiles_per_chunk + (int64_t)(pair ? wave >> 1 : wave * R);
  const bool active = tile0 < a.n_tiles;
  // this wave's quads [qa, qb); `split`: the quad after which a wave that
  // runs both chains starts the second (-1: it runs one)
  const int Qh = a.Q >> 1;
  const int qa = second ? Qh : 0;
  const int qb = pair && !second ? Qh : a.Q;
  const int split = pair ? -1 : Qh;
  if (pair && threadIdx.x < kPairWaves) xflag[threadIdx.x] = 0u;  // ordered by the barrier below

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
  // 1. bit planes of a batch of groups: each plane word is one ballot over
  //    64 activations (groups b0, b0 + nw, ..., this wave's share); from
  //    two rows on (one row per lane) the group's activation bytes
  //    themselves, in matrix-core order (kBytes)
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
      const uint32_t a0 = (uint8_t)y0[i], a1 = (uint8_t)y1[i];
      uint4 mine = make_uint4(0u, 0u, 0u, 0u);
      int cgroup = 0;
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        const uint64_t b0 = ballot((a0 >> p) & 1u), b1 = ballot((a1 >> p) & 1u);
        if (lane == p)
          mine = make_uint4((uint32_t)b0, (uint32_t)(b0 >> 32), (uint32_t)b1, (uint32_t)(b1 >> 32));
        cgroup += (p == 7 ? -128 : 1 << p) * (__popcll(b0) + __popcll(b1));
      }
      if constexpr (kBytes) {  // the activation bytes themselves, in matrix-core order
        uint8_t* slot = reinterpret_cast<uint8_t*>(&pgs[mg]);
        slot[act_byte_slot((uint32_t)lane)] = (uint8_t)a0;
        slot[act_byte_slot(64u + (uint32_t)lane)] = (uint8_t)a1;
      } else {
        if (lane < 8) pgs[mg].plane[lane] = mine;
      }
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
  // row scales: lane m holds row m's (a per-lane load: a scalar load would
  // hold up the barrier below, which waits for every scalar load, by a full
  // memory round trip)
  const float act_sv = a.act_scale[lane < M ? lane : M - 1];
  // lane m: row m's temperature (the draw's logit scale for the normaliser)
  const float temp_v = kSample ? row_temperature(a.out, lane < M ? lane : M - 1, a.act_scale) : 1.f;
  // the call's bitmask bits of this lane's rows, per activation row
  uint32_t allow[M];
  {
    int64_t rows[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t v = (tile0 + r) * 64 + lane;
      rows[r] = v < a.V ? v : a.V - 1;
    }
#pragma unroll
    for (int m = 0; m < M; ++m)
      allow[m] = kExtras ? allowed_bits<R>(a.out, m, rows, a.act_scale) : 0xFFFFFFFFu;
  }
  __builtin_amdgcn_sched_barrier(0);
  // (no barrier here: each wave requests its weights as soon as it has
  // requested its activation bytes, so HBM is busy from the first waves on)

  // 4. first quads of weights (group and quad indices clamped into the head),
  //    issued in the same order as the main loop's refills
  uint4 buf[kQuadBuffers][R][4];
  float4 sbuf[kQuadBuffers][R];
#pragma unroll
  for (int b = 0; b < kQuadBuffers; ++b) {
    const int qc = qa + b < a.Q ? qa + b : a.Q - 1;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      sbuf[b][r] = ld_stream(&sp[r][qc * 64]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int g = 4 * (qa + b) + i;
        buf[b][r][i] = ld_stream(&wp[r][(g < G ? g : G - 1) * 64]);
      }
    }
  }

  __builtin_amdgcn_sched_barrier(0);
  // 5. the first batch's masks, built while the weights are in flight
  build_masks(wave, x0, x1);
  lds_barrier();

  float acc[R][M];  // the running chain
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[r][m] = 0.f;
  // A wave that runs a tile's first chain itself (one wave per tile) parks
  // that chain's sums in LDS until the second chain is done, instead of in
  // registers the main loop needs (at eight rows they cost 5 % in time);
  // slot (wave * R + r, m) of this lane.
  float* park = xch + (size_t)wave * R * M * 64 + lane;
  auto park_chain = [&]() {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int m = 0; m < M; ++m) {
        park[(r * M + m) * 64] = acc[r][m];
        acc[r][m] = 0.f;
      }
  };
  auto after_quad = [&](int qq) {  // a wave running both chains starts the second
    if (qq + 1 == split) park_chain();
  };

  auto compute_group = [&](int g, const uint4 (&w)[R], const float (&s)[R]) {
    if constexpr (kBytes) {
      static_assert(M <= 8, "sums of rows 0-7 come back in two registers");
      uint32_t y0 = w[0].x, y1 = w[0].y, y2 = w[0].z, y3 = w[0].w;
      transpose4(y0, y1, y2, y3);  // y_b: word q of row 16 b + p
      const uint8_t* ag = reinterpret_cast<const uint8_t*>(pgs + (size_t)a_row * G + g) + 32 * (lane >> 4);
      const v4i32_t a0 = *reinterpret_cast<const v4i32_t*>(ag);
      const v4i32_t a1 = *reinterpret_cast<const v4i32_t*>(ag + 16);
      const v4i32_t zero = {0, 0, 0, 0};
      v4i32_t c[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const uint32_t x = b == 0 ? y0 : b == 1 ? y1 : b == 2 ? y2 : y3;
        const v4i32_t lo = {(int)(x & kByteBits), (int)((x >> 1) & kByteBits), (int)((x >> 2) & kByteBits),
                            (int)((x >> 3) & kByteBits)};
        const v4i32_t hi = {(int)((x >> 4) & kByteBits), (int)((x >> 5) & kByteBits),
                            (int)((x >> 6) & kByteBits), (int)((x >> 7) & kByteBits)};
        c[b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, lo, zero, 0, 0, 0);
        c[b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, hi, c[b], 0, 0, 0);
      }
      // activation row 4 j + i of this lane's row: register j of the
      // transpose of (c[0][i], .., c[3][i])
      int d[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t r0 = (uint32_t)c[0][i], r1 = (uint32_t)c[1][i], r2 = (uint32_t)c[2][i], r3 = (uint32_t)c[3][i];
        transpose4(r0, r1, r2, r3);
        d[i] = (int)r0;
        d[4 + i] = (int)r1;
      }
#pragma unroll
      for (int m = 0; m < M; ++m) acc[0][m] = fmaf((float)(2 * d[m] - cg[m * G + g]), s[0], acc[0][m]);
    } else {
#pragma unroll
      for (int m = 0; m < M; ++m) {
        uint32_t u[R];
        plane_dot<R>(w, pgs[(size_t)m * G + g].plane, u);
        const int c = cg[m * G + g];
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r][m] = fmaf((float)(2 * (int)u[r] - c), s[r], acc[r][m]);
      }
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
    const int qe = qb < Qf ? qb : Qf;  // end of this wave's full quads
    int q = qa;
    for (; q + 2 * NB - 1 < qe; q += NB) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        compute_quad(q + b, buf[b], sbuf[b]);
        after_quad(q + b);
        __builtin_amdgcn_sched_barrier(0);
        load_quad(q + b + NB, buf[b], sbuf[b]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // drain: fewer than 2 * NB quads remain
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (q + b < qe) {
        compute_quad(q + b, buf[b], sbuf[b]);
        after_quad(q + b);
        if (q + b + NB < qe) load_quad(q + b + NB, buf[b], sbuf[b]);
      }
    }
#pragma unroll
    for (int b = 0; b < NB; ++b)
      if (q + NB + b < qe) {
        compute_quad(q + NB + b, buf[b], sbuf[b]);
        after_quad(q + NB + b);
      }
    if (qb > Qf) {  // last, partial quad (always in the second chain)
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

  float lo[R][M];  // the first chain
  if (!pair) {
    // parked by this wave (none: an empty first chain, or no tile)
    const bool parked = active && Qh > 0;
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int m = 0; m < M; ++m) lo[r][m] = parked ? park[(r * M + m) * 64] : 0.f;
  } else {
    // each wave of the pair leaves its partial sums of the rows it gives up
    // (the other half of the lanes) in its LDS slot and raises its flag, then
    // takes the partner's; both write before they wait, so the wait ends
    // (bounded all the same)
    const bool keep = (lane < 32) != second;
    float* mine = xch + (size_t)wave * 32 * M + (lane & 31) * M;
    if (!keep) {
#pragma unroll
      for (int m = 0; m < M; ++m) mine[m] = acc[0][m];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    if (lane == 0) *(volatile lds_t<uint32_t>*)&xflag[wave] = 1u;
    for (int spin = 0; spin < kThresholdSpinMax; ++spin) {
      if (uniform(*(volatile lds_t<uint32_t>*)&xflag[wave ^ 1])) break;
      __builtin_amdgcn_s_sleep(1);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    const float* theirs = xch + (size_t)(wave ^ 1) * 32 * M + (lane & 31) * M;
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const float t = theirs[m];
      lo[0][m] = second ? t : acc[0][m];
      acc[0][m] = second ? acc[0][m] : t;
    }
  }
  // the dot part: first chain + second chain
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[r][m] = lo[r][m] + acc[r][m];

  int32_t idx[R];
  uint32_t valid = 0u;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t v = (tile0 + r) * 64 + lane;
    idx[r] = (int32_t)v;
    const bool vv = (tile0 + r) < a.n_tiles && v < a.V && (!pair || (lane < 32) != second);
    valid |= (vv ? 1u : 0u) << r;
    if (a.bias == nullptr || !vv) bias_v[r] = 0.f;
  }
  if constexpr (M == 1) {
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const float s = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(act_sv), m));
      float val[R];
#pragma unroll
      for (int r = 0; r < R; ++r) val[r] = fmaf(acc[r][m], s, bias_v[r]);
      const float zs =
          kSample ? z_scale(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(temp_v), m))) : 1.f;
      chunk_select_write<R, kExtras>(val, idx, valid, m, a.out, ssm, hst, m == M - 1, allow[m], zs);
    }
  } else {
    // every row's selection at once (the small-k stages of all rows share
    // their barriers)
    float val[M][R], zs[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const float s = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(act_sv), m));
#pragma unroll
      for (int r = 0; r < R; ++r) val[m][r] = fmaf(acc[r][m], s, bias_v[r]);
      zs[m] = kSample ? z_scale(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(temp_v), m))) : 1.f;
    }
    chunk_select_rows<R, M, kExtras>(val, idx, valid, a.out, ssm, hst, allow, zs);
  }
  if (a.out.fused)
    fused_merge_tail<kFusedRM, kExtras, kSample, (M >= 2 ? M : 0)>(fused_merge_of(a.out), ssm, csm.fs,
                                                                   last_wg);
}
namespace {

// mode 0: plain; 1: log-sum-exp output or bitmask; 2: also a token draw
// (kernels without them leave that code out)
template <int M, int R>
void (*binary_kernel_mr(int mode))(BinaryArgs) {
  switch (mode) {
    case 0: return k_binary_chunk<M, R, false, false>;
    case 1: return k_binary_chunk<M, R, true, false>;
    case 2: return k_binary_chunk<M, R, true, true>;
  }
  return nullptr;
}
// 2048-row chunks (4 rows per lane) exist for one and two rows only: from
// three rows on their accumulators and weight buffers no longer fit the
// registers (the host refuses that option there).
template <int M>
void (*binary_kernel_m(int rpl, int mode))(BinaryArgs) {
  if (rpl == 1) return binary_kernel_mr<M, 1>(mode);
  if constexpr (M <= kMaxRowsWide) {
    if (rpl == 4) return binary_kernel_mr<M, 4>(mode);
  }
  return nullptr;
}

void (*binary_kernel(int M, int rpl, int mode))(BinaryArgs) {
  switch (M) {
    case 1: return binary_kernel_m<1>(rpl, mode);
    case 2: return binary_kernel_m<2>(rpl, mode);
    case 3: return binary_kernel_m<3>(rpl, mode);
    case 4: return binary_kernel_m<4>(rpl, mode);
    case 5: return binary_kernel_m<5>(rpl, mode);
    case 6: return binary_kernel_m<6>(rpl, mode);
    case 7: return binary_kernel_m<7>(rpl, mode);
    case 8: return binary_kernel_m<8>(rpl, mode);
  }
  return nullptr;
}
}  // namespace

size_t binary_lds_bytes(int64_t M, int64_t H, int ks, int rpl) {
  const int64_t G = H / kGroup;
  const int64_t pair = (int64_t)kPairWaves * (32 * M * 4 + 4);
  // parked first chains: one per wave and row of a lane (16 waves of one
  // row, or 8 waves of four)
  const int64_t parked = (int64_t)(rpl == 1 ? 16 : 32) * M * 64 * 4;
  return (size_t)(M * G * sizeof(PlaneGroup) + M * G * 4 + (ks == 2 ? pair : parked));
}
int launch_binary_chunks(const Geometry& g, const int8_t* act_q, const float* act_scale,
                         const void* wq, const float* wscale, const float* bias, int64_t H,
                         void* workspace, float* values, int64_t* indices, void* stream,
                         void* const* events) {
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
  a.ks = g.ks;
  a.out = chunk_out(g, workspace, values, indices);
  const int mode = g.smp.on ? 2 : (g.lse != nullptr || g.allowed != nullptr) ? 1 : 0;
  auto kern = binary_kernel((int)g.M, g.rpl, mode);
  if (!kern) return (int)hipErrorInvalidValue;
  return (int)launch1(kern, dim3(g.n_chunks), dim3(64 * g.nw),
                      binary_lds_bytes(g.M, H, g.ks, g.rpl), stream, a, events);
}
}  // namespace lmtopk
