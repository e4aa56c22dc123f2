// lmtopk_dense.hip - dense-head chunk kernel (gfx950) and its launcher.
//
// k_dense_chunk: fp32 or bf16 head (lm-head-topk page, section "Usage",
// dense entry point), one workgroup per vocabulary chunk, scores in LDS,
// then the same per-chunk exact top-k as the binary path.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

#include "lmtopk_chunk.hpp"

namespace lmtopk {

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
  __shared__ ChunkSmem csm;
  __shared__ uint32_t last_wg;
  HeadStage& hst = csm.hs;
  head_stage_init(hst);  // ordered by the barriers below
  float* scores = reinterpret_cast<float*>(dyn_lds);  // [M][C]
  const int C = a.chunk_rows;
  const int lane = lane_id();
  const int wave = wave_id();
  const int esz = BF16 ? 2 : 4;
  const int64_t nvec = a.H * esz / 16;
  const int64_t row_bytes = a.H * esz;
  const int64_t base = (int64_t)blockIdx.x * C;
  const int rows_per_wave = 64 * RPL;
  // lane m: row m's temperature (the draw's logit scale for the normaliser)
  const float temp_v = row_temperature(a.out, lane < M ? lane : M - 1, reinterpret_cast<const float*>(a.hidden));

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
    int64_t rows[RPL];
#pragma unroll
    for (int r = 0; r < RPL; ++r) rows[r] = ((valid >> r) & 1u) ? (int64_t)idx[r] : 0;
    const uint32_t allow = allowed_bits<RPL>(a.out, m, rows, a.hidden);
    const float zs = z_scale(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(temp_v), m)));
    chunk_select_write<RPL>(val, idx, valid, m, a.out, ssm, hst, m == M - 1, allow, zs);
  }
  if (a.out.fused) fused_merge_tail<kFusedRM>(fused_merge_of(a.out), ssm, csm.fs, last_wg);
}
namespace {

template <int M, bool BF16>
void (*dense_kernel_mb(int rpl))(DenseArgs) {
  switch (rpl) {
    case 1: return k_dense_chunk<M, BF16, 1>;
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
}  // namespace

size_t dense_lds_bytes(int64_t M, int chunk_rows) { return (size_t)(M * chunk_rows * 4); }
int launch_dense_chunks(const Geometry& g, const void* hidden, const void* weight, int is_bf16,
                        const float* bias, int64_t H, void* workspace, float* values,
                        int64_t* indices, void* stream, void* const* events) {
  DenseArgs a;
  a.hidden = static_cast<const uint8_t*>(hidden);
  a.weight = static_cast<const uint8_t*>(weight);
  a.bias = bias;
  a.V = g.V;
  a.H = H;
  a.chunk_rows = g.chunk_rows;
  a.out = chunk_out(g, workspace, values, indices);
  auto kern = is_bf16 ? dense_kernel_b<true>((int)g.M, g.rpl) : dense_kernel_b<false>((int)g.M, g.rpl);
  if (!kern) return (int)hipErrorInvalidValue;
  return (int)launch1(kern, dim3(g.n_chunks), dim3(64 * g.nw), dense_lds_bytes(g.M, g.chunk_rows),
                      stream, a, events);
}
}  // namespace lmtopk
