// MatmulAllReduce local share: the W partials with one rounding (the chunked
// GEMM over all k-shards) or rounded per rank and combined by ar_sum_kernel,
// for gfx950.
//
// Formulas: "NPU Training Operators - MC2", "底层 API 对照" (npu_mm_all_reduce_base
// fuses the matmul with all_reduce) and "风险" (MC2 may cost precision).
#include "mc2_chunked.hpp"

namespace mc2 {

// ---------------------------------------------------------------- all-reduce sum

// fp64 -> fp32 with rounding to odd (truncate; set the last bit when anything
// was cut off). A following round-to-nearest-even to a format with at least
// two fewer significand bits then rounds the fp64 value correctly (Boldo &
// Melquiond, "Emulation of FMA and correctly rounded sums: proved algorithms
// using rounding to odd").
__device__ __forceinline__ float f64_to_f32_odd(double d) {
  float f = __double2float_rz(d);
  if (static_cast<double>(f) != d) f = __uint_as_float(__float_as_uint(f) | 1u);
  return f;
}

template <Out O>
__device__ __forceinline__ float ar_decode(uint32_t bits) {
  if constexpr (O == Out::BF16) return bf16_bits_to_f32(bits);
  else return f16_bits_to_f32(bits);
}

template <Out O>
__device__ __forceinline__ uint16_t ar_encode(float f) {
  if constexpr (O == Out::BF16) return f32_to_bf16_bits(f);
  else return f32_to_f16_bits(f);
}

// s + p rounded to odd in fp32 (s, p fp32 values): the round-to-nearest sum
// r, its exact error from Knuth's TwoSum, and, when r is inexact and even,
// r's neighbour on the side of the exact sum. A storage format of at most 22
// significand bits then rounds the result to nearest-even exactly as it would
// round the exact sum (Boldo and Melquiond, rounding to odd). An infinite r
// (bf16 operands near the top of the range) is already the correct rounding.
__device__ __forceinline__ float add_round_odd(float s, float p) {
  const float r = s + p;
  if (!__builtin_isfinite(r)) return r;
  const float pv = r - s;
  const float e = (s - (r - pv)) + (p - pv);
  uint32_t b = __float_as_uint(r);
  if (e != 0.0f && !(b & 1u)) b += ((e > 0.0f) == (r > 0.0f)) ? 1u : 0xFFFFFFFFu;
  return __uint_as_float(b);
}

// The all-reduce sum of W stored partials, 8 values (16 bytes) per thread per
// partial; the loads of up to 8 partials are issued before any is used.
// RANK: +0 plus the partials in rank order in fp64, rounded once (the
// fp64 -> fp32 step rounds to odd, so the final rounding is exact). Otherwise
// a running sum rounded to the storage format after every addition.
template <Out O, bool RANK>
__global__ __launch_bounds__(256) void ar_sum_kernel(const uint16_t* __restrict__ parts, int W,
                                                     int64_t elems,
                                                     uint16_t* __restrict__ out) {
  constexpr int G = 8;
  const int64_t n8 = elems / 8;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n8;
       i += static_cast<int64_t>(gridDim.x) * 256) {
    double d[8];
    float f[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) d[j] = 0.0;
    for (int w0 = 0; w0 < W; w0 += G) {
      u32x4_t v[G];
#pragma unroll
      for (int g = 0; g < G; ++g)
        if (w0 + g < W)
          v[g] = __builtin_nontemporal_load(
              reinterpret_cast<const u32x4_t*>(parts + static_cast<int64_t>(w0 + g) * elems) + i);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        if (w0 + g >= W) break;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float x = ar_decode<O>((v[g][j >> 1] >> (16 * (j & 1))) & 0xFFFFu);
          if constexpr (RANK) d[j] += static_cast<double>(x);
          else f[j] = (w0 + g == 0) ? x : ar_decode<O>(ar_encode<O>(add_round_odd(f[j], x)));
        }
      }
    }
    u32x4_t o;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t lo, hi;
      if constexpr (RANK) {
        lo = ar_encode<O>(f64_to_f32_odd(d[2 * q]));
        hi = ar_encode<O>(f64_to_f32_odd(d[2 * q + 1]));
      } else {
        lo = ar_encode<O>(f[2 * q]);
        hi = ar_encode<O>(f[2 * q + 1]);
      }
      o[q] = lo | (hi << 16);
    }
    __builtin_nontemporal_store(o, reinterpret_cast<u32x4_t*>(out) + i);
  }
}

}  // namespace mc2

using namespace mc2;

// ---------------------------------------------------------------- MatmulAllReduce

namespace mc2 {

static int launch_ar_sum(const void* parts, int W, int64_t elems, int dtype, int rounding,
                         void* out, hipStream_t stream) {
  // one 16-byte vector of every partial per thread: many small workgroups keep
  // more loads in flight than a few looping ones (5.7 vs 4.7 TB/s measured on
  // 8 partials of 2^27 elements); the grid-stride loop only covers sizes past
  // the grid limit
  const int64_t n8 = elems / 8;
  int64_t grid = (n8 + 255) / 256;
  const int64_t cap = int64_t{1} << 30;
  grid = grid < 1 ? 1 : (grid > cap ? cap : grid);
  const dim3 g(static_cast<unsigned>(grid)), t(256);
  const auto* p = static_cast<const uint16_t*>(parts);
  auto* o = static_cast<uint16_t*>(out);
  const bool rank = rounding == MC2_AR_RANK_ROUNDED;
  if (dtype == MC2_BF16) {
    if (rank) hipLaunchKernelGGL((ar_sum_kernel<Out::BF16, true>), g, t, 0, stream, p, W, elems, o);
    else hipLaunchKernelGGL((ar_sum_kernel<Out::BF16, false>), g, t, 0, stream, p, W, elems, o);
  } else {
    if (rank) hipLaunchKernelGGL((ar_sum_kernel<Out::F16, true>), g, t, 0, stream, p, W, elems, o);
    else hipLaunchKernelGGL((ar_sum_kernel<Out::F16, false>), g, t, 0, stream, p, W, elems, o);
  }
  return hipGetLastError() == hipSuccess ? MC2_OK : MC2_ERR_HIP;
}

}  // namespace mc2

extern "C" int mc2_ar_sum_local(const void* partials, int world_size, int64_t elems, int dtype,
                                int rounding, void* out, hipStream_t stream) {
  if (!partials || !out) return MC2_ERR_NULL;
  if (world_size < 1 || world_size > 32 || elems <= 0) return MC2_ERR_SHAPE;
  if (dtype != MC2_F16 && dtype != MC2_BF16) return MC2_ERR_DTYPE;
  if (rounding != MC2_AR_RANK_ROUNDED && rounding != MC2_AR_HOP_ROUNDED) return MC2_ERR_SHAPE;
  if (elems % 8 || !aligned16(partials) || !aligned16(out)) return MC2_ERR_ALIGN;
  return launch_ar_sum(partials, world_size, elems, dtype, rounding, out, stream);
}

extern "C" size_t mc2_mm_ar_workspace_size(int64_t m, int64_t n, int world_size, int in_dtype,
                                           int rounding) {
  if (m <= 0 || n <= 0 || !valid_world(world_size)) return 0;
  if (in_dtype != MC2_F16 && in_dtype != MC2_BF16) return 0;
  if (rounding != MC2_AR_RANK_ROUNDED && rounding != MC2_AR_HOP_ROUNDED) return 0;
  return static_cast<size_t>(world_size) * static_cast<size_t>(m) * static_cast<size_t>(n) * 2;
}

extern "C" int mc2_mm_ar_local(const void* x1, const void* x2, int64_t m, int64_t k, int64_t n,
                               int world_size, int x2_trans, int in_dtype, const void* bias,
                               int rounding, void* out, void* workspace, size_t ws_bytes,
                               hipStream_t stream) {
  if (!x1 || !x2 || !out) return MC2_ERR_NULL;
  if (!valid_world(world_size) || m <= 0 || n <= 0 || k <= 0 || k >= 65535) return MC2_ERR_SHAPE;
  if (in_dtype != MC2_F16 && in_dtype != MC2_BF16) return MC2_ERR_DTYPE;
  if (rounding != MC2_AR_ONE_ROUNDING && rounding != MC2_AR_RANK_ROUNDED &&
      rounding != MC2_AR_HOP_ROUNDED)
    return MC2_ERR_SHAPE;
  if (k % 8 || n % 8) return MC2_ERR_ALIGN;
  if (!aligned16(x1) || !aligned16(x2) || !aligned16(out)) return MC2_ERR_ALIGN;
  if (!offsets_fit(k * 2, (x2_trans ? k : n) * 2)) return MC2_ERR_UNSUPPORTED;
  const int W = world_size;
  if (rounding == MC2_AR_ONE_ROUNDING)  // all W partials in one accumulator, all rows kept
    return run_chunked(x1, x2, m, k, n, 1, 0, W, x2_trans, in_dtype, bias, nullptr, nullptr,
                       in_dtype, out, nullptr, nullptr, 0, 1, stream);
  const size_t need = mc2_mm_ar_workspace_size(m, n, W, in_dtype, rounding);
  if (!workspace) return MC2_ERR_NULL;
  if (!aligned16(workspace)) return MC2_ERR_ALIGN;
  if (ws_bytes < need) return MC2_ERR_WORKSPACE;
  // each rank's partial, rounded to in_dtype as it would be sent, then the sum
  for (int w = 0; w < W; ++w) {
    const int st = run_chunked(static_cast<const char*>(x1) + static_cast<int64_t>(w) * m * k * 2,
                               static_cast<const char*>(x2) + static_cast<int64_t>(w) * k * n * 2,
                               m, k, n, 1, 0, 1, x2_trans, in_dtype, bias, nullptr, nullptr,
                               in_dtype, static_cast<char*>(workspace) + static_cast<int64_t>(w) * m * n * 2,
                               nullptr, nullptr, 0, 1, stream);
    if (st) return st;
  }
  return launch_ar_sum(workspace, W, m * n, in_dtype, rounding, out, stream);
}
