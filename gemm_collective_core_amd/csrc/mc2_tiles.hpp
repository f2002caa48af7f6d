// Pieces shared by the kernels built on the contraction main loop: the
// epilogue helpers, the XCD-aware tile order, the tile shapes and the
// host-side shape checks.
#pragma once

#include "../../include/mc2.h"
#include "gemm_core.hpp"
#include "gemm_core_w4.hpp"
#include "mc2_host.hpp"

namespace mc2 {

// ---------------------------------------------------------------- epilogues

template <Out O>
__device__ __forceinline__ void put_out(lds_t* p, float v) {
  if constexpr (O == Out::BF16) *reinterpret_cast<MC2_LDS uint16_t*>(p) = f32_to_bf16_bits(v);
  else if constexpr (O == Out::F16) *reinterpret_cast<MC2_LDS uint16_t*>(p) = f32_to_f16_bits(v);
  else *reinterpret_cast<MC2_LDS float*>(p) = v;
}

template <Out O, class V>
__device__ __forceinline__ void put_out_global(char* p, V v) {
  if constexpr (O == Out::I32) *reinterpret_cast<int32_t*>(p) = v;
  else *reinterpret_cast<float*>(p) = v;
}

template <Elem E>
__device__ __forceinline__ float load_bias(const void* bias, int64_t j) {
  const uint16_t b = static_cast<const uint16_t*>(bias)[j];
  if constexpr (E == Elem::F16) return f16_bits_to_f32(b);
  else return bf16_bits_to_f32(b);  // BF16 inputs, and the bf16 bias of int8 inputs
}

// Elementwise epilogue of the linear kernels: for every accumulator element
// of the wave, computes the output value and hands it with its tile-local row
// and column to `sink`.
//   16-bit inputs: acc + bias_mul * bias[j]  (bias_mul = number of partials)
//   int8 inputs:   (x1_scale[i] * x2_scale[j]) * (float(acc) + bias[j]),
//                  or the raw accumulator for 32-bit integer output
template <Elem E, Out O>
__device__ __forceinline__ float linear_value(float a, float bv, float bias_mul, float sc) {
  if constexpr (E == Elem::I8) return sc * (a + bv);
  else return a + bias_mul * bv;
}

template <Elem E, class TS, Out O, class Sink>
__device__ __forceinline__ void epilogue_linear(const typename Mma<E>::acc_t (&acc)[TS::FM][TS::FN],
                                                int64_t row0, int64_t row_last, int64_t col0,
                                                int64_t n, const void* bias, float bias_mul,
                                                const float* s1, const float* s2, Sink&& sink) {
  using L = AccLayout<TS>;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wrow0 = (wave / TS::WN) * TS::WTM;
  const int wcol0 = (wave % TS::WN) * TS::WTN;
#pragma unroll
  for (int fn = 0; fn < TS::FN; ++fn) {
#pragma unroll
    for (int fm = 0; fm < TS::FM; ++fm) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int lrow = wrow0 + L::row(fm, lane, i);
        const int lcol = wcol0 + L::col(fn, lane, i);
        if constexpr (E == Elem::I8 && O == Out::I32) {
          sink(lrow, lcol, acc[fm][fn][i]);
        } else {
          int64_t gcol = col0 + lcol;
          gcol = gcol < n ? gcol : n - 1;
          const float bv = bias ? load_bias<E>(bias, gcol) : 0.f;
          float sc = 1.f;
          if constexpr (E == Elem::I8) {
            int64_t grow = row0 + lrow;
            grow = grow < row_last ? grow : row_last;
            sc = s1[grow] * s2[gcol];
          }
          sink(lrow, lcol, linear_value<E, O>(static_cast<float>(acc[fm][fn][i]), bv, bias_mul, sc));
        }
      }
    }
  }
}

// The same values for a four-wave tile, whose lanes hold runs of four
// consecutive columns: sink(lrow, lcol, v) receives v[0..3] for columns
// lcol .. lcol + 3 of row lrow (int32 for the raw int8 accumulator, else
// float).
template <Elem E, class TS, Out O, class Sink>
__device__ __forceinline__ void epilogue_quads(const typename Mma<E>::acc_t (&acc)[TS::FM][TS::FN],
                                               int64_t row0, int64_t row_last, int64_t col0,
                                               int64_t n, const void* bias, float bias_mul,
                                               const float* s1, const float* s2, Sink&& sink) {
  static_assert(AccLayout<TS>::kRowRuns, "runs of four columns");
  constexpr bool kRaw = E == Elem::I8 && O == Out::I32;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wrow0 = (wave / TS::WN) * TS::WTM;
  const int wcol0 = (wave % TS::WN) * TS::WTN;
#pragma unroll
  for (int fn = 0; fn < TS::FN; ++fn) {
    const int lcol = wcol0 + fn * 16 + 4 * (lane >> 4);
    float bv[4] = {0.f, 0.f, 0.f, 0.f}, sc2[4] = {1.f, 1.f, 1.f, 1.f};
    if constexpr (!kRaw) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int64_t gcol = col0 + lcol + i;
        gcol = gcol < n ? gcol : n - 1;
        if (bias) bv[i] = load_bias<E>(bias, gcol);
        if constexpr (E == Elem::I8) sc2[i] = s2[gcol];
      }
    }
#pragma unroll
    for (int fm = 0; fm < TS::FM; ++fm) {
      const int lrow = wrow0 + fm * 16 + (lane & 15);
      if constexpr (kRaw) {
        const int32_t v[4] = {acc[fm][fn][0], acc[fm][fn][1], acc[fm][fn][2], acc[fm][fn][3]};
        sink(lrow, lcol, v);
      } else {
        float sc1 = 1.f;
        if constexpr (E == Elem::I8) {
          int64_t grow = row0 + lrow;
          grow = grow < row_last ? grow : row_last;
          sc1 = s1[grow];
        }
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          v[i] = linear_value<E, O>(static_cast<float>(acc[fm][fn][i]), bv[i], bias_mul, sc1 * sc2[i]);
        sink(lrow, lcol, v);
      }
    }
  }
}

// Four 16-bit or 32-bit output values of consecutive columns as one store's
// data (8 or 16 bytes).
template <Out O, class V>
__device__ __forceinline__ auto pack4(const V (&v)[4]) {
  if constexpr (OutInfo<O>::bytes == 2) {
    uint32_t w[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t lo = O == Out::BF16 ? f32_to_bf16_bits(v[2 * j]) : f32_to_f16_bits(v[2 * j]);
      const uint32_t hi = O == Out::BF16 ? f32_to_bf16_bits(v[2 * j + 1]) : f32_to_f16_bits(v[2 * j + 1]);
      w[j] = lo | (hi << 16);
    }
    return u32x2_t{w[0], w[1]};
  } else {
    return u32x4_t{__builtin_bit_cast(uint32_t, v[0]), __builtin_bit_cast(uint32_t, v[1]),
                   __builtin_bit_cast(uint32_t, v[2]), __builtin_bit_cast(uint32_t, v[3])};
  }
}

// Stores four values of consecutive columns at byte offset `off` of `base`:
// non-temporal (the output is not read again here) or, with write_through
// (tiles that raise ready flags), written through to memory so that the
// flag's release has no dirty line of them to write back; `r` is a buffer
// resource at base (every offset below 2^31).
template <Out O, class V>
__device__ __forceinline__ void store4(char* base, __amdgpu_buffer_rsrc_t r, int64_t off,
                                       const V (&v)[4], bool write_through) {
  const auto d = pack4<O>(v);
  if constexpr (OutInfo<O>::bytes == 2) {
    if (write_through)
      __builtin_amdgcn_raw_buffer_store_b64(d, r, static_cast<int>(off), 0, kCpolWriteThrough);
    else
      __builtin_nontemporal_store(d, reinterpret_cast<u32x2_t*>(base + off));
  } else {
    if (write_through)
      __builtin_amdgcn_raw_buffer_store_b128(d, r, static_cast<int>(off), 0, kCpolWriteThrough);
    else
      __builtin_nontemporal_store(d, reinterpret_cast<u32x4_t*>(base + off));
  }
}

// Tile column -> global column of B, clamped to the last 16-byte column block.
struct PlainCols {
  int64_t col0, last_block;
  __device__ __forceinline__ int64_t operator()(int j) const {
    const int64_t c = col0 + j;
    return c < last_block ? c : last_block;
  }
};

// Logical tile of workgroup b. Workgroups are dispatched to the 8 XCDs in
// turn (b mod 8), each XCD with its own L2. Inside every round of `round`
// workgroups (one per CU), XCD x is given the round's logical tiles
// 32x .. 32x+31 (round/8 of them): consecutive tiles, which share rows of A
// and columns of B, then run on the same L2.
__device__ __forceinline__ int xcd_tile(int b, int round, int nblocks) {
  if (round <= 0 || b >= (nblocks / round) * round) return b;
  const int r = b / round, u = b - r * round;
  return r * round + (u & 7) * (round >> 3) + (u >> 3);
}

using TileL = Tile<256, 256, 2, 4>;  // wave sub-tile 128 x 64
using TileM = Tile<128, 256, 2, 4>;  // wave sub-tile 64 x 64, for small tile counts
using TileW = Tile<256, 256, 2, 2>;  // four waves of 128 x 128, operands K-contiguous (B as (n, k))
using TileWM = Tile<128, 256, 2, 2>; // four waves of 64 x 128, for small tile counts

inline bool valid_world(int W) { return W == 1 || W == 2 || W == 4 || W == 8 || W == 16 || W == 32; }

// Per-lane buffer offsets are 32-bit: rows of up to 256 (A, B given as (n, k))
// or 128 (row-major B) per tile must stay below 2^31 bytes.
inline bool offsets_fit(int64_t lda, int64_t ldb) {
  return lda * 256 < 0x7fff0000LL && ldb * 256 < 0x7fff0000LL;
}

}  // namespace mc2
