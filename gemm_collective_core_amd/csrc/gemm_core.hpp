// Device building blocks of the MFMA contraction kernels (gfx950).
//
// Workgroup: 8 waves = 512 threads, two waves per SIMD, computing a BM x BN
// output tile (256 x 256 or 128 x 256); wave (wm, wn) owns a WTM x WTN
// sub-tile. Two waves per SIMD roughly double the loads a CU keeps in flight,
// and the per-CU load rate is what bounds a GEMM tile on this chip.
//
// K advances in stages of 128 bytes per row (64 bf16/fp16 or 128 int8
// values) held in a two-buffer LDS ring. Loads go straight from global memory
// to LDS (buffer loads with the LDS bit): no staging registers, and lanes
// whose offset lies past the buffer's range write zeros, which pads the K
// tail. The loads of stage i+1 are issued right after the barrier that
// publishes stage i and overlap its MFMAs; each wave then waits only for its
// own loads (vmcnt) before the next barrier.
//
// MFMA shapes: v_mfma_f32_16x16x32_{bf16,f16} and v_mfma_i32_16x16x64_i8.
// Lane l supplies row (l & 15) of A and column (l & 15) of B; the four lane
// groups g = l >> 4 supply four consecutive 16-byte K pieces; the
// accumulator of lane l holds C[4g + i][l & 15], i = 0..3.
//
// LDS layouts (per stage):
//  * A (m, k), and B given as (n, k): one 128-byte row per output row /
//    column, K contiguous; 16-byte chunk c of row r at c ^ ((r ^ (r >> 3)) & 7)
//    so that an operand read (16 rows, one chunk) and a load (8 rows, all
//    chunks) both spread over all banks.
//  * B given row-major as (k, n): kept k-major as loaded (rows of BN
//    elements). Operands come from the transposing LDS reads: within a 16-lane
//    group, ds_read_b64_tr_b16 hands lane i element i mod 4 of the 8-byte
//    pieces read by lanes 4e + i/4 (e = 0..3), and ds_read_b64_tr_b8 element
//    i mod 8 of the pieces read by lanes 2e + i/8 (e = 0..7). So lane j reads
//    k row 4h + (j >> 2), columns 4(j & 3).. (16-bit) or k row 8h + (j >> 1),
//    columns 8(j & 1).. (8-bit), and lane i receives consecutive k values of
//    column i. Rows are swizzled in 32-byte pairs (16-bit) or 16-byte chunks
//    (8-bit) so that the rows one read touches sit on distinct banks.
#pragma once

#include <type_traits>

#include "mc2_common.hpp"

namespace mc2 {

constexpr int kThreads = 512;
constexpr int kKBytes = 128;  // K bytes per row per stage

#define MC2_LDS __attribute__((address_space(3)))
typedef MC2_LDS char lds_t;

template <int BM_, int BN_, int WM_, int WN_>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static_assert(WM * WN == 8, "eight waves per workgroup");
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int FM = WTM / 16, FN = WTN / 16;
  static_assert(FM * 16 * WM == BM && FN * 16 * WN == BN, "tile not divisible");
  static_assert(BN == 256 && BM % 64 == 0, "row-major B loads cover whole 256-column rows");
  static constexpr int kABytes = BM * kKBytes;
  static constexpr int kBBytes = BN * kKBytes;  // same size in both B layouts
  static constexpr int kStageBytes = kABytes + kBBytes;
  static constexpr int kStages = 2;
};

template <Elem E> struct Mma;
template <> struct Mma<Elem::BF16> {
  using acc_t = f32x4_t;
  static __device__ __forceinline__ acc_t run(u32x4_t a, u32x4_t b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(bit_cast<bf16x8_t>(a), bit_cast<bf16x8_t>(b), c,
                                                   0, 0, 0);
  }
};
template <> struct Mma<Elem::F16> {
  using acc_t = f32x4_t;
  static __device__ __forceinline__ acc_t run(u32x4_t a, u32x4_t b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(bit_cast<f16x8_t>(a), bit_cast<f16x8_t>(b), c, 0,
                                                  0, 0);
  }
};
template <> struct Mma<Elem::I8> {
  using acc_t = i32x4_t;
  static __device__ __forceinline__ acc_t run(u32x4_t a, u32x4_t b, acc_t c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(bit_cast<i32x4_t>(a), bit_cast<i32x4_t>(b), c, 0,
                                                 0, 0);
  }
};

// K iteration over nsim stacked shards of k values each.
struct KSpan {
  int64_t k;        // K values per shard
  int64_t a_shard;  // bytes between A shards
  int64_t b_shard;  // bytes between B shards
  int ktiles;       // K stages per shard
  int niters;       // nsim * ktiles
};

// Operand B description for the main loop.
struct BDesc {
  const char* base;
  int64_t ld;  // bytes per stored row
  int64_t n;   // columns of B
};

__device__ __forceinline__ int row_off(int r, int c) {
  return r * kKBytes + ((c ^ ((r ^ (r >> 3)) & 7)) << 4);
}

// k-major swizzles: 16-bit rows (512 bytes) move 32-byte pairs, 8-bit rows
// (256 bytes) move 16-byte chunks.
__device__ __forceinline__ int kmaj_swz16(int kr) { return (kr & 3) | (((kr >> 3) & 1) << 2); }
__device__ __forceinline__ int kmaj_swz8(int kr) { return (kr & 7) | (((kr >> 4) & 1) << 3); }

// Waits for all outstanding LDS reads; the fragments are tied to the wait so
// that no instruction using them is scheduled before it.
template <int N>
__device__ __forceinline__ void lds_wait_tied(u32x4_t (&v)[N]) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" : "+v"(v[i]));
}

// B operand of one 16-column block from the k-major layout for k-step ks.
// The transposing reads are inline assembly: the compiler cannot tell that
// they do not overlap the LDS stage still being filled by in-flight loads and
// would otherwise wait for those. Results are consumed after lds_wait_tied().
template <Elem E>
__device__ __forceinline__ u32x4_t read_b_kmaj(const lds_t* lB, int ks, int n0, int lane) {
  const int g = lane >> 4, j = lane & 15;
  u32x4_t out;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    int off;
    if constexpr (ElemInfo<E>::bytes == 2) {
      const int kr = ks * 32 + g * 8 + h * 4 + (j >> 2);
      off = kr * 512 + (((n0 >> 4) ^ kmaj_swz16(kr)) << 5) + ((j & 3) << 3);
    } else {
      const int kr = ks * 64 + g * 16 + h * 8 + (j >> 1);
      off = kr * 256 + (((n0 >> 4) ^ kmaj_swz8(kr)) << 4) + ((j & 1) << 3);
    }
    const uint32_t addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lB + off));
    u32x2_t w;
    if constexpr (ElemInfo<E>::bytes == 2)
      asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(w) : "v"(addr));
    else
      asm volatile("ds_read_b64_tr_b8 %0, %1" : "=v"(w) : "v"(addr));
    out[2 * h] = w[0];
    out[2 * h + 1] = w[1];
  }
  return out;
}

// MFMAs of one K stage (two k-steps) on the wave's FM x FN fragments.
template <Elem E, class TS, bool BT>
__device__ __forceinline__ void mma_stage(const lds_t* lA, const lds_t* lB,
                                          typename Mma<E>::acc_t (&acc)[TS::FM][TS::FN],
                                          int wrow0, int wcol0, int lane) {
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int ch = ks * 4 + (lane >> 4);
    u32x4_t a[TS::FM], b[TS::FN];
#pragma unroll
    for (int fn = 0; fn < TS::FN; ++fn) {
      if constexpr (BT)
        b[fn] = *reinterpret_cast<const MC2_LDS u32x4_t*>(lB + row_off(wcol0 + fn * 16 + (lane & 15), ch));
      else
        b[fn] = read_b_kmaj<E>(lB, ks, wcol0 + fn * 16, lane);
    }
#pragma unroll
    for (int fm = 0; fm < TS::FM; ++fm)
      a[fm] = *reinterpret_cast<const MC2_LDS u32x4_t*>(lA + row_off(wrow0 + fm * 16 + (lane & 15), ch));
    if constexpr (!BT) lds_wait_tied(b);
#pragma unroll
    for (int fm = 0; fm < TS::FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < TS::FN; ++fn)
        acc[fm][fn] = Mma<E>::run(a[fm], b[fn], acc[fm][fn]);
  }
}

constexpr uint32_t kBufFlags = 0x00020000u;  // raw buffer, 32-bit data format
constexpr uint32_t kOffNone = 0x80000000u;   // an offset past every range: loads zero

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const char* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), 0, 0x7ffffff0, kBufFlags);
}

// One 16-byte-per-lane load from `rsrc` at `voff` into LDS at `lds` (wave
// uniform) + 16 * lane.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rsrc, lds_t* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (MC2_LDS void*)lds, 16, voff, 0, 0, 0);
}

// Workgroup barrier that neither waits on outstanding loads nor lets the
// compiler move memory accesses across it.
__device__ __forceinline__ void bar_sync() { asm volatile("s_barrier" ::: "memory"); }

__device__ __forceinline__ void wait_vmcnt0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Main loop over all K stages of all shards. For row-major B, `colmap(c)`
// gives the global column of tile column c (c a multiple of the 16-byte
// column block, clamped to the matrix). Every load instruction moves 1 KiB:
// 8 rows of 128 bytes for A and for B given as (n, k); 2 (16-bit) or 4
// (8-bit) k rows of 256 columns for row-major B. Each wave issues BM/64 A
// loads and 4 B loads per stage.
template <Elem E, bool BT, class TS, class ColMap>
__device__ __forceinline__ void mainloop(lds_t* smem, const char* A, int64_t lda, int64_t row0,
                                         int64_t row_last, const BDesc& B, int64_t col0,
                                         const ColMap& colmap, const KSpan& ks,
                                         typename Mma<E>::acc_t (&acc)[TS::FM][TS::FN]) {
  constexpr int ES = ElemInfo<E>::bytes;
  constexpr int KE = kKBytes / ES;        // K values per stage
  constexpr int CE = 16 / ES;             // K values per 16-byte chunk
  constexpr int NA = TS::BM / 64;         // A loads per wave per stage
  constexpr int NB = 4;                   // B loads per wave per stage
  constexpr int KRI = ES == 2 ? 2 : 4;    // k rows per row-major B load
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wrow0 = (wave / TS::WN) * TS::WTM;
  const int wcol0 = (wave % TS::WN) * TS::WTN;

#pragma unroll
  for (int fm = 0; fm < TS::FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < TS::FN; ++fn) acc[fm][fn] = typename Mma<E>::acc_t{0, 0, 0, 0};

  // Per-lane offsets of this wave's loads: rows are fixed, K moves the base.
  // Row-type loads: lane -> row (lane >> 3), physical chunk lane & 7, holding
  // logical chunk (lane & 7) ^ swizzle (the swizzle is an involution).
  uint32_t a_off[NA], b_off[NB];
  int a_key[NA], b_key[NB];
#pragma unroll
  for (int j = 0; j < NA; ++j) {
    const int r = 8 * (NA * wave + j) + (lane >> 3);
    const int c = (row_off(r, lane & 7) - r * kKBytes) >> 4;
    int64_t gr = row0 + r;
    gr = gr < row_last ? gr : row_last;
    a_off[j] = static_cast<uint32_t>((gr - row0) * lda + c * 16);
    a_key[j] = c * CE;
  }
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    if constexpr (BT) {
      const int r = 8 * (NB * wave + j) + (lane >> 3);
      const int c = (row_off(r, lane & 7) - r * kKBytes) >> 4;
      int64_t gc = col0 + r;
      gc = gc < B.n - 1 ? gc : B.n - 1;
      b_off[j] = static_cast<uint32_t>((gc - col0) * B.ld + c * 16);
      b_key[j] = c * CE;
    } else if constexpr (ES == 2) {
      const int kr = 2 * (NB * wave + j) + (lane >> 5);
      const int pc = lane & 31;
      const int ch = ((((pc >> 1) ^ kmaj_swz16(kr))) << 1) | (pc & 1);
      b_off[j] = static_cast<uint32_t>(kr * B.ld + colmap(ch * 8) * 2);
      b_key[j] = kr;
    } else {
      const int kr = 4 * (NB * wave + j) + (lane >> 4);
      const int ch = (lane & 15) ^ kmaj_swz8(kr);
      b_off[j] = static_cast<uint32_t>(kr * B.ld + colmap(ch * 16));
      b_key[j] = kr;
    }
  }
  const char* a_base = A + row0 * lda;
  const char* b_base = BT ? B.base + col0 * B.ld : B.base;

  auto issue = [&](int it) {
    const int w = it / ks.ktiles;
    const int kt = it - w * ks.ktiles;
    const int64_t kdone = static_cast<int64_t>(kt) * KE;
    const int64_t kleft = ks.k - kdone;  // K values left in this shard
    lds_t* st = smem + (it & 1) * TS::kStageBytes;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(a_base + w * ks.a_shard + kdone * ES);
#pragma unroll
    for (int j = 0; j < NA; ++j)
      dma16(ra, st + 8 * (NA * wave + j) * kKBytes, a_key[j] < kleft ? a_off[j] : kOffNone);
    if constexpr (BT) {
      const __amdgpu_buffer_rsrc_t rb = make_rsrc(b_base + w * ks.b_shard + kdone * ES);
#pragma unroll
      for (int j = 0; j < NB; ++j)
        dma16(rb, st + TS::kABytes + 8 * (NB * wave + j) * kKBytes,
              b_key[j] < kleft ? b_off[j] : kOffNone);
    } else {
      const __amdgpu_buffer_rsrc_t rb = make_rsrc(b_base + w * ks.b_shard + kdone * B.ld);
#pragma unroll
      for (int j = 0; j < NB; ++j)
        dma16(rb, st + TS::kABytes + KRI * (NB * wave + j) * (TS::BN * ES),
              b_key[j] < kleft ? b_off[j] : kOffNone);
    }
  };

  const int n = ks.niters;
  issue(0);
  for (int it = 0; it < n; ++it) {
    wait_vmcnt0();  // this wave's loads of stage `it` have landed
    bar_sync();     // ... and every wave's; stage it-1 is no longer read
    if (it + 1 < n) issue(it + 1);
    const lds_t* cur = smem + (it & 1) * TS::kStageBytes;
    mma_stage<E, TS, BT>(cur, cur + TS::kABytes, acc, wrow0, wcol0, lane);
  }
  bar_sync();
}

// Staged tile -> global with 16-byte coalesced stores; rows >= nrows and bytes
// >= row_bytes_valid of each destination row are skipped.
__device__ __forceinline__ void store_staged(const lds_t* smem, int pitch, int tile_row_bytes,
                                             int tile_rows, char* out, int64_t ldo, int64_t nrows,
                                             int64_t col_byte0, int64_t row_bytes_valid) {
  const int cpr = tile_row_bytes / 16;
  const int total = tile_rows * cpr;
  for (int q = threadIdx.x; q < total; q += kThreads) {
    const int r = q / cpr, c = q - r * cpr;
    if (r < nrows && col_byte0 + c * 16 < row_bytes_valid)
      *reinterpret_cast<u32x4_t*>(out + r * ldo + col_byte0 + c * 16) =
          *reinterpret_cast<const MC2_LDS u32x4_t*>(smem + r * pitch + c * 16);
  }
}

}  // namespace mc2
