// Eight-wave MFMA main loop for 16-bit inputs (gfx950).
//
// One workgroup = 8 waves = 512 threads, two waves per SIMD, computes a
// BM x BN tile (typically 256 x 256; each wave a (BM/WM) x (BN/WN) sub-tile).
// Two waves per SIMD double the loads each CU keeps in flight, which is what
// bounds a GEMM tile on this chip: one CU sustains roughly twice the L2/MALL
// read bandwidth with eight waves as with four.
//
// K advances in stages of 32 elements (64 bytes per row) held in a ring of 4
// LDS buffers. Loads go straight from global memory to LDS (buffer loads with
// the LDS bit: no registers, and lanes past a buffer's range write zeros,
// which pads the K tail); three stages are in flight while one is consumed.
// Each wave waits only for its own loads of the stage it is about to read
// (vmcnt), then one workgroup barrier per stage both publishes the stage and
// frees the buffer that the next load overwrites.
//
// LDS layouts:
//  * A (m, k) and B given as (n, k): one 64-byte row per output row/column,
//    16-byte chunk c of row r stored at c ^ ((r >> 2) & 3) -- the MFMA
//    operand is one 16-byte read, conflict-free for 16 consecutive rows.
//  * B given row-major as (k, n): kept k-major as loaded (32 rows of BN*2
//    bytes); 32-byte pair q of row k stored at q ^ s(k), s(k) = (k & 3) |
//    (((k >> 3) & 1) << 2) (k & 3 for rows of fewer than 8 pairs), which keeps
//    the 16-lane groups of a transposing read on distinct banks. The operand
//    of lane (i, g) -- column i, k values
//    8g..8g+7 -- comes from two ds_read_b64_tr_b16: within a 16-lane group,
//    lane j reads 4 consecutive columns 4(j&3).. of row 4h + (j >> 2), and the
//    transposing read hands lane i the 4 k values of column i.
#pragma once

#include "gemm_core.hpp"

namespace mc2 {

constexpr int kThreads8 = 512;

template <int BM_, int BN_, int WM_, int WN_, int KR_ = 128, int S_ = 2>
struct Tile8 {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static_assert(WM * WN == 8, "eight waves per workgroup");
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int FM = WTM / 16, FN = WTN / 16;
  static_assert(FM * 16 * WM == BM && FN * 16 * WN == BN, "tile not divisible");
  static_assert(BN % 128 == 0 && BM % 128 == 0, "tile sizes");
  static constexpr int kRow = KR_;                // bytes of K per row per stage (64 or 128)
  static constexpr int kKE = KR_ / 2;             // K values per stage
  static constexpr int kSteps = kKE / 32;         // MFMA k-steps per stage
  static constexpr int kABytes = BM * kRow;
  static constexpr int kBBytes = BN * kRow;       // same size in both B layouts
  static constexpr int kStageBytes = kABytes + kBBytes;
  static constexpr int kStages = S_;
  static_assert(KR_ == 64 || KR_ == 128, "stage depth");
};

// Byte offset of 16-byte chunk c of row r in a K-contiguous stage with rows of
// KR bytes: 128-byte rows swizzle c ^ ((r ^ (r >> 3)) & 7), 64-byte rows
// c ^ ((r >> 2) & 3); both keep 16 consecutive rows reading the same logical
// chunk on distinct banks.
template <int KR>
__device__ __forceinline__ int row_off(int r, int c) {
  if constexpr (KR == 128) return r * 128 + ((c ^ ((r ^ (r >> 3)) & 7)) << 4);
  else return r * 64 + ((c ^ ((r >> 2) & 3)) << 4);
}

// K-major B layout (row-major (k, n) input): pair swizzle of k row kr. Rows
// of at least 8 pairs (BN % 128 == 0) use 3 bits, narrower rows 2 bits.
template <int BN>
__device__ __forceinline__ int kmaj_swz(int kr) {
  if constexpr (BN % 128 == 0) return (kr & 3) | (((kr >> 3) & 1) << 2);
  else return kr & 3;
}
// Byte offset of 16-byte chunk ch of k row kr.
template <int BN>
__device__ __forceinline__ int kmaj_off(int kr, int ch) {
  return kr * (BN * 2) + ((((ch >> 1) ^ kmaj_swz<BN>(kr)) << 1) | (ch & 1)) * 16;
}

// B operand of one 16-column block from the k-major layout: two transposing
// 64-bit reads (k values 8g..8g+3 and 8g+4..8g+7 of column n0 + (lane & 15)).
// The reads are issued as inline assembly: the compiler cannot tell that they
// do not overlap the LDS stages still being filled by in-flight loads and
// would otherwise wait for all of them. Their results are consumed only after
// lds_wait_tied() below.
template <int BN>
__device__ __forceinline__ u32x4_t read_b_kmaj(const lds_t* lB, int ks, int n0, int lane) {
  const int g = lane >> 4, j = lane & 15;
  const int q = n0 >> 4;
  u32x4_t out;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int kr = ks * 32 + g * 8 + h * 4 + (j >> 2);
    const int off = kr * (BN * 2) + ((q ^ kmaj_swz<BN>(kr)) << 5) + ((j & 3) << 3);
    const uint32_t addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lB + off));
    u32x2_t w;
    asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(w) : "v"(addr));
    out[2 * h] = w[0];
    out[2 * h + 1] = w[1];
  }
  return out;
}

// Waits for all outstanding LDS reads; the fragments are tied to the wait so
// that no instruction using them is scheduled before it.
template <int N>
__device__ __forceinline__ void lds_wait_tied(u32x4_t (&v)[N]) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" : "+v"(v[i]));
}

// MFMAs of one K stage on the wave's FM x FN fragments.
template <Elem E, class TS, bool BT>
__device__ __forceinline__ void mma_stage8(const lds_t* lA, const lds_t* lB,
                                           f32x4_t (&acc)[TS::FM][TS::FN], int wrow0, int wcol0,
                                           int lane) {
#pragma unroll
  for (int ks = 0; ks < TS::kSteps; ++ks) {
    const int ch = ks * 4 + (lane >> 4);
    u32x4_t a[TS::FM], b[TS::FN];
#pragma unroll
    for (int fn = 0; fn < TS::FN; ++fn) {
      if constexpr (BT)
        b[fn] = *reinterpret_cast<const MC2_LDS u32x4_t*>(
            lB + row_off<TS::kRow>(wcol0 + fn * 16 + (lane & 15), ch));
      else
        b[fn] = read_b_kmaj<TS::BN>(lB, ks, wcol0 + fn * 16, lane);
    }
#pragma unroll
    for (int fm = 0; fm < TS::FM; ++fm)
      a[fm] = *reinterpret_cast<const MC2_LDS u32x4_t*>(
          lA + row_off<TS::kRow>(wrow0 + fm * 16 + (lane & 15), ch));
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
__device__ __forceinline__ void bar_sync() {
  asm volatile("s_barrier" ::: "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N == 0 || N == 4 || N == 8 || N == 16, "vmcnt");
  if constexpr (N == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  else if constexpr (N == 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
  else if constexpr (N == 8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
}

// Main loop over all K stages of all shards (see KSpan). For row-major B,
// `colmap(c)` gives the global column of tile column c (c a multiple of 8).
// Every load instruction moves 1 KiB (64 lanes x 16 bytes): RPI rows of kRow
// bytes for A and for B given as (n, k), two k rows of BN columns for
// row-major B; each wave issues NA + NB of them per stage.
template <Elem E, bool BT, class TS, class ColMap>
__device__ __forceinline__ void mainloop8(lds_t* smem, const char* A, int64_t lda, int64_t row0,
                                          int64_t row_last, const BDesc& B, int64_t col0,
                                          const ColMap& colmap, const KSpan& ks,
                                          f32x4_t (&acc)[TS::FM][TS::FN]) {
  static_assert(ElemInfo<E>::bytes == 2, "16-bit inputs");
  constexpr int KR = TS::kRow, KE = TS::kKE, S = TS::kStages;
  constexpr int RPI = 1024 / KR;                 // rows per load instruction
  constexpr int LPR = KR / 16;                   // lanes per row
  constexpr int NA = TS::BM / RPI / 8;           // A loads per wave per stage
  constexpr int NBT = TS::BN / RPI / 8;          // B (n, k) loads per wave per stage
  constexpr int NBN = KE / 2 / 8;                // B (k, n) loads per wave per stage
  static_assert(TS::BN == 256, "row-major B loads cover two k rows of 256 columns");
  constexpr int NB = BT ? NBT : NBN;
  constexpr int D = NA + NB;                     // loads per wave per stage
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wrow0 = (wave / TS::WN) * TS::WTM;
  const int wcol0 = (wave % TS::WN) * TS::WTN;

#pragma unroll
  for (int fm = 0; fm < TS::FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < TS::FN; ++fn) acc[fm][fn] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Per-lane offsets of this wave's loads (rows fixed; K moves the base).
  uint32_t a_off[NA], b_off[NB];
  int a_key[NA], b_key[NB];
#pragma unroll
  for (int j = 0; j < NA; ++j) {
    const int r = RPI * (NA * wave + j) + lane / LPR;
    const int pc = lane % LPR;
    const int c = (row_off<KR>(r, pc) - r * KR) >> 4;  // swizzle is an involution
    int64_t gr = row0 + r;
    gr = gr < row_last ? gr : row_last;
    a_off[j] = static_cast<uint32_t>((gr - row0) * lda + c * 16);
    a_key[j] = c;
  }
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    if constexpr (BT) {
      const int r = RPI * (NB * wave + j) + lane / LPR;
      const int pc = lane % LPR;
      const int c = (row_off<KR>(r, pc) - r * KR) >> 4;
      int64_t gc = col0 + r;
      gc = gc < B.n - 1 ? gc : B.n - 1;
      b_off[j] = static_cast<uint32_t>((gc - col0) * B.ld + c * 16);
      b_key[j] = c;
    } else {
      const int kr = 2 * (NB * wave + j) + (lane >> 5);
      const int pc = lane & 31;
      const int ch = ((((pc >> 1) ^ kmaj_swz<TS::BN>(kr))) << 1) | (pc & 1);
      const int64_t gcol = colmap(ch * 8);
      b_off[j] = static_cast<uint32_t>(kr * B.ld + gcol * 2);
      b_key[j] = kr;
    }
  }
  const char* a_base = A + row0 * lda;
  const char* b_base = BT ? B.base + col0 * B.ld : B.base;

  auto issue = [&](int it) {
    const int w = it / ks.ktiles;
    const int kt = it - w * ks.ktiles;
    const int64_t kdone = static_cast<int64_t>(kt) * KE;
    lds_t* st = smem + (it % S) * TS::kStageBytes;
    const int64_t kleft = ks.k - kdone;  // K values left in this shard
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(a_base + w * ks.a_shard + kdone * 2);
#pragma unroll
    for (int j = 0; j < NA; ++j)
      dma16(ra, st + RPI * (NA * wave + j) * KR, a_key[j] * 8 < kleft ? a_off[j] : kOffNone);
    if constexpr (BT) {
      const __amdgpu_buffer_rsrc_t rb = make_rsrc(b_base + w * ks.b_shard + kdone * 2);
#pragma unroll
      for (int j = 0; j < NB; ++j)
        dma16(rb, st + TS::kABytes + RPI * (NB * wave + j) * KR,
              b_key[j] * 8 < kleft ? b_off[j] : kOffNone);
    } else {
      const __amdgpu_buffer_rsrc_t rb = make_rsrc(b_base + w * ks.b_shard + kdone * B.ld);
#pragma unroll
      for (int j = 0; j < NB; ++j)
        dma16(rb, st + TS::kABytes + 2 * (NB * wave + j) * (TS::BN * 2),
              b_key[j] < kleft ? b_off[j] : kOffNone);
    }
  };

  const int n = ks.niters;
#pragma unroll
  for (int p = 0; p < S - 1; ++p)
    if (p < n) issue(p);
  for (int it = 0; it < n; ++it) {
    // Own loads of stage `it` done; the stages issued after it may stay in flight.
    if constexpr (S == 4) {
      if (it + 2 < n) wait_vmcnt<2 * D>();
      else if (it + 1 < n) wait_vmcnt<D>();
      else wait_vmcnt<0>();
    } else if constexpr (S == 3) {
      if (it + 1 < n) wait_vmcnt<D>();
      else wait_vmcnt<0>();
    } else {
      wait_vmcnt<0>();
    }
    bar_sync();
    if (it + S - 1 < n) issue(it + S - 1);
    const lds_t* cur = smem + (it % S) * TS::kStageBytes;
    mma_stage8<E, TS, BT>(cur, cur + TS::kABytes, acc, wrow0, wcol0, lane);
  }
  bar_sync();
}

// Staged tile -> global with 16-byte coalesced stores, 512 threads.
__device__ __forceinline__ void store_staged8(const lds_t* smem, int pitch, int tile_row_bytes,
                                              int tile_rows, char* out, int64_t ldo, int64_t nrows,
                                              int64_t col_byte0, int64_t row_bytes_valid) {
  const int cpr = tile_row_bytes / 16;
  const int total = tile_rows * cpr;
  for (int q = threadIdx.x; q < total; q += kThreads8) {
    const int r = q / cpr, c = q - r * cpr;
    if (r < nrows && col_byte0 + c * 16 < row_bytes_valid)
      *reinterpret_cast<u32x4_t*>(out + r * ldo + col_byte0 + c * 16) =
          *reinterpret_cast<const MC2_LDS u32x4_t*>(smem + r * pitch + c * 16);
  }
}

}  // namespace mc2
