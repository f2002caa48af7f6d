// Eight-wave MFMA main loop for 16-bit inputs (gfx950).
//
// One workgroup = 8 waves = 512 threads, two waves per SIMD, computes a
// BM x BN tile (typically 256 x 256; each wave a (BM/WM) x (BN/WN) sub-tile).
// Two waves per SIMD double the loads each CU keeps in flight, which is what
// bounds a GEMM tile on this chip: one CU sustains roughly twice the L2/MALL
// read bandwidth with eight waves as with four.
//
// K advances in stages of 64 elements (128 bytes per row), double-buffered in
// LDS: the global loads of stage i+1 go to registers while the MFMAs of stage
// i run, then land in the other LDS buffer.
//
// LDS layouts:
//  * A (m, k) and B given as (n, k): one 128-byte row per output row/column,
//    16-byte chunk c of row r stored at c ^ ((r ^ (r >> 3)) & 7) -- the MFMA
//    operand is one 16-byte read, conflict-free for 16 consecutive rows.
//  * B given row-major as (k, n): kept k-major as loaded (64 rows of BN*2
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

template <int BM_, int BN_, int WM_, int WN_>
struct Tile8 {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static_assert(WM * WN == 8, "eight waves per workgroup");
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int FM = WTM / 16, FN = WTN / 16;
  static_assert(FM * 16 * WM == BM && FN * 16 * WN == BN, "tile not divisible");
  static_assert(BN % 64 == 0, "B rows are whole 128-byte lines");
  static constexpr int kABytes = BM * kKBytes;
  static constexpr int kBBytes = BN * kKBytes;  // same size in both B layouts
  static constexpr int kStageBytes = kABytes + kBBytes;
};

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

// Rows of 128 bytes, K-contiguous (A, or B given as (n, k)); 512 threads.
template <int ROWS>
struct RowLoader8 {
  static constexpr int kPer = ROWS * 8 / kThreads8;
  static constexpr int kRowStep = kThreads8 / 8;
  static_assert(kPer >= 1 && kPer * kThreads8 == ROWS * 8, "rows per tile");
  const char* ptr[kPer];
  int chunk, row_base;
  u32x4_t v[kPer];

  __device__ __forceinline__ void init(const char* base, int64_t ld, int64_t row0,
                                       int64_t row_last, int tid) {
    chunk = tid & 7;
    row_base = tid >> 3;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      int64_t r = row0 + row_base + i * kRowStep;
      r = r < row_last ? r : row_last;
      ptr[i] = base + r * ld + chunk * 16;
    }
  }
  __device__ __forceinline__ void load(int64_t koff, int64_t kvalid) {
    const bool ok = chunk * 16 < kvalid;
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      v[i] = ok ? *reinterpret_cast<const u32x4_t*>(ptr[i] + koff) : zero_v4();
  }
  __device__ __forceinline__ void store(lds_t* lds) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      *reinterpret_cast<MC2_LDS u32x4_t*>(lds + lds_off(row_base + i * kRowStep, chunk)) = v[i];
  }
};

// Row-major (k, n) B of 16-bit elements, stored k-major: 64 k rows of BN
// columns per stage; thread loads 16-byte chunks along n.
template <int BN>
struct KMajLoader8 {
  static constexpr int CPR = BN / 8;                  // chunks per k row
  static constexpr int kPer = 64 * CPR / kThreads8;   // chunks per thread
  static constexpr int kRowStep = kThreads8 / CPR;    // k rows per pass
  static_assert(kPer >= 1 && kPer * kThreads8 == 64 * CPR, "B tile split");
  const char* ptr;
  int64_t ld;
  int ch, kr0;
  u32x4_t v[kPer];

  // col_elem: global column of this thread's chunk (already clamped).
  static __device__ __forceinline__ int chunk_of(int tid) { return tid % CPR; }
  __device__ __forceinline__ void init(const char* base, int64_t ldb, int64_t col_elem, int tid) {
    ch = tid % CPR;
    kr0 = tid / CPR;
    ld = ldb;
    ptr = base + col_elem * 2 + static_cast<int64_t>(kr0) * ldb;
  }
  // koff: byte offset of the first k row of the stage; krows: k rows left.
  __device__ __forceinline__ void load(int64_t koff, int64_t krows) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const bool ok = kr0 + i * kRowStep < krows;
      v[i] = ok ? *reinterpret_cast<const u32x4_t*>(ptr + koff + (int64_t)(i * kRowStep) * ld)
                : zero_v4();
    }
  }
  __device__ __forceinline__ void store(lds_t* lds) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      *reinterpret_cast<MC2_LDS u32x4_t*>(lds + kmaj_off<BN>(kr0 + i * kRowStep, ch)) = v[i];
  }
};

typedef short v4i16_t __attribute__((ext_vector_type(4)));

// B operand of one 16-column block from the k-major layout: two transposing
// 64-bit reads (k values 8g..8g+3 and 8g+4..8g+7 of column n0 + (lane & 15)).
template <int BN>
__device__ __forceinline__ u32x4_t read_b_kmaj(const lds_t* lB, int ks, int n0, int lane) {
  const int g = lane >> 4, j = lane & 15;
  const int q = n0 >> 4;
  u32x4_t out;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int kr = ks * 32 + g * 8 + h * 4 + (j >> 2);
    const int off = kr * (BN * 2) + ((q ^ kmaj_swz<BN>(kr)) << 5) + ((j & 3) << 3);
    const v4i16_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (MC2_LDS v4i16_t*)(const_cast<lds_t*>(lB) + off));
    const u32x2_t w = bit_cast<u32x2_t>(r);
    out[2 * h] = w[0];
    out[2 * h + 1] = w[1];
  }
  return out;
}

// MFMAs of one 128-byte K stage on the wave's FM x FN fragments.
template <Elem E, class TS, bool BT>
__device__ __forceinline__ void mma_stage8(const lds_t* lA, const lds_t* lB,
                                           f32x4_t (&acc)[TS::FM][TS::FN], int wrow0, int wcol0,
                                           int lane) {
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int ch = ks * 4 + (lane >> 4);
    u32x4_t a[TS::FM], b[TS::FN];
#pragma unroll
    for (int fn = 0; fn < TS::FN; ++fn) {
      if constexpr (BT)
        b[fn] = *reinterpret_cast<const MC2_LDS u32x4_t*>(lB + lds_off(wcol0 + fn * 16 + (lane & 15), ch));
      else
        b[fn] = read_b_kmaj<TS::BN>(lB, ks, wcol0 + fn * 16, lane);
    }
#pragma unroll
    for (int fm = 0; fm < TS::FM; ++fm)
      a[fm] = *reinterpret_cast<const MC2_LDS u32x4_t*>(lA + lds_off(wrow0 + fm * 16 + (lane & 15), ch));
#pragma unroll
    for (int fm = 0; fm < TS::FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < TS::FN; ++fn)
        acc[fm][fn] = Mma<E>::run(a[fm], b[fn], acc[fm][fn]);
  }
}

// Main loop over all K stages of all shards (see KSpan). For row-major B,
// `colmap(c)` gives the global column of tile column c (c a multiple of 8).
template <Elem E, bool BT, class TS, class ColMap>
__device__ __forceinline__ void mainloop8(lds_t* smem, const char* A, int64_t lda, int64_t row0,
                                          int64_t row_last, const BDesc& B, int64_t col0,
                                          const ColMap& colmap, const KSpan& ks,
                                          f32x4_t (&acc)[TS::FM][TS::FN]) {
  static_assert(ElemInfo<E>::bytes == 2, "16-bit inputs");
  constexpr int KE = 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wrow0 = (wave / TS::WN) * TS::WTM;
  const int wcol0 = (wave % TS::WN) * TS::WTN;

#pragma unroll
  for (int fm = 0; fm < TS::FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < TS::FN; ++fn) acc[fm][fn] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  RowLoader8<TS::BM> la;
  la.init(A, lda, row0, row_last, tid);
  using BL = typename std::conditional<BT, RowLoader8<TS::BN>, KMajLoader8<TS::BN>>::type;
  BL lb;
  if constexpr (BT)
    lb.init(B.base, B.ld, col0, B.n - 1, tid);
  else
    lb.init(B.base, B.ld, colmap(BL::chunk_of(tid) * 8), tid);

  auto issue = [&](int it) {
    const int w = it / ks.ktiles;
    const int kt = it - w * ks.ktiles;
    const int64_t kdone = static_cast<int64_t>(kt) * KE;
    la.load(w * ks.a_shard + kdone * 2, (ks.k - kdone) * 2);
    if constexpr (BT)
      lb.load(w * ks.b_shard + kdone * 2, (ks.k - kdone) * 2);
    else
      lb.load(w * ks.b_shard + kdone * B.ld, ks.k - kdone);
  };
  auto commit = [&](lds_t* s) {
    la.store(s);
    lb.store(s + TS::kABytes);
  };

  issue(0);
  commit(smem);
  __syncthreads();
  for (int it = 0; it < ks.niters; ++it) {
    lds_t* cur = smem + (it & 1) * TS::kStageBytes;
    lds_t* nxt = smem + ((it + 1) & 1) * TS::kStageBytes;
    const bool more = it + 1 < ks.niters;
    if (more) issue(it + 1);
    mma_stage8<E, TS, BT>(cur, cur + TS::kABytes, acc, wrow0, wcol0, lane);
    if (more) commit(nxt);
    __syncthreads();
  }
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
