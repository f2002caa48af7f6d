// Device building blocks of the MFMA contraction kernels (gfx950).
//
// One workgroup = 4 waves = 256 threads computes a BM x BN output tile. K is
// consumed in tiles of 128 bytes per row (64 bf16/fp16 or 128 int8 values),
// staged through LDS in two buffers so that the global loads of tile i+1 are
// in flight while the MFMAs of tile i run.
//
// LDS layout of one operand tile: one 128-byte row per output row (A) or per
// output column (B), K contiguous inside the row, so that every MFMA operand
// is a single 16-byte LDS read. The eight 16-byte chunks of row r are stored
// at chunk position c ^ ((r ^ (r >> 3)) & 7): eight consecutive rows reading
// the same logical chunk hit eight different bank groups (the MFMA operand
// reads), and so do rows 8 apart writing the same chunk (the transposing
// store of a row-major B, whose lanes own columns 8 or 16 apart).
//
// MFMA shapes: v_mfma_f32_16x16x32_{bf16,f16} and v_mfma_i32_16x16x64_i8. For
// both, lane l supplies row (l & 15) of A and column (l & 15) of B, and lanes
// l >> 4 = 0..3 supply four consecutive 16-byte K pieces; the accumulator of
// lane l holds C[4*(l >> 4) + i][l & 15], i = 0..3.
#pragma once

#include "mc2_common.hpp"

namespace mc2 {

constexpr int kThreads = 256;
constexpr int kKBytes = 128;

// LDS pointers carry their address space so that every access compiles to a
// ds_read / ds_write (a generic pointer would become a flat access that waits
// on the vector memory counter too).
#define MC2_LDS __attribute__((address_space(3)))
typedef MC2_LDS char lds_t;

template <int BM_, int BN_, int WM_, int WN_>
struct TileShape {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static_assert(WM * WN == 4, "four waves per workgroup");
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int FM = WTM / 16, FN = WTN / 16;
  static_assert(FM * 16 * WM == BM && FN * 16 * WN == BN, "tile not divisible");
  static constexpr int kStageBytes = (BM + BN) * kKBytes;
};

__device__ __forceinline__ int lds_off(int r, int c) {
  return r * kKBytes + ((c ^ ((r ^ (r >> 3)) & 7)) << 4);
}

template <Elem E> struct Mma;
template <> struct Mma<Elem::BF16> {
  using acc_t = f32x4_t;
  static __device__ __forceinline__ acc_t run(u32x4_t a, u32x4_t b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(bit_cast<bf16x8_t>(a), bit_cast<bf16x8_t>(b), c, 0, 0, 0);
  }
};
template <> struct Mma<Elem::F16> {
  using acc_t = f32x4_t;
  static __device__ __forceinline__ acc_t run(u32x4_t a, u32x4_t b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(bit_cast<f16x8_t>(a), bit_cast<f16x8_t>(b), c, 0, 0, 0);
  }
};
template <> struct Mma<Elem::I8> {
  using acc_t = i32x4_t;
  static __device__ __forceinline__ acc_t run(u32x4_t a, u32x4_t b, acc_t c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(bit_cast<i32x4_t>(a), bit_cast<i32x4_t>(b), c, 0, 0, 0);
  }
};

// Loader for an operand whose rows are K-contiguous in memory: A (m, k), and
// B handed over as (n, k). Each thread moves ROWS*8/256 16-byte chunks.
template <int ROWS>
struct RowLoader {
  static constexpr int kPer = ROWS * 8 / kThreads;
  static constexpr int kRowStep = kThreads / 8;
  static_assert(kPer >= 1 && kPer * kThreads == ROWS * 8, "rows per tile");
  const char* ptr[kPer];
  int chunk;
  int row_base;
  u32x4_t v[kPer];

  // Rows row0 + r are clamped to row_last: rows past the end read a valid row
  // whose results are never stored.
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
  // koff: byte offset of the K tile; kvalid: bytes of K left from the tile
  // start (chunks past it load zeros).
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

// Loader for B handed over row-major as (k, n): each thread loads R rows of
// one 16-byte column block and transposes it in registers, so that LDS holds
// B column by column with K contiguous (the same layout as RowLoader).
template <Elem E, int BN>
struct ColLoader {
  static constexpr int ES = ElemInfo<E>::bytes;
  static constexpr int CPB = 16 / ES;         // columns per 16-byte block
  static constexpr int NB = BN / CPB;         // column blocks per tile
  static constexpr int KBLK = kThreads / NB;  // K blocks per tile
  static constexpr int KE = kKBytes / ES;     // K elements per tile
  static constexpr int R = KE / KBLK;         // K rows per thread
  static constexpr int PIECE = R * ES;        // bytes per column piece
  static_assert(NB * KBLK == kThreads && R * KBLK == KE, "B tile split");
  static_assert(PIECE == 4 || PIECE == 8 || PIECE == 16, "piece size");
  const char* ptr;
  int64_t ld;
  int nb, kb;
  u32x4_t v[R];

  static __device__ __forceinline__ int block_of(int tid) { return tid % NB; }

  // col_elem: global column of this thread's first column (already clamped).
  __device__ __forceinline__ void init(const char* base, int64_t ldb, int64_t col_elem, int tid) {
    nb = tid % NB;
    kb = tid / NB;
    ld = ldb;
    ptr = base + col_elem * ES + static_cast<int64_t>(kb * R) * ldb;
  }
  // koff: byte offset of the first K row of the tile; krows: K rows left.
  __device__ __forceinline__ void load(int64_t koff, int64_t krows) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const bool ok = kb * R + r < krows;
      v[r] = ok ? *reinterpret_cast<const u32x4_t*>(ptr + koff + r * ld) : zero_v4();
    }
  }
  __device__ __forceinline__ void store(lds_t* lds) const {
    uint32_t d[R][4];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      d[r][0] = v[r].x; d[r][1] = v[r].y; d[r][2] = v[r].z; d[r][3] = v[r].w;
    }
    const int kbyte = kb * PIECE;
    const int ch = kbyte >> 4, within = kbyte & 15;
#pragma unroll
    for (int j = 0; j < CPB; ++j) {
      uint32_t piece[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int r = 0; r < R; ++r) {
        uint32_t e;
        if constexpr (ES == 2)
          e = (d[r][j >> 1] >> ((j & 1) * 16)) & 0xFFFFu;
        else
          e = (d[r][j >> 2] >> ((j & 3) * 8)) & 0xFFu;
        const int bit = r * ES * 8;
        piece[bit >> 5] |= e << (bit & 31);
      }
      lds_t* dst = lds + lds_off(nb * CPB + j, ch) + within;
      if constexpr (PIECE == 16)
        *reinterpret_cast<MC2_LDS u32x4_t*>(dst) = u32x4_t{piece[0], piece[1], piece[2], piece[3]};
      else if constexpr (PIECE == 8)
        *reinterpret_cast<MC2_LDS u32x2_t*>(dst) = u32x2_t{piece[0], piece[1]};
      else
        *reinterpret_cast<MC2_LDS uint32_t*>(dst) = piece[0];
    }
  }
};

// MFMAs of one 128-byte K tile on the wave's FM x FN fragments.
template <Elem E, class TS>
__device__ __forceinline__ void mma_ktile(const lds_t* lA, const lds_t* lB,
                                          typename Mma<E>::acc_t (&acc)[TS::FM][TS::FN],
                                          int wrow0, int wcol0, int lane) {
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int ch = ks * 4 + (lane >> 4);
    u32x4_t a[TS::FM], b[TS::FN];
#pragma unroll
    for (int fm = 0; fm < TS::FM; ++fm)
      a[fm] = *reinterpret_cast<const MC2_LDS u32x4_t*>(lA + lds_off(wrow0 + fm * 16 + (lane & 15), ch));
#pragma unroll
    for (int fn = 0; fn < TS::FN; ++fn)
      b[fn] = *reinterpret_cast<const MC2_LDS u32x4_t*>(lB + lds_off(wcol0 + fn * 16 + (lane & 15), ch));
#pragma unroll
    for (int fm = 0; fm < TS::FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < TS::FN; ++fn)
        acc[fm][fn] = Mma<E>::run(a[fm], b[fn], acc[fm][fn]);
  }
}

// K iteration over nsim stacked shards of k values each.
struct KSpan {
  int64_t k;          // K elements per shard
  int64_t a_shard;    // bytes between A shards
  int64_t b_shard;    // bytes between B shards
  int ktiles;         // K tiles per shard
  int niters;         // nsim * ktiles
};

// Operand B description for the main loop.
struct BDesc {
  const char* base;
  int64_t ld;     // bytes per stored row
  int64_t n;      // columns of B
};

// The main loop: accumulates A[row0.., :] x B[:, cols of this tile] over all
// K tiles of all shards. For B row-major (k, n) (BT == false) `colmap(j)`
// gives the global column of tile column j (j a multiple of the column block);
// for B as (n, k) (BT == true) tile column j is global column col0 + j.
template <Elem E, bool BT, class TS, class ColMap>
__device__ __forceinline__ void mainloop(lds_t* smem, const char* A, int64_t lda, int64_t row0,
                                         int64_t row_last, const BDesc& B, int64_t col0,
                                         const ColMap& colmap, const KSpan& ks,
                                         typename Mma<E>::acc_t (&acc)[TS::FM][TS::FN]) {
  constexpr int ES = ElemInfo<E>::bytes;
  constexpr int KE = kKBytes / ES;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wrow0 = (wave / TS::WN) * TS::WTM;
  const int wcol0 = (wave % TS::WN) * TS::WTN;

#pragma unroll
  for (int fm = 0; fm < TS::FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < TS::FN; ++fn)
      acc[fm][fn] = typename Mma<E>::acc_t{0, 0, 0, 0};

  RowLoader<TS::BM> la;
  la.init(A, lda, row0, row_last, tid);
  using BL = typename std::conditional<BT, RowLoader<TS::BN>, ColLoader<E, TS::BN>>::type;
  BL lb;
  if constexpr (BT) {
    lb.init(B.base, B.ld, col0, B.n - 1, tid);
  } else {
    int64_t c = colmap(BL::block_of(tid) * BL::CPB);
    lb.init(B.base, B.ld, c, tid);
  }


  auto issue = [&](int it) {
    const int w = it / ks.ktiles;
    const int kt = it - w * ks.ktiles;
    const int64_t kdone = static_cast<int64_t>(kt) * KE;
    la.load(w * ks.a_shard + kdone * ES, (ks.k - kdone) * ES);
    if constexpr (BT)
      lb.load(w * ks.b_shard + kdone * ES, (ks.k - kdone) * ES);
    else
      lb.load(w * ks.b_shard + kdone * B.ld, ks.k - kdone);
  };
  auto commit = [&](lds_t* s) {
    la.store(s);
    lb.store(s + TS::BM * kKBytes);
  };

  issue(0);
  commit(smem);
  __syncthreads();
  for (int it = 0; it < ks.niters; ++it) {
    lds_t* cur = smem + (it & 1) * TS::kStageBytes;
    lds_t* nxt = smem + ((it + 1) & 1) * TS::kStageBytes;
    const bool more = it + 1 < ks.niters;
    if (more) issue(it + 1);
    mma_ktile<E, TS>(cur, cur + TS::BM * kKBytes, acc, wrow0, wcol0, lane);
    if (more) commit(nxt);
    __syncthreads();
  }
}

// Copies a staged BM x cols tile (row pitch `pitch` bytes in LDS) to global
// memory with 16-byte coalesced stores; rows >= nrows and columns >= ncols of
// the destination are skipped.
template <int BM>
__device__ __forceinline__ void store_staged(const lds_t* smem, int pitch, int tile_row_bytes,
                                             char* out, int64_t ldo, int64_t nrows,
                                             int64_t col_byte0, int64_t row_bytes_valid) {
  const int cpr = tile_row_bytes / 16;
  const int total = BM * cpr;
  for (int q = threadIdx.x; q < total; q += kThreads) {
    const int r = q / cpr, c = q - r * cpr;
    if (r < nrows && col_byte0 + c * 16 < row_bytes_valid)
      *reinterpret_cast<u32x4_t*>(out + r * ldo + col_byte0 + c * 16) =
          *reinterpret_cast<const MC2_LDS u32x4_t*>(smem + r * pitch + c * 16);
  }
}

}  // namespace mc2
