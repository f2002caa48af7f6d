// Device building blocks of the MFMA contraction kernels (gfx950).
//
// Workgroup: 8 waves = 512 threads, two waves per SIMD, computing a BM x BN
// output tile (256 x 256 or 128 x 256); wave
// (wm, wn) owns a WTM x WTN sub-tile. Two waves per SIMD let one wave's MFMAs run while the other waits
// on its operand reads or on a load instruction the memory pipeline has not
// yet taken.
//
// K advances in stages of 128 bytes per row (64 bf16/fp16 or 128 int8
// values, two MFMA k-steps) held in a two-buffer LDS ring. Loads go straight
// from global memory to LDS (buffer loads with the LDS bit): no staging
// registers, and lanes whose offset lies past the buffer's range write zeros,
// which pads the K tail.
//
// Software pipeline of one stage, per wave (rows = the wave's FM fragment
// rows of 16):
//   k-step 0: row by row, the MFMAs of the row, then the LDS reads of the
//             same row for k-step 1 (B fragments of k-step 1 after row 0);
//   k-step 1: rows 0..S0; then the stage barrier (all reads of this stage
//             done, every wave's loads of the next stage landed), then the
//             reads of the next stage's k-step 0 and, spread over the
//             remaining rows, the loads of the stage after next into the
//             buffer just released.
// So operand reads overlap MFMAs instead of preceding them, and a wave never
// issues a burst of loads: a load instruction stalls its wave until the
// memory pipeline takes it, which in a burst would idle the MFMA unit. Every
// LDS read is inline assembly and waited for with explicit lgkmcnt values
// (LDS returns in order); the compiler does not track these reads.
//
// MFMA shapes: v_mfma_f32_16x16x32_{bf16,f16} and v_mfma_i32_16x16x64_i8.
// Lane l supplies row (l & 15) of A and column (l & 15) of B; the four lane
// groups g = l >> 4 supply four consecutive 16-byte K pieces; the
// accumulator of lane l holds C[4g + i][l & 15], i = 0..3.
//
// LDS layouts (per stage):
//  * A (m, k), and B given as (n, k): one 128-byte row per output row /
//    column, K contiguous; 16-byte chunk c of row r at c ^ ((r >> 1) & 7).
//    The LDS has 64 four-byte banks (256 bytes), so rows r and r + 1 fall on
//    different bank halves; an operand read (16 rows, one logical chunk) then
//    puts the 8 even and the 8 odd rows on 8 distinct chunks each, and never
//    conflicts. Loads write 1 KiB linearly and never conflict either. The
//    swizzle does not depend on the fragment index (rows 16 apart), so all
//    fragment reads of a wave share one address register per k-step.
//  * B given row-major as (k, n): kept k-major as loaded (rows of BN
//    elements). Operands come from the transposing LDS reads: within a 16-lane
//    group, ds_read_b64_tr_b16 hands lane i element i mod 4 of the 8-byte
//    pieces read by lanes 4e + i/4 (e = 0..3), and ds_read_b64_tr_b8 element
//    i mod 8 of the pieces read by lanes 2e + i/8 (e = 0..7). So lane j reads
//    k row 4h + (j >> 2), columns 4(j & 3).. (16-bit) or k row 8h + (j >> 1),
//    columns 8(j & 1).. (8-bit), and lane i receives consecutive k values of
//    column i. Rows are swizzled in 32-byte pairs (16-bit, XOR) or 16-byte
//    chunks (8-bit) so that the rows one read touches sit on distinct banks.
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
  static constexpr int NW = WM * WN;    // waves per workgroup
  static constexpr int NT = NW * 64;    // threads per workgroup
  static_assert(NW == 8 || NW == 4, "eight or four waves per workgroup");
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int FM = WTM / 16, FN = WTN / 16;
  static_assert(FM * 16 * WM == BM && FN * 16 * WN == BN, "tile not divisible");
  static_assert(BN == 256 && BM % 64 == 0, "tile shapes of the load mapping");
  static constexpr int kABytes = BM * kKBytes;
  static constexpr int kBBytes = BN * kKBytes;  // same size in both B layouts
  static constexpr int kStageBytes = kABytes + kBBytes;
  static constexpr int kStages = 2;
};

// Where accumulator element i of fragment (fm, fn) of a lane sits in the
// wave's sub-tile (add wrow0 / wcol0). The eight-wave loop keeps the MFMA's
// own layout: a lane holds one column, four consecutive rows. The four-wave
// loop passes the two operands the other way round (it computes each 16 x 16
// block transposed), so a lane holds four consecutive columns of one row and
// its epilogue can store 8 or 16 contiguous bytes straight from registers.
template <class TS>
struct AccLayout {
  static constexpr bool kRowRuns = TS::NW == 4;
  static __device__ __forceinline__ int row(int fm, int lane, int i) {
    return kRowRuns ? fm * 16 + (lane & 15) : fm * 16 + 4 * (lane >> 4) + i;
  }
  static __device__ __forceinline__ int col(int fn, int lane, int i) {
    return kRowRuns ? fn * 16 + 4 * (lane >> 4) + i : fn * 16 + (lane & 15);
  }
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
  int niters;       // end of the stages run: nsim * ktiles, or less for a K part
  int it0 = 0;      // first stage run (0, or the start of a K part)
};

// Operand B description for the main loop.
struct BDesc {
  const char* base;
  int64_t ld;  // bytes per stored row
  int64_t n;   // columns of B
};

__device__ __forceinline__ int row_off(int r, int c) {
  return r * kKBytes + ((c ^ ((r >> 1) & 7)) << 4);
}

// k-major swizzles: 16-bit rows (512 bytes) move 32-byte pairs, 8-bit rows
// (256 bytes) move 16-byte chunks.
__device__ __forceinline__ int kmaj_swz16(int kr) { return (kr & 3) | (((kr >> 3) & 1) << 2); }

// Position of 32-byte pair p (16 columns) in 16-bit k row kr of a tile BN
// (256) columns wide, and its inverse: XOR with kmaj_swz16 (an involution).
template <int BN>
__device__ __forceinline__ int kmaj_pos16(int p, int kr) {
  static_assert(BN == 256, "512-byte k rows");
  return p ^ kmaj_swz16(kr);
}
template <int BN>
__device__ __forceinline__ int kmaj_unpos16(int pp, int kr) {
  return kmaj_pos16<BN>(pp, kr);
}
__device__ __forceinline__ int kmaj_swz8(int kr) { return (kr & 7) | (((kr >> 4) & 1) << 3); }

// Waits until at most n LDS operations of this wave are outstanding (n is a
// compile-time constant after unrolling; values above 15, the counter's
// range, wait for 15).
__device__ __forceinline__ void lgkm_wait(int n) {
  switch (n < 15 ? n : 15) {
    case 0: asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); break;
    case 1: asm volatile("s_waitcnt lgkmcnt(1)" ::: "memory"); break;
    case 2: asm volatile("s_waitcnt lgkmcnt(2)" ::: "memory"); break;
    case 3: asm volatile("s_waitcnt lgkmcnt(3)" ::: "memory"); break;
    case 4: asm volatile("s_waitcnt lgkmcnt(4)" ::: "memory"); break;
    case 5: asm volatile("s_waitcnt lgkmcnt(5)" ::: "memory"); break;
    case 6: asm volatile("s_waitcnt lgkmcnt(6)" ::: "memory"); break;
    case 7: asm volatile("s_waitcnt lgkmcnt(7)" ::: "memory"); break;
    case 8: asm volatile("s_waitcnt lgkmcnt(8)" ::: "memory"); break;
    case 9: asm volatile("s_waitcnt lgkmcnt(9)" ::: "memory"); break;
    case 10: asm volatile("s_waitcnt lgkmcnt(10)" ::: "memory"); break;
    case 11: asm volatile("s_waitcnt lgkmcnt(11)" ::: "memory"); break;
    case 12: asm volatile("s_waitcnt lgkmcnt(12)" ::: "memory"); break;
    case 13: asm volatile("s_waitcnt lgkmcnt(13)" ::: "memory"); break;
    case 14: asm volatile("s_waitcnt lgkmcnt(14)" ::: "memory"); break;
    default: asm volatile("s_waitcnt lgkmcnt(15)" ::: "memory"); break;
  }
}

// 16-byte operand read; the value is valid only after a matching lgkm_wait.
__device__ __forceinline__ u32x4_t lds_rd128(const lds_t* p) {
  u32x4_t v;
  asm volatile("ds_read_b128 %0, %1"
               : "=v"(v)
               : "v"(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p)))
               : "memory");
  return v;
}

// Half h (k rows 4h.. of each lane group) of the B operand of the 16-column
// block at n0 for k-step ks, from the k-major layout: a transposing read, 8
// bytes per lane; valid after a matching lgkm_wait.
template <Elem E, int BN>
__device__ __forceinline__ u32x2_t lds_rd_tr(const lds_t* lB, int ks, int n0, int h, int lane) {
  const int g = lane >> 4, j = lane & 15;
  int off;
  if constexpr (ElemInfo<E>::bytes == 2) {
    const int kr = ks * 32 + g * 8 + h * 4 + (j >> 2);
    off = kr * (BN * 2) + (kmaj_pos16<BN>(n0 >> 4, kr) << 5) + ((j & 3) << 3);
  } else {
    const int kr = ks * 64 + g * 16 + h * 8 + (j >> 1);
    off = kr * 256 + (((n0 >> 4) ^ kmaj_swz8(kr)) << 4) + ((j & 1) << 3);
  }
  const uint32_t addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lB + off));
  u32x2_t w;
  if constexpr (ElemInfo<E>::bytes == 2)
    asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(w) : "v"(addr) : "memory");
  else
    asm volatile("ds_read_b64_tr_b8 %0, %1" : "=v"(w) : "v"(addr) : "memory");
  return w;
}

// B operand registers of one k-step. B given as (n, k) keeps whole fragments;
// row-major B keeps the two 8-byte halves the transposing reads return, and
// the 16-byte MFMA operand is formed where it is used, after the wait, so
// that no register copy can read a half still in flight.
template <bool BT, int FN> struct BRegs;
template <int FN> struct BRegs<true, FN> {
  static constexpr int kOps = FN;  // LDS reads per k-step
  u32x4_t q[FN];
  __device__ __forceinline__ void tie() {
#pragma unroll
    for (int i = 0; i < FN; ++i) asm volatile("" : "+v"(q[i]));
  }
  __device__ __forceinline__ u32x4_t get(int fn) const { return q[fn]; }
};
template <int FN> struct BRegs<false, FN> {
  static constexpr int kOps = 2 * FN;
  u32x2_t h[FN][2];
  __device__ __forceinline__ void tie() {
#pragma unroll
    for (int i = 0; i < FN; ++i) {
      asm volatile("" : "+v"(h[i][0]));
      asm volatile("" : "+v"(h[i][1]));
    }
  }
  __device__ __forceinline__ u32x4_t get(int fn) const {
    return u32x4_t{h[fn][0][0], h[fn][0][1], h[fn][1][0], h[fn][1][1]};
  }
};

template <Elem E, bool BT, class TS>
__device__ __forceinline__ void read_b_all(BRegs<BT, TS::FN>& b, const lds_t* lB, int ks, int wcol0,
                                           int lane) {
#pragma unroll
  for (int fn = 0; fn < TS::FN; ++fn) {
    if constexpr (BT) {
      b.q[fn] = lds_rd128(lB + row_off(wcol0 + fn * 16 + (lane & 15), ks * 4 + (lane >> 4)));
    } else {
      b.h[fn][0] = lds_rd_tr<E, TS::BN>(lB, ks, wcol0 + fn * 16, 0, lane);
      b.h[fn][1] = lds_rd_tr<E, TS::BN>(lB, ks, wcol0 + fn * 16, 1, lane);
    }
  }
}

template <class TS>
__device__ __forceinline__ u32x4_t read_a(const lds_t* lA, int fm, int ks, int wrow0, int lane) {
  return lds_rd128(lA + row_off(wrow0 + fm * 16 + (lane & 15), ks * 4 + (lane >> 4)));
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
// 8 rows of 128 bytes for A and for B given as (n, k); 1 KiB of consecutive
// k rows of BN columns for row-major B. Each wave issues BM/64 A loads and
// BN/64 B loads per stage. The schedule is described at the top.
template <Elem E, bool BT, class TS, class ColMap>
__device__ __forceinline__ void mainloop(lds_t* smem, const char* A, int64_t lda, int64_t row0,
                                         int64_t row_last, const BDesc& B, int64_t col0,
                                         const ColMap& colmap, const KSpan& ks,
                                         typename Mma<E>::acc_t (&acc)[TS::FM][TS::FN]) {
  constexpr int ES = ElemInfo<E>::bytes;
  constexpr int KE = kKBytes / ES;        // K values per stage
  constexpr int CE = 16 / ES;             // K values per 16-byte chunk
  constexpr int NA = TS::BM / 64;         // A loads per wave per stage
  constexpr int NB = TS::BN / 64;         // B loads per wave per stage
  static_assert(TS::NW == 8, "the eight-wave schedule");
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
      // 1 KiB per load, written linearly over k rows of BN * 2 bytes
      const int o = (NB * wave + j) * 1024 + 16 * lane;
      const int kr = o / (TS::BN * 2);
      const int pc = (o - kr * (TS::BN * 2)) >> 4;
      const int ch = (kmaj_unpos16<TS::BN>(pc >> 1, kr) << 1) | (pc & 1);
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

  // Loads of stage `it`: the buffer resources are formed once (prep) and the
  // NA + NB instructions issued one by one (issue_j) between MFMA rows.
  struct StageLd {
    __amdgpu_buffer_rsrc_t ra, rb;
    int64_t kleft;  // K values left in this shard
    lds_t* st;
  };
  auto prep = [&](int it) {
    StageLd s;
    const int ia = it + ks.it0;
    const int w = ia / ks.ktiles;
    const int kt = ia - w * ks.ktiles;
    const int64_t kdone = static_cast<int64_t>(kt) * KE;
    s.kleft = ks.k - kdone;
    s.st = smem + (it & 1) * TS::kStageBytes;
    s.ra = make_rsrc(a_base + w * ks.a_shard + kdone * ES);
    s.rb = BT ? make_rsrc(b_base + w * ks.b_shard + kdone * ES)
              : make_rsrc(b_base + w * ks.b_shard + kdone * B.ld);
    return s;
  };
  auto issue_j = [&](const StageLd& s, int j) {
    if (j < NA) {
      dma16(s.ra, s.st + 8 * (NA * wave + j) * kKBytes, a_key[j] < s.kleft ? a_off[j] : kOffNone);
    } else if constexpr (BT) {
      const int jb = j - NA;
      dma16(s.rb, s.st + TS::kABytes + 8 * (NB * wave + jb) * kKBytes,
            b_key[jb] < s.kleft ? b_off[jb] : kOffNone);
    } else {
      const int jb = j - NA;
      dma16(s.rb, s.st + TS::kABytes + (NB * wave + jb) * 1024,
            b_key[jb] < s.kleft ? b_off[jb] : kOffNone);
    }
  };
  auto issue_all = [&](int it) {
    const StageLd s = prep(it);
#pragma unroll
    for (int j = 0; j < NA + NB; ++j) issue_j(s, j);
  };

  const int n = ks.niters - ks.it0;
  constexpr int FM = TS::FM, FN = TS::FN;
  constexpr int NBO = BRegs<BT, FN>::kOps;
  // k-step-1 row followed by the barrier: the middle row for 8 fragment rows,
  // one later for 4 (measured: +2% on the int8 4096 x 8192 x 2048 share with
  // 128-row tiles, no change with 256-row tiles)
  constexpr int S0 = FM >= 8 ? FM / 2 - 1 : FM / 2;
  constexpr int NL = NA + NB;                     // loads per wave per stage
  constexpr int LROWS = FM - 1 - S0;              // k-step-1 rows that carry them
  constexpr int LPER = (NL + LROWS - 1) / LROWS;  // loads per row
  static_assert(NL <= 15, "vmcnt range of the prologue");
  u32x4_t a[FM];  // row fm's A fragment, refilled once the row's MFMAs are issued
  BRegs<BT, FN> b0, b1;
  StageLd nx;     // loads of the stage after next
  if (n > 0) {
    issue_all(0);
    if (n > 1) {
      issue_all(1);
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NL) : "memory");  // stage 0 has landed
    } else {
      wait_vmcnt0();
    }
    bar_sync();
    read_b_all<E, BT, TS>(b0, smem + TS::kABytes, 0, wcol0, lane);
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) a[fm] = read_a<TS>(smem, fm, 0, wrow0, lane);
  }
  // LDS reads in flight at each wait, in issue order: at k-step-0 row fm, the
  // A reads of rows > fm, then the k-step-1 reads issued so far (NBO B reads
  // and one A read at row 0, one more A read per row after that); at
  // k-step-1 row fm <= S0, the A reads of rows > fm.
  for (int it = 0; it < n; ++it) {
    const lds_t* cur = smem + (it & 1) * TS::kStageBytes;
    const lds_t* nxt = smem + ((it + 1) & 1) * TS::kStageBytes;
    const bool more = it + 1 < n;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      lgkm_wait(FM - 1 - fm + (fm == 0 ? 0 : NBO + fm));
      asm volatile("" : "+v"(a[fm]));
      if (fm == 0) b0.tie();
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) acc[fm][fn] = Mma<E>::run(a[fm], b0.get(fn), acc[fm][fn]);
      if (fm == 0) read_b_all<E, BT, TS>(b1, cur + TS::kABytes, 1, wcol0, lane);
      a[fm] = read_a<TS>(cur, fm, 1, wrow0, lane);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      if (fm <= S0) {
        lgkm_wait(FM - 1 - fm);
        asm volatile("" : "+v"(a[fm]));
        if (fm == 0) b1.tie();
      }
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) acc[fm][fn] = Mma<E>::run(a[fm], b1.get(fn), acc[fm][fn]);
      if (fm > S0 && it + 2 < n) {
#pragma unroll
        for (int q = 0; q < LPER; ++q) {
          const int j = (fm - S0 - 1) * LPER + q;
          if (j < NL) issue_j(nx, j);
        }
      }
      if (fm == S0) {
        lgkm_wait(0);   // every read of this stage is done
        wait_vmcnt0();  // this wave's loads of the next stage have landed
        bar_sync();     // ... and every wave's
        if (it + 2 < n) nx = prep(it + 2);
        if (more) {
          read_b_all<E, BT, TS>(b0, nxt + TS::kABytes, 0, wcol0, lane);
#pragma unroll
          for (int f = 0; f <= S0; ++f) a[f] = read_a<TS>(nxt, f, 0, wrow0, lane);
        }
      } else if (fm > S0 && more) {
        a[fm] = read_a<TS>(nxt, fm, 0, wrow0, lane);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  bar_sync();
}

// Cache policy of a store that writes through to memory (sc0 sc1): the line
// is not left dirty in this XCD's L2.
constexpr int kCpolWriteThrough = 0x11;

// Staged tile -> global with 16-byte coalesced stores; rows >= nrows and bytes
// >= row_bytes_valid of each destination row are skipped. The stores are
// non-temporal: output is not read again here. With write_through (for tiles
// that raise ready flags; every byte offset below 2^31), they write through
// to memory instead, so the L2 write-back of the flag release that follows
// has almost nothing to write (measured: about half the cost of the flags).
template <int NT = kThreads>
__device__ __forceinline__ void store_staged(const lds_t* smem, int pitch, int tile_row_bytes,
                                             int tile_rows, char* out, int64_t ldo, int64_t nrows,
                                             int64_t col_byte0, int64_t row_bytes_valid,
                                             bool write_through = false) {
  const int cpr = tile_row_bytes / 16;
  const int total = tile_rows * cpr;
  if (write_through) {
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(out);
    for (int q = threadIdx.x; q < total; q += NT) {
      const int r = q / cpr, c = q - r * cpr;
      if (r < nrows && col_byte0 + c * 16 < row_bytes_valid)
        __builtin_amdgcn_raw_buffer_store_b128(
            *reinterpret_cast<const MC2_LDS u32x4_t*>(smem + r * pitch + c * 16), ro,
            static_cast<int>(r * ldo + col_byte0 + c * 16), 0, kCpolWriteThrough);
    }
    return;
  }
  for (int q = threadIdx.x; q < total; q += NT) {
    const int r = q / cpr, c = q - r * cpr;
    if (r < nrows && col_byte0 + c * 16 < row_bytes_valid)
      __builtin_nontemporal_store(*reinterpret_cast<const MC2_LDS u32x4_t*>(smem + r * pitch + c * 16),
                                  reinterpret_cast<u32x4_t*>(out + r * ldo + col_byte0 + c * 16));
  }
}

}  // namespace mc2
