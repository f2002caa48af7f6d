// Four-wave main loop of the MFMA contraction for operands held K-contiguous
// (A as (m, k) and B as (n, k)), gfx950.
//
// Workgroup: 4 waves = 256 threads, one wave per SIMD, each wave owning a
// 128 x 128 (or, for 128-row tiles, 64 x 128) sub-tile of a 256 x 256 output
// tile: 8 x 8 blocks of 16 x 16, 256 fp32 accumulators per lane, held in the
// accumulation registers. Against eight waves of 128 x 64 this reads a third
// less from LDS per MFMA (each wave's A rows serve 128 columns instead of 64),
// and with one wave per SIMD no wave waits for a faster partner at the stage
// barrier.
//
// K stages, LDS layout, swizzle and the loads straight into LDS are those of
// the eight-wave loop (gemm_core.hpp): a stage holds 128 bytes of K per row,
// two stages live in a two-buffer ring, and a load instruction moves 8 rows
// of 128 bytes.
//
// Each MFMA takes the B fragment as its first operand and the A fragment as
// its second (both are "row j of a 16-row slice, 8 or 16 K values" per lane),
// so it computes the 16 x 16 block transposed: a lane ends with four
// consecutive columns of one output row (AccLayout).
//
// One wave issues everything in one stream, so the stage is a fixed
// interleave of its 2 x 64 MFMAs (16 cycles each) with the memory
// instructions, at most one LDS read and one load after an MFMA, so that a
// memory instruction the pipeline is slow to take stalls the wave for at most
// the MFMA's own latency:
//   the first slots: the operand reads of k-step 1;
//   slot kBarA: the wave waits for them, and a workgroup barrier follows
//     (every wave is done with this stage's buffer);
//   from there to the stage's last slot: the loads of the stage after next
//     into the buffer just released, evenly spread;
//   slot kBarB (in k-step 1): the wave waits for its loads of the next
//     stage, and a barrier follows (every wave's have landed);
//   after it: the operand reads of the next stage's k-step 0.
// Every LDS read is inline assembly (the compiler would otherwise wait for
// all loads before any LDS read); each k-step begins with an lgkmcnt(0) wait
// for the reads issued during the previous one.
#pragma once

#include <utility>

#include "gemm_core.hpp"

namespace mc2 {

template <class F, int... Is>
__device__ __forceinline__ void sfor_impl(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
// f(integral_constant<int, i>) for i = 0 .. N-1, unrolled at compile time.
template <int N, class F>
__device__ __forceinline__ void sfor(F&& f) {
  sfor_impl(f, std::make_integer_sequence<int, N>{});
}

// 16-byte LDS read at addr + OFF; valid only after a matching lgkm_wait.
template <int OFF>
__device__ __forceinline__ u32x4_t lds_rd128_at(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds_read offset field");
  u32x4_t v;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF) : "memory");
  return v;
}

// MFMAs as inline assembly with the accumulators in the accumulation
// registers ("a" operands): 256 accumulators per lane leave the vector
// registers to the operands. init() starts an accumulator (C = 0), acc()
// adds to it. The compiler does not see these as MFMAs, so it inserts no
// wait states for their results: within the loop an accumulator is reused
// only 64 MFMAs later, and settle() waits before anything else reads them.
template <Elem E> struct MmaA;
template <> struct MmaA<Elem::BF16> {
  static __device__ __forceinline__ void init(f32x4_t& c, u32x4_t a, u32x4_t b) {
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=a"(c) : "v"(a), "v"(b));
  }
  static __device__ __forceinline__ void acc(f32x4_t& c, u32x4_t a, u32x4_t b) {
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
  }
};
template <> struct MmaA<Elem::F16> {
  static __device__ __forceinline__ void init(f32x4_t& c, u32x4_t a, u32x4_t b) {
    asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, 0" : "=a"(c) : "v"(a), "v"(b));
  }
  static __device__ __forceinline__ void acc(f32x4_t& c, u32x4_t a, u32x4_t b) {
    asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
  }
};
template <> struct MmaA<Elem::I8> {
  static __device__ __forceinline__ void init(i32x4_t& c, u32x4_t a, u32x4_t b) {
    asm volatile("v_mfma_i32_16x16x64_i8 %0, %1, %2, 0" : "=a"(c) : "v"(a), "v"(b));
  }
  static __device__ __forceinline__ void acc(i32x4_t& c, u32x4_t a, u32x4_t b) {
    asm volatile("v_mfma_i32_16x16x64_i8 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
  }
};

// F operand fragments of a wave for one k-step: 16-byte reads of a
// K-contiguous operand (KC), or two 8-byte transposing reads of a k-major one
// whose halves form the MFMA operand after the wait (so no register copy can
// read a half still in flight).
template <bool KC, int F>
struct FragOps {
  u32x4_t q[KC ? F : 1];
  u32x2_t h[KC ? 1 : F][2];
  __device__ __forceinline__ u32x4_t get(int f) const {
    if constexpr (KC) return q[f];
    else return u32x4_t{h[f][0][0], h[f][0][1], h[f][1][0], h[f][1][1]};
  }
};

// Load j of a stage is issued at slot a + 1 + (j * span) / nl; the load
// issued at slot q, or -1.
constexpr int load_slot_index(int q, int a, int span, int nl) {
  for (int j = 0; j < nl; ++j)
    if (a + 1 + (j * span) / nl == q) return j;
  return -1;
}

// BT: B given as (n, k) (K-contiguous, like A); otherwise row-major (k, n),
// kept k-major in LDS and read with the transposing LDS reads (16-bit only),
// `colmap(c)` giving the global column of tile column c (a multiple of 8).
// AK: A given row-major (k, m) as well (`A` at its k row 0, `lda` bytes per k
// row, m = row0 .. row_last a multiple of 8 wide), kept and read the same way
// as row-major B (with row-major B and 256-row tiles only).
// KTAIL: the shard's K extent may end inside a stage, so every load checks
// its lanes against the K values left (lanes past the end load zeros);
// without it (K a multiple of the stage) the loads carry no per-lane check.
//
// LDS: A of stage 0, B of stage 0, B of stage 1, A of stage 1, so that the
// two B buffers lie within one immediate offset of each other.
template <Elem E, bool BT, class TS, bool KTAIL, bool AK = false, class ColMap>
__device__ __forceinline__ void mainloop_w4(lds_t* smem, const char* A, int64_t lda, int64_t row0,
                                            int64_t row_last, const BDesc& B, int64_t col0,
                                            const ColMap& colmap, const KSpan& ks,
                                            typename Mma<E>::acc_t (&acc)[TS::FM][TS::FN]) {
  constexpr int ES = ElemInfo<E>::bytes;
  constexpr int KE = kKBytes / ES;  // K values per stage
  constexpr int CE = 16 / ES;       // K values per 16-byte chunk
  constexpr int FM = TS::FM, FN = TS::FN;
  constexpr int NA = TS::BM / 32;   // A loads per wave per stage (8 rows each, 4 waves)
  constexpr int NB = TS::BN / 32;   // B loads per wave per stage
  constexpr int NL = NA + NB;
  constexpr int NBR = BT ? FN : 2 * FN;  // B operand reads per k-step (8 bytes each if !BT)
  constexpr int NAR = AK ? 2 * FM : FM;  // A operand reads per k-step (8 bytes each if AK)
  constexpr int NR = NAR + NBR;     // operand reads per wave per k-step
  static_assert(TS::NW == 4 && TS::BN == 256, "four waves, 256-column tiles");
  static_assert(!AK || ES == 2, "row-major A: 16-bit elements");
  static_assert(!AK || (!BT && TS::BM == 256), "row-major A: with row-major B, 256-row tiles");
  static_assert(NL <= 63, "vmcnt range of the prologue");
  constexpr int MM = FM * FN;       // MFMA slots per k-step
  // Slots q = 0 .. 2 MM - 1 of a stage (k-step 1 from MM on), one MFMA each:
  //   q < NR        the k-step-1 operand reads of this stage;
  //   kBarA         wait for them, barrier: this stage's buffer is free;
  //   load slots    the loads of the stage after next into that buffer,
  //                 spread evenly over the rest of the stage (kBarA + 1 to
  //                 the last slot), so that the CU's load path (about one
  //                 1 KiB load per 18 cycles, shared by the four waves)
  //                 never queues them;
  //   kBarB         wait for this wave's loads of the next stage (those of
  //                 the stage after next issued before kBarB may still be in
  //                 flight: loads complete in order), barrier;
  //   after kBarB   the next stage's k-step-0 operand reads, and the rest of
  //                 the loads.
  constexpr int kBarA = NR + 4;
  constexpr int kBarB = 2 * MM - NR - 4;
  constexpr int kLSpan = 2 * MM - kBarA - 2;  // load slots kBarA + 1 .. 2 MM - 1
  static_assert(kLSpan >= NL && kBarB + NR < 2 * MM, "slots for the loads and the reads");
  const int tid = threadIdx.x, lane = tid & 63;
  // the wave index as a wave-uniform value: the LDS destinations of the loads
  // (M0) are then scalar arithmetic
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  auto load_index = [](int q) constexpr { return load_slot_index(q, kBarA, kLSpan, NL); };
  // loads of the stage after next issued before kBarB
  constexpr int kLoadsBeforeB = [] {
    int c = 0;
    for (int j = 0; j < NL; ++j) c += kBarA + 1 + (j * kLSpan) / NL < kBarB;
    return c;
  }();
  const int wrow0 = (wave / TS::WN) * TS::WTM;
  const int wcol0 = (wave % TS::WN) * TS::WTN;

  // Per-lane offsets of this wave's loads: lane -> row (lane >> 3) of the 8
  // rows a load writes, physical chunk lane & 7, holding logical chunk
  // (lane & 7) ^ swizzle.
  // Row-major B: a load writes 1 KiB linearly over consecutive k rows of BN
  // columns (512 bytes each); lane -> k row, 16-byte piece of it, holding the
  // columns of the 32-byte pair the k-major swizzle puts there.
  uint32_t l_off[NL];
  int l_key[NL];
  // row-major A: the 8 rows of a 16-byte piece, the last piece clamped to the matrix
  auto rowmap = [&](int c) {
    const int64_t r = row0 + c;
    return r < row_last - 7 ? r : row_last - 7;
  };
#pragma unroll
  for (int j = 0; j < NL; ++j) {
    const bool isa = j < NA;
    if (AK && isa) {
      const int o = (NA * wave + j) * 1024 + 16 * lane;
      const int kr = o / (TS::BM * 2);
      const int pc = (o - kr * (TS::BM * 2)) >> 4;
      // (the swizzle is defined for 256-wide k rows; only AK tiles get here)
      const int ch = (kmaj_unpos16<(AK ? TS::BM : 256)>(pc >> 1, kr) << 1) | (pc & 1);
      l_off[j] = static_cast<uint32_t>(kr * lda + rowmap(ch * 8) * 2);
      l_key[j] = kr;
    } else if (isa || BT) {
      const int r = 8 * ((isa ? NA : NB) * wave + (isa ? j : j - NA)) + (lane >> 3);
      const int c = (row_off(r, lane & 7) - r * kKBytes) >> 4;
      if (isa) {
        int64_t gr = row0 + r;
        gr = gr < row_last ? gr : row_last;
        l_off[j] = static_cast<uint32_t>((gr - row0) * lda + c * 16);
      } else {
        int64_t gc = col0 + r;
        gc = gc < B.n - 1 ? gc : B.n - 1;
        l_off[j] = static_cast<uint32_t>((gc - col0) * B.ld + c * 16);
      }
      l_key[j] = c * CE;
    } else if constexpr (ES == 2) {
      const int o = (NB * wave + (j - NA)) * 1024 + 16 * lane;
      const int kr = o / (TS::BN * 2);
      const int pc = (o - kr * (TS::BN * 2)) >> 4;
      const int ch = (kmaj_unpos16<TS::BN>(pc >> 1, kr) << 1) | (pc & 1);
      l_off[j] = static_cast<uint32_t>(kr * B.ld + colmap(ch * 8) * 2);
      l_key[j] = kr;
    } else {
      // 8-bit: four k rows of 256 bytes per load, 16-byte units swizzled by
      // kmaj_swz8 (the layout of the eight-wave loop)
      const int kr = 4 * (NB * wave + (j - NA)) + (lane >> 4);
      const int ch = (lane & 15) ^ kmaj_swz8(kr);
      l_off[j] = static_cast<uint32_t>(kr * B.ld + colmap(ch * 16));
      l_key[j] = kr;
    }
  }
  const char* a_base = AK ? A : A + row0 * lda;
  const char* b_base = BT ? B.base + col0 * B.ld : B.base;
  // LDS regions: A of stage p at a_lds(p), B of stage p at b_lds(p); with
  // row-major A both A buffers come first (the transposing reads address
  // them from one register, as the B buffers)
  constexpr int kA1 = AK ? TS::kABytes : TS::kABytes + 2 * TS::kBBytes;
  constexpr int kB0 = AK ? 2 * TS::kABytes : TS::kABytes;
  auto a_lds = [](int p) { return p ? kA1 : 0; };
  auto b_lds = [](int p) { return kB0 + p * TS::kBBytes; };

  // Loads of stage it: the buffer resources are formed once per stage; a
  // stage past the last one gets resources of no records, so its loads (the
  // loop issues them unconditionally, with no branch in the MFMA stream)
  // touch no memory and write zeros into a buffer nobody reads any more.
  struct StageLd {
    __amdgpu_buffer_rsrc_t ra, rb;
    int kleft;  // K values left in this shard (clamped)
    lds_t* st;   // A destination
    lds_t* stb;  // B destination
  };
  // Stages are loaded in order; ld_it counts the stages loaded and (lw, lkt)
  // is the shard and K stage of the next one, advanced with scalar adds (no
  // division per stage). A K part starts at stage ks.it0.
  int ld_it = 0, lw = ks.it0 / ks.ktiles, lkt = ks.it0 - lw * ks.ktiles;
  const int n = ks.niters - ks.it0;  // at least 1
  auto prep = [&]() {
    StageLd s;
    const int64_t kdone = static_cast<int64_t>(lkt) * KE;
    const int64_t kl = ks.k - kdone;
    s.kleft = static_cast<int>(kl < (1 << 30) ? kl : (1 << 30));
    s.st = smem + ((ld_it & 1) ? kA1 : 0);
    s.stb = smem + kB0 + (ld_it & 1) * TS::kBBytes;
    const int nrec = ld_it < n ? 0x7ffffff0 : 0;
    s.ra = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(a_base + lw * ks.a_shard + (AK ? kdone * lda : kdone * ES)), 0, nrec,
        kBufFlags);
    s.rb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(b_base + lw * ks.b_shard + (BT ? kdone * ES : kdone * B.ld)), 0, nrec,
        kBufFlags);
    ++ld_it;
    if (++lkt == ks.ktiles) {
      lkt = 0;
      ++lw;
    }
    return s;
  };
  auto issue_j = [&](const StageLd& s, int j) {
    uint32_t off = l_off[j];
    if constexpr (KTAIL) off = l_key[j] < s.kleft ? off : kOffNone;
    if (j < NA)
      dma16(s.ra, s.st + 8 * (NA * wave + j) * kKBytes, off);
    else
      dma16(s.rb, s.stb + 8 * (NB * wave + (j - NA)) * kKBytes, off);
  };

  // LDS read addresses of the wave's first fragment (row wrow0 + (lane & 15)
  // of A, column wcol0 + (lane & 15) of B) for k-step ks of buffer p; the
  // other fragments sit 16 rows (2048 bytes) further on, an immediate offset.
  const uint32_t s0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(smem));
  uint32_t adA[2][2], adB[2][2];
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      const int ch = k2 * 4 + (lane >> 4);
      adA[p][k2] = s0 + a_lds(p) + row_off(wrow0 + (lane & 15), ch);
      adB[p][k2] = s0 + b_lds(p) + row_off(wcol0 + (lane & 15), ch);
    }
  // Row-major B: the transposing read of half h of fragment fn, k-step k2,
  // buffer p, reads lane j of group g at k row 32 k2 + 8 g + 4 h + (j >> 2),
  // 32-byte pair (wcol0 / 16 + fn) ^ swizzle, byte 8 (j & 3). The swizzle
  // depends only on the lane ((j >> 2) and the parity of g), and the wave's
  // pairs are wcol0 / 16 + 0..7 with wcol0 / 16 in {0, 8}, so the pair is
  // wcol0 / 16 | (fn ^ swizzle): one address register per fragment, with
  // buffer, k-step and half in the immediate offset.
  uint32_t adT[BT ? 1 : FN];
  if constexpr (!BT && ES == 2) {
    const int j = lane & 15, g = lane >> 4;
    const int swz = (j >> 2) | ((g & 1) << 2);
    const uint32_t base = s0 + kB0 + (g * 8 + (j >> 2)) * (TS::BN * 2) + ((j & 3) << 3);
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
      adT[fn] = base + ((((wcol0 >> 4) | (fn ^ swz))) << 5);
  } else if constexpr (!BT) {
    // 8-bit row-major B: lane j of group g reads k row 64 k2 + 16 g + 8 h +
    // (j >> 1) (k-step k2, half h: both in the immediate offset), 16-byte
    // unit (wcol0 / 16 + fn) ^ kmaj_swz8 of that row, byte 8 (j & 1); the
    // swizzle depends only on the lane: (j >> 1) | (g & 1) << 3
    const int j = lane & 15, g = lane >> 4;
    const int swz = (j >> 1) | ((g & 1) << 3);
    const uint32_t base = s0 + kB0 + (g * 16 + (j >> 1)) * TS::BN + ((j & 1) << 3);
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
      adT[fn] = base + ((((wcol0 >> 4) + fn) ^ swz) << 4);
  }
  // Row-major A: the same with the wave's rows (wrow0 / 16 in {0, 8}) and
  // A's buffers.
  uint32_t adTA[AK ? FM : 1];
  if constexpr (AK) {
    const int j = lane & 15, g = lane >> 4;
    const int swz = (j >> 2) | ((g & 1) << 2);
    const uint32_t base = s0 + (g * 8 + (j >> 2)) * (TS::BM * 2) + ((j & 3) << 3);
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
      adTA[fm] = base + ((((wrow0 >> 4) | (fm ^ swz))) << 5);
  }

  using AOps = FragOps<!AK, FM>;
  using BOps = FragOps<BT, FN>;
  AOps a0, a1;
  BOps b0, b1;
  // operand read number i of k-step K2 from buffer P: B reads first, then A
  auto read_op = [&](auto I, auto Pc, auto K2c, AOps& a, BOps& b) {
    constexpr int i = decltype(I)::value, P = decltype(Pc)::value, K2 = decltype(K2c)::value;
    if constexpr (i >= NBR && AK) {
      constexpr int fm = (i - NBR) / 2, h = (i - NBR) % 2;
      constexpr int off = P * TS::kABytes + (32 * K2 + 4 * h) * TS::BM * 2;
      static_assert(off < 65536, "ds_read offset field");
      const uint32_t addr = adTA[fm];
      asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2"
                   : "=v"(a.h[fm][h]) : "v"(addr), "i"(off) : "memory");
    } else if constexpr (i >= NBR) {
      a.q[i - NBR] = lds_rd128_at<(i - NBR) * 16 * kKBytes>(adA[P][K2]);
    } else if constexpr (BT) {
      b.q[i] = lds_rd128_at<i * 16 * kKBytes>(adB[P][K2]);
    } else {
      constexpr int fn = i / 2, h = i % 2;
      const uint32_t addr = adT[fn];
      if constexpr (ES == 2) {
        constexpr int off = P * TS::kBBytes + (32 * K2 + 4 * h) * TS::BN * 2;
        static_assert(off < 65536, "ds_read offset field");
        asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2"
                     : "=v"(b.h[fn][h]) : "v"(addr), "i"(off) : "memory");
      } else {
        constexpr int off = P * TS::kBBytes + (64 * K2 + 8 * h) * TS::BN;
        static_assert(off < 65536, "ds_read offset field");
        asm volatile("ds_read_b64_tr_b8 %0, %1 offset:%2"
                     : "=v"(b.h[fn][h]) : "v"(addr), "i"(off) : "memory");
      }
    }
  };
  auto tie = [&](AOps& a, BOps& b) {
    if constexpr (AK) {
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        asm volatile("" : "+v"(a.h[i][0]));
        asm volatile("" : "+v"(a.h[i][1]));
      }
    } else {
#pragma unroll
      for (int i = 0; i < FM; ++i) asm volatile("" : "+v"(a.q[i]));
    }
    if constexpr (BT) {
#pragma unroll
      for (int i = 0; i < FN; ++i) asm volatile("" : "+v"(b.q[i]));
    } else {
#pragma unroll
      for (int i = 0; i < FN; ++i) {
        asm volatile("" : "+v"(b.h[i][0]));
        asm volatile("" : "+v"(b.h[i][1]));
      }
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;

  StageLd nx;
  {
    nx = prep();  // stage 0
#pragma unroll
    for (int j = 0; j < NL; ++j) issue_j(nx, j);
    nx = prep();  // stage 1 (no records when there is a single stage)
#pragma unroll
    for (int j = 0; j < NL; ++j) issue_j(nx, j);
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NL) : "memory");  // stage 0 has landed
    bar_sync();
    sfor<NR>([&](auto I) { read_op(I, I0{}, I0{}, a0, b0); });
  }

  // One stage from buffer P; the first stage starts the accumulators.
  auto stage = [&](auto Pc, auto First, int it) {
    constexpr int P = decltype(Pc)::value;
    constexpr bool FIRST = decltype(First)::value;
    lgkm_wait(0);  // this stage's k-step-0 operands (read during the previous stage)
    tie(a0, b0);
    sfor<2 * MM>([&](auto Q) {
      constexpr int q = decltype(Q)::value;
      constexpr int s = q % MM, fm = s / FN, fn = s % FN;
      if constexpr (q == MM) tie(a1, b1);
      if constexpr (q < MM) {
        if constexpr (FIRST)
          MmaA<E>::init(acc[fm][fn], b0.get(fn), a0.get(fm));
        else
          MmaA<E>::acc(acc[fm][fn], b0.get(fn), a0.get(fm));
      } else {
        MmaA<E>::acc(acc[fm][fn], b1.get(fn), a1.get(fm));
      }
      if constexpr (q < NR) {
        read_op(std::integral_constant<int, q>{}, Pc, I1{}, a1, b1);
      } else if constexpr (q == kBarA) {
        lgkm_wait(0);  // every read of this stage's buffer is done
        bar_sync();    // ... by every wave: the buffer may be refilled
        nx = prep();  // stage it + 2
      } else if constexpr (q == kBarB) {
        // this wave's loads of the next stage have landed (those of the
        // stage after next issued since kBarA may still be in flight)
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kLoadsBeforeB) : "memory");
        bar_sync();  // ... and every wave's
      } else if constexpr (q > kBarB && (q - kBarB - 1) < NR) {
        // the next stage's k-step-0 operands (after the last stage: reads of
        // a buffer nobody writes any more, never used)
        read_op(std::integral_constant<int, q - kBarB - 1>{}, std::integral_constant<int, 1 - P>{},
                I0{}, a0, b0);
      }
      if constexpr (load_index(q) >= 0) issue_j(nx, load_index(q));
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  using T = std::true_type;
  using F = std::false_type;
  stage(I0{}, T{}, 0);
  for (int it = 1; it < n; it += 2) {
    stage(I1{}, F{}, it);
    if (it + 1 < n) stage(I0{}, F{}, it + 1);
  }
  // the last stage's reads of the next stage's operands (never used) land in
  // registers that stay allocated until they have (an asm output counts as
  // written at once, so without this use the compiler could reuse them early)
  lgkm_wait(0);
  tie(a0, b0);
  wait_vmcnt0();
  bar_sync();
  // the last MFMAs' results are complete before anything reads them
  asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15\n\ts_nop 15" ::: "memory");
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) asm volatile("" : "+a"(acc[fm][fn]));
}

}  // namespace mc2
