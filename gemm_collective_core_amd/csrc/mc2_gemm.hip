// Rank-chunked GEMM (MatmulReduceScatter / AllGatherMatmul compute share), for
// gfx950.
//
// Formulas: torch_npu.npu_mm_reduce_scatter_base API doc, "功能说明" (basic and
// quantized MatmulReduceScatter); CANN hccl issue 158 (AllGatherMatmul).
#include <atomic>

#include "mc2_chunked.hpp"

namespace mc2 {

// ---------------------------------------------------------------- chunked GEMM

// Split policy of the K split, process-wide (mc2_set_split_policy).
static std::atomic<int> g_split_policy{MC2_SPLIT_PAIR};

struct ChunkedArgs {
  const char* A;
  const char* B;
  char* out;
  const void* bias;
  const float* s1;
  const float* s2;
  int64_t m, n;
  int64_t lda, ldb, ldo;  // bytes
  KSpan ks;
  int64_t mc;             // rows per chunk
  int world, first_chunk;
  // Each chunk is cut into `sub` pieces (segments) of sq rows, plus one row
  // for the first sr; a long piece has tiles_m1 tile rows, a short one tiles_m0.
  int sub, sr;
  int64_t sq;
  int tiles_m1, tiles_m0, tiles_n, tiles_long, tiles_short, tiles_per_chunk;
  int round;              // workgroups per dispatch round (CUs, multiple of 8); 0: no remap
  int n_full;             // work units below n_full are whole tiles, the rest half tiles
  float bias_mul;
  uint32_t* flags;
  uint32_t* counters;
  uint32_t epoch;
  const uint32_t* in_flags;  // NULL: inputs are present; else wait for in_flags[segment]
  uint32_t in_epoch;
  uint32_t spin_limit;
  int32_t* dev_err;
  int own_chunk;             // the chunk that needs no input flag
  int store_wt;              // 16-bit outputs written through to memory (flags raised)
  // K split of the last round (NULL: none): per pair two partial slots, and
  // four control words each; sk_alone: the policy in which the first half to
  // start never waits for its partner.
  char* sk_part;
  uint32_t* sk_ctl;
  int sk_alone;
};

// Waits (one thread polls) until input segment g is marked ready, then acquires
// at system scope: the producer is another agent. Bounded: after spin_limit
// polls the tile records MC2_DEVERR_TIMEOUT and goes on.
__device__ __forceinline__ void wait_input_segment(const ChunkedArgs& p, int g) {
  if (threadIdx.x == 0) {
    bool ready = false;
    for (uint32_t i = 0; i < p.spin_limit; ++i) {
      if (__hip_atomic_load(p.in_flags + g, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) ==
          p.in_epoch) {
        ready = true;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    if (!ready) atomic_or_err(p.dev_err, MC2_DEVERR_TIMEOUT);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "");
  }
  __syncthreads();
}

template <class TS, int OS>
constexpr int chunked_smem() {
  // 32-bit outputs are not staged through LDS
  return (OS == 4 || TS::kStages * TS::kStageBytes > TS::BM * (TS::BN * OS + 16))
             ? TS::kStages * TS::kStageBytes
             : TS::BM * (TS::BN * OS + 16);
}

// Where tile `tile` sits. Tiles are numbered chunk by chunk in the order the
// chunks are due (first_chunk, first_chunk + 1, ... mod W), inside a chunk
// piece by piece in row order, and inside a piece row-block fastest, so that
// a run of consecutive tiles forms a compact block and the segments complete
// roughly in order. `bm` is the height a tile row of the schedule spans.
struct TilePos {
  int c, g, seg_tiles;
  int64_t row0, row_end, col0;  // first row (of the whole tile), end of its piece, first column
};

__device__ __forceinline__ TilePos tile_pos(const ChunkedArgs& p, int tile, int bm, int bn) {
  TilePos q;
  const int seq = tile / p.tiles_per_chunk;
  int t = tile - seq * p.tiles_per_chunk;
  int c = p.first_chunk + seq;
  c = c >= p.world ? c - p.world : c;
  const int long_tiles = p.sr * p.tiles_long;
  int j, tiles_mj;
  if (t < long_tiles) {
    j = t / p.tiles_long;
    t -= j * p.tiles_long;
    tiles_mj = p.tiles_m1;
    q.seg_tiles = p.tiles_long;
  } else {
    const int v = (t - long_tiles) / p.tiles_short;
    j = p.sr + v;
    t -= long_tiles + v * p.tiles_short;
    tiles_mj = p.tiles_m0;
    q.seg_tiles = p.tiles_short;
  }
  q.c = c;
  q.g = c * p.sub + j;
  const int64_t seg_row0 = c * p.mc + j * p.sq + (j < p.sr ? j : p.sr);
  q.row_end = seg_row0 + p.sq + (j < p.sr ? 1 : 0);
  const int tm = t % tiles_mj, tn = t / tiles_mj;
  q.row0 = seg_row0 + static_cast<int64_t>(tm) * bm;
  q.col0 = static_cast<int64_t>(tn) * bn;
  return q;
}

// Epilogue and store of the tile rows held by the waves of the row halves in
// `halves` (bit r: the waves of row half r, which hold tile rows
// [r BM/2, (r + 1) BM/2); 3: the whole tile).
template <Elem E, class TS, Out O>
__device__ __forceinline__ void store_tile(const ChunkedArgs& p, lds_t* smem,
                                           const typename Mma<E>::acc_t (&acc)[TS::FM][TS::FN],
                                           int64_t row0, int64_t row_end, int64_t col0,
                                           int halves) {
  static_assert(TS::WM == 2, "two row halves of waves");
  constexpr int OS = OutInfo<O>::bytes;
  const int rh = (threadIdx.x >> 6) / TS::WN;
  const bool mine = (halves >> rh) & 1;  // uniform over the wave
  const int lo = halves == 2 ? TS::BM / 2 : 0;
  const int nr = halves == 3 ? TS::BM : TS::BM / 2;
  if constexpr (TS::NW == 4 && OS == 2) {
    // runs of four columns per lane: one 8-byte LDS write per run, then
    // 16-byte coalesced stores of whole rows (stores of the 8-byte runs
    // straight from the registers, 16 rows x 32 bytes per instruction, were
    // measured far slower: partial lines reach memory)
    constexpr int pitch = TS::BN * OS + 16;
    if (mine)
      epilogue_quads<E, TS, O>(acc, row0, row_end - 1, col0, p.n, p.bias, p.bias_mul, p.s1, p.s2,
                               [&](int rr, int cc, const auto& v) {
                                 *reinterpret_cast<MC2_LDS u32x2_t*>(smem + rr * pitch + cc * OS) =
                                     pack4<O>(v);
                               });
    __syncthreads();
    store_staged<TS::NT>(smem + lo * pitch, pitch, TS::BN * OS, nr, p.out + (row0 + lo) * p.ldo,
                         p.ldo, row_end - (row0 + lo), col0 * OS, p.n * OS, p.store_wt != 0);
  } else if constexpr (TS::NW == 4) {
    // 32-bit test outputs: runs of four columns, 16-byte stores straight from
    // the registers. n is a multiple of 8, so a run is either wholly inside
    // the output or wholly past its last column.
    char* base = p.out + row0 * p.ldo + col0 * OS;
    const int64_t nrows = row_end - row0, ncols = p.n - col0;
    const bool wt = p.store_wt != 0;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(base);
    if (mine)
      epilogue_quads<E, TS, O>(acc, row0, row_end - 1, col0, p.n, p.bias, p.bias_mul, p.s1, p.s2,
                               [&](int rr, int cc, const auto& v) {
                                 if (rr < nrows && cc < ncols)
                                   store4<O>(base, r, rr * p.ldo + cc * OS, v, wt);
                               });
  } else if constexpr (OS == 2) {
    // 16-bit outputs: stage the rows in LDS, then 16-byte coalesced stores.
    constexpr int pitch = TS::BN * OS + 16;
    if (mine)
      epilogue_linear<E, TS, O>(acc, row0, row_end - 1, col0, p.n, p.bias, p.bias_mul, p.s1, p.s2,
                                [&](int r, int cc, float v) { put_out<O>(smem + r * pitch + cc * OS, v); });
    __syncthreads();
    store_staged<TS::NT>(smem + lo * pitch, pitch, TS::BN * OS, nr, p.out + (row0 + lo) * p.ldo,
                         p.ldo, row_end - (row0 + lo), col0 * OS, p.n * OS, p.store_wt != 0);
  } else {
    // 32-bit test outputs: stored straight from the accumulator layout.
    char* base = p.out + row0 * p.ldo + col0 * OS;
    const int64_t nrows = row_end - row0, ncols = p.n - col0;
    if (mine)
      epilogue_linear<E, TS, O>(acc, row0, row_end - 1, col0, p.n, p.bias, p.bias_mul, p.s1, p.s2,
                                [&](int r, int cc, auto v) {
                                  if (r < nrows && cc < ncols) put_out_global<O>(base + r * p.ldo + cc * OS, v);
                                });
  }
}

// Counts `weight` half-tile units of segment g as done; the unit that
// completes the segment raises its ready flag.
//   Each wave waits for its own stores; after the barrier, thread 0's
// agent-scope release (one L2 write-back per tile) covers the whole tile
// before the tile is counted. Only the last tile of a segment acquires the
// other tiles' releases (an acquire invalidates this XCD's L2, so it is kept
// off the other tiles) and then publishes the epoch with a system-scope
// release store.
__device__ __forceinline__ void count_tile(const ChunkedArgs& p, int g, int seg_tiles,
                                           uint32_t weight) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const uint32_t prev = __hip_atomic_fetch_add(&p.counters[g], weight, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    if (prev + weight == 2u * static_cast<uint32_t>(seg_tiles)) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      __hip_atomic_store(&p.counters[g], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&p.flags[g], p.epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
    }
  }
}

// ---------------------------------------------------------------- K split
//
// A tile of a last dispatch round that would leave at least half of the CUs
// idle can run as two K halves on two workgroups (a pair): half 0 sums the
// stages [0, n/2) of the K loop, half 1 the stages [n/2, n), both over the
// whole tile. The halves meet through a workspace: per pair, two slots of
// 128 KiB, slot x holding the fp32 (int32) partial of tile row half 1 - x as
// written by half x or, when one workgroup finalizes the whole tile, by the
// other; and control words: [0] start tickets, [1 + x] "half x has written
// its slot". Every output element is then (sum over the first K half) +
// (sum over the second): one addition, which gives the same bits whichever
// workgroup performs it (and int32 sums are exact in any order).
//
// No workgroup ever waits for a partner that may not be running:
//   - at its start each half takes a ticket; the first (ticket 0) is "early";
//   - early, when its K loop ends, tries to move the tickets from 1 to 3.
//     If that succeeds, the partner has not started: early writes its whole
//     partial (both slots), marks its slot written and leaves, and the
//     partner will finalize the whole tile. If the partner has started
//     (tickets at 2) it is running: early writes the partner's row half,
//     marks its slot, waits for the partner's mark, adds the partner's part
//     of its own row half and finalizes that;
//   - the late half (ticket 1: pair; ticket 3 or 4: early has left or will
//     leave) does the same from its side; it only ever waits for early,
//     which has started.
// The late half resets the control words, so they are zero after every call.
//
// Visibility without cache maintenance: the partials are written and read
// with device-scope (sc1) accesses, the cache policy of relaxed agent-scope
// atomics, which are coherent across the XCDs' L2s by themselves; a writer
// waits for its stores to complete before the control word is set. So no
// L2 write-back or invalidate is taken, which would cost the other tiles on
// the XCD their cached operands.

// The K split is switched off: its first device runs faulted on the partial
// stores (a scalar base address read too soon after v_readfirstlane wrote
// it; fixed below with the wait states), and the fix has not yet run on the
// device. Until it has, a workspace is accepted and ignored, a thin last
// round runs as 128-row halves, and the split code is compiled out.
constexpr bool kSplitEnabled = false;

constexpr int64_t kPartBytes = 128 * 256 * 4;  // a row half of a 256 x 256 tile, 32-bit
constexpr int64_t kSplitCtlBytes = 4096;       // control words of up to 256 pairs
constexpr int kCpolDevice = 0x10;              // sc1: coherent at device scope
constexpr uint32_t kSplitSpin = 1u << 20;      // polls (~2 us each) before giving up

// Accumulators of this wave into the partial slot at base + off0 (waves of
// one row half): vector v = fm * FN + fn of lane l of the wave in column
// position wc sits at byte ((wc * FM * FN + v) * 64 + l) * 16 of the slot, so
// every store is 1 KiB contiguous. The stores take their data straight from
// the accumulation registers (as assembly: a store built from the values
// would first copy all of them into vector registers). The base address is
// made scalar with v_readfirstlane, a vector-ALU write of scalar registers,
// and a vector memory instruction may read such registers only 5 wait states
// later; the compiler does not insert them in front of assembly, so each
// store starts with them (s_nop 4).
template <class TS, class AccT>
__device__ __forceinline__ void part_put(const char* base, uint32_t off0,
                                         const AccT (&acc)[TS::FM][TS::FN]) {
  const int lane = threadIdx.x & 63, wc = (threadIdx.x >> 6) % TS::WN;
  const uint32_t off = off0 + static_cast<uint32_t>((wc * TS::FM * TS::FN * 64 + lane) * 16);
  // the base address in scalar registers (it is the same for every lane);
  // both halves unsigned, so the low one is not sign-extended into the high
  const uint64_t bv = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(bv)));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(bv >> 32)));
  const uint64_t sb = (static_cast<uint64_t>(hi) << 32) | lo;
#pragma unroll
  for (int v = 0; v < TS::FM * TS::FN; ++v) {
    if constexpr (TS::NW == 4)
      asm volatile("s_nop 4\n\tglobal_store_dwordx4 %0, %1, %2 sc1"
                   :: "v"(off + v * 1024), "a"(acc[v / TS::FN][v % TS::FN]), "s"(sb) : "memory");
    else
      asm volatile("s_nop 4\n\tglobal_store_dwordx4 %0, %1, %2 sc1"
                   :: "v"(off + v * 1024), "v"(acc[v / TS::FN][v % TS::FN]), "s"(sb) : "memory");
  }
}

// acc += the partial of this wave's elements in the slot at base + off0
// (layout of part_put), one fragment row (FN loads in flight) at a time so
// that the loaded values never need more registers than one row.
template <class TS, class AccT>
__device__ __forceinline__ void part_add(const char* base, uint32_t off0,
                                         AccT (&acc)[TS::FM][TS::FN]) {
  const int lane = threadIdx.x & 63, wc = (threadIdx.x >> 6) % TS::WN;
  const __amdgpu_buffer_rsrc_t r = make_rsrc(base);
  const uint32_t off = off0 + static_cast<uint32_t>((wc * TS::FM * TS::FN * 64 + lane) * 16);
#pragma unroll
  for (int fm = 0; fm < TS::FM; ++fm) {
    u32x4_t v[TS::FN];
#pragma unroll
    for (int fn = 0; fn < TS::FN; ++fn)
      v[fn] = __builtin_amdgcn_raw_buffer_load_b128(r, off + (fm * TS::FN + fn) * 1024, 0,
                                                    kCpolDevice);
#pragma unroll
    for (int fn = 0; fn < TS::FN; ++fn) {
      acc[fm][fn] += bit_cast<AccT>(v[fn]);
      // four-wave tiles keep the accumulators in the accumulation registers
      if constexpr (TS::NW == 4) asm volatile("" : "+a"(acc[fm][fn]));
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Thread 0 polls *f (relaxed device-scope loads) until it is nonzero; the
// workgroup barrier then releases every wave. The protocol only waits for a
// workgroup that is running and waits for nothing itself; the bound turns a
// broken invariant into MC2_DEVERR_TIMEOUT (and wrong data) rather than a
// hang.
__device__ __forceinline__ void wait_part(uint32_t* f, int32_t* dev_err) {
  if (threadIdx.x == 0) {
    uint32_t i = 0;
    while (__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u) {
      if (++i == kSplitSpin) {
        atomic_or_err(dev_err, MC2_DEVERR_TIMEOUT);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
  __syncthreads();
}

// Exchanges the K halves of pair `pair` after the main loop (see above) and
// returns the row halves this workgroup finalizes (bit r: row half r), or 0.
// Every slot access of a wave is to the slot of its own row half, so each
// wave writes at most once and adds at most once, each at one place.
template <class TS, class AccT>
__device__ __forceinline__ int split_exchange(const ChunkedArgs& p, int pair, int h,
                                              uint32_t ticket, AccT (&acc)[TS::FM][TS::FN]) {
  __shared__ uint32_t sh_alone;
  uint32_t* ctl = p.sk_ctl + 4 * pair;
  const int rh = (threadIdx.x >> 6) / TS::WN;
  const char* base = p.sk_part + 2 * pair * kPartBytes;         // the pair's slots
  const uint32_t slot = static_cast<uint32_t>((1 - rh) * kPartBytes);  // own row half's
  const bool early = ticket == 0;
  if (early) {
    if (threadIdx.x == 0) {
      uint32_t e = 1u;
      __hip_atomic_compare_exchange_strong(ctl, &e, 3u, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
      // 1: moved now; 3 or 4: moved at the start (policy "alone"); 2: partner running
      sh_alone = e != 2u;
    }
    __syncthreads();
  }
  // early alone: hand the whole tile over; pair: send the partner's row half
  const bool alone = early ? sh_alone != 0u : ticket != 1u;
  const bool sends = early ? (alone || rh != h) : (!alone && rh != h);
  if (sends) part_put<TS>(base, slot, acc);
  if (early || !alone) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_store(ctl + 1 + h, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (early && alone) return 0;
  }
  wait_part(ctl + 2 - h, p.dev_err);
  // pair: add the partner's part of the own row half; late alone: of both
  const bool adds = alone || rh == h;
  if (adds) part_add<TS>(base, slot, acc);
  if (threadIdx.x == 0) {
    __hip_atomic_store(ctl + 2 - h, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (!early) __hip_atomic_store(ctl, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  return alone ? 3 : 1 << h;
}

// One work unit: a whole tile (kpart < 0, half 0, weight 2), the row half
// `half` of a tile (a TS of half height: weight 1), or K half kpart of tile
// pair `pair` (a whole-height TS). Main loop, epilogue, store, and the
// segment's ready flag.
template <Elem E, bool BT, class TS, Out O, bool KT>
__device__ __forceinline__ void chunked_tile(const ChunkedArgs& p, lds_t* smem, int tile, int half,
                                             uint32_t weight, int kpart = -1, int pair = 0) {
  const TilePos tp = tile_pos(p, tile, TS::BM << (weight == 1), TS::BN);
  const int64_t row0 = tp.row0 + static_cast<int64_t>(half) * TS::BM;
  // The ticket goes to LDS at once: a register held across the main loop
  // would cost the loop registers it has none to spare of. (Only wave 0
  // waits for the atomic; the others start their loads.)
  __shared__ uint32_t sh_ticket;
  if (kpart >= 0 && threadIdx.x == 0) {
    const uint32_t t = __hip_atomic_fetch_add(p.sk_ctl + 4 * pair, 1u, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
    if (t == 0 && p.sk_alone) {
      uint32_t e = 1u;  // policy "alone": early never waits (see split_exchange)
      __hip_atomic_compare_exchange_strong(p.sk_ctl + 4 * pair, &e, 3u, __ATOMIC_RELAXED,
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    sh_ticket = t;
  }

  if (p.in_flags && tp.c != p.own_chunk) wait_input_segment(p, tp.g);
  // the lower half of a tile that overhangs its piece may hold no rows
  if (row0 < tp.row_end) {
    typename Mma<E>::acc_t acc[TS::FM][TS::FN];
    BDesc bd{p.B, p.ldb, p.n};
    PlainCols cm{tp.col0, p.n - 16 / ElemInfo<E>::bytes};
    KSpan ks = p.ks;
    if (kpart >= 0) {
      const int mid = ks.niters / 2;
      if (kpart == 0) ks.niters = mid;
      else ks.it0 = mid;
    }
    if constexpr (TS::NW == 4)
      mainloop_w4<E, BT, TS, KT>(smem, p.A, p.lda, row0, tp.row_end - 1, bd, tp.col0, cm, ks, acc);
    else
      mainloop<E, BT, TS>(smem, p.A, p.lda, row0, tp.row_end - 1, bd, tp.col0, cm, ks, acc);

    int halves = 3;
    if (kpart >= 0) {
      __syncthreads();  // sh_ticket, written before the main loop's barriers
      halves = split_exchange<TS>(p, pair, kpart, sh_ticket, acc);
      if (halves == 0) return;  // the partner finalizes the whole tile
      weight = halves == 3 ? 2u : 1u;
    }
    store_tile<E, TS, O>(p, smem, acc, row0, tp.row_end, tp.col0, halves);
  }
  if (p.flags) count_tile(p, tp.g, tp.seg_tiles, weight);
}

// One workgroup per work unit. With 256-row tiles, a last dispatch round
// that would leave at least half of the CUs idle runs its tiles (n_full on)
// as K halves on two workgroups each when a workspace is given (units
// n_full + 2i and n_full + 2i + 1), else as two 128-row halves (the round
// then ends after a 128-row tile's time; each half still sums all of K).
// KT: the K extent of a shard may end inside a stage (four-wave tiles
// only; the eight-wave loop always checks).
template <Elem E, bool BT, class TS, Out O, bool KT>
__global__ __launch_bounds__(TS::NT, 1) void chunked_gemm_kernel(ChunkedArgs p) {
  constexpr int kSmem = chunked_smem<TS, OutInfo<O>::bytes>();
  __shared__ __attribute__((aligned(16))) char smem_raw[kSmem];
  lds_t* smem = (lds_t*)smem_raw;
  const int u = xcd_tile(blockIdx.x, p.round, gridDim.x);
  int tile = u, kpart = -1, pair = 0;
  if constexpr (TS::BM == 256) {
    if (u >= p.n_full) {
      const int v = u - p.n_full;
      if (!kSplitEnabled || !p.sk_part) {
        using TH = Tile<128, TS::BN, TS::WM, TS::WN>;
        chunked_tile<E, BT, TH, O, KT>(p, smem, p.n_full + (v >> 1), v & 1, 1u);
        return;
      }
      tile = p.n_full + (v >> 1);
      kpart = v & 1;
      pair = v >> 1;
    }
  }
  // one call site, so the main loop is inlined once for whole and split tiles
  chunked_tile<E, BT, TS, O, KT>(p, smem, tile, 0, 2u, kpart, pair);
}

// ---------------------------------------------------------------- host side


template <Elem E, bool BT, class TS, Out O>
static hipError_t launch_chunked(const ChunkedArgs& a, int blocks, hipStream_t s) {
  if constexpr (TS::NW == 4) {
    if (a.ks.k % (kKBytes / ElemInfo<E>::bytes) == 0) {
      hipLaunchKernelGGL((chunked_gemm_kernel<E, BT, TS, O, false>), dim3(blocks), dim3(TS::NT), 0,
                         s, a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((chunked_gemm_kernel<E, BT, TS, O, true>), dim3(blocks), dim3(TS::NT), 0, s, a);
  return hipGetLastError();
}

// Instantiated combinations: F16 -> {F16, F32}; BF16 -> {BF16, F32};
// I8 -> {BF16, F16, F32, I32} (eight-wave tiles, and four-wave 128-row
// tiles).
template <bool BT, class TS>
static hipError_t dispatch_chunked(int in_dtype, int out_dtype, const ChunkedArgs& a, int blocks,
                                   hipStream_t s) {
  if (in_dtype == MC2_F16)
    return out_dtype == MC2_F32 ? launch_chunked<Elem::F16, BT, TS, Out::F32>(a, blocks, s)
                                : launch_chunked<Elem::F16, BT, TS, Out::F16>(a, blocks, s);
  if (in_dtype == MC2_BF16)
    return out_dtype == MC2_F32 ? launch_chunked<Elem::BF16, BT, TS, Out::F32>(a, blocks, s)
                                : launch_chunked<Elem::BF16, BT, TS, Out::BF16>(a, blocks, s);
  if constexpr (TS::NW == 4 && TS::BM == 256) {
    return hipErrorInvalidValue;
  } else {
    switch (out_dtype) {
      case MC2_BF16: return launch_chunked<Elem::I8, BT, TS, Out::BF16>(a, blocks, s);
      case MC2_F16: return launch_chunked<Elem::I8, BT, TS, Out::F16>(a, blocks, s);
      case MC2_F32: return launch_chunked<Elem::I8, BT, TS, Out::F32>(a, blocks, s);
      default: return launch_chunked<Elem::I8, BT, TS, Out::I32>(a, blocks, s);
    }
  }
}

// The last dispatch round (one workgroup per CU at a time) of `tiles`
// 256-row tiles, when it is at most half full: its tile count, else 0.
static int64_t thin_tail(int64_t tiles, int64_t cus) {
  const int64_t rem = tiles % cus;
  return rem > 0 && 2 * rem <= cus ? rem : 0;
}

// Tiles of one chunk cut into `sub` pieces (sq rows, one more for the first
// sr), for tiles of bm rows and tn tile columns.
static int64_t chunk_tiles(int64_t sq, int sr, int sub, int bm, int64_t tn) {
  return (sr * ((sq + bm) / bm) + (sub - sr) * ((sq + bm - 1) / bm)) * tn;
}

// K loops shorter than this many stages are not split: two 128 KiB partial
// transfers per workgroup cost about as much as 4 stages.
constexpr int kSplitMinStages = 16;


// Tile shape for a problem: 0 = 256 x 256, 1 = 128 x 256. Costs are counted
// in eighths of a round of 256 x 256 tiles: a thin last round costs 5 when
// its tiles are split in K (half the loop, plus the exchange), else 6 (as
// 128-row halves, which cost about 3/4 of a whole tile: measured on the
// 8192 x 3072 x 3072 share); a round of 128 x 256 tiles costs 6.
static int tile_shape(int64_t sq, int sr, int sub, int64_t n, int W, bool can_split) {
  const int64_t cus = num_cus();
  const int64_t tn = (n + 255) / 256;
  const int64_t tl = chunk_tiles(sq, sr, sub, 256, tn) * W;
  const int64_t tm = chunk_tiles(sq, sr, sub, 128, tn) * W;
  const int64_t rl = (tl + cus - 1) / cus, rm = (tm + cus - 1) / cus;
  const bool thin = thin_tail(tl, cus) > 0;
  // without a split, a thin last round of a single round stays whole tiles
  const int64_t last = thin && can_split ? 5 : thin && rl > 1 ? 6 : 8;
  const int64_t cost_l = 8 * (rl - 1) + last;
  const int64_t cost_m = 6 * rm;
  return cost_l <= cost_m ? 0 : 1;
}

int run_chunked(const void* x1, const void* x2, int64_t m, int64_t k, int64_t n, int W,
                int first_chunk, int nsim, int x2_trans, int in_dtype, const void* bias,
                const float* s1, const float* s2, int out_dtype, void* out, uint32_t* flags,
                uint32_t* counters, uint32_t epoch, int sub, hipStream_t stream,
                const InputWait& inw, void* split_ws, size_t split_ws_bytes) {
  const int es = in_dtype == MC2_I8 ? 1 : 2;
  const int os = (out_dtype == MC2_F32 || out_dtype == MC2_I32) ? 4 : 2;
  ChunkedArgs a{};
  a.A = static_cast<const char*>(x1);
  a.B = static_cast<const char*>(x2);
  a.out = static_cast<char*>(out);
  a.bias = bias;
  a.s1 = s1;
  a.s2 = s2;
  a.m = m;
  a.n = n;
  a.lda = k * es;
  a.ldb = (x2_trans ? k : n) * es;
  a.ldo = n * os;
  const int ke = kKBytes / es;  // K values per main-loop stage
  a.ks.k = k;
  a.ks.a_shard = m * k * es;
  a.ks.b_shard = k * n * es;
  a.ks.ktiles = static_cast<int>((k + ke - 1) / ke);
  a.ks.niters = a.ks.ktiles * nsim;
  a.mc = m / W;
  a.world = W;
  a.first_chunk = first_chunk;
  a.sub = sub;
  a.sq = a.mc / sub;
  a.sr = static_cast<int>(a.mc % sub);
  const int64_t cus = num_cus();
  const bool can_split = kSplitEnabled && split_ws != nullptr &&
                         a.ks.niters >= kSplitMinStages && cus / 2 * 4 * 4 <= kSplitCtlBytes;
  const bool tall = tile_shape(a.sq, a.sr, sub, n, W, can_split) == 0;
  const int BM = tall ? TileL::BM : TileM::BM;
  const int BN = TileL::BN;
  a.tiles_m1 = static_cast<int>((a.sq + BM) / BM);
  a.tiles_m0 = static_cast<int>((a.sq + BM - 1) / BM);
  a.tiles_n = static_cast<int>((n + BN - 1) / BN);
  a.tiles_long = a.tiles_m1 * a.tiles_n;
  a.tiles_short = a.tiles_m0 * a.tiles_n;
  const int64_t per_chunk = chunk_tiles(a.sq, a.sr, sub, BM, a.tiles_n);
  if (per_chunk * W > 0x3fffffff) return MC2_ERR_SHAPE;
  a.tiles_per_chunk = static_cast<int>(per_chunk);
  a.round = static_cast<int>(num_cus() / 8 * 8);
  a.bias_mul = static_cast<float>(nsim);
  a.flags = flags;
  a.counters = counters;
  a.epoch = epoch;
  // a tile's stores address at most 256 rows from its first: the buffer offsets
  // of the write-through path stay below 2^31
  a.store_wt = flags != nullptr && a.ldo * 256 < 0x7fff0000LL;
  a.in_flags = inw.flags;
  a.in_epoch = inw.epoch;
  a.spin_limit = inw.spin_limit;
  a.dev_err = inw.dev_err;
  a.own_chunk = first_chunk;
  const int64_t tiles = static_cast<int64_t>(a.tiles_per_chunk) * W;
  if (tiles > 0x3fffffff) return MC2_ERR_SHAPE;
  // A thin last round runs split in K (when the workspace holds its pairs) or
  // as half tiles after a full round (see the kernel).
  int64_t blocks = tiles;
  a.n_full = static_cast<int>(tiles);
  const int64_t rem = tall ? thin_tail(tiles, cus) : 0;
  if (rem > 0 && can_split &&
      static_cast<size_t>(kSplitCtlBytes + rem * 2 * kPartBytes) <= split_ws_bytes) {
    a.sk_ctl = static_cast<uint32_t*>(split_ws);
    a.sk_part = static_cast<char*>(split_ws) + kSplitCtlBytes;
    a.sk_alone = g_split_policy.load(std::memory_order_relaxed) == MC2_SPLIT_ALONE;
    a.n_full = static_cast<int>(tiles - rem);
    blocks = tiles + rem;
  } else if (rem > 0 && tiles > rem) {
    a.n_full = static_cast<int>(tiles - rem);
    blocks = tiles + rem;
  }
  // The four-wave loop runs 16-bit inputs in both B layouts and int8 in
  // 128-row tiles in both B layouts; int8 256-row tiles run the eight-wave
  // loop.
  hipError_t e;
  if (x2_trans && es == 1 && tall)
    e = dispatch_chunked<true, TileL>(in_dtype, out_dtype, a, (int)blocks, stream);
  else if (x2_trans)
    e = tall ? dispatch_chunked<true, TileW>(in_dtype, out_dtype, a, (int)blocks, stream)
             : dispatch_chunked<true, TileWM>(in_dtype, out_dtype, a, (int)blocks, stream);
  else if (es == 2)
    e = tall ? dispatch_chunked<false, TileW>(in_dtype, out_dtype, a, (int)blocks, stream)
             : dispatch_chunked<false, TileWM>(in_dtype, out_dtype, a, (int)blocks, stream);
  else
    e = tall ? dispatch_chunked<false, TileL>(in_dtype, out_dtype, a, (int)blocks, stream)
             : dispatch_chunked<false, TileWM>(in_dtype, out_dtype, a, (int)blocks, stream);
  return e == hipSuccess ? MC2_OK : MC2_ERR_HIP;
}

}  // namespace mc2

using namespace mc2;

extern "C" int mc2_mm_rs_local(const void* x1, const void* x2, int64_t m, int64_t k, int64_t n,
                               int world_size, int rank, int nsim, int x2_trans, int in_dtype,
                               const void* bias, const float* x1_scale, const float* x2_scale,
                               int out_dtype, void* out, uint32_t* ready_flags,
                               uint32_t* flag_counters, uint32_t epoch, int comm_turn,
                               void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!x1 || !x2 || !out) return MC2_ERR_NULL;
  if (workspace && !aligned16(workspace)) return MC2_ERR_ALIGN;
  if (!valid_world(world_size) || rank < 0 || rank >= world_size) return MC2_ERR_SHAPE;
  if (m <= 0 || n <= 0 || m % world_size) return MC2_ERR_SHAPE;
  if (k < 256 || k >= 65535) return MC2_ERR_SHAPE;
  if (nsim != 1 && nsim != world_size) return MC2_ERR_SHAPE;
  if (in_dtype != MC2_F16 && in_dtype != MC2_BF16 && in_dtype != MC2_I8) return MC2_ERR_DTYPE;
  const bool quant = in_dtype == MC2_I8;
  if (quant) {
    if (nsim != 1) return MC2_ERR_UNSUPPORTED;
    if (out_dtype == MC2_I32) {
      if (x1_scale || x2_scale || bias) return MC2_ERR_DTYPE;
    } else if (out_dtype == MC2_BF16 || out_dtype == MC2_F16 || out_dtype == MC2_F32) {
      if (!x1_scale || !x2_scale) return MC2_ERR_NULL;
    } else {
      return MC2_ERR_DTYPE;
    }
    if (k % 16 || n % 16) return MC2_ERR_ALIGN;
  } else {
    if (out_dtype != in_dtype && out_dtype != MC2_F32) return MC2_ERR_DTYPE;
    if (x1_scale || x2_scale) return MC2_ERR_DTYPE;
    if (k % 8 || n % 8) return MC2_ERR_ALIGN;
  }
  if (!aligned16(x1) || !aligned16(x2) || !aligned16(out)) return MC2_ERR_ALIGN;
  const int es = quant ? 1 : 2;
  if (!offsets_fit(k * es, (x2_trans ? k : n) * es)) return MC2_ERR_UNSUPPORTED;
  if ((ready_flags == nullptr) != (flag_counters == nullptr)) return MC2_ERR_NULL;
  if (ready_flags && epoch == 0) return MC2_ERR_SHAPE;
  if (comm_turn < 0 || comm_turn > m / world_size) return MC2_ERR_SHAPE;
  const int first = (rank + 1) % world_size;
  return run_chunked(x1, x2, m, k, n, world_size, first, nsim, x2_trans, in_dtype, bias, x1_scale,
                     x2_scale, out_dtype, out, ready_flags, flag_counters, epoch,
                     comm_turn > 1 ? comm_turn : 1, stream, InputWait{}, workspace, workspace_bytes);
}

static int check_ag(const void* x_gathered, const void* x2, int64_t m_c, int64_t k, int64_t n,
                    int world_size, int rank, int x2_trans, int in_dtype, void* out,
                    uint32_t* ready_flags, uint32_t* flag_counters, uint32_t epoch,
                    int comm_turn, const void* workspace) {
  if (!x_gathered || !x2 || !out) return MC2_ERR_NULL;
  if (workspace && !aligned16(workspace)) return MC2_ERR_ALIGN;
  if (!valid_world(world_size) || rank < 0 || rank >= world_size) return MC2_ERR_SHAPE;
  if (m_c <= 0 || n <= 0 || k <= 0) return MC2_ERR_SHAPE;
  if (in_dtype != MC2_F16 && in_dtype != MC2_BF16) return MC2_ERR_DTYPE;
  if (k % 8 || n % 8) return MC2_ERR_ALIGN;
  if (!aligned16(x_gathered) || !aligned16(x2) || !aligned16(out)) return MC2_ERR_ALIGN;
  if (!offsets_fit(k * 2, (x2_trans ? k : n) * 2)) return MC2_ERR_UNSUPPORTED;
  if ((ready_flags == nullptr) != (flag_counters == nullptr)) return MC2_ERR_NULL;
  if (ready_flags && epoch == 0) return MC2_ERR_SHAPE;
  if (comm_turn < 0 || comm_turn > m_c) return MC2_ERR_SHAPE;
  return MC2_OK;
}

extern "C" int mc2_ag_mm_local_inflags(const void* x_gathered, const void* x2, int64_t m_c,
                                       int64_t k, int64_t n, int world_size, int rank,
                                       int x2_trans, int in_dtype, const void* bias, void* out,
                                       uint32_t* ready_flags, uint32_t* flag_counters,
                                       uint32_t epoch, int comm_turn, const uint32_t* in_flags,
                                       uint32_t in_epoch, uint32_t spin_limit, int32_t* dev_err,
                                       void* workspace, size_t workspace_bytes,
                                       hipStream_t stream) {
  const int st = check_ag(x_gathered, x2, m_c, k, n, world_size, rank, x2_trans, in_dtype, out,
                          ready_flags, flag_counters, epoch, comm_turn, workspace);
  if (st) return st;
  if (!in_flags) return MC2_ERR_NULL;
  if (in_epoch == 0 || spin_limit == 0) return MC2_ERR_SHAPE;
  InputWait w;
  w.flags = in_flags;
  w.epoch = in_epoch;
  w.spin_limit = spin_limit;
  w.dev_err = dev_err;
  return run_chunked(x_gathered, x2, m_c * world_size, k, n, world_size, rank, 1, x2_trans,
                     in_dtype, bias, nullptr, nullptr, in_dtype, out, ready_flags, flag_counters,
                     epoch, comm_turn > 1 ? comm_turn : 1, stream, w, workspace, workspace_bytes);
}

extern "C" int mc2_ag_mm_local(const void* x_gathered, const void* x2, int64_t m_c, int64_t k,
                               int64_t n, int world_size, int rank, int x2_trans, int in_dtype,
                               const void* bias, void* out, uint32_t* ready_flags,
                               uint32_t* flag_counters, uint32_t epoch, int comm_turn,
                               void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const int st = check_ag(x_gathered, x2, m_c, k, n, world_size, rank, x2_trans, in_dtype, out,
                          ready_flags, flag_counters, epoch, comm_turn, workspace);
  if (st) return st;
  return run_chunked(x_gathered, x2, m_c * world_size, k, n, world_size, rank, 1, x2_trans,
                     in_dtype, bias, nullptr, nullptr, in_dtype, out, ready_flags, flag_counters,
                     epoch, comm_turn > 1 ? comm_turn : 1, stream, InputWait{}, workspace,
                     workspace_bytes);
}

extern "C" size_t mc2_split_workspace_size(void) {
  return static_cast<size_t>(kSplitCtlBytes) +
         static_cast<size_t>(num_cus() / 2) * 2 * static_cast<size_t>(kPartBytes);
}

extern "C" int mc2_set_split_policy(int policy) {
  if (policy != MC2_SPLIT_PAIR && policy != MC2_SPLIT_ALONE) return MC2_ERR_SHAPE;
  g_split_policy.store(policy, std::memory_order_relaxed);
  return MC2_OK;
}
