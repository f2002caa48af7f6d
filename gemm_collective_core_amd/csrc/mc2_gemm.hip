// Rank-chunked GEMM (MatmulReduceScatter / AllGatherMatmul compute share), for
// gfx950.
//
// Formulas: torch_npu.npu_mm_reduce_scatter_base API doc, "功能说明" (basic and
// quantized MatmulReduceScatter); CANN hccl issue 158 (AllGatherMatmul).
#include "mc2_chunked.hpp"

namespace mc2 {

// ---------------------------------------------------------------- chunked GEMM

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

// One output tile (or the row half `half` of one, for a TS of half height):
// main loop, epilogue, store, and the segment's ready flag. Tiles are numbered
// chunk by chunk in the order the chunks are due (first_chunk,
// first_chunk + 1, ... mod W), inside a chunk piece by piece in row order, and
// inside a piece row-block fastest, so that a run of consecutive tiles forms a
// compact block and the segments complete roughly in order. `weight` is the
// tile's share of the segment counter (2 for a whole tile, 1 for a half).
template <Elem E, bool BT, class TS, Out O, bool KT>
__device__ __forceinline__ void chunked_tile(const ChunkedArgs& p, lds_t* smem, int tile, int half,
                                             uint32_t weight) {
  constexpr int OS = OutInfo<O>::bytes;
  const int seq = tile / p.tiles_per_chunk;
  int t = tile - seq * p.tiles_per_chunk;
  int c = p.first_chunk + seq;
  c = c >= p.world ? c - p.world : c;
  const int long_tiles = p.sr * p.tiles_long;
  int j, tiles_mj, seg_tiles;
  if (t < long_tiles) {
    j = t / p.tiles_long;
    t -= j * p.tiles_long;
    tiles_mj = p.tiles_m1;
    seg_tiles = p.tiles_long;
  } else {
    const int v = (t - long_tiles) / p.tiles_short;
    j = p.sr + v;
    t -= long_tiles + v * p.tiles_short;
    tiles_mj = p.tiles_m0;
    seg_tiles = p.tiles_short;
  }
  const int g = c * p.sub + j;
  const int64_t seg_row0 = c * p.mc + j * p.sq + (j < p.sr ? j : p.sr);
  const int64_t row_end = seg_row0 + p.sq + (j < p.sr ? 1 : 0);
  const int tm = t % tiles_mj, tn = t / tiles_mj;
  const int64_t row0 = seg_row0 + static_cast<int64_t>(tm) * (TS::BM << (weight == 1)) +
                       static_cast<int64_t>(half) * TS::BM;
  const int64_t col0 = static_cast<int64_t>(tn) * TS::BN;

  if (p.in_flags && c != p.own_chunk) wait_input_segment(p, g);
  // the lower half of a tile that overhangs its piece may hold no rows
  if (row0 < row_end) {
  typename Mma<E>::acc_t acc[TS::FM][TS::FN];
  BDesc bd{p.B, p.ldb, p.n};
  PlainCols cm{col0, p.n - 16 / ElemInfo<E>::bytes};
  if constexpr (TS::NW == 4)
    mainloop_w4<E, BT, TS, KT>(smem, p.A, p.lda, row0, row_end - 1, bd, col0, cm, p.ks, acc);
  else
    mainloop<E, BT, TS>(smem, p.A, p.lda, row0, row_end - 1, bd, col0, cm, p.ks, acc);

  if constexpr (OS == 2) {
    // 16-bit outputs: stage the tile in LDS, then 16-byte coalesced stores.
    constexpr int pitch = TS::BN * OS + 16;
    epilogue_linear<E, TS, O>(acc, row0, row_end - 1, col0, p.n, p.bias, p.bias_mul, p.s1, p.s2,
                              [&](int r, int cc, float v) { put_out<O>(smem + r * pitch + cc * OS, v); });
    __syncthreads();
    store_staged<TS::NT>(smem, pitch, TS::BN * OS, TS::BM, p.out + row0 * p.ldo, p.ldo,
                         row_end - row0, col0 * OS, p.n * OS, p.store_wt != 0);
  } else {
    // 32-bit test outputs: stored straight from the accumulator layout.
    char* base = p.out + row0 * p.ldo + col0 * OS;
    const int64_t nrows = row_end - row0, ncols = p.n - col0;
    epilogue_linear<E, TS, O>(acc, row0, row_end - 1, col0, p.n, p.bias, p.bias_mul, p.s1, p.s2,
                              [&](int r, int cc, auto v) {
                                if (r < nrows && cc < ncols) put_out_global<O>(base + r * p.ldo + cc * OS, v);
                              });
  }
  }

  if (p.flags) {
    // Each wave waits for its own stores; after the barrier, thread 0's
    // agent-scope release (one L2 write-back per tile) covers the whole tile
    // before the tile is counted. Only the last tile of a chunk acquires the
    // other tiles' releases (an acquire invalidates this XCD's L2, so it is
    // kept off the other tiles) and then publishes the epoch with a
    // system-scope release store.
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
}

// One workgroup per work unit. With 256-row tiles, a last dispatch round
// that would leave more than half of the CUs idle is run as half tiles
// instead (units n_full.. map to the two row halves of tiles n_full..): the
// round then ends after a 128-row tile's time. Each half still sums all of K
// once, so results do not depend on the split.
// KT: the K extent of a shard may end inside a stage (four-wave tiles
// only; the eight-wave loop always checks).
template <Elem E, bool BT, class TS, Out O, bool KT>
__global__ __launch_bounds__(TS::NT, 1) void chunked_gemm_kernel(ChunkedArgs p) {
  constexpr int kSmem = chunked_smem<TS, OutInfo<O>::bytes>();
  __shared__ __attribute__((aligned(16))) char smem_raw[kSmem];
  lds_t* smem = (lds_t*)smem_raw;
  const int u = xcd_tile(blockIdx.x, p.round, gridDim.x);
  if constexpr (TS::BM == 256) {
    using TH = Tile<128, TS::BN, TS::WM, TS::WN>;
    if (u >= p.n_full) {
      const int v = u - p.n_full;
      chunked_tile<E, BT, TH, O, KT>(p, smem, p.n_full + (v >> 1), v & 1, 1u);
      return;
    }
  }
  chunked_tile<E, BT, TS, O, KT>(p, smem, u, 0, 2u);
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
// I8 -> {BF16, F16, F32, I32} (eight-wave tiles, and four-wave 128-row tiles
// with B given (n, k)).
template <bool BT, class TS>
static hipError_t dispatch_chunked(int in_dtype, int out_dtype, const ChunkedArgs& a, int blocks,
                                   hipStream_t s) {
  if (in_dtype == MC2_F16)
    return out_dtype == MC2_F32 ? launch_chunked<Elem::F16, BT, TS, Out::F32>(a, blocks, s)
                                : launch_chunked<Elem::F16, BT, TS, Out::F16>(a, blocks, s);
  if (in_dtype == MC2_BF16)
    return out_dtype == MC2_F32 ? launch_chunked<Elem::BF16, BT, TS, Out::F32>(a, blocks, s)
                                : launch_chunked<Elem::BF16, BT, TS, Out::BF16>(a, blocks, s);
  if constexpr (TS::NW == 4 && (TS::BM == 256 || !BT)) {
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

// Whether a last dispatch round (one workgroup per CU at a time) of 256-row
// tiles is at most half full: it then runs as 128-row half tiles. A 128-row
// tile costs about 3/4 of a 256-row one (measured on the 8192 x 3072 x 3072
// share), so such a round costs 3/4 of a round.
static bool half_tail(int64_t tiles, int64_t cus) {
  const int64_t rem = tiles % cus;
  return rem > 0 && tiles > rem && 2 * rem <= cus;
}

// Tiles of one chunk cut into `sub` pieces (sq rows, one more for the first
// sr), for tiles of bm rows and tn tile columns.
static int64_t chunk_tiles(int64_t sq, int sr, int sub, int bm, int64_t tn) {
  return (sr * ((sq + bm) / bm) + (sub - sr) * ((sq + bm - 1) / bm)) * tn;
}

// Tile shape for a problem: 0 = 256 x 256 (a last round at most half full
// runs as 128-row halves), 1 = 128 x 256. Costs are counted in quarter
// rounds of 256 x 256 tiles; a 128 x 256 tile counts 3.
static int tile_shape(int64_t sq, int sr, int sub, int64_t n, int W) {
  const int64_t cus = num_cus();
  const int64_t tn = (n + 255) / 256;
  const int64_t tl = chunk_tiles(sq, sr, sub, 256, tn) * W;
  const int64_t tm = chunk_tiles(sq, sr, sub, 128, tn) * W;
  const int64_t rl = (tl + cus - 1) / cus, rm = (tm + cus - 1) / cus;
  const int64_t cost_l = half_tail(tl, cus) ? 4 * (rl - 1) + 3 : 4 * rl;
  const int64_t cost_m = 3 * rm;
  return cost_l <= cost_m ? 0 : 1;
}

int run_chunked(const void* x1, const void* x2, int64_t m, int64_t k, int64_t n, int W,
                int first_chunk, int nsim, int x2_trans, int in_dtype, const void* bias,
                const float* s1, const float* s2, int out_dtype, void* out, uint32_t* flags,
                uint32_t* counters, uint32_t epoch, int sub, hipStream_t stream,
                const InputWait& inw) {
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
  const bool tall = tile_shape(a.sq, a.sr, sub, n, W) == 0;
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
  // A last round filled to at most half runs as half tiles (see the kernel).
  int64_t blocks = tiles;
  a.n_full = static_cast<int>(tiles);
  if (tall && half_tail(tiles, num_cus())) {
    const int64_t rem = tiles % num_cus();
    a.n_full = static_cast<int>(tiles - rem);
    blocks = tiles + rem;
  }
  // 16-bit inputs run the four-wave loop in both B layouts; int8 with B
  // given (n, k) runs it in 128-row tiles (a load-path-bound share that never
  // fills enough 256-row tiles); int8 with row-major B runs the eight-wave loop.
  hipError_t e;
  if (tall && es == 2)
    e = x2_trans ? dispatch_chunked<true, TileW>(in_dtype, out_dtype, a, (int)blocks, stream)
                 : dispatch_chunked<false, TileW>(in_dtype, out_dtype, a, (int)blocks, stream);
  else if (tall)
    e = x2_trans ? dispatch_chunked<true, TileL>(in_dtype, out_dtype, a, (int)blocks, stream)
                 : dispatch_chunked<false, TileL>(in_dtype, out_dtype, a, (int)blocks, stream);
  else if (x2_trans || es == 2)
    e = x2_trans ? dispatch_chunked<true, TileWM>(in_dtype, out_dtype, a, (int)blocks, stream)
                 : dispatch_chunked<false, TileWM>(in_dtype, out_dtype, a, (int)blocks, stream);
  else
    e = dispatch_chunked<false, TileM>(in_dtype, out_dtype, a, (int)blocks, stream);
  return e == hipSuccess ? MC2_OK : MC2_ERR_HIP;
}

}  // namespace mc2

using namespace mc2;

extern "C" int mc2_mm_rs_local(const void* x1, const void* x2, int64_t m, int64_t k, int64_t n,
                               int world_size, int rank, int nsim, int x2_trans, int in_dtype,
                               const void* bias, const float* x1_scale, const float* x2_scale,
                               int out_dtype, void* out, uint32_t* ready_flags,
                               uint32_t* flag_counters, uint32_t epoch, int comm_turn,
                               hipStream_t stream) {
  if (!x1 || !x2 || !out) return MC2_ERR_NULL;
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
                     comm_turn > 1 ? comm_turn : 1, stream);
}

static int check_ag(const void* x_gathered, const void* x2, int64_t m_c, int64_t k, int64_t n,
                    int world_size, int rank, int x2_trans, int in_dtype, void* out,
                    uint32_t* ready_flags, uint32_t* flag_counters, uint32_t epoch,
                    int comm_turn) {
  if (!x_gathered || !x2 || !out) return MC2_ERR_NULL;
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
                                       hipStream_t stream) {
  const int st = check_ag(x_gathered, x2, m_c, k, n, world_size, rank, x2_trans, in_dtype, out,
                          ready_flags, flag_counters, epoch, comm_turn);
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
                     epoch, comm_turn > 1 ? comm_turn : 1, stream, w);
}

extern "C" int mc2_ag_mm_local(const void* x_gathered, const void* x2, int64_t m_c, int64_t k,
                               int64_t n, int world_size, int rank, int x2_trans, int in_dtype,
                               const void* bias, void* out, uint32_t* ready_flags,
                               uint32_t* flag_counters, uint32_t epoch, int comm_turn,
                               hipStream_t stream) {
  const int st = check_ag(x_gathered, x2, m_c, k, n, world_size, rank, x2_trans, in_dtype, out,
                          ready_flags, flag_counters, epoch, comm_turn);
  if (st) return st;
  return run_chunked(x_gathered, x2, m_c * world_size, k, n, world_size, rank, 1, x2_trans,
                     in_dtype, bias, nullptr, nullptr, in_dtype, out, ready_flags, flag_counters,
                     epoch, comm_turn > 1 ? comm_turn : 1, stream);
}
