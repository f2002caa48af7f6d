// Grouped GEMM of the MoE dispatch / combine pair (fc1 with fused SwiGLU, fc2)
// and its backward (input gradients with the weight read as (n, k) rows and a
// fused SwiGLU backward; weight gradients over the tokens of each expert), for
// gfx950.
//
// Formulas: "NPU Training Operators - MC2", "执行路径" (GroupedMatmul fc1 +
// swiglu, fc2); same page, "PR 改动" and "验证项" (the fused operators'
// backward, fc1 / fc2 gradients).
#include "mc2_tiles.hpp"

namespace mc2 {

// SwiGLU epilogue: tile column blocks alternate gate (even) and up (odd), so
// the fragments fn = 2p and 2p + 1 of a lane hold gate and up of the same
// output columns. h = silu(g) * u, silu(g) = g / (1 + exp(-g)), stored as
// bf16; the division is the hardware reciprocal (within 1 ulp of fp32, far
// below the bf16 rounding that follows), which costs 2 instructions instead
// of an IEEE division's dozen. The four-wave accumulators hold runs of four output columns per lane:
// one 8-byte LDS write per run (staged for whole-row stores).
template <class TS>
__device__ __forceinline__ void stage_swiglu(lds_t* smem, int pitch,
                                             const f32x4_t (&acc)[TS::FM][TS::FN]) {
  static_assert(AccLayout<TS>::kRowRuns, "runs of four columns");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wrow0 = (wave / TS::WN) * TS::WTM;
  const int wcol0 = (wave % TS::WN) * TS::WTN;
#pragma unroll
  for (int p = 0; p < TS::FN / 2; ++p) {
    const int lcol = wcol0 / 2 + p * 16 + 4 * (lane >> 4);
#pragma unroll
    for (int fm = 0; fm < TS::FM; ++fm) {
      const int lrow = wrow0 + fm * 16 + (lane & 15);
      float h[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float g = acc[fm][2 * p][i];
        const float u = acc[fm][2 * p + 1][i];
        h[i] = g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
      }
      *reinterpret_cast<MC2_LDS u32x2_t*>(smem + lrow * pitch + lcol * 2) = pack4<Out::BF16>(h);
    }
  }
}

// ---------------------------------------------------------------- grouped GEMM

// Values read from shared memory are per-lane as far as the compiler knows;
// the ones that feed buffer descriptors and loop bounds are made wave-uniform
// (scalar registers), or every load would run in a per-lane loop.
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int64_t uni(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(static_cast<uint64_t>(v) >> 32));
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

constexpr int kMaxLocalExperts = 256;

struct GroupedArgs {
  const char* A;
  int64_t lda;
  const char* B;
  int64_t ldb, b_group;   // bytes per B row, bytes per expert
  char* out;
  int64_t ldo;
  int64_t K;              // contraction length
  int64_t n_b;            // columns of B per expert
  int64_t n_out;          // output columns
  int64_t inter;          // SwiGLU: output columns (= n_b / 2)
  const int32_t* send_counts;
  const int32_t* recv_counts;
  int ep_rank, num_experts, local_experts;
  int combine;            // 0: rows read at the send offset; 1: rows written there
  int64_t a_cap, o_cap;   // row capacities of the A and output buffers
  int32_t* dev_err;
  int ktiles;
  const char* gsave;      // SwiGLU backward: the fc1 pre-activation (rows, 2*inter) bf16
  int64_t ldg;            // bytes per gsave row
  uint32_t* zero;         // n_zero words that workgroup 0 clears first (the backward's
  int64_t n_zero;         // weight-gradient tile counters, used by the next launch), or null
};

// Epilogue of the grouped kernel.
enum GroupedMode : int {
  kLinear = 0,   // out = acc (bf16)
  kSwiglu = 1,   // out = silu(gate) * up of the interleaved gate / up columns
  kSwigluBwd = 2 // acc = gradient of the SwiGLU output; out = gradient of its input
};

struct GluCols {
  // Tile column j (16-column blocks alternate gate / up) -> global B column,
  // clamped to the last 16-byte block; clamped columns only feed output
  // columns >= inter, which are never stored.
  int64_t j0, inter, last_block;
  __device__ __forceinline__ int64_t operator()(int j) const {
    const int cb = j >> 4;
    const int64_t base = (cb & 1) ? inter : 0;
    const int64_t c = base + j0 + (cb >> 1) * 16 + (j & 15);
    return c < last_block ? c : last_block;
  }
};

// The SwiGLU backward epilogue (below) works in quarters of 64 rows: fp32 dA
// rows (padded) and then the bf16 gate / up rows.
constexpr int kSbQRows = 64;

template <class TS>
constexpr int swiglu_bwd_smem() {
  return kSbQRows * (TS::BN * 4 + 16) + kSbQRows * TS::BN * 4;
}

template <class TS, int MODE>
constexpr int grouped_smem() {
  // kSwigluBwd stages 64 rows of fp32 dA and of gate / up at a time
  constexpr int stage = MODE == kSwigluBwd ? swiglu_bwd_smem<TS>()
                                           : TS::BM * ((MODE == kSwiglu ? TS::BN / 2 : TS::BN) * 2 + 16);
  return TS::kStages * TS::kStageBytes > stage ? TS::kStages * TS::kStageBytes : stage;
}

// SwiGLU backward epilogue: the accumulator holds dA, the gradient of the
// SwiGLU output, for output rows [orow0, orow0 + nrows) and columns
// [ocol0, ocol0 + BN) of the inter columns. With the stored pre-activation
// (gate in columns [0, inter), up in [inter, 2 inter)):
//   d_gate = dA * up * s * (1 + gate * (1 - s)),  d_up = dA * gate * s,
//   s = 1 / (1 + exp(-gate)),
// written as bf16 to the same columns of `out`. The tile goes in quarters of
// 64 rows: dA into LDS in fp32, and the quarter's gate and up rows (1 KiB per
// row) into LDS with loads straight to LDS, all in flight at once; after one
// wait every thread handles 8 consecutive columns of a row from LDS and
// stores them with 16-byte stores. (Loading gate and up into registers
// piece by piece made every piece wait for the stores before it, which share
// the wait counter with the loads.)
template <class TS>
__device__ __forceinline__ void swiglu_bwd_epilogue(lds_t* smem, const f32x4_t (&acc)[TS::FM][TS::FN],
                                                    const GroupedArgs& p, int64_t orow0,
                                                    int64_t nrows, int64_t ocol0) {
  constexpr int QR = kSbQRows;
  constexpr int NQ = TS::BM / QR;
  constexpr int pitch = TS::BN * 4 + 16;  // fp32 dA row
  constexpr int GROW = TS::BN * 4;        // gate then up, bf16: one 1 KiB load per row
  constexpr int GB = QR * pitch;          // gate / up rows after the dA rows
  constexpr int CPR = TS::BN / 8;         // 8-column pieces per row
  static_assert(TS::NW == 4 && TS::BN == 256 && GROW == 1024, "1 KiB gate / up rows");
  static_assert(TS::WTM % QR == 0 && QR % (TS::NW * 4) == 0, "quarters inside one wave row");
  // The thread index through an assembly move: what is derived from it is
  // then computed here, after the main loop, and not kept live through it
  // (the compiler would hoist it and spill).
  int tid;
  asm volatile("v_mov_b32 %0, %1" : "=v"(tid) : "v"(static_cast<int>(threadIdx.x)));
  const int lane = tid & 63, wave = tid >> 6;
  const int wrow0 = (wave / TS::WN) * TS::WTM;
  const int wcol0 = (wave % TS::WN) * TS::WTN;
  // lane l of a row load: gate (l < 32) or up, 8 columns from ocol0 + 8 (l & 31)
  const int64_t gcol = ocol0 + 8 * (lane & 31);
  const bool col_ok = gcol < p.inter;
  const uint32_t coff = static_cast<uint32_t>(((lane >> 5) ? p.inter + gcol : gcol) * 2);
  for (int q = 0; q < NQ; ++q) {
    __syncthreads();  // every read of the previous quarter's LDS rows is done
    // dA of the quarter: the fragment rows fm0 .. fm0 + 3 of the waves whose
    // rows hold it (a compile-time choice per quarter: the accumulators are
    // registers)
    sfor<NQ>([&](auto Qc) {
      constexpr int qq = decltype(Qc)::value;
      constexpr int fm0 = (qq * QR % TS::WTM) / 16;
      if (q == qq && wrow0 == qq * QR / TS::WTM * TS::WTM) {
        // runs of four columns per lane (AccLayout of the four-wave tiles)
        static_assert(AccLayout<TS>::kRowRuns, "runs of four columns");
#pragma unroll
        for (int fn = 0; fn < TS::FN; ++fn) {
          const int lcol = wcol0 + fn * 16 + 4 * (lane >> 4);
#pragma unroll
          for (int f = 0; f < QR / 16; ++f) {
            const int lrow = f * 16 + (lane & 15);
            *reinterpret_cast<MC2_LDS f32x4_t*>(smem + lrow * pitch + lcol * 4) = acc[fm0 + f][fn];
          }
        }
      }
    });
    {
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.gsave + (orow0 + q * QR) * p.ldg);
      constexpr int RW = QR / TS::NW;  // rows loaded per wave
#pragma unroll
      for (int j = 0; j < RW; ++j) {
        const int r = wave * RW + j;
        const bool ok = col_ok && q * QR + r < nrows;
        dma16(rs, smem + GB + r * GROW, ok ? static_cast<uint32_t>(r * p.ldg) + coff : kOffNone);
      }
    }
    wait_vmcnt0();
    __syncthreads();
    // (not unrolled: the accumulators leave few registers for the LDS values)
#pragma unroll 2
    for (int it = tid; it < QR * CPR; it += TS::NT) {
      const int r = it / CPR, c8 = it - r * CPR;
      const int64_t row = q * QR + r;
      const int64_t col = ocol0 + c8 * 8;
      if (row >= nrows || col >= p.inter) continue;
      const MC2_LDS float* src = reinterpret_cast<const MC2_LDS float*>(smem + r * pitch + c8 * 32);
      const u32x4_t gv = *reinterpret_cast<const MC2_LDS u32x4_t*>(smem + GB + r * GROW + c8 * 16);
      const u32x4_t uv =
          *reinterpret_cast<const MC2_LDS u32x4_t*>(smem + GB + r * GROW + TS::BN * 2 + c8 * 16);
      u32x4_t dg, du;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t lo_g = 0, lo_u = 0;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const float da = src[2 * j + h];
          const float g = bf16_bits_to_f32((gv[j] >> (16 * h)) & 0xFFFFu);
          const float u = bf16_bits_to_f32((uv[j] >> (16 * h)) & 0xFFFFu);
          const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-g));  // as in stage_swiglu
          lo_g |= static_cast<uint32_t>(f32_to_bf16_bits(da * u * (sg * (1.0f + g * (1.0f - sg)))))
                  << (16 * h);
          lo_u |= static_cast<uint32_t>(f32_to_bf16_bits(da * (g * sg))) << (16 * h);
        }
        dg[j] = lo_g;
        du[j] = lo_u;
      }
      char* orow = p.out + (orow0 + row) * p.ldo;
      __builtin_nontemporal_store(dg, reinterpret_cast<u32x4_t*>(orow + col * 2));
      __builtin_nontemporal_store(du, reinterpret_cast<u32x4_t*>(orow + (p.inter + col) * 2));
    }
  }
}

// rows [0, BM/2) or [BM/2, BM) of a TS tile
template <class TS>
using TileHalf = Tile<TS::BM / 2, TS::BN, TS::WM, TS::WN>;

// KT: the contraction length may end inside a stage (four-wave tiles only;
// the eight-wave loop always checks).
template <class TS, int MODE, bool BT, bool KT>
__global__ __launch_bounds__(TS::NT, 1) void grouped_gemm_kernel(GroupedArgs p) {
  constexpr bool GLU = MODE == kSwiglu;
  static_assert(!(GLU && BT), "the interleaved gate / up columns need row-major weights");
  constexpr int kSmem = grouped_smem<TS, MODE>();
  __shared__ __attribute__((aligned(16))) char smem_raw[kSmem];
  lds_t* smem = (lds_t*)smem_raw;
  __shared__ int64_t s_gstart[kMaxLocalExperts + 1];
  __shared__ int64_t s_tstart[kMaxLocalExperts + 1];
  __shared__ int64_t s_base;
  __shared__ int32_t s_cnt[kMaxLocalExperts];
  __shared__ int s_bad;

  const int tid = threadIdx.x;
  const int El = p.local_experts;
  const int first = p.ep_rank * El;
  if constexpr (BT) {  // the input-gradient launches of the backward
    if (p.zero && blockIdx.x == 0)
      for (int64_t i = tid; i < p.n_zero; i += TS::NT) p.zero[i] = 0;
  }
  constexpr int OUTC = GLU ? TS::BN / 2 : TS::BN;  // output columns per tile
  const int64_t tiles_n = (p.n_out + OUTC - 1) / OUTC;

  // Counts -> group table.
  if (tid == 0) { s_base = 0; s_bad = 0; }
  __syncthreads();
  int64_t part = 0;
  for (int e = tid; e < first; e += TS::NT) {
    const int32_t v = p.send_counts[e];
    if (v < 0) s_bad = 1;
    part += v;
  }
  for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off);
  if ((tid & 63) == 0 && part) atomicAdd(reinterpret_cast<unsigned long long*>(&s_base),
                                         static_cast<unsigned long long>(part));
  // the counts are read in parallel (one load round trip, not one per
  // expert), then one thread scans them in shared memory
  for (int e = tid; e < El; e += TS::NT) {
    const int32_t rc = p.recv_counts[e];
    if (rc < 0 || rc != p.send_counts[first + e]) s_bad = 1;
    s_cnt[e] = rc > 0 ? rc : 0;
  }
  __syncthreads();
  if (tid == 0) {
    int64_t g = 0, tt = 0;
    for (int e = 0; e < El; ++e) {
      const int64_t c = s_cnt[e];
      s_gstart[e] = g;
      s_tstart[e] = tt;
      g += c;
      tt += (c + TS::BM - 1) / TS::BM * tiles_n;
    }
    s_gstart[El] = g;
    s_tstart[El] = tt;
  }
  __syncthreads();
  {
    const int64_t rows = s_gstart[El];
    const int64_t a_need = (p.combine ? 0 : s_base) + rows;
    const int64_t o_need = (p.combine ? s_base : 0) + rows;
    if (s_bad || a_need > p.a_cap || o_need > p.o_cap) {
      if (tid == 0 && blockIdx.x == 0) atomic_or_err(p.dev_err, MC2_DEVERR_COUNTS);
      return;
    }
  }
  const int64_t a_base = p.combine ? 0 : uni(s_base);
  const int64_t o_base = p.combine ? uni(s_base) : 0;
  const int64_t total = uni(s_tstart[El]);

  KSpan ks{p.K, 0, 0, p.ktiles, p.ktiles};
  // With one workgroup per CU (a multiple of 8), XCD x takes tiles 32x ..
  // 32x+31 of every round of the tile sequence (see xcd_tile).
  const int g8 = gridDim.x;
  const int64_t tfirst = (g8 % 8 == 0) ? (blockIdx.x & 7) * (g8 >> 3) + (blockIdx.x >> 3) : blockIdx.x;
  // Tile t of the sequence -> (group, row tile, column tile) for TS::BM-row tiles.
  struct Place {
    int g;
    int64_t tm, tn;
  };
  // Inside a group, tiles go in bands of `band` row blocks: a band's tiles
  // run row block fastest, column tile by column tile, and the bands follow
  // each other. With band x tiles_n close to the 32 tiles an XCD takes per
  // round, the tiles that share one L2 cover a few row blocks and all column
  // tiles (fc2: 4 x 8), instead of 32 row blocks of one column tile, so the
  // K slabs of each A row block and B column block are fetched into that L2
  // once for all the tiles that use them.
  const int64_t band = tiles_n < 32 ? 32 / tiles_n : 1;
  auto place = [&](int64_t t) {
    int g = 0;
    while (g + 1 < El && s_tstart[g + 1] <= t) ++g;
    g = uni(g);
    const int64_t cnt = uni(s_gstart[g + 1]) - uni(s_gstart[g]);
    const int64_t tiles_m = (cnt + TS::BM - 1) / TS::BM;
    const int64_t lt = t - uni(s_tstart[g]);
    // 64-bit divisions run on the vector ALU: their results are made uniform again
    const int64_t b = uni(lt / (band * tiles_n));
    const int64_t in_b = lt - b * band * tiles_n;
    const int64_t rows_b = tiles_m - b * band < band ? tiles_m - b * band : band;
    return Place{g, uni(b * band + in_b % rows_b), uni(in_b / rows_b)};
  };
  // One output tile of TSX::BM rows (TS, or its 128-row half) from row r0 of
  // group g, column tile tn.
  auto run_tile = [&](auto shape, int g, int64_t r0, int64_t tn) {
    using TSX = decltype(shape);
    static_assert(TSX::BN == TS::BN, "column tiles are shared by both shapes");
    const int64_t gs = uni(s_gstart[g]);
    const int64_t cnt = uni(s_gstart[g + 1]) - gs;
    const int64_t arow0 = a_base + gs + r0;
    const int64_t arow_end = a_base + gs + cnt;
    const int64_t orow0 = o_base + gs + r0;
    const int64_t ocol0 = tn * OUTC;

    f32x4_t acc[TSX::FM][TSX::FN];
    BDesc bd{p.B + g * p.b_group, p.ldb, p.n_b};
    if constexpr (GLU) {
      GluCols cm{ocol0, p.inter, p.n_b - 8};
      if constexpr (TSX::NW == 4)
        mainloop_w4<Elem::BF16, false, TSX, KT>(smem, p.A, p.lda, arow0, arow_end - 1, bd, 0, cm, ks,
                                                acc);
      else
        mainloop<Elem::BF16, false, TSX>(smem, p.A, p.lda, arow0, arow_end - 1, bd, 0, cm, ks, acc);
    } else {
      PlainCols cm{ocol0, p.n_b - 8};
      if constexpr (TSX::NW == 4)
        mainloop_w4<Elem::BF16, BT, TSX, KT>(smem, p.A, p.lda, arow0, arow_end - 1, bd, ocol0, cm, ks,
                                             acc);
      else
        mainloop<Elem::BF16, BT, TSX>(smem, p.A, p.lda, arow0, arow_end - 1, bd, ocol0, cm, ks, acc);
    }
    if constexpr (MODE == kSwigluBwd) {
      swiglu_bwd_epilogue<TSX>(smem, acc, p, orow0, arow_end - arow0, ocol0);
      __syncthreads();
      return;
    }
    constexpr int pitch = OUTC * 2 + 16;
    if constexpr (GLU)
      stage_swiglu<TSX>(smem, pitch, acc);
    else
      epilogue_quads<Elem::BF16, TSX, Out::BF16>(
          acc, orow0, 0, ocol0, p.n_out, nullptr, 0.f, nullptr, nullptr,
          [&](int rr, int cc, const auto& v) {
            *reinterpret_cast<MC2_LDS u32x2_t*>(smem + rr * pitch + cc * 2) = pack4<Out::BF16>(v);
          });
    __syncthreads();
    store_staged<TSX::NT>(smem, pitch, OUTC * 2, TSX::BM, p.out + orow0 * p.ldo, p.ldo, arow_end - arow0,
                 ocol0 * 2, p.n_out * 2);
    __syncthreads();
  };

  // All tiles have the same K, so the sequence runs in rounds of one tile per
  // workgroup. A last round filled to at most half runs as 128-row halves, two
  // workgroups per tile (consecutive tfirst values, so on one XCD).
  const int64_t G = gridDim.x;
  const int64_t rem = total % G;
  const bool halves = rem > 0 && 2 * rem <= G;
  const int64_t n_full = halves ? total - rem : total;
  for (int64_t t = tfirst; t < n_full; t += G) {
    const Place q = place(t);
    run_tile(TS{}, q.g, q.tm * TS::BM, q.tn);
  }
  if (halves && tfirst < 2 * rem) {
    const Place q = place(n_full + tfirst / 2);
    const int64_t r0 = q.tm * TS::BM + (tfirst & 1) * TileHalf<TS>::BM;
    if (r0 < uni(s_gstart[q.g + 1]) - uni(s_gstart[q.g])) run_tile(TileHalf<TS>{}, q.g, r0, q.tn);
  }
}

// ---------------------------------------------------------------- weight gradients

// Group table of the local experts from the device-side counts, in shared
// memory: row starts (gstart) and the send-buffer row of local expert 0
// (base). bad is set when the counts are negative or recv_counts disagree
// with the send counts of this rank's experts. The counts are read by many
// threads at once; one thread then sums them in shared memory.
struct GroupTable {
  int64_t gstart[kMaxLocalExperts + 1];
  int32_t cnt[kMaxLocalExperts];
  int64_t base;
  int bad;
};

__device__ __forceinline__ void load_group_table(GroupTable& t, const int32_t* send_counts,
                                                 const int32_t* recv_counts, int ep_rank, int El) {
  const int tid = threadIdx.x;
  const int first = ep_rank * El;
  if (tid == 0) { t.base = 0; t.bad = 0; }
  __syncthreads();
  int64_t part = 0;
  for (int e = tid; e < first; e += blockDim.x) {
    const int32_t v = send_counts[e];
    if (v < 0) t.bad = 1;
    part += v;
  }
  for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off);
  if ((tid & 63) == 0 && part) atomicAdd(reinterpret_cast<unsigned long long*>(&t.base),
                                         static_cast<unsigned long long>(part));
  for (int e = tid; e < El; e += blockDim.x) {
    const int32_t rc = recv_counts[e];
    if (rc < 0 || rc != send_counts[first + e]) t.bad = 1;
    t.cnt[e] = rc > 0 ? rc : 0;
  }
  __syncthreads();
  if (tid == 0) {
    int64_t g = 0;
    for (int e = 0; e < El; ++e) {
      t.gstart[e] = g;
      g += t.cnt[e];
    }
    t.gstart[El] = g;
  }
  __syncthreads();
}

constexpr int64_t kSliceRows = 4096;  // the shortest slice (workspace and grid bounds)

// Slice length L for N local rows over tiles_per_group tiles per expert on
// `cus` CUs: the rows of K per CU if the work were spread evenly, rounded down
// to a multiple of 2048, and at least kSliceRows. Longer slices mean fewer
// partial tiles and fixed costs, shorter ones a finer balance; on the MoE
// workload (40289 rows) this gives 4096 for fc2's 24 tiles per expert and
// 6144 for fc1's 48, the best of 3072 .. 8192 measured for each.
// (In single precision with the hardware reciprocal: a heuristic, computed
// the same way by every workgroup, and no 64-bit division.)
__device__ __forceinline__ int64_t slice_rows(int64_t n, int tiles_per_group, int cus) {
  const float per_cu = static_cast<float>(n) * static_cast<float>(tiles_per_group) *
                       __builtin_amdgcn_rcpf(static_cast<float>(cus > 0 ? cus : 1));
  const float blocks = per_cu * (1.0f / 2048.0f);
  const int64_t l = blocks < 1e6f ? static_cast<int64_t>(blocks) * 2048 : int64_t{1} << 31;
  return l > kSliceRows ? l : kSliceRows;
}

struct WgradArgs {
  const char* P;      // (rows, M) bf16, this rank's rows from row base (p_at_send) or 0
  int64_t ldp;        // bytes per P row
  int p_at_send;
  int64_t p_cap;
  const char* Q;      // (rows, N) bf16, this rank's rows from row base (at_send) or 0
  int64_t ldq;
  int at_send;
  int64_t q_cap;
  float* out;         // (E_l, M, N) fp32
  int64_t M, N;
  int tiles_m, tiles_n;
  int q;              // units per XCD per slice: ceil(tiles_m * tiles_n / 8)
  int cus;            // compute units (for the slice length)
  int bm, bn;         // an XCD's q tiles of a slice as a bm x bn block (bm = 0: a run of q)
  uint32_t* counters; // E_l * tiles_m * tiles_n, zero on entry (left zero)
  float* partials;    // max_slots slices' partial tiles of split groups
  int64_t max_slots;
  const int32_t* send_counts;
  const int32_t* recv_counts;
  int ep_rank, local_experts;
  int32_t* dev_err;
};

// dW[g] = P_g^T @ Q_g (M x N per local group g). Work unit = (group g, K
// slice s, tile): a 256 x 256 tile over rows [s*L, min((s+1)*L, count g)) of
// the group, L = slice_rows(local rows, ...). Both operands are the group's rows as they lie
// (P's rows for A, Q's for B), read k-major by the main loop: no transposed
// copy is made. Slices are numbered group by group, the groups with most rows
// first (so the longest units are dispatched first and the short ones fill
// the end of the launch). Workgroup b runs on XCD b % 8, and each XCD takes q
// tiles of every slice, slice after slice: the XCDs get the same unit
// lengths, so none of them is left with the long units while the others idle
// (numbering units in order and giving each XCD a run of 32 put the longest
// of every round on the same XCD). An XCD's q tiles of a slice form a
// bm x bn block where the tile grid splits into 8 such blocks, so that they
// share A and B slabs in that XCD's L2; else a run of q tiles in row-fastest
// order. A group of one slice stores its tile (non-temporal: the result is
// not read again here; the same hint on the partials below, which are read
// back, was slower); for a split group every slice stores its partial tile in
// its slot, and the last slice to finish a tile (counted with an agent-scope
// release / acquire, as the ready flags) sums the partials in slice order, so
// the result does not depend on timing. An empty group gets zeros. The grid
// may have more workgroups than units (the host knows only a bound); the
// rest exit. The tile counters start at zero: the input-gradient launch
// before this one clears them.
// KT: the K extent of a unit may end inside a stage.
template <class TS, bool KT>
__global__ __launch_bounds__(TS::NT, 1) void wgrad_kernel(WgradArgs p) {
  static_assert(TS::NW == 4 && TS::BM == 256, "four-wave 256-row tiles (row-major A)");
  constexpr int kSmem = TS::kStages * TS::kStageBytes;
  __shared__ __attribute__((aligned(16))) char smem_raw[kSmem];
  __shared__ GroupTable t;
  __shared__ int64_t s_sstart[kMaxLocalExperts + 1];  // first slice, by position in the order
  __shared__ int64_t s_slot[kMaxLocalExperts + 1];    // by group
  __shared__ int s_order[kMaxLocalExperts];           // position -> group
  __shared__ int s_ns[kMaxLocalExperts];              // slices, by group
  __shared__ int s_last;
  lds_t* smem = (lds_t*)smem_raw;
  load_group_table(t, p.send_counts, p.recv_counts, p.ep_rank, p.local_experts);
  const int El = p.local_experts;
  const int per_group = p.tiles_m * p.tiles_n;
  for (int e = threadIdx.x; e < El; e += TS::NT) {
    const int32_t c = t.cnt[e];
    int rank = 0;
    for (int f = 0; f < El; ++f) rank += t.cnt[f] > c || (t.cnt[f] == c && f < e);
    s_order[rank] = e;
  }
  __syncthreads();
  const int64_t L = uni(slice_rows(t.gstart[El], per_group, p.cus));
  // slices per group, one group per thread (32-bit: counts are int32 and
  // L < 2^31)
  for (int e = threadIdx.x; e < El; e += TS::NT) {
    const uint32_t c = static_cast<uint32_t>(t.cnt[e]), l = static_cast<uint32_t>(L);
    s_ns[e] = c > l ? static_cast<int>((c + l - 1) / l) : 1;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int64_t sl = 0, slot = 0;
    for (int q = 0; q < El; ++q) {
      const int e = s_order[q];
      const int64_t ns = s_ns[e];
      s_sstart[q] = sl;
      s_slot[e] = slot;
      sl += ns;
      slot += ns > 1 ? ns : 0;
    }
    s_sstart[El] = sl;
    s_slot[El] = slot;
  }
  __syncthreads();
  const int64_t base = p.at_send ? uni(t.base) : 0;
  const int64_t pbase = p.p_at_send ? uni(t.base) : 0;
  if (t.bad || base + t.gstart[El] > p.q_cap || pbase + t.gstart[El] > p.p_cap ||
      s_slot[El] > p.max_slots) {
    if (threadIdx.x == 0 && blockIdx.x == 0) atomic_or_err(p.dev_err, MC2_DEVERR_COUNTS);
    return;
  }
  const int x = static_cast<int>(blockIdx.x & 7);
  const int j = static_cast<int>(blockIdx.x >> 3);
  // integer division runs on the vector ALU: its results are made uniform again
  const int sig = uni(j / p.q);
  const int i = uni(j - sig * p.q);
  if (sig >= uni(s_sstart[El])) return;
  int tm, tn;
  if (p.bm) {
    const int xm = p.tiles_m / p.bm;
    tm = uni((x % xm) * p.bm + i % p.bm);
    tn = uni((x / xm) * p.bn + i / p.bm);
  } else {
    const int l = x * p.q + i;
    if (l >= per_group) return;
    tm = uni(l % p.tiles_m);
    tn = uni(l / p.tiles_m);
  }
  const int lt = tm + tn * p.tiles_m;
  int q = 0;
  while (q + 1 < El && s_sstart[q + 1] <= sig) ++q;
  q = uni(q);
  const int g = uni(s_order[q]);
  const int s = uni(static_cast<int>(sig - uni(s_sstart[q])));
  const int64_t row0 = static_cast<int64_t>(tm) * TS::BM;
  const int64_t col0 = static_cast<int64_t>(tn) * TS::BN;
  const int64_t cnt = uni(static_cast<int64_t>(t.cnt[g]));
  const int64_t nslices = uni(s_sstart[q + 1]) - uni(s_sstart[q]);
  const int64_t gstart = uni(t.gstart[g]);
  float* dst = p.out + static_cast<int64_t>(g) * p.M * p.N;
  const int64_t nrows = p.M - row0, ncols = p.N - col0;
  if (cnt == 0) {
    for (int i = threadIdx.x; i < TS::BM * TS::BN; i += TS::NT) {
      const int r = i / TS::BN, c = i - r * TS::BN;
      if (r < nrows && c < ncols) dst[(row0 + r) * p.N + col0 + c] = 0.0f;
    }
    return;
  }
  const int64_t k0 = static_cast<int64_t>(s) * L;
  const int64_t klen = cnt - k0 < L ? cnt - k0 : L;
  const int ktiles = static_cast<int>((klen + 63) / 64);
  KSpan ks{klen, 0, 0, ktiles, ktiles};
  f32x4_t acc[TS::FM][TS::FN];
  BDesc bd{p.Q + (base + gstart + k0) * p.ldq, p.ldq, p.N};
  PlainCols cm{col0, p.N - 8};
  // A = the group's rows of P, read k-major (row-major (k, m)) like B
  mainloop_w4<Elem::BF16, false, TS, KT, true>(smem, p.P + (pbase + gstart + k0) * p.ldp, p.ldp,
                                               row0, p.M - 1, bd, col0, cm, ks, acc);
  if (nslices == 1) {
    char* base_out = reinterpret_cast<char*>(dst + row0 * p.N + col0);
    // runs of four columns (N is a multiple of 8): one 16-byte store each
    epilogue_quads<Elem::BF16, TS, Out::F32>(
        acc, row0, p.M - 1, col0, p.N, nullptr, 0.f, nullptr, nullptr,
        [&](int r, int c, const auto& v) {
          if (r < nrows && c < ncols)
            __builtin_nontemporal_store(pack4<Out::F32>(v),
                                        reinterpret_cast<u32x4_t*>(base_out + (r * p.N + c) * 4));
        });
    return;
  }
  // split group: this slice's partial tile (dense BM x BN) into its slot
  constexpr int64_t kTileElems = static_cast<int64_t>(TS::BM) * TS::BN;
  float* part0 = p.partials + (uni(s_slot[g]) * per_group + lt) * kTileElems;
  const int64_t slice_stride = per_group * kTileElems;
  char* mine = reinterpret_cast<char*>(part0 + s * slice_stride);
  epilogue_quads<Elem::BF16, TS, Out::F32>(acc, row0, p.M - 1, col0, p.N, nullptr, 0.f, nullptr,
                                           nullptr, [&](int r, int c, const auto& v) {
                                             *reinterpret_cast<u32x4_t*>(mine + (r * TS::BN + c) * 4) =
                                                 pack4<Out::F32>(v);
                                           });
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  uint32_t* ctr = p.counters + static_cast<int64_t>(g) * per_group + lt;
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const uint32_t prev = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev + 1 == static_cast<uint32_t>(nslices);
  }
  __syncthreads();
  if (!s_last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  // 16 runs of 4 columns per thread at a time, the loads of one slice's 16
  // issued together: a store shares the wait counter with the loads after it,
  // so one run at a time made every load wait for the previous run's store
  // (about 40 us per launch on the MoE workload's fc2 weight gradient)
  constexpr int U = 16;
  for (int i0 = threadIdx.x; i0 < TS::BM * TS::BN / 4; i0 += TS::NT * U) {
    float4 sum[U];
#pragma unroll
    for (int u = 0; u < U; ++u) sum[u] = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int64_t j = 0; j < nslices; ++j) {
      float4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = i0 + u * TS::NT;
        const int r = i / (TS::BN / 4), c = (i - r * (TS::BN / 4)) * 4;
        v[u] = *reinterpret_cast<const float4*>(part0 + j * slice_stride + r * TS::BN + c);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        sum[u].x += v[u].x;
        sum[u].y += v[u].y;
        sum[u].z += v[u].z;
        sum[u].w += v[u].w;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * TS::NT;
      const int r = i / (TS::BN / 4), c = (i - r * (TS::BN / 4)) * 4;
      if (r < nrows && c < ncols)
        *reinterpret_cast<float4*>(dst + (row0 + r) * p.N + col0 + c) = sum[u];
    }
  }
  if (threadIdx.x == 0) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace mc2

using namespace mc2;

// ---------------------------------------------------------------- grouped entry points

namespace mc2 {

using TileG = TileW;

template <int MODE, bool BT>
static int run_grouped(const GroupedArgs& a, int64_t max_tiles, hipStream_t stream) {
  const int64_t grid64 = max_tiles < num_cus() ? max_tiles : num_cus();
  const int grid = static_cast<int>(grid64 > 0 ? grid64 : 1);
  if (a.K % 64 == 0) {
    hipLaunchKernelGGL((grouped_gemm_kernel<TileG, MODE, BT, false>), dim3(grid), dim3(TileG::NT), 0,
                       stream, a);
    return hipGetLastError() == hipSuccess ? MC2_OK : MC2_ERR_HIP;
  }
  hipLaunchKernelGGL((grouped_gemm_kernel<TileG, MODE, BT, true>), dim3(grid), dim3(TileG::NT), 0, stream,
                     a);
  return hipGetLastError() == hipSuccess ? MC2_OK : MC2_ERR_HIP;
}

static int check_ep(int world_size_src, int ep_rank, int num_experts, int local_experts) {
  if (world_size_src != 1) return MC2_ERR_UNSUPPORTED;
  if (num_experts < 1 || local_experts < 1 || local_experts > kMaxLocalExperts) return MC2_ERR_SHAPE;
  if (num_experts % local_experts) return MC2_ERR_SHAPE;
  if (ep_rank < 0 || ep_rank >= num_experts / local_experts) return MC2_ERR_SHAPE;
  return MC2_OK;
}

}  // namespace mc2

extern "C" int mc2_gmm_dispatch(const void* send_buf, int64_t send_rows, const int32_t* send_counts,
                                const int32_t* recv_counts, int world_size_src, int ep_rank,
                                int num_experts, int local_experts, const void* w1, int64_t H,
                                int64_t I2, int act, void* h_out, int64_t h_rows,
                                int32_t* dev_err, hipStream_t stream) {
  if (!send_buf || !send_counts || !recv_counts || !w1 || !h_out) return MC2_ERR_NULL;
  int st = check_ep(world_size_src, ep_rank, num_experts, local_experts);
  if (st) return st;
  if (H < 1 || I2 < 16 || send_rows < 0 || h_rows < 0) return MC2_ERR_SHAPE;
  if (act != MC2_ACT_NONE && act != MC2_ACT_SWIGLU) return MC2_ERR_SHAPE;
  if (H % 8 || I2 % 16) return MC2_ERR_ALIGN;
  if (!aligned16(send_buf) || !aligned16(w1) || !aligned16(h_out)) return MC2_ERR_ALIGN;
  if (!offsets_fit(H * 2, I2 * 2)) return MC2_ERR_UNSUPPORTED;
  const bool glu = act == MC2_ACT_SWIGLU;
  GroupedArgs a{};
  a.A = static_cast<const char*>(send_buf);
  a.lda = H * 2;
  a.B = static_cast<const char*>(w1);
  a.ldb = I2 * 2;
  a.b_group = H * I2 * 2;
  a.out = static_cast<char*>(h_out);
  a.n_b = I2;
  a.n_out = glu ? I2 / 2 : I2;
  a.inter = I2 / 2;
  a.ldo = a.n_out * 2;
  a.K = H;
  a.send_counts = send_counts;
  a.recv_counts = recv_counts;
  a.ep_rank = ep_rank;
  a.num_experts = num_experts;
  a.local_experts = local_experts;
  a.combine = 0;
  a.a_cap = send_rows;
  a.o_cap = h_rows;
  a.dev_err = dev_err;
  a.ktiles = static_cast<int>((H + 63) / 64);
  const int outc = glu ? TileG::BN / 2 : TileG::BN;
  const int64_t rows = send_rows < h_rows ? send_rows : h_rows;
  const int64_t max_tiles = (rows / TileG::BM + local_experts) * ((a.n_out + outc - 1) / outc);
  return glu ? run_grouped<kSwiglu, false>(a, max_tiles, stream)
             : run_grouped<kLinear, false>(a, max_tiles, stream);
}

extern "C" int mc2_gmm_combine(const void* h, int64_t h_rows, const int32_t* recv_counts,
                               const int32_t* send_counts, int world_size_src, int ep_rank,
                               int num_experts, int local_experts, const void* w2, int64_t I,
                               int64_t H, void* combine_buf, int64_t combine_rows,
                               int32_t* dev_err, hipStream_t stream) {
  if (!h || !send_counts || !recv_counts || !w2 || !combine_buf) return MC2_ERR_NULL;
  int st = check_ep(world_size_src, ep_rank, num_experts, local_experts);
  if (st) return st;
  if (I < 1 || H < 8 || h_rows < 0 || combine_rows < 0) return MC2_ERR_SHAPE;
  if (I % 8 || H % 8) return MC2_ERR_ALIGN;
  if (!aligned16(h) || !aligned16(w2) || !aligned16(combine_buf)) return MC2_ERR_ALIGN;
  if (!offsets_fit(I * 2, H * 2)) return MC2_ERR_UNSUPPORTED;
  GroupedArgs a{};
  a.A = static_cast<const char*>(h);
  a.lda = I * 2;
  a.B = static_cast<const char*>(w2);
  a.ldb = H * 2;
  a.b_group = I * H * 2;
  a.out = static_cast<char*>(combine_buf);
  a.n_b = H;
  a.n_out = H;
  a.inter = 0;
  a.ldo = H * 2;
  a.K = I;
  a.send_counts = send_counts;
  a.recv_counts = recv_counts;
  a.ep_rank = ep_rank;
  a.num_experts = num_experts;
  a.local_experts = local_experts;
  a.combine = 1;
  a.a_cap = h_rows;
  a.o_cap = combine_rows;
  a.dev_err = dev_err;
  a.ktiles = static_cast<int>((I + 63) / 64);
  const int64_t rows = h_rows < combine_rows ? h_rows : combine_rows;
  const int64_t max_tiles =
      (rows / TileG::BM + local_experts) * ((H + TileG::BN - 1) / TileG::BN);
  return run_grouped<kLinear, false>(a, max_tiles, stream);
}

// ---------------------------------------------------------------- EP backward

namespace mc2 {

// Workspace of a weight gradient dW = P^T Q over `rows` rows of P, dW (E_l,
// M, N): the tile counters, then the partial-tile slots of split groups. A
// split group of c > L rows has ceil(c / L) < 2c / L slices, so 2 * rows / L
// slots always suffice.
struct WgradLayout {
  int64_t tiles_m, tiles_n, max_slots;
  size_t off_ctr, off_part, total;
};

static WgradLayout wgrad_layout(int64_t rows, int local_experts, int64_t M, int64_t N) {
  WgradLayout w{};
  w.tiles_m = (M + TileL::BM - 1) / TileL::BM;
  w.tiles_n = (N + TileL::BN - 1) / TileL::BN;
  w.max_slots = 2 * rows / kSliceRows;
  const size_t per_group = static_cast<size_t>(w.tiles_m * w.tiles_n);
  w.off_ctr = 0;
  w.off_part = (per_group * local_experts * 4 + 255) & ~size_t{255};
  w.total = w.off_part + static_cast<size_t>(w.max_slots) * per_group * TileL::BM * TileL::BN * 4;
  return w;
}

// The tile counters of the weight gradient, for the input-gradient launch
// before it to clear.
static void clear_counters(GroupedArgs& a, void* workspace, int64_t rows, int local_experts,
                           int64_t M, int64_t N) {
  const WgradLayout L = wgrad_layout(rows, local_experts, M, N);
  a.zero = reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + L.off_ctr);
  a.n_zero = L.tiles_m * L.tiles_n * local_experts;
}

static int run_wgrad(const char* P, int64_t ldp, int p_at_send, int64_t p_cap, const char* Q,
                     int64_t ldq, int q_at_send, int64_t q_cap, int64_t M, int64_t N,
                     const int32_t* send_counts, const int32_t* recv_counts, int ep_rank,
                     int local_experts, float* dw, void* workspace, int32_t* dev_err,
                     hipStream_t stream) {
  const WgradLayout L = wgrad_layout(p_cap, local_experts, M, N);
  char* ws = static_cast<char*>(workspace);
  const int64_t per_group = L.tiles_m * L.tiles_n;
  WgradArgs w{};
  w.P = P;
  w.ldp = ldp;
  w.p_at_send = p_at_send;
  w.p_cap = p_cap;
  w.Q = Q;
  w.ldq = ldq;
  w.at_send = q_at_send;
  w.q_cap = q_cap;
  w.out = dw;
  w.M = M;
  w.N = N;
  w.tiles_m = static_cast<int>(L.tiles_m);
  w.tiles_n = static_cast<int>(L.tiles_n);
  // q tiles of each slice per XCD; the block shape with the fewest A and B
  // slabs (bm + bn) among those that cut the tile grid into 8 blocks
  w.q = static_cast<int>((per_group + 7) / 8);
  w.cus = static_cast<int>(num_cus());
  for (int a = 1; a <= w.q; ++a) {
    const int b = w.q / a;
    if (a * b != w.q || L.tiles_m % a || L.tiles_n % b || (L.tiles_m / a) * (L.tiles_n / b) != 8)
      continue;
    if (!w.bm || a + b < w.bm + w.bn) w.bm = a, w.bn = b;
  }
  w.counters = reinterpret_cast<uint32_t*>(ws + L.off_ctr);
  w.partials = reinterpret_cast<float*>(ws + L.off_part);
  w.max_slots = L.max_slots;
  w.send_counts = send_counts;
  w.recv_counts = recv_counts;
  w.ep_rank = ep_rank;
  w.local_experts = local_experts;
  w.dev_err = dev_err;
  // at most rows / L + E_l slices in all, q units of each per XCD
  // (L >= kSliceRows, so these bound the slices of any slice length)
  const int64_t units = (p_cap / kSliceRows + local_experts) * 8 * w.q;
  if (units > 0x3fffffff) return MC2_ERR_SHAPE;
  hipLaunchKernelGGL((wgrad_kernel<TileW, true>), dim3(static_cast<unsigned>(units)),
                     dim3(TileW::NT), 0, stream, w);
  return hipGetLastError() == hipSuccess ? MC2_OK : MC2_ERR_HIP;
}

}  // namespace mc2

extern "C" size_t mc2_gmm_backward_workspace_size(int64_t rows, int local_experts, int64_t M,
                                                  int64_t N) {
  if (rows < 0 || M < 1 || N < 1 || local_experts < 1 || local_experts > kMaxLocalExperts) return 0;
  return wgrad_layout(rows, local_experts, M, N).total;
}

extern "C" int mc2_gmm_combine_backward(const void* dy_buf, int64_t dy_rows,
                                        const int32_t* recv_counts, const int32_t* send_counts,
                                        int world_size_src, int ep_rank, int num_experts,
                                        int local_experts, const void* w2, int64_t I, int64_t H,
                                        const void* h, int64_t h_rows, const void* g_saved, int act,
                                        void* dgrad_out, float* dw2_out, void* workspace,
                                        size_t ws_bytes, int32_t* dev_err, hipStream_t stream) {
  if (!dy_buf || !send_counts || !recv_counts || !w2 || !h || !dgrad_out || !dw2_out)
    return MC2_ERR_NULL;
  int st = check_ep(world_size_src, ep_rank, num_experts, local_experts);
  if (st) return st;
  if (I < 8 || H < 8 || dy_rows < 0 || h_rows < 0) return MC2_ERR_SHAPE;
  if (act != MC2_ACT_NONE && act != MC2_ACT_SWIGLU) return MC2_ERR_SHAPE;
  const bool glu = act == MC2_ACT_SWIGLU;
  if (glu && !g_saved) return MC2_ERR_NULL;
  if (I % 8 || H % 8) return MC2_ERR_ALIGN;
  if (!aligned16(dy_buf) || !aligned16(w2) || !aligned16(h) || !aligned16(dgrad_out) ||
      !aligned16(dw2_out) || (glu && !aligned16(g_saved)))
    return MC2_ERR_ALIGN;
  if (!workspace) return MC2_ERR_NULL;
  if (!aligned16(workspace)) return MC2_ERR_ALIGN;
  if (ws_bytes < mc2_gmm_backward_workspace_size(h_rows, local_experts, I, H)) return MC2_ERR_WORKSPACE;
  if (!offsets_fit(H * 2, H * 2) || !offsets_fit(I * 2, H * 2)) return MC2_ERR_UNSUPPORTED;
  // dgrad: dA = dY_g @ w2[g]^T, the weight read as (I, H) rows; SwiGLU backward fused
  GroupedArgs a{};
  a.A = static_cast<const char*>(dy_buf);
  a.lda = H * 2;
  a.B = static_cast<const char*>(w2);
  a.ldb = H * 2;
  a.b_group = I * H * 2;
  a.out = static_cast<char*>(dgrad_out);
  a.n_b = I;
  a.n_out = I;
  a.inter = I;
  a.ldo = (glu ? 2 * I : I) * 2;
  a.K = H;
  a.send_counts = send_counts;
  a.recv_counts = recv_counts;
  a.ep_rank = ep_rank;
  a.num_experts = num_experts;
  a.local_experts = local_experts;
  a.combine = 0;
  a.a_cap = dy_rows;
  a.o_cap = h_rows;
  a.dev_err = dev_err;
  a.ktiles = static_cast<int>((H + 63) / 64);
  a.gsave = static_cast<const char*>(g_saved);
  a.ldg = 2 * I * 2;
  const int64_t rows = dy_rows < h_rows ? dy_rows : h_rows;
  const int64_t max_tiles = (rows / TileG::BM + local_experts) * ((I + TileG::BN - 1) / TileG::BN);
  clear_counters(a, workspace, h_rows, local_experts, I, H);
  st = glu ? run_grouped<kSwigluBwd, true>(a, max_tiles, stream)
           : run_grouped<kLinear, true>(a, max_tiles, stream);
  if (st) return st;
  // wgrad: dW2[g] = h_g^T @ dY_g
  return run_wgrad(static_cast<const char*>(h), I * 2, 0, h_rows, static_cast<const char*>(dy_buf),
                   H * 2, 1, dy_rows, I, H, send_counts, recv_counts, ep_rank, local_experts,
                   dw2_out, workspace, dev_err, stream);
}

extern "C" int mc2_gmm_dispatch_backward(const void* dg, int64_t dg_rows, const int32_t* recv_counts,
                                         const int32_t* send_counts, int world_size_src,
                                         int ep_rank, int num_experts, int local_experts,
                                         const void* w1, int64_t H, int64_t I2,
                                         const void* send_buf, int64_t send_rows, void* dx_buf,
                                         int64_t dx_rows, float* dw1_out, void* workspace,
                                         size_t ws_bytes, int32_t* dev_err, hipStream_t stream) {
  if (!dg || !send_counts || !recv_counts || !w1 || !send_buf || !dx_buf || !dw1_out)
    return MC2_ERR_NULL;
  int st = check_ep(world_size_src, ep_rank, num_experts, local_experts);
  if (st) return st;
  if (H < 8 || I2 < 8 || dg_rows < 0 || send_rows < 0 || dx_rows < 0) return MC2_ERR_SHAPE;
  if (H % 8 || I2 % 8) return MC2_ERR_ALIGN;
  if (!aligned16(dg) || !aligned16(w1) || !aligned16(send_buf) || !aligned16(dx_buf) ||
      !aligned16(dw1_out))
    return MC2_ERR_ALIGN;
  if (!workspace) return MC2_ERR_NULL;
  if (!aligned16(workspace)) return MC2_ERR_ALIGN;
  if (ws_bytes < mc2_gmm_backward_workspace_size(send_rows, local_experts, H, I2))
    return MC2_ERR_WORKSPACE;
  if (!offsets_fit(I2 * 2, I2 * 2) || !offsets_fit(H * 2, I2 * 2)) return MC2_ERR_UNSUPPORTED;
  // dgrad: dX_g = dG_g @ w1[g]^T, the weight read as (H, I2) rows, written at the send rows
  GroupedArgs a{};
  a.A = static_cast<const char*>(dg);
  a.lda = I2 * 2;
  a.B = static_cast<const char*>(w1);
  a.ldb = I2 * 2;
  a.b_group = H * I2 * 2;
  a.out = static_cast<char*>(dx_buf);
  a.n_b = H;
  a.n_out = H;
  a.inter = 0;
  a.ldo = H * 2;
  a.K = I2;
  a.send_counts = send_counts;
  a.recv_counts = recv_counts;
  a.ep_rank = ep_rank;
  a.num_experts = num_experts;
  a.local_experts = local_experts;
  a.combine = 1;
  a.a_cap = dg_rows;
  a.o_cap = dx_rows;
  a.dev_err = dev_err;
  a.ktiles = static_cast<int>((I2 + 63) / 64);
  const int64_t rows = dg_rows < dx_rows ? dg_rows : dx_rows;
  const int64_t max_tiles = (rows / TileG::BM + local_experts) * ((H + TileG::BN - 1) / TileG::BN);
  clear_counters(a, workspace, send_rows, local_experts, H, I2);
  st = run_grouped<kLinear, true>(a, max_tiles, stream);
  if (st) return st;
  // wgrad: dW1[g] = R_g^T @ dG_g over this rank's send rows R
  return run_wgrad(static_cast<const char*>(send_buf), H * 2, 1, send_rows,
                   static_cast<const char*>(dg), I2 * 2, 0, dg_rows, H, I2, send_counts,
                   recv_counts, ep_rank, local_experts, dw1_out, workspace, dev_err, stream);
}
