// Token counting, stable permute and weighted unpermute of the MoE
// expert-parallel local path ("NPU Training Operators - MC2", "执行路径":
// histc, permute(hidden_states, selected_experts), unpermute(h,
// unpermute_indices, probs=routing_weights)), for gfx950.
//
// These kernels move bytes, not FLOPs: they are written for coalesced 16-byte
// accesses and for reading each token row once.
#include <mutex>

#include "../../include/mc2.h"
#include "mc2_common.hpp"
#include "mc2_host.hpp"

namespace mc2 {

constexpr int kMoeThreads = 256;
constexpr int kMaxExperts = 1024;

__global__ __launch_bounds__(kMoeThreads) void fill_i32_kernel(int32_t* p, int64_t n, int32_t v) {
  for (int64_t i = blockIdx.x * (int64_t)kMoeThreads + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * kMoeThreads)
    p[i] = v;
}

// ---------------------------------------------------------------- histc
//
// A block counts chunks of kHistcChunk ids: every thread issues its four
// 16-byte loads (16 ids) before it counts any, so a chunk costs one memory
// latency, and adds them to the block's LDS histogram. The block then adds its
// non-zero counters to `counts` (cleared by the fill kernel launched before).
// The global atomics, E per block on the same E words, are what costs: the
// large chunk keeps the block count, and with it their number, low.

constexpr int kHistcLoads = 4;                              // 16-byte loads per thread
constexpr int kHistcChunk = kMoeThreads * kHistcLoads * 4;  // 4096 ids per chunk

__global__ __launch_bounds__(kMoeThreads) void histc_kernel(const int32_t* __restrict__ sel,
                                                            int64_t n, int E, int vec_ok,
                                                            int32_t* counts, int32_t* dev_err) {
  __shared__ int h[kMaxExperts];
  for (int e = threadIdx.x; e < E; e += kMoeThreads) h[e] = 0;
  __syncthreads();
  bool bad = false;
  for (int64_t c0 = (int64_t)blockIdx.x * kHistcChunk; c0 < n;
       c0 += (int64_t)gridDim.x * kHistcChunk) {
    int v[kHistcLoads * 4];
    const bool full = vec_ok && c0 + kHistcChunk <= n;
    if (full) {
      // load j of the block covers 1024 consecutive ids; lane order within a
      // wave is contiguous, so each wave load reads 1 KiB in one sweep
      const i32x4_t* p = reinterpret_cast<const i32x4_t*>(sel + c0);
#pragma unroll
      for (int j = 0; j < kHistcLoads; ++j) {
        const i32x4_t q = p[j * kMoeThreads + threadIdx.x];
#pragma unroll
        for (int c = 0; c < 4; ++c) v[j * 4 + c] = q[c];
      }
    } else {
#pragma unroll
      for (int j = 0; j < kHistcLoads * 4; ++j) {
        const int64_t i = c0 + (int64_t)j * kMoeThreads + threadIdx.x;
        v[j] = i < n ? sel[i] : 0;
      }
    }
#pragma unroll
    for (int j = 0; j < kHistcLoads * 4; ++j) {
      // ids outside [0, E) are reported and not counted; a lane past the end
      // has nothing to count
      const bool in = full || (int64_t)j * kMoeThreads + threadIdx.x < n - c0;
      const int id = v[j];
      if (in && id >= 0 && id < E) atomicAdd(&h[id], 1);
      else if (in) bad = true;
    }
  }
  if (bad) atomic_or_err(dev_err, MC2_DEVERR_EXPERT_ID);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kMoeThreads)
    if (h[e]) atomicAdd(&counts[e], h[e]);
}

// ---------------------------------------------------------------- permute
//
// Block b owns tokens [b*TB, (b+1)*TB) and so slots [b*TB*K, ...), at most 256
// slots, split into groups of 64 consecutive slots (one per wave).
//   1. count:   per-block expert histogram -> ws_hist[e*nblk + b]
//   2. scan:    per expert, exclusive prefix over blocks (in place) and the
//               expert total
//   3. scatter: position of every slot = expert offset + block offset +
//               earlier groups of the block + rank inside its 64-slot group
//               (wave ballots over the id bits give the lanes holding the
//               same id); write the indices and copy each token row once
//               from x to its K destinations.

static inline int tokens_per_block(int K) { return K >= kMoeThreads ? 1 : kMoeThreads / K; }

__global__ __launch_bounds__(kMoeThreads) void permute_count_kernel(
    const int32_t* __restrict__ sel, int64_t T, int K, int E, int TB, int nblk,
    int32_t* __restrict__ ws_hist, int32_t* dev_err) {
  __shared__ int h[kMaxExperts];
  const int b = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += kMoeThreads) h[e] = 0;
  __syncthreads();
  const int64_t s0 = (int64_t)b * TB * K;
  int64_t s1 = s0 + (int64_t)TB * K;
  const int64_t send = T * K;
  s1 = s1 < send ? s1 : send;
  bool bad = false;
  for (int64_t s = s0 + threadIdx.x; s < s1; s += kMoeThreads) {
    const int32_t v = sel[s];
    if (v >= 0 && v < E) atomicAdd(&h[v], 1);
    else bad = true;
  }
  if (bad) atomic_or_err(dev_err, MC2_DEVERR_EXPERT_ID);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kMoeThreads) ws_hist[(int64_t)e * nblk + b] = h[e];
}

// One workgroup per expert: exclusive scan of its nblk block counts.
__global__ __launch_bounds__(kMoeThreads) void permute_scan_kernel(int32_t* __restrict__ ws_hist,
                                                                   int nblk,
                                                                   int32_t* __restrict__ ws_total) {
  __shared__ int part[kMoeThreads];
  const int e = blockIdx.x;
  int32_t* col = ws_hist + (int64_t)e * nblk;
  const int per = (nblk + kMoeThreads - 1) / kMoeThreads;
  const int lo = threadIdx.x * per;
  const int hi = lo + per < nblk ? lo + per : nblk;
  int s = 0;
  for (int i = lo; i < hi; ++i) s += col[i];
  part[threadIdx.x] = s;
  __syncthreads();
  // Hillis-Steele inclusive scan over the 256 partial sums.
  for (int off = 1; off < kMoeThreads; off <<= 1) {
    const int v = threadIdx.x >= off ? part[threadIdx.x - off] : 0;
    __syncthreads();
    part[threadIdx.x] += v;
    __syncthreads();
  }
  int run = threadIdx.x ? part[threadIdx.x - 1] : 0;
  for (int i = lo; i < hi; ++i) {
    const int v = col[i];
    col[i] = run;
    run += v;
  }
  if (threadIdx.x == kMoeThreads - 1) ws_total[e] = part[kMoeThreads - 1];
}

__global__ __launch_bounds__(kMoeThreads) void permute_scatter_kernel(
    const uint16_t* __restrict__ x, int64_t T, int64_t H, const int32_t* __restrict__ sel, int K,
    int E, int TB, int nblk, const int32_t* __restrict__ ws_hist,
    const int32_t* __restrict__ ws_total, uint16_t* __restrict__ permuted,
    int32_t* __restrict__ sorted_idx, int32_t* __restrict__ unpermute_idx,
    int32_t* __restrict__ expert_offsets) {
  __shared__ int s_off[kMaxExperts + 1];
  __shared__ int s_gcnt[4][kMaxExperts + 1];
  __shared__ int s_pos[kMoeThreads];
  __shared__ int s_part[kMoeThreads];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.x;

  // Expert offsets: exclusive scan of the totals (E <= 1024, 4 per thread).
  {
    int v[4];
    int s = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid * 4 + i;
      v[i] = e < E ? ws_total[e] : 0;
      s += v[i];
    }
    s_part[tid] = s;
    __syncthreads();
    for (int off = 1; off < kMoeThreads; off <<= 1) {
      const int t = tid >= off ? s_part[tid - off] : 0;
      __syncthreads();
      s_part[tid] += t;
      __syncthreads();
    }
    int run = tid ? s_part[tid - 1] : 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid * 4 + i;
      if (e < E) s_off[e] = run;
      run += v[i];
    }
    if (tid == kMoeThreads - 1) s_off[E] = s_part[kMoeThreads - 1];
  }
  for (int i = tid; i < 4 * (kMaxExperts + 1); i += kMoeThreads) (&s_gcnt[0][0])[i] = 0;
  __syncthreads();
  const int n_valid = s_off[E];
  if (b == 0)
    for (int e = tid; e <= E; e += kMoeThreads) expert_offsets[e] = s_off[e];

  const int64_t total_slots = T * K;
  const int64_t s0 = (int64_t)b * TB * K;
  int nslots = TB * K;
  if (s0 + nslots > total_slots) nslots = (int)(total_slots - s0);

  // Tail of sorted_idx: positions n_valid .. T*K-1 hold no slot.
  {
    const int64_t p = (int64_t)n_valid + (int64_t)b * TB * K + tid;
    if (tid < TB * K && p < total_slots) sorted_idx[p] = -1;
  }

  // Rank of each slot among the same-expert slots of its 64-slot group.
  const int sl = wave * 64 + lane;  // slot index inside the block
  const bool active = sl < nslots;
  int id = E;  // E marks an invalid id (or an inactive lane)
  if (active) {
    const int32_t v = sel[s0 + sl];
    if (v >= 0 && v < E) id = v;
  }
  const int nbits = 32 - __clz(E);  // bits needed for 0..E
  uint64_t match = __ballot(active);
  for (int bit = 0; bit < nbits; ++bit) {
    const bool on = (id >> bit) & 1;
    const uint64_t bb = __ballot(on);
    match &= on ? bb : ~bb;
  }
  const int rank = __popcll(match & ((1ull << lane) - 1ull));
  if (active && id < E && rank == 0) s_gcnt[wave][id] = __popcll(match);
  __syncthreads();

  int pos = -1;
  if (active && id < E) {
    int before = 0;
    for (int g = 0; g < wave; ++g) before += s_gcnt[g][id];
    pos = s_off[id] + ws_hist[(int64_t)id * nblk + b] + before + rank;
    sorted_idx[pos] = (int32_t)(s0 + sl);
  }
  if (active) unpermute_idx[s0 + sl] = pos;
  s_pos[sl] = pos;
  __syncthreads();

  // Row copy: wave w takes tokens w, w+4, ... of the block; each token row is
  // read once (16-byte chunks, 4 per lane per pass) and stored to its K
  // destination rows. The permuted buffer is written once and not read here:
  // non-temporal stores keep it from displacing the rows still to be read.
  const int64_t t0 = (int64_t)b * TB;
  int ntok = TB;
  if (t0 + ntok > T) ntok = (int)(T - t0);
  const int64_t CR = H / 8;
  for (int tl = wave; tl < ntok; tl += 4) {
    const uint4* src = reinterpret_cast<const uint4*>(x + (t0 + tl) * H);
    for (int64_t base = 0; base < CR; base += 256) {
      uint4 v[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int64_t j = base + c * 64 + lane;
        v[c] = j < CR ? src[j] : zero4();
      }
      for (int k = 0; k < K; ++k) {
        const int p = s_pos[tl * K + k];
        if (p < 0) continue;
        uint4* dst = reinterpret_cast<uint4*>(permuted + (int64_t)p * H);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int64_t j = base + c * 64 + lane;
          if (j < CR)
            __builtin_nontemporal_store(bit_cast<u32x4_t>(v[c]), reinterpret_cast<u32x4_t*>(dst) + j);
        }
      }
    }
  }
}

// ---------------------------------------------------------------- unpermute

// One wave per token; lanes own 16-byte column chunks (8 bf16), four per lane
// in a pass of 256 chunks (the whole row for H <= 2048). The slot indices and
// weights of a group of 8 slots are loaded once per pass by lanes 0-7 and
// broadcast, so the row addresses are wave-uniform; the 8 rows' loads of a
// pass are all issued before any is accumulated. Every y row is read once and
// every output row written once: both go non-temporal. Sums run in fp32 with k
// ascending, one fma per slot (an invalid slot adds 0 * 0).
__global__ __launch_bounds__(kMoeThreads) void unpermute_kernel(
    const uint16_t* __restrict__ y, int64_t y_rows, const int32_t* __restrict__ idx,
    const float* __restrict__ probs, int64_t T, int K, int64_t H, uint16_t* __restrict__ out,
    int32_t* dev_err) {
  constexpr int kC = 4;  // 16-byte chunks per lane per pass
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int64_t CR = H / 8;
  bool bad = false;
  for (int64_t base = 0; base < CR; base += 64 * kC) {
    float acc[kC][8];
#pragma unroll
    for (int c = 0; c < kC; ++c)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[c][i] = 0.f;
    for (int k0 = 0; k0 < K; k0 += 8) {
      int p_l = -1;
      float w_l = 0.f;
      if (lane < 8 && k0 + lane < K) {
        p_l = idx[t * K + k0 + lane];
        w_l = probs[t * K + k0 + lane];
        if (p_l >= y_rows) { bad = true; p_l = -1; }
        if (p_l < 0) w_l = 0.f;
      }
      uint4 v[8][kC];
      float w[8];
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const int p = __builtin_amdgcn_readlane(p_l, kk);
        w[kk] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w_l), kk));
        const u32x4_t* row = reinterpret_cast<const u32x4_t*>(y + (int64_t)(p < 0 ? 0 : p) * H);
#pragma unroll
        for (int c = 0; c < kC; ++c) {
          const int64_t j = base + c * 64 + lane;
          v[kk][c] = (p >= 0 && j < CR) ? bit_cast<uint4>(__builtin_nontemporal_load(row + j))
                                        : zero4();
        }
      }
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
#pragma unroll
        for (int c = 0; c < kC; ++c) {
          const uint32_t d[4] = {v[kk][c].x, v[kk][c].y, v[kk][c].z, v[kk][c].w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            acc[c][2 * q] = __builtin_fmaf(w[kk], bf16_bits_to_f32(d[q] & 0xFFFFu), acc[c][2 * q]);
            acc[c][2 * q + 1] = __builtin_fmaf(w[kk], bf16_bits_to_f32(d[q] >> 16), acc[c][2 * q + 1]);
          }
        }
      }
    }
#pragma unroll
    for (int c = 0; c < kC; ++c) {
      const int64_t j = base + c * 64 + lane;
      if (j < CR) {
        uint4 o;
        o.x = f32_to_bf16_bits(acc[c][0]) | ((uint32_t)f32_to_bf16_bits(acc[c][1]) << 16);
        o.y = f32_to_bf16_bits(acc[c][2]) | ((uint32_t)f32_to_bf16_bits(acc[c][3]) << 16);
        o.z = f32_to_bf16_bits(acc[c][4]) | ((uint32_t)f32_to_bf16_bits(acc[c][5]) << 16);
        o.w = f32_to_bf16_bits(acc[c][6]) | ((uint32_t)f32_to_bf16_bits(acc[c][7]) << 16);
        __builtin_nontemporal_store(bit_cast<u32x4_t>(o), reinterpret_cast<u32x4_t*>(out + t * H) + j);
      }
    }
  }
  if (bad) atomic_or_err(dev_err, MC2_DEVERR_INDEX);
}

static inline int grid_for(int64_t n, int per_thread, int cap) {
  int64_t g = (n + (int64_t)kMoeThreads * per_thread - 1) / ((int64_t)kMoeThreads * per_thread);
  if (g < 1) g = 1;
  return (int)(g < cap ? g : cap);
}

}  // namespace mc2

using namespace mc2;

extern "C" int mc2_moe_histc(const int32_t* sel, int64_t n_ids, int num_experts, int32_t* counts,
                             int32_t* dev_err, hipStream_t stream) {
  if (!counts || (!sel && n_ids > 0)) return MC2_ERR_NULL;
  if (n_ids < 0 || num_experts < 1 || num_experts > kMaxExperts) return MC2_ERR_SHAPE;
  hipLaunchKernelGGL(fill_i32_kernel, dim3(grid_for(num_experts, 1, 64)), dim3(kMoeThreads), 0,
                     stream, counts, (int64_t)num_experts, 0);
  if (n_ids > 0) {
    const int vec_ok = (reinterpret_cast<uintptr_t>(sel) & 15) == 0;
    hipLaunchKernelGGL(histc_kernel, dim3(grid_for(n_ids, kHistcChunk / kMoeThreads, 1024)),
                       dim3(kMoeThreads), 0, stream, sel, n_ids, num_experts, vec_ok, counts,
                       dev_err);
  }
  return hipGetLastError() == hipSuccess ? MC2_OK : MC2_ERR_HIP;
}

static int64_t permute_blocks(int64_t T, int K) {
  const int TB = tokens_per_block(K);
  return (T + TB - 1) / TB;
}

extern "C" size_t mc2_moe_permute_workspace_size(int64_t T, int K, int num_experts) {
  if (T < 1 || K < 1 || num_experts < 1) return 0;
  const int64_t nblk = permute_blocks(T, K);
  return (size_t)(((int64_t)num_experts * nblk + num_experts + 3) / 4 * 4) * sizeof(int32_t);
}

extern "C" int mc2_moe_permute(const void* x, int64_t T, int64_t H, const int32_t* sel, int K,
                               int num_experts, void* permuted, int32_t* sorted_idx,
                               int32_t* unpermute_idx, int32_t* expert_offsets, void* workspace,
                               size_t ws_bytes, int32_t* dev_err, hipStream_t stream) {
  if (!x || !sel || !permuted || !sorted_idx || !unpermute_idx || !expert_offsets || !workspace)
    return MC2_ERR_NULL;
  if (T < 1 || K < 1 || K > 64 || num_experts < 1 || num_experts > kMaxExperts || H < 8)
    return MC2_ERR_SHAPE;
  if (T * K >= (int64_t)0x7fffffff) return MC2_ERR_SHAPE;
  if (H % 8) return MC2_ERR_ALIGN;
  if (!aligned16(x) || !aligned16(permuted) || !aligned16(workspace)) return MC2_ERR_ALIGN;
  if (ws_bytes < mc2_moe_permute_workspace_size(T, K, num_experts)) return MC2_ERR_WORKSPACE;
  const int TB = tokens_per_block(K);
  const int64_t nblk64 = permute_blocks(T, K);
  if (nblk64 > 0x7fffffff) return MC2_ERR_SHAPE;
  const int nblk = (int)nblk64;
  int32_t* ws_hist = static_cast<int32_t*>(workspace);
  int32_t* ws_total = ws_hist + (int64_t)num_experts * nblk;
  hipLaunchKernelGGL(permute_count_kernel, dim3(nblk), dim3(kMoeThreads), 0, stream, sel, T, K,
                     num_experts, TB, nblk, ws_hist, dev_err);
  hipLaunchKernelGGL(permute_scan_kernel, dim3(num_experts), dim3(kMoeThreads), 0, stream, ws_hist,
                     nblk, ws_total);
  hipLaunchKernelGGL(permute_scatter_kernel, dim3(nblk), dim3(kMoeThreads), 0, stream,
                     static_cast<const uint16_t*>(x), T, H, sel, K, num_experts, TB, nblk, ws_hist,
                     ws_total, static_cast<uint16_t*>(permuted), sorted_idx, unpermute_idx,
                     expert_offsets);
  return hipGetLastError() == hipSuccess ? MC2_OK : MC2_ERR_HIP;
}

// ------------------------------------------------- permute without allocation
//
// The counting workspace of the permute (per-block expert counts and expert
// totals) in a file-scope device array, for callers that cannot allocate.
// Each device holds its own copy; its address is looked up once per device
// with hipGetSymbolAddress (the array's name in host code is only a stand-in)
// and every launch gets that address. The count and scan kernels overwrite
// every entry the scatter reads, so nothing needs clearing between calls.

constexpr size_t kScratchBytes = MC2_PERMUTE_SCRATCH_BYTES;
static __device__ __align__(256) int32_t scratch[kScratchBytes / sizeof(int32_t)];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's scratch array, or NULL on a runtime error.
void* scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}
}  // namespace

extern "C" int mc2_moe_permute_noalloc(const void* x, int64_t T, int64_t H, const int32_t* sel,
                                       int K, int num_experts, void* permuted,
                                       int32_t* sorted_idx, int32_t* unpermute_idx,
                                       int32_t* expert_offsets, int32_t* dev_err,
                                       hipStream_t stream) {
  if (!x || !sel || !permuted || !sorted_idx || !unpermute_idx || !expert_offsets)
    return MC2_ERR_NULL;
  if (T < 1 || K < 1 || K > 64 || num_experts < 1 || num_experts > kMaxExperts) return MC2_ERR_SHAPE;
  const size_t need = mc2_moe_permute_workspace_size(T, K, num_experts);
  if (need == 0 || need > kScratchBytes) return MC2_ERR_WORKSPACE;
  void* ws = scratch_address();
  if (!ws) return MC2_ERR_HIP;
  return mc2_moe_permute(x, T, H, sel, K, num_experts, permuted, sorted_idx, unpermute_idx,
                         expert_offsets, ws, kScratchBytes, dev_err, stream);
}

extern "C" int mc2_moe_unpermute(const void* y_full, int64_t y_rows, const int32_t* unpermute_idx,
                                 const float* probs, int64_t T, int K, int64_t H, void* out,
                                 int32_t* dev_err, hipStream_t stream) {
  if (!y_full || !unpermute_idx || !probs || !out) return MC2_ERR_NULL;
  if (T < 1 || K < 1 || K > 64 || H < 8 || y_rows < 0) return MC2_ERR_SHAPE;
  if (H % 8) return MC2_ERR_ALIGN;
  if (!aligned16(y_full) || !aligned16(out)) return MC2_ERR_ALIGN;
  const int64_t blocks = (T + 3) / 4;
  if (blocks > 0x7fffffff) return MC2_ERR_SHAPE;
  hipLaunchKernelGGL(unpermute_kernel, dim3((int)blocks), dim3(kMoeThreads), 0, stream,
                     static_cast<const uint16_t*>(y_full), y_rows, unpermute_idx, probs, T, K, H,
                     static_cast<uint16_t*>(out), dev_err);
  return hipGetLastError() == hipSuccess ? MC2_OK : MC2_ERR_HIP;
}

extern "C" const char* mc2_status_string(int status) {
  switch (status) {
    case MC2_OK: return "MC2_OK";
    case MC2_ERR_NULL: return "MC2_ERR_NULL: a required pointer is NULL";
    case MC2_ERR_SHAPE: return "MC2_ERR_SHAPE: a size or shape constraint is violated";
    case MC2_ERR_DTYPE: return "MC2_ERR_DTYPE: dtype or dtype combination not allowed";
    case MC2_ERR_UNSUPPORTED: return "MC2_ERR_UNSUPPORTED: valid per the API but not built";
    case MC2_ERR_HIP: return "MC2_ERR_HIP: the HIP runtime reported a launch error";
    case MC2_ERR_WORKSPACE: return "MC2_ERR_WORKSPACE: workspace too small";
    case MC2_ERR_ALIGN: return "MC2_ERR_ALIGN: pointer or row pitch not 16-byte aligned";
    default: return "unknown mc2 status";
  }
}

extern "C" const char* mc2_version(void) { return "mc2-gfx950 0.1.0"; }
