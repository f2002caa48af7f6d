// The chunked GEMM's host entry, shared by the entry points built on it.
#pragma once

#include "mc2_tiles.hpp"

namespace mc2 {

// Waiting for input chunks (AllGatherMatmul consumer side); none by default.
struct InputWait {
  const uint32_t* flags = nullptr;
  uint32_t epoch = 0;
  uint32_t spin_limit = 0;
  int32_t* dev_err = nullptr;
};

// Launches the rank-chunked GEMM: W chunks of m / W rows (each cut into `sub`
// pieces), computed from chunk first_chunk on, over nsim stacked k-shards,
// with optional ready flags and input waits. split_ws (NULL: none) is the
// K-split workspace (zeroed control words, then the partial slots).
// Arguments are checked by the caller. Returns an mc2_status.
int run_chunked(const void* x1, const void* x2, int64_t m, int64_t k, int64_t n, int W,
                int first_chunk, int nsim, int x2_trans, int in_dtype, const void* bias,
                const float* s1, const float* s2, int out_dtype, void* out, uint32_t* flags,
                uint32_t* counters, uint32_t epoch, int sub, hipStream_t stream,
                const InputWait& inw = InputWait{}, void* split_ws = nullptr,
                size_t split_ws_bytes = 0);

}  // namespace mc2
