// Verification inputs of drafted trees on gfx950: the flattened tree of each
// sequence as the target model checks it, with the ancestor-only mask of
// standard tree attention that DominoTree keeps for verification (DominoTree
// summary, gist.science Chinese page, "方法论 / 核心组件", verification).
//
// Entry 0 of a sequence is its anchor, entry k + 1 its node k.  Node k is in
// the tree when its token is >= 0 and its parent is the anchor (-1) or an
// earlier node that is in the tree; every other slot is padding.  A tree
// entry sees itself and its ancestors; a padding entry only itself.
// Position ids: start + depth (anchor depth 0); -1 for padding.
//
// One workgroup of 64 lanes per sequence (at most 65 entries): one lane
// settles membership and depth in node order, then each lane builds its
// rows' ancestor sets as bitmasks by following parent links, and the lanes
// write the mask rows out together, one byte each.
#include "device.h"
#include "internal.h"

namespace dh {

constexpr int kVerifyMaxNodes = 64;

__global__ __launch_bounds__(64) void tree_verify_inputs_k(const int32_t* __restrict__ parents,
                                                           const int32_t* __restrict__ tokens,
                                                           const int32_t* __restrict__ first_tokens,
                                                           const int32_t* __restrict__ start_positions, int N,
                                                           uint8_t* __restrict__ mask, int32_t* __restrict__ positions,
                                                           int32_t* __restrict__ out_tokens) {
  __shared__ int32_t par[kVerifyMaxNodes], tok[kVerifyMaxNodes];
  __shared__ int32_t in_tree[kVerifyMaxNodes + 1], depth[kVerifyMaxNodes + 1];
  __shared__ uint64_t bits_lo[kVerifyMaxNodes + 1];  // entries 0..63 of each row
  __shared__ uint32_t bit_hi[kVerifyMaxNodes + 1];   // entry 64
  const int b = blockIdx.x, t = threadIdx.x, E = N + 1;
  for (int k = t; k < N; k += blockDim.x) {
    par[k] = parents[(size_t)b * N + k];
    tok[k] = tokens[(size_t)b * N + k];
  }
  __syncthreads();
  if (t == 0) {
    in_tree[0] = 1;
    depth[0] = 0;
    for (int k = 0; k < N; ++k) {
      const int q = par[k];
      const int ok = tok[k] >= 0 && q >= -1 && q < k && in_tree[q + 1];
      in_tree[k + 1] = ok;
      depth[k + 1] = ok ? depth[q + 1] + 1 : 0;
    }
  }
  __syncthreads();
  const int32_t start = start_positions ? start_positions[b] : 0;
  for (int i = t; i < E; i += blockDim.x) {
    uint64_t lo = 0;
    uint32_t hi = 0;
    auto set = [&](int e) {
      if (e < 64)
        lo |= 1ull << e;
      else
        hi = 1u;
    };
    set(i);
    if (i > 0 && in_tree[i]) {
      // parents of tree nodes are earlier tree nodes, so the walk ends at the anchor within i steps
      for (int e = i, steps = 0; e != 0 && steps < E; ++steps) {
        e = par[e - 1] + 1;
        set(e);
      }
    }
    bits_lo[i] = lo;
    bit_hi[i] = hi;
    positions[(size_t)b * E + i] = in_tree[i] ? start + depth[i] : -1;
    out_tokens[(size_t)b * E + i] = i == 0 ? first_tokens[b] : (in_tree[i] ? tok[i - 1] : -1);
  }
  __syncthreads();
  uint8_t* m = mask + (size_t)b * E * E;
  for (int q = t; q < E * E; q += blockDim.x) {
    const int i = q / E, j = q - i * E;
    m[q] = j < 64 ? (uint8_t)((bits_lo[i] >> j) & 1ull) : (uint8_t)bit_hi[i];
  }
}

hipError_t launch_tree_verify_inputs(const int32_t* parents, const int32_t* tokens, const int32_t* first_tokens,
                                     const int32_t* start_positions, int B, int N, uint8_t* mask, int32_t* positions,
                                     int32_t* out_tokens, hipStream_t s) {
  if (B <= 0) return hipSuccess;
  if (N < 1 || N > kVerifyMaxNodes) return hipErrorInvalidValue;
  hipLaunchKernelGGL(tree_verify_inputs_k, dim3(B), dim3(64), 0, s, parents, tokens, first_tokens, start_positions, N,
                     mask, positions, out_tokens);
  return hipGetLastError();
}

}  // namespace dh
