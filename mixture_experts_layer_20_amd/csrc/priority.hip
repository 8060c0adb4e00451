// Batch-prioritised capacity: which assignments an expert keeps is decided
// by router score instead of queue position.
//
// Source: "Lab 18 -- Mixture of experts" s.3 (who is dropped depends on the
// priority; the V-MoE alternative ranks assignments by router score).
//
// Reading: the score of an assignment is its gate (float32, as the router
// stores it); each expert keeps the C assignments with the largest score,
// equal scores to the one earlier in the GShard queue (every first choice
// before any second choice, token order inside a rank); the kept ones take
// slots 0.. in queue order, the dropped ones C.. in queue order.
//
// Launch sequence (after the usual histogram/scan/permute pass has given
// every assignment its rank-major queue position q with room for all):
//   score_keys_kernel    key of (t, j) -> keys[e, q] (order code >= 1)
//   ec_select_kernel     per expert, over its count_e queue entries: the C
//                        largest keys, equal keys to the lower q, numbered in
//                        q order (shared with expert-choice routing)
//   score_finish_kernel  per 64-token tile: slot, dropped, row_token, the
//                        fully dropped tokens of the tile, kept = min(count, C)
//   gather_rows_kernel   optional copy of the kept token rows into xe
#include "common.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void score_keys_kernel(ScoreArgs a) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= a.T * a.k) return;
  const int e = a.idx[i];
  const int q = a.queue[i];
  if (e < 0 || e >= a.E || q < 0) return;
  a.keys[static_cast<int64_t>(e) * a.T + q] = max(order_code(a.gates[i]), 1u);
}

// One wavefront per 64-token tile (the tiles of the capacity kernels).
__global__ __launch_bounds__(kThreads) void score_finish_kernel(ScoreArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t g = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (g < a.E) a.kept[g] = static_cast<int32_t>(min<int64_t>(a.counts[g], a.C));
  const int64_t tile = g / kWave;
  if (tile >= a.n_tiles) return;                     // whole wavefronts leave together
  const int64_t t = tile * kWave + lane;
  const bool valid = t < a.T;
  bool kept_any = false;
  if (valid) {
    for (int j = 0; j < a.k; ++j) {
      const int64_t i = t * a.k + j;
      const int e = a.idx[i];
      const int q = a.queue[i];
      if (e < 0 || e >= a.E || q < 0) {              // invalid expert id: no slot
        a.slot[i] = -1;
        a.dropped[i] = 1;
        continue;
      }
      const int v = a.selT[static_cast<int64_t>(e) * a.T + q];
      if (v >= 0) {
        a.slot[i] = v;
        a.dropped[i] = 0;
        if (a.row_token) a.row_token[static_cast<int64_t>(e) * a.C + v] = static_cast<int32_t>(t);
        kept_any = true;
      } else {
        const int before = -v - 1;                   // kept entries ahead of q
        a.slot[i] = static_cast<int32_t>(a.C + (q - before));
        a.dropped[i] = 1;
      }
    }
  }
  const uint64_t fb = __ballot(valid && !kept_any);
  if (lane == 0 && a.fallback_partial) a.fallback_partial[tile] = __popcll(fb);
}

// xe[e, s] = x[row_token[e, s]] for s < kept[e]; one wavefront per row.
__global__ __launch_bounds__(kThreads) void gather_rows_kernel(const void* __restrict__ x, void* __restrict__ xe,
                                                               const int32_t* __restrict__ row_token,
                                                               const int32_t* __restrict__ kept, int64_t C,
                                                               int64_t n_rows, int row_bytes) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t r = (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) / kWave;
  if (r >= n_rows) return;
  const int64_t e = r / C, s = r % C;
  if (s >= kept[e]) return;
  const uint4* src = reinterpret_cast<const uint4*>(static_cast<const char*>(x) +
                                                    static_cast<int64_t>(row_token[r]) * row_bytes);
  uint4* dst = reinterpret_cast<uint4*>(static_cast<char*>(xe) + r * row_bytes);
  for (int c = lane; c < row_bytes / 16; c += kWave) dst[c] = src[c];
}

}  // namespace

hipError_t launch_score_priority(const ScoreArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const unsigned g1 = static_cast<unsigned>((a.T * a.k + kThreads - 1) / kThreads);
  score_keys_kernel<<<g1, kThreads, 0, s>>>(a);
  EcArgs sel{};
  sel.keys = a.keys;
  sel.selT = a.selT;
  sel.lengths = a.counts;
  sel.keep_before = 1;
  sel.T = a.T;
  sel.C = a.C;
  sel.E = a.E;
  hipError_t err = launch_select_top(sel, s);
  if (err != hipSuccess) return err;
  const unsigned g2 = static_cast<unsigned>((a.n_tiles * kWave + kThreads - 1) / kThreads);
  score_finish_kernel<<<max(g2, static_cast<unsigned>((a.E + kThreads - 1) / kThreads)), kThreads, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const void* x, void* xe, const int32_t* row_token, const int32_t* kept, int64_t C,
                              int E, int row_bytes, hipStream_t s) {
  const int64_t n_rows = C * E;
  if (n_rows == 0) return hipSuccess;
  const unsigned g = static_cast<unsigned>((n_rows * kWave + kThreads - 1) / kThreads);
  gather_rows_kernel<<<g, kThreads, 0, s>>>(x, xe, row_token, kept, C, n_rows, row_bytes);
  return hipGetLastError();
}

}  // namespace moe
