// Expert capacity with deterministic slot assignment, and the dispatch of
// token rows into expert-contiguous buffers.
//
// Sources: "Lab 18 -- Mixture of experts" s.3 (C = ceil(cf*T*k/E); GShard
// priority: every first choice before any second choice, token order inside
// a rank; a slot past C is dropped) and Tips (flatten rank-major, one-hot,
// cumulative sum: the entry of the assignment's own expert minus one is its
// queue position); "Lab 01" "Where to start" 4 (first come, first served in
// token order); "Parameters without the FLOPs" s.3 (fixed per-expert buffers).
//
// The queue position of an assignment is the number of earlier assignments
// (in priority order) to the same expert, i.e. a stable counting sort by
// expert.  It is computed without atomics, in three launches:
//   hist    per (rank j, 64-token tile) expert histogram, from wavefront
//           ballots over the bits of the expert id;
//   scan    per expert, an exclusive prefix sum over the (j, tile) sequence
//           in priority order (rank-major) or over tiles (token-major);
//   permute per tile: in-tile rank from the same ballots + the tile's offset
//           = slot; writes slot/dropped/row_token and copies each token row
//           once into every kept destination with 16-byte accesses.
// Dropless mode (packed rows) keeps every choice and lays the experts' rows
// back to back: row = (sum of the counts of lower experts) + queue position.
#include "common.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kCodeBits = 9;         // expert ids 0..255, code 256 = "no token"
constexpr int kNoToken = 256;

// Lanes of this wavefront whose `code` equals `mine` (code is per lane, the
// ballots make the comparison wave-wide with 9 ballots and no LDS).
__device__ __forceinline__ uint64_t match_lanes(int code, int mine) {
  uint64_t m = ~0ull;
#pragma unroll
  for (int b = 0; b < kCodeBits; ++b) {
    const uint64_t bal = __ballot((code >> b) & 1);
    m &= ((mine >> b) & 1) ? bal : ~bal;
  }
  return m;
}

// An expert id outside [0, E) (invalid input) takes no slot and is dropped.
__device__ __forceinline__ int load_code(const CapArgs& a, bool valid, int64_t t, int j) {
  if (!valid) return kNoToken;
  const int v = a.idx[t * a.k + j];
  return (v >= 0 && v < a.E) ? v : kNoToken;
}

__global__ __launch_bounds__(kThreads) void hist_kernel(CapArgs a) {
  __shared__ int cnt[kThreads / kWave][256];
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int tile = blockIdx.x * (kThreads / kWave) + wave;
  const int64_t t = static_cast<int64_t>(tile) * kTileTokens + lane;
  const bool valid = tile < a.n_tiles && t < a.T;
  for (int j = 0; j < a.k; ++j) {
    const int code = load_code(a, valid, t, j);
    const uint64_t m = match_lanes(code, code);
    for (int e = lane; e < a.E; e += kWave) cnt[wave][e] = 0;
    __syncthreads();
    if (code != kNoToken && (m & lanemask_lt()) == 0) cnt[wave][code] = __popcll(m);
    __syncthreads();
    if (tile < a.n_tiles)
      for (int e = lane; e < a.E; e += kWave)
        a.hist[(static_cast<int64_t>(j) * a.n_tiles + tile) * a.E + e] = cnt[wave][e];
    __syncthreads();
  }
}

// One workgroup per expert: exclusive prefix over the priority sequence.
__global__ __launch_bounds__(kThreads) void scan_kernel(CapArgs a) {
  __shared__ int part[kThreads];
  const int e = blockIdx.x;
  const int tid = threadIdx.x;
  const bool tm = a.token_major != 0;
  const int64_t L = tm ? a.n_tiles : static_cast<int64_t>(a.k) * a.n_tiles;
  const int64_t per = (L + kThreads - 1) / kThreads;
  const int64_t lo = min<int64_t>(L, tid * per), hi = min<int64_t>(L, lo + per);
  auto entry = [&](int64_t s) -> int {
    if (!tm) return a.hist[s * a.E + e];
    int v = 0;
    for (int j = 0; j < a.k; ++j) v += a.hist[(static_cast<int64_t>(j) * a.n_tiles + s) * a.E + e];
    return v;
  };
  int sum = 0;
  for (int64_t s = lo; s < hi; ++s) sum += entry(s);
  part[tid] = sum;
  __syncthreads();
  // inclusive Hillis-Steele scan of the 256 chunk sums
  for (int o = 1; o < kThreads; o <<= 1) {
    const int v = tid >= o ? part[tid - o] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int run = part[tid] - sum;         // exclusive prefix of this chunk
  for (int64_t s = lo; s < hi; ++s) {
    const int v = entry(s);
    if (!tm) {
      a.hist[s * a.E + e] = run;
    } else {
      for (int j = 0; j < a.k; ++j) a.hist[(static_cast<int64_t>(j) * a.n_tiles + s) * a.E + e] = run;
    }
    run += v;
  }
  if (tid == kThreads - 1) {
    const int total = part[kThreads - 1];
    a.counts[e] = total;
    if (a.kept) a.kept[e] = static_cast<int>(min<int64_t>(total, a.C));
  }
  // the router's per-workgroup partial sums of P_e (and, in block 0, of
  // LSE^2), reduced in a fixed order: strided per thread, then a fixed tree
  if (a.p_partial) {
    __shared__ double dred[kThreads];
    auto reduce = [&](auto load) {
      double v = 0.0;
      for (int r = tid; r < a.n_rtiles; r += kThreads) v += load(r);
      dred[tid] = v;
      __syncthreads();
      for (int o = kThreads / 2; o > 0; o >>= 1) {
        if (tid < o) dred[tid] += dred[tid + o];
        __syncthreads();
      }
      const double out = dred[0];
      __syncthreads();
      return out;
    };
    const double P = reduce([&](int r) { return a.p_partial[static_cast<int64_t>(r) * a.E + e]; });
    if (tid == 0) a.psum[e] = P;
    if (e == 0) {
      const double z2 = reduce([&](int r) { return a.lse2_partial[r]; });
      if (tid == 0) a.psum[a.E] = z2;
    }
  }
}

template <typename XT>
__global__ __launch_bounds__(kThreads) void permute_kernel(CapArgs a) {
  __shared__ int64_t dest[kTileTokens][32];   // row of xe per (token, choice), -1 dropped
  __shared__ int any_kept[kTileTokens];
  __shared__ int off[kThreads];               // packed rows: first row of each expert
  const int tile = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int k = a.k;
  const int64_t t0 = static_cast<int64_t>(tile) * kTileTokens;
  const int nt = static_cast<int>(min<int64_t>(kTileTokens, a.T - t0));
  if (a.packed) {
    // exclusive prefix sum of the expert counts (E <= 256 = threads)
    const int v = tid < a.E ? a.counts[tid] : 0;
    off[tid] = v;
    __syncthreads();
    for (int o = 1; o < kThreads; o <<= 1) {
      const int u = tid >= o ? off[tid - o] : 0;
      __syncthreads();
      off[tid] += u;
      __syncthreads();
    }
    const int incl = off[tid];
    __syncthreads();
    off[tid] = incl - v;
    __syncthreads();
  }
  if (tid < kWave) {
    const int64_t t = t0 + lane;
    const bool valid = lane < nt;
    bool kept_any = false;
    for (int j = 0; j < k; ++j) {
      const int code = load_code(a, valid, t, j);
      int rank;
      if (!a.token_major) {
        rank = __popcll(match_lanes(code, code) & lanemask_lt());
      } else {
        rank = 0;
        for (int jj = 0; jj < k; ++jj) {
          const int other = load_code(a, valid, t, jj);
          rank += __popcll(match_lanes(other, code) & lanemask_lt());
        }
      }
      if (valid && code == kNoToken) {
        a.slot[t * k + j] = -1;
        a.dropped[t * k + j] = 1;
        dest[lane][j] = -1;
      } else if (valid) {
        const int64_t s = static_cast<int64_t>(a.hist[(static_cast<int64_t>(j) * a.n_tiles + tile) * a.E + code]) + rank;
        // packed rows: nothing is dropped and the slot is the row itself
        const bool drop = !a.packed && s >= a.C;
        const int64_t row = a.packed ? off[code] + s : static_cast<int64_t>(code) * a.C + s;
        a.slot[t * k + j] = static_cast<int32_t>(a.packed ? row : s);
        a.dropped[t * k + j] = drop ? 1 : 0;
        if (!drop) {
          kept_any = true;
          if (a.row_token) a.row_token[row] = static_cast<int32_t>(t);
        }
        dest[lane][j] = drop ? -1 : row;
      }
    }
    const uint64_t fb = __ballot(valid && !kept_any);
    if (lane == 0 && a.fallback_partial) a.fallback_partial[tile] = __popcll(fb);
    any_kept[lane] = valid && kept_any;
  }
  if (a.xe == nullptr) return;
  __syncthreads();
  // copy: each token row read once, written to every kept destination
  const int nvec = a.d * static_cast<int>(sizeof(XT)) / 16;
  const uint4* x = static_cast<const uint4*>(a.x);
  uint4* xe = static_cast<uint4*>(a.xe);
  const int64_t rowvec = nvec;
  const int total = nt * nvec;
  constexpr int kU = 4;
  for (int base = 0; base < total; base += kThreads * kU) {
    uint4 v[kU];
    int tt[kU], c[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i = base + u * kThreads + tid;
      tt[u] = i < total ? i / nvec : -1;
      c[u] = i < total ? i % nvec : 0;
      if (tt[u] >= 0 && any_kept[tt[u]]) v[u] = x[(t0 + tt[u]) * rowvec + c[u]];
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (tt[u] < 0 || !any_kept[tt[u]]) continue;
      for (int j = 0; j < k; ++j) {
        const int64_t r = dest[tt[u]][j];
        if (r >= 0) xe[r * rowvec + c[u]] = v[u];
      }
    }
  }
}

}  // namespace

hipError_t launch_capacity(const CapArgs& a, int dtype, hipStream_t s) {
  if (a.n_tiles > 0) {
    const unsigned g1 = static_cast<unsigned>((a.n_tiles + 3) / 4);
    hist_kernel<<<g1, kThreads, 0, s>>>(a);
  }
  scan_kernel<<<a.E, kThreads, 0, s>>>(a);
  if (a.n_tiles > 0) {
    if (dtype == MOE_BF16)
      permute_kernel<bf16_t><<<a.n_tiles, kThreads, 0, s>>>(a);
    else
      permute_kernel<float><<<a.n_tiles, kThreads, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace moe
