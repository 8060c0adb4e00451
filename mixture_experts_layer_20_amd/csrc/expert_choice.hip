// Expert-choice routing: every expert takes the C tokens with the largest
// router probability for it.
//
// Sources: "Lab 18 -- Mixture of experts", exercise 1 and "Common
// extensions" (the selection runs per expert over the tokens rather than per
// token over the experts, so the load is even by construction, no choice is
// dropped, and a token can receive several experts or none); "Mixture of
// experts" lecture, routing families (selection along the expert axis of the
// token x expert score matrix).
//
// Ties go to the lower token; an expert's picks sit in its rows in token
// order.  The decision is taken on the float32 probabilities as stored.
//
// Kernels:
//   ec_keys_kernel    [T,E] float32 probabilities -> [E,T] uint32 order codes
//                     (an LDS-tiled transpose, so that each expert's column
//                     reads contiguously); codes are at least 1, and 0 marks
//                     "no token" in the selection kernel
//   ec_select_kernel  one 1024-thread workgroup per expert: the n-th largest
//                     code K (n = min(C, T)) by bisection over the 32-bit code
//                     space, each step one count over the expert's codes held
//                     in registers; then, in token order, every code above K
//                     and the first n - #(code > K) codes equal to K are taken,
//                     and a block-wide exclusive scan numbers the picks; the
//                     rows go to an [E,T] staging array, written contiguously
//   ec_sel_kernel     the [E,T] staging array -> sel [T,E] (LDS-tiled transpose)
//   (for E <= 16 both transposes take one thread per token instead)
// The count-based bisection makes no use of atomics and needs no sort: 33
// workgroup-wide sums of per-thread counts.
#include "common.hpp"

namespace moe {
namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / kWave;

// ------------------------------------------------------------------ transpose
constexpr int kTr = 64;          // 64 tokens x 64 experts per tile

__global__ __launch_bounds__(256) void ec_keys_kernel(const float* __restrict__ probs, uint32_t* __restrict__ keys,
                                                      int64_t T, int E) {
  __shared__ uint32_t tile[kTr][kTr + 1];
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kTr;
  const int e0 = blockIdx.y * kTr;
  const int lane = threadIdx.x & (kTr - 1);
  const int row = threadIdx.x / kTr;                 // 0..3
#pragma unroll 4
  for (int r = row; r < kTr; r += 4) {               // read along experts
    const int64_t t = t0 + r;
    const int e = e0 + lane;
    if (t < T && e < E) tile[r][lane] = max(order_code(probs[t * E + e]), 1u);
  }
  __syncthreads();
#pragma unroll 4
  for (int r = row; r < kTr; r += 4) {               // write along tokens
    const int e = e0 + r;
    const int64_t t = t0 + lane;
    if (t < T && e < E) keys[static_cast<int64_t>(e) * T + t] = tile[lane][r];
  }
}

__global__ __launch_bounds__(256) void ec_sel_kernel(const int32_t* __restrict__ selT, int32_t* __restrict__ sel,
                                                     int64_t T, int E) {
  __shared__ int32_t tile[kTr][kTr + 1];
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kTr;
  const int e0 = blockIdx.y * kTr;
  const int lane = threadIdx.x & (kTr - 1);
  const int row = threadIdx.x / kTr;
#pragma unroll 4
  for (int r = row; r < kTr; r += 4) {               // read along tokens
    const int e = e0 + r;
    const int64_t t = t0 + lane;
    if (t < T && e < E) tile[lane][r] = selT[static_cast<int64_t>(e) * T + t];
  }
  __syncthreads();
#pragma unroll 4
  for (int r = row; r < kTr; r += 4) {               // write along experts
    const int64_t t = t0 + r;
    const int e = e0 + lane;
    if (t < T && e < E) sel[t * E + e] = tile[r][lane];
  }
}

// E <= 16: one thread per token, E codes read along the row and written one
// per expert row (consecutive lanes, consecutive tokens)
__global__ __launch_bounds__(256) void ec_keys_rows_kernel(const float* __restrict__ probs,
                                                           uint32_t* __restrict__ keys, int64_t T, int E) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (t >= T) return;
  for (int e = 0; e < E; ++e) keys[static_cast<int64_t>(e) * T + t] = max(order_code(probs[t * E + e]), 1u);
}

__global__ __launch_bounds__(256) void ec_sel_rows_kernel(const int32_t* __restrict__ selT, int32_t* __restrict__ sel,
                                                          int64_t T, int E) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (t >= T) return;
  for (int e = 0; e < E; ++e) sel[t * E + e] = selT[static_cast<int64_t>(e) * T + t];
}

// ------------------------------------------------------------------ selection
// Sum over the wavefront with DPP row shifts and row broadcasts (an inclusive
// scan whose last lane holds the total), read back as a uniform value.  All
// 64 lanes must be active.
__device__ __forceinline__ int wave_sum_i(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);    // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);    // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);    // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);    // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);   // row_bcast:15 into rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);   // row_bcast:31 into rows 2, 3
  return __builtin_amdgcn_readlane(v, 63);
}

// Sum over the workgroup; every thread gets the total.  `buf` holds two banks
// of per-wave sums used alternately, so one barrier per call suffices: a bank
// is rewritten only two calls later, after every thread has passed the
// barrier of the call in between (and so finished reading it).
__device__ __forceinline__ int block_sum(int v, int (*buf)[kSelWaves], int& bank) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  v = wave_sum_i(v);
  if (lane == 0) buf[bank][wave] = v;
  __syncthreads();
  int s = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) s += buf[bank][w];
  bank ^= 1;
  return s;
}

// Exclusive prefix over the workgroup in thread order.
__device__ __forceinline__ int block_excl_scan(int v, int* wtot) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  int inc = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int u = __shfl_up(inc, o, kWave);
    if (lane >= o) inc += u;
  }
  if (lane == kWave - 1) wtot[wave] = inc;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += wtot[w];
  __syncthreads();                                   // wtot is reused by the next scan
  return base + inc - v;
}

// R > 0: thread i holds the codes of tokens [i R, i R + R) in registers
// (T <= 1024 R), code 0 past the last token: every threshold tried is at
// least 1 and K >= 1, so such entries are never counted, equal to K or taken,
// and the counting loops need no per-entry bounds test (whose 64 masks would
// otherwise stay live across the bisection).  R == 0: the same token ranges,
// of P = ceil(T / 1024) codes, re-read from memory in every step (any T).
template <int R>
__global__ __launch_bounds__(kSelThreads) void ec_select_kernel(EcArgs a) {
  __shared__ int sums[2][kSelWaves];
  __shared__ int wtot[kSelWaves];
  __shared__ double dred[kSelThreads];
  __shared__ uint64_t pick_mask[R > 0 ? kSelThreads : 1];
  __shared__ int pick_base[R > 0 ? kSelThreads : 1];
  const int e = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t T = a.T;                             // row stride of keys and selT
  const int64_t len = a.lengths ? a.lengths[e] : T;  // this expert's entries
  const int64_t P = R > 0 ? R : (T + kSelThreads - 1) / kSelThreads;
  const int64_t first = static_cast<int64_t>(tid) * P;
  const int nv = static_cast<int>(max<int64_t>(0, min<int64_t>(P, len - first)));   // codes of this thread
  const uint32_t* __restrict__ col = a.keys + static_cast<int64_t>(e) * T + first;
  const int64_t n = min<int64_t>(a.C, len);

  uint32_t reg[R > 0 ? R : 1];
  if constexpr (R > 0) {
#pragma unroll
    for (int j = 0; j < R; ++j) reg[j] = j < nv ? col[j] : 0u;
  }
  // f(code) over this thread's entries: the register copy (indexed only by
  // unrolled constants; entries past the last token are 0), for the counts
  // of the bisection
  auto each = [&](auto f) {
    if constexpr (R > 0) {
#pragma unroll
      for (int j = 0; j < R; ++j) f(reg[j]);
    } else {
      for (int j = 0; j < nv; ++j) f(col[j]);
    }
  };
  // f(j, code of token first + j) in token order, re-read from memory (the
  // ordered passes of the R == 0 path)
  auto each_in_order = [&](auto f) {
    for (int j = 0; j < nv; ++j) f(j, col[j]);
  };
  // 32-bit compares (a 64-bit one would keep a widened copy of every code)
  auto count_ge = [&](uint32_t v) -> int {
    int c = 0;
    each([&](uint32_t k) { c += k >= v ? 1 : 0; });
    return c;
  };

  // K = the largest v with #(code >= v) >= n, by bisection: invariant
  // #(>= lo) >= n > #(>= hi), every mid in [1, 2^32 - 1].  (Counting several
  // thresholds a step with ballots and scalar popcounts, fewer steps and
  // barriers, measured slower: the scalar adds serialise.)
  int bank = 0;
  uint64_t lo = 0, hi = uint64_t{1} << 32;
  for (int it = 0; it < 32; ++it) {
    const uint64_t mid = (lo + hi) >> 1;
    if (block_sum(count_ge(static_cast<uint32_t>(mid)), sums, bank) >= n) lo = mid;
    else hi = mid;
  }
  const uint32_t K = static_cast<uint32_t>(lo);
  int my_above = 0;
  each([&](uint32_t k) { my_above += k > K ? 1 : 0; });
  const int64_t above = block_sum(my_above, sums, bank);
  const int64_t take_eq = n - above;                 // codes equal to K to take, lowest tokens first
  // in token order: the equal codes before this thread's range, then the picks
  int my_eq = 0;
  each([&](uint32_t k) { my_eq += k == K ? 1 : 0; });
  const int64_t eq_before = block_excl_scan(my_eq, wtot);
  int32_t* __restrict__ rt = a.row_token ? a.row_token + static_cast<int64_t>(e) * a.C : nullptr;
  int32_t* __restrict__ st = a.selT + static_cast<int64_t>(e) * T;
  if constexpr (R > 0) {
    // this thread's picks as a bit mask (R <= 64), numbered through LDS, then
    // written with consecutive lanes on consecutive tokens
    uint64_t gt = 0, eqm = 0;
#pragma unroll
    for (int j = 0; j < R; ++j) {
      gt |= static_cast<uint64_t>(reg[j] > K) << j;
      eqm |= static_cast<uint64_t>(reg[j] == K) << j;
    }
    // of the codes equal to K, the first take_eq - eq_before (if any) are taken
    int64_t room = take_eq - eq_before;
    uint64_t rest = eqm;
    while (room > 0 && rest) {
      rest &= rest - 1;
      --room;
    }
    const uint64_t mask = gt | (eqm ^ rest);
    const int base = block_excl_scan(__popcll(mask), wtot);
    pick_mask[tid] = mask;
    pick_base[tid] = base;
    __syncthreads();
    for (int64_t t = tid; t < len; t += kSelThreads) {
      const int o = static_cast<int>(t / R), j = static_cast<int>(t % R);
      const uint64_t w = pick_mask[o];
      const bool tk = (w >> j) & 1u;
      const int slot = pick_base[o] + __popcll(w & ((uint64_t{1} << j) - 1));
      if (tk && rt) rt[slot] = static_cast<int32_t>(t);
      st[t] = tk ? slot : (a.keep_before ? -slot - 1 : -1);
    }
  } else {
    int my_take = 0;
    {
      int64_t eq = eq_before;
      each_in_order([&](int, uint32_t k) {
        my_take += (k > K || (k == K && eq < take_eq)) ? 1 : 0;
        eq += k == K ? 1 : 0;
      });
    }
    int64_t slot = block_excl_scan(my_take, wtot);
    int64_t eq = eq_before;
    each_in_order([&](int j, uint32_t k) {
      const bool tk = k > K || (k == K && eq < take_eq);
      eq += k == K ? 1 : 0;
      if (tk && rt) rt[slot] = static_cast<int32_t>(first + j);
      st[first + j] = tk ? static_cast<int32_t>(slot) : (a.keep_before ? static_cast<int32_t>(-slot - 1) : -1);
      slot += tk ? 1 : 0;
    });
  }
  if (tid == 0) {
    if (a.counts) a.counts[e] = static_cast<int32_t>(n);
    if (e == 0 && a.fallback_count) a.fallback_count[0] = 0;
  }

  // per-expert probability sums (and, in workgroup 0, the LSE^2 sum) from the
  // router's per-workgroup partials, in a fixed order
  if (a.p_partial) {
    auto reduce = [&](auto load) {
      double v = 0.0;
      for (int r = tid; r < a.n_rtiles; r += kSelThreads) v += load(r);
      dred[tid] = v;
      __syncthreads();
      for (int o = kSelThreads / 2; o > 0; o >>= 1) {
        if (tid < o) dred[tid] += dred[tid + o];
        __syncthreads();
      }
      const double out = dred[0];
      __syncthreads();
      return out;
    };
    const double Ps = reduce([&](int r) { return a.p_partial[static_cast<int64_t>(r) * a.E + e]; });
    if (tid == 0) a.psum[e] = Ps;
    if (e == 0) {
      const double z2 = reduce([&](int r) { return a.lse2_partial[r]; });
      if (tid == 0) a.psum[a.E] = z2;
    }
  }
}

// T = 0: no picks; the counts, the sums and the fallback count are zero.
__global__ __launch_bounds__(256) void ec_empty_kernel(EcArgs a) {
  for (int e = threadIdx.x; e <= a.E; e += blockDim.x) {
    if (e < a.E) a.counts[e] = 0;
    if (a.p_partial) a.psum[e] = 0.0;
  }
  if (threadIdx.x == 0 && a.fallback_count) a.fallback_count[0] = 0;
}

}  // namespace

hipError_t launch_select_top(const EcArgs& a, hipStream_t s) {
  const unsigned grid = static_cast<unsigned>(a.E);
  if (a.T <= int64_t{kSelThreads} * 8)
    ec_select_kernel<8><<<grid, kSelThreads, 0, s>>>(a);
  else if (a.T <= int64_t{kSelThreads} * 16)
    ec_select_kernel<16><<<grid, kSelThreads, 0, s>>>(a);
  else if (a.T <= int64_t{kSelThreads} * 64)
    ec_select_kernel<64><<<grid, kSelThreads, 0, s>>>(a);
  else
    ec_select_kernel<0><<<grid, kSelThreads, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_expert_choice(const EcArgs& a, hipStream_t s) {
  if (a.E == 0) return hipSuccess;
  if (a.T == 0) {
    ec_empty_kernel<<<1, 256, 0, s>>>(a);
    return hipGetLastError();
  }
  const dim3 tg(static_cast<unsigned>((a.T + kTr - 1) / kTr), static_cast<unsigned>((a.E + kTr - 1) / kTr));
  const unsigned rows_grid = static_cast<unsigned>((a.T + 255) / 256);
  const bool by_rows = a.E <= 16;
  if (by_rows)
    ec_keys_rows_kernel<<<rows_grid, 256, 0, s>>>(a.probs, a.keys, a.T, a.E);
  else
    ec_keys_kernel<<<tg, 256, 0, s>>>(a.probs, a.keys, a.T, a.E);
  const hipError_t err = launch_select_top(a, s);
  if (err != hipSuccess) return err;
  if (by_rows)
    ec_sel_rows_kernel<<<rows_grid, 256, 0, s>>>(a.selT, a.sel, a.T, a.E);
  else
    ec_sel_kernel<<<tg, 256, 0, s>>>(a.selT, a.sel, a.T, a.E);
  return hipGetLastError();
}

}  // namespace moe
