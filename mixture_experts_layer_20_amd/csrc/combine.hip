// Gate-weighted combine with residual fallback, and the loss finaliser.
//
// Sources: "Lab 18 -- Mixture of experts" s.1 (y = sum of gated expert
// outputs), s.2 (Switch loss E * sum f_i P_i with f over the T*k assignments;
// router z-loss) and s.3 (dropped slots add nothing; a token left with no
// kept assignment passes its input through); "Lab 01"
// "Where to start" 5 (the residual fallback) and "The traps" (f divides by
// T*k); "Phase 02" concept map (shared expert for every token).
#include "common.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

template <typename T>
struct Vec;  // 16 bytes of storage as float32 lanes
template <> struct Vec<bf16_t> {
  static constexpr int N = 8;
  __device__ static void load(const void* p, float* v) {
    const uint4 r = *static_cast<const uint4*>(p);
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[2 * q] = __uint_as_float(w[q] << 16);
      v[2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u);
    }
  }
  __device__ static void store(void* p, const float* v) {
    uint4 r;
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      w[q] = static_cast<uint32_t>(f32_to_bf16(v[2 * q])) | (static_cast<uint32_t>(f32_to_bf16(v[2 * q + 1])) << 16);
    r.x = w[0]; r.y = w[1]; r.z = w[2]; r.w = w[3];
    *static_cast<uint4*>(p) = r;
  }
};
template <> struct Vec<float> {
  static constexpr int N = 4;
  __device__ static void load(const void* p, float* v) {
    const float4 r = *static_cast<const float4*>(p);
    v[0] = r.x; v[1] = r.y; v[2] = r.z; v[3] = r.w;
  }
  __device__ static void store(void* p, const float* v) {
    *static_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  }
};

// y_t = sum_{j kept} g_tj * ye[e_tj, s_tj] (+ shared_t), float32 in j order,
// one rounding; fallback x_t (or 0) when nothing was kept and no shared expert.
// One wavefront per token.  Lanes j < k read choice j (one round of loads);
// a ballot gives the kept choices, whose row index and gate every lane then
// reads from the owning lane.  Each lane streams 16-byte chunks
// c = lane + 64 u of the row, kChunkRounds at a time, issuing the loads of
// up to kRowsAtOnce kept rows before summing.  Measured: a small batch per
// wave (2 x 2) beats a deep one (4 x 4, 8 x 4), since the lighter wave
// leaves room for more resident wavefronts; the expert rows are read once,
// with non-temporal loads (about 5-10% faster; non-temporal stores of y are
// not).
// Expert choice (EC): lane l reads experts l, l + 64, ... (E <= 256, so up to
// four ballots); the picks are summed in expert order, ballot by ballot.
constexpr int kChunkRounds = 2;
constexpr int kRowsAtOnce = 2;

template <typename T, bool EC>
__global__ __launch_bounds__(kThreads) void combine_kernel(CombineArgs a) {
  constexpr int V = Vec<T>::N;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t t = static_cast<int64_t>(blockIdx.x) * (kThreads / kWave) + threadIdx.x / kWave;
  if (t >= a.T) return;
  const int nvec = a.d / V;
  const int64_t rowbytes = static_cast<int64_t>(a.d) * sizeof(T);
  const char* __restrict__ ye = static_cast<const char*>(a.ye);
  const char* __restrict__ x = static_cast<const char*>(a.x);
  const char* __restrict__ sh = static_cast<const char*>(a.shared_out);
  char* __restrict__ y = static_cast<char*>(a.y);

  // choice j on lane j: kept only if not dropped and its (expert, slot) is in
  // range; its row of ye is e*C + slot, or the slot itself for packed rows
  constexpr int kBal = EC ? 4 : 1;
  int64_t myrow[kBal];
  float mygate[kBal];
  uint64_t kept[kBal];
  int n = 0;
#pragma unroll
  for (int b = 0; b < kBal; ++b) {
    myrow[b] = 0;
    mygate[b] = 0.0f;
    bool keep = false;
    if constexpr (EC) {
      const int e = b * kWave + lane;
      if (e < a.E) {
        const int sl = a.sel[t * a.E + e];
        keep = sl >= 0 && sl < a.C;
        myrow[b] = static_cast<int64_t>(e) * a.C + sl;
        mygate[b] = a.probs[t * a.E + e];
      }
    } else if (lane < a.k) {
      const int64_t tk = t * a.k + lane;
      const int e = a.idx[tk];
      const int sl = a.slot[tk];
      const int64_t bound = a.packed ? a.T * a.k : a.C;
      keep = !a.dropped[tk] && e >= 0 && e < a.E && sl >= 0 && sl < bound;
      myrow[b] = a.packed ? static_cast<int64_t>(sl) : static_cast<int64_t>(e) * a.C + sl;
      mygate[b] = a.gates[tk];
    }
    kept[b] = __ballot(keep);
    n += __popcll(kept[b]);
  }
  char* yt = y + t * rowbytes;

  if (n == 0 && sh == nullptr) {
    if (EC && a.fallback_count && lane == 0) atomicAdd(a.fallback_count, 1);   // integer: order-free
    // fallback: the token's own row, or zeros
    for (int c = lane; c < nvec; c += kWave) {
      float v[V];
      if (a.zero_fallback) {
#pragma unroll
        for (int q = 0; q < V; ++q) v[q] = 0.0f;
      } else {
        Vec<T>::load(x + t * rowbytes + static_cast<int64_t>(c) * 16, v);
      }
      Vec<T>::store(yt + static_cast<int64_t>(c) * 16, v);
    }
    return;
  }

  for (int c0 = 0; c0 < nvec; c0 += kChunkRounds * kWave) {
    float acc[kChunkRounds][V];
#pragma unroll
    for (int u = 0; u < kChunkRounds; ++u)
#pragma unroll
      for (int q = 0; q < V; ++q) acc[u][q] = 0.0f;
    // kept choices in j order, kRowsAtOnce rows per batch
#pragma unroll
    for (int bal = 0; bal < kBal; ++bal) {
      uint64_t rest = kept[bal];
      while (rest) {
        const char* src[kRowsAtOnce];
        float g[kRowsAtOnce];
        int nb = 0;
#pragma unroll
        for (int r = 0; r < kRowsAtOnce; ++r) {
          src[r] = ye;
          g[r] = 0.0f;
          if (rest) {
            const int j = __ffsll(static_cast<unsigned long long>(rest)) - 1;
            rest &= rest - 1;
            src[r] = ye + __shfl(myrow[bal], j, kWave) * rowbytes;
            g[r] = __shfl(mygate[bal], j, kWave);
            nb = r + 1;
          }
        }
        // raw 16-byte chunks in flight (widened only when summed)
        uint4 raw[kRowsAtOnce][kChunkRounds];
#pragma unroll
        for (int r = 0; r < kRowsAtOnce; ++r)
#pragma unroll
          for (int u = 0; u < kChunkRounds; ++u) {
            const int c = c0 + lane + u * kWave;
            if (r < nb && c < nvec) {
              const uint4* pp = reinterpret_cast<const uint4*>(src[r] + static_cast<int64_t>(c) * 16);
              const u32x4_t q = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(pp));
              raw[r][u] = make_uint4(q[0], q[1], q[2], q[3]);
            }
          }
#pragma unroll
        for (int r = 0; r < kRowsAtOnce; ++r)
          if (r < nb)
#pragma unroll
            for (int u = 0; u < kChunkRounds; ++u) {
              float v[V];
              Vec<T>::load(&raw[r][u], v);
#pragma unroll
              for (int q = 0; q < V; ++q) acc[u][q] += g[r] * v[q];
            }
      }
    }
#pragma unroll
    for (int u = 0; u < kChunkRounds; ++u) {
      const int c = c0 + lane + u * kWave;
      if (c >= nvec) continue;
      const int64_t off = static_cast<int64_t>(c) * 16;
      if (sh) {
        float vv[V];
        Vec<T>::load(sh + t * rowbytes + off, vv);
#pragma unroll
        for (int q = 0; q < V; ++q) acc[u][q] += vv[q];
      }
      Vec<T>::store(yt + off, acc[u]);
    }
  }
}

// One workgroup: L_aux = E * sum_i f_i P_i and L_z from the per-expert sums
// the capacity scan reduced, plus the drop statistics; fixed-order trees.
__global__ __launch_bounds__(kThreads) void losses_kernel(LossArgs a) {
  __shared__ double red[kThreads];
  __shared__ long long ired[kThreads];
  __shared__ long long fred[kThreads];
  const int tid = threadIdx.x;
  const double T = static_cast<double>(a.T);
  // f_i divides by the T*k choices (token choice) or by the sum of the picks
  // (expert choice, every expert's count being min(C, T))
  const double fden = a.ec ? static_cast<double>(a.E) * static_cast<double>(min<int64_t>(a.C, a.T))
                           : T * a.k;
  double fp = 0.0;
  long long kept = 0;
  for (int e = tid; e < a.E; e += kThreads) {
    if (a.T > 0) fp += (static_cast<double>(a.counts[e]) / fden) * (a.psum[e] / T);
    kept += min<long long>(a.counts[e], a.C);
  }
  long long fb = 0;
  if (a.fallback_partial)
    for (int r = tid; r < a.n_tiles; r += kThreads) fb += a.fallback_partial[r];
  if (a.ec && a.fallback_count && tid == 0) fb = a.fallback_count[0];
  red[tid] = fp;
  ired[tid] = kept;
  fred[tid] = fb;
  __syncthreads();
  for (int o = kThreads / 2; o > 0; o >>= 1) {
    if (tid < o) {
      red[tid] += red[tid + o];
      ired[tid] += ired[tid + o];
      fred[tid] += fred[tid + o];
    }
    __syncthreads();
  }
  if (tid == 0) {
    const long long n_kept = ired[0];
    a.losses[0] = static_cast<float>(static_cast<double>(a.E) * red[0]);
    a.losses[1] = a.T > 0 ? static_cast<float>(a.psum[a.E] / T) : 0.0f;
    if (a.stats) {
      const long long total = a.ec ? n_kept : a.T * a.k;
      a.stats[0] = static_cast<int32_t>(n_kept);
      a.stats[1] = static_cast<int32_t>(total - n_kept);
      a.stats[2] = a.has_shared ? 0 : static_cast<int32_t>(fred[0]);
      a.stats[3] = a.packed ? 0 : static_cast<int32_t>(static_cast<long long>(a.E) * a.C - n_kept);
    }
  }
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, int dtype, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  constexpr int kTokensPerBlock = kThreads / kWave;     // one wavefront per token
  const unsigned grid = static_cast<unsigned>((a.T + kTokensPerBlock - 1) / kTokensPerBlock);
  if (a.sel) {
    if (dtype == MOE_BF16)
      combine_kernel<bf16_t, true><<<grid, kThreads, 0, s>>>(a);
    else
      combine_kernel<float, true><<<grid, kThreads, 0, s>>>(a);
  } else if (dtype == MOE_BF16) {
    combine_kernel<bf16_t, false><<<grid, kThreads, 0, s>>>(a);
  } else {
    combine_kernel<float, false><<<grid, kThreads, 0, s>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_losses(const LossArgs& a, hipStream_t s) {
  losses_kernel<<<1, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace moe
