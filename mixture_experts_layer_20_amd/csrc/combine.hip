// Gate-weighted combine with residual fallback, and the loss finaliser.
//
// Sources: "Lab 18 -- Mixture of experts" s.1 (y = sum of gated expert
// outputs), s.2 (Switch loss E * sum f_i P_i with f over the T*k assignments;
// router z-loss) and s.3 (a dropped slot contributes nothing; a token whose
// every assignment was dropped reaches the next layer unchanged); "Lab 01"
// "Where to start" 5 (the residual fallback) and "The traps" (f divides by
// T*k); "Phase 02" concept map (shared expert for every token).
#include "common.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kTokensPerBlock = 4;

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
template <typename T>
__global__ __launch_bounds__(kThreads) void combine_kernel(CombineArgs a) {
  constexpr int V = Vec<T>::N;
  const int nvec = a.d / V;
  const int64_t rowbytes = static_cast<int64_t>(a.d) * sizeof(T);
  const char* ye = static_cast<const char*>(a.ye);
  const char* x = static_cast<const char*>(a.x);
  const char* sh = static_cast<const char*>(a.shared_out);
  char* y = static_cast<char*>(a.y);
  for (int i = 0; i < kTokensPerBlock; ++i) {
    const int64_t t = static_cast<int64_t>(blockIdx.x) * kTokensPerBlock + i;
    if (t >= a.T) return;
    const int64_t tk = t * a.k;
    // a choice counts only if it is kept and its (expert, slot) is in range
    auto kept = [&](int j) {
      const int e = a.idx[tk + j];
      const int s = a.slot[tk + j];
      return !a.dropped[tk + j] && e >= 0 && e < a.E && s >= 0 && s < a.C;
    };
    bool any = false;
    for (int j = 0; j < a.k; ++j) any = any || kept(j);
    for (int c = threadIdx.x; c < nvec; c += kThreads) {
      const int64_t off = static_cast<int64_t>(c) * 16;
      float acc[V];
      if (!any && sh == nullptr) {
        if (a.zero_fallback) {
#pragma unroll
          for (int q = 0; q < V; ++q) acc[q] = 0.0f;
        } else {
          Vec<T>::load(x + t * rowbytes + off, acc);
        }
      } else {
#pragma unroll
        for (int q = 0; q < V; ++q) acc[q] = 0.0f;
        for (int j = 0; j < a.k; ++j) {
          if (!kept(j)) continue;
          const int64_t row = static_cast<int64_t>(a.idx[tk + j]) * a.C + a.slot[tk + j];
          const float g = a.gates[tk + j];
          float v[V];
          Vec<T>::load(ye + row * rowbytes + off, v);
#pragma unroll
          for (int q = 0; q < V; ++q) acc[q] += g * v[q];
        }
        if (sh) {
          float v[V];
          Vec<T>::load(sh + t * rowbytes + off, v);
#pragma unroll
          for (int q = 0; q < V; ++q) acc[q] += v[q];
        }
      }
      Vec<T>::store(y + t * rowbytes + off, acc);
    }
  }
}

// One workgroup: fixed-order float64 reductions of the router partials and
// the capacity counts into L_aux, L_z and the drop statistics.
__global__ __launch_bounds__(kThreads) void losses_kernel(LossArgs a) {
  __shared__ double red[kThreads];
  __shared__ long long ired[kThreads];
  const int tid = threadIdx.x;
  // per-expert mean probability P_i, times f_i
  double fp = 0.0;
  long long kept = 0;
  for (int e = tid; e < a.E && a.T > 0; e += kThreads) {
    double P = 0.0;
    for (int r = 0; r < a.n_rtiles; ++r) P += a.p_partial[static_cast<int64_t>(r) * a.E + e];
    const double T = static_cast<double>(a.T);
    const double f = static_cast<double>(a.counts[e]) / (T * a.k);
    fp += f * (P / T);
    kept += min<long long>(a.counts[e], a.C);
  }
  red[tid] = fp;
  ired[tid] = kept;
  __syncthreads();
  for (int o = kThreads / 2; o > 0; o >>= 1) {
    if (tid < o) { red[tid] += red[tid + o]; ired[tid] += ired[tid + o]; }
    __syncthreads();
  }
  const double l_aux = static_cast<double>(a.E) * red[0];
  const long long n_kept = ired[0];
  __syncthreads();
  double z2 = 0.0;
  long long fb = 0;
  for (int r = tid; r < a.n_rtiles; r += kThreads) z2 += a.lse2_partial[r];
  if (a.fallback_partial)
    for (int r = tid; r < a.n_tiles; r += kThreads) fb += a.fallback_partial[r];
  red[tid] = z2;
  ired[tid] = fb;
  __syncthreads();
  for (int o = kThreads / 2; o > 0; o >>= 1) {
    if (tid < o) { red[tid] += red[tid + o]; ired[tid] += ired[tid + o]; }
    __syncthreads();
  }
  if (tid == 0) {
    a.losses[0] = static_cast<float>(l_aux);
    a.losses[1] = a.T > 0 ? static_cast<float>(red[0] / static_cast<double>(a.T)) : 0.0f;
    if (a.stats) {
      const long long total = a.T * a.k;
      a.stats[0] = static_cast<int32_t>(n_kept);
      a.stats[1] = static_cast<int32_t>(total - n_kept);
      a.stats[2] = a.has_shared ? 0 : static_cast<int32_t>(ired[0]);
      a.stats[3] = static_cast<int32_t>(static_cast<long long>(a.E) * a.C - n_kept);
    }
  }
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, int dtype, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const unsigned grid = static_cast<unsigned>((a.T + kTokensPerBlock - 1) / kTokensPerBlock);
  if (dtype == MOE_BF16)
    combine_kernel<bf16_t><<<grid, kThreads, 0, s>>>(a);
  else
    combine_kernel<float><<<grid, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_losses(const LossArgs& a, hipStream_t s) {
  losses_kernel<<<1, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace moe
