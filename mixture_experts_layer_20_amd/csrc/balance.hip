// Balancing variants: the sequence-wise balance loss and the
// auxiliary-loss-free update of the selection bias.
//
// Sources: "Lab 18 -- Mixture of experts" s.2 (auxiliary-loss-free balancing:
// a per-expert bias used for selection only, moved by a fixed small step
// against the observed load; a small sequence-wise balance loss is kept) and
// its exercise 4 (a step of 0.001); "Mixture of experts" lecture, DeepSeek
// section (the balancing unit is where the variants differ; the
// sequence-level term guards against one sequence overwhelming a few experts).
#include "common.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;

// One workgroup per sequence: its choices counted per expert (integer LDS
// atomics, exact in any order), each expert's probabilities summed over the
// sequence's tokens in token order in float64, then E * sum_i f_i P_i for the
// sequence with the experts combined in a fixed tree.
__global__ __launch_bounds__(kThreads) void seq_loss_kernel(SeqLossArgs a) {
  __shared__ int cnt[256];
  __shared__ double red[kThreads];
  const int tid = threadIdx.x;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * a.seq_len;
  for (int e = tid; e < a.E; e += kThreads) cnt[e] = 0;
  __syncthreads();
  const int64_t n = a.seq_len * a.k;
  for (int64_t i = tid; i < n; i += kThreads) {
    const int e = a.idx[t0 * a.k + i];
    if (e >= 0 && e < a.E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  double v = 0.0;
  for (int e = tid; e < a.E; e += kThreads) {
    const float* p = a.probs + t0 * a.E + e;
    double P = 0.0;
    for (int64_t t = 0; t < a.seq_len; ++t) P += static_cast<double>(p[t * a.E]);
    v += (static_cast<double>(cnt[e]) / (static_cast<double>(a.seq_len) * a.k)) *
         (P / static_cast<double>(a.seq_len));
  }
  red[tid] = v;
  __syncthreads();
  for (int o = kThreads / 2; o > 0; o >>= 1) {
    if (tid < o) red[tid] += red[tid + o];
    __syncthreads();
  }
  if (tid == 0) a.partial[blockIdx.x] = static_cast<double>(a.E) * red[0];
}

// The mean over the sequences, in a fixed order: strided per thread, then a tree.
__global__ __launch_bounds__(kThreads) void seq_loss_final_kernel(SeqLossArgs a) {
  __shared__ double red[kThreads];
  const int tid = threadIdx.x;
  double v = 0.0;
  for (int64_t b = tid; b < a.n_seq; b += kThreads) v += a.partial[b];
  red[tid] = v;
  __syncthreads();
  for (int o = kThreads / 2; o > 0; o >>= 1) {
    if (tid < o) red[tid] += red[tid + o];
    __syncthreads();
  }
  if (tid == 0) a.loss[0] = static_cast<float>(red[0] / static_cast<double>(a.n_seq));
}

// b_i -= gamma for an overloaded expert, += gamma for an underloaded one
// (load counts[i] against the mean T*k/E, compared exactly as counts[i]*E
// against T*k), one float32 add.
__global__ __launch_bounds__(kThreads) void bias_update_kernel(const int32_t* counts, float* b, int E, int64_t Tk,
                                                               float gamma) {
  for (int e = threadIdx.x; e < E; e += kThreads) {
    const int64_t load = static_cast<int64_t>(counts[e]) * E;
    if (load < Tk) b[e] = b[e] + gamma;
    else if (load > Tk) b[e] = b[e] - gamma;
  }
}

}  // namespace

hipError_t launch_seq_loss(const SeqLossArgs& a, hipStream_t s) {
  if (a.n_seq > 0) seq_loss_kernel<<<static_cast<unsigned>(a.n_seq), kThreads, 0, s>>>(a);
  seq_loss_final_kernel<<<1, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_bias_update(const int32_t* counts, float* select_bias, int E, int64_t Tk, float gamma,
                              hipStream_t s) {
  bias_update_kernel<<<1, kThreads, 0, s>>>(counts, select_bias, E, Tk, gamma);
  return hipGetLastError();
}

}  // namespace moe
