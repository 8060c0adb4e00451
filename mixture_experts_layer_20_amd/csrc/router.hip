// Fused float32 router for gfx950: logits, softmax statistics, top-k and
// gates in one pass over x, plus per-workgroup partial sums for the losses.
//
// Sources: "Lab 18 -- Mixture of experts" s.1 (z = x W_r, p = softmax(z),
// renormalised vs raw gates) and s.2 (P_i, router z-loss); "Lab 01" "Where to
// start" 1 (subtract the max) and "The traps" (ties broken by expert index);
// "Mixture of experts" lecture field map, stability section (router in
// float32) and DeepSeek-V3 notes (sigmoid affinities, selection-only bias).
//
// Layout: one 256-thread workgroup per 32 tokens.  Each thread owns one
// expert column e (= tid mod EP) and one residue class g of the model
// dimension (the quads of four consecutive d that are congruent to g mod G,
// G = 256/EP).  x is staged through LDS as float32 rows, so one 16-byte LDS
// read gives four d-values of a token for four multiply-adds against weights
// held in registers, and the router weight streams from L1/L2 once per
// workgroup.  Partial dot products of the G residue classes are summed in a
// fixed order, so the result does not depend on scheduling.
#include "common.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kBT = kRouteTokens;    // 32 tokens per workgroup
constexpr int kDC = 128;             // model-dimension chunk staged per step

// ---------------------------------------------------------------- float32 sigmoid key
// The selection key of sigmoid scoring must be one fixed sequence of IEEE
// float32 operations so that routing is reproducible bit for bit: Cody &
// Waite reduction r = (a - n*LN2_HI) - n*LN2_LO with n = rint(a/ln 2), the
// degree-7 Taylor polynomial of exp(r) by Horner, scaling by 2^n, then
// 1/(1 + exp(-z)) with IEEE division.  LN2_HI is ln 2 cut to 16 significant
// bits so n*LN2_HI is exact.  No contraction into fused multiply-adds.
__device__ __noinline__ float exp_key(float a) {
#pragma clang fp contract(off)
  const float kInvLn2 = static_cast<float>(1.0 / 0.6931471805599453094172321);
  const float kLn2Hi = 0.693145751953125f;
  const float kLn2Lo = static_cast<float>(0.6931471805599453094172321 - 0.693145751953125);
  if (a > 88.0f) return __builtin_huge_valf();
  if (a < -87.0f) return 0.0f;
  const float n = __builtin_rintf(a * kInvLn2);
  const float r = (a - n * kLn2Hi) - n * kLn2Lo;
  float p = static_cast<float>(1.0 / 5040.0);
  p = p * r + static_cast<float>(1.0 / 720.0);
  p = p * r + static_cast<float>(1.0 / 120.0);
  p = p * r + static_cast<float>(1.0 / 24.0);
  p = p * r + static_cast<float>(1.0 / 6.0);
  p = p * r + 0.5f;
  p = p * r + 1.0f;
  p = p * r + 1.0f;
  return __builtin_ldexpf(p, static_cast<int>(n));
}

__device__ __forceinline__ float sigmoid_key(float z) {
#pragma clang fp contract(off)
  const float e = exp_key(-z);
  return 1.0f / (1.0f + e);
}

// log(sigmoid(z)) = -softplus(-z), stable at any magnitude (gate maths only).
__device__ __forceinline__ float log_sigmoid(float z) {
  const float t = log1pf(expf(-fabsf(z)));
  return z >= 0.0f ? -t : z - t;
}

// Per-token epilogue, run by one wavefront: statistics, selection, gates.
// z: LDS row of this token's logits (logit bias included), E entries.
template <int EPL>
__device__ void token_epilogue(const RouteArgs& a, const float* z, int64_t t, double* pacc,
                               double& lse2acc) {
  const int lane = threadIdx.x & (kWave - 1);
  const int E = a.E, k = a.k;
  float zv[EPL];
  float m = -__builtin_huge_valf();
#pragma unroll
  for (int r = 0; r < EPL; ++r) {
    const int e = lane + r * kWave;
    zv[r] = e < E ? z[e] : -__builtin_huge_valf();
    m = fmaxf(m, zv[r]);
  }
  m = wave_max(m);
  float s = 0.0f;
#pragma unroll
  for (int r = 0; r < EPL; ++r) s += (lane + r * kWave < E) ? expf(zv[r] - m) : 0.0f;
  s = wave_sum(s);
  const float lse = m + logf(s);

  // full-E probabilities (softmax) or normalised sigmoid scores (log domain)
  float pv[EPL];
  if (a.score == MOE_SIGMOID) {
    float lm = -__builtin_huge_valf();
    float ls[EPL];
#pragma unroll
    for (int r = 0; r < EPL; ++r) {
      ls[r] = (lane + r * kWave < E) ? log_sigmoid(zv[r]) : -__builtin_huge_valf();
      lm = fmaxf(lm, ls[r]);
    }
    lm = wave_max(lm);
    float qs = 0.0f;
#pragma unroll
    for (int r = 0; r < EPL; ++r) {
      pv[r] = (lane + r * kWave < E) ? expf(ls[r] - lm) : 0.0f;
      qs += pv[r];
    }
    qs = wave_sum(qs);
    const float inv = 1.0f / qs;
#pragma unroll
    for (int r = 0; r < EPL; ++r) pv[r] *= inv;
  } else {
    const float inv = 1.0f / s;
#pragma unroll
    for (int r = 0; r < EPL; ++r) pv[r] = (lane + r * kWave < E) ? expf(zv[r] - m) * inv : 0.0f;
  }

  // selection codes
  uint64_t code[EPL];
#pragma unroll
  for (int r = 0; r < EPL; ++r) {
    const int e = lane + r * kWave;
    if (e < E) {
      float key = a.score == MOE_SIGMOID ? sigmoid_key(zv[r]) : zv[r];
      if (a.select_bias) key = key + a.select_bias[e];
      code[r] = select_code(key, e);
    } else {
      code[r] = 0;
    }
  }
  int my_sel = -1;  // lane j < k keeps the j-th choice
  for (int j = 0; j < k; ++j) {
    uint64_t best = 0;
#pragma unroll
    for (int r = 0; r < EPL; ++r) best = code[r] > best ? code[r] : best;
    best = wave_max_u64(best);
    const int e = code_expert(best);
#pragma unroll
    for (int r = 0; r < EPL; ++r)
      if (lane + r * kWave == e) code[r] = 0;
    if (lane == j) my_sel = e;
  }

  // gates, computed by lanes 0..k-1
  const bool mine = lane < k;
  const float zs = mine ? z[my_sel] : -__builtin_huge_valf();
  float g = 0.0f;
  if (a.score == MOE_SIGMOID) {
    if (a.renorm) {
      const float l = mine ? log_sigmoid(zs) : -__builtin_huge_valf();
      const float lmx = wave_max(l);
      const float ex = mine ? expf(l - lmx) : 0.0f;
      g = ex / wave_sum(ex);
    } else {
      g = mine ? 1.0f / (1.0f + expf(-zs)) : 0.0f;
    }
  } else if (a.renorm) {
    const float zmx = wave_max(zs);
    const float ex = mine ? expf(zs - zmx) : 0.0f;
    g = ex / wave_sum(ex);
  } else {
    g = mine ? expf(zs - m) / s : 0.0f;
  }
  if (mine) {
    a.idx[t * k + lane] = my_sel;
    a.gates[t * k + lane] = g;
  }
  if (a.lse && lane == 0) a.lse[t] = lse;
#pragma unroll
  for (int r = 0; r < EPL; ++r) {
    const int e = lane + r * kWave;
    if (e < E) {
      if (a.probs) a.probs[t * E + e] = pv[r];
      if (a.x && a.logits) a.logits[t * E + e] = zv[r];
      pacc[r] += static_cast<double>(pv[r]);
    }
  }
  lse2acc += static_cast<double>(lse) * static_cast<double>(lse);
}

// Epilogue for the workgroup's tokens; zrow(t) gives the LDS logits row.
template <int EPL>
__device__ void workgroup_epilogue(const RouteArgs& a, const float* zbuf, int zstride, int64_t t0,
                                   int nt, double* red) {
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  double pacc[EPL];
#pragma unroll
  for (int r = 0; r < EPL; ++r) pacc[r] = 0.0;
  double lse2 = 0.0;
  for (int i = wave; i < nt; i += kThreads / kWave)
    token_epilogue<EPL>(a, zbuf + i * zstride, t0 + i, pacc, lse2);
  if (!a.p_partial) return;
  // fixed-order combination of the four wavefronts' partial sums
  __syncthreads();
#pragma unroll
  for (int r = 0; r < EPL; ++r) {
    const int e = lane + r * kWave;
    if (e < a.E) red[wave * a.E + e] = pacc[r];
  }
  if (lane == 0) red[4 * a.E + wave] = lse2;
  __syncthreads();
  for (int e = threadIdx.x; e < a.E; e += kThreads) {
    double v = 0.0;
    for (int w = 0; w < kThreads / kWave; ++w) v += red[w * a.E + e];
    a.p_partial[static_cast<int64_t>(blockIdx.x) * a.E + e] = v;
  }
  if (threadIdx.x == 0) {
    double v = 0.0;
    for (int w = 0; w < kThreads / kWave; ++w) v += red[4 * a.E + w];
    a.lse2_partial[blockIdx.x] = v;
  }
}

// LDS: the x chunk [32 tokens][kDC (+4 pad)] as float32, and the
// cross-thread reduction buffer [G][32][EP] which then holds the logits rows
// (stride EP, in place of the g = 0 slice); the x buffer is reused for the
// fixed-order combination of the loss partial sums.
constexpr int kXRow = kDC + 4;
constexpr int kXsFloats = kBT * kXRow;                 // 4224 floats
constexpr int kRedFloats = kThreads * kBT;             // 8192 floats (G*EP*BT)

template <typename XT, int EPL>
__global__ __launch_bounds__(kThreads) void route_kernel(RouteArgs a) {
  __shared__ __align__(16) float xs[kXsFloats];
  __shared__ __align__(16) float red[kRedFloats];
  const int tid = threadIdx.x;
  const int E = a.E, d = a.d;
  int EP = 1;
  while (EP < E) EP <<= 1;
  const int G = kThreads / EP;
  const int e = tid % EP, g = tid / EP;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kBT;
  const int nt = static_cast<int>(min<int64_t>(kBT, a.T - t0));
  const XT* x = static_cast<const XT*>(a.x);

  float acc[kBT];
#pragma unroll
  for (int i = 0; i < kBT; ++i) acc[i] = 0.0f;

  constexpr int kVec = 16 / sizeof(XT);                // elements per 16-byte load
  constexpr int kVecPerRow = kDC / kVec;
  for (int c0 = 0; c0 < d; c0 += kDC) {
    const int dc = min(kDC, d - c0);
    __syncthreads();
    // stage x[t0..t0+32, c0..c0+dc) as float32 rows
    for (int v = tid; v < kBT * kVecPerRow; v += kThreads) {
      const int tt = v / kVecPerRow, dd = (v % kVecPerRow) * kVec;
      float vals[kVec];
      if (tt < nt && dd < dc) {
        const XT* src = x + (t0 + tt) * static_cast<int64_t>(d) + c0 + dd;
        if constexpr (sizeof(XT) == 2) {
          const uint4 raw = *reinterpret_cast<const uint4*>(src);
          const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            vals[2 * q] = __uint_as_float(w4[q] << 16);
            vals[2 * q + 1] = __uint_as_float(w4[q] & 0xFFFF0000u);
          }
        } else {
          const float4 raw = *reinterpret_cast<const float4*>(src);
          vals[0] = raw.x; vals[1] = raw.y; vals[2] = raw.z; vals[3] = raw.w;
        }
      } else {
#pragma unroll
        for (int q = 0; q < kVec; ++q) vals[q] = 0.0f;
      }
      float4* dst = reinterpret_cast<float4*>(xs + tt * kXRow + dd);
#pragma unroll
      for (int q = 0; q < kVec / 4; ++q)
        dst[q] = make_float4(vals[4 * q], vals[4 * q + 1], vals[4 * q + 2], vals[4 * q + 3]);
    }
    __syncthreads();
    if (e < E) {
      // residue class g owns the quads dq = 4g, 4g + 4G, ... of the chunk
      const float* wcol = a.w_router + static_cast<int64_t>(c0) * E + e;
      for (int dq = 4 * g; dq < dc; dq += 4 * G) {
        const float w0 = wcol[static_cast<int64_t>(dq + 0) * E];
        const float w1 = wcol[static_cast<int64_t>(dq + 1) * E];
        const float w2 = wcol[static_cast<int64_t>(dq + 2) * E];
        const float w3 = wcol[static_cast<int64_t>(dq + 3) * E];
#pragma unroll
        for (int i = 0; i < kBT; ++i) {
          const float4 xv = *reinterpret_cast<const float4*>(xs + i * kXRow + dq);
          float s = acc[i];
          s += xv.x * w0;
          s += xv.y * w1;
          s += xv.z * w2;
          s += xv.w * w3;
          acc[i] = s;
        }
      }
    }
  }
  // sum the G residue classes in a fixed order; the logits land in the g = 0
  // slice: zrow(t)[e] = red[t*EP + e]
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kBT; ++i) red[(g * kBT + i) * EP + e] = acc[i];
  __syncthreads();
  for (int i = tid; i < kBT * EP; i += kThreads) {
    const int tt = i / EP, ee = i % EP;
    if (ee >= E) continue;
    float v = 0.0f;
    for (int gg = 0; gg < G; ++gg) v += red[(gg * kBT + tt) * EP + ee];
    if (a.logit_bias) v += a.logit_bias[ee];
    red[tt * EP + ee] = v;
  }
  __syncthreads();
  workgroup_epilogue<EPL>(a, red, EP, t0, nt, reinterpret_cast<double*>(xs));
}

// Routing from given logits: same epilogue, logits rows staged from memory.
template <int EPL>
__global__ __launch_bounds__(kThreads) void route_from_logits_kernel(RouteArgs a) {
  __shared__ float zbuf[kBT * 256];
  __shared__ double red[5 * 256];
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kBT;
  const int nt = static_cast<int>(min<int64_t>(kBT, a.T - t0));
  for (int i = threadIdx.x; i < nt * a.E; i += kThreads) {
    float v = a.logits[t0 * a.E + i];
    if (a.logit_bias) v += a.logit_bias[i % a.E];
    zbuf[i] = v;
  }
  __syncthreads();
  workgroup_epilogue<EPL>(a, zbuf, a.E, t0, nt, red);
}

// ---------------------------------------------------------------- bf16 x: MFMA router
// The router stays float32 (x is bf16, the weight float32): the weight is
// split exactly into three bf16 planes, w = hi + mid + lo (each a bf16
// rounding of what the previous ones leave; exact for 2^-110 < |w| < 2^127),
// so every product x*hi, x*mid, x*lo is exact in the MFMA and only the
// float32 accumulation order differs from a plain float32 dot product.
// Planes are stored transposed, [3][Ep][d] (Ep = E rounded up to 16), so an
// MFMA operand fragment is one 16-byte load.
typedef __bf16 bf16x8_r __attribute__((ext_vector_type(8)));
typedef float f32x4_r __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void split_router_kernel(const float* w, bf16_t* wt, int d, int E, int Ep) {
  const int64_t n = static_cast<int64_t>(Ep) * d;
  for (int64_t i = blockIdx.x * static_cast<int64_t>(kThreads) + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * kThreads) {
    const int e = static_cast<int>(i / d), k = static_cast<int>(i % d);
    const float v = e < E ? w[static_cast<int64_t>(k) * E + e] : 0.0f;
    const bf16_t hi = f32_to_bf16(v);
    const float r1 = v - bf16_to_f32(hi);
    const bf16_t mid = f32_to_bf16(r1);
    const bf16_t lo = f32_to_bf16(r1 - bf16_to_f32(mid));
    wt[i] = hi;
    wt[n + i] = mid;
    wt[2 * n + i] = lo;
  }
}

// One workgroup: TB tokens x all experts.  The d-range is dealt to the four
// wavefronts in 32-wide chunks (chunk c to wave c % 4); each computes partial
// logits with v_mfma_f32_16x16x32_bf16 (tokens as rows, experts as columns),
// x fragments loaded straight from memory U chunks ahead.  The four partial
// tiles are added in wave order in LDS (deterministic), then the shared
// per-token epilogue runs.
template <int TB, int NB, int U>
__global__ __launch_bounds__(kThreads) void route_mfma_kernel(RouteArgs a) {
  constexpr int MB = TB / 16;
  constexpr int EPAD = NB * 16;
  constexpr int EPL = (EPAD + kWave - 1) / kWave;
  __shared__ __align__(16) float zbuf[TB * EPAD];
  __shared__ double red[5 * 256];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int d = a.d;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * TB;
  const int nt = static_cast<int>(min<int64_t>(TB, a.T - t0));
  const bf16_t* x = static_cast<const bf16_t*>(a.x);
  const bf16_t* wt = a.wsplit;
  const int64_t plane = static_cast<int64_t>(EPAD) * d;
  const int koff = 8 * (lane >> 4);
  const bf16_t* xrow[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int64_t t = min<int64_t>(t0 + mb * 16 + (lane & 15), a.T - 1);
    xrow[mb] = x + t * d + koff;
  }
  const bf16_t* wrow[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) wrow[nb] = wt + static_cast<int64_t>(nb * 16 + (lane & 15)) * d + koff;

  f32x4_r acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = f32x4_r{0.0f, 0.0f, 0.0f, 0.0f};

  const int nchunks = (d + 31) / 32;
  for (int c0 = wave; c0 < nchunks; c0 += 4 * U) {
    // all loads of the batch first (x from HBM, weight planes from L2), then
    // the MFMAs, so one batch costs about one memory latency
    bf16x8_r af[U][MB], bw[U][NB][3];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = (c0 + 4 * u) * 32;
      const bool ok = (c0 + 4 * u) < nchunks && k + koff < d;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        af[u][mb] = ok ? __builtin_bit_cast(bf16x8_r, *reinterpret_cast<const uint4*>(xrow[mb] + k))
                       : __builtin_bit_cast(bf16x8_r, make_uint4(0, 0, 0, 0));
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int sp = 0; sp < 3; ++sp)
          bw[u][nb][sp] = ok ? __builtin_bit_cast(bf16x8_r, *reinterpret_cast<const uint4*>(wrow[nb] + sp * plane + k))
                             : __builtin_bit_cast(bf16x8_r, make_uint4(0, 0, 0, 0));
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int sp = 0; sp < 3; ++sp)
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[u][mb], bw[u][nb][sp], acc[mb][nb], 0, 0, 0);
  }
  // add the four partial tiles in wave order (logit bias first)
  for (int w = 0; w < 4; ++w) {
    if (wave == w) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int tl = mb * 16 + 4 * (lane >> 4) + r;
            const int e = nb * 16 + (lane & 15);
            float base;
            if (w == 0) base = (a.logit_bias && e < a.E) ? a.logit_bias[e] : 0.0f;
            else base = zbuf[tl * EPAD + e];
            zbuf[tl * EPAD + e] = base + acc[mb][nb][r];
          }
    }
    __syncthreads();
  }
  workgroup_epilogue<EPL>(a, zbuf, EPAD, t0, nt, red);
}

template <typename XT>
hipError_t dispatch_route(const RouteArgs& a, hipStream_t s) {
  const unsigned grid = static_cast<unsigned>((a.T + kBT - 1) / kBT);
  const int epl = (a.E + kWave - 1) / kWave;
  if (a.x != nullptr && sizeof(XT) == 2) {
    const int ep = (a.E + 15) / 16 * 16;
    split_router_kernel<<<min(1024, (ep * a.d + kThreads - 1) / kThreads), kThreads, 0, s>>>(
        a.w_router, a.wsplit, a.d, a.E, ep);
    const int tb = route_tile_tokens(a.E, MOE_BF16, true);
    const unsigned g = static_cast<unsigned>((a.T + tb - 1) / tb);
    // tile tokens x expert blocks x chunks per batch: sized so one batch's
    // fragments fit in registers beside the accumulators
    if (a.E <= 16) route_mfma_kernel<16, 1, 8><<<g, kThreads, 0, s>>>(a);
    else if (a.E <= 32) route_mfma_kernel<16, 2, 4><<<g, kThreads, 0, s>>>(a);
    else if (a.E <= 64) route_mfma_kernel<32, 4, 2><<<g, kThreads, 0, s>>>(a);
    else if (a.E <= 128) route_mfma_kernel<64, 8, 1><<<g, kThreads, 0, s>>>(a);
    else route_mfma_kernel<32, 16, 1><<<g, kThreads, 0, s>>>(a);
    return hipGetLastError();
  }
  if (a.x == nullptr) {
    switch (epl) {
      case 1: route_from_logits_kernel<1><<<grid, kThreads, 0, s>>>(a); break;
      case 2: route_from_logits_kernel<2><<<grid, kThreads, 0, s>>>(a); break;
      default: route_from_logits_kernel<4><<<grid, kThreads, 0, s>>>(a); break;
    }
  } else {
    switch (epl) {
      case 1: route_kernel<XT, 1><<<grid, kThreads, 0, s>>>(a); break;
      case 2: route_kernel<XT, 2><<<grid, kThreads, 0, s>>>(a); break;
      default: route_kernel<XT, 4><<<grid, kThreads, 0, s>>>(a); break;
    }
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const RouteArgs& a, int dtype, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  return dtype == MOE_BF16 ? dispatch_route<bf16_t>(a, s) : dispatch_route<float>(a, s);
}

}  // namespace moe
