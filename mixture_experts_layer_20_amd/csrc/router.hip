// Float32 router for gfx950: logits, softmax statistics, top-k and gates,
// plus per-workgroup partial sums for the losses.  bf16 x: the logits come
// from MFMAs on an exact bf16 split of the weight (a streaming kernel for at
// most 16 experts, the grouped GEMM beyond), then the per-token epilogue
// runs over them; float32 x: one fused pass.
//
// Sources: "Lab 18 -- Mixture of experts" s.1 (z = x W_r, p = softmax(z),
// renormalised vs raw gates) and s.2 (P_i, router z-loss); "Lab 01" "Where to
// start" 1 (subtract the max) and "The traps" (ties broken by expert index);
// "Mixture of experts" lecture field map, stability section (router in
// float32) and DeepSeek-V3 notes (sigmoid affinities, selection-only bias).
//
// float32 x layout: one 256-thread workgroup per 32 tokens.  Each thread owns one
// expert column e (= tid mod EP) and one residue class g of the model
// dimension (the quads of four consecutive d that are congruent to g mod G,
// G = 256/EP).  x is staged through LDS as float32 rows, so one 16-byte LDS
// read gives four d-values of a token for four multiply-adds against weights
// held in registers, and the router weight streams from L1/L2 once per
// workgroup.  Partial dot products of the G residue classes are summed in a
// fixed order, so the result does not depend on scheduling.
#include <algorithm>
#include <type_traits>

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
__device__ __forceinline__ float exp_key(float a) {
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

// Reductions over a group of G consecutive lanes (G a power of two <= 64):
// every exchange stays inside the group, and every lane of the group ends
// with the same bits.  Groups of 8 and 16 exchange through DPP (a VALU
// operand modifier, no LDS round trip): the 16-lane row mirror (lane i with
// 15 - i), the 8-lane half-row mirror (i with 7 - i), then the quad swaps i^2
// and i^1; each step pairs lanes symmetrically, so the partial sums of the
// two lanes of a pair are the same float additions.  Larger groups use the
// xor butterfly through the cross-lane permute.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppRowMirror = 0x140, kDppHalfMirror = 0x141;
constexpr int kDppQuadSwap2 = 2 | (3 << 2) | (0 << 4) | (1 << 6);   // quad_perm [2,3,0,1]
constexpr int kDppQuadSwap1 = 1 | (0 << 2) | (3 << 4) | (2 << 6);   // quad_perm [1,0,3,2]

template <int G>
__device__ __forceinline__ float group_max(float v) {
  if constexpr (G == 8 || G == 16) {
    if constexpr (G == 16) v = fmaxf(v, dpp_f<kDppRowMirror>(v));
    v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
    v = fmaxf(v, dpp_f<kDppQuadSwap2>(v));
    v = fmaxf(v, dpp_f<kDppQuadSwap1>(v));
  } else {
#pragma unroll
    for (int o = G / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  }
  return v;
}
template <int G>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (G == 8 || G == 16) {
    if constexpr (G == 16) v += dpp_f<kDppRowMirror>(v);
    v += dpp_f<kDppHalfMirror>(v);
    v += dpp_f<kDppQuadSwap2>(v);
    v += dpp_f<kDppQuadSwap1>(v);
  } else {
#pragma unroll
    for (int o = G / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  }
  return v;
}

// Largest 64-bit value over a group of G lanes (same lane pairing as
// group_max: DPP for 8 and 16 lanes, the xor butterfly beyond); every lane of
// the group ends with it.
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const uint32_t lo = static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(v)), CTRL, 0xF, 0xF, false));
  const uint32_t hi = static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(v >> 32)), CTRL, 0xF, 0xF, false));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}
template <int G>
__device__ __forceinline__ uint64_t group_max_u64(uint64_t v) {
  auto mx = [](uint64_t a, uint64_t b) { return a > b ? a : b; };
  if constexpr (G == 8 || G == 16) {
    if constexpr (G == 16) v = mx(v, dpp_u64<kDppRowMirror>(v));
    v = mx(v, dpp_u64<kDppHalfMirror>(v));
    v = mx(v, dpp_u64<kDppQuadSwap2>(v));
    v = mx(v, dpp_u64<kDppQuadSwap1>(v));
  } else {
#pragma unroll
    for (int o = G / 2; o > 0; o >>= 1) v = mx(v, __shfl_xor(v, o, kWave));
  }
  return v;
}

// Per-token epilogue, run by a group of G lanes (lane l of the group holds
// experts l, l + G, ...; EPL = ceil(E / G) of them): statistics, selection,
// gates.  z: LDS row of this token's logits (logit bias included).
// Selection takes k rounds: the largest remaining key of the group (a float
// max; -0 and +0 compare equal), then, by ballot, the lowest expert index
// holding it, which is the order of the pages' top-k (key descending, ties
// to the lower index).
template <int G, int EPL>
__device__ __forceinline__ void token_epilogue(const RouteArgs& a, const float* z, const float (&sbias)[EPL], int64_t t,
                               double* pacc, double& lse2acc) {
  const int lane = threadIdx.x & (kWave - 1);
  const int li = lane & (G - 1);                  // lane within the group
  const int E = a.E, k = a.k;
  float zv[EPL];
  float m = -__builtin_huge_valf();
#pragma unroll
  for (int r = 0; r < EPL; ++r) {
    const int e = li + r * G;
    zv[r] = e < E ? z[e] : -__builtin_huge_valf();
    m = fmaxf(m, zv[r]);
  }
  m = group_max<G>(m);
  float s = 0.0f;
  float ex[EPL];
#pragma unroll
  for (int r = 0; r < EPL; ++r) {
    ex[r] = (li + r * G < E) ? expf(zv[r] - m) : 0.0f;
    s += ex[r];
  }
  s = group_sum<G>(s);
  const float lse = m + logf(s);

  // selection keys (experts past E hold no key) and the full-E probabilities:
  // softmax, or the sigmoid scores normalised over all E.  The sigmoid key
  // before its bias is the float32 sigmoid, so the scores are divided by their
  // sum directly; only a token whose every score underflows (a row of logits
  // below about -87) takes the log domain (a softmax of log sigmoid).
  float key[EPL], pv[EPL];
  if (a.score == MOE_SIGMOID) {
    float qs = 0.0f;
#pragma unroll
    for (int r = 0; r < EPL; ++r) {
      key[r] = (li + r * G < E) ? sigmoid_key(zv[r]) : 0.0f;
      qs += key[r];
    }
    qs = group_sum<G>(qs);
    if (qs > 1e-30f) {
      const float inv = 1.0f / qs;
#pragma unroll
      for (int r = 0; r < EPL; ++r) pv[r] = key[r] * inv;
    } else {
      float lm = -__builtin_huge_valf();
      float ls[EPL];
#pragma unroll
      for (int r = 0; r < EPL; ++r) {
        ls[r] = (li + r * G < E) ? log_sigmoid(zv[r]) : -__builtin_huge_valf();
        lm = fmaxf(lm, ls[r]);
      }
      lm = group_max<G>(lm);
      float q2 = 0.0f;
#pragma unroll
      for (int r = 0; r < EPL; ++r) {
        pv[r] = (li + r * G < E) ? expf(ls[r] - lm) : 0.0f;
        q2 += pv[r];
      }
      q2 = group_sum<G>(q2);
      const float inv = 1.0f / q2;
#pragma unroll
      for (int r = 0; r < EPL; ++r) pv[r] *= inv;
    }
  } else {
    const float inv = 1.0f / s;
#pragma unroll
    for (int r = 0; r < EPL; ++r) {
      pv[r] = ex[r] * inv;
      key[r] = zv[r];
    }
  }

  // top-k on packed codes: order code of the key (plus any selection bias)
  // above the complement of the expert index, so the largest code is the
  // largest key and, among equal keys (-0 == +0), the lowest index; code 0
  // marks no candidate.  Each round takes the group's largest code.
  uint64_t code[EPL];
#pragma unroll
  for (int r = 0; r < EPL; ++r) {
    const int e = li + r * G;
    float kv = key[r];
    if (a.select_bias) kv = kv + sbias[r];
    code[r] = e < E ? select_code(kv, e) : 0ull;
  }
  int my_sel = -1;  // lane j < k of the group keeps the j-th choice
  for (int j = 0; j < k; ++j) {
    uint64_t best = 0;
#pragma unroll
    for (int r = 0; r < EPL; ++r) best = code[r] > best ? code[r] : best;
    best = group_max_u64<G>(best);
#pragma unroll
    for (int r = 0; r < EPL; ++r)
      if (code[r] == best) code[r] = 0;
    if (li == j) my_sel = code_expert(best);
  }

  // gates, computed by lanes 0..k-1 of the group
  const bool mine = li < k;
  const float zs = mine ? z[my_sel] : -__builtin_huge_valf();
  float g = 0.0f;
  if (a.score == MOE_SIGMOID) {
    if (a.renorm) {
      const float l = mine ? log_sigmoid(zs) : -__builtin_huge_valf();
      const float lmx = group_max<G>(l);
      const float ex = mine ? expf(l - lmx) : 0.0f;
      g = ex / group_sum<G>(ex);
    } else {
      g = mine ? 1.0f / (1.0f + expf(-zs)) : 0.0f;
    }
  } else if (a.renorm) {
    const float zmx = group_max<G>(zs);
    const float ex = mine ? expf(zs - zmx) : 0.0f;
    g = ex / group_sum<G>(ex);
  } else {
    g = mine ? expf(zs - m) / s : 0.0f;
  }
  if (mine) {
    a.idx[t * k + li] = my_sel;
    a.gates[t * k + li] = g;
  }
  if (a.lse && li == 0) a.lse[t] = lse;
#pragma unroll
  for (int r = 0; r < EPL; ++r) {
    const int e = li + r * G;
    if (e < E) {
      if (a.probs) a.probs[t * E + e] = pv[r];
      if (a.logits_out) a.logits_out[t * E + e] = zv[r];
      pacc[r] += static_cast<double>(pv[r]);
    }
  }
  if (li == 0) lse2acc += static_cast<double>(lse) * static_cast<double>(lse);
}

// Epilogue for the workgroup's tokens (zbuf row i, stride zstride): token i
// goes to group (i mod 4*TPW) of the workgroup's 4*TPW lane groups, TPW =
// 64/G groups per wavefront.  The loss partial sums of the groups are then
// combined in a fixed order.
template <int G, int EPL>
__device__ void workgroup_epilogue(const RouteArgs& a, const float* zbuf, int zstride, int64_t t0,
                                   int nt, double* red) {
  constexpr int TPW = kWave / G;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int li = lane & (G - 1), q = lane / G;
  double pacc[EPL];
#pragma unroll
  for (int r = 0; r < EPL; ++r) pacc[r] = 0.0;
  double lse2 = 0.0;
  // the selection bias of this lane's experts, read once (in registers: the
  // array goes by reference into the inlined per-token code; through a
  // pointer it lived in scratch memory)
  float sb[EPL];
#pragma unroll
  for (int r = 0; r < EPL; ++r) sb[r] = (a.select_bias && li + r * G < a.E) ? a.select_bias[li + r * G] : 0.0f;
  for (int i = wave * TPW + q; i < nt; i += (kThreads / kWave) * TPW)
    token_epilogue<G, EPL>(a, zbuf + i * zstride, sb, t0 + i, pacc, lse2);
  if (!a.p_partial) return;
  // groups of a wavefront first (xor over the group-index bits, fixed order),
  // then the four wavefronts in order
#pragma unroll
  for (int o = G; o < kWave; o <<= 1) {
#pragma unroll
    for (int r = 0; r < EPL; ++r) pacc[r] += __shfl_xor(pacc[r], o, kWave);
    lse2 += __shfl_xor(lse2, o, kWave);
  }
  __syncthreads();
  if (q == 0) {
#pragma unroll
    for (int r = 0; r < EPL; ++r) {
      const int e = li + r * G;
      if (e < a.E) red[wave * a.E + e] = pacc[r];
    }
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

template <typename XT, int GE, int EPL>
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
  workgroup_epilogue<GE, EPL>(a, red, EP, t0, nt, reinterpret_cast<double*>(xs));
}

// Routing from given logits: same epilogue, logits rows staged from memory.
template <int G, int EPL>
__global__ __launch_bounds__(kThreads) void route_from_logits_kernel(RouteArgs a) {
  __shared__ float zbuf[kBT * 256];
  __shared__ double red[5 * 256];
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kBT;
  const int nt = static_cast<int>(min<int64_t>(kBT, a.T - t0));
  // the slabs (at most 8) summed in order, then the logit bias; the slab
  // loads of four values are all issued before the first add, so the logit
  // rows of many experts take a quarter of the load round trips (up to 8
  // experts, G = 8, every thread has at most one value)
  constexpr int kU = G == 8 ? 1 : 4;
  const int64_t slab = a.T * a.E;
  const int n = nt * a.E;
  for (int i0 = threadIdx.x; i0 < n; i0 += kThreads * kU) {
    float vs[kU][8];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i = i0 + u * kThreads;
#pragma unroll
      for (int sp = 0; sp < 8; ++sp)
        vs[u][sp] = (sp < a.zsplits && i < n) ? a.logits[sp * slab + t0 * a.E + i] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i = i0 + u * kThreads;
      if (i >= n) continue;
      float v = vs[u][0];
#pragma unroll
      for (int sp = 1; sp < 8; ++sp)
        if (sp < a.zsplits) v += vs[u][sp];
      if (a.logit_bias) v += a.logit_bias[i % a.E];
      zbuf[i] = v;
    }
  }
  __syncthreads();
  workgroup_epilogue<G, EPL>(a, zbuf, a.E, t0, nt, red);
}

// ---------------------------------------------------------------- bf16 x: router on the GEMM
// The router stays float32 (x is bf16, the weight float32): the weight is
// split exactly into three bf16 planes, w = hi + mid + lo (each a bf16
// rounding of what the previous ones leave; exact for 2^-110 < |w| < 2^127),
// so every product x*hi, x*mid, x*lo is exact in the bf16 MFMA.  The planes
// are stored as the rows of a [4E, d] matrix, row 4e + p holding plane p of
// expert e (row 4e + 3 is zero), and the grouped GEMM computes x times its
// transpose with float32 accumulation; its router epilogue adds each group
// of four columns (p = 0, 1, 2, 3 in that order) into logit e.  The
// per-token epilogue then runs on those logits as for routing from logits.
// (split3, the exact three-way split, is in common.hpp.)

__global__ __launch_bounds__(kThreads) void split_router_kernel(const float* w, bf16_t* wp, int d, int E) {
  const int64_t n = static_cast<int64_t>(E) * d;
  for (int64_t i = blockIdx.x * static_cast<int64_t>(kThreads) + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * kThreads) {
    const int e = static_cast<int>(i / d), k = static_cast<int>(i % d);
    const float v = w[static_cast<int64_t>(k) * E + e];
    bf16_t hi, mid, lo;
    split3(v, hi, mid, lo);
    bf16_t* row = wp + static_cast<int64_t>(4 * e) * d + k;
    row[0] = hi;
    row[d] = mid;
    row[2 * static_cast<int64_t>(d)] = lo;
    row[3 * static_cast<int64_t>(d)] = 0;
  }
}


// ---------------------------------------------------------------- bf16 x, E <= 16
// Router logits streamed from bf16 tokens for few experts.  The grouped
// GEMM would spend a 256-row weight tile on 4E rows and wait out a load
// latency per k stage; here the token rows are the streamed operand and the
// weight planes sit in LDS.
//
// Workgroup: 16 wavefronts x 16 tokens = 256 tokens, one slice of the model
// dimension (the slices' partial logits go to separate slabs, summed in a
// fixed order by the epilogue).  The float32 weight slice is split into its
// three exact bf16 planes in LDS, 256 k at a time (rows 4e + p; p = 3 and
// rows past 4E are zero), double-buffered.  Each wave loads its tokens' x
// straight into registers in the operand layout of v_mfma_f32_16x16x32_bf16
// (lane l: token l%16, 8 consecutive k at 8*(l/16) of each 32-k step; rows
// past T and k past the slice read zero through the buffer bounds), one
// 256-k chunk ahead of the one it multiplies.  With the planes as the first
// operand, lane l ends with plane rows 4*(l/16) + {0,1,2,3} of token l%16:
// the hi, mid, lo (and zero) products of one expert, summed into its logit in
// the same order as the grouped GEMM's router epilogue.
constexpr int kLgWaves = 16;
constexpr int kLgThreads = kLgWaves * 64;
constexpr int kLgTokens = kLgWaves * 16;
constexpr int kLgSub = 256;                  // k per LDS chunk
constexpr int kLgSteps = kLgSub / 32;        // MFMA k-steps per chunk
constexpr int kLgPitch = kLgSub + 8;         // plane row pitch (bf16): rows 16 B apart in the banks
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

template <int EB>
__global__ __launch_bounds__(kLgThreads) void router_logits_kernel(RouteArgs a, int S) {
  constexpr int kRows = 16 * EB;             // plane rows 4e + p for e < 4*EB
  constexpr int kWPer = kLgSub * 4 * EB / kLgThreads;   // weights each thread splits per chunk
  static_assert(kWPer >= 1, "one weight per thread at least");
  __shared__ __align__(16) bf16_t planes[2][kRows * kLgPitch];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int E = a.E, d = a.d;
  const int64_t T = a.T;
  const int dc = d / S;                      // the slice (a multiple of 8)
  const int kbeg = blockIdx.y * dc, kend = kbeg + dc;
  const int nsub = (dc + kLgSub - 1) / kLgSub;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kLgTokens + wave * 16;

  // the float32 weights of chunk c: thread tid takes entries tid + j*threads
  // of the chunk's [256 k, E] block (contiguous in w's [d, E] layout)
  auto fetch_w = [&](float (&wv)[kWPer], int c) {
#pragma unroll
    for (int j = 0; j < kWPer; ++j) {
      const int i = tid + j * kLgThreads;
      const int kk = i / E, e = i % E;
      const int k = kbeg + c * kLgSub + kk;
      wv[j] = (kk < kLgSub && k < kend) ? a.w_router[static_cast<int64_t>(k) * E + e] : 0.0f;
    }
  };
  auto store_w = [&](const float (&wv)[kWPer], int c) {
    bf16_t* pl = planes[c & 1];
#pragma unroll
    for (int j = 0; j < kWPer; ++j) {
      const int i = tid + j * kLgThreads;
      const int kk = i / E, e = i % E;
      if (kk < kLgSub) {
        bf16_t hi, mid, lo;
        split3(wv[j], hi, mid, lo);
        pl[(4 * e) * kLgPitch + kk] = hi;
        pl[(4 * e + 1) * kLgPitch + kk] = mid;
        pl[(4 * e + 2) * kLgPitch + kk] = lo;
      }
    }
  };
  // this wave's 16 token rows through one descriptor (rows past T read zero)
  const int64_t nrows = max<int64_t>(0, min<int64_t>(16, T - t0));
  const uint64_t bu = reinterpret_cast<uint64_t>(static_cast<const bf16_t*>(a.x) + max<int64_t>(0, min(t0, T)) * d);
  const uint32_t blo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(bu));
  const uint32_t bhi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(bu >> 32));
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      reinterpret_cast<void*>((static_cast<uint64_t>(bhi) << 32) | blo), (short)0,
      __builtin_amdgcn_readfirstlane(static_cast<int>(nrows * d * 2)), 0x00020000);
  const int row = lane & 15, q = lane >> 4;
  auto fetch_x = [&](u32x4_t (&xv)[kLgSteps], int c) {
#pragma unroll
    for (int j = 0; j < kLgSteps; ++j) {
      const int k = kbeg + c * kLgSub + 32 * j + 8 * q;
      const uint32_t off = k < kend ? static_cast<uint32_t>((row * d + k) * 2) : 0x80000000u;
      xv[j] = __builtin_amdgcn_raw_buffer_load_b128(xr, static_cast<int>(off), 0, 0);
    }
  };
  f32x4_t acc[EB];
#pragma unroll
  for (int b = 0; b < EB; ++b) acc[b] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  auto multiply = [&](const u32x4_t (&xv)[kLgSteps], int c) {
    const bf16_t* pl = planes[c & 1];
#pragma unroll
    for (int j = 0; j < kLgSteps; ++j) {
      const bf16x8_t bx = __builtin_bit_cast(bf16x8_t, xv[j]);
#pragma unroll
      for (int b = 0; b < EB; ++b) {
        const bf16x8_t aw = __builtin_bit_cast(
            bf16x8_t, *reinterpret_cast<const u32x4_t*>(pl + (16 * b + row) * kLgPitch + 32 * j + 8 * q));
        acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aw, bx, acc[b], 0, 0, 0);
      }
    }
  };
  // Two chunks in flight at all times.  Loads complete in order, so each
  // chunk's weights are requested before its x, and a chunk's weights are
  // split into LDS only after the previous chunk's MFMAs (the x that wait
  // needs is the x the next MFMAs need anyway).  Plane buffer c%2 is free
  // once every wave has passed the barrier after chunk c-1's MFMAs.
  u32x4_t x0[kLgSteps], x1[kLgSteps];
  float w0[kWPer], w1[kWPer];
  fetch_w(w0, 0);
  if (nsub > 1) fetch_w(w1, 1);
  fetch_x(x0, 0);
  if (nsub > 1) fetch_x(x1, 1);
  // zero rows of both buffers (never rewritten)
  for (int i = tid; i < 2 * kRows * kLgPitch; i += kLgThreads) {
    const int r = (i / kLgPitch) % kRows;
    if ((r & 3) == 3 || (r >> 2) >= E) (&planes[0][0])[i] = 0;
  }
  store_w(w0, 0);
  if (nsub > 1) store_w(w1, 1);
  __syncthreads();
  auto step = [&](u32x4_t (&xc)[kLgSteps], float (&wc)[kWPer], const float (&wn)[kWPer], int c) {
    multiply(xc, c);
    if (c >= 1 && c + 1 < nsub) store_w(wn, c + 1);
    if (c + 2 < nsub) {
      fetch_w(wc, c + 2);
      fetch_x(xc, c + 2);
    }
    __syncthreads();
  };
  for (int c = 0; c < nsub; c += 2) {
    step(x0, w0, w1, c);
    if (c + 1 < nsub) step(x1, w1, w0, c + 1);
  }
  // lane: token t0 + row, expert 4b + q
  if (t0 + row < T) {
    float* zs = a.zraw + (static_cast<int64_t>(blockIdx.y) * T + t0 + row) * E;
#pragma unroll
    for (int b = 0; b < EB; ++b) {
      const int e = 4 * b + q;
      if (e < E) zs[e] = ((acc[b][0] + acc[b][1]) + acc[b][2]) + acc[b][3];
    }
  }
}

// calls f(integral_constant G, integral_constant EPL) for the epilogue's
// lane-group width and experts per lane
template <typename F>
void template_for_group(int E, int k, F&& f) {
  using std::integral_constant;
  if (E <= 8) { f(integral_constant<int, 8>{}, integral_constant<int, 1>{}); return; }
  if (k <= 16) {
    const int epl = (E + 15) / 16;
    if (epl <= 1) f(integral_constant<int, 16>{}, integral_constant<int, 1>{});
    else if (epl <= 2) f(integral_constant<int, 16>{}, integral_constant<int, 2>{});
    else if (epl <= 4) f(integral_constant<int, 16>{}, integral_constant<int, 4>{});
    else if (epl <= 8) f(integral_constant<int, 16>{}, integral_constant<int, 8>{});
    else f(integral_constant<int, 16>{}, integral_constant<int, 16>{});
    return;
  }
  const int epl = (E + 31) / 32;
  if (epl <= 1) f(integral_constant<int, 32>{}, integral_constant<int, 1>{});
  else if (epl <= 2) f(integral_constant<int, 32>{}, integral_constant<int, 2>{});
  else if (epl <= 4) f(integral_constant<int, 32>{}, integral_constant<int, 4>{});
  else f(integral_constant<int, 32>{}, integral_constant<int, 8>{});
}

template <typename XT>
hipError_t dispatch_route(const RouteArgs& a, hipStream_t s) {
  const unsigned grid = static_cast<unsigned>((a.T + kBT - 1) / kBT);
  RouteArgs r = a;
  if (a.x != nullptr && sizeof(XT) == 2 && a.E <= 16) {
    // few experts: the streamed router-logits kernel
    const int S = router_splits(a.T, a.E, a.d);
    const dim3 lg_grid(static_cast<unsigned>((a.T + kLgTokens - 1) / kLgTokens), static_cast<unsigned>(S));
    const int eb = (a.E + 3) / 4;
    if (eb == 1) router_logits_kernel<1><<<lg_grid, kLgThreads, 0, s>>>(a, S);
    else if (eb == 2) router_logits_kernel<2><<<lg_grid, kLgThreads, 0, s>>>(a, S);
    else if (eb == 3) router_logits_kernel<3><<<lg_grid, kLgThreads, 0, s>>>(a, S);
    else router_logits_kernel<4><<<lg_grid, kLgThreads, 0, s>>>(a, S);
    r.logits = a.zraw;
    r.zsplits = S;
  } else if (a.x != nullptr && sizeof(XT) == 2) {
    const int64_t n = static_cast<int64_t>(a.E) * a.d;
    split_router_kernel<<<static_cast<unsigned>(std::min<int64_t>(1024, (n + kThreads - 1) / kThreads)), kThreads, 0, s>>>(
        a.w_router, a.wplanes, a.d, a.E);
    // logits = x [T, d] . planes [4E, d]^T: the d range split into S parts
    // (the GEMM's groups: columns [s*dc, (s+1)*dc) of both operands, partial
    // logits to slab s), in row blocks whose part of x stays below 2^30
    // elements (the GEMM addresses an operand through one buffer descriptor)
    const int S = router_splits(a.T, a.E, a.d);
    const int dc = a.d / S;
    const int64_t max_rows = ((int64_t{1} << 30) - 1) / a.d / 256 * 256;
    for (int64_t r0 = 0; r0 < a.T; r0 += max_rows) {
      GemmArgs g{};
      g.A = static_cast<const bf16_t*>(a.x) + r0 * a.d;
      g.B0 = a.wplanes;
      g.C = a.zraw + r0 * a.E;
      g.rows_per_group = std::min<int64_t>(max_rows, a.T - r0);
      g.groups = S;
      g.N = 4 * a.E;
      g.K = dc;
      g.lda = a.d;
      g.ldb = a.d;
      g.a_gs = dc;
      g.b_gs = dc;
      g.c_gs = a.T * a.E;
      g.act = 3;
      const hipError_t e = launch_gemm(g, MOE_BF16, s);
      if (e != hipSuccess) return e;
    }
    r.logits = a.zraw;
    r.zsplits = S;
  }
  // per-token epilogue: one token per group of G lanes, EPL experts per lane.
  // Small groups let one wavefront instruction serve several tokens and
  // shorten every reduction: G = 8 for E <= 8, else 16 (32 when k > 16,
  // since lanes j < k of a group hold the choices).
  auto launch = [&](auto g_c, auto epl_c) {
    constexpr int G = decltype(g_c)::value, EPL = decltype(epl_c)::value;
    if (r.x == nullptr || sizeof(XT) == 2) route_from_logits_kernel<G, EPL><<<grid, kThreads, 0, s>>>(r);
    else route_kernel<XT, G, EPL><<<grid, kThreads, 0, s>>>(r);
  };
  template_for_group(a.E, a.k, launch);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const RouteArgs& a, int dtype, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  return dtype == MOE_BF16 ? dispatch_route<bf16_t>(a, s) : dispatch_route<float>(a, s);
}

}  // namespace moe
