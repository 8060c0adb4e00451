// Shared device helpers for the gfx950 MoE kernels: bf16 storage, wave-64
// reductions, and the internal launch descriptors.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

constexpr int kWave = 64;            // CDNA wavefront width
constexpr int kTileTokens = 64;      // tokens per capacity tile (one wavefront)

using bf16_t = uint16_t;             // raw bf16 bits in memory

__device__ __forceinline__ float bf16_to_f32(bf16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// float32 -> bf16, round to nearest even (inputs here are finite).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

// The exact three-way bf16 split of a float32 value: hi + mid + lo == v
// (8 + 8 + 8 significant bits cover float32's 24), so each product of a bf16
// value with a plane is exact in the bf16 matrix cores.
__device__ __forceinline__ void split3(float v, bf16_t& hi, bf16_t& mid, bf16_t& lo) {
#pragma clang fp contract(off)
  hi = f32_to_bf16(v);
  const float r1 = v - bf16_to_f32(hi);
  mid = f32_to_bf16(r1);
  lo = f32_to_bf16(r1 - bf16_to_f32(mid));
}

// The standard normal tail Q(|v|) = 0.5 erfc(|v| / sqrt(2)) for the bf16
// GELU paths, from Hastings' approximation as tabulated by Abramowitz &
// Stegun (formula 7.1.26: erfc(z) = (a1 t + ... + a5 t^5) exp(-z^2),
// t = 1 / (1 + p z), absolute error at most 1.5e-7), evaluated with the
// hardware reciprocal and exp2; also returns e = exp(-v^2 / 2), so that
// Phi(v) = v >= 0 ? 1 - Q : Q and phi(v) = e / sqrt(2 pi).
__device__ __forceinline__ float normal_tail(float v, float& e) {
  const float z = fabsf(v) * 0.70710678118654752440f;
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, z, 1.0f));
  float y = fmaf(1.061405429f, t, -1.453152027f);
  y = fmaf(y, t, 1.421413741f);
  y = fmaf(y, t, -0.284496736f);
  y = fmaf(y, t, 0.254829592f);
  // exp(-v^2 / 2) = 2^(-v^2 log2(e) / 2)
  e = __builtin_amdgcn_exp2f(v * v * -0.72134752044448170368f);
  return 0.5f * (y * t) * e;
}

template <typename T> struct Storage;
template <> struct Storage<float> {
  __device__ static __forceinline__ float load(const float* p, int64_t i) { return p[i]; }
  __device__ static __forceinline__ void store(float* p, int64_t i, float v) { p[i] = v; }
};
template <> struct Storage<bf16_t> {
  __device__ static __forceinline__ float load(const bf16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
  __device__ static __forceinline__ void store(bf16_t* p, int64_t i, float v) { p[i] = f32_to_bf16(v); }
};

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    uint64_t w = __shfl_xor(v, o, kWave);
    v = w > v ? w : v;
  }
  return v;
}

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = threadIdx.x & (kWave - 1);
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Monotone map of a float32 key to uint32 (larger key -> larger code);
// -0 is first folded to +0 so that the two compare equal.
__device__ __forceinline__ uint32_t order_code(float key) {
  uint32_t b = __float_as_uint(key);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
// Packed selection code: key first, then the LOWER expert index wins a tie.
__device__ __forceinline__ uint64_t select_code(float key, int e) {
  return (static_cast<uint64_t>(order_code(key)) << 32) | static_cast<uint32_t>(~static_cast<uint32_t>(e));
}
__device__ __forceinline__ int code_expert(uint64_t c) {
  return static_cast<int>(~static_cast<uint32_t>(c & 0xFFFFFFFFull));
}

// ---------------------------------------------------------------- descriptors
struct RouteArgs {
  const void* x;              // [T,d] or null (logits given)
  const float* w_router;      // [d,E]
  const float* logit_bias;    // [E] | null
  const float* select_bias;   // [E] | null
  float* logits;              // [zsplits,T,E] logits in, summed over the slabs | null
  int zsplits;                // slabs of `logits` (routing from given logits: 1)
  float* logits_out;          // [T,E] logits out (logit bias included) | null
  float* probs;               // [T,E] | null
  int32_t* idx;               // [T,k]
  float* gates;               // [T,k]
  float* lse;                 // [T] | null
  double* p_partial;          // [n_rtiles, E] | null
  double* lse2_partial;       // [n_rtiles] | null
  bf16_t* wplanes;            // [4E, d] router weight split in bf16 planes (bf16 x)
  float* zraw;                // [S,T,E] partial logits, one slab per split of d (bf16 x)
  int64_t T;
  int d, E, k;
  int score;                  // moe_score
  int renorm;                 // resolved: 0 / 1
};

struct CapArgs {
  const int32_t* idx;         // [T,k]
  int32_t* hist;              // [k, n_tiles, E]: counts, then exclusive offsets
  int32_t* counts;            // [E]
  int32_t* kept;              // [E] min(counts, C) | null
  int32_t* slot;              // [T,k]
  uint8_t* dropped;           // [T,k]
  int32_t* row_token;         // [E,C] | null
  int32_t* fallback_partial;  // [n_tiles] | null
  const void* x;              // [T,d] | null
  void* xe;                   // [E,C,d] | null
  const double* p_partial;    // [n_rtiles, E] router partial sums of P_i | null
  const double* lse2_partial; // [n_rtiles] | null
  double* psum;               // [E + 1]: sum_t P_ti per expert, then sum_t LSE_t^2
  int64_t T, C;
  int E, k, d, n_tiles, n_rtiles;
  int token_major;
  int packed;                 // dropless: slot = packed row off_e + queue position,
                              // row_token [T*k], xe [T*k, d]; nothing dropped
};

struct GemmArgs {
  const void* A;              // [groups*rows_per_group, K], or [a_rows, K] when gathered
  const int32_t* gather;      // [groups*rows_per_group] row of A for each (group, row) | null
  int64_t a_rows;             // rows of A when gathered
  const void* B0;             // [groups, N, K]
  const void* B1;             // [groups, N, K] (SwiGLU gate) | null
  const void* bias;           // [groups, N] | null
  void* C;                    // [groups*rows_per_group, N]
  const int32_t* rows;        // [groups] | null
  int64_t rows_per_group;
  int groups, N, K;
  // bf16 path only: row strides of A and B0/B1 and per-group offsets, in
  // elements (0: rows of K elements, groups stacked contiguously)
  int64_t lda, ldb;
  int64_t a_gs, b_gs, c_gs;
  int packed;                 // group g's rows start at rows[0] + ... + rows[g-1] of A
                              // (or of gather) and C; rows required (bf16 path:
                              // the launch covers total_rows)
  int64_t total_rows;         // packed: upper bound of the sum of rows
  int act;                    // 0 none (bias only), 1 GELU, 2 SwiGLU (B1 = gate),
                              // 3 router planes: float32 C [rows, N/4], the sum of
                              // each group of 4 output columns
  // bf16 path, ACT 1/2: the pre-activations too, laid out like C (kept for a
  // backward pass): pre0 = A B0^T + bias (GELU) or the gate projection
  // (SwiGLU), pre1 = the up projection (SwiGLU) | null
  void* pre0;
  void* pre1;
  // bf16 path, ACT 0, not packed: split the k range into ksplit parts of
  // kslice (a multiple of 64), float32 partial sums in kpart [ksplit,
  // groups*rows_per_group, N] (kpart_stride elements apart), then summed in
  // part order with the bias into C.  ksplit <= 1: no split.
  int ksplit;
  int64_t kslice;
  float* kpart;
  int64_t kpart_stride;
  // bf16 path, not packed: group g contracts over its first kvar[g] k only
  // (rounded up to 8, at least 8; the operands must be zero from there to the
  // rounded extent), e.g. a weight gradient over an expert's kept rows | null
  const int32_t* kvar;
  // bf16 path, ACT 0-2, device row counts (rows; slabs or packed), no
  // ksplit: a float32 workspace of 256 partial tiles of 256 x 256, in which the tiles
  // of a last, at most half-full round of the GPU are split along k into at
  // most tail_parts parts and then summed in part order | null (no split)
  float* tail_part;
  int tail_parts;
  // bf16 path, with kvar: the operands are per-group blocks packed one
  // after another (e.g. transposed expert rows): group g's A is the
  // [rows_per_group, K_g] block at A + koff[g]*rows_per_group and its B the
  // [N, K_g] block at B0 + koff[g]*N, both with row stride K_g (its kvar
  // extent, rounded up to 8, at least 8) | null
  const int32_t* koff;
  // bf16 path, ACT 0, not packed; no gather, ksplit, tail split or koff:
  // operands stored k-major, as [K, rows] matrices with their rows
  // contiguous, which the kernel reads through the LDS transpose loads
  // instead of a transposed copy.  kmaj bit 0: element (m, k) of group g's A
  // is A[off_g + k * lda + m]; bit 1: element (n, k) of its B is
  // B0[off_g + k * ldb + n], or with B1, for k >= b_split, B1[off_g +
  // (k - b_split) * ldb + n] (two matrices stacked along k; b_split a
  // multiple of 64).  off_g = kstart[g] * ld when kstart is given (packed
  // rows), else g * a_gs (A) or g * b_gs (B).  With kvar the k-major
  // operands are read up to kvar[g] exactly (zeros past it, whatever the
  // memory holds).  0: both operands K-contiguous.
  int kmaj;
  int64_t b_split;
  const int32_t* kstart;
};
// bytes of the tail-split workspace (GemmArgs.tail_part)
constexpr size_t kTailPartBytes = size_t{256} * 256 * 256 * sizeof(float);

struct CombineArgs {
  const void* x;              // [T,d]
  const void* ye;             // [E,C,d]
  const void* shared_out;     // [T,d] | null
  const int32_t* idx;
  const float* gates;
  const int32_t* slot;
  const uint8_t* dropped;
  void* y;                    // [T,d]
  int64_t T, C;
  int d, k, E;
  int zero_fallback;
  int packed;                 // dropless: ye is [T*k, d] and slot the row
  // expert choice (sel != null): the picks of token t are the experts e with
  // sel[t*E + e] >= 0, in e order, row e*C + sel, gate probs[t*E + e];
  // idx, gates, slot and dropped are then not read
  const int32_t* sel;         // [T,E] | null
  const float* probs;         // [T,E] (expert choice)
  int32_t* fallback_count;    // [1] tokens that took the fallback, added to | null
};

struct LossArgs {
  const double* psum;         // [E + 1] from the capacity scan
  const int32_t* counts;      // [E]
  const int32_t* fallback_partial;  // [n_tiles] | null
  float* losses;              // [2]
  int32_t* stats;             // [4] | null
  int64_t T, C;
  int E, k, n_tiles;
  int has_shared;
  int packed;                 // dropless: no padding in the statistics
  int ec;                     // expert choice: f_i = counts_i / sum counts, no drops,
                              // fallback tokens from fallback_count
  const int32_t* fallback_count;  // [1] (expert choice)
};

struct EcArgs {
  const float* probs;         // [T,E] router probabilities
  uint32_t* keys;             // [E,T] order codes (workspace)
  int32_t* row_token;         // [E,C] picked tokens, ascending, first min(C,T) rows
  int32_t* selT;              // [E,T] the same, expert-major (workspace)
  int32_t* sel;               // [T,E] slot of t in e, or -1
  int32_t* counts;            // [E] = min(C,T)
  const double* p_partial;    // [n_rtiles, E] router partial sums | null
  const double* lse2_partial; // [n_rtiles]
  double* psum;               // [E + 1]
  int32_t* fallback_count;    // [1] zeroed here (the combine adds to it) | null
  // selection over lists of different lengths (batch-prioritised capacity):
  // expert e's entries are keys[e*T + 0 .. lengths[e]); counts and row_token
  // are then not written
  const int32_t* lengths;     // [E] | null (every list T long)
  int keep_before;            // entries not taken store -(taken entries before them) - 1
  int64_t T, C;
  int E, n_rtiles;
};

struct ScoreArgs {
  const int32_t* idx;         // [T,k]
  const float* gates;         // [T,k] the scores
  const int32_t* queue;       // [T,k] rank-major queue position (room for all)
  const int32_t* counts;      // [E]
  uint32_t* keys;             // [E,T] workspace
  int32_t* selT;              // [E,T] workspace
  int32_t* slot;              // [T,k]
  uint8_t* dropped;           // [T,k]
  int32_t* row_token;         // [E,C] | null
  int32_t* kept;              // [E] min(counts, C)
  int32_t* fallback_partial;  // [n_tiles] | null
  int64_t T, C;
  int E, k, n_tiles;
};

// Backward pass (token choice, capacity mode, bf16 storage)
struct TransposeArgs {
  const bf16_t* in;           // rows of ld_in elements
  bf16_t* out;                // out[g*out_gs + c*ld_out + r], or packed: group g's block
                              // [Cc][n_g] at out + ocol[g]*Cc, n_g = max(8, round8(valid[g]))
  const int32_t* gather;      // [..] source row of (g, r): gather[g*gather_gs + r] or
                              // gather[gstart[g] + r] | null
  const int32_t* valid;       // [G] rows read per group (the rest zero) | null: R
  const int32_t* ocol;        // [G] the sum of n_h over the groups h < g (packed blocks;
                              // group g then writes its n_g rows) | null: Rpad rows
  const int32_t* gstart;      // [G] first source row (or gather index) of group g | null
  int64_t R, Cc, Rpad;        // rows and columns in, rows written (>= R), an upper bound
                              // of the rows written with ocol
  int64_t in_gs, ld_in, gather_gs, out_gs, ld_out;
  int G;
};

struct BwdArgs {
  const int32_t* idx;         // [T,k]
  const float* gates;         // [T,k]
  const int32_t* slot;        // [T,k]
  const uint8_t* dropped;     // [T,k]
  const int32_t* counts;      // [E] choices per expert (before capacity)
  const float* logits;        // [T,E]
  const void* dy;             // [T,d]
  const void* ye;             // [E,C,d] the forward's expert outputs
  bf16_t* dYe;                // [E,C,d]
  float* dgates;              // [T,k]
  float* dz;                  // [T,E]
  const bf16_t* dA;           // [E,C,d] input gradients of the routed experts
  const bf16_t* dAs;          // [T,d] of the shared experts | null
  const float* wrT;           // [E,d] the router weight, transposed
  void* dx;                   // [T,d]
  int64_t T, C;
  int d, E, k;
  int score, renorm, zero_fallback;
  int packed;                 // dropless: slot is the packed row of ye, dYe and dA
  float alpha_aux, alpha_z;
  // expert choice (sel != null): the picks of token t are the experts e with
  // sel[t*E + e] >= 0 (row e*C + sel), gate probs[t*E + e]; the gate
  // gradients go to dprobs [T,E] (0 where not picked) instead of dgates
  const int32_t* sel;
  const float* probs;
  float* dprobs;
  int64_t fden;               // expert choice: the sum of the picks (f_i = counts_i / fden)
};

struct ActBwdArgs {
  const bf16_t* dH;           // [groups*rpg, F]
  const bf16_t* U;            // GELU: pre-activation; SwiGLU: gate projection
  const bf16_t* U2;           // SwiGLU: up projection | null
  bf16_t* dact;               // [groups*rpg, F] (GELU) or [groups*rpg, 2F] (SwiGLU)
  const int32_t* valid;       // [groups] | null
  int64_t rpg;
  int groups, F;
};

struct SeqLossArgs {
  const float* probs;         // [T,E]
  const int32_t* idx;         // [T,k]
  double* partial;            // [n_seq] per-sequence losses (workspace)
  float* loss;                // [1]
  int64_t seq_len, n_seq;
  int E, k;
};

// host-side launchers (defined in the kernel translation units)
hipError_t launch_route(const RouteArgs& a, int dtype, hipStream_t s);
hipError_t launch_capacity(const CapArgs& a, int dtype, hipStream_t s);
hipError_t launch_gemm(const GemmArgs& a, int dtype, hipStream_t s);
hipError_t launch_combine(const CombineArgs& a, int dtype, hipStream_t s);
hipError_t launch_losses(const LossArgs& a, hipStream_t s);
hipError_t launch_expert_choice(const EcArgs& a, hipStream_t s);
hipError_t launch_select_top(const EcArgs& a, hipStream_t s);
hipError_t launch_score_priority(const ScoreArgs& a, hipStream_t s);
hipError_t launch_gather_rows(const void* x, void* xe, const int32_t* row_token, const int32_t* kept, int64_t C,
                              int E, int row_bytes, hipStream_t s);
hipError_t launch_transpose(const TransposeArgs& a, hipStream_t s);
hipError_t launch_zero(void* p, size_t bytes, hipStream_t s);
hipError_t launch_combine_bwd(const BwdArgs& a, hipStream_t s);
hipError_t launch_router_bwd(const BwdArgs& a, hipStream_t s);
hipError_t launch_act_bwd(const ActBwdArgs& a, int act, hipStream_t s);
hipError_t launch_colsum(const bf16_t* in, void* out, const int32_t* valid, int groups, int64_t rpg, int64_t Cc,
                         int f32out, hipStream_t s, const int32_t* start = nullptr);
hipError_t launch_group_starts(const int32_t* counts, int32_t* start, int E, int pad8, hipStream_t s);
hipError_t launch_router_weight_prep(const float* dz, bf16_t* planes, int64_t T, int64_t Tp, int E,
                                     const float* w_router, float* wrT, int d, hipStream_t s);
hipError_t launch_dz_colsum(const float* dz, float* out, int64_t T, int E, hipStream_t s);
hipError_t launch_slab_sum(const float* slabs, float* out, int64_t n, int S, hipStream_t s);
hipError_t launch_dx(const BwdArgs& a, hipStream_t s);
hipError_t launch_seq_loss(const SeqLossArgs& a, hipStream_t s);
hipError_t launch_bias_update(const int32_t* counts, float* select_bias, int E, int64_t Tk, float gamma,
                              hipStream_t s);

// The bf16 router's logits GEMM splits d into S parts (one partial-logit
// slab each, summed in a fixed order) when the token tiles alone would not
// give the GPU about 256 workgroups: the smallest S in {1, 2, 4, 8} that
// does, among those that keep each part a multiple of 8 wide.
__host__ __device__ inline int router_splits(int64_t T, int E, int d) {
  const int64_t tiles = ((T + 255) / 256) * ((4 * static_cast<int64_t>(E) + 255) / 256);
  int s = 1;
  while (s < 8 && tiles * s < 256 && d % (16 * s) == 0) s *= 2;
  return s;
}

// router tile: tokens per workgroup of the per-token routing epilogue, one
// row of loss partial sums each (partial-sum arrays are sized for the
// smallest tile)
constexpr int kRouteTokens = 32;
constexpr int kMinRouteTile = 16;

}  // namespace moe
