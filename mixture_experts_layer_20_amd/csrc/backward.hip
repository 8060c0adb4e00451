// Backward pass of the token-choice layer: the kernels around the grouped
// GEMM (which the backward pass reuses with transposed operands).
//
// Sources: "Lab 18 -- Mixture of experts" s.1 (the layer and its gates; with
// raw top-1 gates the router learns through the gate value) and s.2 (the
// balance loss reaches the router only through P_i, f being a count; the
// z-loss); "Lab 01" "The traps" (f carries no gradient); "Mixture of
// experts" lecture, training a router.
//
// L = <dy, y> + alpha_aux L_aux + alpha_z L_z.  With r = (t, j) a kept
// choice of expert e in slot s and o_r = ye[e, s] its stored output:
//   dgate_r = <dy_t, o_r>,   dYe[e, s] = gate_r dy_t           (combine_bwd)
//   dz_t    = the gate, balance and z-loss terms               (router_bwd)
//   dU      = dH * gelu'(U)   or   [dGp | dUp]                 (act_bwd)
//   dx_t    = sum_j dA[e_tj, s_tj] + shared + fallback + dz_t W_r^T (dx)
// Transposes put every operand in the grouped GEMM's K-contiguous layout:
// weight gradients contract over the rows of an expert, zero-padded past its
// kept count.
#include "common.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kTr = 64;

// ------------------------------------------------------------------ transpose
// out[g][c][r] = in_row(g, r)[c] for r < valid_g, 0 for valid_g <= r < Rpad;
// in_row(g, r) = in + g*in_gs + r*ld_in, or in + gather[g*gather_gs + r]*ld_in.
// 64 x 64 tiles through LDS with 16-byte accesses (8 bf16) on both sides:
// every row length, stride and the padded row count are multiples of 8.  LDS
// rows are 66 elements (33 words) apart, so the 8-row column reads of a
// wavefront fall in distinct banks.
constexpr int kTrPitch = kTr + 2;

__global__ __launch_bounds__(kThreads) void transpose16_kernel(TransposeArgs a) {
  __shared__ uint32_t tile[kTr * kTrPitch / 2];
  const int g = blockIdx.z;
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * kTr;
  const int64_t c0 = static_cast<int64_t>(blockIdx.y) * kTr;
  const int tid = threadIdx.x;
  const int64_t valid = a.valid ? min<int64_t>(a.valid[g], a.R) : a.R;
  // rows written: Rpad, or with packed output columns the group's own
  // max(8, round8(valid)) (the zero padding a k-varying GEMM contracts over)
  const int64_t rpad = a.ocol ? max<int64_t>(8, (valid + 7) / 8 * 8) : a.Rpad;
  if (r0 >= rpad) return;
  const int64_t src0 = a.gstart ? a.gstart[g] : 0;
  {
    const int tr = tid / 8, tc = tid % 8;            // 32 rows x 8 chunks per pass
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int i = tr + 32 * p;
      const int64_t r = r0 + i, c = c0 + tc * 8;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (r < valid && c < a.Cc) {
        const int64_t src =
            a.gather ? static_cast<int64_t>(a.gather[(a.gstart ? src0 : g * a.gather_gs) + r]) * a.ld_in
            : a.gstart ? (src0 + r) * a.ld_in
                       : g * a.in_gs + r * a.ld_in;
        v = *reinterpret_cast<const uint4*>(a.in + src + c);
      }
      uint32_t* t = tile + (i * kTrPitch + tc * 8) / 2;
      t[0] = v.x;
      t[1] = v.y;
      t[2] = v.z;
      t[3] = v.w;
    }
  }
  __syncthreads();
  const bf16_t* tl = reinterpret_cast<const bf16_t*>(tile);
  const int wr = tid % 8, wc = tid / 8;              // 8 row chunks x 32 columns per pass
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int j = wc + 32 * p;
    const int64_t c = c0 + j, r = r0 + wr * 8;
    if (c >= a.Cc || r >= rpad) continue;
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      w[q] = static_cast<uint32_t>(tl[(wr * 8 + 2 * q) * kTrPitch + j]) |
             (static_cast<uint32_t>(tl[(wr * 8 + 2 * q + 1) * kTrPitch + j]) << 16);
    // packed: group g's block [Cc][rpad] starts ocol[g]*Cc elements in
    bf16_t* o = a.ocol ? a.out + static_cast<int64_t>(a.ocol[g]) * a.Cc + c * rpad + r
                       : a.out + g * a.out_gs + c * a.ld_out + r;
    *reinterpret_cast<uint4*>(o) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// ------------------------------------------------------------------ combine
// One wavefront per token; lanes j < k hold choice j.  For each kept choice:
// dgate = <dy_t, ye row> (per-lane partial sums over 16-byte chunks, then a
// fixed butterfly), and the gate-scaled dy_t goes to the choice's dYe row.
// The choices of token t on the lanes of its wavefront.  Token choice: lane
// j < k holds choice j (kBal = 1).  Expert choice: lane l holds experts l,
// l + 64, ... (kBal = 4 ballots, E <= 256).
template <bool EC>
struct Picks {
  static constexpr int kBal = EC ? 4 : 1;
  int64_t row[kBal];
  float gate[kBal];
  uint64_t kept[kBal];
  __device__ Picks(const BwdArgs& a, int64_t t, int lane) {
#pragma unroll
    for (int b = 0; b < kBal; ++b) {
      row[b] = 0;
      gate[b] = 0.0f;
      bool keep = false;
      if constexpr (EC) {
        const int e = b * kWave + lane;
        if (e < a.E) {
          const int sl = a.sel[t * a.E + e];
          keep = sl >= 0 && sl < a.C;
          row[b] = static_cast<int64_t>(e) * a.C + sl;
          gate[b] = a.probs[t * a.E + e];
        }
      } else if (lane < a.k) {
        const int64_t tk = t * a.k + lane;
        const int e = a.idx[tk];
        const int sl = a.slot[tk];
        // dropless: the slot is the packed row itself
        keep = !a.dropped[tk] && e >= 0 && e < a.E && sl >= 0 && sl < (a.packed ? a.T * a.k : a.C);
        row[b] = a.packed ? static_cast<int64_t>(sl) : static_cast<int64_t>(e) * a.C + sl;
        gate[b] = a.gates[tk];
      }
      kept[b] = __ballot(keep);
    }
  }
  __device__ bool any() const {
    uint64_t m = 0;
#pragma unroll
    for (int b = 0; b < kBal; ++b) m |= kept[b];
    return m != 0;
  }
};

template <bool EC>
__global__ __launch_bounds__(kThreads) void combine_bwd_kernel(BwdArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t t = static_cast<int64_t>(blockIdx.x) * (kThreads / kWave) + threadIdx.x / kWave;
  if (t >= a.T) return;
  const Picks<EC> pk(a, t, lane);
  const int nvec = a.d / 8;
  const uint4* dy = reinterpret_cast<const uint4*>(static_cast<const bf16_t*>(a.dy) + t * a.d);
  float mydg[Picks<EC>::kBal] = {};
#pragma unroll
  for (int bal = 0; bal < Picks<EC>::kBal; ++bal) {
  uint64_t rest = pk.kept[bal];
  while (rest) {
    const int j = __ffsll(static_cast<unsigned long long>(rest)) - 1;
    rest &= rest - 1;
    const int64_t row = __shfl(pk.row[bal], j, kWave);
    const float g = __shfl(pk.gate[bal], j, kWave);
    const uint4* ye = reinterpret_cast<const uint4*>(static_cast<const bf16_t*>(a.ye) + row * a.d);
    uint4* dye = reinterpret_cast<uint4*>(a.dYe + row * a.d);
    float part = 0.0f;
    for (int c = lane; c < nvec; c += kWave) {
      const uint4 u = dy[c], v = ye[c];
      const uint32_t uu[4] = {u.x, u.y, u.z, u.w}, vv[4] = {v.x, v.y, v.z, v.w};
      uint32_t w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float d0 = __uint_as_float(uu[q] << 16), d1 = __uint_as_float(uu[q] & 0xFFFF0000u);
        const float o0 = __uint_as_float(vv[q] << 16), o1 = __uint_as_float(vv[q] & 0xFFFF0000u);
        part += d0 * o0;
        part += d1 * o1;
        w[q] = static_cast<uint32_t>(f32_to_bf16(g * d0)) | (static_cast<uint32_t>(f32_to_bf16(g * d1)) << 16);
      }
      dye[c] = make_uint4(w[0], w[1], w[2], w[3]);
    }
    part = wave_sum(part);
    if (lane == j) mydg[bal] = part;
  }
  }
  if constexpr (EC) {
#pragma unroll
    for (int bal = 0; bal < Picks<EC>::kBal; ++bal) {
      const int e = bal * kWave + lane;
      if (e < a.E) a.dprobs[t * a.E + e] = mydg[bal];  // not picked: 0
    }
  } else if (lane < a.k) {
    a.dgates[t * a.k + lane] = mydg[0];               // dropped choices: 0
  }
}

// ------------------------------------------------------------------ router
// One wavefront per token, lane l holding experts l, l + 64, ... (E <= 256).
// Sums over experts go through wave_sum in float32 after max-shifting.
__global__ __launch_bounds__(kThreads) void router_bwd_kernel(BwdArgs a) {
  constexpr int kPer = 4;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t t = static_cast<int64_t>(blockIdx.x) * (kThreads / kWave) + threadIdx.x / kWave;
  if (t >= a.T) return;
  const int E = a.E, k = a.k;
  float z[kPer], dz[kPer], dgv[kPer];
  bool sel[kPer];
#pragma unroll
  for (int m = 0; m < kPer; ++m) {
    const int e = lane + kWave * m;
    z[m] = e < E ? a.logits[t * E + e] : -__builtin_huge_valf();
    dz[m] = 0.0f;
    dgv[m] = 0.0f;
    sel[m] = false;
  }
  // the gate gradient of each selected expert, placed at its expert
  for (int j = 0; j < k; ++j) {
    const int e = a.idx[t * k + j];
    const float g = a.dgates[t * k + j];
#pragma unroll
    for (int m = 0; m < kPer; ++m)
      if (e == lane + kWave * m) {
        sel[m] = true;
        dgv[m] = g;
      }
  }
  float zmax = -__builtin_huge_valf();
#pragma unroll
  for (int m = 0; m < kPer; ++m) zmax = fmaxf(zmax, z[m]);
  zmax = wave_max(zmax);
  float ex[kPer], sum = 0.0f;
#pragma unroll
  for (int m = 0; m < kPer; ++m) {
    ex[m] = lane + kWave * m < E ? __expf(z[m] - zmax) : 0.0f;
    sum += ex[m];
  }
  sum = wave_sum(sum);
  float p[kPer];
#pragma unroll
  for (int m = 0; m < kPer; ++m) p[m] = ex[m] / sum;
  const bool ren = a.renorm != 0;
  if (a.sel) {
    // expert choice: the gates are the probabilities themselves, so the pick
    // gradients and the balance term both go through the probabilities'
    // Jacobian: dz = q (u - <q, u>) [x s(-z) for sigmoid scores], u = dprobs + v
    float q[kPer], u[kPer], qu = 0.0f;
    if (a.score == MOE_SOFTMAX) {
#pragma unroll
      for (int m = 0; m < kPer; ++m) q[m] = p[m];
    } else {
      float lmax = -__builtin_huge_valf(), ssum = 0.0f;
#pragma unroll
      for (int m = 0; m < kPer; ++m) {
        q[m] = z[m] < 0.0f ? z[m] - log1pf(__expf(z[m])) : -log1pf(__expf(-z[m]));
        if (lane + kWave * m < E) lmax = fmaxf(lmax, q[m]);
      }
      lmax = wave_max(lmax);
#pragma unroll
      for (int m = 0; m < kPer; ++m) {
        q[m] = lane + kWave * m < E ? __expf(q[m] - lmax) : 0.0f;
        ssum += q[m];
      }
      ssum = wave_sum(ssum);
#pragma unroll
      for (int m = 0; m < kPer; ++m) q[m] /= ssum;
    }
#pragma unroll
    for (int m = 0; m < kPer; ++m) {
      const int e = lane + kWave * m;
      u[m] = 0.0f;
      if (e < E) {
        u[m] = a.dprobs[t * E + e];
        if (a.alpha_aux != 0.0f)
          u[m] += static_cast<float>(static_cast<double>(a.alpha_aux) * E *
                                     (static_cast<double>(a.counts[e]) / static_cast<double>(a.fden)) /
                                     static_cast<double>(a.T));
      }
      qu += q[m] * u[m];
    }
    qu = wave_sum(qu);
#pragma unroll
    for (int m = 0; m < kPer; ++m) {
      if (lane + kWave * m >= E) continue;
      float term = q[m] * (u[m] - qu);
      if (a.score != MOE_SOFTMAX) term *= 1.0f / (1.0f + __expf(z[m]));    // s(-z)
      dz[m] = term;
    }
  } else if (a.score == MOE_SOFTMAX) {
    if (ren) {
      // g = softmax over the selected logits (shifted by their own maximum):
      // dz_sel = g (dg - <g, dg>)
      float smax = -__builtin_huge_valf();
#pragma unroll
      for (int m = 0; m < kPer; ++m) smax = sel[m] ? fmaxf(smax, z[m]) : smax;
      smax = wave_max(smax);
      float w[kPer], ssum = 0.0f;
#pragma unroll
      for (int m = 0; m < kPer; ++m) {
        w[m] = sel[m] ? __expf(z[m] - smax) : 0.0f;
        ssum += w[m];
      }
      ssum = wave_sum(ssum);
      float gdg = 0.0f;
#pragma unroll
      for (int m = 0; m < kPer; ++m) gdg += sel[m] ? (w[m] / ssum) * dgv[m] : 0.0f;
      gdg = wave_sum(gdg);
#pragma unroll
      for (int m = 0; m < kPer; ++m)
        if (sel[m]) dz[m] = (w[m] / ssum) * (dgv[m] - gdg);
    } else {
      // g = p_sel: dz = p (dp - <p, dp>), dp = dg at the selected experts
      float pdp = 0.0f;
#pragma unroll
      for (int m = 0; m < kPer; ++m) pdp += sel[m] ? p[m] * dgv[m] : 0.0f;
      pdp = wave_sum(pdp);
#pragma unroll
      for (int m = 0; m < kPer; ++m)
        if (lane + kWave * m < E) dz[m] = p[m] * ((sel[m] ? dgv[m] : 0.0f) - pdp);
    }
  } else {
    // sigmoid scores in the log domain (as the forward pass forms them):
    // ls = log s(z), and 1 - s(z) = s(-z), both without cancellation
    float ls[kPer], sm[kPer];
#pragma unroll
    for (int m = 0; m < kPer; ++m) {
      ls[m] = z[m] < 0.0f ? z[m] - log1pf(__expf(z[m])) : -log1pf(__expf(-z[m]));
      sm[m] = 1.0f / (1.0f + __expf(z[m]));
    }
    if (ren) {
      // g = softmax over the selected log s: dz_sel = g (dg - <g, dg>) s(-z)
      float lmax = -__builtin_huge_valf();
#pragma unroll
      for (int m = 0; m < kPer; ++m) lmax = sel[m] ? fmaxf(lmax, ls[m]) : lmax;
      lmax = wave_max(lmax);
      float w[kPer], ssum = 0.0f;
#pragma unroll
      for (int m = 0; m < kPer; ++m) {
        w[m] = sel[m] ? __expf(ls[m] - lmax) : 0.0f;
        ssum += w[m];
      }
      ssum = wave_sum(ssum);
      float gdg = 0.0f;
#pragma unroll
      for (int m = 0; m < kPer; ++m) gdg += sel[m] ? (w[m] / ssum) * dgv[m] : 0.0f;
      gdg = wave_sum(gdg);
#pragma unroll
      for (int m = 0; m < kPer; ++m)
        if (sel[m]) dz[m] = (w[m] / ssum) * (dgv[m] - gdg) * sm[m];
    } else {
#pragma unroll
      for (int m = 0; m < kPer; ++m)
        if (sel[m]) dz[m] = dgv[m] * __expf(ls[m]) * sm[m];
    }
  }
  // balance loss: dL/dp_ti = alpha E f_i / T, f_i = count_i / (T k)
  if (a.alpha_aux != 0.0f && !a.sel) {
    float v[kPer], q[kPer], qv = 0.0f;
    if (a.score == MOE_SOFTMAX) {
#pragma unroll
      for (int m = 0; m < kPer; ++m) q[m] = p[m];
    } else {
      // q = the sigmoid scores normalised over all E: softmax of log s(z)
      float lmax = -__builtin_huge_valf(), ssum = 0.0f;
#pragma unroll
      for (int m = 0; m < kPer; ++m) {
        q[m] = z[m] < 0.0f ? z[m] - log1pf(__expf(z[m])) : -log1pf(__expf(-z[m]));
        if (lane + kWave * m < E) lmax = fmaxf(lmax, q[m]);
      }
      lmax = wave_max(lmax);
#pragma unroll
      for (int m = 0; m < kPer; ++m) {
        q[m] = lane + kWave * m < E ? __expf(q[m] - lmax) : 0.0f;
        ssum += q[m];
      }
      ssum = wave_sum(ssum);
#pragma unroll
      for (int m = 0; m < kPer; ++m) q[m] /= ssum;
    }
#pragma unroll
    for (int m = 0; m < kPer; ++m) {
      const int e = lane + kWave * m;
      v[m] = e < E ? static_cast<float>(static_cast<double>(a.alpha_aux) * E *
                                        (static_cast<double>(a.counts[e]) / (static_cast<double>(a.T) * k)) /
                                        static_cast<double>(a.T))
                   : 0.0f;
      qv += q[m] * v[m];
    }
    qv = wave_sum(qv);
#pragma unroll
    for (int m = 0; m < kPer; ++m) {
      if (lane + kWave * m >= E) continue;
      float term = q[m] * (v[m] - qv);
      if (a.score != MOE_SOFTMAX) term *= 1.0f / (1.0f + __expf(z[m]));          // s(-z)
      dz[m] += term;
    }
  }
  // z-loss: dL_z/dz_ti = 2 LSE_t p_ti / T
  if (a.alpha_z != 0.0f) {
    const float lse = zmax + __logf(sum);
    const float c = 2.0f * a.alpha_z * lse / static_cast<float>(a.T);
#pragma unroll
    for (int m = 0; m < kPer; ++m)
      if (lane + kWave * m < E) dz[m] += c * p[m];
  }
#pragma unroll
  for (int m = 0; m < kPer; ++m) {
    const int e = lane + kWave * m;
    if (e < E) a.dz[t * E + e] = dz[m];
  }
}

// ------------------------------------------------------------------ activations
// GELU:   dU = dH * (Phi(U) + U phi(U))                      -> dact [rows, F]
// SwiGLU: dGp = dH * Up * s (1 + Gp (1 - s)), dUp = dH * Gp s -> dact [rows, 2F]
// over the first valid_g rows of each group (rows_per_group apart).
template <int ACT>
__global__ __launch_bounds__(kThreads) void act_bwd_kernel(ActBwdArgs a) {
  // eight consecutive columns per thread and step (F is a multiple of 8 and
  // every row starts 16-byte aligned): 16-byte loads and stores
  const int g = blockIdx.y;
  const int64_t valid = a.valid ? min<int64_t>(a.valid[g], a.rpg) : a.rpg;
  const int F8 = a.F / 8;
  const int64_t n = valid * F8;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * kThreads) {
    const int64_t r = i / F8;
    const int c8 = static_cast<int>(i - r * F8) * 8;
    const int64_t row = static_cast<int64_t>(g) * a.rpg + r;
    const uint4 dh4 = *reinterpret_cast<const uint4*>(a.dH + row * a.F + c8);
    const uint4 u4 = *reinterpret_cast<const uint4*>(a.U + row * a.F + c8);
    const uint32_t dh[4] = {dh4.x, dh4.y, dh4.z, dh4.w}, uu[4] = {u4.x, u4.y, u4.z, u4.w};
    uint32_t o0[4], o1[4];
    if (ACT == 1) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t w = 0;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const float d = __uint_as_float(h ? dh[q] & 0xFFFF0000u : dh[q] << 16);
          const float u = __uint_as_float(h ? uu[q] & 0xFFFF0000u : uu[q] << 16);
          // Phi(u) + u phi(u), both from normal_tail's approximation
          float e;
          const float c = normal_tail(u, e);
          const float grad = (u >= 0.0f ? 1.0f - c : c) + u * e * 0.39894228040143268f;
          w |= static_cast<uint32_t>(f32_to_bf16(d * grad)) << (16 * h);
        }
        o0[q] = w;
      }
      *reinterpret_cast<uint4*>(a.dact + row * a.F + c8) = make_uint4(o0[0], o0[1], o0[2], o0[3]);
    } else {
      const uint4 v4 = *reinterpret_cast<const uint4*>(a.U2 + row * a.F + c8);
      const uint32_t vv[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t w0 = 0, w1 = 0;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const float d = __uint_as_float(h ? dh[q] & 0xFFFF0000u : dh[q] << 16);
          const float gp = __uint_as_float(h ? uu[q] & 0xFFFF0000u : uu[q] << 16);
          const float up = __uint_as_float(h ? vv[q] & 0xFFFF0000u : vv[q] << 16);
          const float s = 1.0f / (1.0f + __expf(-gp));
          w0 |= static_cast<uint32_t>(f32_to_bf16(d * up * s * (1.0f + gp * (1.0f - s)))) << (16 * h);
          w1 |= static_cast<uint32_t>(f32_to_bf16(d * gp * s)) << (16 * h);
        }
        o0[q] = w0;
        o1[q] = w1;
      }
      *reinterpret_cast<uint4*>(a.dact + row * 2 * a.F + c8) = make_uint4(o0[0], o0[1], o0[2], o0[3]);
      *reinterpret_cast<uint4*>(a.dact + row * 2 * a.F + a.F + c8) = make_uint4(o1[0], o1[1], o1[2], o1[3]);
    }
  }
}

// ------------------------------------------------------------------ column sums
// out[g*Cc + c] = sum over the first valid_g rows r of in[g*rpg + r][c],
// float32 in row order, stored in the storage type (or float32 with f32out).
__global__ __launch_bounds__(kThreads) void colsum_kernel(const bf16_t* __restrict__ in, void* out,
                                                          const int32_t* valid, const int32_t* start, int64_t rpg,
                                                          int64_t Cc, int f32out) {
  const int g = blockIdx.y;
  const int64_t c = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (c >= Cc) return;
  const int64_t nv = valid ? min<int64_t>(valid[g], rpg) : rpg;
  // group g's rows: from g*rpg, or (packed) from start[g]
  const bf16_t* p = in + (start ? static_cast<int64_t>(start[g]) : static_cast<int64_t>(g) * rpg) * Cc + c;
  float s = 0.0f;
  for (int64_t r = 0; r < nv; ++r) s += bf16_to_f32(p[r * Cc]);
  if (f32out) static_cast<float*>(out)[g * Cc + c] = s;
  else static_cast<bf16_t*>(out)[g * Cc + c] = f32_to_bf16(s);
}

// float32 column sums of dz [T, E] in float64, one thread per expert
__global__ __launch_bounds__(kThreads) void dz_colsum_kernel(const float* __restrict__ dz, float* out, int64_t T,
                                                             int E) {
  const int e = blockIdx.x * kThreads + threadIdx.x;
  if (e >= E) return;
  double s = 0.0;
  for (int64_t t = 0; t < T; ++t) s += dz[t * E + e];
  out[e] = static_cast<float>(s);
}

// dz [T, E] float32 -> its exact bf16 planes [4E, Tp] (row 4e + p: plane p of
// expert e over the tokens, row 4e + 3 and columns past T zero)
__global__ __launch_bounds__(kThreads) void dz_planes_kernel(const float* __restrict__ dz, bf16_t* planes,
                                                             int64_t T, int64_t Tp, int E) {
  const int64_t n = static_cast<int64_t>(E) * Tp;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * kThreads) {
    const int e = static_cast<int>(i / Tp);
    const int64_t t = i % Tp;
    bf16_t hi = 0, mid = 0, lo = 0;
    if (t < T) split3(dz[t * E + e], hi, mid, lo);
    bf16_t* row = planes + static_cast<int64_t>(4 * e) * Tp + t;
    row[0] = hi;
    row[Tp] = mid;
    row[2 * Tp] = lo;
    row[3 * Tp] = 0;
  }
}

// out[i] = sum over s of slabs[s][i], in slab order
__global__ __launch_bounds__(kThreads) void slab_sum_kernel(const float* __restrict__ slabs, float* out, int64_t n,
                                                            int S) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= n) return;
  float s = 0.0f;
  for (int q = 0; q < S; ++q) s += slabs[q * n + i];
  out[i] = s;
}

// w_r [d, E] float32 -> [E, d]
__global__ __launch_bounds__(kThreads) void wr_transpose_kernel(const float* __restrict__ w, float* wt, int d, int E) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= static_cast<int64_t>(d) * E) return;
  const int e = static_cast<int>(i / d), c = static_cast<int>(i % d);
  wt[i] = w[static_cast<int64_t>(c) * E + e];
}

// ------------------------------------------------------------------ dx
// One wavefront per token, 8 columns per lane per round:
//   dx_t = sum_j kept dA[row_j] (j order) + dAs_t (shared) | dy_t (fallback,
//          residual) + sum_e dz_te W_r[:, e]
template <bool EC>
__global__ __launch_bounds__(kThreads) void dx_kernel(BwdArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t t = static_cast<int64_t>(blockIdx.x) * (kThreads / kWave) + threadIdx.x / kWave;
  if (t >= a.T) return;
  const Picks<EC> pk(a, t, lane);
  float dzv[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int e = lane + kWave * m;
    dzv[m] = e < a.E ? a.dz[t * a.E + e] : 0.0f;
  }
  const int nvec = a.d / 8;
  const bool fallback = !pk.any() && a.dAs == nullptr && !a.zero_fallback;
  // every lane runs every round (the shuffles below read all lanes); the
  // loads and the store are those of the lanes whose column c is in the row
  for (int c0 = 0; c0 < nvec; c0 += kWave) {
    const int c = c0 + lane;
    const bool on = c < nvec;
    float acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
    auto add_row = [&](const bf16_t* base) {
      if (!on) return;
      const uint4 u = reinterpret_cast<const uint4*>(base)[c];
      const uint32_t uu[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] += __uint_as_float(uu[q] << 16);
        acc[2 * q + 1] += __uint_as_float(uu[q] & 0xFFFF0000u);
      }
    };
#pragma unroll
    for (int bal = 0; bal < Picks<EC>::kBal; ++bal) {
      uint64_t rest = pk.kept[bal];
      while (rest) {
        const int j = __ffsll(static_cast<unsigned long long>(rest)) - 1;
        rest &= rest - 1;
        add_row(a.dA + __shfl(pk.row[bal], j, kWave) * a.d);
      }
    }
    if (a.dAs) add_row(a.dAs + t * a.d);
    else if (fallback) add_row(static_cast<const bf16_t*>(a.dy) + t * a.d);
    for (int e = 0; e < a.E; ++e) {
      const float g = __shfl(dzv[e / kWave], e % kWave, kWave);
      if (!on) continue;
      const float4* w = reinterpret_cast<const float4*>(a.wrT + static_cast<int64_t>(e) * a.d + c * 8);
      const float4 w0 = w[0], w1 = w[1];
      acc[0] += g * w0.x; acc[1] += g * w0.y; acc[2] += g * w0.z; acc[3] += g * w0.w;
      acc[4] += g * w1.x; acc[5] += g * w1.y; acc[6] += g * w1.z; acc[7] += g * w1.w;
    }
    uint32_t o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      o[q] = static_cast<uint32_t>(f32_to_bf16(acc[2 * q])) | (static_cast<uint32_t>(f32_to_bf16(acc[2 * q + 1])) << 16);
    if (on) reinterpret_cast<uint4*>(static_cast<bf16_t*>(a.dx) + t * a.d)[c] = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// Group starts (one workgroup, E <= 256): start[g] = n[0] + ... + n[g-1] and
// start[E] = the total, with n = counts, or with pad8 n = max(8, round8(counts))
// (the columns of a group in operands packed along k for the weight-gradient
// GEMMs; an empty group keeps 8 zero columns).
__global__ __launch_bounds__(kThreads) void group_starts_kernel(const int32_t* __restrict__ counts, int32_t* start,
                                                                int E, int pad8) {
  __shared__ int v[kThreads];
  const int tid = threadIdx.x;
  int c = tid < E ? max(counts[tid], 0) : 0;
  if (pad8 && tid < E) c = max(8, (c + 7) / 8 * 8);
  v[tid] = c;
  __syncthreads();
  for (int o = 1; o < kThreads; o <<= 1) {
    const int u = tid >= o ? v[tid - o] : 0;
    __syncthreads();
    v[tid] += u;
    __syncthreads();
  }
  if (tid < E) start[tid] = v[tid] - c;
  if (tid == E - 1) start[E] = v[tid];
}

__global__ __launch_bounds__(kThreads) void zero_kernel(uint16_t* p, int64_t n) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * kThreads)
    p[i] = 0;
}

}  // namespace

// Zero `bytes` (even) bytes with a kernel (no memset node in a captured graph).
hipError_t launch_zero(void* p, size_t bytes, hipStream_t s) {
  const int64_t n = static_cast<int64_t>(bytes / 2);
  if (n == 0) return hipSuccess;
  zero_kernel<<<static_cast<unsigned>(std::min<int64_t>(4096, (n + kThreads - 1) / kThreads)), kThreads, 0, s>>>(
      static_cast<uint16_t*>(p), n);
  return hipGetLastError();
}

hipError_t launch_group_starts(const int32_t* counts, int32_t* start, int E, int pad8, hipStream_t s) {
  group_starts_kernel<<<1, kThreads, 0, s>>>(counts, start, E, pad8);
  return hipGetLastError();
}

hipError_t launch_transpose(const TransposeArgs& a, hipStream_t s) {
  if (a.G == 0 || a.Rpad == 0 || a.Cc == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((a.Rpad + kTr - 1) / kTr), static_cast<unsigned>((a.Cc + kTr - 1) / kTr),
                  static_cast<unsigned>(a.G));
  const bool wide = a.Cc % 8 == 0 && a.Rpad % 8 == 0 && a.ld_in % 8 == 0 && a.ld_out % 8 == 0 && a.in_gs % 8 == 0 &&
                    a.out_gs % 8 == 0 && reinterpret_cast<uintptr_t>(a.in) % 16 == 0 &&
                    reinterpret_cast<uintptr_t>(a.out) % 16 == 0;
  if (!wide) return hipErrorInvalidValue;
  transpose16_kernel<<<grid, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_combine_bwd(const BwdArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const unsigned grid = static_cast<unsigned>((a.T + 3) / 4);
  if (a.sel)
    combine_bwd_kernel<true><<<grid, kThreads, 0, s>>>(a);
  else
    combine_bwd_kernel<false><<<grid, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_router_bwd(const BwdArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const unsigned grid = static_cast<unsigned>((a.T + 3) / 4);
  router_bwd_kernel<<<grid, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_act_bwd(const ActBwdArgs& a, int act, hipStream_t s) {
  if (a.groups == 0 || a.rpg == 0) return hipSuccess;
  if (a.F % 8) return hipErrorInvalidValue;
  const int64_t per = a.rpg * (a.F / 8);
  const dim3 grid(static_cast<unsigned>(std::min<int64_t>((per + kThreads - 1) / kThreads, 4096)),
                  static_cast<unsigned>(a.groups));
  if (act == MOE_GELU) act_bwd_kernel<1><<<grid, kThreads, 0, s>>>(a);
  else act_bwd_kernel<2><<<grid, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_colsum(const bf16_t* in, void* out, const int32_t* valid, int groups, int64_t rpg, int64_t Cc,
                         int f32out, hipStream_t s, const int32_t* start) {
  if (groups == 0 || Cc == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((Cc + kThreads - 1) / kThreads), static_cast<unsigned>(groups));
  colsum_kernel<<<grid, kThreads, 0, s>>>(in, out, valid, start, rpg, Cc, f32out);
  return hipGetLastError();
}

hipError_t launch_router_weight_prep(const float* dz, bf16_t* planes, int64_t T, int64_t Tp, int E,
                                     const float* w_router, float* wrT, int d, hipStream_t s) {
  const int64_t n = static_cast<int64_t>(E) * Tp;
  if (n > 0)
    dz_planes_kernel<<<static_cast<unsigned>(std::min<int64_t>(4096, (n + kThreads - 1) / kThreads)), kThreads, 0, s>>>(
        dz, planes, T, Tp, E);
  const int64_t m = static_cast<int64_t>(d) * E;
  wr_transpose_kernel<<<static_cast<unsigned>((m + kThreads - 1) / kThreads), kThreads, 0, s>>>(w_router, wrT, d, E);
  return hipGetLastError();
}

hipError_t launch_dz_colsum(const float* dz, float* out, int64_t T, int E, hipStream_t s) {
  dz_colsum_kernel<<<static_cast<unsigned>((E + kThreads - 1) / kThreads), kThreads, 0, s>>>(dz, out, T, E);
  return hipGetLastError();
}

hipError_t launch_slab_sum(const float* slabs, float* out, int64_t n, int S, hipStream_t s) {
  if (n == 0) return hipSuccess;
  slab_sum_kernel<<<static_cast<unsigned>((n + kThreads - 1) / kThreads), kThreads, 0, s>>>(slabs, out, n, S);
  return hipGetLastError();
}

hipError_t launch_dx(const BwdArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  if (a.sel)
    dx_kernel<true><<<static_cast<unsigned>((a.T + 3) / 4), kThreads, 0, s>>>(a);
  else
    dx_kernel<false><<<static_cast<unsigned>((a.T + 3) / 4), kThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace moe
