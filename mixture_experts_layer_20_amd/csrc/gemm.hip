// Grouped expert GEMMs for gfx950: C[g] = act(A[g] B[g]^T + bias[g]) for every
// expert g, with ragged row counts read on the device.
//
// Sources: "Lab 18 -- Mixture of experts" s.1 (an expert is a 2-matrix GELU
// MLP, or Mixtral's 3-matrix SwiGLU FFN) and Tips (production kernels run one
// grouped matrix multiply over all experts); "Mixture of experts" lecture
// field map, systems section (small ragged per-expert matmuls).
//
// bf16 path: v_mfma_f32_32x32x16_bf16 with float32 accumulation.
//   * Workgroup tile: 256 token rows x 256 weight rows x 64 (k), 8 wavefronts
//     (two per SIMD), each owning 128 weight rows x 64 token rows of the
//     output (4 x 2 MFMA blocks, 128 float32 accumulators per lane).  For
//     SwiGLU the 256 weight rows are 128 gate rows and the 128 matching up
//     rows, so the epilogue has g and u of the same output element in the
//     same lane and register.
//   * The MFMA's first operand is the weight tile and its second the token
//     tile, so each lane ends with four consecutive output columns of one
//     token row.  The epilogue stages the bf16 results through LDS and
//     stores whole row segments.
//   * Direct global -> LDS loads (buffer_load ... lds), 16 bytes per lane:
//     one wavefront instruction fills 8 rows x 128 bytes, i.e. whole cache
//     lines (the load path moves about 1.7x the bytes per cycle it moves
//     for half lines).  The token rows and the weight rows each have their
//     own ring of stage buffers in LDS (2 token stages, 3 weight stages:
//     160 KiB), one barrier per 64-wide k stage;
//     16-byte chunks XOR-swizzled by row so fragment reads spread over the
//     LDS banks.  Token rows may be gathered through a row list (the
//     dispatch is fused into this load).
//   * Tile order: with row counts on the device, only tiles that hold rows
//     are numbered (so no empty tile sits between the chunks below); tiles
//     walk bands of 4 row tiles (2 for narrow outputs) column by column, and
//     32-tile chunks of them are dealt round-robin to the 8 XCDs (blocks
//     reach XCDs round-robin), so the ~32 tiles an XCD runs at once share 4
//     token panels and 8 weight panels in its L2 while every XCD gets an even
//     share of every expert.
//   * Tail split: a last round of tiles that would leave more than half of
//     the 256 compute units idle is split along k into float32 partial tiles
//     (a workspace), summed in part order by a small kernel that applies the
//     bias and activation.
//   * A partial tile (an expert's last, fewer than 256 valid token rows, or
//     one reaching past N) skips the MFMAs of 32-row token blocks without
//     valid rows and of 32-row weight blocks past N.
//   * Rows at or past rows[g] and columns past N read as zero through the
//     buffer bounds and are never stored; k past K reads 0.
// Router mode (ACT 3): C is float32 [rows, N/4], the sum of each group of four
// output columns (the router weight's bf16 planes; see the router).
// float32 path: a plain LDS-tiled FMA kernel (small layers only).
#include <type_traits>

#include "common.hpp"

namespace moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kBM = 256;     // token rows per tile
constexpr int kBW = 256;     // weight rows per tile
constexpr int kBK = 64;      // k per pipeline stage
constexpr int kNX = 2;       // token-row stages in LDS
constexpr int kNW = 3;       // weight-row stages in LDS (one more in flight: the
                             // weight panels are the operand that misses L2)
constexpr int kLoadPositions = 2;   // 16-k steps a stage's loads are spread over
constexpr int kRowBytes = kBK * 2;                         // 128: one full cache line per row
constexpr int kChunks = kRowBytes / 16;                    // 16-byte k-chunks per row
constexpr int kXBytes = kBM * kRowBytes;                   // one token-row stage (32 KiB)
constexpr int kWBytes = kBW * kRowBytes;                   // one weight-row stage (32 KiB)
constexpr int kLdsBytes = kNX * kXBytes + kNW * kWBytes;   // 160 KiB
constexpr int kRowsPerLoad = 1024 / kRowBytes;             // rows one wave instruction fills
// Wavefronts per workgroup: 8, two per SIMD, each owning 64 token rows x 128
// weight rows of the output (measured against 4 waves of 128 x 128, which
// need 256 accumulators a lane and spill or lose the second wave per SIMD
// that hides latency).
template <int W>
struct Geo {
  static_assert(W == 8, "8 wavefronts");
  static constexpr int kWaves = W;
  static constexpr int kThreads = W * 64;
  static constexpr int kHalf = W / 2;                         // waves staging each operand
  static constexpr int kSRows = 256 / kHalf;                  // tile rows one wave stages
  static constexpr int kLoadsPerWave = kSRows / kRowsPerLoad; // load instructions per stage
  static constexpr int kXR = 256 / kHalf;                     // token rows of one wave's output
  static constexpr int kXB = kXR / 32;                        // its 32-row token blocks
  static constexpr int kPairs = 4 * kXB / 2;                  // MFMA pairs (groups) per 16-k step
  static constexpr int kFrags = 4 + kXB;                      // fragment reads per 16-k step
  static_assert(kLoadsPerWave <= 32, "one bit per load in the past-K mask");
  
  // Fragment reads of a 16-k step in the order the step's MFMA groups
  // consume them (token fragments are ids 4.., weight fragments 0..3), and
  // the group that issues read r: the reads are spread over the groups,
  // earliest first.
  struct FragPlan {
    int order[kFrags];
    int group[kFrags];
  };
  static constexpr FragPlan frag_plan() {
    FragPlan f{};
    bool seen[kFrags] = {};
    int n = 0;
    for (int q = 0; q < kPairs; ++q) {
      const int i = (2 * q) / kXB, j0 = (2 * q) % kXB;
      const int need[3] = {4 + j0, 4 + j0 + 1, i};
      for (int u = 0; u < 3; ++u)
        if (!seen[need[u]]) { seen[need[u]] = true; f.order[n++] = need[u]; }
    }
    for (int r = 0; r < kFrags; ++r) f.group[r] = (r * kPairs) / kFrags;
    return f;
  }
};
template <int W>
constexpr typename Geo<W>::FragPlan kPlanOf = Geo<W>::frag_plan();
static_assert(kXBytes == kWBytes, "both rings use one buffer size");
static_assert(kLdsBytes <= 160 * 1024, "gfx950 LDS");

__device__ __forceinline__ float gelu_erf(float v) {
  return 0.5f * v * (1.0f + erff(v * 0.70710678118654752440f));
}
// GELU for the bf16 epilogues: v * Phi(v) with the normal tail of
// normal_tail (common.hpp): about 4e-7 absolute in the float32 result (far
// below the bf16 rounding of the stored output) for a third of the
// instructions of erff; float32 layers keep gelu_erf
__device__ __forceinline__ float gelu_fast(float v) {
  float e;
  const float c = normal_tail(v, e);
  return v * (v >= 0.0f ? 1.0f - c : c);
}
__device__ __forceinline__ float silu(float v) { return v / (1.0f + expf(-v)); }
// SiLU from the hardware exp2 and reciprocal: a few ulps in float32, far
// below the bf16 rounding of the bf16 path's result
__device__ __forceinline__ float silu_fast(float v) {
  return v * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(v * -1.44269504088896341f));
}

// Byte offset of logical 16-byte k-chunk `chunk` of tile row `row` in LDS:
// the chunk index is XORed with the row bits above the ones that already
// separate rows within 128 bytes, so the 16 lanes a 128-bit LDS read serves
// at once (16 consecutive rows, one logical chunk) hit 16 distinct 16-byte
// bank groups.
constexpr int kSwzShift = kRowBytes == 64 ? 2 : 1;
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * kRowBytes + ((chunk ^ ((row >> kSwzShift) & (kChunks - 1))) << 4);
}

// s_waitcnt immediate: vmcnt(n), lgkmcnt(0), expcnt unchanged (gfx9 layout)
__device__ __forceinline__ constexpr int wait_vm_lgkm0(int n) {
  return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4);
}

struct TileCoord {
  int g, mt, nt;
  bool valid;
};

// Row tiles per band of the tile walk: 4, or 2 when the output has at most
// four column tiles (narrow GEMMs of fine-grained experts: 32-tile chunks
// then span fewer of an expert's mostly empty capacity tiles; 5% faster on
// the 64-expert layer, the same elsewhere).
__device__ __forceinline__ int band_rows(int ntiles) { return ntiles <= 4 ? 2 : 4; }

// Tile r of a group of mt row tiles (r < mt * ntiles) -> (row tile, column
// tile): floor(mt / band) bands (at least one), the first taking the
// remainder rows, each walked column by column.
__device__ __forceinline__ void band_walk(int r, int mt, int ntiles, int& rt, int& ct) {
  const int kGM = band_rows(ntiles);
  const int nb = max(1, mt / kGM);
  const int base = mt / nb, extra = mt % nb;                  // the first `extra` bands are one taller
  const int tall = extra * (base + 1) * ntiles;               // tiles in the taller bands
  int first, gm, within;
  if (r < tall) {
    gm = base + 1;
    first = (r / (gm * ntiles)) * gm;
    within = r % (gm * ntiles);
  } else {
    gm = base;
    const int r2 = r - tall;
    first = extra * (base + 1) + (r2 / (gm * ntiles)) * gm;
    within = r2 % (gm * ntiles);
  }
  rt = first + within % gm;
  ct = within / gm;
}

// logical tile -> (group, row tile, column tile): bands of band_rows row
// tiles, walked column by column
__device__ __forceinline__ TileCoord decode_tile(int64_t L, int mt_max, int ntiles, int groups) {
  TileCoord c;
  const int64_t per_group = static_cast<int64_t>(mt_max) * ntiles;
  c.valid = L < per_group * groups;
  if (!c.valid) { c.g = c.mt = c.nt = 0; return c; }
  c.g = static_cast<int>(L / per_group);
  band_walk(static_cast<int>(L % per_group), mt_max, ntiles, c.mt, c.nt);
  return c;
}

// Groups of a packed-rows launch (the ABI's expert limit).
constexpr int kMaxPackedGroups = 256;

// Dense tile table for row counts read on the device (a.rows; packed: rows
// laid back to back).  Wave 0 of the workgroup fills, for every group, its
// first row (packed), valid rows and the end of its range of tiles in the
// dense numbering (only tiles that hold rows); the caller synchronises.
__device__ __forceinline__ void build_tile_table(const GemmArgs& a, int ntiles, int* pk_start, int* pk_rows,
                                                 int* pk_end) {
  const int ln = threadIdx.x & 63;
  if (threadIdx.x >= kWave) return;
  int64_t carry_r = 0;
  int carry_t = 0;
  for (int c = 0; c < a.groups; c += kWave) {
    const int g = c + ln;
    const int64_t rg = g < a.groups ? max(a.rows[g], 0) : 0;
    int64_t vr = rg;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int64_t u = __shfl_up(vr, o, kWave);
      if (ln >= o) vr += u;
    }
    const int64_t start = a.packed ? min(carry_r + vr - rg, a.total_rows) : static_cast<int64_t>(g) * a.rows_per_group;
    const int re = static_cast<int>(a.packed ? max<int64_t>(0, min<int64_t>(rg, a.total_rows - start))
                                             : min<int64_t>(rg, a.rows_per_group));
    int vt = (re + kBM - 1) / kBM * ntiles;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int u = __shfl_up(vt, o, kWave);
      if (ln >= o) vt += u;
    }
    if (g < a.groups) {
      pk_start[g] = static_cast<int>(a.packed ? start : 0);
      pk_rows[g] = re;
      pk_end[g] = carry_t + vt;
    }
    carry_r += __shfl(vr, kWave - 1, kWave);
    carry_t += __shfl(vt, kWave - 1, kWave);
  }
}

// Dense tile L (below the table's total) -> (group, row tile, column tile):
// within a group, bands of band_rows row tiles walked column by column.
__device__ __forceinline__ TileCoord decode_dense(int L, int groups, int ntiles, const int* pk_end) {
  const int ln = threadIdx.x & 63;
  int g = 0;
  for (int c = 0; c < groups; c += kWave) g += __popcll(__ballot(c + ln < groups && pk_end[c + ln] <= L));
  const int first = g ? pk_end[g - 1] : 0;
  const int mt_g = (pk_end[g] - first) / ntiles;
  TileCoord tc;
  tc.g = g;
  band_walk(L - first, mt_g, ntiles, tc.mt, tc.nt);
  tc.valid = true;
  return tc;
}

// Tail split (GEMMs with device row counts and a partial-sum workspace):
// when the dense tiles fill a last round of the GPU's 256 compute units at
// most half, that round's R tiles are split along k into P parts (P*R <= 256,
// parts of at least kTailMinK: shorter tiles lose more to the extra pass than
// the idle compute units cost), written as float32 partial tiles and summed
// in part order by tail_sum_kernel.  F = tiles before the tail (all tiles
// when nothing is split).
constexpr int kCUs = 256;
constexpr int kTailMinK = 2048;
constexpr int kMaxTailParts = 8;
struct TailPlan {
  int F, R, P;
  int kslice;
};
__device__ __forceinline__ TailPlan tail_plan(int NT, int K, int max_parts) {
  TailPlan t{NT, 0, 1, K};
  const int R = NT % kCUs;
  if (NT < kCUs || R == 0 || R > kCUs / 2) return t;
  const int P = min(min(max_parts, kCUs / R), K / kTailMinK);
  if (P < 2) return t;
  t.kslice = ((K + P - 1) / P + 63) / 64 * 64;
  t.P = (K + t.kslice - 1) / t.kslice;
  if (t.P < 2) return TailPlan{NT, 0, 1, K};
  t.F = NT - R;
  t.R = R;
  return t;
}

// Buffer resource word 3 for raw (unswizzled, untyped) buffers on gfx9.
constexpr int kRsrcWord3 = 0x00020000;
// An offset past every operand (operands are kept below 2^31 bytes), which
// stays past them after a stage's k offset is added: loads from it read zero.
constexpr uint32_t kOutOfRange = 0x80000000u;

typedef __attribute__((address_space(3))) void* lds_ptr_t;

template <int ACT, int W, int KM = 0>
__device__ __forceinline__ void gemm_bf16_body(const GemmArgs& a) {
  static_assert(KM == 0 || ACT == 0, "k-major operands: bias-only GEMMs");
  constexpr bool kAkm = (KM & 1) != 0, kBkm = (KM & 2) != 0;
  using G = Geo<W>;
  constexpr int kWaves = G::kWaves, kHalf = G::kHalf, kSRows = G::kSRows, kLoadsPerWave = G::kLoadsPerWave;
  constexpr int kXR = G::kXR, kXB = G::kXB, kPairs = G::kPairs, kFrags = G::kFrags;
  constexpr bool kGlu = ACT == 2;
  constexpr int kNOut = kGlu ? kBW / 2 : kBW;   // output columns per tile
  __shared__ __align__(1024) uint8_t lds[kLdsBytes];

  const int N = a.N;
  const int ntiles = (N + kNOut - 1) / kNOut;
  const int mt_max = static_cast<int>((a.rows_per_group + kBM - 1) / kBM);
  // blocks are dealt round-robin to the 8 XCDs: block b runs on XCD b%8 as
  // that XCD's (b/8)-th block.  XCD x takes the 32-tile chunks x, x+8, x+16,
  // ... in turn, so each XCD works on one chunk (4 row tiles x 8 column
  // tiles, sharing 4 token panels and 8 weight panels in its L2) at a time
  // and every XCD gets an even share of every expert.  The grid is a multiple
  // of 256 blocks.
  const int64_t p = blockIdx.x / 8;
  int64_t L = ((p / 32) * 8 + blockIdx.x % 8) * 32 + p % 32;
  // split k (bias-only GEMMs with too few tiles to fill the GPU): part ks of
  // the k range, float32 partial sums to kpart, summed by ksum_kernel
  int ks = 0;
  if (ACT == 0 && a.ksplit > 1) {
    const int64_t per_split = static_cast<int64_t>(a.groups) * mt_max * ntiles;
    ks = static_cast<int>(L / per_split);
    if (ks >= a.ksplit) return;
    L %= per_split;
  }
  TileCoord tc;
  int64_t rows_g, row_base;   // valid rows of the tile's group, and its first row
  // tail split: this block's part of its tile's k range and its partial tile
  int tail_slot = -1, kpart0 = 0, kpart_len = 0;
  if (a.packed || a.rows) {
    // Row counts on the device (the experts' kept rows; packed: laid back to
    // back).  The table sits at the start of the stage buffers (a second LDS
    // object would make the compiler order every direct-to-LDS load behind
    // the ones before it); L numbers only the tiles that hold rows, so the
    // blocks of empty tiles sit at the end of the grid instead of between the
    // chunks dealt to the XCDs.
    int* pk_start = reinterpret_cast<int*>(lds);
    int* pk_rows = pk_start + kMaxPackedGroups;
    int* pk_end = pk_rows + kMaxPackedGroups;
    build_tile_table(a, ntiles, pk_start, pk_rows, pk_end);
    __syncthreads();
    const int NT = pk_end[a.groups - 1];
    int Lt = static_cast<int>(L);
    if (ACT != 3 && a.tail_part) {
      const TailPlan tp = tail_plan(NT, a.K, a.tail_parts);
      if (L >= tp.F + static_cast<int64_t>(tp.R) * tp.P) return;
      if (L >= tp.F) {
        tail_slot = static_cast<int>(L) - tp.F;
        Lt = tp.F + tail_slot / tp.P;
        kpart0 = (tail_slot % tp.P) * tp.kslice;
        kpart_len = min(tp.kslice, a.K - kpart0);
      }
    } else if (L >= NT) {
      return;
    }
    tc = decode_dense(Lt, a.groups, ntiles, pk_end);
    rows_g = pk_rows[tc.g];
    row_base = a.packed ? static_cast<int64_t>(pk_start[tc.g]) : static_cast<int64_t>(tc.g) * a.rows_per_group;
    // every wave has read the table before the stage loads overwrite it
    __syncthreads();
  } else {
    tc = decode_tile(L, mt_max, ntiles, a.groups);
    if (!tc.valid) return;
    rows_g = a.rows_per_group;
    row_base = static_cast<int64_t>(tc.g) * a.rows_per_group;
  }
  const int m0 = tc.mt * kBM;
  if (m0 >= rows_g) return;
  const int n0 = tc.nt * kNOut;

  // token rows: contiguous per group, or gathered through a.gather (then A
  // is the whole [a_rows, K] input and row m of group g is A[gather[row_base
  // + m]], row_base = g*rpg, or the packed start)
  const bool gathered = a.gather != nullptr;

  // this tile's k range: [k0, k0 + K) of the operands' rows
  const int64_t k0 = tail_slot >= 0 ? kpart0 : static_cast<int64_t>(ks) * a.kslice;
  // (or, with kvar, the group's own k extent: its count rounded up to 8, the
  // operands being zero there; at least 8 so that an empty group sums zeros)
  const int K = tail_slot >= 0 ? kpart_len
                : ACT == 0 && a.ksplit > 1 ? static_cast<int>(min<int64_t>(a.kslice, a.K - k0))
                : a.kvar ? max(8, min(a.K, (max(a.kvar[tc.g], 0) + 7) / 8 * 8))
                         : a.K;
  // row strides (per-group packed blocks: the group's own k extent; a
  // k-major operand: the length of its k rows)
  const int64_t lda = kAkm ? a.lda : a.koff ? K : a.lda ? a.lda : a.K;
  const int64_t ldb = kBkm ? a.ldb : a.koff ? K : a.ldb ? a.ldb : a.K;
  // k rows of a k-major operand holding data (zeros from there)
  const int kdata = KM && a.kvar ? min(K, max(a.kvar[tc.g], 0)) : K;
  const bf16_t* A = static_cast<const bf16_t*>(a.A) +
                    (kAkm ? (a.kstart ? static_cast<int64_t>(a.kstart[tc.g]) * lda
                                      : static_cast<int64_t>(tc.g) * a.a_gs)
                     : k0 + (a.koff ? static_cast<int64_t>(a.koff[tc.g]) * a.rows_per_group
                             : gathered ? 0
                             : a.packed ? row_base * lda
                                        : static_cast<int64_t>(tc.g) * (a.a_gs ? a.a_gs : a.rows_per_group * lda)));
  const int64_t bg = kBkm ? (a.kstart ? static_cast<int64_t>(a.kstart[tc.g]) * ldb
                                      : static_cast<int64_t>(tc.g) * a.b_gs)
                          : (a.koff ? static_cast<int64_t>(a.koff[tc.g]) * N
                                    : static_cast<int64_t>(tc.g) * (a.b_gs ? a.b_gs : N * ldb)) + k0;
  const bf16_t* B0 = static_cast<const bf16_t*>(a.B0) + bg;
  const bf16_t* B1 = kGlu || (kBkm && a.B1) ? static_cast<const bf16_t*>(a.B1) + bg : B0;
  // k-major B stacked along k: stages at or past k row b_split read B1
  int b_split = kBkm && a.B1 ? static_cast<int>(a.b_split) : 1 << 30;
  if (kBkm && k0 > 0) {
    // a tail part's k range starts k0 rows in (a multiple of the stage, as
    // b_split is): the matrix holding row k0 starts there, and a stacked B
    // switches matrix b_split - k0 rows in (or holds B1 only)
    if (k0 < b_split) {
      B0 += k0 * ldb;
      b_split -= static_cast<int>(k0);
    } else {
      B1 += (k0 - b_split) * ldb;
      b_split = 0;
    }
  }

  const int tid = threadIdx.x;
  // the wave index is uniform: say so, so that descriptors and LDS bases live
  // in scalar registers
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // ---- staging: direct global -> LDS, 16 bytes per lane, 1 KiB per
  // wavefront instruction (kRowsPerLoad rows of kBK k).  The first kHalf
  // waves stage the 256 token rows, the others the 256 weight rows (for
  // SwiGLU the first 128 weight rows are gate rows, the rest the matching up
  // rows), kSRows rows each.  Lane i of an instruction fills LDS bytes
  // [16i, 16i+16) of its row block: row i/kChunks, physical chunk i%kChunks,
  // which holds logical k-chunk (i%kChunks) ^ swizzle(row).  Rows past the
  // operand's end (ragged expert rows, columns past N) and k past K read as
  // zero through the buffer bounds.
  const bool stage_x = wave < kHalf;
  // this wave's operand is k-major (bit 0: the token-row operand A, bit 1: B)
  const bool km = stage_x ? kAkm : kBkm;
  const int lr = lane / kChunks, pc = lane % kChunks;
  const int row0 = (wave % kHalf) * kSRows;        // first tile row this wave stages
  __amdgpu_buffer_rsrc_t rsrc, rsrc1;
  // voff: offset of each load's 16 bytes in stage 0; past: bit j set when
  // load j's k-chunk lies at or past K in the last stage (then bit 31 of its
  // offset is set, which sends it past every operand: it reads zero)
  uint32_t voff[kLoadsPerWave], past = 0;
  const int nk = (K + kBK - 1) / kBK;
  const int k_last = K - (nk - 1) * kBK;          // valid k in the last stage
  // k-major: k rows with data in the last stage
  const int kd_last = kdata - (nk - 1) * kBK;
  {
    const bf16_t* base = stage_x ? A : ((kGlu && row0 < 128) ? B1 : B0);
    const int64_t ld = stage_x ? lda : ldb;
    // rows of the operand (k-major: the contiguous dimension)
    const int64_t ext = stage_x ? (gathered ? a.a_rows : rows_g) : static_cast<int64_t>(N);
    // the operand's extent from its base: the last row ends K past its start
    // (k-major: the last k row with data ends ext past its start; a second
    // matrix stacked along k holds the rows from b_split on)
    const int64_t kd0 = km ? min(kdata, b_split) : 0, kd1 = km ? kdata - kd0 : 0;
    const int64_t nbytes = km ? (kd0 > 0 ? ((kd0 - 1) * ld + ext) * 2 : 0) : (ext - 1) * ld * 2 + K * 2;
    const int64_t nbytes1 = kd1 > 0 ? ((kd1 - 1) * ld + ext) * 2 : 0;
    // the descriptor must live in scalar registers: pin its fields to lane 0
    // (they are uniform; without this the compiler may not prove it and wrap
    // every load in a loop over lanes)
    auto make = [&](const bf16_t* b, int64_t n) {
      const uint64_t bu = reinterpret_cast<uint64_t>(b);
      const uint32_t blo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(bu));
      const uint32_t bhi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(bu >> 32));
      const int nrec = __builtin_amdgcn_readfirstlane(static_cast<int>(n));
      return __builtin_amdgcn_make_buffer_rsrc(
          reinterpret_cast<void*>((static_cast<uint64_t>(bhi) << 32) | blo), (short)0, nrec, kRsrcWord3);
    };
    rsrc = make(base, nbytes);
    rsrc1 = kBkm && !stage_x ? make(B1, nbytes1) : rsrc;
    // first operand row of this wave's block 0 (token rows: m0 + row0;
    // weight rows: n0 + row0, or for SwiGLU n0 + row0 mod 128 of its matrix)
    const int orow0 = stage_x ? m0 + row0 : (kGlu ? n0 + (row0 & 127) : n0 + row0);
    if (KM && km) {
      // k-major: the wave stages k rows [kw0, kw0 + 16) of each stage (16 x
      // 512 bytes, the same LDS bytes as its 64 tile rows otherwise).  Lane i
      // of instruction j fills k row kw0 + 2j + i/32, physical 16-byte chunk
      // i%32, which holds logical chunk (i%32) ^ ((k row & 3) << 2): tile
      // rows 8c .. 8c+7 of that k row.  Rows past the operand's end and k
      // rows past the data (last stage) read zero.
      const int kw0 = (wave % kHalf) * (kSRows / 4);
      const int rb = stage_x ? m0 : n0;
#pragma unroll
      for (int j = 0; j < kLoadsPerWave; ++j) {
        const int kk = kw0 + 2 * j + (lane >> 5);
        const int c = (lane & 31) ^ ((kk & 3) << 2);
        const int64_t orow = rb + c * 8;
        voff[j] = orow < ext ? static_cast<uint32_t>((kk * ld + orow) * 2) : kOutOfRange;
        past |= (kk < kd_last ? 0u : 1u) << j;
      }
    } else {
#pragma unroll
    for (int j = 0; j < kLoadsPerWave; ++j) {
      const int trow = row0 + j * kRowsPerLoad + lr;             // tile row (sets the swizzle)
      const int c = pc ^ ((trow >> kSwzShift) & (kChunks - 1));
      int orow = orow0 + j * kRowsPerLoad + lr;
      if (stage_x && gathered) {
        // gathered rows past rows_g read as zero; others come from their token
        orow = orow < rows_g ? a.gather[row_base + orow] : -1;
      }
      // weight rows past N (and token rows past rows_g) land past the
      // operand's extent and read as zero
      voff[j] = orow < 0 ? kOutOfRange : static_cast<uint32_t>((orow * ld + c * 8) * 2);
      past |= (c * 8 < k_last ? 0u : 1u) << j;
    }
    }
  }
  // bytes between consecutive stages of this wave's operand (the k offset
  // rides in the scalar offset), and the descriptor and scalar offset of
  // stage kc (a k-major B stacked along k switches matrix at b_split)
  const int64_t ld_w = stage_x ? lda : ldb;
  const int kstep = KM && km ? static_cast<int>(kBK * ld_w * 2) : kBK * 2;
  auto stage_src = [&](int kc, __amdgpu_buffer_rsrc_t& rs, int& so) __attribute__((always_inline)) {
    if (kBkm && !stage_x && kc * kBK >= b_split) {
      rs = rsrc1;
      so = (kc - b_split / kBK) * kstep;
    } else {
      rs = rsrc;
      so = kc * kstep;
    }
  };
  // the token rows' ring of kNX stage buffers, then the weight rows' ring of kNW
  const int nring = stage_x ? kNX : kNW;
  uint8_t* ring = lds + (stage_x ? 0 : kNX * kXBytes) + row0 * kRowBytes;

  // Stage s of a wave's operand goes to buffer s % nring of its ring; its k
  // offset goes in the scalar offset, so the bounds check sees the row
  // offset, which is what separates valid rows from the rest.  In the last
  // stage the loads flagged in `past` read zeros (k past K).  Stages past the
  // end re-read the last one into a buffer nobody multiplies, so every
  // iteration has the same shape and every wait count is a constant.
  //
  // Issue window.  Buffer s % nring is free once every wave has passed the
  // barrier of iteration s - nring (the barrier sits at the start of an
  // iteration's last 16-k step, after the step's fragments were read).  So
  // stage s is issued over kSteps positions: position 0 is that last step
  // of iteration s - nring, positions 1.. the first steps of iteration
  // s - nring + 1; its loads spread evenly over the first kLoadPos positions
  // (measured best: early enough to land, not one burst).
  auto issue_share = [&](int st, int j_begin, int j_end) {
    const int kc = min(st, nk - 1);
    const uint32_t pm = kc == nk - 1 ? past : 0u;
    uint8_t* dst = ring + (st % nring) * kXBytes;
    __amdgpu_buffer_rsrc_t rs;
    int soff;
    stage_src(kc, rs, soff);
    for (int j = j_begin; j < j_end; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(dst + j * 1024), 16,
                                               voff[j] | (((pm >> j) & 1u) << 31), soff, 0, 0);
  };

  // ---- fragments.  Wave (wn, wm) owns 128 weight rows (4 MFMA blocks of 32)
  // x kXR token rows (kXB blocks of 32).  Block i: weight rows wrow[i] (+
  // lane%32), output columns ncol[i]; for SwiGLU blocks 0-1 are gate rows,
  // 2-3 the matching up rows.  In a partial tile (fewer than 256 valid token
  // rows, or columns past N) a wave multiplies only its blocks that hold
  // valid token rows and weight rows below N (router logits use 4E of the
  // 256 weight rows).
  const int wn = wave & 1, wm = wave >> 1;
  const int valid_rows = static_cast<int>(min<int64_t>(rows_g - m0, kBM));
  const int xbv = max(0, min(kXB, (valid_rows - wm * kXR + 31) / 32));   // valid token blocks of this wave
  // weight blocks of this wave with a column below N (for SwiGLU a gate
  // block and its up block share their columns)
  const int wbv = kGlu ? max(0, min(2, (N - n0 - wn * 64 + 31) / 32)) : max(0, min(4, (N - n0 - wn * 128 + 31) / 32));
  // the predicated loop instance only for a wave that has blocks without
  // valid rows or columns: in a partial tile the waves whose blocks are all
  // valid run the plain loop (its MFMAs on rows past the valid ones would
  // only add zeros, and its stores stop at the valid rows anyway)
  const bool partial = xbv < kXB || wbv < (kGlu ? 2 : 4);
  int wrow[4], ncol[4], xrow[kXB];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ncol[i] = kGlu ? wn * 64 + (i & 1) * 32 : wn * 128 + i * 32;
    wrow[i] = (kGlu ? (i >> 1) * 128 + ncol[i] : ncol[i]) + (lane & 31);
  }
#pragma unroll
  for (int j = 0; j < kXB; ++j) xrow[j] = wm * kXR + j * 32 + (lane & 31);

  bf16x8_t wf[2][4], xf[2][kXB];
  auto xbuf = [&](int st) -> const uint8_t* { return lds + (st % kNX) * kXBytes; };
  auto wbuf = [&](int st) -> const uint8_t* { return lds + kNX * kXBytes + (st % kNW) * kWBytes; };
  // k-major stage: lane l of a 16-lane group g supplies the address of 4
  // consecutive tile rows of one k row, and the transpose load hands each
  // lane 4 consecutive k of its own row: with k row 8c + 4h + kmo and rows
  // rb + rco .. +3, lane l gets row rb + l%32, k 8c + 4h .. +3 (h = 0, 1:
  // the fragment's 8 k).  The rows' 16-byte chunk is swizzled by k row & 3
  // (= kmo) as the stage was written, so the 32 lanes served together hit
  // four distinct 64-byte bank windows.
  const int kmo = (lane & 15) >> 2, rco = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  // (The two reads wait for themselves in the same asm block: through the
  // builtin the compiler cannot tell them from reads of the stage the
  // direct-to-LDS loads are filling and waits for every load in flight first.)
  auto kread = [&](const uint8_t* buf, int rb, int c) __attribute__((always_inline)) {
    const int rowc = rb + rco;
    const int off = (8 * c + kmo) * (2 * kBM) + ((((rowc >> 3) ^ (kmo << 2))) << 4) + (rowc & 7) * 2;
    const uint32_t addr =
        static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const uint8_t*)(buf + off)));
    uint2 lo, hi;
    asm volatile(
        "ds_read_b64_tr_b16 %0, %2\n\t"
        "ds_read_b64_tr_b16 %1, %2 offset:2048\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(lo), "=&v"(hi)
        : "v"(addr)
        : "memory");
    return __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
  };
  // all four weight fragments of a k-major B at once (eight transpose reads,
  // one wait), written to wf[slot]
  auto kread_w4 = [&](const uint8_t* buf, int c, int slot) __attribute__((always_inline)) {
    uint32_t ad[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const int rowc = wrow[f] - (lane & 31) + rco;
      const int off = (8 * c + kmo) * (2 * kBM) + ((((rowc >> 3) ^ (kmo << 2))) << 4) + (rowc & 7) * 2;
      ad[f] = static_cast<uint32_t>(
          reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const uint8_t*)(buf + off)));
    }
    uint2 r[8];
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8\n\t"
        "ds_read_b64_tr_b16 %1, %8 offset:2048\n\t"
        "ds_read_b64_tr_b16 %2, %9\n\t"
        "ds_read_b64_tr_b16 %3, %9 offset:2048\n\t"
        "ds_read_b64_tr_b16 %4, %10\n\t"
        "ds_read_b64_tr_b16 %5, %10 offset:2048\n\t"
        "ds_read_b64_tr_b16 %6, %11\n\t"
        "ds_read_b64_tr_b16 %7, %11 offset:2048\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
        : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3])
        : "memory");
#pragma unroll
    for (int f = 0; f < 4; ++f)
      wf[slot][f] = __builtin_bit_cast(bf16x8_t, make_uint4(r[2 * f].x, r[2 * f].y, r[2 * f + 1].x, r[2 * f + 1].y));
  };
  // both token fragments of a k-major A at once (four transpose reads, one
  // wait), written to xf[slot]
  auto kread_x2 = [&](const uint8_t* buf, int c, int slot) __attribute__((always_inline)) {
    static_assert(kXB == 2, "two token fragments a step");
    uint32_t ad[2];
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      const int rowc = xrow[f] - (lane & 31) + rco;
      const int off = (8 * c + kmo) * (2 * kBM) + ((((rowc >> 3) ^ (kmo << 2))) << 4) + (rowc & 7) * 2;
      ad[f] = static_cast<uint32_t>(
          reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const uint8_t*)(buf + off)));
    }
    uint2 r[4];
    asm volatile(
        "ds_read_b64_tr_b16 %0, %4\n\t"
        "ds_read_b64_tr_b16 %1, %4 offset:2048\n\t"
        "ds_read_b64_tr_b16 %2, %5\n\t"
        "ds_read_b64_tr_b16 %3, %5 offset:2048\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
        : "v"(ad[0]), "v"(ad[1])
        : "memory");
#pragma unroll
    for (int f = 0; f < 2; ++f)
      xf[slot][f] = __builtin_bit_cast(bf16x8_t, make_uint4(r[2 * f].x, r[2 * f].y, r[2 * f + 1].x, r[2 * f + 1].y));
  };
  auto read_frag = [&](const uint8_t* xs, const uint8_t* ws, int c, int slot, int f) {
    if (f < 4) {
      if (kBkm) wf[slot][f] = kread(ws, wrow[f] - (lane & 31), c);
      else wf[slot][f] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(ws + swz(wrow[f], c)));
    } else {
      if (kAkm) xf[slot][f - 4] = kread(xs, xrow[f - 4] - (lane & 31), c);
      else xf[slot][f - 4] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(xs + swz(xrow[f - 4], c)));
    }
  };

  f32x16_t acc[4][kXB];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < kXB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // ---- epilogue: lane holds, for block (i, j), output columns
  // ncol[i] + 8q + 4*(lane/32) + {0..3} of token row xrow[j] (tile-relative).
  // Each loop instance has its own copy, so that the accumulators of the two
  // are never merged into one set of registers.
  auto store_tile = [&]() __attribute__((always_inline)) {
    // the stages issued past the end are still landing
    __builtin_amdgcn_s_waitcnt(0);
    if (ACT == 3) {
      // router planes: columns n..n+3 are the three exact partial products
      // of one expert (and a zero row); their sum is the logit
      float* Cf = static_cast<float*>(a.C) +
                  static_cast<int64_t>(tc.g) * (a.c_gs ? a.c_gs : a.rows_per_group * (N / 4));
#pragma unroll
      for (int j = 0; j < kXB; ++j) {
        const int64_t m = m0 + xrow[j];
        if (m >= rows_g) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int n = n0 + ncol[i] + 8 * q + 4 * (lane >> 5);
            if (n >= N) continue;
            Cf[m * (N / 4) + (n >> 2)] =
                ((acc[i][j][4 * q] + acc[i][j][4 * q + 1]) + acc[i][j][4 * q + 2]) + acc[i][j][4 * q + 3];
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      return;
    }
    if (ACT != 3 && tail_slot >= 0) {
      // tail split: this part's float32 sums as a [256 x 256] partial tile,
      // column = the tile's weight row (SwiGLU: gate rows 0..127, up rows
      // 128..255); no bias or activation yet
      float* P = a.tail_part + static_cast<int64_t>(tail_slot) * (kBM * kBW);
#pragma unroll
      for (int j = 0; j < kXB; ++j) {
        const int m = xrow[j];
        if (m0 + m >= rows_g) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int n = ncol[i] + 8 * q + 4 * (lane >> 5);
            if (n0 + n >= N) continue;
            const int wr = (kGlu ? (i >> 1) * 128 : 0) + n;
            *reinterpret_cast<float4*>(P + m * kBW + wr) =
                make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      return;
    }
    if (ACT == 0 && a.ksplit > 1) {
      // split k: this part's float32 sums, four consecutive columns a lane
      float* P = a.kpart + static_cast<int64_t>(ks) * a.kpart_stride + row_base * N;
#pragma unroll
      for (int j = 0; j < kXB; ++j) {
        const int64_t m = m0 + xrow[j];
        if (m >= rows_g) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int n = n0 + ncol[i] + 8 * q + 4 * (lane >> 5);
            if (n >= N) continue;
            *reinterpret_cast<float4*>(P + m * N + n) =
                make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      return;
    }
    // Output through LDS, 32 token rows at a time per wave: the finished
    // bf16 values go to the wave's own LDS region, come back row-contiguous
    // and leave as whole row segments (16 bytes per lane, kOut*2 contiguous
    // bytes per row).  Stored straight from the MFMA layout, one instruction
    // would write 8 bytes into each of 32 rows, and the L2 would take many
    // more, smaller write requests.
    const bf16_t* bias = a.bias ? static_cast<const bf16_t*>(a.bias) + static_cast<int64_t>(tc.g) * N : nullptr;
    constexpr int kOut = kGlu ? 64 : 128;              // output columns per wave
    constexpr int kPitch = kOut * 2 + 16;              // padded LDS row (bytes)
    constexpr int kLanesPerRow = kOut * 2 / 16;
    constexpr int kRowsPerInst = kWave / kLanesPerRow;
    static_assert(kWaves * 32 * kPitch <= kLdsBytes, "epilogue staging must fit the stage buffers");
    __syncthreads();                                   // every wave is done with the stage buffers
    uint8_t* scr = lds + wave * 32 * kPitch;
    const int colw = wn * kOut;                        // the wave's first tile column
    // what = 0: the activated output into C; 1: the pre-activation (GELU:
    // a w^T + b; SwiGLU: the gate projection) into pre0; 2: the SwiGLU up
    // projection into pre1 (outputs kept for a backward pass)
    auto emit = [&](bf16_t* dst, int what) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < kXB; ++j) {
        const int rowbase = wm * kXR + j * 32;
        if (m0 + rowbase >= rows_g) break;
#pragma unroll
        for (int i = 0; i < (kGlu ? 2 : 4); ++i) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int col = ncol[i] - colw + 8 * q + 4 * (lane >> 5);
            const int n = n0 + ncol[i] + 8 * q + 4 * (lane >> 5);
            // the bias of columns n .. n+3 in one 8-byte load (N is a
            // multiple of 8 and n of 4, so the four are all below N or all
            // past it; the entry points require 16-byte aligned biases)
            float bb[4] = {0.0f, 0.0f, 0.0f, 0.0f};
            if (!kGlu && bias && n < N) {
              const uint2 u = *reinterpret_cast<const uint2*>(bias + n);
              bb[0] = __uint_as_float(u.x << 16);
              bb[1] = __uint_as_float(u.x & 0xFFFF0000u);
              bb[2] = __uint_as_float(u.y << 16);
              bb[3] = __uint_as_float(u.y & 0xFFFF0000u);
            }
            f32x2_t v[2];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              float x = acc[i][j][4 * q + r];
              if (ACT == 2) {
                if (what == 0) x = silu_fast(x) * acc[i + 2][j][4 * q + r];
                else if (what == 2) x = acc[i + 2][j][4 * q + r];
              } else {
                x += bb[r];
                if (ACT == 1 && what == 0) x = gelu_fast(x);
              }
              v[r >> 1][r & 1] = x;
            }
            // hardware round-to-nearest-even conversion, two values at a time
            uint2 packed;
            packed.x = __builtin_bit_cast(uint32_t, __builtin_convertvector(v[0], bf16x2_t));
            packed.y = __builtin_bit_cast(uint32_t, __builtin_convertvector(v[1], bf16x2_t));
            *reinterpret_cast<uint2*>(scr + (lane & 31) * kPitch + col * 2) = packed;
          }
          // one block at a time: keeps the accumulators' copies out of the
          // VGPRs until they are needed
          __builtin_amdgcn_sched_barrier(0);
        }
        // the wave reads back only what it wrote itself
#pragma unroll
        for (int pp = 0; pp < 32 / kRowsPerInst; ++pp) {
          const int row = pp * kRowsPerInst + lane / kLanesPerRow;
          const int ch = lane % kLanesPerRow;
          const uint4 v = *reinterpret_cast<const uint4*>(scr + row * kPitch + ch * 16);
          const int64_t m = m0 + rowbase + row;
          const int n = n0 + colw + ch * 8;
          // N is a multiple of 8: a segment is wholly inside or wholly past it
          if (m < rows_g && n < N) *reinterpret_cast<uint4*>(dst + m * N + n) = v;
        }
      }
    };
    emit(static_cast<bf16_t*>(a.C) + row_base * N, 0);
    if (ACT != 0 && a.pre0) {
      emit(static_cast<bf16_t*>(a.pre0) + row_base * N, 1);
      if (ACT == 2) emit(static_cast<bf16_t*>(a.pre1) + row_base * N, 2);
    }
  };

  // ---- pipeline.  Iteration kt multiplies stage kt.  Its last 16-k step
  // waits for the wave's own loads of stage kt+1, meets the other waves at
  // the barrier, and starts reading stage kt+1's first fragments.  At that
  // barrier the loads a wave may still have in flight are the whole stages
  // of its operand issued after stage kt+1 (nring - 2 of them).
  constexpr int kSteps = kBK / 16;
  static_assert(kSteps % 2 == 0, "fragment slots alternate per 16-k step");
  constexpr int kLoadPos = kLoadPositions < kSteps ? kLoadPositions : kSteps;
  static_assert(kNX >= 2 && kNW >= 2, "two stages at least");
  // loads of window position p: [pos_begin(p), pos_begin(p + 1))
  auto pos_begin = [](int p) { return p >= kLoadPos ? kLoadsPerWave : (kLoadsPerWave * p) / kLoadPos; };
  auto wait_own = [&]() {
    if (stage_x) __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0((kNX - 2) * kLoadsPerWave));
    else __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0((kNW - 2) * kLoadsPerWave));
  };
  // prologue: stages 0 .. nring-2 whole and position 0 of stage nring-1;
  // then stage 0 must have landed: each wave waits for its own stage-0 loads
  // only (loads complete in order; the later stages stay in flight)
  for (int st = 0; st < nring - 1; ++st) issue_share(st, 0, kLoadsPerWave);
  issue_share(nring - 1, 0, pos_begin(1));
  if (stage_x) __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0((kNX - 2) * kLoadsPerWave + pos_begin(1)));
  else __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0((kNW - 2) * kLoadsPerWave + pos_begin(1)));
  __builtin_amdgcn_s_barrier();
  {
    const int c0 = lane >> 5;
#pragma unroll
    for (int f = 0; f < kFrags; ++f) read_frag(xbuf(0), wbuf(0), c0, 0, f);
  }
  // Each 16-k step runs as kPairs fenced groups of two MFMAs, the step's
  // share of the next step's fragment reads and of the loads, so that no
  // burst of loads or reads holds up the MFMAs.  A partial tile skips the
  // MFMAs of blocks without valid token rows or weight rows.
  auto run = [&](auto partial_c) __attribute__((always_inline)) {
    constexpr bool kPartial = decltype(partial_c)::value;
    int rk = 0;                                       // kt % nring
    for (int kt = 0; kt < nk; ++kt) {
      const int rk_prev = rk == 0 ? nring - 1 : rk - 1;
#pragma unroll
      for (int ks = 0; ks < kSteps; ++ks) {
        const int cur = ks & 1;
        const bool next_stage = ks + 1 == kSteps;
        if (next_stage) {
          __builtin_amdgcn_sched_barrier(0);
          wait_own();
          __builtin_amdgcn_s_barrier();
          __builtin_amdgcn_sched_barrier(0);
        }
        // loads of this step: window position p of stage ist
        const int p = next_stage ? 0 : ks + 1;
        const int ist = next_stage ? kt + nring : kt + nring - 1;
        const int j0 = pos_begin(p), nload = pos_begin(p + 1) - j0;
        const int kc = min(ist, nk - 1);
        const uint32_t pm = kc == nk - 1 ? past : 0u;
        // buffer ist % nring: kt % nring at position 0, (kt - 1) % nring after
        uint8_t* dst = ring + (next_stage ? rk : rk_prev) * kXBytes;
        __amdgpu_buffer_rsrc_t rs;
        int soff;
        stage_src(kc, rs, soff);
        const int rstage = next_stage ? kt + 1 : kt;
        const uint8_t* rx = xbuf(rstage);
        const uint8_t* rw = wbuf(rstage);
        const int rc = (next_stage ? 0 : ks + 1) * 2 + (lane >> 5);
#pragma unroll
        for (int q = 0; q < kPairs; ++q) {
          const int i = (2 * q) / kXB, jb = (2 * q) % kXB;
          const bool wvalid = (kGlu ? (i & 1) : i) < wbv;
          if (!kPartial || (jb < xbv && wvalid))
            acc[i][jb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[cur][i], xf[cur][jb], acc[i][jb], 0, 0, 0);
          if (!kPartial || (jb + 1 < xbv && wvalid))
            acc[i][jb + 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[cur][i], xf[cur][jb + 1], acc[i][jb + 1], 0, 0, 0);
          // (a k-major B: its four fragments at once, in the first group)
          // (and a k-major A: its two, in the last group)
          if (kBkm && q == 0) kread_w4(rw, rc, cur ^ 1);
          if (kAkm && q == kPairs - 1) kread_x2(rx, rc, cur ^ 1);
#pragma unroll
          for (int r = 0; r < kFrags; ++r)
            if (kPlanOf<W>.group[r] == q && !(kBkm && kPlanOf<W>.order[r] < 4) && !(kAkm && kPlanOf<W>.order[r] >= 4))
              read_frag(rx, rw, rc, cur ^ 1, kPlanOf<W>.order[r]);
          // this step's loads, spread over the groups
#pragma unroll
          for (int u = 0; u < kLoadsPerWave; ++u) {
            if (u < nload && (u * kPairs) / nload == q) {
              const int j = j0 + u;
              __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(dst + j * 1024), 16,
                                                       voff[j] | (((pm >> j) & 1u) << 31), soff, 0, 0);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      rk = rk + 1 == nring ? 0 : rk + 1;
    }
    store_tile();
  };
  if (!partial) run(std::false_type{});
  else run(std::true_type{});
}

// The bf16 kernel: 8 wavefronts, one workgroup per compute unit (LDS).
template <int ACT>
__global__ __launch_bounds__(512, 1) void gemm_bf16_w8(GemmArgs a) {
  gemm_bf16_body<ACT, 8>(a);
}
// The same, bias only, with k-major operands (GemmArgs.kmaj = KM).
template <int KM>
__global__ __launch_bounds__(512, 1) void gemm_bf16_km(GemmArgs a) {
  gemm_bf16_body<0, 8, KM>(a);
}

// ------------------------------------------------------------------ float32
constexpr int kFT = 32;   // 32 x 32 output tile, 256 threads x 4 outputs

template <int ACT>
__global__ __launch_bounds__(kThreads) void gemm_f32_kernel(GemmArgs a) {
  __shared__ float as[kFT][kFT + 1];
  __shared__ float bs[2][kFT][kFT + 1];
  const int N = a.N, K = a.K;
  const int ntiles = (N + kFT - 1) / kFT;
  const int mt_max = static_cast<int>((a.rows_per_group + kFT - 1) / kFT);
  const int64_t L = blockIdx.x;
  const int g = static_cast<int>(L / (static_cast<int64_t>(mt_max) * ntiles));
  if (g >= a.groups) return;
  const int r = static_cast<int>(L % (static_cast<int64_t>(mt_max) * ntiles));
  const int mt = r / ntiles, nt = r % ntiles;
  int64_t rows_g = a.rows ? min<int64_t>(a.rows[g], a.rows_per_group) : a.rows_per_group;
  int64_t row_base = static_cast<int64_t>(g) * a.rows_per_group;
  if (a.packed) {
    // packed rows: the group starts after the rows of the lower groups
    // (each capped so that none reaches past total_rows)
    int64_t start = 0;
    for (int h = 0; h < g; ++h) start += max(a.rows[h], 0);
    start = min(start, a.total_rows);
    row_base = start;
    rows_g = max<int64_t>(0, min<int64_t>(max(a.rows[g], 0), a.total_rows - start));
  }
  const int m0 = mt * kFT, n0 = nt * kFT;
  if (m0 >= rows_g) return;
  const bool gathered = a.gather != nullptr;
  const float* A = static_cast<const float*>(a.A) + (gathered ? 0 : row_base * K);
  const int32_t* grow = gathered ? a.gather + row_base : nullptr;
  const float* B0 = static_cast<const float*>(a.B0) + static_cast<int64_t>(g) * N * K;
  const float* B1 = ACT == 2 ? static_cast<const float*>(a.B1) + static_cast<int64_t>(g) * N * K : nullptr;
  const int tx = threadIdx.x % kFT, ty = threadIdx.x / kFT;   // ty 0..7
  float acc0[4] = {0, 0, 0, 0}, acc1[4] = {0, 0, 0, 0};
  for (int k0 = 0; k0 < K; k0 += kFT) {
    __syncthreads();
    for (int i = threadIdx.x; i < kFT * kFT; i += kThreads) {
      const int rr = i / kFT, cc = i % kFT;
      const int64_t m = m0 + rr;
      const int n = n0 + rr;
      const int kk = k0 + cc;
      const int64_t ar = (m < rows_g && gathered) ? grow[m] : m;
      as[rr][cc] = (m < rows_g && kk < K) ? A[ar * K + kk] : 0.0f;
      bs[0][rr][cc] = (n < N && kk < K) ? B0[static_cast<int64_t>(n) * K + kk] : 0.0f;
      if (ACT == 2) bs[1][rr][cc] = (n < N && kk < K) ? B1[static_cast<int64_t>(n) * K + kk] : 0.0f;
    }
    __syncthreads();
#pragma unroll 4
    for (int kk = 0; kk < kFT; ++kk) {
      const float b0 = bs[0][tx][kk];
      const float b1 = ACT == 2 ? bs[1][tx][kk] : 0.0f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float av = as[ty + 8 * q][kk];
        acc0[q] += av * b0;
        if (ACT == 2) acc1[q] += av * b1;
      }
    }
  }
  float* C = static_cast<float*>(a.C) + row_base * N;
  const float* bias = a.bias ? static_cast<const float*>(a.bias) + static_cast<int64_t>(g) * N : nullptr;
  const int n = n0 + tx;
  if (n >= N) return;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t m = m0 + ty + 8 * q;
    if (m >= rows_g) continue;
    float v = acc0[q];
    if (ACT == 2) {
      v = silu(acc1[q]) * v;          // B0 = up, B1 = gate
    } else {
      if (bias) v += bias[n];
      if (ACT == 1) v = gelu_erf(v);
    }
    C[m * N + n] = v;
  }
}

}  // namespace

template <int ACT>
void launch_bf16(const GemmArgs& a, unsigned grid, hipStream_t s) {
  if (ACT == 0 && a.kmaj == 1) gemm_bf16_km<1><<<grid, 512, 0, s>>>(a);
  else if (ACT == 0 && a.kmaj == 2) gemm_bf16_km<2><<<grid, 512, 0, s>>>(a);
  else if (ACT == 0 && a.kmaj == 3) gemm_bf16_km<3><<<grid, 512, 0, s>>>(a);
  else gemm_bf16_w8<ACT><<<grid, 512, 0, s>>>(a);
}

namespace {
// Split k: C[row] = bf16(sum over the parts, in order, of kpart + bias) for
// the valid rows of every group, 8 columns a thread.
__global__ __launch_bounds__(kThreads) void ksum_kernel(GemmArgs a) {
  const int64_t c8 = a.N / 8;
  const int64_t item = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (item >= static_cast<int64_t>(a.groups) * a.rows_per_group * c8) return;
  const int64_t row = item / c8, c = (item % c8) * 8;
  const int g = static_cast<int>(row / a.rows_per_group);
  const int64_t r = row % a.rows_per_group;
  if (a.rows && r >= a.rows[g]) return;
  float v[8] = {};
  for (int s = 0; s < a.ksplit; ++s) {
    const float4* q = reinterpret_cast<const float4*>(a.kpart + s * a.kpart_stride + row * a.N + c);
    const float4 x0 = q[0], x1 = q[1];
    v[0] += x0.x; v[1] += x0.y; v[2] += x0.z; v[3] += x0.w;
    v[4] += x1.x; v[5] += x1.y; v[6] += x1.z; v[7] += x1.w;
  }
  if (a.bias) {
    const bf16_t* b = static_cast<const bf16_t*>(a.bias) + static_cast<int64_t>(g) * a.N + c;
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] += bf16_to_f32(b[q]);
  }
  uint32_t w[4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
    w[q] = static_cast<uint32_t>(f32_to_bf16(v[2 * q])) | (static_cast<uint32_t>(f32_to_bf16(v[2 * q + 1])) << 16);
  *reinterpret_cast<uint4*>(static_cast<bf16_t*>(a.C) + row * a.N + c) = make_uint4(w[0], w[1], w[2], w[3]);
}

// Tail split: tile F + t of the tail = act(sum over its parts, in part order,
// of the float32 partial tiles + bias), rounded to bf16, for its valid rows
// and columns (with the pre-activations when kept); the plan is recomputed
// from the same device row counts.  Block b sums rows
// [(b % kTailSlices) * 32, + 32) of tail tile t = b / kTailSlices, so the
// partial tiles stream through many compute units; each thread issues the
// loads of every part before the first add.
constexpr int kTailSlices = kBM / 32;
template <int ACT>
__global__ __launch_bounds__(kThreads) void tail_sum_kernel(GemmArgs a) {
  constexpr bool kGlu = ACT == 2;
  constexpr int kNOut = kGlu ? kBW / 2 : kBW;
  __shared__ int tab[3 * kMaxPackedGroups];
  int* pk_start = tab;
  int* pk_rows = tab + kMaxPackedGroups;
  int* pk_end = tab + 2 * kMaxPackedGroups;
  const int N = a.N;
  const int ntiles = (N + kNOut - 1) / kNOut;
  build_tile_table(a, ntiles, pk_start, pk_rows, pk_end);
  __syncthreads();
  const TailPlan tp = tail_plan(pk_end[a.groups - 1], a.K, a.tail_parts);
  const int t = blockIdx.x / kTailSlices;
  const int r0 = (blockIdx.x % kTailSlices) * 32;
  if (t >= tp.R) return;
  const TileCoord tc = decode_dense(tp.F + t, a.groups, ntiles, pk_end);
  const int m0 = tc.mt * kBM, n0 = tc.nt * kNOut;
  const int vr = min(kBM, pk_rows[tc.g] - m0), vc = min(kNOut, N - n0);
  const int64_t row_base = a.packed ? static_cast<int64_t>(pk_start[tc.g]) : static_cast<int64_t>(tc.g) * a.rows_per_group;
  const bf16_t* bias = a.bias ? static_cast<const bf16_t*>(a.bias) + static_cast<int64_t>(tc.g) * N + n0 : nullptr;
  const int64_t obase = (row_base + m0) * N + n0;
  auto pack = [](const float (&v)[8]) {
    uint32_t w[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      w[u] = static_cast<uint32_t>(f32_to_bf16(v[2 * u])) | (static_cast<uint32_t>(f32_to_bf16(v[2 * u + 1])) << 16);
    return make_uint4(w[0], w[1], w[2], w[3]);
  };
  constexpr int kMaxParts = kMaxTailParts;  // launch_gemm clamps the parts to it
  for (int i = threadIdx.x; i < 32 * (kNOut / 8); i += kThreads) {
    const int r = r0 + i / (kNOut / 8), c = (i % (kNOut / 8)) * 8;
    if (r >= vr || c >= vc) continue;
    const float* src0 = a.tail_part + static_cast<int64_t>(t) * tp.P * (kBM * kBW) + r * kBW + c;
    float4 x[kMaxParts][2], y[kMaxParts][2];
#pragma unroll
    for (int p = 0; p < kMaxParts; ++p) {
      if (p < tp.P) {
        const float* src = src0 + static_cast<int64_t>(p) * (kBM * kBW);
        x[p][0] = reinterpret_cast<const float4*>(src)[0];
        x[p][1] = reinterpret_cast<const float4*>(src)[1];
        if (kGlu) {
          y[p][0] = reinterpret_cast<const float4*>(src + 128)[0];
          y[p][1] = reinterpret_cast<const float4*>(src + 128)[1];
        }
      }
    }
    float v[8] = {}, u[8] = {};
#pragma unroll
    for (int p = 0; p < kMaxParts; ++p) {
      if (p < tp.P) {
        v[0] += x[p][0].x; v[1] += x[p][0].y; v[2] += x[p][0].z; v[3] += x[p][0].w;
        v[4] += x[p][1].x; v[5] += x[p][1].y; v[6] += x[p][1].z; v[7] += x[p][1].w;
        if (kGlu) {
          u[0] += y[p][0].x; u[1] += y[p][0].y; u[2] += y[p][0].z; u[3] += y[p][0].w;
          u[4] += y[p][1].x; u[5] += y[p][1].y; u[6] += y[p][1].z; u[7] += y[p][1].w;
        }
      }
    }
    if (!kGlu && bias) {
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] += bf16_to_f32(bias[c + q]);
    }
    const int64_t o = obase + static_cast<int64_t>(r) * N + c;
    if (ACT != 0 && a.pre0) {
      *reinterpret_cast<uint4*>(static_cast<bf16_t*>(a.pre0) + o) = pack(v);
      if (kGlu) *reinterpret_cast<uint4*>(static_cast<bf16_t*>(a.pre1) + o) = pack(u);
    }
    float out[8];
#pragma unroll
    for (int q = 0; q < 8; ++q)
      out[q] = ACT == 2 ? silu_fast(v[q]) * u[q] : ACT == 1 ? gelu_fast(v[q]) : v[q];
    *reinterpret_cast<uint4*>(static_cast<bf16_t*>(a.C) + o) = pack(out);
  }
}
}  // namespace

hipError_t launch_gemm(const GemmArgs& a_in, int dtype, hipStream_t s) {
  GemmArgs a = a_in;
  // the tail split applies to bf16 GEMMs over device row counts (k-major:
  // only B, read from the part's first k row on, with every group's k range
  // the full K)
  const bool tail = dtype == MOE_BF16 && a.act != 3 && a.tail_part != nullptr && a.rows != nullptr &&
                    !(a.ksplit > 1) && a.tail_parts >= 2 && a.K / kTailMinK >= 2 &&
                    (a.kmaj == 0 || (a.kmaj == 2 && !a.kvar && !a.kstart));
  // (a K below two minimum parts never splits: no extra blocks, no sum launch)
  if (!tail) a.tail_part = nullptr;
  a.tail_parts = min(a.tail_parts, kMaxTailParts);
  if (a.groups <= 0 || a.rows_per_group <= 0 || a.N <= 0) return hipSuccess;
  if (a.kmaj) {
    // k-major operands: bias-only bf16; a k-major A neither packed nor
    // gathered; per-group blocks (koff) only for a K-contiguous B; row
    // lengths given; a stacked B switching matrix at a stage boundary
    if (dtype != MOE_BF16 || a.act != 0 || a.kmaj > 3 || ((a.kmaj & 1) && (a.packed || a.gather)) ||
        a.ksplit > 1 || (a.koff && a.kmaj != 1) ||
        ((a.kmaj & 1) && a.lda <= 0) || ((a.kmaj & 2) && a.ldb <= 0) ||
        ((a.kmaj & 2) && a.B1 && (a.b_split <= 0 || a.b_split % kBK != 0)) || a.N % 8 != 0 ||
        ((a.kmaj & 1) && a.rows_per_group % 8 != 0))
      return hipErrorInvalidValue;
  }
  if (dtype == MOE_BF16) {
    const int nout = a.act == 2 ? kBW / 2 : kBW;
    if ((a.packed || a.rows) && a.groups > kMaxPackedGroups) return hipErrorInvalidValue;
    // packed rows: the groups' row tiles number at most total/256 + groups
    const int64_t row_tiles = a.packed ? (a.total_rows + kBM - 1) / kBM + a.groups
                                       : static_cast<int64_t>(a.groups) * ((a.rows_per_group + kBM - 1) / kBM);
    const bool split = a.act == 0 && a.ksplit > 1 && !a.packed;
    const int64_t tiles = row_tiles * ((a.N + nout - 1) / nout) * (split ? a.ksplit : 1);
    // (tail split: up to 256 more blocks for the parts of the last round's tiles)
    const unsigned grid = static_cast<unsigned>((tiles + 255) / 256 * 256 + (tail ? kCUs : 0));
    switch (a.act) {
      case 0: launch_bf16<0>(a, grid, s); break;
      case 1: launch_bf16<1>(a, grid, s); break;
      case 2: launch_bf16<2>(a, grid, s); break;
      default: launch_bf16<3>(a, grid, s); break;
    }
    if (tail) {
      const unsigned tgrid = kCUs / 2 * kTailSlices;  // tail_plan keeps R <= kCUs / 2
      if (a.act == 0) tail_sum_kernel<0><<<tgrid, kThreads, 0, s>>>(a);
      else if (a.act == 1) tail_sum_kernel<1><<<tgrid, kThreads, 0, s>>>(a);
      else tail_sum_kernel<2><<<tgrid, kThreads, 0, s>>>(a);
    }
    if (split) {
      const int64_t items = static_cast<int64_t>(a.groups) * a.rows_per_group * (a.N / 8);
      ksum_kernel<<<static_cast<unsigned>((items + kThreads - 1) / kThreads), kThreads, 0, s>>>(a);
    }
  } else {
    const int64_t tiles = static_cast<int64_t>(a.groups) * ((a.rows_per_group + kFT - 1) / kFT) *
                          ((a.N + kFT - 1) / kFT);
    const unsigned grid = static_cast<unsigned>(tiles);
    switch (a.act) {
      case 0: gemm_f32_kernel<0><<<grid, kThreads, 0, s>>>(a); break;
      case 1: gemm_f32_kernel<1><<<grid, kThreads, 0, s>>>(a); break;
      default: gemm_f32_kernel<2><<<grid, kThreads, 0, s>>>(a); break;
    }
  }
  return hipGetLastError();
}

}  // namespace moe
