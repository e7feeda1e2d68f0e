// Vocabulary loss behind a linear LM head, without a [T, V] logit matrix,
// for MI355X (gfx950).
//
// The logits z = X W^T (hidden X [T, H], head weight W [V, H], both bf16) are
// produced tile by tile on the matrix cores (v_mfma_f32_32x32x16_bf16, fp32
// accumulation) and consumed in the tile's epilogue:
//  * forward: each workgroup walks a range of vocabulary tiles for 256 rows and
//    keeps per-row online (shift, sum) statistics of the non-target columns and
//    the target logit; ce_rows_finish merges the ranges in fp64 into the loss
//    and the saved per-row state (the collapse-free loss of torchtitan PR #5661,
//    revised PR description, Numerics; the split over vocabulary ranges is its
//    vocabulary-parallel merge, third review inline diff);
//  * backward, per chunk of vocabulary columns: the logit tiles of every row
//    are recomputed and turned into G = dL/dz from the saved state (approving
//    review, "What this PR does": rebuild the softmax, put the target gradient
//    in its slot, scale), written as bf16 in both orientations for that chunk
//    only; then the chunk's rows of dW = G^T X and its share of dX += G W run
//    on the same matrix-core kernel, with operands that fit the last-level
//    cache.
// Every product is C = A B^T with both operands K-contiguous; X^T and the
// chunk's W^T are formed by a transpose kernel so that dX and dW take that
// form.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>

#include "ce_fused.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBM = 256;          // tile rows (A rows)
constexpr int kBN = 256;          // tile columns (B rows)
#ifndef LM_BK
#define LM_BK 64
#endif
#ifndef LM_STAGES
#define LM_STAGES 2
#endif
constexpr int kBK = LM_BK;        // K per LDS stage (32 or 64)
constexpr int kStages = LM_STAGES;  // LDS ring: kStages - 1 stages in flight while one is consumed
constexpr int kCPR = kBK / 8;     // 16-byte chunks per row of a stage
#ifndef LM_WAVES
#define LM_WAVES 8
#endif
// Waves per workgroup: 4 (2 x 2, each 128 x 128 = 4 x 4 MFMA blocks) or 8
// (4 x 2, each 64 x 128 = 2 x 4 blocks, two waves per SIMD).
constexpr int kWaves = LM_WAVES;
constexpr int kThreads = 64 * kWaves;
constexpr int kWM = kWaves / 2;               // waves along M (2 along N)
constexpr int kRW = kBM / kWM;                // rows per wave
constexpr int kMI = kRW / 32;                 // MFMA blocks per wave along M
constexpr int kNI = 4;                        // ... along N (128 columns)
constexpr int kLoadsPerStage = 2 * kBM * kCPR / kThreads;   // buffer loads per thread per stage
constexpr int kChunks = kBM * kBK / 8;   // 16-byte chunks per operand stage (1024)
constexpr int kRowState = 8;
constexpr float kL2E = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr uint32_t kOutOfRange = 0x80000000u;   // a buffer offset past every operand window

// LDS: a ring of stages of both operands as 16-byte chunks; chunk c of row r
// sits at r * kCPR + (c ^ ((r / (16 / kCPR)) % kCPR)). A 128-bit LDS read is
// served 16 lanes (256 bytes, all 64 banks) at a time, and the 16 rows that 16
// consecutive lanes read then land on 16 distinct 16-byte bank groups.
// The statistics kernel reuses it for its final merge of the wave rows.
struct Stages {
  u32x4 a[kStages][kChunks];
  u32x4 b[kStages][kChunks];
};
__device__ __forceinline__ int swz(int row, int kc) {
  return row * kCPR + (kc ^ ((row / (16 / kCPR)) % kCPR));
}

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// (a, b) rounded to bf16 (nearest even), a in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2 f = {a, b};
  const bf16x2 h = __builtin_convertvector(f, bf16x2);
  return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ uint16_t to_bf16(float f) {
  // round to nearest even; NaN stays NaN
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// A row-major bf16 operand [rows, ld] with K contiguous.
struct Operand {
  const uint16_t* p;
  int64_t rows;
  int64_t ld;
};

struct GemmParams {
  Operand a, b;
  int64_t M, N, K;
  int32_t tiles_m, tiles_n;   // tiles of the problem
  int32_t n_ranges;           // statistics: vocabulary ranges (grid = tiles_m * n_ranges)
  // statistics
  const int64_t* targets;     // [M] targets of the A rows
  float* stats;               // [n_ranges, M, 3]
  // gradient
  const float* row_state;     // [M, 8] state of the A rows
  float grad_scale;
  int64_t v0;                 // vocabulary index of B row 0 (targets are global)
  uint16_t* g;                // [M, ld_g] row-major G of this column chunk
  int64_t ld_g;
  uint16_t* gt;               // [tiles_n * kBN, ld_gt] transposed G
  int64_t ld_gt;
  int64_t zero_rows;          // rows >= this (within the chunk) are written as 0
  // store
  void* c;
  int64_t ld_c;
  int32_t accumulate;
};

// Buffer window over the tile's rows [r0, r0 + 256) of an operand: loads past
// its last row or with an offset of kOutOfRange read as zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t window(const Operand& o, int64_t r0) {
  const int64_t rows = o.rows - r0 < kBM ? o.rows - r0 : kBM;
  const uint32_t bytes = rows > 0 ? static_cast<uint32_t>(rows * o.ld * 2) : 0u;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(o.p + (rows > 0 ? r0 * o.ld : 0)),
                                           0, bytes, 0x00020000);
}

// One K stage of one operand, HBM -> LDS without registers: wave w fills row
// groups i * kWaves + w (64 / kCPR rows each); lane l of a group loads row
// g * 64 / kCPR + l / kCPR and the chunk that swz places at LDS chunk 64 g + l.
template <bool KMASK>
__device__ __forceinline__ void load_operand(__amdgpu_buffer_rsrc_t rsrc, const Operand& o,
                                             int64_t K, int64_t k0, u32x4* stage) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < kBM * kCPR / kThreads; ++i) {
    const int grp = i * kWaves + wave;
    const int row = grp * (64 / kCPR) + lane / kCPR;
    const int kc = (lane % kCPR) ^ ((row / (16 / kCPR)) % kCPR);
    const int64_t k = k0 + kc * 8;
    const uint32_t off = (!KMASK || k < K) ? static_cast<uint32_t>((row * o.ld + k) * 2) : kOutOfRange;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rsrc, (__attribute__((address_space(3))) void*)(stage + grp * 64), 16, off, 0, 0, 0);
  }
}

// Wait until at most n stages of this thread's loads are still in flight
// (loads complete in issue order; vmcnt is an immediate).
// s_waitcnt immediate for vmcnt(n) with no wait on the other counters.
constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

__device__ __forceinline__ void wait_stages_left(int64_t n) {
  if constexpr (kStages >= 4) {
    if (n >= 2) {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * kLoadsPerStage));
      return;
    }
  }
  if constexpr (kStages >= 3) {
    if (n >= 1) {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(kLoadsPerStage));
      return;
    }
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
}
static_assert(kStages <= 4 && 2 * kLoadsPerStage <= 63, "vmcnt holds the loads in flight");

// acc[mi][ni] covers rows wm*kRW + mi*32 + {8(q/4) + 4(lane/32) + q%4} and
// column wn*128 + ni*32 + lane%32 of the tile (q = register index 0..15).
// KMASK: K is not a multiple of kBK, so the last stage masks its tail.
// The first kStages - 1 stages of a tile's operands, issued ahead of its
// products (by tile_product itself, or earlier by the caller with
// PREISSUED set, once no wave reads the stages any more).
template <bool KMASK>
__device__ __forceinline__ void issue_first_stages(const GemmParams& p, Stages& s, int64_t m0,
                                                   int64_t n0) {
  const __amdgpu_buffer_rsrc_t ra = window(p.a, m0), rb = window(p.b, n0);
  const int64_t nk = (p.K + kBK - 1) / kBK;
  for (int64_t j = 0; j < kStages - 1 && j < nk; ++j) {
    load_operand<KMASK>(ra, p.a, p.K, j * kBK, s.a[j]);
    load_operand<KMASK>(rb, p.b, p.K, j * kBK, s.b[j]);
  }
}

// Stage 0 alone, with no test of K (with K = 0 the products never read it):
// what PREISSUED expects of a two-stage ring, issued unconditionally.
template <bool KMASK>
__device__ __forceinline__ void issue_stage0(const GemmParams& p, Stages& s, int64_t m0, int64_t n0) {
  static_assert(kStages == 2, "one stage ahead");
  load_operand<KMASK>(window(p.a, m0), p.a, p.K, 0, s.a[0]);
  load_operand<KMASK>(window(p.b, n0), p.b, p.K, 0, s.b[0]);
}

template <bool KMASK, bool PREISSUED = false>
__device__ __forceinline__ void tile_product(const GemmParams& p, Stages& s, int64_t m0,
                                             int64_t n0, f32x16 (&acc)[kMI][kNI]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[mi][ni][q] = 0.f;

  const __amdgpu_buffer_rsrc_t ra = window(p.a, m0), rb = window(p.b, n0);
  const int64_t nk = (p.K + kBK - 1) / kBK;
  // prologue: stages 0 .. kStages - 2 in flight, wait for stage 0
  if (!PREISSUED) issue_first_stages<KMASK>(p, s, m0, n0);
  wait_stages_left(std::min<int64_t>(kStages - 2, nk - 1));
  __syncthreads();
  for (int64_t kt = 0; kt < nk; ++kt) {
    const int slot = static_cast<int>(kt % kStages);
    const int64_t ahead = kt + kStages - 1;
    if (ahead < nk) {
      const int ws = static_cast<int>(ahead % kStages);
      load_operand<KMASK>(ra, p.a, p.K, ahead * kBK, s.a[ws]);
      load_operand<KMASK>(rb, p.b, p.K, ahead * kBK, s.b[ws]);
    }
    const u32x4* sa = s.a[slot];
    const u32x4* sb = s.b[slot];
    // the stage's fragments; the compiler interleaves their reads with the
    // products (pinning all reads first, or double-buffering them per k-step,
    // measured slower on MI355X)
    bf16x8 af[kBK / 16][kMI], bfr[kBK / 16][kNI];
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      const int kc = ks * 2 + (lane >> 5);
#pragma unroll
      for (int mi = 0; mi < kMI; ++mi)
        af[ks][mi] = __builtin_bit_cast(bf16x8, sa[swz(wm * kRW + mi * 32 + (lane & 31), kc)]);
#pragma unroll
      for (int ni = 0; ni < kNI; ++ni)
        bfr[ks][ni] = __builtin_bit_cast(bf16x8, sb[swz(wn * 128 + ni * 32 + (lane & 31), kc)]);
    }
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks)
#pragma unroll
      for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
        for (int ni = 0; ni < kNI; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks][mi], bfr[ks][ni], acc[mi][ni],
                                                                0, 0, 0);
    // stage kt + 1 must have landed: the stages after it may stay in flight
    wait_stages_left(std::min<int64_t>(kStages - 2, std::max<int64_t>(0, nk - 2 - kt)));
    __syncthreads();
  }
}

// Merge a (shift, sum) partial in log2 units into (mL, s); -inf shifts carry
// no mass.
__device__ __forceinline__ void merge(float& mL, float& s, float m2, float s2) {
  const float mn = fmaxf(mL, m2);
  if (mn == kNegInf) return;
  s = (mL == kNegInf ? 0.f : s * fexp2(mL - mn)) + (m2 == kNegInf ? 0.f : s2 * fexp2(m2 - mn));
  mL = mn;
}

// Statistics: grid = tiles_m * n_ranges; each workgroup walks the vocabulary
// tiles of one range for 256 rows. Row tiles in groups of 8 go with ranges in
// fours: the 32 workgroups an XCD runs at once take 8 row tiles by 4 ranges,
// so each weight slice of a K stage is shared through L2 by 8 of them and
// each hidden slice by 4 (otherwise range = block % n_ranges, which gives the
// same sharing for n_ranges a multiple of 32). The products are
// formed transposed, C^T = W X^T, so that a lane holds few rows (4: row m0 +
// wn * 128 + ni * 32 + lane % 32) and many vocabulary columns of each (32 per
// tile: wm * 64 + mi * 32 + 8 (q / 4) + 4 (lane / 32) + q % 4), and keeps the
// rows' online (shift, sum) statistics in registers across the range; lanes and
// waves holding the same rows are merged once at the end. The next tile's
// first stage is in flight while a tile's statistics are formed. A tile takes
// the masked path only when a row's target lies among a wave's columns or the
// tile passes the vocabulary's end.
// The statistics grid in groups of 8 row tiles by 4 ranges (the 32
// workgroups an XCD runs at once), a whole number of groups per XCD.
__host__ __device__ inline bool grouped_ranges(int64_t tiles_m, int64_t n_ranges) {
  return tiles_m % 8 == 0 && n_ranges % 4 == 0 && (tiles_m / 8) * (n_ranges / 4) % 8 == 0;
}

template <bool KMASK>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWaves / 4, kWaves / 4))) void lm_stats_kernel(
    GemmParams p) {
  static_assert(kWaves == 8 && kMI == 2, "statistics layout: 8 waves of 64 x 128");
  __shared__ __align__(16) Stages s;
  int range, mt;
  if (grouped_ranges(p.tiles_m, p.n_ranges)) {
    // XCD x = block % 8 takes groups x, x + 8, ... of 8 row tiles by 4
    // ranges, the 32 workgroups of a group together
    const int x = blockIdx.x % 8, l = blockIdx.x / 8;
    const int k = (l / 32) * 8 + x, q4 = p.n_ranges / 4;
    mt = 8 * (k / q4) + l % 8;
    range = 4 * (k % q4) + (l / 8) % 4;
  } else {
    range = blockIdx.x % p.n_ranges;
    mt = blockIdx.x / p.n_ranges;
  }
  // ranges of tiles_n / n_ranges tiles, rounded down or up
  const int64_t nt0 = range * static_cast<int64_t>(p.tiles_n) / p.n_ranges;
  const int64_t nt1 = (range + 1) * static_cast<int64_t>(p.tiles_n) / p.n_ranges;
  const int64_t m0 = static_cast<int64_t>(mt) * kBM;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  // operands swapped: weight rows on the matrix-core rows, hidden rows on its columns
  GemmParams q = p;
  q.a = p.b;
  q.b = p.a;
  int64_t t[kNI];
  float mL[kNI], sum[kNI], zt[kNI];
#pragma unroll
  for (int ni = 0; ni < kNI; ++ni) {
    const int64_t gr = m0 + wn * 128 + ni * 32 + (lane & 31);
    t[ni] = gr < p.M ? p.targets[gr] : -1;
    mL[ni] = kNegInf;
    sum[ni] = 0.f;
    zt[ni] = kNegInf;
  }
  const int vrow = wm * 64 + 4 * (lane >> 5);   // + mi * 32 + 8 (q / 4) + q % 4
  f32x16 acc[kMI][kNI];
  if (nt0 < nt1) issue_stage0<KMASK>(q, s, nt0 * kBN, m0);
  for (int64_t nt = nt0; nt < nt1; ++nt) {
    const int64_t n0 = nt * kBN;
    tile_product<KMASK, true>(q, s, n0, m0, acc);
    if (nt + 1 < nt1) issue_stage0<KMASK>(q, s, n0 + kBN, m0);
    const int64_t w0 = n0 + wm * 64;
    bool hit = false;
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni) hit |= t[ni] >= w0 && t[ni] < w0 + 64;
    const bool masked = __builtin_amdgcn_ballot_w64(hit) != 0 || n0 + kBN > p.N;
    if (masked) {
      // the target's logit is taken out of the sum, columns past the vocabulary count nothing
#pragma unroll
      for (int ni = 0; ni < kNI; ++ni) {
        const int64_t tl = t[ni] - (n0 + vrow);
        const int64_t cend = p.N - (n0 + vrow);
#pragma unroll
        for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int c = mi * 32 + 8 * (e >> 2) + (e & 3);
            const float v = acc[mi][ni][e];
            if (c == tl) zt[ni] = v;
            acc[mi][ni][e] = (c < cend && c != tl) ? v : kNegInf;
          }
      }
    }
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni) {
      float gmax = acc[0][ni][0];
#pragma unroll
      for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
        for (int e = 0; e < 16; ++e) gmax = fmaxf(gmax, acc[mi][ni][e]);
      const float mn = fmaxf(mL[ni], gmax * kL2E);
      if (mn != kNegInf) {
        float a = 0.f;
#pragma unroll
        for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
          for (int e = 0; e < 16; ++e) a += fexp2(__builtin_fmaf(acc[mi][ni][e], kL2E, -mn));
        sum[ni] = (mL[ni] == kNegInf ? 0.f : sum[ni] * fexp2(mL[ni] - mn)) + a;
        mL[ni] = mn;
      }
    }
  }
  // lanes l and l ^ 32 hold the same rows
#pragma unroll
  for (int ni = 0; ni < kNI; ++ni) {
    const float m2 = __shfl_xor(mL[ni], 32, 64);
    const float s2 = __shfl_xor(sum[ni], 32, 64);
    const float z2 = __shfl_xor(zt[ni], 32, 64);
    merge(mL[ni], sum[ni], m2, s2);
    zt[ni] = fmaxf(zt[ni], z2);
  }
  // the four wave rows wm hold the same rows: merged through LDS in a fixed order
  float (*red)[kBM][3] = reinterpret_cast<float (*)[kBM][3]>(&s);
  __syncthreads();
  if (lane < 32) {
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni) {
      float* r = red[wm][wn * 128 + ni * 32 + lane];
      r[0] = mL[ni];
      r[1] = sum[ni];
      r[2] = zt[ni];
    }
  }
  __syncthreads();
  if (threadIdx.x < kBM) {
    const int row = threadIdx.x;
    float m = red[0][row][0], sm = red[0][row][1], z = red[0][row][2];
#pragma unroll
    for (int w = 1; w < kWM; ++w) {
      merge(m, sm, red[w][row][0], red[w][row][1]);
      z = fmaxf(z, red[w][row][2]);
    }
    const int64_t gr = m0 + row;
    if (gr < p.M) {
      float* st = p.stats + 3 * (static_cast<int64_t>(range) * p.M + gr);
      st[0] = m;
      st[1] = sm;
      st[2] = z;
    }
  }
}

// Tile order of the one-tile-per-workgroup kernels. Tiles are grouped 8 along
// M by 4 along N (32 tiles: the workgroups an XCD runs at once), groups M
// fastest; blocks are dealt to the 8 XCDs in turn (XCD x gets blocks x,
// x + 8, ...), and each XCD gets one contiguous run of groups. The 32
// workgroups of an XCD then read 8 A and 4 B tile slices per K stage, each
// shared through its L2 by 4 or 8 of them (M-fastest runs of single tiles
// shared one B slice but read 32 different A slices).
constexpr int kGM = 8, kGN = 4;

__host__ __device__ inline int64_t tile_slots(int64_t tiles_m, int64_t tiles_n) {
  return (tiles_m + kGM - 1) / kGM * kGM * ((tiles_n + kGN - 1) / kGN * kGN);
}

__device__ __forceinline__ void tile_of_id(const GemmParams& p, int64_t bid, int64_t& m0,
                                           int64_t& n0, bool& live) {
  // 32-bit arithmetic: the host launches at most INT32_MAX blocks
  const int slots = static_cast<int>(tile_slots(p.tiles_m, p.tiles_n));
  const int per = (slots + 7) / 8;
  const int b = static_cast<int>(bid);
  const int id = (b % 8) * per + b / 8;
  const int gms = (p.tiles_m + kGM - 1) / kGM;
  const int g = id / (kGM * kGN), r = id % (kGM * kGN);
  const int mt = (g % gms) * kGM + r % kGM, nt = (g / gms) * kGN + r / kGM;
  live = id < slots && mt < p.tiles_m && nt < p.tiles_n;
  m0 = static_cast<int64_t>(mt) * kBM;
  n0 = static_cast<int64_t>(nt) * kBN;
}

__device__ __forceinline__ void tile_of_block(const GemmParams& p, int64_t& m0, int64_t& n0,
                                              bool& live) {
  tile_of_id(p, blockIdx.x, m0, n0, live);
}

// Persistent walk over the block ids of the one-tile-per-workgroup order:
// workgroup b takes ids b, b + gridDim.x, ... (gridDim.x a multiple of 8
// keeps every id on the XCD it is dealt to, and with 256 workgroups the 32 of
// an XCD take one group of tiles at a time). Advances id to the next live
// tile; false when none is left.
__device__ __forceinline__ bool next_tile(const GemmParams& p, int64_t& id, int64_t& m0,
                                          int64_t& n0) {
  const int64_t nblocks = (tile_slots(p.tiles_m, p.tiles_n) + 7) / 8 * 8;
  for (; id < nblocks; id += gridDim.x) {
    bool live;
    tile_of_id(p, id, m0, n0, live);
    if (live) return true;
  }
  return false;
}

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// 4 x 4 transpose of bf16 values over the lanes of a quad: lane k holds row k
// as (p0 = {x0, x1}, p1 = {x2, x3}); afterwards it holds column k, row j's
// element in position j. Two lane-pair exchanges (DPP quad permutations).
__device__ __forceinline__ void quad_transpose(uint32_t& p0, uint32_t& p1, int quad) {
  constexpr int kXor1 = 0xB1, kXor2 = 0x4E;   // quad_perm (1,0,3,2) and (2,3,0,1)
  const uint32_t r0 = static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(p0), kXor1, 0xF, 0xF, false));
  const uint32_t r1 = static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(p1), kXor1, 0xF, 0xF, false));
  // even lane: (own low, partner low); odd lane: (partner high, own high)
  const bool odd = quad & 1;
  const uint32_t a0 = odd ? ((r0 >> 16) | (p0 & 0xffff0000u)) : ((p0 & 0xffffu) | (r0 << 16));
  const uint32_t a1 = odd ? ((r1 >> 16) | (p1 & 0xffff0000u)) : ((p1 & 0xffffu) | (r1 << 16));
  // lanes 0, 1 keep a0 and take a0 of lanes 2, 3; lanes 2, 3 take a1 of lanes 0, 1 and keep a1
  const bool upper = quad & 2;
  const uint32_t send = upper ? a0 : a1;
  const uint32_t recv = static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(send), kXor2, 0xF, 0xF, false));
  p0 = upper ? recv : a0;
  p1 = upper ? a1 : recv;
}

// Gradient tiles of one column chunk: G = dL/dz for all rows and the chunk's
// vocabulary columns, written row-major and transposed. Persistent over the
// tiles (next_tile); the logits are formed transposed, C^T = W_chunk X^T, so a
// lane holds four rows (m0 + wn * 128 + ni * 32 + lane % 32) and, per row,
// runs of four adjacent columns (wm * 64 + mi * 32 + 8 g + 4 (lane / 32) +
// 0..3): a 4 x 4 transpose over the quad of lanes holding four adjacent rows
// turns each run into one 8-byte store into G^T, and lanes l and l + 32 trade
// runs so that each stores eight adjacent columns of G (16 bytes). The next
// tile's first stage is in flight while a tile's gradient is formed and
// stored.
template <bool KMASK>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWaves / 4, kWaves / 4))) void lm_grad_kernel(
    GemmParams p) {
  static_assert(kWaves == 8 && kMI == 2, "gradient layout: 8 waves of 64 x 128");
  __shared__ __align__(16) Stages s;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1, quad = lane & 3;
  GemmParams q = p;   // weight rows of the chunk on the matrix-core rows
  q.a = p.b;
  q.b = p.a;
  int64_t id = blockIdx.x, m0, n0;
  if (!next_tile(p, id, m0, n0)) return;
  issue_stage0<KMASK>(q, s, n0, m0);
  const int vrow = wm * 64 + 4 * (lane >> 5);   // + mi * 32 + 8 g + 0..3
  while (true) {
    f32x16 acc[kMI][kNI];
    tile_product<KMASK, true>(q, s, n0, m0, acc);
    int64_t idn = id + gridDim.x, m0n = 0, n0n = 0;
    const bool more = next_tile(p, idn, m0n, n0n);
    if (!more) {
      m0n = m0;   // the last tile's stage is issued again (unused): an unconditional
      n0n = n0;   // issue keeps the waits below for the row factors only
    }
    // the rows' factors, loaded before the next tile's stage so that waiting
    // for them leaves its copies in flight
    float kl[kNI], cnt[kNI], gtv[kNI], fill[kNI];
    int64_t tl[kNI];
    bool live[kNI];
    {
      // all loads first (rows past zero_rows read the last row and are not used)
      f32x4 sa[kNI], sb[kNI];
      int64_t tg[kNI];
#pragma unroll
      for (int ni = 0; ni < kNI; ++ni) {
        const int64_t gr = m0 + wn * 128 + ni * 32 + (lane & 31);
        const int64_t grc = gr < p.zero_rows ? gr : p.zero_rows - 1;
        const f32x4* rs = reinterpret_cast<const f32x4*>(p.row_state + kRowState * grc);
        sa[ni] = rs[0];
        sb[ni] = rs[1];
        tg[ni] = p.targets[grc];
      }
#pragma unroll
      for (int ni = 0; ni < kNI; ++ni) {
        const int64_t gr = m0 + wn * 128 + ni * 32 + (lane & 31);
        const bool in = gr < p.zero_rows;
        const float kind = sb[ni][1];   // rs[5]
        const float zw = p.grad_scale * sb[ni][0];   // rs[4]
        live[ni] = in && kind == 0.f;
        kl[ni] = sa[ni][0];
        cnt[ni] = (zw + zw * sa[ni][3]) * fexp2(-sb[ni][2]);   // rs[6]: rounding residue of rs[0]
        gtv[ni] = -zw * sa[ni][1] + zw * sa[ni][3] * sa[ni][2];
        tl[ni] = tg[ni] - p.v0 - (n0 + vrow);   // target's offset from the lane's first column
        fill[ni] = (!in || kind == 1.f) ? 0.f : __builtin_nanf("");
      }
    }
    issue_stage0<KMASK>(q, s, n0n, m0n);
    bool hit = false;
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni) hit |= live[ni] && tl[ni] >= 0 && tl[ni] < 64;
    const bool masked = __builtin_amdgcn_ballot_w64(hit) != 0 || n0 + kBN > p.N;
    const int64_t cend = p.N - (n0 + vrow);   // columns at or past this offset are outside the chunk
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni) {
      const int64_t row = m0 + wn * 128 + ni * 32 + (lane & 31);
#pragma unroll
      for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
        for (int g2 = 0; g2 < 4; g2 += 2) {
          // two runs of four columns: 8 g4 + 4 (lane / 32) + 0..3, g4 = g2, g2 + 1
          uint32_t pk[2][2];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int g4 = g2 + h;
            float gv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int c = mi * 32 + 8 * g4 + e;
              float x = cnt[ni] * fexp2(__builtin_fmaf(acc[mi][ni][4 * g4 + e], kL2E, -kl[ni]));
              if (masked) x = (c == tl[ni]) ? gtv[ni] : x;
              x = live[ni] ? x : fill[ni];
              if (masked) x = (c < cend) ? x : 0.f;
              gv[e] = x;
            }
            // rounded to bf16 in pairs (v_cvt_pk_bf16_f32, RNE)
            pk[h][0] = pack_bf16x2(gv[0], gv[1]);
            pk[h][1] = pack_bf16x2(gv[2], gv[3]);
            uint32_t t0 = pk[h][0], t1 = pk[h][1];
            quad_transpose(t0, t1, quad);
            const int64_t col = n0 + vrow + mi * 32 + 8 * g4;
            const u32x2 colv = {t0, t1};
            *reinterpret_cast<u32x2*>(p.gt + (col + quad) * p.ld_gt + (row - quad)) = colv;
          }
          // G: lane l < 32 takes the upper half's first run (columns 8 g2 + 4..7)
          // and gives it its second run (8 g2 + 8..11): then lane l stores
          // columns 8 g2 + 0..7 and lane l + 32 columns 8 g2 + 8..15 of the
          // same row, 16 bytes each
          const auto s0 = __builtin_amdgcn_permlane32_swap(pk[0][0], pk[1][0], false, false);
          const auto s1 = __builtin_amdgcn_permlane32_swap(pk[0][1], pk[1][1], false, false);
          const int64_t col = n0 + wm * 64 + mi * 32 + 8 * g2 + 8 * (lane >> 5);
          const u32x4 rowv = {s0[0], s1[0], s0[1], s1[1]};
          *reinterpret_cast<u32x4*>(p.g + row * p.ld_g + col) = rowv;
        }
    }
    if (!more) break;
    id = idn;
    m0 = m0n;
    n0 = n0n;
  }
  // the unused stage has landed before the workgroup's LDS is released
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
}

// Plain product C = A B^T (fp32, optionally accumulated into C).
template <bool KMASK>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWaves / 4, kWaves / 4))) void lm_store_kernel(
    GemmParams p) {
  __shared__ __align__(16) Stages s;
  int64_t m0, n0;
  bool live_tile;
  tile_of_block(p, m0, n0, live_tile);
  if (!live_tile) return;
  f32x16 acc[kMI][kNI];
  tile_product<KMASK>(p, s, m0, n0, acc);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni) {
      const int64_t col = n0 + wn * 128 + ni * 32 + (lane & 31);
      const int64_t row0 = m0 + wm * kRW + mi * 32 + 4 * (lane >> 5);
      // the 16 old values of a block are loaded before any is stored, so
      // the loads are in flight together
      float old[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int64_t row = row0 + 8 * (q >> 2) + (q & 3);
        const bool in = col < p.N && row < p.M;
        old[q] = (in && p.accumulate) ? static_cast<const float*>(p.c)[row * p.ld_c + col] : 0.f;
      }
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int64_t row = row0 + 8 * (q >> 2) + (q & 3);
        if (col >= p.N || row >= p.M) continue;
        static_cast<float*>(p.c)[row * p.ld_c + col] = old[q] + acc[mi][ni][q];
      }
    }
}

// out[c, r] = in[r, c] for r < R, c < C; out[c, r] = 0 for R <= r < Rp.
// 64 x 64 tiles through LDS, moved as runs of eight elements (16 bytes) where
// the run lies inside the rows; grid (Rp / 64, ceil(C / 64)). Rp, ld_in and
// ld_out are multiples of 8 and both bases 16-byte aligned.
__global__ __launch_bounds__(256) void lm_transpose_kernel(const uint16_t* __restrict__ in,
                                                           int64_t R, int64_t C, int64_t ld_in,
                                                           uint16_t* __restrict__ out, int64_t Rp,
                                                           int64_t ld_out) {
  __shared__ __align__(16) uint16_t tile[64][72];   // 144-byte rows: every run 16-byte aligned
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * 64, c0 = static_cast<int64_t>(blockIdx.y) * 64;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = threadIdx.x + 256 * i;
    const int row = q >> 3, cc = (q & 7) * 8;
    const int64_t r = r0 + row, c = c0 + cc;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (r < R && c + 8 <= C) {
      v = *reinterpret_cast<const u32x4*>(in + r * ld_in + c);
    } else if (r < R) {
      uint16_t e[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) e[k] = c + k < C ? in[r * ld_in + c + k] : static_cast<uint16_t>(0);
#pragma unroll
      for (int k = 0; k < 4; ++k) v[k] = static_cast<uint32_t>(e[2 * k]) | (static_cast<uint32_t>(e[2 * k + 1]) << 16);
    }
    *reinterpret_cast<u32x4*>(&tile[row][cc]) = v;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = threadIdx.x + 256 * i;
    const int oc = q >> 3, rr = (q & 7) * 8;
    const int64_t c = c0 + oc;
    if (c >= C) continue;
    u32x4 v;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      v[k] = static_cast<uint32_t>(tile[rr + 2 * k][oc]) | (static_cast<uint32_t>(tile[rr + 2 * k + 1][oc]) << 16);
    *reinterpret_cast<u32x4*>(out + c * ld_out + r0 + rr) = v;
  }
}

// lse from the saved state: lse = (state[0] + state[6]) / log2(e) for valid
// rows, 0 for ignored rows, NaN for poisoned ones.
__global__ __launch_bounds__(256) void lm_lse_kernel(const float* __restrict__ row_state,
                                                     int64_t T, float* __restrict__ lse) {
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (r >= T) return;
  const float* rs = row_state + kRowState * r;
  lse[r] = rs[5] == 0.f ? static_cast<float>((static_cast<double>(rs[0]) + static_cast<double>(rs[6])) /
                                              static_cast<double>(kL2E))
                        : (rs[5] == 1.f ? 0.f : __builtin_nanf(""));
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

struct LmLayout {
  int64_t chunk;        // vocabulary columns per backward chunk (multiple of 256)
  int64_t t_pad;        // rows rounded up to a tile (K of dW)
  int64_t n_ranges, tiles_m_all, tiles_n;
  size_t off_stats, off_state, off_g, off_gt, off_wt, off_xt, off_dx, total;
};

int64_t chunk_cols_of(const ce_lmhead* p) {
  const int64_t c = p->chunk_cols > 0 ? p->chunk_cols : 8192;
  return round_up(std::min<int64_t>(c, std::max<int64_t>(p->V, 1)), kBN);
}

LmLayout layout(const ce_lmhead* p, bool backward, bool dx32) {
  LmLayout L{};
  L.chunk = chunk_cols_of(p);
  L.t_pad = round_up(std::max<int64_t>(p->T, 1), kBM);
  L.tiles_n = (p->V + kBN - 1) / kBN;
  L.tiles_m_all = (p->T + kBM - 1) / kBM;
  // A power-of-two number of ranges, about eight workgroups per compute unit
  // in all (2048 = 8 x 256 CUs, run one at a time per CU): the 32 workgroups
  // an XCD runs at once (block % 8) then cover 32 / (n_ranges / 8) row tiles
  // of n_ranges / 8 ranges, sharing both operands' slices through L2 (with
  // one range per XCD they read 32 row tiles' slices; 32 ranges measured 9%
  // faster at T = 16384). Where the row tiles come in groups of 8, fewer and
  // longer ranges in fours instead, each workgroup one whole range: at
  // T = 16384, 4 ranges of 125 or 126 tiles, one workgroup per CU, against 32
  // ranges of 16 tiles with a 5-tile last one (14.5 -> 13.7 ms).
  const int64_t tm = std::max<int64_t>(L.tiles_m_all, 1);
  const int64_t want = (2048 + tm - 1) / tm;
  int64_t nr = 1;
  while (nr < want && nr < L.tiles_n) nr *= 2;
  L.n_ranges = std::min<int64_t>(nr, L.tiles_n);
  // With row tiles in groups of 8: ranges in fours, as few as give one
  // workgroup per compute unit (256), each a whole range of balanced length
  if (tm % 8 == 0) {
    for (int64_t q4 = 1; 4 * q4 <= L.tiles_n; ++q4) {
      if (!grouped_ranges(tm, 4 * q4)) continue;
      if (tm * 4 * q4 >= 256 || 4 * (q4 + 1) > L.tiles_n) {
        L.n_ranges = 4 * q4;
        break;
      }
    }
  }
  size_t off = 0;
  L.off_stats = off;
  off += align_up(static_cast<size_t>(L.n_ranges) * p->T * 3 * sizeof(float));
  L.off_state = off;
  off += align_up(static_cast<size_t>(p->T) * kRowState * sizeof(float));
  if (backward) {
    const size_t H = static_cast<size_t>(p->H);
    L.off_g = off;     // G of a chunk [t_pad, chunk]
    off += align_up(static_cast<size_t>(L.t_pad) * L.chunk * 2);
    L.off_gt = off;    // G^T of a chunk [chunk, t_pad]
    off += align_up(static_cast<size_t>(L.chunk) * L.t_pad * 2);
    L.off_wt = off;    // W^T of a chunk [H, chunk]
    off += align_up(H * L.chunk * 2);
    L.off_xt = off;    // X^T [H, t_pad]
    off += align_up(H * L.t_pad * 2);
    L.off_dx = off;    // fp32 dX accumulator when dX is bf16
    if (dx32) off += align_up(static_cast<size_t>(p->T) * H * 4);
  }
  L.total = off;
  return L;
}

bool aligned16(const void* ptr, int64_t ld) {
  return (reinterpret_cast<uintptr_t>(ptr) % 16 == 0) && (ld % 8 == 0);
}

bool overlaps(const void* a, size_t an, const void* b, size_t bn) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a && b && an && bn && a0 < b0 + bn && b0 < a0 + an;
}

// One-tile-per-workgroup kernels get 8 * ceil(slots / 8) blocks: the grouped
// XCD mapping of tile_of_block covers every tile only then (blocks of padding
// slots exit).
int64_t tile_blocks(int64_t tiles_m, int64_t tiles_n) {
  return (tile_slots(tiles_m, tiles_n) + 7) / 8 * 8;
}

// Compute units of the current device (cached per device); -1 on error.
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return -1;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return -1;
  cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Workgroups of a persistent tile walk over `blocks` block ids: one per
// compute unit (a workgroup's LDS stages fill a CU), a multiple of 8 so that
// every id stays on the XCD it is dealt to.
int64_t persistent_blocks(int64_t blocks) {
  const int cus = device_cus();
  if (cus <= 0) return -1;
  return std::min<int64_t>(blocks, std::max(8, cus / 8 * 8));
}

ce_status launch(void (*kern)(GemmParams), int64_t blocks, const GemmParams& gp, hipStream_t st) {
  if (blocks <= 0) return CE_OK;
  if (blocks > INT32_MAX) return CE_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, st, gp);
  return hipGetLastError() == hipSuccess ? CE_OK : CE_ERR_HIP;
}

// The kernel instance for gp.K: K-tail masking only when K is not a multiple
// of the stage depth.
template <template <bool> class Sel>
ce_status launch_k(int64_t blocks, const GemmParams& gp, hipStream_t st) {
  return gp.K % kBK == 0 ? launch(Sel<false>::fn, blocks, gp, st) : launch(Sel<true>::fn, blocks, gp, st);
}
template <bool KM> struct StatsSel { static constexpr void (*fn)(GemmParams) = lm_stats_kernel<KM>; };
template <bool KM> struct GradSel { static constexpr void (*fn)(GemmParams) = lm_grad_kernel<KM>; };
template <bool KM> struct StoreSel { static constexpr void (*fn)(GemmParams) = lm_store_kernel<KM>; };

ce_status launch_transpose(const uint16_t* in, int64_t R, int64_t C, int64_t ld_in, uint16_t* out,
                           int64_t Rp, int64_t ld_out, hipStream_t st) {
  hipLaunchKernelGGL(lm_transpose_kernel,
                     dim3(static_cast<unsigned>(Rp / 64), static_cast<unsigned>((C + 63) / 64)),
                     dim3(256), 0, st, in, R, C, ld_in, out, Rp, ld_out);
  return hipGetLastError() == hipSuccess ? CE_OK : CE_ERR_HIP;
}

__global__ __launch_bounds__(256) void lm_zero_kernel(float* __restrict__ out, int64_t n) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * 256)
    out[i] = 0.f;
}

// fp32 [n] -> bf16 [n], round to nearest even.
__global__ __launch_bounds__(256) void lm_to_bf16_kernel(const float* __restrict__ in, int64_t n,
                                                         uint16_t* __restrict__ out) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * 256)
    out[i] = to_bf16(in[i]);
}

}  // namespace

extern "C" {

size_t ce_lmhead_workspace_bytes(const ce_lmhead* p, int32_t backward) {
  if (p == nullptr || p->T < 0 || p->V < 1 || p->H < 1) return 0;
  return layout(p, backward != 0, p->dhidden_dtype == CE_DTYPE_BF16).total;
}

ce_status ce_lmhead_fwd_bwd(const ce_lmhead* p, const void* hidden, const void* weight,
                            const int64_t* targets, const uint8_t* mask, float z_alpha,
                            float grad_scale, float* loss_out, float* lse_out, void* dhidden,
                            float* dweight, void* workspace, size_t workspace_bytes,
                            void* stream_ptr) {
  if (p == nullptr) return CE_ERR_INVALID_ARG;
  const int64_t T = p->T, V = p->V, H = p->H;
  if (T < 0 || V < 1 || H < 1 || p->chunk_cols < 0) return CE_ERR_INVALID_ARG;
  if (p->ld_hidden < H || p->ld_weight < H) return CE_ERR_INVALID_ARG;
  if (p->dhidden_dtype != CE_DTYPE_F32 && p->dhidden_dtype != CE_DTYPE_BF16) return CE_ERR_INVALID_ARG;
  if (!std::isfinite(z_alpha) || !std::isfinite(grad_scale)) return CE_ERR_INVALID_ARG;
  // operand windows of 256 rows are addressed with 31-bit byte offsets
  constexpr int64_t kMaxLd = int64_t{1} << 21;
  if (H % 8 != 0 || T > kMaxLd - kBM || V > kMaxLd - kBN || p->ld_hidden > kMaxLd ||
      p->ld_weight > kMaxLd)
    return CE_ERR_UNSUPPORTED;
  if (!weight || (T > 0 && (!hidden || !targets || !loss_out))) return CE_ERR_INVALID_ARG;
  if ((hidden && !aligned16(hidden, p->ld_hidden)) || !aligned16(weight, p->ld_weight))
    return CE_ERR_UNSUPPORTED;
  const bool backward = dhidden != nullptr || dweight != nullptr;
  const bool dx_bf16 = p->dhidden_dtype == CE_DTYPE_BF16;
  const LmLayout L = layout(p, backward, dx_bf16);
  if (workspace_bytes < L.total || (L.total > 0 && workspace == nullptr)) return CE_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign != 0) return CE_ERR_WORKSPACE;
  // outputs may not overlap the inputs or the workspace
  const size_t x_bytes = T > 0 ? static_cast<size_t>((T - 1) * p->ld_hidden + H) * 2 : 0;
  const size_t w_bytes = static_cast<size_t>((V - 1) * p->ld_weight + H) * 2;
  const size_t dh_bytes = static_cast<size_t>(T * H) * (dx_bf16 ? 2 : 4);
  const size_t dw_bytes = static_cast<size_t>(V * H) * 4;
  const void* outs[4] = {loss_out, lse_out, dhidden, dweight};
  const size_t out_n[4] = {static_cast<size_t>(T) * 4, static_cast<size_t>(T) * 4, dh_bytes, dw_bytes};
  for (int i = 0; i < 4; ++i)
    if (overlaps(outs[i], out_n[i], hidden, x_bytes) || overlaps(outs[i], out_n[i], weight, w_bytes) ||
        overlaps(outs[i], out_n[i], workspace, L.total))
      return CE_ERR_ALIAS;

  hipStream_t st = static_cast<hipStream_t>(stream_ptr);
  char* ws = static_cast<char*>(workspace);
  float* stats = reinterpret_cast<float*>(ws + L.off_stats);
  float* state = reinterpret_cast<float*>(ws + L.off_state);
  (void)hipGetLastError();

  if (T == 0) {
    // no rows: dW is zero (a kernel, not a memset, so the call can be captured)
    if (dweight) {
      const int64_t n = V * H;
      const unsigned nb = static_cast<unsigned>(std::min<int64_t>((n + 255) / 256, 8192));
      hipLaunchKernelGGL(lm_zero_kernel, dim3(nb), dim3(256), 0, st, dweight, n);
      if (hipGetLastError() != hipSuccess) return CE_ERR_HIP;
    }
    return CE_OK;
  }

  const Operand X{static_cast<const uint16_t*>(hidden), T, p->ld_hidden};
  const Operand W{static_cast<const uint16_t*>(weight), V, p->ld_weight};

  // ---- forward: statistics over vocabulary ranges, then the fp64 finish ----
  {
    GemmParams gp{};
    gp.a = X;
    gp.b = W;
    gp.M = T;
    gp.N = V;
    gp.K = H;
    gp.tiles_m = static_cast<int32_t>(L.tiles_m_all);
    gp.tiles_n = static_cast<int32_t>(L.tiles_n);
    gp.n_ranges = static_cast<int32_t>(L.n_ranges);
    gp.targets = targets;
    gp.stats = stats;
    const ce_status s1 = launch_k<StatsSel>(L.tiles_m_all * L.n_ranges, gp, st);
    if (s1 != CE_OK) return s1;
  }
  {
    ce_problem fp{};
    fp.T = T;
    fp.V = V;
    fp.ld_logits = V;
    fp.ld_grad = V;
    fp.ignore_index = p->ignore_index;
    const ce_status s2 = ce_rows_finish(&fp, static_cast<int32_t>(L.n_ranges), stats, targets, mask,
                                        nullptr, z_alpha, loss_out, nullptr, state, nullptr, 0, st);
    if (s2 != CE_OK) return s2;
  }
  if (lse_out) {
    hipLaunchKernelGGL(lm_lse_kernel, dim3(static_cast<unsigned>((T + 255) / 256)), dim3(256), 0, st,
                       state, T, lse_out);
    if (hipGetLastError() != hipSuccess) return CE_ERR_HIP;
  }
  if (!backward) return CE_OK;

  // ---- backward, one chunk of vocabulary columns at a time ----
  // G = dL/dz of the chunk for every row; dW rows of the chunk = G^T X
  // (K = T); dX += G W_chunk (K = chunk). Every operand of a chunk stays far
  // below the 256 MB last-level cache.
  uint16_t* g = reinterpret_cast<uint16_t*>(ws + L.off_g);
  uint16_t* gt = reinterpret_cast<uint16_t*>(ws + L.off_gt);
  uint16_t* wt = reinterpret_cast<uint16_t*>(ws + L.off_wt);
  uint16_t* xt = reinterpret_cast<uint16_t*>(ws + L.off_xt);
  float* dx = dx_bf16 ? reinterpret_cast<float*>(ws + L.off_dx) : static_cast<float*>(dhidden);
  if (dweight) {
    const ce_status sx = launch_transpose(X.p, T, H, X.ld, xt, L.t_pad, L.t_pad, st);   // X^T [H, t_pad]
    if (sx != CE_OK) return sx;
  }
  const int64_t tiles_h = (H + kBN - 1) / kBN;
  for (int64_t v0 = 0; v0 < V; v0 += L.chunk) {
    const int64_t cols = std::min<int64_t>(L.chunk, V - v0);
    const int64_t tiles_c = (cols + kBN - 1) / kBN;
    const Operand Wc{W.p + v0 * W.ld, cols, W.ld};
    {
      GemmParams gp{};
      gp.a = X;
      gp.b = Wc;
      gp.M = T;
      gp.N = cols;
      gp.K = H;
      gp.tiles_m = static_cast<int32_t>(L.tiles_m_all);
      gp.tiles_n = static_cast<int32_t>(tiles_c);
      gp.targets = targets;
      gp.row_state = state;
      gp.grad_scale = grad_scale;
      gp.v0 = v0;
      gp.g = g;
      gp.ld_g = L.chunk;
      gp.gt = gt;
      gp.ld_gt = L.t_pad;
      gp.zero_rows = T;
      const int64_t nb = tile_blocks(L.tiles_m_all, tiles_c);
      if (nb > INT32_MAX) return CE_ERR_UNSUPPORTED;   // the tile walk counts block ids in 32 bits
      const int64_t gb = persistent_blocks(nb);
      if (gb < 0) return CE_ERR_HIP;
      const ce_status s3 = launch_k<GradSel>(gb, gp, st);
      if (s3 != CE_OK) return s3;
    }
    if (dhidden) {
      // W_chunk^T [H, chunk], zero past the chunk's columns
      const ce_status sw = launch_transpose(Wc.p, cols, H, W.ld, wt, L.chunk, L.chunk, st);
      if (sw != CE_OK) return sw;
      GemmParams gp{};
      gp.a = Operand{g, T, L.chunk};
      gp.b = Operand{wt, H, L.chunk};
      gp.M = T;
      gp.N = H;
      gp.K = round_up(cols, kBK);
      gp.tiles_m = static_cast<int32_t>(L.tiles_m_all);
      gp.tiles_n = static_cast<int32_t>(tiles_h);
      gp.c = dx;
      gp.ld_c = H;
      gp.accumulate = v0 > 0 ? 1 : 0;
      const ce_status s4 = launch_k<StoreSel>(tile_blocks(L.tiles_m_all, tiles_h), gp, st);
      if (s4 != CE_OK) return s4;
    }
    if (dweight) {
      GemmParams gp{};
      gp.a = Operand{gt, cols, L.t_pad};
      gp.b = Operand{xt, H, L.t_pad};
      gp.M = cols;
      gp.N = H;
      gp.K = L.t_pad;
      gp.tiles_m = static_cast<int32_t>(tiles_c);
      gp.tiles_n = static_cast<int32_t>(tiles_h);
      gp.c = dweight + v0 * H;
      gp.ld_c = H;
      const ce_status s5 = launch_k<StoreSel>(tile_blocks(tiles_c, tiles_h), gp, st);
      if (s5 != CE_OK) return s5;
    }
  }
  if (dhidden && dx_bf16) {
    const int64_t n = T * H;
    const unsigned nb = static_cast<unsigned>(std::min<int64_t>((n + 255) / 256, 8192));
    hipLaunchKernelGGL(lm_to_bf16_kernel, dim3(nb), dim3(256), 0, st, dx, n,
                       static_cast<uint16_t*>(dhidden));
    if (hipGetLastError() != hipSuccess) return CE_ERR_HIP;
  }
  return CE_OK;
}

}  // extern "C"
