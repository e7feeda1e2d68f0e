// Vocabulary loss behind a linear LM head, without a [T, V] logit matrix,
// for MI355X (gfx950).
//
// The logits z = X W^T (hidden X [T, H], head weight W [V, H], both bf16) are
// produced tile by tile on the matrix cores (v_mfma_f32_32x32x16_bf16, fp32
// accumulation) and consumed in the tile's epilogue:
//  * forward: each workgroup walks a range of vocabulary tiles for 128 rows and
//    keeps per-row online (shift, sum) statistics of the non-target columns and
//    the target logit; ce_rows_finish merges the ranges in fp64 into the loss
//    and the saved per-row state (the collapse-free loss of torchtitan PR #5661,
//    revised PR description, Numerics; the split over vocabulary ranges is its
//    vocabulary-parallel merge, third review inline diff);
//  * backward, per chunk of rows: the logit tiles are recomputed and turned into
//    G = dL/dz from the saved state (approving review, "What this PR does":
//    rebuild the softmax, put the target gradient in its slot, scale), written
//    as bf16 in both orientations for one chunk only; then dX = G W and
//    dW += G^T X run on the same matrix-core kernel.
// Every product is C = A B^T with both operands K-contiguous; W^T and the
// chunk's X^T are formed once by a transpose kernel so that dX and dW take the
// same form.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>

#include "ce_fused.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBM = 128;          // tile rows (A rows)
constexpr int kBN = 128;          // tile columns (B rows)
constexpr int kBK = 64;           // K per LDS stage
constexpr int kLdsRow = kBK + 8;  // padded LDS row in bf16 (144 bytes)
constexpr int kThreads = 256;     // 4 waves, 2 x 2, each a 64 x 64 sub-tile
constexpr int kCRow = kBN + 4;    // padded fp32 row of the epilogue tile
constexpr int kRowState = 8;
constexpr float kL2E = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_huge_valf();

// LDS: two operand stages, reused as the fp32 epilogue tile.
struct OperandStages {
  uint16_t a[2][kBM][kLdsRow];
  uint16_t b[2][kBN][kLdsRow];
};
constexpr size_t kSmemBytes = sizeof(OperandStages) > sizeof(float) * kBM * kCRow
                                  ? sizeof(OperandStages)
                                  : sizeof(float) * kBM * kCRow;

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint16_t to_bf16(float f) {
  // round to nearest even; NaN stays NaN
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// A row-major bf16 operand [rows, K] with K contiguous.
struct Operand {
  const uint16_t* p;
  int64_t rows;
  int64_t ld;
};

struct GemmParams {
  Operand a, b;
  int64_t M, N, K;
  // tile walk
  int32_t tiles_m, tiles_n;   // tiles of the problem
  int32_t n_ranges;           // statistics: vocabulary ranges (grid = tiles_m * n_ranges)
  // statistics
  const int64_t* targets;     // [M] targets of the A rows
  float* stats;               // [n_ranges, M, 3]
  // gradient
  const float* row_state;     // [M, 8] state of the A rows
  float grad_scale;
  uint16_t* g;                // [M rows of the chunk, ld_g] row-major G
  int64_t ld_g;
  uint16_t* gt;               // [tiles_n * 128, ld_gt] transposed G
  int64_t ld_gt;
  int64_t zero_rows;          // rows >= this (within the chunk) are written as 0
  // store
  void* c;
  int64_t ld_c;
  int32_t c_bf16;
  int32_t accumulate;
};

// Loads of one K stage: 4 chunks of A and 4 of B per thread, 16 bytes each.
struct StageRegs {
  u32x4 a[4], b[4];
};

__device__ __forceinline__ void load_stage(const GemmParams& p, int64_t m0, int64_t n0, int64_t k0,
                                           StageRegs& r) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + kThreads * i;
    const int row = c >> 3, kc = c & 7;
    const int64_t k = k0 + kc * 8;
    const bool kin = k < p.K;
    const int64_t kk = kin ? k : 0;
    const int64_t ra = std::min<int64_t>(m0 + row, p.a.rows - 1);
    const int64_t rb = std::min<int64_t>(n0 + row, p.b.rows - 1);
    const u32x4 va = *reinterpret_cast<const u32x4*>(p.a.p + ra * p.a.ld + kk);
    const u32x4 vb = *reinterpret_cast<const u32x4*>(p.b.p + rb * p.b.ld + kk);
    const u32x4 zero = {0u, 0u, 0u, 0u};
    r.a[i] = kin ? va : zero;
    r.b[i] = kin ? vb : zero;
  }
}

__device__ __forceinline__ void store_stage(OperandStages& s, int buf, const StageRegs& r) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + kThreads * i;
    const int row = c >> 3, kc = c & 7;
    *reinterpret_cast<u32x4*>(&s.a[buf][row][kc * 8]) = r.a[i];
    *reinterpret_cast<u32x4*>(&s.b[buf][row][kc * 8]) = r.b[i];
  }
}

// acc[mi][ni] covers rows wm*64 + mi*32 + {8(q/4) + 4(lane/32) + q%4} and
// column wn*64 + ni*32 + lane%32 of the tile (q = register index 0..15).
__device__ __forceinline__ void tile_product(const GemmParams& p, OperandStages& s, int64_t m0,
                                             int64_t n0, f32x16 (&acc)[2][2]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[mi][ni][q] = 0.f;

  const int64_t nk = (p.K + kBK - 1) / kBK;
  StageRegs r;
  load_stage(p, m0, n0, 0, r);
  store_stage(s, 0, r);
  __syncthreads();
  for (int64_t kt = 0; kt < nk; ++kt) {
    const int buf = static_cast<int>(kt & 1);
    const bool more = kt + 1 < nk;
    if (more) load_stage(p, m0, n0, (kt + 1) * kBK, r);
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      const int kof = ks * 16 + (lane >> 5) * 8;
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
        af[mi] = *reinterpret_cast<const bf16x8*>(&s.a[buf][wm * 64 + mi * 32 + (lane & 31)][kof]);
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
        bfr[ni] = *reinterpret_cast<const bf16x8*>(&s.b[buf][wn * 64 + ni * 32 + (lane & 31)][kof]);
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bfr[ni], acc[mi][ni], 0, 0, 0);
    }
    if (more) store_stage(s, buf ^ 1, r);
    __syncthreads();
  }
}

// Spill the accumulators to the fp32 LDS tile (after the operand stages are
// no longer read: tile_product ends with a barrier).
__device__ __forceinline__ void acc_to_lds(float (*cs)[kCRow], const f32x16 (&acc)[2][2]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int row = wm * 64 + mi * 32 + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
        const int col = wn * 64 + ni * 32 + (lane & 31);
        cs[row][col] = acc[mi][ni][q];
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

// Statistics: grid = tiles_m * n_ranges; workgroup (mt, range) walks the
// vocabulary tiles of its range. Thread (row = tid / 2, half = tid % 2)
// reduces 64 columns of one row per tile.
__global__ __launch_bounds__(kThreads) void lm_stats_kernel(GemmParams p) {
  __shared__ __align__(16) unsigned char smem[kSmemBytes];
  OperandStages& s = *reinterpret_cast<OperandStages*>(smem);
  float (*cs)[kCRow] = reinterpret_cast<float (*)[kCRow]>(smem);
  const int mt = blockIdx.x % p.tiles_m;
  const int range = blockIdx.x / p.tiles_m;
  const int64_t per = (p.tiles_n + p.n_ranges - 1) / p.n_ranges;
  const int64_t nt0 = range * per, nt1 = std::min<int64_t>(p.tiles_n, nt0 + per);
  const int64_t m0 = static_cast<int64_t>(mt) * kBM;
  const int row = threadIdx.x >> 1, half = threadIdx.x & 1;
  const int64_t gr = m0 + row;
  const int64_t t = gr < p.M ? p.targets[gr] : -1;
  float mL = kNegInf, sum = 0.f, zt = kNegInf;
  f32x16 acc[2][2];
  for (int64_t nt = nt0; nt < nt1; ++nt) {
    const int64_t n0 = nt * kBN;
    tile_product(p, s, m0, n0, acc);
    acc_to_lds(cs, acc);
    __syncthreads();
    // two reads of the row's 64 columns from LDS: masked max, then the sum
    const int64_t c0 = n0 + half * 64;
    const int64_t tl = t - c0;                     // target's column in this half, if any
    const int64_t nv = std::min<int64_t>(64, p.N - c0);   // columns inside the vocabulary
    if (tl >= 0 && tl < 64) zt = cs[row][half * 64 + static_cast<int>(tl)];
    float gmax = kNegInf;
#pragma unroll 16
    for (int j = 0; j < 64; ++j) {
      const float v = cs[row][half * 64 + j];
      gmax = fmaxf(gmax, (j < nv && j != tl) ? v : kNegInf);
    }
    const float mn = fmaxf(mL, gmax * kL2E);
    if (mn != kNegInf) {
      float acc_s = 0.f;
#pragma unroll 16
      for (int j = 0; j < 64; ++j) {
        const float v = (j < nv && j != tl) ? cs[row][half * 64 + j] : kNegInf;
        acc_s += fexp2(__builtin_fmaf(v, kL2E, -mn));
      }
      sum = (mL == kNegInf ? 0.f : sum * fexp2(mL - mn)) + acc_s;
      mL = mn;
    }
    __syncthreads();   // the LDS tile is overwritten by the next tile's stages
  }
  // the two halves of a row meet in adjacent lanes
  const float m2 = __shfl_xor(mL, 1, 64);
  const float s2 = __shfl_xor(sum, 1, 64);
  const float z2 = __shfl_xor(zt, 1, 64);
  merge(mL, sum, m2, s2);
  zt = fmaxf(zt, z2);
  if (half == 0 && gr < p.M) {
    float* st = p.stats + 3 * (static_cast<int64_t>(range) * p.M + gr);
    st[0] = mL;
    st[1] = sum;
    st[2] = zt;
  }
}

// Gradient tiles of one chunk: grid = tiles_m * tiles_n, tile order chosen so
// that consecutive workgroups share the weight tile.
__global__ __launch_bounds__(kThreads) void lm_grad_kernel(GemmParams p) {
  __shared__ __align__(16) unsigned char smem[kSmemBytes];
  OperandStages& s = *reinterpret_cast<OperandStages*>(smem);
  float (*cs)[kCRow] = reinterpret_cast<float (*)[kCRow]>(smem);
  const int mt = blockIdx.x % p.tiles_m;
  const int nt = blockIdx.x / p.tiles_m;
  const int64_t m0 = static_cast<int64_t>(mt) * kBM, n0 = static_cast<int64_t>(nt) * kBN;
  f32x16 acc[2][2];
  tile_product(p, s, m0, n0, acc);
  acc_to_lds(cs, acc);
  __syncthreads();

  // rows: dL/dz in place in the LDS tile, then row-major bf16 stores
  {
    const int row = threadIdx.x >> 1, half = threadIdx.x & 1;
    const int64_t gr = m0 + row;
    float cnt = 0.f, gt = 0.f, kl = 0.f, fill = 0.f;
    int64_t t = -1;
    bool live = false;
    if (gr < p.zero_rows) {
      const float* rs = p.row_state + kRowState * gr;
      const float kind = rs[5];
      if (kind == 0.f) {
        const float zw = p.grad_scale * rs[4];
        kl = rs[0];
        cnt = zw + zw * rs[3];
        gt = -zw * rs[1] + zw * rs[3] * rs[2];
        t = p.targets[gr];
        live = true;
      } else {
        fill = (kind == 1.f) ? 0.f : __builtin_nanf("");
      }
    }
    const int64_t c0 = n0 + half * 64;
    uint16_t out[64];
#pragma unroll
    for (int j = 0; j < 64; ++j) {
      const int64_t col = c0 + j;
      float g;
      if (col >= p.N) {
        g = 0.f;
      } else if (!live) {
        g = fill;
      } else if (col == t) {
        g = gt;
      } else {
        g = cnt * fexp2(__builtin_fmaf(cs[row][half * 64 + j], kL2E, -kl));
      }
      out[j] = to_bf16(g);
      cs[row][half * 64 + j] = __uint_as_float(static_cast<uint32_t>(out[j]) << 16);
    }
    if (gr < p.M) {
      uint16_t* dst = p.g + gr * p.ld_g + c0;
#pragma unroll
      for (int j = 0; j < 64; j += 8) {
        u32x4 v;
        v.x = out[j] | (static_cast<uint32_t>(out[j + 1]) << 16);
        v.y = out[j + 2] | (static_cast<uint32_t>(out[j + 3]) << 16);
        v.z = out[j + 4] | (static_cast<uint32_t>(out[j + 5]) << 16);
        v.w = out[j + 6] | (static_cast<uint32_t>(out[j + 7]) << 16);
        *reinterpret_cast<u32x4*>(dst + j) = v;
      }
    }
  }
  __syncthreads();
  // columns: transposed bf16 stores (rows of G^T), zeros past the chunk's rows
  {
    const int col = threadIdx.x >> 1, half = threadIdx.x & 1;
    const int64_t gc = n0 + col;
    uint16_t* dst = p.gt + gc * p.ld_gt + m0 + half * 64;
    const int64_t rows_left = p.ld_gt - (m0 + half * 64);
    if (rows_left >= 64) {
#pragma unroll
      for (int j = 0; j < 64; j += 8) {
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t lo = __float_as_uint(cs[half * 64 + j + 2 * e][col]) >> 16;
          const uint32_t hi = __float_as_uint(cs[half * 64 + j + 2 * e + 1][col]) >> 16;
          w[e] = lo | (hi << 16);
        }
        const u32x4 v = {w[0], w[1], w[2], w[3]};
        *reinterpret_cast<u32x4*>(dst + j) = v;
      }
    }
  }
}

// Plain product C = A B^T (fp32 or bf16 out, optional accumulate).
__global__ __launch_bounds__(kThreads) void lm_store_kernel(GemmParams p) {
  __shared__ __align__(16) unsigned char smem[kSmemBytes];
  OperandStages& s = *reinterpret_cast<OperandStages*>(smem);
  const int mt = blockIdx.x % p.tiles_m;
  const int nt = blockIdx.x / p.tiles_m;
  const int64_t m0 = static_cast<int64_t>(mt) * kBM, n0 = static_cast<int64_t>(nt) * kBN;
  f32x16 acc[2][2];
  tile_product(p, s, m0, n0, acc);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
      const int64_t col = n0 + wn * 64 + ni * 32 + (lane & 31);
      if (col >= p.N) continue;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int64_t row = m0 + wm * 64 + mi * 32 + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
        if (row >= p.M) continue;
        if (p.c_bf16) {
          static_cast<uint16_t*>(p.c)[row * p.ld_c + col] = to_bf16(acc[mi][ni][q]);
        } else {
          float* dst = static_cast<float*>(p.c) + row * p.ld_c + col;
          *dst = p.accumulate ? *dst + acc[mi][ni][q] : acc[mi][ni][q];
        }
      }
    }
}

// out[c, r] = in[r, c] for r < R, c < C; out[c, r] = 0 for R <= r < Rp.
// 64 x 64 tiles through LDS; grid (ceil(Rp/64), ceil(C/64)).
__global__ __launch_bounds__(256) void lm_transpose_kernel(const uint16_t* __restrict__ in,
                                                           int64_t R, int64_t C, int64_t ld_in,
                                                           uint16_t* __restrict__ out, int64_t Rp,
                                                           int64_t ld_out) {
  __shared__ uint16_t tile[64][66];
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * 64, c0 = static_cast<int64_t>(blockIdx.y) * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4) {
    const int64_t r = r0 + i, c = c0 + tx;
    tile[i][tx] = (r < R && c < C) ? in[r * ld_in + c] : static_cast<uint16_t>(0);
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int64_t c = c0 + i, r = r0 + tx;
    if (c < C && r < Rp) out[c * ld_out + r] = tile[tx][i];
  }
}

// lse from the saved state: lse = state[0] / log2(e) for valid rows, 0 for
// ignored rows, NaN for poisoned ones.
__global__ __launch_bounds__(256) void lm_lse_kernel(const float* __restrict__ row_state,
                                                     int64_t T, float* __restrict__ lse) {
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (r >= T) return;
  const float* rs = row_state + kRowState * r;
  lse[r] = rs[5] == 0.f ? static_cast<float>(static_cast<double>(rs[0]) / static_cast<double>(kL2E))
                        : (rs[5] == 1.f ? 0.f : __builtin_nanf(""));
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

struct LmLayout {
  int64_t chunk, ld_pad, n_ranges, tiles_m_all, tiles_n;
  size_t off_stats, off_state, off_wt, off_g, off_gt, off_xt, total;
};

int64_t chunk_rows_of(const ce_lmhead* p) {
  int64_t c = p->chunk_rows > 0 ? p->chunk_rows : 4096;
  c = round_up(std::min<int64_t>(c, std::max<int64_t>(p->T, 1)), kBM);
  return c;
}

LmLayout layout(const ce_lmhead* p, bool backward) {
  LmLayout L{};
  L.chunk = chunk_rows_of(p);
  L.tiles_n = (p->V + kBN - 1) / kBN;
  L.ld_pad = L.tiles_n * kBN;                       // padded vocabulary (zeros past V)
  L.tiles_m_all = (p->T + kBM - 1) / kBM;
  // about 2048 workgroups (8 per compute unit of the 256), at least one tile each
  const int64_t want = 2048;
  L.n_ranges = std::max<int64_t>(1, std::min<int64_t>(L.tiles_n, (want + L.tiles_m_all - 1) /
                                                                    std::max<int64_t>(L.tiles_m_all, 1)));
  size_t off = 0;
  L.off_stats = off;
  off += align_up(static_cast<size_t>(L.n_ranges) * p->T * 3 * sizeof(float));
  L.off_state = off;
  off += align_up(static_cast<size_t>(p->T) * kRowState * sizeof(float));
  if (backward) {
    L.off_wt = off;
    off += align_up(static_cast<size_t>(p->H) * L.ld_pad * 2);
    L.off_g = off;
    off += align_up(static_cast<size_t>(L.chunk) * L.ld_pad * 2);
    L.off_gt = off;
    off += align_up(static_cast<size_t>(L.ld_pad) * L.chunk * 2);
    L.off_xt = off;
    off += align_up(static_cast<size_t>(p->H) * L.chunk * 2);
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

ce_status launch(void (*kern)(GemmParams), int64_t blocks, const GemmParams& gp, hipStream_t st) {
  if (blocks <= 0) return CE_OK;
  if (blocks > INT32_MAX) return CE_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, st, gp);
  return hipGetLastError() == hipSuccess ? CE_OK : CE_ERR_HIP;
}

}  // namespace

extern "C" {

size_t ce_lmhead_workspace_bytes(const ce_lmhead* p, int32_t backward) {
  if (p == nullptr || p->T < 0 || p->V < 1 || p->H < 1) return 0;
  return layout(p, backward != 0).total;
}

ce_status ce_lmhead_fwd_bwd(const ce_lmhead* p, const void* hidden, const void* weight,
                            const int64_t* targets, const uint8_t* mask, float z_alpha,
                            float grad_scale, float* loss_out, float* lse_out, void* dhidden,
                            float* dweight, void* workspace, size_t workspace_bytes,
                            void* stream_ptr) {
  if (p == nullptr) return CE_ERR_INVALID_ARG;
  const int64_t T = p->T, V = p->V, H = p->H;
  if (T < 0 || V < 1 || H < 1 || p->chunk_rows < 0) return CE_ERR_INVALID_ARG;
  if (p->ld_hidden < H || p->ld_weight < H) return CE_ERR_INVALID_ARG;
  if (p->dhidden_dtype != CE_DTYPE_F32 && p->dhidden_dtype != CE_DTYPE_BF16) return CE_ERR_INVALID_ARG;
  if (!std::isfinite(z_alpha) || !std::isfinite(grad_scale)) return CE_ERR_INVALID_ARG;
  if (H % 8 != 0 || T > INT32_MAX || V > (int64_t{1} << 30) || H > (int64_t{1} << 20))
    return CE_ERR_UNSUPPORTED;
  if (!weight || (T > 0 && (!hidden || !targets || !loss_out))) return CE_ERR_INVALID_ARG;
  if ((hidden && !aligned16(hidden, p->ld_hidden)) || !aligned16(weight, p->ld_weight))
    return CE_ERR_UNSUPPORTED;
  const bool backward = dhidden != nullptr || dweight != nullptr;
  const LmLayout L = layout(p, backward);
  if (workspace_bytes < L.total || (L.total > 0 && workspace == nullptr)) return CE_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign != 0) return CE_ERR_WORKSPACE;
  // outputs may not overlap the inputs
  const size_t x_bytes = T > 0 ? static_cast<size_t>((T - 1) * p->ld_hidden + H) * 2 : 0;
  const size_t w_bytes = static_cast<size_t>((V - 1) * p->ld_weight + H) * 2;
  const size_t dh_bytes = static_cast<size_t>(T * H) * (p->dhidden_dtype == CE_DTYPE_F32 ? 4 : 2);
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
    if (dweight) {
      if (hipMemsetAsync(dweight, 0, dw_bytes, st) != hipSuccess) return CE_ERR_HIP;
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
    const ce_status s1 = launch(lm_stats_kernel, L.tiles_m_all * L.n_ranges, gp, st);
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

  // ---- backward, chunk by chunk ----
  uint16_t* wt = reinterpret_cast<uint16_t*>(ws + L.off_wt);
  uint16_t* g = reinterpret_cast<uint16_t*>(ws + L.off_g);
  uint16_t* gt = reinterpret_cast<uint16_t*>(ws + L.off_gt);
  uint16_t* xt = reinterpret_cast<uint16_t*>(ws + L.off_xt);
  if (dhidden) {
    // W^T [H, ld_pad], zero past V
    hipLaunchKernelGGL(lm_transpose_kernel,
                       dim3(static_cast<unsigned>(L.ld_pad / 64), static_cast<unsigned>((H + 63) / 64)),
                       dim3(256), 0, st, static_cast<const uint16_t*>(weight), V, H, p->ld_weight, wt,
                       L.ld_pad, L.ld_pad);
    if (hipGetLastError() != hipSuccess) return CE_ERR_HIP;
  }
  for (int64_t c0 = 0; c0 < T; c0 += L.chunk) {
    const int64_t rows = std::min<int64_t>(L.chunk, T - c0);
    const int64_t tiles_m = (rows + kBM - 1) / kBM;
    {
      GemmParams gp{};
      gp.a = Operand{X.p + c0 * X.ld, rows, X.ld};
      gp.b = W;
      gp.M = rows;
      gp.N = V;
      gp.K = H;
      gp.tiles_m = static_cast<int32_t>(tiles_m);
      gp.tiles_n = static_cast<int32_t>(L.tiles_n);
      gp.targets = targets + c0;
      gp.row_state = state + kRowState * c0;
      gp.grad_scale = grad_scale;
      gp.g = g;
      gp.ld_g = L.ld_pad;
      gp.gt = gt;
      gp.ld_gt = L.chunk;
      gp.zero_rows = rows;
      const ce_status s3 = launch(lm_grad_kernel, tiles_m * L.tiles_n, gp, st);
      if (s3 != CE_OK) return s3;
    }
    if (dhidden) {
      GemmParams gp{};
      gp.a = Operand{g, rows, L.ld_pad};
      gp.b = Operand{wt, H, L.ld_pad};
      gp.M = rows;
      gp.N = H;
      gp.K = L.ld_pad;
      gp.tiles_m = static_cast<int32_t>(tiles_m);
      gp.tiles_n = static_cast<int32_t>((H + kBN - 1) / kBN);
      const bool bf = p->dhidden_dtype == CE_DTYPE_BF16;
      gp.c = static_cast<char*>(dhidden) + static_cast<size_t>(c0 * H) * (bf ? 2 : 4);
      gp.ld_c = H;
      gp.c_bf16 = bf ? 1 : 0;
      const ce_status s4 = launch(lm_store_kernel, tiles_m * gp.tiles_n, gp, st);
      if (s4 != CE_OK) return s4;
    }
    if (dweight) {
      // X_c^T [H, chunk], zero past the chunk's rows
      hipLaunchKernelGGL(lm_transpose_kernel,
                         dim3(static_cast<unsigned>(L.chunk / 64), static_cast<unsigned>((H + 63) / 64)),
                         dim3(256), 0, st, X.p + c0 * X.ld, rows, H, X.ld, xt, L.chunk, L.chunk);
      if (hipGetLastError() != hipSuccess) return CE_ERR_HIP;
      GemmParams gp{};
      gp.a = Operand{gt, V, L.chunk};
      gp.b = Operand{xt, H, L.chunk};
      gp.M = V;
      gp.N = H;
      gp.K = round_up(rows, kBK);
      gp.tiles_m = static_cast<int32_t>(L.tiles_n);
      gp.tiles_n = static_cast<int32_t>((H + kBN - 1) / kBN);
      gp.c = dweight;
      gp.ld_c = H;
      gp.accumulate = c0 > 0 ? 1 : 0;
      const ce_status s5 = launch(lm_store_kernel, static_cast<int64_t>(gp.tiles_m) * gp.tiles_n, gp, st);
      if (s5 != CE_OK) return s5;
    }
  }
  return CE_OK;
}

}  // extern "C"
