// Fused vocabulary cross-entropy forward + backward for gfx950 (MI355X).
//
// What one call computes is stated in include/ce_fused.h. The method follows
// torchtitan PR #5661 "fix softmax collapse with improved CE perf" (revised PR
// description, Numerics; approving review, "What this PR does"): the target
// column is dropped before the non-target sum, the NLL is a softplus of the
// non-target logsumexp minus the target logit, the target gradient is minus the
// non-target probability, and backward rebuilds the softmax from the input
// logits plus per-row statistics. z-loss rides on the same softmax (Fast-LLM
// PR #552 "Fuse GSPO into the monolithic compiled loss", PR body) and segment
// sums replace its index_add seam.
//
// Device design (bandwidth-bound, no matrix cores):
//  * one workgroup owns one row at a time (persistent grid-stride loop);
//  * 16-byte loads/stores of bf16 or fp32, each thread owning the 16-byte
//    chunks tid, tid + BLOCK, ...;
//  * the first NRES chunks of each thread stay in registers as exps between
//    the two passes, so they are read from HBM once; the rest of the row is
//    streamed in pass 1 (online max / sum of exps) and streamed again in
//    pass 2;
//  * statistics are kept in the log2 domain: every exponential is one
//    v_exp_f32 of an FMA, and a thread's partial is (shift, sum) with the
//    shift a float that the merge uses exactly;
//  * wave reduction by lane shuffles, then one LDS slot per wave;
//  * the per-row epilogue (softplus, logaddexp, sigmoids, z-loss) in fp64;
//  * per-segment NLL sums by a second kernel that walks each segment's rows
//    in a fixed order (deterministic, no atomics).

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "ce_fused.h"

namespace {

constexpr float kL2E = 1.44269504088896340736f;  // log2(e), rounded to float
constexpr float kNegInf = -__builtin_huge_valf();

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

struct bf16_t {};  // tag: storage is the upper 16 bits of a binary32

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2 f = {a, b};
  bf16x2 h = __builtin_convertvector(f, bf16x2);  // v_cvt_pk_bf16_f32: RNE
  return __builtin_bit_cast(uint32_t, h);
}

// ---------------------------------------------------------------------------
// Element access. A "chunk" is W consecutive elements of a row; W is the
// 16-byte width of the element type, or 1 for the unaligned fallback.
// ---------------------------------------------------------------------------

template <typename T>
struct Elem;

template <>
struct Elem<float> {
  static constexpr int BYTES = 4;
  static constexpr int VEC = 4;
  __device__ static float load1(const void* row, int64_t i) {
    return static_cast<const float*>(row)[i];
  }
  __device__ static void store1(void* row, int64_t i, float v) {
    __builtin_nontemporal_store(v, static_cast<float*>(row) + i);
  }
};

template <>
struct Elem<bf16_t> {
  static constexpr int BYTES = 2;
  static constexpr int VEC = 8;
  __device__ static float load1(const void* row, int64_t i) {
    const uint32_t u = static_cast<const uint16_t*>(row)[i];
    return __uint_as_float(u << 16);
  }
  __device__ static void store1(void* row, int64_t i, float v) {
    const uint16_t h = static_cast<uint16_t>(pack_bf16x2(v, 0.f) & 0xffffu);
    __builtin_nontemporal_store(h, static_cast<uint16_t*>(row) + i);
  }
};

// Raw storage of one chunk of W elements of type T.
template <typename T, int W>
struct Chunk {
  static constexpr int NB = W * Elem<T>::BYTES;
  static_assert(NB == 16 || W == 1, "a chunk is 16 bytes or one element");
  u32x4 v;  // W == VEC: the 16 bytes; W == 1: the element's bits in v.x

  __device__ void load(const void* row, int64_t c, bool nt) {
    if constexpr (W == 1) {
      v.x = __float_as_uint(Elem<T>::load1(row, c));
    } else {
      const u32x4* p = static_cast<const u32x4*>(row) + c;
      v = nt ? __builtin_nontemporal_load(p) : *p;
    }
  }
  __device__ void unpack(float (&x)[W]) const {
    if constexpr (W == 1) {
      x[0] = __uint_as_float(v.x);
    } else if constexpr (Elem<T>::BYTES == 4) {
      x[0] = __uint_as_float(v.x);
      x[1] = __uint_as_float(v.y);
      x[2] = __uint_as_float(v.z);
      x[3] = __uint_as_float(v.w);
    } else {
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        x[2 * k] = __uint_as_float(w[k] << 16);
        x[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
      }
    }
  }
};

// Store W consecutive gradient values (chunk index c of a row whose chunks
// are W elements wide) as type TO, non-temporally.
template <typename TO, int W>
__device__ __forceinline__ void store_chunk(void* row, int64_t c, const float (&g)[W]) {
  if constexpr (W == 1) {
    Elem<TO>::store1(row, c, g[0]);
  } else if constexpr (Elem<TO>::BYTES == 4) {
    // W floats: 16 bytes per 4 elements.
#pragma unroll
    for (int q = 0; q < W / 4; ++q) {
      u32x4 o = {__float_as_uint(g[4 * q]), __float_as_uint(g[4 * q + 1]),
                 __float_as_uint(g[4 * q + 2]), __float_as_uint(g[4 * q + 3])};
      __builtin_nontemporal_store(o, static_cast<u32x4*>(row) + c * (W / 4) + q);
    }
  } else if constexpr (W == 8) {
    u32x4 o = {pack_bf16x2(g[0], g[1]), pack_bf16x2(g[2], g[3]),
               pack_bf16x2(g[4], g[5]), pack_bf16x2(g[6], g[7])};
    __builtin_nontemporal_store(o, static_cast<u32x4*>(row) + c);
  } else {  // W == 4 bf16 outputs: 8 bytes
    u32x2 o = {pack_bf16x2(g[0], g[1]), pack_bf16x2(g[2], g[3])};
    __builtin_nontemporal_store(o, static_cast<u32x2*>(row) + c);
  }
}

// Merge partial (m, s) -- s = sum 2^(y - m) over a set, m a float shift in
// log2 units -- with (m2, s2). An empty partial is (-inf, 0).
__device__ __forceinline__ void merge(float& m, float& s, float m2, float s2) {
  const float mn = fmaxf(m, m2);
  const float sh = (mn == kNegInf) ? 0.f : mn;
  s = s * fexp2(m - sh) + s2 * fexp2(m2 - sh);
  m = mn;
}

__device__ __forceinline__ double sigmoid_d(double x) {
  if (x >= 0.0) return 1.0 / (1.0 + exp(-x));
  const double e = exp(x);
  return e / (1.0 + e);
}

struct RowParams {
  const void* logits;
  void* grad;
  const int64_t* targets;
  const uint8_t* mask;
  const int32_t* seg_ids;
  const int32_t* seg_start;  // [S + 1] row offsets of each segment, or null
  float* loss_out;
  float* nll_ws;             // [T] NLL per row for the segment sums, or null
  int64_t T, V, ld_in, ld_out, ignore_index;
  int32_t num_segments;
  int32_t seg_mean;
  float z_alpha, grad_scale;
};

// ---------------------------------------------------------------------------
// Row kernel.
//   TI/TO  : logits / gradient element types
//   W      : elements per chunk (16-byte width, or 1 for the unaligned path)
//   BLOCK  : threads per workgroup
//   NRES   : chunks per thread kept in registers between the passes
//   U      : chunks per thread in flight in the streamed loops
//   WRITE  : write the gradient (false = forward only)
// ---------------------------------------------------------------------------
template <typename TI, typename TO, int W, int BLOCK, int NRES, int U, bool WRITE>
__global__ __launch_bounds__(BLOCK) void ce_rows_kernel(RowParams p) {
  constexpr int NWAVE = BLOCK / 64;
  static_assert(BLOCK % 64 == 0, "whole waves");
  __shared__ float red_m[2][NWAVE];
  __shared__ float red_s[2][NWAVE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int64_t V = p.V;
  const int64_t nchunk = V / W;
  const int tail = static_cast<int>(V - nchunk * W);
  const size_t in_row_bytes = static_cast<size_t>(p.ld_in) * Elem<TI>::BYTES;
  const size_t out_row_bytes = static_cast<size_t>(p.ld_out) * Elem<TO>::BYTES;

  int par = 0;
  for (int64_t r = blockIdx.x; r < p.T; r += gridDim.x, par ^= 1) {
    const int64_t t = p.targets[r];
    const bool valid = (t != p.ignore_index) && (p.mask == nullptr || p.mask[r] != 0);
    void* grow = WRITE ? static_cast<char*>(p.grad) + r * out_row_bytes : nullptr;

    if (!valid || t < 0 || t >= V) {
      // Ignored row: +0.0 everywhere, logits never read. Valid row with an
      // out-of-range target: NaN loss and gradient row.
      const float fill = valid ? __builtin_nanf("") : 0.f;
      if (tid == 0) {
        p.loss_out[r] = fill;
        if (p.nll_ws) p.nll_ws[r] = fill;
      }
      if constexpr (WRITE) {
        float f[W];
#pragma unroll
        for (int k = 0; k < W; ++k) f[k] = fill;
        for (int64_t c = tid; c < nchunk; c += BLOCK) store_chunk<TO, W>(grow, c, f);
        if (tid < tail) Elem<TO>::store1(grow, nchunk * W + tid, fill);
      }
      continue;
    }

    const void* zrow = static_cast<const char*>(p.logits) + r * in_row_bytes;
    const float zt = Elem<TI>::load1(zrow, t);
    const int64_t ct = t / W;              // chunk holding the target column
    const int kt = static_cast<int>(t - ct * W);

    // ---- pass 1a: resident chunks -> exps kept in registers ---------------
    float e[NRES > 0 ? NRES : 1][W];
    float rsh = 0.f;          // shift of the resident exps (log2 units)
    float mL = kNegInf, s = 0.f;
    if constexpr (NRES > 0) {
      Chunk<TI, W> raw[NRES];
#pragma unroll
      for (int i = 0; i < NRES; ++i) {
        const int64_t c = static_cast<int64_t>(i) * BLOCK + tid;
        if (c < nchunk) raw[i].load(zrow, c, false);
      }
      float rmax = kNegInf;
#pragma unroll
      for (int i = 0; i < NRES; ++i) {
        const int64_t c = static_cast<int64_t>(i) * BLOCK + tid;
        if (c < nchunk) {
          raw[i].unpack(e[i]);
        } else {
#pragma unroll
          for (int k = 0; k < W; ++k) e[i][k] = kNegInf;
        }
        if (c == ct) {
#pragma unroll
          for (int k = 0; k < W; ++k)
            if (k == kt) e[i][k] = kNegInf;   // the target is not summed
        }
#pragma unroll
        for (int k = 0; k < W; ++k) rmax = fmaxf(rmax, e[i][k]);
      }
      const float rml = rmax * kL2E;
      rsh = (rml == kNegInf) ? 0.f : rml;
      float rs = 0.f;
#pragma unroll
      for (int i = 0; i < NRES; ++i) {
        float cs = 0.f;
#pragma unroll
        for (int k = 0; k < W; ++k) {
          e[i][k] = fexp2(__builtin_fmaf(e[i][k], kL2E, -rsh));
          cs += e[i][k];
        }
        rs += cs;
      }
      mL = rml;
      s = rs;
    }

    // ---- pass 1b: streamed chunks, online (shift, sum) ---------------------
    for (int64_t c0 = static_cast<int64_t>(NRES) * BLOCK + tid; c0 < nchunk;
         c0 += static_cast<int64_t>(U) * BLOCK) {
      Chunk<TI, W> raw[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t c = c0 + static_cast<int64_t>(u) * BLOCK;
        if (c < nchunk) raw[u].load(zrow, c, false);
      }
      float x[U][W];
      float gmax = kNegInf;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t c = c0 + static_cast<int64_t>(u) * BLOCK;
        if (c < nchunk) {
          raw[u].unpack(x[u]);
        } else {
#pragma unroll
          for (int k = 0; k < W; ++k) x[u][k] = kNegInf;
        }
        if (c == ct) {
#pragma unroll
          for (int k = 0; k < W; ++k)
            if (k == kt) x[u][k] = kNegInf;
        }
#pragma unroll
        for (int k = 0; k < W; ++k) gmax = fmaxf(gmax, x[u][k]);
      }
      const float mn = fmaxf(mL, gmax * kL2E);
      const float sh = (mn == kNegInf) ? 0.f : mn;
      float acc = 0.f;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float cs = 0.f;
#pragma unroll
        for (int k = 0; k < W; ++k) cs += fexp2(__builtin_fmaf(x[u][k], kL2E, -sh));
        acc += cs;
      }
      s = s * fexp2(mL - sh) + acc;
      mL = mn;
    }
    // Elements past the last whole chunk: one per thread.
    if (tid < tail) {
      const int64_t j = nchunk * W + tid;
      const float xv = (j == t) ? kNegInf : Elem<TI>::load1(zrow, j);
      merge(mL, s, xv * kL2E, (xv == kNegInf) ? 0.f : 1.f);
    }

    // ---- workgroup reduction of (shift, sum) -------------------------------
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float m2 = __shfl_xor(mL, off, 64);
      const float s2 = __shfl_xor(s, off, 64);
      merge(mL, s, m2, s2);
    }
    if (lane == 0) {
      red_m[par][wid] = mL;
      red_s[par][wid] = s;
    }
    __syncthreads();
    float M = red_m[par][0], S = red_s[par][0];
#pragma unroll
    for (int w = 1; w < NWAVE; ++w) merge(M, S, red_m[par][w], red_s[par][w]);

    // ---- per-row epilogue in fp64 ------------------------------------------
    const double l2e = static_cast<double>(kL2E);
    const double lse_nt = (M == kNegInf) ? -HUGE_VAL
                                         : static_cast<double>(M) / l2e + log(static_cast<double>(S));
    const double zt_d = static_cast<double>(zt);
    const double xx = lse_nt - zt_d;             // LSE_nt - z_t
    const double l1p = log1p(exp(-fabs(xx)));
    const double nll = (xx > 0.0 ? xx : 0.0) + l1p;              // softplus
    const double lse = (lse_nt > zt_d ? lse_nt : zt_d) + l1p;    // logaddexp
    const double p_nt = sigmoid_d(xx);
    const double p_t = sigmoid_d(-xx);
    double scale = static_cast<double>(p.grad_scale);
    if (p.seg_mean) {
      int32_t sid = p.seg_ids[r];
      sid = sid < 0 ? 0 : (sid >= p.num_segments ? p.num_segments - 1 : sid);
      const int32_t len = p.seg_start[sid + 1] - p.seg_start[sid];
      scale /= static_cast<double>(len > 0 ? len : 1);
    }
    const double alpha = static_cast<double>(p.z_alpha);
    const double zfac = (alpha == 0.0) ? 0.0 : 2.0 * alpha * lse;
    if (tid == 0) {
      const double loss = nll + ((alpha == 0.0) ? 0.0 : alpha * lse * lse);
      p.loss_out[r] = static_cast<float>(loss);
      if (p.nll_ws) p.nll_ws[r] = static_cast<float>(nll);
    }

    // ---- pass 2: gradient ----------------------------------------------------
    if constexpr (WRITE) {
      const double cnt = scale * (1.0 + zfac);               // non-target factor
      const float g_t = static_cast<float>(scale * (-p_nt + zfac * p_t));
      const float cnt_f = static_cast<float>(cnt);
      const float kl = static_cast<float>(l2e * lse);        // lse in log2 units
      if constexpr (NRES > 0) {
        const float f = static_cast<float>(cnt * exp2(static_cast<double>(rsh) - l2e * lse));
#pragma unroll
        for (int i = 0; i < NRES; ++i) {
          const int64_t c = static_cast<int64_t>(i) * BLOCK + tid;
          if (c < nchunk) {
            float g[W];
#pragma unroll
            for (int k = 0; k < W; ++k) g[k] = e[i][k] * f;
            if (c == ct) {
#pragma unroll
              for (int k = 0; k < W; ++k)
                if (k == kt) g[k] = g_t;
            }
            store_chunk<TO, W>(grow, c, g);
          }
        }
      }
      for (int64_t c0 = static_cast<int64_t>(NRES) * BLOCK + tid; c0 < nchunk;
           c0 += static_cast<int64_t>(U) * BLOCK) {
        Chunk<TI, W> raw[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t c = c0 + static_cast<int64_t>(u) * BLOCK;
          if (c < nchunk) raw[u].load(zrow, c, true);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t c = c0 + static_cast<int64_t>(u) * BLOCK;
          if (c < nchunk) {
            float x[W], g[W];
            raw[u].unpack(x);
#pragma unroll
            for (int k = 0; k < W; ++k) g[k] = cnt_f * fexp2(__builtin_fmaf(x[k], kL2E, -kl));
            if (c == ct) {
#pragma unroll
              for (int k = 0; k < W; ++k)
                if (k == kt) g[k] = g_t;
            }
            store_chunk<TO, W>(grow, c, g);
          }
        }
      }
      if (tid < tail) {
        const int64_t j = nchunk * W + tid;
        float g;
        if (j == t) {
          g = g_t;
        } else {
          const float xv = Elem<TI>::load1(zrow, j);
          g = cnt_f * fexp2(__builtin_fmaf(xv, kL2E, -kl));
        }
        Elem<TO>::store1(grow, j, g);
      }
    }
  }
}

// seg_start[s] = first row whose id is >= s, for s in [0, S]; ids sorted.
__global__ __launch_bounds__(256) void ce_seg_bounds_kernel(const int32_t* __restrict__ ids,
                                                            int64_t T, int32_t S,
                                                            int32_t* __restrict__ seg_start) {
  const int64_t s = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (s > S) return;
  int64_t lo = 0, hi = T;
  while (lo < hi) {
    const int64_t mid = lo + ((hi - lo) >> 1);
    if (ids[mid] < s) lo = mid + 1; else hi = mid;
  }
  seg_start[s] = static_cast<int32_t>(lo);
}

// seg_out[s] = sum of nll[r] over rows r of segment s (ignored rows hold 0),
// accumulated in fp64 in a fixed order: one workgroup per segment.
__global__ __launch_bounds__(256) void ce_seg_sum_kernel(const float* __restrict__ nll,
                                                         const int32_t* __restrict__ seg_start,
                                                         int32_t S, float* __restrict__ seg_out) {
  __shared__ double part[256 / 64];
  const int s = blockIdx.x;
  if (s >= S) return;
  int32_t lo = seg_start[s], hi = seg_start[s + 1];
  if (hi < lo) hi = lo;
  double acc = 0.0;
  for (int32_t r = lo + static_cast<int32_t>(threadIdx.x); r < hi; r += 256)
    acc += static_cast<double>(nll[r]);
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    double tot = 0.0;
    for (int w = 0; w < 256 / 64; ++w) tot += part[w];
    seg_out[s] = static_cast<float>(tot);
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

inline int dtype_bytes(int32_t dt) { return dt == CE_DTYPE_F32 ? 4 : 2; }

int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (dev < 0 || dev >= 64) return -1;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return -1;
  cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

template <typename TI, typename TO, int W, int BLOCK, int NRES, int U, bool WRITE>
ce_status launch_rows(const RowParams& rp, hipStream_t stream) {
  auto kern = ce_rows_kernel<TI, TO, W, BLOCK, NRES, U, WRITE>;
  static std::atomic<int> occ{0};
  int per_cu = occ.load(std::memory_order_relaxed);
  if (per_cu <= 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, BLOCK, 0) != hipSuccess || n <= 0)
      return CE_ERR_HIP;
    occ.store(n, std::memory_order_relaxed);
    per_cu = n;
  }
  const int cus = device_cus();
  if (cus <= 0) return CE_ERR_HIP;
  const int64_t want = static_cast<int64_t>(cus) * per_cu;
  const int64_t grid = rp.T < want ? rp.T : want;
  if (grid <= 0) return CE_OK;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(BLOCK), 0, stream, rp);
  return hipGetLastError() == hipSuccess ? CE_OK : CE_ERR_HIP;
}

// Pick a kernel variant for (input type, output type, vector path or not).
template <typename TI, typename TO, bool WRITE>
ce_status dispatch_rows(const RowParams& rp, bool vec, hipStream_t stream) {
  if (!vec) return launch_rows<TI, TO, 1, 256, 0, 8, WRITE>(rp, stream);
  constexpr int W = Elem<TI>::VEC;
  // Rows that fit in registers: keep them resident (read once from HBM).
  const int64_t nchunk = rp.V / W;
  if (nchunk <= 256 * 4) return launch_rows<TI, TO, W, 256, 4, 4, WRITE>(rp, stream);
  return launch_rows<TI, TO, W, 256, 0, 4, WRITE>(rp, stream);
}

template <typename TI>
ce_status dispatch_out(const RowParams& rp, int32_t grad_dtype, bool write, bool vec,
                       hipStream_t stream) {
  if (!write) return dispatch_rows<TI, TI, false>(rp, vec, stream);
  if (grad_dtype == CE_DTYPE_F32) return dispatch_rows<TI, float, true>(rp, vec, stream);
  return dispatch_rows<TI, bf16_t, true>(rp, vec, stream);
}

bool ranges_overlap(uintptr_t a0, size_t an, uintptr_t b0, size_t bn) {
  return an && bn && a0 < b0 + bn && b0 < a0 + an;
}

bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > INT64_MAX / a) return false;
  *out = a * b;
  return true;
}

}  // namespace

extern "C" {

size_t ce_workspace_bytes(const ce_problem* p) {
  if (p == nullptr || p->T < 0 || p->num_segments < 0) return 0;
  if (p->num_segments == 0) return 0;
  return align_up(static_cast<size_t>(p->T) * sizeof(float)) +
         align_up((static_cast<size_t>(p->num_segments) + 1) * sizeof(int32_t));
}

const char* ce_status_string(int status) {
  switch (status) {
    case CE_OK: return "CE_OK";
    case CE_ERR_INVALID_ARG: return "CE_ERR_INVALID_ARG";
    case CE_ERR_UNSUPPORTED: return "CE_ERR_UNSUPPORTED";
    case CE_ERR_ALIAS: return "CE_ERR_ALIAS";
    case CE_ERR_WORKSPACE: return "CE_ERR_WORKSPACE";
    case CE_ERR_HIP: return "CE_ERR_HIP";
    default: return "CE_ERR_UNKNOWN";
  }
}

ce_status ce_fused_fwd_bwd(const ce_problem* p, const void* logits, const int64_t* targets,
                           const uint8_t* mask, const int32_t* segment_ids, float z_alpha,
                           float grad_scale, float* loss_out, float* seg_loss_out,
                           void* grad_out, void* workspace, size_t workspace_bytes,
                           void* stream_ptr) {
  // ---- host validation: nothing is enqueued on failure ----
  if (p == nullptr) return CE_ERR_INVALID_ARG;
  const int64_t T = p->T, V = p->V;
  if (T < 0 || V < 1) return CE_ERR_INVALID_ARG;
  if (p->logits_dtype != CE_DTYPE_F32 && p->logits_dtype != CE_DTYPE_BF16) return CE_ERR_INVALID_ARG;
  if (grad_out && p->grad_dtype != CE_DTYPE_F32 && p->grad_dtype != CE_DTYPE_BF16)
    return CE_ERR_INVALID_ARG;
  if ((p->flags & ~CE_FLAG_SEGMENT_MEAN) != 0) return CE_ERR_INVALID_ARG;
  if (p->ld_logits < V) return CE_ERR_INVALID_ARG;
  if (grad_out && p->ld_grad < V) return CE_ERR_INVALID_ARG;
  if (p->num_segments < 0) return CE_ERR_INVALID_ARG;
  // With rows, segment ids come exactly when segments are declared; with no
  // rows the ids are never read and may be NULL.
  if (T > 0 && (segment_ids != nullptr) != (p->num_segments > 0)) return CE_ERR_INVALID_ARG;
  if (T == 0 && segment_ids != nullptr && p->num_segments == 0) return CE_ERR_INVALID_ARG;
  if (seg_loss_out && p->num_segments == 0) return CE_ERR_INVALID_ARG;
  if ((p->flags & CE_FLAG_SEGMENT_MEAN) && p->num_segments == 0) return CE_ERR_INVALID_ARG;
  if (T > INT32_MAX) return CE_ERR_UNSUPPORTED;  // segment offsets are int32
  if (T > 0 && (!logits || !targets || !loss_out)) return CE_ERR_INVALID_ARG;
  if (!std::isfinite(z_alpha) || !std::isfinite(grad_scale)) return CE_ERR_INVALID_ARG;

  const int bi = dtype_bytes(p->logits_dtype);
  const int bo = grad_out ? dtype_bytes(p->grad_dtype) : bi;
  int64_t in_elems = 0, out_elems = 0, tmp = 0;
  if (T > 0) {
    if (!mul_ok(T - 1, p->ld_logits, &tmp) || tmp > INT64_MAX - V) return CE_ERR_INVALID_ARG;
    in_elems = tmp + V;
    if (!mul_ok(in_elems, bi, &tmp)) return CE_ERR_INVALID_ARG;
    if (grad_out) {
      if (!mul_ok(T - 1, p->ld_grad, &tmp) || tmp > INT64_MAX - V) return CE_ERR_INVALID_ARG;
      out_elems = tmp + V;
      if (!mul_ok(out_elems, bo, &tmp)) return CE_ERR_INVALID_ARG;
    }
  }
  // In place only as an exact alias: same pointer, dtype and row stride.
  if (grad_out && T > 0) {
    const bool same = grad_out == logits && p->grad_dtype == p->logits_dtype &&
                      p->ld_grad == p->ld_logits;
    if (!same && ranges_overlap(reinterpret_cast<uintptr_t>(logits), static_cast<size_t>(in_elems) * bi,
                                reinterpret_cast<uintptr_t>(grad_out),
                                static_cast<size_t>(out_elems) * bo))
      return CE_ERR_ALIAS;
  }
  const size_t need = ce_workspace_bytes(p);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return CE_ERR_WORKSPACE;
  if (need > 0 && (reinterpret_cast<uintptr_t>(workspace) % 4) != 0) return CE_ERR_WORKSPACE;

  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  const int32_t S = p->num_segments;
  float* nll_ws = nullptr;
  int32_t* seg_start = nullptr;
  if (S > 0) {
    nll_ws = static_cast<float*>(workspace);
    seg_start = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) +
                                           align_up(static_cast<size_t>(T) * sizeof(float)));
    (void)hipGetLastError();
    const unsigned nb = static_cast<unsigned>((static_cast<int64_t>(S) + 1 + 255) / 256);
    hipLaunchKernelGGL(ce_seg_bounds_kernel, dim3(nb), dim3(256), 0, stream, segment_ids, T, S,
                       seg_start);
    if (hipGetLastError() != hipSuccess) return CE_ERR_HIP;
  }

  if (T > 0) {
    RowParams rp;
    rp.logits = logits;
    rp.grad = grad_out;
    rp.targets = targets;
    rp.mask = mask;
    rp.seg_ids = segment_ids;
    rp.seg_start = seg_start;
    rp.loss_out = loss_out;
    rp.nll_ws = seg_loss_out ? nll_ws : nullptr;
    rp.T = T;
    rp.V = V;
    rp.ld_in = p->ld_logits;
    rp.ld_out = grad_out ? p->ld_grad : p->ld_logits;
    rp.ignore_index = p->ignore_index;
    rp.num_segments = S;
    rp.seg_mean = (p->flags & CE_FLAG_SEGMENT_MEAN) ? 1 : 0;
    rp.z_alpha = z_alpha;
    rp.grad_scale = grad_scale;

    const bool vec_in = (reinterpret_cast<uintptr_t>(logits) % 16 == 0) &&
                        ((p->ld_logits * bi) % 16 == 0);
    const bool vec_out = !grad_out || ((reinterpret_cast<uintptr_t>(grad_out) % 16 == 0) &&
                                       ((p->ld_grad * bo) % 16 == 0));
    const bool vec = vec_in && vec_out;
    (void)hipGetLastError();
    ce_status st = (p->logits_dtype == CE_DTYPE_F32)
                       ? dispatch_out<float>(rp, p->grad_dtype, grad_out != nullptr, vec, stream)
                       : dispatch_out<bf16_t>(rp, p->grad_dtype, grad_out != nullptr, vec, stream);
    if (st != CE_OK) return st;
  }

  if (seg_loss_out) {
    hipLaunchKernelGGL(ce_seg_sum_kernel, dim3(static_cast<unsigned>(S)), dim3(256), 0, stream,
                       nll_ws, seg_start, S, seg_loss_out);
    if (hipGetLastError() != hipSuccess) return CE_ERR_HIP;
  }
  return CE_OK;
}

}  // extern "C"
