// Cross-entropy + z-loss with a distillation child on the same softmax pass,
// for MI355X (gfx950).
//
// Fast-LLM PR #552 ("Fuse GSPO into the monolithic compiled loss", PR body,
// What) lists distillation with CE and z-loss among the losses that share the
// vocabulary softmax and finish loss and gradient in one pass. Per row, with
// student logits z (the ones differentiated) and teacher logits y:
//   loss = NLL + alpha lse_z^2 + beta KL(softmax(y) || softmax(z))
//   grad = s (1 + 2 alpha lse_z + beta) softmax(z) - s beta softmax(y),
// the target column taken from the non-target logsumexps as for the NLL
// (torchtitan #5661, revised PR description, Numerics):
//   grad_t = s (-pS_nt + 2 alpha lse_z pS_t + beta (pT_nt - pS_nt)).
//
// One workgroup per row. Pass 1 keeps, per lane, the student's non-target
// (shift, sum), the teacher's non-target (shift, sum) and
// U = sum 2^d (y_j - z_j) in the teacher's shifted frame; the epilogue forms,
// in fp64,
//   KL = pT_t (NLL_z - NLL_y) + 2^(M_y - lse_y log2 e) U + pT_nt (lse_z - lse_y),
// every piece from the non-target statistics and the two target logits.
//
// Two kernels:
//  * distill_chunk_kernel (student and teacher of one dtype, 16-byte aligned
//    rows): a row is cut into 16-byte chunks, chunk i * BLOCK + tid being slot
//    i of thread tid. The first NRAW slots of both matrices stay in registers
//    and the next NLDS in LDS (copied there straight from HBM), so they are
//    read once; later slots are streamed U at a time, and pass 2 walks them
//    backwards so the re-reads find the most recently read lines still in the
//    caches. The target element is set to -inf in the one slot that holds it
//    (the slot index is the same for the whole workgroup), so the hot loops
//    carry no per-element test;
//  * distill_rows_kernel (any dtype mix, any alignment): 8 elements per lane
//    and step, both passes streamed.

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <type_traits>

#include "ce_fused.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlock = 256;
constexpr float kL2E = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint16_t to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Element access by dtype: load one element, or 8 consecutive elements of a
// 16-byte-aligned row (chunk c = elements 8c .. 8c + 7); NT marks a last use
// (pass 2), whose loads need not stay in the caches.
template <typename T> struct Ld;
template <> struct Ld<float> {
  static constexpr int BYTES = 4;
  __device__ static float one(const void* row, int64_t j) { return static_cast<const float*>(row)[j]; }
  template <bool NT>
  __device__ static void eight(const void* row, int64_t c, float (&x)[8]) {
    const u32x4* q = reinterpret_cast<const u32x4*>(static_cast<const char*>(row) + c * 32);
    const u32x4 a = NT ? __builtin_nontemporal_load(q) : q[0];
    const u32x4 b = NT ? __builtin_nontemporal_load(q + 1) : q[1];
    x[0] = __uint_as_float(a.x); x[1] = __uint_as_float(a.y);
    x[2] = __uint_as_float(a.z); x[3] = __uint_as_float(a.w);
    x[4] = __uint_as_float(b.x); x[5] = __uint_as_float(b.y);
    x[6] = __uint_as_float(b.z); x[7] = __uint_as_float(b.w);
  }
  __device__ static void put_one(void* row, int64_t j, float g) { static_cast<float*>(row)[j] = g; }
  __device__ static void put_eight(void* row, int64_t c, const float (&g)[8]) {
    u32x4* q = reinterpret_cast<u32x4*>(static_cast<char*>(row) + c * 32);
    const u32x4 a = {__float_as_uint(g[0]), __float_as_uint(g[1]), __float_as_uint(g[2]),
                     __float_as_uint(g[3])};
    const u32x4 b = {__float_as_uint(g[4]), __float_as_uint(g[5]), __float_as_uint(g[6]),
                     __float_as_uint(g[7])};
    __builtin_nontemporal_store(a, q);
    __builtin_nontemporal_store(b, q + 1);
  }
};
template <> struct Ld<uint16_t> {   // bf16
  static constexpr int BYTES = 2;
  __device__ static float one(const void* row, int64_t j) {
    return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(row)[j]) << 16);
  }
  template <bool NT>
  __device__ static void eight(const void* row, int64_t c, float (&x)[8]) {
    const u32x4* q = reinterpret_cast<const u32x4*>(static_cast<const char*>(row) + c * 16);
    const u32x4 a = NT ? __builtin_nontemporal_load(q) : q[0];
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ static void put_one(void* row, int64_t j, float g) {
    static_cast<uint16_t*>(row)[j] = to_bf16(g);
  }
  __device__ static void put_eight(void* row, int64_t c, const float (&g)[8]) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = static_cast<uint32_t>(to_bf16(g[2 * i])) |
             (static_cast<uint32_t>(to_bf16(g[2 * i + 1])) << 16);
    const u32x4 v = {w[0], w[1], w[2], w[3]};
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(static_cast<char*>(row) + c * 16));
  }
};

struct DistillParams {
  const void* logits;
  const void* teacher;
  void* grad;
  const int64_t* targets;
  const uint8_t* mask;
  float* loss_out;
  float* kl_out;
  int64_t T, V, ld_s, ld_t, ld_g, ignore_index;
  float z_alpha, kl_beta, grad_scale;
};

// A row's label with the mask folded in (ignore_index where the mask byte is
// 0: a row counts exactly when its label is not ignore_index and its mask
// byte is nonzero). Both are read-only for the call and are read through the
// scalar cache; the mask byte within its aligned 4-byte word when that word
// lies inside the mask, a plain byte load otherwise. (A vector load would be
// counted with the previous row's gradient stores, and waiting for it would
// wait for all of them.)
__device__ __forceinline__ int64_t row_label(const DistillParams& p, int64_t r) {
  const int64_t t = ((const __attribute__((address_space(4))) int64_t*)p.targets)[r];
  if (p.mask == nullptr) return t;
  const uintptr_t a = reinterpret_cast<uintptr_t>(p.mask + r);
  const uintptr_t w = a & ~uintptr_t{3};
  uint32_t m;
  if (w >= reinterpret_cast<uintptr_t>(p.mask) && w + 4 <= reinterpret_cast<uintptr_t>(p.mask + p.T)) {
    const uint32_t v = *(const __attribute__((address_space(4))) uint32_t*)w;
    m = (v >> (8u * static_cast<uint32_t>(a & 3u))) & 0xffu;
  } else {
    m = p.mask[r];
  }
  return m != 0 ? t : p.ignore_index;
}

// Running (shift, sum) in log2 units plus the teacher's U.
struct Part {
  float ms, ss;      // student non-target
  float mt, st, u;   // teacher non-target, sum 2^d (y - z)
};

// s_old 2^(m - M) + add: the one update of a (shift, sum) pair, used for the
// student and the teacher alike (the same arithmetic on equal inputs gives
// equal statistics, so a teacher equal to the student has KL exactly 0).
__device__ __forceinline__ float rescale(float m, float s, float M) {
  return (m == kNegInf || s == 0.f) ? 0.f : fexp2(m - M);
}
__device__ __forceinline__ void upd(float& m, float& s, float M, float add) {
  s = __builtin_fmaf(s, rescale(m, s, M), add);
  m = M;
}

// Fold N elements into the part: xs / xt with the target element at -inf,
// ws / wt the raw values for the teacher's weight y - z.
template <int N>
__device__ __forceinline__ void fold(Part& p, const float (&xs)[N], const float (&xt)[N],
                                     const float (&ws)[N], const float (&wt)[N]) {
  float gs = kNegInf, gt = kNegInf;
#pragma unroll
  for (int k = 0; k < N; ++k) {
    gs = fmaxf(gs, xs[k]);
    gt = fmaxf(gt, xt[k]);
  }
  const float ns = fmaxf(p.ms, gs * kL2E);
  if (ns != kNegInf) {
    float a = 0.f;
#pragma unroll
    for (int k = 0; k < N; ++k) a += fexp2(__builtin_fmaf(xs[k], kL2E, -ns));
    upd(p.ms, p.ss, ns, a);
  }
  const float nt = fmaxf(p.mt, gt * kL2E);
  if (nt != kNegInf) {
    float a = 0.f, au = 0.f;
#pragma unroll
    for (int k = 0; k < N; ++k) {
      const float e = fexp2(__builtin_fmaf(xt[k], kL2E, -nt));
      a += e;
      au += (e > 0.f) ? e * (wt[k] - ws[k]) : 0.f;
    }
    p.u = __builtin_fmaf(p.u, rescale(p.mt, p.st, nt), au);
    upd(p.mt, p.st, nt, a);
  }
}

__device__ __forceinline__ void merge(Part& a, const Part& b) {
  const float ns = fmaxf(a.ms, b.ms);
  if (ns != kNegInf) upd(a.ms, a.ss, ns, b.ss * rescale(b.ms, b.ss, ns));
  const float nt = fmaxf(a.mt, b.mt);
  if (nt != kNegInf) {
    a.u = __builtin_fmaf(a.u, rescale(a.mt, a.st, nt), b.u * rescale(b.mt, b.st, nt));
    upd(a.mt, a.st, nt, b.st * rescale(b.mt, b.st, nt));
  }
}

__device__ __forceinline__ Part shfl_xor(const Part& p, int off) {
  Part q;
  q.ms = __shfl_xor(p.ms, off, 64);
  q.ss = __shfl_xor(p.ss, off, 64);
  q.mt = __shfl_xor(p.mt, off, 64);
  q.st = __shfl_xor(p.st, off, 64);
  q.u = __shfl_xor(p.u, off, 64);
  return q;
}

__device__ __forceinline__ double sigmoid_d(double x) {
  if (x >= 0.0) return 1.0 / (1.0 + exp(-x));
  const double e = exp(x);
  return e / (1.0 + e);
}

struct Side {   // one distribution's row quantities, fp64
  double lse, nll, p_nt, p_t;
};

// From a non-target (shift, sum) in log2 units and the target logit.
__device__ __forceinline__ Side side(float M, float S, float zt) {
  const double lse_nt = (M == kNegInf || S == 0.f)
                            ? -HUGE_VAL
                            : static_cast<double>(M) / static_cast<double>(kL2E) + log(static_cast<double>(S));
  const double z = static_cast<double>(zt);
  const double x = lse_nt - z;
  const double l1p = log1p(exp(-fabs(x)));
  Side o;
  o.nll = (x > 0.0 ? x : 0.0) + l1p;
  o.lse = (lse_nt > z ? lse_nt : z) + l1p;
  o.p_nt = sigmoid_d(x);
  o.p_t = sigmoid_d(-x);
  return o;
}

struct RowOut {
  float cs, ct, ks, kt, gt;   // student / teacher factors, lse in log2 units, target grad
};

// The row's loss and KL from the block-reduced partial and the two target
// logits (written to the outputs), and the factors pass 2 needs.
__device__ __forceinline__ RowOut finish_row(const DistillParams& p, int64_t r, const Part& tot,
                                          float zs_t, float zt_t) {
  const Side S = side(tot.ms, tot.ss, zs_t);
  const Side Tt = side(tot.mt, tot.st, zt_t);
  const double alpha = p.z_alpha, beta = p.kl_beta, sc = p.grad_scale;
  double kl = (Tt.p_t > 0.0) ? Tt.p_t * (S.nll - Tt.nll) : 0.0;
  if (tot.mt != kNegInf && tot.st > 0.f) {
    const double l2t = static_cast<double>(kL2E) * Tt.lse;
    kl += exp2(static_cast<double>(tot.mt) - l2t) * static_cast<double>(tot.u);
    kl += Tt.p_nt * (S.lse - Tt.lse);
  }
  const double zl = (alpha == 0.0) ? 0.0 : 2.0 * alpha * S.lse;
  p.loss_out[r] = static_cast<float>(S.nll + ((alpha == 0.0) ? 0.0 : alpha * S.lse * S.lse) +
                                     beta * kl);
  if (p.kl_out) p.kl_out[r] = static_cast<float>(kl);
  RowOut o;
  // ks / kt hold lse log2(e) rounded to float; each residue is folded into
  // its side's factor, so an element's exponent is exact up to its own
  // rounding (2^(x - lse log2 e) = 2^(-residue) 2^(x - k)).
  const double ls2 = static_cast<double>(kL2E) * S.lse, lt2 = static_cast<double>(kL2E) * Tt.lse;
  o.ks = static_cast<float>(ls2);
  o.kt = static_cast<float>(lt2);
  const double rs_ = isfinite(ls2) ? ls2 - static_cast<double>(o.ks) : 0.0;
  const double rt_ = isfinite(lt2) ? lt2 - static_cast<double>(o.kt) : 0.0;
  o.cs = static_cast<float>(sc * (1.0 + zl + beta) * exp2(-rs_));
  o.ct = static_cast<float>(sc * beta * exp2(-rt_));
  o.gt = static_cast<float>(sc * (-S.p_nt + zl * S.p_t + beta * (Tt.p_nt - S.p_nt)));
  return o;
}

template <typename TS, typename TT, typename TO, bool VEC>
__global__ __launch_bounds__(kBlock) void distill_rows_kernel(DistillParams p) {
  __shared__ Part red[kBlock / 64];
  __shared__ RowOut out_sh;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int64_t V = p.V;
  const int64_t nch = VEC ? V / 8 : 0;            // full 8-element chunks
  const int64_t tail0 = nch * 8;                  // first element of the tail
  for (int64_t r = blockIdx.x; r < p.T; r += gridDim.x) {
    const int64_t t = row_label(p, r);
    const bool valid = t != p.ignore_index;   // (the mask is folded into the label)
    const bool owned = t >= 0 && t < V;
    void* grow = p.grad ? static_cast<char*>(p.grad) + r * p.ld_g * Ld<TO>::BYTES : nullptr;
    if (!valid || !owned) {
      const float fill = valid ? __builtin_nanf("") : 0.f;
      if (tid == 0) {
        p.loss_out[r] = fill;
        if (p.kl_out) p.kl_out[r] = fill;
      }
      if (grow) {
        const float f8[8] = {fill, fill, fill, fill, fill, fill, fill, fill};
        for (int64_t c = tid; c < nch; c += kBlock) Ld<TO>::put_eight(grow, c, f8);
        for (int64_t j = tail0 + tid; j < V; j += kBlock) Ld<TO>::put_one(grow, j, fill);
      }
      continue;
    }
    const void* srow = static_cast<const char*>(p.logits) + r * p.ld_s * Ld<TS>::BYTES;
    const void* trow = static_cast<const char*>(p.teacher) + r * p.ld_t * Ld<TT>::BYTES;
    const float zs_t = Ld<TS>::one(srow, t), zt_t = Ld<TT>::one(trow, t);

    // ---- pass 1 ----
    Part pa{kNegInf, 0.f, kNegInf, 0.f, 0.f};
    for (int64_t c = tid; c < nch; c += kBlock) {
      float ws[8], wt[8], xs[8], xt[8];
      Ld<TS>::template eight<false>(srow, c, ws);
      Ld<TT>::template eight<false>(trow, c, wt);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const bool tgt = c * 8 + k == t;
        xs[k] = tgt ? kNegInf : ws[k];
        xt[k] = tgt ? kNegInf : wt[k];
      }
      fold<8>(pa, xs, xt, ws, wt);
    }
    for (int64_t j = tail0 + tid; j < V; j += kBlock) {
      float ws[1] = {Ld<TS>::one(srow, j)}, wt[1] = {Ld<TT>::one(trow, j)};
      float xs[1] = {j == t ? kNegInf : ws[0]}, xt[1] = {j == t ? kNegInf : wt[0]};
      fold<1>(pa, xs, xt, ws, wt);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) merge(pa, shfl_xor(pa, off));
    if (lane == 0) red[wid] = pa;
    __syncthreads();
    if (tid == 0) {
      Part tot = red[0];
#pragma unroll
      for (int w = 1; w < kBlock / 64; ++w) merge(tot, red[w]);
      // ---- fp64 epilogue ----
      const RowOut o = finish_row(p, r, tot, zs_t, zt_t);
      out_sh = o;
    }
    __syncthreads();
    const RowOut o = out_sh;

    // ---- pass 2 ----
    if (grow) {
      const bool teach = o.ct != 0.f;
      for (int64_t c = tid; c < nch; c += kBlock) {
        float ws[8], wt[8], g[8];
        Ld<TS>::template eight<true>(srow, c, ws);
        if (teach) Ld<TT>::template eight<true>(trow, c, wt);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          float v = o.cs * fexp2(__builtin_fmaf(ws[k], kL2E, -o.ks));
          if (teach) v -= o.ct * fexp2(__builtin_fmaf(wt[k], kL2E, -o.kt));
          g[k] = (c * 8 + k == t) ? o.gt : v;
        }
        Ld<TO>::put_eight(grow, c, g);
      }
      for (int64_t j = tail0 + tid; j < V; j += kBlock) {
        float v = o.cs * fexp2(__builtin_fmaf(Ld<TS>::one(srow, j), kL2E, -o.ks));
        if (teach) v -= o.ct * fexp2(__builtin_fmaf(Ld<TT>::one(trow, j), kL2E, -o.kt));
        Ld<TO>::put_one(grow, j, j == t ? o.gt : v);
      }
    }
    __syncthreads();   // out_sh and red are rewritten by the next row
  }
}

// ---------------------------------------------------------------------------
// Chunk kernel: student and teacher of one dtype, 16-byte aligned rows
// ---------------------------------------------------------------------------

constexpr int kNT = 2;                   // cache policy bits: non-temporal
constexpr int kBufWord3 = 0x00020000;    // buffer descriptor word 3 (raw buffer)

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2 f = {a, b};
  const bf16x2 h = __builtin_convertvector(f, bf16x2);   // round to nearest even
  return __builtin_bit_cast(uint32_t, h);
}

// A 16-byte chunk of input: W elements; NEG is a word of -inf elements.
template <typename T> struct Chunk;
template <> struct Chunk<float> {
  static constexpr int W = 4;
  static constexpr uint32_t NEG = 0xff800000u;
  __device__ static void unpack(const u32x4 v, float* x) {
    x[0] = __uint_as_float(v.x);
    x[1] = __uint_as_float(v.y);
    x[2] = __uint_as_float(v.z);
    x[3] = __uint_as_float(v.w);
  }
};
template <> struct Chunk<uint16_t> {
  static constexpr int W = 8;
  static constexpr uint32_t NEG = 0xff80ff80u;
  __device__ static void unpack(const u32x4 v, float* x) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};

// The gradient of one chunk (W values) at byte offset vo of the row's window.
template <typename TO, int W>
__device__ __forceinline__ void put_chunk(__amdgpu_buffer_rsrc_t rg, uint32_t vo, const float* g) {
  if constexpr (sizeof(TO) == 2 && W == 8) {
    const u32x4 q = {pack_bf16x2(g[0], g[1]), pack_bf16x2(g[2], g[3]), pack_bf16x2(g[4], g[5]),
                     pack_bf16x2(g[6], g[7])};
    __builtin_amdgcn_raw_buffer_store_b128(q, rg, vo, 0, kNT);
  } else if constexpr (sizeof(TO) == 2) {   // 4 fp32 in -> 4 bf16 out
    const u32x2 q = {pack_bf16x2(g[0], g[1]), pack_bf16x2(g[2], g[3])};
    __builtin_amdgcn_raw_buffer_store_b64(q, rg, vo, 0, kNT);
  } else {
#pragma unroll
    for (int h = 0; h < W / 4; ++h) {
      const u32x4 q = {__float_as_uint(g[4 * h]), __float_as_uint(g[4 * h + 1]),
                       __float_as_uint(g[4 * h + 2]), __float_as_uint(g[4 * h + 3])};
      __builtin_amdgcn_raw_buffer_store_b128(q, rg, vo + 16u * h, 0, kNT);
    }
  }
}

template <int POL>
__device__ __forceinline__ u32x4 ld16(__amdgpu_buffer_rsrc_t rr, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(rr, off, 0, POL);
}

// The window [off, bytes) of a row, off < bytes, formed with scalar
// arithmetic: lanes index it from 0, and the hardware range check returns 0
// for loads past its end and drops stores there.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t window(const void* row, uint32_t off,
                                                         uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(static_cast<const char*>(row)) + off,
                                           0, bytes - off, kBufWord3);
}

// The empty asm marks the registers as rewritten (no instruction is emitted),
// so floats unpacked from a resident chunk in pass 1 are not kept alive for
// pass 2: a resident chunk costs 4 registers between the passes.
__device__ __forceinline__ void touch(u32x4& v) { asm volatile("" : "+v"(v)); }

// Fold N values of each side into the part: xs / xt hold -inf where a value
// is absent (the target column, lanes past the row end). One shift update per
// call; the teacher's U term takes e (y - z) with y - z clamped below at
// -FLT_MAX, so absent pairs (-inf - -inf) and teacher zeros add 0, and a
// student zero under a live teacher value adds +inf.
template <int N>
__device__ __forceinline__ void fold_group(Part& p, const float* xs, const float* xt) {
  float gs = kNegInf, gt = kNegInf;
#pragma unroll
  for (int k = 0; k < N; ++k) {
    gs = fmaxf(gs, xs[k]);
    gt = fmaxf(gt, xt[k]);
  }
  const float ns = fmaxf(p.ms, gs * kL2E);
  const float hs = ns == kNegInf ? 0.f : ns;
  float as = 0.f;
#pragma unroll
  for (int k = 0; k < N; ++k) as += fexp2(__builtin_fmaf(xs[k], kL2E, -hs));
  p.ss = __builtin_fmaf(p.ss, fexp2(p.ms - hs), as);
  p.ms = ns;
  const float nt = fmaxf(p.mt, gt * kL2E);
  const float ht = nt == kNegInf ? 0.f : nt;
  float at = 0.f, au = 0.f;
#pragma unroll
  for (int k = 0; k < N; ++k) {
    const float e = fexp2(__builtin_fmaf(xt[k], kL2E, -ht));
    at += e;
    au = __builtin_fmaf(e, fmaxf(xt[k] - xs[k], -__FLT_MAX__), au);
  }
  const float f = fexp2(p.mt - ht);
  p.st = __builtin_fmaf(p.st, f, at);
  p.u = __builtin_fmaf(p.u, f, au);
  p.mt = nt;
}

//   TI     : student and teacher element type
//   TO     : gradient element type
//   BLOCK  : threads per workgroup
//   NRAW   : slots per thread of each matrix kept in registers between passes
//   NLDS   : slots per thread of each matrix kept in LDS (HBM -> LDS directly)
//   U      : streamed slots per thread and step
template <typename TI, typename TO, int BLOCK, int NRAW, int NLDS, int U>
__global__ __launch_bounds__(BLOCK) void distill_chunk_kernel(DistillParams p) {
  constexpr int W = Chunk<TI>::W;
  constexpr uint32_t OB = W * sizeof(TO);          // gradient bytes per chunk
  constexpr uint32_t NON = NRAW + NLDS;            // on-chip slots per thread
  static_assert(BLOCK % 64 == 0 && BLOCK <= 1024, "whole waves");
  __shared__ Part red[2][BLOCK / 64];
  __shared__ RowOut outs[2];
  __shared__ u32x4 stS[NLDS > 0 ? NLDS : 1][NLDS > 0 ? BLOCK : 1];
  __shared__ u32x4 stT[NLDS > 0 ? NLDS : 1][NLDS > 0 ? BLOCK : 1];

  const uint32_t tid = threadIdx.x, lane = tid & 63u, wid = tid >> 6;
  // In-row byte offsets are 32-bit (the host bounds a row below 2 GiB).
  const uint32_t V = static_cast<uint32_t>(p.V);
  const uint32_t nchunk = V / W;
  const uint32_t c16_last = (nchunk > 0 ? nchunk - 1 : 0) * 16u;
  const uint32_t tail_begin = nchunk * W;
  const uint32_t nslot = (nchunk + BLOCK - 1) / BLOCK;
  const u32x4 neg4 = {Chunk<TI>::NEG, Chunk<TI>::NEG, Chunk<TI>::NEG, Chunk<TI>::NEG};
  // Labels (mask folded in) are read through the scalar cache, one row ahead,
  // so a row does not open by waiting on a vector load (and with it on the
  // previous row's stores).
  int64_t t_next = static_cast<int64_t>(blockIdx.x) < p.T ? row_label(p, blockIdx.x) : 0;
  int par = 0;
  for (int64_t r = blockIdx.x; r < p.T; r += gridDim.x, par ^= 1) {
    const int64_t t64 = t_next;
    if (r + gridDim.x < p.T) t_next = row_label(p, r + gridDim.x);
    const bool valid = t64 != p.ignore_index;   // (the mask is folded into the label)
    const bool owned = t64 >= 0 && t64 < static_cast<int64_t>(V);
    void* grow = p.grad ? static_cast<char*>(p.grad) + r * p.ld_g * static_cast<int64_t>(sizeof(TO))
                        : nullptr;
    if (!valid || !owned) {
      // Ignored row: +0.0 everywhere. Valid row with an out-of-range
      // target: NaN loss, KL and gradient row.
      const float fill = valid ? __builtin_nanf("") : 0.f;
      if (tid == 0) {
        p.loss_out[r] = fill;
        if (p.kl_out) p.kl_out[r] = fill;
      }
      if (grow) {
        float f[W];
#pragma unroll
        for (int k = 0; k < W; ++k) f[k] = fill;
        const __amdgpu_buffer_rsrc_t rg =
            __builtin_amdgcn_make_buffer_rsrc(grow, 0, nchunk * OB, kBufWord3);
        for (uint32_t c = tid; c < nchunk; c += BLOCK) put_chunk<TO, W>(rg, c * OB, f);
        if (tid < V - tail_begin) Ld<TO>::put_one(grow, tail_begin + tid, fill);
      }
      continue;
    }
    const uint32_t t = static_cast<uint32_t>(t64);
    const char* srow = static_cast<const char*>(p.logits) + r * p.ld_s * static_cast<int64_t>(sizeof(TI));
    const char* trow = static_cast<const char*>(p.teacher) + r * p.ld_t * static_cast<int64_t>(sizeof(TI));
    const float zs_t = Ld<TI>::one(srow, t), zt_t = Ld<TI>::one(trow, t);
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(srow), 0, nchunk * 16u, kBufWord3);
    const __amdgpu_buffer_rsrc_t rt =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(trow), 0, nchunk * 16u, kBufWord3);

    // The target: chunk ct, element kt, slot st (the same for every thread),
    // lane `mine`. Word masks put -inf into element kt in that lane only.
    const uint32_t ct = t / W, kt = t - ct * W;
    const bool in_chunks = t < tail_begin;
    const uint32_t st = in_chunks ? ct / BLOCK : 0xffffffffu;
    const bool mine = in_chunks && ct - (ct / BLOCK) * BLOCK == tid;
    const uint32_t kq = (kt * static_cast<uint32_t>(sizeof(TI))) >> 2;
    const uint32_t ksh = (kt * static_cast<uint32_t>(sizeof(TI)) * 8u) & 31u;
    const uint32_t kmask = sizeof(TI) == 4 ? 0xffffffffu : (0xffffu << ksh);
    const uint32_t kput = sizeof(TI) == 4 ? 0xff800000u : (0xff80u << ksh);
    const u32x4 and_m = {mine && kq == 0 ? ~kmask : ~0u, mine && kq == 1 ? ~kmask : ~0u,
                         mine && kq == 2 ? ~kmask : ~0u, mine && kq == 3 ? ~kmask : ~0u};
    const u32x4 or_m = {mine && kq == 0 ? kput : 0u, mine && kq == 1 ? kput : 0u,
                        mine && kq == 2 ? kput : 0u, mine && kq == 3 ? kput : 0u};

    // On-chip slots: offsets clamped to the last chunk, so every load is in
    // bounds. Streamed slots: one window per step of U slots starting at slot
    // i, lane offset (u BLOCK + tid) 16 for its u-th slot.
    // prep() turns lanes past the row end into -inf (only the row's last slot
    // has any) and masks the target in its slot.
    uint32_t vin = tid * 16u;
    asm volatile("" : "+v"(vin));
    auto off = [&](uint32_t slot) { return min(vin + slot * (BLOCK * 16u), c16_last); };
    auto prep = [&](u32x4& v, uint32_t slot) {
      if (slot * BLOCK + BLOCK > nchunk && slot * BLOCK + tid >= nchunk) v = neg4;
      if (slot == st) v = (v & and_m) | or_m;
    };
    auto sload = [&](const char* row, uint32_t i, int u, auto pol) {
      return ld16<decltype(pol)::value>(window(row, i * (BLOCK * 16u), nchunk * 16u),
                                        tid * 16u + u * (BLOCK * 16u));
    };
    // A step of U streamed slots needs fix-ups only if it holds the row's
    // end or the target (the same for the whole workgroup).
    auto special = [&](uint32_t i) { return (i + U) * BLOCK > nchunk || st - i < U; };

    // ---- issue every on-chip load first ----
    u32x4 rS[NRAW > 0 ? NRAW : 1], rT[NRAW > 0 ? NRAW : 1];
    if (nchunk > 0) {
#pragma unroll
      for (int i = 0; i < NRAW; ++i) {
        rS[i] = ld16<kNT>(rs, off(i));
        rT[i] = ld16<kNT>(rt, off(i));
      }
#pragma unroll
      for (int i = 0; i < NLDS; ++i) {
        // lane l of a wave lands at base + 16 l: slot i of thread tid is st*[i][tid]
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void*)(srow + off(NRAW + i)),
            (__attribute__((address_space(3))) void*)(&stS[i][tid & ~63u]), 16, 0, kNT);
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void*)(trow + off(NRAW + i)),
            (__attribute__((address_space(3))) void*)(&stT[i][tid & ~63u]), 16, 0, kNT);
      }
    }

    // ---- pass 1 ----
    Part pa{kNegInf, 0.f, kNegInf, 0.f, 0.f};
    if (NRAW > 0 && nchunk > 0) {
      float xs[NRAW > 0 ? NRAW * W : 1], xt[NRAW > 0 ? NRAW * W : 1];
#pragma unroll
      for (int i = 0; i < NRAW; ++i) {
        prep(rS[i], i);
        prep(rT[i], i);
        Chunk<TI>::unpack(rS[i], xs + i * W);
        Chunk<TI>::unpack(rT[i], xt + i * W);
      }
      fold_group<NRAW * W>(pa, xs, xt);
#pragma unroll
      for (int i = 0; i < NRAW; ++i) {
        touch(rS[i]);
        touch(rT[i]);
      }
    }
    if (NLDS > 0 && nchunk > 0) {
      __builtin_amdgcn_s_waitcnt(0);   // this wave's HBM -> LDS copies have landed
      constexpr int G = NLDS < 4 ? NLDS : 4;
#pragma unroll
      for (int i0 = 0; i0 < NLDS; i0 += G) {
        float xs[G * W], xt[G * W];
#pragma unroll
        for (int i = i0; i < i0 + G && i < NLDS; ++i) {
          u32x4 a = stS[i][tid], b = stT[i][tid];
          prep(a, NRAW + i);
          prep(b, NRAW + i);
          Chunk<TI>::unpack(a, xs + (i - i0) * W);
          Chunk<TI>::unpack(b, xt + (i - i0) * W);
        }
        fold_group<G * W>(pa, xs, xt);
      }
    }
    for (uint32_t i = NON; i < nslot; i += U) {
      u32x4 a[U], b[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        a[u] = sload(srow, i, u, std::integral_constant<int, 0>{});
        b[u] = sload(trow, i, u, std::integral_constant<int, 0>{});
      }
      if (special(i)) {
        // a real branch (not selects): the fix-ups cost nothing elsewhere
        asm volatile("");
#pragma unroll
        for (int u = 0; u < U; ++u) {
          prep(a[u], i + u);
          prep(b[u], i + u);
        }
      }
      float xs[U * W], xt[U * W];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        Chunk<TI>::unpack(a[u], xs + u * W);
        Chunk<TI>::unpack(b[u], xt + u * W);
      }
      fold_group<U * W>(pa, xs, xt);
    }
    if (tid < V - tail_begin) {
      const uint32_t j = tail_begin + tid;
      const float xs[1] = {j == t ? kNegInf : Ld<TI>::one(srow, j)};
      const float xt[1] = {j == t ? kNegInf : Ld<TI>::one(trow, j)};
      fold_group<1>(pa, xs, xt);
    }

    // ---- reduction and fp64 epilogue ----
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) merge(pa, shfl_xor(pa, o));
    if (lane == 0) red[par][wid] = pa;
    __syncthreads();
    if (tid == 0) {
      Part tot = red[par][0];
#pragma unroll
      for (int w = 1; w < BLOCK / 64; ++w) merge(tot, red[par][w]);
      outs[par] = finish_row(p, r, tot, zs_t, zt_t);
    }
    __syncthreads();
    const RowOut o = outs[par];
    if (grow == nullptr) continue;

    // ---- pass 2: gradient; streamed slots newest first, then on-chip ----
    // Stores go through windows like the loads: those past the row end are
    // dropped.
    auto store = [&](uint32_t i, int u, const float* g) {
      put_chunk<TO, W>(window(grow, i * (BLOCK * OB), nchunk * OB), tid * OB + u * (BLOCK * OB), g);
    };
    auto pass2 = [&](auto teach_c) {
      constexpr bool TEACH = decltype(teach_c)::value;
      auto grad = [&](const u32x4 a, const u32x4 b, float* g) {
        float xs[W];
        Chunk<TI>::unpack(a, xs);
        if constexpr (TEACH) {
          float xt[W];
          Chunk<TI>::unpack(b, xt);
#pragma unroll
          for (int k = 0; k < W; ++k)
            g[k] = __builtin_fmaf(o.cs, fexp2(__builtin_fmaf(xs[k], kL2E, -o.ks)),
                                  -o.ct * fexp2(__builtin_fmaf(xt[k], kL2E, -o.kt)));
        } else {
#pragma unroll
          for (int k = 0; k < W; ++k) g[k] = o.cs * fexp2(__builtin_fmaf(xs[k], kL2E, -o.ks));
        }
      };
      if (nslot > NON) {
        for (uint32_t gi = (nslot - NON + U - 1) / U; gi-- > 0;) {
          const uint32_t i = NON + gi * U;
          u32x4 a[U], b[U];
#pragma unroll
          for (int u = 0; u < U; ++u) {
            a[u] = sload(srow, i, u, std::integral_constant<int, kNT>{});
            if constexpr (TEACH) b[u] = sload(trow, i, u, std::integral_constant<int, kNT>{});
          }
#pragma unroll
          for (int u = 0; u < U; ++u) {
            float g[W];
            grad(a[u], b[u], g);
            store(i, u, g);
          }
        }
      }
      if (tid < V - tail_begin) {
        const uint32_t j = tail_begin + tid;
        float v = o.cs * fexp2(__builtin_fmaf(Ld<TI>::one(srow, j), kL2E, -o.ks));
        if constexpr (TEACH) v -= o.ct * fexp2(__builtin_fmaf(Ld<TI>::one(trow, j), kL2E, -o.kt));
        Ld<TO>::put_one(grow, j, j == t ? o.gt : v);
      }
#pragma unroll
      for (int i = 0; i < NLDS; ++i) {
        float g[W];
        grad(stS[i][tid], stT[i][tid], g);
        store(0, NRAW + i, g);
      }
#pragma unroll
      for (int i = 0; i < NRAW; ++i) {
        float g[W];
        grad(rS[i], rT[i], g);
        store(0, i, g);
      }
    };
    if (o.ct != 0.f) {
      pass2(std::integral_constant<bool, true>{});
    } else {
      pass2(std::integral_constant<bool, false>{});
    }
    // The target column: written after its chunk by the same lane, so this
    // store lands last (a lane's stores to one address stay in order).
    if (mine) Ld<TO>::put_one(grow, t, o.gt);
    if constexpr (NLDS > 0) {
      // The next row's HBM -> LDS copies overwrite the staging slots: this
      // wave's reads of them must have returned first.
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

int device_cus_distill() {
  static std::atomic<int> cus{0};
  int c = cus.load();
  if (c == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0)
      c = 256;
    cus.store(c);
  }
  return c;
}

template <typename TI, typename TO, int B, int NRAW, int NLDS, int U>
ce_status launch_chunk(const DistillParams& dp, hipStream_t st) {
  auto kern = distill_chunk_kernel<TI, TO, B, NRAW, NLDS, U>;
  // One resident wave of workgroups: as many per CU as fit.
  static std::atomic<int> per_cu{0};
  int n = per_cu.load();
  if (n == 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, B, 0) != hipSuccess || n < 1) n = 1;
    per_cu.store(n);
  }
  const int64_t grid = std::min<int64_t>(dp.T, static_cast<int64_t>(n) * device_cus_distill());
  if (grid <= 0) return CE_OK;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(B), 0, st, dp);
  return hipGetLastError() == hipSuccess ? CE_OK : CE_ERR_HIP;
}

// Shapes measured on MI355X (one call, both passes, beta != 0):
//  * bf16 rows up to 64 K columns: 256 threads, 4 LDS slots, no register
//    slots -- three workgroups per CU hide each other's row epilogues;
//  * longer bf16 rows: 256 threads, 4 register + 8 LDS slots, two per CU;
//  * fp32 rows: 1024 threads, 2 register + 4 LDS slots, 2 slots per step
//    (512 threads, 4 + 4 slots when the gradient is bf16: the wider shape
//    spills there).
template <typename TI, typename TO>
ce_status dispatch_chunk(const DistillParams& dp, hipStream_t st) {
  if constexpr (sizeof(TI) == 2) {
    if (dp.V <= 65536) return launch_chunk<TI, TO, 256, 0, 4, 4>(dp, st);
    return launch_chunk<TI, TO, 256, 4, 8, 4>(dp, st);
  } else if constexpr (sizeof(TO) == 4) {
    return launch_chunk<TI, TO, 1024, 2, 4, 2>(dp, st);
  } else {
    return launch_chunk<TI, TO, 512, 4, 4, 4>(dp, st);
  }
}

template <typename TS, typename TT, typename TO, bool VEC>
ce_status launch_distill(const DistillParams& dp, hipStream_t st) {
  const int64_t grid = std::min<int64_t>(dp.T, 16LL * device_cus_distill());
  if (grid <= 0) return CE_OK;
  hipLaunchKernelGGL((distill_rows_kernel<TS, TT, TO, VEC>), dim3(static_cast<unsigned>(grid)),
                     dim3(kBlock), 0, st, dp);
  return hipGetLastError() == hipSuccess ? CE_OK : CE_ERR_HIP;
}

template <typename TS, typename TT>
ce_status dispatch_o(const DistillParams& dp, int32_t grad_dtype, bool vec, hipStream_t st) {
  if (grad_dtype == CE_DTYPE_F32)
    return vec ? launch_distill<TS, TT, float, true>(dp, st) : launch_distill<TS, TT, float, false>(dp, st);
  return vec ? launch_distill<TS, TT, uint16_t, true>(dp, st)
             : launch_distill<TS, TT, uint16_t, false>(dp, st);
}

template <typename TS>
ce_status dispatch_t(const DistillParams& dp, int32_t teacher_dtype, int32_t grad_dtype, bool vec,
                     hipStream_t st) {
  return teacher_dtype == CE_DTYPE_F32 ? dispatch_o<TS, float>(dp, grad_dtype, vec, st)
                                       : dispatch_o<TS, uint16_t>(dp, grad_dtype, vec, st);
}

int dbytes(int32_t dt) { return dt == CE_DTYPE_F32 ? 4 : 2; }

bool span(int64_t T, int64_t V, int64_t ld, int b, size_t* out) {
  if (T == 0) {
    *out = 0;
    return true;
  }
  if (ld > (INT64_MAX - V) / T) return false;
  *out = static_cast<size_t>(((T - 1) * ld + V) * b);
  return true;
}

bool overlap(const void* a, size_t an, const void* b, size_t bn) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a && b && an && bn && a0 < b0 + bn && b0 < a0 + an;
}

bool rows16(const void* ptr, int64_t ld, int b) {
  return ptr == nullptr || ((reinterpret_cast<uintptr_t>(ptr) % 16 == 0) && (ld * b) % 16 == 0);
}

}  // namespace

extern "C" ce_status ce_fused_distill(const ce_problem* p, const void* logits, const void* teacher,
                                      int64_t ld_teacher, int32_t teacher_dtype,
                                      const int64_t* targets, const uint8_t* mask, float z_alpha,
                                      float kl_beta, float grad_scale, float* loss_out,
                                      float* kl_out, void* grad_out, void* stream_ptr) {
  if (p == nullptr) return CE_ERR_INVALID_ARG;
  const int64_t T = p->T, V = p->V;
  if (T < 0 || V < 1 || p->ld_logits < V || ld_teacher < V) return CE_ERR_INVALID_ARG;
  const bool dt_ok = [](int32_t d) { return d == CE_DTYPE_F32 || d == CE_DTYPE_BF16; }(p->logits_dtype);
  if (!dt_ok || (teacher_dtype != CE_DTYPE_F32 && teacher_dtype != CE_DTYPE_BF16))
    return CE_ERR_INVALID_ARG;
  if (grad_out && ((p->grad_dtype != CE_DTYPE_F32 && p->grad_dtype != CE_DTYPE_BF16) ||
                   p->ld_grad < V))
    return CE_ERR_INVALID_ARG;
  if (p->flags != 0) return CE_ERR_INVALID_ARG;
  if (p->num_segments != 0) return CE_ERR_UNSUPPORTED;   // no segment sums on this child
  if (!std::isfinite(z_alpha) || !std::isfinite(kl_beta) || !std::isfinite(grad_scale))
    return CE_ERR_INVALID_ARG;
  if (T > 0 && (!logits || !teacher || !targets || !loss_out)) return CE_ERR_INVALID_ARG;
  const int bs = dbytes(p->logits_dtype), bt = dbytes(teacher_dtype);
  const int bo = grad_out ? dbytes(p->grad_dtype) : bs;
  size_t ns = 0, nt = 0, no = 0;
  if (!span(T, V, p->ld_logits, bs, &ns) || !span(T, V, ld_teacher, bt, &nt) ||
      (grad_out && !span(T, V, p->ld_grad, bo, &no)))
    return CE_ERR_INVALID_ARG;
  // The gradient may replace the student logits exactly (same dtype and
  // stride); it may not touch the teacher; the row outputs touch neither.
  if (grad_out) {
    const bool same = grad_out == logits && p->grad_dtype == p->logits_dtype &&
                      p->ld_grad == p->ld_logits;
    if ((!same && overlap(grad_out, no, logits, ns)) || overlap(grad_out, no, teacher, nt))
      return CE_ERR_ALIAS;
  }
  for (const float* o : {static_cast<const float*>(loss_out), static_cast<const float*>(kl_out)})
    if (overlap(o, static_cast<size_t>(T) * 4, logits, ns) ||
        overlap(o, static_cast<size_t>(T) * 4, teacher, nt) ||
        overlap(o, static_cast<size_t>(T) * 4, grad_out, no))
      return CE_ERR_ALIAS;
  if (T == 0) return CE_OK;

  DistillParams dp{};
  dp.logits = logits;
  dp.teacher = teacher;
  dp.grad = grad_out;
  dp.targets = targets;
  dp.mask = mask;
  dp.loss_out = loss_out;
  dp.kl_out = kl_out;
  dp.T = T;
  dp.V = V;
  dp.ld_s = p->ld_logits;
  dp.ld_t = ld_teacher;
  dp.ld_g = grad_out ? p->ld_grad : p->ld_logits;
  dp.ignore_index = p->ignore_index;
  dp.z_alpha = z_alpha;
  dp.kl_beta = kl_beta;
  dp.grad_scale = grad_scale;
  const bool vec = rows16(logits, p->ld_logits, bs) && rows16(teacher, ld_teacher, bt) &&
                   rows16(grad_out, p->ld_grad, bo);
  hipStream_t st = static_cast<hipStream_t>(stream_ptr);
  (void)hipGetLastError();
  // One dtype for both matrices, 16-byte rows and row windows below 2 GiB:
  // the chunk kernel.
  if (vec && teacher_dtype == p->logits_dtype && V <= (int64_t{1} << 31) / 4 - 1) {
    const bool gf = !grad_out || p->grad_dtype == CE_DTYPE_F32;
    if (p->logits_dtype == CE_DTYPE_F32)
      return gf ? dispatch_chunk<float, float>(dp, st) : dispatch_chunk<float, uint16_t>(dp, st);
    return gf ? dispatch_chunk<uint16_t, float>(dp, st) : dispatch_chunk<uint16_t, uint16_t>(dp, st);
  }
  return p->logits_dtype == CE_DTYPE_F32
             ? dispatch_t<float>(dp, teacher_dtype, p->grad_dtype, vec, st)
             : dispatch_t<uint16_t>(dp, teacher_dtype, p->grad_dtype, vec, st);
}
