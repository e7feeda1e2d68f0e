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
//  * rows are read through a per-row buffer descriptor in 16-byte chunks:
//    lane tid of slot i owns chunk i * BLOCK + tid, so one VGPR offset per
//    lane plus a constant SGPR offset per slot address everything;
//  * the first slots of each thread stay on chip between the two passes --
//    as fp32 exps (NRES), as raw input in VGPRs (NRAW) or as raw input in LDS
//    filled straight from HBM (NLDS) -- so they are read from HBM once; any
//    remaining slots are streamed in pass 1 and read again in pass 2;
//  * statistics are kept in the log2 domain: every exponential is one
//    v_exp_f32 of an FMA, and a partial is (shift, sum) with the shift a
//    float that the merges use exactly;
//  * the target column is set to -inf in the raw registers of the one lane
//    that holds it, so no per-element test remains in the hot loops; its
//    gradient is written by that lane after the row's chunk stores;
//  * wave reduction by lane shuffles, then one LDS slot per wave;
//  * the per-row epilogue (softplus, logaddexp, sigmoids, z-loss) in fp64;
//  * per-segment NLL sums by a second kernel that walks each segment's rows
//    in a fixed order (deterministic, no atomics).

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "ce_fused.h"

namespace {

constexpr float kL2E = 1.44269504088896340736f;  // log2(e), rounded to float
constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kNT = 2;                           // cache policy bits: non-temporal
// Read-only int64 in the constant address space: uniform loads become scalar
// loads through the scalar cache.
typedef const __attribute__((address_space(4))) int64_t kconst_i64;
typedef const __attribute__((address_space(4))) int32_t kconst_i32;
constexpr int kBufWord3 = 0x00020000;            // buffer descriptor word 3 (gfx9 raw buffer)
// s_waitcnt immediate (gfx9 layout): wait until at most `vm` vector memory,
// `exp` export and `lgkm` LDS/scalar-memory operations are outstanding.
constexpr int waitcnt_imm(int vm, int exp, int lgkm) {
  return (vm & 15) | ((vm >> 4) << 14) | (exp << 4) | (lgkm << 8);
}

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
// Element types
// ---------------------------------------------------------------------------

template <typename T>
struct Elem;

template <>
struct Elem<float> {
  static constexpr int BYTES = 4;
  static constexpr int VEC = 4;                  // elements per 16 bytes
  static constexpr uint32_t NEG_INF_WORD = 0xff800000u;
  __device__ static float load1(const void* row, uint32_t i) {
    return *reinterpret_cast<const float*>(static_cast<const char*>(row) + i * 4u);
  }
  __device__ static void store1(void* row, uint32_t i, float v) {
    __builtin_nontemporal_store(v, reinterpret_cast<float*>(static_cast<char*>(row) + i * 4u));
  }
  __device__ static void unpack(const u32x4 u, float (&x)[4]) {
    x[0] = __uint_as_float(u.x);
    x[1] = __uint_as_float(u.y);
    x[2] = __uint_as_float(u.z);
    x[3] = __uint_as_float(u.w);
  }
};

template <>
struct Elem<bf16_t> {
  static constexpr int BYTES = 2;
  static constexpr int VEC = 8;
  static constexpr uint32_t NEG_INF_WORD = 0xff80ff80u;
  __device__ static float load1(const void* row, uint32_t i) {
    const uint32_t u = *reinterpret_cast<const uint16_t*>(static_cast<const char*>(row) + i * 2u);
    return __uint_as_float(u << 16);
  }
  __device__ static void store1(void* row, uint32_t i, float v) {
    const uint16_t h = static_cast<uint16_t>(pack_bf16x2(v, 0.f) & 0xffffu);
    __builtin_nontemporal_store(h, reinterpret_cast<uint16_t*>(static_cast<char*>(row) + i * 2u));
  }
  __device__ static void unpack(const u32x4 u, float (&x)[8]) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[2 * k] = __uint_as_float(w[k] << 16);
      x[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
    }
  }
};

// The empty asm marks the registers as rewritten (no instruction is emitted):
// floats widened from them before it cannot be reused after it, so a resident
// chunk costs 4 registers between passes instead of up to 8 live floats.
__device__ __forceinline__ void touch(u32x4& v) { asm volatile("" : "+v"(v)); }

// Merge partial (m, s) -- s = sum 2^(y - m) over a set, m a float shift in
// log2 units -- with (m2, s2). An empty partial is (-inf, 0).
// A (shift, sum) pair's shift must be the rounded float its sum was formed
// against. HIP contracts floating-point expressions across statements by
// default, so a shift written as a product (max * log2e) could reach a later
// subtraction unrounded -- fused into fma(max, log2e, -sh) -- and the rescale
// factor of that pair would pick up the product's rounding residue (up to
// 2.6e-6 relative at |z| ~ 64). Passing the product through an empty asm makes
// it a plain register value that every use sees rounded.
__device__ __forceinline__ float as_rounded(float x) {
  asm volatile("" : "+v"(x));
  return x;
}

__device__ __forceinline__ void merge(float& m, float& s, float m2, float s2) {
  const float mn = fmaxf(m, m2);
  const float sh = (mn == kNegInf) ? 0.f : mn;
  s = s * fexp2(m - sh) + s2 * fexp2(m2 - sh);
  m = mn;
}

// Online update of (mL, s) with G values (-inf = absent).
template <int G>
__device__ __forceinline__ void online_group(float& mL, float& s, const float* x) {
  float gmax = kNegInf;
#pragma unroll
  for (int k = 0; k < G; ++k) gmax = fmaxf(gmax, x[k]);
  const float mn = fmaxf(mL, gmax * kL2E);
  const float sh = (mn == kNegInf) ? 0.f : mn;
  float acc = 0.f;
#pragma unroll
  for (int k = 0; k < G; ++k) acc += fexp2(__builtin_fmaf(x[k], kL2E, -sh));
  s = s * fexp2(mL - sh) + acc;
  mL = mn;
}

// Entropy partials (m, s, u): s = sum 2^d_j and u = sum 2^d_j d_j with
// d_j = y_j - m, y_j the value in log2 units. Rebasing to a shift M >= m
// multiplies both by 2^(m - M) and adds (m - M) s to u.
__device__ __forceinline__ void rebase3(float m, float& s, float& u, float M) {
  if (s == 0.f) {
    u = 0.f;
    return;
  }
  const float dm = m - M;
  const float f = fexp2(dm);
  u = f * (u + dm * s);
  s *= f;
}

__device__ __forceinline__ void merge3(float& m, float& s, float& u, float m2, float s2, float u2) {
  const float mn = fmaxf(m, m2);
  const float sh = (mn == kNegInf) ? 0.f : mn;
  rebase3(m, s, u, sh);
  rebase3(m2, s2, u2, sh);
  s += s2;
  u += u2;
  m = (mn == kNegInf) ? kNegInf : sh;
}

template <int G>
__device__ __forceinline__ void online_group3(float& mL, float& s, float& u, const float* x) {
  float gmax = kNegInf;
#pragma unroll
  for (int k = 0; k < G; ++k) gmax = fmaxf(gmax, x[k]);
  const float mn = fmaxf(mL, gmax * kL2E);
  const float sh = (mn == kNegInf) ? 0.f : mn;
  float acc = 0.f, accu = 0.f;
#pragma unroll
  for (int k = 0; k < G; ++k) {
    // d <= -256 gives e = 0 and e d = 0 (no -inf * 0)
    const float d = fmaxf(__builtin_fmaf(x[k], kL2E, -sh), -256.f);
    const float e = fexp2(d);
    acc += e;
    accu = __builtin_fmaf(e, d, accu);
  }
  rebase3(mL, s, u, sh);
  s += acc;
  u += accu;
  mL = (mn == kNegInf) ? kNegInf : sh;
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
  int64_t v0;                // global index of the first column of these rows
  float* stats;              // statistics mode: [T, 3] (shift, sum, target logit)
  const float* row_state;    // gradient mode: [T, kRowState] saved per-row state
  const float* row_weight;   // gradient mode: [T] weights of the NLL term, or null
  float* lse_out;            // optional [T] full logsumexp
  float* ent_out;            // optional [T] softmax entropy (entropy variant only)
  // pair mode: [T][2] slots of two 64-bit words per half, (shift, sum) and
  // (target logit, 0), set to all-ones before the launch; columns
  // [0, pair_split) are half 0, [pair_split, V) half 1
  uint32_t* pair_part;
  int64_t pair_split;
  uint32_t pair_spin;        // polls of a partner's words before giving up
  // row-resident kernel: tickets[0] is the counter that deals out rows (pair
  // mode: half rows); pair mode: tickets[1] counts the half rows that ended
  // without their partner's statistics. Both start at all-ones.
  uint32_t* tickets;
};

// What a row-kernel launch does.
enum RowMode : int {
  kFused = 0,   // both passes, loss and gradient
  kStats = 1,   // pass 1 only: per-row (shift, sum, target logit) of a shard
  kGrad = 2,    // pass 2 only, from a saved per-row state
  kPair = 3     // both passes over half a row; the two halves exchange statistics
};

// Saved per-row state: kRowState floats per row,
//   [0] lse log2(e) rounded to float   [1] p_nt = sigmoid(LSE_nt - z_t)
//   [2] p_t = sigmoid(z_t - LSE_nt)    [3] 2 alpha lse
//   [4] segment factor (1 / length, or 1)   [5] kind
//   [6] lse log2(e) - [0] (the rounding residue of [0])   [7] zero
constexpr int kRowState = 8;
// Pair mode: polls of a partner's words (each an L2 round trip plus
// s_sleep 2) before the wait is given up, well over 0.1 s. The partner of a
// waiting half is always resident and publishes before it waits, so the
// limit only ends waits that something outside the kernel stalls.
constexpr uint32_t kPairSpin = 1u << 21;
constexpr float kRowValid = 0.f, kRowIgnored = 1.f, kRowPoisoned = 2.f;


// Per-row results of the epilogue that pass 2 needs.
// A row's label with the mask folded in: ignore_index where the mask byte is
// 0, so a row counts exactly when its label is not ignore_index and its mask
// byte is nonzero. Both arrays are read-only for the call and are read
// through the scalar cache: the mask byte within its aligned 4-byte word when
// that word lies inside the mask (a plain byte load otherwise, for the first
// or last rows of an unaligned mask). A vector load here would be counted
// with the previous row's gradient stores, and waiting for it would wait for
// all of them.
__device__ __forceinline__ uint32_t mask_byte(const uint8_t* mask, int64_t r, int64_t T) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(mask + r);
  const uintptr_t w = a & ~uintptr_t{3};
  if (w >= reinterpret_cast<uintptr_t>(mask) && w + 4 <= reinterpret_cast<uintptr_t>(mask + T)) {
    const uint32_t v = *(const __attribute__((address_space(4))) uint32_t*)w;
    return (v >> (8u * static_cast<uint32_t>(a & 3u))) & 0xffu;
  }
  return mask[r];
}
__device__ __forceinline__ int64_t row_label(const RowParams& p, int64_t r) {
  const int64_t t = ((const __attribute__((address_space(4))) int64_t*)p.targets)[r];
  if (p.mask == nullptr) return t;
  return mask_byte(p.mask, r, p.T) != 0 ? t : p.ignore_index;
}

struct RowOut {
  float g_t;     // gradient of the target column
  float cnt;     // scale * (1 + 2 alpha lse): factor of every non-target softmax value
  float kl;      // lse in log2 units
  double cnt_d;
  double lse_l2; // lse in log2 units, fp64
};

// Block-reduced (M, S) of the non-target columns -> loss, NLL, gradient
// factors, all in fp64 (the NLL of a confident row is ~e^-40 and keeps its
// relative accuracy only if LSE_nt - z_t is formed in fp64).
// Gradient factors of a saved row: the NLL term weighted by w (the row's
// weight, or grad_scale * segment factor), the z-loss term by grad_scale *
// segment factor.
__device__ __forceinline__ RowOut saved_row(const RowParams& p, const float* rs, int64_t r) {
  const float zw = p.grad_scale * rs[4];
  const float w = p.row_weight ? p.row_weight[r] : zw;
  RowOut o{};
  o.kl = rs[0];
  // rs[6] is the rounding residue of rs[0]: folded into the row factor
  o.cnt = (w + zw * rs[3]) * fexp2(-rs[6]);
  o.g_t = -w * rs[1] + zw * rs[3] * rs[2];
  return o;
}

// The per-row loss terms from the non-target logsumexp and the target logit.
struct RowLoss {
  double nll;   // softplus(LSE_nt - z_t)
  double lse;   // logaddexp(LSE_nt, z_t)
  double p_nt;  // sigmoid(LSE_nt - z_t): probability off the target
  double p_t;   // sigmoid(z_t - LSE_nt): target probability
};

// One exponential serves all four: with e = exp(-|x|), softplus(x) =
// max(x, 0) + log1p(e), and sigmoid(+-x) is 1 / (1 + e) on the side where
// the argument is >= 0 and e / (1 + e) on the other (the stable forms).
__device__ __forceinline__ RowLoss row_loss(double lse_nt, double zt_d) {
  RowLoss o;
  const double xx = lse_nt - zt_d;                       // LSE_nt - z_t
  const double e = exp(-fabs(xx));
  const double l1p = log1p(e);
  o.nll = (xx > 0.0 ? xx : 0.0) + l1p;                   // softplus
  o.lse = (lse_nt > zt_d ? lse_nt : zt_d) + l1p;         // logaddexp
  const double d = 1.0 + e;
  o.p_nt = (xx >= 0.0) ? 1.0 / d : e / d;                // sigmoid(x)
  o.p_t = (xx <= 0.0) ? 1.0 / d : e / d;                 // sigmoid(-x)
  return o;
}

// LSE_nt from a (shift, sum) partial in log2 units.
__device__ __forceinline__ double lse_from_partial(double M, double S) {
  return (M == -HUGE_VAL) ? -HUGE_VAL : M / static_cast<double>(kL2E) + log(S);
}

// 1 / (rows carrying row r's segment id), or 1.
__device__ __forceinline__ double segment_factor(const int32_t* seg_ids, const int32_t* seg_start,
                                                 int32_t num_segments, int64_t r) {
  int32_t sid = seg_ids[r];
  sid = sid < 0 ? 0 : (sid >= num_segments ? num_segments - 1 : sid);
  const int32_t len = seg_start[sid + 1] - seg_start[sid];
  return 1.0 / static_cast<double>(len > 0 ? len : 1);
}

// seg_f: the row's segment factor (1 / segment length, or 1).
__device__ __forceinline__ RowOut row_epilogue(const RowParams& p, int64_t r, float M, float S,
                                               float zt, bool write_loss, double seg_f) {
  const double l2e = static_cast<double>(kL2E);
  const RowLoss L = row_loss(lse_from_partial(M == kNegInf ? -HUGE_VAL : static_cast<double>(M),
                                              static_cast<double>(S)),
                             static_cast<double>(zt));
  const double nll = L.nll, lse = L.lse, p_nt = L.p_nt, p_t = L.p_t;
  const double scale = static_cast<double>(p.grad_scale) * seg_f;
  const double alpha = static_cast<double>(p.z_alpha);
  const double zfac = (alpha == 0.0) ? 0.0 : 2.0 * alpha * lse;
  if (write_loss) {
    const double loss = nll + ((alpha == 0.0) ? 0.0 : alpha * lse * lse);
    p.loss_out[r] = static_cast<float>(loss);
    if (p.nll_ws) p.nll_ws[r] = static_cast<float>(nll);
    if (p.lse_out) p.lse_out[r] = static_cast<float>(lse);
  }
  RowOut o;
  o.cnt_d = scale * (1.0 + zfac);
  o.g_t = static_cast<float>(scale * (-p_nt + zfac * p_t));
  o.lse_l2 = l2e * lse;
  o.kl = static_cast<float>(o.lse_l2);
  // kl holds lse log2(e) to half a float ulp (up to ~4e-6 at |lse| ~ 40);
  // the residue is folded into the per-row factor, so an element's exponent
  // z log2(e) - kl is exact up to its own rounding: 2^(z log2 e - lse log2 e)
  // = 2^(-residue) 2^(z log2 e - kl).
  const double res = isfinite(o.lse_l2) ? o.lse_l2 - static_cast<double>(o.kl) : 0.0;
  o.cnt = static_cast<float>(o.cnt_d * exp2(-res));
  return o;
}

// Workgroup reduction of per-lane (mL, s); every thread gets the result.
template <int BLOCK>
__device__ __forceinline__ void block_reduce(float& mL, float& s, float (&red_m)[2][BLOCK / 64],
                                             float (&red_s)[2][BLOCK / 64], int par,
                                             uint32_t lane, uint32_t wid) {
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
  for (int w = 1; w < BLOCK / 64; ++w) merge(M, S, red_m[par][w], red_s[par][w]);
  mL = M;
  s = S;
}

// The same for entropy partials (m, s, u).
template <int BLOCK>
__device__ __forceinline__ void block_reduce3(float& mL, float& s, float& u,
                                              float (&red_m)[2][BLOCK / 64],
                                              float (&red_s)[2][BLOCK / 64],
                                              float (&red_u)[2][BLOCK / 64], int par,
                                              uint32_t lane, uint32_t wid) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float m2 = __shfl_xor(mL, off, 64);
    const float s2 = __shfl_xor(s, off, 64);
    const float u2 = __shfl_xor(u, off, 64);
    merge3(mL, s, u, m2, s2, u2);
  }
  if (lane == 0) {
    red_m[par][wid] = mL;
    red_s[par][wid] = s;
    red_u[par][wid] = u;
  }
  __syncthreads();
  float M = red_m[par][0], S = red_s[par][0], Uu = red_u[par][0];
#pragma unroll
  for (int w = 1; w < BLOCK / 64; ++w) merge3(M, S, Uu, red_m[par][w], red_s[par][w], red_u[par][w]);
  mL = M;
  s = S;
  u = Uu;
}

// Softmax entropy from the non-target partial (M, S, U) and the target
// logit, in fp64: H = p_t NLL + ln2 2^(M - L2) ((L2 - M) S - U), L2 = lse
// log2(e). Every term is >= 0, so a confident row (H ~ p_nt) keeps its
// relative accuracy.
__device__ __forceinline__ float row_entropy(float M, float S, float U, float zt) {
  const double Md = M == kNegInf ? -HUGE_VAL : static_cast<double>(M);
  const RowLoss L = row_loss(lse_from_partial(Md, static_cast<double>(S)), static_cast<double>(zt));
  double h = (L.p_t > 0.0) ? L.p_t * L.nll : 0.0;
  if (Md != -HUGE_VAL && S > 0.f) {
    const double L2 = static_cast<double>(kL2E) * L.lse;
    h += 0.6931471805599453 * exp2(Md - L2) * ((L2 - Md) * static_cast<double>(S) -
                                                static_cast<double>(U));
  }
  return static_cast<float>(h);
}

// Fill an ignored (0) or poisoned (NaN) gradient row and its loss.
template <typename TO, int BLOCK>
__device__ __forceinline__ void fill_row(const RowParams& p, int64_t r, void* grow, uint32_t V,
                                         float fill, bool write, bool write_loss = true) {
  if (write_loss && threadIdx.x == 0) {
    p.loss_out[r] = fill;
    if (p.nll_ws) p.nll_ws[r] = fill;
    if (p.lse_out) p.lse_out[r] = fill;
    if (p.ent_out) p.ent_out[r] = fill;
  }
  if (!write) return;
  constexpr int VEC = Elem<TO>::VEC;
  const bool vec = (reinterpret_cast<uintptr_t>(grow) % 16) == 0;
  const uint32_t nvec = vec ? V / VEC : 0;
  const uint32_t fw = Elem<TO>::BYTES == 4 ? __float_as_uint(fill) : (pack_bf16x2(fill, fill));
  const u32x4 f4 = {fw, fw, fw, fw};
  for (uint32_t c = threadIdx.x; c < nvec; c += BLOCK)
    __builtin_nontemporal_store(f4, reinterpret_cast<u32x4*>(static_cast<char*>(grow) + c * 16u));
  for (uint32_t j = nvec * VEC + threadIdx.x; j < V; j += BLOCK) Elem<TO>::store1(grow, j, fill);
}

// ---------------------------------------------------------------------------
// One-element kernel: rows whose start or stride is not 16-byte aligned.
// Two streamed passes, one element per lane and step.
// ---------------------------------------------------------------------------
template <typename TI, typename TO, int BLOCK, bool WRITE, int MODE = kFused, bool ENT = false>
__global__ __launch_bounds__(BLOCK) void ce_rows_scalar_kernel(RowParams p) {
  static_assert(!ENT || (MODE == kFused && !WRITE), "the entropy variant is a forward");
  __shared__ float red_m[2][BLOCK / 64];
  __shared__ float red_s[2][BLOCK / 64];
  __shared__ float red_u[ENT ? 2 : 1][ENT ? BLOCK / 64 : 1];
  const uint32_t tid = threadIdx.x, lane = tid & 63u, wid = tid >> 6;
  const uint32_t V = static_cast<uint32_t>(p.V);
  const size_t in_row_bytes = static_cast<size_t>(p.ld_in) * Elem<TI>::BYTES;
  const size_t out_row_bytes = static_cast<size_t>(p.ld_out) * Elem<TO>::BYTES;
  int par = 0;
  for (int64_t r = blockIdx.x; r < p.T; r += gridDim.x, par ^= 1) {
    const int64_t t64 = row_label(p, r);
    void* grow = WRITE ? static_cast<char*>(p.grad) + r * out_row_bytes : nullptr;
    const int64_t tl = t64 - p.v0;
    const bool owned = tl >= 0 && tl < static_cast<int64_t>(V);
    RowOut o{};
    if constexpr (MODE == kGrad) {
      const float* rs = p.row_state + kRowState * r;
      if (rs[5] != kRowValid) {
        fill_row<TO, BLOCK>(p, r, grow, V, rs[5] == kRowIgnored ? 0.f : __builtin_nanf(""), true,
                            false);
        continue;
      }
      o = saved_row(p, rs, r);
    } else {
      const bool valid = t64 != p.ignore_index;   // (the mask is folded into the label)
      if constexpr (MODE == kStats) {
        if (!valid) {
          if (tid == 0) {
            p.stats[3 * r] = kNegInf;
            p.stats[3 * r + 1] = 0.f;
            p.stats[3 * r + 2] = kNegInf;
          }
          continue;
        }
      } else if (!valid || !owned) {
        fill_row<TO, BLOCK>(p, r, grow, V, valid ? __builtin_nanf("") : 0.f, WRITE);
        continue;
      }
    }
    const uint32_t t = owned ? static_cast<uint32_t>(tl) : V;
    const void* zrow = static_cast<const char*>(p.logits) + r * in_row_bytes;
    if constexpr (MODE != kGrad) {
      const float zt = owned ? Elem<TI>::load1(zrow, t) : kNegInf;
      float mL = kNegInf, s = 0.f;
      [[maybe_unused]] float hs = 0.f;
      for (uint32_t b = 0; b < V; b += 4 * BLOCK) {
        float x[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint32_t j = b + u * BLOCK + tid;
          x[u] = (j < V && j != t) ? Elem<TI>::load1(zrow, j) : kNegInf;
        }
        if constexpr (ENT) {
          online_group3<4>(mL, s, hs, x);
        } else {
          online_group<4>(mL, s, x);
        }
      }
      if constexpr (ENT) {
        block_reduce3<BLOCK>(mL, s, hs, red_m, red_s, red_u, par, lane, wid);
        if (tid == 0) p.ent_out[r] = row_entropy(mL, s, hs, zt);
      } else {
        block_reduce<BLOCK>(mL, s, red_m, red_s, par, lane, wid);
      }
      if constexpr (MODE == kStats) {
        if (tid == 0) {
          p.stats[3 * r] = mL;
          p.stats[3 * r + 1] = s;
          p.stats[3 * r + 2] = zt;
        }
        continue;
      } else {
        o = row_epilogue(p, r, mL, s, zt, tid == 0,
                         p.seg_mean ? segment_factor(p.seg_ids, p.seg_start, p.num_segments, r)
                                    : 1.0);
      }
    }
    if constexpr (WRITE) {
      for (uint32_t j = tid; j < V; j += BLOCK) {
        const float g = (j == t) ? o.g_t
                                 : o.cnt * fexp2(__builtin_fmaf(Elem<TI>::load1(zrow, j), kL2E, -o.kl));
        Elem<TO>::store1(grow, j, g);
      }
    }
  }
}

// v[i] &= and_m, |= or_m for the one slot i == k (k uniform): a compare
// chain on k, so only that slot's registers are touched.
template <int N>
__device__ __forceinline__ void mask_target_slot(u32x4 (&v)[N], uint32_t k, u32x4 and_m,
                                                 u32x4 or_m) {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    if (k == static_cast<uint32_t>(i)) {
      v[i] = (v[i] & and_m) | or_m;
      return;
    }
  }
}

// ---------------------------------------------------------------------------
// Vector kernel (16-byte aligned rows).
//   TI/TO  : logits / gradient element types
//   BLOCK  : threads per workgroup
//   NRES   : slots per thread kept in registers as fp32 exps between passes
//   NRAW   : slots per thread kept in registers as raw input between passes
//   NLDS   : slots per thread staged in LDS (loaded HBM -> LDS directly)
//   U      : slots per thread per step of the streamed loops
//   WRITE  : write the gradient (false = forward only)
//   PF     : double-buffer the streamed loops (2 U slots in flight per lane)
//   EPI1   : one wave runs the fp64 epilogue and shares it through LDS
//   OG     : streamed slots per online (max, sum) update (divides U)
//   ENT    : also accumulate sum e d for the softmax entropy (forward only)
// Slot i of thread tid is chunk c = i * BLOCK + tid (a chunk is 16 bytes of
// input). Slots [0, NRES) are exp-resident, then NRAW raw-resident, then NLDS
// in LDS; later slots are streamed. Loads never branch per lane: a lane past
// the row's last chunk loads the last chunk again (in bounds) and replaces it
// by -inf; only stores are predicated, and only in the row's partial slot.
// ---------------------------------------------------------------------------
template <typename TI, typename TO, int BLOCK, int NRES, int NRAW, int NLDS, int U, bool WRITE,
          bool PF, bool EPI1, int OG = U, int MODE = kFused, bool ENT = false>
__global__ __launch_bounds__(BLOCK) void ce_rows_kernel(RowParams p) {
  static_assert(U % OG == 0, "online groups split the step evenly");
  static_assert(!ENT || (MODE == kFused && !WRITE && NRES + NRAW == 0),
                "the entropy variant is a forward with streamed or LDS-staged slots");
  static_assert(MODE != kGrad || (NRES + NRAW + NLDS == 0 && WRITE), "gradient mode streams");
  static_assert(MODE != kStats || !WRITE, "statistics mode writes no gradient");
  static_assert(MODE != kPair, "two workgroups per row: the row-resident kernel");
  constexpr int W = Elem<TI>::VEC;                 // elements per chunk
  constexpr uint32_t OB = W * Elem<TO>::BYTES;     // gradient bytes per chunk
  constexpr int NON = NRES + NRAW + NLDS;          // on-chip slots per thread
  static_assert(BLOCK % 64 == 0, "whole waves");
  __shared__ float red_m[2][BLOCK / 64];
  __shared__ float red_s[2][BLOCK / 64];
  __shared__ float red_u[ENT ? 2 : 1][ENT ? BLOCK / 64 : 1];
  __shared__ u32x4 stage[NLDS > 0 ? NLDS : 1][NLDS > 0 ? BLOCK : 1];
  __shared__ float epi[2][4];

  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63u;
  const uint32_t wid = tid >> 6;
  const int64_t row0 = static_cast<int64_t>(blockIdx.x);
  const int64_t row_step = gridDim.x;
  // In-row offsets are 32-bit (the host bounds a row below 2 GiB).
  const uint32_t V = static_cast<uint32_t>(p.V);
  const uint32_t nchunk = V / W;
  const uint32_t clast = nchunk > 0 ? nchunk - 1 : 0;
  const uint32_t tail_begin = nchunk * W;
  const uint32_t voff_in = tid * 16u;
  const uint32_t voff_out = tid * OB;
  const size_t in_row_bytes = static_cast<size_t>(p.ld_in) * Elem<TI>::BYTES;
  const size_t out_row_bytes = static_cast<size_t>(p.ld_out) * Elem<TO>::BYTES;
  const uint32_t neg_w = Elem<TI>::NEG_INF_WORD;
  [[maybe_unused]] const u32x4 neg4 = {neg_w, neg_w, neg_w, neg_w};

  // Labels (with the mask folded in) are read through the scalar cache (the
  // constant address space: the kernel never writes them), one row ahead. A
  // scalar load is counted with the LDS operations, not with the vector
  // memory ones, so neither its latency nor the previous row's gradient
  // stores still in flight hold up the start of a row. (Segment bounds come
  // from an earlier launch; each dispatch starts with the scalar cache
  // invalidated.)
  const kconst_i32* seg_ids = (const kconst_i32*)p.seg_ids;
  const kconst_i32* seg_start = (const kconst_i32*)p.seg_start;
  int64_t t_next = row0 < p.T ? row_label(p, row0) : 0;
  int par = 0;
  for (int64_t r = row0; r < p.T; r += row_step, par ^= 1) {
    const int64_t t64 = t_next;
    if (r + row_step < p.T) t_next = row_label(p, r + row_step);
    void* grow = WRITE ? static_cast<char*>(p.grad) + r * out_row_bytes : nullptr;
    // The target's column within these rows (t_local = V: not among them).
    const int64_t tl = t64 - p.v0;
    const bool owned = tl >= 0 && tl < static_cast<int64_t>(V);
    RowOut saved{};
    if constexpr (MODE == kGrad) {
      // The saved state says whether the row is ignored (+0.0), poisoned
      // (NaN) or carries gradient factors.
      const float* rs = p.row_state + kRowState * r;
      const float kind = rs[5];
      if (kind != kRowValid) {
        fill_row<TO, BLOCK>(p, r, grow, V, kind == kRowIgnored ? 0.f : __builtin_nanf(""), true,
                            false);
        continue;
      }
      saved = saved_row(p, rs, r);
    } else {
      const bool valid = t64 != p.ignore_index;   // (the mask is folded into the label)
      if constexpr (MODE == kStats) {
        if (!valid) {
          if (tid == 0) {
            p.stats[3 * r] = kNegInf;
            p.stats[3 * r + 1] = 0.f;
            p.stats[3 * r + 2] = kNegInf;
          }
          continue;
        }
      } else if (!valid || !owned) {
        // Ignored row: +0.0 everywhere, logits never read. Valid row with an
        // out-of-range target: NaN loss and gradient row.
        fill_row<TO, BLOCK>(p, r, grow, V, valid ? __builtin_nanf("") : 0.f, WRITE);
        continue;
      }
    }

    const uint32_t t = owned ? static_cast<uint32_t>(tl) : V;
    const void* zrow = static_cast<const char*>(p.logits) + r * in_row_bytes;
    const float zt = (MODE != kGrad && owned) ? Elem<TI>::load1(zrow, t) : kNegInf;
    const __amdgpu_buffer_rsrc_t rin =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(zrow), 0, nchunk * 16u, kBufWord3);

    // Where the target sits: chunk ct, element kt, slot st, lane `mine`.
    const uint32_t ct = t / W;
    const uint32_t kt = t - ct * W;
    const uint32_t st = ct / BLOCK;
    const bool in_chunks = t < tail_begin;
    const bool mine = in_chunks && (ct - st * BLOCK) == tid;
    // AND/OR word masks that set element kt of a raw chunk to -inf (uniform).
    const uint32_t kq = (kt * Elem<TI>::BYTES) >> 2;             // word of the chunk
    const uint32_t ksh = (kt * Elem<TI>::BYTES * 8u) & 31u;      // bit offset in the word
    const uint32_t kmask = Elem<TI>::BYTES == 4 ? 0xffffffffu : (0xffffu << ksh);
    const uint32_t kput = Elem<TI>::BYTES == 4 ? 0xff800000u : (0xff80u << ksh);
    const u32x4 and_m = {kq == 0 ? ~kmask : ~0u, kq == 1 ? ~kmask : ~0u,
                         kq == 2 ? ~kmask : ~0u, kq == 3 ? ~kmask : ~0u};
    const u32x4 or_m = {kq == 0 ? kput : 0u, kq == 1 ? kput : 0u, kq == 2 ? kput : 0u,
                        kq == 3 ? kput : 0u};

    // Slot loads: lane offsets are clamped to the last chunk, so every load
    // is in bounds and none branches; lanes past the row end are replaced by
    // -inf afterwards. The target's element is set to -inf in the one lane
    // that holds it.
    // The lane offset is re-derived every row (the empty asm hides that it is
    // row-invariant), so the per-slot offsets are formed next to their loads
    // instead of being hoisted out of the row loop and kept live.
    uint32_t vin = voff_in;
    asm volatile("" : "+v"(vin));
    const uint32_t c16_last = clast * 16u;
    auto load_slot = [&](uint32_t base) -> u32x4 {
      return __builtin_amdgcn_raw_buffer_load_b128(rin, min(vin + base * 16u, c16_last), 0, 0);
    };
    auto load_slot_last_use = [&](uint32_t base) -> u32x4 {
      return __builtin_amdgcn_raw_buffer_load_b128(rin, min(vin + base * 16u, c16_last), 0, kNT);
    };
    // On-chip slots are read from memory exactly once: non-temporal.
    auto fix_slot = [&](uint32_t base, u32x4& v) {
      const bool out = base + tid >= nchunk;
      v.x = out ? neg_w : v.x;
      v.y = out ? neg_w : v.y;
      v.z = out ? neg_w : v.z;
      v.w = out ? neg_w : v.w;
    };

    // The row's segment id goes out now (scalar load); its length is read
    // once the on-chip loads are in flight, so the epilogue waits on neither.
    [[maybe_unused]] int32_t sid = 0;
    if (MODE != kGrad && p.seg_mean) sid = seg_ids[r];

    // ---- issue every on-chip load first ------------------------------------
    u32x4 rawe[NRES > 0 ? NRES : 1];
    u32x4 rawv[NRAW > 0 ? NRAW : 1];
    if (MODE != kGrad && nchunk > 0) {
#pragma unroll
      for (int i = 0; i < NRES; ++i) rawe[i] = load_slot_last_use(i * BLOCK);
#pragma unroll
      for (int i = 0; i < NRAW; ++i) rawv[i] = load_slot_last_use((NRES + i) * BLOCK);
      if constexpr (NLDS > 0) {
        // HBM -> LDS without a register round trip: lane l of a wave lands
        // at base + 16 l, so slot i of thread tid is stage[i][tid].
#pragma unroll
        for (int i = 0; i < NLDS; ++i) {
          const uint32_t off = min(vin + (NRES + NRAW + i) * BLOCK * 16u, c16_last);
          __builtin_amdgcn_global_load_lds(
              (const __attribute__((address_space(1))) void*)(static_cast<const char*>(zrow) + off),
              (__attribute__((address_space(3))) void*)(&stage[i][tid & ~63u]), 16, 0, kNT);
        }
      }
    }

    [[maybe_unused]] int32_t seg_len = 1;   // uniform: stays in scalar registers
    if (MODE != kGrad && p.seg_mean) {
      sid = sid < 0 ? 0 : (sid >= p.num_segments ? p.num_segments - 1 : sid);
      const int32_t len = seg_start[sid + 1] - seg_start[sid];
      seg_len = len > 0 ? len : 1;
    }

    float mL = kNegInf, s = 0.f;
    [[maybe_unused]] float hs = 0.f;   // entropy variant: sum e d

    // ---- pass 1a: exp-resident slots ---------------------------------------
    float e[NRES > 0 ? NRES : 1][W];
    float rsh = 0.f;          // shift of the resident exps (log2 units)
    if constexpr (NRES > 0) {
#pragma unroll
      for (int i = 0; i < NRES; ++i) fix_slot(i * BLOCK, rawe[i]);
      if (mine && st < NRES) mask_target_slot<NRES>(rawe, st, and_m, or_m);
      float rmax = kNegInf;
#pragma unroll
      for (int i = 0; i < NRES; ++i) {
        Elem<TI>::unpack(rawe[i], e[i]);
#pragma unroll
        for (int k = 0; k < W; ++k) rmax = fmaxf(rmax, e[i][k]);
      }
      const float rml = as_rounded(rmax * kL2E);
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

    // ---- pass 1b: raw register-resident slots (max, then sum) -------------
    if constexpr (NRAW > 0) {
#pragma unroll
      for (int i = 0; i < NRAW; ++i) fix_slot((NRES + i) * BLOCK, rawv[i]);
      if (mine && st >= NRES && st < NRES + NRAW)
        mask_target_slot<NRAW>(rawv, st - NRES, and_m, or_m);
      float vmax = kNegInf;
#pragma unroll
      for (int i = 0; i < NRAW; ++i) {
        float x[W];
        Elem<TI>::unpack(rawv[i], x);
#pragma unroll
        for (int k = 0; k < W; ++k) vmax = fmaxf(vmax, x[k]);
      }
      const float vml = as_rounded(vmax * kL2E);
      const float vsh = (vml == kNegInf) ? 0.f : vml;
#pragma unroll
      for (int i = 0; i < NRAW; ++i) touch(rawv[i]);
      float vs = 0.f;
#pragma unroll
      for (int i = 0; i < NRAW; ++i) {
        float x[W];
        Elem<TI>::unpack(rawv[i], x);
        float cs = 0.f;
#pragma unroll
        for (int k = 0; k < W; ++k) cs += fexp2(__builtin_fmaf(x[k], kL2E, -vsh));
        vs += cs;
      }
      merge(mL, s, vml, vs);
    }

    // ---- pass 1c: LDS-staged slots -----------------------------------------
    if constexpr (NLDS > 0) {
      constexpr int i0 = NRES + NRAW;
      __builtin_amdgcn_s_waitcnt(0);   // this wave's HBM -> LDS copies have landed
#pragma unroll
      for (int i = 0; i < NLDS; ++i) {
        u32x4 v = stage[i][tid];
        fix_slot((i0 + i) * BLOCK, v);
        if (mine && i0 + i == static_cast<int>(st)) v = (v & and_m) | or_m;
        float x[W];
        Elem<TI>::unpack(v, x);
        if constexpr (ENT) {
          online_group3<W>(mL, s, hs, x);
        } else {
          online_group<W>(mL, s, x);
        }
      }
    }

    // ---- pass 1d: streamed slots, online (shift, sum) ----------------------
    // A step's slots at b + u BLOCK. In the long-row shapes (one online update
    // per slot, OG = 1) slots wholly past the row end are neither loaded nor
    // reduced nor stored (the tests are uniform over the workgroup and only
    // the row's last steps take the slow branch; a skipped slot holds -inf, a
    // constant, so no register stays live from the previous step). With two
    // slots per update the tail wastes at most one group, and the extra
    // branches measured slower there (3% on 16032-chunk rows), so those shapes
    // load and reduce every slot of a step; lanes past the end load the last
    // chunk again (one broadcast line) and fix_slot makes them -inf.
    constexpr bool SKIP_TAIL = OG == 1;
    auto load_group = [&](u32x4 (&raw)[U], uint32_t b, auto load) {
      if (!SKIP_TAIL || b + (U - 1) * BLOCK < nchunk) {
#pragma unroll
        for (int u = 0; u < U; ++u) raw[u] = load(b + u * BLOCK);
      } else {
#pragma unroll
        for (int u = 0; u < U; ++u) raw[u] = b + u * BLOCK < nchunk ? load(b + u * BLOCK) : neg4;
      }
    };
    auto reduce_group = [&](const u32x4 (&raw)[U], int g0) {
      float x[OG * W];
#pragma unroll
      for (int u = g0; u < g0 + OG; ++u) {
        float xu[W];
        Elem<TI>::unpack(raw[u], xu);
#pragma unroll
        for (int k = 0; k < W; ++k) x[(u - g0) * W + k] = xu[k];
      }
      if constexpr (ENT) {
        online_group3<OG * W>(mL, s, hs, x);
      } else {
        online_group<OG * W>(mL, s, x);
      }
    };
    auto stream1 = [&](u32x4 (&raw)[U], uint32_t b) {
      // Only a step that holds the row's end or the target's slot needs the
      // fix-ups. The test is the same for the whole workgroup, and the empty
      // asm keeps it a branch (the compiler would otherwise turn the fix-ups
      // into selects that run in every step).
      if (b + U * BLOCK > nchunk || (in_chunks && st * BLOCK - b < U * BLOCK)) {
        asm volatile("");
#pragma unroll
        for (int u = 0; u < U; ++u) {
          fix_slot(b + u * BLOCK, raw[u]);
          if (mine && b + u * BLOCK == st * BLOCK) raw[u] = (raw[u] & and_m) | or_m;
        }
#pragma unroll
        for (int g0 = 0; g0 < U; g0 += OG) {
          if (SKIP_TAIL && b + g0 * BLOCK >= nchunk) break;
          reduce_group(raw, g0);
        }
      } else {
#pragma unroll
        for (int g0 = 0; g0 < U; g0 += OG) reduce_group(raw, g0);
      }
    };
    if constexpr (MODE == kGrad) {
      // no pass 1
    } else if constexpr (PF) {
      // Two groups in flight: group B's loads run while group A is reduced.
      // A group is loaded only if it holds chunks of the row: a load left
      // unused at the end would still be in flight at the next row's start,
      // where waiting for it would also wait for this row's gradient stores.
      if (NON * BLOCK < nchunk) {
        u32x4 ra[U], rb[U];
        uint32_t b = NON * BLOCK;
        load_group(ra, b, load_slot);
        for (;;) {
          if (b + U * BLOCK >= nchunk) {
            stream1(ra, b);
            break;
          }
          load_group(rb, b + U * BLOCK, load_slot);
          stream1(ra, b);
          if (b + 2 * U * BLOCK >= nchunk) {
            stream1(rb, b + U * BLOCK);
            break;
          }
          load_group(ra, b + 2 * U * BLOCK, load_slot);
          stream1(rb, b + U * BLOCK);
          b += 2 * U * BLOCK;
        }
      }
    } else {
      for (uint32_t b = NON * BLOCK; b < nchunk; b += U * BLOCK) {
        u32x4 raw[U];
        load_group(raw, b, load_slot);
        stream1(raw, b);
      }
    }
    // Elements past the last whole chunk: one per lane.
    if (MODE != kGrad && tid < V - tail_begin) {
      const uint32_t j = tail_begin + tid;
      const float xv = (j == t) ? kNegInf : Elem<TI>::load1(zrow, j);
      if constexpr (ENT) {
        merge3(mL, s, hs, xv * kL2E, (xv == kNegInf) ? 0.f : 1.f, 0.f);
      } else {
        merge(mL, s, xv * kL2E, (xv == kNegInf) ? 0.f : 1.f);
      }
    }

    // Every load of pass 1 has landed. Saying so keeps the compiler from
    // assuming some of them may still be in flight at the next row's start,
    // where it would otherwise wait for every gradient store of this row.
    if constexpr (MODE != kGrad) __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 7, 15));
    if constexpr (ENT) {
      block_reduce3<BLOCK>(mL, s, hs, red_m, red_s, red_u, par, lane, wid);
    } else if constexpr (MODE != kGrad) {
      block_reduce<BLOCK>(mL, s, red_m, red_s, par, lane, wid);
    }
    if constexpr (MODE == kStats) {
      if (tid == 0) {
        p.stats[3 * r] = mL;
        p.stats[3 * r + 1] = s;
        p.stats[3 * r + 2] = zt;
      }
      continue;
    }
    RowOut o;
    [[maybe_unused]] const double seg_f = 1.0 / static_cast<double>(seg_len);
    if constexpr (MODE == kGrad) {
      o = saved;
    } else if constexpr (EPI1) {
      // Wave 0 alone runs the fp64 epilogue; the others wait at the barrier,
      // leaving the SIMDs to other workgroups.
      if (wid == 0) {
        o = row_epilogue(p, r, mL, s, zt, tid == 0, seg_f);
        if (lane == 0) {
          epi[par][0] = o.g_t;
          epi[par][1] = o.cnt;
          epi[par][2] = o.kl;
        }
      }
      if constexpr (ENT) {
        // the entropy's fp64 epilogue runs on another wave, beside the loss's
        if (wid == (BLOCK > 64 ? 1u : 0u) && lane == 0) p.ent_out[r] = row_entropy(mL, s, hs, zt);
      }
      __syncthreads();
      o.g_t = epi[par][0];
      o.cnt = epi[par][1];
      o.kl = epi[par][2];
    } else {
      o = row_epilogue(p, r, mL, s, zt, tid == 0, seg_f);
      if constexpr (ENT) {
        if (tid == 0) p.ent_out[r] = row_entropy(mL, s, hs, zt);
      }
    }

    // ---- pass 2: gradient ----------------------------------------------------
    if constexpr (WRITE) {
      const __amdgpu_buffer_rsrc_t rout =
          __builtin_amdgcn_make_buffer_rsrc(grow, 0, nchunk * OB, kBufWord3);
      uint32_t vout = voff_out;
      asm volatile("" : "+v"(vout));
      auto store_slot = [&](uint32_t base, const float (&g)[W]) {
        uint32_t vo;
        if constexpr (MODE == kGrad && PF) {
          // Every lane stores; lanes past the row end store past the end of
          // the output window, which drops them. Stores outside branches are
          // counted by the compiler, so waiting for the next group's loads
          // does not also wait for this group's stores (measured 4% faster
          // than the branch on 8016-chunk rows, 6% slower on 2000-chunk rows
          // without double-buffered loads).
          vo = base + tid < nchunk ? vout + base * OB : 0x80000000u;
        } else {
          if (base + BLOCK > nchunk && base + tid >= nchunk) return;
          vo = vout + base * OB;
        }
        const uint32_t so = 0u;
        if constexpr (Elem<TO>::BYTES == 2 && W == 8) {
          const u32x4 q = {pack_bf16x2(g[0], g[1]), pack_bf16x2(g[2], g[3]),
                           pack_bf16x2(g[4], g[5]), pack_bf16x2(g[6], g[7])};
          __builtin_amdgcn_raw_buffer_store_b128(q, rout, vo, so, kNT);
        } else if constexpr (Elem<TO>::BYTES == 2) {   // 4 fp32 in -> 4 bf16 out
          const u32x2 q = {pack_bf16x2(g[0], g[1]), pack_bf16x2(g[2], g[3])};
          __builtin_amdgcn_raw_buffer_store_b64(q, rout, vo, so, kNT);
        } else {
#pragma unroll
          for (int h = 0; h < W / 4; ++h) {
            const u32x4 q = {__float_as_uint(g[4 * h]), __float_as_uint(g[4 * h + 1]),
                             __float_as_uint(g[4 * h + 2]), __float_as_uint(g[4 * h + 3])};
            __builtin_amdgcn_raw_buffer_store_b128(q, rout, vo + 16u * h, so, kNT);
          }
        }
      };
      auto grad_of = [&](const u32x4 v, float (&g)[W]) {
        float x[W];
        Elem<TI>::unpack(v, x);
#pragma unroll
        for (int k = 0; k < W; ++k) g[k] = o.cnt * fexp2(__builtin_fmaf(x[k], kL2E, -o.kl));
      };
      if constexpr (NRES > 0) {
        // Resident exps carry the lane's own shift rsh: rescale to lse.
        const float f = o.cnt * fexp2(rsh - o.kl);
#pragma unroll
        for (int i = 0; i < NRES; ++i) {
          float g[W];
#pragma unroll
          for (int k = 0; k < W; ++k) g[k] = e[i][k] * f;
          store_slot(i * BLOCK, g);
        }
      }
#pragma unroll
      for (int i = 0; i < NRAW; ++i) touch(rawv[i]);
#pragma unroll
      for (int i = 0; i < NRAW; ++i) {
        float g[W];
        grad_of(rawv[i], g);
        store_slot((NRES + i) * BLOCK, g);
      }
#pragma unroll
      for (int i = 0; i < NLDS; ++i) {
        float g[W];
        grad_of(stage[i][tid], g);
        store_slot((NRES + NRAW + i) * BLOCK, g);
      }
      auto stream2 = [&](const u32x4 (&raw)[U], uint32_t b) {
        if (SKIP_TAIL && b + U * BLOCK > nchunk) {
          // the row's last step: slots wholly past the end are skipped
#pragma unroll
          for (int u = 0; u < U; ++u) {
            if (b + u * BLOCK >= nchunk) break;
            float g[W];
            grad_of(raw[u], g);
            store_slot(b + u * BLOCK, g);
          }
        } else {
#pragma unroll
          for (int u = 0; u < U; ++u) {
            float g[W];
            grad_of(raw[u], g);
            store_slot(b + u * BLOCK, g);
          }
        }
      };
      if constexpr (PF) {
        // (as in pass 1: only groups that hold chunks of the row are loaded)
        if (NON * BLOCK < nchunk) {
          u32x4 ra[U], rb[U];
          uint32_t b = NON * BLOCK;
          load_group(ra, b, load_slot_last_use);
          for (;;) {
            if (b + U * BLOCK >= nchunk) {
              stream2(ra, b);
              break;
            }
            load_group(rb, b + U * BLOCK, load_slot_last_use);
            stream2(ra, b);
            if (b + 2 * U * BLOCK >= nchunk) {
              stream2(rb, b + U * BLOCK);
              break;
            }
            load_group(ra, b + 2 * U * BLOCK, load_slot_last_use);
            stream2(rb, b + U * BLOCK);
            b += 2 * U * BLOCK;
          }
        }
      } else {
        for (uint32_t b = NON * BLOCK; b < nchunk; b += U * BLOCK) {
          u32x4 raw[U];
          load_group(raw, b, load_slot_last_use);
          stream2(raw, b);
        }
      }
      if (tid < V - tail_begin) {
        const uint32_t j = tail_begin + tid;
        const float g = (j == t) ? o.g_t
                                 : o.cnt * fexp2(__builtin_fmaf(Elem<TI>::load1(zrow, j), kL2E, -o.kl));
        Elem<TO>::store1(grow, j, g);
      }
      // The target column: written after its chunk by the same lane, so this
      // store lands last (a lane's stores to one address stay in order).
      if (mine) Elem<TO>::store1(grow, t, o.g_t);
    }
    if constexpr (NLDS > 0) {
      // The next row's HBM -> LDS copies overwrite the staging slots: every
      // LDS read of them by this wave must have returned first. (Pass 2 has
      // consumed each one before its store; the gradient stores themselves
      // need not land before the next row's loads go out.)
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
  }
}

// ---------------------------------------------------------------------------
// Row-resident kernel: rows (in pair mode, half rows) of up to
// (NREG + NLDS) * 1024 16-byte chunks stay wholly on chip between the two
// passes -- NREG slots per lane in VGPRs, NLDS slots per lane in LDS filled
// straight from HBM -- so every logit is read from HBM exactly once (the
// streamed-tier kernel re-reads what does not fit). Slot i of thread tid is
// chunk i * 1024 + tid. All of a row's loads go out at its start, so pass 1
// reduces slots as they land. (Issuing the next row's slots
// during this row's gradient pass measured slower: it moves every read into
// the gradient pass and leaves pass 1 with no memory traffic of its own.)
//
// Rows are dealt out by a ticket counter in the workspace (all-ones before
// the launch, so the first ticket is 0) to the resident workgroups: one that
// finishes early takes more rows, which evens out rows of unequal cost
// (ignored rows are only written), and the next row's loads go out right
// behind this row's gradient stores. Measured on MI355X against a fixed
// stride (workgroup b takes rows b, b + grid, ...): 201088-column bf16 rows
// 8.95 -> 8.76 ms; 128256-column bf16 rows 1.318 -> 1.298 ms, and with no
// ignored rows 1.575 -> 1.411 ms. In pair mode (fp32 rows too long for one workgroup's chip
// space) the two halves of row r are tickets 2r and 2r + 1, and a
// workgroup takes its next ticket only after its current half has exchanged
// statistics with its partner. That makes the waits deadlock-free without
// co-residency guarantees: a waiting half's partner ticket is either held
// by a running workgroup, which publishes before it waits, or is the newest
// ticket, taken by the next workgroup to finish a half -- so any two
// resident workgroups make progress. (The wait is bounded all the same; a
// partner that never comes gives a NaN row.)
//
// Register discipline: every per-slot test compares the slot index with the
// end slot `se` or the target's slot `st`, both re-read through an empty asm
// at each use, and the lane index is re-derived every row, so the compiler
// keeps a few scalars live instead of a lane mask or offset per slot. In the
// end slot, lanes past the row end load the last chunk again (in bounds),
// count as -inf and store nothing; slots past the end slot load the last
// chunk (one line per wave) and are not reduced or stored.
// ---------------------------------------------------------------------------
template <typename TI, typename TO, int NREG, int NLDS, int MODE>
__global__ __launch_bounds__(1024) void ce_rowres_kernel(RowParams p) {
  static_assert(MODE == kFused || MODE == kPair, "the fused call, whole or half rows");
  constexpr int BLOCK = 1024;
  constexpr bool PAIR = MODE == kPair;
  constexpr int W = Elem<TI>::VEC;                 // elements per chunk
  constexpr uint32_t OB = W * Elem<TO>::BYTES;     // gradient bytes per chunk
  constexpr uint32_t SLOT = BLOCK * 16u;           // bytes of input per slot
  __shared__ float red_m[2][BLOCK / 64];
  __shared__ float red_s[2][BLOCK / 64];
  __shared__ u32x4 stage[NLDS > 0 ? NLDS : 1][NLDS > 0 ? BLOCK : 1];
  __shared__ float epi[2][4];
  [[maybe_unused]] __shared__ float pair_sh[2][4];
  [[maybe_unused]] __shared__ uint32_t tick_sh[2];
  [[maybe_unused]] __shared__ float zt_sh[2];    // whole rows: the target logit

  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63u;
  const uint32_t wid = tid >> 6;
  const size_t in_row_bytes = static_cast<size_t>(p.ld_in) * Elem<TI>::BYTES;
  const size_t out_row_bytes = static_cast<size_t>(p.ld_out) * Elem<TO>::BYTES;
  const uint32_t neg_w = Elem<TI>::NEG_INF_WORD;
  const kconst_i32* seg_ids = (const kconst_i32*)p.seg_ids;
  const kconst_i32* seg_start = (const kconst_i32*)p.seg_start;
  [[maybe_unused]] bool pair_broken = false;     // thread 0: a partner once failed to arrive
  // The counter starts at all-ones: a ticket is the value returned plus one,
  // added where the value is read back (using the return value right away
  // would make the wave wait for it, and with it every earlier access).
  auto take_ticket = [&]() -> uint32_t {
    return __hip_atomic_fetch_add(p.tickets, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  auto read_ticket = [&](uint32_t i) -> uint32_t {
    return __builtin_amdgcn_readfirstlane(tick_sh[i]) + 1u;
  };
  auto ticket_row = [&](uint32_t tk) -> int64_t {
    return static_cast<int64_t>(PAIR ? tk >> 1 : tk);
  };

  // Ticket k is row k (pair mode: row k / 2, half k % 2). Thread 0 takes
  // the next ticket while the current row is in flight (whole rows: right
  // after the row's loads go out; pair mode: once the half's exchange is
  // done, which keeps the pairing deadlock-free) and shares it through LDS
  // at the one barrier every row passes after its last use of the previous
  // value. Tickets are read back as scalars, so the row index and all that
  // derives from it stay uniform. (Tickets taken two rows ahead measured
  // slower.)
  if (tid == 0) tick_sh[0] = take_ticket();
  __syncthreads();
  uint32_t k = read_ticket(0);
  __syncthreads();                                // tick_sh[0] is rewritten by the first row
  int64_t r = ticket_row(k);
  int64_t t_next = r < p.T ? row_label(p, r) : 0;
  int par = 0;
  while (r < p.T) {
    const uint32_t half = PAIR ? (k & 1u) : 0u;
    const int64_t t64 = t_next;
    // this row's (half row's) geometry
    const int64_t c0 = (PAIR && half) ? p.pair_split : 0;
    const uint32_t V = static_cast<uint32_t>(PAIR ? (half ? p.V - p.pair_split : p.pair_split) : p.V);
    const uint32_t nchunk = V / W;
    const uint32_t c16_last = (nchunk > 0 ? nchunk - 1 : 0) * 16u;
    const uint32_t tail_begin = nchunk * W;
    // the slot that holds the (half) row's last chunk (-1: no whole chunk)
    const int se_row = nchunk > 0 ? static_cast<int>((nchunk - 1) / BLOCK) : -1;
    auto end_slot = [&]() -> int {
      int se = __builtin_amdgcn_readfirstlane(se_row);
      asm volatile("" : "+s"(se));
      return se;
    };
    void* grow = static_cast<char*>(p.grad) + r * out_row_bytes + c0 * Elem<TO>::BYTES;
    const bool valid = t64 != p.ignore_index;   // (the mask is folded into the label)
    if (!valid || t64 - p.v0 < 0 || t64 - p.v0 >= p.V) {
      // Ignored row: +0.0 everywhere, logits never read. Valid row with an
      // out-of-range target: NaN loss and gradient row. (Both halves of a
      // pair decide alike; half 0 writes the row's loss.)
      // The next ticket is taken and published before the row's stores go
      // out: loads, atomics and stores share one in-order counter, so
      // reading it after the fill would wait for every store of the fill.
      // (Taking it and reading it in one thread-0 block also keeps the
      // compiler from treating it as pending in the other waves.)
      if (tid == 0) tick_sh[par] = take_ticket();
      fill_row<TO, BLOCK>(p, r, grow, V, valid ? __builtin_nanf("") : 0.f, true,
                          !PAIR || half == 0);
      __syncthreads();
      k = read_ticket(par);
      r = ticket_row(k);
      t_next = r < p.T ? row_label(p, r) : 0;
      par ^= 1;
      continue;
    }
    const int64_t tl = t64 - p.v0 - c0;
    const bool owned = tl >= 0 && tl < static_cast<int64_t>(V);
    const uint32_t t = owned ? static_cast<uint32_t>(tl) : V;
    const char* zrow = static_cast<const char*>(p.logits) + r * in_row_bytes + c0 * Elem<TI>::BYTES;
    // The lane index, re-derived every row: every per-lane mask and offset
    // below is formed inside the row, next to its use.
    uint32_t tid_r = tid;
    asm volatile("" : "+v"(tid_r));
    const uint32_t vin = tid_r * 16u;

    // ---- every slot's load goes out now (read once: non-temporal) --------
    // While an HBM -> LDS copy is outstanding the compiler cannot count the
    // memory counter (the copy writes LDS through the vector memory path):
    // the first use of a register slot then waits for every load of the row.
    // Half rows issue their LDS copies first and wait for them explicitly
    // before pass 1 (the oldest loads, so the register slots stay in flight
    // and get per-slot waits): the half reaches its exchange sooner (151936-
    // column fp32 rows 6.52 -> 6.45 ms). Whole rows issue them last and wait
    // for the whole row (the copies-first order measured 0.5% slower on
    // 201088-column bf16 rows, whose pass-1 latency is hidden by other CUs).
    constexpr bool kCopiesFirst = PAIR;
    auto issue_copies = [&]() {
      // (every LDS slot is loaded, those past the end slot from the last
      // chunk: loads on only some paths would make the first wait cover them)
#pragma unroll
      for (int j = 0; j < NLDS; ++j) {
        // HBM -> LDS without a register round trip: lane l of a wave lands
        // at base + 16 l, so slot j of thread tid is stage[j][tid].
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void*)(zrow + min(vin + (NREG + j) * SLOT, c16_last)),
            (__attribute__((address_space(3))) void*)(&stage[j][tid_r & ~63u]), 16, 0, kNT);
      }
    };
    if constexpr (kCopiesFirst) issue_copies();
    u32x4 raw[NREG];
    {
      const __amdgpu_buffer_rsrc_t rin =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(zrow), 0, nchunk * 16u, kBufWord3);
#pragma unroll
      for (int i = 0; i < NREG; ++i)
        raw[i] = __builtin_amdgcn_raw_buffer_load_b128(rin, min(vin + i * SLOT, c16_last), 0, kNT);
    }
    if constexpr (!kCopiesFirst) issue_copies();
    [[maybe_unused]] int32_t sid = 0;
    if (p.seg_mean) sid = seg_ids[r];
    // The target logit: in pair mode its own load, issued behind the slots
    // and first needed after the exchange; for whole rows the lane whose
    // slot holds it hands it over through LDS (measured 5% faster on
    // 128256-column bf16 rows, level on the others).
    [[maybe_unused]] const float zt_ld = (PAIR && owned) ? Elem<TI>::load1(zrow, t) : kNegInf;
    [[maybe_unused]] uint32_t k_next = 0;          // thread 0: the next ticket
    if (!PAIR && tid == 0) k_next = take_ticket();

    // Where the target sits: chunk ct, element kt, slot st, lane `mine`.
    const uint32_t ct = t / W;
    const uint32_t kt = t - ct * W;
    const int st_row = t < tail_begin ? static_cast<int>(ct / BLOCK) : -1;
    const bool mine = t < tail_begin && (ct % BLOCK) == tid_r;
    const uint32_t kq = (kt * Elem<TI>::BYTES) >> 2;
    const uint32_t ksh = (kt * Elem<TI>::BYTES * 8u) & 31u;
    const uint32_t kmask = Elem<TI>::BYTES == 4 ? 0xffffffffu : (0xffffu << ksh);
    const uint32_t kput = Elem<TI>::BYTES == 4 ? 0xff800000u : (0xff80u << ksh);
    auto tgt_slot = [&]() -> int {
      int st = __builtin_amdgcn_readfirstlane(st_row);
      asm volatile("" : "+s"(st));
      return st;
    };
    // Lanes past the row end (in the end slot) count as -inf; the target's
    // element in its slot too (in the one lane that holds it).
    auto fixed = [&](u32x4 v, int slot) -> u32x4 {
      if (slot == end_slot()) {
        asm volatile("");                         // a branch, not selects in every slot
        const bool out = static_cast<uint32_t>(slot) * BLOCK + tid_r >= nchunk;
        v.x = out ? neg_w : v.x;
        v.y = out ? neg_w : v.y;
        v.z = out ? neg_w : v.z;
        v.w = out ? neg_w : v.w;
      }
      if (slot == tgt_slot()) {
        if (!PAIR && mine) {
          const uint32_t w = kq == 0 ? v.x : (kq == 1 ? v.y : (kq == 2 ? v.z : v.w));
          zt_sh[par] = Elem<TI>::BYTES == 4 ? __uint_as_float(w) : __uint_as_float((w >> ksh) << 16);
        }
        const uint32_t am = mine ? ~kmask : ~0u, om = mine ? kput : 0u;
        v.x = kq == 0 ? (v.x & am) | om : v.x;
        v.y = kq == 1 ? (v.y & am) | om : v.y;
        v.z = kq == 2 ? (v.z & am) | om : v.z;
        v.w = kq == 3 ? (v.w & am) | om : v.w;
      }
      return v;
    };

    [[maybe_unused]] int32_t seg_len = 1;
    if (p.seg_mean) {
      sid = sid < 0 ? 0 : (sid >= p.num_segments ? p.num_segments - 1 : sid);
      const int32_t len = seg_start[sid + 1] - seg_start[sid];
      seg_len = len > 0 ? len : 1;
    }

    // ---- pass 1: register slots, then LDS slots, one online update each ----
    float mL = kNegInf, s = 0.f;
    if constexpr (kCopiesFirst && NLDS > 0) {
      // this wave's HBM -> LDS copies have landed (and the scalar reads of
      // the row set-up); the register slots may still be in flight
      __builtin_amdgcn_s_waitcnt(waitcnt_imm(NREG, 7, 0));
    }
#pragma unroll
    for (int i = 0; i < NREG; ++i) {
      if (i > end_slot()) break;
      float x[W];
      Elem<TI>::unpack(fixed(raw[i], i), x);
      online_group<W>(mL, s, x);
    }
    if constexpr (NLDS > 0) {
      if (NREG <= end_slot()) {
        if constexpr (!kCopiesFirst) __builtin_amdgcn_s_waitcnt(0);   // the copies have landed
#pragma unroll
        for (int j = 0; j < NLDS; ++j) {
          if (NREG + j > end_slot()) break;
          float x[W];
          Elem<TI>::unpack(fixed(stage[j][tid_r], NREG + j), x);
          online_group<W>(mL, s, x);
        }
      }
    }
    if (tid_r < V - tail_begin) {
      const uint32_t j = tail_begin + tid_r;
      float xv = Elem<TI>::load1(zrow, j);
      if (j == t) {
        if (!PAIR) zt_sh[par] = xv;
        xv = kNegInf;
      }
      merge(mL, s, xv * kL2E, (xv == kNegInf) ? 0.f : 1.f);
    }
    // Every load of the row has landed (slots past the end slot were issued
    // with the others). Saying so here keeps the compiler from waiting for
    // each slot's load again in pass 2, where its count would leave out the
    // gradient stores issued in between and stall on them.
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 7, 15));
    block_reduce<BLOCK>(mL, s, red_m, red_s, par, tid_r & 63u, tid_r >> 6);
    // (zt_sh is written before the reduction's barrier)
    const float zt = PAIR ? zt_ld : (owned ? zt_sh[par] : kNegInf);

    float ztm = zt;
    if constexpr (PAIR) {
      // Publish this half's partial, then take the partner's. Each half's
      // slot is two 64-bit words, (shift, sum) and (target logit, 0), filled
      // with all-ones before the launch; each word is stored and polled as
      // one relaxed device-scope atomic, so a word that differs from all-ones
      // is complete and no fence is needed. The merge is symmetric, so both
      // halves hold the same row statistics. The next ticket is taken once
      // the partner has been heard from (or given up on).
      uint64_t* slot = reinterpret_cast<uint64_t*>(p.pair_part) + 4 * r;
      if (tid == 0) {
        const uint64_t ms = (static_cast<uint64_t>(__float_as_uint(s)) << 32) | __float_as_uint(mL);
        __hip_atomic_store(slot + 2 * half, ms, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(slot + 2 * half + 1, static_cast<uint64_t>(__float_as_uint(zt)),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        float pm = __builtin_nanf(""), ps = __builtin_nanf(""), pz = __builtin_nanf("");
        if (!pair_broken) {
          uint64_t w0 = ~0ull, w1 = ~0ull;
          uint32_t n = 0;
          while (n < p.pair_spin) {
            if (w0 == ~0ull)
              w0 = __hip_atomic_load(slot + 2 * (half ^ 1u), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (w1 == ~0ull)
              w1 = __hip_atomic_load(slot + 2 * (half ^ 1u) + 1, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
            if (w0 != ~0ull && w1 != ~0ull) break;
            __builtin_amdgcn_s_sleep(2);
            ++n;
          }
          if (n < p.pair_spin) {
            pm = __uint_as_float(static_cast<uint32_t>(w0));
            ps = __uint_as_float(static_cast<uint32_t>(w0 >> 32));
            pz = __uint_as_float(static_cast<uint32_t>(w1));
          } else {
            pair_broken = true;
          }
        }
        if (pair_broken)   // counted, and reported by a validating call
          __hip_atomic_fetch_add(p.tickets + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        k_next = take_ticket();
        pair_sh[par][0] = pm;
        pair_sh[par][1] = ps;
        pair_sh[par][2] = pz;
      }
      __syncthreads();
      const float pm = pair_sh[par][0], ps = pair_sh[par][1], pz = pair_sh[par][2];
      if (pm != pm) {
        mL = __builtin_nanf("");
        s = __builtin_nanf("");
      } else {
        merge(mL, s, pm, ps);
      }
      ztm = fmaxf(zt, pz);
    }
    // Wave 0 runs the fp64 epilogue and shares the row factors through LDS
    // (with the next ticket, whose atomic has returned by then). The
    // epilogue's scalar inputs pass an empty asm, so their fp64 forms are
    // made here, not hoisted out of the row loop into registers held
    // throughout.
    if (wid == 0) {
      RowParams q = p;
      asm volatile("" : "+s"(q.grad_scale), "+s"(q.z_alpha));
      const RowOut o = row_epilogue(q, r, mL, s, ztm, tid == 0 && (!PAIR || half == 0),
                                    1.0 / static_cast<double>(seg_len));
      if (lane == 0) {
        epi[par][0] = o.g_t;
        epi[par][1] = o.cnt;
        epi[par][2] = o.kl;
        tick_sh[par] = k_next;
      }
    }
    __syncthreads();
    const float cnt = epi[par][1], kl = epi[par][2];
    k = read_ticket(par);
    t_next = ticket_row(k) < p.T ? row_label(p, ticket_row(k)) : 0;
    const int64_t r_next = ticket_row(k);

    // ---- pass 2: gradient ----------------------------------------------
    const __amdgpu_buffer_rsrc_t rout = __builtin_amdgcn_make_buffer_rsrc(grow, 0, nchunk * OB, kBufWord3);
    // (opaque: with equal element sizes the store offsets equal the load
    // offsets, and the compiler would keep every load's offset live for them)
    uint32_t vout = tid_r * OB;
    asm volatile("" : "+v"(vout));
    auto store_slot = [&](int slot, const u32x4 v) {
      float x[W];
      Elem<TI>::unpack(v, x);
      float g[W];
#pragma unroll
      for (int e = 0; e < W; ++e) g[e] = cnt * fexp2(__builtin_fmaf(x[e], kL2E, -kl));
      if (slot == end_slot() && static_cast<uint32_t>(slot) * BLOCK + tid_r >= nchunk) return;
      const uint32_t vo = vout + static_cast<uint32_t>(slot) * BLOCK * OB;
      if constexpr (Elem<TO>::BYTES == 2 && W == 8) {
        const u32x4 q = {pack_bf16x2(g[0], g[1]), pack_bf16x2(g[2], g[3]),
                         pack_bf16x2(g[4], g[5]), pack_bf16x2(g[6], g[7])};
        __builtin_amdgcn_raw_buffer_store_b128(q, rout, vo, 0, kNT);
      } else if constexpr (Elem<TO>::BYTES == 2) {
        const u32x2 q = {pack_bf16x2(g[0], g[1]), pack_bf16x2(g[2], g[3])};
        __builtin_amdgcn_raw_buffer_store_b64(q, rout, vo, 0, kNT);
      } else {
#pragma unroll
        for (int h = 0; h < W / 4; ++h) {
          const u32x4 q = {__float_as_uint(g[4 * h]), __float_as_uint(g[4 * h + 1]),
                           __float_as_uint(g[4 * h + 2]), __float_as_uint(g[4 * h + 3])};
          __builtin_amdgcn_raw_buffer_store_b128(q, rout, vo + 16u * h, 0, kNT);
        }
      }
    };
#pragma unroll
    for (int i = 0; i < NREG; ++i) {
      if (i > end_slot()) break;
      store_slot(i, raw[i]);
    }
#pragma unroll
    for (int j = 0; j < NLDS; ++j) {
      if (NREG + j > end_slot()) break;
      store_slot(NREG + j, stage[j][tid_r]);
    }
    if (tid_r < V - tail_begin) {
      const uint32_t j = tail_begin + tid_r;
      const float g = (j == t) ? epi[par][0]
                               : cnt * fexp2(__builtin_fmaf(Elem<TI>::load1(zrow, j), kL2E, -kl));
      Elem<TO>::store1(grow, j, g);
    }
    // The target column: written after its chunk by the same lane, so this
    // store lands last (a lane's stores to one address stay in order).
    if (mine) Elem<TO>::store1(grow, t, epi[par][0]);
    // The next row's HBM -> LDS copies overwrite the staging slots: every
    // LDS read of them by this wave must have returned first.
    if constexpr (NLDS > 0) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    r = r_next;
    par ^= 1;
  }
}

// Debug scan (CE_FLAG_VALIDATE): block b writes to words[b] the OR over its
// rows of 1 (target neither ignored nor in [0, V)), 2 (segment id outside
// [0, S)) and 4 (segment id below the previous row's). Grid-stride over rows;
// every block writes its word, so the words need no clearing.
constexpr int kValidateBlocks = 1024;

__global__ __launch_bounds__(256) void ce_validate_kernel(const int64_t* __restrict__ targets,
                                                          int64_t T, int64_t V, int64_t ignore,
                                                          const int32_t* __restrict__ seg_ids,
                                                          int32_t S, uint32_t* __restrict__ words) {
  __shared__ uint32_t part[256 / 64];
  uint32_t b = 0;
  for (int64_t r = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; r < T;
       r += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t t = targets[r];
    if (t != ignore && (t < 0 || t >= V)) b |= 1u;
    if (seg_ids) {
      const int32_t s = seg_ids[r];
      if (s < 0 || s >= S) b |= 2u;
      if (r > 0 && seg_ids[r - 1] > s) b |= 4u;
    }
  }
  for (int off = 32; off >= 1; off >>= 1) b |= __shfl_xor(b, off, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = b;
  __syncthreads();
  if (threadIdx.x == 0) words[blockIdx.x] = part[0] | part[1] | part[2] | part[3];
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

// Merge the (shift, sum, target logit) statistics of P column shards of each
// row and finish the row: loss, NLL staging for segment sums, and the saved
// state the gradient pass needs (kRowState floats, laid out above).
struct FinishParams {
  const float* stats;        // [P, T, 3]
  const int64_t* targets;
  const uint8_t* mask;
  const int32_t* seg_ids;
  const int32_t* seg_start;
  float* loss_out;
  float* nll_ws;
  float* row_state;          // [T, kRowState]
  int64_t T, V, ignore_index;
  int32_t P, num_segments, seg_mean;
  float z_alpha;
};

__global__ __launch_bounds__(256) void ce_finish_kernel(FinishParams f) {
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (r >= f.T) return;
  const int64_t t = f.targets[r];
  const bool valid = (t != f.ignore_index) && (f.mask == nullptr || f.mask[r] != 0);
  float* rs = f.row_state + kRowState * r;
  if (!valid || t < 0 || t >= f.V) {
    const float fill = valid ? __builtin_nanf("") : 0.f;
    f.loss_out[r] = fill;
    if (f.nll_ws) f.nll_ws[r] = fill;
#pragma unroll
    for (int k = 0; k < kRowState; ++k) rs[k] = 0.f;
    rs[5] = valid ? kRowPoisoned : kRowIgnored;
    return;
  }
  // Merge in fp64 in shard order: max shift, rescaled sums, owner's logit.
  double M = -HUGE_VAL;
  float zt = kNegInf;
  for (int k = 0; k < f.P; ++k) {
    const float* st = f.stats + 3 * (static_cast<int64_t>(k) * f.T + r);
    M = fmax(M, static_cast<double>(st[0]));
    zt = fmaxf(zt, st[2]);
  }
  double S = 0.0;
  if (M != -HUGE_VAL) {
    for (int k = 0; k < f.P; ++k) {
      const float* st = f.stats + 3 * (static_cast<int64_t>(k) * f.T + r);
      if (st[0] != kNegInf) S += static_cast<double>(st[1]) * exp2(static_cast<double>(st[0]) - M);
    }
  }
  const RowLoss L = row_loss(lse_from_partial(M, S), static_cast<double>(zt));
  const double alpha = static_cast<double>(f.z_alpha);
  const double zfac = (alpha == 0.0) ? 0.0 : 2.0 * alpha * L.lse;
  const double seg = f.seg_mean ? segment_factor(f.seg_ids, f.seg_start, f.num_segments, r) : 1.0;
  f.loss_out[r] = static_cast<float>(L.nll + ((alpha == 0.0) ? 0.0 : alpha * L.lse * L.lse));
  if (f.nll_ws) f.nll_ws[r] = static_cast<float>(L.nll);
  const double lse_l2 = static_cast<double>(kL2E) * L.lse;
  rs[0] = static_cast<float>(lse_l2);
  rs[1] = static_cast<float>(L.p_nt);
  rs[2] = static_cast<float>(L.p_t);
  rs[3] = static_cast<float>(zfac);
  rs[4] = static_cast<float>(seg);
  rs[5] = kRowValid;
  rs[6] = isfinite(lse_l2) ? static_cast<float>(lse_l2 - static_cast<double>(rs[0])) : 0.f;
  rs[7] = 0.f;
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

// Grid: `per_cu` workgroups per compute unit (0: as many as fit), each
// looping over rows; never more workgroups than rows.
template <typename Kern>
ce_status launch_persistent(Kern kern, int block, std::atomic<int>& occ, const RowParams& rp,
                            hipStream_t stream, int per_cu_cap = 0) {
  int per_cu = occ.load(std::memory_order_relaxed);
  if (per_cu <= 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, block, 0) != hipSuccess || n <= 0)
      return CE_ERR_HIP;
    occ.store(n, std::memory_order_relaxed);
    per_cu = n;
  }
  const int cus = device_cus();
  if (cus <= 0) return CE_ERR_HIP;
  if (per_cu_cap > 0) per_cu = per_cu_cap;
  const int64_t want = static_cast<int64_t>(cus) * per_cu;
  const int64_t grid = rp.T < want ? rp.T : want;
  if (grid <= 0) return CE_OK;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(block), 0, stream, rp);
  return hipGetLastError() == hipSuccess ? CE_OK : CE_ERR_HIP;
}

template <typename TI, typename TO, int BLOCK, int NRES, int NRAW, int NLDS, int U, bool WRITE,
          bool PF = false, bool EPI1 = false, int OG = U, int MODE = kFused, bool ENT = false>
ce_status launch_rows(const RowParams& rp, hipStream_t stream, int per_cu_cap = 0) {
  static std::atomic<int> occ{0};
  return launch_persistent(
      ce_rows_kernel<TI, TO, BLOCK, NRES, NRAW, NLDS, U, WRITE, PF, EPI1, OG, MODE, ENT>, BLOCK,
      occ, rp, stream, per_cu_cap);
}

__global__ __launch_bounds__(256) void ce_fill_u32_kernel(uint32_t* __restrict__ p, int64_t n,
                                                          uint32_t v) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * 256)
    p[i] = v;
}

// Row-resident shape: 16 register slots and 9 LDS slots per lane of 1024,
// 25600 chunks (400 KiB) of a row on chip. Rows (half rows) that fit in the
// register slots take an instance without the LDS slots: a load into an LDS
// slot past the row end would still cost its copy, and the first register
// slot's wait would cover it.
constexpr int kResReg = 16, kResLds = 9;
constexpr int64_t kResChunks = int64_t{kResReg + kResLds} * 1024;
constexpr int64_t kResRegChunks = int64_t{kResReg} * 1024;
// Rows of up to this many chunks take the row kernel (512 lanes, the whole
// row in LDS up to 4096 chunks); longer ones the row-resident kernel.
constexpr int64_t kRowsChunks = 8192;

// Whole rows on the row-resident kernel, one workgroup per CU, dealt by
// ticket: the counter is set to all-ones by a one-block fill kernel first
// (capturable), and the grid is the resident workgroups only -- every
// workgroup beyond them would launch after the tickets run out, only to take
// one past the end (16384 workgroups instead of 256 measured 8.77 vs 8.62 ms
// on 201088-column bf16 rows).
template <typename TI, typename TO, int NLDS>
ce_status launch_rowres_shape(const RowParams& rp, hipStream_t stream) {
  if (rp.tickets == nullptr) return CE_ERR_WORKSPACE;
  hipLaunchKernelGGL(ce_fill_u32_kernel, dim3(1), dim3(256), 0, stream, rp.tickets, int64_t{1}, ~0u);
  if (hipGetLastError() != hipSuccess) return CE_ERR_HIP;
  static std::atomic<int> occ{0};
  return launch_persistent(ce_rowres_kernel<TI, TO, kResReg, NLDS, kFused>, 1024, occ, rp, stream);
}

template <typename TI, typename TO>
ce_status launch_rowres(const RowParams& rp, hipStream_t stream) {
  if (rp.V / Elem<TI>::VEC <= kResRegChunks) return launch_rowres_shape<TI, TO, 0>(rp, stream);
  return launch_rowres_shape<TI, TO, kResLds>(rp, stream);
}

// Pair mode: fp32 rows of 25601..51200 chunks, two workgroups per row, each
// holding its half row on chip (the row-resident kernel's pair mode). The
// exchange slots, the ticket counter and the give-up count are filled with
// all-ones first (a kernel, so the call stays capturable in a graph). An
// ordinary launch: the ticket order needs no co-residency guarantee beyond
// two resident workgroups.
template <typename TI, typename TO, int NLDS>
ce_status launch_pair_shape(const RowParams& rp, hipStream_t stream) {
  auto kern = ce_rowres_kernel<TI, TO, kResReg, NLDS, kPair>;
  static std::atomic<int> occ{0};
  int per_cu = occ.load(std::memory_order_relaxed);
  if (per_cu <= 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 1024, 0) != hipSuccess ||
        per_cu <= 0)
      return CE_ERR_HIP;
    occ.store(per_cu, std::memory_order_relaxed);
  }
  const int cus = device_cus();
  if (cus <= 0) return CE_ERR_HIP;
  const int64_t grid = std::max<int64_t>(2, std::min<int64_t>(2 * rp.T, int64_t{cus} * per_cu));
  const int64_t n = 8 * rp.T + 2;   // the slots, the ticket counter, the give-up count
  const unsigned nb = static_cast<unsigned>(std::min<int64_t>((n + 255) / 256, 1024));
  hipLaunchKernelGGL(ce_fill_u32_kernel, dim3(nb), dim3(256), 0, stream, rp.pair_part, n, ~0u);
  if (hipGetLastError() != hipSuccess) return CE_ERR_HIP;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(1024), 0, stream, rp);
  return hipGetLastError() == hipSuccess ? CE_OK : CE_ERR_HIP;
}

template <typename TI, typename TO>
ce_status launch_rows_pair(const RowParams& rp, hipStream_t stream) {
  // the longer half: columns [pair_split, V)
  if ((rp.V - rp.pair_split) / Elem<TI>::VEC <= kResRegChunks)
    return launch_pair_shape<TI, TO, 0>(rp, stream);
  return launch_pair_shape<TI, TO, kResLds>(rp, stream);
}

template <typename TI, typename TO, bool WRITE, int MODE = kFused, bool ENT = false>
ce_status launch_rows_scalar(const RowParams& rp, hipStream_t stream) {
  static std::atomic<int> occ{0};
  return launch_persistent(ce_rows_scalar_kernel<TI, TO, 256, WRITE, MODE, ENT>, 256, occ, rp,
                           stream);
}

// Pick a kernel variant for (input type, output type, vector path or not).
// Kernel shape by row length (chunks of 16 bytes), measured on MI355X; the
// more of a row stays on chip, the less of it pass 2 reads again:
//  * up to 8192 chunks: the row kernel, 512 lanes, 8 slots per lane in LDS
//    (64 KiB: all of a row of up to 4096 chunks), the rest streamed 2 slots
//    per step, one workgroup per row (up to 64 per CU in the grid; the LDS
//    footprint lets two run at once);
//  * 8193..25600 chunks: the row-resident kernel, the whole row on chip
//    (16 register slots, and 9 LDS slots past 16384 chunks), one workgroup
//    per CU, rows dealt by ticket;
//  * fp32 rows of 25601..51200 chunks: the row-resident kernel in pair mode,
//    two workgroups per row;
//  * longer rows: the row kernel, 1024 lanes, 13 slots per lane on chip
//    (4 VGPR + 9 LDS: 208 KiB of a row), the rest streamed with one online
//    update per slot.
template <typename TI, typename TO, bool WRITE>
ce_status dispatch_rows(const RowParams& rp, bool vec, hipStream_t stream) {
  if (!vec) return launch_rows_scalar<TI, TO, WRITE>(rp, stream);
  const int64_t nchunk = rp.V / Elem<TI>::VEC;
  if (nchunk <= kRowsChunks)
    return launch_rows<TI, TO, 512, 0, 0, 8, 2, WRITE, true, true>(rp, stream, 64);
  static_assert(WRITE, "the gradient call: forward-only rows take dispatch_forward");
  if (nchunk <= kResChunks) return launch_rowres<TI, TO>(rp, stream);
  // fp32 rows up to twice that: two workgroups per row, each half on chip
  // (the host sets pair_part exactly for those rows)
  if constexpr (Elem<TI>::BYTES == 4) {
    if (rp.pair_part != nullptr) return launch_rows_pair<TI, TO>(rp, stream);
  }
  return launch_rows<TI, TO, 1024, 0, 4, 9, 4, WRITE, true, true, 1>(rp, stream, 64);
}

// Forward only (no gradient): nothing is reused, so no slot is kept for a
// second pass; LDS staging serves only to keep more of a row in flight.
// Shapes by row length, measured on MI355X (the entropy variant carries two
// more ALU ops per element, so it keeps fewer elements per online update):
//  * short rows (<= 8192 chunks): streamed, 256 lanes;
//  * medium rows (<= 20000 chunks): 256 lanes, plain forward with 8 slots
//    per lane staged in LDS;
//  * long rows: plain fp32 1024 lanes with 9 LDS slots, plain bf16 256 lanes
//    with 16; the fp32 entropy variant 256 lanes with 16 LDS slots.
// The entropy variant streams 4 slots per step with two per online update
// at every length below that (2 slots per step measured 2% slower on 4000-
// chunk rows).
template <typename TI, bool ENT>
ce_status dispatch_forward(const RowParams& rp, bool vec, hipStream_t stream) {
  if (!vec) return launch_rows_scalar<TI, TI, false, kFused, ENT>(rp, stream);
  const int64_t nchunk = rp.V / Elem<TI>::VEC;
  if constexpr (ENT) {
    if (Elem<TI>::BYTES == 4 && nchunk > 20000)
      return launch_rows<TI, TI, 256, 0, 0, 16, 4, false, true, true, 2, kFused, true>(rp, stream, 64);
    return launch_rows<TI, TI, 256, 0, 0, 0, 4, false, true, true, 2, kFused, true>(rp, stream, 64);
  } else {
    if (nchunk <= 8192) return launch_rows<TI, TI, 256, 0, 0, 0, 4, false, true, true>(rp, stream, 64);
    if (nchunk <= 20000) return launch_rows<TI, TI, 256, 0, 0, 8, 4, false, true, true>(rp, stream, 64);
    if (Elem<TI>::BYTES == 4)
      return launch_rows<TI, TI, 1024, 0, 0, 9, 4, false, true, true, 1>(rp, stream, 64);
    return launch_rows<TI, TI, 256, 0, 0, 16, 4, false, true, true>(rp, stream, 64);
  }
}

template <typename TI>
ce_status dispatch_out(const RowParams& rp, int32_t grad_dtype, bool write, bool vec,
                       hipStream_t stream) {
  if (!write) return dispatch_forward<TI, false>(rp, vec, stream);
  if (grad_dtype == CE_DTYPE_F32) return dispatch_rows<TI, float, true>(rp, vec, stream);
  return dispatch_rows<TI, bf16_t, true>(rp, vec, stream);
}

// Statistics and gradient passes of a shard stream whole rows (nothing is
// reused between the two calls). Shapes by shard row length, measured on
// MI355X:
//  * statistics: up to 4096 chunks streamed on 256 lanes; longer rows stage
//    8 (up to 14000 chunks) or 16 slots per lane in LDS, which only deepens
//    the loads in flight (75% -> 81-83% of 8 TB/s on such rows);
//  * gradient: 1024 lanes, 4 slots per step up to 4096 chunks, else 8 with
//    the next 8 in flight while the current ones are written (3-8% faster
//    than 256 lanes; double-buffering: 8016-chunk rows 1.343 -> 1.277 ms).
template <typename TI, int MODE, typename TO = TI>
ce_status dispatch_shard(const RowParams& rp, bool vec, hipStream_t stream) {
  constexpr bool W = MODE == kGrad;
  if (!vec) return launch_rows_scalar<TI, TO, W, MODE>(rp, stream);
  const int64_t nchunk = rp.V / Elem<TI>::VEC;
  if constexpr (MODE == kStats) {
    if (nchunk <= 4096) return launch_rows<TI, TO, 256, 0, 0, 0, 4, W, true, true, 4, MODE>(rp, stream, 64);
    if (nchunk <= 14000) return launch_rows<TI, TO, 256, 0, 0, 8, 4, W, true, true, 4, MODE>(rp, stream, 64);
    return launch_rows<TI, TO, 256, 0, 0, 16, 4, W, true, true, 4, MODE>(rp, stream, 64);
  } else {
    if (nchunk <= 4096) return launch_rows<TI, TO, 1024, 0, 0, 0, 4, W, false, true, 4, MODE>(rp, stream, 64);
    return launch_rows<TI, TO, 1024, 0, 0, 0, 8, W, true, true, 8, MODE>(rp, stream, 64);
  }
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

// Bytes spanned by T rows of V elements at stride ld (false on overflow).
bool span_bytes(int64_t T, int64_t V, int64_t ld, int bytes, size_t* out) {
  if (T == 0) {
    *out = 0;
    return true;
  }
  int64_t tmp = 0;
  if (!mul_ok(T - 1, ld, &tmp) || tmp > INT64_MAX - V) return false;
  if (!mul_ok(tmp + V, bytes, &tmp)) return false;
  *out = static_cast<size_t>(tmp);
  return true;
}

bool valid_dtype(int32_t dt) { return dt == CE_DTYPE_F32 || dt == CE_DTYPE_BF16; }

bool rows_vec(const void* ptr, int64_t ld, int bytes) {
  return (reinterpret_cast<uintptr_t>(ptr) % 16 == 0) && ((ld * bytes) % 16 == 0);
}

// Launch the segment-offset search (segments present) into the workspace.
ce_status launch_seg_bounds(const int32_t* segment_ids, int64_t T, int32_t S, void* workspace,
                            float** nll_ws, int32_t** seg_start, hipStream_t stream) {
  *nll_ws = static_cast<float*>(workspace);
  *seg_start = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) +
                                          align_up(static_cast<size_t>(T) * sizeof(float)));
  (void)hipGetLastError();
  const unsigned nb = static_cast<unsigned>((static_cast<int64_t>(S) + 1 + 255) / 256);
  hipLaunchKernelGGL(ce_seg_bounds_kernel, dim3(nb), dim3(256), 0, stream, segment_ids, T, S,
                     *seg_start);
  return hipGetLastError() == hipSuccess ? CE_OK : CE_ERR_HIP;
}

// Shape checks shared by the shard entry points.
ce_status check_shard(const ce_shard* s, size_t* in_bytes) {
  if (s == nullptr) return CE_ERR_INVALID_ARG;
  if (s->T < 0 || s->V < 1 || s->v0 < 0 || s->ld_logits < s->V) return CE_ERR_INVALID_ARG;
  if (!valid_dtype(s->logits_dtype)) return CE_ERR_INVALID_ARG;
  if (s->T > INT32_MAX || s->V > (int64_t{1} << 28)) return CE_ERR_UNSUPPORTED;
  if (!span_bytes(s->T, s->V, s->ld_logits, dtype_bytes(s->logits_dtype), in_bytes))
    return CE_ERR_INVALID_ARG;
  return CE_OK;
}

RowParams shard_params(const ce_shard* s, const void* logits, const int64_t* targets) {
  RowParams rp{};
  rp.logits = logits;
  rp.targets = targets;
  rp.T = s->T;
  rp.V = s->V;
  rp.ld_in = s->ld_logits;
  rp.ld_out = s->ld_logits;
  rp.ignore_index = s->ignore_index;
  rp.v0 = s->v0;
  return rp;
}

// Workspace bytes of the segment sums: the [T] NLL staging array and the
// [S + 1] segment offsets (none without segments).
size_t segment_ws_bytes(const ce_problem* p) {
  if (p->num_segments == 0) return 0;
  return align_up(static_cast<size_t>(p->T) * sizeof(float)) +
         align_up((static_cast<size_t>(p->num_segments) + 1) * sizeof(int32_t));
}

// Row scheduling space of the gradient pass (placed after the segment
// arrays): rows of 8193..25600 16-byte chunks run the row-resident kernel,
// whose ticket counter takes 4 bytes; fp32 rows of 25601..51200 chunks run
// its pair mode, with 32 bytes of exchange slots per row before the counter.
// A forward-only call needs none.
bool pair_rows(const ce_problem* p) {
  const int64_t nchunk = p->V / 4;
  return p->logits_dtype == CE_DTYPE_F32 && nchunk > kResChunks && nchunk - nchunk / 2 <= kResChunks;
}

// The pair mode's wait limit: kPairSpin, or CE_PAIR_SPIN_LIMIT from the
// environment (a test hook: 0 makes every half row give up at once, which
// forces the give-up path without stalling anything).
uint32_t pair_spin_limit() {
  const char* e = std::getenv("CE_PAIR_SPIN_LIMIT");
  if (e == nullptr || *e == '\0') return kPairSpin;
  char* end = nullptr;
  const unsigned long v = std::strtoul(e, &end, 10);
  return (end != nullptr && *end == '\0' && v <= kPairSpin) ? static_cast<uint32_t>(v) : kPairSpin;
}
// Whole rows on the row-resident kernel (dealt by ticket): 8193..25600
// chunks of 16 bytes.
bool rowres_rows(const ce_problem* p) {
  const int64_t nchunk = p->V / (p->logits_dtype == CE_DTYPE_F32 ? 4 : 8);
  return nchunk > kRowsChunks && nchunk <= kResChunks;
}
size_t sched_ws_bytes(const ce_problem* p, bool grad = true) {
  if (!grad || p->T == 0) return 0;
  if (pair_rows(p)) return align_up(static_cast<size_t>(p->T) * 8 * sizeof(uint32_t) + 2 * sizeof(uint32_t));
  if (rowres_rows(p)) return align_up(sizeof(uint32_t));
  return 0;
}
size_t validate_ws_bytes(const ce_problem* p) {
  return (p->flags & CE_FLAG_VALIDATE) ? align_up(kValidateBlocks * sizeof(uint32_t)) : 0;
}

// Validation and launches shared by the fused entry points. grad_out null
// is a forward; lse_out / ent_out (forward only) are optional [T] outputs.
ce_status run_rows(const ce_problem* p, const void* logits, const int64_t* targets,
                   const uint8_t* mask, const int32_t* segment_ids, float z_alpha,
                   float grad_scale, float* loss_out, float* seg_loss_out, void* grad_out,
                   float* lse_out, float* ent_out, void* workspace, size_t workspace_bytes,
                   void* stream_ptr) {
  // ---- host validation: nothing is enqueued on failure ----
  if (p == nullptr) return CE_ERR_INVALID_ARG;
  const int64_t T = p->T, V = p->V;
  if (T < 0 || V < 1) return CE_ERR_INVALID_ARG;
  if (p->logits_dtype != CE_DTYPE_F32 && p->logits_dtype != CE_DTYPE_BF16) return CE_ERR_INVALID_ARG;
  if (grad_out && p->grad_dtype != CE_DTYPE_F32 && p->grad_dtype != CE_DTYPE_BF16)
    return CE_ERR_INVALID_ARG;
  if ((p->flags & ~(CE_FLAG_SEGMENT_MEAN | CE_FLAG_VALIDATE)) != 0) return CE_ERR_INVALID_ARG;
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
  // two-workgroup rows deal 2 T tickets from a 32-bit counter
  if (grad_out && pair_rows(p) && T > (int64_t{1} << 31) - (int64_t{1} << 20)) return CE_ERR_UNSUPPORTED;
  if (V > (int64_t{1} << 28)) return CE_ERR_UNSUPPORTED;  // in-row byte offsets are 32-bit
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
  // The per-row outputs may not overlap the logits.
  for (const float* o : {static_cast<const float*>(loss_out), static_cast<const float*>(lse_out),
                         static_cast<const float*>(ent_out)}) {
    if (o && T > 0 &&
        ranges_overlap(reinterpret_cast<uintptr_t>(logits), static_cast<size_t>(in_elems) * bi,
                       reinterpret_cast<uintptr_t>(o), static_cast<size_t>(T) * sizeof(float)))
      return CE_ERR_ALIAS;
  }
  // Workspace: segment arrays, pair-mode slots (gradient calls only), the
  // debug scan's words, in that order.
  const bool grad = grad_out != nullptr;
  const size_t need = segment_ws_bytes(p) + sched_ws_bytes(p, grad) + validate_ws_bytes(p);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return CE_ERR_WORKSPACE;
  if (need > 0 && (reinterpret_cast<uintptr_t>(workspace) % 4) != 0) return CE_ERR_WORKSPACE;

  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  const int32_t S = p->num_segments;
  if ((p->flags & CE_FLAG_VALIDATE) && T > 0) {
    // Scan, wait, and refuse before anything else is enqueued.
    uint32_t* words = reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + segment_ws_bytes(p) +
                                                  sched_ws_bytes(p, grad));
    const int64_t nb = std::min<int64_t>(kValidateBlocks, (T + 255) / 256);
    (void)hipGetLastError();
    hipLaunchKernelGGL(ce_validate_kernel, dim3(static_cast<unsigned>(nb)), dim3(256), 0, stream,
                       targets, T, V, p->ignore_index, segment_ids, S, words);
    if (hipGetLastError() != hipSuccess) return CE_ERR_HIP;
    uint32_t host[kValidateBlocks];
    if (hipMemcpyAsync(host, words, static_cast<size_t>(nb) * sizeof(uint32_t),
                       hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
      return CE_ERR_HIP;
    uint32_t bad = 0;
    for (int64_t i = 0; i < nb; ++i) bad |= host[i];
    if (bad != 0) return CE_ERR_INVALID_ARG;
  }
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

  const uint32_t* gave_up = nullptr;   // pair mode's give-up count, when it runs
  if (T > 0) {
    RowParams rp{};
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
    rp.lse_out = lse_out;
    rp.ent_out = ent_out;
    const bool vec_in = (reinterpret_cast<uintptr_t>(logits) % 16 == 0) &&
                        ((p->ld_logits * bi) % 16 == 0);
    const bool vec_out = !grad_out || ((reinterpret_cast<uintptr_t>(grad_out) % 16 == 0) &&
                                       ((p->ld_grad * bo) % 16 == 0));
    const bool vec = vec_in && vec_out;
    if (grad_out && sched_ws_bytes(p) > 0) {
      uint32_t* sched = reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + segment_ws_bytes(p));
      if (pair_rows(p)) {
        // pair_part is set exactly when the pair kernel runs (aligned rows)
        if (vec && !ent_out) {
          rp.pair_part = sched;
          rp.pair_split = (V / 4 / 2) * 4;   // a chunk boundary
          rp.tickets = sched + 8 * T;
          rp.pair_spin = pair_spin_limit();
          gave_up = rp.tickets + 1;
        }
      } else {
        rp.tickets = sched;
      }
    }
    (void)hipGetLastError();
    ce_status st;
    if (ent_out)
      st = (p->logits_dtype == CE_DTYPE_F32) ? dispatch_forward<float, true>(rp, vec, stream)
                                             : dispatch_forward<bf16_t, true>(rp, vec, stream);
    else
      st = (p->logits_dtype == CE_DTYPE_F32)
               ? dispatch_out<float>(rp, p->grad_dtype, grad_out != nullptr, vec, stream)
               : dispatch_out<bf16_t>(rp, p->grad_dtype, grad_out != nullptr, vec, stream);
    if (st != CE_OK) return st;
  }

  if (seg_loss_out) {
    hipLaunchKernelGGL(ce_seg_sum_kernel, dim3(static_cast<unsigned>(S)), dim3(256), 0, stream,
                       nll_ws, seg_start, S, seg_loss_out);
    if (hipGetLastError() != hipSuccess) return CE_ERR_HIP;
  }
  if ((p->flags & CE_FLAG_VALIDATE) && gave_up != nullptr) {
    // Two-workgroup rows: wait, and report half rows that gave up on their
    // partner (the count word starts at all-ones).
    uint32_t host = 0;
    if (hipMemcpyAsync(&host, gave_up, sizeof(host), hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
      return CE_ERR_HIP;
    if (host != ~0u) return CE_ERR_TIMEOUT;
  }
  return CE_OK;
}

}  // namespace

// Scratch of the allocation-free entry point: the workspace of
// ce_fused_fwd_bwd (segment staging and offsets, pair-mode exchange slots,
// the debug scan's words) in a fixed device array, one per GPU, held until
// the process ends. In host code `scratch` names a host-side stand-in: the
// device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[CE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// The device address of this device's `scratch` (dev must be current).
ce_status scratch_address(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return CE_ERR_UNSUPPORTED;
  void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (ptr == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    ptr = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (ptr == nullptr) {
      if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
        (void)hipGetLastError();
        return CE_ERR_HIP;
      }
      g_scratch_ptr[dev].store(ptr, std::memory_order_release);
    }
  }
  *out = ptr;
  return CE_OK;
}

}  // namespace

extern "C" {

ce_status ce_fused_fwd_bwd_noalloc(const ce_problem* p, const void* logits,
                                   const int64_t* targets, const uint8_t* mask,
                                   const int32_t* segment_ids, float z_alpha, float grad_scale,
                                   float* loss_out, float* seg_loss_out, void* grad_out,
                                   float* lse_out, void* stream_ptr) {
  if (p == nullptr || p->T < 0 || p->num_segments < 0) return CE_ERR_INVALID_ARG;
  // What ce_fused_fwd_bwd would ask of a workspace, against the fixed size.
  const size_t need = segment_ws_bytes(p) + sched_ws_bytes(p, grad_out != nullptr) +
                      validate_ws_bytes(p);
  if (need > CE_NOALLOC_SCRATCH_BYTES) return CE_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0) {
    // The scratch of the stream's device, which must be the current one
    // (the symbol's address is looked up with that device current).
    hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
    int cur = -1;
    hipDevice_t sdev = -1;
    if (hipGetDevice(&cur) != hipSuccess || hipStreamGetDevice(stream, &sdev) != hipSuccess) {
      (void)hipGetLastError();
      return CE_ERR_HIP;
    }
    if (static_cast<int>(sdev) != cur) return CE_ERR_INVALID_ARG;
    const ce_status st = scratch_address(cur, &ws);
    if (st != CE_OK) return st;
  }
  return run_rows(p, logits, targets, mask, segment_ids, z_alpha, grad_scale, loss_out,
                  seg_loss_out, grad_out, lse_out, nullptr, ws, need > 0 ? CE_NOALLOC_SCRATCH_BYTES : 0,
                  stream_ptr);
}

size_t ce_workspace_bytes(const ce_problem* p) {
  if (p == nullptr || p->T < 0 || p->num_segments < 0) return 0;
  return segment_ws_bytes(p) + sched_ws_bytes(p) + validate_ws_bytes(p);
}

const char* ce_status_string(int status) {
  switch (status) {
    case CE_OK: return "CE_OK";
    case CE_ERR_INVALID_ARG: return "CE_ERR_INVALID_ARG";
    case CE_ERR_UNSUPPORTED: return "CE_ERR_UNSUPPORTED";
    case CE_ERR_ALIAS: return "CE_ERR_ALIAS";
    case CE_ERR_WORKSPACE: return "CE_ERR_WORKSPACE";
    case CE_ERR_HIP: return "CE_ERR_HIP";
    case CE_ERR_TIMEOUT: return "CE_ERR_TIMEOUT";
    default: return "CE_ERR_UNKNOWN";
  }
}

ce_status ce_fused_fwd_bwd(const ce_problem* p, const void* logits, const int64_t* targets,
                           const uint8_t* mask, const int32_t* segment_ids, float z_alpha,
                           float grad_scale, float* loss_out, float* seg_loss_out,
                           void* grad_out, float* lse_out, void* workspace,
                           size_t workspace_bytes, void* stream_ptr) {
  return run_rows(p, logits, targets, mask, segment_ids, z_alpha, grad_scale, loss_out,
                  seg_loss_out, grad_out, lse_out, nullptr, workspace, workspace_bytes,
                  stream_ptr);
}

ce_status ce_fused_forward(const ce_problem* p, const void* logits, const int64_t* targets,
                           const uint8_t* mask, const int32_t* segment_ids, float z_alpha,
                           float* loss_out, float* seg_loss_out, float* lse_out,
                           float* entropy_out, void* workspace, size_t workspace_bytes,
                           void* stream_ptr) {
  return run_rows(p, logits, targets, mask, segment_ids, z_alpha, 1.0f, loss_out, seg_loss_out,
                  nullptr, lse_out, entropy_out, workspace, workspace_bytes, stream_ptr);
}

ce_status ce_shard_stats(const ce_shard* sh, const void* logits, const int64_t* targets,
                         const uint8_t* mask, float* stats, void* stream_ptr) {
  size_t in_bytes = 0;
  const ce_status chk = check_shard(sh, &in_bytes);
  if (chk != CE_OK) return chk;
  if (sh->T == 0) return CE_OK;
  if (!logits || !targets || !stats) return CE_ERR_INVALID_ARG;
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  RowParams rp = shard_params(sh, logits, targets);
  rp.mask = mask;
  rp.stats = stats;
  const bool vec = rows_vec(logits, sh->ld_logits, dtype_bytes(sh->logits_dtype));
  (void)hipGetLastError();
  return sh->logits_dtype == CE_DTYPE_F32 ? dispatch_shard<float, kStats>(rp, vec, stream)
                                          : dispatch_shard<bf16_t, kStats>(rp, vec, stream);
}

ce_status ce_rows_finish(const ce_problem* p, int32_t num_shards, const float* stats,
                         const int64_t* targets, const uint8_t* mask, const int32_t* segment_ids,
                         float z_alpha, float* loss_out, float* seg_loss_out, float* row_state,
                         void* workspace, size_t workspace_bytes, void* stream_ptr) {
  if (p == nullptr) return CE_ERR_INVALID_ARG;
  const int64_t T = p->T;
  if (T < 0 || p->V < 1 || num_shards < 1) return CE_ERR_INVALID_ARG;
  if ((p->flags & ~CE_FLAG_SEGMENT_MEAN) != 0 || p->num_segments < 0) return CE_ERR_INVALID_ARG;
  if (T > 0 && (segment_ids != nullptr) != (p->num_segments > 0)) return CE_ERR_INVALID_ARG;
  if (T == 0 && segment_ids != nullptr && p->num_segments == 0) return CE_ERR_INVALID_ARG;
  if (seg_loss_out && p->num_segments == 0) return CE_ERR_INVALID_ARG;
  if ((p->flags & CE_FLAG_SEGMENT_MEAN) && p->num_segments == 0) return CE_ERR_INVALID_ARG;
  if (T > INT32_MAX) return CE_ERR_UNSUPPORTED;
  if (T > 0 && (!stats || !targets || !loss_out || !row_state)) return CE_ERR_INVALID_ARG;
  if (!std::isfinite(z_alpha)) return CE_ERR_INVALID_ARG;
  const size_t need = segment_ws_bytes(p);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return CE_ERR_WORKSPACE;
  if (need > 0 && (reinterpret_cast<uintptr_t>(workspace) % 4) != 0) return CE_ERR_WORKSPACE;

  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  const int32_t S = p->num_segments;
  float* nll_ws = nullptr;
  int32_t* seg_start = nullptr;
  if (S > 0) {
    const ce_status st = launch_seg_bounds(segment_ids, T, S, workspace, &nll_ws, &seg_start, stream);
    if (st != CE_OK) return st;
  }
  if (T > 0) {
    FinishParams f{};
    f.stats = stats;
    f.targets = targets;
    f.mask = mask;
    f.seg_ids = segment_ids;
    f.seg_start = seg_start;
    f.loss_out = loss_out;
    f.nll_ws = seg_loss_out ? nll_ws : nullptr;
    f.row_state = row_state;
    f.T = T;
    f.V = p->V;
    f.ignore_index = p->ignore_index;
    f.P = num_shards;
    f.num_segments = S;
    f.seg_mean = (p->flags & CE_FLAG_SEGMENT_MEAN) ? 1 : 0;
    f.z_alpha = z_alpha;
    (void)hipGetLastError();
    hipLaunchKernelGGL(ce_finish_kernel, dim3(static_cast<unsigned>((T + 255) / 256)), dim3(256), 0,
                       stream, f);
    if (hipGetLastError() != hipSuccess) return CE_ERR_HIP;
  }
  if (seg_loss_out) {
    hipLaunchKernelGGL(ce_seg_sum_kernel, dim3(static_cast<unsigned>(S)), dim3(256), 0, stream,
                       nll_ws, seg_start, S, seg_loss_out);
    if (hipGetLastError() != hipSuccess) return CE_ERR_HIP;
  }
  return CE_OK;
}

ce_status ce_shard_grad(const ce_shard* sh, const void* logits, const int64_t* targets,
                        const float* row_state, const float* row_weight, float grad_scale,
                        void* grad_out, void* stream_ptr) {
  size_t in_bytes = 0, out_bytes = 0;
  const ce_status chk = check_shard(sh, &in_bytes);
  if (chk != CE_OK) return chk;
  if (!valid_dtype(sh->grad_dtype) || sh->ld_grad < sh->V) return CE_ERR_INVALID_ARG;
  if (!span_bytes(sh->T, sh->V, sh->ld_grad, dtype_bytes(sh->grad_dtype), &out_bytes))
    return CE_ERR_INVALID_ARG;
  if (!std::isfinite(grad_scale)) return CE_ERR_INVALID_ARG;
  if (sh->T == 0) return CE_OK;
  if (!logits || !targets || !row_state || !grad_out) return CE_ERR_INVALID_ARG;
  const bool same = grad_out == logits && sh->grad_dtype == sh->logits_dtype &&
                    sh->ld_grad == sh->ld_logits;
  if (!same && ranges_overlap(reinterpret_cast<uintptr_t>(logits), in_bytes,
                              reinterpret_cast<uintptr_t>(grad_out), out_bytes))
    return CE_ERR_ALIAS;
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  RowParams rp = shard_params(sh, logits, targets);
  rp.grad = grad_out;
  rp.ld_out = sh->ld_grad;
  rp.row_state = row_state;
  rp.row_weight = row_weight;
  rp.grad_scale = grad_scale;
  const int bi = dtype_bytes(sh->logits_dtype), bo = dtype_bytes(sh->grad_dtype);
  const bool vec = rows_vec(logits, sh->ld_logits, bi) && rows_vec(grad_out, sh->ld_grad, bo);
  (void)hipGetLastError();
  if (sh->logits_dtype == CE_DTYPE_F32)
    return sh->grad_dtype == CE_DTYPE_F32 ? dispatch_shard<float, kGrad, float>(rp, vec, stream)
                                          : dispatch_shard<float, kGrad, bf16_t>(rp, vec, stream);
  return sh->grad_dtype == CE_DTYPE_F32 ? dispatch_shard<bf16_t, kGrad, float>(rp, vec, stream)
                                        : dispatch_shard<bf16_t, kGrad, bf16_t>(rp, vec, stream);
}

}  // extern "C"
