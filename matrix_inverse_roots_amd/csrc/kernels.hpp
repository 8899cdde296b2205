// Bandwidth-bound kernels of the preconditioner step (gfx950, wave64).
//
// pack/unpack   parameter layout <-> zero-padded [nblk, B, B] block stacks
//               ([DASH] "4. Blocking Strategy"), with an LDS tile transpose
//               for the transposed stack the right-factor products read.
// frob_*        s = ||A + eps I||_F over each matrix's valid region
//               ([DASH] "3. Inverse Root Methods", Matrix scaling).
// prep          A_s = (A + eps I)/s with the padding set to the identity (or
//               to zero for the power iteration), and up to three affine
//               images alpha A_s + gamma I that seed the solver chains.
// comb          linear combinations of chain values (the Chebyshev series
//               split into baby and giant steps).
// power_iter_fused  half-precision multi-start power iteration on the Frobenius
//               scaled matrix, largest Rayleigh quotient ([DASH] "3. Inverse
//               Root Methods", Power-Iteration).
// finalize      out = X s^(-1/p) on the valid region, 0 on the padding,
//               non-finite flags.
// graft_*       layer-wise (or block-wise) grafting norms and the weight
//               update ([3DS] "Hyperparameters"; [DASH] "2. Preliminaries on
//               Shampoo").
//
// All reductions run in a fixed order inside one workgroup (no float
// atomics), so repeated calls give identical bits.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm.hpp"
#include "shampoo.h"

namespace shampoo {

// ---------------------------------------------------------------------------
// reductions
// ---------------------------------------------------------------------------
template <typename T> __device__ __forceinline__ T wave_sum(T x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// Sum over a 256-thread workgroup; every thread gets the result.
template <typename T> __device__ __forceinline__ T block_sum256(T x, T* red /* [4] */) {
  x = wave_sum(x);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = x;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// ---------------------------------------------------------------------------
// pack / unpack: 64 x 64 element tiles, 256 threads
// ---------------------------------------------------------------------------
__device__ __forceinline__ const void* desc_data(const shampoo_matrix& m) { return m.data; }
__device__ __forceinline__ const void* desc_data(const shampoo_param& p) { return p.g; }

// E: raw element type of the right width (the copy is bit-exact).
// Desc: shampoo_matrix (data) or shampoo_param (gradient g).  The vector
// path reads the parameter and writes both stacks with non-temporal
// accesses (each byte is touched once here): 5% faster on the decoder step.
template <typename E, typename Desc>
__global__ __launch_bounds__(256) void pack_kernel(const Desc* __restrict__ descs, int nparams,
                                                   const shampoo_block* __restrict__ table, int B,
                                                   int tiles_per_side, E* __restrict__ stack,
                                                   E* __restrict__ stack_t) {
  constexpr int VE = 16 / (int)sizeof(E);  // elements per 16-byte access
  constexpr int CPR = 64 / VE;             // 16-byte chunks per tile row
  constexpr int RPP = 256 / CPR;           // tile rows per pass
  __shared__ __attribute__((aligned(16))) E tile[64][64 + VE];
  const int64_t b = blockIdx.y;
  const int tt = blockIdx.x;
  const int tr = tt / tiles_per_side, tc = tt - tr * tiles_per_side;
  const shampoo_block blk = table[b];
  if (blk.param < 0 || blk.param >= nparams) return;  // uniform per workgroup
  const Desc m = descs[blk.param];
  const E* src = reinterpret_cast<const E*>(desc_data(m));
  const int64_t BB = (int64_t)B * B;
  if (B % 64 != 0 || ((reinterpret_cast<uintptr_t>(stack) | reinterpret_cast<uintptr_t>(stack_t)) & 15) != 0) {
    // general sides: element-wise copy with bounds checks (uniform branch)
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    for (int rr = ty; rr < 64; rr += 4) {
      const int r = tr * 64 + rr, c = tc * 64 + tx;
      E v = E(0);
      if (r < blk.rows && c < blk.cols) v = src[(int64_t)(blk.row0 + r) * m.ld + blk.col0 + c];
      if (r < B && c < B) stack[b * BB + (int64_t)r * B + c] = v;
      tile[rr][tx] = v;
    }
    if (!stack_t) return;
    __syncthreads();
    for (int cc2 = ty; cc2 < 64; cc2 += 4) {
      const int c = tc * 64 + cc2, r = tr * 64 + tx;
      if (r < B && c < B) stack_t[b * BB + (int64_t)c * B + r] = tile[tx][cc2];
    }
    return;
  }
  // 16-byte source access needs 16-byte aligned rows (uniform per workgroup)
  const bool vec = ((reinterpret_cast<uintptr_t>(src) | ((uintptr_t)m.ld * sizeof(E)) |
                     ((uintptr_t)blk.col0 * sizeof(E))) & 15) == 0;
  const int cc = (int)threadIdx.x % CPR, rq = (int)threadIdx.x / CPR;
#pragma unroll
  for (int pass = 0; pass < 64 / RPP; ++pass) {
    const int rr = pass * RPP + rq, r = tr * 64 + rr, c = tc * 64 + cc * VE;
    E v[VE];
    const E* sp = src + (int64_t)(blk.row0 + r) * m.ld + blk.col0 + c;
    if (vec && r < blk.rows && c + VE <= blk.cols) {
      *reinterpret_cast<u32x4*>(v) = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(sp));
    } else {
#pragma unroll
      for (int e = 0; e < VE; ++e) v[e] = (r < blk.rows && c + e < blk.cols) ? sp[e] : E(0);
    }
    __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(v), reinterpret_cast<u32x4*>(stack + b * BB + (int64_t)r * B + c));
    *reinterpret_cast<uint4*>(&tile[rr][cc * VE]) = *reinterpret_cast<const uint4*>(v);
  }
  if (!stack_t) return;
  __syncthreads();
  // transposed tile: output row (column c of the block), VE consecutive r
#pragma unroll
  for (int pass = 0; pass < 64 / RPP; ++pass) {
    const int ccol = pass * RPP + rq, c = tc * 64 + ccol, r0 = tr * 64 + cc * VE;
    E v[VE];
#pragma unroll
    for (int e = 0; e < VE; ++e) v[e] = tile[cc * VE + e][ccol];
    __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(v), reinterpret_cast<u32x4*>(stack_t + b * BB + (int64_t)c * B + r0));
  }
}

__global__ __launch_bounds__(256) void unpack_kernel(const float* __restrict__ stack,
                                                     const shampoo_block* __restrict__ table, int B,
                                                     int tiles_per_side,
                                                     const shampoo_matrix* __restrict__ mats, int nparams) {
  const int64_t b = blockIdx.y;
  const int tt = blockIdx.x;
  const int tr = tt / tiles_per_side, tc = tt - tr * tiles_per_side;
  const shampoo_block blk = table[b];
  if (blk.param < 0 || blk.param >= nparams) return;
  const shampoo_matrix m = mats[blk.param];
  float* dst = reinterpret_cast<float*>(m.data);
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int rr = ty; rr < 64; rr += 4) {
    const int r = tr * 64 + rr, c = tc * 64 + tx;
    if (r < blk.rows && c < blk.cols)
      dst[(int64_t)(blk.row0 + r) * m.ld + blk.col0 + c] = stack[b * (int64_t)B * B + (int64_t)r * B + c];
  }
}

__global__ void valid_from_table_kernel(const shampoo_block* __restrict__ table, int64_t nblk,
                                        int32_t* __restrict__ valid) {
  const int64_t b = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (b >= nblk) return;
  valid[b] = table[b].rows;
  valid[nblk + b] = table[b].cols;
}

// ---------------------------------------------------------------------------
// Four consecutive elements (16-byte aligned) as doubles, and back.
// ---------------------------------------------------------------------------
// load_nt: non-temporal load, for data a kernel reads exactly once (the
// Frobenius sums, the power iteration's first pass): 15% and 3% faster on
// the decoder step and the solve.  Kernels that read a value twice
// (finalize's mirror tile) or whose outputs are read right away (prep) are
// faster with ordinary accesses.
template <typename T> struct Quad;
template <> struct Quad<float> {
  static __device__ __forceinline__ void load(const float* p, double* o) {
    const floatx4 t = *reinterpret_cast<const floatx4*>(p);
    o[0] = t[0]; o[1] = t[1]; o[2] = t[2]; o[3] = t[3];
  }
  static __device__ __forceinline__ void load_nt(const float* p, double* o) {
    const floatx4 t = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(p));
    o[0] = t[0]; o[1] = t[1]; o[2] = t[2]; o[3] = t[3];
  }
  static __device__ __forceinline__ void store(float* p, const double* v) {
    *reinterpret_cast<floatx4*>(p) = floatx4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
  }
};
template <> struct Quad<_Float16> {
  static __device__ __forceinline__ void load(const _Float16* p, double* o) {
    const halfx4 t = *reinterpret_cast<const halfx4*>(p);
    o[0] = (double)t[0]; o[1] = (double)t[1]; o[2] = (double)t[2]; o[3] = (double)t[3];
  }
  static __device__ __forceinline__ void load_nt(const _Float16* p, double* o) {
    const halfx4 t = __builtin_nontemporal_load(reinterpret_cast<const halfx4*>(p));
    o[0] = (double)t[0]; o[1] = (double)t[1]; o[2] = (double)t[2]; o[3] = (double)t[3];
  }
};
template <> struct Quad<double> {
  static __device__ __forceinline__ void load(const double* p, double* o) {
    const doublex2 t0 = *reinterpret_cast<const doublex2*>(p), t1 = *reinterpret_cast<const doublex2*>(p + 2);
    o[0] = t0[0]; o[1] = t0[1]; o[2] = t1[0]; o[3] = t1[1];
  }
  static __device__ __forceinline__ void load_nt(const double* p, double* o) {
    const doublex2 t0 = __builtin_nontemporal_load(reinterpret_cast<const doublex2*>(p));
    const doublex2 t1 = __builtin_nontemporal_load(reinterpret_cast<const doublex2*>(p + 2));
    o[0] = t0[0]; o[1] = t0[1]; o[2] = t1[0]; o[3] = t1[1];
  }
  static __device__ __forceinline__ void store(double* p, const double* v) {
    *reinterpret_cast<doublex2*>(p) = doublex2{v[0], v[1]};
    *reinterpret_cast<doublex2*>(p + 2) = doublex2{v[2], v[3]};
  }
};

// ---------------------------------------------------------------------------
// Frobenius norm of A + eps I over the valid region, in two passes.
// frob_partial: grid (P, n).  The valid region is read as rows of ceil(v/4)
// four-element chunks; part p of matrix b sums the chunks
// [p total / P, (p + 1) total / P) of that sequence, chunk k going to thread
// k % 256, 4 chunks in flight per thread.  frob_finish adds the P partial
// sums of each matrix in order.  The summation order thus depends on the
// valid side v and on P (a function of the batch size) alone: a padded and
// an unpadded stack give the same bits.
// ---------------------------------------------------------------------------
template <typename TI>
__global__ __launch_bounds__(256) void frob_partial_kernel(const TI* __restrict__ in, int B,
                                                           const int32_t* __restrict__ valid, double eps,
                                                           int P, double* __restrict__ part) {
  constexpr int U = 4;  // chunks in flight per thread (more costs occupancy)
  __shared__ double red[4];
  const int p = blockIdx.x;
  const int64_t b = blockIdx.y;
  const int v = valid ? min(max(valid[b], 0), B) : B;
  const TI* A = in + b * (int64_t)B * B;
  const int cv = (v + 3) / 4;
  // row of chunk k: floor(k / cv) through a double reciprocal (exact: the
  // quotient's distance to an integer, >= 0.5 / cv, dwarfs the rounding)
  const double icv = 1.0 / (double)max(cv, 1);
  const int64_t total = (int64_t)v * cv;
  const int k0 = (int)(total * p / P), k1 = (int)(total * (p + 1) / P);
  // one accumulator per element position: four independent chains, added in
  // a fixed order at the end
  double acc[4] = {0.0, 0.0, 0.0, 0.0};
  for (int base = k0; base < k1; base += 256 * U) {
    double x[U][4];
    int rr[U], cc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = base + u * 256 + (int)threadIdx.x;
      rr[u] = (int)(((double)k + 0.5) * icv);
      cc[u] = 4 * (k - rr[u] * cv);
      if (k < k1) Quad<TI>::load_nt(A + (int64_t)rr[u] * B + cc[u], x[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (base + u * 256 + (int)threadIdx.x >= k1) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (cc[u] + e >= v) continue;
        double y = x[u][e];
        if (rr[u] == cc[u] + e) y += eps;
        acc[e] += y * y;
      }
    }
  }
  double t = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  t = block_sum256(t, red);
  if (threadIdx.x == 0) part[b * P + p] = t;
}

__global__ __launch_bounds__(256) void frob_finish_kernel(const double* __restrict__ part, int P, int64_t n,
                                                          double* __restrict__ s_out) {
  const int64_t b = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (b >= n) return;
  double acc = 0.0;
  for (int p = 0; p < P; ++p) acc += part[b * P + p];
  s_out[b] = sqrt(acc);
}

// ---------------------------------------------------------------------------
// prep: a = (A + eps I)/s on the valid region, delta_ij * pad_diag elsewhere;
// out_q = alpha_q a + gamma_q I for up to three outputs.  Grid (chunks, n):
// each thread maps PREP_U four-element chunks of one matrix.
// ---------------------------------------------------------------------------
struct PrepOut {
  void* p;   // output in the iterate type (may be null)
  double alpha, gamma;
  void* ph;  // half copy, rounded through float32 (half operands only; may be null)
};
constexpr int PREP_U = 4;

template <typename TI, typename TS>
__global__ __launch_bounds__(256) void prep_kernel(const TI* __restrict__ in, int B, int64_t nmat,
                                                   const int32_t* __restrict__ valid, double eps,
                                                   const double* __restrict__ s, double pad_diag,
                                                   PrepOut o0, PrepOut o1, PrepOut o2) {
  const int64_t b = blockIdx.y;
  const int64_t BB = (int64_t)B * B;
  const int cpr = B / 4;  // chunks per row
  const int v = valid ? min(max(valid[b], 0), B) : B;
  const double sb = s[b];
  const double inv = (sb > 0.0 && sb < 1.0e300) ? 1.0 / sb : 0.0;
  const TI* A = in + b * BB;
  TS* out[3] = {o0.p ? reinterpret_cast<TS*>(o0.p) + b * BB : nullptr,
                o1.p ? reinterpret_cast<TS*>(o1.p) + b * BB : nullptr,
                o2.p ? reinterpret_cast<TS*>(o2.p) + b * BB : nullptr};
  _Float16* outh[3] = {o0.ph ? reinterpret_cast<_Float16*>(o0.ph) + b * BB : nullptr,
                       o1.ph ? reinterpret_cast<_Float16*>(o1.ph) + b * BB : nullptr,
                       o2.ph ? reinterpret_cast<_Float16*>(o2.ph) + b * BB : nullptr};
  const double al[3] = {o0.alpha, o1.alpha, o2.alpha}, ga[3] = {o0.gamma, o1.gamma, o2.gamma};
  const int total = B * cpr;
  double x[PREP_U][4];
  int rr[PREP_U], cc[PREP_U];
#pragma unroll
  for (int u = 0; u < PREP_U; ++u) {
    const int k = ((int)blockIdx.x * PREP_U + u) * 256 + (int)threadIdx.x;
    rr[u] = k / cpr;
    cc[u] = 4 * (k - rr[u] * cpr);
    if (k < total && rr[u] < v && cc[u] < v) Quad<TI>::load(A + (int64_t)rr[u] * B + cc[u], x[u]);
  }
#pragma unroll
  for (int u = 0; u < PREP_U; ++u) {
    const int k = ((int)blockIdx.x * PREP_U + u) * 256 + (int)threadIdx.x;
    if (k >= total) continue;
    double a[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = rr[u], c = cc[u] + e;
      if (r < v && c < v) {
        a[e] = x[u][e];
        if (r == c) a[e] += eps;
        a[e] *= inv;
      } else {
        a[e] = (r == c) ? pad_diag : 0.0;
      }
    }
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      if (!out[q] && !outh[q]) continue;
      double y[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] = al[q] * a[e] + ga[q] * (rr[u] == cc[u] + e ? 1.0 : 0.0);
      if (out[q]) Quad<TS>::store(out[q] + (int64_t)rr[u] * B + cc[u], y);
      if (outh[q])
        store_h4(outh[q] + (int64_t)rr[u] * B + cc[u], floatx4{(float)y[0], (float)y[1], (float)y[2], (float)y[3]});
    }
  }
}

// ---------------------------------------------------------------------------
// comb: out = sum_q w_q in_q + gamma I over whole matrices, evaluated in
// double and rounded once (as the product epilogue).  The padding is
// included: every chain value is a polynomial in A_s, whose padding is the
// identity, so its padding holds that polynomial's value at 1 and a linear
// combination keeps it so.  An input may be `out` itself (each element is
// read before it is written, by the same thread).  Grid (chunks, n) as prep.
// ---------------------------------------------------------------------------
constexpr int COMB_IN = 4;
struct CombArgs {
  const void* in[COMB_IN];  // the first nin are used
  double w[COMB_IN];
  int nin;
  double gamma;
  void* out;   // iterate type (may be null)
  void* outh;  // half copy (half operands only; may be null)
};

template <typename TS>
__global__ __launch_bounds__(256) void comb_kernel(CombArgs a, int B) {
  const int64_t b = blockIdx.y;
  const int64_t BB = (int64_t)B * B;
  const int cpr = B / 4;
  const int total = B * cpr;
  TS* out = a.out ? reinterpret_cast<TS*>(a.out) + b * BB : nullptr;
  _Float16* outh = a.outh ? reinterpret_cast<_Float16*>(a.outh) + b * BB : nullptr;
  // All loads of the thread's chunks come before any store: an input may be
  // `out` itself, so loads placed after a store could not be moved ahead of
  // it, and the chunks would be read one at a time.
  double y[PREP_U][4];
#pragma unroll
  for (int u = 0; u < PREP_U; ++u) {
    const int k = ((int)blockIdx.x * PREP_U + u) * 256 + (int)threadIdx.x;
    const int r = k / cpr, c = 4 * (k - r * cpr);
    const int64_t off = b * BB + (int64_t)r * B + c;
#pragma unroll
    for (int e = 0; e < 4; ++e) y[u][e] = (r == c + e) ? a.gamma : 0.0;
    if (k >= total) continue;
#pragma unroll
    for (int q = 0; q < COMB_IN; ++q) {
      if (q < a.nin) {
        double x[4];
        Quad<TS>::load(reinterpret_cast<const TS*>(a.in[q]) + off, x);
#pragma unroll
        for (int e = 0; e < 4; ++e) y[u][e] += a.w[q] * x[e];
      }
    }
  }
#pragma unroll
  for (int u = 0; u < PREP_U; ++u) {
    const int k = ((int)blockIdx.x * PREP_U + u) * 256 + (int)threadIdx.x;
    if (k >= total) continue;
    const int r = k / cpr, c = 4 * (k - r * cpr);
    if (out) Quad<TS>::store(out + (int64_t)r * B + c, y[u]);
    if (outh) store_h4(outh + (int64_t)r * B + c, floatx4{(float)y[u][0], (float)y[u][1], (float)y[u][2], (float)y[u][3]});
  }
}

// ---------------------------------------------------------------------------
// mcomb: several linear combinations of the same inputs in one pass,
// out_j = sum_q w[j][q] in_q + gamma_j I: every input is read once.  Same
// arithmetic as comb (double, one rounding), grid (chunks, n) as prep.
// ---------------------------------------------------------------------------
constexpr int MCOMB_IN = 12, MCOMB_OUT = 12;
struct MCombArgs {
  const void* in[MCOMB_IN];
  void* out[MCOMB_OUT];   // iterate type (may be null)
  void* outh[MCOMB_OUT];  // half copies (half operands only; may be null)
  double w[MCOMB_OUT][MCOMB_IN];
  double gamma[MCOMB_OUT];
  int nin, nout;
};

template <typename TS>
__global__ __launch_bounds__(256) void mcomb_kernel(MCombArgs a, int B) {
  const int64_t b = blockIdx.y;
  const int64_t BB = (int64_t)B * B;
  const int cpr = B / 4;
  const int total = B * cpr;
  const int k = (int)blockIdx.x * 256 + (int)threadIdx.x;
  if (k >= total) return;
  const int r = k / cpr, c = 4 * (k - r * cpr);
  const int64_t off = b * BB + (int64_t)r * B + c;
  // predicated, fully unrolled loops: every array index is a constant, so
  // the inputs stay in registers
  double x[MCOMB_IN][4];
#pragma unroll
  for (int q = 0; q < MCOMB_IN; ++q) {
    if (q < a.nin) {
      Quad<TS>::load(reinterpret_cast<const TS*>(a.in[q]) + off, x[q]);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) x[q][e] = 0.0;
    }
  }
#pragma unroll
  for (int j = 0; j < MCOMB_OUT; ++j) {
    if (j < a.nout) {
      double y[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] = (r == c + e) ? a.gamma[j] : 0.0;
#pragma unroll
      for (int q = 0; q < MCOMB_IN; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] += a.w[j][q] * x[q][e];
      if (a.out[j]) Quad<TS>::store(reinterpret_cast<TS*>(a.out[j]) + off, y);
      if (a.outh[j])
        store_h4(reinterpret_cast<_Float16*>(a.outh[j]) + off, floatx4{(float)y[0], (float)y[1], (float)y[2], (float)y[3]});
    }
  }
}

// ---------------------------------------------------------------------------
// Convergence check of the Newton iterations: ||M - I||_F per matrix comes
// from the Frobenius kernels with eps = -1; a matrix above tol sets
// *notdone.  The Frobenius norm bounds every eigenvalue's distance from 1.
// Matrices that cannot converge do not hold the others back: a NaN norm, or
// a scale that is zero or not finite (the final pass zeroes and flags them).
// ---------------------------------------------------------------------------
__global__ void above_tol_kernel(const double* __restrict__ norms, const double* __restrict__ scale, int64_t n,
                                 double tol, int32_t* __restrict__ notdone) {
  const int64_t b = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (b < n && scale[b] > 0.0 && scale[b] < 1.0e300 && norms[b] > tol) atomicOr(notdone, 1);
}

// A necessary condition read from the diagonal alone, one workgroup per
// matrix: ||M - I||_F >= |tr(M) - v| / sqrt(v) (Cauchy-Schwarz on the v
// diagonal entries of M - I).  A matrix whose trace puts it beyond tol
// (with a 1e-12 relative margin over the rounding of the two double sums)
// is not converged whatever its other entries, and the Frobenius pass that
// would say so too is skipped; NaN traces and unusable scales decide
// nothing, as above.
template <typename T>
__global__ __launch_bounds__(256) void trace_gap_kernel(const T* __restrict__ in, int B,
                                                        const int32_t* __restrict__ valid,
                                                        const double* __restrict__ scale, double tol,
                                                        int32_t* __restrict__ notdone) {
  __shared__ double red[4];
  const int64_t b = blockIdx.x;
  const int v = valid ? min(max(valid[b], 0), B) : B;
  const T* M = in + b * (int64_t)B * B;
  double t = 0.0;
  for (int i = (int)threadIdx.x; i < v; i += 256) t += (double)M[(int64_t)i * B + i] - 1.0;
  t = block_sum256(t, red);
  if (threadIdx.x == 0 && v > 0 && scale[b] > 0.0 && scale[b] < 1.0e300 &&
      fabs(t) / sqrt((double)v) > tol * (1.0 + 1e-12))
    atomicOr(notdone, 1);
}

// ---------------------------------------------------------------------------
// Solver residual ||X^p A_s - I||_F / sqrt(v) per matrix, from the Frobenius
// norm of the product X^p A_s - I over the valid region (frob kernels with
// eps = 0).  A matrix whose residual exceeds `bound` (> 0), or is not
// finite, is flagged RESIDUAL unless its scale is zero or not finite (its
// root is then set to 0 and flagged ZERO_SCALE by the final pass).
// ---------------------------------------------------------------------------
__global__ void residual_kernel(const double* __restrict__ norms, const double* __restrict__ scale,
                                const int32_t* __restrict__ valid, int64_t n, int B, double bound,
                                float* __restrict__ out, int32_t* __restrict__ flags) {
  const int64_t b = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (b >= n) return;
  const int v = valid ? min(max(valid[b], 0), B) : B;
  const double r = v > 0 ? norms[b] / sqrt((double)v) : 0.0;
  if (out) out[b] = (float)r;
  const bool scaled = scale[b] > 0.0 && scale[b] < 1.0e300;
  if (flags && bound > 0.0 && scaled && !(r <= bound)) atomicOr(flags + b, SHAMPOO_FLAG_RESIDUAL);
}

// A root computed but not to be committed: not finite, zero scale, or a
// residual above the bound.
constexpr int32_t FAILED_ROOT = SHAMPOO_FLAG_NONFINITE | SHAMPOO_FLAG_ZERO_SCALE | SHAMPOO_FLAG_RESIDUAL;

// ---------------------------------------------------------------------------
// Multi-start power iteration ([DASH] "3. Inverse Root Methods",
// Power-Iteration), fused with its scaling and persistent over the matrices.
// Workgroup w (4 waves) takes matrices w, w + gridDim.x, ...  For each, on
// A_s = (in + eps I)/s_F (valid region; zero padding) rounded to half:
// `iters` rounds normalise the k vectors and multiply by A_s with
// half-precision operands and float32 accumulation (MFMA 16x16x32 f16); a
// final product gives the Rayleigh quotients of the last normalised vectors;
// s_out[b] = sf[b] * max_j rq_j (lowest j on ties), or sf[b] with
// PI_FALLBACK when no quotient is positive and finite.
// Pass 0 computes A_s from `in` (in double, rounded once to half)
// and stores the half matrix in `hcopy`; later passes read that copy, half
// the bytes of a float32 matrix.  Each lane reads back exactly the 16 bytes
// it wrote.  Workgroups of PI_THREADS (16 waves): a matrix's passes are
// streams of its half copy through L2, bound by the loads each workgroup
// keeps in flight, so a workgroup holds as many waves as a CU takes; a
// row block of 16 rows and a vector's norm are each one wave's work, the
// same instructions whichever wave runs them (the result does not depend
// on the number of waves).
// Dynamic LDS: Vh half [k16][B + 8], Wf float [k16][B + 4], k16 floats.
// ---------------------------------------------------------------------------
constexpr int PI_THREADS = 1024;
template <typename TI, int NVB>
__global__ __launch_bounds__(PI_THREADS) void power_iter_fused_kernel(const TI* __restrict__ in, int B, int64_t n,
                                                               const int32_t* __restrict__ valid, double eps,
                                                               const double* __restrict__ sf, int k, int iters,
                                                               const float* __restrict__ v0,
                                                               _Float16* __restrict__ hcopy,
                                                               double* __restrict__ s_out,
                                                               int32_t* __restrict__ flags) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  constexpr int k16 = NVB * 16;
  const int VP = B + 8;
  const int WP = B + 4;
  _Float16* Vh = reinterpret_cast<_Float16*>(smem);
  float* Wf = reinterpret_cast<float*>(smem + (size_t)k16 * VP * 2);
  float* rq = Wf + (size_t)k16 * WP;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nw = (int)(blockDim.x >> 6);
  const int i16 = lane & 15, grp = lane >> 4;
  for (int64_t b = blockIdx.x; b < n; b += gridDim.x) {
    const TI* A = in + b * (int64_t)B * B;
    _Float16* H = hcopy + b * (int64_t)B * B;
    const int v = valid ? min(max(valid[b], 0), B) : B;
    const double sfb = sf[b];
    const double inv = (sfb > 0.0 && sfb < 1.0e300) ? 1.0 / sfb : 0.0;
    __syncthreads();  // the previous matrix's last reads of Wf / Vh are done
    for (int e = tid; e < k16 * B; e += (int)blockDim.x) {
      const int vv = e / B, i = e - vv * B;
      Wf[vv * WP + i] = vv < k ? v0[(int64_t)vv * B + i] : 0.0f;
    }
    for (int it = 0; it <= iters; ++it) {
      __syncthreads();
      for (int vv = wave; vv < k16; vv += nw) {
        float ss = 0.0f;
        for (int i = lane; i < B; i += 64) {
          const float x = Wf[vv * WP + i];
          ss += x * x;
        }
        ss = wave_sum(ss);
        const float nrm = sqrtf(ss);
        const float rn = nrm > 0.0f ? 1.0f / nrm : 1.0f;
        for (int i = lane; i < B; i += 64) Vh[vv * VP + i] = (_Float16)(Wf[vv * WP + i] * rn);
      }
      __syncthreads();
      for (int rb = wave; rb < B / 16; rb += nw) {
        floatx4 acc[NVB];
#pragma unroll
        for (int vb = 0; vb < NVB; ++vb) acc[vb] = floatx4{0.f, 0.f, 0.f, 0.f};
        const int row = rb * 16 + i16;
#pragma unroll 4
        for (int kk = 0; kk < B; kk += 32) {
          const int c0 = kk + 8 * grp;
          halfx8 a;
          if (it == 0) {
            double x[8];
#pragma unroll
            for (int q = 0; q < 8; q += 4) Quad<TI>::load_nt(A + (int64_t)row * B + c0 + q, x + q);
#pragma unroll
            for (int q = 0; q < 8; ++q) {
              const int c = c0 + q;
              double y = 0.0;
              if (row < v && c < v) {
                y = x[q];
                if (row == c) y += eps;
                y *= inv;
              }
              a[q] = (_Float16)y;  // one rounding, double -> half
            }
            *reinterpret_cast<halfx8*>(H + (int64_t)row * B + c0) = a;
          } else {
            a = *reinterpret_cast<const halfx8*>(H + (int64_t)row * B + c0);
          }
#pragma unroll
          for (int vb = 0; vb < NVB; ++vb) {
            const halfx8 bv = *reinterpret_cast<const halfx8*>(Vh + (vb * 16 + i16) * VP + kk + 8 * grp);
            acc[vb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bv, acc[vb], 0, 0, 0);
          }
        }
#pragma unroll
        for (int vb = 0; vb < NVB; ++vb)
#pragma unroll
          for (int q = 0; q < 4; ++q) Wf[(vb * 16 + i16) * WP + rb * 16 + 4 * grp + q] = acc[vb][q];
      }
    }
    __syncthreads();
    for (int vv = wave; vv < k16; vv += nw) {
      float num = 0.0f, den = 0.0f;
      for (int i = lane; i < B; i += 64) {
        const float x = (float)Vh[vv * VP + i];
        num += x * Wf[vv * WP + i];
        den += x * x;
      }
      num = wave_sum(num);
      den = wave_sum(den);
      if (lane == 0) rq[vv] = den > 0.0f ? num / den : 0.0f;
    }
    __syncthreads();
    if (tid == 0) {
      float best = rq[0];
      for (int vv = 1; vv < k; ++vv)
        if (rq[vv] > best) best = rq[vv];
      const bool ok = best > 0.0f && best < 3.0e38f;
      s_out[b] = ok ? sfb * (double)best : sfb;
      if (!ok && flags) atomicOr(flags + b, SHAMPOO_FLAG_PI_FALLBACK);
    }
  }
}

// ---------------------------------------------------------------------------
// finalize: out = X s^(-1/p) on the valid region, 0 elsewhere; with sym_out
// the symmetric part (X + X^T)/2 is taken first.  One workgroup per 64 x 64
// tile: the tile and its mirror are staged through LDS so that every global
// access is a coalesced row segment; one flag update per workgroup.
// ---------------------------------------------------------------------------
// mode FIN_WRITE: write and flag; FIN_CHECK: flag only (out unused);
// FIN_COMMIT: write only matrices whose flags show none of NONFINITE,
// ZERO_SCALE (set by a FIN_CHECK pass) and RESIDUAL, flags untouched.
enum { FIN_WRITE = 0, FIN_CHECK = 1, FIN_COMMIT = 2 };

template <typename TS, typename TO>
__global__ __launch_bounds__(256) void finalize_kernel(const TS* __restrict__ X, TO* __restrict__ out, int B,
                                                       const int32_t* __restrict__ valid,
                                                       const double* __restrict__ s, double inv_p,
                                                       int sym_out, float* __restrict__ scale_out,
                                                       int32_t* __restrict__ flags, int mode) {
  __shared__ TS mir_tile[64][65];
  const int tps = B / 64;
  const int64_t b = blockIdx.y;
  if (mode == FIN_COMMIT && (flags[b] & FAILED_ROOT)) return;  // uniform
  const int tr = blockIdx.x / tps, tc = blockIdx.x - (blockIdx.x / tps) * tps;
  const int64_t BB = (int64_t)B * B;
  const TS* Xb = X + b * BB;
  TO* ob = out + b * BB;
  const int v = valid ? min(max(valid[b], 0), B) : B;
  const double sb = s[b];
  const bool zero = !(sb > 0.0 && sb < 1.0e300);
  const double f = zero ? 0.0 : pow(sb, -inv_p);
  // thread: 4 consecutive columns (c4) of rows rg, rg + 16, rg + 32, rg + 48
  const int c4 = 4 * (threadIdx.x & 15), rg = threadIdx.x >> 4;
  if (sym_out) {
    // mirror tile (tc, tr): mir_tile[cc][rr] = X[tc*64 + cc][tr*64 + rr]
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int cc = rg + 16 * k;
      double t[4];
      Quad<TS>::load(Xb + (int64_t)(tc * 64 + cc) * B + tr * 64 + c4, t);
#pragma unroll
      for (int e = 0; e < 4; ++e) mir_tile[cc][c4 + e] = (TS)t[e];
    }
    __syncthreads();
  }
  int bad = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int rr = rg + 16 * k, r = tr * 64 + rr, c0 = tc * 64 + c4;
    double x[4] = {0.0, 0.0, 0.0, 0.0};
    if (r < v && c0 < v && !zero) {
      double t[4];
      Quad<TS>::load(Xb + (int64_t)r * B + c0, t);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (c0 + e >= v) continue;
        double y = t[e];
        if (sym_out) y = 0.5 * (y + (double)mir_tile[c4 + e][rr]);
        y *= f;
        if (!isfinite(y)) bad = 1;
        x[e] = y;
      }
    }
    if (mode != FIN_CHECK) Quad<TO>::store(ob + (int64_t)r * B + c0, x);
  }
  if (mode == FIN_COMMIT) return;
  bad = __syncthreads_or(bad);
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    if (flags && zero) atomicOr(flags + b, SHAMPOO_FLAG_ZERO_SCALE);
    if (scale_out) scale_out[b] = (float)sb;
  }
  if (threadIdx.x == 0 && bad && flags) atomicOr(flags + b, SHAMPOO_FLAG_NONFINITE);
}

// ---------------------------------------------------------------------------
// step fallback helpers
// ---------------------------------------------------------------------------
// float32 -> bfloat16, rounded to nearest even; n4 four-element chunks
// (16-byte aligned input, 8-byte aligned output), grid-stride.
__global__ __launch_bounds__(256) void f32_to_bf16_kernel(const float* __restrict__ in, __bf16* __restrict__ out,
                                                          int64_t n4) {
  typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
  for (int64_t i = blockIdx.x * (int64_t)256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
    const floatx4 v = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(in) + i);
    const bf16x4_t o = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
    __builtin_nontemporal_store(o, reinterpret_cast<bf16x4_t*>(out) + i);
  }
}

__global__ void fill_i32_kernel(int32_t* __restrict__ p, int64_t n, int32_t v) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// Factor order of the grouped roots: factor f < nblk is the L factor of block
// f (side: valid rows), f >= nblk the R factor of block f - nblk (valid
// columns), side = valid rounded up to 64.  gidx lists the factors by side,
// ascending, and by index within a side (a stable counting sort), the order
// the host plans its groups in.  One workgroup of 1024 threads: a histogram
// of the sides, then for each side that occurs a pass over the factors whose
// ballot prefix sums place them.  nbins = B / 64 <= GROUP_BINS.
constexpr int GROUP_BINS = 128;
__device__ __forceinline__ int factor_bin(const shampoo_block* table, int64_t nblk, int B, int64_t f) {
  const shampoo_block t = table[f < nblk ? f : f - nblk];
  const int v = min(max(f < nblk ? t.rows : t.cols, 1), B);
  return (v + 63) / 64 - 1;
}

__global__ __launch_bounds__(1024) void group_order_kernel(const shampoo_block* __restrict__ table, int64_t nblk,
                                                           int B, int32_t* __restrict__ gidx) {
  __shared__ int hist[GROUP_BINS];
  __shared__ int wsum[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t nf = 2 * nblk;
  const int nbins = B / 64;
  for (int i = tid; i < GROUP_BINS; i += 1024) hist[i] = 0;
  __syncthreads();
  for (int64_t f = tid; f < nf; f += 1024) atomicAdd(&hist[factor_bin(table, nblk, B, f)], 1);
  __syncthreads();
  int base = 0;
  for (int bin = 0; bin < nbins; ++bin) {
    if (hist[bin] == 0) continue;  // uniform: every thread reads the same count
    for (int64_t c0 = 0; c0 < nf; c0 += 1024) {
      const int64_t f = c0 + tid;
      const bool pred = f < nf && factor_bin(table, nblk, B, f) == bin;
      const unsigned long long m = __ballot(pred);
      const int within = __popcll(m & ((1ull << lane) - 1ull));
      if (lane == 0) wsum[wave] = __popcll(m);
      __syncthreads();
      int pre = 0, tot = 0;
#pragma unroll
      for (int w = 0; w < 16; ++w) {
        pre += w < wave ? wsum[w] : 0;
        tot += wsum[w];
      }
      if (pred) gidx[base + pre + within] = (int32_t)f;
      base += tot;
      __syncthreads();
    }
  }
}

__global__ void gather_i32_kernel(const int32_t* __restrict__ src, const int32_t* __restrict__ idx, int m,
                                  int32_t* __restrict__ dst) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < m) dst[i] = src[idx[i]];
}

// dst[i] = src[idx[i]] for matrices of `bytes` bytes (a multiple of 16);
// grid (chunks, m)
__global__ __launch_bounds__(256) void gather_matrices_kernel(const unsigned char* __restrict__ src,
                                                              unsigned char* __restrict__ dst,
                                                              const int32_t* __restrict__ idx, int64_t bytes) {
  const int64_t i = blockIdx.y;
  const uint4* s = reinterpret_cast<const uint4*>(src + (int64_t)idx[i] * bytes);
  uint4* d = reinterpret_cast<uint4*>(dst + i * bytes);
  for (int64_t k = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; k < bytes / 16; k += (int64_t)gridDim.x * blockDim.x)
    d[k] = s[k];
}

// dst[idx[i]] = src[i] where flags_src[i] shows neither NONFINITE nor
// ZERO_SCALE, and then fl_dst[idx[i]] |= RECOMPUTED_F64
__global__ __launch_bounds__(256) void scatter_matrices_kernel(const unsigned char* __restrict__ src,
                                                               unsigned char* __restrict__ dst,
                                                               const int32_t* __restrict__ idx,
                                                               const int32_t* __restrict__ flags_src, int64_t bytes,
                                                               int32_t* __restrict__ fl_dst) {
  const int64_t i = blockIdx.y;
  if (flags_src[i] & (SHAMPOO_FLAG_NONFINITE | SHAMPOO_FLAG_ZERO_SCALE)) return;  // uniform
  const uint4* s = reinterpret_cast<const uint4*>(src + i * bytes);
  uint4* d = reinterpret_cast<uint4*>(dst + (int64_t)idx[i] * bytes);
  for (int64_t k = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; k < bytes / 16; k += (int64_t)gridDim.x * blockDim.x)
    d[k] = s[k];
  if (blockIdx.x == 0 && threadIdx.x == 0) atomicOr(fl_dst + idx[i], SHAMPOO_FLAG_RECOMPUTED_F64);
}

// Factor-side groups.  gather_sub: dst[i] (s x s) = leading s x s block of
// the B x B matrix src[idx[i]]; scatter_sub: the B x B matrix dst[idx[i]] =
// src[i] (s x s) zero-padded to B, skipped where keep is set and flags[i]
// shows a failed root (NONFINITE, ZERO_SCALE or RESIDUAL).  E: raw element type (bit copies); s and B
// multiples of 64; grid (chunks, m).
template <typename E>
__global__ __launch_bounds__(256) void gather_sub_kernel(const E* __restrict__ src, E* __restrict__ dst,
                                                         const int32_t* __restrict__ idx, int B, int s) {
  constexpr int V = 16 / sizeof(E);
  const int64_t i = blockIdx.y;
  const E* a = src + (int64_t)idx[i] * B * B;
  E* d = dst + i * (int64_t)s * s;
  const int cpr = s / V;
  for (int k = blockIdx.x * blockDim.x + threadIdx.x; k < s * cpr; k += gridDim.x * blockDim.x) {
    const int r = k / cpr, c = (k - r * cpr) * V;
    *reinterpret_cast<uint4*>(d + (int64_t)r * s + c) = *reinterpret_cast<const uint4*>(a + (int64_t)r * B + c);
  }
}

template <typename E>
__global__ __launch_bounds__(256) void scatter_sub_kernel(const E* __restrict__ src, E* __restrict__ dst,
                                                          const int32_t* __restrict__ idx, int B, int s,
                                                          const int32_t* __restrict__ flags, int keep) {
  constexpr int V = 16 / sizeof(E);
  const int64_t i = blockIdx.y;
  if (keep && (flags[i] & FAILED_ROOT)) return;  // uniform
  const E* a = src + i * (int64_t)s * s;
  E* d = dst + (int64_t)idx[i] * B * B;
  const int cpr = B / V;
  for (int k = blockIdx.x * blockDim.x + threadIdx.x; k < B * cpr; k += gridDim.x * blockDim.x) {
    const int r = k / cpr, c = (k - r * cpr) * V;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (r < s && c < s) v = *reinterpret_cast<const uint4*>(a + (int64_t)r * s + c);
    *reinterpret_cast<uint4*>(d + (int64_t)r * B + c) = v;
  }
}

// dst[idx[i]] |= src[i] (distinct indices)
__global__ void or_flags_kernel(const int32_t* __restrict__ src, const int32_t* __restrict__ idx, int m,
                                int32_t* __restrict__ dst) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < m) dst[idx[i]] |= src[i];
}

// dst[idx[i]] = src[i] (distinct indices)
__global__ void scatter_f32_kernel(const float* __restrict__ src, const int32_t* __restrict__ idx, int m,
                                   float* __restrict__ dst) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < m) dst[idx[i]] = src[i];
}

// Step flags after the fallback: a factor whose root failed (NONFINITE,
// ZERO_SCALE or RESIDUAL) and was not recomputed kept its previous root; the
// result is OR-ed into the caller's flags.
__global__ void merge_fallback_flags_kernel(const int32_t* __restrict__ fl, int64_t n, int32_t* __restrict__ out) {
  const int64_t b = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (b >= n) return;
  int32_t f = fl[b];
  if ((f & FAILED_ROOT) && !(f & SHAMPOO_FLAG_RECOMPUTED_F64)) f |= SHAMPOO_FLAG_KEPT_PREVIOUS;
  out[b] |= f;
}

// ---------------------------------------------------------------------------
// grafting.  Work item = (block, chunk of GRAFT_ROWS rows of the block).
// The vector paths stream D, G, m, v and W with non-temporal loads and
// stores (each element is touched once per kernel): 63% -> 68% and 62% ->
// 67% of HBM bandwidth on the decoder step's grafting kernels.
// ---------------------------------------------------------------------------
constexpr int GRAFT_ROWS = 16;

template <typename TG> __device__ __forceinline__ float gval(const void* g, int64_t i);
template <> __device__ __forceinline__ float gval<float>(const void* g, int64_t i) {
  return reinterpret_cast<const float*>(g)[i];
}
template <> __device__ __forceinline__ float gval<__bf16>(const void* g, int64_t i) {
  const uint16_t u = reinterpret_cast<const uint16_t*>(g)[i];
  return __uint_as_float((uint32_t)u << 16);
}

struct GraftArgs {
  const shampoo_param* params;
  int nparams;
  const shampoo_block* table;
  const float* dstack;
  int B;
  int nchunk;        // chunks per block
  int graft;         // shampoo_graft
  float lr, momentum, beta1, beta2, eps;
  float bc1, bc2;    // 1 - beta1^t, 1 - beta2^t
  double* partials;  // [nblk][nchunk][2]: sum D^2, sum Delta^2
  float* scales;     // [nblk]: per-block D_g / D factor
};

// Four consecutive gradient values (16-byte aligned float32 or 8-byte
// aligned bfloat16) as float.
template <typename TG> __device__ __forceinline__ void gload4(const void* g, int64_t i, float* o);
template <> __device__ __forceinline__ void gload4<float>(const void* g, int64_t i, float* o) {
  const floatx4 t = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(reinterpret_cast<const float*>(g) + i));
  o[0] = t[0]; o[1] = t[1]; o[2] = t[2]; o[3] = t[3];
}
template <> __device__ __forceinline__ void gload4<__bf16>(const void* g, int64_t i, float* o) {
  const u32x2 t = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(reinterpret_cast<const uint16_t*>(g) + i));
  o[0] = __uint_as_float(t[0] << 16); o[1] = __uint_as_float(t[0] & 0xffff0000u);
  o[2] = __uint_as_float(t[1] << 16); o[3] = __uint_as_float(t[1] & 0xffff0000u);
}

// Parameter rows of a block can be read four elements at a time when every
// row starts 16-byte aligned (uniform per workgroup).
template <typename TG> __device__ __forceinline__ bool graft_vec(const shampoo_param& P, const shampoo_block& blk) {
  const uintptr_t al = reinterpret_cast<uintptr_t>(P.w) | reinterpret_cast<uintptr_t>(P.m) |
                       reinterpret_cast<uintptr_t>(P.v) | ((uintptr_t)P.ld * 4) | ((uintptr_t)blk.col0 * 4);
  const uintptr_t ag = reinterpret_cast<uintptr_t>(P.g) | ((uintptr_t)P.ld * sizeof(TG)) |
                       ((uintptr_t)blk.col0 * sizeof(TG));
  return (al & 15) == 0 && (ag & (4 * sizeof(TG) - 1)) == 0;
}

// Sums of D^2 and Delta^2 over GRAFT_ROWS rows of a block (Adam: m and v
// updated in passing).  Work: chunks of 4 columns, chunk k to thread
// k % 256, visited in increasing k; one accumulator chain per element
// position, added in a fixed order at the end.  Blocks whose rows are
// 16-byte aligned and a multiple of 4 wide take the vector path (GRAFT_U
// chunks loaded before any is used); the others one chunk at a time with
// scalar accesses.  The scalar path is kept out of the unrolled loop so that
// it does not set the register count: the kernels then run 4 (norms) and 7
// (update) waves per SIMD instead of 3 and 2.  Both paths visit the
// same chunks in the same order, so the sums are the same bit for bit.
constexpr int GRAFT_U = 4;

// the per-element Adam step and the two squares added to the chains
__device__ __forceinline__ void graft_elem(const GraftArgs& a, bool adam, float d, float g, float& m, float& v,
                                           double& sd, double& sg) {
  sd += (double)d * d;
  float delta = g;
  if (adam) {
    m = a.beta1 * m + (1.0f - a.beta1) * g;
    v = a.beta2 * v + (1.0f - a.beta2) * g * g;
    delta = (m / a.bc1) / (sqrtf(v / a.bc2) + a.eps);
  }
  sg += (double)delta * delta;
}

template <typename TG>
__global__ __launch_bounds__(256) void graft_partials_kernel(GraftArgs a) {
  __shared__ double red[4];
  const int64_t b = blockIdx.y;
  const int ch = blockIdx.x;
  const shampoo_block blk = a.table[b];
  if (blk.param < 0 || blk.param >= a.nparams) return;
  const shampoo_param P = a.params[blk.param];
  const float* D = a.dstack + b * (int64_t)a.B * a.B;
  const bool adam = a.graft == SHAMPOO_GRAFT_ADAM && P.m && P.v;
  double sd[4] = {0.0, 0.0, 0.0, 0.0}, sg[4] = {0.0, 0.0, 0.0, 0.0};
  const int r0 = ch * GRAFT_ROWS;
  const int r1 = min(blk.rows, r0 + GRAFT_ROWS);
  const int cpr = (blk.cols + 3) / 4;
  const int total = max(r1 - r0, 0) * cpr;
  if (graft_vec<TG>(P, blk) && (blk.cols & 3) == 0) {
    for (int base = (int)threadIdx.x; base < total; base += 256 * GRAFT_U) {
      floatx4 d[GRAFT_U], m[GRAFT_U], v[GRAFT_U];
      float g[GRAFT_U][4];
      int64_t prow[GRAFT_U];
#pragma unroll
      for (int u = 0; u < GRAFT_U; ++u) {
        const int k = base + u * 256;
        if (k >= total) continue;
        const int rr = k / cpr, c = (k - rr * cpr) * 4;
        prow[u] = (int64_t)(blk.row0 + r0 + rr) * P.ld + blk.col0 + c;
        d[u] = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(D + (int64_t)(r0 + rr) * a.B + c));
        gload4<TG>(P.g, prow[u], g[u]);
        if (adam) {
          m[u] = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(P.m + prow[u]));
          v[u] = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(P.v + prow[u]));
        }
      }
#pragma unroll
      for (int u = 0; u < GRAFT_U; ++u) {
        if (base + u * 256 >= total) continue;
        float mm[4], vv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          mm[e] = adam ? m[u][e] : 0.f;
          vv[e] = adam ? v[u][e] : 0.f;
          graft_elem(a, adam, d[u][e], g[u][e], mm[e], vv[e], sd[e], sg[e]);
        }
        if (adam) {
          __builtin_nontemporal_store(floatx4{mm[0], mm[1], mm[2], mm[3]}, reinterpret_cast<floatx4*>(P.m + prow[u]));
          __builtin_nontemporal_store(floatx4{vv[0], vv[1], vv[2], vv[3]}, reinterpret_cast<floatx4*>(P.v + prow[u]));
        }
      }
    }
  } else {
    for (int k = (int)threadIdx.x; k < total; k += 256) {
      const int rr = k / cpr, c = (k - rr * cpr) * 4;
      const int nv = min(4, blk.cols - c);
      const int64_t prow = (int64_t)(blk.row0 + r0 + rr) * P.ld + blk.col0 + c;
      const float* dp = D + (int64_t)(r0 + rr) * a.B + c;
      for (int e = 0; e < nv; ++e) {
        float mm = adam ? P.m[prow + e] : 0.f, vv = adam ? P.v[prow + e] : 0.f;
        graft_elem(a, adam, dp[e], gval<TG>(P.g, prow + e), mm, vv, sd[e], sg[e]);
        if (adam) {
          P.m[prow + e] = mm;
          P.v[prow + e] = vv;
        }
      }
    }
  }
  double td = (sd[0] + sd[1]) + (sd[2] + sd[3]);
  double tg = (sg[0] + sg[1]) + (sg[2] + sg[3]);
  td = block_sum256(td, red);
  tg = block_sum256(tg, red);
  if (threadIdx.x == 0) {
    a.partials[(b * a.nchunk + ch) * 2 + 0] = td;
    a.partials[(b * a.nchunk + ch) * 2 + 1] = tg;
  }
}

// One thread per block: the scale of its norm group (its parameter, or the
// block itself), reduced in a fixed order over the group's blocks and chunks.
__global__ void graft_scale_kernel(GraftArgs a, int64_t nblk, int blockwise) {
  const int64_t b = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (b >= nblk) return;
  int64_t first = b, count = 1;
  if (!blockwise) {
    const shampoo_block blk = a.table[b];
    const shampoo_param P = a.params[blk.param];
    first = P.first_block;
    const int64_t bs = blk.B;  // planning block size (the stack side a.B may be larger)
    count = ((P.rows + bs - 1) / bs) * ((P.cols + bs - 1) / bs);
    if (first < 0) first = 0;
    if (first + count > nblk) count = nblk - first;
  }
  double sd = 0.0, sg = 0.0;
  for (int64_t q = first; q < first + count; ++q)
    for (int ch = 0; ch < a.nchunk; ++ch) {
      sd += a.partials[(q * a.nchunk + ch) * 2 + 0];
      sg += a.partials[(q * a.nchunk + ch) * 2 + 1];
    }
  float sc;
  if (a.graft == SHAMPOO_GRAFT_NONE) sc = 1.0f;
  else sc = sd > 0.0 ? (float)(sqrt(sg) / sqrt(sd)) : 0.0f;
  a.scales[b] = sc;
}

__global__ __launch_bounds__(256) void graft_update_kernel(GraftArgs a) {
  const int64_t b = blockIdx.y;
  const int ch = blockIdx.x;
  const shampoo_block blk = a.table[b];
  if (blk.param < 0 || blk.param >= a.nparams) return;
  const shampoo_param P = a.params[blk.param];
  const float* D = a.dstack + b * (int64_t)a.B * a.B;
  const float sc = a.scales[b];
  const bool mom = a.graft == SHAMPOO_GRAFT_MOMENTUM && P.m;
  const int r0 = ch * GRAFT_ROWS;
  const int r1 = min(blk.rows, r0 + GRAFT_ROWS);
  const int cpr = (blk.cols + 3) / 4;
  const int total = max(r1 - r0, 0) * cpr;
  // w -= lr * D_g (plain) or m = mu m + D_g, w -= lr * m (momentum)
  auto elem = [&](float d, float& w, float& m) {
    const float dg = sc * d;
    if (mom) {
      m = a.momentum * m + dg;
      w -= a.lr * m;
    } else {
      w -= a.lr * dg;
    }
  };
  if (graft_vec<float>(P, blk) && (blk.cols & 3) == 0) {
    for (int base = (int)threadIdx.x; base < total; base += 256 * GRAFT_U) {
      floatx4 d[GRAFT_U], w[GRAFT_U], m[GRAFT_U];
      int64_t prow[GRAFT_U];
#pragma unroll
      for (int u = 0; u < GRAFT_U; ++u) {
        const int k = base + u * 256;
        if (k >= total) continue;
        const int rr = k / cpr, c = (k - rr * cpr) * 4;
        prow[u] = (int64_t)(blk.row0 + r0 + rr) * P.ld + blk.col0 + c;
        d[u] = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(D + (int64_t)(r0 + rr) * a.B + c));
        w[u] = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(P.w + prow[u]));
        if (mom) m[u] = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(P.m + prow[u]));
      }
#pragma unroll
      for (int u = 0; u < GRAFT_U; ++u) {
        if (base + u * 256 >= total) continue;
        float ww[4], mm[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ww[e] = w[u][e];
          mm[e] = mom ? m[u][e] : 0.f;
          elem(d[u][e], ww[e], mm[e]);
        }
        __builtin_nontemporal_store(floatx4{ww[0], ww[1], ww[2], ww[3]}, reinterpret_cast<floatx4*>(P.w + prow[u]));
        if (mom) __builtin_nontemporal_store(floatx4{mm[0], mm[1], mm[2], mm[3]}, reinterpret_cast<floatx4*>(P.m + prow[u]));
      }
    }
  } else {
    for (int k = (int)threadIdx.x; k < total; k += 256) {
      const int rr = k / cpr, c = (k - rr * cpr) * 4;
      const int nv = min(4, blk.cols - c);
      const int64_t prow = (int64_t)(blk.row0 + r0 + rr) * P.ld + blk.col0 + c;
      const float* dp = D + (int64_t)(r0 + rr) * a.B + c;
      for (int e = 0; e < nv; ++e) {
        float ww = P.w[prow + e], mm = mom ? P.m[prow + e] : 0.f;
        elem(dp[e], ww, mm);
        P.w[prow + e] = ww;
        if (mom) P.m[prow + e] = mm;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Matrix-core throughput: each wave runs `iters` rounds of CHAINS independent
// MFMAs on register operands (64 accumulator registers per lane, so the
// compiler keeps them in place across the loop).  `never` is 0 at run time; the store it guards
// keeps the accumulators live.
// ---------------------------------------------------------------------------
template <Mma M> struct PeakOp;
template <> struct PeakOp<Mma::F32> {
  using acc_t = floatx4;
  using op_t = float;
  static constexpr int CHAINS = 16;
  static constexpr double flops = 2.0 * 16 * 16 * 4;
  static __device__ __forceinline__ op_t make(float x) { return x; }
  static __device__ __forceinline__ acc_t mma(op_t a, op_t b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};
template <> struct PeakOp<Mma::F64> {
  using acc_t = doublex4;
  using op_t = double;
  static constexpr int CHAINS = 8;
  static constexpr double flops = 2.0 * 16 * 16 * 4;
  static __device__ __forceinline__ op_t make(float x) { return (double)x; }
  static __device__ __forceinline__ acc_t mma(op_t a, op_t b, acc_t c) {
    return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
  }
};
template <> struct PeakOp<Mma::F16> {
  using acc_t = floatx4;
  using op_t = halfx8;
  static constexpr int CHAINS = 16;
  static constexpr double flops = 2.0 * 16 * 16 * 32;
  static __device__ __forceinline__ op_t make(float x) {
    const _Float16 h = (_Float16)x;
    return op_t{h, h, h, h, h, h, h, h};
  }
  static __device__ __forceinline__ acc_t mma(op_t a, op_t b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};
template <> struct PeakOp<Mma::BF16> {
  using acc_t = floatx4;
  using op_t = bf16x8;
  static constexpr int CHAINS = 16;
  static constexpr double flops = 2.0 * 16 * 16 * 32;
  static __device__ __forceinline__ op_t make(float x) {
    const __bf16 h = (__bf16)x;
    return op_t{h, h, h, h, h, h, h, h};
  }
  static __device__ __forceinline__ acc_t mma(op_t a, op_t b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <Mma M>
__global__ __launch_bounds__(256, 4) void mfma_peak_kernel(int iters, int never, float* __restrict__ sink) {
  using Op = PeakOp<M>;
  constexpr int NC = Op::CHAINS;
  typename Op::acc_t acc[NC];
  const float t = 1.0f + 1e-3f * (float)(threadIdx.x & 63);
  const typename Op::op_t a = Op::make(t), b = Op::make(2.0f - t);
#pragma unroll
  for (int j = 0; j < NC; ++j) acc[j] = typename Op::acc_t{0, 0, 0, 0};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < NC; ++j) acc[j] = Op::mma(a, b, acc[j]);
  }
  if (never) {
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < NC; ++j) s += (float)(acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3]);
    sink[threadIdx.x & 15] = s;
  }
}

}  // namespace shampoo
