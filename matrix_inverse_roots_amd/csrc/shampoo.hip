// C ABI of the batched block preconditioner step (see include/shampoo.h).
//
// Host side: argument validation (before any launch), workspace carving,
// the solver-chain planner and kernel launches.  No entry point allocates
// device memory; every launch goes to the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <type_traits>
#include <vector>

#include "gemm.hpp"
#include "gemm_hsym.hpp"
#include "gemm_nn256.hpp"
#include "kernels.hpp"
#include "shampoo.h"

using namespace shampoo;

namespace {

thread_local std::string g_err;

shampoo_status fail(shampoo_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

#define HIP_TRY(expr)                                                                  \
  do {                                                                                 \
    hipError_t e_ = (expr);                                                            \
    if (e_ != hipSuccess) return fail(SHAMPOO_E_HIP, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

#define LAUNCH_CHECK(what)                                                             \
  do {                                                                                 \
    hipError_t e_ = hipGetLastError();                                                 \
    if (e_ != hipSuccess) return fail(SHAMPOO_E_HIP, "%s launch: %s", what, hipGetErrorString(e_)); \
  } while (0)

constexpr size_t ALIGN = 256;
inline size_t align_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

size_t dtype_size(int dt) {
  switch (dt) {
    case SHAMPOO_F32: return 4;
    case SHAMPOO_F16: return 2;
    case SHAMPOO_BF16: return 2;
    case SHAMPOO_F64: return 8;
    default: return 0;
  }
}

// ---------------------------------------------------------------------------
// GEMM dispatch
// ---------------------------------------------------------------------------
struct GemmCall {
  const void* A = nullptr;
  const void* B = nullptr;
  const void* D = nullptr;
  void* C = nullptr;
  void* C2 = nullptr;
  void* Ch = nullptr;   // half copies (products of half operands)
  void* C2h = nullptr;
  double alpha = 1.0, beta = 0.0, gamma = 0.0, alpha2 = 0.0, gamma2 = 0.0;
  bool sym = true;
  bool transC = false;
  bool nn = false;  // B read k-major: C = A B (no symmetry assumed)
  // Per-matrix row, column and inner extents (gemm_kernel's Extents), or
  // null for n.  With any of them set the product runs on the 64-tile tiled
  // kernel, which skips the tiles and k-stages outside them.
  const int32_t* rext = nullptr;
  const int32_t* cext = nullptr;
  const int32_t* kext = nullptr;
  // Optional work-balanced list of the tiles inside the extents
  // (tile_list_kernel): the tiled kernel then walks it with a fixed grid.
  const int32_t* tiles = nullptr;
  const int32_t* cut = nullptr;
  int tile = 64;  // tile side of that list: 64 (tiled kernel) or 128 (persistent 128-tile kernel)
};

#define HIP_TRY_ERR(expr)         \
  do {                            \
    hipError_t e_ = (expr);       \
    if (e_ != hipSuccess) return e_; \
  } while (0)

constexpr int MAX_DEVICES = 64;

// Compute units of the current device, queried once per device.
hipError_t cu_count(int* cus) {
  static int cache[MAX_DEVICES] = {0};
  int dev = 0;
  HIP_TRY_ERR(hipGetDevice(&dev));
  if (dev >= 0 && dev < MAX_DEVICES && cache[dev] > 0) {
    *cus = cache[dev];
    return hipSuccess;
  }
  int v = 0;
  HIP_TRY_ERR(hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev));
  if (dev >= 0 && dev < MAX_DEVICES) cache[dev] = v;
  *cus = v;
  return hipSuccess;
}

// The large-tile products need 128 KB of dynamic LDS, above the default
// limit; raise each kernel's limit once per device (K tells the kernels
// apart).
template <int K>
hipError_t large_lds_prepare(const void* kernel, int bytes) {
  static bool done[MAX_DEVICES] = {false};
  int dev = 0;
  HIP_TRY_ERR(hipGetDevice(&dev));
  if (dev >= 0 && dev < MAX_DEVICES && done[dev]) return hipSuccess;
  HIP_TRY_ERR(hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes));
  if (dev >= 0 && dev < MAX_DEVICES) done[dev] = true;
  return hipSuccess;
}

// Float32 and float64 NT products: the persistent 128-tile kernel runs 2
// workgroups per CU, the 64-tile kernel 4.  Measured on MI355X, a round of 128-tile slots
// costs as much as 2 / 0.88 rounds of 64-tile slots (half the work per round
// at 88% of the efficiency), so the 64-tile kernel wins when the tiles fill
// the 128-tile slots poorly: small batches, and tile counts just above a
// multiple of the slots (171 blocks of 256^2: 513 tiles for 512 slots, two
// rounds).
bool prefer_64_tiles(int n, int64_t batch, bool sym, int cus) {
  const int64_t nt128 = n / 128, nt64 = n / 64;
  const int64_t t128 = batch * (sym ? nt128 * (nt128 + 1) / 2 : nt128 * nt128);
  const int64_t t64 = batch * (sym ? nt64 * (nt64 + 1) / 2 : nt64 * nt64);
  const int64_t s128 = (int64_t)std::max(8, (cus / 8) * 8) * 2, s64 = (int64_t)std::max(1, cus) * 4;
  const int64_t r128 = (t128 + s128 - 1) / s128, r64 = (t64 + s64 - 1) / s64;
  return r64 * 100 < r128 * 2 * 88;
}

template <Mma MM, typename TA, typename TB, typename TC>
hipError_t gemm(const GemmCall& c, int n, int64_t batch, hipStream_t st) {
  const bool ext = c.rext || c.cext || c.kext;
  const Extents ex{c.rext, c.cext, c.kext};
  {
    constexpr bool one_type = (MM == Mma::F32 && std::is_same<TA, float>::value && std::is_same<TB, float>::value &&
                               std::is_same<TC, float>::value) ||
                              (MM == Mma::F64 && std::is_same<TA, double>::value &&
                               std::is_same<TB, double>::value && std::is_same<TC, double>::value);
    if (c.tiles && c.tile != 64 && !(one_type && c.tile == P128_T && !c.nn && n % P128_T == 0))
      return hipErrorInvalidValue;  // a list of 128-tiles is walked by the persistent kernel only
  }
  int T = (n % 128 == 0 && !ext) ? 128 : 64;
  if constexpr ((MM == Mma::F32 && std::is_same<TA, float>::value && std::is_same<TB, float>::value &&
                 std::is_same<TC, float>::value) ||
                (MM == Mma::F64 && std::is_same<TA, double>::value && std::is_same<TB, double>::value &&
                 std::is_same<TC, double>::value)) {
    if (T == 128 && !c.nn && batch > 0) {
      int cus = 0;
      HIP_TRY_ERR(cu_count(&cus));
      if (prefer_64_tiles(n, batch, c.sym, cus)) T = 64;
    }
  }
  GemmArgs g;
  g.A = c.A;
  g.B = c.B;
  g.D = c.D;
  g.C = c.C;
  g.C2 = c.C2;
  g.Ch = c.Ch;
  g.C2h = c.C2h;
  g.n = n;
  g.nt = n / T;
  g.sym = c.sym ? 1 : 0;
  g.transC = c.transC ? 1 : 0;
  g.tiles = c.sym ? g.nt * (g.nt + 1) / 2 : g.nt * g.nt;
  g.stride = (int64_t)n * n;
  g.total = batch * g.tiles;
  g.alpha = c.alpha;
  g.beta = c.beta;
  g.gamma = c.gamma;
  g.alpha2 = c.alpha2;
  g.gamma2 = c.gamma2;
  if (g.total == 0) return hipSuccess;
  dim3 grid((unsigned)g.total);
  const TileList tl{c.tiles, c.cut};
  if (c.tiles) {
    // a fixed grid of 4 workgroups per CU (a multiple of the 8 XCDs) walks the list
    int cus = 0;
    HIP_TRY_ERR(cu_count(&cus));
    grid = dim3((unsigned)(std::max(8, (cus / 8) * 8) * 4));
  }
  if constexpr (MM == Mma::F32 && std::is_same<TA, float>::value && std::is_same<TB, float>::value &&
                std::is_same<TC, float>::value) {
    if (c.nn && n % NN256_T == 0 && c.D == nullptr && !c.transC && !ext) {
      int cus = 0;
      HIP_TRY_ERR(cu_count(&cus));
      GemmArgs h = g;
      h.nt = n / NN256_T;
      h.tiles = h.nt * h.nt;
      h.total = batch * h.tiles;
      // persistent grid: at most one workgroup per CU, a multiple of the 8 XCDs
      const int64_t wgs = std::min<int64_t>(((h.total + 7) / 8) * 8, std::max(8, (cus / 8) * 8));
      HIP_TRY_ERR(large_lds_prepare<0>((const void*)gemm_f32_nn256_kernel, NN256_LDS));
      hipLaunchKernelGGL(gemm_f32_nn256_kernel, dim3((unsigned)wgs), dim3(512), NN256_LDS, st, h);
      return hipGetLastError();
    }
  }
  // One operand type throughout, float32 or float64, n a multiple of 128:
  // persistent 128-tile kernel (NT in every mode; NN without sym/transC).
  constexpr bool same32 = MM == Mma::F32 && std::is_same<TA, float>::value && std::is_same<TB, float>::value &&
                          std::is_same<TC, float>::value;
  constexpr bool same64 = MM == Mma::F64 && std::is_same<TA, double>::value && std::is_same<TB, double>::value &&
                          std::is_same<TC, double>::value;
  if constexpr (same32 || same64) {
    // extents with a list of 128-tiles: the persistent kernel walks the list
    if (c.tiles && c.tile == P128_T && !c.nn && n % P128_T == 0) {
      using E = typename std::conditional<same32, float, double>::type;
      int cus = 0;
      HIP_TRY_ERR(cu_count(&cus));
      const int64_t wgs = (int64_t)std::max(8, (cus / 8) * 8) * 2;
      hipLaunchKernelGGL((gemm_p128_kernel<E, false, true>), dim3((unsigned)wgs), dim3(256), 0, st, g,
                         TileList{c.tiles, c.cut}, c.kext);
      return hipGetLastError();
    }
    if (T == P128_T && (!c.nn || (!c.sym && !c.transC))) {
      using E = typename std::conditional<same32, float, double>::type;
      int cus = 0;
      HIP_TRY_ERR(cu_count(&cus));
      GemmArgs h = g;
      if (c.nn) {
        h.sym = 0;
        h.tiles = h.nt * h.nt;
        h.total = batch * h.tiles;
      }
      // persistent grid: two workgroups per CU, a multiple of the 8 XCDs
      const int64_t wgs = std::min<int64_t>(((h.total + 7) / 8) * 8, std::max(8, (cus / 8) * 8) * 2);
      if (c.nn)
        hipLaunchKernelGGL((gemm_p128_kernel<E, true, false>), dim3((unsigned)wgs), dim3(256), 0, st, h, TileList{nullptr, nullptr}, nullptr);
      else
        hipLaunchKernelGGL((gemm_p128_kernel<E, false, false>), dim3((unsigned)wgs), dim3(256), 0, st, h, TileList{nullptr, nullptr}, nullptr);
      return hipGetLastError();
    }
  }
  // bfloat16 operands into float32 (statistics of bf16 gradients), NT
  constexpr bool bf16_in = MM == Mma::BF16 && std::is_same<TA, __bf16>::value && std::is_same<TB, __bf16>::value &&
                           std::is_same<TC, float>::value;
  if constexpr (bf16_in) {
    if (T == P128_T && !c.nn) {
      int cus = 0;
      HIP_TRY_ERR(cu_count(&cus));
      const int64_t wgs = std::min<int64_t>(((g.total + 7) / 8) * 8, std::max(8, (cus / 8) * 8) * 2);
      hipLaunchKernelGGL((gemm_p128_kernel<__bf16, false, false>), dim3((unsigned)wgs), dim3(256), 0, st, g, TileList{nullptr, nullptr}, nullptr);
      return hipGetLastError();
    }
  }
  // half operands into float32 (f16 solver chains), NT
  constexpr bool f16_in = MM == Mma::F16 && std::is_same<TA, _Float16>::value &&
                          std::is_same<TB, _Float16>::value && std::is_same<TC, float>::value;
  if constexpr (f16_in) {
    // NN (Newton-DB): 256-tile kernel; symmetric NT with half outputs only:
    // 256-tile symmetric kernel; the other NT products: 128-tile kernel.
    if (c.nn && n % H256_T == 0 && !c.sym && c.D == nullptr && !c.transC && !ext) {
      int cus = 0;
      HIP_TRY_ERR(cu_count(&cus));
      GemmArgs h = g;
      h.sym = 0;
      h.nt = n / H256_T;
      h.tiles = h.nt * h.nt;
      h.total = batch * h.tiles;
      // persistent grid: one workgroup per CU, a multiple of the 8 XCDs
      const int64_t wgs = std::min<int64_t>(((h.total + 7) / 8) * 8, std::max(8, (cus / 8) * 8));
      HIP_TRY_ERR(large_lds_prepare<1>((const void*)gemm_h256_nn_kernel, H256_LDS));
      hipLaunchKernelGGL(gemm_h256_nn_kernel, dim3((unsigned)wgs), dim3(512), H256_LDS, st, h);
      return hipGetLastError();
    }
    // symmetric NT with half outputs only, n a multiple of 256: 256-tiles of
    // 8 waves (1.07x - 1.23x faster than the 128-tile kernel on 288 x 1024^2)
    if (!c.nn && c.sym && !c.transC && n % HS_T == 0 && !ext && c.C == nullptr && c.C2 == nullptr &&
        c.D == nullptr && c.Ch != nullptr) {
      int cus = 0;
      HIP_TRY_ERR(cu_count(&cus));
      GemmArgs h = g;
      h.nt = n / HS_T;
      h.tiles = h.nt * (h.nt + 1) / 2;
      h.total = batch * h.tiles;
      // persistent grid: one workgroup per CU, a multiple of the 8 XCDs
      const int64_t wgs = std::min<int64_t>(((h.total + 7) / 8) * 8, std::max(8, (cus / 8) * 8));
      HIP_TRY_ERR(large_lds_prepare<2>((const void*)gemm_h256_sym_kernel, HS_LDS));
      hipLaunchKernelGGL(gemm_h256_sym_kernel, dim3((unsigned)wgs), dim3(512), HS_LDS, st, h);
      return hipGetLastError();
    }
    if (T == P128_T && !c.nn && !c.transC) {
      int cus = 0;
      HIP_TRY_ERR(cu_count(&cus));
      const int64_t wgs = std::min<int64_t>(((g.total + 7) / 8) * 8, std::max(8, (cus / 8) * 8) * 2);
      hipLaunchKernelGGL((gemm_p128_kernel<_Float16, false, false>), dim3((unsigned)wgs), dim3(256), 0, st, g, TileList{nullptr, nullptr}, nullptr);
      return hipGetLastError();
    }
  }
  if constexpr (std::is_same<TB, float>::value || std::is_same<TB, double>::value || f16_in) {
    if (c.nn) {
      if (T == 128)
        hipLaunchKernelGGL((gemm_kernel<MM, 128, true, TA, TB, TC>), grid, dim3(256), 0, st, g, ex, tl);
      else
        hipLaunchKernelGGL((gemm_kernel<MM, 64, true, TA, TB, TC>), grid, dim3(256), 0, st, g, ex, tl);
      return hipGetLastError();
    }
  }
  if (c.nn) return hipErrorInvalidValue;
  if (T == 128)
    hipLaunchKernelGGL((gemm_kernel<MM, 128, false, TA, TB, TC>), grid, dim3(256), 0, st, g, ex, tl);
  else
    hipLaunchKernelGGL((gemm_kernel<MM, 64, false, TA, TB, TC>), grid, dim3(256), 0, st, g, ex, tl);
  return hipGetLastError();
}

int64_t gemm_wgs(int n, int64_t batch, bool sym) {
  const int T = (n % 128 == 0) ? 128 : 64;
  const int64_t nt = n / T;
  return batch * (sym ? nt * (nt + 1) / 2 : nt * nt);
}

// ---------------------------------------------------------------------------
// Solver-chain planner.  Buffers are small integers handed out by a pool that
// records its peak, so the workspace query and the execution run the very
// same plan.
// ---------------------------------------------------------------------------
enum OpKind { OP_PREP, OP_GEMM, OP_COMB, OP_MCOMB, OP_CHECK, OP_FINAL };

struct Op {
  OpKind kind;
  // PREP: up to three outputs (buffer, alpha, gamma)
  int out[3] = {-1, -1, -1};
  double oa[3] = {0, 0, 0}, og[3] = {0, 0, 0};
  // GEMM: C = alpha A B^T + beta D + gamma I ; C2 = alpha2 C + gamma2 I
  int a = -1, b = -1, d = -1, c = -1, c2 = -1;
  bool nn = false;  // full product A B in the given order (else symmetric NT)
  double alpha = 1, beta = 0, gamma = 0, alpha2 = 0, gamma2 = 0;
  // CHECK: stop once every matrix of buffer a is within alpha * tol of I.
  // Coupled Newton (b = 0): the next op (X T) then gives the result, which
  // is finalised.  Newton-DB (b = call 1 or 2, c = iteration): the chain is
  // planned again with that call ending at this iteration, and runs on from
  // the same point of the new plan.
  // COMB: c = sum_q w[q] in[q] + gamma I (nin <= COMB_IN; an input may be c)
  int in[COMB_IN] = {-1, -1, -1, -1};
  double w[COMB_IN] = {0, 0, 0, 0};
  int nin = 0;
  // MCOMB: mout[j] = sum_q mw[j][q] min[q] + mg[j] I, every input read once
  std::vector<int> min, mout, mneed;
  std::vector<std::vector<double>> mw;
  std::vector<double> mg;
  // FINAL: buffer a -> out
  // Forms of each output that later ops read (NEED_F32: addend D or final
  // output; NEED_HALF: product operand); used by half-operand chains.
  int need[3] = {0, 0, 0};  // PREP outputs
  int need_c = 0, need_c2 = 0;
};
constexpr int NEED_F32 = 1, NEED_HALF = 2;

struct Plan {
  std::vector<Op> ops;
  int peak = 0;
  int gemms = 0;
  bool checks = false;  // the chain holds convergence checks (needs their scratch)
  bool sym_out = false;  // finalize returns the symmetric part (X + X^T)/2
  bool resid = false;    // the solver residual is computed before the final pass
  std::vector<bool> used;
  int get() {
    for (size_t i = 0; i < used.size(); ++i)
      if (!used[i]) {
        used[i] = true;
        return (int)i;
      }
    used.push_back(true);
    peak = (int)used.size() > peak ? (int)used.size() : peak;
    return (int)used.size() - 1;
  }
  void put(int i) {
    if (i >= 0) used[i] = false;
  }
  void prep(int o0, double a0, double g0, int o1 = -1, double a1 = 0, double g1 = 0, int o2 = -1,
            double a2 = 0, double g2 = 0) {
    Op op;
    op.kind = OP_PREP;
    op.out[0] = o0; op.oa[0] = a0; op.og[0] = g0;
    op.out[1] = o1; op.oa[1] = a1; op.og[1] = g1;
    op.out[2] = o2; op.oa[2] = a2; op.og[2] = g2;
    ops.push_back(op);
  }
  void gemm(int a, int b, int c, double alpha, double gamma, int d = -1, double beta = 0, int c2 = -1,
            double alpha2 = 0, double gamma2 = 0, bool nn = false) {
    Op op;
    op.kind = OP_GEMM;
    op.a = a; op.b = b; op.c = c; op.d = d; op.c2 = c2;
    op.alpha = alpha; op.beta = beta; op.gamma = gamma; op.alpha2 = alpha2; op.gamma2 = gamma2;
    op.nn = nn;
    ops.push_back(op);
    ++gemms;
  }
  // c = sum_q w_q in_q + gamma I for any number of (buffer, weight) terms:
  // zero weights are dropped and longer sums are chained through c.
  void comb(int c, const std::vector<std::pair<int, double>>& terms, double gamma) {
    // a term that reads c itself goes first, before any chained op writes c
    std::vector<std::pair<int, double>> t;
    for (const auto& x : terms)
      if (x.second != 0.0 && x.first == c) t.push_back(x);
    for (const auto& x : terms)
      if (x.second != 0.0 && x.first != c) t.push_back(x);
    size_t q = 0;
    bool first = true;
    do {
      Op op;
      op.kind = OP_COMB;
      op.c = c;
      op.gamma = first ? gamma : 0.0;
      if (!first) {
        op.in[0] = c;
        op.w[0] = 1.0;
        op.nin = 1;
      }
      while (q < t.size() && op.nin < COMB_IN) {
        op.in[op.nin] = t[q].first;
        op.w[op.nin] = t[q].second;
        ++op.nin;
        ++q;
      }
      ops.push_back(op);
      first = false;
    } while (q < t.size());
  }
  void check(int m, double scale = 1.0, int call = 0, int iter = 0) {
    Op op;
    op.kind = OP_CHECK;
    op.a = m;
    op.alpha = scale;
    op.b = call;
    op.c = iter;
    ops.push_back(op);
    checks = true;
  }
  void mcomb(const std::vector<int>& in, const std::vector<int>& out, const std::vector<std::vector<double>>& w,
             const std::vector<double>& g) {
    Op op;
    op.kind = OP_MCOMB;
    op.min = in;
    op.mout = out;
    op.mw = w;
    op.mg = g;
    op.mneed.assign(out.size(), 0);
    ops.push_back(op);
  }
  void final_(int x) {
    Op op;
    op.kind = OP_FINAL;
    op.a = x;
    ops.push_back(op);
  }
};

// Coupled Newton ([NOTES] "Roots on idle CPUs ...": coupled iteration of
// Guo-Higham / Iannazzo): X_0 = I, M_0 = A_s; T = ((p+1) I - M)/p;
// X <- X T; M <- T^p M.  X_1 = T_1 comes from the prep pass; the last
// iteration updates X only, and the one before it produces only the T the
// last one needs.  T^p by repeated squaring (p a power of two).
void plan_cn(Plan& P, int p, int iters, bool check) {
  const double ap = -1.0 / p, gp = (p + 1.0) / p;
  int M = P.get(), T = P.get(), X = P.get();
  P.prep(M, 1.0, 0.0, T, ap, gp, X, ap, gp);
  for (int k = 1; k <= iters; ++k) {
    if (k >= 2) {
      const int Xn = P.get();
      P.gemm(X, T, Xn, 1.0, 0.0);
      P.put(X);
      X = Xn;
    }
    if (k == iters) break;
    int Pw = T;
    for (int q = 1; q < p; q *= 2) {
      const int Pn = P.get();
      P.gemm(Pw, Pw, Pn, 1.0, 0.0);
      if (Pw != T) P.put(Pw);
      Pw = Pn;
    }
    if (Pw != T) P.put(T);
    const bool next_is_last = (k + 1 == iters);
    if (next_is_last) {
      const int Tn = P.get();
      P.gemm(Pw, M, Tn, ap, gp);  // T_(k+1) = ((p+1) I - T^p M)/p directly
      if (Pw == T) P.put(T); else P.put(Pw);
      P.put(M);
      M = -1;
      T = Tn;
    } else {
      const int Mn = P.get(), Tn = P.get();
      P.gemm(Pw, M, Mn, 1.0, 0.0, -1, 0.0, Tn, ap, gp);
      if (Pw == T) P.put(T); else P.put(Pw);
      P.put(M);
      M = Mn;
      T = Tn;
      // converged: the next op, X T with this T, is the last update of X
      if (check) P.check(M);
    }
  }
  P.final_(X);
}

// One Newton-DB call ([DASH] "3. Inverse Root Methods", Newton-DB):
// Y_0 = A, Z_0 = I; T = (3 I - Z Y)/2; Y <- Y T; Z <- T Z.  The first
// iteration uses T_0 from the caller and Z_1 = T_0 (one product instead of
// three); products whose results are not used afterwards are skipped.
// On return *Yo / *Zo hold the requested final iterates and *Tn the seed
// 1.5 I - 0.5 Y of a following call.
void ndb_call(Plan& P, int Y, int T0, int iters, bool needY, bool needZ, bool wantTn, int* Yo, int* Zo,
              int* Tn, int call = 0) {
  int Z = -1;
  *Tn = -1;
  // k = 1
  Z = T0;
  if (iters == 1) {
    if (needY || wantTn) {
      const int Yn = P.get();
      int t = -1;
      if (wantTn) t = P.get();
      P.gemm(Y, T0, Yn, 1.0, 0.0, -1, 0.0, t, -0.5, 1.5, true);
      P.put(Y);
      Y = Yn;
      *Tn = t;
    }
  } else {
    const int Yn = P.get();
    P.gemm(Y, T0, Yn, 1.0, 0.0, -1, 0.0, -1, 0.0, 0.0, true);
    P.put(Y);
    Y = Yn;
  }
  for (int k = 2; k <= iters; ++k) {
    const bool last = (k == iters);
    const int T = P.get();
    P.gemm(Z, Y, T, -0.5, 1.5, -1, 0.0, -1, 0.0, 0.0, true);
    // ||ZY - I||_F = 2 ||T - I||_F
    if (call > 0) P.check(T, 0.5, call, k);
    if (!last || needY || wantTn) {
      const int Yn = P.get();
      int t = -1;
      if (last && wantTn) t = P.get();
      P.gemm(Y, T, Yn, 1.0, 0.0, -1, 0.0, t, -0.5, 1.5, true);
      P.put(Y);
      Y = Yn;
      if (t >= 0) *Tn = t;
    }
    if (!last || needZ) {
      const int Zn = P.get();
      P.gemm(T, Z, Zn, 1.0, 0.0, -1, 0.0, -1, 0.0, 0.0, true);
      P.put(Z);
      Z = Zn;
    }
    P.put(T);
  }
  if (!needY) {
    P.put(Y);
    Y = -1;
  }
  if (!needZ) {
    P.put(Z);
    Z = -1;
  }
  *Yo = Y;
  *Zo = Z;
}

// The Newton-DB products are full products in the order of the recurrence
// (see gemm.hpp: symmetrising them destabilises the coupled iteration); the
// converged root is returned as its symmetric part, which is at least as
// close as X itself to the symmetric exact root.
// With `check`, each iteration's T is checked for convergence (calls 1, 2):
// the ops up to any iteration are the same whatever the counts, so a call
// that has converged at iteration k continues in the plan whose count for
// that call is k.
void plan_ndb(Plan& P, int p, int iters1, int iters2, bool check = false) {
  P.sym_out = true;
  const int Y0 = P.get(), T0 = P.get();
  P.prep(Y0, 1.0, 0.0, T0, -0.5, 1.5);
  int Y, Z, Tn;
  if (p == 2) {
    ndb_call(P, Y0, T0, iters1, false, true, false, &Y, &Z, &Tn, check ? 1 : 0);
    P.final_(Z);
    return;
  }
  ndb_call(P, Y0, T0, iters1, true, false, true, &Y, &Z, &Tn, check ? 1 : 0);
  int Y2, Z2, T2;
  ndb_call(P, Y, Tn, iters2, false, true, false, &Y2, &Z2, &T2, check ? 2 : 0);
  P.final_(Z2);
}

// Chebyshev series by Clenshaw's recurrence ([DASH] "A.2 Chebyshev
// polynomials for matrices": initialise B_d and B_(d-1), stop at B_1;
// d - 1 products).  S = 2 A_s - I; B_d = c_d I is kept implicit.
void plan_cheb(Plan& P, const std::vector<double>& c) {
  const int d = (int)c.size() - 1;
  if (d == 0) {
    const int X = P.get();
    P.prep(X, 0.0, c[0]);
    P.final_(X);
    return;
  }
  if (d == 1) {
    const int X = P.get();
    P.prep(X, 2.0 * c[1], c[0] - c[1]);
    P.final_(X);
    return;
  }
  const int S = P.get();
  int Bk1 = P.get();
  int Bk2 = -1;  // -1 stands for B_d = c_d I
  P.prep(S, 2.0, -1.0, Bk1, 4.0 * c[d], c[d - 1] - 2.0 * c[d]);
  for (int k = d - 2; k >= 1; --k) {
    const int N = P.get();
    if (Bk2 < 0) P.gemm(S, Bk1, N, 2.0, c[k] - c[d]);
    else P.gemm(S, Bk1, N, 2.0, c[k], Bk2, -1.0);
    P.put(Bk2);
    Bk2 = Bk1;
    Bk1 = N;
  }
  const int X = P.get();
  if (Bk2 < 0) P.gemm(S, Bk1, X, 1.0, c[0] - c[d]);
  else P.gemm(S, Bk1, X, 1.0, c[0], Bk2, -1.0);
  P.put(S);
  P.put(Bk1);
  P.put(Bk2);
  P.final_(X);
}

// Products of the Paterson-Stockmeyer split with baby-step size m (see
// plan_cheb_ps); a constant outer coefficient a_J saves one.
int cheb_ps_products(int d, int m) { return (m - 1) + d / m - (d % m == 0 ? 1 : 0); }

int cheb_ps_step(int d) {
  int m = 2;
  for (int k = 3; k <= d; ++k)
    if (cheb_ps_products(d, k) < cheb_ps_products(d, m)) m = k;
  return m;
}

// The Chebyshev series sum_k c_k T_k(S) by the baby-step/giant-step split of
// Paterson and Stockmeyer in the Chebyshev basis.  With y = T_m(S):
// T_(mj)(S) = T_j(y), and for 0 < i < m, T_(mj+i) = 2 T_j(y) T_i - T_(mj-i)
// (from 2 T_a T_b = T_(a+b) + T_(a-b)).  Applying these from the top degree
// down (the T_(mj-i) term moves to a lower coefficient) rewrites the series
// as sum_(j=0..J) T_j(y) a_j(S), J = floor(d/m), a_j = sum_(i<m) al[j][i] T_i.
// Baby steps: T_2..T_m, one product each (T_2k = 2 T_k^2 - I,
// T_(2k+1) = 2 T_k T_(k+1) - S).  Giant steps: Clenshaw's recurrence in y
// with matrix coefficients, B_j = a_j + 2 y B_(j+1) - B_(j+2), result
// a_0 + y B_1 - B_2; the a_j - B_(j+2) addends are formed by comb passes.
// Every product is of two polynomials in S, hence symmetric.
void plan_cheb_ps(Plan& P, const std::vector<double>& c) {
  const int d = (int)c.size() - 1;
  const int m = cheb_ps_step(d);
  const int J = d / m;
  std::vector<double> cc(c);
  std::vector<std::vector<double>> al(J + 1, std::vector<double>(m, 0.0));
  for (int k = d; k >= 0; --k) {
    const int j = k / m, i = k - j * m;
    if (j == 0 || i == 0) {
      al[j][i] += cc[k];
    } else {
      al[j][i] += 2.0 * cc[k];
      cc[m * j - i] -= cc[k];
    }
  }
  // baby steps: T[1] = S from the prep pass, T[k] for 2 <= k <= m
  std::vector<int> T(m + 1, -1);
  T[1] = P.get();
  P.prep(T[1], 2.0, -1.0);
  for (int k = 2; k <= m; ++k) {
    T[k] = P.get();
    if (k % 2 == 0) P.gemm(T[k / 2], T[k / 2], T[k], 2.0, -1.0);
    else P.gemm(T[k / 2], T[k / 2 + 1], T[k], 2.0, 0.0, T[1], -1.0);
  }
  const int y = T[m];
  const bool aJ_const = d % m == 0;
  if ((m - 1) + (aJ_const ? 1 : 0) <= MCOMB_IN && J + (aJ_const ? 0 : 1) <= MCOMB_OUT) {
    // Every a_j from one pass over T_1 .. T_(m-1) (and y): A[j] = a_j, with
    // the known multiples of I folded in.  With a_J = al[J][0] I constant,
    // A[J-1] is B_(J-1) = a_(J-1) + 2 al[J][0] y (or + al[J][0] y when J = 1,
    // the last step), and A[J-2] carries - B_J = - al[J][0] I.  Otherwise
    // A[J] = a_J = B_J.  The giant steps then need one in-place pass each,
    // A[j] - B_(j+2), before their product.
    std::vector<int> in;
    for (int i = 1; i < m; ++i) in.push_back(T[i]);
    if (aJ_const) in.push_back(y);
    const int nA = aJ_const ? J : J + 1;
    std::vector<int> A(nA);
    std::vector<std::vector<double>> w(nA, std::vector<double>(in.size(), 0.0));
    std::vector<double> g(nA, 0.0);
    for (int j = 0; j < nA; ++j) {
      A[j] = P.get();
      for (int i = 1; i < m; ++i) w[j][i - 1] = al[j][i];
      g[j] = al[j][0];
    }
    if (aJ_const) {
      w[J - 1][m - 1] = (J - 1 > 0 ? 2.0 : 1.0) * al[J][0];
      if (J >= 2) g[J - 2] -= al[J][0];
    }
    P.mcomb(in, A, w, g);
    for (int k = 1; k < m; ++k) P.put(T[k]);  // only y is multiplied from here on
    int B1 = aJ_const ? A[J - 1] : A[J];  // B_(j+1) for the first product
    int B2 = -1;                          // B_(j+2), once it is a matrix
    for (int j = aJ_const ? J - 2 : J - 1; j >= 0; --j) {
      if (B2 >= 0) P.comb(A[j], {{A[j], 1.0}, {B2, -1.0}}, 0.0);
      const int N = P.get();
      P.gemm(y, B1, N, j > 0 ? 2.0 : 1.0, 0.0, A[j], 1.0);
      P.put(A[j]);
      P.put(B2);
      B2 = B1;
      B1 = N;
    }
    P.put(y);
    P.put(B2);
    P.final_(B1);
    return;
  }
  // Too many terms for one pass: each addend is formed by chained comb passes.
  // The matrix terms of a_j (on T_1 .. T_(m-1)); its constant al[j][0] goes
  // into the comb's multiple of I
  auto a_terms = [&](int j) {
    std::vector<std::pair<int, double>> t;
    for (int i = 1; i < m; ++i) t.push_back({T[i], al[j][i]});
    return t;
  };
  // B_(j+1) and B_(j+2): a buffer, or (buffer -1) the scalar multiple of I in
  // sc1 / sc2 (B_J when a_J is constant), or absent (scalar 0)
  int B1 = -1, B2 = -1;
  double sc1 = 0.0, sc2 = 0.0;
  bool b1_mat = false;
  if (d % m == 0) {
    sc1 = al[J][0];
  } else {
    B1 = P.get();
    P.comb(B1, a_terms(J), al[J][0]);
    b1_mat = true;
  }
  for (int j = J - 1; j >= 0; --j) {
    const double two = j > 0 ? 2.0 : 1.0;  // the last step is a_0 + y B_1 - B_2
    std::vector<std::pair<int, double>> t = a_terms(j);
    double g = al[j][0] - sc2;
    if (B2 >= 0) t.push_back({B2, -1.0});
    const int N = P.get();
    if (!b1_mat) {
      // B_(j+1) = sc1 I: no product
      t.push_back({y, two * sc1});
      P.comb(N, t, g);
    } else {
      // the addend a_j - B_(j+2) goes into B_(j+2)'s buffer when there is one
      const int D = B2 >= 0 ? B2 : P.get();
      P.comb(D, t, g);
      P.gemm(y, B1, N, two, 0.0, D, 1.0);
      P.put(D);
      B2 = -1;
    }
    P.put(B2);
    B2 = B1;
    sc2 = b1_mat ? 0.0 : sc1;
    B1 = N;
    sc1 = 0.0;
    b1_mat = true;
  }
  for (int k = 1; k <= m; ++k) P.put(T[k]);
  P.put(B2);
  P.final_(B1);
}

// Chebyshev coefficients of x^(-1/p) on [eps, 1 + eps] ([DASH] "A.1/A.2"):
// N first-kind nodes t_j = cos(theta_j), theta_j = pi (j + 1/2) / N, mapped
// to x_j = (t_j + 1)/2 + eps; c_k = (2/N) sum_j f(x_j) cos(k theta_j), with
// c_0 halved (the least-squares fit at the nodes).
std::vector<double> cheb_coeffs(int p, int d, int N, double eps) {
  std::vector<double> c(d + 1, 0.0);
  std::vector<double> th(N), fx(N);
  for (int j = 0; j < N; ++j) {
    th[j] = M_PI * (j + 0.5) / N;
    const double x = 0.5 * (std::cos(th[j]) + 1.0) + eps;
    fx[j] = std::pow(x, -1.0 / p);
  }
  for (int k = 0; k <= d; ++k) {
    double s = 0.0;
    for (int j = 0; j < N; ++j) s += fx[j] * std::cos(k * th[j]);
    c[k] = 2.0 * s / N;
  }
  c[0] *= 0.5;
  return c;
}

bool pow2_in(int p, int maxp) {
  for (int q = 1; q <= maxp; q *= 2)
    if (q == p) return true;
  return false;
}

shampoo_status check_root_args(int64_t n, int32_t B, int32_t p, const shampoo_root_opts* o) {
  if (!o) return fail(SHAMPOO_E_INVALID, "opts is NULL");
  if (n < 0) return fail(SHAMPOO_E_INVALID, "n = %lld < 0", (long long)n);
  if (B < 64 || B % 64 != 0) return fail(SHAMPOO_E_UNSUPPORTED, "B = %d: must be a positive multiple of 64", B);
  // the launch limits of the call, here too so that a workspace query never
  // sizes (and overflows on) a batch the call would refuse
  if (n > 65535) return fail(SHAMPOO_E_UNSUPPORTED, "n = %lld > 65535: batch too large for one launch", (long long)n);
  if (p < 1) return fail(SHAMPOO_E_INVALID, "p = %d < 1", p);
  if (o->compute != SHAMPOO_F32 && o->compute != SHAMPOO_F16 && o->compute != SHAMPOO_F64)
    return fail(SHAMPOO_E_UNSUPPORTED, "compute dtype %d not supported (F32, F16, F64)", o->compute);
  if (!(o->eps >= 0.0) || !std::isfinite(o->eps)) return fail(SHAMPOO_E_INVALID, "eps must be finite and >= 0");
  if (!(o->tol >= 0.0) || !std::isfinite(o->tol)) return fail(SHAMPOO_E_INVALID, "tol must be finite and >= 0");
  if (!(o->residual_bound >= 0.0) || !std::isfinite(o->residual_bound))
    return fail(SHAMPOO_E_INVALID, "residual_bound must be finite and >= 0");
  if (o->tol > 0.0 && o->method == SHAMPOO_CHEBYSHEV)
    return fail(SHAMPOO_E_INVALID, "tol applies to the Newton iterations (CN, NDB), not to Chebyshev");
  switch (o->method) {
    case SHAMPOO_CN:
      if (!pow2_in(p, 8)) return fail(SHAMPOO_E_UNSUPPORTED, "coupled Newton supports p in {1, 2, 4, 8}, got %d", p);
      if (o->iters < 1) return fail(SHAMPOO_E_INVALID, "iters = %d < 1", o->iters);
      break;
    case SHAMPOO_NDB:
      if (p != 2 && p != 4) return fail(SHAMPOO_E_UNSUPPORTED, "Newton-DB supports p in {2, 4}, got %d", p);
      if (o->iters < 1) return fail(SHAMPOO_E_INVALID, "iters = %d < 1", o->iters);
      if (p == 4 && o->iters2 < 1) return fail(SHAMPOO_E_INVALID, "iters2 = %d < 1", o->iters2);
      break;
    case SHAMPOO_CHEBYSHEV: {
      if (o->cheb_degree < 0 || o->cheb_degree > 1000) return fail(SHAMPOO_E_INVALID, "cheb_degree = %d", o->cheb_degree);
      const int N = o->cheb_points ? o->cheb_points : 4 * (o->cheb_degree + 1);
      if (N <= o->cheb_degree) return fail(SHAMPOO_E_INVALID, "cheb_points = %d must exceed the degree", N);
      if (!(o->cheb_eps >= 0.0) || !std::isfinite(o->cheb_eps)) return fail(SHAMPOO_E_INVALID, "cheb_eps must be finite and >= 0");
      if (o->cheb_eval != SHAMPOO_CHEB_CLENSHAW && o->cheb_eval != SHAMPOO_CHEB_PS)
        return fail(SHAMPOO_E_INVALID, "cheb_eval = %d (CLENSHAW or PS)", o->cheb_eval);
      break;
    }
    default:
      return fail(SHAMPOO_E_INVALID, "unknown method %d", o->method);
  }
  if (o->scaling != SHAMPOO_SCALE_FROBENIUS && o->scaling != SHAMPOO_SCALE_POWER)
    return fail(SHAMPOO_E_INVALID, "unknown scaling %d", o->scaling);
  if (o->scaling == SHAMPOO_SCALE_POWER) {
    if (o->pi_vectors < 1 || o->pi_vectors > 32) return fail(SHAMPOO_E_INVALID, "pi_vectors = %d not in 1..32", o->pi_vectors);
    if (o->pi_iters < 1) return fail(SHAMPOO_E_INVALID, "pi_iters = %d < 1", o->pi_iters);
    const int k16 = (o->pi_vectors + 15) / 16 * 16;
    if ((int64_t)k16 * B > 16384)
      return fail(SHAMPOO_E_UNSUPPORTED, "power iteration needs ceil16(pi_vectors) * B <= 16384 (got %d * %d)", k16, B);
  }
  return SHAMPOO_OK;
}

// Which forms of every value the chain reads, by a backward scan: a product
// reads its operands as half (in half-operand chains) and its addend D in
// float32; the final pass reads float32.  A buffer written by an op holds a
// new value, so the needs gathered after it belong to that op's output.
// half: a half-operand chain, whose convergence checks read the half copy of
// the checked iterate (the copy later products read), so that a check does
// not add a float32 output to the product before it.
void mark_needs(Plan& P, bool half) {
  std::vector<int> need(P.peak > 0 ? P.peak : 1, 0);
  auto take = [&](int b) {
    const int v = need[b];
    need[b] = 0;
    return v;
  };
  for (auto it = P.ops.rbegin(); it != P.ops.rend(); ++it) {
    Op& op = *it;
    if (op.kind == OP_PREP) {
      for (int q = 0; q < 3; ++q)
        if (op.out[q] >= 0) op.need[q] = take(op.out[q]);
    } else if (op.kind == OP_GEMM) {
      op.need_c = take(op.c);
      if (op.c2 >= 0) op.need_c2 = take(op.c2);
      need[op.a] |= NEED_HALF;
      need[op.b] |= NEED_HALF;
      if (op.d >= 0) need[op.d] |= NEED_F32;
    } else if (op.kind == OP_COMB) {
      op.need_c = take(op.c);
      for (int q = 0; q < op.nin; ++q) need[op.in[q]] |= NEED_F32;
    } else if (op.kind == OP_MCOMB) {
      for (size_t j = 0; j < op.mout.size(); ++j) op.mneed[j] = take(op.mout[j]);
      for (int b : op.min) need[b] |= NEED_F32;
    } else if (op.kind == OP_CHECK) {
      need[op.a] |= half ? NEED_HALF : NEED_F32;
    } else {
      need[op.a] |= NEED_F32;
    }
  }
}

// The solver residual ||X^p A_s - I||_F / sqrt(v) is computed on request:
// A_s regenerated by a prep pass, X^p by repeated squaring (p a power of two)
// or repeated multiplication, then X^p A_s - I.  Three buffers besides X.
constexpr int RESID_BUFS = 3;
bool want_residual(const shampoo_root_opts* o) { return o->residual_out_dev != nullptr || o->residual_bound > 0.0; }

Plan build_plan(int32_t p, const shampoo_root_opts* o) {
  Plan P;
  switch (o->method) {
    case SHAMPOO_CN: plan_cn(P, p, o->iters, o->tol > 0.0); break;
    case SHAMPOO_NDB: plan_ndb(P, p, o->iters, o->iters2, o->tol > 0.0); break;
    default: {
      const int N = o->cheb_points ? o->cheb_points : 4 * (o->cheb_degree + 1);
      const int d = o->cheb_degree;
      if (o->cheb_eval == SHAMPOO_CHEB_PS && d >= 2 && cheb_ps_products(d, cheb_ps_step(d)) < d - 1)
        plan_cheb_ps(P, cheb_coeffs(p, d, N, o->cheb_eps));
      else
        plan_cheb(P, cheb_coeffs(p, d, N, o->cheb_eps));
    }
  }
  mark_needs(P, o->compute == SHAMPOO_F16);
  if (want_residual(o)) {
    // the residual products run after the chain, in any three buffers other
    // than the result, with the Frobenius scratch of the checks
    P.resid = true;
    P.checks = true;
    P.peak = std::max(P.peak, 1 + RESID_BUFS);
  }
  return P;
}

// One iterate buffer: float64 or float32 matrices; half-operand chains add a
// half copy of each matrix after the float32 part.
size_t root_slot_f32_bytes(int64_t n, int32_t B, int compute) {
  return align_up((size_t)n * B * B * (compute == SHAMPOO_F64 ? 8 : 4));
}
size_t root_slot_bytes(int64_t n, int32_t B, int compute) {
  return root_slot_f32_bytes(n, B, compute) + (compute == SHAMPOO_F16 ? align_up((size_t)n * B * B * 2) : 0);
}

// Frobenius partial sums per matrix: about 9216 workgroups in all, at most 32
// per matrix (288 float32 matrices of 1024^2: 15 parts 5.6 TB/s, 32 parts
// 6.3 TB/s on MI355X).
int frob_parts(int64_t n) {
  return n < 1 ? 1 : (int)std::max<int64_t>(1, std::min<int64_t>(32, (9216 + n - 1) / n));
}

// Convergence checks: partial sums, per-matrix norms and the flag, after the
// iterate buffers.
size_t check_bytes(int64_t n) { return align_up((size_t)frob_parts(n) * n * 8) + align_up((size_t)n * 8) + ALIGN; }

size_t root_ws_bytes(int64_t n, int32_t B, const Plan& P, int compute) {
  const int nbuf = P.peak > 1 ? P.peak : 1;  // the power iteration borrows one buffer
  return 2 * align_up((size_t)n * 8) + (size_t)nbuf * root_slot_bytes(n, B, compute) + (P.checks ? check_bytes(n) : 0);
}

// Benchmark timing of the batched products (shampoo_timing_enable).
struct Timing {
  std::vector<hipEvent_t> ev;  // 2 per launch
  int cap = 0;
  int used = 0;
} g_timing;

hipError_t timing_mark(int which, hipStream_t st) {
  if (g_timing.cap == 0 || g_timing.used >= g_timing.cap) return hipSuccess;
  return hipEventRecord(g_timing.ev[2 * g_timing.used + which], st);
}

void timing_advance() {
  if (g_timing.cap && g_timing.used < g_timing.cap) ++g_timing.used;
}

template <typename TI, typename TS>
hipError_t launch_prep(const void* in, int B, int64_t n, const int32_t* valid, double eps, const double* s,
                       double pad_diag, const PrepOut& o0, const PrepOut& o1, const PrepOut& o2,
                       hipStream_t st) {
  const int64_t chunks = (int64_t)B * B / 4;
  const unsigned gx = (unsigned)((chunks + 256 * PREP_U - 1) / (256 * PREP_U));
  hipLaunchKernelGGL((prep_kernel<TI, TS>), dim3(gx, (unsigned)n), dim3(256), 0, st, (const TI*)in, B, n, valid,
                     eps, s, pad_diag, o0, o1, o2);
  return hipGetLastError();
}

// keep_flagged: the final pass first only flags (NONFINITE, ZERO_SCALE; the
// residual pass before it sets RESIDUAL) and then writes just the matrices
// left unflagged, so a flagged matrix keeps the previous content of `out`
// (flags must then be non-null and start at 0).
template <typename TI, typename TS, Mma MM>
shampoo_status run_root(const void* in, void* out, int64_t n, int32_t B, int32_t p, const shampoo_root_opts* o,
                        const Plan& P, const int32_t* valid, float* scale_out, int32_t* flags, void* ws,
                        bool keep_flagged, hipStream_t st) {
  const int64_t BB = (int64_t)B * B;
  unsigned char* w = (unsigned char*)ws;
  double* sf = (double*)w;
  double* s = (double*)(w + align_up((size_t)n * 8));
  unsigned char* bufbase = w + 2 * align_up((size_t)n * 8);
  // Half-operand chains (f16): every product reads half operands, so a value
  // is stored as half where products read it and in float32 where it is an
  // addend or the result (Op::need); each buffer has room for both forms.
  constexpr bool HALF = MM == Mma::F16;
  const size_t slot32 = root_slot_f32_bytes(n, B, o->compute);
  const size_t bufstride = root_slot_bytes(n, B, o->compute);
  auto buf = [&](int i) -> TS* { return (TS*)(bufbase + (size_t)i * bufstride); };
  auto hbuf = [&](int i) -> _Float16* { return (_Float16*)(bufbase + (size_t)i * bufstride + slot32); };

  // Frobenius norms: P workgroups per matrix (frob_parts), partial sums in
  // the first iterate buffer, which prep overwrites afterwards.
  const int parts = frob_parts(n);
  hipLaunchKernelGGL((frob_partial_kernel<TI>), dim3((unsigned)parts, (unsigned)n), dim3(256), 0, st, (const TI*)in,
                     B, valid, o->eps, parts, (double*)buf(0));
  LAUNCH_CHECK("frob_partial");
  hipLaunchKernelGGL(frob_finish_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, (const double*)buf(0),
                     parts, n, sf);
  LAUNCH_CHECK("frob_finish");
  const double* sc = sf;
  if (o->scaling == SHAMPOO_SCALE_POWER) {
    if (!o->pi_start_dev) return fail(SHAMPOO_E_INVALID, "power scaling needs pi_start_dev");
    // Power iteration on (in + eps I)/s_F, scaling fused; its half-precision
    // copy of each scaled matrix lives in the first iterate buffer, which
    // the chain's prep overwrites afterwards.  Persistent: two workgroups
    // per CU walk the matrices.
    const int k16 = (o->pi_vectors + 15) / 16 * 16;
    const size_t lds = (size_t)k16 * (B + 8) * 2 + (size_t)k16 * (B + 4) * 4 + (size_t)k16 * 4;
    const void* pk = k16 == 16 ? (const void*)power_iter_fused_kernel<TI, 1> : (const void*)power_iter_fused_kernel<TI, 2>;
    HIP_TRY(hipFuncSetAttribute(pk, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds));
    int cus = 0;
    HIP_TRY(cu_count(&cus));
    // two workgroups per CU where LDS allows (B <= 512 with 16 vectors)
    const unsigned pgrid = (unsigned)std::min<int64_t>(n, (int64_t)std::max(1, cus) * 2);
    _Float16* hcopy = (_Float16*)buf(0);
    if (k16 == 16)
      hipLaunchKernelGGL((power_iter_fused_kernel<TI, 1>), dim3(pgrid), dim3(PI_THREADS), lds, st, (const TI*)in, B, n, valid,
                         o->eps, sf, o->pi_vectors, o->pi_iters, o->pi_start_dev, hcopy, s, flags);
    else
      hipLaunchKernelGGL((power_iter_fused_kernel<TI, 2>), dim3(pgrid), dim3(PI_THREADS), lds, st, (const TI*)in, B, n, valid,
                         o->eps, sf, o->pi_vectors, o->pi_iters, o->pi_start_dev, hcopy, s, flags);
    LAUNCH_CHECK("power_iter");
    sc = s;
  }
  // convergence checks (Newton tolerance) and the solver residual: scratch
  // after the iterate buffers for the Frobenius partial sums, the per-matrix
  // norms and a flag that the host reads back
  unsigned char* chk = bufbase + (size_t)(P.peak > 1 ? P.peak : 1) * bufstride;
  double* cpart = (double*)chk;
  double* cnorm = (double*)(chk + align_up((size_t)parts * n * 8));
  int32_t* notdone = (int32_t*)(chk + align_up((size_t)parts * n * 8) + align_up((size_t)n * 8));
  // Solver residual of the chain result in buffer x: A_s regenerated from the
  // input, X^p by repeated squaring (p a power of two) or multiplication,
  // R = X^p A_s - I, all full products in the iterate precision (the float32
  // part of half-operand chains); then ||R||_F / sqrt(v) and the flag.
  auto residual = [&](int x) -> shampoo_status {
    int fb[RESID_BUFS], nfb = 0;
    for (int i = 0; i < std::max(P.peak, 1) && nfb < RESID_BUFS; ++i)
      if (i != x) fb[nfb++] = i;
    if (nfb < RESID_BUFS) return fail(SHAMPOO_E_INVALID, "internal: residual buffers");
    const int As = fb[0], t0 = fb[1], t1 = fb[2];
    const PrepOut q0{buf(As), 1.0, 0.0, nullptr}, none{nullptr, 0.0, 0.0, nullptr};
    HIP_TRY((launch_prep<TI, TS>(in, B, n, valid, o->eps, sc, 1.0, q0, none, none, st)));
    constexpr Mma RM = std::is_same<TS, double>::value ? Mma::F64 : Mma::F32;
    auto mul = [&](int a, int b, int c, double gamma) -> hipError_t {
      GemmCall g;
      g.A = buf(a);
      g.B = buf(b);
      g.C = buf(c);
      g.sym = false;
      g.nn = true;
      g.gamma = gamma;
      return gemm<RM, TS, TS, TS>(g, B, n, st);
    };
    // squarings of an exactly symmetric X (every chain but Newton-DB's,
    // whose products are full and whose result is symmetrised only by the
    // final pass) run as symmetric products: (X X)_ij and (X X)_ji then sum
    // the same terms in the same order, so the mirrored upper triangle has
    // the bits the full product would give, at 10 / 16 or 36 / 64 of its
    // work
    auto square = [&](int a, int c) -> hipError_t {
      if (P.sym_out) return mul(a, a, c, 0.0);
      GemmCall g;
      g.A = buf(a);
      g.B = buf(a);
      g.C = buf(c);
      g.sym = true;
      g.nn = false;
      return gemm<RM, TS, TS, TS>(g, B, n, st);
    };
    int cur = x;
    auto other = [&]() { return cur == t0 ? t1 : t0; };
    if ((p & (p - 1)) == 0) {
      for (int q = 1; q < p; q *= 2) {
        const int t = other();
        HIP_TRY(square(cur, t));
        cur = t;
      }
    } else {
      for (int q = 1; q < p; ++q) {
        const int t = other();
        HIP_TRY(mul(cur, x, t, 0.0));
        cur = t;
      }
    }
    const int R = other();
    HIP_TRY(mul(cur, As, R, -1.0));
    hipLaunchKernelGGL((frob_partial_kernel<TS>), dim3((unsigned)parts, (unsigned)n), dim3(256), 0, st,
                       (const TS*)buf(R), B, valid, 0.0, parts, cpart);
    LAUNCH_CHECK("frob_partial");
    hipLaunchKernelGGL(frob_finish_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, (const double*)cpart,
                       parts, n, cnorm);
    LAUNCH_CHECK("frob_finish");
    hipLaunchKernelGGL(residual_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, (const double*)cnorm, sc,
                       valid, n, B, o->residual_bound, o->residual_out_dev, flags);
    LAUNCH_CHECK("residual");
    return SHAMPOO_OK;
  };
  auto exec = [&](const Op& op) -> shampoo_status {
    if (op.kind == OP_PREP) {
      PrepOut q[3];
      for (int i = 0; i < 3; ++i) {
        q[i] = PrepOut{nullptr, op.oa[i], op.og[i], nullptr};
        if (op.out[i] < 0) continue;
        if (!HALF || (op.need[i] & NEED_F32)) q[i].p = buf(op.out[i]);
        if (HALF && (op.need[i] & NEED_HALF)) q[i].ph = hbuf(op.out[i]);
      }
      HIP_TRY((launch_prep<TI, TS>(in, B, n, valid, o->eps, sc, 1.0, q[0], q[1], q[2], st)));
    } else if (op.kind == OP_GEMM) {
      GemmCall c;
      c.D = op.d >= 0 ? buf(op.d) : nullptr;
      c.alpha = op.alpha; c.beta = op.beta; c.gamma = op.gamma; c.alpha2 = op.alpha2; c.gamma2 = op.gamma2;
      c.sym = !op.nn;
      c.nn = op.nn;
      HIP_TRY(timing_mark(0, st));
      if constexpr (HALF) {
        c.A = hbuf(op.a);
        c.B = hbuf(op.b);
        if (op.need_c & NEED_F32) c.C = buf(op.c);
        if (op.need_c & NEED_HALF) c.Ch = hbuf(op.c);
        if (op.c2 >= 0 && (op.need_c2 & NEED_F32)) c.C2 = buf(op.c2);
        if (op.c2 >= 0 && (op.need_c2 & NEED_HALF)) c.C2h = hbuf(op.c2);
        HIP_TRY((gemm<MM, _Float16, _Float16, TS>(c, B, n, st)));
      } else {
        c.A = buf(op.a);
        c.B = buf(op.b);
        c.C = buf(op.c);
        c.C2 = op.c2 >= 0 ? buf(op.c2) : nullptr;
        HIP_TRY((gemm<MM, TS, TS, TS>(c, B, n, st)));
      }
      HIP_TRY(timing_mark(1, st));
      timing_advance();
    } else if (op.kind == OP_MCOMB) {
      MCombArgs ma{};
      ma.nin = (int)op.min.size();
      ma.nout = (int)op.mout.size();
      for (int q = 0; q < ma.nin; ++q) ma.in[q] = buf(op.min[q]);
      for (int j = 0; j < ma.nout; ++j) {
        if (!HALF || (op.mneed[j] & NEED_F32)) ma.out[j] = buf(op.mout[j]);
        if (HALF && (op.mneed[j] & NEED_HALF)) ma.outh[j] = hbuf(op.mout[j]);
        for (int q = 0; q < ma.nin; ++q) ma.w[j][q] = op.mw[j][q];
        ma.gamma[j] = op.mg[j];
      }
      const unsigned gx = (unsigned)(((int64_t)B * B / 4 + 255) / 256);
      hipLaunchKernelGGL((mcomb_kernel<TS>), dim3(gx, (unsigned)n), dim3(256), 0, st, ma, B);
      LAUNCH_CHECK("mcomb");
    } else if (op.kind == OP_COMB) {
      CombArgs ca{};
      for (int q = 0; q < op.nin; ++q) {
        ca.in[q] = buf(op.in[q]);
        ca.w[q] = op.w[q];
      }
      ca.nin = op.nin;
      ca.gamma = op.gamma;
      if (!HALF || (op.need_c & NEED_F32)) ca.out = buf(op.c);
      if (HALF && (op.need_c & NEED_HALF)) ca.outh = hbuf(op.c);
      const unsigned gx = (unsigned)(((int64_t)B * B / 4 + 256 * PREP_U - 1) / (256 * PREP_U));
      hipLaunchKernelGGL((comb_kernel<TS>), dim3(gx, (unsigned)n), dim3(256), 0, st, ca, B);
      LAUNCH_CHECK("comb");
    } else {
      if (P.resid) {
        shampoo_status rr = residual(op.a);
        if (rr != SHAMPOO_OK) return rr;
      }
      const int tps = B / 64;
      const dim3 fgrid((unsigned)(tps * tps), (unsigned)n);
      const int sym = P.sym_out ? 1 : 0;
      if (keep_flagged) {
        hipLaunchKernelGGL((finalize_kernel<TS, TI>), fgrid, dim3(256), 0, st, buf(op.a), (TI*)out, B, valid, sc,
                           1.0 / p, sym, scale_out, flags, (int)FIN_CHECK);
        LAUNCH_CHECK("finalize");
        hipLaunchKernelGGL((finalize_kernel<TS, TI>), fgrid, dim3(256), 0, st, buf(op.a), (TI*)out, B, valid, sc,
                           1.0 / p, sym, scale_out, flags, (int)FIN_COMMIT);
      } else {
        hipLaunchKernelGGL((finalize_kernel<TS, TI>), fgrid, dim3(256), 0, st, buf(op.a), (TI*)out, B, valid, sc,
                           1.0 / p, sym, scale_out, flags, (int)FIN_WRITE);
      }
      LAUNCH_CHECK("finalize");
    }
      return SHAMPOO_OK;
  };
  // Newton-DB re-plans at convergence: `cur` is the plan being run, `gemms`
  // the products run so far, used1 the iterations of call 1 once it ended
  const Plan* cur = &P;
  Plan replanned;
  int gemms = 0, used1 = o->iters;
  for (size_t oi = 0; oi < cur->ops.size(); ++oi) {
    const Op& op = cur->ops[oi];
    if (op.kind != OP_CHECK) {
      shampoo_status r = exec(op);
      if (r != SHAMPOO_OK) return r;
      if (op.kind == OP_GEMM) ++gemms;
      continue;
    }
    // first the diagonal alone: a trace beyond tol settles "not converged"
    // without the Frobenius pass (same decision, a B-th of the reads)
    hipLaunchKernelGGL(fill_i32_kernel, dim3(1), dim3(64), 0, st, notdone, (int64_t)1, 0);
    LAUNCH_CHECK("fill");
    if constexpr (HALF)
      hipLaunchKernelGGL((trace_gap_kernel<_Float16>), dim3((unsigned)n), dim3(256), 0, st,
                         (const _Float16*)hbuf(op.a), B, valid, sc, o->tol * op.alpha, notdone);
    else
      hipLaunchKernelGGL((trace_gap_kernel<TS>), dim3((unsigned)n), dim3(256), 0, st, (const TS*)buf(op.a), B,
                         valid, sc, o->tol * op.alpha, notdone);
    LAUNCH_CHECK("trace_gap");
    {
      int32_t h = 0;
      HIP_TRY(hipMemcpyAsync(&h, notdone, 4, hipMemcpyDeviceToHost, st));
      HIP_TRY(hipStreamSynchronize(st));
      if (h != 0) continue;
    }
    // ||M - I||_F: the Frobenius sums of M + eps I with eps = -1 (half
    // chains: of the half copy that the next products read)
    if constexpr (HALF)
      hipLaunchKernelGGL((frob_partial_kernel<_Float16>), dim3((unsigned)parts, (unsigned)n), dim3(256), 0, st,
                         (const _Float16*)hbuf(op.a), B, valid, -1.0, parts, cpart);
    else
      hipLaunchKernelGGL((frob_partial_kernel<TS>), dim3((unsigned)parts, (unsigned)n), dim3(256), 0, st,
                         (const TS*)buf(op.a), B, valid, -1.0, parts, cpart);
    LAUNCH_CHECK("frob_partial");
    hipLaunchKernelGGL(frob_finish_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, (const double*)cpart,
                       parts, n, cnorm);
    LAUNCH_CHECK("frob_finish");
    hipLaunchKernelGGL(fill_i32_kernel, dim3(1), dim3(64), 0, st, notdone, (int64_t)1, 0);
    LAUNCH_CHECK("fill");
    hipLaunchKernelGGL(above_tol_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, (const double*)cnorm, sc,
                       n, o->tol * op.alpha, notdone);
    LAUNCH_CHECK("above_tol");
    int32_t h = 1;
    HIP_TRY(hipMemcpyAsync(&h, notdone, 4, hipMemcpyDeviceToHost, st));
    HIP_TRY(hipStreamSynchronize(st));
    if (h != 0) continue;
    if (op.b == 0) {
      // coupled Newton has converged: the next op (X T) is X's last update
      if (oi + 1 >= cur->ops.size() || cur->ops[oi + 1].kind != OP_GEMM || cur->ops.back().kind != OP_FINAL)
        return fail(SHAMPOO_E_INVALID, "internal: convergence check placement");
      // it was planned with the outputs a later iteration reads: in a half
      // chain only the half copy; the final pass reads the float32 result
      Op last = cur->ops[oi + 1];
      last.need_c = NEED_F32;
      shampoo_status r = exec(last);
      if (r != SHAMPOO_OK) return r;
      Op fin = cur->ops.back();
      fin.a = cur->ops[oi + 1].c;
      return exec(fin);
    }
    // Newton-DB call op.b has converged at iteration op.c: continue in the
    // plan where that call ends there, after its gemms-th product
    const int it1 = op.b == 1 ? op.c : used1, it2 = op.b == 2 ? op.c : o->iters2;
    if (op.b == 1) used1 = op.c;
    Plan next;
    plan_ndb(next, p, it1, it2, true);
    mark_needs(next, HALF);
    if (next.peak > P.peak) return fail(SHAMPOO_E_INVALID, "internal: re-planned chain needs more buffers");
    size_t j = 0;
    for (int g = 0; j < next.ops.size(); ++j)
      if (next.ops[j].kind == OP_GEMM && ++g == gemms) break;
    if (j >= next.ops.size()) return fail(SHAMPOO_E_INVALID, "internal: re-planned chain is shorter");
    replanned = std::move(next);
    cur = &replanned;
    oi = j;  // the loop's ++oi moves to the op after that product
    if (oi + 1 < cur->ops.size() && cur->ops[oi + 1].kind == OP_CHECK) ++oi;  // already checked
  }
  return SHAMPOO_OK;
}

shampoo_status inverse_root_impl(const void* in, void* out, shampoo_dtype io_dt, int64_t n, int32_t B, int32_t p,
                                 const shampoo_root_opts* o, const int32_t* valid, float* scale_out,
                                 int32_t* flags, void* ws, size_t ws_bytes, hipStream_t st,
                                 bool keep_flagged = false) {
  shampoo_status r = check_root_args(n, B, p, o);
  if (r != SHAMPOO_OK) return r;
  if (io_dt != SHAMPOO_F32 && io_dt != SHAMPOO_F64)
    return fail(SHAMPOO_E_UNSUPPORTED, "io dtype %d not supported (F32, F64)", (int)io_dt);
  if (n == 0) return SHAMPOO_OK;
  if (!in || !out) return fail(SHAMPOO_E_INVALID, "in/out is NULL");
  if (o->scaling == SHAMPOO_SCALE_POWER && !o->pi_start_dev)
    return fail(SHAMPOO_E_INVALID, "power scaling needs pi_start_dev");
  if (gemm_wgs(B, n, false) >= (int64_t)1 << 31 || n > 65535)
    return fail(SHAMPOO_E_UNSUPPORTED, "batch too large for one launch");
  const Plan P = build_plan(p, o);
  const size_t need = root_ws_bytes(n, B, P, o->compute);
  if (!ws || ws_bytes < need)
    return fail(SHAMPOO_E_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
  const bool in64 = io_dt == SHAMPOO_F64;
  switch (o->compute) {
    case SHAMPOO_F32:
      return in64 ? run_root<double, float, Mma::F32>(in, out, n, B, p, o, P, valid, scale_out, flags, ws, keep_flagged, st)
                  : run_root<float, float, Mma::F32>(in, out, n, B, p, o, P, valid, scale_out, flags, ws, keep_flagged, st);
    case SHAMPOO_F16:
      return in64 ? run_root<double, float, Mma::F16>(in, out, n, B, p, o, P, valid, scale_out, flags, ws, keep_flagged, st)
                  : run_root<float, float, Mma::F16>(in, out, n, B, p, o, P, valid, scale_out, flags, ws, keep_flagged, st);
    default:
      return in64 ? run_root<double, double, Mma::F64>(in, out, n, B, p, o, P, valid, scale_out, flags, ws, keep_flagged, st)
                  : run_root<float, double, Mma::F64>(in, out, n, B, p, o, P, valid, scale_out, flags, ws, keep_flagged, st);
  }
}

// ---------------------------------------------------------------------------
// Allocation-free inverse roots: the workspace lives in a file-scope device
// array (one copy per device, held until the process ends).  Host code never
// passes the array's name to a kernel or a copy: in host code it stands for a
// host-side shadow, not a device address.  Each device's address comes from
// hipGetSymbolAddress, taken once per device with that device current.
// ---------------------------------------------------------------------------
constexpr size_t NOALLOC_SCRATCH_BYTES = size_t(64) << 20;
__device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

hipError_t noalloc_scratch(void** ptr) {
  static void* addr[MAX_DEVICES] = {nullptr};
  static std::mutex mu;
  int dev = 0;
  HIP_TRY_ERR(hipGetDevice(&dev));
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    HIP_TRY_ERR(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

shampoo_status inverse_root_noalloc_impl(const void* in, void* out, shampoo_dtype io_dt, int64_t n, int32_t B,
                                         int32_t p, const shampoo_root_opts* o, const int32_t* valid,
                                         float* scale_out, int32_t* flags, hipStream_t st) {
  shampoo_status r = check_root_args(n, B, p, o);
  if (r != SHAMPOO_OK) return r;
  const size_t need = root_ws_bytes(n, B, build_plan(p, o), o->compute);
  if (need > NOALLOC_SCRATCH_BYTES)
    return fail(SHAMPOO_E_WORKSPACE,
                "these arguments need %zu bytes of scratch; the allocation-free entry point holds %zu (use "
                "shampoo_inverse_root with a workspace)", need, NOALLOC_SCRATCH_BYTES);
  if (n == 0) return inverse_root_impl(in, out, io_dt, n, B, p, o, valid, scale_out, flags, nullptr, 0, st);
  void* ws = nullptr;
  HIP_TRY(noalloc_scratch(&ws));
  return inverse_root_impl(in, out, io_dt, n, B, p, o, valid, scale_out, flags, ws, NOALLOC_SCRATCH_BYTES, st);
}

// ---------------------------------------------------------------------------
// pack, statistics, preconditioning
// ---------------------------------------------------------------------------
template <typename E>
hipError_t launch_pack(const shampoo_matrix* mats, int nparams, const shampoo_block* table, int64_t nblk, int B, void* stack,
                       void* stack_t, hipStream_t st) {
  const int tps = (B + 63) / 64;
  dim3 grid((unsigned)(tps * tps), (unsigned)nblk);
  hipLaunchKernelGGL((pack_kernel<E, shampoo_matrix>), grid, dim3(256), 0, st, mats, nparams, table, B, tps,
                     (E*)stack, (E*)stack_t);
  return hipGetLastError();
}

shampoo_status pack_impl(const shampoo_matrix* mats, int32_t nparams, const shampoo_block* table, int64_t nblk,
                         int32_t B, shampoo_dtype dt, void* stack, void* stack_t, hipStream_t st) {
  if (nblk < 0 || B < 1 || nparams < 0) return fail(SHAMPOO_E_INVALID, "bad sizes nblk=%lld B=%d", (long long)nblk, B);
  if (nblk == 0) return SHAMPOO_OK;
  if (!mats || !table || !stack) return fail(SHAMPOO_E_INVALID, "null pointer argument");
  if (nblk > 65535) return fail(SHAMPOO_E_UNSUPPORTED, "nblk = %lld > 65535", (long long)nblk);
  switch (dt) {
    case SHAMPOO_F32: HIP_TRY(launch_pack<uint32_t>(mats, nparams, table, nblk, B, stack, stack_t, st)); break;
    case SHAMPOO_F16:
    case SHAMPOO_BF16: HIP_TRY(launch_pack<uint16_t>(mats, nparams, table, nblk, B, stack, stack_t, st)); break;
    case SHAMPOO_F64: HIP_TRY(launch_pack<uint64_t>(mats, nparams, table, nblk, B, stack, stack_t, st)); break;
    default: return fail(SHAMPOO_E_INVALID, "unknown dtype %d", (int)dt);
  }
  return SHAMPOO_OK;
}

// Work-balanced tile lists of the four products with extents (statistics L
// and R, preconditioning E^T and D), built on the device by tile_list_kernel.
struct ProductTiles {
  const int32_t* tiles[4] = {nullptr, nullptr, nullptr, nullptr};
  const int32_t* cut[4] = {nullptr, nullptr, nullptr, nullptr};
  int T = 64;  // tile side of the lists
};

shampoo_status stats_impl(const void* g, const void* gt, shampoo_dtype gdt, int64_t nblk, int32_t B, void* LR,
                          shampoo_dtype sdt, double beta2, hipStream_t st, const int32_t* valid = nullptr,
                          const ProductTiles* pt = nullptr) {
  if (nblk < 0) return fail(SHAMPOO_E_INVALID, "nblk < 0");
  if (B < 64 || B % 64 != 0) return fail(SHAMPOO_E_UNSUPPORTED, "B = %d: must be a positive multiple of 64", B);
  if (!(beta2 >= 0.0 && beta2 <= 1.0)) return fail(SHAMPOO_E_INVALID, "beta2 = %g not in [0, 1]", beta2);
  if (gdt != SHAMPOO_F32 && gdt != SHAMPOO_BF16) return fail(SHAMPOO_E_UNSUPPORTED, "gradient dtype %d (F32, BF16)", (int)gdt);
  if (sdt != SHAMPOO_F32 && sdt != SHAMPOO_F64) return fail(SHAMPOO_E_UNSUPPORTED, "statistics dtype %d (F32, F64)", (int)sdt);
  if (nblk == 0) return SHAMPOO_OK;
  if (!g || !gt || !LR) return fail(SHAMPOO_E_INVALID, "null pointer argument");
  if (nblk > 65535 || gemm_wgs(B, nblk, true) >= (int64_t)1 << 31) return fail(SHAMPOO_E_UNSUPPORTED, "batch too large");
  const double a = beta2 == 1.0 ? 1.0 : 1.0 - beta2;
  const double b = beta2;
  const size_t half = (size_t)nblk * B * B * (sdt == SHAMPOO_F64 ? 8 : 4);
  // L = beta2 L + (1 - beta2) G G^T and R from G^T, both as symmetric NT products in place
  GemmCall cl;
  cl.A = g; cl.B = g; cl.D = LR; cl.C = LR; cl.C2 = nullptr; cl.alpha = a; cl.beta = b; cl.sym = true;
  GemmCall cr = cl;
  cr.A = gt; cr.B = gt; cr.D = (unsigned char*)LR + half; cr.C = (unsigned char*)LR + half;
  // With the blocks' valid sizes (rows in valid[0, nblk), columns in
  // valid[nblk, 2 nblk)), each product covers only the block's valid region:
  // L (rows x rows) sums over G's columns, R (cols x cols) over its rows;
  // tiles past the valid side are not computed (their zeros stay).
  if (valid) {
    cl.rext = cl.cext = valid;
    cl.kext = valid + nblk;
    cr.rext = cr.cext = valid + nblk;
    cr.kext = valid;
    if (pt) {
      cl.tiles = pt->tiles[0];
      cl.cut = pt->cut[0];
      cr.tiles = pt->tiles[1];
      cr.cut = pt->cut[1];
      cl.tile = cr.tile = pt->T;
    }
  }
  if (sdt == SHAMPOO_F64) {
    if (gdt == SHAMPOO_F32) {
      HIP_TRY((gemm<Mma::F64, float, float, double>(cl, B, nblk, st)));
      HIP_TRY((gemm<Mma::F64, float, float, double>(cr, B, nblk, st)));
    } else {
      HIP_TRY((gemm<Mma::F64, __bf16, __bf16, double>(cl, B, nblk, st)));
      HIP_TRY((gemm<Mma::F64, __bf16, __bf16, double>(cr, B, nblk, st)));
    }
  } else if (gdt == SHAMPOO_F32) {
    HIP_TRY((gemm<Mma::F32, float, float, float>(cl, B, nblk, st)));
    HIP_TRY((gemm<Mma::F32, float, float, float>(cr, B, nblk, st)));
  } else {
    HIP_TRY((gemm<Mma::BF16, __bf16, __bf16, float>(cl, B, nblk, st)));
    HIP_TRY((gemm<Mma::BF16, __bf16, __bf16, float>(cr, B, nblk, st)));
  }
  return SHAMPOO_OK;
}

shampoo_status precond_impl(const void* roots, shampoo_dtype rdt, const void* g, shampoo_dtype gdt, int64_t nblk,
                            int32_t B, float* dstack, void* ws, size_t ws_bytes, hipStream_t st,
                            const int32_t* valid = nullptr, const ProductTiles* pt = nullptr) {
  if (nblk < 0) return fail(SHAMPOO_E_INVALID, "nblk < 0");
  if (B < 64 || B % 64 != 0) return fail(SHAMPOO_E_UNSUPPORTED, "B = %d: must be a positive multiple of 64", B);
  if (gdt != SHAMPOO_F32 && gdt != SHAMPOO_BF16) return fail(SHAMPOO_E_UNSUPPORTED, "gradient dtype %d (F32, BF16)", (int)gdt);
  if (rdt != SHAMPOO_F32 && rdt != SHAMPOO_F64) return fail(SHAMPOO_E_UNSUPPORTED, "roots dtype %d (F32, F64)", (int)rdt);
  if (nblk == 0) return SHAMPOO_OK;
  if (!roots || !g || !dstack) return fail(SHAMPOO_E_INVALID, "null pointer argument");
  const size_t es = rdt == SHAMPOO_F64 ? 8 : 4;
  const size_t need = (size_t)nblk * B * B * es;
  if (!ws || ws_bytes < need) return fail(SHAMPOO_E_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
  if (nblk > 65535 || gemm_wgs(B, nblk, false) >= (int64_t)1 << 31)
    return fail(SHAMPOO_E_UNSUPPORTED, "batch too large");
  const void* Lr = roots;
  const void* Rr = (const unsigned char*)roots + (size_t)nblk * B * B * es;
  // E = G Rr, stored transposed; D = Lr E = Lr (E^T)^T.
  GemmCall c1;
  c1.A = g; c1.B = Rr; c1.D = nullptr; c1.C = ws; c1.C2 = nullptr; c1.sym = false; c1.transC = true;
  GemmCall c2;
  c2.A = Lr; c2.B = ws; c2.D = nullptr; c2.C = dstack; c2.C2 = nullptr; c2.sym = false;
  // With the blocks' valid sizes, both products cover only the rows x cols
  // valid region of E and D (inner extents cols and rows); the roots' and
  // G's zero padding makes the partial tiles at the edges exact.
  if (valid) {
    c1.rext = c2.rext = valid;
    c1.cext = c2.cext = valid + nblk;
    c1.kext = valid + nblk;
    c2.kext = valid;
    if (pt) {
      c1.tiles = pt->tiles[2];
      c1.cut = pt->cut[2];
      c2.tiles = pt->tiles[3];
      c2.cut = pt->cut[3];
      c1.tile = c2.tile = pt->T;
    }
  }
  if (rdt == SHAMPOO_F64) {
    if (gdt == SHAMPOO_F32) HIP_TRY((gemm<Mma::F64, float, double, double>(c1, B, nblk, st)));
    else HIP_TRY((gemm<Mma::F64, __bf16, double, double>(c1, B, nblk, st)));
    HIP_TRY((gemm<Mma::F64, double, double, float>(c2, B, nblk, st)));
  } else {
    if (gdt == SHAMPOO_F32) HIP_TRY((gemm<Mma::F32, float, float, float>(c1, B, nblk, st)));
    else HIP_TRY((gemm<Mma::F32, __bf16, float, float>(c1, B, nblk, st)));
    HIP_TRY((gemm<Mma::F32, float, float, float>(c2, B, nblk, st)));
  }
  return SHAMPOO_OK;
}

// Preconditioning on bfloat16 matrix cores (step option precond_dt = BF16,
// bfloat16 gradients, float32 roots): both roots are rounded to bfloat16, E =
// G Rr is formed (float32 accumulation, stored transposed) and rounded to
// bfloat16, and D = Lr E is accumulated and stored in float32.  ws holds
// E^T in float32, then in bfloat16, then the bfloat16 roots
// (precond_bf16_bytes).  Extents and tile lists as in precond_impl.
size_t precond_bf16_bytes(int64_t nblk, int32_t B) {
  const size_t BB = (size_t)B * B;
  return align_up((size_t)nblk * BB * 4) + align_up((size_t)nblk * BB * 2) + align_up((size_t)nblk * 2 * BB * 2);
}

shampoo_status precond_bf16_impl(const float* roots, const void* g, int64_t nblk, int32_t B, float* dstack,
                                 unsigned char* ws, hipStream_t st, const int32_t* valid, const ProductTiles* pt) {
  if (nblk == 0) return SHAMPOO_OK;
  const size_t BB = (size_t)B * B;
  float* Et = (float*)ws;
  __bf16* Etb = (__bf16*)(ws + align_up((size_t)nblk * BB * 4));
  __bf16* rb = (__bf16*)(ws + align_up((size_t)nblk * BB * 4) + align_up((size_t)nblk * BB * 2));
  auto to_bf16 = [&](const float* in, __bf16* out, int64_t count) -> shampoo_status {
    const int64_t n4 = count / 4;  // B is a multiple of 64
    const int64_t wgs = std::min<int64_t>((n4 + 255) / 256, 8192);
    hipLaunchKernelGGL(f32_to_bf16_kernel, dim3((unsigned)std::max<int64_t>(wgs, 1)), dim3(256), 0, st, in, out, n4);
    LAUNCH_CHECK("f32_to_bf16");
    return SHAMPOO_OK;
  };
  shampoo_status r = to_bf16(roots, rb, 2 * nblk * (int64_t)BB);
  if (r != SHAMPOO_OK) return r;
  GemmCall c1;
  c1.A = g; c1.B = rb + nblk * BB; c1.D = nullptr; c1.C = Et; c1.C2 = nullptr; c1.sym = false; c1.transC = true;
  GemmCall c2;
  c2.A = rb; c2.B = Etb; c2.D = nullptr; c2.C = dstack; c2.C2 = nullptr; c2.sym = false;
  if (valid) {
    c1.rext = c2.rext = valid;
    c1.cext = c2.cext = valid + nblk;
    c1.kext = valid + nblk;
    c2.kext = valid;
    if (pt && pt->T == 64) {
      c1.tiles = pt->tiles[2];
      c1.cut = pt->cut[2];
      c2.tiles = pt->tiles[3];
      c2.cut = pt->cut[3];
      c1.tile = c2.tile = 64;
    }
  }
  HIP_TRY((gemm<Mma::BF16, __bf16, __bf16, float>(c1, B, nblk, st)));
  r = to_bf16(Et, Etb, nblk * (int64_t)BB);
  if (r != SHAMPOO_OK) return r;
  HIP_TRY((gemm<Mma::BF16, __bf16, __bf16, float>(c2, B, nblk, st)));
  return SHAMPOO_OK;
}

// ---------------------------------------------------------------------------
// step
// ---------------------------------------------------------------------------
struct StepLayout {
  size_t g, gt, valid, root, partials, scales, total;
  size_t root_bytes;
  int nchunk;
  // fallback: this step's factor flags; for FALLBACK_F64 the compacted
  // factors (indices, valid sizes, flags, inputs, roots) and their float64
  // chain workspace
  size_t fl, fidx, fvalid, fflags, fin, fout, froot;
  size_t froot_bytes;
  bool redo64;
  // some block is narrower than B (from table_host): the statistics and
  // preconditioning products then skip the padding of each block
  bool ragged;
  size_t tl;        // the four product tile lists (ragged only)
  size_t tl_each;   // bytes per list
  // factor-side groups (table_host given and some factor narrower than B):
  // group g roots gcount[g] factors, listed in gorder from gstart[g], in a
  // stack of side gside[g]; their chains use the root region
  std::vector<int> gside;
  std::vector<int64_t> gstart, gcount;
  std::vector<int32_t> gorder;
  size_t gidx, gvalid, gflags, gres, gin, gout;
};

shampoo_status step_layout(const shampoo_step_args* a, StepLayout* L) {
  if (!a) return fail(SHAMPOO_E_INVALID, "args is NULL");
  if (a->nblk < 0 || a->nparams < 0) return fail(SHAMPOO_E_INVALID, "negative sizes");
  if (a->B < 64 || a->B % 64 != 0) return fail(SHAMPOO_E_UNSUPPORTED, "B = %d: must be a positive multiple of 64", a->B);
  if (a->g_dt != SHAMPOO_F32 && a->g_dt != SHAMPOO_BF16) return fail(SHAMPOO_E_UNSUPPORTED, "gradient dtype %d", (int)a->g_dt);
  if (a->nblk > 32767) return fail(SHAMPOO_E_UNSUPPORTED, "nblk = %lld > 32767", (long long)a->nblk);
  if (a->stats_dt != SHAMPOO_F32 && a->stats_dt != SHAMPOO_F64)
    return fail(SHAMPOO_E_UNSUPPORTED, "statistics dtype %d (F32, F64)", (int)a->stats_dt);
  if (a->fallback < SHAMPOO_FALLBACK_NONE || a->fallback > SHAMPOO_FALLBACK_F64)
    return fail(SHAMPOO_E_INVALID, "unknown fallback %d", a->fallback);
  if (a->precond_dt != SHAMPOO_F32 && a->precond_dt != SHAMPOO_BF16)
    return fail(SHAMPOO_E_UNSUPPORTED, "precondition dtype %d (F32, BF16)", (int)a->precond_dt);
  if (a->precond_dt == SHAMPOO_BF16 && (a->g_dt != SHAMPOO_BF16 || a->stats_dt != SHAMPOO_F32))
    return fail(SHAMPOO_E_UNSUPPORTED, "bfloat16 preconditioning needs bfloat16 gradients and float32 statistics");
  shampoo_status r = check_root_args(2 * a->nblk, a->B, a->p, &a->root);
  if (r != SHAMPOO_OK) return r;
  const Plan P = build_plan(a->p, &a->root);
  const int64_t BB = (int64_t)a->B * a->B;
  const size_t es = dtype_size(a->g_dt);
  L->nchunk = (a->B + GRAFT_ROWS - 1) / GRAFT_ROWS;
  L->root_bytes = root_ws_bytes(2 * a->nblk, a->B, P, a->root.compute);
  size_t root = L->root_bytes;
  // E^T (in the roots' precision) and D (f32) reuse the root workspace
  const size_t ed = (a->precond_dt == SHAMPOO_BF16 ? precond_bf16_bytes(a->nblk, a->B)
                                                    : align_up((size_t)a->nblk * BB * dtype_size(a->stats_dt))) +
                    align_up((size_t)a->nblk * BB * 4);
  if (root < ed) root = ed;
  size_t off = 0;
  L->g = off; off += align_up((size_t)a->nblk * BB * es);
  L->gt = off; off += align_up((size_t)a->nblk * BB * es);
  L->valid = off; off += align_up((size_t)a->nblk * 2 * 4);
  L->root = off; off += root;
  L->partials = off; off += align_up((size_t)a->nblk * L->nchunk * 2 * 8);
  L->scales = off; off += align_up((size_t)a->nblk * 4);
  const int64_t nf = 2 * a->nblk;
  L->fl = L->fidx = L->fvalid = L->fflags = L->fin = L->fout = L->froot = 0;
  L->froot_bytes = 0;
  L->redo64 = a->fallback == SHAMPOO_FALLBACK_F64 && a->root.compute != SHAMPOO_F64;
  if (a->fallback != SHAMPOO_FALLBACK_NONE) {
    L->fl = off; off += align_up((size_t)nf * 4);
  }
  if (L->redo64) {
    const size_t mb = (size_t)BB * dtype_size(a->stats_dt);
    L->froot_bytes = root_ws_bytes(nf, a->B, P, SHAMPOO_F64);
    L->fidx = off; off += align_up((size_t)nf * 4);
    L->fvalid = off; off += align_up((size_t)nf * 4);
    L->fflags = off; off += align_up((size_t)nf * 4);
    L->fin = off; off += align_up((size_t)nf * mb);
    L->fout = off; off += align_up((size_t)nf * mb);
    L->froot = off; off += L->froot_bytes;
  }
  L->gidx = L->gvalid = L->gflags = L->gres = L->gin = L->gout = 0;
  L->ragged = false;
  if (a->table_host && a->B <= 64 * 128)
    for (int64_t b = 0; b < a->nblk && !L->ragged; ++b)
      L->ragged = a->table_host[b].rows < a->B || a->table_host[b].cols < a->B;
  L->tl = L->tl_each = 0;
  if (L->ragged) {
    const int64_t nt = a->B / 64;
    L->tl_each = 2 * align_up((size_t)a->nblk * nt * nt * 4) + align_up((size_t)a->nblk * 4) +
                 align_up((size_t)a->nblk * 8) + ALIGN;
    L->tl = off;
    off += 4 * L->tl_each;
  }
  L->gside.clear();
  L->gstart.clear();
  L->gcount.clear();
  L->gorder.clear();
  if (a->table_host) {
    // factor f < nblk is L of block f (valid rows), f >= nblk is R (valid cols)
    std::vector<int> side((size_t)nf);
    bool narrow = false;
    for (int64_t b = 0; b < a->nblk; ++b) {
      const shampoo_block& t = a->table_host[b];
      const int vr = std::min(std::max(t.rows, 1), a->B), vc = std::min(std::max(t.cols, 1), a->B);
      side[(size_t)b] = (vr + 63) / 64 * 64;
      side[(size_t)(a->nblk + b)] = (vc + 63) / 64 * 64;
      narrow = narrow || side[(size_t)b] < a->B || side[(size_t)(a->nblk + b)] < a->B;
    }
    if (narrow && a->B <= 64 * GROUP_BINS) {
      size_t need_io = 0, need_root = 0;
      for (int sd = 64; sd <= a->B; sd += 64) {
        const int64_t start = (int64_t)L->gorder.size();
        for (int64_t f = 0; f < nf; ++f)
          if (side[(size_t)f] == sd) L->gorder.push_back((int32_t)f);
        const int64_t cnt = (int64_t)L->gorder.size() - start;
        if (cnt == 0) continue;
        L->gside.push_back(sd);
        L->gstart.push_back(start);
        L->gcount.push_back(cnt);
        need_io = std::max(need_io, align_up((size_t)cnt * sd * sd * dtype_size(a->stats_dt)));
        need_root = std::max(need_root, root_ws_bytes(cnt, sd, P, a->root.compute));
      }
      if (need_root > L->root_bytes) return fail(SHAMPOO_E_INVALID, "internal: group workspace");
      L->gidx = off; off += align_up((size_t)nf * 4);
      L->gvalid = off; off += align_up((size_t)nf * 4);
      L->gflags = off; off += align_up((size_t)nf * 4);
      L->gres = off; off += align_up((size_t)nf * 4);
      L->gin = off; off += need_io;
      L->gout = off; off += need_io;
    }
  }
  L->total = off;
  return SHAMPOO_OK;
}

// Roots of the factors grouped by side (StepLayout).  Flags of each factor go
// to fl[f] (OR-ed); with keep_flagged a flagged factor keeps its previous root.
template <typename E>
shampoo_status step_roots_grouped(const shampoo_step_args* a, const StepLayout& L, unsigned char* w,
                                  const int32_t* valid, int32_t* fl, bool keep_flagged, hipStream_t st) {
  const int B = a->B;
  int32_t* gidx = (int32_t*)(w + L.gidx);
  int32_t* gvalid = (int32_t*)(w + L.gvalid);
  int32_t* gflags = (int32_t*)(w + L.gflags);
  const int64_t nf = (int64_t)L.gorder.size();
  // the same order as L.gorder, computed on the device from the device table
  // (no host copy: the step stays capturable in a graph)
  hipLaunchKernelGGL(group_order_kernel, dim3(1), dim3(1024), 0, st, a->table_dev, a->nblk, B, gidx);
  LAUNCH_CHECK("group_order");
  hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)((nf + 255) / 256)), dim3(256), 0, st, gflags, nf, 0);
  LAUNCH_CHECK("fill");
  for (size_t g = 0; g < L.gside.size(); ++g) {
    const int sd = L.gside[g];
    const int m = (int)L.gcount[g];
    int32_t* idx = gidx + L.gstart[g];
    int32_t* gv = gvalid + L.gstart[g];
    int32_t* gf = gflags + L.gstart[g];
    hipLaunchKernelGGL(gather_i32_kernel, dim3((unsigned)((m + 255) / 256)), dim3(256), 0, st, valid, idx, m, gv);
    LAUNCH_CHECK("gather_valid");
    const unsigned gchunks = (unsigned)std::min<int64_t>(64, ((int64_t)sd * sd / (16 / sizeof(E)) + 255) / 256);
    hipLaunchKernelGGL((gather_sub_kernel<E>), dim3(gchunks, (unsigned)m), dim3(256), 0, st, (const E*)a->LR,
                       (E*)(w + L.gin), idx, B, sd);
    LAUNCH_CHECK("gather_sub");
    // the group's residuals (if requested) in group order, scattered below
    shampoo_root_opts og = a->root;
    float* gr = (float*)(w + L.gres) + L.gstart[g];
    if (og.residual_out_dev) og.residual_out_dev = gr;
    shampoo_status r = inverse_root_impl(w + L.gin, w + L.gout, a->stats_dt, m, sd, a->p, &og, gv, nullptr, gf,
                                         w + L.root, L.root_bytes, st, keep_flagged);
    if (r != SHAMPOO_OK) return r;
    if (a->root.residual_out_dev) {
      hipLaunchKernelGGL(scatter_f32_kernel, dim3((unsigned)((m + 255) / 256)), dim3(256), 0, st, (const float*)gr, idx,
                         m, a->root.residual_out_dev);
      LAUNCH_CHECK("scatter_residual");
    }
    const unsigned schunks = (unsigned)std::min<int64_t>(64, ((int64_t)B * B / (16 / sizeof(E)) + 255) / 256);
    hipLaunchKernelGGL((scatter_sub_kernel<E>), dim3(schunks, (unsigned)m), dim3(256), 0, st, (const E*)(w + L.gout),
                       (E*)a->roots, idx, B, sd, gf, keep_flagged ? 1 : 0);
    LAUNCH_CHECK("scatter_sub");
    if (fl) {
      hipLaunchKernelGGL(or_flags_kernel, dim3((unsigned)((m + 255) / 256)), dim3(256), 0, st, gf, idx, m, fl);
      LAUNCH_CHECK("or_flags");
    }
  }
  return SHAMPOO_OK;
}

shampoo_status roots_of_factors(const shampoo_step_args* a, const StepLayout& L, unsigned char* w,
                                const int32_t* valid, int32_t* fl, bool keep_flagged, hipStream_t st) {
  if (!L.gside.empty())
    return a->stats_dt == SHAMPOO_F64 ? step_roots_grouped<uint64_t>(a, L, w, valid, fl, keep_flagged, st)
                                      : step_roots_grouped<uint32_t>(a, L, w, valid, fl, keep_flagged, st);
  return inverse_root_impl(a->LR, a->roots, a->stats_dt, 2 * a->nblk, a->B, a->p, &a->root, valid, nullptr, fl,
                           w + L.root, L.root_bytes, st, keep_flagged);
}

// Inverse roots of the step's 2 nblk factors with the fallback of
// a->fallback for those whose new root is not finite (see shampoo_fallback).
shampoo_status step_roots(const shampoo_step_args* a, const StepLayout& L, unsigned char* w, const int32_t* valid,
                          hipStream_t st) {
  const int64_t nf = 2 * a->nblk;
  const int B = a->B;
  unsigned char* root = w + L.root;
  if (a->fallback == SHAMPOO_FALLBACK_NONE) return roots_of_factors(a, L, w, valid, a->flags_dev, false, st);
  int32_t* fl = (int32_t*)(w + L.fl);
  const unsigned g1 = (unsigned)((nf + 255) / 256);
  hipLaunchKernelGGL(fill_i32_kernel, dim3(g1), dim3(256), 0, st, fl, nf, 0);
  LAUNCH_CHECK("fill");
  shampoo_status r = roots_of_factors(a, L, w, valid, fl, true, st);
  if (r != SHAMPOO_OK) return r;
  if (L.redo64) {
    // count the failed factors (non-finite, or residual above the bound) on
    // the host, then recompute them in float64
    std::vector<int32_t> hf((size_t)nf), idx;
    HIP_TRY(hipMemcpyAsync(hf.data(), fl, (size_t)nf * 4, hipMemcpyDeviceToHost, st));
    HIP_TRY(hipStreamSynchronize(st));
    for (int64_t b = 0; b < nf; ++b)
      if (hf[(size_t)b] & (SHAMPOO_FLAG_NONFINITE | SHAMPOO_FLAG_RESIDUAL)) idx.push_back((int32_t)b);
    const int m = (int)idx.size();
    if (m > 0) {
      int32_t* fidx = (int32_t*)(w + L.fidx);
      int32_t* fvalid = (int32_t*)(w + L.fvalid);
      int32_t* fflags = (int32_t*)(w + L.fflags);
      const int64_t mbytes = (int64_t)B * B * (int64_t)dtype_size(a->stats_dt);
      HIP_TRY(hipMemcpyAsync(fidx, idx.data(), (size_t)m * 4, hipMemcpyHostToDevice, st));
      // the pageable index vector must outlive its copy, also on the error
      // returns below: wait for it here (the stream is idle up to it anyway)
      HIP_TRY(hipStreamSynchronize(st));
      const unsigned chunks = (unsigned)std::min<int64_t>(64, (mbytes / 16 + 255) / 256);
      hipLaunchKernelGGL(gather_matrices_kernel, dim3(chunks, (unsigned)m), dim3(256), 0, st,
                         (const unsigned char*)a->LR, w + L.fin, fidx, mbytes);
      LAUNCH_CHECK("gather");
      hipLaunchKernelGGL(gather_i32_kernel, dim3((unsigned)((m + 255) / 256)), dim3(256), 0, st, valid, fidx, m, fvalid);
      LAUNCH_CHECK("gather_valid");
      hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)((m + 255) / 256)), dim3(256), 0, st, fflags, (int64_t)m, 0);
      LAUNCH_CHECK("fill");
      shampoo_root_opts o64 = a->root;
      o64.compute = SHAMPOO_F64;
      o64.tol = 0.0;  // the recomputation runs the full iteration count
      o64.residual_out_dev = nullptr;  // and keeps its result without a residual check
      o64.residual_bound = 0.0;
      r = inverse_root_impl(w + L.fin, w + L.fout, a->stats_dt, m, B, a->p, &o64, fvalid, nullptr, fflags,
                            w + L.froot, L.froot_bytes, st, true);
      if (r != SHAMPOO_OK) return r;
      hipLaunchKernelGGL(scatter_matrices_kernel, dim3(chunks, (unsigned)m), dim3(256), 0, st,
                         (const unsigned char*)(w + L.fout), (unsigned char*)a->roots, fidx, fflags, mbytes, fl);
      LAUNCH_CHECK("scatter");
    }
  }
  if (a->flags_dev) {
    hipLaunchKernelGGL(merge_fallback_flags_kernel, dim3(g1), dim3(256), 0, st, fl, nf, a->flags_dev);
    LAUNCH_CHECK("merge_flags");
  }
  return SHAMPOO_OK;
}

shampoo_status step_impl(const shampoo_step_args* a, hipStream_t st) {
  StepLayout L;
  shampoo_status r = step_layout(a, &L);
  if (r != SHAMPOO_OK) return r;
  if (a->nblk == 0) return SHAMPOO_OK;
  if (!a->params_dev || !a->table_dev || !a->LR || !a->roots) return fail(SHAMPOO_E_INVALID, "null pointer argument");
  if (a->graft < 0 || a->graft > SHAMPOO_GRAFT_NONE) return fail(SHAMPOO_E_INVALID, "unknown graft %d", a->graft);
  if (a->graft == SHAMPOO_GRAFT_ADAM && (a->t < 1 || !(a->beta1 >= 0 && a->beta1 < 1) || !(a->graft_beta2 >= 0 && a->graft_beta2 < 1)))
    return fail(SHAMPOO_E_INVALID, "Adam grafting needs t >= 1 and beta1, graft_beta2 in [0, 1)");
  if (!a->ws || a->ws_bytes < L.total) return fail(SHAMPOO_E_WORKSPACE, "workspace %zu bytes < %zu needed", a->ws_bytes, L.total);
  unsigned char* w = (unsigned char*)a->ws;
  const int B = a->B;
  const int64_t nblk = a->nblk;
  const int64_t BB = (int64_t)B * B;
  void* g = w + L.g;
  void* gt = w + L.gt;
  int32_t* valid = (int32_t*)(w + L.valid);
  unsigned char* root = w + L.root;

  // 1. pack G and G^T; valid sizes of the 2 nblk factors
  {
    const int tps = (B + 63) / 64;
    dim3 grid((unsigned)(tps * tps), (unsigned)nblk);
    if (a->g_dt == SHAMPOO_F32)
      hipLaunchKernelGGL((pack_kernel<uint32_t, shampoo_param>), grid, dim3(256), 0, st, a->params_dev, a->nparams, a->table_dev,
                         B, tps, (uint32_t*)g, (uint32_t*)gt);
    else
      hipLaunchKernelGGL((pack_kernel<uint16_t, shampoo_param>), grid, dim3(256), 0, st, a->params_dev, a->nparams, a->table_dev,
                         B, tps, (uint16_t*)g, (uint16_t*)gt);
    LAUNCH_CHECK("pack");
    hipLaunchKernelGGL(valid_from_table_kernel, dim3((unsigned)((nblk + 255) / 256)), dim3(256), 0, st, a->table_dev,
                       nblk, valid);
    LAUNCH_CHECK("valid");
  }
  // work-balanced tile lists of the products that skip the blocks' padding
  ProductTiles pt;
  if (L.ragged) {
    TileListArgs ta{};
    const int32_t* vr = valid;
    const int32_t* vc = valid + nblk;
    const int32_t* spec[4][3] = {{vr, vr, vc}, {vc, vc, vr}, {vr, vc, vc}, {vr, vc, vr}};
    for (int q = 0; q < 4; ++q) {
      unsigned char* base = w + L.tl + (size_t)q * L.tl_each;
      const size_t tb = align_up((size_t)nblk * (B / 64) * (B / 64) * 4);
      TileListSpec& sp = ta.s[q];
      sp.r = spec[q][0];
      sp.c = spec[q][1];
      sp.k = spec[q][2];
      sp.sym = q < 2 ? 1 : 0;
      sp.tiles = (int32_t*)base;
      sp.tpre = (int32_t*)(base + tb);
      sp.cpre = (int64_t*)(base + tb + align_up((size_t)nblk * 4));
      sp.cut = (int32_t*)(base + tb + align_up((size_t)nblk * 4) + align_up((size_t)nblk * 8));
      sp.tmp = (int32_t*)(base + tb + align_up((size_t)nblk * 4) + align_up((size_t)nblk * 8) + ALIGN);
      pt.tiles[q] = sp.tiles;
      pt.cut[q] = sp.cut;
    }
    // float32 gradients, statistics and roots, B a multiple of 128: all four
    // products run on the persistent 128-tile kernel (lists of 128-tiles);
    // otherwise on the tiled kernel (lists of 64-tiles)
    pt.T = (a->g_dt == SHAMPOO_F32 && a->stats_dt == SHAMPOO_F32 && B % 128 == 0) ? 128 : 64;
    ta.nmat = nblk;
    ta.n = B;
    ta.T = pt.T;
    ta.BK = 32;
    hipLaunchKernelGGL(tile_list_kernel, dim3(4), dim3(1024), 0, st, ta);
    LAUNCH_CHECK("tile_list");
  }
  // 2. statistics
  r = stats_impl(g, gt, a->g_dt, nblk, B, a->LR, a->stats_dt, a->beta2, st, L.ragged ? valid : nullptr,
                 L.ragged ? &pt : nullptr);
  if (r != SHAMPOO_OK) return r;
  // 3. inverse roots of the 2 nblk factors
  if (a->recompute_roots) {
    r = step_roots(a, L, w, valid, st);
    if (r != SHAMPOO_OK) return r;
  }
  // 4. D = Lr G Rr
  const bool pbf = a->precond_dt == SHAMPOO_BF16;
  const size_t ebytes = pbf ? precond_bf16_bytes(nblk, B) : align_up((size_t)nblk * BB * dtype_size(a->stats_dt));
  void* Et = root;
  float* D = a->dstack ? a->dstack : (float*)(root + ebytes);
  if (pbf)
    r = precond_bf16_impl((const float*)a->roots, g, nblk, B, D, (unsigned char*)Et, st, L.ragged ? valid : nullptr,
                          L.ragged ? &pt : nullptr);
  else
    r = precond_impl(a->roots, a->stats_dt, g, a->g_dt, nblk, B, D, Et, ebytes, st, L.ragged ? valid : nullptr,
                     L.ragged ? &pt : nullptr);
  if (r != SHAMPOO_OK) return r;
  // 5. grafting and update
  GraftArgs ga;
  ga.params = a->params_dev;
  ga.nparams = a->nparams;
  ga.table = a->table_dev;
  ga.dstack = D;
  ga.B = B;
  ga.nchunk = L.nchunk;
  ga.graft = a->graft;
  ga.lr = a->lr;
  ga.momentum = a->momentum;
  ga.beta1 = a->beta1;
  ga.beta2 = a->graft_beta2;
  ga.eps = a->graft_eps;
  ga.bc1 = a->graft == SHAMPOO_GRAFT_ADAM ? (float)(1.0 - std::pow((double)a->beta1, a->t)) : 1.0f;
  ga.bc2 = a->graft == SHAMPOO_GRAFT_ADAM ? (float)(1.0 - std::pow((double)a->graft_beta2, a->t)) : 1.0f;
  ga.partials = (double*)(w + L.partials);
  ga.scales = (float*)(w + L.scales);
  dim3 grid((unsigned)L.nchunk, (unsigned)nblk);
  if (a->g_dt == SHAMPOO_F32) hipLaunchKernelGGL(graft_partials_kernel<float>, grid, dim3(256), 0, st, ga);
  else hipLaunchKernelGGL(graft_partials_kernel<__bf16>, grid, dim3(256), 0, st, ga);
  LAUNCH_CHECK("graft_partials");
  hipLaunchKernelGGL(graft_scale_kernel, dim3((unsigned)((nblk + 255) / 256)), dim3(256), 0, st, ga, nblk,
                     a->graft_blockwise);
  LAUNCH_CHECK("graft_scale");
  hipLaunchKernelGGL(graft_update_kernel, grid, dim3(256), 0, st, ga);
  LAUNCH_CHECK("graft_update");
  return SHAMPOO_OK;
}

}  // namespace

// ---------------------------------------------------------------------------
// exported C ABI
// ---------------------------------------------------------------------------
extern "C" {

const char* shampoo_version(void) { return "shampoo-mi355x 0.1.0 (gfx950)"; }

const char* shampoo_last_error(void) { return g_err.c_str(); }

shampoo_status shampoo_plan_blocks(const int64_t* shapes2d, const int32_t* block_sizes, int32_t nparams,
                                   shampoo_block* out, int64_t* nblk) {
  if (!nblk) return fail(SHAMPOO_E_INVALID, "nblk is NULL");
  if (nparams < 0) return fail(SHAMPOO_E_INVALID, "nparams < 0");
  if (nparams > 0 && (!shapes2d || !block_sizes)) return fail(SHAMPOO_E_INVALID, "null pointer argument");
  int64_t count = 0;
  for (int32_t p = 0; p < nparams; ++p) {
    const int64_t m = shapes2d[2 * p], n = shapes2d[2 * p + 1];
    const int64_t bs = block_sizes[p];
    if (m < 0 || n < 0 || bs < 0) return fail(SHAMPOO_E_INVALID, "parameter %d: negative size", p);
    if (m == 0 || n == 0) continue;
    const int64_t B = bs == 0 ? (m > n ? m : n) : bs;
    if (B > INT32_MAX || m > INT32_MAX || n > INT32_MAX) return fail(SHAMPOO_E_INVALID, "parameter %d too large", p);
    count += ((m + B - 1) / B) * ((n + B - 1) / B);
  }
  if (!out) {
    *nblk = count;
    return SHAMPOO_OK;
  }
  if (count > *nblk) {
    const int64_t cap = *nblk;
    *nblk = count;
    return fail(SHAMPOO_E_INVALID, "table capacity %lld < %lld blocks", (long long)cap, (long long)count);
  }
  int64_t i = 0;
  for (int32_t p = 0; p < nparams; ++p) {
    const int64_t m = shapes2d[2 * p], n = shapes2d[2 * p + 1];
    if (m == 0 || n == 0) continue;
    const int64_t B = block_sizes[p] == 0 ? (m > n ? m : n) : block_sizes[p];
    const int64_t nbr = (m + B - 1) / B, nbc = (n + B - 1) / B;
    for (int64_t br = 0; br < nbr; ++br)
      for (int64_t bc = 0; bc < nbc; ++bc) {
        shampoo_block b;
        b.param = p;
        b.brow = (int32_t)br;
        b.bcol = (int32_t)bc;
        b.row0 = (int32_t)(br * B);
        b.col0 = (int32_t)(bc * B);
        b.rows = (int32_t)((m - br * B) < B ? (m - br * B) : B);
        b.cols = (int32_t)((n - bc * B) < B ? (n - bc * B) : B);
        b.B = (int32_t)B;
        out[i++] = b;
      }
  }
  *nblk = count;
  return SHAMPOO_OK;
}

shampoo_status shampoo_pack_blocks(const shampoo_matrix* mats_dev, int32_t nparams, const shampoo_block* table_dev,
                                   int64_t nblk, int32_t B, shampoo_dtype dt, void* stack, void* stack_t,
                                   hipStream_t stream) {
  return pack_impl(mats_dev, nparams, table_dev, nblk, B, dt, stack, stack_t, stream);
}

shampoo_status shampoo_unpack_blocks(const float* stack, const shampoo_block* table_dev, int64_t nblk, int32_t B,
                                     const shampoo_matrix* mats_dev, int32_t nparams, hipStream_t stream) {
  if (nblk < 0 || B < 1 || nparams < 0) return fail(SHAMPOO_E_INVALID, "bad sizes");
  if (nblk == 0) return SHAMPOO_OK;
  if (!stack || !table_dev || !mats_dev) return fail(SHAMPOO_E_INVALID, "null pointer argument");
  if (nblk > 65535) return fail(SHAMPOO_E_UNSUPPORTED, "nblk = %lld > 65535", (long long)nblk);
  const int tps = (B + 63) / 64;
  dim3 grid((unsigned)(tps * tps), (unsigned)nblk);
  hipLaunchKernelGGL(unpack_kernel, grid, dim3(256), 0, stream, stack, table_dev, B, tps, mats_dev, nparams);
  LAUNCH_CHECK("unpack");
  return SHAMPOO_OK;
}

shampoo_status shampoo_update_stats(const void* gstack, const void* gstack_t, shampoo_dtype g_dt, int64_t nblk,
                                    int32_t B, void* LR, shampoo_dtype stats_dt, double beta2, hipStream_t stream) {
  return stats_impl(gstack, gstack_t, g_dt, nblk, B, LR, stats_dt, beta2, stream);
}

shampoo_status shampoo_inverse_root_workspace(int64_t n, int32_t B, int32_t p, const shampoo_root_opts* opts,
                                              size_t* bytes) {
  if (!bytes) return fail(SHAMPOO_E_INVALID, "bytes is NULL");
  shampoo_status r = check_root_args(n, B, p, opts);
  if (r != SHAMPOO_OK) return r;
  *bytes = root_ws_bytes(n, B, build_plan(p, opts), opts->compute);
  return SHAMPOO_OK;
}

shampoo_status shampoo_inverse_root(const void* in, void* out, shampoo_dtype io_dt, int64_t n, int32_t B, int32_t p,
                                    const shampoo_root_opts* opts, const int32_t* valid_dev, float* scale_out_dev,
                                    int32_t* flags_dev, void* ws, size_t ws_bytes, hipStream_t stream) {
  return inverse_root_impl(in, out, io_dt, n, B, p, opts, valid_dev, scale_out_dev, flags_dev, ws, ws_bytes, stream);
}

shampoo_status shampoo_inverse_root_noalloc(const void* in, void* out, shampoo_dtype io_dt, int64_t n, int32_t B,
                                            int32_t p, const shampoo_root_opts* opts, const int32_t* valid_dev,
                                            float* scale_out_dev, int32_t* flags_dev, hipStream_t stream) {
  return inverse_root_noalloc_impl(in, out, io_dt, n, B, p, opts, valid_dev, scale_out_dev, flags_dev, stream);
}

shampoo_status shampoo_precondition_workspace(int64_t nblk, int32_t B, shampoo_dtype roots_dt, size_t* bytes) {
  if (!bytes || nblk < 0 || B < 1) return fail(SHAMPOO_E_INVALID, "bad arguments");
  if (roots_dt != SHAMPOO_F32 && roots_dt != SHAMPOO_F64) return fail(SHAMPOO_E_UNSUPPORTED, "roots dtype %d", (int)roots_dt);
  if (B % 64 != 0) return fail(SHAMPOO_E_UNSUPPORTED, "B = %d: must be a positive multiple of 64", B);
  // the call's launch limits, so that no size is computed for a batch it refuses
  if (nblk > 65535 || gemm_wgs(B, nblk, false) >= (int64_t)1 << 31)
    return fail(SHAMPOO_E_UNSUPPORTED, "batch too large");
  *bytes = (size_t)nblk * B * B * dtype_size(roots_dt);
  return SHAMPOO_OK;
}

shampoo_status shampoo_precondition(const void* roots, shampoo_dtype roots_dt, const void* gstack,
                                    shampoo_dtype g_dt, int64_t nblk, int32_t B, float* dstack, void* ws,
                                    size_t ws_bytes, hipStream_t stream) {
  return precond_impl(roots, roots_dt, gstack, g_dt, nblk, B, dstack, ws, ws_bytes, stream);
}

shampoo_status shampoo_step_workspace(const shampoo_step_args* args, size_t* bytes) {
  if (!bytes) return fail(SHAMPOO_E_INVALID, "bytes is NULL");
  StepLayout L;
  shampoo_status r = step_layout(args, &L);
  if (r != SHAMPOO_OK) return r;
  *bytes = L.total;
  return SHAMPOO_OK;
}

shampoo_status shampoo_step(const shampoo_step_args* args, hipStream_t stream) { return step_impl(args, stream); }

shampoo_status shampoo_check_flags(const int32_t* flags_dev, int64_t n, hipStream_t stream) {
  if (n < 0) return fail(SHAMPOO_E_INVALID, "n < 0");
  if (n == 0) return SHAMPOO_OK;
  if (!flags_dev) return fail(SHAMPOO_E_INVALID, "flags_dev is NULL");
  int32_t host[4096];
  bool any = false;
  for (int64_t i = 0; i < n; i += 4096) {
    const int64_t m = (n - i) < 4096 ? (n - i) : 4096;
    HIP_TRY(hipMemcpyAsync(host, flags_dev + i, (size_t)m * 4, hipMemcpyDeviceToHost, stream));
    HIP_TRY(hipStreamSynchronize(stream));
    for (int64_t j = 0; j < m; ++j)
      if (host[j]) any = true;
  }
  if (any) return fail(SHAMPOO_E_NONFINITE, "flagged matrices present");
  return SHAMPOO_OK;
}

shampoo_status shampoo_timing_enable(int32_t capacity) {
  if (capacity < 0 || capacity > (1 << 20)) return fail(SHAMPOO_E_INVALID, "capacity %d", capacity);
  for (hipEvent_t e : g_timing.ev) (void)hipEventDestroy(e);
  g_timing.ev.clear();
  g_timing.cap = 0;
  g_timing.used = 0;
  if (capacity == 0) return SHAMPOO_OK;
  g_timing.ev.resize(2 * (size_t)capacity);
  for (auto& e : g_timing.ev) HIP_TRY(hipEventCreate(&e));
  g_timing.cap = capacity;
  return SHAMPOO_OK;
}

shampoo_status shampoo_timing_read(float* ms, int32_t capacity, int32_t* count) {
  if (!count || (capacity > 0 && !ms) || capacity < 0) return fail(SHAMPOO_E_INVALID, "bad arguments");
  const int n = g_timing.used < capacity ? g_timing.used : capacity;
  for (int i = 0; i < n; ++i) {
    HIP_TRY(hipEventSynchronize(g_timing.ev[2 * i + 1]));
    HIP_TRY(hipEventElapsedTime(ms + i, g_timing.ev[2 * i], g_timing.ev[2 * i + 1]));
  }
  *count = n;
  g_timing.used = 0;
  return SHAMPOO_OK;
}

shampoo_status shampoo_mfma_peak(shampoo_dtype dt, void* sink_dev, hipStream_t stream, double* tflops) {
  if (!sink_dev || !tflops) return fail(SHAMPOO_E_INVALID, "null pointer argument");
  int cus = 0;
  HIP_TRY(cu_count(&cus));
  const unsigned grid = (unsigned)(cus * 8);  // 8 workgroups of 4 waves per CU
  const int iters = 4096;
  double flops_per_round = 0;  // per wave and loop round
  auto launch = [&](int it) -> hipError_t {
    switch (dt) {
      case SHAMPOO_F32:
        hipLaunchKernelGGL(mfma_peak_kernel<Mma::F32>, dim3(grid), dim3(256), 0, stream, it, 0, (float*)sink_dev);
        flops_per_round = PeakOp<Mma::F32>::flops * PeakOp<Mma::F32>::CHAINS;
        break;
      case SHAMPOO_F64:
        hipLaunchKernelGGL(mfma_peak_kernel<Mma::F64>, dim3(grid), dim3(256), 0, stream, it, 0, (float*)sink_dev);
        flops_per_round = PeakOp<Mma::F64>::flops * PeakOp<Mma::F64>::CHAINS;
        break;
      case SHAMPOO_F16:
        hipLaunchKernelGGL(mfma_peak_kernel<Mma::F16>, dim3(grid), dim3(256), 0, stream, it, 0, (float*)sink_dev);
        flops_per_round = PeakOp<Mma::F16>::flops * PeakOp<Mma::F16>::CHAINS;
        break;
      case SHAMPOO_BF16:
        hipLaunchKernelGGL(mfma_peak_kernel<Mma::BF16>, dim3(grid), dim3(256), 0, stream, it, 0, (float*)sink_dev);
        flops_per_round = PeakOp<Mma::BF16>::flops * PeakOp<Mma::BF16>::CHAINS;
        break;
      default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
  };
  if (dt != SHAMPOO_F32 && dt != SHAMPOO_F64 && dt != SHAMPOO_F16 && dt != SHAMPOO_BF16)
    return fail(SHAMPOO_E_UNSUPPORTED, "dtype %d (F32, F64, F16, BF16)", (int)dt);
  HIP_TRY(launch(iters / 8));  // warm-up
  hipEvent_t e0, e1;
  HIP_TRY(hipEventCreate(&e0));
  HIP_TRY(hipEventCreate(&e1));
  hipError_t err = hipEventRecord(e0, stream);
  if (err == hipSuccess) err = launch(iters);
  if (err == hipSuccess) err = hipEventRecord(e1, stream);
  if (err == hipSuccess) err = hipEventSynchronize(e1);
  float ms = 0.f;
  if (err == hipSuccess) err = hipEventElapsedTime(&ms, e0, e1);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  HIP_TRY(err);
  const double waves = (double)grid * 4;
  *tflops = waves * iters * flops_per_round / (ms * 1e-3) / 1e12;
  return SHAMPOO_OK;
}

}  // extern "C"
