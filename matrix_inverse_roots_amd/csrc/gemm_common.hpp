// Batched square GEMM on CDNA4 matrix cores (gfx950), with the fused
// epilogues the inverse-root chains need.
//
// For every matrix b of a batch of n x n matrices:
//     acc  = A_b * op(B_b)
//     C_b  = alpha * acc + beta * D_b + gamma * I   (D optional)
//     C2_b = alpha2 * C_b + gamma2 * I              (second output, optional)
// op(B) = B^T when B is read row-wise ("NT") and op(B) = B when B is read
// k-major ("NN").
//
// NT serves the products of symmetric matrices (coupled Newton, Clenshaw,
// statistics G G^T): there A * B = A * B^T.  `sym` mode computes only the
// upper-triangular tiles of such a product and writes each twice (in place
// and mirrored), which keeps the iterate exactly symmetric and skips the
// lower tiles.  NN serves Newton-DB, whose coupled iterates must be
// multiplied as they are, in the order of the recurrence: symmetrising its
// products changes the first-order error map of the iteration from an
// idempotent one into one with eigenvalue 1 - (r + 2 + 1/r)/4 for an
// eigenvalue pair of ratio r^2, unstable once r^2 exceeds about 34.
//
// Five kernels, all row-major with batch stride `stride` elements:
//   gemm_f32_nn256_kernel  (gemm_nn256.hpp) float32 NN, n a multiple of 256:
//                          256 x 256 tiles, one persistent workgroup of 8
//                          waves per CU.
//   gemm_h256_sym_kernel   (gemm_hsym.hpp) half symmetric NT, n a multiple of
//                          256: 256 x 256 tiles, one persistent workgroup of
//                          8 waves per CU, k-stages of 32 in 4 buffers.
//   gemm_h256_nn_kernel    (gemm.hpp) half NN into float32, n a multiple of
//                          256: 256 x 256 tiles, one persistent workgroup of
//                          8 waves per CU.
//   gemm_p128_kernel       (gemm.hpp) float32 / float64 NT or NN, and bfloat16
//                          or half NT into float32, n a multiple of 128:
//                          128 x 128 tiles, two persistent workgroups of 4
//                          waves per CU.
//   gemm_kernel            (gemm.hpp) every other type mix (operands
//                          converted while staged: bf16/f32 -> f64, ...), half
//                          NN, and n = 64 (mod 128): one tile per workgroup,
//                          register-staged loads.
// Products of half operands write float32 results (C, C2) and, where later
// products read them, half copies (Ch, C2h) rounded through float32.
// The persistent kernels load both operand tiles straight into LDS
// (global_load_lds_dwordx4) and store results from the accumulators; the
// tiled kernel stages tiles through registers into padded LDS rows and its
// results through LDS.  All assign k to (lane group, step) the same way and
// evaluate the epilogue with the same FMAs, so they give bit-identical
// results on the same operands.
//
// Matrix-core mapping (16x16 family):
//   f32: v_mfma_f32_16x16x4_f32     (lane supplies 1 value of k per operand)
//   f64: v_mfma_f64_16x16x4_f64
//   f16: v_mfma_f32_16x16x32_f16    (8 values)
//   bf16: v_mfma_f32_16x16x32_bf16
// Lane l supplies row (l % 16) of its A fragment and column (l % 16) of its
// B fragment for k-group (l / 16).  Result element v of lane l is column
// l % 16 and row 4 (l / 16) + v (f32, f16, bf16) or row (l / 16) + 4 v (f64).
// Logical k is assigned to (group, step) by a permutation applied
// identically to A and B, chosen so that each lane reads 16 contiguous bytes
// of its LDS row per fragment read: a stage holds 128 bytes of k per row,
// round r of a stage gives lane group g the 16-byte chunk 4 r + g.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace shampoo {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef double doublex2 __attribute__((ext_vector_type(2)));
typedef double doublex4 __attribute__((ext_vector_type(4)));
typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct GemmArgs {
  const void* A;
  const void* B;
  const void* D;   // may be null (then beta is ignored)
  void* C;         // may be null where Ch is set (half operands)
  void* C2;        // may be null
  void* Ch;        // half copy of C (half operands only; may be null)
  void* C2h;       // half copy of C2 (half operands only; may be null)
  int n;           // side of every matrix, a multiple of the tile
  int tiles;       // tiles per matrix (n/T)^2, or (n/T)(n/T + 1)/2 in sym mode
  int nt;          // n / T
  int sym;         // compute upper tiles only and mirror (NT only)
  int transC;      // write C transposed (no D, no C2, no sym)
  int64_t stride;  // elements between consecutive matrices
  int64_t total;   // batch * tiles (= grid size)
  double alpha, beta, gamma, alpha2, gamma2;
};

// Workgroup id -> linear work index so that the consecutive work items of one
// XCD are contiguous: the hardware deals workgroups to the 8 XCDs round-robin,
// and each XCD has its own L2, so all tiles of a matrix should share an XCD.
__device__ __forceinline__ int64_t xcd_remap(int64_t w, int64_t total) {
  const int64_t q = total >> 3, r = total & 7;
  const int64_t xcd = w & 7, local = w >> 3;
  return xcd * q + (xcd < r ? xcd : r) + local;
}

// The fused epilogue's affine maps in double, written as explicit FMAs so
// that every product kernel rounds them identically:
//   C  = alpha acc + beta D + gamma [diagonal],   C2 = alpha2 C + gamma2 [diagonal].
__device__ __forceinline__ double epi_c(double alpha, double acc, double beta, double d, double diag) {
  return __builtin_fma(alpha, acc, __builtin_fma(beta, d, diag));
}
__device__ __forceinline__ double epi_c2(double alpha2, double c, double diag2) { return __builtin_fma(alpha2, c, diag2); }

template <typename TC> __device__ __forceinline__ void put(TC* p, double v);
template <> __device__ __forceinline__ void put<float>(float* p, double v) { *p = (float)v; }
template <> __device__ __forceinline__ void put<double>(double* p, double v) { *p = v; }

// Half copies of float32 results (operands of later half-precision
// products): each value is rounded to float32 first, then to half (nearest
// even both times), so the copy holds what a float32 iterate rounded to a
// half operand holds.  The empty asm statement pins the float32 value:
// without it the compiler merges a preceding double -> float32 conversion
// and this one into a single double -> half rounding, which differs where
// the float32 rounding lands on a half-way point.
__device__ __forceinline__ _Float16 half_of(float f) {
  asm volatile("" : "+v"(f));
  return (_Float16)f;
}
typedef _Float16 halfx4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store_h4(_Float16* p, floatx4 v) {
  *reinterpret_cast<halfx4*>(p) = halfx4{half_of(v[0]), half_of(v[1]), half_of(v[2]), half_of(v[3])};
}

// LDS tile rows of 128 bytes (8 chunks of 16 bytes): chunk c of LDS row m
// sits at position c ^ swz(m).  A fragment read (ds_read_b128) has lane
// (i16, grp) read chunk 4 rr + grp of row r0 + rho(i16), r0 a multiple of 16.
// Which swizzle keeps such a read free of bank conflicts depends on rho; on
// MI355X (SQ_LDS_BANK_CONFLICT over SQ_LDS_IDX_ACTIVE, 4 active cycles per
// conflict-free read):
//   rho(i) = i (rows in lane order):    lds_swz, conflict-free; the form
//     (m & 7) ^ ((m >> 3) & 1) doubles the cycles of every read (40% of the
//     float32 NN product's LDS cycles, 50% of the half NT product's);
//   rho(i) = 4 (i & 3) + (i >> 2) (the float64 A fragments): lds_swz_t,
//     conflict-free; lds_swz costs 1.5x there.
__device__ __forceinline__ int lds_swz(int m) { return (m & 3) | (((m >> 3) & 1) << 2); }
__device__ __forceinline__ int lds_swz_t(int m) { return (m & 7) ^ ((m >> 3) & 1); }

// Stage barriers of the persistent kernels: each wave waits for its own
// direct-to-LDS loads (vmcnt) and then meets the others at a plain
// s_barrier, without the release fence of __syncthreads(), which would also
// wait for loads issued for later stages.
__device__ __forceinline__ void barrier_no_fence() { asm volatile("s_barrier" ::: "memory"); }
__device__ __forceinline__ void wait_vmcnt0() { __builtin_amdgcn_s_waitcnt(0x3f70); }  // vmcnt(0) only

}  // namespace shampoo
