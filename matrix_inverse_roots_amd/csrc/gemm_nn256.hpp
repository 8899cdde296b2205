// Large-tile float32 NN product (the product family is described in
// gemm_common.hpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_common.hpp"

namespace shampoo {

// ---------------------------------------------------------------------------
// Large-tile float32 NN product (n a multiple of 256, no D operand):
//     C_b = alpha * A_b B_b + gamma * I,   C2_b = alpha2 * C_b + gamma2 * I.
//
// One workgroup per CU (512 threads, 8 waves of 128 x 64 outputs) computes
// 256 x 256 tiles and walks a strided list of them (persistent grid), so the
// loads of a tile's first k-stage overlap the previous tile's last stage and
// its stores overlap the next tile's first.  Per k-stage (32 values of k)
// both operand tiles (32 KB each) go straight from global memory into LDS
// with `global_load_lds_dwordx4` (no staging registers, no LDS store
// instructions); two stage buffers, 128 KB of LDS.  Each wave waits for its
// own loads (vmcnt) and then meets the others at a plain `s_barrier`: the
// release fence of __syncthreads() would wait for every outstanding load,
// including those of the next stage.
//
// LDS layouts:
//   A tile  [256 rows m][128 B of k]: no padding (the DMA writes 1 KB runs);
//           the 16-byte chunk c of row m sits at position c ^ swz(m), which
//           spreads a fragment read over all banks.
//   B tile  [32 rows k][256 columns]: B's own row-major layout, k-major.
// Fragments: A as in gemm_kernel (lane reads 4 consecutive k of its row);
// for B, lane (i16, grp) reads the 4 consecutive columns 4 i16 .. 4 i16 + 3
// of k-row 4 kc + u, one per 16x16 column block.  Output column block j of a
// wave therefore holds columns wn*64 + 4 (l % 16) + j, and a lane owns 4
// consecutive columns of each of its rows: the epilogue stores float4 runs
// straight from the accumulators.  The k order per output element is the
// same as in gemm_kernel, so the two kernels give bit-identical results.
// ---------------------------------------------------------------------------
constexpr int NN256_T = 256;
constexpr int NN256_BK = 32;
constexpr int NN256_ABYTES = NN256_T * 128;               // 32 KB
constexpr int NN256_BBYTES = NN256_BK * NN256_T * 4;      // 32 KB
constexpr int NN256_LDS = 2 * (NN256_ABYTES + NN256_BBYTES);  // 128 KB

__global__ __launch_bounds__(512, 1) void gemm_f32_nn256_kernel(GemmArgs g) {
  constexpr int T = NN256_T, BK = NN256_BK, SB = NN256_ABYTES + NN256_BBYTES;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  // Tiles of XCD x (blockIdx % 8) form one contiguous range; workgroup l of
  // that XCD takes every per-th of them.
  const int per = gridDim.x >> 3;
  const int x = blockIdx.x & 7, l = blockIdx.x >> 3;
  const int64_t q = g.total >> 3, r = g.total & 7;
  const int64_t mine = q + (x < r ? 1 : 0);
  if (mine <= l) return;
  const int64_t first = x * q + (x < r ? x : r) + l;
  const int ntile = (int)((mine - l + per - 1) / per);
  const int n = g.n, nst = n / BK;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  const int i16 = lane & 15, grp = lane >> 4;
  const float* Ag = reinterpret_cast<const float*>(g.A);
  const float* Bg = reinterpret_cast<const float*>(g.B);

  // Each wave issues 4 A loads (8 rows x 128 B each) and 4 B loads (one
  // 1 KB k-row each) per stage; lane offsets in elements.
  int aoff[4], boff[4];
#pragma unroll
  for (int qq = 0; qq < 4; ++qq) {
    const int row = 8 * (4 * wave + qq) + (lane >> 3), pos = lane & 7;
    aoff[qq] = row * n + 4 * (pos ^ lds_swz(row));
    boff[qq] = (4 * wave + qq) * n + 4 * lane;
  }
  auto coords = [&](int it, int64_t& moff, int& ti, int& tj) {
    const int64_t w = first + (int64_t)it * per;
    const int64_t mat = w / g.tiles;
    const int t = (int)(w - mat * g.tiles);
    ti = t / g.nt;
    tj = t - ti * g.nt;
    moff = mat * g.stride;
  };
  // load cursor: tile lt, k-stage lk
  int lt = 0, lk = 0;
  const float *LA, *LB;
  {
    int64_t mo;
    int ti, tj;
    coords(0, mo, ti, tj);
    LA = Ag + mo + (int64_t)ti * T * n;
    LB = Bg + mo + (int64_t)tj * T;
  }
  auto issue = [&](int buf) {
    unsigned char* sa = smem + buf * SB;
    unsigned char* sb = sa + NN256_ABYTES;
    const float* pa = LA + lk * BK;
    const float* pb = LB + (int64_t)lk * BK * n;
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      __builtin_amdgcn_global_load_lds((const void*)(pa + aoff[qq]), (void*)(sa + (4 * wave + qq) * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(pb + boff[qq]), (void*)(sb + (4 * wave + qq) * 1024), 16, 0, 0);
    }
  };
  auto advance = [&]() {
    if (++lk == nst) {
      lk = 0;
      if (++lt < ntile) {
        int64_t mo;
        int ti, tj;
        coords(lt, mo, ti, tj);
        LA = Ag + mo + (int64_t)ti * T * n;
        LB = Bg + mo + (int64_t)tj * T;
      }
    }
  };

  floatx4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  const bool plain = g.alpha == 1.0 && g.gamma == 0.0 && g.C2 == nullptr;
  const int total_steps = ntile * nst;

  issue(0);
  advance();
  wait_vmcnt0();
  barrier_no_fence();
  int ck = 0, ct = 0;
  for (int step = 0; step < total_steps; ++step) {
    const bool more = step + 1 < total_steps;
    if (more) issue((step + 1) & 1);
    const unsigned char* sa = smem + (step & 1) * SB;
    const unsigned char* sb = sa + NN256_ABYTES;
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const int kc = rr * 4 + grp;
      floatx4 a[8], b[4];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int m = wm * 128 + i * 16 + i16;
        a[i] = *reinterpret_cast<const floatx4*>(sa + m * 128 + 16 * (kc ^ lds_swz(m)));
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        b[u] = *reinterpret_cast<const floatx4*>(sb + (kc * 4 + u) * (T * 4) + wn * 256 + 16 * i16);
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i][u], b[u][j], acc[i][j], 0, 0, 0);
    }
    if (more) advance();
    wait_vmcnt0();
    barrier_no_fence();
    if (++ck < nst) continue;
    // Tile done: its stores overlap the next tile's first stage.
    ck = 0;
    int64_t mo;
    int ti, tj;
    coords(ct++, mo, ti, tj);
    float* C = reinterpret_cast<float*>(g.C) + mo;
    float* C2 = g.C2 ? reinterpret_cast<float*>(g.C2) + mo : nullptr;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int R = ti * T + wm * 128 + i * 16 + 4 * grp + v;
        const int c0 = tj * T + wn * 64 + 4 * i16;
        const int64_t at = (int64_t)R * n + c0;
        if (plain) {
          *reinterpret_cast<floatx4*>(C + at) = floatx4{acc[i][0][v], acc[i][1][v], acc[i][2][v], acc[i][3][v]};
          continue;
        }
        double y[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) y[j] = epi_c(g.alpha, (double)acc[i][j][v], 0.0, 0.0, R == c0 + j ? g.gamma : 0.0);
        *reinterpret_cast<floatx4*>(C + at) = floatx4{(float)y[0], (float)y[1], (float)y[2], (float)y[3]};
        if (C2) {
          float z[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) z[j] = (float)epi_c2(g.alpha2, y[j], R == c0 + j ? g.gamma2 : 0.0);
          *reinterpret_cast<floatx4*>(C2 + at) = floatx4{z[0], z[1], z[2], z[3]};
        }
      }
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
}

}  // namespace shampoo
