// Symmetric half-operand NT product with 256 x 256 tiles (the product
// family is described in gemm_common.hpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_common.hpp"

namespace shampoo {

// ---------------------------------------------------------------------------
// Symmetric half NT product, n a multiple of 256, half outputs only:
//     Ch = alpha A B^T + gamma I,   C2h = alpha2 (alpha A B^T + gamma I) + gamma2 I
// (C2h optional), upper tiles only, each written in place and mirrored.  The
// library routes the symmetric products whose results are read only as
// half operands here (the squarings and updates of the half-precision
// coupled-Newton chains); products with float32 outputs or an addend run on
// the 128-tile kernel.
//
// One persistent workgroup per CU of 8 waves, two per SIMD: a single wave
// per SIMD issues matrix-core instructions at about 60% of the rate two
// waves reach (measured on MI355X), so each wave takes 64 x 128 outputs (128
// accumulator registers).  k-stages of 32 (64 bytes of each operand row) go
// straight into LDS, 4 stage buffers of 32 KB, loads issued 3 stages ahead
// of the stage being multiplied.  A wave reads the next stage's A fragments
// before its matrix-core instructions and each next B fragment right after
// the last instruction that uses the current one, so LDS latency overlaps
// the matrix cores.  One barrier per stage.
//
// Both operands are row-major with k contiguous.  The loads write LDS row
// 64 G + 16 i + r from tile row 64 G + 4 r + i, with the 16-byte chunk c of
// a row at c ^ hs_swz(row).  The matrix-core operands are swapped (the B
// side feeds the A operand), so that lane (i16, grp) holds, in value v of
// block (i, 4 gj + jj), C[R0 + i][C0 + jj] with R0 = 64 wm + 4 i16 and
// C0 = 128 wn + 64 gj + 16 grp + 4 v (wave w = 2 wm + wn).
//
// Stores.  A wave's outputs form two 64 x 64 blocks (gj = 0, 1).  A block
// above the diagonal of the matrix is written
//   * in place as rows: lanes i16 and i16 ^ 1 (rows 4 apart) swap half of
//     their 16 columns of a row with a DPP lane swap, so that each 16-byte
//     store instruction writes 8 complete 128-byte row segments;
//   * mirrored as columns: a lane's 4 consecutive rows of one column become
//     8 bytes of a row of the transposed block, 16 lanes one 128-byte
//     segment.
// Stores that leave partial segments (8-byte pieces of 16 rows per
// instruction, the earlier in-place form) were written back to memory
// before the segments were complete: 1.33-1.45x the output bytes for one
// output and 2.2x for two.  With the swap the writes are 1.05x and 1.21x,
// and on 288 x 1024^2 (measured in isolation, steady state) a squaring takes
// 464 us instead of 486 and a product with two outputs 569 instead of 670;
// without any stores it would take 340.  A block on the
// diagonal is written 4 x 4 sub-block by sub-block: its upper sub-blocks in
// place (8-byte rows) and mirrored, the diagonal sub-blocks element by
// element; blocks below the diagonal store nothing.
//
// The k order per output element (k-groups of 8 in the order of the other
// kernels' two rounds per 64-k stage) is the same as in every product
// kernel, and so are the results, bit for bit.
// ---------------------------------------------------------------------------
constexpr int HS_T = 256, HS_BK = 32, HS_NS = 4;
constexpr int HS_OP = HS_T * 64;          // 16 KB per operand and stage
constexpr int HS_STAGE = 2 * HS_OP;       // 32 KB
constexpr int HS_LDS = HS_NS * HS_STAGE;  // 128 KB

// tile row held by LDS row rho (64 G + 16 i + r -> 64 G + 4 r + i)
__device__ __forceinline__ int hs_src_row(int rho) { return (rho & ~63) | (4 * (rho & 15)) | ((rho >> 4) & 3); }
// chunk swizzle of the 64-byte LDS rows (measured the fastest of five)
__device__ __forceinline__ int hs_swz(int m) { return (m >> 1) & 3; }
// wait until at most K vector memory operations of this wave are in flight
template <int K> __device__ __forceinline__ void hs_wait_vm() {
  __builtin_amdgcn_s_waitcnt((K & 15) | (0x7 << 4) | (0xF << 8) | ((K >> 4) << 14));
}
// wait until at most the largest listed count <= k operations are in flight
__device__ __forceinline__ void hs_wait_vm_le(int k) {
  if (k >= 63) hs_wait_vm<63>();
  else if (k >= 48) hs_wait_vm<48>();
  else if (k >= 32) hs_wait_vm<32>();
  else if (k >= 16) hs_wait_vm<16>();
  else if (k >= 4) hs_wait_vm<4>();
  else hs_wait_vm<0>();
}
__device__ __forceinline__ floatx4 mma_h(halfx8 a, halfx8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__global__ __launch_bounds__(512, 1) void gemm_h256_sym_kernel(GemmArgs g) {
  using E = _Float16;
  using frag_t = halfx8;
  constexpr int T = HS_T, BK = HS_BK;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int per = gridDim.x >> 3;
  const int x = blockIdx.x & 7, l = blockIdx.x >> 3;
  const int64_t q = g.total >> 3, r = g.total & 7;
  const int64_t mine = q + (x < r ? 1 : 0);
  if (mine <= l) return;
  const int64_t first = x * q + (x < r ? x : r) + l;
  const int ntile = (int)((mine - l + per - 1) / per);
  const int n = g.n, nst = n / BK;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;  // rows 64 wm .., columns 128 wn ..
  const int i16 = lane & 15, grp = lane >> 4;
  const E* Ag = reinterpret_cast<const E*>(g.A);
  const E* Bg = reinterpret_cast<const E*>(g.B);

  // per stage and operand: 16 loads of 1 KB (16 LDS rows x 64 B); wave w
  // issues loads 2 w and 2 w + 1 of each operand
  int off[2];
#pragma unroll
  for (int qq = 0; qq < 2; ++qq) {
    const int rho = 16 * (2 * wave + qq) + (lane >> 2), pos = lane & 3;
    off[qq] = hs_src_row(rho) * n + 8 * (pos ^ hs_swz(rho));
  }
  auto coords = [&](int it, int64_t& moff, int& ti, int& tj) {
    const int64_t w = first + (int64_t)it * per;
    const int64_t mat = w / g.tiles;
    int t = (int)(w - mat * g.tiles);
    ti = 0;
    int rowlen = g.nt;
    while (t >= rowlen) {
      t -= rowlen;
      ++ti;
      --rowlen;
    }
    tj = ti + t;
    moff = mat * g.stride;
  };
  int lt = 0, lk = 0;
  int64_t cmo;
  int cti, ctj;
  coords(0, cmo, cti, ctj);
  const E* LA = Ag + cmo + (int64_t)cti * T * n;
  const E* LB = Bg + cmo + (int64_t)ctj * T * n;
  auto issue = [&](int buf) {
    unsigned char* sa = smem + buf * HS_STAGE;
    unsigned char* sb = sa + HS_OP;
    const E* pa = LA + lk * BK;
    const E* pb = LB + lk * BK;
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) {
      __builtin_amdgcn_global_load_lds((const void*)(pa + off[qq]), (void*)(sa + (2 * wave + qq) * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(pb + off[qq]), (void*)(sb + (2 * wave + qq) * 1024), 16, 0, 0);
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
        LB = Bg + mo + (int64_t)tj * T * n;
      }
    }
  };
  // A fragment i: LDS row 64 wm + 16 i + i16; B fragment j: LDS row
  // 128 wn + 16 j + i16 (1 KB per 16 rows)
  const int afr = (wm * 64 + i16) * 64 + 16 * (grp ^ hs_swz(i16));
  const int bfr = (wn * 128 + i16) * 64 + 16 * (grp ^ hs_swz(i16));

  floatx4 acc[4][8];
  const bool plain = g.alpha == 1.0 && g.gamma == 0.0 && g.C2h == nullptr;
  const int total_steps = ntile * nst;  // >= 8 (n >= 256)

  issue(0);
  advance();
  issue(1);
  advance();
  issue(2);
  advance();
  hs_wait_vm<4>();  // stages 0 and 1 landed (stage 2 may be in flight)
  barrier_no_fence();
  frag_t fa0[4], fa1[4], fb[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) fa0[i] = *reinterpret_cast<const frag_t*>(smem + afr + i * 1024);
#pragma unroll
  for (int j = 0; j < 8; ++j) fb[j] = *reinterpret_cast<const frag_t*>(smem + HS_OP + bfr + j * 1024);
  // vector memory operations the last epilogue issued (a lower bound): they
  // come after stage s + 2's loads, and all complete in order
  int young = 0;

  // one k-stage: loads of stage s + 3; the A fragments of stage s + 1 read
  // before the matrix-core instructions of stage s, its B fragments each
  // right after the last instruction that uses the current one; the wait
  // for stage s + 2; barrier.  ZERO: the tile's first stage.
#define HS_BODY(S, ZERO, CA, NA)                                                      \
  {                                                                                   \
    const int s_ = (S);                                                               \
    const bool dma = s_ + 3 < total_steps;                                            \
    if (dma) {                                                                        \
      issue((s_ + 3) & 3);                                                            \
      advance();                                                                      \
    }                                                                                 \
    const unsigned char* sa = smem + ((s_ + 1) & 3) * HS_STAGE;                       \
    const unsigned char* sb = sa + HS_OP;                                             \
    /* (after the last stage these read a stale buffer: in bounds, unused) */          \
    _Pragma("unroll") for (int i = 0; i < 4; ++i) NA[i] = *reinterpret_cast<const frag_t*>(sa + afr + i * 1024); \
    _Pragma("unroll") for (int i = 0; i < 3; ++i)                                     \
      _Pragma("unroll") for (int j = 0; j < 8; ++j)                                   \
        acc[i][j] = mma_h(fb[j], CA[i], ZERO ? floatx4{0.f, 0.f, 0.f, 0.f} : acc[i][j]); \
    _Pragma("unroll") for (int j = 0; j < 8; ++j) {                                   \
      acc[3][j] = mma_h(fb[j], CA[3], ZERO ? floatx4{0.f, 0.f, 0.f, 0.f} : acc[3][j]); \
      fb[j] = *reinterpret_cast<const frag_t*>(sb + bfr + j * 1024);                  \
    }                                                                                 \
    if (s_ + 2 < total_steps) hs_wait_vm_le(young + (dma ? 4 : 0));                  \
    young = 0;                                                                        \
    barrier_no_fence();                                                               \
  }
  // nst (n / 32, n a multiple of 256) is even: every tile starts on fa0
  for (int ct = 0; ct < ntile; ++ct) {
    const int s0 = ct * nst;
    HS_BODY(s0, true, fa0, fa1)
    HS_BODY(s0 + 1, false, fa1, fa0)
    for (int ck = 2; ck < nst; ck += 2) {
      HS_BODY(s0 + ck, false, fa0, fa1)
      HS_BODY(s0 + ck + 1, false, fa1, fa0)
    }
    // epilogue of tile ct: lane (i16, grp) holds, in value v of block
    // (i, 4 gj + jj), C[R0 + i][C0 + jj] with R0 = 64 wm + 4 i16 and
    // C0 = 128 wn + 64 gj + 16 grp + 4 v (tile coordinates)
    _Float16* Ch = reinterpret_cast<_Float16*>(g.Ch) + cmo;
    _Float16* C2h = g.C2h ? reinterpret_cast<_Float16*>(g.C2h) + cmo : nullptr;
    const bool two = C2h != nullptr;
    // a 4 x 4 sub-block of a block on the diagonal: upper sub-blocks rows in
    // place and columns mirrored, diagonal ones element by element
    auto sub = [&](int gj, int v, const float (&av)[4][4]) {
      const int R0 = cti * T + wm * 64 + 4 * i16;
      const int C0 = ctj * T + wn * 128 + 64 * gj + 16 * grp + 4 * v;
      const int rel = R0 - C0;
      if (rel > 0) return;
      float y[4][4], z[4][4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bool dg = R0 + i == C0 + j;
          const double t = epi_c(g.alpha, (double)av[i][j], 0.0, 0.0, dg ? g.gamma : 0.0);
          y[i][j] = plain ? av[i][j] : (float)t;
          z[i][j] = two ? (float)epi_c2(g.alpha2, t, dg ? g.gamma2 : 0.0) : 0.f;
        }
      if (rel < 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t at = (int64_t)(R0 + i) * n + C0;
          store_h4(Ch + at, floatx4{y[i][0], y[i][1], y[i][2], y[i][3]});
          if (two) store_h4(C2h + at, floatx4{z[i][0], z[i][1], z[i][2], z[i][3]});
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t at = (int64_t)(C0 + j) * n + R0;
          store_h4(Ch + at, floatx4{y[0][j], y[1][j], y[2][j], y[3][j]});
          if (two) store_h4(C2h + at, floatx4{z[0][j], z[1][j], z[2][j], z[3][j]});
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (i > j) continue;
            const int64_t a1 = (int64_t)(R0 + i) * n + C0 + j, a2 = (int64_t)(C0 + j) * n + R0 + i;
            Ch[a1] = half_of(y[i][j]);
            Ch[a2] = half_of(y[i][j]);
            if (two) {
              C2h[a1] = half_of(z[i][j]);
              C2h[a2] = half_of(z[i][j]);
            }
          }
      }
    };
    // a 64 x 64 block above the diagonal (no element on it): rows in place
    // with the DPP swap, then the mirrored columns
    const int odd = i16 & 1;
    auto upper = [&](int gj) {
      const int R0 = cti * T + wm * 64 + 4 * i16;
      const int Cg = ctj * T + wn * 128 + 64 * gj + 16 * grp;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // qy[v]: the 4 halves of row R0 + i, columns Cg + 4 v .. Cg + 4 v + 3
        u32x2 qy[4], qz[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          halfx4 hy, hz;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const float a_ = acc[i][4 * gj + jj][v];
            const double t = epi_c(g.alpha, (double)a_, 0.0, 0.0, 0.0);
            hy[jj] = half_of(plain ? a_ : (float)t);
            hz[jj] = two ? half_of((float)epi_c2(g.alpha2, t, 0.0)) : (_Float16)0.f;
          }
          qy[v] = __builtin_bit_cast(u32x2, hy);
          qz[v] = __builtin_bit_cast(u32x2, hz);
        }
        // the even lane keeps columns 0..7 of its row and sends 8..15; the
        // odd lane keeps 8..15 of its row and sends 0..7.  Store 1 writes
        // the even lane's row, store 2 the odd lane's row (4 rows below).
        const int row1 = R0 + i - 4 * odd, row2 = row1 + 4, col = Cg + 8 * odd;
        auto put = [&](_Float16* O, const u32x2 (&q)[4]) {
          uint32_t r_[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t snd = odd ? q[e >> 1][e & 1] : q[2 + (e >> 1)][e & 1];
            r_[e] = (uint32_t)__builtin_amdgcn_mov_dpp((int)snd, 0xB1, 0xF, 0xF, false);  // lanes i ^ 1
          }
          const u32x4 rv = u32x4{r_[0], r_[1], r_[2], r_[3]};
          const u32x4 lo = u32x4{q[0][0], q[0][1], q[1][0], q[1][1]};
          const u32x4 hi = u32x4{q[2][0], q[2][1], q[3][0], q[3][1]};
          *reinterpret_cast<u32x4*>(O + (int64_t)row1 * n + col) = odd ? rv : lo;
          *reinterpret_cast<u32x4*>(O + (int64_t)row2 * n + col) = odd ? hi : rv;
        };
        put(Ch, qy);
        if (two) put(C2h, qz);
      }
      asm volatile("" ::: "memory");
      // mirrored: column Cg + 4 v + jj, rows R0 .. R0 + 3
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          halfx4 hy, hz;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float a_ = acc[i][4 * gj + jj][v];
            asm volatile("" : "+v"(a_));  // recomputed here rather than kept live from the rows
            const double t = epi_c(g.alpha, (double)a_, 0.0, 0.0, 0.0);
            hy[i] = half_of(plain ? a_ : (float)t);
            hz[i] = two ? half_of((float)epi_c2(g.alpha2, t, 0.0)) : (_Float16)0.f;
          }
          const int64_t at = (int64_t)(Cg + 4 * v + jj) * n + R0;
          *reinterpret_cast<halfx4*>(Ch + at) = hy;
          if (two) *reinterpret_cast<halfx4*>(C2h + at) = hz;
        }
      asm volatile("" ::: "memory");
    };
    // 64-row block of this wave against the two 64-column blocks
    const int rb = cti * 4 + wm;
    int stores = 0;  // store instructions issued (a lower bound: per output)
#pragma unroll
    for (int gj = 0; gj < 2; ++gj) {
      const int cb = ctj * 4 + 2 * wn + gj;
      if (rb < cb) {
        upper(gj);
        stores += 24;
      } else if (rb == cb) {
#define HS_SUB(GJ, V)                                                                 \
  {                                                                                   \
    float av[4][4];                                                                   \
    _Pragma("unroll") for (int i = 0; i < 4; ++i)                                     \
      _Pragma("unroll") for (int j = 0; j < 4; ++j) av[i][j] = acc[i][(GJ) * 4 + j][V]; \
    sub(GJ, V, av);                                                                   \
    asm volatile("" ::: "memory");                                                    \
  }
        HS_SUB(gj, 0) HS_SUB(gj, 1) HS_SUB(gj, 2) HS_SUB(gj, 3)
#undef HS_SUB
        // every sub-block call has a lane with rel < 0: 4 rows and 4 columns
        stores += 32;
      }
    }
    young = stores;
    if (ct + 1 < ntile) coords(ct + 1, cmo, cti, ctj);
  }
#undef HS_BODY
}

}  // namespace shampoo
