// Batched square products for the solver chains and the statistics: the
// tiled kernel, the persistent 128-tile kernel and the persistent 256-tile
// half-operand NN kernel (the family is described in gemm_common.hpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "gemm_common.hpp"

namespace shampoo {

enum class Mma { F32, F64, F16, BF16 };

template <Mma M> struct MmaTraits;

template <> struct MmaTraits<Mma::F32> {
  using lds_t = float;
  using acc_t = float;
  using accv_t = floatx4;
  using frag_t = floatx4;  // one 16-byte LDS read
  static constexpr int VE = 4;   // elements per 16 bytes
  static constexpr int KV = 1;   // elements per lane per instruction
  static constexpr int BK = 32;  // k per stage (128 bytes of LDS row)
  static __device__ __forceinline__ int row(int grp, int v) { return 4 * grp + v; }
  static __device__ __forceinline__ accv_t mma(const frag_t& a, const frag_t& b, int u, accv_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a[u], b[u], c, 0, 0, 0);
  }
};

template <> struct MmaTraits<Mma::F64> {
  using lds_t = double;
  using acc_t = double;
  using accv_t = doublex4;
  using frag_t = doublex2;
  static constexpr int VE = 2;
  static constexpr int KV = 1;
  static constexpr int BK = 16;
  static __device__ __forceinline__ int row(int grp, int v) { return grp + 4 * v; }
  static __device__ __forceinline__ accv_t mma(const frag_t& a, const frag_t& b, int u, accv_t c) {
    return __builtin_amdgcn_mfma_f64_16x16x4f64(a[u], b[u], c, 0, 0, 0);
  }
};

template <> struct MmaTraits<Mma::F16> {
  using lds_t = _Float16;
  using acc_t = float;
  using accv_t = floatx4;
  using frag_t = halfx8;
  static constexpr int VE = 8;
  static constexpr int KV = 8;
  static constexpr int BK = 64;
  static __device__ __forceinline__ int row(int grp, int v) { return 4 * grp + v; }
  static __device__ __forceinline__ accv_t mma(const frag_t& a, const frag_t& b, int, accv_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};

template <> struct MmaTraits<Mma::BF16> {
  using lds_t = __bf16;
  using acc_t = float;
  using accv_t = floatx4;
  using frag_t = bf16x8;
  static constexpr int VE = 8;
  static constexpr int KV = 8;
  static constexpr int BK = 64;
  static __device__ __forceinline__ int row(int grp, int v) { return 4 * grp + v; }
  static __device__ __forceinline__ accv_t mma(const frag_t& a, const frag_t& b, int, accv_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

// ---------------------------------------------------------------------------
// One 16-byte LDS chunk (VE elements of the LDS type) staged through
// registers from VE consecutive elements of the operand's global type.
// ---------------------------------------------------------------------------
template <typename TG, typename TL, int VE> struct Chunk;

template <> struct Chunk<float, float, 4> {  // f32 -> f32
  u32x4 w;
  __device__ __forceinline__ void load(const float* p) { w = *reinterpret_cast<const u32x4*>(p); }
  __device__ __forceinline__ void store(unsigned char* d) const { *reinterpret_cast<u32x4*>(d) = w; }
  __device__ __forceinline__ float get(int e) const { return __uint_as_float(w[e]); }
};

template <> struct Chunk<__bf16, float, 4> {  // bf16 -> f32 (exact)
  u32x2 w;
  __device__ __forceinline__ void load(const __bf16* p) { w = *reinterpret_cast<const u32x2*>(p); }
  __device__ __forceinline__ float get(int e) const {
    const uint32_t x = w[e >> 1];
    return __uint_as_float((e & 1) ? (x & 0xffff0000u) : (x << 16));
  }
  __device__ __forceinline__ void store(unsigned char* d) const {
    u32x4 o;
    o[0] = w[0] << 16;
    o[1] = w[0] & 0xffff0000u;
    o[2] = w[1] << 16;
    o[3] = w[1] & 0xffff0000u;
    *reinterpret_cast<u32x4*>(d) = o;
  }
};

template <> struct Chunk<double, double, 2> {  // f64 -> f64
  doublex2 w;
  __device__ __forceinline__ void load(const double* p) { w = *reinterpret_cast<const doublex2*>(p); }
  __device__ __forceinline__ void store(unsigned char* d) const { *reinterpret_cast<doublex2*>(d) = w; }
  __device__ __forceinline__ double get(int e) const { return w[e]; }
};

template <> struct Chunk<float, double, 2> {  // f32 -> f64 (exact)
  u32x2 w;
  __device__ __forceinline__ void load(const float* p) { w = *reinterpret_cast<const u32x2*>(p); }
  __device__ __forceinline__ double get(int e) const { return (double)__uint_as_float(w[e]); }
  __device__ __forceinline__ void store(unsigned char* d) const {
    doublex2 o;
    o[0] = (double)__uint_as_float(w[0]);
    o[1] = (double)__uint_as_float(w[1]);
    *reinterpret_cast<doublex2*>(d) = o;
  }
};

template <> struct Chunk<__bf16, double, 2> {  // bf16 -> f64 (exact)
  uint32_t w;
  __device__ __forceinline__ void load(const __bf16* p) { w = *reinterpret_cast<const uint32_t*>(p); }
  __device__ __forceinline__ double get(int e) const {
    return (double)__uint_as_float(e ? (w & 0xffff0000u) : (w << 16));
  }
  __device__ __forceinline__ void store(unsigned char* d) const {
    doublex2 o;
    o[0] = (double)__uint_as_float(w << 16);
    o[1] = (double)__uint_as_float(w & 0xffff0000u);
    *reinterpret_cast<doublex2*>(d) = o;
  }
};

template <> struct Chunk<_Float16, _Float16, 8> {  // f16 -> f16
  halfx8 w;
  __device__ __forceinline__ void load(const _Float16* p) { w = *reinterpret_cast<const halfx8*>(p); }
  __device__ __forceinline__ void store(unsigned char* d) const { *reinterpret_cast<halfx8*>(d) = w; }
  __device__ __forceinline__ _Float16 get(int e) const { return w[e]; }
};

template <> struct Chunk<__bf16, __bf16, 8> {  // bf16 -> bf16
  bf16x8 w;
  __device__ __forceinline__ void load(const __bf16* p) { w = *reinterpret_cast<const bf16x8*>(p); }
  __device__ __forceinline__ void store(unsigned char* d) const { *reinterpret_cast<bf16x8*>(d) = w; }
  __device__ __forceinline__ __bf16 get(int e) const { return w[e]; }
};

// VE x VE block of a k-major operand: rows k..k+VE-1, columns j..j+VE-1,
// written transposed into LDS rows j..j+VE-1 at k.
template <typename TG, typename TL, int VE> struct BlockKN {
  Chunk<TG, TL, VE> r[VE];
  __device__ __forceinline__ void load(const TG* p, int ld) {
#pragma unroll
    for (int i = 0; i < VE; ++i) r[i].load(p + (int64_t)i * ld);
  }
  __device__ __forceinline__ void store_t(unsigned char* d, int rowb) const {
#pragma unroll
    for (int c = 0; c < VE; ++c) {
      TL t[VE];
#pragma unroll
      for (int i = 0; i < VE; ++i) t[i] = (TL)r[i].get(c);
      *reinterpret_cast<u32x4*>(d + c * rowb) = *reinterpret_cast<const u32x4*>(t);
    }
  }
};

// Tiled kernel.  LDS holds, for both operands, tile rows (m for A, j for B)
// of 128 bytes of k plus 16 bytes of padding: a row pitch of 9 16-byte bank
// groups, so the 16 lanes of a b128 fragment read hit distinct banks.  NT
// operands are copied row by row (16-byte global loads, coalesced per
// 128-byte row segment); an NN B operand is loaded as VE x VE element blocks
// (VE = elements per 16 bytes) along its rows and transposed in registers.
// Per-matrix extents (each pointer may be null): a tile whose first row is
// at or past r[b], or whose first column is at or past c[b], is neither
// loaded, computed nor written (its workgroup returns at once); k-stages past
// k[b] are skipped.  Rows and columns refer to the product as computed,
// before a transposed store.  Exact where both operands are zero beyond the
// inner extent (ragged blocks zero-padded on packing) and the caller reads
// only the r x c region (plus partial tiles, which are computed in full).
struct Extents {
  const int32_t* r;
  const int32_t* c;
  const int32_t* k;
};

template <Mma MM, int T, bool BKN, typename TA, typename TB, typename TC>
__device__ __forceinline__ void gemm_tile(const GemmArgs& g, const Extents& ext, int64_t mat, int ti, int tj,
                                          unsigned char* smem) {
  using Tr = MmaTraits<MM>;
  using L = typename Tr::lds_t;
  using acc_t = typename Tr::acc_t;
  using accv_t = typename Tr::accv_t;
  using frag_t = typename Tr::frag_t;
  constexpr int BK = Tr::BK, VE = Tr::VE, KV = Tr::KV;
  constexpr int ROWB = BK * (int)sizeof(L) + 16;  // 144 bytes
  constexpr int WT = T / 2;                       // wave tile (2 x 2 waves)
  constexpr int NB = WT / 16;                     // 16x16 blocks per wave side
  constexpr int CH = T * 8 / 256;                 // 16-byte chunks per thread per row-wise operand
  constexpr int NREAD = BK / (4 * VE);            // 16-byte fragment reads per stage
  constexpr int KNB = (BK / VE) * (T / VE);       // VE x VE blocks of a k-major B tile
  constexpr int KNQ = (KNB + 255) / 256;          // ... per thread
  static_assert(BK * sizeof(L) == 128, "LDS row must hold 128 bytes of k");

  // Two stages of A and B tiles (double buffering: one barrier per k-stage);
  // the epilogue reuses the same bytes to stage the C tile.
  auto sA = [&](int buf) { return smem + buf * T * ROWB; };
  auto sB = [&](int buf) { return smem + (2 + buf) * T * ROWB; };

  // tiles outside the matrix's row / column extent: nothing to do (uniform)
  if ((ext.r && ti * T >= ext.r[mat]) || (ext.c && tj * T >= ext.c[mat])) return;
  const int n = g.n;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int i16 = lane & 15, grp = lane >> 4;

  const TA* Ab = reinterpret_cast<const TA*>(g.A) + mat * g.stride + (int64_t)ti * T * n;
  // NT: rows tj*T.. of B; NN: columns tj*T.. of B
  const TB* Bb = reinterpret_cast<const TB*>(g.B) + mat * g.stride + (BKN ? (int64_t)tj * T : (int64_t)tj * T * n);

  Chunk<TA, L, VE> ra[CH];
  Chunk<TB, L, VE> rb[BKN ? 1 : CH];
  BlockKN<TB, L, VE> kb[BKN ? KNQ : 1];

  accv_t acc[NB][NB];
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[i][j][v] = (acc_t)0;

  auto gload = [&](int k0) {
#pragma unroll
    for (int q = 0; q < CH; ++q) {
      const int c = tid + 256 * q, row = c >> 3, cc = c & 7;
      ra[q].load(Ab + (int64_t)row * n + k0 + cc * VE);
      if constexpr (!BKN) rb[q].load(Bb + (int64_t)row * n + k0 + cc * VE);
    }
    if constexpr (BKN) {
#pragma unroll
      for (int q = 0; q < KNQ; ++q) {
        const int blk = tid + 256 * q;
        if (KNB % 256 == 0 || blk < KNB) {
          const int jb = blk % (T / VE), kq = blk / (T / VE);
          kb[q].load(Bb + (int64_t)(k0 + kq * VE) * n + jb * VE, n);
        }
      }
    }
  };
  auto sstore = [&](int buf) {
    unsigned char* a = sA(buf);
    unsigned char* bb = sB(buf);
#pragma unroll
    for (int q = 0; q < CH; ++q) {
      const int c = tid + 256 * q, row = c >> 3, cc = c & 7;
      ra[q].store(a + row * ROWB + cc * 16);
      if constexpr (!BKN) rb[q].store(bb + row * ROWB + cc * 16);
    }
    if constexpr (BKN) {
#pragma unroll
      for (int q = 0; q < KNQ; ++q) {
        const int blk = tid + 256 * q;
        if (KNB % 256 == 0 || blk < KNB) {
          const int jb = blk % (T / VE), kq = blk / (T / VE);
          kb[q].store_t(bb + (jb * VE) * ROWB + kq * VE * (int)sizeof(L), ROWB);
        }
      }
    }
  };

  // Stage s computes from buffer s % 2 while the loads of stage s + 1 are in
  // flight; their registers go to the other buffer after the compute, and one
  // barrier per stage publishes them.
  gload(0);
  sstore(0);
  __syncthreads();
  int nstage = n / BK;
  if (ext.k) nstage = min(nstage, max(0, (ext.k[mat] + BK - 1) / BK));
  for (int s = 0; s < nstage; ++s) {
    const int cur = s & 1;
    if (s + 1 < nstage) gload((s + 1) * BK);
    const unsigned char* a_s = sA(cur);
    const unsigned char* b_s = sB(cur);
#pragma unroll
    for (int r = 0; r < NREAD; ++r) {
      frag_t a[NB], b[NB];
      const int off = (r * 4 * VE + grp * VE) * (int)sizeof(L);
#pragma unroll
      for (int i = 0; i < NB; ++i)
        a[i] = *reinterpret_cast<const frag_t*>(a_s + (wm * WT + i * 16 + i16) * ROWB + off);
#pragma unroll
      for (int j = 0; j < NB; ++j)
        b[j] = *reinterpret_cast<const frag_t*>(b_s + (wn * WT + j * 16 + i16) * ROWB + off);
#pragma unroll
      for (int u = 0; u < VE / KV; ++u)
#pragma unroll
        for (int i = 0; i < NB; ++i)
#pragma unroll
          for (int j = 0; j < NB; ++j) acc[i][j] = Tr::mma(a[i], b[j], u, acc[i][j]);
    }
    if (s + 1 < nstage) sstore(cur ^ 1);
    __syncthreads();
  }

  // Epilogue.
  TC* C = g.C ? reinterpret_cast<TC*>(g.C) + mat * g.stride : nullptr;
  TC* C2 = g.C2 ? reinterpret_cast<TC*>(g.C2) + mat * g.stride : nullptr;
  _Float16* Ch = g.Ch ? reinterpret_cast<_Float16*>(g.Ch) + mat * g.stride : nullptr;
  _Float16* C2h = g.C2h ? reinterpret_cast<_Float16*>(g.C2h) + mat * g.stride : nullptr;
  const TC* D = g.D ? reinterpret_cast<const TC*>(g.D) + mat * g.stride : nullptr;
  const bool diag = g.sym && ti == tj;
  const bool mirror = g.sym != 0;

  if constexpr (sizeof(acc_t) == 4) {
    // Stage the tile in LDS ([T][T+1] floats, conflict-free by rows and by
    // columns), then write whole rows with 16-byte stores.  The mirrored tile
    // (symmetric mode) and the transposed output read the staged tile by
    // columns; a diagonal tile takes its lower triangle from its upper one.
    constexpr int LP = T + 1;
    float* sC = reinterpret_cast<float*>(smem);
    static_assert(T * LP * 4 <= 4 * T * ROWB, "C tile must fit the operand buffers");
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          sC[(wm * WT + i * 16 + Tr::row(grp, v)) * LP + wn * WT + j * 16 + i16] = acc[i][j][v];
    __syncthreads();
    auto emit = [&](int oti, int otj, bool transposed, bool upper) {
      for (int e = tid; e < T * T / 4; e += 256) {
        const int r = e / (T / 4), c4 = (e - r * (T / 4)) * 4;
        const int R = oti * T + r;
        const int64_t base = (int64_t)R * n + otj * T + c4;
        float x[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          int sr = transposed ? c4 + q : r, sc = transposed ? r : c4 + q;
          if (upper && sr > sc) { const int tmp = sr; sr = sc; sc = tmp; }
          x[q] = sC[sr * LP + sc];
        }
        double y[4];
        double dv[4] = {0.0, 0.0, 0.0, 0.0};
        if (D) {
          if constexpr (sizeof(TC) == 4) {
            const floatx4 d4 = *reinterpret_cast<const floatx4*>(D + base);
#pragma unroll
            for (int q = 0; q < 4; ++q) dv[q] = (double)d4[q];
          } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) dv[q] = (double)D[base + q];
          }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          y[q] = epi_c(g.alpha, (double)x[q], D ? g.beta : 0.0, dv[q], R == otj * T + c4 + q ? g.gamma : 0.0);
        }
        if constexpr (sizeof(TC) == 4) {
          const floatx4 yf = floatx4{(float)y[0], (float)y[1], (float)y[2], (float)y[3]};
          if (C) *reinterpret_cast<floatx4*>(C + base) = yf;
          if (Ch) store_h4(Ch + base, yf);
          if (C2 || C2h) {
            floatx4 z;
#pragma unroll
            for (int q = 0; q < 4; ++q) z[q] = (float)epi_c2(g.alpha2, y[q], R == otj * T + c4 + q ? g.gamma2 : 0.0);
            if (C2) *reinterpret_cast<floatx4*>(C2 + base) = z;
            if (C2h) store_h4(C2h + base, z);
          }
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) put<TC>(C + base + q, y[q]);
          if (C2) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
              put<TC>(C2 + base + q, epi_c2(g.alpha2, y[q], R == otj * T + c4 + q ? g.gamma2 : 0.0));
          }
        }
      }
    };
    if (g.transC) {
      emit(tj, ti, true, false);
    } else if (diag) {
      emit(ti, tj, false, true);
    } else {
      emit(ti, tj, false, false);
      if (mirror) emit(tj, ti, true, false);
    }
    return;
  }

#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = wm * WT + i * 16 + Tr::row(grp, v);
        const int col = wn * WT + j * 16 + i16;
        if (diag && row > col) continue;
        const int R = ti * T + row, Cc = tj * T + col;
        const double x = epi_c(g.alpha, (double)acc[i][j][v], D ? g.beta : 0.0,
                               D ? (double)D[(int64_t)R * n + Cc] : 0.0, R == Cc ? g.gamma : 0.0);
        if (g.transC) {
          put<TC>(C + (int64_t)Cc * n + R, x);
          continue;
        }
        put<TC>(C + (int64_t)R * n + Cc, x);
        double x2 = 0.0;
        if (C2) {
          x2 = epi_c2(g.alpha2, x, R == Cc ? g.gamma2 : 0.0);
          put<TC>(C2 + (int64_t)R * n + Cc, x2);
        }
        if (mirror && R != Cc) {
          put<TC>(C + (int64_t)Cc * n + R, x);
          if (C2) put<TC>(C2 + (int64_t)Cc * n + R, x2);
        }
      }
}

// Tile lists: the tiles of a product with extents, listed matrix by matrix
// and cut into 8 contiguous ranges of about equal cost (see
// tile_list_kernel); range x goes to XCD x (the hardware deals workgroups to
// the XCDs round-robin), whose workgroups walk it.  Packed tile:
// matrix << 16 | ti << 8 | tj.
struct TileList {
  const int32_t* tiles;
  const int32_t* cut;  // [9]
};

template <Mma MM, int T, bool BKN, typename TA, typename TB, typename TC>
__global__ __launch_bounds__(256, 2) void gemm_kernel(GemmArgs g, Extents ext, TileList tl) {
  using L = typename MmaTraits<MM>::lds_t;
  constexpr int ROWB = MmaTraits<MM>::BK * (int)sizeof(L) + 16;
  __shared__ __attribute__((aligned(16))) unsigned char smem[4 * T * ROWB];
  if (tl.tiles) {
    const int x = blockIdx.x & 7, l = blockIdx.x >> 3, per = gridDim.x >> 3;
    for (int i = tl.cut[x] + l; i < tl.cut[x + 1]; i += per) {
      const int32_t p = tl.tiles[i];
      gemm_tile<MM, T, BKN, TA, TB, TC>(g, ext, p >> 16, (p >> 8) & 255, p & 255, smem);
      __syncthreads();  // the epilogue's reads of LDS end before the next tile's stage stores
    }
    return;
  }
  const int64_t w = xcd_remap((int64_t)blockIdx.x, g.total);
  const int64_t mat = w / g.tiles;
  int t = (int)(w - mat * g.tiles);
  int ti, tj;
  if (g.sym) {
    ti = 0;
    int rowlen = g.nt;
    while (t >= rowlen) { t -= rowlen; ++ti; --rowlen; }
    tj = ti + t;
  } else {
    ti = t / g.nt;
    tj = t - ti * g.nt;
  }
  gemm_tile<MM, T, BKN, TA, TB, TC>(g, ext, mat, ti, tj, smem);
}

// Builds up to 4 tile lists for products with extents, one workgroup of
// 1024 threads per list.  A matrix b contributes the tiles (ti, tj) with
// ti T < r[b] and tj T < c[b] (and ti <= tj with sym), row-major; a tile
// costs its k-stages, min(n / BK, ceil(k[b] / BK)), at least 1.  Prefix
// sums of tile counts and costs over the matrices (chunk sums, a scan of
// the 1024 chunk sums in LDS, chunk walks) give each matrix's first list
// slot and cost offset; cut[x] is the first tile whose cost offset reaches
// x C / 8 (C the total cost), found by binary search over the matrices.
// Within each range the tiles are then put in order of decreasing cost (a
// counting sort on the k-stage count): the range's workgroups take its
// tiles round-robin, so the costly tiles are spread over them first
// (longest-processing-time order) instead of falling to a few workgroups
// where blocks of one shape sit together.  Every tile is computed the same
// way in any order.
struct TileListSpec {
  const int32_t* r;
  const int32_t* c;
  const int32_t* k;
  int sym;
  int32_t* tiles;  // [matrices * (n/T)^2]
  int32_t* cut;    // [9]
  int32_t* tpre;   // [matrices] scratch: first list slot of each matrix
  int64_t* cpre;   // [matrices] scratch: cost before each matrix
  int32_t* tmp;    // [matrices * (n/T)^2] scratch: the reordered ranges
};
struct TileListArgs {
  TileListSpec s[4];
  int64_t nmat;
  int n, T, BK;
};

__global__ __launch_bounds__(1024) void tile_list_kernel(TileListArgs a) {
  const TileListSpec sp = a.s[blockIdx.x];
  __shared__ int32_t tsum[1024];
  __shared__ int64_t csum[1024];
  __shared__ int32_t lcut[9];
  __shared__ int32_t hist[256];
  const int tid = threadIdx.x;
  const int nt = a.n / a.T, nsmax = a.n / a.BK;
  const int64_t ch = (a.nmat + 1023) / 1024;
  const int64_t m0 = min(a.nmat, (int64_t)tid * ch), m1 = min(a.nmat, m0 + ch);
  auto info = [&](int64_t m, int& cnt, int& rt, int& ct, int& nst) {
    rt = sp.r ? min(nt, (max(sp.r[m], 0) + a.T - 1) / a.T) : nt;
    ct = sp.c ? min(nt, (max(sp.c[m], 0) + a.T - 1) / a.T) : nt;
    if (sp.sym) {
      const int rr = min(rt, ct);
      cnt = rr * ct - rr * (rr - 1) / 2;  // sum over ti < rr of (ct - ti)
    } else {
      cnt = rt * ct;
    }
    nst = sp.k ? min(nsmax, max(1, (max(sp.k[m], 0) + a.BK - 1) / a.BK)) : nsmax;
  };
  int32_t ts = 0;
  int64_t cs = 0;
  for (int64_t m = m0; m < m1; ++m) {
    int cnt, rt, ct, nst;
    info(m, cnt, rt, ct, nst);
    ts += cnt;
    cs += (int64_t)cnt * nst;
  }
  tsum[tid] = ts;
  csum[tid] = cs;
  __syncthreads();
  // inclusive scan of the chunk sums (Hillis-Steele)
  for (int off = 1; off < 1024; off <<= 1) {
    const int32_t tv = tid >= off ? tsum[tid - off] : 0;
    const int64_t cv = tid >= off ? csum[tid - off] : 0;
    __syncthreads();
    tsum[tid] += tv;
    csum[tid] += cv;
    __syncthreads();
  }
  int32_t tp = tsum[tid] - ts;
  int64_t cp = csum[tid] - cs;
  for (int64_t m = m0; m < m1; ++m) {
    int cnt, rt, ct, nst;
    info(m, cnt, rt, ct, nst);
    sp.tpre[m] = tp;
    sp.cpre[m] = cp;
    for (int ti = 0, j = 0; ti < rt; ++ti)
      for (int tj = sp.sym ? ti : 0; tj < ct; ++tj, ++j) sp.tiles[tp + j] = (int32_t)((m << 16) | (ti << 8) | tj);
    tp += cnt;
    cp += (int64_t)cnt * nst;
  }
  __syncthreads();  // tpre / cpre of every matrix written
  const int32_t N = tsum[1023];
  const int64_t C = csum[1023];
  if (tid <= 8) {
    int32_t cut = tid == 0 ? 0 : N;
    if (tid > 0 && tid < 8 && a.nmat > 0) {
      const int64_t target = C * tid / 8;
      // last matrix whose cost offset is <= target
      int64_t lo = 0, hi = a.nmat - 1;
      while (lo < hi) {
        const int64_t mid = (lo + hi + 1) / 2;
        if (sp.cpre[mid] <= target) lo = mid;
        else hi = mid - 1;
      }
      int cnt, rt, ct, nst;
      info(lo, cnt, rt, ct, nst);
      const int64_t j = min((int64_t)cnt, (target - sp.cpre[lo] + nst - 1) / nst);
      cut = (int32_t)(sp.tpre[lo] + j);
    }
    sp.cut[tid] = cut;
    lcut[tid] = cut;
  }
  __syncthreads();  // the list (global) and the cuts (LDS) are complete
  // per range: counting sort on key nsmax - (k-stages), bins in LDS
  constexpr int NB = 256;
  for (int x = 0; x < 8; ++x) {
    const int lo = lcut[x], hi = lcut[x + 1];
    if (hi - lo < 2) continue;
    if (tid < NB) hist[tid] = 0;
    __syncthreads();
    auto key = [&](int32_t pk) {
      int cnt, rt, ct, nst;
      info(pk >> 16, cnt, rt, ct, nst);
      return min(NB - 1, max(0, nsmax - nst));
    };
    for (int i = lo + tid; i < hi; i += 1024) atomicAdd(&hist[key(sp.tiles[i])], 1);
    __syncthreads();
    if (tid == 0) {
      int acc = 0;
      for (int q = 0; q < NB; ++q) {
        const int h = hist[q];
        hist[q] = acc;
        acc += h;
      }
    }
    __syncthreads();
    for (int i = lo + tid; i < hi; i += 1024) {
      const int32_t pk = sp.tiles[i];
      sp.tmp[lo + atomicAdd(&hist[key(pk)], 1)] = pk;
    }
    __syncthreads();
    for (int i = lo + tid; i < hi; i += 1024) sp.tiles[i] = sp.tmp[i];
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Persistent 128 x 128-tile product for float32 and float64 operands of one
// type (n a multiple of 128), NT (B row-major, k contiguous) or NN (B
// k-major), with every mode of gemm_kernel: D operand, second output,
// symmetric (upper tiles, mirrored) and transposed output (NT).
//
// Same scheme as the large-tile NN product: persistent grid (two workgroups
// of 4 waves per CU, 64 KB of LDS each), direct-to-LDS stage loads one stage
// ahead, fence-free barriers, vector stores straight from the accumulators.
// A stage holds 128 B of k per operand row (32 floats or 16 doubles):
//   A tile  [128 rows][128 B], chunks swizzled by P::aswz: lds_swz, or
//           lds_swz_t for float64, whose A fragments take the rows of a
//           16-row group in the order 4 (i & 3) + (i >> 2).
//   B (NT)  [128 rows][128 B], swizzled by lds_swz, with the LDS row order permuted:
//           output column wn*64 + 4 c + jb (lane c, column block jb) comes
//           from B-tile row wn*64 + 4 c + jb, stored at LDS row
//           wn*64 + 16 jb + c, so a fragment read covers 16 consecutive LDS
//           rows, as for A.
//   B (NN)  [k rows][128 columns], B's own layout; a 16-byte read gives VE
//           consecutive columns of one k-row, so column block jb of lane c
//           is column wn*64 + (jb / VE) 16 VE + VE c + jb % VE.
// The float64 matrix core returns row grp + 4 v of a 16 x 16 block in value
// v of lane group grp; A-lane row r reads tile row 4 (r % 4) + r / 4, which
// turns that into row 4 grp + v, as for float32.  A lane thus owns 4
// consecutive rows and runs of consecutive columns of each block: vector
// runs for the direct output (along columns) and for the mirrored or
// transposed output (along rows).  k is walked in the same order as in
// gemm_kernel, so the results are bit-identical to it.
//
// D may alias C: each element is read before any write to it (a tile's
// stores follow its loads, mirrored writes reach only lower tiles, whose D
// is never read).  float32 reads D during the tile's last k-stage, so its
// latency hides behind the MFMAs; float64 (twice the registers) reads it
// in the epilogue.
// ---------------------------------------------------------------------------
constexpr int P128_T = 128;
constexpr int P128_TILE_BYTES = P128_T * 128;  // 16 KB per operand and stage

// Operand type EI -> 16-byte fragment, accumulator, output type and the
// k-steps (MFMAs) one fragment feeds.  float32/float64 fragments hold 4/2
// consecutive k, one per 16x16x4 MFMA; a bfloat16 or half fragment holds
// the 8 k a lane supplies to one 16x16x32 MFMA (NT only).
template <typename EI> struct P128;
template <> struct P128<float> {
  using acc_t = floatx4;
  using frag_t = floatx4;
  using out_t = float;
  static constexpr int VE = 4, KS = 4;
  static __device__ __forceinline__ acc_t mma_s(float a, float b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ acc_t mma(const frag_t& a, const frag_t& b, int u, acc_t c) {
    return mma_s(a[u], b[u], c);
  }
  static __device__ __forceinline__ int arow(int r) { return r; }
  static __device__ __forceinline__ int aswz(int m) { return lds_swz(m); }
};
template <> struct P128<double> {
  using acc_t = doublex4;
  using frag_t = doublex2;
  using out_t = double;
  static constexpr int VE = 2, KS = 2;
  static __device__ __forceinline__ acc_t mma_s(double a, double b, acc_t c) {
    return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ acc_t mma(const frag_t& a, const frag_t& b, int u, acc_t c) {
    return mma_s(a[u], b[u], c);
  }
  static __device__ __forceinline__ int arow(int r) { return 4 * (r & 3) + (r >> 2); }
  static __device__ __forceinline__ int aswz(int m) { return lds_swz_t(m); }
};
template <> struct P128<__bf16> {
  using acc_t = floatx4;
  using frag_t = bf16x8;
  using out_t = float;
  static constexpr int VE = 8, KS = 1;
  static __device__ __forceinline__ acc_t mma(const frag_t& a, const frag_t& b, int, acc_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ int arow(int r) { return r; }
  static __device__ __forceinline__ int aswz(int m) { return lds_swz(m); }
};

template <> struct P128<_Float16> {
  using acc_t = floatx4;
  using frag_t = halfx8;
  using out_t = float;
  static constexpr int VE = 8, KS = 1;
  static __device__ __forceinline__ acc_t mma(const frag_t& a, const frag_t& b, int, acc_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ int arow(int r) { return r; }
  static __device__ __forceinline__ int aswz(int m) { return lds_swz(m); }
};

// LDS row -> B-tile row of an NT operand (the inverse of
// j -> (j & 64) | 16 (j & 3) | ((j >> 2) & 15))
__device__ __forceinline__ int p128_brow(int rho) { return (rho & 64) | (4 * (rho & 15)) | ((rho >> 4) & 3); }

// RUN consecutive elements with 16-byte accesses
template <typename E, int RUN> __device__ __forceinline__ void store_run(E* p, const E* v) {
#pragma unroll
  for (int s = 0; s < RUN * (int)sizeof(E) / 16; ++s) {
    if constexpr (sizeof(E) == 4)
      *reinterpret_cast<floatx4*>(p + 4 * s) = floatx4{v[4 * s], v[4 * s + 1], v[4 * s + 2], v[4 * s + 3]};
    else
      *reinterpret_cast<doublex2*>(p + 2 * s) = doublex2{v[2 * s], v[2 * s + 1]};
  }
}
// RUN consecutive half copies of float32 results (4 per 8-byte store)
template <typename E, int RUN> __device__ __forceinline__ void store_run_h(_Float16* p, const E* v) {
  static_assert(RUN % 4 == 0, "half runs of 4");
#pragma unroll
  for (int s = 0; s < RUN / 4; ++s)
    store_h4(p + 4 * s, floatx4{(float)v[4 * s], (float)v[4 * s + 1], (float)v[4 * s + 2], (float)v[4 * s + 3]});
}
template <typename E, int RUN> __device__ __forceinline__ void load_run(const E* p, E* v) {
#pragma unroll
  for (int s = 0; s < RUN * (int)sizeof(E) / 16; ++s) {
    if constexpr (sizeof(E) == 4) {
      const floatx4 t = *reinterpret_cast<const floatx4*>(p + 4 * s);
      v[4 * s] = t[0]; v[4 * s + 1] = t[1]; v[4 * s + 2] = t[2]; v[4 * s + 3] = t[3];
    } else {
      const doublex2 t = *reinterpret_cast<const doublex2*>(p + 2 * s);
      v[2 * s] = t[0]; v[2 * s + 1] = t[1];
    }
  }
}

// TL: the workgroups walk a tile list (products whose blocks have valid
// extents: the list holds only the tiles inside each block's rows and
// columns, cut into 8 ranges of equal cost, one per XCD), and each tile's
// k-loop stops at its matrix's inner extent (kext, in elements; the zero
// padding beyond it makes that exact).  Partial tiles at the extents' edges
// are computed whole: their padding rows and columns come out zero.
template <typename E, bool NN, bool TL>
__global__ __launch_bounds__(256, 2) void gemm_p128_kernel(GemmArgs g, TileList tl, const int32_t* kext) {
  using P = P128<E>;
  using EO = typename P::out_t;  // C, D, C2
  using acc_t = typename P::acc_t;
  using frag_t = typename P::frag_t;
  constexpr int T = P128_T, VE = P::VE, BK = 128 / (int)sizeof(E), TB = P128_TILE_BYTES, SB = 2 * TB;
  constexpr int RB = T * (int)sizeof(E);  // bytes per k-row of an NN B tile
  constexpr int RUN = NN ? VE : 4;        // consecutive output columns per lane and run
  constexpr bool PREFETCH_D = sizeof(EO) == 4;
  constexpr bool HALF_OUT = std::is_same<E, _Float16>::value;
  static_assert(!NN || P::KS > 1, "NN operands need fragments of one k per MFMA");
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * SB];
  const int per = gridDim.x >> 3;
  const int x = blockIdx.x & 7, l = blockIdx.x >> 3;
  int64_t first;
  int ntile;
  if constexpr (TL) {
    const int c0 = tl.cut[x], c1 = tl.cut[x + 1];
    if (c0 + l >= c1) return;
    first = c0 + l;
    ntile = (c1 - c0 - l + per - 1) / per;
  } else {
    const int64_t q = g.total >> 3, r = g.total & 7;
    const int64_t mine = q + (x < r ? 1 : 0);
    if (mine <= l) return;
    first = x * q + (x < r ? x : r) + l;
    ntile = (int)((mine - l + per - 1) / per);
  }
  const int n = g.n, nst = n / BK;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int i16 = lane & 15, grp = lane >> 4;
  const E* Ag = reinterpret_cast<const E*>(g.A);
  const E* Bg = reinterpret_cast<const E*>(g.B);
  auto colmap = [&](int jb) { return NN ? (jb / VE) * 16 * VE + VE * i16 + jb % VE : 4 * i16 + jb; };

  // Each wave issues 4 A and 4 B loads of 1 KB per stage; lane offsets in elements.
  int aoff[4], boff[4];
#pragma unroll
  for (int qq = 0; qq < 4; ++qq) {
    const int row = 8 * (4 * wave + qq) + (lane >> 3), pos = lane & 7;
    aoff[qq] = row * n + VE * (pos ^ P::aswz(row));
    if constexpr (NN) {
      const int byte = (4 * wave + qq) * 1024 + 16 * lane;
      boff[qq] = (byte / RB) * n + (byte % RB) / (int)sizeof(E);
    } else {
      boff[qq] = p128_brow(row) * n + VE * (pos ^ lds_swz(row));
    }
  }
  // tile it of this workgroup: matrix offset, tile indices and k-stages
  auto coords = [&](int it, int64_t& moff, int& ti, int& tj, int& ns) {
    ns = nst;
    if constexpr (TL) {
      const int32_t pk = tl.tiles[first + (int64_t)it * per];
      const int64_t mat = pk >> 16;
      ti = (pk >> 8) & 255;
      tj = pk & 255;
      moff = mat * g.stride;
      if (kext) ns = min(nst, max(1, (max(kext[mat], 0) + BK - 1) / BK));
      return;
    }
    const int64_t w = first + (int64_t)it * per;
    const int64_t mat = w / g.tiles;
    int t = (int)(w - mat * g.tiles);
    if (g.sym) {
      ti = 0;
      int rowlen = g.nt;
      while (t >= rowlen) {
        t -= rowlen;
        ++ti;
        --rowlen;
      }
      tj = ti + t;
    } else {
      ti = t / g.nt;
      tj = t - ti * g.nt;
    }
    moff = mat * g.stride;
  };
  auto bbase = [&](int64_t mo, int tj) { return Bg + mo + (NN ? (int64_t)tj * T : (int64_t)tj * T * n); };
  int lt = 0, lk = 0;
  int64_t cmo;  // compute cursor: the current tile's matrix offset, tile indices and k-stages
  int cti, ctj, cns;
  coords(0, cmo, cti, ctj, cns);
  int lns = cns;  // k-stages of the tile being loaded
  const E* LA = Ag + cmo + (int64_t)cti * T * n;
  const E* LB = bbase(cmo, ctj);
  auto issue = [&](int buf) {
    unsigned char* sa = smem + buf * SB;
    unsigned char* sb = sa + TB;
    const E* pa = LA + lk * BK;
    const E* pb = NN ? LB + (int64_t)lk * BK * n : LB + lk * BK;
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      __builtin_amdgcn_global_load_lds((const void*)(pa + aoff[qq]), (void*)(sa + (4 * wave + qq) * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(pb + boff[qq]), (void*)(sb + (4 * wave + qq) * 1024), 16, 0, 0);
    }
  };
  auto advance = [&]() {
    if (++lk == lns) {
      lk = 0;
      if (++lt < ntile) {
        int64_t mo;
        int ti, tj;
        coords(lt, mo, ti, tj, lns);
        LA = Ag + mo + (int64_t)ti * T * n;
        LB = bbase(mo, tj);
      }
    }
  };

  acc_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = acc_t{0, 0, 0, 0};
  const EO* Dg = reinterpret_cast<const EO*>(g.D);
  EO dpre[PREFETCH_D ? 4 : 1][4][4];  // D of the current tile [i][v][jb] (float32)
  const bool plain = g.alpha == 1.0 && g.gamma == 0.0 && Dg == nullptr && g.C2 == nullptr && g.C2h == nullptr;
  int total_steps = ntile * nst;
  if constexpr (TL) {
    if (kext) {
      total_steps = 0;
      for (int it = 0; it < ntile; ++it) {
        int64_t mo;
        int ti, tj, ns;
        coords(it, mo, ti, tj, ns);
        total_steps += ns;
      }
    }
  }
  auto dload = [&](int i, EO (*d)[4]) {  // D at the lane's outputs of row block i
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
      for (int h = 0; h < 4 / RUN; ++h)
        load_run<EO, RUN>(Dg + cmo + (int64_t)(cti * T + wm * 64 + i * 16 + 4 * grp + v) * n + ctj * T + wn * 64 +
                             colmap(h * RUN),
                         &d[v][h * RUN]);
  };

  issue(0);
  advance();
  wait_vmcnt0();
  barrier_no_fence();
  int ck = 0, ct = 0;
  for (int step = 0; step < total_steps; ++step) {
    const bool more = step + 1 < total_steps;
    if (more) issue((step + 1) & 1);
    if constexpr (PREFETCH_D) {
      if (Dg && ck == cns - 1) {
#pragma unroll
        for (int i = 0; i < 4; ++i) dload(i, dpre[i]);
      }
    }
    const unsigned char* sa = smem + (step & 1) * SB;
    const unsigned char* sb = sa + TB;
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const int kc = rr * 4 + grp;
      frag_t a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = wm * 64 + i * 16 + P::arow(i16);
        a[i] = *reinterpret_cast<const frag_t*>(sa + m * 128 + 16 * (kc ^ P::aswz(m)));
      }
      if constexpr (NN) {
        // b[u * (4 / VE) + h]: k-row kc VE + u, columns wn*64 + h 16 VE + VE i16 ..
#pragma unroll
        for (int u = 0; u < VE; ++u)
#pragma unroll
          for (int h = 0; h < 4 / VE; ++h)
            b[u * (4 / VE) + h] =
                *reinterpret_cast<const frag_t*>(sb + (kc * VE + u) * RB + wn * 64 * (int)sizeof(E) + h * 256 + 16 * i16);
#pragma unroll
        for (int u = 0; u < VE; ++u)
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
              acc[i][j] = P::mma_s(a[i][u], b[u * (4 / VE) + j / VE][j % VE], acc[i][j]);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int rho = wn * 64 + 16 * j + i16;
          b[j] = *reinterpret_cast<const frag_t*>(sb + rho * 128 + 16 * (kc ^ lds_swz(rho)));
        }
#pragma unroll
        for (int u = 0; u < P::KS; ++u)
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = P::mma(a[i], b[j], u, acc[i][j]);
      }
    }
    if (more) advance();
    wait_vmcnt0();
    barrier_no_fence();
    if (++ck < cns) continue;
    ck = 0;
    EO* C = g.C ? reinterpret_cast<EO*>(g.C) + cmo : nullptr;
    EO* C2 = g.C2 ? reinterpret_cast<EO*>(g.C2) + cmo : nullptr;
    // half copies: float32 results of half-operand products only
    _Float16* Ch = HALF_OUT && g.Ch ? reinterpret_cast<_Float16*>(g.Ch) + cmo : nullptr;
    _Float16* C2h = HALF_OUT && g.C2h ? reinterpret_cast<_Float16*>(g.C2h) + cmo : nullptr;
    const bool two = C2 || C2h;
    const int R0 = cti * T + wm * 64, C0 = ctj * T + wn * 64;
    const bool diag = g.sym && cti == ctj;
    const bool mirror = (g.sym && !diag) || g.transC;
    const bool direct = !g.transC;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      EO d[4][4];  // [v][jb]
      if constexpr (PREFETCH_D) {
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
          for (int j = 0; j < 4; ++j) d[v][j] = dpre[i][v][j];
      } else {
        if (Dg) dload(i, d);
      }
      // output (v, jb) of row block i: C value, and the second output from it
      auto val = [&](int v, int j, double& t) {
        const int R = R0 + i * 16 + 4 * grp + v, Cc = C0 + colmap(j);
        t = epi_c(g.alpha, (double)acc[i][j][v], Dg ? g.beta : 0.0, Dg ? (double)d[v][j] : 0.0,
                  R == Cc ? g.gamma : 0.0);
        return plain ? (EO)acc[i][j][v] : (EO)t;
      };
      auto val2 = [&](int v, int j, double t) {
        const int R = R0 + i * 16 + 4 * grp + v, Cc = C0 + colmap(j);
        return (EO)epi_c2(g.alpha2, t, R == Cc ? g.gamma2 : 0.0);
      };
      if (diag) {
        // diagonal tile: the upper element (R <= Cc) is written in place and mirrored
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int R = R0 + i * 16 + 4 * grp + v, Cc = C0 + colmap(j);
            if (R > Cc) continue;
            double t;
            const EO y = val(v, j, t);
            if (C) {
              C[(int64_t)R * n + Cc] = y;
              C[(int64_t)Cc * n + R] = y;
            }
            if (Ch) {
              Ch[(int64_t)R * n + Cc] = half_of((float)y);
              Ch[(int64_t)Cc * n + R] = half_of((float)y);
            }
            if (two) {
              const EO z = val2(v, j, t);
              if (C2) {
                C2[(int64_t)R * n + Cc] = z;
                C2[(int64_t)Cc * n + R] = z;
              }
              if (C2h) {
                C2h[(int64_t)R * n + Cc] = half_of((float)z);
                C2h[(int64_t)Cc * n + R] = half_of((float)z);
              }
            }
          }
        continue;
      }
      if (direct) {
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
          for (int h = 0; h < 4 / RUN; ++h) {
            const int64_t at = (int64_t)(R0 + i * 16 + 4 * grp + v) * n + C0 + colmap(h * RUN);
            EO y[RUN], z[RUN];
            double t[RUN];
#pragma unroll
            for (int e = 0; e < RUN; ++e) y[e] = val(v, h * RUN + e, t[e]);
            if (C) store_run<EO, RUN>(C + at, y);
            if constexpr (HALF_OUT) {
              if (Ch) store_run_h<EO, RUN>(Ch + at, y);
            }
            if (two) {
#pragma unroll
              for (int e = 0; e < RUN; ++e) z[e] = val2(v, h * RUN + e, t[e]);
              if (C2) store_run<EO, RUN>(C2 + at, z);
              if constexpr (HALF_OUT) {
                if (C2h) store_run_h<EO, RUN>(C2h + at, z);
              }
            }
          }
      }
      if (mirror) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t at = (int64_t)(C0 + colmap(j)) * n + R0 + i * 16 + 4 * grp;
          EO y[4], z[4];
          double t[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) y[v] = val(v, j, t[v]);
          if (C) store_run<EO, 4>(C + at, y);
          if constexpr (HALF_OUT) {
            if (Ch) store_run_h<EO, 4>(Ch + at, y);
          }
          if (two) {
#pragma unroll
            for (int v = 0; v < 4; ++v) z[v] = val2(v, j, t[v]);
            if (C2) store_run<EO, 4>(C2 + at, z);
            if constexpr (HALF_OUT) {
              if (C2h) store_run_h<EO, 4>(C2h + at, z);
            }
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = acc_t{0, 0, 0, 0};
    if (++ct < ntile) coords(ct, cmo, cti, ctj, cns);
  }
}

// ---------------------------------------------------------------------------
// Half-operand NN product with 256 x 256 tiles (n a multiple of 256), the
// Newton-DB products of the half-precision chains:
//     C = alpha A B + gamma I,   C2 = alpha2 C + gamma2 I,
// float32 results and, where later products read them, half copies.  A half
// k-stage of 64 values carries twice the matrix-core work of a float32 stage
// over the same bytes, so these products need the larger tile to stay ahead
// of their operand traffic: one persistent workgroup of 8 waves (128 x 64
// outputs each) per CU, stage loads straight into LDS one stage ahead,
// 128 KB of LDS (as the float32 NN product).  (Symmetric NT half products
// with half outputs only run on gemm_h256_sym_kernel, the others on the
// 128-tile kernel.)
//
// The matrix-core operands are swapped: the B side feeds the A operand of
// v_mfma_f32_16x16x32_f16 and the A side its B operand, so that lane
// (i16, grp) of a 16 x 16 block holds C[row i16][column 4 grp + v]: four
// consecutive columns, stored as one float4 (or 4-half) run.
//
// LDS layouts (16-byte chunks, XOR-swizzled so fragment reads spread over
// all banks):
//   A [256 rows][128 B of k], chunk c of LDS row r at c ^ lds_swz(r).
//   B [64 k-rows][256 columns], B's own k-major layout, chunk c of k-row k
//     at c ^ bswz(k).  Fragments come from ds_read_b64_tr_b16: in each group
//     of 16 lanes, lane 4 i + q addresses the 4 columns 4 q .. 4 q + 3 of
//     k-row k0 + i, and lane j receives column j of k-rows k0 .. k0 + 3 (the
//     transposed read gives lane j element j % 4 of lane 4 i + j / 4).  Two
//     such reads give a lane the 8 consecutive k of its column.
// Lane group grp supplies k 8 grp .. 8 grp + 7 of each 32-k MFMA, as in the
// other kernels; the per-element k order is the same, and so are the
// results, bit for bit.
// ---------------------------------------------------------------------------
constexpr int H256_T = 256;
constexpr int H256_BK = 64;
constexpr int H256_TILE_BYTES = H256_T * 128;              // 32 KB per operand and stage
constexpr int H256_LDS = 2 * 2 * H256_TILE_BYTES;           // 128 KB

__device__ __forceinline__ int h256_bswz(int k) { return 2 * ((k & 3) | (((k >> 3) & 3) << 2)); }

// vmcnt <= min(n, 63), n the vector stores issued after the awaited loads
__device__ __forceinline__ void wait_vmcnt_after_stores(int n) {
  if (n >= 63) __builtin_amdgcn_s_waitcnt((63 & 15) | (0x7 << 4) | (0xF << 8) | ((63 >> 4) << 14));
  else if (n >= 32) __builtin_amdgcn_s_waitcnt((32 & 15) | (0x7 << 4) | (0xF << 8) | ((32 >> 4) << 14));
  else __builtin_amdgcn_s_waitcnt(0x3f70);
}

typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef short shortx8 __attribute__((ext_vector_type(8)));

__global__ __launch_bounds__(512, 1) void gemm_h256_nn_kernel(GemmArgs g) {
  constexpr int T = H256_T, BK = H256_BK, TB = H256_TILE_BYTES, SB = 2 * TB;
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
  const int wm = wave >> 2, wn = wave & 3;
  const int i16 = lane & 15, grp = lane >> 4;
  const _Float16* Ag = reinterpret_cast<const _Float16*>(g.A);
  const _Float16* Bg = reinterpret_cast<const _Float16*>(g.B);

  // Each wave issues 4 A loads (8 rows x 128 B) and 4 B loads (2 k-rows x
  // 512 B) of 1 KB per stage; lane offsets in elements.
  int aoff[4], boff[4];
#pragma unroll
  for (int qq = 0; qq < 4; ++qq) {
    const int I = 4 * wave + qq;
    const int row = 8 * I + (lane >> 3), pos = lane & 7;
    aoff[qq] = row * n + 8 * (pos ^ lds_swz(row));
    const int k = 2 * I + (lane >> 5), p = lane & 31;
    boff[qq] = k * n + 8 * (p ^ h256_bswz(k));
  }
  auto coords = [&](int it, int64_t& moff, int& ti, int& tj) {
    const int64_t w = first + (int64_t)it * per;
    const int64_t mat = w / g.tiles;
    const int t = (int)(w - mat * g.tiles);
    ti = t / g.nt;
    tj = t - ti * g.nt;
    moff = mat * g.stride;
  };
  int lt = 0, lk = 0;
  int64_t cmo;
  int cti, ctj;
  coords(0, cmo, cti, ctj);
  const _Float16* LA = Ag + cmo + (int64_t)cti * T * n;
  const _Float16* LB = Bg + cmo + (int64_t)ctj * T;
  auto issue = [&](int buf) {
    unsigned char* sa = smem + buf * SB;
    unsigned char* sb = sa + TB;
    const _Float16* pa = LA + lk * BK;
    const _Float16* pb = LB + (int64_t)lk * BK * n;
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
  // byte offsets (within a B stage) of this lane's transposed reads for
  // column block j, first half of its k-group (the second half: + 4 k-rows)
  int troff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int k = 8 * grp + (i16 >> 2);
    const int col = wn * 64 + 16 * j + 4 * (i16 & 3);
    troff[j] = k * (T * 2) + 16 * ((col >> 3) ^ h256_bswz(k)) + 2 * (col & 7);
  }

  floatx4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  const bool plain = g.alpha == 1.0 && g.gamma == 0.0 && g.C2 == nullptr && g.C2h == nullptr;
  const int total_steps = ntile * nst;

  // stores per lane of one epilogue (one instruction per output and block)
  const int nstores = 32 * ((g.C ? 1 : 0) + (g.Ch ? 1 : 0) + (g.C2 ? 1 : 0) + (g.C2h ? 1 : 0));
  issue(0);
  advance();
  wait_vmcnt0();
  barrier_no_fence();
  int ck = 0, ct = 0;
  bool pre = false;  // the next stage was issued before the last epilogue's stores
  for (int step = 0; step < total_steps; ++step) {
    const bool more = step + 1 < total_steps;
    const bool pre_now = pre;
    pre = false;
    if (more && !pre_now) issue((step + 1) & 1);
    const unsigned char* sa = smem + (step & 1) * SB;
    const unsigned char* sb = sa + TB;
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const int kc = rr * 4 + grp;
      halfx8 a[8], b[4];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int m = wm * 128 + i * 16 + i16;
        a[i] = *reinterpret_cast<const halfx8*>(sa + m * 128 + 16 * (kc ^ lds_swz(m)));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        typedef __attribute__((address_space(3))) shortx4 lds_s4;
        const unsigned char* p0 = sb + rr * 32 * (T * 2) + troff[j];
        const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(p0));
        const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(p0 + 4 * (T * 2)));
        b[j] = __builtin_bit_cast(halfx8, shortx8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
      }
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(b[j], a[i], acc[i][j], 0, 0, 0);
    }
    if (more && !pre_now) advance();
    // A stage issued before the last epilogue's stores lets those stay in
    // flight: vector memory operations are counted in issue order.
    if (pre_now) wait_vmcnt_after_stores(nstores);
    else wait_vmcnt0();
    barrier_no_fence();
    if (++ck < nst) continue;
    ck = 0;
    // Every wave is done with buffer (step & 1): stage step + 2 goes into it
    // before this tile's stores, so the next stage wait need not drain them
    // (the stores used to cost 6-10% at n = 512).
    if (step + 2 < total_steps) {
      issue(step & 1);
      advance();
      pre = true;
    }
    float* C = g.C ? reinterpret_cast<float*>(g.C) + cmo : nullptr;
    float* C2 = g.C2 ? reinterpret_cast<float*>(g.C2) + cmo : nullptr;
    _Float16* Ch = g.Ch ? reinterpret_cast<_Float16*>(g.Ch) + cmo : nullptr;
    _Float16* C2h = g.C2h ? reinterpret_cast<_Float16*>(g.C2h) + cmo : nullptr;
    const bool two = C2 || C2h;
    const int R0 = cti * T + wm * 128, C0 = ctj * T + wn * 64;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int R = R0 + i * 16 + i16, c0 = C0 + 16 * j + 4 * grp;
        floatx4 y = acc[i][j], z;
        if (!plain) {
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const double t = epi_c(g.alpha, (double)acc[i][j][v], 0.0, 0.0, R == c0 + v ? g.gamma : 0.0);
            if (two) z[v] = (float)epi_c2(g.alpha2, t, R == c0 + v ? g.gamma2 : 0.0);
            y[v] = (float)t;
          }
        }
        const int64_t at = (int64_t)R * n + c0;
        if (C) *reinterpret_cast<floatx4*>(C + at) = y;
        if (Ch) store_h4(Ch + at, y);
        if (C2) *reinterpret_cast<floatx4*>(C2 + at) = z;
        if (C2h) store_h4(C2h + at, z);
      }
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (++ct < ntile) coords(ct, cmo, cti, ctj);
  }
}

}  // namespace shampoo
