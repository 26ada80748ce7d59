// Dense contractions of the tower: every linear layer and the conv2/conv3 implicit GEMMs.
//
//   C[m, n] = epilogue( sum_k A[m, k] * B[n, k] )
//
// A is an activation (row-major, K contiguous) or, for the 3x3 stride-2 convolutions, the
// im2col view of a channels-last activation generated on the fly by the loader (K ordered as
// tap-major, channel-minor, so each 8-element chunk is one contiguous 16-byte read of one input
// position; out-of-image taps and positions past a window's valid length read as zero).  B is a
// weight matrix [N, K] (PyTorch Linear layout; conv weights permuted to [out][tap][in] at pack
// time).  Epilogues fuse the bias, exact GELU, the fp32 residual update, the sinusoidal
// positions and the SwiGLU gate into the store.
//
// bf16 path: v_mfma_f32_32x32x16_bf16 on gfx950.  Workgroup tile 128x128, K step 64, four
// waves each owning a 64x64 sub-tile (2x2 MFMA blocks, fp32 accumulators).  Global loads of
// the next K step are issued into registers before the MFMAs of the current one and written
// to the second LDS buffer afterwards (LDS double buffering, one barrier per K step).  LDS
// rows are 128 bytes with the 16-byte chunk index XOR-swizzled by (row & 7), so the 32 rows a
// wave reads for one MFMA operand hit distinct banks.
//
// fp32 path (the fp32 tiny configuration): a 64x64 VALU tile with the same loaders and
// epilogues.
#include <algorithm>
#include <type_traits>

#include "ae_internal.h"

namespace ae {
namespace {

// ============================================================================================
// A-operand sources
// ============================================================================================
template <typename T>
struct ALinear {
  const T* A;
  int64_t lda;
  int64_t M;
  int32_t K;
  struct Row { const T* p; };
  struct KC { int k; bool ok; };
  __device__ bool tile_live(int64_t m0, int) const { return m0 < M; }
  __device__ Row row(int64_t r) const { return Row{r < M ? A + r * lda : nullptr}; }
  __device__ KC kc(int k) const { return KC{k, k < K}; }
  __device__ const T* ptr(const Row& x, const KC& c) const {
    return (x.p && c.ok) ? x.p + c.k : nullptr;
  }
  // byte-offset form for buffer loads: rows past M read as zero (offset beyond the range)
  struct BRow { uint32_t off; };
  __device__ BRow brow(int64_t r) const {
    return BRow{r < M ? (uint32_t)(r * lda * (int64_t)sizeof(T)) : 0x80000000u};
  }
  __device__ uint32_t boff(const BRow& x, const KC& c) const {
    return c.ok ? x.off + (uint32_t)(c.k * (int)sizeof(T)) : 0x80000000u;
  }
  __device__ int64_t bytes() const { return M * lda * (int64_t)sizeof(T); }
  __device__ const void* base() const { return A; }
};

// im2col view for a 3x3 stride-2 pad-1 conv.  GEMM row r is output position
// (window w, time t, freq f) with r = w * rows_per_win + t * Fout + f (rows_per_win = Lout_max *
// Fout, so tiles may straddle windows).  Per row the loader keeps the element offset of tap
// (freq 0, time 0) and a 9-bit mask of the taps that fall inside the window's valid image.
template <typename T>
struct AConv {
  const T* in;
  const Win* wins;
  int32_t C, Fin, Fout, Lin_max, level, rows_per_win, K;
  int64_t m_rows;
  struct Row { int32_t off; int32_t mask; };
  struct KC { int32_t toff; int32_t bit; bool ok; };
  __device__ int lout(const Win& wn) const { return level == 2 ? wn.L2 : wn.L3; }
  __device__ bool row_valid(int64_t r) const {
    if (r >= m_rows) return false;
    const int w = (int)(r / rows_per_win);
    const int t = (int)(r - (int64_t)w * rows_per_win) / Fout;
    return t < lout(wins[w]);
  }
  __device__ bool tile_live(int64_t m0, int bm) const {
    const int64_t last = min(m0 + bm - 1, m_rows - 1);
    if (m0 / rows_per_win != last / rows_per_win) return true;  // straddles two windows
    return row_valid(m0);
  }
  __device__ Row row(int64_t r) const {
    Row x{0, 0};
    if (r >= m_rows) return x;
    const int w = (int)(r / rows_per_win);
    const int loc = (int)(r - (int64_t)w * rows_per_win);
    const int t = loc / Fout, f = loc - (loc / Fout) * Fout;
    const Win wn = wins[w];
    if (t >= lout(wn)) return x;
    const int Lin = level == 2 ? wn.L1 : wn.L2;
    int m = 0;
#pragma unroll
    for (int da = 0; da < 3; ++da)
#pragma unroll
      for (int db = 0; db < 3; ++db) {
        const int ti = 2 * t - 1 + db, fi = 2 * f - 1 + da;
        if (ti >= 0 && ti < Lin && fi >= 0 && fi < Fin) m |= 1 << (da * 3 + db);
      }
    x.mask = m;
    x.off = ((w * Lin_max + (2 * t - 1)) * Fin + (2 * f - 1)) * C;
    return x;
  }
  __device__ KC kc(int k) const {
    KC c;
    c.ok = k < K;
    const int tap = k / C;
    const int ci = k - tap * C;
    const int da = tap / 3, db = tap - 3 * (tap / 3);  // frequency tap, time tap
    c.bit = 1 << tap;
    c.toff = (db * Fin + da) * C + ci;
    return c;
  }
  __device__ const T* ptr(const Row& x, const KC& c) const {
    return (c.ok && (x.mask & c.bit)) ? in + (x.off + c.toff) : nullptr;
  }
  using BRow = Row;
  __device__ BRow brow(int64_t r) const { return row(r); }
  __device__ uint32_t boff(const BRow& x, const KC& c) const {
    return (c.ok && (x.mask & c.bit)) ? (uint32_t)((x.off + c.toff) * (int)sizeof(T)) : 0x80000000u;
  }
  __device__ int64_t bytes() const { return (int64_t)wins_bytes; }
  __device__ const void* base() const { return in; }
  int64_t wins_bytes;  // bytes of the input activation
};

// ============================================================================================
// output row maps: element offset of (row, 0) in C, or -1 for rows that are not stored
// ============================================================================================
struct OLinear {
  int64_t M, ldc;
  __device__ int64_t off(int64_t r) const { return r < M ? r * ldc : -1; }
};

struct OConv {
  const Win* wins;
  int32_t rows_per_win, Fout, C, level, Lout_max;
  int64_t m_rows;
  __device__ int64_t off(int64_t r) const {
    if (r >= m_rows) return -1;
    const int w = (int)(r / rows_per_win);
    const int loc = (int)(r - (int64_t)w * rows_per_win);
    const int t = loc / Fout, f = loc - (loc / Fout) * Fout;
    const Win wn = wins[w];
    if (t >= (level == 2 ? wn.L2 : wn.L3)) return -1;
    if (level == 2) return (((int64_t)w * Lout_max + t) * Fout + f) * C;
    return ((int64_t)(wn.tok + t) * Fout + f) * C;  // token rows [tok][16][C]
  }
};

struct EpiP {
  const float* bias;
  void* C;
  const float* pe;
  const int32_t* tok_pos;
};

template <typename T> struct Store4x;
template <> struct Store4x<bf16_t> {
  __device__ static inline void put(bf16_t* p, float a, float b, float c, float d) {
    uint2 o;
    o.x = (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
    o.y = (uint32_t)f32_to_bf16(c) | ((uint32_t)f32_to_bf16(d) << 16);
    *reinterpret_cast<uint2*>(p) = o;
  }
};
template <> struct Store4x<float> {
  __device__ static inline void put(float* p, float a, float b, float c, float d) {
    *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
  }
};

template <int EPI, typename OT>
__device__ inline void epi_store(const EpiP& ep, int64_t off, int64_t row, int col, float v) {
  const float b = ep.bias ? ep.bias[col] : 0.0f;
  if constexpr (EPI == EPI_BIAS) {
    StoreT<OT>::put(reinterpret_cast<OT*>(ep.C) + off + col, v + b);
  } else if constexpr (EPI == EPI_BIAS_GELU) {
    StoreT<OT>::put(reinterpret_cast<OT*>(ep.C) + off + col, gelu_erf(v + b));
  } else if constexpr (EPI == EPI_RESADD) {
    float* p = reinterpret_cast<float*>(ep.C) + off + col;
    *p = *p + (v + b);
  } else if constexpr (EPI == EPI_STORE_F32) {
    reinterpret_cast<float*>(ep.C)[off + col] = v + b;
  }
}

// ============================================================================================
// bf16 MFMA kernel
// ============================================================================================
constexpr int NTHR = 256;

__device__ inline uint4 ld16(const bf16_t* p) {
  return p ? *reinterpret_cast<const uint4*>(p) : make_uint4(0u, 0u, 0u, 0u);
}

// Block tile BM x BN x BK, WGM x WGN waves, each owning (BM/WGM) x (BN/WGN) as TM x TN blocks
// of 32x32 MFMA output.  MINB workgroups are meant to share a CU (occupancy hint).  NPF register
// sets form a ring of K tiles in flight from HBM/L2, so a tile's loads are issued NPF tiles
// before it is written to LDS (the global load latency exceeds one tile of MFMA work).
template <int BM_, int BN_, int WGM_, int WGN_, int BK_ = 64, int MINB_ = 1, int NPF_ = 1>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, WGM = WGM_, WGN = WGN_, BK = BK_, MINB = MINB_;
  static constexpr int NPF = NPF_;  // K tiles in flight between global load and LDS store
  static constexpr int NW = WGM * WGN, NT = 64 * NW;  // waves, threads
  static constexpr int WTM = BM / WGM, WTN = BN / WGN;
  static constexpr int TM = WTM / 32, TN = WTN / 32;
  static constexpr int CPR = BK / 8;                   // 16-byte chunks per tile row
  static constexpr int RS = NT / CPR;                  // rows covered by one loader pass
  static constexpr int AR = BM / RS, BR = BN / RS;     // chunks per thread per K step
  static_assert(TM * 32 == WTM && TN * 32 == WTN && AR * RS == BM && BR * RS == BN, "tile");
  static_assert(BK == 32 || BK == 64, "BK");
};
using TileL = Tile<256, 256, 2, 2>;   // 4 waves, wave tile 128 x 128
using TileL8 = Tile<256, 256, 2, 4>;  // 8 waves, wave tile 128 x 64 (two waves per SIMD)
using TileL8b = Tile<256, 256, 4, 2>; // 8 waves, wave tile 64 x 128
using TileM = Tile<256, 128, 2, 2>;   // 4 waves, wave tile 128 x 64
using TileM8 = Tile<256, 128, 4, 2>;  // 8 waves, wave tile 64 x 64
using TileMk = Tile<256, 128, 2, 2, 32, 2>;  // 4 waves, BK 32, two workgroups per CU
using TileSk = Tile<128, 128, 2, 2, 32, 3>;  // 4 waves, BK 32, three workgroups per CU
using TileS = Tile<128, 128, 2, 2, 64, 2>;   // 4 waves, BK 64, two workgroups per CU
using TileSk3 = Tile<128, 128, 2, 2, 32, 3, 3>;  // + 3 tiles in flight
using TileSk2 = Tile<128, 128, 2, 2, 32, 3, 2>;
using TileMk3 = Tile<256, 128, 2, 2, 32, 2, 3>;
using TileM83 = Tile<256, 128, 4, 2, 32, 1, 3>;  // 8 waves, BK 32
using TileL83 = Tile<256, 256, 2, 4, 32, 1, 2>;  // 8 waves, BK 32, 2 in flight

// Workgroups are dispatched round-robin over the 8 XCDs; remap so that consecutive logical
// tiles (same A rows, neighbouring B columns) run on the same XCD and share its L2.
__device__ inline int xcd_remap(int bid, int G) {
  const int per = G / 8, rem = G % 8;
  const int x = bid % 8, i = bid / 8;
  return x < rem ? x * (per + 1) + i : rem * (per + 1) + (x - rem) * per + i;
}

// (m tile, n tile) of this workgroup: XCD remap, then groups of gm m-tiles walked column by
// column so that the workgroups resident at one time share A rows and B columns in L2.  All
// 32-bit and wave-uniform (kept in scalar registers).
struct TileCoord { int mt, nt; };
__device__ inline TileCoord tile_coord(int n_tiles, int gm) {
  const int G = gridDim.x;
  const int tile = xcd_remap(blockIdx.x, G);
  const int m_tiles = G / n_tiles;
  const int gsize = gm * n_tiles;
  const int g = tile / gsize;
  const int first_m = g * gm;
  const int gh = m_tiles - first_m < gm ? m_tiles - first_m : gm;
  const int in_g = tile - g * gsize;
  return TileCoord{__builtin_amdgcn_readfirstlane(first_m + in_g % gh),
                   __builtin_amdgcn_readfirstlane(in_g / gh)};
}

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Epilogue of SR staged accumulator rows (row-major, stride LDW floats) of one wave: rows
// rbase.., columns wcol..wcol+WTN-1.  Each lane handles 4 consecutive columns per step.
template <int EPI, typename OT, int WTN, int SR, class OM>
__device__ inline void epilogue_rows(const float* stg, int LDW, int64_t rbase, int wcol, int N,
                                     const OM& om, const EpiP& ep, int pe_ld, int lane) {
    if constexpr (EPI == EPI_SWIGLU) {
    constexpr int Q = WTN / 8;  // 4-wide outputs per row
    for (int idx = lane; idx < SR * Q; idx += 64) {
      const int r = idx / Q, q4 = idx - (idx / Q) * Q;
      const int p = (4 * q4) / 32, jj = (4 * q4) % 32;
      if (wcol + 64 * p >= N) continue;
      const int64_t off = om.off(rbase + r);
      if (off < 0) continue;
      const float4 g = *reinterpret_cast<const float4*>(stg + r * LDW + 64 * p + jj);
      const float4 u = *reinterpret_cast<const float4*>(stg + r * LDW + 64 * p + 32 + jj);
      const int col = (wcol + 64 * p) / 2 + jj;
      OT* dst = reinterpret_cast<OT*>(ep.C) + off + col;
      Store4x<OT>::put(dst, silu(g.x) * u.x, silu(g.y) * u.y, silu(g.z) * u.z, silu(g.w) * u.w);
    }
  } else {
    constexpr int Q = WTN / 4;
    for (int idx = lane; idx < SR * Q; idx += 64) {
      const int r = idx / Q, q4 = idx - (idx / Q) * Q;
      const int col = wcol + 4 * q4;
      if (col >= N) continue;
      const int64_t row = rbase + r;
      const int64_t off = om.off(row);
      if (off < 0) continue;
      float4 a = *reinterpret_cast<const float4*>(stg + r * LDW + 4 * q4);
      if constexpr (EPI == EPI_PE) {
        const float4 pe = *reinterpret_cast<const float4*>(ep.pe + (int64_t)ep.tok_pos[row] * pe_ld + col);
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(ep.C) + off + col) =
            make_float4(a.x + pe.x, a.y + pe.y, a.z + pe.z, a.w + pe.w);
      } else {
        if (ep.bias) {
          const float4 b = *reinterpret_cast<const float4*>(ep.bias + col);
          a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w;
        }
        if constexpr (EPI == EPI_RESADD) {
          float4* p = reinterpret_cast<float4*>(reinterpret_cast<float*>(ep.C) + off + col);
          const float4 o = *p;
          *p = make_float4(o.x + a.x, o.y + a.y, o.z + a.z, o.w + a.w);
        } else if constexpr (EPI == EPI_STORE_F32) {
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(ep.C) + off + col) = a;
        } else {
          if constexpr (EPI == EPI_BIAS_GELU) {
            a.x = gelu_erf(a.x); a.y = gelu_erf(a.y); a.z = gelu_erf(a.z); a.w = gelu_erf(a.w);
          }
          Store4x<OT>::put(reinterpret_cast<OT*>(ep.C) + off + col, a.x, a.y, a.z, a.w);
        }
      }
    }
  }
}



// LDS tile rows are BK*2 bytes.  The 16-byte chunk index is XORed with a row hash so that 16
// consecutive rows at one logical chunk cover all 64 banks: for 128-byte rows (BK 64) the row
// parity selects the bank half and (row >> 1) & 7 spreads the 8 chunk slots; for 64-byte rows
// (BK 32) row % 4 selects the bank quarter and (row >> 2) & 3 spreads the 4 slots.
template <int BK>
__device__ __host__ constexpr int swz(int r) { return BK == 64 ? (r >> 1) & 7 : (r >> 2) & 3; }

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* p, int64_t bytes) {
  // raw buffer: stride 0, range check against `bytes`; dword3 0x00020000 (32-bit data format)
  // integer clamp (a 64-bit min lowers to a vector f64 op here, which would drag the whole
  // descriptor into vector registers and wrap every buffer load in a waterfall loop)
  const int n = __builtin_amdgcn_readfirstlane(bytes > 0x7fffffff ? 0x7fffffff : (int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, n, 0x00020000);
}

// TAG only names the call site (one kernel symbol per role, so profiles separate them)
#ifndef AE_GEMM_CPOL
#define AE_GEMM_CPOL 0  // cache policy bits of the tile loads
#endif
#ifndef AE_GEMM_GROUP_M
#define AE_GEMM_GROUP_M 8
#endif
#ifndef AE_GEMM_SCHED
#define AE_GEMM_SCHED 3
#endif

// SCHED bit 0: software-pipeline the K loop across the barrier (the last K-step's MFMAs run
// after the barrier, covering the LDS reads of the next tile's first K-step).  SCHED bit 1:
// order each K-step as [LDS reads of the next K-step][MFMAs of this one] for the scheduler.
template <class TL, class AS, class OM, int EPI, typename OT, int TAG, int SCHED = AE_GEMM_SCHED>
__global__ __launch_bounds__(TL::NT, TL::MINB) void gemm_bf16_kernel(AS as, const bf16_t* __restrict__ Bw,
                                                         int32_t N, int32_t K, OM om, EpiP ep,
                                                         int32_t n_tiles, int32_t pe_ld, int32_t gm) {
  constexpr int BM = TL::BM, BN = TL::BN, TM = TL::TM, TN = TL::TN, AR = TL::AR, BR = TL::BR;
  constexpr int WTN = TL::WTN, BK = TL::BK, CPR = TL::CPR;
  constexpr int SMEM = 2 * (BM + BN) * BK;  // bf16 elements: double-buffered A and B tiles
  // epilogue staging: SR rows of each wave's tile at a time (32, or 16 when 32 do not fit)
  constexpr int SR = (TL::NW * 32 * (WTN + 4) * 4 <= SMEM * 2) ? 32 : 16;
  static_assert(TL::NW * SR * (WTN + 4) * 4 <= SMEM * 2, "epilogue staging must fit in the tiles");
  __shared__ __attribute__((aligned(16))) bf16_t smem[SMEM];
  bf16_t* const sA = smem;                 // [2][BM * BK]
  bf16_t* const sB = smem + 2 * BM * BK;   // [2][BN * BK]

  const int tid = threadIdx.x;
  const int lane = tid & 63, l32 = lane & 31, half = lane >> 5;
  const int wv = tid >> 6;
  const int wm = wv / TL::WGN, wn = wv % TL::WGN;
  // tile order: XCD-contiguous ranges, then groups of `gm` M-tiles swept column by column so the
  // tiles an XCD runs at once share a few A row-panels and B column-panels in its L2
  const TileCoord tc = tile_coord(n_tiles, gm);
  const int64_t mt = tc.mt;
  const int nt = tc.nt;
  const int64_t m0 = mt * BM;
  const int n0 = nt * BN;
  if (!as.tile_live(m0, BM)) return;

  // global -> register loader: 16-byte chunk c of rows lr + 32*i, via buffer loads whose
  // out-of-range offsets return zero (ragged M/N tails, conv padding taps)
  const int c = tid % CPR;
  const int lr = tid / CPR;
  constexpr int RS = TL::RS;
  const __amdgpu_buffer_rsrc_t ra_rsrc = make_rsrc(as.base(), as.bytes());
  const __amdgpu_buffer_rsrc_t rb_rsrc = make_rsrc(Bw, (int64_t)N * K * 2);
  typename AS::BRow arow[AR];
  uint32_t boffr[BR];
#pragma unroll
  for (int i = 0; i < AR; ++i) arow[i] = as.brow(m0 + lr + RS * i);
#pragma unroll
  for (int i = 0; i < BR; ++i) {
    const int n = n0 + lr + RS * i;
    boffr[i] = n < N ? (uint32_t)n * (uint32_t)K * 2u : 0x80000000u;
  }
  constexpr int NSET = TL::NPF > 2 ? TL::NPF : 2;
  u32x4_t ra[NSET][AR], rb[NSET][BR];  // register sets
  auto gload = [&](int kt, int set) {
    const int k = kt * BK + c * 8;
    const auto kc = as.kc(k);
    const bool kok = k < K;
#pragma unroll
    for (int i = 0; i < AR; ++i)
      ra[set][i] = __builtin_amdgcn_raw_buffer_load_b128(ra_rsrc, (int)as.boff(arow[i], kc), 0, AE_GEMM_CPOL);
#pragma unroll
    for (int i = 0; i < BR; ++i) {
      const uint32_t off = (kok && boffr[i] != 0x80000000u) ? boffr[i] + (uint32_t)k * 2u : 0x80000000u;
      rb[set][i] = __builtin_amdgcn_raw_buffer_load_b128(rb_rsrc, (int)off, 0, AE_GEMM_CPOL);
    }
  };
  auto sstore = [&](int buf, int set) {
#pragma unroll
    for (int i = 0; i < AR; ++i) {
      const int r = lr + RS * i;
      *reinterpret_cast<u32x4_t*>(&sA[buf * BM * BK + r * BK + ((c ^ swz<BK>(r)) * 8)]) = ra[set][i];
    }
#pragma unroll
    for (int i = 0; i < BR; ++i) {
      const int r = lr + RS * i;
      *reinterpret_cast<u32x4_t*>(&sB[buf * BN * BK + r * BK + ((c ^ swz<BK>(r)) * 8)]) = rb[set][i];
    }
  };

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // MFMA operand rows of this lane (the swizzle key depends on row % 16 = l32 % 16 only)
  const int arow0 = wm * TL::WTM + l32;
  const int brow0 = wn * TL::WTN + l32;
  const int sw = swz<BK>(l32);
  bf16x8_t af[2][TM], bfr[2][TN];
  auto fload = [&](int buf, int ks, int slot) {
    const bf16_t* pa = sA + buf * BM * BK + arow0 * BK;
    const bf16_t* pb = sB + buf * BN * BK + brow0 * BK;
    const int ch = ((ks * 2 + half) ^ sw) * 8;
#pragma unroll
    for (int i = 0; i < TM; ++i) af[slot][i] = *reinterpret_cast<const bf16x8_t*>(pa + i * 32 * BK + ch);
#pragma unroll
    for (int j = 0; j < TN; ++j) bfr[slot][j] = *reinterpret_cast<const bf16x8_t*>(pb + j * 32 * BK + ch);
  };

  auto mfmas = [&](int slot) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[slot][i], bfr[slot][j], acc[i][j],
                                                            0, 0, 0);
  };
  constexpr int KS = BK / 16;
  const int nk = (K + BK - 1) / BK;
  if constexpr (TL::NPF > 1) {
    // register ring: tile t is loaded into set t % NPF right after that set's previous tile was
    // written to LDS, i.e. NPF tiles of MFMA work before it is needed
    constexpr int NPF = TL::NPF;
#pragma unroll
    for (int p = 0; p < NPF; ++p)
      if (p < nk) gload(p, p);
    sstore(0, 0);
    if (NPF < nk) gload(NPF, 0);
    __syncthreads();
    fload(0, 0, 0);
    auto iter = [&](int kt, auto ph) {
      constexpr int P = decltype(ph)::value;  // kt % NPF
      constexpr int PN = (P + 1) % NPF;       // set of tile kt + 1
      const bool more = kt + 1 < nk;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ks + 1 < KS) {
          fload(kt & 1, ks + 1, (ks + 1) & 1);
        } else if (more) {
          sstore((kt + 1) & 1, PN);
          if (kt + 1 + NPF < nk) gload(kt + 1 + NPF, PN);
          __syncthreads();
          fload((kt + 1) & 1, 0, 0);
        }
        if constexpr (SCHED & 2) {
          __builtin_amdgcn_sched_group_barrier(0x100, TM + TN, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, TM * TN, 0);
        }
        mfmas(ks & 1);
      }
    };
    for (int kt = 0; kt < nk; kt += NPF) {
      iter(kt, std::integral_constant<int, 0>());
      if constexpr (NPF > 1) if (kt + 1 < nk) iter(kt + 1, std::integral_constant<int, 1 % NPF>());
      if constexpr (NPF > 2) if (kt + 2 < nk) iter(kt + 2, std::integral_constant<int, 2 % NPF>());
      if constexpr (NPF > 3) if (kt + 3 < nk) iter(kt + 3, std::integral_constant<int, 3 % NPF>());
    }
    __syncthreads();
  } else if constexpr ((SCHED & 5) == 0) {
    gload(0, 0);
    sstore(0, 0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      if (kt + 1 < nk) gload(kt + 1, 0);
      fload(cur, 0, 0);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ks + 1 < KS) fload(cur, ks + 1, (ks + 1) & 1);
        mfmas(ks & 1);
      }
      if (kt + 1 < nk) sstore(cur ^ 1, 0);
      __syncthreads();
    }
  } else if constexpr ((SCHED & 4) == 0) {
    gload(0, 0);
    sstore(0, 0);
    __syncthreads();
    fload(0, 0, 0);
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      const bool more = kt + 1 < nk;
      if (more) gload(kt + 1, 0);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ks + 1 < KS) {
          fload(cur, ks + 1, (ks + 1) & 1);
        } else if (more) {
          sstore(cur ^ 1, 0);
          __syncthreads();
          fload(cur ^ 1, 0, 0);
        }
        if constexpr (SCHED & 2) {
          __builtin_amdgcn_sched_group_barrier(0x100, TM + TN, 0);  // DS reads (next K-step)
          __builtin_amdgcn_sched_group_barrier(0x008, TM * TN, 0);  // MFMAs (this K-step)
        }
        mfmas(ks & 1);
      }
    }
    __syncthreads();  // the epilogue reuses the tile buffers as staging
  } else {
    // two-deep register prefetch: tile t lives in register set t & 1 from its load (issued two
    // tiles ahead) until its LDS store at the end of tile t - 1
    gload(0, 0);
    sstore(0, 0);
    __syncthreads();
    if (nk > 1) gload(1, 1);
    fload(0, 0, 0);
    auto iter = [&](int kt, auto parity) {
      constexpr int P = decltype(parity)::value;  // kt & 1
      const bool more = kt + 1 < nk;
      if (kt + 2 < nk) gload(kt + 2, P);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ks + 1 < KS) {
          fload(P, ks + 1, (ks + 1) & 1);
        } else if (more) {
          sstore(1 - P, 1 - P);
          __syncthreads();
          fload(1 - P, 0, 0);
        }
        if constexpr (SCHED & 2) {
          __builtin_amdgcn_sched_group_barrier(0x100, TM + TN, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, TM * TN, 0);
        }
        mfmas(ks & 1);
      }
    };
    for (int kt = 0; kt < nk; kt += 2) {
      iter(kt, std::integral_constant<int, 0>());
      if (kt + 1 < nk) iter(kt + 1, std::integral_constant<int, 1>());
    }
    __syncthreads();
  }

  // epilogue through LDS: each wave writes SR rows of its accumulators row-major, then reads
  // them back four columns per lane for 16-byte (fp32) / 8-byte (bf16) stores
  constexpr int LDW = WTN + 4;
  float* stg = reinterpret_cast<float*>(smem) + wv * SR * LDW;
  const int wcol = n0 + wn * TL::WTN;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
  for (int hs = 0; hs < 32 / SR; ++hs) {
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = 8 * (v >> 2) + 4 * half + (v & 3) - hs * SR;
        if (r >= 0 && r < SR) stg[r * LDW + 32 * j + l32] = acc[i][j][v];
      }
    __syncthreads();
    const int64_t rbase = m0 + wm * TL::WTM + i * 32 + hs * SR;
    epilogue_rows<EPI, OT, WTN, SR>(stg, LDW, rbase, wcol, N, om, ep, pe_ld, lane);
    __syncthreads();
  }
  }
}

// Direct-to-LDS variant: the tile loads are buffer_load_dwordx4 ... lds (gfx950 LDS DMA, 16
// bytes per lane), so tile data never passes through VGPRs.  One LDS DMA instruction fills
// 1 KB of LDS at (wave-uniform base + 16 * lane); each lane therefore fetches the global chunk
// whose swizzled LDS slot is base + 16 * lane.  Per K tile:
//   wait for this tile's DMA, barrier -> read all MFMA fragments of the tile into registers ->
//   issue the DMA of the next tile into the other buffer -> MFMAs.
// The DMA of tile kt+1 thus overlaps the MFMAs of tile kt, and the compiler's conservative
// wait before LDS reads never falls between a DMA and the fragment reads it could delay.
template <class TL, class AS, class OM, int EPI, typename OT, int TAG>
__global__ __launch_bounds__(TL::NT, TL::MINB) void gemm_dtl_kernel(AS as, const bf16_t* __restrict__ Bw,
                                                                   int32_t N, int32_t K, OM om, EpiP ep,
                                                                   int32_t n_tiles, int32_t pe_ld, int32_t gm) {
  constexpr int BM = TL::BM, BN = TL::BN, TM = TL::TM, TN = TL::TN;
  constexpr int WTN = TL::WTN, BK = TL::BK, NW = TL::NW;
  constexpr int SMEM = 2 * (BM + BN) * BK;
  constexpr int SR = (NW * 32 * (WTN + 4) * 4 <= SMEM * 2) ? 32 : 16;
  static_assert(NW * SR * (WTN + 4) * 4 <= SMEM * 2, "epilogue staging must fit in the tiles");
  constexpr int ROWS_PER_DMA = 1024 / (BK * 2);           // tile rows filled by one instruction
  constexpr int ADMA = BM / ROWS_PER_DMA / NW;            // DMA instructions per wave per tile
  constexpr int BDMA = BN / ROWS_PER_DMA / NW;
  static_assert(ADMA * ROWS_PER_DMA * NW == BM && BDMA * ROWS_PER_DMA * NW == BN, "dma split");
  constexpr int KS = BK / 16;
  __shared__ __attribute__((aligned(1024))) bf16_t smem[SMEM];
  bf16_t* const sA = smem;
  bf16_t* const sB = smem + 2 * BM * BK;

  const int tid = threadIdx.x;
  const int lane = tid & 63, l32 = lane & 31, half = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv / TL::WGN, wn = wv % TL::WGN;
  const TileCoord tc = tile_coord(n_tiles, gm);
  const int64_t mt = tc.mt;
  const int nt = tc.nt;
  const int64_t m0 = mt * BM;
  const int n0 = nt * BN;
  if (!as.tile_live(m0, BM)) return;

  // lane -> (tile row, logical chunk) of each DMA instruction of this wave
  const __amdgpu_buffer_rsrc_t ra_rsrc = make_rsrc(as.base(), as.bytes());
  const __amdgpu_buffer_rsrc_t rb_rsrc = make_rsrc(Bw, (int64_t)N * K * 2);
  constexpr int CPR = BK / 8;
  typename AS::BRow arow[ADMA];
  int achunk[ADMA];
  uint32_t boffr[BDMA];
  int bchunk[BDMA];
#pragma unroll
  for (int j = 0; j < ADMA; ++j) {
    const int r = (wv * ADMA + j) * ROWS_PER_DMA + lane / CPR;
    achunk[j] = (lane % CPR) ^ swz<BK>(r);
    arow[j] = as.brow(m0 + r);
  }
#pragma unroll
  for (int j = 0; j < BDMA; ++j) {
    const int r = (wv * BDMA + j) * ROWS_PER_DMA + lane / CPR;
    bchunk[j] = (lane % CPR) ^ swz<BK>(r);
    const int n = n0 + r;
    boffr[j] = n < N ? (uint32_t)n * (uint32_t)K * 2u : 0x80000000u;
  }
  auto dma = [&](int kt, int buf) {
#pragma unroll
    for (int j = 0; j < ADMA; ++j) {
      const int k = kt * BK + achunk[j] * 8;
      const uint32_t off = as.boff(arow[j], as.kc(k));
      bf16_t* dst = sA + buf * BM * BK + (wv * ADMA + j) * ROWS_PER_DMA * BK;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra_rsrc, (__attribute__((address_space(3))) void*)dst, 16,
                                               (int)off, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < BDMA; ++j) {
      const int k = kt * BK + bchunk[j] * 8;
      const uint32_t off = (k < K && boffr[j] != 0x80000000u) ? boffr[j] + (uint32_t)k * 2u : 0x80000000u;
      bf16_t* dst = sB + buf * BN * BK + (wv * BDMA + j) * ROWS_PER_DMA * BK;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb_rsrc, (__attribute__((address_space(3))) void*)dst, 16,
                                               (int)off, 0, 0, 0);
    }
  };

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int arow0 = wm * TL::WTM + l32;
  const int brow0 = wn * TL::WTN + l32;
  const int sw = swz<BK>(l32);
  bf16x8_t af[KS][TM], bfr[KS][TN];
  const int nk = (K + BK - 1) / BK;
  dma(0, 0);
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wave's DMA of tile kt has landed
    __syncthreads();                     // every wave's DMA landed; buffer cur^1 is free
    const bf16_t* pa = sA + cur * BM * BK + arow0 * BK;
    const bf16_t* pb = sB + cur * BN * BK + brow0 * BK;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int ch = ((ks * 2 + half) ^ sw) * 8;
#pragma unroll
      for (int i = 0; i < TM; ++i) af[ks][i] = *reinterpret_cast<const bf16x8_t*>(pa + i * 32 * BK + ch);
#pragma unroll
      for (int j = 0; j < TN; ++j) bfr[ks][j] = *reinterpret_cast<const bf16x8_t*>(pb + j * 32 * BK + ch);
    }
    if (kt + 1 < nk) dma(kt + 1, cur ^ 1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks][i], bfr[ks][j], acc[i][j], 0, 0, 0);
  }
  __syncthreads();

  constexpr int LDW = WTN + 4;
  float* stg = reinterpret_cast<float*>(smem) + wv * SR * LDW;
  const int wcol = n0 + wn * TL::WTN;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
  for (int hs = 0; hs < 32 / SR; ++hs) {
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = 8 * (v >> 2) + 4 * half + (v & 3) - hs * SR;
        if (r >= 0 && r < SR) stg[r * LDW + 32 * j + l32] = acc[i][j][v];
      }
    __syncthreads();
    const int64_t rbase = m0 + wm * TL::WTM + i * 32 + hs * SR;
    epilogue_rows<EPI, OT, WTN, SR>(stg, LDW, rbase, wcol, N, om, ep, pe_ld, lane);
    __syncthreads();
  }
  }
}

// Compiler-only barrier: no LDS access moves across it, and unlike __syncthreads() it adds
// no release fence (which would wait for every LDS DMA in flight, deeper stages included).
__device__ inline void cbar() { asm volatile("" ::: "memory"); }

// s_waitcnt vmcnt(VM) lgkmcnt(0) (gfx9 encoding: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8],
// vmcnt[5:4] in bits 15:14)
template <int VM>
__device__ inline void wait_vm_lds0() {
  static_assert(VM >= 0 && VM < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4));
}

// Direct-to-LDS kernel with an NST-stage ring (tile kt+NST-1 is in flight while tile kt is
// multiplied).  Each stage is its own __shared__ array: the compiler then knows which DMA a
// fragment read can depend on, waits for that one only, and is free to interleave the reads of
// one K step with the MFMAs of the previous one.  Per K tile:
//   wait until this wave's DMA of tile kt has landed and its LDS reads of the stage about to
//   be refilled are done; barrier (all waves) -> DMA of tile kt+NST-1 into the stage read at
//   kt-1 -> fragment reads and MFMAs of tile kt.
template <class TL, int NST, class AS, class OM, int EPI, typename OT, int TAG>
__global__ __launch_bounds__(TL::NT, TL::MINB) void gemm_pipe_kernel(AS as, const bf16_t* __restrict__ Bw,
                                                                    int32_t N, int32_t K, OM om, EpiP ep,
                                                                    int32_t n_tiles, int32_t pe_ld, int32_t gm) {
  static_assert(NST >= 2 && NST <= 4, "stages");
  constexpr int BM = TL::BM, BN = TL::BN, TM = TL::TM, TN = TL::TN;
  constexpr int WTN = TL::WTN, BK = TL::BK, NW = TL::NW;
  constexpr int STG = (BM + BN) * BK;  // bf16 elements per stage: A tile, then B tile
  constexpr int SR = (NW * 32 * (WTN + 4) * 4 <= STG * 2) ? 32
                     : (NW * 16 * (WTN + 4) * 4 <= STG * 2) ? 16 : 8;
  static_assert(NW * SR * (WTN + 4) * 4 <= STG * 2, "epilogue staging must fit in one stage");
  constexpr int ROWS_PER_DMA = 1024 / (BK * 2);
  constexpr int ADMA = BM / ROWS_PER_DMA / NW;
  constexpr int BDMA = BN / ROWS_PER_DMA / NW;
  constexpr int P = ADMA + BDMA;  // DMA instructions per wave per K tile
  static_assert(ADMA * ROWS_PER_DMA * NW == BM && BDMA * ROWS_PER_DMA * NW == BN, "dma split");
  static_assert(P * (NST - 2) < 64, "vmcnt range");
  constexpr int KS = BK / 16;
  __shared__ __attribute__((aligned(1024))) bf16_t st0[STG];
  __shared__ __attribute__((aligned(1024))) bf16_t st1[STG];
  __shared__ __attribute__((aligned(1024))) bf16_t st2[NST > 2 ? STG : 8];
  __shared__ __attribute__((aligned(1024))) bf16_t st3[NST > 3 ? STG : 8];
  auto stage = [&](auto sc) -> bf16_t* {
    constexpr int s = decltype(sc)::value;
    if constexpr (s == 0) return st0;
    else if constexpr (s == 1) return st1;
    else if constexpr (s == 2) return st2;
    else return st3;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63, l32 = lane & 31, half = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv / TL::WGN, wn = wv % TL::WGN;
  const TileCoord tc = tile_coord(n_tiles, gm);
  const int64_t mt = tc.mt;
  const int nt = tc.nt;
  const int64_t m0 = mt * BM;
  const int n0 = nt * BN;
  if (!as.tile_live(m0, BM)) return;

  const __amdgpu_buffer_rsrc_t ra_rsrc = make_rsrc(as.base(), as.bytes());
  const __amdgpu_buffer_rsrc_t rb_rsrc = make_rsrc(Bw, (int64_t)N * K * 2);
  constexpr int CPR = BK / 8;
  typename AS::BRow arow[ADMA];
  int achunk[ADMA];
  uint32_t boffr[BDMA];
  int bchunk[BDMA];
#pragma unroll
  for (int j = 0; j < ADMA; ++j) {
    const int r = (wv * ADMA + j) * ROWS_PER_DMA + lane / CPR;
    achunk[j] = (lane % CPR) ^ swz<BK>(r);
    arow[j] = as.brow(m0 + r);
  }
#pragma unroll
  for (int j = 0; j < BDMA; ++j) {
    const int r = (wv * BDMA + j) * ROWS_PER_DMA + lane / CPR;
    bchunk[j] = (lane % CPR) ^ swz<BK>(r);
    const int n = n0 + r;
    boffr[j] = n < N ? (uint32_t)n * (uint32_t)K * 2u : 0x80000000u;
  }
  auto dma = [&](int kt, bf16_t* st) {
#pragma unroll
    for (int j = 0; j < ADMA; ++j) {
      const int k = kt * BK + achunk[j] * 8;
      const uint32_t off = as.boff(arow[j], as.kc(k));
      bf16_t* dst = st + (wv * ADMA + j) * ROWS_PER_DMA * BK;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra_rsrc, (__attribute__((address_space(3))) void*)dst, 16,
                                               (int)off, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < BDMA; ++j) {
      const int k = kt * BK + bchunk[j] * 8;
      const uint32_t off = (k < K && boffr[j] != 0x80000000u) ? boffr[j] + (uint32_t)k * 2u : 0x80000000u;
      bf16_t* dst = st + BM * BK + (wv * BDMA + j) * ROWS_PER_DMA * BK;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb_rsrc, (__attribute__((address_space(3))) void*)dst, 16,
                                               (int)off, 0, 0, 0);
    }
  };

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int arow0 = wm * TL::WTM + l32;
  const int brow0 = wn * TL::WTN + l32;
  const int sw = swz<BK>(l32);
  auto compute = [&](const bf16_t* st) {
    const bf16_t* pa = st + arow0 * BK;
    const bf16_t* pb = st + BM * BK + brow0 * BK;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int ch = ((ks * 2 + half) ^ sw) * 8;
      bf16x8_t af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) af[i] = *reinterpret_cast<const bf16x8_t*>(pa + i * 32 * BK + ch);
#pragma unroll
      for (int j = 0; j < TN; ++j) bfr[j] = *reinterpret_cast<const bf16x8_t*>(pb + j * 32 * BK + ch);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  };

  const int nk = (K + BK - 1) / BK;
  dma(0, st0);
  if constexpr (NST > 2) if (1 < nk) dma(1, st1);
  if constexpr (NST > 3) if (2 < nk) dma(2, st2);
  auto iter = [&](int kt, auto sc) {
    constexpr int s = decltype(sc)::value;
    const int after = min(NST - 2, nk - 1 - kt);  // tiles issued after tile kt
    if constexpr (NST > 3) {
      if (after >= 2) wait_vm_lds0<2 * P>();
      else if (after == 1) wait_vm_lds0<P>();
      else wait_vm_lds0<0>();
    } else if constexpr (NST > 2) {
      if (after >= 1) wait_vm_lds0<P>();
      else wait_vm_lds0<0>();
    } else {
      wait_vm_lds0<0>();
    }
    cbar();
    __builtin_amdgcn_s_barrier();
    cbar();
    if (kt + NST - 1 < nk) dma(kt + NST - 1, stage(std::integral_constant<int, (s + NST - 1) % NST>()));
    compute(stage(std::integral_constant<int, s>()));
  };
  for (int kt = 0; kt < nk; kt += NST) {
    iter(kt, std::integral_constant<int, 0>());
    if (kt + 1 < nk) iter(kt + 1, std::integral_constant<int, 1>());
    if constexpr (NST > 2) if (kt + 2 < nk) iter(kt + 2, std::integral_constant<int, 2>());
    if constexpr (NST > 3) if (kt + 3 < nk) iter(kt + 3, std::integral_constant<int, 3>());
  }
  wait_vm_lds0<0>();
  __syncthreads();

  constexpr int LDW = WTN + 4;
  float* stg = reinterpret_cast<float*>(st0) + wv * SR * LDW;
  const int wcol = n0 + wn * TL::WTN;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
  for (int hs = 0; hs < 32 / SR; ++hs) {
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = 8 * (v >> 2) + 4 * half + (v & 3) - hs * SR;
        if (r >= 0 && r < SR) stg[r * LDW + 32 * j + l32] = acc[i][j][v];
      }
    __syncthreads();
    const int64_t rbase = m0 + wm * TL::WTM + i * 32 + hs * SR;
    epilogue_rows<EPI, OT, WTN, SR>(stg, LDW, rbase, wcol, N, om, ep, pe_ld, lane);
    __syncthreads();
  }
  }
}

// Epilogue straight from the accumulators of a wave (no LDS staging, no barriers).  The MFMAs
// compute the transposed product (B fragment as the first operand), so lane l of a 32x32 block
// holds output row l % 32 and, for register group g = v / 4, the four consecutive columns
// 8 g + 4 (l / 32) .. +3: every lane stores 4-wide runs of its own row.
template <int EPI, typename OT, int TM, int TN, class OM>
__device__ __attribute__((always_inline)) inline void epilogue_direct(const f32x16_t (&acc)[TM][TN], int64_t mrow0, int ncol0,
                                       int N, const OM& om, const EpiP& ep, int pe_ld, int lane) {
  const int l32 = lane & 31, half = lane >> 5;
  const bool vec = (N & 3) == 0;  // 4-wide runs are aligned and never straddle the end
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int64_t row = mrow0 + i * 32 + l32;
    const int64_t off = om.off(row);
    if (off < 0) continue;
    if constexpr (EPI == EPI_SWIGLU) {
      // gate and up columns alternate in blocks of 32 (N % 64 == 0): block pairs (j, j+1)
#pragma unroll
      for (int j = 0; j + 1 < TN; j += 2) {
        if (ncol0 + j * 32 >= N) continue;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int col = (ncol0 + j * 32) / 2 + 8 * g + 4 * half;
          float o[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = silu(acc[i][j][4 * g + e]) * acc[i][j + 1][4 * g + e];
          Store4x<OT>::put(reinterpret_cast<OT*>(ep.C) + off + col, o[0], o[1], o[2], o[3]);
        }
      }
    } else {
      const float* perow = nullptr;
      if constexpr (EPI == EPI_PE) perow = ep.pe + (int64_t)ep.tok_pos[row] * pe_ld;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int col = ncol0 + j * 32 + 8 * g + 4 * half;
          if (col >= N) continue;
          float o[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = acc[i][j][4 * g + e];
          if (vec) {
            if constexpr (EPI == EPI_PE) {
              const float4 pe = *reinterpret_cast<const float4*>(perow + col);
              o[0] += pe.x; o[1] += pe.y; o[2] += pe.z; o[3] += pe.w;
            } else if (ep.bias) {
              const float4 b = *reinterpret_cast<const float4*>(ep.bias + col);
              o[0] += b.x; o[1] += b.y; o[2] += b.z; o[3] += b.w;
            }
            if constexpr (EPI == EPI_RESADD) {
              float4* p = reinterpret_cast<float4*>(reinterpret_cast<float*>(ep.C) + off + col);
              const float4 c = *p;
              *p = make_float4(c.x + o[0], c.y + o[1], c.z + o[2], c.w + o[3]);
            } else if constexpr (EPI == EPI_STORE_F32 || EPI == EPI_PE) {
              *reinterpret_cast<float4*>(reinterpret_cast<float*>(ep.C) + off + col) =
                  make_float4(o[0], o[1], o[2], o[3]);
            } else {
              if constexpr (EPI == EPI_BIAS_GELU) {
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = gelu_erf(o[e]);
              }
              Store4x<OT>::put(reinterpret_cast<OT*>(ep.C) + off + col, o[0], o[1], o[2], o[3]);
            }
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              if (col + e >= N) break;
              if constexpr (EPI == EPI_PE) {
                reinterpret_cast<float*>(ep.C)[off + col + e] = o[e] + perow[col + e];
              } else {
                epi_store<EPI, OT>(ep, off, row, col + e, o[e]);
              }
            }
          }
        }
      }
    }
  }
}

template <int P, int NMAX>
__device__ inline void wait_tiles(int n) {  // vmcnt(P * n) lgkmcnt(0), n in [0, NMAX]
  if constexpr (NMAX >= 3) if (n >= 3) { wait_vm_lds0<3 * P>(); return; }
  if constexpr (NMAX >= 2) if (n >= 2) { wait_vm_lds0<2 * P>(); return; }
  if constexpr (NMAX >= 1) if (n >= 1) { wait_vm_lds0<P>(); return; }
  wait_vm_lds0<0>();
}

// As gemm_pipe_kernel, with the MFMA fragments double-buffered in registers: the fragment
// reads of K step ks+1 are issued before the MFMAs of step ks, and the barrier that publishes
// tile kt+1 sits before the MFMAs of the last step of tile kt, so the matrix pipe is fed across
// tile boundaries even with one wave per SIMD.
//   prologue: DMA tiles 0..NST-1, wait for tile 0, barrier, read step 0.
//   tile kt, step ks < KS-1: read step ks+1; MFMAs of step ks.
//   tile kt, last step: wait for tile kt+1 (and for this wave's reads), barrier, DMA of tile
//   kt+NST into the stage just drained, read step 0 of tile kt+1; MFMAs of the last step.
template <class TL, int NST, class AS, class OM, int EPI, typename OT, int TAG, bool DIRECT = true>
__global__ __launch_bounds__(TL::NT, TL::MINB) void gemm_pipe2_kernel(AS as, const bf16_t* __restrict__ Bw,
                                                                     int32_t N, int32_t K, OM om, EpiP ep,
                                                                     int32_t n_tiles, int32_t pe_ld, int32_t gm) {
  static_assert(NST >= 2 && NST <= 4, "stages");
  constexpr int BM = TL::BM, BN = TL::BN, TM = TL::TM, TN = TL::TN;
  constexpr int WTN = TL::WTN, BK = TL::BK, NW = TL::NW;
  constexpr int STG = (BM + BN) * BK;
  constexpr int SR = (NW * 32 * (WTN + 4) * 4 <= STG * 2) ? 32
                     : (NW * 16 * (WTN + 4) * 4 <= STG * 2) ? 16 : 8;
  static_assert(NW * SR * (WTN + 4) * 4 <= STG * 2, "epilogue staging must fit in one stage");
  constexpr int ROWS_PER_DMA = 1024 / (BK * 2);
  constexpr int ADMA = BM / ROWS_PER_DMA / NW;
  constexpr int BDMA = BN / ROWS_PER_DMA / NW;
  constexpr int P = ADMA + BDMA;
  static_assert(ADMA * ROWS_PER_DMA * NW == BM && BDMA * ROWS_PER_DMA * NW == BN, "dma split");
  static_assert(P * (NST - 1) < 64, "vmcnt range");
  constexpr int KS = BK / 16;
  static_assert(KS % 2 == 0, "fragment buffers alternate by step parity");
  __shared__ __attribute__((aligned(1024))) bf16_t st0[STG];
  __shared__ __attribute__((aligned(1024))) bf16_t st1[STG];
  __shared__ __attribute__((aligned(1024))) bf16_t st2[NST > 2 ? STG : 8];
  __shared__ __attribute__((aligned(1024))) bf16_t st3[NST > 3 ? STG : 8];
  auto stage = [&](auto sc) -> bf16_t* {
    constexpr int s = decltype(sc)::value;
    if constexpr (s == 0) return st0;
    else if constexpr (s == 1) return st1;
    else if constexpr (s == 2) return st2;
    else return st3;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63, l32 = lane & 31, half = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv / TL::WGN, wn = wv % TL::WGN;
  const TileCoord tc = tile_coord(n_tiles, gm);
  const int64_t m0 = (int64_t)tc.mt * BM;
  const int n0 = tc.nt * BN;
  if (!as.tile_live(m0, BM)) return;

  const __amdgpu_buffer_rsrc_t ra_rsrc = make_rsrc(as.base(), as.bytes());
  const __amdgpu_buffer_rsrc_t rb_rsrc = make_rsrc(Bw, (int64_t)N * K * 2);
  constexpr int CPR = BK / 8;
  typename AS::BRow arow[ADMA];
  int achunk[ADMA];
  uint32_t boffr[BDMA];
  int bchunk[BDMA];
#pragma unroll
  for (int j = 0; j < ADMA; ++j) {
    const int r = (wv * ADMA + j) * ROWS_PER_DMA + lane / CPR;
    achunk[j] = (lane % CPR) ^ swz<BK>(r);
    arow[j] = as.brow(m0 + r);
  }
#pragma unroll
  for (int j = 0; j < BDMA; ++j) {
    const int r = (wv * BDMA + j) * ROWS_PER_DMA + lane / CPR;
    bchunk[j] = (lane % CPR) ^ swz<BK>(r);
    const int n = n0 + r;
    boffr[j] = n < N ? (uint32_t)n * (uint32_t)K * 2u : 0x80000000u;
  }
  auto dma = [&](int kt, bf16_t* st) {
#pragma unroll
    for (int j = 0; j < ADMA; ++j) {
      const int k = kt * BK + achunk[j] * 8;
      const uint32_t off = as.boff(arow[j], as.kc(k));
      bf16_t* dst = st + (wv * ADMA + j) * ROWS_PER_DMA * BK;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra_rsrc, (__attribute__((address_space(3))) void*)dst, 16,
                                               (int)off, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < BDMA; ++j) {
      const int k = kt * BK + bchunk[j] * 8;
      const uint32_t off = (k < K && boffr[j] != 0x80000000u) ? boffr[j] + (uint32_t)k * 2u : 0x80000000u;
      bf16_t* dst = st + BM * BK + (wv * BDMA + j) * ROWS_PER_DMA * BK;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb_rsrc, (__attribute__((address_space(3))) void*)dst, 16,
                                               (int)off, 0, 0, 0);
    }
  };

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int aoff = (wm * TL::WTM + l32) * BK;
  const int boff = BM * BK + (wn * TL::WTN + l32) * BK;
  const int sw = swz<BK>(l32);
  bf16x8_t fa[2][TM], fb[2][TN];
  auto rd = [&](const bf16_t* st, int ks, int buf) {
    const int ch = ((ks * 2 + half) ^ sw) * 8;
#pragma unroll
    for (int i = 0; i < TM; ++i) fa[buf][i] = *reinterpret_cast<const bf16x8_t*>(st + aoff + i * 32 * BK + ch);
#pragma unroll
    for (int j = 0; j < TN; ++j) fb[buf][j] = *reinterpret_cast<const bf16x8_t*>(st + boff + j * 32 * BK + ch);
  };
  auto mm = [&](int buf) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        if constexpr (DIRECT)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[buf][j], fa[buf][i], acc[i][j], 0, 0, 0);
        else
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[buf][i], fb[buf][j], acc[i][j], 0, 0, 0);
  };
  auto barrier = [&]() {
    cbar();
    __builtin_amdgcn_s_barrier();
    cbar();
  };

  // The K loop runs over a multiple of NST tiles, and tiles past the end of K are issued like
  // any other: every offset is out of range, so they only write zeros into stages whose
  // products add nothing.  The loop body is then free of branches and each wave always has the
  // same number of DMAs in flight, so every wait below is a constant (the compiler's wait-count
  // tracking merges the states of branches conservatively and would otherwise stall MFMAs on
  // fragment reads they do not use).
  const int nk = (K + BK * NST - 1) / (BK * NST) * NST;
  dma(0, st0);
  dma(1, st1);
  if constexpr (NST > 2) dma(2, st2);
  if constexpr (NST > 3) dma(3, st3);
  wait_vm_lds0<P * (NST - 1)>();
  barrier();
  rd(st0, 0, 0);

  auto tile_step = [&](int kt, auto sc) {
    constexpr int s = decltype(sc)::value;
    const bf16_t* cur = stage(sc);
#pragma unroll
    for (int ks = 0; ks + 1 < KS; ++ks) {
      rd(cur, ks + 1, (ks + 1) & 1);
      __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the MFMAs they overlap
      mm(ks & 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    wait_vm_lds0<P * (NST - 2)>();
    barrier();
    dma(kt + NST, stage(sc));
    rd(stage(std::integral_constant<int, (s + 1) % NST>()), 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    mm((KS - 1) & 1);
    __builtin_amdgcn_sched_barrier(0);
  };
  for (int kt = 0; kt < nk; kt += NST) {
    tile_step(kt, std::integral_constant<int, 0>());
    tile_step(kt + 1, std::integral_constant<int, 1>());
    if constexpr (NST > 2) tile_step(kt + 2, std::integral_constant<int, 2>());
    if constexpr (NST > 3) tile_step(kt + 3, std::integral_constant<int, 3>());
  }
  if constexpr (DIRECT) {
    epilogue_direct<EPI, OT, TM, TN>(acc, m0 + wm * TL::WTM, n0 + wn * TL::WTN, N, om, ep, pe_ld, lane);
    wait_vm_lds0<0>();  // the trailing out-of-range DMAs land before the LDS is released
    return;
  }
  wait_vm_lds0<0>();
  __syncthreads();

  constexpr int LDW = WTN + 4;
  float* stg = reinterpret_cast<float*>(st0) + wv * SR * LDW;
  const int wcol = n0 + wn * TL::WTN;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
  for (int hs = 0; hs < 32 / SR; ++hs) {
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = 8 * (v >> 2) + 4 * half + (v & 3) - hs * SR;
        if (r >= 0 && r < SR) stg[r * LDW + 32 * j + l32] = acc[i][j][v];
      }
    __syncthreads();
    const int64_t rbase = m0 + wm * TL::WTM + i * 32 + hs * SR;
    epilogue_rows<EPI, OT, WTN, SR>(stg, LDW, rbase, wcol, N, om, ep, pe_ld, lane);
    __syncthreads();
  }
  }
}

// NST-stage direct-to-LDS kernel with the refill DMAs spread over the MFMAs.  One barrier per K
// step, at its start: it publishes tile kt and frees the stage read in step kt-1, which is then
// refilled with tile kt+NST-1 in KS slices, one slice issued between the MFMAs of each K
// sub-step (issuing a whole tile's DMAs at once backs up the load queue and stalls the issuing
// waves, MFMAs included).  Fragment reads of sub-step ks+1 are issued before the MFMAs of ks.
template <class TL, int NST, class AS, class OM, int EPI, typename OT, int TAG, bool DIRECT = false>
__global__ __launch_bounds__(TL::NT, TL::MINB) void gemm_ilv_kernel(AS as, const bf16_t* __restrict__ Bw,
                                                                   int32_t N, int32_t K, OM om, EpiP ep,
                                                                   int32_t n_tiles, int32_t pe_ld, int32_t gm) {
  static_assert(NST >= 3 && NST <= 4, "stages: the last refill slice needs a step of slack");
  constexpr int BM = TL::BM, BN = TL::BN, TM = TL::TM, TN = TL::TN;
  constexpr int WTN = TL::WTN, BK = TL::BK, NW = TL::NW;
  constexpr int STG = (BM + BN) * BK;
  constexpr int SR = (NW * 32 * (WTN + 4) * 4 <= STG * 2) ? 32
                     : (NW * 16 * (WTN + 4) * 4 <= STG * 2) ? 16 : 8;
  static_assert(NW * SR * (WTN + 4) * 4 <= STG * 2, "epilogue staging must fit in one stage");
  constexpr int ROWS_PER_DMA = 1024 / (BK * 2);
  constexpr int ADMA = BM / ROWS_PER_DMA / NW;
  constexpr int BDMA = BN / ROWS_PER_DMA / NW;
  constexpr int P = ADMA + BDMA;
  static_assert(ADMA * ROWS_PER_DMA * NW == BM && BDMA * ROWS_PER_DMA * NW == BN, "dma split");
  static_assert(P * (NST - 1) < 64, "vmcnt range");
  constexpr int KS = BK / 16;
  __shared__ __attribute__((aligned(1024))) bf16_t st0[STG];
  __shared__ __attribute__((aligned(1024))) bf16_t st1[STG];
  __shared__ __attribute__((aligned(1024))) bf16_t st2[STG];
  __shared__ __attribute__((aligned(1024))) bf16_t st3[NST > 3 ? STG : 8];
  auto stage = [&](auto sc) -> bf16_t* {
    constexpr int s = decltype(sc)::value;
    if constexpr (s == 0) return st0;
    else if constexpr (s == 1) return st1;
    else if constexpr (s == 2) return st2;
    else return st3;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63, l32 = lane & 31, half = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv / TL::WGN, wn = wv % TL::WGN;
  const TileCoord tc = tile_coord(n_tiles, gm);
  const int64_t m0 = (int64_t)tc.mt * BM;
  const int n0 = tc.nt * BN;
  if (!as.tile_live(m0, BM)) return;

  const __amdgpu_buffer_rsrc_t ra_rsrc = make_rsrc(as.base(), as.bytes());
  const __amdgpu_buffer_rsrc_t rb_rsrc = make_rsrc(Bw, (int64_t)N * K * 2);
  constexpr int CPR = BK / 8;
  typename AS::BRow arow[ADMA];
  int achunk[ADMA];
  uint32_t boffr[BDMA];
  int bchunk[BDMA];
#pragma unroll
  for (int j = 0; j < ADMA; ++j) {
    const int r = (wv * ADMA + j) * ROWS_PER_DMA + lane / CPR;
    achunk[j] = (lane % CPR) ^ swz<BK>(r);
    arow[j] = as.brow(m0 + r);
  }
#pragma unroll
  for (int j = 0; j < BDMA; ++j) {
    const int r = (wv * BDMA + j) * ROWS_PER_DMA + lane / CPR;
    bchunk[j] = (lane % CPR) ^ swz<BK>(r);
    const int n = n0 + r;
    boffr[j] = n < N ? (uint32_t)n * (uint32_t)K * 2u : 0x80000000u;
  }
  // DMA instructions [lo, hi) of tile kt (A rows first, then B rows)
  auto dma_part = [&](int kt, bf16_t* st, int lo, int hi) {
#pragma unroll
    for (int j = 0; j < ADMA; ++j) {
      if (j < lo || j >= hi) continue;
      const int k = kt * BK + achunk[j] * 8;
      const uint32_t off = as.boff(arow[j], as.kc(k));
      bf16_t* dst = st + (wv * ADMA + j) * ROWS_PER_DMA * BK;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra_rsrc, (__attribute__((address_space(3))) void*)dst, 16,
                                               (int)off, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < BDMA; ++j) {
      if (ADMA + j < lo || ADMA + j >= hi) continue;
      const int k = kt * BK + bchunk[j] * 8;
      const uint32_t off = (k < K && boffr[j] != 0x80000000u) ? boffr[j] + (uint32_t)k * 2u : 0x80000000u;
      bf16_t* dst = st + BM * BK + (wv * BDMA + j) * ROWS_PER_DMA * BK;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb_rsrc, (__attribute__((address_space(3))) void*)dst, 16,
                                               (int)off, 0, 0, 0);
    }
  };

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int aoff = (wm * TL::WTM + l32) * BK;
  const int boff = BM * BK + (wn * TL::WTN + l32) * BK;
  const int sw = swz<BK>(l32);
  bf16x8_t fa[2][TM], fb[2][TN];
  auto rd = [&](const bf16_t* st, int ks, int buf) {
    const int ch = ((ks * 2 + half) ^ sw) * 8;
#pragma unroll
    for (int i = 0; i < TM; ++i) fa[buf][i] = *reinterpret_cast<const bf16x8_t*>(st + aoff + i * 32 * BK + ch);
#pragma unroll
    for (int j = 0; j < TN; ++j) fb[buf][j] = *reinterpret_cast<const bf16x8_t*>(st + boff + j * 32 * BK + ch);
  };
  auto mm = [&](int buf) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        if constexpr (DIRECT)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[buf][j], fa[buf][i], acc[i][j], 0, 0, 0);
        else
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[buf][i], fb[buf][j], acc[i][j], 0, 0, 0);
      }
  };
  auto barrier = [&]() {
    cbar();
    __builtin_amdgcn_s_barrier();
    cbar();
  };

  // As in gemm_pipe2_kernel: a multiple of NST steps, with out-of-range tiles past the end of K
  // (zero fill), so every wait is a constant.
  const int nk = (K + BK * NST - 1) / (BK * NST) * NST;
  dma_part(0, st0, 0, P);
  dma_part(1, st1, 0, P);
  if constexpr (NST > 3) dma_part(2, st2, 0, P);

  auto step = [&](int kt, auto sc) {
    constexpr int s = decltype(sc)::value;
    constexpr int sf = (s + NST - 1) % NST;  // stage freed by this step's barrier
    wait_vm_lds0<P * (NST - 2)>();           // tile kt landed; tiles kt+1 .. kt+NST-2 in flight
    barrier();
    const bf16_t* cur = stage(sc);
    bf16_t* nxt = stage(std::integral_constant<int, sf>());
    rd(cur, 0, 0);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + 1 < KS) rd(cur, ks + 1, (ks + 1) & 1);
      __builtin_amdgcn_sched_barrier(0);
      dma_part(kt + NST - 1, nxt, ks * P / KS, (ks + 1) * P / KS);
      mm(ks & 1);
      // alternate refill DMAs and MFMAs
#pragma unroll
      for (int d = ks * P / KS; d < (ks + 1) * P / KS; ++d) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  for (int kt = 0; kt < nk; kt += NST) {
    step(kt, std::integral_constant<int, 0>());
    step(kt + 1, std::integral_constant<int, 1>());
    step(kt + 2, std::integral_constant<int, 2>());
    if constexpr (NST > 3) step(kt + 3, std::integral_constant<int, 3>());
  }
  if constexpr (DIRECT) {
    epilogue_direct<EPI, OT, TM, TN>(acc, m0 + wm * TL::WTM, n0 + wn * TL::WTN, N, om, ep, pe_ld, lane);
    wait_vm_lds0<0>();  // the trailing out-of-range DMAs land before the LDS is released
    return;
  }
  wait_vm_lds0<0>();
  __syncthreads();

  constexpr int LDW = WTN + 4;
  float* stg = reinterpret_cast<float*>(st0) + wv * SR * LDW;
  const int wcol = n0 + wn * TL::WTN;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
  for (int hs = 0; hs < 32 / SR; ++hs) {
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = 8 * (v >> 2) + 4 * half + (v & 3) - hs * SR;
        if (r >= 0 && r < SR) stg[r * LDW + 32 * j + l32] = acc[i][j][v];
      }
    __syncthreads();
    const int64_t rbase = m0 + wm * TL::WTM + i * 32 + hs * SR;
    epilogue_rows<EPI, OT, WTN, SR>(stg, LDW, rbase, wcol, N, om, ep, pe_ld, lane);
    __syncthreads();
  }
  }
}

// Persistent form of gemm_pipe2_kernel: a grid of at most one wave of resident workgroups, each
// walking a sequence of output tiles.  The DMA stream runs NST-1 K steps ahead across tile
// boundaries, so the next tile's first stages load while the current one finishes, and the
// epilogue (straight from registers, no barrier) drains while the next tile's MFMAs run.
//   Tile order: the logical tiles (groups of gm m-tiles walked column by column) are split into
//   8 contiguous chunks, one per XCD (workgroup b runs on XCD b % 8); the workgroups of an XCD
//   take the tiles of its chunk round-robin, so the tiles in flight on one XCD are neighbours
//   and share A rows and B columns in its L2.  Tiles whose rows are all padding are skipped.
template <class TL, int NST, class AS, class OM, int EPI, typename OT, int TAG>
__global__ __launch_bounds__(TL::NT, TL::MINB) void gemm_persist_kernel(AS as, const bf16_t* __restrict__ Bw,
                                                                       int32_t N, int32_t K, OM om, EpiP ep,
                                                                       int32_t m_tiles, int32_t n_tiles,
                                                                       int32_t pe_ld, int32_t gm) {
  static_assert(NST >= 2 && NST <= 4, "stages");
  constexpr int BM = TL::BM, BN = TL::BN, TM = TL::TM, TN = TL::TN;
  constexpr int BK = TL::BK, NW = TL::NW;
  constexpr int STG = (BM + BN) * BK;
  constexpr int ROWS_PER_DMA = 1024 / (BK * 2);
  constexpr int ADMA = BM / ROWS_PER_DMA / NW;
  constexpr int BDMA = BN / ROWS_PER_DMA / NW;
  constexpr int P = ADMA + BDMA;
  static_assert(ADMA * ROWS_PER_DMA * NW == BM && BDMA * ROWS_PER_DMA * NW == BN, "dma split");
  static_assert(P * (NST - 1) < 64, "vmcnt range");
  constexpr int KS = BK / 16;
  static_assert(KS % 2 == 0, "fragment buffers alternate by step parity");
  __shared__ __attribute__((aligned(1024))) bf16_t st0[STG];
  __shared__ __attribute__((aligned(1024))) bf16_t st1[STG];
  __shared__ __attribute__((aligned(1024))) bf16_t st2[NST > 2 ? STG : 8];
  __shared__ __attribute__((aligned(1024))) bf16_t st3[NST > 3 ? STG : 8];
  auto stage = [&](auto sc) -> bf16_t* {
    constexpr int s = decltype(sc)::value;
    if constexpr (s == 0) return st0;
    else if constexpr (s == 1) return st1;
    else if constexpr (s == 2) return st2;
    else return st3;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63, l32 = lane & 31, half = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv / TL::WGN, wn = wv % TL::WGN;

  // this workgroup's tiles: c0 + q + j * Gx for j = 0, 1, ... below c1
  const int T = m_tiles * n_tiles;
  const int G = gridDim.x;
  const int xcd = blockIdx.x % 8, q = blockIdx.x / 8;
  const int Gx = G / 8 + (xcd < G % 8 ? 1 : 0);
  const int before = xcd * (G / 8) + min(xcd, G % 8);
  const int c0 = (int)((int64_t)T * before / G);
  const int c1 = (int)((int64_t)T * (before + Gx) / G);
  const int n_my = c1 - c0 > q ? (c1 - c0 - q + Gx - 1) / Gx : 0;
  const int gsize = gm * n_tiles;
  auto coord = [&](int j) -> TileCoord {
    const int t = c0 + q + j * Gx;
    const int g = t / gsize;
    const int first_m = g * gm;
    const int gh = m_tiles - first_m < gm ? m_tiles - first_m : gm;
    const int in_g = t - g * gsize;
    return TileCoord{__builtin_amdgcn_readfirstlane(first_m + in_g % gh),
                     __builtin_amdgcn_readfirstlane(in_g / gh)};
  };
  auto live = [&](int j) { return as.tile_live((int64_t)coord(j).mt * BM, BM); };
  auto next_live = [&](int j) {
    while (j < n_my && !live(j)) ++j;
    return j;
  };
  int cj = next_live(0);  // tile being multiplied
  if (cj >= n_my) return;

  const __amdgpu_buffer_rsrc_t ra_rsrc = make_rsrc(as.base(), as.bytes());
  const __amdgpu_buffer_rsrc_t rb_rsrc = make_rsrc(Bw, (int64_t)N * K * 2);
  constexpr int CPR = BK / 8;
  int achunk[ADMA], bchunk[BDMA], arl[ADMA], brl[BDMA];
#pragma unroll
  for (int j = 0; j < ADMA; ++j) {
    arl[j] = (wv * ADMA + j) * ROWS_PER_DMA + lane / CPR;
    achunk[j] = (lane % CPR) ^ swz<BK>(arl[j]);
  }
#pragma unroll
  for (int j = 0; j < BDMA; ++j) {
    brl[j] = (wv * BDMA + j) * ROWS_PER_DMA + lane / CPR;
    bchunk[j] = (lane % CPR) ^ swz<BK>(brl[j]);
  }
  // DMA side: tile dj, K step dk, and the per-lane row offsets of tile dj (all out of range once
  // the sequence is exhausted, so the stream keeps its shape with zero-filling loads)
  typename AS::BRow arow[ADMA];
  uint32_t boffr[BDMA];
  int dj = cj, dk = 0;
  auto setup = [&](int j) {
    const bool ok = j < n_my;
    const TileCoord tc = ok ? coord(j) : TileCoord{m_tiles, 0};
    const int64_t m0 = (int64_t)tc.mt * BM;
    const int n0 = tc.nt * BN;
#pragma unroll
    for (int i = 0; i < ADMA; ++i) arow[i] = as.brow(m0 + arl[i]);
#pragma unroll
    for (int i = 0; i < BDMA; ++i) {
      const int n = n0 + brl[i];
      boffr[i] = (ok && n < N) ? (uint32_t)n * (uint32_t)K * 2u : 0x80000000u;
    }
  };
  const int nk = (K + BK * NST - 1) / (BK * NST) * NST;
  auto dma = [&](bf16_t* st) {
#pragma unroll
    for (int j = 0; j < ADMA; ++j) {
      const int k = dk * BK + achunk[j] * 8;
      const uint32_t off = as.boff(arow[j], as.kc(k));
      bf16_t* dst = st + (wv * ADMA + j) * ROWS_PER_DMA * BK;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra_rsrc, (__attribute__((address_space(3))) void*)dst, 16,
                                               (int)off, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < BDMA; ++j) {
      const int k = dk * BK + bchunk[j] * 8;
      const uint32_t off = (k < K && boffr[j] != 0x80000000u) ? boffr[j] + (uint32_t)k * 2u : 0x80000000u;
      bf16_t* dst = st + BM * BK + (wv * BDMA + j) * ROWS_PER_DMA * BK;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb_rsrc, (__attribute__((address_space(3))) void*)dst, 16,
                                               (int)off, 0, 0, 0);
    }
    if (++dk == nk) {
      dk = 0;
      dj = next_live(dj + 1);
      setup(dj);
    }
  };

  f32x16_t acc[TM][TN];
  auto zero = [&]() {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
  };
  zero();

  const int aoff = (wm * TL::WTM + l32) * BK;
  const int boff = BM * BK + (wn * TL::WTN + l32) * BK;
  const int sw = swz<BK>(l32);
  bf16x8_t fa[2][TM], fb[2][TN];
  auto rd = [&](const bf16_t* st, int ks, int buf) {
    const int ch = ((ks * 2 + half) ^ sw) * 8;
#pragma unroll
    for (int i = 0; i < TM; ++i) fa[buf][i] = *reinterpret_cast<const bf16x8_t*>(st + aoff + i * 32 * BK + ch);
#pragma unroll
    for (int j = 0; j < TN; ++j) fb[buf][j] = *reinterpret_cast<const bf16x8_t*>(st + boff + j * 32 * BK + ch);
  };
  auto mm = [&](int buf) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[buf][j], fa[buf][i], acc[i][j], 0, 0, 0);
  };
  auto barrier = [&]() {
    cbar();
    __builtin_amdgcn_s_barrier();
    cbar();
  };

  setup(dj);
  dma(st0);
  dma(st1);
  if constexpr (NST > 2) dma(st2);
  if constexpr (NST > 3) dma(st3);
  wait_vm_lds0<P * (NST - 1)>();
  barrier();
  rd(st0, 0, 0);

  int ck = 0;
  auto step = [&](auto sc) {
    constexpr int s = decltype(sc)::value;
    const bf16_t* cur = stage(sc);
#pragma unroll
    for (int ks = 0; ks + 1 < KS; ++ks) {
      rd(cur, ks + 1, (ks + 1) & 1);
      __builtin_amdgcn_sched_barrier(0);
      mm(ks & 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    wait_vm_lds0<P * (NST - 2)>();
    barrier();
    dma(stage(sc));
    rd(stage(std::integral_constant<int, (s + 1) % NST>()), 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    mm((KS - 1) & 1);
    __builtin_amdgcn_sched_barrier(0);
  };
  while (cj < n_my) {
    step(std::integral_constant<int, 0>());
    step(std::integral_constant<int, 1>());
    if constexpr (NST > 2) step(std::integral_constant<int, 2>());
    if constexpr (NST > 3) step(std::integral_constant<int, 3>());
    ck += NST;  // nk is a multiple of NST: a tile ends on the last step of a group
    if (ck == nk) {
      const TileCoord tc = coord(cj);
      epilogue_direct<EPI, OT, TM, TN>(acc, (int64_t)tc.mt * BM + wm * TL::WTM, tc.nt * BN + wn * TL::WTN,
                                       N, om, ep, pe_ld, lane);
      zero();
      ck = 0;
      cj = next_live(cj + 1);
    }
  }
  wait_vm_lds0<0>();  // the trailing zero-filling DMAs land before the LDS is released
}

// MFMA fragments of one K-step (BK = 32: 32-row blocks 2048 bytes apart) read from LDS by one
// (outputs are early-clobber: no output may share a register with the address inputs)
// inline-asm block that waits for its own reads before it ends, so the compiler never sees an
// LDS read that could alias the in-flight LDS DMA of later stages (it would otherwise wait for
// every outstanding DMA before each read).
typedef __attribute__((address_space(3))) const void* lds_cptr;
template <int TM, int TN> struct FragK32;
template <> struct FragK32<2, 2> {
  __device__ static inline void load(lds_cptr a, lds_cptr b, bf16x8_t* af, bf16x8_t* bf) {
    asm volatile(
        "ds_read_b128 %0, %4\n\t"
        "ds_read_b128 %1, %4 offset:2048\n\t"
        "ds_read_b128 %2, %5\n\t"
        "ds_read_b128 %3, %5 offset:2048\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(af[0]), "=&v"(af[1]), "=&v"(bf[0]), "=&v"(bf[1])
        : "v"(a), "v"(b)
        : "memory");
  }
};
template <> struct FragK32<4, 2> {
  __device__ static inline void load(lds_cptr a, lds_cptr b, bf16x8_t* af, bf16x8_t* bf) {
    asm volatile(
        "ds_read_b128 %0, %6\n\t"
        "ds_read_b128 %1, %6 offset:2048\n\t"
        "ds_read_b128 %2, %6 offset:4096\n\t"
        "ds_read_b128 %3, %6 offset:6144\n\t"
        "ds_read_b128 %4, %7\n\t"
        "ds_read_b128 %5, %7 offset:2048\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(af[0]), "=&v"(af[1]), "=&v"(af[2]), "=&v"(af[3]), "=&v"(bf[0]), "=&v"(bf[1])
        : "v"(a), "v"(b)
        : "memory");
  }
};
template <> struct FragK32<2, 4> {
  __device__ static inline void load(lds_cptr a, lds_cptr b, bf16x8_t* af, bf16x8_t* bf) {
    asm volatile(
        "ds_read_b128 %0, %6\n\t"
        "ds_read_b128 %1, %6 offset:2048\n\t"
        "ds_read_b128 %2, %7\n\t"
        "ds_read_b128 %3, %7 offset:2048\n\t"
        "ds_read_b128 %4, %7 offset:4096\n\t"
        "ds_read_b128 %5, %7 offset:6144\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(af[0]), "=&v"(af[1]), "=&v"(bf[0]), "=&v"(bf[1]), "=&v"(bf[2]), "=&v"(bf[3])
        : "v"(a), "v"(b)
        : "memory");
  }
};

// Ring-pipelined direct-to-LDS GEMM (BK = 32): NST LDS stages; the DMA of tile kt + NST - 1 is
// issued right after the barrier of tile kt, so each tile's loads have NST - 1 tiles of MFMA
// work to land.  Every iteration issues the same number of DMA instructions (tiles past the end
// read as zero into a stage that is never read again), so "this tile has landed" is the fixed
// wait vmcnt <= (NST - 2) * (DMA instructions per tile).
template <class TL, int NST, class AS, class OM, int EPI, typename OT, int TAG>
__global__ __launch_bounds__(TL::NT, TL::MINB) void gemm_ring_kernel(AS as, const bf16_t* __restrict__ Bw,
                                                                    int32_t N, int32_t K, OM om, EpiP ep,
                                                                    int32_t n_tiles, int32_t pe_ld, int32_t gm) {
  constexpr int BM = TL::BM, BN = TL::BN, TM = TL::TM, TN = TL::TN;
  constexpr int WTN = TL::WTN, BK = TL::BK, NW = TL::NW;
  static_assert(BK == 32, "ring kernel uses BK = 32");
  constexpr int STAGE = (BM + BN) * BK;                   // bf16 elements per stage
  constexpr int SMEM = NST * STAGE;
  constexpr int SR = (NW * 32 * (WTN + 4) * 4 <= SMEM * 2) ? 32 : 16;
  static_assert(NW * SR * (WTN + 4) * 4 <= SMEM * 2, "epilogue staging must fit in the tiles");
  constexpr int ROWS_PER_DMA = 1024 / (BK * 2);           // 16 rows of 64 bytes
  constexpr int ADMA = BM / ROWS_PER_DMA / NW;
  constexpr int BDMA = BN / ROWS_PER_DMA / NW;
  static_assert(ADMA * ROWS_PER_DMA * NW == BM && BDMA * ROWS_PER_DMA * NW == BN, "dma split");
  constexpr int NDMA = ADMA + BDMA;
  constexpr int VMC = (NST - 2) * NDMA;
  static_assert(VMC < 64, "vmcnt range");
  constexpr int WAIT_TILE = (VMC & 15) | (7 << 4) | (15 << 8) | ((VMC >> 4) << 14);
  constexpr int KS = BK / 16;
  __shared__ __attribute__((aligned(1024))) bf16_t smem[SMEM];

  const int tid = threadIdx.x;
  const int lane = tid & 63, l32 = lane & 31, half = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv / TL::WGN, wn = wv % TL::WGN;
  const TileCoord tc = tile_coord(n_tiles, gm);
  const int64_t mt = tc.mt;
  const int nt = tc.nt;
  const int64_t m0 = mt * BM;
  const int n0 = nt * BN;
  if (!as.tile_live(m0, BM)) return;

  const __amdgpu_buffer_rsrc_t ra_rsrc = make_rsrc(as.base(), as.bytes());
  const __amdgpu_buffer_rsrc_t rb_rsrc = make_rsrc(Bw, (int64_t)N * K * 2);
  constexpr int CPR = BK / 8;
  typename AS::BRow arow[ADMA];
  int achunk[ADMA];
  uint32_t boffr[BDMA];
  int bchunk[BDMA];
#pragma unroll
  for (int j = 0; j < ADMA; ++j) {
    const int r = (wv * ADMA + j) * ROWS_PER_DMA + lane / CPR;
    achunk[j] = (lane % CPR) ^ swz<BK>(r);
    arow[j] = as.brow(m0 + r);
  }
#pragma unroll
  for (int j = 0; j < BDMA; ++j) {
    const int r = (wv * BDMA + j) * ROWS_PER_DMA + lane / CPR;
    bchunk[j] = (lane % CPR) ^ swz<BK>(r);
    const int n = n0 + r;
    boffr[j] = n < N ? (uint32_t)n * (uint32_t)K * 2u : 0x80000000u;
  }
  auto dma = [&](int kt, int stage) {
    bf16_t* sa = smem + stage * STAGE;
    bf16_t* sb = sa + BM * BK;
#pragma unroll
    for (int j = 0; j < ADMA; ++j) {
      const int k = kt * BK + achunk[j] * 8;
      const uint32_t off = as.boff(arow[j], as.kc(k));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ra_rsrc, (__attribute__((address_space(3))) void*)(sa + (wv * ADMA + j) * ROWS_PER_DMA * BK),
          16, (int)off, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < BDMA; ++j) {
      const int k = kt * BK + bchunk[j] * 8;
      const uint32_t off = (k < K && boffr[j] != 0x80000000u) ? boffr[j] + (uint32_t)k * 2u : 0x80000000u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rb_rsrc, (__attribute__((address_space(3))) void*)(sb + (wv * BDMA + j) * ROWS_PER_DMA * BK),
          16, (int)off, 0, 0, 0);
    }
  };

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int arow0 = wm * TL::WTM + l32;
  const int brow0 = wn * TL::WTN + l32;
  const int sw = swz<BK>(l32);
  const int nk = (K + BK - 1) / BK;
#pragma unroll
  for (int t = 0; t < NST - 1; ++t) dma(t, t);
  int stage = 0;
  for (int kt = 0; kt < nk; ++kt) {
    __builtin_amdgcn_s_waitcnt(WAIT_TILE);  // this wave's DMA of tile kt has landed
    __builtin_amdgcn_s_barrier();           // all waves: tile kt in LDS, tile kt-1 consumed
    dma(kt + NST - 1, stage == 0 ? NST - 1 : stage - 1);
    const bf16_t* sa = smem + stage * STAGE;
    const bf16_t* sb = sa + BM * BK;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int ch = ((ks * 2 + half) ^ sw) * 8;
      bf16x8_t af[TM], bfr[TN];
      FragK32<TM, TN>::load((lds_cptr)(sa + arow0 * BK + ch), (lds_cptr)(sb + brow0 * BK + ch), af, bfr);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    stage = stage + 1 == NST ? 0 : stage + 1;
  }
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): the trailing zero-fill DMAs have landed
  __syncthreads();

  constexpr int LDW = WTN + 4;
  float* stg = reinterpret_cast<float*>(smem) + wv * SR * LDW;
  const int wcol = n0 + wn * TL::WTN;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
  for (int hs = 0; hs < 32 / SR; ++hs) {
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = 8 * (v >> 2) + 4 * half + (v & 3) - hs * SR;
        if (r >= 0 && r < SR) stg[r * LDW + 32 * j + l32] = acc[i][j][v];
      }
    __syncthreads();
    const int64_t rbase = m0 + wm * TL::WTM + i * 32 + hs * SR;
    epilogue_rows<EPI, OT, WTN, SR>(stg, LDW, rbase, wcol, N, om, ep, pe_ld, lane);
    __syncthreads();
  }
  }
}

// ============================================================================================
// fp32 VALU kernel (tiny fp32 configuration; not a throughput path)
// ============================================================================================
constexpr int FBM = 64, FBN = 64, FBK = 16;

template <class AS, class OM, int EPI, int TAG>
__global__ __launch_bounds__(256) void gemm_f32_kernel(AS as, const float* __restrict__ Bw,
                                                       int32_t N, int32_t K, OM om, EpiP ep,
                                                       int32_t n_tiles, int32_t pe_ld) {
  __shared__ float sA[FBK][FBM + 4];
  __shared__ float sB[FBK][FBN + 4];
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int64_t mt = blockIdx.x / n_tiles;
  const int nt = blockIdx.x - (int)(mt * n_tiles);
  const int64_t m0 = mt * FBM;
  const int n0 = nt * FBN;
  if (!as.tile_live(m0, FBM)) return;

  // loader: 4 consecutive k of one row per thread
  const int lrow = tid >> 2;
  const int lk = (tid & 3) * 4;
  const auto arow = as.row(m0 + lrow);
  const int bn = n0 + lrow;
  const float* brow = bn < N ? Bw + (int64_t)bn * K : nullptr;

  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;

  for (int k0 = 0; k0 < K; k0 += FBK) {
    const int k = k0 + lk;
    const float* pa = as.ptr(arow, as.kc(k));
    const float4 va = pa ? *reinterpret_cast<const float4*>(pa) : make_float4(0, 0, 0, 0);
    const float4 vb = (brow && k < K) ? *reinterpret_cast<const float4*>(brow + k)
                                      : make_float4(0, 0, 0, 0);
    sA[lk + 0][lrow] = va.x; sA[lk + 1][lrow] = va.y; sA[lk + 2][lrow] = va.z; sA[lk + 3][lrow] = va.w;
    sB[lk + 0][lrow] = vb.x; sB[lk + 1][lrow] = vb.y; sB[lk + 2][lrow] = vb.z; sB[lk + 3][lrow] = vb.w;
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < FBK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = sA[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = sB[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t row = m0 + ty * 4 + i;
    const int64_t off = om.off(row);
    if (off < 0) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + tx * 4 + j;
      if (col >= N) continue;
      if constexpr (EPI == EPI_PE) {
        reinterpret_cast<float*>(ep.C)[off + col] =
            acc[i][j] + ep.pe[(int64_t)ep.tok_pos[row] * pe_ld + col];
      } else {
        epi_store<EPI, float>(ep, off, row, col, acc[i][j]);
      }
    }
  }
}

// ============================================================================================
// dispatch
// ============================================================================================
// NST = 0: gemm_dtl_kernel (one tile in flight); NST >= 3: gemm_ilv_kernel with NST stages.
template <typename T, class TL, class AS, class OM, int EPI, int TAG, int NST = 0>
hipError_t run(const AS& as, const T* Bw, int32_t N, int32_t K, const OM& om, const EpiP& ep,
               int64_t m_rows, int32_t pe_ld, hipStream_t s) {
  if constexpr (std::is_same<T, bf16_t>::value) {
    const int n_tiles = (N + TL::BN - 1) / TL::BN;
    const int64_t m_tiles = (m_rows + TL::BM - 1) / TL::BM;
    if (m_tiles * n_tiles == 0) return hipSuccess;
    if (m_tiles * n_tiles >= (int64_t(1) << 31)) return hipErrorInvalidValue;
    if constexpr (NST == 0)
      hipLaunchKernelGGL((gemm_dtl_kernel<TL, AS, OM, EPI, bf16_t, TAG>),
                         dim3((unsigned)(m_tiles * n_tiles)), dim3(TL::NT), 0, s, as, Bw, N, K, om, ep,
                         n_tiles, pe_ld, AE_GEMM_GROUP_M);
    else
      hipLaunchKernelGGL((gemm_ilv_kernel<TL, NST, AS, OM, EPI, bf16_t, TAG>),
                         dim3((unsigned)(m_tiles * n_tiles)), dim3(TL::NT), 0, s, as, Bw, N, K, om, ep,
                         n_tiles, pe_ld, AE_GEMM_GROUP_M);
  } else {
    if constexpr (EPI == EPI_SWIGLU) {
      return hipErrorInvalidValue;  // the fp32 path applies SwiGLU in a separate kernel
    } else {
      const int n_tiles = (N + FBN - 1) / FBN;
      const int64_t m_tiles = (m_rows + FBM - 1) / FBM;
      if (m_tiles * n_tiles == 0) return hipSuccess;
      hipLaunchKernelGGL((gemm_f32_kernel<AS, OM, EPI, TAG>), dim3((unsigned)(m_tiles * n_tiles)),
                         dim3(256), 0, s, as, Bw, N, K, om, ep, n_tiles, pe_ld);
    }
  }
  return hipGetLastError();
}

// Tile choice (measured on MI355X with the shapes of the tower, M = 6000):
//  - N = 1280 or 3840 (o-proj, FFN2, conv_out, proj1, QKV): 128x128 tiles, BK 64, two workgroups
//    per CU; a wider tile leaves CUs idle in the last round.
//  - N = 5120 (FFN1): 256x128 tiles, 8 waves (two per SIMD), BK 32.
//  - K >= 2048 (adapter gate/up and down, head proj2): 256x256 tiles, 8 waves, BK 32, four
//    stages with the refill DMAs spread over the MFMAs.
using TileWide = Tile<256, 128, 4, 2, 32, 1>;
using TileNarrow = Tile<128, 128, 2, 2, 64, 2>;
using TileLarge = Tile<256, 256, 2, 4, 32, 1>;
enum class LinKind { Narrow, Wide, Large };
inline LinKind lin_kind(int64_t /*M*/, int64_t N, int64_t K) {
  if (N == 1280 || N == 3840 || N < 2048) return LinKind::Narrow;
  if (K >= 2048) return LinKind::Large;
  return LinKind::Wide;
}

// conv2/conv3 (N = 480 output channels, K = 9 * 480): 256x256 tiles with four stages measured
// fastest (the 480 channels fill two 256-wide column tiles at 94%)
#ifndef AE_CONV_TILE
#define AE_CONV_TILE 1
#endif
#if AE_CONV_TILE == 0
using TileConv = Tile<256, 128, 4, 2, 32, 1>;
constexpr int kConvStages = 0;
#elif AE_CONV_TILE == 1
using TileConv = Tile<256, 256, 2, 4, 32, 1>;
constexpr int kConvStages = 4;
#elif AE_CONV_TILE == 2
using TileConv = Tile<256, 128, 4, 2, 32, 1>;
constexpr int kConvStages = 4;
#else
using TileConv = Tile<128, 128, 2, 2, 64, 2>;
constexpr int kConvStages = 0;
#endif

template <typename T, int TAG, int EPI>
hipError_t lin(const LinearArgs& a, hipStream_t s) {
  ALinear<T> as{reinterpret_cast<const T*>(a.A), a.lda, a.M, a.K};
  OLinear om{a.M, a.ldc};
  EpiP ep{a.bias, a.C, a.pe, a.tok_pos};
  const T* Bw = reinterpret_cast<const T*>(a.W);
  const int pe_ld = EPI == EPI_PE ? a.N : 0;
  switch (lin_kind(a.M, a.N, a.K)) {
    case LinKind::Large:
      return run<T, TileLarge, ALinear<T>, OLinear, EPI, TAG, 4>(as, Bw, a.N, a.K, om, ep, a.M, pe_ld, s);
    case LinKind::Wide:
      return run<T, TileWide, ALinear<T>, OLinear, EPI, TAG>(as, Bw, a.N, a.K, om, ep, a.M, pe_ld, s);
    default:
      return run<T, TileNarrow, ALinear<T>, OLinear, EPI, TAG>(as, Bw, a.N, a.K, om, ep, a.M, pe_ld, s);
  }
}

}  // namespace

// Each forward-pass role has its own kernel symbol with its fixed epilogue; any other
// (role, epilogue) pair runs under the ENC_K_OTHER symbol.
template <typename T>
hipError_t launch_linear(const LinearArgs& a, int epi, int tag, hipStream_t s) {
  constexpr bool BF = std::is_same<T, bf16_t>::value;
  if (tag == ENC_K_QKV && epi == EPI_BIAS) return lin<T, ENC_K_QKV, EPI_BIAS>(a, s);
  if (tag == ENC_K_OPROJ && epi == EPI_RESADD) return lin<T, ENC_K_OPROJ, EPI_RESADD>(a, s);
  if (tag == ENC_K_FFN1 && epi == EPI_BIAS_GELU) return lin<T, ENC_K_FFN1, EPI_BIAS_GELU>(a, s);
  if (tag == ENC_K_FFN2 && epi == EPI_RESADD) return lin<T, ENC_K_FFN2, EPI_RESADD>(a, s);
  if (tag == ENC_K_PROJ1 && epi == EPI_BIAS_GELU) return lin<T, ENC_K_PROJ1, EPI_BIAS_GELU>(a, s);
  if (tag == ENC_K_PROJ2 && epi == EPI_BIAS) return lin<T, ENC_K_PROJ2, EPI_BIAS>(a, s);
  if (tag == ENC_K_CONV_OUT && epi == EPI_PE) return lin<T, ENC_K_CONV_OUT, EPI_PE>(a, s);
  if (tag == ENC_K_DOWN && epi == EPI_BIAS) return lin<T, ENC_K_DOWN, EPI_BIAS>(a, s);
  if constexpr (BF) {
    if (tag == ENC_K_GATE_UP && epi == EPI_SWIGLU) return lin<T, ENC_K_GATE_UP, EPI_SWIGLU>(a, s);
  } else {
    if (tag == ENC_K_GATE_UP && epi == EPI_BIAS) return lin<T, ENC_K_GATE_UP, EPI_BIAS>(a, s);
  }
  switch (epi) {
    case EPI_BIAS: return lin<T, ENC_K_OTHER, EPI_BIAS>(a, s);
    case EPI_BIAS_GELU: return lin<T, ENC_K_OTHER, EPI_BIAS_GELU>(a, s);
    case EPI_RESADD: return lin<T, ENC_K_OTHER, EPI_RESADD>(a, s);
    case EPI_SWIGLU:
      if constexpr (BF) return lin<T, ENC_K_OTHER, EPI_SWIGLU>(a, s);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
hipError_t launch_conv_igemm(const PassGeom& g, int level, const T* in, const T* wpk,
                             const float* bias, int32_t C, T* out, hipStream_t s) {
  const int Fin = level == 2 ? 64 : 32;
  const int Fout = Fin / 2;
  const int Lin_max = level == 2 ? 4 * g.W : 2 * g.W;
  const int Lout_max = Lin_max / 2;
  const int rows_per_win = Lout_max * Fout;
  const int64_t m_rows = (int64_t)g.n_win * rows_per_win;
  if ((int64_t)g.n_win * Lin_max * Fin * C >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  AConv<T> as{in, g.wins, C, Fin, Fout, Lin_max, level, rows_per_win, 9 * C, m_rows,
              (int64_t)g.n_win * Lin_max * Fin * C * (int64_t)sizeof(T)};
  OConv om{g.wins, rows_per_win, Fout, C, level, Lout_max, m_rows};
  EpiP ep{bias, out, nullptr, nullptr};
  if (level == 2)
    return run<T, TileConv, AConv<T>, OConv, EPI_BIAS_GELU, ENC_K_CONV2, kConvStages>(as, wpk, C, 9 * C, om, ep,
                                                                                     m_rows, 0, s);
  return run<T, TileConv, AConv<T>, OConv, EPI_BIAS_GELU, ENC_K_CONV3, kConvStages>(as, wpk, C, 9 * C, om, ep,
                                                                                   m_rows, 0, s);
}

template hipError_t launch_linear<bf16_t>(const LinearArgs&, int, int, hipStream_t);
template hipError_t launch_linear<float>(const LinearArgs&, int, int, hipStream_t);
template hipError_t launch_conv_igemm<bf16_t>(const PassGeom&, int, const bf16_t*, const bf16_t*,
                                              const float*, int32_t, bf16_t*, hipStream_t);
template hipError_t launch_conv_igemm<float>(const PassGeom&, int, const float*, const float*,
                                             const float*, int32_t, float*, hipStream_t);

}  // namespace ae
