// Dense contractions of the tower: every linear layer and the conv2/conv3 implicit GEMMs.
//
//   C[m, n] = epilogue( sum_k A[m, k] * B[n, k] )
//
// A is an activation (row-major, K contiguous) or, for the 3x3 stride-2 convolutions, the
// im2col view of a channels-last activation generated on the fly by the loader (logical K
// ordered as tap-major, channel-minor, so each 8-element chunk is one contiguous 16-byte read of
// one input position; out-of-image taps and positions past a window's valid length read as
// zero; the staged kernels walk K as 32-channel blocks, then taps, then channels, see AConv).
// B is a weight matrix [N, K] (PyTorch Linear layout; conv weights permuted to [out][tap][in]
// at pack time), plain or, for the staged kernel, K-blocked (b_tiled: blocks of 512/BK rows x
// BK columns, so that each LDS-DMA instruction reads one contiguous kilobyte; the forward's own
// weights are stored so).  Epilogues fuse the bias, exact GELU, the fp32 residual update, the
// sinusoidal positions and the SwiGLU gate into the store.
//
// bf16 path: v_mfma_f32_32x32x16_bf16 on gfx950 with fp32 accumulators.  Tiles move from global
// memory straight into LDS with buffer_load_dwordx4 ... lds (16 bytes per lane, no VGPR
// staging); LDS rows are XOR-swizzled so the fragment reads are free of bank conflicts; the
// epilogue stages accumulator rows through LDS for coalesced stores.  Three kernels:
//   gemm_dtl_kernel   one K tile in flight, all fragments of a tile read before the next DMA;
//   gemm_ilv_kernel   NST stages in separate LDS arrays, refill DMAs spread over the MFMAs;
//   gemm_ilvq_kernel  the staged kernel with int4 weights expanded into the stages' B tiles.
// The tile shape and kernel per call are chosen in the dispatch section at the end.
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
  // the staged kernels' K order is the natural one (step base eb, lane offset off)
  __device__ KC kc_step(int eb, int off) const { return kc(eb + off); }
  __device__ int k_logical(int eb, int off) const { return eb + off; }
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
  __host__ __device__ int64_t bytes() const { return M * lda * (int64_t)sizeof(T); }
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
    // k / C without an integer division: (k + 1/2) / C lies at least 1/(2C) inside its unit
    // interval, far more than the float error for k < 2^24 and C <= 65536
    const int tap = (int)(((float)k + 0.5f) * inv_c);
    const int ci = k - tap * C;
    const int da = tap / 3, db = tap - 3 * (tap / 3);  // frequency tap, time tap
    c.bit = 1 << tap;
    c.toff = (db * Fin + da) * C + ci;
    return c;
  }
  // K order of the staged kernels: blocks of 32 input channels outermost, then the nine taps,
  // then the channels of the block (C % 32 == 0), so that the nine taps reading one input
  // neighbourhood run in consecutive K steps and their re-reads of each input position hit in
  // L2.  With 32-wide K steps a step is one (block, tap) pair: the step base eb (a multiple of
  // 32, wave-uniform) selects it, and the lane offset off < 32 the channel within the block.
  // Step element eb + off is logical index tap * C + channel of the packed weights.
  __device__ KC kc_step(int eb, int off) const {
    const int b = eb / 288, tap = (eb - b * 288) >> 5;
    const int da = tap / 3, db = tap - 3 * (tap / 3);
    KC c;
    c.ok = eb < K;
    c.bit = 1 << tap;
    c.toff = (db * Fin + da) * C + (b << 5) + off;
    return c;
  }
  __device__ int k_logical(int eb, int off) const {
    const int b = eb / 288, tap = (eb - b * 288) >> 5;
    return tap * C + (b << 5) + off;
  }
  __device__ const T* ptr(const Row& x, const KC& c) const {
    return (c.ok && (x.mask & c.bit)) ? in + (x.off + c.toff) : nullptr;
  }
  using BRow = Row;
  __device__ BRow brow(int64_t r) const { return row(r); }
  __device__ uint32_t boff(const BRow& x, const KC& c) const {
    return (c.ok && (x.mask & c.bit)) ? (uint32_t)((x.off + c.toff) * (int)sizeof(T)) : 0x80000000u;
  }
  __host__ __device__ int64_t bytes() const { return (int64_t)wins_bytes; }
  __device__ const void* base() const { return in; }
  int64_t wins_bytes;  // bytes of the input activation
  float inv_c;         // 1 / C
};

// ============================================================================================
// output row maps: element offset of (row, 0) in C, or -1 for rows that are not stored
// ============================================================================================
struct OLinear {
  int64_t M, ldc;
  struct Ctx {};
  __device__ Ctx ctx(int64_t) const { return Ctx{}; }
  __device__ int64_t off(const Ctx&, int64_t r) const { return r < M ? r * ldc : -1; }
  __device__ int64_t off_row(int64_t r) const { return r < M ? r * ldc : -1; }
};

template <int LEVEL, bool SPAN2>
struct OConv {
  const Win* wins;
  int32_t rows_per_win, Fout, C, Lout_max;
  int64_t m_rows;  // < 2^31
  // SPAN2: a window has at least as many rows as one wave's share of a tile, so the rows of a
  // wave lie in two windows at most; their two table entries are read once per wave with
  // scalar loads (which do not wait behind the wave's stores).  Otherwise each row reads its
  // own entry.  Straight-line code either way (rows outside the output are rejected by the
  // final select), so that the epilogue's loads and stores are not split by branches.
  struct Ctx { int w0; Win a, b; };
  __device__ Ctx ctx(int64_t r0) const {
    Ctx c{};
    if constexpr (SPAN2) {
      const int n_win = (int)(m_rows / rows_per_win);
      const int w0 = __builtin_amdgcn_readfirstlane((int)((r0 < m_rows ? r0 : m_rows - 1) / rows_per_win));
      c.w0 = w0;
      c.a = wins[w0];
      c.b = wins[w0 + 1 < n_win ? w0 + 1 : w0];
    }
    return c;
  }
  __device__ int64_t off(const Ctx& c, int64_t r) const {
    const bool inr = r < m_rows;
    int w, loc;
    Win wn;
    if constexpr (SPAN2) {
      const int d = inr ? (int)(r - (int64_t)c.w0 * rows_per_win) : 0;
      const bool second = d >= rows_per_win;
      w = c.w0 + (second ? 1 : 0);
      loc = second ? d - rows_per_win : d;
      wn.L2 = second ? c.b.L2 : c.a.L2;
      wn.L3 = second ? c.b.L3 : c.a.L3;
      wn.tok = second ? c.b.tok : c.a.tok;
    } else {
      const int rr = inr ? (int)r : 0;
      w = rr / rows_per_win;
      loc = rr - w * rows_per_win;
      wn = wins[w];
    }
    const int t = loc / Fout, f = loc - (loc / Fout) * Fout;
    int64_t o;
    if constexpr (LEVEL == 2) o = (((int64_t)w * Lout_max + t) * Fout + f) * C;
    else o = ((int64_t)(wn.tok + t) * Fout + f) * C;  // token rows [tok][16][C]
    return (inr && t < (LEVEL == 2 ? wn.L2 : wn.L3)) ? o : -1;
  }
  // any row, its own table entry (fp32 path)
  __device__ int64_t off_row(int64_t r) const {
    const OConv<LEVEL, false> o{wins, rows_per_win, Fout, C, Lout_max, m_rows};
    return o.off(typename OConv<LEVEL, false>::Ctx{}, r);
  }
};

struct EpiP {
  const float* bias;
  void* C;
  const float* pe;
  const int32_t* tok_pos;
  int64_t c_bytes;  // extent of C in bytes (buffer-store range; < 2^31)
  int64_t c_slice;  // split-K: elements between the partial products of consecutive K ranges
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
// Block tile BM x BN x BK, WGM x WGN waves, each owning (BM/WGM) x (BN/WGN) as TM x TN blocks
// of 32x32 MFMA output.  MINB workgroups are meant to share a CU (occupancy hint).
template <int BM_, int BN_, int WGM_, int WGN_, int BK_ = 64, int MINB_ = 1>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, WGM = WGM_, WGN = WGN_, BK = BK_, MINB = MINB_;
  static constexpr int NW = WGM * WGN, NT = 64 * NW;  // waves, threads
  static constexpr int WTM = BM / WGM, WTN = BN / WGN;
  static constexpr int TM = WTM / 32, TN = WTN / 32;
  static_assert(TM * 32 == WTM && TN * 32 == WTN, "tile");
  static_assert(BK == 32 || BK == 64, "BK");
};

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

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* p, int64_t bytes) {
  // raw buffer: stride 0, range check against `bytes`; dword3 0x00020000 (32-bit data format)
  // integer clamp (a 64-bit min lowers to a vector f64 op here, which would drag the whole
  // descriptor into vector registers and wrap every buffer load in a waterfall loop)
  const int n = __builtin_amdgcn_readfirstlane(bytes > 0x7fffffff ? 0x7fffffff : (int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, n, 0x00020000);
}

// Compiler-only barrier: no LDS access moves across it, and unlike __syncthreads() it adds
// no release fence (which would wait for every LDS DMA in flight, deeper stages included).
__device__ inline void cbar() { asm volatile("" ::: "memory"); }

// Epilogue of one wave.  Its TM x TN accumulator blocks (32x32 each; tile rows rbase0..,
// columns wcol..wcol+WTN-1) pass through the wave's own SR staging rows in LDS (stride WTN + 4
// floats), SR rows per round, and leave as 16-byte row pieces: each lane owns CPL consecutive
// columns (4 fp32 or 8 bf16) of every (64 / (WTN / CPL))-th staged row.  The SwiGLU gate writes
// 8-byte pieces of four outputs.
//
// Ordering.  The staging rows belong to this wave alone and a wave's LDS accesses execute in
// order, so compiler fences are all the ordering the staging needs (a workgroup barrier would
// also wait for the wave's outstanding stores).  Global stores and loads share one in-order
// completion counter here, so a load issued after a store cannot be waited for without waiting
// for the store: the bias is loaded once up front, and everything a round reads from global
// memory (its output row offsets, which may read the window table, and the residual of the
// fp32 update) is loaded one round ahead, before the stores of the current round.
template <int EPI, typename OT, int TM, int TN, int WTN, int SR, class OM>
__device__ __attribute__((always_inline)) inline void wave_epilogue(const f32x16_t (&acc)[TM][TN], float* stg,
                                                                   int64_t rbase0, int wcol, int N, const OM& om,
                                                                   const EpiP& ep, int pe_ld, int lane) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  constexpr int LDW = WTN + 4;
  constexpr int HS = 32 / SR;       // rounds per 32-row block
  constexpr int ROUNDS = TM * HS;
  constexpr bool GATE = EPI == EPI_SWIGLU;
  constexpr bool F32OUT = EPI == EPI_RESADD || EPI == EPI_PE || EPI == EPI_STORE_F32;
  constexpr int ES = F32OUT ? 4 : (int)sizeof(OT);
  // output columns per lane: eight for 2-byte outputs (one 16-byte store; N % 8 == 0 there),
  // else four; the gate reads four gate and four up columns for four outputs
  constexpr int CPL = (ES == 2 && !GATE) ? 8 : 4;
  constexpr int Q = GATE ? WTN / 8 : WTN / CPL;  // lanes per staged row
  constexpr int RPI = 64 / Q;                   // staged rows per 64 lanes
  constexpr int T = SR / RPI;                   // rows per lane per round
  static_assert(RPI * Q == 64 && T * RPI == SR, "epilogue lane map");
  constexpr uint32_t NOWHERE = 0x80000000u;     // out of range: loads read 0, stores are dropped
  const int l32 = lane & 31, half = lane >> 5;
  const int q4 = lane % Q, rs = lane / Q;
  // gate: (gate, up) pairs of 32 columns interleaved in 64-column groups; the output column is
  // half the group's start plus the position within the pair
  const int gp = GATE ? (4 * q4) / 32 : 0, gj = GATE ? (4 * q4) % 32 : 0;
  const int scol = GATE ? 64 * gp + gj : CPL * q4;          // staged column
  const int col = GATE ? (wcol + 64 * gp) / 2 + gj : wcol + CPL * q4;  // output column
  const bool colok = GATE ? wcol + 64 * gp < N : col < N;
  const __amdgpu_buffer_rsrc_t crs = make_rsrc(ep.C, ep.c_bytes);
  const int64_t slice = (int64_t)blockIdx.y * ep.c_slice;  // split-K partial of this K range
  float4 bv = make_float4(0.f, 0.f, 0.f, 0.f), bv2 = bv;
  if constexpr (EPI != EPI_PE && !GATE)
    if (ep.bias && colok) {
      bv = *reinterpret_cast<const float4*>(ep.bias + col);
      if constexpr (CPL == 8) bv2 = *reinterpret_cast<const float4*>(ep.bias + col + 4);
    }

  const typename OM::Ctx octx = om.ctx(rbase0);
  auto row_of = [&](int rd, int t) -> int64_t { return rbase0 + (rd / HS) * 32 + (rd % HS) * SR + rs + RPI * t; };
  // byte offset of this lane's 4 outputs in row (rd, t), or NOWHERE
  uint32_t offn[T];
  float4 resn[T];
  auto prefetch = [&](int rd) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
      // computed for every lane and selected, so that no branch splits the loads and stores
      // (the wait-count pass would then wait for all of them where the branches merge)
      const int64_t off = om.off(octx, row_of(rd, t));
      const uint32_t o = (uint32_t)((off + col + slice) * ES);
      offn[t] = (colok & (off >= 0)) ? o : NOWHERE;
      if constexpr (EPI == EPI_RESADD)
        resn[t] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(crs, (int)offn[t], 0, 0));
    }
  };
  prefetch(0);
#pragma unroll
  for (int rd = 0; rd < ROUNDS; ++rd) {
    const int i = rd / HS, hs = rd % HS;
    cbar();  // the previous round's staging reads are issued before these writes
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = 8 * (v >> 2) + 4 * half + (v & 3) - hs * SR;
        if (r >= 0 && r < SR) stg[r * LDW + 32 * j + l32] = acc[i][j][v];
      }
    cbar();
    float4 a[T], g2[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      a[t] = *reinterpret_cast<const float4*>(stg + (rs + RPI * t) * LDW + scol);
      if constexpr (GATE) g2[t] = *reinterpret_cast<const float4*>(stg + (rs + RPI * t) * LDW + scol + 32);
      if constexpr (CPL == 8) g2[t] = *reinterpret_cast<const float4*>(stg + (rs + RPI * t) * LDW + scol + 4);
    }
    uint32_t off[T];
    float4 res[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      off[t] = offn[t];
      res[t] = resn[t];
    }
    if (rd + 1 < ROUNDS) prefetch(rd + 1);
#pragma unroll
    for (int t = 0; t < T; ++t) {
      float4 x = a[t];
      if constexpr (GATE) {
        x = make_float4(silu(x.x) * g2[t].x, silu(x.y) * g2[t].y, silu(x.z) * g2[t].z, silu(x.w) * g2[t].w);
      } else if constexpr (EPI == EPI_PE) {
        // rows outside the output read position 0 (their stores are dropped)
        const int64_t row = row_of(rd, t);
        const int pos = off[t] != NOWHERE ? ep.tok_pos[row] : 0;
        const float4 pe = *reinterpret_cast<const float4*>(ep.pe + (int64_t)pos * pe_ld + (colok ? col : 0));
        x = make_float4(x.x + pe.x, x.y + pe.y, x.z + pe.z, x.w + pe.w);
      } else {
        x.x += bv.x; x.y += bv.y; x.z += bv.z; x.w += bv.w;
        if constexpr (EPI == EPI_RESADD)
          x = make_float4(res[t].x + x.x, res[t].y + x.y, res[t].z + x.z, res[t].w + x.w);
        if constexpr (EPI == EPI_BIAS_GELU) {
          x.x = gelu_erf(x.x); x.y = gelu_erf(x.y); x.z = gelu_erf(x.z); x.w = gelu_erf(x.w);
        }
      }
      if constexpr (CPL == 8) {
        // columns 4..7 of the lane: bias (and GELU), then one 16-byte store of all eight
        float4 y = g2[t];
        y.x += bv2.x; y.y += bv2.y; y.z += bv2.z; y.w += bv2.w;
        if constexpr (EPI == EPI_BIAS_GELU) {
          y.x = gelu_erf(y.x); y.y = gelu_erf(y.y); y.z = gelu_erf(y.z); y.w = gelu_erf(y.w);
        }
        const u32x4 o = {pack_bf16x2(x.x, x.y), pack_bf16x2(x.z, x.w), pack_bf16x2(y.x, y.y),
                         pack_bf16x2(y.z, y.w)};
        __builtin_amdgcn_raw_buffer_store_b128(o, crs, (int)off[t], 0, 0);
      } else if constexpr (ES == 4) {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), crs, (int)off[t], 0, 0);
      } else {
        const u32x2 o = {pack_bf16x2(x.x, x.y), pack_bf16x2(x.z, x.w)};
        __builtin_amdgcn_raw_buffer_store_b64(o, crs, (int)off[t], 0, 0);
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


// TAG only names the call site (one kernel symbol per role, so profiles separate them)
#ifndef AE_GEMM_GROUP_M
#define AE_GEMM_GROUP_M 8
#endif

// int4 weight-only B operand: q [N][K/2] bytes (two's complement nibbles, element k in byte
// k/2, even k in the low nibble) and one bf16 scale per row per group of 128 k, s [N][K/128].
// The kernel multiplies each weight by its scale in fp32 (exact) and rounds the product to bf16.
struct BQuant {
  const uint8_t* q;
  const bf16_t* s;
};

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
  uint32_t boffr[BDMA > 0 ? BDMA : 1];
  int bchunk[BDMA > 0 ? BDMA : 1];
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
  __syncthreads();  // every wave is done with the tiles; the LDS is reused for staging

  wave_epilogue<EPI, OT, TM, TN, WTN, SR>(acc, reinterpret_cast<float*>(smem) + wv * SR * (WTN + 4),
                                          m0 + wm * TL::WTM, n0 + wn * TL::WTN, N, om, ep, pe_ld, lane);
}


// s_waitcnt vmcnt(VM) lgkmcnt(0) (gfx9 encoding: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8],
// vmcnt[5:4] in bits 15:14)
template <int VM>
__device__ inline void wait_vm_lds0() {
  static_assert(VM >= 0 && VM < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4));
}

// NST-stage direct-to-LDS kernel (NST = 2..8).  Each stage is its own __shared__ array, so the
// compiler's wait-count tracking knows which DMA a fragment read depends on and never holds a
// read back for the DMAs of other stages.
//
// Schedule of K step kt (tile kt in stage kt % NST; its first MFMA fragments already in
// registers): the fragment reads of sub-step ks+1 are issued before the MFMAs of ks, so LDS
// latency hides behind MFMAs.  Before the MFMAs of the last sub-step, one barrier publishes tile
// kt+1 and retires every wave's reads of tile kt; the first fragments of tile kt+1 are then
// read, and the freed stage is refilled with tile kt+NST, its DMAs interleaved with those last
// MFMAs.  A tile's DMAs therefore have NST-1 steps to land, and no wave ever waits on LDS
// reads issued after a barrier.
// Split K: workgroup row blockIdx.y covers K range [blockIdx.y * k_span, + k_span) (k_span a
// multiple of BK * NST); a single range covers all of K.
template <class TL, int NST, class AS, class OM, int EPI, typename OT, int TAG>
__global__ __launch_bounds__(TL::NT, TL::MINB) void gemm_ilv_kernel(AS as, const bf16_t* __restrict__ Bw,
                                                                   int32_t N, int32_t K, OM om, EpiP ep,
                                                                   int32_t n_tiles, int32_t pe_ld, int32_t gm,
                                                                   int32_t k_span, int32_t b_tiled) {
  static_assert(NST >= 2 && NST <= 8, "stages");
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
  static_assert(KS % 2 == 0, "the fragment double buffer alternates within a tile");
  __shared__ __attribute__((aligned(1024))) bf16_t st0[STG];
  __shared__ __attribute__((aligned(1024))) bf16_t st1[STG];
  __shared__ __attribute__((aligned(1024))) bf16_t st2[NST > 2 ? STG : 8];
  __shared__ __attribute__((aligned(1024))) bf16_t st3[NST > 3 ? STG : 8];
  __shared__ __attribute__((aligned(1024))) bf16_t st4[NST > 4 ? STG : 8];
  __shared__ __attribute__((aligned(1024))) bf16_t st5[NST > 5 ? STG : 8];
  __shared__ __attribute__((aligned(1024))) bf16_t st6[NST > 6 ? STG : 8];
  __shared__ __attribute__((aligned(1024))) bf16_t st7[NST > 7 ? STG : 8];
  auto stage = [&](auto sc) -> bf16_t* {
    constexpr int s = decltype(sc)::value;
    if constexpr (s == 0) return st0;
    else if constexpr (s == 1) return st1;
    else if constexpr (s == 2) return st2;
    else if constexpr (s == 3) return st3;
    else if constexpr (s == 4) return st4;
    else if constexpr (s == 5) return st5;
    else if constexpr (s == 6) return st6;
    else return st7;
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
    // byte offset of this lane's 16-byte piece at logical k 0, in either weight layout
    if (n >= N)
      boffr[j] = 0x80000000u;
    else if (b_tiled)
      boffr[j] = (uint32_t)(n / ROWS_PER_DMA) * (uint32_t)(K / BK) * 1024u + (uint32_t)(lane / CPR) * (BK * 2u) +
                 (uint32_t)bchunk[j] * 16u;
    else
      boffr[j] = (uint32_t)n * (uint32_t)K * 2u + (uint32_t)bchunk[j] * 16u;
  }
  // all DMA instructions of tile kt into stage st (A rows first, then B rows)
  const int k0 = __builtin_amdgcn_readfirstlane((int)blockIdx.y * k_span);
  const int kend = K < k0 + k_span ? K : k0 + k_span;
  auto dma = [&](int kt, bf16_t* st) {
    const int eb = __builtin_amdgcn_readfirstlane(k0 + kt * BK);
    // B: the step's logical k (a multiple of BK) as a byte offset in the weight layout
    const int kl = as.k_logical(eb, 0);
    const uint32_t kadd = b_tiled ? (uint32_t)(kl / BK) * 1024u : (uint32_t)kl * 2u;
#pragma unroll
    for (int j = 0; j < ADMA; ++j) {
      const int k = k0 + kt * BK + achunk[j] * 8;
      auto kc = as.kc_step(eb, achunk[j] * 8);
      kc.ok = kc.ok && k < kend;
      const uint32_t off = as.boff(arow[j], kc);
      bf16_t* dst = st + (wv * ADMA + j) * ROWS_PER_DMA * BK;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra_rsrc, (__attribute__((address_space(3))) void*)dst, 16,
                                               (int)off, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < BDMA; ++j) {
      const int k = k0 + kt * BK + bchunk[j] * 8;
      const uint32_t off = (k < kend && boffr[j] != 0x80000000u) ? boffr[j] + kadd : 0x80000000u;
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
  // same number of DMAs in flight, so every wait is a constant (the compiler's wait-count
  // tracking merges the states of branches conservatively and would otherwise stall MFMAs on
  // fragment reads they do not use).
  const int nk = (kend - k0 + BK * NST - 1) / (BK * NST) * NST;
  dma(0, st0);
  dma(1, st1);
  if constexpr (NST > 2) dma(2, st2);
  if constexpr (NST > 3) dma(3, st3);
  if constexpr (NST > 4) dma(4, st4);
  if constexpr (NST > 5) dma(5, st5);
  if constexpr (NST > 6) dma(6, st6);
  if constexpr (NST > 7) dma(7, st7);
  wait_vm_lds0<P * (NST - 1)>();  // tile 0 landed
  barrier();
  rd(st0, 0, 0);

  auto step = [&](int kt, auto sc) {
    constexpr int s = decltype(sc)::value;
    bf16_t* cur = stage(sc);
    const bf16_t* nxt = stage(std::integral_constant<int, (s + 1) % NST>());
#pragma unroll
    for (int ks = 0; ks + 1 < KS; ++ks) {
      rd(cur, ks + 1, (ks + 1) & 1);
      __builtin_amdgcn_sched_barrier(0);
      mm(ks & 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    wait_vm_lds0<P * (NST - 2)>();  // tile kt+1 landed; this wave's reads of tile kt retired
    barrier();
    rd(nxt, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    dma(kt + NST, cur);
    mm((KS - 1) & 1);
    // alternate the refill DMAs with the last MFMAs
#pragma unroll
    for (int d = 0; d < P; ++d) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // Every group of NST steps but the last runs branch-free.  The last group always holds a real
  // tile first; its later steps run only while their tiles lie within K (the steps it skips
  // would only multiply the zero tiles).  Its exits are forward branches to the end, so the
  // waits of the loop and of the steps before each exit stay exact.
  const int nreal = (kend - k0 + BK - 1) / BK;
  for (int kt = 0; kt < nk - NST; kt += NST) {
    step(kt, std::integral_constant<int, 0>());
    step(kt + 1, std::integral_constant<int, 1>());
    if constexpr (NST > 2) step(kt + 2, std::integral_constant<int, 2>());
    if constexpr (NST > 3) step(kt + 3, std::integral_constant<int, 3>());
    if constexpr (NST > 4) step(kt + 4, std::integral_constant<int, 4>());
    if constexpr (NST > 5) step(kt + 5, std::integral_constant<int, 5>());
    if constexpr (NST > 6) step(kt + 6, std::integral_constant<int, 6>());
    if constexpr (NST > 7) step(kt + 7, std::integral_constant<int, 7>());
  }
  {
    const int kt = nk - NST;
    auto tail = [&](auto self, auto sc) -> void {
      constexpr int t = decltype(sc)::value;
      step(kt + t, sc);
      if constexpr (t + 1 < NST) {
        if (kt + t + 1 < nreal) self(self, std::integral_constant<int, t + 1>());
      }
    };
    tail(tail, std::integral_constant<int, 0>());
  }
  wait_vm_lds0<0>();  // the trailing zero-fill DMAs land before the stages are reused
  __syncthreads();

  wave_epilogue<EPI, OT, TM, TN, WTN, SR>(acc, reinterpret_cast<float*>(st0) + wv * SR * (WTN + 4),
                                          m0 + wm * TL::WTM, n0 + wn * TL::WTN, N, om, ep, pe_ld, lane);
}

// s_waitcnt vmcnt(VM) only (LDS operations may stay in flight)
template <int VM>
__device__ inline void wait_vm() {
  static_assert(VM >= 0 && VM < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4) | (15 << 8));
}

// The staged kernel with int4 weights (BQuant): A moves by LDS DMA as in gemm_ilv_kernel; B
// arrives as 16-byte chunks of 32 int4 weights plus their bf16 scale, loaded into registers one
// tile ahead of the stage they fill and expanded with the scale into the same swizzled bf16
// layout right after the barrier that frees the stage.  Order of memory operations per K step:
// [int4 chunk and scale of tile kt+NST+1, A DMAs of tile kt+NST], so the wait before the
// expansion leaves the step's A DMAs in flight, and the wait before the barrier (for tile kt+1's
// A) counts the same operations as in the bf16 kernel plus two per step.  The prologue issues
// [int4(t), A(t)] for t < NST-1, then int4(NST-1), int4(NST), A(NST-1), which keeps every loop
// wait exact or stricter.  K is accumulated in the same order as in the bf16 kernels.
template <class TL, int NST, class AS, class OM, int EPI, typename OT, int TAG>
__global__ __launch_bounds__(TL::NT, TL::MINB) void gemm_ilvq_kernel(AS as, int32_t N, int32_t K, OM om, EpiP ep,
                                                                    int32_t n_tiles, int32_t pe_ld, int32_t gm,
                                                                    BQuant bq) {
  static_assert(NST >= 2 && NST <= 6, "stages");
  constexpr int BM = TL::BM, BN = TL::BN, TM = TL::TM, TN = TL::TN;
  constexpr int WTN = TL::WTN, BK = TL::BK, NW = TL::NW;
  static_assert(BK == 64, "int4 groups of 128 span two BK 64 tiles");
  constexpr int STG = (BM + BN) * BK;
  constexpr int SR = (NW * 32 * (WTN + 4) * 4 <= STG * 2) ? 32
                     : (NW * 16 * (WTN + 4) * 4 <= STG * 2) ? 16 : 8;
  static_assert(NW * SR * (WTN + 4) * 4 <= STG * 2, "epilogue staging must fit in one stage");
  constexpr int ROWS_PER_DMA = 1024 / (BK * 2);
  constexpr int ADMA = BM / ROWS_PER_DMA / NW;
  static_assert(ADMA * ROWS_PER_DMA * NW == BM, "dma split");
  constexpr int QOPS = 2;                           // int4 chunk + scale loads per thread per tile
  constexpr int PS = ADMA + QOPS;                   // memory operations per thread per K step
  static_assert(PS * NST < 64, "vmcnt range");
  constexpr int QSEG = BK / 32;                     // 32-weight chunks per tile row
  constexpr int QCH = BN * QSEG;                    // chunks per tile
  static_assert(QCH <= TL::NT, "one int4 chunk per thread at most");
  constexpr int KS = BK / 16;
  static_assert(KS % 2 == 0, "the fragment double buffer alternates within a tile");
  __shared__ __attribute__((aligned(1024))) bf16_t st0[STG];
  __shared__ __attribute__((aligned(1024))) bf16_t st1[STG];
  __shared__ __attribute__((aligned(NST > 2 ? 1024 : 16))) bf16_t st2[NST > 2 ? STG : 8];
  __shared__ __attribute__((aligned(NST > 3 ? 1024 : 16))) bf16_t st3[NST > 3 ? STG : 8];
  __shared__ __attribute__((aligned(NST > 4 ? 1024 : 16))) bf16_t st4[NST > 4 ? STG : 8];
  __shared__ __attribute__((aligned(NST > 5 ? 1024 : 16))) bf16_t st5[NST > 5 ? STG : 8];
  auto stage = [&](auto sc) -> bf16_t* {
    constexpr int s = decltype(sc)::value;
    if constexpr (s == 0) return st0;
    else if constexpr (s == 1) return st1;
    else if constexpr (s == 2) return st2;
    else if constexpr (s == 3) return st3;
    else if constexpr (s == 4) return st4;
    else return st5;
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
  const __amdgpu_buffer_rsrc_t rq_rsrc = make_rsrc(bq.q, (int64_t)N * (K / 2));
  const __amdgpu_buffer_rsrc_t rs_rsrc = make_rsrc(bq.s, (int64_t)N * (K / 128) * 2);
  constexpr int CPR = BK / 8;
  typename AS::BRow arow[ADMA];
  int achunk[ADMA];
#pragma unroll
  for (int j = 0; j < ADMA; ++j) {
    const int r = (wv * ADMA + j) * ROWS_PER_DMA + lane / CPR;
    achunk[j] = (lane % CPR) ^ swz<BK>(r);
    arow[j] = as.brow(m0 + r);
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
  };
  // int4 B: thread tid < QCH owns tile row qr, 32-weight segment qs (rows past N, threads
  // without a chunk and tiles past K read zeros through out-of-range offsets)
  const int qr = tid / QSEG, qs = tid % QSEG;
  const bool qok = tid < QCH && n0 + qr < N;
  const uint32_t qbase = qok ? (uint32_t)(n0 + qr) * (uint32_t)(K / 2) : 0u;
  const uint32_t sbase = qok ? (uint32_t)(n0 + qr) * (uint32_t)(K / 128) * 2u : 0u;
  auto qload = [&](int kt, uint4& qv, uint32_t& sv) {
    const int k = kt * BK + qs * 32;
    const bool ok = qok && k < K;
    qv = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                       rq_rsrc, ok ? (int)(qbase + (uint32_t)k / 2u) : (int)0x80000000, 0, 0));
    sv = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(
        rs_rsrc, ok ? (int)(sbase + (uint32_t)(k / 128) * 2u) : (int)0x80000000, 0, 0);
  };
  auto qstore = [&](bf16_t* st, const uint4& qv, uint32_t sv) {
    if (tid < QCH) {
      const float sf = __uint_as_float(sv << 16);
      const uint32_t w4[4] = {qv.x, qv.y, qv.z, qv.w};
      bf16_t* row = st + BM * BK + qr * BK;
#pragma unroll
      for (int c = 0; c < 4; ++c) {  // 8 weights per word: nibble j holds weight 8c + j
        uint32_t o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int q0 = (int)(w4[c] << (28 - 8 * i)) >> 28;
          const int q1 = (int)(w4[c] << (24 - 8 * i)) >> 28;
          o[i] = pack_bf16x2((float)q0 * sf, (float)q1 * sf);
        }
        const int lc = qs * 4 + c;
        *reinterpret_cast<uint4*>(row + ((lc ^ swz<BK>(qr)) * 8)) = make_uint4(o[0], o[1], o[2], o[3]);
      }
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
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[buf][i], fb[buf][j], acc[i][j], 0, 0, 0);
  };
  auto barrier = [&]() {
    cbar();
    __builtin_amdgcn_s_barrier();
    cbar();
  };

  const int nk = (K + BK * NST - 1) / (BK * NST) * NST;
  // prologue: [q(t), A(t)] for t < NST-1, then q(NST-1), q(NST), A(NST-1)
  uint4 qvp[NST];
  uint32_t svp[NST];
  uint4 qv;
  uint32_t sv;
  {
    auto pro = [&](auto tc_) {
      constexpr int t = decltype(tc_)::value;
      if constexpr (t < NST - 1) {
        qload(t, qvp[t], svp[t]);
        dma(t, stage(std::integral_constant<int, t>()));
      }
    };
    pro(std::integral_constant<int, 0>());
    pro(std::integral_constant<int, 1>());
    pro(std::integral_constant<int, 2>());
    pro(std::integral_constant<int, 3>());
    pro(std::integral_constant<int, 4>());
    qload(NST - 1, qvp[NST - 1], svp[NST - 1]);
    qload(NST, qv, sv);
    dma(NST - 1, stage(std::integral_constant<int, NST - 1>()));
    // expand the first NST B tiles as their chunks arrive (operations issued after q(t):
    // A(t), [q(u), A(u)] for t < u < NST-1, q(NST-1), q(NST), A(NST-1))
    auto expand = [&](auto tc_) {
      constexpr int t = decltype(tc_)::value;
      if constexpr (t < NST - 1) {
        wait_vm<ADMA + (NST - 2 - t) * PS + 2 * QOPS + ADMA>();
        qstore(stage(std::integral_constant<int, t>()), qvp[t], svp[t]);
      } else if constexpr (t == NST - 1) {
        wait_vm<QOPS + ADMA>();
        qstore(stage(std::integral_constant<int, t>()), qvp[t], svp[t]);
      }
    };
    expand(std::integral_constant<int, 0>());
    expand(std::integral_constant<int, 1>());
    expand(std::integral_constant<int, 2>());
    expand(std::integral_constant<int, 3>());
    expand(std::integral_constant<int, 4>());
    expand(std::integral_constant<int, 5>());
  }
  // tile 0's A landed (operations issued after A(0): [q(u), A(u)] for 0 < u < NST-1, q(NST-1),
  // q(NST), A(NST-1)); every wave's expanded B tiles are written
  wait_vm_lds0<(NST - 2) * PS + 2 * QOPS + ADMA>();
  barrier();
  rd(st0, 0, 0);

  auto step = [&](int kt, auto sc) {
    constexpr int s = decltype(sc)::value;
    bf16_t* cur = stage(sc);
    const bf16_t* nxt = stage(std::integral_constant<int, (s + 1) % NST>());
#pragma unroll
    for (int ks = 0; ks + 1 < KS; ++ks) {
      rd(cur, ks + 1, (ks + 1) & 1);
      __builtin_amdgcn_sched_barrier(0);
      mm(ks & 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    wait_vm_lds0<PS * (NST - 2)>();  // tile kt+1's A landed; this wave's reads of tile kt retired
    barrier();
    rd(nxt, 0, 0);
    wait_vm<ADMA>();                 // tile kt+NST's int4 chunk and scale arrived
    qstore(cur, qv, sv);
    __builtin_amdgcn_sched_barrier(0);
    qload(kt + NST + 1, qv, sv);
    dma(kt + NST, cur);
    mm((KS - 1) & 1);
#pragma unroll
    for (int d = 0; d < PS; ++d) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // all groups but the last branch-free; the last stops after its last tile within K (as in
  // gemm_ilv_kernel)
  const int nreal = (K + BK - 1) / BK;
  for (int kt = 0; kt < nk - NST; kt += NST) {
    step(kt, std::integral_constant<int, 0>());
    step(kt + 1, std::integral_constant<int, 1>());
    if constexpr (NST > 2) step(kt + 2, std::integral_constant<int, 2>());
    if constexpr (NST > 3) step(kt + 3, std::integral_constant<int, 3>());
    if constexpr (NST > 4) step(kt + 4, std::integral_constant<int, 4>());
    if constexpr (NST > 5) step(kt + 5, std::integral_constant<int, 5>());
  }
  {
    const int kt = nk - NST;
    auto tail = [&](auto self, auto sc) -> void {
      constexpr int t = decltype(sc)::value;
      step(kt + t, sc);
      if constexpr (t + 1 < NST) {
        if (kt + t + 1 < nreal) self(self, std::integral_constant<int, t + 1>());
      }
    };
    tail(tail, std::integral_constant<int, 0>());
  }
  wait_vm_lds0<0>();  // the trailing zero-fill loads land before the stages are reused
  __syncthreads();

  wave_epilogue<EPI, OT, TM, TN, WTN, SR>(acc, reinterpret_cast<float*>(st0) + wv * SR * (WTN + 4),
                                          m0 + wm * TL::WTM, n0 + wn * TL::WTN, N, om, ep, pe_ld, lane);
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
    const int64_t off = om.off_row(row);
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
// NST = 0: gemm_dtl_kernel (one tile in flight); NST >= 2: gemm_ilv_kernel with NST stages.
template <typename T, class TL, class AS, class OM, int EPI, int TAG, int NST = 0, bool BQ = false>
hipError_t run(const AS& as, const T* Bw, int32_t N, int32_t K, const OM& om, const EpiP& ep,
               int64_t m_rows, int32_t pe_ld, hipStream_t s, BQuant bq = BQuant{nullptr, nullptr},
               int32_t splits = 1, int32_t k_span = 0, int32_t b_tiled = 0) {
  if constexpr (std::is_same<T, bf16_t>::value) {
    const int n_tiles = (N + TL::BN - 1) / TL::BN;
    const int64_t m_tiles = (m_rows + TL::BM - 1) / TL::BM;
    if (m_tiles * n_tiles == 0) return hipSuccess;
    if (m_tiles * n_tiles >= (int64_t(1) << 31)) return hipErrorInvalidValue;
    // every operand is addressed through 32-bit buffer offsets
    constexpr int64_t kMaxBytes = 0x7fffffff;
    if (as.bytes() > kMaxBytes || (int64_t)N * K * 2 > kMaxBytes || ep.c_bytes > kMaxBytes)
      return hipErrorInvalidValue;
    static_assert(!BQ || NST > 0, "int4 weights run in the staged kernel");
    if (splits < 1 || (splits > 1 && (NST == 0 || BQ || k_span <= 0 || (int64_t)(splits - 1) * k_span >= K)))
      return hipErrorInvalidValue;
    // a blocked weight layout (b_tiled = its K block) is read by the staged bf16 kernel with the
    // same BK only
    if (b_tiled != 0 && (NST == 0 || BQ || b_tiled != TL::BK || K % TL::BK != 0 || N % (512 / TL::BK) != 0))
      return hipErrorInvalidValue;
    if constexpr (BQ && NST > 0) {
      if (K % 128 != 0 || (int64_t)N * (K / 2) > kMaxBytes) return hipErrorInvalidValue;
      hipLaunchKernelGGL((gemm_ilvq_kernel<TL, NST, AS, OM, EPI, bf16_t, TAG>),
                         dim3((unsigned)(m_tiles * n_tiles)), dim3(TL::NT), 0, s, as, N, K, om, ep, n_tiles,
                         pe_ld, AE_GEMM_GROUP_M, bq);
    } else if constexpr (NST == 0)
      hipLaunchKernelGGL((gemm_dtl_kernel<TL, AS, OM, EPI, bf16_t, TAG>),
                         dim3((unsigned)(m_tiles * n_tiles)), dim3(TL::NT), 0, s, as, Bw, N, K, om, ep,
                         n_tiles, pe_ld, AE_GEMM_GROUP_M);
    else
      hipLaunchKernelGGL((gemm_ilv_kernel<TL, NST, AS, OM, EPI, bf16_t, TAG>),
                         dim3((unsigned)(m_tiles * n_tiles), (unsigned)splits), dim3(TL::NT), 0, s, as, Bw, N,
                         K, om, ep, n_tiles, pe_ld, AE_GEMM_GROUP_M, splits > 1 ? k_span : K, b_tiled);
  } else {
    if (b_tiled != 0) return hipErrorInvalidValue;
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

// Split-K finish: out = epilogue(sum over the S partial products + bias), the partials summed
// in K-range order (so the result does not depend on scheduling).  ws holds S slices of
// [M][N] fp32; each thread produces 4 consecutive output columns.
template <int EPI, typename OT>
__global__ __launch_bounds__(256) void splitk_finish_kernel(const float* __restrict__ ws, int32_t S, int64_t M,
                                                            int32_t N, const float* __restrict__ bias, void* C,
                                                            int64_t ldc, const float* __restrict__ pe,
                                                            const int32_t* __restrict__ tok_pos, int32_t pe_ld) {
  constexpr bool GATE = EPI == EPI_SWIGLU;
  const int32_t q4 = (GATE ? N / 2 : N) / 4;  // 4-column groups per output row
  const int64_t slice = M * N;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < M * q4; i += (int64_t)gridDim.x * 256) {
    const int64_t m = i / q4;
    const int o = (int)(i - m * q4) * 4;  // output column
    auto sum4 = [&](int col) {
      const float* p = ws + m * N + col;
      float4 a = *reinterpret_cast<const float4*>(p);
      for (int sp = 1; sp < S; ++sp) {
        const float4 b = *reinterpret_cast<const float4*>(p + sp * slice);
        a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w;
      }
      return a;
    };
    if constexpr (GATE) {
      // gate and up columns interleave in groups of 32 within each 64-column group
      const int gcol = (o / 32) * 64 + o % 32;
      const float4 g = sum4(gcol), u = sum4(gcol + 32);
      const uint2 v = make_uint2(pack_bf16x2(silu(g.x) * u.x, silu(g.y) * u.y), pack_bf16x2(silu(g.z) * u.z, silu(g.w) * u.w));
      *reinterpret_cast<uint2*>(reinterpret_cast<OT*>(C) + m * ldc + o) = v;
    } else {
      float4 x = sum4(o);
      float* cf = reinterpret_cast<float*>(C) + m * ldc + o;
      if constexpr (EPI == EPI_PE) {
        const float4 p = *reinterpret_cast<const float4*>(pe + (int64_t)tok_pos[m] * pe_ld + o);
        *reinterpret_cast<float4*>(cf) = make_float4(x.x + p.x, x.y + p.y, x.z + p.z, x.w + p.w);
      } else {
        if (bias) {
          const float4 b = *reinterpret_cast<const float4*>(bias + o);
          x.x += b.x; x.y += b.y; x.z += b.z; x.w += b.w;
        }
        if constexpr (EPI == EPI_RESADD) {
          const float4 r = *reinterpret_cast<const float4*>(cf);
          *reinterpret_cast<float4*>(cf) = make_float4(r.x + x.x, r.y + x.y, r.z + x.z, r.w + x.w);
        } else if constexpr (EPI == EPI_STORE_F32) {
          *reinterpret_cast<float4*>(cf) = x;
        } else {
          if constexpr (EPI == EPI_BIAS_GELU) {
            x.x = gelu_erf(x.x); x.y = gelu_erf(x.y); x.z = gelu_erf(x.z); x.w = gelu_erf(x.w);
          }
          *reinterpret_cast<uint2*>(reinterpret_cast<OT*>(C) + m * ldc + o) =
              make_uint2(pack_bf16x2(x.x, x.y), pack_bf16x2(x.z, x.w));
        }
      }
    }
  }
}

// Tile choice.  Candidates (the staged kernel unless noted):
//   Large  256x256, BK 64, 2 stages, one workgroup per CU
//   Tall   128x256, BK 64, 3 stages, one workgroup per CU
//   Narrow 128x128, BK 64, 2 stages, two workgroups per CU
//   Wide   256x128, BK 32, one-stage kernel, one workgroup per CU
//   Small  64x64, BK 64, 4 stages; SmallW 64x128, BK 64, 6 stages (calls with few rows)
// BK 64 moves 128-byte row pieces, a whole L2 request each (64-byte pieces reach about two
// thirds of the rate).  The kernel is chosen by its predicted time: rounds of tiles over the
// CUs times a per-tile cost proportional to the tile's area.  The constants (microseconds per
// 10^6 x tile area x K) are least-squares fits to measurements on MI355X over the tower's
// shapes at M = 6000 and 7281 (QKV, o-proj, FFN2, proj1/2, adapter); the rule picks the
// fastest kernel, or one within 2% of it, in every measured case.  A GELU epilogue is
// VALU-heavy and runs after the K loop, exposed when a CU has no other workgroup to overlap
// it: there a last round of Narrow that holds at most one workgroup per CU counts as half a
// round (measured: FFN1 at M = 6000 runs 83 us in Large against 94 us in Narrow, proj1 30 us
// in Narrow against 44 us in Large).
using TileWide = Tile<256, 128, 4, 2, 32, 1>;
using TileNarrow = Tile<128, 128, 2, 2, 64, 2>;
using TileLarge = Tile<256, 256, 2, 4, 64, 1>;
using TileTall = Tile<128, 256, 2, 4, 64, 1>;
using TileSmall = Tile<64, 64, 2, 2, 64, 1>;    // four waves of 32x32
using TileSmallW = Tile<64, 128, 2, 2, 64, 1>;  // four waves of 32x64
constexpr int kLargeStages = 2, kTallStages = 3, kNarrowStages = 2, kSmallStages = 4, kSmallWStages = 6;
enum class LinKind { Narrow, Wide, Large, Tall, Small, SmallW };

int cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cached[dev] <= 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

inline int64_t tile_count(int64_t M, int64_t N, int64_t bm, int64_t bn) {
  return ((M + bm - 1) / bm) * ((N + bn - 1) / bn);
}

inline LinKind lin_kind(int64_t M, int64_t N, bool gelu_epilogue, bool gate_epilogue) {
  const int64_t cus = cu_count();
  // Few rows (a single clip, a 64 s piece): the tiles below leave most CUs idle and each runs
  // its K loop at the latency of two stages.  Small tiles with deep stages spread the call over
  // the CUs; the first kind whose tiles fit one per CU wins (the gate epilogue needs 64-column
  // wave tiles).
  if (!gate_epilogue && tile_count(M, N, 64, 64) <= cus) return LinKind::Small;
  if (tile_count(M, N, 64, 128) <= cus) return LinKind::SmallW;
  auto cost = [&](int64_t bm, int64_t bn, int64_t per_cu, double us_per_mel) {
    const int64_t tiles = tile_count(M, N, bm, bn);
    const int64_t slots = per_cu * cus;
    double rounds = (double)((tiles + slots - 1) / slots);
    if (gelu_epilogue && per_cu == 2 && tiles % slots != 0 && tiles % slots <= cus) rounds -= 0.5;
    return rounds * us_per_mel * (double)(bm * bn);
  };
  const double large = cost(256, 256, 1, 0.393), tall = cost(128, 256, 1, 0.448);
  const double narrow = cost(128, 128, 2, 0.912), wide = cost(256, 128, 1, 0.502);
  LinKind k = LinKind::Large;
  double best = large;
  if (tall < best) { best = tall; k = LinKind::Tall; }
  if (narrow < best) { best = narrow; k = LinKind::Narrow; }
  if (wide < best) k = LinKind::Wide;
  return k;
}


// conv2/conv3 (N = 480 output channels, K = 9 * 480): 256x256 tiles, BK 32, four stages (the
// 480 channels fill two 256-wide column tiles at 94%).  Measured on MI355X against 256x256/BK 64
// with two stages, 128x256/BK 64 with three, and 128x128 with two workgroups per CU (BK 64 and
// BK 32): 13-35% slower for conv2.
using TileConv = Tile<256, 256, 2, 4, 32, 1>;
constexpr int kConvStages = 4;

template <typename T, int TAG, int EPI>
hipError_t lin(const LinearArgs& a, hipStream_t s) {
  ALinear<T> as{reinterpret_cast<const T*>(a.A), a.lda, a.M, a.K};
  OLinear om{a.M, a.ldc};
  constexpr bool f32out = EPI == EPI_RESADD || EPI == EPI_PE || EPI == EPI_STORE_F32;
  EpiP ep{a.bias, a.C, a.pe, a.tok_pos, a.M * a.ldc * (int64_t)(f32out ? 4 : sizeof(T))};
  const T* Bw = reinterpret_cast<const T*>(a.W);
  const int pe_ld = EPI == EPI_PE ? a.N : 0;
  if constexpr (std::is_same<T, bf16_t>::value) {
    if (a.Wq) {
      // int4 weights: the same tile choice as bf16, in the staged int4 kernel
      if (a.K % 128 != 0 || !a.Ws) return hipErrorInvalidValue;
      const BQuant bq{a.Wq, a.Ws};
      switch (lin_kind(a.M, a.N, EPI == EPI_BIAS_GELU, EPI == EPI_SWIGLU)) {
        case LinKind::Small:
          if constexpr (EPI != EPI_SWIGLU)
            return run<T, TileSmall, ALinear<T>, OLinear, EPI, TAG, kSmallStages, true>(as, Bw, a.N, a.K, om, ep,
                                                                                        a.M, pe_ld, s, bq);
          return hipErrorInvalidValue;
        case LinKind::SmallW:
          return run<T, TileSmallW, ALinear<T>, OLinear, EPI, TAG, kSmallWStages, true>(as, Bw, a.N, a.K, om, ep,
                                                                                        a.M, pe_ld, s, bq);
        case LinKind::Large:
          return run<T, TileLarge, ALinear<T>, OLinear, EPI, TAG, kLargeStages, true>(as, Bw, a.N, a.K, om, ep,
                                                                                      a.M, pe_ld, s, bq);
        case LinKind::Tall:
          return run<T, TileTall, ALinear<T>, OLinear, EPI, TAG, kTallStages, true>(as, Bw, a.N, a.K, om, ep,
                                                                                    a.M, pe_ld, s, bq);
        default:
          return run<T, TileNarrow, ALinear<T>, OLinear, EPI, TAG, kNarrowStages, true>(as, Bw, a.N, a.K, om, ep,
                                                                                        a.M, pe_ld, s, bq);
      }
    }
    // Split K when even the 128x128 tiles (two per CU) would leave more than half the CUs idle
    // (a single clip: M = 375) and K is long (FFN2, conv_out, the adapter's down projection;
    // for K = 1280 the small deep-stage tiles of the unsplit path are faster).  Each K range
    // writes an fp32 partial product into the scratch, and splitk_finish_kernel sums them in
    // order and applies the epilogue.
    if (a.ws && a.M > 0 && a.K >= 4096) {
      const int64_t cus = cu_count();
      const int64_t tiles = tile_count(a.M, a.N, 128, 128);
      const int64_t step = TileNarrow::BK * kNarrowStages;
      int64_t S = std::min<int64_t>({(2 * cus) / tiles, a.K / (2 * step), 16,
                                     a.ws_bytes / (a.M * a.N * 4)});
      if (2 * tiles <= cus && S >= 2 && a.N % (EPI == EPI_SWIGLU ? 64 : 4) == 0) {
        const int64_t k_span = ((a.K + S - 1) / S + step - 1) / step * step;
        S = (a.K + k_span - 1) / k_span;
        ALinear<T> as_p{reinterpret_cast<const T*>(a.A), a.lda, a.M, a.K};
        OLinear om_p{a.M, a.N};
        EpiP ep_p{nullptr, a.ws, nullptr, nullptr, S * a.M * a.N * 4, a.M * a.N};
        hipError_t err = run<T, TileNarrow, ALinear<T>, OLinear, EPI_STORE_F32, TAG, kNarrowStages>(
            as_p, Bw, a.N, a.K, om_p, ep_p, a.M, 0, s, BQuant{nullptr, nullptr}, (int32_t)S, (int32_t)k_span,
            a.b_tiled);
        if (err != hipSuccess) return err;
        const int64_t groups = a.M * ((EPI == EPI_SWIGLU ? a.N / 2 : a.N) / 4);
        const int64_t blocks = std::min<int64_t>((groups + 255) / 256, 16 * cus);
        hipLaunchKernelGGL((splitk_finish_kernel<EPI, bf16_t>), dim3((unsigned)blocks), dim3(256), 0, s, a.ws,
                           (int32_t)S, a.M, a.N, a.bias, a.C, a.ldc, a.pe, a.tok_pos, pe_ld);
        return hipGetLastError();
      }
    }
  } else {
    if (a.Wq) return hipErrorInvalidValue;
  }
  // the staged kernels read either weight layout; the one-stage Wide kernel only the plain one
  LinKind kind = lin_kind(a.M, a.N, EPI == EPI_BIAS_GELU, EPI == EPI_SWIGLU);
  if (kind == LinKind::Wide && a.b_tiled) kind = LinKind::Large;
  const BQuant nq{nullptr, nullptr};
  switch (kind) {
    case LinKind::Small:
      if constexpr (EPI != EPI_SWIGLU)
        return run<T, TileSmall, ALinear<T>, OLinear, EPI, TAG, kSmallStages>(as, Bw, a.N, a.K, om, ep, a.M, pe_ld, s,
                                                                              nq, 1, 0, a.b_tiled);
      return hipErrorInvalidValue;
    case LinKind::SmallW:
      return run<T, TileSmallW, ALinear<T>, OLinear, EPI, TAG, kSmallWStages>(as, Bw, a.N, a.K, om, ep, a.M, pe_ld, s,
                                                                              nq, 1, 0, a.b_tiled);
    case LinKind::Large:
      return run<T, TileLarge, ALinear<T>, OLinear, EPI, TAG, kLargeStages>(as, Bw, a.N, a.K, om, ep, a.M, pe_ld, s,
                                                                            nq, 1, 0, a.b_tiled);
    case LinKind::Tall:
      return run<T, TileTall, ALinear<T>, OLinear, EPI, TAG, kTallStages>(as, Bw, a.N, a.K, om, ep, a.M, pe_ld, s,
                                                                          nq, 1, 0, a.b_tiled);
    case LinKind::Wide:
      return run<T, TileWide, ALinear<T>, OLinear, EPI, TAG>(as, Bw, a.N, a.K, om, ep, a.M, pe_ld, s);
    default:
      return run<T, TileNarrow, ALinear<T>, OLinear, EPI, TAG, kNarrowStages>(as, Bw, a.N, a.K, om, ep, a.M, pe_ld, s,
                                                                              nq, 1, 0, a.b_tiled);
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

// Few conv rows (a single clip, a 64 s piece): 256x256 tiles would leave over half the CUs idle
// through a K loop of 135 steps.  128x128 (4 waves, 8 stages) or 128x256 (8 waves, 6 stages)
// tiles spread it over more CUs; the smaller tile is taken when its tiles fit one per CU.  K is
// accumulated in the same order, so rows do not depend on the tile.
using TileConvT = Tile<128, 256, 2, 4, 32, 1>;
using TileConvN = Tile<128, 128, 2, 2, 32, 1>;
constexpr int kConvTStages = 6, kConvNStages = 8;

template <typename T, class TL, int NST, int LEVEL, int TAG>
hipError_t conv_run(const AConv<T>& as, const T* wpk, int32_t C, const PassGeom& g, int rows_per_win,
                    int Fout, int Lout_max, int64_t m_rows, const EpiP& ep, hipStream_t s, int32_t w_tiled) {
  static_assert(TL::BK == 32, "the conv K order takes one (channel block, tap) pair per K step");
  // a wave covers TL::WTM rows of the tile
  if (rows_per_win >= TL::WTM) {
    OConv<LEVEL, true> om{g.wins, rows_per_win, Fout, C, Lout_max, m_rows};
    return run<T, TL, AConv<T>, OConv<LEVEL, true>, EPI_BIAS_GELU, TAG, NST>(
        as, wpk, C, 9 * C, om, ep, m_rows, 0, s, BQuant{nullptr, nullptr}, 1, 0, w_tiled);
  }
  OConv<LEVEL, false> om{g.wins, rows_per_win, Fout, C, Lout_max, m_rows};
  return run<T, TL, AConv<T>, OConv<LEVEL, false>, EPI_BIAS_GELU, TAG, NST>(
      as, wpk, C, 9 * C, om, ep, m_rows, 0, s, BQuant{nullptr, nullptr}, 1, 0, w_tiled);
}

template <typename T, int LEVEL, int TAG>
hipError_t conv_dispatch(const AConv<T>& as, const T* wpk, int32_t C, const PassGeom& g, int rows_per_win,
                         int Fout, int Lout_max, int64_t m_rows, const EpiP& ep, hipStream_t s, int32_t w_tiled) {
  const int64_t cus = cu_count();
  if (std::is_same<T, bf16_t>::value && 2 * tile_count(m_rows, C, 256, 256) < cus) {
    if (tile_count(m_rows, C, 128, 128) <= cus)
      return conv_run<T, TileConvN, kConvNStages, LEVEL, TAG>(as, wpk, C, g, rows_per_win, Fout, Lout_max,
                                                              m_rows, ep, s, w_tiled);
    return conv_run<T, TileConvT, kConvTStages, LEVEL, TAG>(as, wpk, C, g, rows_per_win, Fout, Lout_max,
                                                            m_rows, ep, s, w_tiled);
  }
  return conv_run<T, TileConv, kConvStages, LEVEL, TAG>(as, wpk, C, g, rows_per_win, Fout, Lout_max, m_rows,
                                                        ep, s, w_tiled);
}

template <typename T>
hipError_t launch_conv_igemm(const PassGeom& g, int level, const T* in, const T* wpk,
                             const float* bias, int32_t C, T* out, hipStream_t s, int32_t w_tiled) {
  const int Fin = level == 2 ? 64 : 32;
  const int Fout = Fin / 2;
  // the pass's time strides: act1 rows L1s, act2 rows L2s = ceil(L1s / 2); conv3 output rows
  // are token rows (each window's valid ones only)
  const int Lin_max = level == 2 ? g.L1s : g.L2s;
  const int Lout_max = (Lin_max + 1) / 2;
  if (g.L1s < 1 || g.L1s > 4 * g.W || g.L2s != (g.L1s + 1) / 2) return hipErrorInvalidValue;
  const int rows_per_win = Lout_max * Fout;
  const int64_t m_rows = (int64_t)g.n_win * rows_per_win;
  AConv<T> as{in, g.wins, C, Fin, Fout, Lin_max, level, rows_per_win, 9 * C, m_rows,
              (int64_t)g.n_win * Lin_max * Fin * C * (int64_t)sizeof(T), 1.0f / (float)C};
  if (m_rows >= (int64_t(1) << 31) || C > 65536) return hipErrorInvalidValue;
  const int64_t out_rows = level == 2 ? (int64_t)g.n_win * Lout_max * Fout : g.n_tok * Fout;
  EpiP ep{bias, out, nullptr, nullptr, out_rows * C * (int64_t)sizeof(T)};
  if (level == 2)
    return conv_dispatch<T, 2, ENC_K_CONV2>(as, wpk, C, g, rows_per_win, Fout, Lout_max, m_rows, ep, s, w_tiled);
  return conv_dispatch<T, 3, ENC_K_CONV3>(as, wpk, C, g, rows_per_win, Fout, Lout_max, m_rows, ep, s, w_tiled);
}

template hipError_t launch_linear<bf16_t>(const LinearArgs&, int, int, hipStream_t);
template hipError_t launch_linear<float>(const LinearArgs&, int, int, hipStream_t);
template hipError_t launch_conv_igemm<bf16_t>(const PassGeom&, int, const bf16_t*, const bf16_t*,
                                              const float*, int32_t, bf16_t*, hipStream_t, int32_t);
template hipError_t launch_conv_igemm<float>(const PassGeom&, int, const float*, const float*,
                                             const float*, int32_t, float*, hipStream_t, int32_t);

}  // namespace ae
