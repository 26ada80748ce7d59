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
  __device__ bool tile_live(int64_t m0) const { return m0 < M; }
  __device__ Row row(int64_t r) const { return Row{r < M ? A + r * lda : nullptr}; }
  __device__ KC kc(int k) const { return KC{k, k < K}; }
  __device__ const T* ptr(const Row& x, const KC& c) const {
    return (x.p && c.ok) ? x.p + c.k : nullptr;
  }
};

// im2col view for a 3x3 stride-2 pad-1 conv: output row r of window w covers
// (t_out, f_out) = (loc / Fout, loc % Fout) with loc = r - w * rows_per_win.
template <typename T>
struct AConv {
  const T* in;
  const Win* wins;
  int32_t C, Fin, Fout, Lin_max, level, rows_per_win, K;
  struct Row { const T* base; int t2, f2, Lin; };
  struct KC { int ci, da, db; bool ok; };
  __device__ bool tile_live(int64_t m0) const {
    const int w = (int)(m0 / rows_per_win);
    const int loc = (int)(m0 - (int64_t)w * rows_per_win);
    const Win wn = wins[w];
    return loc / Fout < (level == 2 ? wn.L2 : wn.L3);
  }
  __device__ Row row(int64_t r) const {
    const int w = (int)(r / rows_per_win);
    const int loc = (int)(r - (int64_t)w * rows_per_win);
    const int t = loc / Fout, f = loc - (loc / Fout) * Fout;
    const Win wn = wins[w];
    Row x;
    if (t >= (level == 2 ? wn.L2 : wn.L3)) { x.base = nullptr; x.t2 = x.f2 = x.Lin = 0; return x; }
    x.base = in + (int64_t)w * Lin_max * Fin * C;
    x.t2 = 2 * t - 1;
    x.f2 = 2 * f - 1;
    x.Lin = level == 2 ? wn.L1 : wn.L2;
    return x;
  }
  __device__ KC kc(int k) const {
    KC c;
    c.ok = k < K;
    const int tap = k / C;
    c.ci = k - tap * C;
    c.da = tap / 3;          // frequency tap
    c.db = tap - 3 * c.da;   // time tap
    return c;
  }
  __device__ const T* ptr(const Row& x, const KC& c) const {
    if (!x.base || !c.ok) return nullptr;
    const int t = x.t2 + c.db, f = x.f2 + c.da;
    if (t < 0 || t >= x.Lin || f < 0 || f >= Fin) return nullptr;
    return x.base + ((int64_t)t * Fin + f) * C + c.ci;
  }
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
  __device__ int64_t off(int64_t r) const {
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
constexpr int BM = 128, BN = 128, BK = 64, NTHR = 256;

__device__ inline uint4 ld16(const bf16_t* p) {
  return p ? *reinterpret_cast<const uint4*>(p) : make_uint4(0u, 0u, 0u, 0u);
}

// TAG only names the call site (one kernel symbol per role, so profiles separate them)
template <class AS, class OM, int EPI, typename OT, int TAG>
__global__ __launch_bounds__(NTHR) void gemm_bf16_kernel(AS as, const bf16_t* __restrict__ Bw,
                                                         int32_t N, int32_t K, OM om, EpiP ep,
                                                         int32_t n_tiles, int32_t pe_ld) {
  __shared__ __attribute__((aligned(16))) bf16_t sA[2][BM * BK];
  __shared__ __attribute__((aligned(16))) bf16_t sB[2][BN * BK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int wm = wv >> 1, wn = wv & 1;
  const int64_t mt = blockIdx.x / n_tiles;
  const int nt = blockIdx.x - (int)(mt * n_tiles);
  const int64_t m0 = mt * BM;
  const int n0 = nt * BN;
  if (!as.tile_live(m0)) return;

  // loader mapping: 16-byte chunk c of rows lr + 32*i
  const int c = tid & 7;
  const int lr = tid >> 3;
  typename AS::Row arow[4];
  const bf16_t* brow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    arow[i] = as.row(m0 + lr + 32 * i);
    const int n = n0 + lr + 32 * i;
    brow[i] = n < N ? Bw + (int64_t)n * K : nullptr;
  }
  uint4 ra[4], rb[4];
  auto gload = [&](int kt) {
    const int k = kt * BK + c * 8;
    const auto kc = as.kc(k);
    const bool kok = k < K;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[i] = ld16(as.ptr(arow[i], kc));
      rb[i] = ld16((brow[i] && kok) ? brow[i] + k : nullptr);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = lr + 32 * i;
      const int pc = c ^ (r & 7);
      *reinterpret_cast<uint4*>(&sA[buf][r * BK + pc * 8]) = ra[i];
      *reinterpret_cast<uint4*>(&sB[buf][r * BK + pc * 8]) = rb[i];
    }
  };

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int nk = (K + BK - 1) / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8_t af[2], bfr[2];
      const int ch = ks * 2 + (lane >> 5);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = wm * 64 + i * 32 + (lane & 31);
        af[i] = *reinterpret_cast<const bf16x8_t*>(&sA[cur][r * BK + ((ch ^ (r & 7)) * 8)]);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = wn * 64 + j * 32 + (lane & 31);
        bfr[j] = *reinterpret_cast<const bf16x8_t*>(&sB[cur][r * BK + ((ch ^ (r & 7)) * 8)]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) sstore(cur ^ 1);
    __syncthreads();
  }

  // epilogue: element v of a 32x32 block sits at row 8*(v/4) + 4*(lane/32) + v%4, col lane%32
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int64_t row = m0 + wm * 64 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
      const int64_t off = om.off(row);
      if (off < 0) continue;
      if constexpr (EPI == EPI_SWIGLU) {
        if (n0 + wn * 64 >= N) continue;  // this wave's gate|up column pair lies past N
        const int col = (n0 + wn * 64) / 2 + (lane & 31);
        const float g = acc[i][0][v], u = acc[i][1][v];
        StoreT<OT>::put(reinterpret_cast<OT*>(ep.C) + off + col, silu(g) * u);
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int col = n0 + wn * 64 + j * 32 + (lane & 31);
          if (col >= N) continue;
          if constexpr (EPI == EPI_PE) {
            reinterpret_cast<float*>(ep.C)[off + col] =
                acc[i][j][v] + ep.pe[(int64_t)ep.tok_pos[row] * pe_ld + col];
          } else {
            epi_store<EPI, OT>(ep, off, row, col, acc[i][j][v]);
          }
        }
      }
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
  if (!as.tile_live(m0)) return;

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
template <typename T, class AS, class OM, int EPI, int TAG>
hipError_t run(const AS& as, const T* Bw, int32_t N, int32_t K, const OM& om, const EpiP& ep,
               int64_t m_rows, int32_t pe_ld, hipStream_t s) {
  if constexpr (std::is_same<T, bf16_t>::value) {
    const int n_tiles = (N + BN - 1) / BN;
    const int64_t m_tiles = (m_rows + BM - 1) / BM;
    if (m_tiles * n_tiles == 0) return hipSuccess;
    hipLaunchKernelGGL((gemm_bf16_kernel<AS, OM, EPI, bf16_t, TAG>), dim3((unsigned)(m_tiles * n_tiles)),
                       dim3(NTHR), 0, s, as, Bw, N, K, om, ep, n_tiles, pe_ld);
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

template <typename T, int TAG, int EPI>
hipError_t lin(const LinearArgs& a, hipStream_t s) {
  ALinear<T> as{reinterpret_cast<const T*>(a.A), a.lda, a.M, a.K};
  OLinear om{a.M, a.ldc};
  EpiP ep{a.bias, a.C, a.pe, a.tok_pos};
  return run<T, ALinear<T>, OLinear, EPI, TAG>(as, reinterpret_cast<const T*>(a.W), a.N, a.K, om,
                                               ep, a.M, EPI == EPI_PE ? a.N : 0, s);
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
  constexpr int TM = std::is_same<T, bf16_t>::value ? BM : FBM;
  const int Fin = level == 2 ? 64 : 32;
  const int Fout = Fin / 2;
  const int Lin_max = level == 2 ? 4 * g.W : 2 * g.W;
  const int Lout_max = Lin_max / 2;
  const int rows = Lout_max * Fout;
  const int rows_per_win = ((rows + TM - 1) / TM) * TM;
  AConv<T> as{in, g.wins, C, Fin, Fout, Lin_max, level, rows_per_win, 9 * C};
  OConv om{g.wins, rows_per_win, Fout, C, level, Lout_max};
  EpiP ep{bias, out, nullptr, nullptr};
  const int64_t m_rows = (int64_t)g.n_win * rows_per_win;
  if (level == 2)
    return run<T, AConv<T>, OConv, EPI_BIAS_GELU, ENC_K_CONV2>(as, wpk, C, 9 * C, om, ep, m_rows, 0, s);
  return run<T, AConv<T>, OConv, EPI_BIAS_GELU, ENC_K_CONV3>(as, wpk, C, 9 * C, om, ep, m_rows, 0, s);
}

template hipError_t launch_linear<bf16_t>(const LinearArgs&, int, int, hipStream_t);
template hipError_t launch_linear<float>(const LinearArgs&, int, int, hipStream_t);
template hipError_t launch_conv_igemm<bf16_t>(const PassGeom&, int, const bf16_t*, const bf16_t*,
                                              const float*, int32_t, bf16_t*, hipStream_t);
template hipError_t launch_conv_igemm<float>(const PassGeom&, int, const float*, const float*,
                                             const float*, int32_t, float*, hipStream_t);

}  // namespace ae
