// Projection GEMMs of the CCA layer (cca_proj): the down-projection of x to
// the latent q~ | k~ | v~ (CCA-es §2.A "Principio Fundamental"; CCA-fr §2
// "Projection vers l'Espace Latent"), the output projection O W_o^T, and the
// GEMMs of the backward pass.
//
// bf16 path: 128x128x32 work-group tiles, 4 waves of 64x64, each wave a 2x2
// block of v_mfma_f32_32x32x16_bf16, operands staged k-contiguous in LDS with
// double buffering.  fp32 path: a plain LDS-tiled VALU kernel.
#include "cca_internal.h"

namespace cca {
namespace {

__device__ __forceinline__ int seg_of(int r, const int* start, int nseg) {
  int s = 0;
  if (nseg > 1 && r >= start[1]) s = 1;
  if (nseg > 2 && r >= start[2]) s = 2;
  return s;
}

template <typename T>
__device__ __forceinline__ const T* b_row(const GemmArgs& g, int r) {
  int s = seg_of(r, g.b_start, g.b_nseg);
  return reinterpret_cast<const T*>(g.b_ptr[s]) + (long)(r - g.b_start[s]) * g.ldb;
}

template <typename OutT>
__device__ __forceinline__ OutT* c_row(const GemmArgs& g, int m) {
  int s = seg_of(m, g.c_start, g.c_nseg);
  return reinterpret_cast<OutT*>(g.c_ptr[s]) + (long)(m - g.c_start[s]) * g.ldc;
}

__device__ __forceinline__ void store_out(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_out(bf16* p, float v) { *p = (bf16)v; }

// ------------------------------------------------------------ bf16 MFMA GEMM
constexpr int BM = 128, BN = 128, BK = 32, LDK = BK + 8;   // LDS row stride 80 B

// Loads one BK slice of an operand tile (rows = m or n, 128 of them) into
// registers: 2 chunks of 8 bf16 per thread.  kc: operand is k-contiguous in
// global memory; otherwise the row index is contiguous.
struct TileRegs {
  bf16x8 v[2];
};

template <bool KC, bool IS_B>
__device__ __forceinline__ void load_tile(const GemmArgs& g, int row0, int k0, int rows_total,
                                          TileRegs& r) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = t + 256 * i;
    bf16x8 val;
#pragma unroll
    for (int e = 0; e < 8; ++e) val[e] = (bf16)0.0f;
    if (KC) {
      const int row = c >> 2, kc = (c & 3) * 8;
      const int gr = row0 + row, gk = k0 + kc;
      if (gr < rows_total && gk < g.K) {
        const bf16* p = IS_B ? b_row<bf16>(g, gr) + gk
                             : reinterpret_cast<const bf16*>(g.a) + (long)gr * g.lda + gk;
        val = *reinterpret_cast<const bf16x8*>(p);
      }
    } else {
      const int kk = c >> 4, rc = (c & 15) * 8;
      const int gk = k0 + kk, gr = row0 + rc;
      if (gk < g.K && gr < rows_total) {
        const bf16* p = IS_B ? b_row<bf16>(g, gk) + gr
                             : reinterpret_cast<const bf16*>(g.a) + (long)gk * g.lda + gr;
        val = *reinterpret_cast<const bf16x8*>(p);
      }
    }
    r.v[i] = val;
  }
}

template <bool KC>
__device__ __forceinline__ void store_tile(bf16* lds, const TileRegs& r) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = t + 256 * i;
    if (KC) {
      const int row = c >> 2, kc = (c & 3) * 8;
      *reinterpret_cast<bf16x8*>(lds + row * LDK + kc) = r.v[i];
    } else {
      const int kk = c >> 4, rc = (c & 15) * 8;
#pragma unroll
      for (int e = 0; e < 8; ++e) lds[(rc + e) * LDK + kk] = r.v[i][e];
    }
  }
}

template <bool A_KC, bool B_KC, typename OutT>
__global__ __launch_bounds__(256) void gemm_bf16_mfma(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) bf16 As[2][BM * LDK];
  __shared__ __attribute__((aligned(16))) bf16 Bs[2][BN * LDK];

  const int tiles_m = (g.M + BM - 1) / BM;
  const int tiles_n = (g.N + BN - 1) / BN;
  // grouped raster: 8 row-tiles share a column sweep, for L2 reuse of B
  const int bid = blockIdx.x;
  const int group = 8;
  const int per_group = group * tiles_n;
  const int gid = bid / per_group;
  const int first_m = gid * group;
  const int gsize = min(group, tiles_m - first_m);
  const int tm = first_m + (bid % per_group) % gsize;
  const int tn = (bid % per_group) / gsize;
  const int m0 = tm * BM, n0 = tn * BN;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int nk = (g.K + BK - 1) / BK;
  TileRegs ra, rb;
  load_tile<A_KC, false>(g, m0, 0, g.M, ra);
  load_tile<B_KC, true>(g, n0, 0, g.N, rb);
  store_tile<A_KC>(As[0], ra);
  store_tile<B_KC>(Bs[0], rb);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) {
      load_tile<A_KC, false>(g, m0, (kt + 1) * BK, g.M, ra);
      load_tile<B_KC, true>(g, n0, (kt + 1) * BK, g.N, rb);
    }
    const bf16* as = As[cur];
    const bf16* bs = Bs[cur];
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        af[i] = *reinterpret_cast<const bf16x8*>(
            as + (wm * 64 + i * 32 + (lane & 31)) * LDK + ks * 16 + 8 * (lane >> 5));
        bfr[i] = *reinterpret_cast<const bf16x8*>(
            bs + (wn * 64 + i * 32 + (lane & 31)) * LDK + ks * 16 + 8 * (lane >> 5));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) {
      store_tile<A_KC>(As[cur ^ 1], ra);
      store_tile<B_KC>(Bs[cur ^ 1], rb);
    }
    __syncthreads();
  }

  // D layout of 32x32 MFMA: lane holds column lane%32, rows 8*(r/4)+4*(lane/32)+r%4
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + wn * 64 + j * 32 + (lane & 31);
      if (n >= g.N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (m < g.M) store_out(c_row<OutT>(g, m) + n, acc[i][j][r]);
      }
    }
}

// ------------------------------------------------------------ fp32 VALU GEMM
template <typename T>
__device__ __forceinline__ float ld_a(const GemmArgs& g, int m, int k, bool kc) {
  if (m >= g.M || k >= g.K) return 0.0f;
  const T* a = reinterpret_cast<const T*>(g.a);
  return (float)(kc ? a[(long)m * g.lda + k] : a[(long)k * g.lda + m]);
}

template <typename T>
__device__ __forceinline__ float ld_b(const GemmArgs& g, int k, int n, bool kc) {
  if (n >= g.N || k >= g.K) return 0.0f;
  return (float)(kc ? b_row<T>(g, n)[k] : b_row<T>(g, k)[n]);
}

template <typename T, typename OutT, bool A_KC, bool B_KC>
__global__ __launch_bounds__(256) void gemm_simple(GemmArgs g) {
  constexpr int TM = 64, TN = 64, TK = 16;
  __shared__ float As[TK][TM + 1];
  __shared__ float Bs[TK][TN + 1];
  const int tiles_n = (g.N + TN - 1) / TN;
  const int m0 = (blockIdx.x / tiles_n) * TM, n0 = (blockIdx.x % tiles_n) * TN;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < g.K; k0 += TK) {
    for (int i = threadIdx.x; i < TK * TM; i += 256) {
      const int kk = i / TM, mm = i % TM;
      As[kk][mm] = ld_a<T>(g, m0 + mm, k0 + kk, A_KC);
      Bs[kk][mm] = ld_b<T>(g, k0 + kk, n0 + mm, B_KC);
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < TK; ++kk) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        av[i] = As[kk][ty * 4 + i];
        bv[i] = Bs[kk][tx * 4 + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] += av[i] * bv[j];
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= g.M) continue;
    OutT* crow = c_row<OutT>(g, m);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n < g.N) store_out(crow + n, acc[i][j]);
    }
  }
}

template <bool A_KC, bool B_KC>
hipError_t launch_layout(const GemmArgs& g, bool in_bf16, bool out_f32, hipStream_t s) {
  if (in_bf16) {
    const int tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
    if (out_f32)
      hipLaunchKernelGGL((gemm_bf16_mfma<A_KC, B_KC, float>), dim3(tiles), dim3(256), 0, s, g);
    else
      hipLaunchKernelGGL((gemm_bf16_mfma<A_KC, B_KC, bf16>), dim3(tiles), dim3(256), 0, s, g);
  } else {
    const int tiles = ((g.M + 63) / 64) * ((g.N + 63) / 64);
    hipLaunchKernelGGL((gemm_simple<float, float, A_KC, B_KC>), dim3(tiles), dim3(256), 0, s, g);
  }
  return hipGetLastError();
}

}  // namespace

bool launch_gemm_nt_small(const GemmArgs& g, bool out_f32, hipStream_t s, hipError_t* err);

hipError_t launch_gemm(const GemmArgs& g, GemmLayout layout, bool in_bf16, bool out_f32,
                       hipStream_t s) {
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  hipError_t err = hipSuccess;
  if (layout == GemmLayout::NT && in_bf16 &&
      (launch_gemm_nt_big(g, out_f32, s, &err) || launch_gemm_nt_small(g, out_f32, s, &err)))
    return err;
  switch (layout) {
    case GemmLayout::NT: return launch_layout<true, true>(g, in_bf16, out_f32, s);
    case GemmLayout::NN: return launch_layout<true, false>(g, in_bf16, out_f32, s);
    case GemmLayout::TN: return launch_layout<false, false>(g, in_bf16, out_f32, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace cca
