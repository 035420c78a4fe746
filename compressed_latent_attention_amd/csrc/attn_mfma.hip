// cca_attn for bf16, d = 128: causal flash attention on the latent heads with
// MFMA (CCA-es §2.A "Principio Fundamental": attention run entirely in the
// compressed space; §2.C "CCGQA": query head h reads KV head h / G).
//
// Work-group = 4 waves = 128 query rows of one head; each wave owns 32 rows.
// Tiles of 64 keys: K [key][c] and V^T [c][key] (the mix kernel writes V'
// transposed) are staged in LDS, double-buffered with one barrier per tile,
// the tile after next prefetched into registers meanwhile.  Per tile and wave:
//   S^T = K Q^T    v_mfma_f32_32x32x16_bf16 with A = K rows (LDS), B = Q^T kept
//                  in registers: one query per lane, so the online-softmax row
//                  max and row sum are in-lane plus one exchange with lane ^ 32;
//   O^T += V^T P^T A = V^T rows (LDS), B = P^T straight from the S^T
//                  accumulators rounded to bf16.  Within each 16-key group the
//                  V^T row is stored in the order {0-3, 8-11, 4-7, 12-15}, the
//                  order in which a lane holds P, so each A fragment is one
//                  16-byte LDS read.
// Softmax in base 2 with log2(e)/sqrt(d) folded into one FMA per score; fp32
// accumulators throughout.  Blocks with the most keys go first.
#include "cca_internal.h"

namespace cca {
namespace {

constexpr int D = 128;
constexpr int BM = 128;        // query rows per work-group
constexpr int BN = 64;         // keys per tile
constexpr int KLD = D + 8;     // K tile row stride (elements): 272 B
constexpr int VLD = BN + 8;    // V^T tile row stride (elements): 144 B
constexpr int KT_ELEMS = BN * KLD;
constexpr int VT_ELEMS = D * VLD;

struct TileRegs {
  bf16x8 k[4], v[4];
};

// K tile: 64 keys x 128 channels; V^T tile: 128 channels x 64 keys.
__device__ __forceinline__ void load_tile(const bf16* kb, const bf16* vtb, int s_pad, int key0,
                                          int nkeys, TileRegs& r) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int f = t + 256 * i;
    const int row = f >> 4, ch = (f & 15) * 8;      // K: key row, channel chunk
    const int key = key0 + row;
    if (key < nkeys) {
      r.k[i] = *reinterpret_cast<const bf16x8*>(kb + (long)key * D + ch);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) r.k[i][e] = (bf16)0.0f;
    }
    const int c = f >> 3, m = f & 7;                // V^T: channel row, 8-key chunk
    r.v[i] = *reinterpret_cast<const bf16x8*>(vtb + (long)c * s_pad + key0 + 8 * m);
  }
}

__device__ __forceinline__ void store_tile(bf16* ks, bf16* vs, const TileRegs& r) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int f = t + 256 * i;
    const int row = f >> 4, ch = (f & 15) * 8;
    *reinterpret_cast<bf16x8*>(ks + row * KLD + ch) = r.k[i];
    const int c = f >> 3, m = f & 7;
    // keys 8m..8m+3 -> 16*(m/2) + 4*(m%2); keys 8m+4..8m+7 -> 16*(m/2) + 8 + 4*(m%2)
    const int p0 = 16 * (m >> 1) + 4 * (m & 1);
    bf16x4 lo, hi;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      lo[e] = r.v[i][e];
      hi[e] = r.v[i][e + 4];
    }
    *reinterpret_cast<bf16x4*>(vs + c * VLD + p0) = lo;
    *reinterpret_cast<bf16x4*>(vs + c * VLD + p0 + 8) = hi;
  }
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_fwd_mfma_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) bf16 Ks[2][KT_ELEMS];
  __shared__ __attribute__((aligned(16))) bf16 Vs[2][VT_ELEMS];

  const Dims& dm = a.dm;
  const int S = a.Sq;
  const int nqb = (S + BM - 1) / BM;
  const int per_qb = dm.Hq * a.B;
  const int qb = nqb - 1 - (int)(blockIdx.x / per_qb);      // heaviest blocks first
  const int hb = blockIdx.x % per_qb;
  const int h = hb % dm.Hq, b = hb / dm.Hq;
  const int g = h / dm.G;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int q0 = qb * BM;
  const int r0 = q0 + wave * 32;             // first query row of this wave
  const int my_q = r0 + l32;                 // this lane's query row

  const bf16* qbase = reinterpret_cast<const bf16*>(a.q) + ((long)(b * dm.Hq + h) * S) * D;
  const bf16* kbase = reinterpret_cast<const bf16*>(a.k) + (long)b * a.kv_bs + (long)g * a.kv_hs;
  const bf16* vtbase =
      reinterpret_cast<const bf16*>(a.vt) + (long)(b * dm.Hkv + g) * D * a.s_pad;

  // Q^T fragments: lane holds query my_q, channels 16*ks + 8*hi + 0..7
  bf16x8 qf[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    if (my_q < S) {
      qf[ks] = *reinterpret_cast<const bf16x8*>(qbase + (long)my_q * D + ks * 16 + hi * 8);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[ks][e] = (bf16)0.0f;
    }
  }

  f32x16 oacc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[i][r] = 0.0f;
  float m_raw = -INFINITY, l_run = 0.0f;      // running max of raw scores, row sum
  const float scale = 1.44269504088896340736f / sqrtf((float)D);

  const int q_last = min(S, q0 + BM) - 1;
  const int ntiles = q_last / BN + 1;
  TileRegs pre;
  load_tile(kbase, vtbase, a.s_pad, 0, S, pre);
  store_tile(Ks[0], Vs[0], pre);
  if (ntiles > 1) load_tile(kbase, vtbase, a.s_pad, BN, S, pre);
  __syncthreads();

  for (int kt = 0; kt < ntiles; ++kt) {
    const int cur = kt & 1;
    const bf16* ks_ = Ks[cur];
    const bf16* vs_ = Vs[cur];
    const int key0 = kt * BN;
    if (key0 <= r0 + 31) {                   // else the tile is above this wave's diagonal
      // ---- S^T = K Q^T : two 32-key blocks
      f32x16 sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.0f;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          const bf16x8 kf =
              *reinterpret_cast<const bf16x8*>(ks_ + (kb * 32 + l32) * KLD + ks * 16 + hi * 8);
          sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], sacc[kb], 0, 0, 0);
        }
      }
      // ---- online softmax for this lane's query
      if (key0 + BN - 1 > r0) {              // diagonal tile: mask keys after the query
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = key0 + kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
            if (key > my_q) sacc[kb][r] = -INFINITY;
          }
      }
      float mt = m_raw;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sacc[kb][r]);
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      const float alpha = __builtin_amdgcn_exp2f((m_raw - mt) * scale);
      const float moff = -mt * scale;
      float ls = 0.0f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(fmaf(sacc[kb][r], scale, moff));
          sacc[kb][r] = p;
          ls += p;
        }
      ls += __shfl_xor(ls, 32);
      l_run = l_run * alpha + ls;
      m_raw = mt;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;

      // ---- O^T += V^T P^T : 4 k-steps of 16 keys, 4 blocks of 32 channels
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        bf16x8 pf;
#pragma unroll
        for (int s8 = 0; s8 < 8; ++s8) pf[s8] = (bf16)sacc[ks >> 1][8 * (ks & 1) + s8];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          const bf16x8 vf =
              *reinterpret_cast<const bf16x8*>(vs_ + (mb * 32 + l32) * VLD + ks * 16 + hi * 8);
          oacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, oacc[mb], 0, 0, 0);
        }
      }
    }
    if (kt + 1 < ntiles) {
      store_tile(Ks[cur ^ 1], Vs[cur ^ 1], pre);
      if (kt + 2 < ntiles) load_tile(kbase, vtbase, a.s_pad, (kt + 2) * BN, S, pre);
    }
    __syncthreads();
  }

  // ---- epilogue: lane holds query my_q, channels 32*mb + 8*(r/4) + 4*hi + r%4
  if (my_q < S) {
    const float inv = 1.0f / l_run;
    bf16* orow = reinterpret_cast<bf16*>(a.o) + ((long)(b * S + my_q) * dm.Hq + h) * D;
    float* orow32 = a.o32 ? a.o32 + ((long)(b * S + my_q) * dm.Hq + h) * D : nullptr;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = mb * 32 + 8 * j + 4 * hi;
        bf16x4 v4;
        f32x4 f4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          f4[i] = oacc[mb][4 * j + i] * inv;
          v4[i] = (bf16)f4[i];
        }
        *reinterpret_cast<bf16x4*>(orow + c) = v4;
        if (orow32) *reinterpret_cast<f32x4*>(orow32 + c) = f4;
      }
    if (hi == 0 && a.lse)
      a.lse[(long)(b * dm.Hq + h) * S + my_q] =
          (m_raw * scale + __builtin_amdgcn_logf(l_run)) * 0.69314718055994530942f;
  }
}

}  // namespace

hipError_t launch_attn_fwd_mfma(const AttnArgs& a, hipStream_t s) {
  if (a.dm.d != D || a.vt == nullptr || a.s_pad < a.Sq || a.s_pad % BN != 0)
    return hipErrorInvalidValue;
  const int nqb = (a.Sq + BM - 1) / BM;
  dim3 grid(nqb * a.dm.Hq * a.B);
  hipLaunchKernelGGL(attn_fwd_mfma_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace cca
