// cca_attn for bf16, d = 128: causal flash attention on the latent heads with
// MFMA (CCA-es §2.A "Principio Fundamental": attention run entirely in the
// compressed space; §2.C "CCGQA": query head h reads KV head h / G).
//
// Work-group = 4 waves = 128 query rows of one head; each wave owns 32 rows.
// K and V tiles of 64 keys are staged in LDS (next tile prefetched into
// registers while the current one is used).  Per tile and wave:
//   S^T = K Q^T   (v_mfma_f32_32x32x16_bf16; A = K rows from LDS, B = Q^T kept
//                  in registers).  The transposed product puts one query per
//                  lane, so the row max and row sum of the online softmax are
//                  in-lane reductions plus one exchange with lane ^ 32.
//   O^T += V^T P^T (A = V^T gathered from LDS, B = P^T straight from the S^T
//                  accumulators, rounded to bf16; no trip through LDS).
// Softmax runs in base 2 with log2(e)/sqrt(d) folded into the scale; fp32
// accumulators throughout; O is written as bf16 (and fp32 when asked) with
// the natural-log LSE.  Blocks with the most keys (largest query index) are
// scheduled first to even out the causal imbalance.
#include "cca_internal.h"

namespace cca {
namespace {

constexpr int D = 128;
constexpr int BM = 128;        // query rows per work-group
constexpr int BN = 64;         // keys per tile
constexpr int LDR = D + 8;     // LDS row stride (elements): 272 B, conflict-free b128 reads

struct KVRegs {
  bf16x8 k[4], v[4];
};

__device__ __forceinline__ void load_kv(const bf16* kb, const bf16* vb, int key0, int nkeys,
                                        KVRegs& r) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int f = t + 256 * i;
    const int row = f >> 4, ch = (f & 15) * 8;
    const int key = key0 + row;
    bf16x8 kk, vv;
    if (key < nkeys) {
      kk = *reinterpret_cast<const bf16x8*>(kb + (long)key * D + ch);
      vv = *reinterpret_cast<const bf16x8*>(vb + (long)key * D + ch);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) { kk[e] = (bf16)0.0f; vv[e] = (bf16)0.0f; }
    }
    r.k[i] = kk;
    r.v[i] = vv;
  }
}

__device__ __forceinline__ void store_kv(bf16* ks, bf16* vs, const KVRegs& r) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int f = t + 256 * i;
    const int row = f >> 4, ch = (f & 15) * 8;
    *reinterpret_cast<bf16x8*>(ks + row * LDR + ch) = r.k[i];
    *reinterpret_cast<bf16x8*>(vs + row * LDR + ch) = r.v[i];
  }
}

__global__ __launch_bounds__(256, 2) void attn_fwd_mfma_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) bf16 Ks[BN * LDR];
  __shared__ __attribute__((aligned(16))) bf16 Vs[BN * LDR];

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
  const bf16* vbase = reinterpret_cast<const bf16*>(a.v) + (long)b * a.kv_bs + (long)g * a.kv_hs;

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
  float m_run = -INFINITY, l_run = 0.0f;
  const float scale = 1.44269504088896340736f / sqrtf((float)D);

  const int q_last = min(S, q0 + BM) - 1;
  const int ntiles = q_last / BN + 1;
  KVRegs pre;
  load_kv(kbase, vbase, 0, S, pre);

  for (int kt = 0; kt < ntiles; ++kt) {
    __syncthreads();                       // previous tile fully consumed
    store_kv(Ks, Vs, pre);
    __syncthreads();
    if (kt + 1 < ntiles) load_kv(kbase, vbase, (kt + 1) * BN, S, pre);

    const int key0 = kt * BN;
    if (key0 > r0 + 31) continue;          // whole tile above this wave's diagonal

    // ---- S^T = K Q^T : two 32-key blocks
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.0f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const bf16x8 kf =
            *reinterpret_cast<const bf16x8*>(Ks + (kb * 32 + l32) * LDR + ks * 16 + hi * 8);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], sacc[kb], 0, 0, 0);
      }
    }

    // ---- online softmax for this lane's query
    const bool diag = key0 + BN - 1 > r0;
    float mt = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float s = sacc[kb][r] * scale;
        if (diag) {
          const int key = key0 + kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
          if (key > my_q) s = -INFINITY;
        }
        sacc[kb][r] = s;
        mt = fmaxf(mt, s);
      }
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float m_new = fmaxf(m_run, mt);
    const float alpha = exp2f(m_run - m_new);
    float ls = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = exp2f(sacc[kb][r] - m_new);
        sacc[kb][r] = p;
        ls += p;
      }
    ls += __shfl_xor(ls, 32);
    l_run = l_run * alpha + ls;
    m_run = m_new;
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
        bf16x8 vf;
        const int c = mb * 32 + l32;
#pragma unroll
        for (int s8 = 0; s8 < 8; ++s8) {
          const int key = ks * 16 + 8 * (s8 >> 2) + 4 * hi + (s8 & 3);
          vf[s8] = Vs[key * LDR + c];
        }
        oacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, oacc[mb], 0, 0, 0);
      }
    }
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
      a.lse[(long)(b * dm.Hq + h) * S + my_q] = (m_run + log2f(l_run)) * 0.69314718055994530942f;
  }
}

}  // namespace

bool attn_fwd_mfma_supported(const Dims& dm) { return dm.bf16 && dm.d == D; }

hipError_t launch_attn_fwd_mfma(const AttnArgs& a, hipStream_t s) {
  const int nqb = (a.Sq + BM - 1) / BM;
  dim3 grid(nqb * a.dm.Hq * a.B);
  hipLaunchKernelGGL(attn_fwd_mfma_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace cca
