// cca_mix for bf16, d = 128, on MFMA: the causal grouped convolution of q~ and
// k~ (CCA-es §2.B.1 "Mezcla Convolucional"), QK-mean (§2.B.2), value shift
// (§2.B.3) and RoPE (§3 item 2) in one pass per (128 tokens, KV group).
//
// The convolution of one head is a GEMM: out[t, c] = sum_{j, c'} u[t - j, c'] *
// A_j[c, c'] with M = tokens, N = channels, K = k * d.  Operand A (u) comes
// from the fp32 latent in two bf16 halves (hi = bf16(u), lo = bf16(u - hi)), so
// the product keeps ~16 mantissa bits of q~ and k~ with fp32 accumulation;
// operand B is the bf16 tap row A_j[c, 8 channels], read straight from L2.
// With lane = output channel and registers = tokens, every element a wave
// needs for QK-mean (the same token and channel of the group's G query heads
// and its K head) and for RoPE (channels c and c + d/2) sits in one lane.
//
// Wave w of the 4: tokens t0 + 64*(w/2) .. +63 (two 32-token blocks), channel
// blocks {w%2, w%2 + 2} (32 channels each: RoPE partners).
#include "cca_internal.h"

namespace cca {
namespace {

constexpr int D = 128;
constexpr int TW = 128;          // tokens per work-group

struct ConvAcc {
  f32x16 v[2][2];                // [token block][channel block]
};

__device__ __forceinline__ void zero(ConvAcc& a) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) a.v[i][j][r] = 0.0f;
}

// acc += conv of one head: u column `col` of the fp32 latent (row stride
// nqkv), taps [k][D][D] bf16.
__device__ __forceinline__ void conv_head(ConvAcc& acc, const float* qkv_b, int nqkv, int col,
                                          int S, int tw0, const bf16* taps, int k, int cb0,
                                          int lane) {
  const int l32 = lane & 31, hi = lane >> 5;
  for (int j = 0; j < k; ++j) {
#pragma unroll 2
    for (int ks = 0; ks < 8; ++ks) {
      bf16x8 ahi[2], alo[2], bt[2];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        const int t = tw0 + tb * 32 + l32 - j;
        f32x4 x0 = {0.f, 0.f, 0.f, 0.f}, x1 = {0.f, 0.f, 0.f, 0.f};
        if (t >= 0 && t < S) {
          const float* p = qkv_b + (long)t * nqkv + col + ks * 16 + hi * 8;
          x0 = *reinterpret_cast<const f32x4*>(p);
          x1 = *reinterpret_cast<const f32x4*>(p + 4);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bf16 h0 = (bf16)x0[e], h1 = (bf16)x1[e];
          ahi[tb][e] = h0;
          ahi[tb][e + 4] = h1;
          alo[tb][e] = (bf16)(x0[e] - (float)h0);
          alo[tb][e + 4] = (bf16)(x1[e] - (float)h1);
        }
      }
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const int c = (cb0 + 2 * cb) * 32 + l32;
        bt[cb] = *reinterpret_cast<const bf16x8*>(taps + ((long)j * D + c) * D + ks * 16 + hi * 8);
      }
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
          acc.v[tb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi[tb], bt[cb], acc.v[tb][cb], 0, 0, 0);
          acc.v[tb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo[tb], bt[cb], acc.v[tb][cb], 0, 0, 0);
        }
    }
  }
}

__global__ __launch_bounds__(256) void mix_fwd_mfma_kernel(MixArgs a) {
  // k^ of every wave, kept lane-private: element (tb, cb, r) of thread x at
  // kbuf[((tb * 2 + cb) * 16 + r) * 256 + x]
  __shared__ float kbuf[64 * 256];
  const Dims& dm = a.dm;
  const int G = dm.G, S = a.S;
  const int g = blockIdx.y, b = blockIdx.z;
  const int t0 = blockIdx.x * TW;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int tw0 = t0 + 64 * (wave >> 1);     // this wave's first token
  const int cb0 = wave & 1;                  // channel blocks cb0 and cb0 + 2
  const float* qkv_b = a.qkv + (long)b * S * dm.nqkv;
  const float A = (dm.flags & kQkPre) ? 0.5f : 0.0f;
  const float Bc = (dm.flags & kQkPost) ? 0.5f : 0.0f;
  const bool rope = (dm.flags & kRope) != 0;
  const int kcol = dm.nq + g * D;

  // token of register r in token block tb; channel of channel block cb
  auto tok = [&](int tb, int r) { return tw0 + tb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3); };
  const int c_lo = cb0 * 32 + l32;           // < 64: RoPE pair (c_lo, c_lo + 64)

  ConvAcc qacc, mpost;
  zero(qacc);
  conv_head(qacc, qkv_b, dm.nqkv, kcol, S, tw0,
            reinterpret_cast<const bf16*>(a.conv_k) + (long)g * dm.kk * D * D, dm.kk, cb0, lane);
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) kbuf[((tb * 2 + cb) * 16 + r) * 256 + threadIdx.x] = qacc.v[tb][cb][r];
  zero(mpost);

  for (int i = 0; i < G; ++i) {
    const int h = g * G + i;
    zero(qacc);
    conv_head(qacc, qkv_b, dm.nqkv, h * D, S, tw0,
              reinterpret_cast<const bf16*>(a.conv_q) + (long)h * dm.kq * D * D, dm.kq, cb0,
              lane);
    bf16* qo = reinterpret_cast<bf16*>(a.q_out) + ((long)(b * dm.Hq + h) * S) * D;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = tok(tb, r);
        if (t >= S) continue;
        float x[2];
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
          const int c = c_lo + 64 * cb;
          const float qh = qacc.v[tb][cb][r];
          const float kh = kbuf[((tb * 2 + cb) * 16 + r) * 256 + threadIdx.x];
          mpost.v[tb][cb][r] += qh;
          const float qp = qkv_b[(long)t * dm.nqkv + h * D + c];
          const float kp = qkv_b[(long)t * dm.nqkv + kcol + c];
          x[cb] = qh + A * (qp + kp) + Bc * (qh + kh);
        }
        float2 cs = make_float2(1.f, 0.f);
        if (rope) cs = a.rope[(long)t * (D / 2) + c_lo];
        qo[(long)t * D + c_lo] = (bf16)(x[0] * cs.x - x[1] * cs.y);
        qo[(long)t * D + c_lo + 64] = (bf16)(x[1] * cs.x + x[0] * cs.y);
        __builtin_amdgcn_sched_barrier(0);
      }
  }

  // k' = k^ + a/2 (mean_g q~ + k~) + b/2 (mean_g q^ + k^)
  const float invG = 1.0f / (float)G;
  bf16* ko = reinterpret_cast<bf16*>(a.k_out) + ((long)(b * dm.Hkv + g) * S) * D;
  bf16* ko2 = a.k_out2 ? reinterpret_cast<bf16*>(a.k_out2) + ((long)(b * dm.Hkv + g) * a.cap2) * D
                       : nullptr;
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int t = tok(tb, r);
      if (t >= S) continue;
      float x[2];
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const int c = c_lo + 64 * cb;
        float mpre = 0.0f;
        for (int i = 0; i < G; ++i) mpre += qkv_b[(long)t * dm.nqkv + (g * G + i) * D + c];
        const float kh = kbuf[((tb * 2 + cb) * 16 + r) * 256 + threadIdx.x];
        const float kp = qkv_b[(long)t * dm.nqkv + kcol + c];
        x[cb] = kh + A * (mpre * invG + kp) + Bc * (mpost.v[tb][cb][r] * invG + kh);
      }
      float2 cs = make_float2(1.f, 0.f);
      if (rope) cs = a.rope[(long)t * (D / 2) + c_lo];
      const bf16 lo = (bf16)(x[0] * cs.x - x[1] * cs.y);
      const bf16 hv = (bf16)(x[1] * cs.x + x[0] * cs.y);
      ko[(long)t * D + c_lo] = lo;
      ko[(long)t * D + c_lo + 64] = hv;
      if (ko2) {
        ko2[(long)t * D + c_lo] = lo;
        ko2[(long)t * D + c_lo + 64] = hv;
      }
      __builtin_amdgcn_sched_barrier(0);
    }

  // value shift.  Pass 1: the shifted V of these 128 tokens, read coalesced
  // from the fp32 latent, rounded to bf16 into an LDS tile (rows past S are
  // zero) and written in the standard layout when asked.  Pass 2: the tile is
  // written transposed, V'^T[c][t], which the MFMA attention reads.
  __syncthreads();                           // kbuf is free again
  constexpr int VLD = D + 8;
  bf16* vtile = reinterpret_cast<bf16*>(kbuf);   // [TW][VLD]
  const int vcol = dm.nq + dm.nk + g * D;
  bf16* vo = a.v_out ? reinterpret_cast<bf16*>(a.v_out) + ((long)(b * dm.Hkv + g) * S) * D
                     : nullptr;
  bf16* vo2 = a.v_out2 ? reinterpret_cast<bf16*>(a.v_out2) + ((long)(b * dm.Hkv + g) * a.cap2) * D
                       : nullptr;
  const int first_shift = (dm.flags & kVShift) ? D - dm.sv : D;
  for (int e = threadIdx.x; e < TW * D; e += 256) {
    const int tt = e / D, c = e % D;
    const int t = t0 + tt;
    float v = 0.0f;
    if (t < S) {
      if (c >= first_shift)
        v = t > 0 ? qkv_b[(long)(t - 1) * dm.nqkv + vcol + c] : 0.0f;
      else
        v = qkv_b[(long)t * dm.nqkv + vcol + c];
    }
    const bf16 vb = (bf16)v;
    vtile[tt * VLD + c] = vb;
    if (t < S) {
      if (vo) vo[(long)t * D + c] = vb;
      if (vo2) vo2[(long)t * D + c] = vb;
    }
  }
  if (a.vt_out) {
    __syncthreads();
    bf16* vt = reinterpret_cast<bf16*>(a.vt_out) + (long)(b * dm.Hkv + g) * D * a.s_pad;
    for (int e = threadIdx.x; e < D * (TW / 8); e += 256) {
      const int c = e / (TW / 8), m = e % (TW / 8);
      const int t = t0 + 8 * m;
      if (t >= a.s_pad) continue;
      bf16x8 pk;
#pragma unroll
      for (int i = 0; i < 8; ++i) pk[i] = vtile[(8 * m + i) * VLD + c];
      *reinterpret_cast<bf16x8*>(vt + (long)c * a.s_pad + t) = pk;
    }
  }
}

}  // namespace

bool mix_fwd_mfma_supported(const Dims& dm) { return dm.bf16 && dm.d == D; }

hipError_t launch_mix_fwd_mfma(const MixArgs& a, hipStream_t s) {
  dim3 grid((a.S + TW - 1) / TW, a.dm.Hkv, a.B);
  hipLaunchKernelGGL(mix_fwd_mfma_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace cca
