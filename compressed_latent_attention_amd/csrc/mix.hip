// cca_mix: the operations CCA applies to the compressed latents before
// attention (CCA-es §2.B "Innovaciones Clave"; CCA-fr §2 "Innovations Clés"):
//   1. causal grouped convolution of q~ and k~ along the sequence, mixing the
//      channels of each head (k taps of d x d, tap j on lag j),
//   2. QK-mean: adds the mean of Q and K before and after the convolution,
//   3. value shift: the last s_v channels of each KV head come from token t-1,
//   4. RoPE in the latent (CCA-es §3 item 2), rotate-half, angles from a
//      float64-built cos/sin table.
// Everything one KV group needs (its G query heads and its K head) is handled
// by one work-group, so QK-mean and RoPE need no cross-group traffic.
//
// This file holds the generic kernels (any even d <= 128, fp32 or bf16
// storage, fp32 arithmetic) and the decode-step mix; the MFMA prefill mix for
// bf16 lives in mix_mfma.hip.
#include "cca_internal.h"

#include <algorithm>

namespace cca {
namespace {

template <typename T>
__device__ __forceinline__ float ldf(const void* p, long i) {
  return (float)reinterpret_cast<const T*>(p)[i];
}
template <typename T>
__device__ __forceinline__ void stf(void* p, long i, float v) {
  reinterpret_cast<T*>(p)[i] = (T)v;
}
// Element i of the latent: fp32, or bf16 (the inference latent).
__device__ __forceinline__ float lat(const void* p, bool f32, long i) {
  return f32 ? reinterpret_cast<const float*>(p)[i] : (float)reinterpret_cast<const bf16*>(p)[i];
}

constexpr int TT = 4;   // tokens per work-group in the generic prefill mix

// QK-mean for one channel of one token, from the pre-conv (u) and post-conv
// (cv) values of the group's heads laid out [head][d] (q heads 0..G-1, then
// the k head at index G).  hh < G gives q'_hh, hh == G gives k'.
__device__ __forceinline__ float qk_mixed(const float* u, const float* cv, int G, int d, int hh,
                                          int ch, uint32_t flags) {
  const float a = (flags & kQkPre) ? 0.5f : 0.0f;
  const float b = (flags & kQkPost) ? 0.5f : 0.0f;
  const float pre_k = u[G * d + ch], post_k = cv[G * d + ch];
  if (hh < G) {
    const float pre_q = u[hh * d + ch], post_q = cv[hh * d + ch];
    return post_q + a * (pre_q + pre_k) + b * (post_q + post_k);
  }
  float mpre = 0.0f, mpost = 0.0f;
  for (int i = 0; i < G; ++i) {
    mpre += u[i * d + ch];
    mpost += cv[i * d + ch];
  }
  mpre /= (float)G;
  mpost /= (float)G;
  return post_k + a * (mpre + pre_k) + b * (mpost + post_k);
}

__device__ __forceinline__ float rope_rot(float x, float partner, int c, int half, float2 cs) {
  // (lo, hi) -> (lo cos - hi sin, hi cos + lo sin)
  return c < half ? x * cs.x - partner * cs.y : x * cs.x + partner * cs.y;
}

template <typename T>
__global__ __launch_bounds__(256) void mix_fwd_simple(MixArgs a) {
  extern __shared__ float smem[];
  const Dims& dm = a.dm;
  const int d = dm.d, G = dm.G, NH = G + 1;
  const int KM = max(dm.kq, dm.kk);
  const int g = blockIdx.y, b = blockIdx.z;
  const int t0 = blockIdx.x * TT;
  float* u = smem;                                  // [TT+KM-1][NH][d]
  float* cv = smem + (TT + KM - 1) * NH * d;        // [TT][NH][d]
  const int rows = TT + KM - 1;
  for (int i = threadIdx.x; i < rows * NH * d; i += blockDim.x) {
    const int r = i / (NH * d), hh = (i / d) % NH, c = i % d;
    const int t = t0 - (KM - 1) + r;
    const int col = hh < G ? (g * G + hh) * d : dm.nq + g * d;
    u[i] = (t >= 0 && t < a.S) ? lat(a.qkv, a.qkv_f32, (long)(b * a.S + t) * dm.nqkv + col + c)
                               : 0.0f;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < TT * NH * d; i += blockDim.x) {
    const int tt = i / (NH * d), hh = (i / d) % NH, c = i % d;
    const bool isq = hh < G;
    const int k = isq ? dm.kq : dm.kk;
    const long tap0 = isq ? (long)(g * G + hh) * dm.kq * d * d : (long)g * dm.kk * d * d;
    const void* taps = isq ? a.conv_q : a.conv_k;
    float s = 0.0f;
    for (int j = 0; j < k; ++j) {
      const float* src = u + ((tt + KM - 1 - j) * NH + hh) * d;
      const long base = tap0 + ((long)j * d + c) * d;
      for (int e = 0; e < d; ++e) s += ldf<T>(taps, base + e) * src[e];
    }
    cv[i] = s;
  }
  __syncthreads();
  const int half = d / 2;
  for (int i = threadIdx.x; i < TT * d; i += blockDim.x) {
    const int tt = i / d, c = i % d;
    const int t = t0 + tt;
    if (t >= a.S) continue;
    const float* ut = u + (tt + KM - 1) * NH * d;
    const float* ct = cv + tt * NH * d;
    const int cp = c < half ? c + half : c - half;
    const float2 cs = (dm.flags & kRope) ? a.rope[(long)t * half + (c % half)] : make_float2(1.f, 0.f);
    for (int hh = 0; hh < NH; ++hh) {
      const float x = qk_mixed(ut, ct, G, d, hh, c, dm.flags);
      const float xp = qk_mixed(ut, ct, G, d, hh, cp, dm.flags);
      const float r = rope_rot(x, xp, c, half, cs);
      if (hh < G) {
        stf<T>(a.q_out, ((long)(b * dm.Hq + g * G + hh) * a.S + t) * d + c, r);
      } else {
        stf<T>(a.k_out, ((long)(b * dm.Hkv + g) * a.S + t) * d + c, r);
        if (a.k_out2) stf<T>(a.k_out2, ((long)(b * dm.Hkv + g) * a.cap2 + t) * d + c, r);
      }
    }
    const bool shifted = (dm.flags & kVShift) && c >= d - dm.sv;
    const long vcol = dm.nq + dm.nk + g * d + c;
    float v;
    if (shifted)
      v = t > 0 ? lat(a.qkv, a.qkv_f32, (long)(b * a.S + t - 1) * dm.nqkv + vcol) : 0.0f;
    else
      v = lat(a.qkv, a.qkv_f32, (long)(b * a.S + t) * dm.nqkv + vcol);
    stf<T>(a.v_out, ((long)(b * dm.Hkv + g) * a.S + t) * d + c, v);
    if (a.v_out2) stf<T>(a.v_out2, ((long)(b * dm.Hkv + g) * a.cap2 + t) * d + c, v);
  }
}

template <typename T>
__global__ __launch_bounds__(256) void write_state_kernel(Dims dm, int S, const void* qkv,
                                                          bool qkv_f32, void* state) {
  const int b = blockIdx.x;
  const int nqpart = (dm.kq - 1) * dm.nq, nkpart = (dm.kk - 1) * dm.nk;
  for (int i = threadIdx.x; i < dm.state_w; i += blockDim.x) {
    int lag, col;
    if (i < nqpart) {
      lag = i / dm.nq + 1;
      col = i % dm.nq;
    } else if (i < nqpart + nkpart) {
      lag = (i - nqpart) / dm.nk + 1;
      col = dm.nq + (i - nqpart) % dm.nk;
    } else {
      lag = 1;
      col = dm.nq + dm.nk + (i - nqpart - nkpart);
    }
    const int t = S - lag;
    const float v = t >= 0 ? lat(qkv, qkv_f32, (long)(b * S + t) * dm.nqkv + col) : 0.0f;
    stf<T>(state, (long)b * dm.state_w + i, v);
  }
}

// Decode-step mix, part 1: the causal grouped convolution of the new token of
// every sequence, for every query and key head: cv[b, hg, c] =
// sum_j sum_c' u_j[b, hg, c'] A_{hg, j}[c, c'], where u_0 is the token's
// latent (qkv) and u_j (j >= 1) the lag-j latent from the rolling state; hg
// runs over the query heads, then the key heads.  Work-group = one head x CB
// output channels x BC sequences: its tap rows go to LDS (fp32, rows padded by
// 4 so the 16 lanes that read 16 different rows hit different banks), then the
// lags of its sequences; thread = one (sequence, channel) dot product over
// k * d inputs, 4 at a time.  The staging loads use clamped indices (a
// duplicate load is stored nowhere), so they issue back to back.
constexpr int CB = 16;                  // output channels per work-group
constexpr int BCMAX = 16;               // sequences per work-group (256 threads / CB)

template <typename T>
__global__ __launch_bounds__(256) void mix_decode_conv_kernel(MixDecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) float smem[];
  const Dims& dm = a.dm;
  const int d = dm.d, TS = d + 4;       // tap row stride (floats)
  const int hg = blockIdx.x, c0 = blockIdx.y * CB, b0 = blockIdx.z * BCMAX;
  const int nb = min(BCMAX, a.B - b0);
  const bool isq = hg < dm.Hq;
  const int k = isq ? dm.kq : dm.kk;
  const int nqpart = (dm.kq - 1) * dm.nq;
  float* tap = smem;                    // [k][CB][TS]
  float* u = smem + k * CB * TS;        // [BCMAX][k][d]
  const T* taps = reinterpret_cast<const T*>(isq ? a.conv_q : a.conv_k) +
                  (long)(isq ? hg : hg - dm.Hq) * k * d * d;
  const int col0 = isq ? hg * d : dm.nq + (hg - dm.Hq) * d;   // column in qkv and in the state
  const int t = threadIdx.x;
  constexpr int EV = 16 / sizeof(T);    // tap elements per 16-byte load
  if (d % EV == 0) {
    // tap rows (rows past d read row d - 1 and store zeros)
    const int dv = d / EV, nvec = k * CB * dv;
    for (int base = 0; base < nvec; base += 2 * 256) {
      T v[2][EV];
      int dst[2];
      bool ok[2];
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int i = base + r * 256 + t, ic = min(i, nvec - 1);
        const int j = ic / (CB * dv), cl = (ic / dv) % CB, e = (ic % dv) * EV;
        dst[r] = i < nvec ? (j * CB + cl) * TS + e : -1;
        ok[r] = c0 + cl < d;
        *reinterpret_cast<f32x4*>(v[r]) = *reinterpret_cast<const f32x4*>(
            taps + ((long)j * d + min(c0 + cl, d - 1)) * d + e);
      }
#pragma unroll
      for (int r = 0; r < 2; ++r)
        if (dst[r] >= 0)
#pragma unroll
          for (int q = 0; q < EV; ++q) tap[dst[r] + q] = ok[r] ? (float)v[r][q] : 0.0f;
    }
  } else {
    for (int i = t; i < k * CB * d; i += blockDim.x) {
      const int j = i / (CB * d), cl = (i / d) % CB, e = i % d;
      tap[(j * CB + cl) * TS + e] =
          c0 + cl < d ? (float)taps[((long)j * d + c0 + cl) * d + e] : 0.0f;
    }
  }
  if (d % 4 == 0) {
    // lag 0 from qkv, 4 channels per load
    const int n0 = nb * (d / 4);
    for (int base = 0; base < n0; base += 2 * 256) {
      f32x4 v[2];
      int dst[2];
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int i = base + r * 256 + t, ic = min(i, n0 - 1);
        const int bb = ic / (d / 4), e = (ic % (d / 4)) * 4;
        dst[r] = i < n0 ? bb * k * d + e : -1;
        v[r] = *reinterpret_cast<const f32x4*>(a.qkv + (long)(b0 + bb) * dm.nqkv + col0 + e);
      }
#pragma unroll
      for (int r = 0; r < 2; ++r)
        if (dst[r] >= 0) *reinterpret_cast<f32x4*>(u + dst[r]) = v[r];
    }
    // lags 1 .. k - 1 from the state
    const int nl = nb * (k - 1) * (d / 4);
    for (int base = 0; base < nl; base += 2 * 256) {
      float v[2][4];
      int dst[2];
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int i = base + r * 256 + t, ic = min(i, nl - 1);
        const int e = (ic % (d / 4)) * 4, j = 1 + (ic / (d / 4)) % (k - 1),
                  bb = ic / ((k - 1) * (d / 4));
        dst[r] = i < nl ? (bb * k + j) * d + e : -1;
        const long srow = (long)(b0 + bb) * dm.state_w;
        const long off = isq ? srow + (long)(j - 1) * dm.nq + col0 + e
                             : srow + nqpart + (long)(j - 1) * dm.nk + (col0 - dm.nq) + e;
#pragma unroll
        for (int q = 0; q < 4; ++q) v[r][q] = ldf<T>(a.state, off + q);
      }
#pragma unroll
      for (int r = 0; r < 2; ++r)
        if (dst[r] >= 0)
#pragma unroll
          for (int q = 0; q < 4; ++q) u[dst[r] + q] = v[r][q];
    }
  } else {
    for (int i = t; i < nb * k * d; i += blockDim.x) {
      const int bb = i / (k * d), j = (i / d) % k, e = i % d;
      const int b = b0 + bb;
      float v;
      if (j == 0) {
        v = a.qkv[(long)b * dm.nqkv + col0 + e];
      } else {
        const long srow = (long)b * dm.state_w;
        v = isq ? ldf<T>(a.state, srow + (long)(j - 1) * dm.nq + col0 + e)
                : ldf<T>(a.state, srow + nqpart + (long)(j - 1) * dm.nk + (col0 - dm.nq) + e);
      }
      u[i] = v;
    }
  }
  __syncthreads();
  const int cl = t % CB, o = t / CB;
  if (o >= nb || c0 + cl >= d) return;
  float s0 = 0.0f, s1 = 0.0f;
  for (int j = 0; j < k; ++j) {
    const float* ur = u + (o * k + j) * d;
    const float* tr = tap + (j * CB + cl) * TS;
    if (d % 8 == 0) {
#pragma unroll 4
      for (int e = 0; e < d; e += 8) {
        const f32x4 x0 = *reinterpret_cast<const f32x4*>(ur + e);
        const f32x4 w0 = *reinterpret_cast<const f32x4*>(tr + e);
        const f32x4 x1 = *reinterpret_cast<const f32x4*>(ur + e + 4);
        const f32x4 w1 = *reinterpret_cast<const f32x4*>(tr + e + 4);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          s0 = fmaf(w0[q], x0[q], s0);
          s1 = fmaf(w1[q], x1[q], s1);
        }
      }
    } else {
      for (int e = 0; e < d; ++e) s0 = fmaf(tr[e], ur[e], s0);
    }
  }
  a.cv[((long)(b0 + o) * (dm.Hq + dm.Hkv) + hg) * d + c0 + cl] = s0 + s1;
}

// Decode-step mix, part 2: one token per sequence at position pos[b].  From
// the convolution outputs cv and the pre-convolution latents (lag 0 from qkv,
// the lags of the state) it forms QK-mean, RoPE, the value shift, writes q and
// the caches, and advances the rolling state in place.  One work-group per (KV
// group, sequence).
template <typename T>
__global__ __launch_bounds__(256) void mix_decode_kernel(MixDecodeArgs a) {
  extern __shared__ float smem[];
  const Dims& dm = a.dm;
  const int d = dm.d, G = dm.G, NH = G + 1;
  const int KM = max(dm.kq, dm.kk);
  const int g = blockIdx.x, b = blockIdx.y;
  const int p = a.pos.p[b];
  float* u = smem;                       // [KM][NH][d]  lag j = row j
  float* cv = u + KM * NH * d;           // [NH][d]
  float* vprev = cv + NH * d;            // [d]
  const long srow = (long)b * dm.state_w;
  const int nqpart = (dm.kq - 1) * dm.nq, nkpart = (dm.kk - 1) * dm.nk;
#pragma unroll 4
  for (int i = threadIdx.x; i < KM * NH * d; i += blockDim.x) {
    const int j = i / (NH * d), hh = (i / d) % NH, c = i % d;
    const bool isq = hh < G;
    float v = 0.0f;
    if (j == 0) {
      const int col = isq ? (g * G + hh) * d : dm.nq + g * d;
      v = a.qkv[(long)b * dm.nqkv + col + c];
    } else if (isq && j < dm.kq) {
      v = ldf<T>(a.state, srow + (long)(j - 1) * dm.nq + (g * G + hh) * d + c);
    } else if (!isq && j < dm.kk) {
      v = ldf<T>(a.state, srow + nqpart + (long)(j - 1) * dm.nk + g * d + c);
    }
    u[i] = v;
  }
#pragma unroll 4
  for (int i = threadIdx.x; i < NH * d; i += blockDim.x) {
    const int hh = i / d, c = i % d;
    const int hgl = hh < G ? g * G + hh : dm.Hq + g;
    cv[i] = a.cv[((long)b * (dm.Hq + dm.Hkv) + hgl) * d + c];
  }
  for (int c = threadIdx.x; c < d; c += blockDim.x)
    vprev[c] = ldf<T>(a.state, srow + nqpart + nkpart + g * d + c);
  __syncthreads();
  const int half = d / 2;
  for (int c = threadIdx.x; c < d; c += blockDim.x) {
    const int cp = c < half ? c + half : c - half;
    const float2 cs = (dm.flags & kRope) ? a.rope[(long)p * half + (c % half)] : make_float2(1.f, 0.f);
    for (int hh = 0; hh < NH; ++hh) {
      const float x = qk_mixed(u, cv, G, d, hh, c, dm.flags);
      const float xp = qk_mixed(u, cv, G, d, hh, cp, dm.flags);
      const float r = rope_rot(x, xp, c, half, cs);
      if (hh < G)
        stf<T>(a.q_out, (long)(b * dm.Hq + g * G + hh) * d + c, r);
      else
        stf<T>(a.k_cache, ((long)(b * dm.Hkv + g) * dm.max_seq_len + p) * d + c, r);
    }
    const bool shifted = (dm.flags & kVShift) && c >= d - dm.sv;
    const float vnew = a.qkv[(long)b * dm.nqkv + dm.nq + dm.nk + g * d + c];
    stf<T>(a.v_cache, ((long)(b * dm.Hkv + g) * dm.max_seq_len + p) * d + c,
           shifted ? vprev[c] : vnew);
  }
  // advance the state: the new token becomes lag 1 (every read above is done)
  for (int i = threadIdx.x; i < NH * d; i += blockDim.x) {
    const int hh = i / d, c = i % d;
    const bool isq = hh < G;
    const int k = isq ? dm.kq : dm.kk;
    for (int j = 1; j < k; ++j) {
      const float v = u[((j - 1) * NH + hh) * d + c];
      if (isq)
        stf<T>(a.state, srow + (long)(j - 1) * dm.nq + (g * G + hh) * d + c, v);
      else
        stf<T>(a.state, srow + nqpart + (long)(j - 1) * dm.nk + g * d + c, v);
    }
  }
  for (int c = threadIdx.x; c < d; c += blockDim.x)
    stf<T>(a.state, srow + nqpart + nkpart + g * d + c,
           a.qkv[(long)b * dm.nqkv + dm.nq + dm.nk + g * d + c]);
}

// Sum over each row of 16 lanes, left in every lane of the row: DPP swap of
// neighbours, of pairs, mirror within 8, mirror within 16.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
// The same over rows of 8 lanes (neighbours, pairs, mirror within 8).
__device__ __forceinline__ float row8_sum(float v) {
  v += dpp_mov<0xB1>(v);    // quad_perm [1, 0, 3, 2]
  v += dpp_mov<0x4E>(v);    // quad_perm [2, 3, 0, 1]
  v += dpp_mov<0x141>(v);   // row_half_mirror
  return v;
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_mov<0xB1>(v);    // quad_perm [1, 0, 3, 2]
  v += dpp_mov<0x4E>(v);    // quad_perm [2, 3, 0, 1]
  v += dpp_mov<0x141>(v);   // row_half_mirror
  v += dpp_mov<0x140>(v);   // row_mirror
  return v;
}

// Decode-step mix in one kernel (bf16 storage, d = 128 or 64, at most 4 taps):
// one work-group of 1024 threads per (KV group g, sequence b) does what the
// two kernels above do for that group, with the token's latents summed from
// the projection's K-slice partials as they are read.  The step is a chain of
// tiny dependent phases, so every global read is issued at the start, in one
// round: the K-slice partials, the state's lags and previous v, the RoPE pairs
// of position p, and the tap rows of each wave's first 12 convolution groups.
//   1. lag 0 of the G query heads, the key head and the new v (sums of the
//      partials), the lags >= 1 and the previous v to LDS;
//   2. convolution: a group = the 1024 / 2d consecutive output channels of
//      one (head, tap) pair whose tap rows make 1 KB: one 16-byte load per
//      lane (lane = row slot L / (d / 8), input channels 8 (L % (d / 8)) ..
//      + 7), partial dot products with the lag-j latent from LDS, summed over
//      the d / 8 lanes of a row by DPP;
//   3. the taps' terms summed per (head, channel), then QK-mean, RoPE, value
//      shift, the q / cache stores and the advanced state as above.
// The group's state is read in 1. and written in 3. by this work-group only.
constexpr int FKMAX = 4;                // taps per convolution at most
constexpr int FNH = kMaxGroup + 1;      // heads of a KV group: G query heads + 1 key head
constexpr int FZ = 8;                   // K-slice partials read in the first round

template <int FD>
__global__ __launch_bounds__(1024) void mix_decode_fused_kernel(MixDecodeArgs a) {
  constexpr int LPR = FD / 8;             // lanes per tap row
  constexpr int GCH = 64 / LPR;           // output channels (tap rows) per group
  constexpr int GPP = FD / GCH;           // groups per (head, tap) pair
  __shared__ __attribute__((aligned(16))) float u[FKMAX][FNH][FD];     // pre-conv latents by lag
  __shared__ __attribute__((aligned(16))) float cvp[FKMAX][FNH][FD];   // convolution terms by tap
  __shared__ __attribute__((aligned(16))) float cv[FNH][FD];           // convolution outputs
  __shared__ __attribute__((aligned(16))) float vnew[FD];
  __shared__ __attribute__((aligned(16))) float vprev[FD];
  __shared__ float2 rope_cs[FD / 2];
  const Dims& dm = a.dm;
  const int G = dm.G, NH = G + 1, kq = dm.kq, kk = dm.kk, KM = max(kq, kk);
  const int g = blockIdx.x, b = blockIdx.y, p = a.pos.p[b];
  // the wave index in a scalar register: group indices, (head, tap) pairs and
  // the choice of tap tensor are then uniform, with no per-lane pointer select
  const int t = threadIdx.x, lane = t & 63, wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int slot = lane / LPR, ci = (lane % LPR) * 8;
  const long srow = (long)b * dm.state_w;
  const int nqpart = (kq - 1) * dm.nq, nkpart = (kk - 1) * dm.nk;
  const bf16* st = reinterpret_cast<const bf16*>(a.state);
  const int half = FD / 2;
  const int nr = G * kq + kk, ngroups = nr * GPP;
  // integer division by run-time values expands to long scalar sequences that
  // every wave would issue; the divisors here are small: k <= 4 as
  // r * ceil(65536 / k) >> 16 (exact for r < 4096), NH <= 9 through a float
  // reciprocal ((r + 0.5) / NH stays >= 0.5 / NH away from an integer)
  const int mkq = (65536 + kq - 1) / kq;
  auto div_kq = [&](int r) { return (r * mkq) >> 16; };
  const float inv_nh = 1.0f / (float)NH;
  auto div_nh = [&](int r) { return (int)(((float)r + 0.5f) * inv_nh); };
  auto pair_of = [&](int r, int& hh, int& j) {      // (head, tap) pair r (r < 36)
    const int qh = div_kq(r);
    hh = r < G * kq ? qh : G;
    j = r < G * kq ? r - qh * kq : r - G * kq;
  };
  // tap matrix of pair r: conv_q matrix g G kq + r for r < G kq (pairs run
  // head-major, tap-minor), else conv_k matrix g kk + r - G kq; the tensor is
  // chosen by a byte offset, not a pointer select
  const char* tq = reinterpret_cast<const char*>(a.conv_q);
  const long dqk = reinterpret_cast<const char*>(a.conv_k) - tq;
  const int GK = G * kq;
  auto tap_load = [&](int q) {                      // this lane's 16 bytes of group q
    const int r = q / GPP, c = (q % GPP) * GCH + slot;
    const long mat = r < GK ? (long)g * GK + r : (long)g * kk + (r - GK);
    const char* row = tq + (r < GK ? 0 : dqk) + ((mat * FD + c) * FD + ci) * 2;
    return *reinterpret_cast<const bf16x8*>(row);
  };

  // ---- every global read, one round (clamped indices: a duplicate read is stored nowhere)
  constexpr int NB = 12;                            // groups per wave per round (192 = 16 x 12)
  bf16x8 w[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) w[i] = tap_load(min(wave + 16 * i, ngroups - 1));
  // lag 0: row hh (query heads, key head, then v) x 4 channels per thread
  const int n0 = (NH + 1) * (FD / 4);
  const int t0 = min(t, n0 - 1), hh0 = t0 / (FD / 4), c0 = (t0 % (FD / 4)) * 4;
  const int col0 = hh0 < G ? (g * G + hh0) * FD : hh0 == G ? dm.nq + g * FD : dm.nq + dm.nk + g * FD;
  const float* src0 = a.qkv + (long)b * a.qkv_ld + col0 + c0;
  f32x4 part0[FZ];
#pragma unroll
  for (int z = 0; z < FZ; ++z)
    part0[z] = *reinterpret_cast<const f32x4*>(src0 + (long)min(z, a.qkv_ks - 1) * a.qkv_kstride);
  // lags 1 .. k - 1 (item = lag, head, 8 channels), then the previous v
  const int nl = (KM - 1) * NH * (FD / 8);
  const int e1 = min(t, nl + FD / 8 - 1), cl = (e1 % (FD / 8)) * 8, rl = e1 / (FD / 8);
  const int rq = div_nh(rl), hl = rl - rq * NH, jl = 1 + rq;
  const bool lag_ok = t < nl && jl < (hl < G ? kq : kk);
  const long offl = !lag_ok ? srow + nqpart + nkpart + g * FD + cl
                  : hl < G ? srow + (long)(jl - 1) * dm.nq + (g * G + hl) * FD + cl
                           : srow + nqpart + (long)(jl - 1) * dm.nk + g * FD + cl;
  const bf16x8 lagv = *reinterpret_cast<const bf16x8*>(st + offl);
  // RoPE pairs of position p
  const float2 csv = (dm.flags & kRope) ? a.rope[(long)p * half + min(t, half - 1)] : make_float2(1.f, 0.f);

  // ---- 1. to LDS
  if (t < n0) {
    f32x4 sum = part0[0];
#pragma unroll
    for (int z = 1; z < FZ; ++z)
      if (z < a.qkv_ks) sum += part0[z];
    for (int z = FZ; z < a.qkv_ks; ++z)               // more slices than the first round took
      sum += *reinterpret_cast<const f32x4*>(src0 + (long)z * a.qkv_kstride);
    *reinterpret_cast<f32x4*>(hh0 <= G ? &u[0][hh0][c0] : &vnew[c0]) = sum;
  }
  if (lag_ok || (t >= nl && t < nl + FD / 8)) {
    float* dst = lag_ok ? &u[jl][hl][cl] : &vprev[cl];
#pragma unroll
    for (int q = 0; q < 8; ++q) dst[q] = (float)lagv[q];
  }
  if (t < half) rope_cs[t] = csv;
  __syncthreads();

  // ---- 2. convolution terms: wave takes groups wave + 16 i
  for (int q0 = wave; q0 < ngroups; q0 += 16 * NB) {
    if (q0 != wave) {                                  // groups past the first round's
#pragma unroll
      for (int i = 0; i < NB; ++i) w[i] = tap_load(min(q0 + 16 * i, ngroups - 1));
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int q = q0 + 16 * i;
      if (q >= ngroups) break;                         // uniform over the wave
      int hh, j;
      pair_of(q / GPP, hh, j);
      const f32x4 x0 = *reinterpret_cast<const f32x4*>(&u[j][hh][ci]);
      const f32x4 x1 = *reinterpret_cast<const f32x4*>(&u[j][hh][ci + 4]);
      float sum = 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sum = fmaf((float)w[i][e], x0[e], sum);
        sum = fmaf((float)w[i][4 + e], x1[e], sum);
      }
      // every lane of the row holds the sum: all of them store it (same address, same value)
      cvp[j][hh][(q % GPP) * GCH + slot] = LPR == 16 ? row16_sum(sum) : row8_sum(sum);
    }
  }
  __syncthreads();
  for (int e = t; e < NH * FD; e += 1024) {
    const int hh = e / FD, c = e % FD, k = hh < G ? kq : kk;
    float sum = cvp[0][hh][c];
    for (int j = 1; j < k; ++j) sum += cvp[j][hh][c];
    cv[hh][c] = sum;
  }
  __syncthreads();

  // ---- 3. QK-mean and RoPE: item = (head, channel), up to 9 x 128 of them
  for (int e = t; e < NH * FD; e += 1024) {
    const int hh = e / FD, c = e % FD, cp = c < half ? c + half : c - half;
    const float x = qk_mixed(&u[0][0][0], &cv[0][0], G, FD, hh, c, dm.flags);
    const float xp = qk_mixed(&u[0][0][0], &cv[0][0], G, FD, hh, cp, dm.flags);
    const float r = rope_rot(x, xp, c, half, rope_cs[c % half]);
    if (hh < G)
      stf<bf16>(a.q_out, (long)(b * dm.Hq + g * G + hh) * FD + c, r);
    else
      stf<bf16>(a.k_cache, ((long)(b * dm.Hkv + g) * dm.max_seq_len + p) * FD + c, r);
  }
  // value shift, the v cache row and the v of the state
  if (t < FD) {
    const bool shifted = (dm.flags & kVShift) && t >= FD - dm.sv;
    stf<bf16>(a.v_cache, ((long)(b * dm.Hkv + g) * dm.max_seq_len + p) * FD + t,
              shifted ? vprev[t] : vnew[t]);
    stf<bf16>(a.state, srow + nqpart + nkpart + g * FD + t, vnew[t]);
  }
  // the rolling state advances: lag j takes lag j - 1 (item = head x 8 channels of one lag)
  for (int j = 1; j < KM; ++j)
    for (int e = t; e < NH * (FD / 8); e += 1024) {
      const int hh = e / (FD / 8), c = (e % (FD / 8)) * 8;
      const bool isq = hh < G;
      if (j >= (isq ? kq : kk)) continue;
      const long off = isq ? srow + (long)(j - 1) * dm.nq + (g * G + hh) * FD + c
                           : srow + nqpart + (long)(j - 1) * dm.nk + g * FD + c;
      bf16x8 v;
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = (bf16)u[j - 1][hh][c + q];
      *reinterpret_cast<bf16x8*>(reinterpret_cast<bf16*>(a.state) + off) = v;
    }
}

}  // namespace

hipError_t launch_mix_fwd_mfma(const MixArgs& a, hipStream_t s);          // mix_mfma.hip
hipError_t launch_mix_fwd_mfma_f32lat(const MixArgs& a, hipStream_t s);   // mix_mfma_f32lat.hip
bool mix_fwd_mfma_supported(const Dims& dm);

bool prefill_uses_mfma(const Dims& dm) { return dm.bf16 && mix_fwd_mfma_supported(dm); }

hipError_t launch_mix_fwd(const MixArgs& a, hipStream_t s) {
  const Dims& dm = a.dm;
  if (prefill_uses_mfma(dm))
    return a.qkv_f32 ? launch_mix_fwd_mfma_f32lat(a, s) : launch_mix_fwd_mfma(a, s);
  const int KM = max(dm.kq, dm.kk);
  const size_t lds = (size_t)((TT + KM - 1) + TT) * (dm.G + 1) * dm.d * sizeof(float);
  dim3 grid((a.S + TT - 1) / TT, dm.Hkv, a.B);
  if (dm.bf16)
    hipLaunchKernelGGL(mix_fwd_simple<bf16>, grid, dim3(256), lds, s, a);
  else
    hipLaunchKernelGGL(mix_fwd_simple<float>, grid, dim3(256), lds, s, a);
  return hipGetLastError();
}

hipError_t launch_write_state(const Dims& dm, int B, int S, const void* qkv, bool qkv_f32,
                              void* state, hipStream_t s) {
  if (dm.bf16)
    hipLaunchKernelGGL(write_state_kernel<bf16>, dim3(B), dim3(256), 0, s, dm, S, qkv, qkv_f32,
                       state);
  else
    hipLaunchKernelGGL(write_state_kernel<float>, dim3(B), dim3(256), 0, s, dm, S, qkv, qkv_f32,
                       state);
  return hipGetLastError();
}

size_t mix_decode_cv_floats(const Dims& dm, int B) { return (size_t)B * (dm.Hq + dm.Hkv) * dm.d; }

bool mix_decode_fused_ok(const Dims& dm) {
  return dm.bf16 && (dm.d == 128 || dm.d == 64) && dm.G <= kMaxGroup && dm.kq >= 1 &&
         dm.kq <= FKMAX && dm.kk >= 1 && dm.kk <= FKMAX;
}

hipError_t launch_mix_decode(const MixDecodeArgs& a, hipStream_t s) {
  const Dims& dm = a.dm;
  if (a.qkv_ks < 1 || a.qkv_ld < dm.nqkv) return hipErrorInvalidValue;
  if (mix_decode_fused_ok(dm)) {
    if (dm.d == 128)
      hipLaunchKernelGGL(mix_decode_fused_kernel<128>, dim3(dm.Hkv, a.B), dim3(1024), 0, s, a);
    else
      hipLaunchKernelGGL(mix_decode_fused_kernel<64>, dim3(dm.Hkv, a.B), dim3(1024), 0, s, a);
    return hipGetLastError();
  }
  if (a.cv == nullptr || a.qkv_ks != 1 || a.qkv_ld != dm.nqkv) return hipErrorInvalidValue;
  // part 1: LDS = k CB (d + 4) tap floats + BCMAX k d lag floats
  const int k = max(dm.kq, dm.kk);
  const size_t lds1 = ((size_t)k * CB * (dm.d + 4) + (size_t)BCMAX * k * dm.d) * sizeof(float);
  if (lds1 > 64 * 1024) return hipErrorInvalidValue;
  dim3 grid1(dm.Hq + dm.Hkv, (dm.d + CB - 1) / CB, (a.B + BCMAX - 1) / BCMAX);
  if (dm.bf16)
    hipLaunchKernelGGL(mix_decode_conv_kernel<bf16>, grid1, dim3(256), lds1, s, a);
  else
    hipLaunchKernelGGL(mix_decode_conv_kernel<float>, grid1, dim3(256), lds1, s, a);
  // part 2
  const int KM = max(dm.kq, dm.kk);
  const size_t lds = (size_t)((KM + 1) * (dm.G + 1) * dm.d + dm.d) * sizeof(float);
  dim3 grid(dm.Hkv, a.B);
  if (dm.bf16)
    hipLaunchKernelGGL(mix_decode_kernel<bf16>, grid, dim3(256), lds, s, a);
  else
    hipLaunchKernelGGL(mix_decode_kernel<float>, grid, dim3(256), lds, s, a);
  return hipGetLastError();
}

}  // namespace cca
