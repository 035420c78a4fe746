// cca_bwd, latent-mixing part: adjoints of RoPE, QK-mean, the causal grouped
// convolution and the value shift (the operations of CCA-es §2.B and §3
// item 2, taken in reverse order), plus the conv-tap gradients.
//
//   RoPE:     dq' = R(-phi) dQ''                 (rotation is orthogonal)
//   QK-mean:  dq^_h = (1 + b/2) dq'_h + b/(2G) dk'_g
//             dk^_g = (1 + b/2) dk'_g + b/2 sum_h dq'_h
//             dq~_h += a/2 dq'_h + a/(2G) dk'_g,  dk~_g += a/2 sum_h dq'_h + a/2 dk'_g
//   conv:     dq~[t] += sum_j A_j^T dq^[t + j],   dA_j = sum_t dq^[t] q~[t - j]^T
//   shift:    dv~[t, c] = mask(c) ? dV'[t + 1, c] (0 at the last token) : dV'[t, c]
// with a = [QK-mean pre], b = [QK-mean post] halves folded in as in the forward.
// Tap gradients are summed per block of tokens and then over blocks in a
// fixed order (deterministic).
#include <algorithm>

#include "cca_internal.h"

namespace cca {
namespace {

constexpr int TB = 512;        // tokens per tap-gradient partial block

template <typename T>
__device__ __forceinline__ float ldf(const void* p, long i) {
  return (float)reinterpret_cast<const T*>(p)[i];
}
template <typename T>
__device__ __forceinline__ void stf(void* p, long i, float v) {
  reinterpret_cast<T*>(p)[i] = (T)v;
}

// scratch row layout per token: [dq^ (nq) | dk^ (nk) | dq~ direct (nq) | dk~ direct (nk)]
template <typename T>
__global__ __launch_bounds__(256) void mix_bwd_pointwise(MixBwdArgs a) {
  __shared__ float dqp[kMaxGroup + 1][128];   // dq'_h (h < G), dk'_g at [G]
  const Dims& dm = a.dm;
  const int d = dm.d, G = dm.G, half = d / 2;
  const int t = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const float2 one = make_float2(1.f, 0.f);
  for (int i = threadIdx.x; i < (G + 1) * d; i += blockDim.x) {
    const int hh = i / d, c = i % d;
    const float* src = hh < G ? a.dq : a.dk;
    const long row = hh < G ? ((long)(b * dm.Hq + g * G + hh) * a.S + t) * d
                            : ((long)(b * dm.Hkv + g) * a.S + t) * d;
    const int cp = c < half ? c + half : c - half;
    const float x = src[row + c], xp = src[row + cp];
    const float2 cs = (dm.flags & kRope) ? a.rope[(long)t * half + (c % half)] : one;
    // inverse rotation: (lo, hi) -> (lo cos + hi sin, hi cos - lo sin)
    dqp[hh][c] = c < half ? x * cs.x + xp * cs.y : x * cs.x - xp * cs.y;
  }
  __syncthreads();
  const float A = (dm.flags & kQkPre) ? 0.5f : 0.0f;
  const float Bc = (dm.flags & kQkPost) ? 0.5f : 0.0f;
  const int W = 2 * (dm.nq + dm.nk);
  float* srow = a.scratch + (long)(b * a.S + t) * W;
  for (int c = threadIdx.x; c < d; c += blockDim.x) {
    float sum_q = 0.0f;
    for (int i = 0; i < G; ++i) sum_q += dqp[i][c];
    const float dkp = dqp[G][c];
    for (int i = 0; i < G; ++i) {
      const int h = g * G + i;
      srow[h * d + c] = (1.0f + Bc) * dqp[i][c] + (Bc / G) * dkp;
      srow[dm.nq + dm.nk + h * d + c] = A * dqp[i][c] + (A / G) * dkp;
    }
    srow[dm.nq + g * d + c] = (1.0f + Bc) * dkp + Bc * sum_q;
    srow[2 * dm.nq + dm.nk + g * d + c] = A * sum_q + A * dkp;
    // value shift adjoint
    const bool shifted = (dm.flags & kVShift) && c >= d - dm.sv;
    const long vrow = (long)(b * dm.Hkv + g) * a.S;
    float dvv;
    if (shifted)
      dvv = t + 1 < a.S ? a.dv[(vrow + t + 1) * d + c] : 0.0f;
    else
      dvv = a.dv[(vrow + t) * d + c];
    stf<T>(a.dqkv, (long)(b * a.S + t) * dm.nqkv + dm.nq + dm.nk + g * d + c, dvv);
  }
}

// dq~ = direct + conv adjoint, one work-group per (token, head, sequence) over
// all Hq + Hkv heads.
template <typename T>
__global__ __launch_bounds__(128) void mix_bwd_conv_input(MixBwdArgs a) {
  const Dims& dm = a.dm;
  const int d = dm.d;
  const int t = blockIdx.x, hh = blockIdx.y, b = blockIdx.z;
  const bool isq = hh < dm.Hq;
  const int h = isq ? hh : hh - dm.Hq;
  const int k = isq ? dm.kq : dm.kk;
  const void* taps = isq ? a.conv_q : a.conv_k;
  const long tap0 = (long)h * k * d * d;
  const int W = 2 * (dm.nq + dm.nk);
  const int col = isq ? h * d : dm.nq + h * d;              // dq^ / dk^ column in scratch
  const int dcol = dm.nq + dm.nk + col;                      // direct term column
  for (int c2 = threadIdx.x; c2 < d; c2 += blockDim.x) {
    float s = a.scratch[(long)(b * a.S + t) * W + dcol + c2];
    for (int j = 0; j < k; ++j) {
      if (t + j >= a.S) break;
      const float* g = a.scratch + (long)(b * a.S + t + j) * W + col;
      for (int c = 0; c < d; ++c) s += ldf<T>(taps, tap0 + ((long)j * d + c) * d + c2) * g[c];
    }
    const int ocol = isq ? h * d : dm.nq + h * d;
    stf<T>(a.dqkv, (long)(b * a.S + t) * dm.nqkv + ocol + c2, s);
  }
}

// Partial tap gradients over one block of TB tokens for one head:
// part[blk][head taps] = sum_{t in blk} dq^[t][c] * q~[t - j][c2].
template <typename T>
__global__ __launch_bounds__(256) void mix_bwd_tap_partial(MixBwdArgs a) {
  const Dims& dm = a.dm;
  const int d = dm.d;
  const int blk = blockIdx.x, hh = blockIdx.y;
  const int nblk_s = (a.S + TB - 1) / TB;
  const int b = blk / nblk_s, t0 = (blk % nblk_s) * TB;
  const bool isq = hh < dm.Hq;
  const int h = isq ? hh : hh - dm.Hq;
  const int k = isq ? dm.kq : dm.kk;
  const int W = 2 * (dm.nq + dm.nk);
  const int gcol = isq ? h * d : dm.nq + h * d;
  const int xcol = isq ? h * d : dm.nq + h * d;               // q~ / k~ in qkv
  const long per_blk = (long)dm.Hq * dm.kq * d * d + (long)dm.Hkv * dm.kk * d * d;
  const long off = isq ? (long)h * dm.kq * d * d : (long)dm.Hq * dm.kq * d * d + (long)h * dm.kk * d * d;
  float* out = a.dconv_part + blk * per_blk + off;
  const int t1 = min(a.S, t0 + TB);
  for (int e = threadIdx.x; e < k * d * d; e += blockDim.x) {
    const int j = e / (d * d), c = (e / d) % d, c2 = e % d;
    float s = 0.0f;
    for (int t = max(t0, j); t < t1; ++t)
      s += a.scratch[(long)(b * a.S + t) * W + gcol + c] *
           a.qkv[(long)(b * a.S + t - j) * dm.nqkv + xcol + c2];
    out[e] = s;
  }
}

// ---- d = 128: LDS-tiled, register-blocked fp32 versions of the two kernels
// above (same sums, exact fp32).
constexpr int TD = 128;

// dq~ = direct + sum_j A_j^T dq^[t + j] for 64 tokens of one head: the dq^ tile
// (64 tokens plus the k - 1 after them) sits transposed in LDS, the taps of
// one lag go through LDS 32 input channels at a time; thread = 4 tokens x 8
// output channels.
template <typename T>
__global__ __launch_bounds__(256) void mix_bwd_conv_input_128(MixBwdArgs a) {
  constexpr int TT = 64, TR = TT + kMaxConv;          // tile rows incl. halo, padded
  __shared__ __attribute__((aligned(16))) float gT[TD][TR];   // dq^ transposed [c][t - t0]
  __shared__ __attribute__((aligned(16))) float tp[32][TD];   // taps A_j[c0 + i][c2]
  const Dims& dm = a.dm;
  const int t0 = blockIdx.x * TT, hh = blockIdx.y, b = blockIdx.z;
  const bool isq = hh < dm.Hq;
  const int h = isq ? hh : hh - dm.Hq;
  const int k = isq ? dm.kq : dm.kk;
  const T* taps = reinterpret_cast<const T*>(isq ? a.conv_q : a.conv_k) + (long)h * k * TD * TD;
  const int W = 2 * (dm.nq + dm.nk);
  const int col = isq ? h * TD : dm.nq + h * TD;       // dq^ / dk^ column in scratch
  const int dcol = dm.nq + dm.nk + col;                // direct term
  const float* srow0 = a.scratch + (long)b * a.S * W;
  for (int e = threadIdx.x; e < TR * (TD / 4); e += 256) {
    const int r = e / (TD / 4), c4 = (e % (TD / 4)) * 4;
    const int t = t0 + r;
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (r < TT + k - 1 && t < a.S) v = *reinterpret_cast<const f32x4*>(srow0 + (long)t * W + col + c4);
#pragma unroll
    for (int i = 0; i < 4; ++i) gT[c4 + i][r] = v[i];
  }
  const int ty = threadIdx.x >> 4, tx = threadIdx.x & 15;   // tokens 4ty.., channels 8tx..
  float acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int n = 0; n < 8; ++n) acc[i][n] = 0.0f;
  for (int j = 0; j < k; ++j) {
    for (int c0 = 0; c0 < TD; c0 += 32) {
      __syncthreads();                                   // tile ready / previous taps read
      for (int e = threadIdx.x; e < 32 * TD; e += 256) {
        const int i = e / TD, c2 = e % TD;
        tp[i][c2] = (float)taps[((long)j * TD + c0 + i) * TD + c2];
      }
      __syncthreads();
#pragma unroll 4
      for (int i = 0; i < 32; ++i) {
        const int c = c0 + i;
        float g[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) g[r] = gT[c][4 * ty + r + j];
        const f32x4 w0 = *reinterpret_cast<const f32x4*>(&tp[i][8 * tx]);
        const f32x4 w1 = *reinterpret_cast<const f32x4*>(&tp[i][8 * tx + 4]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
#pragma unroll
          for (int n = 0; n < 4; ++n) {
            acc[r][n] = fmaf(g[r], w0[n], acc[r][n]);
            acc[r][n + 4] = fmaf(g[r], w1[n], acc[r][n + 4]);
          }
        }
      }
    }
  }
  const int ocol = isq ? h * TD : dm.nq + h * TD;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int t = t0 + 4 * ty + r;
    if (t >= a.S) continue;
    const float* dir = srow0 + (long)t * W + dcol + 8 * tx;
    T* out = reinterpret_cast<T*>(a.dqkv) + (long)(b * a.S + t) * dm.nqkv + ocol + 8 * tx;
#pragma unroll
    for (int n = 0; n < 8; ++n) out[n] = (T)(acc[r][n] + dir[n]);
  }
}

// Partial tap gradient of one head and lag over one block of TB tokens:
// part[blk][taps of (head, j)][c][c2] = sum_t dq^[t][c] q~[t - j][c2].  Tokens
// pass through LDS 32 at a time; thread = 8 c x 8 c2.
template <typename T>
__global__ __launch_bounds__(256) void mix_bwd_tap_partial_128(MixBwdArgs a) {
  __shared__ __attribute__((aligned(16))) float gq[32][TD];
  __shared__ __attribute__((aligned(16))) float xq[32][TD];
  const Dims& dm = a.dm;
  const int blk = blockIdx.x, hh = blockIdx.y, j = blockIdx.z;
  const int nblk_s = (a.S + TB - 1) / TB;
  const int b = blk / nblk_s, tb0 = (blk % nblk_s) * TB;
  const bool isq = hh < dm.Hq;
  const int h = isq ? hh : hh - dm.Hq;
  const int k = isq ? dm.kq : dm.kk;
  if (j >= k) return;
  const int W = 2 * (dm.nq + dm.nk);
  const int gcol = isq ? h * TD : dm.nq + h * TD;
  const long per_blk = (long)dm.Hq * dm.kq * TD * TD + (long)dm.Hkv * dm.kk * TD * TD;
  const long off = isq ? (long)h * dm.kq * TD * TD
                       : (long)dm.Hq * dm.kq * TD * TD + (long)h * dm.kk * TD * TD;
  const int ty = threadIdx.x >> 4, tx = threadIdx.x & 15;   // c = 8ty.., c2 = 8tx..
  float acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int n = 0; n < 8; ++n) acc[i][n] = 0.0f;
  const int tend = min(a.S, tb0 + TB);
  for (int t0 = tb0; t0 < tend; t0 += 32) {
    __syncthreads();
    for (int e = threadIdx.x; e < 32 * (TD / 4); e += 256) {
      const int r = e / (TD / 4), c4 = (e % (TD / 4)) * 4;
      const int t = t0 + r;
      f32x4 gv = {0.f, 0.f, 0.f, 0.f}, xv = {0.f, 0.f, 0.f, 0.f};
      if (t < tend) {
        gv = *reinterpret_cast<const f32x4*>(a.scratch + (long)(b * a.S + t) * W + gcol + c4);
        if (t - j >= 0)
          xv = *reinterpret_cast<const f32x4*>(a.qkv + (long)(b * a.S + t - j) * dm.nqkv + gcol + c4);
      }
      *reinterpret_cast<f32x4*>(&gq[r][c4]) = gv;
      *reinterpret_cast<f32x4*>(&xq[r][c4]) = xv;
    }
    __syncthreads();
#pragma unroll 2
    for (int r = 0; r < 32; ++r) {
      const f32x4 g0 = *reinterpret_cast<const f32x4*>(&gq[r][8 * ty]);
      const f32x4 g1 = *reinterpret_cast<const f32x4*>(&gq[r][8 * ty + 4]);
      const f32x4 x0 = *reinterpret_cast<const f32x4*>(&xq[r][8 * tx]);
      const f32x4 x1 = *reinterpret_cast<const f32x4*>(&xq[r][8 * tx + 4]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int n = 0; n < 4; ++n) {
          acc[i][n] = fmaf(g0[i], x0[n], acc[i][n]);
          acc[i][n + 4] = fmaf(g0[i], x1[n], acc[i][n + 4]);
          acc[i + 4][n] = fmaf(g1[i], x0[n], acc[i + 4][n]);
          acc[i + 4][n + 4] = fmaf(g1[i], x1[n], acc[i + 4][n + 4]);
        }
    }
  }
  float* out = a.dconv_part + blk * per_blk + off + (long)j * TD * TD;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    f32x4 v0, v1;
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      v0[n] = acc[i][n];
      v1[n] = acc[i][n + 4];
    }
    *reinterpret_cast<f32x4*>(out + (long)(8 * ty + i) * TD + 8 * tx) = v0;
    *reinterpret_cast<f32x4*>(out + (long)(8 * ty + i) * TD + 8 * tx + 4) = v1;
  }
}

// ---- d = 128 or 64, group size G = 1, 2, 4 or 8 (compile-time, so the
// group's rows stay in named registers): the pointwise adjoints with 256 / (d
// / 8) tokens per work-group.  Thread = (token t0 + tid / (d / 8), channels 4
// (tid % (d / 8)) .. + 3 of the low half and their RoPE partners + d / 2 in
// the high half) for every head of the KV group, so the inverse rotation, the
// QK-mean adjoint (which mixes the group's heads at one channel) and the
// value-shift adjoint stay in registers, with 16-byte loads and stores.
template <int TD>
struct PW {
  static constexpr int TPT = TD / 8;         // threads per token
  static constexpr int PT = 256 / TPT;       // tokens per work-group
};

template <typename T, int G, int TD>
__global__ __launch_bounds__(256) void mix_bwd_pointwise_group(MixBwdArgs a) {
  const Dims& dm = a.dm;
  const int S = a.S;
  constexpr int H = TD / 2, TPT = PW<TD>::TPT;
  const int g = blockIdx.y, b = blockIdx.z;
  const int t = blockIdx.x * PW<TD>::PT + threadIdx.x / TPT, cq = (threadIdx.x % TPT) * 4;
  if (t >= S) return;
  // every read first (the group's rows, both dV' rows, then the RoPE pairs),
  // so they are in flight together
  f32x4 lo[G + 1], hi[G + 1];
#pragma unroll
  for (int hh = 0; hh <= G; ++hh) {
    const float* src = hh < G ? a.dq + ((long)(b * dm.Hq + g * G + hh) * S + t) * TD
                              : a.dk + ((long)(b * dm.Hkv + g) * S + t) * TD;
    lo[hh] = *reinterpret_cast<const f32x4*>(src + cq);
    hi[hh] = *reinterpret_cast<const f32x4*>(src + cq + H);
  }
  // dK'' partial of the key block's second query half, when left to this kernel
  f32x4 k2l = {0.f, 0.f, 0.f, 0.f}, k2h = {0.f, 0.f, 0.f, 0.f};
  if (a.dk2) {
    const float* src2 = a.dk2 + ((long)(b * dm.Hkv + g) * S + t) * TD;
    k2l = *reinterpret_cast<const f32x4*>(src2 + cq);
    k2h = *reinterpret_cast<const f32x4*>(src2 + cq + H);
  }
  const long vrow = (long)(b * dm.Hkv + g) * S;
  f32x4 dvn[2], dvx[2];
#pragma unroll
  for (int part = 0; part < 2; ++part) {
    const int c0 = cq + part * H;
    dvn[part] = *reinterpret_cast<const f32x4*>(a.dv + (vrow + t) * TD + c0);
    dvx[part] = *reinterpret_cast<const f32x4*>(a.dv + (vrow + min(t + 1, S - 1)) * TD + c0);
    if (a.dv2) {
      dvn[part] += *reinterpret_cast<const f32x4*>(a.dv2 + (vrow + t) * TD + c0);
      dvx[part] += *reinterpret_cast<const f32x4*>(a.dv2 + (vrow + min(t + 1, S - 1)) * TD + c0);
    }
  }
  lo[G] += k2l;
  hi[G] += k2h;
  // cos / sin of pairs cq .. cq + 3 at position t
  f32x4 cs_c = {1.f, 1.f, 1.f, 1.f}, cs_s = {0.f, 0.f, 0.f, 0.f};
  if (dm.flags & kRope) {
    const f32x4 r0 = *reinterpret_cast<const f32x4*>(a.rope + (long)t * H + cq);
    const f32x4 r1 = *reinterpret_cast<const f32x4*>(a.rope + (long)t * H + cq + 2);
    cs_c = f32x4{r0[0], r0[2], r1[0], r1[2]};
    cs_s = f32x4{r0[1], r0[3], r1[1], r1[3]};
  }
  // dq'_h (h < G) and dk'_g (index G): inverse rotation of dQ'' / dK'',
  // (lo, hi) -> (lo cos + hi sin, hi cos - lo sin)
#pragma unroll
  for (int hh = 0; hh <= G; ++hh) {
    const f32x4 xl = lo[hh], xh = hi[hh];
    lo[hh] = xl * cs_c + xh * cs_s;
    hi[hh] = xh * cs_c - xl * cs_s;
  }
  const float A = (dm.flags & kQkPre) ? 0.5f : 0.0f;
  const float Bc = (dm.flags & kQkPost) ? 0.5f : 0.0f;
  const int W = 2 * (dm.nq + dm.nk);
  float* srow = a.scratch + ((long)b * S + t) * W;
  f32x4 sl = {0.f, 0.f, 0.f, 0.f}, sh = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < G; ++i) {
    sl += lo[i];
    sh += hi[i];
  }
  const f32x4 kl = lo[G], kh = hi[G];
#pragma unroll
  for (int i = 0; i < G; ++i) {
    const int h = g * G + i;
    *reinterpret_cast<f32x4*>(srow + h * TD + cq) = (1.0f + Bc) * lo[i] + (Bc / G) * kl;
    *reinterpret_cast<f32x4*>(srow + h * TD + cq + H) = (1.0f + Bc) * hi[i] + (Bc / G) * kh;
    *reinterpret_cast<f32x4*>(srow + dm.nq + dm.nk + h * TD + cq) = A * lo[i] + (A / G) * kl;
    *reinterpret_cast<f32x4*>(srow + dm.nq + dm.nk + h * TD + cq + H) = A * hi[i] + (A / G) * kh;
  }
  *reinterpret_cast<f32x4*>(srow + dm.nq + g * TD + cq) = (1.0f + Bc) * kl + Bc * sl;
  *reinterpret_cast<f32x4*>(srow + dm.nq + g * TD + cq + H) = (1.0f + Bc) * kh + Bc * sh;
  *reinterpret_cast<f32x4*>(srow + 2 * dm.nq + dm.nk + g * TD + cq) = A * sl + A * kl;
  *reinterpret_cast<f32x4*>(srow + 2 * dm.nq + dm.nk + g * TD + cq + H) = A * sh + A * kh;
  // value shift adjoint: shifted channels take dV' of token t + 1 (zero at the last)
  T* dvo = reinterpret_cast<T*>(a.dqkv) + ((long)b * S + t) * dm.nqkv + dm.nq + dm.nk + g * TD;
  const int first_shift = (dm.flags & kVShift) ? TD - dm.sv : TD;
#pragma unroll
  for (int part = 0; part < 2; ++part) {
    const int c0 = cq + part * H;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      dvo[c0 + q] = (T)(c0 + q >= first_shift ? (t + 1 < S ? dvx[part][q] : 0.0f) : dvn[part][q]);
  }
}

// ---- bf16 storage, d = 128 or 64: the convolution adjoint on MFMA.
// The adjoint contracts the taps over their first index (dq~[c'] = sum_c
// A_j[c][c'] dq^[c]), and an MFMA operand lane holds 8 consecutive elements of
// the contracted index, so the tap matrices are transposed once per call:
// tapT[m][c'][c] = A_m[c][c'], m running over (head, tap) pairs as the taps are
// stored (query heads, then key heads).
// Work-group (m, quarter): source rows quarter * TD / 4 .. + TD / 4 - 1 of
// tap matrix m, i.e. that column strip of every tapT row.  The strip is staged
// in LDS with 16-byte row copies; a thread then gathers 8 consecutive source
// rows of one column (consecutive lanes take consecutive columns, so every
// 2-byte LDS read of a wave hits distinct banks) and stores them as one
// 16-byte piece of a tapT row.
template <int TD>
__global__ __launch_bounds__(256) void mix_bwd_tap_transpose(MixBwdArgs a) {
  constexpr int QR = TD / 4;                           // source rows per work-group
  __shared__ __attribute__((aligned(16))) bf16 tile[QR][TD + 8];
  const Dims& dm = a.dm;
  const int m = blockIdx.x, r0 = blockIdx.y * QR, nqm = dm.Hq * dm.kq;
  const bf16* src = m < nqm ? reinterpret_cast<const bf16*>(a.conv_q) + (long)m * TD * TD
                            : reinterpret_cast<const bf16*>(a.conv_k) + (long)(m - nqm) * TD * TD;
  bf16* dst = reinterpret_cast<bf16*>(a.tapT) + (long)m * TD * TD;
  for (int e = threadIdx.x; e < QR * TD / 8; e += 256) {
    const int r = e / (TD / 8), c8 = (e % (TD / 8)) * 8;
    *reinterpret_cast<bf16x8*>(&tile[r][c8]) =
        *reinterpret_cast<const bf16x8*>(src + (long)(r0 + r) * TD + c8);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < TD * QR / 8; e += 256) {
    const int c = e % TD, r8 = (e / TD) * 8;           // tapT row c, strip columns r8 .. + 7
    bf16x8 v;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = tile[r8 + i][c];
    *reinterpret_cast<bf16x8*>(dst + (long)c * TD + r0 + r8) = v;
  }
}

// dq~ = direct + sum_j A_j^T dq^[t + j] for 64 tokens of one head: a GEMM with
// M = tokens, N = c', K = (j, c).  The dq^ tile (64 tokens plus the k - 1 after
// them, zero past S) is staged in LDS once as two bf16 halves, hi = bf16(g) and
// lo = bf16(g - hi), and operand A is read from both (~16 mantissa bits of dq^,
// fp32 accumulation); operand B is a row of tapT (exact bf16 taps) from L2.
// With P = d / 64 pairs of 32-channel output blocks, wave w takes tokens 32 (w
// / P) .. + 31 and output channel blocks 2 (w % P), + 1: a work-group covers
// 64 tokens at d = 128, 128 at d = 64.
template <int TD>
struct CG {
  static constexpr int P = TD / 64;
  static constexpr int CT = 32 * 4 / P;              // tokens per work-group
  static constexpr int GLD = TD + 8;                 // LDS row stride (bf16): conflict-free reads
  static constexpr int GPLANE = (CT + kMaxConv - 1) * GLD;
};

template <int TD>
__global__ __launch_bounds__(256) void mix_bwd_conv_input_mfma(MixBwdArgs a) {
  constexpr int CT = CG<TD>::CT, GLD = CG<TD>::GLD, GPLANE = CG<TD>::GPLANE, P = CG<TD>::P;
  __shared__ __attribute__((aligned(16))) bf16 gs[2 * GPLANE];
  const Dims& dm = a.dm;
  const int S = a.S;
  const int t0 = blockIdx.x * CT, hh = blockIdx.y, b = blockIdx.z;
  const bool isq = hh < dm.Hq;
  const int h = isq ? hh : hh - dm.Hq;
  const int k = isq ? dm.kq : dm.kk;
  const int m0 = isq ? h * dm.kq : dm.Hq * dm.kq + h * dm.kk;   // the head's first tap matrix
  const int W = 2 * (dm.nq + dm.nk);
  const int col = isq ? h * TD : dm.nq + h * TD;                // dq^ column in scratch = dq~ column
  const int dcol = dm.nq + dm.nk + col;                         // direct term
  const float* srow0 = a.scratch + (long)b * S * W;
  const int t = threadIdx.x;

  // tile row i = token t0 + i; a resource over the rows inside [t0, S) reads
  // the rest as zero without a branch
  const int nrow = CT + k - 1, r1 = min(S, t0 + nrow);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(srow0 + (long)t0 * W + col), 0, r1 > t0 ? ((r1 - t0 - 1) * W + TD) * 4 : 0, 0x00020000);
  const int n = nrow * (TD / 4);
  constexpr int CNB = 9;                       // 9 x 256 >= (CT + 3) rows x TD / 4 float4: one round
  for (int base = 0; base < n; base += CNB * 256) {
    f32x4 v[CNB];
#pragma unroll
    for (int r = 0; r < CNB; ++r) {
      const int e = min(base + r * 256 + t, n - 1);
      const int i = e / (TD / 4), c4 = (e % (TD / 4)) * 4;
      v[r] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (i * W + c4) * 4, 0, 0));
    }
#pragma unroll
    for (int r = 0; r < CNB; ++r) {
      const int e = base + r * 256 + t;
      if (e < n) {
        const int i = e / (TD / 4), c4 = (e % (TD / 4)) * 4;
        bf16x4 hv, lv;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          hv[q] = (bf16)v[r][q];
          lv[q] = (bf16)(v[r][q] - (float)hv[q]);
        }
        *reinterpret_cast<bf16x4*>(gs + i * GLD + c4) = hv;
        *reinterpret_cast<bf16x4*>(gs + GPLANE + i * GLD + c4) = lv;
      }
    }
  }
  __syncthreads();

  const int lane = t & 63, wave = t >> 6, l32 = lane & 31, hi = lane >> 5;
  const int tw = 32 * (wave / P), nb0 = 2 * (wave % P);
  f32x16 acc[2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.0f;
  // The MFMAs take the tap fragment as their first operand, so each
  // accumulator is transposed: lane = token tw + l32, registers 4 q .. 4 q + 3
  // = the 4 consecutive channels (nb0 + nbi) 32 + 8 q + 4 hi + 0..3.
  // The epilogue's direct terms, loaded now (16 bytes per 4 channels) so their
  // latency overlaps the MFMAs.
  const float* dir = srow0 + (long)t0 * W + dcol + (long)min(tw + l32, S - 1 - t0) * W;
  f32x4 dv[2][4];
#pragma unroll
  for (int nbi = 0; nbi < 2; ++nbi)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      dv[nbi][q] = *reinterpret_cast<const f32x4*>(dir + (nb0 + nbi) * 32 + 8 * q + 4 * hi);
  for (int j = 0; j < k; ++j) {
    // A: lane (token tw + l32, hi) holds channels 16 ks + 8 hi .. of dq^[t + j];
    // B: lane (c' = nb 32 + l32, hi) holds the same channels of tapT row c'
    const bf16* arow = gs + (tw + l32 + j) * GLD + hi * 8;
    const bf16* b0p = reinterpret_cast<const bf16*>(a.tapT) + ((long)(m0 + j) * TD + nb0 * 32 + l32) * TD + hi * 8;
    const bf16* b1p = b0p + 32 * TD;
    // the lag's tap fragments (from L2) all requested before its MFMAs, so the
    // wave waits for L2 once per lag rather than once per k-step
    bf16x8 b0[TD / 16], b1[TD / 16];
#pragma unroll
    for (int ks = 0; ks < TD / 16; ++ks) {
      b0[ks] = *reinterpret_cast<const bf16x8*>(b0p + ks * 16);
      b1[ks] = *reinterpret_cast<const bf16x8*>(b1p + ks * 16);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < TD / 16; ++ks) {
      const bf16x8 ahi = *reinterpret_cast<const bf16x8*>(arow + ks * 16);
      const bf16x8 alo = *reinterpret_cast<const bf16x8*>(arow + GPLANE + ks * 16);
      acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b0[ks], ahi, acc[0], 0, 0, 0);
      acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b0[ks], alo, acc[0], 0, 0, 0);
      acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b1[ks], ahi, acc[1], 0, 0, 0);
      acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b1[ks], alo, acc[1], 0, 0, 0);
    }
  }
  // The CT x TD output tile leaves through LDS (the staged dq^ is no longer
  // read): 8-byte writes of 4 channels into rows of GLD elements, then
  // 16-byte stores of whole rows.
  __syncthreads();
  bf16* const so = gs;
#pragma unroll
  for (int nbi = 0; nbi < 2; ++nbi)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bf16x4 v = {(bf16)(acc[nbi][4 * q] + dv[nbi][q][0]), (bf16)(acc[nbi][4 * q + 1] + dv[nbi][q][1]),
                        (bf16)(acc[nbi][4 * q + 2] + dv[nbi][q][2]), (bf16)(acc[nbi][4 * q + 3] + dv[nbi][q][3])};
      *reinterpret_cast<bf16x4*>(so + (tw + l32) * GLD + (nb0 + nbi) * 32 + 8 * q + 4 * hi) = v;
    }
  __syncthreads();
  bf16* out = reinterpret_cast<bf16*>(a.dqkv) + ((long)b * S + t0) * dm.nqkv + col;
  static_assert(CT * TD / 8 % 256 == 0, "whole rows per pass");
#pragma unroll
  for (int u = 0; u < CT * TD / 8 / 256; ++u) {
    const int e = t + 256 * u, tr = e / (TD / 8), c8 = (e % (TD / 8)) * 8;
    if (t0 + tr < S)
      *reinterpret_cast<bf16x8*>(out + (long)tr * dm.nqkv + c8) =
          *reinterpret_cast<const bf16x8*>(so + tr * GLD + c8);
  }
}

// Partial tap gradient of one head and tap j over one block of TB tokens on
// MFMA: part[blk][taps of (head, j)][c][c'] = sum_t dq^[t][c] q~[t - j][c'], a
// GEMM with M = c, N = c', K = tokens.  Both operands need 8 consecutive
// tokens per lane, so chunks of 64 tokens of dq^ and of q~ (shifted by j) are
// staged transposed, [channel][token], as bf16 hi / lo halves; each product
// takes hi*hi + hi*lo + lo*hi (~16 mantissa bits, fp32 accumulation).
// With NI = d / 64 blocks of 32 per wave and dimension, wave w takes c blocks
// NI (w / 2) .. + NI - 1 and c' blocks NI (w % 2) .. + NI - 1.
constexpr int GT = 64;                       // tokens per LDS chunk
constexpr int TLDT = GT + 8;                 // transposed row stride (bf16)

template <int TD>
__global__ __launch_bounds__(256) void mix_bwd_tap_partial_mfma(MixBwdArgs a) {
  constexpr int TPLANE = TD * TLDT;
  constexpr int NI = TD / 64;                          // 32-blocks per wave in c and in c'
  constexpr int NLD = TD / 16;                         // staging loads per thread and operand
  __shared__ __attribute__((aligned(16))) bf16 gT[2 * TPLANE];   // dq^ [c][t], hi then lo
  __shared__ __attribute__((aligned(16))) bf16 xT[2 * TPLANE];   // q~[t - j] [c'][t], hi then lo
  const Dims& dm = a.dm;
  const int S = a.S;
  const int blk = blockIdx.x, hh = blockIdx.y, j = blockIdx.z;
  const int nblk_s = (S + TB - 1) / TB;
  const int b = blk / nblk_s, tb0 = (blk % nblk_s) * TB;
  const bool isq = hh < dm.Hq;
  const int h = isq ? hh : hh - dm.Hq;
  const int k = isq ? dm.kq : dm.kk;
  if (j >= k) return;
  const int W = 2 * (dm.nq + dm.nk);
  const int gcol = isq ? h * TD : dm.nq + h * TD;      // dq^ in scratch, q~ in qkv
  const long per_blk = (long)dm.Hq * dm.kq * TD * TD + (long)dm.Hkv * dm.kk * TD * TD;
  const long off = isq ? (long)h * dm.kq * TD * TD
                       : (long)dm.Hq * dm.kq * TD * TD + (long)h * dm.kk * TD * TD;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, l32 = lane & 31, hi = lane >> 5;
  const int mb0 = NI * (wave >> 1), nb0 = NI * (wave & 1);
  const int tend = min(S, tb0 + TB);
  // resources over the rows this block reads: dq^ rows [tb0, tend), q~ rows
  // [max(tb0 - j, 0), tend - j); rows outside read as zero without a branch
  const float* gbase = a.scratch + ((long)b * S + tb0) * W + gcol;
  const __amdgpu_buffer_rsrc_t grs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)gbase, 0, ((tend - tb0 - 1) * W + TD) * 4, 0x00020000);
  const int xr0 = max(tb0 - j, 0), xr1 = tend - j;
  const float* xbase = a.qkv + ((long)b * S + xr0) * dm.nqkv + gcol;
  const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)xbase, 0, xr1 > xr0 ? ((xr1 - xr0 - 1) * dm.nqkv + TD) * 4 : 0, 0x00020000);

  f32x16 acc[NI][NI];
#pragma unroll
  for (int mi = 0; mi < NI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.0f;

  // Staging map: item e = t + 256 i (i < NIT) covers tokens 4 (e % 16) .. + 3
  // and channels 4 (e / 16) .. + 3 of the chunk, one float4 load per token;
  // its 4 tokens of each channel go to the transposed tiles as one 8-byte
  // store per plane.  The 16 lanes of a channel group write one 128-byte run
  // of a channel row, and each load instruction reads 64 contiguous bytes of
  // 16 rows.
  constexpr int NIT = GT * TD / 16 / 256;              // items per thread and operand
  static_assert(NIT * 4 == NLD, "one float4 per token of an item");
  for (int c0 = tb0; c0 < tend; c0 += GT) {
    // GT tokens x TD / 4 float4 per operand: NLD of each per thread, all in flight
    f32x4 gv[NIT][4], xv[NIT][4];
#pragma unroll
    for (int i = 0; i < NIT; ++i) {
      const int e = t + 256 * i, r0 = 4 * (e % 16), c4 = 4 * (e / 16);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int tok = c0 + r0 + u;
        gv[i][u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                 grs, ((tok - tb0) * W + c4) * 4, 0, 0));
        // q~ row tok - j; before row 0 the offset wraps past the range (zero)
        xv[i][u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                 xrs, ((tok - j - xr0) * dm.nqkv + c4) * 4, 0, 0));
      }
    }
    __syncthreads();                                     // the previous chunk's reads are done
#pragma unroll
    for (int i = 0; i < NIT; ++i) {
      const int e = t + 256 * i, r0 = 4 * (e % 16), c4 = 4 * (e / 16);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        bf16x4 gh, gl, xh, xl;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const bool live = c0 + r0 + u < tend;          // tokens past the block: zero
          const float g = live ? gv[i][u][q] : 0.0f, x = live ? xv[i][u][q] : 0.0f;
          gh[u] = (bf16)g;
          gl[u] = (bf16)(g - (float)gh[u]);
          xh[u] = (bf16)x;
          xl[u] = (bf16)(x - (float)xh[u]);
        }
        const int o = (c4 + q) * TLDT + r0;
        *reinterpret_cast<bf16x4*>(gT + o) = gh;
        *reinterpret_cast<bf16x4*>(gT + TPLANE + o) = gl;
        *reinterpret_cast<bf16x4*>(xT + o) = xh;
        *reinterpret_cast<bf16x4*>(xT + TPLANE + o) = xl;
      }
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < GT / 16; ++ks) {
      bf16x8 ah[NI], al[NI], bh[NI], bl[NI];
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int ar = ((mb0 + i) * 32 + l32) * TLDT + ks * 16 + hi * 8;
        const int br = ((nb0 + i) * 32 + l32) * TLDT + ks * 16 + hi * 8;
        ah[i] = *reinterpret_cast<const bf16x8*>(gT + ar);
        al[i] = *reinterpret_cast<const bf16x8*>(gT + TPLANE + ar);
        bh[i] = *reinterpret_cast<const bf16x8*>(xT + br);
        bl[i] = *reinterpret_cast<const bf16x8*>(xT + TPLANE + br);
      }
#pragma unroll
      for (int mi = 0; mi < NI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[mi], bh[ni], acc[mi][ni], 0, 0, 0);
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[mi], bl[ni], acc[mi][ni], 0, 0, 0);
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[mi], bh[ni], acc[mi][ni], 0, 0, 0);
        }
    }
  }
  // D: lane holds column c' = nb 32 + l32, register r row c = mb 32 + 8 (r / 4) + 4 hi + r % 4
  float* out = a.dconv_part + blk * per_blk + off + (long)j * TD * TD;
#pragma unroll
  for (int mi = 0; mi < NI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int c = (mb0 + mi) * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
        out[(long)c * TD + (nb0 + ni) * 32 + l32] = acc[mi][ni][r];
      }
}

__global__ __launch_bounds__(256) void mix_bwd_tap_reduce(MixBwdArgs a, int nblk) {
  const Dims& dm = a.dm;
  const long nq = (long)dm.Hq * dm.kq * dm.d * dm.d;
  const long per_blk = nq + (long)dm.Hkv * dm.kk * dm.d * dm.d;
  const long e = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= per_blk) return;
  // 16 loads in flight per batch, added in block order (the same fixed order
  // as one at a time)
  constexpr int RB = 16;
  float s = 0.0f;
  int i = 0;
  for (; i + RB <= nblk; i += RB) {
    float v[RB];
#pragma unroll
    for (int u = 0; u < RB; ++u) v[u] = a.dconv_part[(long)(i + u) * per_blk + e];
#pragma unroll
    for (int u = 0; u < RB; ++u) s += v[u];
  }
  for (; i < nblk; ++i) s += a.dconv_part[(long)i * per_blk + e];
  if (e < nq)
    a.dconv_q[e] = s;
  else
    a.dconv_k[e - nq] = s;
}

int tap_blocks(int B, int S) { return B * ((S + TB - 1) / TB); }

}  // namespace

size_t mix_bwd_part_floats(const Dims& dm, int B, int S) {
  const long per_blk = (long)dm.Hq * dm.kq * dm.d * dm.d + (long)dm.Hkv * dm.kk * dm.d * dm.d;
  return (size_t)tap_blocks(B, S) * per_blk;
}

// The register-blocked pointwise kernel (d = 128 or 64) for the group sizes
// it is instantiated for; false (nothing launched) for others.
template <typename T, int D>
bool launch_pointwise_d(const MixBwdArgs& a, hipStream_t s) {
  const dim3 grid((a.S + PW<D>::PT - 1) / PW<D>::PT, a.dm.Hkv, a.B);
  switch (a.dm.G) {
    case 1: hipLaunchKernelGGL((mix_bwd_pointwise_group<T, 1, D>), grid, dim3(256), 0, s, a); return true;
    case 2: hipLaunchKernelGGL((mix_bwd_pointwise_group<T, 2, D>), grid, dim3(256), 0, s, a); return true;
    case 4: hipLaunchKernelGGL((mix_bwd_pointwise_group<T, 4, D>), grid, dim3(256), 0, s, a); return true;
    case 8: hipLaunchKernelGGL((mix_bwd_pointwise_group<T, 8, D>), grid, dim3(256), 0, s, a); return true;
    default: return false;
  }
}
template <typename T>
bool launch_pointwise_group(const MixBwdArgs& a, hipStream_t s) {
  if (a.dm.d == 128) return launch_pointwise_d<T, 128>(a, s);
  if (a.dm.d == 64) return launch_pointwise_d<T, 64>(a, s);
  return false;
}

bool mfma_d(const Dims& dm) { return dm.d == 128 || dm.d == 64; }

bool mix_bwd_adds_dkdv2(const Dims& dm) {
  return mfma_d(dm) && (dm.G == 1 || dm.G == 2 || dm.G == 4 || dm.G == 8);
}

size_t mix_bwd_tapT_bytes(const Dims& dm) {
  return dm.bf16 && mfma_d(dm) ? (size_t)(dm.Hq * dm.kq + dm.Hkv * dm.kk) * dm.d * dm.d * 2 : 0;
}

size_t mix_bwd_scratch_floats(const Dims& dm, int B, int S) {
  return (size_t)B * S * 2 * (dm.nq + dm.nk);
}

hipError_t launch_mix_bwd(const MixBwdArgs& a, hipStream_t s) {
  const Dims& dm = a.dm;
  const int nblk = tap_blocks(a.B, a.S);
  const long per_blk = (long)dm.Hq * dm.kq * dm.d * dm.d + (long)dm.Hkv * dm.kk * dm.d * dm.d;
  const int kmax = std::max(dm.kq, dm.kk);
  if ((a.dk2 || a.dv2) && !mix_bwd_adds_dkdv2(dm)) return hipErrorInvalidValue;
  if (dm.bf16 && mfma_d(dm)) {
    if (a.tapT == nullptr) return hipErrorInvalidValue;
    const dim3 gtap(nblk, dm.Hq + dm.Hkv, kmax), gtr(dm.Hq * dm.kq + dm.Hkv * dm.kk, 4);
    if (!launch_pointwise_group<bf16>(a, s))
      hipLaunchKernelGGL(mix_bwd_pointwise<bf16>, dim3(a.S, dm.Hkv, a.B), dim3(256), 0, s, a);
    if (dm.d == 128) {
      hipLaunchKernelGGL(mix_bwd_tap_transpose<128>, gtr, dim3(256), 0, s, a);
      hipLaunchKernelGGL(mix_bwd_conv_input_mfma<128>,
                         dim3((a.S + CG<128>::CT - 1) / CG<128>::CT, dm.Hq + dm.Hkv, a.B),
                         dim3(256), 0, s, a);
      hipLaunchKernelGGL(mix_bwd_tap_partial_mfma<128>, gtap, dim3(256), 0, s, a);
    } else {
      hipLaunchKernelGGL(mix_bwd_tap_transpose<64>, gtr, dim3(256), 0, s, a);
      hipLaunchKernelGGL(mix_bwd_conv_input_mfma<64>,
                         dim3((a.S + CG<64>::CT - 1) / CG<64>::CT, dm.Hq + dm.Hkv, a.B),
                         dim3(256), 0, s, a);
      hipLaunchKernelGGL(mix_bwd_tap_partial_mfma<64>, gtap, dim3(256), 0, s, a);
    }
  } else if (dm.d == TD) {
    const dim3 gin((a.S + 63) / 64, dm.Hq + dm.Hkv, a.B), gtap(nblk, dm.Hq + dm.Hkv, kmax);
    {
      if (!launch_pointwise_group<float>(a, s))
        hipLaunchKernelGGL(mix_bwd_pointwise<float>, dim3(a.S, dm.Hkv, a.B), dim3(256), 0, s, a);
      hipLaunchKernelGGL(mix_bwd_conv_input_128<float>, gin, dim3(256), 0, s, a);
      hipLaunchKernelGGL(mix_bwd_tap_partial_128<float>, gtap, dim3(256), 0, s, a);
    }
  } else if (dm.bf16) {
    hipLaunchKernelGGL(mix_bwd_pointwise<bf16>, dim3(a.S, dm.Hkv, a.B), dim3(256), 0, s, a);
    hipLaunchKernelGGL(mix_bwd_conv_input<bf16>, dim3(a.S, dm.Hq + dm.Hkv, a.B), dim3(128), 0, s, a);
    hipLaunchKernelGGL(mix_bwd_tap_partial<bf16>, dim3(nblk, dm.Hq + dm.Hkv), dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL(mix_bwd_pointwise<float>, dim3(a.S, dm.Hkv, a.B), dim3(256), 0, s, a);
    hipLaunchKernelGGL(mix_bwd_conv_input<float>, dim3(a.S, dm.Hq + dm.Hkv, a.B), dim3(128), 0, s, a);
    hipLaunchKernelGGL(mix_bwd_tap_partial<float>, dim3(nblk, dm.Hq + dm.Hkv), dim3(256), 0, s, a);
  }
  hipLaunchKernelGGL(mix_bwd_tap_reduce, dim3((per_blk + 255) / 256), dim3(256), 0, s, a, nblk);
  return hipGetLastError();
}

}  // namespace cca
