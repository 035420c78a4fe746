// cca_mix for bf16 storage with an fp32 latent, d = 128 or 64, on MFMA: the causal
// grouped convolution of q~ and k~ (CCA-es §2.B.1 "Mezcla Convolucional"),
// QK-mean (§2.B.2), value shift (§2.B.3) and RoPE (§3 item 2) in one pass per
// (64 tokens (128 for d = 64), KV group).  This is the prefill that saves its stages for the
// backward: the latent stays fp32 (split into bf16 hi / lo halves for the
// MFMAs) because the softmax gradient amplifies a rounding of q~ and k~ into
// dQ and dK.  The bf16-latent pass for inference is in mix_mfma.hip.
//
// The convolution of one head is a GEMM: out[t, c] = sum_{j, c'} u[t - j, c'] *
// A_j[c, c'] with M = tokens, N = channels, K = k * d.  The fp32 latent tile of
// the head (64 tokens plus the k - 1 halo tokens before them) is read with
// coalesced 16-byte loads and staged in LDS as two bf16 halves, hi = bf16(u)
// and lo = bf16(u - hi), each converted once; operand A is read from both, so
// the product keeps ~16 mantissa bits of q~ and k~ with fp32 accumulation
// (hi + lo also stands in for u in QK-mean, and V' = bf16(v~) is hi itself);
// operand B is the bf16 tap row A_j[c, 8 channels] read from L2.  With lane = output channel and registers = tokens,
// everything QK-mean needs (the same token and channel of the group's query
// heads and its K head) and both channels of a RoPE pair (c, c + d/2) sit in
// one lane.
//
// The d / 32 channel blocks of 32 pair up as (cb, cb + d / 64) (RoPE partners
// d / 2 apart).  Wave w of the 4, with P = d / 64 pairs: tokens t0 + 32 (w / P)
// .. + 31, channel blocks {w % P, w % P + P}; so a work-group covers 64 tokens
// at d = 128 and 128 at d = 64.
#include "cca_internal.h"

namespace cca {
namespace {

template <int D>
struct FGeom {
  static constexpr int P = D / 64;             // channel-block pairs (waves per token block)
  static constexpr int TW = 32 * 4 / P;        // tokens per work-group
  static constexpr int ULD = D + 8;            // LDS row stride (bf16): one 16-byte chunk of pad,
                                               // conflict-free b128 reads
  static constexpr int UROWS = TW + kMaxConv - 1;
  static constexpr int UHALF = UROWS * ULD;    // lo rows follow the hi rows
};

typedef f32x16 Acc2[2];              // [channel block]

__device__ __forceinline__ void zero(Acc2& a) {
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) a[j][r] = 0.0f;
}

// Rows t0 - halo .. t0 + TW - 1 of latent column block `col` into LDS as hi
// (u[0 .. UHALF)) and lo (u[UHALF ..)) bf16 halves (zero outside [0, S)).  LDS
// row i holds token t0 - halo + i.  The loads go through a buffer resource over
// the tile's rows inside [0, S) (a row before it wraps to a huge offset):
// out-of-range rows read as zero without a branch, so each batch of four loads is in flight
// together before its conversions and LDS stores.
template <int D>
__device__ __forceinline__ void load_tile(bf16* u, const float* qkv_b, int nqkv, int col, int S,
                                          int t0, int halo) {
  constexpr int TW = FGeom<D>::TW, ULD = FGeom<D>::ULD, UHALF = FGeom<D>::UHALF;
  const int n = (TW + halo) * (D / 4);
  // resource over the tile's rows inside [0, S), based at its first one
  const int r0 = max(t0 - halo, 0), r1 = min(S, t0 + TW);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(qkv_b + (long)r0 * nqkv + col), 0, r1 > r0 ? ((r1 - r0 - 1) * nqkv + D) * 4 : 0,
      0x00020000);
  constexpr int NB = 4;
  for (int base = 0; base < n; base += NB * 256) {
    f32x4 v[NB];
#pragma unroll
    for (int r = 0; r < NB; ++r) {
      const int e = min(base + r * 256 + (int)threadIdx.x, n - 1);
      const int i = e / (D / 4), ch = (e % (D / 4)) * 4;
      const int t = t0 - halo + i;
      v[r] = __builtin_bit_cast(
          f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, ((t - r0) * nqkv + ch) * 4, 0, 0));
    }
#pragma unroll
    for (int r = 0; r < NB; ++r) {
      const int e = base + r * 256 + (int)threadIdx.x;
      if (e < n) {
        const int i = e / (D / 4), ch = (e % (D / 4)) * 4;
        bf16x4 h, l;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          h[q] = (bf16)v[r][q];
          l[q] = (bf16)(v[r][q] - (float)h[q]);
        }
        *reinterpret_cast<bf16x4*>(u + i * ULD + ch) = h;
        *reinterpret_cast<bf16x4*>(u + UHALF + i * ULD + ch) = l;
      }
    }
  }
}

// cos / sin of channel pair c_lo for the 16 token rows a lane's accumulator
// registers hold (row r: first + 8 (r / 4) + r % 4, relative to the tile), all
// 16 loads in flight together; (1, 0) without RoPE.  Rows past the sequence
// (nrem = tokens of the tile inside it) read the last row: no branch, and
// their results are never stored.
template <int D>
__device__ __forceinline__ void load_rope(float2 (&cs)[16], const float2* rope_t0, int first,
                                          int c_lo, int nrem) {
  if (rope_t0) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int tr = min(first + 8 * (r >> 2) + (r & 3), nrem - 1);
      cs[r] = rope_t0[tr * (D / 2) + c_lo];
    }
  } else {
#pragma unroll
    for (int r = 0; r < 16; ++r) cs[r] = make_float2(1.f, 0.f);
  }
}

// The pre-convolution value hi + lo of LDS row i, channel c.
template <int D>
__device__ __forceinline__ float uval(const bf16* u, int i, int c) {
  constexpr int ULD = FGeom<D>::ULD, UHALF = FGeom<D>::UHALF;
  return (float)u[i * ULD + c] + (float)u[UHALF + i * ULD + c];
}

// acc += conv of one head whose tile is in LDS (row of token t: t - t0 + halo).
template <int D>
__device__ __forceinline__ void conv_head(Acc2& acc, const bf16* u, int halo, int tw0_rel,
                                          const bf16* taps, int k, int cb0, int lane) {
  constexpr int ULD = FGeom<D>::ULD, UHALF = FGeom<D>::UHALF;
  const int l32 = lane & 31, hi = lane >> 5;
  for (int j = 0; j < k; ++j) {
    const bf16* urow = u + (tw0_rel + l32 - j + halo) * ULD + hi * 8;
    const bf16* trow0 = taps + ((long)j * D + cb0 * 32 + l32) * D + hi * 8;
    const bf16* trow1 = trow0 + (D / 2) * D;
#pragma unroll 4
    for (int ks = 0; ks < D / 16; ++ks) {
      const bf16x8 ahi = *reinterpret_cast<const bf16x8*>(urow + ks * 16);
      const bf16x8 alo = *reinterpret_cast<const bf16x8*>(urow + UHALF + ks * 16);
      const bf16x8 b0 = *reinterpret_cast<const bf16x8*>(trow0 + ks * 16);
      const bf16x8 b1 = *reinterpret_cast<const bf16x8*>(trow1 + ks * 16);
      acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi, b0, acc[0], 0, 0, 0);
      acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo, b0, acc[0], 0, 0, 0);
      acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi, b1, acc[1], 0, 0, 0);
      acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo, b1, acc[1], 0, 0, 0);
    }
  }
}

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void mix_fwd_mfma_f32lat_kernel(MixArgs a) {
  using FG = FGeom<D>;
  constexpr int TW = FG::TW, ULD = FG::ULD, UHALF = FG::UHALF, P = FG::P;
  __shared__ __attribute__((aligned(16))) bf16 uk[2 * UHALF];   // k~ tile (hi, lo)
  __shared__ __attribute__((aligned(16))) bf16 uq[2 * UHALF];   // current q~ tile, then v~
  const Dims& dm = a.dm;
  const int G = dm.G, S = a.S;
  const int g = blockIdx.y, b = blockIdx.z;
  const int t0 = blockIdx.x * TW;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int tw0_rel = 32 * (wave / P);       // this wave's first token, relative to t0
  const int cb0 = wave % P;                  // channel blocks cb0 and cb0 + P
  const float* qkv_b = reinterpret_cast<const float*>(a.qkv) + (long)b * S * dm.nqkv;
  const float A = (dm.flags & kQkPre) ? 0.5f : 0.0f;
  const float Bc = (dm.flags & kQkPost) ? 0.5f : 0.0f;
  const bool rope = (dm.flags & kRope) != 0;
  const int kcol = dm.nq + g * D;
  const int hq = dm.kq - 1, hk = dm.kk - 1;  // halo rows of the q and k tiles
  const int c_lo = cb0 * 32 + l32;           // < D / 2: RoPE pair (c_lo, c_lo + D / 2)
  // register r holds token tw0_rel + 8*(r/4) + 4*hi + r%4 (relative to t0)
  auto trel = [&](int r) { return tw0_rel + 8 * (r >> 2) + 4 * hi + (r & 3); };

  const float2* rope_t0 = rope ? a.rope + (long)t0 * (D / 2) : nullptr;
  load_tile<D>(uk, qkv_b, dm.nqkv, kcol, S, t0, hk);
  __syncthreads();
  Acc2 kacc, qacc, mpost, mpre;
  zero(kacc);
  conv_head<D>(kacc, uk, hk, tw0_rel,
            reinterpret_cast<const bf16*>(a.conv_k) + (long)g * dm.kk * D * D, dm.kk, cb0, lane);
  zero(mpost);
  zero(mpre);

  for (int i = 0; i < G; ++i) {
    const int h = g * G + i;
    if (i > 0) __syncthreads();              // every wave is done with the previous q tile
    load_tile<D>(uq, qkv_b, dm.nqkv, h * D, S, t0, hq);
    __syncthreads();
    zero(qacc);
    conv_head<D>(qacc, uq, hq, tw0_rel,
              reinterpret_cast<const bf16*>(a.conv_q) + (long)h * dm.kq * D * D, dm.kq, cb0,
              lane);
    // tile bases plus 32-bit offsets (tokens relative to t0)
    bf16* qo = reinterpret_cast<bf16*>(a.q_out) + ((long)(b * dm.Hq + h) * S + t0) * D;
    float2 csr[16];
    load_rope<D>(csr, rope_t0, trel(0), c_lo, S - t0);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int tr = trel(r);
      const int t = t0 + tr;
      float x[2];
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const int c = c_lo + (D / 2) * cb;
        const float qh = qacc[cb][r], kh = kacc[cb][r];
        const float qp = uval<D>(uq, tr + hq, c);
        const float kp = uval<D>(uk, tr + hk, c);
        mpost[cb][r] += qh;
        mpre[cb][r] += qp;
        x[cb] = qh + A * (qp + kp) + Bc * (qh + kh);
      }
      if (t < S) {
        const float2 cs = csr[r];
        qo[tr * D + c_lo] = (bf16)(x[0] * cs.x - x[1] * cs.y);
        qo[tr * D + c_lo + D / 2] = (bf16)(x[1] * cs.x + x[0] * cs.y);
      }
    }
  }

  // k' = k^ + a/2 (mean_g q~ + k~) + b/2 (mean_g q^ + k^)
  const float invG = 1.0f / (float)G;
  bf16* ko = reinterpret_cast<bf16*>(a.k_out) + ((long)(b * dm.Hkv + g) * S + t0) * D;
  bf16* ko2 = a.k_out2
                  ? reinterpret_cast<bf16*>(a.k_out2) + ((long)(b * dm.Hkv + g) * a.cap2 + t0) * D
                  : nullptr;
  float2 csr[16];
  load_rope<D>(csr, rope_t0, trel(0), c_lo, S - t0);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int tr = trel(r);
    const int t = t0 + tr;
    float x[2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const int c = c_lo + (D / 2) * cb;
      const float kh = kacc[cb][r];
      const float kp = uval<D>(uk, tr + hk, c);
      x[cb] = kh + A * (mpre[cb][r] * invG + kp) + Bc * (mpost[cb][r] * invG + kh);
    }
    if (t < S) {
      const float2 cs = csr[r];
      const bf16 lo = (bf16)(x[0] * cs.x - x[1] * cs.y);
      const bf16 hv = (bf16)(x[1] * cs.x + x[0] * cs.y);
      ko[tr * D + c_lo] = lo;
      ko[tr * D + c_lo + D / 2] = hv;
      if (ko2) {
        ko2[tr * D + c_lo] = lo;
        ko2[tr * D + c_lo + D / 2] = hv;
      }
    }
  }

  // value shift: v~ rows t0 - 1 .. t0 + TW - 1 into LDS (reusing the q tile),
  // then V' in the standard layout (when asked) and transposed, V'^T[c][t]
  __syncthreads();
  const int vcol = dm.nq + dm.nk + g * D;
  load_tile<D>(uq, qkv_b, dm.nqkv, vcol, S, t0, 1);
  __syncthreads();
  const int first_shift = (dm.flags & kVShift) ? D - dm.sv : D;
  bf16* vo = a.v_out ? reinterpret_cast<bf16*>(a.v_out) + ((long)(b * dm.Hkv + g) * S) * D
                     : nullptr;
  bf16* vo2 = a.v_out2 ? reinterpret_cast<bf16*>(a.v_out2) + ((long)(b * dm.Hkv + g) * a.cap2) * D
                       : nullptr;
  if (vo || vo2) {
    for (int e = threadIdx.x; e < TW * D; e += 256) {
      const int tr = e / D, c = e % D;
      const int t = t0 + tr;
      if (t >= S) break;
      const bf16 v = uq[(tr + (c >= first_shift ? 0 : 1)) * ULD + c];   // hi = bf16(v~)
      if (vo) vo[(long)t * D + c] = v;
      if (vo2) vo2[(long)t * D + c] = v;
    }
  }
  if (a.vt_out) {
    // V'^T feeds only the attention's P V product, which runs in fp16 so that P
    // keeps 11 significant bits.  It holds the stored bf16 V' values, converted
    // exactly, so the forward's O and the backward (which reads the bf16 V')
    // see the same V'.
    _Float16* vt = reinterpret_cast<_Float16*>(a.vt_out) + (long)(b * dm.Hkv + g) * D * a.s_pad;
    typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
    for (int e = threadIdx.x; e < D * (TW / 8); e += 256) {
      const int c = e % D, m = e / D;
      const int t = t0 + 8 * m;
      if (t >= a.s_pad) continue;
      const int row_off = c >= first_shift ? 0 : 1;
      f16x8 pk;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        // tokens at or past S are zero: the padding of V'^T up to s_pad
        const bf16 v = t + i < S ? uq[(8 * m + i + row_off) * ULD + c] : (bf16)0.0f;
        pk[i] = (_Float16)(float)v;
      }
      *reinterpret_cast<f16x8*>(vt + (long)c * a.s_pad + t) = pk;
    }
  }
}

}  // namespace

hipError_t launch_mix_fwd_mfma_f32lat(const MixArgs& a, hipStream_t s) {
  if (a.vt_out && (a.s_pad % 64 != 0 || a.s_pad < a.S)) return hipErrorInvalidValue;
  if (a.dm.d == 128) {
    dim3 grid((a.S + FGeom<128>::TW - 1) / FGeom<128>::TW, a.dm.Hkv, a.B);
    hipLaunchKernelGGL(mix_fwd_mfma_f32lat_kernel<128>, grid, dim3(256), 0, s, a);
  } else if (a.dm.d == 64) {
    dim3 grid((a.S + FGeom<64>::TW - 1) / FGeom<64>::TW, a.dm.Hkv, a.B);
    hipLaunchKernelGGL(mix_fwd_mfma_f32lat_kernel<64>, grid, dim3(256), 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace cca
