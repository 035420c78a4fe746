// cca_bwd, attention part (generic path): gradients of causal softmax
// attention on the latent heads (CCA-es §4, training backward; CCA-fr §4
// "Rétropropagation").  Probabilities are recomputed from Q'', K'' and the
// saved log-sum-exp, never stored:
//   P = exp(Q K^T / sqrt(d) - lse), D_t = <dO_t, O_t>,
//   dV = P^T dO, dS = P * (dO V^T - D) / sqrt(d), dQ = dS K, dK = dS^T Q,
// with dK and dV of a KV head summed over its G query heads in registers (no
// atomics: run-to-run deterministic).  Any even d <= 128, fp32 arithmetic.
// The bf16 MFMA kernels in attn_bwd_mfma.hip take over for d = 128.
#include "cca_internal.h"

namespace cca {
namespace {

constexpr int BT = 128;

template <typename T>
__device__ __forceinline__ float ldf(const void* p, long i) {
  return (float)reinterpret_cast<const T*>(p)[i];
}

template <typename T>
__global__ __launch_bounds__(64) void attn_bwd_dsum(AttnBwdArgs a) {
  const Dims& dm = a.dm;
  const int t = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const long base = ((long)(b * a.S + t) * dm.Hq + h) * dm.d;
  float s = 0.0f;
  for (int c = threadIdx.x; c < dm.d; c += 64) s += ldf<T>(a.dO, base + c) * a.o32[base + c];
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
  if (threadIdx.x == 0) a.Dsum[(long)(b * dm.Hq + h) * a.S + t] = s;
}

// dQ for one (query row, head, sequence).
template <typename T>
__global__ __launch_bounds__(BT) void attn_bwd_dq_simple(AttnBwdArgs a) {
  __shared__ float qs[128], dos[128], ds[BT];
  const Dims& dm = a.dm;
  const int d = dm.d;
  const int t = blockIdx.x, h = blockIdx.y, b = blockIdx.z, g = h / dm.G;
  const float scale = 1.0f / sqrtf((float)d);
  const long qoff = ((long)(b * dm.Hq + h) * a.S + t) * d;
  const long ooff = ((long)(b * a.S + t) * dm.Hq + h) * d;
  const long kvoff = (long)(b * dm.Hkv + g) * a.S * d;
  for (int c = threadIdx.x; c < d; c += BT) {
    qs[c] = ldf<T>(a.q, qoff + c);
    dos[c] = ldf<T>(a.dO, ooff + c);
  }
  const float lse = a.lse[(long)(b * dm.Hq + h) * a.S + t];
  const float D = a.Dsum[(long)(b * dm.Hq + h) * a.S + t];
  __syncthreads();
  float acc = 0.0f;
  for (int k0 = 0; k0 <= t; k0 += BT) {
    const int j = k0 + threadIdx.x;
    float dsv = 0.0f;
    if (j <= t) {
      float s = 0.0f, dp = 0.0f;
      for (int c = 0; c < d; ++c) {
        s += qs[c] * ldf<T>(a.k, kvoff + (long)j * d + c);
        dp += dos[c] * ldf<T>(a.v, kvoff + (long)j * d + c);
      }
      const float p = __expf(s * scale - lse);
      dsv = p * (dp - D) * scale;
    }
    ds[threadIdx.x] = dsv;
    __syncthreads();
    if (threadIdx.x < d) {
      const int n = min(BT, t + 1 - k0);
      for (int i = 0; i < n; ++i) acc += ds[i] * ldf<T>(a.k, kvoff + (long)(k0 + i) * d + threadIdx.x);
    }
    __syncthreads();
  }
  if (threadIdx.x < d) a.dq[qoff + threadIdx.x] = acc;
}

// dK, dV for one (key row, KV head, sequence), summed over the group's heads.
template <typename T>
__global__ __launch_bounds__(BT) void attn_bwd_dkdv_simple(AttnBwdArgs a) {
  __shared__ float ks[128], vs[128], ps[BT], ds[BT];
  const Dims& dm = a.dm;
  const int d = dm.d;
  const int j = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const float scale = 1.0f / sqrtf((float)d);
  const long kvoff = ((long)(b * dm.Hkv + g) * a.S + j) * d;
  for (int c = threadIdx.x; c < d; c += BT) {
    ks[c] = ldf<T>(a.k, kvoff + c);
    vs[c] = ldf<T>(a.v, kvoff + c);
  }
  __syncthreads();
  float dk = 0.0f, dv = 0.0f;
  for (int hi = 0; hi < dm.G; ++hi) {
    const int h = g * dm.G + hi;
    const long qbase = (long)(b * dm.Hq + h) * a.S * d;
    for (int t0 = j; t0 < a.S; t0 += BT) {
      const int t = t0 + threadIdx.x;
      float pv = 0.0f, dsv = 0.0f;
      if (t < a.S) {
        float s = 0.0f, dp = 0.0f;
        const long ooff = ((long)(b * a.S + t) * dm.Hq + h) * d;
        for (int c = 0; c < d; ++c) {
          s += ldf<T>(a.q, qbase + (long)t * d + c) * ks[c];
          dp += ldf<T>(a.dO, ooff + c) * vs[c];
        }
        const long r = (long)(b * dm.Hq + h) * a.S + t;
        pv = __expf(s * scale - a.lse[r]);
        dsv = pv * (dp - a.Dsum[r]) * scale;
      }
      ps[threadIdx.x] = pv;
      ds[threadIdx.x] = dsv;
      __syncthreads();
      if (threadIdx.x < d) {
        const int n = min(BT, a.S - t0);
        for (int i = 0; i < n; ++i) {
          const int tt = t0 + i;
          dv += ps[i] * ldf<T>(a.dO, ((long)(b * a.S + tt) * dm.Hq + h) * d + threadIdx.x);
          dk += ds[i] * ldf<T>(a.q, qbase + (long)tt * d + threadIdx.x);
        }
      }
      __syncthreads();
    }
  }
  if (threadIdx.x < d) {
    a.dk[kvoff + threadIdx.x] = dk;
    a.dv[kvoff + threadIdx.x] = dv;
  }
}

}  // namespace

hipError_t launch_attn_bwd_mfma(const AttnBwdArgs& a, hipStream_t s);   // attn_bwd_mfma.hip
bool attn_bwd_mfma_supported(const Dims& dm);

hipError_t launch_attn_bwd(const AttnBwdArgs& a, hipStream_t s) {
  const Dims& dm = a.dm;
  if (dm.bf16 && attn_bwd_mfma_supported(dm)) return launch_attn_bwd_mfma(a, s);
  dim3 gq(a.S, dm.Hq, a.B), gk(a.S, dm.Hkv, a.B);
  if (dm.bf16) {
    hipLaunchKernelGGL(attn_bwd_dsum<bf16>, gq, dim3(64), 0, s, a);
    hipLaunchKernelGGL(attn_bwd_dq_simple<bf16>, gq, dim3(BT), 0, s, a);
    hipLaunchKernelGGL(attn_bwd_dkdv_simple<bf16>, gk, dim3(BT), 0, s, a);
  } else {
    hipLaunchKernelGGL(attn_bwd_dsum<float>, gq, dim3(64), 0, s, a);
    hipLaunchKernelGGL(attn_bwd_dq_simple<float>, gq, dim3(BT), 0, s, a);
    hipLaunchKernelGGL(attn_bwd_dkdv_simple<float>, gk, dim3(BT), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace cca
