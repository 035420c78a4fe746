// cca_attn (generic path): causal softmax attention run entirely on the
// latent heads, query head h reading KV head h / G (CCA-es §2.A "Principio
// Fundamental", §2.C "CCGQA"; CCA-fr §2 "Opération d'Attention Compressée",
// "Extension CCGQA").  Scale 1/sqrt(d); query at position p sees keys 0..p.
//
// One work-group per (query row, head, sequence), online softmax over blocks
// of 128 keys.  Any even d <= 128, fp32 or bf16 storage, fp32 arithmetic.
// The bf16 MFMA kernels (attn_mfma.hip, decode.hip) take over for d = 128.
#include "cca_internal.h"

namespace cca {
namespace {

constexpr int AT = 128;   // threads = keys per block

__device__ __forceinline__ float block_reduce(float v, float* red, bool is_max) {
  // 128 threads = 2 waves
  for (int off = 32; off > 0; off >>= 1) {
    const float o = __shfl_xor(v, off);
    v = is_max ? fmaxf(v, o) : v + o;
  }
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return is_max ? fmaxf(red[0], red[1]) : red[0] + red[1];
}

template <typename T>
__global__ __launch_bounds__(AT) void attn_fwd_simple(AttnArgs a) {
  __shared__ float qs[128];
  __shared__ float ps[AT];
  __shared__ float red[2];
  const Dims& dm = a.dm;
  const int d = dm.d;
  const int t = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int g = h / dm.G;
  const int pos = a.decode ? a.pos.p[b] : t;
  const int nkeys = pos + 1;
  const T* q = reinterpret_cast<const T*>(a.q) + ((long)(b * dm.Hq + h) * a.Sq + t) * d;
  const T* kb = reinterpret_cast<const T*>(a.k) + (long)b * a.kv_bs + (long)g * a.kv_hs;
  const T* vb = reinterpret_cast<const T*>(a.v) + (long)b * a.kv_bs + (long)g * a.kv_hs;
  const float scale = 1.0f / sqrtf((float)d);
  for (int c = threadIdx.x; c < d; c += AT) qs[c] = (float)q[c];
  __syncthreads();
  float m = -INFINITY, l = 0.0f, acc = 0.0f;
  for (int k0 = 0; k0 < nkeys; k0 += AT) {
    const int j = k0 + threadIdx.x;
    float s = -INFINITY;
    if (j < nkeys) {
      const T* kr = kb + (long)j * d;
      float dot = 0.0f;
      for (int c = 0; c < d; ++c) dot += qs[c] * (float)kr[c];
      s = dot * scale;
    }
    const float mb = block_reduce(s, red, true);
    const float mn = fmaxf(m, mb);
    const float p = j < nkeys ? __expf(s - mn) : 0.0f;
    const float sp = block_reduce(p, red, false);
    ps[threadIdx.x] = p;
    __syncthreads();
    const float alpha = __expf(m - mn);
    l = l * alpha + sp;
    if (threadIdx.x < d) {
      float o = 0.0f;
      const int n = min(AT, nkeys - k0);
      for (int i = 0; i < n; ++i) o += ps[i] * (float)vb[(long)(k0 + i) * d + threadIdx.x];
      acc = acc * alpha + o;
    }
    m = mn;
    __syncthreads();
  }
  if (threadIdx.x < d) {
    const long off = ((long)(b * a.Sq + t) * dm.Hq + h) * d + threadIdx.x;
    reinterpret_cast<T*>(a.o)[off] = (T)(acc / l);
    if (a.o32) a.o32[off] = acc / l;
  }
  if (threadIdx.x == 0 && a.lse) a.lse[(long)(b * dm.Hq + h) * a.Sq + t] = m + logf(l);
}

}  // namespace

hipError_t launch_attn_fwd_mfma(const AttnArgs& a, hipStream_t s);   // attn_mfma.hip

hipError_t launch_attn_fwd(const AttnArgs& a, hipStream_t s) {
  if (!a.decode && prefill_uses_mfma(a.dm)) return launch_attn_fwd_mfma(a, s);
  dim3 grid(a.Sq, a.dm.Hq, a.B);
  if (a.dm.bf16)
    hipLaunchKernelGGL(attn_fwd_simple<bf16>, grid, dim3(AT), 0, s, a);
  else
    hipLaunchKernelGGL(attn_fwd_simple<float>, grid, dim3(AT), 0, s, a);
  return hipGetLastError();
}

}  // namespace cca
