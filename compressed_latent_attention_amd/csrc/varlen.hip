// Helpers of the chunked, variable-length batched prefill (the serving
// handoff of the compressed latent cache, CCA-es §2.C and §1 item 2; CCA-fr §4
// "Décodage"): the rolling conv / value-shift state advanced past each
// sequence's chunk, and the fp16 V'^T of each sequence's cache rows that the
// MFMA attention's P V product reads.  No layer arithmetic beyond copies.
#include "cca_internal.h"

namespace cca {
namespace {

constexpr int D = 128;

// One work-group per sequence.  The state holds, most recent first, q~ at lags
// 1..kq-1, k~ at lags 1..kk-1 and v~ at lag 1; after a chunk of n >= 1 tokens,
// lag l is the chunk's token n - l when that exists, else the old state's lag
// l - n.  Every new value is formed before any is written (the old state is
// read in place).
__global__ __launch_bounds__(256) void state_varlen_kernel(Dims dm, VarlenMap vm, const bf16* lat,
                                                           bf16* state) {
  extern __shared__ bf16 nst[];                 // the new state of this sequence
  const int b = blockIdx.x;
  const int n = vm.tok[b + 1] - vm.tok[b];
  if (n == 0) return;
  bf16* st = state + (long)b * dm.state_w;
  const bf16* lb = lat + (long)vm.tok[b] * dm.nqkv;
  const int nqp = (dm.kq - 1) * dm.nq, nkp = (dm.kk - 1) * dm.nk;
  for (int i = threadIdx.x; i < dm.state_w; i += 256) {
    int lag, col, width, base;                  // width: elements per lag of the part
    if (i < nqp) {
      width = dm.nq; base = 0; lag = i / width + 1; col = i % width;
    } else if (i < nqp + nkp) {
      width = dm.nk; base = nqp; lag = (i - nqp) / width + 1; col = (i - nqp) % width;
    } else {
      width = dm.nk; base = nqp + nkp; lag = 1; col = i - nqp - nkp;
    }
    const int lcol = i < nqp ? col : (i < nqp + nkp ? dm.nq + col : dm.nq + dm.nk + col);
    const int t = n - lag;
    nst[i] = t >= 0 ? lb[(long)t * dm.nqkv + lcol] : st[base + (lag - n - 1) * width + col];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < dm.state_w; i += 256) st[i] = nst[i];
}

// V'^T of sequence b, KV head g, keys c0 .. c0 + 63 (one work-group): cache
// rows (bf16 [cap][d]) to columns of vt ([d][s_pad] fp16, the stored values
// converted exactly within fp16's range); keys at or past start + n are zero.
__global__ __launch_bounds__(256) void vt_varlen_kernel(Dims dm, VarlenMap vm, const bf16* v_cache,
                                                        int cap, _Float16* vt, int s_pad) {
  __shared__ bf16 tile[64][D + 2];
  const int c0 = blockIdx.x * 64, g = blockIdx.y, b = blockIdx.z;
  const int L = vm.start[b] + vm.tok[b + 1] - vm.tok[b];
  if (c0 >= (L + 63) / 64 * 64) return;
  const bf16* src = v_cache + ((long)(b * dm.Hkv + g) * cap) * D;
  for (int e = threadIdx.x; e < 64 * (D / 8); e += 256) {
    const int r = e / (D / 8), c8 = (e % (D / 8)) * 8;
    bf16x8 v;
    if (c0 + r < L) {
      v = *reinterpret_cast<const bf16x8*>(src + (long)(c0 + r) * D + c8);
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = (bf16)0.0f;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) tile[r][c8 + k] = v[k];
  }
  __syncthreads();
  typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
  _Float16* dst = vt + ((long)(b * dm.Hkv + g) * D) * s_pad + c0;
  for (int e = threadIdx.x; e < D * 8; e += 256) {
    const int c = e / 8, k8 = (e % 8) * 8;
    f16x8 o;
#pragma unroll
    for (int k = 0; k < 8; ++k) o[k] = (_Float16)(float)tile[k8 + k][c];
    *reinterpret_cast<f16x8*>(dst + (long)c * s_pad + k8) = o;
  }
}

}  // namespace

hipError_t launch_state_varlen(const Dims& dm, const VarlenMap& vm, const void* lat, void* state,
                               hipStream_t s) {
  if (!dm.bf16 || vm.B < 1 || vm.B > kMaxVarlenBatch) return hipErrorInvalidValue;
  const size_t lds = (size_t)dm.state_w * sizeof(bf16);
  if (lds > 64 * 1024) return hipErrorInvalidValue;
  hipLaunchKernelGGL(state_varlen_kernel, dim3(vm.B), dim3(256), lds, s, dm, vm,
                     reinterpret_cast<const bf16*>(lat), reinterpret_cast<bf16*>(state));
  return hipGetLastError();
}

hipError_t launch_vt_varlen(const Dims& dm, const VarlenMap& vm, const void* v_cache, int cap,
                            void* vt, int s_pad, hipStream_t s) {
  if (!dm.bf16 || dm.d != D || s_pad % 64 != 0 || vm.B < 1 || vm.B > kMaxVarlenBatch)
    return hipErrorInvalidValue;
  if (s_pad == 0) return hipSuccess;
  hipLaunchKernelGGL(vt_varlen_kernel, dim3(s_pad / 64, dm.Hkv, vm.B), dim3(256), 0, s, dm, vm,
                     reinterpret_cast<const bf16*>(v_cache), cap,
                     reinterpret_cast<_Float16*>(vt), s_pad);
  return hipGetLastError();
}

}  // namespace cca
