// cca_decode, attention part: one new token per sequence attends over the
// compressed latent KV cache (CCA-es §2.C "CCGQA": the smaller cache speeds up
// decoding; CCA-fr §4 "Décodage").  The step streams the K and V caches once,
// so it is bound by HBM bandwidth.
//
// Split over keys (flash-decoding): work-group (chunk, KV head g, sequence b)
// takes keys [512 chunk, 512 chunk + 512) of that sequence's cache, up to its
// position, and serves all G query heads that read KV head g, so each cache
// byte is read once per step.
//   1. S = Q K^T on MFMA: A = the G queries (rows, padded to 32 with zeros,
//      scaled to log2 units), B = K^T straight from global memory (lane = key,
//      16 bytes of its row per load); 4 waves x 4 blocks of 32 keys.
//   2. The chunk's row max m and sum l of p = exp2(s - m) (scores in LDS).
//   3. O_chunk = P V on the vector ALU: lane = 8 channels of one of 4 keys,
//      so a wave load covers four 256-byte V rows; p broadcast from LDS.
// Partials (O_chunk, m, l) go to the workspace; a second kernel merges the
// chunks of each (sequence, query head) and writes O in bf16.
// bf16 storage, d = 128; fp32 accumulation and softmax.
#include "cca_internal.h"

namespace cca {
namespace {

constexpr int D = 128;
constexpr int CK = 512;          // keys per work-group
constexpr int NW = 4;            // waves per work-group
constexpr int PSTRIDE = D + 2;   // floats per partial: O[0..D), m, l

constexpr int MAX_SPLIT = 1024;  // chunks per sequence the merge kernel holds: caches up to 512K

bool fast_decode(const Dims& dm) {
  return dm.bf16 && dm.d == D && dm.G <= kMaxGroup && dm.max_seq_len <= MAX_SPLIT * CK;
}

// GQ: the group size rounded up to a power of two (the kernel is instantiated
// for 1, 2, 4, 8), so P V keeps only that many accumulator rows in registers.
template <int GQ>
__global__ __launch_bounds__(256) void attn_decode_split_kernel(AttnArgs a) {
  constexpr int PW = GQ < 4 ? 4 : GQ;                              // p row: 16-byte aligned
  // scores, then p; after P V the same memory holds the waves' partial O
  __shared__ __attribute__((aligned(16))) float ps[CK * PW > NW * GQ * D ? CK * PW : NW * GQ * D];
  __shared__ float stat[GQ][2];                                    // m, l per query

  const Dims& dm = a.dm;
  const int G = dm.G;
  const int chunk = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int nsplit = gridDim.x;
  const int nkeys = a.pos.p[b] + 1;
  const int k0 = chunk * CK;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  // partial of (b, query head g*G + q, chunk): part[((b*Hq + g*G + q)*nsplit + chunk)*PSTRIDE]
  float* part = a.part + ((long)(b * dm.Hq + g * G) * nsplit + chunk) * PSTRIDE;
  if (k0 >= nkeys) {                         // chunk past this sequence's position
    if (threadIdx.x < G) {
      part[(long)threadIdx.x * nsplit * PSTRIDE + D] = -INFINITY;
      part[(long)threadIdx.x * nsplit * PSTRIDE + D + 1] = 0.0f;
    }
    return;
  }
  const int kend = min(nkeys, k0 + CK);
  const bf16* kb = reinterpret_cast<const bf16*>(a.k) + (long)b * a.kv_bs + (long)g * a.kv_hs;
  const bf16* vb = reinterpret_cast<const bf16*>(a.v) + (long)b * a.kv_bs + (long)g * a.kv_hs;
  // K and V through buffer resources that end at key nkeys - 1: keys past the
  // sequence read as zero without a branch (their scores are masked anyway),
  // so the load loops stay single blocks with every load in flight
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void*)kb, 0, nkeys * D * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)vb, 0, nkeys * D * 2, 0x00020000);

  // ---- 1. scores.  A operand: lane (l32 = query row, hi) holds channels
  // 16 ks + 8 hi + 0..7 of query g*G + l32 (zero rows past G).
  const float scale = 1.44269504088896340736f / sqrtf((float)D);
  bf16x8 qf[8];
  {
    const bf16* qrow = reinterpret_cast<const bf16*>(a.q) + ((long)b * dm.Hq + g * G + l32) * D;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      bf16x8 v;
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = (bf16)0.0f;
      if (l32 < G) v = *reinterpret_cast<const bf16x8*>(qrow + ks * 16 + hi * 8);
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[ks][e] = (bf16)((float)v[e] * scale);
    }
  }
  // One ring of eight 16-byte fragments per lane streams the wave's whole
  // share of the chunk: K fragment ks of the next key block is requested as
  // soon as the MFMA that reads fragment ks of this block has been issued, and
  // after the last block the same slots request the first eight V rows of
  // P V, which stay in flight through the softmax.
  constexpr int NB = CK / 32 / NW;                 // key blocks per wave
  const int slot = lane >> 4, cc = (lane & 15) * 8;
  const int i0 = wave * (CK / NW) + slot;          // P V: this lane's first key
  auto kload = [&](int bi, int ks) {
    const int key = k0 + (wave + bi * NW) * 32 + l32;
    return __builtin_bit_cast(
        bf16x8, __builtin_amdgcn_raw_buffer_load_b128(krs, (key * D + ks * 16 + hi * 8) * 2, 0, 0));
  };
  auto vload = [&](int it) {
    return __builtin_bit_cast(
        bf16x8, __builtin_amdgcn_raw_buffer_load_b128(vrs, ((k0 + i0 + 4 * it) * D + cc) * 2, 0, 0));
  };
  bf16x8 ring[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) ring[ks] = kload(0, ks);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int bi = 0; bi < NB; ++bi) {
    const int blk = wave + bi * NW;
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[ks], ring[ks], acc, 0, 0, 0);
      ring[ks] = bi + 1 < NB ? kload(bi + 1, ks) : vload(ks);
    }
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {     // masks: 0x008 MFMA, 0x020 vector memory read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
    const bool valid = k0 + blk * 32 + l32 < kend;
    // D[query][key]: lane holds key column l32, query rows 8*(r/4) + 4*hi + r%4.
    // Rows G .. GQ-1 come from zero query rows and are never read.
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int q = 8 * (r >> 2) + 4 * hi + (r & 3);
      if (q < GQ) ps[(blk * 32 + l32) * PW + q] = valid ? acc[r] : -INFINITY;
    }
  }
  __syncthreads();

  // ---- 2. max and sum over the chunk, one wave per query (G <= 8 queries)
  for (int q = wave; q < G; q += NW) {
    float m = -INFINITY;
    for (int i = lane; i < CK; i += 64) m = fmaxf(m, ps[i * PW + q]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    float l = 0.0f;
    for (int i = lane; i < CK; i += 64) {
      const float p = __builtin_amdgcn_exp2f(ps[i * PW + q] - m);   // masked keys: 0
      ps[i * PW + q] = p;
      l += p;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) l += __shfl_xor(l, off);
    if (lane == 0) {
      stat[q][0] = m;
      stat[q][1] = l;
    }
  }
  __syncthreads();

  // ---- 3. O_chunk = P V: wave w takes keys w*128 .. w*128+127 of the chunk;
  // lane = (key slot L / 16, channels 8 (L % 16) .. + 7), so one wave load
  // covers 4 whole 256-byte V rows.  The 4 key slots are summed with two
  // shuffles, the 4 waves through LDS.
  float o[GQ][8];
#pragma unroll
  for (int q = 0; q < GQ; ++q)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[q][e] = 0.0f;
  // keys past the sequence have p = 0 and read V as zero; rows q >= G use
  // unwritten scores and are never stored, so the loop has no branch
  // P V continues the ring: slot it % 8 holds V rows of iteration it and is
  // refilled with iteration it + 8 once read
  constexpr int NIT = CK / NW / 4;
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const bf16x8 v8 = ring[it & 7];
    if (it + 8 < NIT) ring[it & 7] = vload(it + 8);
    const int i = i0 + 4 * it;
    const f32x4 pa = *reinterpret_cast<const f32x4*>(&ps[i * PW]);
    f32x4 pb = pa;
    if (GQ > 4) pb = *reinterpret_cast<const f32x4*>(&ps[i * PW + 4]);
#pragma unroll
    for (int q = 0; q < GQ; ++q) {
      const float p = q < 4 ? pa[q] : pb[q - 4];
#pragma unroll
      for (int e = 0; e < 8; ++e) o[q][e] = fmaf(p, (float)v8[e], o[q][e]);
    }
  }
  // the four key slots of a wave are summed with two shuffles, the waves
  // through LDS (over the scores, once every wave is done with them)
#pragma unroll
  for (int q = 0; q < GQ; ++q)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      o[q][e] += __shfl_xor(o[q][e], 16);
      o[q][e] += __shfl_xor(o[q][e], 32);
    }
  __syncthreads();
  float* opart = ps;                          // [NW][GQ][D]
#pragma unroll
  for (int q = 0; q < GQ; ++q)
    if (q < G && slot == 0)
#pragma unroll
      for (int e = 0; e < 8; ++e) opart[(wave * GQ + q) * D + cc + e] = o[q][e];
  __syncthreads();
  for (int e = threadIdx.x; e < G * D; e += 256) {
    const int q = e / D, c = e % D;
    float sum = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) sum += opart[(w * GQ + q) * D + c];
    part[(long)q * nsplit * PSTRIDE + c] = sum;
  }
  if (threadIdx.x < G) {
    part[(long)threadIdx.x * nsplit * PSTRIDE + D] = stat[threadIdx.x][0];
    part[(long)threadIdx.x * nsplit * PSTRIDE + D + 1] = stat[threadIdx.x][1];
  }
}

// Merge of the chunk partials of (sequence b, query head h): the chunk maxima
// and weights in parallel (one thread per chunk, through LDS), then one thread
// per channel sums its weighted partial O over the chunks.  Chunk 0 always
// holds key 0, so the merged max is finite and the weight sum is >= 1.
__global__ __launch_bounds__(D) void attn_decode_merge_kernel(AttnArgs a) {
  __shared__ float wgt[MAX_SPLIT];
  __shared__ float red[D / 64][2];
  const Dims& dm = a.dm;
  const int h = blockIdx.x, b = blockIdx.y;
  const int nsplit = a.nsplit;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const float* part = a.part + (long)(b * dm.Hq + h) * nsplit * PSTRIDE;
  float m = -INFINITY;
  for (int c = t; c < nsplit; c += D) m = fmaxf(m, part[(long)c * PSTRIDE + D]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if (lane == 0) red[wave][0] = m;
  __syncthreads();
  m = red[0][0];
#pragma unroll
  for (int w = 1; w < D / 64; ++w) m = fmaxf(m, red[w][0]);
  float l = 0.0f;
  for (int c = t; c < nsplit; c += D) {
    const float mc = part[(long)c * PSTRIDE + D];
    const float wc = mc == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mc - m);
    wgt[c] = wc;
    l = fmaf(part[(long)c * PSTRIDE + D + 1], wc, l);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) l += __shfl_xor(l, off);
  __syncthreads();
  if (lane == 0) red[wave][1] = l;
  __syncthreads();
  l = red[0][1];
#pragma unroll
  for (int w = 1; w < D / 64; ++w) l += red[w][1];
  float o = 0.0f;
#pragma unroll 8
  for (int c = 0; c < nsplit; ++c) o = fmaf(part[(long)c * PSTRIDE + t], wgt[c], o);
  reinterpret_cast<bf16*>(a.o)[((long)b * dm.Hq + h) * D + t] = (bf16)(o / l);
}

}  // namespace

int decode_nsplit(const Dims& dm, int) {
  return fast_decode(dm) ? (dm.max_seq_len + CK - 1) / CK : 1;
}

size_t decode_part_floats(const Dims& dm, int B) {
  return fast_decode(dm) ? (size_t)B * dm.Hq * decode_nsplit(dm, B) * PSTRIDE : 0;
}

hipError_t launch_attn_decode(const AttnArgs& a, hipStream_t s) {
  if (!fast_decode(a.dm)) return launch_attn_fwd(a, s);
  if (a.part == nullptr || a.nsplit != decode_nsplit(a.dm, a.B) || a.nsplit > MAX_SPLIT)
    return hipErrorInvalidValue;
  const dim3 grid(a.nsplit, a.dm.Hkv, a.B);
  if (a.dm.G <= 1)
    hipLaunchKernelGGL(attn_decode_split_kernel<1>, grid, dim3(256), 0, s, a);
  else if (a.dm.G <= 2)
    hipLaunchKernelGGL(attn_decode_split_kernel<2>, grid, dim3(256), 0, s, a);
  else if (a.dm.G <= 4)
    hipLaunchKernelGGL(attn_decode_split_kernel<4>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(attn_decode_split_kernel<8>, grid, dim3(256), 0, s, a);
  hipLaunchKernelGGL(attn_decode_merge_kernel, dim3(a.dm.Hq, a.B), dim3(D), 0, s, a);
  return hipGetLastError();
}

}  // namespace cca
