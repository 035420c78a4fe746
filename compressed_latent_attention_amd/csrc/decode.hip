// cca_decode, attention part: one new token per sequence attends over the
// compressed latent KV cache (CCA-es §2.C "CCGQA": the smaller cache speeds up
// decoding; CCA-fr §4 "Décodage").  The step streams the K and V caches once,
// so it is bound by HBM bandwidth.
//
// Split over keys (flash-decoding): about 256 work-groups in all, nsplit_b per
// (KV head g, sequence b) in proportion to the sequence's length (a ragged
// batch spreads its long caches over the chip), each serving all G query
// heads that read head g, so each cache byte is read once per step.  The 4 nsplit waves of one (b, g)
// take its 32-key blocks round robin, so together they sweep its K and V as
// one window; every wave keeps its own online softmax:
//   1. S = Q K^T on MFMA: A = the G queries as stored (rows, padded to 32
//      with zeros), B = K^T straight from global memory (lane = key, 16 bytes
//      of its row per load); the fp32 scores are then scaled to log2 units.
//   2. Block max over the 32 keys by DPP and a swizzle, rescale of the running
//      O and l, p = exp2(s - m) to a per-wave LDS row block.
//   3. O += P V on the vector ALU: lane = 8 channels of one of 64 / (d / 8)
//      keys, so a wave load covers 1 KB of whole V rows (4 rows at d = 128,
//      8 at d = 64).
// The next block's K and V rows are requested while the current one is
// computed.  The four waves of a work-group merge in LDS into one partial
// (O, m, l); a second kernel merges the partials of each (sequence, query
// head) and writes O in bf16.
// bf16 storage, d = 128 or 64; fp32 accumulation and softmax.
#include "cca_internal.h"

#include <algorithm>

namespace cca {
namespace {

constexpr int NW = 4;            // waves per work-group
constexpr int TARGET_WGS = 256;  // work-groups per launch: two per CU, all resident at once

constexpr int MAX_SPLIT = 1024;  // work-groups per (sequence, KV head) at most

bool fast_decode(const Dims& dm) {
  return dm.bf16 && (dm.d == 128 || dm.d == 64) && dm.G <= kMaxGroup;
}
// floats per partial: O[0..d), m, l
int pstride(const Dims& dm) { return dm.d + 2; }

// Max over each 32-lane half of the wave: DPP within rows of 16 lanes (swap
// neighbours, pairs, mirror in 8, mirror in 16), then a swizzle that exchanges
// the two rows of each half.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float half_max(float v) {
  v = fmaxf(v, dpp_mov<0xB1>(v));    // quad_perm [1, 0, 3, 2]
  v = fmaxf(v, dpp_mov<0x4E>(v));    // quad_perm [2, 3, 0, 1]
  v = fmaxf(v, dpp_mov<0x141>(v));   // row_half_mirror
  v = fmaxf(v, dpp_mov<0x140>(v));   // row_mirror
  // swizzle, bit mode: and_mask 0x1F, or_mask 0, xor_mask 0x10
  return fmaxf(v, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F)));
}

// GQ: the group size rounded up to a power of two (the kernel is instantiated
// for 1, 2, 4, 8), so P V keeps only that many accumulator rows in registers.
//
// Work-group (flattened split index over the sequences, KV head g): sequence
// b owns indices pos.off[b] .. pos.off[b + 1] - 1 (nsplit of them); its wave w
// takes the 32-key blocks (i nsplit + split) NW + w, i = 0, 1, ..., so the
// nsplit NW waves of
// one (sequence, head) read consecutive 8 KB blocks and sweep its K and V as
// one wide window.  Each wave runs its own online softmax over its blocks with
// no barrier: while block n is scored and accumulated, the K and V rows of
// block n + 1 are already requested (a ring of 8 + 8 fragment registers, each
// slot refilled as soon as it has been read).  The four waves are merged in
// LDS at the end.
template <int D, int GQ>
__global__ __launch_bounds__(256, 2) void attn_decode_split_kernel(AttnArgs a) {
  constexpr int PSTRIDE = D + 2;
  constexpr int NKS = D / 16;                        // 16-channel k-steps of S = Q K^T
  constexpr int CPL = D / 8;                         // lanes per V row in P V
  constexpr int SLOTS = 64 / CPL;                    // V rows per wave load
  constexpr int NV = 32 / SLOTS;                     // V loads per 32-key block
  constexpr int PW = 8;                              // p row per key: queries 0..7
  constexpr int NR = GQ < 4 ? GQ : 4;                // score rows per lane half that matter
  __shared__ __attribute__((aligned(16))) float pbuf[NW][32 * PW];   // p of the current block
  __shared__ __attribute__((aligned(16))) float ow[NW][GQ][D];       // per-wave O, then merged
  __shared__ float mlw[NW][GQ][2];                                   // per-wave m, l

  const Dims& dm = a.dm;
  const int G = dm.G;
  const int g = blockIdx.y;
  int b = 0;
  {
    int lo = 0, hi2 = a.B - 1;                        // last b with off[b] <= blockIdx.x
    while (lo < hi2) {
      const int mid = (lo + hi2 + 1) >> 1;
      if (a.pos.off[mid] <= (int)blockIdx.x) lo = mid; else hi2 = mid - 1;
    }
    b = lo;
  }
  const int off_b = a.pos.off[b];
  const int split = (int)blockIdx.x - off_b, nsplit = a.pos.off[b + 1] - off_b;
  const int nkeys = a.pos.p[b] + 1;
  const int nblk = (nkeys + 31) / 32;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int first = split * NW + wave, stride = nsplit * NW;
  const int nit = first < nblk ? (nblk - first + stride - 1) / stride : 0;
  const bf16* kb = reinterpret_cast<const bf16*>(a.k) + (long)b * a.kv_bs + (long)g * a.kv_hs;
  const bf16* vb = reinterpret_cast<const bf16*>(a.v) + (long)b * a.kv_bs + (long)g * a.kv_hs;
  // K and V through buffer resources that end at key nkeys - 1: keys past the
  // sequence (the tail of the last block, the prefetch after it) read as zero
  // without a branch; their scores are masked
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void*)kb, 0, nkeys * D * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)vb, 0, nkeys * D * 2, 0x00020000);

  // S = Q K^T on MFMA.  A operand: lane (l32 = query row, hi) holds channels
  // 16 ks + 8 hi + 0..7 of query g*G + l32 as stored (zero rows past G); B
  // operand: lane (l32 = key, hi) holds the same channels of its key.  The
  // fp32 scores are scaled to log2 units (log2(e) / sqrt(d)) before the
  // softmax, so Q is not rounded a second time.
  // D[query][key]: lane holds key l32, query rows 4 hi + r in acc[r], r < 4.
  const float scale = 1.44269504088896340736f / sqrtf((float)D);
  bf16x8 qf[NKS];
  {
    const bf16* qrow = reinterpret_cast<const bf16*>(a.q) + ((long)b * dm.Hq + g * G + l32) * D;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[ks][e] = (bf16)0.0f;
      if (l32 < G) qf[ks] = *reinterpret_cast<const bf16x8*>(qrow + ks * 16 + hi * 8);
    }
  }
  // P V on the vector ALU: lane = (key slot L / CPL, channels 8 (L % CPL) ..
  // + 7) takes keys slot + SLOTS i (i < NV) of a block, so one wave load
  // covers SLOTS whole V rows.
  const int slot = lane / CPL, cc = (lane % CPL) * 8;
  auto kload = [&](int blk, int ks) {
    return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                          krs, ((blk * 32 + l32) * D + ks * 16 + hi * 8) * 2, 0, 0));
  };
  auto vload = [&](int blk, int i) {
    return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                          vrs, ((blk * 32 + slot + SLOTS * i) * D + cc) * 2, 0, 0));
  };

  float m[NR], lsum[NR];                 // running max and this lane's share of the sum
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    m[r] = -INFINITY;
    lsum[r] = 0.0f;
  }
  float o[GQ][8];
#pragma unroll
  for (int q = 0; q < GQ; ++q)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[q][e] = 0.0f;

  bf16x8 kr[NKS], vr[NV];
  int blk = first;
#pragma unroll
  for (int j = 0; j < NKS; ++j) kr[j] = kload(blk, j);
#pragma unroll
  for (int j = 0; j < NV; ++j) vr[j] = vload(blk, j);
  float* pw = pbuf[wave];
  for (int it = 0; it < nit; ++it) {
    const int nxt = blk + stride;
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[ks], kr[ks], acc, 0, 0, 0);
      kr[ks] = kload(nxt, ks);
    }
    __builtin_amdgcn_sched_barrier(0);   // V work stays below: its waits come later
    // online softmax over this block (block max over the 32 keys of each half)
    const bool valid = blk * 32 + l32 < nkeys;
    float p[4], al[4];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const float s = valid ? acc[r] * scale : -INFINITY;
      float mb = s;
      mb = half_max(mb);
      const float mn = fmaxf(m[r], mb);            // finite: key 32 blk is valid
      al[r] = __builtin_amdgcn_exp2f(m[r] - mn);
      m[r] = mn;
      p[r] = __builtin_amdgcn_exp2f(s - mn);
      lsum[r] = fmaf(lsum[r], al[r], p[r]);
    }
#pragma unroll
    for (int r = NR; r < 4; ++r) p[r] = 0.0f;
    // p to this wave's LDS row block: [key l32][query 4 hi + r].  LDS accesses
    // of one wave complete in order, so the reads below see these writes and
    // the next block's writes follow these reads.
    *reinterpret_cast<f32x4*>(&pw[l32 * PW + 4 * hi]) = f32x4{p[0], p[1], p[2], p[3]};
    // rescale O by each query's factor (uniform over its lane half)
#pragma unroll
    for (int q = 0; q < GQ; ++q) {
      const float aq = __int_as_float(
          __builtin_amdgcn_readlane(__float_as_int(al[q & 3]), (q >> 2) * 32));
#pragma unroll
      for (int e = 0; e < 8; ++e) o[q][e] *= aq;
    }
    // the p rows of this lane's NV keys, read together (one wait)
    f32x4 pa[NV], pb[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      pa[i] = *reinterpret_cast<const f32x4*>(&pw[(slot + SLOTS * i) * PW]);
      if (GQ > 4) pb[i] = *reinterpret_cast<const f32x4*>(&pw[(slot + SLOTS * i) * PW + 4]);
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      // the slot is refilled only once its rows are converted, so the new
      // load lands in the same registers (no copy that would wait for it)
      float vf[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) vf[e] = (float)vr[i][e];
      __builtin_amdgcn_sched_barrier(0);
      vr[i] = vload(nxt, i);
#pragma unroll
      for (int q = 0; q < GQ; ++q) {
        const float pq = q < 4 ? pa[i][q] : pb[i][q - 4];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[q][e] = fmaf(pq, vf[e], o[q][e]);
      }
    }
    blk = nxt;
  }
  // this wave's l (over the 32 lanes of each half) and O (over the key slots)
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int off = 1; off < 32; off <<= 1) lsum[r] += __shfl_xor(lsum[r], off);
#pragma unroll
  for (int q = 0; q < GQ; ++q)
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int off = CPL; off < 64; off <<= 1) o[q][e] += __shfl_xor(o[q][e], off);
  if (slot == 0)
#pragma unroll
    for (int q = 0; q < GQ; ++q)
#pragma unroll
      for (int e = 0; e < 8; ++e) ow[wave][q][cc + e] = o[q][e];
  if (l32 == 0)
#pragma unroll
    for (int r = 0; r < NR; ++r)
      if (4 * hi + r < GQ) {
        mlw[wave][4 * hi + r][0] = m[r];
        mlw[wave][4 * hi + r][1] = lsum[r];
      }
  __syncthreads();
  // merge the four waves (a wave with no block has m = -inf, l = 0, O = 0)
  // partial of (b, query head h, split): part[(off_b Hq + h nsplit + split) PSTRIDE]
  float* part = a.part + ((long)off_b * dm.Hq + (long)g * G * nsplit + split) * PSTRIDE;
  for (int e = threadIdx.x; e < G * D; e += 256) {
    const int q = e / D, c = e % D;
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) mx = fmaxf(mx, mlw[w][q][0]);
    float sum = 0.0f;
    if (mx != -INFINITY)
#pragma unroll
      for (int w = 0; w < NW; ++w) sum = fmaf(ow[w][q][c], __builtin_amdgcn_exp2f(mlw[w][q][0] - mx), sum);
    part[(long)q * nsplit * PSTRIDE + c] = sum;
  }
  if (threadIdx.x < G) {
    const int q = threadIdx.x;
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) mx = fmaxf(mx, mlw[w][q][0]);
    float l = 0.0f;
    if (mx != -INFINITY)
#pragma unroll
      for (int w = 0; w < NW; ++w) l = fmaf(mlw[w][q][1], __builtin_amdgcn_exp2f(mlw[w][q][0] - mx), l);
    part[(long)q * nsplit * PSTRIDE + D] = mx;
    part[(long)q * nsplit * PSTRIDE + D + 1] = l;
  }
}

// Merge of the nsplit partials of (sequence b, query head h), one thread per
// channel.  Every thread reads the partials' (max, weight) pairs itself
// (broadcast loads) along with its channel of their O, eight partials per
// round, so a sequence with at most eight partials costs one memory round and
// no barrier; further rounds rescale the running sums to the new maximum.
// Partial 0 always holds key 0, so the maximum is finite after the first round
// and the weight sum is >= 1.
template <int D>
__global__ __launch_bounds__(D) void attn_decode_merge_kernel(AttnArgs a) {
  constexpr int PSTRIDE = D + 2, CH = 8;
  const Dims& dm = a.dm;
  const int h = blockIdx.x, b = blockIdx.y;
  const int off_b = a.pos.off[b], nsplit = a.pos.off[b + 1] - off_b;
  const int t = threadIdx.x;
  const float* part = a.part + ((long)off_b * dm.Hq + (long)h * nsplit) * PSTRIDE;
  float m = -INFINITY, l = 0.0f, o = 0.0f;
  for (int c0 = 0; c0 < nsplit; c0 += CH) {
    float mc[CH], lc[CH], oc[CH];
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const float* p = part + (long)min(c0 + i, nsplit - 1) * PSTRIDE;
      mc[i] = p[D];
      lc[i] = p[D + 1];
      oc[i] = p[t];
    }
    float mn = m;
#pragma unroll
    for (int i = 0; i < CH; ++i)
      if (c0 + i < nsplit) mn = fmaxf(mn, mc[i]);
    if (c0 > 0) {
      const float sc = __builtin_amdgcn_exp2f(m - mn);
      l *= sc;
      o *= sc;
    }
    // weight 0 for the clamped repeats past nsplit (finite partials), so every
    // load is used unconditionally and all of them go out together
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const float wc = c0 + i >= nsplit || mc[i] == -INFINITY ? 0.0f
                                                              : __builtin_amdgcn_exp2f(mc[i] - mn);
      l = fmaf(lc[i], wc, l);
      o = fmaf(oc[i], wc, o);
    }
    m = mn;
  }
  reinterpret_cast<bf16*>(a.o)[((long)b * dm.Hq + h) * D + t] = (bf16)(o / l);
}

}  // namespace

// Work-groups per (sequence, KV head): about TARGET_WGS in all, shared in
// proportion to the sequences' 32-key block counts, at least one, at most one
// wave per block and MAX_SPLIT.  Equal lengths give every sequence
// TARGET_WGS / (B Hkv).
int decode_splits(const Dims& dm, int B, DecodePos& pos) {
  long total_blk = 0;
  for (int b = 0; b < B; ++b) total_blk += (pos.p[b] + 1 + 31) / 32;
  pos.off[0] = 0;
  for (int b = 0; b < B; ++b) {
    const long nb = (pos.p[b] + 1 + 31) / 32;
    const long share = (long)(TARGET_WGS / dm.Hkv) * nb / std::max(1L, total_blk);
    const int ns = (int)std::max(1L, std::min({share, nb / NW, (long)MAX_SPLIT}));
    pos.off[b + 1] = pos.off[b] + ns;
  }
  return pos.off[B];
}

// Partials: at most TARGET_WGS / Hkv + B split work-groups per KV head (the
// shares sum to at most the first term, the one-per-sequence floor adds B).
size_t decode_part_floats(const Dims& dm, int B) {
  return fast_decode(dm)
             ? (size_t)(TARGET_WGS / dm.Hkv + B) * dm.Hq * pstride(dm)
             : 0;
}

namespace {
template <int D>
void launch_decode_d(const AttnArgs& a, hipStream_t s) {
  const dim3 grid(a.nsplit, a.dm.Hkv);
  if (a.dm.G <= 1)
    hipLaunchKernelGGL((attn_decode_split_kernel<D, 1>), grid, dim3(256), 0, s, a);
  else if (a.dm.G <= 2)
    hipLaunchKernelGGL((attn_decode_split_kernel<D, 2>), grid, dim3(256), 0, s, a);
  else if (a.dm.G <= 4)
    hipLaunchKernelGGL((attn_decode_split_kernel<D, 4>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((attn_decode_split_kernel<D, 8>), grid, dim3(256), 0, s, a);
  hipLaunchKernelGGL(attn_decode_merge_kernel<D>, dim3(a.dm.Hq, a.B), dim3(D), 0, s, a);
}
}  // namespace

hipError_t launch_attn_decode(const AttnArgs& a, hipStream_t s) {
  if (!fast_decode(a.dm)) return launch_attn_fwd(a, s);
  // a.nsplit: the flattened split count, pos.off[B]
  if (a.part == nullptr || a.nsplit < a.B || a.nsplit != a.pos.off[a.B] ||
      a.nsplit > TARGET_WGS / a.dm.Hkv + a.B)
    return hipErrorInvalidValue;
  if (a.dm.d == 128)
    launch_decode_d<128>(a, s);
  else
    launch_decode_d<64>(a, s);
  return hipGetLastError();
}

}  // namespace cca
