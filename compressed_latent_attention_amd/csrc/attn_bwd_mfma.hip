// cca_bwd, attention part, bf16 with d = 128 (CCA-es §4, training backward;
// CCA-fr §4 "Rétropropagation"): gradients of causal softmax attention on the
// latent heads, recompute-style (P is never stored):
//   P = exp(Q K^T / sqrt(d) - lse),  D_t = <dO_t, O_t>,
//   dV = P^T dO,  dS = P * (dO V^T - D),  dQ = dS K / sqrt(d),  dK = dS^T Q / sqrt(d),
// with dK and dV of a KV head summed over its G query heads.
//
// Three kernels, no atomics (every sum has a fixed order, so results are
// run-to-run identical):
//   prep  — Q''^T, K''^T, dO^T (channel-major copies, rows padded to s_pad) and
//           D = rowsum(dO * O) from the saved fp32 O;
//   dkdv  — work-group = 128 keys of one KV head, 4 waves of 32 keys; loops over
//           the query blocks (32 queries) of every head of the group; two
//           work-groups share each key block's query range (first and second
//           half, the second writing to scratch that a small kernel adds in),
//           so that the causal triangle spreads over twice as many CUs:
//             S = Q K^T, dP = dO V^T (A = Q / dO rows from LDS, B = the wave's
//             K / V rows held in registers; S starts at -inf for the causally
//             masked pairs of diagonal steps, so exp2 needs no per-element
//             test), P and dS in registers, then
//             dV += P^T dO and dK += dS^T Q (A = P^T / dS^T straight from the
//             accumulators, B = dO^T / Q^T columns from LDS);
//   dq    — work-group = 128 queries of one head, 4 waves of 32 queries; loops
//           over the key blocks (32 keys) up to the diagonal:
//             S^T = K Q^T, dP^T = V dO^T (B = the wave's Q / dO held in
//             registers), dQ += dS K (B = K^T columns from LDS).
// S and dP use v_mfma_f32_32x32x16_bf16 on the stored bf16 tensors; dV, dK and
// dQ use v_mfma_f32_32x32x16_f16: P and dS are rounded to fp16 (11 significant
// bits), and the transposed copies of Q'', K'' and dO are written in fp16
// (exact for bf16 values in fp16's normal range).  dS = P (dP - D) has rows
// that sum to zero, so dQ and dK cancel heavily; bf16 dS (8 bits) would cost
// ~1% in them.  fp32 accumulation throughout.  The A
// rows of S (queries in dkdv, keys in dq) are read with bits 2 and 3 of the
// row index swapped, so that the 8 accumulator registers a lane passes on
// cover 8 consecutive queries (keys) and P / dS feed the next MFMA without a
// shuffle.  Tiles are staged through registers into padded LDS rows
// (conflict-free 16-byte reads), with one barrier per step.
#include "cca_internal.h"

namespace cca {
namespace {

constexpr int D = 128;
constexpr int NLD = D + 8;      // natural tile row stride (elements), 272 B
constexpr int TB = 32;          // tokens per step
constexpr int TLD = TB + 8;     // transposed tile row stride (elements), 80 B
constexpr float kLog2e = 1.44269504088896340736f;

typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

bool mfma_bwd(const Dims& dm) { return dm.bf16 && dm.d == D; }

__device__ __forceinline__ int perm_row(int i) {   // swap bits 2 and 3
  return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1);
}

__device__ __forceinline__ bf16x8 zero8() {
  bf16x8 z;
#pragma unroll
  for (int e = 0; e < 8; ++e) z[e] = (bf16)0.0f;
  return z;
}

__device__ __forceinline__ f16x8 to_f16(const bf16x8& v) {
  f16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (f16)(float)v[e];
  return r;
}

// ------------------------------------------------------------------ prep
// Tile of 64 tokens x 128 channels of one head: transpose through LDS.
// blockIdx.y: 0..Hq-1 -> Q''^T and dO^T of head y (and D); Hq.. -> K''^T.
__global__ __launch_bounds__(256) void bwd_prep_kernel(AttnBwdArgs a) {
  __shared__ bf16 tq[64][D + 2];
  __shared__ bf16 tdo[64][D + 2];
  const Dims& dm = a.dm;
  const int S = a.S, sp = a.s_pad;
  const int t0 = blockIdx.x * 64, y = blockIdx.y, b = blockIdx.z;
  const bool is_q = y < dm.Hq;
  const int h = is_q ? y : y - dm.Hq;
  const bf16* src = is_q ? reinterpret_cast<const bf16*>(a.q) + ((long)(b * dm.Hq + h) * S) * D
                         : reinterpret_cast<const bf16*>(a.k) + ((long)(b * dm.Hkv + h) * S) * D;
  const bf16* dob = reinterpret_cast<const bf16*>(a.dO) + (long)b * S * dm.nq + h * D;
  // load: thread -> (row, 8 channels)
  for (int f = threadIdx.x; f < 64 * (D / 8); f += 256) {
    const int r = f / (D / 8), c = (f % (D / 8)) * 8;
    const int t = t0 + r;
    bf16x8 v = zero8(), w = zero8();
    if (t < S) {
      v = *reinterpret_cast<const bf16x8*>(src + (long)t * D + c);
      if (is_q) w = *reinterpret_cast<const bf16x8*>(dob + (long)t * dm.nq + c);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      tq[r][c + e] = v[e];
      tdo[r][c + e] = w[e];
    }
  }
  // D_t = <dO_t, O_t> in fp32 (one wave per 16 tokens, 4 lanes per token... 64
  // tokens x 128 channels: each thread sums 32 channels of one token)
  if (is_q) {
    const int r = threadIdx.x >> 2, part = threadIdx.x & 3;
    const int t = t0 + r;
    float sacc = 0.0f;
    if (t < S) {
      const float* orow = a.o32 + ((long)(b * S + t) * dm.Hq + h) * D + part * 32;
      const bf16* drow = dob + (long)t * dm.nq + part * 32;
#pragma unroll 8
      for (int c = 0; c < 32; ++c) sacc = fmaf((float)drow[c], orow[c], sacc);
    }
    sacc += __shfl_xor(sacc, 1);
    sacc += __shfl_xor(sacc, 2);
    if (part == 0 && t < S) a.Dsum[(long)(b * dm.Hq + h) * S + t] = sacc;
  }
  __syncthreads();
  // store: thread -> (channel, 8 tokens); tokens past S are zero (tile zeroed)
  f16* dstq = reinterpret_cast<f16*>(is_q ? a.qT : a.kT) +
              ((long)(b * (is_q ? dm.Hq : dm.Hkv) + h) * D) * sp;
  f16* dstd = reinterpret_cast<f16*>(a.dOT) + ((long)(b * dm.Hq + h) * D) * sp;
  for (int f = threadIdx.x; f < D * 8; f += 256) {
    const int c = f / 8, r = (f % 8) * 8;
    if (t0 + r >= sp) continue;
    bf16x8 v, w;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      v[e] = tq[r + e][c];
      w[e] = tdo[r + e][c];
    }
    *reinterpret_cast<f16x8*>(dstq + (long)c * sp + t0 + r) = to_f16(v);
    if (is_q) *reinterpret_cast<f16x8*>(dstd + (long)c * sp + t0 + r) = to_f16(w);
  }
}

// ------------------------------------------------------------------ dkdv
struct DkdvStage {
  bf16 qn[TB * NLD];     // Q rows      [32 q][128 c]
  bf16 don[TB * NLD];    // dO rows     [32 q][128 c]
  f16 qt[D * TLD];       // Q^T         [128 c][32 q], fp16
  f16 dot[D * TLD];      // dO^T        [128 c][32 q], fp16
  float lse2[TB];        // lse * log2(e); +inf past the sequence
  float dsum[TB];
};

struct DkdvRegs {
  bf16x8 qn[2], don[2];
  f16x8 qt[2], dot[2];
  float lse2, dsum;
};

// Registers of one step: buffer loads whose resources end at row S - 1, so rows
// past the sequence read as zero without a branch (the loop body stays one
// block); lse of a query past S becomes +inf (its P is zero).
__device__ __forceinline__ void dkdv_load(const AttnBwdArgs& a, int b, int h, int q0, int t,
                                          DkdvRegs& r) {
  const Dims& dm = a.dm;
  const int S = a.S;
  const bf16* qb = reinterpret_cast<const bf16*>(a.q) + ((long)(b * dm.Hq + h) * S) * D;
  const bf16* dob = reinterpret_cast<const bf16*>(a.dO) + (long)b * S * dm.nq + h * D;
  const f16* qtb = reinterpret_cast<const f16*>(a.qT) + ((long)(b * dm.Hq + h) * D) * a.s_pad;
  const f16* dtb = reinterpret_cast<const f16*>(a.dOT) + ((long)(b * dm.Hq + h) * D) * a.s_pad;
  const __amdgpu_buffer_rsrc_t qrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)qb, 0, S * D * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t drs =
      __builtin_amdgcn_make_buffer_rsrc((void*)dob, 0, ((S - 1) * dm.nq + D) * 2, 0x00020000);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int f = t + 256 * i;
    const int row = f >> 4, ch = (f & 15) * 8;           // natural: 32 rows x 16 chunks
    const int q = q0 + row;
    r.qn[i] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(qrs, (q * D + ch) * 2, 0, 0));
    r.don[i] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(drs, (q * dm.nq + ch) * 2, 0, 0));
    const int c = f >> 2, col = (f & 3) * 8;             // transposed: 128 rows x 4 chunks
    r.qt[i] = *reinterpret_cast<const f16x8*>(qtb + (long)c * a.s_pad + q0 + col);
    r.dot[i] = *reinterpret_cast<const f16x8*>(dtb + (long)c * a.s_pad + q0 + col);
  }
  // every thread loads query q0 + t % 32 (the stage stores the 32 values from
  // all waves: the same value to the same address)
  const int q = q0 + (t & (TB - 1));
  const __amdgpu_buffer_rsrc_t lrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.lse + (long)(b * dm.Hq + h) * S), 0, S * 4, 0x00020000);
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.Dsum + (long)(b * dm.Hq + h) * S), 0, S * 4, 0x00020000);
  const float lv = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(lrs, q * 4, 0, 0));
  r.dsum = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(srs, q * 4, 0, 0));
  r.lse2 = fmaf(lv, kLog2e, q < S ? 0.0f : INFINITY);
}

__device__ __forceinline__ void dkdv_store(DkdvStage& st, int t, const DkdvRegs& r) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int f = t + 256 * i;
    const int row = f >> 4, ch = (f & 15) * 8;
    *reinterpret_cast<bf16x8*>(st.qn + row * NLD + ch) = r.qn[i];
    *reinterpret_cast<bf16x8*>(st.don + row * NLD + ch) = r.don[i];
    const int c = f >> 2, col = (f & 3) * 8;
    *reinterpret_cast<f16x8*>(st.qt + c * TLD + col) = r.qt[i];
    *reinterpret_cast<f16x8*>(st.dot + c * TLD + col) = r.dot[i];
  }
  st.lse2[t & (TB - 1)] = r.lse2;
  st.dsum[t & (TB - 1)] = r.dsum;
}

// S = Q K^T and dP = dO V^T of one step: the stage's Q / dO rows (A, read with
// the permuted row so that P / dS come out as 8 consecutive queries per lane)
// times the wave's K / V rows held in registers (B).
// S starts from `sinit` (0, or -inf where a key follows a query: the causal
// mask, so that exp2 gives P = 0 there without a per-element test).
__device__ __forceinline__ void dkdv_sdp(const DkdvStage& st, const bf16x8 (&kf)[8],
                                         const bf16x8 (&vf)[8], int prow, int hi,
                                         const f32x16& sinit, f32x16& sacc, f32x16& pacc) {
  sacc = sinit;
#pragma unroll
  for (int r = 0; r < 16; ++r) pacc[r] = 0.0f;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    const bf16x8 qa = *reinterpret_cast<const bf16x8*>(st.qn + prow * NLD + ks * 16 + hi * 8);
    const bf16x8 da = *reinterpret_cast<const bf16x8*>(st.don + prow * NLD + ks * 16 + hi * 8);
    sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[ks], sacc, 0, 0, 0);
    pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da, vf[ks], pacc, 0, 0, 0);
  }
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_dkdv_kernel(AttnBwdArgs a) {
  __shared__ __attribute__((aligned(16))) DkdvStage stg[3];
  const Dims& dm = a.dm;
  const int S = a.S, G = dm.G;
  // two work-groups per key block, each taking half of its query blocks (the
  // first half holds the diagonal); low blocks = most work, dispatched first
  const int part = blockIdx.x & 1;
  const int k0 = (blockIdx.x >> 1) * 128, g = blockIdx.y, b = blockIdx.z;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int kw0 = k0 + wave * 32;
  const int my_key = kw0 + l32;
  const float c1 = kLog2e / sqrtf((float)D);

  // B operands for S = Q K^T and dP = dO V^T: lane (key l32, hi) holds channels
  // 16 ks + 8 hi + 0..7 of its key's K'' and V' rows.
  bf16x8 kf[8], vf[8];
  {
    const bf16* kb = reinterpret_cast<const bf16*>(a.k) + ((long)(b * dm.Hkv + g) * S) * D;
    const bf16* vb = reinterpret_cast<const bf16*>(a.v) + ((long)(b * dm.Hkv + g) * S) * D;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      kf[ks] = my_key < S ? *reinterpret_cast<const bf16x8*>(kb + (long)my_key * D + ks * 16 + hi * 8)
                          : zero8();
      vf[ks] = my_key < S ? *reinterpret_cast<const bf16x8*>(vb + (long)my_key * D + ks * 16 + hi * 8)
                          : zero8();
    }
  }
  f32x16 dk[4], dv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) dk[i][r] = dv[i][r] = 0.0f;

  // steps: (head hh of the group, query block) for this part's query blocks
  const int nqb_all = (S + TB - 1) / TB - k0 / TB;
  const int nfirst = (nqb_all + 1) / 2;
  const int qb0 = k0 / TB + (part ? nfirst : 0);
  const int nqb = part ? nqb_all - nfirst : nfirst;
  const int nsteps = G * nqb;
  const int prow = perm_row(l32);
  // Steps run head-major: step s = (head s / nqb, query block s % nqb).  The
  // current step's block and the loaded step's (head, block) advance by
  // counters (a division per step would cost ~40 scalar instructions in every
  // wave); the loaded step stops at the last one, so the pipeline's loads past
  // the end repeat it into a stage nobody reads again.
  int cur_qi = 0;                                   // block index of step s
  int ld_s = min(3, nsteps - 1);                    // step loaded next (s + 3, clamped)
  int ld_h = ld_s / max(nqb, 1), ld_qi = ld_s - ld_h * nqb;
  auto advance_load = [&]() {
    if (ld_s < nsteps - 1) {
      ++ld_s;
      if (++ld_qi == nqb) {
        ld_qi = 0;
        ++ld_h;
      }
    }
  };

  // Software pipeline over three LDS stages (step s in stage s % 3).  Iteration
  // s computes S and dP of step s + 1 and the softmax of step s in one block
  // (the MFMAs run while the vector ALU exponentiates), then dV and dK of step
  // s; it stores the registers of step s + 2 into the stage step s - 1 used and
  // loads step s + 3 into registers.  A barrier per step waits only for LDS
  // operations, so the global loads stay in flight across it.  Steps whose
  // queries all precede the wave's keys are computed like the others: their P
  // is exactly zero.
  if (nsteps > 0) {
    DkdvRegs pre;
    // steps 0, 1, 2 (clamped): the few divisions happen once
    for (int i = 0; i < 3; ++i) {
      const int si = min(i, nsteps - 1), hi_ = si / nqb;
      dkdv_load(a, b, g * G + hi_, (qb0 + si - hi_ * nqb) * TB, t, pre);
      if (i < 2) dkdv_store(stg[i], t, pre);
    }
    __syncthreads();
    // initial S of a step: -inf where the wave's key follows the query (only
    // the steps whose queries reach below the wave's last key have any)
    // lane (key l32, hi): register r is query q0 + 16 (r / 8) + 8 hi + r % 8
    auto s_init = [&](int q0n, f32x16& si) {
      if (q0n < kw0 + 31) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          si[r] = my_key > q0n + 16 * (r >> 3) + 8 * hi + (r & 7) ? -INFINITY : 0.0f;
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) si[r] = 0.0f;
      }
    };
    f32x16 sacc, pacc, sinit;
    s_init(qb0 * TB, sinit);
    dkdv_sdp(stg[0], kf, vf, prow, hi, sinit, sacc, pacc);

    for (int s = 0; s < nsteps; ++s) {
      const DkdvStage& st = stg[s % 3];
      const int q0 = (qb0 + cur_qi) * TB;
      if (++cur_qi == nqb) cur_qi = 0;
      dkdv_store(stg[(s + 2) % 3], t, pre);
      dkdv_load(a, b, g * G + ld_h, (qb0 + ld_qi) * TB, t, pre);
      advance_load();
      f32x16 sn, pn;
      s_init((qb0 + cur_qi) * TB, sinit);           // step s + 1's block (cur_qi has advanced)
      dkdv_sdp(stg[(s + 1) % 3], kf, vf, prow, hi, sinit, sn, pn);
      // lane (key l32, hi): register r is query q0 + 16 (r / 8) + 8 hi + r % 8
      f16x8 pf[2], sf[2];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int qi = 16 * half + 8 * hi;
        const f32x4 l0 = *reinterpret_cast<const f32x4*>(st.lse2 + qi);
        const f32x4 l1 = *reinterpret_cast<const f32x4*>(st.lse2 + qi + 4);
        const f32x4 d0 = *reinterpret_cast<const f32x4*>(st.dsum + qi);
        const f32x4 d1 = *reinterpret_cast<const f32x4*>(st.dsum + qi + 4);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = 8 * half + e;
          const float lse2 = e < 4 ? l0[e] : l1[e - 4];
          const float dsm = e < 4 ? d0[e] : d1[e - 4];

          // masked pairs have S = -inf and queries past S lse2 = +inf: P = 0
          const float p = __builtin_amdgcn_exp2f(fmaf(sacc[r], c1, -lse2));
          pf[half][e] = (f16)p;
          sf[half][e] = (f16)(p * (pacc[r] - dsm));
        }
      }
      // dV += P^T dO, dK += dS^T Q: 4 channel blocks x 2 steps of 16 queries
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const int c = nb * 32 + l32;
          const f16x8 db = *reinterpret_cast<const f16x8*>(st.dot + c * TLD + ks * 16 + hi * 8);
          const f16x8 qbv = *reinterpret_cast<const f16x8*>(st.qt + c * TLD + ks * 16 + hi * 8);
          dv[nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(pf[ks], db, dv[nb], 0, 0, 0);
          dk[nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(sf[ks], qbv, dk[nb], 0, 0, 0);
        }
      sacc = sn;
      pacc = pn;
      __builtin_amdgcn_s_waitcnt(0xC07F);      // this wave's LDS reads and stores are done
      __builtin_amdgcn_s_barrier();
    }
  }

  // D layout: lane holds channel nb*32 + l32, key rows 8 (r/4) + 4 hi + r%4
  const float inv = 1.0f / sqrtf((float)D);
  float* dkb = (part ? a.dk2 : a.dk) + ((long)(b * dm.Hkv + g) * S) * D;
  float* dvb = (part ? a.dv2 : a.dv) + ((long)(b * dm.Hkv + g) * S) * D;
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = kw0 + 8 * (r >> 2) + 4 * hi + (r & 3);
      if (key < S) {
        dkb[(long)key * D + nb * 32 + l32] = dk[nb][r] * inv;
        dvb[(long)key * D + nb * 32 + l32] = dv[nb][r];
      }
    }
}

// dk += dk2, dv += dv2: the two halves of every key block, in a fixed order.
__global__ __launch_bounds__(256) void bwd_dkdv_sum_kernel(float* dk, const float* dk2, float* dv,
                                                           const float* dv2, long n4) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  reinterpret_cast<f32x4*>(dk)[i] += reinterpret_cast<const f32x4*>(dk2)[i];
  reinterpret_cast<f32x4*>(dv)[i] += reinterpret_cast<const f32x4*>(dv2)[i];
}

// ------------------------------------------------------------------ dq
struct DqStage {
  bf16 kn[TB * NLD];     // K rows   [32 keys][128 c]
  bf16 vn[TB * NLD];     // V rows   [32 keys][128 c]
  f16 kt[D * TLD];       // K^T      [128 c][32 keys], fp16
};

struct DqRegs {
  bf16x8 kn[2], vn[2];
  f16x8 kt[2];
};

__device__ __forceinline__ void dq_load(const AttnBwdArgs& a, int b, int g, int j0, int t,
                                        DqRegs& r) {
  const Dims& dm = a.dm;
  const int S = a.S;
  const bf16* kb = reinterpret_cast<const bf16*>(a.k) + ((long)(b * dm.Hkv + g) * S) * D;
  const bf16* vb = reinterpret_cast<const bf16*>(a.v) + ((long)(b * dm.Hkv + g) * S) * D;
  const f16* ktb = reinterpret_cast<const f16*>(a.kT) + ((long)(b * dm.Hkv + g) * D) * a.s_pad;
  // K and V rows through resources that end at row S - 1: rows past it read as
  // zero without a branch, so the six loads of a thread issue back to back
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)kb, 0, S * D * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)vb, 0, S * D * 2, 0x00020000);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int f = t + 256 * i;
    const int row = f >> 4, ch = (f & 15) * 8;
    const int j = j0 + row;
    r.kn[i] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(krs, (j * D + ch) * 2, 0, 0));
    r.vn[i] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(vrs, (j * D + ch) * 2, 0, 0));
    const int c = f >> 2, col = (f & 3) * 8;
    r.kt[i] = *reinterpret_cast<const f16x8*>(ktb + (long)c * a.s_pad + j0 + col);
  }
}

__device__ __forceinline__ void dq_store(DqStage& st, int t, const DqRegs& r) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int f = t + 256 * i;
    const int row = f >> 4, ch = (f & 15) * 8;
    *reinterpret_cast<bf16x8*>(st.kn + row * NLD + ch) = r.kn[i];
    *reinterpret_cast<bf16x8*>(st.vn + row * NLD + ch) = r.vn[i];
    const int c = f >> 2, col = (f & 3) * 8;
    *reinterpret_cast<f16x8*>(st.kt + c * TLD + col) = r.kt[i];
  }
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dq_kernel(AttnBwdArgs a) {
  __shared__ __attribute__((aligned(16))) DqStage stg[2];
  const Dims& dm = a.dm;
  const int S = a.S;
  const int nqb = (S + 127) / 128;
  const int per = dm.Hq * a.B;
  const int qb = nqb - 1 - (int)(blockIdx.x / per);          // heaviest blocks first
  const int h = (blockIdx.x % per) % dm.Hq, b = (blockIdx.x % per) / dm.Hq;
  const int g = h / dm.G;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int q0 = qb * 128;
  const int qw0 = q0 + wave * 32;
  const int my_q = qw0 + l32;
  const float c1 = kLog2e / sqrtf((float)D);

  // B operands for S^T = K Q^T and dP^T = V dO^T: lane (query l32, hi) holds
  // channels 16 ks + 8 hi + 0..7 of its query's Q'' and dO rows.
  bf16x8 qf[8], df[8];
  {
    const bf16* qbp = reinterpret_cast<const bf16*>(a.q) + ((long)(b * dm.Hq + h) * S) * D;
    const bf16* dob = reinterpret_cast<const bf16*>(a.dO) + (long)b * S * dm.nq + h * D;
    // rows past S read as zero through the resources' range check
    const __amdgpu_buffer_rsrc_t qrs =
        __builtin_amdgcn_make_buffer_rsrc((void*)qbp, 0, S * D * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t drs =
        __builtin_amdgcn_make_buffer_rsrc((void*)dob, 0, ((S - 1) * dm.nq + D) * 2, 0x00020000);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      qf[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                              qrs, (my_q * D + ks * 16 + hi * 8) * 2, 0, 0));
      df[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                              drs, (my_q * dm.nq + ks * 16 + hi * 8) * 2, 0, 0));
    }
  }
  const float lse2 = my_q < S ? a.lse[(long)(b * dm.Hq + h) * S + my_q] * kLog2e : INFINITY;
  const float dsm = my_q < S ? a.Dsum[(long)(b * dm.Hq + h) * S + my_q] : 0.0f;
  f32x16 dq[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[i][r] = 0.0f;

  const int q_last = min(S, q0 + 128) - 1;
  const int nsteps = q_last / TB + 1;
  const int prow = perm_row(l32);
  DqRegs pre;
  dq_load(a, b, g, 0, t, pre);
  dq_store(stg[0], t, pre);
  if (nsteps > 1) dq_load(a, b, g, TB, t, pre);
  __syncthreads();

  for (int s = 0; s < nsteps; ++s) {
    const DqStage& st = stg[s & 1];
    const int j0 = s * TB;
    if (j0 <= qw0 + 31) {                    // else every key follows every query of the wave
      f32x16 sacc, pacc;
#pragma unroll
      for (int r = 0; r < 16; ++r) pacc[r] = 0.0f;
      // S^T starts at -inf where the key follows the lane's query (only the
      // steps whose keys reach past the wave's first query have any), so exp2
      // gives P = 0 there without a per-element test.  Lane (query l32, hi):
      // register r is key j0 + 16 (r / 8) + 8 hi + r % 8.
      if (j0 + 31 > qw0) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          sacc[r] = j0 + 16 * (r >> 3) + 8 * hi + (r & 7) > my_q ? -INFINITY : 0.0f;
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[r] = 0.0f;
      }
      // K and V fragments through a ring of 4: the reads run 4 k slices ahead
      // of the MFMAs instead of one read-wait-MFMA per slice
      bf16x8 ka[4], va[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        ka[ks] = *reinterpret_cast<const bf16x8*>(st.kn + prow * NLD + ks * 16 + hi * 8);
        va[ks] = *reinterpret_cast<const bf16x8*>(st.vn + prow * NLD + ks * 16 + hi * 8);
      }
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks & 3], qf[ks], sacc, 0, 0, 0);
        pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[ks & 3], df[ks], pacc, 0, 0, 0);
        if (ks + 4 < 8) {
          ka[ks & 3] = *reinterpret_cast<const bf16x8*>(st.kn + prow * NLD + (ks + 4) * 16 + hi * 8);
          va[ks & 3] = *reinterpret_cast<const bf16x8*>(st.vn + prow * NLD + (ks + 4) * 16 + hi * 8);
        }
      }
      // K^T fragments of dQ += dS K, read before the softmax arithmetic covers them
      f16x8 kt[2][4];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          kt[ks][nb] = *reinterpret_cast<const f16x8*>(st.kt + (nb * 32 + l32) * TLD + ks * 16 + hi * 8);
      // lane (query l32, hi): register r is key j0 + 16 (r / 8) + 8 hi + r % 8
      f16x8 sf[2];
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = 8 * half + e;
          const float p = __builtin_amdgcn_exp2f(fmaf(sacc[r], c1, -lse2));
          sf[half][e] = (f16)(p * (pacc[r] - dsm));
        }
      // dQ += dS K: A = dS (lane = query row), B = K^T columns
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          dq[nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(sf[ks], kt[ks][nb], dq[nb], 0, 0, 0);
    }
    if (s + 1 < nsteps) {
      dq_store(stg[(s + 1) & 1], t, pre);
      if (s + 2 < nsteps) dq_load(a, b, g, (s + 2) * TB, t, pre);
    }
    __syncthreads();
  }

  // D layout: lane holds channel nb*32 + l32, query rows 8 (r/4) + 4 hi + r%4
  const float inv = 1.0f / sqrtf((float)D);
  float* dqb = a.dq + ((long)(b * dm.Hq + h) * S) * D;
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int q = qw0 + 8 * (r >> 2) + 4 * hi + (r & 3);
      if (q < S) dqb[(long)q * D + nb * 32 + l32] = dq[nb][r] * inv;
    }
}

}  // namespace

bool attn_bwd_mfma_supported(const Dims& dm) { return mfma_bwd(dm); }

size_t attn_bwd_transpose_bytes(const Dims& dm, int B, int S) {
  if (!mfma_bwd(dm)) return 0;
  const size_t sp = (size_t)(S + 63) / 64 * 64;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  return al((size_t)B * dm.nq * sp * 2) + al((size_t)B * dm.nk * sp * 2) +
         al((size_t)B * dm.nq * sp * 2) + 2 * al((size_t)B * S * dm.nk * 4);
}

hipError_t launch_attn_bwd_mfma(const AttnBwdArgs& a, hipStream_t s) {
  const Dims& dm = a.dm;
  if (!mfma_bwd(dm) || !a.qT || !a.kT || !a.dOT || a.s_pad < a.S || a.s_pad % 64 != 0)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(bwd_prep_kernel, dim3(a.s_pad / 64, dm.Hq + dm.Hkv, a.B), dim3(256), 0, s,
                     a);
  if (!a.dk2 || !a.dv2) return hipErrorInvalidValue;
  hipLaunchKernelGGL(bwd_dkdv_kernel, dim3(2 * ((a.S + 127) / 128), dm.Hkv, a.B), dim3(256), 0, s,
                     a);
  if (!a.sum_by_consumer) {
    const long n4 = (long)a.B * dm.Hkv * a.S * D / 4;
    hipLaunchKernelGGL(bwd_dkdv_sum_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s,
                       a.dk, a.dk2, a.dv, a.dv2, n4);
  }
  hipLaunchKernelGGL(bwd_dq_kernel, dim3(((a.S + 127) / 128) * dm.Hq * a.B), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace cca
