// cca_bwd, attention part, bf16 with d = 128 or 64 (CCA-es §4, training backward;
// CCA-fr §4 "Rétropropagation"): gradients of causal softmax attention on the
// latent heads, recompute-style (P is never stored):
//   P = exp(Q K^T / sqrt(d) - lse),  D_t = <dO_t, O_t>,
//   dV = P^T dO,  dS = P * (dO V^T - D),  dQ = dS K / sqrt(d),  dK = dS^T Q / sqrt(d),
// with dK and dV of a KV head summed over its G query heads.
//
// Three kernels, no atomics (every sum has a fixed order, so results are
// run-to-run identical):
//   prep  — fp16 copies of Q'', K'', V' and dO as head-major rows (zero from
//           row S to s_pad) and D = rowsum(dO * O) from the saved fp32 O;
//   dkdv  — work-group = 128 keys of one KV group, 8 waves.  Producers (waves
//           0-3, 32 keys each, K and V rows in registers) compute S = Q K^T and
//           dP = dO V^T, the softmax, dS and dK += dS^T Q, and leave P in LDS;
//           consumers (waves 4-7, wave w + 4 on the SIMD of wave w) stage the
//           Q / dO tiles into LDS and add dV += P^T dO one step behind.  The two
//           waves of a SIMD overlap one's softmax with the other's MFMAs.  Two
//           or four work-groups per key block: each takes a half (a quarter,
//           when the group size is a multiple of 4) of the group's heads, or
//           with an odd group size half of each head's query range;
//           query blocks run in descending order, so the work-groups of a head
//           read the same tile at about the same time;
//   dq    — work-group = 128 queries of one head, 8 waves, looping over the keys
//           up to the diagonal, 64 per step (two 32-key blocks per barrier).  Producers (waves 0-3, 32
//           queries each, Q and dO rows in registers) compute S^T = K Q^T,
//           dP^T = V dO^T and dS; consumers stage the K / V tiles and add
//           dQ += dS K one step behind.
// Every product is a v_mfma_f32_32x32x16_f16 with fp32 accumulation.  The fp16
// copies of Q'', K'' and V' hold the stored bf16 values exactly while they lie
// in fp16's normal range (|x| in [2^-14, 65504]; below it a value keeps an
// absolute error under 2^-25).  dO is different: the upstream gradient of a
// loss averaged over many tokens is tiny (2^-20 and less), so its copy is
// taken as dO * 2^e with e chosen per call from max|dO| (an absmax pass before
// prep) to put that maximum in [4, 8).  D, dP, dS, dV, dQ and dK are all
// linear in dO and scale with it; the epilogues multiply by 2^-e.  Both
// scalings are exact, and dS = P (dP - D) stays in fp16's range for value rows
// of norm up to ~360.  P and dS are rounded to fp16 (11 significant bits).  dS = P (dP - D) has rows
// that sum to zero, so dQ and dK cancel heavily; bf16 dS (8 bits) would cost
// ~1% in them.  The transposed operands (Q^T and dO^T of dK and dV, K^T of dQ)
// are read from the natural LDS tiles with ds_read_b64_tr_b16, so only natural
// rows cross HBM.  The A rows of S (queries in dkdv, keys in dq) are read with
// bits 2 and 3 of the row index swapped, so that the 8 accumulator registers a
// lane passes on cover 8 consecutive queries (keys) and P / dS feed the next
// MFMA without a shuffle.
#include "cca_internal.h"

namespace cca {
namespace {

constexpr int TB = 32;          // tokens per step
constexpr int TROW = 160;       // LDS tile row stride, fp16 elements (320 B = 20 chunks of 16 B)
constexpr int TILE = TB * TROW; // one tile: 32 token rows of up to 128 channels
constexpr float kLog2e = 1.44269504088896340736f;

typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

bool mfma_bwd(const Dims& dm) { return dm.bf16 && (dm.d == 128 || dm.d == 64); }

// Counts that follow the head dimension D: 16-channel k-steps, 32-channel
// output blocks, 16-byte chunks per row.
template <int D>
struct BG {
  static constexpr int NKS = D / 16, NMB = D / 32, CPR = D / 8;
};

__device__ __forceinline__ int perm_row(int i) {   // swap bits 2 and 3
  return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1);
}

__device__ __forceinline__ f16x8 to_f16(const bf16x8& v) {
  f16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (f16)(float)v[e];
  return r;
}

// ------------------------------------------------------------------ LDS tiles
// A tile holds 32 token rows of D fp16 channels (the row stride is the same
// for D = 64, which uses the first 8 chunks); chunk ch (channels 8 ch ..
// 8 ch + 7) of row r sits at chunk ch ^ ((r >> 2) & 3) of a 20-chunk row.  The
// row stride (4 chunks past a multiple of 16) spreads the 4 rows of a
// transposing read over the 64 banks and the XOR spreads the 16 rows of an
// A-operand read, so the three access patterns below (A-operand rows, the
// transposing reads and the staging stores) are free of bank conflicts.
__device__ __forceinline__ int tile_off(int r, int ch) {
  return r * TROW + ((ch ^ ((r >> 2) & 3)) << 3);
}

// A operand of an MFMA over the channels: lane (row l32, hi) reads chunk
// 2 ks + hi of row perm_row(l32), at ao[ks & 1] + 32 (ks >> 1).
__device__ __forceinline__ void a_offsets(int prow, int hi, int (&ao)[2]) {
  ao[0] = tile_off(prow, hi);
  ao[1] = tile_off(prow, 2 + hi);
}

// B operand over the tokens (k = token rows, n = channels) straight from a
// natural tile: lane (n = l32, hi) needs rows 16 ks + 8 hi + 0..7 of column
// 32 nb + l32.  ds_read_b64_tr_b16 gives lane i of a 16-lane group, as its
// element j, element i & 3 of the 8 bytes addressed by lane (i >> 2) + 4 j of
// the group; so lane c of a group addresses row R + (c >> 2), columns
// C + 4 (c & 3) .. + 3, and lane i receives rows R .. R + 3 of column C + i.
// Two reads (R = 16 ks + 8 hi and R + 4) make the fragment; the lane's offsets
// are to[r] + 2560 ks + 32 nb.
__device__ __forceinline__ void t_offsets(int lane, int (&to)[2]) {
  const int c = lane & 15, g = (lane >> 4) & 1, hi = lane >> 5;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int row = 8 * hi + 4 * r + (c >> 2);
    const int chunk = 2 * g + ((c & 3) >> 1);
    to[r] = row * TROW + ((chunk ^ ((row >> 2) & 3)) << 3) + (c & 1) * 4;
  }
}

__device__ __forceinline__ f16x8 read_t(const f16* tile, const int (&to)[2], int ks, int nb) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)(tile + to[0] + 2560 * ks + 32 * nb));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)(tile + to[1] + 2560 * ks + 32 * nb));
  return __builtin_bit_cast(f16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ f16x8 read_a(const f16* tile, const int (&ao)[2], int ks) {
  return *reinterpret_cast<const f16x8*>(tile + ao[ks & 1] + 32 * (ks >> 1));
}

template <int D>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows16(const void* base, long row0, int nrows) {
  return __builtin_amdgcn_make_buffer_rsrc(
      (void*)(reinterpret_cast<const f16*>(base) + row0 * D), 0, nrows * D * 2, 0x00020000);
}

__device__ __forceinline__ f16x8 load16(const __amdgpu_buffer_rsrc_t& rs, int elem) {
  return __builtin_bit_cast(f16x8, __builtin_amdgcn_raw_buffer_load_b128(rs, elem * 2, 0, 0));
}

// Work-group barrier that waits only for this wave's LDS operations, so
// global loads stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ------------------------------------------------------------------ dO scale
// max|dO| over the whole [B*S, nq] tensor, per work-group (grid-stride over
// 16-byte chunks); prep combines the kAmaxParts partials.
__global__ __launch_bounds__(256) void bwd_do_absmax_kernel(const bf16* dO, long n8,
                                                            float* part) {
  __shared__ float red[4];
  float m = 0.0f;
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n8; i += (long)gridDim.x * 256) {
    const bf16x8 v = reinterpret_cast<const bf16x8*>(dO)[i];
#pragma unroll
    for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf((float)v[e]));
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) part[blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// 2^e with e such that m * 2^e lies in [4, 8) (1 for m = 0), clamped so both
// 2^e and 2^-e are normal fp32 numbers.
__device__ __forceinline__ int do_scale_exp(float m) {
  if (!(m > 0.0f)) return 0;
  int k;
  frexpf(m, &k);                       // m in [2^(k-1), 2^k)
  return min(max(3 - k, -120), 120);
}

// ------------------------------------------------------------------ prep
// 64 tokens of one head per work-group.  blockIdx.y: 0..Hq-1 -> Q'' and dO of
// head y (and D); Hq.. -> K'' and V' of KV head y - Hq.
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(AttnBwdArgs a) {
  constexpr int CPR = BG<D>::CPR, NI = 64 * CPR / 256;   // 16-byte chunks per thread and array
  const Dims& dm = a.dm;
  const int S = a.S, sp = a.s_pad;
  const int t0 = blockIdx.x * 64, y = blockIdx.y, b = blockIdx.z;
  const bool is_q = y < dm.Hq;
  const int h = is_q ? y : y - dm.Hq;
  const long hrow = (long)(b * (is_q ? dm.Hq : dm.Hkv) + h);
  const bf16* src0 = is_q ? reinterpret_cast<const bf16*>(a.q) + hrow * S * D
                          : reinterpret_cast<const bf16*>(a.k) + hrow * S * D;
  const bf16* src1 = is_q ? reinterpret_cast<const bf16*>(a.dO) + (long)b * S * dm.nq + h * D
                          : reinterpret_cast<const bf16*>(a.v) + hrow * S * D;
  const long ld1 = is_q ? dm.nq : D;
  f16* dst0 = reinterpret_cast<f16*>(is_q ? a.q16 : a.k16) + hrow * sp * D;
  f16* dst1 = reinterpret_cast<f16*>(is_q ? a.do16 : a.v16) + hrow * sp * D;
  // dO's scale 2^e from the absmax partials (every Q work-group reduces them
  // alike; the first one publishes 2^-e for the dK / dV and dQ epilogues)
  float dscale = 1.0f;
  if (is_q) {
    __shared__ float red[4];
    float m = a.amax_part[threadIdx.x];            // kAmaxParts == blockDim.x
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const int e = do_scale_exp(m);
    dscale = ldexpf(1.0f, e);
    if (blockIdx.x == 0 && y == 0 && b == 0 && threadIdx.x == 0) a.dscale[0] = ldexpf(1.0f, -e);
  }
  // thread -> (row, 8 channels), four rows apart; every load is issued before
  // the first store (the copies may not alias the sources as far as the
  // compiler knows, so a load-convert-store loop would run its four memory
  // round trips one after another).  The resources end at row S - 1: rows past
  // it read as zero, and are written as zero.
  const __amdgpu_buffer_rsrc_t rs0 =
      __builtin_amdgcn_make_buffer_rsrc((void*)src0, 0, S * D * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t rs1 =
      __builtin_amdgcn_make_buffer_rsrc((void*)src1, 0, (int)(((long)(S - 1) * ld1 + D) * 2),
                                        0x00020000);
  bf16x8 v[NI], w[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int f = threadIdx.x + 256 * i;
    const int t = t0 + f / CPR, c = (f % CPR) * 8;
    v[i] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rs0, (t * D + c) * 2, 0, 0));
    w[i] = __builtin_bit_cast(bf16x8,
                              __builtin_amdgcn_raw_buffer_load_b128(rs1, (int)((t * ld1 + c) * 2), 0, 0));
  }
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int f = threadIdx.x + 256 * i;
    const int t = t0 + f / CPR, c = (f % CPR) * 8;
    *reinterpret_cast<f16x8*>(dst0 + (long)t * D + c) = to_f16(v[i]);
    f16x8 o;                               // V' as stored, or dO * 2^e
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (f16)((float)w[i][e] * dscale);
    *reinterpret_cast<f16x8*>(dst1 + (long)t * D + c) = o;
  }
  // D_t = <dO_t, O_t> in fp32 from the dO chunks above and the same chunks of
  // O (fp32, rows past S read as zero): each thread's 8 channels, then a sum
  // over the CPR consecutive lanes that hold one token
  if (is_q) {
    const long orow0 = ((long)b * S * dm.Hq + h) * D;
    const int ldo = dm.Hq * D;
    const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.o32 + orow0), 0, ((S - 1) * ldo + D) * 4, 0x00020000);
    f32x4 ov[NI][2];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int f = threadIdx.x + 256 * i;
      const int t = t0 + f / CPR, c = (f % CPR) * 8;
      ov[i][0] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(ro, (t * ldo + c) * 4, 0, 0));
      ov[i][1] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(ro, (t * ldo + c + 4) * 4, 0, 0));
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int f = threadIdx.x + 256 * i;
      const int t = t0 + f / CPR;
      float sacc = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) sacc = fmaf((float)w[i][e], ov[i][e >> 2][e & 3], sacc);
#pragma unroll
      for (int off = 1; off < CPR; off <<= 1) sacc += __shfl_xor(sacc, off);
      if (f % CPR == 0 && t < S) a.Dsum[hrow * S + t] = sacc * dscale;
    }
  }
}

// ------------------------------------------------------------------ dkdv
struct DkdvStage {
  f16 q[TILE];           // Q'' rows of the step's 32 queries
  f16 dO[TILE];          // dO rows
  float lse2[TB];        // lse * log2(e); +inf past the sequence
  float dsum[TB];
};

struct DkdvSmem {
  DkdvStage stg[3];
  f16 pbuf[2][4][2 * 64 * 8];    // P of a step per producer: [parity][producer][ks][lane][8]
};

template <int D>
struct DkdvRegs {
  static constexpr int NL = TB * BG<D>::CPR / 256;   // 16-byte chunks per thread and tile
  f16x8 q[NL], dO[NL];
  float lse, dsum, pad;
};

// Registers of one step (thread tc of the 256 consumers): rows of the fp16
// copies (in range up to s_pad, so no test), lse / D of the step's queries
// through resources that end at row S - 1 (past it: lse +inf, so P = 0).
template <int D>
__device__ __forceinline__ void dkdv_load(const AttnBwdArgs& a, int b, int h, int q0, int tc,
                                          DkdvRegs<D>& r) {
  constexpr int CPR = BG<D>::CPR;
  const Dims& dm = a.dm;
  const int S = a.S;
  const long hrow = (long)(b * dm.Hq + h);
  const __amdgpu_buffer_rsrc_t qrs = rows16<D>(a.q16, hrow * a.s_pad, a.s_pad);
  const __amdgpu_buffer_rsrc_t drs = rows16<D>(a.do16, hrow * a.s_pad, a.s_pad);
#pragma unroll
  for (int i = 0; i < DkdvRegs<D>::NL; ++i) {
    const int f = tc + 256 * i;
    const int row = f / CPR, ch = (f % CPR) * 8;
    r.q[i] = load16(qrs, (q0 + row) * D + ch);
    r.dO[i] = load16(drs, (q0 + row) * D + ch);
  }
  const int q = q0 + (tc & (TB - 1));
  const __amdgpu_buffer_rsrc_t lrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.lse + hrow * S), 0, S * 4, 0x00020000);
  const __amdgpu_buffer_rsrc_t srs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.Dsum + hrow * S), 0, S * 4, 0x00020000);
  r.lse = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(lrs, q * 4, 0, 0));
  r.dsum = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(srs, q * 4, 0, 0));
  r.pad = q < S ? 0.0f : INFINITY;
}

template <int D>
__device__ __forceinline__ void dkdv_store(DkdvStage& st, int tc, const DkdvRegs<D>& r) {
#pragma unroll
  for (int i = 0; i < DkdvRegs<D>::NL; ++i) {
    const int f = tc + 256 * i;
    const int row = f / BG<D>::CPR, ch = f % BG<D>::CPR;
    *reinterpret_cast<f16x8*>(st.q + tile_off(row, ch)) = r.q[i];
    *reinterpret_cast<f16x8*>(st.dO + tile_off(row, ch)) = r.dO[i];
  }
  // every consumer wave stores the same 32 values (query tc % 32)
  st.lse2[tc & (TB - 1)] = fmaf(r.lse, kLog2e, r.pad);
  st.dsum[tc & (TB - 1)] = r.dsum;
}

template <int D>
__global__ __launch_bounds__(512) void bwd_dkdv_kernel(AttnBwdArgs a) {
  constexpr int NKS = BG<D>::NKS, NMB = BG<D>::NMB;
  __shared__ __attribute__((aligned(16))) DkdvSmem sm;
  const Dims& dm = a.dm;
  const int S = a.S, G = dm.G;
  const int nparts = dm.G % 4 == 0 ? 4 : 2;          // work-groups per key block
  const int part = blockIdx.x % nparts;
  const int k0 = (int)(blockIdx.x / nparts) * 128, g = blockIdx.y, b = blockIdx.z;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int pair = wave & 3;
  const int l32 = lane & 31, hi = lane >> 5;
  const int kw0 = k0 + pair * 32;
  const int my_key = kw0 + l32;

  // Steps: (head, query block), head-major, query blocks in descending order.
  const int qb_last = (S + TB - 1) / TB - 1;
  const int nqb_all = qb_last + 1 - k0 / TB;
  const bool split_heads = G % nparts == 0;           // else two parts, odd G
  const int nfirst = (nqb_all + 1) / 2;
  const int hbase = g * G + (split_heads ? part * (G / nparts) : 0);
  const int nh = split_heads ? G / nparts : G;
  const int qtop = split_heads || part ? qb_last : k0 / TB + nfirst - 1;
  const int nqb = split_heads ? nqb_all : (part ? nqb_all - nfirst : nfirst);
  const int nsteps = nh * nqb;
  const long kvrow = (long)(b * dm.Hkv + g);
  int to[2];
  t_offsets(lane, to);
  // D layout of dK / dV: lane holds channel nb*32 + l32, key rows 8 (r/4) + 4 hi + r%4

  if (wave < 4) {
    // ---------------- producer: S, dP, softmax, dS, dK
    const float c1 = kLog2e / sqrtf((float)D);
    // B operands for S = Q K^T and dP = dO V^T: lane (key l32, hi) holds
    // channels 16 ks + 8 hi + 0..7 of its key's K'' and V' rows (fp16 copies;
    // rows past s_pad read as zero).
    f16x8 kf[NKS], vf[NKS];
    {
      const __amdgpu_buffer_rsrc_t krs = rows16<D>(a.k16, kvrow * a.s_pad, a.s_pad);
      const __amdgpu_buffer_rsrc_t vrs = rows16<D>(a.v16, kvrow * a.s_pad, a.s_pad);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        kf[ks] = load16(krs, my_key * D + ks * 16 + hi * 8);
        vf[ks] = load16(vrs, my_key * D + ks * 16 + hi * 8);
      }
    }
    f32x16 dk[NMB];
#pragma unroll
    for (int i = 0; i < NMB; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) dk[i][r] = 0.0f;
    if (nsteps > 0) {
      int ao[2];
      a_offsets(perm_row(l32), hi, ao);
      int cur_qi = 0;                              // query block index of step s
      lds_barrier();                               // the consumers have staged step 0
      for (int s = 0; s < nsteps; ++s) {
        const DkdvStage& st = sm.stg[s % 3];
        const int q0 = (qtop - cur_qi) * TB;
        cur_qi = cur_qi + 1 == nqb ? 0 : cur_qi + 1;
        f16x8 qa[NKS], da[NKS];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          qa[ks] = read_a(st.q, ao, ks);
          da[ks] = read_a(st.dO, ao, ks);
        }
        // S starts at -inf where the key follows the query (the causal mask;
        // only steps whose queries reach below the wave's last key have such
        // pairs), so that exp2 gives P = 0 there without a per-element test.
        // lane (key l32, hi): register r is query q0 + 16 (r / 8) + 8 hi + r % 8
        f32x16 sacc, pacc;
        if (q0 < kw0 + 31) {
          const int dlt = my_key - q0 - 8 * hi;
#pragma unroll
          for (int r = 0; r < 16; ++r) sacc[r] = dlt > 16 * (r >> 3) + (r & 7) ? -INFINITY : 0.0f;
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) sacc[r] = 0.0f;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) pacc[r] = 0.0f;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          sacc = __builtin_amdgcn_mfma_f32_32x32x16_f16(qa[ks], kf[ks], sacc, 0, 0, 0);
          pacc = __builtin_amdgcn_mfma_f32_32x32x16_f16(da[ks], vf[ks], pacc, 0, 0, 0);
        }
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
        f16* pw = sm.pbuf[s & 1][pair] + lane * 8;
        *reinterpret_cast<f16x8*>(pw) = pf[0];
        *reinterpret_cast<f16x8*>(pw + 512) = pf[1];
        // dK += dS^T Q: D / 32 channel blocks x 2 steps of 16 queries, Q^T
        // read transposed from the Q tile
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int nb = 0; nb < NMB; ++nb)
            dk[nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(sf[ks], read_t(st.q, to, ks, nb), dk[nb],
                                                            0, 0, 0);
        lds_barrier();
      }
      lds_barrier();                               // the consumers' last step
    }
    const float inv = a.dscale[0] / sqrtf((float)D);   // 2^-e exactly, then 1/sqrt(d)
    float* dkb = (part == 0 ? a.dk : part == 1 ? a.dk2 : part == 2 ? a.dk3 : a.dk4) + kvrow * S * D;
#pragma unroll
    for (int nb = 0; nb < NMB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kw0 + 8 * (r >> 2) + 4 * hi + (r & 3);
        if (key < S) dkb[(long)key * D + nb * 32 + l32] = dk[nb][r] * inv;
      }
  } else {
    // ---------------- consumer: staging and dV += P^T dO, one step behind
    const int tc = t - 256;
    f32x16 dv[NMB];
#pragma unroll
    for (int i = 0; i < NMB; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) dv[i][r] = 0.0f;
    if (nsteps > 0) {
      // steps are loaded in order; the loaded step stops at the last one, so
      // loads past the end repeat it into registers nobody stores
      int ld_s = 0, ld_h = 0, ld_qi = 0;
      auto load_next = [&](DkdvRegs<D>& r) {
        dkdv_load(a, b, hbase + ld_h, (qtop - ld_qi) * TB, tc, r);
        const bool more = ld_s < nsteps - 1;
        const bool wrap = more && ld_qi + 1 == nqb;
        ld_s += more ? 1 : 0;
        ld_qi = wrap ? 0 : ld_qi + (more ? 1 : 0);
        ld_h += wrap ? 1 : 0;
      };
      DkdvRegs<D> r0, r1;                          // step j is staged through r(j % 2)
      load_next(r0);
      load_next(r1);
      dkdv_store(sm.stg[0], tc, r0);
      load_next(r0);
      lds_barrier();
      // iteration s: stage step s + 1 and load step s + 3, then dV of step
      // s - 1 (its MFMAs then run while the producer's softmax does)
      auto iter = [&](int s, DkdvRegs<D>& rs) {
        if (s + 1 < nsteps) {
          dkdv_store(sm.stg[(s + 1) % 3], tc, rs);
          load_next(rs);
        }
        if (s >= 1) {
          const DkdvStage& sp = sm.stg[(s - 1) % 3];
          const f16* pr = sm.pbuf[(s - 1) & 1][pair] + lane * 8;
          f16x8 pa[2];
          pa[0] = *reinterpret_cast<const f16x8*>(pr);
          pa[1] = *reinterpret_cast<const f16x8*>(pr + 512);
#pragma unroll
          for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int nb = 0; nb < NMB; ++nb)
              dv[nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(pa[ks], read_t(sp.dO, to, ks, nb),
                                                              dv[nb], 0, 0, 0);
        }
        lds_barrier();
      };
      for (int s = 0; s <= nsteps; s += 2) {
        iter(s, r1);                               // stores step s + 1 (in r1), loads s + 3
        if (s + 1 <= nsteps) iter(s + 1, r0);
      }
    }
    float* dvb = (part == 0 ? a.dv : part == 1 ? a.dv2 : part == 2 ? a.dv3 : a.dv4) + kvrow * S * D;
    const float unscale = a.dscale[0];               // 2^-e: exact
#pragma unroll
    for (int nb = 0; nb < NMB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kw0 + 8 * (r >> 2) + 4 * hi + (r & 3);
        if (key < S) dvb[(long)key * D + nb * 32 + l32] = dv[nb][r] * unscale;
      }
  }
}

// dk += dk2 (+ dk3 + dk4), dv likewise: the partials of every key block's
// work-groups, in a fixed order.
__global__ __launch_bounds__(256) void bwd_dkdv_sum_kernel(AttnBwdArgs a, long n4) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  f32x4 k = reinterpret_cast<const f32x4*>(a.dk)[i] + reinterpret_cast<const f32x4*>(a.dk2)[i];
  f32x4 v = reinterpret_cast<const f32x4*>(a.dv)[i] + reinterpret_cast<const f32x4*>(a.dv2)[i];
  if (a.dk3) {
    k = k + reinterpret_cast<const f32x4*>(a.dk3)[i];
    k = k + reinterpret_cast<const f32x4*>(a.dk4)[i];
    v = v + reinterpret_cast<const f32x4*>(a.dv3)[i];
    v = v + reinterpret_cast<const f32x4*>(a.dv4)[i];
  }
  reinterpret_cast<f32x4*>(a.dk)[i] = k;
  reinterpret_cast<f32x4*>(a.dv)[i] = v;
}

// ------------------------------------------------------------------ dq
constexpr int DQ_KB = 2;         // 32-key blocks per dQ step
struct DqStage {
  f16 k[DQ_KB * TILE];   // K'' rows of the step's 64 keys
  f16 v[DQ_KB * TILE];   // V' rows
};

template <int D>
struct DqRegs {
  static constexpr int NL = DQ_KB * TB * BG<D>::CPR / 256;   // 16-byte chunks per thread and array
  f16x8 k[NL], v[NL];
};

template <int D>
__device__ __forceinline__ void dq_load(const AttnBwdArgs& a, int b, int g, int j0, int t,
                                        DqRegs<D>& r) {
  constexpr int CPR = BG<D>::CPR;
  const long kvrow = (long)(b * a.dm.Hkv + g) * a.s_pad;
  const __amdgpu_buffer_rsrc_t krs = rows16<D>(a.k16, kvrow, a.s_pad);
  const __amdgpu_buffer_rsrc_t vrs = rows16<D>(a.v16, kvrow, a.s_pad);
#pragma unroll
  for (int i = 0; i < DqRegs<D>::NL; ++i) {
    const int f = t + 256 * i;
    const int row = f / CPR, ch = (f % CPR) * 8;
    r.k[i] = load16(krs, (j0 + row) * D + ch);
    r.v[i] = load16(vrs, (j0 + row) * D + ch);
  }
}

template <int D>
__device__ __forceinline__ void dq_store(DqStage& st, int t, const DqRegs<D>& r) {
#pragma unroll
  for (int i = 0; i < DqRegs<D>::NL; ++i) {
    const int f = t + 256 * i;
    const int row = f / BG<D>::CPR, ch = f % BG<D>::CPR;
    *reinterpret_cast<f16x8*>(st.k + tile_off(row, ch)) = r.k[i];
    *reinterpret_cast<f16x8*>(st.v + tile_off(row, ch)) = r.v[i];
  }
}

// Producer / consumer split as in dkdv: waves 0-3 (producers, 32 queries
// each, Q and dO rows in registers) compute S^T, dP^T and dS and leave dS in
// LDS; waves 4-7 (consumers, same queries) stage the K / V tiles and add
// dQ += dS K one step behind, with K^T read transposed from that step's tile.
struct DqSmem {
  DqStage stg[3];
  f16 sbuf[2][4][DQ_KB][2 * 64 * 8];  // dS per producer: [parity][producer][key block][ks][lane][8]
};

template <int D>
__global__ __launch_bounds__(512) void bwd_dq_kernel(AttnBwdArgs a) {
  constexpr int NKS = BG<D>::NKS, NMB = BG<D>::NMB;
  __shared__ __attribute__((aligned(16))) DqSmem sm;
  const Dims& dm = a.dm;
  const int S = a.S;
  const int nqb = (S + 127) / 128;
  const int per = dm.Hq * a.B;
  const int qb = nqb - 1 - (int)(blockIdx.x / per);          // heaviest blocks first
  const int h = (blockIdx.x % per) % dm.Hq, b = (blockIdx.x % per) / dm.Hq;
  const int g = h / dm.G;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int pair = wave & 3;
  const int l32 = lane & 31, hi = lane >> 5;
  const int q0 = qb * 128;
  const int qw0 = q0 + pair * 32;
  const int my_q = qw0 + l32;
  const long hrow = (long)(b * dm.Hq + h);
  const int q_last = min(S, q0 + 128) - 1;
  const int nsteps = q_last / (DQ_KB * TB) + 1;

  if (wave < 4) {
    // ---------------- producer: S^T, dP^T, dS
    const float c1 = kLog2e / sqrtf((float)D);
    // B operands for S^T = K Q^T and dP^T = V dO^T: lane (query l32, hi) holds
    // channels 16 ks + 8 hi + 0..7 of its query's Q'' and dO rows (fp16 copies).
    f16x8 qf[NKS], df[NKS];
    {
      const __amdgpu_buffer_rsrc_t qrs = rows16<D>(a.q16, hrow * a.s_pad, a.s_pad);
      const __amdgpu_buffer_rsrc_t drs = rows16<D>(a.do16, hrow * a.s_pad, a.s_pad);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        qf[ks] = load16(qrs, my_q * D + ks * 16 + hi * 8);
        df[ks] = load16(drs, my_q * D + ks * 16 + hi * 8);
      }
    }
    const float lse2 = my_q < S ? a.lse[hrow * S + my_q] * kLog2e : INFINITY;
    const float dsm = my_q < S ? a.Dsum[hrow * S + my_q] : 0.0f;
    int ao[2];
    a_offsets(perm_row(l32), hi, ao);
    lds_barrier();                                 // the consumers have staged step 0
    for (int s = 0; s < nsteps; ++s) {
      const DqStage& st = sm.stg[s % 3];
#pragma unroll
      for (int kb = 0; kb < DQ_KB; ++kb) {
      const int j0 = (s * DQ_KB + kb) * TB;
      const f16* tk = st.k + kb * TILE;
      const f16* tv = st.v + kb * TILE;
      if (j0 <= qw0 + 31) {                  // else every key follows every query of the wave
        f32x16 sacc, pacc;
#pragma unroll
        for (int r = 0; r < 16; ++r) pacc[r] = 0.0f;
        // S^T starts at -inf where the key follows the lane's query (only the
        // blocks whose keys reach past the wave's first query have any), so
        // exp2 gives P = 0 there without a per-element test.  Lane (query l32,
        // hi): register r is key j0 + 16 (r / 8) + 8 hi + r % 8.
        if (j0 + 31 > qw0) {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            sacc[r] = j0 + 16 * (r >> 3) + 8 * hi + (r & 7) > my_q ? -INFINITY : 0.0f;
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) sacc[r] = 0.0f;
        }
        f16x8 ka[NKS], va[NKS];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          ka[ks] = read_a(tk, ao, ks);
          va[ks] = read_a(tv, ao, ks);
        }
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          sacc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka[ks], qf[ks], sacc, 0, 0, 0);
          pacc = __builtin_amdgcn_mfma_f32_32x32x16_f16(va[ks], df[ks], pacc, 0, 0, 0);
        }
        f16x8 sf[2];
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int r = 8 * half + e;
            const float p = __builtin_amdgcn_exp2f(fmaf(sacc[r], c1, -lse2));
            sf[half][e] = (f16)(p * (pacc[r] - dsm));
          }
        f16* sw = sm.sbuf[s & 1][pair][kb] + lane * 8;
        *reinterpret_cast<f16x8*>(sw) = sf[0];
        *reinterpret_cast<f16x8*>(sw + 512) = sf[1];
      }
      }
      lds_barrier();
    }
    lds_barrier();                                 // the consumers' last step
  } else {
    // ---------------- consumer: staging and dQ += dS K, one step behind
    const int tc = t - 256;
    f32x16 dq[NMB];
#pragma unroll
    for (int i = 0; i < NMB; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) dq[i][r] = 0.0f;
    int to[2];
    t_offsets(lane, to);
    constexpr int SB = DQ_KB * TB;                 // keys per step
    DqRegs<D> r0, r1;                              // step j is staged through r(j % 2)
    dq_load(a, b, g, 0, tc, r0);
    dq_load(a, b, g, min(1, nsteps - 1) * SB, tc, r1);
    dq_store(sm.stg[0], tc, r0);
    dq_load(a, b, g, min(2, nsteps - 1) * SB, tc, r0);
    lds_barrier();
    // iteration s: stage step s + 1 and load step s + 3, then dQ of step s - 1
    auto iter = [&](int s, DqRegs<D>& rs) {
      if (s + 1 < nsteps) {
        dq_store(sm.stg[(s + 1) % 3], tc, rs);
        dq_load(a, b, g, min(s + 3, nsteps - 1) * SB, tc, rs);
      }
      if (s >= 1) {
        const DqStage& sp = sm.stg[(s - 1) % 3];
#pragma unroll
        for (int kb = 0; kb < DQ_KB; ++kb) {
          if (((s - 1) * DQ_KB + kb) * TB > qw0 + 31) break;
          const f16* sr = sm.sbuf[(s - 1) & 1][pair][kb] + lane * 8;
          f16x8 sa[2];
          sa[0] = *reinterpret_cast<const f16x8*>(sr);
          sa[1] = *reinterpret_cast<const f16x8*>(sr + 512);
          // dQ += dS K: A = dS (lane = query row), B = K^T read transposed
#pragma unroll
          for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int nb = 0; nb < NMB; ++nb)
              dq[nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                  sa[ks], read_t(sp.k + kb * TILE, to, ks, nb), dq[nb], 0, 0, 0);
        }
      }
      lds_barrier();
    };
    for (int s = 0; s <= nsteps; s += 2) {
      iter(s, r1);                                 // stores step s + 1 (in r1), loads s + 3
      if (s + 1 <= nsteps) iter(s + 1, r0);
    }
    // D layout: lane holds channel nb*32 + l32, query rows 8 (r/4) + 4 hi + r%4
    const float inv = a.dscale[0] / sqrtf((float)D);   // 2^-e exactly, then 1/sqrt(d)
    float* dqb = a.dq + hrow * S * D;
#pragma unroll
    for (int nb = 0; nb < NMB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int q = qw0 + 8 * (r >> 2) + 4 * hi + (r & 3);
        if (q < S) dqb[(long)q * D + nb * 32 + l32] = dq[nb][r] * inv;
      }
  }
}

}  // namespace

bool attn_bwd_mfma_supported(const Dims& dm) { return mfma_bwd(dm); }

int attn_bwd_parts(const Dims& dm) { return dm.G % 4 == 0 ? 4 : 2; }

size_t attn_bwd_transpose_bytes(const Dims& dm, int B, int S) {
  if (!mfma_bwd(dm)) return 0;
  const size_t sp = (size_t)(S + 63) / 64 * 64;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  return 2 * al((size_t)B * dm.nq * sp * 2) + 2 * al((size_t)B * dm.nk * sp * 2) +
         2 * (attn_bwd_parts(dm) - 1) * al((size_t)B * S * dm.nk * 4);
}

hipError_t launch_attn_bwd_mfma(const AttnBwdArgs& a, hipStream_t s) {
  const Dims& dm = a.dm;
  if (!mfma_bwd(dm) || !a.q16 || !a.k16 || !a.v16 || !a.do16 || a.s_pad < a.S ||
      a.s_pad % 64 != 0 || !a.dk2 || !a.dv2)
    return hipErrorInvalidValue;
  const int nparts = attn_bwd_parts(dm);
  if (nparts == 4 && (!a.dk3 || !a.dv3 || !a.dk4 || !a.dv4 || a.sum_by_consumer))
    return hipErrorInvalidValue;
  // 32-bit byte offsets within one sequence's token-major dO (bf16) and O (fp32) rows
  if ((long)a.S * dm.nq * 4 >= (1L << 31)) return hipErrorInvalidValue;
  if (!a.amax_part || !a.dscale || dm.nq % 8 != 0) return hipErrorInvalidValue;
  const long n8 = (long)a.B * a.S * dm.nq / 8;
  hipLaunchKernelGGL(bwd_do_absmax_kernel, dim3(kAmaxParts), dim3(256), 0, s,
                     reinterpret_cast<const bf16*>(a.dO), n8, a.amax_part);
  const dim3 gprep(a.s_pad / 64, dm.Hq + dm.Hkv, a.B);
  const dim3 gdkdv(nparts * ((a.S + 127) / 128), dm.Hkv, a.B);
  if (dm.d == 128) {
    hipLaunchKernelGGL(bwd_prep_kernel<128>, gprep, dim3(256), 0, s, a);
    hipLaunchKernelGGL(bwd_dkdv_kernel<128>, gdkdv, dim3(512), 0, s, a);
  } else {
    hipLaunchKernelGGL(bwd_prep_kernel<64>, gprep, dim3(256), 0, s, a);
    hipLaunchKernelGGL(bwd_dkdv_kernel<64>, gdkdv, dim3(512), 0, s, a);
  }
  if (!a.sum_by_consumer) {
    AttnBwdArgs sa = a;
    if (nparts == 2) sa.dk3 = sa.dv3 = sa.dk4 = sa.dv4 = nullptr;
    const long n4 = (long)a.B * dm.Hkv * a.S * dm.d / 4;
    hipLaunchKernelGGL(bwd_dkdv_sum_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s,
                       sa, n4);
  }
  const dim3 gdq(((a.S + 127) / 128) * dm.Hq * a.B);
  if (dm.d == 128)
    hipLaunchKernelGGL(bwd_dq_kernel<128>, gdq, dim3(512), 0, s, a);
  else
    hipLaunchKernelGGL(bwd_dq_kernel<64>, gdq, dim3(512), 0, s, a);
  return hipGetLastError();
}

}  // namespace cca
