// cca_attn for bf16, d = 128: causal flash attention on the latent heads with
// MFMA (CCA-es §2.A "Principio Fundamental": attention run entirely in the
// compressed space; §2.C "CCGQA": query head h reads KV head h / G).
//
// Work-group = 8 waves = 128 query rows of one head, split over the keys:
// waves 0-3 (half 0) take the even 64-key tiles, waves 4-7 (half 1) the odd
// ones, each half with its own double-buffered LDS tiles; wave w and w + 4
// own the same 32 query rows and their two partial softmax states are merged
// through LDS at the end.  The split halves the longest work-group, and with
// one 8-wave work-group per CU the grid holds two query blocks per CU on
// average: launched heaviest first, the dispatcher pairs a long block with a
// short one on each CU, so the causal triangle finishes evenly.
//
// The two halves run out of phase (ping-pong): every SIMD holds one wave of
// each half, and between two work-group barriers one half does its matrix
// phase (P V for tile j - 1 and S = Q K^T for tile j, 32 MFMAs) while the other
// does its softmax phase (mask, max, exp2, row sum, P to bf16, and the tile
// copies), so the MFMA unit and the vector ALU of each SIMD are busy at once.
//
// Per tile and wave:
//   S^T = K Q^T    v_mfma_f32_32x32x16_bf16 with A = K rows (LDS), B = Q^T kept
//                  in registers: one query per lane, so the online-softmax row
//                  max and row sum are in-lane plus one exchange with lane ^ 32.
//                  Accumulator row i of each 16-row group holds key
//                  8*((i/4)%2) ... permuted so that the 8 scores a lane passes
//                  to P V are 8 consecutive keys;
//   O^T += V^T P^T v_mfma_f32_32x32x16_f16 with A = V^T rows (LDS, the fp16
//                  copy of V' the mix writes), B = P^T straight from the S^T
//                  accumulators rounded to fp16: 11 significant bits keep the
//                  saved O accurate enough for the backward's rowsum(dO * O),
//                  which the softmax gradient amplifies.
// Tiles move from global memory to LDS with buffer loads that write LDS
// directly (16 bytes per lane), so no registers stage them.  LDS rows are
// unpadded; 16-byte chunks are XOR-swizzled by row so that the MFMA operand
// reads are free of bank conflicts.
// Softmax in base 2: each S^T chain starts from -m (m = the row's running
// offset, in raw score units), so the MFMA result minus the offset only needs
// one multiply by log2(e)/sqrt(d) before exp2.  Q stays exactly the stored
// bf16 Q'' (scaling it before the MFMA would round it a second time, and the
// saved LSE would then disagree with the scores the backward recomputes).  The
// offset is only raised when a row's max grows by more than 2^8 in
// probability (lazy rescaling); until then probabilities stay below 256, which
// fp32 and bf16 hold as well as any other value, and the tile needs no
// rescale of O and no subtraction.  fp32 accumulators throughout.
#include "cca_internal.h"

namespace cca {
namespace {

constexpr int BM = 128;        // query rows per work-group
constexpr int BN = 64;         // keys per tile
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
constexpr float kLazyLog2 = 8.0f;                        // rescale when the max grows by > 2^8

// Sizes that follow the head dimension D (128 or 64).
template <int D>
struct Geom {
  static constexpr int NKS = D / 16;                     // 16-channel k-steps of S = K Q^T
  static constexpr int NMB = D / 32;                     // 32-channel blocks of O^T
  static constexpr int KT_BYTES = BN * D * 2;            // K tile: 64 rows of 2D bytes
  static constexpr int VT_BYTES = D * BN * 2;            // V^T tile: D rows of 128 B
  static constexpr int HALF_BYTES = 2 * (KT_BYTES + VT_BYTES);  // one half's two K + V^T buffers
  static constexpr int MERGE_STRIDE = NMB * 16 + 2;      // floats per lane: O^T, m, l
};

typedef __attribute__((address_space(3))) void lds_void;

// LDS byte offset of 16-byte chunk c of K-tile row r (D / 8 chunks per row)
// and of V^T-tile row r (8 chunks per row).  The XOR spreads the 16 rows a
// half-wave reads in one ds_read_b128 over all 64 banks: with 256-byte rows
// the 16 rows take distinct chunk positions; with 128-byte rows (two rows per
// bank sweep) each parity class of 8 rows does.
__device__ __forceinline__ int v_off(int r, int c) { return r * 128 + ((c ^ ((r >> 1) & 7)) << 4); }
template <int D>
__device__ __forceinline__ int k_off(int r, int c) {
  if constexpr (D == 128) return r * 256 + ((c ^ (r & 15)) << 4);
  else return v_off(r, c);
}

// K tile of keys key0 .. key0+63 into LDS at kt: each wave of the half (wq)
// writes a quarter of the tile as buffer loads of 1 KB (64 lanes x 16 B), lane
// L of block blk landing at row (blk * 1024 / 2D + L / (D / 8)), chunk
// position L % (D / 8), so it fetches the global chunk that the swizzle puts
// there.  The resource ends at row nkeys - 1: rows past the sequence read as
// zero.
template <int D>
__device__ __forceinline__ void dma_k(char* kt, const bf16* kb, int key0, int nkeys, int wq,
                                      int lane) {
  constexpr int NB = Geom<D>::KT_BYTES / 4096, CPR = D / 8;   // blocks per wave, chunks per row
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(kb + (long)key0 * D), 0, max(nkeys - key0, 0) * D * 2, 0x00020000);
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int blk = wq * NB + i;                // 1 KB block of the tile
    const int r = blk * (1024 / (2 * D)) + lane / CPR, pos = lane % CPR;
    const int src = k_off<D>(r, pos);           // the swizzle is an involution per row
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(kt + blk * 1024), 16, src, 0, 0, 0);
  }
}

// V^T tile (D channel rows x keys key0 .. key0+63) into LDS at vt, the same
// way: row (8 blk + L / 8), chunk position L % 8.
template <int D>
__device__ __forceinline__ void dma_v(char* vt, const bf16* vtb, int s_pad, int key0, int wq,
                                      int lane) {
  constexpr int NB = Geom<D>::VT_BYTES / 4096;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(vtb + key0), 0, (D - 1) * s_pad * 2 + BN * 2, 0x00020000);
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int blk = wq * NB + i;
    const int r = blk * 8 + (lane >> 3), pos = lane & 7;
    const int src = r * s_pad * 2 + ((pos ^ ((r >> 1) & 7)) << 4);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(vt + blk * 1024), 16, src, 0, 0, 0);
  }
}

// Waits for this wave's buffer-to-LDS loads (vmcnt(0); lgkmcnt and expcnt left
// alone).
__device__ __forceinline__ void wait_dma() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Value of lane ^ 32 folded in: returns (x op partner) in every lane.
__device__ __forceinline__ float xhalf_max(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto s = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto s = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// One matrix phase of a wave: O^T += V^T P^T for the previous tile (when pv,
// four accumulator chains), then S^T - m = K Q^T started from minit (= -m) for
// the current tile (when qk, two chains).  krow: the K row this lane's
// accumulator column block reads, l32 with bits 2 and 3 swapped.
template <int D>
__device__ __forceinline__ void mfma_phase(bool pv, bool qk, f32x16 (&oacc)[Geom<D>::NMB],
                                           const f16x8 (&pf)[4], const char* vs_,
                                           f32x16 (&sacc)[2], const char* ks_,
                                           const bf16x8 (&qf)[Geom<D>::NKS], const f32x16& minit,
                                           int l32, int krow, int hi) {
  if (pv) {
#pragma unroll
    for (int pk = 0; pk < 4; ++pk)
#pragma unroll
      for (int mb = 0; mb < Geom<D>::NMB; ++mb) {
        const f16x8 vf =
            *reinterpret_cast<const f16x8*>(vs_ + v_off(mb * 32 + l32, 2 * pk + hi));
        oacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pf[pk], oacc[mb], 0, 0, 0);
      }
  }
  if (qk) {
    // K fragment i: k-step i / 2, key block i % 2.  The reads run four
    // fragments ahead of the MFMAs (the scheduler alone keeps two in flight,
    // and an MFMA then waits out most of an LDS round trip).
    constexpr int NQ = 2 * Geom<D>::NKS, AHEAD = 4;
    bf16x8 kf[NQ];
#pragma unroll
    for (int i = 0; i < NQ; ++i)
      kf[i] = *reinterpret_cast<const bf16x8*>(ks_ + k_off<D>((i & 1) * 32 + krow,
                                                              2 * (i >> 1) + hi));
#pragma unroll
    for (int i = 0; i < NQ; ++i)
      sacc[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i], qf[i >> 1],
                                                            i < 2 ? minit : sacc[i & 1], 0, 0, 0);
    // order: AHEAD LDS reads, then (MFMA, LDS read) pairs, then the last MFMAs
#pragma unroll
    for (int i = 0; i < AHEAD; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
    for (int i = 0; i < NQ - AHEAD; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
#pragma unroll
    for (int i = 0; i < AHEAD; ++i) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  }
}

// ------------------------------------------------------------------ fused Q
// The mix's query side inside the attention (the convolution fused with the
// attention, as CCA-es §3 item 4 and CCA-fr §3 describe the authors' kernel):
// the work-group forms Q'' of its 128 queries itself from the bf16 latent,
// Q'' = RoPE(q^ + a/2 (q~ + k~) + b/2 (q^ + k^)) with q^, k^ the causal
// grouped convolutions of its head's q~ and its KV head's k~ (CCA-es §2.B.1,
// §2.B.2), in the arithmetic and order of the mix kernel.  LDS (before the
// K / V tiles use it): the q~ and k~ tiles (the 128 rows plus 4 halo rows,
// 272-byte rows) and the Q'' tile.
constexpr int FQ_HALO = 4;
constexpr int FQ_ROWB = 272;
constexpr int FQ_TROWS = BM + FQ_HALO;
constexpr int FQ_TBYTES = FQ_TROWS * FQ_ROWB;
constexpr int FQ_QOFF = 2 * FQ_TBYTES;                     // Q'' tile: 128 rows of FQ_ROWB

__device__ __forceinline__ float fq_val(const char* tile, int r, int ch) {
  return (float)*reinterpret_cast<const bf16*>(tile + r * FQ_ROWB + ch * 2);
}

// Q'' rows q0 .. q0 + 127 of head h (KV head g, sequence b of S tokens) into
// the LDS tile at lds + FQ_QOFF (rows past S hold values never read).
__device__ __forceinline__ void fused_q_tile(const AttnArgs& a, char* lds, int b, int h, int g,
                                             int q0, int S) {
  constexpr int D = 128, CPR = D / 8, CH = FQ_TROWS * CPR;   // 16-byte chunks per tile
  constexpr int PER = (CH + 511) / 512;
  const Dims& dm = a.dm;
  const bf16* lat = reinterpret_cast<const bf16*>(a.qlat) + (long)b * S * dm.nqkv;
  char* tq = lds;
  char* tk = lds + FQ_TBYTES;
  char* qo = lds + FQ_QOFF;
  // wave w: MFMA column set w % 4 (column n < 16 is channel 16 (w % 4) + n,
  // n >= 16 its RoPE partner + 64) for tokens 64 (w / 4) .. + 63 (two blocks
  // of 32), so each tap fragment serves two MFMAs and a work-group reads each
  // tap row twice
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const bool lo_lane = l32 < 16;
  const int tb = 64 * (wave >> 2);
  const int pair = 16 * (wave & 3) + (l32 & 15);
  const int ch = lo_lane ? pair : pair + 64;
  const bf16* tq_taps = reinterpret_cast<const bf16*>(a.conv_q) + (long)h * dm.kq * D * D;
  const bf16* tk_taps = reinterpret_cast<const bf16*>(a.conv_k) + (long)g * dm.kk * D * D;
  // the B fragments of one lag (8 k-steps), all in flight together
  bf16x8 bf[8];
  auto load_taps = [&](const bf16* taps, int j) {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      bf[ks] = *reinterpret_cast<const bf16x8*>(taps + ((long)j * D + ch) * D + hi * 8 + ks * 16);
  };
  // both tiles and the first lag's taps in one round; rows outside [0, S) read
  // as zero (resource bounds)
  {
    const int r0 = max(q0 - FQ_HALO, 0), r1 = min(S, q0 + BM);
    bf16x8 v[2][PER];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int col = i == 0 ? h * D : dm.nq + g * D;
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(lat + (long)r0 * dm.nqkv + col), 0,
          r1 > r0 ? ((r1 - r0 - 1) * dm.nqkv + D) * 2 : 0, 0x00020000);
#pragma unroll
      for (int p = 0; p < PER; ++p) {
        const int e = min((int)threadIdx.x + 512 * p, CH - 1);
        const int t = q0 - FQ_HALO + e / CPR;
        v[i][p] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                                 rs, ((t - r0) * dm.nqkv + (e % CPR) * 8) * 2, 0, 0));
      }
    }
    load_taps(tq_taps, 0);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int p = 0; p < PER; ++p) {
        const int e = (int)threadIdx.x + 512 * p;
        if (e < CH)
          *reinterpret_cast<bf16x8*>((i ? tk : tq) + (e / CPR) * FQ_ROWB + (e % CPR) * 16) = v[i][p];
      }
  }
  __syncthreads();
  f32x16 qacc[2], kacc[2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) qacc[i][r] = kacc[i][r] = 0.0f;
  // lag j of one head's convolution with the taps in bf (loaded beforehand);
  // acc[mb] holds token block mb of the wave
  auto conv_lag = [&](f32x16 (&acc)[2], const char* tile, int j) {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const bf16x8 af = *reinterpret_cast<const bf16x8*>(
            tile + (tb + 32 * mb + l32 - j + FQ_HALO) * FQ_ROWB + hi * 16 + ks * 32);
        acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bf[ks], acc[mb], 0, 0, 0);
      }
  };
  for (int j = 0; j < dm.kq; ++j) {
    if (j > 0) load_taps(tq_taps, j);
    conv_lag(qacc, tq, j);
  }
  for (int j = 0; j < dm.kk; ++j) {
    load_taps(tk_taps, j);
    conv_lag(kacc, tk, j);
  }
  const float A = (dm.flags & kQkPre) ? 0.5f : 0.0f;
  const float Bc = (dm.flags & kQkPost) ? 0.5f : 0.0f;
  const bool rope = (dm.flags & kRope) != 0;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int tr = tb + 32 * mb + 8 * (r >> 2) + 4 * hi + (r & 3);
      const float qh = qacc[mb][r], kh = kacc[mb][r];
      const float qp = fq_val(tq, tr + FQ_HALO, ch);
      const float kp = fq_val(tk, tr + FQ_HALO, ch);
      // (1 + b/2) q^ + a/2 q~ + (a/2 k~ + b/2 k^)
      const float x = __builtin_fmaf(1.0f + Bc, qh, __builtin_fmaf(A, qp, __builtin_fmaf(A, kp, Bc * kh)));
      const float2 cs = rope ? a.rope[(long)min(q0 + tr, S - 1) * (D / 2) + pair]
                             : make_float2(1.f, 0.f);
      const float xp = __shfl_xor(x, 16);
      const float y = __builtin_fmaf(x, cs.x, lo_lane ? -(xp * cs.y) : xp * cs.y);
      *reinterpret_cast<bf16*>(qo + tr * FQ_ROWB + ch * 2) = (bf16)y;
    }
  __syncthreads();
}

// The work-group's query block.  Fixed length: B sequences of a.Sq tokens, Q
// head-major per sequence, query t at position t.  Variable length (VARLEN):
// sequence b has nq = tok[b + 1] - tok[b] queries at positions start[b] ..,
// Q packed [Hq][T][d] over all T tokens, K and V'^T covering keys 0 ..
// start[b] + nq - 1, O rows packed like the tokens.
// (The body sits in the kernel template itself: moved into a device function
// it compiles to a slower schedule of the same arithmetic.)
// FQ: Q'' formed in the kernel from the latent (fixed length, D = 128).
// SPL: key-split (fixed length): a.ksplit = P work-groups per query block,
// part p taking the block's key tiles t = p, p + P, p + 2P, ... (half 0 the
// even ones of that list, half 1 the odd ones); each writes its unnormalised
// (O, m, l) to a.part and attn_split_merge_kernel forms O and the LSE.  For
// grids that would leave CUs idle (short sequences): P times the work-groups,
// and the longest block no longer sets the kernel's length.
struct NoMap {};
template <int D, bool VARLEN, bool FQ, typename Map, bool SPL = false>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_mfma_kernel(AttnArgs a, Map vm) {
  static_assert(!FQ || (D == 128 && !VARLEN), "fused Q: fixed length, d = 128");
  static_assert(!SPL || (!VARLEN && !FQ), "key split: fixed length, Q'' as stored");
  using GM = Geom<D>;
  constexpr int NKS = GM::NKS, NMB = GM::NMB, KT_BYTES = GM::KT_BYTES, VT_BYTES = GM::VT_BYTES;
  constexpr int HALF_BYTES = GM::HALF_BYTES, MERGE_STRIDE = GM::MERGE_STRIDE;
  __shared__ __attribute__((aligned(1024))) char lds[2 * HALF_BYTES];

  const Dims& dm = a.dm;
  int b, h, qb, nq, pos0;
  int part = 0;                              // SPL: this work-group's share of the key tiles
  long qrow0, orow0;                         // Q row and O row of query 0 of the block's sequence
  if constexpr (SPL) {
    nq = a.Sq;
    pos0 = 0;
    const int nqb = (nq + BM - 1) / BM;
    const int per_qb = dm.Hq * a.B * a.ksplit;
    qb = nqb - 1 - (int)(blockIdx.x / per_qb);             // heaviest blocks first
    const int rem = blockIdx.x % per_qb;
    const int hb = rem / a.ksplit;
    part = rem % a.ksplit;
    h = hb % dm.Hq;
    b = hb / dm.Hq;
    qrow0 = (long)(b * dm.Hq + h) * nq;
    orow0 = (long)b * nq;
  } else if constexpr (!VARLEN) {
    nq = a.Sq;
    pos0 = 0;
    const int nqb = (nq + BM - 1) / BM;
    const int per_qb = dm.Hq * a.B;
    qb = nqb - 1 - (int)(blockIdx.x / per_qb);             // heaviest blocks first
    const int hb = blockIdx.x % per_qb;
    h = hb % dm.Hq;
    b = hb / dm.Hq;
    qrow0 = (long)(b * dm.Hq + h) * nq;
    orow0 = (long)b * nq;
  } else {
    // blocks numbered (sequence, query block, head); the last ones (the
    // longest key ranges of each sequence) start first
    const int L = vm.blk[vm.B] * dm.Hq - 1 - (int)blockIdx.x;
    const int blk = L / dm.Hq;
    h = L % dm.Hq;
    int lo = 0, hi2 = vm.B - 1;                             // last b with blk[b] <= blk
    while (lo < hi2) {
      const int mid = (lo + hi2 + 1) >> 1;
      if (vm.blk[mid] <= blk) lo = mid; else hi2 = mid - 1;
    }
    b = lo;
    qb = blk - vm.blk[b];
    nq = vm.tok[b + 1] - vm.tok[b];
    pos0 = vm.start[b];
    qrow0 = (long)h * vm.tok[vm.B] + vm.tok[b];
    orow0 = vm.tok[b];
  }
  const int nkeys = pos0 + nq;               // keys 0 .. nkeys - 1 exist
  const int g = h / dm.G;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = wave >> 2;                // 0: even key tiles, 1: odd key tiles
  const int wq = wave & 3;                   // query sub-block of this wave
  const int l32 = lane & 31, hi = lane >> 5;
  const int q0 = qb * BM;
  const int r0 = q0 + wq * 32;               // first query row of this wave
  const int my_q = r0 + l32;                 // this lane's query row
  // S^T accumulator row i (of 32) holds key 16 (i / 16) + 8 ((i / 4) % 2) +
  // 4 ((i / 8) % 2) + i % 4: bits 2 and 3 of the row swapped, so the scores in
  // registers 8 s .. 8 s + 7 of a lane are keys 16 s + 8 hi + 0..7.
  const int krow = (l32 & ~12) | ((l32 & 4) << 1) | ((l32 & 8) >> 1);

  // This half's buffers: K0, K1, V0, V1; tile j of the half (key tile 2j + half)
  // has its K in K[j % 2] and its V^T in V[j % 2].  Plain offsets from the
  // __shared__ array keep every access a ds_read / ds_write.
  char* const hbase = lds + half * HALF_BYTES;
  auto kbuf = [&](int i) { return hbase + i * KT_BYTES; };
  auto vbuf = [&](int i) { return hbase + 2 * KT_BYTES + i * VT_BYTES; };

  const bf16* qbase = reinterpret_cast<const bf16*>(a.q) + qrow0 * D;
  const bf16* kbase = reinterpret_cast<const bf16*>(a.k) + (long)b * a.kv_bs + (long)g * a.kv_hs;
  const bf16* vtbase =
      reinterpret_cast<const bf16*>(a.vt) + (long)(b * dm.Hkv + g) * D * a.s_pad;

  const int q_last = min(nq, q0 + BM) - 1;
  // SPL: the part's tiles are the block's tiles part, part + P, ...; ntiles
  // counts them, and tile j of a half is the part's tile 2 j + half
  const int ntl = (pos0 + q_last) / BN + 1;        // key tiles of the block
  const int ntiles = SPL ? (part < ntl ? (ntl - part + a.ksplit - 1) / a.ksplit : 0) : ntl;
  if (SPL && ntiles == 0) return;                  // a part with no tile: the merge skips it
  const int niter = (ntiles + 1) / 2;              // tiles of half 0 (>= those of half 1)
  const int nj = (ntiles - half + 1) / 2;          // tiles of this half
  auto key_of = [&](int j) {
    if constexpr (SPL) return ((2 * j + half) * a.ksplit + part) * BN;
    else return (2 * j + half) * BN;
  };
  // tiles this wave computes: those of its half up to its last row's diagonal
  const int kt_max = min(ntl - 1, (pos0 + r0 + 31) / BN);
  int nvalid;
  if constexpr (SPL) {
    const int t0 = part + a.ksplit * half;           // the half's first tile
    nvalid = kt_max >= t0 ? (kt_max - t0) / (2 * a.ksplit) + 1 : 0;
  } else {
    nvalid = kt_max >= half ? (kt_max - half) / 2 + 1 : 0;
  }
  const float scale = 1.44269504088896340736f / sqrtf((float)D);

  // Q^T fragments first: the prologue's waits then cover them, so no later
  // wait stalls on them.
  // Lane holds query my_q, channels 16*ks + 8*hi + 0..7.
  bf16x8 qf[NKS];
  if constexpr (FQ) {
    fused_q_tile(a, lds, b, h, g, q0, nq);
    const char* qrow = lds + FQ_QOFF + (wq * 32 + l32) * FQ_ROWB + hi * 16;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      if (my_q < nq) {
        qf[ks] = *reinterpret_cast<const bf16x8*>(qrow + ks * 32);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[ks][e] = (bf16)0.0f;
      }
    }
    __syncthreads();                         // every wave has its Q before the tiles land
  } else {
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      if (my_q < nq) {
        qf[ks] = *reinterpret_cast<const bf16x8*>(qbase + (long)my_q * D + ks * 16 + hi * 8);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[ks][e] = (bf16)0.0f;
      }
    }
  }

  // prologue: K and V of tile 0 and K of tile 1 into LDS.  Tile 0 is loaded
  // unconditionally (a one-tile block has half 1 load key tile 0, which it
  // never uses).
  {
    const int key = SPL ? key_of(0) : min(half, ntiles - 1) * BN;   // SPL: past the keys reads zero
    dma_k<D>(kbuf(0), kbase, key, nkeys, wq, lane);
    // (SPL: an empty half's first tile may lie past s_pad; any in-range tile serves)
    dma_v<D>(vbuf(0), vtbase, a.s_pad, SPL ? min(key, a.s_pad - BN) : key, wq, lane);
  }
  if (nj > 1) dma_k<D>(kbuf(1), kbase, key_of(1), nkeys, wq, lane);
  wait_dma();

  f32x16 oacc[NMB];
#pragma unroll
  for (int i = 0; i < NMB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[i][r] = 0.0f;
  float m_use = 0.0f, l_run = 0.0f;    // exponent offset (raw score units), row sum
  const float lazy_raw = kLazyLog2 / scale;
  f32x16 minit;                        // -m_use in every register
#pragma unroll
  for (int r = 0; r < 16; ++r) minit[r] = 0.0f;
  f32x16 sacc[2];                      // S^T - m of the tile between its two phases
  f16x8 pf[4];                         // P^T (fp16) of the tile between softmax and P V
  __syncthreads();

  // Phases: each half runs M0 V0 M1 V1 ... M(niter) V(niter), where M(j) = the
  // matrix phase (P V of tile j - 1, S of tile j) and V(j) = the softmax of
  // tile j plus the tile copies, with a work-group barrier after every phase.
  // Half 1 passes one extra barrier first and half 0 one at the end, so both
  // count the same barriers and half 1 runs exactly one phase behind: between
  // two barriers one half multiplies while the other exponentiates.
  if (half == 1) __builtin_amdgcn_s_barrier();
  for (int j = 0; j <= niter; ++j) {
    // ---- matrix phase M(j)
    mfma_phase<D>(j >= 1 && j - 1 < nvalid, j < nvalid, oacc, pf, vbuf((j - 1) & 1), sacc,
               kbuf(j & 1), qf, minit, l32, krow, hi);
    __builtin_amdgcn_s_barrier();

    // ---- softmax phase V(j)
    // With positions aligned to the tiles (fixed length), every lane of a wave
    // that takes a tile sees the tile's first key; with a position offset a
    // lane may see none (its max is then -inf, see the offset rule below).
    if (j < nvalid) {
      const int key0 = key_of(j);
      if (key0 + BN - 1 > pos0 + r0) {       // diagonal tile: mask keys after the query
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = key0 + kb * 32 + 16 * (r >> 3) + 8 * hi + (r & 7);
            if (key > pos0 + my_q) sacc[kb][r] = -INFINITY;
          }
      }
      float mt = fmaxf(sacc[0][0], sacc[1][0]);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 1; r < 16; ++r) mt = fmaxf(mt, sacc[kb][r]);
      mt = xhalf_max(mt);
      // The first tile with a visible key sets the offset to the row max
      // (tile 0 at fixed length; with a position offset l_run is 0 until
      // then, and at least 1 after: the max scores exp2(0)); later tiles
      // raise it only for rows that outgrew it by more than 2^8.  The branch
      // is taken when any row of the wave needs it, but every other row
      // shifts by an exact 0, so a row's arithmetic never depends on another
      // row's scores (an earlier row stays bit-identical whatever later
      // tokens hold).
      const bool first = (VARLEN || SPL) ? (l_run == 0.0f && mt != -INFINITY) : j == 0;
      const bool grow = first || mt > lazy_raw;
      if (__any(grow)) {
        const float delta = grow ? mt : 0.0f;
        float alpha = __builtin_amdgcn_exp2f(-delta * scale);
        // SPL: a row's first visible tile may lie far below the offset; O and
        // l are still 0 then, so the rescale is skipped (no 0 * inf)
        if constexpr (SPL) alpha = first ? 1.0f : alpha;
        m_use += delta;
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < NMB; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) sacc[kb][r] -= delta;
#pragma unroll
        for (int r = 0; r < 16; ++r) minit[r] = -m_use;
      }
      float ls = 0.0f;
#pragma unroll
      for (int pk = 0; pk < 4; ++pk)
#pragma unroll
        for (int s8 = 0; s8 < 8; ++s8) {
          const float pv = __builtin_amdgcn_exp2f(sacc[pk >> 1][8 * (pk & 1) + s8] * scale);
          ls += pv;
          pf[pk][s8] = (_Float16)pv;
        }
      l_run += xhalf_sum(ls);
    }
    // Tile copies of this half: wait for the ones issued in V(j - 1) (V of tile
    // j and K of tile j + 1, read from M(j + 1) on, after the barrier), then
    // issue V of tile j + 1 into the V buffer tile j - 1 used and K of tile
    // j + 2 into the K buffer tile j used (both last read in M(j)).
    wait_dma();
    if (j + 1 < nj) dma_v<D>(vbuf((j + 1) & 1), vtbase, a.s_pad, key_of(j + 1), wq, lane);
    if (j + 2 < nj) dma_k<D>(kbuf(j & 1), kbase, key_of(j + 2), nkeys, wq, lane);
    __builtin_amdgcn_s_barrier();
  }
  if (half == 0) __builtin_amdgcn_s_barrier();

  // ---- merge: half 1 hands its (O^T, m, l) to the wave of half 0 with the same
  // rows.  Layout [wave][value][lane] (floats), conflict-free.  The loop's last
  // barrier has retired every read of the tile buffers.  A wave that took no
  // tile hands over m = -inf (weight 0).
  if (nvalid == 0) m_use = -INFINITY;
  if constexpr (SPL) {
    if (l_run == 0.0f) m_use = -INFINITY;    // a row that saw no key of its part's tiles
  }
  float* mg = reinterpret_cast<float*>(lds) + wq * MERGE_STRIDE * 64 + lane;
  wait_dma();
  if (half == 1) {
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mg[(mb * 16 + r) * 64] = oacc[mb][r];
    mg[NMB * 16 * 64] = m_use;
    mg[(NMB * 16 + 1) * 64] = l_run;
  }
  __syncthreads();
  if (half == 1) return;
  {
    // half 0 always took tile 0, so its offset is finite (not with SPL: an
    // empty half has m = -inf and weight 0)
    const float m_b = mg[NMB * 16 * 64], l_b = mg[(NMB * 16 + 1) * 64];
    const float mn = fmaxf(m_use, m_b);
    float wa = __builtin_amdgcn_exp2f((m_use - mn) * scale);
    float wb = __builtin_amdgcn_exp2f((m_b - mn) * scale);
    if constexpr (SPL) {
      wa = m_use == -INFINITY ? 0.0f : wa;
      wb = m_b == -INFINITY ? 0.0f : wb;
    }
    l_run = l_run * wa + l_b * wb;
    m_use = mn;
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[mb][r] = oacc[mb][r] * wa + mg[(mb * 16 + r) * 64] * wb;
  }

  // ---- epilogue: lane holds query my_q, channels 32*mb + 8*(r/4) + 4*hi + r%4
  if constexpr (SPL) {
    // the part's unnormalised O and its (m, l): partial ((b Hq + h) P + part) S + my_q
    if (my_q < nq) {
      const long pi = ((long)(b * dm.Hq + h) * a.ksplit + part) * nq + my_q;
      float* po = a.part + pi * D;
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *reinterpret_cast<f32x4*>(po + mb * 32 + 8 * j + 4 * hi) =
              f32x4{oacc[mb][4 * j], oacc[mb][4 * j + 1], oacc[mb][4 * j + 2], oacc[mb][4 * j + 3]};
      if (hi == 0) {
        float* pml = a.part + (long)a.B * dm.Hq * a.ksplit * nq * D + pi * 2;
        pml[0] = m_use;
        pml[1] = l_run;
      }
    }
    return;
  }
  if (my_q < nq) {
    const float inv = 1.0f / l_run;
    const long row = VARLEN ? orow0 + my_q : (long)(b * nq + my_q);
    bf16* orow = reinterpret_cast<bf16*>(a.o) + (row * dm.Hq + h) * D;
    float* orow32 = a.o32 ? a.o32 + (row * dm.Hq + h) * D : nullptr;
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = mb * 32 + 8 * j + 4 * hi;
        bf16x4 v4;
        f32x4 f4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          f4[i] = oacc[mb][4 * j + i] * inv;
          v4[i] = (bf16)f4[i];
        }
        *reinterpret_cast<bf16x4*>(orow + c) = v4;
        if (orow32) *reinterpret_cast<f32x4*>(orow32 + c) = f4;
      }
    // natural-log LSE of the scaled scores: (m log2(e)/sqrt(d) + log2 l) ln 2
    if (hi == 0 && a.lse)
      a.lse[qrow0 + my_q] =
          (m_use * scale + __builtin_amdgcn_logf(l_run)) * 0.69314718055994530942f;
  }
}

// The key-split partials of each query combined in a fixed order (parts 0 ..
// P - 1; a part with no tile of the query's block, or whose rows saw no key,
// has weight 0): O = sum_p w_p O_p / sum_p w_p l_p with w_p = 2^((m_p - m) s),
// m the largest m_p; the LSE as in the unsplit kernel.  Thread = 4 channels of
// one query of one head.
template <int D>
__global__ __launch_bounds__(256) void attn_split_merge_kernel(AttnArgs a) {
  const Dims& dm = a.dm;
  const int S = a.Sq, P = a.ksplit;
  const long t = (long)blockIdx.x * 256 + threadIdx.x;
  const long nqh = (long)a.B * dm.Hq * S;
  if (t >= nqh * (D / 4)) return;
  const long qi = t / (D / 4);                 // ((b Hq + h) S + q)
  const int c = (int)(t % (D / 4)) * 4;
  const int q = (int)(qi % S);
  const long bh = qi / S;
  const int h = (int)(bh % dm.Hq), b = (int)(bh / dm.Hq);
  const int qb = q / BM;
  const int ntl = (min(S, qb * BM + BM) - 1) / BN + 1;
  const int np = min(P, ntl);
  const float scale = 1.44269504088896340736f / sqrtf((float)D);
  const float* pml = a.part + nqh * P * D;
  float mn = -INFINITY;
  for (int p = 0; p < np; ++p) {
    const long pi = (bh * P + p) * S + q;
    if (pml[pi * 2 + 1] > 0.0f) mn = fmaxf(mn, pml[pi * 2]);
  }
  float L = 0.0f;
  f32x4 o = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int p = 0; p < np; ++p) {
    const long pi = (bh * P + p) * S + q;
    const float lp = pml[pi * 2 + 1];
    const float w = lp > 0.0f ? __builtin_amdgcn_exp2f((pml[pi * 2] - mn) * scale) : 0.0f;
    const f32x4 v = *reinterpret_cast<const f32x4*>(a.part + pi * D + c);
    L = __builtin_fmaf(w, lp, L);
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = __builtin_fmaf(w, v[e], o[e]);
  }
  const float inv = 1.0f / L;
  const long row = (long)b * S + q;
  bf16x4 v4;
  f32x4 f4;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f4[e] = o[e] * inv;
    v4[e] = (bf16)f4[e];
  }
  *reinterpret_cast<bf16x4*>(reinterpret_cast<bf16*>(a.o) + (row * dm.Hq + h) * D + c) = v4;
  if (a.o32) *reinterpret_cast<f32x4*>(a.o32 + (row * dm.Hq + h) * D + c) = f4;
  if (c == 0 && a.lse)
    a.lse[bh * S + q] = (mn * scale + __builtin_amdgcn_logf(L)) * 0.69314718055994530942f;
}

}  // namespace

size_t attn_split_part_bytes(const Dims& dm, int B, int S, int P) {
  return P > 1 ? (size_t)B * dm.Hq * P * S * (dm.d + 2) * 4 : 0;
}

hipError_t launch_attn_fwd_mfma(const AttnArgs& a, hipStream_t s) {
  if ((a.dm.d != 128 && a.dm.d != 64) || a.vt == nullptr || a.s_pad < a.Sq || a.s_pad % BN != 0)
    return hipErrorInvalidValue;
  const int nqb = (a.Sq + BM - 1) / BM;
  dim3 grid(nqb * a.dm.Hq * a.B);
  if (a.ksplit > 1) {
    if (a.qlat || a.part == nullptr || a.ksplit > kMaxAttnSplit) return hipErrorInvalidValue;
    dim3 gsplit(nqb * a.dm.Hq * a.B * a.ksplit);
    const long nt = (long)a.B * a.dm.Hq * a.Sq * (a.dm.d / 4);
    const dim3 gm((unsigned)((nt + 255) / 256));
    if (a.dm.d == 128) {
      hipLaunchKernelGGL((attn_fwd_mfma_kernel<128, false, false, NoMap, true>), gsplit, dim3(512),
                         0, s, a, NoMap{});
      hipLaunchKernelGGL(attn_split_merge_kernel<128>, gm, dim3(256), 0, s, a);
    } else {
      hipLaunchKernelGGL((attn_fwd_mfma_kernel<64, false, false, NoMap, true>), gsplit, dim3(512),
                         0, s, a, NoMap{});
      hipLaunchKernelGGL(attn_split_merge_kernel<64>, gm, dim3(256), 0, s, a);
    }
    return hipGetLastError();
  }
  if (a.qlat) {
    if (a.dm.d != 128 || !a.dm.bf16 || !a.conv_q || !a.conv_k || !a.rope || a.dm.kq > FQ_HALO + 1 ||
        a.dm.kk > FQ_HALO + 1 || (long)a.Sq * a.dm.nqkv * 2 >= (1L << 31))
      return hipErrorInvalidValue;
    hipLaunchKernelGGL((attn_fwd_mfma_kernel<128, false, true, NoMap>), grid, dim3(512), 0, s, a,
                       NoMap{});
  } else if (a.dm.d == 128) {
    hipLaunchKernelGGL((attn_fwd_mfma_kernel<128, false, false, NoMap>), grid, dim3(512), 0, s, a,
                       NoMap{});
  } else {
    hipLaunchKernelGGL((attn_fwd_mfma_kernel<64, false, false, NoMap>), grid, dim3(512), 0, s, a,
                       NoMap{});
  }
  return hipGetLastError();
}

// Variable-length attention: a.q packed [Hq][T][d], a.k / a.v the caches (kv_bs,
// kv_hs), a.vt the V'^T of every sequence [B][Hkv][d][s_pad], a.o packed
// [T][Hq*d]; vm.blk counts 128-query blocks.  No lse / o32.
hipError_t launch_attn_varlen_mfma(const AttnArgs& a, const VarlenMap& vm, hipStream_t s) {
  if (a.dm.d != 128 || a.vt == nullptr || a.s_pad % BN != 0 || a.lse || a.o32 || vm.B < 1 ||
      vm.B > kMaxVarlenBatch)
    return hipErrorInvalidValue;
  const long nblk = (long)vm.blk[vm.B] * a.dm.Hq;
  if (nblk == 0) return hipSuccess;
  hipLaunchKernelGGL((attn_fwd_mfma_kernel<128, true, false, VarlenMap>), dim3((unsigned)nblk), dim3(512), 0, s,
                     a, vm);
  return hipGetLastError();
}

}  // namespace cca
