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

constexpr int D = 128;
constexpr int BM = 128;        // query rows per work-group
constexpr int BN = 64;         // keys per tile
constexpr int KT_BYTES = BN * D * 2;      // K tile: 64 rows of 256 B
constexpr int VT_BYTES = D * BN * 2;      // V^T tile: 128 rows of 128 B
constexpr int HALF_BYTES = 2 * (KT_BYTES + VT_BYTES);   // one half's two K + V^T buffers
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
constexpr float kLazyLog2 = 8.0f;                        // rescale when the max grows by > 2^8
constexpr int MERGE_STRIDE = 66;                         // floats per lane: 64 of O^T, m, l

typedef __attribute__((address_space(3))) void lds_void;

// LDS byte offset of 16-byte chunk c of K-tile row r (16 chunks per row) and of
// V^T-tile row r (8 chunks per row).  The XOR spreads the 16 rows a half-wave
// reads in one ds_read_b128 over all 64 banks.
__device__ __forceinline__ int k_off(int r, int c) { return r * 256 + ((c ^ (r & 15)) << 4); }
__device__ __forceinline__ int v_off(int r, int c) { return r * 128 + ((c ^ ((r >> 1) & 7)) << 4); }

// K tile of keys key0 .. key0+63 into LDS at kt: each wave of the half (wq)
// writes 4 KB as 4 buffer loads of 1 KB (64 lanes x 16 B), lane L landing at
// row (4 (4 wq + i) + L / 16), chunk position L % 16, so it fetches the global
// chunk that the swizzle puts there.  The resource ends at row nkeys - 1: rows
// past the sequence read as zero.
__device__ __forceinline__ void dma_k(char* kt, const bf16* kb, int key0, int nkeys, int wq,
                                      int lane) {
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(kb + (long)key0 * D), 0, max(nkeys - key0, 0) * D * 2, 0x00020000);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int blk = wq * 4 + i;                 // 1 KB block of the tile
    const int r = blk * 4 + (lane >> 4), pos = lane & 15;
    const int src = r * 256 + ((pos ^ (r & 15)) << 4);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(kt + blk * 1024), 16, src, 0, 0, 0);
  }
}

// V^T tile (128 channel rows x keys key0 .. key0+63) into LDS at vt, the same
// way: row (8 (4 wq + i) + L / 8), chunk position L % 8.
__device__ __forceinline__ void dma_v(char* vt, const bf16* vtb, int s_pad, int key0, int wq,
                                      int lane) {
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(vtb + key0), 0, (D - 1) * s_pad * 2 + BN * 2, 0x00020000);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int blk = wq * 4 + i;
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
__device__ __forceinline__ void mfma_phase(bool pv, bool qk, f32x16 (&oacc)[4],
                                           const f16x8 (&pf)[4], const char* vs_,
                                           f32x16 (&sacc)[2], const char* ks_,
                                           const bf16x8 (&qf)[8], const f32x16& minit, int l32,
                                           int krow, int hi) {
  if (pv) {
#pragma unroll
    for (int pk = 0; pk < 4; ++pk)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const f16x8 vf =
            *reinterpret_cast<const f16x8*>(vs_ + v_off(mb * 32 + l32, 2 * pk + hi));
        oacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pf[pk], oacc[mb], 0, 0, 0);
      }
  }
  if (qk) {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 kf =
            *reinterpret_cast<const bf16x8*>(ks_ + k_off(kb * 32 + krow, 2 * ks + hi));
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], ks == 0 ? minit : sacc[kb],
                                                           0, 0, 0);
      }
  }
}

__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_mfma_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(1024))) char lds[2 * HALF_BYTES];

  const Dims& dm = a.dm;
  const int S = a.Sq;
  const int nqb = (S + BM - 1) / BM;
  const int per_qb = dm.Hq * a.B;
  const int qb = nqb - 1 - (int)(blockIdx.x / per_qb);      // heaviest blocks first
  const int hb = blockIdx.x % per_qb;
  const int h = hb % dm.Hq, b = hb / dm.Hq;
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

  const bf16* qbase = reinterpret_cast<const bf16*>(a.q) + ((long)(b * dm.Hq + h) * S) * D;
  const bf16* kbase = reinterpret_cast<const bf16*>(a.k) + (long)b * a.kv_bs + (long)g * a.kv_hs;
  const bf16* vtbase =
      reinterpret_cast<const bf16*>(a.vt) + (long)(b * dm.Hkv + g) * D * a.s_pad;

  const int q_last = min(S, q0 + BM) - 1;
  const int ntiles = q_last / BN + 1;
  const int niter = (ntiles + 1) / 2;              // tiles of half 0 (>= those of half 1)
  const int nj = (ntiles - half + 1) / 2;          // tiles of this half
  auto key_of = [&](int j) { return (2 * j + half) * BN; };
  // tiles this wave computes: those of its half up to its last row's diagonal
  const int kt_max = min(ntiles - 1, (r0 + 31) / BN);
  const int nvalid = kt_max >= half ? (kt_max - half) / 2 + 1 : 0;
  const float scale = 1.44269504088896340736f / sqrtf((float)D);

  // Q^T fragments first: the prologue's waits then cover them, so no later
  // wait stalls on them.
  // Lane holds query my_q, channels 16*ks + 8*hi + 0..7.
  bf16x8 qf[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    if (my_q < S) {
      qf[ks] = *reinterpret_cast<const bf16x8*>(qbase + (long)my_q * D + ks * 16 + hi * 8);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[ks][e] = (bf16)0.0f;
    }
  }

  // prologue: K and V of tile 0 and K of tile 1 into LDS.  Tile 0 is loaded
  // unconditionally (a one-tile block has half 1 load key tile 0, which it
  // never uses).
  {
    const int key = min(half, ntiles - 1) * BN;
    dma_k(kbuf(0), kbase, key, S, wq, lane);
    dma_v(vbuf(0), vtbase, a.s_pad, key, wq, lane);
  }
  if (nj > 1) dma_k(kbuf(1), kbase, key_of(1), S, wq, lane);
  wait_dma();

  f32x16 oacc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
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
    mfma_phase(j >= 1 && j - 1 < nvalid, j < nvalid, oacc, pf, vbuf((j - 1) & 1), sacc,
               kbuf(j & 1), qf, minit, l32, krow, hi);
    __builtin_amdgcn_s_barrier();

    // ---- softmax phase V(j)
    // Every lane of a wave that takes a tile sees its first key (key0 <= r0):
    // tiles start at multiples of 64 and wave rows at multiples of 32.
    if (j < nvalid) {
      const int key0 = key_of(j);
      if (key0 + BN - 1 > r0) {              // diagonal tile: mask keys after the query
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = key0 + kb * 32 + 16 * (r >> 3) + 8 * hi + (r & 7);
            if (key > my_q) sacc[kb][r] = -INFINITY;
          }
      }
      float mt = fmaxf(sacc[0][0], sacc[1][0]);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 1; r < 16; ++r) mt = fmaxf(mt, sacc[kb][r]);
      mt = xhalf_max(mt);
      // The first tile sets the offset to the row max; later tiles raise it
      // only for rows that outgrew it by more than 2^8.  The branch is taken
      // when any row of the wave needs it, but every other row shifts by an
      // exact 0, so a row's arithmetic never depends on another row's scores
      // (an earlier row stays bit-identical whatever later tokens hold).
      const bool grow = j == 0 || mt > lazy_raw;
      if (__any(grow)) {
        const float delta = grow ? mt : 0.0f;
        const float alpha = __builtin_amdgcn_exp2f(-delta * scale);
        m_use += delta;
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < 4; ++i)
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
    if (j + 1 < nj) dma_v(vbuf((j + 1) & 1), vtbase, a.s_pad, key_of(j + 1), wq, lane);
    if (j + 2 < nj) dma_k(kbuf(j & 1), kbase, key_of(j + 2), S, wq, lane);
    __builtin_amdgcn_s_barrier();
  }
  if (half == 0) __builtin_amdgcn_s_barrier();

  // ---- merge: half 1 hands its (O^T, m, l) to the wave of half 0 with the same
  // rows.  Layout [wave][value][lane] (floats), conflict-free.  The loop's last
  // barrier has retired every read of the tile buffers.  A wave that took no
  // tile hands over m = -inf (weight 0).
  if (nvalid == 0) m_use = -INFINITY;
  float* mg = reinterpret_cast<float*>(lds) + wq * MERGE_STRIDE * 64 + lane;
  wait_dma();
  if (half == 1) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mg[(mb * 16 + r) * 64] = oacc[mb][r];
    mg[64 * 64] = m_use;
    mg[65 * 64] = l_run;
  }
  __syncthreads();
  if (half == 1) return;
  {
    // half 0 always took tile 0, so its offset is finite.
    const float m_b = mg[64 * 64], l_b = mg[65 * 64];
    const float mn = fmaxf(m_use, m_b);
    const float wa = __builtin_amdgcn_exp2f((m_use - mn) * scale);
    const float wb = __builtin_amdgcn_exp2f((m_b - mn) * scale);
    l_run = l_run * wa + l_b * wb;
    m_use = mn;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[mb][r] = oacc[mb][r] * wa + mg[(mb * 16 + r) * 64] * wb;
  }

  // ---- epilogue: lane holds query my_q, channels 32*mb + 8*(r/4) + 4*hi + r%4
  if (my_q < S) {
    const float inv = 1.0f / l_run;
    bf16* orow = reinterpret_cast<bf16*>(a.o) + ((long)(b * S + my_q) * dm.Hq + h) * D;
    float* orow32 = a.o32 ? a.o32 + ((long)(b * S + my_q) * dm.Hq + h) * D : nullptr;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
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
      a.lse[(long)(b * dm.Hq + h) * S + my_q] =
          (m_use * scale + __builtin_amdgcn_logf(l_run)) * 0.69314718055994530942f;
  }
}

}  // namespace

hipError_t launch_attn_fwd_mfma(const AttnArgs& a, hipStream_t s) {
  if (a.dm.d != D || a.vt == nullptr || a.s_pad < a.Sq || a.s_pad % BN != 0)
    return hipErrorInvalidValue;
  const int nqb = (a.Sq + BM - 1) / BM;
  dim3 grid(nqb * a.dm.Hq * a.B);
  hipLaunchKernelGGL(attn_fwd_mfma_kernel, grid, dim3(512), 0, s, a);
  return hipGetLastError();
}

}  // namespace cca
