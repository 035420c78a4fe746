// Large bf16 GEMM for the projections of the CCA layer (cca_proj): C = A B^T
// with A [M, K] and B [N, K] both K-contiguous ("NT"), fp32 accumulation,
// fp32 or bf16 output.  It serves the down-projection of x to the latent
// q~ | k~ | v~ (CCA-es §2.A "Principio Fundamental"; CCA-fr §2 "Projection
// vers l'Espace Latent") and the output projection O W_o^T.
//
// Work-group tile 256 x 256 x 64 as eight waves of 128 x 64, two per SIMD
// (each wave holds 8 accumulator blocks of v_mfma_f32_32x32x16_bf16 and issues
// 8 MFMAs per 16-wide k step; the template also has a four-wave form of
// 128 x 128, one wave per SIMD, which measured slower); when 256-row tiles
// would leave CUs idle (and nothing splits K), 128 x 256 tiles of eight waves
// of 64 x 64.  Operand fragments are double-buffered.  Tiles of A and B move
// from global memory to LDS with buffer loads that write LDS directly (16
// bytes per lane), two stages deep; the next stage's 1 KB copies (8 per wave)
// are issued at MFMA issue points over the first half of the k step rather
// than in a burst: a copy's issue waits until the address unit takes it, and a
// burst would leave the MFMA unit idle for that long, while copies spread over
// the whole step leave the last ones' memory latency exposed at the
// end-of-step wait.  LDS rows (64 k = 128 B) are unpadded with their
// 16-byte chunks XOR-swizzled by row, so that the fragment reads are free of
// bank conflicts.
// Grids of 512 or more bf16 tiles run two tiles per work-group: the second
// tile's first stage is copied during the first tile's last k step, and the
// first tile leaves through the other stage, so its stores drain while the
// second tile computes.
// Rows past M or past the end of B's segment read as zero (buffer range
// check), so ragged M and N need no special path.
// TN layout (C = A^T B with A [K, M] and B [K, N] both row-major, as the weight
// gradients dY^T O and dQKV^T x over the tokens): the tiles are copied as 64
// k-rows of 256 elements (512 B) and the MFMA fragments, 8 consecutive k per
// lane, are read transposed with ds_read_b64_tr_b16; k-rows at or past k_valid
// read as zero.  Tiles are numbered so that
// the tiles of one XCD (work-groups are dealt to the 8 XCDs round-robin) are
// consecutive and share rows of A in that XCD's L2.
#include "cca_internal.h"

namespace cca {
namespace {

constexpr int TM = 256, TN = 256, TK = 64;
constexpr int B_BYTES = TN * TK * 2;

typedef __attribute__((address_space(3))) void lds_void;

// LDS byte offset of 16-byte chunk c (of 8) in tile row r.
__device__ __forceinline__ int sw(int r, int c) { return r * 128 + ((c ^ ((r >> 1) & 7)) << 4); }

__device__ __forceinline__ void wait_dma() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

__device__ __forceinline__ void store_out(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_out(bf16* p, float v) { *p = (bf16)v; }
// 16 bytes of OutT elements
template <typename T> struct OutVT;
template <> struct OutVT<float> { typedef f32x4 type; };
template <> struct OutVT<bf16> { typedef bf16x8 type; };
template <typename T> using OutV = typename OutVT<T>::type;
__device__ __forceinline__ void store4(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<f32x4*>(p) = f32x4{a, b, c, d};
}
__device__ __forceinline__ void store4(bf16* p, float a, float b, float c, float d) {
  *reinterpret_cast<bf16x4*>(p) = bf16x4{(bf16)a, (bf16)b, (bf16)c, (bf16)d};
}

// One 256-row x 64-k operand tile into LDS: rows row0 .. of a K-contiguous
// matrix at base (row stride ld elements), `rows` of them valid; k from k0.
// With NW waves, wave w writes 1 KB blocks CB w .. CB w + CB - 1 (CB = 32 / NW,
// 8 rows each); lane L lands at row 8 blk + L / 8, chunk position L % 8 and
// fetches the chunk the swizzle puts there.
template <int CB>
__device__ __forceinline__ void dma_tile(char* dst, const bf16* base, long ld, int rows, int K,
                                         int k0, int wave, int lane) {
  const int nrec = ((rows - 1) * (int)ld + K - k0) * 2;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(base + k0), 0, nrec, 0x00020000);
#pragma unroll
  for (int i = 0; i < CB; ++i) {
    const int blk = wave * CB + i;
    const int r = blk * 8 + (lane >> 3), pos = lane & 7;
    const int src = r * (int)ld * 2 + ((pos ^ ((r >> 1) & 7)) << 4);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(dst + blk * 1024), 16, src, 0, 0, 0);
  }
}

// Block i (0 .. CB - 1) of this wave's share of dma_tile, alone.
template <int CB>
__device__ __forceinline__ void dma_part(char* dst, const bf16* base, long ld, int rows, int K,
                                         int k0, int wave, int lane, int i) {
  const int nrec = ((rows - 1) * (int)ld + K - k0) * 2;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(base + k0), 0, nrec, 0x00020000);
  const int blk = wave * CB + i;
  const int r = blk * 8 + (lane >> 3), pos = lane & 7;
  const int src = r * (int)ld * 2 + ((pos ^ ((r >> 1) & 7)) << 4);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(dst + blk * 1024), 16, src, 0, 0, 0);
}

// Block i of this wave's share of a B tile whose 256 rows may cross segments
// of B (the concatenated q / k / v weights when a segment does not start at a
// multiple of 256): each 1 KB block (8 rows) resolves its own segment, so a
// segment start must be a multiple of 8.  Rows past the end of B read as zero.
template <int CB>
__device__ __forceinline__ void dma_part_seg(char* dst, const GemmArgs& g, int n0, int k0,
                                             int wave, int lane, int i) {
  const int blk = wave * CB + i;
  const int row0 = n0 + blk * 8;
  int s = 0;
  if (g.b_nseg > 1 && row0 >= g.b_start[1]) s = 1;
  if (g.b_nseg > 2 && row0 >= g.b_start[2]) s = 2;
  const int seg_end = s + 1 < g.b_nseg ? g.b_start[s + 1] : g.N;
  const int rows = min(seg_end - row0, 8);
  const bf16* base = reinterpret_cast<const bf16*>(g.b_ptr[s]) + (long)(row0 - g.b_start[s]) * g.ldb;
  const int nrec = rows > 0 ? ((rows - 1) * (int)g.ldb + g.K - k0) * 2 : 0;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(base + k0), 0, nrec, 0x00020000);
  const int r = blk * 8 + (lane >> 3), pos = lane & 7;
  const int src = (lane >> 3) * (int)g.ldb * 2 + ((pos ^ ((r >> 1) & 7)) << 4);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(dst + blk * 1024), 16, src, 0, 0, 0);
}

// K-major operand tile: k-rows k0 .. k0 + 63, columns r0 .. r0 + 255 of a
// row-major [K, R] matrix (row stride ld), as 64 LDS rows of 512 B with chunk c
// (columns 8 c .. 8 c + 7) of row k at chunk c ^ 4 (k & 3): the 4 k-rows of a
// transposing read then fall on distinct banks.  Block i of this wave's share:
// 1 KB = two k-rows; lane L lands at row 2 blk + L / 32, chunk position L % 32.
// The resource ends at row k_valid - 1: later rows read as zero, and columns
// past R (next row's data, or zero past the end) only reach C rows / columns
// that are never stored.
template <int CB>
__device__ __forceinline__ void dma_part_t(char* dst, const bf16* mat, long ld, int r0,
                                           int kvalid, int k0, int wave, int lane, int i) {
  const long rem = (long)(kvalid - k0) * ld - r0;
  const int nrec = rem > 0 ? (int)(rem * 2) : 0;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(mat + (long)k0 * ld + r0), 0, nrec, 0x00020000);
  const int blk = wave * CB + i;
  const int kr = 2 * blk + (lane >> 5), pos = lane & 31;
  const int src = (kr * (int)ld + 8 * (pos ^ (4 * (kr & 3)))) * 2;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(dst + blk * 1024), 16, src, 0, 0, 0);
}

template <int CB>
__device__ __forceinline__ void dma_tile_t(char* dst, const bf16* mat, long ld, int r0, int kvalid,
                                           int k0, int wave, int lane) {
#pragma unroll
  for (int i = 0; i < CB; ++i) dma_part_t<CB>(dst, mat, ld, r0, kvalid, k0, wave, lane, i);
}

// Byte offset (within a stage's K-major tile, before + 8192 ks) of the
// transposing reads that give lane (column col0 + l32, hi) the k-rows
// 16 ks + 8 hi + 0..7: lane c of each 16-lane group addresses k-row
// 8 hi + (c >> 2) (+ 4 for the second read) and columns col0 + 16 g + 4 (c & 3).
__device__ __forceinline__ int t_frag_off(int lane, int col0) {
  const int c = lane & 15, g = (lane >> 4) & 1, hi = lane >> 5;
  const int kr = 8 * hi + (c >> 2);
  const int col = col0 + 16 * g + 4 * (c & 3);
  return kr * 512 + (((col >> 3) ^ (4 * (kr & 3))) << 4) + (col & 7) * 2;
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ bf16x8 t_frag(const char* p) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 2048));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// NW = 4: waves of 128 x 128 (256 accumulator registers), one per SIMD;
// NW = 8: waves of 128 x 64, two per SIMD, so one wave's MFMAs cover the
// other's copy issue, fragment waits and barrier.
// KT: both operands K-major (TN layout).  SB: B tiles may cross segments of
// B (dma_part_seg).  TMT: tile rows, 256 or (NT only) 128, which doubles the
// tiles of a grid that would leave CUs idle (waves of 64 x 64 with NW = 8).
template <typename OutT, int NW, bool KT, bool SB = false, int TMT = TM, int TPW = 1>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4)))
void gemm_nt_256_kernel(GemmArgs g, int tiles_m, int tiles_n) {
  static_assert(TMT == TM || (TMT == 128 && !KT), "128-row tiles: NT layout only");
  static_assert(TPW == 1 || (!KT && !SB && TMT == TM), "several tiles per work-group: NT, one B segment");
  constexpr int WN = NW / 2;                 // waves along N
  constexpr int NJ = TN / WN / 32;           // 32-column blocks per wave: 4 or 2
  constexpr int MI = TMT / 64;               // 32-row blocks per wave: 4 or 2
  constexpr int CB = 32 / NW;                // 1 KB copy blocks per wave per B tile
  constexpr int CBA = TMT / 8 / NW;          // and per A tile
  constexpr int ABYTES = TMT * TK * 2, STG = ABYTES + B_BYTES;
  const int nsplit = g.ksplit > 1 ? g.ksplit : 1;
  __shared__ __attribute__((aligned(1024))) char lds[2 * STG];

  // tile (and K range) of this work-group: XCD x (= dispatch index % 8) takes
  // a consecutive run of tiles; with split K, a consecutive run of
  // (K range, tile) pairs, K range outermost, so the work-groups of one XCD
  // read the same k-rows of A and B at about the same time and each XCD's L2
  // fetches its K range once rather than every tile's rows over all of K
  const int nt = tiles_m * tiles_n;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int l32 = lane & 31, hi = lane >> 5;
  // With TPW tiles per work-group (one K range), XCD x takes its nt / 8 tiles
  // as TPW passes of its work-groups; the last k step of a tile copies the
  // next tile's first k range, and the tile leaves through the other stage,
  // so its stores drain while the next tile's MFMAs run.
#pragma unroll 1
  for (int it = 0; it < TPW; ++it) {
  int t, split = 0;
  if constexpr (TPW > 1) {
    const int xcd = blockIdx.x & 7, loc = blockIdx.x >> 3, P = nt >> 3;
    t = xcd * P + loc + it * (P / TPW);
  } else if (nsplit > 1) {
    const int W = nt * nsplit, lin = blockIdx.x + gridDim.x * blockIdx.y;
    const int xcd = lin & 7, loc = lin >> 3;
    const int q = xcd * (W >> 3) + min(xcd, W & 7) + loc;
    split = q / nt;
    t = q - split * nt;
  } else {
    const int xcd = blockIdx.x & 7, loc = blockIdx.x >> 3;
    t = xcd * (nt >> 3) + min(xcd, nt & 7) + loc;
  }
  // split K: this work-group sums k in [kbeg, kbeg + klen)
  const int klen = g.K / nsplit, kbeg = split * klen;
  const int tm = t / tiles_n, tn = t % tiles_n;
  const int m0 = tm * TMT, n0 = tn * TN;

  // A rows m0 .., B rows n0 .. (inside one segment of B, checked by the host)
  const bf16* abase = reinterpret_cast<const bf16*>(g.a) + (long)m0 * g.lda;
  const int arows = min(g.M - m0, TMT);
  int s = 0;
  if (g.b_nseg > 1 && n0 >= g.b_start[1]) s = 1;
  if (g.b_nseg > 2 && n0 >= g.b_start[2]) s = 2;
  const int seg_end = s + 1 < g.b_nseg ? g.b_start[s + 1] : g.N;
  const bf16* bbase = reinterpret_cast<const bf16*>(g.b_ptr[s]) + (long)(n0 - g.b_start[s]) * g.ldb;
  const int brows = min(seg_end - n0, TN);

  const int nk = klen / TK;
  const int kvalid = g.k_valid > 0 ? g.k_valid : g.K;
  const bf16* amat = reinterpret_cast<const bf16*>(g.a);
  const bf16* bmat = reinterpret_cast<const bf16*>(g.b_ptr[0]);
  // the next tile's operand bases (TPW > 1: K range 0, one B segment)
  const bf16* nabase = abase;
  const bf16* nbbase = bbase;
  int narows = arows, nbrows = brows;
  if constexpr (TPW > 1) {
    if (it + 1 < TPW) {
      const int P = nt >> 3;
      const int t2 = t + P / TPW, tm2 = t2 / tiles_n, tn2 = t2 % tiles_n;
      nabase = reinterpret_cast<const bf16*>(g.a) + (long)(tm2 * TMT) * g.lda;
      narows = min(g.M - tm2 * TMT, TMT);
      nbbase = reinterpret_cast<const bf16*>(g.b_ptr[0]) + (long)(tn2 * TN) * g.ldb;
      nbrows = min(g.N - tn2 * TN, TN);
    }
  }
  if (TPW == 1 || it == 0) {
  if constexpr (KT) {
    dma_tile_t<CB>(lds, amat, g.lda, m0, kvalid, kbeg, wave, lane);
    dma_tile_t<CB>(lds + ABYTES, bmat, g.ldb, n0, kvalid, kbeg, wave, lane);
  } else {
    dma_tile<CBA>(lds, abase, g.lda, arows, g.K, kbeg, wave, lane);
    if constexpr (SB) {
#pragma unroll
      for (int i = 0; i < CB; ++i) dma_part_seg<CB>(lds + ABYTES, g, n0, kbeg, wave, lane, i);
    } else {
      dma_tile<CB>(lds + ABYTES, bbase, g.ldb, brows, g.K, kbeg, wave, lane);
    }
  }
  }

  f32x16 acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // fragment addresses within a stage: row (wm*128 + i*32 + l32) of A and
  // (wn*128 + j*32 + l32) of B, chunk 2 ks + hi; the swizzle term depends on
  // l32 only, so the i / j blocks are immediate offsets.
  // K-major tiles: per block i / j instead (t_frag_off), ks as + 8192 ks.
  int aoff[4], boff[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    if constexpr (KT) {
      aoff[u] = t_frag_off(lane, wm * 128 + u * 32);
      boff[u] = ABYTES + t_frag_off(lane, wn * (NJ * 32) + (u % NJ) * 32);
    } else {
      aoff[u] = sw(wm * (TMT / 2) + l32, 2 * u + hi);
      boff[u] = ABYTES + sw(wn * (NJ * 32) + l32, 2 * u + hi);
    }
  }
  auto frag_a = [&](const char* st, int ks, int i) -> bf16x8 {
    if constexpr (KT) return t_frag(st + aoff[i] + 8192 * ks);
    else return *reinterpret_cast<const bf16x8*>(st + aoff[ks] + i * 32 * 128);
  };
  auto frag_b = [&](const char* st, int ks, int j) -> bf16x8 {
    if constexpr (KT) return t_frag(st + boff[j] + 8192 * ks);
    else return *reinterpret_cast<const bf16x8*>(st + boff[ks] + j * 32 * 128);
  };
  if (TPW == 1 || it == 0) {
    wait_dma();
    __syncthreads();
  }

  for (int kt = 0; kt < nk; ++kt) {
    const char* st = lds + (kt & 1) * STG;
    // next stage's copy, one 1 KB block after every four MFMAs (the last step
    // copies its own k range again into the idle stage, so the loop body has
    // no branch)
    char* nx = lds + ((kt + 1) & 1) * STG;
    const bool ntile = TPW > 1 && it + 1 < TPW && kt == nk - 1;
    const int knx = ntile ? 0 : kbeg + min(kt + 1, nk - 1) * TK;
    const bf16* cabase = ntile ? nabase : abase;
    const bf16* cbbase = ntile ? nbbase : bbase;
    const int carows = ntile ? narows : arows, cbrows = ntile ? nbrows : brows;
    bf16x8 fa[2][MI], fb[2][NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i) fa[0][i] = frag_a(st, 0, i);
#pragma unroll
    for (int j = 0; j < NJ; ++j) fb[0][j] = frag_b(st, 0, j);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int cur = ks & 1;
      if (ks + 1 < 4) {
#pragma unroll
        for (int i = 0; i < MI; ++i) fa[cur ^ 1][i] = frag_a(st, ks + 1, i);
#pragma unroll
        for (int j = 0; j < NJ; ++j) fb[cur ^ 1][j] = frag_b(st, ks + 1, j);
      }
#pragma unroll
      for (int i = 0; i < MI; ++i) {
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[cur][j], fa[cur][i], acc[i][j],
                                                              0, 0, 0);
        // issue points 0 .. 4 MI - 1; the CBA + CB copies go out over the
        // first half, PER at each
        constexpr int HALF = 2 * MI, PER = (CBA + CB + HALF - 1) / HALF;
        const int pt = ks * MI + i;
        __builtin_amdgcn_sched_barrier(0);
        if (pt < HALF) {
#pragma unroll
          for (int u = 0; u < PER; ++u) {
            const int blk = pt * PER + u;        // A blocks 0 .. CBA-1, then B
            if constexpr (KT) {
              if (blk < CBA) dma_part_t<CB>(nx, amat, g.lda, m0, kvalid, knx, wave, lane, blk);
              else dma_part_t<CB>(nx + ABYTES, bmat, g.ldb, n0, kvalid, knx, wave, lane, blk - CBA);
            } else {
              if (blk < CBA) dma_part<CBA>(nx, cabase, g.lda, carows, g.K, knx, wave, lane, blk);
              else if (blk < CBA + CB) {
                if constexpr (SB) dma_part_seg<CB>(nx + ABYTES, g, n0, knx, wave, lane, blk - CBA);
                else dma_part<CB>(nx + ABYTES, cbbase, g.ldb, cbrows, g.K, knx, wave, lane, blk - CBA);
              }
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    wait_dma();
    __syncthreads();
  }

  // The MFMAs take B's fragment as their first operand, so each accumulator
  // block is C^T: lane = output row l32 of the block, registers 4 q .. 4 q + 3
  // = the 4 consecutive output columns 8 q + 4 hi + 0..3.  The tile leaves
  // through LDS (free after the loop's last barrier) in MI passes of 64 rows
  // (block i of every wave): 8- or 16-byte LDS writes, then whole-row 16-byte
  // global stores.  Staging rows carry 8 elements of padding, so the 32 rows
  // one write instruction touches fall on distinct banks.  One C segment
  // (checked by the host, with 16-byte aligned rows): a uniform tile base plus
  // 32-bit offsets.
  char* cbase = reinterpret_cast<char*>(g.c_ptr[0]) +
                ((long)split * g.c_split_stride + (long)m0 * g.ldc + n0) * sizeof(OutT);
  const int ldc = (int)g.ldc;
  const int mrem = g.M - m0, nrem = g.N - n0;
  constexpr int ES = sizeof(OutT), SROWB = (TN + 8) * ES, CPRO = TN * ES / 16, EPC = 16 / ES;
  static_assert(64 * SROWB <= 2 * STG, "staging fits the operand buffers");
  static_assert(TPW == 1 || 64 * SROWB <= STG, "staging fits one stage");
  char* const ebuf = lds + (TPW > 1 ? STG : 0);
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    char* srow = ebuf + (wm * 32 + l32) * SROWB;
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int nl = wn * (NJ * 32) + j * 32 + 8 * q + 4 * hi;
        store4(reinterpret_cast<OutT*>(srow + nl * ES), acc[i][j][4 * q], acc[i][j][4 * q + 1],
               acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
      }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 64 * CPRO / (64 * NW); ++u) {
      const int e = (int)threadIdx.x + 64 * NW * u;
      const int r = e / CPRO, c = e % CPRO;
      const int ml = (r >> 5) * (TMT / 2) + i * 32 + (r & 31), nl = c * EPC;
      if (ml < mrem && nl < nrem) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(ebuf + r * SROWB + c * 16);
        char* dst = cbase + (ml * ldc + nl) * ES;
        if (nl + EPC <= nrem) {
          *reinterpret_cast<f32x4*>(dst) = v;
        } else {
          // the row's last columns, one element at a time (constant indices
          // keep v in registers)
          const auto ve = __builtin_bit_cast(OutV<OutT>, v);
#pragma unroll
          for (int x = 0; x < EPC; ++x)
            if (nl + x < nrem) reinterpret_cast<OutT*>(dst)[x] = ve[x];
        }
      }
    }
    __syncthreads();
  }
  }
}

}  // namespace

// Launches the 256 x 256 NT kernel when the shape suits it: K a multiple of 64,
// every B segment starting at a multiple of 256, one C segment, row strides
// that keep 16-byte alignment, and enough tiles to fill the chip.  Returns false (nothing
// launched) otherwise.
bool launch_gemm_nt_big(const GemmArgs& g, bool out_f32, hipStream_t s, hipError_t* err,
                        GemmLayout layout) {
  if (g.K % TK != 0 || g.K <= 0 || g.lda % 8 != 0 || g.ldb % 8 != 0 || g.c_nseg != 1)
    return false;
  // C rows (and split-K slices) 16-byte aligned for the 4-column stores
  if (g.ldc % 4 != 0 || reinterpret_cast<uintptr_t>(g.c_ptr[0]) % 16 != 0 ||
      (g.ksplit > 1 && g.c_split_stride % 4 != 0))
    return false;
  const bool kt = layout == GemmLayout::TN;
  if (layout == GemmLayout::NN) return false;
  if (kt) {
    // fp32 output only (the weight gradients), one B segment, 32-bit offsets
    const long kv = g.k_valid > 0 ? g.k_valid : g.K;
    if (!out_f32 || g.b_nseg != 1 || kv * g.lda * 2 >= (1L << 31) || kv * g.ldb * 2 >= (1L << 31))
      return false;
  }
  if ((long)TM * g.ldc * 4 >= (1L << 31)) return false;
  // B segments starting inside a tile: per-block segment lookup (NT only)
  bool sb = false;
  for (int i = 1; i < g.b_nseg; ++i) {
    if (g.b_start[i] % 8 != 0) return false;
    if (g.b_start[i] % TN != 0) sb = true;
  }
  if (sb && (kt || (long)8 * g.ldb * 2 >= (1L << 31))) return false;
  if ((long)TM * g.lda * 2 >= (1L << 31) || (long)TN * g.ldb * 2 >= (1L << 31)) return false;
  const int tiles_m = (g.M + TM - 1) / TM, tiles_n = (g.N + TN - 1) / TN;
  const int nsplit = g.ksplit > 1 ? g.ksplit : 1;
  if (nsplit > 1 && (!out_f32 || (g.K / nsplit) % TK != 0 || g.K % nsplit != 0)) return false;
  if ((long)tiles_m * tiles_n * nsplit < 64) return false;
  // fewer 256-row tiles than CUs (a narrow output such as the backward's
  // dY W_o with N = 512): 128-row tiles, twice as many work-groups
  if (!kt && !sb && nsplit == 1 && tiles_m * tiles_n < 256) {
    const int tm128 = (g.M + 127) / 128;
    dim3 grid128(tm128 * tiles_n);
    if (out_f32)
      hipLaunchKernelGGL((gemm_nt_256_kernel<float, 8, false, false, 128>), grid128, dim3(512), 0, s,
                         g, tm128, tiles_n);
    else
      hipLaunchKernelGGL((gemm_nt_256_kernel<bf16, 8, false, false, 128>), grid128, dim3(512), 0, s,
                         g, tm128, tiles_n);
    *err = hipGetLastError();
    return true;
  }
  dim3 grid(tiles_m * tiles_n, nsplit);
  // eight waves of 128 x 64, two per SIMD, also when the grid is one round:
  // the second wave of a SIMD covers the other's fragment waits, copy issue
  // and barrier (measured faster than four waves of 128 x 128 on every layout
  // here, although those read less LDS per MFMA)
  if (kt)
    hipLaunchKernelGGL((gemm_nt_256_kernel<float, 8, true>), grid, dim3(512), 0, s, g, tiles_m, tiles_n);
  else if (sb && out_f32)
    hipLaunchKernelGGL((gemm_nt_256_kernel<float, 8, false, true>), grid, dim3(512), 0, s, g, tiles_m, tiles_n);
  else if (sb)
    hipLaunchKernelGGL((gemm_nt_256_kernel<bf16, 8, false, true>), grid, dim3(512), 0, s, g, tiles_m, tiles_n);
  else if (out_f32)
    hipLaunchKernelGGL((gemm_nt_256_kernel<float, 8, false>), grid, dim3(512), 0, s, g, tiles_m, tiles_n);
  // bf16 output over two or more rounds of tiles (the up-projection, the
  // backward's dx): each work-group takes two tiles, the first tile's stores
  // drain during the second tile's MFMAs and the second tile's first stage
  // loads during the first tile's last k step (proj_up 45.0 -> 43.6 us)
  else if (nsplit == 1 && g.b_nseg == 1 && (g.K / TK) % 2 == 0 && tiles_m * tiles_n >= 512 &&
           (tiles_m * tiles_n) % 16 == 0)
    hipLaunchKernelGGL((gemm_nt_256_kernel<bf16, 8, false, false, TM, 2>),
                       dim3(tiles_m * tiles_n / 2), dim3(512), 0, s, g, tiles_m, tiles_n);
  else
    hipLaunchKernelGGL((gemm_nt_256_kernel<bf16, 8, false>), grid, dim3(512), 0, s, g, tiles_m, tiles_n);
  *err = hipGetLastError();
  return true;
}

}  // namespace cca

// ------------------------------------------------------------------ small M
// C = A B^T for few rows of A (the decode step's tokens): work-group = 32
// output columns x 32 rows; its eight waves split K eight ways, each issuing
// the global loads of up to eight 16-wide k steps (both fragments, 16 bytes per
// lane, straight into registers) before their chain of
// v_mfma_f32_32x32x16_bf16, so one memory round trip covers most of K; the
// eight partial tiles are summed in LDS in a fixed order.  B's rows may come
// from up to three segments (the concatenated W_q | W_k | W_v).  Requires
// K % 128 == 0.
namespace cca {
namespace {

constexpr int SW = 8;   // waves per small-M work-group

__device__ __forceinline__ void store_small(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_small(bf16* p, float v) { *p = (bf16)v; }

template <typename OutT>
__global__ __launch_bounds__(64 * SW) void gemm_nt_small_kernel(GemmArgs g) {
  __shared__ float part[SW][32][33];
  const int n0 = blockIdx.x * 32, m0 = blockIdx.y * 32;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int m = m0 + l32, n = n0 + l32;
  // rows past M or N read row 0 (valid memory); their results are never stored
  const bf16* arow = reinterpret_cast<const bf16*>(g.a) + (long)(m < g.M ? m : 0) * g.lda;
  const int nn = n < g.N ? n : 0;
  int s = 0;
  if (g.b_nseg > 1 && nn >= g.b_start[1]) s = 1;
  if (g.b_nseg > 2 && nn >= g.b_start[2]) s = 2;
  const bf16* brow = reinterpret_cast<const bf16*>(g.b_ptr[s]) + (long)(nn - g.b_start[s]) * g.ldb;
  const int kw = g.K / SW, k0 = wave * kw;
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
  for (int kb = k0; kb < k0 + kw; kb += 128) {
    bf16x8 af[8], bfr[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int k = kb + 16 * i + 8 * hi;
      if (kb + 16 * i < k0 + kw) {
        af[i] = *reinterpret_cast<const bf16x8*>(arow + k);
        bfr[i] = *reinterpret_cast<const bf16x8*>(brow + k);
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (kb + 16 * i < k0 + kw)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[i], acc, 0, 0, 0);
  }
  // D layout: lane holds column l32 (n), rows 8*(r/4) + 4*hi + r%4 (m)
#pragma unroll
  for (int r = 0; r < 16; ++r) part[wave][8 * (r >> 2) + 4 * hi + (r & 3)][l32] = acc[r];
  __syncthreads();
  for (int e = threadIdx.x; e < 32 * 32; e += 64 * SW) {
    const int mi = e / 32, ni = e % 32;
    if (m0 + mi >= g.M || n0 + ni >= g.N) continue;
    float v = part[0][mi][ni];
#pragma unroll
    for (int w = 1; w < SW; ++w) v += part[w][mi][ni];
    int cs = 0;
    if (g.c_nseg > 1 && m0 + mi >= g.c_start[1]) cs = 1;
    if (g.c_nseg > 2 && m0 + mi >= g.c_start[2]) cs = 2;
    OutT* crow = reinterpret_cast<OutT*>(g.c_ptr[cs]) + (long)(m0 + mi - g.c_start[cs]) * g.ldc;
    store_small(crow + n0 + ni, v);
  }
}

}  // namespace

// Launches the small-M kernel for M <= 64 rows (decode); false otherwise.
bool launch_gemm_nt_small(const GemmArgs& g, bool out_f32, hipStream_t s, hipError_t* err) {
  if (g.M > 64 || g.K % (16 * SW) != 0 || g.K <= 0 || g.lda % 8 != 0 || g.ldb % 8 != 0)
    return false;
  dim3 grid((g.N + 31) / 32, (g.M + 31) / 32);
  if (out_f32)
    hipLaunchKernelGGL(gemm_nt_small_kernel<float>, grid, dim3(64 * SW), 0, s, g);
  else
    hipLaunchKernelGGL(gemm_nt_small_kernel<bf16>, grid, dim3(64 * SW), 0, s, g);
  *err = hipGetLastError();
  return true;
}

}  // namespace cca

// ------------------------------------------------------------------ skinny, split K
// C = A B^T for the decode step's few rows (M <= 256) spread over the whole
// chip: work-group = 32 rows x 32 columns x one of KS slices of K (KS chosen so
// that the grid holds about 256 work-groups).  Its four waves take a quarter
// of the slice each and issue the loads of four 16-wide k steps (both
// fragments, 16 bytes per lane) together before their MFMAs; the four partial
// tiles are summed in LDS in a fixed order and written to an fp32 partial
// buffer [KS, Mp, Np]; a second kernel sums the KS partials in order and
// writes C (fp32 or bf16).  Same operand conventions as the small-M kernel.
namespace cca {
namespace {

constexpr int SK_WGS = 256;      // target work-groups
constexpr int SK_MAX_PART = SK_WGS * 32 * 32;   // partial floats at most (KS > 1)

__global__ __launch_bounds__(256) void gemm_skinny_partial_kernel(GemmArgs g, int kc, int Mp,
                                                                  int Np, float* part) {
  __shared__ float red[4][32][33];
  const int n0 = blockIdx.x * 32, m0 = blockIdx.y * 32, ks = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int m = m0 + l32, n = n0 + l32;
  // rows past M or N read row 0 (valid memory); their sums land in the
  // partial buffer's padding and are never read
  const bf16* arow = reinterpret_cast<const bf16*>(g.a) + (long)(m < g.M ? m : 0) * g.lda;
  const int nn = n < g.N ? n : 0;
  int sg = 0;
  if (g.b_nseg > 1 && nn >= g.b_start[1]) sg = 1;
  if (g.b_nseg > 2 && nn >= g.b_start[2]) sg = 2;
  const bf16* brow =
      reinterpret_cast<const bf16*>(g.b_ptr[sg]) + (long)(nn - g.b_start[sg]) * g.ldb;
  const int kw = kc / 4, k0 = ks * kc + wave * kw;
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
  for (int kb = k0; kb < k0 + kw; kb += 64) {
    bf16x8 af[4], bfr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k = kb + 16 * i + 8 * hi;
      af[i] = *reinterpret_cast<const bf16x8*>(arow + k);
      bfr[i] = *reinterpret_cast<const bf16x8*>(brow + k);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[i], acc, 0, 0, 0);
  }
  // D layout: lane holds column l32 (n), rows 8*(r/4) + 4*hi + r%4 (m)
#pragma unroll
  for (int r = 0; r < 16; ++r) red[wave][8 * (r >> 2) + 4 * hi + (r & 3)][l32] = acc[r];
  __syncthreads();
  float* pb = part + ((long)ks * Mp + m0) * Np + n0;
  for (int e = threadIdx.x; e < 32 * 32; e += 256) {
    const int mi = e / 32, ni = e % 32;
    pb[(long)mi * Np + ni] = ((red[0][mi][ni] + red[1][mi][ni]) + red[2][mi][ni]) + red[3][mi][ni];
  }
}

__device__ __forceinline__ void store4s(float* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }
__device__ __forceinline__ void store4s(bf16* p, f32x4 v) {
  *reinterpret_cast<bf16x4*>(p) = bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
}

template <typename OutT>
__global__ __launch_bounds__(256) void gemm_skinny_reduce_kernel(GemmArgs g, int KS, int Mp, int Np,
                                                                 const float* part) {
  const int nq = g.N / 4;
  const long q = (long)blockIdx.x * 256 + threadIdx.x;   // group of 4 columns
  if (q >= (long)g.M * nq) return;
  const int m = (int)(q / nq), n = (int)(q % nq) * 4;
  f32x4 s = *reinterpret_cast<const f32x4*>(part + (long)m * Np + n);
  for (int z = 1; z < KS; ++z) s += *reinterpret_cast<const f32x4*>(part + ((long)z * Mp + m) * Np + n);
  int cs = 0;
  if (g.c_nseg > 1 && m >= g.c_start[1]) cs = 1;
  if (g.c_nseg > 2 && m >= g.c_start[2]) cs = 2;
  store4s(reinterpret_cast<OutT*>(g.c_ptr[cs]) + (long)(m - g.c_start[cs]) * g.ldc + n, s);
}

}  // namespace

size_t gemm_skinny_part_floats() { return SK_MAX_PART; }

// Launches the split-K pair when it suits the shape (M <= 256, fewer than 64
// output tiles of 32 x 32, K a multiple of 256 so that four waves get whole
// 16-wide steps in every slice, N and ldc multiples of 4 for the 4-wide output
// stores, and at least two slices to go around); false (nothing launched)
// otherwise.  With keep set only the partials are written, for a consumer
// that sums them itself.
bool launch_gemm_skinny(const GemmArgs& g, bool out_f32, float* part, hipStream_t s,
                        hipError_t* err, SkinnyPartials* keep) {
  if (part == nullptr || g.M <= 0 || g.M > 256 || g.K % 256 != 0 || g.lda % 8 != 0 ||
      g.ldb % 8 != 0 || g.N % 4 != 0 || g.ldc % 4 != 0)
    return false;
  const int mb = (g.M + 31) / 32, nb = (g.N + 31) / 32;
  // with 64 or more 32 x 32 tiles the small-M kernel (one launch, eight
  // waves per tile) fills enough CUs; the second launch would cost more
  if (mb * nb >= 64) return false;
  int KS = 1;
  while ((long)mb * nb * KS * 2 <= SK_WGS && g.K % (KS * 2 * 256) == 0) KS *= 2;
  if (KS < 2) return false;
  const int Mp = mb * 32, Np = nb * 32;
  if ((long)KS * Mp * Np > SK_MAX_PART) return false;
  hipLaunchKernelGGL(gemm_skinny_partial_kernel, dim3(nb, mb, KS), dim3(256), 0, s, g, g.K / KS,
                     Mp, Np, part);
  if (keep != nullptr) {
    *keep = SkinnyPartials{part, KS, (long)Mp * Np, Np};
    *err = hipGetLastError();
    return true;
  }
  const long groups = (long)g.M * (g.N / 4);
  const dim3 rgrid((unsigned)((groups + 255) / 256));
  if (out_f32)
    hipLaunchKernelGGL(gemm_skinny_reduce_kernel<float>, rgrid, dim3(256), 0, s, g, KS, Mp, Np,
                       (const float*)part);
  else
    hipLaunchKernelGGL(gemm_skinny_reduce_kernel<bf16>, rgrid, dim3(256), 0, s, g, KS, Mp, Np,
                       (const float*)part);
  *err = hipGetLastError();
  return true;
}

}  // namespace cca

// ------------------------------------------------------------------ helpers
// Transpose of a bf16 matrix through a 64 x 64 LDS tile (16-byte loads and
// stores), and the fixed-order sum of split-K partials.  They let the
// backward pass run its transposed-operand GEMMs on the NT kernel above.
namespace cca {
namespace {

__global__ __launch_bounds__(256) void transpose_bf16_kernel(const bf16* in, long ld_in, int R,
                                                             int C, int Rp, bf16* out,
                                                             long ld_out) {
  __shared__ bf16 tile[64][64 + 2];
  const int r0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  for (int f = threadIdx.x; f < 64 * 8; f += 256) {
    const int row = f >> 3, c8 = (f & 7) * 8;
    const int r = r0 + row, c = c0 + c8;
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (bf16)0.0f;
    if (r < R && c < C) v = *reinterpret_cast<const bf16x8*>(in + (long)r * ld_in + c);
#pragma unroll
    for (int e = 0; e < 8; ++e) tile[row][c8 + e] = v[e];
  }
  __syncthreads();
  for (int f = threadIdx.x; f < 64 * 8; f += 256) {
    const int col = f >> 3, r8 = (f & 7) * 8;
    const int c = c0 + col, r = r0 + r8;
    if (c >= C || r >= Rp) continue;
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = tile[r8 + e][col];
    *reinterpret_cast<bf16x8*>(out + (long)c * ld_out + r) = v;
  }
}

struct ReduceArgs {
  const float* part;
  int ksplit, M, N;
  float* out[3];
  int start[3];
  int nseg;
  long ld;
};

__global__ __launch_bounds__(256) void splitk_reduce_kernel(ReduceArgs a) {
  const long e = ((long)blockIdx.x * 256 + threadIdx.x) * 4;
  const long total = (long)a.M * a.N;
  if (e >= total) return;
  f32x4 s = *reinterpret_cast<const f32x4*>(a.part + e);
  for (int z = 1; z < a.ksplit; ++z) s += *reinterpret_cast<const f32x4*>(a.part + z * total + e);
  const int m = (int)(e / a.N), n = (int)(e % a.N);
  int sg = 0;
  if (a.nseg > 1 && m >= a.start[1]) sg = 1;
  if (a.nseg > 2 && m >= a.start[2]) sg = 2;
  *reinterpret_cast<f32x4*>(a.out[sg] + (long)(m - a.start[sg]) * a.ld + n) = s;
}

}  // namespace

hipError_t launch_transpose_bf16(const void* in, long ld_in, int R, int C, int Rp, void* out,
                                 long ld_out, hipStream_t s) {
  if (C % 8 != 0 || Rp % 8 != 0 || Rp < R || ld_in % 8 != 0 || ld_out % 8 != 0)
    return hipErrorInvalidValue;
  dim3 grid((Rp + 63) / 64, (C + 63) / 64);
  hipLaunchKernelGGL(transpose_bf16_kernel, grid, dim3(256), 0, s, (const bf16*)in, ld_in, R, C,
                     Rp, (bf16*)out, ld_out);
  return hipGetLastError();
}

hipError_t launch_splitk_reduce(const float* part, int ksplit, int M, int N, float* const out[3],
                                const int start[3], int nseg, long ld, hipStream_t s) {
  if (N % 4 != 0 || ld % 4 != 0) return hipErrorInvalidValue;
  ReduceArgs a{};
  a.part = part; a.ksplit = ksplit; a.M = M; a.N = N; a.nseg = nseg; a.ld = ld;
  for (int i = 0; i < 3; ++i) { a.out[i] = out[i]; a.start[i] = start[i]; }
  const long total = (long)M * N / 4;
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((total + 255) / 256), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace cca
