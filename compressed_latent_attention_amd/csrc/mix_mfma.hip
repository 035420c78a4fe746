// cca_mix for bf16, d = 128, on MFMA: the causal grouped convolution of q~ and
// k~ (CCA-es §2.B.1 "Mezcla Convolucional"), QK-mean (§2.B.2), value shift
// (§2.B.3) and RoPE (§3 item 2) in one pass per (64 tokens, KV group).
//
// The convolution of one head is a GEMM, taken transposed: out[c, t] =
// sum_{j, c'} A_j[c, c'] u[t - j, c'] with M = channels, N = tokens, K = k * d.
// The bf16 latent tiles the work-group needs (k~, v~ and up to two q~ heads, 64
// tokens plus a 4-row halo before them, enough for k <= 4 taps and the
// one-token value shift) are read with 16-byte buffer loads, all issued in one
// round at the start, so a work-group waits for memory once, and stored to LDS
// in rows padded to 272 bytes: the MFMA operand reads (32 consecutive token
// rows, one 16-byte chunk each) are free of bank conflicts.  Operand A is the
// bf16 tap row A_j[c, 8 channels] read from L2, operand B the tile.  With lane
// = token and each 4 registers = 4 consecutive channels, everything QK-mean
// needs (the same token and channels of the group's query heads and its K head)
// sits in one lane, the epilogue reads the pre-convolution values and the RoPE
// cos / sin of 4 channels at once, and writes 4 outputs at once.
//
// Wave w of the 4 owns a quarter of the output channels, all 64 tokens: MFMA
// row m < 16 is channel 16 w + m and row m >= 16 its RoPE partner
// 64 + 16 w + m - 16, so a rotation pair sits in registers r and r + 8 of one
// lane; every tap fragment feeds the MFMAs of both 32-token blocks, and the
// four waves together read each tap row of the group once.
// Work-groups are numbered so the KV groups of one token tile run on the same
// XCD (ids 8 apart): the second reads the tile's RoPE rows from that XCD's L2.
#include "cca_internal.h"

#include <type_traits>

namespace cca {
namespace {

constexpr int HALO = 4;                     // staged rows before the tile (>= kMaxConv - 1)
constexpr int NQS = 2;                      // q~ tiles resident at once
constexpr int XCDS = 8;

// Sizes that follow the head dimension D (128 or 64).  The 4 waves split the
// D / 32 channel groups of 32 MFMA columns first, then the tokens: with
// D = 64 two waves share each channel group and the tile is 128 tokens, so a
// wave still holds two 32-token blocks.
template <int D>
struct MGeom {
  static constexpr int NCW = D / 32;                 // channel groups (waves per token group)
  static constexpr int NTG = 4 / NCW;                // token groups of 64
  static constexpr int TW = 64 * NTG;                // tokens per work-group
  static constexpr int TROWS = TW + HALO;            // tile row i = token t0 - HALO + i
  static constexpr int ROWB = 2 * D + 16;            // LDS row stride in bytes (one chunk of pad)
  static constexpr int TBYTES = TROWS * ROWB;
  static constexpr int CPR = D / 8;                  // 16-byte chunks per row
  static constexpr int CHUNKS = TROWS * CPR;         // 16-byte chunks per tile
  static constexpr int NKS = D / 16;                 // 16-channel k-steps of one tap
};

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

// The latent tiles of column blocks cols[0 .. n) (D channels each), rows
// t0 - HALO .. t0 + TW - 1, into LDS tiles dst[0 .. n): every load of the
// work-group is issued before the first LDS store.  Each resource spans the
// rows inside [0, S): rows before 0 (an offset that wraps) and past S read as
// zero without a branch.
template <int D, int NMAX>
__device__ __forceinline__ void load_tiles(char* const (&dst)[NMAX], const int (&cols)[NMAX],
                                           int n, const bf16* qkv_b, int nqkv, int S, int t0) {
  constexpr int TW = MGeom<D>::TW, CHUNKS = MGeom<D>::CHUNKS, CPR = MGeom<D>::CPR;
  constexpr int ROWB = MGeom<D>::ROWB;
  constexpr int PER = (CHUNKS + 255) / 256;  // chunks per thread per tile
  const int r0 = max(t0 - HALO, 0), r1 = min(S, t0 + TW);
  bf16x8 v[NMAX][PER];
#pragma unroll
  for (int i = 0; i < NMAX; ++i) {
    if (i >= n) break;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(qkv_b + (long)r0 * nqkv + cols[i]), 0,
        r1 > r0 ? ((r1 - r0 - 1) * nqkv + D) * 2 : 0, 0x00020000);
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int e = min((int)threadIdx.x + 256 * p, CHUNKS - 1);
      const int r = e / CPR, c = e % CPR;
      const int t = t0 - HALO + r;
      v[i][p] = __builtin_bit_cast(
          bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rs, ((t - r0) * nqkv + c * 8) * 2, 0, 0));
    }
  }
#pragma unroll
  for (int i = 0; i < NMAX; ++i) {
    if (i >= n) break;
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int e = (int)threadIdx.x + 256 * p;
      if (e < CHUNKS)
        *reinterpret_cast<bf16x8*>(dst[i] + (e / CPR) * ROWB + (e % CPR) * 16) = v[i][p];
    }
  }
}

typedef f32x16 Acc2[2];                     // [channel block]

__device__ __forceinline__ void zero(Acc2& a) {
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) a[j][r] = 0.0f;
}

// The tap fragments of lag j this lane feeds to its MFMAs: output channel ch
// (its MFMA row), input channels 16 ks + 8 hi .. + 7 for ks = 0 .. D / 16 - 1.
template <int D>
__device__ __forceinline__ void load_taps(bf16x8 (&bf)[MGeom<D>::NKS], const bf16* taps, int j,
                                          int ch, int hi) {
  const bf16* trow = taps + ((long)j * D + ch) * D + hi * 8;
#pragma unroll
  for (int ks = 0; ks < MGeom<D>::NKS; ++ks)
    bf[ks] = *reinterpret_cast<const bf16x8*>(trow + ks * 16);
}

// acc[mb] = conv of the head whose tile is at `tile` for the wave's token
// block mb, transposed (rows = output channels, columns = tokens): A =
// taps[j][ch][c_in] for output channel ch of MFMA row l32, B = the tile rows of
// tokens tb0 + 32 mb + l32 at lag j (tile row tb0 + 32 mb + l32 - j + HALO).
// cur holds lag 0's tap fragments on entry (requested earlier); each lag's
// MFMAs run while the next lag's fragments are in flight, and after the last
// lag those of the next head's lag 0 (next_taps; none when null), which cur
// holds on return.  Each fragment serves both token blocks.
template <int D>
__device__ __forceinline__ void conv_head(Acc2& acc, const char* tile, const bf16* taps, int k,
                                          int ch, int lane, int tb0,
                                          bf16x8 (&cur)[MGeom<D>::NKS], const bf16* next_taps) {
  constexpr int NKS = MGeom<D>::NKS, ROWB = MGeom<D>::ROWB;
  const int l32 = lane & 31, hi = lane >> 5;
  // lag j; the first one starts both chains from zero
  auto lag = [&](int j, auto first) {
    bf16x8 nxt[NKS];
    const bool more = j + 1 < k;
    if (more) load_taps<D>(nxt, taps, j + 1, ch, hi);
    else if (next_taps) load_taps<D>(nxt, next_taps, 0, ch, hi);
    __builtin_amdgcn_sched_barrier(0);       // the requests go out before the MFMAs
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int row = tb0 + 32 * mb + l32 - j + HALO;
        const bf16x8 u = *reinterpret_cast<const bf16x8*>(tile + row * ROWB + (2 * ks + hi) * 16);
        if (decltype(first)::value && ks == 0)
          acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur[ks], u, f32x16{}, 0, 0, 0);
        else
          acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur[ks], u, acc[mb], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);     // keep the B reads next to their MFMAs
    }
    if (more || next_taps) {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) cur[ks] = nxt[ks];
    }
  };
  lag(0, std::true_type{});
  for (int j = 1; j < k; ++j) lag(j, std::false_type{});
}

// Channels c0 .. c0 + 3 of tile row r as floats (one 8-byte LDS read).
template <int D>
__device__ __forceinline__ f32x4 tile_vec4(const char* tile, int r, int c0) {
  const bf16x4 v = *reinterpret_cast<const bf16x4*>(tile + r * MGeom<D>::ROWB + c0 * 2);
  return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}

// cos / sin of RoPE pairs p0 .. p0 + 3 of tile token tr (the last token inside
// the sequence past its end, whose results are never stored): two 16-byte
// loads; (1, 0) without RoPE.
template <int D>
__device__ __forceinline__ void load_rope4(f32x4& cs, f32x4& sn, const float2* rope_t0, int tr,
                                           int p0, int nrem) {
  if (rope_t0) {
    const float* rp = reinterpret_cast<const float*>(rope_t0 + min(tr, nrem - 1) * (D / 2) + p0);
    const f32x4 r0 = *reinterpret_cast<const f32x4*>(rp);
    const f32x4 r1 = *reinterpret_cast<const f32x4*>(rp + 4);
    cs = f32x4{r0[0], r0[2], r1[0], r1[2]};
    sn = f32x4{r0[1], r0[3], r1[1], r1[3]};
  } else {
    cs = f32x4{1.f, 1.f, 1.f, 1.f};
    sn = f32x4{0.f, 0.f, 0.f, 0.f};
  }
}

// 4 values to channels c0 .. c0 + 3 of staging row r (one 8-byte LDS write).
template <int D>
__device__ __forceinline__ void stage4(char* so, int r, int c0, const f32x4& v) {
  const bf16x4 b = {(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
  *reinterpret_cast<bf16x4*>(so + r * MGeom<D>::ROWB + c0 * 2) = b;
}

// Rows 0 .. HALO - 1 of the first tile of a chunk (tokens -4 .. -1) from the
// rolling state: st holds lag 1 of this tile's D channels, lag l at + (l - 1)
// * lag_stride; lags past nlag are zero.
template <int D>
__device__ __forceinline__ void fill_halo(char* tile, const bf16* st, int nlag, long lag_stride) {
  for (int e = threadIdx.x; e < HALO * D; e += 256) {
    const int r = e / D, c = e % D, lag = HALO - r;
    const bf16 v = lag <= nlag ? st[(lag - 1) * lag_stride + c] : (bf16)0.0f;
    *reinterpret_cast<bf16*>(tile + r * MGeom<D>::ROWB + c * 2) = v;
  }
}

// GC: the group size when known at compile time (1 or 2: every q~ tile stays
// resident, so the K side's pre-convolution group mean is read back from LDS
// instead of being summed in registers, and the head loop unrolls), 0 for any
// other group size.
// VARLEN (D = 128): a chunk of a variable-length batch (vm, 64-token tiles in vm.blk):
// sequence b's tokens are latent rows vm.tok[b] .., at positions vm.start[b]
// ..; the conv and shift history before its first token comes from a.state;
// Q'' goes to the packed [Hq][T][d] (T = a.S), K'' and V' to the caches at
// their positions, and no V'^T is written.
// A variable-length launch, and the general group size (GC = 0: the group
// loop is not unrolled and the pre-convolution group mean stays in
// registers), run one work-group per CU with the full register file: at two
// per CU they spill (the general instance 112 registers, its 16x-layer mix
// 70 us against 46 us at one per CU).  The body sits in the kernel template
// itself: moved into a device function it compiles to a slower schedule of
// the same arithmetic.
// NOQ: the attention forms Q'' itself (fused Q): the query heads are still
// convolved for the key side's group means, but no Q'' is written.
struct NoMap {};
template <int D, int GC, bool VARLEN, bool NOQ, typename Map>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(VARLEN || GC == 0 ? 1 : 2,
                                                                     VARLEN || GC == 0 ? 1 : 2)))
void mix_fwd_mfma_kernel(MixArgs a, int ntiles8, Map vm) {
  // no implicit contraction: every fused multiply-add is written out, so the
  // instances with and without Q'' (and the attention's fused-Q prologue)
  // compute K'' and Q'' bit for bit alike
#pragma clang fp contract(off)
  using MG = MGeom<D>;
  constexpr int TW = MG::TW, TBYTES = MG::TBYTES, ROWB = MG::ROWB;
  static_assert(!VARLEN || D == 128, "variable-length chunks use 64-token tiles");
  constexpr bool QRES = GC > 0;
  __shared__ __attribute__((aligned(1024))) char lds[(2 + NQS) * TBYTES];
  char* tk = lds;                            // k~ tile
  char* tv = lds + TBYTES;                   // v~ tile
  char* tq = lds + 2 * TBYTES;               // q~ tiles, NQS slots
  const Dims& dm = a.dm;
  const int G = GC > 0 ? GC : dm.G;
  // (tile, KV group, sequence) from the work-group id: the Hkv groups of tiles
  // 8 i .. 8 i + 7 take ids 8 Hkv i + 8 g + (tile % 8)
  const int q = blockIdx.x % (ntiles8 * dm.Hkv);
  const int g = (q % (XCDS * dm.Hkv)) / XCDS;
  const int tile = (q / (XCDS * dm.Hkv)) * XCDS + q % XCDS;
  int b, t0, S, pos0;
  long lat0, q_row0, q_hstride;              // latent row of token 0; Q'' row of (head 0, token 0)
  if constexpr (!VARLEN) {
    b = blockIdx.x / (ntiles8 * dm.Hkv);
    S = a.S;
    t0 = tile * TW;
    pos0 = 0;
    lat0 = (long)b * S;
    q_row0 = (long)b * dm.Hq * S;
    q_hstride = S;
  } else {
    if (tile >= vm.blk[vm.B]) return;
    int lo = 0, hi2 = vm.B - 1;             // last b with blk[b] <= tile
    while (lo < hi2) {
      const int mid = (lo + hi2 + 1) >> 1;
      if (vm.blk[mid] <= tile) lo = mid; else hi2 = mid - 1;
    }
    b = lo;
    S = vm.tok[b + 1] - vm.tok[b];
    t0 = (tile - vm.blk[b]) * TW;
    pos0 = vm.start[b];
    lat0 = vm.tok[b];
    q_row0 = vm.tok[b];
    q_hstride = a.S;
  }
  if (t0 >= S) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int cw = MG::NTG == 1 ? wave : wave % MG::NCW;       // channel group of this wave
  const int tb0 = MG::NTG == 1 ? 0 : 64 * (wave / MG::NCW);  // first tile token of its two blocks
  // output channel of MFMA row l32 (the tap row this lane loads): rows 0..15
  // are channels 16 cw + 0..15, rows 16..31 their RoPE partners D / 2 further
  const int ch = l32 < 16 ? 16 * cw + l32 : D / 2 + 16 * cw + l32 - 16;
  const bf16* qkv_b = reinterpret_cast<const bf16*>(a.qkv) + lat0 * dm.nqkv;
  const float A = (dm.flags & kQkPre) ? 0.5f : 0.0f;
  const float Bc = (dm.flags & kQkPost) ? 0.5f : 0.0f;
  const bool rope = (dm.flags & kRope) != 0;
  // accumulator of token block mb: the lane holds tile token tb0 + 32 mb + l32;
  // registers 4 g .. 4 g + 3 (g = 0, 1) channels 16 cw + 8 g + 4 hi + 0..3 and
  // registers 8 + 4 g .. their RoPE partners D / 2 further (MFMA row 8 (r / 4) +
  // 4 hi + r % 4 is channel ch of lane row l32 = that row)

  const bf16* const taps_q = reinterpret_cast<const bf16*>(a.conv_q);
  const bf16* const taps_k = reinterpret_cast<const bf16*>(a.conv_k) + (long)g * dm.kk * D * D;
  auto qtaps = [&](int h) { return taps_q + (long)h * dm.kq * D * D; };
  // the K head's lag-0 taps, then every tile the work-group needs, in one round
  bf16x8 tf[MG::NKS];
  load_taps<D>(tf, taps_k, 0, ch, hi);
  {
    char* const dst[2 + NQS] = {tk, tv, tq, tq + TBYTES};
    const int cols[2 + NQS] = {dm.nq + g * D, dm.nq + dm.nk + g * D, g * G * D, (g * G + 1) * D};
    load_tiles<D>(dst, cols, 2 + min(G, NQS), qkv_b, dm.nqkv, S, t0);
  }
  // the state: [q~ lags 1..kq-1 | k~ lags 1..kk-1 | v~ lag 1], most recent first
  const bf16* st = VARLEN ? reinterpret_cast<const bf16*>(a.state) + (long)b * dm.state_w : nullptr;
  const long st_k = (long)(dm.kq - 1) * dm.nq, st_v = st_k + (long)(dm.kk - 1) * dm.nk;
  if (VARLEN && t0 == 0) {
    __syncthreads();                         // the zero halo rows are stored
    fill_halo<D>(tk, st + st_k + g * D, dm.kk - 1, dm.nk);
    fill_halo<D>(tv, st + st_v + g * D, 1, dm.nk);
    for (int i = 0; i < min(G, NQS); ++i)
      fill_halo<D>(tq + i * TBYTES, st + (g * G + i) * D, dm.kq - 1, dm.nq);
  }
  const float2* rope_t0 = rope ? a.rope + (long)(pos0 + t0) * (D / 2) : nullptr;
  __syncthreads();

  // value shift from the v~ tile: V'[t, c] = v~[t - 1, c] for the last s_v
  // channels (tile row tr + HALO - 1; row HALO - 1 is token t0 - 1, zero
  // before token 0), else v~[t, c]
  const int first_shift = (dm.flags & kVShift) ? D - dm.sv : D;
  bf16* vo = a.v_out ? reinterpret_cast<bf16*>(a.v_out) + ((long)(b * dm.Hkv + g) * S) * D
                     : nullptr;
  bf16* vo2 = a.v_out2 ? reinterpret_cast<bf16*>(a.v_out2) +
                             ((long)(b * dm.Hkv + g) * a.cap2 + pos0) * D
                       : nullptr;
  // the 8 channels c8 .. c8 + 7 of V' at tile token tr: one 16-byte read of
  // the token's row, and of the row before when the chunk reaches the shifted
  // channels
  auto vchunk = [&](int tr, int c8) {
    bf16x8 v = *reinterpret_cast<const bf16x8*>(tv + (tr + HALO) * ROWB + c8 * 2);
    if (c8 + 8 > first_shift) {
      const bf16x8 p = *reinterpret_cast<const bf16x8*>(tv + (tr + HALO - 1) * ROWB + c8 * 2);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (c8 + i >= first_shift) v[i] = p[i];
    }
    return v;
  };
  if (vo || vo2) {
    // thread = (token, 8 channels): 16-byte stores
    for (int e = threadIdx.x; e < TW * (D / 8); e += 256) {
      const int tr = e / (D / 8), c8 = (e % (D / 8)) * 8;
      const int t = t0 + tr;
      if (t >= S) break;
      const bf16x8 v = vchunk(tr, c8);
      if (vo) *reinterpret_cast<bf16x8*>(vo + (long)t * D + c8) = v;
      if (vo2) *reinterpret_cast<bf16x8*>(vo2 + (long)t * D + c8) = v;
    }
  }
  if (!VARLEN && a.vt_out) {
    // V'^T feeds only the attention's P V product, which runs in fp16 so that P
    // keeps 11 significant bits.  It holds the stored bf16 V' values, converted
    // exactly (within fp16's range), so the forward's O and the backward (which
    // reads the bf16 V') see the same V'.
    // Thread = (4 tokens, 8 channels): four 16-byte row reads, eight 8-byte
    // stores, one per channel row; the 4-token groups of a channel chunk sit
    // in consecutive lanes, so a store instruction writes whole 128-byte runs.
    _Float16* vt = reinterpret_cast<_Float16*>(a.vt_out) + (long)(b * dm.Hkv + g) * D * a.s_pad;
    static_assert((TW / 4) * (D / 8) == 256, "one (4 tokens, 8 channels) item per thread");
    const int m4 = threadIdx.x % (TW / 4), c8 = (threadIdx.x / (TW / 4)) * 8;
    const int t = t0 + 4 * m4;
    if (t < a.s_pad) {
      f16x4 pk[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16x8 v = vchunk(4 * m4 + i, c8);
#pragma unroll
        for (int x = 0; x < 8; ++x)   // tokens at or past S: the zero padding up to s_pad
          pk[x][i] = t + i < S ? (_Float16)(float)v[x] : (_Float16)0.0f;
      }
#pragma unroll
      for (int x = 0; x < 8; ++x)
        *reinterpret_cast<f16x4*>(vt + (long)(c8 + x) * a.s_pad + t) = pk[x];
    }
  }
  // every read of the v~ tile is done: it now stages each output tile (Q'' of
  // a head, then K''), so that the global stores are whole 16-byte row pieces
  __syncthreads();
  char* const so = tv;
  // the staged tile's rows inside the sequence to global rows dst + tr * D
  auto flush = [&](bf16* dst, bf16* dst2) {
    __syncthreads();
    for (int e = threadIdx.x; e < TW * (D / 8); e += 256) {
      const int tr = e / (D / 8), c8 = (e % (D / 8)) * 8;
      if (t0 + tr >= S) break;
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(so + tr * ROWB + c8 * 2);
      if (dst) *reinterpret_cast<bf16x8*>(dst + (long)tr * D + c8) = v;
      if (dst2) *reinterpret_cast<bf16x8*>(dst2 + (long)tr * D + c8) = v;
    }
    __syncthreads();
  };

  Acc2 kacc, qacc, mpost, mpre;
  conv_head<D>(kacc, tk, taps_k, dm.kk, ch, lane, tb0, tf, qtaps(g * G));
  zero(mpost);
  if (!QRES) zero(mpre);
  // The query side's key terms, the same for every head of the group:
  // q' = (1 + b/2) q^ + a/2 q~ + kq with kq = a/2 k~ + b/2 k^ (per token and
  // channel, in the accumulator layout)
  Acc2 kq;
  if constexpr (!NOQ) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int tr = tb0 + 32 * mb + l32;
#pragma unroll
      for (int g4 = 0; g4 < 2; ++g4) {
        const int c0 = 16 * cw + 8 * g4 + 4 * hi;
        const f32x4 kpl = tile_vec4<D>(tk, tr + HALO, c0), kph = tile_vec4<D>(tk, tr + HALO, c0 + D / 2);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int rl = 4 * g4 + e, rh = rl + 8;
          kq[mb][rl] = __builtin_fmaf(A, kpl[e], Bc * kacc[mb][rl]);
          kq[mb][rh] = __builtin_fmaf(A, kph[e], Bc * kacc[mb][rh]);
        }
      }
    }
  }
  const float Bp1 = 1.0f + Bc;

#pragma unroll
  for (int i = 0; i < G; ++i) {
    __builtin_amdgcn_sched_barrier(0);         // heads one after another (registers)
    const int h = g * G + i;
    if (i > 0 && i % NQS == 0) {
      // the next q~ tiles into the slots once every wave is done with them
      __syncthreads();
      char* const dst[NQS] = {tq, tq + TBYTES};
      const int cols[NQS] = {h * D, (h + 1) * D};
      load_tiles<D>(dst, cols, min(NQS, G - i), qkv_b, dm.nqkv, S, t0);
      if (VARLEN && t0 == 0) {
        __syncthreads();
        for (int s2 = 0; s2 < NQS && i + s2 < G; ++s2)
          fill_halo<D>(tq + s2 * TBYTES, st + (h + s2) * D, dm.kq - 1, dm.nq);
      }
      __syncthreads();
    }
    const char* tqi = tq + (i % NQS) * TBYTES;
    conv_head<D>(qacc, tqi, qtaps(h), dm.kq, ch, lane, tb0, tf, i + 1 < G ? qtaps(h + 1) : nullptr);
    if constexpr (NOQ) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int tr = tb0 + 32 * mb + l32;
#pragma unroll
        for (int g4 = 0; g4 < 2; ++g4) {
          const int c0 = 16 * cw + 8 * g4 + 4 * hi;
          f32x4 qpl = {0.f, 0.f, 0.f, 0.f}, qph = {0.f, 0.f, 0.f, 0.f};
          if (!QRES) {
            qpl = tile_vec4<D>(tqi, tr + HALO, c0);
            qph = tile_vec4<D>(tqi, tr + HALO, c0 + D / 2);
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int rl = 4 * g4 + e, rh = rl + 8;
            mpost[mb][rl] += qacc[mb][rl];
            mpost[mb][rh] += qacc[mb][rh];
            if (!QRES) {
              mpre[mb][rl] += qpl[e];
              mpre[mb][rh] += qph[e];
            }
          }
        }
      }
      continue;
    }
    const long qrow = VARLEN ? q_row0 + h * q_hstride + t0 : (long)(b * dm.Hq + h) * S + t0;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      __builtin_amdgcn_sched_barrier(0);       // one token block at a time (registers)
      const int tr = tb0 + 32 * mb + l32;
      // the same rows for every head: an opaque copy of the base keeps the
      // compiler from hoisting these loads out of the head loop (they would
      // hold their registers through every convolution)
      const float2* rp = rope_t0;
      asm volatile("" : "+s"(rp));
#pragma unroll
      for (int g4 = 0; g4 < 2; ++g4) {
        const int c0 = 16 * cw + 8 * g4 + 4 * hi;   // this group's pairs; partners c0 + D / 2
        f32x4 cs, sn;
        load_rope4<D>(cs, sn, rp, tr, c0, S - t0);
        const f32x4 qpl = tile_vec4<D>(tqi, tr + HALO, c0), qph = tile_vec4<D>(tqi, tr + HALO, c0 + D / 2);
        f32x4 ylo, yhi;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int rl = 4 * g4 + e, rh = rl + 8;
          const float qhl = qacc[mb][rl], qhh = qacc[mb][rh];
          mpost[mb][rl] += qhl;
          mpost[mb][rh] += qhh;
          if (!QRES) {
            mpre[mb][rl] += qpl[e];
            mpre[mb][rh] += qph[e];
          }
          const float xl = __builtin_fmaf(Bp1, qhl, __builtin_fmaf(A, qpl[e], kq[mb][rl]));
          const float xh = __builtin_fmaf(Bp1, qhh, __builtin_fmaf(A, qph[e], kq[mb][rh]));
          // RoPE of the pair (low channel, partner)
          ylo[e] = __builtin_fmaf(xl, cs[e], -(xh * sn[e]));
          yhi[e] = __builtin_fmaf(xh, cs[e], xl * sn[e]);
        }
        stage4<D>(so, tr, c0, ylo);
        stage4<D>(so, tr, c0 + D / 2, yhi);
      }
    }
    flush(reinterpret_cast<bf16*>(a.q_out) + qrow * D, nullptr);
  }

  // k' = k^ + a/2 (mean_g q~ + k~) + b/2 (mean_g q^ + k^)
  __builtin_amdgcn_sched_barrier(0);
  const float invG = 1.0f / (float)G;
  bf16* ko = VARLEN ? nullptr
                    : reinterpret_cast<bf16*>(a.k_out) + ((long)(b * dm.Hkv + g) * S + t0) * D;
  bf16* ko2 = a.k_out2 ? reinterpret_cast<bf16*>(a.k_out2) +
                             ((long)(b * dm.Hkv + g) * a.cap2 + pos0 + t0) * D
                       : nullptr;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    __builtin_amdgcn_sched_barrier(0);
    const int tr = tb0 + 32 * mb + l32;
    const float2* rp = rope_t0;
    asm volatile("" : "+s"(rp));
#pragma unroll
    for (int g4 = 0; g4 < 2; ++g4) {
      const int c0 = 16 * cw + 8 * g4 + 4 * hi;
      f32x4 cs, sn;
      load_rope4<D>(cs, sn, rp, tr, c0, S - t0);
      const f32x4 kpl = tile_vec4<D>(tk, tr + HALO, c0), kph = tile_vec4<D>(tk, tr + HALO, c0 + D / 2);
      f32x4 qsl = {0.f, 0.f, 0.f, 0.f}, qsh = {0.f, 0.f, 0.f, 0.f};
      if (QRES) {
        for (int i = 0; i < G; ++i) {
          qsl += tile_vec4<D>(tq + i * TBYTES, tr + HALO, c0);
          qsh += tile_vec4<D>(tq + i * TBYTES, tr + HALO, c0 + D / 2);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          qsl[e] = mpre[mb][4 * g4 + e];
          qsh[e] = mpre[mb][8 + 4 * g4 + e];
        }
      }
      f32x4 ylo, yhi;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int rl = 4 * g4 + e, rh = rl + 8;
        const float khl = kacc[mb][rl], khh = kacc[mb][rh];
        const float xl = __builtin_fmaf(Bc, __builtin_fmaf(mpost[mb][rl], invG, khl),
                                        __builtin_fmaf(A, __builtin_fmaf(qsl[e], invG, kpl[e]), khl));
        const float xh = __builtin_fmaf(Bc, __builtin_fmaf(mpost[mb][rh], invG, khh),
                                        __builtin_fmaf(A, __builtin_fmaf(qsh[e], invG, kph[e]), khh));
        ylo[e] = __builtin_fmaf(xl, cs[e], -(xh * sn[e]));
        yhi[e] = __builtin_fmaf(xh, cs[e], xl * sn[e]);
      }
      stage4<D>(so, tr, c0, ylo);
      stage4<D>(so, tr, c0 + D / 2, yhi);
    }
  }
  flush(ko, ko2);

}

}  // namespace

bool mix_fwd_mfma_supported(const Dims& dm) { return dm.bf16 && (dm.d == 128 || dm.d == 64); }

// Variable-length mix (see mix_body): a.S = T, the packed token count; vm.blk
// counts 64-token tiles; a.state holds each sequence's history before its chunk.
hipError_t launch_mix_varlen_mfma(const MixArgs& a, const VarlenMap& vm, hipStream_t s) {
  if (a.dm.d != 128 || !a.dm.bf16 || a.qkv_f32 || !a.state || !a.k_out2 || !a.v_out2 ||
      a.k_out || a.v_out || vm.B < 1 || vm.B > kMaxVarlenBatch)
    return hipErrorInvalidValue;
  if ((long)a.S * a.dm.nqkv * 2 >= (1L << 31)) return hipErrorInvalidValue;
  const int ntiles = vm.blk[vm.B];
  if (ntiles == 0) return hipSuccess;
  const int ntiles8 = (ntiles + XCDS - 1) / XCDS * XCDS;
  const dim3 grid((unsigned)(ntiles8 * a.dm.Hkv));
  if (a.dm.G == 1)
    hipLaunchKernelGGL((mix_fwd_mfma_kernel<128, 1, true, false, VarlenMap>), grid, dim3(256), 0, s, a,
                       ntiles8, vm);
  else if (a.dm.G == 2)
    hipLaunchKernelGGL((mix_fwd_mfma_kernel<128, 2, true, false, VarlenMap>), grid, dim3(256), 0, s, a,
                       ntiles8, vm);
  else
    hipLaunchKernelGGL((mix_fwd_mfma_kernel<128, 0, true, false, VarlenMap>), grid, dim3(256), 0, s, a,
                       ntiles8, vm);
  return hipGetLastError();
}

template <int D, bool NOQ>
hipError_t launch_mix_fwd_mfma_d(const MixArgs& a, hipStream_t s) {
  const int ntiles = (a.S + MGeom<D>::TW - 1) / MGeom<D>::TW;
  const int ntiles8 = (ntiles + XCDS - 1) / XCDS * XCDS;
  const dim3 grid((unsigned)(ntiles8 * a.dm.Hkv * a.B));
  if (a.dm.G == 1)
    hipLaunchKernelGGL((mix_fwd_mfma_kernel<D, 1, false, NOQ, NoMap>), grid, dim3(256), 0, s, a,
                       ntiles8, NoMap{});
  else if (a.dm.G == 2)
    hipLaunchKernelGGL((mix_fwd_mfma_kernel<D, 2, false, NOQ, NoMap>), grid, dim3(256), 0, s, a,
                       ntiles8, NoMap{});
  else
    hipLaunchKernelGGL((mix_fwd_mfma_kernel<D, 0, false, NOQ, NoMap>), grid, dim3(256), 0, s, a,
                       ntiles8, NoMap{});
  return hipGetLastError();
}

hipError_t launch_mix_fwd_mfma(const MixArgs& a, hipStream_t s) {
  if (a.vt_out && (a.s_pad % 64 != 0 || a.s_pad < a.S)) return hipErrorInvalidValue;
  // 32-bit byte offsets within one sequence's latent rows
  if ((long)a.S * a.dm.nqkv * 2 >= (1L << 31)) return hipErrorInvalidValue;
  // no Q'' output: the fused-Q prefill (d = 128), whose attention forms Q''
  if (!a.q_out) return a.dm.d == 128 ? launch_mix_fwd_mfma_d<128, true>(a, s) : hipErrorInvalidValue;
  if (a.dm.d == 128) return launch_mix_fwd_mfma_d<128, false>(a, s);
  if (a.dm.d == 64) return launch_mix_fwd_mfma_d<64, false>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace cca
