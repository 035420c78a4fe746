// Internal declarations shared by the host sequencing code (api.cpp) and the
// HIP kernels of the CCA / CCGQA layer.  gfx950 (CDNA4) only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cca {

using bf16 = __bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxDecodeBatch = 256;
constexpr int kMaxConv = 4;
constexpr int kMaxGroup = 8;
constexpr uint32_t kQkPre = 1u, kQkPost = 2u, kRope = 4u, kVShift = 8u;

// Per-layer sizes, derived once from the config and passed to kernels by value.
struct Dims {
  int E, Hq, Hkv, d, G, kq, kk, sv;
  int nq, nk, nqkv;         // Hq*d, Hkv*d, (Hq+2*Hkv)*d
  int state_w;              // elements of rolling state per sequence
  int max_seq_len;
  uint32_t flags;
  bool bf16;
};

struct DecodePos {
  int32_t p[kMaxDecodeBatch];
  // split-key decode: sequence b's work-groups per KV head are off[b] ..
  // off[b + 1] - 1 of the flattened grid (sized per sequence from its length)
  int32_t off[kMaxDecodeBatch + 1];
};

// ------------------------------------------------------------------ GEMM
// C(m, n) = sum_k A(m, k) * B(k, n), fp32 accumulation.
//   A(m, k) = a[m*lda + k] when a_kc (K-contiguous) else a[k*lda + m].
//   B(k, n) = b[n*ldb + k] when b_kc else b[k*ldb + n].  B's storage rows
//   (n when b_kc, k otherwise) may be split over up to 3 buffers: storage row
//   r lives in segment s = the last with b_start[s] <= r, at
//   b_ptr[s] + (r - b_start[s]) * ldb.
//   C(m, n) = c_ptr[s][(m - c_start[s]) * ldc + n], segments along m.
struct GemmArgs {
  int M, N, K;
  const void* a;
  long lda;
  const void* b_ptr[3];
  int b_start[3];
  int b_nseg;
  long ldb;
  void* c_ptr[3];
  int c_start[3];
  int c_nseg;
  long ldc;
  // split-K (256 x 256 NT kernel only): ksplit > 1 makes work-group z of the
  // grid's y dimension sum k in [z K/ksplit, (z+1) K/ksplit) into fp32
  // c_ptr[0] + z * c_split_stride (one segment); 0 or 1 = no split
  int ksplit;
  long c_split_stride;
  // K-major operands (256 x 256 kernel, TN layout): rows of A and B at or past
  // k_valid read as zero, so K may be rounded up; 0 = K
  int k_valid;
};

enum class GemmLayout { NT, NN, TN };   // (a_kc, b_kc) = (1,1), (1,0), (0,0)

// in_bf16: A and B are bf16 (else fp32); out_f32: C is fp32 (else same as inputs).
hipError_t launch_gemm(const GemmArgs& g, GemmLayout layout, bool in_bf16, bool out_f32,
                       hipStream_t s);

// The 256 x 256 bf16 NT kernel when the shape suits it (see gemm_nt_mfma.hip);
// false and nothing launched otherwise.
bool launch_gemm_nt_big(const GemmArgs& g, bool out_f32, hipStream_t s, hipError_t* err,
                        GemmLayout layout = GemmLayout::NT);
// Split-K NT GEMM for few rows of A (the decode step): partial tiles in an fp32
// buffer of gemm_skinny_part_floats() floats, then a fixed-order sum; false when
// the shape does not suit it (nothing launched).
// With keep set, the sum is left to the consumer: only the partials are
// written, C(m, n) = sum over z < keep->KS of part[z * keep->kstride + m * keep->ld + n].
struct SkinnyPartials {
  const float* part;
  int KS;
  long kstride;
  int ld;
};
bool launch_gemm_skinny(const GemmArgs& g, bool out_f32, float* part, hipStream_t s,
                        hipError_t* err, SkinnyPartials* keep = nullptr);
size_t gemm_skinny_part_floats();
// out[c][r] = in[r][c] for r < R, c < C (bf16), zero for R <= r < Rp;
// C and Rp multiples of 8, 16-byte aligned rows.
hipError_t launch_transpose_bf16(const void* in, long ld_in, int R, int C, int Rp, void* out,
                                 long ld_out, hipStream_t s);
// Sums split-K partials part[z][m][n] (z < ksplit, fixed order) into fp32
// outputs: row m goes to out[seg] + (m - start[seg]) * ld, segments along m.
hipError_t launch_splitk_reduce(const float* part, int ksplit, int M, int N, float* const out[3],
                                const int start[3], int nseg, long ld, hipStream_t s);

// ------------------------------------------------------------------ mix
// Causal conv + QK-mean + value shift + RoPE over a prefill.
//   qkv [B*S, nqkv] (q~ | k~ | v~), fp32 when qkv_f32 else bf16 (bf16 storage
//   only: the latent of an inference prefill; one that saves for the backward
//   keeps fp32); rope [max_seq_len, d/2] float2 (cos, sin).
//   Outputs (row stride in tokens given by *_ld, batch stride by *_bs elems):
//   q_out [B, Hq, S, d]; k_out, v_out [B, Hkv, ld, d].  k2/v2 optional second
//   destination (the cache) with its own row capacity.
struct MixArgs {
  Dims dm;
  int B, S;
  const void* qkv;
  bool qkv_f32;
  const void* conv_q;
  const void* conv_k;
  const float2* rope;
  void* q_out;
  void* k_out;
  void* v_out;
  void* k_out2;
  void* v_out2;
  int cap2;                 // row capacity of k_out2 / v_out2
  void* vt_out;             // V' transposed [B, Hkv, d, s_pad] (MFMA path), nullable
  int s_pad;                // S rounded up to a multiple of 64; rows [S, s_pad) are zero
  const void* state;        // variable-length chunks: rolling state [B, state_w] before them
};
hipError_t launch_mix_fwd(const MixArgs& a, hipStream_t s);
// True when prefill uses the MFMA mix + attention pair, which exchange V' in
// the transposed layout (and need the standard one only for saved / cache).
bool prefill_uses_mfma(const Dims& dm);

// Writes the rolling state after the last token of each sequence.
hipError_t launch_write_state(const Dims& dm, int B, int S, const void* qkv, bool qkv_f32,
                              void* state, hipStream_t s);

// Decode: one token per sequence; reads/updates state, writes the cache row
// pos[b] and q_out [B, Hq, d].
struct MixDecodeArgs {
  Dims dm;
  int B;
  DecodePos pos;
  const float* qkv;         // [B, nqkv] fp32, or the first of qkv_ks K-slice partials:
  int qkv_ks;               // qkv~(b, col) = sum_z qkv[z * qkv_kstride + b * qkv_ld + col]
  long qkv_kstride;
  int qkv_ld;
  const void* conv_q;
  const void* conv_k;
  const float2* rope;
  void* state;              // [B, state_w], updated in place
  void* k_cache;            // [B, Hkv, max_seq_len, d]
  void* v_cache;
  void* q_out;              // [B, Hq, d]
  float* cv;                // [B, Hq + Hkv, d] fp32 workspace: convolution outputs
};
hipError_t launch_mix_decode(const MixDecodeArgs& a, hipStream_t s);
// The single-kernel decode mix (bf16, d = 128, up to 4 taps) takes qkv~ as
// K-slice partials; the two-kernel path needs qkv_ks == 1.
bool mix_decode_fused_ok(const Dims& dm);
size_t mix_decode_cv_floats(const Dims& dm, int B);

// ------------------------------------------------------------------ variable length
// Per-sequence layout of a chunked, variable-length batched prefill (host
// arrays passed by value): sequence b owns packed token rows tok[b] ..
// tok[b + 1] - 1, which sit at positions start[b] .. of its cache; blk[b] is
// the prefix sum of its work blocks for the kernel the map is built for.
constexpr int kMaxVarlenBatch = 128;
struct VarlenMap {
  int32_t tok[kMaxVarlenBatch + 1];
  int32_t start[kMaxVarlenBatch];
  int32_t blk[kMaxVarlenBatch + 1];
  int32_t B;
};

// Chunked variable-length prefill (bf16, d = 128): the mix (vm.blk over
// 64-token tiles; a.S = T packed tokens, Q'' to [Hq][T][d], K'' / V' to the
// caches at their positions, history from a.state), the state advanced past
// each chunk (from the bf16 latent), the fp16 V'^T of each sequence's cache
// rows 0 .. start + n - 1 ([B][Hkv][d][s_pad], zero past them), and the
// attention over them (vm.blk over 128-query blocks).
hipError_t launch_mix_varlen_mfma(const MixArgs& a, const VarlenMap& vm, hipStream_t s);
hipError_t launch_state_varlen(const Dims& dm, const VarlenMap& vm, const void* lat, void* state,
                               hipStream_t s);
hipError_t launch_vt_varlen(const Dims& dm, const VarlenMap& vm, const void* v_cache, int cap,
                            void* vt, int s_pad, hipStream_t s);

// ------------------------------------------------------------------ attention
// Causal attention.  Query row t of sequence b sits at position
// (decode ? pos[b] : t) and sees keys 0..position.
//   q [B, Hq, Sq, d]; k, v: element (b, g, j, c) at k[b*kv_bs + g*kv_hs + j*d + c];
//   o: token-major [B, Sq, Hq*d]; lse [B, Hq, Sq] fp32 (nullable).
struct AttnArgs {
  Dims dm;
  int B, Sq;
  const void* q;
  const void* k;
  const void* v;
  long kv_bs, kv_hs;
  const void* vt;           // V' transposed [B, Hkv, d, s_pad] (MFMA prefill path)
  int s_pad;
  void* o;
  float* o32;               // optional fp32 copy of o (same layout), nullable
  float* lse;
  bool decode;
  DecodePos pos;
  // split-key partials for decode (fp32 workspace), see launch_attn_decode
  float* part;
  int nsplit;
  // fused-Q prefill (inference, bf16, d = 128): when qlat is set the attention
  // forms Q'' itself from the bf16 latent [B*S, nqkv] (q~ of its head, k~ of
  // its KV head), the taps and the RoPE table, and a.q is not read
  const void* qlat;
  const void* conv_q;
  const void* conv_k;
  const float2* rope;
  // key-split prefill (fixed length, Q'' as stored): ksplit > 1 work-groups per
  // query block, their partials in `part` (attn_split_part_bytes), merged by a
  // second kernel; 0 or 1: one work-group per query block
  int ksplit;
};
constexpr int kMaxAttnSplit = 8;
// fp32 bytes of the key-split partials: (O, m, l) per query, head and part
size_t attn_split_part_bytes(const Dims& dm, int B, int S, int P);
hipError_t launch_attn_fwd(const AttnArgs& a, hipStream_t s);
hipError_t launch_attn_varlen_mfma(const AttnArgs& a, const VarlenMap& vm, hipStream_t s);
hipError_t launch_attn_decode(const AttnArgs& a, hipStream_t s);
// Split-key work-groups per KV head for each sequence (into pos.off, from
// pos.p); returns their total.  The fast path only.
int decode_splits(const Dims& dm, int B, DecodePos& pos);
size_t decode_part_floats(const Dims& dm, int B);

// ------------------------------------------------------------------ backward
struct AttnBwdArgs {
  Dims dm;
  int B, S;
  const void* q;     // Q'' [B,Hq,S,d]
  const void* k;     // K'' [B,Hkv,S,d]
  const void* v;     // V'  [B,Hkv,S,d]
  const float* o32;  // O   [B,S,Hq*d] fp32 (saved by the forward)
  const void* dO;    // dO  [B,S,Hq*d]
  const float* lse;  // [B,Hq,S]
  float* Dsum;       // [B,Hq,S] workspace
  float* dq;         // dQ'' [B,Hq,S,d] fp32
  float* dk;         // dK'' [B,Hkv,S,d] fp32
  float* dv;         // dV'  [B,Hkv,S,d] fp32
  // MFMA path workspace (bf16 storage, d = 128): fp16 copies as head-major
  // rows, s_pad rows per head (zero from row S)
  void* q16;         // Q'' [B,Hq,s_pad,d] fp16
  void* k16;         // K'' [B,Hkv,s_pad,d]
  void* v16;         // V'  [B,Hkv,s_pad,d]
  void* do16;        // dO  [B,Hq,s_pad,d]
  int s_pad;         // S rounded up to a multiple of 64
  // dK / dV partials of the other work-groups of each key block (fp32, same
  // layout as dk / dv; dk3 .. dv4 only with four parts, see attn_bwd_parts),
  // added into dk / dv before the kernels return, unless the consumer adds
  // dk2 / dv2 as it reads dk / dv (sum_by_consumer, two parts only)
  float* dk2;
  float* dv2;
  float* dk3;
  float* dv3;
  float* dk4;
  float* dv4;
  bool sum_by_consumer;
  // MFMA path: dO enters its fp16 copy multiplied by 2^e, chosen from max|dO|
  // so the copy and dS stay inside fp16's normal range whatever the size of the
  // upstream gradient; every product is linear in dO, so the fp32 results are
  // multiplied by 2^-e on the way out (both scalings exact).  amax_part holds
  // the per-work-group maxima of an absmax pass (kAmaxParts floats); dscale[0]
  // receives 2^-e.
  float* amax_part;
  float* dscale;
};
constexpr int kAmaxParts = 256;
hipError_t launch_attn_bwd(const AttnBwdArgs& a, hipStream_t s);
// True when launch_attn_bwd takes the MFMA kernels (bf16, d = 128), which
// produce the dk2 / dv2 second-half partials.
bool attn_bwd_mfma_supported(const Dims& dm);
// Work-groups per key block of the MFMA dK / dV kernel: 4 when the group size
// is a multiple of 4 (each takes a quarter of the group's heads), else 2.
int attn_bwd_parts(const Dims& dm);
// Bytes of the MFMA attention backward's workspace: the fp16 copies and
// the second-half dK / dV partials (0 when the config takes the generic path).
size_t attn_bwd_transpose_bytes(const Dims& dm, int B, int S);

struct MixBwdArgs {
  Dims dm;
  int B, S;
  const float* qkv;      // saved q~ | k~ | v~ [B*S, nqkv] fp32
  const void* conv_q;
  const void* conv_k;
  const float2* rope;
  const float* dq;       // dQ'' [B,Hq,S,d] fp32
  const float* dk;       // dK'' fp32
  const float* dv;       // dV'  fp32
  void* dqkv;            // out: dq~ | dk~ | dv~ [B*S, nqkv]
  float* dconv_part;     // [nblk, Hq*kq*d*d + Hkv*kk*d*d] partial tap grads
  float* dconv_q;        // final fp32 [Hq,kq,d,d]
  float* dconv_k;        // final fp32 [Hkv,kk,d,d]
  float* scratch;        // fp32 workspace for dq^ / dk^ [B*S, nq + nk]
  void* tapT;            // bf16, d = 128: workspace for the transposed taps (mix_bwd_tapT_bytes)
  // nullable: second-half partials the attention backward left for the
  // consumer, added to dk / dv as they are read (only when mix_bwd_adds_dkdv2)
  const float* dk2;
  const float* dv2;
};
hipError_t launch_mix_bwd(const MixBwdArgs& a, hipStream_t s);
size_t mix_bwd_tapT_bytes(const Dims& dm);
bool mix_bwd_adds_dkdv2(const Dims& dm);
size_t mix_bwd_part_floats(const Dims& dm, int B, int S);
size_t mix_bwd_scratch_floats(const Dims& dm, int B, int S);

// ------------------------------------------------------------------ utilities
// Fills `bytes` (a multiple of 16, 16-byte aligned) at p with the 32-bit v.
hipError_t launch_fill(void* p, size_t bytes, uint32_t v, hipStream_t s);

}  // namespace cca
