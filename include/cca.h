/*
 * cca.h — C ABI of the MI355X (gfx950) Compressed Convolutional Attention
 * library: one CCA / CCGQA attention layer, forward prefill, single-token
 * decode and backward.
 *
 * Sources (page titles; sections as named on each page):
 *   CCA-es   "Compressed Convolutional Attention: Efficient Attention in a
 *            Compressed Latent Space", gist.science summary, Spanish.
 *   CCA-fr   the same title, gist.science summary, French (technical part).
 *
 * What the layer computes (CCA-es §2.A-§2.C, §3 item 2; CCA-fr §2):
 *   q~ = x W_q^T, k~ = x W_k^T, v~ = x W_v^T        latent of size E/C per token
 *   q^ = causal grouped conv of q~ along the sequence (k taps of d x d per head),
 *        k^ likewise with its own taps
 *   q' = q^ + a(q~ + k~_g)/2 + b(q^ + k^_g)/2       QK-mean before/after the conv
 *   k' = k^ + a(mean_g q~ + k~)/2 + b(mean_g q^ + k^)/2
 *   v' = v~ with the masked channels of each KV head taken from token t-1
 *   Q'', K'' = RoPE(q', k') at the token's position (rotate-half, full head dim)
 *   O = causal softmax(Q'' K''^T / sqrt(d)) V'   with query head h reading KV head h / G
 *   y = O W_o^T
 * d = E / (C * n_q_heads) is the latent head dim, G = n_q_heads / n_kv_heads.
 *
 * Conventions for every entry point below:
 *   - Tensor arguments are DEVICE pointers into caller-owned memory,
 *     contiguous row-major, 16-byte aligned, with the shapes stated.  The
 *     element type is cca_config.dtype ("dt": fp32 or bf16) unless a shape says
 *     fp32.  The library never allocates, frees or synchronises after
 *     cca_create; every call enqueues kernels on `stream` (a hipStream_t; NULL =
 *     the null stream) and returns.
 *   - Weights (cca_weights): w_q [Hq*d, E], w_k [Hkv*d, E], w_v [Hkv*d, E],
 *     w_o [E, Hq*d] (all [out, in]); conv_q [Hq, kq, d, d], conv_k [Hkv, kk, d, d]
 *     where [h, j, c_out, c_in] is tap j (it multiplies the token at lag j).
 *   - Errors: a non-CCA_OK status means nothing was launched, except
 *     CCA_ERR_HIP, which reports a launch error (hipGetLastError) after some
 *     kernels may already have been enqueued.  Device faults surface at the
 *     caller's next synchronisation.  No C++ exception crosses this ABI.
 *   - Threading: a handle is read-only after cca_create, so concurrent calls
 *     on one handle with distinct workspaces are safe — except while kernel
 *     timing (cca_profile_*) is enabled, which records into the handle.
 */
#ifndef CCA_H
#define CCA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CCA_OK = 0,
  CCA_ERR_INVALID_CONFIG = 1,  /* cca_config fails validation */
  CCA_ERR_INVALID_ARG = 2,     /* null pointer, misaligned pointer, bad size */
  CCA_ERR_UNSUPPORTED = 3,     /* valid config this build has no kernel for */
  CCA_ERR_CAPACITY = 4,        /* a position or length exceeds max_seq_len */
  CCA_ERR_HIP = 5,             /* HIP runtime error */
  CCA_ERR_OOM = 6,             /* cca_create could not allocate its table */
  CCA_ERR_SCRATCH = 7          /* the call needs more than the static scratch area */
} cca_status;

typedef enum { CCA_F32 = 0, CCA_BF16 = 1 } cca_dtype;   /* accumulation is fp32 */

/* Switches for the three extra operations and RoPE (CCA-es §2.B, §3 item 2). */
enum {
  CCA_QKMEAN_PRE = 1u,    /* add the pre-convolution mean (q~ + k~)/2 */
  CCA_QKMEAN_POST = 2u,   /* add the post-convolution mean (q^ + k^)/2 */
  CCA_ROPE = 4u,          /* rotate Q and K by their positions */
  CCA_VSHIFT = 8u,        /* value shift of the last v_shift_channels of each KV head */
  CCA_DEFAULT_FLAGS = 15u
};

/* Operation selector for cca_workspace_bytes. */
enum { CCA_OP_PREFILL = 0, CCA_OP_DECODE = 1, CCA_OP_BACKWARD = 2 };

/* The problem statement: hidden size E, compression C, query heads, KV heads,
 * the sequence bound and the conv kernel sizes (CCA-es §2.A, §2.B.1, §2.C). */
typedef struct {
  uint32_t struct_size;      /* = sizeof(cca_config) */
  int32_t E;                 /* hidden size */
  int32_t C;                 /* compression factor: query latent = E / C */
  int32_t n_q_heads;         /* Hq; d = E / (C * Hq) */
  int32_t n_kv_heads;        /* Hkv; Hq % Hkv == 0 */
  int32_t max_seq_len;       /* bound on prefill S and on decode positions (cache capacity) */
  int32_t conv_kernel_q;     /* kq >= 1 sequence taps for Q */
  int32_t conv_kernel_k;     /* kk >= 1 sequence taps for K */
  int32_t v_shift_channels;  /* s_v: the LAST s_v channels of each KV head shift; 0 <= s_v <= d */
  uint32_t flags;            /* CCA_* switches */
  double rope_base;          /* > 1, e.g. 10000 */
  int32_t dtype;             /* cca_dtype of x, weights, taps, caches, state, y, dx */
} cca_config;

typedef struct {
  const void *w_q, *w_k, *w_v, *w_o, *conv_q, *conv_k;
} cca_weights;

/* Backward outputs, all overwritten (not accumulated).  dx [B, S, E] in dt;
 * dw_* and dconv_* are fp32 with the shapes of the matching weights. */
typedef struct {
  void *dx, *dw_q, *dw_k, *dw_v, *dw_o, *dconv_q, *dconv_k;
} cca_grads;

typedef struct cca_handle cca_handle;

/* Host-only check of a config (no GPU needed).  Writes a reason into msg
 * (NUL-terminated, at most msg_len bytes) when msg is not NULL.  Returns
 * CCA_OK, CCA_ERR_INVALID_CONFIG (inconsistent sizes) or CCA_ERR_UNSUPPORTED
 * (consistent, but no kernel here: bf16 needs d = 64 or 128; fp32 needs even
 * d <= 128; kq, kk <= 4; G <= 8). */
cca_status cca_validate_config(const cca_config* cfg, char* msg, size_t msg_len);

/* Validates cfg and builds a handle on the current HIP device.  The handle owns
 * one device table: cos/sin of the RoPE angles, computed in float64 on the
 * host and stored as fp32, max_seq_len * d/2 * 8 bytes.  *out is set to NULL
 * on failure. */
cca_status cca_create(const cca_config* cfg, cca_handle** out);

/* Frees the handle and its table.  NULL-safe. */
void cca_destroy(cca_handle* h);

/* Bytes of scratch the caller passes as `workspace` to the named operation
 * (CCA_OP_*) with batch B and length S (S is ignored for decode).  0 on a bad
 * argument.  For CCA_OP_PREFILL it is the saved-buffer size plus, when the
 * prefill's attention grid would hold fewer than 512 work-groups of 128
 * queries over more than 8 query blocks (short sequences, bf16 with d = 128
 * or 64), the fp32 partials of its two-way key split. */
size_t cca_workspace_bytes(const cca_handle* h, int op, int32_t B, int32_t S);

/* Bytes of the `saved` buffer a prefill fills for cca_backward.  Its layout,
 * each region 256-byte aligned, in this order:
 *   qkv_lat [B*S, (Hq+2*Hkv)*d] fp32  (q~ | k~ | v~ per token)
 *   q_rope  [B, Hq, S, d]       dt    (Q'')
 *   k_rope  [B, Hkv, S, d]      dt    (K'')
 *   v_shift [B, Hkv, S, d]      dt    (V')
 *   o       [B, S, Hq*d]        dt    (attention output before W_o)
 *   lse     [B, Hq, S]          fp32  (natural log of each softmax denominator)
 *   o_f32   [B, S, Hq*d]        fp32  (the same output before rounding to dt)
 *   v_t     [B, Hkv, d, S64]    fp16  (V' transposed, S64 = S rounded up to 64;
 *                                      written only on the bf16 d = 128 path,
 *                                      holding the bf16 V' values exactly)
 * The backward forms rowsum(dO * O) from o_f32, and the softmax gradient
 * amplifies any error in it (O rounded to bf16 would cost ~3% in dQ and dK;
 * the forward therefore multiplies P, rounded to fp16, by this fp16 V'^T).
 * cca_saved_offsets writes the 8 byte offsets into offsets[0..7]. */
size_t cca_saved_bytes(const cca_handle* h, int32_t B, int32_t S);
cca_status cca_saved_offsets(const cca_handle* h, int32_t B, int32_t S, size_t offsets[8]);

/* Bytes of rolling decode state per batch: B * W elements of dt where
 * W = (kq-1)*Hq*d + (kk-1)*Hkv*d + Hkv*d holds, per sequence,
 * [q~ at lags 1..kq-1 | k~ at lags 1..kk-1 | v~ at lag 1], most recent lag
 * first.  A new sequence starts from all zeros (zero history before token 0). */
size_t cca_state_bytes(const cca_handle* h, int32_t B);

/* Forward prefill of B sequences of S tokens (CCA-es §2.A-§2.C).
 *   x [B, S, E] dt -> y [B, S, E] dt.
 *   saved (nullable): filled as described at cca_saved_bytes, for cca_backward.
 *   k_cache, v_cache (nullable, both or neither): [B, Hkv, max_seq_len, d] dt;
 *     rows 0..S-1 receive K'' and V' of every token (the compressed latent
 *     cache, CCA-es §2.C).
 *   state (nullable): [B, W] dt, receives the rolling decode state after token S-1.
 *   workspace: cca_workspace_bytes(h, CCA_OP_PREFILL, B, S) bytes (used only
 *     when saved is NULL; the saved buffer serves as the workspace otherwise).
 * Precision: with bf16 storage, a prefill that saves for the backward keeps
 * the latent q~|k~|v~ in fp32 (the softmax gradient amplifies its rounding
 * into dQ and dK); without saved (inference) the latent is rounded to bf16.
 * Both stay within the bf16 parity bound on y, the cache and the state.
 * Requires 1 <= S <= max_seq_len and B >= 1 (else CCA_ERR_CAPACITY /
 * CCA_ERR_INVALID_ARG). */
cca_status cca_forward_prefill(cca_handle* h, const cca_weights* w, const void* x, int32_t B,
                               int32_t S, void* y, void* saved, void* k_cache, void* v_cache,
                               void* state, void* workspace, void* stream);

/* One decode step: one new token per sequence (CCA-es §1 item 2 on the cache;
 * CCA-fr §4 "Décodage").
 *   x_new [B, E] dt; pos_host: HOST array of B int32, pos_host[b] = tokens
 *     already cached for sequence b (the new token's position).
 *   k_cache, v_cache [B, Hkv, max_seq_len, d] dt: row pos_host[b] is written
 *     with the new token's K'' and V', then attention reads rows 0..pos_host[b].
 *   state [B, W] dt: read, then advanced by one token in place.
 *   y_new [B, E] dt.  workspace: cca_workspace_bytes(h, CCA_OP_DECODE, B, 0).
 * Returns CCA_ERR_CAPACITY if any pos_host[b] >= max_seq_len or < 0, and
 * CCA_ERR_UNSUPPORTED if B > 256; nothing is launched then. */
cca_status cca_decode_step(cca_handle* h, const cca_weights* w, const void* x_new,
                           const int32_t* pos_host, int32_t B, void* k_cache, void* v_cache,
                           void* state, void* y_new, void* workspace, void* stream);

/* cca_decode_step without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, outputs and errors as
 * cca_decode_step; its workspace is a static device array of 16 MiB per GPU
 * (allocated with the library's code object, held until the process ends),
 * whose address cca_create resolves once per device.  The call allocates and
 * frees nothing and records no timing events.  Returns CCA_ERR_SCRATCH when
 * cca_workspace_bytes(h, CCA_OP_DECODE, B, 0) exceeds 16 MiB (the 32-sequence
 * CCGQA step at E = 2048 needs ~1.5 MiB) and CCA_ERR_INVALID_ARG when the
 * current device is not the handle's.  Every call on one GPU shares that
 * GPU's array: calls that may overlap on one GPU (other streams, other
 * threads, other handles) race and must be serialised by the caller.  The
 * array keeps the last call's contents; no part of it needs to start at zero. */
cca_status cca_decode_step_noalloc(cca_handle* h, const cca_weights* w, const void* x_new,
                                   const int32_t* pos_host, int32_t B, void* k_cache,
                                   void* v_cache, void* state, void* y_new, void* stream);

/* Chunked, variable-length batched prefill: the serving handoff that fills the
 * compressed latent cache (CCA-es §2.C and §1 item 2; CCA-fr §4 "Décodage").
 * Sequence b (b < B <= 128) contributes n_b = offsets_host[b + 1] -
 * offsets_host[b] >= 0 new tokens, packed rows offsets_host[b] .. of x and y,
 * at positions s_b .. s_b + n_b - 1 where s_b = start_host[b] (start_host
 * NULL: all 0) is the number of tokens already in its cache.  The result is
 * the same as n_b decode steps of sequence b: the convolution and value-shift
 * history before its first new token comes from state, each new token
 * attends over cache rows 0 .. its position, rows s_b .. s_b + n_b - 1 of
 * k_cache and v_cache receive the new K'' and V', and state is advanced past
 * the chunk.  For a new sequence pass s_b = 0 and a zeroed state row.
 *   x, y [T, E] dt with T = offsets_host[B]; offsets_host: HOST array of B + 1
 *     int32, offsets_host[0] = 0, nondecreasing; start_host: HOST array of B
 *     int32 or NULL.
 *   k_cache, v_cache [B, Hkv, max_seq_len, d] dt; state [B, W] dt (read and
 *     advanced in place); workspace: cca_varlen_workspace_bytes(h, offsets_host,
 *     start_host, B) bytes.
 * bf16 storage with d = 128 only (else CCA_ERR_UNSUPPORTED).  Returns
 * CCA_ERR_CAPACITY if some s_b + n_b > max_seq_len, CCA_ERR_INVALID_ARG for a
 * negative length or start, CCA_ERR_UNSUPPORTED for B > 128; nothing is
 * launched then.  T = 0 launches nothing.  Inference only (nothing is saved
 * for a backward; the latent is rounded to bf16). */
cca_status cca_forward_prefill_varlen(cca_handle* h, const cca_weights* w, const void* x,
                                      const int32_t* offsets_host, const int32_t* start_host,
                                      int32_t B, void* y, void* k_cache, void* v_cache,
                                      void* state, void* workspace, void* stream);
/* Workspace bytes of cca_forward_prefill_varlen for these host arrays; 0 on
 * an invalid argument. */
size_t cca_varlen_workspace_bytes(const cca_handle* h, const int32_t* offsets_host,
                                  const int32_t* start_host, int32_t B);

/* Backward of cca_forward_prefill for L = <dy, y> (CCA-es §4, training
 * backward): x, dy [B, S, E] dt; saved: what the prefill of the same x wrote.
 * Fills every pointer of g (all required).  Attention probabilities are
 * recomputed from saved Q'', K'' and lse, never stored.  Weight and tap
 * gradients are reduced in a fixed order (run-to-run deterministic).
 * workspace: cca_workspace_bytes(h, CCA_OP_BACKWARD, B, S). */
cca_status cca_backward(cca_handle* h, const cca_weights* w, const void* x, const void* dy,
                        const void* saved, int32_t B, int32_t S, const cca_grads* g,
                        void* workspace, void* stream);

/* Kernel timing with HIP events recorded on the caller's stream around every
 * launch.  enable != 0 starts recording (and clears earlier records);
 * cca_profile_read synchronises on the recorded events, then writes up to
 * `max` entries (kernel name, launches, total milliseconds) and returns the
 * number of distinct kernels.  Not thread-safe while enabled. */
typedef struct {
  char name[48];
  int32_t launches;
  double total_ms;
} cca_kernel_time;
cca_status cca_profile_enable(cca_handle* h, int enable);
int cca_profile_read(cca_handle* h, cca_kernel_time* out, int max);
/* Cold-cache timing: while timing is enabled and buf is not NULL, every timed
 * launch is preceded (outside its events) by a write of `bytes` over the
 * caller's device buffer buf (16-byte aligned, bytes a multiple of 16), which
 * evicts L2 and the 256 MB MALL when bytes exceeds them, so the launch reads
 * its inputs from HBM.  buf = NULL turns it off.  The buffer's contents are
 * overwritten. */
cca_status cca_profile_flush(cca_handle* h, void* buf, size_t bytes);

/* Prefill variant with the query side of the mix fused into the attention
 * (CCA-es §3 item 4, "Implementación Eficiente", and CCA-fr §3 "Implémentation
 * Efficace": the authors' kernel fuses the convolutions with the attention).
 * When on, an inference prefill (saved == NULL) of bf16 storage with d = 128
 * has its attention form Q'' from the latent itself: the mix then writes only
 * K'', V' and the cache, and Q'' never reaches HBM.  Results equal the
 * separate passes up to the rounding of Q'' to bf16.  Other calls ignore the
 * switch.  Off by default; on = 0 turns it off.  CCA_ERR_INVALID_ARG for a
 * NULL handle. */
cca_status cca_set_prefill_fusion(cca_handle* h, int32_t on);

/* Static text for a status code. */
const char* cca_status_string(cca_status s);

/* Build identification: the hex SHA-256 of the sources this library was
 * compiled from (static text; "unknown" when built without it).  The binding
 * compares it with the sources beside the library and refuses a stale build. */
const char* cca_source_hash(void);

#ifdef __cplusplus
}
#endif

#endif /* CCA_H */
