// Host side of the C ABI declared in include/cca.h: config validation, size
// queries, the RoPE table, launch sequencing and the event-based kernel timer.
// No kernel arithmetic lives here.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "../../include/cca.h"
#include "cca_internal.h"

using namespace cca;

struct ProfRec {
  const char* name;
  hipEvent_t start, stop;
};

struct cca_handle {
  cca_config cfg;
  Dims dm;
  float2* rope = nullptr;     // [max_seq_len][d/2] (cos, sin)
  int device = 0;
  void* scratch = nullptr;    // this device's copy of `scratch` (below), or null
  bool profiling = false;
  bool fuse_q = false;        // cca_set_prefill_fusion
  void* flush_buf = nullptr;  // written before each timed launch when set
  size_t flush_bytes = 0;
  std::vector<ProfRec> recs;
  std::vector<hipEvent_t> pool;
};

// Workspace of cca_decode_step_noalloc: a file-scope device array, one copy
// per GPU, held until the process ends.  Host code never passes `scratch`
// itself to a kernel (on the host it names a stand-in, not device memory):
// cca_create resolves each device's address once with hipGetSymbolAddress
// and every use goes through that pointer.
constexpr size_t kScratchBytes = size_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];          // resolved address per device
bool g_scratch_done[kMaxDevices];

// The current device's scratch address (resolved on first use per device),
// or null if the lookup failed.
void* device_scratch(int device) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_done[device]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) {
      (void)hipGetLastError();
      ptr = nullptr;
    }
    g_scratch_ptr[device] = ptr;
    g_scratch_done[device] = true;
  }
  return g_scratch_ptr[device];
}

void put_msg(char* msg, size_t len, const char* fmt, ...) {
  if (!msg || len == 0) return;
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(msg, len, fmt, ap);
  va_end(ap);
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t esize(const Dims& dm) { return dm.bf16 ? 2 : 4; }

Dims make_dims(const cca_config& c) {
  Dims dm{};
  dm.E = c.E;
  dm.Hq = c.n_q_heads;
  dm.Hkv = c.n_kv_heads;
  dm.d = c.E / (c.C * c.n_q_heads);
  dm.G = dm.Hq / dm.Hkv;
  dm.kq = c.conv_kernel_q;
  dm.kk = c.conv_kernel_k;
  dm.sv = c.v_shift_channels;
  dm.nq = dm.Hq * dm.d;
  dm.nk = dm.Hkv * dm.d;
  dm.nqkv = dm.nq + 2 * dm.nk;
  dm.state_w = (dm.kq - 1) * dm.nq + (dm.kk - 1) * dm.nk + dm.nk;
  dm.max_seq_len = c.max_seq_len;
  dm.flags = c.flags;
  dm.bf16 = c.dtype == CCA_BF16;
  return dm;
}

// Saved-buffer regions (see cca_saved_bytes).
constexpr int kSavedRegions = 8;
long pad64(long S) { return (S + 63) / 64 * 64; }
struct SavedLayout {
  size_t off[kSavedRegions];
  size_t total;
};

SavedLayout saved_layout(const Dims& dm, long B, long S) {
  const size_t es = esize(dm);
  const size_t sz[kSavedRegions] = {
      (size_t)(B * S * dm.nqkv) * 4,                                // q~|k~|v~ fp32
      (size_t)(B * S * dm.nq) * es, (size_t)(B * S * dm.nk) * es,   // Q'', K''
      (size_t)(B * S * dm.nk) * es, (size_t)(B * S * dm.nq) * es,   // V', O
      (size_t)(B * dm.Hq * S) * 4,                                  // lse
      (size_t)(B * S * dm.nq) * 4,                                  // O fp32
      (size_t)(B * pad64(S) * dm.nk) * es};                         // V' transposed
  SavedLayout L{};
  size_t o = 0;
  for (int i = 0; i < kSavedRegions; ++i) {
    L.off[i] = o;
    o = align256(o + sz[i]);
  }
  L.total = o;
  return L;
}

// Key-split parts per query block of an inference prefill's attention: with
// fewer than two work-groups per CU (512 on the 256-CU MI355X, one 8-wave
// work-group per CU at a time) the grid would leave CUs idle and the longest
// query block alone would set the kernel's length; its key tiles are then
// split over two work-groups (merged by a second kernel).  More parts measured
// slower (CCA prefill at S = 4096, 128 blocks: attention 55.6 us unsplit,
// 43.3 us with 2 parts, 44.6 / 56.4 / 67.1 us with 4 / 6 / 8): each part pays
// its own Q load, pipeline fill and fp32 partials.
// Sequences of at most 8 blocks (16 key tiles or fewer per block) stay
// unsplit: their chains are short and the partials and merge would cost more.
// Splitting in proportion to the block's length (ceil((qb + 1) / c) parts)
// measured slower still: 54.5 us with c = 8, 61.9 with c = 4.
constexpr int kAttnTargetWGs = 512;
constexpr int kAttnMinSplitBlocks = 9;
int prefill_ksplit(const Dims& dm, long B, long S) {
  if (!prefill_uses_mfma(dm)) return 1;
  const long nqb = (S + 127) / 128;
  return nqb * dm.Hq * B < kAttnTargetWGs && nqb >= kAttnMinSplitBlocks ? 2 : 1;
}

struct DecodeLayout {
  size_t qkv, q, o, part, cv, gpart, total;
};

DecodeLayout decode_layout(const Dims& dm, long B) {
  const size_t es = esize(dm);
  DecodeLayout L{};
  size_t o = 0;
  L.qkv = o; o = align256(o + B * dm.nqkv * 4);
  L.q = o;   o = align256(o + B * dm.nq * es);
  L.o = o;   o = align256(o + B * dm.nq * es);
  L.part = o; o = align256(o + decode_part_floats(dm, (int)B) * 4);
  L.cv = o;   o = align256(o + mix_decode_cv_floats(dm, (int)B) * 4);
  L.gpart = o; o = align256(o + (dm.bf16 ? gemm_skinny_part_floats() * 4 : 0));
  L.total = o;
  return L;
}

struct BwdLayout {
  size_t dO, Dsum, dq, dk, dv, dqkv, part, scratch, trans, tapT, amax;
  size_t wT, tA, tB, gpart;   // bf16 backward GEMMs: transposed operands, split-K partials
  size_t total;
};

constexpr int kMaxSplit = 16;

// bf16 backward GEMMs run on the NT kernels with transposed operands.
bool bwd_gemm_nt(const Dims& dm) { return dm.bf16 && dm.E % 64 == 0 && dm.nqkv % 64 == 0; }

BwdLayout bwd_layout(const Dims& dm, long B, long S) {
  const size_t es = esize(dm);
  BwdLayout L{};
  size_t o = 0;
  L.dO = o;      o = align256(o + (size_t)(B * S * dm.nq) * es);
  L.Dsum = o;    o = align256(o + (size_t)(B * dm.Hq * S) * 4);
  L.dq = o;      o = align256(o + (size_t)(B * S * dm.nq) * 4);
  L.dk = o;      o = align256(o + (size_t)(B * S * dm.nk) * 4);
  L.dv = o;      o = align256(o + (size_t)(B * S * dm.nk) * 4);
  L.dqkv = o;    o = align256(o + (size_t)(B * S * dm.nqkv) * es);
  L.part = o;    o = align256(o + mix_bwd_part_floats(dm, (int)B, (int)S) * 4);
  L.scratch = o; o = align256(o + mix_bwd_scratch_floats(dm, (int)B, (int)S) * 4);
  L.trans = o;   o = align256(o + attn_bwd_transpose_bytes(dm, (int)B, (int)S));
  L.tapT = o;    o = align256(o + mix_bwd_tapT_bytes(dm));
  L.amax = o;    o = align256(o + (kAmaxParts + 1) * 4);   // dO absmax partials, then 2^-e
  L.wT = L.tA = L.tB = L.gpart = o;
  if (bwd_gemm_nt(dm)) {
    const size_t Mp = (size_t)pad64(B * S);
    const size_t wmax = std::max((size_t)dm.nq * dm.E, (size_t)dm.E * dm.nqkv);
    L.wT = o;    o = align256(o + wmax * 2);
    L.tA = o;    o = align256(o + (size_t)dm.E * Mp * 2);
    L.tB = o;    o = align256(o + (size_t)std::max(dm.nq, dm.nqkv) * Mp * 2);
    L.gpart = o; o = align256(o + (size_t)kMaxSplit * wmax * 4);
  }
  L.total = o;
  return L;
}

// Runs one launch, bracketed by timing events when profiling is on (never for
// the allocation-free entry point, whose `h` is null here: event creation may
// allocate).
template <typename F>
hipError_t timed(cca_handle* h, const char* name, hipStream_t s, F&& launch) {
  if (!h || !h->profiling) return launch();
  ProfRec r{name, nullptr, nullptr};
  for (hipEvent_t* e : {&r.start, &r.stop}) {
    if (!h->pool.empty()) {
      *e = h->pool.back();
      h->pool.pop_back();
    } else if (hipEventCreate(e) != hipSuccess) {
      return hipErrorOutOfMemory;
    }
  }
  if (h->flush_buf) {
    // evict the caches so the launch reads its inputs from HBM
    const hipError_t e = launch_fill(h->flush_buf, h->flush_bytes, 0u, s);
    if (e != hipSuccess) return e;
  }
  hipEventRecord(r.start, s);
  hipError_t err = launch();
  hipEventRecord(r.stop, s);
  h->recs.push_back(r);
  return err;
}

GemmArgs gemm_nt(int M, int N, int K, const void* a, long lda, const void* b, long ldb, void* c,
                 long ldc) {
  GemmArgs g{};
  g.M = M; g.N = N; g.K = K;
  g.a = a; g.lda = lda;
  g.b_ptr[0] = b; g.b_start[0] = 0; g.b_nseg = 1; g.ldb = ldb;
  g.c_ptr[0] = c; g.c_start[0] = 0; g.c_nseg = 1; g.ldc = ldc;
  return g;
}

// Down-projection: C[M, nqkv] = A[M, E] * [W_q; W_k; W_v]^T
GemmArgs gemm_down(const Dims& dm, int M, const void* a, const cca_weights* w, void* c) {
  GemmArgs g = gemm_nt(M, dm.nqkv, dm.E, a, dm.E, w->w_q, dm.E, c, dm.nqkv);
  g.b_ptr[1] = w->w_k; g.b_start[1] = dm.nq;
  g.b_ptr[2] = w->w_v; g.b_start[2] = dm.nq + dm.nk;
  g.b_nseg = 3;
  return g;
}

// Variable-length prefill: per-sequence maps for the mix (64-token tiles)
// and the attention (128-query blocks), and the workspace regions.
// the variable-length attention kernel takes both by value (4 KB of kernel arguments at most)
static_assert(sizeof(AttnArgs) + sizeof(VarlenMap) <= 4096, "kernel arguments exceed 4 KB");

struct VarlenPlan {
  VarlenMap mix, attn;
  int T, s_pad;
  size_t lat, q, vt, o, total;
};

cca_status varlen_plan(const cca_handle* h, const int32_t* off, const int32_t* start, int32_t B,
                       VarlenPlan* P) {
  if (!h || !off || B < 1) return CCA_ERR_INVALID_ARG;
  if (B > kMaxVarlenBatch) return CCA_ERR_UNSUPPORTED;
  if (off[0] != 0) return CCA_ERR_INVALID_ARG;
  const Dims& dm = h->dm;
  std::memset(P, 0, sizeof(*P));
  P->mix.B = P->attn.B = B;
  int lmax = 0;
  for (int b = 0; b < B; ++b) {
    const long n = (long)off[b + 1] - off[b];
    const long st = start ? start[b] : 0;
    if (n < 0 || st < 0) return CCA_ERR_INVALID_ARG;
    if (st + n > dm.max_seq_len) return CCA_ERR_CAPACITY;
    P->mix.tok[b] = P->attn.tok[b] = off[b];
    P->mix.start[b] = P->attn.start[b] = (int32_t)st;
    P->mix.blk[b + 1] = P->mix.blk[b] + (int32_t)((n + 63) / 64);
    P->attn.blk[b + 1] = P->attn.blk[b] + (int32_t)((n + 127) / 128);
    lmax = std::max(lmax, (int)(st + n));
  }
  P->mix.tok[B] = P->attn.tok[B] = off[B];
  P->T = off[B];
  P->s_pad = (int)pad64(lmax);
  const size_t T = (size_t)P->T;
  size_t o = 0;
  P->lat = o; o = align256(o + T * dm.nqkv * 2);
  P->q = o;   o = align256(o + T * dm.nq * 2);
  P->vt = o;  o = align256(o + (size_t)B * dm.nk * P->s_pad * 2);
  P->o = o;   o = align256(o + T * dm.nq * 2);
  P->total = o;
  return CCA_OK;
}

#define CCA_TRY_HIP(expr)                         \
  do {                                            \
    hipError_t e_ = (expr);                       \
    if (e_ != hipSuccess) return CCA_ERR_HIP;     \
  } while (0)

}  // namespace

#ifndef CCA_SOURCE_SHA256
#define CCA_SOURCE_SHA256 "unknown"
#endif

extern "C" {

const char* cca_source_hash(void) { return CCA_SOURCE_SHA256; }

const char* cca_status_string(cca_status s) {
  switch (s) {
    case CCA_OK: return "ok";
    case CCA_ERR_INVALID_CONFIG: return "invalid config";
    case CCA_ERR_INVALID_ARG: return "invalid argument";
    case CCA_ERR_UNSUPPORTED: return "unsupported configuration";
    case CCA_ERR_CAPACITY: return "position or length exceeds max_seq_len";
    case CCA_ERR_HIP: return "HIP runtime error";
    case CCA_ERR_OOM: return "out of device memory";
    case CCA_ERR_SCRATCH: return "workspace needed exceeds the static scratch area";
  }
  return "unknown status";
}

cca_status cca_validate_config(const cca_config* c, char* msg, size_t msg_len) {
  if (!c) { put_msg(msg, msg_len, "config is NULL"); return CCA_ERR_INVALID_CONFIG; }
  if (c->struct_size != sizeof(cca_config)) {
    put_msg(msg, msg_len, "struct_size %u != %zu", c->struct_size, sizeof(cca_config));
    return CCA_ERR_INVALID_CONFIG;
  }
  if (c->E <= 0 || c->C <= 0 || c->n_q_heads <= 0 || c->n_kv_heads <= 0) {
    put_msg(msg, msg_len, "E, C and head counts must be positive");
    return CCA_ERR_INVALID_CONFIG;
  }
  if (c->E % (c->C * c->n_q_heads) != 0) {
    put_msg(msg, msg_len, "E %% (C * n_q_heads) != 0");
    return CCA_ERR_INVALID_CONFIG;
  }
  if (c->n_q_heads % c->n_kv_heads != 0) {
    put_msg(msg, msg_len, "n_q_heads %% n_kv_heads != 0");
    return CCA_ERR_INVALID_CONFIG;
  }
  const int d = c->E / (c->C * c->n_q_heads);
  if (d < 2 || d % 2 != 0) {
    put_msg(msg, msg_len, "head dim d = %d must be even", d);
    return CCA_ERR_INVALID_CONFIG;
  }
  if (c->max_seq_len < 1) { put_msg(msg, msg_len, "max_seq_len < 1"); return CCA_ERR_INVALID_CONFIG; }
  if (c->conv_kernel_q < 1 || c->conv_kernel_k < 1) {
    put_msg(msg, msg_len, "conv kernel sizes must be >= 1");
    return CCA_ERR_INVALID_CONFIG;
  }
  if (c->v_shift_channels < 0 || c->v_shift_channels > d) {
    put_msg(msg, msg_len, "v_shift_channels must be in [0, d]");
    return CCA_ERR_INVALID_CONFIG;
  }
  if (c->flags & ~(uint32_t)CCA_DEFAULT_FLAGS) {
    put_msg(msg, msg_len, "unknown flag bits");
    return CCA_ERR_INVALID_CONFIG;
  }
  if ((c->flags & CCA_ROPE) && !(c->rope_base > 1.0)) {
    put_msg(msg, msg_len, "rope_base must be > 1");
    return CCA_ERR_INVALID_CONFIG;
  }
  if (c->dtype != CCA_F32 && c->dtype != CCA_BF16) {
    put_msg(msg, msg_len, "dtype must be CCA_F32 or CCA_BF16");
    return CCA_ERR_INVALID_CONFIG;
  }
  // consistent, but outside what the kernels here implement
  if (d > 128) { put_msg(msg, msg_len, "head dim %d > 128", d); return CCA_ERR_UNSUPPORTED; }
  if (c->conv_kernel_q > kMaxConv || c->conv_kernel_k > kMaxConv) {
    put_msg(msg, msg_len, "conv kernel size > %d", kMaxConv);
    return CCA_ERR_UNSUPPORTED;
  }
  if (c->n_q_heads / c->n_kv_heads > kMaxGroup) {
    put_msg(msg, msg_len, "more than %d query heads per KV head", kMaxGroup);
    return CCA_ERR_UNSUPPORTED;
  }
  if (c->dtype == CCA_BF16 && (c->E % 8 != 0 || d % 8 != 0)) {
    put_msg(msg, msg_len, "bf16 needs E and d multiples of 8");
    return CCA_ERR_UNSUPPORTED;
  }
  if ((long)c->max_seq_len * d > (1L << 31)) {
    put_msg(msg, msg_len, "max_seq_len * d too large");
    return CCA_ERR_UNSUPPORTED;
  }
  put_msg(msg, msg_len, "ok");
  return CCA_OK;
}

cca_status cca_create(const cca_config* cfg, cca_handle** out) {
  if (!out) return CCA_ERR_INVALID_ARG;
  *out = nullptr;
  cca_status st = cca_validate_config(cfg, nullptr, 0);
  if (st != CCA_OK) return st;
  cca_handle* h = new (std::nothrow) cca_handle();
  if (!h) return CCA_ERR_OOM;
  h->cfg = *cfg;
  h->dm = make_dims(*cfg);
  if (hipGetDevice(&h->device) != hipSuccess) { delete h; return CCA_ERR_HIP; }
  h->scratch = device_scratch(h->device);
  // RoPE angles p * base^(-2i/d) in float64, stored as fp32 cos/sin pairs
  const int half = h->dm.d / 2;
  const size_t n = (size_t)cfg->max_seq_len * half;
  std::vector<float2> tab;
  try {
    tab.resize(n);
  } catch (...) {
    delete h;
    return CCA_ERR_OOM;
  }
  for (int i = 0; i < half; ++i) {
    const double inv = std::pow(cfg->rope_base > 1.0 ? cfg->rope_base : 10000.0,
                                -2.0 * (double)i / (double)h->dm.d);
    for (int p = 0; p < cfg->max_seq_len; ++p) {
      const double ang = (double)p * inv;
      tab[(size_t)p * half + i] = make_float2((float)std::cos(ang), (float)std::sin(ang));
    }
  }
  if (hipMalloc((void**)&h->rope, n * sizeof(float2)) != hipSuccess) {
    delete h;
    return CCA_ERR_OOM;
  }
  if (hipMemcpy(h->rope, tab.data(), n * sizeof(float2), hipMemcpyHostToDevice) != hipSuccess) {
    hipFree(h->rope);
    delete h;
    return CCA_ERR_HIP;
  }
  *out = h;
  return CCA_OK;
}

void cca_destroy(cca_handle* h) {
  if (!h) return;
  for (auto& r : h->recs) { hipEventDestroy(r.start); hipEventDestroy(r.stop); }
  for (auto e : h->pool) hipEventDestroy(e);
  if (h->rope) hipFree(h->rope);
  delete h;
}

size_t cca_saved_bytes(const cca_handle* h, int32_t B, int32_t S) {
  if (!h || B <= 0 || S <= 0) return 0;
  return saved_layout(h->dm, B, S).total;
}

cca_status cca_saved_offsets(const cca_handle* h, int32_t B, int32_t S, size_t offsets[8]) {
  if (!h || B <= 0 || S <= 0 || !offsets) return CCA_ERR_INVALID_ARG;
  SavedLayout L = saved_layout(h->dm, B, S);
  for (int i = 0; i < kSavedRegions; ++i) offsets[i] = L.off[i];
  return CCA_OK;
}

size_t cca_state_bytes(const cca_handle* h, int32_t B) {
  if (!h || B <= 0) return 0;
  return (size_t)B * h->dm.state_w * esize(h->dm);
}

size_t cca_workspace_bytes(const cca_handle* h, int op, int32_t B, int32_t S) {
  if (!h || B <= 0) return 0;
  switch (op) {
    case CCA_OP_PREFILL:
      // the saved-tensor regions, then the key-split attention partials (inference)
      return S > 0 ? saved_layout(h->dm, B, S).total +
                         attn_split_part_bytes(h->dm, B, S, prefill_ksplit(h->dm, B, S))
                   : 0;
    case CCA_OP_DECODE: return decode_layout(h->dm, B).total;
    case CCA_OP_BACKWARD: return S > 0 ? bwd_layout(h->dm, B, S).total : 0;
  }
  return 0;
}

cca_status cca_forward_prefill(cca_handle* h, const cca_weights* w, const void* x, int32_t B,
                               int32_t S, void* y, void* saved, void* k_cache, void* v_cache,
                               void* state, void* workspace, void* stream) {
  try {
    if (!h || !w || !x || !y) return CCA_ERR_INVALID_ARG;
    if (B < 1 || S < 1) return CCA_ERR_INVALID_ARG;
    if (S > h->cfg.max_seq_len) return CCA_ERR_CAPACITY;
    if (!w->w_q || !w->w_k || !w->w_v || !w->w_o || !w->conv_q || !w->conv_k)
      return CCA_ERR_INVALID_ARG;
    if ((k_cache == nullptr) != (v_cache == nullptr)) return CCA_ERR_INVALID_ARG;
    void* buf = saved ? saved : workspace;
    if (!buf) return CCA_ERR_INVALID_ARG;
    for (const void* p : {x, (const void*)y, w->w_q, w->w_k, w->w_v, w->w_o, w->conv_q,
                          w->conv_k, (const void*)buf, (const void*)k_cache,
                          (const void*)v_cache, (const void*)state})
      if (!aligned16(p)) return CCA_ERR_INVALID_ARG;
    const Dims& dm = h->dm;
    hipStream_t s = (hipStream_t)stream;
    SavedLayout L = saved_layout(dm, B, S);
    char* base = (char*)buf;
    void* qkv = base + L.off[0];
    void* qr = base + L.off[1];
    void* kr = base + L.off[2];
    void* vs = base + L.off[3];
    void* o = base + L.off[4];
    float* lse = (float*)(base + L.off[5]);
    float* o32 = saved ? (float*)(base + L.off[6]) : nullptr;
    void* vt = base + L.off[7];
    const bool mfma = prefill_uses_mfma(dm);
    const int M = B * S;

    GemmArgs gd = gemm_down(dm, M, x, w, qkv);
    // The latent q~|k~|v~ is fp32 when the call saves for the backward (whose
    // dQ and dK amplify any rounding of it) or the storage is fp32; an
    // inference prefill of bf16 storage keeps it in bf16 (half the bytes).
    const bool lat_f32 = saved != nullptr || !dm.bf16;
    CCA_TRY_HIP(timed(h, "proj_down", s, [&] { return launch_gemm(gd, GemmLayout::NT, dm.bf16, lat_f32, s); }));

    // fused Q: the attention forms Q'' from the bf16 latent (inference, d = 128)
    const bool fuse_q = h->fuse_q && !saved && mfma && dm.bf16 && dm.d == 128 && !lat_f32;
    MixArgs ma{};
    ma.dm = dm; ma.B = B; ma.S = S; ma.qkv = qkv; ma.qkv_f32 = lat_f32;
    ma.conv_q = w->conv_q; ma.conv_k = w->conv_k; ma.rope = h->rope;
    ma.q_out = fuse_q ? nullptr : qr; ma.k_out = kr; ma.v_out = (saved || !mfma) ? vs : nullptr;
    ma.k_out2 = k_cache; ma.v_out2 = v_cache; ma.cap2 = dm.max_seq_len;
    ma.vt_out = vt; ma.s_pad = (int)pad64(S);
    CCA_TRY_HIP(timed(h, "mix", s, [&] { return launch_mix_fwd(ma, s); }));
    if (state)
      CCA_TRY_HIP(timed(h, "write_state", s, [&] { return launch_write_state(dm, B, S, qkv, lat_f32, state, s); }));

    AttnArgs aa{};
    aa.dm = dm; aa.B = B; aa.Sq = S;
    aa.q = qr; aa.k = kr; aa.v = vs;
    aa.kv_bs = (long)dm.Hkv * S * dm.d; aa.kv_hs = (long)S * dm.d;
    aa.vt = vt; aa.s_pad = (int)pad64(S);
    aa.o = o; aa.o32 = o32; aa.lse = lse; aa.decode = false;
    if (fuse_q) {
      aa.qlat = qkv; aa.conv_q = w->conv_q; aa.conv_k = w->conv_k; aa.rope = h->rope;
    } else if (!saved && mfma) {
      // an inference prefill's workspace holds the key-split partials after
      // the saved-tensor regions (cca_workspace_bytes)
      const int P = prefill_ksplit(dm, B, S);
      if (P > 1) {
        aa.ksplit = P;
        aa.part = (float*)(base + L.total);
      }
    }
    CCA_TRY_HIP(timed(h, "attn", s, [&] { return launch_attn_fwd(aa, s); }));

    GemmArgs gu = gemm_nt(M, dm.E, dm.nq, o, dm.nq, w->w_o, dm.nq, y, dm.E);
    CCA_TRY_HIP(timed(h, "proj_up", s, [&] { return launch_gemm(gu, GemmLayout::NT, dm.bf16, false, s); }));
    return CCA_OK;
  } catch (const std::bad_alloc&) {
    return CCA_ERR_OOM;
  } catch (...) {
    return CCA_ERR_HIP;
  }
}

}  // extern "C"

namespace {

// One decode step (both entry points).  th is the handle events are recorded
// into, or null (no timing).
cca_status decode_step(cca_handle* h, cca_handle* th, const cca_weights* w, const void* x_new,
                       const int32_t* pos_host, int32_t B, void* k_cache, void* v_cache,
                       void* state, void* y_new, void* workspace, void* stream) {
  try {
    if (!h || !w || !x_new || !pos_host || !k_cache || !v_cache || !state || !y_new || !workspace)
      return CCA_ERR_INVALID_ARG;
    if (B < 1) return CCA_ERR_INVALID_ARG;
    if (B > kMaxDecodeBatch) return CCA_ERR_UNSUPPORTED;
    if (!w->w_q || !w->w_k || !w->w_v || !w->w_o || !w->conv_q || !w->conv_k)
      return CCA_ERR_INVALID_ARG;
    for (const void* p : {x_new, (const void*)k_cache, (const void*)v_cache, (const void*)state,
                          (const void*)y_new, (const void*)workspace, w->w_q, w->w_k, w->w_v,
                          w->w_o, w->conv_q, w->conv_k})
      if (!aligned16(p)) return CCA_ERR_INVALID_ARG;
    DecodePos pos{};
    for (int b = 0; b < B; ++b) {
      if (pos_host[b] < 0 || pos_host[b] >= h->cfg.max_seq_len) return CCA_ERR_CAPACITY;
      pos.p[b] = pos_host[b];
    }
    const Dims& dm = h->dm;
    hipStream_t s = (hipStream_t)stream;
    DecodeLayout L = decode_layout(dm, B);
    char* base = (char*)workspace;
    float* qkv = (float*)(base + L.qkv);
    void* qn = base + L.q;
    void* on = base + L.o;

    GemmArgs gd = gemm_down(dm, B, x_new, w, qkv);
    float* gpart = dm.bf16 ? (float*)(base + L.gpart) : nullptr;
    // few rows: the split-K skinny GEMM when the shape suits it, else the generic path
    auto gemm_decode = [&](const GemmArgs& ga, bool out_f32) {
      hipError_t e = hipSuccess;
      if (dm.bf16 && launch_gemm_skinny(ga, out_f32, gpart, s, &e)) return e;
      return launch_gemm(ga, GemmLayout::NT, dm.bf16, out_f32, s);
    };
    // the fused mix sums the skinny GEMM's K-slice partials itself (no reduce launch)
    SkinnyPartials sp{qkv, 1, 0, dm.nqkv};
    CCA_TRY_HIP(timed(th, "decode_proj_down", s, [&] {
      hipError_t e = hipSuccess;
      if (mix_decode_fused_ok(dm) && launch_gemm_skinny(gd, true, gpart, s, &e, &sp)) return e;
      sp = SkinnyPartials{qkv, 1, 0, dm.nqkv};
      return gemm_decode(gd, true);
    }));

    MixDecodeArgs md{};
    md.dm = dm; md.B = B; md.pos = pos;
    md.qkv = sp.part; md.qkv_ks = sp.KS; md.qkv_kstride = sp.kstride; md.qkv_ld = sp.ld;
    md.conv_q = w->conv_q; md.conv_k = w->conv_k; md.rope = h->rope;
    md.state = state; md.k_cache = k_cache; md.v_cache = v_cache; md.q_out = qn;
    md.cv = (float*)(base + L.cv);
    CCA_TRY_HIP(timed(th, "decode_mix", s, [&] { return launch_mix_decode(md, s); }));

    AttnArgs aa{};
    aa.dm = dm; aa.B = B; aa.Sq = 1;
    aa.q = qn; aa.k = k_cache; aa.v = v_cache;
    aa.kv_bs = (long)dm.Hkv * dm.max_seq_len * dm.d; aa.kv_hs = (long)dm.max_seq_len * dm.d;
    aa.o = on; aa.lse = nullptr; aa.decode = true; aa.pos = pos;
    aa.part = (float*)(base + L.part); aa.nsplit = decode_splits(dm, B, aa.pos);
    CCA_TRY_HIP(timed(th, "decode_attn", s, [&] { return launch_attn_decode(aa, s); }));

    GemmArgs gu = gemm_nt(B, dm.E, dm.nq, on, dm.nq, w->w_o, dm.nq, y_new, dm.E);
    CCA_TRY_HIP(timed(th, "decode_proj_up", s, [&] { return gemm_decode(gu, false); }));
    return CCA_OK;
  } catch (const std::bad_alloc&) {
    return CCA_ERR_OOM;
  } catch (...) {
    return CCA_ERR_HIP;
  }
}

}  // namespace

extern "C" {

cca_status cca_decode_step(cca_handle* h, const cca_weights* w, const void* x_new,
                           const int32_t* pos_host, int32_t B, void* k_cache, void* v_cache,
                           void* state, void* y_new, void* workspace, void* stream) {
  return decode_step(h, h, w, x_new, pos_host, B, k_cache, v_cache, state, y_new, workspace,
                     stream);
}

cca_status cca_decode_step_noalloc(cca_handle* h, const cca_weights* w, const void* x_new,
                                   const int32_t* pos_host, int32_t B, void* k_cache,
                                   void* v_cache, void* state, void* y_new, void* stream) {
  if (!h) return CCA_ERR_INVALID_ARG;
  if (B < 1) return CCA_ERR_INVALID_ARG;
  if (B > kMaxDecodeBatch) return CCA_ERR_UNSUPPORTED;
  if (decode_layout(h->dm, B).total > kScratchBytes) return CCA_ERR_SCRATCH;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != h->device) return CCA_ERR_INVALID_ARG;
  if (!h->scratch) return CCA_ERR_HIP;
  return decode_step(h, nullptr, w, x_new, pos_host, B, k_cache, v_cache, state, y_new,
                     h->scratch, stream);
}


size_t cca_varlen_workspace_bytes(const cca_handle* h, const int32_t* offsets_host,
                                  const int32_t* start_host, int32_t B) {
  VarlenPlan P;
  if (varlen_plan(h, offsets_host, start_host, B, &P) != CCA_OK) return 0;
  return P.total;
}

cca_status cca_forward_prefill_varlen(cca_handle* h, const cca_weights* w, const void* x,
                                      const int32_t* offsets_host, const int32_t* start_host,
                                      int32_t B, void* y, void* k_cache, void* v_cache,
                                      void* state, void* workspace, void* stream) {
  try {
    if (!h || !w || !offsets_host) return CCA_ERR_INVALID_ARG;
    VarlenPlan P;
    const cca_status st = varlen_plan(h, offsets_host, start_host, B, &P);
    if (st != CCA_OK) return st;
    const Dims& dm = h->dm;
    // the variable-length kernels are built for bf16 with d = 128
    if (!prefill_uses_mfma(dm) || dm.d != 128) return CCA_ERR_UNSUPPORTED;
    if (P.T == 0) return CCA_OK;
    if (!x || !y || !k_cache || !v_cache || !state || !workspace) return CCA_ERR_INVALID_ARG;
    if (!w->w_q || !w->w_k || !w->w_v || !w->w_o || !w->conv_q || !w->conv_k)
      return CCA_ERR_INVALID_ARG;
    for (const void* p : {x, (const void*)y, (const void*)k_cache, (const void*)v_cache,
                          (const void*)state, (const void*)workspace, w->w_q, w->w_k, w->w_v,
                          w->w_o, w->conv_q, w->conv_k})
      if (!aligned16(p)) return CCA_ERR_INVALID_ARG;
    if ((long)P.T * dm.nqkv * 2 >= (1L << 31)) return CCA_ERR_UNSUPPORTED;
    hipStream_t s = (hipStream_t)stream;
    char* base = (char*)workspace;
    void* lat = base + P.lat;
    void* q = base + P.q;
    void* vt = base + P.vt;
    void* o = base + P.o;

    GemmArgs gd = gemm_down(dm, P.T, x, w, lat);
    CCA_TRY_HIP(timed(h, "varlen_proj_down", s, [&] { return launch_gemm(gd, GemmLayout::NT, true, false, s); }));

    MixArgs ma{};
    ma.dm = dm; ma.B = B; ma.S = P.T; ma.qkv = lat; ma.qkv_f32 = false;
    ma.conv_q = w->conv_q; ma.conv_k = w->conv_k; ma.rope = h->rope;
    ma.q_out = q; ma.k_out = nullptr; ma.v_out = nullptr;
    ma.k_out2 = k_cache; ma.v_out2 = v_cache; ma.cap2 = dm.max_seq_len;
    ma.vt_out = nullptr; ma.s_pad = 0; ma.state = state;
    CCA_TRY_HIP(timed(h, "varlen_mix", s, [&] { return launch_mix_varlen_mfma(ma, P.mix, s); }));
    // the mix has read the old state: advance it past each chunk
    CCA_TRY_HIP(timed(h, "varlen_state", s, [&] { return launch_state_varlen(dm, P.mix, lat, state, s); }));
    CCA_TRY_HIP(timed(h, "varlen_vt", s, [&] {
      return launch_vt_varlen(dm, P.mix, v_cache, dm.max_seq_len, vt, P.s_pad, s);
    }));

    AttnArgs aa{};
    aa.dm = dm; aa.B = B; aa.Sq = P.T;
    aa.q = q; aa.k = k_cache; aa.v = v_cache;
    aa.kv_bs = (long)dm.Hkv * dm.max_seq_len * dm.d; aa.kv_hs = (long)dm.max_seq_len * dm.d;
    aa.vt = vt; aa.s_pad = P.s_pad;
    aa.o = o; aa.o32 = nullptr; aa.lse = nullptr; aa.decode = false;
    CCA_TRY_HIP(timed(h, "varlen_attn", s, [&] { return launch_attn_varlen_mfma(aa, P.attn, s); }));

    GemmArgs gu = gemm_nt(P.T, dm.E, dm.nq, o, dm.nq, w->w_o, dm.nq, y, dm.E);
    CCA_TRY_HIP(timed(h, "varlen_proj_up", s, [&] { return launch_gemm(gu, GemmLayout::NT, true, false, s); }));
    return CCA_OK;
  } catch (const std::bad_alloc&) {
    return CCA_ERR_OOM;
  } catch (...) {
    return CCA_ERR_HIP;
  }
}

cca_status cca_backward(cca_handle* h, const cca_weights* w, const void* x, const void* dy,
                        const void* saved, int32_t B, int32_t S, const cca_grads* g,
                        void* workspace, void* stream) {
  try {
    if (!h || !w || !x || !dy || !saved || !g || !workspace) return CCA_ERR_INVALID_ARG;
    if (B < 1 || S < 1) return CCA_ERR_INVALID_ARG;
    if (S > h->cfg.max_seq_len) return CCA_ERR_CAPACITY;
    if (!g->dx || !g->dw_q || !g->dw_k || !g->dw_v || !g->dw_o || !g->dconv_q || !g->dconv_k)
      return CCA_ERR_INVALID_ARG;
    if (!w->w_q || !w->w_k || !w->w_v || !w->w_o || !w->conv_q || !w->conv_k)
      return CCA_ERR_INVALID_ARG;
    for (const void* p : {x, dy, saved, (const void*)workspace, (const void*)g->dx,
                          (const void*)g->dw_q, (const void*)g->dw_k, (const void*)g->dw_v,
                          (const void*)g->dw_o, (const void*)g->dconv_q, (const void*)g->dconv_k,
                          w->w_q, w->w_k, w->w_v, w->w_o, w->conv_q, w->conv_k})
      if (!aligned16(p)) return CCA_ERR_INVALID_ARG;
    const Dims& dm = h->dm;
    hipStream_t s = (hipStream_t)stream;
    SavedLayout SL = saved_layout(dm, B, S);
    BwdLayout L = bwd_layout(dm, B, S);
    const char* sb = (const char*)saved;
    char* wb = (char*)workspace;
    const float* qkv = (const float*)(sb + SL.off[0]);
    const void* qr = sb + SL.off[1];
    const void* kr = sb + SL.off[2];
    const void* vs = sb + SL.off[3];
    const void* o = sb + SL.off[4];
    const float* lse = (const float*)(sb + SL.off[5]);
    const float* o32 = (const float*)(sb + SL.off[6]);
    void* dO = wb + L.dO;
    float* Dsum = (float*)(wb + L.Dsum);
    float* dq = (float*)(wb + L.dq);
    float* dk = (float*)(wb + L.dk);
    float* dv = (float*)(wb + L.dv);
    void* dqkv = wb + L.dqkv;
    const int M = B * S;

    const bool nt = bwd_gemm_nt(dm);
    const int Mp = (int)pad64(M);
    void* wT = wb + L.wT;
    void* tA = wb + L.tA;
    void* tB = wb + L.tB;
    float* gpart = (float*)(wb + L.gpart);
    // weight gradient C[Mo x No] (fp32, segments along Mo) = A^T-major operands
    // at[Mo x Mp] . bt[No x Mp]^T on the NT kernel, split over K when the
    // output alone cannot fill the chip; partials summed in a fixed order.
    auto weight_grad = [&](int Mo, int No, const void* at, const void* bt, GemmArgs gout) {
      GemmArgs gg = gemm_nt(Mo, No, Mp, at, Mp, bt, Mp, gpart, No);
      const int tiles = ((Mo + 255) / 256) * ((No + 255) / 256);
      int ks = 1;
      while (ks < kMaxSplit && tiles * ks < 256 && (Mp / 64) % (2 * ks) == 0) ks *= 2;
      gg.ksplit = ks;
      gg.c_split_stride = (long)Mo * No;
      hipError_t e = hipSuccess;
      if (ks > 1 && launch_gemm_nt_big(gg, true, s, &e)) {
        if (e != hipSuccess) return e;
        float* outs[3] = {(float*)gout.c_ptr[0], (float*)gout.c_ptr[1], (float*)gout.c_ptr[2]};
        return launch_splitk_reduce(gpart, ks, Mo, No, outs, gout.c_start, gout.c_nseg, gout.ldc,
                                    s);
      }
      gout.a = at; gout.lda = Mp; gout.b_ptr[0] = bt; gout.ldb = Mp; gout.K = Mp;
      return launch_gemm(gout, GemmLayout::NT, true, true, s);
    };
    // The same product straight from the token-major operands a_tok [M x Mo]
    // and b_tok [M x No] (K-major tiles, no transposed copies), split over K
    // into the fp32 partials; false (nothing launched) when the shape does
    // not suit the 256 x 256 kernel.
    auto weight_grad_tn = [&](int Mo, int No, const void* a_tok, long lda, const void* b_tok,
                              long ldb, GemmArgs gout, hipError_t* e) -> bool {
      GemmArgs gg = gemm_nt(Mo, No, Mp, a_tok, lda, b_tok, ldb, gpart, No);
      gg.k_valid = (int)M;
      const int tiles = ((Mo + 255) / 256) * ((No + 255) / 256);
      int ks = 1;
      while (ks < kMaxSplit && tiles * ks < 256 && (Mp / 64) % (2 * ks) == 0) ks *= 2;
      if (ks < 2) return false;
      gg.ksplit = ks;
      gg.c_split_stride = (long)Mo * No;
      if (!launch_gemm_nt_big(gg, true, s, e, GemmLayout::TN)) return false;
      if (*e != hipSuccess) return true;
      float* outs[3] = {(float*)gout.c_ptr[0], (float*)gout.c_ptr[1], (float*)gout.c_ptr[2]};
      *e = launch_splitk_reduce(gpart, ks, Mo, No, outs, gout.c_start, gout.c_nseg, gout.ldc, s);
      return true;
    };

    // dO = dY W_o ; dW_o = dY^T O
    if (nt) {
      CCA_TRY_HIP(timed(h, "bwd_proj_up_dx", s, [&] {
        hipError_t e = launch_transpose_bf16(w->w_o, dm.nq, dm.E, dm.nq, dm.E, wT, dm.E, s);
        if (e != hipSuccess) return e;
        GemmArgs g1 = gemm_nt(M, dm.nq, dm.E, dy, dm.E, wT, dm.E, dO, dm.nq);
        return launch_gemm(g1, GemmLayout::NT, true, false, s);
      }));
      CCA_TRY_HIP(timed(h, "bwd_proj_up_dw", s, [&] {
        GemmArgs gout = gemm_nt(dm.E, dm.nq, Mp, nullptr, 0, nullptr, 0, g->dw_o, dm.nq);
        hipError_t e = hipSuccess;
        if (weight_grad_tn(dm.E, dm.nq, dy, dm.E, o, dm.nq, gout, &e)) return e;
        e = launch_transpose_bf16(dy, dm.E, M, dm.E, Mp, tA, Mp, s);
        if (e == hipSuccess) e = launch_transpose_bf16(o, dm.nq, M, dm.nq, Mp, tB, Mp, s);
        if (e != hipSuccess) return e;
        return weight_grad(dm.E, dm.nq, tA, tB, gout);
      }));
    } else {
      GemmArgs g1 = gemm_nt(M, dm.nq, dm.E, dy, dm.E, w->w_o, dm.nq, dO, dm.nq);
      CCA_TRY_HIP(timed(h, "bwd_proj_up_dx", s, [&] { return launch_gemm(g1, GemmLayout::NN, dm.bf16, false, s); }));
      GemmArgs g2 = gemm_nt(dm.E, dm.nq, M, dy, dm.E, o, dm.nq, g->dw_o, dm.nq);
      CCA_TRY_HIP(timed(h, "bwd_proj_up_dw", s, [&] { return launch_gemm(g2, GemmLayout::TN, dm.bf16, true, s); }));
    }

    AttnBwdArgs ab{};
    ab.dm = dm; ab.B = B; ab.S = S;
    ab.q = qr; ab.k = kr; ab.v = vs; ab.o32 = o32; ab.dO = dO; ab.lse = lse; ab.Dsum = Dsum;
    ab.dq = dq; ab.dk = dk; ab.dv = dv;
    ab.amax_part = (float*)(wb + L.amax);
    ab.dscale = ab.amax_part + kAmaxParts;
    {
      // fp16 copies for the MFMA path: Q'' | K'' | V' | dO, each 256-byte aligned
      const long sp = pad64(S);
      char* t = wb + L.trans;
      ab.s_pad = (int)sp;
      ab.q16 = t;
      ab.k16 = t + align256((size_t)B * dm.nq * sp * 2);
      ab.v16 = (char*)ab.k16 + align256((size_t)B * dm.nk * sp * 2);
      ab.do16 = (char*)ab.v16 + align256((size_t)B * dm.nk * sp * 2);
      ab.dk2 = (float*)((char*)ab.do16 + align256((size_t)B * dm.nq * sp * 2));
      ab.dv2 = (float*)((char*)ab.dk2 + align256((size_t)B * S * dm.nk * 4));
      if (attn_bwd_mfma_supported(dm) && attn_bwd_parts(dm) == 4) {
        ab.dk3 = (float*)((char*)ab.dv2 + align256((size_t)B * S * dm.nk * 4));
        ab.dv3 = (float*)((char*)ab.dk3 + align256((size_t)B * S * dm.nk * 4));
        ab.dk4 = (float*)((char*)ab.dv3 + align256((size_t)B * S * dm.nk * 4));
        ab.dv4 = (float*)((char*)ab.dk4 + align256((size_t)B * S * dm.nk * 4));
      }
    }
    // the mix backward's pointwise pass adds the second-half dK / dV partials
    // as it reads dK / dV, when it can (no separate sum launch)
    const bool sum_in_mix = attn_bwd_mfma_supported(dm) && mix_bwd_adds_dkdv2(dm) &&
                            attn_bwd_parts(dm) == 2;
    ab.sum_by_consumer = sum_in_mix;
    CCA_TRY_HIP(timed(h, "bwd_attn", s, [&] { return launch_attn_bwd(ab, s); }));

    MixBwdArgs mb{};
    mb.dm = dm; mb.B = B; mb.S = S; mb.qkv = qkv;
    mb.conv_q = w->conv_q; mb.conv_k = w->conv_k; mb.rope = h->rope;
    mb.dq = dq; mb.dk = dk; mb.dv = dv; mb.dqkv = dqkv;
    mb.dconv_part = (float*)(wb + L.part);
    mb.dconv_q = (float*)g->dconv_q; mb.dconv_k = (float*)g->dconv_k;
    mb.scratch = (float*)(wb + L.scratch);
    mb.tapT = mix_bwd_tapT_bytes(dm) ? (void*)(wb + L.tapT) : nullptr;
    mb.dk2 = sum_in_mix ? ab.dk2 : nullptr;
    mb.dv2 = sum_in_mix ? ab.dv2 : nullptr;
    CCA_TRY_HIP(timed(h, "bwd_mix", s, [&] { return launch_mix_bwd(mb, s); }));

    // dx = dq~ W_q + dk~ W_k + dv~ W_v ; dW_* = d*~^T x
    GemmArgs g4 = gemm_nt(dm.nqkv, dm.E, M, dqkv, dm.nqkv, x, dm.E, g->dw_q, dm.E);
    g4.c_ptr[1] = g->dw_k; g4.c_start[1] = dm.nq;
    g4.c_ptr[2] = g->dw_v; g4.c_start[2] = dm.nq + dm.nk;
    g4.c_nseg = 3;
    if (nt) {
      CCA_TRY_HIP(timed(h, "bwd_proj_down_dx", s, [&] {
        // [W_q; W_k; W_v]^T [E x nqkv], one segment at a time
        const void* seg[3] = {w->w_q, w->w_k, w->w_v};
        const int rows[3] = {dm.nq, dm.nk, dm.nk}, col0[3] = {0, dm.nq, dm.nq + dm.nk};
        for (int i = 0; i < 3; ++i) {
          hipError_t e = launch_transpose_bf16(seg[i], dm.E, rows[i], dm.E, rows[i],
                                               (char*)wT + (size_t)col0[i] * 2, dm.nqkv, s);
          if (e != hipSuccess) return e;
        }
        GemmArgs g3 = gemm_nt(M, dm.E, dm.nqkv, dqkv, dm.nqkv, wT, dm.nqkv, g->dx, dm.E);
        return launch_gemm(g3, GemmLayout::NT, true, false, s);
      }));
      CCA_TRY_HIP(timed(h, "bwd_proj_down_dw", s, [&] {
        hipError_t e = hipSuccess;
        if (weight_grad_tn(dm.nqkv, dm.E, dqkv, dm.nqkv, x, dm.E, g4, &e)) return e;
        e = launch_transpose_bf16(dqkv, dm.nqkv, M, dm.nqkv, Mp, tB, Mp, s);
        if (e == hipSuccess) e = launch_transpose_bf16(x, dm.E, M, dm.E, Mp, tA, Mp, s);
        if (e != hipSuccess) return e;
        return weight_grad(dm.nqkv, dm.E, tB, tA, g4);
      }));
    } else {
      GemmArgs g3 = gemm_nt(M, dm.E, dm.nqkv, dqkv, dm.nqkv, w->w_q, dm.E, g->dx, dm.E);
      g3.b_ptr[1] = w->w_k; g3.b_start[1] = dm.nq;
      g3.b_ptr[2] = w->w_v; g3.b_start[2] = dm.nq + dm.nk;
      g3.b_nseg = 3;
      CCA_TRY_HIP(timed(h, "bwd_proj_down_dx", s, [&] { return launch_gemm(g3, GemmLayout::NN, dm.bf16, false, s); }));
      CCA_TRY_HIP(timed(h, "bwd_proj_down_dw", s, [&] { return launch_gemm(g4, GemmLayout::TN, dm.bf16, true, s); }));
    }
    return CCA_OK;
  } catch (const std::bad_alloc&) {
    return CCA_ERR_OOM;
  } catch (...) {
    return CCA_ERR_HIP;
  }
}

cca_status cca_profile_enable(cca_handle* h, int enable) {
  if (!h) return CCA_ERR_INVALID_ARG;
  for (auto& r : h->recs) { h->pool.push_back(r.start); h->pool.push_back(r.stop); }
  h->recs.clear();
  h->profiling = enable != 0;
  return CCA_OK;
}

cca_status cca_set_prefill_fusion(cca_handle* h, int32_t on) {
  if (!h) return CCA_ERR_INVALID_ARG;
  h->fuse_q = on != 0;
  return CCA_OK;
}

cca_status cca_profile_flush(cca_handle* h, void* buf, size_t bytes) {
  if (!h) return CCA_ERR_INVALID_ARG;
  if (buf && (!aligned16(buf) || bytes % 16 != 0 || bytes == 0)) return CCA_ERR_INVALID_ARG;
  h->flush_buf = buf;
  h->flush_bytes = buf ? bytes : 0;
  return CCA_OK;
}

int cca_profile_read(cca_handle* h, cca_kernel_time* out, int max) {
  if (!h) return -1;
  std::vector<std::string> order;
  std::map<std::string, std::pair<int, double>> acc;
  for (auto& r : h->recs) {
    float ms = 0.0f;
    if (hipEventSynchronize(r.stop) != hipSuccess) return -1;
    if (hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) return -1;
    auto it = acc.find(r.name);
    if (it == acc.end()) {
      order.push_back(r.name);
      acc[r.name] = {1, ms};
    } else {
      it->second.first += 1;
      it->second.second += ms;
    }
  }
  int n = 0;
  for (auto& name : order) {
    if (out && n < max) {
      std::memset(out[n].name, 0, sizeof(out[n].name));
      std::strncpy(out[n].name, name.c_str(), sizeof(out[n].name) - 1);
      out[n].launches = acc[name].first;
      out[n].total_ms = acc[name].second;
    }
    ++n;
  }
  return n;
}

}  // extern "C"
