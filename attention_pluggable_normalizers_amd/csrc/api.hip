// libattn C ABI: argument validation, kernel selection and launch.
//
// The selection is a static table on (dtype, head dim, paged, Lq); every
// accepted request has exactly one kernel family and nothing falls back at
// run time ("HF Attention Normalizers", "Strict vs Fallback Mode": strict).

#include <math.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "common.h"

namespace attn {
namespace {

thread_local char g_detail[256] = "";

int fail(int status, const char* fmt, const char* what = nullptr) {
  snprintf(g_detail, sizeof(g_detail), fmt, what ? what : "");
  return status;
}

int check_tensor(const attn_tensor* t, const char* name) {
  if (!t) return fail(ATTN_E_INVALID, "%s descriptor is NULL", name);
  if (t->reserved != 0) return fail(ATTN_E_INVALID, "%s.reserved must be 0", name);
  const bool empty = t->shape[0] == 0 || t->shape[1] == 0 || t->shape[2] == 0 || t->shape[3] == 0;
  if (!t->data && !empty) return fail(ATTN_E_INVALID, "%s data pointer is NULL", name);
  if (t->dtype != ATTN_F32 && t->dtype != ATTN_BF16)
    return fail(ATTN_E_UNSUPPORTED, "%s dtype is neither f32 nor bf16", name);
  for (int d = 0; d < 4; ++d) {
    if (t->shape[d] < 0) return fail(ATTN_E_INVALID, "%s has a negative extent", name);
    if (t->stride[d] < 0) return fail(ATTN_E_INVALID, "%s has a negative stride", name);
  }
  if (t->stride[3] != 1) return fail(ATTN_E_INVALID, "%s last dimension is not contiguous", name);
  return ATTN_OK;
}

// Validates everything and fills the kernel arguments.
int validate(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
             const attn_paged_kv* paged, const attn_params* p, const attn_tensor* out,
             float* row_stats, FwdArgs* a, bool need_data) {
  g_detail[0] = 0;
  int st;
  if (!p) return fail(ATTN_E_INVALID, "params pointer is NULL");
  if (need_data) {
    if ((st = check_tensor(q, "q")) || (st = check_tensor(k, "k")) || (st = check_tensor(v, "v")) ||
        (st = check_tensor(out, "out")))
      return st;
  } else {
    attn_tensor qq, kk, vv;
    if (!q || !k || !v) return fail(ATTN_E_INVALID, "q, k or v descriptor is NULL");
    qq = *q; kk = *k; vv = *v;
    qq.data = kk.data = vv.data = (void*)1;  // sizes only
    if ((st = check_tensor(&qq, "q")) || (st = check_tensor(&kk, "k")) || (st = check_tensor(&vv, "v")))
      return st;
  }
  if (k->dtype != q->dtype || v->dtype != q->dtype || (out && out->dtype != q->dtype))
    return fail(ATTN_E_INVALID, "q, k, v and out must share one dtype");
  if (p->normalizer < ATTN_SOFTMAX || p->normalizer > ATTN_ENTMAX15)
    return fail(ATTN_E_INVALID, "unknown normalizer");
  if (p->causal != 0 && p->causal != 1) return fail(ATTN_E_INVALID, "causal must be 0 or 1");
  if (p->window < 0) return fail(ATTN_E_INVALID, "window must be >= 0");
  if (p->window > 0 && !p->causal)
    return fail(ATTN_E_INVALID, "a sliding window requires causal masking");
  if (!(p->softcap >= 0.f) || !isfinite(p->softcap))
    return fail(ATTN_E_INVALID, "softcap must be finite and >= 0");
  if (!isfinite(p->scaling)) return fail(ATTN_E_INVALID, "scaling must be finite");
  if (p->sinks && p->normalizer != ATTN_SOFTMAX1)
    return fail(ATTN_E_INVALID, "sink logits apply to softmax1 only");

  const int64_t B = q->shape[0], Hq = q->shape[1], Lq = q->shape[2], D = q->shape[3];
  int64_t Hkv, Lk;
  memset(a, 0, sizeof(*a));
  if (!paged) {
    if (k->shape[0] != B || v->shape[0] != B) return fail(ATTN_E_INVALID, "k/v batch differs from q");
    Hkv = k->shape[1];
    Lk = k->shape[2];
    if (v->shape[1] != Hkv || v->shape[2] != Lk) return fail(ATTN_E_INVALID, "k and v shapes differ");
    if (k->shape[3] != D || v->shape[3] != D) return fail(ATTN_E_INVALID, "head dims of q, k, v differ");
    a->k_sb = k->stride[0]; a->k_sh = k->stride[1]; a->k_sl = k->stride[2];
    a->v_sb = v->stride[0]; a->v_sh = v->stride[1]; a->v_sl = v->stride[2];
  } else {
    if (!paged->block_table || !paged->seq_lens)
      return fail(ATTN_E_INVALID, "paged block_table or seq_lens is NULL");
    if (paged->block_size <= 0 || paged->max_blocks <= 0)
      return fail(ATTN_E_INVALID, "paged block_size and max_blocks must be > 0");
    if (k->shape[1] != paged->block_size || v->shape[1] != paged->block_size)
      return fail(ATTN_E_INVALID, "cache slot dimension differs from block_size");
    if ((int64_t)paged->max_blocks * paged->block_size > (int64_t)INT32_MAX / 2)
      return fail(ATTN_E_UNSUPPORTED, "max_blocks * block_size too large");
    Hkv = k->shape[2];
    Lk = (int64_t)paged->max_blocks * paged->block_size;
    if (v->shape[0] != k->shape[0] || v->shape[2] != Hkv)
      return fail(ATTN_E_INVALID, "k and v cache shapes differ");
    if (k->shape[3] != D || v->shape[3] != D) return fail(ATTN_E_INVALID, "head dims of q, k, v differ");
    a->k_sb = k->stride[0]; a->k_sl = k->stride[1]; a->k_sh = k->stride[2];
    a->v_sb = v->stride[0]; a->v_sl = v->stride[1]; a->v_sh = v->stride[2];
    a->paged = 1;
    a->block_table = paged->block_table;
    a->seq_lens = paged->seq_lens;
    a->block_size = paged->block_size;
    a->max_blocks = paged->max_blocks;
    if (k->shape[0] > INT32_MAX) return fail(ATTN_E_UNSUPPORTED, "too many cache pages");
    a->num_blocks = (int)k->shape[0];
  }
  if (Hkv <= 0 && Hq > 0) return fail(ATTN_E_INVALID, "k/v have no heads");
  if (Hkv > 0 && Hq % Hkv != 0) return fail(ATTN_E_INVALID, "Hq must be a multiple of Hkv");
  if (D < 1 || D > 256) return fail(ATTN_E_UNSUPPORTED, "head dim must be in 1..256");
  if (B > INT32_MAX || Hq > INT32_MAX || Lq > INT32_MAX / 2 || Lk > INT32_MAX / 2)
    return fail(ATTN_E_UNSUPPORTED, "an extent exceeds the 32-bit index range");
  if (B * Hq * Lq > (int64_t)INT32_MAX) return fail(ATTN_E_UNSUPPORTED, "too many query rows");
  if (out) {
    for (int d = 0; d < 4; ++d)
      if (out->shape[d] != q->shape[d]) return fail(ATTN_E_INVALID, "out shape differs from q");
    a->out = out->data;
    a->o_sb = out->stride[0]; a->o_sh = out->stride[1]; a->o_sl = out->stride[2];
  }
  a->q = q->data; a->k = k->data; a->v = v->data;
  a->q_sb = q->stride[0]; a->q_sh = q->stride[1]; a->q_sl = q->stride[2];
  a->stats = row_stats;
  a->dtype = q->dtype;
  a->B = (int)B; a->Hq = (int)Hq; a->Hkv = (int)Hkv; a->G = Hkv > 0 ? (int)(Hq / Hkv) : 1;
  a->Lq = (int)Lq; a->Lk = (int)Lk; a->D = (int)D;
  a->norm = p->normalizer; a->causal = p->causal; a->window = p->window;
  a->softcap = p->softcap; a->scaling = p->scaling;
  a->sinks = p->sinks;
  if (p->block_mask) {
    const attn_block_mask* m = p->block_mask;
    if (paged) return fail(ATTN_E_UNSUPPORTED, "block masks apply to contiguous K/V only");
    if (m->block_q <= 0 || m->block_k <= 0) return fail(ATTN_E_INVALID, "block mask block sizes must be > 0");
    if (m->num_heads != 1 && m->num_heads != Hq)
      return fail(ATTN_E_INVALID, "block mask num_heads must be 1 or Hq");
    if (m->max_kv_blocks < 0) return fail(ATTN_E_INVALID, "block mask max_kv_blocks must be >= 0");
    if (!m->kv_num_blocks || (m->max_kv_blocks > 0 && !m->kv_indices))
      return fail(ATTN_E_INVALID, "block mask kv_num_blocks or kv_indices is NULL");
    if ((Lk + m->block_k - 1) / m->block_k > 16384)
      return fail(ATTN_E_UNSUPPORTED, "block mask has more than 16384 key blocks");
    const int64_t nqb = (Lq + m->block_q - 1) / m->block_q;
    if (B * m->num_heads * nqb * (int64_t)m->max_kv_blocks > (int64_t)INT32_MAX * 8)
      return fail(ATTN_E_UNSUPPORTED, "block mask too large");
    a->bm_num = m->kv_num_blocks;
    a->bm_idx = m->kv_indices;
    a->bm_bq = m->block_q;
    a->bm_bk = m->block_k;
    a->bm_heads = m->num_heads;
    a->bm_max = m->max_kv_blocks;
  }
  return ATTN_OK;
}

// attn_fwd's validation plus the packed-batch descriptor of attn_fwd_varlen.
int validate_varlen(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
                    const attn_varlen* varlen, const attn_params* p, const attn_tensor* out,
                    float* row_stats, FwdArgs* a) {
  int st = validate(q, k, v, nullptr, p, out, row_stats, a, true);
  if (st) return st;
  if (!varlen) return fail(ATTN_E_INVALID, "varlen descriptor is NULL");
  if (a->bm_num) return fail(ATTN_E_UNSUPPORTED, "block masks apply to a padded batch only");
  if (q->shape[0] != 1 || k->shape[0] != 1)
    return fail(ATTN_E_INVALID, "packed q, k, v must have batch extent 1");
  if (varlen->num_seqs < 0 || varlen->max_seqlen_q < 0)
    return fail(ATTN_E_INVALID, "num_seqs and max_seqlen_q must be >= 0");
  if (varlen->num_seqs > 0 && (!varlen->cu_seqlens_q || !varlen->cu_seqlens_k))
    return fail(ATTN_E_INVALID, "cu_seqlens_q or cu_seqlens_k is NULL");
  if ((int64_t)varlen->num_seqs * a->Hq * varlen->max_seqlen_q > (int64_t)INT32_MAX)
    return fail(ATTN_E_UNSUPPORTED, "too many query rows");
  a->cu_q = varlen->cu_seqlens_q;
  a->cu_k = varlen->cu_seqlens_k;
  a->B = varlen->num_seqs;
  a->max_q = varlen->max_seqlen_q;
  return ATTN_OK;
}

enum class Path { kNone, kGeneric, kPrefill, kDecode };

Path select(const FwdArgs& a) {
  if ((int64_t)a.B * a.Hq * a.Lq == 0) return Path::kNone;
  if (a.paged && decode_supported(a)) return Path::kDecode;
  if (prefill_mfma_supported(a)) return Path::kPrefill;
  return Path::kGeneric;
}

size_t workspace_for(const FwdArgs& a) {
  return select(a) == Path::kDecode ? decode_workspace_bytes(a) : 0;
}

}  // namespace

// For the backward entry points (backward.hip): the forward's validation of
// q, k, v and the parameters (contiguous K/V), and the error-detail setter.
int validate_fwd_args(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
                      const attn_params* p, FwdArgs* a, bool need_data) {
  return validate(q, k, v, nullptr, p, need_data ? q : nullptr, nullptr, a, need_data);
}
int bwd_fail(int status, const char* msg) { return fail(status, "%s", msg); }

}  // namespace attn

using namespace attn;

extern "C" int attn_fwd(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
                        const attn_paged_kv* paged, const attn_params* p,
                        const attn_tensor* out, float* row_stats, void* workspace,
                        size_t workspace_bytes, void* stream) {
  FwdArgs a;
  int st = validate(q, k, v, paged, p, out, row_stats, &a, true);
  if (st) return st;
  const Path path = select(a);
  const size_t need = workspace_for(a);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(ATTN_E_WORKSPACE, "workspace smaller than attn_fwd_workspace_bytes()");
  if (path == Path::kNone) return ATTN_OK;
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();  // clear a launch error left pending on this thread
  hipError_t e;
  switch (path) {
    case Path::kPrefill: e = launch_prefill_mfma(a, s); break;
    case Path::kDecode: e = launch_decode(a, workspace, s); break;
    default: e = launch_generic(a, s); break;
  }
  if (e != hipSuccess) return fail(ATTN_E_LAUNCH, "HIP launch failed: %s", hipGetErrorString(e));
  return ATTN_OK;
}

// ---------------------------------------------------------------------------
// Allocation-free variant of attn_fwd: the workspace is a fixed device array
// of this library (each GPU the library runs on holds its own copy until the
// process ends).  In host code `scratch` names a host-side stand-in, not the
// device memory: its device address is taken once per device with
// hipGetSymbolAddress and only that address is ever passed to a kernel.
namespace {

constexpr size_t kScratchBytes = (size_t)128 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device (nullptr: not yet)

// Device address of this device's `scratch` (looked up on the first call on
// the device, with it current); nullptr with *err set on failure.
void* scratch_for(int dev, hipError_t* err) {
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      *err = e != hipSuccess ? e : hipErrorInvalidSymbol;
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" int attn_fwd_noalloc(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
                                const attn_paged_kv* paged, const attn_params* p,
                                const attn_tensor* out, float* row_stats, void* stream) {
  FwdArgs a;
  int st = validate(q, k, v, paged, p, out, row_stats, &a, true);
  if (st) return st;
  const Path path = select(a);
  const size_t need = workspace_for(a);
  if (need > kScratchBytes) {
    snprintf(g_detail, sizeof(g_detail),
             "needs %zu bytes of workspace, more than the %zu bytes of the library's fixed "
             "scratch; call attn_fwd with a workspace",
             need, kScratchBytes);
    return ATTN_E_WORKSPACE;
  }
  if (path == Path::kNone) return ATTN_OK;
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  void* ws = nullptr;
  if (need > 0) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= kMaxDevices)
      return fail(ATTN_E_LAUNCH, "no usable current device for the fixed scratch");
    ws = scratch_for(dev, &e);
    if (!ws) return fail(ATTN_E_LAUNCH, "hipGetSymbolAddress of the scratch failed: %s",
                         hipGetErrorString(e));
  }
  hipError_t e;
  switch (path) {
    case Path::kPrefill: e = launch_prefill_mfma(a, s); break;
    case Path::kDecode: e = launch_decode(a, ws, s); break;
    default: e = launch_generic(a, s); break;
  }
  if (e != hipSuccess) return fail(ATTN_E_LAUNCH, "HIP launch failed: %s", hipGetErrorString(e));
  return ATTN_OK;
}

extern "C" int attn_fwd_varlen(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
                               const attn_varlen* varlen, const attn_params* p,
                               const attn_tensor* out, float* row_stats, void* workspace,
                               size_t workspace_bytes, void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  FwdArgs a;
  int st = validate_varlen(q, k, v, varlen, p, out, row_stats, &a);
  if (st) return st;
  if ((int64_t)a.B * a.Hq * a.max_q == 0 || a.Lq == 0) return ATTN_OK;
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  const hipError_t e = prefill_mfma_supported(a) ? launch_prefill_mfma(a, s) : launch_generic(a, s);
  if (e != hipSuccess) return fail(ATTN_E_LAUNCH, "HIP launch failed: %s", hipGetErrorString(e));
  return ATTN_OK;
}

extern "C" int attn_fwd_path(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
                             const attn_paged_kv* paged, const attn_params* p,
                             const attn_tensor* out, int* path) {
  if (!path) return fail(ATTN_E_INVALID, "path pointer is NULL");
  FwdArgs a;
  int st = validate(q, k, v, paged, p, out, nullptr, &a, true);
  if (st) return st;
  switch (select(a)) {
    case Path::kNone: *path = ATTN_PATH_NONE; break;
    case Path::kPrefill: *path = ATTN_PATH_PREFILL_MFMA; break;
    case Path::kDecode: *path = ATTN_PATH_DECODE_SPLIT; break;
    default: *path = ATTN_PATH_PER_ROW; break;
  }
  return ATTN_OK;
}

extern "C" int attn_fwd_varlen_path(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
                                    const attn_varlen* varlen, const attn_params* p,
                                    const attn_tensor* out, int* path) {
  if (!path) return fail(ATTN_E_INVALID, "path pointer is NULL");
  FwdArgs a;
  int st = validate_varlen(q, k, v, varlen, p, out, nullptr, &a);
  if (st) return st;
  if ((int64_t)a.B * a.Hq * a.max_q == 0 || a.Lq == 0)
    *path = ATTN_PATH_NONE;
  else
    *path = prefill_mfma_supported(a) ? ATTN_PATH_PREFILL_MFMA : ATTN_PATH_PER_ROW;
  return ATTN_OK;
}

extern "C" int attn_fwd_workspace_bytes(const attn_tensor* q, const attn_tensor* k,
                                        const attn_tensor* v, const attn_paged_kv* paged,
                                        const attn_params* p, size_t* bytes) {
  if (!bytes) return fail(ATTN_E_INVALID, "bytes pointer is NULL");
  attn_paged_kv pk;
  const attn_paged_kv* pp = paged;
  if (paged) {  // sizes only: the device pointers are not needed here
    pk = *paged;
    if (!pk.block_table) pk.block_table = (const int32_t*)1;
    if (!pk.seq_lens) pk.seq_lens = (const int32_t*)1;
    pp = &pk;
  }
  FwdArgs a;
  int st = validate(q, k, v, pp, p, nullptr, nullptr, &a, false);
  if (st) return st;
  *bytes = workspace_for(a);
  return ATTN_OK;
}

extern "C" const char* attn_strerror(int status) {
  switch (status) {
    case ATTN_OK: return "ATTN_OK: success";
    case ATTN_E_INVALID: return "ATTN_E_INVALID: invalid argument";
    case ATTN_E_UNSUPPORTED: return "ATTN_E_UNSUPPORTED: unsupported request";
    case ATTN_E_WORKSPACE: return "ATTN_E_WORKSPACE: workspace missing or too small";
    case ATTN_E_LAUNCH: return "ATTN_E_LAUNCH: kernel launch failed";
    default: return "unknown attn status";
  }
}

extern "C" const char* attn_last_error_detail(void) { return g_detail; }

extern "C" int attn_abi_version(void) { return ATTN_ABI_VERSION; }
