// Backward of the attention forward: dQ, dK, dV (and softmax1 sink
// gradients) for the four normalizers, recomputing the weights from the row
// statistics the forward saved ("HF Attention Normalizers", "Important
// Limitations": softmax1 saves row max and denominator and recomputes P in
// its fused backward; the sparse kernels save one threshold per query row
// and recompute tiles).  fp32 arithmetic, one wave per row:
//
//   query kernel (one wave per query row i):
//     pass 1   over the row's keys j: p_ij from the statistics, dP_ij =
//              dO_i . v_j, and the row constant c_i of the normalizer's
//              Jacobian -- softmax family: sum_j p dP; sparsemax: the mean of
//              dP over the support; 1.5-entmax: sum u dP / sum u with
//              u = sqrt(p) (= z - tau on the support); stored per row
//     pass 2   ds_ij (softmax family p (dP - c); sparsemax dP - c on the
//              support; 1.5-entmax u (dP - c) on the support), through
//              softcap and scaling to draw_ij; dQ_i = sum_j draw_ij k_j
//   key kernel (one wave per key row j of a key/value head): over the query
//     rows i of the head's G query heads that see j: dV_j = sum p_ij dO_i,
//     dK_j = sum draw_ij q_i (c_i from the query kernel)
//   sink kernel (softmax1 with sinks): d b_h = -sum_i p_sink,i c_i.
// Contiguous K/V, padded or packed ("HF Attention Normalizers", "Packed
// Variable-Length Attention": each request differentiated as a batch entry
// of its own, tokens outside every request get zero gradients), with or
// without a block mask (keys outside the listed blocks carry no weight and
// no gradient).  Every sum runs in a fixed order (deterministic).

#include <string.h>

#include <algorithm>

#include "common.h"

namespace attn {
namespace {

constexpr int kMaxD = 256;
constexpr int kMaxBlocks = 16384;  // block masks: query / key blocks per bitmap in LDS

// Packed batch: the request that holds token `tok` under the cumulative
// offsets cu[0..nreq] is the last r < nreq with cu[r] <= tok (the caller
// checks that tok lies inside it).
__device__ __forceinline__ int request_of(const int32_t* cu, int nreq, int tok) {
  int lo = 0, hi = nreq;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= tok) lo = mid;
    else hi = mid;
  }
  return lo;
}

// Weight of one score from the row statistics, and u = sqrt(p) for entmax.
template <int NORM>
__device__ __forceinline__ float weight(float s, float st0, float st1, float& u) {
  if (NORM == ATTN_SOFTMAX || NORM == ATTN_SOFTMAX1) {
    u = 0.f;
    return expf(s - st0) / st1;
  }
  const float z = NORM == ATTN_ENTMAX15 ? 0.5f * s : s;
  const float d = z - st0;
  u = d > 0.f ? d : 0.f;
  return NORM == ATTN_ENTMAX15 ? u * u : u;
}

template <typename T>
__device__ __forceinline__ float dot_row(const float* x_lds, const T* y, int D) {
  float acc = 0.f;
  for (int d = 0; d < D; ++d) acc = fmaf(x_lds[d], to_f32(y[d]), acc);
  return acc;
}

// score s and ds/draw of one raw product
__device__ __forceinline__ float score(const FwdArgs& a, float raw, float& dsdraw) {
  if (a.softcap > 0.f) {
    const float t = tanhf(raw * a.scaling / a.softcap);
    dsdraw = a.scaling * (1.f - t * t);
    return a.softcap * t;
  }
  dsdraw = a.scaling;
  return raw * a.scaling;
}

template <typename T, int NORM>
__global__ __launch_bounds__(64) void bwd_query_kernel(BwdArgs w) {
  const FwdArgs& a = w.f;
  __shared__ float qs[kMaxD], dos[kMaxD], dsv[64];
  __shared__ unsigned kb_bits[kMaxBlocks / 32];  // block mask: listed key blocks of this row
  const int64_t row = blockIdx.x;  // ((b * Hq) + h) * Lq + i; packed: h * Lq + token
  const int lane = threadIdx.x, D = a.D;
  int b = 0, h, i, tok, nq, live, key0 = 0;
  bool inside = true;
  if (!a.cu_q) {
    i = (int)(row % a.Lq);
    const int64_t bh = row / a.Lq;
    h = (int)(bh % a.Hq);
    b = (int)(bh / a.Hq);
    tok = i;
    nq = a.Lq;
    live = a.Lk;
  } else {
    tok = (int)(row % a.Lq);
    h = (int)(row / a.Lq);
    i = nq = live = 0;
    inside = a.B > 0;
    if (inside) {
      b = request_of(a.cu_q, a.B, tok);
      int q0, q1, k0, k1;
      varlen_ranges(a, b, q0, q1, k0, k1);
      inside = tok >= q0 && tok < q1;
      i = tok - q0;
      nq = q1 - q0;
      live = k1 - k0;
      key0 = k0;
    }
  }
  const int kvh = h / a.G;
  const int64_t ba = a.cu_q ? 0 : b;  // batch index of the arrays
  T* dqrow = (T*)w.dq + ba * w.dq_sb + (int64_t)h * w.dq_sh + (int64_t)tok * w.dq_sl;
  if (!inside) {  // token outside every request: zero gradient, no sink term
    for (int d = lane; d < D; d += 64) dqrow[d] = from_f32<T>(0.f);
    if (lane == 0) {
      w.crow[row] = 0.f;
      if (NORM == ATTN_SOFTMAX1 && w.dsinks) w.srow[row] = 0.f;
    }
    return;
  }
  const T* qrow = (const T*)a.q + ba * a.q_sb + (int64_t)h * a.q_sh + (int64_t)tok * a.q_sl;
  const T* dorow = (const T*)w.dout + ba * w.do_sb + (int64_t)h * w.do_sh + (int64_t)tok * w.do_sl;
  for (int d = lane; d < D; d += 64) {
    qs[d] = to_f32(qrow[d]);
    dos[d] = to_f32(dorow[d]);
  }
  const T* kb = (const T*)a.k + ba * a.k_sb + (int64_t)kvh * a.k_sh + (int64_t)key0 * a.k_sl;
  const T* vb = (const T*)a.v + ba * a.v_sb + (int64_t)kvh * a.v_sh + (int64_t)key0 * a.v_sl;
  int lo, hi;
  key_range(i, nq, live, a.causal, a.window, lo, hi);
  const float st0 = a.stats[row * 2], st1 = a.stats[row * 2 + 1];

  // block mask: a bitmap of the key blocks listed for this row's query block
  const bool bm = a.bm_num != nullptr;
  if (bm) {
    const int nkb = (live + a.bm_bk - 1) / a.bm_bk;
    for (int x = lane; x < (nkb + 31) / 32; x += 64) kb_bits[x] = 0u;
    __syncthreads();
    int n;
    const int32_t* list = a.bm_idx + bm_list(a, b, h, i / a.bm_bq, n);
    for (int e = lane; e < n; e += 64)
      if (bm_entry_ok(list, e, nkb)) atomicOr(&kb_bits[list[e] >> 5], 1u << (list[e] & 31));
  }
  __syncthreads();
  auto allowed = [&](int j) -> bool {
    if (!bm) return true;
    const int c = j / a.bm_bk;
    return (kb_bits[c >> 5] >> (c & 31)) & 1u;
  };

  // pass 1: the row constant of the Jacobian
  float c1 = 0.f, c2 = 0.f;
  for (int j = lo + lane; j < hi; j += 64) {
    if (!allowed(j)) continue;
    float dsdraw, u;
    const float s = score(a, dot_row(qs, kb + (int64_t)j * a.k_sl, D), dsdraw);
    const float p = weight<NORM>(s, st0, st1, u);
    const float dP = dot_row(dos, vb + (int64_t)j * a.v_sl, D);
    if (NORM == ATTN_SOFTMAX || NORM == ATTN_SOFTMAX1) {
      c1 += p * dP;
    } else if (NORM == ATTN_SPARSEMAX) {
      if (p > 0.f) { c1 += dP; c2 += 1.f; }
    } else {
      c1 += u * dP;
      c2 += u;
    }
  }
  c1 = wave_sum(c1);
  c2 = wave_sum(c2);
  const float c = (NORM == ATTN_SOFTMAX || NORM == ATTN_SOFTMAX1) ? c1 : (c2 > 0.f ? c1 / c2 : 0.f);
  if (lane == 0) {
    w.crow[row] = c;
    if (NORM == ATTN_SOFTMAX1 && w.dsinks) {
      const float sink = a.sinks ? a.sinks[h] : 0.f;
      w.srow[row] = -expf(sink - st0) / st1 * c;  // empty rows: c = 0
    }
  }

  // pass 2: dQ
  float acc[kMaxD / 64];
#pragma unroll
  for (int t = 0; t < kMaxD / 64; ++t) acc[t] = 0.f;
  for (int base = lo; base < hi; base += 64) {
    const int j = base + lane;
    float draw = 0.f;
    if (j < hi && allowed(j)) {
      float dsdraw, u;
      const float s = score(a, dot_row(qs, kb + (int64_t)j * a.k_sl, D), dsdraw);
      const float p = weight<NORM>(s, st0, st1, u);
      const float dP = dot_row(dos, vb + (int64_t)j * a.v_sl, D);
      float ds;
      if (NORM == ATTN_SOFTMAX || NORM == ATTN_SOFTMAX1) ds = p * (dP - c);
      else if (NORM == ATTN_SPARSEMAX) ds = p > 0.f ? dP - c : 0.f;
      else ds = u * (dP - c);
      draw = ds * dsdraw;
    }
    dsv[lane] = draw;
    __syncthreads();
    const int n = min(64, hi - base);
    for (int jj = 0; jj < n; ++jj) {
      const float g = dsv[jj];
      if (g != 0.f) {
        const T* kp = kb + (int64_t)(base + jj) * a.k_sl;
#pragma unroll
        for (int t = 0; t < kMaxD / 64; ++t) {
          const int d = lane + 64 * t;
          if (d < D) acc[t] = fmaf(g, to_f32(kp[d]), acc[t]);
        }
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int t = 0; t < kMaxD / 64; ++t) {
    const int d = lane + 64 * t;
    if (d < D) dqrow[d] = from_f32<T>(acc[t]);
  }
}

// Query rows [ilo, ihi) that see key j (inverse of key_range).
__device__ __forceinline__ void query_range(int j, int lq, int lk, int causal, int window, int& ilo,
                                            int& ihi) {
  const int off = lk - lq;  // query i sits at key position i + off
  ilo = causal ? max(0, j - off) : 0;
  ihi = window ? min(lq, j - off + window) : lq;
  ihi = max(ihi, ilo);
}

template <typename T, int NORM>
__global__ __launch_bounds__(64) void bwd_key_kernel(BwdArgs w) {
  const FwdArgs& a = w.f;
  __shared__ float ks[kMaxD], vs[kMaxD], pv[64], gv[64];
  __shared__ unsigned qb_bits[kMaxBlocks / 32];  // block mask: query blocks that list this key's block
  const int64_t krow = blockIdx.x;  // ((b * Hkv) + kvh) * Lk + j; packed: kvh * Lk + token
  const int lane = threadIdx.x, D = a.D;
  int b = 0, kvh, j, tok, nq, live, qtok0 = 0;
  bool inside = true;
  if (!a.cu_q) {
    j = (int)(krow % a.Lk);
    const int64_t bk = krow / a.Lk;
    kvh = (int)(bk % a.Hkv);
    b = (int)(bk / a.Hkv);
    tok = j;
    nq = a.Lq;
    live = a.Lk;
  } else {
    tok = (int)(krow % a.Lk);
    kvh = (int)(krow / a.Lk);
    j = nq = live = 0;
    inside = a.B > 0;
    if (inside) {
      b = request_of(a.cu_k, a.B, tok);
      int q0, q1, k0, k1;
      varlen_ranges(a, b, q0, q1, k0, k1);
      inside = tok >= k0 && tok < k1;
      j = tok - k0;
      nq = q1 - q0;
      live = k1 - k0;
      qtok0 = q0;
    }
  }
  const int64_t ba = a.cu_q ? 0 : b;  // batch index of the arrays
  T* dkr = (T*)w.dk + ba * w.dk_sb + (int64_t)kvh * w.dk_sh + (int64_t)tok * w.dk_sl;
  T* dvr = (T*)w.dv + ba * w.dv_sb + (int64_t)kvh * w.dv_sh + (int64_t)tok * w.dv_sl;
  if (!inside) {  // token outside every request: zero gradients
    for (int d = lane; d < D; d += 64) {
      dkr[d] = from_f32<T>(0.f);
      dvr[d] = from_f32<T>(0.f);
    }
    return;
  }
  const T* kp = (const T*)a.k + ba * a.k_sb + (int64_t)kvh * a.k_sh + (int64_t)tok * a.k_sl;
  const T* vp = (const T*)a.v + ba * a.v_sb + (int64_t)kvh * a.v_sh + (int64_t)tok * a.v_sl;
  for (int d = lane; d < D; d += 64) {
    ks[d] = to_f32(kp[d]);
    vs[d] = to_f32(vp[d]);
  }
  __syncthreads();
  int ilo, ihi;
  query_range(j, nq, live, a.causal, a.window, ilo, ihi);
  const bool bm = a.bm_num != nullptr;
  float ak[kMaxD / 64], av[kMaxD / 64];
#pragma unroll
  for (int t = 0; t < kMaxD / 64; ++t) ak[t] = av[t] = 0.f;
  for (int hh = 0; hh < a.G; ++hh) {
    const int h = kvh * a.G + hh;
    const T* qb = (const T*)a.q + ba * a.q_sb + (int64_t)h * a.q_sh + (int64_t)qtok0 * a.q_sl;
    const T* dob = (const T*)w.dout + ba * w.do_sb + (int64_t)h * w.do_sh + (int64_t)qtok0 * w.do_sl;
    const int64_t row0 = (ba * a.Hq + h) * a.Lq + qtok0;
    // block mask: bit r set when query block r of head h lists key j's block
    // (rebuilt per head unless the mask is shared by all heads)
    if (bm && ihi > ilo && (hh == 0 || a.bm_heads != 1)) {
      const int kbj = j / a.bm_bk, nkb = (live + a.bm_bk - 1) / a.bm_bk;
      const int r0 = ilo / a.bm_bq, r1 = (ihi - 1) / a.bm_bq + 1;
      __syncthreads();  // the previous head's readers are done
      for (int x = (r0 >> 5) + lane; x < (r1 + 31) >> 5; x += 64) qb_bits[x] = 0u;
      __syncthreads();
      for (int r = r0 + lane; r < r1; r += 64) {
        int n;
        const int32_t* list = a.bm_idx + bm_list(a, b, h, r, n);
        bool hit = false;
        for (int e = 0; e < n; ++e) hit |= list[e] == kbj && bm_entry_ok(list, e, nkb);
        if (hit) atomicOr(&qb_bits[r >> 5], 1u << (r & 31));
      }
      __syncthreads();
    }
    for (int base = ilo; base < ihi; base += 64) {
      const int i = base + lane;
      float p = 0.f, g = 0.f;
      const bool on = i < ihi && (!bm || ((qb_bits[(i / a.bm_bq) >> 5] >> ((i / a.bm_bq) & 31)) & 1u));
      if (on) {
        const float st0 = a.stats[(row0 + i) * 2], st1 = a.stats[(row0 + i) * 2 + 1];
        float raw = 0.f, dP = 0.f;
        const T* qr = qb + (int64_t)i * a.q_sl;
        const T* dr = dob + (int64_t)i * w.do_sl;
        for (int d = 0; d < D; ++d) {
          raw = fmaf(to_f32(qr[d]), ks[d], raw);
          dP = fmaf(to_f32(dr[d]), vs[d], dP);
        }
        float dsdraw, u;
        const float s = score(a, raw, dsdraw);
        p = weight<NORM>(s, st0, st1, u);
        const float c = w.crow[row0 + i];
        float ds;
        if (NORM == ATTN_SOFTMAX || NORM == ATTN_SOFTMAX1) ds = p * (dP - c);
        else if (NORM == ATTN_SPARSEMAX) ds = p > 0.f ? dP - c : 0.f;
        else ds = u * (dP - c);
        g = ds * dsdraw;
      }
      pv[lane] = p;
      gv[lane] = g;
      __syncthreads();
      const int n = min(64, ihi - base);
      for (int ii = 0; ii < n; ++ii) {
        const float pi = pv[ii], gi = gv[ii];
        if (pi != 0.f || gi != 0.f) {
          const T* qr = qb + (int64_t)(base + ii) * a.q_sl;
          const T* dr = dob + (int64_t)(base + ii) * w.do_sl;
#pragma unroll
          for (int t = 0; t < kMaxD / 64; ++t) {
            const int d = lane + 64 * t;
            if (d < D) {
              av[t] = fmaf(pi, to_f32(dr[d]), av[t]);
              ak[t] = fmaf(gi, to_f32(qr[d]), ak[t]);
            }
          }
        }
      }
      __syncthreads();
    }
  }
#pragma unroll
  for (int t = 0; t < kMaxD / 64; ++t) {
    const int d = lane + 64 * t;
    if (d < D) {
      dkr[d] = from_f32<T>(ak[t]);
      dvr[d] = from_f32<T>(av[t]);
    }
  }
}

// d b_h = sum over the head's rows (b, i) of -p_sink c (fixed order).
__global__ __launch_bounds__(64) void bwd_sink_kernel(BwdArgs w) {
  const FwdArgs& a = w.f;
  const int h = blockIdx.x, lane = threadIdx.x;
  float s = 0.f;
  const int nb = a.cu_q ? 1 : a.B;  // packed: one row array over all requests
  for (int b = 0; b < nb; ++b) {
    const int64_t row0 = ((int64_t)b * a.Hq + h) * a.Lq;
    for (int i = lane; i < a.Lq; i += 64) s += w.srow[row0 + i];
  }
  s = wave_sum(s);
  if (lane == 0) w.dsinks[h] = s;
}

hipError_t launch_bwd_sinks(const BwdArgs& w, hipStream_t stream) {
  bwd_sink_kernel<<<dim3((unsigned)w.f.Hq), dim3(64), 0, stream>>>(w);
  return hipGetLastError();
}

template <typename T, int NORM>
hipError_t launch_norm(const BwdArgs& w, hipStream_t stream) {
  const FwdArgs& a = w.f;
  const int64_t nb = a.cu_q ? 1 : a.B;  // packed: [1, H, tokens] arrays
  const int64_t qrows = nb * a.Hq * a.Lq, krows = nb * a.Hkv * a.Lk;
  if (qrows) bwd_query_kernel<T, NORM><<<dim3((unsigned)qrows), dim3(64), 0, stream>>>(w);
  if (krows) bwd_key_kernel<T, NORM><<<dim3((unsigned)krows), dim3(64), 0, stream>>>(w);
  if (NORM == ATTN_SOFTMAX1 && w.dsinks && a.Hq)
    bwd_sink_kernel<<<dim3((unsigned)a.Hq), dim3(64), 0, stream>>>(w);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const BwdArgs& w, hipStream_t stream) {
  switch (w.f.norm) {
    case ATTN_SOFTMAX: return launch_norm<T, ATTN_SOFTMAX>(w, stream);
    case ATTN_SOFTMAX1: return launch_norm<T, ATTN_SOFTMAX1>(w, stream);
    case ATTN_SPARSEMAX: return launch_norm<T, ATTN_SPARSEMAX>(w, stream);
    default: return launch_norm<T, ATTN_ENTMAX15>(w, stream);
  }
}

}  // namespace
}  // namespace attn

using namespace attn;

// C ABI entry points (declared in attn.h); validation shares the forward's.
namespace attn {
int validate_fwd_args(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
                      const attn_params* p, FwdArgs* a, bool need_data);
int bwd_fail(int status, const char* msg);
}  // namespace attn

static int same_shape(const attn_tensor* a, const attn_tensor* b) {
  for (int d = 0; d < 4; ++d)
    if (a->shape[d] != b->shape[d]) return 0;
  return a->dtype == b->dtype;
}

static int bwd_prepare(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
                       const attn_tensor* out, const attn_tensor* dout, const float* row_stats,
                       const attn_params* p,
                       const attn_tensor* dq, const attn_tensor* dk, const attn_tensor* dv,
                       BwdArgs* w, bool need_data) {
  memset(w, 0, sizeof(*w));
  int st = validate_fwd_args(q, k, v, p, &w->f, need_data);
  if (st) return st;
  // block masks: the key kernel keeps a bitmap of query blocks in LDS (the
  // forward's validation bounds the key blocks the same way)
  if (w->f.bm_num && (w->f.Lq + w->f.bm_bq - 1) / w->f.bm_bq > kMaxBlocks)
    return bwd_fail(ATTN_E_UNSUPPORTED, "block mask has more than 16384 query blocks");
  if (!dout || !dq || !dk || !dv) return bwd_fail(ATTN_E_INVALID, "dout, dq, dk or dv descriptor is NULL");
  if (!same_shape(dout, q) || !same_shape(dq, q))
    return bwd_fail(ATTN_E_INVALID, "dout and dq must match q in shape and dtype");
  if (out) {
    if (!same_shape(out, q)) return bwd_fail(ATTN_E_INVALID, "out must match q in shape and dtype");
    if (out->stride[3] != 1) return bwd_fail(ATTN_E_INVALID, "out needs a contiguous last dimension");
    for (int d = 0; d < 4; ++d)
      if (out->stride[d] < 0) return bwd_fail(ATTN_E_INVALID, "out has a negative stride");
    if (need_data && !out->data && out->shape[0] * out->shape[1] * out->shape[2] * out->shape[3] != 0)
      return bwd_fail(ATTN_E_INVALID, "out data pointer is NULL");
  }
  if (!same_shape(dk, k) || !same_shape(dv, v))
    return bwd_fail(ATTN_E_INVALID, "dk and dv must match k and v in shape and dtype");
  const attn_tensor* ts[] = {dout, dq, dk, dv};
  for (const attn_tensor* t : ts) {
    if (t->stride[3] != 1) return bwd_fail(ATTN_E_INVALID, "gradient tensors need a contiguous last dimension");
    for (int d = 0; d < 4; ++d)
      if (t->stride[d] < 0) return bwd_fail(ATTN_E_INVALID, "gradient tensors have a negative stride");
    if (need_data && !t->data && t->shape[0] * t->shape[1] * t->shape[2] * t->shape[3] != 0)
      return bwd_fail(ATTN_E_INVALID, "a gradient data pointer is NULL");
  }
  if (need_data && !row_stats) return bwd_fail(ATTN_E_INVALID, "row_stats of the forward are required");
  w->dout = dout->data;
  w->dq = dq->data;
  w->dk = dk->data;
  w->dv = dv->data;
  w->do_sb = dout->stride[0]; w->do_sh = dout->stride[1]; w->do_sl = dout->stride[2];
  w->dq_sb = dq->stride[0]; w->dq_sh = dq->stride[1]; w->dq_sl = dq->stride[2];
  w->dk_sb = dk->stride[0]; w->dk_sh = dk->stride[1]; w->dk_sl = dk->stride[2];
  w->dv_sb = dv->stride[0]; w->dv_sh = dv->stride[1]; w->dv_sl = dv->stride[2];
  w->f.stats = (float*)row_stats;
  w->have_out = out != nullptr;
  if (out) {
    w->f.out = out->data;
    w->f.o_sb = out->stride[0]; w->f.o_sh = out->stride[1]; w->f.o_sl = out->stride[2];
  }
  return ATTN_OK;
}

// Per-row path: c_i and the sink term per query row.  Matrix-core path: the
// record blocks, the sink term per query row, then (G > 1) the fp32 partial
// dK / dV of every query head.
// byte offset of the partials: 256-byte aligned (16-byte vector accesses)
static size_t bwd_part_offset(const FwdArgs& a) {
  const size_t rows = (size_t)a.B * a.Hq * a.Lq;
  return (bwd_mfma_rec_bytes(a) + rows * sizeof(float) + 255) / 256 * 256;
}

static size_t bwd_workspace(const FwdArgs& a) {
  const size_t rows = (size_t)a.B * a.Hq * a.Lq;
  return std::max(rows * 2 * sizeof(float), bwd_part_offset(a) + bwd_mfma_part_bytes(a));
}

extern "C" int attn_bwd(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
                        const attn_tensor* out, const attn_tensor* dout, const float* row_stats,
                        const attn_params* p, const attn_tensor* dq, const attn_tensor* dk,
                        const attn_tensor* dv, float* dsinks, void* workspace,
                        size_t workspace_bytes, void* stream) {
  BwdArgs w;
  int st = bwd_prepare(q, k, v, out, dout, row_stats, p, dq, dk, dv, &w, true);
  if (st) return st;
  if (dsinks && w.f.norm != ATTN_SOFTMAX1)
    return bwd_fail(ATTN_E_INVALID, "sink gradients apply to softmax1 only");
  const size_t need = bwd_workspace(w.f);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return bwd_fail(ATTN_E_WORKSPACE, "workspace smaller than attn_bwd_workspace_bytes()");
  w.dsinks = dsinks;
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  hipError_t e;
  if (bwd_mfma_supported(w)) {
    w.rec = (float*)workspace;
    w.rec_bytes = bwd_mfma_rec_bytes(w.f);
    w.srow = (float*)((char*)workspace + w.rec_bytes);
    w.part = (float*)((char*)workspace + bwd_part_offset(w.f));
    w.key_split = bwd_key_split(w.f) ? 1 : 0;
    e = launch_bwd_mfma(w, s);
    if (e == hipSuccess && w.dsinks && w.f.Hq)
      e = launch_bwd_sinks(w, s);
  } else {
    w.crow = (float*)workspace;
    w.srow = w.crow + (size_t)w.f.B * w.f.Hq * w.f.Lq;
    e = w.f.dtype == ATTN_BF16 ? launch_t<bf16_t>(w, s) : launch_t<float>(w, s);
  }
  if (e != hipSuccess) return bwd_fail(ATTN_E_LAUNCH, "HIP launch failed");
  return ATTN_OK;
}

extern "C" int attn_bwd_varlen(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
                               const attn_tensor* out, const attn_tensor* dout,
                               const float* row_stats, const attn_varlen* varlen,
                               const attn_params* p, const attn_tensor* dq, const attn_tensor* dk,
                               const attn_tensor* dv, float* dsinks, void* workspace,
                               size_t workspace_bytes, void* stream) {
  BwdArgs w;
  int st = bwd_prepare(q, k, v, out, dout, row_stats, p, dq, dk, dv, &w, true);
  if (st) return st;
  if (!varlen) return bwd_fail(ATTN_E_INVALID, "varlen descriptor is NULL");
  if (w.f.bm_num) return bwd_fail(ATTN_E_UNSUPPORTED, "block masks apply to a padded batch only");
  if (q->shape[0] != 1 || k->shape[0] != 1)
    return bwd_fail(ATTN_E_INVALID, "packed q, k, v must have batch extent 1");
  if (varlen->num_seqs < 0 || varlen->max_seqlen_q < 0)
    return bwd_fail(ATTN_E_INVALID, "num_seqs and max_seqlen_q must be >= 0");
  if (varlen->num_seqs > 0 && (!varlen->cu_seqlens_q || !varlen->cu_seqlens_k))
    return bwd_fail(ATTN_E_INVALID, "cu_seqlens_q or cu_seqlens_k is NULL");
  if (dsinks && w.f.norm != ATTN_SOFTMAX1)
    return bwd_fail(ATTN_E_INVALID, "sink gradients apply to softmax1 only");
  const size_t need = (size_t)w.f.Hq * w.f.Lq * 2 * sizeof(float);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return bwd_fail(ATTN_E_WORKSPACE, "workspace smaller than 8 bytes per query head and token");
  // The kernels tell a packed batch by a non-NULL cu_q; with no requests the
  // arrays are never read (every token lies outside and gets zeros), so any
  // non-NULL address stands in.
  static const int32_t no_requests[2] = {0, 0};
  w.f.cu_q = varlen->num_seqs > 0 ? varlen->cu_seqlens_q : no_requests;
  w.f.cu_k = varlen->num_seqs > 0 ? varlen->cu_seqlens_k : no_requests;
  w.f.B = varlen->num_seqs;
  w.f.max_q = varlen->max_seqlen_q;
  w.dsinks = dsinks;
  w.crow = (float*)workspace;
  w.srow = w.crow + (size_t)w.f.Hq * w.f.Lq;
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  const hipError_t e = w.f.dtype == ATTN_BF16 ? launch_t<bf16_t>(w, s) : launch_t<float>(w, s);
  if (e != hipSuccess) return bwd_fail(ATTN_E_LAUNCH, "HIP launch failed");
  return ATTN_OK;
}

extern "C" int attn_bwd_path(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
                             const attn_tensor* out, const attn_tensor* dout, const attn_params* p,
                             const attn_tensor* dq, const attn_tensor* dk, const attn_tensor* dv,
                             int* path) {
  if (!path) return bwd_fail(ATTN_E_INVALID, "path pointer is NULL");
  BwdArgs w;
  int st = bwd_prepare(q, k, v, out, dout, nullptr, p, dq, dk, dv, &w, false);
  if (st) return st;
  if ((int64_t)w.f.B * w.f.Hq * w.f.Lq == 0 && (int64_t)w.f.B * w.f.Hkv * w.f.Lk == 0)
    *path = ATTN_PATH_NONE;
  else
    *path = bwd_mfma_supported(w) ? ATTN_PATH_BWD_MFMA : ATTN_PATH_BWD_PER_ROW;
  return ATTN_OK;
}

extern "C" int attn_bwd_workspace_bytes(const attn_tensor* q, const attn_tensor* k,
                                        const attn_tensor* v, const attn_params* p, size_t* bytes) {
  if (!bytes) return bwd_fail(ATTN_E_INVALID, "bytes is NULL");
  FwdArgs a;
  int st = validate_fwd_args(q, k, v, p, &a, false);
  if (st) return st;
  *bytes = bwd_workspace(a);
  return ATTN_OK;
}
