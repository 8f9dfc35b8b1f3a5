// Internal definitions shared by the libattn kernels and the host dispatcher.
// Not part of the public ABI (see include/attn.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn.h"

namespace attn {

// Everything a kernel needs, validated and flattened by the dispatcher.
// Strides are in elements.  For contiguous K/V: (sb, sh, sl) = strides of the
// batch, head and token dimensions.  For a paged cache [NB, bs, Hkv, D]:
// sb = page stride, sl = slot stride, sh = head stride.
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* stats;
  int64_t q_sb, q_sh, q_sl;
  int64_t k_sb, k_sh, k_sl;
  int64_t v_sb, v_sh, v_sl;
  int64_t o_sb, o_sh, o_sl;
  int dtype;  // attn_dtype of q, k, v and out
  int B, Hq, Hkv, G, Lq, Lk, D;
  int paged;
  const int32_t* block_table;
  const int32_t* seq_lens;
  int block_size, max_blocks;
  int num_blocks;  // pages in each paged cache (page indices are clamped to it)
  int norm, causal, window;
  float softcap, scaling;
  const float* sinks;  // softmax1: per query head logit of the virtual key (NULL = 0)
  // packed variable-length batch (cu_q != nullptr): B = number of requests,
  // Lq / Lk = packed token counts, max_q bounds every request's query count
  const int32_t* cu_q;
  const int32_t* cu_k;
  int max_q;
  // block-sparse key mask (bm_num != nullptr): counts [B, bm_heads, nqb] and
  // ascending key-block lists [B, bm_heads, nqb, bm_max], blocks bm_bq x bm_bk
  const int32_t* bm_num;
  const int32_t* bm_idx;
  int bm_bq, bm_bk, bm_heads, bm_max;
};

// Key-block list of query block r of (b, h) under a block mask: entries e of
// bm_idx + list_off(...), count clamped to [0, bm_max].
__device__ __forceinline__ int64_t bm_list(const FwdArgs& a, int b, int h, int r, int& n) {
  const int hm = a.bm_heads == 1 ? 0 : h;
  const int nqb = (a.Lq + a.bm_bq - 1) / a.bm_bq;
  const int64_t cell = ((int64_t)b * a.bm_heads + hm) * nqb + r;
  n = min(max(a.bm_num[cell], 0), a.bm_max);
  return cell * a.bm_max;
}
// Entry e of a list is used when it lies in [0, nkb) and above its predecessor.
__device__ __forceinline__ bool bm_entry_ok(const int32_t* list, int e, int nkb) {
  const int v = list[e];
  return v >= 0 && v < nkb && (e == 0 || v > list[e - 1]);
}

// Query/key token ranges of packed request r, clamped into the packed arrays.
__device__ __forceinline__ void varlen_ranges(const FwdArgs& a, int r, int& q0, int& q1, int& k0,
                                              int& k1) {
  q0 = min(max(a.cu_q[r], 0), a.Lq);
  q1 = min(max(a.cu_q[r + 1], q0), a.Lq);
  k0 = min(max(a.cu_k[r], 0), a.Lk);
  k1 = min(max(a.cu_k[r + 1], k0), a.Lk);
}

typedef __bf16 bf16_t;

// Paged caches: live keys of sequence b (clamped to the table's reach; none
// when the cache has no pages) and a block-table entry clamped into the
// cache, so a bad entry yields wrong values instead of a stray access.
__device__ __forceinline__ int paged_live(const FwdArgs& a, int b) {
  return a.num_blocks > 0 ? max(0, min(a.seq_lens[b], a.max_blocks * a.block_size)) : 0;
}
__device__ __forceinline__ int64_t page_of(const int32_t* table_row, int idx, int num_blocks) {
  return (int64_t)min(max(table_row[idx], 0), num_blocks - 1);
}

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return (float)x; }

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) { return (bf16_t)x; }  // RNE

// Wave64 reductions through cross-lane shuffles.
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ float wave_min(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fminf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}
__device__ __forceinline__ double wave_sum(double x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}
__device__ __forceinline__ int wave_sum(int x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// Visible key interval [lo, hi) of query row i when `live` keys exist:
// bottom-right aligned causal bound and sliding window.
__device__ __forceinline__ void key_range(int i, int lq, int live, int causal, int window,
                                          int& lo, int& hi) {
  const int qp = i + live - lq;
  int h = causal ? min(live, qp + 1) : live;
  h = max(h, 0);
  int l = window ? max(0, qp - window + 1) : 0;
  lo = min(l, h);
  hi = h;
}

// Arguments of the backward: the forward's (with row_stats in f.stats), the
// upstream gradient, the three gradients (strides in elements) and the
// workspace rows.
struct BwdArgs {
  FwdArgs f;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  int64_t do_sb, do_sh, do_sl;
  int64_t dq_sb, dq_sh, dq_sl;
  int64_t dk_sb, dk_sh, dk_sl;
  int64_t dv_sb, dv_sh, dv_sl;
  float* dsinks;
  float* crow;   // workspace: c_i per query row (per-row kernels)
  float* srow;   // workspace: -p_sink,i c_i per query row (softmax1 with sinks)
  float* rec;    // workspace: per-row records of the matrix-core kernels
  size_t rec_bytes;
  int have_out;  // f.out / f.o_* hold the forward's output
  float* part;   // workspace: fp32 partial dK then dV per query head [B, Hq, Lk, D]
  int key_split; // key kernel: one query head per workgroup, partials in `part`
};

// Launchers, one per kernel family (defined in their own translation units).
hipError_t launch_generic(const FwdArgs& a, hipStream_t stream);
hipError_t launch_prefill_mfma(const FwdArgs& a, hipStream_t stream);
// Matrix-core backward (bf16, D = 64, 128 or 256, contiguous K/V): query kernel
// (row constants, records, dQ) then key kernel (dK, dV).
bool bwd_mfma_supported(const BwdArgs& w);
size_t bwd_mfma_rec_bytes(const FwdArgs& a);
size_t bwd_mfma_part_bytes(const FwdArgs& a);
bool bwd_key_split(const FwdArgs& a);
hipError_t launch_bwd_mfma(const BwdArgs& w, hipStream_t stream);
hipError_t launch_decode(const FwdArgs& a, void* workspace, hipStream_t stream);
size_t decode_workspace_bytes(const FwdArgs& a);
bool prefill_mfma_supported(const FwdArgs& a);
bool decode_supported(const FwdArgs& a);

}  // namespace attn
