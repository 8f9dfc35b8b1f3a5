// Per-row attention forward: one wave64 per query row, fp32 arithmetic.
//
// Covers every case the ABI accepts (f32 or bf16 inputs, any head dim up to
// 256, contiguous or paged K/V, every normalizer and mask).  It is the path
// for f32 inputs and for shapes the tiled matrix-core kernels do not cover.
//
// Scores are recomputed in every pass instead of being stored, so the kernel
// needs no workspace:
//   pass 1        row max of z (z = s, or s/2 for entmax15)
//   softmax(1)    one pass: weights exp(z - m) and the weighted sum of V
//   sparse        threshold passes, then one pass for the weighted sum of V.
// The threshold passes solve sum_j g(z_j - tau) = 1 (g(x) = x+ for
// sparsemax, x+^2 for 1.5-entmax; "HF Attention Normalizers", "Supported
// Normalizers" and "Important Limitations": one threshold per row).  Each
// pass collects, over the candidate set L = {z > t} of a proven lower bound
// t <= tau, the count, sum and sum of squares (shifted by the row max) and
// the smallest member.  tau is the closed form over L (sparsemax:
// (sum - 1)/|L|; entmax15: mean - sqrt((1 - sum of squared deviations)/|L|))
// as soon as that value lies below every member of L (then L is exactly the
// support).  Otherwise t rises to a larger lower bound -- the Michelot /
// Newton step, which cannot pass tau because g is convex, or the smallest
// member of L when that is larger -- and at least one candidate leaves L,
// so the loop ends after at most |L| passes.

#include "common.h"

namespace attn {
namespace {

constexpr int kMaxD = 256;
constexpr int kMaxKeyBlocks = 16384;  // block masks: key blocks per row (bitmap in LDS)

template <typename T>
struct RowCtx {
  const FwdArgs& a;
  const T* kbase;      // contiguous: K of (b, kv head); paged: cache base + head offset
  const T* vbase;
  const int32_t* table;  // paged: this sequence's block-table row
  // key0: first key token of a packed request (0 otherwise)
  __device__ RowCtx(const FwdArgs& a_, int b, int kvh, int key0) : a(a_) {
    if (a.paged) {
      kbase = (const T*)a.k + (int64_t)kvh * a.k_sh;
      vbase = (const T*)a.v + (int64_t)kvh * a.v_sh;
      table = a.block_table + (int64_t)b * a.max_blocks;
    } else if (a.cu_q) {
      kbase = (const T*)a.k + (int64_t)key0 * a.k_sl + (int64_t)kvh * a.k_sh;
      vbase = (const T*)a.v + (int64_t)key0 * a.v_sl + (int64_t)kvh * a.v_sh;
      table = nullptr;
    } else {
      kbase = (const T*)a.k + (int64_t)b * a.k_sb + (int64_t)kvh * a.k_sh;
      vbase = (const T*)a.v + (int64_t)b * a.v_sb + (int64_t)kvh * a.v_sh;
      table = nullptr;
    }
  }
  __device__ const T* key(int j) const {
    if (a.paged) {
      const int64_t page = page_of(table, j / a.block_size, a.num_blocks);
      return kbase + page * a.k_sb + (int64_t)(j % a.block_size) * a.k_sl;
    }
    return kbase + (int64_t)j * a.k_sl;
  }
  __device__ const T* value(int j) const {
    if (a.paged) {
      const int64_t page = page_of(table, j / a.block_size, a.num_blocks);
      return vbase + page * a.v_sb + (int64_t)(j % a.block_size) * a.v_sl;
    }
    return vbase + (int64_t)j * a.v_sl;
  }
};

template <typename T, int NORM>
__global__ __launch_bounds__(64) void generic_fwd_kernel(FwdArgs a) {
  __shared__ float qs[kMaxD];
  __shared__ float ps[64];
  __shared__ unsigned kb_bits[kMaxKeyBlocks / 32];  // block mask: listed key blocks of this row

  const int64_t row = blockIdx.x;  // ((b * Hq) + h) * Lq + i; packed: h * Lq + token
  const int lane = threadIdx.x;
  const int D = a.D;
  int b, h, i, tok, nq, live, key0 = 0;
  if (!a.cu_q) {
    i = (int)(row % a.Lq);
    const int64_t bh = row / a.Lq;
    h = (int)(bh % a.Hq);
    b = (int)(bh / a.Hq);
    tok = i;
    nq = a.Lq;
    live = a.paged ? paged_live(a, b) : a.Lk;
  } else {
    // packed: the request holding this query token (binary search)
    tok = (int)(row % a.Lq);
    h = (int)(row / a.Lq);
    int lo_r = 0, hi_r = a.B;  // last r with cu_q[r] <= tok
    while (hi_r - lo_r > 1) {
      const int mid = (lo_r + hi_r) >> 1;
      if (a.cu_q[mid] <= tok) lo_r = mid;
      else hi_r = mid;
    }
    b = lo_r;
    int q0, q1, k0, k1;
    varlen_ranges(a, b, q0, q1, k0, k1);
    if (tok < q0 || tok >= q1) return;  // token outside every request: left unwritten
    i = tok - q0;
    nq = q1 - q0;
    live = k1 - k0;
    key0 = k0;
  }
  const int kvh = h / a.G;
  const int64_t bq = a.cu_q ? 0 : b;  // batch index of the q / out / stats arrays

  const T* qrow = (const T*)a.q + bq * a.q_sb + (int64_t)h * a.q_sh + (int64_t)tok * a.q_sl;
  for (int d = lane; d < D; d += 64) qs[d] = to_f32(qrow[d]);
  __syncthreads();

  int lo, hi;
  key_range(i, nq, live, a.causal, a.window, lo, hi);

  // block mask: a bitmap of the key blocks listed for this row's query block
  const bool bm = a.bm_num != nullptr;
  if (bm) {
    const int nkb = (live + a.bm_bk - 1) / a.bm_bk;
    for (int w = lane; w < (nkb + 31) / 32; w += 64) kb_bits[w] = 0u;
    __syncthreads();
    int n;
    const int32_t* list = a.bm_idx + bm_list(a, b, h, i / a.bm_bq, n);
    for (int e = lane; e < n; e += 64)
      if (bm_entry_ok(list, e, nkb)) atomicOr(&kb_bits[list[e] >> 5], 1u << (list[e] & 31));
    __syncthreads();
  }
  auto allowed = [&](int j) -> bool {
    if (!bm) return true;
    const int c = j / a.bm_bk;
    return (kb_bits[c >> 5] >> (c & 31)) & 1u;
  };

  RowCtx<T> ctx(a, b, kvh, key0);
  const bool entmax = (NORM == ATTN_ENTMAX15);
  auto zval = [&](int j) -> float {
    const T* kp = ctx.key(j);
    float acc = 0.f;
    for (int d = 0; d < D; ++d) acc = fmaf(qs[d], to_f32(kp[d]), acc);
    float s = acc * a.scaling;
    if (a.softcap > 0.f) s = a.softcap * tanhf(s / a.softcap);
    return entmax ? 0.5f * s : s;
  };

  T* orow = (T*)a.out + bq * a.o_sb + (int64_t)h * a.o_sh + (int64_t)tok * a.o_sl;
  float* srow = a.stats ? a.stats + row * 2 : nullptr;

  // softmax1: logit of the virtual key (0, or the head's learned sink)
  const float sink = (NORM == ATTN_SOFTMAX1 && a.sinks) ? a.sinks[h] : 0.f;
  auto write_empty = [&]() {  // a row without keys
    for (int d = lane; d < D; d += 64) orow[d] = from_f32<T>(0.f);
    if (srow && lane == 0) {
      srow[0] = NORM == ATTN_SOFTMAX ? -INFINITY : (NORM == ATTN_SOFTMAX1 ? sink : INFINITY);
      srow[1] = NORM == ATTN_SOFTMAX1 ? 1.f : 0.f;
    }
  };
  if (hi <= lo) {
    write_empty();
    return;
  }

  // pass 1: row max (scores are finite, so -inf means no allowed key)
  float m = -INFINITY;
  for (int j = lo + lane; j < hi; j += 64)
    if (allowed(j)) m = fmaxf(m, zval(j));
  m = wave_max(m);
  if (m == -INFINITY) {
    write_empty();
    return;
  }

  // Threshold search (sparse normalizers), in the shifted domain y = z - m.
  float tau_y = 0.f;
  int support = 0;
  if (NORM == ATTN_SPARSEMAX || NORM == ATTN_ENTMAX15) {
    double t = -1.0;  // tau >= m - 1: the top key alone already has weight >= 1 there
    for (int it = 0; it <= hi - lo + 1; ++it) {
      int cnt = 0;
      double s1 = 0.0, s2 = 0.0;
      float mn = INFINITY;
      for (int j = lo + lane; j < hi; j += 64) {
        if (!allowed(j)) continue;
        const float y = zval(j) - m;
        if ((double)y > t) {
          cnt += 1;
          s1 += y;
          s2 += (double)y * y;
          mn = fminf(mn, y);
        }
      }
      cnt = wave_sum(cnt);
      s1 = wave_sum(s1);
      s2 = wave_sum(s2);
      mn = wave_min(mn);
      const double c = (double)cnt;
      double tcf;
      bool valid;
      double step;
      if (NORM == ATTN_SPARSEMAX) {
        tcf = (s1 - 1.0) / c;
        valid = true;
        step = tcf;  // Michelot step: a lower bound on tau
      } else {
        const double mu = s1 / c;
        const double ss = s2 - s1 * mu;  // sum of squared deviations from the mean
        const double delta = (1.0 - ss) / c;
        valid = delta >= 0.0;
        tcf = valid ? mu - sqrt(delta) : 0.0;
        // Newton step on f(t) = sum (y - t)^2 - 1 over L, from the left
        const double f = s2 - 2.0 * t * s1 + c * t * t - 1.0;
        const double fp = 2.0 * (s1 - c * t);
        step = t + f / fp;
      }
      if (valid && tcf < (double)mn) {
        tau_y = (float)tcf;
        support = cnt;
        break;
      }
      t = fmax(step, (double)mn);
    }
  }

  // weighted sum of V
  float acc[kMaxD / 64];
#pragma unroll
  for (int c = 0; c < kMaxD / 64; ++c) acc[c] = 0.f;
  const float mref = (NORM == ATTN_SOFTMAX1) ? fmaxf(m, sink) : m;
  float lsum = 0.f;
  for (int base = lo; base < hi; base += 64) {
    const int j = base + lane;
    float p = 0.f;
    if (j < hi && allowed(j)) {
      const float z = zval(j);
      if (NORM == ATTN_SOFTMAX || NORM == ATTN_SOFTMAX1) {
        p = expf(z - mref);
      } else {
        const float d = (z - m) - tau_y;
        p = d > 0.f ? (NORM == ATTN_ENTMAX15 ? d * d : d) : 0.f;
      }
    }
    lsum += p;
    ps[lane] = p;
    __syncthreads();
    const int n = min(64, hi - base);
    for (int jj = 0; jj < n; ++jj) {
      const float pj = ps[jj];
      if (pj != 0.f) {
        const T* vp = ctx.value(base + jj);
#pragma unroll
        for (int c = 0; c < kMaxD / 64; ++c) {
          const int d = lane + 64 * c;
          if (d < D) acc[c] = fmaf(pj, to_f32(vp[d]), acc[c]);
        }
      }
    }
    __syncthreads();
  }

  float inv = 1.f;
  float st0, st1;
  if (NORM == ATTN_SOFTMAX || NORM == ATTN_SOFTMAX1) {
    float l = wave_sum(lsum);
    if (NORM == ATTN_SOFTMAX1) l += expf(sink - mref);
    inv = 1.f / l;
    st0 = mref;
    st1 = l;
  } else {
    st0 = m + tau_y;
    st1 = (float)support;
  }
#pragma unroll
  for (int c = 0; c < kMaxD / 64; ++c) {
    const int d = lane + 64 * c;
    if (d < D) orow[d] = from_f32<T>(acc[c] * inv);
  }
  if (srow && lane == 0) {
    srow[0] = st0;
    srow[1] = st1;
  }
}

template <typename T>
hipError_t launch_t(const FwdArgs& a, hipStream_t stream) {
  const int64_t rows = (int64_t)(a.cu_q ? 1 : a.B) * a.Hq * a.Lq;
  dim3 grid((unsigned)rows), block(64);
  switch (a.norm) {
    case ATTN_SOFTMAX:
      generic_fwd_kernel<T, ATTN_SOFTMAX><<<grid, block, 0, stream>>>(a);
      break;
    case ATTN_SOFTMAX1:
      generic_fwd_kernel<T, ATTN_SOFTMAX1><<<grid, block, 0, stream>>>(a);
      break;
    case ATTN_SPARSEMAX:
      generic_fwd_kernel<T, ATTN_SPARSEMAX><<<grid, block, 0, stream>>>(a);
      break;
    default:
      generic_fwd_kernel<T, ATTN_ENTMAX15><<<grid, block, 0, stream>>>(a);
      break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_generic(const FwdArgs& a, hipStream_t stream) {
  return a.dtype == ATTN_BF16 ? launch_t<bf16_t>(a, stream) : launch_t<float>(a, stream);
}

}  // namespace attn
