// Paged decode (one query token per sequence) with split-KV reduction.
//
// The K/V cache is read page by page through the block table ("HF Attention
// Normalizers", "Differentiable Paged Attention": physical pages are read
// directly, no gathered K/V copy).  The keys of a sequence are cut into
// splits (kSplit keys for the sparse normalizers; for the softmax family a
// size chosen per launch so that the last round of workgroups is nearly
// full); a one-wave plan kernel lists the live splits of all sequences in
// order, and the split kernel's grid walks that list, so no empty split sits
// among the live ones.  One wave handles one (split, kv head, sequence) and
// serves all G = Hq / Hkv query heads of the group, so every K/V byte is read
// once:
//
//   scores  S^T (16 keys x 16 query heads) = K_block . Q^T on
//           v_mfma_f32_16x16x32_bf16; lanes 0..G-1 of each 16 hold real
//           heads, K rows are loaded straight from their pages;
//   softmax / softmax1: online (max, sum) per head over the split, then the
//           weighted sum of V on the vector ALUs (each lane owns 8 dims of
//           one key row per step), written as a partial (m, l, acc[D]);
//           a combine kernel merges the partials ("two-stage KV-tile
//           reduction without atomics", same page) and adds softmax1's "+1";
//   sparsemax / entmax15: the split kernel stores z for every key; a solver
//           kernel per (sequence, query head) finds the row threshold over
//           the candidates above (max z - 1) kept in LDS, then sums
//           g(z - tau) V over the support only, so V rows of zero-weight keys
//           are never read.

#include <map>
#include <mutex>
#include <tuple>

#include "common.h"

namespace attn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kSplit = 512;      // keys per split (sparse normalizers)
static_assert((kSplit & (kSplit - 1)) == 0, "split lists store key offsets masked to the split");
// Softmax family: the split size is chosen per launch among the multiples of
// 32 in [kMinSplit, kMaxSplit] (see decode_plan_kernel); the sparse
// normalizers keep kSplit.  The workspace starts with a header of ints --
// [0] the split size, [1] the number of live splits, [2 + b] the first live
// split of sequence b in the packed list (B + 1 entries) -- rounded up to 64
// words; the partials or split lists follow.  At most 61 16-key blocks per
// split, so a lane per block fits the wave.
constexpr int kMinSplit = 448;
constexpr int kMaxSplit = 960;
__host__ __device__ inline int64_t hdr_words(int B) { return ((int64_t)B + 3 + 63) / 64 * 64; }
constexpr int kSolveCap = 2048;  // candidate capacity of the sparse solver (LDS)

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float bf_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

struct SeqView {
  int n;    // live keys of the sequence (clamped to the table's reach)
  int lo;   // first visible key (sliding window)
};

__device__ __forceinline__ SeqView seq_view(const FwdArgs& a, int b) {
  SeqView v;
  v.n = paged_live(a, b);
  // one query at position n - 1 (bottom-right): causal keeps every live key
  v.lo = a.window ? max(0, v.n - a.window) : 0;
  return v;
}

// Byte offset of key j's row (kv head folded into `head_off`) in a cache.
__device__ __forceinline__ int64_t key_row(const int32_t* table, int bs, int nb, int64_t sb, int64_t sl,
                                           int j) {
  const int64_t page = page_of(table, j / bs, nb);
  return page * sb + (int64_t)(j % bs) * sl;
}

// Partial record per (sequence, query head, split): m, l, 2 pad, acc[D] (fp32;
// acc 16-byte aligned).
__device__ __forceinline__ float* partial_ptr(float* ws, const FwdArgs& a, int b, int qh, int s, int ns) {
  return ws + hdr_words(a.B) + (((int64_t)b * a.Hq + qh) * ns + s) * (a.D + 4);
}

// Split of a softmax-family workgroup: the plan's packed list of live splits
// (sequence-major) is walked by `item`; items past its end get b = -1.
struct SplitRef {
  int b, s, ks;
};
__device__ __forceinline__ SplitRef split_of(const FwdArgs& a, const float* ws, int item) {
  const int* hdr = (const int*)ws;
  SplitRef r;
  r.ks = __builtin_amdgcn_readfirstlane(hdr[0]);
  r.b = -1;
  r.s = 0;
  if (item >= __builtin_amdgcn_readfirstlane(hdr[1])) return r;
  int lo = 0, hi = a.B;  // last b with first[b] <= item
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (__builtin_amdgcn_readfirstlane(hdr[2 + mid]) <= item) lo = mid;
    else hi = mid;
  }
  r.b = lo;
  r.s = seq_view(a, lo).lo / r.ks + (item - __builtin_amdgcn_readfirstlane(hdr[2 + lo]));
  return r;
}

// Threshold search step over the candidate set L = {z > t} (see the
// prefill kernels): returns tau when the closed form over L lies below every
// member of L (then L is the support), else a larger lower bound.
template <int NORM>
__device__ __forceinline__ double solve_step(double c, double s1, double s2, float mn, double mref,
                                             double t, bool& exact) {
  const double ty = t - mref;
  double tcf, step;
  bool valid;
  if (NORM == ATTN_SPARSEMAX) {
    tcf = (s1 - 1.0) / c;
    valid = true;
    step = tcf;
  } else {
    const double mu = s1 / c;
    const double ss = s2 - s1 * mu;
    const double delta = (1.0 - ss) / c;
    valid = delta >= 0.0;
    tcf = valid ? mu - sqrt(delta) : 0.0;
    const double f = s2 - 2.0 * ty * s1 + c * ty * ty - 1.0;
    const double fp = 2.0 * (s1 - c * ty);
    step = ty + f / fp;
  }
  const double mny = (double)mn - mref;
  if (valid && tcf < mny) {
    exact = true;
    return mref + tcf;
  }
  exact = false;
  return mref + fmax(step, mny);
}

// Sparse normalizers.  The threshold of a subset of a row's keys never
// exceeds the row's threshold (more keys need a higher tau to keep the sum at
// one), so a lower bound on the threshold of one split's keys alone ("split
// floor") is a lower bound on tau: every key at or below it has zero weight.
// Per (row, split) the split kernel keeps the keys above its floor, with the
// split's max and floor:
//   smax, sfloor [rows][ns] f32;  cnt [rows][ns] i32;
//   cz [rows][ns][kSplit] f32, ci [rows][ns][kSplit] u16 (key - s kSplit),
// lists in key order; rows = B Hq.
struct SparseLists {
  float* smax;
  float* sfloor;
  int* cnt;
  float* cz;
  uint16_t* ci;
};
__device__ __forceinline__ SparseLists sparse_lists(float* ws, const FwdArgs& a, int ns) {
  const int64_t rn = (int64_t)a.B * a.Hq * ns;
  ws += hdr_words(a.B);  // after the plan's header
  SparseLists l;
  l.smax = ws;
  l.sfloor = ws + rn;
  l.cnt = (int*)(ws + 2 * rn);
  l.cz = ws + 3 * rn;
  l.ci = (uint16_t*)(ws + 3 * rn + rn * kSplit);
  return l;
}
constexpr int kZPad = kSplit + 32;  // LDS row of a split's z values (chunk overhang included)
constexpr int kFloorSteps = 3;      // threshold steps on a split's own keys

// Rounding margin of a split floor (z units).  The floor steps run in fp64
// over at most kSplit keys whose y = z - mh lie in (-1, 0]: y and y^2 are
// exact in fp64, and each of the sums c, s1 = sum y, s2 = sum y^2 is off by
// at most kSplit * 2^-53 * kSplit < 3e-11.  The sparsemax step (s1 - 1) / c
// and the 1.5-entmax Newton step (f / f' with f' = 2 sum (z - t) >= 2 while
// f > 0) inherit errors of the same order; the 1.5-entmax closed form
// mu - sqrt(delta) is the worst conditioned: delta = (1 - ss) / c carries an
// error e of at most ~1e-13, which moves sqrt(delta) by at most sqrt(e) <
// 4e-7.  The jump of a step to the set's minimum is taken only when the
// closed form is inconsistent, and lands at most as far above tau as that
// closed form's own error.  So every computed step stays below the split's
// exact threshold plus 5e-7; the floor subtracts 1e-6 (and the rounding of
// mh + y, 2^-40 |mh|), then rounds towards -inf to a float.
__device__ __forceinline__ double floor_margin(float mh) { return 1e-6 + 0x1p-40 * fabs((double)mh); }

// Largest float not above x.
__device__ __forceinline__ float float_below(double x) {
  float f = (float)x;
  if ((double)f > x) {  // step one ulp towards -inf
    unsigned u = __float_as_uint(f);
    u = f > 0.f ? u - 1u : (f < 0.f ? u + 1u : 0x80000001u);
    f = __uint_as_float(u);
  }
  return f;
}

// End of a sparse split.  The heads of the group run side by side (64 / GP
// lanes each, GP = G rounded up to a power of two): per head the split max
// mh, up to kFloorSteps threshold steps in fp64 over the split's own keys
// starting at mh - 1 (the row solver's step: the closed form over {z > t} if
// it lies below that set's minimum, else a larger lower bound).  The
// threshold of a subset of a row's keys never exceeds the row's, so every
// step is a lower bound on tau; the floor is the last one minus the rounding
// margin above, and the keys above it are compacted in key order with
// ballots.  zs[h][key - s kSplit] holds z of the split's keys [k_begin,
// k_end); mx is the lane's running max of its head (lane % 16); one wave.
template <int NORM, int GM>
__device__ __forceinline__ void sparse_split_lists(const FwdArgs& a, float* ws, int ns, int b, int kvh,
                                                   int s, int k_begin, int k_end, float mx,
                                                   float (*zs)[kZPad], uint16_t (*zi)[kSplit]) {
  const int lane = threadIdx.x & 63;
  mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  const SparseLists L = sparse_lists(ws, a, ns);
  const int lo = k_begin - s * kSplit, hi = k_end - s * kSplit;
  const int G = min(a.G, GM);
  int gp = 1;
  while (gp < G) gp <<= 1;
  const int lph = 64 / gp;                 // lanes per head
  const int h = lane / lph, sub = lane - h * lph;
  const bool act = h < G;
  const int hr = act ? h : 0;
  const float mh = __shfl(mx, hr, 64);     // lane h holds head h's max
  const double mref = (double)mh;
  double t = mref - 1.0;
  bool done = false;
  for (int it = 0; it < kFloorSteps; ++it) {
    double c = 0.0, s1 = 0.0, s2 = 0.0;
    float mn = INFINITY;
    if (!done) {
      for (int idx = lo + sub; idx < hi; idx += lph) {
        const float v = zs[hr][idx];
        if ((double)v > t) {
          const double y = (double)v - mref;
          c += 1.0;
          s1 += y;
          s2 += y * y;
          mn = fminf(mn, v);
        }
      }
    }
    for (int o = 1; o < lph; o <<= 1) {  // sums over the head's lanes
      c += __shfl_xor(c, o, 64);
      s1 += __shfl_xor(s1, o, 64);
      s2 += __shfl_xor(s2, o, 64);
      mn = fminf(mn, __shfl_xor(mn, o, 64));
    }
    if (!done && c > 0.0) {
      bool ex;
      const double tn = solve_step<NORM>(c, s1, s2, mn, mref, t, ex);
      done = ex;
      t = ex ? tn : fmax(t, tn);
    }
  }
  const float tf = mh == -INFINITY ? -INFINITY : float_below(t - floor_margin(mh));
  // compact in LDS, in place (an entry moves to a position at or below the
  // one it was read from, and every read of a round precedes its writes),
  // then copy the list out with contiguous stores
  const unsigned long long grp = (lph == 64 ? ~0ull : ((1ull << lph) - 1ull)) << (h * lph);
  const unsigned long long below = grp & ((1ull << lane) - 1ull);
  int count = 0;
  for (int c0 = lo; c0 < hi; c0 += lph) {
    const int idx = c0 + sub;
    const float z = (act && idx < hi) ? zs[hr][idx] : -INFINITY;
    const bool f = z > tf;
    const unsigned long long bal = __ballot(f);
    if (f) {
      const int pos = count + __popcll(bal & below);
      zs[hr][pos] = z;
      zi[hr][pos] = (uint16_t)idx;
    }
    count += __popcll(bal & grp);
  }
  const int64_t slot = ((int64_t)b * a.Hq + (int64_t)kvh * a.G + hr) * ns + s;
  float* czp = L.cz + slot * kSplit;
  uint16_t* cip = L.ci + slot * kSplit;
  if (act) {
    for (int e = sub; e < count; e += lph) {
      czp[e] = zs[hr][e];
      cip[e] = zi[hr][e];
    }
  }
  if (act && sub == 0) {
    L.smax[slot] = mh;
    L.sfloor[slot] = tf;
    L.cnt[slot] = count;
  }
}

// GM: compile-time bound on the group size G (query heads per kv head).
template <int D, int NORM, bool CAP, int GM>
__global__ __launch_bounds__(64) void decode_split_kernel(FwdArgs a, float* ws, int ns) {
  constexpr int NKC = D / 32;     // k-steps of the 16x16x32 QK product
  constexpr int CPR = D / 8;      // 16-byte chunks per row
  constexpr int KS = 64 / CPR;    // key rows per PV step (lanes per chunk column)
  __shared__ float ps[32][17];    // weights of the 32 keys of a chunk, per head (padded)

  const int lane = threadIdx.x;
  // the plan's packed live splits, kv head fastest; the grid's tail past
  // them exits
  const int kvh = blockIdx.x % a.Hkv;
  const SplitRef r = split_of(a, ws, blockIdx.x / a.Hkv);
  if (r.b < 0) return;
  const int b = r.b, s = r.s, ksp = r.ks;
  const int G = a.G;
  const SeqView sv = seq_view(a, b);
  const int k_begin = max(sv.lo, s * ksp);
  const int k_end = min(sv.n, (s + 1) * ksp);

  const int hh = lane & 15;        // query head of this lane's MFMA column
  const bool head_ok = hh < G;
  const int qh = kvh * G + (head_ok ? hh : 0);
  const int32_t* table = a.block_table + (int64_t)b * a.max_blocks;
  const bf16_t* kc = (const bf16_t*)a.k + (int64_t)kvh * a.k_sh;
  const bf16_t* vc = (const bf16_t*)a.v + (int64_t)kvh * a.v_sh;

  if (k_begin >= k_end) return;  // (a live split is never empty; kept as a guard)

  // Q^T operand: lane l holds head l%16, dims 32c + 8 (l/16) .. +7
  bf16x8 qreg[NKC];
  {
    const bf16_t* qrow = (const bf16_t*)a.q + (int64_t)b * a.q_sb + (int64_t)qh * a.q_sh;
#pragma unroll
    for (int c = 0; c < NKC; ++c)
      qreg[c] = head_ok ? *(const bf16x8*)(qrow + 32 * c + 8 * (lane >> 4)) : bf16x8{};
  }
  const float scale = NORM == ATTN_ENTMAX15 ? 0.5f * a.scaling : a.scaling;  // z units
  const float c2 = a.scaling * kLog2e;
  const float sc_over_cap = CAP ? a.scaling / a.softcap : 0.f;
  const float capz = CAP ? (NORM == ATTN_ENTMAX15 ? 0.5f : 1.f) * a.softcap : 0.f;

  // PV lane layout: key slot ks = lane / CPR, 8 dims from chunk ch = lane % CPR
  const int ks = lane / CPR, ch = lane % CPR;
  float acc[GM][8];  // [head][dim] for this lane's chunk (heads < G used)
#pragma unroll
  for (int h = 0; h < GM; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  float m2 = -INFINITY;  // running max of this lane's head, log2 units
  float lsum = 0.f;      // running sum (this lane's keys only; reduced at the end)

  constexpr bool SPARSE = NORM == ATTN_SPARSEMAX || NORM == ATTN_ENTMAX15;
  __shared__ float zs[SPARSE ? GM : 1][SPARSE ? kZPad : 1];  // z of the split, per head
  __shared__ uint16_t zi[SPARSE ? GM : 1][SPARSE ? kSplit : 1];  // list key offsets
  float mx = -INFINITY;                                      // lane's running max of z

  for (int k0 = k_begin; k0 < k_end; k0 += 32) {
    // ---- scores of keys k0 .. k0+31 (two 16-key MFMA blocks)
    f32x4 sacc[2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      sacc[sb] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int j = k0 + sb * 16 + (lane & 15);
      const int jj = min(j, k_end - 1);  // rows past the end are masked below
      const bf16_t* krow = kc + key_row(table, a.block_size, a.num_blocks, a.k_sb, a.k_sl, jj);
#pragma unroll
      for (int c = 0; c < NKC; ++c) {
        const bf16x8 kv = *(const bf16x8*)(krow + 32 * c + 8 * (lane >> 4));
        sacc[sb] = mfma16(kv, qreg[c], sacc[sb]);
      }
    }
    // lane holds head hh, keys k0 + 16 sb + 4 (lane/16) + r
    float x[8];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = k0 + sb * 16 + 4 * (lane >> 4) + r;
        float v = sacc[sb][r];
        if (NORM == ATTN_SPARSEMAX || NORM == ATTN_ENTMAX15) {
          if (CAP) {
            v = capz * tanhf(v * sc_over_cap);  // accurate near 0 (support test)
          } else {
            v = v * scale;
          }
        } else {
          if (CAP) {
            const float y = v * sc_over_cap;
            const float e = __builtin_amdgcn_exp2f(2.f * kLog2e * y);
            v = a.softcap * kLog2e * (1.f - 2.f * __builtin_amdgcn_rcpf(1.f + e));
          } else {
            v = v * c2;
          }
        }
        x[sb * 4 + r] = j < k_end ? v : -INFINITY;
      }

    if (SPARSE) {
      // z to LDS (k0 is not 4-aligned here: scalar stores); the rows are padded
      // for the keys past k_end of the last chunk
      if (hh < GM) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          zs[hh][k0 - s * kSplit + (i >> 2) * 16 + 4 * (lane >> 4) + (i & 3)] = x[i];
          mx = fmaxf(mx, x[i]);
        }
      }
      continue;
    }

    // ---- online softmax per head (lanes sharing lane%16 share the head)
    float mt = -INFINITY;
#pragma unroll
    for (int i = 0; i < 8; ++i) mt = fmaxf(mt, x[i]);
    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float m_new = fmaxf(m2, mt);
    const float mref = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m2 - mref);
    m2 = m_new;
    lsum *= alpha;
    float p[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      p[i] = __builtin_amdgcn_exp2f(x[i] - mref);
      lsum += p[i];
    }
    // weights to LDS: ps[key][head]
    __syncthreads();  // previous chunk's PV reads are done
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int r = 0; r < 4; ++r) ps[sb * 16 + 4 * (lane >> 4) + r][hh] = p[sb * 4 + r];
    // alpha of every head, for the PV accumulators
    __shared__ float alph[16];
    if (lane < 16) alph[lane] = alpha;
    __syncthreads();
    float al[GM];
#pragma unroll
    for (int h = 0; h < GM; ++h) al[h] = alph[h];
#pragma unroll
    for (int h = 0; h < GM; ++h)
      if (h < G)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] *= al[h];
    // ---- weighted sum of V: rows k0 + ks, k0 + ks + KS, ...
    for (int kk = ks; kk < 32; kk += KS) {
      const int j = k0 + kk;
      if (j < k_end) {
        const bf16_t* vrow = vc + key_row(table, a.block_size, a.num_blocks, a.v_sb, a.v_sl, j);
        const u32x4 w = *(const u32x4*)(vrow + 8 * ch);
        float vv[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          vv[2 * q] = bf_lo(w[q]);
          vv[2 * q + 1] = bf_hi(w[q]);
        }
#pragma unroll
        for (int h = 0; h < GM; ++h)
          if (h < G) {
            const float pj = ps[kk][h];
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(pj, vv[e], acc[h][e]);
          }
      }
    }
  }

  if constexpr (SPARSE) {
    sparse_split_lists<NORM, GM>(a, ws, ns, b, kvh, s, k_begin, k_end, mx, zs, zi);
    return;
  }

  // ---- partial record: reduce acc over the KS key slots, l over the 4 lanes of a head
  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    if (h < G) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float v = acc[h][e];
        for (int o = CPR; o < 64; o <<= 1) v += __shfl_xor(v, o, 64);
        acc[h][e] = v;
      }
    }
  }
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    if (h >= G) break;
    float* pp = partial_ptr(ws, a, b, kvh * G + h, s, ns);
    if (lane == h) {
      pp[0] = m2;
      pp[1] = lsum;
    }
    if (ks == 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) pp[4 + 8 * ch + e] = acc[h][e];
    }
  }
}

// Raw buffer access: a load at byte offset >= `bytes` returns zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, (int)bytes, 0x00020000);
}
// POLICY: the load's cache policy bits (2: non-temporal, for data read once)
template <int POLICY = 0>
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, POLICY));
}

// Split kernel for caches whose page size is a multiple of 16 keys, so a
// 16-key block never straddles two pages.  The split is walked in 16-key
// blocks aligned to the page grid; lane i holds the page and in-page row of
// block i (a split of 512 keys spans at most 33 blocks), so no block-table
// read sits on the load path.  Each block is read through a buffer resource
// whose size is the block's live rows: rows past the sequence end read as
// zeros, so neither K nor V of a partial last page is touched.  K of the next
// 32-key chunk and V of the current one are in flight while the current
// chunk's scores, weights and PV sum are computed.
template <int D, int NORM, bool CAP, int GM>
__global__ __launch_bounds__(512) void decode_split_paged16_kernel(FwdArgs a, float* ws, int ns) {
  constexpr bool SPARSE = NORM == ATTN_SPARSEMAX || NORM == ATTN_ENTMAX15;
  constexpr int NKC = D / 32;     // k-steps of the 16x16x32 QK product
  constexpr int CPR = D / 8;      // 16-byte chunks per row
  constexpr int KS = 64 / CPR;    // key rows per PV step (lanes per chunk column)
  constexpr int RPB = 16 / KS;    // V rows per lane per 16-key block
  constexpr int NV = 32 / KS;     // V rows per lane per 32-key chunk
  // The softmax family reads every K/V byte once: non-temporal loads (the
  // sparse split kernel measured faster with the default policy).
  constexpr int kPolicy = SPARSE ? 0 : 2;

  // A workgroup is WPG waves on WPG consecutive kv heads of one split, so the
  // slot rows of a page (all heads side by side) are read together; the
  // waves never synchronize.  Dynamic LDS: per wave the chunk's weights
  // [32][GM]; sparse: per wave the split's z values [GM][kZPad], then per
  // wave the list key offsets [GM][kSplit] (u16).
  extern __shared__ float dyn_lds[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wpg = blockDim.x >> 6;
  const int ngrp = a.Hkv / wpg;
  const int kvh = (blockIdx.x % ngrp) * wpg + wave;
  // the plan's packed live splits; the grid's tail past them exits
  const SplitRef r = split_of(a, ws, blockIdx.x / ngrp);
  if (r.b < 0) return;
  const int b = r.b, s = r.s, ksp = r.ks;
  float (*ps)[GM] = (float (*)[GM])(dyn_lds + wave * 32 * GM);
  const int G = a.G;
  const SeqView sv = seq_view(a, b);
  const int k_begin = max(sv.lo, s * ksp);
  const int k_end = min(sv.n, (s + 1) * ksp);

  const int hh = lane & 15;
  const bool head_ok = hh < G;
  const int qh = kvh * G + (head_ok ? hh : 0);

  if (k_begin >= k_end) return;  // (a live split is never empty; kept as a guard)

  // blocks of the split: lane i < nblk (at most 61) holds block i's K and V
  // row addresses and live byte ranges; other lanes hold empty ranges
  const int kb = k_begin & ~15;
  const int nblk = (k_end - kb + 15) >> 4;
  const int nchunk = (nblk + 1) >> 1;
  uint64_t kaddr = 0, vaddr = 0;
  uint32_t kbytes = 0, vbytes = 0;
  if (lane < nblk) {
    const int j0 = kb + 16 * lane;
    const int pi = j0 / a.block_size;
    const int64_t pg = page_of(a.block_table + (int64_t)b * a.max_blocks, pi, a.num_blocks);
    const int64_t r = j0 - (int64_t)pi * a.block_size;
    const int live = min(16, k_end - j0);
    kaddr = (uint64_t)((const bf16_t*)a.k + (int64_t)kvh * a.k_sh + pg * a.k_sb + r * a.k_sl);
    vaddr = (uint64_t)((const bf16_t*)a.v + (int64_t)kvh * a.v_sh + pg * a.v_sb + r * a.v_sl);
    kbytes = (uint32_t)(live * a.k_sl * 2);
    vbytes = (uint32_t)(live * a.v_sl * 2);
  }
  // resource over block c's live rows; c may run up to nblk + 2 (< 64), where
  // the range is empty and loads return zeros without touching memory
  auto block_rsrc = [&](uint64_t addr, uint32_t bytes, int c) __attribute__((always_inline)) {
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)addr, c);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(addr >> 32), c);
    const uint32_t n = __builtin_amdgcn_readlane(bytes, c);
    return make_rsrc((const void*)(((uint64_t)hi << 32) | lo), n);
  };

  // Q^T operand: lane l holds head l%16, dims 32c + 8 (l/16) .. +7
  bf16x8 qreg[NKC];
  {
    const bf16_t* qrow = (const bf16_t*)a.q + (int64_t)b * a.q_sb + (int64_t)qh * a.q_sh;
#pragma unroll
    for (int c = 0; c < NKC; ++c)
      qreg[c] = head_ok ? *(const bf16x8*)(qrow + 32 * c + 8 * (lane >> 4)) : bf16x8{};
  }
  const float scale = NORM == ATTN_ENTMAX15 ? 0.5f * a.scaling : a.scaling;  // z units
  const float c2 = a.scaling * kLog2e;
  const float sc_over_cap = CAP ? a.scaling / a.softcap : 0.f;
  const float capz = CAP ? (NORM == ATTN_ENTMAX15 ? 0.5f : 1.f) * a.softcap : 0.f;

  const uint32_t k_voff = (uint32_t)((lane & 15) * a.k_sl * 2 + 16 * (lane >> 4));
  const int ks = lane / CPR, ch = lane % CPR;
  const uint32_t v_voff = (uint32_t)(ks * a.v_sl * 2 + 16 * ch);
  const uint32_t v_step = (uint32_t)(KS * a.v_sl * 2);

  typedef bf16x8 KTile[2][NKC];   // K rows of one 32-key chunk (two 16-key blocks)
  auto load_k = [&](KTile& kt, int t) __attribute__((always_inline)) {
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const __amdgpu_buffer_rsrc_t rk = block_rsrc(kaddr, kbytes, 2 * t + sb);
#pragma unroll
      for (int c = 0; c < NKC; ++c)
        kt[sb][c] = __builtin_bit_cast(bf16x8, buf_load16<kPolicy>(rk, k_voff + 64 * c, 0));
    }
  };
  // scores of chunk t in z units (sparse) or log2 units (softmax family);
  // lane holds head hh, keys k0 + 16 sb + 4 (lane/16) + r at x[4 sb + r]
  auto scores = [&](const KTile& kt, int t, float (&x)[8]) __attribute__((always_inline)) {
    const int k0 = kb + 32 * t;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NKC; ++c) sacc = mfma16(kt[sb][c], qreg[c], sacc);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = k0 + sb * 16 + 4 * (lane >> 4) + r;
        float v = sacc[r];
        if (CAP && SPARSE) {
          v = capz * tanhf(v * sc_over_cap);  // accurate near 0 (support test)
        } else if (CAP) {
          const float y = v * sc_over_cap;
          const float e = __builtin_amdgcn_exp2f(2.f * kLog2e * y);
          v = a.softcap * kLog2e * (1.f - 2.f * __builtin_amdgcn_rcpf(1.f + e));
        } else {
          v = v * (SPARSE ? scale : c2);
        }
        x[sb * 4 + r] = (j >= k_begin && j < k_end) ? v : -INFINITY;
      }
    }
  };

  if (SPARSE) {
    // z of the split to LDS (k0 is 16-aligned: one 16-byte store per block;
    // the padded rows take the empty block past an odd block count), then
    // the per-head lists.  Two chunks of K are in flight: ka holds even
    // chunks, kb_ odd ones.
    float (*zs)[kZPad] = (float (*)[kZPad])(dyn_lds + wpg * 32 * GM + wave * GM * kZPad);
    uint16_t (*zi)[kSplit] =
        (uint16_t (*)[kSplit])(dyn_lds + wpg * (32 * GM + GM * kZPad)) + wave * GM;
    float mx = -INFINITY;
    auto stage_z = [&](int t, const float (&x)[8]) __attribute__((always_inline)) {
      if (hh < GM) {
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
          const int loc = kb + 32 * t + sb * 16 + 4 * (lane >> 4) - s * kSplit;
          *(f32x4*)&zs[hh][loc] = f32x4{x[sb * 4], x[sb * 4 + 1], x[sb * 4 + 2], x[sb * 4 + 3]};
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) mx = fmaxf(mx, x[i]);
      }
    };
    KTile ka, kb_;
    load_k(ka, 0);
    load_k(kb_, 1);
    for (int t = 0; t < nchunk; t += 2) {
      float x[8];
      scores(ka, t, x);
      load_k(ka, t + 2);
      stage_z(t, x);
      if (t + 1 >= nchunk) break;
      scores(kb_, t + 1, x);
      load_k(kb_, t + 3);
      stage_z(t + 1, x);
    }
    sparse_split_lists<NORM, GM>(a, ws, ns, b, kvh, s, k_begin, k_end, mx, zs, zi);
    return;
  }

  // softmax / softmax1: K of chunk t+1 and V of chunk t+1 are issued while
  // chunk t is reduced, so about two chunks stay in flight per wave
  auto load_v = [&](u32x4 (&vr)[NV], int t) __attribute__((always_inline)) {
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const __amdgpu_buffer_rsrc_t rv = block_rsrc(vaddr, vbytes, 2 * t + sb);
#pragma unroll
      for (int i = 0; i < RPB; ++i) vr[sb * RPB + i] = buf_load16<kPolicy>(rv, v_voff, i * v_step);
    }
  };
  float acc[GM][8];
#pragma unroll
  for (int h = 0; h < GM; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  float m2 = -INFINITY;  // running max of this lane's head, log2 units
  float lsum = 0.f;      // running sum over this lane's keys

  KTile kt;
  u32x4 vr[NV];
  load_k(kt, 0);
  load_v(vr, 0);
  for (int t = 0; t < nchunk; ++t) {
    float x[8];
    scores(kt, t, x);
    load_k(kt, t + 1);  // unconditional: past the last chunk the ranges are empty

    // ---- online softmax per head (the 4 lanes with equal lane%16 share a head)
    float mt = -INFINITY;
#pragma unroll
    for (int i = 0; i < 8; ++i) mt = fmaxf(mt, x[i]);
    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float m_new = fmaxf(m2, mt);
    const float mref = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m2 - mref);
    m2 = m_new;
    lsum *= alpha;
    // One wave per workgroup: LDS accesses of the wave complete in issue
    // order, so the weights written here are visible to the reads below and
    // the previous chunk's reads are done before these writes.
    if (hh < GM) {
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = __builtin_amdgcn_exp2f(x[sb * 4 + r] - mref);
          lsum += p;
          ps[sb * 16 + 4 * (lane >> 4) + r][hh] = p;
        }
    }
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      const float al = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), h));
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] *= al;
    }
    // ---- weighted sum of V: lane rows ks + KS i of each block
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int kk = (i / RPB) * 16 + ks + KS * (i % RPB);
      float vv[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        vv[2 * q] = bf_lo(vr[i][q]);
        vv[2 * q + 1] = bf_hi(vr[i][q]);
      }
#pragma unroll
      for (int h = 0; h < GM; ++h) {
        const float pj = ps[kk][h];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(pj, vv[e], acc[h][e]);
      }
    }
    load_v(vr, t + 1);
  }


  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
#pragma unroll
  for (int h = 0; h < GM; ++h) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = acc[h][e];
#pragma unroll
      for (int o = CPR; o < 64; o <<= 1) v += __shfl_xor(v, o, 64);
      acc[h][e] = v;
    }
  }
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    if (h >= G) break;
    float* pp = partial_ptr(ws, a, b, kvh * G + h, s, ns);
    if (lane == h) {
      pp[0] = m2;
      pp[1] = lsum;
    }
    if (ks == 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) pp[4 + 8 * ch + e] = acc[h][e];
    }
  }
}

// Merge the split partials of one (sequence, query head).  All in log2 units.
// The block's threads form NG groups of D/4 lanes; group g sums the float4
// chunks of splits g, g + NG, ..., then the groups are added through LDS.
template <int D, int NORM>
__global__ __launch_bounds__(256) void decode_combine_kernel(FwdArgs a, const float* ws, int ns) {
  constexpr int CH = D / 4;      // float4 chunks of acc
  constexpr int NG = 256 / CH;   // split groups
  constexpr int REC = D + 4;     // record stride (floats)
  const int row = blockIdx.x;    // b * Hq + qh
  const int b = row / a.Hq, qh = row - b * a.Hq;
  const int tid = threadIdx.x;
  __shared__ float red[256];
  __shared__ f32x4 part[NG][CH];
  // the row's live splits s0 .. s0 + nsp - 1 (the plan's list)
  const int* hdr = (const int*)ws;
  const int nsp = hdr[2 + b + 1] - hdr[2 + b];
  const int s0 = seq_view(a, b).lo / hdr[0];
  const float* rec = ws + hdr_words(a.B) + ((int64_t)row * ns + s0) * REC;
  // global max over the splits (softmax1 also counts its logit-0 sink)
  float m = -INFINITY;
  for (int s = tid; s < nsp; s += 256) m = fmaxf(m, rec[(int64_t)s * REC]);
  red[tid] = m;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (tid < o) red[tid] = fmaxf(red[tid], red[tid + o]);
    __syncthreads();
  }
  float M = red[0];
  __syncthreads();
  // softmax1: the virtual key at logit b (0, or the head's learned sink)
  const float sink2 = (NORM == ATTN_SOFTMAX1 && a.sinks) ? a.sinks[qh] * kLog2e : 0.f;
  if (NORM == ATTN_SOFTMAX1) M = fmaxf(M, sink2);
  const float mref = M == -INFINITY ? 0.f : M;
  float l = 0.f;
  for (int s = tid; s < nsp; s += 256) {
    const float* pp = rec + (int64_t)s * REC;
    l += pp[1] * __builtin_amdgcn_exp2f(pp[0] - mref);
  }
  red[tid] = l;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (tid < o) red[tid] += red[tid + o];
    __syncthreads();
  }
  float L = red[0];
  if (NORM == ATTN_SOFTMAX1) L += __builtin_amdgcn_exp2f(sink2 - mref);
  const float inv = L > 0.f ? 1.f / L : 0.f;
  // weighted sum of the acc chunks
  const int g = tid / CH, c = tid - g * CH;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s = g; s < nsp; s += NG) {
    const float* pp = rec + (int64_t)s * REC;
    const float w = __builtin_amdgcn_exp2f(pp[0] - mref);
    const f32x4 v = *(const f32x4*)(pp + 4 + 4 * c);
    acc += w * v;
  }
  part[g][c] = acc;
  __syncthreads();
  bf16_t* orow = (bf16_t*)a.out + (int64_t)b * a.o_sb + (int64_t)qh * a.o_sh;
  if (tid < CH) {
    f32x4 t = part[0][tid];
#pragma unroll
    for (int g2 = 1; g2 < NG; ++g2) t += part[g2][tid];
#pragma unroll
    for (int e = 0; e < 4; ++e) orow[4 * tid + e] = (bf16_t)(t[e] * inv);
  }
  if (a.stats && tid == 0) {
    float* st = a.stats + (int64_t)row * 2;
    const bool any = M != -INFINITY;
    st[0] = any ? M * (1.f / kLog2e) : -INFINITY;
    st[1] = any ? L : 0.f;
  }
}

// Block-wide reductions over 256 threads.
__device__ __forceinline__ double block_sum(double v, double* red) {
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}
__device__ __forceinline__ float block_max(float v, float* red) {
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}
__device__ __forceinline__ float block_min(float v, float* red) {
  for (int o = 32; o >= 1; o >>= 1) v = fminf(v, __shfl_xor(v, o, 64));
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return fminf(fminf(red[0], red[1]), fminf(red[2], red[3]));
}


// Exclusive prefix sum over the 256 threads of a block; returns the block total.
__device__ __forceinline__ int block_scan_excl(int v, int& excl, int* wtot) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) wtot[w] = incl;
  __syncthreads();
  int before = 0;
  for (int w2 = 0; w2 < w; ++w2) before += wtot[w2];
  excl = before + incl - v;
  const int total = wtot[0] + wtot[1] + wtot[2] + wtot[3];
  __syncthreads();
  return total;
}

// One (sequence, query head) row of a sparse normalizer.
//  1. row max M and t0 = the largest split floor (a lower bound on tau);
//  2. the entries above t0 of the split lists are gathered into LDS,
//     concatenated in split order, so they stay in key order (each list
//     holds every key of its split above t0);
//  3. threshold search from t0 over the entries (over the lists in global
//     memory if they outgrow LDS);
//  4. the support's weights and V row offsets are compacted in LDS, then
//     16-byte V chunks of several support rows are summed per wave, so V
//     rows of zero-weight keys are never read.
template <int D, int NORM>
__global__ __launch_bounds__(256) void decode_sparse_solve_kernel(FwdArgs a, float* ws, int ns) {
  constexpr int LPK = D / 8;      // lanes per V row (8 dims each)
  constexpr int KPW = 64 / LPK;   // V rows per wave and step
  __shared__ float cz[kSolveCap];      // z, later the support weights
  __shared__ int ci[kSolveCap];        // key index
  __shared__ int64_t voff[kSolveCap];  // V row offsets of the support (elements)
  __shared__ int pf[257];
  __shared__ int wtot[4];
  __shared__ double redd[4][3];
  __shared__ float redf[4];
  __shared__ float oacc[4][D];

  const int row = blockIdx.x;
  const int b = row / a.Hq, qh = row - b * a.Hq, kvh = qh / a.G;
  const int tid = threadIdx.x, w = tid >> 6, ln = tid & 63;
  const SeqView sv = seq_view(a, b);
  bf16_t* orow = (bf16_t*)a.out + (int64_t)b * a.o_sb + (int64_t)qh * a.o_sh;

  if (sv.lo >= sv.n) {  // no visible key
    for (int d = tid; d < D; d += 256) orow[d] = (bf16_t)0.f;
    if (a.stats && tid == 0) {
      a.stats[(int64_t)row * 2] = INFINITY;
      a.stats[(int64_t)row * 2 + 1] = 0.f;
    }
    return;
  }
  // the splits holding visible keys, all of them non-empty
  const int s0 = sv.lo / kSplit, s1 = (sv.n - 1) / kSplit;
  const SparseLists L = sparse_lists(ws, a, ns);
  const float* smax = L.smax + (int64_t)row * ns;
  const int* cnt = L.cnt + (int64_t)row * ns;
  auto list_z = [&](int s) { return L.cz + ((int64_t)row * ns + s) * kSplit; };
  auto list_i = [&](int s) { return L.ci + ((int64_t)row * ns + s) * kSplit; };

  // 1. row max and the largest split floor (tau >= every split floor)
  const float* sfloor = L.sfloor + (int64_t)row * ns;
  float m = -INFINITY, fl = -INFINITY;
  for (int s = s0 + tid; s <= s1; s += 256) {
    m = fmaxf(m, smax[s]);
    fl = fmaxf(fl, sfloor[s]);
  }
  m = block_max(m, redf);
  fl = block_max(fl, redf);
  const double mref = (double)m;
  const double t0 = (double)fl;  // every list holds all of its split's keys above t0

  // 2. entries above t0 of the qualifying lists into LDS, in key order;
  // 256 splits at a time, their entries flattened by a prefix sum over the
  // list lengths, then compacted with ballots
  int base = 0;
  for (int sb0 = s0; sb0 <= s1; sb0 += 256) {
    const int s = sb0 + tid;
    const int c = (s <= s1 && (double)smax[s] > t0) ? min(max(cnt[s], 0), kSplit) : 0;
    int excl;
    const int T = block_scan_excl(c, excl, wtot);
    pf[tid] = excl;
    if (tid == 0) pf[256] = T;
    __syncthreads();
    for (int f0 = 0; f0 < T; f0 += 256) {
      const int f = f0 + tid;
      float v = -INFINITY;
      int key = 0;
      if (f < T) {
        int lo = 0, hi = 256;  // last i with pf[i] <= f (that split has entries)
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (pf[mid] <= f) lo = mid;
          else hi = mid;
        }
        const int e = f - pf[lo], sx = sb0 + lo;
        v = list_z(sx)[e];
        key = min(sx * kSplit + ((int)list_i(sx)[e] & (kSplit - 1)), sv.n - 1);
      }
      const bool flag = (double)v > t0;
      const unsigned long long bal = __ballot(flag);
      const int before = __popcll(bal & ((1ull << ln) - 1ull));
      if (ln == 0) wtot[w] = __popcll(bal);
      __syncthreads();
      int off = base;
      for (int w2 = 0; w2 < w; ++w2) off += wtot[w2];
      if (flag && off + before < kSolveCap) {
        cz[off + before] = v;
        ci[off + before] = key;
      }
      base += wtot[0] + wtot[1] + wtot[2] + wtot[3];
      __syncthreads();
    }
  }
  const int ncand = base;
  const bool in_lds = ncand <= kSolveCap;

  // every list entry (z, key) of a qualifying split, threads (or waves) strided
  auto for_lists = [&](int first, int stride, auto&& f) __attribute__((always_inline)) {
    for (int s = s0; s <= s1; ++s) {
      if (!((double)smax[s] > t0)) continue;
      const int n_s = min(max(cnt[s], 0), kSplit);
      const float* lz = list_z(s);
      const uint16_t* li = list_i(s);
      for (int e = first; e < n_s; e += stride)
        f(lz[e], min(s * kSplit + ((int)li[e] & (kSplit - 1)), sv.n - 1));
    }
  };

  // 3. Newton / closed form over {z > t}
  double t = t0;
  double tau = INFINITY;
  double ksup = 0.0;
  const int lim = ncand + 2;
  for (int it = 0; it < lim; ++it) {
    double c = 0.0, s1d = 0.0, s2 = 0.0;
    float mn = INFINITY;
    auto add = [&](float v, int) __attribute__((always_inline)) {
      if ((double)v > t) {
        const double y = (double)v - mref;
        c += 1.0;
        s1d += y;
        s2 += y * y;
        mn = fminf(mn, v);
      }
    };
    if (in_lds) {
      for (int e = tid; e < ncand; e += 256) add(cz[e], 0);
    } else {
      for_lists(tid, 256, add);
    }
    for (int o = 32; o >= 1; o >>= 1) {
      c += __shfl_xor(c, o, 64);
      s1d += __shfl_xor(s1d, o, 64);
      s2 += __shfl_xor(s2, o, 64);
      mn = fminf(mn, __shfl_xor(mn, o, 64));
    }
    if (ln == 0) {
      redd[w][0] = c;
      redd[w][1] = s1d;
      redd[w][2] = s2;
      redf[w] = mn;
    }
    __syncthreads();
    c = redd[0][0] + redd[1][0] + redd[2][0] + redd[3][0];
    s1d = redd[0][1] + redd[1][1] + redd[2][1] + redd[3][1];
    s2 = redd[0][2] + redd[1][2] + redd[2][2] + redd[3][2];
    mn = fminf(fminf(redf[0], redf[1]), fminf(redf[2], redf[3]));
    __syncthreads();
    bool ex;
    const double tn = solve_step<NORM>(c, s1d, s2, mn, mref, t, ex);
    if (ex) {
      tau = tn;
      ksup = c;
      break;
    }
    t = fmax(t, tn);
  }
  // Every split floor is a provable lower bound on tau (see floor_margin), so
  // the search ends with an exact closed form at or above t0.  A row for
  // which it does not (the loop ran out, or tau < t0) cannot come out of the
  // arithmetic above; it is reported rather than hidden: out and row_stats
  // are NaN.
  if (!(tau < INFINITY) || tau < t0) {
    for (int d = tid; d < D; d += 256) orow[d] = (bf16_t)NAN;
    if (a.stats && tid == 0) {
      a.stats[(int64_t)row * 2] = NAN;
      a.stats[(int64_t)row * 2 + 1] = NAN;
    }
    return;
  }

  // 4. weighted sum of the support's V rows
  const float tauf = (float)tau;
  const int32_t* table = a.block_table + (int64_t)b * a.max_blocks;
  const bf16_t* vc = (const bf16_t*)a.v + (int64_t)kvh * a.v_sh;
  auto weight = [&](float v) __attribute__((always_inline)) {
    const float dz = v - tauf;
    return dz > 0.f ? (NORM == ATTN_ENTMAX15 ? dz * dz : dz) : 0.f;
  };
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  const int dch = ln % LPK;
  if (in_lds) {
    // compact the support (weight, V row offset) in place, in key order
    int nsup = 0;
    for (int e0 = 0; e0 < ncand; e0 += 256) {
      const int e = e0 + tid;
      const float p = e < ncand ? weight(cz[e]) : 0.f;
      const int key = e < ncand ? ci[e] : 0;
      const bool flag = p > 0.f;
      const unsigned long long bal = __ballot(flag);
      const int before = __popcll(bal & ((1ull << ln) - 1ull));
      if (ln == 0) wtot[w] = __popcll(bal);
      __syncthreads();  // every entry of this round has been read
      int off = nsup;
      for (int w2 = 0; w2 < w; ++w2) off += wtot[w2];
      if (flag) {
        cz[off + before] = p;
        voff[off + before] = page_of(table, key / a.block_size, a.num_blocks) * a.v_sb +
                             (int64_t)(key % a.block_size) * a.v_sl;
      }
      nsup += wtot[0] + wtot[1] + wtot[2] + wtot[3];
      __syncthreads();
    }
    // LPK lanes per row, KPW rows per wave, 4 waves: rows e = slot + 4 KPW i
    const int slot = w * KPW + ln / LPK;
    int e = slot;
    for (; e + 12 * KPW < nsup; e += 16 * KPW) {  // four rows in flight per lane
      u32x4 v4[4];
      float p4[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        v4[u] = *(const u32x4*)(vc + voff[e + 4 * KPW * u] + 8 * dch);
        p4[u] = cz[e + 4 * KPW * u];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[2 * q] = fmaf(p4[u], bf_lo(v4[u][q]), acc[2 * q]);
          acc[2 * q + 1] = fmaf(p4[u], bf_hi(v4[u][q]), acc[2 * q + 1]);
        }
    }
    for (; e < nsup; e += 4 * KPW) {
      const u32x4 v = *(const u32x4*)(vc + voff[e] + 8 * dch);
      const float p = cz[e];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] = fmaf(p, bf_lo(v[q]), acc[2 * q]);
        acc[2 * q + 1] = fmaf(p, bf_hi(v[q]), acc[2 * q + 1]);
      }
    }
  } else {
    // lists outgrew LDS: the wave's lanes split one row (LPK lanes), rows by wave
    for_lists(w * KPW + ln / LPK, 4 * KPW, [&](float v, int key) __attribute__((always_inline)) {
      const float p = weight(v);
      if (p > 0.f) {
        const bf16_t* vrow = vc + key_row(table, a.block_size, a.num_blocks, a.v_sb, a.v_sl, key);
        const u32x4 x = *(const u32x4*)(vrow + 8 * dch);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[2 * q] = fmaf(p, bf_lo(x[q]), acc[2 * q]);
          acc[2 * q + 1] = fmaf(p, bf_hi(x[q]), acc[2 * q + 1]);
        }
      }
    });
  }
  // reduce over the KPW row slots of the wave, then over the waves
#pragma unroll
  for (int q = 0; q < 8; ++q)
    for (int o = LPK; o < 64; o <<= 1) acc[q] += __shfl_xor(acc[q], o, 64);
  if (ln < LPK) {
#pragma unroll
    for (int q = 0; q < 8; ++q) oacc[w][8 * ln + q] = acc[q];
  }
  __syncthreads();
  for (int d = tid; d < D; d += 256)
    orow[d] = (bf16_t)(oacc[0][d] + oacc[1][d] + oacc[2][d] + oacc[3][d]);
  if (a.stats && tid == 0) {
    a.stats[(int64_t)row * 2] = (float)tau;
    a.stats[(int64_t)row * 2 + 1] = (float)ksup;
  }
}

// Split size of a softmax-family launch.  The split workgroups all do the
// same work (a full split) except at sequence ends, so the launch ends when
// the last of ceil(items / slots) rounds of workgroups does; with `slots`
// workgroups resident on the GPU, a size whose item count leaves the last
// round nearly empty wastes most of a round.  Among the multiples of 32 in
// [kMinSplit, kMaxSplit] the size with the fullest last round (items / slots
// over its ceiling) is taken, the larger one on ties (the sparse
// normalizers pass their fixed kSplit); one wave, lane i summing sequences
// i, i + 64, ...  Writes the header: the size, and the packed list of live
// splits that the split kernels walk in grid order, so no workgroup of the
// grid's head is an empty split.
__global__ __launch_bounds__(64) void decode_plan_kernel(FwdArgs a, float* ws, int slots, int groups,
                                                          int fixed_ks) {
  const int lane = threadIdx.x;
  float best = -1.f;
  int best_ks = fixed_ks > 0 ? fixed_ks : kSplit;
  if (fixed_ks == 0) {
    // every candidate size's item count from one read of the lengths (a
    // read per size puts a global-memory round trip per size on this
    // kernel's critical path)
    constexpr int NKS = (kMaxSplit - kMinSplit) / 32 + 1;
    int items[NKS];
#pragma unroll
    for (int i = 0; i < NKS; ++i) items[i] = 0;
    for (int b = lane; b < a.B; b += 64) {
      const SeqView sv = seq_view(a, b);
      if (sv.n > sv.lo) {
#pragma unroll
        for (int i = 0; i < NKS; ++i) {
          const int ks = kMinSplit + 32 * i;
          items[i] += (sv.n + ks - 1) / ks - sv.lo / ks;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < NKS; ++i) {
      const int n = wave_sum(items[i]) * groups;
      const float rounds = (float)n / (float)slots;
      const float eff = rounds <= 0.f ? 0.f : rounds / ceilf(rounds);
      if (eff >= best) {  // ascending sizes: the larger one on ties
        best = eff;
        best_ks = kMinSplit + 32 * i;
      }
    }
  }
  // packed list: first live split of each sequence (exclusive prefix sum)
  int* hdr = (int*)ws;
  int base = 0;
  for (int b0 = 0; b0 < a.B; b0 += 64) {
    const int b = b0 + lane;
    int n = 0;
    if (b < a.B) {
      const SeqView sv = seq_view(a, b);
      if (sv.n > sv.lo) n = (sv.n + best_ks - 1) / best_ks - sv.lo / best_ks;
    }
    int incl = n;  // inclusive scan over the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(incl, o, 64);
      if (lane >= o) incl += t;
    }
    if (b < a.B) hdr[2 + b] = base + incl - n;
    base += __shfl(incl, 63, 64);
  }
  if (lane == 0) {
    hdr[0] = best_ks;
    hdr[1] = base;
    hdr[2 + a.B] = base;
  }
}

// Page size a multiple of 16 and cache rows that fit the 32-bit buffer
// offsets of the paged16 split kernel.
bool paged16(const FwdArgs& a) {
  const int64_t zbytes = (int64_t)a.G * a.max_blocks * a.block_size * 4;  // sparse z rows of a group
  return a.block_size % 16 == 0 && a.k_sl >= a.D && a.v_sl >= a.D && a.k_sl <= (1 << 26) &&
         a.v_sl <= (1 << 26) && zbytes < ((int64_t)1 << 31);
}

int num_splits(const FwdArgs& a) {
  const int64_t maxlen = (int64_t)a.max_blocks * a.block_size;
  const int ks = (a.norm == ATTN_SOFTMAX || a.norm == ATTN_SOFTMAX1) ? kMinSplit : kSplit;
  return (int)((maxlen + ks - 1) / ks);
}

// Workgroups of `kern` resident on the current device at once (cached per
// device and kernel configuration).
int resident_groups(const void* kern, int threads, size_t lds) {
  static std::mutex mu;
  static std::map<std::tuple<int, const void*, int, size_t>, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  const auto key = std::make_tuple(dev, kern, threads, lds);
  std::lock_guard<std::mutex> lock(mu);
  const auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int cus = 0, per = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kern, threads, lds) != hipSuccess || per <= 0)
    per = 1;
  return cache[key] = cus * per;
}

template <int D, int NORM>
hipError_t launch_d(const FwdArgs& a, void* workspace, hipStream_t stream) {
  float* ws = (float*)workspace;
  const int ns = num_splits(a);
  const bool cap = a.softcap > 0.f;
  dim3 g1((unsigned)((int64_t)a.B * a.Hkv * ns)), b1(64);
  if (paged16(a)) {
    const int gm = a.G <= 4 ? 4 : a.G <= 8 ? 8 : 16;
    const bool sparse = NORM == ATTN_SPARSEMAX || NORM == ATTN_ENTMAX15;
    auto lds_bytes = [&](int w) {
      return (size_t)w * ((32 * gm + (sparse ? gm * kZPad : 0)) * sizeof(float) +
                          (sparse ? gm * kSplit * sizeof(uint16_t) : 0));
    };
    // waves (kv heads) per workgroup: divides Hkv, LDS leaves room for two
    // groups; the sparse kernels (LDS-heavy) measured best with two
    int wpg = sparse ? 2 : 8;
    while (wpg > 1 && (a.Hkv % wpg != 0 || lds_bytes(wpg) > 80 * 1024)) wpg >>= 1;
    const size_t lds = lds_bytes(wpg);
    dim3 g16((unsigned)((int64_t)a.B * ns * (a.Hkv / wpg))), b16(64 * wpg);
    auto go = [&](auto kern) {
      hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
      const int slots = resident_groups((const void*)kern, 64 * wpg, lds);
      decode_plan_kernel<<<dim3(1), dim3(64), 0, stream>>>(a, ws, slots, a.Hkv / wpg, sparse ? kSplit : 0);
      kern<<<g16, b16, lds, stream>>>(a, ws, ns);
      return hipSuccess;
    };
    hipError_t e0;
    if (gm == 4) e0 = cap ? go(decode_split_paged16_kernel<D, NORM, true, 4>) : go(decode_split_paged16_kernel<D, NORM, false, 4>);
    else if (gm == 8) e0 = cap ? go(decode_split_paged16_kernel<D, NORM, true, 8>) : go(decode_split_paged16_kernel<D, NORM, false, 8>);
    else e0 = cap ? go(decode_split_paged16_kernel<D, NORM, true, 16>) : go(decode_split_paged16_kernel<D, NORM, false, 16>);
    if (e0 != hipSuccess) return e0;
  } else {
    {
      const bool sparse = NORM == ATTN_SPARSEMAX || NORM == ATTN_ENTMAX15;
      const void* k1 = a.G <= 4 ? (const void*)decode_split_kernel<D, NORM, false, 4>
                                : a.G <= 8 ? (const void*)decode_split_kernel<D, NORM, false, 8>
                                           : (const void*)decode_split_kernel<D, NORM, false, 16>;
      decode_plan_kernel<<<dim3(1), dim3(64), 0, stream>>>(a, ws, resident_groups(k1, 64, 0), a.Hkv,
                                                           sparse ? kSplit : 0);
    }
    if (a.G <= 4) {
      if (cap) decode_split_kernel<D, NORM, true, 4><<<g1, b1, 0, stream>>>(a, ws, ns);
      else decode_split_kernel<D, NORM, false, 4><<<g1, b1, 0, stream>>>(a, ws, ns);
    } else if (a.G <= 8) {
      if (cap) decode_split_kernel<D, NORM, true, 8><<<g1, b1, 0, stream>>>(a, ws, ns);
      else decode_split_kernel<D, NORM, false, 8><<<g1, b1, 0, stream>>>(a, ws, ns);
    } else {
      if (cap) decode_split_kernel<D, NORM, true, 16><<<g1, b1, 0, stream>>>(a, ws, ns);
      else decode_split_kernel<D, NORM, false, 16><<<g1, b1, 0, stream>>>(a, ws, ns);
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 g2((unsigned)((int64_t)a.B * a.Hq)), b2(256);
  if (NORM == ATTN_SOFTMAX || NORM == ATTN_SOFTMAX1)
    decode_combine_kernel<D, NORM><<<g2, b2, 0, stream>>>(a, ws, ns);
  else
    decode_sparse_solve_kernel<D, NORM><<<g2, b2, 0, stream>>>(a, ws, ns);
  return hipGetLastError();
}

template <int D>
hipError_t launch_dn(const FwdArgs& a, void* workspace, hipStream_t stream) {
  switch (a.norm) {
    case ATTN_SOFTMAX: return launch_d<D, ATTN_SOFTMAX>(a, workspace, stream);
    case ATTN_SOFTMAX1: return launch_d<D, ATTN_SOFTMAX1>(a, workspace, stream);
    case ATTN_SPARSEMAX: return launch_d<D, ATTN_SPARSEMAX>(a, workspace, stream);
    default: return launch_d<D, ATTN_ENTMAX15>(a, workspace, stream);
  }
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

}  // namespace

bool decode_supported(const FwdArgs& a) {
  if (a.dtype != ATTN_BF16 || !a.paged || a.Lq != 1) return false;
  if (a.D != 64 && a.D != 128 && a.D != 256) return false;
  if (a.G < 1 || a.G > 16) return false;
  if (!(a.scaling > 0.f)) return false;
  if (!aligned16(a.q) || !aligned16(a.k) || !aligned16(a.v)) return false;
  const int64_t s[] = {a.q_sb, a.q_sh, a.k_sb, a.k_sh, a.k_sl, a.v_sb, a.v_sh, a.v_sl};
  for (int64_t x : s)
    if (x % 8) return false;
  return true;
}

size_t decode_workspace_bytes(const FwdArgs& a) {
  if (a.norm == ATTN_SOFTMAX || a.norm == ATTN_SOFTMAX1)
    return (size_t)hdr_words(a.B) * sizeof(float) +
           (size_t)a.B * a.Hq * num_splits(a) * (a.D + 4) * sizeof(float);
  // header, then the split lists: max, floor, length, z and key offset per
  // (row, split)
  return (size_t)hdr_words(a.B) * sizeof(float) +
         (size_t)a.B * a.Hq * num_splits(a) * (3 * sizeof(float) + kSplit * (sizeof(float) + sizeof(uint16_t)));
}

hipError_t launch_decode(const FwdArgs& a, void* workspace, hipStream_t stream) {
  switch (a.D) {
    case 64: return launch_dn<64>(a, workspace, stream);
    case 128: return launch_dn<128>(a, workspace, stream);
    default: return launch_dn<256>(a, workspace, stream);
  }
}

}  // namespace attn
