// Matrix-core backward for bf16 inputs with head dim 64, 128 or 256 ("HF Attention
// Normalizers", "Important Limitations": the fused kernels save the row max
// and denominator, or one threshold per query row, and recompute the weights
// tile by tile in the backward).  Two kernels, the flash-attention-2 split:
//
//   query kernel, one workgroup per 128 query rows of one (batch, head), lane
//   per query as in the forward:
//     pass 1   S^T = K Q^T and dP^T = V dO^T per key tile, the weights from the
//              row statistics, and the row constant of the normalizer's
//              Jacobian (softmax family sum p dP; sparsemax the mean of dP
//              over the support; 1.5-entmax sum u dP / sum u, u = (z - tau)+),
//              written with the row's weight parameters to a per-row record;
//              for the softmax family with the forward's output at hand the
//              constant is dO . O (the weights sum to one and the sink's value
//              is zero) and the pass is skipped
//     pass 2   dS^T = w (dP^T - c) through softcap and scaling, and
//              dQ^T += K^T dS^T (K^T from a transposing LDS read)
//   key kernel, one workgroup per 128 keys of one (batch, kv head), lane per
//   key; K and V rows stay in registers while the Q and dO tiles of the G
//   query heads stream through LDS:
//     S = Q K^T, dP = dO V^T, weights from the records,
//     dV^T += dO^T P and dK^T += Q^T dS (transposing LDS reads of the tiles).
//   When that grid is small (under 1024 workgroups, with G > 1) the causal
//   grid would be too coarse and too unequal to fill the chip: then each
//   workgroup takes one query head, writes fp32 partial sums, and a small
//   kernel adds the G partials in head order.
//
// w is the Jacobian weight of a score: p for the softmax family, 1 on the
// support for sparsemax, u for 1.5-entmax; dS = w (dP - c) is the gradient
// with respect to the (capped) score s, and ds/draw = scaling, or
// scaling (1 - tanh^2) under softcap.  Every tile is staged K-swizzled, so the
// same LDS image serves the row reads of the score products and the
// transposing reads of the gradient products.

#include "tiles.h"

namespace attn {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int N>
struct Mode {  // a compile-time int carried by an argument's type
  static constexpr int value = N;
};

constexpr int kRecRows = 32;  // rows per block of the record workspace

// Record workspace: per (batch, query head), blocks of 32 rows, each
// [3][32] floats: field 0 softmax family m log2(e), sparse tau; field 1
// softmax family 1 / l (0 for a row without keys); field 2 the row constant c.
__device__ __host__ __forceinline__ int64_t rec_blocks(int Lq) { return (Lq + kRecRows - 1) / kRecRows; }
__device__ __forceinline__ int64_t rec_offset(int64_t bh, int Lq, int i) {
  return (bh * rec_blocks(Lq) + i / kRecRows) * (3 * kRecRows) + i % kRecRows;
}

// Query rows [ilo, ihi) that see key j (inverse of the row bounds).
__device__ __forceinline__ void query_bounds(int j, int lq, int lk, int causal, int window, int& ilo,
                                             int& ihi) {
  const int off = lk - lq;  // query i sits at key position i + off
  ilo = causal ? max(0, j - off) : 0;
  ihi = window ? min(lq, j - off + window) : lq;
  ihi = max(ihi, ilo);
}

// Transposed operand (32 dims x 16 rows) of gradient step t and dim block db
// from a K-swizzled row-major tile: the same lane pattern as the forward's
// V^T read, with the K swizzle of rows r and r + 8 (which differ in it).
// Rows r + 16 t share row r's swizzle for both swizzle functions.
template <class C>
struct TrK {
  uint32_t lo[C::NDB], hi[C::NDB];
  __device__ __forceinline__ void init(int lane) {
    const int G = lane >> 4, s = lane & 15, j = s >> 2, q = s & 3;
    const int r0 = 4 * (G >> 1) + j, r1 = r0 + 8;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
      const int lc = db * 4 + 2 * (G & 1) + (q >> 1);
      lo[db] = (uint32_t)((r0 * C::D + k_chunk<C::D>(r0, lc) * 8 + (q & 1) * 4) * 2);
      hi[db] = (uint32_t)((r1 * C::D + k_chunk<C::D>(r1, lc) * 8 + (q & 1) * 4) * 2);
    }
  }
  __device__ __forceinline__ bf16x8 read(const bf16_t* tile, int t, int db) const {
    const char* base = (const char*)tile + t * 16 * C::D * 2;
    const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(base + lo[db]));
    const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(base + hi[db]));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
  }
};

// K-swizzled staging of one tile of ROWS rows x D through direct transfers
// (the forward's K-tile pattern, for any row stride).
template <class C>
struct RowDma {
  static constexpr int NI = C::KCH / 64 / C::NW;  // transfers per wave per tile
  static_assert(C::KCH % (64 * C::NW) == 0, "tile must split into 1 KB transfers per wave");
  uint32_t off[NI];
  uint32_t str;
  int wave;
  __device__ __forceinline__ void init(int64_t row_stride, int wave_u, int lane) {
    str = (uint32_t)(row_stride * 2);
    wave = wave_u;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int pos = (i * C::NW + wave) * 64 + lane;
      const int row = pos / C::CPR, pc = pos % C::CPR;
      off[i] = row * str + k_chunk<C::D>(row, pc) * 16;
    }
  }
  // rows r0 .. r0 + BN - 1 of the buffer; a transfer that is not needed is
  // sent wholly out of range (every wave issues the same count)
  __device__ __forceinline__ void issue(i32x4 rsrc, const bf16_t* tile, int r0, bool live) const {
    const uint32_t la = lds_addr(tile) + wave * 1024;
    const uint32_t so = live ? (uint32_t)r0 * str : 0x80000000u;
#pragma unroll
    for (int i = 0; i < NI; ++i) dma16(rsrc, la + i * C::NW * 1024, off[i], so);
  }
};

struct ElemConst {
  float cz;           // raw -> z (softmax family: s log2(e))
  float sc_over_cap;  // softcap: raw -> tanh argument
  float capz;         // softcap: tanh -> z
  float scaling;
};

template <int NORM, bool CAP>
__device__ __forceinline__ ElemConst elem_const(const FwdArgs& a) {
  ElemConst e;
  const float f = (NORM == ATTN_SOFTMAX || NORM == ATTN_SOFTMAX1) ? kLog2e : (NORM == ATTN_ENTMAX15 ? 0.5f : 1.f);
  e.cz = a.scaling * f;
  e.sc_over_cap = CAP ? a.scaling / a.softcap : 0.f;
  e.capz = CAP ? a.softcap * f : 0.f;
  e.scaling = a.scaling;
  return e;
}

// Forward weight p, Jacobian weight w and ds/draw of one raw score, from the
// row's record fields r0, r1.  The sparse z is formed as in the forward
// (same rounding), so the support matches it.  Every result is finite for
// any finite raw score, masked ones included (the softmax exponent is
// clamped at the row max), so masking is a multiply by 0 or 1: no
// data-dependent branch in the element loops.
template <int NORM, bool CAP>
__device__ __forceinline__ void elem(float raw, float r0, float r1, const ElemConst& k, float& p, float& w,
                                     float& dsdraw) {
#pragma clang fp contract(off)
  float z;
  if (CAP) {
    const float y = raw * k.sc_over_cap;
    float t;
    if (NORM == ATTN_SOFTMAX || NORM == ATTN_SOFTMAX1) {
      const float e = __builtin_amdgcn_exp2f(2.f * kLog2e * y);  // exp(2y)
      t = 1.f - 2.f * __builtin_amdgcn_rcpf(1.f + e);            // tanh(y)
    } else {
      t = tanhf(y);  // the forward's sparse z (same support)
    }
    z = k.capz * t;
    dsdraw = k.scaling * (1.f - t * t);
  } else {
    z = raw * k.cz;
    dsdraw = k.scaling;
  }
  if (NORM == ATTN_SOFTMAX || NORM == ATTN_SOFTMAX1) {
    p = __builtin_amdgcn_exp2f(fminf(z - r0, 0.f)) * r1;
    w = p;
  } else {
    const float d = z - r0;
    const float u = d > 0.f ? d : 0.f;
    p = NORM == ATTN_ENTMAX15 ? u * u : u;
    w = NORM == ATTN_ENTMAX15 ? u : (d > 0.f ? 1.f : 0.f);
  }
}

// ---------------------------------------------------------------------------
// query kernel
// D = 256: Q, dO and the dQ accumulators need one wave per SIMD
template <class C, int NORM, bool CAP, bool OUT>
__global__ __launch_bounds__(C::NT, C::D == 256 ? 1 : 2) void bwd_query_mfma(BwdArgs w) {
  static_assert(!OUT || NORM == ATTN_SOFTMAX || NORM == ATTN_SOFTMAX1, "dO . O is the softmax-family constant");
  const FwdArgs& a = w.f;
  constexpr int KT = C::BN * C::D;
  __shared__ __attribute__((aligned(16))) bf16_t lds[2 * 2 * KT];  // 2 stages x (K, V)
  auto kt = [&](int u) { return lds + u * 2 * KT; };
  auto vt = [&](int u) { return lds + u * 2 * KT + KT; };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  const int Lq = a.Lq, Lk = a.Lk;
  const int nqb = (Lq + C::BM - 1) / C::BM;
  int bh, qb;
  block_coords(nqb, bh, qb);  // per-XCD ranges of heads, longest (causal) blocks first
  const int b = bh / a.Hq, h = bh - b * a.Hq, kvh = h / a.G;
  const int q0 = qb * C::BM;

  const bf16_t* qbase = (const bf16_t*)a.q + (int64_t)b * a.q_sb + (int64_t)h * a.q_sh;
  const bf16_t* dobase = (const bf16_t*)w.dout + (int64_t)b * w.do_sb + (int64_t)h * w.do_sh;
  const bf16_t* kbase = (const bf16_t*)a.k + (int64_t)b * a.k_sb + (int64_t)kvh * a.k_sh;
  const bf16_t* vbase = (const bf16_t*)a.v + (int64_t)b * a.v_sb + (int64_t)kvh * a.v_sh;

  const int qlast = min(q0 + C::BM, Lq) - 1;
  const RowBounds first = row_bounds(q0, Lq, Lk, a.causal, a.window);
  const RowBounds last = row_bounds(qlast, Lq, Lk, a.causal, a.window);
  const int t0 = first.lo / C::BN;
  const int t1 = last.hi > first.lo ? (last.hi + C::BN - 1) / C::BN : t0;
  const int nt = t1 - t0;

  const int wq0 = q0 + 32 * wave;
  const int wq1 = min(wq0 + 31, Lq - 1);
  const bool wave_rows = wq0 < Lq;
  const RowBounds wfirst = row_bounds(wq0, Lq, Lk, a.causal, a.window);
  const RowBounds wlast = row_bounds(wq1, Lq, Lk, a.causal, a.window);
  const int myq = wq0 + l32;
  const bool row_ok = myq < Lq;
  const RowBounds mine = row_bounds(row_ok ? myq : wq1, Lq, Lk, a.causal, a.window);

  bf16x8 qreg[C::NQC], doreg[C::NQC];
  {
    const bf16_t* qrow = qbase + (int64_t)myq * a.q_sl;
    const bf16_t* dorow = dobase + (int64_t)myq * w.do_sl;
#pragma unroll
    for (int c = 0; c < C::NQC; ++c) {
      qreg[c] = row_ok ? *(const bf16x8*)(qrow + 16 * c + 8 * g) : bf16x8{};
      doreg[c] = row_ok ? *(const bf16x8*)(dorow + 16 * c + 8 * g) : bf16x8{};
    }
  }
  const int64_t row = (int64_t)bh * Lq + myq;
  const float st0 = row_ok ? a.stats[row * 2] : 0.f, st1 = row_ok ? a.stats[row * 2 + 1] : 0.f;
  const bool soft = NORM == ATTN_SOFTMAX || NORM == ATTN_SOFTMAX1;
  const float r0 = soft ? st0 * kLog2e : st0;
  const float r1 = soft ? (st1 > 0.f ? 1.f / st1 : 0.f) : 0.f;
  const ElemConst ek = elem_const<NORM, CAP>(a);

  const i32x4 rk = rsrc_words(kbase, (uint32_t)((int64_t)Lk * a.k_sl * 2));
  const i32x4 rv = rsrc_words(vbase, (uint32_t)((int64_t)Lk * a.v_sl * 2));
  RowDma<C> dk_, dv_;
  dk_.init(a.k_sl, wave, lane);
  dv_.init(a.v_sl, wave, lane);
  auto issue = [&](int stage, int u) __attribute__((always_inline)) {
    const bool live = u < nt;
    const int r = (t0 + u) * C::BN;
    dk_.issue(rk, kt(stage), r, live);
    dv_.issue(rv, vt(stage), r, live);
  };
  // one pass over the key tiles; body(kl, vl, k0) runs on the active ones
  auto pass = [&](auto&& body) __attribute__((always_inline)) {
    issue(0, 0);
    wait_vmcnt<0>();
    lds_barrier();
    for (int u = 0; u < nt; ++u) {
      const int cur = u & 1;
      issue(cur ^ 1, u + 1);
      const int k0 = (t0 + u) * C::BN;
      if (wave_rows && k0 < wlast.hi && k0 + C::BN > wfirst.lo) body(kt(cur), vt(cur), k0);
      wait_vmcnt<0>();
      lds_barrier();
    }
  };
  auto edge_of = [&](int k0) { return (k0 + C::BN > wfirst.hi) || (k0 < wlast.lo); };

  // ---- pass 1: the row constant ---------------------------------------------
  float c1 = 0.f, c2 = 0.f;
  if (OUT) {
    // dO . O over this lane's half of the row (the chunks it holds of dO)
    if (row_ok) {
      const bf16_t* orow = (const bf16_t*)a.out + (int64_t)b * a.o_sb + (int64_t)h * a.o_sh + (int64_t)myq * a.o_sl;
#pragma unroll
      for (int c = 0; c < C::NQC; ++c) {
        const bf16x8 o8 = *(const bf16x8*)(orow + 16 * c + 8 * g);
#pragma unroll
        for (int e = 0; e < 8; ++e) c1 += (float)o8[e] * (float)doreg[c][e];
      }
    }
  } else
  pass([&](const bf16_t* kl, const bf16_t* vl, int k0) __attribute__((always_inline)) {
    f32x16 s[C::NKB], dp[C::NKB];
    qk_tile<C>(kl, qreg, l32, g, s);
    qk_tile<C>(vl, doreg, l32, g, dp);
    const bool edge = edge_of(k0);
#pragma unroll
    for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = s_key(k0, kb, r, g);
        const float okf = (!edge || (key >= mine.lo && key < mine.hi)) ? 1.f : 0.f;
        float p, wt, dsdraw;
        elem<NORM, CAP>(s[kb][r], r0, r1, ek, p, wt, dsdraw);
        wt *= okf;
        c1 += wt * dp[kb][r];
        if (!soft) c2 += wt;
      }
  });
  c1 = pair_sum(c1);
  c2 = pair_sum(c2);
  const float c = soft ? c1 : (c2 > 0.f ? c1 / c2 : 0.f);
  // rows past Lq in the last record block get zeros: the key kernel reads
  // whole blocks and masks by multiplying, so every field must be finite
  if (g == 0 && myq < rec_blocks(Lq) * kRecRows) {
    const int64_t ro = rec_offset(bh, Lq, myq);
    w.rec[ro] = row_ok ? r0 : 0.f;
    w.rec[ro + kRecRows] = row_ok ? r1 : 0.f;
    w.rec[ro + 2 * kRecRows] = row_ok ? c : 0.f;
  }
  if (row_ok && g == 0) {
    if (NORM == ATTN_SOFTMAX1 && w.dsinks) {
      const float sink = a.sinks ? a.sinks[h] : 0.f;
      w.srow[row] = -__expf(sink - st0) * r1 * c;
    }
  }

  // ---- pass 2: dQ -------------------------------------------------------------
  f32x16 o[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) o[db] = f32x16{};
  TrK<C> ktr;
  ktr.init(lane);
  pass([&](const bf16_t* kl, const bf16_t* vl, int k0) __attribute__((always_inline)) {
    f32x16 s[C::NKB], dp[C::NKB];
    qk_tile<C>(kl, qreg, l32, g, s);
    qk_tile<C>(vl, doreg, l32, g, dp);
    const bool edge = edge_of(k0);
    bf16x8 op[2 * C::NKB];
#pragma unroll
    for (int kb = 0; kb < C::NKB; ++kb) {
      float d16[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = s_key(k0, kb, r, g);
        const float okf = (!edge || (key >= mine.lo && key < mine.hi)) ? 1.f : 0.f;
        float p, wt, dsdraw;
        elem<NORM, CAP>(s[kb][r], r0, r1, ek, p, wt, dsdraw);
        d16[r] = okf * (wt * (dp[kb][r] - c) * dsdraw);
      }
      op[2 * kb] = p_operand(d16);
      op[2 * kb + 1] = p_operand(d16 + 8);
    }
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int u = 0; u < 2 * C::NKB; ++u) o[db] = mfma(ktr.read(kl, u, db), op[u], o[db]);
  });
  wait_vmcnt<0>();
  if (row_ok) {
    bf16_t* dqrow = (bf16_t*)w.dq + (int64_t)b * w.dq_sb + (int64_t)h * w.dq_sh + (int64_t)myq * w.dq_sl;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        bf16x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = (bf16_t)o[db][4 * rq + e];
        *(bf16x4*)(dqrow + db * 32 + 8 * rq + 4 * g) = v4;
      }
  }
}

// ---------------------------------------------------------------------------
// key kernel: C describes the streamed query tiles (BN = 32 or 64 query rows,
// one or two record blocks).  Dynamic LDS: two stages of (Q tile, dO tile,
// the tile's record blocks per wave).
template <class C>
struct KeyLds {
  static constexpr int STAGE = 2 * C::BN * C::D * 2 + C::NW * 1024;
  static constexpr int BYTES = 2 * STAGE;
};

template <class C, int NORM, bool CAP>
// D = 256: one wave per SIMD even with dK and dV in separate passes
__global__ __launch_bounds__(C::NT, C::D >= 256 ? 1 : 2) void bwd_key_mfma(BwdArgs w) {
  static_assert(C::BN % kRecRows == 0 && C::BN / kRecRows * 3 * kRecRows * 4 <= 1024,
                "a query tile's record blocks must fit one 1 KB transfer");
  const FwdArgs& a = w.f;
  constexpr int QT = C::BN * C::D;            // elements of one Q (or dO) tile
  constexpr int STAGE = KeyLds<C>::STAGE;
  extern __shared__ __attribute__((aligned(16))) char lds[];  // KeyLds<C>::BYTES
  auto qt_of = [&](int u) { return (const bf16_t*)(lds + u * STAGE); };
  auto dt_of = [&](int u) { return (const bf16_t*)(lds + u * STAGE + QT * 2); };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  const int Lq = a.Lq, Lk = a.Lk;
  constexpr int BK = 32 * C::NW;  // keys per workgroup
  const int nkb = (Lk + BK - 1) / BK;
  // per-XCD ranges of heads (the query heads of a kv head are adjacent, so
  // its K / V rows stay in one L2), the first key blocks -- seen by the most
  // causal queries -- first
  int bh, rev;
  block_coords(nkb, bh, rev);
  const int kblk = nkb - 1 - rev;
  const bool split = w.key_split != 0;  // one query head per workgroup
  const int nh = split ? a.Hq : a.Hkv;
  const int b = bh / nh, hx = bh - b * nh;
  const int kvh = split ? hx / a.G : hx;
  const int h0 = split ? hx : kvh * a.G;  // first query head of the workgroup
  const int nheads = split ? 1 : a.G;
  const float* rec_lds = (const float*)(lds + 2 * QT * 2 + wave * 1024);  // + stage offset

  // keys of this workgroup, this wave and this lane
  const int kg0 = kblk * BK, kg1 = min(kg0 + BK, Lk) - 1;
  const int kw0 = kg0 + 32 * wave, kw1 = min(kw0 + 31, Lk - 1);
  const bool wave_keys = kw0 < Lk;
  const int myk = kw0 + l32;
  const bool key_ok = myk < Lk;
  int ilo_g, ihi_g, ilo_w0, ihi_w0, ilo_w1, ihi_w1, ilo, ihi;
  query_bounds(kg0, Lq, Lk, a.causal, a.window, ilo_g, ihi_g);
  {
    int x, y;
    query_bounds(kg1, Lq, Lk, a.causal, a.window, x, y);
    ihi_g = max(ihi_g, y);
  }
  query_bounds(kw0, Lq, Lk, a.causal, a.window, ilo_w0, ihi_w0);
  query_bounds(wave_keys ? kw1 : kw0, Lq, Lk, a.causal, a.window, ilo_w1, ihi_w1);
  query_bounds(myk, Lq, Lk, a.causal, a.window, ilo, ihi);
  if (!key_ok) ilo = ihi = 0;
  const int wlo = ilo_w0, whi = ihi_w1;  // queries any key of the wave sees

  const bf16_t* kbase = (const bf16_t*)a.k + (int64_t)b * a.k_sb + (int64_t)kvh * a.k_sh;
  const bf16_t* vbase = (const bf16_t*)a.v + (int64_t)b * a.v_sb + (int64_t)kvh * a.v_sh;
  bf16x8 kreg[C::NQC], vreg[C::NQC];
  {
    const bf16_t* krow = kbase + (int64_t)myk * a.k_sl;
    const bf16_t* vrow = vbase + (int64_t)myk * a.v_sl;
#pragma unroll
    for (int c = 0; c < C::NQC; ++c) {
      kreg[c] = key_ok ? *(const bf16x8*)(krow + 16 * c + 8 * g) : bf16x8{};
      vreg[c] = key_ok ? *(const bf16x8*)(vrow + 16 * c + 8 * g) : bf16x8{};
    }
  }
  const ElemConst ek = elem_const<NORM, CAP>(a);

  // positions: nheads query heads x query tiles [qt0, qt1)
  const int qt0 = ilo_g / C::BN;
  const int qt1 = ihi_g > ilo_g ? (ihi_g + C::BN - 1) / C::BN : qt0;
  const int ntq = qt1 - qt0;
  const int npos = nheads * ntq;
  RowDma<C> dq_, dd_;
  dq_.init(a.q_sl, wave, lane);
  dd_.init(w.do_sl, wave, lane);
  const uint32_t rec_bytes = (uint32_t)min(w.rec_bytes, (size_t)0xffffffffu);
  const i32x4 rr = rsrc_words(w.rec, rec_bytes);
  auto issue = [&](int stage, int u) __attribute__((always_inline)) {
    const bool live = u < npos;
    const int hh = live ? u / ntq : 0;
    const int qt = qt0 + (live ? u - hh * ntq : 0);
    const int h = h0 + hh;
    const i32x4 rq = rsrc_words((const bf16_t*)a.q + (int64_t)b * a.q_sb + (int64_t)h * a.q_sh,
                                (uint32_t)((int64_t)Lq * a.q_sl * 2));
    const i32x4 rd = rsrc_words((const bf16_t*)w.dout + (int64_t)b * w.do_sb + (int64_t)h * w.do_sh,
                                (uint32_t)((int64_t)Lq * w.do_sl * 2));
    dq_.issue(rq, qt_of(stage), qt * C::BN, live);
    dd_.issue(rd, dt_of(stage), qt * C::BN, live);
    // the record blocks of (b, h, qt), contiguous (the transfer's tail is unused)
    const int64_t blk = ((int64_t)b * a.Hq + h) * rec_blocks(Lq) + (int64_t)qt * (C::BN / kRecRows);
    const uint32_t so = live ? (uint32_t)(blk * (3 * kRecRows) * 4) : 0x80000000u;
    dma16(rr, lds_addr((const bf16_t*)(lds + stage * STAGE + 2 * QT * 2 + wave * 1024)),
          (uint32_t)lane * 16, __builtin_amdgcn_readfirstlane(so));
  };

  TrK<C> tr;
  tr.init(lane);

  // one gradient (dK or dV) of this lane's key: fp32 partial of this query
  // head ([B, Hq, Lk, D] for dK, then for dV) or the bf16 result
  auto store = [&](const f32x16* acc, bool is_v) __attribute__((always_inline)) {
    if (!key_ok) return;
    if (split) {
      const int64_t half = (int64_t)a.B * a.Hq * Lk * C::D;
      const int64_t prow = (is_v ? half : 0) + (((int64_t)b * a.Hq + h0) * Lk + myk) * C::D;
#pragma unroll
      for (int db = 0; db < C::NDB; ++db)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq)
          *(f32x4*)(w.part + prow + db * 32 + 8 * rq + 4 * g) =
              f32x4{acc[db][4 * rq], acc[db][4 * rq + 1], acc[db][4 * rq + 2], acc[db][4 * rq + 3]};
    } else {
      bf16_t* row = is_v ? (bf16_t*)w.dv + (int64_t)b * w.dv_sb + (int64_t)kvh * w.dv_sh + (int64_t)myk * w.dv_sl
                         : (bf16_t*)w.dk + (int64_t)b * w.dk_sb + (int64_t)kvh * w.dk_sh + (int64_t)myk * w.dk_sl;
#pragma unroll
      for (int db = 0; db < C::NDB; ++db)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          bf16x4 x4;
#pragma unroll
          for (int e = 0; e < 4; ++e) x4[e] = (bf16_t)acc[db][4 * rq + e];
          *(bf16x4*)(row + db * 32 + 8 * rq + 4 * g) = x4;
        }
    }
  };

  // one pass over the positions accumulating dK and / or dV (MODE 0 both,
  // 1 dV only, 2 dK only; the type of the argument carries MODE)
  auto run = [&](auto mode_c) __attribute__((always_inline)) {
    constexpr int MODE = decltype(mode_c)::value;
    constexpr bool DK = MODE != 1, DV = MODE != 2;
    f32x16 dk[DK ? C::NDB : 1], dv[DV ? C::NDB : 1];
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
      if (DK) dk[db] = f32x16{};
      if (DV) dv[db] = f32x16{};
    }
    issue(0, 0);
    wait_vmcnt<0>();
    lds_barrier();
    for (int u = 0; u < npos; ++u) {
      const int cur = u & 1;
      issue(cur ^ 1, u + 1);
      const int hh = u / ntq;
      const int qa = (qt0 + u - hh * ntq) * C::BN;  // first query of the tile
      if (wave_keys && qa < whi && qa + C::BN > wlo) {
        const bf16_t* ql = qt_of(cur);
        const bf16_t* dl = dt_of(cur);
        const float* rl = (const float*)((const char*)rec_lds + cur * STAGE);
        f32x16 s[C::NKB], dp[DK ? C::NKB : 1];
        qk_tile<C>(ql, kreg, l32, g, s);
        if (DK) qk_tile<C>(dl, vreg, l32, g, dp);
        // every (query, key) pair of the tile is visible unless the tile
        // reaches past the wave's bounds
        const bool edge = (qa < ilo_w1) || (qa + C::BN > ihi_w0);
        bf16x8 pp[2 * C::NKB], pd[2 * C::NKB];
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb) {
          float p16[16], d16[16];
#pragma unroll
          for (int rg = 0; rg < 4; ++rg) {
            const int qi = kb * 32 + 8 * rg + 4 * g;  // tile row of element r = 4 rg
            const float* rb = rl + kb * (3 * kRecRows) + 8 * rg + 4 * g;  // its record block (32 rows)
            const f32x4 m4 = *(const f32x4*)(rb);
            const f32x4 l4 = *(const f32x4*)(rb + kRecRows);
            const f32x4 c4 = *(const f32x4*)(rb + 2 * kRecRows);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = 4 * rg + e;
              const int i = qa + qi + e;
              const float okf = (!edge || (i >= ilo && i < ihi)) ? 1.f : 0.f;
              float p, wt, dsdraw;
              elem<NORM, CAP>(s[kb][r], m4[e], l4[e], ek, p, wt, dsdraw);
              p16[r] = okf * p;
              d16[r] = DK ? okf * (wt * (dp[DK ? kb : 0][r] - c4[e]) * dsdraw) : 0.f;
            }
          }
          if (DV) {
            pp[2 * kb] = p_operand(p16);
            pp[2 * kb + 1] = p_operand(p16 + 8);
          }
          if (DK) {
            pd[2 * kb] = p_operand(d16);
            pd[2 * kb + 1] = p_operand(d16 + 8);
          }
        }
#pragma unroll
        for (int db = 0; db < C::NDB; ++db)
#pragma unroll
          for (int t = 0; t < 2 * C::NKB; ++t) {
            if (DV) dv[DV ? db : 0] = mfma(tr.read(dl, t, db), pp[t], dv[DV ? db : 0]);
            if (DK) dk[DK ? db : 0] = mfma(tr.read(ql, t, db), pd[t], dk[DK ? db : 0]);
          }
      }
      wait_vmcnt<0>();
      lds_barrier();
    }
    wait_vmcnt<0>();
    if (DK) store(dk, false);
    if (DV) store(dv, true);
  };
  // D >= 128: dK and dV together with K and V do not fit the registers of
  // two waves per SIMD (D = 128) or of one (D = 256); two passes over the
  // tiles (dV from P, then dK from dS) instead, a quarter more matrix work
  if (C::D >= 128) {
    run(Mode<1>{});
    run(Mode<2>{});
  } else {
    run(Mode<0>{});
  }
}

// dK, dV of one kv head = the sum of its G query heads' partials, added in
// head order; one thread per 8 dims of one key row.
template <int D>
__global__ __launch_bounds__(256) void bwd_kv_reduce(BwdArgs w) {
  const FwdArgs& a = w.f;
  const int64_t n8 = (int64_t)a.B * a.Hkv * a.Lk * (D / 8);
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const int d8 = (int)(i % (D / 8));
  const int64_t row = i / (D / 8);  // (b * Hkv + kvh) * Lk + key
  const int key = (int)(row % a.Lk);
  const int64_t bk = row / a.Lk;
  const int kvh = (int)(bk % a.Hkv), b = (int)(bk / a.Hkv);
  const int64_t half = (int64_t)a.B * a.Hq * a.Lk * D;
  f32x4 k0 = {}, k1 = {}, v0 = {}, v1 = {};
  for (int hh = 0; hh < a.G; ++hh) {
    const int64_t src = (((int64_t)b * a.Hq + kvh * a.G + hh) * a.Lk + key) * D + d8 * 8;
    k0 += *(const f32x4*)(w.part + src);
    k1 += *(const f32x4*)(w.part + src + 4);
    v0 += *(const f32x4*)(w.part + half + src);
    v1 += *(const f32x4*)(w.part + half + src + 4);
  }
  bf16x8 ko, vo;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    ko[e] = (bf16_t)k0[e];
    ko[e + 4] = (bf16_t)k1[e];
    vo[e] = (bf16_t)v0[e];
    vo[e + 4] = (bf16_t)v1[e];
  }
  *(bf16x8*)((bf16_t*)w.dk + (int64_t)b * w.dk_sb + (int64_t)kvh * w.dk_sh + (int64_t)key * w.dk_sl + d8 * 8) = ko;
  *(bf16x8*)((bf16_t*)w.dv + (int64_t)b * w.dv_sb + (int64_t)kvh * w.dv_sh + (int64_t)key * w.dv_sl + d8 * 8) = vo;
}

template <int D, int NORM, bool CAP>
hipError_t launch_d(const BwdArgs& w, hipStream_t stream) {
  const FwdArgs& a = w.f;
  using CQ = Cfg<D, (D == 64 ? 64 : 32), 4>;   // query kernel: key tiles
  using CK = Cfg<D, (D == 256 ? 32 : 64), 4>;  // key kernel: query tiles
  const int nqb = (a.Lq + CQ::BM - 1) / CQ::BM;
  const int64_t gq = (int64_t)nqb * a.B * a.Hq;
  constexpr bool SOFT = NORM == ATTN_SOFTMAX || NORM == ATTN_SOFTMAX1;
  if (gq) {
    if (SOFT && w.have_out)
      bwd_query_mfma<CQ, NORM, CAP, SOFT><<<dim3((unsigned)gq), dim3(CQ::NT), 0, stream>>>(w);
    else
      bwd_query_mfma<CQ, NORM, CAP, false><<<dim3((unsigned)gq), dim3(CQ::NT), 0, stream>>>(w);
  }
  const int nkb = (a.Lk + 32 * CK::NW - 1) / (32 * CK::NW);
  const int64_t gk = (int64_t)nkb * a.B * (w.key_split ? a.Hq : a.Hkv);
  if (gk) {
    constexpr int lds = KeyLds<CK>::BYTES;
    const hipError_t e = hipFuncSetAttribute((const void*)bwd_key_mfma<CK, NORM, CAP>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    bwd_key_mfma<CK, NORM, CAP><<<dim3((unsigned)gk), dim3(CK::NT), lds, stream>>>(w);
    if (w.key_split) {
      const int64_t n8 = (int64_t)a.B * a.Hkv * a.Lk * (D / 8);
      bwd_kv_reduce<D><<<dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, stream>>>(w);
    }
  }
  return hipGetLastError();
}

template <int NORM>
hipError_t launch_n(const BwdArgs& w, hipStream_t stream) {
  const bool cap = w.f.softcap > 0.f;
  if (w.f.D == 64) return cap ? launch_d<64, NORM, true>(w, stream) : launch_d<64, NORM, false>(w, stream);
  if (w.f.D == 128) return cap ? launch_d<128, NORM, true>(w, stream) : launch_d<128, NORM, false>(w, stream);
  return cap ? launch_d<256, NORM, true>(w, stream) : launch_d<256, NORM, false>(w, stream);
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

}  // namespace

size_t bwd_mfma_rec_bytes(const FwdArgs& a) {
  return (size_t)a.B * a.Hq * rec_blocks(a.Lq) * 3 * kRecRows * sizeof(float);
}

bool bwd_key_split(const FwdArgs& a) {
  const int64_t nkb = (a.Lk + 127) / 128;
  return a.G > 1 && nkb * a.B * a.Hkv < 1024;
}

size_t bwd_mfma_part_bytes(const FwdArgs& a) {
  return bwd_key_split(a) ? (size_t)2 * a.B * a.Hq * a.Lk * a.D * sizeof(float) : 0;
}

bool bwd_mfma_supported(const BwdArgs& w) {
  const FwdArgs& a = w.f;
  if (a.dtype != ATTN_BF16 || (a.D != 64 && a.D != 128 && a.D != 256)) return false;
  if (a.paged || a.cu_q || a.bm_num) return false;
  if (!(a.scaling > 0.f)) return false;
  const void* ptrs[] = {a.q, a.k, a.v, w.dout, w.dq, w.dk, w.dv, w.have_out ? a.out : a.q};
  for (const void* p : ptrs)
    if (!aligned16(p)) return false;
  if (w.have_out && (a.o_sb % 8 || a.o_sh % 8 || a.o_sl % 8)) return false;
  const int64_t s[] = {a.q_sb, a.q_sh, a.q_sl, a.k_sb, a.k_sh, a.k_sl, a.v_sb, a.v_sh, a.v_sl,
                       w.do_sb, w.do_sh, w.do_sl, w.dq_sb, w.dq_sh, w.dq_sl,
                       w.dk_sb, w.dk_sh, w.dk_sl, w.dv_sb, w.dv_sh, w.dv_sl};
  for (int64_t x : s)
    if (x % 8) return false;
  // per-head slices and the record workspace are addressed through 32-bit
  // buffer records
  const int64_t lim = (int64_t)1 << 31;
  if ((int64_t)a.Lk * a.k_sl * 2 >= lim || (int64_t)a.Lk * a.v_sl * 2 >= lim) return false;
  if ((int64_t)a.Lq * a.q_sl * 2 >= lim || (int64_t)a.Lq * w.do_sl * 2 >= lim) return false;
  if ((int64_t)bwd_mfma_rec_bytes(a) >= lim) return false;
  const int64_t gq = (int64_t)((a.Lq + 127) / 128) * a.B * a.Hq;
  const int64_t gk = (int64_t)((a.Lk + 127) / 128) * a.B * a.Hq;
  const int64_t gr = ((int64_t)a.B * a.Hkv * a.Lk * (a.D / 8) + 255) / 256;
  return gq <= INT32_MAX && gk <= INT32_MAX && gr <= INT32_MAX;
}

hipError_t launch_bwd_mfma(const BwdArgs& w, hipStream_t stream) {
  switch (w.f.norm) {
    case ATTN_SOFTMAX: return launch_n<ATTN_SOFTMAX>(w, stream);
    case ATTN_SOFTMAX1: return launch_n<ATTN_SOFTMAX1>(w, stream);
    case ATTN_SPARSEMAX: return launch_n<ATTN_SPARSEMAX>(w, stream);
    default: return launch_n<ATTN_ENTMAX15>(w, stream);
  }
}

}  // namespace attn
