// Tiled bf16 prefill on the gfx950 matrix cores (v_mfma_f32_32x32x16_bf16).
//
// One workgroup owns BM = 32 * NW query rows of one (batch, query head); each
// wave owns 32 rows.  K/V tiles of BN keys go from global memory straight
// into LDS (two to three tiles in flight), shared by the waves.  Per tile and
// wave:
//
//   S^T (keys x queries) = K_tile . Q^T      A = K rows (LDS), B = Q (registers)
//   O^T (d x queries)   += V_tile^T . P^T    A = V^T (LDS),   B = P (registers)
//
// Computing the transposed products puts one query in each lane (lanes l and
// l+32 share query l%32 and hold complementary halves of its keys), so the
// row reductions of the normalizer are in-lane plus one exchange with the
// partner lane, and the probabilities P leave the S accumulators already in
// the register layout the PV product consumes.  The contraction of the PV
// product runs over keys: V stays row-major in LDS and its transposed operand
// comes from the transposing LDS read (ds_read_b64_tr_b16).
//
// Masking is computed, never stored: the workgroup visits only key tiles
// inside its causal / window bounds ("Attention variants": a kernel that
// skips blocks outside the window), a wave skips tiles its own 32 rows
// cannot see, and the per-element test runs only on tiles that straddle a
// bound.
//
// Normalizers: softmax and softmax1 use the online (running max, running
// sum) update; for softmax1 the "+1" enters as a virtual key with logit 0
// and value 0, i.e. the running max starts at 0 and the running sum at 1
// ("HF Attention Normalizers", "Important Limitations").

#include "tiles.h"

namespace attn {
namespace {

// Query-row extent of the grid: the longest packed request, or Lq.
__device__ __host__ __forceinline__ int q_extent(const FwdArgs& a) { return a.cu_q ? a.max_q : a.Lq; }

// The sequence of one workgroup: batch entry b, or packed request b.
struct SeqSpan {
  int Lq, Lk;                            // its query and key counts
  int64_t q_off, k_off, v_off, o_off;    // element offsets of its first query / key
  int64_t st_row;                        // row_stats row of its query 0 for head h
};
__device__ __forceinline__ SeqSpan seq_span(const FwdArgs& a, int b, int h) {
  SeqSpan s;
  if (a.paged) {  // chunked prefill: Lq queries align bottom-right against the sequence's keys
    s.Lq = a.Lq;
    s.Lk = paged_live(a, b);
    s.q_off = (int64_t)b * a.q_sb;
    s.k_off = 0;  // pages are addressed through the block table
    s.v_off = 0;
    s.o_off = (int64_t)b * a.o_sb;
    s.st_row = ((int64_t)b * a.Hq + h) * a.Lq;
  } else if (!a.cu_q) {
    s.Lq = a.Lq;
    s.Lk = a.Lk;
    s.q_off = (int64_t)b * a.q_sb;
    s.k_off = (int64_t)b * a.k_sb;
    s.v_off = (int64_t)b * a.v_sb;
    s.o_off = (int64_t)b * a.o_sb;
    s.st_row = ((int64_t)b * a.Hq + h) * a.Lq;
  } else {
    int q0, q1, k0, k1;
    varlen_ranges(a, b, q0, q1, k0, k1);
    s.Lq = q1 - q0;
    s.Lk = k1 - k0;
    s.q_off = (int64_t)q0 * a.q_sl;
    s.k_off = (int64_t)k0 * a.k_sl;
    s.v_off = (int64_t)k0 * a.v_sl;
    s.o_off = (int64_t)q0 * a.o_sl;
    s.st_row = (int64_t)h * a.Lq + q0;
  }
  return s;
}

// Lazy rescaling: the accumulators O and l are kept relative to a reference
// max m_use that only moves when the running max exceeds it by more than
// kRescale (log2 units), so most tiles skip the O *= alpha pass; weights
// stay <= 2^kRescale.  The true running max is tracked for row_stats.
constexpr float kRescale = 8.f;

// Paged K/V (chunked prefill through the block table).  One transfer covers
// 64 / CPR consecutive keys, which lie in one page when the block size is a
// multiple of 8 (checked on the host), so its page is wave-uniform: the
// page's byte offset goes in the scalar offset, and the descriptor's record
// count is cut at the sequence's last key, so the rows past it read as zeros
// (their cache slots may hold anything, NaN included).
struct PageCtx {
  const int32_t* row;  // block-table row of the sequence; nullptr for contiguous K/V
  int bs, max_blocks, nblk, Lk;
  uint32_t kpage, vpage;  // page strides in bytes
};

__device__ __forceinline__ i32x4 with_records(i32x4 r, uint32_t n) {
  r[2] = (int)n;
  return r;
}

template <class C>
struct DmaTiles {
  static constexpr int NI = C::KCH / 64 / C::NW;  // transfers per wave per K (and per V) tile
  static constexpr int ROWS = 64 / C::CPR;        // tile rows one transfer covers
  static_assert(C::KCH % (64 * C::NW) == 0, "K/V tile must split into 1 KB transfers per wave");
  static constexpr int PER_TILE = 2 * NI;         // vmcnt events per tile
  // Transfer i of a wave covers tile rows RSTEP i + (its rows of transfer 0).
  // The swizzles repeat every 16 rows (K) and 4 rows (V), so the lane's
  // offsets of transfer i are those of transfer i mod 2 (K) or 0 (V) plus
  // RSTEP i rows, which go to the scalar offset: three VGPRs instead of 2 NI.
  static constexpr int RSTEP = C::NW * ROWS;
  static_assert((2 * RSTEP) % 16 == 0 && RSTEP % 4 == 0, "swizzles must repeat across transfers");
  uint32_t ko0, ko1, vo0;                         // per-lane byte offsets (transfers 0, 1; V: 0)
  uint32_t kstr, vstr;
  int wave;                                       // wave-uniform

  __device__ __forceinline__ void init(int64_t ksl, int64_t vsl, int wave_u, int lane) {
    kstr = (uint32_t)(ksl * 2);
    vstr = (uint32_t)(vsl * 2);
    wave = wave_u;
    const int pos = wave * 64 + lane;  // LDS chunk this lane fills in transfer 0
    const int row = pos / C::CPR, pc = pos % C::CPR;
    ko0 = row * kstr + k_chunk<C::D>(row, pc) * 16;
    ko1 = row * kstr + k_chunk<C::D>(row + RSTEP, pc) * 16;
    vo0 = row * vstr + (pc ^ v_swz<C>(row)) * 16;
  }
  __device__ __forceinline__ uint32_t ko(int i) const { return (i & 1) ? ko1 : ko0; }
  // paged: byte offset of transfer i's first key and the records up to the
  // sequence's last key (0 when none of its keys is live)
  __device__ __forceinline__ void page_span(const PageCtx& pg, int key0, bool live, uint32_t kstride,
                                            uint32_t page_bytes, uint32_t& soff, uint32_t& nrec) const {
    const int valid = live ? min(max(pg.Lk - key0, 0), ROWS) : 0;
    soff = 0;
    nrec = 0;
    if (valid > 0) {
      // the table is read-only here: a constant-space read of a uniform index
      // is a scalar load (no vector-memory count shared with the transfers)
      const int idx = __builtin_amdgcn_readfirstlane(min(key0 / pg.bs, pg.max_blocks - 1));
      const int raw = ((const __attribute__((address_space(4))) int32_t*)pg.row)[idx];
      const int64_t page = min(max(raw, 0), pg.nblk - 1);
      soff = (uint32_t)(page * page_bytes) + (uint32_t)(key0 % pg.bs) * kstride;
      nrec = soff + (uint32_t)valid * kstride;
    }
    // wave-uniform by construction; made explicit for the scalar operands
    soff = __builtin_amdgcn_readfirstlane(soff);
    nrec = __builtin_amdgcn_readfirstlane(nrec);
  }
  __device__ __forceinline__ void issue_k(i32x4 rk, const bf16_t* kl, int k0, bool live,
                                          const PageCtx& pg) {
    const uint32_t kla = lds_addr(kl) + wave * 1024;
    if (!pg.row) {
      const uint32_t ks = live ? (uint32_t)k0 * kstr : 0x80000000u;
#pragma unroll
      for (int i = 0; i < NI; ++i) dma16(rk, kla + i * C::NW * 1024, ko(i), ks + (uint32_t)(i * RSTEP) * kstr);
    } else {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int r0 = (i * C::NW + wave) * ROWS;
        uint32_t ks, kn;
        page_span(pg, k0 + r0, live, kstr, pg.kpage, ks, kn);
        dma16(with_records(rk, kn), kla + i * C::NW * 1024, ko(i) - (uint32_t)(r0 - i * RSTEP) * kstr, ks);
      }
    }
  }
  __device__ __forceinline__ void issue(i32x4 rk, i32x4 rv, const bf16_t* kl, const bf16_t* vl, int k0,
                                        bool live, const PageCtx& pg) {
    const uint32_t kla = lds_addr(kl) + wave * 1024, vla = lds_addr(vl) + wave * 1024;
    if (!pg.row) {
      const uint32_t ks = live ? (uint32_t)k0 * kstr : 0x80000000u;
      const uint32_t vs = live ? (uint32_t)k0 * vstr : 0x80000000u;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        dma16(rk, kla + i * C::NW * 1024, ko(i), ks + (uint32_t)(i * RSTEP) * kstr);
        dma16(rv, vla + i * C::NW * 1024, vo0, vs + (uint32_t)(i * RSTEP) * vstr);
      }
    } else {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int r0 = (i * C::NW + wave) * ROWS;
        uint32_t ks, kn, vs, vn;
        page_span(pg, k0 + r0, live, kstr, pg.kpage, ks, kn);
        page_span(pg, k0 + r0, live, vstr, pg.vpage, vs, vn);
        dma16(with_records(rk, kn), kla + i * C::NW * 1024, ko(i) - (uint32_t)(r0 - i * RSTEP) * kstr, ks);
        dma16(with_records(rv, vn), vla + i * C::NW * 1024, vo0 - (uint32_t)(r0 - i * RSTEP) * vstr, vs);
      }
    }
  }
};

// Key tiles a workgroup visits, in order: the tiles [t0, t1) inside its
// causal / window bounds, or, under a block mask, the tiles of its query
// block's listed key blocks (sub tiles per block) that fall inside them.
// tile(u) is the tile at position u, or -1 where there is nothing to do (an
// entry the mask ignores, or a tile outside the bounds).  The lists are
// read-only here: constant-space reads of uniform indices are scalar loads.
struct TileSeq {
  const __attribute__((address_space(4))) int32_t* list;  // nullptr: contiguous
  int t0, t1, n, sub, nkb;
  __device__ __forceinline__ int tile(int u) const {
    if (!list) return t0 + u;
    const int e = u / sub;
    const int c = list[e];
    const bool ok = c >= 0 && c < nkb && (e == 0 || c > list[e - 1]);
    const int t = c * sub + (u - e * sub);
    return (ok && t >= t0 && t < t1) ? t : -1;
  }
};

template <class C>
__device__ __forceinline__ TileSeq tile_seq(const FwdArgs& a, int b, int h, int qb, int t0, int t1,
                                            int Lk) {
  TileSeq ts;
  ts.t0 = t0;
  ts.t1 = t1;
  ts.list = nullptr;
  ts.n = t1 - t0;
  ts.sub = 1;
  ts.nkb = 0;
  if (a.bm_num) {  // block_q == BM and block_k a multiple of BN (checked on the host)
    int n;
    const int64_t off = bm_list(a, b, h, qb, n);
    ts.list = (const __attribute__((address_space(4))) int32_t*)(a.bm_idx + off);
    ts.sub = a.bm_bk / C::BN;
    ts.n = n * ts.sub;
    ts.nkb = (Lk + a.bm_bk - 1) / a.bm_bk;
  }
  return ts;
}

__device__ __forceinline__ PageCtx page_ctx(const FwdArgs& a, int b, int Lk) {
  PageCtx pg;
  pg.row = a.paged ? a.block_table + (int64_t)b * a.max_blocks : nullptr;
  pg.bs = a.block_size;
  pg.max_blocks = a.max_blocks;
  pg.nblk = a.num_blocks;
  pg.Lk = Lk;
  pg.kpage = (uint32_t)(a.k_sb * 2);
  pg.vpage = (uint32_t)(a.v_sb * 2);
  return pg;
}

// V^T operand (32 dims x 16 keys) of PV step t and dim block db, read from a
// row-major V tile by two transposing LDS reads (ds_read_b64_tr_b16).  In each
// group of 16 lanes, source lane 4 j + q names 4 dims of key j and result
// lane i receives dim i of the 4 keys; the groups are placed so that lane
// (d, half g) ends with the keys 4g..4g+3 and 8+4g..8+4g+3 of the step, the
// keys its half of the P operand holds (S^T accumulator layout).
template <class C>
struct VTr {
  // The V swizzle only permutes 16-byte chunks within groups of four, so dim
  // block db reads at the offset of block db mod 4 plus (db / 4) * 256 bytes
  // (a constant of the LDS instruction): at most four VGPRs per lane.
  static constexpr int NO = C::NDB < 4 ? C::NDB : 4;
  uint32_t off[NO];  // byte offset of this lane's first read for step 0, dim blocks 0 .. NO - 1
  __device__ __forceinline__ void init(int lane) {
    const int G = lane >> 4, s = lane & 15, j = s >> 2, q = s & 3;
    const int r0 = 4 * (G >> 1) + j;
#pragma unroll
    for (int db = 0; db < NO; ++db) {
      const int lc = db * 4 + 2 * (G & 1) + (q >> 1);
      off[db] = (uint32_t)((r0 * C::D + (lc ^ v_swz<C>(r0)) * 8 + (q & 1) * 4) * 2);
    }
  }
  __device__ __forceinline__ bf16x8 read(const bf16_t* vl, int t, int db) const {
    const char* p = (const char*)vl + off[db & 3] + (db >> 2) * 256 + t * 16 * C::D * 2;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p);
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(p + 8 * C::D * 2));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  }
};

// GEN: paged K/V or a block mask (tile sequence and page lookups compiled in)
template <class C, int NBUF, int NORM, bool CAP, bool GEN>
__global__ __launch_bounds__(C::NT, C::D == 64 ? 4 : 2) void prefill_softmax_kernel(FwdArgs a) {
  static_assert(NBUF == 2 || NBUF == 3, "two or three tiles in flight");
  __shared__ __attribute__((aligned(16))) bf16_t lds[NBUF * 2 * C::BN * C::D];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  const int nqb = (q_extent(a) + C::BM - 1) / C::BM;
  int bh, qb;
  block_coords_lpt(nqb, bh, qb, a.paged || a.cu_q, a.Hq, a.Hkv);
  const int b = bh / a.Hq, h = bh - b * a.Hq, kvh = h / a.G;
  const int q0 = qb * C::BM;
  const SeqSpan sp = seq_span(a, b, h);
  if (q0 >= sp.Lq) return;  // packed request shorter than the longest one
  const int Lq = sp.Lq, Lk = sp.Lk;

  const bf16_t* qbase = (const bf16_t*)a.q + sp.q_off + (int64_t)h * a.q_sh;
  const bf16_t* kbase = (const bf16_t*)a.k + sp.k_off + (int64_t)kvh * a.k_sh;
  const bf16_t* vbase = (const bf16_t*)a.v + sp.v_off + (int64_t)kvh * a.v_sh;

  // key tiles the workgroup visits
  const int qlast = min(q0 + C::BM, Lq) - 1;
  const RowBounds first = row_bounds(q0, Lq, Lk, a.causal, a.window);
  const RowBounds last = row_bounds(qlast, Lq, Lk, a.causal, a.window);
  const int klo = first.lo, khi = last.hi;
  const int t0 = klo / C::BN;
  const int t1 = khi > klo ? (khi + C::BN - 1) / C::BN : t0;
  // LDS stage u: K [BN][D] then V [BN][D], both row-major and swizzled
  auto kl_of = [&](int u) { return lds + u * 2 * C::BN * C::D; };
  auto vl_of = [&](int u) { return lds + u * 2 * C::BN * C::D + C::BN * C::D; };

  // this wave's rows and this lane's row
  const int wq0 = q0 + 32 * wave;
  const int wq1 = min(wq0 + 31, Lq - 1);
  const bool wave_rows = wq0 < Lq;
  const RowBounds wfirst = row_bounds(wq0, Lq, Lk, a.causal, a.window);
  const RowBounds wlast = row_bounds(wq1, Lq, Lk, a.causal, a.window);
  const int myq = wq0 + l32;
  const bool row_ok = myq < Lq;
  const RowBounds mine = row_bounds(row_ok ? myq : wq1, Lq, Lk, a.causal, a.window);
  auto tile_active = [&](int t) {
    const int k0 = t * C::BN;
    return wave_rows && k0 < wlast.hi && k0 + C::BN > wfirst.lo;
  };

  bf16x8 qreg[C::NQC];
  {
    const bf16_t* qrow = qbase + (int64_t)myq * a.q_sl;
#pragma unroll
    for (int c = 0; c < C::NQC; ++c)
      qreg[c] = row_ok ? *(const bf16x8*)(qrow + 16 * c + 8 * g) : bf16x8{};
  }

  f32x16 o[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) o[db] = f32x16{};
  // log2-domain reference max (accumulators are relative to it) and true max
  // softmax1: the virtual key's logit b (0, or the head's learned sink) is
  // the initial max, and its weight exp(b - m) = 1 the initial sum
  const float sink2 = (NORM == ATTN_SOFTMAX1 && a.sinks) ? a.sinks[h] * kLog2e : 0.f;
  float m_use = (NORM == ATTN_SOFTMAX1) ? sink2 : -INFINITY;
  float m_true = m_use;
  float lsum = (NORM == ATTN_SOFTMAX1 && g == 0) ? 1.f : 0.f;
  const float c2 = a.scaling * kLog2e;
  const float sc_over_cap = CAP ? a.scaling / a.softcap : 0.f;
  const float cap_log2e = CAP ? a.softcap * kLog2e : 0.f;
  VTr<C> vtr;
  vtr.init(lane);

  // weights of one tile from its raw scores s, then O += V^T P^T
  auto consume = [&](f32x16 (&s)[C::NKB], int t, const bf16_t* vl) __attribute__((always_inline)) {
    const int k0 = t * C::BN;
    // (the V operands are read right before their products: held across the
    // softmax they would take the registers of a fourth wave per SIMD at
    // head dim 64)
    if (CAP) {
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = capped_log2(s[kb][r], sc_over_cap, cap_log2e);
    }
    if ((k0 + C::BN > wfirst.hi) || (k0 < wlast.lo)) {  // tile straddles a mask bound
      const int base = k0 + 4 * g - mine.lo;
      const unsigned span = (unsigned)(mine.hi - mine.lo);
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const unsigned off = (unsigned)(base + kb * 32 + 8 * (r >> 2) + (r & 3));
          s[kb][r] = off < span ? s[kb][r] : -INFINITY;
        }
    }
    // row max and (below) row sum in four independent chains: a single chain
    // of dependent instructions per tile stalls the wave
    float m4[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
    for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) m4[r & 3] = fmaxf(m4[r & 3], s[kb][r]);
    float mt = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]));
    mt = pair_max(mt);
    const float mt2 = CAP ? mt : mt * c2;
    m_true = fmaxf(m_true, mt2);
    const bool need = mt2 > m_use + kRescale;
    if (__any(need)) {
      // lanes that do not need it keep their reference (alpha = 1); a lane
      // whose reference is still -inf gets alpha = 0 (nothing accumulated yet)
      const float m_new = need ? mt2 : m_use;
      const float alpha = need ? __builtin_amdgcn_exp2f(m_use - m_new) : 1.f;
      m_use = m_new;
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) o[db] *= alpha;
    }
    const float mref = m_use == -INFINITY ? 0.f : m_use;
    float ps4[4] = {0.f, 0.f, 0.f, 0.f};
    bf16x8 pk[2 * C::NKB];
#pragma unroll
    for (int kb = 0; kb < C::NKB; ++kb) {
      float p[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        p[r] = CAP ? __builtin_amdgcn_exp2f(s[kb][r] - mref)
                   : __builtin_amdgcn_exp2f(fmaf(s[kb][r], c2, -mref));
        ps4[r & 3] += p[r];
      }
      pk[2 * kb] = p_operand(p);
      pk[2 * kb + 1] = p_operand(p + 8);
    }
    lsum += (ps4[0] + ps4[1]) + (ps4[2] + ps4[3]);
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int u = 0; u < 2 * C::NKB; ++u)
        o[db] = mfma(vtr.read(vl, u, db), pk[u], o[db]);
  };

  const i32x4 rk = rsrc_words(kbase, (uint32_t)((int64_t)Lk * a.k_sl * 2));
  const i32x4 rv = rsrc_words(vbase, (uint32_t)((int64_t)Lk * a.v_sl * 2));
  PageCtx pg = page_ctx(a, b, Lk);
  if (!GEN) pg.row = nullptr;
  DmaTiles<C> dma;
  dma.init(a.k_sl, a.v_sl, wave, lane);
  constexpr int kAhead = (NBUF - 2) * DmaTiles<C>::PER_TILE;  // transfers left in flight at a wait

  TileSeq ts = tile_seq<C>(a, b, h, qb, t0, t1, Lk);
  if (!GEN) {
    ts.list = nullptr;
    ts.n = t1 - t0;
  }
  auto tile_at = [&](int u) { return u < ts.n ? ts.tile(u) : -1; };
  // position u of the sequence lives in stage u % NBUF; positions 0 .. NBUF - 2 first
#pragma unroll
  for (int u = 0; u < NBUF - 1; ++u) {
    const int tt = tile_at(u);
    dma.issue(rk, rv, kl_of(u), vl_of(u), tt * C::BN, tt >= 0, pg);
  }
  // everything, the Q loads included: the compiler then knows Q is in
  // registers and places no vmcnt wait inside the loop
  wait_vmcnt<0>();
  lds_barrier();
  int cur = 0;
  for (int u = 0; u < ts.n; ++u) {
    // the stage of position u + NBUF - 1 held position u - 1, whose reads all
    // ended before the barrier that closed the previous step
    const int nxt = cur == 0 ? NBUF - 1 : cur - 1;
    const int tn = tile_at(u + NBUF - 1);
    dma.issue(rk, rv, kl_of(nxt), vl_of(nxt), tn * C::BN, tn >= 0, pg);
    const int t = ts.tile(u);
    if (t >= 0 && tile_active(t)) {
      f32x16 s[C::NKB];
      __builtin_amdgcn_s_setprio(2);  // keep the matrix cores fed while others do VALU work
      qk_tile<C>(kl_of(cur), qreg, l32, g, s);
      __builtin_amdgcn_s_setprio(0);
      consume(s, t, vl_of(cur));
    }
    wait_vmcnt<kAhead>();  // this wave's part of tile t + 1 has landed
    lds_barrier();
    cur = cur == NBUF - 1 ? 0 : cur + 1;
  }
  wait_vmcnt<0>();  // no transfer may outlive the workgroup's LDS

  // epilogue
  const float ltot = pair_sum(lsum);
  if (row_ok) {
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
    bf16_t* orow = (bf16_t*)a.out + sp.o_off + (int64_t)h * a.o_sh + (int64_t)myq * a.o_sl;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const u32x2 w = {pack_bf16(o[db][4 * rq] * inv, o[db][4 * rq + 1] * inv),
                         pack_bf16(o[db][4 * rq + 2] * inv, o[db][4 * rq + 3] * inv)};
        *(u32x2*)(orow + db * 32 + 8 * rq + 4 * g) = w;
      }
    }
    if (a.stats && g == 0) {
      float* st = a.stats + (sp.st_row + myq) * 2;
      const bool any_key = m_true != -INFINITY;
      st[0] = any_key ? m_true * (1.f / kLog2e) : -INFINITY;
      // denominator relative to the true max
      st[1] = any_key ? ltot * __builtin_amdgcn_exp2f(m_use - m_true) : 0.f;
    }
  }
}

// ---------------------------------------------------------------------------
// sparsemax and 1.5-entmax
//
// p = g(z - tau) with g(x) = max(x, 0) (sparsemax, z = s) or max(x, 0)^2
// (1.5-entmax, z = s / 2), tau fixed per row by sum_j g(z_j - tau) = 1
// ("HF Attention Normalizers", "Supported Normalizers"; "Important
// Limitations": stream K tiles, find one threshold per query row, then
// recompute the tiles for the weighted sum of V).
//
// Pass A streams the K tiles once.  Each row keeps a provable lower bound
// `floor` <= tau and, in LDS, every score seen so far that lies above it (the
// candidates; each lane keeps its own half of the row).  Valid lower bounds:
// max z - 1 (the top key alone already has weight 1 there), and the threshold
// of any subset of the row's scores (adding scores can only raise tau), which
// Michelot's step (sparsemax) or a Newton step from the left (1.5-entmax; g
// is convex) approaches from below.  When a lane's buffer fills, the row
// raises its floor by such steps over its candidates and drops those at or
// below it.  After the pass the candidates contain the support, and tau is
// the closed form over the candidate set once that value lies below every
// remaining candidate (then the set is exactly the support):
//   sparsemax: tau = (sum z - 1) / k
//   1.5-entmax: tau = mean - sqrt((1 - sum (z - mean)^2) / k).
// A row whose support does not fit its buffer is finished by extra passes
// over the K tiles that accumulate (count, sum, sum of squares, minimum)
// above its floor and step the floor until the closed form is consistent.
// Pass B recomputes the scores with the same instruction sequence (so every
// z is bit-identical) and accumulates g(z - tau) V; the weights already sum
// to one.
// ---------------------------------------------------------------------------

// LDS of the sparse kernel (dynamic): NA K stages for the threshold passes,
// then one candidate region per wave; the output pass either gathers V rows
// through the buffers or reuses all of the LDS for NB K/V stages.  Two
// workgroups per CU below D = 256 (their register use allows no more), one
// at D = 256.
//
// A wave's region holds, per lane, entry e at byte 256 e + 4 lane: the float
// value.  While the wave is "keyed" its entries stop at SCAP_K and each has a
// 16-bit key index at KEYS_OFF + 128 e + 2 lane; a wave whose candidates
// outgrow that drops the keys and uses the whole region for SCAP_F values
// (the first SCAP_K values stay where they are).
//
// Key indices (KEYS) are kept, with two K stages in pass A to leave room for
// them.  Where the running floors of pass A admit several times the support
// (broad scores: a fresh row's first floor, z max - 1, lies far below tau)
// the lookahead after the first tile starts the floors at their final
// values, so the keyed buffers do not overflow.
// The extra passes always stream K through NX = 3 stages: once a row is in
// them its wave has dropped the keys (the output runs on the matrix cores),
// so the candidate regions move behind the third stage (WREG_X, SCAP_X).
template <int N>
struct Stages {
  static constexpr int value = N;
};

template <class C, int NORM>
struct SparseCfg {
  static constexpr bool KEYS = true;               // candidates carry key indices at first
  static constexpr int LDS_BYTES = C::D == 256 ? 160 * 1024 : 80 * 1024;
  static constexpr int NA = KEYS ? 2 : 3;          // K tiles in flight, threshold passes
  static constexpr int NX = 3;                     // K tiles in flight, extra passes
  static constexpr int NB = 3;                     // K/V tiles in flight, output pass
  static constexpr int KTILE = C::BN * C::D * 2;   // bytes of one K (or V) tile
  static constexpr int WREG = (LDS_BYTES - NA * KTILE) / C::NW / 256 * 256;  // bytes per wave
  static constexpr int SCAP_F = WREG / 256 / 8 * 8;        // values per lane, no keys
  static constexpr int SCAP_K = WREG / 384 / 8 * 8;        // values per lane with keys
  static constexpr int KEYS_OFF = SCAP_K * 256;            // key indices, from the region start
  static constexpr int WREG_X = (LDS_BYTES - NX * KTILE) / C::NW / 256 * 256;
  static constexpr int SCAP_X = WREG_X / 256 / 8 * 8;      // values per lane, extra passes
  // histogram pass: 16-bit bin counts, two per word, 32 rows per wave
  static constexpr int NBIN = WREG_X / 64 < 256 ? WREG_X / 64 / 8 * 8 : 256;
  static_assert(NBIN >= 64 && NBIN * 64 <= WREG_X, "histogram bins must fit the wave's region");
  static_assert(KEYS_OFF + SCAP_K * 128 + 4 <= WREG, "keyed layout leaves the region's last word free");
  static_assert(NB * 2 * KTILE <= LDS_BYTES, "output pass stages must fit");
  static_assert(SCAP_K >= 32 && KEYS_OFF + SCAP_K * 128 <= WREG && SCAP_X >= 32 && SCAP_X <= SCAP_F,
                "candidate buffer too small");
  static_assert(NA <= NX, "extra passes take at least the stages of pass A");
};

typedef unsigned short u16;

__device__ __forceinline__ float max16(const f32x16& v) {
  float m = v[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) m = fmaxf(m, v[r]);
  return m;
}

// Max of z over one 32-key block.  Without softcap z = cz * raw is monotone
// under rounding, so z(max raw) is exact; the softcapped transform is taken
// per element.
template <bool CAP>
__device__ __forceinline__ float block_zmax(const f32x16& v, float cz, float sc_over_cap, float capz) {
  if (!CAP) return zval<false>(max16(v), cz, sc_over_cap, capz);
  float m = -INFINITY;
#pragma unroll
  for (int r = 0; r < 16; ++r) m = fmaxf(m, zval<true>(v[r], cz, sc_over_cap, capz));
  return m;
}

// Sets scores of keys outside this lane's row interval to -inf.  `base` is
// k0 + 4 * (lane / 32) - lo and `span` = hi - lo of the row.
template <class C>
__device__ __forceinline__ void mask_tile(f32x16* s, int base, int span) {
#pragma unroll
  for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const unsigned off = (unsigned)(base + kb * 32 + 8 * (r >> 2) + (r & 3));
      s[kb][r] = off < (unsigned)span ? s[kb][r] : -INFINITY;
    }
}

__device__ __forceinline__ double partner_d(double x) {
  const unsigned long long u = (unsigned long long)__double_as_longlong(x);
  const unsigned lo = (unsigned)u, hi = (unsigned)(u >> 32);
  const auto rl = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
  const auto rh = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
  const bool own0 = rl[0] == lo && rh[0] == hi;
  const unsigned plo = own0 ? rl[1] : rl[0], phi = own0 ? rh[1] : rh[0];
  return __longlong_as_double((long long)(((unsigned long long)phi << 32) | plo));
}
__device__ __forceinline__ int partner_i(int x) { return (int)partner_u((unsigned)x); }

// One step of the threshold search from lower bound t over the candidate set
// L = {z > t} with row totals (count c, sum and sum of squares of z - mref,
// smallest member mn).  Sets `exact` and returns tau when the closed form
// over L is consistent; otherwise returns a larger lower bound that drops at
// least the smallest member of L.
template <int NORM>
__device__ __forceinline__ double thr_step(double c, double s1, double s2, float mn, double mref,
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

// f(t) = sum over {z > t} of g(z - t) - 1 from the totals of that set about
// mref (count c, sums s1, s2 of z - mref), ty = t - mref.  f is convex and
// decreasing in t, positive below tau and not positive from tau on.
template <int NORM>
__device__ __forceinline__ double thr_f(double c, double s1, double s2, double ty) {
  return NORM == ATTN_SPARSEMAX ? s1 - c * ty - 1.0 : s2 - 2.0 * ty * s1 + c * ty * ty - 1.0;
}

// Largest float not above x.
__device__ __forceinline__ float float_floor(double x) {
  float f = (float)x;
  if ((double)f > x) {  // step one ulp towards -inf
    unsigned u = __float_as_uint(f);
    u = f > 0.f ? u - 1u : (f < 0.f ? u + 1u : 0x80000001u);
    f = __uint_as_float(u);
  }
  return f;
}

// Candidates are stored in the domain of the score test: the raw score q.k
// without softcap (z = fl(raw * cz) is monotone in raw, so a raw threshold
// decides z > floor exactly and the product is only formed when a candidate
// is read), z itself with softcap.
//
// Largest float r with fl(r * cz) <= f, for cz > 0: then, for every float
// raw, fl(raw * cz) > f exactly when raw > r.  Starts from f / cz (within an
// ulp or two of r) and steps by ulps with the same multiply the scores use.
__device__ __forceinline__ float next_up(float x) {
  const unsigned u = __float_as_uint(x);
  return x == 0.f ? __uint_as_float(1u) : __uint_as_float(x > 0.f ? u + 1u : u - 1u);
}
__device__ __forceinline__ float next_down(float x) {
  const unsigned u = __float_as_uint(x);
  return x == 0.f ? __uint_as_float(0x80000001u) : __uint_as_float(x > 0.f ? u - 1u : u + 1u);
}
__device__ __forceinline__ float raw_floor(float f, float cz) {
#pragma clang fp contract(off)
  if (!(f > -INFINITY) || !(f < INFINITY)) return f;  // -inf: every finite raw passes; +inf: none
  float r = f / cz;
  if (!(r > -INFINITY && r < INFINITY)) return -INFINITY;  // out of range: let everything through
  for (int i = 0; i < 8 && r * cz > f; ++i) r = next_down(r);
  if (r * cz > f) return -INFINITY;  // (cannot happen) stay on the safe side: admit more
  for (int i = 0; i < 8; ++i) {
    const float u = next_up(r);
    if (!(u * cz <= f)) break;
    r = u;
  }
  return r;
}

template <bool CAP>
__device__ __forceinline__ float stored_z(float v, float cz) {
#pragma clang fp contract(off)
  return CAP ? v : v * cz;
}

// Keeps this lane's candidates with z above t (compacting them) and returns
// their partial sums of y = z - mref.  Entries are read 8 at a time so their
// LDS latencies overlap (the capacities are multiples of 8, so the reads stay
// inside the lane's buffer); compaction only writes to slots already read.
// KEYED: the key indices move with their values.
template <bool CAP, bool KEYED>
__device__ __forceinline__ void scan_buf(float* buf, u16* kbuf, int& cnt, double t, double mref, float cz,
                                         double& c, double& s1, double& s2, float& mn) {
  int w = 0;
  c = s1 = s2 = 0.0;
  mn = INFINITY;
  for (int e0 = 0; e0 < cnt; e0 += 8) {
    float v[8], z[8];
    u16 key[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      v[j] = buf[(e0 + j) * 64];
      if (KEYED) key[j] = kbuf[(e0 + j) * 64];
      z[j] = stored_z<CAP>(v[j], cz);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (e0 + j < cnt && (double)z[j] > t) {
        buf[w * 64] = v[j];
        if (KEYED) kbuf[w * 64] = key[j];
        ++w;
        const double y = (double)z[j] - mref;
        c += 1.0;
        s1 += y;
        s2 += y * y;
        mn = fminf(mn, z[j]);
      }
    }
  }
  cnt = w;
}

// Keeps this lane's candidates above t, a threshold in the stored domain
// (compacting them in place).
template <bool KEYED>
__device__ __forceinline__ void compact_buf(float* buf, u16* kbuf, int& cnt, float t) {
  int w = 0;
  for (int e0 = 0; e0 < cnt; e0 += 8) {
    float z[8];
    u16 key[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      z[j] = buf[(e0 + j) * 64];
      if (KEYED) key[j] = kbuf[(e0 + j) * 64];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (e0 + j < cnt && z[j] > t) {
        buf[w * 64] = z[j];
        if (KEYED) kbuf[w * 64] = key[j];
        ++w;
      }
    }
  }
  cnt = w;
}

// Output of a row whose support is the contents of its two lanes' candidate
// buffers (value and key index per entry): both lanes walk the same entries,
// lane l32's first, then lane l32 + 32's, and each accumulates
// g(z - tau) * v over its half of the head dimension in fp32 (V rows are read
// through the key indices, and for a paged cache through the block table; no
// score is recomputed).  The weights sum to one up to rounding; the output
// is divided by the fp32 sum of the weights as they enter the sums (rounded
// to bf16 where entries are taken in pairs).
template <class C, int NORM, bool CAP>
__device__ __forceinline__ void gather_rows(const float* buf, const u16* kbuf, int cnt, int g, float tauf,
                                            float cz, const bf16_t* vbase, int64_t v_sl, int64_t v_sb,
                                            const PageCtx& pg, bf16_t* orow, bool row_ok) {
  constexpr int DH = C::D / 2;                  // dims of this lane
  constexpr int NV = DH / 8;                    // 16-byte pieces of its half row
  constexpr int U = C::D == 64 ? 4 : (C::D == 128 ? 2 : 1);  // entries in flight
  const int pc = partner_i(cnt);
  const int n0 = g ? pc : cnt;                  // entries of lane l32
  const int n = cnt + pc;
  const int lead = g ? -32 : 0;                 // lane l32's slot relative to this lane
  const bf16_t* const vcol = vbase + g * DH;
  float acc[DH];
#pragma unroll
  for (int d = 0; d < DH; ++d) acc[d] = 0.f;
  float wsum = 0.f;
  // weight and V row (this lane's half) of entry i (past the end: weight 0
  // and key 0, a row of this sequence whenever any lane of the wave has
  // entries)
  // (both LDS reads are unconditional, from an entry inside the buffers, so
  // that the entries of a group issue their reads back to back)
  auto fetch = [&](int i, float& pj, u32x4 (&wj)[NV]) __attribute__((always_inline)) {
    const bool ok = i < n;
    const int s0 = lead + i * 64, s1 = lead + 32 + (i - n0) * 64;
    const int slot = ok ? (i < n0 ? s0 : s1) : 0;
    const float v = buf[slot];
    const int kraw = kbuf[slot];
    const int key = ok ? kraw : 0;
    float pw;
    {
#pragma clang fp contract(off)
      const float d = stored_z<CAP>(v, cz) - tauf;
      pw = d > 0.f ? d : 0.f;
      if (NORM == ATTN_ENTMAX15) pw = pw * pw;
    }
    pj = ok ? pw : 0.f;
    int64_t off;
    if (pg.row) {
      const int64_t page = page_of(pg.row, min(key / pg.bs, pg.max_blocks - 1), pg.nblk);
      off = page * v_sb + (int64_t)(key % pg.bs) * v_sl;
    } else {
      off = (int64_t)((uint32_t)key * (uint32_t)v_sl);  // < 2^31: the slice fits a 32-bit buffer record
    }
    const u32x4* vr = (const u32x4*)(vcol + off);
#pragma unroll
    for (int c = 0; c < NV; ++c) wj[c] = vr[c];
  };
  // entries j, j + 1 taken together: the two weights rounded to bf16 (as the
  // matrix-core output rounds P; wsum sums the rounded weights) and, per dim,
  // the two entries' values side by side, so one bf16 dot product adds both
  // (exact bf16 products, fp32 sums)
  auto add_pair = [&](float p0, float p1, const u32x4 (&w0)[NV], const u32x4 (&w1)[NV])
                      __attribute__((always_inline)) {
    const unsigned pp = pack_bf16(p0, p1);
    wsum += __uint_as_float(pp << 16) + __uint_as_float(pp & 0xffff0000u);
    const bf16x2 pb = __builtin_bit_cast(bf16x2, pp);
#pragma unroll
    for (int c = 0; c < NV; ++c)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const unsigned a0 = w0[c][q], a1 = w1[c][q];
        // byte permutes (bytes 0-3 of the second operand, 4-7 of the first)
        const unsigned lo = __builtin_amdgcn_perm(a1, a0, 0x05040100u);  // dim 2q of both
        const unsigned hi = __builtin_amdgcn_perm(a1, a0, 0x07060302u);  // dim 2q + 1 of both
        acc[8 * c + 2 * q] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, lo), pb,
                                                             acc[8 * c + 2 * q], false);
        acc[8 * c + 2 * q + 1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, hi), pb,
                                                                 acc[8 * c + 2 * q + 1], false);
      }
  };
  if constexpr (U % 2 == 0) {
    // two groups of U entries in flight: the next group's reads are issued
    // before the current group is added
    float pa[U], pb[U];
    u32x4 wa[U][NV], wb[U][NV];
#pragma unroll
    for (int j = 0; j < U; ++j) fetch(j, pa[j], wa[j]);
    for (int e = 0; __any(e < n); e += 2 * U) {
#pragma unroll
      for (int j = 0; j < U; ++j) fetch(e + U + j, pb[j], wb[j]);
#pragma unroll
      for (int j = 0; j < U; j += 2) add_pair(pa[j], pa[j + 1], wa[j], wa[j + 1]);
      if (!__any(e + U < n)) break;
#pragma unroll
      for (int j = 0; j < U; ++j) fetch(e + 2 * U + j, pa[j], wa[j]);
#pragma unroll
      for (int j = 0; j < U; j += 2) add_pair(pb[j], pb[j + 1], wb[j], wb[j + 1]);
    }
  } else {
    for (int e = 0; __any(e < n); e += U) {
      float p[U];
      u32x4 w[U][NV];
#pragma unroll
      for (int j = 0; j < U; ++j) fetch(e + j, p[j], w[j]);
#pragma unroll
      for (int j = 0; j < U; ++j) {
        wsum += p[j];
#pragma unroll
        for (int c = 0; c < NV; ++c)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            acc[8 * c + 2 * q] += p[j] * __uint_as_float(w[j][c][q] << 16);
            acc[8 * c + 2 * q + 1] += p[j] * __uint_as_float(w[j][c][q] & 0xffff0000u);
          }
      }
    }
  }
  if (row_ok) {
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
#pragma unroll
    for (int c = 0; c < NV; ++c) {
      bf16x8 o;
#pragma unroll
      for (int q = 0; q < 8; ++q) o[q] = (bf16_t)(acc[8 * c + q] * inv);
      *(bf16x8*)(orow + g * DH + 8 * c) = o;
    }
  }
}

// GEN: paged K/V or a block mask (tile sequence and page lookups); without
// it both are compiled out of this register-heavy kernel.
template <class C, int NORM, bool CAP, bool GEN>
__global__ __launch_bounds__(C::NT, (C::D <= 128 ? 2 : 1)) void prefill_sparse_kernel(FwdArgs a) {
  using SC = SparseCfg<C, NORM>;
  extern __shared__ __attribute__((aligned(16))) bf16_t lds[];  // SC::LDS_BYTES
  constexpr int KT = C::BN * C::D;  // elements of one K or V tile
  auto ka_of = [&](int u) { return lds + u * KT; };  // threshold passes: K stage u
  auto kb_of = [&](int u) { return lds + u * 2 * KT; };  // output pass: K stage u ...
  auto vb_of = [&](int u) { return lds + u * 2 * KT + KT; };  // ... and its V

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  const int nqb = (q_extent(a) + C::BM - 1) / C::BM;
  int bh, qb;
  block_coords_lpt(nqb, bh, qb, a.paged || a.cu_q, a.Hq, a.Hkv);
  const int b = bh / a.Hq, h = bh - b * a.Hq, kvh = h / a.G;
  const int q0 = qb * C::BM;
  const SeqSpan sp = seq_span(a, b, h);
  if (q0 >= sp.Lq) return;  // packed request shorter than the longest one
  const int Lq = sp.Lq, Lk = sp.Lk;

  const bf16_t* qbase = (const bf16_t*)a.q + sp.q_off + (int64_t)h * a.q_sh;
  const bf16_t* kbase = (const bf16_t*)a.k + sp.k_off + (int64_t)kvh * a.k_sh;
  const bf16_t* vbase = (const bf16_t*)a.v + sp.v_off + (int64_t)kvh * a.v_sh;

  const int qlast = min(q0 + C::BM, Lq) - 1;
  const RowBounds first = row_bounds(q0, Lq, Lk, a.causal, a.window);
  const RowBounds last = row_bounds(qlast, Lq, Lk, a.causal, a.window);
  const int klo = first.lo, khi = last.hi;
  const int t0 = klo / C::BN;
  const int t1 = khi > klo ? (khi + C::BN - 1) / C::BN : t0;

  const int wq0 = q0 + 32 * wave;
  const int wq1 = min(wq0 + 31, Lq - 1);
  const bool wave_rows = wq0 < Lq;
  const RowBounds wfirst = row_bounds(wq0, Lq, Lk, a.causal, a.window);
  const RowBounds wlast = row_bounds(wq1, Lq, Lk, a.causal, a.window);
  const int myq = wq0 + l32;
  const bool row_ok = myq < Lq;
  const RowBounds mine = row_bounds(row_ok ? myq : wq1, Lq, Lk, a.causal, a.window);

  bf16x8 qreg[C::NQC];
  {
    const bf16_t* qrow = qbase + (int64_t)myq * a.q_sl;
#pragma unroll
    for (int c = 0; c < C::NQC; ++c)
      qreg[c] = row_ok ? *(const bf16x8*)(qrow + 16 * c + 8 * g) : bf16x8{};
  }

  const bool ent = (NORM == ATTN_ENTMAX15);
  const float cz = ent ? 0.5f * a.scaling : a.scaling;
  const float sc_over_cap = CAP ? a.scaling / a.softcap : 0.f;
  const float capz = CAP ? (ent ? 0.5f * a.softcap : a.softcap) : 0.f;

  // ---- pass A: row max, floor and candidates --------------------------------
  char* const region = (char*)(lds + SC::NA * KT) + wave * SC::WREG;
  float* buf = (float*)region + lane;  // moves for the extra passes
  u16* const kbuf = (u16*)(region + SC::KEYS_OFF) + lane;
  float mrun = -INFINITY;     // running max of z over the row (both lanes)
  double floor_ = -INFINITY;  // lower bound on tau (z units)
  float floor_f = -INFINITY;  // largest float <= floor_
  float floor_v = -INFINITY;  // the same test in the stored domain: v > floor_v <=> z > floor_f
  auto set_floor = [&](double f) __attribute__((always_inline)) {
    floor_ = f;
    floor_f = float_floor(f);
    floor_v = CAP ? floor_f : raw_floor(floor_f, cz);
  };
  int cnt = 0;                // this lane's candidates
  float cfloor = -INFINITY;   // floor_v at this lane's last compaction
  bool keyed = SC::KEYS;     // wave-uniform: the buffers carry key indices
  int cap = SC::KEYS ? SC::SCAP_K : SC::SCAP_F;  // wave-uniform: entries per lane
  auto scan = [&](double t, double mref, double& c, double& s1, double& s2, float& mn)
                  __attribute__((always_inline)) {
    if (SC::KEYS && keyed)
      scan_buf<CAP, true>(buf, kbuf, cnt, t, mref, cz, c, s1, s2, mn);
    else
      scan_buf<CAP, false>(buf, kbuf, cnt, t, mref, cz, c, s1, s2, mn);
  };
  bool ovf = !row_ok;         // row left to the extra passes (or no row at all)
  bool settled = false;       // floor has reached the exact threshold of the keys seen once
  // refloor steps are taken at most kMaxRefloors times per wave in pass A:
  // where most rows outgrow their buffers (large supports) every row's
  // overflow would otherwise re-run them for the whole wave, while the
  // extra passes finish such rows exactly anyway
  constexpr int kMaxRefloors = 4;
  // longest key range (per workgroup) that takes the lookahead below
  constexpr int kLookaheadKeys = 8192;
  // crowding below which a row skips the candidate pass (see the lookahead)
  constexpr float kCrowd = 0.15f;
  int nrefloor = 0;

  // The kTop largest lane-block maxima of z this lane has seen, descending.
  // Each is the z of one key, so the threshold of the row's 2 kTop such
  // values (both lanes) bounds tau from below -- and tightly, since the
  // support consists mostly of block maxima.  Sparsemax supports are
  // smaller than 1.5-entmax supports of the same scores, so its list is
  // shorter (cheaper to keep and to merge); a power of two for the merge.
  constexpr int kTop = NORM == ATTN_SPARSEMAX ? 4 : 8;
  float top[kTop];
#pragma unroll
  for (int i = 0; i < kTop; ++i) top[i] = -INFINITY;
  bool dirty = false;  // the list changed since the floor last used it
  auto push_top = [&](float v) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kTop; ++i) {  // compare-exchange chain keeps the list sorted
      const float hi = fmaxf(top[i], v);
      v = fminf(top[i], v);
      top[i] = hi;
    }
  };
  // Threshold of the row's 2 kTop listed values (both lanes): a lower bound
  // on tau.  The two descending lists merge into one (bitonic merge: own list
  // descending, partner's reversed), then the closed form over each prefix
  // of m largest values is consistent for the subset's support size, and the
  // largest consistent one is the subset's threshold (sparsemax: (S_m - 1) / m
  // with S_m the prefix sum; 1.5-entmax: mean - sqrt((1 - ss) / m) with ss the
  // prefix's sum of squared deviations, invalid once ss > 1, which only grows
  // with m).  Both lanes of a row see the same union, so they agree.
  //
  // With `crowd`, also the mass the listed values would take above the
  // smallest of them, sum of g(u_i - u_min) (+inf for a list that is not
  // full).  A small value means values crowd just below the list's
  // threshold: the support reaches far beyond the listed values.
  auto top_floor = [&](float* crowd = nullptr) __attribute__((always_inline)) -> double {
    constexpr int M = 2 * kTop;
    float u[M];
#pragma unroll
    for (int i = 0; i < kTop; ++i) {
      u[i] = top[i];
      u[M - 1 - i] = partner(top[i]);
    }
#pragma unroll
    for (int span = M / 2; span >= 1; span >>= 1)
#pragma unroll
      for (int i = 0; i < M; ++i)
        if ((i & span) == 0) {
          const float hi = fmaxf(u[i], u[i + span]), lo = fminf(u[i], u[i + span]);
          u[i] = hi;
          u[i + span] = lo;
        }
    if (crowd) {
      float r = 0.f;
#pragma unroll
      for (int i = 0; i < M - 1; ++i) {
        const float d = u[i] - u[M - 1];
        r += NORM == ATTN_SPARSEMAX ? d : d * d;
      }
      *crowd = u[M - 1] > -INFINITY ? r : INFINITY;
    }
    const double mref = (double)u[0];
    // closed form over the first m values, and whether it lies below the
    // m-th (then it is that subset's threshold)
    auto prefix_t = [&](int m, double s1, double s2, double y, bool& ok) __attribute__((always_inline)) {
      double t;
      ok = true;
      if (NORM == ATTN_SPARSEMAX) {
        t = (s1 - 1.0) / m;
      } else {
        const double mu = s1 / m;
        const double d = (1.0 - (s2 - s1 * mu)) / m;
        ok = d >= 0.0;
        t = ok ? mu - sqrt(d) : 0.0;
      }
      ok = ok && t < y;
      return t;
    };
    // The thresholds of the consistent prefixes grow with m, so the subset
    // threshold is taken at the largest prefix that passes the same test
    // multiplied through by m (no division or root per prefix): sparsemax
    // s1 - 1 < m y; 1.5-entmax, with q = m (1 - s2) + s1^2 = m^2 d,
    // q >= 0 and (s1 - m y)^2 < q (s1 - m y >= 0: y is the prefix's
    // smallest).  That prefix's closed form is then checked as before; if
    // rounding makes the two tests disagree, every prefix is tried.
    double s1 = 0.0, s2 = 0.0, s1s = 0.0, s2s = 0.0, ys = 0.0;
    int ms = 0;
#pragma unroll
    for (int m = 1; m <= M; ++m) {
      if (!(u[m - 1] > -INFINITY)) break;
      const double y = (double)u[m - 1] - mref;
      s1 += y;
      s2 += y * y;
      bool pass;
      if (NORM == ATTN_SPARSEMAX) {
        pass = s1 - 1.0 < m * y;
      } else {
        const double q = m * (1.0 - s2) + s1 * s1;
        if (q < 0.0) break;
        const double a = s1 - m * y;
        pass = a * a < q;
      }
      if (pass) {
        ms = m;
        s1s = s1;
        s2s = s2;
        ys = y;
      }
    }
    double best = -INFINITY;
    bool ok = false;
    if (ms > 0) {
      const double t = prefix_t(ms, s1s, s2s, ys, ok);
      if (ok) best = t;
    }
    if (ms > 0 && !ok) {
      s1 = s2 = 0.0;
      for (int m = 1; m <= M; ++m) {
        if (!(u[m - 1] > -INFINITY)) break;
        const double y = (double)u[m - 1] - mref;
        s1 += y;
        s2 += y * y;
        bool okm;
        const double t = prefix_t(m, s1, s2, y, okm);
        if (NORM != ATTN_SPARSEMAX && !(1.0 - (s2 - s1 * (s1 / m)) >= 0.0)) break;
        if (okm) best = fmax(best, t);
      }
    }
    return mref + best;
  };

  // Raises the floors until every row has room for a full block in both of
  // its lanes or its floor is the exact threshold of the keys seen so far
  // (then the buffer holds their support only, after one more compaction);
  // at most kRefloorSteps steps.  Wave-uniform: every lane takes part
  // (partner exchanges inside).
  constexpr int kRefloorSteps = 8;
  auto refloor = [&]() __attribute__((always_inline)) {
    bool done_ = ovf;
    for (int it = 0; it < kRefloorSteps; ++it) {
      double c, s1, s2;
      float mn;
      scan(floor_, (double)mrun, c, s1, s2, mn);
      c += partner_d(c);
      s1 += partner_d(s1);
      s2 += partner_d(s2);
      mn = fminf(mn, partner(mn));
      bool fresh = false;
      if (!done_ && c > 0.0) {
        bool ex;
        const double tn = thr_step<NORM>(c, s1, s2, mn, (double)mrun, floor_, ex);
        if (tn > floor_) set_floor(tn);
        done_ = fresh = ex;
        settled = settled || ex;
      } else {
        done_ = true;
      }
      const int pc = partner_i(cnt);
      const bool need = (cnt + 16 > cap || pc + 16 > cap) && (!done_ || fresh);
      if (!__any(need)) break;
    }
  };

  const i32x4 rk = rsrc_words(kbase, (uint32_t)((int64_t)Lk * a.k_sl * 2));
  const i32x4 rv = rsrc_words(vbase, (uint32_t)((int64_t)Lk * a.v_sl * 2));
  PageCtx pg = page_ctx(a, b, Lk);
  if (!GEN) pg.row = nullptr;
  DmaTiles<C> dma;
  dma.init(a.k_sl, a.v_sl, wave, lane);
  constexpr int NA = SC::NA;
  // K tiles t0 .. t0 + NA - 2 into stages 0 .. NA - 2; tile t sits in stage
  // (t - t0) mod NA.  Everything is waited for here, the Q loads included, so
  // that the compiler needs no vmcnt wait inside the loops.
  TileSeq ts = tile_seq<C>(a, b, h, qb, t0, t1, Lk);
  if (!GEN) {
    ts.list = nullptr;
    ts.n = t1 - t0;
  }
  auto tile_at = [&](int u) { return u < ts.n ? ts.tile(u) : -1; };
  // (the stage count NS comes in as the type of the first argument)
  auto k_prologue = [&](auto ns) __attribute__((always_inline)) {
    constexpr int NS = decltype(ns)::value;
#pragma unroll
    for (int u = 0; u < NS - 1; ++u) {
      const int tt = tile_at(u);
      dma.issue_k(rk, ka_of(u), tt * C::BN, tt >= 0, pg);
    }
    wait_vmcnt<0>();
    lds_barrier();
  };
  // start of step u: K of position u + NS - 1 into the stage position u - 1 left
  auto k_next = [&](auto ns, int u, int cur) __attribute__((always_inline)) {
    constexpr int NS = decltype(ns)::value;
    const int nxt = cur == 0 ? NS - 1 : cur - 1;
    const int tn = tile_at(u + NS - 1);
    dma.issue_k(rk, ka_of(nxt), tn * C::BN, tn >= 0, pg);
  };
  // end of step t: this wave's part of tile t + 1 has landed, then the barrier
  auto k_done = [&](auto ns, int& cur) __attribute__((always_inline)) {
    constexpr int NS = decltype(ns)::value;
    wait_vmcnt<(NS - 2) * DmaTiles<C>::NI>();
    lds_barrier();
    cur = cur == NS - 1 ? 0 : cur + 1;
  };
  constexpr Stages<NA> sa{};
  constexpr Stages<SC::NX> sx{};
  int cur = 0;
  // workgroup OR through one word of K stage 0, called only while no
  // transfer is in flight (the closing barrier keeps the next transfers from
  // landing before every wave has read it); the runtime's __syncthreads_or
  // would take static LDS on top of the dynamic allocation and cost the
  // second workgroup per CU
  int* const any_word = (int*)ka_of(0);
  auto block_any = [&](bool v) __attribute__((always_inline)) {
    __syncthreads();
    if (tid == 0) *(volatile int*)any_word = 0;
    __syncthreads();
    if (v) *(volatile int*)any_word = 1;
    __syncthreads();
    const bool r = *(volatile int*)any_word != 0;
    __syncthreads();
    return r;
  };
  bool run_a = true;    // workgroup-uniform: some row takes the candidate pass
  bool voted = false;   // workgroup-uniform: the waves posted crowding counts
  auto vote_word = [&](int w) __attribute__((always_inline)) {
    return (volatile int*)((char*)(lds + SC::NA * KT) + w * SC::WREG + SC::WREG - 4);
  };
  k_prologue(sa);
  cur = 0;
  if (ts.n > 1 && ts.n * C::BN <= kLookaheadKeys) {
    // Lookahead.  The first tile is scored for block maxima, and the
    // workgroup votes on whether its rows would crowd their buffers: some
    // lane has more than a quarter of its capacity in values above the first
    // floor the candidate pass would use (the tile's row max - 1).  If so,
    // the remaining tiles are scored for block maxima too, so that row
    // maxima and lists of block maxima cover every key and the candidate
    // pass starts from floors at their final values: far fewer candidates,
    // rows stay in their keyed buffers and the output is gathered.  Peaked
    // scores fail the vote; on longer key ranges the running floors settle
    // early anyway and the extra scoring pass would cost more than it saves.
    // Either way the lists are emptied afterwards (the candidate pass lists
    // each block once more) and the K stream restarts at the first tile.
    float mlook = -INFINITY;
    bool go = false;
    for (int p = 0; p < ts.n; ++p) {
      const bf16_t* kl = ka_of(cur);
      k_next(sa, p, cur);
      const int t = ts.tile(p);
      const int k0 = t * C::BN;
      f32x16 s[C::NKB];
      const bool active = t >= 0 && wave_rows && k0 < wlast.hi && k0 + C::BN > wfirst.lo;
      if (active) {
        qk_tile<C>(kl, qreg, l32, g, s);
        if ((k0 + C::BN > wfirst.hi) || (k0 < wlast.lo))
          mask_tile<C>(s, k0 + 4 * g - mine.lo, mine.hi - mine.lo);
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb) {
          const float z = block_zmax<CAP>(s[kb], cz, sc_over_cap, capz);
          mlook = fmaxf(mlook, z);
          if (z > top[kTop - 1]) push_top(z);
        }
      }
      if (p == 0) {
        // values of the first tile above its row max - 1
        const float m0 = pair_max(mlook);
        const double f0 = (double)m0 - 1.0;
        int n0 = 0;
        if (active) {
          const float f0v = CAP ? float_floor(f0) : raw_floor(float_floor(f0), cz);
#pragma unroll
          for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const float v = CAP ? zval<true>(s[kb][r], cz, sc_over_cap, capz) : s[kb][r];
              n0 += v > f0v ? 1 : 0;
            }
        }
        // workgroup vote through a word of the stage that held tile 0,
        // idle until the transfer issued at the next step
        k_done(sa, cur);
        int* const vote = (int*)ka_of(cur == 0 ? NA - 1 : cur - 1);
        if (tid == 0) *(volatile int*)vote = 0;
        wait_lgkm0();
        lds_barrier();
        if (row_ok && n0 * 4 > cap) *(volatile int*)vote = 1;
        wait_lgkm0();
        lds_barrier();
        go = *(volatile int*)vote != 0;
        wait_lgkm0();
        lds_barrier();
        if (!go) break;
      } else {
        k_done(sa, cur);
      }
    }
    wait_vmcnt<0>();
    if (go) {
      mrun = pair_max(mlook);
      float crowd;
      const double fl = fmax((double)mrun - 1.0, top_floor(&crowd));
      if (!ovf && fl > floor_) set_floor(fl);
      // A row whose listed block maxima crowd (they take less than kCrowd of
      // the unit mass above the smallest of them) has a support far larger
      // than its buffers.  Where most rows of the workgroup do, the
      // workgroup skips the candidate pass: every row goes to the histogram
      // and collecting passes at once (its output would run on the matrix
      // cores anyway); a few such rows alone keep the candidate pass, since
      // they would cost the whole workgroup its gathered output.  Each wave
      // posts its counts (crowded rows, rows; both lanes count) in the last
      // word of its candidate region, which the keyed layout leaves unused,
      // and the barrier that starts the candidate pass publishes them.
      if (Lk <= 65535) {
        const bool crowded = !ovf && crowd < kCrowd;
        const int nc = __popcll(__ballot(crowded)), nv = __popcll(__ballot(!ovf));
        if (lane == 0) *vote_word(wave) = (nc << 16) | nv;
        wait_lgkm0();  // the write lands before the barrier
        voted = true;
      }
    }
#pragma unroll
    for (int i = 0; i < kTop; ++i) top[i] = -INFINITY;
    // every wave is past the last barrier: no stage is being read
    k_prologue(sa);
    cur = 0;
    if (voted) {
      int votes = 0;
#pragma unroll
      for (int w = 0; w < C::NW; ++w) votes += *vote_word(w);
      if (__builtin_expect(2 * (votes >> 16) > (votes & 0xffff), 0)) {
        ovf = true;
        run_a = false;
      }
    }
  }
  for (int u = 0; run_a && u < ts.n; ++u) {
    const bf16_t* kl = ka_of(cur);
    k_next(sa, u, cur);
    const int t = ts.tile(u);
    const int k0 = t * C::BN;
    const bool active = t >= 0 && wave_rows && k0 < wlast.hi && k0 + C::BN > wfirst.lo;
    if (active) {
      f32x16 s[C::NKB];
      qk_tile<C>(kl, qreg, l32, g, s);
      if ((k0 + C::BN > wfirst.hi) || (k0 < wlast.lo))
        mask_tile<C>(s, k0 + 4 * g - mine.lo, mine.hi - mine.lo);
      // z is monotone in the raw score: per-block maxima decide whether a
      // block can hold a candidate at all
      float bz[C::NKB];
      float mt = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb) {
        bz[kb] = block_zmax<CAP>(s[kb], cz, sc_over_cap, capz);
        mt = fmaxf(mt, bz[kb]);
      }
      mt = pair_max(mt);
      if (mt > mrun) {
        mrun = mt;
        const double fl = (double)mrun - 1.0;
        if (fl > floor_) set_floor(fl);
      }
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb) {
        if (bz[kb] > top[kTop - 1]) {
          push_top(bz[kb]);
          dirty = true;
        }
      }
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb) {
        if (__any(bz[kb] > floor_f && !ovf)) {
          float v[16];  // stored-domain values of the block
#pragma unroll
          for (int r = 0; r < 16; ++r) v[r] = CAP ? zval<true>(s[kb][r], cz, sc_over_cap, capz) : s[kb][r];
          auto count = [&]() __attribute__((always_inline)) {
            int n = 0;
#pragma unroll
            for (int r = 0; r < 16; ++r) n += v[r] > floor_v ? 1 : 0;
            return n;
          };
          if (__any(!ovf && cnt + 16 > cap)) {
            int na = count();
            if (__any(!ovf && cnt + na > cap)) {
              // a lane cannot take the block: raise the floors from the lists
              // of block maxima and drop what fell below them ...
              if (__any(dirty)) {
                const double tf = top_floor();
                if (!ovf && tf > floor_) set_floor(tf);
                dirty = false;
              }
              // (a lane whose floor has not moved since its last compaction
              // holds nothing to drop)
              if (__any(floor_v != cfloor)) {
                if (SC::KEYS && keyed)
                  compact_buf<true>(buf, kbuf, cnt, floor_v);
                else
                  compact_buf<false>(buf, kbuf, cnt, floor_v);
                cfloor = floor_v;
              }
              na = count();
              // ... and, if that is not enough, step the floors on the buffers
              if (nrefloor < kMaxRefloors && __any(!ovf && cnt + na > cap)) {
                ++nrefloor;
                refloor();
                na = count();
              }
              // ... and, still short, give up the key indices for room
              if (SC::KEYS && keyed && __any(!ovf && cnt + na > cap)) {
                keyed = false;
                cap = SC::SCAP_F;
              }
            }
            // a row whose lanes cannot take the block goes to the extra passes
            const int full = (!ovf && cnt + na > cap) ? 1 : 0;
            if (__any(full)) ovf = ovf || (full | partner_i(full)) != 0;
          }
          if (!ovf) {
            // only the accepting lanes write: a 16-key block rarely holds
            // more than one or two candidates of a row, and the writes of a
            // value no lane accepts are skipped altogether
            const int kk = s_key(k0, kb, 0, g);  // key of value 0; value r adds s_key(0, 0, r, 0)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              if (v[r] > floor_v) {
                buf[cnt * 64] = v[r];
                if (SC::KEYS && keyed) kbuf[cnt * 64] = (u16)(kk + s_key(0, 0, r, 0));
                ++cnt;
              }
            }
          }
        }
      }
    }
    k_done(sa, cur);
  }
  wait_vmcnt<0>();

  // ---- exact threshold over the candidates ---------------------------------
  // the lists of block maxima give a floor that often is tau itself (when the
  // support is made of listed values), so most rows settle in one step
  if (__any(dirty)) {
    const double tf = top_floor();
    if (!ovf && tf > floor_) set_floor(tf);
  }
  double tau = INFINITY;
  int ksup = 0;
  bool done = !row_ok || mrun == -INFINITY || ovf;  // empty rows: tau = +inf, k = 0
  bool pending = row_ok && mrun != -INFINITY && ovf;  // left to the extra passes
  // the row's support is exactly the contents of its two lanes' buffers
  // (an empty row's are empty); false for a row solved from running totals
  bool inbuf = !ovf;
  for (int it = 0; it < 2 * SC::SCAP_F + 4; ++it) {
    if (!__any(!done)) break;
    double c, s1, s2;
    float mn;
    scan(floor_, (double)mrun, c, s1, s2, mn);
    c += partner_d(c);
    s1 += partner_d(s1);
    s2 += partner_d(s2);
    mn = fminf(mn, partner(mn));
    if (!done) {
      bool ex;
      const double tn = thr_step<NORM>(c, s1, s2, mn, (double)mrun, floor_, ex);
      if (ex) {
        tau = tn;
        ksup = (int)c;
        done = true;
      } else {
        if (tn > floor_) set_floor(tn);
      }
    }
  }
  if (!done) {  // cannot happen (each step drops a candidate); kept as a guard
    pending = true;
    inbuf = false;
  }

  // ---- extra passes for rows whose candidates outgrew the buffer -----------
  // The first (the histogram pass below) brackets each pending row's tau to
  // a few bins.  Each later pass re-streams the K tiles and, for every
  // pending row, both accumulates (count, sums, minimum) above the floor and
  // collects the values above it into the lane buffers.  When both halves
  // fit, the row is solved exactly from the buffers as above; otherwise the
  // totals give one threshold step and the next pass starts from the raised
  // floor.
  // Bracket of a pending row: floor_ <= tau <= ub.  Each pass also takes the
  // totals above hi (floor_ < hi <= ub, +inf at first) and collects only the
  // values in the window (floor_, hi].  When f(hi) <= 0 and the window fits,
  // the row is solved exactly from the window plus the totals above hi.
  // Otherwise the floor takes a left-Newton step (from hi as well when
  // f(hi) > 0), the secant through the best known points on both sides
  // bounds tau from above (f is convex), and the next window is the whole
  // bracket when a linear count model says it fits, else its lower part.
  double ub = (double)mrun;  // point with f(ub) = fub <= 0 known
  double fub = -1.0;         // (no key lies above the row max)
  double hi_ = INFINITY;     // window top of a pending row (z units)
  float hi_v = INFINITY;     // the same test in the stored domain
  auto set_hi = [&](double x) __attribute__((always_inline)) {
    hi_ = x;
    const float xf = float_floor(x);
    hi_v = CAP ? xf : raw_floor(xf, cz);
  };
  // Histogram pass: one K pass that brackets tau to a few bins before the
  // passes that collect.  A pending row counts its values above the floor
  // in NBIN bins of width w over (floor, E(NBIN)], E(b) = floor + b w and
  // E(NBIN) >= row max, as 16-bit counts n_b in LDS (both lanes of a row
  // add into the same words).  A value counted in bin b lies in
  // [E(b) - m, E(b + 1) + m], m = w / 1024 far above the rounding of the
  // bin index, so with g the normalizer's map (x+ or x+^2)
  //   f(E(b) - m) >= sum over b' > b  of n_b' g((b' - b) w) - 1,
  //   f(E(b) + m) <= sum over b' >= b of n_b' g((b' - b + 1) w) - 1,
  // integer sums (exact in fp64) times w or w^2.  The largest E(b) - m where
  // the first bound is positive lies below tau, the smallest E(b) + m where
  // the second is not positive lies at or above it, and the next pass
  // collects the few bins between the two.
  // Every wave takes part (barriers inside); `part` marks the rows that are
  // counted, and such a row's floor and window top move to the bracket.
  // Runs after a full pass over the keys (the row max is final); counts stay
  // below 2^16 while a row has fewer than 65536 keys.
  constexpr int NBIN = SC::NBIN;
  auto hist_pass = [&](bool part) __attribute__((always_inline)) {
    unsigned* const hist = (unsigned*)((char*)(lds + SC::NX * KT) + wave * SC::WREG_X);
    // (called where no candidate region or K stage is live)
    for (int i = lane; i < NBIN * 16 / 4; i += 64) ((u32x4*)hist)[i] = u32x4{0u, 0u, 0u, 0u};
    float invw = 0.f;
    bool use = false;
    if (part && floor_f > -INFINITY && mrun > floor_f) {
      float iw = (float)((double)NBIN / ((double)mrun - (double)floor_f));
      for (int i = 0; i < 4 && (double)floor_f + (double)NBIN / (double)iw < (double)mrun; ++i) iw = next_down(iw);
      use = iw > 0.f && iw < INFINITY && (double)floor_f + (double)NBIN / (double)iw >= (double)mrun;
      invw = iw;
    }
    unsigned* const hrow = hist + l32;  // word j of this row at hrow[32 j]: bins 2j (low half), 2j + 1
    k_prologue(sx);
    cur = 0;
    for (int u = 0; u < ts.n; ++u) {
      const bf16_t* kl = ka_of(cur);
      k_next(sx, u, cur);
      const int t = ts.tile(u);
      const int k0 = t * C::BN;
      const bool active = t >= 0 && wave_rows && k0 < wlast.hi && k0 + C::BN > wfirst.lo && __any(use);
      if (active) {
        f32x16 s[C::NKB];
        qk_tile<C>(kl, qreg, l32, g, s);
        const bool edge = (k0 + C::BN > wfirst.hi) || (k0 < wlast.lo);
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
#pragma clang fp contract(off)
            float v = CAP ? zval<true>(s[kb][r], cz, sc_over_cap, capz) : s[kb][r];
            if (edge) {
              const int key = s_key(k0, kb, r, g);
              if (key < mine.lo || key >= mine.hi) v = -INFINITY;
            }
            if (use && v > floor_v) {  // z > floor_f, so the bin position is >= 0
              const float z = stored_z<CAP>(v, cz);
              const int bi = min((int)((z - floor_f) * invw), NBIN - 1);
              atomicAdd(hrow + 32 * (bi >> 1), 1u << ((bi & 1) << 4));
            }
          }
        }
      }
      k_done(sx, cur);
    }
    wait_vmcnt<0>();
    if (use) {
      // walk down from the top bin; (N, P, Q) = sum over the bins above of
      // n, n d, n d^2 with d the distance in bins to the current bin
      const bool ent2 = NORM == ATTN_ENTMAX15;
      const double w = 1.0 / (double)invw, w2 = w * w;
      double N = 0.0, P = 0.0, Q = 0.0;
      int blo = -1, bhi = NBIN;
      for (int j0 = NBIN / 2 - 4; j0 >= 0 && blo < 0; j0 -= 4) {
        unsigned wd[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) wd[i] = hrow[32 * (j0 + i)];
#pragma unroll
        for (int i = 3; i >= 0; --i)
#pragma unroll
          for (int hf = 1; hf >= 0; --hf) {
            if (blo < 0) {
              const int bb = 2 * (j0 + i) + hf;
              Q += 2.0 * P + N;
              P += N;
              N += (double)((wd[i] >> (16 * hf)) & 0xffffu);
              const double flo = (ent2 ? Q * w2 : P * w) - 1.0;               // bound at E(bb) - m
              const double fhi = (ent2 ? (Q + 2.0 * P + N) * w2 : (P + N) * w) - 1.0;  // at E(bb) + m
              if (fhi <= 0.0) bhi = bb;
              if (flo > 0.0) blo = bb;
            }
          }
      }
      const double m = w * (1.0 / 1024.0), base = (double)floor_f;
      if (blo >= 0 && base + blo * w - m > floor_) set_floor(base + blo * w - m);
      if (bhi < NBIN) set_hi(base + bhi * w + m);
    }
  };

  // (the extra passes are marked unlikely so that register allocation
  // favours the candidate pass; most workgroups never enter them)
  if (__builtin_expect(Lk <= 65535 && block_any(pending), 0)) hist_pass(pending);

  bool first_x = true;
  while (__builtin_expect(block_any(pending), 0)) {
    if (SC::NX != NA && first_x) {
      // pass A's buffers are dead: a wave with a pending row has dropped its
      // keys, so the output runs on the matrix cores
      first_x = false;
      buf = (float*)((char*)(lds + SC::NX * KT) + wave * SC::WREG_X) + lane;
      keyed = false;
      cap = SC::SCAP_X - 1;  // the last entry takes values that are not kept
      cnt = 0;
    }
    // Totals above the floor and above hi, and the window values (floor, hi]
    // into the lane's buffer, without branches per value: every value takes
    // the same instructions (masked operands; a window value that is not
    // kept is written to the buffer's last entry, which holds no candidate
    // here).
    double s1 = 0.0, s2 = 0.0, s1h = 0.0, s2h = 0.0;  // sums of y = z - mref
    float mn = INFINITY, mnh = INFINITY;
    int na = 0, nh = 0;  // counts above the floor, above hi
    const double mref = (double)mrun;
    if (pending) cnt = 0;  // solved rows keep their support
    int fits = pending ? 1 : 0;
    constexpr int kSpare = SC::SCAP_X - 1;  // entry that takes the values not kept
    k_prologue(sx);
    cur = 0;
    for (int u = 0; u < ts.n; ++u) {
      const bf16_t* kl = ka_of(cur);
      k_next(sx, u, cur);
      const int t = ts.tile(u);
      const int k0 = t * C::BN;
      const bool active = t >= 0 && wave_rows && k0 < wlast.hi && k0 + C::BN > wfirst.lo && __any(pending);
      if (active) {
        f32x16 s[C::NKB];
        qk_tile<C>(kl, qreg, l32, g, s);
        const bool edge = (k0 + C::BN > wfirst.hi) || (k0 < wlast.lo);
        const bool collect = __any(fits != 0);  // some row still keeps its window
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float v = CAP ? zval<true>(s[kb][r], cz, sc_over_cap, capz) : s[kb][r];
            if (edge) {
              const int key = s_key(k0, kb, r, g);
              if (key < mine.lo || key >= mine.hi) v = -INFINITY;
            }
            const float z = stored_z<CAP>(v, cz);
            const bool above = pending && v > floor_v;  // z > floor_
            const bool top = above && v > hi_v;
            const double y = (double)z - mref;
            const double ya = above ? y : 0.0, yh = top ? y : 0.0;
            na += above ? 1 : 0;
            s1 += ya;
            s2 += ya * ya;
            mn = fminf(mn, above ? z : INFINITY);
            nh += top ? 1 : 0;
            s1h += yh;
            s2h += yh * yh;
            mnh = fminf(mnh, top ? z : INFINITY);
            if (collect) {
              const bool want = above && !top && fits != 0;
              const bool keep = want && cnt < cap;
              fits = want && !keep ? 0 : fits;
              buf[(keep ? cnt : kSpare) * 64] = v;
              cnt += keep ? 1 : 0;
            }
          }
        }
      }
      k_done(sx, cur);
    }
    wait_vmcnt<0>();
    double c = (double)na, ch = (double)nh;
    c += partner_d(c);
    s1 += partner_d(s1);
    s2 += partner_d(s2);
    mn = fminf(mn, partner(mn));
    ch += partner_d(ch);
    s1h += partner_d(s1h);
    s2h += partner_d(s2h);
    mnh = fminf(mnh, partner(mnh));
    fits = fits & partner_i(fits);
    const double fh = hi_ < INFINITY ? thr_f<NORM>(ch, s1h, s2h, hi_ - mref) : -1.0;
    bool solving = pending && fits && fh <= 0.0;
    if (pending && !solving) {
      bool ex;
      const double tn = thr_step<NORM>(c, s1, s2, mn, mref, floor_, ex);
      if (ex) {
        tau = tn;
        ksup = (int)c;
        pending = false;
        cnt = 0;
      } else {
        double lo = fmax(tn, floor_);
        double tl = floor_, fl = thr_f<NORM>(c, s1, s2, floor_ - mref);  // best point below tau
        bool ex2 = false;
        if (fh > 0.0) {  // hi lies below tau
          const double tn2 = thr_step<NORM>(ch, s1h, s2h, mnh, mref, hi_, ex2);
          if (ex2) {
            tau = tn2;
            ksup = (int)ch;
            pending = false;
            cnt = 0;
          } else {
            lo = fmax(lo, fmax(tn2, hi_));
            tl = hi_;
            fl = fh;
          }
        } else if (hi_ < ub) {
          ub = hi_;
          fub = fh;
        }
        if (!ex2) {
          // secant through (tl, fl > 0) and (ub, fub <= 0): an upper bound on tau
          double top = ub;
          if (fl > fub) {
            const double sec = tl + fl * (ub - tl) / (fl - fub);
            if (sec >= lo && sec < top) top = sec;
          }
          // row counts above the floor and above hi (or none above the max),
          // linear in between: the estimated count of (lo, top]
          const double ta = floor_, tb = hi_ < INFINITY ? hi_ : mref;
          const double cb = hi_ < INFINITY ? ch : 0.0;
          const double est = tb > ta ? (c - cb) * (top - lo) / (tb - ta) : c;
          const double budget = 1.5 * cap;  // two lanes' buffers, with a margin for imbalance
          set_floor(lo);
          set_hi(est <= budget ? top : lo + (top - lo) * (budget / est));
        }
      }
    }
    for (int it = 0; it < 2 * SC::SCAP_F + 4; ++it) {
      if (!__any(solving)) break;
      double cc, a1, a2;
      float m1;
      scan(floor_, mref, cc, a1, a2, m1);
      cc += partner_d(cc);
      a1 += partner_d(a1);
      a2 += partner_d(a2);
      m1 = fminf(m1, partner(m1));
      if (solving) {
        // the window's values above the floor plus everything above hi
        cc += ch;
        a1 += s1h;
        a2 += s2h;
        m1 = fminf(m1, mnh);
        bool ex;
        const double tn = thr_step<NORM>(cc, a1, a2, m1, mref, floor_, ex);
        if (ex) {
          tau = tn;
          ksup = (int)cc;
          solving = false;
          pending = false;
          inbuf = true;
        } else if (tn > hi_) {
          // a step never passes tau, so hi lay below it after all (f(hi)
          // within rounding of 0): hi is a floor; the passes go on
          set_floor(hi_);
          set_hi(INFINITY);
          ub = mref;
          fub = -1.0;
          solving = false;
          cnt = 0;
        } else {
          if (tn > floor_) set_floor(tn);
        }
      }
    }
  }

  // ---- pass B: weighted sum of V ------------------------------------------------
  const float tauf = (float)tau;
  bf16_t* const orow = (bf16_t*)a.out + sp.o_off + (int64_t)h * a.o_sh + (int64_t)myq * a.o_sl;
  if (row_ok && a.stats && g == 0) {
    float* st = a.stats + (sp.st_row + myq) * 2;
    st[0] = (float)tau;
    st[1] = (float)ksup;
  }
  // When the support of every row of the workgroup sits in the buffers (and
  // the keys fit their 16-bit indices), the output gathers the V rows of the
  // support; otherwise the scores are recomputed tile by tile and the
  // weighted sum runs on the matrix cores.
  if (SC::KEYS && Lk <= 65536 && !block_any(!keyed || (row_ok && !inbuf))) {
    gather_rows<C, NORM, CAP>(buf, kbuf, cnt, g, tauf, cz, vbase, a.v_sl, a.v_sb, pg, orow, row_ok);
    return;
  }
  // the weights sum to one; the output is divided by the sum of their
  // bf16-rounded values, which cancels most of the rounding of P
  float wsum = 0.f;
  f32x16 o[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) o[db] = f32x16{};
  // the candidate buffers are dead once every wave is past its solve
  lds_barrier();
  constexpr int NB = SC::NB;
  VTr<C> vtr;
  vtr.init(lane);
#pragma unroll
  for (int u = 0; u < NB - 1; ++u) {
    const int tt = tile_at(u);
    dma.issue(rk, rv, kb_of(u), vb_of(u), tt * C::BN, tt >= 0, pg);
  }
  wait_vmcnt<0>();
  lds_barrier();
  cur = 0;
  for (int u = 0; u < ts.n; ++u) {
    const bf16_t* kl = kb_of(cur);
    const bf16_t* vl = vb_of(cur);
    {
      const int nxt = cur == 0 ? NB - 1 : cur - 1;
      const int tn = tile_at(u + NB - 1);
      dma.issue(rk, rv, kb_of(nxt), vb_of(nxt), tn * C::BN, tn >= 0, pg);
    }
    const int t = ts.tile(u);
    const int k0 = t * C::BN;
    const bool active = t >= 0 && wave_rows && k0 < wlast.hi && k0 + C::BN > wfirst.lo;
    if (active) {
      f32x16 s[C::NKB];
      qk_tile<C>(kl, qreg, l32, g, s);
      const bool edge = (k0 + C::BN > wfirst.hi) || (k0 < wlast.lo);
      bf16x8 pk[2 * C::NKB];
      bool any = false;
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb) {
        float p[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
#pragma clang fp contract(off)
          float z = zval<CAP>(s[kb][r], cz, sc_over_cap, capz);
          if (edge) {
            const int key = s_key(k0, kb, r, g);
            if (key < mine.lo || key >= mine.hi) z = -INFINITY;
          }
          const float d = z - tauf;
          p[r] = d > 0.f ? d : 0.f;
          if (ent) p[r] = p[r] * p[r];
          any |= p[r] > 0.f;
        }
        pk[2 * kb] = p_operand(p);
        pk[2 * kb + 1] = p_operand(p + 8);
      }
      // sum of the bf16-rounded weights (a bf16 is the high half of its float)
#pragma unroll
      for (int u = 0; u < 2 * C::NKB; ++u) {
        const u32x4 w = __builtin_bit_cast(u32x4, pk[u]);
#pragma unroll
        for (int e = 0; e < 4; ++e) wsum += __uint_as_float(w[e] << 16) + __uint_as_float(w[e] & 0xffff0000u);
      }
      if (__any(any)) {
#pragma unroll
        for (int db = 0; db < C::NDB; ++db)
#pragma unroll
          for (int u = 0; u < 2 * C::NKB; ++u) o[db] = mfma(vtr.read(vl, u, db), pk[u], o[db]);
      }
    }
    wait_vmcnt<(NB - 2) * DmaTiles<C>::PER_TILE>();
    lds_barrier();
    cur = cur == NB - 1 ? 0 : cur + 1;
  }
  wait_vmcnt<0>();  // no transfer may outlive the workgroup's LDS

  const float wtot = wsum + partner(wsum);
  if (row_ok) {
    const float inv = wtot > 0.f ? 1.f / wtot : 0.f;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (bf16_t)(o[db][4 * rq + e] * inv);
        *(bf16x4*)(orow + db * 32 + 8 * rq + 4 * g) = w;
      }
    }
  }
}

// K/V tiles in flight per workgroup (LDS: NBUF * 2 * BN * D * 2 bytes; two
// keep four workgroups per CU at head dim 64, two at 128 and 256)
template <class C>
constexpr int kStages = 2;

template <class C, int NORM>
hipError_t launch_cfg(const FwdArgs& a, hipStream_t stream) {
  const int nqb = (q_extent(a) + C::BM - 1) / C::BM;
  dim3 grid((unsigned)(nqb * a.B * a.Hq)), block(C::NT);
  const bool cap = a.softcap > 0.f;
  if constexpr (NORM == ATTN_SPARSEMAX || NORM == ATTN_ENTMAX15) {
    constexpr int lds = SparseCfg<C, NORM>::LDS_BYTES;
    auto go = [&](auto kern) {
      hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
      if (e != hipSuccess) return e;
      kern<<<grid, block, lds, stream>>>(a);
      return hipGetLastError();
    };
    if (a.paged || a.bm_num)
      return cap ? go(prefill_sparse_kernel<C, NORM, true, true>) : go(prefill_sparse_kernel<C, NORM, false, true>);
    return cap ? go(prefill_sparse_kernel<C, NORM, true, false>) : go(prefill_sparse_kernel<C, NORM, false, false>);
  } else {
    const bool gen = a.paged || a.bm_num;
    if (gen && cap)
      prefill_softmax_kernel<C, kStages<C>, NORM, true, true><<<grid, block, 0, stream>>>(a);
    else if (gen)
      prefill_softmax_kernel<C, kStages<C>, NORM, false, true><<<grid, block, 0, stream>>>(a);
    else if (cap)
      prefill_softmax_kernel<C, kStages<C>, NORM, true, false><<<grid, block, 0, stream>>>(a);
    else
      prefill_softmax_kernel<C, kStages<C>, NORM, false, false><<<grid, block, 0, stream>>>(a);
  }
  return hipGetLastError();
}

template <int NORM>
hipError_t launch_norm(const FwdArgs& a, hipStream_t stream) {
  switch (a.D) {
    case 64: return launch_cfg<Cfg<64, 64, 4>, NORM>(a, stream);
    case 128:
      // the sparse kernel takes 32-key tiles: more LDS left for candidates
      if constexpr (NORM == ATTN_SPARSEMAX || NORM == ATTN_ENTMAX15)
        return launch_cfg<Cfg<128, 32, 4>, NORM>(a, stream);
      else
        return launch_cfg<Cfg<128, 64, 4>, NORM>(a, stream);
    default: return launch_cfg<Cfg<256, 32, 4>, NORM>(a, stream);
  }
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

}  // namespace

bool prefill_mfma_supported(const FwdArgs& a) {
  if (a.dtype != ATTN_BF16) return false;
  // block masks: one query block per workgroup, key blocks of whole tiles
  if (a.bm_num && (a.bm_bq != 128 || a.bm_bk % 64 != 0)) return false;
  if (a.paged) {
    // chunked prefill: a transfer's keys must share a page, and every page
    // offset must fit the 32-bit buffer offsets
    if (a.Lq < 2 || a.block_size % 8 != 0) return false;
    if ((int64_t)a.num_blocks * a.k_sb * 2 >= ((int64_t)1 << 32) ||
        (int64_t)a.num_blocks * a.v_sb * 2 >= ((int64_t)1 << 32))
      return false;
    if (a.k_sl < a.D || a.v_sl < a.D) return false;
    if ((int64_t)a.block_size * a.k_sl > a.k_sb || (int64_t)a.block_size * a.v_sl > a.v_sb) return false;
  }
  if (a.D != 64 && a.D != 128 && a.D != 256) return false;
  if (!(a.scaling > 0.f)) return false;
  if (!aligned16(a.q) || !aligned16(a.k) || !aligned16(a.v) || !aligned16(a.out)) return false;
  const int64_t s[] = {a.q_sb, a.q_sh, a.q_sl, a.k_sb, a.k_sh, a.k_sl,
                       a.v_sb, a.v_sh, a.v_sl, a.o_sb, a.o_sh, a.o_sl};
  for (int64_t x : s)
    if (x % 8) return false;
  // K/V slices are addressed through 32-bit buffer records
  if (!a.paged &&
      ((int64_t)a.Lk * a.k_sl * 2 >= ((int64_t)1 << 31) || (int64_t)a.Lk * a.v_sl * 2 >= ((int64_t)1 << 31)))
    return false;
  const int nqb_min = (q_extent(a) + 127) / 128;
  return (int64_t)nqb_min * a.B * a.Hq <= (int64_t)INT32_MAX;
}

hipError_t launch_prefill_mfma(const FwdArgs& a, hipStream_t stream) {
  switch (a.norm) {
    case ATTN_SOFTMAX: return launch_norm<ATTN_SOFTMAX>(a, stream);
    case ATTN_SOFTMAX1: return launch_norm<ATTN_SOFTMAX1>(a, stream);
    case ATTN_SPARSEMAX: return launch_norm<ATTN_SPARSEMAX>(a, stream);
    default: return launch_norm<ATTN_ENTMAX15>(a, stream);
  }
}

}  // namespace attn
