// Building blocks shared by the matrix-core kernels (forward prefill and
// backward): bf16 vector types, the tile configuration, the 32x32x16 bf16
// MFMA, partner-lane exchanges, the K-row LDS swizzle, row bounds of the
// causal / window mask, the score tile S^T = K Q^T, bf16 packing of a
// weight tile into the PV operand, the softcap transform, and the direct
// global -> LDS transfers with their explicit waits and barrier.
#pragma once

#include "common.h"

namespace attn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

template <int D_, int BN_, int NW_>
struct Cfg {
  static constexpr int D = D_, BN = BN_, NW = NW_;
  static constexpr int NT = NW * 64;          // threads per workgroup
  static constexpr int BM = NW * 32;          // query rows per workgroup
  static constexpr int CPR = D / 8;           // 16-byte chunks per K/V row
  static constexpr int KCH = BN * CPR;        // chunks per K tile
  static constexpr int NKB = BN / 32;         // 32-key blocks per tile
  static constexpr int NDB = D / 32;          // 32-dim blocks of the output
  static constexpr int NQC = D / 16;          // 16-dim steps of QK^T
  static_assert(CPR >= 8, "head dim must be >= 64");
  static_assert(BN % 32 == 0, "BN must be a multiple of 32");
};

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Value held by the partner lane (l ^ 32), through v_permlane32_swap (no LDS
// round trip).  The swap returns this lane's value and the partner's in its
// two result slots; the slot that differs from the own value is the
// partner's (if the two are equal the choice does not matter).
__device__ __forceinline__ unsigned partner_u(unsigned x) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return r[0] == x ? r[1] : r[0];
}
__device__ __forceinline__ float partner(float x) { return __uint_as_float(partner_u(__float_as_uint(x))); }

// XOR swizzle of 16-byte chunks inside an LDS row of K.  The 64 LDS banks
// (256 bytes) serve 16 lanes of a 16-byte read per cycle, and those lanes
// read 16 consecutive rows at one logical chunk: with 128-byte rows (D = 64)
// rows of equal parity share a bank window, so the chunk is XORed with
// (row / 2) mod 8; with rows of 256 bytes or more, with row mod 16.
template <int D>
__device__ __forceinline__ int k_chunk(int row, int ch) {
  return ch ^ (D == 64 ? (row >> 1) & 7 : row & 15);
}

struct RowBounds {
  int lo, hi;  // visible keys [lo, hi) of one query row
};

__device__ __forceinline__ RowBounds row_bounds(int q, int Lq, int Lk, int causal, int window) {
  RowBounds r;
  const int qp = q + Lk - Lq;
  int hi = causal ? min(Lk, qp + 1) : Lk;
  hi = max(hi, 0);
  int lo = window ? max(0, qp - window + 1) : 0;
  r.lo = min(lo, hi);
  r.hi = hi;
  return r;
}

template <class C>
__device__ __forceinline__ void qk_tile(const bf16_t* kl, const bf16x8* qreg, int l32, int g,
                                        f32x16* s) {
  // operand reads are issued in groups of QG ahead of the MFMAs that use them
  constexpr int NOP = C::NQC * C::NKB;
  constexpr int QG = NOP < 8 ? NOP : 8;
#pragma unroll
  for (int kb = 0; kb < C::NKB; ++kb) s[kb] = f32x16{};
#pragma unroll
  for (int g0 = 0; g0 < NOP; g0 += QG) {
    bf16x8 kv[QG];
#pragma unroll
    for (int j = 0; j < QG; ++j) {
      const int c = (g0 + j) / C::NKB, kb = (g0 + j) % C::NKB;
      const int row = kb * 32 + l32;
      kv[j] = *(const bf16x8*)(kl + row * C::D + k_chunk<C::D>(row, 2 * c + g) * 8);
    }
#pragma unroll
    for (int j = 0; j < QG; ++j) {
      const int c = (g0 + j) / C::NKB, kb = (g0 + j) % C::NKB;
      s[kb] = mfma(kv[j], qreg[c], s[kb]);
    }
  }
}

__device__ __forceinline__ int s_key(int k0, int kb, int r, int g) {
  return k0 + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Maps the hardware workgroup id to (batch*head, q-block).  Workgroups are
// dealt round-robin to the 8 XCDs; renumbering gives every XCD a contiguous
// range of (batch, head) pairs, so the query heads sharing one K/V head stay
// in one L2, and within a pair the longest (last) q-blocks start first.
__device__ __forceinline__ void block_coords(int nqb, int& bh, int& qb) {
  const int nblk = gridDim.x;
  int id = blockIdx.x;
  if ((nblk & 7) == 0) id = (id & 7) * (nblk >> 3) + (id >> 3);
  bh = id / nqb;
  qb = nqb - 1 - (id - bh * nqb);
}

// The same XCD-contiguous ranges, ordered longest first across the range:
// an XCD's workgroups run the last (longest causal) q-block of every head of
// its range, then the one before, and so on, so its CUs are packed
// longest-job-first (a per-head order leaves the short blocks of early heads
// occupying CUs while long blocks of later heads wait).
//
// Sequences of different lengths (a paged cache or a packed batch: `spread`)
// would load the XCDs unevenly with contiguous ranges of whole sequences, so
// there each XCD takes, from every sequence, the kv heads congruent to it
// modulo 8 (with their G query heads, which share K/V in its L2): every XCD
// gets the same share of every sequence.  Needs Hkv a multiple of 8.
__device__ __forceinline__ void block_coords_lpt(int nqb, int& bh, int& qb, bool spread = false,
                                                 int Hq = 0, int Hkv = 0) {
  const int nblk = gridDim.x;
  int id = blockIdx.x;
  const bool xcd = (nblk & 7) == 0;
  if (xcd) id = (id & 7) * (nblk >> 3) + (id >> 3);
  const int per = xcd ? nblk >> 3 : nblk;  // ids per XCD range
  if (per % nqb == 0) {
    const int heads = per / nqb;           // whole heads per range
    const int x = id / per, j = id - x * per;
    qb = nqb - 1 - j / heads;
    const int lh = j - (j / heads) * heads;  // head of the range
    if (xcd && spread && Hkv % 8 == 0 && Hq % Hkv == 0 && heads % (Hq / 8) == 0) {
      // the q-blocks of one head, then the heads of one kv head, run
      // together: they stream the same K/V tiles through the XCD's L2
      const int lh = j / nqb;
      qb = nqb - 1 - (j - lh * nqb);
      const int hx = Hq / 8;                 // query heads of one sequence per XCD
      const int G = Hq / Hkv, b = lh / hx, r = lh - b * hx;
      const int kk = r / G, g = r - kk * G;  // kv head kk * 8 + x, query head g of it
      bh = b * Hq + (kk * 8 + x) * G + g;
    } else {
      bh = x * heads + lh;
    }
  } else {
    bh = id / nqb;
    qb = nqb - 1 - (id - bh * nqb);
  }
}

// Max / sum over the two lanes that share a query row (lanes l and l ^ 32):
// v_permlane32_swap hands each half the other half's value.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Two floats to a packed pair of bf16 (round to nearest even).
__device__ __forceinline__ unsigned pack_bf16(float a, float b) {
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// P operand of PV step t = 2 kb + h from the 16 S^T values of block kb.
__device__ __forceinline__ bf16x8 p_operand(const float* p8) {
  const u32x4 w = {pack_bf16(p8[0], p8[1]), pack_bf16(p8[2], p8[3]), pack_bf16(p8[4], p8[5]),
                   pack_bf16(p8[6], p8[7])};
  return __builtin_bit_cast(bf16x8, w);
}

// logit softcap in the log2 domain: log2(e) * cap * tanh(raw * scaling / cap)
__device__ __forceinline__ float capped_log2(float raw, float sc_over_cap, float cap_log2e) {
  const float y = raw * sc_over_cap;
  const float e = __builtin_amdgcn_exp2f(2.f * kLog2e * y);  // exp(2y)
  const float t = 1.f - 2.f * __builtin_amdgcn_rcpf(1.f + e);  // tanh(y)
  return cap_log2e * t;
}

// z of one raw score q.k (the value the threshold acts on).
// Monotone in raw (cz, capz > 0); a masked score (-inf) stays -inf.  Under
// softcap the support test compares z with tau directly, so tanh is the
// library's (a few ulp relative error at every argument), not the
// 1 - 2 / (1 + e^2y) form of the softmax path, which loses relative accuracy
// near 0 (about 2e-7 absolute, i.e. 1e-5 in z at cap 50).
template <bool CAP>
__device__ __forceinline__ float zval(float raw, float cz, float sc_over_cap, float capz) {
#pragma clang fp contract(off)
  if (CAP) {
    const float t = tanhf(raw * sc_over_cap);
    return raw == -INFINITY ? -INFINITY : capz * t;
  }
  return raw * cz;
}

// Direct global -> LDS staging (buffer_load ... lds): no staging registers
// and no vector-ALU work, so several tiles can be in flight.
// One transfer moves 1 KB per wave; lane l's 16 bytes land at byte 16 l of
// the destination, and the lane's source chunk is chosen so that the LDS
// image of a tile is row-major with an XOR chunk swizzle:
//   K: chunk c of key r at position k_chunk(r, c)
//   V: chunk c of key r at position c ^ v_swz(r)
// Keys past the end of the sequence read as zeros (buffer range check, which
// covers the scalar offset too); a transfer that is not needed is sent wholly
// out of range, so every wave issues the same number per tile.
//
// The transfer is issued from inline assembly, so the compiler neither sees
// it as an LDS write nor counts it: every wait for it is explicit (wait_vmcnt
// before the barrier that publishes a tile).  Left to the compiler, a
// transposing LDS read would wait for all transfers in flight, the prefetch
// included.  Compiler-counted waits stay correct, since vector-memory loads
// complete in issue order and extra loads only make a vmcnt wait stricter.
typedef int i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer descriptor (stride 0, num_records = bytes) in scalar registers.
__device__ __forceinline__ i32x4 rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t p = (uint64_t)base;
  return i32x4{__builtin_amdgcn_readfirstlane((int)(uint32_t)p),
               __builtin_amdgcn_readfirstlane((int)((p >> 32) & 0xffffu)),
               __builtin_amdgcn_readfirstlane((int)bytes), 0x00020000};
}

// 16 bytes per lane from buffer offset voff + soff to LDS byte lds_addr + 16 l.
// The compiler's hazard check does not look inside inline assembly, so the
// block starts with the wait states its operands may need: the transfer
// takes its LDS address from M0, which needs one after a scalar write of M0
// (the compiler often writes M0 right before the block; its own LDS
// transfers get an s_nop there), and a scalar operand written by a vector
// instruction (an SGPR restored from a spill lane) needs five before a
// vector-memory read.  Without them the transfer can land at the previous
// transfer's address.
__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t lds_addr, uint32_t voff, uint32_t soff) {
  asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :: "v"(voff), "s"(rsrc), "s"(soff), "{m0}"(lds_addr) : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const bf16_t* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

template <class C>
__device__ __forceinline__ int v_swz(int r) { return C::D == 64 ? 4 * ((r >> 1) & 1) : 4 * (r & 3); }

// s_waitcnt for "at most N vector-memory operations of this wave in flight"
// (gfx9 encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt left at max)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Waits for this wave's LDS accesses only (lgkmcnt 0; vmcnt and expcnt at
// their maxima, so transfers in flight are not waited for).
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Workgroup barrier without the release/acquire fences of __syncthreads()
// (which would wait for every transfer in flight); LDS hazards are covered by
// explicit vmcnt waits and by each wave consuming its LDS reads before it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace
}  // namespace attn
