// MFMA main loop shared by every projection kernel (gfx950).
//
// Computes a 256 x 256 fp32 tile  acc[m][n] = sum_k A[m][k] * B[k][n]  with
// v_mfma_f32_32x32x16_bf16 (bf16 operands) or v_mfma_f32_32x32x2_f32 (fp32
// operands). Both operands are stored row-major with K contiguous
// ([rows][K]); the tile's rows are contiguous in memory (a row stride `ld`).
//
// Data path: global memory -> LDS by direct buffer loads (buffer_load_dwordx4
// ... lds: each lane's 16 bytes land at M0 + 16*lane, no register staging),
// in stages of 128 bytes of K per row (whole cache lines), then LDS ->
// registers (ds_read_b128) -> MFMA. One operand (the "early" one, chosen per
// kernel) has three stage buffers and the other two (160 KB, the whole LDS of
// a CU): the early operand's loads for stage k+2 start at the beginning of
// stage k, the other's once stage k has been read into registers, so both
// have more than a stage of memory latency to land in. Rows and K bytes outside the operand read as zero (buffer range
// checks). The loads are issued from inline assembly so that the compiler
// does not order every LDS read behind them; their completion is awaited
// explicitly with s_waitcnt vmcnt before the stage barrier.
//
// LDS layout of one operand stage buffer: 256 rows x 128 bytes, the eight
// 16-byte granules of row r permuted by g ^ ((r >> 1) & 7) so that the 16
// rows read together by an MFMA fragment load fall in distinct banks.
//
// The A operand may instead be stored K-major across rows ("MN-major":
// [K][rows], the tile's rows contiguous along each K row; DmaOperandMN). Its
// stage buffer holds 64 K rows x 256 tile rows (512 bytes per K row), and its
// fragments are read with ds_read_b64_tr_b16, which hands each lane four
// values of one tile row at four consecutive K (bf16 only).
//
// Result layout (per wave w = 2*wm + wn, lane l, block (i, j), register r):
//   m = wm*128 + i*32 + 8*(r/4) + 4*(l/32) + r%4,   n = wn*128 + j*32 + l%32.
#pragma once

#include "kd_common.hpp"

namespace kd {

constexpr int kKB = 128;                         // K bytes per row per stage (a cache line)
constexpr int kOpBuf = kTile * kKB;              // 32 KB: one operand of one stage
constexpr int kEBufs = 3;                        // stage buffers of the early operand
constexpr int kLBase = kEBufs * kOpBuf;          // the other operand's two buffers follow
constexpr int kMainLds = (kEBufs + 2) * kOpBuf;  // 160 KB
constexpr uint32_t kOob = 0x80000000u;           // an offset at or past this reads zero

__device__ inline uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)p;
}

// Raw buffer resource over [p, p + bytes) (bytes clamped below 2^31).
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* p, int64_t bytes) {
  if (bytes < 0) bytes = 0;
  if (bytes > 0x7FFFFFFFll) bytes = 0x7FFFFFFFll;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// The same for a pointer and size that are the same on every lane but that
// the compiler cannot prove uniform (it must keep a resource in scalar
// registers).
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc_uniform(const void* p, int64_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  if (bytes < 0) bytes = 0;
  if (bytes > 0x7FFFFFFFll) bytes = 0x7FFFFFFFll;
  const int n = __builtin_amdgcn_readfirstlane((int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc((void*)(uintptr_t)(((uint64_t)hi << 32) | lo), (short)0,
                                           n, 0x00020000);
}

// 16 bytes per lane from rs at voff into LDS at m0 + 16 * lane. M0 is written
// and consumed inside the one asm statement. The compiler warns that it does
// not preserve a reserved register named as a clobber; no code it generates
// for these kernels reads M0 (no indirect register indexing, no LDS-DMA
// builtins, no messages), which the generated assembly shows: its only M0
// references are the writes of this statement.
__device__ __forceinline__ void dma16(uint32_t m0, uint32_t voff, __amdgpu_buffer_rsrc_t rs) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(m0), "v"(voff), "s"(rs) : "memory", "m0");
}

// Opaque copy: keeps the compiler from hoisting per-tile address arithmetic
// out of the tile loop (which would keep it live, and spilled, across the
// epilogues).
template <typename X>
__device__ __forceinline__ X opaque(X x) {
  asm volatile("" : "+v"(x));
  return x;
}

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// ---------------------------------------------------------------------------
// One operand tile: 256 rows starting at `tile0`, row stride `ld` bytes,
// `rows_valid` rows inside the operand, K bytes [kb0, kb_lim) of each row.
// Wave w fills rows [64w, 64w + 64) of each stage with 8 loads of 8 rows.
// ---------------------------------------------------------------------------
struct DmaOperand {
  __amdgpu_buffer_rsrc_t rs;
  uint32_t voff;      // lane's offset for load q = 0 (row and permuted granule)
  uint32_t qstride;   // 8 rows
  uint32_t gofs;      // lane's granule offset inside the 128-byte stage row
  uint32_t ldsoff;    // wave block inside a stage buffer
  int64_t kb0, kb_lim;

  __device__ void init(const char* tile0, int64_t ld, int rows_valid, int64_t kb0_,
                       int64_t kb_lim_) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (rows_valid > kTile) rows_valid = kTile;
    rs = make_rsrc(tile0, rows_valid > 0 ? (int64_t)rows_valid * ld : 0);
    // lane -> row w*64 + 8q + lane/8, physical granule lane%8; the swizzle
    // term ((8q + lane/8) >> 1) & 7 is (lane >> 4) for even q and (lane >> 4) ^ 4
    // for odd q
    const int row = lane >> 3;
    const int g = (lane & 7) ^ (lane >> 4);
    gofs = (uint32_t)(g * 16);
    voff = opaque((uint32_t)((w * 64 + row) * ld) + gofs);
    qstride = (uint32_t)(8 * ld);
    ldsoff = (uint32_t)(w * 64 * kKB);
    kb0 = kb0_;
    kb_lim = kb_lim_;
  }
  // enqueue the 8 loads of stage kt into the stage buffer at LDS address `stage`
  __device__ __forceinline__ void issue(int kt, uint32_t stage) const {
#pragma unroll
    for (int q = 0; q < 8; ++q) issue_one(kt, stage, q);
  }
  // load q (rows 8q .. 8q+7 of this wave's 64-row block) of stage kt
  __device__ __forceinline__ void issue_one(int kt, uint32_t stage, int q) const {
    const int64_t kb = kb0 + (int64_t)kt * kKB;
    // odd q: granule g ^ 4, i.e. 64 bytes further or back inside the row
    const uint32_t gq = (q & 1) ? (gofs ^ 64u) : gofs;
    uint32_t o = voff - gofs + gq + (uint32_t)kb + q * qstride;
    if (kb + kKB > kb_lim && kb + gq >= kb_lim) o = kOob;
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(stage + ldsoff);
    dma16(m0 + q * 1024, o, rs);
  }
};

// ---------------------------------------------------------------------------
// K-major operand stored in column blocks: K bytes [512 b, 512 b + 512) of
// every row sit in block b, rows 512 bytes apart inside a block and blocks
// `bstride` bytes apart (the bf16 gradient tiles: blocks of 256 vocabulary
// columns). `tile0` is the tile's first row in block 0. A stage (128 bytes of
// K) never straddles two blocks; the buffer resource is set per stage, over
// the block's `rows_valid` rows of the tile. Same LDS layout and lane mapping
// as DmaOperand.
// ---------------------------------------------------------------------------
struct DmaOperandBlk {
  const char* tile0;
  int64_t bstride;
  int rows_valid;
  uint32_t voff;      // lane's offset for load q = 0 (row and permuted granule)
  uint32_t gofs, ldsoff;
  int64_t kb0, kb_lim;

  __device__ void init(const char* tile0_, int64_t bstride_, int rows_valid_, int64_t kb0_,
                       int64_t kb_lim_) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    tile0 = tile0_;
    bstride = bstride_;
    rows_valid = rows_valid_ < 0 ? 0 : (rows_valid_ > kTile ? kTile : rows_valid_);
    const int row = lane >> 3;
    const int g = (lane & 7) ^ (lane >> 4);
    gofs = (uint32_t)(g * 16);
    voff = opaque((uint32_t)((w * 64 + row) * 512) + gofs);
    ldsoff = (uint32_t)(w * 64 * kKB);
    kb0 = kb0_;
    kb_lim = kb_lim_;
  }
  __device__ __forceinline__ void issue(int kt, uint32_t stage) const {
#pragma unroll
    for (int q = 0; q < 8; ++q) issue_one(kt, stage, q);
  }
  __device__ __forceinline__ void issue_one(int kt, uint32_t stage, int q) const {
    const int64_t kb = kb0 + (int64_t)kt * kKB;
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc_uniform(tile0 + (kb >> 9) * bstride, (int64_t)rows_valid * 512);
    const uint32_t gq = (q & 1) ? (gofs ^ 64u) : gofs;
    uint32_t o = voff - gofs + gq + (uint32_t)(kb & 511) + q * 8 * 512;
    if (kb + kKB > kb_lim && kb + gq >= kb_lim) o = kOob;
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(stage + ldsoff);
    dma16(m0 + q * 1024, o, rs);
  }
};

// ---------------------------------------------------------------------------
// MN-major bf16 operand tile: K rows [0, krows) of the tile, row stride `ld`
// bytes, the tile's 256 rows (512 bytes) contiguous in each K row from
// `tile0`. Stage kt holds K rows [64 kt, 64 kt + 64) as 64 LDS rows of 512
// bytes; the 16-byte granule g of LDS row t holds logical granule
// g ^ ((t & 3) << 2), so that the four K rows read together by a transposed
// fragment read (rows 4u .. 4u+3) fall in distinct 64-byte bank groups. Wave w
// fills LDS rows [16w, 16w + 16) with 8 loads of 2 rows. The buffer resource is
// set per stage, over the stage's K rows that exist: the rows past krows (and
// the whole of a stage past the end) read as zero, and no offset exceeds
// 64 K rows, whatever the operand's size.
// ---------------------------------------------------------------------------
struct DmaOperandMN {
  const char* tile0;
  int64_t ld;
  int krows;
  uint32_t voff[2];   // lane's offset for even / odd q (K row 16w + lane/32, permuted granule)
  uint32_t ldsoff;    // wave block inside a stage buffer

  __device__ void init(const char* tile0_, int64_t ld_, int krows_) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int h = lane >> 5, pg = lane & 31;
    tile0 = tile0_;
    ld = ld_;
    krows = krows_;
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      // LDS row 16w + 2q + h has (row & 3) = (2 (q & 1) + h) & 3
      const int lg = pg ^ ((((2 * par + h) & 3)) << 2);
      voff[par] = opaque((uint32_t)((int64_t)(16 * w + h) * ld + lg * 16));
    }
    ldsoff = (uint32_t)(w * 16 * 512);
  }
  __device__ __forceinline__ void issue(int kt, uint32_t stage) const {
#pragma unroll
    for (int q = 0; q < 8; ++q) issue_one(kt, stage, q);
  }
  __device__ __forceinline__ void issue_one(int kt, uint32_t stage, int q) const {
    const int r0 = kt * 64;
    int nr = krows - r0;
    nr = nr < 0 ? 0 : (nr > 64 ? 64 : nr);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc_uniform(tile0 + (int64_t)r0 * ld, (int64_t)nr * ld);
    const uint32_t o = voff[q & 1] + (uint32_t)(2 * q) * (uint32_t)ld;
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(stage + ldsoff);
    dma16(m0 + q * 1024, o, rs);
  }
};

// 16 bytes per lane from the 64-bit address `ga` into LDS at m0 + 16 * lane.
__device__ __forceinline__ void dma16_global(uint32_t m0, const char* ga) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(m0), "v"(ga) : "memory", "m0");
}

// ---------------------------------------------------------------------------
// Operand tile whose rows are gathered through a row map (selected or
// compacted positions): 64-bit per-lane addresses, no range checks. Rows past
// mn_lim repeat the tile's first row and K granules past kb_lim re-read the
// row's first granule: both only feed outputs that are discarded or products
// with the other operand's exact zeros, so the data only has to be finite.
// ---------------------------------------------------------------------------
struct DmaOperandMap {
  const char* base;
  int64_t ld;
  int srow[8];           // lane's storage row for load q
  uint32_t gofs, ldsoff;
  int64_t kb0, kb_lim;

  __device__ void init(const char* base_, int64_t ld_, const int32_t* map, int mn0, int mn_lim,
                       int64_t kb0_, int64_t kb_lim_) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int row = lane >> 3;
    const int g = (lane & 7) ^ (lane >> 4);   // even q; odd q use g ^ 4
    base = base_;
    ld = ld_;
    gofs = (uint32_t)(g * 16);
    ldsoff = (uint32_t)(w * 64 * kKB);
    const int first = map[mn0];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int r = mn0 + w * 64 + q * 8 + row;
      srow[q] = opaque(r < mn_lim ? map[r] : first);
    }
    kb0 = kb0_;
    kb_lim = kb_lim_;
  }
  __device__ __forceinline__ void issue(int kt, uint32_t stage) const {
#pragma unroll
    for (int q = 0; q < 8; ++q) issue_one(kt, stage, q);
  }
  __device__ __forceinline__ void issue_one(int kt, uint32_t stage, int q) const {
    const int64_t kb = kb0 + (int64_t)kt * kKB;
    const uint32_t gq = (q & 1) ? (gofs ^ 64u) : gofs;
    const int64_t o = (kb + gq < kb_lim) ? kb + gq : 0;
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(stage + ldsoff);
    dma16_global(m0 + q * 1024, base + (int64_t)srow[q] * ld + o);
  }
};

// ---------------------------------------------------------------------------
// MFMAs of one sub-step (K = 16 bf16 / 8 fp32; a stage holds four).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void mfma16(floatx16 (&acc)[4][4], const bf16x8 (&a)[4],
                                       const bf16x8 (&b)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
}

__device__ __forceinline__ void mfma16(floatx16 (&acc)[4][4], const floatx4 (&a)[4],
                                       const floatx4 (&b)[4]) {
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i][q], b[j][q], acc[i][j], 0, 0, 0);
}

template <typename T> struct Frag;
template <> struct Frag<__bf16> { using type = bf16x8; };
template <> struct Frag<float> { using type = floatx4; };

// Per-lane fragment addressing inside a stage buffer: rows wm*128 + i*32 +
// (l & 31) (A) and wn*128 + j*32 + (l & 31) (B), logical granule 2s + (l >> 5)
// for sub-step s.
//
// MN-major A (DmaOperandMN layout): block i, sub-step s of lane l = 32h +
// 16g + 4u + e (g, u, e < 4 as bit fields: g < 2, u < 4, e < 4) reads two
// 64-bit pieces, at K rows 16s + 8h + 4p + u (p = 0, 1) and tile rows
// wm*128 + 32i + 16g + 4e .. +3. The transposed read gives the lane the four
// values of tile row wm*128 + 32i + 16g + 4(l%16 / 4) + l%4 at K rows
// 16s + 8h + 4p + 0..3, so the pair holds that row's 8 consecutive K values
// 16s + 8h .. +7, which is the K-major fragment. amn[i] is the lane's LDS
// offset at s = p = 0 (the granule swizzle makes it depend on i).
struct FragAddr {
  uint32_t a[4], b[4];
  uint32_t amn[4];
  __device__ void init(int wm, int wn, int lane) {
    const int r = lane & 31, swz = (r >> 1) & 7, half = lane >> 5;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int pg = (2 * s + half) ^ swz;
      a[s] = (uint32_t)((wm * 128 + r) * kKB + pg * 16);
      b[s] = (uint32_t)((wn * 128 + r) * kKB + pg * 16);
    }
  }
  __device__ void init_mn(int wm, int lane) {
    const int e = lane & 3, u = (lane >> 2) & 3, g = (lane >> 4) & 1, h = lane >> 5;
    // logical granule wm*16 + 4i + 2g + e/2, byte 8 (e & 1) inside it; the
    // K row's (row & 3) is u
    const uint32_t base = (uint32_t)((8 * h + u) * 512 + wm * 256 + (2 * g + (e >> 1)) * 16 +
                                     8 * (e & 1));
#pragma unroll
    for (int i = 0; i < 4; ++i) amn[i] = base + (uint32_t)((i ^ u) << 6);
  }
};

typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef short shortx8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ shortx4 ds_read_tr16(const char* p) {
  typedef __attribute__((address_space(3))) shortx4 lds_shortx4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_shortx4*)((__attribute__((address_space(3))) char*)const_cast<char*>(p)));
}

// A fragment of block i, sub-step s
template <bool A_MN, class V>
__device__ __forceinline__ V read_a(const char* sa, const FragAddr& fa, int s, int i) {
  if constexpr (A_MN) {
    const char* p = sa + fa.amn[i] + s * 16 * 512;
    const shortx4 lo = ds_read_tr16(p), hi = ds_read_tr16(p + 4 * 512);
    return __builtin_bit_cast(V, (shortx8)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  } else {
    return *(const V*)(sa + fa.a[s] + i * 32 * kKB);
  }
}

// ---------------------------------------------------------------------------
// Main loop over nk stages (nk = ceil(K bytes / 128)). Every thread of the
// work-group must call it with the same nk. `lds` points at kMainLds bytes.
// A_EARLY selects the operand with three buffers (A if true, else B).
//
// Stage kt (early buffer kt % 3, late buffer kt % 2) has four sub-steps of 16
// MFMAs; the fragments of sub-step s+1 are read while sub-step s computes.
// The 8 loads of the early operand for stage kt+2 go out one per two MFMAs
// over the first sub-step (their buffer held stage kt-1, released by the
// previous barrier). Before the last sub-step: wait for this wave's loads of
// stage kt+1 (the early operand's for kt+2 may still be in flight) and
// barrier (stage kt+1 visible to all waves; every wave holds its stage-kt
// fragments, so stage kt's late buffer is free). The 8 loads of the late
// operand for stage kt+2 into that buffer are spread over the last sub-step,
// with the 8 sub-step-0 fragment reads of stage kt+1. Issued in one burst,
// the loads back up the vector memory queue and stall the wave's in-order
// issue while its MFMA pipe runs dry. A stage at or past the end of K reads
// zeros (or, for a row-mapped operand, a valid granule) into a free buffer,
// so the issue needs no branch. The last stage is peeled: it issues no loads.
// ---------------------------------------------------------------------------
template <typename V>
struct SubFrags {
  V a[4], b[4];
};

template <bool A_MN, class V>
__device__ __forceinline__ void read_sub(SubFrags<V>& f, const char* sa, const char* sb,
                                         const FragAddr& fa, int s) {
#pragma unroll
  for (int i = 0; i < 4; ++i) f.a[i] = read_a<A_MN, V>(sa, fa, s, i);
#pragma unroll
  for (int j = 0; j < 4; ++j) f.b[j] = *(const V*)(sb + fa.b[s] + j * 32 * kKB);
}

__device__ __forceinline__ void mfma_ij(floatx16& acc, const bf16x8& a, const bf16x8& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ void mfma_ij(floatx16& acc, const floatx4& a, const floatx4& b) {
#pragma unroll
  for (int q = 0; q < 4; ++q) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[q], b[q], acc, 0, 0, 0);
}

// A sub-step whose MFMAs are interleaved with the 8 loads of one operand of
// stage kn (into the buffer at `sbase`), one load per two MFMA blocks.
template <class V, class OP>
__device__ __forceinline__ void mfma_sub_loads(floatx16 (&acc)[4][4], const SubFrags<V>& f,
                                               const OP& op, int kn, uint32_t sbase) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int q = i * 4 + j;
      mfma_ij(acc[i][j], f.a[i], f.b[j]);
      if ((q & 1) == 0) op.issue_one(kn, sbase, q >> 1);
      __builtin_amdgcn_sched_barrier(0);
    }
}

// The same with the sub-step-0 fragment reads of the next stage as well.
template <bool A_MN, class V, class OP>
__device__ __forceinline__ void mfma_sub_loads_reads(floatx16 (&acc)[4][4], const SubFrags<V>& f,
                                                     const OP& op, int kn, uint32_t sbase,
                                                     SubFrags<V>& fn, const char* na,
                                                     const char* nb, const FragAddr& fa) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int q = i * 4 + j;
      mfma_ij(acc[i][j], f.a[i], f.b[j]);
      if ((q & 1) == 0) op.issue_one(kn, sbase, q >> 1);
      if (q < 4) fn.a[q] = read_a<A_MN, V>(na, fa, 0, q);
      else if (q < 8) fn.b[q - 4] = *(const V*)(nb + fa.b[0] + (q - 4) * 32 * kKB);
      __builtin_amdgcn_sched_barrier(0);
    }
}

// Issue stages 0 and 1 of the next main loop ahead of time, into the buffers
// its own prologue would use, so that they load while the caller works on the
// previous tile's accumulators; that main loop is then called with
// prefetched = true. Nothing may use the LDS in between. (Memory waits the
// compiler places in between, such as spill reloads, wait for these loads as
// well: the vector memory counter retires in order.)
template <bool A_EARLY, class OA, class OB>
__device__ inline void gemm_prefetch(const OA& la, const OB& lb, int nk, char* lds) {
  if (nk <= 0) return;
  const uint32_t base = lds_addr(lds);
  // every wave has read its last fragments of the previous call
  __syncthreads();
  if constexpr (A_EARLY) { la.issue(0, base); lb.issue(0, base + kLBase); }
  else { lb.issue(0, base); la.issue(0, base + kLBase); }
  if (nk > 1) {
    if constexpr (A_EARLY) { la.issue(1, base + kOpBuf); lb.issue(1, base + kLBase + kOpBuf); }
    else { lb.issue(1, base + kOpBuf); la.issue(1, base + kLBase + kOpBuf); }
  }
}

template <typename T, bool A_EARLY, bool A_MN = false, class OA, class OB>
__device__ inline void gemm_mainloop(floatx16 (&acc)[4][4], const OA& la, const OB& lb, int nk,
                                     char* lds, bool prefetched = false) {
  using V = typename Frag<T>::type;
  static_assert(!A_MN || sizeof(T) == 2, "the transposed fragment read is for bf16");
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, wm = w >> 1, wn = w & 1;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  if (nk <= 0) return;
  FragAddr fa;
  fa.init(wm, wn, lane);
  if constexpr (A_MN) fa.init_mn(wm, lane);
  const uint32_t base = lds_addr(lds);
  // buffer i of the early / late operand
  auto ebuf = [&](int i) { return lds + i * kOpBuf; };
  auto lbuf = [&](int i) { return lds + kLBase + i * kOpBuf; };
  auto issue_e = [&](int kt, int i) {
    if constexpr (A_EARLY) la.issue(kt, base + i * kOpBuf);
    else lb.issue(kt, base + i * kOpBuf);
  };
  auto issue_l = [&](int kt, int i) {
    if constexpr (A_EARLY) lb.issue(kt, base + kLBase + i * kOpBuf);
    else la.issue(kt, base + kLBase + i * kOpBuf);
  };
  if (prefetched) {
    wait_vmcnt<0>();
  } else {
    // every wave has finished reading the stages of a previous call
    __syncthreads();
    issue_e(0, 0);
    issue_l(0, 0);
    if (nk > 1) {
      issue_e(1, 1);
      issue_l(1, 1);
      wait_vmcnt<16>();
    } else {
      wait_vmcnt<0>();
    }
  }
  __syncthreads();
  SubFrags<V> f0, f1;
  read_sub<A_MN>(f0, A_EARLY ? ebuf(0) : lbuf(0), A_EARLY ? lbuf(0) : ebuf(0), fa, 0);
  int ie = 0;  // early buffer of stage kt
  for (int kt = 0; kt + 1 < nk; ++kt) {
    const int ie1 = ie == kEBufs - 1 ? 0 : ie + 1;    // stage kt+1
    const int ie2 = ie1 == kEBufs - 1 ? 0 : ie1 + 1;  // stage kt+2 (stage kt-1's, free)
    const char* sa = A_EARLY ? ebuf(ie) : lbuf(kt & 1);
    const char* sb = A_EARLY ? lbuf(kt & 1) : ebuf(ie);
    __builtin_amdgcn_sched_barrier(0);
    read_sub<A_MN>(f1, sa, sb, fa, 1);
    __builtin_amdgcn_sched_barrier(0);
    // the early operand of stage kt+2
    if constexpr (A_EARLY) mfma_sub_loads(acc, f0, la, kt + 2, base + ie2 * kOpBuf);
    else mfma_sub_loads(acc, f0, lb, kt + 2, base + ie2 * kOpBuf);
    __builtin_amdgcn_sched_barrier(0);
    read_sub<A_MN>(f0, sa, sb, fa, 2);
    __builtin_amdgcn_sched_barrier(0);
    mfma16(acc, f1.a, f1.b);
    __builtin_amdgcn_sched_barrier(0);
    read_sub<A_MN>(f1, sa, sb, fa, 3);
    __builtin_amdgcn_sched_barrier(0);
    mfma16(acc, f0.a, f0.b);
    __builtin_amdgcn_sched_barrier(0);
    // this wave's loads of stage kt+1 (issued before the 8 of the early
    // operand for kt+2, and loads complete in order) have landed
    wait_vmcnt<8>();
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    // the late operand of stage kt+2 into stage kt's late buffer, and stage
    // kt+1's first reads
    const uint32_t lnext = base + kLBase + (kt & 1) * kOpBuf;
    const char* na = A_EARLY ? ebuf(ie1) : lbuf((kt + 1) & 1);
    const char* nb = A_EARLY ? lbuf((kt + 1) & 1) : ebuf(ie1);
    if constexpr (A_EARLY) mfma_sub_loads_reads<A_MN>(acc, f1, lb, kt + 2, lnext, f0, na, nb, fa);
    else mfma_sub_loads_reads<A_MN>(acc, f1, la, kt + 2, lnext, f0, na, nb, fa);
    ie = ie1;
  }
  {
    const char* sa = A_EARLY ? ebuf(ie) : lbuf((nk - 1) & 1);
    const char* sb = A_EARLY ? lbuf((nk - 1) & 1) : ebuf(ie);
    __builtin_amdgcn_sched_barrier(0);
    read_sub<A_MN>(f1, sa, sb, fa, 1);
    __builtin_amdgcn_sched_barrier(0);
    mfma16(acc, f0.a, f0.b);
    __builtin_amdgcn_sched_barrier(0);
    read_sub<A_MN>(f0, sa, sb, fa, 2);
    __builtin_amdgcn_sched_barrier(0);
    mfma16(acc, f1.a, f1.b);
    __builtin_amdgcn_sched_barrier(0);
    read_sub<A_MN>(f1, sa, sb, fa, 3);
    __builtin_amdgcn_sched_barrier(0);
    mfma16(acc, f0.a, f0.b);
    __builtin_amdgcn_sched_barrier(0);
    mfma16(acc, f1.a, f1.b);
  }
  // the loads of the stages past the end (zeros into free buffers) have
  // landed before the caller reuses the LDS
  wait_vmcnt<0>();
  __builtin_amdgcn_sched_barrier(0);
}

}  // namespace kd
