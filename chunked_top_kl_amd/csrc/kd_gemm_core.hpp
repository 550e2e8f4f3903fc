// MFMA main loop shared by every projection kernel (gfx950).
//
// Computes a 256 x 256 fp32 tile  acc[m][n] = sum_k A[m][k] * B[k][n]  with
// v_mfma_f32_32x32x16_bf16 (bf16 operands) or v_mfma_f32_32x32x2_f32 (fp32
// operands). Operands are staged through LDS in a K-contiguous layout
// ([row][k], 144-byte padded rows), double-buffered, one k-step (128 bytes of
// K per row) at a time. Two global layouts are supported per operand:
//   LoaderKC - operand stored [MN rows][K] (K contiguous), optional row map;
//   LoaderKS - operand stored [K rows][MN] (MN contiguous): each thread loads
//              an 8 x 8 (bf16) or 8 x 4 (fp32) block and transposes it in
//              registers before the LDS store, so the MFMA loop is the same.
// Out-of-range rows and K columns are loaded as zeros.
//
// Result layout (per wave w = 2*wm + wn, lane l, block (i, j), register r):
//   m = wm*128 + i*32 + 8*(r/4) + 4*(l/32) + r%4,   n = wn*128 + j*32 + l%32.
#pragma once

#include "kd_common.hpp"

namespace kd {

__device__ inline uint4 zero4() { return make_uint4(0u, 0u, 0u, 0u); }

// Raw buffer resource over [p, p + bytes): loads at offsets >= bytes return 0.
// Callers keep bytes < 2^31 and mark a lane's load invalid by adding kOob.
constexpr uint32_t kOob = 0x80000000u;
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* p, int64_t bytes) {
  if (bytes < 0) bytes = 0;
  if (bytes > 0x7FFFFFFFll) bytes = 0x7FFFFFFFll;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ inline uint4 bload(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, 0));
}

// ---------------------------------------------------------------------------
// [MN][K] operand with contiguous rows (no map): one buffer resource per tile.
// Thread t loads rows (t>>3) + 32*i (i < 8), 16-byte granule t&7 of a k-step.
// ---------------------------------------------------------------------------
struct LoaderKC {
  __amdgpu_buffer_rsrc_t rs;
  uint32_t voff, rstride;
  int64_t kb0, kb_lim;

  // tile0: address of the tile's first row; ld: row stride (bytes);
  // rows_valid: rows of the tile inside the operand; kb0: first K byte of
  // k-step 0; kb_lim: valid K bytes per row.
  __device__ void init(const char* tile0, int64_t ld, int rows_valid, int64_t kb0_,
                       int64_t kb_lim_) {
    const int t = threadIdx.x;
    if (rows_valid > kTile) rows_valid = kTile;
    rs = make_rsrc(tile0, rows_valid > 0 ? (int64_t)rows_valid * ld : 0);
    voff = (uint32_t)((t >> 3) * ld + (t & 7) * 16);
    rstride = (uint32_t)(32 * ld);
    kb0 = kb0_;
    kb_lim = kb_lim_;
  }
  __device__ void load(int kt, uint4 (&r)[8]) const {
    const int64_t kb = kb0 + (int64_t)kt * kStepBytes;
    uint32_t vo = voff + (uint32_t)kb;
    if (kb + kStepBytes > kb_lim && kb + (threadIdx.x & 7) * 16 >= kb_lim) vo += kOob;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = bload(rs, vo + i * rstride);
  }
  __device__ void store(char* tile, const uint4 (&r)[8]) const {
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      *(uint4*)(tile + ((t >> 3) + 32 * i) * kLdsRow + (t & 7) * 16) = r[i];
  }
};

// ---------------------------------------------------------------------------
// [MN][K] operand whose rows are gathered through a row map (hidden rows of
// the selected / compacted positions): 64-bit addressed global loads.
// ---------------------------------------------------------------------------
struct LoaderKCMap {
  const char* base;
  int64_t ld;
  int srow[8];
  uint32_t rowmask;
  int64_t kb0, kb_lim;

  // map: logical row -> storage row; mn0: first logical row of the tile;
  // mn_lim: number of valid logical rows.
  __device__ void init(const char* base_, int64_t ld_, const int32_t* map, int mn0, int mn_lim,
                       int64_t kb0_, int64_t kb_lim_) {
    const int t = threadIdx.x;
    base = base_;
    ld = ld_;
    kb0 = kb0_ + (t & 7) * 16;
    kb_lim = kb_lim_;
    rowmask = 0;
    const int safe = map[mn0];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = mn0 + (t >> 3) + 32 * i;
      const bool ok = row < mn_lim;
      srow[i] = ok ? map[row] : safe;
      rowmask |= (ok ? 1u : 0u) << i;
    }
  }
  __device__ void load(int kt, uint4 (&r)[8]) const {
    const int64_t kb = kb0 + (int64_t)kt * kStepBytes;
    const bool kok = kb < kb_lim;
    const int64_t kbs = kok ? kb : (kb0 & (kStepBytes - 1));
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint4 v = *(const uint4*)(base + (int64_t)srow[i] * ld + kbs);
      const bool ok = kok && ((rowmask >> i) & 1u);
      r[i] = ok ? v : zero4();
    }
  }
  __device__ void store(char* tile, const uint4 (&r)[8]) const {
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      *(uint4*)(tile + ((t >> 3) + 32 * i) * kLdsRow + (t & 7) * 16) = r[i];
  }
};

// ---------------------------------------------------------------------------
// [K][MN] operand (MN contiguous). A buffer resource is formed per k-step
// over the k-step's K rows.
//   bf16: thread t takes k-group kg = t&7 (8 rows) and MN granule mg = t>>3
//         (8 elements); one k-step covers 64 K rows x 256 MN.
//   fp32: kg = t&3, mg = t>>2 (4 elements); 32 K rows x 256 MN.
// ---------------------------------------------------------------------------
template <typename T>
struct LoaderKS {
  static constexpr int kKRows = 128 / (int)sizeof(T);   // K rows per k-step: 64 | 32
  static constexpr int kKG = kKRows / 8;                 // k-groups of 8 rows: 8 | 4
  const char* base;
  int64_t ld;
  int k0, k_lim;
  uint32_t voff;

  // base: address of (K row 0, first MN column of the tile); ld: row stride
  // (bytes); k0/k_lim: first K row of k-step 0 and the valid K rows;
  // mn_valid_bytes: bytes of the tile's MN extent inside the operand.
  __device__ void init(const char* base_, int64_t ld_, int k0_, int k_lim_,
                       int64_t mn_valid_bytes) {
    const int t = threadIdx.x;
    base = base_;
    ld = ld_;
    k0 = k0_;
    k_lim = k_lim_;
    const int kg = t % kKG, mg = t / kKG;
    voff = (uint32_t)(kg * 8 * ld + mg * 16);
    if ((int64_t)mg * 16 >= mn_valid_bytes) voff += kOob;
  }
  __device__ void load(int kt, uint4 (&r)[8]) const {
    const int kr = k0 + kt * kKRows;
    const int nrows = k_lim - kr;
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(base + (int64_t)kr * ld, nrows > 0 ? (int64_t)(nrows < kKRows ? nrows : kKRows) * ld : 0);
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = bload(rs, voff + (uint32_t)(e * ld));
  }
  __device__ void store(char* tile, const uint4 (&r)[8]) const;
};

template <>
__device__ inline void LoaderKS<__bf16>::store(char* tile, const uint4 (&r)[8]) const {
  const int t = threadIdx.x;
  const int kg = t & 7, mg = t >> 3;
  // element n of K row e sits in dword n/2, half n%2 of r[e]
  const uint32_t* w = (const uint32_t*)r;
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    const int d = n >> 1;
    uint4 o;
    if (n & 1) {
      o.x = (w[0 * 4 + d] >> 16) | (w[1 * 4 + d] & 0xFFFF0000u);
      o.y = (w[2 * 4 + d] >> 16) | (w[3 * 4 + d] & 0xFFFF0000u);
      o.z = (w[4 * 4 + d] >> 16) | (w[5 * 4 + d] & 0xFFFF0000u);
      o.w = (w[6 * 4 + d] >> 16) | (w[7 * 4 + d] & 0xFFFF0000u);
    } else {
      o.x = (w[0 * 4 + d] & 0xFFFFu) | (w[1 * 4 + d] << 16);
      o.y = (w[2 * 4 + d] & 0xFFFFu) | (w[3 * 4 + d] << 16);
      o.z = (w[4 * 4 + d] & 0xFFFFu) | (w[5 * 4 + d] << 16);
      o.w = (w[6 * 4 + d] & 0xFFFFu) | (w[7 * 4 + d] << 16);
    }
    *(uint4*)(tile + (mg * 8 + n) * kLdsRow + kg * 16) = o;
  }
}

template <>
__device__ inline void LoaderKS<float>::store(char* tile, const uint4 (&r)[8]) const {
  const int t = threadIdx.x;
  const int kg = t & 3, mg = t >> 2;
  const uint32_t* w = (const uint32_t*)r;   // w[e*4 + n]
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    uint4 lo = make_uint4(w[0 * 4 + n], w[1 * 4 + n], w[2 * 4 + n], w[3 * 4 + n]);
    uint4 hi = make_uint4(w[4 * 4 + n], w[5 * 4 + n], w[6 * 4 + n], w[7 * 4 + n]);
    char* row = tile + (mg * 4 + n) * kLdsRow + kg * 32;
    *(uint4*)(row) = lo;
    *(uint4*)(row + 16) = hi;
  }
}

// ---------------------------------------------------------------------------
// One k-step of MFMAs on the staged tiles (4 sub-steps).
// ---------------------------------------------------------------------------
template <typename T>
__device__ inline void mfma_step(floatx16 (&acc)[4][4], const char* A, const char* B, int wm,
                                 int wn, int lane);

template <>
__device__ inline void mfma_step<__bf16>(floatx16 (&acc)[4][4], const char* A, const char* B,
                                         int wm, int wn, int lane) {
  const char* pa = A + (wm * 128 + (lane & 31)) * kLdsRow + (lane >> 5) * 16;
  const char* pb = B + (wn * 128 + (lane & 31)) * kLdsRow + (lane >> 5) * 16;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    bf16x8 a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = *(const bf16x8*)(pa + i * 32 * kLdsRow + s * 32);
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = *(const bf16x8*)(pb + j * 32 * kLdsRow + s * 32);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  }
}

template <>
__device__ inline void mfma_step<float>(floatx16 (&acc)[4][4], const char* A, const char* B,
                                        int wm, int wn, int lane) {
  const char* pa = A + (wm * 128 + (lane & 31)) * kLdsRow + (lane >> 5) * 16;
  const char* pb = B + (wn * 128 + (lane & 31)) * kLdsRow + (lane >> 5) * 16;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    floatx4 a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = *(const floatx4*)(pa + i * 32 * kLdsRow + s * 32);
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = *(const floatx4*)(pb + j * 32 * kLdsRow + s * 32);
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i][q], b[j][q], acc[i][j], 0, 0, 0);
  }
}

// ---------------------------------------------------------------------------
// Double-buffered main loop over nk k-steps. Every thread of the work-group
// must call it with the same nk. LDS: A0 | B0 | A1 | B1 (kLdsBytes).
// ---------------------------------------------------------------------------
template <typename T, class LA, class LB>
__device__ inline void gemm_mainloop(floatx16 (&acc)[4][4], const LA& la, const LB& lb, int nk,
                                     char* lds) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, wm = w >> 1, wn = w & 1;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  if (nk <= 0) return;
  uint4 ra[8], rb[8];
  la.load(0, ra);
  lb.load(0, rb);
  la.store(lds, ra);
  lb.store(lds + kLdsTile, rb);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    char* cur = lds + (kt & 1) * 2 * kLdsTile;
    char* nxt = lds + ((kt + 1) & 1) * 2 * kLdsTile;
    const bool more = kt + 1 < nk;
    if (more) {
      la.load(kt + 1, ra);
      lb.load(kt + 1, rb);
    }
    mfma_step<T>(acc, cur, cur + kLdsTile, wm, wn, lane);
    if (more) {
      la.store(nxt, ra);
      lb.store(nxt + kLdsTile, rb);
    }
    __syncthreads();
  }
}

}  // namespace kd
