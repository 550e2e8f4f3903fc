// Backward contractions of one chunk ("backward recomputes the chunk"):
//   dHidden rows = G W        (K = vocabulary, split-K with a fixed-order reduce)
//   dW          (+)= G^T X_c  (K = chunk rows, fp32 read-modify-write of dW)
// plus the small kernels around them (transposed gather of the chunk's hidden
// rows, transpose of W, split-K reduce, zero rows for positions that take no
// part). Every operand is read K-contiguous by the direct-to-LDS main loop.
#include "kd_gemm_core.hpp"
#include "kd_kernels.hpp"

namespace kd {

// operand with the third stage buffer (longer load lead): A (true) or B
#ifndef KD_DH_A_EARLY
#define KD_DH_A_EARLY 1
#endif
#ifndef KD_DW_A_EARLY
#define KD_DW_A_EARLY 1
#endif
constexpr bool kDhAEarly = KD_DH_A_EARLY;
constexpr bool kDwAEarly = KD_DW_A_EARLY;

// rows of this chunk actually present (device count N)
__device__ inline int chunk_rows(const int32_t* nrows_dev, int row_begin, int row_cap) {
  int n = *nrows_dev - row_begin;
  return n < row_cap ? n : row_cap;
}

// ---------------------------------------------------------------------------
// dHidden partials: part[split][r][h] = sum_{v in split} G[r][v] W[v][h]
//   M = chunk rows, N = h (B = W^T [H][Vp]); K = vocabulary. A = G: bf16 in
//   blocks of 256 vocabulary columns (rows 512 bytes apart, blocks ldg bytes
//   apart), fp32 as rows [rows][Vp] (row pitch ldg). The vocabulary is split
//   into `ks` ranges.
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ void dh_body(DhArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[kMainLds];
  const int rows = chunk_rows(a.nrows_dev, a.row_begin, a.row_cap);
  if (rows <= 0) return;
  constexpr int esz = Elem<T>::size;
  const int mt = (int)ceil_div(rows, kTile), nt = (int)ceil_div(a.H, kTile);
  const int nks_total = (int)ceil_div((int64_t)a.V * esz, kKB);
  const int ks = a.ks;
  const int total = mt * nt * ks;
  if ((int)blockIdx.x >= total) return;
  const int L = xcd_remap(blockIdx.x, total);
  const int split = L / (mt * nt), rem = L % (mt * nt);
  const int n = rem / mt, m = rem % mt;
  const int per = (int)ceil_div(nks_total, ks);
  const int kbeg = split * per;
  const int kend = (kbeg + per < nks_total) ? kbeg + per : nks_total;
  const int nk = kend > kbeg ? kend - kbeg : 0;

  DmaOperand lb;
  lb.init(a.WT + (int64_t)n * kTile * a.ldwt, a.ldwt, a.H - n * kTile, (int64_t)kbeg * kKB,
          (int64_t)a.V * esz);
  floatx16 acc[4][4];
  if constexpr (sizeof(T) == 2) {
    DmaOperandBlk la;
    la.init(a.G + (int64_t)m * kTile * 512, a.ldg, rows - m * kTile, (int64_t)kbeg * kKB,
            (int64_t)a.V * esz);
    gemm_mainloop<T, kDhAEarly>(acc, la, lb, nk, lds);
  } else {
    DmaOperand la;
    la.init(a.G + (int64_t)m * kTile * a.ldg, a.ldg, rows - m * kTile, (int64_t)kbeg * kKB,
            (int64_t)a.V * esz);
    gemm_mainloop<T, kDhAEarly>(acc, la, lb, nk, lds);
  }

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, wm = w >> 1, wn = w & 1;
  float* part = a.part + (int64_t)split * dh_split_stride(a.row_cap, a.H);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int h = n * kTile + wn * 128 + j * 32 + (lane & 31);
      if (h >= a.H) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m * kTile + wm * 128 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row < rows) part[(int64_t)row * a.H + h] = acc[i][j][r];
      }
    }
}

__host__ __device__ int dh_splits(int rows, int V, int H, int ncu, int f32) {
  const int esz = f32 ? 4 : 2;
  const int mt = (int)ceil_div(rows, kTile), nt = (int)ceil_div(H, kTile);
  return splitk_factor(mt * nt, (int)ceil_div((int64_t)V * esz, kKB), ncu);
}

int dh_grid(int row_cap, int V, int H, int ncu, int f32) {
  const int mt = (int)ceil_div(row_cap, kTile), nt = (int)ceil_div(H, kTile);
  return mt * nt * dh_splits(row_cap, V, H, ncu, f32);
}

extern "C" __global__ __launch_bounds__(256, 1) void kd_bwd_dhidden_bf16(DhArgs a) { dh_body<__bf16>(a); }
extern "C" __global__ __launch_bounds__(256, 1) void kd_bwd_dhidden_f32(DhArgs a) { dh_body<float>(a); }

hipError_t launch_dh(int f32, const DhArgs& a, int grid, hipStream_t st) {
  if (grid <= 0) return hipSuccess;
  if (f32) hipLaunchKernelGGL(kd_bwd_dhidden_f32, dim3(grid), dim3(kThreads), 0, st, a);
  else hipLaunchKernelGGL(kd_bwd_dhidden_bf16, dim3(grid), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

// dHidden[idx[row_begin + r]][h] = sum over splits (fixed order) of part[s][r][h]
__global__ __launch_bounds__(256) void dh_reduce_kernel(DhReduceArgs a) {
  const int rows = chunk_rows(a.nrows_dev, a.row_begin, a.row_cap);
  const int r = blockIdx.x;   // one work-group per compacted row of the chunk
  if (r >= rows) return;
  const int ks = a.ks;
  const int64_t sstride = dh_split_stride(a.row_cap, a.H);
  const float* src = a.part + (int64_t)r * a.H;
  float* dst = a.dH + (int64_t)a.idx[a.row_begin + r] * a.H;
  for (int c = threadIdx.x; c < a.H / 4; c += 256) {
    // the first 8 partials are requested together (indices clamped, so the
    // loads are unconditional) and added in split order: one memory round
    // trip instead of one per split, and the same sum on every run
    float4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int s = u < ks ? u : ks - 1;
      v[u] = *(const float4*)(src + s * sstride + 4 * c);
    }
    float4 acc = v[0];
#pragma unroll
    for (int u = 1; u < 8; ++u) {
      if (u < ks) {
        acc.x += v[u].x;
        acc.y += v[u].y;
        acc.z += v[u].z;
        acc.w += v[u].w;
      }
    }
    for (int s = 8; s < ks; ++s) {
      const float4 w = *(const float4*)(src + s * sstride + 4 * c);
      acc.x += w.x;
      acc.y += w.y;
      acc.z += w.z;
      acc.w += w.w;
    }
    *(float4*)(dst + 4 * c) = acc;
  }
}

hipError_t launch_dh_reduce(const DhReduceArgs& a, hipStream_t st) {
  if (a.row_cap <= 0) return hipSuccess;
  hipLaunchKernelGGL(dh_reduce_kernel, dim3(a.row_cap), dim3(256), 0, st, a);
  return hipGetLastError();
}

// dH rows of positions that take no part are zero
__global__ __launch_bounds__(256) void zero_rows_kernel(const int32_t* pos, int64_t S, int H,
                                                        float* dH) {
  const int h4 = H / 4;
  const int64_t total = S * h4;
  for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < total;
       q += (int64_t)gridDim.x * 256) {
    const int64_t t = q / h4;
    if (pos[t] < 0) *(float4*)(dH + t * H + 4 * (q % h4)) = make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

hipError_t launch_zero_invalid_rows(const int32_t* pos, int64_t S, int H, float* dH,
                                    hipStream_t st) {
  if (S <= 0) return hipSuccess;
  int64_t grid = ceil_div(S * (H / 4), 256);
  if (grid > 8192) grid = 8192;
  hipLaunchKernelGGL(zero_rows_kernel, dim3((int)grid), dim3(256), 0, st, pos, S, H, dH);
  return hipGetLastError();
}

// x[i] *= g[0] over n floats (16-byte accesses where x is 16-byte aligned)
__global__ __launch_bounds__(256) void scale_kernel(float* x, int64_t n, const float* g) {
  const float f = g[0];
  const int64_t n4 = ((uintptr_t)x & 15u) == 0 ? n / 4 : 0;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < n4; q += stride) {
    float4 v = ((float4*)x)[q];
    v.x *= f;
    v.y *= f;
    v.z *= f;
    v.w *= f;
    ((float4*)x)[q] = v;
  }
  for (int64_t i = 4 * n4 + (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) x[i] *= f;
}

hipError_t launch_scale(float* x, int64_t n, const float* g, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  int64_t grid = ceil_div(ceil_div(n, 4), 256);
  if (grid > 8192) grid = 8192;
  hipLaunchKernelGGL(scale_kernel, dim3((int)grid), dim3(256), 0, st, x, n, g);
  return hipGetLastError();
}

// out[h][r] = X[idx[row_begin + r]][h] for the chunk's rows r < rows and
// out[h][r] = 0 for rows <= r < Cp (the gathered rows, transposed: the dW
// product reads them with K = chunk rows contiguous). 64 x 64 tiles via LDS.
// The same rows are also written in order, xc[r][h] (row pitch ldx), for the
// gradient tile, which then reads its token operand as one contiguous block.
template <typename T>
__global__ __launch_bounds__(256) void gather_rows_t_kernel(const char* X, int64_t ldx,
                                                            const int32_t* idx,
                                                            const int32_t* nrows_dev,
                                                            int row_begin, int row_cap, int H,
                                                            char* out, int64_t ldo, int Cp,
                                                            char* xc) {
  __shared__ T tile[64][65];
  const int rows = chunk_rows(nrows_dev, row_begin, row_cap);
  if (rows <= 0) return;
  const int r0 = blockIdx.x * 64, h0 = blockIdx.y * 64;
  if (r0 >= Cp) return;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int rr = ty; rr < 64; rr += 4) {
    const int r = r0 + rr, h = h0 + tx;
    T v = (T)0.0f;
    if (r < rows && h < H) {
      v = ((const T*)(X + (int64_t)idx[row_begin + r] * ldx))[h];
      ((T*)(xc + (int64_t)r * ldx))[h] = v;
    }
    tile[rr][tx] = v;
  }
  __syncthreads();
  for (int hh = ty; hh < 64; hh += 4) {
    const int h = h0 + hh, r = r0 + tx;
    if (h < H && r < Cp) ((T*)(out + (int64_t)h * ldo))[r] = tile[tx][hh];
  }
}

// The same for bf16 with 16-byte accesses: each row of a 64 (r) x 64 (h) tile
// is read (and copied to xc) as 8 granules of 8 h, and each h row of the
// output is written as granules of 8 r (H, Cp, ldo and ldx are multiples of
// 8 elements, so no granule straddles an edge).
__global__ __launch_bounds__(256) void gather_rows_t_b16_kernel(const char* X, int64_t ldx,
                                                                const int32_t* idx,
                                                                const int32_t* nrows_dev,
                                                                int row_begin, int row_cap, int H,
                                                                char* out, int64_t ldo, int Cp,
                                                                char* xc) {
  __shared__ uint16_t tile[64][66];
  const int rows = chunk_rows(nrows_dev, row_begin, row_cap);
  if (rows <= 0) return;
  const int r0 = blockIdx.x * 64, h0 = blockIdx.y * 64;
  if (r0 >= Cp) return;
  const int tid = threadIdx.x;
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int rr = pass * 32 + (tid >> 3), g = tid & 7;
    const int r = r0 + rr, h = h0 + 8 * g;
    uint4 x = make_uint4(0u, 0u, 0u, 0u);
    if (r < rows && h < H) {
      x = *(const uint4*)(X + (int64_t)idx[row_begin + r] * ldx + (int64_t)h * 2);
      *(uint4*)(xc + (int64_t)r * ldx + (int64_t)h * 2) = x;
    }
    const uint32_t w4[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      tile[rr][8 * g + 2 * e] = (uint16_t)(w4[e] & 0xFFFFu);
      tile[rr][8 * g + 2 * e + 1] = (uint16_t)(w4[e] >> 16);
    }
  }
  __syncthreads();
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int hh = pass * 32 + (tid >> 3), j = tid & 7;
    const int h = h0 + hh, r = r0 + 8 * j;
    if (h < H && r < Cp) {
      uint32_t o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        o[e] = (uint32_t)tile[8 * j + 2 * e][hh] | ((uint32_t)tile[8 * j + 2 * e + 1][hh] << 16);
      *(uint4*)(out + (int64_t)h * ldo + (int64_t)r * 2) = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
}

hipError_t launch_gather_rows_t(int f32, const char* X, int64_t ldx, const int32_t* idx,
                                const int32_t* nrows_dev, int row_begin, int row_cap, int H,
                                char* out, int64_t ldo, int Cp, char* xc, hipStream_t st) {
  dim3 grid((unsigned)ceil_div(Cp, 64), (unsigned)ceil_div(H, 64));
  if (f32)
    hipLaunchKernelGGL(gather_rows_t_kernel<float>, grid, dim3(256), 0, st, X, ldx, idx, nrows_dev,
                       row_begin, row_cap, H, out, ldo, Cp, xc);
  else
    hipLaunchKernelGGL(gather_rows_t_b16_kernel, grid, dim3(256), 0, st, X, ldx, idx, nrows_dev,
                       row_begin, row_cap, H, out, ldo, Cp, xc);
  return hipGetLastError();
}

// WT[h][v] = W[v][h] for v < V, 0 for V <= v < Vp (64 x 64 tiles via LDS)
template <typename T>
__global__ __launch_bounds__(256) void transpose_w_kernel(const T* W, int V, int H, T* WT,
                                                          int Vp, int ldwt) {
  __shared__ T tile[64][65];
  const int v0 = blockIdx.x * 64, h0 = blockIdx.y * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int vv = ty; vv < 64; vv += 4) {
    const int v = v0 + vv, h = h0 + tx;
    T x = (T)0.0f;
    if (v < V && h < H) x = W[(int64_t)v * H + h];
    tile[vv][tx] = x;
  }
  __syncthreads();
  for (int hh = ty; hh < 64; hh += 4) {
    const int h = h0 + hh, v = v0 + tx;
    if (h < H && v < Vp) WT[(int64_t)h * ldwt + v] = tile[tx][hh];
  }
}

// The bf16 transpose with 16-byte accesses on both sides: a 64 (v) x 64 (h)
// tile is read as 8 granules of 8 h per row and written as 8 granules of 8 v
// per h row (H and Vp are multiples of 8, so no granule straddles an edge).
// The LDS tile's row pitch of 66 elements puts the 8 rows read for one output
// granule in distinct banks.
__global__ __launch_bounds__(256) void transpose_w_b16_kernel(const uint16_t* W, int V, int H,
                                                              uint16_t* WT, int Vp, int ldwt) {
  __shared__ uint16_t tile[64][66];
  const int v0 = blockIdx.x * 64, h0 = blockIdx.y * 64;
  const int tid = threadIdx.x;
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int row = pass * 32 + (tid >> 3), g = tid & 7;
    const int v = v0 + row, h = h0 + 8 * g;
    uint4 x = make_uint4(0u, 0u, 0u, 0u);
    if (v < V && h < H) x = *(const uint4*)(W + (int64_t)v * H + h);
    const uint32_t w4[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      tile[row][8 * g + 2 * e] = (uint16_t)(w4[e] & 0xFFFFu);
      tile[row][8 * g + 2 * e + 1] = (uint16_t)(w4[e] >> 16);
    }
  }
  __syncthreads();
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int hh = pass * 32 + (tid >> 3), j = tid & 7;
    const int h = h0 + hh, v = v0 + 8 * j;
    if (h < H && v < Vp) {
      uint32_t o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        o[e] = (uint32_t)tile[8 * j + 2 * e][hh] | ((uint32_t)tile[8 * j + 2 * e + 1][hh] << 16);
      *(uint4*)(WT + (int64_t)h * ldwt + v) = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
}

hipError_t launch_transpose_w(int f32, const char* W, int V, int H, char* WT, int Vp, int ldwt,
                              hipStream_t st) {
  dim3 grid((unsigned)ceil_div(Vp, 64), (unsigned)ceil_div(H, 64));
  if (f32)
    hipLaunchKernelGGL(transpose_w_kernel<float>, grid, dim3(256), 0, st, (const float*)W, V, H,
                       (float*)WT, Vp, ldwt);
  else
    hipLaunchKernelGGL(transpose_w_b16_kernel, grid, dim3(256), 0, st, (const uint16_t*)W, V, H,
                       (uint16_t*)WT, Vp, ldwt);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// dW[v][h] (+)= sum_r G[r][v] X_c[r][h]
//   M = v, N = h (B = X_c^T [H][slots]); K = the token rows of a group of
//   chunks. bf16: A is the group's G itself, in blocks of 256 vocabulary
//   columns ([slots][256] per block, blocks ldg bytes apart), read MN-major
//   (transposed fragment reads); fp32: A = G^T [Vp][slots]. Group 0 with
//   beta_first = 0 overwrites dW (and writes zeros when it is empty); later
//   groups add, and return at once when they hold no rows.
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ void dw_body(DwArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[kMainLds];
  // token columns of the group that hold data: whole slots of the full
  // chunks, then the padded rows of a last partial one
  int grows = chunk_rows(a.nrows_dev, a.group_begin, a.group_chunks * a.chunk);
  if (grows <= 0) {
    if (a.group_begin > 0) return;
    grows = 0;
  }
  const int rows = (grows / a.chunk) * a.slot + (int)round_up(grows % a.chunk, 8);
  constexpr int esz = Elem<T>::size;
  const int mt = (int)ceil_div(a.V, kTile), nt = (int)ceil_div(a.H, kTile);
  const int total = mt * nt;
  if ((int)blockIdx.x >= total) return;
  // grouped raster: 4 vocabulary tiles x all h tiles per group
  const int L = xcd_remap(blockIdx.x, total);
  const int GM = 4;
  const int group = L / (GM * nt);
  const int first_m = group * GM;
  const int gsz = (mt - first_m) < GM ? (mt - first_m) : GM;
  const int in = L % (GM * nt);
  const int m = first_m + in % gsz, n = in / gsz;

  DmaOperand lb;
  lb.init(a.XcT + (int64_t)n * kTile * a.ldxt, a.ldxt, a.H - n * kTile, 0, (int64_t)rows * esz);
  floatx16 acc[4][4];
  const int nk = (int)ceil_div((int64_t)rows * esz, kKB);
  if constexpr (sizeof(T) == 2) {
    // block m; its columns past Vp only feed rows of dW that are never stored
    DmaOperandMN la;
    la.init(a.G + (int64_t)m * a.ldg, 512, rows);
    gemm_mainloop<T, kDwAEarly, true>(acc, la, lb, nk, lds);
  } else {
    DmaOperand la;
    la.init(a.GT + (int64_t)m * kTile * a.ldgt, a.ldgt, a.Vp - m * kTile, 0, (int64_t)rows * esz);
    gemm_mainloop<T, kDwAEarly>(acc, la, lb, nk, lds);
  }

  const bool beta = (a.group_begin > 0) || a.beta_first;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, wm = w >> 1, wn = w & 1;
  // Read-modify-write of the tile's dW rows through a buffer resource over
  // them: rows past V fall outside it and a column past H gets an offset past
  // it, so loads read 0 and stores are dropped without a branch. Straight-line
  // code lets the loads of one group (32 values) be in flight while the
  // previous group is added and stored.
  const int vrows = (a.V - m * kTile) < kTile ? (a.V - m * kTile) : kTile;
  const __amdgpu_buffer_rsrc_t rs =
      make_rsrc(a.dW + (int64_t)m * kTile * a.H, (int64_t)vrows * a.H * 4);
  // lane offset of column block j at the tile's first row of this lane; the
  // element of accumulator (i, j, r) is a wave-uniform number of rows further.
  // A column past H starts at kOob; adding at most 256 rows (< 2^30 bytes for
  // H <= 2^20) keeps it at or past 2^31, outside the resource, with no wrap.
  uint32_t vb[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int h = n * kTile + wn * 128 + j * 32 + (lane & 31);
    const int row0 = wm * 128 + 4 * (lane >> 5);
    vb[j] = h < a.H ? (uint32_t)((row0 * a.H + h) * 4) : kOob;
  }
  auto addr = [&](int j, int i, int r) -> int {
    const uint32_t d = (uint32_t)((32 * i + 8 * (r >> 2) + (r & 3)) * a.H) * 4u;
    return (int)(vb[j] + d);
  };
  // group g: block j = g / 2, blocks i = 2 (g % 2) and 2 (g % 2) + 1
  auto ld = [&](int g, float (&o)[32]) {
    const int j = g >> 1, i0 = (g & 1) * 2;
#pragma unroll
    for (int ii = 0; ii < 2; ++ii)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        o[ii * 16 + r] = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(rs, addr(j, i0 + ii, r), 0, 0));
  };
  auto st = [&](int g, const float (&o)[32]) {
    const int j = g >> 1, i0 = (g & 1) * 2;
#pragma unroll
    for (int ii = 0; ii < 2; ++ii)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        __builtin_amdgcn_raw_buffer_store_b32(
            __builtin_bit_cast(uint32_t, o[ii * 16 + r] + acc[i0 + ii][j][r]), rs,
            addr(j, i0 + ii, r), 0, 0);
  };
  float b0[32], b1[32];
  if (beta) {
    ld(0, b0);
#pragma unroll
    for (int g = 0; g < 8; g += 2) {
      ld(g + 1, b1);
      st(g, b0);
      if (g + 2 < 8) ld(g + 2, b0);
      st(g + 1, b1);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 32; ++e) b0[e] = 0.0f;
#pragma unroll
    for (int g = 0; g < 8; ++g) st(g, b0);
  }
}

extern "C" __global__ __launch_bounds__(256, 1) void kd_bwd_dw_bf16(DwArgs a) { dw_body<__bf16>(a); }
extern "C" __global__ __launch_bounds__(256, 1) void kd_bwd_dw_f32(DwArgs a) { dw_body<float>(a); }

hipError_t launch_dw(int f32, const DwArgs& a, hipStream_t st) {
  const int grid = (int)(ceil_div(a.V, kTile) * ceil_div(a.H, kTile));
  if (f32) hipLaunchKernelGGL(kd_bwd_dw_f32, dim3(grid), dim3(kThreads), 0, st, a);
  else hipLaunchKernelGGL(kd_bwd_dw_bf16, dim3(grid), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace kd
