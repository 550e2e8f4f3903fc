// Sampled sparse teacher targets ("Rethinking Selective Knowledge
// Distillation", Method section 2: RS-KD, the class axis of SE-KD3X): N ids
// per position drawn from the teacher's softmax at temperature T by inverse
// transform in vocabulary order, each draw given by a caller's uniform u: the
// smallest id v with F(v) > u, F the cumulative probability over ids 0..v.
//
// The vocabulary sweeps (kd_sweep.hip) store the mass of every 128-entry
// unit of each row, each in its own scale, and later resolve a draw inside
// its unit. Between them, these kernels turn the unit masses into a
// cumulative sum in one scale per row and give every draw its unit and the
// residual mass inside it.
#include "kd_common.hpp"
#include "kd_kernels.hpp"

#include <algorithm>

namespace kd {

__global__ void draw_zero_flag_kernel(int32_t* flag) {
  if (threadIdx.x == 0) flag[0] = 0;
}

// flag <- 1 when a uniform is outside [0, 1) (NaN included) or a row of them
// decreases
__global__ __launch_bounds__(256) void draw_check_kernel(const double* u, int64_t S, int N,
                                                         int32_t* flag) {
  const int64_t n_all = S * N;
  bool bad = false;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n_all;
       i += (int64_t)gridDim.x * blockDim.x) {
    const double x = u[i];
    bad |= !(x >= 0.0 && x < 1.0);
    if (i % N != 0) bad |= u[i - 1] > x;
  }
  if (bad) flag[0] = 1;
}

hipError_t launch_draw_check(const double* u, int64_t S, int N, int32_t* flag, hipStream_t st) {
  hipLaunchKernelGGL(draw_zero_flag_kernel, dim3(1), dim3(64), 0, st, flag);
  const int64_t n = S * N;
  const int grid = (int)std::min<int64_t>(ceil_div(n, 256), 2048);
  if (grid > 0) hipLaunchKernelGGL(draw_check_kernel, dim3(grid), dim3(256), 0, st, u, S, N, flag);
  return hipGetLastError();
}

// One thread per row. Each unit's mass is stored in its own scale 2^-sc
// (sc = c times the unit's largest logit); with M the row's largest sc, the
// masses are brought to the scale 2^-M and become their running sum in
// vocabulary order, in fp64 and in place ([unit][row], pitch ldm), so that
// neighbouring threads touch neighbouring addresses. Sequential addition of
// non-negative terms keeps the sum non-decreasing, which the search below
// relies on. A row with non-finite logits gets a NaN sum.
__global__ __launch_bounds__(256) void draw_cumsum_kernel(double* m, const float* sc, int64_t ldm,
                                                          int nu, int rows, float* rowmax) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= rows) return;
  // 32 units at a time: their loads are issued together, then used in order
  constexpr int kB = 32;
  float M = -INFINITY;
  for (int k0 = 0; k0 < nu; k0 += kB) {
    float v[kB];
#pragma unroll
    for (int i = 0; i < kB; ++i) v[i] = (k0 + i < nu) ? sc[(int64_t)(k0 + i) * ldm + t] : -INFINITY;
#pragma unroll
    for (int i = 0; i < kB; ++i) M = fmaxf(M, v[i]);
  }
  rowmax[t] = M;
  double run = 0.0;
  double* p = m + t;
  for (int k0 = 0; k0 < nu; k0 += kB) {
    double v[kB];
    float f[kB];
#pragma unroll
    for (int i = 0; i < kB; ++i) {
      const bool in = k0 + i < nu;
      v[i] = in ? p[(int64_t)(k0 + i) * ldm] : 0.0;
      f[i] = in ? sc[(int64_t)(k0 + i) * ldm + t] : M;
    }
    // the scale factor in fp32 (the exponent difference is exact in fp64 and
    // small where it matters): its 1e-7 relative error is far below that of
    // the weights themselves
#pragma unroll
    for (int i = 0; i < kB; ++i) {
      const float d = (float)((double)f[i] - (double)M);
      run += v[i] * (double)__builtin_amdgcn_exp2f(d);
      v[i] = run;
    }
#pragma unroll
    for (int i = 0; i < kB; ++i)
      if (k0 + i < nu) p[(int64_t)(k0 + i) * ldm] = v[i];
  }
}

hipError_t launch_draw_cumsum(double* tmass, const float* tscale, int64_t ldm, int nu, int rows,
                              float* rowmax, hipStream_t st) {
  if (rows > 0)
    hipLaunchKernelGGL(draw_cumsum_kernel, dim3((unsigned)ceil_div(rows, 256)), dim3(256), 0, st,
                       tmass, tscale, ldm, nu, rows, rowmax);
  return hipGetLastError();
}

// One thread per draw (row t, draw n). With Z the row's total mass, the draw
// aims at mass u Z: its unit is the first whose cumulative mass exceeds that,
// and its residual the aim less the mass of the units before, given in the
// unit's own scale. An aim at or above Z (u within rounding of 1) takes the
// unit where the cumulative mass first reaches Z (the last unit of positive
// mass) with an unbounded residual: the draw pass then takes that unit's last
// entry of positive weight. A row whose total is not a positive finite number
// (non-finite logits) gets unit -1, which no unit matches, and keeps the id -1
// written here.
__global__ __launch_bounds__(256) void draw_assign_kernel(const double* cum, const float* sc,
                                                          const float* rowmax, int64_t ldm, int nu,
                                                          int rows, const double* u, int N,
                                                          int32_t* dunit, double* dres,
                                                          int32_t* sids) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= (int64_t)rows * N) return;
  const int t = (int)(i / N);
  const double* c = cum + t;
  const double Z = c[(int64_t)(nu - 1) * ldm];
  sids[i] = -1;
  if (!(Z > 0.0) || !(Z < INFINITY)) {
    dunit[i] = -1;
    dres[i] = 0.0;
    return;
  }
  const double aim = u[i] * Z;
  const bool top = aim >= Z;
  // first unit k with cum[k] > aim (or, at the top, cum[k] >= Z)
  int lo = 0, hi = nu - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    const double v = c[(int64_t)mid * ldm];
    const bool past = top ? v >= Z : v > aim;
    if (past) hi = mid;
    else lo = mid + 1;
  }
  dunit[i] = lo;
  if (top) {
    dres[i] = INFINITY;
  } else {
    const double r = aim - (lo > 0 ? c[(int64_t)(lo - 1) * ldm] : 0.0);
    dres[i] = r * exp2((double)rowmax[t] - (double)sc[(int64_t)lo * ldm + t]);
  }
}

hipError_t launch_draw_assign(const double* cum, const float* tscale, const float* rowmax,
                              int64_t ldm, int nu, int rows, const double* u, int N,
                              int32_t* dunit, double* dres, int32_t* sids, hipStream_t st) {
  const int64_t n = (int64_t)rows * N;
  if (n > 0)
    hipLaunchKernelGGL(draw_assign_kernel, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, st, cum,
                       tscale, rowmax, ldm, nu, rows, u, N, dunit, dres, sids);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Rows per drawn-in vocabulary tile. A row's draws are ordered by unit (its
// uniforms do not decrease), so the tiles it draws in are runs of its unit
// list; a row of non-finite logits has unit -1 on every draw and none.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void draw_tiles_zero_kernel(int32_t* a, int32_t* b, int n) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) {
    a[i] = 0;
    b[i] = 0;
  }
}

// one thread per draw; the first draw of each run of a row's draws in one
// tile stands for the row there
__device__ inline int draw_tile_start(const int32_t* du, int64_t i, int N) {
  const int u = du[i];
  if (u < 0) return -1;
  const int tile = u >> 1;
  if (i % N != 0 && (du[i - 1] >> 1) == tile) return -1;
  return tile;
}

__global__ __launch_bounds__(256) void draw_tile_count_kernel(const int32_t* du, int rows, int N,
                                                              int32_t* tcnt) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)rows * N) return;
  const int tile = draw_tile_start(du, i, N);
  if (tile >= 0) atomicAdd(&tcnt[tile], 1);
}

// exclusive running sum of cnt[0..n) into off, one work-group of 1024 threads
__global__ __launch_bounds__(1024) void draw_tile_scan_kernel(const int32_t* cnt, int n,
                                                              int32_t* off) {
  __shared__ int32_t wsum[16];
  __shared__ int32_t carry;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  if (tid == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base < n; base += 1024) {
    const int i = base + tid;
    const int v = i < n ? cnt[i] : 0;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o);
      if (lane >= o) x += y;
    }
    if (lane == 63) wsum[wv] = x;
    __syncthreads();
    int pre = carry;
    for (int q = 0; q < wv; ++q) pre += wsum[q];
    if (i < n) off[i] = pre + x - v;
    __syncthreads();
    if (tid == 1023) carry = pre + x;
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void draw_tile_fill_kernel(const int32_t* du, int rows, int N,
                                                             const int32_t* toff, int32_t* tfill,
                                                             int32_t* tlist) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)rows * N) return;
  const int tile = draw_tile_start(du, i, N);
  if (tile >= 0) tlist[toff[tile] + atomicAdd(&tfill[tile], 1)] = (int32_t)(i / N);
}

hipError_t launch_draw_tiles(const int32_t* dunit, int rows, int N, int nvt, int32_t* tcnt,
                             int32_t* toff, int32_t* tfill, int32_t* tlist, hipStream_t st) {
  if (rows <= 0 || nvt <= 0) return hipSuccess;
  const int zg = (int)std::min<int64_t>(ceil_div(nvt, 256), 1024);
  hipLaunchKernelGGL(draw_tiles_zero_kernel, dim3(zg), dim3(256), 0, st, tcnt, tfill, nvt);
  const int64_t dg = ceil_div((int64_t)rows * N, 256);
  if (dg > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(draw_tile_count_kernel, dim3((unsigned)dg), dim3(256), 0, st, dunit, rows, N,
                     tcnt);
  hipLaunchKernelGGL(draw_tile_scan_kernel, dim3(1), dim3(1024), 0, st, tcnt, nvt, toff);
  hipLaunchKernelGGL(draw_tile_fill_kernel, dim3((unsigned)dg), dim3(256), 0, st, dunit, rows, N,
                     toff, tfill, tlist);
  return hipGetLastError();
}

}  // namespace kd
