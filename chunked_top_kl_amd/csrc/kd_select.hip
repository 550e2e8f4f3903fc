// Top-fraction position selection by student entropy ("Rethinking Selective
// Knowledge Distillation", Method section 2: SE-KD keeps the top-k% most
// uncertain positions).
//
// The entropies from the projection sweep carry fp32 rounding (|error| <
// eps). The k-th largest value H_k is found by a radix select; positions with
// E > H_k + 2 eps are certainly kept, E < H_k - 2 eps certainly dropped, and
// the band in between is recomputed in fp64 from hidden and W (in pieces of
// at most kRefinePiece rows, whatever its size) and ranked by (entropy
// descending, position ascending). The kept set is then the one an fp64
// evaluation of the entropies decides.
#include <algorithm>

#include "kd_common.hpp"
#include "kd_kernels.hpp"

namespace kd {

__device__ inline unsigned long long ord_key(double e) {
  unsigned long long b = (unsigned long long)__double_as_longlong(e);
  return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}
__device__ inline double ord_inv(unsigned long long k) {
  unsigned long long b = (k >> 63) ? (k & 0x7FFFFFFFFFFFFFFFull) : ~k;
  return __longlong_as_double((long long)b);
}

// Single work-group: radix select of the k-th largest entropy, then the
// certain-keep count and the band list (ascending positions).
__global__ __launch_bounds__(1024) void select_threshold_kernel(const double* E, int64_t S,
                                                                int64_t k, double eps, SelectWs w) {
  __shared__ unsigned int hist[256];
  __shared__ unsigned long long s_prefix;
  __shared__ int64_t s_krem;
  __shared__ int32_t sc[1024];
  __shared__ int32_t sa[1024];
  const int tid = threadIdx.x;
  if (tid == 0) {
    s_prefix = 0ull;
    s_krem = k;
  }
  __syncthreads();
  unsigned long long mask = 0ull;
  for (int shift = 56; shift >= 0 && k > 0; shift -= 8) {
    if (tid < 256) hist[tid] = 0u;
    __syncthreads();
    const unsigned long long prefix = s_prefix;
    for (int64_t t = tid; t < S; t += 1024) {
      const unsigned long long key = ord_key(E[t]);
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid == 0) {
      int64_t krem = s_krem, cum = 0;
      int d = 255;
      for (; d > 0; --d) {
        if (cum + (int64_t)hist[d] >= krem) break;
        cum += hist[d];
      }
      s_krem = krem - cum;
      s_prefix = prefix | ((unsigned long long)d << shift);
    }
    mask |= 255ull << shift;
    __syncthreads();
  }
  const double hk = (k > 0) ? ord_inv(s_prefix) : INFINITY;
  const double delta = 2.0 * eps;
  // band list and certain-keep count
  const int64_t seg = ceil_div(S, 1024);
  const int64_t t0 = tid * seg, t1 = (t0 + seg < S) ? t0 + seg : S;
  int cb = 0, ca = 0;
  for (int64_t t = t0; t < t1; ++t) {
    const double e = E[t];
    if (e > hk + delta) ++ca;
    else if (e >= hk - delta) ++cb;
  }
  sc[tid] = cb;
  sa[tid] = ca;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int vb = tid >= o ? sc[tid - o] : 0;
    const int va = tid >= o ? sa[tid - o] : 0;
    __syncthreads();
    sc[tid] += vb;
    sa[tid] += va;
    __syncthreads();
  }
  int off = sc[tid] - cb;
  for (int64_t t = t0; t < t1; ++t) {
    const double e = E[t];
    if (!(e > hk + delta) && e >= hk - delta) w.band[off++] = (int32_t)t;
  }
  if (tid == 1023) {
    w.scal[0] = sc[1023];
    w.scal[1] = sa[1023];
    w.dscal[0] = hk;
    w.dscal[1] = delta;
  }
}

hipError_t launch_select_threshold(const double* entropy, int64_t S, int64_t k, double eps,
                                   const SelectWs& w, hipStream_t st) {
  hipLaunchKernelGGL(select_threshold_kernel, dim3(1), dim3(1024), 0, st, entropy, S, k, eps, w);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// fp64 entropy of band rows: z_v = sum_h x_h w_vh with fp64 products and sums
// (exact products of bf16 / fp32 inputs), then the online triple
// (m, s = sum e^(z-m), u = sum e^(z-m)(z-m)) over a vocabulary block.
// Partials rpart[row][blk] = (m, s, u).
// ---------------------------------------------------------------------------

// The band rows' hidden states widened to fp64 once: xb[r][h], r < n.
template <typename T>
__global__ __launch_bounds__(256) void band_rows_f64_kernel(const char* X, int64_t ldx, int H,
                                                            const int32_t* band, int off, int n,
                                                            double* xb) {
  const int64_t total = (int64_t)n * H;
  for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < total;
       q += (int64_t)gridDim.x * 256) {
    const int r = (int)(q / H), h = (int)(q % H);
    const char* src = X + (int64_t)band[off + r] * ldx;
    xb[q] = (sizeof(T) == 2) ? (double)bf16_to_f32(((const uint16_t*)src)[h])
                             : (double)((const float*)src)[h];
  }
}

// fp64 entropy partials of the band rows: z = x . w in fp64 from the exactly
// widened inputs, then the online (m, s, u) of each band row over the
// vocabulary rows of one tile. A work-group takes 8 band rows and a tile of
// 256 vocabulary rows; each lane holds 8 vocabulary rows x 8 band rows of
// sums. The 8 lanes that share a vocabulary row each take one 16-byte granule
// of h per step, so a load instruction reads 8 whole 128-byte lines. The band
// rows' values pass through LDS in pieces of kRefHc h, laid out [h][8 rows]
// with 16 bytes of padding after every 8 h so the 8 granules of a step fall
// in different banks; h past the end of a piece is zero there. Band rows past
// the end repeat the last one so every FMA is unconditional; their results
// are not written.
constexpr int kRefTR = 8;        // band rows per work-group
constexpr int kRefTV = 8;        // vocabulary rows per lane
constexpr int kRefTile = 256;    // vocabulary rows per work-group
constexpr int kRefHc = 1024;     // h per LDS piece
constexpr int kRefLdsDoubles = kRefHc * kRefTR + (kRefHc / 8) * 2;

__device__ __forceinline__ int ref_xs(int h, int r) { return h * kRefTR + (h >> 3) * 2 + r; }

// (m, s, u) of a set of logits: m the max, s = sum e^(z-m), u = sum e^(z-m)(z-m)
__device__ __forceinline__ void msu_merge(double& m1, double& s1, double& u1, double m2, double s2,
                                          double u2) {
  if (m2 == -INFINITY) return;
  if (m1 == -INFINITY) {
    m1 = m2;
    s1 = s2;
    u1 = u2;
    return;
  }
  const double mn = fmax(m1, m2), f1 = exp(m1 - mn), f2 = exp(m2 - mn);
  u1 = (u1 + s1 * (m1 - mn)) * f1 + (u2 + s2 * (m2 - mn)) * f2;
  s1 = s1 * f1 + s2 * f2;
  m1 = mn;
}

template <typename T>
__global__ __launch_bounds__(256) void refine_kernel(const double* __restrict__ xb, const char* Wm,
                                                     int64_t ldw, int V, int H, SelectWs w,
                                                     int band_off, int n, int nblk) {
  __shared__ __attribute__((aligned(16))) double xs[kRefLdsDoubles];
  __shared__ double red[3][4][kRefTR];
  // work-group order: the band groups of one vocabulary tile are consecutive
  // on one XCD (work-groups are dealt to the 8 XCDs in turn), so the tile's
  // W rows are fetched from HBM about once
  const int ng = (n + kRefTR - 1) / kRefTR;
  const int total = ng * nblk;
  const int per_xcd = (total + 7) / 8;
  const int logical = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
  if (logical >= total) return;
  const int grp = logical % ng, vt = logical / ng;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = lane & 7, a = lane >> 3;
  const int r0 = grp * kRefTR;
  const int nr = (n - r0) < kRefTR ? (n - r0) : kRefTR;
  const int vbase = vt * kRefTile + wave * 64 + a * kRefTV;
  int64_t roff[kRefTV];
#pragma unroll
  for (int j = 0; j < kRefTV; ++j) roff[j] = (int64_t)((vbase + j) < V ? vbase + j : V - 1) * ldw;
  constexpr int per = 16 / (int)sizeof(T);
  constexpr int step = 8 * per;
  double acc[kRefTV][kRefTR];
#pragma unroll
  for (int j = 0; j < kRefTV; ++j)
#pragma unroll
    for (int r = 0; r < kRefTR; ++r) acc[j][r] = 0.0;
  for (int hc = 0; hc < H; hc += kRefHc) {
    const int hn = (H - hc) < kRefHc ? (H - hc) : kRefHc;
    const int hp = (hn + step - 1) / step * step;
    __syncthreads();
    for (int q = tid; q < kRefTR * hp; q += 256) {
      const int r = q / hp, h = q % hp;
      const int rr = r < nr ? r : nr - 1;
      xs[ref_xs(h, r)] = h < hn ? xb[(int64_t)(r0 + rr) * H + hc + h] : 0.0;
    }
    __syncthreads();
    // W granules are loaded one step ahead; a granule past the end of the
    // row reads the row's first granule, and the band values it meets in LDS
    // are zero
    uint4 raw[kRefTV], nxt[kRefTV];
    {
      const int64_t ho = (int64_t)(b * per < hn ? hc + b * per : 0) * (int64_t)sizeof(T);
#pragma unroll
      for (int j = 0; j < kRefTV; ++j) raw[j] = *(const uint4*)(Wm + roff[j] + ho);
    }
    for (int hs = 0; hs < hp; hs += step) {
      const int h0 = hs + b * per;
      {
        const int hq = h0 + step;
        const int64_t ho = (int64_t)(hq < hn ? hc + hq : 0) * (int64_t)sizeof(T);
#pragma unroll
        for (int j = 0; j < kRefTV; ++j) nxt[j] = *(const uint4*)(Wm + roff[j] + ho);
        __builtin_amdgcn_sched_barrier(0);   // keep the loads ahead of this step's FMAs
      }
#pragma unroll
      for (int e = 0; e < per; ++e) {
        const double2* xp = (const double2*)(xs + ref_xs(h0 + e, 0));
        double xv[kRefTR];
#pragma unroll
        for (int r = 0; r < kRefTR / 2; ++r) {
          const double2 t = xp[r];
          xv[2 * r] = t.x;
          xv[2 * r + 1] = t.y;
        }
#pragma unroll
        for (int j = 0; j < kRefTV; ++j) {
          const uint32_t* wd = (const uint32_t*)&raw[j];
          double wv;
          if constexpr (sizeof(T) == 2) wv = (double)bf16_to_f32((uint16_t)(wd[e >> 1] >> ((e & 1) * 16)));
          else wv = (double)__uint_as_float(wd[e]);
#pragma unroll
          for (int r = 0; r < kRefTR; ++r) acc[j][r] = fma(xv[r], wv, acc[j][r]);
        }
      }
#pragma unroll
      for (int j = 0; j < kRefTV; ++j) raw[j] = nxt[j];
    }
  }
  // sum over the 8 granule lanes, leaving band row b's sums on lane b:
  // halve the band rows held at each of the three exchange steps
  double t4[kRefTV][4], t2[kRefTV][2], z[kRefTV];
  const bool u4 = (b & 4) != 0, u2 = (b & 2) != 0, u1 = (b & 1) != 0;
#pragma unroll
  for (int j = 0; j < kRefTV; ++j) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const double keep = u4 ? acc[j][r + 4] : acc[j][r];
      const double send = u4 ? acc[j][r] : acc[j][r + 4];
      t4[j][r] = keep + __shfl_xor(send, 4);
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const double keep = u2 ? t4[j][r + 2] : t4[j][r];
      const double send = u2 ? t4[j][r] : t4[j][r + 2];
      t2[j][r] = keep + __shfl_xor(send, 2);
    }
    const double keep = u1 ? t2[j][1] : t2[j][0];
    const double send = u1 ? t2[j][0] : t2[j][1];
    z[j] = keep + __shfl_xor(send, 1);
  }
  // (m, s, u) of band row b over this lane's 8 vocabulary rows
  double m = -INFINITY, sum = 0.0, uu = 0.0;
#pragma unroll
  for (int j = 0; j < kRefTV; ++j)
    if (vbase + j < V) m = fmax(m, z[j]);
  if (m != -INFINITY) {
#pragma unroll
    for (int j = 0; j < kRefTV; ++j) {
      if (vbase + j < V) {
        const double d = z[j] - m, e = exp(d);
        sum += e;
        uu += e * d;
      }
    }
  }
  // over the 8 lanes of the wave that hold the same band row, then the waves
#pragma unroll
  for (int o = 8; o < 64; o <<= 1) {
    const double m2 = __shfl_xor(m, o), s2 = __shfl_xor(sum, o), v2 = __shfl_xor(uu, o);
    msu_merge(m, sum, uu, m2, s2, v2);
  }
  if (a == 0) {
    red[0][wave][b] = m;
    red[1][wave][b] = sum;
    red[2][wave][b] = uu;
  }
  __syncthreads();
  if (tid < kRefTR && tid < nr) {
    double M = red[0][0][tid], Ssum = red[1][0][tid], U = red[2][0][tid];
    for (int q = 1; q < 4; ++q) msu_merge(M, Ssum, U, red[0][q][tid], red[1][q][tid], red[2][q][tid]);
    double* o = w.rpart + ((int64_t)(band_off + r0 + tid) * nblk + vt) * 3;
    o[0] = M;
    o[1] = Ssum;
    o[2] = U;
  }
}

// The same partials on the fp64 matrix cores (bf16 W): a work-group takes 16
// band rows and a tile of 256 vocabulary rows, each wave 64 of them as four
// 16 x 16 blocks of v_mfma_f64_16x16x4f64 (D[i][j] += sum over k < 4 of
// A[i][k] B[k][j]; lane l holds A[l%16][l/16] and B[l/16][l%16], and D[4r +
// l/16][l%16] in register r). The K order is permuted so that each lane loads
// whole 16-byte pieces: in a step of 32 h, lane l takes h = hs + 8 (l/16) + e
// for the MFMA of index e < 8, as both operands' k = l/16. Band rows past the
// end repeat the last one and vocabulary rows past V the last row; neither
// result is used. Every product is exact in fp64 (bf16 by widened bf16 or
// fp64-widened inputs) and the sums are fp64.
constexpr int kRefMR = 16;   // band rows per work-group
typedef double doublex4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void refine_mfma_kernel(const char* X, int64_t ldx,
                                                          const char* Wm, int64_t ldw, int V,
                                                          int H, SelectWs w, int band_off, int n,
                                                          int nblk) {
  __shared__ double red[3][4][kRefMR];
  // work-group order: the band groups of one vocabulary tile are consecutive
  // on one XCD, so the tile's W rows are fetched from HBM about once
  const int ng = (n + kRefMR - 1) / kRefMR;
  const int total = ng * nblk;
  const int per_xcd = (total + 7) / 8;
  const int logical = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
  if (logical >= total) return;
  const int grp = logical % ng, vt = logical / ng;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, q = lane >> 4;
  const int r0 = grp * kRefMR;
  const int nr = (n - r0) < kRefMR ? (n - r0) : kRefMR;
  // band rows past the end repeat the last one (their results are not kept)
  const int brow = w.band[band_off + r0 + (col < nr ? col : nr - 1)];
  const char* xr = X + (int64_t)brow * ldx + 16 * q;
  const int vb = vt * kRefTile + wave * 64 + col;
  const char* wr[4];
#pragma unroll
  for (int jb = 0; jb < 4; ++jb) {
    const int v = vb + 16 * jb;
    wr[jb] = Wm + (int64_t)(v < V ? v : V - 1) * ldw + 16 * q;
  }
  doublex4 acc[4];
#pragma unroll
  for (int jb = 0; jb < 4; ++jb) acc[jb] = doublex4{0.0, 0.0, 0.0, 0.0};
  // steps of 32 h: lane quarter q takes h = hs + 8q .. hs + 8q + 7, and MFMA e
  // of a step its element e (the same permutation of h on both operands)
  auto widen = [](const uint4& c, int e) {
    const uint32_t word = (e >> 1) == 0 ? c.x : (e >> 1) == 1 ? c.y : (e >> 1) == 2 ? c.z : c.w;
    return (double)__uint_as_float((e & 1) ? (word & 0xFFFF0000u) : (word << 16));
  };
  auto step = [&](const uint4 (&cw)[4], const uint4& cx) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const double a = widen(cx, e);
#pragma unroll
      for (int jb = 0; jb < 4; ++jb) {
        acc[jb] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, widen(cw[jb], e), acc[jb], 0, 0, 0);
      }
    }
  };
  // full steps: every lane's 8 h lie inside the row, so the loads need no
  // test. Two operand sets alternate: the next step's operands are loaded
  // before this step's MFMAs (the last load of the loop reloads a step in
  // bounds when there is no next one; it is not used)
  const int hfull = H & ~31;
  uint4 wa[4], wb[4], xa, xn;
  auto load = [&](uint4 (&wv)[4], uint4& xv, int hs) {
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) wv[jb] = *(const uint4*)(wr[jb] + (int64_t)hs * 2);
    xv = *(const uint4*)(xr + (int64_t)hs * 2);
  };
  {
    // the first step's operands through a select, so that the loop-carried
    // operands are not all plain loads (a PHI of loads would be folded into
    // one load at the top of the loop, which then waits for it at once)
    const bool in = hfull > 0;
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) wa[jb] = in ? *(const uint4*)wr[jb] : make_uint4(0u, 0u, 0u, 0u);
    xa = in ? *(const uint4*)xr : make_uint4(0u, 0u, 0u, 0u);
  }
  int hs = 0;
  // (the scheduling barriers keep each load ahead of the MFMAs it overlaps)
  for (; hs + 64 <= hfull; hs += 64) {
    load(wb, xn, hs + 32);
    __builtin_amdgcn_sched_barrier(0);
    step(wa, xa);
    load(wa, xa, hs + 64 < hfull ? hs + 64 : hs);
    __builtin_amdgcn_sched_barrier(0);
    step(wb, xn);
  }
  if (hs < hfull) step(wa, xa);   // an odd number of full steps: the last one
  if (hfull < H) {
    // the last, partial step: H is a multiple of 8, so a lane's 8 h are all
    // inside the row or all past it (then zeros)
    const bool in = hfull + 8 * q < H;
    uint4 tw[4];
#pragma unroll
    for (int jb = 0; jb < 4; ++jb)
      tw[jb] = in ? *(const uint4*)(wr[jb] + (int64_t)hfull * 2) : make_uint4(0u, 0u, 0u, 0u);
    const uint4 tx = in ? *(const uint4*)(xr + (int64_t)hfull * 2) : make_uint4(0u, 0u, 0u, 0u);
    step(tw, tx);
  }
  // (m, s, u) of band row 4r + q over this lane's 4 vocabulary rows, then over
  // the 16 lanes of the row (one per vocabulary column), then the 4 waves
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    double m = -INFINITY, sum = 0.0, uu = 0.0;
#pragma unroll
    for (int jb = 0; jb < 4; ++jb)
      if (vb + 16 * jb < V) m = fmax(m, acc[jb][r]);
    if (m != -INFINITY) {
#pragma unroll
      for (int jb = 0; jb < 4; ++jb) {
        if (vb + 16 * jb < V) {
          const double d = acc[jb][r] - m, ex = exp(d);
          sum += ex;
          uu += ex * d;
        }
      }
    }
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const double m2 = __shfl_xor(m, o), s2 = __shfl_xor(sum, o), v2 = __shfl_xor(uu, o);
      msu_merge(m, sum, uu, m2, s2, v2);
    }
    if (col == 0) {
      red[0][wave][4 * r + q] = m;
      red[1][wave][4 * r + q] = sum;
      red[2][wave][4 * r + q] = uu;
    }
  }
  __syncthreads();
  if (tid < kRefMR && tid < nr) {
    double M = red[0][0][tid], Ssum = red[1][0][tid], U = red[2][0][tid];
    for (int qq = 1; qq < 4; ++qq) msu_merge(M, Ssum, U, red[0][qq][tid], red[1][qq][tid], red[2][qq][tid]);
    double* o = w.rpart + ((int64_t)(band_off + r0 + tid) * nblk + vt) * 3;
    o[0] = M;
    o[1] = Ssum;
    o[2] = U;
  }
}

hipError_t launch_refine(int f32, const char* X, int64_t ldx, const char* W, int64_t ldw, int V,
                         int H, const SelectWs& w, double* xb, int band_off, int band_n, int nblk,
                         hipStream_t st) {
  if (band_n <= 0) return hipSuccess;
  const int64_t widen = ceil_div((int64_t)band_n * H, 256);
  const int64_t nwg = ceil_div((int64_t)ceil_div(band_n, kRefTR) * nblk, 8) * 8;
  if (nwg > INT32_MAX) return hipErrorInvalidValue;
  const dim3 grid((unsigned)nwg);
  if (f32) {
    hipLaunchKernelGGL(band_rows_f64_kernel<float>, dim3((unsigned)std::min<int64_t>(widen, 4096)),
                       dim3(256), 0, st, X, ldx, H, w.band, band_off, band_n, xb);
    hipLaunchKernelGGL(refine_kernel<float>, grid, dim3(256), 0, st, xb, W, ldw, V, H, w,
                       band_off, band_n, nblk);
  } else {
    // bf16 band rows are read in place (the fp64 widening is exact)
    const int64_t nwm = ceil_div((int64_t)ceil_div(band_n, kRefMR) * nblk, 8) * 8;
    if (nwm > INT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL(refine_mfma_kernel, dim3((unsigned)nwm), dim3(256), 0, st, X, ldx, W, ldw,
                       V, H, w, band_off, band_n, nblk);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Keep `need` of the n values vals[0..n), largest first, lower index first
// among equal values, by setting mask[tgt[b]] = 1 for each kept b. One
// work-group of 1024 threads: a radix select of the need-th largest value on
// order-preserving 64-bit keys (8 passes of 8 bits), then the entries above
// it and the first ties in index order. Every thread must call it.
// ---------------------------------------------------------------------------
struct BandKeepSmem {
  unsigned int hist[256];
  unsigned long long prefix;
  int64_t krem;
  int32_t sc[1024];
};

__device__ void band_keep(BandKeepSmem& sm, const double* vals, int n, int64_t need,
                          const int32_t* tgt, uint8_t* mask) {
  const int tid = threadIdx.x;
  if (need > n) need = n;
  if (need <= 0) return;
  if (tid == 0) {
    sm.prefix = 0ull;
    sm.krem = need;
  }
  __syncthreads();
  unsigned long long msk = 0ull;
  for (int shift = 56; shift >= 0; shift -= 8) {
    if (tid < 256) sm.hist[tid] = 0u;
    __syncthreads();
    const unsigned long long prefix = sm.prefix;
    for (int b = tid; b < n; b += 1024) {
      const unsigned long long key = ord_key(vals[b]);
      if ((key & msk) == prefix) atomicAdd(&sm.hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid == 0) {
      int64_t krem = sm.krem, cum = 0;
      int d = 255;
      for (; d > 0; --d) {
        if (cum + (int64_t)sm.hist[d] >= krem) break;
        cum += sm.hist[d];
      }
      sm.krem = krem - cum;
      sm.prefix = prefix | ((unsigned long long)d << shift);
    }
    msk |= 255ull << shift;
    __syncthreads();
  }
  // kstar: the need-th largest key; ties_kept of the entries equal to it are kept
  const unsigned long long kstar = sm.prefix;
  const int64_t ties_kept = sm.krem;
  const int seg = (n + 1023) / 1024;
  const int b0 = tid * seg, b1 = (b0 + seg < n) ? b0 + seg : n;
  int c = 0;
  for (int b = b0; b < b1; ++b) c += (ord_key(vals[b]) == kstar) ? 1 : 0;
  sm.sc[tid] = c;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int v = tid >= o ? sm.sc[tid - o] : 0;
    __syncthreads();
    sm.sc[tid] += v;
    __syncthreads();
  }
  int64_t r = sm.sc[tid] - c;   // ties before this thread's entries
  for (int b = b0; b < b1; ++b) {
    const unsigned long long key = ord_key(vals[b]);
    if (key > kstar) {
      mask[tgt[b]] = 1;
    } else if (key == kstar) {
      if (r < ties_kept) mask[tgt[b]] = 1;
      ++r;
    }
  }
  __syncthreads();
}

// Ascending list of the positions t < n with mask[t] set, and its length in
// *count (one work-group of 1024 threads; every thread must call it).
__device__ void mask_list(int32_t* sc, const uint8_t* mask, int64_t n, int32_t* idx_out,
                          int32_t* count) {
  const int tid = threadIdx.x;
  const int64_t seg = ceil_div(n, 1024);
  const int64_t t0 = tid * seg, t1 = (t0 + seg < n) ? t0 + seg : n;
  int c = 0;
  for (int64_t t = t0; t < t1; ++t) c += mask[t];
  sc[tid] = c;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int v = tid >= o ? sc[tid - o] : 0;
    __syncthreads();
    sc[tid] += v;
    __syncthreads();
  }
  if (idx_out) {
    int off = sc[tid] - c;
    for (int64_t t = t0; t < t1; ++t)
      if (mask[t]) idx_out[off++] = (int32_t)t;
  }
  if (tid == 1023) count[0] = sc[1023];
}

// ---------------------------------------------------------------------------
// Final decision (one work-group): positions above the band are kept; the
// band rows, whose fp64 entropies are in w.refined (band order = ascending
// position), are ranked by (entropy desc, position asc) and the first
// k - n_above kept; then the mask and the ascending index list.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void select_final_kernel(const double* E, int64_t S, int64_t k,
                                                            SelectWs w, int n_band, uint8_t* mask,
                                                            int32_t* idx_out) {
  __shared__ BandKeepSmem sm;
  const int tid = threadIdx.x;
  const double hk = w.dscal[0];
  const int n_above = w.scal[1];
  const double delta = w.dscal[1];
  for (int64_t t = tid; t < S; t += 1024) mask[t] = (E[t] > hk + delta) ? 1 : 0;
  __syncthreads();
  band_keep(sm, w.refined, n_band, k - n_above, w.band, mask);
  mask_list(sm.sc, mask, S, idx_out, w.scal + 2);
}

hipError_t launch_select_final(const double* entropy, int64_t S, int64_t k, const SelectWs& w,
                               int n_band, uint8_t* mask, int32_t* idx_out, hipStream_t st) {
  hipLaunchKernelGGL(select_final_kernel, dim3(1), dim3(1024), 0, st, entropy, S, k, w, n_band,
                     mask, idx_out);
  return hipGetLastError();
}

}  // namespace kd

namespace kd {

// ---------------------------------------------------------------------------
// Sample selection ("Rethinking Selective Knowledge Distillation", Method
// section 2, SE-KD3X sample axis: keep the top l% of training samples by the
// mean student entropy of a frozen student's forward pass). Sample b is the
// positions [off[b], off[b+1]). Its mean from the sweep's entropies is within
// eps of the fp64 mean (each term is); the k-th largest mean and the band
// within 2 eps of it come from select_threshold_kernel over the means, and
// when the band straddles the cut, the entropies of its samples' positions
// are recomputed in fp64 (refine_kernel) before the band is ranked by (mean
// descending, sample ascending).
// ---------------------------------------------------------------------------

__global__ void sample_zero_flag_kernel(int32_t* flag) {
  if (threadIdx.x == 0) flag[0] = 0;
}

// off must be non-decreasing within [0, S]; flag[0] = 1 otherwise
__global__ __launch_bounds__(256) void sample_offsets_check_kernel(const int64_t* off, int64_t B,
                                                                   int64_t S, int32_t* flag) {
  for (int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x; b <= B;
       b += (int64_t)gridDim.x * 256) {
    const int64_t o = off[b];
    bool bad = o < 0 || o > S;
    if (b < B) bad = bad || off[b + 1] < o;
    if (bad) flag[0] = 1;
  }
}

// means[b]: fp64 mean of E over the sample (threads' strided partial sums,
// then a fixed tree); -inf for an empty sample
__global__ __launch_bounds__(256) void sample_mean_kernel(const double* E, const int64_t* off,
                                                          int64_t B, double* means) {
  __shared__ double red[256];
  const int tid = threadIdx.x;
  for (int64_t b = blockIdx.x; b < B; b += gridDim.x) {
    const int64_t a0 = off[b], a1 = off[b + 1];
    double s = 0.0;
    for (int64_t t = a0 + tid; t < a1; t += 256) s += E[t];
    red[tid] = s;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
      if (tid < o) red[tid] += red[tid + o];
      __syncthreads();
    }
    if (tid == 0) means[b] = a1 > a0 ? red[0] / (double)(a1 - a0) : -INFINITY;
    __syncthreads();
  }
}

// flag[t] = 1 for every position t of a band sample (one work-group per band
// sample; samples may overlap)
__global__ __launch_bounds__(256) void sample_mark_kernel(const int64_t* off, SelectWs w,
                                                          int n_band, uint8_t* flag) {
  for (int i = blockIdx.x; i < n_band; i += gridDim.x) {
    const int64_t a0 = off[w.band[i]], a1 = off[w.band[i] + 1];
    for (int64_t t = a0 + threadIdx.x; t < a1; t += 256) flag[t] = 1;
  }
}

// w.refined[i]: fp64 mean over band sample i's positions of their refined
// entropies pent[pos[t]] (threads' strided partial sums, then a fixed tree);
// -inf for an empty sample
__global__ __launch_bounds__(256) void sample_band_mean_kernel(const int64_t* off, SelectWs w,
                                                               int n_band, const int32_t* pos,
                                                               const double* pent) {
  __shared__ double red[256];
  const int tid = threadIdx.x;
  for (int i = blockIdx.x; i < n_band; i += gridDim.x) {
    const int64_t a0 = off[w.band[i]], a1 = off[w.band[i] + 1];
    double s = 0.0;
    for (int64_t t = a0 + tid; t < a1; t += 256) s += pent[pos[t]];
    red[tid] = s;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
      if (tid < o) red[tid] += red[tid + o];
      __syncthreads();
    }
    if (tid == 0) w.refined[i] = a1 > a0 ? red[0] / (double)(a1 - a0) : -INFINITY;
    __syncthreads();
  }
}

// fp64 entropies of n refined positions from their partials (rows 0..n-1 of
// rpart), written to pent[0..n)
__global__ __launch_bounds__(256) void sample_refined_entropy_kernel(SelectWs w, int n, int nblk,
                                                                     double* pent) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b >= n) return;
  double M = -INFINITY, Ssum = 0.0, U = 0.0;
  for (int q = 0; q < nblk; ++q) {
    const double* o = w.rpart + ((int64_t)b * nblk + q) * 3;
    const double m2 = o[0], s2 = o[1], u2 = o[2];
    if (m2 == -INFINITY) continue;
    if (M == -INFINITY) {
      M = m2;
      Ssum = s2;
      U = u2;
      continue;
    }
    const double mn = fmax(M, m2), f1 = exp(M - mn), f2 = exp(m2 - mn);
    U = (U + Ssum * (M - mn)) * f1 + (u2 + s2 * (m2 - mn)) * f2;
    Ssum = Ssum * f1 + s2 * f2;
    M = mn;
  }
  pent[b] = log(Ssum) - U / Ssum;
}

// Final decision (one work-group): samples above the band are kept; the band
// (ascending sample order) is ranked by (mean desc, sample asc) on its fp64
// means in w.refined when `refined`, else on the sweep's means, and the first
// k - n_above kept; then the mask and the ascending list of kept samples.
__global__ __launch_bounds__(1024) void sample_final_kernel(const double* means, int64_t B,
                                                            int64_t k, SelectWs w, int n_band,
                                                            int refined, uint8_t* mask,
                                                            int32_t* idx_out) {
  __shared__ BandKeepSmem sm;
  const int tid = threadIdx.x;
  const double hk = w.dscal[0];
  const int n_above = w.scal[1];
  const double delta = w.dscal[1];
  if (!refined)
    for (int i = tid; i < n_band; i += 1024) w.refined[i] = means[w.band[i]];
  for (int64_t b = tid; b < B; b += 1024) mask[b] = (means[b] > hk + delta) ? 1 : 0;
  __syncthreads();
  band_keep(sm, w.refined, n_band, k - n_above, w.band, mask);
  mask_list(sm.sc, mask, B, idx_out, w.scal + 2);
}

hipError_t launch_sample_check(const int64_t* off, int64_t B, int64_t S, int32_t* flag,
                               hipStream_t st) {
  hipLaunchKernelGGL(sample_zero_flag_kernel, dim3(1), dim3(64), 0, st, flag);
  const int64_t grid = std::min<int64_t>(ceil_div(B + 1, 256), 4096);
  hipLaunchKernelGGL(sample_offsets_check_kernel, dim3((unsigned)grid), dim3(256), 0, st, off, B, S,
                     flag);
  return hipGetLastError();
}

hipError_t launch_sample_means(const double* E, const int64_t* off, int64_t B, double* means,
                               hipStream_t st) {
  if (B <= 0) return hipSuccess;
  hipLaunchKernelGGL(sample_mean_kernel, dim3((unsigned)std::min<int64_t>(B, 8192)), dim3(256), 0,
                     st, E, off, B, means);
  return hipGetLastError();
}

hipError_t launch_sample_mark(const int64_t* off, const SelectWs& w, int n_band, uint8_t* flag,
                              hipStream_t st) {
  if (n_band <= 0) return hipSuccess;
  hipLaunchKernelGGL(sample_mark_kernel, dim3((unsigned)std::min(n_band, 8192)), dim3(256), 0, st,
                     off, w, n_band, flag);
  return hipGetLastError();
}

hipError_t launch_sample_band_means(const int64_t* off, const SelectWs& w, int n_band,
                                    const int32_t* pos, const double* pent, hipStream_t st) {
  if (n_band <= 0) return hipSuccess;
  hipLaunchKernelGGL(sample_band_mean_kernel, dim3((unsigned)std::min(n_band, 8192)), dim3(256), 0,
                     st, off, w, n_band, pos, pent);
  return hipGetLastError();
}

hipError_t launch_sample_refined_entropy(const SelectWs& w, int n, int nblk, double* pent,
                                         hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(sample_refined_entropy_kernel, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0,
                     st, w, n, nblk, pent);
  return hipGetLastError();
}

hipError_t launch_sample_final(const double* means, int64_t B, int64_t k, const SelectWs& w,
                               int n_band, int refined, uint8_t* mask, int32_t* idx_out,
                               hipStream_t st) {
  hipLaunchKernelGGL(sample_final_kernel, dim3(1), dim3(1024), 0, st, means, B, k, w, n_band,
                     refined, mask, idx_out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Error probe: n positions spread evenly over [0, S) (list[i] = floor(i*S/n)),
// and the largest |E[list[i]] - ref[i]| over them (NaN terms are skipped).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void probe_list_kernel(int32_t* list, int n, int64_t S) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) list[i] = (int32_t)(((int64_t)i * S) / n);
}

__global__ __launch_bounds__(256) void max_abs_diff_kernel(const double* E, const int32_t* list,
                                                           int n, const double* ref, double* out) {
  __shared__ double red[256];
  const int tid = threadIdx.x;
  double m = 0.0;
  for (int i = tid; i < n; i += 256) m = fmax(m, fabs(E[list[i]] - ref[i]));
  red[tid] = m;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (tid < o) red[tid] = fmax(red[tid], red[tid + o]);
    __syncthreads();
  }
  if (tid == 0) *out = red[0];
}

hipError_t launch_probe_list(int32_t* list, int n, int64_t S, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(probe_list_kernel, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, st, list,
                     n, S);
  return hipGetLastError();
}

hipError_t launch_max_abs_diff(const double* E, const int32_t* list, int n, const double* ref,
                               double* out, hipStream_t st) {
  hipLaunchKernelGGL(max_abs_diff_kernel, dim3(1), dim3(256), 0, st, E, list, n, ref, out);
  return hipGetLastError();
}

}  // namespace kd
