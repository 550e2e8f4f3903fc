// Top-fraction position selection by student entropy ("Rethinking Selective
// Knowledge Distillation", Method section 2: SE-KD keeps the top-k% most
// uncertain positions).
//
// The entropies from the projection sweep carry fp32 rounding (|error| <
// eps). The k-th largest value H_k is found by a radix select; positions with
// E > H_k + 2 eps are certainly kept, E < H_k - 2 eps certainly dropped, and
// the band in between is recomputed in fp64 from hidden and W and ranked by
// (entropy descending, position ascending). The kept set is then the one an
// fp64 evaluation of the entropies decides.
#include "kd_common.hpp"
#include "kd_kernels.hpp"

namespace kd {

constexpr int kBandCap = 4096;   // band rows refined in fp64; above this the fp32 values decide

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
constexpr int kRefineRows = 16;
constexpr int kRefineLdsBytes = 96 * 1024;

int refine_rows_per_pass(int H, int /*f32*/) {
  int r = kRefineLdsBytes / (H * 4);
  if (r > kRefineRows) r = kRefineRows;
  if (r < 1) r = 1;
  return r;
}

template <typename T, int R>
__global__ __launch_bounds__(256) void refine_kernel(const char* X, int64_t ldx, const char* Wm,
                                                     int64_t ldw, int V, int H, SelectWs w,
                                                     int band_off, int band_n, int nblk) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  float* xs = (float*)smem;                       // [R][H]
  __shared__ double red[3][256];
  const int tid = threadIdx.x;
  const int nr = band_n < R ? band_n : R;
  for (int q = tid; q < nr * H; q += 256) {
    const int r = q / H, h = q % H;
    const int64_t row = w.band[band_off + r];
    const char* src = X + row * ldx;
    xs[q] = (sizeof(T) == 2) ? bf16_to_f32(((const uint16_t*)src)[h]) : ((const float*)src)[h];
  }
  __syncthreads();
  const int vper = (int)ceil_div(V, nblk);
  const int v0 = blockIdx.x * vper;
  const int v1 = (v0 + vper < V) ? v0 + vper : V;
  double m[R], s[R], u[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    m[r] = -INFINITY;
    s[r] = 0.0;
    u[r] = 0.0;
  }
  for (int v = v0 + tid; v < v1; v += 256) {
    double acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.0;
    const char* wr = Wm + (int64_t)v * ldw;
    constexpr int per = 16 / (int)sizeof(T);
    for (int h = 0; h < H; h += per) {
      const uint4 raw = *(const uint4*)(wr + (int64_t)h * sizeof(T));
      const uint32_t* wd = (const uint32_t*)&raw;
#pragma unroll
      for (int e = 0; e < per; ++e) {
        double wv;
        if constexpr (sizeof(T) == 2) wv = (double)bf16_to_f32((uint16_t)(wd[e >> 1] >> ((e & 1) * 16)));
        else wv = (double)__uint_as_float(wd[e]);
#pragma unroll
        for (int r = 0; r < R; ++r)
          if (r < nr) acc[r] = fma((double)xs[r * H + h + e], wv, acc[r]);
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (r >= nr) continue;
      const double z = acc[r];
      if (z > m[r]) {
        if (m[r] == -INFINITY) {
          s[r] = 0.0;
          u[r] = 0.0;
        } else {
          const double f = exp(m[r] - z);
          u[r] = (u[r] + s[r] * (m[r] - z)) * f;
          s[r] = s[r] * f;
        }
        m[r] = z;
      }
      const double d = z - m[r];
      const double e = exp(d);
      s[r] += e;
      u[r] += e * d;
    }
  }
  // block merge per row (fixed tree order)
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (r >= nr) continue;  // uniform
    red[0][tid] = m[r];
    red[1][tid] = s[r];
    red[2][tid] = u[r];
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
      if (tid < o) {
        double m1 = red[0][tid], s1 = red[1][tid], u1 = red[2][tid];
        const double m2 = red[0][tid + o], s2 = red[1][tid + o], u2 = red[2][tid + o];
        if (m2 != -INFINITY) {
          if (m1 == -INFINITY) {
            m1 = m2; s1 = s2; u1 = u2;
          } else {
            const double mn = fmax(m1, m2), f1 = exp(m1 - mn), f2 = exp(m2 - mn);
            u1 = (u1 + s1 * (m1 - mn)) * f1 + (u2 + s2 * (m2 - mn)) * f2;
            s1 = s1 * f1 + s2 * f2;
            m1 = mn;
          }
        }
        red[0][tid] = m1;
        red[1][tid] = s1;
        red[2][tid] = u1;
      }
      __syncthreads();
    }
    if (tid == 0) {
      double* o = w.rpart + ((int64_t)(band_off + r) * nblk + blockIdx.x) * 3;
      o[0] = red[0][0];
      o[1] = red[1][0];
      o[2] = red[2][0];
    }
    __syncthreads();
  }
}

hipError_t launch_refine(int f32, const char* X, int64_t ldx, const char* W, int64_t ldw, int V,
                         int H, const SelectWs& w, int band_off, int band_n, int nblk,
                         hipStream_t st) {
  const size_t lds = (size_t)refine_rows_per_pass(H, f32) * H * 4;
  if (f32)
    hipLaunchKernelGGL((refine_kernel<float, kRefineRows>), dim3(nblk), dim3(256), lds, st, X, ldx,
                       W, ldw, V, H, w, band_off, band_n, nblk);
  else
    hipLaunchKernelGGL((refine_kernel<__bf16, kRefineRows>), dim3(nblk), dim3(256), lds, st, X,
                       ldx, W, ldw, V, H, w, band_off, band_n, nblk);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Final decision (single work-group): refined band entropies, rank within the
// band by (entropy desc, position asc), mask and ascending index list.
// n_band <= kBandCap uses the fp64 values; a larger band is ranked on the
// fp32-path values.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void select_final_kernel(const double* E, int64_t S, int64_t k,
                                                            SelectWs w, int n_band, int nblk,
                                                            uint8_t* mask, int32_t* idx_out) {
  __shared__ int32_t sc[1024];
  const int tid = threadIdx.x;
  const double hk = w.dscal[0];
  const int n_above = w.scal[1];
  const double delta = w.dscal[1];
  const bool refined = n_band <= kBandCap;
  // 1. refined entropies of band rows
  for (int b = tid; b < n_band; b += 1024) {
    double val;
    if (refined) {
      double M = -INFINITY, Ssum = 0.0, U = 0.0;
      for (int q = 0; q < nblk; ++q) {
        const double* o = w.rpart + ((int64_t)b * nblk + q) * 3;
        const double m2 = o[0], s2 = o[1], u2 = o[2];
        if (m2 == -INFINITY) continue;
        if (M == -INFINITY) {
          M = m2; Ssum = s2; U = u2;
          continue;
        }
        const double mn = fmax(M, m2), f1 = exp(M - mn), f2 = exp(m2 - mn);
        U = (U + Ssum * (M - mn)) * f1 + (u2 + s2 * (m2 - mn)) * f2;
        Ssum = Ssum * f1 + s2 * f2;
        M = mn;
      }
      val = log(Ssum) - U / Ssum;
    } else {
      val = E[w.band[b]];
    }
    w.refined[b] = val;
  }
  // 2. mask of certain keeps
  for (int64_t t = tid; t < S; t += 1024) mask[t] = (E[t] > hk + delta) ? 1 : 0;
  __syncthreads();
  // 3. band rows ranked by (refined desc, position asc); keep the first k - n_above
  const int64_t need = k - n_above;
  for (int b = tid; b < n_band; b += 1024) {
    const double vb = w.refined[b];
    const int32_t tb = w.band[b];
    int64_t rank = 0;
    for (int q = 0; q < n_band; ++q) {
      const double vq = w.refined[q];
      rank += (vq > vb || (vq == vb && w.band[q] < tb)) ? 1 : 0;
    }
    if (rank < need) mask[tb] = 1;
  }
  __syncthreads();
  // 4. ascending index list of kept positions
  const int64_t seg = ceil_div(S, 1024);
  const int64_t t0 = tid * seg, t1 = (t0 + seg < S) ? t0 + seg : S;
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
  if (tid == 1023) w.scal[2] = sc[1023];
}

hipError_t launch_select_final(const double* entropy, int64_t S, int64_t k, const SelectWs& w,
                               int n_band, int nblk, uint8_t* mask, int32_t* idx_out,
                               hipStream_t st) {
  hipLaunchKernelGGL(select_final_kernel, dim3(1), dim3(1024), 0, st, entropy, S, k, w, n_band,
                     nblk, mask, idx_out);
  return hipGetLastError();
}

}  // namespace kd
