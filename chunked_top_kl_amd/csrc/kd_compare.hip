// The two comparator forms of the loss that "Making Knowledge Distillation
// Cheap Enough to Run at Scale" (section "what chunked KL loss does")
// measures against the fused chunked loss:
//  - dense: the cached top-K entries expanded into a dense teacher
//    probability grid P [rows][V], the student's log-probabilities over the
//    whole grid logQ [rows][V], KL per row from the two grids; the backward
//    takes the logit gradient from the stored grids;
//  - forward-chunked: the teacher stays sparse and positions are processed
//    chunk by chunk, but the student logits Z [rows][V] of every row are kept
//    for the backward, which takes the logit gradient from them instead of
//    projecting again.
// Both start from the bf16 logits that the projection sweep stores (the
// logits kind of kd_sweep.hip); the contractions of the backward are the
// fused path's dHidden and dW kernels. These kernels are HBM-bound passes
// over [rows][V] grids: one work-group per row, 16-byte accesses along V.
#include "kd_common.hpp"
#include "kd_kernels.hpp"

namespace kd {

namespace {

__device__ inline int cmp_rows(const int32_t* nrows_dev, int row_begin, int row_cap) {
  int n = *nrows_dev - row_begin;
  return n < row_cap ? n : row_cap;
}

// 8 bf16 values of a 16-byte granule, widened
__device__ inline void unpack8(const uint4 g, float (&x)[8]) {
  const uint32_t w[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[2 * e] = __uint_as_float(w[e] << 16);
    x[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
  }
}

__device__ inline uint4 pack8(const float (&x)[8]) {
  uint32_t w[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) w[e] = f32_to_bf16_bits(x[2 * e]) | (f32_to_bf16_bits(x[2 * e + 1]) << 16);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// block-wide max and sum (256 threads)
__device__ inline float block_max(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  v = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  return v;
}

__device__ inline double block_sum(double v, double* red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  v = (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();
  return v;
}

// log-normaliser of z/T over the row's V stored logits (bf16)
__device__ inline float row_lse(const uint16_t* z, int V, float invT, float* redf, double* redd) {
  const int tid = threadIdx.x;
  const int ng = V / 8;
  float m = -INFINITY;
  for (int g = tid; g < ng; g += 256) {
    float x[8];
    unpack8(*(const uint4*)(z + 8 * g), x);
#pragma unroll
    for (int e = 0; e < 8; ++e) m = fmaxf(m, x[e]);
  }
  for (int v = 8 * ng + tid; v < V; v += 256) m = fmaxf(m, __uint_as_float((uint32_t)z[v] << 16));
  m = block_max(m, redf);
  const float ms = m * invT;
  float s = 0.0f;
  for (int g = tid; g < ng; g += 256) {
    float x[8];
    unpack8(*(const uint4*)(z + 8 * g), x);
#pragma unroll
    for (int e = 0; e < 8; ++e) s += __expf(fmaf(x[e], invT, -ms));
  }
  for (int v = 8 * ng + tid; v < V; v += 256)
    s += __expf(fmaf(__uint_as_float((uint32_t)z[v] << 16), invT, -ms));
  const double S = block_sum((double)s, redd);
  return ms + (float)log(S);
}

}  // namespace

// Forward-chunked: per row of a chunk, lse_t = log-normaliser of z/T over the
// stored row, and KL_t = negH_t - sum_k p_k z_{id_k} / T + lse_t over the
// row's usable teacher entries (the id-sorted tables of the prepass).
__global__ __launch_bounds__(256) void cmp_kl_sparse_kernel(CmpRowArgs a) {
  __shared__ float redf[4];
  __shared__ double redd[4];
  const int rows = cmp_rows(a.nrows_dev, a.row_begin, a.row_cap);
  const int r = blockIdx.x;
  if (r >= rows) return;
  const int cr = a.row_begin + r;
  const int t = a.idx[cr];
  const float invT = 1.0f / a.T;
  const uint16_t* z = a.Z + (int64_t)cr * a.ldz;
  const float lse = row_lse(z, a.V, invT, redf, redd);
  double dot = 0.0;
  const int64_t base = (int64_t)t * a.K;
  for (int k = threadIdx.x; k < a.K; k += 256) {
    const int id = a.ids_s[base + k];
    if (id == 0x7FFFFFFF) continue;   // out-of-range ids sort last and take no part
    dot += (double)a.p_s[base + k] * (double)__uint_as_float((uint32_t)z[id] << 16);
  }
  dot = block_sum(dot, redd);
  if (threadIdx.x == 0) {
    a.lse[t] = lse;
    a.kl[t] = (float)((double)a.negH[t] - dot * (double)invT + (double)lse);
  }
}

// Dense: the teacher grid P[r][v] of the chunk's rows: zeros, then at each
// teacher id the summed probability of its run of equal ids.
__global__ __launch_bounds__(256) void cmp_dense_grid_kernel(CmpRowArgs a) {
  const int rows = cmp_rows(a.nrows_dev, a.row_begin, a.row_cap);
  const int r = blockIdx.x;
  if (r >= rows) return;
  const int cr = a.row_begin + r;
  const int t = a.idx[cr];
  float* P = a.P + (int64_t)cr * a.ldd;
  for (int v = threadIdx.x; v < a.Vp; v += 256) P[v] = 0.0f;
  __syncthreads();
  const int64_t base = (int64_t)t * a.K;
  for (int k = threadIdx.x; k < a.K; k += 256) {
    const int id = a.ids_s[base + k];
    if (id == 0x7FFFFFFF || (k > 0 && a.ids_s[base + k - 1] == id)) continue;
    float p = 0.0f;
    for (int q = k; q < a.K && a.ids_s[base + q] == id; ++q) p += a.p_s[base + q];
    P[id] = p;
  }
}

// Dense: logQ[r][v] = z/T - lse over the row (-inf past V), and
// KL_t = sum over v with P > 0 of P (log P - logQ), read from the two grids.
__global__ __launch_bounds__(256) void cmp_kl_dense_kernel(CmpRowArgs a) {
  __shared__ float redf[4];
  __shared__ double redd[4];
  const int rows = cmp_rows(a.nrows_dev, a.row_begin, a.row_cap);
  const int r = blockIdx.x;
  if (r >= rows) return;
  const int cr = a.row_begin + r;
  const int t = a.idx[cr];
  const float invT = 1.0f / a.T;
  const uint16_t* z = a.Z + (int64_t)cr * a.ldz;
  const float lse = row_lse(z, a.V, invT, redf, redd);
  float* lq = a.logQ + (int64_t)cr * a.ldd;
  const float* P = a.P + (int64_t)cr * a.ldd;
  double kl = 0.0;
  for (int v = threadIdx.x; v < a.Vp; v += 256) {
    if (v >= a.V) {
      lq[v] = -INFINITY;
      continue;
    }
    const float q = fmaf(__uint_as_float((uint32_t)z[v] << 16), invT, -lse);
    lq[v] = q;
    const float p = P[v];
    if (p > 0.0f) kl += (double)p * ((double)__logf(p) - (double)q);
  }
  kl = block_sum(kl, redd);
  if (threadIdx.x == 0) {
    a.lse[t] = lse;
    a.kl[t] = (float)kl;
  }
}

// Logit gradient of a chunk's rows into G (bf16, zeros in [V, Vp)), stored in
// blocks of 256 columns as the fused path stores it (rows 256 elements apart
// inside a block, blocks ldg elements apart):
//   forward-chunked: coef (exp(z/T - lse) - p) with p at the teacher ids
//     (summed over a run of equal ids), from the stored logits;
//   dense: coef (exp(logQ) - P) from the stored grids;
// coef = grad_loss / (T N). Rows in [rows, round_up(rows, 8)) are written as
// zeros: the dW contraction reads whole groups of 8 rows.
template <bool DENSE>
__global__ __launch_bounds__(256) void cmp_grad_kernel(CmpRowArgs a) {
  const int rows = cmp_rows(a.nrows_dev, a.row_begin, a.row_cap);
  const int r = blockIdx.x;
  if (r >= ((rows + 7) & ~7)) return;
  // granule g (8 columns) of row r
  uint16_t* G = a.G + (int64_t)r * 256;
  auto gran = [&](int g) { return G + (int64_t)(g >> 5) * a.ldg + 8 * (g & 31); };
  if (r >= rows) {
    for (int g = threadIdx.x; g < a.Vp / 8; g += 256) *(uint4*)gran(g) = make_uint4(0u, 0u, 0u, 0u);
    return;
  }
  const int cr = a.row_begin + r;
  const int t = a.idx[cr];
  const int n = *a.nrows_dev;
  const float coef = n > 0 ? a.grad_loss[0] / ((float)n * a.T) : 0.0f;
  const float invT = 1.0f / a.T;
  const float lse = a.lse[t];
  const uint16_t* z = a.Z + (int64_t)cr * a.ldz;
  const int ng = a.Vp / 8;
  for (int g = threadIdx.x; g < ng; g += 256) {
    float x[8];
    if constexpr (DENSE) {
      const float* lq = a.logQ + (int64_t)cr * a.ldd + 8 * g;
      const float* P = a.P + (int64_t)cr * a.ldd + 8 * g;
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = (8 * g + e < a.V) ? coef * (__expf(lq[e]) - P[e]) : 0.0f;
    } else {
      unpack8(*(const uint4*)(z + 8 * g), x);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        x[e] = (8 * g + e < a.V) ? coef * __expf(fmaf(x[e], invT, -lse)) : 0.0f;
    }
    *(uint4*)gran(g) = pack8(x);
  }
  if constexpr (!DENSE) {
    __syncthreads();
    const int64_t base = (int64_t)t * a.K;
    for (int k = threadIdx.x; k < a.K; k += 256) {
      const int id = a.ids_s[base + k];
      if (id == 0x7FFFFFFF || (k > 0 && a.ids_s[base + k - 1] == id)) continue;
      float p = 0.0f;
      for (int q = k; q < a.K && a.ids_s[base + q] == id; ++q) p += a.p_s[base + q];
      const float qv = __expf(fmaf(__uint_as_float((uint32_t)z[id] << 16), invT, -lse));
      gran(id >> 3)[id & 7] = (uint16_t)f32_to_bf16_bits(coef * (qv - p));
    }
  }
}

// Loss from the per-row KL: rows in the loss (pos >= 0) summed per block (a
// fixed tree), rows outside it get lse = kl = 0.
__global__ __launch_bounds__(256) void cmp_loss_blocks_kernel(const int32_t* pos, int64_t S,
                                                              float* lse, float* kl,
                                                              float* kl_out, double* block_sums) {
  __shared__ double red[256];
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  double c = 0.0;
  if (t < S) {
    if (pos[t] < 0) {
      lse[t] = 0.0f;
      kl[t] = 0.0f;
    } else {
      c = kl[t];
    }
    if (kl_out) kl_out[t] = kl[t];
  }
  red[threadIdx.x] = c;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) block_sums[blockIdx.x] = red[0];
}

hipError_t launch_cmp_rows(int what, const CmpRowArgs& a, hipStream_t st) {
  if (a.row_cap <= 0) return hipSuccess;
  // the gradient kinds also cover the zero rows up to round_up(rows, 8)
  const bool grad = what == kCmpGradSparse || what == kCmpGradDense;
  const dim3 g((unsigned)(grad ? round_up(a.row_cap, 8) : a.row_cap)), b(256);
  switch (what) {
    case kCmpKlSparse: hipLaunchKernelGGL(cmp_kl_sparse_kernel, g, b, 0, st, a); break;
    case kCmpDenseGrid: hipLaunchKernelGGL(cmp_dense_grid_kernel, g, b, 0, st, a); break;
    case kCmpKlDense: hipLaunchKernelGGL(cmp_kl_dense_kernel, g, b, 0, st, a); break;
    case kCmpGradSparse: hipLaunchKernelGGL(cmp_grad_kernel<false>, g, b, 0, st, a); break;
    case kCmpGradDense: hipLaunchKernelGGL(cmp_grad_kernel<true>, g, b, 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_cmp_loss(const int32_t* pos, int64_t S, float* lse, float* kl, float* kl_out,
                           double* block_sums, const int32_t* nrows_dev, float* loss,
                           hipStream_t st) {
  const int nblk = (int)ceil_div(S, 256);
  if (nblk > 0)
    hipLaunchKernelGGL(cmp_loss_blocks_kernel, dim3(nblk), dim3(256), 0, st, pos, S, lse, kl,
                       kl_out, block_sums);
  return launch_loss_final(block_sums, nblk, nrows_dev, loss, st);
}

}  // namespace kd
