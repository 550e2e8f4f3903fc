// Position importance signals and selection policies ("Rethinking Selective
// Knowledge Distillation", Method section 1: the signals compared are the
// student's cross-entropy, the teacher's uncertainty 1 - p_t(y_t), the
// teacher-student KL and the student's entropy; the policies include top-k%
// selection and a global threshold).
//
//  signals_kernel      one wave per position: ce_t = lse_t - z_{t,y_t} (the
//                      student at T = 1, lse_t from the entropy sweep, z_{t,y}
//                      a dot product of exact products summed in fp64), and
//                      1 - p_t(y_t) with p_t the row's KD target in fp64 (the
//                      usable entries and the "present" rule of the prepass).
//  select_segments     one work-group per segment: the floor(num*len/den)
//                      largest non-NaN signals, lower index first among equal
//                      values, found by an 8-pass radix select on order
//                      preserving 64-bit keys, then an ordered pass that keeps
//                      the first ties.
//  select_above        signal >= tau (NaN never).
#include "kd_common.hpp"
#include "kd_kernels.hpp"

namespace kd {

__device__ inline double elem_hw(const char* row, int h, int f32) {
  return f32 ? (double)((const float*)row)[h] : (double)bf16_to_f32(((const uint16_t*)row)[h]);
}

__device__ inline double load_tl(const void* tl, int tl_f32, int64_t i) {
  return tl_f32 ? (double)((const float*)tl)[i] : (double)bf16_to_f32(((const uint16_t*)tl)[i]);
}

__global__ __launch_bounds__(256) void signals_kernel(SignalArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.S) return;
  const int y = a.labels ? a.labels[t] : -1;
  const bool has = y >= 0 && y < a.V;
  if (a.ce) {
    // z_{t,y}: each product of two bf16 (or fp32) values is exact in fp64
    double acc = 0.0;
    if (has) {
      const char* hr = a.hidden + t * a.ldh;
      const char* wr = a.W + (int64_t)y * a.ldw;
      for (int h = lane; h < a.H; h += 64) acc += elem_hw(hr, h, a.hw_f32) * elem_hw(wr, h, a.hw_f32);
    }
    acc = wave_sum_d(acc);
    if (lane == 0) a.ce[t] = has ? a.lse[t] - acc : __builtin_nan("");
  }
  if (a.tunc) {
    const int64_t base = t * a.K;
    // 1. flags and row maximum over the usable entries (id in [0, V), finite)
    double mx = -INFINITY;
    int bad = 0;
    for (int k = lane; k < a.K; k += 64) {
      const int id = a.ids[base + k];
      const double l = load_tl(a.tl, a.tl_f32, base + k);
      if (a.probs) {
        if (!(isfinite(l) && l >= 0.0)) bad = 1;
      } else {
        if (isnan(l) || l == INFINITY) bad = 1;
        if (id >= 0 && id < a.V && isfinite(l)) mx = fmax(mx, l * a.invT);
      }
    }
    for (int o = 32; o > 0; o >>= 1) mx = fmax(mx, __shfl_xor(mx, o, 64));
    bad = __any(bad);
    // 2. the row's total weight and the weight at the label
    double tot = 0.0, hit = 0.0;
    if (a.probs || mx != -INFINITY) {
      for (int k = lane; k < a.K; k += 64) {
        const int id = a.ids[base + k];
        const double l = load_tl(a.tl, a.tl_f32, base + k);
        if (id >= 0 && id < a.V && isfinite(l)) {
          const double wgt = a.probs ? (l > 0.0 ? l : 0.0) : exp(l * a.invT - mx);
          tot += wgt;
          if (id == y) hit += wgt;
        }
      }
    }
    tot = wave_sum_d(tot);
    hit = wave_sum_d(hit);
    const bool present = !bad && (a.probs ? tot > 0.0 : mx != -INFINITY);
    if (lane == 0) a.tunc[t] = (has && present) ? 1.0 - hit / tot : __builtin_nan("");
  }
}

hipError_t launch_signals(const SignalArgs& a, hipStream_t st) {
  if (a.S <= 0) return hipSuccess;
  hipLaunchKernelGGL(signals_kernel, dim3((unsigned)ceil_div(a.S, 4)), dim3(256), 0, st, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Order-preserving key of a non-NaN double (-0 taken as +0): larger value,
// larger key.
__device__ inline unsigned long long dkey(double x) {
  x = x + 0.0;   // -0 -> +0
  const unsigned long long u = (unsigned long long)__double_as_longlong(x);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

__device__ inline double dkey_value(unsigned long long k) {
  const unsigned long long u = (k >> 63) ? (k & 0x7FFFFFFFFFFFFFFFull) : ~k;
  return __longlong_as_double((long long)u);
}

// exclusive prefix of `v` over the 256 threads in index order; `tot` = sum
__device__ inline int block_scan_excl(int v, int& tot, int* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) red[w] = x;
  __syncthreads();
  int before = 0;
  tot = 0;
  for (int i = 0; i < 4; ++i) {
    if (i < w) before += red[i];
    tot += red[i];
  }
  __syncthreads();
  return before + x - v;
}

__global__ __launch_bounds__(256) void select_segments_kernel(const double* x,
                                                              const int64_t* off, int64_t S,
                                                              int64_t num, int64_t den,
                                                              uint8_t* mask, double* thr) {
  __shared__ unsigned int hist[4][256];
  __shared__ int red[4];
  __shared__ unsigned long long s_prefix;
  __shared__ int s_want;
  const int tid = threadIdx.x, w = tid >> 6;
  const int64_t b = blockIdx.x;
  const int64_t a0 = off ? off[b] : 0, a1 = off ? off[b + 1] : S;
  const int64_t len = a1 - a0;
  // candidates: the non-NaN signals
  int nc = 0;
  for (int64_t t = a0 + tid; t < a1; t += 256) nc += isnan(x[t]) ? 0 : 1;
  int ncand = 0;
  block_scan_excl(nc, ncand, red);
  // num <= den < 2^31 and len < 2^31 (checked on the host): no overflow
  int64_t k = (num * len) / den;
  if (k > ncand) k = ncand;
  if (k <= 0) {
    for (int64_t t = a0 + tid; t < a1; t += 256) mask[t] = 0;
    if (thr && tid == 0) thr[b] = __builtin_nan("");
    return;
  }
  // radix select of the k-th largest key, 8 bits at a time from the top
  unsigned long long prefix = 0;
  int want = (int)k;   // elements still to take at or below the current prefix
  for (int pass = 7; pass >= 0; --pass) {
    const int shift = pass * 8;
    for (int i = tid; i < 4 * 256; i += 256) (&hist[0][0])[i] = 0;
    __syncthreads();
    const unsigned long long hmask = pass == 7 ? 0ull : (~0ull << (shift + 8));
    for (int64_t t = a0 + tid; t < a1; t += 256) {
      const double v = x[t];
      if (isnan(v)) continue;
      const unsigned long long kk = dkey(v);
      if ((kk & hmask) == prefix) atomicAdd(&hist[w][(kk >> shift) & 255], 1u);
    }
    __syncthreads();
    if (tid == 0) {
      int acc = 0, d = 255;
      for (; d > 0; --d) {
        const int c = (int)(hist[0][d] + hist[1][d] + hist[2][d] + hist[3][d]);
        if (acc + c >= want) break;
        acc += c;
      }
      s_prefix = prefix | ((unsigned long long)d << shift);
      s_want = want - acc;
    }
    __syncthreads();
    prefix = s_prefix;
    want = s_want;
    __syncthreads();
  }
  // prefix is the k-th largest key; keep every larger key and the first
  // `want` equal ones in index order
  int seen = 0;
  for (int64_t c0 = a0; c0 < a1; c0 += 256) {
    const int64_t t = c0 + tid;
    bool gt = false, eq = false;
    if (t < a1) {
      const double v = x[t];
      if (!isnan(v)) {
        const unsigned long long kk = dkey(v);
        gt = kk > prefix;
        eq = kk == prefix;
      }
    }
    int neq = 0;
    const int r = block_scan_excl(eq ? 1 : 0, neq, red);
    if (t < a1) mask[t] = (gt || (eq && seen + r < want)) ? 1 : 0;
    seen += neq;
  }
  if (thr && tid == 0) thr[b] = dkey_value(prefix);
}

hipError_t launch_select_segments(const double* x, const int64_t* off, int64_t B, int64_t S,
                                  int64_t num, int64_t den, uint8_t* mask, double* thr,
                                  hipStream_t st) {
  if (B <= 0) return hipSuccess;
  hipLaunchKernelGGL(select_segments_kernel, dim3((unsigned)B), dim3(256), 0, st, x, off, S, num,
                     den, mask, thr);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Per-sequence top-k% by student entropy, decided as fp64 entropies decide.
// The sweep's entropies E are within eps of fp64, so with T_b the k_b-th
// largest E of segment b every entry with E > T_b + 2 eps is in the fp64 top
// k_b and every entry with E < T_b - 2 eps is out; the band in between is
// recomputed in fp64 and ranked (entropy desc, index asc) when it straddles
// the cut.

// per segment: the band's size and the count above it (0 when nothing is kept)
__global__ __launch_bounds__(256) void seg_band_count_kernel(const double* E, const int64_t* off,
                                                             const double* thr, double eps2,
                                                             int32_t* nband, int32_t* nabove) {
  __shared__ int red[4];
  const int64_t b = blockIdx.x;
  const int64_t a0 = off[b], a1 = off[b + 1];
  const double T = thr[b];
  int nb = 0, na = 0;
  if (!isnan(T)) {
    for (int64_t t = a0 + threadIdx.x; t < a1; t += 256) {
      const double d = E[t] - T;
      nb += (fabs(d) <= eps2) ? 1 : 0;
      na += (d > eps2) ? 1 : 0;
    }
  }
  int tb = 0, ta = 0;
  block_scan_excl(nb, tb, red);
  block_scan_excl(na, ta, red);
  if (threadIdx.x == 0) {
    nband[b] = tb;
    nabove[b] = ta;
  }
}

// the band positions of each refined segment (boff[b] >= 0), in index order
__global__ __launch_bounds__(256) void seg_band_list_kernel(const double* E, const int64_t* off,
                                                            const double* thr, double eps2,
                                                            const int32_t* boff, int32_t* list) {
  __shared__ int red[4];
  const int64_t b = blockIdx.x;
  const int o = boff[b];
  if (o < 0) return;
  const int64_t a0 = off[b], a1 = off[b + 1];
  const double T = thr[b];
  int seen = 0;
  for (int64_t c0 = a0; c0 < a1; c0 += 256) {
    const int64_t t = c0 + threadIdx.x;
    const bool in = t < a1 && fabs(E[t] - T) <= eps2;
    int n = 0;
    const int r = block_scan_excl(in ? 1 : 0, n, red);
    if (in) list[o + seen + r] = (int32_t)t;
    seen += n;
  }
}

// a refined segment's band: keep the need[b] entries of largest fp64 entropy,
// lower index first among equal values
__global__ __launch_bounds__(256) void seg_band_final_kernel(const int32_t* boff,
                                                             const int32_t* nband,
                                                             const int32_t* need,
                                                             const int32_t* list,
                                                             const double* pent, uint8_t* mask) {
  const int64_t b = blockIdx.x;
  const int o = boff[b];
  if (o < 0) return;
  const int m = nband[b], k = need[b];
  for (int i = threadIdx.x; i < m; i += 256) {
    const double e = pent[o + i];
    const int pos = list[o + i];
    int rank = 0;
    for (int j = 0; j < m; ++j) {
      const double f = pent[o + j];
      rank += (f > e || (f == e && list[o + j] < pos)) ? 1 : 0;
    }
    mask[pos] = rank < k ? 1 : 0;
  }
}

hipError_t launch_seg_band_count(const double* E, const int64_t* off, int64_t B, const double* thr,
                                 double eps2, int32_t* nband, int32_t* nabove, hipStream_t st) {
  if (B <= 0) return hipSuccess;
  hipLaunchKernelGGL(seg_band_count_kernel, dim3((unsigned)B), dim3(256), 0, st, E, off, thr, eps2,
                     nband, nabove);
  return hipGetLastError();
}

hipError_t launch_seg_band_list(const double* E, const int64_t* off, int64_t B, const double* thr,
                                double eps2, const int32_t* boff, int32_t* list, hipStream_t st) {
  if (B <= 0) return hipSuccess;
  hipLaunchKernelGGL(seg_band_list_kernel, dim3((unsigned)B), dim3(256), 0, st, E, off, thr, eps2,
                     boff, list);
  return hipGetLastError();
}

hipError_t launch_seg_band_final(int64_t B, const int32_t* boff, const int32_t* nband,
                                 const int32_t* need, const int32_t* list, const double* pent,
                                 uint8_t* mask, hipStream_t st) {
  if (B <= 0) return hipSuccess;
  hipLaunchKernelGGL(seg_band_final_kernel, dim3((unsigned)B), dim3(256), 0, st, boff, nband, need,
                     list, pent, mask);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void select_above_kernel(const double* x, int64_t S, double tau,
                                                           uint8_t* mask) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t < S) mask[t] = (x[t] >= tau) ? 1 : 0;   // false for NaN
}

hipError_t launch_select_above(const double* x, int64_t S, double tau, uint8_t* mask,
                               hipStream_t st) {
  if (S <= 0) return hipSuccess;
  hipLaunchKernelGGL(select_above_kernel, dim3((unsigned)ceil_div(S, 256)), dim3(256), 0, st, x,
                     S, tau, mask);
  return hipGetLastError();
}

}  // namespace kd
