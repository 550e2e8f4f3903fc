// Teacher top-K cache writer: the steps around the pilot and emit sweeps.
//
// "Making Knowledge Distillation Cheap Enough to Run at Scale" (as written up
// by aibase.it), section "offline top-K logits": the teacher's output is
// computed once and only the logits of each position's K most likely tokens
// are cached; section "operations": the cache holds token ids and logits per
// position, and its validation checks the top-K order. Softmax is monotone, so
// the K most likely tokens are the K largest logits; the cache lists them by
// logit descending, the lower id first among equal logits.
//
// For a chunk of rows:
//  1. pilot sweep (kd_sweep.hip) over vocabulary rows [0, P): the maximum of
//     each group of 16 fp32 logits, gm[g][r];
//  2. teacher_threshold_kernel: per row, tau = the K-th largest group maximum
//     (exact: radix select on order-preserving keys; -inf when the row has
//     fewer than K groups) and a bound B on |fp32 logit - exact logit|; the
//     emission threshold te = tau - 2B, rounded down;
//  3. emit sweep over [0, V): every logit >= te joins the row's candidates;
//  4. teacher_final_kernel: tau2 = the K-th largest candidate (fp32); the
//     candidates with logit >= tau2 - 2B (the band) are recomputed in fp64 from
//     the inputs and ranked by (logit desc, id asc); the first K are written,
//     with their logits rounded from fp64 to fp32 (then to bf16 for a bf16
//     cache). A row whose band exceeds the LDS list goes to
//     teacher_final_big_kernel, which ranks it in global scratch.
//
// Why the result is the exact top K: with |z32 - z| <= B for every entry (in
// either pass), K groups have a maximum >= tau, so K entries have z >= tau - B:
// the K-th largest exact logit y_K >= tau - B and every top-K entry has
// z32 >= y_K - B >= te, i.e. it is a candidate (and so are those K entries). The candidates hold K entries with z32 >= tau2, so y_K >= tau2 - B
// and an entry with z32 < tau2 - 2B has z < y_K: it cannot be in the top K.
// B = 1.01 (H + 16) 2^-23 ||h||_2 max_v ||w_v||_2 + H 2^-90: an fp32 sum of H
// products with at most one rounding per term, each at most 2^-23 relative
// (round to nearest gives 2^-24), |sum of |h_i w_i|| <= ||h|| ||w||
// (Cauchy-Schwarz), and the last term covers products flushed to zero.
#include "kd_common.hpp"
#include "kd_kernels.hpp"

namespace kd {

constexpr int kBandLds = 1024;   // band entries ranked in LDS (a larger band goes to the second kernel)

// order-preserving key of an fp32 value (larger value, larger key)
__device__ inline uint32_t fkey(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ inline float funkey(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

template <typename T>
__device__ inline double elem_f64(const char* row, int h) {
  if constexpr (sizeof(T) == 2) return (double)bf16_to_f32(((const uint16_t*)row)[h]);
  else return (double)((const float*)row)[h];
}

// the part of an fp64 dot product that lane `sub` of `nsub` takes (16-byte
// granules sub, sub + nsub, ...; H is a multiple of the granule). The loads
// of 8 granules are issued before their FMAs, so the loop waits for memory
// once per 8 granules rather than once per granule.
template <typename T>
__device__ inline double dot_f64_part(const char* x, const char* w, int H, int sub, int nsub) {
  constexpr int per = 16 / (int)sizeof(T);
  constexpr int U = 8;
  const int ng = H / per;              // granules in a row
  double acc = 0.0;
  for (int g0 = sub; g0 < ng; g0 += U * nsub) {
    uint4 xr[U], wr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int g = g0 + u * nsub;
      const int gg = g < ng ? g : 0;   // past the row: a valid granule, not used
      xr[u] = *(const uint4*)(x + (int64_t)gg * 16);
      wr[u] = *(const uint4*)(w + (int64_t)gg * 16);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (g0 + u * nsub >= ng) break;
      const uint32_t* xd = (const uint32_t*)&xr[u];
      const uint32_t* wd = (const uint32_t*)&wr[u];
#pragma unroll
      for (int e = 0; e < per; ++e) {
        double xv, wv;
        if constexpr (sizeof(T) == 2) {
          xv = (double)bf16_to_f32((uint16_t)(xd[e >> 1] >> ((e & 1) * 16)));
          wv = (double)bf16_to_f32((uint16_t)(wd[e >> 1] >> ((e & 1) * 16)));
        } else {
          xv = (double)__uint_as_float(xd[e]);
          wv = (double)__uint_as_float(wd[e]);
        }
        acc = fma(xv, wv, acc);
      }
    }
  }
  return acc;
}

// fp64 logits of n listed vocabulary entries of one row: 8 lanes per entry,
// their parts added in a fixed order
template <typename T>
__device__ inline void band_logits(const char* x, const TeacherArgs& a, const int32_t* ids,
                                   double* out, int n) {
  const int tid = threadIdx.x, grp = tid >> 3, sub = tid & 7;
  for (int e0 = 0; e0 < n; e0 += 32) {
    const int e = e0 + grp;
    double d = 0.0;
    if (e < n) d = dot_f64_part<T>(x, a.W + (int64_t)ids[e] * a.ldw, a.H, sub, 8);
    d += __shfl_xor(d, 1);
    d += __shfl_xor(d, 2);
    d += __shfl_xor(d, 4);
    if (e < n && sub == 0) out[e] = d;
  }
}

// ---------------------------------------------------------------------------
// max over v of ||w_v||_2: one wave per row, per-work-group maxima, then one
// work-group over those.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void teacher_wnorm_kernel(const char* W, int64_t ldw, int V, int H,
                                                            double* part) {
  __shared__ double best[4];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  double m = 0.0;
  // one wave per row, 16 bytes per lane per load (H is a multiple of 8, so
  // a row is whole 16-byte granules)
  constexpr int per = 16 / (int)sizeof(T);
  const int ng = H / per;
  for (int v = blockIdx.x * 4 + wv; v < V; v += gridDim.x * 4) {
    const char* row = W + (int64_t)v * ldw;
    double ss = 0.0;
    for (int g = lane; g < ng; g += 64) {
      const uint4 raw = *(const uint4*)(row + (int64_t)g * 16);
      const uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int e = 0; e < per; ++e) {
        double x;
        if constexpr (sizeof(T) == 2) x = (double)bf16_to_f32((uint16_t)(wd[e >> 1] >> ((e & 1) * 16)));
        else x = (double)__uint_as_float(wd[e]);
        ss = fma(x, x, ss);
      }
    }
    for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
    m = fmax(m, ss);
  }
  if (lane == 0) best[wv] = m;
  __syncthreads();
  if (threadIdx.x == 0)
    part[blockIdx.x] = fmax(fmax(best[0], best[1]), fmax(best[2], best[3]));
}

__global__ __launch_bounds__(256) void teacher_wnorm_final_kernel(const double* part, int n,
                                                                  double* wmax) {
  __shared__ double red[256];
  double m = 0.0;
  for (int i = threadIdx.x; i < n; i += 256) m = fmax(m, part[i]);
  red[threadIdx.x] = m;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) red[threadIdx.x] = fmax(red[threadIdx.x], red[threadIdx.x + o]);
    __syncthreads();
  }
  if (threadIdx.x == 0) wmax[0] = sqrt(red[0]);
}

hipError_t launch_teacher_wnorm(int f32, const char* W, int64_t ldw, int V, int H, double* part,
                                double* wmax, hipStream_t st) {
  if (f32)
    hipLaunchKernelGGL(teacher_wnorm_kernel<float>, dim3(kTeacherWnormGroups), dim3(256), 0, st, W, ldw,
                       V, H, part);
  else
    hipLaunchKernelGGL(teacher_wnorm_kernel<__bf16>, dim3(kTeacherWnormGroups), dim3(256), 0, st, W, ldw,
                       V, H, part);
  hipLaunchKernelGGL(teacher_wnorm_final_kernel, dim3(1), dim3(256), 0, st, (const double*)part,
                     kTeacherWnormGroups, wmax);
  return hipGetLastError();
}

// the bound B on |fp32 logit - exact logit| of a row with ||h|| = hn
__device__ inline double logit_bound(int H, double hn, double wmax) {
  return 1.01 * (double)(H + 16) * 0x1p-23 * hn * wmax + (double)H * 0x1p-90;
}

// ---------------------------------------------------------------------------
// Per-row threshold from the pilot's group maxima (a.P groups); 16 rows per
// work-group, thread (row = tid & 15, sub = tid >> 4) reads every 16th group of
// its row, so 16 consecutive threads read 16 consecutive rows of a gm line. The
// K-th largest key is found digit by digit (4 passes of 8 bits, MSB first)
// from per-row LDS histograms.
// ---------------------------------------------------------------------------
constexpr int kThrRows = 16;
// a row's histogram is 257 words apart from the next, so the same bin of the
// 16 rows (the rows of a row block hold similar values, and pass 0 puts most
// of them in one or two bins) falls in 16 different LDS banks
constexpr int kThrHist = 257;
constexpr int kThrVals = 64;   // group maxima per thread: the pilot has at most 16 * 64 groups

template <typename T>
__global__ __launch_bounds__(256) void teacher_threshold_kernel(TeacherArgs a, int32_t* nbig) {
  __shared__ uint32_t hist[kThrRows][kThrHist];
  __shared__ uint32_t prefix[kThrRows];
  __shared__ int krem[kThrRows];
  __shared__ double nrm[16][kThrRows];
  const int tid = threadIdx.x, row = tid & (kThrRows - 1), sub = tid >> 4;
  const int r0 = blockIdx.x * kThrRows, r = r0 + row;
  const bool live = r < a.rows;
  if (blockIdx.x == 0 && tid == 0) *nbig = 0;
  {
    double ss = 0.0;
    if (live) {
      const char* x = a.X + (int64_t)r * a.ldx;
      for (int h = sub; h < a.H; h += 16) {
        const double v = elem_f64<T>(x, h);
        ss = fma(v, v, ss);
      }
    }
    nrm[sub][row] = ss;
  }
  if (tid < kThrRows) {
    prefix[tid] = 0u;
    krem[tid] = a.K;
  }
  // the thread's group maxima as order-preserving keys, read once
  uint32_t key[kThrVals];
#pragma unroll
  for (int u = 0; u < kThrVals; ++u) {
    const int g = sub + 16 * u;
    key[u] = (live && g < a.P) ? fkey(a.zp[(int64_t)g * a.ldp + r]) : 0u;
  }
  const int lane = tid & 63, wv = tid >> 6;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    const uint32_t hmask = pass == 0 ? 0u : (0xFFFFFFFFu << (shift + 8));
    __syncthreads();
    for (int q = tid; q < kThrRows * kThrHist; q += 256) (&hist[0][0])[q] = 0u;
    __syncthreads();
    if (live) {
      const uint32_t pre = prefix[row];
#pragma unroll
      for (int u = 0; u < kThrVals; ++u)
        if (sub + 16 * u < a.P && (key[u] & hmask) == pre)
          atomicAdd(&hist[row][(key[u] >> shift) & 255u], 1u);
    }
    __syncthreads();
    // each row's digit: the largest d whose bins d..255 hold at least krem
    // keys (0 if none do), and krem less the keys above d. Wave wv takes rows
    // 4wv .. 4wv + 3; lane l holds bins 255 - 4l .. 252 - 4l, and a scan over
    // the lanes gives the keys above them, so the one lane whose bins hold
    // the crossing sets the row's digit.
    for (int rr = 0; rr < 4; ++rr) {
      const int q = wv * 4 + rr;
      if (r0 + q >= a.rows) break;   // the same on every lane of the wave
      const int k = krem[q];
      int c[4], sum = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c[j] = (int)hist[q][255 - 4 * lane - j];
        sum += c[j];
      }
      int incl = sum;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o);
        if (lane >= o) incl += y;
      }
      int above = incl - sum;
      if (above < k) {
        int d = -1;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int dd = 255 - 4 * lane - j;
          if (d >= 0) continue;
          if (above + c[j] >= k || dd == 0) d = dd;
          else above += c[j];
        }
        if (d >= 0) {
          prefix[q] |= (uint32_t)d << shift;
          krem[q] = k - above;
        }
      }
    }
  }
  __syncthreads();
  if (tid < kThrRows && r0 + tid < a.rows) {
    // fewer groups than K: no bound from the pilot, every logit is a candidate
    const float tau = a.K <= a.P ? funkey(prefix[tid]) : -INFINITY;
    double ssum = 0.0;
    for (int q = 0; q < 16; ++q) ssum += nrm[q][tid];
    const double b = logit_bound(a.H, sqrt(ssum), a.wmax[0]);
    // rounded down: the margins exceed the rounding of the fp32 result
    const double t = (double)tau - 2.0 * b * (1.0 + 0x1p-20) - fabs((double)tau) * 0x1p-22;
    a.te[r0 + tid] = (float)t;
    a.bnd[r0 + tid] = b;
    a.cnt[r0 + tid] = 0;
  }
}

__device__ inline void write_entry(const TeacherArgs& a, int r, int rank, int id, double z) {
  const int64_t o = (int64_t)r * a.K + rank;
  a.ids_out[o] = id;
  const float f = (float)z;   // round to nearest even
  if (a.out_bf16) ((uint16_t*)a.logits_out)[o] = (uint16_t)f32_to_bf16_bits(f);
  else ((float*)a.logits_out)[o] = f;
}

// ---------------------------------------------------------------------------
// Final ranking: one work-group per row (persistent over rows). A row's
// candidate logits stay in registers (kRegCand per thread) across the radix
// passes and the band test when they fit; otherwise they are read again from
// the list each time.
// ---------------------------------------------------------------------------
constexpr int kRegCand = 16;

__device__ inline void radix_step(const uint32_t* hist, uint32_t* s_prefix, int* s_krem, int shift,
                                  int* s_wsum) {
  // the largest d whose bins d..255 hold at least krem keys (0 if none do),
  // and krem less the keys above d: thread t holds bin 255 - t, and a scan
  // over the threads gives the keys above it, so the one thread whose bin
  // holds the crossing sets the digit. All threads call it.
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int d = 255 - t;
  const int c = (int)hist[d];
  const int k = *s_krem;
  int incl = c;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == 63) s_wsum[wv] = incl;
  __syncthreads();
  for (int q = 0; q < wv; ++q) incl += s_wsum[q];
  const int above = incl - c;
  if (above < k && (incl >= k || d == 0)) {
    *s_prefix |= (uint32_t)d << shift;
    *s_krem = k - above;
  }
}

template <typename T>
__global__ __launch_bounds__(256) void teacher_final_kernel(TeacherArgs a, int32_t* big,
                                                            int32_t* nbig, float* tau2_out) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t s_prefix;
  __shared__ int s_krem, s_m, s_wsum[4];
  __shared__ int lid[kBandLds];
  __shared__ double lz[kBandLds];
  const int tid = threadIdx.x;
  for (int r = blockIdx.x; r < a.rows; r += gridDim.x) {
    const int n = (int)min((int64_t)a.cnt[r], a.cap);
    const int32_t* cid = a.cid + (int64_t)r * a.cap;
    const float* cz = a.cz + (int64_t)r * a.cap;
    const bool in_regs = n <= kRegCand * 256;
    float zc[kRegCand];
#pragma unroll
    for (int u = 0; u < kRegCand; ++u) {
      const int i = tid + 256 * u;
      zc[u] = (in_regs && i < n) ? cz[i] : -INFINITY;
    }
    // tau2: the K-th largest candidate key, digit by digit
    if (tid == 0) {
      s_prefix = 0u;
      s_krem = a.K;
    }
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      const uint32_t hmask = pass == 0 ? 0u : (0xFFFFFFFFu << (shift + 8));
      __syncthreads();
      hist[tid] = 0u;
      __syncthreads();
      const uint32_t pre = s_prefix;
      if (in_regs) {
#pragma unroll
        for (int u = 0; u < kRegCand; ++u) {
          const uint32_t key = fkey(zc[u]);
          if (tid + 256 * u < n && (key & hmask) == pre) atomicAdd(&hist[(key >> shift) & 255u], 1u);
        }
      } else {
        for (int i = tid; i < n; i += 256) {
          const uint32_t key = fkey(cz[i]);
          if ((key & hmask) == pre) atomicAdd(&hist[(key >> shift) & 255u], 1u);
        }
      }
      __syncthreads();
      radix_step(hist, &s_prefix, &s_krem, shift, s_wsum);
    }
    __syncthreads();
    const float tau2 = funkey(s_prefix);
    const double thr = (double)tau2 - 2.0 * a.bnd[r];
    if (tid == 0) s_m = 0;
    __syncthreads();
    // the band; a row with more than kBandLds entries is ranked by the
    // second kernel (its list here is abandoned once full)
    if (in_regs) {
#pragma unroll
      for (int u = 0; u < kRegCand; ++u) {
        const int i = tid + 256 * u;
        if (i < n && (double)zc[u] >= thr) {
          const int pos = atomicAdd(&s_m, 1);
          if (pos < kBandLds) lid[pos] = cid[i];
        }
      }
    } else {
      for (int i = tid; i < n; i += 256) {
        if ((double)cz[i] >= thr) {
          const int pos = atomicAdd(&s_m, 1);
          if (pos < kBandLds) lid[pos] = cid[i];
        }
      }
    }
    __syncthreads();
    const int m = s_m;
    if (m > kBandLds) {
      if (tid == 0) {
        big[atomicAdd(nbig, 1)] = r;
        tau2_out[r] = tau2;
      }
      __syncthreads();
      continue;
    }
    band_logits<T>(a.X + (int64_t)r * a.ldx, a, lid, lz, m);
    __syncthreads();
    // rank by (logit desc, id asc); ids are distinct, so ranks are
    for (int e = tid; e < m; e += 256) {
      const double ze = lz[e];
      const int ie = lid[e];
      int rank = 0;
      for (int f = 0; f < m; ++f) {
        const double zf = lz[f];
        rank += (zf > ze || (zf == ze && lid[f] < ie)) ? 1 : 0;
      }
      if (rank < a.K) write_entry(a, r, rank, ie, ze);
    }
    __syncthreads();
  }
}

// Rows whose band exceeds the LDS list (many logits equal to within the
// bound): the band goes to this work-group's scratch and the K entries are
// taken by K rounds of arg-max over it.
template <typename T>
__global__ __launch_bounds__(256) void teacher_final_big_kernel(TeacherArgs a, const int32_t* big,
                                                                const int32_t* nbig,
                                                                const float* tau2_in) {
  __shared__ int s_m;
  __shared__ double rz[256];
  __shared__ int ri[256], rp[256];
  const int tid = threadIdx.x;
  // this work-group's scratch: capE ids, then capE fp64 logits (capE even, so
  // the fp64 array stays 8-byte aligned)
  const int64_t capE = teacher_scratch_entries(a.cap);
  int32_t* sid = (int32_t*)(a.scratch + (int64_t)blockIdx.x * capE * 12);
  double* sz = (double*)(a.scratch + (int64_t)blockIdx.x * capE * 12 + capE * 4);
  const int nb = *nbig;
  for (int q = blockIdx.x; q < nb; q += gridDim.x) {
    const int r = big[q];
    const int n = (int)min((int64_t)a.cnt[r], a.cap);
    const int32_t* cid = a.cid + (int64_t)r * a.cap;
    const float* cz = a.cz + (int64_t)r * a.cap;
    const double thr = (double)tau2_in[r] - 2.0 * a.bnd[r];
    if (tid == 0) s_m = 0;
    __syncthreads();
    for (int i = tid; i < n; i += 256) {
      if ((double)cz[i] >= thr) sid[atomicAdd(&s_m, 1)] = cid[i];
    }
    __syncthreads();
    const int m = s_m;
    band_logits<T>(a.X + (int64_t)r * a.ldx, a, sid, sz, m);
    __syncthreads();
    for (int k = 0; k < a.K; ++k) {
      double bz = -INFINITY;
      int bi = 0x7FFFFFFF, bp = -1;
      for (int e = tid; e < m; e += 256) {
        const int ie = sid[e];
        if (ie < 0) continue;   // taken
        const double ze = sz[e];
        if (bp < 0 || ze > bz || (ze == bz && ie < bi)) {
          bz = ze;
          bi = ie;
          bp = e;
        }
      }
      rz[tid] = bz;
      ri[tid] = bi;
      rp[tid] = bp;
      __syncthreads();
      for (int o = 128; o > 0; o >>= 1) {
        if (tid < o) {
          const int p2 = rp[tid + o];
          if (p2 >= 0 && (rp[tid] < 0 || rz[tid + o] > rz[tid] ||
                          (rz[tid + o] == rz[tid] && ri[tid + o] < ri[tid]))) {
            rz[tid] = rz[tid + o];
            ri[tid] = ri[tid + o];
            rp[tid] = p2;
          }
        }
        __syncthreads();
      }
      if (tid == 0) {
        write_entry(a, r, k, ri[0], rz[0]);
        sid[rp[0]] = -1;
      }
      __syncthreads();
    }
  }
}

// Gather of the emit pass's candidates. The pass wrote each row's candidates
// into one sub-list per writer: vocabulary range b (tiles [b nvt / ns,
// (b + 1) nvt / ns)) and writer w (wave and lane half) start at tile_begin *
// 256 + w * (tiles in the range) * 64 of the row's list. One work-group per
// row forms the running total of the sub-list lengths, then moves the
// candidates to the front of the list, 256 at a time: candidate i (in
// sub-list order) goes to position i from a position at or after i, and each
// round's reads have all returned before any of its writes (a wait for the
// loads, then a barrier), so no candidate is overwritten before it is read.
constexpr int kGatherMaxSub = 4096;

__global__ __launch_bounds__(256) void teacher_gather_kernel(int32_t* cid, float* cz, int64_t cap,
                                                             const int32_t* scnt, int64_t scnt_ld,
                                                             int ns, int nvt, int rows,
                                                             int32_t* cnt) {
  __shared__ int pre[kGatherMaxSub + 1];
  const int tid = threadIdx.x;
  const int t = blockIdx.x;
  const int nsub = ns * 4;
  const int32_t* sc = scnt + (int64_t)t * scnt_ld;
  if (tid < 64) {
    // exclusive running total of the lengths, 64 sub-lists at a time
    int run = 0;
    for (int c0 = 0; c0 < nsub; c0 += 64) {
      const int v = (c0 + tid < nsub) ? sc[c0 + tid] : 0;
      int x = v;
      for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(x, d, 64);
        if (tid >= d) x += y;
      }
      if (c0 + tid < nsub) pre[c0 + tid] = run + x - v;
      run += __shfl(x, 63, 64);
    }
    if (tid == 0) pre[nsub] = run;
  }
  __syncthreads();
  const int total = pre[nsub];
  int32_t* ci = cid + (int64_t)t * cap;
  float* cv = cz + (int64_t)t * cap;
  for (int r0 = 0; r0 < total; r0 += 256) {
    const int i = r0 + tid;
    const bool has = i < total;
    int32_t id = 0;
    float z = 0.0f;
    if (has) {
      // the sub-list holding candidate i: the last s with pre[s] <= i
      int lo = 0, hi = nsub - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (pre[mid] <= i) lo = mid;
        else hi = mid - 1;
      }
      const int b = lo >> 2, w = lo & 3;
      const int vb = (int)((int64_t)b * nvt / ns), ve = (int)((int64_t)(b + 1) * nvt / ns);
      const int64_t src = (int64_t)vb * 256 + (int64_t)w * (ve - vb) * 64 + (i - pre[lo]);
      id = ci[src];
      z = cv[src];
    }
    // the loads must have returned before any thread stores: a work-group
    // barrier alone does not wait for them
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (has) {
      ci[i] = id;
      cv[i] = z;
    }
  }
  if (tid == 0) cnt[t] = total;
}

hipError_t launch_teacher_gather(int32_t* cid, float* cz, int64_t cap, const int32_t* scnt,
                                 int64_t scnt_ld, int ns, int nvt, int rows, int32_t* cnt,
                                 hipStream_t st) {
  if (ns * 4 > kGatherMaxSub) return hipErrorInvalidValue;
  if (rows > 0)
    hipLaunchKernelGGL(teacher_gather_kernel, dim3((unsigned)rows), dim3(256), 0, st, cid, cz, cap,
                       scnt, scnt_ld, ns, nvt, rows, cnt);
  return hipGetLastError();
}

hipError_t launch_teacher_threshold(int f32, const TeacherArgs& a, int32_t* nbig, hipStream_t st) {
  const int grid = (int)ceil_div(a.rows, kThrRows);
  if (grid <= 0) return hipSuccess;
  if (f32)
    hipLaunchKernelGGL(teacher_threshold_kernel<float>, dim3(grid), dim3(256), 0, st, a, nbig);
  else
    hipLaunchKernelGGL(teacher_threshold_kernel<__bf16>, dim3(grid), dim3(256), 0, st, a, nbig);
  return hipGetLastError();
}

hipError_t launch_teacher_final(int f32, const TeacherArgs& a, int32_t* big, int32_t* nbig,
                                float* tau2, int grid, int grid_big, hipStream_t st) {
  if (a.rows <= 0) return hipSuccess;
  if (f32) {
    hipLaunchKernelGGL(teacher_final_kernel<float>, dim3(grid), dim3(256), 0, st, a, big, nbig,
                       tau2);
    hipLaunchKernelGGL(teacher_final_big_kernel<float>, dim3(grid_big), dim3(256), 0, st, a,
                       (const int32_t*)big, (const int32_t*)nbig, (const float*)tau2);
  } else {
    hipLaunchKernelGGL(teacher_final_kernel<__bf16>, dim3(grid), dim3(256), 0, st, a, big, nbig,
                       tau2);
    hipLaunchKernelGGL(teacher_final_big_kernel<__bf16>, dim3(grid_big), dim3(256), 0, st, a,
                       (const int32_t*)big, (const int32_t*)nbig, (const float*)tau2);
  }
  return hipGetLastError();
}

}  // namespace kd
