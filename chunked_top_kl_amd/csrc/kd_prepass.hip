// Teacher-side prepass, row compaction and cache validation.
//
// Prepass, one wave per position ("offline top-K logits": K cached ids and
// logits per position, softened by the stored temperature):
//   p_k   = softmax over the row's usable entries of l_k / T
//   negH  = sum over distinct ids of P log P, P = sum of p_k sharing the id
//           (0 log 0 = 0)
//   (id, p, k) sorted by id ascending, ties by k, so that the projection
//   epilogue can walk each row's ids in vocabulary order.
// An entry is usable when its id lies in [0, V) and its logit is finite;
// -inf entries get p = 0; an id outside [0, V) is never dereferenced later
// (it is stored as 0x7FFFFFFF, past every vocabulary tile). A row takes part
// ("present") when it has a usable entry and no NaN / +inf logit.
// Targets given as probabilities (sampled sparse targets, "Rethinking
// Selective Knowledge Distillation" SE-KD3X class axis): p_k = v_k / sum of
// the row's usable v (id in [0, V), v > 0), the temperature left to the
// student side; the row takes part when no value is negative or non-finite
// and the usable values have a positive sum.
#include "kd_common.hpp"
#include "kd_kernels.hpp"

namespace kd {

__device__ inline float load_logit(const void* tl, int tl_f32, int64_t i) {
  return tl_f32 ? ((const float*)tl)[i] : bf16_to_f32(((const uint16_t*)tl)[i]);
}

__global__ void prepass_kernel(const int32_t* ids, const void* tl, int tl_f32, int probs, int64_t S,
                               int K, int V, float invT, int n2, int32_t* ids_s, float* p_s,
                               int32_t* korig_s, float* negH_out, uint8_t* present,
                               float* z_topk) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int rpb = blockDim.x >> 6;
  unsigned long long* key = (unsigned long long*)smem + (int64_t)wv * n2;
  float* pv = (float*)(smem + (int64_t)rpb * n2 * 8) + (int64_t)wv * n2;
  const int64_t t = (int64_t)blockIdx.x * rpb + wv;
  const bool live = t < S;
  const int64_t base = (live ? t : 0) * K;

  // 1. row max over usable entries (logits), flags
  float mx = -INFINITY;
  int bad = 0;
  for (int k = lane; k < K; k += 64) {
    const int id = live ? ids[base + k] : 0;
    const float l = live ? load_logit(tl, tl_f32, base + k) : -INFINITY;
    if (probs) {
      if (live && !(isfinite(l) && l >= 0.0f)) bad = 1;
    } else {
      if (isnan(l) || l == INFINITY) bad = 1;
      if (id >= 0 && id < V && isfinite(l)) mx = fmaxf(mx, l * invT);
    }
  }
  mx = wave_max(mx);
  bad = (int)wave_sum((float)bad) > 0;
  // 2. normaliser: sum of exp(l/T - max) (logits) or of the usable values
  float z = 0.0f;
  if (probs || mx != -INFINITY) {
    for (int k = lane; k < K; k += 64) {
      const int id = live ? ids[base + k] : 0;
      const float l = live ? load_logit(tl, tl_f32, base + k) : -INFINITY;
      if (id >= 0 && id < V && isfinite(l)) {
        if (probs) z += l > 0.0f ? l : 0.0f;
        else z += __expf(l * invT - mx);
      }
    }
  }
  z = wave_sum(z);
  const float logz = __logf(z);
  const bool has_mass = probs ? (z > 0.0f) : (mx != -INFINITY);
  // 3. probabilities, entropy term, sort keys
  float nh = 0.0f;
  for (int k = lane; k < n2; k += 64) {
    unsigned long long kk = ~0ull;
    float p = 0.0f;
    if (k < K && live) {
      const int id = ids[base + k];
      const float l = load_logit(tl, tl_f32, base + k);
      const bool inr = id >= 0 && id < V;
      if (inr && isfinite(l) && has_mass) {
        if (probs) p = l > 0.0f ? l / z : 0.0f;
        else p = __expf((l * invT - mx) - logz);
      }
      const uint32_t kid = inr ? (uint32_t)id : 0x7FFFFFFFu;
      kk = ((unsigned long long)kid << 32) | (uint32_t)k;
      if (z_topk) z_topk[base + k] = __int_as_float(0x7FC00000);  // NaN until gathered
    }
    key[k] = kk;
    pv[k] = p;
  }
  __syncthreads();
  // 4. bitonic sort of (key, p) ascending by key (each wave its own row)
  for (int kk = 2; kk <= n2; kk <<= 1) {
    for (int j = kk >> 1; j > 0; j >>= 1) {
      for (int i = lane; i < n2; i += 64) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const bool up = (i & kk) == 0;
          const unsigned long long a = key[i], b = key[ixj];
          if ((a > b) == up) {
            key[i] = b;
            key[ixj] = a;
            const float tp = pv[i];
            pv[i] = pv[ixj];
            pv[ixj] = tp;
          }
        }
      }
      __syncthreads();
    }
  }
  // teacher entropy term over merged probabilities: entries sharing an id form
  // one run after the sort and their probabilities add
  for (int k = lane; k < K; k += 64) {
    const uint32_t id = (uint32_t)(key[k] >> 32);
    if (id == 0x7FFFFFFFu || (k > 0 && (uint32_t)(key[k - 1] >> 32) == id)) continue;
    float P = 0.0f;
    for (int q = k; q < K && (uint32_t)(key[q] >> 32) == id; ++q) P += pv[q];
    if (P > 0.0f) nh += P * __logf(P);
  }
  nh = wave_sum(nh);
  if (!live) return;
  for (int k = lane; k < K; k += 64) {
    const unsigned long long kk = key[k];
    ids_s[base + k] = (int32_t)(kk >> 32);
    p_s[base + k] = pv[k];
    korig_s[base + k] = (int32_t)(kk & 0xFFFFFFFFu);
  }
  if (lane == 0) {
    negH_out[t] = nh;
    present[t] = (!bad && has_mass) ? 1 : 0;
  }
}

// The same steps for rows of at most 128 entries, held in registers: entries
// lane and lane + 64 of the row in each lane, sorted by a bitonic network whose
// exchanges are cross-lane shuffles (and, at distance 64, a swap inside the
// lane), so that the four rows of a work-group never wait for each other and
// nothing goes through LDS. The probability of a run of equal ids is a
// segmented running sum over the sorted entries, read at the run's last entry.
__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, m, 64);
  const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), m, 64);
  return ((uint64_t)hi << 32) | lo;
}

__global__ __launch_bounds__(256) void prepass_reg_kernel(const int32_t* ids, const void* tl,
                                                          int tl_f32, int probs, int64_t S, int K,
                                                          int V, float invT, int32_t* ids_s,
                                                          float* p_s, int32_t* korig_s,
                                                          float* negH_out, uint8_t* present,
                                                          float* z_topk) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= S) return;   // wave-uniform; the kernel has no work-group barrier
  const int64_t base = t * K;
  int id[2];
  float l[2];
  bool has[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int k = lane + 64 * s;
    has[s] = k < K;
    id[s] = has[s] ? ids[base + k] : 0;
    l[s] = has[s] ? load_logit(tl, tl_f32, base + k) : -INFINITY;
  }
  // 1. row max over usable entries (logits), flags
  float mx = -INFINITY;
  int bad = 0;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    if (!has[s]) continue;
    if (probs) {
      if (!(isfinite(l[s]) && l[s] >= 0.0f)) bad = 1;
    } else {
      if (isnan(l[s]) || l[s] == INFINITY) bad = 1;
      if (id[s] >= 0 && id[s] < V && isfinite(l[s])) mx = fmaxf(mx, l[s] * invT);
    }
  }
  mx = wave_max(mx);
  bad = (int)wave_sum((float)bad) > 0;
  // 2. normaliser
  float z = 0.0f;
  if (probs || mx != -INFINITY) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (has[s] && id[s] >= 0 && id[s] < V && isfinite(l[s])) {
        if (probs) z += l[s] > 0.0f ? l[s] : 0.0f;
        else z += __expf(l[s] * invT - mx);
      }
    }
  }
  z = wave_sum(z);
  const float logz = __logf(z);
  const bool has_mass = probs ? (z > 0.0f) : (mx != -INFINITY);
  // 3. probabilities and sort keys (id, k); entries past K sort last
  uint64_t key[2];
  float p[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int k = lane + 64 * s;
    key[s] = ~0ull;
    p[s] = 0.0f;
    if (has[s]) {
      const bool inr = id[s] >= 0 && id[s] < V;
      if (inr && isfinite(l[s]) && has_mass) {
        if (probs) p[s] = l[s] > 0.0f ? l[s] / z : 0.0f;
        else p[s] = __expf((l[s] * invT - mx) - logz);
      }
      const uint32_t kid = inr ? (uint32_t)id[s] : 0x7FFFFFFFu;
      key[s] = ((uint64_t)kid << 32) | (uint32_t)k;
      if (z_topk) z_topk[base + k] = __int_as_float(0x7FC00000);  // NaN until gathered
    }
  }
  // 4. bitonic sort of entry i = lane + 64 s, ascending by key
  for (int kk = 2; kk <= 128; kk <<= 1) {
    for (int j = kk >> 1; j > 0; j >>= 1) {
      if (j == 64) {   // only for kk = 128: ascending across the two slots
        if (key[1] < key[0]) {
          const uint64_t tk = key[0];
          key[0] = key[1];
          key[1] = tk;
          const float tp = p[0];
          p[0] = p[1];
          p[1] = tp;
        }
        continue;
      }
      const bool lower = (lane & j) == 0;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int i = lane + 64 * s;
        const bool up = (i & kk) == 0;
        const uint64_t ok = shfl_xor_u64(key[s], j);
        const float op = __shfl_xor(p[s], j, 64);
        const bool take = (lower == up) ? (ok < key[s]) : (ok > key[s]);
        if (take) {
          key[s] = ok;
          p[s] = op;
        }
      }
    }
  }
  // 5. runs of equal ids: segmented inclusive sum of p within each slot, the
  // second slot continuing the first slot's last run
  uint32_t idv[2];
  idv[0] = (uint32_t)(key[0] >> 32);
  idv[1] = (uint32_t)(key[1] >> 32);
  const uint32_t last0 = (uint32_t)__shfl((int)idv[0], 63, 64);
  const uint32_t first1 = (uint32_t)__shfl((int)idv[1], 0, 64);
  float v[2];
  int f[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const uint32_t up1 = (uint32_t)__shfl_up((int)idv[s], 1, 64);
    const uint32_t prev = lane > 0 ? up1 : (s == 0 ? ~idv[s] : last0);
    f[s] = prev != idv[s] ? 1 : 0;
    v[s] = p[s];
    for (int d = 1; d < 64; d <<= 1) {
      const float vu = __shfl_up(v[s], d, 64);
      const int fu = __shfl_up(f[s], d, 64);
      if (lane >= d) {
        if (!f[s]) v[s] = vu + v[s];
        f[s] |= fu;
      }
    }
  }
  const float carry = __shfl(v[0], 63, 64);
  if (!f[1]) v[1] = carry + v[1];
  float nh = 0.0f;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const uint32_t dn = (uint32_t)__shfl_down((int)idv[s], 1, 64);
    const bool tail = lane < 63 ? dn != idv[s] : (s == 0 ? first1 != idv[0] : true);
    const bool valid = idv[s] < 0x7FFFFFFFu;
    if (tail && valid && v[s] > 0.0f) nh += v[s] * __logf(v[s]);
  }
  nh = wave_sum(nh);
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int k = lane + 64 * s;
    if (k < K) {
      ids_s[base + k] = (int32_t)idv[s];
      p_s[base + k] = p[s];
      korig_s[base + k] = (int32_t)(key[s] & 0xFFFFFFFFu);
    }
  }
  if (lane == 0) {
    negH_out[t] = nh;
    present[t] = (!bad && has_mass) ? 1 : 0;
  }
}

hipError_t launch_prepass(const int32_t* ids, const void* tl, int tl_f32, int probs, int64_t S,
                          int K, int V, float T, int32_t* ids_s, float* p_s, int32_t* korig_s,
                          float* negH, uint8_t* present, float* z_topk, hipStream_t st) {
  if (S <= 0) return hipSuccess;
  if (K <= 128) {
    hipLaunchKernelGGL(prepass_reg_kernel, dim3((unsigned)ceil_div(S, 4)), dim3(256), 0, st, ids, tl,
                       tl_f32, probs, S, K, V, 1.0f / T, ids_s, p_s, korig_s, negH, present, z_topk);
    return hipGetLastError();
  }
  int n2 = 1;
  while (n2 < K) n2 <<= 1;
  const int rpb = n2 <= 1024 ? 4 : 1;
  const size_t lds = (size_t)rpb * n2 * 12;
  const int64_t grid = ceil_div(S, rpb);
  hipLaunchKernelGGL(prepass_kernel, dim3((unsigned)grid), dim3(64 * rpb), lds, st, ids, tl, tl_f32,
                     probs, S, K, V, 1.0f / T, n2, ids_s, p_s, korig_s, negH, present, z_topk);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Compaction: valid_t = present_t && (mask_t != 0 or no mask). idx[r] lists
// the valid positions in ascending order, pos[t] = r or -1, count = N.
// One work-group of 1024 threads; each thread owns a contiguous segment.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void compact_kernel(const uint8_t* present, const uint8_t* mask,
                                                       int64_t S, int32_t* idx, int32_t* pos,
                                                       int32_t* count) {
  __shared__ int32_t sc[1024];
  const int tid = threadIdx.x;
  const int64_t seg = ceil_div(S, 1024);
  const int64_t t0 = tid * seg;
  const int64_t t1 = (t0 + seg < S) ? t0 + seg : S;
  int c = 0;
  for (int64_t t = t0; t < t1; ++t) c += (present[t] && (!mask || mask[t])) ? 1 : 0;
  sc[tid] = c;
  __syncthreads();
  // Hillis-Steele inclusive scan
  for (int o = 1; o < 1024; o <<= 1) {
    const int v = tid >= o ? sc[tid - o] : 0;
    __syncthreads();
    sc[tid] += v;
    __syncthreads();
  }
  int off = sc[tid] - c;
  for (int64_t t = t0; t < t1; ++t) {
    if (present[t] && (!mask || mask[t])) {
      idx[off] = (int32_t)t;
      pos[t] = off++;
    } else {
      pos[t] = -1;
    }
  }
  if (tid == 1023) count[0] = sc[1023];
}

hipError_t launch_compact(const uint8_t* present, const uint8_t* mask, int64_t S, int32_t* idx,
                          int32_t* pos, int32_t* count, hipStream_t st) {
  hipLaunchKernelGGL(compact_kernel, dim3(1), dim3(1024), 0, st, present, mask, S, idx, pos, count);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Validation counters: [0] ids outside [0, V), [1] rows whose logits are all
// -inf (probabilities: no positive value), [2] NaN / +inf logits
// (probabilities: negative or non-finite values). Integer atomics: the totals
// do not depend on the order of the additions.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void validate_kernel(const int32_t* ids, const void* tl,
                                                       int tl_f32, int probs, int64_t S, int K,
                                                       int V, unsigned long long* counters) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= S) return;
  int nbad = 0, nlog = 0, nfin = 0;
  for (int k = lane; k < K; k += 64) {
    const int id = ids[t * K + k];
    const float l = load_logit(tl, tl_f32, t * K + k);
    nbad += (id < 0 || id >= V) ? 1 : 0;
    if (probs) {
      nlog += (isfinite(l) && l >= 0.0f) ? 0 : 1;
      nfin += (isfinite(l) && l > 0.0f) ? 1 : 0;
    } else {
      nlog += (isnan(l) || l == INFINITY) ? 1 : 0;
      nfin += (l != -INFINITY) ? 1 : 0;
    }
  }
  for (int o = 32; o > 0; o >>= 1) {
    nbad += __shfl_xor(nbad, o, 64);
    nlog += __shfl_xor(nlog, o, 64);
    nfin += __shfl_xor(nfin, o, 64);
  }
  if (lane == 0) {
    if (nbad) atomicAdd(&counters[0], (unsigned long long)nbad);
    if (nfin == 0) atomicAdd(&counters[1], 1ull);
    if (nlog) atomicAdd(&counters[2], (unsigned long long)nlog);
  }
}

__global__ void zero_u64_kernel(unsigned long long* p, int n) {
  if ((int)threadIdx.x < n) p[threadIdx.x] = 0ull;
}

hipError_t launch_validate(const int32_t* ids, const void* tl, int tl_f32, int probs, int64_t S,
                           int K, int V, unsigned long long* counters, hipStream_t st) {
  hipLaunchKernelGGL(zero_u64_kernel, dim3(1), dim3(64), 0, st, counters, 3);
  if (S > 0)
    hipLaunchKernelGGL(validate_kernel, dim3((unsigned)ceil_div(S, 4)), dim3(256), 0, st, ids, tl,
                       tl_f32, probs, S, K, V, counters);
  return hipGetLastError();
}

// The cache's top-K order ("operations" lists the top-K sorting among the
// cache checks), one wave per row: [0] rows with some value smaller than the
// next (NaN compares with nothing), [1] rows holding an id more than once.
__global__ __launch_bounds__(64) void validate_order_kernel(const int32_t* ids, const void* tl,
                                                           int tl_f32, int64_t S, int K,
                                                           unsigned long long* counters) {
  extern __shared__ int32_t rid[];
  const int lane = threadIdx.x;
  const int64_t t = blockIdx.x;
  if (t >= S) return;
  int uns = 0, dup = 0;
  for (int k = lane; k < K; k += 64) {
    rid[k] = ids[t * K + k];
    if (k + 1 < K) uns |= load_logit(tl, tl_f32, t * K + k) < load_logit(tl, tl_f32, t * K + k + 1);
  }
  __syncthreads();
  for (int k = lane; k < K; k += 64) {
    const int id = rid[k];
    for (int j = k + 1; j < K; ++j) dup |= (rid[j] == id) ? 1 : 0;
  }
  uns = __any(uns);
  dup = __any(dup);
  if (lane == 0) {
    if (uns) atomicAdd(&counters[0], 1ull);
    if (dup) atomicAdd(&counters[1], 1ull);
  }
}

hipError_t launch_validate_order(const int32_t* ids, const void* tl, int tl_f32, int64_t S, int K,
                                 unsigned long long* counters, hipStream_t st) {
  hipLaunchKernelGGL(zero_u64_kernel, dim3(1), dim3(64), 0, st, counters, 2);
  if (S > 0)
    hipLaunchKernelGGL(validate_order_kernel, dim3((unsigned)S), dim3(64), (size_t)K * 4, st, ids,
                       tl, tl_f32, S, K, counters);
  return hipGetLastError();
}

__global__ void fill_u8_kernel(uint8_t* p, uint8_t v, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    p[i] = v;
}

hipError_t launch_fill_u8(uint8_t* p, uint8_t v, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  int64_t grid = ceil_div(n, 256);
  if (grid > 4096) grid = 4096;
  hipLaunchKernelGGL(fill_u8_kernel, dim3((unsigned)grid), dim3(256), 0, st, p, v, n);
  return hipGetLastError();
}

}  // namespace kd
