// Shared device/host helpers of the top-K KL library for gfx950 (CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kd {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Tile geometry of every projection kernel: a work-group of 256 threads
// (4 wave64) computes a 256 x 256 output tile as 2 x 2 waves of 128 x 128,
// each wave 4 x 4 MFMA 32x32 blocks. The staging pipeline is described in
// kd_gemm_core.hpp.
// ---------------------------------------------------------------------------
constexpr int kThreads = 256;
constexpr int kTile = 256;          // rows of each operand tile (M and N)

template <typename T> struct Elem;
template <> struct Elem<__bf16> { static constexpr int size = 2; };
template <> struct Elem<float> { static constexpr int size = 4; };

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
__host__ __device__ inline int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

// Map a hardware work-group id to a logical one so that each XCD (work-groups
// are dealt to the 8 XCDs round-robin) receives a contiguous range of logical
// ids: work-groups that share operand panels then share one L2.
__device__ inline int xcd_remap(int hid, int total) {
  const int nx = 8;
  int x = hid % nx, local = hid / nx;
  int per = total / nx, rem = total % nx;
  return (x < rem) ? x * (per + 1) + local : rem * (per + 1) + (x - rem) * per + local;
}

// Vocabulary-sweep split: a work-group owns one 256-row token tile and a
// contiguous range of 256-row vocabulary tiles. Choose the number of ranges so
// that (rounds of work-groups over the CUs) x (tiles per work-group) is least,
// the fewest ranges (at least 6) among equal costs. Fewer, longer ranges put
// more token tiles and fewer W ranges on an XCD at once: at the 32K-context
// shapes the forward took 33.3 ms with 10 ranges, 32.3 with 8 and 30.9 with 6
// or 4 (A/B on one MI355X), and the entropy sweep at the entropy-selective
// shapes 18.3 ms with 18 ranges and 17.7 with 6.
__host__ __device__ inline int sweep_splits(int ntok_tiles, int nvt, int ncu) {
  if (ntok_tiles <= 0) return 1;
  int lo = nvt < 6 ? nvt : 6;
  int hi = nvt < 64 ? nvt : 64;
  int best = lo;
  int64_t best_cost = -1;
  for (int ns = lo; ns <= hi; ++ns) {
    int64_t wgs = (int64_t)ntok_tiles * ns;
    int64_t rounds = ceil_div(wgs, ncu);
    int64_t cost = rounds * ceil_div(nvt, ns);
    if (best_cost < 0 || cost < best_cost) { best_cost = cost; best = ns; }
  }
  return best;
}

// Split-K factor of the dHidden product (K = vocabulary): enough work-groups
// to cover the CUs a few times without tiny K ranges.
__host__ __device__ inline int splitk_factor(int tiles, int nksteps, int ncu) {
  if (tiles <= 0) return 1;
  int best = 1;
  int64_t best_cost = -1;
  for (int s = 1; s <= 64; ++s) {
    int64_t per = ceil_div(nksteps, s);
    if (per < 16 && s > 1) break;
    int64_t rounds = ceil_div((int64_t)tiles * s, ncu);
    int64_t cost = rounds * per + 4 * s;   // 4 k-steps ~ cost of reducing one more partial
    if (best_cost < 0 || cost < best_cost) { best_cost = cost; best = s; }
  }
  return best;
}

__device__ inline float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ inline float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ inline double wave_sum_d(double v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ inline float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// fp32 -> bf16 bits, round to nearest even (inputs here are finite).
__device__ inline uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ inline uint64_t ballot(bool p) { return __ballot(p); }

// Merge two (max, sum) pairs of a base-2 log-sum-exp: sum_i s_i 2^(m_i - m).
__device__ inline void lse2_merge(float& m, float& s, float m2, float s2) {
  if (m2 == -INFINITY) return;
  if (m == -INFINITY) { m = m2; s = s2; return; }
  float mn = fmaxf(m, m2);
  s = s * exp2f(m - mn) + s2 * exp2f(m2 - mn);
  m = mn;
}

}  // namespace kd
