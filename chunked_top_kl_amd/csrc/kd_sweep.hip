// Vocabulary-sweep projection kernels: the fused lm_head GEMM with
//  - forward: online base-2 log-sum-exp of z/T and the gather of z at the
//    teacher ids ("what chunked KL loss does": project, fold into the loss,
//    discard - nothing of [rows, V] is stored);
//  - backward: the logit gradient (softmax(z/T) - p)/T * g/N as a bf16 tile,
//    with p scattered at the teacher ids ("backward recomputes the chunk");
//  - entropy: online (max, sum, sum e*y) of softmax(z) for H(q_t)
//    ("Rethinking Selective Knowledge Distillation", chunked entropy);
//  - teacher cache writer ("offline top-K logits": the teacher's logits are
//    computed once and only each position's K largest kept): a pilot pass
//    that stores the maxima of groups of 16 logits of the first vocabulary
//    rows, and an emit pass that appends every logit at or above a per-row
//    threshold to the row's candidate list, in one sub-list per writer
//    (kd_teacher.hip gathers them and picks the K);
//  - logits (the dense and forward-chunked comparator forms of "what
//    chunked KL loss does", which keep the student logits): z itself stored
//    as a bf16 tile [rows][Vp] through the gradient tile's staged store;
//  - sampled targets (RS-KD: ids drawn from the teacher's softmax at T by
//    inverse transform in vocabulary order): a mass pass that stores the
//    probability mass of every 128-entry vocabulary unit of each row (in the
//    unit's own scale, with that scale), and a draw pass that, for the draws
//    assigned to a unit (kd_sample.hip), finds the entry where the running
//    mass passes the draw's residual.
//
// Orientation: MFMA rows (M) are vocabulary entries (A = W tile), MFMA columns
// (N) are tokens (B = hidden rows). Each lane therefore owns whole token
// columns, so the per-token running state stays in registers for the entire
// sweep and needs only one cross-lane merge at the end.
#include "kd_gemm_core.hpp"
#include "kd_kernels.hpp"

#include <map>
#include <type_traits>
#include <mutex>
#include <tuple>

namespace kd {

// operand with the third stage buffer (longer load lead): A = W (true) or the
// token rows
#ifndef KD_SWEEP_A_EARLY
#define KD_SWEEP_A_EARLY 0
#endif
constexpr bool kSweepAEarly = KD_SWEEP_A_EARLY;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// vocabulary index of accumulator element (i, r) for this lane, relative to vw0
__device__ inline int acc_row(int i, int r, int half) { return i * 32 + 8 * (r >> 2) + 4 * half + (r & 3); }

__device__ inline int lower_bound_ids(const int32_t* p, int K, int key) {
  int lo = 0, hi = K;
  while (lo < hi) {
    int mid = (lo + hi) >> 1;
    if (p[mid] < key) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

// Merge two partial entropy triples (max m in log2 units, S = sum 2^(y-m),
// U = sum 2^(y-m) (y-m)) into the first.
__device__ inline void ent_merge(float& m, double& S, double& U, float m2, double S2, double U2) {
  if (m2 == -INFINITY) return;
  if (m == -INFINITY) {
    m = m2;
    S = S2;
    U = U2;
    return;
  }
  const float mn = fmaxf(m, m2);
  const double d1 = (double)(m - mn), d2 = (double)(m2 - mn);
  const double f1 = exp2(d1), f2 = exp2(d2);
  U = (U + S * d1) * f1 + (U2 + S2 * d2) * f2;
  S = S * f1 + S2 * f2;
  m = mn;
}

// Teacher cursor of one token column: position `cur` in the row's id-sorted
// table (row offset `base` = original row * K) and the id found there.
struct Cursor {
  int64_t base;
  int cur, nid;
};

__device__ inline void cursor_adv(Cursor& c, const int32_t* ids_s, int K) {
  ++c.cur;
  c.nid = c.cur < K ? ids_s[c.base + c.cur] : 0x7FFFFFFF;
}

// Register of this lane's half tile that holds local row `local` of the
// half tile [lo, lo+128), or -1 when the row belongs to the other lane half.
// The two lanes of a token column (lane halves) see the same ids; a local row
// r belongs to the lane whose half is bit 2 of r, at register
// (r >> 5) * 16 + ((r >> 3) & 3) * 4 + (r & 3).
__device__ __forceinline__ int hit_reg(bool h, int local, int half) {
  const bool mine = h && (((local >> 2) & 1) == half);
  return mine ? (local >> 5) * 16 + ((local >> 3) & 3) * 4 + (local & 3) : -1;
}

// Walk the teacher ids of one token column that fall in [lo, lo+128) (this
// wave's half tile) one id at a time. Each round calls on(tgt, e) on every
// lane, with tgt the register of the lane's own hit or -1, and e the hit's
// index in the sorted table; then every lane with a hit advances.
template <class F>
__device__ __forceinline__ void walk_hits(Cursor& c, const int32_t* ids_s, int K, int lo, int half,
                                          F&& on) {
  while (c.nid < lo) cursor_adv(c, ids_s, K);
  const int hi = lo + 128;
  while (true) {
    const bool h = c.nid < hi;
    if (ballot(h) == 0) break;
    on(hit_reg(h, c.nid - lo, half), c.base + c.cur);
    if (h) cursor_adv(c, ids_s, K);
  }
}

// The same walk over a window of the next kWin ids of the column, loaded
// before the tile's log-sum-exp so that their latency is hidden: ids below lo
// (the other wave's half of the previous tile) are passed over, ids in
// [lo, hi) are hits, and the cursor moves past every id below hi. Only when a
// lane's whole window lies below hi does the one-id-at-a-time walk continue.
constexpr int kWin = 4;

__device__ __forceinline__ void window_load(int64_t base, int cur, const int32_t* ids_s, int K,
                                            int (&n)[kWin]) {
#pragma unroll
  for (int q = 0; q < kWin; ++q) {
    const int p = cur + q;
    const int v = ids_s[base + (p < K ? p : K - 1)];
    n[q] = p < K ? v : 0x7FFFFFFF;
  }
}

template <class F>
__device__ __forceinline__ void walk_window(int64_t base, int& cur, const int (&n)[kWin],
                                            const int32_t* ids_s, int K, int lo, int half,
                                            F&& on) {
  const int hi = lo + 128;
  int used = 0;
#pragma unroll
  for (int q = 0; q < kWin; ++q) {
    const bool h = n[q] >= lo && n[q] < hi;
    used += n[q] < hi ? 1 : 0;
    if (ballot(h) == 0) continue;
    on(hit_reg(h, n[q] - lo, half), base + cur + q);
  }
  cur += used;
  const bool more = used == kWin;
  if (ballot(more) != 0) {
    Cursor c{base, cur, 0x7FFFFFFF};
    if (more && cur < K) c.nid = ids_s[base + cur];
    walk_hits(c, ids_s, K, lo, half, on);
    cur = c.cur;
  }
}

// Column reductions of the forward and entropy epilogues. TAIL excludes the
// entries at or past the vocabulary (W rows there read as zero, so those
// logits are 0). The caller branches on its half tile being the last one, so
// that the per-entry test runs on that tile only: folded into selects it
// cost every tile about five instructions per entry. The row limit passes
// through an empty volatile asm so that the tests stay inside the branch
// (otherwise they are shared between reductions and computed, and spilled,
// ahead of it on every tile).
template <bool TAIL>
__device__ __forceinline__ int col_lim(int vw0, int half, int V) {
  int lim = V - vw0 - 4 * half;
  if constexpr (TAIL) asm volatile("" : "+v"(lim));
  return lim;
}
template <bool TAIL>
__device__ __forceinline__ bool col_in(int e, int lim) {
  return !TAIL || acc_row(e >> 4, e & 15, 0) < lim;
}

// z(e) gives entry e of the lane's column (an accumulator register, so that
// the forward keeps no copy of the column in VGPRs)
template <bool TAIL, class Z>
__device__ __forceinline__ float col_max(const Z& z, int vw0, int half, int V) {
  const int lim = col_lim<TAIL>(vw0, half, V);
  float mx = -INFINITY;
#pragma unroll
  for (int e = 0; e < 64; ++e)
    if (col_in<TAIL>(e, lim)) mx = fmaxf(mx, z(e));
  return mx;
}

// sum of 2^(z c - mn) over the column
template <bool TAIL, class Z>
__device__ __forceinline__ float col_sum_exp2(const Z& z, float c, float mn, int vw0, int half,
                                              int V) {
  const int lim = col_lim<TAIL>(vw0, half, V);
  float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
  for (int e = 0; e < 64; e += 4) {
    const float t0 = fast_exp2(fmaf(z(e + 0), c, -mn)), t1 = fast_exp2(fmaf(z(e + 1), c, -mn));
    const float t2 = fast_exp2(fmaf(z(e + 2), c, -mn)), t3 = fast_exp2(fmaf(z(e + 3), c, -mn));
    s0 += col_in<TAIL>(e + 0, lim) ? t0 : 0.f;
    s1 += col_in<TAIL>(e + 1, lim) ? t1 : 0.f;
    s2 += col_in<TAIL>(e + 2, lim) ? t2 : 0.f;
    s3 += col_in<TAIL>(e + 3, lim) ? t3 : 0.f;
  }
  return (s0 + s1) + (s2 + s3);
}

// sums of 2^y and 2^y y, y = z c - mn, over the column
template <bool TAIL, class Z>
__device__ __forceinline__ void col_ent(const Z& z, float c, float mn, int vw0, int half, int V,
                                        float& st, float& ut) {
  const int lim = col_lim<TAIL>(vw0, half, V);
  float st0 = 0.f, st1 = 0.f, ut0 = 0.f, ut1 = 0.f;
#pragma unroll
  for (int e = 0; e < 64; e += 2) {
    const float y0 = fmaf(z(e), c, -mn), y1 = fmaf(z(e + 1), c, -mn);
    float e0 = fast_exp2(y0), e1 = fast_exp2(y1);
    if (!col_in<TAIL>(e, lim)) e0 = 0.f;
    if (!col_in<TAIL>(e + 1, lim)) e1 = 0.f;
    st0 += e0;
    st1 += e1;
    ut0 += (e0 > 0.f) ? e0 * y0 : 0.f;
    ut1 += (e1 > 0.f) ? e1 * y1 : 0.f;
  }
  st = st0 + st1;
  ut = ut0 + ut1;
}

// z(tgt) (tgt in [0, 64)); 0 for tgt < 0.
template <class Z>
__device__ __forceinline__ float pick64(const Z& z, int tgt) {
  float v = 0.0f;
#pragma unroll
  for (int e = 0; e < 64; ++e) v = (e == tgt) ? z(e) : v;
  return v;
}

// ---------------------------------------------------------------------------
// Gradient tile epilogue (bf16): G = coef * 2^(z*c - lse2) (the teacher term
// is applied afterwards by grad_teacher_kernel) for the 256 x 256 tile,
// written through LDS as whole 16-byte granules. G is stored in blocks of 256
// vocabulary columns: block b holds columns [256 b, 256 b + 256) of every row,
// rows 512 bytes apart, blocks a.ldg bytes apart, so a tile's 256 rows are one
// contiguous 128 KB store. The dW contraction reads a block's rows as they are
// (transposed fragment reads), so no transposed copy is written.
//
// The tile is staged in the idle main-loop stage area as [256 t][256 v] bf16,
// rows kGPitch = 528 B apart (padding puts the rows that consecutive lanes
// write in distinct banks), then all 256 threads store rows. Every wave takes
// part in the barriers; a wave whose half tile lies past the vocabulary
// computes nothing (its rows are at or past Vp and never stored).
// ---------------------------------------------------------------------------
// fp32 gradient tile, one token column t of a lane (its 64 logits z of the
// half tile from vocabulary row vw0): coef * q (the teacher term is applied by
// grad_teacher_kernel) into G [rows][Vp], which feeds dHidden, and G^T
// [Vp][Cp], which feeds dW. Token columns in [rows, round_up(rows, 8)) are
// written as zeros into G^T, so that the 16-byte granules the contractions
// read never hold stale data; vocabulary rows in [V, Vp) hold finite values
// that meet zero rows of W^T.
__device__ __forceinline__ void grad_column_f32(float (&z)[64], const SweepArgs& a, int t, int vw0,
                                                int half, int rows, float c, float coef,
                                                float lse2) {
  const int Vp = (int)round_up(a.V, 8);
  const int tpad = (int)round_up(rows, 8);
#pragma unroll
  for (int e = 0; e < 64; ++e) z[e] = fast_exp2(fmaf(z[e], c, -lse2));
  if (t >= tpad) return;
  const bool gv = t < rows;
  char* grow = a.G + (int64_t)t * a.ldg;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int v = vw0 + i * 32 + 8 * q + 4 * half;
      if (v >= Vp) continue;
      // token columns past `rows` hold a repeated row: exact zeros
      const float g0 = gv ? z[i * 16 + 4 * q + 0] * coef : 0.0f;
      const float g1 = gv ? z[i * 16 + 4 * q + 1] * coef : 0.0f;
      const float g2 = gv ? z[i * 16 + 4 * q + 2] * coef : 0.0f;
      const float g3 = gv ? z[i * 16 + 4 * q + 3] * coef : 0.0f;
      char* gt = a.GT + (int64_t)v * a.ldgt + (int64_t)t * 4;
      if (gv) *(float4*)(grow + (int64_t)v * 4) = make_float4(g0, g1, g2, g3);
      *(float*)(gt) = g0;
      *(float*)(gt + a.ldgt) = g1;
      *(float*)(gt + 2 * a.ldgt) = g2;
      *(float*)(gt + 3 * a.ldgt) = g3;
    }
}

constexpr int kGPitch = 528;
constexpr int kStagingLds = 256 * kGPitch;   // inside the main-loop stage area

// The scale coef is folded into the exponent, coef * 2^x = 2^(x + log2|coef|),
// and its sign applied to the bf16 bits (lc2 = log2|coef|, -inf for 0;
// sgn = the sign bit of coef in both halves of a bf16 pair). Token rows in
// [rows, round_up(rows, 8)) are written as zeros (the dW contraction reads
// whole groups of 8 token rows).
// LOGITS: the same store of z itself (no exponential, no scale), rows < rows
// only, as rows [rows][Vld] (a.ldg bytes per row).
template <bool LOGITS>
__device__ __forceinline__ void grad_tile_staged(floatx16 (&acc)[4][4], const SweepArgs& a, int vt,
                                                 int jt, int rows, int tl0, float c, float lc2,
                                                 uint32_t sgn, const float (&lse2)[4], char* lds) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, wm = w >> 1, wn = w & 1;
  const int half = lane >> 5;
  const int vw0 = vt * kTile + wm * 128;
  const bool live = vw0 < a.V;
  const int Vp = (int)round_up(a.V, 8);
  const int tlim = LOGITS ? rows : (int)round_up(rows, 8);
  char* sg = lds;
  // every wave has read its last main-loop fragments before the area is reused
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    __builtin_amdgcn_sched_barrier(0);
    if (live) {
      // vocabulary rows past V have z = 0 (zero W rows): their finite values
      // land in G's padding columns [V, Vp), which the contractions multiply
      // by zeros or never read
      float z[64];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) z[i * 16 + r] = acc[i][j][r];
      if constexpr (!LOGITS) {
        // token columns past `rows` hold a repeated row: exact zeros
        const float off = (tl0 + 32 * j < rows) ? lc2 - lse2[j] : -INFINITY;
#pragma unroll
        for (int e = 0; e < 64; ++e) z[e] = fast_exp2(fmaf(z[e], c, off));
      }
      // this lane's token row of the tile and its first vocabulary column
      // (wm*128 + 4*half); entry (i, r) is at column + i*32 + 8*(r/4) + r%4
      char* gb = sg + (wn * 128 + 32 * j + (lane & 31)) * kGPitch + (wm * 128 + 4 * half) * 2;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int dv = i * 32 + 8 * q;
          const bf16x2 p01 = {(__bf16)z[i * 16 + 4 * q + 0], (__bf16)z[i * 16 + 4 * q + 1]};
          const bf16x2 p23 = {(__bf16)z[i * 16 + 4 * q + 2], (__bf16)z[i * 16 + 4 * q + 3]};
          const uint32_t u01 = __builtin_bit_cast(uint32_t, p01) ^ sgn;
          const uint32_t u23 = __builtin_bit_cast(uint32_t, p23) ^ sgn;
          *(uint2*)(gb + dv * 2) = make_uint2(u01, u23);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  __syncthreads();
  // 256 rows x 32 granules of 8 vocabulary entries
  char* gt = LOGITS ? a.G + (int64_t)vt * kTile * 2 : a.G + (int64_t)vt * a.ldg;
  const int64_t rpitch = LOGITS ? a.ldg : 512;
#pragma unroll 4
  for (int it = 0; it < 32; ++it) {
    const int g = it * 256 + tid;
    const int tp = g >> 5, gr = g & 31;
    const int t = jt * kTile + tp;
    const int v = vt * kTile + gr * 8;
    if (t < tlim && v < Vp) {
      const u32x4 val = *(const u32x4*)(sg + tp * kGPitch + gr * 16);
      __builtin_nontemporal_store(val, (u32x4*)(gt + (int64_t)t * rpitch + gr * 16));
    }
  }
  // the next tile's loads reuse the area
  __syncthreads();
}

template <typename T, int KIND, bool MAP>
__device__ __forceinline__ void sweep_body(SweepArgs a) {
  // main-loop stages; the gradient tile epilogue stages its output here too
  __shared__ __attribute__((aligned(16))) char lds[kMainLds];
  static_assert(kStagingLds <= kMainLds, "staging area");
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, wm = w >> 1, wn = w & 1;
  const int half = lane >> 5;
  // the forward, and the forward that also stores its logits
  constexpr bool kFwd = KIND == kSweepFwd || KIND == kSweepFwdZ;
  static_assert(KIND != kSweepFwdZ || !MAP, "stored logits: no row map");

  int rows = a.row_cap;
  int ntt, jt, b, vt_begin, vt_end;
  if constexpr (KIND == kSweepSDrawTiles) {
    // one vocabulary tile and up to kTile of the launch rows that draw in it
    // (listed at idx + toff[vt]). Work-groups go slice by slice over all
    // tiles: the first slices, nearly all of the work, are dispatched first
    // and spread over every XCD; the later slices of most tiles are empty and
    // end at once.
    const int nvt = (int)ceil_div(a.V, kTile);
    const int nsl = (int)ceil_div(a.row_cap, kTile);
    if ((int)blockIdx.x >= nvt * nsl) return;
    const int vt = (int)blockIdx.x % nvt, sl = (int)blockIdx.x / nvt;
    const int n = a.tcnt[vt] - sl * kTile;
    if (n <= 0) return;
    a.idx += a.toff[vt];
    a.row_begin = sl * kTile;
    rows = n < kTile ? n : kTile;
    ntt = 1;
    jt = 0;
    b = 0;
    vt_begin = vt;
    vt_end = vt + 1;
  } else {
    if (a.nrows_dev) {
      int n = *a.nrows_dev - a.row_begin;
      rows = n < rows ? n : rows;
    }
    if (rows <= 0) return;
    ntt = (int)ceil_div(rows, kTile);
    const int nvt = (int)ceil_div(a.V, kTile);
    const int ns = sweep_splits(ntt, nvt, a.ncu);
    const int total = ntt * ns;
    if ((int)blockIdx.x >= total) return;
    // Raster. A launch of at most 8 token tiles (one chunk) takes them in
    // pairs: the 32 work-groups an XCD runs at once cover 2 token tiles (whose
    // panels, 2.9 MB at H = 2880, stay in its 4 MB L2) and 16 vocabulary
    // ranges, each W panel shared 2 ways and each range of W read by 4 XCDs.
    // Measured on the gradient tile at the 32K-context shapes (ms per launch):
    // all 8 token tiles per XCD 2.27, 4 tiles 2.22, 2 tiles 2.20, 1 tile 2.24.
    // A launch over many token tiles walks the vocabulary ranges fastest
    // instead, so that an XCD holds few token panels at a time.
    const int L = xcd_remap(blockIdx.x, total);
    const int GM = ntt <= 8 ? (ntt < 2 ? ntt : 2) : 1;
    const int grp = L / (GM * ns), in = L % (GM * ns);
    const int gm = (ntt - grp * GM) < GM ? (ntt - grp * GM) : GM;
    jt = grp * GM + in % gm;
    b = in / gm;
    vt_begin = (int)((int64_t)b * nvt / ns);
    vt_end = (int)((int64_t)(b + 1) * nvt / ns);
  }

  constexpr int esz = Elem<T>::size;
  const int64_t kbytes = (int64_t)a.H * esz;
  const int nk = (int)ceil_div(kbytes, kKB);
  const float c = kLog2e / a.T;

  // token columns owned by this lane: launch rows tl0 + 32*j
  const int tl0 = jt * kTile + wn * 128 + (lane & 31);
  int orow[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int cr = a.row_begin + ((tl0 + 32 * j) < rows ? tl0 + 32 * j : 0);
    orow[j] = a.idx ? a.idx[cr] : cr;
  }

  // per-kind running state
  float m[4], s[4];
  double S64[4], U64[4];
  int64_t cbase[4];
  int ccur[4];
  float lse2[4];
  float tej[4];   // emission threshold of each token column (teacher cache writer)
  int dcur[4], dnext[4];   // sampled targets: next draw of the column and its unit
  int ecnt[4];             // teacher cache writer: candidates this lane appended per column
  float coef = 0.0f, lc2 = -INFINITY;
  uint32_t sgn = 0u;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    m[j] = -INFINITY;
    s[j] = 0.0f;
    S64[j] = 0.0;
    U64[j] = 0.0;
    lse2[j] = 0.0f;
    cbase[j] = 0;
    ccur[j] = 0;
    if constexpr (kFwd) {
      cbase[j] = (int64_t)orow[j] * a.K;
      ccur[j] = (tl0 + 32 * j < rows) ? lower_bound_ids(a.ids_s + cbase[j], a.K, vt_begin * kTile)
                                      : a.K;
    }
    if constexpr (KIND == kSweepBwdG)
      lse2[j] = (tl0 + 32 * j < rows) ? a.lse[orow[j]] * kLog2e : 0.0f;
    tej[j] = INFINITY;
    ecnt[j] = 0;
    if constexpr (KIND == kSweepEmit)
      if (tl0 + 32 * j < rows) tej[j] = a.te[tl0 + 32 * j];
    dcur[j] = a.N;
    dnext[j] = 0x7FFFFFFF;
    if constexpr (KIND == kSweepSDrawTiles) {
      // a row's draws are ordered by unit; start at the first one in this
      // work-group's vocabulary tile
      if (tl0 + 32 * j < rows) {
        const int32_t* du = a.dunit + (int64_t)orow[j] * a.N;
        dcur[j] = lower_bound_ids(du, a.N, 2 * vt_begin);
        dnext[j] = dcur[j] < a.N ? du[dcur[j]] : 0x7FFFFFFF;
      }
    }
  }
  if constexpr (KIND == kSweepBwdG) {
    const int n = *a.nrows_dev;
    coef = (n > 0) ? a.grad_loss[0] / ((float)n * a.T) : 0.0f;
    lc2 = coef != 0.0f ? log2f(fabsf(coef)) : -INFINITY;
    sgn = coef < 0.0f ? 0x80008000u : 0u;
  }

  bool pf = false;
  for (int vt = vt_begin; vt < vt_end; ++vt) {
    // operand state is rebuilt per tile so that nothing of the main loop stays
    // live (and spillable) across the register-heavy epilogues
    DmaOperand la;
    la.init(a.W + (int64_t)vt * kTile * a.ldw, a.ldw, a.V - vt * kTile, 0, kbytes);
    typename std::conditional<MAP, DmaOperandMap, DmaOperand>::type lb;
    if constexpr (MAP) {
      lb.init(a.X, a.ldx, a.idx, a.row_begin + jt * kTile, a.row_begin + rows, 0, kbytes);
    } else {
      lb.init(a.X + (int64_t)(a.x_row0 + jt * kTile) * a.ldx, a.ldx, rows - jt * kTile, 0,
              kbytes);
    }
    floatx16 acc[4][4];
    gemm_mainloop<T, kSweepAEarly>(acc, la, lb, nk, lds, pf);
    pf = false;
    if constexpr (KIND != kSweepBwdG && KIND != kSweepLogits) {
      // the next tile's first two stages load while this tile's epilogue runs
      // (these epilogues use no LDS; the gradient and logits tiles stage
      // their stores there)
      if (vt + 1 < vt_end) {
        DmaOperand ln;
        ln.init(a.W + (int64_t)(vt + 1) * kTile * a.ldw, a.ldw, a.V - (vt + 1) * kTile, 0, kbytes);
        gemm_prefetch<kSweepAEarly>(ln, lb, nk, lds);
        pf = true;
      }
    }

    const int vw0 = vt * kTile + wm * 128;
    if constexpr (KIND == kSweepBwdG && sizeof(T) == 2) {
      grad_tile_staged<false>(acc, a, vt, jt, rows, tl0, c, lc2, sgn, lse2, lds);
      continue;
    }
    if constexpr (KIND == kSweepLogits) {
      static_assert(sizeof(T) == 2, "the logits tile is stored as bf16");
      grad_tile_staged<true>(acc, a, vt, jt, rows, tl0, c, 0.0f, 0u, lse2, lds);
      continue;
    }
    if (vw0 >= a.V) continue;  // wave-uniform: this half tile is past the vocabulary
    const bool tail = vw0 + 128 > a.V;

    // the next teacher ids of every token column, for the walks below. The
    // row offsets pass through an opaque copy each tile, so that the
    // addresses derived from them are formed here rather than hoisted out of
    // the tile loop (eight live 64-bit pointers, spilled and reloaded with a
    // wait for memory on every tile).
    int win[4][kWin];
    int64_t cb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) cb[j] = opaque(cbase[j]);
    if constexpr (kFwd) {
#pragma unroll
      for (int j = 0; j < 4; ++j) window_load(cb[j], ccur[j], a.ids_s, a.K, win[j]);
    }

    // One token column at a time; the next column starts only after this one
    // is done (sched_barrier), which bounds the live registers of the
    // epilogue. The body is instantiated per column, so that every
    // accumulator index is a constant: the forward and entropy reductions read
    // the accumulators directly, the other kinds through a copy (z).
    auto column = [&](auto jc) {
      constexpr int j = decltype(jc)::value;
      __builtin_amdgcn_sched_barrier(0);
      // Entries past V hold 0 (zero W rows). The forward and entropy
      // reductions exclude them on the last tile; the gradient tile writes
      // their finite values into padding only; the teacher cache writer sets
      // them to -inf here.
      float z[64];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = acc[i][j][r];
          if constexpr (KIND == kSweepPilot || KIND == kSweepEmit)
            if (tail && vw0 + acc_row(i, r, half) >= a.V) x = -INFINITY;
          z[i * 16 + r] = x;
        }

      if constexpr (KIND == kSweepPilot) {
        // the maximum of each group of 16 logits this lane holds (block i of
        // the lane's half tile), stored transposed: group
        // vt*16 + wm*8 + 2i + half, the 32 lanes of a group row writing 32
        // consecutive tokens. Entries past V hold -inf.
        const int t = tl0 + 32 * j;
        if (t < rows) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float gmx = z[i * 16];
#pragma unroll
            for (int r = 1; r < 16; ++r) gmx = fmaxf(gmx, z[i * 16 + r]);
            const int g = vt * 16 + wm * 8 + 2 * i + half;
            a.zp[(int64_t)g * a.ldp + t] = gmx;
          }
        }
      }

      if constexpr (KIND == kSweepEmit) {
        // every logit at or above the row's threshold joins the row's
        // candidates (columns past the rows have an infinite threshold and
        // are excluded besides). Entries past V are tested explicitly: they
        // hold -inf, which a threshold of -inf (a row with fewer pilot groups
        // than K) admits. Each writer - this work-group's vocabulary range,
        // and within it this wave and lane half - appends to a sub-list of
        // its own in the row's list, with room for every entry it can see
        // (64 per tile of the range), so no atomic is needed; the gather
        // kernel then closes the gaps.
        const int t = tl0 + 32 * j;
        const int nr = vt_end - vt_begin;
        const int64_t sb = (int64_t)t * a.cap + (int64_t)vt_begin * kTile +
                           (int64_t)(wm * 2 + half) * nr * 64;
#pragma unroll
        for (int e = 0; e < 64; ++e) {
          const int v = vw0 + acc_row(e >> 4, e & 15, half);
          if (z[e] >= tej[j] && t < rows && (!tail || v < a.V)) {
            a.cid[sb + ecnt[j]] = v + a.id_offset;
            a.cz[sb + ecnt[j]] = z[e];
            ++ecnt[j];
          }
        }
      }

      if constexpr (kFwd) {
        const auto za = [&](int e) { return acc[e >> 4][j][e & 15]; };
        const float mx = tail ? col_max<true>(za, vw0, half, a.V) : col_max<false>(za, vw0, half, a.V);
        const float mn = fmaxf(m[j], mx * c);
        if (mn != -INFINITY) {
          const float sc = fast_exp2(m[j] - mn);
          const float st = tail ? col_sum_exp2<true>(za, c, mn, vw0, half, a.V)
                                : col_sum_exp2<false>(za, c, mn, vw0, half, a.V);
          s[j] = s[j] * sc + st;
          m[j] = mn;
        }
        // z at the teacher ids, stored at their sorted positions; the
        // combine forms sum_k p_k z_k from them
        walk_window(cb[j], ccur[j], win[j], a.ids_s, a.K, vw0, half,
                    [&](int tgt, int64_t e) {
                      const float val = pick64(za, tgt);
                      if (tgt >= 0) a.zs[e] = val;
                    });
      }

      if constexpr (KIND == kSweepEnt) {
        const auto za = [&](int e) { return acc[e >> 4][j][e & 15]; };
        const float mx = tail ? col_max<true>(za, vw0, half, a.V) : col_max<false>(za, vw0, half, a.V);
        const float mn = fmaxf(m[j], mx * c);
        if (mn != -INFINITY) {
          float st, ut;
          if (tail) col_ent<true>(za, c, mn, vw0, half, a.V, st, ut);
          else col_ent<false>(za, c, mn, vw0, half, a.V, st, ut);
          if (m[j] == -INFINITY) {
            S64[j] = st;
            U64[j] = ut;
          } else {
            const float dm = m[j] - mn;
            const double f = (double)fast_exp2(dm);
            U64[j] = (U64[j] + S64[j] * (double)dm) * f + (double)ut;
            S64[j] = S64[j] * f + (double)st;
          }
          m[j] = mn;
        }
      }

      if constexpr (KIND == kSweepSMass || KIND == kSweepSDrawTiles) {
        // weights 2^(z c - mc) of the teacher softmax at T in the unit's own
        // scale, mc = c times the largest z of the unit's 128 entries (entries
        // past V weigh 0), summed per quad: four consecutive vocabulary
        // entries. The lane's quad k = 4i + q sits at position 2k + half of
        // the unit; the partner lane (other half) holds the others. Both
        // passes compute the same values in the same order, so the draw pass
        // sees the masses the mass pass stored.
        float mx = -INFINITY;
#pragma unroll
        for (int e = 0; e < 64; ++e) {
          const bool in = !tail || vw0 + acc_row(e >> 4, e & 15, half) < a.V;
          mx = in ? fmaxf(mx, z[e]) : mx;
        }
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float mc = mx * c;
#pragma unroll
        for (int e = 0; e < 64; ++e) {
          const bool in = !tail || vw0 + acc_row(e >> 4, e & 15, half) < a.V;
          z[e] = in ? fast_exp2(fmaf(z[e], c, -mc)) : 0.0f;
        }
        float g[16], gp[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) g[k] = (z[4 * k] + z[4 * k + 1]) + (z[4 * k + 2] + z[4 * k + 3]);
#pragma unroll
        for (int k = 0; k < 16; ++k) gp[k] = __shfl_xor(g[k], 32, 64);
        // quad at position 2k is half 0's, at 2k + 1 half 1's
        const auto quad = [&](int k, int s) { return (s == half) ? g[k] : gp[k]; };
        const int t = tl0 + 32 * j;
        const int unit = vw0 >> 7;
        if constexpr (KIND == kSweepSMass) {
          float run = 0.0f;
#pragma unroll
          for (int k = 0; k < 16; ++k) {
            run += quad(k, 0);
            run += quad(k, 1);
          }
          if (t < rows && half == 0) {
            a.tmass[(int64_t)unit * a.ldm + t] = (double)run;
            a.tscale[(int64_t)unit * a.ldm + t] = mc;
          }
        } else {
          // the column's draws up to this unit: those of lower units belong
          // to the other wave and are passed over
          const int64_t rb = (int64_t)orow[j] * a.N;
          while (true) {
            const bool act = dnext[j] <= unit;
            if (ballot(act) == 0) break;
            if (act && dnext[j] == unit) {
              double r = a.dres[rb + dcur[j]];
              // the first quad whose running mass passes r; past the unit's
              // mass (rounding, or a draw at the top of the distribution),
              // the last quad of positive mass with r unbounded
              float run = 0.0f, pb = 0.0f, pbl = 0.0f;
              int qs = -1, ql = -1;
#pragma unroll
              for (int k = 0; k < 16; ++k)
#pragma unroll
                for (int sh = 0; sh < 2; ++sh) {
                  const float gq = quad(k, sh);
                  const float pa = run + gq;
                  if (qs < 0 && (double)pa > r) {
                    qs = 2 * k + sh;
                    pb = run;
                  }
                  if (gq > 0.0f) {
                    ql = 2 * k + sh;
                    pbl = run;
                  }
                  run = pa;
                }
              if (qs < 0) {
                qs = ql;
                pb = pbl;
                r = INFINITY;
              }
              if (qs >= 0 && (qs & 1) == half) {
                // inside the quad: the first entry whose running mass passes
                // the rest of r, else its last entry of positive weight
                const int kq = qs >> 1;
                float e0 = 0.0f, e1 = 0.0f, e2 = 0.0f, e3 = 0.0f;
#pragma unroll
                for (int k = 0; k < 16; ++k)
                  if (k == kq) {
                    e0 = z[4 * k];
                    e1 = z[4 * k + 1];
                    e2 = z[4 * k + 2];
                    e3 = z[4 * k + 3];
                  }
                const double rq = r - (double)pb;
                const float c0 = e0, c1 = c0 + e1, c2 = c1 + e2, c3 = c2 + e3;
                int pick = (double)c0 > rq ? 0 : (double)c1 > rq ? 1 : (double)c2 > rq ? 2
                         : (double)c3 > rq ? 3 : -1;
                if (pick < 0) pick = e3 > 0.0f ? 3 : e2 > 0.0f ? 2 : e1 > 0.0f ? 1 : 0;
                a.sids[rb + dcur[j]] = vw0 + 4 * qs + pick;
              }
            }
            if (act) {
              ++dcur[j];
              dnext[j] = dcur[j] < a.N ? a.dunit[rb + dcur[j]] : 0x7FFFFFFF;
            }
          }
        }
      }

      if constexpr (KIND == kSweepBwdG && sizeof(T) == 4)
        grad_column_f32(z, a, tl0 + 32 * j, vw0, half, rows, c, coef, lse2[j]);
      if constexpr (KIND == kSweepFwdZ) {
        // the column's logits as the lanes hold them, each store instruction
        // 1 KB of consecutive lanes, after the column's reductions (so that
        // the column's accumulators are free again afterwards). A buffer
        // resource over the tile keeps the addresses in scalar registers.
        const __amdgpu_buffer_rsrc_t zr = make_rsrc_uniform(
            a.Zt + ((int64_t)jt * ceil_div(a.V, kTile) + vt) * kZTile, kZTile * 4);
        const int wofs = __builtin_amdgcn_readfirstlane(w) * 64 * 1024;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const u32x4 v = {__float_as_uint(acc[i][j][4 * q]), __float_as_uint(acc[i][j][4 * q + 1]),
                             __float_as_uint(acc[i][j][4 * q + 2]),
                             __float_as_uint(acc[i][j][4 * q + 3])};
            __builtin_amdgcn_raw_buffer_store_b128(v, zr, lane * 16,
                                                   wofs + ((i * 4 + j) * 4 + q) * 1024, 0);
          }
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    column(std::integral_constant<int, 0>());
    column(std::integral_constant<int, 1>());
    column(std::integral_constant<int, 2>());
    column(std::integral_constant<int, 3>());
  }

  if constexpr (KIND == kSweepEmit) {
    // the length of each of this lane's sub-lists: [row][range][writer]
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = tl0 + 32 * j;
      if (t < rows) a.scnt[(int64_t)t * a.scnt_ld + b * 4 + wm * 2 + half] = ecnt[j];
    }
  }
  if constexpr (KIND == kSweepBwdG || KIND == kSweepLogits || KIND == kSweepPilot ||
                KIND == kSweepEmit ||
                KIND == kSweepSMass || KIND == kSweepSDrawTiles)
    return;

  // ---- end of sweep: merge lane halves, then the two waves sharing tokens
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if constexpr (kFwd) {
      const float m2 = __shfl_xor(m[j], 32, 64), s2 = __shfl_xor(s[j], 32, 64);
      lse2_merge(m[j], s[j], m2, s2);
    } else {
      const float m2 = __shfl_xor(m[j], 32, 64);
      const double S2 = __shfl_xor(S64[j], 32, 64), U2 = __shfl_xor(U64[j], 32, 64);
      ent_merge(m[j], S64[j], U64[j], m2, S2, U2);
    }
  }
  __syncthreads();
  // exchange area: [wn][128] x {m, s|S, d|U}
  float* xm = (float*)lds;
  double* xa = (double*)(lds + 2 * 128 * 4);
  double* xb = xa + 2 * 128;
  if (wm == 1 && lane < 32) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = wn * 128 + j * 32 + lane;
      xm[t] = m[j];
      if constexpr (kFwd) {
        xa[t] = s[j];
      } else {
        xa[t] = S64[j];
        xb[t] = U64[j];
      }
    }
  }
  __syncthreads();
  if (wm == 0 && lane < 32) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = wn * 128 + j * 32 + lane;
      if (tl0 + 32 * j >= rows) continue;
      const int64_t o = (int64_t)b * ntt * kTile + tl0 + 32 * j;
      if constexpr (kFwd) {
        lse2_merge(m[j], s[j], xm[t], (float)xa[t]);
        a.pm[o] = m[j];
        a.ps[o] = s[j];
      } else {
        ent_merge(m[j], S64[j], U64[j], xm[t], xa[t], xb[t]);
        a.em[o] = m[j];
        a.es[o] = S64[j];
        a.eu[o] = U64[j];
      }
    }
  }
}

// grid size: the largest work-group count any row count up to rows_max can use
int sweep_grid(int64_t rows_max, int V, int ncu) {
  static std::mutex mu;
  static std::map<std::tuple<int64_t, int, int>, int> memo;
  std::lock_guard<std::mutex> g(mu);
  auto key = std::make_tuple(rows_max, V, ncu);
  auto it = memo.find(key);
  if (it != memo.end()) return it->second;
  const int nvt = (int)ceil_div(V, kTile);
  const int ntt_max = (int)ceil_div(rows_max, kTile);
  int best = 1;
  for (int n = 1; n <= ntt_max; ++n) {
    int g2 = n * sweep_splits(n, nvt, ncu);
    if (g2 > best) best = g2;
  }
  memo[key] = best;
  return best;
}

// One kernel symbol per variant, named after the step it performs (these are
// the names that traces and counter dumps show).
#define KD_SWEEP_KERNEL(NAME, T, KIND, MAP)                                  \
  extern "C" __global__ __launch_bounds__(256, 1) void NAME(SweepArgs a) { \
    sweep_body<T, KIND, MAP>(a);                                           \
  }
KD_SWEEP_KERNEL(kd_fwd_lse_gather_bf16, __bf16, kSweepFwd, false)
KD_SWEEP_KERNEL(kd_fwd_lse_gather_rows_bf16, __bf16, kSweepFwd, true)
KD_SWEEP_KERNEL(kd_bwd_grad_tile_bf16, __bf16, kSweepBwdG, false)
KD_SWEEP_KERNEL(kd_entropy_sweep_bf16, __bf16, kSweepEnt, false)
KD_SWEEP_KERNEL(kd_fwd_lse_gather_f32, float, kSweepFwd, false)
KD_SWEEP_KERNEL(kd_fwd_lse_gather_rows_f32, float, kSweepFwd, true)
KD_SWEEP_KERNEL(kd_bwd_grad_tile_f32, float, kSweepBwdG, false)
KD_SWEEP_KERNEL(kd_entropy_sweep_f32, float, kSweepEnt, false)
KD_SWEEP_KERNEL(kd_teacher_pilot_bf16, __bf16, kSweepPilot, false)
KD_SWEEP_KERNEL(kd_teacher_emit_bf16, __bf16, kSweepEmit, false)
KD_SWEEP_KERNEL(kd_teacher_pilot_f32, float, kSweepPilot, false)
KD_SWEEP_KERNEL(kd_teacher_emit_f32, float, kSweepEmit, false)
KD_SWEEP_KERNEL(kd_sample_mass_bf16, __bf16, kSweepSMass, false)
KD_SWEEP_KERNEL(kd_sample_mass_f32, float, kSweepSMass, false)
KD_SWEEP_KERNEL(kd_sample_draw_tiles_bf16, __bf16, kSweepSDrawTiles, true)
KD_SWEEP_KERNEL(kd_sample_draw_tiles_f32, float, kSweepSDrawTiles, true)
KD_SWEEP_KERNEL(kd_cmp_logits_bf16, __bf16, kSweepLogits, false)
KD_SWEEP_KERNEL(kd_cmp_logits_rows_bf16, __bf16, kSweepLogits, true)
KD_SWEEP_KERNEL(kd_fwd_lse_gather_keep_bf16, __bf16, kSweepFwdZ, false)
KD_SWEEP_KERNEL(kd_fwd_lse_gather_keep_f32, float, kSweepFwdZ, false)
#undef KD_SWEEP_KERNEL

hipError_t launch_sweep(int kind, int f32, int map, const SweepArgs& a, int grid, hipStream_t st) {
  if (grid <= 0) return hipSuccess;
  dim3 g(grid), blk(kThreads);
#define KD_SWEEP(NAME) hipLaunchKernelGGL(NAME, g, blk, 0, st, a)
  if (!f32) {
    if (kind == kSweepFwd && map) KD_SWEEP(kd_fwd_lse_gather_rows_bf16);
    else if (kind == kSweepFwd) KD_SWEEP(kd_fwd_lse_gather_bf16);
    else if (kind == kSweepFwdZ && map) return hipErrorInvalidValue;   // no row map
    else if (kind == kSweepFwdZ) KD_SWEEP(kd_fwd_lse_gather_keep_bf16);
    else if (kind == kSweepBwdG) KD_SWEEP(kd_bwd_grad_tile_bf16);
    else if (kind == kSweepPilot) KD_SWEEP(kd_teacher_pilot_bf16);
    else if (kind == kSweepEmit) KD_SWEEP(kd_teacher_emit_bf16);
    else if (kind == kSweepSMass) KD_SWEEP(kd_sample_mass_bf16);
    else if (kind == kSweepSDrawTiles) KD_SWEEP(kd_sample_draw_tiles_bf16);
    else if (kind == kSweepLogits && map) KD_SWEEP(kd_cmp_logits_rows_bf16);
    else if (kind == kSweepLogits) KD_SWEEP(kd_cmp_logits_bf16);
    else KD_SWEEP(kd_entropy_sweep_bf16);
  } else {
    if (kind == kSweepFwd && map) KD_SWEEP(kd_fwd_lse_gather_rows_f32);
    else if (kind == kSweepFwd) KD_SWEEP(kd_fwd_lse_gather_f32);
    else if (kind == kSweepBwdG) KD_SWEEP(kd_bwd_grad_tile_f32);
    else if (kind == kSweepPilot) KD_SWEEP(kd_teacher_pilot_f32);
    else if (kind == kSweepEmit) KD_SWEEP(kd_teacher_emit_f32);
    else if (kind == kSweepSMass) KD_SWEEP(kd_sample_mass_f32);
    else if (kind == kSweepSDrawTiles) KD_SWEEP(kd_sample_draw_tiles_f32);
    else if (kind == kSweepFwdZ && map) return hipErrorInvalidValue;   // no row map
    else if (kind == kSweepFwdZ) KD_SWEEP(kd_fwd_lse_gather_keep_f32);
    else if (kind == kSweepLogits) return hipErrorInvalidValue;   // bf16 only
    else KD_SWEEP(kd_entropy_sweep_f32);
  }
#undef KD_SWEEP
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Gradient tile of one chunk from the logits its forward sweep stored (the
// forward and backward in one call): work-group (jt, vt) reads tile (jt, vt)
// back into the accumulator layout and runs the gradient tile's own epilogue,
// so G is the one the recomputing sweep would write from the same logits.
// Launch rows, lse, coef and the store are those of kd_bwd_grad_tile_bf16.
// ---------------------------------------------------------------------------
extern "C" __global__ __launch_bounds__(256, 1) void kd_grad_tile_from_logits_bf16(SweepArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[kStagingLds];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, wm = w >> 1, wn = w & 1;
  int rows = *a.nrows_dev - a.row_begin;
  rows = rows < a.row_cap ? rows : a.row_cap;
  if (rows <= 0) return;
  const int ntt = (int)ceil_div(rows, kTile), nvt = (int)ceil_div(a.V, kTile);
  if ((int)blockIdx.x >= ntt * nvt) return;
  const int jt = (int)blockIdx.x / nvt, vt = (int)blockIdx.x % nvt;
  const float c = kLog2e / a.T;
  const int tl0 = jt * kTile + wn * 128 + (lane & 31);
  float lse2[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = tl0 + 32 * j;
    lse2[j] = r < rows ? a.lse[a.idx[a.row_begin + r]] * kLog2e : 0.0f;
  }
  const int n = *a.nrows_dev;
  const float coef = (n > 0) ? a.grad_loss[0] / ((float)n * a.T) : 0.0f;
  const float lc2 = coef != 0.0f ? log2f(fabsf(coef)) : -INFINITY;
  const uint32_t sgn = coef < 0.0f ? 0x80008000u : 0u;
  floatx16 acc[4][4];
  if (vt * kTile + wm * 128 < a.V) {
    // half tiles past the vocabulary were not stored (and are not read below);
    // the logits are read once: non-temporal loads (0.47 -> 0.44 ms per chunk
    // of 2048 rows at V = 201088; non-temporal stores in the sweep made it
    // slower by as much)
    const float* zt = a.Zt + ((int64_t)jt * nvt + vt) * kZTile + (w * 64 * 64 + lane) * 4;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const floatx4 v =
              __builtin_nontemporal_load((const floatx4*)(zt + ((i * 4 + j) * 4 + q) * 256));
          acc[i][j][4 * q] = v[0];
          acc[i][j][4 * q + 1] = v[1];
          acc[i][j][4 * q + 2] = v[2];
          acc[i][j][4 * q + 3] = v[3];
        }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  }
  grad_tile_staged<false>(acc, a, vt, jt, rows, tl0, c, lc2, sgn, lse2, lds);
}

// The same for fp32 inputs: the fp32 tile's epilogue (G and G^T, no staging),
// one token column at a time.
extern "C" __global__ __launch_bounds__(256) void kd_grad_tile_from_logits_f32(SweepArgs a) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, wm = w >> 1, wn = w & 1;
  const int half = lane >> 5;
  int rows = *a.nrows_dev - a.row_begin;
  rows = rows < a.row_cap ? rows : a.row_cap;
  if (rows <= 0) return;
  const int ntt = (int)ceil_div(rows, kTile), nvt = (int)ceil_div(a.V, kTile);
  if ((int)blockIdx.x >= ntt * nvt) return;
  const int jt = (int)blockIdx.x / nvt, vt = (int)blockIdx.x % nvt;
  const int vw0 = vt * kTile + wm * 128;
  if (vw0 >= a.V) return;   // wave-uniform: this half tile is past the vocabulary
  const float c = kLog2e / a.T;
  const int tl0 = jt * kTile + wn * 128 + (lane & 31);
  const int n = *a.nrows_dev;
  const float coef = (n > 0) ? a.grad_loss[0] / ((float)n * a.T) : 0.0f;
  const float* zt = a.Zt + ((int64_t)jt * nvt + vt) * kZTile + (w * 64 * 64 + lane) * 4;
#pragma unroll 1
  for (int j = 0; j < 4; ++j) {
    const int r = tl0 + 32 * j;
    const float lse2 = r < rows ? a.lse[a.idx[a.row_begin + r]] * kLog2e : 0.0f;
    float z[64];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const floatx4 v =
            __builtin_nontemporal_load((const floatx4*)(zt + ((i * 4 + j) * 4 + q) * 256));
        z[i * 16 + 4 * q] = v[0];
        z[i * 16 + 4 * q + 1] = v[1];
        z[i * 16 + 4 * q + 2] = v[2];
        z[i * 16 + 4 * q + 3] = v[3];
      }
    grad_column_f32(z, a, r, vw0, half, rows, c, coef, lse2);
  }
}

hipError_t launch_zgrad(int f32, const SweepArgs& a, int grid, hipStream_t st) {
  if (grid <= 0) return hipSuccess;
  if (f32)
    hipLaunchKernelGGL(kd_grad_tile_from_logits_f32, dim3(grid), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL(kd_grad_tile_from_logits_bf16, dim3(grid), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Teacher term of the gradient tile. The tile kernel stores coef * q for
// every vocabulary entry; this kernel rewrites the entries at the teacher ids
// of each chunk row as coef * q - coef * P, P the summed probability of a run
// of equal ids in the sorted table (duplicates add), in G (and, for fp32, in
// G^T). One
// thread per (row, k); the first entry of a run does the update, so no two
// threads touch one element. The stored value is read back, so the entry is
// rounded to the storage type twice (once as coef * q); the second rounding
// is of a value dominated by coef * P.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void grad_teacher_kernel(GradTeacherArgs a) {
  int rows = a.row_cap;
  {
    const int n = *a.nrows_dev - a.row_begin;
    rows = n < rows ? n : rows;
  }
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int r = (int)(q / a.K), k = (int)(q % a.K);
  if (rows <= 0 || r >= rows) return;
  const int64_t base = (int64_t)a.idx[a.row_begin + r] * a.K;
  const int id = a.ids_s[base + k];
  if (id == 0x7FFFFFFF || (k > 0 && a.ids_s[base + k - 1] == id)) return;
  float P = 0.0f;
  for (int e = k; e < a.K && a.ids_s[base + e] == id; ++e) P += a.p_s[base + e];
  const int n = *a.nrows_dev;
  const float coef = (n > 0) ? a.grad_loss[0] / ((float)n * a.T) : 0.0f;
  const float d = coef * P;
  if constexpr (sizeof(T) == 2) {
    // bf16: G only, in blocks of 256 columns (the dW contraction reads G itself)
    uint16_t* g = (uint16_t*)(a.G + (int64_t)(id >> 8) * a.ldg + (int64_t)r * 512) + (id & 255);
    const float x = bf16_to_f32(*g);
    const bf16x2 y = {(__bf16)(x - d), (__bf16)0.0f};
    *g = (uint16_t)__builtin_bit_cast(uint32_t, y);
  } else {
    T* g = (T*)(a.G + (int64_t)r * a.ldg) + id;
    T* gt = (T*)(a.GT + (int64_t)id * a.ldgt) + r;
    const float y = *g - d;
    *g = y;
    *gt = y;
  }
}

hipError_t launch_grad_teacher(int f32, const GradTeacherArgs& a, hipStream_t st) {
  const int64_t grid = ceil_div((int64_t)a.row_cap * a.K, 256);
  if (grid <= 0) return hipSuccess;
  if (f32) hipLaunchKernelGGL(grad_teacher_kernel<float>, dim3((unsigned)grid), dim3(256), 0, st, a);
  else hipLaunchKernelGGL(grad_teacher_kernel<__bf16>, dim3((unsigned)grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Forward combine: merge the split partials of each row into lse and KL_t,
// then fp64 block sums of KL over valid rows (fixed order, no atomics).
//   KL_t = sum_k p log p - (sum_k p z_k)/T + log sum_v exp(z_v/T)
// ---------------------------------------------------------------------------
// One row: merge its ns split partials (at pm/ps[b * stride + r]) into lse,
// write lse and z_topk of original row t, and return KL_t.
__device__ inline float combine_row(const CombineArgs& a, int t, int64_t r, int ns, int64_t stride) {
  float M = -INFINITY, sum = 0.0f;
  for (int b = 0; b < ns; ++b) {
    const int64_t o = (int64_t)b * stride + r;
    lse2_merge(M, sum, a.pm[o], a.ps[o]);
  }
  // sum_k p_k z_k over the row's usable ids, in sorted order; z_topk in
  // the caller's order
  const int64_t base = (int64_t)t * a.K;
  const float invT = 1.0f / a.T;
  double dot = 0.0;
  for (int k = 0; k < a.K; ++k) {
    if (a.ids_s[base + k] == 0x7FFFFFFF) break;   // out-of-range ids sort last
    const float zv = a.zs[base + k];
    dot += (double)a.p_s[base + k] * (double)zv;
    if (a.z_topk) a.z_topk[base + a.korig_s[base + k]] = zv * invT;
  }
  const float lse = (M + __log2f(sum)) * kLn2;
  a.lse[t] = lse;
  return (float)((double)a.negH[t] - dot / (double)a.T + (double)lse);
}

// A row outside the loss: lse and KL 0, z_topk NaN.
__device__ inline void combine_row_out(const CombineArgs& a, int t) {
  a.lse[t] = 0.0f;
  if (a.kl_rows) a.kl_rows[t] = 0.0f;
  if (a.z_topk)
    for (int k = 0; k < a.K; ++k) a.z_topk[(int64_t)t * a.K + k] = __int_as_float(0x7FC00000);
}

// Fixed-order fp64 sum of the 256 contributions of a work-group into
// block_sums[blockIdx.x].
__device__ inline void block_sum_kl(const CombineArgs& a, double contrib) {
  __shared__ double red[256];
  red[threadIdx.x] = contrib;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) a.block_sums[blockIdx.x] = red[0];
}

__global__ __launch_bounds__(256) void fwd_combine_kernel(CombineArgs a) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  double contrib = 0.0;
  if (t < a.S) {
    const int pr = a.pos[t];
    if (pr < 0) {
      combine_row_out(a, t);
    } else {
      // partial row: the original row when the forward ran over all rows
      const int r = a.identity ? t : pr;
      const int n = a.identity ? a.S : *a.nrows_dev;
      const int ns = sweep_splits((int)ceil_div(n, kTile), (int)ceil_div(a.V, kTile), a.ncu);
      const float kl = combine_row(a, t, r, ns, ceil_div(n, kTile) * kTile);
      if (a.kl_rows) a.kl_rows[t] = kl;
      contrib = kl;
    }
  }
  block_sum_kl(a, contrib);
}

// The rows of one chunk launch (launch row r, compacted row row_begin + r):
// the chunk's sweep wrote their partials with the split count of its own
// token tiles. One wave per row: lane b merges splits b, b + 64, ..., lane k
// takes teacher entries k, k + 64, ...; both are then folded over the wave in
// a fixed order (the row's result does not depend on timing).
__global__ __launch_bounds__(256) void fwd_combine_chunk_kernel(CombineArgs a, int row_begin,
                                                                int row_cap, float* kl_out) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  int n = *a.nrows_dev - row_begin;
  n = n < row_cap ? n : row_cap;
  if (r >= n) return;
  const int t = a.idx[row_begin + r];
  const int ns = sweep_splits((int)ceil_div(n, kTile), (int)ceil_div(a.V, kTile), a.ncu);
  const int64_t stride = ceil_div(n, kTile) * kTile;
  float M = -INFINITY, sum = 0.0f;
  for (int b = lane; b < ns; b += 64) lse2_merge(M, sum, a.pm[(int64_t)b * stride + r],
                                                 a.ps[(int64_t)b * stride + r]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(M, o, 64), s2 = __shfl_xor(sum, o, 64);
    lse2_merge(M, sum, m2, s2);
  }
  // sum_k p_k z_k over the row's usable ids (out-of-range ids sort last and
  // are left out); z_topk in the caller's order
  const int64_t base = (int64_t)t * a.K;
  const float invT = 1.0f / a.T;
  double dot = 0.0;
  for (int k = lane; k < a.K; k += 64) {
    if (a.ids_s[base + k] == 0x7FFFFFFF) break;
    const float zv = a.zs[base + k];
    dot += (double)a.p_s[base + k] * (double)zv;
    if (a.z_topk) a.z_topk[base + a.korig_s[base + k]] = zv * invT;
  }
  dot = wave_sum_d(dot);
  if (lane == 0) {
    const float lse = (M + __log2f(sum)) * kLn2;
    a.lse[t] = lse;
    kl_out[t] = (float)((double)a.negH[t] - dot / (double)a.T + (double)lse);
  }
}

// After every chunk's combine: the rows outside the loss, kl_rows, and the
// block sums of KL over the rows in the loss (the same fixed order as the
// one-pass combine).
__global__ __launch_bounds__(256) void fwd_finish_kernel(CombineArgs a, const float* kl_in) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  double contrib = 0.0;
  if (t < a.S) {
    if (a.pos[t] < 0) {
      combine_row_out(a, t);
    } else {
      const float kl = kl_in[t];
      if (a.kl_rows && a.kl_rows != kl_in) a.kl_rows[t] = kl;
      contrib = kl;
    }
  }
  block_sum_kl(a, contrib);
}

__global__ __launch_bounds__(256) void loss_final_kernel(const double* block_sums, int nblk,
                                                         const int32_t* nrows_dev, float* loss) {
  __shared__ double red[256];
  double acc = 0.0;
  for (int i = threadIdx.x; i < nblk; i += 256) acc += block_sums[i];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const int n = *nrows_dev;
    loss[0] = n > 0 ? (float)(red[0] / (double)n) : 0.0f;
  }
}

hipError_t launch_loss_final(const double* block_sums, int nblk, const int32_t* nrows_dev,
                             float* loss, hipStream_t st) {
  hipLaunchKernelGGL(loss_final_kernel, dim3(1), dim3(256), 0, st, block_sums, nblk, nrows_dev,
                     loss);
  return hipGetLastError();
}

hipError_t launch_fwd_combine(const CombineArgs& a, hipStream_t st) {
  const int nblk = (int)ceil_div(a.S, 256);
  if (nblk > 0) hipLaunchKernelGGL(fwd_combine_kernel, dim3(nblk), dim3(256), 0, st, a);
  hipLaunchKernelGGL(loss_final_kernel, dim3(1), dim3(256), 0, st, (const double*)a.block_sums,
                     nblk, a.nrows_dev, a.loss);
  return hipGetLastError();
}

hipError_t launch_fwd_combine_chunk(const CombineArgs& a, int row_begin, int row_cap,
                                    float* kl_out, hipStream_t st) {
  const int nblk = (int)ceil_div(row_cap, 4);
  if (nblk > 0)
    hipLaunchKernelGGL(fwd_combine_chunk_kernel, dim3(nblk), dim3(256), 0, st, a, row_begin,
                       row_cap, kl_out);
  return hipGetLastError();
}

hipError_t launch_fwd_finish(const CombineArgs& a, const float* kl_in, hipStream_t st) {
  const int nblk = (int)ceil_div(a.S, 256);
  if (nblk > 0) hipLaunchKernelGGL(fwd_finish_kernel, dim3(nblk), dim3(256), 0, st, a, kl_in);
  hipLaunchKernelGGL(loss_final_kernel, dim3(1), dim3(256), 0, st, (const double*)a.block_sums,
                     nblk, a.nrows_dev, a.loss);
  return hipGetLastError();
}

// Entropy combine in fp64:  H = ln(sum) - ln2 * U / sum  (U in log2 units).
__global__ __launch_bounds__(256) void ent_combine_kernel(EntCombineArgs a) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= a.S) return;
  const int ns = sweep_splits((int)ceil_div(a.S, kTile), (int)ceil_div(a.V, kTile), a.ncu);
  double M = -INFINITY, Ssum = 0.0, U = 0.0;
  const int64_t stride = ceil_div(a.S, kTile) * kTile;
  for (int b = 0; b < ns; ++b) {
    const int64_t o = (int64_t)b * stride + t;
    const double m2 = a.em[o], S2 = a.es[o], U2 = a.eu[o];
    if (m2 == -INFINITY) continue;
    if (M == -INFINITY) {
      M = m2; Ssum = S2; U = U2;
      continue;
    }
    const double mn = fmax(M, m2);
    const double f1 = exp2(M - mn), f2 = exp2(m2 - mn);
    U = (U + Ssum * (M - mn)) * f1 + (U2 + S2 * (m2 - mn)) * f2;
    Ssum = Ssum * f1 + S2 * f2;
    M = mn;
  }
  if (a.entropy) a.entropy[t] = log(Ssum) - 0.6931471805599453 * U / Ssum;
  if (a.lse) a.lse[t] = 0.6931471805599453 * (M + log2(Ssum));
}

hipError_t launch_ent_combine(const EntCombineArgs& a, hipStream_t st) {
  const int nblk = (int)ceil_div(a.S, 256);
  if (nblk > 0) hipLaunchKernelGGL(ent_combine_kernel, dim3(nblk), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace kd
