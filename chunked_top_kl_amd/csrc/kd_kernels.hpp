// Kernel argument blocks and host launchers (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kd {

enum SweepKind { kSweepFwd = 0, kSweepBwdG = 1, kSweepEnt = 2, kSweepPilot = 3, kSweepEmit = 4,
                 kSweepSMass = 5, kSweepLogits = 7, kSweepSDrawTiles = 8, kSweepFwdZ = 9 };

constexpr int64_t kZTile = 65536;     // floats of one stored 256 x 256 logit tile

// Vocabulary-sweep projection (forward LSE + gather, backward gradient tile,
// entropy). Rows are "launch rows" r in [0, rows): compacted row
// row_begin + r, original row idx[row_begin + r] (identity when idx is NULL).
struct SweepArgs {
  const char* W; int64_t ldw;         // [V,H] storage, row stride in bytes
  const char* X; int64_t ldx;         // token rows: hidden [S,H] (row map) or a gathered chunk
  int x_row0;                         // row of X holding launch row 0 (when X is read without a map)
  const int32_t* idx;                 // compacted -> original row (teacher tables, lse), or NULL
  const int32_t* nrows_dev;           // device row count N, or NULL (use row_cap)
  int row_begin, row_cap;             // this launch covers compacted rows [row_begin, row_begin+row_cap) ∩ [0,N)
  int V, H, K, ncu;
  float T;
  // teacher tables from the prepass, indexed by original row
  const int32_t* ids_s; const float* p_s; const int32_t* korig_s;
  // forward outputs: partials [split][r], split stride = (token tiles) * 256,
  // and z at every teacher id, at its position in the sorted table
  float* pm; float* ps;
  float* zs;                          // [S,K], indexed like ids_s
  // the forward that keeps its logits (no row map): the fp32
  // accumulators of tile (token tile jt, vocabulary tile vt) as the lanes hold
  // them, at Zt + (jt * ceil(V/256) + vt) * kZTile floats; within a tile, wave
  // w's lane l holds the 16 bytes of (block i, column j, quad q) at float
  // ((w * 64 + (i * 4 + j) * 4 + q) * 64 + l) * 4
  float* Zt;
  // backward
  const float* lse; const float* grad_loss;
  char* G; int64_t ldg;               // gradient tile: bf16 in blocks of 256 vocabulary
                                      // columns, [rows][256] each, blocks ldg bytes
                                      // apart; fp32 [row_cap, Vp], ldg bytes per row.
                                      // The logits kind stores z as rows [rows][Vld]
                                      // (ldg bytes per row).
  char* GT; int64_t ldgt;             // fp32: the same tile transposed [Vp, Cp] (bf16: unused)
  // entropy partials
  float* em; double* es; double* eu;
  // teacher cache writer: pilot group maxima zp[g][r] (pitch ldp floats); per-row
  // emission threshold te, append counter cnt and candidate lists cid / cz
  // (row r at r * cap); ids are stored + id_offset
  float* zp; int64_t ldp;
  const float* te; int32_t* cnt; int32_t* cid; float* cz; int64_t cap; int id_offset;
  // sampled targets (launch row r): the mass of each 128-entry vocabulary
  // unit u (one wave's half tile), tmass[u * ldm + r], in the unit's own scale
  // 2^-tscale[u * ldm + r] (tscale = its largest z * log2(e) / T); per draw n
  // of row r its unit dunit[r * N + n] and the residual mass dres[r * N + n]
  // inside that unit, in the unit's scale; the sampled id sids[r * N + n]
  double* tmass; float* tscale; int64_t ldm;
  const int32_t* dunit; const double* dres; int32_t* sids; int N;
  // the draw pass over the drawn-in tiles only: vocabulary tile vt's rows
  // (launch rows that draw in units 2vt or 2vt + 1) are idx[toff[vt] ..],
  // tcnt[vt] of them; one work-group per tile and 256 of its rows
  const int32_t* tcnt; const int32_t* toff;
  // teacher cache writer: length of each writer's candidate sub-list,
  // scnt[r * scnt_ld + range * 4 + writer]
  int32_t* scnt; int64_t scnt_ld;
};

constexpr int kTeacherWnormGroups = 1024;   // work-groups of the max ||w_v|| pass

// entries per work-group of the teacher writer's large-band scratch (12 bytes each)
__host__ __device__ inline int64_t teacher_scratch_entries(int64_t cap) { return (cap + 1) & ~int64_t(1); }

struct TeacherArgs {
  const char* X; int64_t ldx;         // the chunk's hidden rows (row 0 of the chunk)
  const char* W; int64_t ldw;
  int rows, H, V, K, P;               // P: groups of the pilot (rows of zp)
  const float* zp; int64_t ldp;       // pilot group maxima [P][ldp]
  const double* wmax;                 // max over v of ||w_v||_2
  float* te; double* bnd;             // per row: emission threshold, error bound
  int32_t* cnt; int32_t* cid; float* cz; int64_t cap;
  char* scratch;                      // per work-group: cap x (id, fp64) for large bands
  int32_t* ids_out; char* logits_out; int out_bf16;  // the chunk's rows of the cache
};

struct CombineArgs {
  int S, V, ncu, K;
  const int32_t* idx;                 // compacted -> original row (the per-chunk combine)
  int identity;                       // forward ran over all S rows in order (no row map)
  float T;
  const int32_t* pos; const int32_t* nrows_dev;
  const float* pm; const float* ps;
  const int32_t* ids_s; const float* p_s; const int32_t* korig_s; const float* zs;
  const float* negH;
  float* lse; float* kl_rows; float* z_topk;
  double* block_sums;
  float* loss;
};

struct EntCombineArgs {
  int S, V, ncu;
  const float* em; const double* es; const double* eu;
  double* entropy;                    // or NULL
  double* lse;                        // natural log-normaliser at T = 1, or NULL
};

// Position signals (one wave per position).
struct SignalArgs {
  int64_t S;
  int V, H, K, hw_f32, tl_f32, probs;
  double invT;
  const char* hidden; int64_t ldh;
  const char* W; int64_t ldw;
  const int32_t* labels;              // [S]
  const double* lse;                  // [S] at T = 1 (for ce)
  const int32_t* ids; const void* tl; // teacher rows (for tunc)
  double* ce;                         // [S] or NULL
  double* tunc;                       // [S] or NULL
};

struct DhArgs {
  const char* G; int64_t ldg;         // bf16: the chunk's rows of the blocked gradient
                                      // tiles (ldg = block stride); fp32: [rows, Vp]
  const char* WT; int64_t ldwt;       // W transposed [H, Vp]
  const int32_t* nrows_dev;
  int row_begin, row_cap, V, H, ncu;
  int ks;                             // vocabulary splits (chosen for row_cap rows)
  float* part;                        // [split][row_cap][H] fp32
};

// Floats between the dHidden partials of consecutive splits: rows x H plus
// 64 (256 bytes), so that the partials of one element, summed together by
// the reduction, do not all sit at one offset modulo the HBM channel
// interleave.
__host__ __device__ inline int64_t dh_split_stride(int row_cap, int H) {
  return (int64_t)row_cap * H + 64;
}

struct DhReduceArgs {
  const float* part; const int32_t* idx; const int32_t* nrows_dev;
  int row_begin, row_cap, V, H, ncu, ks;
  float* dH;
};

// dW contracts a group of consecutive chunks at once: chunk k of the group
// occupies token rows [k*slot, k*slot + round_up(rows_k, 8)) of the gradient
// tiles (bf16; token columns of G^T for fp32) and token columns of X_c^T
// (zeros past rows_k), slot = round_up(C, 8).
struct DwArgs {
  const char* G; int64_t ldg;                       // bf16: the group's blocked gradient tiles
                                                    // (ldg = block stride)
  const char* GT; int64_t ldgt; int Vp;             // fp32: the same transposed [Vp, slots]
  const char* XcT; int64_t ldxt;                    // gathered hidden rows transposed [H, slots]
  const int32_t* nrows_dev;
  int group_begin;                                  // first compacted row of the group
  int group_chunks, chunk, slot;                    // chunks in the group, C, round_up(C, 8)
  int V, H, beta_first;
  float* dW;
};

// Teacher term of the gradient tile of one chunk (see kd_sweep.hip).
struct GradTeacherArgs {
  char* G; int64_t ldg;            // bf16: blocked (ldg = block stride); fp32: [rows][Vld]
  char* GT; int64_t ldgt;          // fp32: [Vp][slots], this chunk's slot; bf16: null
  const int32_t* idx;              // compacted row -> original row
  const int32_t* nrows_dev;
  int row_begin, row_cap, K;
  const int32_t* ids_s;            // id-sorted teacher tables
  const float* p_s;
  const float* grad_loss;
  float T;
};

// Comparator loss forms (dense, forward-chunked): per-row passes over the
// stored bf16 logits Z (compacted row cr at Z + cr * ldz) and, for the dense
// form, the fp32 grids P and logQ (row cr at + cr * ldd). Teacher tables, lse
// and kl are indexed by original row; G by launch row r (row_begin + r).
struct CmpRowArgs {
  const uint16_t* Z; int64_t ldz;
  const int32_t* idx; const int32_t* nrows_dev;
  int row_begin, row_cap, V, Vp, K;
  float T;
  const int32_t* ids_s; const float* p_s; const float* negH;
  float* lse; float* kl;
  float* P; float* logQ; int64_t ldd;
  const float* grad_loss;
  uint16_t* G; int64_t ldg;   // the chunk's rows of the blocked gradient tiles (ldg = block
                              // stride, elements)
};
enum CmpRowKind { kCmpKlSparse = 0, kCmpDenseGrid = 1, kCmpKlDense = 2, kCmpGradSparse = 3,
                  kCmpGradDense = 4 };

// ------------------------------------------------------------------ launchers
// Each returns hipSuccess or the launch error.
hipError_t launch_prepass(const int32_t* ids, const void* tl, int tl_f32, int probs, int64_t S,
                          int K, int V, float T, int32_t* ids_s, float* p_s, int32_t* korig_s,
                          float* negH, uint8_t* present, float* z_topk, hipStream_t st);
hipError_t launch_compact(const uint8_t* present, const uint8_t* mask, int64_t S, int32_t* idx,
                          int32_t* pos, int32_t* count, hipStream_t st);
hipError_t launch_sweep(int kind, int f32, int map, const SweepArgs& a, int grid, hipStream_t st);
hipError_t launch_teacher_wnorm(int f32, const char* W, int64_t ldw, int V, int H, double* part,
                                double* wmax, hipStream_t st);
hipError_t launch_teacher_threshold(int f32, const TeacherArgs& a, int32_t* nbig, hipStream_t st);
hipError_t launch_teacher_final(int f32, const TeacherArgs& a, int32_t* big, int32_t* nbig,
                                float* tau2, int grid, int grid_big, hipStream_t st);
hipError_t launch_grad_teacher(int f32, const GradTeacherArgs& a, hipStream_t st);
// teacher cache writer: closes the gaps between the emit pass's sub-lists of
// each of `rows` rows (ns vocabulary ranges x 4 writers) and sets cnt
hipError_t launch_teacher_gather(int32_t* cid, float* cz, int64_t cap, const int32_t* scnt,
                                 int64_t scnt_ld, int ns, int nvt, int rows, int32_t* cnt,
                                 hipStream_t st);
// sampled targets: the uniforms check (flag set when a value is outside [0, 1)
// or a row decreases); the in-place cumulative sum of the unit masses of
// `rows` rows, brought to the row's largest scale (rowmax); the unit and
// residual of each draw of those rows
hipError_t launch_draw_check(const double* u, int64_t S, int N, int32_t* flag, hipStream_t st);
hipError_t launch_draw_cumsum(double* tmass, const float* tscale, int64_t ldm, int nu, int rows,
                              float* rowmax, hipStream_t st);
hipError_t launch_draw_assign(const double* cum, const float* tscale, const float* rowmax,
                              int64_t ldm, int nu, int rows, const double* u, int N,
                              int32_t* dunit, double* dres, int32_t* sids, hipStream_t st);
// the rows of a chunk that draw in each vocabulary tile of 256 entries (units
// 2vt and 2vt + 1): tcnt[vt] rows, listed in tlist[toff[vt] ..] (a row once per
// tile it draws in, in no particular order); tfill is scratch, nvt entries
hipError_t launch_draw_tiles(const int32_t* dunit, int rows, int N, int nvt, int32_t* tcnt,
                             int32_t* toff, int32_t* tfill, int32_t* tlist, hipStream_t st);
int sweep_grid(int64_t rows_max, int V, int ncu);
hipError_t launch_fwd_combine(const CombineArgs& a, hipStream_t st);
// The forward and backward in one call: the forward combine of one chunk's
// launch rows (lse, KL_t into kl_out[t] and z_topk of original row t), the
// loss over every row once all chunks are combined, and the chunk's gradient
// tile from the logits its forward sweep stored (grid: token tiles x
// vocabulary tiles of a full chunk).
hipError_t launch_fwd_combine_chunk(const CombineArgs& a, int row_begin, int row_cap,
                                    float* kl_out, hipStream_t st);
hipError_t launch_fwd_finish(const CombineArgs& a, const float* kl_in, hipStream_t st);
hipError_t launch_zgrad(int f32, const SweepArgs& a, int grid, hipStream_t st);
hipError_t launch_loss_final(const double* block_sums, int nblk, const int32_t* nrows_dev,
                             float* loss, hipStream_t st);
hipError_t launch_cmp_rows(int what, const CmpRowArgs& a, hipStream_t st);
hipError_t launch_cmp_loss(const int32_t* pos, int64_t S, float* lse, float* kl, float* kl_out,
                           double* block_sums, const int32_t* nrows_dev, float* loss,
                           hipStream_t st);
hipError_t launch_ent_combine(const EntCombineArgs& a, hipStream_t st);
hipError_t launch_gather_rows_t(int f32, const char* X, int64_t ldx, const int32_t* idx,
                                const int32_t* nrows_dev, int row_begin, int row_cap, int H,
                                char* out, int64_t ldo, int Cp, char* xc, hipStream_t st);
hipError_t launch_transpose_w(int f32, const char* W, int V, int H, char* WT, int Vp, int ldwt,
                              hipStream_t st);
hipError_t launch_scale(float* x, int64_t n, const float* g, hipStream_t st);
hipError_t launch_zero_invalid_rows(const int32_t* pos, int64_t S, int H, float* dH,
                                    hipStream_t st);
hipError_t launch_dh(int f32, const DhArgs& a, int grid, hipStream_t st);
int dh_grid(int row_cap, int V, int H, int ncu, int f32);
__host__ __device__ int dh_splits(int rows, int V, int H, int ncu, int f32);
hipError_t launch_dh_reduce(const DhReduceArgs& a, hipStream_t st);
hipError_t launch_dw(int f32, const DwArgs& a, hipStream_t st);
hipError_t launch_validate(const int32_t* ids, const void* tl, int tl_f32, int probs, int64_t S,
                           int K, int V, unsigned long long* counters, hipStream_t st);
hipError_t launch_fill_u8(uint8_t* p, uint8_t v, int64_t n, hipStream_t st);
hipError_t launch_validate_order(const int32_t* ids, const void* tl, int tl_f32, int64_t S, int K,
                                 unsigned long long* counters, hipStream_t st);

hipError_t launch_signals(const SignalArgs& a, hipStream_t st);
hipError_t launch_select_segments(const double* x, const int64_t* off, int64_t B, int64_t S,
                                  int64_t num, int64_t den, uint8_t* mask, double* thr,
                                  hipStream_t st);
hipError_t launch_select_above(const double* x, int64_t S, double tau, uint8_t* mask,
                               hipStream_t st);
hipError_t launch_seg_band_count(const double* E, const int64_t* off, int64_t B, const double* thr,
                                 double eps2, int32_t* nband, int32_t* nabove, hipStream_t st);
hipError_t launch_seg_band_list(const double* E, const int64_t* off, int64_t B, const double* thr,
                                double eps2, const int32_t* boff, int32_t* list, hipStream_t st);
hipError_t launch_seg_band_final(int64_t B, const int32_t* boff, const int32_t* nband,
                                 const int32_t* need, const int32_t* list, const double* pent,
                                 uint8_t* mask, hipStream_t st);

// selection
struct SelectWs {
  unsigned long long* keys;   // [S]
  int32_t* band;              // [S] band rows
  double* refined;            // [S] fp64 entropies (or sample means) of band rows, band order
  int32_t* scal;              // small scalars: [0]=n_band [1]=n_above [2]=k
  double* dscal;              // [0]=threshold value
  double* rpart;              // refine partials [cap][nblk][3]
  unsigned int* hist;         // scratch
};
hipError_t launch_select_threshold(const double* entropy, int64_t S, int64_t k, double eps,
                                   const SelectWs& w, hipStream_t st);
hipError_t launch_sample_check(const int64_t* off, int64_t B, int64_t S, int32_t* flag,
                               hipStream_t st);
hipError_t launch_sample_means(const double* E, const int64_t* off, int64_t B, double* means,
                               hipStream_t st);
// sample selection: flag the positions of the band samples; the fp64 mean of
// each band sample's refined entropies (pent[pos[t]]) into w.refined
hipError_t launch_sample_mark(const int64_t* off, const SelectWs& w, int n_band, uint8_t* flag,
                              hipStream_t st);
hipError_t launch_sample_band_means(const int64_t* off, const SelectWs& w, int n_band,
                                    const int32_t* pos, const double* pent, hipStream_t st);
hipError_t launch_sample_refined_entropy(const SelectWs& w, int n, int nblk, double* pent,
                                         hipStream_t st);
hipError_t launch_sample_final(const double* means, int64_t B, int64_t k, const SelectWs& w,
                               int n_band, int refined, uint8_t* mask, int32_t* idx_out,
                               hipStream_t st);
// fp64 refinement partials of band rows [band_off, band_off + band_n) of w.band
// (xb: fp32 rows widened there, at most kRefineBatch of them; bf16 rows are
// read in place and xb is not used)
hipError_t launch_refine(int f32, const char* X, int64_t ldx, const char* W, int64_t ldw, int V,
                         int H, const SelectWs& w, double* xb, int band_off, int band_n, int nblk,
                         hipStream_t st);
// list[i] = floor(i*S/n), i < n; *out = max_i |E[list[i]] - ref[i]| (NaN terms skipped)
hipError_t launch_probe_list(int32_t* list, int n, int64_t S, hipStream_t st);
hipError_t launch_max_abs_diff(const double* E, const int32_t* list, int n, const double* ref,
                               double* out, hipStream_t st);
hipError_t launch_select_final(const double* entropy, int64_t S, int64_t k, const SelectWs& w,
                               int n_band, uint8_t* mask, int32_t* idx_out, hipStream_t st);

}  // namespace kd
