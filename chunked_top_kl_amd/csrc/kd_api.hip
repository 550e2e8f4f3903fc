// C ABI of the fused chunked top-K KL loss: argument checks, workspace plan,
// and the launch sequences of the forward, backward, entropy, selection and
// validation entry points. Declarations and contracts: include/kd_topk_kl.h.
#include "kd_topk_kl.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <limits>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "kd_common.hpp"
#include "kd_kernels.hpp"

namespace {

using kd::ceil_div;
using kd::round_up;

// Work-group scheduling (splits, split-K) is planned for the MI355X's 256
// compute units whatever the device reports, so that workspace sizes are a
// pure function of the problem.
constexpr int kCostCUs = 256;
constexpr int64_t kMaxK = 4096;
constexpr int64_t kMaxRows = int64_t(1) << 30;
constexpr double kSelectEps = 2e-5;    // least bound on |fp32-path entropy - fp64 entropy| (nats)
constexpr int kEpsProbe = 16;           // positions whose entropy error is measured per selection
constexpr int64_t kDwDepth = 8192;     // tokens per dW contraction (a multiple of chunks)
constexpr int kRefineBatch = 256;      // band rows widened to fp64 per refinement launch
constexpr int kRefinePiece = 4096;     // band rows whose fp64 refinement partials are held at once
// refinement work-groups: one vocabulary row per thread, 256 per group
inline int64_t refine_blocks(int64_t V) { return ceil_div(V, 256); }

// ------------------------------------------------------------------ profiling
struct ProfRec {
  const char* name;
  hipEvent_t a, b;
};
// Profiling (kd_profile_*): an opt-in measurement facility, off by default.
// While it is off a launch scope reads one atomic flag and records nothing.
std::mutex g_prof_mu;
std::atomic<bool> g_prof_on{false};
thread_local bool t_prof_off = false;   // set while a call that must not create events runs
std::vector<ProfRec> g_prof_recs;
std::vector<hipEvent_t> g_event_pool;

hipEvent_t pool_event() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

struct Prof {
  hipStream_t st;
  const char* name;
  hipEvent_t a = nullptr, b = nullptr;
  Prof(const char* n, hipStream_t s) : st(s), name(n) {
    if (!g_prof_on.load(std::memory_order_relaxed) || t_prof_off) return;
    std::lock_guard<std::mutex> g(g_prof_mu);
    if (!g_prof_on.load(std::memory_order_relaxed)) return;
    a = pool_event();
    b = pool_event();
    // a scope whose events cannot be recorded is not kept
    if (a && b && hipEventRecord(a, st) != hipSuccess) a = nullptr;
  }
  ~Prof() {
    if (!a || !b) return;
    if (hipEventRecord(b, st) != hipSuccess) return;
    std::lock_guard<std::mutex> g(g_prof_mu);
    g_prof_recs.push_back({name, a, b});
  }
};

// ------------------------------------------------------------------ device check
constexpr int kMaxDevices = 64;

int check_device() {
  static std::mutex mu;
  static signed char ok_by_dev[kMaxDevices];   // 0 not checked yet, 1 gfx950, -1 other
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return KD_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return KD_ERR_HIP;
  std::lock_guard<std::mutex> g(mu);
  if (ok_by_dev[dev] == 0) {
    hipDeviceProp_t p;
    if (hipGetDeviceProperties(&p, dev) != hipSuccess) return KD_ERR_HIP;
    ok_by_dev[dev] = std::strncmp(p.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
  }
  return ok_by_dev[dev] > 0 ? KD_OK : KD_ERR_ARCH;
}

// ------------------------------------------------------------------ workspace plan
struct Layout {
  size_t count, present, pos, idx, ids_s, p_s, korig_s, negH;
  size_t pm, ps, zs, bsum;
  size_t fwd_total;   // the forward uses only the buffers laid out before this offset
  size_t G, GT, WT, XcT, Xc, dhp;   // GT: fp32 only
  size_t em, es, eu;
  size_t band, refined, scal, dscal, rpart, xb, counters;
  size_t smean, spos, pent;
  size_t lse64, segw;
  size_t total;
  int64_t C;          // rows per backward chunk (<= S, >= 1)
  int64_t Vp;         // vocabulary columns of the gradient tile: round_up(V, 8)
  int64_t Vld;        // row pitch (elements) of W^T (and of fp32's G): an odd multiple of 128 bytes,
                      // so that the 256 rows of an operand tile spread over all
                      // 128-byte offsets modulo 4 KB (L2 channels)
  int64_t slot;       // token rows (columns, transposed) of one chunk in a dW group: round_up(C, 8)
  int64_t nd;         // chunks per dW contraction (group)
  int64_t Cp;         // token columns of X_c^T (and fp32's G^T): nd slots rounded to 32
  int64_t Cld;        // their row pitch in elements: Cp plus 128 bytes, so that the
                      // 256 rows of a dW operand tile do not share one offset
                      // modulo a large power of two (L2 channel conflicts)
  int64_t esz;
  int64_t Gbs;        // bf16: bytes between the column blocks of the gradient tiles
  int ks;             // dHidden vocabulary splits
};

Layout plan(const kd_problem* p) {
  Layout L;
  std::memset(&L, 0, sizeof(L));
  const int64_t S = p->S, H = p->H, V = p->V, K = p->K;
  L.esz = p->hw_dtype == KD_F32 ? 4 : 2;
  L.C = p->chunk < S ? p->chunk : (S > 0 ? S : 1);
  L.Vp = round_up(V, 8);
  {
    int64_t b = round_up(L.Vp * L.esz, 128);
    if ((b / 128) % 2 == 0) b += 128;
    L.Vld = b / L.esz;
  }
  L.slot = round_up(L.C, 8);
  {
    // dW contracts about kDwDepth tokens per launch: its fp32 read-modify-write
    // of dW is paid once per group instead of once per chunk
    const int64_t nch = S > 0 ? ceil_div(S, L.C) : 1;
    int64_t nd = kDwDepth / L.slot;
    if (nd < 1) nd = 1;
    if (nd > nch) nd = nch;
    L.nd = nd;
  }
  L.Cp = round_up(L.nd * L.slot, 32);
  L.Cld = L.Cp + 128 / L.esz;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (size_t)round_up((int64_t)bytes, 256);
    return o;
  };
  const int64_t Sx = S > 0 ? S : 1;
  L.count = take(64 * 4);
  L.present = take(Sx);
  L.pos = take(Sx * 4);
  L.idx = take(Sx * 4);
  L.ids_s = take(Sx * K * 4);
  L.p_s = take(Sx * K * 4);
  L.korig_s = take(Sx * K * 4);
  L.negH = take(Sx * 4);
  const int64_t pe = (int64_t)kd::sweep_grid(Sx, (int)V, kCostCUs) * kd::kTile;
  L.pm = take(pe * 4);
  L.ps = take(pe * 4);
  L.zs = take(Sx * K * 4);
  L.bsum = take((ceil_div(Sx, 256) + 1) * 8);
  L.fwd_total = off;
  if (L.esz == 2) {
    // bf16: the gradient tiles of a whole dW group (slot s at rows
    // [s * slot, s * slot + slot)) in blocks of 256 vocabulary columns, rows
    // 512 bytes apart inside a block; dW reads them as they are
    L.Gbs = L.nd * L.slot * 512;
    L.G = take(ceil_div(L.Vp, 256) * L.Gbs);
    L.GT = off;   // no transposed copy
  } else {
    // fp32: one chunk's tile, and the group's tiles transposed for dW
    L.G = take(L.C * L.Vld * L.esz);
    L.GT = take(L.Vp * L.Cld * L.esz);
  }
  L.WT = take(H * L.Vld * L.esz);
  L.XcT = take(H * L.Cld * L.esz);
  L.Xc = take(L.C * H * L.esz);
  // dHidden: vocabulary splits chosen for a full chunk, used for every chunk
  L.ks = kd::dh_splits((int)L.C, (int)V, (int)H, kCostCUs, p->hw_dtype == KD_F32);
  L.dhp = take((size_t)L.ks * kd::dh_split_stride((int)L.C, (int)H) * 4);
  L.em = take(pe * 4);
  L.es = take(pe * 8);
  L.eu = take(pe * 8);
  L.band = take((Sx + kEpsProbe) * 4);     // band list, then the error probe's positions
  L.refined = take((Sx + kEpsProbe) * 8);
  L.scal = take(16 * 4);
  L.dscal = take(16 * 8);
  L.rpart = take((size_t)kRefinePiece * refine_blocks(V) * 3 * 8);
  L.xb = take((size_t)kRefineBatch * H * 8);
  L.counters = take(4 * 8);
  L.smean = take(Sx * 8);
  L.spos = take((Sx + kEpsProbe) * 4);
  L.pent = take((Sx + kEpsProbe) * 8);
  L.lse64 = take(Sx * 8);
  L.segw = take(Sx * 4 * 4);
  L.total = off;
  return L;
}

// ------------------------------------------------------------------ problem checks
int check_problem(const kd_problem* p) {
  if (!p) return KD_ERR_NULL;
  if (p->hw_dtype != KD_BF16 && p->hw_dtype != KD_F32) return KD_ERR_DTYPE;
  if (p->tl_dtype != KD_BF16 && p->tl_dtype != KD_F32) return KD_ERR_DTYPE;
  if (p->tl_kind != KD_TEACHER_LOGITS && p->tl_kind != KD_TEACHER_PROBS) return KD_ERR_ARG;
  if (p->S < 0 || p->S > kMaxRows) return KD_ERR_SHAPE;
  if (p->H <= 0 || p->V <= 0 || p->K <= 0) return KD_ERR_SHAPE;
  if (p->K > p->V || p->K > kMaxK) return KD_ERR_SHAPE;
  if (p->H % 8 != 0 || p->H > (int64_t(1) << 20)) return KD_ERR_SHAPE;
  if (p->V > (int64_t(1) << 30)) return KD_ERR_SHAPE;
  if (!(p->temperature > 0.0f) || !std::isfinite(p->temperature)) return KD_ERR_TEMPERATURE;
  if (p->chunk <= 0) return KD_ERR_CHUNK;
  // every operand tile of the contractions (256 rows of the widest pitch, the
  // gradient tile and W^T rows or the transposed chunk rows) must lie in one
  // buffer range, whose size is below 2^31 bytes
  const Layout L = plan(p);
  if (256 * L.Vld * L.esz >= (int64_t(1) << 31) || 256 * L.Cld * L.esz >= (int64_t(1) << 31))
    return KD_ERR_SHAPE;
  return KD_OK;
}

template <typename T>
T* at(void* ws, size_t off) {
  return (T*)((char*)ws + off);
}

int check_ws(const Layout& L, void* ws, size_t ws_bytes) {
  if (!ws || ((uintptr_t)ws & 255u) != 0 || ws_bytes < L.total) return KD_ERR_WORKSPACE;
  return KD_OK;
}

#define KD_HIP(x)                              \
  do {                                         \
    if ((x) != hipSuccess) return KD_ERR_HIP;  \
  } while (0)

// teacher prepass + compaction, shared by fwd and bwd
int teacher_tables(const kd_problem* p, const Layout& L, const int32_t* ids, const void* tl,
                   const uint8_t* mask, float* z_topk, void* ws, hipStream_t st) {
  {
    Prof pr("prepass", st);
    KD_HIP(kd::launch_prepass(ids, tl, p->tl_dtype == KD_F32, p->tl_kind == KD_TEACHER_PROBS,
                              p->S, (int)p->K, (int)p->V,
                              p->temperature, at<int32_t>(ws, L.ids_s), at<float>(ws, L.p_s),
                              at<int32_t>(ws, L.korig_s), at<float>(ws, L.negH),
                              at<uint8_t>(ws, L.present), z_topk, st));
  }
  {
    Prof pr("compact", st);
    KD_HIP(kd::launch_compact(at<uint8_t>(ws, L.present), mask, p->S, at<int32_t>(ws, L.idx),
                              at<int32_t>(ws, L.pos), at<int32_t>(ws, L.count), st));
  }
  return KD_OK;
}

}  // namespace

extern "C" {

int kd_abi_version(void) { return KD_ABI_VERSION; }

const char* kd_status_str(int s) {
  switch (s) {
    case KD_OK: return "KD_OK: success";
    case KD_ERR_NULL: return "KD_ERR_NULL: a required pointer is NULL";
    case KD_ERR_SHAPE: return "KD_ERR_SHAPE: invalid problem sizes";
    case KD_ERR_DTYPE: return "KD_ERR_DTYPE: unknown dtype code";
    case KD_ERR_TEMPERATURE: return "KD_ERR_TEMPERATURE: temperature must be finite and > 0";
    case KD_ERR_CHUNK: return "KD_ERR_CHUNK: chunk must be > 0";
    case KD_ERR_WORKSPACE: return "KD_ERR_WORKSPACE: workspace NULL, misaligned or too small";
    case KD_ERR_BAD_ID: return "KD_ERR_BAD_ID: teacher id outside [0, V)";
    case KD_ERR_HIP: return "KD_ERR_HIP: HIP runtime or launch failure";
    case KD_ERR_ARCH: return "KD_ERR_ARCH: current device is not gfx950";
    case KD_ERR_ARG: return "KD_ERR_ARG: invalid argument";
    default: return "unknown kd_status";
  }
}

size_t kd_topk_kl_workspace_bytes(const kd_problem* p) {
  if (check_problem(p) != KD_OK) return 0;
  return plan(p).total;
}

}  // extern "C"

namespace {

// The forward's launches, with its buffers at the plan's offsets in ws (only
// those before L.fwd_total are touched). Arguments are checked by the caller.
int fwd_run(const kd_problem* p, const Layout& L, const void* hidden, const void* W,
            const int32_t* ids, const void* tl, const uint8_t* mask, float* loss, float* lse,
            float* kl_rows, float* z_topk, void* ws, hipStream_t st) {
  int rc;
  if ((rc = teacher_tables(p, L, ids, tl, mask, z_topk, ws, st))) return rc;
  const int S = (int)p->S, V = (int)p->V, H = (int)p->H, K = (int)p->K;
  const int f32 = p->hw_dtype == KD_F32;
  if (S > 0) {
    kd::SweepArgs a;
    std::memset(&a, 0, sizeof(a));
    a.W = (const char*)W;
    a.ldw = (int64_t)H * L.esz;
    a.X = (const char*)hidden;
    a.ldx = (int64_t)H * L.esz;
    a.x_row0 = 0;
    const bool map = mask != nullptr;
    a.idx = map ? at<int32_t>(ws, L.idx) : nullptr;
    a.nrows_dev = map ? at<int32_t>(ws, L.count) : nullptr;
    a.row_begin = 0;
    a.row_cap = S;
    a.V = V;
    a.H = H;
    a.K = K;
    a.ncu = kCostCUs;
    a.T = p->temperature;
    a.ids_s = at<int32_t>(ws, L.ids_s);
    a.p_s = at<float>(ws, L.p_s);
    a.korig_s = at<int32_t>(ws, L.korig_s);
    a.pm = at<float>(ws, L.pm);
    a.ps = at<float>(ws, L.ps);
    a.zs = at<float>(ws, L.zs);
    Prof pr("fwd_lse_gather", st);
    KD_HIP(kd::launch_sweep(kd::kSweepFwd, f32, map, a, kd::sweep_grid(S, V, kCostCUs), st));
  }
  kd::CombineArgs c;
  std::memset(&c, 0, sizeof(c));
  c.S = S;
  c.V = V;
  c.ncu = kCostCUs;
  c.K = K;
  c.identity = mask == nullptr;
  c.T = p->temperature;
  c.pos = at<int32_t>(ws, L.pos);
  c.nrows_dev = at<int32_t>(ws, L.count);
  c.pm = at<float>(ws, L.pm);
  c.ps = at<float>(ws, L.ps);
  c.ids_s = at<int32_t>(ws, L.ids_s);
  c.p_s = at<float>(ws, L.p_s);
  c.korig_s = at<int32_t>(ws, L.korig_s);
  c.zs = at<float>(ws, L.zs);
  c.negH = at<float>(ws, L.negH);
  c.lse = lse;
  c.kl_rows = kl_rows;
  c.z_topk = z_topk;
  c.block_sums = at<double>(ws, L.bsum);
  c.loss = loss;
  {
    Prof pr("fwd_combine", st);
    KD_HIP(kd::launch_fwd_combine(c, st));
  }
  return KD_OK;
}

int fwd_check(const kd_problem* p, const void* hidden, const void* W, const int32_t* ids,
              const void* tl, const float* loss, const float* lse) {
  int rc = check_problem(p);
  if (rc) return rc;
  if (!W || !loss || (p->S > 0 && (!hidden || !ids || !tl || !lse))) return KD_ERR_NULL;
  return KD_OK;
}

}  // namespace

// Scratch of kd_topk_kl_fwd_noalloc: a fixed device array, one copy on each
// GPU the library runs on, held until the process ends. In host code its name
// stands for no device address: kernels and copies get the address that
// hipGetSymbolAddress returns for the current device, taken once per device.
static __device__ __attribute__((aligned(256))) char scratch[KD_NOALLOC_SCRATCH_BYTES];

namespace {

std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices];

int scratch_of_current_device(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return KD_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return KD_ERR_HIP;
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return KD_ERR_HIP;
    g_scratch_dev[dev] = ptr;
  }
  *out = g_scratch_dev[dev];
  return KD_OK;
}

struct NoProfile {
  NoProfile() { t_prof_off = true; }
  ~NoProfile() { t_prof_off = false; }
};

}  // namespace

extern "C" {

int kd_topk_kl_fwd(const kd_problem* p, const void* hidden, const void* W, const int32_t* ids,
                   const void* tl, const uint8_t* mask, float* loss, float* lse, float* kl_rows,
                   float* z_topk, void* ws, size_t ws_bytes, void* stream) {
  int rc = fwd_check(p, hidden, W, ids, tl, loss, lse);
  if (rc) return rc;
  const Layout L = plan(p);
  if ((rc = check_ws(L, ws, ws_bytes))) return rc;
  if ((rc = check_device())) return rc;
  return fwd_run(p, L, hidden, W, ids, tl, mask, loss, lse, kl_rows, z_topk, ws,
                 (hipStream_t)stream);
}

int kd_topk_kl_fwd_noalloc(const kd_problem* p, const void* hidden, const void* W,
                           const int32_t* ids, const void* tl, const uint8_t* mask, float* loss,
                           float* lse, float* kl_rows, float* z_topk, void* stream) {
  int rc = fwd_check(p, hidden, W, ids, tl, loss, lse);
  if (rc) return rc;
  const Layout L = plan(p);
  if (L.fwd_total > (size_t)KD_NOALLOC_SCRATCH_BYTES) return KD_ERR_WORKSPACE;
  if ((rc = check_device())) return rc;
  void* ws = nullptr;
  if ((rc = scratch_of_current_device(&ws))) return rc;
  NoProfile np;
  return fwd_run(p, L, hidden, W, ids, tl, mask, loss, lse, kl_rows, z_topk, ws,
                 (hipStream_t)stream);
}

}  // extern "C"

namespace {

// Where the backward's logit gradient of a chunk comes from: the fused path
// projects the chunk again (gradient tile sweep and teacher scatter); the
// comparator forms read it from the grids their forward stored.
struct CmpGrids {
  int form;                  // KD_FORM_FUSED, KD_FORM_DENSE or KD_FORM_FORWARD_CHUNKED
  const uint16_t* Z; int64_t ldz;
  float* P; float* logQ; int64_t ldd;
};

int bwd_check(const kd_problem* p, const void* hidden, const void* W, const int32_t* ids,
              const void* tl, const float* lse, const float* grad_loss, const float* dhidden,
              const float* dW, int accumulate_dW) {
  int rc = check_problem(p);
  if (rc) return rc;
  if (!W || !dW || !grad_loss || (p->S > 0 && (!hidden || !ids || !tl || !lse || !dhidden)))
    return KD_ERR_NULL;
  if (accumulate_dW != 0 && accumulate_dW != 1) return KD_ERR_ARG;
  return KD_OK;
}

// Chunk ci's rows, gathered in order into Xc (for its sweep) and transposed
// into its slot of X_c^T (for the dW contraction).
int gather_chunk_rows(const kd_problem* p, const Layout& L, const void* hidden, int ci, void* ws,
                      hipStream_t st) {
  const int H = (int)p->H, C = (int)L.C;
  const int slot = (int)(ci % L.nd);
  Prof pr("gather_rows_t", st);
  KD_HIP(kd::launch_gather_rows_t(p->hw_dtype == KD_F32, (const char*)hidden, (int64_t)H * L.esz,
                                  at<int32_t>(ws, L.idx), at<int32_t>(ws, L.count), ci * C, C, H,
                                  at<char>(ws, L.XcT) + slot * L.slot * L.esz, L.Cld * L.esz,
                                  (int)L.slot, at<char>(ws, L.Xc), st));
  return KD_OK;
}

// Sweep arguments over chunk ci's gathered rows, with its gradient tile: its
// slot of the dW group, blocked (bf16: ldg is the block stride), or the one
// row-major tile (fp32: ldg is the row pitch) and its slot of G^T.
kd::SweepArgs chunk_sweep_args(const kd_problem* p, const Layout& L, const void* W, int ci,
                               const float* lse, const float* grad_loss, void* ws) {
  const int f32 = p->hw_dtype == KD_F32;
  const int slot = (int)(ci % L.nd);
  const int64_t row_bytes = p->H * L.esz;
  kd::SweepArgs a;
  std::memset(&a, 0, sizeof(a));
  a.W = (const char*)W;
  a.ldw = row_bytes;
  a.X = at<char>(ws, L.Xc);
  a.ldx = row_bytes;
  a.x_row0 = 0;
  a.idx = at<int32_t>(ws, L.idx);
  a.nrows_dev = at<int32_t>(ws, L.count);
  a.row_begin = ci * (int)L.C;
  a.row_cap = (int)L.C;
  a.V = (int)p->V;
  a.H = (int)p->H;
  a.K = (int)p->K;
  a.ncu = kCostCUs;
  a.T = p->temperature;
  a.ids_s = at<int32_t>(ws, L.ids_s);
  a.p_s = at<float>(ws, L.p_s);
  a.korig_s = at<int32_t>(ws, L.korig_s);
  a.lse = lse;
  a.grad_loss = grad_loss;
  a.G = at<char>(ws, L.G) + (f32 ? 0 : (int64_t)slot * L.slot * 512);
  a.ldg = f32 ? L.Vld * L.esz : L.Gbs;
  a.GT = f32 ? at<char>(ws, L.GT) + slot * L.slot * L.esz : nullptr;
  a.ldgt = L.Cld * L.esz;
  return a;
}

// Teacher term of a chunk's gradient tile, after the tile itself (a: the
// tile's sweep arguments).
int grad_teacher(const kd_problem* p, const Layout& L, const kd::SweepArgs& a, int row_begin,
                 const float* grad_loss, void* ws, hipStream_t st) {
  (void)ws;
  kd::GradTeacherArgs gt;
  gt.G = a.G;
  gt.ldg = a.ldg;
  gt.GT = a.GT;
  gt.ldgt = a.ldgt;
  gt.idx = a.idx;
  gt.nrows_dev = a.nrows_dev;
  gt.row_begin = row_begin;
  gt.row_cap = (int)L.C;
  gt.K = (int)p->K;
  gt.ids_s = a.ids_s;
  gt.p_s = a.p_s;
  gt.grad_loss = grad_loss;
  gt.T = p->temperature;
  Prof pr("bwd_grad_teacher", st);
  KD_HIP(kd::launch_grad_teacher(p->hw_dtype == KD_F32, gt, st));
  return KD_OK;
}

// dHidden of chunk ci from its gradient tile Gc, and dW once the chunk closes
// a dW group (or is the last chunk; with no rows that launch still writes dW,
// zeros unless accumulating).
int chunk_contractions(const kd_problem* p, const Layout& L, char* Gc, int64_t ldg, int ci,
                       int nchunks, float* dhidden, float* dW, int accumulate_dW, void* ws,
                       hipStream_t st) {
  const int S = (int)p->S, V = (int)p->V, H = (int)p->H;
  const int f32 = p->hw_dtype == KD_F32;
  const int C = (int)L.C;
  const int row_begin = ci * C;
  const int slot = (int)(ci % L.nd);
  if (S > 0) {
    kd::DhArgs d;
    d.G = Gc;
    d.ldg = ldg;
    d.WT = at<char>(ws, L.WT);
    d.ldwt = L.Vld * L.esz;
    d.nrows_dev = at<int32_t>(ws, L.count);
    d.row_begin = row_begin;
    d.row_cap = C;
    d.V = V;
    d.H = H;
    d.ncu = kCostCUs;
    d.ks = L.ks;
    d.part = at<float>(ws, L.dhp);
    {
      Prof pr("bwd_dhidden", st);
      KD_HIP(kd::launch_dh(f32, d, kd::dh_grid(C, V, H, kCostCUs, f32), st));
    }
    kd::DhReduceArgs r;
    r.ks = L.ks;
    r.part = at<float>(ws, L.dhp);
    r.idx = at<int32_t>(ws, L.idx);
    r.nrows_dev = at<int32_t>(ws, L.count);
    r.row_begin = row_begin;
    r.row_cap = C;
    r.V = V;
    r.H = H;
    r.ncu = kCostCUs;
    r.dH = dhidden;
    Prof pr("bwd_dhidden_reduce", st);
    KD_HIP(kd::launch_dh_reduce(r, st));
  }
  if (slot == L.nd - 1 || ci == nchunks - 1) {
    kd::DwArgs w;
    w.G = at<char>(ws, L.G);
    w.ldg = L.Gbs;
    w.GT = f32 ? at<char>(ws, L.GT) : nullptr;
    w.ldgt = L.Cld * L.esz;
    w.Vp = (int)L.Vp;
    w.XcT = at<char>(ws, L.XcT);
    w.ldxt = L.Cld * L.esz;
    w.nrows_dev = at<int32_t>(ws, L.count);
    w.group_begin = (ci - slot) * C;
    w.group_chunks = slot + 1;
    w.chunk = C;
    w.slot = (int)L.slot;
    w.V = V;
    w.H = H;
    w.beta_first = accumulate_dW;
    w.dW = dW;
    Prof pr("bwd_dw", st);
    KD_HIP(kd::launch_dw(f32, w, st));
  }
  return KD_OK;
}

int bwd_run(const kd_problem* p, const Layout& L, const CmpGrids& cg, const void* hidden,
            const void* W, const int32_t* ids, const void* tl, const uint8_t* mask,
            const float* lse, const float* grad_loss, float* dhidden, float* dW,
            int accumulate_dW, void* ws, hipStream_t st) {
  int rc;
  if ((rc = teacher_tables(p, L, ids, tl, mask, nullptr, ws, st))) return rc;
  const int S = (int)p->S, V = (int)p->V, H = (int)p->H, K = (int)p->K;
  const int f32 = p->hw_dtype == KD_F32;
  const int C = (int)L.C;
  if (S > 0) {
    Prof pr("zero_rows", st);
    KD_HIP(kd::launch_zero_invalid_rows(at<int32_t>(ws, L.pos), S, H, dhidden, st));
  }
  const int nchunks = S > 0 ? (int)ceil_div(S, C) : 1;
  const int sgrid = kd::sweep_grid(C, V, kCostCUs);
  const int Vp = (int)L.Vp;
  if (S > 0) {
    Prof pr("transpose_w", st);
    KD_HIP(kd::launch_transpose_w(f32, (const char*)W, V, H, at<char>(ws, L.WT), Vp, (int)L.Vld,
                                  st));
  }
  for (int ci = 0; ci < nchunks; ++ci) {
    const int row_begin = ci * C;
    const int slot = (int)(ci % L.nd);   // this chunk's columns in the dW group
    // this chunk's gradient tile: its slot of the group, blocked (bf16: ldg is
    // the block stride), or the one row-major tile (fp32: ldg is the row pitch)
    char* Gc = at<char>(ws, L.G) + (f32 ? 0 : (int64_t)slot * L.slot * 512);
    const int64_t ldg = f32 ? L.Vld * L.esz : L.Gbs;
    if (S > 0 && (rc = gather_chunk_rows(p, L, hidden, ci, ws, st))) return rc;
    if (S > 0 && cg.form != KD_FORM_FUSED) {
      // the chunk's logit gradient from the stored grids, then its transpose
      kd::CmpRowArgs ra;
      std::memset(&ra, 0, sizeof(ra));
      ra.Z = cg.Z;
      ra.ldz = cg.ldz;
      ra.idx = at<int32_t>(ws, L.idx);
      ra.nrows_dev = at<int32_t>(ws, L.count);
      ra.row_begin = row_begin;
      ra.row_cap = C;
      ra.V = V;
      ra.Vp = Vp;
      ra.K = K;
      ra.T = p->temperature;
      ra.ids_s = at<int32_t>(ws, L.ids_s);
      ra.p_s = at<float>(ws, L.p_s);
      ra.lse = const_cast<float*>(lse);
      ra.P = cg.P;
      ra.logQ = cg.logQ;
      ra.ldd = cg.ldd;
      ra.grad_loss = grad_loss;
      ra.G = (uint16_t*)Gc;
      ra.ldg = ldg / 2;
      Prof pr("cmp_grad", st);
      KD_HIP(kd::launch_cmp_rows(cg.form == KD_FORM_DENSE ? kd::kCmpGradDense
                                                          : kd::kCmpGradSparse, ra, st));
    } else if (S > 0) {
      const kd::SweepArgs a = chunk_sweep_args(p, L, W, ci, lse, grad_loss, ws);
      {
        Prof pr("bwd_grad_tile", st);
        KD_HIP(kd::launch_sweep(kd::kSweepBwdG, f32, 0, a, sgrid, st));
      }
      if ((rc = grad_teacher(p, L, a, row_begin, grad_loss, ws, st))) return rc;
    }
    if ((rc = chunk_contractions(p, L, Gc, ldg, ci, nchunks, dhidden, dW, accumulate_dW, ws,
                                 st)))
      return rc;
  }
  return KD_OK;
}

// ------------------------------------------------------------------ forward and backward in one call
// The workspace of the one-call path: the two-call plan, then one chunk's
// logits (fp32, as the sweep's lanes hold them) and KL_t of every row.
struct FbLayout {
  size_t Z, kl, total;
};

FbLayout plan_fb(const kd_problem* p, const Layout& L) {
  FbLayout F;
  size_t off = L.total;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (size_t)round_up((int64_t)bytes, 256);
    return o;
  };
  F.Z = take((size_t)ceil_div(L.C, kd::kTile) * ceil_div(p->V, kd::kTile) * kd::kZTile * 4);
  F.kl = take((size_t)(p->S > 0 ? p->S : 1) * 4);
  F.total = off;
  return F;
}

// Per chunk: its rows gathered; one sweep gives the partials of its rows'
// log-normalisers and the logits at their teacher ids, and stores every
// logit; the chunk's combine gives lse and KL_t; the gradient tile is formed
// from the stored logits (no second projection); then the teacher term,
// dHidden and, at the end of a dW group, dW. The loss is formed once every
// row's KL_t is known.
int fwd_bwd_run(const kd_problem* p, const Layout& L, const FbLayout& F, const void* hidden,
                const void* W, const int32_t* ids, const void* tl, const uint8_t* mask,
                const float* grad_loss, float* loss, float* lse, float* kl_rows, float* z_topk,
                float* dhidden, float* dW, int accumulate_dW, void* ws, hipStream_t st) {
  int rc;
  if ((rc = teacher_tables(p, L, ids, tl, mask, z_topk, ws, st))) return rc;
  const int S = (int)p->S, V = (int)p->V, H = (int)p->H, K = (int)p->K;
  const int C = (int)L.C;
  const int f32 = p->hw_dtype == KD_F32;
  if (S > 0) {
    {
      Prof pr("zero_rows", st);
      KD_HIP(kd::launch_zero_invalid_rows(at<int32_t>(ws, L.pos), S, H, dhidden, st));
    }
    Prof pr("transpose_w", st);
    KD_HIP(kd::launch_transpose_w(f32, (const char*)W, V, H, at<char>(ws, L.WT), (int)L.Vp,
                                  (int)L.Vld, st));
  }
  float* klbuf = kl_rows ? kl_rows : at<float>(ws, F.kl);
  kd::CombineArgs c;
  std::memset(&c, 0, sizeof(c));
  c.S = S;
  c.V = V;
  c.ncu = kCostCUs;
  c.K = K;
  c.idx = at<int32_t>(ws, L.idx);
  c.T = p->temperature;
  c.pos = at<int32_t>(ws, L.pos);
  c.nrows_dev = at<int32_t>(ws, L.count);
  c.pm = at<float>(ws, L.pm);
  c.ps = at<float>(ws, L.ps);
  c.ids_s = at<int32_t>(ws, L.ids_s);
  c.p_s = at<float>(ws, L.p_s);
  c.korig_s = at<int32_t>(ws, L.korig_s);
  c.zs = at<float>(ws, L.zs);
  c.negH = at<float>(ws, L.negH);
  c.lse = lse;
  c.kl_rows = kl_rows;
  c.z_topk = z_topk;
  c.block_sums = at<double>(ws, L.bsum);
  c.loss = loss;
  const int nchunks = S > 0 ? (int)ceil_div(S, C) : 1;
  const int sgrid = kd::sweep_grid(C, V, kCostCUs);
  const int zgrid = (int)(ceil_div(C, kd::kTile) * ceil_div(V, kd::kTile));
  for (int ci = 0; ci < nchunks; ++ci) {
    const int row_begin = ci * C;
    kd::SweepArgs a = chunk_sweep_args(p, L, W, ci, lse, grad_loss, ws);
    if (S > 0) {
      if ((rc = gather_chunk_rows(p, L, hidden, ci, ws, st))) return rc;
      a.pm = at<float>(ws, L.pm);
      a.ps = at<float>(ws, L.ps);
      a.zs = at<float>(ws, L.zs);
      a.Zt = at<float>(ws, F.Z);
      {
        Prof pr("fwd_lse_gather_keep", st);
        KD_HIP(kd::launch_sweep(kd::kSweepFwdZ, f32, 0, a, sgrid, st));
      }
      {
        Prof pr("fwd_combine", st);
        KD_HIP(kd::launch_fwd_combine_chunk(c, row_begin, C, klbuf, st));
      }
      {
        Prof pr("grad_tile_from_logits", st);
        KD_HIP(kd::launch_zgrad(f32, a, zgrid, st));
      }
      if ((rc = grad_teacher(p, L, a, row_begin, grad_loss, ws, st))) return rc;
    }
    if ((rc = chunk_contractions(p, L, a.G, a.ldg, ci, nchunks, dhidden, dW, accumulate_dW, ws,
                                 st)))
      return rc;
  }
  Prof pr("fwd_finish", st);
  KD_HIP(kd::launch_fwd_finish(c, klbuf, st));
  return KD_OK;
}

}  // namespace

extern "C" {

int kd_topk_kl_bwd(const kd_problem* p, const void* hidden, const void* W, const int32_t* ids,
                   const void* tl, const uint8_t* mask, const float* lse, const float* grad_loss,
                   float* dhidden, float* dW, int accumulate_dW, void* ws, size_t ws_bytes,
                   void* stream) {
  int rc = bwd_check(p, hidden, W, ids, tl, lse, grad_loss, dhidden, dW, accumulate_dW);
  if (rc) return rc;
  const Layout L = plan(p);
  if ((rc = check_ws(L, ws, ws_bytes))) return rc;
  if ((rc = check_device())) return rc;
  CmpGrids cg;
  std::memset(&cg, 0, sizeof(cg));
  cg.form = KD_FORM_FUSED;
  return bwd_run(p, L, cg, hidden, W, ids, tl, mask, lse, grad_loss, dhidden, dW, accumulate_dW,
                 ws, (hipStream_t)stream);
}

size_t kd_topk_kl_fwd_bwd_workspace_bytes(const kd_problem* p) {
  if (check_problem(p) != KD_OK) return 0;
  return plan_fb(p, plan(p)).total;
}

int kd_topk_kl_fwd_bwd(const kd_problem* p, const void* hidden, const void* W, const int32_t* ids,
                       const void* tl, const uint8_t* mask, const float* grad_loss, float* loss,
                       float* lse, float* kl_rows, float* z_topk, float* dhidden, float* dW,
                       int accumulate_dW, void* ws, size_t ws_bytes, void* stream) {
  int rc = fwd_check(p, hidden, W, ids, tl, loss, lse);
  if (rc) return rc;
  if ((rc = bwd_check(p, hidden, W, ids, tl, lse, grad_loss, dhidden, dW, accumulate_dW)))
    return rc;
  const Layout L = plan(p);
  const FbLayout F = plan_fb(p, L);
  if (!ws || ((uintptr_t)ws & 255u) != 0 || ws_bytes < F.total) return KD_ERR_WORKSPACE;
  if ((rc = check_device())) return rc;
  return fwd_bwd_run(p, L, F, hidden, W, ids, tl, mask, grad_loss, loss, lse, kl_rows, z_topk,
                     dhidden, dW, accumulate_dW, ws, (hipStream_t)stream);
}

int kd_scale_f32(float* x, int64_t n, const float* g, void* stream) {
  if (n < 0) return KD_ERR_SHAPE;
  if (n > 0 && (!x || !g)) return KD_ERR_NULL;
  if (n == 0) return KD_OK;
  int rc;
  if ((rc = check_device())) return rc;
  Prof pr("scale_grads", (hipStream_t)stream);
  KD_HIP(kd::launch_scale(x, n, g, (hipStream_t)stream));
  return KD_OK;
}

}  // extern "C"

namespace {

// Workspace of the comparator forms: the fused layout (teacher tables, the
// chunk's gradient tile and its transpose, W^T, dHidden partials), then the
// stored grids: the bf16 logits of every row (both forms) and, for the dense
// form, the fp32 teacher grid P and log-probabilities logQ of every row.
struct CmpLayout {
  size_t Z, kl, P, logQ, total;
  int64_t ldz, ldd;   // row pitches in elements
};

CmpLayout plan_cmp(const kd_problem* p, int form, const Layout& L) {
  CmpLayout c;
  std::memset(&c, 0, sizeof(c));
  const int64_t Sx = p->S > 0 ? p->S : 1;
  size_t off = L.total;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (size_t)round_up((int64_t)bytes, 256);
    return o;
  };
  c.ldz = L.Vld;
  c.Z = take((size_t)Sx * c.ldz * 2);
  c.kl = take((size_t)Sx * 4);
  if (form == KD_FORM_DENSE) {
    c.ldd = L.Vld;
    c.P = take((size_t)Sx * c.ldd * 4);
    c.logQ = take((size_t)Sx * c.ldd * 4);
  }
  c.total = off;
  return c;
}

int cmp_check(const kd_problem* p, int form) {
  int rc = check_problem(p);
  if (rc) return rc;
  if (form != KD_FORM_DENSE && form != KD_FORM_FORWARD_CHUNKED) return KD_ERR_ARG;
  if (p->hw_dtype != KD_BF16) return KD_ERR_DTYPE;
  return KD_OK;
}

CmpGrids cmp_grids(const kd_problem* p, int form, const CmpLayout& c, void* ws) {
  (void)p;
  CmpGrids g;
  std::memset(&g, 0, sizeof(g));
  g.form = form;
  g.Z = at<uint16_t>(ws, c.Z);
  g.ldz = c.ldz;
  if (form == KD_FORM_DENSE) {
    g.P = at<float>(ws, c.P);
    g.logQ = at<float>(ws, c.logQ);
    g.ldd = c.ldd;
  }
  return g;
}

}  // namespace

extern "C" {

size_t kd_kl_comparator_workspace_bytes(const kd_problem* p, int form) {
  if (cmp_check(p, form) != KD_OK) return 0;
  const Layout L = plan(p);
  return plan_cmp(p, form, L).total;
}

int kd_kl_comparator_fwd(const kd_problem* p, int form, const void* hidden, const void* W,
                         const int32_t* ids, const void* tl, const uint8_t* mask, float* loss,
                         float* lse, float* kl_rows, void* ws, size_t ws_bytes, void* stream) {
  int rc = cmp_check(p, form);
  if (rc) return rc;
  if ((rc = fwd_check(p, hidden, W, ids, tl, loss, lse))) return rc;
  const Layout L = plan(p);
  const CmpLayout CL = plan_cmp(p, form, L);
  if (!ws || ((uintptr_t)ws & 255u) != 0 || ws_bytes < CL.total) return KD_ERR_WORKSPACE;
  if ((rc = check_device())) return rc;
  hipStream_t st = (hipStream_t)stream;
  if ((rc = teacher_tables(p, L, ids, tl, mask, nullptr, ws, st))) return rc;
  const CmpGrids g = cmp_grids(p, form, CL, ws);
  const int S = (int)p->S, V = (int)p->V, H = (int)p->H;
  float* kl = at<float>(ws, CL.kl);
  // the dense form projects every row in one pass, the forward-chunked form
  // a chunk of rows at a time; both keep the logits of every row
  const int RL = form == KD_FORM_DENSE ? std::max(S, 1) : (int)L.C;
  for (int c0 = 0; c0 < S; c0 += RL) {
    const int rcap = std::min(RL, S - c0);
    kd::SweepArgs a;
    std::memset(&a, 0, sizeof(a));
    a.W = (const char*)W;
    a.ldw = (int64_t)H * 2;
    a.X = (const char*)hidden;
    a.ldx = (int64_t)H * 2;
    a.idx = at<int32_t>(ws, L.idx);
    a.nrows_dev = at<int32_t>(ws, L.count);
    a.row_begin = c0;
    a.row_cap = rcap;
    a.V = V;
    a.H = H;
    a.K = (int)p->K;
    a.ncu = kCostCUs;
    a.T = p->temperature;
    a.G = (char*)(g.Z + (int64_t)c0 * g.ldz);
    a.ldg = g.ldz * 2;
    {
      Prof pr("cmp_logits", st);
      KD_HIP(kd::launch_sweep(kd::kSweepLogits, 0, 1, a, kd::sweep_grid(rcap, V, kCostCUs), st));
    }
    kd::CmpRowArgs ra;
    std::memset(&ra, 0, sizeof(ra));
    ra.Z = g.Z;
    ra.ldz = g.ldz;
    ra.idx = a.idx;
    ra.nrows_dev = a.nrows_dev;
    ra.row_begin = c0;
    ra.row_cap = rcap;
    ra.V = V;
    ra.Vp = (int)L.Vp;
    ra.K = (int)p->K;
    ra.T = p->temperature;
    ra.ids_s = at<int32_t>(ws, L.ids_s);
    ra.p_s = at<float>(ws, L.p_s);
    ra.negH = at<float>(ws, L.negH);
    ra.lse = lse;
    ra.kl = kl;
    ra.P = g.P;
    ra.logQ = g.logQ;
    ra.ldd = g.ldd;
    Prof pr("cmp_rows", st);
    if (form == KD_FORM_DENSE) {
      KD_HIP(kd::launch_cmp_rows(kd::kCmpDenseGrid, ra, st));
      KD_HIP(kd::launch_cmp_rows(kd::kCmpKlDense, ra, st));
    } else {
      KD_HIP(kd::launch_cmp_rows(kd::kCmpKlSparse, ra, st));
    }
  }
  Prof pr("cmp_loss", st);
  KD_HIP(kd::launch_cmp_loss(at<int32_t>(ws, L.pos), p->S, lse, kl, kl_rows,
                             at<double>(ws, L.bsum), at<int32_t>(ws, L.count), loss, st));
  return KD_OK;
}

int kd_kl_comparator_bwd(const kd_problem* p, int form, const void* hidden, const void* W,
                         const int32_t* ids, const void* tl, const uint8_t* mask,
                         const float* lse, const float* grad_loss, float* dhidden, float* dW,
                         int accumulate_dW, void* ws, size_t ws_bytes, void* stream) {
  int rc = cmp_check(p, form);
  if (rc) return rc;
  if ((rc = bwd_check(p, hidden, W, ids, tl, lse, grad_loss, dhidden, dW, accumulate_dW)))
    return rc;
  const Layout L = plan(p);
  const CmpLayout CL = plan_cmp(p, form, L);
  if (!ws || ((uintptr_t)ws & 255u) != 0 || ws_bytes < CL.total) return KD_ERR_WORKSPACE;
  if ((rc = check_device())) return rc;
  return bwd_run(p, L, cmp_grids(p, form, CL, ws), hidden, W, ids, tl, mask, lse, grad_loss,
                 dhidden, dW, accumulate_dW, ws, (hipStream_t)stream);
}

int kd_student_entropy(const kd_problem* p, const void* hidden, const void* W, double* entropy,
                       void* ws, size_t ws_bytes, void* stream) {
  int rc = check_problem(p);
  if (rc) return rc;
  if (!W || (p->S > 0 && (!hidden || !entropy))) return KD_ERR_NULL;
  const Layout L = plan(p);
  if ((rc = check_ws(L, ws, ws_bytes))) return rc;
  if ((rc = check_device())) return rc;
  hipStream_t st = (hipStream_t)stream;
  const int S = (int)p->S, V = (int)p->V, H = (int)p->H;
  if (S == 0) return KD_OK;
  kd::SweepArgs a;
  std::memset(&a, 0, sizeof(a));
  a.W = (const char*)W;
  a.ldw = (int64_t)H * L.esz;
  a.X = (const char*)hidden;
  a.ldx = (int64_t)H * L.esz;
  a.row_begin = 0;
  a.row_cap = S;
  a.V = V;
  a.H = H;
  a.K = (int)p->K;
  a.ncu = kCostCUs;
  a.T = 1.0f;
  a.em = at<float>(ws, L.em);
  a.es = at<double>(ws, L.es);
  a.eu = at<double>(ws, L.eu);
  {
    Prof pr("entropy_sweep", st);
    KD_HIP(kd::launch_sweep(kd::kSweepEnt, p->hw_dtype == KD_F32, 0, a,
                            kd::sweep_grid(S, V, kCostCUs), st));
  }
  kd::EntCombineArgs c;
  c.S = S;
  c.V = V;
  c.ncu = kCostCUs;
  c.em = a.em;
  c.es = a.es;
  c.eu = a.eu;
  c.entropy = entropy;
  c.lse = nullptr;
  Prof pr("entropy_combine", st);
  KD_HIP(kd::launch_ent_combine(c, st));
  return KD_OK;
}

// ------------------------------------------------------------------ position signals
int kd_position_signals(const kd_problem* p, const void* hidden, const void* W,
                        const int32_t* topk_ids, const void* topk_logits, const int32_t* labels,
                        double* entropy, double* ce, double* teacher_unc, void* ws,
                        size_t ws_bytes, void* stream) {
  int rc = check_problem(p);
  if (rc) return rc;
  const bool sweep = entropy || ce;
  if (p->S > 0) {
    if (sweep && (!hidden || !W)) return KD_ERR_NULL;
    if ((ce || teacher_unc) && !labels) return KD_ERR_NULL;
    if (teacher_unc && (!topk_ids || !topk_logits)) return KD_ERR_NULL;
  }
  const Layout L = plan(p);
  if ((rc = check_ws(L, ws, ws_bytes))) return rc;
  if ((rc = check_device())) return rc;
  hipStream_t st = (hipStream_t)stream;
  const int S = (int)p->S, V = (int)p->V, H = (int)p->H;
  if (S == 0 || (!sweep && !teacher_unc)) return KD_OK;
  double* lse = at<double>(ws, L.lse64);
  if (sweep) {
    // the student at T = 1 over the full vocabulary: entropy and log-normaliser
    kd::SweepArgs a;
    std::memset(&a, 0, sizeof(a));
    a.W = (const char*)W;
    a.ldw = (int64_t)H * L.esz;
    a.X = (const char*)hidden;
    a.ldx = (int64_t)H * L.esz;
    a.row_begin = 0;
    a.row_cap = S;
    a.V = V;
    a.H = H;
    a.K = (int)p->K;
    a.ncu = kCostCUs;
    a.T = 1.0f;
    a.em = at<float>(ws, L.em);
    a.es = at<double>(ws, L.es);
    a.eu = at<double>(ws, L.eu);
    {
      Prof pr("entropy_sweep", st);
      KD_HIP(kd::launch_sweep(kd::kSweepEnt, p->hw_dtype == KD_F32, 0, a,
                              kd::sweep_grid(S, V, kCostCUs), st));
    }
    kd::EntCombineArgs c;
    c.S = S;
    c.V = V;
    c.ncu = kCostCUs;
    c.em = a.em;
    c.es = a.es;
    c.eu = a.eu;
    c.entropy = entropy;
    c.lse = ce ? lse : nullptr;
    Prof pr("entropy_combine", st);
    KD_HIP(kd::launch_ent_combine(c, st));
  }
  if (ce || teacher_unc) {
    kd::SignalArgs g;
    std::memset(&g, 0, sizeof(g));
    g.S = S;
    g.V = V;
    g.H = H;
    g.K = (int)p->K;
    g.hw_f32 = p->hw_dtype == KD_F32;
    g.tl_f32 = p->tl_dtype == KD_F32;
    g.probs = p->tl_kind == KD_TEACHER_PROBS;
    g.invT = 1.0 / (double)p->temperature;
    g.hidden = (const char*)hidden;
    g.ldh = (int64_t)H * L.esz;
    g.W = (const char*)W;
    g.ldw = (int64_t)H * L.esz;
    g.labels = labels;
    g.lse = lse;
    g.ids = topk_ids;
    g.tl = topk_logits;
    g.ce = ce;
    g.tunc = teacher_unc;
    Prof pr("position_signals", st);
    KD_HIP(kd::launch_signals(g, st));
  }
  return KD_OK;
}

// fp64 entropies of the n positions list[0..n) into out[0..n): refinement
// partials for at most kRefinePiece positions at a time; bf16 rows are read in
// place, one launch per piece, fp32 rows widened kRefineBatch per launch
static int refine_positions(const kd_problem* p, const Layout& L, void* ws, const void* hidden,
                            const void* W, kd::SelectWs w, const int32_t* list, int64_t n,
                            double* out, hipStream_t st,
                            const char* scope = "select_refine_fp64") {
  const int f32 = p->hw_dtype == KD_F32;
  const int64_t ld = p->H * L.esz;
  const int nblk = (int)refine_blocks(p->V);
  for (int64_t rs = 0; rs < n; rs += kRefinePiece) {
    const int np = (int)std::min<int64_t>(kRefinePiece, n - rs);
    kd::SelectWs wr = w;
    wr.band = const_cast<int32_t*>(list) + rs;
    const int batch = f32 ? kRefineBatch : np;
    for (int o = 0; o < np; o += batch) {
      Prof pr(scope, st);
      KD_HIP(kd::launch_refine(f32, (const char*)hidden, ld, (const char*)W, ld, (int)p->V,
                               (int)p->H, wr, at<double>(ws, L.xb), o, std::min(batch, np - o),
                               nblk, st));
    }
    Prof pr(scope, st);
    KD_HIP(kd::launch_sample_refined_entropy(wr, np, nblk, out + rs, st));
  }
  return KD_OK;
}

// The bound eps on |entropy - fp64 entropy| that the selections' bands use is
// kSelectEps, or four times the largest error measured on the positions that
// a selection refines in fp64 if that is larger: its band (computed first
// with kSelectEps) and kEpsProbe positions spread evenly over [0, S), which
// ride along in the same refinement. A selection whose measured bound exceeds
// kSelectEps is redone once with the wider band, so that entropies less
// accurate than kSelectEps assumes widen the band instead of deciding the cut.
//
// refine_and_measure: the fp64 entropies of list[0..n) into out[0..n); with
// probe set, the probe positions are appended (list[n..], out[n..]: the arrays
// hold S + kEpsProbe entries) and *h is the largest |entropy - fp64 entropy|
// over all of them (NaN terms skipped). Synchronises the host when probing.
static int refine_and_measure(const kd_problem* p, const Layout& L, void* ws, const void* hidden,
                              const void* W, const kd::SelectWs& w, int32_t* list, int64_t n,
                              double* out, const double* entropy, bool probe, double* h,
                              hipStream_t st) {
  *h = 0.0;
  const int64_t np = probe ? std::min<int64_t>(p->S, kEpsProbe) : 0;
  if (np > 0) KD_HIP(kd::launch_probe_list(list + n, (int)np, p->S, st));
  if (n + np == 0) return KD_OK;
  // a refinement of the probe positions alone is profiled on its own
  int rc = refine_positions(p, L, ws, hidden, W, w, list, n + np, out, st,
                            n > 0 ? "select_refine_fp64" : "select_error_probe");
  if (rc || !probe) return rc;
  double* err = at<double>(ws, L.dscal) + 4;
  KD_HIP(kd::launch_max_abs_diff(entropy, list, (int)(n + np), out, err, st));
  KD_HIP(hipMemcpyAsync(h, err, sizeof(double), hipMemcpyDeviceToHost, st));
  KD_HIP(hipStreamSynchronize(st));
  return KD_OK;
}

// the wider bound when the measured error h calls for it (false for NaN)
static bool widen_eps(double h, double* eps) {
  if (!(4.0 * h > *eps)) return false;
  *eps = 4.0 * h;
  return true;
}

// ------------------------------------------------------------------ selection by a signal
// count of the kept positions (mask) into idx (and its host copy)
static int compact_mask(const Layout& L, void* ws, int64_t S, const uint8_t* mask, int32_t* idx_out,
                        int64_t* count_out, hipStream_t st) {
  int32_t* cnt = at<int32_t>(ws, L.count);
  KD_HIP(kd::launch_compact(mask, nullptr, S, idx_out ? idx_out : at<int32_t>(ws, L.idx),
                            at<int32_t>(ws, L.pos), cnt, st));
  int32_t h = 0;
  KD_HIP(hipMemcpyAsync(&h, cnt, sizeof(int32_t), hipMemcpyDeviceToHost, st));
  KD_HIP(hipStreamSynchronize(st));
  *count_out = h;
  return KD_OK;
}

int kd_select_by_signal(const kd_problem* p, const double* signal, const int64_t* offsets,
                        int64_t B, int64_t num, int64_t den, uint8_t* mask_out, int32_t* idx_out,
                        double* thresholds_out, int64_t* count_out, void* ws, size_t ws_bytes,
                        void* stream) {
  int rc = check_problem(p);
  if (rc) return rc;
  if (!count_out) return KD_ERR_NULL;
  if (den <= 0 || den > 0x7FFFFFFF || num < 0 || num > den) return KD_ERR_ARG;
  if (!offsets) B = 1;
  if (B < 0 || B > std::max<int64_t>(p->S, 1)) return KD_ERR_ARG;
  if (p->S > 0 && (!signal || !mask_out)) return KD_ERR_NULL;
  const Layout L = plan(p);
  if ((rc = check_ws(L, ws, ws_bytes))) return rc;
  if ((rc = check_device())) return rc;
  hipStream_t st = (hipStream_t)stream;
  *count_out = 0;
  const int64_t S = p->S;
  if (offsets && B > 0) {
    int32_t* flag = at<int32_t>(ws, L.scal) + 8;
    KD_HIP(kd::launch_sample_check(offsets, B, S, flag, st));
    int32_t h_flag = 0;
    KD_HIP(hipMemcpyAsync(&h_flag, flag, sizeof(int32_t), hipMemcpyDeviceToHost, st));
    KD_HIP(hipStreamSynchronize(st));
    if (h_flag) return KD_ERR_ARG;
  }
  if (S == 0) {
    if (thresholds_out && B > 0) {
      // segments of an empty problem are empty: nothing kept
      const double nan = std::numeric_limits<double>::quiet_NaN();
      std::vector<double> h((size_t)B, nan);
      KD_HIP(hipMemcpyAsync(thresholds_out, h.data(), (size_t)B * 8, hipMemcpyHostToDevice, st));
      KD_HIP(hipStreamSynchronize(st));
    }
    return KD_OK;
  }
  {
    Prof pr("select_segments", st);
    // positions outside every segment are never kept
    if (offsets) KD_HIP(kd::launch_fill_u8(mask_out, 0, S, st));
    KD_HIP(kd::launch_select_segments(signal, offsets, B, S, num, den, mask_out, thresholds_out, st));
  }
  return compact_mask(L, ws, S, mask_out, idx_out, count_out, st);
}

int kd_select_top_fraction_segments(const kd_problem* p, const void* hidden, const void* W,
                                    const double* entropy, const int64_t* offsets, int64_t B,
                                    int64_t num, int64_t den, uint8_t* mask_out, int32_t* idx_out,
                                    int64_t* count_out, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_problem(p);
  if (rc) return rc;
  if (!count_out) return KD_ERR_NULL;
  if (den <= 0 || den > 0x7FFFFFFF || num < 0 || num > den) return KD_ERR_ARG;
  if (B < 0 || B > std::max<int64_t>(p->S, 1)) return KD_ERR_ARG;
  const int64_t S = p->S;
  if (S > 0 && (!mask_out || !W || !hidden || !entropy || (B > 0 && !offsets))) return KD_ERR_NULL;
  const Layout L = plan(p);
  if ((rc = check_ws(L, ws, ws_bytes))) return rc;
  if ((rc = check_device())) return rc;
  hipStream_t st = (hipStream_t)stream;
  *count_out = 0;
  if (S == 0) return KD_OK;
  KD_HIP(kd::launch_fill_u8(mask_out, 0, S, st));   // positions outside every segment
  if (B == 0) return KD_OK;
  int32_t* flag = at<int32_t>(ws, L.scal) + 8;
  KD_HIP(kd::launch_sample_check(offsets, B, S, flag, st));
  int32_t h_flag = 0;
  KD_HIP(hipMemcpyAsync(&h_flag, flag, sizeof(int32_t), hipMemcpyDeviceToHost, st));
  KD_HIP(hipStreamSynchronize(st));
  if (h_flag) return KD_ERR_ARG;
  double* thr = at<double>(ws, L.smean);
  int32_t* nband = at<int32_t>(ws, L.segw);
  int32_t* nabove = nband + S;
  int32_t* boff = nband + 2 * S;
  int32_t* need = nband + 3 * S;
  int32_t* plist = at<int32_t>(ws, L.spos);
  double* pent = at<double>(ws, L.pent);
  kd::SelectWs w;
  std::memset(&w, 0, sizeof(w));
  w.rpart = at<double>(ws, L.rpart);
  std::vector<int32_t> hb((size_t)B), ha((size_t)B), ho((size_t)B), hn((size_t)B);
  std::vector<int64_t> hoff((size_t)B + 1);
  double eps = kSelectEps;
  for (int pass = 0; pass < 2; ++pass) {
    const double eps2 = 2.0 * eps;
    {
      // the decision on the sweep's entropies, and each segment's k-th largest
      Prof pr("select_segments", st);
      KD_HIP(kd::launch_select_segments(entropy, offsets, B, S, num, den, mask_out, thr, st));
      KD_HIP(kd::launch_seg_band_count(entropy, offsets, B, thr, eps2, nband, nabove, st));
    }
    KD_HIP(hipMemcpyAsync(hb.data(), nband, (size_t)B * 4, hipMemcpyDeviceToHost, st));
    KD_HIP(hipMemcpyAsync(ha.data(), nabove, (size_t)B * 4, hipMemcpyDeviceToHost, st));
    KD_HIP(hipMemcpyAsync(hoff.data(), offsets, (size_t)(B + 1) * 8, hipMemcpyDeviceToHost, st));
    KD_HIP(hipStreamSynchronize(st));
    // segments whose band straddles the cut are refined (segments are
    // disjoint, so their bands list at most S positions); the others keep the
    // decision on the sweep's entropies, which no band position can change
    int64_t total = 0;
    for (int64_t b = 0; b < B; ++b) {
      const int64_t k = (num * (hoff[b + 1] - hoff[b])) / den;
      const int64_t nd = k - ha[b];
      hn[b] = (int32_t)nd;
      ho[b] = -1;
      if (nd > 0 && nd < hb[b]) {
        ho[b] = (int32_t)total;
        total += hb[b];
      }
    }
    if (total > 0) {
      KD_HIP(hipMemcpyAsync(boff, ho.data(), (size_t)B * 4, hipMemcpyHostToDevice, st));
      KD_HIP(hipMemcpyAsync(need, hn.data(), (size_t)B * 4, hipMemcpyHostToDevice, st));
      KD_HIP(kd::launch_seg_band_list(entropy, offsets, B, thr, eps2, boff, plist, st));
    }
    // the first pass measures the error on the band and the probe positions
    double h = 0.0;
    if ((rc = refine_and_measure(p, L, ws, hidden, W, w, plist, total, pent, entropy, pass == 0,
                                 &h, st)))
      return rc;
    if (pass == 0 && widen_eps(h, &eps)) continue;
    if (total > 0) {
      Prof pr("select_segments_final", st);
      KD_HIP(kd::launch_seg_band_final(B, boff, nband, need, plist, pent, mask_out, st));
    }
    break;
  }
  return compact_mask(L, ws, S, mask_out, idx_out, count_out, st);
}

int kd_select_above(const kd_problem* p, const double* signal, double tau, uint8_t* mask_out,
                    int32_t* idx_out, int64_t* count_out, void* ws, size_t ws_bytes,
                    void* stream) {
  int rc = check_problem(p);
  if (rc) return rc;
  if (!count_out) return KD_ERR_NULL;
  if (p->S > 0 && (!signal || !mask_out)) return KD_ERR_NULL;
  if (std::isnan(tau)) return KD_ERR_ARG;
  const Layout L = plan(p);
  if ((rc = check_ws(L, ws, ws_bytes))) return rc;
  if ((rc = check_device())) return rc;
  hipStream_t st = (hipStream_t)stream;
  *count_out = 0;
  if (p->S == 0) return KD_OK;
  {
    Prof pr("select_above", st);
    KD_HIP(kd::launch_select_above(signal, p->S, tau, mask_out, st));
  }
  return compact_mask(L, ws, p->S, mask_out, idx_out, count_out, st);
}

int kd_select_top_fraction(const kd_problem* p, const void* hidden, const void* W,
                           const double* entropy, int64_t num, int64_t den, uint8_t* mask_out,
                           int32_t* idx_out, int64_t* count_out, void* ws, size_t ws_bytes,
                           void* stream) {
  int rc = check_problem(p);
  if (rc) return rc;
  if (!count_out || !W || (p->S > 0 && (!hidden || !entropy || !mask_out))) return KD_ERR_NULL;
  if (den <= 0 || num < 0 || num > den) return KD_ERR_ARG;
  const Layout L = plan(p);
  if ((rc = check_ws(L, ws, ws_bytes))) return rc;
  if ((rc = check_device())) return rc;
  hipStream_t st = (hipStream_t)stream;
  const int64_t S = p->S;
  const int64_t k = (num * S) / den;
  *count_out = 0;
  if (S == 0) return KD_OK;
  kd::SelectWs w;
  w.keys = nullptr;
  w.band = at<int32_t>(ws, L.band);
  w.refined = at<double>(ws, L.refined);
  w.scal = at<int32_t>(ws, L.scal);
  w.dscal = at<double>(ws, L.dscal);
  w.rpart = at<double>(ws, L.rpart);
  w.hist = nullptr;
  double eps = kSelectEps;
  int32_t n_band = 0;
  for (int pass = 0; pass < 2; ++pass) {
    {
      Prof pr("select_threshold", st);
      KD_HIP(kd::launch_select_threshold(entropy, S, k, eps, w, st));
    }
    KD_HIP(hipMemcpyAsync(&n_band, w.scal, sizeof(int32_t), hipMemcpyDeviceToHost, st));
    KD_HIP(hipStreamSynchronize(st));
    // every band row is recomputed in fp64, in pieces, whatever the band's
    // size; the first pass also measures the error (band and probe positions)
    double h = 0.0;
    if ((rc = refine_and_measure(p, L, ws, hidden, W, w, w.band, n_band, w.refined, entropy,
                                 pass == 0, &h, st)))
      return rc;
    if (pass == 0 && widen_eps(h, &eps)) continue;
    break;
  }
  {
    Prof pr("select_final", st);
    KD_HIP(kd::launch_select_final(entropy, S, k, w, n_band, mask_out, idx_out, st));
  }
  int32_t cnt = 0;
  KD_HIP(hipMemcpyAsync(&cnt, w.scal + 2, sizeof(int32_t), hipMemcpyDeviceToHost, st));
  KD_HIP(hipStreamSynchronize(st));
  *count_out = cnt;
  return KD_OK;
}

// ------------------------------------------------------------------ sample selection
int kd_select_samples(const kd_problem* p, const void* hidden, const void* W, const double* entropy,
                      const int64_t* offsets, int64_t B, int64_t num, int64_t den,
                      uint8_t* mask_out, int32_t* idx_out, int64_t* count_out, void* ws,
                      size_t ws_bytes, void* stream) {
  int rc = check_problem(p);
  if (rc) return rc;
  if (!count_out || !W || (B > 0 && (!offsets || !entropy || !mask_out || !hidden)))
    return KD_ERR_NULL;
  if (den <= 0 || num < 0 || num > den || B < 0 || B > std::max<int64_t>(p->S, 1)) return KD_ERR_ARG;
  const Layout L = plan(p);
  if ((rc = check_ws(L, ws, ws_bytes))) return rc;
  if ((rc = check_device())) return rc;
  hipStream_t st = (hipStream_t)stream;
  *count_out = 0;
  if (B == 0) return KD_OK;
  kd::SelectWs w;
  w.keys = nullptr;
  w.band = at<int32_t>(ws, L.band);
  w.refined = at<double>(ws, L.refined);
  w.scal = at<int32_t>(ws, L.scal);
  w.dscal = at<double>(ws, L.dscal);
  w.rpart = at<double>(ws, L.rpart);
  w.hist = nullptr;
  int32_t* flag = w.scal + 8;
  KD_HIP(kd::launch_sample_check(offsets, B, p->S, flag, st));
  int32_t h_flag = 0;
  KD_HIP(hipMemcpyAsync(&h_flag, flag, sizeof(int32_t), hipMemcpyDeviceToHost, st));
  KD_HIP(hipStreamSynchronize(st));
  if (h_flag) return KD_ERR_ARG;
  double* means = at<double>(ws, L.smean);
  const int64_t k = (num * B) / den;
  {
    Prof pr("sample_means", st);
    KD_HIP(kd::launch_sample_means(entropy, offsets, B, means, st));
  }
  const int64_t S = p->S;
  uint8_t* pflag = at<uint8_t>(ws, L.segw);
  int32_t* plist = at<int32_t>(ws, L.spos);
  int32_t* ppos = at<int32_t>(ws, L.pos);
  double* pent = at<double>(ws, L.pent);
  int32_t* cnt_dev = at<int32_t>(ws, L.count);
  double eps = kSelectEps;
  int n_band = 0, refined = 0;
  for (int pass = 0; pass < 2; ++pass) {
    {
      Prof pr("select_threshold", st);
      KD_HIP(kd::launch_select_threshold(means, B, k, eps, w, st));
    }
    int32_t hs[2] = {0, 0};
    KD_HIP(hipMemcpyAsync(hs, w.scal, sizeof(hs), hipMemcpyDeviceToHost, st));
    KD_HIP(hipStreamSynchronize(st));
    n_band = hs[0];
    const int64_t need = k - hs[1];
    // the band straddles the cut: the entropies of every position of its
    // samples are recomputed in fp64 (each position once, whatever the band's
    // size or the samples' overlap) and the band is ranked on fp64 means
    refined = need > 0 && need < n_band;
    int32_t total = 0;
    if (refined) {
      KD_HIP(kd::launch_fill_u8(pflag, 0, S, st));
      KD_HIP(kd::launch_sample_mark(offsets, w, n_band, pflag, st));
      KD_HIP(kd::launch_compact(pflag, nullptr, S, plist, ppos, cnt_dev, st));
      KD_HIP(hipMemcpyAsync(&total, cnt_dev, sizeof(int32_t), hipMemcpyDeviceToHost, st));
      KD_HIP(hipStreamSynchronize(st));
    }
    // the first pass also measures the error (those positions and the probe)
    double herr = 0.0;
    if ((rc = refine_and_measure(p, L, ws, hidden, W, w, plist, total, pent, entropy, pass == 0,
                                 &herr, st)))
      return rc;
    if (pass == 0 && widen_eps(herr, &eps)) continue;
    if (refined) KD_HIP(kd::launch_sample_band_means(offsets, w, n_band, ppos, pent, st));
    break;
  }
  {
    Prof pr("sample_final", st);
    KD_HIP(kd::launch_sample_final(means, B, k, w, n_band, refined, mask_out, idx_out, st));
  }
  int32_t cnt = 0;
  KD_HIP(hipMemcpyAsync(&cnt, w.scal + 2, sizeof(int32_t), hipMemcpyDeviceToHost, st));
  KD_HIP(hipStreamSynchronize(st));
  *count_out = cnt;
  return KD_OK;
}

// ------------------------------------------------------------------ teacher cache writer
constexpr int64_t kPilotRows = 16384;      // vocabulary rows of the pilot pass
constexpr int kTeacherFinalGroups = 4096;  // work-groups of the final ranking (one per row of a chunk up to this)
constexpr int kTeacherBigGroups = 16;      // work-groups (and scratch areas) for large bands

struct TeacherLayout {
  int64_t C, P, NG, ldp, cap;   // P pilot vocabulary rows, NG groups of 16 of them
  int64_t scnt_ld;              // per row: 4 emit writers for each vocabulary range
  size_t zp, cid, cz, cnt, scnt, te, bnd, tau2, big, nbig, wpart, wmax, scratch, total;
};

TeacherLayout plan_teacher(const kd_problem* p) {
  TeacherLayout L{};
  const int64_t S = p->S, V = p->V;
  L.C = std::min<int64_t>(p->chunk, std::max<int64_t>(S, 1));
  L.P = std::min<int64_t>(V, kPilotRows);
  L.NG = kd::ceil_div(L.P, kd::kTile) * 16;
  L.ldp = kd::round_up(L.C, 64);
  // a row's candidates are distinct vocabulary entries; the emit pass lays
  // them out in per-writer sub-lists that together span whole 256-entry tiles
  L.cap = kd::round_up(V, kd::kTile);
  {
    const int nvt = (int)kd::ceil_div(V, kd::kTile);
    int nsmax = 1;
    for (int n = 1; n <= (int)kd::ceil_div(L.C, kd::kTile); ++n)
      nsmax = std::max(nsmax, kd::sweep_splits(n, nvt, kCostCUs));
    L.scnt_ld = (int64_t)nsmax * 4;
  }
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (size_t)kd::round_up((int64_t)bytes, 256);
    return o;
  };
  L.zp = take((size_t)L.NG * L.ldp * 4);
  L.cid = take((size_t)L.C * L.cap * 4);
  L.cz = take((size_t)L.C * L.cap * 4);
  L.cnt = take((size_t)L.C * 4);
  L.scnt = take((size_t)L.C * L.scnt_ld * 4);
  L.te = take((size_t)L.C * 4);
  L.bnd = take((size_t)L.C * 8);
  L.tau2 = take((size_t)L.C * 4);
  L.big = take((size_t)L.C * 4);
  L.nbig = take(8);
  L.wpart = take((size_t)kd::kTeacherWnormGroups * 8);
  L.wmax = take(8);
  L.scratch = take((size_t)kTeacherBigGroups * kd::teacher_scratch_entries(L.cap) * 12);
  L.total = off;
  return L;
}

size_t kd_teacher_topk_workspace_bytes(const kd_problem* p) {
  if (check_problem(p)) return 0;
  return plan_teacher(p).total;
}

int kd_teacher_topk(const kd_problem* p, const void* hidden, const void* W, int32_t* topk_ids,
                    void* topk_logits, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_problem(p);
  if (rc) return rc;
  if (!W || (p->S > 0 && (!hidden || !topk_ids || !topk_logits))) return KD_ERR_NULL;
  const TeacherLayout L = plan_teacher(p);
  if (!ws || ((uintptr_t)ws & 255u) != 0 || ws_bytes < L.total) return KD_ERR_WORKSPACE;
  if ((rc = check_device())) return rc;
  if (p->S == 0) return KD_OK;
  hipStream_t st = (hipStream_t)stream;
  const int f32 = p->hw_dtype == KD_F32;
  const int64_t esz = f32 ? 4 : 2;
  const int64_t oesz = p->tl_dtype == KD_F32 ? 4 : 2;
  const int S = (int)p->S, H = (int)p->H, V = (int)p->V, K = (int)p->K;
  const int P = (int)L.P;
  const int64_t ld = (int64_t)H * esz;
  {
    Prof pr("teacher_wnorm", st);
    KD_HIP(kd::launch_teacher_wnorm(f32, (const char*)W, ld, V, H, at<double>(ws, L.wpart),
                                    at<double>(ws, L.wmax), st));
  }
  for (int64_t c0 = 0; c0 < S; c0 += L.C) {
    const int rows = (int)std::min<int64_t>(L.C, S - c0);
    const char* X = (const char*)hidden + c0 * ld;
    kd::SweepArgs a;
    std::memset(&a, 0, sizeof(a));
    a.W = (const char*)W;
    a.ldw = ld;
    a.X = X;
    a.ldx = ld;
    a.row_cap = rows;
    a.V = P;
    a.H = H;
    a.K = K;
    a.ncu = kCostCUs;
    a.T = 1.0f;
    a.zp = at<float>(ws, L.zp);
    a.ldp = L.ldp;
    {
      Prof pr("teacher_pilot", st);
      KD_HIP(kd::launch_sweep(kd::kSweepPilot, f32, 0, a, kd::sweep_grid(rows, P, kCostCUs), st));
    }
    kd::TeacherArgs t;
    std::memset(&t, 0, sizeof(t));
    t.X = X;
    t.ldx = ld;
    t.W = (const char*)W;
    t.ldw = ld;
    t.rows = rows;
    t.H = H;
    t.V = V;
    t.K = K;
    t.P = (int)L.NG;
    t.zp = at<float>(ws, L.zp);
    t.ldp = L.ldp;
    t.wmax = at<double>(ws, L.wmax);
    t.te = at<float>(ws, L.te);
    t.bnd = at<double>(ws, L.bnd);
    t.cnt = at<int32_t>(ws, L.cnt);
    t.cid = at<int32_t>(ws, L.cid);
    t.cz = at<float>(ws, L.cz);
    t.cap = L.cap;
    t.scratch = at<char>(ws, L.scratch);
    t.ids_out = topk_ids + c0 * K;
    t.logits_out = (char*)topk_logits + c0 * K * oesz;
    t.out_bf16 = p->tl_dtype == KD_BF16;
    int32_t* nbig = at<int32_t>(ws, L.nbig);
    {
      Prof pr("teacher_threshold", st);
      KD_HIP(kd::launch_teacher_threshold(f32, t, nbig, st));
    }
    {
      kd::SweepArgs e = a;
      e.V = V;
      e.te = t.te;
      e.cnt = t.cnt;
      e.cid = t.cid;
      e.cz = t.cz;
      e.cap = t.cap;
      e.id_offset = 0;
      e.scnt = at<int32_t>(ws, L.scnt);
      e.scnt_ld = L.scnt_ld;
      {
        Prof pr("teacher_emit", st);
        KD_HIP(kd::launch_sweep(kd::kSweepEmit, f32, 0, e, kd::sweep_grid(rows, V, kCostCUs), st));
      }
      Prof pr("teacher_gather", st);
      const int nvt = (int)kd::ceil_div(V, kd::kTile);
      const int ns = kd::sweep_splits((int)kd::ceil_div(rows, kd::kTile), nvt, kCostCUs);
      KD_HIP(kd::launch_teacher_gather(t.cid, t.cz, t.cap, e.scnt, e.scnt_ld, ns, nvt, rows, t.cnt,
                                       st));
    }
    {
      Prof pr("teacher_final", st);
      KD_HIP(kd::launch_teacher_final(f32, t, at<int32_t>(ws, L.big), nbig, at<float>(ws, L.tau2),
                                      std::min(rows, kTeacherFinalGroups), kTeacherBigGroups, st));
    }
  }
  return KD_OK;
}

// ------------------------------------------------------------------ sampled teacher targets
struct SampleLayout {
  int64_t C, ldm, nu, nvt;   // rows per chunk, unit-mass pitch, 128-entry units, 256-entry tiles
  size_t flag, mass, scale, rowmax, dunit, dres, tcnt, toff, tfill, tlist, total;
};

SampleLayout plan_sample(const kd_problem* p) {
  SampleLayout L{};
  const int64_t S = std::max<int64_t>(p->S, 1), N = p->K;
  L.nu = kd::ceil_div(p->V, 128);
  L.nvt = kd::ceil_div(p->V, 256);
  // rows per chunk; the draw pass's row lists (at most min(N, tiles) entries
  // per row) keep int32 offsets, so a chunk holds fewer than 2^31 of them
  // (each row is sampled on its own: the chunking does not change the ids)
  L.C = std::min<int64_t>(std::min<int64_t>(p->chunk, S),
                          INT32_MAX / std::max<int64_t>(std::min<int64_t>(N, L.nvt), 1));
  L.ldm = kd::round_up(L.C, 64);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (size_t)kd::round_up((int64_t)bytes, 256);
    return o;
  };
  L.flag = take(8);
  L.mass = take((size_t)L.nu * L.ldm * 8);
  L.scale = take((size_t)L.nu * L.ldm * 4);
  L.rowmax = take((size_t)L.C * 4);
  L.dunit = take((size_t)L.C * N * 4);
  L.dres = take((size_t)L.C * N * 8);
  // the draw pass's rows per drawn-in tile: a row is listed once per tile,
  // at most min(N, tiles) times
  L.tcnt = take((size_t)L.nvt * 4);
  L.toff = take((size_t)L.nvt * 4);
  L.tfill = take((size_t)L.nvt * 4);
  L.tlist = take((size_t)L.C * std::min<int64_t>(N, L.nvt) * 4);
  L.total = off;
  return L;
}

size_t kd_teacher_sample_workspace_bytes(const kd_problem* p) {
  if (check_problem(p)) return 0;
  return plan_sample(p).total;
}

int kd_teacher_sample(const kd_problem* p, const void* hidden, const void* W,
                      const double* uniforms, int32_t* ids_out, void* ws, size_t ws_bytes,
                      void* stream) {
  int rc = check_problem(p);
  if (rc) return rc;
  if (!W || (p->S > 0 && (!hidden || !uniforms || !ids_out))) return KD_ERR_NULL;
  const SampleLayout L = plan_sample(p);
  if (!ws || ((uintptr_t)ws & 255u) != 0 || ws_bytes < L.total) return KD_ERR_WORKSPACE;
  if ((rc = check_device())) return rc;
  if (p->S == 0) return KD_OK;
  hipStream_t st = (hipStream_t)stream;
  const int f32 = p->hw_dtype == KD_F32;
  const int64_t esz = f32 ? 4 : 2;
  const int S = (int)p->S, H = (int)p->H, V = (int)p->V, N = (int)p->K;
  const int64_t ld = (int64_t)H * esz;
  int32_t* flag = at<int32_t>(ws, L.flag);
  KD_HIP(kd::launch_draw_check(uniforms, S, N, flag, st));
  int32_t h_flag = 0;
  KD_HIP(hipMemcpyAsync(&h_flag, flag, sizeof(int32_t), hipMemcpyDeviceToHost, st));
  KD_HIP(hipStreamSynchronize(st));
  if (h_flag) return KD_ERR_ARG;
  double* mass = at<double>(ws, L.mass);
  float* scale = at<float>(ws, L.scale);
  float* rowmax = at<float>(ws, L.rowmax);
  int32_t* dunit = at<int32_t>(ws, L.dunit);
  double* dres = at<double>(ws, L.dres);
  int32_t* tcnt = at<int32_t>(ws, L.tcnt);
  int32_t* toff = at<int32_t>(ws, L.toff);
  int32_t* tfill = at<int32_t>(ws, L.tfill);
  int32_t* tlist = at<int32_t>(ws, L.tlist);
  for (int64_t c0 = 0; c0 < S; c0 += L.C) {
    const int rows = (int)std::min<int64_t>(L.C, S - c0);
    kd::SweepArgs b;
    std::memset(&b, 0, sizeof(b));
    b.W = (const char*)W;
    b.ldw = ld;
    b.X = (const char*)hidden + c0 * ld;
    b.ldx = ld;
    b.row_cap = rows;
    b.V = V;
    b.H = H;
    b.K = N;
    b.ncu = kCostCUs;
    b.T = p->temperature;
    b.tmass = mass;
    b.tscale = scale;
    b.ldm = L.ldm;
    b.N = N;
    const int grid = kd::sweep_grid(rows, V, kCostCUs);
    {
      Prof pr("sample_mass", st);
      KD_HIP(kd::launch_sweep(kd::kSweepSMass, f32, 0, b, grid, st));
    }
    {
      Prof pr("sample_assign", st);
      KD_HIP(kd::launch_draw_cumsum(mass, scale, L.ldm, (int)L.nu, rows, rowmax, st));
      KD_HIP(kd::launch_draw_assign(mass, scale, rowmax, L.ldm, (int)L.nu, rows, uniforms + c0 * N,
                                    N, dunit, dres, ids_out + c0 * N, st));
    }
    b.dunit = dunit;
    b.dres = dres;
    b.sids = ids_out + c0 * N;
    {
      // each draw resolved inside its unit: only the vocabulary tiles some
      // row draws in are recomputed, for the rows that draw there
      {
        Prof pt("sample_draw_tiles", st);
        KD_HIP(kd::launch_draw_tiles(dunit, rows, N, (int)L.nvt, tcnt, toff, tfill, tlist, st));
      }
      Prof pr("sample_draw", st);
      b.idx = tlist;
      b.tcnt = tcnt;
      b.toff = toff;
      const int64_t tgrid = L.nvt * kd::ceil_div(rows, kd::kTile);
      if (tgrid > INT32_MAX) return KD_ERR_SHAPE;
      KD_HIP(kd::launch_sweep(kd::kSweepSDrawTiles, f32, 1, b, (int)tgrid, st));
    }
  }
  return KD_OK;
}

int kd_validate_topk(const kd_problem* p, const int32_t* ids, const void* tl, int64_t* n_bad_id,
                     int64_t* n_empty_row, int64_t* n_bad_logit, void* ws, size_t ws_bytes,
                     void* stream) {
  int rc = check_problem(p);
  if (rc) return rc;
  if (!n_bad_id || !n_empty_row || !n_bad_logit || (p->S > 0 && (!ids || !tl))) return KD_ERR_NULL;
  const Layout L = plan(p);
  if ((rc = check_ws(L, ws, ws_bytes))) return rc;
  if ((rc = check_device())) return rc;
  hipStream_t st = (hipStream_t)stream;
  unsigned long long* cnt = at<unsigned long long>(ws, L.counters);
  {
    Prof pr("validate", st);
    KD_HIP(kd::launch_validate(ids, tl, p->tl_dtype == KD_F32, p->tl_kind == KD_TEACHER_PROBS,
                               p->S, (int)p->K, (int)p->V, cnt,
                               st));
  }
  unsigned long long h[3] = {0, 0, 0};
  KD_HIP(hipMemcpyAsync(h, cnt, sizeof(h), hipMemcpyDeviceToHost, st));
  KD_HIP(hipStreamSynchronize(st));
  *n_bad_id = (int64_t)h[0];
  *n_empty_row = (int64_t)h[1];
  *n_bad_logit = (int64_t)h[2];
  return KD_OK;
}

int kd_validate_topk_order(const kd_problem* p, const int32_t* ids, const void* tl,
                           int64_t* n_unsorted_row, int64_t* n_duplicate_row, void* ws,
                           size_t ws_bytes, void* stream) {
  int rc = check_problem(p);
  if (rc) return rc;
  if (!n_unsorted_row || !n_duplicate_row || (p->S > 0 && (!ids || !tl))) return KD_ERR_NULL;
  const Layout L = plan(p);
  if ((rc = check_ws(L, ws, ws_bytes))) return rc;
  if ((rc = check_device())) return rc;
  hipStream_t st = (hipStream_t)stream;
  unsigned long long* cnt = at<unsigned long long>(ws, L.counters);
  {
    Prof pr("validate_order", st);
    KD_HIP(kd::launch_validate_order(ids, tl, p->tl_dtype == KD_F32, p->S, (int)p->K, cnt, st));
  }
  unsigned long long h[2] = {0, 0};
  KD_HIP(hipMemcpyAsync(h, cnt, sizeof(h), hipMemcpyDeviceToHost, st));
  KD_HIP(hipStreamSynchronize(st));
  *n_unsorted_row = (int64_t)h[0];
  *n_duplicate_row = (int64_t)h[1];
  return KD_OK;
}

int kd_profile_enable(int on) {
  std::lock_guard<std::mutex> g(g_prof_mu);
  g_prof_on = on != 0;
  return KD_OK;
}

int kd_profile_reset(void) {
  std::lock_guard<std::mutex> g(g_prof_mu);
  for (auto& r : g_prof_recs) {
    g_event_pool.push_back(r.a);
    g_event_pool.push_back(r.b);
  }
  g_prof_recs.clear();
  return KD_OK;
}

int kd_profile_read(kd_kernel_stat* out, int max_entries) {
  std::vector<ProfRec> recs;
  {
    std::lock_guard<std::mutex> g(g_prof_mu);
    recs = g_prof_recs;
  }
  std::vector<std::string> names;
  std::map<std::string, std::pair<int64_t, double>> agg;
  for (auto& r : recs) {
    if (hipEventSynchronize(r.b) != hipSuccess) return -KD_ERR_HIP;
    float ms = 0.0f;
    if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) return -KD_ERR_HIP;
    auto it = agg.find(r.name);
    if (it == agg.end()) {
      names.push_back(r.name);
      it = agg.emplace(r.name, std::make_pair((int64_t)0, 0.0)).first;
    }
    it->second.first += 1;
    it->second.second += ms;
  }
  int n = 0;
  for (auto& nm : names) {
    if (n >= max_entries || !out) break;
    std::memset(&out[n], 0, sizeof(kd_kernel_stat));
    std::strncpy(out[n].name, nm.c_str(), sizeof(out[n].name) - 1);
    out[n].launches = agg[nm].first;
    out[n].total_ms = agg[nm].second;
    ++n;
  }
  return n;
}

}  // extern "C"
