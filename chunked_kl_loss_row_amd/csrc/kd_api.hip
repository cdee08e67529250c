// C ABI of the fused chunked top-K KL loss: argument checks, workspace
// layout and the chunk scheduler.  See include/kd_chunked.h for the contract.
//
// The scheduler walks the rows in contiguous chunks of `chunk` rows (the last
// one ragged) and enqueues each chunk's kernels on the caller's stream, reusing
// one workspace whose size depends on the chunk, never on n: memory grows with
// the sequence only through the caller's own inputs and outputs (aivibenews.ru
// page "Дистилляция LLM на одной GPU…", section "Два приёма"; agentlenshq.com
// page "LLMのための効率的な知識蒸留…", section "2. Fused Chunked KL Loss").
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "kd_chunked.h"
#include "kd_gemm.h"  // blocked dZ layout (blk_pitch)
#include "kd_internal.h"
#include "kd_profile.h"
#include "kd_topk.h"

namespace {

using kd::ChunkArgs;

constexpr size_t kAlign = 256;
// Projection tiles per chunk: 512 work-items each, the grid rounded up to a
// multiple of 8, below 2^32 work-items in all.
constexpr int64_t kMaxProjTiles = (int64_t{1} << 23) - 8;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool dtype_ok(int t) { return t == KD_F32 || t == KD_BF16; }

// Workspace regions, as byte offsets from the aligned base.
struct Layout {
  int nvt, ldz, split, kslice;
  int rows;  // row capacity of the per-row regions (one backward unit: a group of chunks)
  size_t keys, psort, zgs, negent, ssum, lb, pm, ps, rl, loss_acc, dz, dhp, zc, ht, hk;
  int ldt;
  size_t lmax, thr, cnt, cand;  // teacher top-K producer
  size_t total;  // bytes from the aligned base
};

enum class Mode { kLoss, kLossCached, kTopk, kForward };

// Chunks whose dZ one dW GEMM reads (kd_problem.dw_chunks; 0 means 1).
int dw_group(const kd_problem& p) { return p.dw_chunks > 1 ? p.dw_chunks : 1; }

// kLossCached: the single-call path also keeps the chunk's fp32 logits;
// kTopk: the teacher top-K producer (no dZ; per-row thresholds and
// candidate lists instead); kForward: the regions kd_chunked_fwd uses (no
// dZ, no dH partials, no H^T).
// The backward walks groups of dw_chunks chunks (one launch of each kernel per
// group), so in the backward modes every per-row region holds a group's rows.
// The dH split stays that of one chunk: each row's dH is then summed over the
// same V slices in the same order whatever the grouping.
Layout layout_for(const kd_problem& p, Mode mode = Mode::kLoss) {
  Layout L{};
  const bool bwd = mode == Mode::kLoss || mode == Mode::kLossCached;
  const size_t G = static_cast<size_t>(dw_group(p));
  const size_t C = static_cast<size_t>(p.chunk) * (bwd ? G : 1), K = static_cast<size_t>(p.k);
  L.rows = static_cast<int>(C);
  L.nvt = (p.v + kd::kProjBN - 1) / kd::kProjBN;
  L.ldz = L.nvt * kd::kProjBN;
  L.split = kd::dh_split_for(p.chunk, p.d, L.ldz, &L.kslice);
  const size_t xs = p.x_dtype == KD_BF16 ? 2 : 4;
  size_t o = 0;
  auto take = [&o](size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  L.keys = take(C * K * 4);
  L.psort = take(C * K * 4);
  L.zgs = take(C * K * 4);
  L.negent = take(C * 4);
  L.ssum = take(C * 4);
  L.lb = take(C * (static_cast<size_t>(L.nvt) + 1) * 2);
  L.pm = take(C * L.nvt * 4);
  L.ps = take(C * L.nvt * 4);
  L.rl = take(C * 8);
  L.loss_acc = take(8);
  const bool loss = mode != Mode::kTopk;
  // dZ and the cached logits are blocked (32 x 32 blocks): whole blocks of rows
  L.dz = take(bwd ? (C + 31) / 32 * static_cast<size_t>(xs == 2 ? kd::blk_pitch<2>(L.ldz) : kd::blk_pitch<4>(L.ldz))
                  : 0);
  L.dhp = take(bwd && L.split > 1 ? static_cast<size_t>(L.split) * C * static_cast<size_t>(p.d) * 4 : 0);
  // the single-call path keeps one chunk of fp32 logits at a time
  L.zc = take(mode == Mode::kLossCached ? (static_cast<size_t>(p.chunk) + 31) / 32 * kd::blk_pitch<4>(L.ldz) : 0);
  L.ldt = static_cast<int>((C + 31) / 32 * 32);  // whole k tiles of H_c^T
  L.ht = take(bwd ? static_cast<size_t>(L.ldt) * static_cast<size_t>(p.d) * xs : 0);
  // H_c in k tiles of 64 bytes (the A operand of every projection)
  L.hk = take(C * ((static_cast<size_t>(p.d) * xs + 63) / 64) * 64);
  L.lmax = take(loss ? 0 : C * static_cast<size_t>(L.nvt) * kd::kTopkLanes * 4);
  L.thr = take(loss ? 0 : C * 4);
  L.cnt = take(loss ? 0 : C * 4);
  L.cand = take(loss ? 0 : C * static_cast<size_t>(kd::kTopkCap) * 8);
  L.total = o;
  return L;
}

// Rows one kd_chunked_fwd pass covers: up to 8 chunks.  The forward keeps
// no dZ, so its per-row regions for several chunks fit in the workspace the
// backward needs for one; larger passes fill the chip better (fewer partly
// filled rounds of projection tiles, fewer launches).  Every row's results
// are computed the same way whatever the pass, and the running loss adds
// chunk-sized slices in order, so the outputs do not depend on it.  Passes
// stay at or below 65536 rows (one chunk if the chunk is larger).
int fwd_pass_rows(const kd_problem& p, size_t room) {
  for (int g = 8; g > 1; g >>= 1) {
    const int64_t rows = static_cast<int64_t>(g) * p.chunk;
    if (rows > 65536) continue;
    if (static_cast<int64_t>(g / 2) * p.chunk >= p.n) continue;  // half as many chunks cover n
    const int64_t nvt = (static_cast<int64_t>(p.v) + kd::kProjBN - 1) / kd::kProjBN;
    if ((rows + kd::kProjBM - 1) / kd::kProjBM * nvt > kMaxProjTiles) continue;  // the grid's limit
    kd_problem q = p;
    q.chunk = static_cast<int32_t>(rows);
    if (layout_for(q, Mode::kForward).total <= room) return static_cast<int>(rows);
  }
  return p.chunk;
}

int check_problem(const kd_problem* p) {
  if (!p) return KD_ERR_NULL;
  if (p->n < 0 || p->d < 1 || p->d > 65536 || p->v < 1 || p->v > 16777215 || p->k < 1 || p->k > 256 || p->k > p->v ||
      p->chunk < 1)
    return KD_ERR_SHAPE;
  if (!dtype_ok(p->x_dtype) || !dtype_ok(p->t_dtype)) return KD_ERR_DTYPE;
  // temperature: 0 means 1; otherwise a finite value in [0.01, 100]
  if (!(p->tau == 0.f || (p->tau >= 0.01f && p->tau <= 100.f))) return KD_ERR_SHAPE;
  if (p->dw_chunks < 0 || p->dw_chunks > 8) return KD_ERR_SHAPE;
  // The matrix-core tiles address an operand panel (256 rows of its leading
  // dimension) with 32-bit byte offsets: dZ (leading dimension 384 * ceil(v
  // / 384), blocked, every 32 rows one contiguous block row) in dH must stay
  // below 2^31 bytes per panel.  The
  // rows of one dW group (dw_chunks * chunk, rounded up to 8) are held to the
  // same bound: the launch code and the kernels count group rows and the
  // transposed H_c's row offsets in 32-bit ints, and this cap keeps them, with
  // the rounding to whole k tiles, far from overflow.
  if (dtype_ok(p->x_dtype)) {
    const int64_t xs = p->x_dtype == KD_BF16 ? 2 : 4;
    const int64_t ldz = (static_cast<int64_t>(p->v) + kd::kProjBN - 1) / kd::kProjBN * kd::kProjBN;
    const int64_t ldt = (static_cast<int64_t>(p->chunk) * (p->dw_chunks > 1 ? p->dw_chunks : 1) + 7) / 8 * 8;
    if (256 * ldz * xs + 8 * kd::kBlPad > 0x7FFFFFF0LL || 256 * ldt * xs > 0x7FFFFFF0LL) return KD_ERR_SHAPE;
  }
  // One projection launch covers the (row tile, vocabulary tile) pairs of a
  // chunk -- of a group of dw_chunks chunks in the backward -- with 512
  // work-items each; its work-item count must fit in 32 bits, and so must
  // that of the group's dH launch (row tiles x hidden tiles x V slices).
  const int64_t grows = static_cast<int64_t>(p->chunk) * (p->dw_chunks > 1 ? p->dw_chunks : 1);
  const int64_t ptiles = (grows + kd::kProjBM - 1) / kd::kProjBM *
                         ((static_cast<int64_t>(p->v) + kd::kProjBN - 1) / kd::kProjBN);
  if (ptiles > kMaxProjTiles) return KD_ERR_SHAPE;
  {
    int kslice = 0;
    const int ldz = (p->v + kd::kProjBN - 1) / kd::kProjBN * kd::kProjBN;
    const int split = kd::dh_split_for(p->chunk, p->d, ldz, &kslice);
    const int64_t dtiles = (grows + kd::kDhBM - 1) / kd::kDhBM * ((p->d + kd::kDhBN - 1) / kd::kDhBN) * split;
    if (dtiles > kMaxProjTiles) return KD_ERR_SHAPE;
  }
  if (p->d % 8 != 0) return KD_ERR_ALIGN;
  return KD_OK;
}

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

// 0 = unknown, 1 = gfx950, 2 = other
std::atomic<int> g_dev_kind[256];

int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 256) return KD_ERR_DEVICE;
  int kind = g_dev_kind[dev].load(std::memory_order_relaxed);
  if (kind == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return KD_ERR_DEVICE;
    kind = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_dev_kind[dev].store(kind, std::memory_order_relaxed);
  }
  return kind == 1 ? KD_OK : KD_ERR_DEVICE;
}

char* ws_base(void* ws) {
  return reinterpret_cast<char*>((reinterpret_cast<uintptr_t>(ws) + kAlign - 1) / kAlign * kAlign);
}

// ---- optional per-kernel event timing (kd_profile.h) ----
struct ProfRec {
  int kind;
  hipEvent_t a, b;
};
std::mutex g_prof_mu;
std::atomic<bool> g_prof_on{false};
std::vector<ProfRec> g_prof_pending;
std::vector<hipEvent_t> g_prof_pool;
double g_prof_ms[KD_K_COUNT];
int64_t g_prof_n[KD_K_COUNT];
const char* const g_prof_names[KD_K_COUNT] = {"prep",      "fwd_proj",       "merge",         "loss_fold",
                                              "bwd_dz",    "bwd_dh",         "dh_reduce",     "bwd_dw",
                                              "dz_cached", "topk_maxima",    "topk_threshold", "topk_collect",
                                              "topk_select", "h_transpose", "h_tile"};

hipEvent_t prof_event() {
  if (!g_prof_pool.empty()) {
    hipEvent_t e = g_prof_pool.back();
    g_prof_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

void prof_drain() {  // caller holds g_prof_mu
  for (const ProfRec& r : g_prof_pending) {
    float ms = 0.f;
    if (hipEventSynchronize(r.b) == hipSuccess && hipEventElapsedTime(&ms, r.a, r.b) == hipSuccess) {
      g_prof_ms[r.kind] += ms;
      g_prof_n[r.kind] += 1;
    }
    g_prof_pool.push_back(r.a);
    g_prof_pool.push_back(r.b);
  }
  g_prof_pending.clear();
}

// Enqueue `launch` on stream `s`, bracketed by events when profiling is on.
template <class F>
void timed(int kind, hipStream_t s, F&& launch) {
  if (!g_prof_on.load(std::memory_order_relaxed)) {
    launch();
    return;
  }
  std::lock_guard<std::mutex> lk(g_prof_mu);
  hipEvent_t a = prof_event(), b = prof_event();
  if (a) (void)hipEventRecord(a, s);
  launch();
  if (b) (void)hipEventRecord(b, s);
  if (a && b) g_prof_pending.push_back({kind, a, b});
}

// The dH and dW GEMMs of a group that ends at chunk `a` (its last), in the
// single-call path: one GEMM each over the dZ rows of all the group's chunks
// (their slots are contiguous), as in the two-call backward, and the H^T
// columns they wrote.  dH keeps one chunk's split of the V reduction, so
// every row's dH is the same as chunk by chunk.
void launch_group_dh_dw(ChunkArgs a, const kd_problem& p, float* dH, float* dW, hipStream_t s) {
  const int64_t group_row0 = a.ht_off;  // rows of the group before chunk `a`
  a.rows = a.ht_off + a.rows;           // rows of the whole group
  a.dz_row0 = 0;
  float* dh = dH - group_row0 * p.d;    // dH of the group's first row (dH points at chunk `a`'s)
  timed(KD_K_BWD_DH, s, [&] { kd::launch_bwd_dh(a, dh, s); });
  if (a.dh_split > 1) timed(KD_K_DH_REDUCE, s, [&] { kd::launch_dh_reduce(a, dh, s); });
  timed(KD_K_BWD_DW, s, [&] { kd::launch_bwd_dw(a, dW, s); });
}

// Arguments of the kernels of `rows` rows from row0 (a chunk, a forward pass
// or a backward group).  `slot` (single-call path, which walks the chunks of
// a dW group one by one) is the chunk's place in its group: its dZ goes to
// slot `slot` of the dZ region and its H^T to the columns from slot * chunk
// (the chunks before it in the group are full).
ChunkArgs chunk_args(const kd_problem& p, const Layout& L, char* base, const void* H, const void* W,
                     const int32_t* ids, const void* logits, const uint8_t* mask, int64_t row0, int rows,
                     bool cached = false, int slot = 0) {
  ChunkArgs a{};
  const size_t xs = p.x_dtype == KD_BF16 ? 2 : 4, ts = p.t_dtype == KD_BF16 ? 2 : 4;
  a.rows = rows;
  a.tau = p.tau == 0.f ? 1.f : p.tau;
  a.d = p.d;
  a.v = p.v;
  a.k = p.k;
  a.nvt = L.nvt;
  a.ldz = L.ldz;
  a.x_bf16 = p.x_dtype == KD_BF16;
  a.t_bf16 = p.t_dtype == KD_BF16;
  a.H = static_cast<const char*>(H) + static_cast<size_t>(row0) * p.d * xs;
  a.W = W;
  a.ids = ids + row0 * p.k;
  a.logits = static_cast<const char*>(logits) + static_cast<size_t>(row0) * p.k * ts;
  a.mask = mask ? mask + row0 : nullptr;
  a.keys = reinterpret_cast<uint32_t*>(base + L.keys);
  a.psort = reinterpret_cast<float*>(base + L.psort);
  a.zgs = reinterpret_cast<float*>(base + L.zgs);
  a.negent = reinterpret_cast<float*>(base + L.negent);
  a.ssum = reinterpret_cast<float*>(base + L.ssum);
  a.lb = reinterpret_cast<uint16_t*>(base + L.lb);
  a.pm = reinterpret_cast<float*>(base + L.pm);
  a.ps = reinterpret_cast<float*>(base + L.ps);
  a.rl = reinterpret_cast<double*>(base + L.rl);
  a.loss_acc = reinterpret_cast<double*>(base + L.loss_acc);
  a.dz = base + L.dz;
  a.dz_row0 = slot * p.chunk;
  a.dhp = reinterpret_cast<float*>(base + L.dhp);
  a.dh_split = L.split;
  a.dh_kslice = L.kslice;
  a.zc = cached ? reinterpret_cast<float*>(base + L.zc) : nullptr;
  a.ht = base + L.ht;
  a.ldt = L.ldt;
  a.hk = base + L.hk;
  a.ldk = L.rows;
  a.ht_off = slot * p.chunk;
  a.ht_span = rows;
  return a;
}

// ---- scratch of kd_chunked_fwd_noalloc ----
// File-scope device array standing in for the caller's workspace.  Each GPU
// the library runs on holds its own copy until the process ends.  In host
// code `scratch` names a host-side stand-in, not the device array: its device
// address is looked up once per device (hipGetSymbolAddress, with that device
// current) and only that address is passed to kernels.
constexpr size_t kScratchBytes = KD_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kScratchBytes];
std::mutex g_scratch_mu;
char* g_scratch_ptr[256];  // per device, null until looked up

int scratch_for_current_device(char** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 256) return KD_ERR_DEVICE;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return KD_ERR_LAUNCH;
    g_scratch_ptr[dev] = static_cast<char*>(ptr);
  }
  *out = g_scratch_ptr[dev];
  return KD_OK;
}

// The forward's chunk walk in passes of `pass_rows` rows (a multiple of the
// chunk, or the chunk), with the kForward layout of one pass at `base`.
void forward_passes(const kd_problem& p, int pass_rows, const void* H, const void* W, const int32_t* t_ids,
                    const void* t_logits, const uint8_t* mask, float* loss, float* lse, float* row_loss,
                    float* zg, char* base, hipStream_t s) {
  kd_problem q = p;
  q.chunk = pass_rows;
  const Layout L = layout_for(q, Mode::kForward);
  const int64_t npass = (p.n + q.chunk - 1) / q.chunk;
  for (int64_t c = 0; c < npass; ++c) {
    const int64_t row0 = c * q.chunk;
    const int rows = static_cast<int>(p.n - row0 < q.chunk ? p.n - row0 : q.chunk);
    const ChunkArgs a = chunk_args(q, L, base, H, W, t_ids, t_logits, mask, row0, rows);
    timed(KD_K_PREP, s, [&] { kd::launch_prep(a, s); });
    timed(KD_K_H_TILE, s, [&] { kd::launch_tile_h(a, s); });
    timed(KD_K_FWD_PROJ, s, [&] { kd::launch_fwd_proj(a, s); });
    timed(KD_K_MERGE, s, [&] {
      kd::launch_merge(a, lse + row0, row_loss ? row_loss + row0 : nullptr, zg ? zg + row0 * p.k : nullptr, s);
    });
    timed(KD_K_LOSS, s, [&] { kd::launch_loss_fold(a, p.chunk, c == 0, c == npass - 1, loss, s); });
  }
}

}  // namespace

extern "C" {

size_t kd_chunked_workspace_size(const kd_problem* prob) {
  if (check_problem(prob) != KD_OK) return 0;
  return layout_for(*prob).total + kAlign;  // slack to align the caller's base
}

const char* kd_status_string(int status) {
  switch (status) {
    case KD_OK: return "KD_OK";
    case KD_ERR_NULL: return "KD_ERR_NULL: a required pointer is NULL";
    case KD_ERR_SHAPE: return "KD_ERR_SHAPE: invalid problem sizes";
    case KD_ERR_DTYPE: return "KD_ERR_DTYPE: unsupported dtype";
    case KD_ERR_ALIGN: return "KD_ERR_ALIGN: d must be a multiple of 8 and tensors 16-byte aligned";
    case KD_ERR_WORKSPACE: return "KD_ERR_WORKSPACE: workspace too small";
    case KD_ERR_DEVICE: return "KD_ERR_DEVICE: current device is not a gfx950 GPU";
    case KD_ERR_LAUNCH: return "KD_ERR_LAUNCH: the HIP runtime reported a launch error";
    default: return "unknown kd_status";
  }
}

int kd_chunked_validate(const kd_problem* prob, const int32_t* t_ids, const uint8_t* mask, int64_t* out,
                        void* stream) {
  int st = check_problem(prob);
  if (st != KD_OK) return st;
  const kd_problem& p = *prob;
  if (!out || (p.n > 0 && !t_ids)) return KD_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(out) & 7u) != 0) return KD_ERR_ALIGN;
  if ((p.n + 3) / 4 > 0x7FFFFFFF) return KD_ERR_SHAPE;  // one wave per row, four per workgroup
  st = check_device();
  if (st != KD_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  kd::launch_validate(t_ids, mask, static_cast<long>(p.n), p.k, p.v, out, s);
  return hipGetLastError() == hipSuccess ? KD_OK : KD_ERR_LAUNCH;
}

int kd_chunked_fwd(const kd_problem* prob, const void* H, const void* W, const int32_t* t_ids,
                   const void* t_logits, const uint8_t* mask, float* loss, float* lse, float* row_loss,
                   float* zg, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_problem(prob);
  if (st != KD_OK) return st;
  const kd_problem& p = *prob;
  if (!loss) return KD_ERR_NULL;
  if (p.n > 0 && (!H || !W || !t_ids || !t_logits || !lse || !workspace)) return KD_ERR_NULL;
  if (p.n > 0 && (!aligned16(H) || !aligned16(W))) return KD_ERR_ALIGN;
  if (p.n > 0 && workspace_bytes < kd_chunked_workspace_size(prob)) return KD_ERR_WORKSPACE;
  st = check_device();
  if (st != KD_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (p.n == 0) {
    kd::launch_zero_loss(loss, s);
    return hipGetLastError() == hipSuccess ? KD_OK : KD_ERR_LAUNCH;
  }
  // passes of up to 8 chunks (fwd_pass_rows), laid out in the same workspace
  forward_passes(p, fwd_pass_rows(p, layout_for(p).total), H, W, t_ids, t_logits, mask, loss, lse, row_loss, zg,
                 ws_base(workspace), s);
  return hipGetLastError() == hipSuccess ? KD_OK : KD_ERR_LAUNCH;
}

int kd_chunked_fwd_noalloc(const kd_problem* prob, const void* H, const void* W, const int32_t* t_ids,
                           const void* t_logits, const uint8_t* mask, float* loss, float* lse, float* row_loss,
                           float* zg, void* stream) {
  int st = check_problem(prob);
  if (st != KD_OK) return st;
  const kd_problem& p = *prob;
  if (!loss) return KD_ERR_NULL;
  if (p.n > 0 && (!H || !W || !t_ids || !t_logits || !lse)) return KD_ERR_NULL;
  if (p.n > 0 && (!aligned16(H) || !aligned16(W))) return KD_ERR_ALIGN;
  if (layout_for(p, Mode::kForward).total > kScratchBytes) return KD_ERR_WORKSPACE;
  st = check_device();
  if (st != KD_OK) return st;
  char* base = nullptr;
  st = scratch_for_current_device(&base);
  if (st != KD_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (p.n == 0) {
    kd::launch_zero_loss(loss, s);
    return hipGetLastError() == hipSuccess ? KD_OK : KD_ERR_LAUNCH;
  }
  // Nothing in the scratch must start at zero: every region the forward
  // reads is written earlier in the same pass (the running loss starts from
  // 0 in the first pass), so what an earlier call left there is never read.
  forward_passes(p, fwd_pass_rows(p, kScratchBytes), H, W, t_ids, t_logits, mask, loss, lse, row_loss, zg, base,
                 s);
  return hipGetLastError() == hipSuccess ? KD_OK : KD_ERR_LAUNCH;
}

int kd_chunked_bwd(const kd_problem* prob, const void* H, const void* W, const int32_t* t_ids,
                   const void* t_logits, const uint8_t* mask, const float* lse, const float* grad_loss,
                   float* dH, float* dW, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_problem(prob);
  if (st != KD_OK) return st;
  const kd_problem& p = *prob;
  if (p.n > 0 && (!H || !W || !t_ids || !t_logits || !lse || !dH || !dW || !workspace)) return KD_ERR_NULL;
  if (p.n > 0 && (!aligned16(H) || !aligned16(W) || !aligned16(dH) || !aligned16(dW))) return KD_ERR_ALIGN;
  if (p.n > 0 && workspace_bytes < kd_chunked_workspace_size(prob)) return KD_ERR_WORKSPACE;
  st = check_device();
  if (st != KD_OK) return st;
  if (p.n == 0) return KD_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const Layout L = layout_for(p);
  char* base = ws_base(workspace);
  // groups of dw_chunks chunks: each kernel runs once over a group's rows
  // (per row the same arithmetic as chunk by chunk; dH keeps one chunk's
  // split of the V reduction), and one dW GEMM reads the group's dZ
  const int64_t unit = L.rows;
  const int64_t ngroups = (p.n + unit - 1) / unit;
  for (int64_t c = 0; c < ngroups; ++c) {
    const int64_t row0 = c * unit;
    const int rows = static_cast<int>(p.n - row0 < unit ? p.n - row0 : unit);
    ChunkArgs a = chunk_args(p, L, base, H, W, t_ids, t_logits, mask, row0, rows);
    a.ht_span = (rows + 31) / 32 * 32;  // H_c^T zero-padded to a whole k tile
    timed(KD_K_PREP, s, [&] { kd::launch_prep(a, s); });
    timed(KD_K_H_TILE, s, [&] { kd::launch_tile_h(a, s); });
    timed(KD_K_BWD_DZ, s, [&] { kd::launch_bwd_dz(a, lse + row0, grad_loss, s); });
    // one dH launch per group: the chunks' launches one by one were slower
    // (measured), as each then reads a dZ the cache no longer holds
    timed(KD_K_BWD_DH, s, [&] { kd::launch_bwd_dh(a, dH + row0 * p.d, s); });
    if (a.dh_split > 1) timed(KD_K_DH_REDUCE, s, [&] { kd::launch_dh_reduce(a, dH + row0 * p.d, s); });
    timed(KD_K_H_TRANSPOSE, s, [&] { kd::launch_transpose_h(a, s); });
    timed(KD_K_BWD_DW, s, [&] { kd::launch_bwd_dw(a, dW, s); });
  }
  return hipGetLastError() == hipSuccess ? KD_OK : KD_ERR_LAUNCH;
}

size_t kd_chunked_fwd_bwd_workspace_size(const kd_problem* prob) {
  if (check_problem(prob) != KD_OK) return 0;
  return layout_for(*prob, Mode::kLossCached).total + kAlign;
}

int kd_chunked_fwd_bwd(const kd_problem* prob, const void* H, const void* W, const int32_t* t_ids,
                       const void* t_logits, const uint8_t* mask, const float* grad_loss, float* loss,
                       float* lse, float* dH, float* dW, void* workspace, size_t workspace_bytes,
                       void* stream) {
  int st = check_problem(prob);
  if (st != KD_OK) return st;
  const kd_problem& p = *prob;
  if (!loss) return KD_ERR_NULL;
  if (p.n > 0 && (!H || !W || !t_ids || !t_logits || !lse || !dH || !dW || !workspace)) return KD_ERR_NULL;
  if (p.n > 0 && (!aligned16(H) || !aligned16(W) || !aligned16(dH) || !aligned16(dW))) return KD_ERR_ALIGN;
  if (p.n > 0 && workspace_bytes < kd_chunked_fwd_bwd_workspace_size(prob)) return KD_ERR_WORKSPACE;
  st = check_device();
  if (st != KD_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (p.n == 0) {
    kd::launch_zero_loss(loss, s);
    return hipGetLastError() == hipSuccess ? KD_OK : KD_ERR_LAUNCH;
  }
  const Layout L = layout_for(p, Mode::kLossCached);
  char* base = ws_base(workspace);
  const int64_t nchunks = (p.n + p.chunk - 1) / p.chunk;
  const int G = dw_group(p);
  for (int64_t c = 0; c < nchunks; ++c) {
    const int64_t row0 = c * p.chunk;
    const int rows = static_cast<int>(p.n - row0 < p.chunk ? p.n - row0 : p.chunk);
    const int slot = static_cast<int>(c % G);
    const bool group_end = slot == G - 1 || c == nchunks - 1;
    ChunkArgs a = chunk_args(p, L, base, H, W, t_ids, t_logits, mask, row0, rows, true, slot);
    if (group_end) a.ht_span = (a.ht_off + rows + 31) / 32 * 32 - a.ht_off;
    timed(KD_K_PREP, s, [&] { kd::launch_prep(a, s); });
    timed(KD_K_H_TILE, s, [&] { kd::launch_tile_h(a, s); });
    timed(KD_K_FWD_PROJ, s, [&] { kd::launch_fwd_proj(a, s); });
    timed(KD_K_MERGE, s, [&] { kd::launch_merge(a, lse + row0, nullptr, nullptr, s); });
    timed(KD_K_LOSS, s, [&] { kd::launch_loss_fold(a, p.chunk, c == 0, c == nchunks - 1, loss, s); });
    timed(KD_K_DZ_CACHED, s, [&] { kd::launch_dz_cached(a, lse + row0, grad_loss, s); });
    timed(KD_K_H_TRANSPOSE, s, [&] { kd::launch_transpose_h(a, s); });
    if (group_end) launch_group_dh_dw(a, p, dH + row0 * p.d, dW, s);
  }
  return hipGetLastError() == hipSuccess ? KD_OK : KD_ERR_LAUNCH;
}

size_t kd_teacher_topk_workspace_size(const kd_problem* prob) {
  if (check_problem(prob) != KD_OK) return 0;
  return layout_for(*prob, Mode::kTopk).total + kAlign;
}

int kd_teacher_topk(const kd_problem* prob, const void* H, const void* W, int32_t* ids, float* logits,
                    int* overflow_rows, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_problem(prob);
  if (st != KD_OK) return st;
  const kd_problem& p = *prob;
  if (p.n > 0 && (!H || !W || !ids || !logits || !workspace)) return KD_ERR_NULL;
  if (p.n > 0 && (!aligned16(H) || !aligned16(W))) return KD_ERR_ALIGN;
  if (p.n > 0 && workspace_bytes < kd_teacher_topk_workspace_size(prob)) return KD_ERR_WORKSPACE;
  st = check_device();
  if (st != KD_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (overflow_rows) kd::launch_fill_u32(reinterpret_cast<uint32_t*>(overflow_rows), 1, 0u, s);
  if (p.n == 0) return hipGetLastError() == hipSuccess ? KD_OK : KD_ERR_LAUNCH;
  const Layout L = layout_for(p, Mode::kTopk);
  char* base = ws_base(workspace);
  uint32_t* lmax = reinterpret_cast<uint32_t*>(base + L.lmax);
  uint32_t* thr = reinterpret_cast<uint32_t*>(base + L.thr);
  int* cnt = reinterpret_cast<int*>(base + L.cnt);
  uint64_t* cand = reinterpret_cast<uint64_t*>(base + L.cand);
  const int64_t nchunks = (p.n + p.chunk - 1) / p.chunk;
  for (int64_t c = 0; c < nchunks; ++c) {
    const int64_t row0 = c * p.chunk;
    const int rows = static_cast<int>(p.n - row0 < p.chunk ? p.n - row0 : p.chunk);
    ChunkArgs a = chunk_args(p, L, base, H, W, nullptr, nullptr, nullptr, 0, rows);
    const size_t xs = p.x_dtype == KD_BF16 ? 2 : 4;
    a.H = static_cast<const char*>(H) + static_cast<size_t>(row0) * p.d * xs;
    timed(KD_K_H_TILE, s, [&] { kd::launch_tile_h(a, s); });
    timed(KD_K_TOPK_MAXIMA, s, [&] { kd::launch_topk_maxima(a, lmax, s); });
    timed(KD_K_TOPK_THRESHOLD, s, [&] { kd::launch_topk_threshold(a, lmax, thr, cnt, s); });
    timed(KD_K_TOPK_COLLECT, s, [&] { kd::launch_topk_collect(a, thr, cnt, cand, s); });
    timed(KD_K_TOPK_SELECT, s, [&] {
      kd::launch_topk_select(a, cnt, cand, ids + row0 * p.k, logits + row0 * p.k, overflow_rows, s);
    });
  }
  return hipGetLastError() == hipSuccess ? KD_OK : KD_ERR_LAUNCH;
}

int kd_profile_enable(int on) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  prof_drain();
  for (int i = 0; i < KD_K_COUNT; ++i) {
    g_prof_ms[i] = 0.0;
    g_prof_n[i] = 0;
  }
  g_prof_on.store(on != 0, std::memory_order_relaxed);
  return KD_OK;
}

int kd_profile_read(int kind, const char** name, double* total_ms, int64_t* launches) {
  if (kind < 0 || kind >= KD_K_COUNT) return KD_ERR_SHAPE;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  prof_drain();
  if (name) *name = g_prof_names[kind];
  if (total_ms) *total_ms = g_prof_ms[kind];
  if (launches) *launches = g_prof_n[kind];
  return KD_OK;
}

}  // extern "C"
