// C ABI of libbeam_moe: argument validation, workspace layout, launch order.
// The contract of every entry point is documented in include/beam_moe.h.
#include <math.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "beam_moe.h"
#include "common.h"
#include "kernels.h"

using namespace beam;

namespace {

constexpr int64_t kMaxT = int64_t(1) << 24;
constexpr int kMaxE = 512;
constexpr int kMaxK = 32;
constexpr int kMaxDim = 32768;
constexpr int64_t kMaxAttnT = int64_t(1) << 16;  // 32-bit load offsets of the projections

// ---------------------------------------------------------------- validation
bool bad_dim64(int v) { return v < 64 || v > kMaxDim || (v % 64) != 0; }
bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

int check_route_dims(int64_t T, int H, int E, int groups, int topk_groups, int k, float scale) {
  if (T < 0 || T > kMaxT || bad_dim64(H)) return BEAM_MOE_ERR_INVALID_DIM;
  if (E < 1 || E > kMaxE || groups < 1 || E % groups != 0 || E / groups < 2)
    return BEAM_MOE_ERR_INVALID_DIM;
  if (topk_groups < 1 || topk_groups > groups) return BEAM_MOE_ERR_INVALID_DIM;
  if (k < 1 || k > kMaxK || k > topk_groups * (E / groups)) return BEAM_MOE_ERR_INVALID_DIM;
  if (!isfinite(scale)) return BEAM_MOE_ERR_INVALID_DIM;
  return BEAM_MOE_OK;
}

int check_forward_dims(int64_t T, int H, int I, int E, int k) {
  if (T < 0 || T > kMaxT || bad_dim64(H) || bad_dim64(I)) return BEAM_MOE_ERR_INVALID_DIM;
  if (E < 1 || E > kMaxE || k < 1 || k > kMaxK) return BEAM_MOE_ERR_INVALID_DIM;
  return BEAM_MOE_OK;
}

// nullable: pointers that may be NULL.
int check_ptrs(std::initializer_list<const void*> required, std::initializer_list<const void*> nullable) {
  for (const void* p : required)
    if (!p) return BEAM_MOE_ERR_NULL_POINTER;
  for (const void* p : required)
    if (misaligned(p)) return BEAM_MOE_ERR_MISALIGNED;
  for (const void* p : nullable)
    if (p && misaligned(p)) return BEAM_MOE_ERR_MISALIGNED;
  return BEAM_MOE_OK;
}

// ---------------------------------------------------------------- workspace
size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

struct Layout {
  size_t zpart, ids, w, counts, offsets, hist, base, sorted, rowof, h, o, xin, y, tctr, total;
  int S;
};

// Route needs only the logit partials; permute only the histograms.
Layout route_layout(int64_t T, int H, int E) {
  Layout L{};
  L.S = router_splits(T, H, E);
  L.zpart = 0;
  L.total = align256((size_t)L.S * T * E * 4);
  return L;
}

Layout perm_layout(int64_t T, int E, int k) {
  Layout L{};
  const size_t NB = (size_t)perm_blocks(T * k);
  L.counts = 0;
  L.hist = align256((size_t)E * 4);
  L.base = L.hist + align256(NB * E * 4);
  L.total = L.base + align256(NB * E * 4);
  return L;
}

Layout layout(int64_t T, int H, int I, int E, int k) {
  Layout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off += align256(bytes);
    return at;
  };
  const size_t Tk = (size_t)T * k;
  const size_t NB = (size_t)perm_blocks((int64_t)Tk);
  L.S = router_splits(T, H, E);
  L.zpart = take((size_t)L.S * T * E * 4);
  L.ids = take(Tk * 4);
  L.w = take(Tk * 4);
  L.counts = take((size_t)E * 4);
  L.offsets = take((size_t)(E + 1) * 4);
  L.hist = take(NB * E * 4);
  L.base = take(NB * E * 4);
  L.sorted = take(Tk * 4);
  L.rowof = take(Tk * 4);
  L.h = take(Tk * (size_t)I * 2);
  L.o = take(Tk * (size_t)H * 4);
  L.xin = take((size_t)T * H * 2);
  L.y = take((size_t)T * H * 2);
  L.tctr = take(16 * 4);  // tile-claim counters: 8 for gate/up, 8 for down
  L.total = off;
  return L;
}

// Attention sublayer workspace (Tp = T rounded up to 128).
struct AttnLayout {
  size_t qkvg, qn, kn, vb, vt, o, vmx, counts, offsets, ctr, total;
};
AttnLayout attn_layout(int64_t T) {
  AttnLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off += align256(bytes);
    return at;
  };
  const size_t Tp = (size_t)((T + 127) / 128 * 128);
  L.qkvg = take((size_t)T * kAttnProjRows * 4);
  L.qn = take((size_t)kAttnQHeads * Tp * kAttnHeadDim * 2);
  L.kn = take((size_t)kAttnKVHeads * Tp * kAttnHeadDim * 2);
  L.vb = take((size_t)T * kAttnKVHeads * kAttnHeadDim * 2);
  L.vt = take((size_t)kAttnKVHeads * kAttnHeadDim * Tp * 2);
  L.o = take((size_t)T * kAttnQHeads * kAttnHeadDim * 2);
  L.vmx = take((size_t)T * kAttnKVHeads * 4);
  L.counts = take(4);
  L.offsets = take(8);
  L.ctr = take(32 * 4);
  L.total = off;
  return L;
}

// ---------------------------------------------------------------- device
struct DevInfo {
  std::atomic<int> state{0};  // 0 unknown, 1 ok, -1 unsupported
  int num_cu = 256;
};
DevInfo g_dev[64];
std::mutex g_dev_mu;

int device_check(int* num_cu) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return BEAM_MOE_ERR_HIP;
  DevInfo& d = g_dev[dev];
  int s = d.state.load(std::memory_order_acquire);
  if (s == 0) {
    std::lock_guard<std::mutex> lk(g_dev_mu);
    s = d.state.load(std::memory_order_relaxed);
    if (s == 0) {
      hipDeviceProp_t p;
      if (hipGetDeviceProperties(&p, dev) != hipSuccess) return BEAM_MOE_ERR_HIP;
      d.num_cu = p.multiProcessorCount;
      s = (strncmp(p.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
      d.state.store(s, std::memory_order_release);
    }
  }
  if (s < 0) return BEAM_MOE_ERR_UNSUPPORTED_DEVICE;
  *num_cu = d.num_cu;
  return BEAM_MOE_OK;
}

// ---------------------------------------------------------------- static scratch
// Workspace of beam_moe_block_noalloc, for callers that cannot allocate: a
// device array of BEAM_MOE_NOALLOC_SCRATCH_BYTES that every GPU the library
// runs on holds until the process ends.  In host code `scratch` names a host
// stand-in, not device memory: the device address comes from
// hipGetSymbolAddress, once per device with that device current, and only
// that address is ever handed to a kernel.
static __device__ __align__(256) unsigned char scratch[BEAM_MOE_NOALLOC_SCRATCH_BYTES];

std::atomic<void*> g_scratch_ptr[64];
std::mutex g_scratch_mu;

int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return BEAM_MOE_ERR_HIP;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return BEAM_MOE_ERR_HIP;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return BEAM_MOE_OK;
}

// ---------------------------------------------------------------- schedule knob
std::atomic<int> g_schedule{0};  // 0 auto, 1 stream, 2 tiled

// The tiled kernels address one expert's packed weight matrix and the
// activation tensor with 32-bit buffer offsets; larger tensors take the
// streaming path.
bool tiled_fits(int64_t T, int H, int I, int k) {
  const int64_t lim = int64_t(1) << 31;
  return packed_expert_bytes(I, H) < lim && packed_expert_bytes(H, I) < lim && T * H * 2 < lim &&
         T * k * I * 2 < lim;
}

bool use_stream(int64_t T, int H, int I, int k, int E) {
  if (!tiled_fits(T, H, I, k)) return true;
  const int m = g_schedule.load(std::memory_order_relaxed);
  if (m == 1) return true;
  if (m == 2) return false;
  // measured crossover at Beam shape: the streaming schedule wins up to ~16
  // assignments per expert on average (T = 512), the tiled one from ~24 (T = 768)
  return (double)T * k < 20.0 * E;
}

// ---------------------------------------------------------------- stage timer
enum Stage { ST_LOGITS, ST_SELECT, ST_PERMUTE, ST_GATEUP, ST_DOWN, ST_COMBINE,
             ST_ATT_PROJ, ST_ATT_PREP, ST_ATT_FLASH, ST_ATT_OUT, NST };
const char* kStageNames[NST] = {"router_logits", "select", "permute", "gateup", "down", "combine",
                                "attn_proj", "attn_prep", "attn_flash", "attn_out"};

struct Timer {
  std::mutex mu;
  bool on = false;
  unsigned mask = 0;           // stages that record events
  int max_calls = 0, n_calls = 0;
  std::vector<hipEvent_t> ev;  // [call][stage][2]
  std::vector<char> used;      // [call][stage]
} g_timer;

int timer_claim() {
  std::lock_guard<std::mutex> lk(g_timer.mu);
  if (!g_timer.on || g_timer.n_calls >= g_timer.max_calls) return -1;
  return g_timer.n_calls++;
}

struct StageScope {
  int slot, stage;
  hipStream_t st;
  StageScope(int slot_, int stage_, hipStream_t st_) : slot(slot_), stage(stage_), st(st_) {
    // mask is set before `on`, under the lock that timer_claim takes
    if (slot >= 0 && !((g_timer.mask >> stage) & 1u)) slot = -1;
    if (slot >= 0) {
      (void)hipEventRecord(g_timer.ev[(size_t)(slot * NST + stage) * 2], st);
      g_timer.used[(size_t)slot * NST + stage] = 1;
    }
  }
  ~StageScope() {
    if (slot >= 0) (void)hipEventRecord(g_timer.ev[(size_t)(slot * NST + stage) * 2 + 1], st);
  }
};

#define BEAM_TRY(expr)                                     \
  do {                                                     \
    if ((expr) != hipSuccess) return BEAM_MOE_ERR_HIP;     \
  } while (0)

// ---------------------------------------------------------------- pipelines
int run_route(hipStream_t st, int64_t T, int H, int E, int groups, int topk_groups, int k, float scale,
              const uint16_t* x, const uint16_t* wr, const float* off, int32_t* ids, float* w,
              int32_t* user_counts, const Layout& L, char* ws, int slot) {
  float* zpart = reinterpret_cast<float*>(ws + L.zpart);
  {
    StageScope sc(slot, ST_LOGITS, st);
    BEAM_TRY(launch_router_logits(st, x, wr, zpart, (int)T, H, E, L.S));
  }
  {
    StageScope sc(slot, ST_SELECT, st);
    if (user_counts) BEAM_TRY(launch_fill_i32(st, user_counts, E, 0));
    BEAM_TRY(launch_select(st, zpart, L.S, off, (int)T, E, groups, topk_groups, k, scale, ids, w,
                           user_counts));
  }
  return BEAM_MOE_OK;
}

int run_permute(hipStream_t st, int64_t T, int E, int k, const int32_t* ids, int32_t* user_counts,
                const Layout& L, char* ws, int32_t* offsets_out, int32_t* sorted_out, int32_t* rowof_out,
                int32_t* clear16 = nullptr) {
  const int64_t Tk = T * k;
  BEAM_TRY(launch_permute(st, ids, Tk, k, E, reinterpret_cast<int32_t*>(ws + L.hist),
                          reinterpret_cast<int32_t*>(ws + L.base), reinterpret_cast<int32_t*>(ws + L.counts),
                          offsets_out, sorted_out, rowof_out, user_counts, clear16));
  return BEAM_MOE_OK;
}

// Expert weights as the kernels take them: packed bf16 (scales NULL) or
// packed FP8 codes with per-row scales.
struct Experts {
  const uint16_t *wg, *wu, *wd;
  const float *sg, *su, *sd;
};

// exact_rows: every row of the single matrix (E = 1, k = 1) is used, so the
// tiled GEMMs may pick their token-tile count from T.
int run_forward(hipStream_t st, int64_t T, int H, int I, int E, int k, const uint16_t* x,
                const int32_t* ids, const float* w, const Experts& ex, uint16_t* y,
                int32_t* user_counts, const Layout& L, char* ws, int slot, int num_cu,
                bool exact_rows = false) {
  const bool one = exact_rows && E == 1 && k == 1;
  const int64_t Tk = T * k;
  int32_t* counts = reinterpret_cast<int32_t*>(ws + L.counts);
  int32_t* offsets = reinterpret_cast<int32_t*>(ws + L.offsets);
  int32_t* sorted = reinterpret_cast<int32_t*>(ws + L.sorted);
  int32_t* rowof = reinterpret_cast<int32_t*>(ws + L.rowof);
  uint16_t* h = reinterpret_cast<uint16_t*>(ws + L.h);
  float* o = reinterpret_cast<float*>(ws + L.o);
  const bool stream = use_stream(T, H, I, k, E);
  int32_t* tctr = reinterpret_cast<int32_t*>(ws + L.tctr);
  {
    // the tiled GEMMs' tile-claim counters start at 0: cleared by the
    // permutation's scan workgroup (a kernel store, not a memset: graph-safe)
    StageScope sc(slot, ST_PERMUTE, st);
    int rc = run_permute(st, T, E, k, ids, user_counts, L, ws, offsets, sorted, rowof,
                         stream ? nullptr : tctr);
    if (rc) return rc;
  }
  {
    StageScope sc(slot, ST_GATEUP, st);
    GroupedArgs a{x, sorted, ex.wg, ex.wu, ex.sg, ex.su, counts, offsets, h, I, H, E, Tk, tctr};
    if (one) a.m_tiles = tiled_token_tiles(T, I, 2, num_cu);
    BEAM_TRY(stream ? launch_gateup_stream(st, a, T, k) : launch_gateup_tiled(st, a, num_cu));
  }
  {
    StageScope sc(slot, ST_DOWN, st);
    GroupedArgs a{h, nullptr, ex.wd, nullptr, ex.sd, nullptr, counts, offsets, o, H, I, E, Tk, tctr + 8};
    if (one) a.m_tiles = tiled_token_tiles(T, H, 1, num_cu);
    BEAM_TRY(stream ? launch_down_stream(st, a, T, k) : launch_down_tiled(st, a, num_cu));
  }
  {
    StageScope sc(slot, ST_COMBINE, st);
    BEAM_TRY(launch_combine(st, o, rowof, w, (int)T, H, k, y));
  }
  return BEAM_MOE_OK;
}

}  // namespace

// ============================================================================
// Public entry points
// ============================================================================
extern "C" {

const char* beam_moe_status_string(int status) {
  switch (status) {
    case BEAM_MOE_OK: return "ok";
    case BEAM_MOE_ERR_INVALID_DIM: return "invalid dimension";
    case BEAM_MOE_ERR_NULL_POINTER: return "null pointer";
    case BEAM_MOE_ERR_MISALIGNED: return "pointer not 16-byte aligned";
    case BEAM_MOE_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case BEAM_MOE_ERR_UNSUPPORTED_DEVICE: return "unsupported device (needs gfx950)";
    case BEAM_MOE_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* beam_moe_version(void) { return "0.1.0"; }

size_t beam_moe_packed_weight_bytes(int N, int K) {
  if (bad_dim64(N) || bad_dim64(K)) return 0;
  return (size_t)packed_expert_bytes(N, K);
}

int beam_moe_pack_weights(void* stream, int E, int N, int K, const uint16_t* src, uint16_t* dst) {
  if (E < 1 || E > kMaxE || bad_dim64(N) || bad_dim64(K)) return BEAM_MOE_ERR_INVALID_DIM;
  int rc = check_ptrs({src, dst}, {});
  if (rc) return rc;
  // the source and the packed copy must not overlap
  const char* s0 = reinterpret_cast<const char*>(src);
  const char* d0 = reinterpret_cast<const char*>(dst);
  const int64_t sb = (int64_t)E * N * K * 2, db = (int64_t)E * packed_expert_bytes(N, K);
  if (s0 < d0 + db && d0 < s0 + sb) return BEAM_MOE_ERR_INVALID_DIM;
  int num_cu;
  if ((rc = device_check(&num_cu))) return rc;
  return launch_pack((hipStream_t)stream, src, dst, E, N, K) == hipSuccess ? BEAM_MOE_OK
                                                                           : BEAM_MOE_ERR_HIP;
}

size_t beam_moe_packed_fp8_bytes(int N, int K) {
  if (bad_dim64(N) || bad_dim64(K)) return 0;
  return (size_t)packed8_expert_bytes(N, K);
}

int beam_moe_pack_weights_fp8(void* stream, int E, int N, int K, const uint16_t* src,
                              uint8_t* dst, float* scales) {
  if (E < 1 || E > kMaxE || bad_dim64(N) || bad_dim64(K)) return BEAM_MOE_ERR_INVALID_DIM;
  int rc = check_ptrs({src, dst, scales}, {});
  if (rc) return rc;
  const char* s0 = reinterpret_cast<const char*>(src);
  const int64_t sb = (int64_t)E * N * K * 2;
  const char* d0 = reinterpret_cast<const char*>(dst);
  const int64_t db = (int64_t)E * packed8_expert_bytes(N, K);
  const char* c0 = reinterpret_cast<const char*>(scales);
  const int64_t cb = (int64_t)E * N * 4;
  if ((s0 < d0 + db && d0 < s0 + sb) || (s0 < c0 + cb && c0 < s0 + sb) || (d0 < c0 + cb && c0 < d0 + db))
    return BEAM_MOE_ERR_INVALID_DIM;
  int num_cu;
  if ((rc = device_check(&num_cu))) return rc;
  return launch_pack_fp8((hipStream_t)stream, src, dst, scales, E, N, K) == hipSuccess
             ? BEAM_MOE_OK
             : BEAM_MOE_ERR_HIP;
}

size_t beam_moe_workspace_bytes(int64_t T, int H, int I, int E, int k) {
  if (check_forward_dims(T, H, I, E, k) != BEAM_MOE_OK) return 0;
  return layout(T, H, I, E, k).total;
}

int beam_moe_route(void* stream, int64_t T, int H, int E, int groups, int topk_groups, int k,
                   float scale, const uint16_t* x, const uint16_t* w_router,
                   const float* logit_offset, int32_t* topk_ids, float* topk_weights,
                   int32_t* expert_counts, void* workspace, size_t workspace_bytes) {
  int rc = check_route_dims(T, H, E, groups, topk_groups, k, scale);
  if (rc) return rc;
  if (T == 0) return BEAM_MOE_OK;
  rc = check_ptrs({x, w_router, topk_ids, topk_weights, workspace}, {logit_offset, expert_counts});
  if (rc) return rc;
  const Layout L = route_layout(T, H, E);
  if (workspace_bytes < L.total) return BEAM_MOE_ERR_WORKSPACE_TOO_SMALL;
  int num_cu;
  if ((rc = device_check(&num_cu))) return rc;
  return run_route((hipStream_t)stream, T, H, E, groups, topk_groups, k, scale, x, w_router,
                   logit_offset, topk_ids, topk_weights, expert_counts, L,
                   static_cast<char*>(workspace), -1);
}

int beam_moe_permute(void* stream, int64_t T, int E, int k, const int32_t* topk_ids,
                     int32_t* expert_counts, int32_t* expert_offsets, int32_t* sorted_tokens,
                     int32_t* row_of, void* workspace, size_t workspace_bytes) {
  if (T < 0 || T > kMaxT || E < 1 || E > kMaxE || k < 1 || k > kMaxK) return BEAM_MOE_ERR_INVALID_DIM;
  if (T == 0) return BEAM_MOE_OK;
  int rc = check_ptrs({topk_ids, expert_counts, expert_offsets, sorted_tokens, row_of, workspace}, {});
  if (rc) return rc;
  const Layout L = perm_layout(T, E, k);
  if (workspace_bytes < L.total) return BEAM_MOE_ERR_WORKSPACE_TOO_SMALL;
  int num_cu;
  if ((rc = device_check(&num_cu))) return rc;
  return run_permute((hipStream_t)stream, T, E, k, topk_ids, expert_counts, L,
                     static_cast<char*>(workspace), expert_offsets, sorted_tokens, row_of);
}

int beam_moe_forward(void* stream, int64_t T, int H, int I, int E, int k, const uint16_t* x,
                     const int32_t* topk_ids, const float* topk_weights, const uint16_t* w_gate,
                     const uint16_t* w_up, const uint16_t* w_down, uint16_t* y,
                     int32_t* expert_counts, void* workspace, size_t workspace_bytes) {
  int rc = check_forward_dims(T, H, I, E, k);
  if (rc) return rc;
  if (T == 0) return BEAM_MOE_OK;
  rc = check_ptrs({x, topk_ids, topk_weights, w_gate, w_up, w_down, y, workspace}, {expert_counts});
  if (rc) return rc;
  const Layout L = layout(T, H, I, E, k);
  if (workspace_bytes < L.total) return BEAM_MOE_ERR_WORKSPACE_TOO_SMALL;
  int num_cu;
  if ((rc = device_check(&num_cu))) return rc;
  const int slot = timer_claim();
  const Experts ex{w_gate, w_up, w_down, nullptr, nullptr, nullptr};
  return run_forward((hipStream_t)stream, T, H, I, E, k, x, topk_ids, topk_weights, ex, y,
                     expert_counts, L, static_cast<char*>(workspace), slot, num_cu);
}

int beam_moe_forward_fp8(void* stream, int64_t T, int H, int I, int E, int k, const uint16_t* x,
                         const int32_t* topk_ids, const float* topk_weights,
                         const uint8_t* w_gate, const float* s_gate, const uint8_t* w_up,
                         const float* s_up, const uint8_t* w_down, const float* s_down,
                         uint16_t* y, int32_t* expert_counts, void* workspace,
                         size_t workspace_bytes) {
  int rc = check_forward_dims(T, H, I, E, k);
  if (rc) return rc;
  if (T == 0) return BEAM_MOE_OK;
  rc = check_ptrs({x, topk_ids, topk_weights, w_gate, s_gate, w_up, s_up, w_down, s_down, y,
                   workspace},
                  {expert_counts});
  if (rc) return rc;
  const Layout L = layout(T, H, I, E, k);
  if (workspace_bytes < L.total) return BEAM_MOE_ERR_WORKSPACE_TOO_SMALL;
  int num_cu;
  if ((rc = device_check(&num_cu))) return rc;
  const int slot = timer_claim();
  const Experts ex{reinterpret_cast<const uint16_t*>(w_gate), reinterpret_cast<const uint16_t*>(w_up),
                   reinterpret_cast<const uint16_t*>(w_down), s_gate, s_up, s_down};
  return run_forward((hipStream_t)stream, T, H, I, E, k, x, topk_ids, topk_weights, ex, y,
                     expert_counts, L, static_cast<char*>(workspace), slot, num_cu);
}

}  // extern "C"

namespace {
int block_common(void* stream, int64_t T, int H, int I, int E, int groups, int topk_groups, int k,
                 float scale, const uint16_t* x, const uint16_t* w_router,
                 const float* logit_offset, const Experts& ex, uint16_t* y, int32_t* topk_ids,
                 float* topk_weights, int32_t* expert_counts, void* workspace,
                 size_t workspace_bytes) {
  int rc = check_route_dims(T, H, E, groups, topk_groups, k, scale);
  if (rc) return rc;
  if ((rc = check_forward_dims(T, H, I, E, k))) return rc;
  if (T == 0) return BEAM_MOE_OK;
  rc = check_ptrs({x, w_router, ex.wg, ex.wu, ex.wd, y, workspace},
                  {logit_offset, topk_ids, topk_weights, expert_counts});
  if (rc) return rc;
  if (ex.sg && (rc = check_ptrs({ex.sg, ex.su, ex.sd}, {}))) return rc;
  const Layout L = layout(T, H, I, E, k);
  if (workspace_bytes < L.total) return BEAM_MOE_ERR_WORKSPACE_TOO_SMALL;
  int num_cu;
  if ((rc = device_check(&num_cu))) return rc;
  char* ws = static_cast<char*>(workspace);
  int32_t* ids = topk_ids ? topk_ids : reinterpret_cast<int32_t*>(ws + L.ids);
  float* w = topk_weights ? topk_weights : reinterpret_cast<float*>(ws + L.w);
  hipStream_t st = (hipStream_t)stream;
  const int slot = timer_claim();
  rc = run_route(st, T, H, E, groups, topk_groups, k, scale, x, w_router, logit_offset, ids, w,
                 nullptr, L, ws, slot);
  if (rc) return rc;
  return run_forward(st, T, H, I, E, k, x, ids, w, ex, y, expert_counts, L, ws, slot, num_cu);
}
}  // namespace

extern "C" {

int beam_moe_block(void* stream, int64_t T, int H, int I, int E, int groups, int topk_groups, int k,
                   float scale, const uint16_t* x, const uint16_t* w_router,
                   const float* logit_offset, const uint16_t* w_gate, const uint16_t* w_up,
                   const uint16_t* w_down, uint16_t* y, int32_t* topk_ids, float* topk_weights,
                   int32_t* expert_counts, void* workspace, size_t workspace_bytes) {
  const Experts ex{w_gate, w_up, w_down, nullptr, nullptr, nullptr};
  return block_common(stream, T, H, I, E, groups, topk_groups, k, scale, x, w_router, logit_offset,
                      ex, y, topk_ids, topk_weights, expert_counts, workspace, workspace_bytes);
}

int beam_moe_block_fp8(void* stream, int64_t T, int H, int I, int E, int groups, int topk_groups,
                       int k, float scale, const uint16_t* x, const uint16_t* w_router,
                       const float* logit_offset, const uint8_t* w_gate, const float* s_gate,
                       const uint8_t* w_up, const float* s_up, const uint8_t* w_down,
                       const float* s_down, uint16_t* y, int32_t* topk_ids, float* topk_weights,
                       int32_t* expert_counts, void* workspace, size_t workspace_bytes) {
  if (!s_gate || !s_up || !s_down) {
    const int rc = check_route_dims(T, H, E, groups, topk_groups, k, scale);
    if (rc) return rc;
    if (check_forward_dims(T, H, I, E, k)) return BEAM_MOE_ERR_INVALID_DIM;
    if (T == 0) return BEAM_MOE_OK;
    return BEAM_MOE_ERR_NULL_POINTER;
  }
  const Experts ex{reinterpret_cast<const uint16_t*>(w_gate), reinterpret_cast<const uint16_t*>(w_up),
                   reinterpret_cast<const uint16_t*>(w_down), s_gate, s_up, s_down};
  return block_common(stream, T, H, I, E, groups, topk_groups, k, scale, x, w_router, logit_offset,
                      ex, y, topk_ids, topk_weights, expert_counts, workspace, workspace_bytes);
}

int beam_moe_block_noalloc(void* stream, int64_t T, int H, int I, int E, int groups,
                           int topk_groups, int k, float scale, const uint16_t* x,
                           const uint16_t* w_router, const float* logit_offset,
                           const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_down,
                           uint16_t* y, int32_t* topk_ids, float* topk_weights,
                           int32_t* expert_counts) {
  int rc = check_route_dims(T, H, E, groups, topk_groups, k, scale);
  if (rc) return rc;
  if ((rc = check_forward_dims(T, H, I, E, k))) return rc;
  if (T == 0) return BEAM_MOE_OK;
  if (layout(T, H, I, E, k).total > (size_t)BEAM_MOE_NOALLOC_SCRATCH_BYTES)
    return BEAM_MOE_ERR_WORKSPACE_TOO_SMALL;
  rc = check_ptrs({x, w_router, w_gate, w_up, w_down, y},
                  {logit_offset, topk_ids, topk_weights, expert_counts});
  if (rc) return rc;
  int num_cu;
  if ((rc = device_check(&num_cu))) return rc;
  void* ws = nullptr;
  if ((rc = scratch_address(&ws))) return rc;
  const Experts ex{w_gate, w_up, w_down, nullptr, nullptr, nullptr};
  return block_common(stream, T, H, I, E, groups, topk_groups, k, scale, x, w_router, logit_offset,
                      ex, y, topk_ids, topk_weights, expert_counts, ws,
                      (size_t)BEAM_MOE_NOALLOC_SCRATCH_BYTES);
}

int beam_moe_stream_init(void* stream, int64_t T, int H, const uint16_t* x, float* stream_out) {
  if (T < 0 || T > kMaxT || bad_dim64(H)) return BEAM_MOE_ERR_INVALID_DIM;
  if (T == 0) return BEAM_MOE_OK;
  int rc = check_ptrs({x, stream_out}, {});
  if (rc) return rc;
  int num_cu;
  if ((rc = device_check(&num_cu))) return rc;
  BEAM_TRY(launch_stream_init((hipStream_t)stream, x, stream_out, T, H));
  return BEAM_MOE_OK;
}

int beam_moe_rmsnorm(void* stream, int64_t T, int H, float eps, const float* in, uint16_t* out) {
  if (T < 0 || T > kMaxT || bad_dim64(H) || !(eps >= 0.f) || !isfinite(eps)) return BEAM_MOE_ERR_INVALID_DIM;
  if (T == 0) return BEAM_MOE_OK;
  int rc = check_ptrs({in, out}, {});
  if (rc) return rc;
  int num_cu;
  if ((rc = device_check(&num_cu))) return rc;
  BEAM_TRY(launch_rmsnorm((hipStream_t)stream, in, out, T, H, eps));
  return BEAM_MOE_OK;
}

int beam_moe_residual_update(void* stream, int64_t T, int H, float eps, int step, const uint16_t* y,
                             float* stream_io) {
  if (T < 0 || T > kMaxT || bad_dim64(H) || step < 2 || !(eps >= 0.f) || !isfinite(eps))
    return BEAM_MOE_ERR_INVALID_DIM;
  if (T == 0) return BEAM_MOE_OK;
  int rc = check_ptrs({y, stream_io}, {});
  if (rc) return rc;
  int num_cu;
  if ((rc = device_check(&num_cu))) return rc;
  BEAM_TRY(launch_residual((hipStream_t)stream, y, stream_io, T, H, eps, step));
  return BEAM_MOE_OK;
}

}  // extern "C"

namespace {
int sublayer_common(void* stream, int64_t T, int H, int I, int E, int groups, int topk_groups, int k,
                    float scale, float eps, int step, float* stream_io, const uint16_t* w_router,
                    const Experts& ex, uint16_t* moe_input, uint16_t* moe_output, int32_t* topk_ids,
                    float* topk_weights, int32_t* expert_counts, void* workspace,
                    size_t workspace_bytes) {
  int rc = check_route_dims(T, H, E, groups, topk_groups, k, scale);
  if (rc) return rc;
  if ((rc = check_forward_dims(T, H, I, E, k))) return rc;
  if (step < 2 || !(eps >= 0.f) || !isfinite(eps)) return BEAM_MOE_ERR_INVALID_DIM;
  if (T == 0) return BEAM_MOE_OK;
  rc = check_ptrs({stream_io, w_router, ex.wg, ex.wu, ex.wd, workspace},
                  {moe_input, moe_output, topk_ids, topk_weights, expert_counts});
  if (rc) return rc;
  if (ex.sg && (rc = check_ptrs({ex.sg, ex.su, ex.sd}, {}))) return rc;
  const Layout L = layout(T, H, I, E, k);
  if (workspace_bytes < L.total) return BEAM_MOE_ERR_WORKSPACE_TOO_SMALL;
  int num_cu;
  if ((rc = device_check(&num_cu))) return rc;
  char* ws = static_cast<char*>(workspace);
  hipStream_t st = (hipStream_t)stream;
  uint16_t* xin = moe_input ? moe_input : reinterpret_cast<uint16_t*>(ws + L.xin);
  uint16_t* yb = moe_output ? moe_output : reinterpret_cast<uint16_t*>(ws + L.y);
  int32_t* ids = topk_ids ? topk_ids : reinterpret_cast<int32_t*>(ws + L.ids);
  float* w = topk_weights ? topk_weights : reinterpret_cast<float*>(ws + L.w);
  BEAM_TRY(launch_rmsnorm(st, stream_io, xin, T, H, eps));
  const int slot = timer_claim();
  rc = run_route(st, T, H, E, groups, topk_groups, k, scale, xin, w_router, nullptr, ids, w, nullptr,
                 L, ws, slot);
  if (rc) return rc;
  rc = run_forward(st, T, H, I, E, k, xin, ids, w, ex, yb, expert_counts, L, ws,
                   slot, num_cu);
  if (rc) return rc;
  BEAM_TRY(launch_residual(st, yb, stream_io, T, H, eps, step));
  return BEAM_MOE_OK;
}
}  // namespace

extern "C" {

int beam_moe_sublayer(void* stream, int64_t T, int H, int I, int E, int groups, int topk_groups, int k,
                      float scale, float eps, int step, float* stream_io, const uint16_t* w_router,
                      const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_down,
                      uint16_t* moe_input, uint16_t* moe_output, int32_t* topk_ids,
                      float* topk_weights, int32_t* expert_counts, void* workspace,
                      size_t workspace_bytes) {
  const Experts ex{w_gate, w_up, w_down, nullptr, nullptr, nullptr};
  return sublayer_common(stream, T, H, I, E, groups, topk_groups, k, scale, eps, step, stream_io,
                         w_router, ex, moe_input, moe_output, topk_ids, topk_weights, expert_counts,
                         workspace, workspace_bytes);
}

int beam_moe_sublayer_fp8(void* stream, int64_t T, int H, int I, int E, int groups, int topk_groups,
                          int k, float scale, float eps, int step, float* stream_io,
                          const uint16_t* w_router, const uint8_t* w_gate, const float* s_gate,
                          const uint8_t* w_up, const float* s_up, const uint8_t* w_down,
                          const float* s_down, uint16_t* moe_input, uint16_t* moe_output,
                          int32_t* topk_ids, float* topk_weights, int32_t* expert_counts,
                          void* workspace, size_t workspace_bytes) {
  if (!s_gate || !s_up || !s_down) return BEAM_MOE_ERR_NULL_POINTER;
  const Experts ex{reinterpret_cast<const uint16_t*>(w_gate), reinterpret_cast<const uint16_t*>(w_up),
                   reinterpret_cast<const uint16_t*>(w_down), s_gate, s_up, s_down};
  return sublayer_common(stream, T, H, I, E, groups, topk_groups, k, scale, eps, step, stream_io,
                         w_router, ex, moe_input, moe_output, topk_ids, topk_weights, expert_counts,
                         workspace, workspace_bytes);
}

// ---------------------------------------------------------------- schedule / timer
int beam_moe_set_schedule(int mode) {
  if (mode < 0 || mode > 2) return BEAM_MOE_ERR_INVALID_DIM;
  g_schedule.store(mode, std::memory_order_relaxed);
  return BEAM_MOE_OK;
}

// the projections' 32-bit activation offsets: u [T, H] and o [T, 6144] bf16
bool attn_bad_dims(int64_t T, int H) {
  return T < 0 || T > kMaxAttnT || bad_dim64(H) || T * H * 2 >= (int64_t(1) << 31);
}

size_t beam_attn_workspace_bytes(int64_t T, int H) {
  if (attn_bad_dims(T, H)) return 0;
  return attn_layout(T).total;
}

int beam_attn_forward(void* stream, int64_t T, int H, int global_layer, int window, float theta,
                      const uint16_t* u, const uint16_t* w_qkvg, const uint16_t* w_o, uint16_t* y,
                      void* workspace, size_t workspace_bytes) {
  if (attn_bad_dims(T, H)) return BEAM_MOE_ERR_INVALID_DIM;
  if (global_layer != 0 && global_layer != 1) return BEAM_MOE_ERR_INVALID_DIM;
  if (!global_layer && window < 1) return BEAM_MOE_ERR_INVALID_DIM;
  if (!global_layer && !(isfinite(theta) && theta > 0.f)) return BEAM_MOE_ERR_INVALID_DIM;
  if (T == 0) return BEAM_MOE_OK;
  int rc = check_ptrs({u, w_qkvg, w_o, y, workspace}, {});
  if (rc) return rc;
  const AttnLayout L = attn_layout(T);
  if (workspace_bytes < L.total) return BEAM_MOE_ERR_WORKSPACE_TOO_SMALL;
  int num_cu;
  if ((rc = device_check(&num_cu))) return rc;
  const int slot = timer_claim();
  char* ws = static_cast<char*>(workspace);
  AttnArgs a{T, H, global_layer, window, theta, u, w_qkvg, w_o, y,
             reinterpret_cast<float*>(ws + L.qkvg), reinterpret_cast<uint16_t*>(ws + L.qn),
             reinterpret_cast<uint16_t*>(ws + L.kn), reinterpret_cast<uint16_t*>(ws + L.vb),
             reinterpret_cast<uint16_t*>(ws + L.vt), reinterpret_cast<uint16_t*>(ws + L.o),
             reinterpret_cast<float*>(ws + L.vmx),
             reinterpret_cast<int32_t*>(ws + L.counts), reinterpret_cast<int32_t*>(ws + L.offsets),
             reinterpret_cast<int32_t*>(ws + L.ctr)};
  hipStream_t st = (hipStream_t)stream;
  {
    StageScope sc(slot, ST_ATT_PROJ, st);
    BEAM_TRY(launch_attn_proj(st, a, num_cu));
  }
  {
    StageScope sc(slot, ST_ATT_PREP, st);
    BEAM_TRY(launch_attn_prep(st, a));
  }
  {
    StageScope sc(slot, ST_ATT_FLASH, st);
    BEAM_TRY(launch_attn_flash(st, a));
  }
  {
    StageScope sc(slot, ST_ATT_OUT, st);
    BEAM_TRY(launch_attn_out(st, a, num_cu));
  }
  return BEAM_MOE_OK;
}

}  // extern "C"

// ---- dense SwiGLU layer as C chunks of its intermediate dimension
namespace {
int check_dense_dims(int64_t T, int H, int I, int C) {
  if (C < 1 || C > kMaxK || I % C != 0) return BEAM_MOE_ERR_INVALID_DIM;
  return check_forward_dims(T, H, I / C, C, C);
}

// dims and pointers checked by the caller; T > 0
int dense_common(void* stream, int64_t T, int H, int I, int C, const uint16_t* x, const Experts& ex,
                 uint16_t* y, void* workspace, size_t workspace_bytes) {
  const int Ic = I / C;
  const Layout L = layout(T, H, Ic, C, C);
  if (workspace_bytes < L.total) return BEAM_MOE_ERR_WORKSPACE_TOO_SMALL;
  int num_cu, rc;
  if ((rc = device_check(&num_cu))) return rc;
  const int slot = timer_claim();
  hipStream_t st = (hipStream_t)stream;
  char* ws = static_cast<char*>(workspace);
  int32_t* ids = reinterpret_cast<int32_t*>(ws + L.ids);
  float* w = reinterpret_cast<float*>(ws + L.w);
  {
    StageScope sc(slot, ST_SELECT, st);
    BEAM_TRY(launch_dense_routing(st, ids, w, T, C));
  }
  return run_forward(st, T, H, Ic, C, C, x, ids, w, ex, y, nullptr, L, ws, slot, num_cu,
                     /*exact_rows=*/true);
}
}  // namespace

extern "C" {

size_t beam_dense_workspace_bytes(int64_t T, int H, int I, int chunks) {
  if (check_dense_dims(T, H, I, chunks) != BEAM_MOE_OK) return 0;
  return layout(T, H, I / chunks, chunks, chunks).total;
}

int beam_dense_mlp(void* stream, int64_t T, int H, int I, int chunks, const uint16_t* x,
                   const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_down, uint16_t* y,
                   void* workspace, size_t workspace_bytes) {
  int rc = check_dense_dims(T, H, I, chunks);
  if (rc) return rc;
  if (T == 0) return BEAM_MOE_OK;
  if ((rc = check_ptrs({x, w_gate, w_up, w_down, y, workspace}, {}))) return rc;
  const Experts ex{w_gate, w_up, w_down, nullptr, nullptr, nullptr};
  return dense_common(stream, T, H, I, chunks, x, ex, y, workspace, workspace_bytes);
}

int beam_dense_mlp_fp8(void* stream, int64_t T, int H, int I, int chunks, const uint16_t* x,
                       const uint8_t* w_gate, const float* s_gate, const uint8_t* w_up,
                       const float* s_up, const uint8_t* w_down, const float* s_down, uint16_t* y,
                       void* workspace, size_t workspace_bytes) {
  int rc = check_dense_dims(T, H, I, chunks);
  if (rc) return rc;
  if (T == 0) return BEAM_MOE_OK;
  if ((rc = check_ptrs({x, w_gate, s_gate, w_up, s_up, w_down, s_down, y, workspace}, {}))) return rc;
  const Experts ex{reinterpret_cast<const uint16_t*>(w_gate), reinterpret_cast<const uint16_t*>(w_up),
                   reinterpret_cast<const uint16_t*>(w_down), s_gate, s_up, s_down};
  return dense_common(stream, T, H, I, chunks, x, ex, y, workspace, workspace_bytes);
}

int beam_moe_stage_count(void) { return NST; }

const char* beam_moe_stage_name(int stage) {
  return (stage >= 0 && stage < NST) ? kStageNames[stage] : "";
}

int beam_moe_timer_begin(int max_calls) { return beam_moe_timer_begin_stages(max_calls, (1u << NST) - 1u); }

int beam_moe_timer_begin_stages(int max_calls, unsigned stage_mask) {
  if (max_calls < 1 || max_calls > 100000) return BEAM_MOE_ERR_INVALID_DIM;
  if (stage_mask == 0u || (stage_mask >> NST) != 0u) return BEAM_MOE_ERR_INVALID_DIM;
  std::lock_guard<std::mutex> lk(g_timer.mu);
  if (g_timer.on) return BEAM_MOE_ERR_INVALID_DIM;
  g_timer.ev.assign((size_t)max_calls * NST * 2, nullptr);
  g_timer.used.assign((size_t)max_calls * NST, 0);
  for (auto& e : g_timer.ev)
    if (hipEventCreate(&e) != hipSuccess) return BEAM_MOE_ERR_HIP;
  g_timer.max_calls = max_calls;
  g_timer.n_calls = 0;
  g_timer.mask = stage_mask;
  g_timer.on = true;
  return BEAM_MOE_OK;
}

int beam_moe_timer_end(double* stage_ms, int n_stages, int* n_calls) {
  if (!stage_ms || !n_calls) return BEAM_MOE_ERR_NULL_POINTER;
  if (n_stages < NST) return BEAM_MOE_ERR_INVALID_DIM;
  std::lock_guard<std::mutex> lk(g_timer.mu);
  if (!g_timer.on) return BEAM_MOE_ERR_INVALID_DIM;
  int rc = BEAM_MOE_OK;
  for (int s = 0; s < n_stages; ++s) stage_ms[s] = 0.0;
  for (int c = 0; c < g_timer.n_calls; ++c)
    for (int s = 0; s < NST; ++s) {
      if (!g_timer.used[(size_t)c * NST + s]) continue;
      hipEvent_t a = g_timer.ev[(size_t)(c * NST + s) * 2], b = g_timer.ev[(size_t)(c * NST + s) * 2 + 1];
      float ms = 0.f;
      if (hipEventSynchronize(b) != hipSuccess || hipEventElapsedTime(&ms, a, b) != hipSuccess) {
        rc = BEAM_MOE_ERR_HIP;
        continue;
      }
      stage_ms[s] += ms;
    }
  *n_calls = g_timer.n_calls;
  for (auto& e : g_timer.ev)
    if (e) (void)hipEventDestroy(e);
  g_timer.ev.clear();
  g_timer.used.clear();
  g_timer.on = false;
  return rc;
}

}  // extern "C"
