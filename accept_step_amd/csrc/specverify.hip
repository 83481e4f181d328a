// specverify.hip -- host side of the verify-step library: argument checking,
// workspace planning and the launch sequence behind the C ABI in specverify.h.
//
// One call = one verify pass ([Infra-ch8] "why one forward pass can verify several
// tokens"): logits of all gamma+1 slots (LM-head product, or the full decoder
// forward), the vocab-wide row statistics fused into the product's epilogue, then
// the acceptance rule and -- for sampling -- the correction/bonus draw.  Everything
// is enqueued on the caller's stream; nothing here synchronises or allocates.
#include "specverify.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <algorithm>
#include <atomic>
#include <mutex>
#include <string>
#include <vector>

#include "sv_accept.hpp"
#include "sv_decoder.hpp"
#include "sv_device.hpp"
#include "sv_gemm.hpp"
#include "sv_head.hpp"
#include "sv_masked.hpp"
#include "sv_filter.hpp"
#include "sv_drafter.hpp"
#include "sv_rounds.hpp"
#include "sv_diag.hpp"
#include "sv_wide.hpp"

using namespace sv;

// The scratch array of spec_verify_sample_noalloc (see below); file scope.
constexpr size_t NOALLOC_SCRATCH_BYTES = size_t(4) << 20;
static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int32_t VERSION = 10000;   // 1.0.0
constexpr size_t ALIGN = 256;
constexpr int GEMM_WAVES = 4;
constexpr int GEMM_MAX_WG = 2048;    // upper bound of workgroups along the vocabulary
constexpr size_t GEMM_LDS_BUDGET = 64 * 1024;
constexpr int SAMPLE_CHUNK = 1024;          // the sampler's smallest vocabulary chunk
constexpr int SAMPLE_MAX_WG = 2048;         // ... doubled until the grid is at most this many workgroups
constexpr int ATT_SPLITS_MAX = ATT_SPLITS_CAP;
constexpr int FUSE_ACCEPT_MAX_ROWS = 20;   // B * (gamma + 1) merged by the product's last workgroup
// sequences finished by the sampler's last workgroup; more are merged by a launch of
// their own, one wavefront per sequence (at B = 64 the last workgroup's 16 sequences per
// wavefront and 16384 workgroups counting on one word took the sampler to 250 us)
constexpr int FUSE_FINISH_MAX_B = 8;
constexpr size_t STATIC_LDS_RESERVE = 2048;

thread_local std::string g_err;

sv_status fail(sv_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

#define SV_HIP(call)                                                                     \
  do {                                                                                   \
    hipError_t e_ = (call);                                                              \
    if (e_ != hipSuccess) return fail(SV_ERR_HIP, "%s: %s", #call, hipGetErrorString(e_)); \
  } while (0)

size_t align_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

// ---------------------------------------------------------------------------
// device properties (per device, lazily)
struct DevInfo {
  int dev = 0;
  int cus = 0;
  size_t lds_max = 64 * 1024;   // dynamic LDS per workgroup the streaming product may use
};
std::mutex g_dev_mu;
std::vector<DevInfo> g_dev;

sv_status dev_info(DevInfo* out) {
  int dev = 0;
  SV_HIP(hipGetDevice(&dev));
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if (int(g_dev.size()) <= dev) g_dev.resize(dev + 1);
  if (g_dev[dev].cus == 0) {
    int cus = 0, lds = 0;
    SV_HIP(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
    SV_HIP(hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev));
    g_dev[dev].cus = cus > 0 ? cus : 1;
    g_dev[dev].lds_max = lds >= 64 * 1024 ? size_t(lds) : size_t(64 * 1024);
  }
  *out = g_dev[dev];
  out->dev = dev;
  return SV_OK;
}

// Item sizes chosen by sv_tune_verify for the fused step, per (device, M, K, V).  The
// item size changes how the stream's loads are grouped, not the summation order: the
// logits and every decision are the same bits whichever is used.
struct TunedItem {
  int dev, M, K, N, grp;
};
std::mutex g_tune_mu;
std::vector<TunedItem> g_tuned;

int tuned_item(int dev, int M, int K, int N) {
  std::lock_guard<std::mutex> lk(g_tune_mu);
  for (const TunedItem& t : g_tuned)
    if (t.dev == dev && t.M == M && t.K == K && t.N == N) return t.grp;
  return 0;
}

void set_tuned_item(int dev, int M, int K, int N, int grp) {
  std::lock_guard<std::mutex> lk(g_tune_mu);
  for (TunedItem& t : g_tuned)
    if (t.dev == dev && t.M == M && t.K == K && t.N == N) { t.grp = grp; return; }
  g_tuned.push_back({dev, M, K, N, grp});
}

// Process-wide options (sv_set_option).
std::atomic<unsigned> g_wait_limit{HEAD_SPIN_LIMIT};

// ---------------------------------------------------------------------------
// The scratch of spec_verify_sample_noalloc: a fixed device array, one copy per device
// the library runs on, kept until the process ends.  Host code never uses its name as an
// address (that is a host-side stand-in): each device's address comes from
// hipGetSymbolAddress, taken once per device with that device current, and only that
// address is passed to kernels.  Its first CNT_BYTES (the counter block) start at zero
// (cleared by a fill kernel when the address is taken) and every call leaves them so.
std::mutex g_scratch_mu;
std::vector<void*> g_scratch;   // per device

// timing with events on the caller's stream
struct Timer {
  std::mutex mu;
  unsigned mask = 0;      // bit c: record kernel class c
  std::vector<hipEvent_t> pool;
  struct Rec { int which; hipEvent_t a, b; };
  std::vector<Rec> recs;
} g_timer;

struct TimeScope {
  hipStream_t s;
  int which;
  hipEvent_t a = nullptr, b = nullptr;
  TimeScope(hipStream_t s_, int w) : s(s_), which(w) {
    std::lock_guard<std::mutex> lk(g_timer.mu);
    if (!(g_timer.mask >> which & 1u)) return;
    for (hipEvent_t* e : {&a, &b}) {
      if (!g_timer.pool.empty()) { *e = g_timer.pool.back(); g_timer.pool.pop_back(); }
      else if (hipEventCreate(e) != hipSuccess) { *e = nullptr; }
    }
    if (a && b) (void)hipEventRecord(a, s);
  }
  ~TimeScope() {
    if (!(a && b)) return;
    (void)hipEventRecord(b, s);
    std::lock_guard<std::mutex> lk(g_timer.mu);
    g_timer.recs.push_back({which, a, b});
  }
};

// ---------------------------------------------------------------------------
// argument checks

bool is_aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct Shape {
  int B, gamma, G1, M, V, d;
  sv_input_kind kind;
  bool decoder;
};

sv_status check_common(const sv_model* m, sv_input_kind kind, const void* input, int32_t B, int32_t gamma,
                       const sv_kv_cache* kv, Shape* sh) {
  if (!m) return fail(SV_ERR_ARG, "model is NULL");
  if (!input) return fail(SV_ERR_ARG, "input is NULL");
  if (B < 1) return fail(SV_ERR_ARG, "B must be >= 1 (got %d)", B);
  if (gamma < 1 || gamma > 15) return fail(SV_ERR_ARG, "gamma must be in [1, 15] (got %d)", gamma);
  if (m->vocab < 2) return fail(SV_ERR_ARG, "vocab must be >= 2 (got %d)", m->vocab);
  if (int64_t(B) * (gamma + 1) > (int64_t(1) << 30)) return fail(SV_ERR_SHAPE, "B * (gamma + 1) too large");
  if (int64_t(B) * (gamma + 1) * m->vocab > (int64_t(1) << 40)) return fail(SV_ERR_SHAPE, "logits too large");
  if (int64_t(B) * ((m->vocab + 4095) / 4096) > 0x7fffffffLL) return fail(SV_ERR_SHAPE, "B * V too large");
  if (kind != SV_IN_LOGITS && int64_t(B) * (gamma + 1) > 64LL * 65535)
    return fail(SV_ERR_SHAPE, "B * (gamma + 1) must be <= %lld for model inputs", 64LL * 65535);
  sh->B = B; sh->gamma = gamma; sh->G1 = gamma + 1; sh->M = B * (gamma + 1);
  sh->V = m->vocab; sh->d = m->d_model; sh->kind = kind; sh->decoder = false;
  switch (kind) {
    case SV_IN_LOGITS:
      if (!is_aligned(input, 4)) return fail(SV_ERR_ARG, "logits input must be 4-byte aligned");
      break;
    case SV_IN_HIDDEN:
      if (m->n_layers != 0) return fail(SV_ERR_ARG, "SV_IN_HIDDEN needs an LM-head-only model (n_layers == 0)");
      if (!m->lm_head) return fail(SV_ERR_ARG, "lm_head is NULL");
      if (m->d_model < 1) return fail(SV_ERR_ARG, "d_model must be >= 1");
      if (m->wdtype == SV_BF16) {
        if (m->d_model % 32) return fail(SV_ERR_SHAPE, "bf16 LM head needs d_model %% 32 == 0 (got %d)", m->d_model);
        if (!is_aligned(m->lm_head, 16) || !is_aligned(input, 16))
          return fail(SV_ERR_ARG, "bf16 lm_head and hidden states must be 16-byte aligned");
      } else if (m->wdtype == SV_F32) {
        if (size_t(sh->M) * m->d_model * 4 > 48 * 1024)
          return fail(SV_ERR_UNSUPPORTED, "float32 LM head supports M * d_model <= 12288 only");
      } else {
        return fail(SV_ERR_DTYPE, "unknown wdtype %d", int(m->wdtype));
      }
      break;
    case SV_IN_TOKENS: {
      if (m->n_layers < 1) return fail(SV_ERR_ARG, "SV_IN_TOKENS needs n_layers >= 1");
      if (m->wdtype != SV_BF16) return fail(SV_ERR_DTYPE, "decoder weights must be bf16");
      if (m->head_dim != 64 && m->head_dim != 128) return fail(SV_ERR_SHAPE, "head_dim must be 64 or 128");
      if (m->n_heads < 1 || m->d_model < 32 || m->d_ff < 32) return fail(SV_ERR_ARG, "bad decoder dimensions");
      if (m->d_model % 32 || m->d_ff % 32 || (m->n_heads * m->head_dim) % 32)
        return fail(SV_ERR_SHAPE, "d_model, d_ff and n_heads * head_dim must be multiples of 32");
      if (!m->embed || !m->layers || !m->final_norm || !m->lm_head) return fail(SV_ERR_ARG, "model pointer is NULL");
      for (int i = 0; i < m->n_layers * 9; ++i) {
        if (!m->layers[i]) return fail(SV_ERR_ARG, "layer pointer %d is NULL", i);
        if (!is_aligned(m->layers[i], 16)) return fail(SV_ERR_ARG, "layer pointer %d is not 16-byte aligned", i);
      }
      if (!is_aligned(m->lm_head, 16) || !is_aligned(m->embed, 16) || !is_aligned(m->final_norm, 16))
        return fail(SV_ERR_ARG, "weights must be 16-byte aligned");
      if (m->d_model > 256 * 4 * RMS_VEC) return fail(SV_ERR_SHAPE, "d_model must be <= %d", 256 * 4 * RMS_VEC);
      if (!(m->rms_eps >= 0.0f) || !std::isfinite(m->rms_eps)) return fail(SV_ERR_ARG, "rms_eps must be finite and >= 0");
      if (!(m->rope_theta > 0.0f) || !std::isfinite(m->rope_theta)) return fail(SV_ERR_ARG, "rope_theta must be finite and > 0");
      if (!kv || !kv->k || !kv->v || !kv->len) return fail(SV_ERR_ARG, "SV_IN_TOKENS needs a KV cache");
      if (kv->max_len < gamma + 1) return fail(SV_ERR_ARG, "kv max_len must be >= gamma + 1");
      sh->decoder = true;
      break;
    }
    default:
      return fail(SV_ERR_ARG, "unknown input kind %d", int(kind));
  }
  return SV_OK;
}

// ---------------------------------------------------------------------------
// GEMM planning
struct GemmPlan {
  int MB, mgroups, KC, grid_x_max;
  bool stream;        // streaming kernel (X fully in LDS, K % 256 == 0)
  size_t lds;
};

// ``lds_limit`` = 0 plans without device knowledge (workspace sizing only needs grid_x_max).
GemmPlan plan_gemm(int M, int N_total_tiles, int K, size_t lds_limit = 0) {
  GemmPlan p;
  const int mblocks = (M + 15) / 16;
  p.MB = mblocks < 4 ? mblocks : 4;
  p.mgroups = (mblocks + p.MB - 1) / p.MB;
  const int rows = std::min(16 * p.MB, M);
  const size_t stats = size_t(GEMM_WAVES) * 16 * p.MB * 12;
  const size_t full = size_t(rows) * (K + 8) * 2;
  p.stream = lds_limit > STATIC_LDS_RESERVE && K % (32 * GEMM_GRP) == 0 && full <= lds_limit - STATIC_LDS_RESERVE;
  int KC = K;
  if (!p.stream && full > GEMM_LDS_BUDGET) {
    KC = int((GEMM_LDS_BUDGET / (size_t(rows) * 2) - 8) / 256 * 256);
    if (KC < 256) KC = 256;
  }
  p.KC = KC;
  p.lds = std::max(size_t(rows) * (std::min(KC, K) + 8) * 2, stats);
  const int nblk = (N_total_tiles + GEMM_WAVES - 1) / GEMM_WAVES;
  p.grid_x_max = std::min(nblk, GEMM_MAX_WG);
  return p;
}

int gemm_grid_x(const GemmPlan& p, const DevInfo& di) { return std::max(1, std::min(di.cus, p.grid_x_max)); }

template <int MB>
sv_status launch_gemm_mb(const GemmPlan& p, const GemmArgs& a, dim3 grid, hipStream_t s) {
  if (p.stream) {
    // raise the kernel's dynamic LDS limit to what this launch needs (monotone)
    static std::mutex mu;
    static size_t lds_set = 64 * 1024;
    {
      std::lock_guard<std::mutex> lk(mu);
      if (p.lds > lds_set) {
        SV_HIP(hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm_stream<MB, GEMM_WAVES>),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, int(p.lds)));
        lds_set = p.lds;
      }
    }
    hipLaunchKernelGGL((k_gemm_stream<MB, GEMM_WAVES>), grid, dim3(GEMM_WAVES * 64), p.lds, s, a);
  } else {
    hipLaunchKernelGGL((k_gemm_chunked<MB, GEMM_WAVES>), grid, dim3(GEMM_WAVES * 64), p.lds, s, a);
  }
  SV_HIP(hipGetLastError());
  return SV_OK;
}

sv_status launch_gemm(const GemmPlan& p, GemmArgs a, const DevInfo& di, hipStream_t s, int* grid_x_out = nullptr) {
  a.KC = p.KC;
  const int gx = gemm_grid_x(p, di);
  if (grid_x_out) *grid_x_out = gx;
  dim3 grid(gx, p.mgroups);
  switch (p.MB) {
    case 1: return launch_gemm_mb<1>(p, a, grid, s);
    case 2: return launch_gemm_mb<2>(p, a, grid, s);
    case 3: return launch_gemm_mb<3>(p, a, grid, s);
    default: return launch_gemm_mb<4>(p, a, grid, s);
  }
}

GemmArgs gemm_args(const bf16_t* X, int M, int K) {
  GemmArgs a;
  memset(&a, 0, sizeof a);
  a.X = X; a.M = M; a.K = K;
  return a;
}

void gemm_add_seg(GemmArgs& a, const void* W, float* out, int N) {
  const int i = a.nseg++;
  a.W[i] = static_cast<const bf16_t*>(W);
  a.out[i] = out;
  a.N[i] = N;
  a.tile_end[i] = (i ? a.tile_end[i - 1] : 0) + (N + 15) / 16;
}

// ---------------------------------------------------------------------------
// k-split product (sv_head.hpp) planning
// The k-split kernel's static LDS (reductions, the rule's per-row inputs: 3,760 bytes
// per instantiation as compiled for gfx950), checked against each instantiation before
// its first launch.  Reserving 8 KB, the plan for 12 rows of a 4096-wide head (156.5 KB
// of X and products) did not fit the 160 KB.
constexpr size_t HEAD_STATIC_LDS = 4 * 1024;

struct HeadPlan {
  bool ok = false;
  int S = 0, NB = 0, GRP = 0, grid = 0, gpt = 0, nloc = 0;
  bool pair = false;   // gate and up tiles paired in each wavefront, SwiGLU in the epilogue
  size_t lds = 0;
};

// Largest column-block count instantiated per split factor.
int head_nb_max(int S) { return S == 4 ? 5 : 3; }

// Plan of the k-split kernel, one workgroup per CU.  Loads per lane per work item are
// tried in the order 4, 8, 6 for products (decoder linears, verify_forward) and 4, 6, 8
// for the LM-head launch that applies the rule (rule = true).  For the latter the better
// item depends on the device's clocks: on the 805 MB head (K = 1536) items of 4 took
// 124.5 us against 128.6 with items of 6 under sustained load (greedy 119.5 against
// 123.5), and 137.1 against 130.6 on a device just out of idle; sv_tune_verify measures
// it per device (a tuned item size, want_grp, wins over this order).  only_s != 0 admits
// that split factor alone.  The plan depends on the shapes and the device only, so the summation order
// (and so every logit bit) is the same from call to call.
HeadPlan plan_head(int M, int K, const int* N, int nseg, const DevInfo& di, bool rule = false, int only_s = 0,
                   int want_grp = 0, bool pair = false) {
  HeadPlan p;
  if (M < 1 || M > HEAD_MAX_ROWS || K % 8) return p;
  if (pair && (nseg != 2 || N[0] != N[1])) return p;
  for (int i = 0; i < nseg; ++i)    // weights are addressed with 32-bit byte offsets
    if (int64_t(N[i]) * K * 2 > int64_t(0xffffffffLL) - 4096) return p;
  const int order_product[3] = {4, 8, 6}, order_rule[3] = {4, 6, 8};
  const int* order = rule ? order_rule : order_product;
  for (int S : {4, 2}) {
    if (only_s && S != only_s) continue;
    const int TR = 16 / S, NB = (M + TR - 1) / TR;
    if (NB > head_nb_max(S) || K % (32 * S)) continue;
    const int steps = K / (32 * S);
    int GRP = want_grp && steps % want_grp == 0 ? want_grp : 0;
    for (int i = 0; i < 3 && !GRP; ++i) {
      const int gc = order[i];
      if (steps % gc == 0) GRP = gc;
    }
    if (!GRP) GRP = 4;   // the last item of a tile runs past K over zeros in X
    const int gpt = (steps + GRP - 1) / GRP, Kp = gpt * GRP * 32 * S;
    int ntiles = 0;
    for (int i = 0; i < nseg; ++i) ntiles += (N[i] + TR - 1) / TR;
    int grid = std::min(di.cus, GEMM_MAX_WG);
    grid = std::max(1, std::min(grid, (ntiles + HEAD_WAVES - 1) / HEAD_WAVES));
    const int span = grid * HEAD_WAVES;
    // paired: a wavefront takes the gate and the up tile of each of its rows
    const int tpw = pair ? 2 * ((ntiles / 2 + span - 1) / span) * HEAD_WAVES
                         : (ntiles + span - 1) / span * HEAD_WAVES;
    const size_t lds = head_lds(M, Kp, S, tpw * TR);
    if (lds + HEAD_STATIC_LDS > di.lds_max) continue;
    p.ok = true; p.S = S; p.NB = NB; p.GRP = GRP; p.grid = grid; p.gpt = gpt; p.nloc = tpw * TR; p.pair = pair;
    p.lds = lds;
    return p;
  }
  return p;
}

// The plan of an LM-head launch that applies the rule, on the split factor of the
// product plan: the split fixes the summation order, so the logits are the same bits
// as verify_forward's.
HeadPlan plan_head_rule(int M, int K, const int* N, const DevInfo& di) {
  HeadPlan hp = plan_head(M, K, N, 1, di);
  if (!hp.ok) return hp;
  const HeadPlan r = plan_head(M, K, N, 1, di, true, hp.S, tuned_item(di.dev, M, K, N[0]));
  return r.ok ? r : hp;
}

template <int S, int NB>
const void* head_fn_grp(int GRP) {
  switch (GRP) {
    case 8: return reinterpret_cast<const void*>(&k_head<S, NB, 8>);
    case 6: return reinterpret_cast<const void*>(&k_head<S, NB, 6>);
    default: return reinterpret_cast<const void*>(&k_head<S, NB, 4>);
  }
}

const void* head_fn(const HeadPlan& p) {
  if (p.S == 4) {
    switch (p.NB) {
      case 1: return head_fn_grp<4, 1>(p.GRP);
      case 2: return head_fn_grp<4, 2>(p.GRP);
      case 3: return head_fn_grp<4, 3>(p.GRP);
      case 4: return head_fn_grp<4, 4>(p.GRP);
      default: return head_fn_grp<4, 5>(p.GRP);
    }
  }
  switch (p.NB) {
    case 1: return head_fn_grp<2, 1>(p.GRP);
    case 2: return head_fn_grp<2, 2>(p.GRP);
    default: return head_fn_grp<2, 3>(p.GRP);
  }
}

HeadArgs head_args(const bf16_t* X, int M, int K) {
  HeadArgs a;
  memset(&a, 0, sizeof a);
  a.X = X; a.M = M; a.K = K;
  return a;
}

void head_add_seg(HeadArgs& a, const void* W, float* out, int N, int TR) {
  const int i = a.nseg++;
  a.W[i] = static_cast<const bf16_t*>(W);
  a.out[i] = out;
  a.N[i] = N;
  a.tile_end[i] = (i ? a.tile_end[i - 1] : 0) + (N + TR - 1) / TR;
}

// Raise the kernel's dynamic LDS limit to what a launch needs (monotone per kernel); on
// a kernel's first use, check that its static LDS is within what the plans reserve.
sv_status head_set_lds(const void* fn, size_t lds) {
  static std::mutex mu;
  static std::vector<std::pair<const void*, size_t>> lds_set;
  std::lock_guard<std::mutex> lk(mu);
  size_t cur = 0;
  bool known = false;
  for (auto& e : lds_set)
    if (e.first == fn) { cur = e.second; known = true; }
  if (!known) {
    hipFuncAttributes fa;
    SV_HIP(hipFuncGetAttributes(&fa, fn));
    if (fa.sharedSizeBytes > HEAD_STATIC_LDS)
      return fail(SV_ERR_UNSUPPORTED, "a streaming kernel uses %zu bytes of static LDS, more than the %zu its "
                  "plans reserve", size_t(fa.sharedSizeBytes), HEAD_STATIC_LDS);
    lds_set.push_back({fn, size_t(64 * 1024)});
    cur = 64 * 1024;
  }
  if (lds <= cur) return SV_OK;
  SV_HIP(hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, int(lds)));
  for (auto& e : lds_set) if (e.first == fn) e.second = lds;
  return SV_OK;
}

// Whether the fused sampler can run: its workgroups wait for each other, so they must
// all be resident at once.  The step runs only at one workgroup per CU with the whole
// grid within the CUs and within what the occupancy query admits; otherwise the
// two-launch path runs.  A plain launch does not promise co-residency (with two
// workgroups per CU the query admitted the grid, yet in back-to-back launches some
// workgroups started only after others had given up waiting), and a cooperative launch,
// which would, cost 16-18 us more per step on this device than the whole tail; the
// bounded waits and the epoch check handle the case (see k_head).  The group merge
// takes a lane per member.
sv_status head_all_resident(const HeadPlan& p, const DevInfo& di, bool* yes) {
  *yes = false;
  const void* fn = head_fn(p);
  sv_status st = head_set_lds(fn, p.lds);
  if (st) return st;
  int per_cu = 0;
  SV_HIP(hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, HEAD_WAVES * 64, p.lds));
  *yes = per_cu >= 1 && p.grid <= per_cu * di.cus && p.grid <= di.cus && p.grid <= 64 * CNT_GROUPS;
  return SV_OK;
}

// The decoder products' instantiation (honours HeadArgs::pair): split 4, items of 4.
bool head_pairable(const HeadPlan& p) { return p.S == 4 && p.GRP == 4; }
const void* head_fn_pairable(int NB) {
  switch (NB) {
    case 1: return reinterpret_cast<const void*>(&k_head<4, 1, 4, true>);
    case 2: return reinterpret_cast<const void*>(&k_head<4, 2, 4, true>);
    case 3: return reinterpret_cast<const void*>(&k_head<4, 3, 4, true>);
    case 4: return reinterpret_cast<const void*>(&k_head<4, 4, 4, true>);
    default: return reinterpret_cast<const void*>(&k_head<4, 5, 4, true>);
  }
}

sv_status launch_head(const HeadPlan& p, HeadArgs a, hipStream_t s, bool pairable = false) {
  a.gpt = p.gpt;
  a.nloc = p.nloc;
  const void* fn = pairable ? head_fn_pairable(p.NB) : head_fn(p);
  sv_status st = head_set_lds(fn, p.lds);
  if (st) return st;
  void* args[] = {&a};
  SV_HIP(hipLaunchKernel(fn, dim3(p.grid), dim3(HEAD_WAVES * 64), args, p.lds, s));
  return SV_OK;
}

// Plan of the wide-batch product (sv_wide.hpp), for batches above 16 rows (up to 16
// rows the streaming product keeps all of X in LDS and needs no barrier per chunk:
// 446 against 505 us at 12 rows of the 4096-wide head).  The 16-row blocks of X are
// split into as few M-tiles of at most WIDE_MB_MAX blocks as possible, the tile size
// rounded up to an instantiated one (rows past M are zeros in LDS, their products
// discarded).  Every tile size keeps four W blocks of 16 rows per wavefront (chunks
// of 128 k): one or two blocks per wavefront with longer chunks (runs of 1 KB / 512 B
// of each W row per chunk instead of 256 B) measured slower, 615 against 511 us at 12
// rows, 687 against 646 at 80.
constexpr int WIDE_MAX_ROWS = 16 * WIDE_MB_MAX * 8;
struct WidePlan {
  bool ok = false;
  int MB = 0, BLK = 0, m_tiles = 0, n_tiles = 0, grid = 0;
  bool nt = true, wl = false;
  size_t lds = 0;
};

WidePlan plan_wide(int M, int K, int N) {
  WidePlan p;
  if (M <= 16 || M > WIDE_MAX_ROWS || N < 1) return p;
  const int mblocks = (M + 15) / 16;
  const int tiles = (mblocks + WIDE_MB_MAX - 1) / WIDE_MB_MAX;
  const int per = (mblocks + tiles - 1) / tiles;
  p.MB = per <= 4 ? 4 : per <= 8 ? 8 : WIDE_MB_MAX;
  p.BLK = 4;
  const int kch = wide_kch(p.BLK);
  if (K < 2 * kch || K % (2 * kch)) return p;
  p.m_tiles = (mblocks + p.MB - 1) / p.MB;
  p.nt = p.m_tiles == 1;                      // sibling M-tiles read W again from L2
  p.n_tiles = (N + 64 * p.BLK - 1) / (64 * p.BLK);
  p.grid = (p.n_tiles + 7) / 8 * 8 * p.m_tiles;
  p.wl = p.MB <= 8;                          // W through LDS in 256-byte runs (sv_wide.hpp)
  p.lds = size_t(2) * 16 * p.MB * (kch + 8) * 2 + (p.wl ? size_t(4) * 64 * WIDE_WLD * 2 : 0);
  p.ok = true;
  return p;
}

sv_status launch_wide(const WidePlan& p, WideArgs a, hipStream_t s) {
  a.m_tiles = p.m_tiles; a.n_tiles = p.n_tiles;
  const void* fn = p.MB == 4 ? reinterpret_cast<const void*>(&k_wide<4, 4, true, true>)
                 : p.MB == 8 ? reinterpret_cast<const void*>(&k_wide<8, 4, true, true>)
                 : p.nt ? reinterpret_cast<const void*>(&k_wide<WIDE_MB_MAX, 4, true>)
                        : reinterpret_cast<const void*>(&k_wide<WIDE_MB_MAX, 4, false>);
  sv_status st = head_set_lds(fn, p.lds);
  if (st) return st;
  void* args[] = {&a};
  SV_HIP(hipLaunchKernel(fn, dim3(p.grid), dim3(256), args, p.lds, s));
  return SV_OK;
}

// Decoder fusions of a k-split product: X normalised from float32 rows while it is
// staged (norm_w set), and the products added into out with per-workgroup sums of
// squares of the updated rows (residual).
struct ProductFuse {
  const float* Xf = nullptr;
  const bf16_t* norm_w = nullptr;
  const float* ss_in = nullptr;
  int ss_parts = 0;
  float eps = 0.0f;
  bool residual = false;
  float* ss_out = nullptr;
  bf16_t* silu_out = nullptr;   // gate and up (two segments of equal N): bf16 SiLU(gate) * up here instead
  bool pairable = false;        // launch on the instantiation that pairs (set for every product of a
                                // decoder whose gate/up pairs: one kernel's code for all of them)
};

// Whether the decoder's fused sequence applies: every product of a layer runs on the
// k-split kernel.
bool fused_products_ok(int M, int d, int HD, int ff, const DevInfo& di) {
  const int n3[3] = {HD, HD, HD}, n1[1] = {d}, n2[2] = {ff, ff};
  return plan_head(M, d, n3, 3, di).ok && plan_head(M, HD, n1, 1, di).ok &&
         plan_head(M, d, n2, 2, di).ok && plan_head(M, ff, n1, 1, di).ok && M <= ACC_MAX_ROWS;
}

// Whether a decoder's gate/up product [2 x ff, K] pairs its tiles (SwiGLU in the
// epilogue): the paired plan exists on the pairing instantiation and gives no wavefront
// more tiles than the plain plan (a wavefront of a paired plan takes whole pairs; where
// the plain plan gives each wavefront one tile, pairing doubles the chain of a launch
// that is latency-bound: the drafter's 2048-wide FFN measured 758 -> 780 us per round).
bool swiglu_paired(int M, int K, int ff, const DevInfo& di) {
  const int n2[2] = {ff, ff};
  const HeadPlan pp = plan_head(M, K, n2, 2, di, false, 0, 0, true), p = plan_head(M, K, n2, 2, di);
  return pp.ok && p.ok && head_pairable(pp) && pp.nloc <= p.nloc;
}

// A k-split product with decoder fusions; *grid_out receives the launch's grid (the
// number of sums-of-squares partials it leaves).
sv_status run_product_fused(const bf16_t* X, int M, int K, int nseg, const void* const* W, float* const* out,
                            const int* N, const ProductFuse& f, int* grid_out, const DevInfo& di, hipStream_t s) {
  HeadPlan hp;
  if (f.silu_out && f.pairable) {
    hp = plan_head(M, K, N, nseg, di, false, 0, 0, true);
    if (!head_pairable(hp)) hp = HeadPlan();
  }
  const bool pair = hp.ok;
  if (!pair) hp = plan_head(M, K, N, nseg, di);
  if (!hp.ok) return fail(SV_ERR_UNSUPPORTED, "fused decoder product does not fit the k-split kernel");
  HeadArgs a = head_args(X, M, K);
  for (int i = 0; i < nseg; ++i) head_add_seg(a, W[i], out[i], N[i], 16 / hp.S);
  a.write_out = pair ? 2 : 1;
  a.hout = pair ? f.silu_out : nullptr;
  a.mode = HEAD_PRODUCT;
  a.Xf = f.Xf; a.norm_w = f.norm_w; a.ss_in = f.ss_in; a.ss_parts = f.ss_parts; a.eps = f.eps;
  a.residual = f.residual ? 1 : 0;
  a.ss_out = f.ss_out;
  if (grid_out) *grid_out = hp.grid;
  // every fused product on one instantiation where it can: products of one kernel in a
  // row keep its code in the instruction caches (with the paired gate/up on a kernel of
  // its own, the other products of a layer took 0.5-1.6 us longer each)
  sv_status st = launch_head(hp, a, s, f.pairable && head_pairable(hp));
  if (st || pair || !f.silu_out) return st;
  // no paired plan (split 2, other items, LDS): the products, then SiLU(gate) * up
  const int n = M * N[0];
  hipLaunchKernelGGL(k_silu_mul, dim3((n + 255) / 256), dim3(256), 0, s, out[0], out[1], f.silu_out, n);
  SV_HIP(hipGetLastError());
  return SV_OK;
}

// A product out_s[M, N_s] = X[M, K] W_s^T for up to three weights sharing X: the
// k-split kernel where it applies, else the 16-row streaming / chunked kernels.
sv_status run_product(const bf16_t* X, int M, int K, int nseg, const void* const* W, float* const* out, const int* N,
                      const DevInfo& di, hipStream_t s) {
  const HeadPlan hp = plan_head(M, K, N, nseg, di);
  if (hp.ok) {
    HeadArgs a = head_args(X, M, K);
    for (int i = 0; i < nseg; ++i) head_add_seg(a, W[i], out[i], N[i], 16 / hp.S);
    a.write_out = 1;
    a.mode = HEAD_PRODUCT;
    return launch_head(hp, a, s);
  }
  GemmArgs a = gemm_args(X, M, K);
  int tiles = 0;
  for (int i = 0; i < nseg; ++i) { gemm_add_seg(a, W[i], out[i], N[i]); tiles += (N[i] + 15) / 16; }
  return launch_gemm(plan_gemm(M, tiles, K, di.lds_max), a, di, s);
}

// ---------------------------------------------------------------------------
// workspace layout
// The sampler's vocabulary chunk: SAMPLE_CHUNK, doubled while B chunks per sequence would
// need more than SAMPLE_MAX_WG workgroups (any partition draws the same token).
int sample_chunk(int V, int B) {
  int c = SAMPLE_CHUNK;
  while (c < V && int64_t((V + c - 1) / c) * B > SAMPLE_MAX_WG) c *= 2;
  return c;
}

struct Layout {
  size_t counters = 0;   // CNT_BYTES of one-shot counters; zero before first use, left zero
  size_t logits = 0, part = 0, state = 0, spart = 0, invalid = 0, xlogit = 0, recs = 0;
  size_t rope = 0, x = 0, h = 0, q = 0, k = 0, v = 0, attp = 0, att = 0, gate = 0, up = 0;
  size_t attcnt = 0;    // [B, n_heads, query groups] split counters of the attention; zeroed by k_prep each call
  size_t ss = 0;        // [GEMM_MAX_WG, M] partial sums of squares of the residual stream's rows
  size_t diag_rows = 0, diag_draws = 0;   // the margins' partials (sv_diag.hpp), when asked for
  size_t total = 0;
  int P = 0;          // row-statistics partials per row
  int nch = 0;        // sampling chunks per sequence
  int chunk = 0;      // ... of this many vocabulary entries
  int S = 0;          // attention key splits
  GemmPlan head;
};

struct Bump {
  size_t off = 0;
  size_t take(size_t bytes) {
    size_t o = off;
    off = align_up(off + std::max<size_t>(bytes, 1));
    return o;
  }
};

// Query groups of the attention (at most ATT_QMAX new positions per workgroup) and
// the query slots of each group's kernel.
int att_query_groups(int G1) { return (G1 + ATT_QMAX - 1) / ATT_QMAX; }
int att_query_slots(int G1) {
  const int per = (G1 + att_query_groups(G1) - 1) / att_query_groups(G1);
  return per <= 2 ? 2 : per <= 4 ? 4 : per <= 5 ? 5 : 8;
}

int att_splits(const sv_kv_cache* kv) {
  int S = (kv->max_len + 255) / 256;
  return std::max(1, std::min(S, ATT_SPLITS_MAX));
}

Layout plan(const sv_model* m, const Shape& sh, const sv_kv_cache* kv, bool need_logits_buf, bool sample,
            bool diag = false) {
  Layout L;
  Bump b;
  const int M = sh.M, V = sh.V;
  L.counters = b.take(CNT_BYTES);
  if (need_logits_buf) L.logits = b.take(size_t(M) * V * 4);
  if (sh.kind == SV_IN_LOGITS) {
    L.P = (V + LCH - 1) / LCH;
  } else if (sh.kind == SV_IN_HIDDEN && m->wdtype == SV_F32) {
    L.P = (V + 255) / 256;
  } else {
    L.head = plan_gemm(M, (V + 15) / 16, sh.decoder ? m->d_model : sh.d);
    L.P = L.head.grid_x_max;
    const WidePlan wp = plan_wide(M, sh.decoder ? m->d_model : sh.d, V);
    if (wp.ok) L.P = std::max(L.P, wp.n_tiles);
  }
  // per-workgroup partials of either product kernel, then the k-split kernel's group partials
  L.part = b.take(size_t(std::max(L.P, GEMM_MAX_WG) + CNT_GROUPS) * M * sizeof(RowPart));
  L.state = b.take(size_t(sh.B) * sizeof(SeqState));
  L.xlogit = b.take(size_t(M) * 4);
  L.chunk = sample_chunk(V, sh.B);
  L.nch = (V + L.chunk - 1) / L.chunk;
  if (sample) L.spart = b.take(size_t(sh.B) * std::max(L.nch, GEMM_MAX_WG) * sizeof(SamplePart));   // either sampler
  L.invalid = b.take(size_t(sh.B) * 4);
  // the fused sampler's epoch-tagged hand-off records (k-split kernel with a bf16 head and
  // at most ACC_MAX_ROWS rows; grids up to GEMM_MAX_WG)
  const bool bf16_head = sh.kind != SV_IN_LOGITS && !(sh.kind == SV_IN_HIDDEN && m->wdtype == SV_F32);
  if (sample && bf16_head && M <= ACC_MAX_ROWS)
    L.recs = b.take((size_t(GEMM_MAX_WG + CNT_GROUPS) * M * 4 + M + size_t(sh.B) * GEMM_MAX_WG * 4) * 8);
  if (sh.decoder) {
    const int d = m->d_model, HD = m->n_heads * m->head_dim, ff = m->d_ff;
    L.S = att_splits(kv);
    L.rope = b.take(size_t(M) * (m->head_dim / 2) * sizeof(float2));
    L.x = b.take(size_t(M) * d * 4);
    L.h = b.take(size_t(M) * std::max(std::max(d, ff), HD) * 2);
    L.q = b.take(size_t(M) * HD * 4);
    L.k = b.take(size_t(M) * HD * 4);
    L.v = b.take(size_t(M) * HD * 4);
    L.attp = b.take(size_t(sh.B) * m->n_heads * L.S * sh.G1 * (m->head_dim + 2) * 4);
    L.attcnt = b.take(size_t(sh.B) * m->n_heads * att_query_groups(sh.G1) * 4);
    L.ss = b.take(size_t(GEMM_MAX_WG) * M * 4);
    L.att = b.take(size_t(M) * HD * 2);
    L.gate = b.take(size_t(M) * ff * 4);
    L.up = b.take(size_t(M) * std::max(ff, d) * 4);
  }
  if (diag) {
    const int dch = (V + DIAG_CHUNK - 1) / DIAG_CHUNK;
    L.diag_rows = b.take(size_t(M) * dch * sizeof(DiagRow));
    L.diag_draws = b.take(size_t(sh.B) * dch * sizeof(DiagDraw));
  }
  L.total = b.off;
  return L;
}

template <class T>
T* at(void* ws, size_t off) { return reinterpret_cast<T*>(static_cast<char*>(ws) + off); }

sv_status check_ws(void* ws, size_t* ws_bytes, const Layout& L, bool* query) {
  if (!ws_bytes) return fail(SV_ERR_ARG, "ws_bytes is NULL");
  if (!ws) {
    *ws_bytes = L.total;
    *query = true;
    return SV_OK;
  }
  *query = false;
  if (*ws_bytes < L.total)
    return fail(SV_ERR_WORKSPACE, "workspace too small: %zu bytes given, %zu needed", *ws_bytes, L.total);
  if (!is_aligned(ws, ALIGN)) return fail(SV_ERR_WORKSPACE, "workspace must be %zu-byte aligned", ALIGN);
  return SV_OK;
}

// ---------------------------------------------------------------------------
// forward passes

// Full decoder up to (and including) the final RMSNorm: leaves bf16 h [M, d] in
// the workspace.  [Infra-ch8] "why one forward pass can verify several tokens".
sv_status run_decoder(const sv_model* m, const Shape& sh, const int* tokens, const sv_kv_cache* kv,
                      const Layout& L, void* ws, const DevInfo& di, hipStream_t s) {
  TimeScope ts(s, 1);
  const int M = sh.M, d = m->d_model, H = m->n_heads, hd = m->head_dim, ff = m->d_ff, HD = H * hd;
  DecArgs da;
  da.B = sh.B; da.G1 = sh.G1; da.d = d; da.H = H; da.hd = hd; da.ff = ff; da.V = sh.V;
  da.max_len = kv->max_len; da.n_layers = m->n_layers; da.eps = m->rms_eps;
  int* invalid = at<int>(ws, L.invalid);
  float2* rope = at<float2>(ws, L.rope);
  float* x = at<float>(ws, L.x);
  bf16_t* h = at<bf16_t>(ws, L.h);
  float* q = at<float>(ws, L.q);
  float* k = at<float>(ws, L.k);
  float* v = at<float>(ws, L.v);
  float* attp = at<float>(ws, L.attp);
  unsigned* attcnt = at<unsigned>(ws, L.attcnt);
  bf16_t* att = at<bf16_t>(ws, L.att);
  float* gate = at<float>(ws, L.gate);
  float* up = at<float>(ws, L.up);
  bf16_t* kc = static_cast<bf16_t*>(kv->k);
  bf16_t* vc = static_cast<bf16_t*>(kv->v);

  const int ncnt = sh.B * H * att_query_groups(sh.G1);
  const int nprep = std::max(std::max(sh.B, M * (hd / 2)), ncnt);
  hipLaunchKernelGGL(k_prep, dim3((nprep + 255) / 256), dim3(256), 0, s, kv->len, rope, invalid, attcnt, ncnt, sh.B,
                     sh.G1, hd, kv->max_len, m->rope_theta);
  const bool fused = fused_products_ok(M, d, HD, ff, di);
  float* ss = at<float>(ws, L.ss);
  hipLaunchKernelGGL(k_embed, dim3(M), dim3(256), 0, s, tokens, static_cast<const bf16_t*>(m->embed), x, invalid,
                     fused ? ss : nullptr, sh.G1, sh.V, d);
  SV_HIP(hipGetLastError());

  const float scale = 1.0f / sqrtf(float(hd));
  // Attention over the cache and the new positions, which the same launch rotates and
  // appends (RoPE on the queries as they are staged and on the new keys as the workgroup
  // holding their cache rows writes them; the last workgroup of each head merges the
  // key splits).
  auto attention = [&](int l) -> sv_status {
    const int NQ = att_query_groups(sh.G1), QS = att_query_slots(sh.G1);
    const dim3 ag(H, sh.B * NQ, L.S);
    const float qscale = scale * 1.4426950408889634f;   // scores in base-2 units
#define SV_ATTN(HDv, QGv) hipLaunchKernelGGL((k_attn<HDv, QGv>), ag, dim3(256), 0, s, q, kc, vc, kv->len, invalid, attp, \
                                             att, attcnt, da, l, L.S, NQ, qscale, rope, k, v)
#define SV_ATTN_Q(HDv) do { if (QS == 2) SV_ATTN(HDv, 2); else if (QS == 4) SV_ATTN(HDv, 4); \
                            else if (QS == 5) SV_ATTN(HDv, 5); else SV_ATTN(HDv, 8); } while (0)
    if (hd == 128) SV_ATTN_Q(128); else SV_ATTN_Q(64);
#undef SV_ATTN_Q
#undef SV_ATTN
    SV_HIP(hipGetLastError());
    return SV_OK;
  };
  const int nf = M * ff;
  sv_status st;
  const float* pending = nullptr;
  if (fused) {
    // Every RMSNorm happens while the next product stages X from the float32 residual
    // stream, with the row scales from the sums of squares that the producer of the
    // rows left (k_embed: one per row; the output projections: one per workgroup, as
    // they add their products into x).
    int parts = 1;
    const bool pairs = swiglu_paired(M, d, ff, di);
    for (int l = 0; l < m->n_layers; ++l) {
      const void* const* w = m->layers + size_t(l) * 9;
      ProductFuse fn;
      fn.Xf = x; fn.ss_in = ss; fn.ss_parts = parts; fn.eps = m->rms_eps; fn.pairable = pairs;
      ProductFuse fr;
      fr.residual = true; fr.ss_out = ss; fr.pairable = pairs;
      {
        const void* ws3[3] = {w[1], w[2], w[3]};
        float* o3[3] = {q, k, v};
        const int n3[3] = {HD, HD, HD};
        fn.norm_w = static_cast<const bf16_t*>(w[0]);
        if ((st = run_product_fused(nullptr, M, d, 3, ws3, o3, n3, fn, nullptr, di, s))) return st;
      }
      if ((st = attention(l))) return st;
      {
        const void* w1[1] = {w[4]};
        float* o1[1] = {x};
        const int n1[1] = {d};
        if ((st = run_product_fused(att, M, HD, 1, w1, o1, n1, fr, &parts, di, s))) return st;
      }
      {
        const void* w2[2] = {w[6], w[7]};
        float* o2[2] = {gate, up};
        const int n2[2] = {ff, ff};
        fn.ss_parts = parts;
        fn.norm_w = static_cast<const bf16_t*>(w[5]);
        ProductFuse fg = fn;
        fg.silu_out = h;   // SwiGLU in the epilogue: each wavefront holds matching gate and up tiles
        if ((st = run_product_fused(nullptr, M, d, 2, w2, o2, n2, fg, nullptr, di, s))) return st;
      }
      {
        const void* w1[1] = {w[8]};
        float* o1[1] = {x};
        const int n1[1] = {d};
        if ((st = run_product_fused(h, M, ff, 1, w1, o1, n1, fr, &parts, di, s))) return st;
      }
    }
  } else {
    // Residual adds are folded into the next RMSNorm: the output projections write
    // ``delta`` and the following k_add_rmsnorm adds it to x.
    float* delta = up;    // the up-projection buffer holds [M, max(d, d_ff)] floats
    for (int l = 0; l < m->n_layers; ++l) {
      const void* const* w = m->layers + size_t(l) * 9;
      hipLaunchKernelGGL(k_add_rmsnorm, dim3(M), dim3(256), 0, s, x, pending, static_cast<const bf16_t*>(w[0]), h, d,
                         m->rms_eps);
      {
        const void* ws3[3] = {w[1], w[2], w[3]};
        float* o3[3] = {q, k, v};
        const int n3[3] = {HD, HD, HD};
        if ((st = run_product(h, M, d, 3, ws3, o3, n3, di, s))) return st;
      }
      if ((st = attention(l))) return st;
      {
        const void* w1[1] = {w[4]};
        float* o1[1] = {delta};
        const int n1[1] = {d};
        if ((st = run_product(att, M, HD, 1, w1, o1, n1, di, s))) return st;
      }
      hipLaunchKernelGGL(k_add_rmsnorm, dim3(M), dim3(256), 0, s, x, delta, static_cast<const bf16_t*>(w[5]), h, d,
                         m->rms_eps);
      {
        const void* w2[2] = {w[6], w[7]};
        float* o2[2] = {gate, up};
        const int n2[2] = {ff, ff};
        if ((st = run_product(h, M, d, 2, w2, o2, n2, di, s))) return st;
      }
      hipLaunchKernelGGL(k_silu_mul, dim3((nf + 255) / 256), dim3(256), 0, s, gate, up, h, nf);
      {
        const void* w1[1] = {w[8]};
        float* o1[1] = {delta};
        const int n1[1] = {d};
        if ((st = run_product(h, M, ff, 1, w1, o1, n1, di, s))) return st;
      }
      pending = delta;
    }
  }
  hipLaunchKernelGGL(k_add_rmsnorm, dim3(M), dim3(256), 0, s, x, pending, static_cast<const bf16_t*>(m->final_norm), h,
                     d, m->rms_eps);
  SV_HIP(hipGetLastError());
  return SV_OK;
}

// The rule inside the bf16 LM-head launch (k-split kernel).  Greedy: the whole
// step.  Sampling: the whole step when every workgroup can be resident at once and
// the batch fits the counter block's keys (logits stay on chip and are written only
// to ``logits_out``); otherwise the acceptance, with the logits written to
// ``logits`` for the separate sampler.
struct HeadRule {
  float* logits_out;
  bool sample;
  AcceptArgs acc;
  bool done = false;      // nothing else to launch for the step
  bool accepted = false;  // the acceptance ran (the sampler still has to)
};

// The acceptance as a launch of its own (after the wide product, or before the
// two-launch sampler): a wavefront per row of a sequence.
sv_status launch_accept(const AcceptArgs& a, hipStream_t s) {
  const int waves = std::min(a.gamma + 1, 16);   // gamma <= 15
  hipLaunchKernelGGL(k_accept, dim3(a.B), dim3(64 * std::max(waves, 4)), 0, s, a);
  SV_HIP(hipGetLastError());
  return SV_OK;
}

// Logits of all slots plus (if part != NULL) the row-statistics partials.
// Returns the number of partials per row in *P.
// With ``acc`` non-null, the bf16 LM-head product records each slot's draft-token
// logit; with ``fuse`` as well, its last workgroup runs the acceptance for all
// sequences.  With ``rule`` non-null the k-split kernel runs the rule when it fits
// (rule->fused is then true and nothing else is launched for the step).
sv_status run_logits(const sv_model* m, const Shape& sh, const void* input, const sv_kv_cache* kv,
                     const Layout& L, void* ws, float* logits, RowPart* part, float c, int* P, hipStream_t s,
                     const AcceptArgs* acc = nullptr, bool fuse = false, HeadRule* rule = nullptr) {
  DevInfo di;
  sv_status st = dev_info(&di);
  if (st) return st;
  const int M = sh.M, V = sh.V;
  if (sh.kind == SV_IN_LOGITS) {
    if (part) {
      TimeScope ts(s, 2);
      const int nch = (V + LCH - 1) / LCH;
      const long items = long(M) * nch;
      hipLaunchKernelGGL(k_stats_logits, dim3(unsigned((items + 3) / 4)), dim3(256), 0, s,
                         static_cast<const float*>(input), part, M, V, c);
      SV_HIP(hipGetLastError());
      *P = nch;
    }
    return SV_OK;
  }
  const bf16_t* hb = nullptr;
  if (sh.decoder) {
    if ((st = run_decoder(m, sh, static_cast<const int*>(input), kv, L, ws, di, s))) return st;
    hb = at<bf16_t>(ws, L.h);
  } else if (m->wdtype == SV_F32) {
    TimeScope ts(s, 0);
    const int d = sh.d;
    hipLaunchKernelGGL(k_gemm_f32, dim3((V + 255) / 256), dim3(256), size_t(M) * d * 4, s,
                       static_cast<const float*>(m->lm_head), static_cast<const float*>(input), logits, part, M, V, d,
                       c, part ? 1 : 0);
    SV_HIP(hipGetLastError());
    *P = (V + 255) / 256;
    return SV_OK;
  } else {
    hb = static_cast<const bf16_t*>(input);
  }
  TimeScope ts(s, 0);
  const int K = sh.decoder ? m->d_model : sh.d;
  const int Nv[1] = {V};
  HeadPlan hp = rule ? plan_head_rule(M, K, Nv, di) : plan_head(M, K, Nv, 1, di);
  if (hp.ok && (rule || !part)) {
    HeadArgs a = head_args(hb, M, K);
    float* out = rule ? rule->logits_out : logits;
    a.mode = HEAD_PRODUCT;
    if (rule) {
      bool fused = !rule->sample;
      if (rule->sample && (st = head_all_resident(hp, di, &fused))) return st;
      a.mode = !rule->sample ? HEAD_ACCEPT : (fused ? HEAD_SAMPLE : HEAD_ACCEPT);
      if (rule->sample && !fused) {
        out = logits;                                // the separate sampler reads them
        if (!out) return fail(SV_ERR_WORKSPACE, "the fused step does not apply on this device: no logits buffer");
      }
      a.part = part;
      a.c_stat = c;
      a.xlogit = at<float>(ws, L.xlogit);
      a.counter = at<unsigned>(ws, L.counters);
      a.acc = rule->acc;
      a.acc.P = hp.grid;
      a.acc.xlogit = a.xlogit;
      a.spart = at<SamplePart>(ws, L.spart);
      a.recs = rule->sample ? at<unsigned long long>(ws, L.recs) : nullptr;   // planned whenever this path can run
      a.rec_grid = GEMM_MAX_WG;
      a.spin_limit = g_wait_limit.load(std::memory_order_relaxed);   // sv_set_option(SV_OPT_WAIT_LIMIT)
      rule->done = fused;
      rule->accepted = true;
    }
    head_add_seg(a, m->lm_head, out, V, 16 / hp.S);
    a.write_out = out != nullptr;
    *P = hp.grid;
    return launch_head(hp, a, s);
  }
  // wider batches: the tiled product that reads W once per M-tile (sv_wide.hpp); the
  // acceptance runs as its own launch
  const WidePlan wp = plan_wide(M, K, V);
  if (wp.ok) {
    WideArgs w;
    memset(&w, 0, sizeof w);
    w.W = static_cast<const bf16_t*>(m->lm_head); w.X = hb; w.out = logits; w.part = part;
    w.M = M; w.N = V; w.K = K; w.c_stat = c;
    if (acc) {
      w.xlogit = at<float>(ws, L.xlogit);
      w.draft = acc->draft; w.draft_stride = acc->draft_stride; w.draft_offset = acc->draft_offset;
      w.gamma = acc->gamma;
    }
    if ((st = launch_wide(wp, w, s))) return st;
    *P = wp.n_tiles;
    if (acc && fuse) {                     // the caller expects the rule to have run
      AcceptArgs aa = *acc;
      aa.P = wp.n_tiles;
      aa.xlogit = w.xlogit;
      if ((st = launch_accept(aa, s))) return st;
      if (rule) rule->accepted = true;
    }
    return SV_OK;
  }
  GemmArgs a = gemm_args(hb, M, K);
  gemm_add_seg(a, m->lm_head, logits, V);
  a.part = part;
  a.want_stats = part ? 1 : 0;
  a.c_stat = c;
  const GemmPlan ph = plan_gemm(M, (V + 15) / 16, K, di.lds_max);
  if (acc) {                              // record the drafts' logits for the rule
    a.acc = *acc;
    a.xlogit = at<float>(ws, L.xlogit);
  }
  if (acc && fuse) {
    a.acc.P = gemm_grid_x(ph, di);
    a.counter = at<unsigned>(ws, L.counters);
  }
  int gx = 0;
  if ((st = launch_gemm(ph, a, di, s, &gx))) return st;
  *P = gx;
  return SV_OK;
}

// Whether the bf16 LM-head step runs as the one fused launch that keeps the logits on
// chip (the same decision run_logits takes on this device).
sv_status fused_step(const sv_model* m, const Shape& sh, bool sample, bool* yes) {
  *yes = false;
  if (sh.M > HEAD_MAX_ROWS) return SV_OK;   // never fused, whatever the device
  DevInfo di;
  sv_status st = dev_info(&di);
  if (st) return st;
  const int K = sh.decoder ? m->d_model : sh.d;
  const int Nv[1] = {sh.V};
  const HeadPlan hp = plan_head_rule(sh.M, K, Nv, di);
  if (!hp.ok) return SV_OK;
  bool resident = true;
  if (sample && (st = head_all_resident(hp, di, &resident))) return st;
  *yes = resident;
  return SV_OK;
}

// exact_query: with ws == NULL, report the bytes this call needs on the current device
// (the plain query is device-independent and covers every path).
sv_status verify_common(const sv_model* m, sv_input_kind kind, const void* input, int32_t B, int32_t gamma,
                        const int32_t* draft, const void* q, sv_dtype q_dtype, float temperature, uint64_t seed,
                        const int64_t* pos0, const sv_kv_cache* kv, int32_t* n_accepted, int32_t* tokens_out,
                        float* logits_out, float* diag, void* ws, size_t* ws_bytes, void* stream, bool sample,
                        bool exact_query = false) {
  g_err.clear();
  Shape sh;
  sv_status st = check_common(m, kind, input, B, gamma, kv, &sh);
  if (st) return st;
  if (!n_accepted || !tokens_out) return fail(SV_ERR_ARG, "n_accepted and tokens_out must not be NULL");
  if (!draft && kind != SV_IN_TOKENS) return fail(SV_ERR_ARG, "draft is NULL");
  if (sample) {
    if (!std::isfinite(temperature) || temperature < 0.0f)
      return fail(SV_ERR_ARG, "temperature must be finite and >= 0");
    if (temperature == 0.0f) sample = false;   // the greedy rule, exactly
  }
  if (sample) {
    if (!q) return fail(SV_ERR_ARG, "q is NULL");
    if (!pos0) return fail(SV_ERR_ARG, "pos0 is NULL");
    if (q_dtype != SV_F32 && q_dtype != SV_BF16) return fail(SV_ERR_DTYPE, "q_dtype must be SV_F32 or SV_BF16");
  }
  const bool bf16_head = kind != SV_IN_LOGITS && !(kind == SV_IN_HIDDEN && m->wdtype == SV_F32);
  bool need_buf = kind != SV_IN_LOGITS && logits_out == nullptr;
  Layout L = plan(m, sh, kv, need_buf, sample, diag != nullptr);
  // The fused step needs no logits buffer: where the caller's workspace is smaller than
  // the device-independent size (or the exact size is asked for), see whether this device
  // runs it (no device: keep the full size)
  if (need_buf && !diag && bf16_head && ((ws && ws_bytes && *ws_bytes < L.total) || exact_query)) {
    bool fused = false;
    if (fused_step(m, sh, sample, &fused) != SV_OK) {
      fused = false;
      g_err.clear();
    }
    if (fused) {
      need_buf = false;
      L = plan(m, sh, kv, false, sample);
    }
  }
  bool query = false;
  if ((st = check_ws(ws, ws_bytes, L, &query))) return st;
  if (query) return SV_OK;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const float c = sample ? LOG2E / temperature : 0.0f;
  // (no buffer planned: the fused step keeps the logits on chip and never needs one)
  float* logits = kind == SV_IN_LOGITS ? const_cast<float*>(static_cast<const float*>(input))
                                       : (logits_out ? logits_out : need_buf ? at<float>(ws, L.logits) : nullptr);
  RowPart* part = at<RowPart>(ws, L.part);
  int* invalid = at<int>(ws, L.invalid);
  AcceptArgs aa;
  memset(&aa, 0, sizeof aa);
  aa.part = part; aa.logits = logits;
  if (draft) { aa.draft = draft; aa.draft_stride = gamma; aa.draft_offset = 0; }
  else { aa.draft = static_cast<const int*>(input); aa.draft_stride = gamma + 1; aa.draft_offset = 1; }
  aa.q = q; aa.q_bf16 = q_dtype == SV_BF16; aa.pos0 = pos0; aa.invalid = sh.decoder ? invalid : nullptr;
  aa.len = kv ? kv->len : nullptr;
  aa.n_accepted = n_accepted; aa.tokens_out = tokens_out;
  aa.state = at<SeqState>(ws, L.state);
  aa.seed = seed; aa.B = sh.B; aa.gamma = gamma; aa.V = sh.V; aa.c = c; aa.sample = sample ? 1 : 0;
  const bool fuse = bf16_head && sh.M <= FUSE_ACCEPT_MAX_ROWS;
  if (bf16_head) aa.xlogit = at<float>(ws, L.xlogit);
  int P = 0;
  HeadRule rule;
  rule.logits_out = diag && !logits_out ? logits : logits_out;   // the margins read the logits from memory
  rule.sample = sample;
  rule.acc = aa;
  // the optional margins, after the step (sv_diag.hpp)
  auto finish = [&]() -> sv_status {
    if (!diag) return SV_OK;
    DiagArgs da;
    memset(&da, 0, sizeof da);
    da.logits = logits; da.draft = aa.draft; da.draft_stride = aa.draft_stride; da.draft_offset = aa.draft_offset;
    da.q = q; da.q_bf16 = aa.q_bf16; da.pos0 = pos0; da.n_accepted = n_accepted; da.diag = diag;
    da.rows = at<DiagRow>(ws, L.diag_rows); da.draws = at<DiagDraw>(ws, L.diag_draws);
    da.seed = seed; da.B = sh.B; da.gamma = gamma; da.V = sh.V; da.nch = (sh.V + DIAG_CHUNK - 1) / DIAG_CHUNK;
    da.c = c;
    hipLaunchKernelGGL(k_diag_rows, dim3(da.nch, sh.M), dim3(256), 0, s, da);
    if (sample) hipLaunchKernelGGL(k_diag_draw, dim3(da.nch, sh.B), dim3(256), 0, s, da);
    hipLaunchKernelGGL(k_diag_finish, dim3(sh.B), dim3(256), 0, s, da);
    SV_HIP(hipGetLastError());
    return SV_OK;
  };
  if ((st = run_logits(m, sh, input, kv, L, ws, logits, part, c, &P, s, bf16_head ? &aa : nullptr, fuse,
                       bf16_head ? &rule : nullptr)))
    return st;
  if (rule.done) return finish();
  if (kind == SV_IN_LOGITS && logits_out)
    SV_HIP(hipMemcpyAsync(logits_out, input, size_t(sh.M) * sh.V * 4, hipMemcpyDeviceToDevice, s));

  TimeScope ts(s, 2);
  if (!fuse && !rule.accepted) {
    aa.P = P;
    if ((st = launch_accept(aa, s))) return st;
  }
  if (!sample) return finish();
  SampleArgs sa;
  memset(&sa, 0, sizeof sa);
  sa.logits = logits; sa.q = q; sa.q_bf16 = aa.q_bf16; sa.pos0 = pos0; sa.state = aa.state;
  sa.spart = at<SamplePart>(ws, L.spart); sa.seed = seed; sa.B = sh.B; sa.gamma = gamma; sa.V = sh.V;
  sa.chunk = L.chunk; sa.nch = L.nch; sa.c = c;
  sa.n_accepted = n_accepted; sa.tokens_out = tokens_out; sa.len = aa.len;
  const bool fuse_finish = sh.B <= FUSE_FINISH_MAX_B;
  if (fuse_finish) sa.counter = at<unsigned>(ws, L.counters) + 1;
  hipLaunchKernelGGL(k_sample, dim3(unsigned(L.nch) * unsigned(sh.B)), dim3(256), 0, s, sa);
  if (!fuse_finish) hipLaunchKernelGGL(k_sample_finish, dim3((sh.B + 3) / 4), dim3(256), 0, s, sa);
  SV_HIP(hipGetLastError());
  return finish();
}

}  // namespace

extern "C" {

sv_status verify_forward(const sv_model* m, sv_input_kind kind, const void* input, int32_t B, int32_t gamma,
                         const sv_kv_cache* kv, float* logits, void* ws, size_t* ws_bytes, void* stream) {
  g_err.clear();
  Shape sh;
  sv_status st = check_common(m, kind, input, B, gamma, kv, &sh);
  if (st) return st;
  if (!logits) return fail(SV_ERR_ARG, "logits is NULL");
  Layout L = plan(m, sh, kv, false, false);
  bool query = false;
  if ((st = check_ws(ws, ws_bytes, L, &query))) return st;
  if (query) return SV_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (kind == SV_IN_LOGITS) {
    if (logits != input) SV_HIP(hipMemcpyAsync(logits, input, size_t(sh.M) * sh.V * 4, hipMemcpyDeviceToDevice, s));
    return SV_OK;
  }
  int P = 0;
  return run_logits(m, sh, input, kv, L, ws, logits, nullptr, 0.0f, &P, s);
}

sv_status spec_verify_greedy(const sv_model* m, sv_input_kind kind, const void* input, int32_t B, int32_t gamma,
                             const int32_t* draft, const sv_kv_cache* kv, int32_t* n_accepted, int32_t* tokens_out,
                             float* logits_out, float* diag, void* ws, size_t* ws_bytes, void* stream) {
  return verify_common(m, kind, input, B, gamma, draft, nullptr, SV_F32, 0.0f, 0, nullptr, kv, n_accepted,
                       tokens_out, logits_out, diag, ws, ws_bytes, stream, false);
}

sv_status spec_verify_sample(const sv_model* m, sv_input_kind kind, const void* input, int32_t B, int32_t gamma,
                             const int32_t* draft, const void* q, sv_dtype q_dtype, float temperature, uint64_t seed,
                             const int64_t* pos0, const sv_kv_cache* kv, int32_t* n_accepted, int32_t* tokens_out,
                             float* logits_out, float* diag, void* ws, size_t* ws_bytes, void* stream) {
  return verify_common(m, kind, input, B, gamma, draft, q, q_dtype, temperature, seed, pos0, kv, n_accepted,
                       tokens_out, logits_out, diag, ws, ws_bytes, stream, true);
}

sv_status spec_verify_sample_noalloc(const sv_model* m, sv_input_kind kind, const void* input, int32_t B,
                                     int32_t gamma, const int32_t* draft, const void* q, sv_dtype q_dtype,
                                     float temperature, uint64_t seed, const int64_t* pos0, const sv_kv_cache* kv,
                                     int32_t* n_accepted, int32_t* tokens_out, float* logits_out, float* diag,
                                     void* stream) {
  g_err.clear();
  // the scratch this call needs (the size query of the workspace path: nothing launched)
  size_t need = 0;
  sv_status st = verify_common(m, kind, input, B, gamma, draft, q, q_dtype, temperature, seed, pos0, kv, n_accepted,
                               tokens_out, logits_out, diag, nullptr, &need, stream, true, true);
  if (st) return st;
  if (need > NOALLOC_SCRATCH_BYTES)
    return fail(SV_ERR_UNSUPPORTED, "this request needs %zu bytes of scratch; the allocation-free entry point has %zu "
                "(pass logits_out, or use spec_verify_sample with a workspace)", need, NOALLOC_SCRATCH_BYTES);
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* ptr = nullptr;
  {
    int dev = 0;
    SV_HIP(hipGetDevice(&dev));
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (int(g_scratch.size()) <= dev) g_scratch.resize(dev + 1, nullptr);
    if (!g_scratch[dev]) {
      SV_HIP(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)));
      if (!ptr) return fail(SV_ERR_HIP, "hipGetSymbolAddress returned no address for the scratch array");
      hipLaunchKernelGGL(k_zero_bytes, dim3(1), dim3(256), 0, s, static_cast<unsigned char*>(ptr), size_t(CNT_BYTES));
      SV_HIP(hipGetLastError());
      g_scratch[dev] = ptr;
    }
    ptr = g_scratch[dev];
  }
  size_t have = NOALLOC_SCRATCH_BYTES;
  return verify_common(m, kind, input, B, gamma, draft, q, q_dtype, temperature, seed, pos0, kv, n_accepted,
                       tokens_out, logits_out, diag, ptr, &have, stream, true);
}

sv_status sv_tune_verify(const sv_model* m, int32_t B, int32_t gamma, void* stream) {
  g_err.clear();
  if (!m) return fail(SV_ERR_ARG, "model is NULL");
  if (m->n_layers != 0 || m->wdtype != SV_BF16) return SV_OK;     // only the bf16 LM-head step is tuned
  Shape sh;
  alignas(16) const bf16_t dummy[8] = {};   // a size query reads no argument's memory
  sv_status st = check_common(m, SV_IN_HIDDEN, dummy, B, gamma, nullptr, &sh);
  if (st) return st;
  DevInfo di;
  if ((st = dev_info(&di))) return st;
  const int M = sh.M, K = sh.d, Nv[1] = {sh.V};
  const HeadPlan hp = plan_head(M, K, Nv, 1, di);
  if (!hp.ok) return SV_OK;                                        // no fused step for this shape
  const int steps = K / (32 * hp.S);
  std::vector<int> cand;
  for (int gc : {6, 4, 8})
    if (steps % gc == 0) cand.push_back(gc);
  if (cand.size() < 2) return SV_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // the workspace the greedy step needs (size query), then zero inputs: the stream's
  // timing does not depend on the values
  size_t need = 0;
  int32_t hn = 0, ht = 0;
  if ((st = spec_verify_greedy(m, SV_IN_HIDDEN, dummy, B, gamma, &hn, nullptr, &hn, &ht, nullptr, nullptr, nullptr,
                               &need, stream)))
    return st;
  void *x = nullptr, *dr = nullptr, *n = nullptr, *tok = nullptr, *ws = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  auto cleanup = [&]() {
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    for (void* p : {x, dr, n, tok, ws})
      if (p) (void)hipFree(p);
  };
  const int before = tuned_item(di.dev, M, K, sh.V);
  std::vector<std::vector<float>> times(cand.size());
  hipError_t he = hipSuccess;
  do {
    if ((he = hipMalloc(&x, size_t(M) * K * 2)) || (he = hipMalloc(&dr, size_t(B) * gamma * 4)) ||
        (he = hipMalloc(&n, size_t(B) * 4)) || (he = hipMalloc(&tok, size_t(M) * 4)) || (he = hipMalloc(&ws, need)) ||
        (he = hipMemsetAsync(x, 0, size_t(M) * K * 2, s)) || (he = hipMemsetAsync(dr, 0, size_t(B) * gamma * 4, s)) ||
        (he = hipMemsetAsync(ws, 0, need, s)) || (he = hipEventCreate(&e0)) || (he = hipEventCreate(&e1)))
      break;
    for (int round = 0; round < 3 && he == hipSuccess && !st; ++round)
      for (size_t ci = 0; ci < cand.size() && he == hipSuccess && !st; ++ci) {
        set_tuned_item(di.dev, M, K, sh.V, cand[ci]);
        for (int i = 0; i < 10 && he == hipSuccess && !st; ++i) {
          if (i == 2) he = hipEventRecord(e0, s);
          size_t have = need;
          st = spec_verify_greedy(m, SV_IN_HIDDEN, x, B, gamma, static_cast<const int32_t*>(dr), nullptr,
                                  static_cast<int32_t*>(n), static_cast<int32_t*>(tok), nullptr, nullptr, ws, &have,
                                  stream);
        }
        float ms = 0.0f;
        if (he == hipSuccess && !st && (he = hipEventRecord(e1, s)) == hipSuccess &&
            (he = hipEventSynchronize(e1)) == hipSuccess && (he = hipEventElapsedTime(&ms, e0, e1)) == hipSuccess)
          times[ci].push_back(ms);
      }
  } while (false);
  if (he != hipSuccess || st) {
    set_tuned_item(di.dev, M, K, sh.V, before);
    cleanup();
    if (st) return st;
    return fail(SV_ERR_HIP, "tuning: %s", hipGetErrorString(he));
  }
  size_t best = 0;
  float best_t = 0.0f;
  for (size_t ci = 0; ci < cand.size(); ++ci) {
    std::vector<float> t = times[ci];
    std::sort(t.begin(), t.end());
    const float med = t[t.size() / 2];
    if (ci == 0 || med < best_t) { best = ci; best_t = med; }
  }
  set_tuned_item(di.dev, M, K, sh.V, cand[best]);
  cleanup();
  return SV_OK;
}

int32_t sv_tuned_item(const sv_model* m, int32_t B, int32_t gamma) {
  if (!m || m->n_layers != 0 || m->wdtype != SV_BF16 || B < 1 || gamma < 1) return 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  return tuned_item(dev, B * (gamma + 1), m->d_model, m->vocab);
}

sv_status draft_masked_logits(const sv_masked_head* head, const void* hidden, int32_t M, int32_t top_k,
                              int32_t* clusters, float* logits, float* cluster_logits, void* ws, size_t* ws_bytes,
                              void* stream) {
  g_err.clear();
  if (!head || !hidden || !clusters || !logits) return fail(SV_ERR_ARG, "NULL argument");
  if (!head->embed || !head->centroids) return fail(SV_ERR_ARG, "embed or centroids is NULL");
  if (head->wdtype != SV_BF16) return fail(SV_ERR_DTYPE, "the masked head takes bf16 tables");
  const int V = head->vocab, d = head->d_model, C = head->n_clusters;
  if (C < 1 || V < 2 || V % C) return fail(SV_ERR_SHAPE, "vocab must be a positive multiple of n_clusters");
  if (C > MASK_MAX_CLUSTERS) return fail(SV_ERR_UNSUPPORTED, "at most %d clusters", MASK_MAX_CLUSTERS);
  if (d < 32 || d % 32 || d > 16384) return fail(SV_ERR_SHAPE, "d_model must be a multiple of 32 in [32, 16384]");
  if (M < 1 || M > HEAD_MAX_ROWS) return fail(SV_ERR_ARG, "M must be in [1, %d]", HEAD_MAX_ROWS);
  if (top_k < 1 || top_k > C) return fail(SV_ERR_ARG, "top_k must be in [1, n_clusters]");
  if (!is_aligned(hidden, 16) || !is_aligned(head->embed, 16) || !is_aligned(head->centroids, 16))
    return fail(SV_ERR_ARG, "hidden, embed and centroids must be 16-byte aligned");
  Bump b;
  b.take(CNT_BYTES);                 // the counter block other calls keep state in: never scratch
  const size_t cl_off = cluster_logits ? 0 : b.take(size_t(M) * C * 4);
  Layout L;
  L.total = b.off;   // never 0: a NULL ws is always the size query, never a call that runs
  bool query = false;
  sv_status st = check_ws(ws, ws_bytes, L, &query);
  if (st || query) return st;
  DevInfo di;
  if ((st = dev_info(&di))) return st;
  const int N1[1] = {C};
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* cl = cluster_logits ? cluster_logits : at<float>(ws, cl_off);
  const void* W1[1] = {head->centroids};
  float* O1[1] = {cl};
  if ((st = run_product(static_cast<const bf16_t*>(hidden), M, d, 1, W1, O1, N1, di, s))) return st;
  const int cs = V / C;
  const dim3 gg(top_k, (cs + MASK_ROWS_PER_WG - 1) / MASK_ROWS_PER_WG, M);
  if (top_k <= MASK_FAST_K) {   // the gather's workgroups select the clusters themselves
    if (C <= 2048)
      hipLaunchKernelGGL((k_gather_logits<true, 8>), gg, dim3(256), size_t(d) * 4, s,
                         static_cast<const bf16_t*>(head->embed), static_cast<const bf16_t*>(hidden), clusters, d, cs,
                         top_k, logits, cl, C);
    else
      hipLaunchKernelGGL((k_gather_logits<true, 16>), gg, dim3(256), size_t(d) * 4, s,
                         static_cast<const bf16_t*>(head->embed), static_cast<const bf16_t*>(hidden), clusters, d, cs,
                         top_k, logits, cl, C);
  } else {
    int P = 1;
    while (P < C) P <<= 1;
    hipLaunchKernelGGL(k_select_clusters, dim3(M), dim3(256), 0, s, cl, C, P, top_k, clusters);
    hipLaunchKernelGGL(k_gather_logits<false>, gg, dim3(256), size_t(d) * 4, s, static_cast<const bf16_t*>(head->embed),
                       static_cast<const bf16_t*>(hidden), clusters, d, cs, top_k, logits, nullptr, 0);
  }
  SV_HIP(hipGetLastError());
  return SV_OK;
}

sv_status spec_verify_sample_filtered(const sv_model* m, sv_input_kind kind, const void* input, int32_t B,
                                      int32_t gamma, const int32_t* draft, const void* q, sv_dtype q_dtype,
                                      float temperature, int32_t top_k, float top_p, uint64_t seed, const int64_t* pos0,
                                      const sv_kv_cache* kv, int32_t* n_accepted, int32_t* tokens_out,
                                      float* logits_out, void* ws, size_t* ws_bytes, void* stream) {
  g_err.clear();
  if (!std::isfinite(temperature) || temperature < 0.0f) return fail(SV_ERR_ARG, "temperature must be finite and >= 0");
  if (top_k < 1 || top_k > MASK_FAST_K) return fail(SV_ERR_UNSUPPORTED, "top_k must be in [1, %d]", MASK_FAST_K);
  if (!(top_p > 0.0f && top_p <= 1.0f)) return fail(SV_ERR_ARG, "top_p must be in (0, 1]");
  if (temperature == 0.0f)   // the greedy rule: the filters always keep the argmax
    return verify_common(m, kind, input, B, gamma, draft, nullptr, SV_F32, 0.0f, 0, nullptr, kv, n_accepted,
                         tokens_out, logits_out, nullptr, ws, ws_bytes, stream, false);
  Shape sh;
  sv_status st = check_common(m, kind, input, B, gamma, kv, &sh);
  if (st) return st;
  if (!n_accepted || !tokens_out) return fail(SV_ERR_ARG, "n_accepted and tokens_out must not be NULL");
  if (!draft && kind != SV_IN_TOKENS) return fail(SV_ERR_ARG, "draft is NULL");
  if (!q) return fail(SV_ERR_ARG, "q is NULL");
  if (!pos0) return fail(SV_ERR_ARG, "pos0 is NULL");
  if (q_dtype != SV_F32 && q_dtype != SV_BF16) return fail(SV_ERR_DTYPE, "q_dtype must be SV_F32 or SV_BF16");
  const int nch = (sh.V + FILT_CHUNK - 1) / FILT_CHUNK;
  if (int64_t(nch) * top_k > MASK_MAX_CLUSTERS)
    return fail(SV_ERR_UNSUPPORTED, "vocabulary too large for top_k %d (at most %d entries)", int(top_k),
                MASK_MAX_CLUSTERS / top_k * FILT_CHUNK);
  const bool need_buf = kind != SV_IN_LOGITS && logits_out == nullptr;
  Layout L = plan(m, sh, kv, need_buf, false);
  Bump b;
  b.off = L.total;
  const size_t o_cand = b.take(size_t(sh.M) * nch * top_k * 8);
  const size_t o_id = b.take(size_t(sh.M) * top_k * 4);
  const size_t o_p = b.take(size_t(sh.M) * top_k * 4);
  const size_t o_q = b.take(size_t(sh.M) * top_k * 4);
  const size_t o_dpx = b.take(size_t(sh.M) * 4);
  const size_t o_dqx = b.take(size_t(sh.M) * 4);
  L.total = b.off;
  bool query = false;
  if ((st = check_ws(ws, ws_bytes, L, &query))) return st;
  if (query) return SV_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* logits = kind == SV_IN_LOGITS ? const_cast<float*>(static_cast<const float*>(input))
                                       : (logits_out ? logits_out : at<float>(ws, L.logits));
  if (kind != SV_IN_LOGITS) {
    int P = 0;
    if ((st = run_logits(m, sh, input, kv, L, ws, logits, nullptr, 0.0f, &P, s))) return st;
  } else if (logits_out && logits_out != input) {
    SV_HIP(hipMemcpyAsync(logits_out, input, size_t(sh.M) * sh.V * 4, hipMemcpyDeviceToDevice, s));
  }
  FiltArgs fa;
  memset(&fa, 0, sizeof fa);
  fa.logits = logits; fa.M = sh.M; fa.V = sh.V; fa.G1 = sh.G1; fa.gamma = gamma; fa.B = sh.B;
  fa.top_k = top_k; fa.nch = nch; fa.inv_t = 1.0 / double(temperature); fa.top_p = double(top_p);
  fa.cand = at<unsigned long long>(ws, o_cand);
  fa.kept_id = at<int>(ws, o_id); fa.kept_p = at<float>(ws, o_p); fa.kept_q = at<float>(ws, o_q);
  fa.dpx = at<float>(ws, o_dpx); fa.dqx = at<float>(ws, o_dqx);
  fa.counters = at<unsigned>(ws, L.counters);
  if (draft) { fa.draft = draft; fa.draft_stride = gamma; fa.draft_offset = 0; }
  else { fa.draft = static_cast<const int*>(input); fa.draft_stride = gamma + 1; fa.draft_offset = 1; }
  fa.q = q; fa.q_bf16 = q_dtype == SV_BF16 ? 1 : 0; fa.pos0 = pos0;
  fa.invalid = sh.decoder ? at<int>(ws, L.invalid) : nullptr;
  fa.len = kv ? kv->len : nullptr;
  fa.seed = seed; fa.n_accepted = n_accepted; fa.tokens_out = tokens_out;
  TimeScope ts(s, 2);
  hipLaunchKernelGGL(k_filter_tail, dim3(nch, sh.M), dim3(256), 0, s, fa);
  SV_HIP(hipGetLastError());
  return SV_OK;
}

// The MTP drafter's gamma steps.  [X-thread] "Gemma 4's MTP", [MTP-deep-dive] 3.1-3.4.
sv_status mtp_draft(const sv_drafter* dr, const sv_shared_kv* kv, int32_t B, int32_t gamma,
                    const int32_t* last_token, const void* h_target, float temperature, uint64_t seed,
                    int32_t* draft, void* q, sv_dtype q_dtype, void* ws, size_t* ws_bytes, void* stream) {
  g_err.clear();
  if (!dr || !kv || !last_token || !h_target || !draft) return fail(SV_ERR_ARG, "NULL argument");
  if (!dr->embed || !dr->pre_proj || !dr->layers || !dr->final_norm || !dr->post_proj)
    return fail(SV_ERR_ARG, "drafter weight pointer is NULL");
  if (!kv->k || !kv->v || !kv->len) return fail(SV_ERR_ARG, "shared cache pointer is NULL");
  const int nl = dr->n_layers, D = dr->d_model, H = dr->hidden, nh = dr->n_heads, hd = dr->head_dim;
  const int ff = dr->d_ff, V = dr->vocab, HQ = nh * hd;
  if (nl < 1 || nl > 64) return fail(SV_ERR_ARG, "n_layers must be in [1, 64]");
  if (D < 32 || D % 32 || D > 16384) return fail(SV_ERR_SHAPE, "d_model must be a multiple of 32 in [32, 16384]");
  if (H < 32 || H % 32 || H > 256 * 4 * RMS_VEC) return fail(SV_ERR_SHAPE, "hidden must be a multiple of 32, <= 8192");
  if (hd != 64 && hd != 128) return fail(SV_ERR_SHAPE, "head_dim must be 64 or 128");
  if (nh < 1 || HQ > 16384) return fail(SV_ERR_SHAPE, "n_heads * head_dim must be in [64, 16384]");
  if (ff < 32 || ff % 32) return fail(SV_ERR_SHAPE, "d_ff must be a positive multiple of 32");
  if (V < 2) return fail(SV_ERR_ARG, "vocab must be >= 2");
  if (gamma < 1 || gamma > 15) return fail(SV_ERR_ARG, "gamma must be in [1, 15]");
  if (kv->max_len < 1) return fail(SV_ERR_ARG, "max_len must be >= 1");
  if (!std::isfinite(temperature) || temperature < 0.0f) return fail(SV_ERR_ARG, "temperature must be finite and >= 0");
  const bool greedy = temperature == 0.0f;
  if (!greedy && !q) return fail(SV_ERR_ARG, "q is NULL");
  if (!greedy && q_dtype != SV_F32 && q_dtype != SV_BF16) return fail(SV_ERR_DTYPE, "q_dtype must be SV_F32 or SV_BF16");
  if (!greedy && !is_aligned(q, 16)) return fail(SV_ERR_ARG, "q must be 16-byte aligned");
  const bool masked = dr->centroids != nullptr;
  const int C = dr->n_clusters, tk = dr->top_k_clusters;
  int cs = 1, n_scored = V;
  if (masked) {
    if (C < 1 || V % C) return fail(SV_ERR_SHAPE, "vocab must be a positive multiple of n_clusters");
    if (C > MASK_MAX_CLUSTERS) return fail(SV_ERR_UNSUPPORTED, "at most %d clusters", MASK_MAX_CLUSTERS);
    if (tk < 1 || tk > MASK_FAST_K || tk > C) return fail(SV_ERR_ARG, "top_k_clusters must be in [1, min(64, n_clusters)]");
    cs = V / C;
    n_scored = tk * cs;
  }
  if (B < 1 || B > (masked ? HEAD_MAX_ROWS : 64)) return fail(SV_ERR_ARG, "B must be in [1, %d]", masked ? HEAD_MAX_ROWS : 64);
  if (!is_aligned(h_target, 16) || !is_aligned(dr->embed, 16) || (masked && !is_aligned(dr->centroids, 16)))
    return fail(SV_ERR_ARG, "h_target, embed and centroids must be 16-byte aligned");
  for (int l = 0; l < nl; ++l) {
    for (int i = 0; i < 7; ++i)
      if (!dr->layers[size_t(l) * 7 + i]) return fail(SV_ERR_ARG, "layer %d weight %d is NULL", l, i);
    if (!kv->k[l] || !kv->v[l]) return fail(SV_ERR_ARG, "shared cache of layer %d is NULL", l);
  }
  const int S = std::max(1, std::min((kv->max_len + 255) / 256, ATT_SPLITS_MAX));
  Bump b;
  b.take(CNT_BYTES);                 // the counter block other calls keep state in: never scratch
  const size_t o_lenq = b.take(size_t(B) * 4), o_inv = b.take(size_t(B) * 4), o_tok = b.take(size_t(B) * 4);
  const size_t o_cnt = b.take(size_t(B) * nh * 4);
  const size_t o_attp = b.take(size_t(B) * nh * S * (hd + 2) * 4);
  const size_t o_z = b.take(size_t(B) * 2 * D * 2);
  const size_t o_x = b.take(size_t(B) * H * 4), o_delta = b.take(size_t(B) * H * 4);
  const size_t o_h = b.take(size_t(B) * H * 2), o_f = b.take(size_t(B) * ff * 2);
  const size_t o_q = b.take(size_t(B) * HQ * 4), o_att = b.take(size_t(B) * HQ * 2);
  const size_t o_gate = b.take(size_t(B) * ff * 4), o_up = b.take(size_t(B) * ff * 4);
  const size_t o_gp = b.take(size_t(B) * D * 4), o_g = b.take(size_t(B) * D * 2);
  const size_t o_log = b.take(size_t(B) * n_scored * 4);
  const size_t o_ss = b.take(size_t(GEMM_MAX_WG) * B * 4);
  const size_t o_rope = b.take(size_t(gamma) * B * (hd / 2) * sizeof(float2));
  const size_t o_cl = masked ? b.take(size_t(B) * C * 4) : 0, o_sel = masked ? b.take(size_t(B) * tk * 4) : 0;
  Layout L;
  L.total = b.off;
  bool query = false;
  sv_status st = check_ws(ws, ws_bytes, L, &query);
  if (st || query) return st;
  DevInfo di;
  if ((st = dev_info(&di))) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int* lenq = at<int>(ws, o_lenq);
  int* invalid = at<int>(ws, o_inv);
  int* tok = at<int>(ws, o_tok);
  unsigned* cnt = at<unsigned>(ws, o_cnt);
  float* attp = at<float>(ws, o_attp);
  bf16_t* z = at<bf16_t>(ws, o_z);
  float* x = at<float>(ws, o_x);
  float* delta = at<float>(ws, o_delta);
  bf16_t* h = at<bf16_t>(ws, o_h);
  bf16_t* f = at<bf16_t>(ws, o_f);
  float* qb = at<float>(ws, o_q);
  bf16_t* att = at<bf16_t>(ws, o_att);
  float* gate = at<float>(ws, o_gate);
  float* up = at<float>(ws, o_up);
  float* gp = at<float>(ws, o_gp);
  bf16_t* g = at<bf16_t>(ws, o_g);
  float* logits = at<float>(ws, o_log);
  const int ncnt = B * nh;
  hipLaunchKernelGGL(k_mtp_prep, dim3((std::max(B, ncnt) + 255) / 256), dim3(256), 0, s, kv->len, last_token, lenq,
                     invalid, tok, cnt, ncnt, B, kv->max_len, V);
  if (!greedy && masked) {   // q is written at the scored tokens only
    const size_t bytes = size_t(B) * gamma * V * (q_dtype == SV_BF16 ? 2 : 4);
    hipLaunchKernelGGL(k_zero_bytes, dim3(unsigned(std::min<size_t>((bytes / 16 + 255) / 256 + 1, 4096))), dim3(256),
                       0, s, static_cast<unsigned char*>(q), bytes);
  }
  DecArgs da;
  da.B = B; da.G1 = 1; da.d = H; da.H = nh; da.hd = hd; da.ff = ff; da.V = V; da.max_len = kv->max_len;
  da.n_layers = nl; da.eps = dr->rms_eps;
  const float qscale = 1.0f / sqrtf(float(hd)) * 1.4426950408889634f;
  const bf16_t* hcur = static_cast<const bf16_t*>(h_target);
  // The head over the new hidden state g and the draw of step k.
  auto draft_head_and_sample = [&](int k, bool feed) -> sv_status {
    int32_t* sel = nullptr;
    if (masked) {
      float* cl = at<float>(ws, o_cl);
      sel = at<int32_t>(ws, o_sel);
      const void* w1[1] = {dr->centroids};
      float* o1[1] = {cl};
      const int n1[1] = {C};
      sv_status r = run_product(g, B, D, 1, w1, o1, n1, di, s);
      if (r) return r;
      // the gather's workgroups select the kept clusters themselves (tk <= MASK_FAST_K)
      const dim3 gg(tk, (cs + MASK_ROWS_PER_WG - 1) / MASK_ROWS_PER_WG, B);
      if (C <= 2048)
        hipLaunchKernelGGL((k_gather_logits<true, 8>), gg, dim3(256), size_t(D) * 4, s,
                           static_cast<const bf16_t*>(dr->embed), g, sel, D, cs, tk, logits, cl, C);
      else
        hipLaunchKernelGGL((k_gather_logits<true, 16>), gg, dim3(256), size_t(D) * 4, s,
                           static_cast<const bf16_t*>(dr->embed), g, sel, D, cs, tk, logits, cl, C);
    } else {
      const void* w1[1] = {dr->embed};
      float* o1[1] = {logits};
      const int n1[1] = {V};
      sv_status r = run_product(g, B, D, 1, w1, o1, n1, di, s);
      if (r) return r;
    }
    DraftSampleArgs sa;
    sa.logits = logits; sa.clusters = sel; sa.n = n_scored; sa.cs = cs; sa.top_k = tk; sa.V = V; sa.gamma = gamma;
    sa.k = k; sa.inv_t = greedy ? 0.0f : 1.0f / temperature; sa.greedy = greedy ? 1 : 0; sa.seed = seed;
    sa.len = kv->len; sa.invalid = invalid; sa.draft = draft; sa.tok = tok; sa.q = q;
    sa.q_bf16 = q_dtype == SV_BF16 ? 1 : 0;
    sa.z = feed ? z : nullptr;
    sa.embed = static_cast<const bf16_t*>(dr->embed);
    sa.x_res = x;
    sa.D = D;
    sa.H = H;
    hipLaunchKernelGGL(k_mtp_sample, dim3(B), dim3(MTP_SAMPLE_THREADS), 0, s, sa);
    return SV_OK;
  };
  // Every product on the k-split kernel: the RMSNorms happen while the next product
  // stages its rows from the float32 residual stream (sums of squares left by the
  // products that add into it), as in the target decoder.
  bool fused = B <= ACC_MAX_ROWS;
  {
    const int nH[1] = {H}, nQ[1] = {HQ}, nF[2] = {ff, ff}, nD[1] = {D};
    fused = fused && plan_head(B, 2 * D, nH, 1, di).ok && plan_head(B, H, nQ, 1, di).ok &&
            plan_head(B, HQ, nH, 1, di).ok && plan_head(B, H, nF, 2, di).ok && plan_head(B, ff, nH, 1, di).ok &&
            plan_head(B, H, nD, 1, di).ok;
  }
  float* ss = at<float>(ws, o_ss);
  float2* rope = at<float2>(ws, o_rope);
  if (fused) {
    const int nrope = gamma * B * (hd / 2);
    hipLaunchKernelGGL(k_mtp_rope_table, dim3(std::min((nrope + 255) / 256, 1024)), dim3(256), 0, s, kv->len, rope, B,
                       gamma, hd, dr->rope_theta);
  }
  for (int k = 0; k < gamma && fused; ++k) {
    // step 0 joins [embedding, target hidden state]; later steps' inputs were written by
    // the previous step's conversion (hidden half) and draw (embedding half, cleared x)
    if (k == 0)
      hipLaunchKernelGGL(k_mtp_join, dim3(B), dim3(256), 0, s, tok, static_cast<const bf16_t*>(dr->embed), hcur, z, D,
                         x, H);
    const bool pairs = swiglu_paired(B, H, ff, di);
    ProductFuse fr;
    fr.residual = true;
    fr.pairable = pairs;
    fr.ss_out = ss;
    int parts = 1;
    {
      const void* w1[1] = {dr->pre_proj};
      float* o1[1] = {x};
      const int n1[1] = {H};
      if ((st = run_product_fused(z, B, 2 * D, 1, w1, o1, n1, fr, &parts, di, s))) return st;
    }
    for (int l = 0; l < nl; ++l) {
      const void* const* w = dr->layers + size_t(l) * 7;
      ProductFuse fn;
      fn.Xf = x; fn.ss_in = ss; fn.ss_parts = parts; fn.eps = dr->rms_eps; fn.pairable = pairs;
      fn.norm_w = static_cast<const bf16_t*>(w[0]);
      {
        const void* w1[1] = {w[1]};
        float* o1[1] = {qb};
        const int n1[1] = {HQ};
        if ((st = run_product_fused(nullptr, B, H, 1, w1, o1, n1, fn, nullptr, di, s))) return st;
      }
      const bf16_t* kc = static_cast<const bf16_t*>(kv->k[l]);
      const bf16_t* vc = static_cast<const bf16_t*>(kv->v[l]);
      const float2* rk = rope + size_t(k) * B * (hd / 2);   // RoPE applied while the queries are staged
      if (hd == 128)
        hipLaunchKernelGGL((k_attn<128, 2>), dim3(nh, B, S), dim3(256), 0, s, qb, kc, vc, lenq, invalid, attp, att,
                           cnt, da, 0, S, 1, qscale, rk);
      else
        hipLaunchKernelGGL((k_attn<64, 2>), dim3(nh, B, S), dim3(256), 0, s, qb, kc, vc, lenq, invalid, attp, att,
                           cnt, da, 0, S, 1, qscale, rk);
      {
        const void* w1[1] = {w[2]};
        float* o1[1] = {x};
        const int n1[1] = {H};
        if ((st = run_product_fused(att, B, HQ, 1, w1, o1, n1, fr, &parts, di, s))) return st;
      }
      fn.ss_parts = parts;
      fn.norm_w = static_cast<const bf16_t*>(w[3]);
      {
        const void* w2[2] = {w[4], w[5]};
        float* o2[2] = {gate, up};
        const int n2[2] = {ff, ff};
        ProductFuse fg = fn;
        fg.silu_out = f;   // SwiGLU in the epilogue
        if ((st = run_product_fused(nullptr, B, H, 2, w2, o2, n2, fg, nullptr, di, s))) return st;
      }
      {
        const void* w1[1] = {w[6]};
        float* o1[1] = {x};
        const int n1[1] = {H};
        if ((st = run_product_fused(f, B, ff, 1, w1, o1, n1, fr, &parts, di, s))) return st;
      }
    }
    {
      ProductFuse fn;
      fn.Xf = x; fn.ss_in = ss; fn.ss_parts = parts; fn.eps = dr->rms_eps; fn.pairable = pairs;
      fn.norm_w = static_cast<const bf16_t*>(dr->final_norm);
      const void* w1[1] = {dr->post_proj};
      float* o1[1] = {gp};
      const int n1[1] = {D};
      if ((st = run_product_fused(nullptr, B, H, 1, w1, o1, n1, fn, nullptr, di, s))) return st;
    }
    hipLaunchKernelGGL(k_f32_to_bf16, dim3((B * D + 255) / 256), dim3(256), 0, s, gp, g, B * D,
                       k + 1 < gamma ? z : nullptr, D);
    hcur = g;
    if ((st = draft_head_and_sample(k, k + 1 < gamma))) return st;
  }
  for (int k = 0; k < gamma && !fused; ++k) {
    hipLaunchKernelGGL(k_mtp_join, dim3(B), dim3(256), 0, s, tok, static_cast<const bf16_t*>(dr->embed), hcur, z, D,
                       nullptr, H);
    {
      const void* w1[1] = {dr->pre_proj};
      float* o1[1] = {x};
      const int n1[1] = {H};
      if ((st = run_product(z, B, 2 * D, 1, w1, o1, n1, di, s))) return st;
    }
    const float* pending = nullptr;
    for (int l = 0; l < nl; ++l) {
      const void* const* w = dr->layers + size_t(l) * 7;
      hipLaunchKernelGGL(k_add_rmsnorm, dim3(B), dim3(256), 0, s, x, pending, static_cast<const bf16_t*>(w[0]), h, H,
                         dr->rms_eps);
      {
        const void* w1[1] = {w[1]};
        float* o1[1] = {qb};
        const int n1[1] = {HQ};
        if ((st = run_product(h, B, H, 1, w1, o1, n1, di, s))) return st;
      }
      hipLaunchKernelGGL(k_mtp_rope_q, dim3(B, nh), dim3(hd / 2), 0, s, qb, kv->len, k, nh, hd, dr->rope_theta);
      const bf16_t* kc = static_cast<const bf16_t*>(kv->k[l]);
      const bf16_t* vc = static_cast<const bf16_t*>(kv->v[l]);
      if (hd == 128)
        hipLaunchKernelGGL((k_attn<128, 2>), dim3(nh, B, S), dim3(256), 0, s, qb, kc, vc, lenq, invalid, attp, att,
                           cnt, da, 0, S, 1, qscale);
      else
        hipLaunchKernelGGL((k_attn<64, 2>), dim3(nh, B, S), dim3(256), 0, s, qb, kc, vc, lenq, invalid, attp, att,
                           cnt, da, 0, S, 1, qscale);
      {
        const void* w1[1] = {w[2]};
        float* o1[1] = {delta};
        const int n1[1] = {H};
        if ((st = run_product(att, B, HQ, 1, w1, o1, n1, di, s))) return st;
      }
      hipLaunchKernelGGL(k_add_rmsnorm, dim3(B), dim3(256), 0, s, x, delta, static_cast<const bf16_t*>(w[3]), h, H,
                         dr->rms_eps);
      {
        const void* w2[2] = {w[4], w[5]};
        float* o2[2] = {gate, up};
        const int n2[2] = {ff, ff};
        if ((st = run_product(h, B, H, 2, w2, o2, n2, di, s))) return st;
      }
      hipLaunchKernelGGL(k_silu_mul, dim3((B * ff + 255) / 256), dim3(256), 0, s, gate, up, f, B * ff);
      {
        const void* w1[1] = {w[6]};
        float* o1[1] = {delta};
        const int n1[1] = {H};
        if ((st = run_product(f, B, ff, 1, w1, o1, n1, di, s))) return st;
      }
      pending = delta;
    }
    hipLaunchKernelGGL(k_add_rmsnorm, dim3(B), dim3(256), 0, s, x, pending, static_cast<const bf16_t*>(dr->final_norm),
                       h, H, dr->rms_eps);
    {
      const void* w1[1] = {dr->post_proj};
      float* o1[1] = {gp};
      const int n1[1] = {D};
      if ((st = run_product(h, B, H, 1, w1, o1, n1, di, s))) return st;
    }
    hipLaunchKernelGGL(k_f32_to_bf16, dim3((B * D + 255) / 256), dim3(256), 0, s, gp, g, B * D, nullptr, D);
    hcur = g;
    if ((st = draft_head_and_sample(k, false))) return st;
  }
  SV_HIP(hipGetLastError());
  return SV_OK;
}
// Round policies.  [MTP-drafters] 6, [MTP-deep-dive] 5.1, [Self-spec] 3.3.
sv_status round_pad_drafts(int32_t B, int32_t G, int32_t V, int32_t* gamma_b, int32_t* draft, void* q,
                           sv_dtype q_dtype, float tau, void* ws, size_t* ws_bytes, void* stream) {
  g_err.clear();
  if (B < 1 || G < 1 || G > 15 || V < 1) return fail(SV_ERR_ARG, "need B >= 1, 1 <= G <= 15, V >= 1");
  if (!gamma_b || !draft) return fail(SV_ERR_ARG, "gamma_b and draft must not be NULL");
  if (!std::isfinite(tau) || tau < 0.0f) return fail(SV_ERR_ARG, "tau must be finite and >= 0");
  if (tau > 0.0f && !q) return fail(SV_ERR_ARG, "the confidence cut needs q");
  if (q && q_dtype != SV_F32 && q_dtype != SV_BF16) return fail(SV_ERR_DTYPE, "q_dtype must be SV_F32 or SV_BF16");
  Bump b;
  b.take(CNT_BYTES);                 // the counter block other calls keep state in: never scratch
  const size_t o_conf = tau > 0.0f ? b.take(size_t(B) * G * 4) : 0;
  Layout L;
  L.total = tau > 0.0f ? b.off : 0;
  bool query = false;
  sv_status st = check_ws(ws, ws_bytes, L, &query);
  if (st || query) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int qb = q_dtype == SV_BF16 ? 1 : 0;
  float* conf = nullptr;
  if (tau > 0.0f) {
    conf = at<float>(ws, o_conf);
    hipLaunchKernelGGL(k_round_conf, dim3(G, B), dim3(256), 0, s, q, qb, G, V, conf);
  }
  hipLaunchKernelGGL(k_round_cut, dim3((B + 255) / 256), dim3(256), 0, s, gamma_b, conf, tau, B, G);
  hipLaunchKernelGGL(k_round_pad, dim3(G, B, q ? (V + 4095) / 4096 : 1), dim3(256), 0, s, gamma_b, draft, q, qb, G, V);
  SV_HIP(hipGetLastError());
  return SV_OK;
}

sv_status round_update_gamma(int32_t B, const int32_t* n_accepted, int32_t* gamma_b, int32_t gamma_min,
                             int32_t gamma_max, void* stream) {
  g_err.clear();
  if (B < 1 || !n_accepted || !gamma_b) return fail(SV_ERR_ARG, "need B >= 1 and non-NULL arrays");
  if (gamma_min < 1 || gamma_min > gamma_max || gamma_max > 15)
    return fail(SV_ERR_ARG, "need 1 <= gamma_min <= gamma_max <= 15");
  hipLaunchKernelGGL(k_round_schedule, dim3((B + 255) / 256), dim3(256), 0, static_cast<hipStream_t>(stream),
                     n_accepted, gamma_b, B, gamma_min, gamma_max);
  SV_HIP(hipGetLastError());
  return SV_OK;
}

sv_status round_select_candidates(int32_t B, int32_t C, int32_t G1, const int32_t* n_accepted,
                                  const int32_t* tokens, int32_t* best, int32_t* n_out, int32_t* tokens_out,
                                  void* stream) {
  g_err.clear();
  if (B < 1 || C < 1 || G1 < 2 || G1 > 16) return fail(SV_ERR_ARG, "need B >= 1, C >= 1, 2 <= G1 <= 16");
  if (!n_accepted || !tokens || !n_out || !tokens_out) return fail(SV_ERR_ARG, "NULL array");
  hipLaunchKernelGGL(k_round_select, dim3((B + 255) / 256), dim3(256), 0, static_cast<hipStream_t>(stream),
                     n_accepted, tokens, B, C, G1, best, n_out, tokens_out);
  SV_HIP(hipGetLastError());
  return SV_OK;
}

sv_status sv_set_option(int32_t option, int64_t value) {
  g_err.clear();
  switch (option) {
    case SV_OPT_WAIT_LIMIT:
      g_wait_limit.store(value < 0 ? HEAD_SPIN_LIMIT : unsigned(std::min<int64_t>(value, 0xfffffff0LL)),
                         std::memory_order_relaxed);
      return SV_OK;
    default:
      return fail(SV_ERR_ARG, "unknown option %d", int(option));
  }
}

int32_t sv_version(void) { return VERSION; }

const char* sv_status_string(int32_t status) {
  switch (status) {
    case SV_OK: return "SV_OK";
    case SV_ERR_ARG: return "SV_ERR_ARG";
    case SV_ERR_DTYPE: return "SV_ERR_DTYPE";
    case SV_ERR_SHAPE: return "SV_ERR_SHAPE";
    case SV_ERR_WORKSPACE: return "SV_ERR_WORKSPACE";
    case SV_ERR_HIP: return "SV_ERR_HIP";
    case SV_ERR_UNSUPPORTED: return "SV_ERR_UNSUPPORTED";
    default: return "SV_ERR_UNKNOWN";
  }
}

const char* sv_last_error(void) { return g_err.c_str(); }

sv_status sv_timing_enable(int32_t mask) {
  std::lock_guard<std::mutex> lk(g_timer.mu);
  for (auto& r : g_timer.recs) { g_timer.pool.push_back(r.a); g_timer.pool.push_back(r.b); }
  g_timer.recs.clear();
  g_timer.mask = unsigned(mask) & 7u;
  return SV_OK;
}

sv_status sv_timing_read(int32_t which, double* total_ms, int64_t* count) {
  if (!total_ms || !count) return fail(SV_ERR_ARG, "NULL output");
  std::lock_guard<std::mutex> lk(g_timer.mu);
  double tot = 0.0;
  int64_t n = 0;
  for (auto& r : g_timer.recs) {
    if (r.which != which) continue;
    SV_HIP(hipEventSynchronize(r.b));
    float ms = 0.0f;
    SV_HIP(hipEventElapsedTime(&ms, r.a, r.b));
    tot += ms;
    ++n;
  }
  *total_ms = tot;
  *count = n;
  return SV_OK;
}

}  // extern "C"
