// abi.hip -- the C ABI declared in include/qlora.h: argument checks, workspace
// planning, the NF4 codebook, kernel sequencing and measurement hooks.
//
// Every entry point validates all of its arguments before its first HIP call,
// returns a QLORA_E* code instead of aborting, and enqueues its kernels on the
// caller's stream without synchronizing or allocating device memory.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "adamw.h"
#include "device.h"
#include "launch.h"
#include "recip_div.h"
#include "qlora.h"
#include "qlora_timing.h"

using namespace qlora;

LaunchEvents &qlora::launch_events() {
  static thread_local LaunchEvents ev;
  return ev;
}

bool &qlora::launch_refused() {
  static thread_local bool refused = false;
  return refused;
}

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

// ------------------------------------------------------------------ codebook
// Standard-normal quantile by Newton's method on the CDF written with erfc,
// started from the logistic approximation of the normal CDF.
double normal_quantile(double p) {
  double x = log(p / (1.0 - p)) / 1.702;
  for (int it = 0; it < 64; ++it) {
    const double f = 0.5 * erfc(-x / sqrt(2.0)) - p;
    const double dens = exp(-0.5 * x * x) / sqrt(2.0 * M_PI);
    const double dx = f / dens;
    x -= dx;
    if (fabs(dx) <= 1e-17 * (1.0 + fabs(x))) break;
  }
  return x;
}

struct Codebook {
  Levels lv;
  Thresholds thr;
};

// Levels: quantiles at probabilities equally spaced between 1/2 and
// p_hi = 1 - (1/30 + 1/32)/2 (seven negative, eight positive, plus zero),
// divided by the largest, rounded to binary32 once.  Thresholds: for each pair
// of neighbouring levels, the largest binary32 value not above their exact
// midpoint, so that x > thr_i  <=>  x is strictly above the midpoint, and a
// value exactly on a midpoint keeps the lower code.
const Codebook &codebook() {
  static Codebook cb;
  static std::once_flag once;
  std::call_once(once, [] {
    const double p_hi = 1.0 - 0.5 * (1.0 / 30.0 + 1.0 / 32.0);
    const double top = normal_quantile(p_hi);
    double v[16];
    for (int j = 7; j >= 1; --j) v[7 - j] = -normal_quantile(0.5 + j * (p_hi - 0.5) / 7.0) / top;
    v[7] = 0.0;
    for (int i = 1; i <= 8; ++i) v[7 + i] = normal_quantile(0.5 + i * (p_hi - 0.5) / 8.0) / top;
    v[15] = 1.0;  // top / top
    v[0] = -1.0;
    for (int i = 0; i < 16; ++i) cb.lv.v[i] = (float)v[i];
    for (int i = 0; i < 15; ++i) {
      const double mid = ((double)cb.lv.v[i] + (double)cb.lv.v[i + 1]) * 0.5;  // exact in binary64
      float t = (float)mid;
      if ((double)t > mid) t = nextafterf(t, -INFINITY);
      cb.thr.v[i] = t;
    }
  });
  return cb;
}

// ------------------------------------------------------------ device check
std::atomic<int> g_dev_ok[64];

int check_device(int *dev_out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return fail(QLORA_ENODEV, "no HIP device available");
  }
  if (dev < 64) {
    int st = g_dev_ok[dev].load(std::memory_order_relaxed);
    if (st == 0) {
      hipDeviceProp_t prop;
      if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
        (void)hipGetLastError();
        return fail(QLORA_ENODEV, "hipGetDeviceProperties failed for device %d", dev);
      }
      st = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
      g_dev_ok[dev].store(st, std::memory_order_relaxed);
    }
    if (st < 0) return fail(QLORA_ENODEV, "device %d is not gfx950 (this library holds gfx950 code only)", dev);
  }
  if (dev_out) *dev_out = dev;
  return QLORA_OK;
}

bool debug_sync() {
  static int v = -1;
  if (v < 0) {
    const char *e = getenv("QLORA_DEBUG_SYNC");
    v = (e && e[0] == '1') ? 1 : 0;
  }
  return v == 1;
}

// -------------------------------------------------- allocation-free forward
// The workspace of qlora_linear_fwd_noalloc: one array per GPU, alive until the process ends.  In
// host code `scratch` is only a host-side stand-in for the array; its device address comes from
// hipGetSymbolAddress, taken once per device with that device current, and only that address is
// handed to kernels.
constexpr size_t kScratchBytes = (size_t)128 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
std::mutex g_scratch_mu;
void *g_scratch_ptr[64] = {};

int scratch_address(int dev, void **out) {
  if (dev < 0 || dev >= 64) return fail(QLORA_ENODEV, "device index %d out of range for the static workspace", dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return fail(QLORA_EHIP, "hipGetSymbolAddress of the static workspace failed: %s", hipGetErrorString(e));
    }
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return QLORA_OK;
}

// --------------------------------------------------------------- timing
std::mutex g_tmu;
std::vector<std::string> g_timed;  // kernel names being timed; "*" = all
std::atomic<int> g_ntimed{0};      // g_timed.size(): with none enabled a launch takes no lock
struct EventPair {
  hipEvent_t a, b;
  int dev;
};
std::map<std::string, std::vector<EventPair>> g_events;
// Events read back are kept for reuse, per device.
std::map<int, std::vector<hipEvent_t>> g_event_pool;

hipEvent_t pooled_event(int dev) {  // caller holds g_tmu
  auto &pool = g_event_pool[dev];
  if (!pool.empty()) {
    hipEvent_t e = pool.back();
    pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  return e;
}

bool is_timed(const char *kname) {
  for (const auto &n : g_timed)
    if (n == "*" || n == kname) return true;
  return false;
}

// A timed launch gets a pair of events stamped by its own dispatch packet.
struct Timed {
  hipEvent_t a = nullptr, b = nullptr;
  int dev = 0;
  std::string name;
  Timed(const char *kname) {
    if (g_ntimed.load(std::memory_order_acquire) == 0) return;
    std::lock_guard<std::mutex> lk(g_tmu);
    if (!is_timed(kname)) return;
    if (hipGetDevice(&dev) != hipSuccess) {
      (void)hipGetLastError();
      return;
    }
    a = pooled_event(dev);
    b = a ? pooled_event(dev) : nullptr;
    if (!b) {
      if (a) g_event_pool[dev].push_back(a);
      a = nullptr;
      return;
    }
    name = kname;
    launch_events() = LaunchEvents{a, b};
  }
  ~Timed() {
    if (!a) return;
    launch_events() = LaunchEvents{};
    std::lock_guard<std::mutex> lk(g_tmu);
    g_events[name].push_back({a, b, dev});
  }
};

int launched(hipError_t e, const char *what, hipStream_t s) {
  if (launch_refused()) {
    launch_refused() = false;
    return fail(QLORA_EINVAL, "%s: a grid dimension would reach 2^32 work-items", what);
  }
  if (e == hipSuccess && debug_sync()) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail(QLORA_EHIP, "%s: %s", what, hipGetErrorString(e));
  return QLORA_OK;
}

#define LAUNCH(name, call)                             \
  do {                                                 \
    hipError_t e_;                                     \
    {                                                  \
      Timed t_(name);                                  \
      e_ = (call);                                     \
    }                                                  \
    int rc_ = launched(e_, name, s);                   \
    if (rc_ != QLORA_OK) return rc_;                   \
  } while (0)

// ------------------------------------------------------------- validation
bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
constexpr int64_t kMaxDim = (int64_t)1 << 22;
// Largest weight (n_out n_in) and activation (T n_out, T n_in) element counts: every launch then stays
// below 2^32 work-items per grid dimension (the dequantization runs one work-item per 8 weights, the
// ordered finalize of a split reduction one per output element).
constexpr int64_t kMaxWeights = (int64_t)1 << 34;
constexpr int64_t kMaxActs = ((int64_t)1 << 32) - 256;

int check_acts(int64_t T, int64_t n_out, int64_t n_in) {
  if (T * n_out > kMaxActs || T * n_in > kMaxActs)
    return fail(QLORA_EINVAL, "T x n_out and T x n_in must stay below 2^32 (got T=%lld, %lld x %lld)", (long long)T,
                (long long)n_out, (long long)n_in);
  return QLORA_OK;
}

int check_nf4(const qlora_nf4 *q, bool for_gemm) {
  if (!q) return fail(QLORA_EINVAL, "q is NULL");
  if (!q->codes || !q->absmax_q || !q->absmax_step) return fail(QLORA_EINVAL, "q has a NULL array");
  if (!aligned16(q->codes) || !aligned16(q->absmax_q) || !aligned16(q->absmax_step))
    return fail(QLORA_EINVAL, "q arrays must be 16-byte aligned");
  if (q->n_out < 1 || q->n_in < 64 || q->n_in % 64 != 0)
    return fail(QLORA_EINVAL, "need n_out >= 1 and n_in a positive multiple of 64 (got %lld x %lld)",
                (long long)q->n_out, (long long)q->n_in);
  if (q->n_out > kMaxDim || q->n_in > kMaxDim || q->n_out * q->n_in > kMaxWeights)
    return fail(QLORA_EINVAL, "weight too large (%lld x %lld; at most 2^22 per side and 2^34 weights)",
                (long long)q->n_out, (long long)q->n_in);
  if (for_gemm && q->n_out % 8 != 0) return fail(QLORA_EINVAL, "n_out must be a multiple of 8 (got %lld)", (long long)q->n_out);
  return QLORA_OK;
}

// --------------------------------------------------------------- planning
constexpr size_t kAlign = 256;
size_t up(size_t x, size_t a) { return (x + a - 1) / a * a; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct Split {
  int n = 0;
  int64_t kchunk = 0;
};

// Reduction split of a skinny LoRA GEMM with M output rows.
Split plan_skinny(int64_t M, int64_t Kred) {
  Split sp;
  if (Kred <= 0 || M <= 0) return sp;
  skinny_plan(M, Kred, &sp.n, &sp.kchunk);
  return sp;
}

struct Plan {
  int64_t rp = 0;  // row length of the padded rank-wide copies (r rounded up to 64)
  int rn = 0;      // rank columns of the skinny GEMMs' partial sums
  int64_t rv = 0;  // r rounded up to 8: rank columns read from padded copies
  size_t off_bp = 0, off_v = 0, off_du = 0, off_part = 0, off_part2 = 0, total = 0;
  Split su, sdu, sdb, sda;
  bool gemv = false;  // forward through the small-token kernels
  int gemv_rg = 0, gemv_w = 0, gemv_split = 0, gemv_main = 0;
  bool gemv_rows = false;  // one or two tokens: the row-streaming kernel (gemv_split = its U K ranges)
  bool gemv_mrows = false; // 3..64 tokens: the row-group kernel (gemv_split = its U K ranges)
  int fwd_split = 1;       // reduction ranges of the tiled forward GEMM (partial sums in the part region)
  size_t off_upart = 0;
};

// Row-streaming GEMV: the K ranges of its U partials (the main grid is sized at launch).
int gemv_rows_usplit(int64_t K) {
  for (int c = 16; c > 1; --c)
    if (K % (c * 128) == 0) return c;
  return 1;
}

bool use_gemv(int64_t T, int64_t K) { return T >= 1 && T <= kGemvMaxT && K % 128 == 0; }

Plan make_plan(int op, int64_t T, int64_t N, int64_t K, int32_t r) {
  Plan p;
  p.rp = (int64_t)up((size_t)r, 64);
  p.rn = skinny_rn(r);
  p.rv = (int64_t)up((size_t)r, 8);
  size_t off = 0;
  p.off_bp = off;
  off = up(off + (size_t)(N * p.rp * 2), kAlign);
  p.off_v = off;  // fwd: V = bf16(s U) padded; bwd: U padded
  off = up(off + (size_t)(T * p.rp * 2), kAlign);
  size_t part = 0;
  if (op == QLORA_OP_FWD || op == QLORA_OP_FWD_DROPOUT || op == QLORA_OP_FWD_MULTI) {
    p.su = plan_skinny(T, K);
    part = (size_t)p.su.n * T * p.rn * 4;
    if (op == QLORA_OP_FWD && use_gemv(T, K) && nf4_gemv_rows_ok(T, K)) {  // one or two tokens
      p.gemv = p.gemv_rows = true;
      p.gemv_split = gemv_rows_usplit(K);
      part = up((size_t)nf4_gemv_rows_nseg(T, K) * T * N * 4, kAlign);  // one partial per row segment
      p.off_upart = part;
      part += (size_t)4 * p.gemv_split * T * r * 4;
    } else if (op == QLORA_OP_FWD && use_gemv(T, K) && nf4_gemv_mrows_nseg(T, K) > 0) {  // 3..64 tokens
      p.gemv = p.gemv_mrows = true;
      p.gemv_split = gemv_rows_usplit(K);
      part = up((size_t)nf4_gemv_mrows_nparts(T, K) * T * N * 4, kAlign);  // per segment or group of segments
      p.off_upart = part;
      part += (size_t)4 * p.gemv_split * T * r * 4;
    } else if ((op == QLORA_OP_FWD || op == QLORA_OP_FWD_MULTI) && use_gemv(T, K)) {  // dropout: the tiled path
      p.gemv = true;
      nf4_gemv_plan(T, N, K, &p.gemv_rg, &p.gemv_w, &p.gemv_split, &p.gemv_main);
      part = up((size_t)p.gemv_split * T * N * 4, kAlign);
      p.off_upart = part;  // relative to off_part
      part += (size_t)4 * p.gemv_split * T * r * 4;
    }
    if (!p.gemv) {  // the tiled GEMM; its partial sums follow U's, which are consumed first
      p.fwd_split = nf4_gemm_fwd_split(nf4_gemm_pick_tile_fwd(T, N, K), T, N, K);
      const size_t gp = p.fwd_split > 1 ? (size_t)p.fwd_split * T * N * 4 : 0;
      part = gp > part ? gp : part;
    }
  } else {
    p.off_du = off;
    off = up(off + (size_t)(T * p.rp * 2), kAlign);
    p.su = plan_skinny(T, K);
    p.sdu = plan_skinny(T, N);
    p.sdb = plan_skinny(N, T);
    p.sda = plan_skinny(K, T);
    // dA's partial sums get a region of their own, so that dB and dA are finalized in one launch
    const size_t cands[3] = {(size_t)p.su.n * T * p.rn * 4, (size_t)p.sdu.n * T * p.rn * 4,
                             (size_t)p.sdb.n * N * p.rn * 4};
    for (size_t c : cands) part = c > part ? c : part;
    p.off_part2 = up(off + part, kAlign);
    part = p.off_part2 - off + (size_t)p.sda.n * K * p.rn * 4;
  }
  p.off_part = off;
  off = up(off + part, kAlign);
  p.total = off;
  return p;
}

int check_lora_args(int64_t T, const qlora_nf4 *q, const void *A, const void *B, int32_t r, float alpha) {
  int rc = check_nf4(q, true);
  if (rc) return rc;
  if (T < 0 || T > kMaxDim) return fail(QLORA_EINVAL, "T must be in [0, 2^22] (got %lld)", (long long)T);
  if ((rc = check_acts(T, q->n_out, q->n_in))) return rc;
  if (r < 1 || r > QLORA_MAX_RANK) return fail(QLORA_EINVAL, "r must be in [1, %d] (got %d)", QLORA_MAX_RANK, (int)r);
  if (!isfinite(alpha)) return fail(QLORA_EINVAL, "alpha must be finite");
  if (!A || !B) return fail(QLORA_EINVAL, "A and B must not be NULL");
  if (!aligned16(A) || !aligned16(B)) return fail(QLORA_EINVAL, "A and B must be 16-byte aligned");
  return QLORA_OK;
}

// Dropout probability p in [0, 1): drop threshold D = round_half_even(p 65536)
// on 16-bit draws, scale q = fl32(1 / (1 - p)).
int check_dropout(float p, const void *mask, int64_t T) {
  if (!(p >= 0.f && p < 1.f)) return fail(QLORA_EINVAL, "dropout probability must be in [0, 1) (got %g)", (double)p);
  if (T > 0 && !mask) return fail(QLORA_EINVAL, "the keep-bit mask must not be NULL");
  if (mask && !aligned16(mask)) return fail(QLORA_EINVAL, "the keep-bit mask must be 16-byte aligned");
  return QLORA_OK;
}

DropParams drop_params(float p, uint8_t *mask, uint64_t seed, uint64_t offset) {
  DropParams d;
  d.mask = mask;
  d.thr = (uint32_t)nearbyint((double)p * 65536.0);
  d.q = (float)(1.0 / (1.0 - (double)p));
  d.key0 = (uint32_t)seed;
  d.key1 = (uint32_t)(seed >> 32);
  d.off0 = (uint32_t)offset;
  d.off1 = (uint32_t)(offset >> 32);
  return d;
}

int check_ws(int op, int64_t T, int64_t N, int64_t K, int32_t r, const void *ws, size_t ws_bytes, Plan *p) {
  *p = make_plan(op, T, N, K, r);
  if (ws_bytes < p->total)
    return fail(QLORA_EWORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, p->total);
  if (p->total > 0 && (!ws || ((uintptr_t)ws & (kAlign - 1))))
    return fail(QLORA_EINVAL, "workspace must be non-NULL and 256-byte aligned");
  return QLORA_OK;
}

}  // namespace

// =========================================================== C ABI
extern "C" {

const char *qlora_strerror(int code) {
  switch (code) {
    case QLORA_OK: return "ok";
    case QLORA_EINVAL: return "invalid argument";
    case QLORA_EWORKSPACE: return "workspace too small";
    case QLORA_ENODEV: return "no gfx950 device";
    case QLORA_EHIP: return "HIP error";
    default: return "unknown error";
  }
}

const char *qlora_last_error(void) { return g_err; }

int qlora_nf4_storage(int64_t n_out, int64_t n_in, size_t *codes_bytes, size_t *absmax_q_bytes,
                      size_t *absmax_step_bytes) {
  if (!codes_bytes || !absmax_q_bytes || !absmax_step_bytes) return fail(QLORA_EINVAL, "NULL output pointer");
  if (n_out < 1 || n_in < 64 || n_in % 64 != 0 || n_out > kMaxDim || n_in > kMaxDim || n_out * n_in > kMaxWeights)
    return fail(QLORA_EINVAL,
                "need n_out >= 1, n_in a positive multiple of 64, each at most 2^22 and at most 2^34 weights "
                "(got %lld x %lld)", (long long)n_out, (long long)n_in);
  const int64_t n = n_out * n_in, nblk = n / 64;
  *codes_bytes = (size_t)(n / 2);
  *absmax_q_bytes = (size_t)nblk;
  *absmax_step_bytes = (size_t)(4 * ceil_div(nblk, 256));
  return QLORA_OK;
}

int qlora_nf4_codebook(float levels[16]) {
  if (!levels) return fail(QLORA_EINVAL, "levels is NULL");
  memcpy(levels, codebook().lv.v, sizeof(float) * 16);
  return QLORA_OK;
}

int qlora_workspace_bytes(int op, int64_t T, int64_t n_out, int64_t n_in, int32_t r, size_t *bytes) {
  if (!bytes) return fail(QLORA_EINVAL, "bytes is NULL");
  if (op != QLORA_OP_FWD && op != QLORA_OP_BWD && op != QLORA_OP_FWD_DROPOUT && op != QLORA_OP_FWD_MULTI)
    return fail(QLORA_EINVAL, "unknown op %d", op);
  if (T < 0 || T > kMaxDim || n_out < 8 || n_out % 8 != 0 || n_out > kMaxDim || n_in < 64 || n_in % 64 != 0 ||
      n_in > kMaxDim || r < 1 || r > QLORA_MAX_RANK)
    return fail(QLORA_EINVAL, "bad sizes T=%lld n_out=%lld n_in=%lld r=%d", (long long)T, (long long)n_out,
                (long long)n_in, (int)r);
  if (int rc = check_acts(T, n_out, n_in)) return rc;
  *bytes = make_plan(op, T, n_out, n_in, r).total;
  return QLORA_OK;
}

int qlora_quantize_nf4(const float *W, const qlora_nf4 *q, void *stream) {
  int rc = check_nf4(q, false);
  if (rc) return rc;
  if (!W || !aligned16(W)) return fail(QLORA_EINVAL, "W must be non-NULL and 16-byte aligned");
  if ((rc = check_device(nullptr))) return rc;
  hipStream_t s = (hipStream_t)stream;
  LAUNCH("quantize_nf4",
         launch_quantize_nf4(W, q->n_out, q->n_in, q->codes, q->absmax_q, q->absmax_step, codebook().thr, s));
  return QLORA_OK;
}

int qlora_dequant(const qlora_nf4 *q, qlora_bf16 *W_out, void *stream) {
  int rc = check_nf4(q, false);
  if (rc) return rc;
  if (!W_out || !aligned16(W_out)) return fail(QLORA_EINVAL, "W_out must be non-NULL and 16-byte aligned");
  if ((rc = check_device(nullptr))) return rc;
  hipStream_t s = (hipStream_t)stream;
  LAUNCH("dequant", launch_dequant(q->codes, q->absmax_q, q->absmax_step, q->n_out, q->n_in, W_out, codebook().lv, s));
  return QLORA_OK;
}

}  // extern "C"

namespace {

// Forward, without dropout (drop == NULL) or with it.
int linear_fwd(const qlora_bf16 *X, int64_t T, const qlora_nf4 *q, const qlora_bf16 *A, const qlora_bf16 *B,
               int32_t r, float alpha, const DropParams *drop, qlora_bf16 *Y, qlora_bf16 *U_out, void *ws,
               size_t ws_bytes, void *stream) {
  int rc = check_lora_args(T, q, A, B, r, alpha);
  if (rc) return rc;
  if (T > 0 && (!X || !Y)) return fail(QLORA_EINVAL, "X and Y must not be NULL");
  if ((X && !aligned16(X)) || (Y && !aligned16(Y)) || (U_out && !aligned16(U_out)))
    return fail(QLORA_EINVAL, "X, Y and U_out must be 16-byte aligned");
  const int64_t N = q->n_out, K = q->n_in;
  Plan p;
  if ((rc = check_ws(drop ? QLORA_OP_FWD_DROPOUT : QLORA_OP_FWD, T, N, K, r, ws, ws_bytes, &p))) return rc;
  if ((rc = check_device(nullptr))) return rc;
  if (T == 0) return QLORA_OK;
  hipStream_t s = (hipStream_t)stream;
  char *w = (char *)ws;
  bf16_t *Bp = (bf16_t *)(w + p.off_bp);
  bf16_t *V = (bf16_t *)(w + p.off_v);
  float *part = (float *)(w + p.off_part);
  const float sc = alpha / (float)r;
  const Levels &lv = codebook().lv;
  if (p.gemv_rows) {  // one or two tokens: bound by the weight stream, one wave per weight row
    float *upart = (float *)(w + p.off_part + p.off_upart);
    int nseg = 1;
    LAUNCH("nf4_gemv", launch_nf4_gemv_rows(X, T, K, q->codes, q->absmax_q, q->absmax_step, N, p.gemv_split, A, r,
                                            part, upart, lv, s, &nseg));
    LAUNCH("gemv_finish", launch_gemv_finish(part, upart, nseg, T, N, B, r, sc, Y, U_out, s, p.gemv_split));
    return QLORA_OK;
  }
  if (p.gemv_mrows) {  // 3..64 tokens: bound by the weight stream, 16 rows per wave, activations in registers
    float *upart = (float *)(w + p.off_part + p.off_upart);
    int nseg = 1;
    LAUNCH("nf4_gemv", launch_nf4_gemv_mrows(X, T, K, q->codes, q->absmax_q, q->absmax_step, N, p.gemv_split, A, r,
                                             part, upart, lv, s, &nseg));
    LAUNCH("gemv_finish", launch_gemv_finish(part, upart, nseg, T, N, B, r, sc, Y, U_out, s, p.gemv_split));
    return QLORA_OK;
  }
  if (p.gemv) {  // few tokens: bound by the weight stream
    float *upart = (float *)(w + p.off_part + p.off_upart);
    LAUNCH("nf4_gemv", launch_nf4_gemv(X, T, K, q->codes, q->absmax_q, q->absmax_step, N, p.gemv_rg, p.gemv_w,
                                       p.gemv_split, p.gemv_main, A, r, part, upart, lv, s));
    LAUNCH("gemv_finish", launch_gemv_finish(part, upart, p.gemv_split, T, N, B, r, sc, Y, U_out, s));
    return QLORA_OK;
  }
  if (drop) {  // U = Xd A^T, drawing the keep bits of X on the way
    LAUNCH("lora_u_dropout", launch_skinny(false, false, p.rn, X, K, T, A, K, r, K, p.su.kchunk, p.su.n, part, s,
                                           DROP_GENERATE, *drop));
  } else if (lora_rows_ok(p.rn, T)) {  // many rows, narrow rank: the whole reduction per workgroup
    LAUNCH("lora_u", launch_lora_rows(false, p.rn, X, K, T, A, K, r, K, U_out, r, U_out ? r : 0, 1.0f, V, p.rp, p.rp,
                                      r, sc, s));
  } else {
    LAUNCH("lora_u", launch_skinny(false, false, p.rn, X, K, T, A, K, r, K, p.su.kchunk, p.su.n, part, s));
  }
  if (drop || !lora_rows_ok(p.rn, T))
    LAUNCH("lora_u_finalize",
           launch_finalize(part, p.su.n, T, p.rn, U_out, r, U_out ? r : 0, 1.0f, V, p.rp, p.rp, r, sc, s));
  // B is read in place when its rows are 16-byte multiples, else from a zero-padded copy
  const bool b_direct = (r % 8) == 0;
  if (!b_direct) LAUNCH("pad_b", launch_pad_copy(B, r, r, N, Bp, p.rp, s));
  LAUNCH("nf4_gemm_fwd", launch_nf4_gemm_fwd(nf4_gemm_pick_tile_fwd(T, N, K), X, T, K, q->codes, q->absmax_q,
                                             q->absmax_step, N, V, b_direct ? B : Bp, b_direct ? r : p.rp, r, p.rp,
                                             Y, lv, s, SegTable(), p.fwd_split, part));
  if (p.fwd_split > 1)  // few output tiles: the reduction ran in ranges; add them in order
    LAUNCH("gemm_fwd_reduce", launch_finalize(part, p.fwd_split, T, N, Y, N, N, 1.0f, nullptr, 0, 0, 0, 0.f, s));
  return QLORA_OK;
}

// Backward, without dropout (drop == NULL) or with the keep bits in drop->mask.
int linear_bwd(const qlora_bf16 *X, const qlora_bf16 *dY, int64_t T, const qlora_nf4 *q, const qlora_bf16 *A,
               const qlora_bf16 *B, int32_t r, float alpha, const DropParams *drop, const qlora_bf16 *U,
               qlora_bf16 *dX, qlora_bf16 *dA, qlora_bf16 *dB, void *ws, size_t ws_bytes, void *stream) {
  int rc = check_lora_args(T, q, A, B, r, alpha);
  if (rc) return rc;
  if (!dA || !dB) return fail(QLORA_EINVAL, "dA and dB must not be NULL");
  if (T > 0 && (!X || !dY)) return fail(QLORA_EINVAL, "X and dY must not be NULL");
  if ((X && !aligned16(X)) || (dY && !aligned16(dY)) || (U && !aligned16(U)) || (dX && !aligned16(dX)) ||
      !aligned16(dA) || !aligned16(dB))
    return fail(QLORA_EINVAL, "X, dY, U, dX, dA and dB must be 16-byte aligned");
  const int64_t N = q->n_out, K = q->n_in;
  Plan p;
  if ((rc = check_ws(QLORA_OP_BWD, T, N, K, r, ws, ws_bytes, &p))) return rc;
  if ((rc = check_device(nullptr))) return rc;
  hipStream_t s = (hipStream_t)stream;
  char *w = (char *)ws;
  bf16_t *Bp = (bf16_t *)(w + p.off_bp);
  bf16_t *Up = (bf16_t *)(w + p.off_v);
  bf16_t *dUp = (bf16_t *)(w + p.off_du);
  float *part = (float *)(w + p.off_part);
  const float sc = alpha / (float)r;
  const Levels &lv = codebook().lv;
  if (T == 0) {  // empty batch: the gradients of A and B are sums over no tokens
    LAUNCH("zero_da", launch_finalize(part, 0, r, K, dA, K, K, 1.0f, nullptr, 0, 0, 0, 0.f, s));
    LAUNCH("zero_db", launch_finalize(part, 0, N, r, dB, r, r, 1.0f, nullptr, 0, 0, 0, 0.f, s));
    return QLORA_OK;
  }
  // B and U are read in place when their rows are 16-byte multiples, else from zero-padded copies
  const bool direct = (r % 8) == 0;
  // (the copies are zero past column r, so r rounded up to 8 columns of them are read)
  const bf16_t *Bsrc = B, *Usrc = U;
  int64_t ldb = r, ldu = r, rvb = r, rvu = r;
  if (!direct) {
    LAUNCH("pad_b", launch_pad_copy(B, r, r, N, Bp, p.rp, s));
    Bsrc = Bp;
    ldb = p.rp;
    rvb = p.rv;
  }
  if (U && !direct) {
    LAUNCH("pad_u", launch_pad_copy(U, r, r, T, Up, p.rp, s));
    Usrc = Up;
    ldu = p.rp;
    rvu = p.rv;
  } else if (!U) {
    if (drop) {
      LAUNCH("lora_u_dropout", launch_skinny(false, false, p.rn, X, K, T, A, K, r, K, p.su.kchunk, p.su.n, part, s,
                                             DROP_APPLY, *drop));
    } else if (lora_rows_ok(p.rn, T)) {
      LAUNCH("lora_u", launch_lora_rows(false, p.rn, X, K, T, A, K, r, K, nullptr, 0, 0, 0.f, Up, p.rp, p.rp, r, 1.0f,
                                        s));
    } else {
      LAUNCH("lora_u", launch_skinny(false, false, p.rn, X, K, T, A, K, r, K, p.su.kchunk, p.su.n, part, s));
    }
    if (drop || !lora_rows_ok(p.rn, T))
      LAUNCH("lora_u_finalize",
             launch_finalize(part, p.su.n, T, p.rn, nullptr, 0, 0, 0.f, Up, p.rp, p.rp, r, 1.0f, s));
    Usrc = Up;
    ldu = p.rp;
    rvu = p.rv;
  }
  // dU = s dY B  -> dUp [T, rp]
  if (lora_rows_ok(p.rn, T)) {
    LAUNCH("lora_du", launch_lora_rows(true, p.rn, dY, N, T, Bsrc, ldb, rvb, N, nullptr, 0, 0, 0.f, dUp, p.rp, p.rp, r,
                                       sc, s));
  } else {
    LAUNCH("lora_du", launch_skinny(false, true, p.rn, dY, N, T, Bsrc, ldb, rvb, N, p.sdu.kchunk, p.sdu.n, part, s));
    LAUNCH("lora_du_finalize",
           launch_finalize(part, p.sdu.n, T, p.rn, nullptr, 0, 0, 0.f, dUp, p.rp, p.rp, r, sc, s));
  }
  // dB = s dY^T U  -> [N, r]
  LAUNCH("lora_db", launch_skinny(true, true, p.rn, dY, N, N, Usrc, ldu, rvu, T, p.sdb.kchunk, p.sdb.n, part, s));
  // dA^T = X^T dU  -> [K, r], its partial sums stored by rank as [split][rn][K]
  float *part2 = (float *)(w + p.off_part2);
  if (drop)  // dA^T = Xd^T dU
    LAUNCH("lora_da_dropout", launch_skinny(true, true, p.rn, X, K, K, dUp, p.rp, p.rv, T, p.sda.kchunk, p.sda.n,
                                            part2, s, DROP_APPLY, *drop, true));
  else
    LAUNCH("lora_da", launch_skinny(true, true, p.rn, X, K, K, dUp, p.rp, p.rv, T, p.sda.kchunk, p.sda.n, part2, s,
                                    DROP_NONE, DropParams(), true));
  // dB = s (sum of dB's partials) [N, r], dA = (sum of dA's partials) [r, K] (rows r of rn), one launch
  LAUNCH("lora_dadb_finalize", launch_finalize_pair(part, p.sdb.n, N, p.rn, dB, r, r, sc, part2, p.sda.n, r, K,
                                                    (int64_t)p.rn * K, dA, K, K, 1.0f, s));
  // dX = dY W' + dU A   (with dropout: + (keep q) o (dU A))
  if (dX)
    LAUNCH("nf4_gemm_dx",
           launch_nf4_gemm_dx(nf4_gemm_pick_tile(T, K), dY, T, N, q->codes, q->absmax_q, q->absmax_step, K, dUp, A,
                              r, p.rp, dX, lv, s, drop ? drop->mask : nullptr, drop ? drop->q : 1.f));
  return QLORA_OK;
}

}  // namespace

extern "C" {

int qlora_linear_fwd(const qlora_bf16 *X, int64_t T, const qlora_nf4 *q, const qlora_bf16 *A, const qlora_bf16 *B,
                     int32_t r, float alpha, qlora_bf16 *Y, qlora_bf16 *U_out, void *ws, size_t ws_bytes,
                     void *stream) {
  return linear_fwd(X, T, q, A, B, r, alpha, nullptr, Y, U_out, ws, ws_bytes, stream);
}

int qlora_linear_fwd_noalloc(const qlora_bf16 *X, int64_t T, const qlora_nf4 *q, const qlora_bf16 *A,
                             const qlora_bf16 *B, int32_t r, float alpha, qlora_bf16 *Y, qlora_bf16 *U_out,
                             void *stream) {
  int rc = check_lora_args(T, q, A, B, r, alpha);
  if (rc) return rc;
  const size_t need = make_plan(QLORA_OP_FWD, T, q->n_out, q->n_in, r).total;
  if (need > kScratchBytes)
    return fail(QLORA_EWORKSPACE, "this forward needs %zu workspace bytes; the static workspace holds %zu", need,
                kScratchBytes);
  int dev = 0;
  if ((rc = check_device(&dev))) return rc;
  void *ws = nullptr;
  if ((rc = scratch_address(dev, &ws))) return rc;
  return linear_fwd(X, T, q, A, B, r, alpha, nullptr, Y, U_out, ws, kScratchBytes, stream);
}

int qlora_linear_bwd(const qlora_bf16 *X, const qlora_bf16 *dY, int64_t T, const qlora_nf4 *q, const qlora_bf16 *A,
                     const qlora_bf16 *B, int32_t r, float alpha, const qlora_bf16 *U, qlora_bf16 *dX,
                     qlora_bf16 *dA, qlora_bf16 *dB, void *ws, size_t ws_bytes, void *stream) {
  return linear_bwd(X, dY, T, q, A, B, r, alpha, nullptr, U, dX, dA, dB, ws, ws_bytes, stream);
}

int qlora_linear_fwd_multi(const qlora_bf16 *X, int64_t T, const qlora_nf4 *q, const qlora_bf16 *A_pool,
                           const qlora_bf16 *B_pool, int32_t n_pool, int32_t r, float alpha, const int32_t *seg_offsets,
                           const int32_t *seg_adapter, int32_t n_seg, qlora_bf16 *Y, void *ws, size_t ws_bytes,
                           void *stream) {
  int rc = check_lora_args(T, q, A_pool, B_pool, r, alpha);
  if (rc) return rc;
  if (r % 8 != 0) return fail(QLORA_EINVAL, "r must be a multiple of 8 for adapter pools (got %d)", (int)r);
  if (n_pool < 1) return fail(QLORA_EINVAL, "n_pool must be >= 1 (got %d)", (int)n_pool);
  if (n_seg < 1 || n_seg > (1 << 24)) return fail(QLORA_EINVAL, "n_seg must be in [1, 2^24] (got %d)", (int)n_seg);
  if (!seg_offsets || !seg_adapter || ((uintptr_t)seg_offsets & 3) || ((uintptr_t)seg_adapter & 3))
    return fail(QLORA_EINVAL, "segment arrays must be non-NULL and 4-byte aligned");
  if (T > 0 && (!X || !Y)) return fail(QLORA_EINVAL, "X and Y must not be NULL");
  if ((X && !aligned16(X)) || (Y && !aligned16(Y))) return fail(QLORA_EINVAL, "X and Y must be 16-byte aligned");
  const int64_t N = q->n_out, K = q->n_in;
  Plan p;
  if ((rc = check_ws(QLORA_OP_FWD_MULTI, T, N, K, r, ws, ws_bytes, &p))) return rc;
  if ((rc = check_device(nullptr))) return rc;
  if (T == 0) return QLORA_OK;
  hipStream_t s = (hipStream_t)stream;
  char *w = (char *)ws;
  bf16_t *V = (bf16_t *)(w + p.off_v);
  float *part = (float *)(w + p.off_part);
  const float sc = alpha / (float)r;
  const Levels &lv = codebook().lv;
  SegTable sg;
  sg.seg = seg_offsets;
  sg.ad = seg_adapter;
  sg.n_seg = n_seg;
  sg.n_pool = n_pool;
  if (p.gemv) {  // few tokens: the U partials of every segment ride along in the weight-streaming launch
    float *upart = (float *)(w + p.off_part + p.off_upart);
    LAUNCH("nf4_gemv", launch_nf4_gemv(X, T, K, q->codes, q->absmax_q, q->absmax_step, N, p.gemv_rg, p.gemv_w,
                                       p.gemv_split, p.gemv_main, A_pool, r, part, upart, lv, s, sg));
    LAUNCH("gemv_finish", launch_gemv_finish_multi(part, upart, p.gemv_split, T, N, B_pool, r, sc, sg, Y, s));
    return QLORA_OK;
  }
  // U = X A_a^T per segment, then V = bf16(s U), zero-padded to rp columns
  int gns;
  int64_t gkc;
  skinny_plan_grouped(T, n_seg, K, &gns, &gkc);  // at most p.su.n ranges: fits the workspace
  LAUNCH("lora_u_multi", launch_skinny_grouped(p.rn, X, K, T, A_pool, K, (int64_t)r * K, r, K, gkc, gns, sg, part, s));
  LAUNCH("lora_u_finalize", launch_finalize(part, gns, T, p.rn, nullptr, 0, 0, 1.0f, V, p.rp, p.rp, r, sc, s));
  LAUNCH("nf4_gemm_fwd", launch_nf4_gemm_fwd(nf4_gemm_pick_tile_fwd(T, N, K), X, T, K, q->codes, q->absmax_q,
                                             q->absmax_step, N, V, B_pool, r, r, p.rp, Y, lv, s, sg, p.fwd_split, part));
  if (p.fwd_split > 1)
    LAUNCH("gemm_fwd_reduce", launch_finalize(part, p.fwd_split, T, N, Y, N, N, 1.0f, nullptr, 0, 0, 0, 0.f, s));
  return QLORA_OK;
}

int qlora_linear_fwd_dropout(const qlora_bf16 *X, int64_t T, const qlora_nf4 *q, const qlora_bf16 *A,
                             const qlora_bf16 *B, int32_t r, float alpha, float p, uint64_t seed, uint64_t offset,
                             uint8_t *mask_out, qlora_bf16 *Y, qlora_bf16 *U_out, void *ws, size_t ws_bytes,
                             void *stream) {
  int rc = check_dropout(p, mask_out, T);
  if (rc) return rc;
  const DropParams d = drop_params(p, mask_out, seed, offset);
  return linear_fwd(X, T, q, A, B, r, alpha, &d, Y, U_out, ws, ws_bytes, stream);
}

int qlora_linear_bwd_dropout(const qlora_bf16 *X, const qlora_bf16 *dY, int64_t T, const qlora_nf4 *q,
                             const qlora_bf16 *A, const qlora_bf16 *B, int32_t r, float alpha, float p,
                             const uint8_t *mask, const qlora_bf16 *U, qlora_bf16 *dX, qlora_bf16 *dA,
                             qlora_bf16 *dB, void *ws, size_t ws_bytes, void *stream) {
  int rc = check_dropout(p, mask, T);
  if (rc) return rc;
  const DropParams d = drop_params(p, const_cast<uint8_t *>(mask), 0, 0);  // read only on this path
  return linear_bwd(X, dY, T, q, A, B, r, alpha, &d, U, dX, dA, dB, ws, ws_bytes, stream);
}

int qlora_merge(const qlora_nf4 *q, const qlora_bf16 *W_base, int64_t n_out, int64_t n_in, const qlora_bf16 *A,
                const qlora_bf16 *B, int32_t r, float alpha, qlora_bf16 *W_out, float *W_out_f32, void *stream) {
  if ((q == nullptr) == (W_base == nullptr)) return fail(QLORA_EINVAL, "give exactly one of q and W_base");
  int rc;
  if (q) {
    if ((rc = check_nf4(q, false))) return rc;
    if (q->n_out != n_out || q->n_in != n_in)
      return fail(QLORA_EINVAL, "q is %lld x %lld, the merge asks for %lld x %lld", (long long)q->n_out,
                  (long long)q->n_in, (long long)n_out, (long long)n_in);
  } else if (!aligned16(W_base)) {
    return fail(QLORA_EINVAL, "W_base must be 16-byte aligned");
  }
  if (n_out < 1 || n_in < 64 || n_in % 64 != 0 || n_out > kMaxDim || n_in > kMaxDim || n_out * n_in > kMaxWeights)
    return fail(QLORA_EINVAL, "need n_out >= 1 and n_in a positive multiple of 64 (got %lld x %lld)",
                (long long)n_out, (long long)n_in);
  if (r < 1 || r > QLORA_MAX_RANK) return fail(QLORA_EINVAL, "r must be in [1, %d] (got %d)", QLORA_MAX_RANK, (int)r);
  if (!isfinite(alpha)) return fail(QLORA_EINVAL, "alpha must be finite");
  if (!A || !B || !aligned16(A) || !aligned16(B)) return fail(QLORA_EINVAL, "A and B must be non-NULL and 16-byte aligned");
  if (!W_out && !W_out_f32) return fail(QLORA_EINVAL, "give W_out, W_out_f32 or both");
  if ((W_out && !aligned16(W_out)) || (W_out_f32 && !aligned16(W_out_f32)))
    return fail(QLORA_EINVAL, "outputs must be 16-byte aligned");
  if ((rc = check_device(nullptr))) return rc;
  hipStream_t s = (hipStream_t)stream;
  LAUNCH("merge", launch_merge(q ? q->codes : nullptr, q ? q->absmax_q : nullptr, q ? q->absmax_step : nullptr,
                               W_base, n_out, n_in, A, B, r, alpha / (float)r, W_out, W_out_f32, codebook().lv, s));
  return QLORA_OK;
}

int qlora_adamw_step(const qlora_adamw_tensor *tensors, int32_t count, double lr, double beta1, double beta2,
                     double eps, double weight_decay, int64_t step, void *stream) {
  if (count < 0 || (count > 0 && !tensors)) return fail(QLORA_EINVAL, "tensors is NULL or count < 0");
  if (!(beta1 >= 0.0 && beta1 < 1.0 && beta2 >= 0.0 && beta2 < 1.0))
    return fail(QLORA_EINVAL, "betas must be in [0, 1) (got %g, %g)", beta1, beta2);
  if (!(eps > 0.0) || !isfinite(eps)) return fail(QLORA_EINVAL, "eps must be positive and finite");
  if (!(lr >= 0.0) || !isfinite(lr) || !(weight_decay >= 0.0) || !isfinite(weight_decay))
    return fail(QLORA_EINVAL, "lr and weight_decay must be finite and >= 0");
  if (step < 1) return fail(QLORA_EINVAL, "step must be >= 1 (got %lld)", (long long)step);
  for (int32_t i = 0; i < count; ++i) {
    const qlora_adamw_tensor &t = tensors[i];
    if (t.n < 0) return fail(QLORA_EINVAL, "tensor %d: n < 0", (int)i);
    if (t.n == 0) continue;
    if (!t.param || !t.grad || !t.exp_avg || !t.exp_avg_sq)
      return fail(QLORA_EINVAL, "tensor %d: NULL array", (int)i);
    if (!aligned16(t.param) || !aligned16(t.grad) || !aligned16(t.exp_avg) || !aligned16(t.exp_avg_sq) ||
        (t.master && !aligned16(t.master)))
      return fail(QLORA_EINVAL, "tensor %d: arrays must be 16-byte aligned", (int)i);
  }
  int64_t total = 0;
  for (int32_t i = 0; i < count; ++i) total += tensors[i].n;
  if (total == 0) return QLORA_OK;  // nothing to update: no HIP call
  int rc;
  if ((rc = check_device(nullptr))) return rc;
  hipStream_t s = (hipStream_t)stream;
  AdamParams a;
  a.b1 = (float)beta1;
  a.omb1 = (float)(1.0 - beta1);
  a.b2 = (float)beta2;
  a.omb2 = (float)(1.0 - beta2);
  a.eps = (float)eps;
  a.decay = (float)(1.0 - lr * weight_decay);
  a.step_size = (float)(lr / (1.0 - pow(beta1, (double)step)));
  a.sqrt_bc2 = (float)sqrt(1.0 - pow(beta2, (double)step));
  a.rbc2 = (float)(1.0 / (double)a.sqrt_bc2);  // correctly rounded: binary64 has more than 2 * 24 + 2 bits
  a.fast_bc2 = a.sqrt_bc2 >= kRecipDivMinB && a.sqrt_bc2 <= kRecipDivMaxB;
  for (int32_t first = 0; first < count; first += kAdamMaxTensors) {
    const int32_t cnt = (count - first < kAdamMaxTensors) ? count - first : kAdamMaxTensors;
    int64_t blocks = 0;
    for (int32_t i = 0; i < kAdamMaxTensors; ++i) {
      AdamTensor &d = a.t[i];
      if (i < cnt) {
        const qlora_adamw_tensor &t = tensors[first + i];
        d = AdamTensor{t.param, t.grad, t.exp_avg, t.exp_avg_sq, t.master, t.n, blocks};
        blocks += (t.n + kAdamChunk - 1) / kAdamChunk;
      } else {
        d = AdamTensor{nullptr, nullptr, nullptr, nullptr, nullptr, 0, INT64_MAX};
      }
    }
    a.count = cnt;
    LAUNCH("adamw", launch_adamw(a, blocks, s));
  }
  return QLORA_OK;
}

int qlora_adamw8_step(const qlora_adamw8_tensor *tensors, int32_t count, double lr, double beta1, double beta2,
                      double eps, double weight_decay, int64_t step, void *stream) {
  if (count < 0 || (count > 0 && !tensors)) return fail(QLORA_EINVAL, "tensors is NULL or count < 0");
  if (!(beta1 >= 0.0 && beta1 < 1.0 && beta2 >= 0.0 && beta2 < 1.0))
    return fail(QLORA_EINVAL, "betas must be in [0, 1) (got %g, %g)", beta1, beta2);
  if (!(eps > 0.0) || !isfinite(eps)) return fail(QLORA_EINVAL, "eps must be positive and finite");
  if (!(lr >= 0.0) || !isfinite(lr) || !(weight_decay >= 0.0) || !isfinite(weight_decay))
    return fail(QLORA_EINVAL, "lr and weight_decay must be finite and >= 0");
  if (step < 1) return fail(QLORA_EINVAL, "step must be >= 1 (got %lld)", (long long)step);
  int64_t total = 0;
  for (int32_t i = 0; i < count; ++i) {
    const qlora_adamw8_tensor &t = tensors[i];
    if (t.n < 0) return fail(QLORA_EINVAL, "tensor %d: n < 0", (int)i);
    if (t.n == 0) continue;
    if (!t.param || !t.grad || !t.exp_avg_code || !t.exp_avg_absmax || !t.exp_avg_sq_code || !t.exp_avg_sq_absmax)
      return fail(QLORA_EINVAL, "tensor %d: NULL array", (int)i);
    if (!aligned16(t.param) || !aligned16(t.grad) || !aligned16(t.exp_avg_code) || !aligned16(t.exp_avg_sq_code) ||
        ((uintptr_t)t.exp_avg_absmax & 3) || ((uintptr_t)t.exp_avg_sq_absmax & 3) || (t.master && !aligned16(t.master)))
      return fail(QLORA_EINVAL, "tensor %d: misaligned array", (int)i);
    total += t.n;
  }
  if (total == 0) return QLORA_OK;
  int rc;
  if ((rc = check_device(nullptr))) return rc;
  hipStream_t s = (hipStream_t)stream;
  Adam8Params a;
  a.b1 = (float)beta1;
  a.omb1 = (float)(1.0 - beta1);
  a.b2 = (float)beta2;
  a.omb2 = (float)(1.0 - beta2);
  a.eps = (float)eps;
  a.decay = (float)(1.0 - lr * weight_decay);
  a.step_size = (float)(lr / (1.0 - pow(beta1, (double)step)));
  a.sqrt_bc2 = (float)sqrt(1.0 - pow(beta2, (double)step));
  a.rbc2 = (float)(1.0 / (double)a.sqrt_bc2);  // correctly rounded: binary64 has more than 2 * 24 + 2 bits
  a.fast_bc2 = a.sqrt_bc2 >= kRecipDivMinB && a.sqrt_bc2 <= kRecipDivMaxB;
  for (int32_t first = 0; first < count; first += kAdamMaxTensors) {
    const int32_t cnt = (count - first < kAdamMaxTensors) ? count - first : kAdamMaxTensors;
    int64_t blocks = 0;
    for (int32_t i = 0; i < kAdamMaxTensors; ++i) {
      Adam8Tensor &d = a.t[i];
      if (i < cnt) {
        const qlora_adamw8_tensor &t = tensors[first + i];
        d = Adam8Tensor{t.param, t.grad, t.exp_avg_code, t.exp_avg_absmax, t.exp_avg_sq_code, t.exp_avg_sq_absmax,
                        t.master, t.n, blocks};
        blocks += (t.n + kAdam8Block - 1) / kAdam8Block;
      } else {
        d = Adam8Tensor{nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, INT64_MAX};
      }
    }
    a.count = cnt;
    LAUNCH("adamw8", launch_adamw8(a, blocks, s));
  }
  return QLORA_OK;
}

int qlora_timing_enable(const char *kernel, int enable) {
  if (!kernel) return fail(QLORA_EINVAL, "kernel name is NULL");
  std::lock_guard<std::mutex> lk(g_tmu);
  if (!strcmp(kernel, "*") && !enable) {
    g_timed.clear();
    g_ntimed.store(0, std::memory_order_release);
    return QLORA_OK;
  }
  for (auto it = g_timed.begin(); it != g_timed.end(); ++it)
    if (*it == kernel) {
      g_timed.erase(it);
      break;
    }
  if (enable) g_timed.push_back(kernel);
  g_ntimed.store((int)g_timed.size(), std::memory_order_release);
  return QLORA_OK;
}

// Waits for and releases the recorded events of `kernel`; per-launch milliseconds in launch order go
// to ms[0 .. cap) (ms may be NULL when cap is 0), their sum to *total_ms.
static int timing_collect(const char *kernel, double *ms_each, int64_t cap, int64_t *launches, double *total_ms) {
  std::vector<EventPair> ev;
  {
    std::lock_guard<std::mutex> lk(g_tmu);
    auto it = g_events.find(kernel);
    if (it != g_events.end()) {
      ev.swap(it->second);
      g_events.erase(it);
    }
  }
  double tot = 0.0;
  int rc = QLORA_OK;
  for (size_t i = 0; i < ev.size(); ++i) {
    float ms = 0.f;
    if (hipEventSynchronize(ev[i].b) != hipSuccess || hipEventElapsedTime(&ms, ev[i].a, ev[i].b) != hipSuccess) {
      (void)hipGetLastError();
      rc = fail(QLORA_EHIP, "reading timing events failed");
    }
    tot += ms;
    if ((int64_t)i < cap) ms_each[i] = ms;
  }
  {
    std::lock_guard<std::mutex> lk(g_tmu);
    for (const EventPair &e : ev) {
      g_event_pool[e.dev].push_back(e.a);
      g_event_pool[e.dev].push_back(e.b);
    }
  }
  *launches = (int64_t)ev.size();
  if (total_ms) *total_ms = tot;
  return rc;
}

int qlora_timing_read(const char *kernel, int64_t *launches, double *total_ms) {
  if (!kernel || !launches || !total_ms) return fail(QLORA_EINVAL, "NULL argument");
  return timing_collect(kernel, nullptr, 0, launches, total_ms);
}

int qlora_timing_read_each(const char *kernel, double *ms, int64_t cap, int64_t *launches) {
  if (!kernel || !launches || (cap > 0 && !ms) || cap < 0) return fail(QLORA_EINVAL, "NULL argument or cap < 0");
  return timing_collect(kernel, ms, cap, launches, nullptr);
}

}  // extern "C"
