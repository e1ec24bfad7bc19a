// extern "C" entry points: argument validation, workspace layout and launch
// order. Everything is validated before the first launch, so an error
// return means nothing was enqueued. The host never synchronises.
#include <mutex>

#include "moe_mxfp4.h"
#include "moe_internal.h"

// Scratch of moe_layer_forward_noalloc: device memory the library holds on
// each GPU it runs on, from the module's load until the process ends. In
// host code `scratch` names a host-side stand-in, not a device address:
// only the per-device address from hipGetSymbolAddress (noalloc_scratch
// below) is ever passed to a kernel.
constexpr size_t kNoallocScratchBytes = 16u << 20;
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {

using namespace moe;

constexpr int kMaxE = 1024;
constexpr int kMaxK = 64;
constexpr int kMaxH = 8192;
constexpr int kMaxI = 4096;
constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) & ~(kAlign - 1); }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shape checks shared by the calls. INVALID_ARG for malformed values,
// UNSUPPORTED for well-formed values outside the compiled limits.
int check_dims(int T, int H, int E, int k, int I) {
  if (T < 0 || H <= 0 || E <= 0 || k <= 0 || I <= 0) return MOE_ERR_INVALID_ARG;
  if (H % 32 || I % 32 || k > E) return MOE_ERR_INVALID_ARG;
  if (E > kMaxE || k > kMaxK || H > kMaxH || I > kMaxI) return MOE_ERR_UNSUPPORTED;
  if ((long long)T * k >= (1ll << 31) || (long long)T * H >= (1ll << 40)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

int check_bank(const moe_mxfp4_bank* b) {
  if (!b || !b->gate_up_codes || !b->gate_up_scales || !b->down_codes || !b->down_scales)
    return MOE_ERR_INVALID_ARG;
  if (!aligned16(b->gate_up_codes) || !aligned16(b->down_codes)) return MOE_ERR_INVALID_ARG;
  if (b->E <= 0 || b->H <= 0 || b->I <= 0 || b->H % 32 || b->I % 32) return MOE_ERR_INVALID_ARG;
  if (b->E > kMaxE || b->H > kMaxH || b->I > kMaxI) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

BankView view(const moe_mxfp4_bank* b) {
  return BankView{b->gate_up_codes, b->gate_up_scales, b->down_codes, b->down_scales, b->E};
}

int launch_status() {
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int check_nv_bank(const moe_nvfp4_bank* b) {
  if (!b || !b->gate_up_codes || !b->gate_up_scales || !b->down_codes || !b->down_scales)
    return MOE_ERR_INVALID_ARG;
  if (!aligned16(b->gate_up_codes) || !aligned16(b->down_codes)) return MOE_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(b->gate_up_scales) | reinterpret_cast<uintptr_t>(b->down_scales)) & 3u)
    return MOE_ERR_INVALID_ARG;
  if (b->E <= 0 || b->H <= 0 || b->I <= 0 || b->H % 32 || b->I % 32) return MOE_ERR_INVALID_ARG;
  if (b->E > kMaxE || b->H > kMaxH || b->I > kMaxI) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

BankView view_nv(const moe_nvfp4_bank* b) {
  return BankView{b->gate_up_codes, b->gate_up_scales, b->down_codes, b->down_scales, b->E,
                  kCodecNvfp4, b->global_scales};
}

int check_fp8_bank(const moe_fp8_bank* b) {
  if (!b || !b->gate_up_w || !b->gate_up_scales || !b->down_w || !b->down_scales)
    return MOE_ERR_INVALID_ARG;
  if (!aligned16(b->gate_up_w) || !aligned16(b->down_w)) return MOE_ERR_INVALID_ARG;
  if (b->E != 1 || b->H <= 0 || b->I <= 0 || b->H % 32 || b->I % 32) return MOE_ERR_INVALID_ARG;
  if (b->H > kMaxH || b->I > kMaxI) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// Scratch of the FP8 expert over T rows: the grouped GEMM's where it tiles
// the shape and T exceeds the few-token kernels, else fp32 h for at most
// kDecodeMaxT rows at a time.
bool fp8_uses_gemm(int T, int H, int I) { return T > kDecodeMaxT && gemm_supported(T, H, I, 0, true); }
size_t fp8_ffn_ws(int T, int H, int I) {
  return fp8_uses_gemm(T, H, I) ? fp8_gemm_ws_bytes(T, H, I)
                                : fp8_gemv_ws_bytes(T < kDecodeMaxT ? T : kDecodeMaxT, I);
}

// Workspace of the few-token layer with an FP8 shared expert: the decode
// path's (no MXFP4 shared expert), then y_sh [T][H], then the FP8 scratch.
// (One token and blocks of 2..8 tokens may instead stream the FP8 expert
// inside the few-token launches, which needs the decode layout with a shared
// expert.)
size_t few_fp8_ws(int T, int H, int I, int E, int k) {
  const size_t sep = align_up(decode_ws_bytes(T, H, I, E, k, T * k, false, false)) +
                     align_up((size_t)T * H * sizeof(float)) + fp8_ffn_ws(T, H, I);
  const size_t fused = decode_ws_bytes(T, H, I, E, k, T * k, false, true);
  return sep > fused ? sep : fused;
}

// The FP8 expert over rows x[0..T) into y[0..T); `scratch` holds fp8_ffn_ws.
void launch_fp8_ffn(const uint16_t* x, const moe_fp8_bank* b, int T, float* y, void* scratch,
                    hipStream_t stream) {
  Fp8Ffn p{};
  p.H = b->H;
  p.I = b->I;
  p.gu_w = b->gate_up_w;
  p.gu_s = b->gate_up_scales;
  p.d_w = b->down_w;
  p.d_s = b->down_scales;
  if (fp8_uses_gemm(T, b->H, b->I)) {
    p.x = x;
    p.T = T;
    p.y = y;
    launch_fp8_gemm(p, scratch, stream);
    return;
  }
  p.h = static_cast<float*>(scratch);
  for (int t0 = 0; t0 < T; t0 += kDecodeMaxT) {
    p.x = x + (size_t)t0 * b->H;
    p.y = y + (size_t)t0 * b->H;
    p.T = T - t0 < kDecodeMaxT ? T - t0 : kDecodeMaxT;
    launch_fp8_ffn_gemv(p, stream);
  }
}

// Bump allocator over the caller's workspace.
struct Carve {
  char* base;
  size_t off = 0;
  explicit Carve(void* p) : base(static_cast<char*>(p)) {}
  template <class T>
  T* take(size_t count) {
    T* p = reinterpret_cast<T*>(base ? base + off : nullptr);
    off += align_up(count * sizeof(T));
    return p;
  }
};

// Workspace of moe_layer_forward; the other calls need a subset of it.
struct LayerWs {
  float* logits;
  int32_t* ids;
  float* w;
  int32_t* offsets;
  int32_t* active;
  int32_t* row_token;
  int32_t* inv_row;
  void* perm;
  void* ffn;  // FFN scratch: the GEMV path's fp32 h and h_sh, or the GEMM's
  float* h;
  float* h_sh;
  float* y;
  float* y_sh;
  size_t bytes;
};

LayerWs layer_ws(void* ws, int T, int H, int I, int E, int k) {
  const size_t R = (size_t)T * k;
  Carve c(ws);
  LayerWs L;
  L.logits = c.take<float>((size_t)T * E * router_split(T, H, E));  // the router's partials
  L.ids = c.take<int32_t>(R);
  L.w = c.take<float>(R);
  L.offsets = c.take<int32_t>((size_t)E + 1);
  L.active = c.take<int32_t>((size_t)E);
  L.row_token = c.take<int32_t>(R);
  L.inv_row = c.take<int32_t>(R);
  L.perm = c.take<char>(permute_ws_bytes(T, k, E));
  const size_t gemv = align_up(R * I * sizeof(float)) + align_up((size_t)T * I * sizeof(float));
  const size_t gemm = gemm_ws_bytes(T, H, I, E, (int)R, true);
  const size_t mx = gemm_mx_ws_bytes(T, H, I, E, (int)R, true);
  size_t big = gemm > mx ? gemm : mx;
  const size_t f8 = fp8_ffn_ws(T, H, I);
  big = big > f8 ? big : f8;
  char* ffn = c.take<char>(gemv > big ? gemv : big);
  L.ffn = ffn;
  L.h = reinterpret_cast<float*>(ffn);
  L.h_sh = reinterpret_cast<float*>(ffn ? ffn + align_up(R * I * sizeof(float)) : nullptr);
  L.y = c.take<float>(R * H);
  L.y_sh = c.take<float>((size_t)T * H);
  L.bytes = c.off;
  return L;
}

// The device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept; MOE_ERR_HIP if the lookup
// fails, MOE_ERR_UNSUPPORTED beyond kMaxDevices devices.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int noalloc_scratch(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

// Launch log of the last entry-point call on this host thread.
constexpr int kMaxLogged = 32;
struct LaunchLog {
  hipEvent_t* events = nullptr;
  int cap = 0;
  int n = 0;
  const char* names[kMaxLogged];
};
thread_local LaunchLog g_log;

void begin_call() { g_log.n = 0; }

}  // namespace

namespace moe {
void next_launch_events(hipEvent_t* start, hipEvent_t* stop) {
  const bool on = g_log.events && g_log.n < g_log.cap;
  *start = on ? g_log.events[2 * g_log.n] : nullptr;
  *stop = on ? g_log.events[2 * g_log.n + 1] : nullptr;
}
void log_launch(const char* name) {
  if (g_log.n < kMaxLogged) g_log.names[g_log.n] = name;
  ++g_log.n;
}
}  // namespace moe

extern "C" {

int moe_set_kernel_events(hipEvent_t* events, int n) {
  if (n < 0 || (n > 0 && !events)) return MOE_ERR_INVALID_ARG;
  g_log.events = n > 0 ? events : nullptr;
  g_log.cap = n;
  return MOE_OK;
}

int moe_last_call_launches(void) { return g_log.n; }

int moe_workspace_status(const void* ws) {
  if (!ws) return MOE_ERR_INVALID_ARG;
  const int code = read_decode_status(ws);
  return code < 0 ? MOE_ERR_HIP : code == 0 ? MOE_OK : MOE_ERR_TIMEOUT;
}

int moe_set_wait_test(int on) {
  set_force_wait_timeout(on != 0);
  return MOE_OK;
}

const char* moe_launch_name(int i) {
  return (i >= 0 && i < g_log.n && i < kMaxLogged) ? g_log.names[i] : nullptr;
}

size_t moe_workspace_bytes(int T, int H, int I, int E, int k) {
  if (T < 0 || H <= 0 || I <= 0 || E <= 0 || k <= 0) return 0;
  const int R = T * k;
  size_t b = layer_ws(nullptr, T, H, I, E, k).bytes;
  const size_t d = decode_ws_bytes(T, H, I, E, k, R, false, true);
  const size_t f = decode_ws_bytes(T, H, I, E, k, R, true, false);
  b = b > d ? b : d;
  b = b > f ? b : f;
  if (T <= kDecodeMaxT) {
    const size_t g = few_fp8_ws(T, H, I, E, k);
    b = b > g ? b : g;
  }
  const size_t e8 = fp8_ffn_ws(T, H, I);
  return b > e8 ? b : e8;
}

const char* moe_status_str(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    case MOE_ERR_TIMEOUT: return "MOE_ERR_TIMEOUT";
    default: return "MOE_ERR_UNKNOWN";
  }
}

int moe_router_topk(const void* x_bf16, const void* w_router_bf16, const float* logit_bias,
                    int T, int H, int E, int k, int32_t* topk_ids, float* topk_w,
                    float* logits_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  begin_call();
  int st = check_dims(T, H, E, k, 32);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!x_bf16 || !w_router_bf16 || !topk_ids || !topk_w) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x_bf16) || !aligned16(w_router_bf16)) return MOE_ERR_INVALID_ARG;
  float* logits = logits_out;
  if (!logits) {
    if (!ws || !aligned16(ws)) return MOE_ERR_INVALID_ARG;
    if (ws_bytes < (size_t)T * E * sizeof(float)) return MOE_ERR_WORKSPACE;
    logits = static_cast<float*>(ws);
  }
  launch_router_logits(static_cast<const uint16_t*>(x_bf16),
                       static_cast<const uint16_t*>(w_router_bf16), logit_bias, T, H, E, logits,
                       stream);
  launch_topk(logits, T, E, k, topk_ids, topk_w, stream);
  return launch_status();
}

int moe_permute(const int32_t* topk_ids, int T, int k, int E, int32_t* expert_offsets,
                int32_t* row_token, int32_t* inv_row, void* ws, size_t ws_bytes,
                hipStream_t stream) {
  begin_call();
  int st = check_dims(T, 32, E, k, 32);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!topk_ids || !expert_offsets || !row_token || !inv_row) return MOE_ERR_INVALID_ARG;
  const size_t need = align_up((size_t)E * sizeof(int32_t)) + permute_ws_bytes(T, k, E);
  if (!ws || !aligned16(ws)) return MOE_ERR_INVALID_ARG;
  if (ws_bytes < need) return MOE_ERR_WORKSPACE;
  Carve c(ws);
  int32_t* active = c.take<int32_t>(E);
  void* perm = c.take<char>(permute_ws_bytes(T, k, E));
  launch_permute(topk_ids, T, k, E, expert_offsets, row_token, inv_row, active, perm, stream);
  return launch_status();
}

int moe_expert_ffn_mxfp4(const void* x_bf16, const moe_mxfp4_bank* bank,
                         const int32_t* expert_offsets, const int32_t* row_token, int T, int R,
                         float* y_rows, void* ws, size_t ws_bytes, hipStream_t stream) {
  begin_call();
  int st = check_bank(bank);
  if (st != MOE_OK) return st;
  st = check_dims(T, bank->H, bank->E, 1, bank->I);
  if (st != MOE_OK) return st;
  if (R < 0) return MOE_ERR_INVALID_ARG;
  if (T == 0 || R == 0) return MOE_OK;
  if (!x_bf16 || !y_rows || !aligned16(x_bf16) || !aligned16(y_rows))
    return MOE_ERR_INVALID_ARG;
  if (!expert_offsets && bank->E != 1) return MOE_ERR_INVALID_ARG;
  if (!row_token && R > T) return MOE_ERR_INVALID_ARG;
  const bool few = R <= kDecodeFfnMaxR;
  const bool mfma = !few && gemm_supported(T, bank->H, bank->I, R, false);
  const int E = expert_offsets ? bank->E : 1;
  const size_t need = few    ? decode_ws_bytes(T, bank->H, bank->I, bank->E, 1, R, true, false)
                      : mfma ? gemm_ws_bytes(T, bank->H, bank->I, E, R, false)
                             : ffn_ws_bytes(T, bank->H, bank->I, R, false);
  if (need && (!ws || !aligned16(ws))) return MOE_ERR_INVALID_ARG;
  if (ws_bytes < need) return MOE_ERR_WORKSPACE;
  if (few) {
    DecodeLaunch d{};
    d.ffn_mode = 1;
    d.x = static_cast<const uint16_t*>(x_bf16);
    d.routed = view(bank);
    d.T = T;
    d.H = bank->H;
    d.I = bank->I;
    d.E = bank->E;
    d.k = 1;
    d.R = R;
    d.offsets = expert_offsets;
    d.row_token = row_token;
    d.y_rows = y_rows;
    launch_decode(d, ws, stream);
    return launch_status();
  }
  FfnProblem p{};
  p.x = static_cast<const uint16_t*>(x_bf16);
  p.T = T;
  p.H = bank->H;
  p.I = bank->I;
  p.routed = view(bank);
  p.offsets = expert_offsets;
  p.active = nullptr;
  p.row_token = row_token;
  p.R = R;
  p.routed_slots = expert_offsets ? (bank->E < R ? bank->E : R) : 1;
  p.h = static_cast<float*>(ws);
  p.y = y_rows;
  p.has_shared = false;
  if (mfma)
    launch_expert_gemm(p, ws, stream);
  else
    launch_expert_ffn(p, stream);
  return launch_status();
}

int moe_combine(const float* y_rows, const int32_t* inv_row, const float* topk_w,
                const float* y_shared, int T, int k, int H, int R, float* out,
                hipStream_t stream) {
  begin_call();
  int st = check_dims(T, H, k, k, 32);
  if (st != MOE_OK) return st;
  if (R < 0) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!inv_row || !topk_w || !out || (R > 0 && !y_rows)) return MOE_ERR_INVALID_ARG;
  if (!aligned16(out) || (y_rows && !aligned16(y_rows)) || (y_shared && !aligned16(y_shared)))
    return MOE_ERR_INVALID_ARG;
  launch_combine(y_rows, inv_row, topk_w, y_shared, T, k, H, R, out, stream);
  return launch_status();
}

int moe_quantize_mxfp8(const void* x_bf16, int T, int H, uint8_t* codes, uint8_t* scales,
                       hipStream_t stream) {
  begin_call();
  if (T < 0 || H <= 0 || H % 32) return MOE_ERR_INVALID_ARG;
  if ((long long)T * H >= (1ll << 40)) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x_bf16 || !codes || !scales || !aligned16(x_bf16) || !aligned16(codes))
    return MOE_ERR_INVALID_ARG;
  launch_quant_mxfp8(static_cast<const uint16_t*>(x_bf16), (long)T * H / 32, codes, scales, stream);
  return launch_status();
}

}  // extern "C"

namespace {

// Both layer entry points: the default mode (exact weights, bf16 / fp32
// activations; few tokens take the persistent kernels) and the MXFP8-
// activation mode (every T on the grouped scaled-MFMA GEMM).
int layer_forward(const void* x_bf16, const void* w_router_bf16, const float* logit_bias,
                  const moe_mxfp4_bank* routed, const moe_mxfp4_bank* shared, int T, int k,
                  float* out, int32_t* topk_ids_out, float* topk_w_out, void* ws,
                  size_t ws_bytes, hipStream_t stream, bool mx_act,
                  const moe_fp8_bank* shared8 = nullptr) {
  begin_call();
  int st = check_bank(routed);
  if (st != MOE_OK) return st;
  const int E = routed->E, H = routed->H, I = routed->I;
  st = check_dims(T, H, E, k, I);
  if (st != MOE_OK) return st;
  if (shared) {
    st = check_bank(shared);
    if (st != MOE_OK) return st;
    if (shared->E != 1 || shared->H != H || shared->I != I) return MOE_ERR_INVALID_ARG;
  }
  if (shared8) {
    st = check_fp8_bank(shared8);
    if (st != MOE_OK) return st;
    if (shared8->H != H || shared8->I != I) return MOE_ERR_INVALID_ARG;
  }
  if (mx_act && !gemm_mx_supported(T, H, I, T * k, shared != nullptr)) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x_bf16 || !w_router_bf16 || !out) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x_bf16) || !aligned16(w_router_bf16) || !aligned16(out))
    return MOE_ERR_INVALID_ARG;
  const bool few = T <= kDecodeMaxT && !mx_act;
  const size_t need = few ? (shared8 ? few_fp8_ws(T, H, I, E, k)
                                     : decode_ws_bytes(T, H, I, E, k, T * k, false, shared != nullptr))
                          : layer_ws(nullptr, T, H, I, E, k).bytes;
  if (!ws || !aligned16(ws)) return MOE_ERR_INVALID_ARG;
  if (ws_bytes < need) return MOE_ERR_WORKSPACE;
  if (few) {
    DecodeLaunch d{};
    d.ffn_mode = 0;
    d.x = static_cast<const uint16_t*>(x_bf16);
    d.wr = static_cast<const uint16_t*>(w_router_bf16);
    d.bias = logit_bias;
    d.routed = view(routed);
    d.has_shared = shared != nullptr;
    if (shared) d.shared = view(shared);
    d.T = T;
    d.H = H;
    d.I = I;
    d.E = E;
    d.k = k;
    d.R = T * k;
    d.out = out;
    d.ids_out = topk_ids_out;
    d.w_out = topk_w_out;
    if (shared8) {
      // one token, and blocks of 2..8 tokens: the FP8 expert streams inside
      // the few-token launches, like the MXFP4 shared expert
      DecodeLaunch f = d;
      f.has_shared = true;
      f.shared_fp8 = true;
      f.sh8_gu_w = shared8->gate_up_w;
      f.sh8_gu_s = shared8->gate_up_scales;
      f.sh8_d_w = shared8->down_w;
      f.sh8_d_s = shared8->down_scales;
      if (decode_fuses_fp8_shared(f)) {
        launch_decode(f, ws, stream);
        return launch_status();
      }
      // otherwise the FP8 expert runs first (it needs no routing); the
      // routed launches' combine adds its rows first, in the fixed order
      char* w8 = static_cast<char*>(ws) + align_up(decode_ws_bytes(T, H, I, E, k, T * k, false, false));
      float* y_sh = reinterpret_cast<float*>(w8);
      launch_fp8_ffn(static_cast<const uint16_t*>(x_bf16), shared8, T, y_sh,
                     w8 + align_up((size_t)T * H * sizeof(float)), stream);
      d.y_shared_ext = y_sh;
    }
    launch_decode(d, ws, stream);
    return launch_status();
  }

  const LayerWs L = layer_ws(ws, T, H, I, E, k);
  int32_t* ids = topk_ids_out ? topk_ids_out : L.ids;
  float* w = topk_w_out ? topk_w_out : L.w;
  const int R = T * k;

  const int rsplit = router_split(T, H, E);
  launch_router_logits(static_cast<const uint16_t*>(x_bf16),
                       static_cast<const uint16_t*>(w_router_bf16), logit_bias, T, H, E, L.logits,
                       stream, rsplit);
  launch_topk(L.logits, T, E, k, ids, w, stream, rsplit);
  launch_permute(ids, T, k, E, L.offsets, L.row_token, L.inv_row, L.active, L.perm, stream);

  FfnProblem p{};
  p.x = static_cast<const uint16_t*>(x_bf16);
  p.T = T;
  p.H = H;
  p.I = I;
  p.routed = view(routed);
  p.offsets = L.offsets;
  p.active = L.active;
  p.row_token = L.row_token;
  p.R = R;
  p.routed_slots = E < R ? E : R;
  p.h = L.h;
  p.y = L.y;
  p.has_shared = shared != nullptr;
  if (shared) {
    p.shared = view(shared);
    p.h_sh = L.h_sh;
    p.y_sh = L.y_sh;
  }
  if (mx_act) {
    launch_expert_gemm_mx(p, L.ffn, stream);
  } else if (gemm_supported(T, H, I, R, shared != nullptr)) {
    if (shared) {
      // the shared expert's down tiles may combine each token
      p.inv_row = L.inv_row;
      p.topk_w = w;
      p.k = k;
      p.out = out;
      if (launch_expert_gemm(p, L.ffn, stream)) return launch_status();
      launch_combine(L.y, L.inv_row, w, L.y_sh, T, k, H, R, out, stream);
      return launch_status();
    }
    launch_expert_gemm(p, L.ffn, stream);
  } else {
    launch_expert_ffn(p, stream);
  }
  // an FP8 shared expert runs after the routed FFN, in the same scratch
  if (shared8)
    launch_fp8_ffn(static_cast<const uint16_t*>(x_bf16), shared8, T, L.y_sh, L.ffn, stream);
  launch_combine(L.y, L.inv_row, w, (shared || shared8) ? L.y_sh : nullptr, T, k, H, R, out,
                 stream);
  return launch_status();
}

}  // namespace

extern "C" {

int moe_layer_forward(const void* x_bf16, const void* w_router_bf16, const float* logit_bias,
                      const moe_mxfp4_bank* routed, const moe_mxfp4_bank* shared, int T, int k,
                      float* out, int32_t* topk_ids_out, float* topk_w_out, void* ws,
                      size_t ws_bytes, hipStream_t stream) {
  return layer_forward(x_bf16, w_router_bf16, logit_bias, routed, shared, T, k, out, topk_ids_out,
                       topk_w_out, ws, ws_bytes, stream, false);
}

int moe_expert_ffn_fp8(const void* x_bf16, const moe_fp8_bank* bank, int T, float* y,
                       void* ws, size_t ws_bytes, hipStream_t stream) {
  begin_call();
  int st = check_fp8_bank(bank);
  if (st != MOE_OK) return st;
  st = check_dims(T, bank->H, 1, 1, bank->I);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!x_bf16 || !y || !aligned16(x_bf16) || !aligned16(y)) return MOE_ERR_INVALID_ARG;
  if (!ws || !aligned16(ws)) return MOE_ERR_INVALID_ARG;
  if (ws_bytes < fp8_ffn_ws(T, bank->H, bank->I)) return MOE_ERR_WORKSPACE;
  launch_fp8_ffn(static_cast<const uint16_t*>(x_bf16), bank, T, y, ws, stream);
  return launch_status();
}

int moe_layer_forward_fp8_shared(const void* x_bf16, const void* w_router_bf16,
                                 const float* logit_bias, const moe_mxfp4_bank* routed,
                                 const moe_fp8_bank* shared, int T, int k, float* out,
                                 int32_t* topk_ids_out, float* topk_w_out, void* ws,
                                 size_t ws_bytes, hipStream_t stream) {
  if (!shared) return MOE_ERR_INVALID_ARG;
  return layer_forward(x_bf16, w_router_bf16, logit_bias, routed, nullptr, T, k, out,
                       topk_ids_out, topk_w_out, ws, ws_bytes, stream, false, shared);
}

int moe_expert_ffn_nvfp4(const void* x_bf16, const moe_nvfp4_bank* bank,
                         const int32_t* expert_offsets, const int32_t* row_token, int T, int R,
                         float* y_rows, void* ws, size_t ws_bytes, hipStream_t stream) {
  begin_call();
  int st = check_nv_bank(bank);
  if (st != MOE_OK) return st;
  st = check_dims(T, bank->H, bank->E, 1, bank->I);
  if (st != MOE_OK) return st;
  if (R < 0) return MOE_ERR_INVALID_ARG;
  if (T == 0 || R == 0) return MOE_OK;
  if (!x_bf16 || !y_rows || !aligned16(x_bf16) || !aligned16(y_rows))
    return MOE_ERR_INVALID_ARG;
  if (!expert_offsets && bank->E != 1) return MOE_ERR_INVALID_ARG;
  if (!row_token && R > T) return MOE_ERR_INVALID_ARG;
  const int E = expert_offsets ? bank->E : 1;
  const bool mfma = R > kDecodeFfnMaxR && gemm_supported(T, bank->H, bank->I, R, false);
  const size_t need = mfma ? gemm_ws_bytes(T, bank->H, bank->I, E, R, false)
                           : ffn_ws_bytes(T, bank->H, bank->I, R, false);
  if (!ws || !aligned16(ws)) return MOE_ERR_INVALID_ARG;
  if (ws_bytes < need) return MOE_ERR_WORKSPACE;
  FfnProblem p{};
  p.x = static_cast<const uint16_t*>(x_bf16);
  p.T = T;
  p.H = bank->H;
  p.I = bank->I;
  p.routed = view_nv(bank);
  p.offsets = expert_offsets;
  p.row_token = row_token;
  p.R = R;
  p.routed_slots = expert_offsets ? (bank->E < R ? bank->E : R) : 1;
  p.h = static_cast<float*>(ws);
  p.y = y_rows;
  if (mfma)
    launch_expert_gemm(p, ws, stream);
  else
    launch_expert_ffn(p, stream);
  return launch_status();
}

int moe_layer_forward_nvfp4(const void* x_bf16, const void* w_router_bf16,
                            const float* logit_bias, const moe_nvfp4_bank* routed,
                            const moe_nvfp4_bank* shared, int T, int k, float* out,
                            int32_t* topk_ids_out, float* topk_w_out, void* ws, size_t ws_bytes,
                            hipStream_t stream) {
  begin_call();
  int st = check_nv_bank(routed);
  if (st != MOE_OK) return st;
  const int E = routed->E, H = routed->H, I = routed->I;
  st = check_dims(T, H, E, k, I);
  if (st != MOE_OK) return st;
  if (shared) {
    st = check_nv_bank(shared);
    if (st != MOE_OK) return st;
    if (shared->E != 1 || shared->H != H || shared->I != I) return MOE_ERR_INVALID_ARG;
  }
  if (T == 0) return MOE_OK;
  if (!x_bf16 || !w_router_bf16 || !out) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x_bf16) || !aligned16(w_router_bf16) || !aligned16(out))
    return MOE_ERR_INVALID_ARG;
  if (!ws || !aligned16(ws)) return MOE_ERR_INVALID_ARG;
  if (T <= kDecodeMaxT) {
    // one token: the fused launch; a block of 2..8 tokens: the block
    // launches; both with NVFP4 items
    DecodeLaunch d{};
    d.ffn_mode = 0;
    d.x = static_cast<const uint16_t*>(x_bf16);
    d.wr = static_cast<const uint16_t*>(w_router_bf16);
    d.bias = logit_bias;
    d.routed = view_nv(routed);
    d.has_shared = shared != nullptr;
    if (shared) d.shared = view_nv(shared);
    d.T = T;
    d.H = H;
    d.I = I;
    d.E = E;
    d.k = k;
    d.R = T * k;
    d.out = out;
    d.ids_out = topk_ids_out;
    d.w_out = topk_w_out;
    if (decode_fuses_nvfp4(d)) {
      if (ws_bytes < decode_ws_bytes(T, H, I, E, k, T * k, false, shared != nullptr))
        return MOE_ERR_WORKSPACE;
      launch_decode(d, ws, stream);
      return launch_status();
    }
  }
  if (ws_bytes < layer_ws(nullptr, T, H, I, E, k).bytes) return MOE_ERR_WORKSPACE;
  const LayerWs L = layer_ws(ws, T, H, I, E, k);
  int32_t* ids = topk_ids_out ? topk_ids_out : L.ids;
  float* w = topk_w_out ? topk_w_out : L.w;
  const int R = T * k;
  const int rsplit = router_split(T, H, E);
  launch_router_logits(static_cast<const uint16_t*>(x_bf16),
                       static_cast<const uint16_t*>(w_router_bf16), logit_bias, T, H, E, L.logits,
                       stream, rsplit);
  launch_topk(L.logits, T, E, k, ids, w, stream, rsplit);
  launch_permute(ids, T, k, E, L.offsets, L.row_token, L.inv_row, L.active, L.perm, stream);
  FfnProblem p{};
  p.x = static_cast<const uint16_t*>(x_bf16);
  p.T = T;
  p.H = H;
  p.I = I;
  p.routed = view_nv(routed);
  p.offsets = L.offsets;
  p.active = L.active;
  p.row_token = L.row_token;
  p.R = R;
  p.routed_slots = E < R ? E : R;
  p.h = L.h;
  p.y = L.y;
  p.has_shared = shared != nullptr;
  if (shared) {
    p.shared = view_nv(shared);
    p.h_sh = L.h_sh;
    p.y_sh = L.y_sh;
  }
  if (T > kDecodeMaxT && gemm_supported(T, H, I, R, shared != nullptr)) {
    if (shared) {
      // the shared expert's down tiles may combine each token
      p.inv_row = L.inv_row;
      p.topk_w = w;
      p.k = k;
      p.out = out;
      if (launch_expert_gemm(p, L.ffn, stream)) return launch_status();
      launch_combine(L.y, L.inv_row, w, L.y_sh, T, k, H, R, out, stream);
      return launch_status();
    }
    launch_expert_gemm(p, L.ffn, stream);
  } else {
    launch_expert_ffn(p, stream);
  }
  launch_combine(L.y, L.inv_row, w, shared ? L.y_sh : nullptr, T, k, H, R, out, stream);
  return launch_status();
}

int moe_layer_forward_noalloc(const void* x_bf16, const void* w_router_bf16,
                              const float* logit_bias, const moe_mxfp4_bank* routed,
                              const moe_mxfp4_bank* shared, int T, int k, float* out,
                              int32_t* topk_ids_out, float* topk_w_out, hipStream_t stream) {
  void* ws = nullptr;
  const int st = noalloc_scratch(&ws);
  if (st != MOE_OK) {
    begin_call();
    return st;
  }
  return layer_forward(x_bf16, w_router_bf16, logit_bias, routed, shared, T, k, out, topk_ids_out,
                       topk_w_out, ws, kNoallocScratchBytes, stream, false);
}

int moe_layer_forward_mxfp8_act(const void* x_bf16, const void* w_router_bf16,
                                const float* logit_bias, const moe_mxfp4_bank* routed,
                                const moe_mxfp4_bank* shared, int T, int k, float* out,
                                int32_t* topk_ids_out, float* topk_w_out, void* ws,
                                size_t ws_bytes, hipStream_t stream) {
  return layer_forward(x_bf16, w_router_bf16, logit_bias, routed, shared, T, k, out, topk_ids_out,
                       topk_w_out, ws, ws_bytes, stream, true);
}

}  // extern "C"
