// Internal launchers behind the C ABI. Arguments are already validated by
// the entry points; each launcher only enqueues work on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Timing hook state (abi.hip): the start / stop events for the next launch
// (null when the hook is off), and the log of launch names of the call.
void next_launch_events(hipEvent_t* start, hipEvent_t* stop);
void log_launch(const char* name);

// Every kernel launch goes through here. With the hook set, the launch
// carries the caller's start / stop events, which the runtime stamps at the
// kernel's own dispatch begin and end (no marker packets between kernels).
template <typename F, typename... Args>
inline void launch(const char* name, F kernel, dim3 grid, dim3 block, uint32_t shmem,
                   hipStream_t s, Args... args) {
  hipEvent_t start = nullptr, stop = nullptr;
  next_launch_events(&start, &stop);
  hipExtLaunchKernelGGL(kernel, grid, block, shmem, s, start, stop, 0, args...);
  log_launch(name);
}

// Token counts up to this use the GEMV router; above it the MFMA GEMM.
constexpr int kRouterGemvMaxT = 16;
// Pair counts up to this are bucketed by one workgroup.
constexpr int kPermuteChunk = 2048;

// split > 1 (router_split): the router writes `split` partial logit arrays
// of [T][E] over consecutive ranges of H (the bias in the first), and the
// top-k sums them in order.
int router_split(int T, int H, int E);
void launch_router_logits(const uint16_t* x, const uint16_t* wr, const float* bias,
                          int T, int H, int E, float* logits, hipStream_t s, int split = 1);
void launch_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                 hipStream_t s, int split = 1);

size_t permute_ws_bytes(int T, int k, int E);
// `active` [E] receives the ids of experts with rows, ascending, then -1s.
void launch_permute(const int32_t* ids, int T, int k, int E, int32_t* offsets,
                    int32_t* row_token, int32_t* inv_row, int32_t* active,
                    void* ws, hipStream_t s);

// One expert bank as the kernels see it. codec 0: MXFP4 (E8M0 scale per
// 32 codes); codec 1: NVFP4 (E4M3 scale per 16 codes, scale rows K / 16
// bytes, plus an optional fp32 scale per expert and matrix, gscale [E][3]:
// gate, up, down). The few-token persistent kernels take MXFP4 only.
struct BankView {
  const uint8_t* gu_codes;
  const uint8_t* gu_scales;
  const uint8_t* d_codes;
  const uint8_t* d_scales;
  int E;
  int codec;
  const float* gscale;
};
constexpr int kCodecMxfp4 = 0;
constexpr int kCodecNvfp4 = 1;

// Expert FFN over bucketed rows: routed bank rows (offsets/active/row_token)
// plus, optionally, the shared expert over all T tokens.
struct FfnProblem {
  const uint16_t* x;   // [T][H] bf16
  int T, H, I;
  BankView routed;
  const int32_t* offsets;    // [E+1] or null (single expert, rows [0, R))
  const int32_t* active;     // [E] active expert list or null (derive from offsets)
  const int32_t* row_token;  // [R] or null (row r is token r)
  int R;                     // routed rows
  int routed_slots;          // upper bound of experts with rows
  float* h;                  // [R][I] fp32 scratch
  float* y;                  // [R][H] fp32 out
  bool has_shared;
  BankView shared;
  float* h_sh;               // [T][I]
  float* y_sh;               // [T][H]
  // Layer calls on the grouped GEMM with a shared expert: the combine's
  // inputs and output. With out set and enough tokens, the shared expert's
  // down tiles run in a launch of their own after the routed ones and
  // combine each token in their epilogue (no y_sh round trip, no combine
  // launch).
  const int32_t* inv_row;    // [T][k]
  const float* topk_w;       // [T][k]
  int k;
  float* out;                // [T][H] or null
};

size_t ffn_ws_bytes(int T, int H, int I, int R, bool shared);
void launch_expert_ffn(const FfnProblem& p, hipStream_t s);

// The MFMA grouped GEMM for many rows (h in fp16 in its own workspace; the
// FfnProblem's h / h_sh are unused). Call only where gemm_supported().
bool gemm_supported(int T, int H, int I, int R, bool shared);
size_t gemm_ws_bytes(int T, int H, int I, int E, int R, bool shared);
// Returns whether the launches also wrote p.out (the combine folded into
// the shared expert's down tiles); otherwise the caller combines.
bool launch_expert_gemm(const FfnProblem& p, void* ws, hipStream_t s);

// MXFP8-activation mode of the grouped GEMM: x and h rounded to E4M3 with
// one E8M0 scale per 32, the bank's E2M1 codes fed to the scaled MFMA as
// they are. Call only where gemm_mx_supported().
bool gemm_mx_supported(int T, int H, int I, int R, bool shared);
size_t gemm_mx_ws_bytes(int T, int H, int I, int E, int R, bool shared);
void launch_expert_gemm_mx(const FfnProblem& p, void* ws, hipStream_t s);
// bf16 values in blocks of 32 -> E4M3 codes + E8M0 scales (n_blocks blocks).
void launch_quant_mxfp8(const uint16_t* x, long n_blocks, uint8_t* q, uint8_t* s, hipStream_t st);

// One FP8 expert (E4M3, one E8M0 scale per 32 x 32 block) over T rows,
// row t = token t: few-token GEMVs (h fp32 [T][I] in `h`) or the grouped
// GEMM (h fp16 in its own workspace).
struct Fp8Ffn {
  const uint16_t* x;     // [T][H] bf16
  int T, H, I;
  const uint8_t* gu_w;   // [2][I][H]
  const uint8_t* gu_s;   // [2][I/32][H/32]
  const uint8_t* d_w;    // [H][I]
  const uint8_t* d_s;    // [H/32][I/32]
  float* h;              // GEMV path: [T][I] fp32 scratch
  float* y;              // [T][H] fp32 out
};
size_t fp8_gemv_ws_bytes(int T, int I);
void launch_fp8_ffn_gemv(const Fp8Ffn& p, hipStream_t s);  // T <= kDecodeMaxT
size_t fp8_gemm_ws_bytes(int T, int H, int I);
void launch_fp8_gemm(const Fp8Ffn& p, void* ws, hipStream_t s);  // where gemm_supported()

// The persistent few-token kernel (layer mode: router..combine in one
// launch; FFN mode: bucketed rows given by offsets, writes y_rows).
constexpr int kDecodeMaxT = 16;
constexpr int kDecodeFfnMaxR = 128;

struct DecodeLaunch {
  int ffn_mode;
  const uint16_t* x;
  const uint16_t* wr;
  const float* bias;
  BankView routed, shared;
  bool has_shared;
  int T, H, I, E, k, R;
  const int32_t* offsets;    // FFN mode
  const int32_t* row_token;  // FFN mode
  float* out;
  int32_t* ids_out;
  float* w_out;
  float* y_rows;             // FFN mode output
  // layer mode, one token: the shared expert in FP8 (E4M3, 32 x 32 E8M0
  // blocks: gate_up [2][I][H] + scales [2][I/32][H/32], down [H][I] +
  // scales [H/32][I/32]) streamed inside the fused launches; with has_shared
  const uint8_t *sh8_gu_w, *sh8_gu_s, *sh8_d_w, *sh8_d_s;
  bool shared_fp8;
  const float* y_shared_ext; // layer mode: [T][H] shared-expert rows computed
                             // by earlier launches (the combine adds them
                             // first), or null
};

size_t decode_ws_bytes(int T, int H, int I, int E, int k, int R, bool ffn, bool shared);
// Whether launch_decode streams an FP8 shared expert inside its fused
// one-token launches for this call (layer mode, one token, shapes the fused
// kernels take); otherwise the caller runs the FP8 expert separately.
bool decode_fuses_fp8_shared(const DecodeLaunch& d);
// Whether launch_decode takes this call with NVFP4 banks (BankView codec):
// only the one-token fused launches hold NVFP4 items.
bool decode_fuses_nvfp4(const DecodeLaunch& d);
void launch_decode(const DecodeLaunch& d, void* ws, hipStream_t s);
// Test hook: while on, the routing's first bounded wait of each few-token
// layer call gives up after a few polls (calling thread only).
void set_force_wait_timeout(int on);
// Wait code recorded by the last few-token call made with workspace `ws`
// (0 = every wait completed; blocking 16-byte copy), or -1 if the copy fails.
int read_decode_status(const void* ws);

void launch_combine(const float* y_rows, const int32_t* inv_row, const float* w,
                    const float* y_shared, int T, int k, int H, int R, float* out,
                    hipStream_t s);

}  // namespace moe
