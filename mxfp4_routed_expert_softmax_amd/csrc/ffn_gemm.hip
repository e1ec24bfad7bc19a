// Expert FFN for many rows (prefill): a grouped GEMM over the experts'
// buckets on gfx950 MFMA, with the MXFP4 weights dequantised exactly in
// registers.
//
// A prefill chunk of a few hundred tokens or more touches nearly every
// expert (FreeToken issue #444, janit's comment, section 3), so the bank is
// read once per 64 bucket rows and the arithmetic sits on the matrix cores:
//
//   gate/up:  h = silu(X_e W_gate[e]^T) * (X_e W_up[e]^T)   bf16 MFMA, h -> fp16
//   down:     y = h_e W_down[e]^T                            fp16 MFMA, y -> fp32
//
// X_e are the token rows of expert e's bucket, gathered through row_token;
// the shared expert is one more bucket over all T tokens. Every bucket is
// cut into 64-row blocks; a plan kernel lists
// the (row block, column block) tiles of both GEMMs in an L2-friendly
// order, and each XCD takes a consecutive stretch of the list.
//
// Per workgroup (256 threads, two a CU): 64 rows x 256 weight rows (for
// gate/up: 128 gate + the 128 up rows of the same output columns), 4 waves
// of 64 x 64 built from v_mfma_f32_16x16x32_bf16 / _f16. K advances 128 per
// step through a 2-stage LDS pipeline filled by direct global -> LDS loads:
//  * A: 64 rows x 128 K (bf16 x or fp16 h), each row's 16-byte pieces
//    permuted (piece p at slot p ^ (row & 15));
//  * B: 256 weight rows x 64 bytes of packed E2M1 codes (piece p of row r
//    at slot p ^ ((r / 4) & 3));
//  * the step's E8M0 scales, 4 bytes per weight row.
// A stage is 33 KB (34 KB with an NVFP4 bank's 8 scale bytes per weight
// row), so two workgroups share a CU and one's copies overlap the other's
// matrix-core work. Gate/up, whose scale rows are a multiple of 16 bytes at
// the layer's shape, instead copies each weight row's scales 16 bytes at a
// time (4 K steps; 2 for NVFP4) into two chunk buffers after the stages.
// A bucket of at most 16 rows takes a 16-row tile: 4 KB of A a step, so
// three stages fit in the same LDS and its weight copies run two steps
// ahead (such tiles are bound by their copies).
// Lane (column c, lane group g) of a wave takes the 32 codes of K range
// [32 g, 32 g + 32) of its weight row, one E8M0 block, and converts them
// with the gfx950 scaled FP4 conversion (exact: an E2M1 value times a power
// of two in range is representable in bf16 and fp16). MFMA sub-step s uses
// K values 32 g + 8 s .. + 7 of lane group g for both operands; an MFMA dot
// product only needs A and B to agree on that assignment.
//
// Precision: x and the dequantised weights are exact in bf16; h is rounded
// once to fp16 (relative 2^-11; |h| < 65504), the down weights are exact in
// fp16 for E8M0 exponents in [-23, 13]; every sum is fp32.
#include <type_traits>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kBM = 128;        // bucket rows per tile (gemm_kernel: 64)
constexpr int kBK = 128;        // K per pipeline step
constexpr int kWRows = 256;     // weight rows per tile
constexpr int kThreads = 512;   // 8 waves: 2 (rows) x 4 (weight rows)
constexpr int kStages = 2;
constexpr int kAPieces = kBM * kBK / 8;       // 16-byte pieces of A per stage (2048)
constexpr int kBPieces = kWRows * kBK / 32;   // 16-byte pieces of codes per stage (1024)
constexpr int kABytes = kAPieces * 16;        // 32 KB
constexpr int kBBytes = kBPieces * 16;        // 16 KB
// E8M0 bytes of the tile's 256 weight rows over all of K (K <= 8192: 64 KB),
// loaded once per tile
constexpr int kScaleBytes = kWRows * (8192 / 32);
constexpr int kNvSBytes = kWRows * 8;        // NVFP4: 8 scale bytes per weight row and K step
constexpr int kALoads = kAPieces / kThreads;  // 4 per thread per stage
constexpr int kBLoads = kBPieces / kThreads;  // 2 per thread per stage

struct GemmArgs {
  const uint16_t* x;  // [T][H] bf16
  int T, H, I, E, R;
  BankView routed, shared;
  int has_shared;
  const int32_t* offsets;    // [E+1] routed buckets, or null (one expert, rows [0, R))
  const int32_t* row_token;  // [R] or null (row r is token r)
  int32_t* tile_b[2];    // per GEMM (0 gate/up, 1 down): bucket of tile t
  int32_t* tile_mn[2];   // (row block << 8) | column block of tile t
  int32_t* tile_count;   // [2] tiles of each GEMM
  int max_rb;            // capacity in row blocks
  int bm;                // rows per tile (row block): 64, or 128 (FP8, MX)
  _Float16* h;    // [R + T][I]: routed rows, then the shared expert's T rows
  float* y;       // [R][H]
  float* y_sh;    // [T][H]
  // Down tiles of one launch: 0 all; 1 the routed buckets' (the list up to
  // tile_count[2]); 2 the shared expert's, whose epilogue writes the
  // combined output out = y_sh + sum_j w[j] y[inv_row[j]] (j ascending)
  // from its accumulators and the routed rows of launch 1.
  int part;
  const int32_t* inv_row;  // [T][k]
  const float* topk_w;     // [T][k]
  int k;
  float* out;              // [T][H]
  // MXFP8-activation mode: x and h as E4M3 codes with one E8M0 scale per 32
  const uint8_t* xq;  // [T][H]
  const uint8_t* xs;  // [T][H / 32]
  uint8_t* hq;        // [R + T][I]
  uint8_t* hs;        // [R + T][I / 32]
};

struct Bucket {
  int e;        // slot in its bank
  int begin;    // first row (into h; routed rows also index row_token and y)
  int count;    // rows
  bool shared;
};

// Bucket b: routed expert b for b < E, the shared expert for b == E.
__device__ __forceinline__ Bucket bucket_of(const GemmArgs& g, int b) {
  if (b >= g.E) return Bucket{0, g.R, g.T, true};
  if (!g.offsets) return Bucket{0, 0, g.R, false};
  const int lo = min(max(g.offsets[b], 0), g.R);
  const int hi = min(max(g.offsets[b + 1], lo), g.R);
  return Bucket{b, lo, hi - lo, false};
}

// Workgroups of the plan kernel: each repeats the (small) scan over the
// buckets and writes every kPlanBlocks-th stretch of 1024 tiles.
constexpr int kPlanBlocks = 64;

// Tile lists of both GEMMs, in an order that keeps shared data in one L2:
// buckets in order (routed experts by id, then the shared expert); each
// bucket's 128-row blocks in chunks of up to `chunk` blocks; inside a chunk
// the column block outer and the row block inner. So the row blocks of a
// chunk (A, re-read by every column block) stay in cache while its column
// blocks go by, and the row blocks sharing a weight tile (B) run together.
// The GEMMs hand consecutive stretches of this list to each XCD.
// Workgroups of 1024 threads (at most 1025 buckets).
__device__ __forceinline__ int plan_chunk(int K, int bm) {
  // row blocks whose activations take about 2.5 MB (L2 is 4 MB per XCD)
  return min(max((5 << 19) / (bm * K * 2), 1), 16);
}

__global__ __launch_bounds__(1024) void gemm_plan_kernel(GemmArgs g) {
  __shared__ int s_tmp[32];
  __shared__ int s_rb[1026];    // exclusive scan of row blocks per bucket
  const int nb = g.E + (g.has_shared ? 1 : 0);
  int cnt[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int b = threadIdx.x + q * 1024;
    cnt[q] = b < nb ? (bucket_of(g, b).count + g.bm - 1) / g.bm : 0;
  }
  int total0 = 0, total1 = 0;
  const int base0 = block_exclusive_scan(cnt[0], s_tmp, &total0);
  const int base1 = total0 + block_exclusive_scan(cnt[1], s_tmp, &total1);
  s_rb[threadIdx.x] = base0;
  if (threadIdx.x + 1024 < 1026) s_rb[threadIdx.x + 1024] = base1;
  const int total_rb = min(total0 + total1, g.max_rb);
  __syncthreads();
#pragma unroll
  for (int kind = 0; kind < 2; ++kind) {
    const int ncol = kind == 0 ? g.I / (kWRows / 2) : g.H / kWRows;
    const int chunk = plan_chunk(kind == 0 ? g.H : g.I, g.bm);
    const int total = total_rb * ncol;
    for (int q = blockIdx.x * 1024 + threadIdx.x; q < total; q += gridDim.x * 1024) {
      // bucket: the last b with s_rb[b] * ncol <= q (buckets without rows
      // have equal bases; the search lands on the one that owns q)
      int lo = 0, hi = nb;  // invariant: s_rb[lo] * ncol <= q < s_rb[hi] * ncol
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_rb[mid] * ncol <= q) lo = mid; else hi = mid;
      }
      const int nblk = s_rb[lo + 1] - s_rb[lo];
      const int local = q - s_rb[lo] * ncol;
      const int c = local / (chunk * ncol);
      const int csz = min(chunk, nblk - c * chunk);
      const int idx = local - c * chunk * ncol;
      const int nt = idx / csz;
      const int mt = c * chunk + (idx - nt * csz);
      g.tile_b[kind][q] = lo;
      g.tile_mn[kind][q] = (mt << 8) | nt;
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) {
      g.tile_count[kind] = total;
      // the down list's routed tiles come first, the shared bucket's last
      if (kind == 1) g.tile_count[2] = g.has_shared ? min(s_rb[g.E], total_rb) * ncol : total;
    }
  }
}

// 8 E2M1 codes (one word) times `sc` -> 8 bf16 / fp16
__device__ __forceinline__ bf16x8_t fp4x8_bf16(uint32_t w, float sc) {
  const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0);
  const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1);
  const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2);
  const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3);
  return bf16x8_t{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}
__device__ __forceinline__ f16x8_t fp4x8_f16(uint32_t w, float sc) {
  const f16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sc, 0);
  const f16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sc, 1);
  const f16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sc, 2);
  const f16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sc, 3);
  return f16x8_t{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

// MFMA operand type, conversion and product of each GEMM: gate/up in bf16,
// down in fp16 (h is carried in fp16).
template <bool GU>
using Op = typename std::conditional<GU, bf16x8_t, f16x8_t>::type;
template <bool GU>
__device__ __forceinline__ Op<GU> cvt8(uint32_t w, float sc) {
  if constexpr (GU)
    return fp4x8_bf16(w, sc);
  else
    return fp4x8_f16(w, sc);
}
template <bool GU>
__device__ __forceinline__ f32x4_t mma(uint4 a, Op<GU> b, f32x4_t c) {
  if constexpr (GU)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), b, c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), b, c, 0, 0, 0);
}
// NVFP4: 8 E2M1 codes times an E4M3 scale that is generally not a power of
// two. The scaled conversions above are only ever given powers of two (an
// NVFP4 GEMM that passed the E4M3 value there came out 0.71 rel-L2 off, while
// the GEMV that multiplies after converting matched): convert at scale 1
// and multiply exactly (E2M1 x E4M3 has at most 6 significant bits), in fp32
// then packed to bf16 for gate/up, in fp16 for down.
template <bool GU>
__device__ __forceinline__ Op<GU> cvt8_nv(uint32_t w, float sc) {
  if constexpr (GU) {
    bf16x8_t r;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x2_t f = q == 0 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0)
                        : q == 1 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1)
                        : q == 2 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2)
                                 : __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
      r[2 * q] = (__bf16)(f.x * sc);
      r[2 * q + 1] = (__bf16)(f.y * sc);
    }
    return r;
  } else {
    const _Float16 h = (_Float16)sc;
    const f16x2_t s2 = f16x2_t{h, h};
    const f16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s2;
    const f16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s2;
    const f16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s2;
    const f16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s2;
    return f16x8_t{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
  }
}

__device__ __forceinline__ uint32_t word_of(uint4 v, int s) {
  return s == 0 ? v.x : s == 1 ? v.y : s == 2 ? v.z : v.w;
}

// Direct global -> LDS loads: lane l's 16 (4) bytes at base + voff land at
// LDS byte address lds + 16 l (4 l); lds is wave-uniform. Written as inline
// asm so the compiler does not guard every later LDS read with a wait for
// them: the kernel waits explicitly (vmcnt + barrier) before reading a
// stage. The compiler's own waits for register loads stay correct, as
// vector loads complete in issue order.
// m0 is named as clobbered so the compiler knows each copy rewrites it: it
// then keeps no value of its own there and puts the wait state the
// hardware needs between a copy and the next write of m0. (clang warns that
// m0 is a reserved register; the warning is silenced for these two only.)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_load16(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, %2"
               :
               : "v"(voff), "s"(lds), "s"(base)
               : "memory", "m0");
}
__device__ __forceinline__ void lds_load4(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, %2"
               :
               : "v"(voff), "s"(lds), "s"(base)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Weight-row tiling of a workgroup's 256 rows r, and the output columns
// (n0 = tile column offset): gate/up: r < 128 -> gate row n0 + r, else the
// up row n0 + r - 128 (128 output columns per tile); down: row n0 + r (256
// output columns). Wave (wm, wn) with lane column c owns fragment j:
//   gate/up: r = 32 wn + 16 (j % 2) + c + 128 (j / 2)
//   down:    r = 64 wn + 16 j + c
template <bool GU>
__device__ __forceinline__ int frag_row(int wn, int j, int c) {
  return GU ? 32 * wn + 16 * (j & 1) + c + 128 * (j >> 1) : 64 * wn + 16 * j + c;
}

// LDS slot swizzles of the fragment reads (16 consecutive rows per lane
// group read one piece index each): code rows (64 B, 4 slots) at
// p ^ ((r / 4) % 4), E4M3 activation rows (128 B, 8 slots) at
// p ^ ((r / 2) % 8). Variants that make every 8 and every 16 consecutive
// rows hit distinct 16-byte bank groups lowered the bank-conflict counter
// but measured 5 % slower on the MX gate/up GEMM, so these stay.
__device__ __forceinline__ int code_swz(int r) { return (r >> 2) & 3; }
__device__ __forceinline__ int act8_swz(int r) { return (r >> 1) & 7; }
// Scale rows in LDS: srow bytes (K / 32, a multiple of 4) padded to an odd
// number of 4-byte words, so 16 consecutive rows hit distinct banks; at
// K = 8192 the padded rows would not fit and stay unpadded.
__device__ __forceinline__ uint32_t scale_stride(uint32_t srow) {
  return (((srow >> 2) & 1u) == 0u && srow < 256u) ? srow + 4u : srow;
}
// Copies `nrows` rows of srow bytes (source byte offset src_row(r) of row r)
// into LDS at lds + r * stride, one row per wave iteration, one 4-byte
// piece per lane (srow <= 256).
template <class F>
__device__ __forceinline__ void load_scale_rows(const void* src, F src_row, int nrows,
                                                uint32_t srow, uint32_t stride, uint32_t lds,
                                                int wave, int lane, int nwaves) {
  for (int r = wave; r < nrows; r += nwaves)
    if (lane < (int)(srow >> 2)) lds_load4(src, src_row(r) + 4u * (uint32_t)lane, lds + (uint32_t)r * stride);
}

// NV: NVFP4 bank (E4M3 scale per 16 codes, fp32 matrix scale). Its scales,
// 8 bytes per weight row and K step, travel with each stage (the tile's
// scales over all of K would take 80 KB at K = 5120); a lane's 32 codes
// span two scales, one for MFMA sub-steps 0-1 and one for 2-3. The
// products E2M1 x E4M3 are exact in bf16 and fp16; the matrix scale
// multiplies the fp32 sums in the epilogue.
// BM: bucket rows per tile, 64 (4 waves, two workgroups a CU; the one
// instantiated) or 128 (8 waves, one a CU, measured slower); the waves are
// 1 or 2 (rows) x 4 (weight rows). The step's scales travel with each stage
// (PSC) except for MXFP4 at 128 rows, whose tile scales over all of K are
// loaded once.
// The combine of token m at columns n, n + 16, n + 32, n + 48, from its
// shared row's values ys: out = ys + sum_j w[j] y[inv_row[j]], j ascending,
// one fp32 FMA per term (the combine kernel's arithmetic). The routing row
// is read first, 8 choices at a time, then their y values.
__device__ __forceinline__ void combine_row(const GemmArgs& g, int m, int n, const float (&ys)[4]) {
  float acc[4] = {ys[0], ys[1], ys[2], ys[3]};
  const int32_t* ir = g.inv_row + (size_t)m * g.k;
  const float* wr = g.topk_w + (size_t)m * g.k;
  for (int j0 = 0; j0 < g.k; j0 += 8) {
    int r[8];
    float w[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      r[j] = j0 + j < g.k ? ir[j0 + j] : -1;
      w[j] = j0 + j < g.k ? wr[j0 + j] : 0.0f;
    }
    float yv[8][4];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float* yr = g.y + (size_t)min(max(r[j], 0), max(g.R - 1, 0)) * g.H + n;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        yv[j][q] = r[j] >= 0 && r[j] < g.R ? yr[16 * q] : __builtin_nanf("");
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (r[j] < 0) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] = fmaf(w[j], yv[j][q], acc[q]);
    }
  }
  float* o = g.out + (size_t)m * g.H + n;
#pragma unroll
  for (int q = 0; q < 4; ++q) o[16 * q] = acc[q];
}

template <bool GU, bool NV, int BM>
__global__ __launch_bounds__(BM == 128 ? 512 : 256, BM == 128 ? 1 : 2) void gemm_kernel(GemmArgs g) {
  constexpr int NT = BM == 128 ? 512 : 256;
  constexpr bool PSC = NV || BM == 64;
  constexpr int kABy = BM * kBK * 2;           // A bytes per stage
  constexpr int kSBy = NV ? kNvSBytes : (BM == 64 ? kWRows * 4 : 0);
  constexpr int kSt = kABy + kBBytes + kSBy;   // bytes per stage
  constexpr int kAL = BM * 16 / NT, kBL = kBPieces / NT;  // copies per thread and stage
  // gate/up at 64 rows: two 16-byte scale chunks per weight row (4 K steps
  // of MXFP4 scales, 2 of NVFP4) after the stages (down, K = I, has 72-byte
  // MXFP4 scale rows at the layer's shape and keeps the per-step loads)
  constexpr int kChunkBy = BM != 64 || !GU ? 0 : kWRows * 16;
  constexpr int kCkSteps = NV ? 2 : 4;  // K steps per chunk
  __shared__ __align__(16) char lds[PSC ? kStages * kSt + 2 * kChunkBy
                                        : kStages * kSt + kScaleBytes];
  constexpr int kBN = GU ? kWRows / 2 : kWRows;  // output columns per tile
  const int N = GU ? g.I : g.H;
  const int K = GU ? g.H : g.I;
  const int ncol = N / kBN;
  // Workgroups are dispatched to the 8 XCDs round-robin by index: hand XCD
  // x (blocks x, x + 8, ...) the consecutive tiles [x * per, (x + 1) * per)
  // of the list, so the tiles that share data share an L2.
  const int all = min(g.tile_count[GU ? 0 : 1], g.max_rb * ncol);
  const int split = GU || g.part == 0 ? all : min(max(g.tile_count[2], 0), all);
  const int lo = !GU && g.part == 2 ? split : 0, hi = !GU && g.part == 1 ? split : all;
  const int total = hi - lo;
  const int per = (total + 7) / 8;
  const int slot = blockIdx.x >> 3;
  const int t = lo + (blockIdx.x & 7) * per + slot;
  if (slot >= per || t >= hi) return;
  const int nb = g.E + (g.has_shared ? 1 : 0);
  const Bucket bk = bucket_of(g, min(max(g.tile_b[GU ? 0 : 1][t], 0), nb - 1));
  const int mn = g.tile_mn[GU ? 0 : 1][t];
  const int m0 = (mn >> 8) * BM;
  const int n0 = min(mn & 255, ncol - 1) * kBN;
  if (m0 < 0 || m0 >= bk.count) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3, c = lane & 15, grp = lane >> 4;
  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds;

  // A: thread tid fills slot (row 32 u + tid / 16, piece tid % 16), which
  // holds K piece (tid % 16) ^ (row % 16) of that row.
  const void* a_src = GU ? static_cast<const void*>(g.x) : static_cast<const void*>(g.h);
  uint32_t a_off[kAL];
  {
    const int piece = (tid & 15) ^ ((tid >> 4) & 15);
#pragma unroll
    for (int u = 0; u < kAL; ++u) {
      const int m = min(m0 + (NT / 16) * u + (tid >> 4), bk.count - 1);
      int row;
      if (GU) {
        row = bk.shared ? m : (g.row_token ? g.row_token[bk.begin + m] : bk.begin + m);
        row = min(max(row, 0), g.T - 1);
      } else {
        row = bk.begin + m;
      }
      a_off[u] = ((uint32_t)row * (uint32_t)K + (uint32_t)(piece * 8)) * 2u;
    }
  }

  // B: thread tid fills code slot (r = 128 u + tid / 4, piece tid % 4),
  // which holds piece (tid % 4) ^ ((r / 4) % 4) of weight row r.
  const BankView bv = bk.shared ? g.shared : g.routed;
  const uint32_t crow = (uint32_t)K / 2, srow = (uint32_t)K / (NV ? 16 : 32);
  const size_t mat_rows = GU ? 2 * (size_t)g.I : (size_t)g.H;
  const uint8_t* cbase = (GU ? bv.gu_codes : bv.d_codes) + (size_t)bk.e * mat_rows * crow;
  const uint8_t* sbase = (GU ? bv.gu_scales : bv.d_scales) + (size_t)bk.e * mat_rows * srow;
  auto wrow = [&](int r) -> uint32_t {  // tile weight row -> row of the expert's matrix
    return GU ? (uint32_t)(r < 128 ? n0 + r : g.I + n0 + r - 128) : (uint32_t)(n0 + r);
  };
  uint32_t b_off[kBL];
#pragma unroll
  for (int u = 0; u < kBL; ++u) {
    const int r = (NT / 4) * u + (tid >> 2);
    b_off[u] = wrow(r) * crow + 16u * (uint32_t)((tid & 3) ^ ((r >> 2) & 3));
  }
  const uint32_t s_lds = lds_base + kStages * kSt;
  // NV: dword d of the stage's scales is dword d % 2 of weight row d / 2's
  // 8 scale bytes of the K step (thread tid copies d = tid, and with 256
  // threads also d = tid + 256); MXFP4 at 64 rows: thread tid copies the 4
  // scale bytes of weight row tid
  const uint32_t nv_off = NV ? wrow(tid >> 1) * srow + 4u * (uint32_t)(tid & 1)
                              : PSC ? wrow(tid) * srow : 0u;
  const uint32_t nv_off2 = NV && NT == 256 ? wrow((tid + 256) >> 1) * srow + 4u * (uint32_t)(tid & 1)
                                           : 0u;
  // Scale rows a multiple of 16 bytes: thread tid copies row tid's scale
  // bytes of kCkSteps K steps at a time, one 16-byte load in place of a
  // 4-byte load (two for NVFP4) every step, each of which touches the cache
  // lines of 256 scale rows for 1 KB (2 KB)
  bool chunked = false;
  if constexpr (kChunkBy > 0) chunked = (srow & 15u) == 0 && ((uintptr_t)sbase & 15u) == 0;
  const uint32_t c_lds = lds_base + kStages * kSt;
  const uint32_t ck_off = kChunkBy > 0 ? wrow(tid) * srow : 0u;

  // Stage `st` <- K step `ks`.
  auto issue = [&](int st, int ks) {
    const uint32_t base = lds_base + (uint32_t)(st * kSt);
    const uint32_t k0 = (uint32_t)(ks * kBK);
#pragma unroll
    for (int u = 0; u < kAL; ++u)
      lds_load16(a_src, a_off[u] + 2u * k0, base + (uint32_t)((u * NT + 64 * wave) * 16));
#pragma unroll
    for (int u = 0; u < kBL; ++u)
      lds_load16(cbase, b_off[u] + k0 / 2, base + kABy + (uint32_t)((u * NT + 64 * wave) * 16));
    if constexpr (kChunkBy > 0) {
      if (chunked) {
        if (ks % kCkSteps == 0)
          lds_load16(sbase, ck_off + k0 / (NV ? 16 : 32),
                     c_lds + (uint32_t)(((ks / kCkSteps) & 1) * kChunkBy + 64 * wave * 16));
        return;
      }
    }
    if constexpr (NV) {
      lds_load4(sbase, nv_off + k0 / 16, base + kABy + kBBytes + (uint32_t)(64 * wave * 4));
      if constexpr (NT == 256)
        lds_load4(sbase, nv_off2 + k0 / 16,
                  base + kABy + kBBytes + (uint32_t)((256 + 64 * wave) * 4));
    } else if constexpr (PSC) {
      lds_load4(sbase, nv_off + k0 / 32, base + kABy + kBBytes + (uint32_t)(64 * wave * 4));
    }
  };
  // The tile's scales: rows r of the tile (gate/up: two runs of 128 rows,
  // down: one run of 256), srow bytes each, contiguous in the bank and in
  // LDS ([r][K / 32]); 4-byte pieces, srow is a multiple of 4. (Rows padded
  // to an odd word count, and the code swizzle of the MX kernel, measured
  // 2 % slower here.)
  auto load_scales = [&]() {
    const int pieces = kWRows * (int)srow / 4;
    for (int p0 = 64 * wave; p0 < pieces; p0 += NT) {
      const int p = min(p0 + lane, pieces - 1);
      const uint32_t b = 4u * (uint32_t)p;
      const uint32_t r = b / srow;
      lds_load4(sbase, wrow((int)r) * srow + (b - r * srow), s_lds + 4u * (uint32_t)p0);
    }
  };

  // A bucket of at most 16 rows: one row group, so the tile holds 16 x
  // rows (4 KB a step) and three stages of it fit in the same LDS, letting
  // the weight copies run two steps ahead of the MFMAs (such tiles are bound
  // by their copies, not by matrix work). Each wave converts its 64 weight
  // rows as in the 64-row tile and runs 4 MFMAs per sub-step.
  if constexpr (BM == 64) {
    if (bk.count <= 16) {
      constexpr int kSA = 16 * kBK * 2;          // A bytes per stage
      constexpr int kSS = kSA + kBBytes + kSBy;  // bytes per stage
      constexpr int kS3 = 3;                     // stages
      static_assert(kS3 * kSS + 2 * kChunkBy <= (int)sizeof(lds), "skinny stages exceed the LDS");
      // the waits below count 1 A copy and 4 B copies per stage, plus its scales
      static_assert(kBL == 4 && 16 * 16 == NT, "skinny stage copies per thread");
      const uint32_t ck3 = lds_base + kS3 * kSS;  // the two scale chunks
      auto issue_s = [&](int st, int ks) {
        const uint32_t base = lds_base + (uint32_t)(st * kSS);
        const uint32_t k0 = (uint32_t)(ks * kBK);
        lds_load16(a_src, a_off[0] + 2u * k0, base + (uint32_t)(64 * wave * 16));
#pragma unroll
        for (int u = 0; u < kBL; ++u)
          lds_load16(cbase, b_off[u] + k0 / 2, base + kSA + (uint32_t)((u * NT + 64 * wave) * 16));
        if (chunked) {
          if (ks % kCkSteps == 0)
            lds_load16(sbase, ck_off + k0 / (NV ? 16 : 32),
                       ck3 + (uint32_t)(((ks / kCkSteps) & 1) * kChunkBy + 64 * wave * 16));
        } else if constexpr (NV) {
          lds_load4(sbase, nv_off + k0 / 16, base + kSA + kBBytes + (uint32_t)(64 * wave * 4));
          lds_load4(sbase, nv_off2 + k0 / 16, base + kSA + kBBytes + (uint32_t)((256 + 64 * wave) * 4));
        } else {
          lds_load4(sbase, nv_off + k0 / 32, base + kSA + kBBytes + (uint32_t)(64 * wave * 4));
        }
      };
      // copies per thread of step ks's stage
      auto n_loads = [&](int ks) {
        return 1 + kBL + (chunked ? (ks % kCkSteps == 0 ? 1 : 0) : (NV ? 2 : 1));
      };
      f32x4_t as[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) as[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      auto compute_s = [&](int st, int st_k) {
        const char* sb = lds + st * kSS;
        const uint4* sa = reinterpret_cast<const uint4*>(sb);
        const uint4* sbk = reinterpret_cast<const uint4*>(sb + kSA);
        const uint16_t* ssn = reinterpret_cast<const uint16_t*>(sb + kSA + kBBytes);
        const uint8_t* ssp = reinterpret_cast<const uint8_t*>(sb + kSA + kBBytes);
        int nst = 4, sst = 4;
        if (chunked) {
          const char* ck = lds + kS3 * kSS + ((st_k / kCkSteps) & 1) * kChunkBy;
          ssn = reinterpret_cast<const uint16_t*>(ck + (st_k & 1) * 8);
          ssp = reinterpret_cast<const uint8_t*>(ck + (st_k & 3) * 4);
          nst = 8;
          sst = 16;
        }
        uint4 bc[4];
        float sc[4], sc2[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = frag_row<GU>(wn, j, c);
          bc[j] = sbk[r * 4 + (grp ^ ((r >> 2) & 3))];
          if constexpr (NV) {
            const f32x2_t f =
                __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(ssn[r * nst + grp], 1.0f, false);
            sc[j] = f.x;
            sc2[j] = f.y;
          } else {
            sc[j] = sc2[j] = e8m0_to_f32(ssp[r * sst + grp]);
          }
        }
        // A row c, K values 32 grp + 8 s: piece 4 grp + s
        Op<GU> bcur[4], bnext[4];
        uint4 acur = sa[c * 16 + ((4 * grp) ^ c)], anext = acur;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if constexpr (NV)
            bcur[j] = cvt8_nv<GU>(word_of(bc[j], 0), sc[j]);
          else
            bcur[j] = cvt8<GU>(word_of(bc[j], 0), sc[j]);
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          if (s < 3) {
            anext = sa[c * 16 + ((4 * grp + s + 1) ^ c)];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              if constexpr (NV)
                bnext[j] = cvt8_nv<GU>(word_of(bc[j], s + 1), s + 1 < 2 ? sc[j] : sc2[j]);
              else
                bnext[j] = cvt8<GU>(word_of(bc[j], s + 1), sc[j]);
            }
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) as[j] = mma<GU>(acur, bcur[j], as[j]);
          if (s < 3) {
            acur = anext;
#pragma unroll
            for (int q = 0; q < 4; ++q) bcur[q] = bnext[q];
          }
        }
      };
      // Stage ks lands while ks - 1 computes; at the top of step ks only
      // stage ks + 1's copies may still be in flight (loads complete in
      // order), then one barrier makes stage ks visible and frees the
      // buffer of step ks - 1 for ks + 2.
      const int steps_s = K / kBK;
      issue_s(0, 0);
      if (steps_s > 1) issue_s(1, 1);
      for (int ks = 0; ks < steps_s; ++ks) {
        const int n1 = ks + 1 < steps_s ? n_loads(ks + 1) : 0;
        if (n1 == 0)
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        else if (n1 == 5)
          asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
        else if (n1 == 6)
          asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
        else
          asm volatile("s_waitcnt vmcnt(7)" ::: "memory");
        __syncthreads();
        if (ks + 2 < steps_s) issue_s((ks + 2) % kS3, ks + 2);
        compute_s(ks % kS3, ks);
      }
      float mg = 1.0f, mu = 1.0f;
      if constexpr (NV) {
        if (bv.gscale) {
          mg = bv.gscale[bk.e * 3 + (GU ? 0 : 2)];
          mu = bv.gscale[bk.e * 3 + 1];
        }
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = 4 * grp + v;
        if (m >= bk.count) continue;
        if constexpr (GU) {
          _Float16* hr = g.h + (size_t)(bk.begin + m) * g.I + n0 + 32 * wn + c;
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            if constexpr (NV)
              hr[16 * j] = (_Float16)silu_mul(as[j][v] * mg, as[j + 2][v] * mu);
            else
              hr[16 * j] = (_Float16)silu_mul(as[j][v], as[j + 2][v]);
          }
        } else if (g.part == 2) {
          float ys[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) ys[j] = NV ? as[j][v] * mg : as[j][v];
          combine_row(g, m, n0 + 64 * wn + c, ys);
        } else {
          float* yr = (bk.shared ? g.y_sh + (size_t)m * g.H : g.y + (size_t)(bk.begin + m) * g.H) +
                      n0 + 64 * wn + c;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if constexpr (NV)
              yr[16 * j] = as[j][v] * mg;
            else
              yr[16 * j] = as[j][v];
          }
        }
      }
      return;
    }
  }

  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // rows of this wave beyond the bucket need no arithmetic
  const bool active = m0 + 64 * wm < bk.count;

  // One K step in four MFMA sub-steps, software pipelined: while the 16
  // MFMAs of sub-step s run, the A fragments of s + 1 are read from LDS and
  // its B fragments converted, into a second set of registers.
  auto compute = [&](int st, int st_k) {
    const char* sb = lds + st * kSt;
    const uint4* sa = reinterpret_cast<const uint4*>(sb);
    const uint4* sbk = reinterpret_cast<const uint4*>(sb + kABy);
    const uint8_t* ss = reinterpret_cast<const uint8_t*>(lds + kStages * kSt) +
                        (size_t)st_k * 4;  // this K step's 4 scale bytes of each row
    // this step's scale pair grp of row r (NVFP4): ssn[r * nst + grp]; its
    // scale byte grp of row r (MXFP4): ssp[r * sst + grp]
    const uint16_t* ssn = reinterpret_cast<const uint16_t*>(sb + kABy + kBBytes);
    const uint8_t* ssp = reinterpret_cast<const uint8_t*>(sb + kABy + kBBytes);
    int nst = 4, sst = 4;
    if constexpr (kChunkBy > 0) {
      if (chunked) {
        const char* ck = lds + kStages * kSt + ((st_k / kCkSteps) & 1) * kChunkBy;
        ssn = reinterpret_cast<const uint16_t*>(ck + (st_k & 1) * 8);
        ssp = reinterpret_cast<const uint8_t*>(ck + (st_k & 3) * 4);
        nst = 8;
        sst = 16;
      }
    }
    uint4 bc[4];
    float sc[4], sc2[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = frag_row<GU>(wn, j, c);
      bc[j] = sbk[r * 4 + (grp ^ ((r >> 2) & 3))];
      if constexpr (NV) {
        const f32x2_t f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(ssn[r * nst + grp], 1.0f, false);
        sc[j] = f.x;
        sc2[j] = f.y;
      } else if constexpr (PSC) {
        sc[j] = sc2[j] = e8m0_to_f32(ssp[r * sst + grp]);
      } else {
        sc[j] = sc2[j] = e8m0_to_f32(ss[r * srow + grp]);
      }
    }
    // A row 64 wm + 16 i + c, K values 32 grp + 8 s: piece 4 grp + s
    auto a_frag = [&](int i, int s) {
      return sa[(64 * wm + 16 * i + c) * 16 + ((4 * grp + s) ^ c)];
    };
    Op<GU> bcur[4], bnext[4];
    uint4 acur[4], anext[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) acur[i] = a_frag(i, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {  // sub-step 0
      if constexpr (NV)
        bcur[j] = cvt8_nv<GU>(word_of(bc[j], 0), sc[j]);
      else
        bcur[j] = cvt8<GU>(word_of(bc[j], 0), sc[j]);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s < 3) {
#pragma unroll
        for (int i = 0; i < 4; ++i) anext[i] = a_frag(i, s + 1);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if constexpr (NV)
            bnext[j] = cvt8_nv<GU>(word_of(bc[j], s + 1), s + 1 < 2 ? sc[j] : sc2[j]);
          else
            bnext[j] = cvt8<GU>(word_of(bc[j], s + 1), sc[j]);
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i][j] = mma<GU>(acur[i], bcur[j], acc[i][j]);
      if (s < 3) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acur[q] = anext[q];
          bcur[q] = bnext[q];
        }
      }
    }
  };

  // Pipeline: stage ks + 1 loads while step ks computes. Each step starts
  // with a full wait for this wave's loads and one barrier, which makes
  // stage ks visible to every wave and frees the other buffer (read at
  // step ks - 1) for ks + 1.
  const int steps = K / kBK;
  if constexpr (!PSC) load_scales();
  issue(0, 0);
  for (int ks = 0; ks < steps; ++ks) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (ks + 1 < steps) issue((ks + 1) % kStages, ks + 1);
    if (active) compute(ks % kStages, ks);
  }

  // D layout: lane (c, grp), element v -> row 4 grp + v, column c
  if (!active) return;
  float mg = 1.0f, mu = 1.0f;
  if constexpr (NV) {
    if (bv.gscale) {
      mg = bv.gscale[bk.e * 3 + (GU ? 0 : 2)];
      mu = bv.gscale[bk.e * 3 + 1];
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = m0 + 64 * wm + 16 * i + 4 * grp + v;
      if (m >= bk.count) continue;
      if constexpr (GU) {
        _Float16* hr = g.h + (size_t)(bk.begin + m) * g.I + n0 + 32 * wn + c;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          if constexpr (NV)
            hr[16 * j] = (_Float16)silu_mul(acc[i][j][v] * mg, acc[i][j + 2][v] * mu);
          else
            hr[16 * j] = (_Float16)silu_mul(acc[i][j][v], acc[i][j + 2][v]);
        }
      } else if (g.part == 2) {
        float ys[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) ys[j] = NV ? acc[i][j][v] * mg : acc[i][j][v];
        combine_row(g, m, n0 + 64 * wn + c, ys);
      } else {
        float* yr = (bk.shared ? g.y_sh + (size_t)m * g.H : g.y + (size_t)(bk.begin + m) * g.H) +
                    n0 + 64 * wn + c;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if constexpr (NV)
            yr[16 * j] = acc[i][j][v] * mg;
          else
            yr[16 * j] = acc[i][j][v];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// FP8 weights (E4M3, one E8M0 scale per 32 x 32 block; the checkpoint's
// dense format, used for an FP8 shared expert): gemm_kernel with a B
// operand of 128 bytes per weight row and K step. A weight row's K range
// [32 g, 32 g + 32) is pieces 2 g and 2 g + 1 of its row (piece p at slot
// p ^ act8_swz(r)); MFMA sub-step s takes bytes 8 s .. 8 s + 7 of those 32
// and converts them with the gfx950 scaled FP8 conversion (exact: E4M3
// times a power of two is representable in bf16, and in fp16 for scale
// exponents in [-15, 7]). The scales of the tile's 8 blocks of 32 weight
// rows over all of K take 8 x K / 32 bytes of LDS.
// ---------------------------------------------------------------------------

constexpr int kF8BBytes = kWRows * kBK;               // 32 KB of E4M3 per stage
constexpr int kF8StageBytes = kABytes + kF8BBytes;    // 64 KB
constexpr int kF8BLoads = kF8BBytes / 16 / kThreads;  // 4 per thread per stage
constexpr int kF8ScaleBytes = 8 * (8192 / 32);        // 2 KB

template <bool GU>
__device__ __forceinline__ Op<GU> cvt8_fp8(uint32_t w0, uint32_t w1, float sc) {
  if constexpr (GU) {
    const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, sc, false);
    const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, sc, true);
    const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, sc, false);
    const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, sc, true);
    return bf16x8_t{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
  } else {
    const f16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, sc, false);
    const f16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, sc, true);
    const f16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, sc, false);
    const f16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, sc, true);
    return f16x8_t{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
  }
}

template <bool GU>
__global__ __launch_bounds__(kThreads, 1) void gemm_fp8w_kernel(GemmArgs g) {
  __shared__ __align__(16) char lds[kStages * kF8StageBytes + kF8ScaleBytes];  // 130 KB
  constexpr int kBN = GU ? kWRows / 2 : kWRows;
  const int N = GU ? g.I : g.H;
  const int K = GU ? g.H : g.I;
  const int ncol = N / kBN;
  const int total = min(g.tile_count[GU ? 0 : 1], g.max_rb * ncol);
  const int per = (total + 7) / 8;
  const int slot = blockIdx.x >> 3;
  const int t = (blockIdx.x & 7) * per + slot;
  if (slot >= per || t >= total) return;
  const int nb = g.E + (g.has_shared ? 1 : 0);
  const Bucket bk = bucket_of(g, min(max(g.tile_b[GU ? 0 : 1][t], 0), nb - 1));
  const int mn = g.tile_mn[GU ? 0 : 1][t];
  const int m0 = (mn >> 8) * kBM;
  const int n0 = min(mn & 255, ncol - 1) * kBN;
  if (m0 < 0 || m0 >= bk.count) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3, c = lane & 15, grp = lane >> 4;
  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds;

  // A exactly as in gemm_kernel
  const void* a_src = GU ? static_cast<const void*>(g.x) : static_cast<const void*>(g.h);
  uint32_t a_off[kALoads];
  {
    const int piece = (tid & 15) ^ ((tid >> 4) & 15);
#pragma unroll
    for (int u = 0; u < kALoads; ++u) {
      const int m = min(m0 + 32 * u + (tid >> 4), bk.count - 1);
      int row;
      if (GU) {
        row = bk.shared ? m : (g.row_token ? g.row_token[bk.begin + m] : bk.begin + m);
        row = min(max(row, 0), g.T - 1);
      } else {
        row = bk.begin + m;
      }
      a_off[u] = ((uint32_t)row * (uint32_t)K + (uint32_t)(piece * 8)) * 2u;
    }
  }

  // B: thread tid fills slot (r = 64 u + tid / 8, slot tid % 8) with piece
  // (tid % 8) ^ act8_swz(r) of weight row r.
  const BankView bv = bk.shared ? g.shared : g.routed;
  const uint32_t srow = (uint32_t)K / 32;
  const size_t mat_rows = GU ? 2 * (size_t)g.I : (size_t)g.H;
  const uint8_t* wbase = (GU ? bv.gu_codes : bv.d_codes) + (size_t)bk.e * mat_rows * K;
  const uint8_t* sbase = (GU ? bv.gu_scales : bv.d_scales) + (size_t)bk.e * (mat_rows / 32) * srow;
  auto wrow = [&](int r) -> uint32_t {
    return GU ? (uint32_t)(r < 128 ? n0 + r : g.I + n0 + r - 128) : (uint32_t)(n0 + r);
  };
  uint32_t b_off[kF8BLoads];
#pragma unroll
  for (int u = 0; u < kF8BLoads; ++u) {
    const int r = 64 * u + (tid >> 3);
    b_off[u] = wrow(r) * (uint32_t)K + 16u * (uint32_t)((tid & 7) ^ act8_swz(r));
  }
  const uint32_t s_lds = lds_base + kStages * kF8StageBytes;

  auto issue = [&](int st, int ks) {
    const uint32_t base = lds_base + (uint32_t)(st * kF8StageBytes);
    const uint32_t k0 = (uint32_t)(ks * kBK);
#pragma unroll
    for (int u = 0; u < kALoads; ++u)
      lds_load16(a_src, a_off[u] + 2u * k0, base + (uint32_t)((u * kThreads + 64 * wave) * 16));
#pragma unroll
    for (int u = 0; u < kF8BLoads; ++u)
      lds_load16(wbase, b_off[u] + k0, base + kABytes + (uint32_t)((u * kThreads + 64 * wave) * 16));
  };
  // scales of the tile's 8 blocks of 32 weight rows, [block][K / 32]
  auto load_scales = [&]() {
    load_scale_rows(sbase, [&](int rb) { return (wrow(32 * rb) >> 5) * srow; }, 8, srow, srow,
                    s_lds, wave, lane, kThreads / 64);
  };

  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const bool active = m0 + 64 * wm < bk.count;

  auto compute = [&](int st, int st_k) {
    const char* sb = lds + st * kF8StageBytes;
    const uint4* sa = reinterpret_cast<const uint4*>(sb);
    const uint4* sbk = reinterpret_cast<const uint4*>(sb + kABytes);
    const uint8_t* ss = reinterpret_cast<const uint8_t*>(lds + kStages * kF8StageBytes) +
                        (size_t)st_k * 4 + grp;
    uint4 lo[4], hi[4];
    float sc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = frag_row<GU>(wn, j, c);
      const int sw = act8_swz(r);
      lo[j] = sbk[r * 8 + ((2 * grp) ^ sw)];
      hi[j] = sbk[r * 8 + ((2 * grp + 1) ^ sw)];
      sc[j] = e8m0_to_f32(ss[(r >> 5) * srow]);
    }
    auto a_frag = [&](int i, int s) {
      return sa[(64 * wm + 16 * i + c) * 16 + ((4 * grp + s) ^ c)];
    };
    auto b_sub = [&](int j, int s) -> Op<GU> {
      const uint4 v = s < 2 ? lo[j] : hi[j];
      return (s & 1) ? cvt8_fp8<GU>(v.z, v.w, sc[j]) : cvt8_fp8<GU>(v.x, v.y, sc[j]);
    };
    Op<GU> bcur[4], bnext[4];
    uint4 acur[4], anext[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) acur[i] = a_frag(i, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) bcur[j] = b_sub(j, 0);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s < 3) {
#pragma unroll
        for (int i = 0; i < 4; ++i) anext[i] = a_frag(i, s + 1);
#pragma unroll
        for (int j = 0; j < 4; ++j) bnext[j] = b_sub(j, s + 1);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i][j] = mma<GU>(acur[i], bcur[j], acc[i][j]);
      if (s < 3) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acur[q] = anext[q];
          bcur[q] = bnext[q];
        }
      }
    }
  };

  const int steps = K / kBK;
  load_scales();
  issue(0, 0);
  for (int ks = 0; ks < steps; ++ks) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (ks + 1 < steps) issue((ks + 1) % kStages, ks + 1);
    if (active) compute(ks % kStages, ks);
  }

  if (!active) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = m0 + 64 * wm + 16 * i + 4 * grp + v;
      if (m >= bk.count) continue;
      if constexpr (GU) {
        _Float16* hr = g.h + (size_t)(bk.begin + m) * g.I + n0 + 32 * wn + c;
#pragma unroll
        for (int j = 0; j < 2; ++j) hr[16 * j] = (_Float16)silu_mul(acc[i][j][v], acc[i][j + 2][v]);
      } else {
        float* yr = (bk.shared ? g.y_sh + (size_t)m * g.H : g.y + (size_t)(bk.begin + m) * g.H) +
                    n0 + 64 * wn + c;
#pragma unroll
        for (int j = 0; j < 4; ++j) yr[16 * j] = acc[i][j][v];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// MXFP8-activation mode: both operands microscaled, on the gfx950 scaled
// MFMA (v_mfma_scale_f32_16x16x128_f8f6f4: A = E4M3 activations, B = the
// bank's E2M1 codes as stored, each with one E8M0 scale per 32 K). The
// weights need no conversion at all; the activations are rounded to MXFP8
// once (x before the gate/up GEMM, h in its epilogue), which is the one
// approximation of this mode.
//
// Operand layout of the 16x16x128 instruction (lane l, c = l % 16,
// g = l / 16): A row c, bytes 0..15 = K 16 g .. 16 g + 15 and bytes 16..31
// = K 64 + 16 g .. 64 + 16 g + 15; B column c, 16 bytes = K 32 g .. 32 g +
// 31 in the bank's nibble order; the scale operand of lane l is that of row
// (column) c over K block g; D as for the other MFMAs (element v -> row
// 4 g + v, column c).
//
// Tile and pipeline as in gemm_kernel, with A at one byte per element:
// stage = 128 rows x 128 B of E4M3 (piece p of row r at slot
// p ^ act8_swz(r)) + 256 weight rows x 64 B of codes. The E8M0 scales of
// both operands over all of K sit in LDS for the whole tile.
// ---------------------------------------------------------------------------

constexpr int kMxABytes = kBM * kBK;                   // 16 KB of E4M3 per stage
constexpr int kMxStageBytes = kMxABytes + kBBytes;     // 32 KB
constexpr int kMxALoads = kMxABytes / 16 / kThreads;   // 2 per thread per stage
constexpr int kMxLds = 160 * 1024;                     // stages + both operands' scales
constexpr int kMxIssueLoads = kMxALoads + kBLoads;     // loads per thread per stage
static_assert(kMxIssueLoads == 4, "the pipeline waits below count 4 loads per stage");

// Pipeline depth of the MX GEMM at reduction length K: as many 32 KB stages
// (up to 4) as fit beside the tile's scales (384 rows at the padded stride).
inline int mx_stages(int K) {
  const int sr = K / 32;
  const int stride = ((sr / 4) % 2 == 0 && sr < 256) ? sr + 4 : sr;
  const int free = kMxLds - (kWRows + kBM) * stride;
  return free >= 4 * kMxStageBytes ? 4 : free >= 3 * kMxStageBytes ? 3 : 2;
}

typedef int v8i_t __attribute__((ext_vector_type(8)));

// E8M0 exponent of a block whose largest magnitude is `amax` (OCP MX: the
// binade of amax minus 8, the largest E4M3 exponent, clamped to [-127, 127];
// an all-zero block takes -127).
__device__ __forceinline__ int mx_block_exp(float amax) {
  const uint32_t b = __float_as_uint(amax);
  const int ef = (int)(b >> 23);
  const uint32_t mant = b & 0x7fffffu;
  const int fl = ef ? ef - 127 : (31 - __builtin_clz(mant | 1u)) - 149;
  return amax == 0.0f ? -127 : min(max(fl - 8, -127), 127);
}

// |v| / 2^se (0 <= q < 512) -> E4M3 magnitude code: nearest, ties to even,
// clamped to 448 (0x7E). Below 2^-6 the steps are 2^-9 and the step count is
// the code (8 steps = 2^-6 = code 0x08).
__device__ __forceinline__ uint32_t e4m3_mag_code(float q) {
  if (q < 0x1p-6f) return (uint32_t)rintf(q * 512.0f);
  uint32_t b = __float_as_uint(q);
  b += 0x7ffffu + ((b >> 20) & 1u);
  const uint32_t code = (((b >> 23) - 120u) << 3) | ((b >> 20) & 7u);
  return min(code, 0x7eu);
}

// x [n_blocks * 32] bf16 -> E4M3 codes + one E8M0 byte per 32 (one thread
// per block of 32).
__global__ __launch_bounds__(256) void quant_mxfp8_kernel(const uint16_t* __restrict__ x,
                                                          long n_blocks, uint8_t* __restrict__ q,
                                                          uint8_t* __restrict__ s) {
  const long b = (long)blockIdx.x * 256 + threadIdx.x;
  if (b >= n_blocks) return;
  const uint4* src = reinterpret_cast<const uint4*>(x + b * 32);
  uint32_t w[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 v = src[i];
    w[4 * i + 0] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
  }
  // magnitudes of bf16 values order like their bit patterns without the sign
  uint32_t am = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) am = max(am, max(w[i] & 0x7fffu, (w[i] >> 16) & 0x7fffu));
  const int se = mx_block_exp(__uint_as_float(am << 16));
  uint32_t out[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t bits = (w[2 * i + (j >> 1)] >> (16 * (j & 1))) & 0xffffu;
      const float mag = __uint_as_float((bits & 0x7fffu) << 16);
      const uint32_t code = e4m3_mag_code(ldexpf(mag, -se)) | ((bits >> 8) & 0x80u);
      word |= code << (8 * j);
    }
    out[i] = word;
  }
  uint4* dst = reinterpret_cast<uint4*>(q + b * 32);
  dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
  dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
  s[b] = (uint8_t)(se + 127);
}

// PS: the scales travel with each of two stages (4 bytes per weight row and
// activation row per K step, 1.5 KB), so a workgroup takes 67 KB of LDS and
// two share a CU.
constexpr int kMxPsStage = kMxStageBytes + (kWRows + kBM) * 4;

template <bool GU, int S, bool PS>
__global__ __launch_bounds__(kThreads, PS ? 2 : 1) void gemm_mx_kernel(GemmArgs g) {
  static_assert(!PS || S == 2, "per-stage scales use two stages");
  __shared__ __align__(16) char lds[PS ? 2 * kMxPsStage : kMxLds];
  constexpr int kSt = PS ? kMxPsStage : kMxStageBytes;
  constexpr int kBN = GU ? kWRows / 2 : kWRows;
  const int N = GU ? g.I : g.H;
  const int K = GU ? g.H : g.I;
  const int ncol = N / kBN;
  const int total = min(g.tile_count[GU ? 0 : 1], g.max_rb * ncol);
  const int per = (total + 7) / 8;
  const int slot = blockIdx.x >> 3;
  const int t = (blockIdx.x & 7) * per + slot;
  if (slot >= per || t >= total) return;
  const int nb = g.E + (g.has_shared ? 1 : 0);
  const Bucket bk = bucket_of(g, min(max(g.tile_b[GU ? 0 : 1][t], 0), nb - 1));
  const int mn = g.tile_mn[GU ? 0 : 1][t];
  const int m0 = (mn >> 8) * kBM;
  const int n0 = min(mn & 255, ncol - 1) * kBN;
  if (m0 < 0 || m0 >= bk.count) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3, c = lane & 15, grp = lane >> 4;
  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds;
  const uint32_t srow = (uint32_t)K / 32;

  // activation row of tile row m (clamped into the bucket)
  auto act_row = [&](int m) -> int {
    m = min(m0 + m, bk.count - 1);
    if (GU) {
      const int row = bk.shared ? m : (g.row_token ? g.row_token[bk.begin + m] : bk.begin + m);
      return min(max(row, 0), g.T - 1);
    }
    return bk.begin + m;
  };

  // A: thread tid fills slot (row 64 u + tid / 8, slot tid % 8), which holds
  // K piece (tid % 8) ^ ((row / 2) % 8) of that row.
  const uint8_t* a_src = GU ? g.xq : g.hq;
  const uint8_t* as_src = GU ? g.xs : g.hs;
  uint32_t a_off[kMxALoads];
#pragma unroll
  for (int u = 0; u < kMxALoads; ++u) {
    const int r = 64 * u + (tid >> 3);
    const int piece = (tid & 7) ^ act8_swz(r);
    a_off[u] = (uint32_t)act_row(r) * (uint32_t)K + (uint32_t)(piece * 16);
  }

  const BankView bv = bk.shared ? g.shared : g.routed;
  const uint32_t crow = (uint32_t)K / 2;
  const size_t mat_rows = GU ? 2 * (size_t)g.I : (size_t)g.H;
  const uint8_t* cbase = (GU ? bv.gu_codes : bv.d_codes) + (size_t)bk.e * mat_rows * crow;
  const uint8_t* sbase = (GU ? bv.gu_scales : bv.d_scales) + (size_t)bk.e * mat_rows * srow;
  auto wrow = [&](int r) -> uint32_t {
    return GU ? (uint32_t)(r < 128 ? n0 + r : g.I + n0 + r - 128) : (uint32_t)(n0 + r);
  };
  uint32_t b_off[kBLoads];
#pragma unroll
  for (int u = 0; u < kBLoads; ++u) {
    const int r = 128 * u + (tid >> 2);
    b_off[u] = wrow(r) * crow + 16u * (uint32_t)((tid & 3) ^ code_swz(r));
  }
  const uint32_t sstride = scale_stride(srow);
  if (!PS && S * kMxStageBytes + (kWRows + kBM) * (int)sstride > kMxLds) return;  // launcher picks S
  const uint32_t bs_lds = lds_base + S * kMxStageBytes;
  const uint32_t as_lds = bs_lds + kWRows * sstride;

  // PS: thread tid < 256 copies weight row tid's 4 scale bytes of the step,
  // 256 <= tid < 384 activation row tid - 256's
  uint32_t ps_off = 0;
  if constexpr (PS) {
    if (tid < kWRows)
      ps_off = wrow(tid) * srow;
    else if (tid < kWRows + kBM) {
      ps_off = (uint32_t)act_row(tid - kWRows) * srow;
    }
  }
  auto issue = [&](int st, int ks) {
    const uint32_t base = lds_base + (uint32_t)(st * kSt);
    const uint32_t k0 = (uint32_t)(ks * kBK);
#pragma unroll
    for (int u = 0; u < kMxALoads; ++u)
      lds_load16(a_src, a_off[u] + k0, base + (uint32_t)((u * kThreads + 64 * wave) * 16));
#pragma unroll
    for (int u = 0; u < kBLoads; ++u)
      lds_load16(cbase, b_off[u] + k0 / 2,
                 base + kMxABytes + (uint32_t)((u * kThreads + 64 * wave) * 16));
    if constexpr (PS) {
      if (wave < (kWRows + kBM) / 64)
        lds_load4(wave < kWRows / 64 ? sbase : as_src, ps_off + (uint32_t)(ks * 4),
                  base + kMxStageBytes + (uint32_t)(64 * wave * 4));
    }
  };
  // Scales of the tile over all of K, [row][K / 32] at LDS row stride
  // sstride: the 256 weight rows', then the 128 activation rows'.
  auto load_scales = [&]() {
    load_scale_rows(sbase, [&](int r) { return wrow(r) * srow; }, kWRows, srow, sstride, bs_lds,
                    wave, lane, kThreads / 64);
    load_scale_rows(as_src, [&](int r) { return (uint32_t)act_row(r) * srow; }, kBM, srow,
                    sstride, as_lds, wave, lane, kThreads / 64);
  };

  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const bool active = m0 + 64 * wm < bk.count;

  // One K step of 128: 16 scaled MFMAs per wave (4 row x 4 column fragments).
  auto compute = [&](int st, int ks) {
    const char* sb = lds + st * kSt;
    const uint4* sa = reinterpret_cast<const uint4*>(sb);
    const uint4* sbk = reinterpret_cast<const uint4*>(sb + kMxABytes);
    const uint8_t* bsc = PS ? reinterpret_cast<const uint8_t*>(sb + kMxStageBytes) + grp
                            : reinterpret_cast<const uint8_t*>(lds + S * kMxStageBytes) + ks * 4 + grp;
    const uint8_t* asc = PS ? bsc + kWRows * 4 : bsc + kWRows * sstride;
    const uint32_t rs = PS ? 4u : sstride;  // scale row stride in LDS
    v8i_t b[4];
    int sbv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = frag_row<GU>(wn, j, c);
      const uint4 q = sbk[r * 4 + (grp ^ code_swz(r))];
      b[j] = v8i_t{(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
      sbv[j] = bsc[r * rs];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 64 * wm + 16 * i + c;
      const int sw = act8_swz(r);
      const uint4 lo = sa[r * 8 + (grp ^ sw)];
      const uint4 hi = sa[r * 8 + ((4 + grp) ^ sw)];
      const v8i_t a = v8i_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                            (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      const int sav = asc[r * rs];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b[j], acc[i][j], 0, 4, 0,
                                                                      sav, 0, sbv[j]);
    }
  };

  // S-stage pipeline: stages ks + 1 .. ks + S - 2 stay in flight while step
  // ks computes. At the top of step ks the wait leaves only the loads of the
  // later stages already issued outstanding (vector loads complete in
  // order), so stage ks has landed; the barrier makes it visible to every
  // wave and frees the buffer of step ks - 1 for stage ks + S - 1.
  const int steps = K / kBK;
  if constexpr (!PS) load_scales();
#pragma unroll
  for (int st = 0; st < S - 1; ++st)
    if (st < steps) issue(st, st);
  for (int ks = 0; ks < steps; ++ks) {
    if (steps - 1 - ks >= S - 2) {
      if constexpr (S == 4)
        asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
      else if constexpr (S == 3)
        asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
      else
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    } else if (S == 4 && steps - 1 - ks == 1) {
      asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __syncthreads();
    if (ks + S - 1 < steps) issue((ks + S - 1) % S, ks + S - 1);
    if (active) compute(ks % S, ks);
  }

  if (!active) return;
  if constexpr (GU) {
    // h = silu(g) * u for 32 consecutive columns per row (two fragments of
    // the 16 lanes of a lane group), rounded to one MXFP8 block.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = m0 + 64 * wm + 16 * i + 4 * grp + v;
        const float h0 = silu_mul(acc[i][0][v], acc[i][2][v]);
        const float h1 = silu_mul(acc[i][1][v], acc[i][3][v]);
        float am = fmaxf(fabsf(h0), fabsf(h1));
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) am = fmaxf(am, __shfl_xor(am, o, kWave));
        const int se = mx_block_exp(am);
        const uint32_t c0 = e4m3_mag_code(ldexpf(fabsf(h0), -se)) | ((__float_as_uint(h0) >> 24) & 0x80u);
        const uint32_t c1 = e4m3_mag_code(ldexpf(fabsf(h1), -se)) | ((__float_as_uint(h1) >> 24) & 0x80u);
        if (m < bk.count) {
          uint8_t* hr = g.hq + (size_t)(bk.begin + m) * g.I + n0 + 32 * wn + c;
          hr[0] = (uint8_t)c0;
          hr[16] = (uint8_t)c1;
          if (c == 0) g.hs[(size_t)(bk.begin + m) * (g.I / 32) + (n0 + 32 * wn) / 32] = (uint8_t)(se + 127);
        }
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = m0 + 64 * wm + 16 * i + 4 * grp + v;
        if (m >= bk.count) continue;
        float* yr = (bk.shared ? g.y_sh + (size_t)m * g.H : g.y + (size_t)(bk.begin + m) * g.H) +
                    n0 + 64 * wn + c;
#pragma unroll
        for (int j = 0; j < 4; ++j) yr[16 * j] = acc[i][j][v];
      }
    }
  }
}

struct GemmLayout {
  _Float16* h;
  int32_t* tiles;
  int max_rb, ncol_gu, ncol_dn;
  size_t bytes;
};

GemmLayout gemm_layout(void* ws, int T, int H, int I, int E, int R, bool shared) {
  GemmLayout L;
  const size_t rows = (size_t)R + (shared ? T : 0);
  L.max_rb = (R + 63) / 64 + E + (shared ? (T + 63) / 64 + 1 : 0);  // blocks of >= 64 rows
  L.ncol_gu = I / (kWRows / 2);
  L.ncol_dn = H / kWRows;
  const size_t hb = (rows * I * sizeof(_Float16) + 255) & ~(size_t)255;
  const size_t nt = 2 * (size_t)L.max_rb * (L.ncol_gu + L.ncol_dn) + 3;
  char* w = static_cast<char*>(ws);
  L.h = reinterpret_cast<_Float16*>(w);
  L.tiles = reinterpret_cast<int32_t*>(w ? w + hb : nullptr);
  L.bytes = hb + ((nt * sizeof(int32_t) + 255) & ~(size_t)255);
  return L;
}

struct MxLayout {
  uint8_t *xq, *xs, *hq, *hs;
  int32_t* tiles;
  int max_rb, ncol_gu, ncol_dn;
  size_t bytes;
};

MxLayout mx_layout(void* ws, int T, int H, int I, int E, int R, bool shared) {
  auto al = [](size_t v) { return (v + 255) & ~(size_t)255; };
  MxLayout L;
  const size_t rows = (size_t)R + (shared ? T : 0);
  L.max_rb = (R + 63) / 64 + E + (shared ? (T + 63) / 64 + 1 : 0);  // blocks of >= 64 rows
  L.ncol_gu = I / (kWRows / 2);
  L.ncol_dn = H / kWRows;
  const size_t nt = 2 * (size_t)L.max_rb * (L.ncol_gu + L.ncol_dn) + 3;
  const size_t sz[5] = {al((size_t)T * H), al((size_t)T * H / 32), al(rows * I), al(rows * I / 32),
                        al(nt * sizeof(int32_t))};
  char* w = static_cast<char*>(ws);
  size_t off = 0;
  char* part[5];
  for (int i = 0; i < 5; ++i) {
    part[i] = w ? w + off : nullptr;
    off += sz[i];
  }
  L.xq = reinterpret_cast<uint8_t*>(part[0]);
  L.xs = reinterpret_cast<uint8_t*>(part[1]);
  L.hq = reinterpret_cast<uint8_t*>(part[2]);
  L.hs = reinterpret_cast<uint8_t*>(part[3]);
  L.tiles = reinterpret_cast<int32_t*>(part[4]);
  L.bytes = off;
  return L;
}

}  // namespace

bool gemm_mx_supported(int T, int H, int I, int R, bool shared) {
  // 32-bit byte offsets of the activation rows; scales of a tile fit LDS
  const size_t rows = (size_t)R + (shared ? T : 0);
  return H % kBK == 0 && I % kBK == 0 && I % (kWRows / 2) == 0 && H % kWRows == 0 && H <= 8192 &&
         I <= 8192 && (size_t)T * H < (1ull << 31) && rows * I < (1ull << 31);
}

size_t gemm_mx_ws_bytes(int T, int H, int I, int E, int R, bool shared) {
  return mx_layout(nullptr, T, H, I, E, R, shared).bytes;
}

void launch_quant_mxfp8(const uint16_t* x, long n_blocks, uint8_t* q, uint8_t* s, hipStream_t st) {
  const long grid = (n_blocks + 255) / 256;
  launch("quant_mxfp8_kernel", quant_mxfp8_kernel, dim3((unsigned)grid), dim3(256), 0, st, x,
         n_blocks, q, s);
}

void launch_expert_gemm_mx(const FfnProblem& p, void* ws, hipStream_t s) {
  const int E = p.offsets ? p.routed.E : 1;
  const MxLayout L = mx_layout(ws, p.T, p.H, p.I, E, p.R, p.has_shared);
  GemmArgs g{};
  g.x = p.x;
  g.T = p.T;
  g.H = p.H;
  g.I = p.I;
  g.E = E;
  g.R = p.R;
  g.routed = p.routed;
  g.shared = p.shared;
  g.has_shared = p.has_shared;
  g.offsets = p.offsets;
  g.row_token = p.row_token;
  const size_t n_gu = (size_t)L.max_rb * L.ncol_gu, n_dn = (size_t)L.max_rb * L.ncol_dn;
  g.tile_b[0] = L.tiles;
  g.tile_mn[0] = L.tiles + n_gu;
  g.tile_b[1] = L.tiles + 2 * n_gu;
  g.tile_mn[1] = L.tiles + 2 * n_gu + n_dn;
  g.tile_count = L.tiles + 2 * (n_gu + n_dn);
  g.max_rb = L.max_rb;
  g.y = p.y;
  g.y_sh = p.y_sh;
  g.xq = L.xq;
  g.xs = L.xs;
  g.hq = L.hq;
  g.hs = L.hs;
  g.bm = kBM;  // these kernels tile 128 rows
  launch("gemm_plan_kernel", gemm_plan_kernel, dim3(kPlanBlocks), dim3(1024), 0, s, g);
  launch_quant_mxfp8(p.x, (long)p.T * p.H / 32, L.xq, L.xs, s);
  const int grid_gu = (int)((n_gu + 7) / 8 * 8), grid_dn = (int)((n_dn + 7) / 8 * 8);
  // gate/up: the deepest pipeline that fits beside the full-K scales (3
  // stages at K = 5120); down: two stages with per-stage scales, two
  // workgroups a CU. Measured at 16k tokens: gate/up 3.41 ms against 3.49 ms
  // with per-stage scales; down 1.74 ms against 1.85 ms with 4 stages.
  const int s_gu = mx_stages(p.H);
  auto gu = s_gu == 4 ? gemm_mx_kernel<true, 4, false> : s_gu == 3 ? gemm_mx_kernel<true, 3, false>
                                                                    : gemm_mx_kernel<true, 2, false>;
  auto dn = gemm_mx_kernel<false, 2, true>;
  launch("gemm_mx_gateup_kernel", gu, dim3(grid_gu), dim3(kThreads), 0, s, g);
  launch("gemm_mx_down_kernel", dn, dim3(grid_dn), dim3(kThreads), 0, s, g);
}

size_t fp8_gemm_ws_bytes(int T, int H, int I) {
  return gemm_layout(nullptr, T, H, I, 0, 0, true).bytes;
}

// The FP8 expert over all T rows (row t = token t) as the one bucket of the
// grouped GEMM: no routed experts, the shared slot holds the FP8 bank.
void launch_fp8_gemm(const Fp8Ffn& p, void* ws, hipStream_t s) {
  const GemmLayout L = gemm_layout(ws, p.T, p.H, p.I, 0, 0, true);
  GemmArgs g{};
  g.x = p.x;
  g.T = p.T;
  g.H = p.H;
  g.I = p.I;
  g.E = 0;
  g.R = 0;
  g.shared = BankView{p.gu_w, p.gu_s, p.d_w, p.d_s, 1};
  g.routed = g.shared;
  g.has_shared = 1;
  const size_t n_gu = (size_t)L.max_rb * L.ncol_gu, n_dn = (size_t)L.max_rb * L.ncol_dn;
  g.tile_b[0] = L.tiles;
  g.tile_mn[0] = L.tiles + n_gu;
  g.tile_b[1] = L.tiles + 2 * n_gu;
  g.tile_mn[1] = L.tiles + 2 * n_gu + n_dn;
  g.tile_count = L.tiles + 2 * (n_gu + n_dn);
  g.max_rb = L.max_rb;
  g.h = L.h;
  g.y_sh = p.y;
  g.bm = kBM;  // these kernels tile 128 rows
  launch("gemm_plan_kernel", gemm_plan_kernel, dim3(kPlanBlocks), dim3(1024), 0, s, g);
  const int grid_gu = (int)((n_gu + 7) / 8 * 8), grid_dn = (int)((n_dn + 7) / 8 * 8);
  launch("gemm_fp8w_gateup_kernel", gemm_fp8w_kernel<true>, dim3(grid_gu), dim3(kThreads), 0, s, g);
  launch("gemm_fp8w_down_kernel", gemm_fp8w_kernel<false>, dim3(grid_dn), dim3(kThreads), 0, s, g);
}

bool gemm_supported(int T, int H, int I, int R, bool shared) {
  // 32-bit byte offsets of the activation rows
  const size_t rows = (size_t)R + (shared ? T : 0);
  return H % kBK == 0 && I % kBK == 0 && I % (kWRows / 2) == 0 && H % kWRows == 0 &&
         (size_t)T * H * 2 < (1ull << 31) && rows * I * 2 < (1ull << 31);
}

size_t gemm_ws_bytes(int T, int H, int I, int E, int R, bool shared) {
  return gemm_layout(nullptr, T, H, I, E, R, shared).bytes;
}

bool launch_expert_gemm(const FfnProblem& p, void* ws, hipStream_t s) {
  const int E = p.offsets ? p.routed.E : 1;
  const GemmLayout L = gemm_layout(ws, p.T, p.H, p.I, E, p.R, p.has_shared);
  GemmArgs g{};
  g.x = p.x;
  g.T = p.T;
  g.H = p.H;
  g.I = p.I;
  g.E = E;
  g.R = p.R;
  g.routed = p.routed;
  g.shared = p.shared;
  g.has_shared = p.has_shared;
  g.offsets = p.offsets;
  g.row_token = p.row_token;
  const size_t n_gu = (size_t)L.max_rb * L.ncol_gu, n_dn = (size_t)L.max_rb * L.ncol_dn;
  g.tile_b[0] = L.tiles;
  g.tile_mn[0] = L.tiles + n_gu;
  g.tile_b[1] = L.tiles + 2 * n_gu;
  g.tile_mn[1] = L.tiles + 2 * n_gu + n_dn;
  g.tile_count = L.tiles + 2 * (n_gu + n_dn);
  g.max_rb = L.max_rb;
  g.h = L.h;
  g.y = p.y;
  g.y_sh = p.y_sh;
  g.bm = 64;
  // The shared expert's down tiles combine the tokens where they are
  // enough to fill the GPU a few times over (at least 2048 tiles: 6.5k
  // tokens at H = 5120). Measured: 16k tokens 8.52-8.55 ms against
  // 8.65-8.70 ms with the combine launch; 2k tokens (640 such tiles) 1.91
  // against 1.90 ms.
  const bool fuse = p.out != nullptr && p.has_shared &&
                    (size_t)((p.T + 63) / 64) * L.ncol_dn >= 2048;
  if (fuse) {
    g.inv_row = p.inv_row;
    g.topk_w = p.topk_w;
    g.k = p.k;
    g.out = p.out;
  }
  launch("gemm_plan_kernel", gemm_plan_kernel, dim3(kPlanBlocks), dim3(1024), 0, s, g);
  // grids: every tile the lists can hold, rounded up to the 8 XCDs
  const int grid_gu = (int)((n_gu + 7) / 8 * 8), grid_dn = (int)((n_dn + 7) / 8 * 8);
  const bool nv = p.routed.codec == kCodecNvfp4;
  auto gu = nv ? gemm_kernel<true, true, 64> : gemm_kernel<true, false, 64>;
  auto dn = nv ? gemm_kernel<false, true, 64> : gemm_kernel<false, false, 64>;
  launch("gemm_gateup_kernel", gu, dim3(grid_gu), dim3(256), 0, s, g);
  if (!fuse) {
    launch("gemm_down_kernel", dn, dim3(grid_dn), dim3(256), 0, s, g);
    return false;
  }
  // the routed buckets' down tiles, then the shared expert's, which combine
  // each token with the routed rows now in y
  g.part = 1;
  launch("gemm_down_kernel", dn, dim3(grid_dn), dim3(256), 0, s, g);
  g.part = 2;
  const int grid_sh = (int)((((size_t)(p.T + 63) / 64 + 1) * L.ncol_dn + 7) / 8 * 8);
  launch("gemm_down_combine_kernel", dn, dim3(grid_sh), dim3(256), 0, s, g);
  return true;
}

}  // namespace moe
