// Shared device-side definitions of the self-speculative round engine (gfx950).
//
// Numerics contract (holds for every kernel here): the value computed for one
// row never depends on how many rows share the launch, on the row's slot in
// the window, or on how work is split across workgroups.  Reductions run in a
// fixed order over fixed structures (per-wave K slices in GEMMs, 64-key
// position chunks in attention, vocabulary tiles in the argmax); no
// floating-point atomics are used.  Consequently the verify rows of a round
// reproduce an AR step at the same position bit for bit, which is what makes
// greedy self-speculative output identical to greedy AR output on the GPU as
// it is in exact arithmetic (GravityOCR review, Appendix B.3).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ssb_limits.h"

namespace ssb {

typedef uint16_t bf16_t;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

constexpr int kWave = 64;
constexpr int kThreads = 256;      // 4 waves per workgroup
constexpr float kLog2e = 1.4426950408889634f;   // exp(x) = exp2(x * log2(e))

__device__ __forceinline__ float bf2f(bf16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ bf16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_t)0x7fc0;  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);                               // round to nearest even
  return (bf16_t)(u >> 16);
}

// Storage-type traits of the weights.  A "fragment" is the 16 bytes one lane feeds to the
// matrix core per step: 8 16-bit or 4 f32 values along K.
template <typename T> struct Ty;
template <> struct Ty<bf16_t> {
  static constexpr int kStepK = 32;   // K covered by one 16-byte-per-lane step
  static constexpr int kPerFrag = 8;
  static __device__ __forceinline__ float to_f(bf16_t v) { return bf2f(v); }
  static __device__ __forceinline__ bf16_t from_f(float v) { return f2bf(v); }
};
template <> struct Ty<float> {
  static constexpr int kStepK = 16;
  static constexpr int kPerFrag = 4;
  static __device__ __forceinline__ float to_f(float v) { return v; }
  static __device__ __forceinline__ float from_f(float v) { return v; }
};

// Activations of a model whose weights are bf16 are stored as IEEE fp16 in the same 16 bits:
// GEMM inputs, q, the KV cache, attention probabilities and outputs, SwiGLU outputs.  fp16 keeps
// 11 significant bits against bf16's 8, so each rounding of an activation costs 8x less; the
// 24-layer decoder then stays within a few 1e-3 of exact arithmetic in its logits, where bf16
// activations (and a bf16 KV cache) had drifted to about 6e-2.  The range condition is that
// every activation stays below 65504 in magnitude; an overflow becomes inf and then NaN logits,
// which the engine reports.  Weights stay bf16 in memory and are widened to fp16 in registers
// right before the matrix core (exact for |w| >= 2^-17 and |w| < 65504).  f32 models keep f32
// activations.
// The empty asm materializes f as an fp32 register value: without it the compiler may fuse a
// preceding multiply with the conversion (v_fma_mixlo_f16, one rounding of the exact product)
// in one kernel and not in another, and rows would no longer be bit-identical across kernels.
__device__ __forceinline__ uint16_t f2h(float f) {
  asm("" : "+v"(f));
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}
__device__ __forceinline__ float h2f(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }
template <typename T> struct Act;
template <> struct Act<bf16_t> {
  static __device__ __forceinline__ float to_f(uint16_t v) { return h2f(v); }
  static __device__ __forceinline__ uint16_t from_f(float v) { return f2h(v); }
};
template <> struct Act<float> {
  static __device__ __forceinline__ float to_f(float v) { return v; }
  static __device__ __forceinline__ float from_f(float v) { return v; }
};

typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
// Two bf16 values (low half first) widened to two fp16 values, packed the same way.
__device__ __forceinline__ uint32_t bf2_to_h2(uint32_t w) {
  typedef _Float16 h2v __attribute__((ext_vector_type(2)));
  typedef float f2v __attribute__((ext_vector_type(2)));
  const f2v f = {__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u)};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, h2v));
}
__device__ __forceinline__ uint4 bf8_to_h8(uint4 w) {
  return make_uint4(bf2_to_h2(w.x), bf2_to_h2(w.y), bf2_to_h2(w.z), bf2_to_h2(w.w));
}

// One 16x16 output tile step: acc[n][m] += sum_k A[n][k] * B[k][m].
// Lane l supplies A row (l % 16) and B column (l % 16), and the K values
// [kStepK/4 * (l/16), kStepK/4 * (l/16 + 1)) of the step; A and B use the
// same lane->K map, so any fixed K permutation inside a step is harmless.
// Result layout: lane l, element i holds acc[4*(l/16) + i][l % 16].
// mma_aa: both operands are activations (fp16 for a bf16 model).
__device__ __forceinline__ void mma_aa(f32x4_t& acc, uint4 a, uint4 b, bf16_t) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), acc,
                                               0, 0, 0);
}
__device__ __forceinline__ void mma_aa(f32x4_t& acc, uint4 a, uint4 b, float) {
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
}
// mma_wa: A is a packed weight fragment (fp16 for a bf16 model: converted once when packed), B an
// activation fragment.
__device__ __forceinline__ void mma_wa(f32x4_t& acc, uint4 w, uint4 x, bf16_t) { mma_aa(acc, w, x, bf16_t()); }
__device__ __forceinline__ void mma_wa(f32x4_t& acc, uint4 w, uint4 x, float) { mma_aa(acc, w, x, float()); }

// Kernel timing stamps of one launch (measurement only), on the device's real-time counter:
// word 0 is the start of workgroup 0 (dispatched first), word 1 + w % kStampWgs the end of
// workgroup w (grids of more workgroups share words; the last store of a word is close to the
// latest end).  Plain stores to distinct words: atomics from hundreds of workgroups finishing
// together would queue on one address and slow the very kernel being timed.  Slots are not reset
// between launches: the host keeps the end words at or after the launch's own start.  A null
// pointer disables the stamps.
constexpr int kStampWgs = 2047;
struct ProfStamp { unsigned long long t[1 + kStampWgs]; };
__device__ __forceinline__ int stamp_wg() {
  return (int)(blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z));
}
__device__ __forceinline__ void stamp_begin(ProfStamp* s) {
  if (s && threadIdx.x == 0 && stamp_wg() == 0) s->t[0] = __builtin_amdgcn_s_memrealtime();
}
// Every thread of the workgroup calls it at the kernel's end (s is uniform): once each thread's
// memory operations have completed, one thread records the time.
__device__ __forceinline__ void stamp_end(ProfStamp* s) {
  if (!s) return;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const int w = stamp_wg();
  if (threadIdx.x == 0) s->t[1 + w % kStampWgs] = __builtin_amdgcn_s_memrealtime();
}

// Element offset of one K or V value in the paged KV pool [layer][page][K|V][kv head][block].  A K
// block is token-major ([16 tokens][hd]: a key row is contiguous, the operand layout of S = K q);
// a V block is dim-major ([hd][16 tokens]: consecutive tokens of one dimension are contiguous, the
// operand layout of V^T in the P V product, so it loads without a transpose).
__host__ __device__ __forceinline__ size_t kv_off(int layer, int n_pages, int page, int kv, int n_kv, int head,
                                                  int tok, int dim, int hd) {
  const size_t base = (((size_t)layer * n_pages + page) * 2 + kv) * n_kv + head;
  return base * kPage * hd + (kv == 0 ? (size_t)tok * hd + dim : (size_t)dim * kPage + tok);
}

// Element offset of value (m, k) of a [rows][K] 16-bit activation matrix in fragment-major order,
// the layout the large-tile GEMM reads its activations in when a forward is tall: rows in tiles of
// 16 and K in steps of 32, each (row tile, K step) a 1 KiB block in matrix-core operand order (lane
// l holds row l % 16 and the 8 values from k = 8 (l / 16)), so one operand fragment is one
// contiguous 1 KiB load instead of 16 rows of 64 B.  Rows are padded to a multiple of 16.
__host__ __device__ __forceinline__ size_t pk_off(int m, int k, int K) {
  return ((size_t)((m >> 4) * (K >> 5) + (k >> 5)) * 64 + (m & 15) + 16 * ((k & 31) >> 3)) * 8 + (k & 7);
}

// Four 16-bit values to 8-byte-aligned memory in one store (a fragment-major group of four).
template <typename T>
__device__ __forceinline__ void st4h(T* p, const T (&v)[4]) {
  if constexpr (sizeof(T) == 2) {
    *reinterpret_cast<uint2*>(p) = make_uint2((uint32_t)v[0] | ((uint32_t)v[1] << 16),
                                              (uint32_t)v[2] | ((uint32_t)v[3] << 16));
  }
}

// Per-request launch arguments (passed by value).
struct ReqArgs {
  int n;                              // requests in this launch
  int B;                              // block size (mask tokens per window)
  int p[kMaxReq];                     // position of the boundary token x0 (= cache length)
  int x0[kMaxReq];                    // boundary token
  int row0[kMaxReq];                  // first row of this request's window
  int max_commit[kMaxReq];            // remaining output budget
  const int32_t* pt[kMaxReq];         // device page table of the request
  int npg[kMaxReq];                   // valid entries of pt
  const int32_t* planted[kMaxReq];    // nullable device [B]: -1 keeps the draft's own token
  const int32_t* cont[kMaxReq];       // nullable device AR continuation for planting
  int cont_len[kMaxReq];
  int cont_c[kMaxReq];                // output tokens committed before this round
  int astar[kMaxReq];                 // planted accept length (continuation mode)
  // direct block diffusion: the request's block tokens (device [B], [M] while undecided).
  // DRAFT rows 1..B embed win[j-1]; VERIFY rows j embed win[j] (the cache-write forward).
  int32_t* win[kMaxReq];              // [B + 1]: slot B gets window row B's latest prediction
  float tau;                          // confidence threshold of the denoising step
  int dsteps;                         // > 0: draft schedule of at most dsteps steps, the last commits all
  // stochastic rounds: the request's uniforms [2B + 2] = u_a0, u_d[1..B], u_acc[1..B], u_t
  // (prefill and AR sampling steps: u[0] draws the token)
  const float* u[kMaxReq];
};

// Row task of the attention kernel.  lim_mode 0: max_lim given; 1: draft
// window (max limit p + B); 2: verify window (max limit p + B + 1), with p
// read from the device request state.
struct AttnTask { int req, row0, nrows, max_lim, lim_mode; };
struct AttnTasks { int n; AttnTask t[kMaxTasks]; };


enum PrepMode { PREP_PREFILL = 0, PREP_DRAFT = 1, PREP_VERIFY = 2, PREP_TOKENS = 3 };

struct PrepArgs {
  int mode;
  int M, hidden, vocab, mask_id;
  int pos0;                    // PREFILL / TOKENS: position of row 0
  const void* prefix;          // PREFILL: [*][hidden] of T, row pos0 + m
  const int32_t* tokens;       // TOKENS: device [M]
  const int32_t* am_prev;      // VERIFY: argmax rows of the draft forward
  const void* embed;           // [vocab][hidden] of T
  const float* gain;           // attn_norm gain of layer 0
  int32_t* row_tok; int32_t* row_pos; int32_t* row_lim; int32_t* row_req;
  int32_t* row_slot;           // physical KV slot (page * 16 + offset) of each row
  float2* row_cs;              // rotary (cos, sin) of each row [M][hd/2]
  const float2* rope; int half;   // rotary table [max_positions][hd/2]
  int32_t* fwd_pt; int pt_ld;     // page ids of this forward's requests [req][pt_ld] (0 past npg)
  float* h; void* xg; float* ssq; int ssq_ld;   // ssq: per-16-column sums of squares [M][ssq_ld]
  int xpk;                     // xg in fragment-major order (pk_off) instead of [M][hidden]
  const ReqArgs* req;          // device request state
  ProfStamp* stamp;            // nullable timing stamps of this launch
};

enum Epi { EPI_QKV = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_LOGITS = 3, EPI_PARTIAL = 4 };

struct GemmArgs {
  const uint4* W; int K; int n_tiles; int M;
  int NT, KSL, S;                               // tiles per workgroup, K slices per tile, K ranges (grid y)
  float* part; int part_ld;                     // PARTIAL: [S][M][part_ld] fp32 sums
  const void* x; int ldx;                       // input rows [M][ldx] of T
  const float* ssq; int ssq_ld; int n_ssq; float eps; int hidden;   // 1/rms row scale: ssq [M][ssq_ld]
  float* h; const float* gain_next; void* xg_out; float* ssq_out;   // RESID: residual, next input
  void* q; int q_ld; int n_heads, n_kv, head_dim, layer, n_pages;   // QKV
  void* kv_pool;
  const int32_t* row_slot; const float2* row_cs;   // QKV: physical KV slot, rotary (cos, sin) [M][hd/2]
  void* act; int act_ld;                        // SWIGLU
  float* logits; int vocab; int mask_id;        // LOGITS
  float* am_v1; int32_t* am_i1; float* am_v2; int am_ld;   // LOGITS: records [M][am_ld]
  float* am_s;                                  // LOGITS, nullable: sum of exp((z - group max) / T) [M][am_ld]
  float am_scale;                               // log2(e) / T for am_s
  int xpk, opk;                                 // large-tile GEMM: x, and xg_out / act, fragment-major (pk_off)
  ProfStamp* stamp;                             // nullable timing stamps of this launch
};

// Inverse-CDF sampling of window rows from their LM-head records and logits.
struct SampleArgs {
  const float* v1; const float* gs; int ld, n_groups, gcols;   // per-group max and exp-sum [M][ld]
  const float* logits; int vocab, mask_id;                    // [M][vocab]
  const float* rmax; const float* rz; float sc;               // row max, row exp-sum, log2(e) / T
  const ReqArgs* req;
  int32_t* tok;                                               // out: sampled token per row
};

// Acceptance test and residual / bonus draw of a stochastic round.
struct AcceptSampleArgs {
  const int32_t* row_tok;                                     // verify rows: a0, d_1..d_B
  const float* lg_d; const float* dmax; const float* dz;      // draft logits and row stats
  const float* lg_v; const float* vmax; const float* vz;      // verify logits and row stats
  int vocab, mask_id, eos_id; float sc;
  const ReqArgs* req;
  int32_t* acc;                                               // [kMaxReq] accepted count A
  int32_t* out; int out_stride;                               // commit records (as k_accept)
  const int* err;                                             // nullable: layer-tail barrier failure flag
};

// Dynamic LDS layout of k_gemm (byte offsets), shared by the kernel and its launcher:
// activation slab [MB][K range + 16 B pad], K-slice partial tiles [W][MT][64] f32x4,
// result tiles [NT][MB][17] f32, epilogue inputs.
struct GemmLds { int red, ctile, ssq, pre, total; };
__host__ __device__ inline GemmLds gemm_lds(int MT, int kr_bytes, int NT, int KSL, int n_ssq, int epi) {
  const int MB = 16 * MT;
  GemmLds L;
  L.red = MB * (kr_bytes + 16);
  L.ctile = L.red + NT * KSL * MT * 64 * 16;
  L.ssq = L.ctile + NT * MB * 17 * 4;
  const bool norm = epi == EPI_QKV || epi == EPI_SWIGLU || epi == EPI_LOGITS;
  (void)norm; (void)n_ssq;
  L.pre = (L.ssq + 15) / 16 * 16;
  int pre = 0;
  if (epi == EPI_QKV) pre = MB * 8 * 8 + MB * 4;           // (cos, sin) of 8 pairs per row, KV slot per row
  if (epi == EPI_RESID) pre = NT * MB * 16 * 4 + NT * 16 * 4;   // h tile, next gain
  L.total = L.pre + pre;
  return L;
}
constexpr int kGemmMaxLds = 160 * 1024 - 1024;   // dynamic LDS budget (static arrays take < 1 KiB)
constexpr int kGemmThreads = 512;                 // 8 waves per GEMM workgroup
constexpr int kGemmPersistentWgs = 256;           // LM head: resident workgroups (one per CU)
// Word 3 of a raw buffer resource (32-bit data format): loads past num_records return zero
// without a memory request.
constexpr int kBufWord3 = 0x00020000;
constexpr int kAttnThreads = 256;                 // 4 waves per attention workgroup: one query head each

struct AttnArgs {
  const void* q; int q_ld;                 // [rows][n_heads*hd]
  const void* kv_pool; int layer; int n_pages; int n_heads; int n_kv;
  const ReqArgs* req;                      // device request state (p, B)
  const int32_t* fwd_pt; int pt_ld;        // page ids [req][pt_ld], gathered by the prep kernel
  const int32_t* row_lim;
  float* part; int max_chunks;             // records [row][head][chunk][hd+4]
  void* out; int out_ld;                   // fold: [rows][n_heads*hd]
  int fold;
  int opk;                                 // fold: out in fragment-major order (pk_off, K = out_ld)
  float scale;
  ProfStamp* stamp;                        // nullable timing stamps of this launch
  AttnTasks tasks;
};

// Fused layer tail (O, gate|up, down) of decode forwards of at most 48 rows: one launch of
// kTailWgs workgroups, one per CU, with two grid barriers (see k_layer_tail).
constexpr int kTailWgs = 256;
constexpr int kTailSyncWords = 16 * 33;   // generation word, 2 barriers x (8 partition counters + 8 done flags), 128 B apart
struct TailArgs {
  GemmArgs o, gu, d;                 // the three GEMMs as k_gemm runs them
  unsigned long long* sync;          // [kTailSyncWords] barrier counters, zero at model creation
  int* err;                          // set to 1 when a barrier wait exceeds its bound
  ProfStamp* stamp;                  // nullable timing stamps of this launch
};

// Timing hook of the launchers: while g_prof_ev[0] is set, launches use hipExtLaunchKernel with
// this start/stop pair (single-threaded use, set and cleared by the engine around one launch).
extern hipEvent_t g_prof_ev[2];

// Launchers (defined in ssb_kernels.hip).
template <typename T>
// bf16 weights are packed as fp16 (*range_err set to 1 if a value exceeds fp16's range)
hipError_t launch_pack(uint4* dst, int n_tiles, int K, int mode, const void* s0, const void* s1, const void* s2,
                       int n0, int n1, int hd, int* range_err, hipStream_t st);
template <typename T> hipError_t launch_prep(const PrepArgs& a, hipStream_t st);
template <typename T> hipError_t launch_gemm(const GemmArgs& a, int epi, hipStream_t st);
template <typename T> hipError_t launch_resid_reduce(const GemmArgs& a, hipStream_t st);
hipError_t launch_gemm_big(const GemmArgs& a, int epi, bool exact, hipStream_t st);
hipError_t launch_layer_tail(const TailArgs& a, hipStream_t st);
int gemm_max_mt(int elem, int K, int S, int NT, int KSL, int n_ssq, int epi);
// gs (nullable, then zs too): per-group exp-sums of the LM head at scale sc = log2(e) / T;
// zs [M] gets the row's sum of exp((z - top1) / T) over the vocabulary without [M].
hipError_t launch_argmax(const float* v1, const int32_t* i1, const float* v2, const float* gs, float sc, int n_groups,
                         int ld, int M, int32_t* tok, float* top1, float* top2, float* zs, hipStream_t st,
                         ProfStamp* stamp = nullptr, const int* err = nullptr);
hipError_t launch_sample_rows(const SampleArgs& a, int rows_per_req, int n_req, hipStream_t st);
hipError_t launch_accept_sample(const AcceptSampleArgs& a, int n_req, hipStream_t st);
template <typename T> hipError_t launch_attn(const AttnArgs& a, int n_chunk_slots, int head_dim, hipStream_t st);
template <typename T>
hipError_t launch_attn_combine(const float* part, int max_chunks, int n_slots, int n_heads, int head_dim,
                               const int32_t* row_lim, int M, void* out, int out_ld, hipStream_t st,
                               ProfStamp* stamp = nullptr);
template <typename T>
hipError_t launch_poison_kv(const ReqArgs* req, int R, const int32_t* acc, int acc_stride, int lo_abs, int hi_abs,
                            void* kv_pool, int n_layers, int n_pages, int n_kv, int hd, hipStream_t st);
hipError_t launch_accept(const int32_t* row_tok, const int32_t* am, const ReqArgs* ra, int n_req, int eos_id,
                         int32_t* out, int out_stride, hipStream_t st, const int* err = nullptr,
                         ProfStamp* stamp = nullptr);
hipError_t launch_dd_init(const ReqArgs* ra, int n_req, int mask_id, int32_t* rec, int rec_stride, hipStream_t st);
hipError_t launch_dd_select(const int32_t* am, const float* zs, const ReqArgs* ra, int n_req, int mask_id,
                            int vocab, int32_t* rec, int rec_stride, hipStream_t st);

}  // namespace ssb
